"""Benchmark of the balanced expert-parallel hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
plan (histogram, balance, layout, placement, duplicate records, prefetch
index) -> dispatch (one-pass scatter of every route's row + weights +
zero-fill) -> combine (weighted K-sum + weight gather).  Inputs are resident
in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload r16-e384-k8|dsv3|r8-e64-k6] [--step-only]

Prints one JSON line.  The headline workload is the largest single-GPU
configuration (R=16, E=384, K=8, S=8192, H=7168, half of the tokens inside
one home rank).  `value` is the dispatch+combine algorithmic HBM bytes of a
step divided by the measured time of the whole step (plan included), in
GB/s; the line also carries tokens/s, per-call times inside the step (HIP
events on the stream the kernels run on), the roofline of the dominant
kernel (its duration from back-to-back launches on the timed inputs), the
memory-system ceilings of the same access patterns measured on the same
buffers, a maxvio sweep on the same shapes, the dedup ablations, a
secondary section on the r8-e64-k6 shape (whose data partly stays in the
256 MB last-level cache) with weight prefetch, gradient reduction and the
padded serving workload, and the oracle timed on the host as a CPU
baseline.  --step-only keeps just the step (the profiler runs use it).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD published peak
METRIC = "dispatch+combine HBM GB/s (% of peak) and tokens/s vs maxvio; plan µs"
PROFILES = os.path.join(ROOT, "profiles")
HEADLINE = "r16-e384-k8"
SECONDARY = "r8-e64-k6"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Inputs:
    """One batch of seeded synthetic input, resident on the GPU (the routing
    also kept on the host)."""

    def __init__(self, moon, ctx, config, seed, alpha, dev):
        import torch

        import synth
        import synth.gpu as sg
        c = synth.WORKLOADS[synth.workload_id(config)]
        R, E, K, S, H = c["R"], c["E"], c["K"], c["S"], c["H"]
        topk, w = synth.routing(config, seed, alpha)
        self.seed = seed
        self.topk_h, self.w_h = topk, w
        self.maxvio = synth.maxvio(topk, E)
        self.topk = torch.from_numpy(topk).to(dev)
        self.w = torch.from_numpy(w).to(dev)
        self.hidden = sg.hidden(seed, R, S, H, dev)
        self.y = sg.y(seed, R * ctx.NvS, H, dev)
        self.out = torch.empty((R, S, H), dtype=torch.bfloat16, device=dev)
        self.wsk = torch.empty((R, S, K), dtype=torch.float32, device=dev)
        self.plan = moon.moon_plan_create(ctx)


def bytes_from_counts(R, S, K, H, n_grp, n_dup, n_pad):
    """Bytes the method must move in dispatch and combine, from a plan's
    duplicate groups, duplicate rows and padding rows (all ranks).
    `dispatch` is the one-pass dispatch (every route's row written once from
    the token's row, read once); `dispatch_epilogue` adds the epilogue's one
    read of each duplicate group's primary row."""
    n_route = R * S * K
    row = 2 * H
    d_min = (row * R * S + row * n_route + row * n_pad + 4 * n_route * 3 + 4 * n_pad
             + 12 * n_grp + 4 * n_dup)
    combine = row * n_route + row * R * S + 4 * n_route * 2 + 4 * n_route  # + weight gather
    return dict(dispatch=d_min, dispatch_epilogue=d_min + row * n_grp, combine=combine,
                n_route=n_route, n_dup=n_dup, n_grp=n_grp, n_pad=n_pad)


def plan_counts(dup_counts, zero_fill_ranges):
    """(duplicate groups, duplicate rows, padding rows) of a plan."""
    return (int(dup_counts[:, 0].sum()), int(dup_counts[:, 1].sum()),
            int((zero_fill_ranges[..., 1] - zero_fill_ranges[..., 0]).sum()))


def algorithmic_bytes(moon, ctx, plan):
    """Bytes the method must move in dispatch and combine for this plan."""
    c = ctx.cfg
    pt = {k: v.cpu().numpy() for k, v in moon.plan_tensors(plan).items()}
    nb = bytes_from_counts(c.R, c.S, c.K, c.H, *plan_counts(pt["dup_counts"],
                                                             pt["zero_fill_ranges"]))
    nb.update(slots_used=int(pt["remote_stats"][:, 0].sum()),
              routes_in_slots=int(pt["remote_stats"][:, 1].sum()))
    return nb


def step_calls(moon, ctx, s, wwin, stream, ev=None):
    """One step: plan (with the prefetch index) -> dispatch -> combine, with
    optional HIP events between the calls."""
    if ev is not None:
        ev[0].record(stream)
    moon.moon_plan(ctx, s.topk, None, s.plan, stream=stream)
    if ev is not None:
        ev[1].record(stream)
    moon.moon_dispatch(ctx, s.plan, s.hidden, s.w, stream=stream)
    if ev is not None:
        ev[2].record(stream)
    moon.moon_combine(ctx, s.plan, s.y, wwin, moon.MOON_COMBINE_WEIGHTED, s.out, s.wsk,
                      stream=stream)
    if ev is not None:
        ev[3].record(stream)


def run_steps(moon, ctx, sets, steps, warmup, stream):
    """Warm up, then time exactly `steps` steps; per-call HIP events on `stream`."""
    import torch
    _, wwin = moon.window_tensors(ctx)

    for i in range(max(warmup, len(sets))):  # every input set planned at least once
        step_calls(moon, ctx, sets[i % len(sets)], wwin, stream)
    torch.cuda.synchronize()
    for s in sets:
        st = moon.moon_plan_status(s.plan, stream)
        if st != moon.MOON_OK:
            raise RuntimeError(f"plan status {moon.moon_status_str(st)}")

    # whole-step timing: K steps back to back
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        step_calls(moon, ctx, sets[i % len(sets)], wwin, stream)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = t0.elapsed_time(t1) / steps

    # per-call timing: the same steps again, each call bracketed by events
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step_calls(moon, ctx, sets[i % len(sets)], wwin, stream, evs[i])
    torch.cuda.synchronize()
    names = ["plan", "dispatch", "combine"]
    calls = {n: sum(ev[j].elapsed_time(ev[j + 1]) for ev in evs) / steps * 1e3
             for j, n in enumerate(names)}  # microseconds

    # launch durations: the same calls back to back between two events (no
    # event markers between launches), on the input sets of the timed steps;
    # each of dispatch and combine is one kernel launch
    launch = {
        "combine": time_call(lambda i=0: moon.moon_combine(
            ctx, sets[i % len(sets)].plan, sets[i % len(sets)].y, wwin,
            moon.MOON_COMBINE_WEIGHTED, sets[i % len(sets)].out, sets[i % len(sets)].wsk,
            stream=stream), steps, stream),
        "dispatch": time_call(lambda i=0: moon.moon_dispatch(
            ctx, sets[i % len(sets)].plan, sets[i % len(sets)].hidden, sets[i % len(sets)].w,
            stream=stream), steps, stream),
    }
    return ms_step, wall, calls, launch


def time_call(fn, iters, stream):
    """Average microseconds of `fn` over `iters` back-to-back calls (HIP events
    on `stream`); `fn` may take the call index."""
    import torch
    for _ in range(3):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(iters):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters * 1e3


def measure_copy(stream, nbytes=1 << 30, iters=20):
    """The runtime's plain device-to-device copy of `nbytes` (torch's copy_ of
    a contiguous tensor, a hipMemcpyAsync) on the same GPU: read + write bytes
    per second, reported beside the published peak as context."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    t = time_call(lambda i=0: b.copy_(a), iters, stream)
    del a, b
    torch.cuda.empty_cache()
    return {"what": "hipMemcpyAsync device-to-device (torch copy_)", "bytes_per_copy": 2 * nbytes,
            "us": round(t, 2),
            "GBps": round(2 * nbytes / (t * 1e-6) / 1e9, 1)}


_CEIL = None


def _ceiling_lib():
    """The benchmark's reference kernels (libmoon_ceiling.so, built beside libmoon)."""
    global _CEIL
    if _CEIL is None:
        import ctypes
        import torch  # noqa: F401  (bind to the HIP runtime torch loaded)
        path = os.path.join(ROOT, "combine_balanced_planning_amd", "libmoon_ceiling.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.moon_ceiling_read.argtypes = [vp, i64, vp, vp]
        lib.moon_ceiling_fill.argtypes = [vp, i64, vp]
        lib.moon_ceiling_copy.argtypes = [vp, vp, i64, vp]
        lib.moon_ceiling_write_rows.argtypes = [vp, vp, i64, i32, i32, vp]
        lib.moon_ceiling_read_rows.argtypes = [vp, vp, i64, i32, i32, vp, vp]
        lib.moon_ceiling_scatter_cached.argtypes = [vp, vp, vp, i64, i32, i32, vp]
        for f in ("read", "fill", "copy", "write_rows", "read_rows", "scatter_cached"):
            getattr(lib, "moon_ceiling_" + f).restype = ctypes.c_int
        _CEIL = lib
    return _CEIL


def measure_ceilings(moon, ctx, s, nb, stream, iters):
    """What the memory system delivers for the access patterns of the step,
    each alone, on the step's own buffers and row lists (HIP events, average
    of back-to-back launches):
      write_rows  dispatch's stores without its loads (every route's row of
                  the plan's dst, same grid and slice order as dispatch)
      scatter_cached  dispatch with its token rows served from the last-level
                  cache (token t stores the row of token t mod 4096)
      read_rows   combine's loads without its stores (the K routed rows of
                  every token, same grid as combine)
      fill / read contiguous non-temporal stores / loads over the windows and
                  the y array
      copy        contiguous load + store, the token rows into the output
    The dispatch and combine launch times are put beside them."""
    import ctypes

    import torch
    lib = _ceiling_lib()
    c = ctx.cfg
    win, _ = moon.window_tensors(ctx)
    sink = torch.zeros(4, dtype=torch.int32, device=win.device)
    dst = moon.plan_tensors(s.plan)["dst"]
    st = ctypes.c_void_p(stream.cuda_stream)
    row = 2 * c.H
    ntok = c.R * c.S

    def chk(rc):
        if rc != 0:
            raise RuntimeError(f"ceiling kernel failed: hip error {rc}")

    legs = {
        "write_rows": (nb["n_route"] * row, lambda i=0: chk(lib.moon_ceiling_write_rows(
            win.data_ptr(), dst.data_ptr(), ntok, c.K, c.H, st))),
        "scatter_cached": (nb["n_route"] * row + ntok * row,
                           lambda i=0: chk(lib.moon_ceiling_scatter_cached(
                               s.hidden.data_ptr(), win.data_ptr(), dst.data_ptr(), ntok, c.K,
                               c.H, st))),
        "read_rows": (nb["n_route"] * row, lambda i=0: chk(lib.moon_ceiling_read_rows(
            s.y.data_ptr(), dst.data_ptr(), ntok, c.K, c.H, sink.data_ptr(), st))),
        "fill": (win.numel() * 2, lambda i=0: chk(lib.moon_ceiling_fill(
            win.data_ptr(), win.numel() * 2, st))),
        "read": (s.y.numel() * 2, lambda i=0: chk(lib.moon_ceiling_read(
            s.y.data_ptr(), s.y.numel() * 2, sink.data_ptr(), st))),
        "copy": (2 * s.hidden.numel() * 2, lambda i=0: chk(lib.moon_ceiling_copy(
            s.hidden.data_ptr(), s.out.data_ptr(), s.hidden.numel() * 2, st))),
    }
    out = {}
    for name, (nbytes, fn) in legs.items():
        t = time_call(fn, iters, stream)
        out[name] = {"bytes": int(nbytes), "us": round(t, 2),
                     "GBps": round(nbytes / (t * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(nbytes / (t * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
    torch.cuda.synchronize()
    return out


def measure_ablations(moon, ctx, s, nb, stream, iters):
    """The pages' two-pass structures on the same input: dispatch with the
    dedup epilogue (the scatter stores primaries only, then the epilogue
    reads each duplicate group's primary back and stores its duplicates) and
    combine with the duplicate prologue (folds into the window, then gathers
    primaries)."""
    c = ctx.cfg
    row = 2 * c.H
    win, wwin = moon.window_tensors(ctx)
    t_epi = time_call(lambda i=0: moon.moon_dispatch(ctx, s.plan, s.hidden, s.w,
                                                 flags=moon.MOON_DISPATCH_DEDUP_EPILOGUE,
                                                 stream=stream), iters, stream)
    t_one = time_call(lambda i=0: moon.moon_dispatch(ctx, s.plan, s.hidden, s.w, stream=stream),
                      iters, stream)
    flags = moon.MOON_COMBINE_WEIGHTED | moon.MOON_COMBINE_DUP_PROLOGUE
    t_pro = time_call(lambda i=0: moon.moon_combine(ctx, s.plan, s.y, wwin, flags, s.out, s.wsk,
                                                stream=stream), iters, stream)
    t_plain = time_call(lambda i=0: moon.moon_combine(ctx, s.plan, s.y, wwin,
                                                  moon.MOON_COMBINE_WEIGHTED, s.out, s.wsk,
                                                  stream=stream), iters, stream)
    # prologue: every group reads its m+1 rows (and weights) and writes one
    # folded row; the gather then reads one row per primary route
    pro_bytes = (row * (nb["n_grp"] + nb["n_dup"]) + 4 * (nb["n_grp"] + nb["n_dup"])
                 + 12 * nb["n_grp"] + 4 * nb["n_dup"] + row * nb["n_grp"]
                 + row * (nb["n_route"] - nb["n_dup"]) + row * c.R * c.S + 4 * nb["n_route"] * 3)
    moon.moon_dispatch(ctx, s.plan, s.hidden, s.w, stream=stream)  # restore the windows
    return {
        "dispatch_one_pass_us": round(t_one, 2),
        "dispatch_epilogue_us": round(t_epi, 2),
        "dispatch_epilogue_bytes": int(nb["dispatch_epilogue"]),
        "dispatch_epilogue_GBps": round(nb["dispatch_epilogue"] / (t_epi * 1e-6) / 1e9, 1),
        "combine_plain_us": round(t_plain, 2),
        "combine_dup_prologue_us": round(t_pro, 2),
        "combine_dup_prologue_bytes": int(pro_bytes),
        "combine_dup_prologue_GBps": round(pro_bytes / (t_pro * 1e-6) / 1e9, 1),
        "dup_groups": nb["n_grp"], "dup_rows": nb["n_dup"],
    }


# maxvio sweeps: workload -> (workload of the skewed levels, levels);
# r8-e64-k6 sweeps the skewed workload of its shapes, the large R=16
# workload its own levels 1.. (level 0 is the timed base run).
SWEEPS = {"r8-e64-k6": ("r8-e64-k6-skewed", [0, 1, 2, 3]),
          "r16-e384-k8": ("r16-e384-k8", [1, 2, 3, 4])}

# Expert FFN intermediate width H' per workload: DeepSeek-V3's expert width for
# the DSv3-shaped workload and for the R=16 workload, whose hidden width is
# DeepSeek-V3's too; H/2 for r8-e64-k6 (readings: the pages give none).
FFN_WIDTH = {"r8-e64-k6": 1024, "dsv3": 2048, "r16-e384-k8": 2048}


class WeightBufs:
    """Expert weights (gate, up, down: [E, H*H'] bf16, seeded) and their slot
    rows ([R, B, H*H'] bf16) for timing the weight prefetch on any plan of
    the context."""

    def __init__(self, ctx, hp):
        import torch
        import synth
        import synth.gpu as sg
        c = ctx.cfg
        self.ctx, self.hp, self.L = ctx, hp, c.H * hp
        key = synth.stream_key(12345, 21)
        self.w = [sg.fill_bf16(torch.empty((c.E, self.L), dtype=torch.bfloat16, device="cuda"),
                               key, i * c.E * self.L) for i in range(3)]
        self.sl = [torch.zeros((c.R, ctx.B, self.L), dtype=torch.bfloat16, device="cuda")
                   for _ in range(3)]

    def prefetch(self, moon, plan, stream, iters):
        """(µs per call, slots used, experts held, bytes per slot copy, minimum bytes)."""
        import torch
        etc = moon.plan_tensors(plan)["experts_to_copy"].cpu()
        n_used = int((etc >= 0).sum())
        n_held = int(torch.unique(etc[etc >= 0]).numel())
        t = time_call(lambda i=0: moon.moon_prefetch_weight(self.ctx, plan, self.w, self.sl,
                                                          stream=stream), iters, stream)
        L = self.L
        return t, n_used, n_held, 3 * n_used * L * 2 * 2, 3 * (n_held + n_used) * L * 2

    def release(self):
        import torch
        del self.w, self.sl
        torch.cuda.empty_cache()


def measure_weights(moon, ctx, s, stream, iters, hp, wb=None):
    """Gradient reduction and weight prefetch for the plan of `s`: gate, up and
    down tensors [E, H*H'] (bf16 weights, fp32 gradients) and their slots.
    The reduction's buffers are freed before the prefetch's are taken (or
    `wb`, already allocated, is used)."""
    import torch
    import synth
    import synth.gpu as sg
    c = ctx.cfg
    L = c.H * hp
    key = synth.stream_key(12345, 21)
    g = [sg.fill_bf16(torch.empty((c.E, L), dtype=torch.bfloat16, device="cuda"), key).float()
         for _ in range(3)]
    sgr = [torch.zeros((c.R, ctx.B, L), dtype=torch.float32, device="cuda") for _ in range(3)]
    t_rg = time_call(lambda i=0: moon.moon_reduce_grad(ctx, s.plan, g, sgr, stream=stream), iters,
                     stream)
    del g, sgr
    torch.cuda.empty_cache()
    own = wb is None
    if own:
        wb = WeightBufs(ctx, hp)
    t_pw, n_used, n_held, pw_bytes, pw_min = wb.prefetch(moon, s.plan, stream, iters)
    if own:
        wb.release()
    rg_bytes = 3 * (n_held + n_used) * L * 4 * 2  # expert row read+write; slot read+clear
    return {
        "ffn_width": hp, "tensors": 3, "slots_used": n_used, "experts_held": n_held,
        "prefetch_weight_us": round(t_pw, 2), "prefetch_weight_bytes": pw_bytes,
        "prefetch_weight_GBps": round(pw_bytes / (t_pw * 1e-6) / 1e9, 1),
        "prefetch_weight_min_bytes": pw_min,
        "prefetch_weight_min_GBps": round(pw_min / (t_pw * 1e-6) / 1e9, 1),
        "reduce_grad_us": round(t_rg, 2), "reduce_grad_bytes": rg_bytes,
        "reduce_grad_GBps": round(rg_bytes / (t_rg * 1e-6) / 1e9, 1),
    }


def measure_serving(moon, dev, stream, steps, warmup):
    """The padded serving workload per level: plan (with the tokens_per_expert
    histogram; the prefetch index included) -> dispatch -> plain K-sum
    combine, timed per call with HIP events on `stream`."""
    import torch
    import synth
    import synth.gpu as sg
    res = []
    for level in range(len(synth.SERVING_LEVELS)):
        wl = synth.serving_workload(level)
        R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
        ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
        plan = moon.moon_plan_create(ctx)
        topk = torch.from_numpy(wl["topk"]).to(dev)
        tpe = torch.from_numpy(wl["tokens_per_expert"]).to(dev)
        w = torch.from_numpy(wl["w"]).to(dev)
        hidden = sg.hidden(wl["seed"], R, S, H, dev)
        for r in range(R):
            hidden[r, int(wl["n_tok"][r]):] = 0
        y = sg.y(wl["seed"], R * ctx.NvS, H, dev)
        out = torch.empty((R, S, H), dtype=torch.bfloat16, device=dev)
        win, wwin = moon.window_tensors(ctx)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            moon.moon_plan(ctx, topk, tpe, plan, stream=stream)
            if ev is not None:
                ev[1].record(stream)
            moon.moon_dispatch(ctx, plan, hidden, w, stream=stream)
            if ev is not None:
                ev[2].record(stream)
            moon.moon_combine(ctx, plan, y, None, 0, out, None, stream=stream)
            if ev is not None:
                ev[3].record(stream)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        st = moon.moon_plan_status(plan, stream)
        if st != moon.MOON_OK:
            raise RuntimeError(f"serving plan status {moon.moon_status_str(st)}")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for ev in evs:
            step(ev)
        torch.cuda.synchronize()
        t = [sum(ev[i].elapsed_time(ev[i + 1]) for ev in evs) / steps * 1e3 for i in range(3)]
        nb = algorithmic_bytes(moon, ctx, plan)
        nb["combine"] -= 4 * nb["n_route"] * 2  # no weight read, no weight gather
        real = int(wl["n_tok"].sum())
        res.append({
            "level": wl["level_name"], "S": S, "real_tokens": real, "maxvio": round(wl["maxvio"], 2),
            "ms_per_step": round(ms, 4), "plan_us": round(t[0], 2), "dispatch_us": round(t[1], 2),
            "combine_us": round(t[2], 2),
            "dispatch_GBps": round(nb["dispatch"] / (t[1] * 1e-6) / 1e9, 1),
            "combine_GBps": round(nb["combine"] / (t[2] * 1e-6) / 1e9, 1),
            "real_tokens_per_s": round(real / (ms * 1e-3)),
            "capacity_tokens_per_s": round(R * S / (ms * 1e-3)),
            "dup_rows": nb["n_dup"], "slots_used": nb["slots_used"]})
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)
        del hidden, y, out, win, wwin
        torch.cuda.empty_cache()
    return res


def _code_only(text, path):
    """Source text without comments and blank space (C/C++/HIP and Python), so
    that editing a comment does not invalidate recorded counter readings."""
    if path.endswith(".py"):
        text = re.sub(r"(?m)#.*$", "", text)
    else:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", " ", text).strip()


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read(), f).encode())
    return h.hexdigest()[:16]


# Sources whose change invalidates a kernel's recorded counter readings: its
# own file, the shared header and host code (layout, launch checks) and the
# input generator.
PMC_COMMON = ["combine_balanced_planning_amd/csrc/moon_internal.h",
              "combine_balanced_planning_amd/csrc/moon_api.hip",
              "synth/__init__.py"]
PMC_KERNEL_FILES = {"k_plan": "combine_balanced_planning_amd/csrc/moon_plan.hip",
                    "k_dispatch": "combine_balanced_planning_amd/csrc/moon_dispatch.hip",
                    "k_combine": "combine_balanced_planning_amd/csrc/moon_combine.hip",
                    "k_prefetch_index": "combine_balanced_planning_amd/csrc/moon_combine.hip"}
PMC_SOURCES = PMC_COMMON + sorted(set(PMC_KERNEL_FILES.values()))


def kernel_sources(kernel):
    """Files whose content decides `kernel`'s memory traffic."""
    base = kernel.split("<", 1)[0]
    own = [f for p, f in PMC_KERNEL_FILES.items() if base.startswith(p)]
    return PMC_COMMON + own[:1]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary of `workload`, if its sources are unchanged since (else None)."""
    path = os.path.join(PROFILES, f"pmc_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    hashes = rec.get("source_hashes", {})
    if any(hashes.get(f) != source_hash([f]) for f in kernel_sources(kernel)):
        return None
    # kernel names carry their template arguments; take the instantiation of
    # `kernel` with the most launches (the counter runs time the step only)
    cands = [v for n, v in rec.get("kernels", {}).items() if n.split("<", 1)[0] == kernel]
    if not cands:
        return None
    return max(cands, key=lambda v: v["launches"])["hbm_bytes_per_launch"]


def short_kernel_name(name):
    """Kernel name without 'void', this library's namespaces and the argument list."""
    n = name[5:] if name.startswith("void ") else name
    n = n.replace("moon::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return n.split("(", 1)[0].strip()


def read_counter_csv(d):
    """{kernel: [values per dispatch]} from a rocprofv3 --pmc csv output folder."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                out.setdefault(short_kernel_name(row["Kernel_Name"]), []).append(
                    float(row["Counter_Value"]))
    return out


def summarize_pmc(workload, dirs, commands):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the same counters
    read for a plain 1 GiB copy, and write profiles/pmc_<workload>.{json,md}."""
    fetch, write, cfetch, cwrite = (read_counter_csv(d) for d in dirs)

    def calib(tab):
        # the copy kernel is the one launched exactly five times
        cands = [v for v in tab.values() if len(v) == 5]
        if len(cands) != 1:
            raise SystemExit("calibration run: expected one kernel with 5 launches")
        return (1 << 30) / (sum(cands[0]) / 5 * 1024.0)

    ff, wf = calib(cfetch), calib(cwrite)
    kernels = {}
    for name in sorted(set(fetch) & set(write)):
        if not name.startswith("k_"):
            continue
        f_kib = sum(fetch[name]) / len(fetch[name])
        w_kib = sum(write[name]) / len(write[name])
        kernels[name] = {"launches": len(fetch[name]), "fetch_kib": round(f_kib, 1),
                         "write_kib": round(w_kib, 1),
                         "hbm_bytes_per_launch": int(f_kib * 1024 * ff + w_kib * 1024 * wf)}
    rec = {"workload": workload, "commands": commands,
           "calibration": {"kernel": "torch.add(a, 0, out=b), 1 GiB read + 1 GiB written",
                           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "source_hashes": {f: source_hash([f]) for f in PMC_SOURCES}, "kernels": kernels}
    with open(os.path.join(PROFILES, f"pmc_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    lines = [f"# HBM traffic counters — workload {workload}", "",
             "Commands (repo root, one MI355X):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", f"Calibration: a plain 1 GiB copy reads {1 / ff:.4f} GiB by FETCH_SIZE and "
              f"writes {1 / wf:.4f} GiB by WRITE_SIZE; factors {ff:.4f} and {wf:.4f} scale "
              "the kernels' readings below.", "",
              "| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM MB per launch |",
              "|---|---|---|---|---|"]
    for n, k in kernels.items():
        lines.append(f"| {n} | {k['launches']} | {k['fetch_kib']:.1f} | {k['write_kib']:.1f} | "
                     f"{k['hbm_bytes_per_launch'] / 1e6:.2f} |")
    with open(os.path.join(PROFILES, f"pmc_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(rec))


def _trace_rows(d):
    """Per-dispatch rows of a rocprofv3 --kernel-trace csv folder:
    (kernel, grid size in work-items, duration ns)."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                grid = 1
                for ax in ("X", "Y", "Z"):
                    grid *= int(row.get(f"Grid_Size_{ax}", 1) or 1)
                rows.append((short_kernel_name(row["Kernel_Name"]), grid,
                             int(row["End_Timestamp"]) - int(row["Start_Timestamp"])))
    return rows


def summarize_trace(workload, d, command, bench_line=None):
    """Write profiles/kernels_<workload>.md from a rocprofv3 --kernel-trace
    csv folder, one line per (kernel, grid size): the same kernel launched on
    another workload's shape is a line of its own."""
    groups = {}
    for name, grid, ns in _trace_rows(d):
        groups.setdefault((name, grid), []).append(ns)
    total = sum(sum(v) for v in groups.values())
    lines = [f"# Kernel trace — workload {workload}", "", "Command (repo root, one MI355X):", "",
             "    " + command, "",
             "One line per kernel and grid size (work-items); durations from the per-dispatch "
             "kernel trace.", "",
             "| kernel | grid | calls | total µs | avg µs | min µs | max µs | % of GPU time |",
             "|---|---|---|---|---|---|---|---|"]
    omitted = 0
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        if sum(v) < 1e-3 * total:
            omitted += 1
            continue
        lines.append(f"| {name} | {grid} | {len(v)} | {sum(v) / 1e3:.1f} | "
                     f"{sum(v) / len(v) / 1e3:.2f} | {min(v) / 1e3:.2f} | {max(v) / 1e3:.2f} | "
                     f"{100.0 * sum(v) / total:.1f} |")
    if omitted:
        lines.append(f"| ({omitted} more lines, each under 0.1 % of GPU time) | | | | | | | |")
    if bench_line:
        with open(bench_line) as f:
            js = [ln for ln in f if ln.startswith("{")]
        if js:
            b = json.loads(js[-1])
            lines += ["", f"Bench line of the same run: step {b['ms_per_step']} ms; HIP-event call "
                      f"times (µs) {b['call_us']}; roofline {b['roofline']}."]
    with open(os.path.join(PROFILES, f"kernels_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


# Memory-queue counters of the L2 (TCC) to memory interface, two passes
# (at most four TCC counters a pass), each with the GPU's busy cycles.
STALL_PASSES = [["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_RDREQ_sum",
                 "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "GRBM_GUI_ACTIVE"],
                ["TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum", "TCC_TAG_STALL_sum",
                 "TCC_EA0_WRREQ_LEVEL_sum", "TCC_EA0_RDREQ_LEVEL_sum", "GRBM_GUI_ACTIVE"]]
STALL_KERNELS = ["k_dispatch_scatter", "k_combine_staged", "k_write_rows", "k_scatter_cached",
                 "k_read_rows", "k_fill", "k_read", "k_copy"]


def read_counter_table(d):
    """{kernel: {counter: mean value per dispatch}} from a rocprofv3 --pmc csv folder."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    acc = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                k = short_kernel_name(row["Kernel_Name"]).split("<", 1)[0]
                per = acc.setdefault(k, {}).setdefault(row["Counter_Name"], {})
                per[row.get("Dispatch_Id", len(per))] = float(row["Counter_Value"])
    return {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def summarize_stalls(workload, dirs, commands):
    """profiles/stalls_<workload>.md: per kernel of the step and of the ceiling
    legs, the L2-to-memory requests and queue occupancy per busy cycle and the
    cycles requests waited for memory-controller credit."""
    a, b = (read_counter_table(d) for d in dirs)
    lines = [f"# Memory-queue counters — workload {workload}", "",
             "Commands (repo root, one MI355X):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", "Per kernel, means over its launches; counters are sums over the L2 "
              "channels, divided by the GPU's busy cycles (GRBM_GUI_ACTIVE).  Requests to "
              "memory are 64 B (writes) and 128 B (reads) here.", "",
              "| kernel | busy cycles | write req / cycle | read req / cycle | writes in flight "
              "| reads in flight | write-credit stall / cycle | read-credit stall / cycle "
              "| tag stall / cycle |", "|---|---|---|---|---|---|---|---|---|"]
    for k in STALL_KERNELS:
        if k not in a or k not in b:
            continue
        ca, cb = a[k], b[k]
        cyc = ca["GRBM_GUI_ACTIVE"]
        cyc_b = cb["GRBM_GUI_ACTIVE"]
        lines.append(
            f"| {k} | {cyc:.4g} | {ca['TCC_EA0_WRREQ_sum'] / cyc:.3f} | "
            f"{ca['TCC_EA0_RDREQ_sum'] / cyc:.3f} | {cb['TCC_EA0_WRREQ_LEVEL_sum'] / cyc_b:.0f} | "
            f"{cb['TCC_EA0_RDREQ_LEVEL_sum'] / cyc_b:.0f} | "
            f"{cb['TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum'] / cyc_b:.3f} | "
            f"{ca['TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum'] / cyc:.3f} | "
            f"{cb['TCC_TAG_STALL_sum'] / cyc_b:.3f} |")
    with open(os.path.join(PROFILES, f"stalls_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def cpu_baseline(config, topk, w, seed, budget_s=12.0, sample_tokens=512):
    """The oracle, as it stands, on one host core.  Its plan is timed once on
    the full routing; then plan + dispatch + combine run for about `budget_s`
    seconds on a bounded sample of the same workload: the first
    `sample_tokens` tokens of every source rank with their routing, their
    token rows and the routed rows of y drawn from the workload's seeded
    streams.  Combine runs the oracle's fp32 path alone (its float64
    reference sum is not computed).  The rate is the sample's dispatch +
    combine algorithmic bytes over the sample's plan + dispatch + combine
    time."""
    import numpy as np

    import oracle
    import synth
    c = synth.WORKLOADS[synth.workload_id(config)]
    R, E, K, S, H, B, P = (c[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    t0 = time.perf_counter()
    full = oracle.plan(topk, E, B, P)
    t_full = time.perf_counter() - t0
    if full.status != oracle.OK:
        raise RuntimeError(f"oracle plan status {full.status}")
    Ss = min(S, sample_tokens)
    topk_s = np.ascontiguousarray(topk[:, :Ss])
    w_s = np.ascontiguousarray(w[:, :Ss])
    ids = (np.arange(R)[:, None] * S + np.arange(Ss)[None, :]).reshape(-1)
    hidden = synth.bf16_rows(synth.stream_key(seed, synth.TAG_HIDDEN), ids, H).reshape(R, Ss, H)
    pl = oracle.plan(topk_s, E, B, P)
    rows = np.unique(np.where(pl.dst >= 0, pl.dst, -pl.dst - 1).astype(np.int64))
    y = np.zeros((R * pl.NvS, H), np.uint16)
    y[rows] = synth.bf16_rows(synth.stream_key(seed, synth.TAG_Y), rows, H)
    nb = bytes_from_counts(R, Ss, K, H, *plan_counts(pl.dup_counts, pl.zero_fill_ranges))
    bytes_dc = nb["dispatch"] + nb["combine"]
    n = 0
    t_plan = t_disp = t_comb = 0.0
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        pl = oracle.plan(topk_s, E, B, P)
        t1 = time.perf_counter()
        _, wwin = oracle.dispatch(pl, hidden, w_s)
        t2 = time.perf_counter()
        oracle.combine(pl, y, wwin, weighted=True, exact=False)
        t3 = time.perf_counter()
        t_plan += t1 - t0
        t_disp += t2 - t1
        t_comb += t3 - t2
        n += 1
        del wwin
        if time.perf_counter() - t_start >= budget_s:
            break
    total = t_plan + t_disp + t_comb
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         model)
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": round(bytes_dc * n / total / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "host_cpu": model, "host_cores_available": avail,
            "tokens_per_s": round(R * Ss * n / total),
            "plan_full_ms": round(t_full * 1e3, 2),
            "sample": f"{c['name']} (seed {seed}): oracle plan of the full routing "
                      f"{t_full * 1e3:.1f} ms; then the first {Ss} of the {S} tokens of every "
                      f"source rank ({R * Ss} tokens, {bytes_dc / 1e9:.3f} GB of dispatch + "
                      f"combine bytes) x {n}: plan {t_plan / n * 1e3:.1f} ms, dispatch "
                      f"{t_disp / n * 1e3:.1f} ms, combine (fp32 path) {t_comb / n * 1e3:.1f} ms "
                      f"per pass on 1 host core"}


def measure_step(moon, config, dev, stream, steps, warmup):
    """A context and two input sets of `config` (alternated, so a step never
    finds the previous step's data in the 256 MB last-level cache), the step
    timing, the step's algorithmic bytes and the roofline figures of its two
    bulk kernels.  Returns (results, ctx, sets)."""
    import synth
    c = synth.WORKLOADS[synth.workload_id(config)]
    R, E, K, S, H, B, P = (c[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    log(f"[bench] workload {c['name']}: building inputs")
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    seed = synth.seed_of(config, 0)
    sets = [Inputs(moon, ctx, config, seed, 0.0, dev),
            Inputs(moon, ctx, config, seed + 500, 0.0, dev)]
    log(f"[bench] workload {c['name']}: timing")
    ms_step, wall, calls, launch = run_steps(moon, ctx, sets, steps, warmup, stream)
    nbs = [algorithmic_bytes(moon, ctx, s.plan) for s in sets]

    def avg(k):
        return 0.5 * (nbs[0][k] + nbs[1][k])

    bytes_dc = avg("dispatch") + avg("combine")
    value = bytes_dc / (ms_step * 1e-3) / 1e9
    t_dc = (calls["dispatch"] + calls["combine"]) * 1e-6
    # Roofline figures of the step's two bulk kernels (each call is one
    # launch): algorithmic bytes per launch over the average launch duration
    # of back-to-back launches on the timed inputs.
    kernels = {}
    for kname, call in (("k_dispatch_scatter", "dispatch"), ("k_combine_staged", "combine")):
        nbytes = avg(call)
        ach = nbytes / (launch[call] * 1e-6) / 1e9
        kernels[kname] = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS,
                          "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4),
                          "traffic": measured_traffic(kname, c["name"]), "kernel": kname,
                          "algorithmic_bytes_per_launch": int(nbytes),
                          "avg_launch_us": round(launch[call], 2),
                          "in_step_call_us": round(calls[call], 2)}
    dominant = max(kernels, key=lambda k: kernels[k]["avg_launch_us"])
    res = {
        "workload": c["name"], "R": R, "E": E, "K": K, "S": S, "H": H, "token_padding": P,
        "B": B, "maxvio": round(sets[0].maxvio, 4), "ms_per_step": round(ms_step, 4),
        "value": value, "wall_s_timed": round(wall, 4),
        "tokens_per_s": round(R * S / (ms_step * 1e-3)),
        "dispatch_combine_GBps": round(bytes_dc / t_dc / 1e9, 1),
        "tokens_per_s_excl_plan": round(R * S / t_dc),
        "call_us": {k: round(v, 2) for k, v in calls.items()},
        "plan_us": round(calls["plan"], 2),
        "bytes_per_step": {"dispatch": int(avg("dispatch")), "combine": int(avg("combine")),
                           "dispatch_epilogue": int(avg("dispatch_epilogue")),
                           "dup_groups": nbs[0]["n_grp"], "dup_rows": nbs[0]["n_dup"],
                           "pad_rows": nbs[0]["n_pad"]},
        "slots_used": nbs[0]["slots_used"], "routes_in_slots": nbs[0]["routes_in_slots"],
        "roofline": kernels[dominant], "kernels": kernels,
    }
    return res, ctx, sets, nbs[0]


def measure_sweep(moon, ctx, config, base, steps, warmup, stream, dev, wb=None, base_plan=None):
    """maxvio sweep on the same shapes: the base run, then the skewed levels.
    With `wb`, each level also times the weight prefetch of its plan (the
    pages stack the planning and weight-prefetch kernels onto dispatch)."""
    import synth
    c = synth.WORKLOADS[synth.workload_id(config)]
    R, S = c["R"], c["S"]
    sweep = [{"maxvio": base["maxvio"], "ms_per_step": base["ms_per_step"],
              "GBps": round(base["value"], 1), "tokens_per_s": base["tokens_per_s"],
              "plan_us": base["plan_us"], "slots_used": base["slots_used"],
              "routes_in_slots": base["routes_in_slots"]}]

    def with_prefetch(point, plan):
        if wb is not None:
            t = wb.prefetch(moon, plan, stream, 5)[0]
            point["prefetch_weight_us"] = round(t, 2)
            point["ms_per_step_with_weight_prefetch"] = round(point["ms_per_step"] + t * 1e-3, 4)

    with_prefetch(sweep[0], base_plan)
    sc, levels = SWEEPS[config]
    for level in levels:
        target = synth.LEVELS[synth.workload_id(sc)][level]
        log(f"[bench] maxvio level {target}")
        s4 = [Inputs(moon, ctx, sc, synth.seed_of(sc, level), synth.alpha_for(sc, level), dev),
              Inputs(moon, ctx, sc, synth.seed_of(sc, level) + 500, synth.alpha_for(sc, level),
                     dev)]
        ms4, _, calls4, _ = run_steps(moon, ctx, s4, steps, warmup, stream)
        b4 = [algorithmic_bytes(moon, ctx, s.plan) for s in s4]
        by4 = 0.5 * sum(b["dispatch"] + b["combine"] for b in b4)
        sweep.append({"maxvio": round(s4[0].maxvio, 4), "target": target,
                      "ms_per_step": round(ms4, 4), "GBps": round(by4 / (ms4 * 1e-3) / 1e9, 1),
                      "tokens_per_s": round(R * S / (ms4 * 1e-3)),
                      "plan_us": round(calls4["plan"], 2),
                      "dispatch_us": round(calls4["dispatch"], 2),
                      "combine_us": round(calls4["combine"], 2),
                      "slots_used": b4[0]["slots_used"],
                      "routes_in_slots": b4[0]["routes_in_slots"]})
        with_prefetch(sweep[-1], s4[0].plan)
        for s in s4:
            moon.moon_plan_destroy(s.plan)
        del s4
    times = [p["ms_per_step"] for p in sweep]
    return sweep, round(max(times) / min(times), 4)


def release(moon, ctx, sets):
    import torch
    for s in sets:
        moon.moon_plan_destroy(s.plan)
    moon.moon_ctx_destroy(ctx)
    sets.clear()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=["r16-e384-k8", "dsv3", "r8-e64-k6"])
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary r8-e64-k6 section")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step only: no ceilings, ablations, sweep, secondary section "
                         "or CPU baseline (the counter runs use this)")
    ap.add_argument("--ceilings-only", action="store_true",
                    help="the step and the memory-system ceiling legs only (the stall-counter "
                         "runs use this)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate", action="store_true",
                    help="run only a plain 1 GiB elementwise copy (scales HBM counters)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar="DIR",
                    help="rocprofv3 csv folders: FETCH_SIZE run, WRITE_SIZE run, and the same two "
                         "for --calibrate; writes profiles/pmc_<workload>.{json,md}")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="rocprofv3 --kernel-trace --stats csv folder; writes "
                         "profiles/kernels_<workload>.md")
    ap.add_argument("--commands", nargs="*", default=[],
                    help="the profiler commands, recorded in the summary")
    ap.add_argument("--bench-log", help="log of the traced run (its JSON line is quoted)")
    ap.add_argument("--summarize-stalls", nargs=2, metavar="DIR",
                    help="rocprofv3 csv folders of the two memory-queue counter passes of a "
                         "--ceilings-only run; writes profiles/stalls_<workload>.md")
    args = ap.parse_args()
    if args.summarize_pmc or args.summarize_trace or args.summarize_stalls:
        import synth
        name = synth.WORKLOADS[synth.workload_id(args.workload)]["name"]
        if args.summarize_pmc:
            summarize_pmc(name, args.summarize_pmc, args.commands)
        elif args.summarize_stalls:
            summarize_stalls(name, args.summarize_stalls, args.commands)
        else:
            summarize_trace(name, args.summarize_trace, " ".join(args.commands), args.bench_log)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the library emulates "
              "the R expert-parallel ranks as windows of one GPU's memory and has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate:
        n = 1 << 30
        a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            torch.add(a, 0.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate": "torch.add(a, 0, out=b)", "bytes_read": n,
                          "bytes_written": n, "launches": 5}), flush=True)
        return

    import combine_balanced_planning_amd as moon
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    config = args.workload
    full = not args.step_only
    head, ctx, sets, nb0 = measure_step(moon, config, dev, stream, args.steps, args.warmup)

    ceilings = ablations = weights = serving = copy = cpu = secondary = None
    sweep, flat = [], None
    iters = max(10, args.steps // 5)
    if args.ceilings_only:
        ceilings = measure_ceilings(moon, ctx, sets[0], nb0, stream, max(3, args.steps))
        release(moon, ctx, sets)
    elif full:
        log("[bench] memory-system ceilings")
        ceilings = measure_ceilings(moon, ctx, sets[0], nb0, stream, iters)
        copy = measure_copy(stream)
        k = head["kernels"]
        k["k_dispatch_scatter"]["write_rows_us_over_launch_us"] = round(
            ceilings["write_rows"]["us"] / k["k_dispatch_scatter"]["avg_launch_us"], 4)
        k["k_combine_staged"]["read_rows_us_over_launch_us"] = round(
            ceilings["read_rows"]["us"] / k["k_combine_staged"]["avg_launch_us"], 4)
        # Sum of the parts, each at the rate the memory system gives it alone:
        # dispatch = its token-row reads at the contiguous read rate + the
        # rest (route rows, padding, weights) at the row-write rate; combine
        # = its output at the contiguous fill rate + the rest (route rows,
        # dst, weights) at the row-read rate.
        rate = {n: v["bytes"] / v["us"] for n, v in ceilings.items()}  # bytes per µs
        tok_bytes = 2 * head["H"] * head["R"] * head["S"]
        t_d = tok_bytes / rate["read"] + (nb0["dispatch"] - tok_bytes) / rate["write_rows"]
        t_c = tok_bytes / rate["fill"] + (nb0["combine"] - tok_bytes) / rate["read_rows"]
        for kn, t in (("k_dispatch_scatter", t_d), ("k_combine_staged", t_c)):
            k[kn]["sum_of_parts_us"] = round(t, 2)
            k[kn]["sum_of_parts_over_launch_us"] = round(t / k[kn]["avg_launch_us"], 4)
        for kk in k.values():
            kk["frac_of_measured_copy"] = round(kk["achieved"] / ceilings["copy"]["GBps"], 4)
        log("[bench] ablations")
        ablations = measure_ablations(moon, ctx, sets[0], nb0, stream, iters)
        wb = None
        if config in FFN_WIDTH:
            log("[bench] gradient reduction and weight prefetch")
            weights = measure_weights(moon, ctx, sets[0], stream, max(5, args.steps // 10),
                                      FFN_WIDTH[config])
            wb = WeightBufs(ctx, FFN_WIDTH[config])
        if not args.no_sweep and config in SWEEPS:
            sweep, flat = measure_sweep(moon, ctx, config, head, max(10, args.steps // 2),
                                        args.warmup, stream, dev, wb, sets[0].plan)
        if wb is not None:
            wb.release()
            del wb
        topk_h, w_h, seed0 = sets[0].topk_h, sets[0].w_h, sets[0].seed
        release(moon, ctx, sets)
        if not args.no_secondary and config != SECONDARY:
            sec, sctx, ssets, _ = measure_step(moon, SECONDARY, dev, stream, args.steps,
                                               args.warmup)
            secondary = dict(sec, cache_affected=True)
            secondary["value"] = round(secondary["value"], 1)
            secondary["pct_of_hbm_peak"] = round(100 * sec["value"] / PEAK_HBM_GBPS, 2)
            log("[bench] weight prefetch and gradient reduction (secondary)")
            secondary["weights"] = measure_weights(moon, sctx, ssets[0], stream,
                                                   max(5, args.steps // 10),
                                                   FFN_WIDTH[SECONDARY])
            if not args.no_sweep:
                secondary["maxvio_sweep"], secondary["sweep_max_over_min_time"] = measure_sweep(
                    moon, sctx, SECONDARY, sec, max(10, args.steps // 2), args.warmup, stream,
                    dev)
            release(moon, sctx, ssets)
        if config == SECONDARY or not args.no_secondary:
            log("[bench] padded serving workload")
            serving = measure_serving(moon, dev, stream, max(10, args.steps // 5), 3)
        if not args.no_cpu_baseline:
            log("[bench] cpu baseline (oracle)")
            cpu = cpu_baseline(config, topk_h, w_h, seed0, args.cpu_budget)
    else:
        release(moon, ctx, sets)

    line = {
        "metric": METRIC, "value": round(head["value"], 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded routing, bf16 N(0,1) activations)",
        "config": {"workload": head["workload"], "R": head["R"], "E": head["E"],
                   "K": head["K"], "S": head["S"], "H": head["H"],
                   "token_padding": head["token_padding"], "B": head["B"],
                   "maxvio": head["maxvio"], "global_batch": head["R"] * head["S"],
                   "parallelism": "ep emulated as R windows on 1 GPU"},
        "pct_of_hbm_peak": round(100 * head["value"] / PEAK_HBM_GBPS, 2),
        "tokens_per_s": head["tokens_per_s"],
        "dispatch_combine_GBps": head["dispatch_combine_GBps"],
        "tokens_per_s_excl_plan": head["tokens_per_s_excl_plan"],
        "call_us": head["call_us"], "plan_us": head["plan_us"],
        "bytes_per_step": head["bytes_per_step"],
        "slots_used": head["slots_used"], "routes_in_slots": head["routes_in_slots"],
        "maxvio_sweep": sweep, "sweep_max_over_min_time": flat,
        "wall_s_timed": head["wall_s_timed"],
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "ceilings": ceilings,
        "plain_copy": copy,
        "ablations": ablations,
        "weights": weights,
        "secondary": secondary,
        "serving": serving,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
