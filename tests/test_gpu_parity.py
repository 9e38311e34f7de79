"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Plan, cu_seqlens, dispatched rows and weights must match bit for bit; combine
must stay within |d| <= 1e-2 max|ref| + 1e-3 (and within the derived fp32
bound of parity.combine_bound); gathered weights and the prefetch index are
bit-exact.  Everything goes through the C ABI (the package binding).
"""
import zlib

import numpy as np
import pytest

import oracle
import parity as pt
import plan_checks as pc
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_balanced_planning_amd as moon
    return moon, torch.device("cuda", 0)


def say(*a):
    print(*a, flush=True)


def run_full(moon, dev, topk, w, hidden, y, R, E, K, S, H, B, P, dflags=0, weighted=True,
             label="", tpe=None):
    """Plan + dispatch + combine on the GPU with full comparisons to the oracle."""
    import torch
    say(f"[case] {label} R={R} E={E} K={K} S={S} H={H} B={B} P={P} dflags={dflags}")
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        topk_d = pt.to_dev(topk, dev)
        moon.moon_plan(ctx, topk_d, pt.to_dev(tpe, dev) if tpe is not None else None, plan)
        moon.moon_dispatch(ctx, plan, pt.bf16_to_dev(hidden, dev),
                           pt.to_dev(w, dev) if w is not None else None, flags=dflags)
        win, wwin = moon.window_tensors(ctx)
        y_d = pt.bf16_to_dev(y, dev)
        out = torch.empty((R, S, H), dtype=torch.bfloat16, device=dev)
        wsk = torch.empty((R, S, K), dtype=torch.float32, device=dev) if w is not None else None
        moon.moon_combine(ctx, plan, y_d, wwin if w is not None else None,
                          moon.MOON_COMBINE_WEIGHTED if weighted else 0, out, wsk)
        pidx = torch.empty((R, ctx.B, 2), dtype=torch.int32, device=dev)
        moon.moon_prefetch_index(ctx, plan, pidx)
        assert moon.moon_plan_status(plan) == moon.MOON_OK
        got = pt.gpu_plan_arrays(plan)

        ref = oracle.plan(topk, E, ctx.B, P, tpe)
        assert ref.status == oracle.OK and ref.NvS == ctx.NvS
        pt.compare_plan(got, ref)
        pc.check_all(pt.gpu_plan_view(got, ref), topk, dups=R * S <= 4096)

        ewin, ewwin = oracle.dispatch(ref, hidden, w)
        src = oracle.row_sources(ref)
        cov = src != -2
        gwin = pt.dev_bits(win)
        assert np.array_equal(gwin[cov], ewin[cov]), "dispatched rows differ"
        if w is not None:
            assert np.array_equal(wwin.cpu().numpy()[cov].view(np.uint32),
                                  ewwin[cov].view(np.uint32)), "dispatched weights differ"

        eout, ewsk, acc = oracle.combine(ref, y, ewwin, weighted=weighted)
        rows = np.arange(R * ref.NvS)
        absum = pt.abs_sum(ref.dst.reshape(R * S, K), rows, y,
                           ewwin if ewwin is not None else np.zeros(R * ref.NvS, np.float32),
                           weighted).reshape(R, S, H)
        dmax, ndiff = pt.check_combine(pt.dev_bits(out), eout, acc, absum, K)
        say(f"   combine max|d|={dmax:.3g} bf16 mismatches={ndiff}/{eout.size}")
        if w is not None:
            assert np.array_equal(wsk.cpu().numpy().view(np.uint32), ewsk.view(np.uint32))
        assert np.array_equal(pidx.cpu().numpy(), oracle.prefetch_index(ref))
        return ref, got
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


def workload_inputs(config, level=0):
    wl = synth.workload(config, level)
    R, S, H, E, K, B, P = (wl[k] for k in ("R", "S", "H", "E", "K", "B", "P"))
    nvs = oracle.nvs(R, E, K, S, B, P)
    hidden = synth.hidden_bf16(wl["seed"], R, S, H)
    y = synth.y_bf16(wl["seed"], R * nvs, H)
    return wl, hidden, y


@pytest.mark.parametrize("config,level", [("tiny", 0), ("r8-e64-k6", 0)] +
                         [("r8-e64-k6-skewed", lv) for lv in range(4)])
@pytest.mark.parametrize("path", ["fused", "epilogue"])
def test_workload_full_parity(env, config, level, path):
    """The default one-pass dispatch and the pages' two-pass (epilogue)
    structure, each against the oracle in full."""
    moon, dev = env
    wl, hidden, y = workload_inputs(config, level)
    say(f"[workload] {wl['name']} level {level} maxvio={wl['maxvio']:.3f} {path}")
    run_full(moon, dev, wl["topk"], wl["w"], hidden, y, wl["R"], wl["E"], wl["K"], wl["S"],
             wl["H"], wl["B"], wl["P"], label=wl["name"],
             dflags=moon.MOON_DISPATCH_DEDUP_EPILOGUE if path == "epilogue" else 0,
             weighted=level % 2 == 0)


@pytest.mark.parametrize("config", ["tiny", "r8-e64-k6"])
@pytest.mark.parametrize("path", ["fused", "epilogue"])
def test_workload_unweighted_full_parity(env, config, path):
    """The same two workloads without route weights: dispatch leaves the
    weight window alone and combine is the plain K-sum."""
    moon, dev = env
    wl, hidden, y = workload_inputs(config, 0)
    say(f"[workload] {wl['name']} unweighted {path}")
    run_full(moon, dev, wl["topk"], None, hidden, y, wl["R"], wl["E"], wl["K"], wl["S"],
             wl["H"], wl["B"], wl["P"], label=wl["name"] + " unweighted",
             dflags=moon.MOON_DISPATCH_DEDUP_EPILOGUE if path == "epilogue" else 0,
             weighted=False)


def _edge_topk(rng, R, S, K, E, mode):
    if mode == "uniform":
        return np.stack([rng.permutation(E)[:K] for _ in range(R * S)]).reshape(R, S, K).astype(
            np.int32)
    if mode == "skewed":
        p = 1.0 / np.arange(1, E + 1) ** 2.0
        p /= p.sum()
        return np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(R * S)]).reshape(
            R, S, K).astype(np.int32)
    if mode == "repeats":  # ids may repeat inside a token; a third of tokens all expert 0
        t = rng.integers(0, E, size=(R, S, K)).astype(np.int32)
        t[:, ::3, :] = 0
        return t
    if mode == "one_expert":
        return np.zeros((R, S, K), np.int32) + (E - 1)
    if mode == "home_block":  # every token picks its K experts inside one rank
        Eg = E // R
        h = rng.integers(0, R, size=R * S)
        return np.stack([h[i] * Eg + rng.choice(Eg, K, replace=Eg < K)
                         for i in range(R * S)]).reshape(R, S, K).astype(np.int32)
    raise ValueError(mode)


EDGE = [
    # label, R, E, K, S, H, B, P, mode
    ("single-rank", 1, 8, 2, 100, 64, 0, 4, "uniform"),
    ("top1", 4, 16, 1, 130, 32, 0, 8, "skewed"),
    ("ragged-tiles", 3, 12, 3, 1000, 24, 0, 5, "skewed"),
    ("one-expert-per-rank", 4, 4, 2, 64, 16, 0, 2, "repeats"),
    ("no-padding", 4, 16, 4, 77, 16, 0, 1, "skewed"),
    ("min-width", 2, 8, 2, 33, 8, 0, 4, "uniform"),
    ("wide-rows", 2, 8, 2, 40, 8192, 0, 16, "uniform"),
    ("dsv3-rows", 2, 16, 4, 40, 7168, 0, 8, "skewed"),
    ("repeated-ids", 4, 8, 4, 50, 64, 0, 4, "repeats"),
    ("all-one-expert", 2, 8, 3, 64, 32, 0, 8, "one_expert"),
    ("home-block-dedup", 4, 32, 8, 96, 64, 0, 16, "home_block"),
    ("many-ranks", 32, 64, 3, 40, 16, 0, 4, "skewed"),
    ("k16", 4, 64, 16, 50, 16, 0, 4, "uniform"),
    ("k64", 2, 8, 64, 9, 8, 0, 4, "repeats"),
    ("b-small-ok", 4, 16, 2, 64, 16, 1, 4, "uniform"),
    ("large-e", 8, 512, 8, 128, 16, 0, 8, "skewed"),
    ("max-tiles-e512", 32, 512, 8, 1024, 16, 0, 4, "skewed"),  # 256 planner tiles
    ("max-width", 2, 8, 3, 12, 65536, 0, 4, "repeats"),  # the widest rows accepted
    # 18 chunks per planner wave: more than a wave stages in LDS at once
    ("long-waves", 2, 16, 64, 35000, 8, 0, 4, "repeats"),
]


@pytest.mark.parametrize("path", ["fused", "epilogue"])
@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_shapes(env, case, path):
    moon, dev = env
    label, R, E, K, S, H, B, P, mode = case
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    topk = _edge_topk(rng, R, S, K, E, mode)
    Bx = B if B > 0 else E // R
    ref = oracle.plan(topk, E, Bx, P)
    if ref.status == oracle.SLOT_BUDGET:
        pytest.skip("this routing needs more slots than B")
    w = rng.random((R, S, K)).astype(np.float32)
    hidden = synth.bf16_normal(rng.integers(1 << 62), 0, R * S * H).reshape(R, S, H)
    y = synth.bf16_normal(rng.integers(1 << 62), 0, R * ref.NvS * H).reshape(R * ref.NvS, H)
    run_full(moon, dev, topk, w, hidden, y, R, E, K, S, H, B, P, label=f"{label} {path}",
             dflags=moon.MOON_DISPATCH_DEDUP_EPILOGUE if path == "epilogue" else 0)


def test_fused_duplicates_and_unweighted_round_trip(env):
    """The default dispatch, the explicit FUSED_DUPS flag and the epilogue
    flag write the same windows; unweighted combine of the dispatched windows
    gives K * x exactly (closed form); both flags at once are refused."""
    import torch
    moon, dev = env
    wl, hidden, _ = workload_inputs("r8-e64-k6")
    R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    say(f"[case] fused + round trip {wl['name']}")
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        moon.moon_plan(ctx, pt.to_dev(wl["topk"], dev), None, plan)
        h_d = pt.bf16_to_dev(hidden, dev)
        moon.moon_dispatch(ctx, plan, h_d, None, flags=moon.MOON_DISPATCH_DEDUP_EPILOGUE)
        win, _ = moon.window_tensors(ctx)
        a = win.clone()
        for fl in (0, moon.MOON_DISPATCH_FUSED_DUPS):
            win.zero_()
            moon.moon_dispatch(ctx, plan, h_d, None, flags=fl)
            assert torch.equal(a.view(torch.int16), win.view(torch.int16)), fl
        with pytest.raises(moon.MoonError) as ei:
            moon.moon_dispatch(ctx, plan, h_d, None, flags=moon.MOON_DISPATCH_FUSED_DUPS |
                               moon.MOON_DISPATCH_DEDUP_EPILOGUE)
        assert ei.value.status == moon.MOON_ERR_INVALID_ARG
        out = torch.empty((R, S, H), dtype=torch.bfloat16, device=dev)
        moon.moon_combine(ctx, plan, win, None, 0, out)
        exp = (K * h_d.float()).to(torch.bfloat16)  # K*x is exact in fp32
        assert torch.equal(out.view(torch.int16), exp.view(torch.int16))
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


# bf16 bit patterns of the special values (column j of every expert-output
# row gets special value j): +Inf, -Inf, a NaN, -0, the smallest subnormals of
# both signs, a mid subnormal, the largest finite value and its negative.
SPECIAL_BF16 = np.array([0x7F80, 0xFF80, 0x7FC1, 0x8000, 0x0001, 0x8001, 0x0040, 0x7F7F,
                         0xFF7F], np.uint16)


@pytest.mark.parametrize("flags", ["weighted", "plain", "prologue"])
def test_combine_special_values(env, flags):
    """Expert outputs holding infinities, a NaN, -0, bf16 subnormals and the
    largest finite values, with some tokens mixing +Inf and -Inf: the
    combine's fp32 sum rounded to bf16 equals the oracle's bit for bit (any
    NaN becomes 0x7FC0, overflow becomes an infinity, subnormal products are
    kept, not flushed)."""
    import torch
    moon, dev = env
    rng = np.random.default_rng(4242)
    R, E, K, S, H, B, P = 2, 8, 4, 96, 64, 0, 4
    topk = np.stack([rng.permutation(E)[:K] for _ in range(R * S)]).reshape(R, S, K).astype(
        np.int32)
    w = rng.random((R, S, K)).astype(np.float32)
    w[:, ::5, 1] = 0.0  # zero weights meet infinities: 0 * Inf is NaN
    ref = oracle.plan(topk, E, E // R, P)
    hidden = synth.bf16_normal(1234, 0, R * S * H).reshape(R, S, H)
    y = synth.bf16_normal(5678, 0, R * ref.NvS * H).reshape(R * ref.NvS, H).copy()
    ns = SPECIAL_BF16.size
    y[:, :ns] = SPECIAL_BF16
    # columns ns..: every other row +Inf, the rest -Inf or subnormal, so a
    # token's K rows mix them in route order
    y[0::2, ns] = 0x7F80
    y[1::2, ns] = 0xFF80
    y[0::3, ns + 1] = 0x0003
    y[1::3, ns + 1] = 0x8002
    y[2::3, ns + 1] = 0x7F7F
    say(f"[case] special values {flags}")
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        moon.moon_plan(ctx, pt.to_dev(topk, dev), None, plan)
        moon.moon_dispatch(ctx, plan, pt.bf16_to_dev(hidden, dev), pt.to_dev(w, dev))
        _, wwin = moon.window_tensors(ctx)
        _, ewwin = oracle.dispatch(ref, hidden, w)
        out = torch.empty((R, S, H), dtype=torch.bfloat16, device=dev)
        if flags == "prologue":
            fl = moon.MOON_COMBINE_DUP_PROLOGUE | moon.MOON_COMBINE_WEIGHTED
            eout = oracle.combine_prologue(ref, y, ewwin, weighted=True)[0]
        else:
            fl = moon.MOON_COMBINE_WEIGHTED if flags == "weighted" else 0
            eout = oracle.combine(ref, y, ewwin, weighted=flags == "weighted", exact=False)[0]
        moon.moon_combine(ctx, plan, pt.bf16_to_dev(y, dev), wwin, fl, out)
        assert moon.moon_plan_status(plan) == moon.MOON_OK
        got = pt.dev_bits(out)
        bad = np.argwhere(got != eout)
        assert bad.size == 0, (f"{len(bad)} outputs differ, first at {bad[0].tolist()}: "
                               f"{got[tuple(bad[0])]:#06x} vs {eout[tuple(bad[0])]:#06x}")
        # the special columns did produce special results
        assert (got[..., 2] == 0x7FC0).all()  # a NaN in every routed row
        assert ((got[..., ns] & 0x7FFF) >= 0x7F80).any()
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


def test_clone_repeat_and_backward_reuse(env):
    """A plan is bit-reproducible, clone() copies it, and dispatching a second
    tensor with an existing plan (the backward path) needs no new planning."""
    import torch
    moon, dev = env
    wl, hidden, _ = workload_inputs("tiny")
    R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    p1, p2 = moon.moon_plan_create(ctx), moon.moon_plan_create(ctx)
    try:
        t = pt.to_dev(wl["topk"], dev)
        moon.moon_plan(ctx, t, None, p1)
        moon.moon_plan(ctx, t, None, p2)
        a, b = pt.gpu_plan_arrays(p1), pt.gpu_plan_arrays(p2)
        for k in a:
            if k not in ("dup_groups", "dup_loffs"):
                assert np.array_equal(a[k], b[k])
        c = moon.moon_plan_clone(p1)
        torch.cuda.synchronize()
        cc = pt.gpu_plan_arrays(c)
        for k in a:
            assert np.array_equal(a[k], cc[k])
        # backward: a gradient dispatched with the saved plan
        g = synth.bf16_normal(77, 0, R * S * H).reshape(R, S, H)
        out = torch.zeros((R * ctx.NvS, H), dtype=torch.bfloat16, device=dev)
        moon.moon_dispatch(ctx, c, pt.bf16_to_dev(g, dev), None, hidden_out=out)
        ref = oracle.plan(wl["topk"], E, B, P)
        ewin, _ = oracle.dispatch(ref, g, None)
        cov = oracle.row_sources(ref) != -2
        assert np.array_equal(pt.dev_bits(out)[cov], ewin[cov])
        moon.moon_plan_destroy(c)
    finally:
        moon.moon_plan_destroy(p1)
        moon.moon_plan_destroy(p2)
        moon.moon_ctx_destroy(ctx)


def test_two_contexts_on_two_streams(env):
    """Contexts are independent: two of them, each planning, dispatching and
    combining on its own stream (default priority) at the same time, give the
    oracle's results, call after call."""
    import torch
    moon, dev = env
    shapes = [(4, 32, 4, 300, 64, 0, 4), (8, 64, 6, 160, 32, 0, 16)]
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    runs = []
    for n, (R, E, K, S, H, B, P) in enumerate(shapes):
        rng = np.random.default_rng(900 + n)
        ins = []
        for rep in range(2):
            topk = _edge_topk(rng, R, S, K, E, "skewed" if rep else "uniform")
            w = rng.random((R, S, K)).astype(np.float32)
            hidden = synth.bf16_normal(int(rng.integers(1 << 62)), 0, R * S * H).reshape(R, S, H)
            ins.append((topk, w, hidden))
        ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
        y = synth.bf16_normal(int(rng.integers(1 << 62)), 0, R * ctx.NvS * H).reshape(
            R * ctx.NvS, H)
        runs.append(dict(ctx=ctx, plan=moon.moon_plan_create(ctx), ins=ins, y=y,
                         dev=[(pt.to_dev(t, dev), pt.to_dev(w, dev), pt.bf16_to_dev(h, dev))
                              for t, w, h in ins],
                         y_d=pt.bf16_to_dev(y, dev),
                         out=torch.empty((R, S, H), dtype=torch.bfloat16, device=dev),
                         shape=(R, E, K, S, H, B, P)))
    torch.cuda.synchronize()
    say("[case] two contexts on two streams")
    try:
        for it in range(6):
            for n, r in enumerate(runs):  # issue both before waiting on either
                t_d, w_d, h_d = r["dev"][it % 2]
                st = streams[n]
                moon.moon_plan(r["ctx"], t_d, None, r["plan"], stream=st)
                moon.moon_dispatch(r["ctx"], r["plan"], h_d, w_d, stream=st)
                _, wwin = moon.window_tensors(r["ctx"])
                moon.moon_combine(r["ctx"], r["plan"], r["y_d"], wwin, moon.MOON_COMBINE_WEIGHTED,
                                  r["out"], stream=st)
            for n, r in enumerate(runs):
                R, E, K, S, H, B, P = r["shape"]
                assert moon.moon_plan_status(r["plan"], streams[n]) == moon.MOON_OK
                topk, w, hidden = r["ins"][it % 2]
                ref = oracle.plan(topk, E, r["ctx"].B, P)
                pt.compare_plan(pt.gpu_plan_arrays(r["plan"]), ref)
                win, wwin = moon.window_tensors(r["ctx"])
                ewin, ewwin = oracle.dispatch(ref, hidden, w)
                cov = oracle.row_sources(ref) != -2
                assert np.array_equal(pt.dev_bits(win)[cov], ewin[cov]), (it, n)
                eout, _, _ = oracle.combine(ref, r["y"], ewwin, weighted=True)
                assert np.array_equal(pt.dev_bits(r["out"]), eout), (it, n)
    finally:
        for r in runs:
            moon.moon_plan_destroy(r["plan"])
            moon.moon_ctx_destroy(r["ctx"])


@pytest.mark.parametrize("what", ["bad_high", "bad_negative", "bad_minus2", "bad_int_min",
                                  "histogram", "slot_budget", "not_planned", "tpe_ok"])
def test_device_status_and_skip(env, what):
    """Data errors set the plan status; later kernels write nothing."""
    import torch
    moon, dev = env
    R, E, K, S, H, P = 2, 8, 2, 8, 16, 2
    B = 4
    topk = np.tile(np.array([[0, 1], [2, 3], [4, 5], [6, 7]], np.int32), (R, 2, 1))
    tpe = None
    expect = moon.MOON_OK
    if what == "bad_high":
        topk[1, 3, 1] = E
        expect = moon.MOON_ERR_BAD_EXPERT
    elif what == "bad_negative":
        topk[0, 0, 0] = -1
        expect = moon.MOON_ERR_BAD_EXPERT
    elif what == "bad_minus2":
        topk[1, 5, 0] = -2
        expect = moon.MOON_ERR_BAD_EXPERT
    elif what == "bad_int_min":
        topk[0, 7, 1] = np.iinfo(np.int32).min
        expect = moon.MOON_ERR_BAD_EXPERT
    elif what in ("histogram", "tpe_ok"):
        tpe = np.stack([np.bincount(topk[r].reshape(-1), minlength=E) for r in range(R)]).astype(
            np.int32)
        if what == "histogram":
            tpe[1, 2] += 1
            expect = moon.MOON_ERR_HISTOGRAM
    elif what == "slot_budget":
        topk = np.array([0] * 16 + [1] * 6 + [2] * 5 + [3] * 5, np.int32).reshape(R, S, K)
        B = 2
        expect = moon.MOON_ERR_SLOT_BUDGET
    elif what == "not_planned":
        expect = moon.MOON_ERR_NOT_PLANNED
    say(f"[case] status {what}")
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        if what != "not_planned":
            moon.moon_plan(ctx, pt.to_dev(topk, dev),
                           pt.to_dev(tpe, dev) if tpe is not None else None, plan)
        win, wwin = moon.window_tensors(ctx)
        win.fill_(3.0)
        wwin.fill_(5.0)
        hidden = torch.ones((R, S, H), dtype=torch.bfloat16, device=dev)
        moon.moon_dispatch(ctx, plan, hidden, torch.ones((R, S, K), device=dev))
        out = torch.full((R, S, H), 7.0, dtype=torch.bfloat16, device=dev)
        moon.moon_combine(ctx, plan, win, wwin, moon.MOON_COMBINE_WEIGHTED, out)
        st = moon.moon_plan_status(plan)
        assert st == expect, moon.moon_status_str(st)
        if expect != moon.MOON_OK:
            assert bool((win.float() == 3.0).all()) and bool((wwin == 5.0).all())
            assert bool((out.float() == 7.0).all())
        assert oracle.plan(topk, E, B, P, tokens_per_expert=tpe).status == \
            {moon.MOON_OK: 0, moon.MOON_ERR_BAD_EXPERT: -7, moon.MOON_ERR_HISTOGRAM: -9,
             moon.MOON_ERR_SLOT_BUDGET: -8, moon.MOON_ERR_NOT_PLANNED: 0}[expect]
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


@pytest.mark.parametrize("R,E,K,S", [(32, 512, 8, 1024), (8, 256, 8, 256), (3, 12, 3, 1000)],
                         ids=["256-tiles", "16-tiles", "ragged"])
def test_histogram_check_every_expert(env, R, E, K, S):
    """tokens_per_expert is checked for every (rank, expert): a plan with the
    true histogram equals the oracle's; moving one route's count between two
    experts of one rank, anywhere in the matrix, gives HISTOGRAM."""
    import torch
    moon, dev = env
    rng = np.random.default_rng(zlib.crc32(f"hist-{R}-{E}".encode()))
    topk = _edge_topk(rng, R, S, K, E, "skewed")
    tpe = np.stack([np.bincount(topk[r].reshape(-1), minlength=E) for r in range(R)]).astype(
        np.int32)
    H, P = 16, 4
    hidden = synth.bf16_normal(int(rng.integers(1 << 62)), 0, R * S * H).reshape(R, S, H)
    nvs = oracle.nvs(R, E, K, S, E // R, P)
    y = synth.bf16_normal(int(rng.integers(1 << 62)), 0, R * nvs * H).reshape(R * nvs, H)
    run_full(moon, dev, topk, None, hidden, y, R, E, K, S, H, 0, P, weighted=False,
             label=f"histogram given R={R} E={E}", tpe=tpe)
    ctx = moon.moon_ctx_create(R, E, K, S, H, 0, P)
    plan = moon.moon_plan_create(ctx)
    try:
        topk_d = pt.to_dev(topk, dev)
        spots = sorted({(r, e) for r in (0, R // 2, R - 1)
                        for e in (0, 15, 16, 17, E // 2, E - 17, E - 1) if 0 <= e < E})
        say(f"[case] histogram perturbations R={R} E={E}: {len(spots)}")
        for r, e in spots:
            bad = tpe.copy()
            bad[r, e] += 1
            bad[r, (e + 1) % E] -= 1
            moon.moon_plan(ctx, topk_d, pt.to_dev(bad, dev), plan)
            st = moon.moon_plan_status(plan)
            assert st == moon.MOON_ERR_HISTOGRAM, (r, e, moon.moon_status_str(st))
        moon.moon_plan(ctx, topk_d, pt.to_dev(tpe, dev), plan)
        assert moon.moon_plan_status(plan) == moon.MOON_OK
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


def test_call_tag_wraps(env):
    """Tiles exchange duplicate counts in words tagged with the low 16 bits of
    a per-context call counter; planning past the point where the tag wraps
    still gives the oracle's plan, call after call."""
    moon, dev = env
    R, E, K, S, H, B, P = 2, 8, 2, 300, 8, 0, 4  # two tiles per rank
    rng = np.random.default_rng(4242)
    topks = [_edge_topk(rng, R, S, K, E, m) for m in ("uniform", "repeats")]
    refs = [oracle.plan(t, E, E // R, P) for t in topks]
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        ts = [pt.to_dev(t, dev) for t in topks]
        say("[case] call tag wrap: 65540 planning calls")
        for i in range(65540):
            moon.moon_plan(ctx, ts[i % 2], None, plan)
            if i >= 65530 or i < 2:
                assert moon.moon_plan_status(plan) == moon.MOON_OK, i
                pt.compare_plan(pt.gpu_plan_arrays(plan), refs[i % 2])
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


def test_plan_mismatch_is_rejected(env):
    moon, dev = env
    c1 = moon.moon_ctx_create(2, 8, 2, 8, 16, 4, 2)
    c2 = moon.moon_ctx_create(2, 8, 2, 8, 16, 4, 2)
    p = moon.moon_plan_create(c1)
    try:
        import torch
        with pytest.raises(moon.MoonError) as ei:
            moon.moon_plan(c2, torch.zeros((2, 8, 2), dtype=torch.int32, device=dev), None, p)
        assert ei.value.status == moon.MOON_ERR_PLAN_MISMATCH
    finally:
        moon.moon_plan_destroy(p)
        moon.moon_ctx_destroy(c1)
        moon.moon_ctx_destroy(c2)


@pytest.mark.parametrize("name", ["alias_worked_example.json", "alias_served_order.json"])
def test_hand_worked_examples(env, name):
    """The hand-worked balance examples (tests/golden) through the GPU planner:
    slots and group sizes as worked out on paper, everything else as the oracle."""
    import json
    import os
    moon, dev = env
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        g = json.load(f)
    R, E, B, K = g["R"], g["E"], g["B"], 2
    S, P, H = g["C"] // K, 4, 64
    routes = np.repeat(np.arange(E), g["T"]).astype(np.int32)
    topk = routes[np.random.default_rng(9).permutation(routes.shape[0])].reshape(R, S, K)
    rng = np.random.default_rng(10)
    w = rng.random((R, S, K)).astype(np.float32)
    hidden = synth.bf16_normal(synth.stream_key(77, synth.TAG_HIDDEN), 0, R * S * H).reshape(R, S, H)
    nvs = oracle.nvs(R, E, K, S, B, P)
    y = synth.bf16_normal(synth.stream_key(77, synth.TAG_Y), 0, R * nvs * H).reshape(R * nvs, H)
    ref, got = run_full(moon, dev, topk, w, hidden, y, R, E, K, S, H, B, P, label=name)
    assert got["experts_to_copy"].tolist() == g["experts_to_copy"]
    start, n, end = pc.group_table(pt.gpu_plan_view(got, ref))
    assert n.tolist() == g["n"]


def _random_case(i):
    """A seeded random valid configuration: R, E = R * E/R, K, S, H (multiple
    of 8, often not of 512 so slices end ragged), P, B (sometimes below E/R)
    and a routing mode."""
    rng = np.random.default_rng(1000 + i)
    R = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 32]))
    Eg = int(rng.integers(1, max(2, 512 // R // 4) + 1))
    E = R * Eg
    K = int(rng.integers(1, min(16, 64) + 1)) if rng.random() < 0.85 else int(rng.integers(17, 65))
    S = int(rng.integers(1, 161))
    H = 8 * int(rng.choice([1, 2, 17, 64, 65, 300, 896]))
    P = int(rng.choice([1, 2, 3, 8, 16, 33]))
    B = 0 if rng.random() < 0.7 else int(rng.integers(1, Eg + 1))
    mode = str(rng.choice(["uniform", "skewed", "repeats", "home_block"]))
    if mode in ("uniform", "skewed") and K > E:
        mode = "repeats"
    return R, E, K, S, H, B, P, mode


@pytest.mark.parametrize("i", range(40))
def test_random_shapes(env, i):
    """Seeded random shapes and routings, compared with the oracle in full;
    when B < E/R makes the plan infeasible, the status must agree."""
    moon, dev = env
    R, E, K, S, H, B, P, mode = _random_case(i)
    rng = np.random.default_rng(2000 + i)
    topk = _edge_topk(rng, R, S, K, E, mode)
    Bx = B if B > 0 else E // R
    ref = oracle.plan(topk, E, Bx, P)
    if ref.status == oracle.SLOT_BUDGET:
        say(f"[case] random {i}: R={R} E={E} K={K} S={S} B={B} -> slot budget")
        ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
        plan = moon.moon_plan_create(ctx)
        try:
            moon.moon_plan(ctx, pt.to_dev(topk, dev), None, plan)
            assert moon.moon_plan_status(plan) == moon.MOON_ERR_SLOT_BUDGET
        finally:
            moon.moon_plan_destroy(plan)
            moon.moon_ctx_destroy(ctx)
        return
    assert ref.status == oracle.OK
    w = rng.random((R, S, K)).astype(np.float32)
    hidden = synth.bf16_normal(int(rng.integers(1 << 62)), 0, R * S * H).reshape(R, S, H)
    y = synth.bf16_normal(int(rng.integers(1 << 62)), 0, R * ref.NvS * H).reshape(R * ref.NvS, H)
    run_full(moon, dev, topk, w, hidden, y, R, E, K, S, H, B, P, label=f"random-{i}-{mode}",
             weighted=bool(i % 3), dflags=moon.MOON_DISPATCH_DEDUP_EPILOGUE if i % 2 else 0)
