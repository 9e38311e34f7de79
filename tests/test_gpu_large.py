"""GPU parity at the full workload sizes, in the launch configuration the
benchmark uses.

The whole plan (dst, layout, slots, duplicate records, prefetch index) is
compared bit for bit with the oracle.  Bulk inputs are filled on the GPU by
the seeded generator (the fill itself is checked against the host generator
first) and the rows a comparison needs are regenerated on the host:

* DSv3 shape: every covered row of every rank window (routed rows against
  their token's row, padding rows against zero) and the weight windows in
  full, for the default one-pass dispatch and for the pages' two-pass
  structure (whose epilogue reads the primaries with non-temporal loads at
  this size); combine over every token of one source rank.
* R=16 shape at maxvio 8: every covered row of all sixteen rank windows
  (one-pass dispatch) and the window of the rank with the most slots (the
  two-pass path), and combine over every token of one source rank; the other
  maxvio levels on sampled rows and tokens.
* Without route weights (DSv3 in full, R=16 at maxvio 4 sampled): the weight
  windows stay untouched and combine is the plain K-sum.
"""
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


def sample_rows(rng, ref, src, n_routes=2048, n_groups=4):
    """Window rows to check: random route rows, whole groups (with padding),
    and the first and last used row of every rank."""
    R, NvS, EB = ref.R, ref.NvS, ref.E + ref.B
    covered = np.nonzero(src >= 0)[0]
    rows = set(rng.choice(covered, size=min(n_routes, covered.shape[0]), replace=False).tolist())
    for _ in range(n_groups):
        u, g = int(rng.integers(R)), int(rng.integers(EB))
        start = 0 if g == 0 else int(ref.cu_seqlens[u, g - 1])
        rows.update(range(u * NvS + start, u * NvS + int(ref.cu_seqlens[u, g])))
    for u in range(R):
        end = int(ref.cu_seqlens[u, -1])
        rows.update([u * NvS, u * NvS + max(end - 1, 0)])
        zr = ref.zero_fill_ranges[u]
        pad = np.nonzero(zr[:, 1] > zr[:, 0])[0]
        if pad.shape[0]:
            g = int(pad[-1])
            rows.update(range(u * NvS + int(zr[g, 0]), u * NvS + int(zr[g, 1])))
    return np.array(sorted(rows), np.int64)


class Run:
    """Plan + dispatch + combine of one full-size workload on the GPU, and the
    oracle's plan of the same routing (compared bit for bit)."""

    def __init__(self, moon, dev, config, level, dflags, weighted=True):
        import torch

        import synth.gpu as sg
        wl = synth.workload(config, level)
        self.wl = wl
        R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
        self.R, self.E, self.K, self.S, self.H = R, E, K, S, H
        seed = wl["seed"]
        say(f"[case] {wl['name']} level {level} maxvio={wl['maxvio']:.3f} R={R} E={E} K={K} "
            f"S={S} H={H} dflags={dflags}")
        self.ctx = ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
        self.plan = plan = moon.moon_plan_create(ctx)
        NvS = ctx.NvS
        self.hidden = sg.hidden(seed, R, S, H, dev)
        self.y = sg.y(seed, R * NvS, H, dev)
        self.kh = synth.stream_key(seed, synth.TAG_HIDDEN)
        self.ky = synth.stream_key(seed, synth.TAG_Y)
        rng = np.random.default_rng(seed)
        self.rng = rng
        # the GPU fill is the host generator, bit for bit
        probe = np.array([0, 1, R * S - 1, int(rng.integers(R * S))])
        assert np.array_equal(
            pt.dev_bits(self.hidden.view(R * S, H)[torch.from_numpy(probe).to(dev)]),
            synth.bf16_rows(self.kh, probe, H))
        # unweighted: dispatch without route weights, plain K-sum combine
        self.weighted = weighted
        w_d = pt.to_dev(wl["w"], dev) if weighted else None
        moon.moon_plan(ctx, pt.to_dev(wl["topk"], dev), None, plan)
        self.win, self.wwin = moon.window_tensors(ctx)
        if not weighted:
            self.wwin.fill_(-3.0)  # must stay untouched
        moon.moon_dispatch(ctx, plan, self.hidden, w_d, flags=dflags)
        self.out = torch.empty((R, S, H), dtype=torch.bfloat16, device=dev)
        self.wsk = torch.empty((R, S, K), dtype=torch.float32, device=dev)
        moon.moon_combine(ctx, plan, self.y, self.wwin,
                          moon.MOON_COMBINE_WEIGHTED if weighted else 0, self.out, self.wsk)
        self.pidx = torch.empty((R, ctx.B, 2), dtype=torch.int32, device=dev)
        moon.moon_prefetch_index(ctx, plan, self.pidx)
        assert moon.moon_plan_status(plan) == moon.MOON_OK
        got = pt.gpu_plan_arrays(plan)

        self.ref = ref = oracle.plan(wl["topk"], E, B, P)
        assert ref.status == oracle.OK
        pt.compare_plan(got, ref)
        pv = pt.gpu_plan_view(got, ref)
        pc.check_layout(pv)
        pc.check_routes(pv, wl["topk"])
        pc.check_slots(pv)
        say(f"   plan bit-exact; slots used {int(ref.remote_stats[:, 0].sum())}, "
            f"dup rows {int(ref.dup_counts[:, 1].sum())}")
        assert np.array_equal(self.pidx.cpu().numpy(), oracle.prefetch_index(ref))
        self.src = oracle.row_sources(ref)
        cov = self.src != -2
        if weighted:
            _, self.ewwin = oracle.dispatch(ref, np.zeros((R, S, 0), np.uint16), wl["w"])
            # every covered weight-window entry, bit for bit
            assert np.array_equal(self.wwin.cpu().numpy()[cov].view(np.uint32),
                                  self.ewwin[cov].view(np.uint32)), "weight windows differ"
        else:
            assert bool((self.wwin == -3.0).all()), "dispatch without weights wrote weights"
            self.ewwin = np.full(R * ctx.NvS, -3.0, np.float32)  # what combine gathers

    def close(self, moon):
        moon.moon_plan_destroy(self.plan)
        moon.moon_ctx_destroy(self.ctx)

    def check_window(self, u, hidden_host):
        """Every covered row of rank u's window: routed rows equal their
        token's row, padding rows are zero."""
        NvS, H, K = self.ctx.NvS, self.H, self.K
        g = pt.dev_bits(self.win[u * NvS:(u + 1) * NvS])
        s = self.src[u * NvS:(u + 1) * NvS]
        routed, pad = s >= 0, s == -1
        assert np.array_equal(g[routed], hidden_host[s[routed] // K]), \
            f"routed rows of rank {u} differ"
        assert not g[pad].any(), f"padding rows of rank {u} are not zero"
        return int(routed.sum()), int(pad.sum())

    def check_rows(self, rows):
        """Sampled window rows against the regenerated source rows."""
        import torch
        H, K = self.H, self.K
        rows_d = torch.from_numpy(rows).to(self.win.device)
        g_rows = pt.dev_bits(self.win[rows_d])
        s = self.src[rows]
        routed = s >= 0
        exp = np.zeros((rows.shape[0], H), np.uint16)
        exp[routed] = synth.bf16_rows(self.kh, s[routed] // K, H)
        cov = s != -2
        assert np.array_equal(g_rows[cov], exp[cov]), "sampled window rows differ"
        return int(cov.sum())

    def check_combine(self, toks):
        """Combine outputs and gathered weights of tokens `toks` (global token
        ids) against the oracle on regenerated rows."""
        import torch
        R, S, K, H = self.R, self.S, self.K, self.H
        dst_tok = self.ref.dst.reshape(R * S, K)[toks]
        need = np.unique(pc.decode(dst_tok).reshape(-1))
        yrows = synth.bf16_rows(self.ky, need, H)
        eout, ewsk, acc = oracle.combine_rows(dst_tok, need, yrows, self.ewwin[need],
                                              weighted=self.weighted)
        toks_d = torch.from_numpy(toks).to(self.out.device)
        g_out = pt.dev_bits(self.out.view(R * S, H)[toks_d])
        absum = pt.abs_sum(dst_tok, need, yrows, self.ewwin[need], self.weighted)
        dmax, ndiff = pt.check_combine(g_out, eout, acc, absum, K)
        assert np.array_equal(self.wsk.view(R * S, K)[toks_d].cpu().numpy().view(np.uint32),
                              ewsk.view(np.uint32))
        return dmax, ndiff, g_out.size


def _flags(moon, path):
    return moon.MOON_DISPATCH_DEDUP_EPILOGUE if path == "epilogue" else 0


@pytest.mark.parametrize("path", ["fused", "epilogue"])
def test_dsv3_every_window_row(env, path):
    """DSv3 shape: all eight rank windows compared row for row; combine over
    every token of source rank 3."""
    moon, dev = env
    run = Run(moon, dev, "dsv3", 0, _flags(moon, path))
    try:
        hidden_host = synth.hidden_bf16(run.wl["seed"], run.R, run.S, run.H).reshape(
            run.R * run.S, run.H)
        tot_r = tot_p = 0
        for u in range(run.R):
            r, p = run.check_window(u, hidden_host)
            tot_r, tot_p = tot_r + r, tot_p + p
        say(f"   all windows bit-exact: {tot_r} routed rows, {tot_p} padding rows")
        del hidden_host
        toks = np.arange(3 * run.S, 4 * run.S)
        dmax, ndiff, n = run.check_combine(toks)
        say(f"   combine on rank 3's {toks.shape[0]} tokens: max|d|={dmax:.3g}, "
            f"bf16 mismatches {ndiff}/{n}")
    finally:
        run.close(moon)


@pytest.mark.parametrize("path", ["fused", "epilogue"])
def test_r16_maxvio8_windows(env, path):
    """R=16 shape at maxvio 8 (half the tokens inside one home rank): with
    the default one-pass dispatch every covered row of all sixteen rank
    windows, with the two-pass path the window of the rank with the most
    slots, compared row for row (then a sample of all ranks); combine over
    every token of source rank 0."""
    moon, dev = env
    run = Run(moon, dev, "r16-e384-k8", 4, _flags(moon, path))
    try:
        NvS, K = run.ctx.NvS, run.K
        if path == "fused":
            ranks = list(range(run.R))
            hidden_host = synth.hidden_bf16(run.wl["seed"], run.R, run.S, run.H).reshape(
                run.R * run.S, run.H)
        else:
            ranks = [int(np.argmax(run.ref.remote_stats[:, 0]))]
            s = run.src[ranks[0] * NvS:(ranks[0] + 1) * NvS]
            toks = np.unique(s[s >= 0] // K)  # tokens routed to that rank
            hidden_host = np.zeros((run.R * run.S, run.H), np.uint16)
            hidden_host[toks] = synth.bf16_rows(run.kh, toks, run.H)
        tot_r = tot_p = 0
        for u in ranks:
            r, p = run.check_window(u, hidden_host)
            tot_r, tot_p = tot_r + r, tot_p + p
        del hidden_host
        say(f"   ranks {ranks if len(ranks) < 4 else 'all'}: {tot_r} routed rows, {tot_p} "
            f"padding rows bit-exact")
        n = run.check_rows(sample_rows(run.rng, run.ref, run.src))
        say(f"   {n} sampled rows of all ranks bit-exact")
        toks = np.arange(0, run.S)
        dmax, ndiff, n = run.check_combine(toks)
        say(f"   combine on rank 0's {toks.shape[0]} tokens: max|d|={dmax:.3g}, "
            f"bf16 mismatches {ndiff}/{n}")
    finally:
        run.close(moon)


def test_dsv3_unweighted_every_window_row(env):
    """DSv3 shape without route weights: the weight windows stay untouched,
    every covered window row as above, and the plain K-sum combine over every
    token of source rank 6."""
    moon, dev = env
    run = Run(moon, dev, "dsv3", 0, 0, weighted=False)
    try:
        hidden_host = synth.hidden_bf16(run.wl["seed"], run.R, run.S, run.H).reshape(
            run.R * run.S, run.H)
        for u in range(run.R):
            run.check_window(u, hidden_host)
        del hidden_host
        toks = np.arange(6 * run.S, 7 * run.S)
        dmax, ndiff, n = run.check_combine(toks)
        say(f"   unweighted combine on rank 6's tokens: max|d|={dmax:.3g}, "
            f"bf16 mismatches {ndiff}/{n}")
    finally:
        run.close(moon)


@pytest.mark.parametrize("level,weighted", [(0, True), (2, True), (3, False)])
def test_r16_other_levels_sampled(env, level, weighted):
    """R=16 shape at maxvio about 0, 2 and 4: plan in full, sampled window
    rows and combine tokens (maxvio 4 without route weights)."""
    moon, dev = env
    run = Run(moon, dev, "r16-e384-k8", level, 0, weighted=weighted)
    try:
        n = run.check_rows(sample_rows(run.rng, run.ref, run.src))
        say(f"   {n} sampled window rows bit-exact")
        toks = np.unique(np.concatenate([run.rng.choice(run.R * run.S, 384, replace=False),
                                         [0, run.R * run.S - 1]]))
        dmax, ndiff, n = run.check_combine(toks)
        say(f"   combine on {toks.shape[0]} tokens: max|d|={dmax:.3g}, bf16 mismatches {ndiff}/{n}")
    finally:
        run.close(moon)
