"""GPU parity at the full workload sizes, in the launch configuration the
benchmark uses.

The whole plan (dst, layout, slots, duplicate records) is compared bit for
bit with the oracle.  Windows and combine outputs are compared on samples the
oracle computes one by one: bulk inputs are filled on the GPU by the seeded
generator and the needed rows are regenerated on the host (the fill itself is
checked against the host generator first).
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


@pytest.mark.parametrize("config,level", [("dsv3", 0), ("r16-e384-k8", 0),
                                          ("r16-e384-k8", 2), ("r16-e384-k8", 4)])
def test_full_size_sampled_parity(env, config, level):
    import torch

    import synth.gpu as sg
    moon, dev = env
    wl = synth.workload(config, level)
    R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    seed = wl["seed"]
    say(f"[case] {wl['name']} level {level} maxvio={wl['maxvio']:.3f} R={R} E={E} K={K} "
        f"S={S} H={H}")
    rng = np.random.default_rng(seed)
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        NvS = ctx.NvS
        hidden = sg.hidden(seed, R, S, H, dev)
        y = sg.y(seed, R * NvS, H, dev)
        # the GPU fill is the host generator, bit for bit
        kh, ky = synth.stream_key(seed, synth.TAG_HIDDEN), synth.stream_key(seed, synth.TAG_Y)
        probe = np.array([0, 1, R * S - 1, int(rng.integers(R * S))])
        assert np.array_equal(pt.dev_bits(hidden.view(R * S, H)[torch.from_numpy(probe).to(dev)]),
                              synth.bf16_rows(kh, probe, H))
        w_d = pt.to_dev(wl["w"], dev)
        moon.moon_plan(ctx, pt.to_dev(wl["topk"], dev), None, plan)
        moon.moon_dispatch(ctx, plan, hidden, w_d)
        win, wwin = moon.window_tensors(ctx)
        out = torch.empty((R, S, H), dtype=torch.bfloat16, device=dev)
        wsk = torch.empty((R, S, K), dtype=torch.float32, device=dev)
        moon.moon_combine(ctx, plan, y, wwin, moon.MOON_COMBINE_WEIGHTED, out, wsk)
        pidx = torch.empty((R, ctx.B, 2), dtype=torch.int32, device=dev)
        moon.moon_prefetch_index(ctx, plan, pidx)
        assert moon.moon_plan_status(plan) == moon.MOON_OK
        got = pt.gpu_plan_arrays(plan)

        ref = oracle.plan(wl["topk"], E, B, P)
        assert ref.status == oracle.OK
        pt.compare_plan(got, ref)
        pv = pt.gpu_plan_view(got, ref)
        pc.check_layout(pv)
        pc.check_routes(pv, wl["topk"])
        pc.check_slots(pv)
        say(f"   plan bit-exact; slots used {int(ref.remote_stats[:, 0].sum())}, "
            f"dup rows {int(ref.dup_counts[:, 1].sum())}")
        assert np.array_equal(pidx.cpu().numpy(), oracle.prefetch_index(ref))

        # dispatch: sampled rows against the regenerated source rows
        src = oracle.row_sources(ref)
        _, ewwin = oracle.dispatch(ref, np.zeros((R, S, 0), np.uint16), wl["w"])
        rows = sample_rows(rng, ref, src)
        rows_d = torch.from_numpy(rows).to(dev)
        g_rows = pt.dev_bits(win[rows_d])
        g_w = wwin[rows_d].cpu().numpy()
        s = src[rows]
        routed = s >= 0
        exp = np.zeros((rows.shape[0], H), np.uint16)
        exp[routed] = synth.bf16_rows(kh, s[routed] // K, H)
        cov = s != -2
        assert np.array_equal(g_rows[cov], exp[cov]), "sampled window rows differ"
        assert np.array_equal(g_w[cov].view(np.uint32), ewwin[rows][cov].view(np.uint32))
        say(f"   {int(cov.sum())} window rows ({int((s == -1).sum())} padding) bit-exact")

        # combine: sampled tokens, the oracle on regenerated rows
        toks = np.unique(np.concatenate([rng.choice(R * S, 384, replace=False),
                                         [0, R * S - 1]]))
        dst_tok = ref.dst.reshape(R * S, K)[toks]
        need = np.unique(pc.decode(dst_tok).reshape(-1))
        yrows = synth.bf16_rows(ky, need, H)
        eout, ewsk, acc = oracle.combine_rows(dst_tok, need, yrows, ewwin[need], weighted=True)
        toks_d = torch.from_numpy(toks).to(dev)
        g_out = pt.dev_bits(out.view(R * S, H)[toks_d])
        absum = pt.abs_sum(dst_tok, need, yrows, ewwin[need], True)
        dmax, ndiff = pt.check_combine(g_out, eout, acc, absum, K)
        assert np.array_equal(wsk.view(R * S, K)[toks_d].cpu().numpy().view(np.uint32),
                              ewsk.view(np.uint32))
        say(f"   combine on {toks.shape[0]} tokens: max|d|={dmax:.3g}, "
            f"bf16 mismatches {ndiff}/{g_out.size}")
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)
