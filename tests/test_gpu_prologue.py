"""GPU parity of combine with the duplicate prologue (MOON_COMBINE_DUP_PROLOGUE).

The folded primary rows the prologue stores in the context window must equal
the oracle's bit for bit (the fold is an fp32 sum in a fixed order, rounded
once); the combine output must stay within |d| <= 1e-2 max|ref| + 1e-3 of the
oracle's and within the derived fp32 bound; the gathered weights are
bit-exact.  Checked with y in a caller buffer (the window keeps its
dispatched rows except at folded primaries) and with y being the window
itself (the zero-copy, in-place case).
"""
import zlib

import numpy as np
import pytest

import oracle
import parity as pt
import synth
from test_gpu_parity import _edge_topk, workload_inputs

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


def prologue_abs_sum(ref, y, wwin, folded, weighted):
    """sum over the summed terms of |term| per token and column: folded
    primaries count |fold|, other primaries |c_k y|, duplicates nothing."""
    R, S, K = ref.R, ref.S, ref.K
    dst = ref.dst.reshape(R * S, K)
    G = np.where(dst >= 0, dst, -dst - 1)
    rank = G // ref.NvS
    out = np.zeros((R * S, y.shape[1]))
    for k in range(K):
        prim = dst[:, k] >= 0
        has_dup = np.zeros(R * S, bool)
        for k2 in range(K):
            has_dup |= (dst[:, k2] < 0) & (rank[:, k2] == rank[:, k])
        f = prim & has_dup
        p = prim & ~has_dup
        out[f] += np.abs(pt.bits_to_f32(folded[G[f, k]]).astype(np.float64))
        term = np.abs(pt.bits_to_f32(y[G[p, k]]).astype(np.float64))
        if weighted:
            term *= np.abs(wwin[G[p, k]].astype(np.float64))[:, None]
        out[p] += term
    return out


def run_prologue(moon, dev, topk, w, hidden, y, R, E, K, S, H, B, P, weighted, in_place, label):
    import torch
    say(f"[case] prologue {label} R={R} E={E} K={K} S={S} H={H} weighted={weighted} "
        f"in_place={in_place}")
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        moon.moon_plan(ctx, pt.to_dev(topk, dev), None, plan)
        moon.moon_dispatch(ctx, plan, pt.bf16_to_dev(hidden, dev), pt.to_dev(w, dev))
        win, wwin = moon.window_tensors(ctx)
        ref = oracle.plan(topk, E, ctx.B, P)
        ewin, ewwin = oracle.dispatch(ref, hidden, w)
        if in_place:
            y_d = win
            # the oracle's y is the dispatched window; rows it never writes are
            # whatever the window held, so take them from the GPU
            y_ref = pt.dev_bits(win).copy()
        else:
            y_d = pt.bf16_to_dev(y, dev)
            y_ref = y
            win_before = pt.dev_bits(win).copy()
        flags = moon.MOON_COMBINE_DUP_PROLOGUE | (moon.MOON_COMBINE_WEIGHTED if weighted else 0)
        out = torch.empty((R, S, H), dtype=torch.bfloat16, device=dev)
        wsk = torch.empty((R, S, K), dtype=torch.float32, device=dev)
        moon.moon_combine(ctx, plan, y_d, wwin, flags, out, wsk)
        assert moon.moon_plan_status(plan) == moon.MOON_OK

        eout, ewsk, acc, folded = oracle.combine_prologue(ref, y_ref, ewwin, weighted=weighted)
        n_grp = int(ref.dup_counts[:, 0].sum())
        prow = np.concatenate([u * ref.NvS + ref.dup_groups[u, :ref.dup_counts[u, 0], 0]
                               for u in range(R)]).astype(np.int64)
        assert prow.shape[0] == n_grp
        gwin = pt.dev_bits(win)
        assert np.array_equal(gwin[prow], folded[prow]), "folded primary rows differ"
        if not in_place:
            keep = np.ones(R * ref.NvS, bool)
            keep[prow] = False
            assert np.array_equal(gwin[keep], win_before[keep]), "window changed off the primaries"
        absum = prologue_abs_sum(ref, y_ref, ewwin, folded, weighted).reshape(R, S, H)
        dmax, ndiff = pt.check_combine(pt.dev_bits(out), eout, acc, absum, K)
        say(f"   groups={n_grp} combine max|d|={dmax:.3g} bf16 mismatches={ndiff}/{eout.size}")
        assert np.array_equal(wsk.cpu().numpy().view(np.uint32), ewsk.view(np.uint32))
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


@pytest.mark.parametrize("config,level", [("tiny", 0), ("r8-e64-k6", 0),
                                          ("r8-e64-k6-skewed", 3)])
@pytest.mark.parametrize("weighted", [True, False])
def test_prologue_workloads(env, config, level, weighted):
    moon, dev = env
    wl, hidden, y = workload_inputs(config, level)
    run_prologue(moon, dev, wl["topk"], wl["w"], hidden, y, wl["R"], wl["E"], wl["K"], wl["S"],
                 wl["H"], wl["B"], wl["P"], weighted, False, wl["name"])


PROLOGUE_EDGE = [
    # label, R, E, K, S, H, B, P, mode
    ("home-block-dedup", 4, 32, 8, 96, 64, 0, 16, "home_block"),
    ("repeated-ids", 4, 8, 4, 50, 64, 0, 4, "repeats"),
    ("all-one-expert", 2, 8, 3, 64, 32, 0, 8, "one_expert"),
    ("k16", 4, 64, 16, 50, 16, 0, 4, "uniform"),
    ("k64", 2, 8, 64, 9, 8, 0, 4, "repeats"),
    ("dsv3-rows", 2, 16, 4, 40, 7168, 0, 8, "skewed"),
    ("top1", 4, 16, 1, 130, 32, 0, 8, "skewed"),
    ("ragged-width", 3, 12, 3, 200, 1000, 0, 5, "home_block"),
]


@pytest.mark.parametrize("case", PROLOGUE_EDGE, ids=[c[0] for c in PROLOGUE_EDGE])
@pytest.mark.parametrize("in_place", [False, True])
def test_prologue_edges(env, case, in_place):
    moon, dev = env
    label, R, E, K, S, H, B, P, mode = case
    rng = np.random.default_rng(zlib.crc32(("prologue-" + label).encode()))
    topk = _edge_topk(rng, R, S, K, E, mode)
    Bx = B if B > 0 else E // R
    ref = oracle.plan(topk, E, Bx, P)
    if ref.status == oracle.SLOT_BUDGET:
        pytest.skip("this routing needs more slots than B")
    w = rng.random((R, S, K)).astype(np.float32)
    hidden = synth.bf16_normal(rng.integers(1 << 62), 0, R * S * H).reshape(R, S, H)
    y = synth.bf16_normal(rng.integers(1 << 62), 0, R * ref.NvS * H).reshape(R * ref.NvS, H)
    run_prologue(moon, dev, topk, w, hidden, y, R, E, K, S, H, B, P, True, in_place, label)
