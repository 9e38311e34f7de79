"""The planner's intermediate per-tile histogram (the count matrix the
placement tiles reduce) against numpy.bincount over each tile's token range,
read through the moon_debug_tile_counts test hook.  Also checks the tiling:
tiles cover every token once, never span two ranks and number at most 256.
The final plan arrays built from these counts are compared with the oracle
in the parity tests."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def expected_counts(topk, E, tt, tpr):
    R, S, _ = topk.shape
    out = np.zeros((E + 1, R * tpr), np.int32)
    for t in range(R * tpr):
        r, i = divmod(t, tpr)
        ids = topk[r, i * tt:min(S, (i + 1) * tt)].reshape(-1)
        ok = (ids >= 0) & (ids < E)
        out[:E, t] = np.bincount(ids[ok], minlength=E)
        out[E, t] = int((~ok).any())
    return out


def run_case(topk, E, B, P, H, label, expect_bad=False):
    import torch
    import combine_balanced_planning_amd as moon
    dev = torch.device("cuda", 0)
    R, S, K = topk.shape
    say(f"[case] tile counts {label} R={R} E={E} K={K} S={S}")
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        moon.moon_plan(ctx, torch.from_numpy(np.ascontiguousarray(topk)).to(dev), None, plan)
        st = moon.moon_plan_status(plan)
        assert st == (moon.MOON_ERR_BAD_EXPERT if expect_bad else moon.MOON_OK), st
        tt, tpr = moon.moon_debug_tile_counts(ctx)
        assert tt >= 1 and tpr >= 1 and R * tpr <= 256
        assert (tpr - 1) * tt < S <= tpr * tt, (tt, tpr, S)
        got = torch.empty((E + 1, R * tpr), dtype=torch.int32, device=dev)
        moon.moon_debug_tile_counts(ctx, got)
        got = got.cpu().numpy()
        want = expected_counts(topk, E, tt, tpr)
        assert np.array_equal(got, want), np.argwhere(got != want)[:5]
        # per rank, the tiles add up to the rank's histogram
        for r in range(R):
            ids = topk[r].reshape(-1)
            ids = ids[(ids >= 0) & (ids < E)]
            assert np.array_equal(got[:E, r * tpr:(r + 1) * tpr].sum(1),
                                  np.bincount(ids, minlength=E))
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("config,level", [("tiny", 0), ("r8-e64-k6", 0),
                                          ("r8-e64-k6-skewed", 3), ("dsv3", 0),
                                          ("r16-e384-k8", 4)])
def test_tile_counts_workloads(gpu, config, level):
    wl = synth.workload(config, level)
    run_case(wl["topk"], wl["E"], wl["B"], wl["P"], 64, f"{wl['name']} level {level}")


@pytest.mark.parametrize("R,E,K,S", [(1, 8, 3, 1), (3, 12, 5, 1000), (2, 512, 64, 70),
                                     (32, 64, 2, 333), (4, 16, 1, 4097)])
def test_tile_counts_edge_shapes(gpu, R, E, K, S):
    rng = np.random.default_rng(R * 1000 + S)
    topk = rng.integers(0, E, size=(R, S, K)).astype(np.int32)
    run_case(topk, E, 0, 4, 8, "random")


def test_tile_counts_flag_bad_ids(gpu):
    rng = np.random.default_rng(9)
    R, E, K, S = 4, 16, 4, 600
    topk = rng.integers(0, E, size=(R, S, K)).astype(np.int32)
    topk[1, 5, 2] = E
    topk[3, S - 1, 0] = -1
    run_case(topk, E, 0, 4, 8, "out-of-range ids", expect_bad=True)
