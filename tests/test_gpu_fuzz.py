"""Seeded random shapes through the whole path against the oracle, with
longer token ranges than the random-shape parity cases (up to 3000 tokens per
rank, so the planner runs up to its 256 tiles and the duplicate look-back
spans many of them), narrow rows, every routing mode, both dispatch paths
and, in half of the cases, the tokens_per_expert check.  MOON_FUZZ_CASES
sets the number of seeds (default 100)."""
import os

import numpy as np
import pytest

import oracle
import synth
import test_gpu_parity as tg

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("MOON_FUZZ_CASES", "100"))


def fuzz_case(i):
    rng = np.random.default_rng(77000 + i)
    R = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 32]))
    Eg = int(rng.integers(1, max(2, 512 // R) + 1))
    E = R * Eg
    K = int(rng.integers(1, 17)) if rng.random() < 0.9 else int(rng.integers(17, 65))
    S = int(rng.integers(1, 3001)) if R <= 8 else int(rng.integers(1, 1025))
    H = 8 * int(rng.choice([1, 2, 8]))
    P = int(rng.choice([1, 2, 5, 16, 128]))
    B = 0 if rng.random() < 0.7 else int(rng.integers(1, Eg + 1))
    mode = str(rng.choice(["uniform", "skewed", "repeats", "home_block", "one_expert"]))
    if mode in ("uniform", "skewed") and K > E:
        mode = "repeats"
    return rng, R, E, K, S, H, B, P, mode


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_shapes(i):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_balanced_planning_amd as moon
    dev = torch.device("cuda", 0)
    rng, R, E, K, S, H, B, P, mode = fuzz_case(i)
    topk = tg._edge_topk(rng, R, S, K, E, mode)
    tpe = None
    if rng.random() < 0.5:
        tpe = np.stack([np.bincount(topk[r].reshape(-1), minlength=E)
                        for r in range(R)]).astype(np.int32)
    ref = oracle.plan(topk, E, B if B > 0 else E // R, P, tpe)
    label = f"fuzz {i}: R={R} E={E} K={K} S={S} H={H} B={B} P={P} {mode} tpe={tpe is not None}"
    if ref.status == oracle.SLOT_BUDGET:
        tg.say(f"[case] {label} -> slot budget")
        ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
        plan = moon.moon_plan_create(ctx)
        try:
            moon.moon_plan(ctx, torch.from_numpy(topk).to(dev), None, plan)
            assert moon.moon_plan_status(plan) == moon.MOON_ERR_SLOT_BUDGET
        finally:
            moon.moon_plan_destroy(plan)
            moon.moon_ctx_destroy(ctx)
        return
    w = rng.random((R, S, K)).astype(np.float32)
    hidden = synth.bf16_normal(int(rng.integers(1 << 62)), 0, R * S * H).reshape(R, S, H)
    y = synth.bf16_normal(int(rng.integers(1 << 62)), 0, R * ref.NvS * H).reshape(
        R * ref.NvS, H)
    tg.run_full(moon, dev, topk, w, hidden, y, R, E, K, S, H, B, P, label=label,
                weighted=bool(i % 2), tpe=tpe,
                dflags=moon.MOON_DISPATCH_DEDUP_EPILOGUE if i % 4 >= 2 else 0)
