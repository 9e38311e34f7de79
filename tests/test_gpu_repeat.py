"""Run-to-run identity of the planner, the one kernel whose workgroups
exchange words inside a launch (per-tile duplicate counts tagged with the
call's epoch, read by later tiles).  Two input sets are planned alternately
into two plans of one context, 100 times each, with and without the
tokens_per_expert check; after every call all plan arrays must equal the
first call's bit for bit (and the first calls equal the oracle's plan)."""
import numpy as np
import pytest

import oracle
import parity as pt
import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("config,level", [("r8-e64-k6", 0), ("dsv3", 0), ("r16-e384-k8", 4)])
def test_plan_repeats_bit_identical(config, level):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_balanced_planning_amd as moon
    dev = torch.device("cuda", 0)
    wl = synth.workload(config, level)
    R, E, K, S, B, P = (wl[k] for k in ("R", "E", "K", "S", "B", "P"))
    say(f"[case] plan repeats {wl['name']} level {level}")
    ctx = moon.moon_ctx_create(R, E, K, S, 64, B, P)
    inputs = []
    for seed in (wl["seed"], wl["seed"] + 500):
        topk = wl["topk"] if seed == wl["seed"] else synth.routing(config, seed,
                                                                   synth.alpha_for(config, level))[0]
        tpe = np.stack([np.bincount(topk[r].reshape(-1), minlength=E) for r in range(R)])
        inputs.append((topk, torch.from_numpy(topk).to(dev),
                       torch.from_numpy(tpe.astype(np.int32)).to(dev)))
    plans = [moon.moon_plan_create(ctx) for _ in inputs]
    try:
        ref = []
        for (topk, tk, _), plan in zip(inputs, plans):
            moon.moon_plan(ctx, tk, None, plan)
            assert moon.moon_plan_status(plan) == moon.MOON_OK
            ref.append({k: v.clone() for k, v in moon.plan_tensors(plan).items()})
        pt.compare_plan(pt.gpu_plan_arrays(plans[0]), oracle.plan(inputs[0][0], E, ctx.B, P))
        views = [moon.plan_tensors(p) for p in plans]
        bad = []
        for it in range(200):
            i = it % 2
            moon.moon_plan(ctx, inputs[i][1], inputs[i][2] if it % 4 >= 2 else None, plans[i])
            for k in ref[i]:
                if not torch.equal(views[i][k], ref[i][k]):
                    bad.append((it, k))
        assert moon.moon_plan_status(plans[0]) == moon.MOON_OK
        assert not bad, bad[:10]
        say(f"[case] plan repeats {wl['name']}: 200 calls bit-identical")
    finally:
        torch.cuda.synchronize()
        for p in plans:
            moon.moon_plan_destroy(p)
        moon.moon_ctx_destroy(ctx)
