"""moon_plan_noalloc: planning with no context and no allocation (the
planner's scratch is the library's static device block), through the C ABI.

Calls in a row, each smaller than the one before, on one GPU's shared
scratch block: every plan array must equal the plan of moon_plan (context
scratch) on the same routing bit for bit (duplicate records on their valid
prefixes), and the oracle's.  Shapes whose scratch exceeds the block, and
array descriptions that do not match the configuration, are refused.  The
call captured in a HIP graph replans whatever routing its captured input
buffer holds, replay after replay."""
import numpy as np
import pytest

import oracle
import parity as pt
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


def _arrays(moon, dev, R, E, K, S, B, P, fill=-7):
    import torch
    shapes, NvS, Bx = moon.plan_array_shapes(R, E, K, S, B, P)
    return {k: torch.full(s, fill, dtype=torch.int32, device=dev) for k, s in shapes.items()}, NvS


def _compare(got, exp, R):
    """got/exp: dicts of host arrays; duplicate records on the valid prefix."""
    for k in exp:
        if k in ("dup_groups", "dup_loffs"):
            continue
        assert np.array_equal(got[k], exp[k]), f"{k} differs from moon_plan's"
    for r in range(R):
        ng, nd = exp["dup_counts"][r]
        assert np.array_equal(got["dup_groups"][r, :ng], exp["dup_groups"][r, :ng])
        assert np.array_equal(got["dup_loffs"][r, :nd], exp["dup_loffs"][r, :nd])


CALLS = [("r16-e384-k8", 4), ("r8-e64-k6", 0), ("tiny", 0)]


def test_calls_in_a_row_match_moon_plan(env):
    moon, dev = env
    import torch
    for config, level in CALLS:
        wl = synth.workload(config, level)
        R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
        say(f"[case] no-alloc plan {wl['name']} level {level} R={R} E={E} S={S}")
        topk = pt.to_dev(wl["topk"], dev)
        arrays, NvS = _arrays(moon, dev, R, E, K, S, B, P)
        moon.moon_plan_noalloc(R, E, K, S, H, B, P, topk, None, arrays)
        got = {k: v.cpu().numpy() for k, v in arrays.items()}
        ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
        plan = moon.moon_plan_create(ctx)
        try:
            assert ctx.NvS == NvS
            moon.moon_plan(ctx, topk, None, plan)
            assert moon.moon_plan_status(plan) == moon.MOON_OK
            exp = pt.gpu_plan_arrays(plan)
        finally:
            moon.moon_plan_destroy(plan)
            moon.moon_ctx_destroy(ctx)
        torch.cuda.synchronize()
        assert int(got["status"][0]) == 0
        _compare(got, exp, R)
        ref = oracle.plan(wl["topk"], E, B, P)
        pt.compare_plan(got, ref)
        say(f"   equal to moon_plan and the oracle ({int(ref.dup_counts[:, 1].sum())} dup rows)")


def test_status_and_histogram_input(env):
    """A bad expert id sets the status word; a given histogram is checked."""
    moon, dev = env
    import torch
    wl = synth.workload("tiny")
    R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    topk = wl["topk"].copy()
    tpe = np.stack([np.bincount(topk[r].reshape(-1), minlength=E) for r in range(R)]).astype(
        np.int32)
    arrays, _ = _arrays(moon, dev, R, E, K, S, B, P)
    moon.moon_plan_noalloc(R, E, K, S, H, B, P, pt.to_dev(topk, dev), pt.to_dev(tpe, dev), arrays)
    torch.cuda.synchronize()
    assert int(arrays["status"][0]) == 0
    pt.compare_plan({k: v.cpu().numpy() for k, v in arrays.items()},
                    oracle.plan(topk, E, B, P, tokens_per_expert=tpe))
    tpe[1, 3] += 1
    moon.moon_plan_noalloc(R, E, K, S, H, B, P, pt.to_dev(topk, dev), pt.to_dev(tpe, dev), arrays)
    torch.cuda.synchronize()
    assert int(arrays["status"][0]) == 4  # histogram bit
    topk[0, 5, 1] = -2
    moon.moon_plan_noalloc(R, E, K, S, H, B, P, pt.to_dev(topk, dev), None, arrays)
    torch.cuda.synchronize()
    assert int(arrays["status"][0]) & 1  # bad-expert bit


def test_refusals(env):
    moon, dev = env
    import ctypes

    import torch
    # a description whose capacity does not match the configuration
    R, E, K, S, H, B, P = 2, 8, 2, 64, 128, 4, 8
    arrays, NvS = _arrays(moon, dev, R, E, K, S, B, P)
    cfg = moon.moon_config(R, E, K, S, H, B, P, 0)
    pa = moon.moon_plan_arrays()
    for k, v in arrays.items():
        setattr(pa, k, ctypes.c_void_p(v.data_ptr()))
    topk = torch.zeros((R, S, K), dtype=torch.int32, device=dev)
    pa.N, pa.R, pa.E, pa.B, pa.NvS, pa.K = S * K, R, E, B, NvS + P, K
    st = moon._lib.moon_plan_noalloc(ctypes.byref(cfg), ctypes.c_void_p(topk.data_ptr()), None,
                                     ctypes.byref(pa), None)
    assert st == moon.MOON_ERR_INVALID_ARG
    pa.NvS = NvS
    pa.dup_loffs = None
    st = moon._lib.moon_plan_noalloc(ctypes.byref(cfg), ctypes.c_void_p(topk.data_ptr()), None,
                                     ctypes.byref(pa), None)
    assert st == moon.MOON_ERR_INVALID_ARG
    # E = 512 experts over 256 planner tiles need more scratch than the block
    if torch.cuda.get_device_properties(dev).multi_processor_count >= 256:
        R, E, K, S, H, B, P = 32, 512, 8, 1024, 16, 0, 4
        arrays, _ = _arrays(moon, dev, R, E, K, S, B, P)
        topk = torch.zeros((R, S, K), dtype=torch.int32, device=dev)
        with pytest.raises(moon.MoonError) as ei:
            moon.moon_plan_noalloc(R, E, K, S, H, B, P, topk, None, arrays)
        assert ei.value.status == moon.MOON_ERR_UNSUPPORTED


def test_noalloc_plan_in_a_graph(env):
    """The no-alloc planner captured in a HIP graph (what it is for): the
    graph replans whatever routing sits in its captured input buffer; every
    replay, with eager planning calls on the same GPU between replays, equals
    moon_plan on that routing."""
    moon, dev = env
    import torch
    wl = synth.workload("r8-e64-k6")
    R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    routings = [wl["topk"], synth.workload("r8-e64-k6-skewed", 3)["topk"]]
    topk_buf = pt.to_dev(routings[0], dev)
    arrays, _ = _arrays(moon, dev, R, E, K, S, B, P)
    other, _ = _arrays(moon, dev, R, E, K, S, B, P)
    st = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(st):
        moon.moon_plan_noalloc(R, E, K, S, H, B, P, topk_buf, None, arrays, stream=st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        moon.moon_plan_noalloc(R, E, K, S, H, B, P, topk_buf, None, arrays,
                               stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        exp = []
        for tk in routings:
            moon.moon_plan(ctx, pt.to_dev(tk, dev), None, plan)
            assert moon.moon_plan_status(plan) == moon.MOON_OK
            exp.append(pt.gpu_plan_arrays(plan))
        say("[case] no-alloc plan in a graph: 6 replays")
        for r in range(6):
            i = r % 2
            topk_buf.copy_(pt.to_dev(routings[i], dev))
            for v in arrays.values():
                v.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            # an eager no-alloc call on the other routing between replays
            moon.moon_plan_noalloc(R, E, K, S, H, B, P, pt.to_dev(routings[1 - i], dev), None,
                                   other)
            torch.cuda.synchronize()
            got = {k: v.cpu().numpy() for k, v in arrays.items()}
            assert int(got["status"][0]) == 0
            _compare(got, exp[i], R)
            _compare({k: v.cpu().numpy() for k, v in other.items()}, exp[1 - i], R)
        del g
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)
