"""The step (plan, dispatch, combine, prefetch index) captured in a HIP graph:
the calls launch kernels only (no allocation, copy, memset or host wait), so
a captured step replays; every replay must reproduce the eager results bit
for bit, with eager steps on another input set run between the replays, and
the eager plan must equal the oracle's.  Two input sets share one context
(its windows and planner scratch), as in a training loop."""
import pytest

import oracle
import parity as pt
import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("config", ["tiny", "r8-e64-k6"])
def test_graph_replay_matches_eager(config):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_balanced_planning_amd as moon
    import synth.gpu as sg
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    c = synth.WORKLOADS[synth.workload_id(config)]
    R, E, K, S, H, B, P = (c[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    say(f"[case] graph replay {c['name']}")
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    _, wwin = moon.window_tensors(ctx)
    sets = []
    for seed in (synth.seed_of(config), synth.seed_of(config) + 500):
        topk, w = synth.routing(config, seed)
        sets.append(dict(
            topk_h=topk, topk=torch.from_numpy(topk).to(dev), w=torch.from_numpy(w).to(dev),
            hidden=sg.hidden(seed, R, S, H, dev), y=sg.y(seed, R * ctx.NvS, H, dev),
            out=torch.empty((R, S, H), dtype=torch.bfloat16, device=dev),
            wsk=torch.empty((R, S, K), dtype=torch.float32, device=dev),
            pidx=torch.empty((R, ctx.B, 2), dtype=torch.int32, device=dev),
            plan=moon.moon_plan_create(ctx)))
    st = torch.cuda.Stream(device=dev)

    def step(s, stream):
        moon.moon_plan(ctx, s["topk"], None, s["plan"], stream=stream)
        moon.moon_dispatch(ctx, s["plan"], s["hidden"], s["w"], stream=stream)
        moon.moon_combine(ctx, s["plan"], s["y"], wwin, moon.MOON_COMBINE_WEIGHTED, s["out"],
                          s["wsk"], stream=stream)
        moon.moon_prefetch_index(ctx, s["plan"], s["pidx"], stream=stream)

    def snapshot(s):
        return dict(out=s["out"].view(torch.int16).clone(), wsk=s["wsk"].clone(),
                    pidx=s["pidx"].clone(),
                    **{k: v.clone() for k, v in moon.plan_tensors(s["plan"]).items()})

    def clear(s):
        # Outputs and plan arrays overwritten with values every kernel can
        # still read safely (dst 0 is a valid row, no groups, no padding), and
        # the status set to "not planned", so a replay that skipped a kernel
        # leaves a difference behind.
        s["out"].zero_()
        s["wsk"].zero_()
        s["pidx"].fill_(-7)
        pt_ = moon.plan_tensors(s["plan"])
        for k in ("dst", "zero_fill_ranges", "remote_stats", "dup_counts", "cu_seqlens"):
            pt_[k].zero_()
        pt_["experts_to_copy"].fill_(-1)
        pt_["prefetch_index"].fill_(-7)
        pt_["status"].fill_(8)

    try:
        ref = []
        with torch.cuda.stream(st):
            for s in sets:
                step(s, st)
                assert moon.moon_plan_status(s["plan"], st) == moon.MOON_OK
                ref.append(snapshot(s))
        got = pt.gpu_plan_arrays(sets[0]["plan"])
        pt.compare_plan(got, oracle.plan(sets[0]["topk_h"], E, ctx.B, P))

        torch.cuda.synchronize()
        graphs = []
        for s in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=st):
                step(s, torch.cuda.current_stream())
            graphs.append(g)
        torch.cuda.synchronize()

        def check(i, what):
            now = snapshot(sets[i])
            for k, v in ref[i].items():
                assert torch.equal(now[k], v), f"{what}: {k} differs from the eager step"

        with torch.cuda.stream(st):
            for r in range(6):
                i = r % 2
                for s in sets:
                    clear(s)
                graphs[i].replay()
                assert moon.moon_plan_status(sets[i]["plan"], st) == moon.MOON_OK
                check(i, f"replay {r}")
                step(sets[1 - i], st)  # an eager step between replays
                assert moon.moon_plan_status(sets[1 - i]["plan"], st) == moon.MOON_OK
                check(1 - i, f"eager step after replay {r}")
        say(f"[case] graph replay {c['name']}: 6 replays bit-identical")
        del graphs
    finally:
        torch.cuda.synchronize()
        for s in sets:
            moon.moon_plan_destroy(s["plan"])
        moon.moon_ctx_destroy(ctx)
