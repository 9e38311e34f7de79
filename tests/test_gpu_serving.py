"""GPU parity on the padded serving workload (MoonEP vLLM integration page:
power-of-two buffer capacities, padding and invalid ids mapped to expert 0
with weight 0, tokens_per_expert handed to dispatch, combine as a plain K-sum).

* narrow rows, both levels: everything compared with the oracle in full;
* full rows (H = 7168), both levels, in the benchmark's launch configuration:
  the plan bit for bit, window rows and combine outputs on samples;
* full rows, decode level: combine(dispatch(x)) without weights equals K*x
  bit for bit (torch's bf16 rounding of K*x on the GPU is the reference), so
  every pad token's output is zero.
"""
import numpy as np
import pytest

import oracle
import parity as pt
import plan_checks as pc
import synth
from test_gpu_large import sample_rows
from test_gpu_parity import run_full

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


@pytest.mark.parametrize("level", [0, 1])
def test_serving_full_parity_narrow_rows(env, level):
    moon, dev = env
    wl = dict(synth.serving_workload(level))
    wl["H"] = 128
    R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    hidden = synth.serving_hidden_bf16(wl)
    y = synth.y_bf16(wl["seed"], R * oracle.nvs(R, E, K, S, B, P), H)
    say(f"[serving] {wl['level_name']} S={S} n_tok={wl['n_tok'].tolist()} "
        f"maxvio={wl['maxvio']:.1f}")
    run_full(moon, dev, wl["topk"], wl["w"], hidden, y, R, E, K, S, H, B, P, weighted=False,
             label=f"serving-{wl['level_name']}-narrow", tpe=wl["tokens_per_expert"])


def test_serving_empty_and_full_ranks(env):
    """Ranks with no real tokens next to ranks filled to capacity."""
    moon, dev = env
    wl = dict(synth.serving_workload(0, n_tok=[0, 256, 100, 0, 37, 256, 1, 200]))
    wl["H"] = 256
    R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    hidden = synth.serving_hidden_bf16(wl)
    y = synth.y_bf16(wl["seed"], R * oracle.nvs(R, E, K, S, B, P), H)
    for weighted in (False, True):
        run_full(moon, dev, wl["topk"], wl["w"], hidden, y, R, E, K, S, H, B, P,
                 weighted=weighted, label=f"serving-empty-ranks-w{int(weighted)}",
                 tpe=wl["tokens_per_expert"])


def _gpu_inputs(moon, dev, wl, ctx):
    import torch

    import synth.gpu as sg
    R, S, H = wl["R"], wl["S"], wl["H"]
    hidden = sg.hidden(wl["seed"], R, S, H, dev)
    for r in range(R):
        hidden[r, int(wl["n_tok"][r]):] = 0
    y = sg.y(wl["seed"], R * ctx.NvS, H, dev)
    return hidden, y


@pytest.mark.parametrize("level", [0, 1])
def test_serving_full_size_sampled(env, level):
    import torch
    moon, dev = env
    wl = synth.serving_workload(level)
    R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    say(f"[serving] {wl['level_name']} full rows S={S} H={H}")
    rng = np.random.default_rng(wl["seed"])
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        hidden, y = _gpu_inputs(moon, dev, wl, ctx)
        moon.moon_plan(ctx, pt.to_dev(wl["topk"], dev), pt.to_dev(wl["tokens_per_expert"], dev),
                       plan)
        moon.moon_dispatch(ctx, plan, hidden, pt.to_dev(wl["w"], dev))
        win, wwin = moon.window_tensors(ctx)
        out = torch.empty((R, S, H), dtype=torch.bfloat16, device=dev)
        wsk = torch.empty((R, S, K), dtype=torch.float32, device=dev)
        moon.moon_combine(ctx, plan, y, wwin, 0, out, wsk)
        pidx = torch.empty((R, ctx.B, 2), dtype=torch.int32, device=dev)
        moon.moon_prefetch_index(ctx, plan, pidx)
        assert moon.moon_plan_status(plan) == moon.MOON_OK
        got = pt.gpu_plan_arrays(plan)

        ref = oracle.plan(wl["topk"], E, B, P, wl["tokens_per_expert"])
        assert ref.status == oracle.OK
        pt.compare_plan(got, ref)
        pv = pt.gpu_plan_view(got, ref)
        pc.check_layout(pv)
        pc.check_routes(pv, wl["topk"])
        pc.check_slots(pv)
        assert np.array_equal(pidx.cpu().numpy(), oracle.prefetch_index(ref))
        say(f"   plan bit-exact; slots used {int(ref.remote_stats[:, 0].sum())}, "
            f"dup rows {int(ref.dup_counts[:, 1].sum())} of {R * S * K} routes")

        kh = synth.stream_key(wl["seed"], synth.TAG_HIDDEN)
        ky = synth.stream_key(wl["seed"], synth.TAG_Y)
        src = oracle.row_sources(ref)
        _, ewwin = oracle.dispatch(ref, np.zeros((R, S, 0), np.uint16), wl["w"])
        rows = sample_rows(rng, ref, src)
        rows_d = torch.from_numpy(rows).to(dev)
        g_rows = pt.dev_bits(win[rows_d])
        s = src[rows]
        tok = s // K
        routed = s >= 0
        exp = np.zeros((rows.shape[0], H), np.uint16)
        exp[routed] = synth.bf16_rows(kh, tok[routed], H)
        # pad tokens' rows are zero in the source, hence in the window
        padtok = routed & ((tok % S) >= wl["n_tok"][np.maximum(tok, 0) // S])
        exp[padtok] = 0
        cov = s != -2
        assert np.array_equal(g_rows[cov], exp[cov]), "sampled window rows differ"
        assert np.array_equal(wwin[rows_d].cpu().numpy()[cov].view(np.uint32),
                              ewwin[rows][cov].view(np.uint32))
        say(f"   {int(cov.sum())} window rows ({int(padtok.sum())} of pad tokens) bit-exact")

        toks = np.unique(np.concatenate([rng.choice(R * S, 256, replace=False), [0, R * S - 1]]))
        dst_tok = ref.dst.reshape(R * S, K)[toks]
        need = np.unique(pc.decode(dst_tok).reshape(-1))
        yrows = synth.bf16_rows(ky, need, H)
        eout, ewsk, acc = oracle.combine_rows(dst_tok, need, yrows, ewwin[need], weighted=False)
        toks_d = torch.from_numpy(toks).to(dev)
        absum = pt.abs_sum(dst_tok, need, yrows, ewwin[need], False)
        dmax, ndiff = pt.check_combine(pt.dev_bits(out.view(R * S, H)[toks_d]), eout, acc, absum, K)
        assert np.array_equal(wsk.view(R * S, K)[toks_d].cpu().numpy().view(np.uint32),
                              ewsk.view(np.uint32))
        say(f"   unweighted combine on {toks.shape[0]} tokens: max|d|={dmax:.3g}, "
            f"bf16 mismatches {ndiff}")
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


def test_serving_round_trip_full_rows(env):
    import torch
    moon, dev = env
    wl = synth.serving_workload(0)
    R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        hidden, _ = _gpu_inputs(moon, dev, wl, ctx)
        moon.moon_plan(ctx, pt.to_dev(wl["topk"], dev), pt.to_dev(wl["tokens_per_expert"], dev),
                       plan)
        moon.moon_dispatch(ctx, plan, hidden, pt.to_dev(wl["w"], dev))
        win, _ = moon.window_tensors(ctx)
        out = torch.empty((R, S, H), dtype=torch.bfloat16, device=dev)
        moon.moon_combine(ctx, plan, win, None, 0, out, None)
        assert moon.moon_plan_status(plan) == moon.MOON_OK
        exp = (hidden.float() * K).to(torch.bfloat16)
        assert torch.equal(out.view(torch.int16), exp.view(torch.int16))
        pad = torch.arange(S, device=dev)[None, :] >= torch.from_numpy(wl["n_tok"]).to(dev)[:, None]
        assert int(pad.sum()) > 0 and bool((out[pad].view(torch.int16) == 0).all())
        say(f"   round trip K*x bit-exact over {R * S} tokens, {int(pad.sum())} pad tokens zero")
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)
