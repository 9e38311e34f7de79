"""GPU parity of the weight prefetch and the gradient reduction.

Small cases compare every slot and every expert row with the oracle bit for
bit (the prefetch moves bytes; the reduction is an fp32 sum in the pages'
order, seeded with the expert's gradient, ranks ascending).  Full-size
cases (DSv3-shaped and the R=16 dedup workload, H' = 2048) check every used
slot on the device against its expert row and recompute sampled experts'
reductions with the oracle from rows the seeded generator regenerates on
the host.
"""
import zlib

import numpy as np
import pytest

import oracle
import parity as pt
import synth

pytestmark = pytest.mark.gpu

TAG_W, TAG_G, TAG_SG = 21, 22, 23


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_balanced_planning_amd as moon
    return moon, torch.device("cuda", 0)


def say(*a):
    print(*a, flush=True)


def planned(moon, dev, topk, R, E, K, S, H, B, P):
    ctx = moon.moon_ctx_create(R, E, K, S, H, B, P)
    plan = moon.moon_plan_create(ctx)
    moon.moon_plan(ctx, pt.to_dev(topk, dev), None, plan)
    assert moon.moon_plan_status(plan) == moon.MOON_OK
    etc = moon.plan_tensors(plan)["experts_to_copy"].cpu().numpy()
    return ctx, plan, etc


SMALL = [
    # label, R, E, K, S, B, P, skew, row shapes (per tensor, elements)
    ("r2-uniform", 2, 8, 2, 64, 4, 8, 0.0, [(16, 8), (8,), (48,)]),
    ("r4-skewed", 4, 16, 4, 96, 4, 4, 2.5, [(24, 40), (1000,), (16,)]),
    ("r8-skewed", 8, 64, 6, 256, 8, 16, 1.5, [(64, 32)]),
    ("r16-hot", 16, 64, 8, 128, 4, 8, 3.0, [(8, 8), (4, 4), (2048,)]),
    ("b-small", 4, 16, 2, 64, 2, 4, 1.0, [(16,)]),
    # more than 64 slots: the copy lists the used slots first (1, 2 and 32 rounds)
    ("slots-256", 8, 256, 8, 256, 32, 16, 2.0, [(8, 8), (100,)]),
    ("slots-512", 16, 512, 8, 128, 32, 8, 2.5, [(16,), (8, 4)]),
    ("slots-8192", 32, 512, 4, 64, 256, 4, 3.0, [(8,)]),
    # the most tensors one call takes (gate, up, down and five more)
    ("eight-tensors", 4, 16, 4, 96, 4, 4, 2.0,
     [(8, 4), (16,), (4, 4), (24,), (8,), (4, 4), (32,), (12,)]),
]


def _routing(rng, R, S, K, E, skew):
    from test_oracle_plan import rand_topk
    return rand_topk(rng, R, S, K, E, skew=skew)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_prefetch_weight_small(env, case):
    import torch
    moon, dev = env
    label, R, E, K, S, B, P, skew, shapes = case
    rng = np.random.default_rng(zlib.crc32(("pw-" + label).encode()))
    topk = _routing(rng, R, S, K, E, skew)
    ref = oracle.plan(topk, E, B, P)
    if ref.status != oracle.OK:
        pytest.skip("routing needs more slots than B")
    say(f"[case] prefetch_weight {label} R={R} E={E} B={B} shapes={shapes}")
    ctx, plan, etc = planned(moon, dev, topk, R, E, K, S, 8, B, P)
    try:
        assert np.array_equal(etc, ref.experts_to_copy)
        # bf16 weights, fp32 (e.g. scales) and raw bytes (packed formats)
        dts = [np.uint16, np.float32, np.uint8]
        experts, slots0 = [], []
        for i, shp in enumerate(shapes):
            dt = dts[i % 3]
            nbytes = int(np.prod(shp)) * np.dtype(dt).itemsize
            assert nbytes % 16 == 0
            x = rng.integers(0, 1 << 16, size=(E,) + shp).astype(dt) if dt != np.float32 else \
                rng.standard_normal((E,) + shp).astype(np.float32)
            experts.append(x)
            slots0.append(np.full((R, B) + shp, 0x5A if dt == np.uint8 else 77, dt))
        tdt = {np.uint16: torch.int16, np.float32: torch.float32, np.uint8: torch.uint8}
        xd = [torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).to(dev)
              for x in experts]
        sd = [torch.from_numpy(s.view(np.int16) if s.dtype == np.uint16 else s.copy()).to(dev)
              for s in slots0]
        assert all(t.dtype == tdt[x.dtype.type] for t, x in zip(xd, experts))
        moon.moon_prefetch_weight(ctx, plan, xd, sd)
        exp = oracle.prefetch_weight(etc, E, experts, [s.copy() for s in slots0])
        for t, (got, e) in enumerate(zip(sd, exp)):
            g = got.cpu().numpy()
            g = g.view(np.uint16) if e.dtype == np.uint16 else g
            assert np.array_equal(g.view(np.uint8), e.view(np.uint8)), f"tensor {t} differs"
        say(f"   slots used {int((etc >= 0).sum())}")
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_reduce_grad_small(env, case):
    import torch
    moon, dev = env
    label, R, E, K, S, B, P, skew, shapes = case
    rng = np.random.default_rng(zlib.crc32(("rg-" + label).encode()))
    topk = _routing(rng, R, S, K, E, skew)
    ref = oracle.plan(topk, E, B, P)
    if ref.status != oracle.OK:
        pytest.skip("routing needs more slots than B")
    shapes = [s for s in shapes if int(np.prod(s)) % 4 == 0]
    say(f"[case] reduce_grad {label} R={R} E={E} B={B} shapes={shapes}")
    ctx, plan, etc = planned(moon, dev, topk, R, E, K, S, 8, B, P)
    try:
        g0 = [rng.standard_normal((E,) + s).astype(np.float32) for s in shapes]
        s0 = [rng.standard_normal((R, B) + s).astype(np.float32) for s in shapes]
        gd = [torch.from_numpy(x.copy()).to(dev) for x in g0]
        sd = [torch.from_numpy(x.copy()).to(dev) for x in s0]
        moon.moon_reduce_grad(ctx, plan, gd, sd)
        eg, es = oracle.reduce_grad(etc, E, [x.copy() for x in g0], [x.copy() for x in s0])
        for t in range(len(shapes)):
            assert np.array_equal(gd[t].cpu().numpy().view(np.uint32), eg[t].view(np.uint32)), \
                f"expert gradients of tensor {t} differ"
            assert np.array_equal(sd[t].cpu().numpy().view(np.uint32), es[t].view(np.uint32)), \
                f"slot gradients of tensor {t} differ"
        say(f"   slots used {int((etc >= 0).sum())}, experts held "
            f"{len(np.unique(etc[etc >= 0]))}")
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


@pytest.mark.parametrize("R,E,B", [(2, 8, 4), (8, 64, 16)], ids=["8-slots", "128-slots"])
def test_weights_skip_on_bad_plan(env, R, E, B):
    """A plan whose device status is an error writes nothing (the per-slot
    copy up to 64 slots, the grouped copy beyond)."""
    import torch
    moon, dev = env
    K, S, P = 2, 32, 4
    topk = np.zeros((R, S, K), np.int32)
    topk[1, 3, 1] = E  # out of range
    ctx = moon.moon_ctx_create(R, E, K, S, 8, B, P)
    plan = moon.moon_plan_create(ctx)
    try:
        moon.moon_plan(ctx, pt.to_dev(topk, dev), None, plan)
        assert moon.moon_plan_status(plan) == moon.MOON_ERR_BAD_EXPERT
        x = torch.arange(E * 16, dtype=torch.float32, device=dev).reshape(E, 16)
        sl = torch.full((R, B, 16), 3.0, device=dev)
        moon.moon_prefetch_weight(ctx, plan, [x], [sl])
        moon.moon_reduce_grad(ctx, plan, [x], [sl])
        torch.cuda.synchronize()
        assert (sl == 3.0).all()
        assert torch.equal(x, torch.arange(E * 16, dtype=torch.float32, device=dev).reshape(E, 16))
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


def test_weights_reject_bad_shapes(env):
    import torch
    moon, dev = env
    ctx = moon.moon_ctx_create(2, 8, 2, 16, 8, 4, 4)
    plan = moon.moon_plan_create(ctx)
    try:
        x = torch.zeros((8, 12), dtype=torch.uint8, device=dev)  # 12-byte rows
        sl = torch.zeros((2, 4, 12), dtype=torch.uint8, device=dev)
        with pytest.raises(moon.MoonError) as ei:
            moon.moon_prefetch_weight(ctx, plan, [x], [sl])
        assert ei.value.status == moon.MOON_ERR_INVALID_ARG
        g = torch.zeros((8, 6), device=dev)
        sg = torch.zeros((2, 4, 6), device=dev)
        with pytest.raises(moon.MoonError):
            moon.moon_reduce_grad(ctx, plan, [g], [sg])
        with pytest.raises(ValueError):
            moon.moon_prefetch_weight(ctx, plan, [torch.zeros((7, 16), device=dev)],
                                      [torch.zeros((2, 4, 16), device=dev)])
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)


HP = 2048  # expert FFN intermediate width H' of the DSv3-shaped and R=16 workloads


@pytest.mark.parametrize("config,level", [("dsv3", 0), ("r16-e384-k8", 4)])
def test_weights_full_size(env, config, level):
    """One projection at the workload's real shape: [E, H, H'] bf16 weights and
    [E, H, H'] fp32 gradients with the slots the workload's plan uses."""
    import torch
    import synth.gpu as sg
    moon, dev = env
    wl = synth.workload(config, level)
    R, E, K, S, H, B, P = (wl[k] for k in ("R", "E", "K", "S", "H", "B", "P"))
    L = H * HP
    say(f"[case] weights full size {wl['name']} level {level} E={E} R={R} B={B} row={L}")
    ctx, plan, etc = planned(moon, dev, wl["topk"], R, E, K, S, H, B, P)
    try:
        ref = oracle.plan(wl["topk"], E, B, P)
        assert np.array_equal(etc, ref.experts_to_copy)
        used = np.argwhere(etc >= 0)
        say(f"   slots used {used.shape[0]}")
        kw = synth.stream_key(wl["seed"], TAG_W)
        w = sg.fill_bf16(torch.empty((E, L), dtype=torch.bfloat16, device=dev), kw)
        slots = torch.zeros((R, B, L), dtype=torch.bfloat16, device=dev)
        moon.moon_prefetch_weight(ctx, plan, [w], [slots])
        torch.cuda.synchronize()
        for u, j in used:
            assert torch.equal(slots[u, j].view(torch.int16), w[etc[u, j]].view(torch.int16)), \
                f"slot ({u},{j}) differs from expert {etc[u, j]}"
        unused = np.argwhere(etc < 0)
        for u, j in unused[:: max(1, unused.shape[0] // 16)]:
            assert not slots[u, j].view(torch.int16).any()
        # spot check one slot against the host generator
        u, j = used[0]
        assert np.array_equal(pt.dev_bits(slots[u, j, :4096]),
                              synth.bf16_normal(kw, int(etc[u, j]) * L, 4096))
        del w, slots
        torch.cuda.empty_cache()

        kg, ks = synth.stream_key(wl["seed"], TAG_G), synth.stream_key(wl["seed"], TAG_SG)
        g = sg.fill_bf16(torch.empty((E, L), dtype=torch.bfloat16, device=dev), kg).float()
        sgr = sg.fill_bf16(torch.empty((R, B, L), dtype=torch.bfloat16, device=dev), ks).float()
        torch.cuda.synchronize()
        moon.moon_reduce_grad(ctx, plan, [g], [sgr])
        torch.cuda.synchronize()
        held = np.unique(etc[etc >= 0])
        rng = np.random.default_rng(wl["seed"])
        picks = rng.choice(held, size=min(3, held.shape[0]), replace=False)
        cols = np.arange(0, L, 7)[:65536]  # a strided sample of each row
        npre = int(cols[-1]) + 1

        def regen(key, row):
            return synth.bf16_to_float(synth.bf16_normal(key, int(row) * L, npre))[cols]

        for e in picks:
            slots_e = np.argwhere(etc == e)  # (u, j), ascending u
            g0 = regen(kg, e)[None, :]
            s0 = np.stack([regen(ks, int(u) * B + int(j)) for u, j in slots_e])
            # the expert's slots alone, as a one-expert problem for the oracle
            etc1 = np.full((R, B), -1, np.int32)
            s1 = np.zeros((R, B, cols.shape[0]), np.float32)
            for i, (u, j) in enumerate(slots_e):
                etc1[u, j] = 0
                s1[u, j] = s0[i]
            eg, _ = oracle.reduce_grad(etc1, 1, [g0.copy()], [s1])
            got = g[int(e)].cpu().numpy()[cols]
            assert np.array_equal(got.view(np.uint32), eg[0][0].view(np.uint32)), \
                f"expert {e} reduction differs"
        for u, j in used:
            assert not sgr[u, j].any(), f"slot ({u},{j}) not cleared"
        notheld = np.setdiff1d(np.arange(E), held)[:2]
        for e in notheld:
            g0 = synth.bf16_to_float(synth.bf16_normal(kg, int(e) * L, 4096))
            assert np.array_equal(g[int(e), :4096].cpu().numpy(), g0)
        say(f"   experts held {held.shape[0]}, checked {picks.tolist()}")
    finally:
        moon.moon_plan_destroy(plan)
        moon.moon_ctx_destroy(ctx)
