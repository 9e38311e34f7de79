"""The padded serving workload (MoonEP vLLM integration page: the buffer pool's
power-of-two capacities; padding and invalid ids mapped to expert 0 with
weight 0; combine as a plain K-sum), on the CPU oracle.

Pins: the capacity rule's closed forms, the generator's structure, the plan's
guarantees under a hot expert with repeated ids (exact balance, one donor per
receiver, slot budget, sign rule and duplicate records), the histogram input
check, and the closed form combine(dispatch(x)) = K*x without weights, which
makes every pad token's output exactly zero.
"""
import numpy as np
import pytest
import torch

import oracle
import plan_checks as pc
import synth

NARROW_H = 64  # the row width does not enter the plan; narrow rows keep the CPU cases small


def _f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bits(x_f32):
    return torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("n,cap", [(0, 128), (1, 128), (128, 128), (129, 256), (256, 256),
                                   (257, 512), (3000, 4096), (4096, 4096), (9000, 4096)])
def test_capacity_is_the_smallest_power_of_two_in_range(n, cap):
    assert synth.serving_capacity(n, 128, 4096) == cap


@pytest.mark.parametrize("level", [0, 1])
def test_generator_structure(level):
    wl = synth.serving_workload(level)
    lv = synth.SERVING_LEVELS[level]
    R, S, K, E = wl["R"], wl["S"], wl["K"], wl["E"]
    n = wl["n_tok"]
    assert ((n >= lv["lo"]) & (n <= lv["hi"])).all()
    assert S & (S - 1) == 0 and S >= n.max() and (S // 2 < n.max() or S == 128)
    topk, w = wl["topk"], wl["w"]
    assert topk.shape == (R, S, K) and w.shape == (R, S, K)
    assert ((topk >= 0) & (topk < E)).all()
    pad = np.arange(S)[None, :] >= n[:, None]
    assert (topk[pad] == 0).all() and (w[pad] == 0).all()
    real = ~pad
    # real tokens: softmax weights (zero only where an invalid slot was masked)
    zero = w[real] == 0
    assert (topk[real][zero] == 0).all()
    frac = zero.mean()
    assert 0.5 / wl["invalid_every"] < frac < 2.0 / wl["invalid_every"]
    tpe = np.stack([np.bincount(topk[r].reshape(-1), minlength=E) for r in range(R)])
    assert (tpe == wl["tokens_per_expert"]).all()


def _plan(wl):
    pl = oracle.plan(wl["topk"], wl["E"], wl["B"], wl["P"], wl["tokens_per_expert"])
    assert pl.status == oracle.OK, pl.status
    return pl


@pytest.mark.parametrize("level", [0, 1])
def test_plan_balances_the_hot_expert(level):
    wl = synth.serving_workload(level)
    pl = _plan(wl)
    pv = pc.PlanView.of(pl)
    pc.check_all(pv, wl["topk"], readings=True, dups=(level == 0))
    R, S, K = wl["R"], wl["S"], wl["K"]
    C = S * K
    # Expert 0 carries more than one rank's share, so it must be spread over
    # at least ceil(T0 / C) destination ranks.
    t0 = int((wl["topk"] == 0).sum())
    assert t0 > C
    G, u, row, g = pc.route_table(pv)
    on0 = wl["topk"].reshape(-1) == 0
    assert np.unique(u[on0]).shape[0] >= -(-t0 // C)


def test_pad_tokens_deduplicate_to_one_row_per_rank():
    """A pad token sends all K routes to expert 0: one primary per destination
    rank, the rest duplicates of it."""
    wl = synth.serving_workload(0)
    pl = _plan(wl)
    R, S, K = wl["R"], wl["S"], wl["K"]
    dst = pl.dst.reshape(R, S, K).astype(np.int64)
    u = pc.decode(dst) // pl.NvS
    pad = np.arange(S)[None, :] >= wl["n_tok"][:, None]
    for r in range(R):
        for s in np.nonzero(pad[r])[0]:
            ranks = u[r, s]
            assert (dst[r, s] >= 0).sum() == np.unique(ranks).shape[0]
    total_dups = int(pl.dup_counts[:, 1].sum())
    assert total_dups >= int(pad.sum()) * (K - 1) - R * S  # nearly every pad route beyond the first
    pc.check_dups_canonical(pc.PlanView.of(pl))


def test_histogram_input_mismatch_is_reported():
    wl = synth.serving_workload(0)
    tpe = wl["tokens_per_expert"].copy()
    tpe[3, 0] -= 1
    tpe[3, 1] += 1
    pl = oracle.plan(wl["topk"], wl["E"], wl["B"], wl["P"], tpe)
    assert pl.status == oracle.HISTOGRAM


def test_unweighted_round_trip_zeroes_pad_tokens():
    """combine(dispatch(x)) without weights is K*x exactly (K equal bf16 values
    sum exactly in fp32); pad tokens have x = 0, so their output is +0."""
    wl = dict(synth.serving_workload(0))
    wl["H"] = NARROW_H
    hidden = synth.serving_hidden_bf16(wl)
    pl = _plan(wl)
    win, wwin = oracle.dispatch(pl, hidden, wl["w"])
    pc.check_windows(pc.PlanView.of(pl), hidden, wl["w"], win, wwin)
    out, wsk, acc = oracle.combine(pl, win, wwin, weighted=False)
    K = wl["K"]
    assert (acc == K * _f32(hidden).astype(np.float64)).all()
    assert (out == _bits(K * _f32(hidden))).all()
    pad = np.arange(wl["S"])[None, :] >= wl["n_tok"][:, None]
    assert (out[pad] == 0).all()
    assert (wsk.view(np.uint32) == wl["w"].view(np.uint32)).all()


def test_empty_and_full_ranks():
    """One rank with no real tokens (its whole capacity is padding, all on
    expert 0) and one filled to capacity: still a valid, balanced plan, and
    the empty rank's outputs are all zero."""
    n = [0, 256, 100, 0, 37, 256, 1, 200]
    wl = dict(synth.serving_workload(0, n_tok=n))
    assert wl["S"] == 256
    assert (wl["topk"][0] == 0).all() and (wl["topk"][3] == 0).all()
    wl["H"] = NARROW_H
    pl = _plan(wl)
    pc.check_all(pc.PlanView.of(pl), wl["topk"])
    hidden = synth.serving_hidden_bf16(wl)
    win, _ = oracle.dispatch(pl, hidden, None)
    out, _, _ = oracle.combine(pl, win, None, weighted=False)
    assert (out[0] == 0).all() and (out[3] == 0).all()
    assert (out == _bits(wl["K"] * _f32(hidden))).all()
