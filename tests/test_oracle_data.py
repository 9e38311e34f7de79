"""Pins of the CPU oracle's dispatch, combine, rounding and prefetch index."""
import numpy as np
import pytest
import torch

import oracle
import plan_checks as pc
from test_oracle_plan import rand_topk


def _bits(x_f32):
    """float32 -> bf16 bits with torch's CPU conversion (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rand_bf16(rng, shape):
    return _bits(rng.standard_normal(shape).astype(np.float32))


CASES = [
    # R, E, K, S, B, P, H, skew
    (1, 4, 2, 8, 4, 4, 16, 0.0),
    (2, 8, 2, 64, 4, 8, 128, 0.0),
    (3, 12, 3, 20, 4, 4, 24, 2.0),
    (4, 16, 4, 16, 4, 8, 64, 3.0),
    (4, 8, 1, 9, 2, 2, 8, 1.0),
]


def test_single_rank_dispatch_is_a_sort_permute():
    """R = 1: the window is the token rows permuted by a stable sort of the
    route experts, each expert block zero-padded to P."""
    rng = np.random.default_rng(1)
    S, K, E, P, H = 12, 3, 5, 4, 8
    topk = rng.integers(0, E, size=(1, S, K)).astype(np.int32)
    hidden = _rand_bf16(rng, (1, S, H))
    w = rng.random((1, S, K)).astype(np.float32)
    pl = oracle.plan(topk, E, E, P)
    win, wwin = oracle.dispatch(pl, hidden, w)
    flat = topk.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    exp_rows, exp_w = [], []
    pos = 0
    for e in range(E):
        ids = order[pos:pos + counts[e]]
        pos += counts[e]
        if counts[e] == 0:
            continue
        pad = -(-counts[e] // P) * P - counts[e]
        exp_rows += [hidden[0, i // K] for i in ids] + [np.zeros(H, np.uint16)] * pad
        exp_w += [w.reshape(-1)[i] for i in ids] + [0.0] * pad
    n = len(exp_rows)
    assert (win[:n] == np.stack(exp_rows)).all()
    assert (wwin[:n] == np.asarray(exp_w, np.float32)).all()


@pytest.mark.parametrize("case", CASES)
def test_dispatch_content(case):
    R, E, K, S, B, P, H, skew = case
    rng = np.random.default_rng(R * 7 + K)
    topk = rand_topk(rng, R, S, K, E, distinct=K <= E, skew=skew)
    hidden = _rand_bf16(rng, (R, S, H))
    w = rng.random((R, S, K)).astype(np.float32)
    pl = oracle.plan(topk, E, B, P)
    assert pl.status == oracle.OK
    win, wwin = oracle.dispatch(pl, hidden, w, win=np.full((R * pl.NvS, H), 0xABCD, np.uint16),
                                wwin=np.full(R * pl.NvS, 7.0, np.float32))
    pv = pc.PlanView.of(pl)
    pc.check_windows(pv, hidden, w, win, wwin)
    # rows that no group covers are left as they were
    src = oracle.row_sources(pl)
    assert (win[src == -2] == 0xABCD).all() and (wwin[src == -2] == 7.0).all()
    # row_sources agrees with dst
    routes = src[src >= 0]
    assert np.unique(routes).shape[0] == R * S * K
    # without weights the weight window is not touched
    win2, wwin2 = oracle.dispatch(pl, hidden, None)
    assert wwin2 is None and (win2[src >= 0] == win[src >= 0]).all()


@pytest.mark.parametrize("case", CASES)
def test_unweighted_round_trip_is_k_times_x(case):
    """combine(dispatch(x)) without weights = K * x exactly: K copies of one
    bf16 value sum exactly in any order, so only the final rounding remains,
    and torch's float32 -> bf16 conversion supplies it independently."""
    R, E, K, S, B, P, H, skew = case
    rng = np.random.default_rng(R * 11 + K)
    topk = rand_topk(rng, R, S, K, E, distinct=K <= E, skew=skew)
    hidden = _rand_bf16(rng, (R, S, H))
    pl = oracle.plan(topk, E, B, P)
    win, _ = oracle.dispatch(pl, hidden, None)
    out, _, acc = oracle.combine(pl, win, None, weighted=False)
    assert (acc == K * _f32(hidden).astype(np.float64)).all()
    assert (out == _bits(K * _f32(hidden))).all()


@pytest.mark.parametrize("case", CASES)
def test_weighted_combine_brute_force(case):
    """Route-major fp64 brute force: accumulate w * y over all routes into
    their tokens, then compare the pre-rounding sum and the rounding."""
    R, E, K, S, B, P, H, skew = case
    rng = np.random.default_rng(R * 13 + K)
    topk = rand_topk(rng, R, S, K, E, distinct=K <= E, skew=skew)
    w = rng.random((R, S, K)).astype(np.float32)
    pl = oracle.plan(topk, E, B, P)
    y = _rand_bf16(rng, (R * pl.NvS, H))
    _, wwin = oracle.dispatch(pl, np.zeros((R, S, H), np.uint16), w)
    out, wsk, acc = oracle.combine(pl, y, wwin, weighted=True)
    ref = np.zeros((R * S, H), np.float64)
    G = pc.decode(pl.dst).reshape(-1)
    for i in range(R * S * K):
        ref[i // K] += np.float64(wwin[G[i]]) * _f32(y[G[i]]).astype(np.float64)
    assert np.allclose(acc.reshape(R * S, H), ref, rtol=1e-12, atol=1e-12)
    assert (wsk.view(np.uint32) == w.view(np.uint32)).all()
    # out is the nearest bf16 to acc: no neighbour is closer
    o = _f32(out).astype(np.float64).reshape(-1)
    a = acc.reshape(-1)
    ob = out.reshape(-1).astype(np.int64)
    up = _f32(((ob + 1) & 0xFFFF).astype(np.uint16)).astype(np.float64)
    dn = _f32(((ob - 1) & 0xFFFF).astype(np.uint16)).astype(np.float64)
    assert (np.abs(o - a) <= np.abs(up - a)).all() and (np.abs(o - a) <= np.abs(dn - a)).all()


def test_combine_rows_matches_full_combine():
    rng = np.random.default_rng(5)
    R, E, K, S, B, P, H = 3, 12, 3, 20, 4, 4, 24
    topk = rand_topk(rng, R, S, K, E, skew=1.0)
    w = rng.random((R, S, K)).astype(np.float32)
    pl = oracle.plan(topk, E, B, P)
    y = _rand_bf16(rng, (R * pl.NvS, H))
    _, wwin = oracle.dispatch(pl, np.zeros((R, S, H), np.uint16), w)
    out, wsk, acc = oracle.combine(pl, y, wwin, weighted=True)
    toks = np.array([0, 5, 17, R * S - 1])
    dst_tok = pl.dst.reshape(R * S, K)[toks]
    rows = np.unique(pc.decode(dst_tok).reshape(-1))
    o2, w2, a2 = oracle.combine_rows(dst_tok, rows, y[rows], wwin[rows], weighted=True)
    assert (o2 == out.reshape(R * S, H)[toks]).all()
    assert (a2 == acc.reshape(R * S, H)[toks]).all()
    assert (w2 == wsk.reshape(R * S, K)[toks]).all()


def test_bf16_rounding_against_torch_on_float32_values():
    rng = np.random.default_rng(6)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # subnormal range
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1.00390625, 1.01171875], np.float32),
    ])
    exp = _bits(x)
    got = np.array([oracle.bf16_from_double(float(v)) for v in x], np.uint16)
    assert (got == exp).all()


def test_bf16_rounding_of_doubles_is_single_rounding():
    # 1 + 2^-8 + 2^-30: nearest bf16 is 1 + 2^-7 (above the halfway point);
    # rounding through float32 first would land exactly on the tie and go to 1.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.bf16_from_double(v) == 0x3F81
    assert oracle.bf16_from_double(1.0 + 2.0 ** -8) == 0x3F80  # exact tie -> even
    assert oracle.bf16_from_double(1.0 + 3 * 2.0 ** -8) == 0x3F82  # tie -> even (up)


def test_prefetch_index_splits_expert_ids():
    rng = np.random.default_rng(7)
    R, E, K, S, B, P = 4, 16, 2, 32, 4, 4
    topk = rand_topk(rng, R, S, K, E, skew=3.0)
    pl = oracle.plan(topk, E, B, P)
    idx = oracle.prefetch_index(pl)
    Eg = E // R
    etc = pl.experts_to_copy
    used = etc >= 0
    assert used.any()
    assert (idx[~used] == -1).all()
    owner, local = idx[..., 0][used], idx[..., 1][used]
    assert (owner * Eg + local == etc[used]).all()
    assert ((0 <= local) & (local < Eg)).all() and ((0 <= owner) & (owner < R)).all()
