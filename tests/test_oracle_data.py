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


def _assert_nearest_bf16(out, acc):
    """No bf16 bit neighbour of out is closer to acc.  Stepping past +-0 or
    the largest finite value gives a NaN pattern, which is no competitor."""
    o = _f32(out).astype(np.float64).reshape(-1)
    a = np.asarray(acc, np.float64).reshape(-1)
    ob = np.asarray(out).reshape(-1).astype(np.int64)
    up = _f32(((ob + 1) & 0xFFFF).astype(np.uint16)).astype(np.float64)
    dn = _f32(((ob - 1) & 0xFFFF).astype(np.uint16)).astype(np.float64)
    d_up = np.nan_to_num(np.abs(up - a), nan=np.inf)
    d_dn = np.nan_to_num(np.abs(dn - a), nan=np.inf)
    assert (np.abs(o - a) <= d_up).all() and (np.abs(o - a) <= d_dn).all()


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
    # out, the fp32 sum rounded to bf16, lies within the rounding of bf16
    # plus the fp32 error of a K-term sum of the exact value
    absum = np.zeros((R * S, H), np.float64)
    for i in range(R * S * K):
        absum[i // K] += abs(np.float64(wwin[G[i]])) * np.abs(_f32(y[G[i]]).astype(np.float64))
    g = 1.01 * K * 2.0 ** -24
    lim = 2.0 ** -8 * (np.abs(acc.reshape(R * S, H)) + g * absum) + g * absum + 1e-30
    assert (np.abs(_f32(out).reshape(R * S, H).astype(np.float64) - acc.reshape(R * S, H))
            <= lim).all()


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
        # infinities, the largest finite float32 (rounds up to infinity) and
        # the largest finite bf16, 0x7F7F (kept)
        np.array([np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 3.3895314e38, -3.3895314e38],
                 np.float32),
    ])
    exp = _bits(x)
    got = np.array([oracle.bf16_from_double(float(v)) for v in x], np.uint16)
    assert (got == exp).all()


def test_bf16_rounding_keeps_nan_a_nan():
    """A NaN sum rounds to a bf16 NaN (exponent all ones, mantissa not zero),
    whatever its sign or payload; which NaN is a convention (the oracle and
    the kernels use 0x7FC0; torch's CPU conversion gives 0xFFFF)."""
    for bits in (0x7FC00000, 0xFFC00000, 0x7F800001, 0x7FBFFFFF, 0xFFFFFFFF):
        v = float(np.array([bits], np.uint32).view(np.float32)[0])
        r = oracle.bf16_from_double(v)
        assert (r & 0x7F80) == 0x7F80 and (r & 0x007F) != 0, (hex(bits), hex(r))


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


# ---- combine with the duplicate prologue -------------------------------------

def _prologue_brute_force(pl, y, wwin, weighted):
    """Fold driven by the plan's duplicate records (the pages' structure): per
    record, primary then its duplicate rows, fp32 separate multiply and add
    (numpy float32), rounded by torch; then a route-major float64 sum over
    primary routes, folded primaries with coefficient 1."""
    R, S, K, NvS = pl.R, pl.S, pl.K, pl.NvS
    H = y.shape[1]
    folded = y.copy()
    is_folded = np.zeros(R * NvS, bool)
    for u in range(R):
        for j in range(int(pl.dup_counts[u, 0])):
            prow, lb, m = (int(v) for v in pl.dup_groups[u, j])
            rows = [u * NvS + prow] + [u * NvS + int(pl.dup_loffs[u, lb + i]) for i in range(m)]
            a = np.zeros(H, np.float32)
            for G in rows:
                c = np.float32(wwin[G]) if weighted else np.float32(1.0)
                a = (a + (c * _f32(y[G])).astype(np.float32)).astype(np.float32)
            folded[rows[0]] = _bits(a)
            is_folded[rows[0]] = True
    acc = np.zeros((R * S, H), np.float64)
    dst = pl.dst.reshape(R * S, K)
    for t in range(R * S):
        for k in range(K):
            d = int(dst[t, k])
            if d < 0:
                continue
            if is_folded[d]:
                acc[t] += _f32(folded[d]).astype(np.float64)
            else:
                c = np.float64(wwin[d]) if weighted else 1.0
                acc[t] += c * _f32(y[d]).astype(np.float64)
    return folded, is_folded, acc


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("weighted", [True, False])
def test_prologue_combine_against_duplicate_records(case, weighted):
    R, E, K, S, B, P, H, skew = case
    rng = np.random.default_rng(R * 17 + K + int(weighted))
    topk = rand_topk(rng, R, S, K, E, distinct=K <= E, skew=skew)
    w = rng.random((R, S, K)).astype(np.float32)
    pl = oracle.plan(topk, E, B, P)
    y = _rand_bf16(rng, (R * pl.NvS, H))
    _, wwin = oracle.dispatch(pl, np.zeros((R, S, H), np.uint16), w)
    out, wsk, acc, folded = oracle.combine_prologue(pl, y, wwin, weighted=weighted)
    f_ref, is_f, acc_ref = _prologue_brute_force(pl, y, wwin, weighted)
    assert int(is_f.sum()) == int(pl.dup_counts[:, 0].sum())
    assert (folded == f_ref).all()
    assert (acc.reshape(R * S, H) == acc_ref).all()
    # out is the nearest bf16 to acc
    _assert_nearest_bf16(out, acc)
    assert (wsk.view(np.uint32) == w.view(np.uint32)).all()


def test_prologue_unweighted_power_of_two_groups_is_k_times_x():
    """K = 4 over 4 ranks of 4 experts; every token splits its routes over
    ranks in groups of 1, 2 or 4, the ranks shifted cyclically so that every
    rank's load is exactly S*K and nothing moves to a slot.  Folding m copies
    of x gives m*x exactly (m a power of two, so the bf16 rounding of the fold
    is exact), the outer sum is exact, so out = 4x exactly."""
    rng = np.random.default_rng(21)
    R, E, K, S, B, P, H = 4, 16, 4, 24, 4, 4, 32
    patterns = [(1, 1, 1, 1), (2, 1, 1), (2, 2), (4,)]
    topk = np.empty((R * S, K), np.int32)
    for t in range(R * S):
        sizes, shift = patterns[(t // R) % len(patterns)], t % R
        row = []
        for j, m in enumerate(sizes):
            rk = (shift + j) % R
            row += list(rk * 4 + rng.permutation(4)[:m])
        topk[t] = rng.permutation(np.array(row))
    topk = topk.reshape(R, S, K)
    hidden = _rand_bf16(rng, (R, S, H))
    pl = oracle.plan(topk, E, B, P)
    assert pl.status == oracle.OK and int(pl.dup_counts[:, 0].sum()) > 0
    assert int(pl.remote_stats.sum()) == 0
    win, _ = oracle.dispatch(pl, hidden, None)
    out, _, acc, folded = oracle.combine_prologue(pl, win, None, weighted=False)
    assert (acc == K * _f32(hidden).astype(np.float64)).all()
    assert (out == _bits(K * _f32(hidden))).all()


def test_prologue_without_duplicates_equals_plain_combine():
    """Every token's K routes on K distinct ranks, shifted cyclically so that
    every rank's load is exactly S*K and nothing moves to a slot: nothing to
    fold, so the prologue variant is the plain combine, bit for bit."""
    rng = np.random.default_rng(22)
    R, E, K, S, B, P, H = 4, 16, 3, 20, 4, 4, 24
    topk = np.empty((R * S, K), np.int32)
    for t in range(R * S):
        ranks = (t + np.arange(K)) % R
        topk[t] = rng.permutation(ranks * 4 + rng.integers(0, 4, size=K))
    topk = topk.reshape(R, S, K)
    w = rng.random((R, S, K)).astype(np.float32)
    pl = oracle.plan(topk, E, B, P)
    assert int(pl.dup_counts.sum()) == 0 and int(pl.remote_stats.sum()) == 0
    y = _rand_bf16(rng, (R * pl.NvS, H))
    _, wwin = oracle.dispatch(pl, np.zeros((R, S, H), np.uint16), w)
    o1, w1, a1 = oracle.combine(pl, y, wwin, weighted=True)
    o2, w2, a2, f2 = oracle.combine_prologue(pl, y, wwin, weighted=True)
    assert (o1 == o2).all() and (a1 == a2).all() and (w1 == w2).all() and (f2 == y).all()


def test_prologue_rows_matches_full():
    rng = np.random.default_rng(23)
    R, E, K, S, B, P, H = 3, 12, 4, 20, 4, 4, 24
    topk = rand_topk(rng, R, S, K, E, skew=1.0)
    w = rng.random((R, S, K)).astype(np.float32)
    pl = oracle.plan(topk, E, B, P)
    y = _rand_bf16(rng, (R * pl.NvS, H))
    _, wwin = oracle.dispatch(pl, np.zeros((R, S, H), np.uint16), w)
    out, wsk, acc, folded = oracle.combine_prologue(pl, y, wwin, weighted=True)
    toks = np.array([0, 3, 17, 31, R * S - 1])
    dst_tok = pl.dst.reshape(R * S, K)[toks]
    rows = np.unique(pc.decode(dst_tok).reshape(-1))
    o2, w2, a2, f2 = oracle.combine_prologue_rows(dst_tok, rows, y[rows], pl.NvS, wwin[rows],
                                                  weighted=True)
    assert (o2 == out.reshape(R * S, H)[toks]).all()
    assert (a2 == acc.reshape(R * S, H)[toks]).all()
    assert (w2 == wsk.reshape(R * S, K)[toks]).all()
    assert (f2 == folded[rows]).all()


def _one_token_plan(K, E=8):
    """R = 1, S = 1: a token whose K routes go to K distinct experts, so row
    k of the window is route k's row (global route order within groups)."""
    topk = np.arange(K, dtype=np.int32).reshape(1, 1, K)
    pl = oracle.plan(topk, E, E, 1)
    assert pl.status == oracle.OK
    return pl


def _rows_for(pl, vals):
    """A window whose route rows hold the given bf16 bit patterns (H = 1)."""
    y = np.zeros((pl.NvS, 1), np.uint16)
    G = pc.decode(pl.dst).reshape(-1)
    for k, v in enumerate(vals):
        y[G[k], 0] = v
    return y, G


def test_combine_accumulates_in_fp32_in_ascending_k():
    """Rows 2^24, 1, -2^24 (unweighted): in fp32, ascending k, 2^24 + 1 rounds
    back to 2^24 (a tie, to even) and the sum is 0; the exact sum is 1."""
    pl = _one_token_plan(3)
    y, _ = _rows_for(pl, [0x4B80, 0x3F80, 0xCB80])  # 2^24, 1.0, -2^24 as bf16 bits
    out, _, acc = oracle.combine(pl, y, None, weighted=False)
    assert acc[0, 0, 0] == 1.0
    assert out[0, 0, 0] == 0x0000


def test_combine_rounds_product_and_sum_separately():
    """c0 = 1, y0 = 1; c1 = 1 + 2^-23, y1 = 1 + 2^-7.  The product rounds to
    1 + 2^-7 + 2^-23 (the 2^-30 term is below half an ulp); the sum
    2 + 2^-7 + 2^-23 is a tie in fp32 and goes to even, 2 + 2^-7, which is a
    tie in bf16 and goes to even, 2.0 (0x4000).  A fused multiply-add (or an
    exact sum) keeps the 2^-30 and ends at 2 + 2^-6 (0x4001)."""
    pl = _one_token_plan(2)
    y, G = _rows_for(pl, [0x3F80, 0x3F81])  # 1.0, 1 + 2^-7
    wnvs = np.zeros(pl.NvS, np.float32)
    wnvs[G[0]] = 1.0
    wnvs[G[1]] = np.float32(1.0 + 2.0 ** -23)
    out, _, acc = oracle.combine(pl, y, wnvs, weighted=True)
    assert out[0, 0, 0] == 0x4000
    assert _bits(np.float32(acc[0, 0, 0]))[()] == 0x4001


def test_combine_single_route_is_one_rounded_product():
    """K = 1: out = bf16(fp32(c * y)), torch's conversion supplying the bf16."""
    rng = np.random.default_rng(21)
    pl = _one_token_plan(1)
    for _ in range(50):
        yb = _rand_bf16(rng, (1,))
        c = np.float32(rng.random() * 3)
        y, G = _rows_for(pl, [int(yb[0])])
        wnvs = np.zeros(pl.NvS, np.float32)
        wnvs[G[0]] = c
        out, _, _ = oracle.combine(pl, y, wnvs, weighted=True)
        assert out[0, 0, 0] == _bits(np.array([c * _f32(yb)[0]], np.float32))[0]
