"""Pins of the oracle's weight prefetch and gradient reduction (CPU only).

Weight prefetch is pinned to the planner through the property the pages give
it (README, weight buffer: the planner points a duplicated expert's token
segment at a prefetch slot via cu_seqlens): for every route, the weight row
the grouped GEMM of its physical group reads (row g < E of the expert rows,
or slot g - E of its rank) must hold the weights of the expert the route
chose.  Gradient reduction is pinned by an exact integer-valued case against
numpy's scatter-add, conservation of the total, the cleared slots, and two
rounding cases that only the pages' order (seed with the expert's own
gradient, then ranks ascending) gets right.
"""
import numpy as np
import pytest

import oracle
import plan_checks as pc
from test_oracle_plan import rand_topk


def route_groups(pl):
    """(dest rank, physical group) of every route, from dst and cu_seqlens."""
    R, NvS = pl.R, pl.NvS
    G = pc.decode(pl.dst).reshape(-1).astype(np.int64)
    u = G // NvS
    row = G % NvS
    g = np.array([np.searchsorted(pl.cu_seqlens[uu], rr, side="right")
                  for uu, rr in zip(u, row)], np.int64)
    return u, g


WEIGHT_CASES = [
    # R, E, K, S, B, P, skew
    (2, 8, 2, 64, 4, 8, 0.0),
    (4, 16, 4, 40, 4, 4, 2.0),
    (3, 12, 3, 30, 4, 2, 3.0),
    (8, 64, 6, 64, 8, 16, 1.5),
]


@pytest.mark.parametrize("case", WEIGHT_CASES)
def test_prefetched_slot_serves_the_routes_of_its_group(case):
    R, E, K, S, B, P, skew = case
    rng = np.random.default_rng(100 + R * 7 + K)
    topk = rand_topk(rng, R, S, K, E, skew=skew)
    pl = oracle.plan(topk, E, B, P)
    assert pl.status == oracle.OK
    # three "projections" of different byte widths and dtypes, plus a scale
    experts = [rng.integers(0, 1 << 16, size=(E, 3, 5), dtype=np.uint16),
               rng.standard_normal((E, 7)).astype(np.float32),
               rng.integers(0, 256, size=(E, 16), dtype=np.uint8)]
    canary = [np.full((R, B) + x.shape[1:], v, x.dtype)
              for x, v in zip(experts, (0xA5A5, -123.5, 0xA5))]
    slots = [c.copy() for c in canary]
    oracle.prefetch_weight(pl.experts_to_copy, E, experts, slots)
    u, g = route_groups(pl)
    chosen = topk.reshape(-1)
    for x, sl in zip(experts, slots):
        served = np.where((g < E)[:, None], x[np.minimum(g, E - 1)].reshape(len(g), -1),
                          sl[u, np.maximum(g - E, 0)].reshape(len(g), -1))
        assert np.array_equal(served, x[chosen].reshape(len(g), -1))
    # unused slots keep their bytes
    unused = pl.experts_to_copy < 0
    for c, sl in zip(canary, slots):
        assert np.array_equal(sl[unused], c[unused])
    # a skewed routing must have exercised the slots
    if skew > 0:
        assert (~unused).any()


def test_prefetch_without_used_slots_changes_nothing():
    R, E, B = 4, 8, 2
    etc = np.full((R, B), -1, np.int32)
    x = np.arange(E * 6, dtype=np.float32).reshape(E, 6)
    sl = np.full((R, B, 6), 7.0, np.float32)
    oracle.prefetch_weight(etc, E, [x], [sl])
    assert (sl == 7.0).all()


def _random_etc(rng, R, E, B):
    """Slots like the planner's: each rank's used slots hold distinct experts,
    compact from slot 0, ascending."""
    etc = np.full((R, B), -1, np.int32)
    for u in range(R):
        n = int(rng.integers(0, B + 1))
        etc[u, :n] = np.sort(rng.choice(E, n, replace=False))
    return etc


@pytest.mark.parametrize("seed", range(4))
def test_reduce_grad_integer_values_equal_scatter_add(seed):
    rng = np.random.default_rng(seed)
    R, E, B, L = 5, 10, 4, 12
    etc = _random_etc(rng, R, E, B)
    g0 = [rng.integers(-50, 50, size=(E, L)).astype(np.float32) for _ in range(3)]
    s0 = [rng.integers(-50, 50, size=(R, B, L)).astype(np.float32) for _ in range(3)]
    g, s = [x.copy() for x in g0], [x.copy() for x in s0]
    oracle.reduce_grad(etc, E, g, s)
    used = etc >= 0
    for t in range(3):
        exp = g0[t].astype(np.float64)
        np.add.at(exp, etc[used], s0[t][used].astype(np.float64))  # exact: small integers
        assert np.array_equal(g[t].astype(np.float64), exp)
        assert (s[t][used] == 0).all() and not np.signbit(s[t][used]).any()
        assert np.array_equal(s[t][~used], s0[t][~used])
        # conservation of the total
        assert g[t].astype(np.float64).sum() == g0[t].astype(np.float64).sum() + \
            s0[t][used].astype(np.float64).sum()


def test_reduce_grad_seeds_with_the_expert_gradient():
    """1 + 2^-24 rounds back to 1 in fp32: adding two such slot values one by
    one to a seed of 1 keeps 1, while summing the slots first gives
    1 + 2^-23."""
    R, E, B = 2, 2, 1
    etc = np.array([[0], [0]], np.int32)
    g = [np.array([[1.0], [5.0]], np.float32)]
    s = [np.full((R, B, 1), 2.0 ** -24, np.float32)]
    oracle.reduce_grad(etc, E, g, s)
    assert g[0][0, 0] == np.float32(1.0) and g[0][1, 0] == np.float32(5.0)


def test_reduce_grad_visits_ranks_ascending():
    """Seed 0, slots 1, 2^-24, 2^-24 on ranks 0, 1, 2: ascending gives 1,
    descending gives 1 + 2^-23."""
    R, E, B = 3, 3, 1
    etc = np.array([[2], [2], [2]], np.int32)
    g = [np.zeros((E, 1), np.float32)]
    s = [np.array([1.0, 2.0 ** -24, 2.0 ** -24], np.float32).reshape(R, B, 1)]
    oracle.reduce_grad(etc, E, g, s)
    assert g[0][2, 0] == np.float32(1.0)
    assert (g[0][:2] == 0).all() and (s[0] == 0).all()


def test_prefetch_then_reduce_round_trip_on_a_plan():
    """Slots filled by the prefetch, their gradients set to the prefetched
    weights, then reduced: every expert row gains its weights times the
    number of slots that held it (exact for small integers)."""
    rng = np.random.default_rng(9)
    R, E, K, S, B, P = 4, 16, 4, 40, 4, 4
    topk = rand_topk(rng, R, S, K, E, skew=2.5)
    pl = oracle.plan(topk, E, B, P)
    w = rng.integers(-8, 8, size=(E, 6)).astype(np.float32)
    sl = np.zeros((R, B, 6), np.float32)
    oracle.prefetch_weight(pl.experts_to_copy, E, [w], [sl])
    g = np.zeros((E, 6), np.float32)
    oracle.reduce_grad(pl.experts_to_copy, E, [g], [sl])
    cnt = np.bincount(pl.experts_to_copy[pl.experts_to_copy >= 0], minlength=E)
    assert cnt.sum() > 0
    assert np.array_equal(g, w * cnt[:, None].astype(np.float32))
    assert (sl == 0).all()
