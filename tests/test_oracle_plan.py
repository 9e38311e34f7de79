"""Pins of the CPU oracle's planner against what the pages and mathematics fix.

Each test ties the oracle to something other than itself: numpy's bincount and
stable argsort (textbook special cases), exhaustive brute force over small
load vectors, a hand-worked example, and the invariants of plan_checks.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import plan_checks as pc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_topk(rng, R, S, K, E, distinct=True, skew=0.0):
    """Routes for tests: distinct per token (or with repeats), optionally skewed."""
    p = np.exp(-skew * np.log(np.arange(1, E + 1)))
    p = p[rng.permutation(E)]
    p /= p.sum()
    out = np.empty((R * S, K), np.int32)
    for t in range(R * S):
        out[t] = rng.choice(E, size=K, replace=not distinct, p=p)
    return out.reshape(R, S, K)


SHAPES = [
    # R, E, K, S, B, P
    (1, 4, 2, 8, 4, 4),
    (2, 8, 2, 64, 4, 8),
    (2, 4, 3, 5, 2, 1),
    (3, 12, 2, 17, 4, 4),
    (3, 6, 1, 9, 2, 2),
    (4, 16, 4, 16, 4, 8),
    (4, 8, 2, 7, 2, 3),
    (5, 20, 3, 11, 4, 2),
    (8, 64, 6, 32, 8, 16),
]


def test_capacity_of_the_five_workloads():
    # Capacity reading: S*K + (E/R + B)*(P - 1), rounded up to P.
    assert oracle.nvs(2, 8, 2, 64, 4, 8) == 184
    assert oracle.nvs(8, 64, 6, 2048, 8, 16) == 12528
    assert oracle.nvs(8, 256, 8, 4096, 32, 128) == 40960
    assert oracle.nvs(16, 384, 8, 8192, 24, 128) == 71680


@pytest.mark.parametrize("shape", SHAPES)
def test_histogram_is_bincount(shape):
    R, E, K, S, B, P = shape
    rng = np.random.default_rng(11)
    topk = rand_topk(rng, R, S, K, E, distinct=K <= E, skew=1.0)
    pl = oracle.plan(topk, E, B, P)
    assert pl.status == oracle.OK
    for r in range(R):
        assert (pl.debug["cnt"][r] == np.bincount(topk[r].reshape(-1), minlength=E)).all()
    assert (pl.debug["T"] == np.bincount(topk.reshape(-1), minlength=E)).all()


@pytest.mark.parametrize("S,K,E,P", [(8, 2, 4, 4), (13, 3, 7, 5), (40, 1, 6, 8), (16, 4, 4, 1)])
def test_single_rank_is_a_stable_counting_sort(S, K, E, P):
    """R = 1: nothing to balance; the layout is a stable sort of the routes by
    expert with each non-empty expert block padded to P, and every route after
    the first of a token is a local duplicate."""
    rng = np.random.default_rng(S * 100 + K)
    topk = rng.integers(0, E, size=(1, S, K)).astype(np.int32)
    pl = oracle.plan(topk, E, E, P)
    assert pl.status == oracle.OK
    flat = topk.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    padded = np.where(counts > 0, -(-counts // P) * P, 0)
    starts = np.concatenate([[0], np.cumsum(padded)[:-1]])
    exp_row = np.empty_like(flat, dtype=np.int64)
    pos = 0
    for e in range(E):
        ids = order[pos:pos + counts[e]]
        exp_row[ids] = starts[e] + np.arange(counts[e])
        pos += counts[e]
    G = pc.decode(pl.dst[0])
    assert (G == exp_row).all()
    k_idx = np.arange(S * K) % K
    assert ((pl.dst[0] < 0) == (k_idx > 0)).all()
    assert (pl.cu_seqlens[0, :E] == np.cumsum(padded)).all()
    assert (pl.cu_seqlens[0, E:] == pl.cu_seqlens[0, E - 1]).all()
    assert (pl.experts_to_copy == -1).all()
    # one duplicate group per token with K > 1, in token order
    if K > 1:
        assert pl.dup_counts[0].tolist() == [S, S * (K - 1)]
        for s in range(S):
            assert pl.dup_groups[0, s].tolist() == [exp_row[s * K], s * (K - 1), K - 1]
            assert pl.dup_loffs[0, s * (K - 1):(s + 1) * (K - 1)].tolist() == \
                exp_row[s * K + 1:(s + 1) * K].tolist()
    else:
        assert pl.dup_counts[0].tolist() == [0, 0]


def _alias_invariants(R, C, L, keep, donor, take):
    L = np.asarray(L)
    assert ((keep + take) == C).all(), "rank does not end with C"
    for u in range(R):
        if take[u] > 0:
            assert 0 <= donor[u] < R and donor[u] != u
        else:
            assert donor[u] == -1
        assert 0 <= keep[u] <= L[u]
        if L[u] <= C:
            assert keep[u] == L[u], "an under-loaded rank gave routes away"
    for o in range(R):
        given = take[donor == o].sum()
        assert keep[o] + given == L[o], "donor's routes not conserved"


@pytest.mark.parametrize("R", [1, 2, 3, 4])
def test_alias_exhaustive_small(R):
    """Every integer load vector with sum R*C for C <= 5: perfect balance, at
    most one donor per receiver, under-loaded ranks keep everything, and the
    first receiver is the lowest under-loaded rank served by the lowest
    over-loaded rank."""
    for C in range(0, 6):
        for L in itertools.product(range(R * C + 1), repeat=R):
            if sum(L) != R * C:
                continue
            st, keep, donor, take = oracle.alias(C, L)
            assert st == 0
            _alias_invariants(R, C, L, keep, donor, take)
            small = [h for h in range(R) if L[h] < C]
            large = [h for h in range(R) if L[h] > C]
            if small:
                assert donor[small[0]] == large[0]
                assert take[small[0]] == C - L[small[0]]


def test_alias_rejects_bad_totals():
    assert oracle.alias(4, [3, 4])[0] == oracle.INVALID
    assert oracle.alias(4, [9, -1])[0] == oracle.INVALID


# Hand-worked balance examples: the first shows why the fill is an alias
# construction (a plain spill would exceed E/R slots), the second fixes the
# order in which a donor's receivers cut its stream (the order served).
GOLDEN_FILES = ["alias_worked_example.json", "alias_served_order.json"]


def _worked(name="alias_worked_example.json"):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("name", GOLDEN_FILES)
def test_alias_worked_example(name):
    g = _worked(name)
    assert sum(g["L"]) == g["R"] * g["C"]
    st, keep, donor, take = oracle.alias(g["C"], g["L"])
    assert st == 0
    assert keep.tolist() == g["keep"]
    assert donor.tolist() == g["donor"]
    assert take.tolist() == g["take"]


@pytest.mark.parametrize("name", GOLDEN_FILES)
def test_plan_worked_example(name):
    g = _worked(name)
    R, E, B = g["R"], g["E"], g["B"]
    K = 2
    S = g["C"] // K
    P = 8 if name == GOLDEN_FILES[0] else 2
    assert K * S == g["C"]
    routes = np.repeat(np.arange(E), g["T"]).astype(np.int32)
    routes = routes[np.random.default_rng(5).permutation(routes.shape[0])]
    topk = routes.reshape(R, S, K)
    pl = oracle.plan(topk, E, B, P)
    assert pl.status == oracle.OK
    assert pl.experts_to_copy.tolist() == g["experts_to_copy"]
    start, n, end = pc.group_table(pc.PlanView.of(pl))
    assert n.tolist() == g["n"]
    pad = np.where(np.asarray(g["n"]) > 0, -(-np.asarray(g["n"]) // P) * P, 0)
    assert (end == np.cumsum(pad, axis=1)).all()
    pc.check_all(pc.PlanView.of(pl), topk)


def _plan_cases():
    rng = np.random.default_rng(2024)
    cases = []
    for (R, E, K, S, B, P) in SHAPES:
        for skew in (0.0, 1.0, 3.0):
            distinct = K <= E
            cases.append((R, E, K, S, B, P, skew, distinct, int(rng.integers(1 << 30))))
    # repeated experts inside a token (padded-token pattern: all K on expert 0)
    cases.append((4, 8, 4, 16, 2, 4, 0.0, False, 7))
    cases.append((2, 8, 3, 12, 4, 2, 5.0, False, 8))
    return cases


@pytest.mark.parametrize("case", _plan_cases())
def test_plan_invariants_random(case):
    R, E, K, S, B, P, skew, distinct, seed = case
    rng = np.random.default_rng(seed)
    topk = rand_topk(rng, R, S, K, E, distinct=distinct, skew=skew)
    pl = oracle.plan(topk, E, B, P)
    if pl.status == oracle.SLOT_BUDGET:
        assert B < E // R
        return
    assert pl.status == oracle.OK
    pv = pc.PlanView.of(pl)
    pc.check_all(pv, topk)
    pc.check_dups_canonical(pv)


def test_all_routes_to_one_expert_per_token():
    # The padded-token convention of a serving integration: every route of a
    # padded token goes to expert 0 (repeated id inside one token).
    R, E, K, S, B, P = 4, 16, 4, 32, 4, 8
    topk = np.zeros((R, S, K), np.int32)
    topk[:, ::2, :] = np.arange(K)  # even tokens: experts 0..K-1
    pl = oracle.plan(topk, E, B, P)
    assert pl.status == oracle.OK
    pc.check_all(pc.PlanView.of(pl), topk)


def test_balanced_loads_need_no_slots():
    R, E, K, S, B, P = 4, 8, 2, 16, 2, 4
    Eg = E // R
    # each token routes to two experts of rank (token % R): home loads are all S*K
    topk = np.empty((R, S, K), np.int32)
    for r in range(R):
        for s in range(S):
            h = (r + s) % R
            topk[r, s] = [h * Eg, h * Eg + 1]
    assert (np.bincount(topk.reshape(-1) // Eg, minlength=R) == S * K).all()
    pl = oracle.plan(topk, E, B, P)
    assert pl.status == oracle.OK
    assert (pl.experts_to_copy == -1).all()
    assert (pl.remote_stats == 0).all()
    pc.check_all(pc.PlanView.of(pl), topk)


def test_top1_has_no_duplicates():
    rng = np.random.default_rng(3)
    topk = rand_topk(rng, 4, 64, 1, 16, skew=2.0)
    pl = oracle.plan(topk, 16, 4, 4)
    assert pl.status == oracle.OK
    assert (pl.dup_counts == 0).all() and (pl.dst >= 0).all()


def test_bad_expert_id():
    topk = np.zeros((2, 4, 2), np.int32)
    topk[1, 2, 1] = 8
    assert oracle.plan(topk, 8, 4, 4).status == oracle.BAD_EXPERT
    topk[1, 2, 1] = -1
    assert oracle.plan(topk, 8, 4, 4).status == oracle.BAD_EXPERT


def test_histogram_mismatch():
    rng = np.random.default_rng(4)
    topk = rand_topk(rng, 2, 8, 2, 8)
    tpe = np.stack([np.bincount(topk[r].reshape(-1), minlength=8) for r in range(2)])
    assert oracle.plan(topk, 8, 4, 4, tokens_per_expert=tpe).status == oracle.OK
    tpe[1, 3] += 1
    assert oracle.plan(topk, 8, 4, 4, tokens_per_expert=tpe).status == oracle.HISTOGRAM


def test_slot_budget_exceeded():
    # All routes go to rank 0's experts; rank 0 keeps e0 (16 routes = C) and
    # spills e1, e2, e3 to rank 1: three pieces, more than B = 2.
    R, E, K, S, P = 2, 8, 2, 8, 2
    topk = np.array([0] * 16 + [1] * 6 + [2] * 5 + [3] * 5, np.int32).reshape(R, S, K)
    pl = oracle.plan(topk, E, 4, P)
    assert pl.status == oracle.OK
    assert pl.experts_to_copy[1].tolist() == [1, 2, 3, -1]
    assert oracle.plan(topk, E, 2, P).status == oracle.SLOT_BUDGET
