"""Independent checks of a plan and of dispatched windows (numpy only).

These checks encode what the pages guarantee, not how any planner computes a
plan, and run on plans from either the CPU oracle or the GPU library:

* every rank receives exactly S*K routes (MoonEP README, "Perfect balance");
* each route lands once, in its own physical row of a group holding its
  expert; non-empty groups are padded to token_padding and cu_seqlens holds
  padded end offsets (Visual Guide, Buffer(...) token_padding; dispatch table,
  cu_seqlens);
* unused prefetch slots are -1 and empty (Visual Guide, prefetch_weight);
* every slot expert of a rank is homed on one and the same other rank
  (README, "How to set B");
* positive dst entries are primaries, negative ones local duplicates, and the
  duplicate records list exactly the duplicates (Visual Guide, combine and
  MoonEPCommPlan).

The readings taken where the pages are silent (group order = global route
order, home-first prefix, compact slot numbering in ascending expert id, token
order of duplicate records) are checked too, each in its own function, so a
plan that is valid but follows another reading fails only those.
"""
import numpy as np


def decode(dst):
    dst = np.asarray(dst, np.int64)
    return np.where(dst >= 0, dst, -dst - 1)


class PlanView:
    """Plain numpy view of a plan with a leading rank dimension."""

    def __init__(self, R, E, K, S, B, P, NvS, dst, experts_to_copy, zero_fill_ranges,
                 remote_stats, dup_groups, dup_loffs, dup_counts, cu_seqlens):
        self.R, self.E, self.K, self.S, self.B, self.P, self.NvS = R, E, K, S, B, P, NvS
        self.dst = np.asarray(dst).reshape(R, S * K)
        self.experts_to_copy = np.asarray(experts_to_copy).reshape(R, B)
        self.zero_fill_ranges = np.asarray(zero_fill_ranges).reshape(R, E + B, 2)
        self.remote_stats = np.asarray(remote_stats).reshape(R, 2)
        self.dup_groups = np.asarray(dup_groups).reshape(R, NvS, 3)
        self.dup_loffs = np.asarray(dup_loffs).reshape(R, NvS)
        self.dup_counts = np.asarray(dup_counts).reshape(R, 2)
        self.cu_seqlens = np.asarray(cu_seqlens).reshape(R, E + B)

    @classmethod
    def of(cls, pl):
        return cls(pl.R, pl.E, pl.K, pl.S, pl.B, pl.P, pl.NvS, pl.dst, pl.experts_to_copy,
                   pl.zero_fill_ranges, pl.remote_stats, pl.dup_groups, pl.dup_loffs,
                   pl.dup_counts, pl.cu_seqlens)


def group_table(pv):
    """start, n, end per (rank, group) from cu_seqlens and zero_fill_ranges."""
    cu = pv.cu_seqlens.astype(np.int64)
    start = np.concatenate([np.zeros((pv.R, 1), np.int64), cu[:, :-1]], axis=1)
    n = pv.zero_fill_ranges[:, :, 0].astype(np.int64) - start
    return start, n, cu


def check_layout(pv):
    start, n, end = group_table(pv)
    assert (pv.zero_fill_ranges[:, :, 1] == end).all(), "zero_fill_ranges end != cu_seqlens"
    assert (n >= 0).all() and (start + n <= end).all(), "bad valid span"
    size = end - start
    assert (size >= 0).all(), "cu_seqlens not monotone"
    assert (size % pv.P == 0).all(), "group not padded to token_padding"
    assert ((size == 0) == (n == 0)).all(), "empty group padded / non-empty group empty"
    assert (size - n < pv.P).all(), "more padding than needed"
    assert (end[:, -1] <= pv.NvS).all(), "layout exceeds NvS"


def route_table(pv):
    """Per route: global row G, rank u, local row, group g (via cu search)."""
    G = decode(pv.dst).reshape(-1)
    u = G // pv.NvS
    row = G % pv.NvS
    start, n, end = group_table(pv)
    g = np.empty_like(G)
    for r in range(pv.R):
        sel = u == r
        g[sel] = np.searchsorted(end[r], row[sel], side="right")
    return G, u, row, g


def check_routes(pv, topk):
    """Bijection routes -> valid rows, group expert matches, exact balance."""
    R, E, B, K, S = pv.R, pv.E, pv.B, pv.K, pv.S
    Eg = E // R
    topk = np.asarray(topk).reshape(-1).astype(np.int64)
    G, u, row, g = route_table(pv)
    assert (G >= 0).all() and (G < R * pv.NvS).all(), "dst out of range"
    assert np.unique(G).shape[0] == G.shape[0], "two routes share a row"
    counts = np.bincount(u, minlength=R)
    assert (counts == S * K).all(), f"not perfectly balanced: {counts.tolist()}"
    assert (g < E + B).all(), "row beyond the last group"
    start, n, end = group_table(pv)
    assert (row >= start[u, g]).all() and (row < start[u, g] + n[u, g]).all(), \
        "route outside the valid span of its group"
    per_group = np.zeros((R, E + B), np.int64)
    np.add.at(per_group, (u, g), 1)
    assert (per_group == n).all(), "group sizes disagree with routes"
    home = g < E
    assert (topk[home] == g[home]).all(), "home group holds another expert"
    assert (g[home] // Eg == u[home]).all(), "home group on a foreign rank"
    slot = ~home
    e_slot = pv.experts_to_copy[u[slot], g[slot] - E]
    assert (e_slot == topk[slot]).all(), "slot group holds an expert other than experts_to_copy"
    assert (topk[slot] // Eg != u[slot]).all(), "slot holds a local expert"


def check_slots(pv):
    R, E, B = pv.R, pv.E, pv.B
    Eg = E // R
    start, n, end = group_table(pv)
    etc = pv.experts_to_copy
    for r in range(R):
        used = etc[r] >= 0
        assert (n[r, E:][~used] == 0).all(), "unused slot has routes"
        assert (etc[r][~used] == -1).all(), "unused slot not -1"
        donors = set((etc[r][used] // Eg).tolist())
        assert len(donors) <= 1, f"rank {r} takes from {len(donors)} home ranks"
        assert r not in donors, "slot duplicates a local expert"
        assert int(pv.remote_stats[r, 0]) == int(used.sum()), "remote_stats slot count"
        assert int(pv.remote_stats[r, 1]) == int(n[r, E:].sum()), "remote_stats routed count"
        assert len(set(etc[r][used].tolist())) == int(used.sum()), "expert in two slots"


def check_reading_slot_order(pv):
    """Reading: used slots are a compact prefix in ascending expert id."""
    for r in range(pv.R):
        etc = pv.experts_to_copy[r]
        used = etc >= 0
        k = int(used.sum())
        assert used[:k].all(), "slots not compact from 0"
        assert (np.diff(etc[:k]) > 0).all(), "slots not in ascending expert order"


def check_reading_group_order(pv):
    """Reading: inside each group, routes sit in global route order (r, s, k)."""
    G, u, row, g = route_table(pv)
    rid = np.arange(G.shape[0])
    key = (u * (pv.E + pv.B) + g)
    order = np.lexsort((row, key))
    ks, rs = key[order], rid[order]
    same = ks[1:] == ks[:-1]
    assert (rs[1:][same] > rs[:-1][same]).all(), "group rows not in route order"


def check_reading_home_first(pv, topk):
    """Reading: along each home rank's stream (expert ascending, then route
    order) the kept part is a prefix and each receiver gets one contiguous block."""
    R, E = pv.R, pv.E
    Eg = E // R
    topk = np.asarray(topk).reshape(-1).astype(np.int64)
    G, u, row, g = route_table(pv)
    rid = np.arange(topk.shape[0])
    for h in range(R):
        sel = (topk // Eg) == h
        order = np.lexsort((rid[sel], topk[sel]))
        dest = u[sel][order]
        if dest.shape[0] == 0:
            continue
        change = np.nonzero(dest[1:] != dest[:-1])[0] + 1
        blocks = np.split(dest, change)
        firsts = [int(b[0]) for b in blocks]
        assert len(set(firsts)) == len(firsts), "a receiver's block is not contiguous"
        kept = dest == h
        if kept.any():
            assert firsts[0] == h, "home part is not a prefix of the stream"


def check_dups(pv):
    """Sign rule on dst and duplicate records (content, then token order)."""
    R, K, S, NvS = pv.R, pv.K, pv.S, pv.NvS
    dst = pv.dst.reshape(R * S, K).astype(np.int64)
    G = decode(dst)
    u = G // NvS
    # primary iff no earlier route of the token goes to the same rank
    earlier = np.zeros_like(dst, dtype=bool)
    for k in range(1, K):
        earlier[:, k] = (u[:, :k] == u[:, k:k + 1]).any(axis=1)
    assert ((dst < 0) == earlier).all(), "dst sign disagrees with first-occurrence rule"
    for r in range(R):
        ng, nd = int(pv.dup_counts[r, 0]), int(pv.dup_counts[r, 1])
        recs = pv.dup_groups[r, :ng].astype(np.int64)
        loffs = pv.dup_loffs[r, :nd].astype(np.int64)
        # expected: per token (global order) with dups on r
        mine = (u == r)
        dup_mask = mine & (dst < 0)
        toks = np.nonzero(dup_mask.any(axis=1))[0]
        assert ng == toks.shape[0], f"rank {r}: {ng} groups, expected {toks.shape[0]}"
        assert nd == int(dup_mask.sum()), f"rank {r}: dup count"
        lb = 0
        for j, t in enumerate(toks):
            prim_k = np.nonzero(mine[t] & (dst[t] >= 0))[0]
            assert prim_k.shape[0] == 1
            exp_rows = G[t][dup_mask[t]] - r * NvS
            assert recs[j, 0] == G[t, prim_k[0]] - r * NvS, "primary row"
            assert recs[j, 1] == lb, "loff begin"
            assert recs[j, 2] == exp_rows.shape[0], "dup count in record"
            assert (loffs[lb:lb + exp_rows.shape[0]] == exp_rows).all(), "dup rows"
            lb += exp_rows.shape[0]


def check_dups_canonical(pv):
    """Order-free version of the duplicate-record check (any record order)."""
    R, K, S, NvS = pv.R, pv.K, pv.S, pv.NvS
    dst = pv.dst.reshape(R * S, K).astype(np.int64)
    G = decode(dst)
    u = G // NvS
    for r in range(R):
        ng = int(pv.dup_counts[r, 0])
        got = set()
        for rec in pv.dup_groups[r, :ng]:
            p, lb, m = (int(x) for x in rec)
            got.add((p, tuple(sorted(int(x) for x in pv.dup_loffs[r, lb:lb + m]))))
        exp = set()
        for t in range(R * S):
            mine = u[t] == r
            if (mine & (dst[t] < 0)).any():
                p = int(G[t][mine & (dst[t] >= 0)][0] - r * NvS)
                exp.add((p, tuple(sorted(int(x) for x in G[t][mine & (dst[t] < 0)] - r * NvS))))
        assert got == exp, f"rank {r}: duplicate groups differ"


def check_all(pv, topk, readings=True, dups=True):
    check_layout(pv)
    check_routes(pv, topk)
    check_slots(pv)
    if dups:
        check_dups(pv)
    if readings:
        check_reading_slot_order(pv)
        check_reading_group_order(pv)
        check_reading_home_first(pv, topk)


def check_windows(pv, hidden, w, win, wwin):
    """Dispatched content: each route's row holds its token's row, each route
    weight sits at its row, padding rows are zero (bits)."""
    R, S, K, H = pv.R, pv.S, pv.K, hidden.shape[-1]
    G = decode(pv.dst).reshape(-1)
    tok = np.arange(R * S * K) // K
    hid = np.asarray(hidden).reshape(R * S, H)
    assert (np.asarray(win)[G] == hid[tok]).all(), "window row differs from its source row"
    if w is not None:
        assert (np.asarray(wwin)[G].view(np.uint32) ==
                np.asarray(w, np.float32).reshape(-1).view(np.uint32)).all(), "route weight bits"
    for r in range(R):
        for g in range(pv.E + pv.B):
            a, b = (int(x) for x in pv.zero_fill_ranges[r, g])
            if b > a:
                assert (np.asarray(win)[r * pv.NvS + a:r * pv.NvS + b] == 0).all(), "padding not zero"
                if w is not None:
                    assert (np.asarray(wwin)[r * pv.NvS + a:r * pv.NvS + b].view(np.uint32)
                            == 0).all(), "padding weight not +0"
