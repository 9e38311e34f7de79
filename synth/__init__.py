"""Seeded synthetic inputs for balanced expert-parallel dispatch/combine.

This module holds no part of the method: it only draws routing decisions,
route weights and bf16 activations, and serves the tests, the smoke check and
the benchmark alike (both the CPU oracle and the GPU library receive what it
produces).

Randomness is counter-based so any element can be regenerated on its own:

* ``mix64`` is the SplitMix64 output function (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014); word ``i`` of a
  stream with key ``k`` is ``mix64(k + (i + 1) * GAMMA)`` modulo 2^64, i.e. the
  i-th output of a SplitMix64 generator whose state starts at ``k``.
* bf16 "N(0,1)" values take 16-bit fields of those words (four per word, low
  field first) as an index into a table of the 65536 standard-normal quantiles
  at (m + 0.5) / 65536, each rounded to bf16.  Only integer operations and a
  table lookup are involved, so the GPU fill in ``synth/csrc`` produces the
  same bits (``synth.gpu``).
* Router logits are float64 Box-Muller normals from two word streams.

The routing recipe (top-K of router logits, optional per-expert bias
-alpha * ln(rank_e) from a seeded expert permutation, softmax route weights
over the chosen K logits) stands in for the pages' benchmark, which sweeps
router imbalance measured by maxvio (MoonEP README, Performance equation).
"""
import json
import math
import os

import numpy as np

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15

TAG_HIDDEN, TAG_Y, TAG_LOGIT_A, TAG_LOGIT_B, TAG_PERM, TAG_HOME = 1, 2, 3, 4, 5, 6
TAG_NTOK, TAG_INVALID = 7, 8


def _mix64_int(z):
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def mix64(z):
    """SplitMix64 output function on a uint64 numpy array (wrapping arithmetic, in place)."""
    z = np.array(z, dtype=np.uint64, copy=True)
    _mix64_inplace(z, np.empty_like(z))
    return z


def _mix64_inplace(z, t):
    np.right_shift(z, np.uint64(30), out=t)
    np.bitwise_xor(z, t, out=z)
    np.multiply(z, np.uint64(0xBF58476D1CE4E5B9), out=z)
    np.right_shift(z, np.uint64(27), out=t)
    np.bitwise_xor(z, t, out=z)
    np.multiply(z, np.uint64(0x94D049BB133111EB), out=z)
    np.right_shift(z, np.uint64(31), out=t)
    np.bitwise_xor(z, t, out=z)


def stream_key(seed, tag):
    """Key of stream `tag` for run `seed`."""
    return _mix64_int(_mix64_int(int(seed) & M64) ^ (int(tag) & M64))


_CHUNK = 1 << 22


def words(key, start, count, out=None):
    """Words start..start+count-1 of the stream with the given key (uint64)."""
    out = np.empty(count, np.uint64) if out is None else out
    t = np.empty(min(count, _CHUNK), np.uint64)
    for c0 in range(0, count, _CHUNK):
        c1 = min(count, c0 + _CHUNK)
        z = out[c0:c1]
        z[:] = np.arange(start + c0 + 1, start + c1 + 1, dtype=np.uint64)
        np.multiply(z, np.uint64(GAMMA), out=z)
        np.add(z, np.uint64(key), out=z)
        _mix64_inplace(z, t[:c1 - c0])
    return out


def _float_to_bf16_bits(x):
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


_TABLE = None


def normal_table():
    """65536 bf16 bit patterns: the N(0,1) quantiles at (m + 0.5) / 65536."""
    global _TABLE
    if _TABLE is None:
        from scipy.special import ndtri
        m = np.arange(65536, dtype=np.float64)
        q = ndtri((m + 0.5) / 65536.0)
        _TABLE = _float_to_bf16_bits(q.astype(np.float32))
    return _TABLE


def bf16_normal(key, start, count):
    """Elements start..start+count-1 (bf16 bits) of the bf16 normal stream `key`."""
    out = np.empty(count, np.uint16)
    if count == 0:
        return out
    table = normal_table()
    w0 = start // 4
    nw = (start + count + 3) // 4 - w0
    off = start - 4 * w0
    done = 0
    for c0 in range(0, nw, _CHUNK):
        c1 = min(nw, c0 + _CHUNK)
        # Little-endian uint16 view: field j of a word is bits [16j, 16j+16).
        f = words(key, w0 + c0, c1 - c0).view(np.uint16)
        lo = off if c0 == 0 else 0
        take = min(f.shape[0] - lo, count - done)
        np.take(table, f[lo:lo + take], out=out[done:done + take])
        done += take
    return out


def bf16_rows(key, row_ids, width):
    """Rows `row_ids` of a [*, width] bf16 normal array generated from stream `key`."""
    row_ids = np.asarray(row_ids, np.int64)
    out = np.empty((row_ids.shape[0], width), np.uint16)
    for j, r in enumerate(row_ids):
        out[j] = bf16_normal(key, int(r) * width, width)
    return out


def bf16_to_float(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f64(key_a, key_b, count):
    """float64 N(0,1) by Box-Muller from two word streams."""
    out = np.empty(count, np.float64)
    for c0 in range(0, count, _CHUNK):
        c1 = min(count, c0 + _CHUNK)
        ua = (words(key_a, c0, c1 - c0) >> np.uint64(11)).astype(np.float64)
        ub = (words(key_b, c0, c1 - c0) >> np.uint64(11)).astype(np.float64)
        u1 = (ua + 0.5) * 2.0 ** -53
        u2 = (ub + 0.5) * 2.0 ** -53
        out[c0:c1] = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)
    return out


# ---------------------------------------------------------------------------
# Workloads, by a stable integer id (it enters the seeds: seed = 1000 * id +
# level) and by name; `dedup_stress` makes every odd token choose all K
# experts among one uniformly drawn home rank.
WORKLOADS = {
    1: dict(name="tiny", R=2, E=8, K=2, S=64, H=128, P=8, B=4, dedup_stress=False),
    2: dict(name="r8-e64-k6-s2048-h2048", R=8, E=64, K=6, S=2048, H=2048, P=16, B=8,
            dedup_stress=False),
    3: dict(name="dsv3-r8-e256-k8-s4096-h7168", R=8, E=256, K=8, S=4096, H=7168, P=128, B=32,
            dedup_stress=False),
    4: dict(name="r8-e64-k6-s2048-h2048-skewed", R=8, E=64, K=6, S=2048, H=2048, P=16, B=8,
            dedup_stress=False),
    5: dict(name="r16-e384-k8-s8192-h7168-dedup", R=16, E=384, K=8, S=8192, H=7168, P=128, B=24,
            dedup_stress=True),
}
# Serving workload with capacity padding (the serving integration's buffer
# pool): per rank a step holds n_r real tokens drawn uniformly from [lo, hi];
# the buffer capacity S is the smallest power of two >= max_r n_r, clamped to
# [min_capacity, max_tokens].  Real tokens route like the DSv3-shaped
# configuration; about one real route slot in `invalid_every` is an invalid
# id that the engine maps to expert 0 with weight 0; pad tokens have zero
# hidden rows, all K ids 0 and weights 0.  Combine is the plain K-sum.
SERVING = dict(name="serving-padded-r8-e256-k8-h7168", R=8, E=256, K=8, H=7168, P=128, B=32,
               max_tokens=4096, min_capacity=128, invalid_every=64, dedup_stress=False)
SERVING_LEVELS = [dict(name="decode", lo=48, hi=200), dict(name="prefill", lo=1200, hi=3000)]
# Serving seeds are 6000 + level, clear of the workloads' 1000 * id + level.
_SERVING_SEED_BASE = 6000

# Short names accepted beside the full ones.
_ALIASES = {"r8-e64-k6": 2, "dsv3": 3, "r8-e64-k6-skewed": 4, "r16-e384-k8": 5}


def workload_id(key):
    """The integer id of a workload given by id, full name or short name."""
    if isinstance(key, (int, np.integer)):
        if int(key) not in WORKLOADS:
            raise KeyError(f"no workload {key}")
        return int(key)
    if key in _ALIASES:
        return _ALIASES[key]
    for i, c in WORKLOADS.items():
        if c["name"] == key:
            return i
    raise KeyError(f"no workload named {key!r}")


# maxvio targets per workload id (level index -> target); None = no bias.
LEVELS = {1: [None], 2: [None], 3: [None], 4: [0.5, 1.0, 2.0, 4.0], 5: [None, 1.0, 2.0, 4.0, 8.0]}

_ALPHA_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "alpha_table.json")


def seed_of(config, level=0):
    return 1000 * workload_id(config) + int(level)


def maxvio(topk, E):
    """max_e(T_e / T_bar) - 1 with T_bar = routes / E (README, Performance)."""
    t = np.bincount(np.asarray(topk).reshape(-1).astype(np.int64), minlength=E)
    tbar = t.sum() / E
    return float(t.max() / tbar - 1.0)


def _topk_desc(x, K):
    """Indices of the K largest entries per row, largest first, ties -> lower index."""
    n, E = x.shape
    if K >= E:
        return np.argsort(-x, axis=1, kind="stable")[:, :K]
    part = np.argpartition(-x, K - 1, axis=1)[:, :K]
    vals = np.take_along_axis(x, part, axis=1)
    kth = vals.min(axis=1)
    # Rows where another entry equals the K-th value need the exact tie rule.
    ties = (x == kth[:, None]).sum(axis=1) > (vals == kth[:, None]).sum(axis=1)
    order = np.lexsort((part, -vals), axis=1)  # value descending, then lower index
    sel = np.take_along_axis(part, order, axis=1)
    if ties.any():
        rows = np.nonzero(ties)[0]
        sel[rows] = np.argsort(-x[rows], axis=1, kind="stable")[:, :K]
    return sel


def base_logits(c, seed):
    """Unbiased router logits [R*S, E] (float64) of one run."""
    n = c["R"] * c["S"]
    return normal_f64(stream_key(seed, TAG_LOGIT_A), stream_key(seed, TAG_LOGIT_B),
                      n * c["E"]).reshape(n, c["E"])


def route_from_logits(c, seed, logits, alpha):
    """Bias, restrict (dedup stress), pick top-K, softmax the chosen logits."""
    R, E, K, S = c["R"], c["E"], c["K"], c["S"]
    n = R * S
    if alpha:
        perm = np.argsort(words(stream_key(seed, TAG_PERM), 0, E), kind="stable")
        rank = np.empty(E, np.float64)
        rank[perm] = np.arange(1, E + 1, dtype=np.float64)
        logits = logits - alpha * np.log(rank)[None, :]
    if c.get("dedup_stress"):
        Eg = E // R
        home = (words(stream_key(seed, TAG_HOME), 0, n) % np.uint64(R)).astype(np.int64)
        odd = (np.arange(n) % S) % 2 == 1
        expert_rank = np.arange(E) // Eg
        mask = odd[:, None] & (expert_rank[None, :] != home[:, None])
        logits = np.where(mask, -np.inf, logits)
    sel = _topk_desc(logits, K)
    chosen = np.take_along_axis(logits, sel, axis=1)
    z = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return sel.astype(np.int32).reshape(R, S, K), w.reshape(R, S, K)


def routing(config, seed, alpha=0.0, cfg=None):
    """Top-K routing for one run: returns (topk [R,S,K] int32, weights [R,S,K] fp32)."""
    c = dict(WORKLOADS[workload_id(config)]) if cfg is None else dict(cfg)
    return route_from_logits(c, seed, base_logits(c, seed), alpha)


def load_alpha_table():
    if not os.path.exists(_ALPHA_FILE):
        return {}
    with open(_ALPHA_FILE) as f:
        return json.load(f)


def alpha_for(config, level):
    """Bias strength for a workload's maxvio level (0.0 when unbiased)."""
    config = workload_id(config)
    target = LEVELS[config][level]
    if target is None:
        return 0.0
    tab = load_alpha_table()
    key = f"{config}:{level}"
    if key not in tab:
        raise KeyError(f"no tuned alpha for {WORKLOADS[config]['name']} level {level}; "
                       "run python -m synth.tune")
    return float(tab[key]["alpha"])


def workload(config, level=0):
    """Routing of one workload (id or name) and maxvio level: dict with shapes,
    topk, w, maxvio."""
    config = workload_id(config)
    c = dict(WORKLOADS[config])
    seed = seed_of(config, level)
    alpha = alpha_for(config, level)
    topk, w = routing(config, seed, alpha)
    c.update(seed=seed, alpha=alpha, topk=topk, w=w, maxvio=maxvio(topk, c["E"]),
             target=LEVELS[config][level], config=config, level=level)
    return c


def hidden_bf16(seed, R, S, H):
    return bf16_normal(stream_key(seed, TAG_HIDDEN), 0, R * S * H).reshape(R, S, H)


def y_bf16(seed, rows, H):
    return bf16_normal(stream_key(seed, TAG_Y), 0, rows * H).reshape(rows, H)


def serving_capacity(n_max, min_capacity, max_tokens):
    """Padded capacity of a serving step: the least power of two that is at
    least n_max (1 for an empty step), raised to min_capacity and capped at
    max_tokens."""
    p = 1
    while p < n_max:
        p *= 2
    return min(max_tokens, max(min_capacity, p))


def serving_workload(level, n_tok=None):
    """The padded serving workload at `level` (index into SERVING_LEVELS): dict
    with the shapes (S = capacity), n_tok [R], topk [R,S,K], w [R,S,K],
    tokens_per_expert [R,E] (bincount of the padded ids) and maxvio.
    `n_tok` overrides the drawn per-rank real token counts."""
    c = dict(SERVING)
    lv = SERVING_LEVELS[level]
    seed = _SERVING_SEED_BASE + int(level)
    R, E, K = c["R"], c["E"], c["K"]
    span = np.uint64(lv["hi"] - lv["lo"] + 1)
    if n_tok is None:
        n_tok = (lv["lo"] + (words(stream_key(seed, TAG_NTOK), 0, R) % span)).astype(np.int64)
    else:
        n_tok = np.asarray(n_tok, np.int64)
        assert n_tok.shape == (R,) and (n_tok >= 0).all()
    S = serving_capacity(int(n_tok.max()), c["min_capacity"], c["max_tokens"])
    c.update(S=S)
    topk, w = routing(None, seed, 0.0, cfg=c)
    invalid = (words(stream_key(seed, TAG_INVALID), 0, R * S * K) %
               np.uint64(c["invalid_every"]) == 0).reshape(R, S, K)
    pad = np.arange(S)[None, :] >= n_tok[:, None]
    invalid |= pad[:, :, None]
    topk = np.where(invalid, 0, topk).astype(np.int32)
    w = np.where(invalid, np.float32(0.0), w).astype(np.float32)
    tpe = np.stack([np.bincount(topk[r].reshape(-1), minlength=E) for r in range(R)])
    c.update(seed=seed, level=level, level_name=lv["name"], n_tok=n_tok, topk=topk, w=w,
             tokens_per_expert=tpe.astype(np.int32), maxvio=maxvio(topk, E),
             config=SERVING["name"])
    return c


def serving_hidden_bf16(wl):
    """bf16 hidden [R,S,H] of a serving workload: N(0,1) rows, pad rows zero."""
    h = hidden_bf16(wl["seed"], wl["R"], wl["S"], wl["H"])
    for r in range(wl["R"]):
        h[r, wl["n_tok"][r]:] = 0
    return h
