"""CPU oracle for balanced expert-parallel planning, dispatch and combine.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.

A thin ctypes layer over ``liboracle.so`` (built from ``moon_oracle.cpp`` by
``oracle.build()``), taking and returning numpy arrays.  See the C header for
what each function follows on the pages.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "moon_oracle.cpp")

OK, INVALID, BAD_EXPERT, SLOT_BUDGET, HISTOGRAM = 0, -1, -7, -8, -9


def build(extra_flags=(), out=None):
    """Compile the oracle with g++ (plain C++17, single-threaded)."""
    out = out or _SO
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-Wall", "-Wextra", "-shared",
           "-fPIC", *extra_flags, _SRC, "-o", out]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def _load(path=None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        # A planted-mistake build may stand in for the oracle in the mutation test.
        so = os.environ.get("MOON_ORACLE_SO")
        if so is None:
            so = _SO
            # rebuild when the source is newer than the library
            if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(_SRC):
                build(out=so)
        _lib = _bind(ctypes.CDLL(so))
    return _lib


def _bind(lib):
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.orc_nvs.argtypes = [i32] * 6
    lib.orc_nvs.restype = i32
    lib.orc_alias.argtypes = [i32, i64, vp, vp, vp, vp]
    lib.orc_alias.restype = i32
    lib.orc_plan.argtypes = [i32] * 6 + [vp] * 11
    lib.orc_plan.restype = i32
    lib.orc_dispatch.argtypes = [i32] * 7 + [vp] * 6
    lib.orc_dispatch.restype = i32
    lib.orc_row_sources.argtypes = [i32] * 6 + [vp] * 4
    lib.orc_row_sources.restype = i32
    lib.orc_combine.argtypes = [i32] * 5 + [vp, vp, vp, i32, vp, vp, vp]
    lib.orc_combine.restype = i32
    lib.orc_combine_rows.argtypes = [i32, i32, i32, vp, i64, vp, vp, vp, i32, vp, vp, vp]
    lib.orc_combine_rows.restype = i32
    lib.orc_combine_prologue.argtypes = [i32] * 5 + [vp, vp, vp, i32, vp, vp, vp, vp]
    lib.orc_combine_prologue.restype = i32
    lib.orc_combine_prologue_rows.argtypes = [i32, i32, i32, i32, vp, i64, vp, vp, vp, i32, vp,
                                              vp, vp, vp]
    lib.orc_combine_prologue_rows.restype = i32
    lib.orc_prefetch_index.argtypes = [i32, i32, i32, vp, vp]
    lib.orc_prefetch_index.restype = i32
    lib.orc_prefetch_weight.argtypes = [i32, i32, i32, vp, i32, vp, vp, vp]
    lib.orc_prefetch_weight.restype = i32
    lib.orc_reduce_grad.argtypes = [i32, i32, i32, vp, i32, vp, vp, vp]
    lib.orc_reduce_grad.restype = i32
    lib.orc_bf16_from_double.argtypes = [ctypes.c_double]
    lib.orc_bf16_from_double.restype = ctypes.c_uint16
    return lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


class Plan:
    """Host copy of a plan: the seven plan tensors plus cu_seqlens, with a leading R."""

    FIELDS = ("dst", "experts_to_copy", "zero_fill_ranges", "remote_stats", "dup_groups",
              "dup_loffs", "dup_counts", "cu_seqlens")

    def __init__(self, R, E, K, S, B, P, NvS):
        self.R, self.E, self.K, self.S, self.B, self.P, self.NvS = R, E, K, S, B, P, NvS
        EB = E + B
        self.dst = np.zeros((R, S * K), np.int32)
        self.experts_to_copy = np.zeros((R, B), np.int32)
        self.zero_fill_ranges = np.zeros((R, EB, 2), np.int32)
        self.remote_stats = np.zeros((R, 2), np.int32)
        self.dup_groups = np.full((R, NvS, 3), -1, np.int32)
        self.dup_loffs = np.full((R, NvS), -1, np.int32)
        self.dup_counts = np.zeros((R, 2), np.int32)
        self.cu_seqlens = np.zeros((R, EB), np.int32)
        self.status = None
        self.debug = None


def nvs(R, E, K, S, B, P):
    return int(_load().orc_nvs(R, E, K, S, B, P))


def alias(C, L):
    """Balance step alone: returns (status, keep, donor, take)."""
    L = _c(L, np.int64)
    R = L.shape[0]
    keep = np.zeros(R, np.int64)
    donor = np.zeros(R, np.int32)
    take = np.zeros(R, np.int64)
    st = _load().orc_alias(R, int(C), _p(L), _p(keep), _p(donor), _p(take))
    return st, keep, donor, take


def plan(topk, E, B, P, tokens_per_expert=None, lib=None):
    """Plan for topk [R,S,K] int32.  Returns a Plan (status in .status)."""
    lib = lib or _load()
    topk = _c(topk, np.int32)
    R, S, K = topk.shape
    NvS = lib.orc_nvs(R, E, K, S, B, P)
    if NvS < 0:
        raise ValueError("invalid plan shape")
    pl = Plan(R, E, K, S, B, P, NvS)
    tpe = _c(tokens_per_expert, np.int32)
    dbg = np.zeros(R * E + 2 * E + 5 * R, np.int64)
    pl.status = lib.orc_plan(R, E, K, S, B, P, _p(topk), _p(tpe), _p(pl.dst),
                             _p(pl.experts_to_copy), _p(pl.zero_fill_ranges),
                             _p(pl.remote_stats), _p(pl.dup_groups), _p(pl.dup_loffs),
                             _p(pl.dup_counts), _p(pl.cu_seqlens), _p(dbg))
    o = 0
    d = {}
    for name, size in (("cnt", R * E), ("T", E), ("Pe", E), ("L", R), ("keep", R),
                       ("donor", R), ("take", R), ("seg_a", R)):
        d[name] = dbg[o:o + size].copy()
        o += size
    d["cnt"] = d["cnt"].reshape(R, E)
    pl.debug = d
    return pl


def dispatch(pl, hidden, w=None, win=None, wwin=None, lib=None):
    """hidden [R,S,H] bf16 bits (uint16), w [R,S,K] fp32 or None.
    Returns (win [R*NvS,H] uint16, wwin [R*NvS] fp32 or None).  Rows no group
    covers keep the value they had in `win` (zeros when allocated here)."""
    lib = lib or _load()
    hidden = _c(hidden, np.uint16)
    R, S, H = hidden.shape
    w = _c(w, np.float32)
    if win is None:
        win = np.zeros((R * pl.NvS, H), np.uint16)
    if w is not None and wwin is None:
        wwin = np.zeros(R * pl.NvS, np.float32)
    st = lib.orc_dispatch(R, pl.E, pl.K, S, H, pl.B, pl.NvS, _p(pl.dst), _p(pl.zero_fill_ranges),
                          _p(hidden), _p(w), _p(win), _p(wwin) if w is not None else None)
    if st != OK:
        raise RuntimeError(f"orc_dispatch status {st}")
    return win, (wwin if w is not None else None)


def row_sources(pl):
    lib = _load()
    src = np.zeros(pl.R * pl.NvS, np.int64)
    lib.orc_row_sources(pl.R, pl.E, pl.K, pl.S, pl.B, pl.NvS, _p(pl.dst),
                        _p(pl.zero_fill_ranges), _p(pl.cu_seqlens), _p(src))
    return src


def combine(pl, y, wnvs=None, weighted=True, H=None, lib=None, exact=True):
    """y [R*NvS,H] bf16 bits.  Returns (out [R,S,H] uint16, wsk [R,S,K] fp32,
    acc fp64 -- the exact float64 sum, None when `exact` is False)."""
    lib = lib or _load()
    y = _c(y, np.uint16)
    H = y.shape[1]
    wnvs = _c(wnvs, np.float32)
    R, S, K = pl.R, pl.S, pl.K
    out = np.zeros((R, S, H), np.uint16)
    wsk = np.zeros((R, S, K), np.float32) if wnvs is not None else None
    acc = np.zeros((R, S, H), np.float64) if exact else None
    st = lib.orc_combine(R, K, S, H, pl.NvS, _p(pl.dst), _p(y), _p(wnvs), int(bool(weighted)),
                         _p(out), _p(wsk), _p(acc))
    if st != OK:
        raise RuntimeError(f"orc_combine status {st}")
    return out, wsk, acc


def combine_rows(dst_tok, rows, yrows, wrows=None, weighted=True, lib=None):
    """Combine for sampled tokens: dst_tok [n,K]; rows [M] sorted global rows;
    yrows [M,H] bf16 bits; wrows [M] fp32."""
    lib = lib or _load()
    dst_tok = _c(dst_tok, np.int32)
    rows = _c(rows, np.int64)
    yrows = _c(yrows, np.uint16)
    wrows = _c(wrows, np.float32)
    n, K = dst_tok.shape
    H = yrows.shape[1]
    out = np.zeros((n, H), np.uint16)
    wsk = np.zeros((n, K), np.float32) if wrows is not None else None
    acc = np.zeros((n, H), np.float64)
    st = lib.orc_combine_rows(n, K, H, _p(dst_tok), rows.shape[0], _p(rows), _p(yrows),
                              _p(wrows), int(bool(weighted)), _p(out), _p(wsk), _p(acc))
    if st != OK:
        raise RuntimeError(f"orc_combine_rows status {st}")
    return out, wsk, acc


def combine_prologue(pl, y, wnvs=None, weighted=True, lib=None):
    """Combine with the duplicate prologue.  Returns (out [R,S,H] uint16,
    wsk [R,S,K] fp32 or None, acc fp64, folded [R*NvS,H] uint16 = y with
    every folded primary row replaced)."""
    lib = lib or _load()
    y = _c(y, np.uint16)
    H = y.shape[1]
    wnvs = _c(wnvs, np.float32)
    R, S, K = pl.R, pl.S, pl.K
    out = np.zeros((R, S, H), np.uint16)
    wsk = np.zeros((R, S, K), np.float32) if wnvs is not None else None
    acc = np.zeros((R, S, H), np.float64)
    folded = np.zeros_like(y)
    st = lib.orc_combine_prologue(R, K, S, H, pl.NvS, _p(pl.dst), _p(y), _p(wnvs),
                                  int(bool(weighted)), _p(out), _p(wsk), _p(acc), _p(folded))
    if st != OK:
        raise RuntimeError(f"orc_combine_prologue status {st}")
    return out, wsk, acc, folded


def combine_prologue_rows(dst_tok, rows, yrows, NvS, wrows=None, weighted=True, lib=None):
    """combine_prologue for sampled tokens (as combine_rows); returns
    (out, wsk, acc, folded_rows [M,H])."""
    lib = lib or _load()
    dst_tok = _c(dst_tok, np.int32)
    rows = _c(rows, np.int64)
    yrows = _c(yrows, np.uint16)
    wrows = _c(wrows, np.float32)
    n, K = dst_tok.shape
    H = yrows.shape[1]
    out = np.zeros((n, H), np.uint16)
    wsk = np.zeros((n, K), np.float32) if wrows is not None else None
    acc = np.zeros((n, H), np.float64)
    folded = np.zeros_like(yrows)
    st = lib.orc_combine_prologue_rows(n, K, H, NvS, _p(dst_tok), rows.shape[0], _p(rows),
                                       _p(yrows), _p(wrows), int(bool(weighted)), _p(out),
                                       _p(wsk), _p(acc), _p(folded))
    if st != OK:
        raise RuntimeError(f"orc_combine_prologue_rows status {st}")
    return out, wsk, acc, folded


def _ptr_array(arrs):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def prefetch_weight(etc, E, experts, slots):
    """Weight prefetch.  etc [R,B] int32; experts: list of [E, ...] arrays;
    slots: list of [R, B, ...] arrays of the same dtypes, updated in place
    (and returned)."""
    etc = _c(etc, np.int32)
    R, B = etc.shape
    experts = [np.ascontiguousarray(x) for x in experts]
    for x, sl in zip(experts, slots):
        assert sl.flags.c_contiguous and sl.dtype == x.dtype and sl.shape[:2] == (R, B)
        assert x.shape[0] == E and sl.shape[2:] == x.shape[1:]
    rb = np.array([x[0].nbytes if E else 0 for x in experts], np.int64)
    st = _load().orc_prefetch_weight(R, E, B, _p(etc), len(experts), _ptr_array(experts),
                                     _ptr_array(slots), _p(rb))
    if st != OK:
        raise RuntimeError(f"orc_prefetch_weight status {st}")
    return slots


def reduce_grad(etc, E, grads, slot_grads):
    """Gradient reduction.  etc [R,B] int32; grads: list of [E, ...] float32
    arrays; slot_grads: list of [R, B, ...] float32 arrays; both updated in
    place (and returned)."""
    etc = _c(etc, np.int32)
    R, B = etc.shape
    for g, sg in zip(grads, slot_grads):
        assert g.flags.c_contiguous and sg.flags.c_contiguous
        assert g.dtype == np.float32 and sg.dtype == np.float32
        assert g.shape[0] == E and sg.shape[:2] == (R, B) and sg.shape[2:] == g.shape[1:]
    le = np.array([g[0].size if E else 0 for g in grads], np.int64)
    st = _load().orc_reduce_grad(R, E, B, _p(etc), len(grads), _ptr_array(grads),
                                 _ptr_array(slot_grads), _p(le))
    if st != OK:
        raise RuntimeError(f"orc_reduce_grad status {st}")
    return grads, slot_grads


def prefetch_index(pl):
    out = np.zeros((pl.R, pl.B, 2), np.int32)
    _load().orc_prefetch_index(pl.R, pl.E, pl.B, _p(pl.experts_to_copy), _p(out))
    return out


def bf16_from_double(v):
    return int(_load().orc_bf16_from_double(float(v)))
