"""MI355X-native balanced expert-parallel planning, dispatch and combine.

A thin ctypes binding of ``libmoon.so`` (C ABI in ``include/moon.h``).  The
functions carry the C names and only marshal arguments: tensors become device
pointers (after dtype / device / contiguity / size checks), the stream
defaults to torch's current stream.  Every step of the path runs in the HIP
kernels of the library; there is no fallback.  torch is imported first so
the library binds to the HIP runtime torch has already loaded.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoon.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
_lib = ctypes.CDLL(LIB_PATH)

MOON_OK = 0
MOON_ERR_INVALID_ARG = -1
MOON_ERR_TOPOLOGY = -2
MOON_ERR_UNSUPPORTED = -3
MOON_ERR_OOM = -4
MOON_ERR_HIP = -5
MOON_ERR_PLAN_MISMATCH = -6
MOON_ERR_BAD_EXPERT = -7
MOON_ERR_SLOT_BUDGET = -8
MOON_ERR_HISTOGRAM = -9
MOON_ERR_NOT_PLANNED = -10
MOON_ERR_INTERNAL = -11

MOON_COMBINE_WEIGHTED = 0x1
MOON_DISPATCH_FUSED_DUPS = 0x2  # the default dispatch, named explicitly
MOON_COMBINE_DUP_PROLOGUE = 0x4
MOON_DISPATCH_DEDUP_EPILOGUE = 0x8

_i32, _u32, _vp = ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p


class moon_config(ctypes.Structure):
    _fields_ = [("R", _i32), ("E", _i32), ("K", _i32), ("S", _i32), ("H", _i32), ("B", _i32),
                ("token_padding", _i32), ("flags", _u32)]


class moon_layout(ctypes.Structure):
    _fields_ = [("N", _i32), ("NvS", _i32), ("NvS_padded", _i32), ("E_plus_B", _i32),
                ("B", _i32), ("hidden_windows", _vp), ("weight_windows", _vp)]


class moon_plan_arrays(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("dst", "experts_to_copy", "zero_fill_ranges", "remote_stats",
                                   "dup_groups", "dup_loffs", "dup_counts", "cu_seqlens",
                                   "status")] + \
               [(n, _i32) for n in ("N", "R", "E", "B", "NvS", "K")] + \
               [("prefetch_index", _vp)]


class moon_weight_tensor(ctypes.Structure):
    _fields_ = [("experts", _vp), ("slots", _vp), ("row_bytes", ctypes.c_int64)]


class moon_grad_tensor(ctypes.Structure):
    _fields_ = [("expert_grads", _vp), ("slot_grads", _vp), ("row_elems", ctypes.c_int64)]


_P = ctypes.POINTER
_lib.moon_ctx_create.argtypes = [_P(moon_config), _P(_vp)]
_lib.moon_ctx_layout.argtypes = [_vp, _P(moon_layout)]
_lib.moon_ctx_destroy.argtypes = [_P(_vp)]
_lib.moon_ctx_destroy.restype = None
_lib.moon_plan_create.argtypes = [_vp, _P(_vp)]
_lib.moon_plan_clone.argtypes = [_vp, _P(_vp), _vp]
_lib.moon_plan_destroy.argtypes = [_P(_vp)]
_lib.moon_plan_destroy.restype = None
_lib.moon_plan_view.argtypes = [_vp, _P(moon_plan_arrays)]
_lib.moon_plan_status.argtypes = [_vp, _vp]
_lib.moon_plan.argtypes = [_vp, _vp, _vp, _vp, _vp]
_lib.moon_dispatch.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _u32, _vp]
_lib.moon_combine.argtypes = [_vp, _vp, _vp, _vp, _u32, _vp, _vp, _vp]
_lib.moon_prefetch_index.argtypes = [_vp, _vp, _vp, _vp]
_lib.moon_prefetch_weight.argtypes = [_vp, _vp, _P(moon_weight_tensor), _i32, _vp]
_lib.moon_reduce_grad.argtypes = [_vp, _vp, _P(moon_grad_tensor), _i32, _vp]
_lib.moon_status_str.argtypes = [_i32]
_lib.moon_status_str.restype = ctypes.c_char_p
_lib.moon_debug_tile_counts.argtypes = [_vp, _vp, _P(_i32), _P(_i32), _vp]
_lib.moon_plan_noalloc.argtypes = [_P(moon_config), _vp, _vp, _P(moon_plan_arrays), _vp]
for _f in ("moon_ctx_create", "moon_ctx_layout", "moon_plan_create", "moon_plan_clone",
           "moon_plan_view", "moon_plan_status", "moon_plan", "moon_dispatch", "moon_combine",
           "moon_prefetch_index", "moon_prefetch_weight", "moon_reduce_grad",
           "moon_debug_tile_counts", "moon_plan_noalloc"):
    getattr(_lib, _f).restype = _i32


class MoonError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {moon_status_str(status)} ({status})")
        self.status = status


def moon_status_str(status):
    return _lib.moon_status_str(int(status)).decode()


def _check(status, what):
    if status != MOON_OK:
        raise MoonError(status, what)


class Ctx:
    """Handle of a moon_ctx (windows + planner scratch on one device)."""

    def __init__(self, ptr, cfg, layout, device):
        self.ptr, self.cfg, self.layout, self.device = ptr, cfg, layout, device

    @property
    def NvS(self):
        return self.layout.NvS

    @property
    def B(self):
        return self.layout.B


class Plan:
    """Handle of a moon_comm_plan bound to its context."""

    def __init__(self, ptr, ctx):
        self.ptr, self.ctx = ptr, ctx


def _stream(stream, device=None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return _vp(s.cuda_stream)


def _ptr(t, dtype, numel, name, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return _vp(t.data_ptr())


def moon_ctx_create(R, E, K, S, H, B=0, token_padding=1, flags=0):
    cfg = moon_config(R, E, K, S, H, B, token_padding, flags)
    out = _vp()
    _check(_lib.moon_ctx_create(ctypes.byref(cfg), ctypes.byref(out)), "moon_ctx_create")
    lay = moon_layout()
    _check(_lib.moon_ctx_layout(out, ctypes.byref(lay)), "moon_ctx_layout")
    return Ctx(out, cfg, lay, torch.cuda.current_device())


def moon_ctx_layout(ctx):
    lay = moon_layout()
    _check(_lib.moon_ctx_layout(ctx.ptr, ctypes.byref(lay)), "moon_ctx_layout")
    return lay


def moon_ctx_destroy(ctx):
    p = _vp(ctx.ptr.value if ctx.ptr is not None else None)
    _lib.moon_ctx_destroy(ctypes.byref(p))
    ctx.ptr = _vp()


def moon_plan_create(ctx):
    out = _vp()
    _check(_lib.moon_plan_create(ctx.ptr, ctypes.byref(out)), "moon_plan_create")
    return Plan(out, ctx)


def moon_plan_clone(plan, stream=None):
    out = _vp()
    _check(_lib.moon_plan_clone(plan.ptr, ctypes.byref(out), _stream(stream)), "moon_plan_clone")
    return Plan(out, plan.ctx)


def moon_plan_destroy(plan):
    p = _vp(plan.ptr.value if plan.ptr is not None else None)
    _lib.moon_plan_destroy(ctypes.byref(p))
    plan.ptr = _vp()


def moon_plan_view(plan):
    v = moon_plan_arrays()
    _check(_lib.moon_plan_view(plan.ptr, ctypes.byref(v)), "moon_plan_view")
    return v


def moon_plan_status(plan, stream=None):
    """Synchronises the stream; returns the plan's status code (0 = valid)."""
    return int(_lib.moon_plan_status(plan.ptr, _stream(stream)))


def moon_plan(ctx, topk, tokens_per_expert, plan, stream=None):
    c = ctx.cfg
    _check(_lib.moon_plan(ctx.ptr, _ptr(topk, torch.int32, c.R * c.S * c.K, "topk"),
                          _ptr(tokens_per_expert, torch.int32, c.R * c.E, "tokens_per_expert",
                               optional=True), plan.ptr, _stream(stream)), "moon_plan")


def moon_dispatch(ctx, plan, hidden, weights=None, hidden_out=None, weights_out=None, flags=0,
                  stream=None):
    c, rows = ctx.cfg, ctx.cfg.R * ctx.NvS
    _check(_lib.moon_dispatch(
        ctx.ptr, plan.ptr, _ptr(hidden, torch.bfloat16, c.R * c.S * c.H, "hidden"),
        _ptr(weights, torch.float32, c.R * c.S * c.K, "weights", optional=True),
        _ptr(hidden_out, torch.bfloat16, rows * c.H, "hidden_out", optional=True),
        _ptr(weights_out, torch.float32, rows, "weights_out", optional=True), flags,
        _stream(stream)), "moon_dispatch")


def moon_combine(ctx, plan, y, w_nvs, flags, out, w_rsk_out=None, stream=None):
    c, rows = ctx.cfg, ctx.cfg.R * ctx.NvS
    _check(_lib.moon_combine(
        ctx.ptr, plan.ptr, _ptr(y, torch.bfloat16, rows * c.H, "y"),
        _ptr(w_nvs, torch.float32, rows, "w_nvs", optional=True), flags,
        _ptr(out, torch.bfloat16, c.R * c.S * c.H, "out"),
        _ptr(w_rsk_out, torch.float32, c.R * c.S * c.K, "w_rsk_out", optional=True),
        _stream(stream)), "moon_combine")


def moon_prefetch_index(ctx, plan, out, stream=None):
    c = ctx.cfg
    _check(_lib.moon_prefetch_index(ctx.ptr, plan.ptr,
                                    _ptr(out, torch.int32, c.R * ctx.B * 2, "out"),
                                    _stream(stream)), "moon_prefetch_index")


def moon_debug_tile_counts(ctx, out=None, stream=None):
    """Test hook: the planner's per-tile histogram of the latest moon_plan call
    (see include/moon.h).  Returns (tile_tokens, tiles_per_rank); when `out`
    (int32 [E+1, R*tiles_per_rank] on the GPU) is given, fills it."""
    c = ctx.cfg
    tt, tpr = _i32(0), _i32(0)
    _check(_lib.moon_debug_tile_counts(ctx.ptr, None, ctypes.byref(tt), ctypes.byref(tpr), None),
           "moon_debug_tile_counts")
    if out is not None:
        n = (c.E + 1) * c.R * tpr.value
        _check(_lib.moon_debug_tile_counts(ctx.ptr, _ptr(out, torch.int32, n, "out"), None, None,
                                           _stream(stream)), "moon_debug_tile_counts")
    return tt.value, tpr.value


def _expert_pair(ctx, rows, slots, name, dtype=None):
    """Check an ([E, ...], [R, B, ...]) tensor pair; returns (ptrs, row elements)."""
    c = ctx.cfg
    for t, what in ((rows, f"{name} rows"), (slots, f"{name} slots")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{what} must be a contiguous CUDA tensor")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if rows.dtype != slots.dtype:
        raise ValueError(f"{name}: rows and slots differ in dtype")
    if rows.shape[0] != c.E or tuple(slots.shape[:2]) != (c.R, ctx.B) or \
            tuple(slots.shape[2:]) != tuple(rows.shape[1:]):
        raise ValueError(f"{name}: expected rows [E={c.E}, ...] and slots [R={c.R}, B={ctx.B}, "
                         f"...] of one row shape, got {tuple(rows.shape)} and "
                         f"{tuple(slots.shape)}")
    return _vp(rows.data_ptr()), _vp(slots.data_ptr()), rows[0].numel()


def moon_prefetch_weight(ctx, plan, experts, slots, stream=None):
    """experts: list of [E, ...] tensors (rows [0, E) of each weight tensor);
    slots: list of [R, B, ...] tensors of the same dtypes, written in place."""
    if len(experts) != len(slots):
        raise ValueError("experts and slots must pair up")
    arr = (moon_weight_tensor * max(len(experts), 1))()
    for i, (x, sl) in enumerate(zip(experts, slots)):
        px, ps, n = _expert_pair(ctx, x, sl, f"tensor {i}")
        arr[i] = moon_weight_tensor(px, ps, n * x.element_size())
    _check(_lib.moon_prefetch_weight(ctx.ptr, plan.ptr, arr, len(experts), _stream(stream)),
           "moon_prefetch_weight")


def moon_reduce_grad(ctx, plan, grads, slot_grads, stream=None):
    """grads: list of [E, ...] float32 tensors (updated); slot_grads: list of
    [R, B, ...] float32 tensors (used slots cleared)."""
    if len(grads) != len(slot_grads):
        raise ValueError("grads and slot_grads must pair up")
    arr = (moon_grad_tensor * max(len(grads), 1))()
    for i, (g, sg) in enumerate(zip(grads, slot_grads)):
        pg, ps, n = _expert_pair(ctx, g, sg, f"gradient {i}", torch.float32)
        arr[i] = moon_grad_tensor(pg, ps, n)
    _check(_lib.moon_reduce_grad(ctx.ptr, plan.ptr, arr, len(grads), _stream(stream)),
           "moon_reduce_grad")


# ---------------------------------------------------------------------------
# Zero-copy tensor views of memory the library owns (they alias it: keep the
# context / plan alive while a view is in use).
class _CudaArray:
    def __init__(self, ptr, shape, typestr):
        self.__cuda_array_interface__ = {"shape": tuple(shape), "typestr": typestr,
                                         "data": (int(ptr), False), "version": 2}


def device_view(ptr, shape, dtype, device=None):
    typestr = {torch.int32: "<i4", torch.float32: "<f4", torch.int16: "<i2"}[
        torch.int16 if dtype == torch.bfloat16 else dtype]
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    t = torch.as_tensor(_CudaArray(ptr, shape, typestr), device=dev)
    return t.view(torch.bfloat16) if dtype == torch.bfloat16 else t


def plan_array_shapes(R, E, K, S, B, token_padding):
    """Shapes of the plan arrays (all int32) for moon_plan_noalloc, with the
    capacity NvS = round_up(S*K + (E/R + B)*(P - 1), P) documented at
    moon_ctx_create and B <= 0 meaning E/R.  Returns (shapes, NvS, B)."""
    B = B if B > 0 else E // R
    P = token_padding
    NvS = (S * K + (E // R + B) * (P - 1) + P - 1) // P * P
    EB = E + B
    return ({"dst": (R, S * K), "experts_to_copy": (R, B), "zero_fill_ranges": (R, EB, 2),
             "remote_stats": (R, 2), "dup_groups": (R, NvS, 3), "dup_loffs": (R, NvS),
             "dup_counts": (R, 2), "cu_seqlens": (R, EB), "status": (1,),
             "prefetch_index": (R, B, 2)}, NvS, B)


def moon_plan_noalloc(R, E, K, S, H, B, token_padding, topk, tokens_per_expert, arrays,
                      stream=None):
    """Planning without a context into caller-owned arrays (a dict of int32
    device tensors with the shapes of plan_array_shapes); allocates nothing."""
    shapes, NvS, Bx = plan_array_shapes(R, E, K, S, B, token_padding)
    cfg = moon_config(R, E, K, S, H, B, token_padding, 0)
    pa = moon_plan_arrays()
    for k, shp in shapes.items():
        n = 1
        for x in shp:
            n *= x
        setattr(pa, k, _ptr(arrays[k], torch.int32, n, k))
    pa.N, pa.R, pa.E, pa.B, pa.NvS, pa.K = S * K, R, E, Bx, NvS, K
    _check(_lib.moon_plan_noalloc(ctypes.byref(cfg), _ptr(topk, torch.int32, R * S * K, "topk"),
                                  _ptr(tokens_per_expert, torch.int32, R * E, "tokens_per_expert",
                                       optional=True), ctypes.byref(pa), _stream(stream)),
           "moon_plan_noalloc")


def plan_tensors(plan):
    """Views of the plan arrays, each with a leading R (see include/moon.h)."""
    v = moon_plan_view(plan)
    c = plan.ctx.cfg
    R, EB, NvS = c.R, c.E + v.B, v.NvS
    dev = torch.device("cuda", plan.ctx.device)
    shapes = {"dst": (R, v.N), "experts_to_copy": (R, v.B), "zero_fill_ranges": (R, EB, 2),
              "remote_stats": (R, 2), "dup_groups": (R, NvS, 3), "dup_loffs": (R, NvS),
              "dup_counts": (R, 2), "cu_seqlens": (R, EB), "status": (1,),
              "prefetch_index": (R, v.B, 2)}
    return {k: device_view(getattr(v, k), s, torch.int32, dev) for k, s in shapes.items()}


def window_tensors(ctx):
    """(hidden windows [R*NvS, H] bf16, weight windows [R*NvS] fp32) of the context."""
    lay, c = ctx.layout, ctx.cfg
    dev = torch.device("cuda", ctx.device)
    rows = c.R * lay.NvS_padded
    return (device_view(lay.hidden_windows, (rows, c.H), torch.bfloat16, dev),
            device_view(lay.weight_windows, (rows,), torch.float32, dev))
