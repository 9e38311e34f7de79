"""GPU fill of the seeded bf16 input arrays (bit-identical to synth.bf16_normal).

Input generation only; loads synth/libsynth.so built from synth/csrc/synth_fill.hip.
"""
import ctypes
import os

import numpy as np

import synth

_HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(_HERE, "libsynth.so")
SRC = os.path.join(_HERE, "csrc", "synth_fill.hip")
_lib = None
_tables = {}


def _load():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (share torch's HIP runtime)
        if not os.path.exists(SO):
            raise RuntimeError(f"{SO} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(SO)
        lib.synth_fill_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_fill_bf16.restype = ctypes.c_int
        _lib = lib
    return _lib


def _table(device):
    import torch
    key = str(device)
    if key not in _tables:
        t = torch.from_numpy(synth.normal_table().view(np.int16).copy()).to(device)
        _tables[key] = t
    return _tables[key]


def fill_bf16(t, key, start=0, stream=None):
    """Fill a contiguous CUDA tensor `t` (bf16 or int16/uint16 bits) with stream `key`."""
    import torch
    assert t.is_cuda and t.is_contiguous() and t.element_size() == 2
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    rc = _load().synth_fill_bf16(ctypes.c_void_p(t.data_ptr()), t.numel(), ctypes.c_uint64(key),
                                 start, ctypes.c_void_p(_table(t.device).data_ptr()),
                                 ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_bf16 failed: {rc}")
    return t


def hidden(seed, R, S, H, device="cuda"):
    import torch
    t = torch.empty((R, S, H), dtype=torch.bfloat16, device=device)
    return fill_bf16(t, synth.stream_key(seed, synth.TAG_HIDDEN))


def y(seed, rows, H, device="cuda"):
    import torch
    t = torch.empty((rows, H), dtype=torch.bfloat16, device=device)
    return fill_bf16(t, synth.stream_key(seed, synth.TAG_Y))
