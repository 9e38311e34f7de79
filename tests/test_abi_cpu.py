"""The C ABI without a GPU: exported symbols, the header as C, host validation."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moon.h")
LIB = os.path.join(ROOT, "combine_balanced_planning_amd", "libmoon.so")


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moon_status|void|const char\s*\*)\s*(moon_\w+)\s*\(",
                                 src, flags=re.M)))


def test_header_declares_the_path():
    names = declared_functions()
    for n in ("moon_plan", "moon_dispatch", "moon_combine", "moon_prefetch_index",
              "moon_ctx_create", "moon_ctx_destroy", "moon_plan_create", "moon_plan_clone",
              "moon_plan_destroy", "moon_plan_status", "moon_plan_view", "moon_ctx_layout",
              "moon_status_str", "moon_prefetch_weight", "moon_reduce_grad"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_ceiling_library_exports_its_legs():
    """The benchmark's reference kernels load on their own (no GPU needed to
    resolve the symbols) and refuse bad sizes before any launch."""
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_balanced_planning_amd", "libmoon_ceiling.so"))
    for f in ("read", "fill", "copy", "write_rows", "read_rows", "scatter_cached"):
        assert hasattr(lib, "moon_ceiling_" + f)
    lib.moon_ceiling_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.moon_ceiling_fill.restype = ctypes.c_int
    assert lib.moon_ceiling_fill(None, 16, None) != 0       # null pointer
    assert lib.moon_ceiling_fill(ctypes.c_void_p(16), 24, None) != 0  # not a multiple of 16


def test_header_is_plain_c(tmp_path):
    c = tmp_path / "use.c"
    c.write_text('#include "moon.h"\nint main(void){ moon_ctx* c = 0; moon_ctx_destroy(&c);'
                 ' return (int)moon_status_str(MOON_OK)[0]; }\n')
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(c)],
                   check=True)


@pytest.fixture(scope="module")
def moon():
    import combine_balanced_planning_amd as m
    return m


@pytest.mark.parametrize("cfg,status", [
    (dict(R=3, E=8, K=2, S=16, H=64, B=0, token_padding=4), -2),      # E % R
    (dict(R=2, E=8, K=2, S=16, H=60, B=0, token_padding=4), -3),      # H % 8
    (dict(R=64, E=64, K=2, S=16, H=64, B=0, token_padding=4), -3),    # R > 32
    (dict(R=2, E=1024, K=2, S=16, H=64, B=0, token_padding=4), -3),   # E > 512
    (dict(R=2, E=8, K=65, S=16, H=64, B=0, token_padding=4), -3),     # K > 64
    (dict(R=2, E=8, K=2, S=0, H=64, B=0, token_padding=4), -1),       # S < 1
    (dict(R=2, E=8, K=2, S=16, H=64, B=0, token_padding=0), -1),      # P < 1
    (dict(R=32, E=512, K=8, S=16, H=64, B=512, token_padding=4), -3),  # R*B > 8192
    (dict(R=8, E=64, K=64, S=1 << 23, H=64, B=0, token_padding=4), -3),  # too many routes
])
def test_host_validation_needs_no_gpu(moon, cfg, status):
    with pytest.raises(moon.MoonError) as ei:
        moon.moon_ctx_create(**cfg)
    assert ei.value.status == status


def test_null_handles_are_rejected(moon):
    lib = moon._lib
    out = ctypes.c_void_p()
    assert lib.moon_ctx_create(None, ctypes.byref(out)) == moon.MOON_ERR_INVALID_ARG
    assert lib.moon_plan_create(None, ctypes.byref(out)) == moon.MOON_ERR_INVALID_ARG
    assert lib.moon_plan(None, None, None, None, None) == moon.MOON_ERR_INVALID_ARG
    assert lib.moon_dispatch(None, None, None, None, None, None, 0, None) == \
        moon.MOON_ERR_INVALID_ARG
    assert lib.moon_combine(None, None, None, None, 0, None, None, None) == \
        moon.MOON_ERR_INVALID_ARG
    assert lib.moon_prefetch_index(None, None, None, None) == moon.MOON_ERR_INVALID_ARG
    assert lib.moon_prefetch_weight(None, None, None, 0, None) == moon.MOON_ERR_INVALID_ARG
    assert lib.moon_reduce_grad(None, None, None, 0, None) == moon.MOON_ERR_INVALID_ARG
    assert lib.moon_plan_status(None, None) == moon.MOON_ERR_INVALID_ARG
    # destroy is idempotent on NULL
    p = ctypes.c_void_p()
    lib.moon_ctx_destroy(ctypes.byref(p))
    lib.moon_plan_destroy(ctypes.byref(p))


def test_status_strings(moon):
    for s in range(0, -12, -1):
        assert moon.moon_status_str(s) != "unknown status"
    assert moon.moon_status_str(-99) == "unknown status"


def test_noalloc_planning_validates_on_the_host(moon):
    """moon_plan_noalloc refuses missing arguments, a bad configuration and
    an array description that does not match the configuration before it
    touches the GPU."""
    lib = moon._lib
    pa = moon.moon_plan_arrays()
    topk = ctypes.c_void_p(256)
    cfg = moon.moon_config(2, 8, 2, 64, 128, 0, 8, 0)
    assert lib.moon_plan_noalloc(None, topk, None, ctypes.byref(pa), None) == \
        moon.MOON_ERR_INVALID_ARG
    assert lib.moon_plan_noalloc(ctypes.byref(cfg), topk, None, None, None) == \
        moon.MOON_ERR_INVALID_ARG
    bad = moon.moon_config(3, 8, 2, 64, 128, 0, 8, 0)  # E % R != 0
    assert lib.moon_plan_noalloc(ctypes.byref(bad), topk, None, ctypes.byref(pa), None) == \
        moon.MOON_ERR_TOPOLOGY
    shapes, NvS, B = moon.plan_array_shapes(2, 8, 2, 64, 0, 8)
    for i, k in enumerate(shapes):
        setattr(pa, k, ctypes.c_void_p(4096 * (i + 1)))
    pa.N, pa.R, pa.E, pa.B, pa.NvS, pa.K = 64 * 2, 2, 8, B, NvS + 8, 2  # wrong capacity
    assert lib.moon_plan_noalloc(ctypes.byref(cfg), topk, None, ctypes.byref(pa), None) == \
        moon.MOON_ERR_INVALID_ARG
    pa.NvS = NvS
    pa.dup_loffs = ctypes.c_void_p(4098)  # misaligned
    assert lib.moon_plan_noalloc(ctypes.byref(cfg), topk, None, ctypes.byref(pa), None) == \
        moon.MOON_ERR_INVALID_ARG


@pytest.mark.parametrize("R,E,K,S,B,P", [(2, 8, 2, 64, 0, 8), (8, 64, 6, 2048, 8, 16),
                                         (16, 384, 8, 8192, 24, 128), (4, 16, 3, 7, 1, 5)])
def test_plan_array_shapes_capacity(moon, R, E, K, S, B, P):
    """The binding sizes no-alloc plan arrays with the capacity the oracle
    derives from the same configuration."""
    import oracle
    shapes, NvS, Bx = moon.plan_array_shapes(R, E, K, S, B, P)
    assert Bx == (B if B > 0 else E // R)
    assert NvS == oracle.nvs(R, E, K, S, Bx, P)
    assert shapes["dup_groups"] == (R, NvS, 3) and shapes["prefetch_index"] == (R, Bx, 2)
