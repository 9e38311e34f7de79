"""libmoon.so used from C: tests/c_abi_example.c (C11, hipMalloc'd pointers,
no Python or torch) plans, dispatches and combines a skewed routing and
checks what the method fixes exactly (S*K routes per rank, the default B and
NvS, combine over the dispatched windows = K*x plain and x with weights 1/K,
the prefetch index, a device-reported bad expert id, a refused plan of
another context).  It runs as a child process on the same GPU."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_through_the_abi():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_moon_build", os.path.join(ROOT, "combine_balanced_planning_amd", "_build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    if not os.path.exists(b.C_EXAMPLE_BIN):  # normally built by __graft_entry__.build()
        b.build_c_example()
    print("[case] c_abi_example", flush=True)
    r = subprocess.run([b.C_EXAMPLE_BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi ok" in r.stdout
