"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): built with g++ into a temporary directory and exercised in a
child process that preloads the sanitizer runtimes, on shapes that reach
its edge paths (one rank, repeated ids, a slot budget exceeded, padding,
K = 1, the prologue, weight prefetch and gradient reduction).  Any report
fails the test."""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = textwrap.dedent("""
    import numpy as np
    import oracle, synth
    rng = np.random.default_rng(5)
    shapes = [(1, 8, 2, 50, 8, 0, 4), (4, 16, 4, 77, 16, 0, 1), (2, 8, 3, 64, 32, 2, 8),
              (4, 16, 1, 130, 8, 0, 8), (8, 64, 6, 300, 16, 0, 16), (3, 12, 3, 200, 24, 1, 5)]
    for R, E, K, S, H, B, P in shapes:
        Bx = B if B > 0 else E // R
        for mode in range(3):
            if mode == 0:
                topk = rng.integers(0, E, size=(R, S, K)).astype(np.int32)
            elif mode == 1:
                topk = np.zeros((R, S, K), np.int32) + (E - 1)
            else:
                topk = rng.integers(0, max(1, E // R), size=(R, S, K)).astype(np.int32)
                topk[:, ::3, :] = 0
            tpe = np.stack([np.bincount(topk[r].reshape(-1), minlength=E)
                            for r in range(R)]).astype(np.int32)
            pl = oracle.plan(topk, E, Bx, P, tpe)
            if pl.status != oracle.OK:
                continue
            w = rng.random((R, S, K)).astype(np.float32)
            hidden = synth.bf16_normal(int(rng.integers(1 << 62)), 0, R * S * H).reshape(R, S, H)
            win, wwin = oracle.dispatch(pl, hidden, w)
            y = synth.bf16_normal(int(rng.integers(1 << 62)), 0, R * pl.NvS * H).reshape(
                R * pl.NvS, H)
            oracle.combine(pl, y, wwin, weighted=True)
            oracle.combine(pl, y, None, weighted=False)
            oracle.combine_prologue(pl, y.copy(), wwin, weighted=True)
            oracle.prefetch_index(pl)
            ex = [rng.random((E, 4)).astype(np.float32)]
            oracle.prefetch_weight(pl.experts_to_copy, E, ex, [np.zeros((R, Bx, 4), np.float32)])
            oracle.reduce_grad(pl.experts_to_copy, E, [ex[0].copy()],
                               [rng.random((R, Bx, 4)).astype(np.float32)])
        bad = np.zeros((R, S, K), np.int32)
        bad[0, 0, 0] = E
        assert oracle.plan(bad, E, Bx, P).status == oracle.BAD_EXPERT
    print("sanitized oracle ok")
""")


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout
    p = p.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_is_clean_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("sanitizer runtimes not installed")
    so = str(tmp_path / "liboracle_sanitized.so")
    oracle.build(extra_flags=["-O1", "-g", "-fsanitize=address,undefined",
                              "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"],
                 out=so)
    env = dict(os.environ, MOON_ORACLE_SO=so, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", SCRIPT], capture_output=True, text=True,
                       timeout=600, env=env, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "sanitized oracle ok" in r.stdout
    for marker in ("AddressSanitizer", "runtime error", "UndefinedBehaviorSanitizer"):
        assert marker not in r.stderr, r.stderr[-3000:]
