"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle,
compare.  Imports the library lazily so CPU-only collection never needs it."""
import numpy as np

import oracle
import plan_checks as pc
import synth

PLAIN_FIELDS = ("dst", "experts_to_copy", "zero_fill_ranges", "remote_stats", "dup_counts",
                "cu_seqlens")


def bits_to_f32(bits):
    return synth.bf16_to_float(bits)


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_to_dev(bits, dev):
    import torch
    return to_dev(np.ascontiguousarray(bits).view(np.int16), dev).view(torch.bfloat16)


def dev_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_plan_arrays(plan):
    import combine_balanced_planning_amd as moon
    return {k: v.cpu().numpy() for k, v in moon.plan_tensors(plan).items()}


def compare_plan(got, ref):
    """Bit-exact plan comparison; duplicate arrays on their valid prefixes."""
    for f in PLAIN_FIELDS:
        g, e = got[f], getattr(ref, f)
        if not np.array_equal(g, e):
            bad = np.argwhere(g != e)[:5]
            raise AssertionError(f"plan field {f} differs at {bad.tolist()}: "
                                 f"{g[tuple(bad[0])]} vs {e[tuple(bad[0])]}")
    if "prefetch_index" in got:  # the planner's split of experts_to_copy
        assert np.array_equal(got["prefetch_index"], oracle.prefetch_index(ref)), \
            "plan prefetch_index differs from the oracle's prefetch index"
    for r in range(ref.R):
        ng, nd = ref.dup_counts[r]
        assert np.array_equal(got["dup_groups"][r, :ng], ref.dup_groups[r, :ng]), \
            f"dup_groups of rank {r} differ"
        assert np.array_equal(got["dup_loffs"][r, :nd], ref.dup_loffs[r, :nd]), \
            f"dup_loffs of rank {r} differ"


def gpu_plan_view(got, ref):
    return pc.PlanView(ref.R, ref.E, ref.K, ref.S, ref.B, ref.P, ref.NvS, got["dst"],
                       got["experts_to_copy"], got["zero_fill_ranges"], got["remote_stats"],
                       got["dup_groups"], got["dup_loffs"], got["dup_counts"], got["cu_seqlens"])


def combine_bound(acc, absum, K):
    """Per-element bound on |gpu - exact| for an fp32 ascending-k sum of K
    products rounded once to bf16: 2^-8 |S| (bf16 rounding, with the fp32
    error folded in) + gamma_K * sum|c_k y_k| with gamma_K < 1.01 * K * 2^-24."""
    g = 1.01 * K * 2.0 ** -24
    return 2.0 ** -8 * (np.abs(acc) + g * absum) + g * absum + 1e-30


def check_combine(out_bits, ref_out_bits, ref_acc, absum, K):
    """Combine against the oracle: bit for bit with its fp32 result (the pages
    accumulate combine in fp32: ascending k, separate multiply and add, one
    rounding to bf16), within the combine tolerance |d| <= 1e-2 max|ref| +
    1e-3, and within the derived bound of the exact (float64) sum."""
    o = bits_to_f32(out_bits).astype(np.float64)
    e = bits_to_f32(ref_out_bits).astype(np.float64)
    tol = 1e-2 * np.abs(e).max() + 1e-3
    d = np.abs(o - e)
    assert d.max() <= tol, f"combine |d| {d.max()} > tolerance {tol}"
    lim = combine_bound(ref_acc, absum, K)
    over = np.abs(o - ref_acc) > lim
    assert not over.any(), f"{int(over.sum())} combine outputs beyond the derived fp32 bound"
    differ = np.asarray(out_bits) != np.asarray(ref_out_bits)
    assert not differ.any(), f"{int(differ.sum())} combine outputs differ in bits from the oracle"
    return float(d.max()), int(differ.sum())


def abs_sum(dst_tok, rows, yrows, wrows, weighted):
    """sum_k |c_k y_k| per token and column (fp64), for the derived bound."""
    G = pc.decode(dst_tok)
    idx = np.searchsorted(rows, G)
    out = np.zeros((dst_tok.shape[0], yrows.shape[1]))
    for k in range(dst_tok.shape[1]):
        yk = np.abs(bits_to_f32(yrows[idx[:, k]]).astype(np.float64))
        if weighted:
            yk *= np.abs(wrows[idx[:, k]].astype(np.float64))[:, None]
        out += yk
    return out
