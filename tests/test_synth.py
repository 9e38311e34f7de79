"""The seeded input generator: published SplitMix64 outputs, table, recipe."""
import numpy as np

import synth


def test_splitmix64_reference_sequence():
    # First outputs of SplitMix64 with state 0 (Steele, Lea, Flood 2014;
    # the seeding generator of the xoshiro family).
    got = [int(v) for v in synth.words(0, 0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_slices_agree():
    key = synth.stream_key(123, synth.TAG_HIDDEN)
    full = synth.bf16_normal(key, 0, 4096)
    for start, count in ((0, 1), (1, 7), (4, 4), (1001, 2000), (4095, 1)):
        assert (synth.bf16_normal(key, start, count) == full[start:start + count]).all()
    rows = synth.bf16_rows(key, [3, 0, 7], 512)
    assert (rows[0] == full[3 * 512:4 * 512]).all() and (rows[2] == full[7 * 512:8 * 512]).all()


def test_normal_table_is_standard_normal():
    t = synth.bf16_to_float(synth.normal_table()).astype(np.float64)
    assert (np.diff(t) >= 0).all()
    assert np.allclose(t, -t[::-1], atol=0)  # symmetric quantiles
    assert abs(t.mean()) < 1e-3 and abs(t.std() - 1.0) < 2e-3
    v = synth.bf16_to_float(synth.bf16_normal(synth.stream_key(1, 1), 0, 1 << 20))
    assert abs(v.mean()) < 5e-3 and abs(v.std() - 1.0) < 5e-3


def test_maxvio_closed_forms():
    E = 8
    assert synth.maxvio(np.arange(E).repeat(5), E) == 0.0
    # all routes on one expert: T_max / T_bar - 1 = E - 1
    assert synth.maxvio(np.zeros(40, np.int64), E) == E - 1
    assert abs(synth.maxvio(np.array([0, 0, 1, 2]), 4) - 1.0) < 1e-12


def test_topk_ties_choose_lower_expert_first():
    x = np.array([[1.0, 3.0, 3.0, 2.0], [0.0, 0.0, 0.0, 0.0], [5.0, 1.0, 5.0, 5.0]])
    assert synth._topk_desc(x, 2).tolist() == [[1, 2], [0, 1], [0, 2]]


def test_routing_recipe_tiny():
    topk, w = synth.routing("tiny", synth.seed_of("tiny"))
    assert topk.shape == (2, 64, 2) and w.shape == (2, 64, 2)
    assert ((topk >= 0) & (topk < 8)).all()
    assert (topk[..., 0] != topk[..., 1]).all()
    assert np.allclose(w.sum(-1), 1.0, atol=1e-6) and (w[..., 0] >= w[..., 1]).all()
    t2, w2 = synth.routing("tiny", synth.seed_of("tiny"))
    assert (t2 == topk).all() and (w2 == w).all()


def test_skewed_levels_hit_their_targets():
    skewed = synth.workload_id("r8-e64-k6-skewed")
    for level, target in enumerate(synth.LEVELS[skewed]):
        wl = synth.workload("r8-e64-k6-skewed", level)
        assert abs(wl["maxvio"] - target) <= 0.02 * target, (level, wl["maxvio"])
