"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of moon_oracle.cpp with one plausible mistake (a dropped
term, a wrong index or sign, a swapped order, a wrong rounding).  It is
compiled to a temporary library and the pin tests run against it in a
subprocess; every mutant must make them fail.  The oracle source itself is
never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "histogram_drops_other_ranks": ("T[e] += 1;", "T[e] += (r == 0);"),
    "stream_offset_off_by_one_group": ("      Pe[e] = acc;\n      acc += T[e];",
                                       "      acc += T[e];\n      Pe[e] = acc;"),
    "alias_take_from_original_load": ("int64_t f = C - rem[u];", "int64_t f = C - L[u];"),
    "alias_last_donor_first": ("int o = large.front();", "int o = large.back();"),
    "slot_index_ignores_segment_start": ("idx = q - std::max(Pe[e], seg_a[u]);",
                                         "idx = q - Pe[e];"),
    "layout_without_padding": ("acc += padded(n[ug], P);", "acc += n[ug];"),
    "zero_fill_from_group_start": ("zfr[ug * 2 + 0] = (int32_t)(start[ug] + n[ug]);",
                                   "zfr[ug * 2 + 0] = (int32_t)(start[ug]);"),
    "dedup_counts_itself": ("for (int k2 = 0; k2 < k; ++k2)", "for (int k2 = 0; k2 <= k; ++k2)"),
    "dup_loff_begin_wrong": ("rec[1] = (int32_t)nd;", "rec[1] = (int32_t)ng;"),
    "route_weight_of_first_k": ("if (w != nullptr) wwin[G] = w[t * K + k];",
                                "if (w != nullptr) wwin[G] = w[t * K];"),
    "combine_drops_weight": ("float c32 = weighted ? wk : 1.0f;", "float c32 = 1.0f;"),
    "combine_fused_multiply_add": ("      sum32[h] = sum32[h] + prod;\n    }\n    if (acc != nullptr)",
                                   "      sum32[h] = std::fma(c32, yv, sum32[h]);\n    }\n"
                                   "    if (acc != nullptr)"),
    "combine_output_from_float64": ("    if (wsk != nullptr) wsk[k] = wk;\n  }\n  for (int h = 0; h < H; ++h) {\n"
                                    "    out[h] = orc_bf16_from_double((double)sum32[h]);",
                                    "    if (wsk != nullptr) wsk[k] = wk;\n  }\n  for (int h = 0; h < H; ++h) {\n"
                                    "    out[h] = orc_bf16_from_double(sum[h]);"),
    "combine_descending_k": ("  for (int k = 0; k < K; ++k) {\n    int64_t G = decode_row(d[k]);\n"
                             "    const uint16_t* y = row(G);",
                             "  for (int k = K - 1; k >= 0; --k) {\n    int64_t G = decode_row(d[k]);\n"
                             "    const uint16_t* y = row(G);"),
    "dst_decode_off_by_one": ("return d >= 0 ? (int64_t)d : -(int64_t)d - 1;",
                              "return d >= 0 ? (int64_t)d : -(int64_t)d;"),
    "rounding_truncates": ("double r = std::nearbyint(scaled);", "double r = std::trunc(scaled);"),
    "remote_stats_counts_all_slots": ("if (etc[(size_t)u * B + j] >= 0) {", "if (true) {"),
    "prologue_fold_drops_weight": ("float c = weighted ? wat(Gm) : 1.0f;", "float c = 1.0f;"),
    "prefetch_copies_neighbour_expert": ("std::memcpy(dst, experts[t] + (int64_t)e * row_bytes[t],",
                                         "std::memcpy(dst, experts[t] + (int64_t)(e ^ 1) * "
                                         "row_bytes[t],"),
    "prefetch_slot_index_transposed": ("uint8_t* dst = slots[t] + ((int64_t)u * B + j) * row_bytes[t];",
                                       "uint8_t* dst = slots[t] + ((int64_t)j * R + u) * row_bytes[t];"),
    "reduce_grad_ranks_descending": ("      for (int u = 0; u < R; ++u) {\n        for (int j = 0; j < B; ++j) {\n"
                                     "          if (etc[u * B + j] != e) continue;",
                                     "      for (int u = R - 1; u >= 0; --u) {\n        for (int j = 0; j < B; ++j) {\n"
                                     "          if (etc[u * B + j] != e) continue;"),
    "reduce_grad_keeps_slots": ("        if (etc[u * B + j] >= 0)\n          std::fill(",
                                "        if (etc[u * B + j] >= 1 << 30)\n          std::fill("),
    "reduce_grad_overwrites_seed": ("g[x] = g[x] + sg[x];", "g[x] = sg[x];"),
    "segments_in_rank_order": ("  for (int u : served) {\n    int o = donor[u];",
                               "  for (int u = 0; u < R; ++u) {\n    int o = donor[u];\n"
                               "    if (o < 0) continue;"),
    "cu_seqlens_exclusive": ("cu[ug] = (int32_t)acc;", "cu[ug] = (int32_t)start[ug];"),
    "primary_is_last_route": ("for (int k2 = 0; k2 < k; ++k2)", "for (int k2 = k + 1; k2 < K; ++k2)"),
    "expert_id_E_accepted": ("if (e < 0 || e >= E) return ST_BAD_EXPERT;",
                             "if (e < 0 || e > E) return ST_BAD_EXPERT;"),
    "padding_weights_kept": ("if (w != nullptr) wwin[G] = 0.0f;", "(void)w;"),
    "gathered_weight_of_first_route": ("    if (wsk != nullptr) wsk[k] = wk;",
                                       "    if (wsk != nullptr) wsk[k] = wat(decode_row(d[0]));"),
    "capacity_without_slot_padding": ("(Eg + B) * (int64_t)(P - 1)", "Eg * (int64_t)(P - 1)"),
    "histogram_checks_rank_zero_only": ("for (int64_t j = 0; j < (int64_t)R * E; ++j)\n"
                                        "      if ((int64_t)tpe[j] != cnt[j]) return ST_HISTOGRAM;",
                                        "for (int64_t j = 0; j < (int64_t)E; ++j)\n"
                                        "      if ((int64_t)tpe[j] != cnt[j]) return ST_HISTOGRAM;"),
    "slot_budget_not_reported": ("if (over_budget) return ST_SLOT_BUDGET;",
                                 "if (over_budget && false) return ST_SLOT_BUDGET;"),
    "prefetch_index_owner_and_row_swapped": ("out[j * 2 + 0] = e >= 0 ? e / Eg : -1;\n"
                                             "    out[j * 2 + 1] = e >= 0 ? e % Eg : -1;",
                                             "out[j * 2 + 0] = e >= 0 ? e % Eg : -1;\n"
                                             "    out[j * 2 + 1] = e >= 0 ? e / Eg : -1;"),
    "nan_rounds_to_infinity": ("if (std::isnan(v)) return 0x7FC0;",
                               "if (std::isnan(v)) return 0x7F80;"),
}

PIN_TESTS = ["tests/test_oracle_plan.py", "tests/test_oracle_data.py", "tests/test_oracle_weights.py"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(os.path.join(ROOT, "oracle", "moon_oracle.cpp")) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mdir = tmp_path / "oracle"
    mdir.mkdir()
    (mdir / "moon_oracle.cpp").write_text(src.replace(old, new))
    (mdir / "moon_oracle.h").write_text(open(os.path.join(ROOT, "oracle", "moon_oracle.h")).read())
    so = str(mdir / "liboracle_mutant.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-ffp-contract=off", "-shared", "-fPIC",
                    str(mdir / "moon_oracle.cpp"),
                    "-o", so], check=True)
    env = dict(os.environ, MOON_ORACLE_SO=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_TESTS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"


def test_unmutated_oracle_passes_pins():
    oracle._load()  # builds if needed
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_TESTS], cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
