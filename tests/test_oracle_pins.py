"""The oracle against its pins (CPU only).

The pins themselves live in ``oracle_pins.py``; this file runs them on the
oracle, checks the closed form on the pages' worked example and on every
workload shape, and shows that mutated copies of the oracle fail the pins.
"""
import json
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle
import oracle_pins
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


def test_offsets_match_numpy_layouts(lib):
    oracle_pins.check_offsets(lib)


def test_brute_force_coordinate_decoding(lib):
    oracle_pins.check_brute_force(lib)


def test_numpy_transpose_special_cases(lib):
    oracle_pins.check_numpy(lib)


def test_round_trip_and_untouched_regions(lib):
    oracle_pins.check_round_trip(lib)


def test_prompt_ranges_hand_worked(lib):
    oracle_pins.check_prompt_ranges(lib)


def test_ring_restore_last_writer_wins(lib):
    oracle_pins.check_ring(lib)


def test_restart_point_hand_worked(lib):
    oracle_pins.check_restart_point(lib)


def test_stream_split_and_merge(lib):
    oracle_pins.check_stream(lib)


def test_paged_pool(lib):
    oracle_pins.check_paged(lib)


def test_swap_pays_closed_forms(lib):
    oracle_pins.check_swap_pays(lib)


def test_closed_form_on_the_pages_example(lib):
    """KV bytes of the lsln.cn 100K-context example equal 2 x B x S x H x D x P x N."""
    with open(os.path.join(HERE, "golden", "kv_capacity_100k.json")) as f:
        g = json.load(f)
    dims = (g["N"], g["B"], g["H"], g["D"], g["S"])
    elems = oracle.pack_elems(dims, g["N"], [g["S"]] * g["B"], lib=lib)
    page = 2 * g["B"] * g["S"] * g["H"] * g["D"] * g["P"] * g["N"]
    assert elems * g["P"] == page == 24_576_000_000


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_closed_form_every_workload(lib, name):
    """One pack of every row's first S tokens over all N layers moves 2BSHDPN bytes."""
    w = synth.WORKLOADS[name]
    for S in (1, w.Smax // 2, w.Smax):
        elems = oracle.pack_elems(w.dims, w.L, [S] * w.B, lib=lib)
        assert elems * 2 == 2 * w.B * S * w.H * w.D * 2 * w.L


# ---- mutants: each is a plausible mistake planted in a copy of oracle.c ----
MUTANTS = {
    "key_chunk_lane_swapped": ("int64_t chunk = d / 8;", "int64_t chunk = d % 8;"),
    "key_layout_transposed": ("* (D / 8) + chunk) * Smax + s) * 8 + lane",
                              "* Smax + s) * (D / 8) + chunk) * 8 + lane"),
    "key_row_term_dropped": ("return ((((l * B + b) * H + h) * (D / 8)",
                             "return ((((l * B + 0) * H + h) * (D / 8)"),
    "value_layout_transposed": ("return (((l * B + b) * H + h) * Smax + s) * D + d;",
                                "return (((l * B + b) * H + h) * D + d) * Smax + s;"),
    "value_head_term_dropped": ("return (((l * B + b) * H + h) * Smax + s) * D + d;",
                                "return (((l * B + b) * H + 0) * Smax + s) * D + d;"),
    "pack_start_dropped": ("  int64_t s = start[b] + t;\n                            if (kv == 0)\n                                out",
                           "  int64_t s = t;\n                            if (kv == 0)\n                                out"),
    "pack_kv_swapped": ("  int64_t s = start[b] + t;\n                            if (kv == 0)\n                                out[o] = key[",
                        "  int64_t s = start[b] + t;\n                            if (kv == 0)\n                                out[o] = value["),
    "pack_last_token_dropped": ("for (int64_t t = 0; t < count[b]; ++t)\n                        for (int64_t d = 0; d < D; ++d) {\n                            int64_t s = start[b] + t;\n                            if (kv == 0)\n                                out",
                                "for (int64_t t = 0; t + 1 < count[b]; ++t)\n                        for (int64_t d = 0; d < D; ++d) {\n                            int64_t s = start[b] + t;\n                            if (kv == 0)\n                                out"),
    "unpack_kv_swapped": ("  int64_t s = start[b] + t;\n                            if (kv == 0)\n                                key[oracle_key_offset(L, B, H, D, Smax, l, b, h, s, d)] = in[o];",
                          "  int64_t s = start[b] + t;\n                            if (kv == 0)\n                                value[oracle_key_offset(L, B, H, D, Smax, l, b, h, s, d)] = in[o];"),
    "unpack_start_dropped": ("  int64_t s = start[b] + t;\n                            if (kv == 0)\n                                key",
                             "  int64_t s = t;\n                            if (kv == 0)\n                                key"),
    "size_factor_dropped": ("return 2 * layer_count * H * D * tokens;",
                            "return layer_count * H * D * tokens;"),
    "prompt_clip_missing": ("if (row_len != NULL && row_len[b] < end)",
                            "if (row_len != NULL && row_len[b] > end)"),
    "restart_worker_any_not_all": ("                    if (ack_x[a] == x && ack_j[a] == j && ack_t[a] >= t)",
                                   "                    if (ack_j[a] == j && ack_t[a] >= t)"),
    "restart_order_mb_major": ("    for (int64_t t = 0; t <= max_step; ++t)\n        for (int64_t j = 0; j < microbatches; ++j)\n            for (int64_t x = 0; x < workers; ++x) {",
                               "    for (int64_t j = 0; j < microbatches; ++j)\n        for (int64_t t = 0; t <= max_step; ++t)\n            for (int64_t x = 0; x < workers; ++x) {"),
    "restart_ack_exclusive": ("ack_t[a] >= t)", "ack_t[a] > t)"),
    "swap_pays_upper_bound_exclusive": ("for (int64_t i = p; i <= N + p; ++i) {\n        double transfer",
                                        "for (int64_t i = p; i < N + p; ++i) {\n        double transfer"),
    "swap_pays_batch_dropped": ("double transfer = (double)i * (double)B * C / bw;",
                                "double transfer = (double)i * C / bw;"),
    "swap_pays_single_run": ("*lhs = 2.0 * (double)N * t;", "*lhs = (double)N * t;"),
    "stream_out_head_from_meet": ("b = gr - src[4], h = gh - src[2];", "b = gr - src[4], h = gh - h_lo;"),
    "stream_in_row_from_source": ("const int64_t l = gl - dst[0], b = gr - dst[4]",
                                  "const int64_t l = gl - dst[0], b = gr - src[4]"),
    "stream_meet_upper_from_first": ("*hi = (a0 + an) < (b0 + bn) ? (a0 + an) : (b0 + bn);",
                                     "*hi = a0 + an;"),
    "stream_out_heads_before_rows": ("            for (int64_t gr = r_lo; gr < r_hi; ++gr)\n                for (int64_t gh = h_lo; gh < h_hi; ++gh) {\n                    const int64_t l = gl - src[0]",
                                     "            for (int64_t gh = h_lo; gh < h_hi; ++gh)\n                for (int64_t gr = r_lo; gr < r_hi; ++gr) {\n                    const int64_t l = gl - src[0]"),
    "stream_size_counts_destination_rows": ("tokens += count[r - src[4]];", "tokens += count[r - dst[4]];"),
    "paged_block_and_slot_swapped": ("const int64_t blk = table[b * stride + s / P];\n                        const int64_t slot = s % P;\n                        for (int64_t d = 0; d < D; ++d) {\n                            if (kv == 0)\n                                out",
                                     "const int64_t blk = table[b * stride + s % P];\n                        const int64_t slot = s / P;\n                        for (int64_t d = 0; d < D; ++d) {\n                            if (kv == 0)\n                                out"),
    "paged_table_stride_ignored": ("const int64_t blk = table[b * stride + s / P];\n                        const int64_t slot = s % P;\n                        for (int64_t d = 0; d < D; ++d) {\n                            if (kv == 0)\n                                out",
                                   "const int64_t blk = table[b + s / P];\n                        const int64_t slot = s % P;\n                        for (int64_t d = 0; d < D; ++d) {\n                            if (kv == 0)\n                                out"),
    "paged_key_layout_transposed": ("* (D / 8) + d / 8) * P + o) * 8 + d % 8;",
                                    "* P + o) * (D / 8) + d / 8) * 8 + d % 8;"),
    "paged_value_block_term_dropped": ("return (((l * NB + blk) * H + h) * P + o) * D + d;",
                                       "return (((l * NB + 0) * H + h) * P + o) * D + d;"),
    "unpack_paged_slot_from_t": ("const int64_t slot = s % P;\n                        for (int64_t d = 0; d < D; ++d) {\n                            if (kv == 0)\n                                key",
                                 "const int64_t slot = t % P;\n                        for (int64_t d = 0; d < D; ++d) {\n                            if (kv == 0)\n                                key"),
    "ring_order_reversed": ("for (int64_t j = 0; j < steps; ++j)\n        oracle_unpack(L, B, H, D, Smax, key, value, 0, L, pos + j * B",
                            "for (int64_t j = steps - 1; j >= 0; --j)\n        oracle_unpack(L, B, H, D, Smax, key, value, 0, L, pos + j * B"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    oracle.build(str(so), str(mutant))
    # run the pins in a child: a mutant may also crash; either way it must not pass
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), str(so)],
                       cwd=os.path.dirname(HERE), capture_output=True, text=True,
                       env={**os.environ, "PYTHONPATH": os.path.dirname(HERE)}, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin"


def test_pins_pass_on_the_real_oracle_in_a_child():
    """The child-process route used for mutants exits 0 on the unmodified oracle."""
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), oracle._LIB],
                       cwd=os.path.dirname(HERE), capture_output=True, text=True,
                       env={**os.environ, "PYTHONPATH": os.path.dirname(HERE)}, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
