"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of oracle/kivi_oracle.c with one plausible mistake
(a dropped term, a wrong sign or index, a transposed operand, the wrong
rounding), built with the same flags into a temporary directory.  The test
requires at least one pin in tests/oracle_pins.py to fail on every mutant,
which shows the pins constrain each part of the oracle.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle.build_oracle import CMD, LIB, SRC
from oracle_pins import ALL_PINS

MUTANTS = [
    ("range_sign", "float range = mx - mn;", "float range = mx + mn;"),
    ("zero_is_max", "*zero = mn;", "*zero = mx;"),
    ("levels_off_by_one", "float levels = (float)((1 << bits) - 1);",
     "float levels = (float)(1 << bits);"),
    ("round_half_away", "float r = rintf(t);", "float r = roundf(t);"),
    ("truncate", "float r = rintf(t);", "float r = truncf(t);"),
    ("reciprocal_multiply", "float t = a / scale;",
     "float t = a * (1.0f / scale);"),
    ("fused_recon", "float p = (float)code * scale;\n    float r = p + zero;",
     "float r = fmaf((float)code, scale, zero);"),
    ("no_clip_top", "r = fminf(r, maxc);", "(void)maxc;"),
    ("no_signed_zero_canon", "if (mn == 0.0f) mn = 0.0f;", ""),
    ("pack_msb_first", "byte |= c << (i * bits);",
     "byte |= c << ((per - 1 - i) * bits);"),
    ("unpack_msb_first",
     "codes[r * D + d] = (uint8_t)((byte >> ((d % per) * bits)) & mask);",
     "codes[r * D + d] = (uint8_t)((byte >> ((per - 1 - d % per) * bits)) "
     "& mask);"),
    ("key_param_transposed",
     "scale[(bh * NG + g) * D + d] = sc;\n                zero[(bh * NG + g) * D + d] = z;",
     "scale[(bh * D + d) * NG + g] = sc;\n                zero[(bh * D + d) * NG + g] = z;"),
    ("key_group_bound_short", "int64_t s1 = s0 + group < S ? s0 + group : S;",
     "int64_t s1 = s0 + group - 1 < S ? s0 + group - 1 : S;"),
    ("value_group_bound_short",
     "int64_t d1 = d0 + group < D ? d0 + group : D;",
     "int64_t d1 = d0 + group - 1 < D ? d0 + group - 1 : D;"),
    ("dequant_key_group_index", "int64_t p = (bh * NG + s / group) * D + d;",
     "int64_t p = (bh * NG + s % NG) * D + d;"),
    ("dequant_value_group_index", "int64_t p = (bh * S + s) * NGD + d / group;",
     "int64_t p = (bh * S + s) * NGD + d % NGD;"),
    ("f16_round_half_up",
     "if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;",
     "if (rem >= 0x1000u) h += 1u;"),
    ("f16_truncate_subnormal",
     "if (rem > half || (rem == half && (q & 1u))) q += 1u;", ""),
    ("f16_overflow_threshold", "if (a >= 0x477ff000u)", "if (a >= 0x477fe000u)"),
    ("bf16_round_half_up", "uint32_t r = u + 0x7fffu + ((u >> 16) & 1u);",
     "uint32_t r = u + 0x8000u;"),
    ("f16_subnormal_scale", "v = ldexpf((float)m, -24);",
     "v = ldexpf((float)m, -25);"),
    ("subtract_dropped", "float a = f - zero;", "float a = f;"),
    ("cache_flush_early", "while (c->T - c->Q >= c->R + c->G_k) {",
     "while (c->T - c->Q >= c->R) {"),
    ("cache_flush_late", "while (c->T - c->Q >= c->R + c->G_k) {",
     "while (c->T - c->Q > c->R + c->G_k) {"),
    ("cache_key_group_slot",
     "c->k_scale + (bh * NG + c->Q / G) * D,",
     "c->k_scale + (bh * NG + c->T / G) * D,"),
    ("cache_value_rows_shifted",
     "c->v_codes + row * row_bytes,",
     "c->v_codes + (row + 1) * row_bytes,"),
    ("cache_history_overwrite",
     "memcpy(c->k + (bh * c->S_max + c->T) * D, k_new + (bh * n + i) * D,",
     "memcpy(c->k + (bh * c->S_max + c->Q) * D, k_new + (bh * n + i) * D,"),
    ("sink_in_minmax",
     "if (!sink[s - s0]) vals[n++] = widen(x[(bh * S + s) * D + d], dtype);",
     "vals[n++] = widen(x[(bh * S + s) * D + d], dtype);"),
    ("sink_code_not_zero",
     "sink[s - s0] ? 0 : (uint8_t)kivi_ref_code(f, sc, z, bits);",
     "(uint8_t)kivi_ref_code(f, sc, z, bits);"),
    ("sink_wrong_sequence", "int64_t b = bh / H;", "int64_t b = bh % H;"),
    ("sink_tie_higher_position",
     "if (best < 0 || score[b * S + s] > score[b * S + best]) best = s;",
     "if (best < 0 || score[b * S + s] >= score[b * S + best]) best = s;"),
    ("sink_select_repeats", "taken[best] = 1;", "(void)taken;"),
    ("sink_score_no_sqrt", "total = total + sqrtf(ss);", "total = total + ss;"),
    ("sink_score_no_mean", "score[b * S + s] = total / (float)H;",
     "score[b * S + s] = total;"),
    ("sink_score_head_stride",
     "const uint16_t* row = k + ((b * H + h) * S + s) * D;",
     "const uint16_t* row = k + ((b * H + h) * S + s) * D + (h > 0);"),
    ("sink_restore_row",
     "memcpy(out + (bh * S + s) * D, x_sink + (bh * n_sink + i) * D,",
     "memcpy(out + (bh * S + s) * D, x_sink + (bh * n_sink) * D,"),
    ("sink_gather_range",
     "if (s < 0 || s >= S) continue;\n            memcpy(x_sink",
     "if (s < 0 || s > S) continue;\n            memcpy(x_sink"),
    ("partition_tie_higher_first", "return (i > j) - (i < j);",
     "return (i < j) - (i > j);"),
    ("partition_lowest_scores", "    if (si > sj) return -1;\n    if (si < sj) return 1;",
     "    if (si > sj) return 1;\n    if (si < sj) return -1;"),
    ("partition_rank_from_bottom", "for (int64_t r = 0; r < n_hi; ++r) hi[order[r]] = 1;",
     "for (int64_t r = 0; r < n_hi; ++r) hi[order[S - 1 - r]] = 1;"),
    ("rows_gather_first_sequence",
     "memcpy(out + (bh * n + j) * D, x + (bh * S + pos[(bh / H) * n + j]) * D,",
     "memcpy(out + (bh * n + j) * D, x + (bh * S + pos[j]) * D,"),
    ("rows_scatter_shifted",
     "memcpy(out + (bh * S + pos[(bh / H) * n + j]) * D, r + (bh * n + j) * D,",
     "memcpy(out + (bh * S + pos[(bh / H) * n + j]) * D, r + (bh * n) * D,"),
    ("rows_values_group_doubled",
     "    int st = kivi_ref_quant_values(g, dtype, B * H, n, D, bits, group, packed,",
     "    int st = kivi_ref_quant_values(g, dtype, B * H, n, D, bits, group * 2, packed,"),
]


def _build_mutant(tmp, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name}: anchor not unique"
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    # the header sits next to the real source
    lib = os.path.join(tmp, f"lib{name}.so")
    cmd = list(CMD)
    cmd[cmd.index(LIB)] = lib
    cmd[cmd.index(SRC)] = path
    cmd.insert(1, "-I" + os.path.dirname(SRC))
    subprocess.run(cmd, check=True, capture_output=True)
    return lib


@pytest.fixture(scope="module")
def tmpdir_mut():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmpdir_mut, name, old, new):
    lib = _build_mutant(tmpdir_mut, name, old, new)
    o = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin catches mutant {name}"
