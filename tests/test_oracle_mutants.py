"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each mutant is a copy of ``oracle/pc_oracle.c`` with one plausible mistake (a
wrong index, a dropped term, a swapped stride, an off-by-one), compiled to a
temporary library.  The pins run against it; at least one must fail.  Mistakes are
only ever planted in the oracle, on the CPU.
"""

import os

import pytest

import oracle
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "pc_oracle.c")

MUTANTS = {
    "gqa_modulo": ("int kv = h / G;", "int kv = h % j->num_kv_heads;"),
    "slot_offset_shift": ("int64_t off = slot % block_size;", "int64_t off = (slot + 1) % block_size;"),
    "slot_block_divisor": ("int64_t blk = slot / block_size;", "int64_t blk = slot / (block_size + 1);"),
    "write_strides_swapped": ("int64_t dst = blk * block_stride + off * token_stride + (int64_t)h * head_stride;",
                              "int64_t dst = blk * block_stride + off * head_stride + (int64_t)h * token_stride;"),
    "negative_slot_written": ("if (slot < 0)\n            continue;", "if (slot < -1)\n            continue;"),
    "read_logical_block": ("int lb = t / j->block_size;", "int lb = t / (2 * j->block_size);"),
    "read_offset_shift": ("int off = t % j->block_size;", "int off = (t + 1) % j->block_size;"),
    "value_from_key_pool": ("load_elem(j->v_pool, base + d, j->kv_fmt) * vs;",
                            "load_elem(j->k_pool, base + d, j->kv_fmt) * vs;"),
    "query_head_swapped": ("qv[d] = load_elem(j->q, ((int64_t)s * j->num_q_heads + h) * D + d, j->fmt);",
                           "qv[d] = load_elem(j->q, ((int64_t)s * j->num_q_heads + (h ^ 1)) * D + d, j->fmt);"),
    "scale_dropped": ("x[t] = scale * dot + slope", "x[t] = dot + slope"),
    "max_not_subtracted": ("x[t] = exp(x[t] - m);", "x[t] = exp(x[t]);"),
    "epsilon_denominator": ("o[d] = acc / l;", "o[d] = acc / (l + 1e-6);"),
    "last_token_dropped": ("dense_attention(qv, K, V, L, D, j->scale,", "dense_attention(qv, K, V, L > 1 ? L - 1 : L, D, j->scale,"),
    "partition_not_clipped": ("int t1 = t0 + j->partition_size < L ? t0 + j->partition_size : L;",
                              "int t1 = t0 + j->partition_size;"),
    "merge_without_rescale": (
        "double w = exp_sums[sh * max_partitions + p] * exp(max_logits[sh * max_partitions + p] - M);",
        "double w = exp_sums[sh * max_partitions + p];"),
    "bf16_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "f16_exponent_bias": ("v = ldexp((double)(m + 1024), e - 25);", "v = ldexp((double)(m + 1024), e - 24);"),
    "f16_subnormal_scale": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "e4m3_exponent_bias": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 9)"),
    "e4m3_subnormal_scale": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "e4m3_ties_to_odd": ("((lo & 1) ? lo + 1 : lo)", "((lo & 1) ? lo : lo + 1)"),
    "e4m3_overflow_to_nan": ("if (a >= 448.0)\n        return sign | 0x7e;", "if (a >= 464.0)\n        return sign | 0x7f;"),
    "kv8_scale_multiplied": ("k_pool[dst + d] = e4m3_from_float(kx / ks);", "k_pool[dst + d] = e4m3_from_float(kx * ks);"),
    "kv8_write_scale_head0": ("float vs = v_scale[(int64_t)h * scale_stride];", "float vs = v_scale[0];"),
    "kv8_read_scale_dropped": ("ks = (double)j->k_scale[(int64_t)kv * j->scale_stride];", "ks = 1.0;"),
    "kv8_read_v_scale_from_k": ("vs = (double)j->v_scale[(int64_t)kv * j->scale_stride];",
                                "vs = (double)j->k_scale[(int64_t)kv * j->scale_stride];"),
    "alibi_sign_flipped": ("+ slope * (double)(pos0 + t);", "- slope * (double)(pos0 + t);"),
    "alibi_slope_of_kv_head": ("int kv = h / G;\n    double slope = j->alibi_slopes ? (double)j->alibi_slopes[h]",
                               "int kv = h / G;\n    double slope = j->alibi_slopes ? (double)j->alibi_slopes[kv]"),
    "varlen_alibi_slope_of_kv_head": ("(double)j->alibi_slopes[h] : 0.0;\n    double m, l;",
                                      "(double)j->alibi_slopes[h / G] : 0.0;\n    double m, l;"),
    "alibi_partition_origin": ("(int64_t)t0 - (L - 1)", "-(int64_t)(L - 1)"),
    "alibi_partials_off_by_one": ("(int64_t)t0 - (L - 1)", "(int64_t)t0 - L"),
    "varlen_causal_off_by_one": ("int visible = j->causal ? p + 1 : L;", "int visible = j->causal ? p : L;"),
    "varlen_top_left_causal": ("int visible = j->causal ? p + 1 : L;", "int visible = j->causal ? i + 1 : L;"),
    "varlen_causal_ignored": ("int visible = j->causal ? p + 1 : L;", "int visible = L;"),
    "varlen_request_lookup": ("if (qs[mid] <= row)", "if (qs[mid] < row)"),
}


def _build_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    # a site shared by the plain and the 8-bit write is mutated in both
    assert text.count(old) >= 1, f"mutation site for {name} is not present"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    out = tmp_path / f"{name}.so"
    oracle.build(force=True, src=str(src), out=str(out))
    return str(out)


def _failures():
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, oracle.OracleError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert _failures() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    path = _build_mutant(name, tmp_path)
    with oracle.using(path):
        failed = _failures()
    assert failed, f"planted mistake '{name}' passed every pin"
