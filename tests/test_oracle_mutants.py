"""The oracle's pins must catch plausible mistakes (CPU only).

Each mutant is a copy of ``oracle/pkv_oracle.c`` with one planted mistake (a
dropped term, a wrong index, a swapped operand, a wrong log base ...),
compiled into a temporary library.  Every pin of ``test_oracle_pins`` is run
against it and at least one must fail.  Every mutant keeps its memory accesses
inside the arrays, so a mutant can only give wrong numbers, never crash.
"""
from __future__ import annotations

import os

import pytest

import oracle
from test_oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "pkv_oracle.c")

MUTANTS = {
    "prefill_not_causal": (
        "qrow, hq / group, pages, 0, pos + 1, sm_scale, scores,",
        "qrow, hq / group, pages, 0, len, sm_scale, scores,"),
    "prefill_causal_excludes_self": (
        "qrow, hq / group, pages, 0, pos + 1, sm_scale, scores,",
        "qrow, hq / group, pages, 0, pos + (pos == 0), sm_scale, scores,"),
    "prefill_position_from_start": (
        "int64_t pos = len - n + j;",
        "int64_t pos = j;"),
    "prefill_gqa_modulo": (
        "qrow, hq / group, pages, 0, pos + 1, sm_scale, scores,",
        "qrow, hq % num_kv_heads, pages, 0, pos + 1, sm_scale, scores,"),
    "append_rows_shifted": (
        "int64_t t = len - n + j;",
        "int64_t t = (len - n + j + 1) % len;"),
    "append_rows_v_into_k": (
        "cache[dk + d] = k_new[src + d];\n                    cache[dv + d] = v_new[src + d];",
        "cache[dk + d] = v_new[src + d];\n                    cache[dv + d] = v_new[src + d];"),
    "rope_sin_sign": (
        "y[i] = lo * c - hi * s;",
        "y[i] = lo * c + hi * s;"),
    "rope_second_half_sign": (
        "y[i + half] = hi * c + lo * s;",
        "y[i + half] = hi * c - lo * s;"),
    "rope_frequency_exponent": (
        "pow(theta, -2.0 * (double)i / (double)head_dim)",
        "pow(theta, -1.0 * (double)i / (double)head_dim)"),
    "rope_interleaved_pairs": (
        "double lo = y[i], hi = y[i + half];",
        "double lo = y[(2 * i) % head_dim], hi = y[(2 * i + 1) % head_dim];"),
    "rope_position_off_by_one": (
        "pair_pos[i] = (double)positions[b * pos_stride + axis];",
        "pair_pos[i] = (double)positions[b * pos_stride + axis] + 1.0;"),
    "mrope_axis_ignored": (
        "int64_t axis = pair_axis ? pair_axis[i] : 0;",
        "int64_t axis = 0;"),
    "mrope_axis_shifted": (
        "int64_t axis = pair_axis ? pair_axis[i] : 0;",
        "int64_t axis = pair_axis ? pair_axis[(i + 1) % (head_dim / 2)] : 0;"),
    "mrope_position_stride_dropped": (
        "pair_pos[i] = (double)positions[b * pos_stride + axis];",
        "pair_pos[i] = (double)positions[b + axis];"),
    "rmsnorm_eps_dropped": (
        "sqrt(ss / (double)head_dim + eps)",
        "sqrt(ss / (double)head_dim + 0.0 * eps)"),
    "rmsnorm_sum_not_mean": (
        "sqrt(ss / (double)head_dim + eps)",
        "sqrt(ss + eps)"),
    "rmsnorm_weight_dropped": (
        "y[d] = widen_bf16(x[d]) * inv * widen_bf16(w[d]);",
        "y[d] = widen_bf16(x[d]) * inv * (w[d] != 0 ? 1.0 : 1.0);"),
    "k_norm_uses_q_weight": (
        "rms_norm_row(k_new + row, k_w, head_dim, eps, k_out + row);",
        "rms_norm_row(k_new + row, q_w, head_dim, eps, k_out + row);"),
    "norm_rope_v_from_k": (
        "cache[dv + d] = v_new[row + d];",
        "cache[dv + d] = k_new[row + d];"),
    "bf16_round_ties_away": (
        "u += 0x7FFFu + ((u >> 16) & 1u);",
        "u += 0x8000u;"),
    "bf16_round_double_rounding": (
        "if ((u & 0xFFFFu) == 0x8000u && (double)f != x) {",
        "if ((u & 0xFFFFu) == 0x8000u && (double)f != x && 0) {"),
    "append_slot_off_by_one": (
        "int64_t slot = last_page_len[b] - 1;",
        "int64_t slot = last_page_len[b] % page_size;"),
    "append_first_page_not_last": (
        "int64_t page = page_indices[page_indptr[b + 1] - 1];",
        "int64_t page = page_indices[page_indptr[b]];"),
    "append_v_into_k": (
        "cache[dk + d] = k_new[src + d];",
        "cache[dk + d] = v_new[src + d];"),
    "append_wrong_head_row": (
        "int64_t src = (b * num_kv_heads + h) * head_dim;",
        "int64_t src = (b * num_kv_heads + (num_kv_heads - 1 - h)) * head_dim;"),
    "gqa_modulo_head_map": (
        "int64_t h = hq / group;",
        "int64_t h = hq % num_kv_heads;"),
    "length_counts_whole_last_page": (
        "return (n - 1) * page_size + last_len[b];",
        "return n * page_size;"),
    "length_drops_new_row": (
        "return (n - 1) * page_size + last_len[b];",
        "return (n - 1) * page_size + last_len[b] - (last_len[b] > 1);"),
    "token_slot_shifted": (
        "page, 0, t % page_size, h);",
        "page, 0, (t + 1) % page_size, h);"),
    "scale_dropped": (
        "scores[t - t0] = sm_scale * dot;",
        "scores[t - t0] = dot;"),
    "no_max_shift": (
        "z += exp(scores[t - t0] - m);\n    *lse = m + log(z);",
        "z += exp(scores[t - t0]);\n    *lse = log(z);"),
    "lse_log2": (
        "*lse = m + log(z);",
        "*lse = m + log2(z);"),
    "weights_not_normalised": (
        "double w = exp(scores[t - t0] - *lse);",
        "double w = exp(scores[t - t0] - m);"),
    "values_read_from_k_half": (
        "page, 1, t % page_size, h);",
        "page, 0, t % page_size, h);"),
    "key_elements_reversed": (
        "dot += widen_bf16(qrow[d]) * widen_bf16(cache[kr + d]);",
        "dot += widen_bf16(qrow[d]) * widen_bf16(cache[kr + (head_dim - 1 - d)]);"),
    "query_heads_reversed": (
        "const uint16_t *qrow = q + (b * num_qo_heads + hq) * head_dim;",
        "const uint16_t *qrow = q + (b * num_qo_heads + (num_qo_heads - 1 - hq)) "
        "* head_dim;"),
    "merge_plain_average": (
        "double w = exp(lse_c[c] - *lse);",
        "double w = 1.0 / (double)nchunks;"),
    "merge_lse_without_max": (
        "*lse = mx + log(s);",
        "*lse = log(s);"),
    "widen_drops_low_mantissa": (
        "uint32_t u = (uint32_t)bits << 16;",
        "uint32_t u = (uint32_t)(bits & 0xFFF0) << 16;"),
    "layer_ignored": (
        "int64_t r = layer;",
        "int64_t r = 0 * layer;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    mutated = text.replace(old, new)
    src = tmp_path / "mutant.c"
    src.write_text(mutated)
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))
    failed = []
    for pin in PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
        except ValueError:       # the wrapper saw an error code: also caught
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
