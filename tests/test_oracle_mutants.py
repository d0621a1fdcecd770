"""Power of the oracle's pins: plant a plausible mistake in a copy of
``oracle/oracle.c``, build it, and require that at least one pin fails.

Every mutant keeps all memory accesses in bounds (it only changes values),
so a mutant can fail but never crash the test process.  CPU only.
"""
import os

import pytest

import oracle
import oracle_pins as P

SRC = open(oracle.SRC).read()

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("decode_bias", "ldexp(1.0 + (double)m / 8.0, e - 7)",
     "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    ("decode_subnormal_exp", "ldexp((double)m / 8.0, -6)",
     "ldexp((double)m / 8.0, -7)"),
    ("decode_mantissa_width", "1.0 + (double)m / 8.0", "1.0 + (double)m / 16.0"),
    ("decode_sign_dropped", "return s ? -v : v;", "return v;"),
    ("decode_nan_as_max", "if (e == 15 && m == 7)", "if (e == 15 && m == 8)"),
    ("encode_truncates", "mant = nearbyint((2.0 * f - 1.0) * 8.0);",
     "mant = floor((2.0 * f - 1.0) * 8.0);"),
    ("encode_rounds_half_up", "mant = nearbyint((2.0 * f - 1.0) * 8.0);",
     "mant = floor((2.0 * f - 1.0) * 8.0 + 0.5);"),
    ("encode_subnormal_truncates", "mant = nearbyint(a * 512.0);",
     "mant = floor(a * 512.0);"),
    ("encode_no_saturation", "if (a >= 448.0)\n        return s | 0x7E;",
     "if (a >= 480.0)\n        return s | 0x7E;"),
    ("encode_nan_sign_dropped", "return s | 0x7F;", "return 0x7F;"),
    ("encode_subnormal_band_edge", "if (a < ldexp(1.0, -6)) {",
     "if (a < ldexp(1.0, -7)) {"),
    ("encode_exponent_bias", "return s | (uint8_t)(((k + 7) << 3) | (int)mant);",
     "return s | (uint8_t)(((k + 6) << 3) | (int)mant);"),
    ("bf16_widen_shift", "uint32_t u = (uint32_t)h << 16;",
     "uint32_t u = (uint32_t)h << 15;"),
    ("writer_scale_448", "scale = amax == 0.0f ? 1.0f : amax / 448.0f;",
     "scale = amax == 0.0f ? 1.0f : amax / 447.0f;"),
    ("writer_scale_reciprocal", "dst[g * ORC_GROUP + j] = orc_fp8_encode(v / scale);",
     "dst[g * ORC_GROUP + j] = orc_fp8_encode(v * (1.0f / scale));"),
    ("writer_scale_order", "memcpy(dst + ORC_D + 4 * g, &scale, 4);",
     "memcpy(dst + ORC_D + 4 * (3 - g), &scale, 4);"),
    ("writer_zero_group_scale", "scale = amax == 0.0f ? 1.0f : amax / 448.0f;",
     "scale = amax == 0.0f ? 0.5f : amax / 448.0f;"),
    ("writer_error_count", "if (slot >= num_slots) {\n            errors++;",
     "if (slot >= num_slots) {\n            errors += 2;"),
    ("q_scale_448", "return amax == 0.0f ? 1.0f : amax / 448.0f;\n}",
     "return amax == 0.0f ? 1.0f : amax / 440.0f;\n}"),
    ("q_quantize_multiplies", "q8[i] = orc_fp8_encode(bf16_to_f32(q[i]) / scale);",
     "q8[i] = orc_fp8_encode(bf16_to_f32(q[i]) * scale);"),
    ("resolve_offset", "slot = (int64_t)phys * page_size + (i % page_size);",
     "slot = (int64_t)phys * page_size + ((i + 1) % page_size);"),
    ("resolve_page_stride", "slot = (int64_t)phys * page_size + (i % page_size);",
     "slot = (int64_t)(phys ^ 1) * page_size + (i % page_size);"),
    ("resolve_seq_len_inclusive", "if (seq_lens && i >= seq_lens[seq]) {",
     "if (seq_lens && i > seq_lens[seq]) {"),
    ("resolve_padding_counted", "    if (i == -1)\n        return -1;\n", ""),
    ("resolve_no_seq_lens", "if (seq_lens && i >= seq_lens[seq]) {",
     "if (seq_lens && i >= (1 << 30)) {"),
    ("dequant_group_index", "(double)scale[d / ORC_GROUP]", "(double)scale[d % 4]"),
    ("dequant_scale_ignored", "x[d] = orc_fp8_decode(row[d]) * (double)scale[d / ORC_GROUP];",
     "x[d] = orc_fp8_decode(row[d]);"),
    ("score_scale_dropped", "s[j] = (double)jb->softmax_scale * dot;", "s[j] = dot;"),
    ("score_scale_squared", "s[j] = (double)jb->softmax_scale * dot;",
     "s[j] = (double)jb->softmax_scale * (double)jb->softmax_scale * dot;"),
    ("softmax_sign", "double w = exp(s[j] - M);", "double w = exp(M - s[j]);"),
    ("softmax_no_normalise", "o[d] /= L;", "o[d] /= 1.0;"),
    ("lse_log_dropped", "jb->lse[(int64_t)t * jb->H + h] = M + log(L);",
     "jb->lse[(int64_t)t * jb->H + h] = M;"),
    ("query_head_ignored", "int64_t qoff = ((int64_t)t * jb->H + h) * (ORC_D + rope);",
     "int64_t qoff = ((int64_t)t * jb->H + (h & ~1)) * (ORC_D + rope);"),
    ("rope_term_dropped", "dot += qh[ORC_D + r] * xr[(int64_t)j * ORC_ROPE + r];",
     "dot += 0.0 * qh[ORC_D + r] * xr[(int64_t)j * ORC_ROPE + r];"),
    ("rope_byte_order", "(row[ORC_SCALED_BYTES + 2 * r + 1] << 8)", "(row[ORC_SCALED_BYTES + 2 * r + 1] << 7)"),
    ("bf16_row_byte_order", "x[d] = bf16_to_f32((uint16_t)(row[2 * d] | (row[2 * d + 1] << 8)));",
     "x[d] = bf16_to_f32((uint16_t)(row[2 * d + 1] | (row[2 * d] << 8)));"),
    ("bf16_writer_high_byte", "dst[2 * d + 1] = (uint8_t)(src[d] >> 8);", "dst[2 * d + 1] = (uint8_t)(src[d] >> 9);"),
    ("writer_rope_not_copied", "dst[ORC_SCALED_BYTES + 2 * r] = (uint8_t)(src[ORC_D + r] & 0xff);",
     "dst[ORC_SCALED_BYTES + 2 * r] = 0;"),
    ("query_fp8_scale_ignored", "(double)jb->q_scale;", "1.0;"),
    ("all_masked_nan", "if (nv == 0) {", "if (nv < 0) {"),
    ("all_masked_lse_zero", "jb->lse[(int64_t)t * jb->H + h] = -INFINITY;",
     "jb->lse[(int64_t)t * jb->H + h] = 0.0;"),
    ("duplicates_dropped", "            nv++;\n",
     "            if (nv == 0 || memcmp(x + (int64_t)(nv - 1) * ORC_D, "
     "x + (int64_t)nv * ORC_D, ORC_D * sizeof(double)) != 0) nv++;\n"),
    ("token_sequence_ignored", "int seq = jb->token_seq ? jb->token_seq[t] : t;",
     "int seq = jb->token_seq ? 0 : t;"),
    ("transform_keeps_masked", "            if (slot >= 0)\n                row[n++] = (int32_t)slot;",
     "            if (slot >= -1)\n                row[n++] = (int32_t)slot;"),
    ("transform_reverses", "row[n++] = (int32_t)slot;", "row[k_in - 1 - n++] = (int32_t)slot;"),
    ("transform_pads_zero", "        for (int j = n; j < k_out; j++)\n            row[j] = -1;",
     "        for (int j = n; j < k_out; j++)\n            row[j] = 0;"),
    ("transform_count_off", "counts[t] = n;", "counts[t] = n + (t & 1);"),
]


def test_every_mutation_site_exists():
    for name, old, new in MUTANTS:
        assert SRC.count(old) >= 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    assert old in SRC
    src = tmp_path / "oracle_mutant.c"
    src.write_text(SRC.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    oracle.build(str(src), str(lib))
    mut = oracle.Oracle(str(lib))
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mut)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin catches mutant {name}"
