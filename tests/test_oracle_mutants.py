"""Each pin must bite: plant a plausible mistake in a copy of the oracle source,
build it with gcc, and check that at least one pin fails. Also checks that the
written pool layout is a bijection onto the slab."""
import pytest

import oracle
from tests import test_oracle_attention as TA
from tests import test_oracle_calibration as TC
from tests import test_oracle_extend as TE
from tests import test_oracle_fp8 as T8
from tests import test_oracle_format as TF

# (name, original text, replacement) — each is a single plausible slip that keeps every
# memory access in bounds (the variants run in this process)
MUTANTS = [
    ("e2m1_exponent_bias", "ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    ("e2m1_mantissa_weight", "ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.25 * m, e - 1)"),
    ("e4m3_exponent_bias", "mag = ldexp(1.0 + m / 8.0, e - 7);", "mag = ldexp(1.0 + m / 8.0, e - 8);"),
    ("e4m3_subnormal_exponent", "mag = ldexp(m / 8.0, -6);", "mag = ldexp(m / 8.0, -7);"),
    ("scale_ties_to_odd", "if (amax > thr || (amax == thr && (k & 1)))",
     "if (amax > thr || (amax == thr && !(k & 1)))"),
    ("scale_ties_up", "if (amax > thr || (amax == thr && (k & 1)))", "if (amax >= thr)"),
    ("scale_table_shifted", "orc_e4m3_table[k] = orc_e4m3_value(k);", "orc_e4m3_table[k] = orc_e4m3_value(k + 1);"),
    ("scale_divisor_4", "6.0 * (double)g", "4.0 * (double)g"),
    ("scale_clamps_too_low", "while (k < 126) {", "while (k < 125) {"),
    ("code_ties_to_odd", "if (ax > thr || (ax == thr && (k & 1)))", "if (ax > thr || (ax == thr && !(k & 1)))"),
    ("code_sign_dropped", "int sign = signbit(x) ? 8 : 0;", "int sign = 0;"),
    ("code_divisor_without_scale", "double D = orc_e4m3_value(s) * (double)g;", "double D = (double)g;"),
    ("nibbles_swapped_on_write", "codes8[i] = (uint8_t)(lo | (hi << 4));", "codes8[i] = (uint8_t)(hi | (lo << 4));"),
    ("amax_misses_last", "for (i = 0; i < 16; ++i) {\n    float a", "for (i = 0; i < 15; ++i) {\n    float a"),
    ("dequant_drops_scale", "out128[d] = orc_e2m1_value(code) * orc_e4m3_value(s) * (double)g;",
     "out128[d] = orc_e2m1_value(code) * (double)g;"),
    ("dequant_wrong_nibble", "int code = orc_get_nibble(slab, orc_code_nibble(kind, row, d));",
     "int code = orc_get_nibble(slab, orc_code_nibble(kind, row, d) ^ 1);"),
    ("v_rows_share_a_nibble", "high = (row % 4) >= 2;", "high = 0;"),
    ("put_nibble_clears_neighbour", "*b = (uint8_t)((*b & 0x0F) | (code << 4));", "*b = (uint8_t)(code << 4);"),
    ("dequant_wrong_block", "int s = slab[orc_scale_byte_offset(kind, row, d / 16)];",
     "int s = slab[orc_scale_byte_offset(kind, row, d / 32)];"),
    ("gqa_head_modulo", "int h = qh / group;", "int h = qh % J->num_kv_heads;"),
    ("no_sm_scale", "z[t] = J->sm_scale * dot;", "z[t] = dot;"),
    ("value_row_shifted", "orc_attn_row(J, page, (int)(t % ORC_PAGE), h, 1,",
     "orc_attn_row(J, page, (int)((t + 1) % ORC_PAGE), h, 1,"),
    ("value_uses_key_slab", "orc_attn_row(J, page, (int)(t % ORC_PAGE), h, 1,",
     "orc_attn_row(J, page, (int)(t % ORC_PAGE), h, 0,"),
    ("last_token_dropped", "for (t = 0; t < L; ++t) { /* weights", "for (t = 0; t < L - 1; ++t) { /* weights"),
    ("lse_without_max", "J->lse[(int64_t)b * J->num_q_heads + qh] = m + log(sum);",
     "J->lse[(int64_t)b * J->num_q_heads + qh] = log(sum);"),
    ("key_row_reversed", "orc_attn_row(J, page, (int)(t % ORC_PAGE), h, 0,",
     "orc_attn_row(J, page, (int)(15 - t % ORC_PAGE), h, 0,"),
    ("workspace_row_offset", "int64_t o = ((cu_rows[s] + t) * num_kv_heads + h) * ORC_D;",
     "int64_t o = ((cu_rows[s] + t) * num_kv_heads) * ORC_D;"),
    ("fp8_workspace_sign_dropped", "return (signbit(x) ? 0x80 : 0) | mag;", "return mag;"),
    ("extend_not_causal", "int64_t n_vis = J->prefix_len + i + 1;", "int64_t n_vis = J->prefix_len + J->chunk_len;"),
    ("extend_misses_own_row", "int64_t n_vis = J->prefix_len + i + 1;", "int64_t n_vis = J->prefix_len + i;"),
    ("extend_gqa_head_modulo", "int h = qh / group;\n  int64_t n_vis", "int h = qh % J->num_kv_heads;\n  int64_t n_vis"),
    ("extend_no_sm_scale", "orc_ext_kv(J, 0, t, h, d);\n    z[t] = J->sm_scale * dot;",
     "orc_ext_kv(J, 0, t, h, d);\n    z[t] = dot;"),
    ("extend_value_from_key", "acc[d] += w * orc_ext_kv(J, 1, t, h, d);", "acc[d] += w * orc_ext_kv(J, 0, t, h, d);"),
    ("extend_lse_without_max", "J->lse[i * J->num_q_heads + qh] = m + log(sum);",
     "J->lse[i * J->num_q_heads + qh] = log(sum);"),
    ("extend_bf16_workspace_read_as_fp8", "if (dtype == 1) return", "if (dtype == 3) return"),
    ("extend_chunk_head_ignored", "((t - J->prefix_len) * J->num_kv_heads + h) * ORC_D + d]",
     "((t - J->prefix_len) * J->num_kv_heads) * ORC_D + d]"),
    ("fp8_v_rows_collapsed", "(d % 8) * 4 + row % 4;", "(d % 8) * 4;"),
    ("fp8_code_sign_dropped", "(double)s);\n  return (signbit(x) ? 0x80 : 0) | mag;", "(double)s);\n  return mag;"),
    ("fp8_scale_ignored_on_decode", "orc_fp8_byte_offset(kind, row, d)]) * (double)scale;",
     "orc_fp8_byte_offset(kind, row, d)]);"),
    ("fp8_k_scale_used_for_v", "orc_fp8_code(x, kind ? v_scale : k_scale)", "orc_fp8_code(x, k_scale)"),
    ("fp8_attn_v_scale_for_k", "kind ? J->v_scale : J->k_scale", "J->v_scale"),
    ("fp8_slab_kind_ignored", "((page * num_kv_heads + head) * 2 + kind) * (int64_t)ORC_FP8_SLAB",
     "((page * num_kv_heads + head) * 2) * (int64_t)ORC_FP8_SLAB"),
    ("amax_ignores_sign", "if (fabs(x) > m) m = fabs(x);", "if (x > m) m = x;"),
    ("calibration_stops_before_ties", "while (amax / (6.0 * (g / 2.0)) <= 448.0) g /= 2.0;",
     "while (amax / (6.0 * (g / 2.0)) < 448.0) g /= 2.0;"),
    ("calibration_limit_halved", "while (amax / (6.0 * (g / 2.0)) <= 448.0) g /= 2.0;",
     "while (amax / (6.0 * (g / 2.0)) <= 224.0) g /= 2.0;"),
    ("slab_kind_ignored", "return ((page * num_kv_heads + head) * 2 + kind) * (int64_t)ORC_SLAB;",
     "return ((page * num_kv_heads + head) * 2) * (int64_t)ORC_SLAB;"),
    # non-finite inputs (reading: NaN left out of amax and coded as magnitude 0)
    ("amax_takes_nan", "if (a > amax) amax = a;", "if (!(a <= amax)) amax = a;"),
    ("nan_code_saturates", "double ax = fabs((double)x);", "double ax = isnan(x) ? INFINITY : fabs((double)x);"),
    # any finite global scale g: every threshold and dequantized value exact in double
    ("scale_divisor_rounded_to_float", "orc_e4m3_nearest_of_quotient((double)amax, 6.0 * (double)g)",
     "orc_e4m3_nearest_of_quotient((double)amax, (double)(6.0f * g))"),
    ("code_divisor_rounded_to_float", "double D = orc_e4m3_value(s) * (double)g;",
     "double D = (double)(float)(orc_e4m3_value(s) * (double)g);"),
    ("dequant_product_rounded_to_float", "out128[d] = orc_e2m1_value(code) * orc_e4m3_value(s) * (double)g;",
     "out128[d] = (double)(float)(orc_e2m1_value(code) * orc_e4m3_value(s) * (double)g);"),
    ("bf16_ties_away", "nearbyint(ldexp(a, 8 - e))", "round(ldexp(a, 8 - e))"),
    ("bf16_truncates", "nearbyint(ldexp(a, 8 - e))", "floor(ldexp(a, 8 - e))"),
    ("tight_scale_not_raised", "while (!(amax <= 2688.0 * (double)g)) g = nextafterf(g, INFINITY);", ""),
    ("tight_scale_wrong_limit",
     "g = (float)(amax / 2688.0);\n  while (!(amax <= 2688.0 * (double)g)) g = nextafterf(g, INFINITY);\n"
     "  while (g > 0.0f && amax <= 2688.0 * (double)nextafterf(g, 0.0f))",
     "g = (float)(amax / 2048.0);\n  while (!(amax <= 2048.0 * (double)g)) g = nextafterf(g, INFINITY);\n"
     "  while (g > 0.0f && amax <= 2048.0 * (double)nextafterf(g, 0.0f))"),
]


def _pins(o):
    yield lambda: TF.test_e2m1_closed_form(o)
    yield lambda: TF.test_e4m3_decode_all_bytes_vs_library(o)
    yield lambda: TF.test_worked_example_block_of_ones(o)
    yield lambda: TF.test_scale_byte_saturates(o)
    yield lambda: TF.test_scale_byte_vs_library_rne(o)
    yield lambda: TF.test_e2m1_code_threshold_edges(o)
    yield lambda: TF.test_round_trip_of_representable_blocks(o)
    yield lambda: TF.test_zero_scale_reading(o)
    yield lambda: TF.test_non_finite_reading(o)
    yield lambda: TF.test_fp8_workspace_rounding_vs_library(o)
    yield lambda: TA.test_attention_vs_library_sdpa_on_representable_kv(o, 8, 2, [16, 50, 1])
    yield lambda: TA.test_dequant_workspace_returns_representable_values_exactly(o)
    yield lambda: TA.test_seq_len_one_returns_first_value_row(o)
    yield lambda: TE.test_first_chunk_query_without_prefix_sees_only_itself(o)
    yield lambda: TE.test_constant_keys_give_running_mean_of_values(o)
    yield lambda: TC.test_amax_vs_library(o)
    yield lambda: TC.test_global_scale_closed_forms(o)
    yield lambda: TC.test_tight_global_scale_closed_forms(o)
    yield lambda: TC.test_tight_global_scale_is_the_smallest_binary32_without_saturation(o, 0)
    yield lambda: TF.test_scale_byte_non_power_of_two_global_scale(o)
    yield lambda: TF.test_quantize_block_non_power_of_two_global_scale(o)
    yield lambda: TF.test_dequant_values_are_exact_products_for_any_g(o)
    yield lambda: TF.test_bf16_rounding_of_exact_values(o)
    yield lambda: T8.test_fp8_layout_is_a_bijection(o)
    yield lambda: T8.test_fp8_codes_vs_library_cast(o, 0.5)
    yield lambda: T8.test_fp8_codes_saturate_and_keep_sign(o)
    yield lambda: T8.test_fp8_round_trip_and_attention_vs_library_sdpa(o, 0.5, 2.0)
    for kind in TE.PRE_DTYPES:
        yield lambda kind=kind: TE.test_extend_vs_library_sdpa(o, kind, 37, 19, 8, 2)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    path = oracle.build_variant(src.replace(old, new, 1), str(tmp_path / f"mut_{name}.so"))
    caught = None
    with oracle.use_library(path):
        for i, pin in enumerate(_pins(oracle)):
            try:
                pin()
            except AssertionError:
                caught = i
                break
    assert caught is not None, f"no pin catches mutant {name}"


def test_unmutated_oracle_passes_all_mutation_pins():
    oracle.lib()
    for pin in _pins(oracle):
        pin()


def test_pool_layout_is_a_bijection(oracle_lib):
    for kind in (0, 1):
        codes = {oracle_lib.code_nibble(kind, r, d) for r in range(16) for d in range(128)}
        scales = {oracle_lib.scale_byte_offset(kind, r, j) for r in range(16) for j in range(8)}
        assert codes == set(range(2048)) and scales == set(range(1024, 1152))
    # K rows are token-major (64 contiguous code bytes, low nibble = even channel;
    # 8 contiguous scale bytes per token)
    assert [oracle_lib.code_nibble(0, 3, d) for d in range(128)] == list(range(384, 512))
    assert [oracle_lib.scale_byte_offset(0, 3, j) for j in range(8)] == list(range(1048, 1056))
    # V: 16-byte chunk c = 16 (r // 4) + d // 8 holds channels 8 (c % 16) .. +7 of
    # rows 4 (c // 16) .. +3; a byte holds rows r and r + 2 of one channel
    for c in range(64):
        nib = {oracle_lib.code_nibble(1, 4 * (c // 16) + i, 8 * (c % 16) + e) for i in range(4) for e in range(8)}
        assert nib == set(range(32 * c, 32 * c + 32))
    for r in range(16):
        for d in range(128):
            lo, hi = oracle_lib.code_nibble(1, r, d), oracle_lib.code_nibble(1, r ^ 2, d)
            assert lo // 2 == hi // 2 and (lo % 2) == (r % 4 >= 2)
    # V scales: block-major, 16 rows per block
    assert [oracle_lib.scale_byte_offset(1, r, 5) for r in range(16)] == list(range(1104, 1120))
    assert oracle_lib.slab_offset(2, 1, 1, 8) == ((2 * 8 + 1) * 2 + 1) * 1152
