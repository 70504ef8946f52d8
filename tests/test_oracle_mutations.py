"""Planted mistakes in the CPU oracle must each trip at least one pin.

Each case copies the oracle's C source, plants one plausible mistake with a
textual substitution (in the encoder and decoder alike where a symmetric
mistake would survive a round trip), builds it with gcc into a temporary
directory, and runs the pins against that build.  Nothing here touches the
HIP library or a GPU.
"""
import os

import pytest

import oracle
import oracle_pins

MUTATIONS = {
    "planes_swapped_both_sides": [
        ("{out + L.off_p0, out + L.off_p1, out + L.off_p2}", "{out + L.off_p1, out + L.off_p0, out + L.off_p2}"),
        ("{in + L.off_p0, in + L.off_p1, in + L.off_p2}", "{in + L.off_p1, in + L.off_p0, in + L.off_p2}"),
    ],
    "plane_bit_order_reversed_both_sides": [
        ("(uint8_t)(1u << (i % 8))", "(uint8_t)(1u << (7 - i % 8))"),
        ("(plane[b][i / 8] >> (i % 8))", "(plane[b][i / 8] >> (7 - i % 8))"),
    ],
    "sign_bit_misplaced": [("sm[i] = (uint8_t)((sign << 7) | mantissa);",
                            "sm[i] = (uint8_t)((sign << 6) | mantissa);")],
    "code_zero_based": [("if (exps[k] == exponent) code = k + 1;", "if (exps[k] == exponent) code = k;")],
    "codes_descending_both_sides": [
        ("if (exps[k] == exponent) code = k + 1;", "if (exps[k] == exponent) code = 7 - k;"),
        ("unsigned exponent = c ? exps[c - 1] : zp[k++];", "unsigned exponent = c ? exps[7 - c] : zp[k++];"),
    ],
    "tie_break_to_larger_exponent": [("if (best < 0 || w[e] > w[best]) best = e;",
                                      "if (best < 0 || w[e] >= w[best]) best = e;")],
    "missing_sqrt2": [("const double s = sigma * sqrt(2.0);", "const double s = sigma;")],
    "octave_off_by_one": [("double lo = ldexp(1.0, e - 127);", "double lo = ldexp(1.0, e - 128);"),
                          ("double hi = ldexp(1.0, e - 126);", "double hi = ldexp(1.0, e - 127);")],
    "dropped_upper_tail_term": [("p[e] = erfc(lo / s) - erfc(hi / s);", "p[e] = erfc(lo / s);")],
    "no_zero_subnormal_bucket": [("p[0] = erf(ldexp(1.0, -126) / s);", "p[0] = 0.0;")],
    "table_counts_after_append": [
        ("        if (i % ZCO_GROUP == 0) put_u32(tab + 4 * (i / ZCO_GROUP), (uint32_t)zp_count);\n", ""),
        ("        if (code == 0) zp[zp_count++] = (uint8_t)exponent;\n",
         "        if (code == 0) zp[zp_count++] = (uint8_t)exponent;\n"
         "        if (i % ZCO_GROUP == 0) put_u32(tab + 4 * (i / ZCO_GROUP), (uint32_t)zp_count);\n"),
    ],
    "zero_point_byte_altered": [("if (code == 0) zp[zp_count++] = (uint8_t)exponent;",
                                 "if (code == 0) zp[zp_count++] = (uint8_t)(exponent ^ 1u);")],
    "mantissa_mask_short": [("unsigned mantissa = v & 0x7Fu;", "unsigned mantissa = v & 0x3Fu;")],
    "sm_section_unaligned": [("L.off_p0 = round_up_128(L.off_sm + n);", "L.off_p0 = L.off_sm + n;")],
    # local reduction of the reduce-scatter path (section 2.D)
    "reduce_local_added_last": [
        ("        for (uint64_t i = 0; i < n; ++i) acc[i] = bf16_to_float(local[i]);\n        first = 0;\n", ""),
        ("    for (uint64_t i = 0; i < n; ++i) out[i] = zco_float_to_bf16(acc[i]);\n",
         "    if (local)\n        for (uint64_t i = 0; i < n; ++i)\n"
         "            acc[i] = first ? bf16_to_float(local[i]) : acc[i] + bf16_to_float(local[i]);\n"
         "    for (uint64_t i = 0; i < n; ++i) out[i] = zco_float_to_bf16(acc[i]);\n"),
    ],
    "reduce_streams_reversed": [("int rc = zco_decode(streams[s], in_bytes[s], n, term);",
                                 "int rc = zco_decode(streams[k - 1 - s], in_bytes[k - 1 - s], n, term);")],
    "reduce_accumulates_from_zero": [
        ("acc[i] = first ? bf16_to_float(term[i]) : acc[i] + bf16_to_float(term[i]);",
         "acc[i] = (first ? 0.0f : acc[i]) + bf16_to_float(term[i]);")],
    "reduce_double_accumulator": [("float *acc = (float *)malloc((n ? n : 1) * sizeof(float));",
                                   "double *acc = (double *)malloc((n ? n : 1) * sizeof(double));")],
    "bf16_ties_away_from_zero": [("if (rest > 0x8000u || (rest == 0x8000u && (lower & 1u))) lower += 1;",
                                  "if (rest >= 0x8000u) lower += 1;")],
    "bf16_truncates": [("if (rest > 0x8000u || (rest == 0x8000u && (lower & 1u))) lower += 1;", "(void)rest;")],
    "bf16_nan_not_canonical": [("    if (isnan(f)) return 0x7FC0u;\n", "")],
    # plan variants (section 2.A): exponent histogram and sigma estimate
    "histogram_shift_off_by_one": [("hist[(x[i] >> 7) & 0xFFu] += 1;", "hist[(x[i] >> 8) & 0xFFu] += 1;")],
    "histogram_plan_unsorted": [("    top7_ascending(w, exps);\n",
                                 "    top7_ascending(w, exps);\n"
                                 "    { uint8_t t = exps[0]; for (int k = 0; k < 6; ++k) exps[k] = exps[k + 1]; exps[6] = t; }\n")],
    "histogram_plan_counts_truncated": [("for (int e = 0; e < 256; ++e) w[e] = (double)hist[e];",
                                         "for (int e = 0; e < 256; ++e) w[e] = (double)(uint32_t)hist[e];")],
    "sigma_counts_nonfinite": [("        if (((x[i] >> 7) & 0xFFu) == 0xFFu) continue;\n", "")],
    "sigma_divides_by_n": [("return m ? sqrt(sum / (double)m) : 0.0;", "return m ? sqrt(sum / (double)n) : 0.0;")],
    "sigma_float_accumulator": [("    double sum = 0.0;\n    uint64_t m = 0;", "    float sum = 0.0f;\n    uint64_t m = 0;")],
    "sigma_no_sqrt": [("return m ? sqrt(sum / (double)m) : 0.0;", "return m ? sum / (double)m : 0.0;")],
    "sigma_abs_not_square": [("        sum += v * v;\n", "        sum += fabs(v);\n")],
    # raw fallback
    "fallback_tie_goes_raw": [("if (*total_bytes > raw_total) {", "if (*total_bytes >= raw_total) {")],
    "fallback_never_taken": [("if (*total_bytes > raw_total) {", "if (0) {")],
    "fallback_mode_byte_not_set": [("        out[31] = ZCO_MODE_RAW;\n", "")],
    "fallback_payload_byte_swapped_both_sides": [
        ("put_u16(out + ZCO_HEADER_BYTES + 2 * i, x[i]);",
         "put_u16(out + ZCO_HEADER_BYTES + 2 * i, (uint16_t)((x[i] >> 8) | (x[i] << 8)));"),
        ("x[i] = get_u16(in + ZCO_HEADER_BYTES + 2 * i);",
         "{ uint16_t w = get_u16(in + ZCO_HEADER_BYTES + 2 * i); x[i] = (uint16_t)((w >> 8) | (w << 8)); }"),
    ],
    "raw_decoder_skips_pad_check": [
        ("        if (!bytes_are_zero(in + 48, ZCO_HEADER_BYTES - 48)) return ZCO_ERR_CORRUPT;\n"
         "        for (uint64_t i = 0; i < n; ++i) x[i] = get_u16",
         "        for (uint64_t i = 0; i < n; ++i) x[i] = get_u16")],
    "raw_decoder_skips_total_check": [("        if (total != ZCO_HEADER_BYTES + 2 * n) return ZCO_ERR_CORRUPT;\n", "")],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(oracle.SOURCE).read()
    for old, new in MUTATIONS[name]:
        assert src.count(old) == 1, "mutation anchor not found: %r" % old
        src = src.replace(old, new)
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(src)
    lib = oracle.compile_source(str(path), str(tmp_path / ("libmut_%s.so" % name)))
    mutant = oracle.Oracle(lib)
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception as exc:  # an assertion, or the mutant rejecting its own output
            failures.append((pin.__name__, type(exc).__name__))
            break
    assert failures, "planted mistake %r passed every pin" % name
    os.remove(lib)
