"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one (so that a passing pin suite means something)."""
import os
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, planted mistake); each original occurs exactly once.
MUTANTS = [
    ("drop_min_term", "acc += main_term - corr_term;", "acc += main_term;"),
    ("min_term_sign", "acc += main_term - corr_term;", "acc += main_term + corr_term;"),
    ("sc_m_swapped", "main_term = (d * sc[j]) * da", "main_term = (d * mn[j]) * da"),
    ("nibble_halves_swapped", "q[64 * p + i] = qs[32 * p + i] & 15;",
     "q[64 * p + i] = qs[32 * p + i] >> 4;"),
    ("subblock_index_off", "(dmin * mn[j]) * da", "(dmin * mn[(j + 1) & 7]) * da"),
    ("high_scale_bits_wrong", "sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);",
     "sc[j] = (s[j + 4] & 15) | ((s[j] >> 6) << 4);"),
    ("ties_to_even", "float r = roundf(xb[i] / da);", "float r = rintf(xb[i] / da);"),
    ("reciprocal_multiply", "float r = roundf(xb[i] / da);",
     "float r = roundf(xb[i] * (1.0f / da));"),
    ("scale_128", "const float da = amax / 127.0f;", "const float da = amax / 128.0f;"),
    ("ssum_high_half_unsigned", "const int ssum = (int16_t)(uint16_t)(word >> 16);",
     "const int ssum = (uint16_t)(word >> 16);"),
    ("f16_truncates", "const double n = rint(a / quantum);",
     "const double n = floor(a / quantum);"),
    ("f16_no_subnormals", "v = ldexp((double)f, -24);", "v = 0.0;"),
    ("dmin_is_d", "*dmin = oracle_f16_to_double(hm);", "*dmin = oracle_f16_to_double(hd);"),
    ("dot_skips_last", "for (int i = 0; i < 32; i++)\n                        D += q4[j * 32 + i] * a[i];",
     "for (int i = 0; i < 31; i++)\n                        D += q4[j * 32 + i] * a[i];"),
    ("q6_offset_dropped", "D += (q6[j * 16 + i] - 32) * a[i];", "D += q6[j * 16 + i] * a[i];"),
    ("q6_dots_offset_dropped", "acc += (q6[j * 16 + i] - 32) * a[i];", "acc += q6[j * 16 + i] * a[i];"),
    ("q6_qh_shift_wrong", "(qh[32 * h + l] >> (2 * g)) & 3", "(qh[32 * h + l] >> g) & 3"),
    ("q6_nibble_choice_wrong", ">> (4 * (g >> 1))) & 15", ">> (4 * (g & 1))) & 15"),
    ("q6_ql_half_wrong", "ql[64 * h + 32 * (g & 1) + l]", "ql[64 * h + 32 * (g >> 1) + l]"),
    ("q6_scale_unsigned", "sc[j] = (int8_t)b[192 + j];", "sc[j] = b[192 + j];"),
    ("q6_da_chunk_wrong", "ds[t * C + b * 8 + j / 2]", "ds[t * C + b * 8 + (j & 7)]"),
    ("q6_scale_per_32", "acc += (d * sc[j]) * da * (double)D;", "acc += (d * sc[j & 14]) * da * (double)D;"),
    ("q6_d_from_block_start", "*d = oracle_f16_to_double((uint16_t)(b[208] | (b[209] << 8)));",
     "*d = oracle_f16_to_double((uint16_t)(b[0] | (b[1] << 8)));"),
    ("q6_group_skips_last", "for (int i = 0; i < 16; i++)\n                        acc += (q6",
     "for (int i = 0; i < 15; i++)\n                        acc += (q6"),
    ("silu_without_up", "h[i] = (float)(gd * (double)u[i] / s);", "h[i] = (float)(gd / s);"),
    ("sigmoid_sign", "const double s = 1.0 + exp(-gd);", "const double s = 1.0 + exp(gd);"),
    ("silu_in_float32", "const double s = 1.0 + exp(-gd);", "const double s = (float)(1.0f + expf((float)-gd));"),
    ("repack_scales_swapped", "sw[2] = (uint8_t)mn[2 * p];\n                sw[3] = (uint8_t)mn[2 * p + 1];",
     "sw[2] = (uint8_t)mn[2 * p + 1];\n                sw[3] = (uint8_t)mn[2 * p];"),
    ("repack_halves_swapped", "memcpy(rec + 320 + 512 * p + 256 * h + 16 * r, blk + 16 + 32 * p + 16 * h, 16);",
     "memcpy(rec + 320 + 512 * p + 256 * (1 - h) + 16 * r, blk + 16 + 32 * p + 16 * h, 16);"),
    ("tiles_h_g_swapped", "const int64_t row = (c * 2 + h) * 2 + g;", "const int64_t row = (c * 2 + g) * 2 + h;"),
    ("tiles_natural_order", "static const int order[8] = {0, 2, 1, 3, 4, 6, 5, 7};",
     "static const int order[8] = {0, 1, 2, 3, 4, 5, 6, 7};"),
    ("tiles_padding_repeats_last", "slot[e] = t < n ? oracle_f32_to_f16((float)q8[t * k + kk]) : 0;",
     "slot[e] = oracle_f32_to_f16((float)q8[(t < n ? t : n - 1) * k + kk]);"),
    ("quantize_gate_not_h", "rc |= oracle_q8_quantize(row, 1, k,", "rc |= oracle_q8_quantize(g + t * k, 1, k,"),
]


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, orig, bad):
    src = open(SRC).read()
    assert src.count(orig) == 1, "mutation anchor for %s not unique" % name
    msrc = tmp_path / "oracle_mut.c"
    msrc.write_text(src.replace(orig, bad))
    so = str(tmp_path / "liboracle_mut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", str(msrc),
                    "-o", so, "-lm"], check=True)
    lib = oracle.load(so)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, "no pin caught planted mistake %s" % name
