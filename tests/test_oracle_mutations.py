"""Planted mistakes: each mutant of the oracle must fail at least one pin.

A copy of oracle/q4k_oracle.c gets one plausible mistake (a swapped nibble, a
wrong sub-block index, a flipped sign, a dropped term, transposed scale/min
fields, a wrong exponent bias, ...), is built into a temporary library, and
the checks of oracle_pins.py run against it.  The real oracle is untouched;
the mistakes live only in the temporary copies, on the CPU.
"""
import importlib.util
import os
import shutil
import subprocess

import pytest

import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "q4k_oracle.c")

MUTANTS = {
    "nibble_swap": ("*q = hi ? (byte / 16) : (byte % 16);", "*q = hi ? (byte % 16) : (byte / 16);"),
    "subblock_index": ("*j = 2 * c + hi;", "*j = c + 4 * hi;"),
    "chunk_stride": ("const uint8_t byte = qs[32 * c + i];", "const uint8_t byte = qs[32 * (c % 2) + i];"),
    "min_sign": ("out[e] = prod - dm;", "out[e] = prod + dm;"),
    "min_dropped": ("out[e] = prod - dm;", "out[e] = prod;"),
    "scale_min_transposed": (
        "sc[j] = (uint8_t)(s[j] % 64);\n            m[j] = (uint8_t)(s[j + 4] % 64);",
        "sc[j] = (uint8_t)(s[j + 4] % 64);\n            m[j] = (uint8_t)(s[j] % 64);"),
    "high_bits_from_wrong_byte": ("(s[j - 4] / 64) * 16", "(s[j] / 64) * 16"),
    "six_bit_mask": ("sc[j] = (uint8_t)(s[j] % 64);", "sc[j] = (uint8_t)(s[j] % 32);"),
    "d_dmin_swapped": (
        "const float d = oq_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));\n"
        "    const float dmin = oq_f16_to_f32((uint16_t)(blk[2] | (blk[3] << 8)));",
        "const float d = oq_f16_to_f32((uint16_t)(blk[2] | (blk[3] << 8)));\n"
        "    const float dmin = oq_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));"),
    "big_endian_d": ("oq_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)))", "oq_f16_to_f32((uint16_t)(blk[1] | (blk[0] << 8)))"),
    "exponent_bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "implicit_bit_dropped": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)f, e - 25);"),
    "x_vector_ignored": ("const double xv = (double)xb[c];", "const double xv = (double)x[c];"),
    "bound_without_abs": ("mag += fabs(wv) * fabs(xv);", "mag += wv * xv;"),
    "dot_in_float": ("acc += wv * xv;", "acc = (float)(acc + (float)(wv * xv));"),
    "encoder_truncates": ("double sig = nearbyint(ldexp(fr, 11));", "double sig = floor(ldexp(fr, 11));"),
    "quantizer_min_sign": ("q = oq_clampi(nearbyint(((double)xs[e] + dm) / dsc), 0, 15);",
                           "q = oq_clampi(nearbyint(((double)xs[e] - dm) / dsc), 0, 15);"),
    "q8_truncates": ("(int)rintf(v)", "(int)truncf(v)"),
    "q8_scale_128": ("d[b] = amax / 127.0f;", "d[b] = amax / 128.0f;"),
    "q8_nan_ignored": ("            amax = NAN;\n", "            amax = amax;\n"),
    "q8_block_scale_index": ("(double)d[b * (k / 32) + c / 32]", "(double)d[b * (k / 32) + c / 64]"),
    "q8_codes_of_vector_0": ("(double)q[b * k + c]", "(double)q[c]"),
    "q6_ql_half_stride": ("blk[64 * h + 32 * (t % 2) + l]", "blk[32 * h + 32 * (t % 2) + l]"),
    "q6_ql_nibble_select": ("(t < 2) ? (lo_byte % 16) : (lo_byte / 16)",
                            "(t % 2 == 0) ? (lo_byte % 16) : (lo_byte / 16)"),
    "q6_qh_shift": ("(hi_byte >> (2 * t)) % 4", "(hi_byte >> t) % 4"),
    "q6_qh_byte": ("blk[128 + 32 * h + l]", "blk[128 + h + 2 * l]"),
    "q6_high_bits_weight": ("*q = lo + 16 * hi;", "*q = lo + 32 * hi;"),
    "q6_scale_index": ("*s = e / 16;", "*s = e / 32;"),
    "q6_offset_dropped": ("out[e] = dsc * (float)(q - 32);", "out[e] = dsc * (float)q;"),
    "q6_scale_unsigned": ("(float)(int8_t)blk[192 + s]", "(float)blk[192 + s]"),
    "q6_d_offset": ("oq_f16_to_f32((uint16_t)(blk[208] | (blk[209] << 8)))",
                    "oq_f16_to_f32((uint16_t)(blk[192] | (blk[193] << 8)))"),
    "q6_row_stride_ignored": ("oq6_dequant_superblock(w + r * row_stride + s * OQ6_SB, out",
                              "oq6_dequant_superblock(w + r * S * OQ6_SB + s * OQ6_SB, out"),
    "q6_gemv_x_vector_ignored": ("                    const float* xb = x + b * k;",
                                 "                    const float* xb = x;"),
    "f16_gemm_transposed": ("(double)oq_f16_to_f32(w16[r * k + c])", "(double)oq_f16_to_f32(w16[c * n + r])"),
    "f16_gemm_x_row_0": ("(double)oq_f16_to_f32(x16[b * k + c])", "(double)oq_f16_to_f32(x16[c])"),
    "mirror_drops_lsb": ("out[r * k + c] = oq_f32_to_f16_rne(wrow[c]);",
                         "out[r * k + c] = (uint16_t)(oq_f32_to_f16_rne(wrow[c]) & 0xFFFEu);"),
    "mirror_q6_stride": ("oq6_dequant_superblock(w + r * row_stride + s * OQ6_SB, wrow + s * OQ_QK);\n                    }\n                }\n                for (int64_t c",
                         "oq6_dequant_superblock(w + r * S * OQ6_SB + s * OQ6_SB, wrow + s * OQ_QK);\n                    }\n                }\n                for (int64_t c"),
}


def _load_variant(lib_path, src_path):
    spec = importlib.util.spec_from_file_location("oracle_mutant_%d" % abs(hash(lib_path)),
                                                  os.path.join(ROOT, "oracle", "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._SRC = src_path
    mod._LIB = lib_path
    mod._lib = None
    mod._load()
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor not found: %s" % name
    mutated = text.replace(old, new, 1)
    src = tmp_path / "q4k_oracle.c"
    src.write_text(mutated)
    lib = tmp_path / "liboracle_q4k.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(lib), str(src), "-lm"], check=True)
    mod = _load_variant(str(lib), str(src))
    failed = None
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except AssertionError:
            failed = check.__name__
            break
    assert failed is not None, "mutant %s passed every pin" % name
    shutil.rmtree(tmp_path, ignore_errors=True)
