"""Every plausible single mistake planted in a copy of the oracle must fail at least one pin.

Each mutant is a textual edit of iir_oracle.c compiled into a temporary library on the CPU; the real
oracle is never modified. This shows the pins would notice a dropped term, a wrong sign or index,
a transposed operand or a wrong constant in the oracle.
"""
import os

import pytest

import oracle
from tests import oracle_pins

MUTANTS = [
    ("half_sample_mirror_low", "i = -i;", "i = -i - 1;"),
    ("half_sample_mirror_high", "i = 2 * n - 2 - i;", "i = 2 * n - 1 - i;"),
    ("no_vertical_round", "v[i * w + j] = (acc + vround) >> bpc;", "v[i * w + j] = acc >> bpc;"),
    ("no_horizontal_round", "(uint16_t)((acc + 32768) >> 16)", "(uint16_t)(acc >> 16)"),
    ("vertical_shift_fixed_8", "(acc + vround) >> bpc;", "(acc + vround) >> 8;"),
    ("dropped_vertical_tap", "for (int k = 0; k < 5; ++k)\n                acc",
     "for (int k = 0; k < 4; ++k)\n                acc"),
    ("dropped_horizontal_tap",
     "for (int l = 0; l < 5; ++l)\n                acc += (int64_t)g[l] * v[i * w + mirror(j + l - 2, w)];\n            out[i * out_pitch + j] = (uint16_t)",
     "for (int l = 1; l < 5; ++l)\n                acc += (int64_t)g[l] * v[i * w + mirror(j + l - 2, w)];\n            out[i * out_pitch + j] = (uint16_t)"),
    ("vertical_pass_on_columns", "sample(plane, pitch, mirror(i + k - 2, h), j, bpc)",
     "sample(plane, pitch, i, mirror(j + k - 2, w), bpc)"),
    ("horizontal_pass_on_rows", "v[i * w + mirror(j + l - 2, w)];\n            out[i * out_pitch + j] = (uint16_t)",
     "v[mirror(i + l - 2, h) * w + j];\n            out[i * out_pitch + j] = (uint16_t)"),
    ("off_by_one_window", "mirror(j + l - 2, w)];\n            out[i * out_pitch + j] = (uint16_t)", "mirror(j + l - 1, w)];\n            out[i * out_pitch + j] = (uint16_t)"),
    ("truncated_taps", "floor(65536.0 * w[k] / s + 0.5)", "floor(65536.0 * w[k] / s)"),
    ("sigma_two", "exp(-0.5 * (double)(k * k))", "exp(-0.125 * (double)(k * k))"),
    ("sse_abs_not_square", "s += (uint64_t)(d * d);", "s += (uint64_t)(d < 0 ? -d : d);"),
    ("sse_signed_square", "s += (uint64_t)(d * d);", "s += (uint64_t)(d * (d < 0 ? 1 : d));"),
    ("sad_signed", "(uint64_t)(a[n] > b[n] ? a[n] - b[n] : b[n] - a[n])", "(uint64_t)(a[n] - b[n])"),
    ("sad_against_first_frame", "        prev = cur;\n        cur = tmp;",
     "        if (!have_prev) { prev = cur; cur = tmp; }"),
    ("first_frame_has_motion", "has_motion[t] = have_prev;", "has_motion[t] = 1;"),
    ("chroma_floor_size", "wc = (w + 1) / 2, hc = (h + 1) / 2;\n    const int64_t ybytes = (int64_t)w * h * bps, cbytes = (int64_t)wc * hc * bps;\n    const int64_t n",
     "wc = w / 2, hc = h / 2;\n    const int64_t ybytes = (int64_t)w * h * bps, cbytes = (int64_t)wc * hc * bps;\n    const int64_t n"),
    ("ignores_prev_blur", "int have_prev = prev_blur != NULL;", "int have_prev = 0;"),
    ("motion_over_255", "(256.0 * npx[0])", "(255.0 * npx[0])"),
    ("psnr_peak_not_squared", "log10(peak * peak / mse)", "log10(peak / mse)"),
    ("psnr_uses_sse", "10.0 * log10(peak * peak / mse)", "10.0 * log10(peak * peak / (double)sums[1 + c])"),
    ("range_check_off", "if (sample(plane, pitch, i, j, bpc) > maxv)",
     "if (sample(plane, pitch, i, j, bpc) > maxv + 1)"),
    ("moment_not_squared", "s2 += x * x;", "s2 += x;"),
    ("motion2_max", "out[t] = b < a ? b : a;", "out[t] = b > a ? b : a;"),
    ("motion2_previous_frame", "const double b = t + 1 < n ? motion[t + 1] : a;",
     "const double b = t > 0 ? motion[t - 1] : a;"),
    ("apsnr_mean_of_psnr_count", "const double mse = (double)total[c] / ((double)n * npx[c]);",
     "const double mse = (double)total[c] / npx[c];"),
    ("apsnr_peak_not_squared", "const double peak_sq = peak * peak;", "const double peak_sq = peak;"),
    ("mean_motion_skips_first", "m1 += motion[t];", "m1 += t ? motion[t] : motion[1 % n];"),
    ("sample_signed_16", "uint16_t v;\n    memcpy", "int16_t v;\n    memcpy"),
    ("sse_32bit_total", "    uint64_t s = 0;\n    for (int64_t i = 0; i < h; ++i)\n        for (int64_t j = 0; j < w; ++j) {\n            int64_t d",
     "    uint32_t s = 0;\n    for (int64_t i = 0; i < h; ++i)\n        for (int64_t j = 0; j < w; ++j) {\n            int64_t d"),
    ("moments_32bit_squares", "uint64_t s1 = 0, s2 = 0;", "uint64_t s1 = 0; uint32_t s2 = 0;"),
    ("v2_truncating_shift", "return x >= 0 ? x / d : -((-x + d - 1) / d);", "return x / d;"),
    ("v2_cur_minus_prev",
     "(sample(prev, pitch, r, j, bpc) - sample(cur, pitch, r, j, bpc))",
     "(sample(cur, pitch, r, j, bpc) - sample(prev, pitch, r, j, bpc))"),
    ("v2_no_vertical_round", "floor_shift(acc + ((int64_t)1 << (bpc - 1)), bpc)",
     "floor_shift(acc, bpc)"),
    ("v2_no_horizontal_round", "floor_shift(acc + 32768, 16)", "floor_shift(acc, 16)"),
    ("v2_signed_sum", "o[0] += (uint64_t)(f[n] < 0 ? -(int64_t)f[n] : (int64_t)f[n]);",
     "o[0] += (uint64_t)(int64_t)f[n];"),
    ("v2_against_first_frame", "t > 0 ? (const void *)(fy - ybytes) : prev_luma",
     "t > 0 ? ry : prev_luma"),
    ("v2_vertical_mirror_clamped", "const int64_t r = mirror(i + k - 2, h);",
     "const int64_t r = i + k - 2 < 0 ? 0 : (i + k - 2 >= h ? h - 1 : i + k - 2);"),
]


def _run_pins(lib):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except Exception as e:  # an AssertionError, or an error the mutant's bad output raised
            failed.append((pin.__name__, type(e).__name__))
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique in the oracle source"
    mpath = tmp_path / f"{name}.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.OracleLib(oracle.compile_source(str(mpath), str(tmp_path / f"lib{name}.so")))
    failed = _run_pins(lib)
    assert failed, f"mutant {name} passed every pin"
