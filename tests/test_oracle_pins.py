"""Runs the oracle pin battery (tests/oracle_pins.py) and shows that it has teeth: each
planted mistake — a plausible slip in the oracle's C source, applied to a copy on the
CPU — must make at least one pin fail."""
import os

import numpy as np
import pytest

import oracle
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


# (text in nvfp4_oracle.c, planted replacement)
MUTANTS = {
    "e2m1_ties_to_odd": ("(c % 2) == 0 && (best % 2) != 0", "(c % 2) != 0 && (best % 2) == 0"),
    "e2m1_ties_down": ("(d == bestd && (c % 2) == 0 && (best % 2) != 0)", "(0)"),
    "e2m1_no_saturation": ("if (a > 6.0) return sign | 7;", ""),
    "e2m1_sign_by_compare": ("int sign = signbit(q) ? 8 : 0;", "int sign = (q < 0) ? 8 : 0;"),
    "e2m1_value_unsigned": ("return (code & 8) ? -m : m;", "return m;"),
    "e4m3_ties_up": ("return (lo % 2 == 0) ? lo : hi;", "return hi;"),
    "e4m3_saturate_to_nan": ("if (v >= 448.0) return 0x7E;", "if (v >= 448.0) return 0x7F;"),
    "e4m3_subnormal_exp": ("(f / 8.0) * ldexp(1.0, -6)", "(f / 8.0) * ldexp(1.0, -7)"),
    "e4m3_bias": ("ldexp(1.0, e - 7)", "ldexp(1.0, e - 8)"),
    "pack_high_nibble_first": ("c[2 * j] | (c[2 * j + 1] << 4)", "c[2 * j + 1] | (c[2 * j] << 4)"),
    "dequant_high_nibble_first": ("(k % 2 == 0) ? (byte & 15) : (byte >> 4)", "(k % 2 == 0) ? (byte >> 4) : (byte & 15)"),
    "dequant_drops_ts": ("oracle_e2m1_value(code) * s * t;", "oracle_e2m1_value(code) * s;"),
    "dequant_scale_index": ("scales[r * (K / 16) + k / 16]", "scales[r * (K / 16) + k / 32]"),
    "ratio_op_order": ("(amax_b / 6.0f) / t", "amax_b / (6.0f * t)"),
    "ratio_divisor": ("(amax_b / 6.0f) / t", "(amax_b / 4.0f) / t"),
    "ts_divisor": ("ts[0] = amax / 2688.0f;", "ts[0] = amax / 448.0f;"),
    "row_amax_half_row": ("for (int64_t k = 0; k < K; k++) amax = fmaxf(amax, fabsf(wr[k]));",
                          "for (int64_t k = 0; k < K / 2; k++) amax = fmaxf(amax, fabsf(wr[k]));"),
    "den_uses_ratio": ("float den = sd * t;", "float den = ratio * t;"),
    "linear_drops_last_term": ("for (int64_t k = 0; k < K; k++) {\n        double p",
                               "for (int64_t k = 0; k < K - 1; k++) {\n        double p"),
    "bf16_round_ties_away": ("(rem == 0.5 && fmod(fl, 2.0) != 0.0)", "(rem == 0.5)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "nvfp4_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutant anchor for {name} not found"
    mut_src = tmp_path / "mutant.c"
    mut_src.write_text(src.replace(old, new, 1))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build_lib(src=str(mut_src), out=lib_path)
    o = oracle.Oracle(oracle.load(lib_path))
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(o)
        except Exception:  # any failure of a pin counts as caught
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every pin"


# planted mistakes in the SwiGLU reading (Python), each of which must fail pin_swiglu
SWIGLU_MUTANTS = {
    "sigmoid_without_g": lambda h: (lambda g, u: 1.0 / (1.0 + np.exp(-g)) * u)(*np.split(h, 2, axis=1)),
    "exp_sign_flipped": lambda h: (lambda g, u: g / (1.0 + np.exp(g)) * u)(*np.split(h, 2, axis=1)),
    "halves_swapped": lambda h: (lambda u, g: g / (1.0 + np.exp(-g)) * u)(*np.split(h, 2, axis=1)),
    "gelu_tanh_instead": lambda h: (lambda g, u: 0.5 * g * (1 + np.tanh(0.7978845608 * (g + 0.044715 * g ** 3))) * u)(*np.split(h, 2, axis=1)),
    "fp32_arithmetic": lambda h: (lambda g, u: (g.astype(np.float32) / (1 + np.exp(-g.astype(np.float32))) * u.astype(np.float32)).astype(np.float64))(*np.split(np.asarray(h, np.float64), 2, axis=1)),
}


@pytest.mark.parametrize("name", sorted(SWIGLU_MUTANTS))
def test_planted_swiglu_mistake_is_caught(orc, name):
    o = oracle.Oracle(orc.lib)
    o.swiglu = SWIGLU_MUTANTS[name]
    with pytest.raises(AssertionError):
        P.pin_swiglu(o)
