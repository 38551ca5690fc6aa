"""Pins of the oracle's E2M1 / E4M3 codec against sources other than itself.

* E2M1 decode: the bit-field definition of the OCP MX v1.0 E2M1 element (1 sign bit,
  2 exponent bits with bias 1, 1 mantissa bit; exponent 0 is subnormal).
* E4M3 decode: PyTorch's float8_e4m3fn dtype (the OCP E4M3FN encoding) on all 256 bytes.
* E4M3 encode: PyTorch's round-to-nearest-even float32 -> float8_e4m3fn conversion on
  every float32 in [0, 448]; above 448 the oracle saturates (the library reading) where
  PyTorch produces NaN.
* E2M1 encode: an independent round-half-even formulation with numpy.rint per binade,
  on every float32 near each rounding threshold and a strided sweep of [0, 8], both
  signs, plus the far range (saturation).
* Tie tables worked by hand, idempotence, and exactness of every code*scale product in
  BF16 (which the GPU decode relies on).

The format itself is the one the FP4-Local checkpoints carry (bloomery issue #565,
section 4 "Round 1", PRs #489/#490: U8 code bytes, F8_E4M3 scales, one tensor scale).
"""
import numpy as np
import pytest
import torch

from synth import bf16_bits_to_f32, f32_to_bf16_bits


def e2m1_from_bits(c: int) -> float:
    s = -1.0 if c & 8 else 1.0
    e = (c >> 1) & 3
    m = c & 1
    if e == 0:
        return s * m * 0.5  # subnormal: m * 2^(1-bias) * 2^-1
    return s * 2.0 ** (e - 1) * (1.0 + m / 2.0)


def test_e2m1_decode_bitfield(orc):
    for c in range(16):
        got = orc.e2m1_value(c)
        want = e2m1_from_bits(c)
        assert got == want and np.signbit(got) == np.signbit(want), (c, got, want)


def test_e4m3_decode_all_bytes_vs_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        got = orc.e4m3_value(b)
        if np.isnan(ref[b]):
            assert np.isnan(got), b
        else:
            assert got == ref[b] and np.signbit(got) == np.signbit(ref[b]), (b, got, ref[b])
    # spot values of the encoding
    assert orc.e4m3_value(0x01) == 2.0 ** -9
    assert orc.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert orc.e4m3_value(0x08) == 2.0 ** -6
    assert orc.e4m3_value(0x38) == 1.0
    assert orc.e4m3_value(0x7E) == 448.0
    assert np.isnan(orc.e4m3_value(0x7F)) and np.isnan(orc.e4m3_value(0xFF))
    z = orc.e4m3_value(0x80)
    assert z == 0.0 and np.signbit(z)


def _f32_range(lo_bits: int, hi_bits: int, chunk: int = 1 << 21):
    for a in range(lo_bits, hi_bits, chunk):
        b = min(hi_bits, a + chunk)
        yield np.arange(a, b, dtype=np.uint32).view(np.float32)


@pytest.mark.slow
def test_e4m3_encode_every_float_in_range_vs_torch(orc):
    hi = int(np.array(448.0, np.float32).view(np.uint32)) + 1
    n = 0
    for v in _f32_range(0, hi):
        got = orc.e4m3_encode(v)
        want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int16)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (v[bad[:5]], got[bad[:5]], want[bad[:5]])
        n += v.size
    assert n == hi


def test_e4m3_encode_saturation_and_refusals(orc):
    above = np.array([448.0, 448.00003, 463.9, 464.0, 464.1, 479.0, 480.0, 1e6, 3.0e38], np.float32)
    assert np.all(orc.e4m3_encode(above) == 0x7E)
    bad = np.array([-1.0, -1e-30, np.nan, np.inf], np.float32)
    assert np.all(orc.e4m3_encode(bad) == -1)
    assert orc.e4m3_encode(np.array([-0.0], np.float32))[0] == 0


def e2m1_encode_rint(q: np.ndarray) -> np.ndarray:
    """Independent RNE: round |q| on the grid of its binade with numpy.rint (half to even),
    then map the value to its code. Grid step 0.5 on [0,2), 1 on [2,4), 2 on [4,inf) with
    a cap at 6."""
    a = np.abs(q.astype(np.float64))
    v = np.where(a < 2.0, np.rint(a * 2.0) / 2.0,
                 np.where(a < 4.0, np.rint(a), np.minimum(2.0 * np.rint(a / 2.0), 6.0)))
    lut = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    code = np.zeros(q.shape, dtype=np.int8)
    for val, c in lut.items():
        code[v == val] = c
    return (code | np.where(np.signbit(q), 8, 0)).astype(np.int8)


def test_e2m1_encode_dense_near_thresholds_and_strided(orc):
    """Every float32 within 2^17 ulps of each rounding threshold (0.25, 0.75, 1.25, 1.75,
    2.5, 3.5, 5, 6), plus every 7th float32 in [0, 8], both signs."""
    pts = []
    for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0):
        tb = int(np.array(t, np.float32).view(np.uint32))
        pts.append(np.arange(tb - (1 << 17), tb + (1 << 17), dtype=np.uint32))
    hi = int(np.array(8.0, np.float32).view(np.uint32)) + 1
    step = 7 << 20
    for a in range(0, hi, step):
        pts.append(np.arange(a, min(hi, a + step), 7, dtype=np.uint32))
    for chunk in pts:
        v = chunk.view(np.float32)
        for sgn in (1.0, -1.0):
            w = (v * np.float32(sgn)).astype(np.float32)
            got = orc.e2m1_encode(w)
            want = e2m1_encode_rint(w)
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (w[bad[:5]], got[bad[:5]], want[bad[:5]])
    big = np.array([8.0, 100.0, 3e38, -9.0, -3e38], np.float32)
    assert list(orc.e2m1_encode(big)) == [7, 7, 7, 15, 15]
    assert list(orc.e2m1_encode(np.array([np.nan, np.inf, -np.inf], np.float32))) == [-1, -1, -1]


def test_tie_tables(orc):
    # E2M1 ties (exact midpoints) go to the even code
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for q, c in ties.items():
        assert orc.e2m1_encode(np.array([q], np.float32))[0] == c, q
        assert orc.e2m1_encode(np.array([-q], np.float32))[0] == (c | 8), -q
    # negative values that round to zero keep the sign
    assert orc.e2m1_encode(np.array([-0.1, -0.0, -0.25], np.float32)).tolist() == [8, 8, 8]
    # E4M3 ties: 17 between 16 (0x58) and 18 (0x59); 19 between 18 and 20 (0x5A);
    # 7.5*2^-9 between 7*2^-9 (0x07) and 2^-6 (0x08); 0.5*2^-9 between 0 and 2^-9
    e4 = {17.0: 0x58, 19.0: 0x5A, 7.5 * 2 ** -9: 0x08, 0.5 * 2 ** -9: 0x00,
          1.5 * 2 ** -9: 0x02, 1.0625: 0x38, 1.1875: 0x3A, 432.0: 0x7E, 400.0: 0x7C}
    for r, c in e4.items():
        assert orc.e4m3_encode(np.array([r], np.float32))[0] == c, (r, c)


def test_encode_decode_idempotent(orc):
    for c in range(16):
        v = orc.e2m1_value(c)
        assert orc.e2m1_encode(np.array([v], np.float32))[0] == c
    for b in range(0x7F):
        v = orc.e4m3_value(b)
        assert orc.e4m3_encode(np.array([v], np.float32))[0] == b


def test_every_code_times_scale_is_exact_in_bf16(orc):
    """e2m1(c) * e4m3(s) has at most 2 + 4 significant bits and lies in [2^-10, 2688], so
    it is a BF16 value: rounding it to BF16 and back must give it unchanged."""
    n = 0
    for b in range(256):
        s = orc.e4m3_value(b)
        if np.isnan(s):
            continue
        for c in range(16):
            p = np.float32(orc.e2m1_value(c) * s)
            assert float(p) == orc.e2m1_value(c) * s  # exact in fp32
            rt = bf16_bits_to_f32(f32_to_bf16_bits(np.array([p], np.float32)))[0]
            assert rt == p and np.signbit(rt) == np.signbit(p), (b, c)
            n += 1
    assert n == 16 * 254
