"""Pin battery for the oracle's quantizer, dequantizer, linear layer and MoE reading.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with something fixed outside it: a value worked by hand from the
definitions, exact rational arithmetic (brute force on tiny inputs), a property the
mathematics guarantees, or an independent library routine. The same battery runs
against planted-mistake builds of the oracle (negative controls), which must fail it.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

from synth import act_bf16, bf16_bits_to_f32, weight_f32

F32 = np.float32

# ---- independent references -----------------------------------------------------------

# E4M3 values from PyTorch's float8_e4m3fn decoding (not from the oracle)
_E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e4m3_rne_exact(r: np.float32) -> int:
    """Nearest non-negative finite E4M3 by exact rational distance; ties to the even code;
    >= 448 saturates to 0x7E."""
    R = Fraction(float(r))
    if R >= 448:
        return 0x7E
    best, bd = None, None
    for c in range(0x7F):
        d = abs(Fraction(float(_E4M3[c])) - R)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best


def e2m1_rne_exact(q: np.float32) -> int:
    sign = 8 if np.signbit(q) else 0
    Q = abs(Fraction(float(q)))
    if Q > 6:
        return sign | 7
    best, bd = None, None
    for c, v in enumerate(_E2M1):
        d = abs(Fraction(v) - Q)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return sign | best


def quantize_bruteforce(w: np.ndarray, per_row: bool):
    """The quantization rule evaluated step by step with numpy float32 scalars (each a
    correctly rounded IEEE operation) and exact-rational rounding to the grids."""
    w = np.asarray(w, dtype=F32)
    rows, K = w.shape
    codes = np.zeros((rows, K // 2), np.uint8)
    scales = np.zeros((rows, K // 16), np.uint8)
    ts_all = []
    if not per_row:
        ts_all = [F32(np.max(np.abs(w))) / F32(2688.0)]
    for r in range(rows):
        ts = F32(np.max(np.abs(w[r]))) / F32(2688.0) if per_row else ts_all[0]
        if per_row:
            ts_all.append(ts)
        for b in range(K // 16):
            blk = w[r, 16 * b:16 * b + 16]
            amax_b = F32(np.max(np.abs(blk)))
            ratio = F32(0.0) if ts == 0 else (amax_b / F32(6.0)) / ts
            s = e4m3_rne_exact(ratio)
            scales[r, b] = s
            den = F32(_E4M3[s]) * ts
            cs = []
            for x in blk:
                q = np.copysign(F32(0.0), x) if den == 0 else F32(x) / den
                cs.append(e2m1_rne_exact(F32(q)))
            for j in range(8):
                codes[r, 8 * b + j] = cs[2 * j] | (cs[2 * j + 1] << 4)
    return codes, scales, np.array(ts_all, dtype=F32)


def dequant_exact(codes, scales, ts, per_row):
    rows, half = codes.shape
    K = 2 * half
    out = []
    for r in range(rows):
        t = Fraction(float(ts[r] if per_row else ts[0]))
        row = []
        for k in range(K):
            byte = int(codes[r, k // 2])
            c = byte & 15 if k % 2 == 0 else byte >> 4
            v = Fraction(_E2M1[c & 7]) * (-1 if c & 8 else 1)
            row.append(v * Fraction(float(_E4M3[scales[r, k // 16]])) * t)
        out.append(row)
    return out


# ---- pins -------------------------------------------------------------------------------

WORKED_W = [1.0, -0.5, 0.25, 0.75, 3.0, 6.0, -6.0, 0.1, -0.1, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 0.0]


def pin_worked_example(o):
    """One row, K = 16, per-tensor. By hand: amax = 6, ts = fp32(6/2688) = 0x3B124925,
    which lies just above 1/448, so ratio = fp32(fp32(6/6)/ts) = 447.99997 rounds to the
    E4M3 value 448 (0x7E) and den = fp32(448 * ts) = 1.0 exactly. Then q = w and the
    E2M1 codes follow from the grid {0,.5,1,1.5,2,3,4,6} with ties to the even code:
    2,9,0,2,5,7,F,0,8,2,4,4,6,6,E,0 (0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2, 2.5->2,
    3.5->4, 5->4, -0.1 -> -0). Packed low nibble first: 92 20 75 0F 28 44 66 0E."""
    codes, scales, ts = o.quantize(np.array([WORKED_W], F32), per_row=False)
    assert int(ts.view(np.uint32)[0]) == 0x3B124925
    assert scales.tolist() == [[0x7E]]
    assert bytes(codes[0]).hex() == "922075" "0f2844660e"
    # with x = all ones the exact product is 13.5 * 448 * ts
    x = np.ones((1, 16), np.float64)
    y, b = o.linear_f64(x, o.dequant(codes, scales, ts, per_row=False))
    want = Fraction(27, 2) * 448 * Fraction(float(ts[0]))
    assert Fraction(float(y[0, 0])) == want


def pin_quantizer_bruteforce(o, seed=7):
    rng = np.random.default_rng(seed)
    cases = []
    for rows, K in ((1, 16), (3, 32), (2, 64)):
        cases.append(rng.normal(0, 0.02, (rows, K)).astype(F32))
        cases.append((rng.standard_cauchy((rows, K)) * 0.1).astype(F32))  # wide dynamic range
    # a block full of E2M1 ties (values c.5 * den for den = 1 after the block max 6)
    cases.append(np.array([[6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25,
                            -1.75, -2.5, -3.5, -5.0, -0.0]], F32))
    # zero blocks, a zero row, tiny and huge magnitudes
    z = np.zeros((2, 32), F32)
    z[1, 16:] = rng.normal(0, 1, 16).astype(F32)
    cases.append(z)
    cases.append(np.array([np.r_[np.full(16, 1e-30), np.full(16, 3e20)]], F32))
    # blocks whose scale ratio lands exactly on an E4M3 tie only when evaluated in the
    # stated order fp32(fp32(amax_b / 6) / ts): with a tensor/row maximum of 1.0, block
    # maxima 0x3F524924, 0x3CF6DB6D and 0x3EC00001 give ratios 368, 13.5 and 168.00002,
    # whereas amax_b / (6 * ts) gives 367.99997, 13.499999 and 168.0 (different scales)
    crafted = np.zeros((1, 64), F32)
    crafted[0, 0] = 1.0
    for blk, bits in ((1, 0x3F524924), (2, 0x3CF6DB6D), (3, 0x3EC00001)):
        crafted[0, 16 * blk + 3] = np.array(bits, np.uint32).view(F32)
        crafted[0, 16 * blk + 7] = -0.5 * crafted[0, 16 * blk + 3]
    cases.append(crafted)
    for w in cases:
        for per_row in (False, True):
            c, s, t = o.quantize(w, per_row)
            c2, s2, t2 = quantize_bruteforce(w, per_row)
            assert np.array_equal(t.view(np.uint32), t2.view(np.uint32)), (w, per_row)
            assert np.array_equal(s, s2), (w, per_row, s, s2)
            assert np.array_equal(c, c2), (w, per_row)


def pin_quantizer_properties(o, seed=11):
    """Properties the rule guarantees: the per-tensor maximum maps to scale 448 (0x7E);
    in every block whose scale is a normal E4M3 value, the largest element's code has
    magnitude 6 (its q lies in [6/1.0625, 6/0.9375]); zero blocks give scale 0 and codes
    +-0; the dequantized value is within half an E2M1 step (times s*ts) of w unless
    |w| exceeds 6*s*ts."""
    w = weight_f32(seed, 64, 256)
    codes, scales, ts = o.quantize(w, per_row=False)
    n, k = np.unravel_index(np.argmax(np.abs(w)), w.shape)
    assert scales[n, k // 16] == 0x7E
    dq = o.dequant(codes, scales, ts, per_row=False)
    for r in range(w.shape[0]):
        for b in range(w.shape[1] // 16):
            blk = w[r, 16 * b:16 * b + 16]
            j = int(np.argmax(np.abs(blk)))
            code = (codes[r, (16 * b + j) // 2] >> (4 * (j % 2))) & 7
            if scales[r, b] >= 0x08:
                assert code == 7, (r, b)
            den = float(_E4M3[scales[r, b]]) * float(ts[0])
            for i in range(16):
                a = abs(float(blk[i])) / den
                step = 0.5 if a < 2 else (1.0 if a < 4 else 2.0)
                if a <= 6:
                    assert abs(dq[r, 16 * b + i] - float(blk[i])) <= 0.5 * step * den * (1 + 1e-6)
    z = np.zeros((3, 48), F32)
    cz, sz, tz = o.quantize(z, per_row=True)
    assert not cz.any() and not sz.any() and not tz.any()
    zneg = -np.zeros((1, 16), F32)
    cn, _, _ = o.quantize(zneg, per_row=False)
    assert set(cn.ravel().tolist()) == {0x88}


def pin_quantizer_refuses_nonfinite(o):
    for bad in (np.nan, np.inf, -np.inf):
        w = np.zeros((1, 32), F32)
        w[0, 5] = bad
        try:
            o.quantize(w, per_row=True)
        except ValueError:
            continue
        raise AssertionError(f"non-finite {bad} accepted")


def pin_dequant_exact(o, seed=13):
    rng = np.random.default_rng(seed)
    rows, K = 3, 48
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (rows, K // 16), dtype=np.uint8)
    ts = np.array([0.00123, 2.5, 1e-3], F32)
    for per_row in (True, False):
        got = o.dequant(codes, scales, ts, per_row)
        want = dequant_exact(codes, scales, ts, per_row)
        for r in range(rows):
            for k in range(K):
                assert Fraction(float(got[r, k])) == want[r][k], (r, k)


def pin_linear_bruteforce(o, seed=17):
    """y must equal the exact rational sum rounded once to float64, within the fp64
    summation error bound K * 2^-53 * sum|terms| (Higham)."""
    rng = np.random.default_rng(seed)
    for M, N, K in ((1, 1, 32), (2, 3, 32), (3, 2, 64), (3, 3, 64)):
        w = rng.normal(0, 0.02, (N, K)).astype(F32)
        codes, scales, ts = o.quantize(w, per_row=False)
        xb = act_bf16(seed + M, M, K)
        y, b = o.linear(xb, codes, scales, ts)
        wq = dequant_exact(codes, scales, ts, per_row=False)
        xf = bf16_bits_to_f32(xb)
        for m in range(M):
            for n in range(N):
                terms = [Fraction(float(xf[m, k])) * wq[n][k] for k in range(K)]
                exact = sum(terms)
                babs = sum(abs(t) for t in terms)
                assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(K, 2 ** 52) * babs
                assert abs(Fraction(float(b[m, n])) - babs) <= Fraction(K, 2 ** 52) * babs


def pin_linear_invariants(o, seed=19):
    M, N, K = 3, 5, 64
    w = weight_f32(seed, N, K)
    codes, scales, ts = o.quantize(w, per_row=False)
    wdq = o.dequant(codes, scales, ts, per_row=False)
    # one-hot rows pick a column of the dequantized weight (ts included)
    for k in (0, 17, 63):
        x = np.zeros((1, K))
        x[0, k] = 1.0
        y, _ = o.linear_f64(x, wdq)
        assert np.array_equal(y[0], wdq[:, k])
        want = np.array([_E2M1[((codes[n, k // 2] >> (4 * (k % 2))) & 7)]
                         * (-1 if (codes[n, k // 2] >> (4 * (k % 2))) & 8 else 1)
                         * float(_E4M3[scales[n, k // 16]]) * float(ts[0]) for n in range(N)])
        assert np.array_equal(y[0], want)
    # a zero scale removes its block
    s0 = scales.copy()
    s0[:, 1] = 0
    xb = act_bf16(seed, M, K)
    y0, _ = o.linear(xb, codes, s0, ts)
    x = o.bf16_to_f64(xb)
    x_cut = x.copy()
    x_cut[:, 16:32] = 0
    y1, _ = o.linear_f64(x_cut, wdq)
    assert np.allclose(y0, y1, rtol=1e-13, atol=1e-300)
    # power-of-two scaling of x is exact; transposed or mis-indexed operands are caught by
    # comparing against numpy's float64 matrix product on a non-square shape
    y, b = o.linear_f64(x, wdq)
    y2, _ = o.linear_f64(2.0 * x, wdq)
    assert np.array_equal(y2, 2.0 * y)
    ref = x @ wdq.T
    assert np.all(np.abs(y - ref) <= 1e-13 * b)
    # permuting whole 16-blocks of x and W together leaves y unchanged up to fp64 order
    perm = np.array([3, 0, 2, 1])
    kidx = np.concatenate([np.arange(16 * p, 16 * p + 16) for p in perm])
    yp, _ = o.linear_f64(x[:, kidx], wdq[:, kidx])
    assert np.all(np.abs(yp - y) <= 1e-13 * b)
    # linearity in x
    xb2 = act_bf16(seed + 1, M, K)
    xa, xc = o.bf16_to_f64(xb), o.bf16_to_f64(xb2)
    ya, ba = o.linear_f64(xa, wdq)
    yc, bc = o.linear_f64(xc, wdq)
    ys, _ = o.linear_f64(xa + xc, wdq)
    assert np.all(np.abs(ys - (ya + yc)) <= 1e-13 * (ba + bc))


def pin_w4a4(o, seed=23):
    """W4A4 = W4A16 on the activation rows replaced by their own dequantized values:
    e2m1 * e4m3 is exact in BF16, and the row's tensor scale is a per-row factor."""
    M, N, K = 3, 4, 64
    w = weight_f32(seed, N, K)
    codes, scales, ts = o.quantize(w, per_row=False)
    xb = act_bf16(seed, M, K)
    xc, xs, xt = o.quantize_bf16(xb, per_row=True)
    y, b = o.linear_w4a4(xc, xs, xt, codes, scales, ts)
    xhat = np.array(dequant_exact(xc, xs, np.ones(M, F32), per_row=True), dtype=np.float64)
    wdq = o.dequant(codes, scales, ts, per_row=False)
    yr, _ = o.linear_f64(xhat, wdq)
    yr = yr * xt.astype(np.float64)[:, None]
    assert np.all(np.abs(y - yr) <= 1e-13 * b)
    # per-row ts is amax_row / 2688 in fp32
    xf = bf16_bits_to_f32(xb)
    for m in range(M):
        assert xt[m] == F32(np.max(np.abs(xf[m]))) / F32(2688.0)


def pin_moe(o, seed=29):
    """Expert-grouped reading: each route's gate_up row equals the dense product with its
    expert; top_k = 1 with router weight 1 reduces the combine to the dense down product
    times ts; permuting tokens permutes outputs; SwiGLU matches g * sigmoid(g) * u."""
    E, T, k, K1, N1, K2, N2 = 4, 3, 2, 32, 32, 16, 48
    gu = [weight_f32(seed, N1, K1, stream=100 + e) for e in range(E)]
    dn = [weight_f32(seed, N2, K2, stream=200 + e) for e in range(E)]
    q_gu = [o.quantize(w, per_row=False) for w in gu]
    q_dn = [o.quantize(w, per_row=False) for w in dn]
    gc = np.stack([q[0] for q in q_gu]); gs = np.stack([q[1] for q in q_gu]); gt = np.concatenate([q[2] for q in q_gu])
    dc = np.stack([q[0] for q in q_dn]); ds = np.stack([q[1] for q in q_dn]); dt = np.concatenate([q[2] for q in q_dn])
    ids = np.array([[2, 0], [1, 3], [3, 2]], np.int32)
    xb = act_bf16(seed, T, K1)
    h, hb = o.moe_gate_up(xb, ids, gc, gs, gt)
    x = o.bf16_to_f64(xb)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            ref = x[t] @ o.dequant(gc[e], gs[e], gt[e:e + 1], per_row=False).T
            assert np.all(np.abs(h[t * k + j] - ref) <= 1e-13 * hb[t * k + j])
    a = o.swiglu(h)
    g, u = h[:, :N1 // 2], h[:, N1 // 2:]
    sig = np.array([[1.0 / (1.0 + math.exp(-v)) for v in row] for row in g])
    assert np.allclose(a, g * sig * u, rtol=1e-14, atol=0)
    assert o.swiglu(np.zeros((1, 4)))[0].tolist() == [0.0, 0.0]
    a_bits = np.array([[o.bf16_round(v) for v in row] for row in a], np.uint16)
    # top_k = 1, r = 1: combine = dense down product
    ids1 = ids[:, :1].copy()
    rw1 = np.ones((T, 1), F32)
    a1 = a_bits[0::k]
    y1, _ = o.moe_down_combine(a1, ids1, rw1, dc, ds, dt)
    for t in range(T):
        e = ids1[t, 0]
        ref, rb = o.linear(a1[t:t + 1], dc[e], ds[e], dt[e:e + 1])
        assert np.all(np.abs(y1[t] - ref[0]) <= 1e-13 * rb[0])
    # weighted combine, and token permutation
    rw = np.array([[0.25, 0.75], [0.5, 0.5], [0.9, 0.1]], F32)
    y, yb = o.moe_down_combine(a_bits, ids, rw, dc, ds, dt)
    ref = np.zeros_like(y)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            r, _ = o.linear(a_bits[t * k + j:t * k + j + 1], dc[e], ds[e], dt[e:e + 1])
            ref[t] += float(rw[t, j]) * r[0]
    assert np.all(np.abs(y - ref) <= 1e-13 * yb)
    perm = [2, 0, 1]
    a_perm = np.concatenate([a_bits[p * k:(p + 1) * k] for p in perm])
    yperm, _ = o.moe_down_combine(a_perm, ids[perm], rw[perm], dc, ds, dt)
    assert np.all(np.abs(yperm - y[perm]) <= 1e-13 * yb[perm])


def pin_bf16_round(o):
    """Rounding a float64 to BF16: agrees with PyTorch's float32 -> bfloat16 conversion on
    values that are float32, and rounds a true midpoint to even."""
    rng = np.random.default_rng(31)
    v = np.concatenate([rng.normal(0, 1, 2000), rng.normal(0, 1e-30, 200), [1.0, -2.5, 0.0]]).astype(F32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([o.bf16_round(float(a)) for a in v], np.uint16)
    assert np.array_equal(got, ref)
    assert o.bf16_round(1.0 + 2.0 ** -8) == 0x3F80       # midpoint -> even (1.0)
    assert o.bf16_round(1.0 + 3 * 2.0 ** -8) == 0x3F82   # midpoint -> even (1 + 2^-6)
    assert o.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81


# silu(g) = g / (1 + e^-g) at fixed points, to 19+ significant digits (the logistic
# function's closed form evaluated in 40-digit decimal arithmetic, not by the oracle)
SILU_FIXED = {
    1.0: 0.7310585786300048792511592418218362743650,
    -1.0: -0.2689414213699951207488407581781637256349,
    0.5: 0.3112296656009272823194502828727542393766,
    -4.0: -0.07194483984836623210717255179815369948994,
    30.0: 29.99999999999719271310934821031384813121,
    -30.0: -2.807286890651789686151868795985495233474e-12,
}


def pin_swiglu(o):
    """SwiGLU a = silu(g) * u with g the first half of a gate_up row and u the second:
    fixed silu values; the identity silu(g) - silu(-g) = g (the logistic function's
    sigma(g) + sigma(-g) = 1); an all-zero up half or gate half gives zeros; the halves
    are not swapped."""
    gs = np.array(list(SILU_FIXED), np.float64)
    h = np.concatenate([gs, np.ones_like(gs)])[None, :]
    a = o.swiglu(h)[0]
    for g, got in zip(gs, a):
        want = SILU_FIXED[float(g)]
        assert abs(got - want) <= 4e-16 * abs(want), (g, got, want)
    # up half scales the result, gate half goes through silu
    u = np.array([2.0, -3.0, 0.25, 8.0, 1.0, -1.0])
    a2 = o.swiglu(np.concatenate([gs, u])[None, :])[0]
    for g, uu, got in zip(gs, u, a2):
        want = SILU_FIXED[float(g)] * uu
        assert abs(got - want) <= 4e-16 * abs(want), (g, uu, got, want)
    # silu(g) - silu(-g) = g
    g = np.linspace(-12.0, 12.0, 97)
    ap = o.swiglu(np.concatenate([g, np.ones_like(g)])[None, :])[0]
    am = o.swiglu(np.concatenate([-g, np.ones_like(g)])[None, :])[0]
    assert np.all(np.abs((ap - am) - g) <= 1e-14 * np.maximum(1.0, np.abs(g)))
    # hand-built gate_up rows: zero up half, zero gate half
    rng = np.random.default_rng(41)
    gate = rng.normal(0, 3, 64)
    z = o.swiglu(np.concatenate([gate, np.zeros(64)])[None, :])[0]
    assert np.all(z == 0.0)
    z = o.swiglu(np.concatenate([np.zeros(64), rng.normal(0, 3, 64)])[None, :])[0]
    assert np.all(z == 0.0)
    # large |g|: silu(g) -> g above, -> 0 below
    a3 = o.swiglu(np.array([[60.0, -60.0, 1.0, 1.0]]))[0]
    assert a3[0] == 60.0 and -1e-24 < a3[1] < 0.0


def pin_bf16_round_array(o):
    """The batch BF16 rounding equals the scalar one (itself pinned against PyTorch and on
    hand-made midpoints by pin_bf16_round) element for element, over normal, tiny, huge,
    signed-zero and exact-midpoint values."""
    rng = np.random.default_rng(43)
    v = np.concatenate([rng.normal(0, 1, 3000), rng.normal(0, 1e-36, 300),
                        rng.normal(0, 1e30, 300), [0.0, -0.0, 1.0 + 2.0 ** -8,
                                                   1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)]])
    got = o.bf16_round_array(v.reshape(-1, 1)).ravel()
    want = np.array([o.bf16_round(float(x)) for x in v], np.uint16)
    assert np.array_equal(got, want)
    assert got[-4] == 0x8000 and got[-3] == 0x3F80 and got[-2] == 0x3F82 and got[-1] == 0xBF80


def pin_moe_combine_rows(o, seed=47):
    """The ordered combine over float64 route rows (the form used for NVFP4 route rows)
    equals, per token, the router-weighted sum of the W4A4 linear of each route's NVFP4
    row with its expert, and reduces to moe_down_combine on BF16 rows."""
    E, T, k, K, N = 3, 4, 2, 32, 24
    qs = [o.quantize(weight_f32(seed, N, K, stream=300 + e), per_row=False) for e in range(E)]
    dc = np.stack([q[0] for q in qs]); ds = np.stack([q[1] for q in qs])
    dt = np.concatenate([q[2] for q in qs])
    ids = np.array([[2, 0], [1, 2], [0, 1], [2, 1]], np.int32)
    rw = np.array([[0.5, 0.25], [1.0, -0.5], [0.125, 2.0], [0.75, 0.75]], F32)
    xb = act_bf16(seed, T * k, K)
    xc, xs, xt = o.quantize_bf16(xb, per_row=True)
    a = o.dequant(xc, xs, xt, per_row=True)
    y, b = o.moe_combine_rows(a, ids, rw, dc, ds, dt)
    for t in range(T):
        ref = np.zeros(N)
        for j in range(k):
            e = ids[t, j]
            r = t * k + j
            yr, _ = o.linear_w4a4(xc[r:r + 1], xs[r:r + 1], xt[r:r + 1], dc[e], ds[e], dt[e:e + 1])
            ref += float(rw[t, j]) * yr[0]
        assert np.all(np.abs(y[t] - ref) <= 1e-13 * b[t]), t
    yb, _ = o.moe_down_combine(xb, ids, rw, dc, ds, dt)
    yc, _ = o.moe_combine_rows(o.bf16_to_f64(xb), ids, rw, dc, ds, dt)
    assert np.array_equal(yb, yc)


ALL_PINS = [pin_worked_example, pin_quantizer_bruteforce, pin_quantizer_properties,
            pin_quantizer_refuses_nonfinite, pin_dequant_exact, pin_linear_bruteforce,
            pin_linear_invariants, pin_w4a4, pin_moe, pin_bf16_round, pin_swiglu,
            pin_bf16_round_array, pin_moe_combine_rows]


def pin_codec_quick(o):
    """Fast codec checks for the planted-mistake runs (the exhaustive forms live in
    test_oracle_codec.py): all 256 E4M3 bytes against PyTorch, all 16 E2M1 codes against
    the bit-field definition, and the hand-worked tie tables."""
    for b in range(256):
        got, ref = o.e4m3_value(b), _E4M3[b]
        assert (np.isnan(got) and np.isnan(ref)) or (got == ref and np.signbit(got) == np.signbit(ref)), b
    for c in range(16):
        e, m = (c >> 1) & 3, c & 1
        v = (m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)) * (-1 if c & 8 else 1)
        assert o.e2m1_value(c) == v and np.signbit(o.e2m1_value(c)) == (c >= 8)
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, -0.1: 8, 7.0: 7, 3e38: 7}
    got = o.e2m1_encode(np.array(list(ties), F32)).tolist()
    assert got == list(ties.values()), got
    e4 = {17.0: 0x58, 19.0: 0x5A, 7.5 * 2 ** -9: 0x08, 1.5 * 2 ** -9: 0x02, 500.0: 0x7E}
    got = o.e4m3_encode(np.array(list(e4), F32)).tolist()
    assert got == list(e4.values()), got


ALL_PINS.insert(0, pin_codec_quick)
