"""GPU parity of libnvfp4 against the CPU oracle: device decode, quantizer, W4A16 and
W4A4 linear on ragged shapes and on the full workload shapes.

Bar: codes, scales and tensor scales bit-exact; every linear output within
|gpu - oracle| <= 1e-4 * sum_k |x_k w_k| + 1e-6 (the oracle sums in float64)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_linear_amd as nv
import oracle
from gpu_helpers import assert_within, device, quantize_both, to_dev_bf16
from synth import WORKLOADS, act_bf16, weight_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def _say(*a):
    print(*a, flush=True)


# ---- decode ------------------------------------------------------------------------------

def _decode_weight(dev):
    """256 rows (row n uses scale byte n for both of its 16-blocks), K = 32, row codes
    0..15 twice (low nibble first), ts = 1."""
    codes = np.zeros((256, 16), np.uint8)
    for j in range(16):
        codes[:, j] = ((2 * j) % 16) | (((2 * j + 1) % 16) << 4)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 2, axis=1)
    ts = np.ones(1, np.float32)
    return [torch.from_numpy(a).to(dev) for a in (codes, scales, ts)]


@pytest.mark.parametrize("M", [16, 32])  # 16: weight-streaming kernel; 32: tiled MFMA kernel
def test_decode_every_code_and_scale(dev, o, M):
    """One-hot rows pick single weight elements: y[m][n] = e2m1(m % 16) * e4m3(n) exactly,
    for all 16 codes x 256 scale bytes (NaN scale bytes give NaN)."""
    _say(f"decode exhaustive through the M={M} path")
    c, s, t = _decode_weight(dev)
    x = np.zeros((M, 32), np.float32)
    for m in range(M):
        x[m, m] = 1.0
    y = nv.linear(torch.from_numpy(x).to(dev).to(torch.bfloat16), c, s, t).cpu().numpy()
    for m in range(M):
        for n in range(256):
            want = o.e2m1_value(m % 16) * o.e4m3_value(n)
            got = y[m, n]
            if np.isnan(want):
                assert np.isnan(got), (m, n)
            else:
                assert got == np.float32(want), (m, n, got, want)


# ---- quantizer ---------------------------------------------------------------------------

def _edge_tensors():
    rng = np.random.default_rng(5)
    tie = np.array([[6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25,
                     -1.75, -2.5, -3.5, -5.0, -0.0] * 2], np.float32)
    crafted = np.zeros((1, 64), np.float32)
    crafted[0, 0] = 1.0
    for blk, bits in ((1, 0x3F524924), (2, 0x3CF6DB6D), (3, 0x3EC00001)):
        crafted[0, 16 * blk + 3] = np.array(bits, np.uint32).view(np.float32)
        crafted[0, 16 * blk + 7] = -0.5 * crafted[0, 16 * blk + 3]
    zero_rows = np.zeros((3, 96), np.float32)
    zero_rows[1] = rng.normal(0, 1, 96)
    zero_rows[2, :16] = -0.0
    wide = np.r_[np.full(16, 1e-30), np.full(16, 3e20), np.full(16, 1e-40), rng.normal(0, 1, 16)]
    return {
        "tie_block": tie,
        "op_order_ties": crafted,
        "zero_and_negzero_rows": zero_rows,
        "wide_range": wide.astype(np.float32)[None, :],
        "cauchy": (rng.standard_cauchy((5, 160)) * 0.1).astype(np.float32),
        "normal_ragged": rng.normal(0, 0.02, (7, 96)).astype(np.float32),
    }


@pytest.mark.parametrize("name", sorted(_edge_tensors()))
@pytest.mark.parametrize("per_tensor", [False, True])
def test_quantizer_edges_bit_exact(dev, o, name, per_tensor):
    w = _edge_tensors()[name]
    _say(f"quantize {name} {w.shape} per_tensor={per_tensor}")
    quantize_both(o, w, dev, per_tensor=per_tensor)


@pytest.mark.parametrize("M", WORKLOADS["w4a4"]["Ms"] + (3,))
def test_quantizer_bf16_rows_bit_exact(dev, o, M):
    K = WORKLOADS["w4a4"]["K"]
    xb = act_bf16(WORKLOADS["w4a4"]["x_seed_base"] + M, M, K)
    _say(f"quantize bf16 rows M={M} K={K}")
    c, s, t = nv.quantize_act(to_dev_bf16(xb, dev))
    oc, os_, ot = o.quantize_bf16(xb, per_row=True)
    assert np.array_equal(t.cpu().numpy().view(np.uint32), ot.view(np.uint32))
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(c.cpu().numpy(), oc)


@pytest.mark.parametrize("name", ["single_linear", "decode_sweep", "prefill", "w4a4"])
def test_quantizer_weights_bit_exact(dev, o, name):
    cfg = WORKLOADS[name]
    w = weight_f32(cfg["w_seed"], cfg["N"], cfg["K"])
    _say(f"quantize weight {name} {w.shape}")
    quantize_both(o, w, dev, per_tensor=True)


def _decision_point_rows():
    """fp32 rows whose blocks have divisor e4m3(s) * ts == 1 exactly: the row amax 2688
    (block 0) gives ts = 1, and every other block holds a 6, so ratio = 1 and s = 1.0
    (0x38). The other 15 values of such a block are then the quotients q themselves:
    every fp32 within 64 ulps of each E2M1 decision point (0.25, 0.75, 1.25, 1.75, 2.5,
    3.5, 5) and of 6, of both signs, then +-0 and values just above 0."""
    vals = []
    for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0):
        u = np.array([t], np.float32).view(np.uint32)[0]
        vals.append((np.arange(-64, 65, dtype=np.int64) + int(u)).astype(np.uint32).view(np.float32))
    v = np.concatenate(vals)
    v = v[np.abs(v) <= 6.0]
    v = np.concatenate([v, -v, np.array([0.0, -0.0, 1e-30, -1e-30, 2 ** -149, -(2 ** -149)], np.float32)])
    nblk = (len(v) + 14) // 15
    v = np.concatenate([v, np.zeros(nblk * 15 - len(v), np.float32)]).reshape(nblk, 15)
    blocks = np.concatenate([np.full((nblk, 1), 6.0, np.float32), v], axis=1)
    head = np.zeros((1, 16), np.float32)
    head[0, 0] = 2688.0
    flat = np.concatenate([head, blocks]).reshape(-1)
    K = 256
    flat = np.concatenate([flat, np.zeros((-len(flat)) % K, np.float32)])
    rows = flat.reshape(-1, K)
    rows[:, 0] = 2688.0  # each row's amax (per-row ts = 1)
    return np.ascontiguousarray(rows)


@pytest.mark.parametrize("per_tensor", [False, True])
def test_quantizer_every_e2m1_decision_point(dev, o, per_tensor):
    """The device's E2M1 encoding (the hardware FP4 conversion at scale 1.0) against the
    oracle's nearest-value encoder on quotients packed densely around every decision point,
    through nvfp4_quantize_act: codes, scales and ts bit for bit."""
    w = _decision_point_rows()
    _say(f"quantize decision points {w.shape} per_tensor={per_tensor}")
    quantize_both(o, w, dev, per_tensor=per_tensor)


def test_quantizer_flags_nonfinite(dev):
    faults = torch.zeros(1, dtype=torch.int32, device=dev)
    for bad in (np.nan, np.inf):
        w = np.ones((2, 32), np.float32)
        w[1, 7] = bad
        faults.zero_()
        nv.quantize_act(torch.from_numpy(w).to(dev), faults=faults)
        assert int(faults.item()) & nv.FAULT_NONFINITE
        faults.zero_()
        nv.quantize_act(torch.from_numpy(w).to(dev), per_tensor=True, faults=faults)
        assert int(faults.item()) & nv.FAULT_NONFINITE
    faults.zero_()
    nv.quantize_act(torch.ones((2, 32), device=dev), faults=faults)
    assert int(faults.item()) == 0


# ---- linear, ragged shapes ------------------------------------------------------------------

def _linear_case(dev, o, M, N, K, seed, pad_x=0, pad_y=0):
    w = weight_f32(seed, N, K)
    (c, s, t), (oc, os_, ot) = quantize_both(o, w, dev)
    xb = act_bf16(seed + 1000, M, K + pad_x)
    xd = to_dev_bf16(xb, dev)[:, :K]
    out = torch.full((M, N + pad_y), float("nan"), device=dev)[:, :N]
    y = nv.linear(xd, c, s, t, out=out)
    yr, b = o.linear(xb[:, :K], oc, os_, ot)
    return y.cpu().numpy(), yr, b


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 17, 96), (16, 200, 544), (5, 1000, 4128),
                                   (2, 3000, 64), (16, 48, 8192), (12, 777, 4096), (9, 130, 2048)])
def test_linear_stream_ragged(dev, o, M, N, K):
    _say(f"stream linear M={M} N={N} K={K}")
    y, yr, b = _linear_case(dev, o, M, N, K, seed=M * 7 + N)
    assert_within(y, yr, b, f"M={M} N={N} K={K}")


# decode-sweep-sized N with ragged N (the last workgroup's tiles partly or wholly empty),
# ragged K (the last wave's K range shorter than the others; K % 256 != 0 takes the scales
# from memory), 48-row tiles (M=12, 16) and a long K
@pytest.mark.parametrize("M,N,K", [(5, 12300, 4128), (12, 12320, 2048), (1, 12288, 8192),
                                   (16, 12256, 544)])
def test_linear_stream_large_n_ragged(dev, o, M, N, K):
    _say(f"stream linear M={M} N={N} K={K}")
    y, yr, b = _linear_case(dev, o, M, N, K, seed=M * 11 + N)
    assert_within(y, yr, b, f"M={M} N={N} K={K}")


def test_column_subsets_bit_identical(dev, o):
    """Columns of the full decode-sized product equal, bit for bit, the same columns
    computed from a slice of the weight (a different grid and, at M=16, tile width): a
    row's arithmetic does not depend on the workgroup shape."""
    K = 4096
    w = weight_f32(31, 12288, K)
    (c, s, t), _ = quantize_both(o, w, dev)
    for M in (1, 4, 8, 16):
        xd = to_dev_bf16(act_bf16(900 + M, M, K), dev)
        y_all = nv.linear(xd, c, s, t)
        for lo in (0, 4096, 12288 - 1024):
            y_part = nv.linear(xd, c[lo:lo + 1024].contiguous(), s[lo:lo + 1024].contiguous(), t)
            assert torch.equal(y_part, y_all[:, lo:lo + 1024]), (M, lo)


def test_w4a4_large_n(dev, o):
    K, N, M = 4096, 12288, 6
    w = weight_f32(33, N, K)
    (c, s, t), oq = quantize_both(o, w, dev)
    xb = act_bf16(34, M, K)
    xc, xs, xt = nv.quantize_act(to_dev_bf16(xb, dev))
    oc, os_, ot = o.quantize_bf16(xb, per_row=True)
    assert np.array_equal(xc.cpu().numpy(), oc) and np.array_equal(xs.cpu().numpy(), os_)
    y = nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt).cpu().numpy()
    yr, b = o.linear_w4a4(oc, os_, ot, *oq)
    assert_within(y, yr, b, "w4a4 N=12288")


@pytest.mark.parametrize("M,N,K", [(17, 255, 64), (130, 600, 1056), (300, 130, 96), (64, 256, 32),
                                   (40, 300, 512), (90, 770, 768)])
def test_linear_gemm_ragged(dev, o, M, N, K):
    _say(f"gemm linear M={M} N={N} K={K}")
    y, yr, b = _linear_case(dev, o, M, N, K, seed=M * 3 + N)
    assert_within(y, yr, b, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("K", [544, 512])
def test_linear_wide_tiles_ragged(dev, o, K):
    """The 256 x 256-tile GEMM (chosen when it gives every CU a workgroup) on ragged M and
    N, with an odd number of 64-k steps (K = 544: one 2-byte scale load per step) and with
    K = 512 (the scales in 16-byte pieces of four steps); sampled rows, including every row
    of the last, partial row tile."""
    M, N = 600, 86 * 256 - 100
    _say(f"wide-tile gemm M={M} N={N} K={K} (sampled rows)")
    w = weight_f32(71, N, K)
    (c, s, t), oq = quantize_both(o, w, dev)
    xb = act_bf16(72, M, K)
    y = nv.linear(to_dev_bf16(xb, dev), c, s, t)
    rows = np.unique(np.r_[0, 255, 256, 511, np.arange(512, M, 7), M - 1])
    wdq = o.dequant(*oq, per_row=False)
    yr, b = o.linear_f64(o.bf16_to_f64(xb[rows]), wdq)
    assert_within(y[torch.from_numpy(rows).to(dev)].cpu().numpy(), yr, b, "wide ragged rows")
    assert bool(torch.isfinite(y).all())
    # the same tiles with NVFP4 activations (W4A4)
    xc, xs, xt = nv.quantize_act(to_dev_bf16(xb, dev))
    oc, os_, ot = o.quantize_bf16(xb, per_row=True)
    assert np.array_equal(xc.cpu().numpy(), oc) and np.array_equal(xs.cpu().numpy(), os_)
    y4 = nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt)
    yr4, b4 = o.linear_w4a4(oc[rows], os_[rows], ot[rows], *oq)
    assert_within(y4[torch.from_numpy(rows).to(dev)].cpu().numpy(), yr4, b4, "wide ragged w4a4")


def test_linear_wide_persistent_several_tiles(dev, o):
    """With more 256 x 256 tiles than CUs the wide GEMM runs as a persistent pipeline, each
    workgroup taking its XCD's tiles in turn, the next tile's loads issued while the last
    steps of the current one run. Here 6 row blocks (the last one 20 rows) x 128 column
    blocks (the last one ragged) = 768 tiles, three per workgroup on 256 CUs: sampled rows
    and every row of the ragged block against the oracle, the same bits on a second call,
    and the first 64 rows equal to the 64-row kernel's product of those rows alone (one k
    order for every tiling)."""
    M, N, K = 1300, 128 * 256 - 40, 512
    _say(f"wide-tile gemm, several tiles per workgroup, M={M} N={N} K={K} (sampled rows)")
    w = weight_f32(75, N, K)
    (c, s, t), oq = quantize_both(o, w, dev)
    xb = act_bf16(76, M, K)
    xd = to_dev_bf16(xb, dev)
    y = nv.linear(xd, c, s, t)
    rows = np.unique(np.r_[0, 255, 256, 1023, 1024, 1279, np.arange(1280, M), np.arange(3, 1280, 41)])
    wdq = o.dequant(*oq, per_row=False)
    yr, b = o.linear_f64(o.bf16_to_f64(xb[rows]), wdq)
    assert_within(y[torch.from_numpy(rows).to(dev)].cpu().numpy(), yr, b, "persistent wide rows")
    assert torch.equal(nv.linear(xd, c, s, t), y)
    assert torch.equal(nv.linear(xd[:64].contiguous(), c, s, t), y[:64])


def test_linear_wide_tiles_padded_rows(dev, o):
    """The 256 x 256-tile GEMM on ragged M, N and K with an odd number of 64-k steps and
    padded activation and output rows; sampled rows, including every row of the last,
    partial row tile, with BF16 and with NVFP4 activations."""
    M, N, K = 1100, 29 * 512 + 152, 544
    _say(f"wide-tile gemm, padded rows, M={M} N={N} K={K} (sampled rows)")
    w = weight_f32(73, N, K)
    (c, s, t), oq = quantize_both(o, w, dev)
    xb = act_bf16(74, M, K + 24)
    xd = to_dev_bf16(xb, dev)[:, :K]
    out = torch.full((M, N + 8), float("nan"), device=dev)[:, :N]
    y = nv.linear(xd, c, s, t, out=out)
    rows = np.unique(np.r_[0, 127, 128, 1023, np.arange(1024, M), np.arange(5, 1024, 37)])
    wdq = o.dequant(*oq, per_row=False)
    yr, b = o.linear_f64(o.bf16_to_f64(xb[rows, :K]), wdq)
    assert_within(y[torch.from_numpy(rows).to(dev)].cpu().numpy(), yr, b, "wide padded rows")
    assert bool(torch.isfinite(y).all())
    xc, xs, xt = nv.quantize_act(xd.contiguous())
    oc, os_, ot = o.quantize_bf16(np.ascontiguousarray(xb[:, :K]), per_row=True)
    assert np.array_equal(xc.cpu().numpy(), oc) and np.array_equal(xs.cpu().numpy(), os_)
    y4 = nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt)
    yr4, b4 = o.linear_w4a4(oc[rows], os_[rows], ot[rows], *oq)
    assert_within(y4[torch.from_numpy(rows).to(dev)].cpu().numpy(), yr4, b4, "wide padded w4a4")


def _offset_scales(s):
    """A copy of the scales whose base is 2 bytes past a 16-byte boundary (the ABI's
    minimum alignment), so the GEMMs take their per-step scale loads."""
    buf = torch.empty(s.numel() + 16, dtype=torch.uint8, device=s.device)
    v = buf[2:2 + s.numel()].view(s.shape)
    assert v.data_ptr() % 16 == 2
    v.copy_(s)
    return v


@pytest.mark.parametrize("M,N,K", [(40, 300, 512), (600, 86 * 256 - 100, 512), (90, 770, 768)])
def test_gemm_scale_pieces_match_per_step_scales(dev, o, M, N, K):
    """With K a multiple of 256 and 16-byte aligned scale rows, the GEMMs load the weight
    scales in 16-byte pieces of four 64-k steps; with a scale base that is only 2-byte
    aligned they load each step's two bytes. Both read the same scale values, so the outputs
    are the same bits (64-row tiles, 256 x 256 tiles, BF16 and NVFP4 activations), and the
    piece form matches the oracle."""
    _say(f"gemm scale pieces vs per-step scales M={M} N={N} K={K}")
    w = weight_f32(M + N, N, K)
    (c, s, t), oq = quantize_both(o, w, dev)
    xb = act_bf16(M + N + 1, M, K)
    x = to_dev_bf16(xb, dev)
    assert s.data_ptr() % 16 == 0
    y = nv.linear(x, c, s, t)
    assert torch.equal(nv.linear(x, c, _offset_scales(s), t), y)
    rows = np.unique(np.r_[0, M - 1, np.arange(1, M, 13)])
    yr, b = o.linear_f64(o.bf16_to_f64(xb[rows]), o.dequant(*oq, per_row=False))
    assert_within(y[torch.from_numpy(rows).to(dev)].cpu().numpy(), yr, b, "scale pieces")
    xc, xs, xt = nv.quantize_act(x)
    y4 = nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt)
    assert torch.equal(nv.linear(xc, c, _offset_scales(s), t, x_scales=xs, x_ts=xt), y4)


def test_linear_splitk_ragged(dev, o):
    """The K-split GEMM (chosen when 64 x 256 tiles would leave CUs idle) on ragged M and
    N with 36 K steps: the quarters take whole rounds of four steps (12, 12, 12), so the
    last quarter lies wholly past K and reads zeros; padded activation and output rows;
    BF16 and NVFP4 activations, every output."""
    M, N, K = 300, 1000, 2304
    _say(f"split-K gemm M={M} N={N} K={K}")
    y, yr, b = _linear_case(dev, o, M, N, K, seed=91, pad_x=40, pad_y=24)
    assert_within(y, yr, b, "split-K bf16")
    w = weight_f32(92, N, K)
    (c, s, t), oq = quantize_both(o, w, dev)
    xb = act_bf16(93, M, K)
    xc, xs, xt = nv.quantize_act(to_dev_bf16(xb, dev))
    oc, os_, ot = o.quantize_bf16(xb, per_row=True)
    assert np.array_equal(xc.cpu().numpy(), oc) and np.array_equal(xs.cpu().numpy(), os_)
    y4 = nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt)
    yr4, b4 = o.linear_w4a4(oc, os_, ot, *oq)
    assert_within(y4.cpu().numpy(), yr4, b4, "split-K w4a4")
    # five 128-column tiles: not a multiple of the eight XCDs, so the plain tile order
    M, N, K = 200, 600, 1024
    _say(f"split-K gemm M={M} N={N} K={K}")
    y, yr, b = _linear_case(dev, o, M, N, K, seed=94)
    assert_within(y, yr, b, "split-K bf16, five column tiles")


def test_linear_leading_dimensions(dev, o):
    _say("linear with padded x and y rows")
    for M in (4, 40):
        y, yr, b = _linear_case(dev, o, M, 300, 256, seed=11, pad_x=40, pad_y=13)
        assert_within(y, yr, b, f"padded M={M}")


# ---- the workloads at full size --------------------------------------------------------------

def test_single_linear_full(dev, o):
    cfg = WORKLOADS["single_linear"]
    _say("single linear M=1 K=2048 N=2048")
    w = weight_f32(cfg["w_seed"], cfg["N"], cfg["K"])
    (c, s, t), (oc, os_, ot) = quantize_both(o, w, dev)
    xb = act_bf16(cfg["x_seed"], cfg["M"], cfg["K"])
    y = nv.linear(to_dev_bf16(xb, dev), c, s, t).cpu().numpy()
    yr, b = o.linear(xb, oc, os_, ot)
    assert_within(y, yr, b, "single_linear")


@pytest.fixture(scope="module")
def sweep_weight(dev, o):
    cfg = WORKLOADS["decode_sweep"]
    w = weight_f32(cfg["w_seed"], cfg["N"], cfg["K"])
    dq, oq = quantize_both(o, w, dev)
    wdq = o.dequant(*oq, per_row=False)
    return dq, oq, wdq


@pytest.mark.parametrize("M", WORKLOADS["decode_sweep"]["Ms"])
def test_decode_sweep_full(dev, o, sweep_weight, M):
    cfg = WORKLOADS["decode_sweep"]
    _say(f"decode sweep M={M} K={cfg['K']} N={cfg['N']}")
    (c, s, t), _, wdq = sweep_weight
    xb = act_bf16(cfg["x_seed_base"] + M, M, cfg["K"])
    y = nv.linear(to_dev_bf16(xb, dev), c, s, t).cpu().numpy()
    yr, b = o.linear_f64(o.bf16_to_f64(xb), wdq)
    assert_within(y, yr, b, f"decode sweep M={M}")


def test_decode_rows_batch_invariant_and_deterministic(dev, sweep_weight):
    """Row m's bits do not depend on the other rows of the pass, and repeat exactly."""
    cfg = WORKLOADS["decode_sweep"]
    (c, s, t), _, _ = sweep_weight
    xb = act_bf16(cfg["x_seed_base"] + 16, 16, cfg["K"])
    xd = to_dev_bf16(xb, dev)
    y16 = nv.linear(xd, c, s, t)
    for m in (0, 5, 15):
        y1 = nv.linear(xd[m:m + 1], c, s, t)
        assert torch.equal(y1[0], y16[m]), m
    for rows in (4, 8, 12):  # other row-set counts, tile widths and ring depths
        assert torch.equal(nv.linear(xd[:rows], c, s, t), y16[:rows]), rows
    for _ in range(3):
        assert torch.equal(nv.linear(xd, c, s, t), y16)


def test_negative_control_corrupted_scale_is_detected(dev, o, sweep_weight):
    """One flipped scale byte in the GPU's copy of the weight must break parity."""
    cfg = WORKLOADS["decode_sweep"]
    (c, s, t), _, wdq = sweep_weight
    s_bad = s.clone()
    s_bad[123, 45] ^= 0x08  # changes that block's scale by a power of two
    xb = act_bf16(cfg["x_seed_base"] + 4, 4, cfg["K"])
    y = nv.linear(to_dev_bf16(xb, dev), c, s_bad, t).cpu().numpy()
    yr, b = o.linear_f64(o.bf16_to_f64(xb), wdq)
    ok, worst = oracle.within_bound(y, yr, b)
    assert not ok and worst > 1.0
    bad_cols = np.nonzero(np.any(np.abs(y - yr) > 1e-4 * b + 1e-6, axis=0))[0]
    assert bad_cols.tolist() == [123]


@pytest.mark.parametrize("M", [4, 40])  # the streaming kernel, the K-split GEMM
def test_negative_control_flipped_nibble_is_detected(dev, o, sweep_weight, M):
    """One weight code with its exponent bit flipped (a magnitude from {0, 1/2, 1, 3/2}
    swapped with one from {2, 3, 4, 6}) must break parity, in that column only."""
    cfg = WORKLOADS["decode_sweep"]
    (c, s, t), _, wdq = sweep_weight
    xb = act_bf16(cfg["x_seed_base"] + 7, M, cfg["K"])
    xf = o.bf16_to_f64(xb)
    k = int(np.argmax(np.max(np.abs(xf), axis=0)))  # a k where some row has a large |x|
    c_bad = c.clone()
    c_bad[77, k // 2] ^= 0x04 if k % 2 == 0 else 0x40  # low nibble holds the even k
    y = nv.linear(to_dev_bf16(xb, dev), c_bad, s, t).cpu().numpy()
    yr, b = o.linear_f64(xf, wdq)
    ok, _ = oracle.within_bound(y, yr, b)
    assert not ok
    bad_cols = np.nonzero(np.any(np.abs(y - yr) > 1e-4 * b + 1e-6, axis=0))[0]
    assert bad_cols.tolist() == [77]


def test_prefill_full_sampled_rows(dev, o):
    cfg = WORKLOADS["prefill"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    _say(f"prefill M={M} K={K} N={N} (64 sampled rows vs oracle)")
    w = weight_f32(cfg["w_seed"], N, K)
    (c, s, t), oq = quantize_both(o, w, dev)
    xb = act_bf16(cfg["x_seed"], M, K)
    y = nv.linear(to_dev_bf16(xb, dev), c, s, t)
    rows = np.unique(np.r_[0, 1, 127, 128, 1023, 2047, np.random.default_rng(1).choice(M, 58, replace=False)])
    wdq = o.dequant(*oq, per_row=False)
    yr, b = o.linear_f64(o.bf16_to_f64(xb[rows]), wdq)
    assert_within(y[torch.from_numpy(rows).to(dev)].cpu().numpy(), yr, b, "prefill rows")
    # rows do not depend on M while the kernel keeps the same k order: M = 320 runs the
    # 64 x 256 tiles, M = 2048 the 256 x 256 tiles
    y_small = nv.linear(to_dev_bf16(xb[:320], dev), c, s, t)
    assert torch.equal(y_small, y[:320])
    assert bool(torch.isfinite(y).all())
    # M = 130 runs the K-split kernel (K summed in quarters): within the bound, and
    # identical from run to run
    y_k = nv.linear(to_dev_bf16(xb[:130], dev), c, s, t)
    kr = np.array([0, 1, 63, 64, 127, 128, 129])
    yr_k, b_k = o.linear_f64(o.bf16_to_f64(xb[kr]), wdq)
    assert_within(y_k[torch.from_numpy(kr).to(dev)].cpu().numpy(), yr_k, b_k, "prefill rows, K split")
    assert torch.equal(y_k, nv.linear(to_dev_bf16(xb[:130], dev), c, s, t))


@pytest.mark.parametrize("M", WORKLOADS["w4a4"]["Ms"])
def test_w4a4_full(dev, o, M):
    cfg = WORKLOADS["w4a4"]
    K, N = cfg["K"], cfg["N"]
    _say(f"w4a4 M={M} K={K} N={N}")
    w = weight_f32(cfg["w_seed"], N, K)
    (c, s, t), oq = quantize_both(o, w, dev)
    xb = act_bf16(cfg["x_seed_base"] + M, M, K)
    xc, xs, xt = nv.quantize_act(to_dev_bf16(xb, dev))
    oc, os_, ot = o.quantize_bf16(xb, per_row=True)
    assert np.array_equal(xc.cpu().numpy(), oc) and np.array_equal(xs.cpu().numpy(), os_)
    assert np.array_equal(xt.cpu().numpy().view(np.uint32), ot.view(np.uint32))
    y = nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt).cpu().numpy()
    rows = np.arange(M) if M <= 64 else np.unique(np.r_[0, M - 1, np.random.default_rng(2).choice(M, 62, replace=False)])
    yr, b = o.linear_w4a4(oc[rows], os_[rows], ot[rows], *oq)
    assert_within(y[rows], yr, b, f"w4a4 M={M}")


def test_w4a4_equals_w4a16_on_decoded_rows(dev, o):
    """W4A4 = ts_a[m] * (W4A16 with x' = e2m1 * e4m3 of the activation codes, exact in
    BF16), bit for bit through the same kernel."""
    cfg = WORKLOADS["w4a4"]
    K, N = cfg["K"], cfg["N"]
    w = weight_f32(cfg["w_seed"], N, K)
    (c, s, t), _ = quantize_both(o, w, dev)
    xb = act_bf16(77, 4, K)
    xc, xs, xt = nv.quantize_act(to_dev_bf16(xb, dev))
    y4 = nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt)
    xhat = o.dequant(xc.cpu().numpy(), xs.cpu().numpy(), np.ones(4, np.float32), per_row=True)
    y16 = nv.linear(torch.from_numpy(xhat.astype(np.float32)).to(dev).to(torch.bfloat16), c, s, t)
    want = y16 / t * (xt[:, None] * t)
    assert torch.allclose(y4, want, rtol=1e-6, atol=1e-30)


def test_read_probe_reads_every_byte(dev):
    """The measurement probe's loads cover the buffer: a fold mark placed at the start of
    one thread's run (and nowhere else) reaches the sink, a zero buffer leaves it alone."""
    mark = 0x9E3779B9
    for u in (1, 2, 4, 8, 16):
        nbytes = 3 * u * 4096 + 4096 + 32  # ragged last workgroup
        for where in (0, nbytes - 16 - (nbytes - 16) % (u * 4096)):  # first / last workgroup
            buf = torch.zeros((nbytes,), dtype=torch.uint8, device=dev)
            sink = torch.zeros((1,), dtype=torch.int32, device=dev)
            nv.read_probe(buf, u, sink)
            torch.cuda.synchronize()
            assert sink.item() == 0
            buf.view(torch.int32)[where // 4] = int(np.array(mark, dtype=np.uint32).view(np.int32))
            nv.read_probe(buf, u, sink)
            torch.cuda.synchronize()
            assert sink.cpu().view(torch.int32).numpy().view(np.uint32)[0] == mark, (u, where)


def _in_call(xd, c, s, t):
    """W4A4 with in-call quantization, one row per call (the form takes one row)."""
    return torch.cat([nv.linear(xd[m:m + 1], c, s, t, quantize_x=True) for m in range(xd.shape[0])])


# W4A4 with the activation quantization inside the call (one row per call)
@pytest.mark.parametrize("M,N,K,pad", [(1, 4096, 4096, 0), (4, 4096, 4096, 0), (3, 1000, 4128, 24),
                                       (4, 777, 544, 8), (2, 12288, 8192, 0), (4, 64, 32, 0)])
def test_w4a4_in_call_quantization(dev, o, M, N, K, pad):
    """Each row bit for bit the two-call W4A4 (quantize_act, then the NVFP4-activation
    linear, on all M rows at once), and within the bound of the oracle's W4A4 on the
    oracle's own quantization."""
    _say(f"w4a4 in-call quantization M={M} N={N} K={K}")
    w = weight_f32(40 + M, N, K)
    (c, s, t), oq = quantize_both(o, w, dev)
    xb = act_bf16(41 + M, M, K + pad)
    xd = to_dev_bf16(xb, dev)[:, :K]
    y = _in_call(xd, c, s, t)
    xc, xs, xt = nv.quantize_act(xd)
    y2 = nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt)
    assert torch.equal(y, y2)
    oc, os_, ot = o.quantize_bf16(np.ascontiguousarray(xb[:, :K]), per_row=True)
    yr, b = o.linear_w4a4(oc, os_, ot, *oq)
    assert_within(y.cpu().numpy(), yr, b, f"w4a4 in-call M={M} N={N} K={K}")


def test_w4a4_in_call_quantization_ties(dev, o):
    """Rows whose quotients land exactly on every E2M1 decision point (the hand-checked
    block: amax 6 gives a scale of 448 and a denominator of exactly 1), on E2M1 values,
    and just beside them: bit for bit the two-call result."""
    K, N = 1024, 256
    w = weight_f32(47, N, K)
    (c, s, t), _ = quantize_both(o, w, dev)
    blk = np.array([1, -0.5, 0.25, 0.75, 3, 6, -6, 0.1, -0.1, 1.25, 1.75, 2.5, 3.5, 5, -5, 0],
                   np.float32)
    rows = np.tile(blk, (4, K // 16))
    rows[1] *= np.float32(1.0 + 2.0 ** -7)  # one BF16 step above each point
    rows[2] *= np.float32(1.0 - 2.0 ** -8)  # one BF16 step below
    rows[3, ::5] = 0.0
    xd = torch.from_numpy(rows).to(dev).to(torch.bfloat16)
    y = _in_call(xd, c, s, t)
    xc, xs, xt = nv.quantize_act(xd)
    assert torch.equal(y, nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt))


def test_w4a4_in_call_quantization_nonfinite_row(dev, o):
    """A NaN or Inf activation makes its row's outputs NaN; the other rows' calls are unaffected."""
    M, N, K = 4, 512, 1024
    w = weight_f32(45, N, K)
    (c, s, t), _ = quantize_both(o, w, dev)
    xd = to_dev_bf16(act_bf16(46, M, K), dev)
    ref = _in_call(xd, c, s, t).clone()
    for bad in (float("nan"), float("inf")):
        xbad = xd.clone()
        xbad[1, 77] = bad
        y = _in_call(xbad, c, s, t)
        assert torch.isnan(y[1]).all()
        for m in (0, 2, 3):
            assert torch.equal(y[m], ref[m])
