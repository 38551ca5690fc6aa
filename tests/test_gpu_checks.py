"""GPU tests of the linear calls' check mode (NVFP4_F_CHECK) and of the K-split GEMM's
alignment fallback.

Check mode scans the operands before the product: an E4M3 NaN scale byte (0x7F / 0xFF)
or a non-finite tensor scale sets NVFP4_FAULT_NAN_SCALE, a non-finite BF16 activation
sets NVFP4_FAULT_NONFINITE (the pages' engine refuses NaN scale bytes and values that
overflow once scaled: bloomery issue #565, section 10, PRs #597 and #710). Without the
flag nothing is scanned and nothing is reported, and the outputs are the same bits."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_linear_amd as nv
import oracle
from gpu_helpers import assert_within, device, quantize_both, to_dev_bf16
from synth import act_bf16, moe_routes, weight_f32

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def _word(dev):
    return torch.zeros(1, dtype=torch.int32, device=dev)


@pytest.mark.parametrize("M", [1, 8, 40])  # streaming kernel (one and two row sets), GEMM
def test_check_mode_nan_scale_byte(dev, o, M):
    N, K = 96, 512
    _say(f"check mode: NaN scale byte, M={M}")
    (c, s, t), oq = quantize_both(o, weight_f32(301, N, K), dev)
    xb = act_bf16(302, M, K)
    x = to_dev_bf16(xb, dev)
    # clean data: no fault with the flag, and the same bits as without it
    f = _word(dev)
    y_chk = nv.linear(x, c, s, t, check=True, faults=f)
    y = nv.linear(x, c, s, t)
    assert int(f.item()) == 0
    assert torch.equal(y, y_chk)
    yr, b = o.linear(xb, *oq)
    assert_within(y.cpu().numpy(), yr, b, "check-mode clean")
    for bad in (0x7F, 0xFF):
        s_bad = s.clone()
        s_bad[N - 1, K // 16 - 1] = bad
        f_off = _word(dev)
        nv.linear(x, c, s_bad, t, faults=f_off)  # no flag: nothing scanned
        assert int(f_off.item()) == 0
        f_on = _word(dev)
        y_bad = nv.linear(x, c, s_bad, t, check=True, faults=f_on)
        assert int(f_on.item()) == nv.FAULT_NAN_SCALE, hex(int(f_on.item()))
        # the product still ran: the NaN reaches that column only
        yb = y_bad.cpu().numpy()
        assert np.all(np.isnan(yb[:, N - 1]))
        assert np.array_equal(yb[:, :N - 1], y.cpu().numpy()[:, :N - 1])
    # the largest finite scale bytes are not faults
    s_max = s.clone()
    s_max[0, 0] = 0x7E
    s_max[1, 1] = 0xFE
    f = _word(dev)
    nv.linear(x, c, s_max, t, check=True, faults=f)
    assert int(f.item()) == 0


def test_check_mode_tensor_scale_and_activations(dev, o):
    N, K, M = 64, 256, 4
    _say("check mode: tensor scale, BF16 activations, NVFP4 activations")
    (c, s, t), _ = quantize_both(o, weight_f32(311, N, K), dev)
    xb = act_bf16(312, M, K)
    x = to_dev_bf16(xb, dev)
    for v in (float("nan"), float("inf"), -float("inf")):
        f = _word(dev)
        nv.linear(x, c, s, torch.tensor([v], device=dev), check=True, faults=f)
        assert int(f.item()) == nv.FAULT_NAN_SCALE
    # a non-finite BF16 activation (also through the in-call quantization form)
    for v in (float("nan"), float("inf")):
        xn = x.clone()
        xn[2, 77] = v
        f = _word(dev)
        nv.linear(xn, c, s, t, check=True, faults=f)
        assert int(f.item()) == nv.FAULT_NONFINITE
        f = _word(dev)
        nv.linear(xn[2:3], c, s, t, check=True, faults=f, quantize_x=True)
        assert int(f.item()) == nv.FAULT_NONFINITE
    # NVFP4 activations: their scale bytes and their row tensor scales
    xc, xs, xt = nv.quantize_act(x)
    f = _word(dev)
    nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt, check=True, faults=f)
    assert int(f.item()) == 0
    xs_bad = xs.clone()
    xs_bad[3, 5] = 0xFF
    f = _word(dev)
    nv.linear(xc, c, s, t, x_scales=xs_bad, x_ts=xt, check=True, faults=f)
    assert int(f.item()) == nv.FAULT_NAN_SCALE
    xt_bad = xt.clone()
    xt_bad[1] = float("inf")
    f = _word(dev)
    nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt_bad, check=True, faults=f)
    assert int(f.item()) == nv.FAULT_NAN_SCALE


def test_check_mode_misaligned_scale_view(dev, o):
    """Scales at a 2-byte offset (a sliced view): the scan takes its 2-byte path."""
    N, K, M = 48, 256, 2
    (c, s, t), oq = quantize_both(o, weight_f32(321, N, K), dev)
    buf = torch.zeros(s.numel() + 16, dtype=torch.uint8, device=dev)
    sv = buf[2:2 + s.numel()].view(N, K // 16)
    sv.copy_(s)
    buf[0] = 0x7F  # outside the view: not scanned
    buf[1] = 0xFF
    buf[2 + s.numel()] = 0x7F
    x = to_dev_bf16(act_bf16(322, M, K), dev)
    f = _word(dev)
    y = nv.linear(x, c, sv, t, check=True, faults=f)
    assert int(f.item()) == 0
    assert torch.equal(y, nv.linear(x, c, s, t))
    sv[N - 1, K // 16 - 1] = 0x7F
    f = _word(dev)
    nv.linear(x, c, sv, t, check=True, faults=f)
    assert int(f.item()) == nv.FAULT_NAN_SCALE


def test_check_mode_grouped(dev, o):
    """The grouped call scans every expert's scales (also experts no route picks) and the
    activation rows; without the flag the outputs are the same bits and nothing is set."""
    E, N, K, T, k = 6, 64, 128, 8, 2
    _say("check mode: grouped call")
    ws = [quantize_both(o, weight_f32(331, N, K, stream=10 + e), dev) for e in range(E)]
    wc = torch.stack([q[0][0] for q in ws])
    wsc = torch.stack([q[0][1] for q in ws])
    wts = torch.cat([q[0][2] for q in ws])
    ids = torch.from_numpy(np.array([[e % 5, (e + 1) % 5] for e in range(T)], np.int32)).to(dev)
    x = to_dev_bf16(act_bf16(332, T, K), dev)
    f = _word(dev)
    h_chk = nv.grouped_linear(x, wc, wsc, wts, ids, check=True, faults=f)
    assert int(f.item()) == 0
    assert torch.equal(h_chk, nv.grouped_linear(x, wc, wsc, wts, ids))
    wsc_bad = wsc.clone()
    wsc_bad[5, N - 1, 3] = 0x7F  # expert 5 is never routed
    f = _word(dev)
    nv.grouped_linear(x, wc, wsc_bad, wts, ids, faults=f)
    assert int(f.item()) == 0
    nv.grouped_linear(x, wc, wsc_bad, wts, ids, check=True, faults=f)
    assert int(f.item()) == nv.FAULT_NAN_SCALE
    wts_bad = wts.clone()
    wts_bad[4] = float("nan")
    f = _word(dev)
    nv.grouped_linear(x, wc, wsc, wts_bad, ids, check=True, faults=f)
    assert int(f.item()) == nv.FAULT_NAN_SCALE
    xn = x.clone()
    xn[T - 1, K - 1] = float("-inf")
    f = _word(dev)
    nv.grouped_linear(xn, wc, wsc, wts, ids, check=True, faults=f)
    assert int(f.item()) == nv.FAULT_NONFINITE


def test_splitk_shape_with_offset_scale_views(dev, o):
    """A shape that takes the K-split GEMM, with weight and activation scales at a 2-byte
    offset: the call takes the 64-row kernel instead (the K-split kernel loads scales as
    16-byte pieces) and matches the oracle on every output, and the aligned call."""
    M, N, K = 300, 1000, 2304
    _say(f"split-K shape with offset scales M={M} N={N} K={K}")
    (c, s, t), oq = quantize_both(o, weight_f32(341, N, K), dev)
    buf = torch.zeros(s.numel() + 16, dtype=torch.uint8, device=dev)
    sv = buf[2:2 + s.numel()].view(N, K // 16)
    sv.copy_(s)
    xb = act_bf16(342, M, K)
    x = to_dev_bf16(xb, dev)
    y = nv.linear(x, c, sv, t).cpu().numpy()
    yr, b = o.linear(xb, *oq)
    assert_within(y, yr, b, "offset weight scales")
    xc, xs, xt = nv.quantize_act(x)
    xbuf = torch.zeros(xs.numel() + 16, dtype=torch.uint8, device=dev)
    xsv = xbuf[2:2 + xs.numel()].view(M, K // 16)
    xsv.copy_(xs)
    oc, os_, ot = o.quantize_bf16(xb, per_row=True)
    assert np.array_equal(xc.cpu().numpy(), oc) and np.array_equal(xs.cpu().numpy(), os_)
    yr4, b4 = o.linear_w4a4(oc, os_, ot, *oq)
    for ws_, xs_ in ((s, xsv), (sv, xs), (sv, xsv)):
        y4 = nv.linear(xc, c, ws_, t, x_scales=xs_, x_ts=xt).cpu().numpy()
        assert_within(y4, yr4, b4, "offset scales w4a4")


def test_prefetch_reads_without_writing(dev, o):
    """nvfp4_prefetch reads a buffer on a stream and changes nothing: the buffer's bytes
    and a following linear on the prefetched weight are unchanged, for the smallest size,
    a size that is not a whole number of its load rounds, and with each workgroup cap."""
    N, K = 640, 1024
    (c, s, t), oq = quantize_both(o, weight_f32(351, N, K), dev)
    x = to_dev_bf16(act_bf16(352, 4, K), dev)
    y0 = nv.linear(x, c, s, t)
    c0, s0 = c.clone(), s.clone()
    for wg in (0, 1, 7, 512):
        nv.prefetch(c, wg)
        nv.prefetch(s, wg)
        nv.prefetch(c[:1, :16].contiguous(), wg)  # 16 bytes
    torch.cuda.synchronize()
    assert torch.equal(c, c0) and torch.equal(s, s0)
    assert torch.equal(nv.linear(x, c, s, t), y0)
    with pytest.raises(nv.NVFP4Error, match="ALIGN"):
        nv.prefetch(c.view(-1)[8:8 + 4096])
