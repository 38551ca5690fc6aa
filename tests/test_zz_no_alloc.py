"""The no-allocation grouped call (nvfp4_grouped_linear_noalloc, through the C ABI) against
the workspace form (nvfp4_grouped_linear) on the same inputs: two calls in a row, the
second smaller, in each output form, on the decode-sized (weight-streaming) and the
prompt-sized (grouped GEMM, and its wide form) paths. The two forms run the same kernels,
so their outputs must agree bit for bit; the workspace form is itself checked against the
oracle by the MoE parity tests."""
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


def _experts(o, dev, E, N, K, seed):
    ws = [quantize_both(o, weight_f32(seed, N, K, stream=70 + e), dev) for e in range(E)]
    return (torch.stack([q[0][0] for q in ws]), torch.stack([q[0][1] for q in ws]),
            torch.cat([q[0][2] for q in ws]), ws)


def _pair(dev, x, w, ids_d, rw_d, out_mode, rows_per_route=False):
    """(workspace form, no-allocation form) outputs; the latter's buffer starts dirty."""
    ref = nv.grouped_linear(x, *w, ids_d, topk_w=rw_d, out_mode=out_mode,
                            rows_per_route=rows_per_route)
    out = torch.full_like(ref.view(torch.uint8), 0x7F).view(ref.dtype)
    got = nv.grouped_linear_noalloc(x, *w, ids_d, topk_w=rw_d, out_mode=out_mode,
                                    rows_per_route=rows_per_route, out=out)
    return ref, got


@pytest.mark.parametrize("case", [
    # (E, N, K, T, top_k): a decode-sized layer, then a smaller one
    [(32, 256, 512, 16, 8), (12, 96, 256, 3, 2)],
    # prompt-sized (grouped GEMM: >= 32 routes per expert), then a smaller prompt
    [(8, 320, 256, 512, 2), (4, 64, 128, 160, 1)],
    # the grouped GEMM's wide form (>= 192 routes per expert), then a smaller prompt
    [(4, 320, 256, 560, 2), (4, 64, 128, 160, 1)],
])
def test_noalloc_matches_workspace_form(dev, o, case):
    for i, (E, N, K, T, k) in enumerate(case):
        _say(f"no-alloc call {i}: E={E} N={N} K={K} T={T} top_k={k}")
        wc, wsc, wts, _ = _experts(o, dev, E, N, K, 400 + i)
        ids, rw = moe_routes(410 + i, T, E, k)
        ids_d = torch.from_numpy(ids.astype(np.int32)).to(dev)
        rw_d = torch.from_numpy(rw.astype(np.float32)).to(dev)
        x = to_dev_bf16(act_bf16(420 + i, T, K), dev)
        for mode in (nv.OUT_ROUTES, nv.OUT_SWIGLU_BF16, nv.OUT_COMBINE):
            ref, got = _pair(dev, x, (wc, wsc, wts), ids_d, rw_d, mode)
            assert torch.equal(ref.view(torch.uint8), got.view(torch.uint8)), (i, mode)


def test_noalloc_layer_reuses_its_own_grouping(dev, o):
    """A MoE decode layer on the no-allocation call: gate_up with SwiGLU, then down with
    the ordered combine reusing the grouping that the first call left in the scratch; equal
    to the workspace form's layer, then a second, smaller layer; and the oracle's combine
    on the GPU's BF16 rows."""
    for i, (E, T, k) in enumerate([(64, 16, 8), (16, 4, 4)]):
        Ng, Kg, Nd, Kd = 384, 512, 256, 192
        _say(f"no-alloc layer {i}: E={E} T={T} top_k={k}")
        gc, gs, gt, _ = _experts(o, dev, E, Ng, Kg, 430 + i)
        dc, ds, dt, dq = _experts(o, dev, E, Nd, Kd, 440 + i)
        ids, rw = moe_routes(450 + i, T, E, k)
        ids = ids.astype(np.int32)
        rw = rw.astype(np.float32)
        ids_d = torch.from_numpy(ids).to(dev)
        rw_d = torch.from_numpy(rw).to(dev)
        x = to_dev_bf16(act_bf16(460 + i, T, Kg), dev)
        a = torch.empty((T * k, Ng // 2), dtype=torch.bfloat16, device=dev)
        y = torch.empty((T, Nd), dtype=torch.float32, device=dev)
        nv.grouped_linear_noalloc(x, gc, gs, gt, ids_d, out_mode=nv.OUT_SWIGLU_BF16, out=a)
        nv.grouped_linear_noalloc(a, dc, ds, dt, ids_d, topk_w=rw_d, out_mode=nv.OUT_COMBINE,
                                  rows_per_route=True, out=y, reuse_grouping=True)
        a_ref = nv.grouped_linear(x, gc, gs, gt, ids_d, out_mode=nv.OUT_SWIGLU_BF16)
        y_ref = nv.grouped_linear(a_ref, dc, ds, dt, ids_d, topk_w=rw_d, out_mode=nv.OUT_COMBINE,
                                  rows_per_route=True)
        assert torch.equal(a.view(torch.int16), a_ref.view(torch.int16))
        assert torch.equal(y, y_ref)
        oc = np.stack([q[1][0] for q in dq]); os_ = np.stack([q[1][1] for q in dq])
        ot = np.concatenate([q[1][2] for q in dq])
        a_bits = a.view(torch.int16).cpu().numpy().view(np.uint16)
        yr, b = o.moe_down_combine(a_bits, ids, rw, oc, os_, ot)
        assert_within(y.cpu().numpy(), yr, b, f"no-alloc layer {i}")


def test_noalloc_refuses_beyond_its_scratch(dev, o):
    E, N, K, T, k = 4, 2048, 256, 1024, 2  # combine rows: 2048 routes x 2048 x 4 B = 16 MiB
    wc, wsc, wts, _ = _experts(o, dev, E, N, K, 470)
    ids, rw = moe_routes(471, T, E, k)
    x = to_dev_bf16(act_bf16(472, T, K), dev)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)
    with pytest.raises(nv.NVFP4Error, match="WORKSPACE"):
        nv.grouped_linear_noalloc(x, wc, wsc, wts, torch.from_numpy(ids.astype(np.int32)).to(dev),
                                  topk_w=torch.from_numpy(rw.astype(np.float32)).to(dev),
                                  out_mode=nv.OUT_COMBINE, out=y)
