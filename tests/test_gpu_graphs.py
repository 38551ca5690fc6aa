"""Every entry point recorded into a HIP graph and replayed: the library allocates nothing,
clears scratch words with its own fill kernels (no memset nodes) and keeps no state
between calls, so a captured call must give the eager result on every replay. Each graph
is replayed several times with other eager work of the same entry points and host
synchronization in between, its outputs overwritten before each replay, and every replay
is compared bit for bit with the eager result."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_linear_amd as nv
from gpu_helpers import device, to_dev_bf16
from synth import act_bf16, moe_routes, weight_f32

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def dev():
    return device()


def _weight(dev, seed, N, K):
    wd = torch.from_numpy(weight_f32(seed, N, K)).to(dev)
    return nv.quantize_act(wd, per_tensor=True)


def _check_replays(fn, outs, disturb):
    """fn() writes `outs`; eager result first, then a captured graph replayed REPLAYS times
    with the outputs overwritten and `disturb()` (other eager launches) between replays."""
    fn()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for o in outs:
            o.view(torch.uint8).fill_(0xA5)
        disturb()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o.view(torch.uint8), w.view(torch.uint8)), f"replay {i}"


@pytest.mark.parametrize("M", [1, 4, 12, 64])  # streaming forms (one / three row sets), GEMM
def test_graph_linear(dev, M):
    N, K = 1000, 1024
    c, s, t = _weight(dev, 60 + M, N, K)
    x = to_dev_bf16(act_bf16(61 + M, M, K), dev)
    x2 = to_dev_bf16(act_bf16(62 + M, M, K), dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    _check_replays(lambda: nv.linear(x, c, s, t, out=y), [y],
                   lambda: nv.linear(x2, c, s, t))


def test_graph_linear_persistent_gemm(dev):
    """The wide GEMM's persistent pipeline (more 256 x 256 tiles than CUs: 3 x 86 = 258,
    ragged in M and N): each replay bit-equal to the eager call."""
    M, N, K = 600, 86 * 256 - 100, 512
    c, s, t = _weight(dev, 66, N, K)
    x = to_dev_bf16(act_bf16(67, M, K), dev)
    x2 = to_dev_bf16(act_bf16(68, M, K), dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    _check_replays(lambda: nv.linear(x, c, s, t, out=y), [y],
                   lambda: nv.linear(x2, c, s, t))


def test_graph_w4a4_two_calls_and_in_call(dev):
    N, K, M = 768, 2048, 1
    c, s, t = _weight(dev, 63, N, K)
    x = to_dev_bf16(act_bf16(64, M, K), dev)
    xc, xs, xt = nv.quantize_act(x)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    y1 = torch.empty((M, N), dtype=torch.float32, device=dev)

    def two_calls():
        nv.quantize_act(x, codes=xc, scales=xs, ts=xt)
        nv.linear(xc, c, s, t, x_scales=xs, x_ts=xt, out=y)

    _check_replays(two_calls, [xc, xs, xt, y], lambda: nv.quantize_act(x * 2))
    _check_replays(lambda: nv.linear(x, c, s, t, out=y1, quantize_x=True), [y1],
                   lambda: nv.linear(x * 2, c, s, t, quantize_x=True))
    assert torch.equal(y, y1)


def test_graph_quantize_per_tensor(dev):
    """The per-tensor form clears its amax word with a fill kernel inside the call."""
    w = torch.from_numpy(weight_f32(65, 300, 512)).to(dev)
    c = torch.empty((300, 256), dtype=torch.uint8, device=dev)
    sc = torch.empty((300, 32), dtype=torch.uint8, device=dev)
    ts = torch.empty((1,), dtype=torch.float32, device=dev)
    _check_replays(lambda: nv.quantize_act(w, per_tensor=True, codes=c, scales=sc, ts=ts),
                   [c, sc, ts], lambda: nv.quantize_act(w * 3, per_tensor=True))


# decode-sized, GEMM and wide GEMM paths (the last: 300 routes per expert on average)
@pytest.mark.parametrize("T,E,k", [(4, 16, 4), (256, 8, 2), (600, 4, 2)])
def test_graph_moe_layer(dev, T, E, k):
    """gate_up with SwiGLU, then down with the ordered combine reusing the grouping, in one
    graph, as the MoE layer runs them."""
    Ngu, Kgu, Nd, Kd = 256, 512, 512, 128
    gu = [_weight(dev, 700 + e, Ngu, Kgu) for e in range(E)]
    dn = [_weight(dev, 800 + e, Nd, Kd) for e in range(E)]
    gc, gs, gt = (torch.stack([q[0] for q in gu]), torch.stack([q[1] for q in gu]),
                  torch.cat([q[2] for q in gu]))
    dc, ds, dt = (torch.stack([q[0] for q in dn]), torch.stack([q[1] for q in dn]),
                  torch.cat([q[2] for q in dn]))
    ids, rw = moe_routes(66, T, E, k)
    ids_d = torch.from_numpy(ids).to(dev)
    rw_d = torch.from_numpy(rw).to(dev)
    x = to_dev_bf16(act_bf16(67, T, Kgu), dev)
    a = torch.empty((T * k, Ngu // 2), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, Nd), dtype=torch.float32, device=dev)
    ws = torch.empty(max(nv.grouped_workspace_size(T, k, Ngu, Kgu, E, nv.OUT_SWIGLU_BF16),
                         nv.grouped_workspace_size(T, k, Nd, Kd, E, nv.OUT_COMBINE)),
                     dtype=torch.uint8, device=dev)
    ids2 = torch.from_numpy(np.ascontiguousarray(ids[::-1])).to(dev)

    def layer():
        nv.grouped_linear(x, gc, gs, gt, ids_d, out_mode=nv.OUT_SWIGLU_BF16, out=a, workspace=ws)
        nv.grouped_linear(a, dc, ds, dt, ids_d, topk_w=rw_d, out_mode=nv.OUT_COMBINE,
                          rows_per_route=True, out=y, workspace=ws, reuse_grouping=True)

    def disturb():  # another grouping through the same workspace, eagerly
        nv.grouped_linear(x, gc, gs, gt, ids2, out_mode=nv.OUT_SWIGLU_BF16, workspace=ws)

    _check_replays(layer, [a, y], disturb)
