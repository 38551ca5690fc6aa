"""GPU parity of the expert-grouped call (nvfp4_grouped_linear) against the oracle's MoE
reading: 128 experts, gate_up 2048 -> 1536 and down 768 -> 2048, 16 tokens, top-8.

Stage-wise, on the GPU's own intermediates:
 (i)   gate_up per-route rows within the linear bound;
 (ii)  SwiGLU -> BF16 equal to the BF16 rounding of the float64 SwiGLU of the GPU's
       fp32 rows, up to one BF16 ulp where fp32 and fp64 straddle a rounding point;
 (iii) down + ordered combine within 1e-4 * sum_routes |r| sum_k |a_k w_k| + 1e-6;
 (iv)  end-to-end against the oracle's own chain: error/bound ratio reported only."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_linear_amd as nv
import oracle
from gpu_helpers import assert_within, device, quantize_both, to_dev_bf16
from synth import WORKLOADS, act_bf16, moe_expert_weights, moe_routes, weight_f32

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


@pytest.fixture(scope="module")
def moe(dev, o):
    cfg = WORKLOADS["moe_decode"]
    E, T, k = cfg["E"], cfg["T"], cfg["top_k"]
    _say(f"MoE weights: {E} experts, quantized on both sides")
    g = {name: [] for name in ("gc", "gs", "gt", "dc", "ds", "dt", "ogc", "ogs", "ogt", "odc", "ods", "odt")}
    for e in range(E):
        gu, dn = moe_expert_weights(cfg["w_seed"], e, cfg["N_gu"], cfg["K_gu"], cfg["N_d"], cfg["K_d"])
        (c, s, t), (oc, os_, ot) = quantize_both(o, gu, dev)
        g["gc"].append(c); g["gs"].append(s); g["gt"].append(t)
        g["ogc"].append(oc); g["ogs"].append(os_); g["ogt"].append(ot)
        (c, s, t), (oc, os_, ot) = quantize_both(o, dn, dev)
        g["dc"].append(c); g["ds"].append(s); g["dt"].append(t)
        g["odc"].append(oc); g["ods"].append(os_); g["odt"].append(ot)
    d = {}
    for key in ("gc", "gs", "dc", "ds"):
        d[key] = torch.stack(g[key])
    for key in ("gt", "dt"):
        d[key] = torch.cat(g[key])
    for key in ("ogc", "ogs", "odc", "ods"):
        d[key] = np.stack(g[key])
    for key in ("ogt", "odt"):
        d[key] = np.concatenate(g[key])
    ids, rw = moe_routes(cfg["route_seed"], T, E, k)
    xb = act_bf16(cfg["x_seed"], T, cfg["K_gu"])
    d.update(ids=ids, rw=rw, xb=xb, ids_d=torch.from_numpy(ids).to(dev),
             rw_d=torch.from_numpy(rw).to(dev), x_d=to_dev_bf16(xb, dev))
    return d


def test_moe_gate_up_routes(dev, o, moe):
    _say("MoE stage (i): gate_up per-route rows")
    h = nv.grouped_linear(moe["x_d"], moe["gc"], moe["gs"], moe["gt"], moe["ids_d"])
    hr, hb = o.moe_gate_up(moe["xb"], moe["ids"], moe["ogc"], moe["ogs"], moe["ogt"])
    assert_within(h.cpu().numpy(), hr, hb, "gate_up rows")


def test_moe_swiglu_bf16(dev, o, moe):
    _say("MoE stage (ii): SwiGLU to BF16 on the GPU's rows")
    h = nv.grouped_linear(moe["x_d"], moe["gc"], moe["gs"], moe["gt"], moe["ids_d"])
    a = nv.grouped_linear(moe["x_d"], moe["gc"], moe["gs"], moe["gt"], moe["ids_d"],
                          out_mode=nv.OUT_SWIGLU_BF16)
    a_bits = a.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = o.swiglu(h.cpu().numpy().astype(np.float64))
    ref_bits = np.array([o.bf16_round(v) for v in ref.ravel()], np.uint16).reshape(ref.shape)
    exact = np.mean(a_bits == ref_bits)
    # within one BF16 ulp: adjacent bit patterns of the same sign
    diff = np.abs(a_bits.astype(np.int32) - ref_bits.astype(np.int32))
    assert np.all(diff <= 1), np.argwhere(diff > 1)[:5]
    assert exact >= 0.999, exact
    _say(f"SwiGLU BF16 bit-exact fraction {exact:.6f}")
    for _ in range(2):  # deterministic
        a2 = nv.grouped_linear(moe["x_d"], moe["gc"], moe["gs"], moe["gt"], moe["ids_d"],
                               out_mode=nv.OUT_SWIGLU_BF16)
        assert torch.equal(a2.view(torch.int16), a.view(torch.int16))


def test_moe_down_combine_and_end_to_end(dev, o, moe):
    _say("MoE stage (iii): down + ordered combine on the GPU's BF16 activations")
    a = nv.grouped_linear(moe["x_d"], moe["gc"], moe["gs"], moe["gt"], moe["ids_d"],
                          out_mode=nv.OUT_SWIGLU_BF16)
    y = nv.grouped_linear(a, moe["dc"], moe["ds"], moe["dt"], moe["ids_d"], topk_w=moe["rw_d"],
                          out_mode=nv.OUT_COMBINE, rows_per_route=True)
    a_bits = a.view(torch.int16).cpu().numpy().view(np.uint16)
    yr, yb = o.moe_down_combine(a_bits, moe["ids"], moe["rw"], moe["odc"], moe["ods"], moe["odt"])
    assert_within(y.cpu().numpy(), yr, yb, "down+combine")
    # (iv) the oracle's own chain end to end: reported, not gated
    hr, _ = o.moe_gate_up(moe["xb"], moe["ids"], moe["ogc"], moe["ogs"], moe["ogt"])
    ar = o.swiglu(hr)
    ar_bits = np.array([o.bf16_round(v) for v in ar.ravel()], np.uint16).reshape(ar.shape)
    ye, eb = o.moe_down_combine(ar_bits, moe["ids"], moe["rw"], moe["odc"], moe["ods"], moe["odt"])
    ratio = np.max(np.abs(y.cpu().numpy() - ye) / (1e-4 * eb + 1e-6))
    _say(f"MoE end-to-end worst error/bound ratio (not gated): {ratio:.4f}")


def test_moe_deterministic_and_token_permutation(dev, moe):
    a = nv.grouped_linear(moe["x_d"], moe["gc"], moe["gs"], moe["gt"], moe["ids_d"],
                          out_mode=nv.OUT_SWIGLU_BF16)
    y1 = nv.grouped_linear(a, moe["dc"], moe["ds"], moe["dt"], moe["ids_d"], topk_w=moe["rw_d"],
                           out_mode=nv.OUT_COMBINE, rows_per_route=True)
    for _ in range(3):
        y2 = nv.grouped_linear(a, moe["dc"], moe["ds"], moe["dt"], moe["ids_d"], topk_w=moe["rw_d"],
                               out_mode=nv.OUT_COMBINE, rows_per_route=True)
        assert torch.equal(y1, y2)
    T, k = moe["ids"].shape
    perm = torch.from_numpy(np.random.default_rng(4).permutation(T)).to(dev)
    ids_p = moe["ids_d"][perm].contiguous()
    rw_p = moe["rw_d"][perm].contiguous()
    a_p = a.view(T, k, -1)[perm].reshape(T * k, -1).contiguous()
    y_p = nv.grouped_linear(a_p, moe["dc"], moe["ds"], moe["dt"], ids_p, topk_w=rw_p,
                            out_mode=nv.OUT_COMBINE, rows_per_route=True)
    assert torch.equal(y_p, y1[perm])


def test_grouped_top1_equals_dense(dev, moe):
    """With one route per token, each route row is the dense linear of that expert,
    bit for bit (same kernel, same K split)."""
    ids1 = moe["ids_d"][:, :1].contiguous()
    h = nv.grouped_linear(moe["x_d"], moe["gc"], moe["gs"], moe["gt"], ids1)
    for t in range(ids1.shape[0]):
        e = int(ids1[t, 0])
        yd = nv.linear(moe["x_d"][t:t + 1], moe["gc"][e], moe["gs"][e], moe["gt"][e:e + 1])
        assert torch.equal(h[t], yd[0]), t


def test_grouped_bad_routes_flagged_and_dropped(dev, o):
    E, N, K, T, k = 6, 40, 64, 4, 3
    ws = [quantize_both(o, weight_f32(8, N, K, stream=30 + e), dev) for e in range(E)]
    wc = torch.stack([q[0][0] for q in ws]); wsc = torch.stack([q[0][1] for q in ws])
    wts = torch.cat([q[0][2] for q in ws])
    ids = np.array([[0, 5, 2], [1, 1, 3], [7, 2, -1], [4, 0, 5]], np.int32)
    xb = act_bf16(12, T, K)
    faults = torch.zeros(1, dtype=torch.int32, device=dev)
    h = nv.grouped_linear(to_dev_bf16(xb, dev), wc, wsc, wts, torch.from_numpy(ids).to(dev),
                          faults=faults).cpu().numpy()
    assert int(faults.item()) & nv.FAULT_BAD_ROUTE
    dropped = {(1, 1), (2, 0), (2, 2)}
    for t in range(T):
        for j in range(k):
            r = t * k + j
            if (t, j) in dropped:
                assert np.all(h[r] == 0), (t, j)
            else:
                e = ids[t, j]
                yr, b = o.linear(xb[t:t + 1], ws[e][1][0], ws[e][1][1], ws[e][1][2])
                assert_within(h[r:r + 1], yr, b, f"route {t},{j}")
    # the SwiGLU form: dropped routes give zero rows too (the output buffer starts dirty)
    a = torch.full((T * k, N // 2), 0x7F7F, dtype=torch.int16, device=dev).view(torch.bfloat16)
    nv.grouped_linear(to_dev_bf16(xb, dev), wc, wsc, wts, torch.from_numpy(ids).to(dev),
                      out_mode=nv.OUT_SWIGLU_BF16, out=a)
    a_bits = a.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = o.swiglu(h.astype(np.float64))
    ref_bits = np.array([o.bf16_round(v) for v in ref.ravel()], np.uint16).reshape(ref.shape)
    for t in range(T):
        for j in range(k):
            r = t * k + j
            if (t, j) in dropped:
                assert np.all(a_bits[r] == 0), (t, j)
            else:
                d = np.abs(a_bits[r].astype(np.int32) - ref_bits[r].astype(np.int32))
                assert np.all(d <= 1), (t, j)


def test_grouped_w4a4_and_many_routes_per_expert(dev, o):
    """NVFP4 activations per token, and an expert with more than 16 routes (several
    16-row passes over its weight)."""
    E, N, K, T, k = 3, 72, 96, 40, 2
    ws = [quantize_both(o, weight_f32(9, N, K, stream=40 + e), dev) for e in range(E)]
    wc = torch.stack([q[0][0] for q in ws]); wsc = torch.stack([q[0][1] for q in ws])
    wts = torch.cat([q[0][2] for q in ws])
    ids = np.stack([np.zeros(T, np.int32), 1 + (np.arange(T) % 2)], axis=1).astype(np.int32)
    xb = act_bf16(13, T, K)
    xc, xs, xt = nv.quantize_act(to_dev_bf16(xb, dev))
    h = nv.grouped_linear(xc, wc, wsc, wts, torch.from_numpy(ids).to(dev), x_scales=xs,
                          x_ts=xt).cpu().numpy()
    oc, os_, ot = o.quantize_bf16(xb, per_row=True)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            yr, b = o.linear_w4a4(oc[t:t + 1], os_[t:t + 1], ot[t:t + 1], *ws[e][1])
            assert_within(h[t * k + j:t * k + j + 1], yr, b, f"w4a4 route {t},{j}")


def _small_experts(o, dev, E, N, K, seed):
    ws = [quantize_both(o, weight_f32(seed, N, K, stream=60 + e), dev) for e in range(E)]
    wc = torch.stack([q[0][0] for q in ws]); wsc = torch.stack([q[0][1] for q in ws])
    wts = torch.cat([q[0][2] for q in ws])
    oc = np.stack([q[1][0] for q in ws]); os_ = np.stack([q[1][1] for q in ws])
    ot = np.concatenate([q[1][2] for q in ws])
    return wc, wsc, wts, oc, os_, ot


def _combine_check(dev, o, ids, E, N, K, seed, label):
    """COMBINE output (rows read per token) against the oracle's ordered combine; a
    dropped route enters the oracle with router weight 0 (an exact zero term)."""
    T, k = ids.shape
    wc, wsc, wts, oc, os_, ot = _small_experts(o, dev, E, N, K, seed)
    xb = act_bf16(seed + 1, T, K)
    rw = np.random.default_rng(seed).random((T, k)).astype(np.float32)
    faults = torch.zeros(1, dtype=torch.int32, device=dev)
    y = nv.grouped_linear(to_dev_bf16(xb, dev), wc, wsc, wts, torch.from_numpy(ids).to(dev),
                          topk_w=torch.from_numpy(rw).to(dev), out_mode=nv.OUT_COMBINE,
                          faults=faults).cpu().numpy()
    valid = np.zeros_like(ids, dtype=bool)
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(ids[t, j])
            valid[t, j] = 0 <= e < E and e not in seen
            if valid[t, j]:
                seen.add(e)
    ids_o = np.where(valid, ids, 0).astype(np.int32)
    rw_o = np.where(valid, rw, 0.0).astype(np.float32)
    a_bits = np.repeat(xb, k, axis=0)  # the route rows are the token rows
    yr, b = o.moe_down_combine(a_bits, ids_o, rw_o, oc, os_, ot)
    assert_within(y, yr, b, label)
    return int(faults.item())


def test_grouped_combine_with_dropped_routes(dev, o):
    ids = np.array([[0, 5, 2], [1, 1, 3], [7, 2, -1], [4, 0, 5]], np.int32)
    f = _combine_check(dev, o, ids, 6, 40, 64, 81, "combine with dropped routes")
    assert f & nv.FAULT_BAD_ROUTE


def test_grouped_stream_with_grouping_kernel(dev, o):
    """320 routes on the streaming kernels (more routes than experts, several per expert):
    per-route rows against the oracle (dropped routes zero), the combine, and bit
    equality with the same routes split into two calls of 160 routes each."""
    E, N, K, T, k = 64, 48, 128, 40, 8
    ids, _ = moe_routes(141, T, E, k)
    ids = ids.astype(np.int32)
    dropped = [(2, 3), (17, 0), (39, 7)]
    ids[2, 3] = ids[2, 1]
    ids[17, 0] = -5
    ids[39, 7] = E
    _say(f"grouped stream, 320 routes: T={T} k={k} E={E}")
    f = _combine_check(dev, o, ids, E, N, K, 142, "grouping kernel + stream: combine")
    assert f & nv.FAULT_BAD_ROUTE
    wc, wsc, wts, oc, os_, ot = _small_experts(o, dev, E, N, K, 142)
    xb = act_bf16(143, T, K)
    x = to_dev_bf16(xb, dev)
    faults = torch.zeros(1, dtype=torch.int32, device=dev)
    h = nv.grouped_linear(x, wc, wsc, wts, torch.from_numpy(ids).to(dev), faults=faults)
    assert int(faults.item()) & nv.FAULT_BAD_ROUTE
    hn = h.cpu().numpy()
    for t, j in dropped:
        assert np.all(hn[t * k + j] == 0), (t, j)
    for r in np.r_[0, T * k - 1, np.random.default_rng(7).choice(T * k, 24, replace=False)]:
        t, j = divmod(int(r), k)
        if (t, j) in dropped:
            continue
        e = int(ids[t, j])
        yr, b = o.linear(xb[t:t + 1], oc[e], os_[e], ot[e:e + 1])
        assert_within(hn[r:r + 1], yr, b, f"grouping kernel + stream: route {t},{j}")
    half = T // 2
    parts = [nv.grouped_linear(x[p * half:(p + 1) * half].contiguous(), wc, wsc, wts,
                               torch.from_numpy(ids[p * half:(p + 1) * half].copy()).to(dev))
             for p in range(2)]
    assert torch.equal(torch.cat(parts), h)


def test_grouped_many_experts_few_routes(dev, o):
    """2600 experts, 14 of them routed (ids up to 2599, far apart): each active expert's
    slot record and weight offset; dropped routes (repeat, out of range) zeroed and
    flagged; the experts no route picks hold zero weights, which no output may touch."""
    E, N, K, T, k = 2600, 32, 64, 6, 4
    ids = np.array([[5, 2100, 2599, 64], [2100, 7, 2047, 2048], [0, 5, 5, 2600],
                    [2599, 2598, 1, 2], [3000, 2049, 2100, 6], [64, 65, 2047, 0]], np.int32)
    dropped = [(2, 2), (2, 3), (4, 0)]
    used = sorted({int(e) for e in ids.ravel() if 0 <= e < E})
    _say(f"many experts: E={E}, {len(used)} experts routed")
    q = {e: quantize_both(o, weight_f32(151, N, K, stream=200 + e), dev) for e in used}
    wc = torch.zeros((E, N, K // 2), dtype=torch.uint8, device=dev)
    wsc = torch.zeros((E, N, K // 16), dtype=torch.uint8, device=dev)
    wts = torch.zeros(E, dtype=torch.float32, device=dev)
    for e in used:
        wc[e], wsc[e], wts[e] = q[e][0][0], q[e][0][1], q[e][0][2][0]
    xb = act_bf16(152, T, K)
    faults = torch.zeros(1, dtype=torch.int32, device=dev)
    h = nv.grouped_linear(to_dev_bf16(xb, dev), wc, wsc, wts, torch.from_numpy(ids).to(dev),
                          faults=faults).cpu().numpy()
    assert int(faults.item()) & nv.FAULT_BAD_ROUTE
    for t in range(T):
        for j in range(k):
            if (t, j) in dropped:
                assert np.all(h[t * k + j] == 0), (t, j)
                continue
            e = int(ids[t, j])
            yr, b = o.linear(xb[t:t + 1], *q[e][1])
            assert_within(h[t * k + j:t * k + j + 1], yr, b, f"many experts: route {t},{j}")


def test_grouped_many_routes_general_sort(dev, o):
    """More routes than one sorting workgroup holds at once (T * top_k > 1024): the
    chunked route grouping (one chunk here), several 16-row passes per expert, in both
    output forms."""
    E, N, K, T, k = 16, 48, 64, 160, 8
    ids, _ = moe_routes(91, T, E, k)
    ids = ids.astype(np.int32)
    ids[3, 5] = ids[3, 1]  # one repeated id: flagged and dropped
    f = _combine_check(dev, o, ids, E, N, K, 92, "many routes: combine")
    assert f & nv.FAULT_BAD_ROUTE
    wc, wsc, wts, oc, os_, ot = _small_experts(o, dev, E, N, K, 92)
    xb = act_bf16(93, T, K)
    h = nv.grouped_linear(to_dev_bf16(xb, dev), wc, wsc, wts, torch.from_numpy(ids).to(dev)).cpu().numpy()
    assert np.all(h[3 * k + 5] == 0)
    for r in np.r_[0, 1, 7, 400, 401, 1279, np.random.default_rng(5).choice(T * k, 20, replace=False)]:
        t, j = divmod(int(r), k)
        if (t, j) == (3, 5):
            continue
        e = int(ids[t, j])
        yr, b = o.linear(xb[t:t + 1], oc[e], os_[e], ot[e:e + 1])
        assert_within(h[r:r + 1], yr, b, f"many routes: route {t},{j}")


@pytest.mark.parametrize("T,k,E", [(700, 4, 24), (64, 20, 40)])
def test_grouped_chunked_and_wide_topk_grouping(dev, o, T, k, E):
    """Route sets beyond one workgroup: several token chunks (T = 700: three chunks of
    256 tokens), and top_k above 16 (the general single-workgroup grouping); dropped routes
    (repeated, out of range, negative) in both; combine and per-route rows against the
    oracle."""
    N, K = 40, 64
    _say(f"grouping T={T} top_k={k} E={E}")
    ids, _ = moe_routes(95 + k, T, E, k)
    ids = ids.astype(np.int32)
    dropped = [(3, 1), (T - 2, k - 1), (T // 2, 0)]
    ids[3, 1] = ids[3, 0]
    ids[T - 2, k - 1] = E + 1
    ids[T // 2, 0] = -1
    f = _combine_check(dev, o, ids, E, N, K, 96 + k, f"grouping T={T} k={k}: combine")
    assert f & nv.FAULT_BAD_ROUTE
    wc, wsc, wts, oc, os_, ot = _small_experts(o, dev, E, N, K, 96 + k)
    xb = act_bf16(97, T, K)
    h = nv.grouped_linear(to_dev_bf16(xb, dev), wc, wsc, wts, torch.from_numpy(ids).to(dev)).cpu().numpy()
    for t, j in dropped:
        assert np.all(h[t * k + j] == 0), (t, j)
    for r in np.r_[0, T * k - 1, np.random.default_rng(6).choice(T * k, 24, replace=False)]:
        t, j = divmod(int(r), k)
        if (t, j) in dropped:
            continue
        e = int(ids[t, j])
        yr, b = o.linear(xb[t:t + 1], oc[e], os_[e], ot[e:e + 1])
        assert_within(h[r:r + 1], yr, b, f"grouping T={T} k={k}: route {t},{j}")


def _prefill_case(dev, o, E, N, K, T, k, seed):
    wc, wsc, wts, oc, os_, ot = _small_experts(o, dev, E, N, K, seed)
    ids, rw = moe_routes(seed + 1, T, E, k)
    ids = ids.astype(np.int32)
    xb = act_bf16(seed + 2, T, K)
    return wc, wsc, wts, oc, os_, ot, ids, rw.astype(np.float32), xb


def test_grouped_prefill_gemm(dev, o):
    """Prompt-sized batches (routes average >= 32 per expert) take the MFMA GEMM path:
    per-route rows vs the oracle, one route per token = the dense linear bit for bit,
    SwiGLU from those rows, the ordered combine, determinism."""
    E, N, K, T, k = 8, 96, 256, 512, 2
    wc, wsc, wts, oc, os_, ot, ids, rw, xb = _prefill_case(dev, o, E, N, K, T, k, 101)
    x = to_dev_bf16(xb, dev)
    ids_d = torch.from_numpy(ids).to(dev)
    h = nv.grouped_linear(x, wc, wsc, wts, ids_d)
    hn = h.cpu().numpy()
    for r in np.r_[0, 1, 511, 512, 1023, np.random.default_rng(7).choice(T * k, 40, replace=False)]:
        t, j = divmod(int(r), k)
        e = int(ids[t, j])
        yr, b = o.linear(xb[t:t + 1], oc[e], os_[e], ot[e:e + 1])
        assert_within(hn[r:r + 1], yr, b, f"prefill route {t},{j}")
    assert torch.equal(nv.grouped_linear(x, wc, wsc, wts, ids_d), h)
    # one route per token: each expert's rows equal the dense product
    ids1 = ids_d[:, :1].contiguous()
    h1 = nv.grouped_linear(x, wc, wsc, wts, ids1)
    for e in range(E):
        toks = np.nonzero(ids[:, 0] == e)[0]
        if len(toks) <= 16:
            continue
        dense = nv.linear(x[torch.from_numpy(toks).to(dev)].contiguous(), wc[e], wsc[e], wts[e:e + 1])
        assert torch.equal(h1[torch.from_numpy(toks).to(dev)], dense), e
    # SwiGLU from the same rows
    a = nv.grouped_linear(x, wc, wsc, wts, ids_d, out_mode=nv.OUT_SWIGLU_BF16)
    a_bits = a.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = o.swiglu(hn.astype(np.float64))
    ref_bits = np.array([o.bf16_round(v) for v in ref.ravel()], np.uint16).reshape(ref.shape)
    assert np.all(np.abs(a_bits.astype(np.int32) - ref_bits.astype(np.int32)) <= 1)
    # ordered combine
    y = nv.grouped_linear(x, wc, wsc, wts, ids_d, topk_w=torch.from_numpy(rw).to(dev),
                          out_mode=nv.OUT_COMBINE).cpu().numpy()
    yr, b = o.moe_down_combine(np.repeat(xb, k, axis=0), ids, rw, oc, os_, ot)
    assert_within(y, yr, b, "prefill combine")


def test_grouped_prefill_gemm_many_routes(dev, o):
    """More than 1024 routes: the general grouping (order inside an expert's group is not
    fixed there) still gives bit-identical outputs run to run."""
    E, N, K, T, k = 16, 64, 128, 1024, 4
    wc, wsc, wts, oc, os_, ot, ids, rw, xb = _prefill_case(dev, o, E, N, K, T, k, 111)
    x = to_dev_bf16(xb, dev)
    ids_d = torch.from_numpy(ids).to(dev)
    h = nv.grouped_linear(x, wc, wsc, wts, ids_d)
    for _ in range(3):
        assert torch.equal(nv.grouped_linear(x, wc, wsc, wts, ids_d), h)
    hn = h.cpu().numpy()
    for r in np.r_[0, 4095, np.random.default_rng(8).choice(T * k, 40, replace=False)]:
        t, j = divmod(int(r), k)
        e = int(ids[t, j])
        yr, b = o.linear(xb[t:t + 1], oc[e], os_[e], ot[e:e + 1])
        assert_within(hn[r:r + 1], yr, b, f"many-route prefill {t},{j}")
    rw_d = torch.from_numpy(rw).to(dev)
    y = nv.grouped_linear(x, wc, wsc, wts, ids_d, topk_w=rw_d, out_mode=nv.OUT_COMBINE)
    assert torch.equal(nv.grouped_linear(x, wc, wsc, wts, ids_d, topk_w=rw_d,
                                         out_mode=nv.OUT_COMBINE), y)
    yr, b = o.moe_down_combine(np.repeat(xb, k, axis=0), ids, rw, oc, os_, ot)
    assert_within(y.cpu().numpy(), yr, b, "many-route prefill combine")


def _reuse_check(dev, x, g, d, ids_d, rw_d, tag):
    """gate_up (SwiGLU) then down + combine: the down call reusing the grouping the
    gate_up call left in a shared workspace equals the down call that regroups, bit for
    bit."""
    gc, gs, gt = g
    dc, ds, dt = d
    T, k = ids_d.shape
    N_gu, K = gc.shape[1], 2 * gc.shape[2]
    N_d, K_d = dc.shape[1], 2 * dc.shape[2]
    E = gc.shape[0]
    need = max(nv.grouped_workspace_size(T, k, N_gu, K, E, nv.OUT_SWIGLU_BF16),
               nv.grouped_workspace_size(T, k, N_d, K_d, E, nv.OUT_COMBINE))
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=dev)
    a = nv.grouped_linear(x, gc, gs, gt, ids_d, out_mode=nv.OUT_SWIGLU_BF16, workspace=ws)
    y_reuse = nv.grouped_linear(a, dc, ds, dt, ids_d, topk_w=rw_d, out_mode=nv.OUT_COMBINE,
                                rows_per_route=True, workspace=ws, reuse_grouping=True)
    y = nv.grouped_linear(a, dc, ds, dt, ids_d, topk_w=rw_d, out_mode=nv.OUT_COMBINE,
                          rows_per_route=True)
    assert torch.equal(y_reuse, y), tag
    with pytest.raises(ValueError):
        nv.grouped_linear(a, dc, ds, dt, ids_d, topk_w=rw_d, out_mode=nv.OUT_COMBINE,
                          rows_per_route=True, reuse_grouping=True)


def test_grouped_reuse_grouping_decode(dev, moe):
    _say("MoE decode layer: down + combine reusing the gate_up call's grouping")
    _reuse_check(dev, moe["x_d"], (moe["gc"], moe["gs"], moe["gt"]),
                 (moe["dc"], moe["ds"], moe["dt"]), moe["ids_d"], moe["rw_d"], "decode")


def test_grouped_reuse_grouping_prefill(dev, o):
    _say("MoE prefill: down + combine reusing the gate_up call's grouping (GEMM path)")
    E, N, K, T, k = 16, 64, 128, 1024, 4
    wc, wsc, wts, _, _, _, ids, rw, xb = _prefill_case(dev, o, E, N, K, T, k, 121)
    dc, dsc, dts, _, _, _ = _small_experts(o, dev, E, 96, N // 2, 122)
    _reuse_check(dev, to_dev_bf16(xb, dev), (wc, wsc, wts), (dc, dsc, dts),
                 torch.from_numpy(ids).to(dev), torch.from_numpy(rw).to(dev), "prefill")


# ---- the grouped GEMM beyond one column block, at the layer's real shape, and with NVFP4
# activations -----------------------------------------------------------------------------

def _swiglu_bits_check(o, a, h, label):
    """GPU SwiGLU BF16 rows against the BF16 rounding of the float64 SwiGLU of the GPU's
    own fp32 rows (same call shape): within one BF16 ulp everywhere, bit-exact nearly
    everywhere (an fp32 product can straddle a BF16 rounding point)."""
    a_bits = a.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_bits = o.bf16_round_array(o.swiglu(np.asarray(h, np.float64)))
    diff = np.abs(a_bits.astype(np.int32) - ref_bits.astype(np.int32))
    assert np.all(diff <= 1), (label, np.argwhere(diff > 1)[:5].tolist())
    exact = float(np.mean(diff == 0))
    assert exact >= 0.999, (label, exact)
    _say(f"{label}: SwiGLU BF16 bit-exact fraction {exact:.6f}")


def test_grouped_prefill_gemm_several_column_blocks(dev, o):
    """Prompt-sized routes (128 per expert) with N = 800: four 256-column blocks per tile
    for the per-route rows (the last ragged) and four 128-column gate/up blocks for SwiGLU
    (half = 400, the last ragged); every output of every route against the oracle, the
    SwiGLU rows from them, the ordered combine."""
    E, N, K, T, k = 8, 800, 256, 512, 2
    _say(f"grouped GEMM, several column blocks: E={E} N={N} K={K} T={T} k={k}")
    wc, wsc, wts, oc, os_, ot, ids, rw, xb = _prefill_case(dev, o, E, N, K, T, k, 131)
    x = to_dev_bf16(xb, dev)
    ids_d = torch.from_numpy(ids).to(dev)
    h = nv.grouped_linear(x, wc, wsc, wts, ids_d).cpu().numpy()
    x64 = o.bf16_to_f64(xb)
    for e in range(E):
        routes = np.nonzero(ids.ravel() == e)[0]
        wdq = o.dequant(oc[e], os_[e], ot[e:e + 1], per_row=False)
        yr, b = o.linear_f64(x64[routes // k], wdq)
        assert_within(h[routes], yr, b, f"column blocks: expert {e} rows")
    a = nv.grouped_linear(x, wc, wsc, wts, ids_d, out_mode=nv.OUT_SWIGLU_BF16)
    _swiglu_bits_check(o, a, h, "column blocks")
    y = nv.grouped_linear(x, wc, wsc, wts, ids_d, topk_w=torch.from_numpy(rw).to(dev),
                          out_mode=nv.OUT_COMBINE).cpu().numpy()
    yr, b = o.moe_down_combine(np.repeat(xb, k, axis=0), ids, rw, oc, os_, ot)
    assert_within(y, yr, b, "column blocks: combine")


@pytest.mark.parametrize("K", [320, 512, 544])
def test_grouped_wide_tiles_every_output_form(dev, o, K):
    """Routes averaging >= 192 per expert take the wide grouped form: each expert's first
    256 routes in one 256-route tile (wave-specialized), the rest in 32-route tiles. Here
    1600 routes over 6 experts (some above 256, so both kinds of tile run), N = 544 (a
    ragged third column block; half = 272, a ragged third gate block), K = 320 (an odd
    number of 64-k steps, one 2-byte scale load per step), 512 (the scales in 16-byte
    pieces of four steps) or 544 (nine steps, per-step scale loads); from eight steps the
    wide tiles take the persistent form, whose workgroups run several tiles each (six
    experts of three column blocks on 256 workgroups: one tile each here, several in the
    prefill layer test). Dropped routes: every output of every kept route against the
    oracle, dropped routes' rows zero, padded activation rows, SwiGLU from the rows, the
    ordered combine, determinism, one route per token equal to the dense product bit for
    bit, and (K = 512) the same bits from a scale copy that takes the per-step loads."""
    E, N, T, k = 6, 544, 400, 4
    _say(f"grouped GEMM, wide tiles: E={E} N={N} K={K} T={T} k={k}")
    wc, wsc, wts, oc, os_, ot, ids, rw, xb = _prefill_case(dev, o, E, N, K, T, k, 151)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.max() > 256 and counts.mean() >= 192, counts
    ids[3, 1] = -1  # dropped routes (flagged, their rows zero)
    ids[250, 3] = E + 2
    x = to_dev_bf16(xb, dev)
    ids_d = torch.from_numpy(ids).to(dev)
    faults = torch.zeros(1, dtype=torch.int32, device=dev)
    h_d = nv.grouped_linear(x, wc, wsc, wts, ids_d, faults=faults)
    assert int(faults.item()) & nv.FAULT_BAD_ROUTE
    h = h_d.cpu().numpy()
    x64 = o.bf16_to_f64(xb)
    for e in range(E):
        routes = np.nonzero(ids.ravel() == e)[0]
        wdq = o.dequant(oc[e], os_[e], ot[e:e + 1], per_row=False)
        yr, b = o.linear_f64(x64[routes // k], wdq)
        assert_within(h[routes], yr, b, f"wide tiles: expert {e} rows")
    assert not np.any(h[3 * k + 1]) and not np.any(h[250 * k + 3])
    assert torch.equal(nv.grouped_linear(x, wc, wsc, wts, ids_d), h_d)
    # padded activation rows (pitch K + 24, NaN in the padding, which is never read)
    xp = torch.full((T, K + 24), float("nan"), dtype=torch.bfloat16, device=dev)
    xp[:, :K] = x
    assert torch.equal(nv.grouped_linear(xp[:, :K], wc, wsc, wts, ids_d), h_d)
    a = nv.grouped_linear(x, wc, wsc, wts, ids_d, out_mode=nv.OUT_SWIGLU_BF16)
    kept = np.nonzero((ids.ravel() >= 0) & (ids.ravel() < E))[0]
    _swiglu_bits_check(o, a[torch.from_numpy(kept).to(dev)], h[kept], "wide tiles")
    rw_d = torch.from_numpy(rw).to(dev)
    y = nv.grouped_linear(x, wc, wsc, wts, ids_d, topk_w=rw_d, out_mode=nv.OUT_COMBINE)
    assert torch.equal(nv.grouped_linear(x, wc, wsc, wts, ids_d, topk_w=rw_d,
                                         out_mode=nv.OUT_COMBINE), y)
    valid = (ids >= 0) & (ids < E)
    yr, b = o.moe_down_combine(np.repeat(xb, k, axis=0), np.where(valid, ids, 0).astype(np.int32),
                               np.where(valid, rw, 0.0).astype(np.float32), oc, os_, ot)
    assert_within(y.cpu().numpy(), yr, b, "wide tiles: combine")
    # one route per token (800 tokens over 3 experts): each expert's rows, from its wide
    # tile and its 32-route tiles, equal the dense product (64-row kernel, same k order)
    T1 = 800
    ids1 = moe_routes(152, T1, 3, 1)[0].astype(np.int32)
    x1b = act_bf16(153, T1, K)
    x1 = to_dev_bf16(x1b, dev)
    h1 = nv.grouped_linear(x1, wc[:3], wsc[:3], wts[:3], torch.from_numpy(ids1).to(dev))
    for e in range(3):
        toks = torch.from_numpy(np.nonzero(ids1[:, 0] == e)[0]).to(dev)
        assert len(toks) > 256
        dense = nv.linear(x1[toks].contiguous(), wc[e], wsc[e], wts[e:e + 1])
        assert torch.equal(h1[toks], dense), e
    if K % 256 == 0:
        # scales 2 bytes past a 16-byte boundary: per-step scale loads, the same bits
        buf = torch.empty(wsc.numel() + 16, dtype=torch.uint8, device=dev)
        wsc2 = buf[2:2 + wsc.numel()].view(wsc.shape)
        wsc2.copy_(wsc)
        assert wsc.data_ptr() % 16 == 0 and wsc2.data_ptr() % 16 == 2
        assert torch.equal(nv.grouped_linear(x, wc, wsc2, wts, ids_d), h_d)
        assert torch.equal(nv.grouped_linear(x, wc, wsc2, wts, ids_d,
                                             out_mode=nv.OUT_SWIGLU_BF16), a)


@pytest.mark.parametrize("K", [544, 512])
def test_grouped_wide_persistent_several_tiles(dev, o, K):
    """The persistent form of the wide grouped tiles with several tiles per workgroup: 96
    experts of ~192 routes and N = 1024 (four column blocks) make 384 tiles on 256
    workgroups, so a third of the workgroups run two tiles, the second staged while the
    first one's results are stored. K = 544 (nine steps, per-step scale loads) and 512
    (scale pieces). Every output of every route against the oracle, SwiGLU from the rows
    (its 1024/2 columns are four gate/up blocks), determinism."""
    E, N, T, k = 96, 1024, 4608, 4
    _say(f"grouped GEMM, persistent wide tiles: E={E} N={N} K={K} T={T} k={k}")
    wc, wsc, wts, oc, os_, ot, ids, rw, xb = _prefill_case(dev, o, E, N, K, T, k, 171)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.mean() >= 192 and counts.min() > 0, counts
    x = to_dev_bf16(xb, dev)
    ids_d = torch.from_numpy(ids).to(dev)
    h_d = nv.grouped_linear(x, wc, wsc, wts, ids_d)
    h = h_d.cpu().numpy()
    x64 = o.bf16_to_f64(xb)
    for e in range(E):
        routes = np.nonzero(ids.ravel() == e)[0]
        wdq = o.dequant(oc[e], os_[e], ot[e:e + 1], per_row=False)
        yr, b = o.linear_f64(x64[routes // k], wdq)
        assert_within(h[routes], yr, b, f"persistent wide tiles: expert {e} rows")
    assert torch.equal(nv.grouped_linear(x, wc, wsc, wts, ids_d), h_d)
    a = nv.grouped_linear(x, wc, wsc, wts, ids_d, out_mode=nv.OUT_SWIGLU_BF16)
    _swiglu_bits_check(o, a, h, f"persistent wide tiles K={K}")
    assert torch.equal(nv.grouped_linear(x, wc, wsc, wts, ids_d, out_mode=nv.OUT_SWIGLU_BF16), a)


def test_grouped_chunked_grouping_both_forms(dev, o):
    """Route sets in chunks of 256 tokens are grouped in two launches up to 32 chunks (the
    counts, then the scan folded into the scatter workgroups, each summing the chunks'
    counts itself) and in three beyond (counts, one scan workgroup, scatter). Here 9000
    tokens (36 chunks: three launches), top-2 over 64 experts with dropped routes: every
    output of sampled routes against the oracle, dropped routes' rows zero, a repeated
    call equal bit for bit, and the first 8192 tokens' rows equal to those of a call on
    those tokens alone (32 chunks: two launches), since a route's row depends on neither
    the grouping's form nor its order. Both forms with the combine as well."""
    E, N, K, T, k = 64, 64, 128, 9000, 2
    _say(f"grouped GEMM, chunked grouping in both forms: E={E} N={N} K={K} T={T} k={k}")
    wc, wsc, wts, oc, os_, ot, ids, rw, xb = _prefill_case(dev, o, E, N, K, T, k, 181)
    ids[17, 1] = ids[17, 0]  # repeated within its token: dropped
    ids[8500, 0] = -3        # out of range: dropped
    x = to_dev_bf16(xb, dev)
    ids_d = torch.from_numpy(ids).to(dev)
    faults = torch.zeros(1, dtype=torch.int32, device=dev)
    h_d = nv.grouped_linear(x, wc, wsc, wts, ids_d, faults=faults)
    assert int(faults.item()) & nv.FAULT_BAD_ROUTE
    h = h_d.cpu().numpy()
    assert not np.any(h[17 * k + 1]) and not np.any(h[8500 * k])
    x64 = o.bf16_to_f64(xb)
    rng = np.random.default_rng(182)
    for r in np.r_[0, 1, 8191 * k, 8192 * k, T * k - 1, rng.choice(T * k, 60, replace=False)]:
        t, j = divmod(int(r), k)
        e = int(ids[t, j])
        if e < 0 or e >= E or (j == 1 and t == 17):
            continue
        wdq = o.dequant(oc[e], os_[e], ot[e:e + 1], per_row=False)
        yr, b = o.linear_f64(x64[t:t + 1], wdq)
        assert_within(h[r:r + 1], yr, b, f"chunked grouping route {t},{j}")
    assert torch.equal(nv.grouped_linear(x, wc, wsc, wts, ids_d), h_d)
    T2 = 8192
    h2 = nv.grouped_linear(x[:T2].contiguous(), wc, wsc, wts, ids_d[:T2].contiguous())
    assert torch.equal(h2, h_d[:T2 * k])
    rw_d = torch.from_numpy(rw).to(dev)
    y = nv.grouped_linear(x, wc, wsc, wts, ids_d, topk_w=rw_d, out_mode=nv.OUT_COMBINE)
    y2 = nv.grouped_linear(x[:T2].contiguous(), wc, wsc, wts, ids_d[:T2].contiguous(),
                           topk_w=rw_d[:T2].contiguous(), out_mode=nv.OUT_COMBINE)
    assert torch.equal(y2, y[:T2])


def test_moe_prefill_layer_full_shape(dev, o, moe):
    """The MoE layer at prompt size as the benchmark runs it: 4096 tokens over the 128
    experts, top-8 (32768 routes, the chunked grouping, six SwiGLU column blocks of the
    1536-wide gate_up and eight of the 2048-wide down), checked stage by stage on the GPU's
    own intermediates: 128 sampled routes' gate_up rows element-wise, every SwiGLU BF16
    value from the GPU's fp32 rows, and 64 sampled tokens' down + ordered combine."""
    cfg = WORKLOADS["moe_decode"]
    E, k, T = cfg["E"], cfg["top_k"], 4096
    _say(f"MoE prefill layer: T={T} E={E} top-{k}")
    ids, rw = moe_routes(cfg["route_seed"] + 1, T, E, k)
    ids = ids.astype(np.int32)
    rw = rw.astype(np.float32)
    xb = act_bf16(cfg["x_seed"] + 1, T, cfg["K_gu"])
    x = to_dev_bf16(xb, dev)
    ids_d = torch.from_numpy(ids).to(dev)
    rw_d = torch.from_numpy(rw).to(dev)
    # (i) gate_up per-route rows
    h_d = nv.grouped_linear(x, moe["gc"], moe["gs"], moe["gt"], ids_d)
    rng = np.random.default_rng(17)
    routes = np.r_[0, T * k - 1, rng.choice(T * k, 126, replace=False)]
    h_s = h_d[torch.from_numpy(routes).to(dev)].cpu().numpy()
    toks, js = routes // k, routes % k
    hr, hb = o.moe_gate_up(xb[toks], ids[toks, js][:, None].astype(np.int32), moe["ogc"],
                           moe["ogs"], moe["ogt"])
    assert_within(h_s, hr, hb, "prefill layer: gate_up rows")
    # (ii) SwiGLU -> BF16, every value, from the GPU's own rows
    a = nv.grouped_linear(x, moe["gc"], moe["gs"], moe["gt"], ids_d, out_mode=nv.OUT_SWIGLU_BF16)
    _swiglu_bits_check(o, a, h_d.cpu().numpy(), "prefill layer")
    del h_d
    # (iii) down + ordered combine on the GPU's BF16 rows, reusing the grouping as the
    # layer does, and without the reuse: the same bits
    need = max(nv.grouped_workspace_size(T, k, cfg["N_gu"], cfg["K_gu"], E, nv.OUT_SWIGLU_BF16),
               nv.grouped_workspace_size(T, k, cfg["N_d"], cfg["K_d"], E, nv.OUT_COMBINE))
    ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    nv.grouped_linear(x, moe["gc"], moe["gs"], moe["gt"], ids_d, out_mode=nv.OUT_SWIGLU_BF16,
                      out=a, workspace=ws)
    y = nv.grouped_linear(a, moe["dc"], moe["ds"], moe["dt"], ids_d, topk_w=rw_d,
                          out_mode=nv.OUT_COMBINE, rows_per_route=True, workspace=ws,
                          reuse_grouping=True)
    y2 = nv.grouped_linear(a, moe["dc"], moe["ds"], moe["dt"], ids_d, topk_w=rw_d,
                           out_mode=nv.OUT_COMBINE, rows_per_route=True)
    assert torch.equal(y, y2)
    a_bits = a.view(torch.int16).cpu().numpy().view(np.uint16)
    tsel = np.r_[0, T - 1, rng.choice(T, 62, replace=False)]
    a_sel = np.concatenate([a_bits[t * k:(t + 1) * k] for t in tsel])
    yr, yb = o.moe_down_combine(a_sel, ids[tsel], rw[tsel], moe["odc"], moe["ods"], moe["odt"])
    assert_within(y.cpu().numpy()[tsel], yr, yb, "prefill layer: down + combine")


def _w4a4_experts_case(dev, o, E, N, K, T, k, seed):
    wc, wsc, wts, oc, os_, ot = _small_experts(o, dev, E, N, K, seed)
    ids, rw = moe_routes(seed + 1, T, E, k)
    ids = ids.astype(np.int32)
    xb = act_bf16(seed + 2, T, K)
    xc, xs, xt = nv.quantize_act(to_dev_bf16(xb, dev))
    qc, qs, qt = o.quantize_bf16(xb, per_row=True)
    assert np.array_equal(xc.cpu().numpy(), qc) and np.array_equal(xs.cpu().numpy(), qs)
    assert np.array_equal(xt.cpu().numpy().view(np.uint32), qt.view(np.uint32))
    return (wc, wsc, wts, oc, os_, ot, ids, rw.astype(np.float32), (xc, xs, xt),
            (qc, qs, qt))


@pytest.mark.parametrize("E,N,K,T,k", [(8, 320, 256, 512, 2),   # GEMM path (128 per expert)
                                       (4, 320, 256, 560, 2),   # wide grouped form (280)
                                       (4, 544, 544, 560, 2),   # its persistent form, 10 steps
                                       (16, 192, 256, 4, 4)])    # streaming path (decode size)
def test_grouped_w4a4_every_output_form(dev, o, E, N, K, T, k):
    """NVFP4 activations (quantized on the device, bit-exact with the oracle) through the
    grouped call in all three output forms: per-route rows against the oracle's W4A4
    linear, SwiGLU BF16 from those rows, and the ordered combine against the oracle's
    combine of the exactly decoded rows."""
    _say(f"grouped W4A4: E={E} N={N} K={K} T={T} k={k}")
    (wc, wsc, wts, oc, os_, ot, ids, rw, (xc, xs, xt),
     (qc, qs, qt)) = _w4a4_experts_case(dev, o, E, N, K, T, k, 141 + T)
    ids_d = torch.from_numpy(ids).to(dev)
    h = nv.grouped_linear(xc, wc, wsc, wts, ids_d, x_scales=xs, x_ts=xt).cpu().numpy()
    xhat = o.dequant(qc, qs, qt, per_row=True)
    for e in np.unique(ids):
        routes = np.nonzero(ids.ravel() == e)[0]
        wdq = o.dequant(oc[e], os_[e], ot[e:e + 1], per_row=False)
        yr, b = o.linear_f64(xhat[routes // k], wdq)
        assert_within(h[routes], yr, b, f"grouped w4a4 rows, expert {e}")
    a = nv.grouped_linear(xc, wc, wsc, wts, ids_d, x_scales=xs, x_ts=xt,
                          out_mode=nv.OUT_SWIGLU_BF16)
    _swiglu_bits_check(o, a, h, f"grouped w4a4 T={T}")
    y = nv.grouped_linear(xc, wc, wsc, wts, ids_d, x_scales=xs, x_ts=xt,
                          topk_w=torch.from_numpy(rw).to(dev), out_mode=nv.OUT_COMBINE).cpu().numpy()
    yr, b = o.moe_combine_rows(np.repeat(xhat, k, axis=0), ids, rw, oc, os_, ot)
    assert_within(y, yr, b, f"grouped w4a4 T={T}: combine")
