"""Benchmark of the NVFP4 block-scaled linear layer on one MI355X.

The step (what `--steps` counts) is the decode-bucket sweep: one NVFP4 linear launch per
M in {1, 2, 4, 8, 16} on a fused-QKV-sized weight (K=4096, N=12288), BF16 activations,
fp32 output. Every launch streams a different copy of the packed weight (the copies
total > 1 GiB, well past the 256 MB Infinity Cache), so each reads its weight from HBM
as a real decode step does for each layer. Launches are replayed from a HIP graph so the
GPU runs them back to back; HIP events on the launching stream time the replays.

Printed: one JSON line. `value` is the sweep's algorithmic bytes per second; `roofline`
is the weight-streaming kernel against the 8 TB/s HBM peak; `cpu_baseline` is the CPU
oracle (plain C, float64) on the same sweep. Other workloads (the single 2048x2048
linear, the prefill GEMM, the MoE decode layer and W4A4) are timed the same way and
reported under their own keys.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

METRIC = "NVFP4 linear µs & achieved HBM GB/s (M=1..16); prefill TFLOP/s; % roofline"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 1 << 30
LEG_REPLAYS = 25  # timed graph replays per leg (--leg-replays)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(N, K):
    return N * K // 2 + N * K // 16


def linear_bytes(M, N, K):
    """Algorithmic HBM bytes of one linear launch: packed weight + tensor scale + BF16
    activations read once + fp32 output written once."""
    return weight_bytes(N, K) + 4 + 2 * M * K + 4 * M * N


class Timer:
    """Times graph replays with HIP events on the current stream."""

    def __init__(self):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def time(self, fn, reps):
        torch.cuda.synchronize()
        self.a.record()
        for _ in range(reps):
            fn()
        self.b.record()
        torch.cuda.synchronize()
        return self.a.elapsed_time(self.b) / reps  # ms per fn()

    @staticmethod
    def samples(fn, reps):
        """ms of each of `reps` back-to-back calls of fn, from one event recorded between
        consecutive calls on the current stream."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]


def timed(g, reps, per):
    """Mean ms per unit over `reps` timed replays of graph g holding `per` units, and the
    spread of the per-replay means (us)."""
    samp = [t / per * 1e3 for t in Timer.samples(g.replay, reps)]
    return float(np.mean(samp)) * 1e-3, spread(samp)


def spread(per_launch_us):
    """Median, p10 and p90 of per-launch times (each sample: one replay's mean launch)."""
    a = np.asarray(per_launch_us, dtype=np.float64)
    return {"us_med": round(float(np.median(a)), 3), "us_p10": round(float(np.percentile(a, 10)), 3),
            "us_p90": round(float(np.percentile(a, 90)), 3), "replays": int(a.size)}


def warm_until(fn, seconds):
    """Untimed repetitions of fn for about `seconds` of wall time."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()


class PowerSampler:
    """Clock and power through amdsmi (read-only queries) over a window of GPU work: the
    GFX clock sampled by a background thread (median), the average socket power from the
    energy accumulator, and the fraction of the window spent at the package power limit
    (the power-limit residency counter over the firmware's accumulation counter). Every
    figure is None where amdsmi or a metric is not available."""

    def __init__(self, period_s=0.004):
        self.period = period_s
        self.clk = []
        self.ok = False
        self.res = None

    def _state(self):
        e = self.smi.amdsmi_get_energy_count(self.h)
        m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
        return (float(e["energy_accumulator"]) * float(e["counter_resolution"]) * 1e-6,
                float(e["timestamp"]) * 1e-9, m.get("ppt_residency_acc"),
                m.get("accumulation_counter"))

    def __enter__(self):
        import threading
        try:
            import amdsmi
            self.smi = amdsmi
            amdsmi.amdsmi_init()
            self.h = amdsmi.amdsmi_get_processor_handles()[0]
            self.s0 = self._state()
            self.ok = True
        except Exception:
            return self
        self.stop = threading.Event()

        def poll():
            while not self.stop.is_set():
                try:
                    self.clk.append(float(self.smi.amdsmi_get_clock_info(
                        self.h, self.smi.AmdSmiClkType.GFX)["clk"]))
                except Exception:
                    pass
                time.sleep(self.period)
        self.th = threading.Thread(target=poll, daemon=True)
        self.th.start()
        return self

    def __exit__(self, *exc):
        if not self.ok:
            return False
        self.stop.set()
        self.th.join()
        power = resid = None
        try:
            s1 = self._state()
            if s1[1] > self.s0[1]:
                power = round((s1[0] - self.s0[0]) / (s1[1] - self.s0[1]), 1)
            if all(isinstance(v, (int, float)) for v in (self.s0[2], self.s0[3], s1[2], s1[3])) \
                    and s1[3] > self.s0[3]:
                resid = round((s1[2] - self.s0[2]) / (s1[3] - self.s0[3]), 3)
        except Exception:
            pass
        try:
            self.smi.amdsmi_shut_down()
        except Exception:
            pass
        self.res = {"gfx_clock_mhz_median": round(float(np.median(self.clk)), 1) if self.clk else None,
                    "socket_power_w_avg": power, "power_limit_residency": resid,
                    "clock_samples": len(self.clk)}
        return False


def capture(fn):
    """Records fn's launches into a HIP graph (torch's capture on a side stream)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the allocator / library outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def quantize_weight(nv, w, dev):
    wd = torch.from_numpy(w).to(dev)
    c, s, t = nv.quantize_act(wd, per_tensor=True)
    del wd
    return c, s, t


def copies(c, s, n):
    return [(c.clone(), s.clone()) for _ in range(n)]


def to_bf16(xb, dev):
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).to(dev).view(torch.bfloat16)


# ---------------------------------------------------------------------------------------
def bench_decode_sweep(nv, dev, steps, warmup):
    from synth import WORKLOADS, act_bf16, weight_f32
    cfg = WORKLOADS["decode_sweep"]
    N, K, Ms = cfg["N"], cfg["K"], cfg["Ms"]
    c, s, t = quantize_weight(nv, weight_f32(cfg["w_seed"], N, K), dev)
    R = max(len(Ms), math.ceil(ROTATE_BYTES / weight_bytes(N, K)))
    R = len(Ms) * math.ceil(R / len(Ms))
    W = copies(c, s, R)
    xs = {M: to_bf16(act_bf16(cfg["x_seed_base"] + M, M, K), dev) for M in Ms}
    ys = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms}
    steps_per_graph = R // len(Ms)

    def sweep_steps():
        j = 0
        for _ in range(steps_per_graph):
            for M in Ms:
                nv.linear(xs[M], W[j][0], W[j][1], t, out=ys[M])
                j += 1

    # eager reference for the replay check
    ref = {M: nv.linear(xs[M], c, s, t).clone() for M in Ms}
    g = capture(sweep_steps)
    g.replay()
    torch.cuda.synchronize()
    for M in Ms:
        assert torch.equal(ys[M], ref[M]), f"graph replay differs from eager at M={M}"
    timer = Timer()
    reps_w = max(1, math.ceil(warmup / steps_per_graph))
    reps = max(1, math.ceil(steps / steps_per_graph))
    timer.time(g.replay, reps_w)
    ms_graph = timer.time(g.replay, reps)
    ms_step = ms_graph / steps_per_graph
    timed_steps = reps * steps_per_graph
    step_bytes = sum(linear_bytes(M, N, K) for M in Ms)

    # per-M launches (same kernel, one M at a time), for the per-bucket table
    per_m = {}
    for M in Ms:
        def one_m(M=M):
            for j in range(R):
                nv.linear(xs[M], W[j][0], W[j][1], t, out=ys[M])
        gm = capture(one_m)
        timer.time(gm.replay, 1)
        # each replay launches the kernel R times, each on its own weight copy
        samp = [t / R * 1e3 for t in Timer.samples(gm.replay, max(25, reps))]
        ms = float(np.mean(samp)) * 1e-3
        b = linear_bytes(M, N, K)
        per_m[str(M)] = {"us": round(ms * 1e3, 3), **spread(samp), "launches_per_replay": R,
                         "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                         "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "bytes": b}
        del gm
    del g
    probe = read_probe_roof(nv, dev, linear_bytes(1, N, K), timer)
    for M in Ms:
        per_m[str(M)]["frac_read_probe"] = round(per_m[str(M)]["GBps"] / probe["GBps"], 4)
    return dict(N=N, K=K, Ms=Ms, R=R, ms_step=ms_step, step_bytes=step_bytes,
                timed_steps=timed_steps, per_m=per_m, launches_per_step=len(Ms), probe=probe)


def bench_decode_prefetch(nv, dev):
    """A chain of decode launches over distinct weights (the sweep's K=4096, N=12288 weight
    in 40 copies, M cycling through 1, 2, 4, 8, 16), as consecutive layers of a decode step
    run: without prefetch, and with each next layer's weight (codes and scales) read into
    the caches by nvfp4_prefetch on a second stream while the current layer runs (forked
    before it, joined before the next layer). Per-layer time over the chain."""
    from synth import WORKLOADS, act_bf16, weight_f32
    cfg = WORKLOADS["decode_sweep"]
    N, K, Ms = cfg["N"], cfg["K"], cfg["Ms"]
    c, s, t = quantize_weight(nv, weight_f32(cfg["w_seed"], N, K), dev)
    R = len(Ms) * math.ceil(max(len(Ms), math.ceil(ROTATE_BYTES / weight_bytes(N, K))) / len(Ms))
    W = copies(c, s, R)
    xs = {M: to_bf16(act_bf16(cfg["x_seed_base"] + M, M, K), dev) for M in Ms}
    ys = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms}
    side = torch.cuda.Stream()
    ref = {M: nv.linear(xs[M], c, s, t).clone() for M in Ms}

    def chain(workgroups):
        for j in range(R):
            M = Ms[j % len(Ms)]
            if workgroups:
                nxt = W[(j + 1) % R]
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    nv.prefetch(nxt[0], workgroups)
                    nv.prefetch(nxt[1], workgroups)
            nv.linear(xs[M], W[j][0], W[j][1], t, out=ys[M])
            if workgroups:
                torch.cuda.current_stream().wait_stream(side)
    out = {"layers_per_replay": R, "bytes_per_layer_avg": sum(linear_bytes(M, N, K) for M in Ms) // len(Ms)}
    for wg in (0, 128, 256, 512):
        g = capture(lambda: chain(wg))
        g.replay()
        torch.cuda.synchronize()
        for M in Ms:
            assert torch.equal(ys[M], ref[M]), f"prefetch changed a result at M={M}"
        warm_until(g.replay, 0.05)
        ms, sp = timed(g, LEG_REPLAYS, R)
        key = "no_prefetch" if wg == 0 else f"prefetch_wg{wg}"
        out[key] = {"us_per_layer": round(ms * 1e3, 3), **sp,
                    "GBps": round(out["bytes_per_layer_avg"] / (ms * 1e-3) / 1e9, 1)}
        del g
    # eager launches (host-enqueued, no graph), where the host leaves gaps between layers
    for wg in (0, 256):
        chain(wg)
        torch.cuda.synchronize()
        samp = []
        for _ in range(5):
            t0 = time.perf_counter()
            chain(wg)
            torch.cuda.synchronize()
            samp.append((time.perf_counter() - t0) / R * 1e6)
        key = "eager_no_prefetch" if wg == 0 else f"eager_prefetch_wg{wg}"
        out[key] = {"us_per_layer": round(float(np.median(samp)), 3)}
    return out


def read_probe_roof(nv, dev, nbytes, timer):
    """The measured single-launch read roof: the library's plain streaming-read kernel over
    buffers of the M=1 launch's algorithmic size, rotated over >= 1 GiB like the weights,
    timed in the same way; the best of its launch shapes."""
    nbytes = (nbytes + 15) // 16 * 16
    R = max(2, math.ceil(ROTATE_BYTES / nbytes))
    bufs = [torch.full((nbytes,), 1, dtype=torch.uint8, device=dev) for _ in range(R)]
    sink = torch.zeros((1,), dtype=torch.int32, device=dev)
    best = None
    for u in (1, 2, 4, 8, 16):
        def run(u=u):
            for b in bufs:
                nv.read_probe(b, u, sink)
        g = capture(run)
        timer.time(g.replay, 1)
        ms = min(timer.time(g.replay, 3) for _ in range(3)) / R
        if best is None or ms < best[0]:
            best = (ms, u)
        del g
    ms, u = best
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"bytes": nbytes, "us": round(ms * 1e3, 3), "GBps": round(gbps, 1),
            "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4), "loads_per_thread": u,
            "kernel": "read_probe (plain streaming read, one launch per buffer)"}


def bench_single(nv, dev):
    from synth import WORKLOADS, act_bf16, weight_f32
    cfg = WORKLOADS["single_linear"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    c, s, t = quantize_weight(nv, weight_f32(cfg["w_seed"], N, K), dev)
    R = math.ceil(ROTATE_BYTES / weight_bytes(N, K))
    W = copies(c, s, R)
    x = to_bf16(act_bf16(cfg["x_seed"], M, K), dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)

    def run():
        for j in range(R):
            nv.linear(x, W[j][0], W[j][1], t, out=y)
    g = capture(run)
    timer = Timer()
    timer.time(g.replay, 1)
    ms, sp = timed(g, LEG_REPLAYS, R)
    b = linear_bytes(M, N, K)
    del g
    # a launch this small is latency: the plain streaming read of the same bytes, timed the
    # same way, is its measured floor
    probe = read_probe_roof(nv, dev, b, timer)
    gbps = b / (ms * 1e-3) / 1e9
    return {"workload": "M=1 K=2048 N=2048", "us": round(ms * 1e3, 3), **sp,
            "launches_per_replay": R,
            "GBps": round(gbps, 1), "bytes": b, "read_probe_us": probe["us"],
            "frac_read_probe": round(gbps / probe["GBps"], 4)}


def bench_prefill(nv, dev):
    from synth import WORKLOADS, act_bf16, weight_f32
    cfg = WORKLOADS["prefill"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    c, s, t = quantize_weight(nv, weight_f32(cfg["w_seed"], N, K), dev)
    R = 8
    W = copies(c, s, R)
    x = to_bf16(act_bf16(cfg["x_seed"], M, K), dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)

    def run():
        for j in range(R):
            nv.linear(x, W[j][0], W[j][1], t, out=y)
    g = capture(run)
    timer = Timer()
    warm_until(g.replay, 0.15)  # the clock settles under sustained MFMA load
    ms, sp = timed(g, LEG_REPLAYS, R)
    # clock and power under the same load, back-to-back replays outside the timed region
    with PowerSampler() as ps:
        for _ in range(max(1, int(0.3 / (ms * R * 1e-3)))):
            g.replay()
        torch.cuda.synchronize()
    flops = 2.0 * M * N * K
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": "M=2048 K=4096 N=14336", "us": round(ms * 1e3, 2), **sp,
            "launches_per_replay": R, "TFLOPs": round(tf, 1),
            "frac_bf16_mfma": round(tf / BF16_PEAK_TFLOPS, 4), "flop": flops,
            "clock_power": ps.res}


def bench_w4a4(nv, dev):
    from synth import WORKLOADS, act_bf16, weight_f32
    cfg = WORKLOADS["w4a4"]
    N, K = cfg["N"], cfg["K"]
    c, s, t = quantize_weight(nv, weight_f32(cfg["w_seed"], N, K), dev)
    R = math.ceil(ROTATE_BYTES / weight_bytes(N, K))
    W = copies(c, s, R)
    out = {}
    timer = Timer()
    for M in cfg["Ms"]:
        x = to_bf16(act_bf16(cfg["x_seed_base"] + M, M, K), dev)
        xc, xs_, xt = nv.quantize_act(x)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        reps_in = R if M <= 16 else 8

        def run():
            for j in range(reps_in):
                nv.quantize_act(x, codes=xc, scales=xs_, ts=xt)
                nv.linear(xc, W[j][0], W[j][1], t, x_scales=xs_, x_ts=xt, out=y)
        g = capture(run)
        warm_until(g.replay, 0.1)
        ms, sp = timed(g, LEG_REPLAYS, reps_in)
        b = weight_bytes(N, K) + 4 + M * (2 * K + K // 2 + K // 16 + 4) + M * (K // 2 + K // 16 + 4) + 4 * M * N
        fl = 2.0 * M * N * K
        out[str(M)] = {"us_quantize_plus_linear": round(ms * 1e3, 3), **sp,
                       "pairs_per_replay": reps_in,
                       "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                       "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 2)}
        del g
    return out


def bench_w4a4_probe(nv, dev):
    """The read probe for the W4A4 weight's bytes (K = N = 4096: 9.4 MB), timed as the
    launches above: the single-launch floor beside the quantize + linear figures."""
    from synth import WORKLOADS
    cfg = WORKLOADS["w4a4"]
    p = read_probe_roof(nv, dev, weight_bytes(cfg["N"], cfg["K"]), Timer())
    return {"bytes": p["bytes"], "us": p["us"], "GBps": p["GBps"]}


def bench_w4a4_in_call(nv, dev):
    """W4A4 for one row two ways on the W4A4 weight (K = N = 4096): the quantizer launch
    followed by the NVFP4-activation linear, and the one-launch form that quantizes the
    row inside the weight-streaming kernel (bit for bit the same result)."""
    from synth import WORKLOADS, act_bf16, weight_f32
    cfg = WORKLOADS["w4a4"]
    N, K = cfg["N"], cfg["K"]
    c, s, t = quantize_weight(nv, weight_f32(cfg["w_seed"], N, K), dev)
    R = math.ceil(ROTATE_BYTES / weight_bytes(N, K))
    W = copies(c, s, R)
    out = {}
    timer = Timer()
    for M in (1,):
        x = to_bf16(act_bf16(cfg["x_seed_base"] + M, M, K), dev)
        xc, xs_, xt = nv.quantize_act(x)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)

        def two_calls():
            for j in range(R):
                nv.quantize_act(x, codes=xc, scales=xs_, ts=xt)
                nv.linear(xc, W[j][0], W[j][1], t, x_scales=xs_, x_ts=xt, out=y)

        def in_call():
            for j in range(R):
                nv.linear(x, W[j][0], W[j][1], t, out=y, quantize_x=True)
        rec = {}
        for name, fn in (("us_two_calls", two_calls), ("us_in_call", in_call)):
            g = capture(fn)
            warm_until(g.replay, 0.05)
            ms, sp = timed(g, LEG_REPLAYS, R)
            rec[name] = round(ms * 1e3, 3)
            rec[name + "_p10_p90"] = [sp["us_p10"], sp["us_p90"]]
            del g
        out[str(M)] = rec
    return out


def bench_moe(nv, dev):
    from synth import WORKLOADS, act_bf16, moe_expert_weights, moe_routes
    cfg = WORKLOADS["moe_decode"]
    E, T, k = cfg["E"], cfg["T"], cfg["top_k"]
    gc, gs, gt, dc, ds, dt = [], [], [], [], [], []
    for e in range(E):
        gu, dn = moe_expert_weights(cfg["w_seed"], e, cfg["N_gu"], cfg["K_gu"], cfg["N_d"], cfg["K_d"])
        c, s, t = quantize_weight(nv, gu, dev); gc.append(c); gs.append(s); gt.append(t)
        c, s, t = quantize_weight(nv, dn, dev); dc.append(c); ds.append(s); dt.append(t)
    sets = [(torch.stack(gc), torch.stack(gs), torch.cat(gt), torch.stack(dc), torch.stack(ds), torch.cat(dt))]
    per_set = sum(x.numel() for x in sets[0][:2]) + sum(x.numel() for x in sets[0][3:5])
    R = max(1, math.ceil(ROTATE_BYTES / per_set))
    sets += [tuple(x.clone() for x in sets[0]) for _ in range(R - 1)]
    ids, rw = moe_routes(cfg["route_seed"], T, E, k)
    ids_d = torch.from_numpy(ids).to(dev)
    rw_d = torch.from_numpy(rw).to(dev)
    x = to_bf16(act_bf16(cfg["x_seed"], T, cfg["K_gu"]), dev)
    a = torch.empty((T * k, cfg["N_gu"] // 2), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, cfg["N_d"]), dtype=torch.float32, device=dev)
    # one workspace for the layer: the down call reuses the gate_up call's route grouping
    ws = torch.empty(max(nv.grouped_workspace_size(T, k, cfg["N_gu"], cfg["K_gu"], E, nv.OUT_SWIGLU_BF16),
                         nv.grouped_workspace_size(T, k, cfg["N_d"], cfg["K_d"], E, nv.OUT_COMBINE)),
                     dtype=torch.uint8, device=dev)

    def run():
        for st in sets:
            nv.grouped_linear(x, st[0], st[1], st[2], ids_d, out_mode=nv.OUT_SWIGLU_BF16, out=a,
                              workspace=ws)
            nv.grouped_linear(a, st[3], st[4], st[5], ids_d, topk_w=rw_d, out_mode=nv.OUT_COMBINE,
                              rows_per_route=True, out=y, workspace=ws, reuse_grouping=True)
    g = capture(run)
    timer = Timer()
    timer.time(g.replay, 1)
    ms, sp = timed(g, LEG_REPLAYS, R)
    D = len(np.unique(ids))
    per_expert = weight_bytes(cfg["N_gu"], cfg["K_gu"]) + weight_bytes(cfg["N_d"], cfg["K_d"]) + 8
    b = D * per_expert + T * cfg["K_gu"] * 2 + T * cfg["N_d"] * 4
    return {"workload": "128 experts, gate_up 2048->1536 + down 768->2048, 16 tokens, top-8",
            "distinct_experts": D, "us_layer": round(ms * 1e3, 2), **sp, "layers_per_replay": R,
            "GBps": round(b / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "bytes": b}


def bench_moe_prefill(nv, dev):
    """The MoE layer at prompt size: 4096 tokens over the same 128 experts, top-8 (the
    grouped GEMM path: each routed expert read once per batch)."""
    from synth import WORKLOADS, act_bf16, moe_expert_weights, moe_routes
    cfg = WORKLOADS["moe_decode"]
    E, k = cfg["E"], cfg["top_k"]
    T = 4096
    gc, gs, gt, dc, ds, dt = [], [], [], [], [], []
    for e in range(E):
        gu, dn = moe_expert_weights(cfg["w_seed"], e, cfg["N_gu"], cfg["K_gu"], cfg["N_d"], cfg["K_d"])
        c, s, t = quantize_weight(nv, gu, dev); gc.append(c); gs.append(s); gt.append(t)
        c, s, t = quantize_weight(nv, dn, dev); dc.append(c); ds.append(s); dt.append(t)
    st = (torch.stack(gc), torch.stack(gs), torch.cat(gt), torch.stack(dc), torch.stack(ds), torch.cat(dt))
    ids, rw = moe_routes(cfg["route_seed"] + 1, T, E, k)
    ids_d = torch.from_numpy(ids).to(dev)
    rw_d = torch.from_numpy(rw).to(dev)
    x = to_bf16(act_bf16(cfg["x_seed"] + 1, T, cfg["K_gu"]), dev)
    a = torch.empty((T * k, cfg["N_gu"] // 2), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, cfg["N_d"]), dtype=torch.float32, device=dev)
    ws = torch.empty(max(nv.grouped_workspace_size(T, k, cfg["N_gu"], cfg["K_gu"], E, nv.OUT_SWIGLU_BF16),
                         nv.grouped_workspace_size(T, k, cfg["N_d"], cfg["K_d"], E, nv.OUT_COMBINE)),
                     dtype=torch.uint8, device=dev)

    def run():
        nv.grouped_linear(x, st[0], st[1], st[2], ids_d, out_mode=nv.OUT_SWIGLU_BF16, out=a,
                          workspace=ws)
        nv.grouped_linear(a, st[3], st[4], st[5], ids_d, topk_w=rw_d, out_mode=nv.OUT_COMBINE,
                          rows_per_route=True, out=y, workspace=ws, reuse_grouping=True)
    g = capture(run)
    timer = Timer()
    warm_until(g.replay, 0.15)
    ms, sp = timed(g, LEG_REPLAYS, 1)
    R = T * k
    flops = 2.0 * R * (cfg["N_gu"] * cfg["K_gu"] + cfg["N_d"] * cfg["K_d"])
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": f"{T} tokens, 128 experts, top-8, gate_up 2048->1536 + down 768->2048",
            "us_layer": round(ms * 1e3, 2), **sp, "TFLOPs": round(tf, 1),
            "frac_bf16_mfma": round(tf / BF16_PEAK_TFLOPS, 4), "flop": flops}


def hbm_copy_probe(dev):
    """Device-to-device copy of 1 GiB: measured read+write bandwidth of a plain copy."""
    n = 1 << 29  # int16 elements = 1 GiB
    a = torch.empty(n, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    timer = Timer()
    timer.time(lambda: b.copy_(a), 2)
    ms = timer.time(lambda: b.copy_(a), 5)
    return round(2 * a.numel() * 2 / (ms * 1e-3) / 1e9, 1)


STREAM_SOURCES = ("nvfp4_block_scaled_linear_amd/csrc/stream.hip",
                  "nvfp4_block_scaled_linear_amd/csrc/device.hpp",
                  "nvfp4_block_scaled_linear_amd/csrc/kernels.hpp")
PMC_SUMMARY = "profiles/stream_dense_decode_sweep_pmc.txt"


def stream_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in STREAM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the streaming kernel over the decode sweep, from the
    committed counter summary; None when the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, PMC_SUMMARY)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != stream_source_hash():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def summarize_rocprof(out_dir, calib_bytes):
    """Prints a short text summary of rocprofv3 output under out_dir: per-kernel dispatch
    counts and mean durations from --kernel-trace --stats; per-kernel median, p10 and p90
    of the dispatch durations from the kernel trace itself; and per-kernel mean
    FETCH_SIZE / WRITE_SIZE from --pmc runs, scaled by what the same counters read for
    the 1 GiB device copy (calib_bytes read and written)."""
    import csv
    import glob
    traces = sorted(glob.glob(os.path.join(out_dir, "**", "*kernel_trace.csv"), recursive=True))
    for f in traces:
        durs = {}
        with open(f) as fh:
            for r in csv.DictReader(fh):
                d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                durs.setdefault(r["Kernel_Name"], []).append(d)
        print(f"dispatch durations (us) from {os.path.relpath(f, out_dir)}: median p10 p90")
        for name, d in sorted(durs.items(), key=lambda kv: -len(kv[1])):
            a = np.asarray(d)
            print(f"  {name[:110]:110s} n {a.size:6d} med {np.median(a):9.3f} "
                  f"p10 {np.percentile(a, 10):9.3f} p90 {np.percentile(a, 90):9.3f}")
    stats = sorted(glob.glob(os.path.join(out_dir, "**", "*kernel_stats.csv"), recursive=True))
    for f in stats:
        print(f"kernel stats: {os.path.relpath(f, out_dir)}")
        with open(f) as fh:
            for r in csv.DictReader(fh):
                print(f"  {r['Name'][:110]:110s} calls {int(r['Calls']):6d} "
                      f"avg_us {float(r['AverageNs']) / 1e3:9.3f} min_us {float(r['MinNs']) / 1e3:9.3f} "
                      f"max_us {float(r['MaxNs']) / 1e3:9.3f}")
    pmc = sorted(glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True))
    per = {}
    for f in pmc:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (r["Kernel_Name"], r["Counter_Name"])
                d = per.setdefault(key, {})
                d[r["Dispatch_Id"] + f] = d.get(r["Dispatch_Id"] + f, 0.0) + float(r["Counter_Value"])
    if not per:
        return
    means = {k: (sum(v.values()) / len(v), len(v)) for k, v in per.items()}
    # calibration: the largest single dispatch outside this library is the 1 GiB device
    # copy (it reads and writes calib_bytes)
    factors = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        cands = [(k[0], max(v.values())) for k, v in per.items() if k[1] == ctr
                 and "nvfp4" not in k[0]]
        if cands:
            kname, kib = max(cands, key=lambda c: c[1])
            if kib * 1024 > 0.3 * calib_bytes:
                factors[ctr] = calib_bytes / (kib * 1024)
                print(f"calibration {ctr}: a {calib_bytes}-byte device copy counts {kib:.1f} KiB "
                      f"-> factor {factors[ctr]:.4f} ({kname[:60]})")
    for (kname, ctr), (kib, n) in sorted(means.items()):
        f = factors.get(ctr)
        scaled = f"{kib * 1024 * f:14.0f} B" if f else "   (uncalibrated)"
        print(f"  {ctr:10s} {kname[:100]:100s} dispatches {n:6d} mean {kib:12.1f} KiB {scaled}")
    # per kernel: scaled FETCH + WRITE per dispatch (the HBM bytes one launch moves)
    if "FETCH_SIZE" in factors and "WRITE_SIZE" in factors:
        names = sorted({k for k, c in means if c == "FETCH_SIZE"} & {k for k, c in means if c == "WRITE_SIZE"})
        for kname in names:
            b = sum(means[(kname, c)][0] * 1024 * factors[c] for c in ("FETCH_SIZE", "WRITE_SIZE"))
            print(f"  traffic {kname[:100]:100s} {b:14.0f} B per dispatch")
    # the streaming kernel over every launch of the run (each decode M launches equally often)
    if "FETCH_SIZE" in factors and "WRITE_SIZE" in factors:
        tot = 0.0
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = [x for (kname, c), v in per.items() if c == ctr and "stream_dense" in kname
                    for x in v.values()]
            if vals:
                tot += sum(vals) / len(vals) * 1024 * factors[ctr]
        print(f"traffic_bytes_per_launch: {tot:.0f}")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _clock(fn, min_s=0.3, max_reps=1000):
    """Seconds per call of fn, repeated for at least min_s of wall time."""
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= min_s or n >= max_reps:
            return el / n


def cpu_baseline(decode):
    """The CPU oracle (the code the tests check against, not tuned for speed) on the same
    workloads, on the host's threads: the headline figure on the full decode sweep
    (dequantize the weight once, then the float64 linear for M = 1, 2, 4, 8, 16), and per
    workload the quantizer and the linear timed separately, on the sample stated."""
    import oracle
    from synth import WORKLOADS, act_bf16, moe_expert_weights, moe_routes, weight_f32
    o = oracle.Oracle()
    cores = o.num_threads()
    per = {}
    # decode sweep (the headline): weight quantize, then dequantize + linear per step
    cfg = WORKLOADS["decode_sweep"]
    N, K = cfg["N"], cfg["K"]
    w = weight_f32(cfg["w_seed"], N, K)
    t_q = _clock(lambda: o.quantize(w, per_row=False), min_s=0.5, max_reps=3)
    oc, os_, ot = o.quantize(w, per_row=False)
    xs = {M: o.bf16_to_f64(act_bf16(cfg["x_seed_base"] + M, M, K)) for M in cfg["Ms"]}
    t_dq = _clock(lambda: o.dequant(oc, os_, ot, per_row=False), min_s=0.5, max_reps=5)
    wdq = o.dequant(oc, os_, ot, per_row=False)
    t_lin = {str(M): _clock(lambda M=M: o.linear_f64(xs[M], wdq), min_s=1.0) for M in cfg["Ms"]}
    per_step = t_dq + sum(t_lin.values())
    per["decode_sweep"] = {"quantize_weight_s": round(t_q, 4), "dequantize_s": round(t_dq, 4),
                           "linear_s": {m: round(v, 5) for m, v in t_lin.items()},
                           "sample": "full (12288x4096 weight, all five M)"}
    # single linear
    cfg = WORKLOADS["single_linear"]
    w = weight_f32(cfg["w_seed"], cfg["N"], cfg["K"])
    t_q = _clock(lambda: o.quantize(w, per_row=False))
    q = o.quantize(w, per_row=False)
    xb = act_bf16(cfg["x_seed"], cfg["M"], cfg["K"])
    t_lin = _clock(lambda: o.linear(xb, *q))
    per["single_linear"] = {"quantize_weight_s": round(t_q, 5), "linear_s": round(t_lin, 5),
                            "sample": "full"}
    # prefill: the weight quantize in full, the linear on 16 of the 2048 rows
    cfg = WORKLOADS["prefill"]
    w = weight_f32(cfg["w_seed"], cfg["N"], cfg["K"])
    t_q = _clock(lambda: o.quantize(w, per_row=False), min_s=0.5, max_reps=2)
    q = o.quantize(w, per_row=False)
    del w
    wdq = o.dequant(*q, per_row=False)
    rows = 16
    xb = o.bf16_to_f64(act_bf16(cfg["x_seed"], rows, cfg["K"]))
    t_lin = _clock(lambda: o.linear_f64(xb, wdq), min_s=1.0, max_reps=3)
    per["prefill"] = {"quantize_weight_s": round(t_q, 4),
                      "linear_s_per_row": round(t_lin / rows, 5),
                      "linear_s_full_estimate": round(t_lin / rows * cfg["M"], 2),
                      "sample": f"linear on {rows} of {cfg['M']} rows (time per row scaled to all)"}
    del wdq
    # W4A4: activation quantize per row and the W4A4 linear
    cfg = WORKLOADS["w4a4"]
    w = weight_f32(cfg["w_seed"], cfg["N"], cfg["K"])
    qw = o.quantize(w, per_row=False)
    wdq = o.dequant(*qw, per_row=False)
    rec = {}
    for M in cfg["Ms"]:
        xb = act_bf16(cfg["x_seed_base"] + M, M, cfg["K"])
        t_qa = _clock(lambda: o.quantize_bf16(xb, per_row=True), min_s=0.2)
        xq = o.quantize_bf16(xb, per_row=True)
        m_s = min(M, 16)
        t_l = _clock(lambda: o.linear_w4a4(xq[0][:m_s], xq[1][:m_s], xq[2][:m_s], *qw, wdq=wdq),
                     min_s=0.3)
        rec[str(M)] = {"quantize_act_s": round(t_qa, 6), "linear_s_per_row": round(t_l / m_s, 6),
                       "sample": "full" if m_s == M else f"linear on {m_s} of {M} rows"}
    per["w4a4"] = rec
    # MoE decode layer: the oracle's stages on the 16 tokens (each routed expert
    # dequantized once); expert weights quantized for the routed experts only
    cfg = WORKLOADS["moe_decode"]
    E, T, k = cfg["E"], cfg["T"], cfg["top_k"]
    ids, rw = moe_routes(cfg["route_seed"], T, E, k)
    used = sorted(set(int(e) for e in np.unique(ids)))
    shape = (cfg["N_gu"], cfg["K_gu"], cfg["N_d"], cfg["K_d"])
    gq, dq = {}, {}
    t0 = time.perf_counter()
    for e in used:
        gu, dn = moe_expert_weights(cfg["w_seed"], e, *shape)
        gq[e] = o.quantize(gu, per_row=False)
        dq[e] = o.quantize(dn, per_row=False)
    t_q = time.perf_counter() - t0

    def stack(qs, i, shp, dt):
        out = np.zeros((E,) + shp, dt)
        for e, qq in qs.items():
            out[e] = qq[i] if i < 2 else qq[2][0]
        return out
    gc = stack(gq, 0, (cfg["N_gu"], cfg["K_gu"] // 2), np.uint8)
    gs = stack(gq, 1, (cfg["N_gu"], cfg["K_gu"] // 16), np.uint8)
    gt = np.array([gq[e][2][0] if e in gq else 0.0 for e in range(E)], np.float32)
    dc = stack(dq, 0, (cfg["N_d"], cfg["K_d"] // 2), np.uint8)
    ds = stack(dq, 1, (cfg["N_d"], cfg["K_d"] // 16), np.uint8)
    dt = np.array([dq[e][2][0] if e in dq else 0.0 for e in range(E)], np.float32)
    xb = act_bf16(cfg["x_seed"], T, cfg["K_gu"])

    def layer():
        h, _ = o.moe_gate_up(xb, ids, gc, gs, gt)
        a = o.bf16_round_array(o.swiglu(h))
        o.moe_down_combine(a, ids, rw, dc, ds, dt)
    t_layer = _clock(layer, min_s=1.0, max_reps=3)
    per["moe_decode"] = {"quantize_weights_s": round(t_q, 3), "layer_s": round(t_layer, 4),
                         "sample": f"full layer; weights quantized for the {len(used)} routed experts"}
    return {"value": round(decode["step_bytes"] / per_step / 1e9, 3), "unit": "GB/s",
            "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"full decode sweep: dequantize the 12288x4096 weight once, then the "
                      f"float64 linear for M=1,2,4,8,16 ({per_step:.3f} s per sweep) on {cores} "
                      f"OpenMP threads ({os.cpu_count()} host CPUs visible)",
            "per_config": per}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", choices=["all", "decode", "single", "prefill", "w4a4", "moe",
                                       "moe_prefill", "prefetch"],
                    default="all", help="run the decode sweep plus one other workload (all: every one)")
    ap.add_argument("--legs", default=None,
                    help="comma-separated workloads to run besides the decode sweep "
                         "(single, prefill, w4a4, moe, moe_prefill, prefetch); overrides --only")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode sweep (profiling runs of other workloads; the line "
                         "then has no headline value)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--leg-replays", type=int, default=25,
                    help="timed graph replays of each leg other than the decode sweep")
    ap.add_argument("--copy-probe", action="store_true", help="also time a 1 GiB device copy")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="print a text summary of rocprofv3 output under DIR and exit")
    args = ap.parse_args()
    globals()["LEG_REPLAYS"] = max(5, args.leg_replays)
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, calib_bytes=1 << 30)
        print(f"kernel_sources_sha256: {stream_source_hash()}")
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import nvfp4_block_scaled_linear_amd as nv
    if not os.path.exists(nv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nv.load_library()

    legs = set(args.legs.split(",")) if args.legs else None
    if args.no_decode:
        rec = {"metric": METRIC, "value": None, "note": "decode sweep skipped (--no-decode)"}
        run_legs(nv, dev, args, legs, rec)
        print(json.dumps(rec), flush=True)
        return
    log("decode sweep ...")
    d = bench_decode_sweep(nv, dev, args.steps, args.warmup)
    value = d["step_bytes"] / (d["ms_step"] * 1e-3) / 1e9
    achieved = value  # one kernel (the weight-streaming kernel) makes every launch of the step
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": d["timed_steps"],
        "steps_requested": args.steps,  # timed in whole replays of the sweep graph
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode bucket sweep: NVFP4 linear K=4096 N=12288, one launch per "
                               "M in {1,2,4,8,16} per step, BF16 activations, fp32 out; weight "
                               f"rotated over {d['R']} copies ({d['R'] * weight_bytes(d['N'], d['K']) / 2**30:.2f} GiB) "
                               "so every launch streams it from HBM",
                   "global_batch": 31, "parallelism": "none (one GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "stream_dense (weight-streaming MFMA kernel)",
                     "avg_launch_us": round(d["ms_step"] * 1e3 / d["launches_per_step"], 3),
                     "bytes_per_launch_avg": d["step_bytes"] // d["launches_per_step"],
                     "achievable": d["probe"]["GBps"],
                     "frac_achievable": round(achieved / d["probe"]["GBps"], 4)},
        "per_m": d["per_m"],
        "read_probe": d["probe"],
    }
    run_legs(nv, dev, args, legs, rec)
    if args.copy_probe or (args.only == "all" and legs is None):
        rec["hbm_copy_GBps"] = hbm_copy_probe(dev)
    if not args.no_cpu:
        log("cpu oracle baseline ...")
        rec["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(rec), flush=True)


def run_legs(nv, dev, args, legs, rec):
    """The workloads besides the decode sweep, each under its own key of rec."""
    def want(name):
        return name in legs if legs is not None else args.only in ("all", name)
    if want("single"):
        log("single linear ...")
        rec["single_linear"] = bench_single(nv, dev)
    if want("prefill"):
        log("prefill ...")
        rec["prefill"] = bench_prefill(nv, dev)
    if want("w4a4"):
        log("w4a4 ...")
        rec["w4a4"] = bench_w4a4(nv, dev)
        rec["w4a4_in_call_quantize"] = bench_w4a4_in_call(nv, dev)
        rec["w4a4_weight_read_probe"] = bench_w4a4_probe(nv, dev)
    if want("moe"):
        log("moe ...")
        rec["moe"] = bench_moe(nv, dev)
    if want("moe_prefill"):
        log("moe prefill ...")
        rec["moe_prefill"] = bench_moe_prefill(nv, dev)
    if want("prefetch"):
        log("decode chain with next-weight prefetch ...")
        rec["decode_prefetch"] = bench_decode_prefetch(nv, dev)
    if args.no_decode and args.copy_probe:
        rec["hbm_copy_GBps"] = hbm_copy_probe(dev)


if __name__ == "__main__":
    main()
