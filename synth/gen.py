"""Seeded input generators (no NVFP4 arithmetic here; see the package docstring).

Workload recipes follow the NVFP4 linear-layer problem statement used throughout
this repository: weights W ~ N(0, 0.02) in fp32 (0.02 is the standard deviation),
activations ~ N(0, 1) rounded to BF16, MoE routes drawn uniformly without
replacement per token, router weights a softmax of N(0, 1) logits over the
token's chosen experts.

The random streams live in ``synth.c`` (compiled to ``libsynth.so`` next to this
file by ``build_lib``); this file only shapes them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build_lib() -> str:
    """Compile synth.c into libsynth.so with gcc (plain C, -O2, no fast-math)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-fno-fast-math",
                           "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build_lib()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.synth_u64.argtypes = [u64, u64, i64, vp]
        lib.synth_uniform.argtypes = [u64, u64, i64, vp]
        lib.synth_normal_f32.argtypes = [u64, i64, ctypes.c_double, vp]
        lib.synth_normal_f64.argtypes = [u64, i64, vp]
        for f in (lib.synth_u64, lib.synth_uniform, lib.synth_normal_f32, lib.synth_normal_f64):
            f.restype = None
        _lib = lib
    return _lib


def _key(seed: int, stream: int) -> int:
    # distinct (seed, stream) pairs map to distinct 64-bit stream keys
    return (((int(seed) & 0xFFFFFFFF) << 32) ^ ((int(stream) & 0xFFFFFFFF) * 0x2545F491)) & (2**64 - 1)


def splitmix64(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs start..start+n-1 of the SplitMix64 stream keyed by (seed, stream)."""
    out = np.empty(n, dtype=np.uint64)
    _load().synth_u64(_key(seed, stream), start, n, out.ctypes.data)
    return out


def uniform(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    """Uniform float64 in [0, 1) with 53 random bits."""
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform(_key(seed, stream), start, n, out.ctypes.data)
    return out


def normal(seed: int, stream: int, n: int) -> np.ndarray:
    """Standard normal float64 via Box-Muller over consecutive uniform pairs."""
    out = np.empty(n, dtype=np.float64)
    _load().synth_normal_f64(_key(seed, stream), n, out.ctypes.data)
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (round to nearest, ties to even), returned as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def weight_f32(seed: int, N: int, K: int, std: float = 0.02, stream: int = 0) -> np.ndarray:
    """fp32 weight [N][K]: N(0, std^2) drawn in float64, rounded once to float32."""
    out = np.empty((N, K), dtype=np.float32)
    _load().synth_normal_f32(_key(seed, stream), N * K, float(std), out.ctypes.data)
    return out


def act_bf16(seed: int, M: int, K: int, stream: int = 1) -> np.ndarray:
    """BF16 activation rows [M][K] as uint16 bits: N(0,1) float64 -> float32 -> BF16 RNE."""
    x = np.empty((M, K), dtype=np.float32)
    _load().synth_normal_f32(_key(seed, stream), M * K, 1.0, x.ctypes.data)
    return f32_to_bf16_bits(x).reshape(M, K)


def moe_routes(seed: int, T: int, E: int, top_k: int, stream: int = 3):
    """Per token, top_k distinct expert ids drawn uniformly without replacement (partial
    Fisher-Yates), and router weights = softmax of top_k N(0,1) logits (float64 -> fp32).
    Returns (ids int32 [T][top_k], weights float32 [T][top_k])."""
    u = uniform(seed, stream, T * top_k)
    ids = np.empty((T, top_k), dtype=np.int32)
    for t in range(T):
        perm = np.arange(E, dtype=np.int64)
        for j in range(top_k):
            r = j + int(u[t * top_k + j] * (E - j))
            perm[j], perm[r] = perm[r], perm[j]
        ids[t] = perm[:top_k]
    logits = normal(seed, stream + 1, T * top_k).reshape(T, top_k)
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def moe_expert_weights(seed: int, e: int, N_gu: int, K_gu: int, N_d: int, K_d: int):
    """fp32 gate_up [N_gu][K_gu] and down [N_d][K_d] weights of expert e."""
    gu = weight_f32(seed, N_gu, K_gu, stream=1000 + e)
    dn = weight_f32(seed, N_d, K_d, stream=5000 + e)
    return gu, dn


# The five workloads (shapes, seeds and streams). Seeds are fixed per workload;
# activation rows of the sweeps use seed x_seed_base + M.
WORKLOADS = {
    "single_linear": dict(M=1, K=2048, N=2048, w_seed=1, x_seed=101),
    "decode_sweep": dict(Ms=(1, 2, 4, 8, 16), K=4096, N=12288, w_seed=2, x_seed_base=200),
    "moe_decode": dict(E=128, T=16, top_k=8, K_gu=2048, N_gu=1536, K_d=768, N_d=2048,
                       w_seed=3, x_seed=103, route_seed=33),
    "prefill": dict(M=2048, K=4096, N=14336, w_seed=4, x_seed=104),
    "w4a4": dict(Ms=(4, 16, 512), K=4096, N=4096, w_seed=5, x_seed_base=500),
}
