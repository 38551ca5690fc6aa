"""CPU oracle for the NVFP4 block-scaled linear layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()`` and by
the CPU-baseline leg of ``bench.py``, never by the product package. The arithmetic
lives in ``nvfp4_oracle.c`` (plain C, float64, compiled with gcc into
``liboracle.so``); this file marshals numpy arrays and composes the MoE reading from
the C primitives. Each function names the definition it follows; the C file's header
lists the sources.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fexcess-precision=standard"]
_lib = None


def build_lib(src: str = _SRC, out: str = _LIB_PATH, defines=()) -> str:
    """Compile the oracle with gcc. ``defines`` exist only so tests can build planted
    mistakes into a separate copy of the library (negative controls)."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", *_CFLAGS, *[f"-D{d}" for d in defines], "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def _bind(lib):
    vp, i64, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
    sig = {
        "oracle_e2m1_value": (f64, [i32]),
        "oracle_e4m3_value": (f64, [i32]),
        "oracle_e2m1_encode": (i32, [f32]),
        "oracle_e4m3_encode": (i32, [f32]),
        "oracle_bf16_value": (f64, [ctypes.c_uint16]),
        "oracle_bf16_round": (ctypes.c_uint16, [f64]),
        "oracle_quantize": (i32, [vp, i64, i64, i32, vp, vp, vp]),
        "oracle_dequant": (None, [vp, vp, vp, i32, i64, i64, vp]),
        "oracle_linear": (None, [vp, i64, vp, i64, i64, vp, vp]),
        "oracle_num_threads": (i32, []),
        "oracle_e2m1_encode_batch": (None, [vp, i64, vp]),
        "oracle_e4m3_encode_batch": (None, [vp, i64, vp]),
        "oracle_bf16_round_batch": (None, [vp, i64, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def load(path: str | None = None):
    """Load the oracle library (building it first if missing or stale). With ``path``,
    load that specific build (used for planted-mistake copies)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build_lib()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


class Oracle:
    """numpy-facing wrapper over one build of the C oracle."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    # -- codec -------------------------------------------------------------------
    def e2m1_value(self, code: int) -> float:
        return self.lib.oracle_e2m1_value(int(code))

    def e4m3_value(self, byte: int) -> float:
        return self.lib.oracle_e4m3_value(int(byte))

    def e2m1_encode(self, q) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.float32)
        out = np.empty(q.shape, dtype=np.int8)
        self.lib.oracle_e2m1_encode_batch(q.ctypes.data, q.size, out.ctypes.data)
        return out

    def e4m3_encode(self, r) -> np.ndarray:
        r = np.ascontiguousarray(r, dtype=np.float32)
        out = np.empty(r.shape, dtype=np.int16)
        self.lib.oracle_e4m3_encode_batch(r.ctypes.data, r.size, out.ctypes.data)
        return out

    def bf16_round(self, v: float) -> int:
        return int(self.lib.oracle_bf16_round(float(v)))

    def bf16_value(self, bits: int) -> float:
        return self.lib.oracle_bf16_value(int(bits))

    def bf16_round_array(self, v) -> np.ndarray:
        """bf16_round of every element of a float64 array (same shape, uint16 bits)."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.oracle_bf16_round_batch(v.ctypes.data, v.size, out.ctypes.data)
        return out

    # -- quantizer -----------------------------------------------------------------
    def quantize(self, w, per_row: bool):
        """NVFP4-quantize fp32 w [rows][K]: per-tensor (weights) or per-row ts (W4A4
        activations). Returns (codes u8 [rows][K/2], scales u8 [rows][K/16],
        ts f32 [rows] or [1])."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        rows, K = w.shape
        assert K % 16 == 0
        codes = np.empty((rows, K // 2), dtype=np.uint8)
        scales = np.empty((rows, K // 16), dtype=np.uint8)
        ts = np.empty(rows if per_row else 1, dtype=np.float32)
        rc = self.lib.oracle_quantize(w.ctypes.data, rows, K, int(per_row), codes.ctypes.data,
                                      scales.ctypes.data, ts.ctypes.data)
        if rc != 0:
            raise ValueError("non-finite value in quantizer input")
        return codes, scales, ts

    def quantize_bf16(self, x_bits, per_row: bool):
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        return self.quantize(self.bf16_to_f64(x_bits).astype(np.float32), per_row)

    # -- dequantization and products -------------------------------------------------
    @staticmethod
    def bf16_to_f64(bits) -> np.ndarray:
        b = np.ascontiguousarray(bits, dtype=np.uint16)
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)

    def dequant(self, codes, scales, ts, per_row: bool) -> np.ndarray:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        ts = np.ascontiguousarray(ts, dtype=np.float32)
        rows, half = codes.shape
        K = 2 * half
        assert scales.shape == (rows, K // 16)
        out = np.empty((rows, K), dtype=np.float64)
        self.lib.oracle_dequant(codes.ctypes.data, scales.ctypes.data, ts.ctypes.data,
                                int(per_row), rows, K, out.ctypes.data)
        return out

    def linear_f64(self, x, w):
        """y = x w^T summed in float64 in k order, with bound = |x| |w|^T."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        M, K = x.shape
        N, K2 = w.shape
        assert K == K2
        y = np.empty((M, N), dtype=np.float64)
        b = np.empty((M, N), dtype=np.float64)
        self.lib.oracle_linear(x.ctypes.data, M, w.ctypes.data, N, K, y.ctypes.data, b.ctypes.data)
        return y, b

    def linear(self, x_bits, codes, scales, ts, wdq=None):
        """W4A16: BF16 rows x [M][K] times the NVFP4 weight [N][K] (per-tensor ts).
        ``wdq`` may pass the weight already dequantized by ``dequant``."""
        if wdq is None:
            wdq = self.dequant(codes, scales, ts, per_row=False)
        return self.linear_f64(self.bf16_to_f64(x_bits), wdq)

    def linear_w4a4(self, xc, xs, xts, codes, scales, ts, wdq=None):
        """W4A4: NVFP4 rows (per-row ts) times the NVFP4 weight (per-tensor ts)."""
        if wdq is None:
            wdq = self.dequant(codes, scales, ts, per_row=False)
        return self.linear_f64(self.dequant(xc, xs, xts, per_row=True), wdq)

    # -- expert-grouped MoE reading ---------------------------------------------------
    def moe_gate_up(self, x_bits, ids, gu_codes, gu_scales, gu_ts):
        """Per-route rows h[t*k + j] = x[t] W_gu[ids[t][j]]^T (ts applied), fp64, with
        bounds. Each routed expert is dequantized once for all its routes (the pages'
        expert-once reading: issue #565 section 4, PR #808)."""
        T, k = ids.shape
        N = gu_codes.shape[1]
        x = self.bf16_to_f64(x_bits)
        h = np.zeros((T * k, N))
        b = np.zeros((T * k, N))
        for e in np.unique(ids):
            rows = [(t, j) for t in range(T) for j in range(k) if ids[t, j] == e]
            wdq = self.dequant(gu_codes[e], gu_scales[e], gu_ts[e:e + 1], per_row=False)
            xr = np.stack([x[t] for t, _ in rows])
            y, bb = self.linear_f64(xr, wdq)
            for i, (t, j) in enumerate(rows):
                h[t * k + j] = y[i]
                b[t * k + j] = bb[i]
        return h, b

    def swiglu(self, h):
        """a = silu(g) * u with g = h[:, :N/2], u = h[:, N/2:], silu(g) = g / (1 + e^-g),
        in float64 (the BF16 rounding of the result is compared separately)."""
        h = np.asarray(h, dtype=np.float64)
        half = h.shape[1] // 2
        g, u = h[:, :half], h[:, half:]
        return g / (1.0 + np.exp(-g)) * u

    def moe_down_combine(self, a_bits, ids, rw, d_codes, d_scales, d_ts):
        """y[t] = sum over t's routes, in ascending expert id, of r * ts_e * (a W_d^T) —
        the ordered FP32 combine with the expert's tensor scale folded into the router
        weight (Rocket log entry "The expert split decodes the same tokens; ...",
        section "Why rows and not partial sums"). float64 here; bound per token is
        sum |r| * sum_k |a_k w_k ts_e|."""
        return self.moe_combine_rows(self.bf16_to_f64(a_bits), ids, rw, d_codes, d_scales, d_ts)

    def moe_combine_rows(self, a, ids, rw, d_codes, d_scales, d_ts):
        """The same ordered combine on float64 route rows a [T*k][K] (route t*k + j): for
        route rows that are not BF16, e.g. NVFP4 rows decoded exactly by ``dequant``."""
        T, k = ids.shape
        N = d_codes.shape[1]
        a = np.asarray(a, dtype=np.float64)
        y = np.zeros((T, N))
        b = np.zeros((T, N))
        cache = {}
        for t in range(T):
            for j in np.argsort(ids[t], kind="stable"):
                e = int(ids[t, j])
                if e not in cache:
                    cache[e] = self.dequant(d_codes[e], d_scales[e], d_ts[e:e + 1], per_row=False)
                o, ob = self.linear_f64(a[t * k + j][None, :], cache[e])
                y[t] += float(rw[t, j]) * o[0]
                b[t] += abs(float(rw[t, j])) * ob[0]
        return y, b

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())


def within_bound(y_gpu, y_ref, bound, rel=1e-4, abs_=1e-6):
    """The acceptance rule |y_gpu - y| <= rel * sum_k |x_k w_k| + abs for every output.
    Returns (ok, worst ratio error / allowed)."""
    err = np.abs(np.asarray(y_gpu, dtype=np.float64) - y_ref)
    allowed = rel * bound + abs_
    ratio = err / allowed
    return bool(np.all(err <= allowed)), float(ratio.max()) if ratio.size else 0.0
