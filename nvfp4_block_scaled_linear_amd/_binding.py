"""ctypes binding over libnvfp4.so: marshals torch tensors (device memory) and the current
HIP stream into the C ABI of include/nvfp4.h. No computation happens here; every step
of the layer runs in the library's kernels. The library must be built (build.py); a
missing library raises instead of falling back to anything else."""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

ACT_BF16, ACT_NVFP4, ACT_BF16_QUANTIZE = 0, 1, 2
IN_BF16, IN_F32 = 0, 1
TS_PER_ROW, TS_PER_TENSOR = 0, 1
ROWS_PER_TOKEN, ROWS_PER_ROUTE = 0, 1
OUT_ROUTES, OUT_SWIGLU_BF16, OUT_COMBINE = 0, 1, 2
OUT_REUSE_GROUPING = 0x100
FAULT_NONFINITE, FAULT_BAD_ROUTE, FAULT_NAN_SCALE = 1, 2, 4
F_CHECK = 1

EXPORTS = ("nvfp4_status_string", "nvfp4_linear", "nvfp4_quantize_act", "nvfp4_grouped_linear",
           "nvfp4_grouped_linear_noalloc", "nvfp4_prefetch", "nvfp4_read_probe")
NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def load_library(path: str = LIB_PATH):
    """Load libnvfp4.so once. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with nvfp4_block_scaled_linear_amd/build.py "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    vp, i64, i32, u32p = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    lib.nvfp4_status_string.argtypes = [i32]
    lib.nvfp4_linear.restype = i32
    u32 = ctypes.c_uint32
    lib.nvfp4_linear.argtypes = [i32, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, i64, u32,
                                 u32p, vp]
    lib.nvfp4_quantize_act.restype = i32
    lib.nvfp4_quantize_act.argtypes = [i32, vp, i64, i64, i64, i32, vp, vp, vp, u32p, vp]
    lib.nvfp4_grouped_linear.restype = i32
    lib.nvfp4_grouped_linear.argtypes = [i32, vp, vp, vp, i64, i32, i64, i32, i64, i64, i32, vp,
                                         vp, vp, vp, vp, i32, vp, vp,
                                         ctypes.POINTER(ctypes.c_size_t), u32, u32p, vp]
    lib.nvfp4_grouped_linear_noalloc.restype = i32
    lib.nvfp4_grouped_linear_noalloc.argtypes = [i32, vp, vp, vp, i64, i32, i64, i32, i64, i64,
                                                 i32, vp, vp, vp, vp, vp, i32, vp, u32, u32p, vp]
    lib.nvfp4_prefetch.restype = i32
    lib.nvfp4_prefetch.argtypes = [vp, i64, i32, vp]
    lib.nvfp4_read_probe.restype = i32
    lib.nvfp4_read_probe.argtypes = [vp, i64, i32, u32p, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().nvfp4_status_string(int(status)).decode()


def _p(t):
    """Device address of a tensor. Host tensors and rows with a non-unit inner stride are
    refused here: the kernels would read a host pointer as device memory."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libnvfp4 takes device tensors only")
    if t.dim() > 0 and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("libnvfp4 needs rows with unit inner stride")
    return ctypes.c_void_p(t.data_ptr())


def _ld(t):
    """Row pitch in elements. A one-row view may carry any stride (numpy gives 0 for an
    added axis), so its pitch is its row length."""
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise NVFP4Error(status, what)


def linear(x, w_codes, w_scales, w_ts, *, x_scales=None, x_ts=None, out=None,
           quantize_x=False, check=False, faults=None):
    """y = x W^T for an NVFP4 weight (codes [N][K/2] u8, scales [N][K/16] u8, ts [1] f32).
    x is BF16 [M][K] (W4A16), or NVFP4 codes [M][K/2] u8 with x_scales/x_ts (W4A4).
    quantize_x=True (BF16 x, one row): W4A4 with x quantized inside the call.
    check=True scans the operands first and ORs FAULT_* bits into `faults` (a device
    int32 word, required then)."""
    N = w_codes.shape[0]
    K = 2 * w_codes.shape[1]
    if x_scales is None:
        act, M, ldx = (ACT_BF16_QUANTIZE if quantize_x else ACT_BF16), x.shape[0], _ld(x)
    else:
        act, M, ldx = ACT_NVFP4, x.shape[0], K
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=w_codes.device)
    st = load_library().nvfp4_linear(act, _p(x), _p(x_scales), _p(x_ts), ldx, M, N, K,
                                     _p(w_codes), _p(w_scales), _p(w_ts), _p(out),
                                     _ld(out), F_CHECK if check else 0, _p(faults), _stream())
    _check(st, "nvfp4_linear")
    return out


def quantize_act(x, *, per_tensor: bool = False, faults=None, codes=None, scales=None, ts=None):
    """Quantize x (BF16 or fp32, [M][K]) to NVFP4 on the device; returns (codes, scales, ts)."""
    M, K = x.shape
    in_type = IN_BF16 if x.dtype in (torch.bfloat16, torch.int16, torch.uint16) else IN_F32
    dev = x.device
    codes = codes if codes is not None else torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = scales if scales is not None else torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    ts = ts if ts is not None else torch.empty((1 if per_tensor else M,), dtype=torch.float32, device=dev)
    st = load_library().nvfp4_quantize_act(in_type, _p(x), _ld(x), M, K,
                                           TS_PER_TENSOR if per_tensor else TS_PER_ROW,
                                           _p(codes), _p(scales), _p(ts), _p(faults), _stream())
    _check(st, "nvfp4_quantize_act")
    return codes, scales, ts


def grouped_workspace_size(T: int, top_k: int, N: int, K: int, num_experts: int,
                           out_mode: int) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().nvfp4_grouped_linear(ACT_BF16, None, None, None, K, ROWS_PER_TOKEN, T,
                                             top_k, N, K, num_experts, None, None, None, None,
                                             None, out_mode, None, None, ctypes.byref(n), 0,
                                             None, None)
    _check(st, "nvfp4_grouped_linear (workspace query)")
    return n.value


def grouped_linear(x, w_codes, w_scales, w_ts, topk_ids, *, topk_w=None, out_mode=OUT_ROUTES,
                   rows_per_route=False, x_scales=None, x_ts=None, out=None, workspace=None,
                   faults=None, reuse_grouping=False, check=False):
    """Expert-grouped NVFP4 linear. w_codes [E][N][K/2], w_scales [E][N][K/16], w_ts [E];
    topk_ids [T][top_k] int32. See include/nvfp4.h for the output forms. reuse_grouping
    (OUT_COMBINE with the workspace of the layer's earlier call on the same topk_ids)
    skips the route grouping. check=True scans every expert's scales and the activations
    first (see linear)."""
    if reuse_grouping and workspace is None:
        raise ValueError("reuse_grouping needs the workspace that holds the grouping")
    E, N, half = w_codes.shape
    K = 2 * half
    T, top_k = topk_ids.shape
    R = T * top_k
    act = ACT_BF16 if x_scales is None else ACT_NVFP4
    ldx = _ld(x) if act == ACT_BF16 else K
    dev = w_codes.device
    if out is None:
        if out_mode == OUT_ROUTES:
            out = torch.empty((R, N), dtype=torch.float32, device=dev)
        elif out_mode == OUT_SWIGLU_BF16:
            out = torch.empty((R, N // 2), dtype=torch.bfloat16, device=dev)
        else:
            out = torch.empty((T, N), dtype=torch.float32, device=dev)
    need = grouped_workspace_size(T, top_k, N, K, E, out_mode)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    nbytes = ctypes.c_size_t(workspace.numel())
    st = load_library().nvfp4_grouped_linear(
        act, _p(x), _p(x_scales), _p(x_ts), ldx, ROWS_PER_ROUTE if rows_per_route else ROWS_PER_TOKEN,
        T, top_k, N, K, E, _p(w_codes), _p(w_scales), _p(w_ts), _p(topk_ids), _p(topk_w),
        out_mode | (OUT_REUSE_GROUPING if reuse_grouping else 0),
        _p(out), _p(workspace), ctypes.byref(nbytes), F_CHECK if check else 0, _p(faults),
        _stream())
    _check(st, "nvfp4_grouped_linear")
    return out


def grouped_linear_noalloc(x, w_codes, w_scales, w_ts, topk_ids, *, out, topk_w=None,
                           out_mode=OUT_ROUTES, rows_per_route=False, x_scales=None, x_ts=None,
                           faults=None, reuse_grouping=False, check=False):
    """grouped_linear on the library's fixed per-device scratch (no workspace argument and
    no allocation: `out` must be given). Calls on one device share that scratch, so they
    must not overlap; reuse_grouping reuses the grouping of the previous such call."""
    E, N, half = w_codes.shape
    K = 2 * half
    T, top_k = topk_ids.shape
    act = ACT_BF16 if x_scales is None else ACT_NVFP4
    ldx = _ld(x) if act == ACT_BF16 else K
    st = load_library().nvfp4_grouped_linear_noalloc(
        act, _p(x), _p(x_scales), _p(x_ts), ldx, ROWS_PER_ROUTE if rows_per_route else ROWS_PER_TOKEN,
        T, top_k, N, K, E, _p(w_codes), _p(w_scales), _p(w_ts), _p(topk_ids), _p(topk_w),
        out_mode | (OUT_REUSE_GROUPING if reuse_grouping else 0), _p(out),
        F_CHECK if check else 0, _p(faults), _stream())
    _check(st, "nvfp4_grouped_linear_noalloc")
    return out


def prefetch(buf, workgroups: int = 0, stream=None):
    """Next-weight prefetch: read the bytes of `buf` (a contiguous device tensor) into the
    caches on `stream` (default: the current stream), values discarded."""
    nbytes = buf.numel() * buf.element_size()
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream()
    st = load_library().nvfp4_prefetch(_p(buf), nbytes, int(workgroups), s)
    _check(st, "nvfp4_prefetch")


def read_probe(buf, loads_per_thread: int, sink):
    """Measurement support: one plain streaming read of the bytes of `buf` (a contiguous
    device tensor) in one launch; `sink` is a device int32 the kernel may overwrite."""
    nbytes = buf.numel() * buf.element_size()
    st = load_library().nvfp4_read_probe(_p(buf), nbytes, int(loads_per_thread), _p(sink),
                                         _stream())
    _check(st, "nvfp4_read_probe")
