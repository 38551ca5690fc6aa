"""The C ABI on the host (no GPU needed): the library loads, exports every entry point
include/nvfp4.h declares, and refuses bad arguments by name before enqueuing anything.
Every call here fails host-side validation, so no kernel is launched; the fake device
addresses are never dereferenced."""
import ctypes
import os
import re
import subprocess

import pytest

import nvfp4_block_scaled_linear_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ARG, ERR_WORKSPACE = 0, 1, 2, 3, 4, 5
P = 0x7F0000000000  # an aligned fake device address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    # NVFP4_TEST_LIB: another build of the same sources (the sanitizer test runs this file
    # against a host-instrumented copy)
    alt = os.environ.get("NVFP4_TEST_LIB")
    if alt:
        return nv.load_library(alt)
    if not os.path.exists(nv.LIB_PATH):
        from nvfp4_block_scaled_linear_amd import build
        build.build()
    return nv.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:nvfp4_status|const char\*)\s+(nvfp4_\w+)\(", text, re.M)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("nvfp4_linear", "nvfp4_grouped_linear", "nvfp4_quantize_act", "nvfp4_status_string"):
        assert n in names
    assert set(names) == set(nv.EXPORTS)


def test_every_declared_symbol_is_exported_unmangled(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", nv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for s, frag in ((0, "NVFP4_OK"), (1, "NULL"), (2, "SHAPE"), (3, "ALIGN"), (4, "ARG"),
                    (5, "WORKSPACE"), (6, "LAUNCH"), (99, "unknown")):
        assert frag in nv.status_string(s)


def lin(lib, act=0, x=P, xs=None, xt=None, ldx=4096, M=4, N=128, K=4096, wc=P, ws=P, wt=P,
        y=P, ldy=128, flags=0, faults=None):
    return lib.nvfp4_linear(act, x, xs, xt, ldx, M, N, K, wc, ws, wt, y, ldy, flags, faults,
                            None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=0), ERR_SHAPE), (dict(K=48), ERR_SHAPE), (dict(K=-32), ERR_SHAPE),
    (dict(M=0), ERR_SHAPE), (dict(N=0), ERR_SHAPE), (dict(M=1 << 31), ERR_SHAPE),
    (dict(act=7), ERR_ARG), (dict(x=None), ERR_NULL), (dict(x=P + 8), ERR_ALIGN),
    (dict(ldx=4000), ERR_SHAPE), (dict(ldx=4100), ERR_ALIGN), (dict(xs=P), ERR_ARG),
    (dict(act=1, xs=None, xt=P), ERR_NULL), (dict(act=1, xs=P + 1, xt=P), ERR_ALIGN),
    (dict(wc=None), ERR_NULL), (dict(ws=None), ERR_NULL), (dict(wt=None), ERR_NULL),
    (dict(wc=P + 4), ERR_ALIGN), (dict(ws=P + 1), ERR_ALIGN), (dict(wt=P + 2), ERR_ALIGN),
    (dict(y=None), ERR_NULL), (dict(ldy=100), ERR_SHAPE), (dict(y=P + 2), ERR_ALIGN),
    # W4A4 with in-call quantization: BF16 x, at most four rows, K <= 8192, no x scales
    (dict(act=2, M=5), ERR_SHAPE), (dict(act=2, M=2), ERR_SHAPE), (dict(act=2, M=1, K=8224, ldx=8224), ERR_SHAPE),
    (dict(act=2, xs=P), ERR_ARG), (dict(act=2, xt=P), ERR_ARG), (dict(act=2, ldx=4100), ERR_ALIGN),
    (dict(act=3), ERR_ARG),
    # check mode: a known flag bit only, and a fault word to report into
    (dict(flags=2), ERR_ARG), (dict(flags=1), ERR_NULL), (dict(flags=1, faults=P + 2), ERR_ALIGN),
    (dict(faults=P + 1), ERR_ALIGN), (dict(flags=0x80000001, faults=P), ERR_ARG),
])
def test_linear_refusals(lib, kw, status):
    assert lin(lib, **kw) == status


def quant(lib, in_type=0, x=P, ldx=4096, M=4, K=4096, mode=0, c=P, s=P, ts=P, faults=None):
    return lib.nvfp4_quantize_act(in_type, x, ldx, M, K, mode, c, s, ts, faults, None)


@pytest.mark.parametrize("kw,status", [
    (dict(in_type=3), ERR_ARG), (dict(mode=2), ERR_ARG), (dict(K=40), ERR_SHAPE),
    (dict(M=0), ERR_SHAPE), (dict(ldx=100), ERR_SHAPE), (dict(x=None), ERR_NULL),
    (dict(c=None), ERR_NULL), (dict(s=None), ERR_NULL), (dict(ts=None), ERR_NULL),
    (dict(x=P + 4), ERR_ALIGN), (dict(ldx=4100), ERR_ALIGN), (dict(in_type=1, ldx=4098), ERR_ALIGN),
    (dict(c=P + 8), ERR_ALIGN), (dict(ts=P + 1), ERR_ALIGN), (dict(faults=P + 2), ERR_ALIGN),
])
def test_quantize_refusals(lib, kw, status):
    assert quant(lib, **kw) == status


def grouped(lib, act=0, x=P, xs=None, xt=None, ldx=2048, rows_mode=0, T=16, k=8, N=1536,
            K=2048, E=128, wc=P, ws=P, wt=P, ids=P, tw=P, out_mode=0, y=P, work=P,
            nbytes=1 << 30, flags=0, faults=None, pass_nbytes=True):
    n = ctypes.c_size_t(nbytes)
    return lib.nvfp4_grouped_linear(act, x, xs, xt, ldx, rows_mode, T, k, N, K, E, wc, ws, wt,
                                    ids, tw, out_mode, y, work,
                                    ctypes.byref(n) if pass_nbytes else None, flags, faults,
                                    None), n.value


def test_grouped_workspace_query(lib):
    st, need_routes = grouped(lib, work=None, nbytes=0, out_mode=0)
    assert st == OK and need_routes > 0
    st, need_swiglu = grouped(lib, work=None, nbytes=0, out_mode=1)
    assert st == OK
    st, need_combine = grouped(lib, work=None, nbytes=0, out_mode=2)
    assert st == OK
    # per-route rows and the SwiGLU rows go straight to y; the combine keeps fp32 rows
    # [T*k][N] in scratch
    assert need_swiglu == need_routes
    assert need_combine - need_routes >= 16 * 8 * 1536 * 4
    assert nv.grouped_workspace_size(16, 8, 1536, 2048, 128, nv.OUT_SWIGLU_BF16) == need_swiglu
    # reusing a grouping needs the same workspace as the combine itself
    st, need_reuse = grouped(lib, work=None, nbytes=0, out_mode=2 | 0x100)
    assert st == OK and need_reuse == need_combine


@pytest.mark.parametrize("kw,status", [
    (dict(pass_nbytes=False), ERR_NULL), (dict(E=0), ERR_ARG), (dict(E=5000), ERR_ARG),
    (dict(k=0), ERR_ARG), (dict(k=129), ERR_ARG), (dict(rows_mode=2), ERR_ARG),
    (dict(out_mode=3), ERR_ARG), (dict(out_mode=0x100), ERR_ARG), (dict(out_mode=0x101), ERR_ARG),
    (dict(out_mode=0x200), ERR_ARG), (dict(T=0), ERR_SHAPE), (dict(K=2047), ERR_SHAPE),
    (dict(out_mode=1, N=1535), ERR_SHAPE), (dict(nbytes=1000), ERR_WORKSPACE),
    (dict(work=P + 16), ERR_ALIGN), (dict(x=None), ERR_NULL), (dict(ids=None), ERR_NULL),
    (dict(y=None), ERR_NULL), (dict(out_mode=2, tw=None), ERR_NULL), (dict(ids=P + 2), ERR_ALIGN),
    (dict(wc=P + 8), ERR_ALIGN),
    # the in-call quantization is a dense-call form: refused here, also with every output
    # form and for the workspace query
    (dict(act=2), ERR_ARG), (dict(act=2, out_mode=1), ERR_ARG), (dict(act=2, out_mode=2), ERR_ARG),
    (dict(act=2, work=None, nbytes=0), ERR_ARG), (dict(act=3), ERR_ARG),
    (dict(act=1, xs=None, xt=P), ERR_NULL), (dict(act=1, xs=P, xt=None), ERR_NULL),
    (dict(act=0, xs=P), ERR_ARG),
    (dict(flags=2), ERR_ARG), (dict(flags=1), ERR_NULL), (dict(faults=P + 2), ERR_ALIGN),
])
def test_grouped_refusals(lib, kw, status):
    assert grouped(lib, **kw)[0] == status


@pytest.mark.parametrize("args,status", [
    ((None, 4096, 4, P), ERR_NULL), ((P, 4096, 4, None), ERR_NULL), ((P, 0, 4, P), ERR_SHAPE),
    ((P, 4100, 4, P), ERR_SHAPE), ((P, 1 << 31, 4, P), ERR_SHAPE), ((P + 8, 4096, 4, P), ERR_ALIGN),
    ((P, 4096, 4, P + 2), ERR_ALIGN), ((P, 4096, 3, P), ERR_ARG), ((P, 4096, 32, P), ERR_ARG),
])
def test_read_probe_refusals(lib, args, status):
    assert lib.nvfp4_read_probe(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, 4096, 0), ERR_NULL), ((P, 0, 0), ERR_SHAPE), ((P, 4100, 0), ERR_SHAPE),
    ((P, 1 << 31, 0), ERR_SHAPE), ((P + 8, 4096, 0), ERR_ALIGN), ((P, 4096, -1), ERR_ARG),
    ((P, 4096, 9000), ERR_ARG),
])
def test_prefetch_refusals(lib, args, status):
    assert lib.nvfp4_prefetch(*args, None) == status


def test_binding_fails_loudly_without_library(tmp_path):
    from nvfp4_block_scaled_linear_amd import _binding
    saved = _binding._lib
    try:
        _binding._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            _binding.load_library(str(tmp_path / "absent.so"))
    finally:
        _binding._lib = saved


def noalloc(lib, act=0, x=P, ldx=2048, rows_mode=0, T=16, k=8, N=1536, K=2048, E=128, wc=P,
            ws=P, wt=P, ids=P, tw=P, out_mode=0, y=P, flags=0, faults=None):
    return lib.nvfp4_grouped_linear_noalloc(act, x, None, None, ldx, rows_mode, T, k, N, K, E, wc,
                                            ws, wt, ids, tw, out_mode, y, flags, faults, None)


@pytest.mark.parametrize("kw,status", [
    (dict(E=0), ERR_ARG), (dict(k=0), ERR_ARG), (dict(out_mode=3), ERR_ARG),
    (dict(out_mode=0x100), ERR_ARG), (dict(T=0), ERR_SHAPE), (dict(K=2047), ERR_SHAPE),
    (dict(act=2), ERR_ARG), (dict(flags=1), ERR_NULL), (dict(flags=4), ERR_ARG),
    # beyond the fixed scratch: the combine of 4096 tokens x 8 routes x 2048 fp32 columns
    (dict(T=4096, N=2048, K=768, out_mode=2), ERR_WORKSPACE),
    (dict(T=2048, k=8, N=512, K=768, out_mode=2), ERR_WORKSPACE),
])
def test_noalloc_refusals(lib, kw, status):
    """The no-allocation grouped call refuses bad arguments, and calls whose workspace
    would exceed its fixed scratch, on the host: before it touches a device."""
    assert noalloc(lib, **kw) == status


def test_noalloc_scratch_limit_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define NVFP4_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == nv.NOALLOC_SCRATCH_BYTES
    # the largest combine that fits: a decode-sized MoE layer (16 tokens x top-8 x 2048)
    assert nv.grouped_workspace_size(16, 8, 2048, 768, 128, nv.OUT_COMBINE) < nv.NOALLOC_SCRATCH_BYTES
