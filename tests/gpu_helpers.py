"""Shared pieces of the GPU parity tests: device handles, weight preparation on both
sides (each side quantizes the same seeded fp32 weight with its own quantizer, and the
results must agree bit for bit before any product is compared), and the bound check."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import nvfp4_block_scaled_linear_amd as nv  # noqa: E402
import oracle  # noqa: E402


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    if not os.path.exists(nv.LIB_PATH):
        from nvfp4_block_scaled_linear_amd import build
        build.build()
    nv.load_library()
    return torch.device("cuda:0")


def to_dev_bf16(xb: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).to(dev).view(torch.bfloat16)


def quantize_both(o: oracle.Oracle, w: np.ndarray, dev, per_tensor=True):
    """GPU quantizer and oracle quantizer on the same fp32 weight; asserts bit equality."""
    wd = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
    c, s, t = nv.quantize_act(wd, per_tensor=per_tensor)
    oc, os_, ot = o.quantize(w, per_row=not per_tensor)
    gc, gs, gt = c.cpu().numpy(), s.cpu().numpy(), t.cpu().numpy()
    assert np.array_equal(gt.view(np.uint32), ot.view(np.uint32)), (gt[:4], ot[:4])
    bad_s = np.argwhere(gs != os_)
    assert bad_s.size == 0, f"scale mismatch at {bad_s[:5].tolist()}"
    bad_c = np.argwhere(gc != oc)
    assert bad_c.size == 0, f"code mismatch at {bad_c[:5].tolist()}"
    return (c, s, t), (oc, os_, ot)


def assert_within(y_gpu, y_ref, bound, what=""):
    ok, worst = oracle.within_bound(y_gpu, y_ref, bound)
    assert ok, f"{what}: worst |err| / (1e-4*B + 1e-6) = {worst:.3g}"
    return worst
