"""Builds libnvfp4.so (the HIP kernels and the C ABI) in-tree, for gfx950 only."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libnvfp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops off: packed fp32 VALU forms are avoided on this hardware.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]

# Per-source flags. The weight-streaming kernels feed every 4x4x4 MFMA result straight
# into VALU FMAs (the per-block scale); in the accumulation-register form each of those
# reads costs one v_accvgpr_read, so their MFMAs write ordinary VGPRs.
EXTRA = {"stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libnvfp4.so")


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory() as d:
        jobs = []
        for src in sources():
            name = os.path.basename(src)
            obj = os.path.join(d, name + ".o")
            jobs.append(([HIPCC, *FLAGS, *EXTRA.get(name, []), "-c", "-o", obj, src], obj))
        with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as pool:
            list(pool.map(lambda j: _run(j[0], verbose), jobs))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for _, o in jobs]],
             verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
