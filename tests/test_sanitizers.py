"""The CPU side under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

* The oracle's C code (oracle/nvfp4_oracle.c) runs every entry point on small and edge
  inputs in a gcc build with ASan + UBSan (tests/oracle_sanitize_driver.c).
* The library's host code (the C ABI's argument checks and dispatch) is built with
  clang's ASan + UBSan on the host side only (device code as usual) and the whole ABI
  refusal suite (tests/test_abi_cpu.py) runs against that build in a child process.
* A planted overflow and a planted signed overflow show that the flags really instrument:
  a build that silently dropped them would pass the two checks above without proving
  anything.
"""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
GCC_SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all"]
ORACLE_FLAGS = ["-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                "-fexcess-precision=standard"]


def _need(tool):
    if shutil.which(tool) is None and not os.path.exists(tool):
        pytest.skip(f"{tool} not found")


def _run(cmd, env=None, timeout=600):
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)


def test_sanitizer_flags_catch_planted_mistakes(tmp_path):
    _need("gcc")
    src = tmp_path / "planted.c"
    src.write_text(
        "#include <stdlib.h>\n#include <limits.h>\n#include <string.h>\n"
        "int main(int argc, char** argv) {\n"
        "  if (argc > 1 && strcmp(argv[1], \"ub\") == 0) { volatile int a = INT_MAX; int i = a + argc; return i & 1; }\n"
        "  int* p = malloc(4 * sizeof(int)); int r = p[argc + 3]; free(p); return r;\n"
        "}\n")
    exe = tmp_path / "planted"
    subprocess.check_call(["gcc", *GCC_SAN, "-o", str(exe), str(src)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = _run([str(exe)], env=env)
    # ASan's report, or UBSan's object-size check when that one fires first
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr
                                  or "insufficient space" in r.stderr), r.stderr[-2000:]
    r = _run([str(exe), "ub"], env=env)
    assert r.returncode != 0 and "runtime error" in r.stderr, r.stderr[-2000:]


def test_oracle_under_asan_and_ubsan(tmp_path):
    _need("gcc")
    exe = tmp_path / "oracle_san"
    subprocess.check_call(["gcc", *GCC_SAN, *ORACLE_FLAGS, "-o", str(exe),
                           os.path.join(HERE, "oracle_sanitize_driver.c"),
                           os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), "-lm"])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1")
    r = _run([str(exe)], env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ok" in r.stdout


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    from nvfp4_block_scaled_linear_amd import build as B
    _need(B.HIPCC)
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    # host side instrumented (each option right after -Xarch_host), device code unchanged
    host_san = ["-Xarch_host", "-fsanitize=address,undefined",
                "-Xarch_host", "-fno-sanitize-recover=all",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    jobs = []
    for src in B.sources():
        name = os.path.basename(src)
        obj = str(tmp_path / (name + ".o"))
        jobs.append(([B.HIPCC, *B.FLAGS, *B.EXTRA.get(name, []), *host_san, "-c", "-o", obj, src], obj))

    def compile_one(job):
        r = _run(job[0], timeout=900)
        assert r.returncode == 0, r.stderr[-3000:]

    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as pool:
        list(pool.map(compile_one, jobs))
    lib = str(tmp_path / "libnvfp4_san.so")
    r = _run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
              "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-shared-libasan",
              "-o", lib, *[o for _, o in jobs]])
    assert r.returncode == 0, r.stderr[-3000:]
    if shutil.which("nm"):  # the host code really calls into both runtimes
        syms = _run(["nm", "-D", "--undefined-only", lib]).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, NVFP4_TEST_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = _run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi_cpu.py"), "-q",
              "-p", "no:cacheprovider", "-m", "not gpu"], env=env, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout and "error" not in r.stdout.lower().split("passed")[-1]
