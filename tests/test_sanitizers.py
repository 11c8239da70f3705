"""AddressSanitizer and UndefinedBehaviorSanitizer over the host code (CPU).

Two C drivers in tests/sanitize/ are built with both sanitizers and run:
  - oracle_driver.c with oracle/pda_oracle.c (gcc): the oracle's entry points
    over seeded random small problems (layouts, block sizes, empty sequences,
    out-of-range counts, page ids outside the pool, masks, row selections,
    prefill, rotary);
  - abi_driver.c against the library's host code (every source built with
    hipcc, the sanitizers on the host side only; linked with clang): every
    C-ABI entry point through its host-side checks and no-op calls, sizes and
    strides over a grid of dimensions up to 2^31 - 1.
Each driver exits 0 only when every call returned what its arguments call
for; any sanitizer report aborts it.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = os.path.join(HERE, "sanitize")
CSRC = os.path.join(ROOT, "paged_gqa_decode_pda_amd", "csrc")
LIB_SOURCES = ["pda_api", "pda_kernels", "pda_attend", "pda_prefill", "pda_rope"]
ROCM = "/opt/rocm"
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
HIPCC = os.path.join(ROCM, "bin", "hipcc")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def _check_clean(rc, out, what):
    assert "AddressSanitizer" not in out and "runtime error" not in out, f"{what}:\n{out[-4000:]}"
    assert rc == 0, f"{what} exited {rc}:\n{out[-4000:]}"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-fopenmp", "-o", exe,
                    os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "pda_oracle.c"), "-lm"])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    rc, out = _run([exe, "300"], env=env)
    _check_clean(rc, out, "oracle driver")
    assert "0 failures" in out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not available")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    san_host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    procs, objs = [], []
    for name in LIB_SOURCES:
        obj = str(tmp_path / f"{name}.o")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-I", os.path.join(ROOT, "include"), "-fno-gpu-sanitize", *san_host,
               "-fno-omit-frame-pointer", "-Wno-unused-command-line-argument",
               "-c", os.path.join(CSRC, f"{name}.hip"), "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate(timeout=900)
        assert p.returncode == 0, out[-4000:]
    drv = str(tmp_path / "drv.o")
    rc, out = _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(SAN, "abi_driver.c"), "-o", drv])
    assert rc == 0, out
    exe = str(tmp_path / "abi_driver")
    rc, out = _run([CLANG + "++", "-fsanitize=address,undefined", "-o", exe, drv, *objs,
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    assert rc == 0, out
    # the HIP runtime keeps allocations until exit: leaks are not checked here
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    rc, out = _run([exe], env=env)
    _check_clean(rc, out, "abi driver")
    assert "0 failures" in out
