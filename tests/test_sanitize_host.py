"""The host planner and the C ABI's argument validation built with AddressSanitizer and
UndefinedBehaviorSanitizer and exercised by tests/sanitize/abi_sanitize.cpp (a stand-in
replaces the kernel launcher; no GPU is used).  The HIP translation unit of the ABI is
compiled with the sanitizers on its host pass only; the pure host sources with clang++."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_grouped_gemm_block_amd", "csrc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm toolchain")
def test_planner_and_abi_under_sanitizers(tmp_path):
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    api_o = str(tmp_path / "api.o")
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer"] + host_san +
         inc + ["-c", os.path.join(CSRC, "fp8bs_api.cpp"), "-o", api_o])
    objs = [api_o]
    for src in (os.path.join(CSRC, "fp8bs_planner.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "abi_sanitize.cpp")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([CLANG, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer"] + SAN + inc +
             ["-c", src, "-o", o])
        objs.append(o)
    exe = str(tmp_path / "abi_sanitize")
    _run([CLANG] + SAN + objs + ["-o", exe, "-L/opt/rocm/lib", "-lamdhip64",
                                 "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env, timeout=600)
    assert "0 failed" in r.stdout, r.stdout + r.stderr
