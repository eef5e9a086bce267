"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every HIP source is compiled for gfx950 as in the normal build, with the
sanitizers on the host side only (`-Xarch_host`), and linked with a C++
driver (`host_abi_driver.cpp`) that calls every path returning before a
launch: dims validation and workspace sizing over ordinary, limit and
invalid sizes, the argument checks of each entry point and the host-only
slot planner on random sequences. No GPU is needed. A sanitizer report
(heap or stack overflow, use after free, signed overflow, misaligned access
and the other UBSan checks) or a failed expectation fails the test.
"""

import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_rank_amd", "csrc")
SOURCES = ["api", "k_hkv", "k_select", "k_attn", "k_sparse32", "k_linear", "k_proj32", "k_lowrank32",
           "k_backward"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def _tool(name):
    for cand in (shutil.which(name), os.path.join("/opt/rocm/bin", name), os.path.join("/opt/rocm/lib/llvm/bin", name)):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip(f"{name} not found")


@pytest.mark.timeout(600)
def test_host_code_under_sanitizers(tmp_path):
    hipcc, clangxx = _tool("hipcc"), _tool("clang++")
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    common = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer"]

    def compile_one(name):
        cmd = [hipcc, "--offload-arch=gfx950", *common, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               *SAN, *inc, "-c", os.path.join(CSRC, name + ".hip"), "-o", str(tmp_path / (name + ".o"))]
        return subprocess.run(cmd, capture_output=True, text=True)

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for name, r in zip(SOURCES, results):
        assert r.returncode == 0, f"{name}: {r.stderr[-2000:]}"
    drv_o = str(tmp_path / "driver.o")
    r = subprocess.run([clangxx, *common, *SAN, *inc, "-c", os.path.join(ROOT, "tests", "host_abi_driver.cpp"),
                        "-o", drv_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "host_abi_driver")
    r = subprocess.run([clangxx, *SAN, "--hip-link", "--offload-arch=gfx950", drv_o,
                        *[str(tmp_path / (n + ".o")) for n in SOURCES], "-L/opt/rocm/lib", "-lamdhip64", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
