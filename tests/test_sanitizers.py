"""Sanitizer builds on the CPU: the C oracle under AddressSanitizer + UBSan
(with leak checks) and under ThreadSanitizer (its worker pool), and the host
side of the C ABI (moba_api.hip's host code, instrumented through
-Xarch_host, linked with the library's kernel objects) under
AddressSanitizer + UBSan.  Each runs a C driver from tests/sanitize/ that
exercises every entry point it can call without a GPU; any report makes the
run fail (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ORACLE_C = os.path.join(ROOT, "oracle", "moba_oracle.c")
BUILD = os.path.join(ROOT, "block_sparse_long_key_amd", "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, env=None, timeout=600):
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)


def _build_oracle_driver(tmp_path, sanitize):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "oracle_driver")
    r = _run([gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
              *sanitize, "-pthread", ORACLE_C, os.path.join(SAN, "oracle_driver.c"), "-lm",
              "-o", exe])
    if r.returncode != 0:
        pytest.skip(f"sanitizer build unavailable: {r.stderr[-400:]}")
    return exe


def _check(r):
    out = r.stdout + r.stderr
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), out[-4000:]
    assert "runtime error" not in out and "Sanitizer" not in out, out[-4000:]


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = _build_oracle_driver(tmp_path, ["-fsanitize=address,undefined",
                                          "-fno-sanitize-recover=all"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    _check(_run([exe, "3"], env=env))


def test_oracle_worker_pool_under_thread_sanitizer(tmp_path):
    exe = _build_oracle_driver(tmp_path, ["-fsanitize=thread"])
    r = _run([exe, "4"])
    if r.returncode != 0 and "FATAL: ThreadSanitizer" in r.stderr:
        pytest.skip("ThreadSanitizer cannot map its shadow memory here")
    _check(r)


def test_host_abi_under_address_and_ub_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG) and os.path.exists(CLANGXX)):
        pytest.skip("the ROCm toolchain is not available")
    others = ["attn", "attn_bwd", "attn_bwd_f32", "invert", "key_conv_bwd", "key_conv_pool",
              "router"]
    objs = [os.path.join(BUILD, n + ".o") for n in others]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's objects are not built (run the package build first)")
    inc = os.path.join(ROOT, "include")
    api = str(tmp_path / "moba_api.o")
    # host pass instrumented only: every -fsanitize= goes to the host
    r = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form=true",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
              "-I", inc, "-c", os.path.join(ROOT, "block_sparse_long_key_amd", "csrc", "moba_api.hip"),
              "-o", api])
    assert r.returncode == 0, r.stderr[-2000:]
    drv = str(tmp_path / "drv.o")
    r = _run([CLANG, "-std=c99", "-g", "-O1", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", inc,
              "-I", "/opt/rocm/include", "-c", os.path.join(SAN, "host_abi_driver.c"), "-o", drv])
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "host_abi_driver")
    r = _run([CLANGXX, "-fsanitize=address,undefined", drv, api, *objs, "-L/opt/rocm/lib",
              "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert r.returncode == 0, r.stderr[-2000:]
    # leaks of the HIP runtime itself are not this library's
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    _check(_run([exe], env=env))
