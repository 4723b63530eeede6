"""The C-ABI's argument checking under host AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (every entry point's validation, workspace arithmetic and error text) is compiled
again with the sanitizers on its host code only, linked with the already-built kernel
objects into a temporary copy of the library, and driven by tests/abi_sanitize_driver.c:
every entry point called with NULL pointers, out-of-range and extreme sizes, bad patterns
and short or misaligned workspaces.  Every call must return its error status without an
out-of-bounds access, signed overflow or invalid shift.  No call passes validation, so no
kernel is launched and no GPU is needed."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "dsa_lightning_indexer_scores_amd")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
OBJS = ("indexer.o", "topk.o", "attn.o", "overlap.o", "distill.o")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    objs = [os.path.join(PKG, "_build", o) for o in OBJS]
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not found")
    if not all(os.path.exists(o) for o in objs):
        pytest.fail("kernel objects missing under dsa_lightning_indexer_scores_amd/_build: run the build first")
    d = str(tmp_path_factory.mktemp("sanitized"))
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = os.path.join(d, "api.o")
    _run([HIPCC, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fvisibility=hidden",
          "-I", os.path.join(ROOT, "include"), *san, "-c", os.path.join(PKG, "csrc", "api.cpp"), "-o", api_o])
    lib = os.path.join(d, "libindexcache_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, api_o, *objs, "-Wl,-rpath,/opt/rocm/lib"])
    exe = os.path.join(d, "abi_driver")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_sanitize_driver.c"), lib,
          f"-Wl,-rpath,{d}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    return exe


def test_argument_checks_under_asan_and_ubsan(driver):
    env = dict(os.environ)
    # the HIP runtime's own allocations are not this library's to answer for
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert "all argument checks behaved" in r.stdout
