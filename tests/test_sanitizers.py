"""The library's host code under sanitizers (CPU only, no GPU needed).

* The host page pool (csrc/page_pool.cpp), driven by eight threads at once
  (tests/native/pool_stress.cpp), built with AddressSanitizer +
  UndefinedBehaviorSanitizer and again with ThreadSanitizer.
* The C ABI's argument validation and sizing arithmetic
  (tests/native/abi_checks.cpp) against the whole library, its host code
  built with AddressSanitizer + UndefinedBehaviorSanitizer (the device code
  is compiled normally; nothing is launched: every call is refused first).

Each binary must print "ok"; any sanitizer report fails it.
"""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "fp8_e4m3_paged_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
GPU_SOURCES = ["kv_cache_ops.hip", "decode_attn.hip", "ingest.hip", "gemv.hip", "kvfp8_api.hip"]


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.fixture(scope="module")
def tmp():
    d = tempfile.mkdtemp(prefix="kvfp8_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("sanitizer", ["address,undefined", "thread"])
def test_page_pool_under_sanitizers(tmp, sanitizer):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = os.path.join(tmp, "pool_" + sanitizer.replace(",", "_"))
    _run(["g++", "-std=c++17", "-O1", "-g", f"-fsanitize={sanitizer}", "-fno-sanitize-recover=all",
          "-I", INC, os.path.join(NATIVE, "pool_stress.cpp"), os.path.join(CSRC, "page_pool.cpp"),
          "-pthread", "-o", exe])
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="halt_on_error=1")
    assert _run([exe], env=env).strip() == "ok"


def test_abi_validation_under_address_and_ub_sanitizers(tmp):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ not available")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "-I", INC]
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    procs, objs = [], []
    for src in GPU_SOURCES:
        obj = os.path.join(tmp, src + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen(
            [HIPCC, "--offload-arch=gfx950", *flags, *host_san, "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-c", os.path.join(CSRC, src), "-o", obj],
            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, err[-4000:]
    drv = os.path.join(tmp, "abi_checks.o")
    _run([CLANGXX, *flags, "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c",
          os.path.join(NATIVE, "abi_checks.cpp"), "-o", drv])
    exe = os.path.join(tmp, "abi_asan")
    _run([CLANGXX, "-fsanitize=address,undefined", drv, *objs, "-L", os.path.join(ROCM, "lib"),
          "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    # the HIP runtime's own start-up allocations are not this library's leaks
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               HIP_VISIBLE_DEVICES="-1" if "HIP_VISIBLE_DEVICES" not in os.environ else
               os.environ["HIP_VISIBLE_DEVICES"])
    assert _run([exe], env=env).strip() == "ok"
