"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two drivers (tests/sanitize/) are built with every sanitizer finding fatal:
- the CPU oracle, run on small inputs that reach its edges (ragged group
  tails, one-element groups, sinks covering a call, empty fits, every width,
  subnormal / signed-zero / extreme fp16 values);
- the C ABI's host side (csrc/api.hip with sanitized host code), every entry
  point's validation driven with NULL and misaligned pointers, negative, zero
  and extreme sizes (products of int32 arguments) and unknown widths. No call
  reaches a kernel launch (the launch functions are stand-ins that fail if
  reached), so this runs without a GPU.
Builds are cached under the system temp directory by source hash.
"""
import hashlib
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _cache_dir(*files):
    h = hashlib.sha1()
    for f in files:
        h.update(open(f, "rb").read())
    d = os.path.join(tempfile.gettempdir(), "kvq_sanitize_" + h.hexdigest()[:16])
    os.makedirs(d, exist_ok=True)
    return d


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_asan_ubsan():
    src = [os.path.join(SAN, "oracle_driver.cpp"), os.path.join(ROOT, "oracle", "kvq_oracle.cpp")]
    d = _cache_dir(*src)
    exe = os.path.join(d, "oracle_driver")
    if not os.path.exists(exe):
        _run(["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all", "-o", exe + ".tmp", *src])
        os.replace(exe + ".tmp", exe)
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1",
                         "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert "oracle driver ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("g++") is None, reason="needs hipcc and g++")
def test_c_abi_host_validation_under_asan_ubsan():
    csrc = os.path.join(ROOT, "kv_cache_quantization_row_amd", "csrc")
    api = os.path.join(csrc, "api.hip")
    drv = os.path.join(SAN, "abi_driver.cpp")
    d = _cache_dir(api, drv, os.path.join(csrc, "kernels.h"), os.path.join(ROOT, "include", "kvq.h"))
    exe = os.path.join(d, "abi_driver")
    if not os.path.exists(exe):
        api_o, drv_o = os.path.join(d, "api.o"), os.path.join(d, "drv.o")
        # sanitizers on the host code only (device code is built as usual)
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-c", api, "-o", api_o])
        _run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"), "-c", drv, "-o", drv_o])
        _run(["g++", "-fsanitize=address,undefined", "-o", exe + ".tmp", drv_o, api_o,
              "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
        os.replace(exe + ".tmp", exe)
    # the HIP runtime's own allocations are not this code's: leak checking off
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                         "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert "abi driver ok" in r.stdout
