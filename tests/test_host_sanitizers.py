"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/host_api_check.c (a C caller) drives the C ABI through every
plan kind and every documented error path; it is linked with the C-ABI sources and the
smaller kernel files compiled with the sanitizers on the host side (device
code for gfx950 is built as usual and never runs here), and with host-only
stand-ins for the launchers of the largest kernel files
(tests/sanitize/stub_launchers.cpp).  Any sanitizer report fails the run."""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "group_dft_structured_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
REAL = ["eqlinear_api.hip", "eqconv_api.hip", "k_spectra.hip", "k_spectral_gemm.hip",
        "k_bwd_weight.hip", "k_bwd_weight_ws.hip", "k_p4m_pairs.hip"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined",
         "-Xarch_host", "-fno-omit-frame-pointer",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src, out_dir):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return obj


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_host_code_under_asan_and_ubsan(tmp_path):
    srcs = [os.path.join(CSRC, s) for s in REAL] + [
        os.path.join(ROOT, "tests", "sanitize", "stub_launchers.cpp")]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
        objs = list(ex.map(lambda s: _compile(s, str(tmp_path)), srcs))
    # the driver is C: a C caller may pass any int for an enumeration argument
    drv = os.path.join(str(tmp_path), "host_api_check.o")
    r = subprocess.run([CLANG, "-x", "c", "-std=c11", "-O1", "-g", "-fsanitize=address",
                        "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                        "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "sanitize", "host_api_check.c"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    objs.append(drv)
    exe = os.path.join(str(tmp_path), "host_api_check")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-o", exe] + objs,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0 and "ok" in r.stdout, out[-4000:]
