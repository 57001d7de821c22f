"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A second copy of libkvlr is built with the sanitizers on the host side only
(device code unoptimised, to keep the build short; no kernel is launched),
linked into tests/sanitize/abi_host.cpp, and run without a GPU: config
validation, buffer and workspace sizes, the rank helper and every argument
check that must fail before a device is touched, with leak detection on.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_decode_s4r_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    return res.returncode, res.stdout, err


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm clang not found")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    lib = tmp_path / "libkvlr_san.so"
    srcs = [os.path.join(CSRC, f) for f in ("api.hip", "decode.hip", "prefill.hip", "probe.hip")]
    host_flags = []
    for f in ["-O1", "-g"] + SAN:
        host_flags += ["-Xarch_host", f]
    rc, _, err = _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
                       "-Xarch_device", "-O0", "-Xclang", "-target-feature", "-Xclang",
                       "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
                       "-Wno-unused-result", "-Wno-pass-failed", "-o", str(lib)] + host_flags + srcs)
    assert rc == 0, err
    exe = tmp_path / "abi_host"
    rc, _, err = _run([CLANG, "-std=c++17", "-O1", "-g"] + SAN + [
        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "sanitize", "abi_host.cpp"),
        "-o", str(exe), "-L", str(tmp_path), "-lkvlr_san", f"-Wl,-rpath,{tmp_path}",
        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    assert rc == 0, err
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    rc, out, err = _run([str(exe)], env=env)
    assert rc == 0, out + err
    assert "host ABI checks passed" in out
    assert "ERROR: AddressSanitizer" not in err and "runtime error" not in err
    shutil.rmtree(tmp_path, ignore_errors=True)
