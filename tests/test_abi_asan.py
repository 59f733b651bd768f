"""The C-ABI layer's host-side argument handling under AddressSanitizer (CPU only): the library's
sources are built with ASan on their host code (device code as usual) and linked into a small
driver that calls every entry point with invalid arguments; no GPU is touched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "packed_sequence_causal_pk_amd", "csrc")
OUT = os.path.join(ROOT, "packed_sequence_causal_pk_amd", "_build", "asan")
DRIVER = os.path.join(ROOT, "tests", "host_asan", "abi_host_check.cpp")


def _tool(name, fallback):
    return shutil.which(name) or fallback


def test_abi_host_paths_under_asan():
    from packed_sequence_causal_pk_amd import build
    hipcc = _tool("hipcc", "/opt/rocm/bin/hipcc")
    clangxx = "/opt/rocm/lib/llvm/bin/clang++"
    if not os.path.exists(hipcc) or not os.path.exists(clangxx):
        pytest.skip("ROCm compilers not present")
    os.makedirs(OUT, exist_ok=True)
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["-O1", "-std=c++17", "-fPIC", "--offload-arch=" + build.ARCH, "-munsafe-fp-atomics",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
    procs, objs = [], []
    for src in build.SOURCES + [DRIVER]:
        obj = os.path.join(OUT, os.path.splitext(os.path.basename(src))[0] + ".o")
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        lang = ["-x", "hip"] if path.endswith(".cpp") else []
        procs.append(subprocess.Popen([hipcc] + lang + flags + host_asan + ["-c", path, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out[-2000:]
    exe = os.path.join(OUT, "abi_host_check")
    link = subprocess.run([clangxx, "-fsanitize=address", "-o", exe] + objs +
                          ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                          capture_output=True, text=True, timeout=300)
    assert link.returncode == 0, link.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert "AddressSanitizer" not in run.stderr, run.stderr[-3000:]
    assert run.returncode == 0 and run.stdout.strip().endswith("OK"), run.stdout + run.stderr[-2000:]
