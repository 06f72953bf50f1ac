"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The argument checks of every entry point (attn_api.hip, softmax_rows.hip,
gpu_clock.hip) are recompiled with the sanitizers on their host code only (the
gfx950 device code is unchanged and untouched by them), linked with the normal
device objects, and tests/test_abi.py runs against that library in a child
process with the sanitizer runtime preloaded: any out-of-bounds access, overflow
or other undefined behaviour in the validation path aborts the run.  CPU only.
"""

import os
import shutil
import subprocess
import sys

import pytest

from exact_attention_89_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SOURCES = ["attn_api.hip", "softmax_rows.hip", "gpu_clock.hip"]
CLANG = "/opt/rocm/lib/llvm/bin/clang"


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_library(tmp_path_factory):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("sanitizer runtime not found")
    srcs = [os.path.join(B.CSRC, f) for f in sorted(os.listdir(B.CSRC)) if f.endswith(".hip")]
    objs = [os.path.join(B.BUILD, os.path.basename(s) + ".o") for s in srcs]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    out = tmp_path_factory.mktemp("asan")
    flags = [f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"),
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    link = []
    for src, obj in zip(srcs, objs):
        if os.path.basename(src) in HOST_SOURCES:
            o = str(out / (os.path.basename(src) + ".o"))
            r = subprocess.run([B.HIPCC, *flags, "-c", src, "-o", o], capture_output=True,
                               text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            link.append(o)
        else:
            link.append(obj)
    lib = str(out / "libattn89.so")
    r = subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libsan",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        f"-Wl,-rpath,{os.path.dirname(runtime)}", "-o", lib, *link],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return lib, runtime


def test_abi_checks_under_sanitizers(sanitized_library):
    lib, runtime = sanitized_library
    env = dict(os.environ)
    env.update({
        "ATTN89_LIBRARY": lib,
        "LD_PRELOAD": runtime,
        # the interpreter itself is not instrumented: leaks at exit are not ours
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p",
                        "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail, tail
    assert "runtime error" not in tail, tail
