"""Build the HIP library ``libattn89.so`` in-tree for gfx950.

    python -m exact_attention_89_amd.build [--verbose]

Each ``csrc/*.hip`` file is compiled with hipcc for gfx950 only and the objects
are linked into ``exact_attention_89_amd/libattn89.so``.  Flags:

* ``-O3``, never fast-math: the kernels rely on IEEE -inf for masking.
* ``-Xclang -target-feature -Xclang -packed-fp32-ops`` turns off packed FP32
  instructions (hipcc warns that the host pass does not know the feature).
* ``-Rpass-analysis=kernel-resource-usage`` is kept in the log so register,
  scratch and LDS use of every kernel can be read after a build.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(HERE, "libattn89.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> tuple:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r.returncode, r.stdout + r.stderr


def build(verbose: bool = False) -> str:
    """Compile every kernel source and link the shared library; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    log = []
    for src, obj, rc, out in results:
        log.append(f"== {os.path.basename(src)} (rc={rc})\n{out}")
        if rc != 0:
            sys.stderr.write("\n".join(log))
            raise RuntimeError(f"hipcc failed on {src}")
    with open(os.path.join(BUILD, "resource_usage.log"), "w") as f:
        f.write("\n".join(log))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[obj for _, obj, _, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    _check_loads(tmp)
    os.replace(tmp, OUT)
    if verbose:
        sys.stdout.write("\n".join(log))
    _check_resources("\n".join(log))
    return OUT


def _check_loads(path: str) -> None:
    """dlopen the freshly linked library (in a child process, so this process never
    maps it): an unresolved symbol, e.g. a kernel stub the host pass did not emit,
    fails the build here rather than at first use."""
    code = f"import ctypes; ctypes.CDLL({path!r})"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"built library does not load: {r.stderr.strip()[-400:]}")


def _check_resources(log: str) -> None:
    """Fail the build if any kernel spills to scratch (a register-tiling failure)."""
    for line in log.splitlines():
        if "ScratchSize [bytes/lane]:" in line:
            n = int(line.rsplit(":", 1)[1].split()[0])
            if n != 0:
                raise RuntimeError(f"a kernel uses scratch memory: {line.strip()}")


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
