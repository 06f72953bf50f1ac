"""The C ABI without a GPU: the library loads, exports every function the header
declares, and rejects invalid arguments before launching anything (these calls
return from host-side checks and never touch a device)."""

import ctypes
import glob
import os
import re

import pytest

from exact_attention_89_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:attn|softmax_rows)\w*)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.library_path()):
        from exact_attention_89_amd import build
        build.build()
    return api.load_library()


def test_header_declares_the_boundary():
    names = _declared()
    assert names == sorted(["attn_fwd", "attn_fwd_f32", "attn_materialized",
                            "attn_materialized_workspace_bytes", "attn_strerror",
                            "attn_abi_version", "attn_fwd_select_kernel",
                            "softmax_rows_f32", "softmax_rows_unfused_workspace_bytes",
                            "softmax_rows_unfused_f32", "attn_partial",
                            "attn_partial_workspace_bytes", "attn_fwd_splitkv",
                            "attn_splitkv_num_splits", "attn_splitkv_workspace_bytes",
                            "attn_fwd_fp8", "attn_fwd_varlen", "attn_fwd_splitkv_noalloc",
                            "attn_clock_sampler",
                            "attn_clock_mark", "attn_clock_wall_hz"])


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in api.EXPORTS, f"binding does not describe {name}"


def test_status_strings(lib):
    assert lib.attn_abi_version() == 2
    for st in range(-9, 1):
        assert lib.attn_strerror(st)
    assert lib.attn_strerror(-99) == b"unknown status"


def test_workspace_size(lib):
    # S fp32 + P bf16 over [B][H][Nq][round_up(Nk, 64)], P starting 256-byte aligned
    assert lib.attn_materialized_workspace_bytes(1, 32, 8192, 8192) == 32 * 8192 * 8192 * 6
    assert lib.attn_materialized_workspace_bytes(2, 3, 5, 70) == 2 * 3 * 5 * 128 * 6 + 0
    assert lib.attn_materialized_workspace_bytes(0, 1, 1, 1) == 0
    assert lib.attn_materialized_workspace_bytes(1, 1, 1, -5) == 0


A = 1 << 20  # a 16-byte aligned fake address: these calls must fail before any use


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_f32"])
def test_invalid_arguments(lib, fn):
    f = getattr(lib, fn)

    def call(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, Nq=8, Nk=8, D=64, scale=0.125, causal=0,
             kv=None):
        return f(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, kv, None)

    assert call(q=None) == -1
    assert call(lse=None) == -1
    assert call(B=0) == -2
    assert call(Nk=-1) == -2
    assert call(B=1 << 30, H=1 << 30, Nq=1 << 30) == -2
    assert call(D=96) == -3
    assert call(D=0) == -3
    assert call(q=A + 8) == -4
    assert call(o=A + 2) == -4
    assert call(lse=A + 2) == -4
    assert call(kv=A + 1) == -4
    assert call(scale=float("nan")) == -5
    assert call(scale=float("-inf")) == -5


def test_materialized_invalid_arguments(lib):
    f = lib.attn_materialized
    need = lib.attn_materialized_workspace_bytes(1, 1, 8, 8)
    assert f(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 0, None, None, need, None) == -6
    assert f(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 0, None, A, need - 1, None) == -6
    assert f(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 0, None, A + 16, need, None) == -6
    assert f(A, A, A, A, A, 1, 1, 8, 8, 80, 0.1, 0, None, A, need, None) == -3


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        api.attn_fwd(x, x, x)


def test_product_path_does_not_touch_the_oracle():
    """The package never imports the oracle (it is test infrastructure only)."""
    pkg = os.path.join(ROOT, "exact_attention_89_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), fn
                assert "attn_oracle" not in text, fn


def test_select_kernel_validates_and_returns_previous(lib):
    """Setting the bf16 kernel choice launches nothing (safe without a GPU)."""
    assert lib.attn_fwd_select_kernel(7) == -3
    assert lib.attn_fwd_select_kernel(-1) == -3
    prev = lib.attn_fwd_select_kernel(api.ATTN_KERNEL_FOURWAVE)
    assert prev == api.ATTN_KERNEL_AUTO
    assert lib.attn_fwd_select_kernel(api.ATTN_KERNEL_PINGPONG) == api.ATTN_KERNEL_FOURWAVE
    assert api.attn_fwd_select_kernel(api.ATTN_KERNEL_AUTO) == api.ATTN_KERNEL_PINGPONG



def test_softmax_rows_rejects_bad_arguments(lib):
    """Host-side checks of the row-softmax entry points (nothing is launched)."""
    p = ctypes.c_void_p(0x10000)          # aligned, never dereferenced
    odd = ctypes.c_void_p(0x10002)        # not 4-byte aligned
    assert lib.softmax_rows_f32(None, p, 1, 1, None) == -1
    assert lib.softmax_rows_f32(p, p, 0, 4, None) == -2
    assert lib.softmax_rows_f32(p, p, 4, 0, None) == -2
    assert lib.softmax_rows_f32(p, p, 1, 1 << 30, None) == -8
    assert lib.softmax_rows_f32(odd, p, 1, 4, None) == -4
    assert lib.softmax_rows_unfused_workspace_bytes(0) == 0
    need = lib.softmax_rows_unfused_workspace_bytes(1000)
    assert need >= 2 * 1000 * 4 and need % 256 == 0
    assert lib.softmax_rows_unfused_f32(p, p, 1000, 8, p, need - 1, None) == -6
    assert lib.softmax_rows_unfused_f32(p, p, 1000, 8, None, need, None) == -6
    assert lib.softmax_rows_unfused_f32(p, p, 1000, 8, ctypes.c_void_p(0x10040), need,
                                        None) == -6


def test_splitkv_plan_and_checks(lib):
    """The number of key ranges used for an explicit request (whole 64-key tiles) and
    the host-side checks of attn_fwd_splitkv (nothing is launched)."""
    assert lib.attn_splitkv_num_splits(1, 1, 1, 100, 5) == 2        # 2 tiles
    assert lib.attn_splitkv_num_splits(1, 1, 1, 640, 1) == 1
    assert lib.attn_splitkv_num_splits(1, 1, 1, 640, 3) == 3        # 4 + 4 + 2 tiles
    assert lib.attn_splitkv_num_splits(1, 1, 1, 640, 4) == 4        # 3 + 3 + 3 + 1
    assert lib.attn_splitkv_num_splits(1, 1, 1, 640, 6) == 5        # 2 tiles each
    assert lib.attn_splitkv_num_splits(0, 1, 1, 640, 6) == -2
    assert lib.attn_splitkv_workspace_bytes(1, 1, 1, 640, 96, 3) == 0   # unsupported D
    need = lib.attn_splitkv_workspace_bytes(2, 3, 5, 640, 128, 3)
    assert need >= 3 * 2 * 3 * 5 * (128 + 1) * 4 and need % 256 == 0
    p = ctypes.c_void_p(0x10000)
    args = [p, p, p, p, p, 2, 3, 5, 640, 128, ctypes.c_float(0.1), 0, None, 3]
    assert lib.attn_fwd_splitkv(*args, p, need - 1, None) == -6
    assert lib.attn_fwd_splitkv(*args, None, need, None) == -6
    assert lib.attn_fwd_splitkv(None, *args[1:], p, need, None) == -1


def test_headers_compile_and_link_as_c(tmp_path, lib):
    """A C99 program (gcc, -Wall -Wextra -pedantic -Werror) includes every header,
    takes the address of every declared function (so the linker resolves each one
    against libattn89.so) and calls the host-side checks: the boundary is plain C."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    names = _declared()
    src = tmp_path / "abi.c"
    src.write_text(
        "#include <stdio.h>\n" +
        "".join(f"#include \"{os.path.basename(h)}\"\n" for h in HEADERS) +
        "typedef void (*fn_t)(void);\n"
        "static const fn_t all[] = {" + ", ".join(f"(fn_t){n}" for n in names) + "};\n"
        "int main(void) {\n"
        "  int st = attn_fwd(NULL, NULL, NULL, NULL, NULL, 1, 1, 1, 1, 64, 0.125f, 0, NULL, NULL);\n"
        "  int st2 = softmax_rows_f32(NULL, NULL, 1, 1, NULL);\n"
        "  printf(\"%d %d %d %u\\n\", attn_abi_version(), st, st2, (unsigned)(sizeof all / sizeof *all));\n"
        "  return (st == ATTN_ERR_NULL && st2 == ATTN_ERR_NULL) ? 0 : 1;\n}\n")
    exe = tmp_path / "abi"
    libdir = os.path.dirname(api.library_path())
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-Wno-cast-function-type", "-I", os.path.join(ROOT, "include"), str(src),
           "-L", libdir, "-l:libattn89.so", f"-Wl,-rpath,{libdir}",
           "-Wl,-rpath-link,/opt/rocm/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.split() == ["2", "-1", "-1", str(len(names))]


def test_splitkv_noalloc_host_checks(lib):
    """attn_fwd_splitkv_noalloc: argument checks and the fixed-scratch limit are host
    checks, decided before the scratch address is looked up or anything is launched."""
    p = ctypes.c_void_p(0x10000)
    limit = 16 << 20                                   # ATTN_NOALLOC_SCRATCH_BYTES
    assert api.NOALLOC_SCRATCH_BYTES == limit
    big = (1, 64, 4096, 65536, 128, 64)                # B, H, Nq, Nk, D, splits
    assert lib.attn_splitkv_workspace_bytes(*big) > limit

    def call(q=p, B=1, H=64, Nq=4096, Nk=65536, D=128, splits=64, scale=0.1):
        return lib.attn_fwd_splitkv_noalloc(q, p, p, p, p, B, H, Nq, Nk, D,
                                            ctypes.c_float(scale), 0, None, splits, None)

    assert call() == -9                                # does not fit the scratch
    assert lib.attn_strerror(-9)
    assert call(q=None) == -1
    assert call(D=96) == -3
    assert call(B=0) == -2
    assert call(scale=float("nan")) == -5
