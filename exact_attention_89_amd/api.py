"""Python binding of the C ABI in ``include/attn.h`` (argument marshalling only).

Every step of attention runs in the HIP library ``libattn89.so`` that sits next
to this file.  torch is used for device memory and streams: tensors are
checked for device, dtype, shape and contiguity, and their pointers are passed
through ctypes together with the current HIP stream.  There is no CPU fallback:
if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libattn89.so"
_lib = None

ATTN_OK = 0
_STATUS_NAMES = {
    -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_UNSUPPORTED",
    -4: "ATTN_ERR_ALIGN", -5: "ATTN_ERR_SCALE", -6: "ATTN_ERR_WORKSPACE",
    -7: "ATTN_ERR_HIP", -8: "ATTN_ERR_TOO_LARGE", -9: "ATTN_ERR_SCRATCH",
}

# bf16 forward kernel choice (attn_fwd_select_kernel)
ATTN_KERNEL_AUTO = 0
ATTN_KERNEL_PINGPONG = 1
ATTN_KERNEL_FOURWAVE = 2
ATTN_KERNEL_KEYGROUPS = 3

# exported symbol -> (restype, argtypes); must match include/attn.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_U64 = ctypes.c_uint64
EXPORTS = {
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P]),
    "attn_fwd_select_kernel": (_I, [_I]),
    "attn_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P]),
    "attn_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                             _P]),
    "attn_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _I, _P, _P]),
    "attn_materialized_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "attn_materialized": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P, _SZ,
                               _P]),
    "attn_partial_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "attn_splitkv_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "attn_splitkv_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "attn_fwd_splitkv": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _I, _P, _SZ,
                              _P]),
    "attn_partial": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P, _SZ, _P]),
    "attn_fwd_splitkv_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _I,
                                      _P]),
    "attn_strerror": (ctypes.c_char_p, [_I]),
    "attn_abi_version": (_I, []),
    "softmax_rows_f32": (_I, [_P, _P, _I, _I, _P]),
    "softmax_rows_unfused_workspace_bytes": (_SZ, [_I]),
    "softmax_rows_unfused_f32": (_I, [_P, _P, _I, _I, _P, _SZ, _P]),
    "attn_clock_sampler": (_I, [_P, _P, _I, _I, _U64, _U64, _P]),
    "attn_clock_mark": (_I, [_P, _I, _P]),
    "attn_clock_wall_hz": (ctypes.c_int64, []),
}


class AttnError(RuntimeError):
    """A negative status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.attn_strerror(status).decode() if _lib is not None else "?"
        super().__init__(f"{where}: {_STATUS_NAMES.get(status, status)} ({msg})")


def library_path() -> str:
    """The in-tree HIP library, or the build named by ATTN89_LIBRARY (used by the tests
    to load a host-sanitised build of the same sources)."""
    return os.environ.get("ATTN89_LIBRARY") or os.path.join(_HERE, _LIB_NAME)


def load_library(path: Optional[str] = None):
    """Load (once) and return the ctypes handle of the HIP library; raise if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()'"
            " or python -m exact_attention_89_amd.build)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != ATTN_OK:
        raise AttnError(status, where)


def _stream_handle(torch, device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _prep(q, k, v, kv_lens, dtype):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, D]")
    B, H, Nq, D = q.shape
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} "
                         f"v {tuple(v.shape)}")
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    if kv_lens is not None:
        if not isinstance(kv_lens, torch.Tensor):
            kv_lens = torch.tensor(kv_lens, dtype=torch.int32, device=q.device)
        kv_lens = kv_lens.to(device=q.device, dtype=torch.int32).contiguous()
        if kv_lens.numel() != B:
            raise ValueError("kv_lens must hold one length per batch entry")
    return torch, q, k, v, kv_lens, (B, H, Nq, k.shape[2], D)


def _outputs(torch, q, out, lse, dtype, lse_shape):
    """Allocate O (like q, of `dtype`) and the LSE, or check the caller's: the kernels
    write every element, so a wrong shape, type or layout would write out of bounds."""
    o = torch.empty(q.shape, dtype=dtype, device=q.device) if out is None else out
    l = torch.empty(lse_shape, dtype=torch.float32, device=q.device) if lse is None else lse
    if (not isinstance(o, torch.Tensor) or o.shape != q.shape or o.dtype != dtype
            or not o.is_contiguous() or o.device != q.device):
        raise ValueError(f"out must be a contiguous {dtype} tensor shaped like q on q's device")
    if (not isinstance(l, torch.Tensor) or tuple(l.shape) != tuple(lse_shape)
            or l.dtype != torch.float32 or not l.is_contiguous() or l.device != q.device):
        raise ValueError(f"lse must be a contiguous float32 {list(lse_shape)} tensor on q's "
                         "device")
    return o, l


def _workspace(torch, q, workspace, need):
    """Allocate the workspace, or check the caller's (the library checks its size)."""
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=q.device)
    if (not isinstance(workspace, torch.Tensor) or workspace.device != q.device
            or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on q's device")
    return workspace


def _call_fwd(fname, q, k, v, scale, causal, kv_lens, out, lse, dtype):
    torch, q, k, v, kv_lens, (B, H, Nq, Nk, D) = _prep(q, k, v, kv_lens, dtype)
    if scale is None:
        scale = D ** -0.5
    o, l = _outputs(torch, q, out, lse, dtype, (B, H, Nq))
    lib = load_library()
    st = getattr(lib, fname)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             l.data_ptr(), B, H, Nq, Nk, D, float(scale), int(bool(causal)),
                             kv_lens.data_ptr() if kv_lens is not None else None,
                             _stream_handle(torch, q.device))
    _check(st, fname)
    return o, l


def attn_fwd(q, k, v, scale: Optional[float] = None, causal: bool = False, kv_lens=None,
             out=None, lse=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Fused attention forward, bf16 in/out, fp32 LSE.  Returns (o, lse)."""
    import torch
    return _call_fwd("attn_fwd", q, k, v, scale, causal, kv_lens, out, lse, torch.bfloat16)


def attn_fwd_select_kernel(which: int) -> int:
    """Choose the bf16 forward kernel (ATTN_KERNEL_*); returns the previous choice."""
    st = load_library().attn_fwd_select_kernel(int(which))
    if st < 0:
        raise AttnError(st, "attn_fwd_select_kernel")
    return st


def attn_fwd_f32(q, k, v, scale: Optional[float] = None, causal: bool = False, kv_lens=None,
                 out=None, lse=None):
    """Fused attention forward, fp32 in/out.  Returns (o, lse)."""
    import torch
    return _call_fwd("attn_fwd_f32", q, k, v, scale, causal, kv_lens, out, lse, torch.float32)


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: Optional[int] = None,
                    max_seqlen_k: Optional[int] = None, scale: Optional[float] = None,
                    causal: bool = False, out=None, lse=None):
    """Fused forward over packed variable-length sequences, bf16.

    q [total_q, H, D], k and v [total_k, H, D] (token-major); cu_seqlens_q / _k: B + 1
    cumulative offsets (int32, device or host).  Returns (o [total_q, H, D] bf16,
    lse [H, total_q] fp32).  The longest lengths are taken from the offsets when not
    given (a host copy of them)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a bf16 GPU tensor")
        if t.dim() != 3:
            raise ValueError(f"{name} must be [tokens, H, D]")
    total_q, H, D = q.shape
    total_k = k.shape[0]
    if k.shape[1:] != (H, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} "
                         f"v {tuple(v.shape)}")
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    cus = []
    for cu in (cu_seqlens_q, cu_seqlens_k):
        if not isinstance(cu, torch.Tensor):
            cu = torch.tensor(cu, dtype=torch.int32)
        cus.append(cu.to(device=q.device, dtype=torch.int32).contiguous())
    cu_q, cu_k = cus
    B = cu_q.numel() - 1
    if B < 1 or cu_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must hold B + 1 >= 2 offsets each")
    if max_seqlen_q is None or max_seqlen_k is None:
        hq, hk = cu_q.cpu(), cu_k.cpu()
        if max_seqlen_q is None:
            max_seqlen_q = max(1, int((hq[1:] - hq[:-1]).max()))
        if max_seqlen_k is None:
            max_seqlen_k = max(1, int((hk[1:] - hk[:-1]).max()))
    if scale is None:
        scale = D ** -0.5
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((H, total_q), dtype=torch.float32, device=q.device) if lse is None else lse
    if o.shape != q.shape or o.dtype != torch.bfloat16 or not o.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    if l.shape != (H, total_q) or l.dtype != torch.float32 or not l.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [H, total_q] tensor")
    st = load_library().attn_fwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), cu_q.data_ptr(),
        cu_k.data_ptr(), B, H, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), D,
        float(scale), int(bool(causal)), _stream_handle(torch, q.device))
    _check(st, "attn_fwd_varlen")
    return o, l


def attn_fwd_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float,
                 scale: Optional[float] = None, causal: bool = False, kv_lens=None, out=None,
                 lse=None):
    """Fused attention forward on E4M3 codes (uint8 or float8_e4m3fn tensors) with one
    descale factor per tensor; bf16 output.  Returns (o, lse)."""
    import torch
    codes = []
    for name, t in (("q", q), ("k", k), ("v", v)):
        if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
            t = t.view(torch.uint8)
        codes.append(t)
    torch, q, k, v, kv_lens, (B, H, Nq, Nk, D) = _prep(*codes, kv_lens, torch.uint8)
    if scale is None:
        scale = D ** -0.5
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
    l = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    if o.shape != q.shape or o.dtype != torch.bfloat16 or not o.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    if l.shape != (B, H, Nq) or l.dtype != torch.float32 or not l.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    st = load_library().attn_fwd_fp8(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), B, H, Nq, Nk, D,
        float(scale), float(q_descale), float(k_descale), float(v_descale), int(bool(causal)),
        kv_lens.data_ptr() if kv_lens is not None else None, _stream_handle(torch, q.device))
    _check(st, "attn_fwd_fp8")
    return o, l


def attn_materialized_workspace_bytes(B: int, H: int, Nq: int, Nk: int) -> int:
    return int(load_library().attn_materialized_workspace_bytes(B, H, Nq, Nk))


def attn_materialized(q, k, v, scale: Optional[float] = None, causal: bool = False,
                      kv_lens=None, workspace=None, out=None, lse=None):
    """The unfused three-launch baseline (S and P go through device memory)."""
    torch, q, k, v, kv_lens, (B, H, Nq, Nk, D) = _prep(q, k, v, kv_lens, torch_bf16())
    if scale is None:
        scale = D ** -0.5
    lib = load_library()
    need = 0 if workspace is not None else int(lib.attn_materialized_workspace_bytes(B, H, Nq, Nk))
    workspace = _workspace(torch, q, workspace, need)
    o, l = _outputs(torch, q, out, lse, torch_bf16(), (B, H, Nq))
    st = lib.attn_materialized(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               l.data_ptr(), B, H, Nq, Nk, D, float(scale), int(bool(causal)),
                               kv_lens.data_ptr() if kv_lens is not None else None,
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               _stream_handle(torch, q.device))
    _check(st, "attn_materialized")
    return o, l


def _rows_prep(x, out):
    import torch
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a CUDA (HIP) tensor")
    if x.dtype != torch.float32:
        raise ValueError("x must be float32")
    if x.dim() < 1:
        raise ValueError("x needs at least one dimension")
    x = x.contiguous()
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != torch.float32 or not y.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like x")
    return torch, x, y, rows, cols


def softmax_rows(x, out=None):
    """Row softmax along the last dimension, fp32, fused kernel (one launch)."""
    torch, x, y, rows, cols = _rows_prep(x, out)
    st = load_library().softmax_rows_f32(x.data_ptr(), y.data_ptr(), rows, cols,
                                         _stream_handle(torch, x.device))
    _check(st, "softmax_rows_f32")
    return y


def softmax_rows_unfused(x, out=None, workspace=None):
    """Row softmax along the last dimension, fp32, the unfused four-launch baseline."""
    torch, x, y, rows, cols = _rows_prep(x, out)
    lib = load_library()
    need = int(lib.softmax_rows_unfused_workspace_bytes(rows))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    st = lib.softmax_rows_unfused_f32(x.data_ptr(), y.data_ptr(), rows, cols,
                                      workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(),
                                      _stream_handle(torch, x.device))
    _check(st, "softmax_rows_unfused_f32")
    return y


def attn_partial_workspace_bytes(B: int, H: int, Nq: int, Nk: int) -> int:
    return int(load_library().attn_partial_workspace_bytes(B, H, Nq, Nk))


def attn_partial(q, k, v, scale: Optional[float] = None, causal: bool = False,
                 kv_lens=None, workspace=None, out=None, lse=None):
    """Partial fusion: QK^T + softmax in one launch writing P, then P V (two launches)."""
    torch, q, k, v, kv_lens, (B, H, Nq, Nk, D) = _prep(q, k, v, kv_lens, torch_bf16())
    if scale is None:
        scale = D ** -0.5
    lib = load_library()
    need = 0 if workspace is not None else int(lib.attn_partial_workspace_bytes(B, H, Nq, Nk))
    workspace = _workspace(torch, q, workspace, need)
    o, l = _outputs(torch, q, out, lse, torch_bf16(), (B, H, Nq))
    st = lib.attn_partial(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          l.data_ptr(), B, H, Nq, Nk, D, float(scale), int(bool(causal)),
                          kv_lens.data_ptr() if kv_lens is not None else None,
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          _stream_handle(torch, q.device))
    _check(st, "attn_partial")
    return o, l


def attn_splitkv_workspace_bytes(B: int, H: int, Nq: int, Nk: int, D: int,
                                 num_splits: int = 0) -> int:
    return int(load_library().attn_splitkv_workspace_bytes(B, H, Nq, Nk, D, num_splits))


def attn_fwd_splitkv(q, k, v, scale: Optional[float] = None, causal: bool = False,
                     kv_lens=None, num_splits: int = 0, workspace=None, out=None, lse=None):
    """Fused forward with the keys split across workgroups, then merged (two launches)."""
    torch, q, k, v, kv_lens, (B, H, Nq, Nk, D) = _prep(q, k, v, kv_lens, torch_bf16())
    if scale is None:
        scale = D ** -0.5
    lib = load_library()
    need = 0 if workspace is not None else int(
        lib.attn_splitkv_workspace_bytes(B, H, Nq, Nk, D, int(num_splits)))
    workspace = _workspace(torch, q, workspace, need)
    o, l = _outputs(torch, q, out, lse, torch_bf16(), (B, H, Nq))
    st = lib.attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              l.data_ptr(), B, H, Nq, Nk, D, float(scale), int(bool(causal)),
                              kv_lens.data_ptr() if kv_lens is not None else None,
                              int(num_splits), workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(),
                              _stream_handle(torch, q.device))
    _check(st, "attn_fwd_splitkv")
    return o, l


NOALLOC_SCRATCH_BYTES = 16 << 20   # ATTN_NOALLOC_SCRATCH_BYTES of include/attn.h


def attn_fwd_splitkv_noalloc(q, k, v, scale: Optional[float] = None, causal: bool = False,
                             kv_lens=None, num_splits: int = 0, out=None, lse=None):
    """attn_fwd_splitkv with the library's fixed scratch instead of a workspace (the
    C entry point allocates nothing; pass ``out`` and ``lse`` to allocate nothing here
    either)."""
    torch, q, k, v, kv_lens, (B, H, Nq, Nk, D) = _prep(q, k, v, kv_lens, torch_bf16())
    if scale is None:
        scale = D ** -0.5
    o, l = _outputs(torch, q, out, lse, torch_bf16(), (B, H, Nq))
    st = load_library().attn_fwd_splitkv_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), B, H, Nq, Nk, D,
        float(scale), int(bool(causal)), kv_lens.data_ptr() if kv_lens is not None else None,
        int(num_splits), _stream_handle(torch, q.device))
    _check(st, "attn_fwd_splitkv_noalloc")
    return o, l


def torch_bf16():
    import torch
    return torch.bfloat16


# ---- shader-clock sampling (include/gpu_clock.h), a measurement aid ----

def clock_wall_hz() -> int:
    """Frequency of the device's wall-clock counter in Hz."""
    hz = int(load_library().attn_clock_wall_hz())
    if hz <= 0:
        raise AttnError(hz, "attn_clock_wall_hz")
    return hz


def clock_sampler(samples, phase, stop_value: int, max_samples: int, interval_ticks: int,
                  duration_ticks: int, stream=None) -> None:
    """Start the one-wave sampler writing (wall ticks, shader cycles, phase) triples into
    ``samples`` (int64 GPU tensor of 3 * max_samples + 1 entries; ``phase`` an int32 GPU
    tensor) on ``stream``; it ends once ``phase`` holds ``stop_value``."""
    import torch
    if samples.dtype != torch.int64 or samples.numel() < 3 * max_samples + 1:
        raise ValueError("samples must be an int64 tensor of 3 * max_samples + 1 entries")
    if phase.dtype != torch.int32 or phase.numel() < 1:
        raise ValueError("phase must be an int32 tensor")
    s = (stream or torch.cuda.current_stream(samples.device)).cuda_stream
    _check(load_library().attn_clock_sampler(samples.data_ptr(), phase.data_ptr(),
                                             int(stop_value), int(max_samples),
                                             int(interval_ticks), int(duration_ticks), s),
           "attn_clock_sampler")


def clock_mark(phase, value: int, stream=None) -> None:
    """Store ``value`` into ``phase`` (int32 GPU tensor) when ``stream`` reaches this point."""
    import torch
    if phase.dtype != torch.int32 or phase.numel() < 1:
        raise ValueError("phase must be an int32 tensor")
    s = (stream or torch.cuda.current_stream(phase.device)).cuda_stream
    _check(load_library().attn_clock_mark(phase.data_ptr(), int(value), s), "attn_clock_mark")
