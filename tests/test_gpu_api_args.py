"""The Python binding checks caller-supplied outputs and workspaces before anything is
launched: the kernels write every element of O and LSE and use the whole workspace, so a
wrong shape, dtype, layout or device would mean writes out of bounds.  Valid caller
buffers give the same bits as the ones the binding allocates."""

import sys

import pytest

from exact_attention_89_amd import api

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

B, H, N, D = 1, 2, 64, 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    api.load_library()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(dtype=torch.bfloat16):
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    return [torch.randn((B, H, N, D), device="cuda", generator=g).to(dtype) for _ in range(3)]


WS = {"attn_partial": lambda: api.attn_partial_workspace_bytes(B, H, N, N),
      "attn_materialized": lambda: api.attn_materialized_workspace_bytes(B, H, N, N),
      "attn_fwd_splitkv": lambda: api.attn_splitkv_workspace_bytes(B, H, N, N, D, 0)}
FNS = ["attn_fwd", "attn_partial", "attn_materialized", "attn_fwd_splitkv",
       "attn_fwd_splitkv_noalloc", "attn_fwd_f32"]


@pytest.mark.parametrize("name", FNS)
def test_bad_outputs_rejected(name):
    _say(f"[api] {name}: output checks")
    dt = torch.float32 if name == "attn_fwd_f32" else torch.bfloat16
    q, k, v = _inputs(dt)
    fn = getattr(api, name)
    bad_out = [torch.empty((B, H, N - 1, D), dtype=dt, device="cuda"),
               torch.empty((B, H, N, D), dtype=torch.float16, device="cuda"),
               torch.empty((B, H, D, N), dtype=dt, device="cuda").transpose(2, 3),
               torch.empty((B, H, N, D), dtype=dt)]                       # host memory
    for o in bad_out:
        with pytest.raises(ValueError):
            fn(q, k, v, out=o)
    bad_lse = [torch.empty((B, H, N + 1), device="cuda"),
               torch.empty((B, H, N), dtype=torch.float64, device="cuda"),
               torch.empty((B, H, 2 * N), device="cuda")[..., ::2],
               torch.empty((B, H, N))]
    for l in bad_lse:
        with pytest.raises(ValueError):
            fn(q, k, v, lse=l)
    o_ref, l_ref = fn(q, k, v, causal=True)
    o = torch.full_like(o_ref, float("nan"))
    l = torch.full_like(l_ref, float("nan"))
    fn(q, k, v, causal=True, out=o, lse=l)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


@pytest.mark.parametrize("name", sorted(WS))
def test_bad_workspace_rejected(name):
    _say(f"[api] {name}: workspace checks")
    q, k, v = _inputs()
    fn = getattr(api, name)
    need = WS[name]()
    for ws in (torch.empty(need, dtype=torch.uint8),                                  # host
               torch.empty(2 * need, dtype=torch.uint8, device="cuda")[::2]):       # strided
        with pytest.raises(ValueError):
            fn(q, k, v, workspace=ws)
    o_ref, l_ref = fn(q, k, v)
    o, l = fn(q, k, v, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
