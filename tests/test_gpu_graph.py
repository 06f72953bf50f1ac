"""Calls captured in a HIP graph (torch.cuda.CUDAGraph over the library's launches on the
capturing stream) and replayed: every replay, with new inputs copied in between by
ordinary eager work, must give bit for bit what the eager call gives on the same inputs.
The no-allocation split-key entry point exists for such callers; attn_fwd, the
allocating split-key entry point (with a workspace made before capture), the FP8 and
variable-length entry points and the row softmax are covered too.
Nothing is allocated inside a capture: outputs, workspaces and inputs are made first."""

import math
import sys

import numpy as np
import pytest

import oracle
from exact_attention_89_amd import api
from exact_attention_89_amd.workloads import random_case, random_fp8_case
from tests.parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    api.load_library()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _fill(dst, seed, B, H, Nq, Nk, D, lens):
    q, k, v, lens = random_case(seed, B, H, Nq, Nk, D, "bf16", lens)
    for t, x in zip(dst, (q, k, v)):
        t.copy_(torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16))
    return q, k, v, lens


def _run_captured(name, B, H, Nq, Nk, D, causal, lens, call, with_oracle_first=True):
    """Capture call(q, k, v, kvl, o, l) once, then replay it on fresh inputs."""
    _say(f"[graph] {name}: B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} lens={lens}")
    dev = torch.device("cuda")
    q = torch.empty((B, H, Nq, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty((B, H, Nk, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    kvl = None if lens is None else torch.tensor(np.asarray(lens, np.int32), device=dev)
    o = torch.empty_like(q)
    l = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    o_ref = torch.empty_like(o)
    l_ref = torch.empty_like(l)
    _fill((q, k, v), 900, B, H, Nq, Nk, D, lens)
    # warm-up on a side stream, as torch requires before capturing
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(q, k, v, kvl, o, l)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(q, k, v, kvl, o, l)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        qh, kh, vh, lens_h = _fill((q, k, v), 901 + r, B, H, Nq, Nk, D, lens)
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        o_g, l_g = o.clone(), l.clone()
        call(q, k, v, kvl, o_ref, l_ref)          # the same call, eager
        torch.cuda.synchronize()
        _say(f"[graph]   replay {r}")
        assert torch.equal(o_g, o_ref), f"{name}: replay {r} O differs from the eager call"
        assert torch.equal(l_g, l_ref), f"{name}: replay {r} LSE differs from the eager call"
        if with_oracle_first and r == 0:
            scale = 1.0 / math.sqrt(D)
            ro, rl = oracle.attention_oracle(qh, kh, vh, scale, causal=causal, kv_lens=lens_h)
            check(o_g.float().cpu().numpy(), l_g.cpu().numpy(), ro, rl, "bf16", name)


@pytest.mark.parametrize("B,H,Nq,Nk,D,causal,lens,splits", [
    (2, 4, 1, 3000, 128, False, [3000, 1700], 0),
    (1, 3, 5, 700, 64, True, None, 3),
])
def test_splitkv_noalloc_replays(B, H, Nq, Nk, D, causal, lens, splits):
    scale = 1.0 / math.sqrt(D)

    def call(q, k, v, kvl, o, l):
        api.attn_fwd_splitkv_noalloc(q, k, v, scale=scale, causal=causal, kv_lens=kvl,
                                     num_splits=splits, out=o, lse=l)
    _run_captured("attn_fwd_splitkv_noalloc", B, H, Nq, Nk, D, causal, lens, call)


def test_splitkv_workspace_replays():
    B, H, Nq, Nk, D = 1, 8, 2, 4096, 128
    scale = 1.0 / math.sqrt(D)
    ws = torch.empty(api.attn_splitkv_workspace_bytes(B, H, Nq, Nk, D, 0), dtype=torch.uint8,
                     device="cuda")

    def call(q, k, v, kvl, o, l):
        api.attn_fwd_splitkv(q, k, v, scale=scale, kv_lens=kvl, workspace=ws, out=o, lse=l)
    _run_captured("attn_fwd_splitkv", B, H, Nq, Nk, D, False, None, call)


@pytest.mark.parametrize("B,H,N,D,causal,lens", [
    (1, 32, 2048, 128, True, None),        # the 8-wave kernel (grid of 256 blocks)
    (2, 4, 333, 64, False, [333, 100]),     # the 4-wave kernels
])
def test_attn_fwd_replays(B, H, N, D, causal, lens):
    scale = 1.0 / math.sqrt(D)

    def call(q, k, v, kvl, o, l):
        api.attn_fwd(q, k, v, scale=scale, causal=causal, kv_lens=kvl, out=o, lse=l)
    _run_captured("attn_fwd", B, H, N, N, D, causal, lens, call,
                  with_oracle_first=(B * H * N <= 2 * 4 * 333))


def _capture_and_replay(name, refill, call, outs):
    """Capture call() (which writes the tensors in `outs`), then for each replay refill
    the inputs eagerly, replay, and compare every output bit for bit with the same call
    made eagerly on the same inputs."""
    _say(f"[graph] {name}")
    refill(900)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        refill(901 + r)
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        call()
        torch.cuda.synchronize()
        _say(f"[graph]   replay {r}")
        for a, b in zip(got, outs):
            assert torch.equal(a, b), f"{name}: replay {r} differs from the eager call"
            assert not torch.isnan(a.float()).any(), f"{name}: replay {r} left NaN"


def test_fp8_replays():
    B, H, N, D = 2, 4, 300, 128
    dev = "cuda"
    q, k, v = (torch.empty((B, H, N, D), dtype=torch.uint8, device=dev) for _ in range(3))
    kvl = torch.tensor([300, 170], dtype=torch.int32, device=dev)
    o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    l = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    def refill(seed):
        # fresh E4M3 codes; the descale factors are kernel arguments, fixed at capture
        for t, x in zip((q, k, v), random_fp8_case(seed, B, H, N, N, D)[:3]):
            t.copy_(torch.from_numpy(np.ascontiguousarray(x)))

    def call():
        api.attn_fwd_fp8(q, k, v, 0.02, 0.03, 0.01, causal=True, kv_lens=kvl, out=o, lse=l)
    _capture_and_replay("attn_fwd_fp8 B=2 H=4 N=300 D=128 causal, key lengths", refill, call,
                        [o, l])


def test_varlen_replays():
    H, D = 4, 64
    lens_q, lens_k = [70, 1, 200], [90, 130, 200]
    dev = "cuda"
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32), device=dev)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32), device=dev)
    q = torch.empty((sum(lens_q), H, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty((sum(lens_k), H, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    o = torch.empty_like(q)
    l = torch.empty((H, sum(lens_q)), dtype=torch.float32, device=dev)

    def refill(seed):
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        for t in (q, k, v):
            t.copy_(torch.randn(t.shape, device=dev, generator=g).to(torch.bfloat16))

    def call():
        api.attn_fwd_varlen(q, k, v, cu_q, cu_k, max_seqlen_q=max(lens_q),
                            max_seqlen_k=max(lens_k), causal=True, out=o, lse=l)
    _capture_and_replay("attn_fwd_varlen H=4 D=64 causal, 3 sequences", refill, call, [o, l])


@pytest.mark.parametrize("rows,cols", [(300, 1000), (4, 70000)])
def test_softmax_rows_replays(rows, cols):
    dev = "cuda"
    x = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    y = torch.empty_like(x)

    def refill(seed):
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        x.copy_(torch.randn(x.shape, device=dev, generator=g) * 4)

    def call():
        api.softmax_rows(x, out=y)
    _capture_and_replay(f"softmax_rows {rows}x{cols}", refill, call, [y])
