"""Calls captured in a HIP graph (torch.cuda.CUDAGraph over the library's launches on the
capturing stream) and replayed: every replay, with new inputs copied in between by
ordinary eager work, must give bit for bit what the eager call gives on the same inputs.
The no-allocation split-key entry point exists for such callers; attn_fwd and the
allocating split-key entry point (with a workspace made before capture) are covered too.
Nothing is allocated inside a capture: outputs, workspaces and inputs are made first."""

import math
import sys

import numpy as np
import pytest

import oracle
from exact_attention_89_amd import api
from exact_attention_89_amd.workloads import random_case
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
