"""Parity at key counts where the kernels' 32-bit byte offsets grow large: about 2
million keys per head (512 MiB of K, 512 MiB of V in bf16), checked on every query row
against the fp64 oracle.  One entry point per test; each prints its case first."""

import math
import sys

import numpy as np
import pytest

import oracle
from exact_attention_89_amd import api
from exact_attention_89_amd.workloads import quantize_e4m3, round_to_bf16
from tests.parity import check, check_fp8, fp8_o_bound, fp8_score_abs

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]

NK = (1 << 21) + 77


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    api.load_library()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def big():
    rng = np.random.default_rng(77)
    q = round_to_bf16(rng.standard_normal((1, 1, 3, 128), dtype=np.float32))
    k = round_to_bf16(rng.standard_normal((1, 1, NK, 128), dtype=np.float32))
    v = round_to_bf16(rng.standard_normal((1, 1, NK, 128), dtype=np.float32))
    return q, k, v


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)


@pytest.mark.parametrize("lens", [None, [NK - 5]])
def test_fused_two_million_keys(big, lens):
    q, k, v = big
    _say(f"[large] attn_fwd Nq=3 Nk={NK} lens={lens}")
    ld = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = api.attn_fwd(_dev(q), _dev(k), _dev(v), scale=0.09, kv_lens=ld)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_oracle(q, k, v, 0.09, kv_lens=lens)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16", "large fused")


def test_splitkv_two_million_keys(big):
    q, k, v = big
    _say(f"[large] attn_fwd_splitkv Nq=3 Nk={NK}")
    o, lse = api.attn_fwd_splitkv(_dev(q), _dev(k), _dev(v), scale=0.09)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_oracle(q, k, v, 0.09)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16", "large splitkv")


def test_fp8_two_million_keys(big):
    q, k, v = big
    _say(f"[large] attn_fwd_fp8 Nq=3 Nk={NK}")
    (q8, qd), (k8, kd), (v8, vd) = (quantize_e4m3(x) for x in (q, k, v))
    dev = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q8, k8, v8)]
    o, lse = api.attn_fwd_fp8(*dev, qd, kd, vd, scale=0.09)
    torch.cuda.synchronize()
    o_ref, lse_ref, P = oracle.attention_fp8_oracle(q8, k8, v8, 0.09, qd, kd, vd,
                                                    return_probs=True)
    sa = fp8_score_abs(oracle.dequantize(q8, qd), oracle.dequantize(k8, kd), 0.09)
    bound = fp8_o_bound(P, oracle.dequantize(v8, vd), o_ref, sa)
    check_fp8(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, bound, "large fp8")


def test_varlen_sequence_far_into_the_pack():
    """Two sequences; the second starts about 1.1 million tokens into a pack of H = 2,
    so its rows begin about 563 MiB past the tensor start."""
    rng = np.random.default_rng(78)
    H, D = 2, 128
    lq, lk = [5, 7], [1_100_000, 300_003]
    tq, tk = sum(lq), sum(lk)
    q = round_to_bf16(rng.standard_normal((tq, H, D), dtype=np.float32))
    k = round_to_bf16(rng.standard_normal((tk, H, D), dtype=np.float32))
    v = round_to_bf16(rng.standard_normal((tk, H, D), dtype=np.float32))
    cu_q = np.array([0, lq[0], tq], dtype=np.int32)
    cu_k = np.array([0, lk[0], tk], dtype=np.int32)
    _say(f"[large] attn_fwd_varlen lq={lq} lk={lk} H={H}")
    o, lse = api.attn_fwd_varlen(_dev(q), _dev(k), _dev(v), torch.from_numpy(cu_q).cuda(),
                                 torch.from_numpy(cu_k).cuda(), scale=0.09, causal=False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_varlen_oracle(q, k, v, cu_q, cu_k, 0.09)
    check(o.float().cpu().numpy(), lse.cpu().numpy().T, o_ref, lse_ref.T, "bf16",
          "large varlen")
