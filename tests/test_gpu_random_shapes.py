"""Seeded sweep of random problem shapes for every forward entry point, against the
fp64 oracle (bf16 tolerances of tests/parity.py; the FP8 bound for attn_fwd_fp8).

Hand-picked edge cases cover the boundaries the kernels are built around (tile and
block edges, empty and over-long key ranges); this sweep adds shapes nobody picked:
B, H, Nq, Nk, D, causal, per-sequence key lengths, split counts and packed lengths
drawn from a fixed seed, each case small enough for the oracle to check every
element."""

import math
import sys

import numpy as np
import pytest

import oracle
from exact_attention_89_amd import api
from exact_attention_89_amd.workloads import random_case, random_fp8_case, round_to_bf16
from tests.parity import check, check_fp8, fp8_o_bound

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    api.load_library()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _shape(rng):
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 5))
    Nq = int(rng.choice([1, 2, 7, 31, 64, 100, 129, 255, 256, 300, 511, 700]))
    Nk = int(rng.choice([1, 5, 63, 64, 65, 128, 200, 333, 512, 777, 1100]))
    if rng.random() < 0.4:
        Nk = Nq
    D = int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.5)
    lens = None
    if rng.random() < 0.4:
        lens = [int(x) for x in rng.integers(-2, Nk + 3, size=B)]
    return B, H, Nq, Nk, D, causal, lens


def _dev_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)


def _lens(lens):
    return None if lens is None else torch.tensor(np.asarray(lens, np.int32), device="cuda")


@pytest.mark.parametrize("kernel", [api.ATTN_KERNEL_AUTO, api.ATTN_KERNEL_PINGPONG,
                                    api.ATTN_KERNEL_FOURWAVE])
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_bf16(i, kernel):
    B, H, Nq, Nk, D, causal, lens = _shape(np.random.default_rng(1000 + i))
    q, k, v, lens = random_case(2000 + i, B, H, Nq, Nk, D, "bf16", lens)
    scale = 1.0 / math.sqrt(D)
    _say(f"[random] bf16 kernel={kernel} B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} "
         f"lens={lens}")
    prev = api.attn_fwd_select_kernel(kernel)
    try:
        o, lse = api.attn_fwd(_dev_bf16(q), _dev_bf16(k), _dev_bf16(v), scale=scale,
                              causal=causal, kv_lens=_lens(lens))
        torch.cuda.synchronize()
    finally:
        api.attn_fwd_select_kernel(prev)
    o_ref, lse_ref = oracle.attention_oracle(q, k, v, scale, causal=causal, kv_lens=lens)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16", f"random {i}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_splitkv(i):
    rng = np.random.default_rng(3000 + i)
    B, H, _, Nk, D, causal, lens = _shape(rng)
    Nq = int(rng.choice([1, 2, 5, 16, 33, 130]))
    splits = int(rng.choice([0, 1, 2, 3, 8, 17]))
    q, k, v, lens = random_case(4000 + i, B, H, Nq, Nk, D, "bf16", lens)
    scale = 1.0 / math.sqrt(D)
    _say(f"[random] splitkv B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} lens={lens} "
         f"splits={splits}")
    o, lse = api.attn_fwd_splitkv(_dev_bf16(q), _dev_bf16(k), _dev_bf16(v), scale=scale,
                                  causal=causal, kv_lens=_lens(lens), num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_oracle(q, k, v, scale, causal=causal, kv_lens=lens)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16",
          f"random splitkv {i}")


@pytest.mark.parametrize("kernel", [api.ATTN_KERNEL_AUTO, api.ATTN_KERNEL_PINGPONG])
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_fp8(i, kernel):
    B, H, Nq, Nk, D, causal, lens = _shape(np.random.default_rng(5000 + i))
    q8, k8, v8, ds = random_fp8_case(6000 + i, B, H, Nq, Nk, D)
    scale = 1.0 / math.sqrt(D)
    _say(f"[random] fp8 kernel={kernel} B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} "
         f"lens={lens}")
    dev = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q8, k8, v8)]
    prev = api.attn_fwd_select_kernel(kernel)
    try:
        o, lse = api.attn_fwd_fp8(*dev, *ds, scale=scale, causal=causal, kv_lens=_lens(lens))
        torch.cuda.synchronize()
    finally:
        api.attn_fwd_select_kernel(prev)
    o_ref, lse_ref, P = oracle.attention_fp8_oracle(q8, k8, v8, scale, *ds, causal=causal,
                                                    kv_lens=lens, return_probs=True)
    bound = fp8_o_bound(P, oracle.dequantize(v8, ds[2]), o_ref)
    check_fp8(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, bound,
              f"random fp8 {i}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_varlen(i):
    rng = np.random.default_rng(7000 + i)
    nseq = int(rng.integers(1, 9))
    H = int(rng.integers(1, 5))
    D = int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.5)
    lq = [int(x) for x in rng.integers(0, 400, size=nseq)]
    lk = [int(x) for x in rng.integers(0, 400, size=nseq)] if rng.random() < 0.5 else list(lq)
    lq[0] = max(lq[0], 1)
    tq, tk = max(1, sum(lq)), max(1, sum(lk))
    q = round_to_bf16(rng.standard_normal((tq, H, D), dtype=np.float32))
    k = round_to_bf16(rng.standard_normal((tk, H, D), dtype=np.float32))
    v = round_to_bf16(rng.standard_normal((tk, H, D), dtype=np.float32))
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    scale = 1.0 / math.sqrt(D)
    mq, mk = max(1, max(lq)), max(1, max(lk))
    _say(f"[random] varlen H={H} D={D} causal={causal} lq={lq} lk={lk}")
    o, lse = api.attn_fwd_varlen(_dev_bf16(q), _dev_bf16(k), _dev_bf16(v),
                                 torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(),
                                 mq, mk, scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_varlen_oracle(q, k, v, cu_q, cu_k, scale, causal, mq, mk)
    cov = ~np.isnan(lse_ref[0])
    if cov.any():
        check(o.float().cpu().numpy()[cov], lse.cpu().numpy()[:, cov].T, o_ref[cov],
              lse_ref[:, cov].T, "bf16", f"random varlen {i}")
