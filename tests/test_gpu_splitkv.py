"""GPU parity of the split-key forward (attn_fwd_splitkv: key ranges in separate
workgroups, merged by their LSE) against the fp64 CPU oracle, through the C ABI.
Tolerances are those of the bf16 fused forward (``tests/parity.py``)."""

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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    api.load_library()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(B, H, Nq, Nk, D, causal, lens, splits, seed):
    q, k, v, lens = random_case(seed, B, H, Nq, Nk, D, "bf16", lens)
    scale = 1.0 / math.sqrt(D)
    _say(f"[splitkv] B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} lens="
         f"{None if lens is None else list(lens)} splits={splits}")
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)
                  for x in (q, k, v))
    ld = None if lens is None else torch.tensor(np.asarray(lens, np.int32), device="cuda")
    o, lse = api.attn_fwd_splitkv(qd, kd, vd, scale=scale, causal=causal, kv_lens=ld,
                                  num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_oracle(q, k, v, scale, causal=causal, kv_lens=lens)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16",
          f"splitkv {B}x{H}x{Nq}x{Nk}x{D} splits={splits}")
    return qd, kd, vd, ld, scale, o, lse


@pytest.mark.parametrize("splits", [0, 1, 2, 7])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 65), (3, 1000), (16, 4097), (33, 640),
                                   (130, 300)])
@pytest.mark.parametrize("D", [64, 128])
def test_splitkv_shapes(Nq, Nk, D, splits):
    _run(2, 3, Nq, Nk, D, False, None, splits, seed=Nq * 13 + Nk + D + splits)


@pytest.mark.parametrize("splits", [0, 3, 16])
@pytest.mark.parametrize("causal,lens", [(False, [0, 1, 700, 2000]), (False, [-5, 64, 65, 3000]),
                                         (True, None), (True, [10, 0, 2999, 100])])
def test_splitkv_masks(causal, lens, splits):
    """Ragged kv_len (empty ranges and whole sequences without keys), causal."""
    _run(4, 2, 5 if not causal else 200, 3000, 128, causal, lens, splits,
         seed=splits + (7 if causal else 3))


def test_splitkv_matches_fused_forward():
    qd, kd, vd, ld, scale, o, lse = _run(2, 4, 8, 5000, 128, False, [4999, 1234], 9, seed=77)
    o2, lse2 = api.attn_fwd(qd, kd, vd, scale=scale, kv_lens=ld)
    torch.cuda.synchronize()
    assert (o.float() - o2.float()).abs().max().item() <= 2e-2
    assert (lse - lse2).abs().max().item() <= 1e-3 * max(1.0, lse2.abs().max().item())


@pytest.mark.parametrize("B,H,Nk,ragged", [(16, 32, 8192, True), (1, 8, 65536, False)])
def test_splitkv_decode_sizes(B, H, Nk, ragged):
    """The decode shapes the measurements use (one query per head), sampled heads
    against the oracle."""
    rng = np.random.default_rng(B * H + Nk)
    D = 128
    lens = rng.integers(1, Nk + 1, size=B).astype(np.int32) if ragged else None
    qd = torch.randn(B, H, 1, D, device="cuda").to(torch.bfloat16)
    kd = torch.randn(B, H, Nk, D, device="cuda").to(torch.bfloat16)
    vd = torch.randn(B, H, Nk, D, device="cuda").to(torch.bfloat16)
    ld = None if lens is None else torch.from_numpy(lens).cuda()
    _say(f"[splitkv] decode B={B} H={H} Nk={Nk} ragged={ragged}")
    o, lse = api.attn_fwd_splitkv(qd, kd, vd, kv_lens=ld)
    torch.cuda.synchronize()
    for b in sorted({0, B - 1}):
        for h in sorted({0, H - 1}):
            q = qd[b:b + 1, h:h + 1].float().cpu().numpy()
            k = kd[b:b + 1, h:h + 1].float().cpu().numpy()
            v = vd[b:b + 1, h:h + 1].float().cpu().numpy()
            o_ref, lse_ref = oracle.attention_oracle(
                q, k, v, 1 / math.sqrt(D), kv_lens=None if lens is None else lens[b:b + 1])
            check(o[b:b + 1, h:h + 1].float().cpu().numpy(), lse[b:b + 1, h:h + 1].cpu().numpy(),
                  o_ref, lse_ref, "bf16", f"decode b={b} h={h}")
