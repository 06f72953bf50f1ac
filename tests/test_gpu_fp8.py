"""GPU parity of the FP8 fused forward (attn_fwd_fp8) against the fp64 CPU oracle of
the dequantised inputs, through the C ABI.

The kernel rounds the probabilities to E4M3 before the P.V product, so O is held to
the element-wise bound ``tests.parity.fp8_o_bound`` derived from that rounding (not
to the bf16 path's 2e-2); LSE, the -inf rules and the NaN rule are those of the bf16
path.  Inputs: N(0, std^2) draws quantised per tensor to E4M3 (``random_fp8_case``).
"""

import math
import sys

import numpy as np
import pytest

import oracle
from exact_attention_89_amd import api
from exact_attention_89_amd.workloads import WORKLOADS, generate_fp8, random_fp8_case
from tests.parity import check_fp8, fp8_o_bound, fp8_score_abs

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


@pytest.fixture(params=["pingpong", "fourwave"])
def fp8_kernel(request):
    """Run an FP8 test on each of the two FP8 forward kernels (forced, not auto-picked)."""
    which = {"pingpong": api.ATTN_KERNEL_PINGPONG,
             "fourwave": api.ATTN_KERNEL_FOURWAVE}[request.param]
    prev = api.attn_fwd_select_kernel(which)
    _say(f"[fp8] kernel: {request.param}")
    yield request.param
    api.attn_fwd_select_kernel(prev)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _gpu_fp8(q8, k8, v8, ds, scale, causal, lens):
    ld = None if lens is None else torch.tensor(np.asarray(lens, np.int32), device="cuda")
    o, lse = api.attn_fwd_fp8(_dev(q8), _dev(k8), _dev(v8), *ds, scale=scale, causal=causal,
                              kv_lens=ld)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _run(B, H, Nq, Nk, D, causal=False, lens=None, seed=0, std=1.0, scale=None, ds=None):
    q8, k8, v8, ds0 = random_fp8_case(seed, B, H, Nq, Nk, D, std=std)
    ds = ds0 if ds is None else ds
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    what = (f"fp8 B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} lens={lens} std={std} "
            f"scale={scale:.4g} seed={seed}")
    _say(f"[fp8] {what}")
    o, lse = _gpu_fp8(q8, k8, v8, ds, scale, causal, lens)
    o_ref, lse_ref, P = oracle.attention_fp8_oracle(q8, k8, v8, scale, *ds, causal=causal,
                                                    kv_lens=lens, return_probs=True)
    sa = fp8_score_abs(oracle.dequantize(q8, ds[0]), oracle.dequantize(k8, ds[1]), scale)
    bound = fp8_o_bound(P, oracle.dequantize(v8, ds[2]), o_ref, sa)
    res = check_fp8(o, lse, o_ref, lse_ref, bound, what)
    _say(f"[fp8]   max|dO| {res[0]:.3e}  max|dO|/bound {res[1]:.3f}  rms {res[2]:.3e}  "
         f"LSE {res[3]:.2e}")
    return res


@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 200), (77, 77), (128, 128), (200, 333),
                                   (300, 300), (513, 130)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_shapes(Nq, Nk, D, causal, fp8_kernel):
    _run(2, 3, Nq, Nk, D, causal, seed=Nq * 7 + Nk + D + int(causal))


@pytest.mark.parametrize("causal,lens", [(False, [0, 1, 65, 700]), (False, [-3, 64, 129, 2000]),
                                         (True, [700, 0, 5, 64]), (True, None)])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_kv_lens(causal, lens, D, fp8_kernel):
    _run(4, 2, 700, 700, D, causal, lens=lens, seed=11 + D)


@pytest.mark.parametrize("B,H,N,D,causal,lens", [
    (1, 16, 1024, 128, True, None),           # B*H = 16, causal: heads two at a time per XCD
    (2, 16, 600, 64, True, [600, 377]),       # B*H = 32, ragged query blocks and key lengths
    (1, 24, 520, 128, True, None),            # B*H = 24: a multiple of 8 but not of 16
])
def test_fp8_schedules(B, H, N, D, causal, lens, fp8_kernel):
    """Each (batch, head, query block) is computed once whichever order the workgroups
    take them in: O and LSE start as NaN and every element is checked against the
    oracle's bound."""
    q8, k8, v8, ds = random_fp8_case(B * 1000 + H + N, B, H, N, N, D)
    scale = 1.0 / math.sqrt(D)
    _say(f"[fp8] schedules B={B} H={H} N={N} D={D} causal={causal} lens={lens}")
    ld = None if lens is None else torch.tensor(np.asarray(lens, np.int32), device="cuda")
    o = torch.full((B, H, N, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    api.attn_fwd_fp8(_dev(q8), _dev(k8), _dev(v8), *ds, scale=scale, causal=causal,
                     kv_lens=ld, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref, P = oracle.attention_fp8_oracle(q8, k8, v8, scale, *ds, causal=causal,
                                                    kv_lens=lens, return_probs=True)
    sa = fp8_score_abs(oracle.dequantize(q8, ds[0]), oracle.dequantize(k8, ds[1]), scale)
    bound = fp8_o_bound(P, oracle.dequantize(v8, ds[2]), o_ref, sa)
    check_fp8(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, bound,
              f"fp8 schedules {B}x{H}x{N}x{D}")


@pytest.mark.parametrize("std", [0.25, 2.0, 4.0])
def test_fp8_peaked_and_flat_rows(std, fp8_kernel):
    """Larger std gives peaked rows (one key dominates), smaller nearly uniform rows."""
    _run(1, 4, 256, 1024, 128, True, seed=5, std=std)


@pytest.mark.parametrize("scale", [0.0, -0.2, 1.5])
def test_fp8_scale_values(scale, fp8_kernel):
    """scale <= 0 takes the pre-scaled instantiation; 0 gives the mean of valid values."""
    _run(2, 2, 130, 260, 128, False, lens=[260, 100], seed=3, scale=scale)


def test_fp8_descales_not_amax(fp8_kernel):
    """Descales need not come from amax: any positive factors are honoured."""
    _run(1, 2, 200, 200, 128, True, seed=8, ds=(0.03125, 0.0078125, 3.0))


def test_fp8_zero_query(fp8_kernel):
    """q = 0: every valid key weighs the same, O = mean of the values, LSE = ln(#keys)."""
    q8, k8, v8, ds = random_fp8_case(4, 1, 2, 100, 300, 64)
    q8[:] = 0
    o, lse = _gpu_fp8(q8, k8, v8, ds, 0.125, False, None)
    mean = oracle.dequantize(v8, ds[2]).mean(axis=2, keepdims=True)
    assert np.allclose(lse, math.log(300), rtol=0, atol=1e-5)
    # uniform weights 2^6 are exact in E4M3: only fp32 sums and the bf16 output round
    assert np.max(np.abs(o - mean)) <= 2.0 ** -8 * np.max(np.abs(mean)) + 1e-5


def test_fp8_single_key_is_exact(fp8_kernel):
    """Nk = 1: the one weight is 2^6 (exact), O = the dequantised value row in bf16."""
    q8, k8, v8, ds = random_fp8_case(9, 2, 2, 40, 1, 128)
    o, _ = _gpu_fp8(q8, k8, v8, ds, 0.1, False, None)
    ref = np.broadcast_to(oracle.dequantize(v8, ds[2]), o.shape)
    bf16 = torch.from_numpy(np.ascontiguousarray(ref, dtype=np.float32)).to(torch.bfloat16)
    assert np.array_equal(o, bf16.float().numpy())


@pytest.mark.parametrize("B,H,N,D,causal,lens", [
    (1, 4, 300, 128, True, None), (2, 3, 513, 128, False, [513, 77]), (1, 2, 1000, 64, True, None),
    (2, 2, 256, 64, False, [0, 200]),
    (2, 4, 700, 128, False, [700, 100]), (1, 16, 520, 64, False, None),
    (2, 4, 600, 128, True, [600, 333])])
def test_fp8_both_kernels_bitwise_equal(B, H, N, D, causal, lens):
    """The two FP8 kernels run the same per-wave arithmetic in the same order.  The
    four-wave one also runs the key tiles every row of its workgroup sees whole without
    mask code, and for non-causal calls with B*H a multiple of 8 takes the heads of
    each XCD one at a time; equal bits show neither changes a result."""
    q8, k8, v8, ds = random_fp8_case(N + D, B, H, N, N, D)
    out = []
    for which in (api.ATTN_KERNEL_PINGPONG, api.ATTN_KERNEL_FOURWAVE):
        prev = api.attn_fwd_select_kernel(which)
        try:
            _say(f"[fp8] kernel {which} {B}x{H}x{N}x{D} causal={causal} lens={lens}")
            out.append(_gpu_fp8(q8, k8, v8, ds, D ** -0.5, causal, lens))
        finally:
            api.attn_fwd_select_kernel(prev)
    assert np.array_equal(out[0][0], out[1][0]) and np.array_equal(out[0][1], out[1][1])


def test_fp8_deterministic():
    q8, k8, v8, ds = random_fp8_case(21, 1, 4, 300, 300, 128)
    a = _gpu_fp8(q8, k8, v8, ds, 0.09, True, None)
    b = _gpu_fp8(q8, k8, v8, ds, 0.09, True, None)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fp8_float8_dtype_accepted():
    """torch.float8_e4m3fn tensors go through the same entry point as uint8 codes."""
    q8, k8, v8, ds = random_fp8_case(2, 1, 1, 64, 64, 64)
    a = _gpu_fp8(q8, k8, v8, ds, 0.125, False, None)
    f8 = [_dev(x).view(torch.float8_e4m3fn) for x in (q8, k8, v8)]
    o, lse = api.attn_fwd_fp8(*f8, *ds, scale=0.125)
    torch.cuda.synchronize()
    assert np.array_equal(a[0], o.float().cpu().numpy())


def test_fp8_rejects_bad_descale():
    q8, k8, v8, ds = random_fp8_case(2, 1, 1, 64, 64, 64)
    for bad in ((0.0, 1.0, 1.0), (1.0, -1.0, 1.0), (1.0, 1.0, float("nan")),
                (1.0, float("inf"), 1.0)):
        with pytest.raises(api.AttnError, match="ATTN_ERR_SCALE"):
            api.attn_fwd_fp8(_dev(q8), _dev(k8), _dev(v8), *bad, scale=0.125)


@pytest.mark.slow
def test_fp8_headline_shape_sampled_rows():
    """B=1 H=32 N=8192 D=128 causal, the draw of the bf16 throughput workload quantised
    per tensor to E4M3 (the configuration the FP8 throughput line times): sampled rows
    against the oracle, each with its own bound."""
    w = WORKLOADS["bf16_causal_b1h32_n8192_d128"]
    q8, k8, v8, (qd, kd, vd), _ = generate_fp8(w)
    _say("[fp8] headline shape: B=1 H=32 N=8192 D=128 causal")
    o, lse = _gpu_fp8(q8, k8, v8, (qd, kd, vd), w.scale, True, None)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    r = np.random.default_rng(99)
    rows = [0, 1, 63, 64, 127, 128, 255, 4095, 8191] + list(r.integers(0, w.Nq, 7))
    heads = [0, 13, 31]
    Q, K, V = (oracle.dequantize(c, d) for c, d in ((q8, qd), (k8, kd), (v8, vd)))
    sigma = oracle.effective_scale(w.scale)
    worst = 0.0
    for h in heads:
        for i in rows:
            valid = oracle.valid_keys(i, i + 1, w.Nk, True, w.Nk)
            o_ref, lse_ref, P = oracle.attention_rows(Q[0, h, i:i + 1], K[0, h], V[0, h], sigma,
                                                      valid, return_probs=True)
            bound = fp8_o_bound(P, V[0, h], o_ref,
                                fp8_score_abs(Q[0, h, i:i + 1], K[0, h], w.scale))
            res = check_fp8(o[0, h, i:i + 1], lse[0, h, i:i + 1], o_ref, lse_ref, bound,
                            f"fp8 headline h={h} i={i}")
            worst = max(worst, res[1])
    _say(f"[fp8] headline sampled rows: worst |dO|/bound {worst:.3f}")
