"""GPU parity: the HIP kernels, called through the C ABI, against the fp64 CPU oracle.

Small cases compare every output element; the five full-size workloads compare
sampled rows (computed one by one by the oracle) and check properties of every
row (no NaN, -inf exactly on rows without valid keys).  Tolerances are those of
``tests/parity.py``.
"""

import dataclasses
import math
import sys

import numpy as np
import pytest

import oracle
from exact_attention_89_amd import api
from exact_attention_89_amd.workloads import WORKLOADS, generate, random_case
from tests.parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    api.load_library()


@pytest.fixture(params=["pingpong", "fourwave", "keygroups"])
def bf16_kernel(request):
    """Run a bf16 test on each of the three forward kernels (forced, not auto-picked)."""
    which = {"pingpong": api.ATTN_KERNEL_PINGPONG,
             "fourwave": api.ATTN_KERNEL_FOURWAVE,
             "keygroups": api.ATTN_KERNEL_KEYGROUPS}[request.param]
    prev = api.attn_fwd_select_kernel(which)
    _say(f"[parity] bf16 kernel: {request.param}")
    yield request.param
    api.attn_fwd_select_kernel(prev)


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t.float()


def _lens_dev(lens):
    return None if lens is None else torch.tensor(np.asarray(lens, np.int32), device="cuda")


def _run(impl, q, k, v, scale, causal, lens, dtype):
    qd, kd, vd = _dev(q, dtype), _dev(k, dtype), _dev(v, dtype)
    ld = _lens_dev(lens)
    if impl == "fused":
        fn = api.attn_fwd if dtype == "bf16" else api.attn_fwd_f32
        o, lse = fn(qd, kd, vd, scale=scale, causal=causal, kv_lens=ld)
    elif impl == "partial":
        o, lse = api.attn_partial(qd, kd, vd, scale=scale, causal=causal, kv_lens=ld)
    else:
        o, lse = api.attn_materialized(qd, kd, vd, scale=scale, causal=causal, kv_lens=ld)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _case(impl, B, H, Nq, Nk, D, causal, lens=None, dtype="bf16", seed=0, scale=None, std=1.0):
    q, k, v, lens = random_case(seed, B, H, Nq, Nk, D, dtype, lens, std)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _say(f"[parity] {impl} {dtype} B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} "
         f"lens={None if lens is None else list(lens)} scale={scale} std={std} seed={seed}")
    o, lse = _run(impl, q, k, v, scale, causal, lens, dtype)
    o_ref, lse_ref = oracle.attention_oracle(q, k, v, scale, causal=causal, kv_lens=lens)
    return check(o, lse, o_ref, lse_ref, dtype, what=f"{impl} {B}x{H}x{Nq}x{Nk}x{D}")


# ---------------------------------------------------------------------------
# small shapes: every element against the oracle
# ---------------------------------------------------------------------------

EDGE_N = [1, 3, 63, 64, 65, 127, 128, 129, 200, 257]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", EDGE_N)
def test_fused_bf16_square(N, causal, D, bf16_kernel):
    _case("fused", 1, 2, N, N, D, causal, seed=N + D)


@pytest.mark.parametrize("Nq,Nk", [(64, 200), (200, 64), (129, 1000), (1, 300), (300, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_fused_bf16_rectangular(Nq, Nk, causal, bf16_kernel):
    _case("fused", 2, 1, Nq, Nk, 128, causal, seed=Nq * 7 + Nk)


@pytest.mark.parametrize("lens", [[0, 1], [63, 64], [65, 300], [300, 1000], [-3, 999]])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_fused_bf16_kv_lens(lens, causal, D, bf16_kernel):
    """kv_len in {0, 1, BC-1, BC, BC+1, Nk, > Nk, < 0}; with causal, tiles that are
    fully masked for some rows of a wave (later tiles) and for whole waves."""
    _case("fused", 2, 2, 300, 300, D, causal, lens=lens, seed=sum(map(abs, lens)) + D)


def test_fused_bf16_beyond_4096_keys(bf16_kernel):
    """More than 4096 keys per row (page 'Attention softmax fusion', 'Things that
    break': a per-row buffer with a fixed 4096-column capacity), odd length."""
    _case("fused", 1, 2, 130, 4097, 128, False, seed=4097)
    _case("fused", 1, 1, 4099, 4099, 64, True, seed=4099)


def test_fused_bf16_large_scores(bf16_kernel):
    """Score magnitudes of several tens: exponent range and the max subtraction."""
    _case("fused", 1, 2, 256, 256, 128, False, seed=7, std=2.5)
    _case("fused", 1, 2, 256, 256, 64, True, seed=8, std=2.5)


@pytest.mark.parametrize("scale", [0.0, -0.2, 1e-3, 1.0])
def test_fused_bf16_scale_values(scale, bf16_kernel):
    """scale <= 0 takes the pre-scaled path; tiny and unit scales the normal one."""
    _case("fused", 1, 2, 150, 150, 64, True, seed=11, scale=scale)
    _case("fused", 1, 1, 150, 190, 128, False, lens=[170], seed=12, scale=scale)


def test_fused_bf16_rising_max(bf16_kernel):
    """Keys that drift along one direction (the long-context recipe, stronger drift so
    a short sequence shows it): the running max rises on most tiles and the output
    must still match."""
    rng = np.random.default_rng(21)
    D, N = 128, 2048
    g = rng.standard_normal(D).astype(np.float32)
    u = g / np.linalg.norm(g)
    from exact_attention_89_amd.workloads import round_to_bf16
    q = round_to_bf16(rng.standard_normal((1, 2, N, D), dtype=np.float32))
    k = rng.standard_normal((1, 2, N, D), dtype=np.float32)
    k = round_to_bf16(k + np.float32(0.02) * np.arange(N, dtype=np.float32)[:, None] * u)
    v = round_to_bf16(rng.standard_normal((1, 2, N, D), dtype=np.float32))
    scale = 1 / math.sqrt(D)
    _say("[parity] fused bf16 rising-max N=2048 D=128 causal")
    o, lse = _run("fused", q, k, v, scale, True, None, "bf16")
    o_ref, lse_ref = oracle.attention_oracle(q, k, v, scale, causal=True)
    check(o, lse, o_ref, lse_ref, "bf16", "rising max")


@pytest.mark.parametrize("B,H,N,D,causal,lens", [
    (1, 16, 1024, 64, True, None),            # B*H = 16, causal: heads two at a time per XCD
    (2, 16, 600, 128, True, [600, 377]),      # B*H = 32, ragged query blocks and key lengths
    (1, 24, 520, 128, True, None),            # B*H = 24: a multiple of 8 but not of 16
    (3, 8, 700, 64, False, [700, 1, 450]),    # non-causal: heads one at a time per XCD
])
def test_fused_bf16_schedules(B, H, N, D, causal, lens, bf16_kernel):
    """Each (batch, head, query block) is computed once whichever order the workgroups
    take them in: O and LSE start as NaN and every element is compared with the oracle."""
    q, k, v, lens = random_case(B * 1000 + H + N, B, H, N, N, D, "bf16", lens)
    scale = 1.0 / math.sqrt(D)
    _say(f"[parity] schedules B={B} H={H} N={N} D={D} causal={causal} lens={lens}")
    o = torch.full((B, H, N, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    api.attn_fwd(_dev(q, "bf16"), _dev(k, "bf16"), _dev(v, "bf16"), scale=scale, causal=causal,
                 kv_lens=_lens_dev(lens), out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_oracle(q, k, v, scale, causal=causal, kv_lens=lens)
    check(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16",
          what=f"schedules {B}x{H}x{N}x{D}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_fused_bf16_reference_moves(D, causal, bf16_kernel):
    """Scores placed exactly (one-hot Q, key weights on the same axis, all integers, so
    s * scale * log2(e) is about the weight in log2 units) to drive each branch of the
    lazy exponent reference: keys 64.. at +6 over the first tile (every exponential
    about 2^6: lane sums far above 2^7 but no reference moves), one key at +13 at
    position 777 (a move caused by one key), keys 1000..1063 at +21 (a move of whole
    rows late in the sequence) and a negative plateau after them."""
    rng = np.random.default_rng(31 + D)
    Nq = Nk = 1100                                # causal rows reach every key
    from exact_attention_89_amd.workloads import round_to_bf16
    c = math.log2(math.e) / math.sqrt(D)
    alpha = 8.0                                   # exact in bf16
    w = np.zeros(Nk, np.float32)
    w[64:] = 6.0
    w[777] = 13.0
    w[1000:1064] = 21.0
    w[1064:] = -4.0
    beta = np.round(w / (alpha * c)).astype(np.float32)   # integers, exact in bf16
    q = np.zeros((1, 2, Nq, D), np.float32)
    q[..., 0] = alpha
    k = round_to_bf16(np.float32(0.05) * rng.standard_normal((1, 2, Nk, D), dtype=np.float32))
    k[..., 0] = beta
    v = round_to_bf16(rng.standard_normal((1, 2, Nk, D), dtype=np.float32))
    scale = 1 / math.sqrt(D)
    _say(f"[parity] fused bf16 reference moves D={D} causal={causal}")
    o, lse = _run("fused", q, k, v, scale, causal, None, "bf16")
    o_ref, lse_ref = oracle.attention_oracle(q, k, v, scale, causal=causal)
    check(o, lse, o_ref, lse_ref, "bf16", "reference moves")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,lens", [(False, None), (True, None), (False, [0, 77]),
                                         (True, [130, 2])])
@pytest.mark.parametrize("N", [1, 33, 64, 129, 200])
def test_fused_f32(N, causal, lens, D):
    _case("fused", 2, 2, N, N, D, causal, lens=lens, dtype="fp32", seed=N + D)


@pytest.mark.parametrize("causal,lens", [(False, None), (True, None), (False, [0, 100]),
                                         (True, [97, 300])])
@pytest.mark.parametrize("D", [64, 128])
def test_materialized_bf16(causal, lens, D):
    _case("materialized", 2, 2, 200, 200, D, causal, lens=lens, seed=5 + D)
    _case("materialized", 2, 1, 65, 300, D, causal, lens=lens, seed=6 + D)


# ---------------------------------------------------------------------------
# metamorphic and robustness checks on the GPU output itself
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 63, 64, 65, 129, 200, 300])
@pytest.mark.parametrize("causal,lens", [(False, None), (True, None), (False, [0, 77]),
                                         (True, [150, 1]), (False, [-3, 999])])
@pytest.mark.parametrize("D", [64, 128])
def test_partial_bf16(N, causal, lens, D):
    """Partial fusion (QK^T + softmax fused, P through memory, then P V)."""
    _case("partial", 2, 2, N, N, D, causal, lens=lens, seed=N * 3 + D)


@pytest.mark.parametrize("scale", [0.0, -0.2, 1.0])
def test_partial_bf16_scale_and_rectangular(scale):
    _case("partial", 1, 2, 150, 333, 128, False, seed=31, scale=scale)
    _case("partial", 1, 1, 333, 150, 64, True, lens=[120], seed=32, scale=scale)


def test_partial_workspace_holds_p():
    """After attn_partial the workspace holds P: rows sum to 1 over valid keys, zeros
    elsewhere (causal, so the upper triangle is zero)."""
    B, H, N, D = 1, 2, 200, 128
    q, k, v, _ = random_case(41, B, H, N, N, D)
    qd, kd, vd = (_dev(x, "bf16") for x in (q, k, v))
    ld = (N + 63) // 64 * 64
    ws = torch.empty(api.attn_partial_workspace_bytes(B, H, N, N), dtype=torch.uint8,
                     device="cuda")
    _say("[gpu] partial workspace P 1x2x200x128 causal")
    api.attn_partial(qd, kd, vd, causal=True, workspace=ws)
    torch.cuda.synchronize()
    P = ws[:B * H * N * ld * 2].view(torch.bfloat16).view(B, H, N, ld).float().cpu().numpy()
    assert np.all(np.triu(P[0, 0, :, :N], 1) == 0) and np.all(P[..., N:] == 0)
    assert np.max(np.abs(P.sum(-1) - 1.0)) <= 2e-2


def test_deterministic(bf16_kernel):
    q, k, v, _ = random_case(3, 2, 4, 700, 700, 128)
    qd, kd, vd = (_dev(x, "bf16") for x in (q, k, v))
    _say("[gpu] determinism 2x4x700x128 causal")
    o1, l1 = api.attn_fwd(qd, kd, vd, causal=True)
    o2, l2 = api.attn_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_keys_beyond_kv_len_are_never_read(bf16_kernel):
    """Keys and values at or after kv_len (even NaN) change nothing, bit for bit."""
    q, k, v, _ = random_case(4, 2, 2, 300, 300, 128)
    lens = np.array([130, 257], np.int32)
    qd, kd, vd = (_dev(x, "bf16") for x in (q, k, v))
    ld = _lens_dev(lens)
    _say("[gpu] kv_len prefix 2x2x300 lens=[130,257]")
    o1, l1 = api.attn_fwd(qd, kd, vd, kv_lens=ld)
    k2, v2 = kd.clone(), vd.clone()
    for b, L in enumerate(lens):
        k2[b, :, L:] = float("nan")
        v2[b, :, L:] = float("nan")
    o2, l2 = api.attn_fwd(qd, k2, v2, kv_lens=ld)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("path", ["partial", "materialized", "splitkv", "fp8"])
def test_keys_beyond_kv_len_are_never_read_other_paths(path):
    """The same for every other entry point that takes kv_lens: NaN keys and values at
    or after kv_len leave the output bit for bit unchanged (and NaN-free)."""
    q, k, v, _ = random_case(5, 2, 2, 200, 300, 64)
    lens = np.array([0, 193], np.int32)
    ld = _lens_dev(lens)
    _say(f"[gpu] kv_len prefix, {path} path, 2x2x200x300 lens=[0,193]")
    if path == "fp8":
        qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.float8_e4m3fn)
                      .view(torch.uint8) for x in (q, k, v))
        nan = 0x7F                                     # an E4M3 NaN code
    else:
        qd, kd, vd = (_dev(x, "bf16") for x in (q, k, v))
        nan = float("nan")

    def run(kk, vv):
        if path == "partial":
            return api.attn_partial(qd, kk, vv, kv_lens=ld)
        if path == "materialized":
            return api.attn_materialized(qd, kk, vv, kv_lens=ld)
        if path == "splitkv":
            return api.attn_fwd_splitkv(qd, kk, vv, kv_lens=ld, num_splits=3)
        return api.attn_fwd_fp8(qd, kk, vv, 0.02, 0.02, 0.02, kv_lens=ld)

    o1, l1 = run(kd, vd)
    k2, v2 = kd.clone(), vd.clone()
    for b, L in enumerate(lens):
        k2[b, :, L:] = nan
        v2[b, :, L:] = nan
    o2, l2 = run(k2, v2)
    torch.cuda.synchronize()
    assert not torch.isnan(o2.float()).any() and not torch.isnan(l2).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("B,H,N,D,causal,lens", [
    (1, 2, 300, 128, True, None), (2, 2, 333, 64, False, [0, 200]),
    (2, 3, 513, 128, False, [512, 7]), (1, 1, 1000, 64, True, None)])
def test_both_kernels_bitwise_equal(B, H, N, D, causal, lens):
    """The two bf16 kernels run the same per-wave arithmetic in the same order, so
    their outputs are identical bit for bit."""
    q, k, v, lens = random_case(N + D, B, H, N, N, D, "bf16", lens)
    qd, kd, vd = (_dev(x, "bf16") for x in (q, k, v))
    ld = _lens_dev(lens)
    out = {}
    for which in (api.ATTN_KERNEL_PINGPONG, api.ATTN_KERNEL_FOURWAVE):
        prev = api.attn_fwd_select_kernel(which)
        try:
            _say(f"[gpu] kernel {which} {B}x{H}x{N}x{D} causal={causal} lens={lens}")
            out[which] = api.attn_fwd(qd, kd, vd, causal=causal, kv_lens=ld)
            torch.cuda.synchronize()
        finally:
            api.attn_fwd_select_kernel(prev)
    (o1, l1), (o2, l2) = out.values()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("B,H,Nq,Nk,D,causal,lens,scale", [
    (1, 2, 1300, 1300, 128, True, None, None),      # six 256-row blocks, growing interiors
    (2, 2, 777, 1500, 128, True, [1500, 900], None),  # Nq < Nk, causal and key lengths
    (2, 1, 1500, 700, 128, True, [650, 3], None),     # Nq > Nk: rows past every key
    (1, 2, 600, 1000, 128, False, [777], None),       # key-length tail inside a tile
    (1, 1, 513, 513, 128, True, None, -0.05),         # scale <= 0: every tile checked
    (1, 1, 520, 520, 64, True, [300], None),
    (2, 4, 700, 700, 128, False, [700, 333], None),   # B*H = 8: head-by-head order
    (1, 16, 600, 900, 128, False, None, None),         # B*H = 16, two heads per XCD
    (4, 4, 300, 300, 64, False, [0, 1, 299, 300], None)])
def test_both_kernels_bitwise_equal_interior_split(B, H, Nq, Nk, D, causal, lens, scale):
    """The ping-pong kernel runs the key tiles every row of a workgroup sees whole
    without mask code and the rest with it; the four-wave kernel checks every tile.
    Equal bits on shapes that move that boundary show the split masks nothing it
    should keep and keeps nothing it should mask.  The non-causal cases with B*H a
    multiple of 8 take the ping-pong kernel's head-by-head workgroup order: a block
    it skipped or ran twice would show here too."""
    q, k, v, lens = random_case(Nq + 7 * Nk + D, B, H, Nq, Nk, D, "bf16", lens)
    qd, kd, vd = (_dev(x, "bf16") for x in (q, k, v))
    ld = _lens_dev(lens)
    out = {}
    for which in (api.ATTN_KERNEL_PINGPONG, api.ATTN_KERNEL_FOURWAVE):
        prev = api.attn_fwd_select_kernel(which)
        try:
            _say(f"[gpu] kernel {which} {B}x{H}x{Nq}x{Nk}x{D} causal={causal} lens={lens} "
                 f"scale={scale}")
            out[which] = api.attn_fwd(qd, kd, vd, scale=scale, causal=causal, kv_lens=ld)
            torch.cuda.synchronize()
        finally:
            api.attn_fwd_select_kernel(prev)
    (o1, l1), (o2, l2) = out.values()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    sc = D ** -0.5 if scale is None else scale
    o_ref, lse_ref = oracle.attention_oracle(q, k, v, sc, causal=causal, kv_lens=lens)
    check(o1.float().cpu().numpy(), l1.cpu().numpy(), o_ref, lse_ref, "bf16",
          f"interior split {B}x{H}x{Nq}x{Nk}x{D}")


def test_key_permutation_invariance():
    """Without a causal mask, permuting (k_j, v_j) jointly changes O only by rounding."""
    q, k, v, _ = random_case(5, 1, 2, 256, 512, 128)
    perm = np.random.default_rng(0).permutation(512)
    _say("[gpu] key permutation 1x2x256x512")
    o1, l1 = _run("fused", q, k, v, 0.09, False, None, "bf16")
    o2, l2 = _run("fused", q, k[:, :, perm], v[:, :, perm], 0.09, False, None, "bf16")
    assert np.max(np.abs(o1 - o2)) <= 2e-2
    assert np.max(np.abs(l1 - l2)) <= 1e-3 * max(1.0, np.abs(l1).max())


def test_no_write_outside_outputs(bf16_kernel):
    """Guard regions around o and lse keep their canary bytes (no out-of-bounds store)."""
    B, H, N, D = 1, 3, 190, 128
    q, k, v, _ = random_case(6, B, H, N, N, D)
    qd, kd, vd = (_dev(x, "bf16") for x in (q, k, v))
    G = 4096
    obuf = torch.full((G + B * H * N * D + G,), 12345, dtype=torch.int16, device="cuda")
    lbuf = torch.full((G + B * H * N + G,), -7.0, dtype=torch.float32, device="cuda")
    o = obuf[G:G + B * H * N * D].view(torch.bfloat16).view(B, H, N, D)
    lse = lbuf[G:G + B * H * N].view(B, H, N)
    _say("[gpu] canary 1x3x190x128 causal")
    api.attn_fwd(qd, kd, vd, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:G] == 12345) and torch.all(obuf[G + B * H * N * D:] == 12345)
    assert torch.all(lbuf[:G] == -7.0) and torch.all(lbuf[G + B * H * N:] == -7.0)


def test_errors_leave_outputs_untouched():
    """An invalid call returns its status and writes nothing."""
    q, k, v, _ = random_case(7, 1, 1, 64, 64, 64)
    qd, kd, vd = (_dev(x, "bf16") for x in (q, k, v))
    o = torch.full_like(qd, 3.0)
    lse = torch.full((1, 1, 64), 5.0, device="cuda")
    lib = api.load_library()
    s = torch.cuda.current_stream().cuda_stream
    st = lib.attn_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      1, 1, 64, 64, 96, 0.1, 0, None, s)
    assert st == -3
    st = lib.attn_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      1, 1, 64, 64, 64, float("inf"), 0, None, s)
    assert st == -5
    st = lib.attn_fwd(qd.data_ptr() + 2, kd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                      lse.data_ptr(), 1, 1, 63, 64, 64, 0.1, 0, None, s)
    assert st == -4
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    st = lib.attn_materialized(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), 1, 1, 64, 64, 64, 0.1, 0, None, ws.data_ptr(), 16,
                               s)
    assert st == -6
    torch.cuda.synchronize()
    assert torch.all(o.float() == 3.0) and torch.all(lse == 5.0)


# ---------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the bench times
# ---------------------------------------------------------------------------

def _samples(w, lens, rng, n_random=96):
    rows = {0, 1, 63, 64, 127, 128, 129, w.Nq // 2, w.Nq - 2, w.Nq - 1}
    if w.Nq > 4096:
        rows |= {4095, 4096, 4097}
    out = []
    for b in range(w.B):
        for h in sorted({0, w.H - 1, w.H // 2}):
            for i in sorted(r for r in rows if 0 <= r < w.Nq):
                out.append((b, h, i))
    for _ in range(n_random):
        out.append((int(rng.integers(w.B)), int(rng.integers(w.H)), int(rng.integers(w.Nq))))
    return out


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size(name):
    w = WORKLOADS[name]
    _say(f"[parity] workload {name}: generating inputs")
    q, k, v, lens = generate(w)
    _say(f"[parity] workload {name}: attn_fwd on GPU")
    o, lse = _run("fused", q, k, v, w.scale, w.causal, lens, w.dtype)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    if w.B * w.H * w.Nq * w.Nk <= 4 * 8 * 1024 * 1024:
        o_ref, lse_ref = oracle.attention_oracle(q, k, v, w.scale, causal=w.causal, kv_lens=lens)
        err = check(o, lse, o_ref, lse_ref, w.dtype, name)
    else:
        rng = np.random.default_rng(w.seed)
        smp = _samples(w, lens, rng)
        o_ref, lse_ref = oracle.attention_oracle_rows(q, k, v, w.scale, w.causal, lens, smp)
        idx = tuple(np.array(smp).T)
        err = check(o[idx], lse[idx], o_ref, lse_ref, w.dtype, name)
    if lens is not None:
        for b in np.nonzero(np.asarray(lens) <= 0)[0]:
            assert np.all(o[b] == 0.0) and np.all(np.isneginf(lse[b]))
        for b in np.nonzero(np.asarray(lens) > 0)[0]:
            assert np.all(np.isfinite(lse[b]))
    else:
        assert np.all(np.isfinite(lse))
    _say(f"[parity] workload {name}: max|dO| = {err[0]:.3e}, LSE rel err = {err[1]:.3e}")
