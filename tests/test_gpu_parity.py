"""GPU parity: the HIP library against the oracle, element by element.

Gates (bf16 in, fp32 sums, bf16 out):
* integer-valued inputs: bit-exact bf16 and exact fp32 debug output;
* N(0,1)-type inputs: within 1 bf16 ulp of the oracle's rounded result, or
  within 1e-4 * sqrt(K) * sigma_A * sigma_B of the exact sum near zero;
* fp32 debug output: within 1e-4 * sqrt(K) * sigma_A * sigma_B.

Shapes are those of the workloads in ``synthetic_inputs``: 512^3, 4096^3,
the M = 8192 prefill and M = 256 decode linear layers, the 512 x 8192 x 5376
projection and ragged M in {1, 17, 64, 200}; plus edge cases.  Every call
goes through the C ABI (``gemm_bf16_ex``) with the automatic configuration
unless a test names one.
"""
import numpy as np
import pytest

from oracle.compare import check_bf16, check_f32
from synthetic_inputs import WORKLOADS, f32_to_bf16_bits, int_bf16, normal_bf16
from tests.gpu_util import run_gemm

pytestmark = pytest.mark.gpu


def _oracle():
    import oracle

    return oracle


def _full_check(w, A, B, exact):
    """bf16 output against the oracle's rounded sums, the fp32 debug output
    against its exact sums, and the debug output rounded to bf16 against the
    bf16 output: the two calls share plan and summation order, so they must
    agree bit for bit (this also holds on plans that split K, where the fp32
    result comes out of the reduction kernel's fp32 branch)."""
    o = _oracle()
    ref16, ref64 = o.gemm(A, B, K=w.K)
    got = run_gemm(A, B, K=w.K)
    import dense_gemm_bf16_amd as g

    plan = g.config_name(w.M, w.N, w.K)
    rep = check_bf16(got, ref16, ref64, w.K, w.sigma_a, w.sigma_b, exact=exact)
    print(w.name, plan, "bf16", rep, flush=True)
    assert rep["ok"], rep
    got32 = run_gemm(A, B, K=w.K, out_f32=True)
    rep32 = check_f32(got32, ref64, w.K, w.sigma_a, w.sigma_b, exact=exact)
    print(w.name, plan, "f32", rep32, flush=True)
    assert rep32["ok"], rep32
    rounded = f32_to_bf16_bits(got32)
    assert np.array_equal(rounded, got), (w.name, int(np.count_nonzero(rounded != got)))


@pytest.mark.parametrize("name", ["square512_int", "square512_normal"])
def test_square512(name):
    w = WORKLOADS[name]
    A, B = w.make()
    _full_check(w, A, B, exact=(w.dist == "int"))


@pytest.mark.parametrize("name", ["square4096_int", "square4096_normal"])
def test_square4096_full(name):
    w = WORKLOADS[name]
    A, B = w.make()
    _full_check(w, A, B, exact=(w.dist == "int"))


@pytest.mark.parametrize("name", ["decode_attn_out", "decode_qkv", "decode_mlp_up",
                                  "decode_mlp_down"])
def test_decode_full(name):
    """Every element, bf16 and fp32 output; attention-out, QKV and MLP-down
    split K, so their fp32 output comes from the reduction kernel."""
    w = WORKLOADS[name]
    A, B = w.make()
    _full_check(w, A, B, exact=False)


@pytest.mark.parametrize("name", ["proj_512x8192x5376", "ragged_m1", "ragged_m17",
                                  "ragged_m64", "ragged_m200"])
def test_irregular_full(name):
    """Every element, bf16 and fp32 output: M = 1 and 17 run the small-M
    kernel (its own fp32 store), M = 64 and 200 split K."""
    w = WORKLOADS[name]
    A, B = w.make()
    _full_check(w, A, B, exact=False)


@pytest.mark.parametrize("name", ["prefill_attn_out", "prefill_mlp_up"])
def test_prefill_sampled(name):
    """Full rows and full columns of the product (the oracle cannot afford
    all of it in test time): the first and last 32 rows/columns (edge tiles)
    plus 32 spread through the middle."""
    w = WORKLOADS[name]
    A, B = w.make()
    got = run_gemm(A, B)
    o = _oracle()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([np.arange(32), np.arange(w.M - 32, w.M),
                                     rng.choice(w.M, 32, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(32), np.arange(w.N - 32, w.N),
                                     rng.choice(w.N, 32, replace=False)]))
    r16, r64 = o.gemm(np.ascontiguousarray(A[rows]), B, K=w.K)
    rep = check_bf16(got[rows], r16, r64, w.K, w.sigma_a, w.sigma_b)
    print(name, "rows", rep, flush=True)
    assert rep["ok"], rep
    c16, c64 = o.gemm(A, np.ascontiguousarray(B[cols]), K=w.K)
    rep = check_bf16(got[:, cols], c16, c64, w.K, w.sigma_a, w.sigma_b)
    print(name, "cols", rep, flush=True)
    assert rep["ok"], rep


# ------------------------------------------------------------- edge cases

def test_every_config_bit_exact_on_ragged_shape():
    """Each built tile configuration, with and without split-K and K-step
    rotation, on a shape that is ragged in M, N and K: integer inputs, so
    bit-exact."""
    import dense_gemm_bf16_amd as g

    M, N, K = 300, 520, 456
    A = int_bf16(M, K, seed=101)
    B = int_bf16(N, K, seed=102)
    ref16, ref64 = _oracle().gemm(A, B)
    for cfg in g.config_names():
        # plain, split K, and split K with the K-step order rotated per tile
        for suffix in ("_k1", "_k3", "_k2_g4_r1"):
            name = cfg + suffix
            got = run_gemm(A, B, config=name)
            rep = check_bf16(got, ref16, None, K, exact=True)
            print(name, rep, flush=True)
            assert rep["ok"], (name, rep)
        # fp32 debug output: the kernel's own fp32 store and the reduction's
        for suffix in ("_k1", "_k3"):
            name = cfg + suffix
            got32 = run_gemm(A, B, config=name, out_f32=True)
            rep = check_f32(got32, ref64, K, exact=True)
            print(name, "f32", rep, flush=True)
            assert rep["ok"], (name, rep)


def test_every_config_bit_exact_with_k_not_multiple_of_8():
    """Each built configuration, plain and split with rotation, where a
    16-byte chunk straddles K (K = 203) and the rows are padded with NaN:
    the chunk's tail must be trimmed and nothing past K read."""
    import dense_gemm_bf16_amd as g

    M, N, K = 200, 136, 203
    ld = 216
    A = np.full((M, ld), 0x7FC0, np.uint16)
    B = np.full((N, ld), 0x7FC0, np.uint16)
    A[:, :K] = int_bf16(M, K, seed=103)
    B[:, :K] = int_bf16(N, K, seed=104)
    ref16, ref64 = _oracle().gemm(A, B, K=K)
    for cfg in g.config_names():
        for suffix in ("_k1", "_k2_g4_r1"):
            name = cfg + suffix
            got = run_gemm(A, B, K=K, config=name)
            rep = check_bf16(got, ref16, None, K, exact=True)
            print(name, rep, flush=True)
            assert rep["ok"], (name, rep)
            got32 = run_gemm(A, B, K=K, config=name, out_f32=True)
            rep = check_f32(got32, ref64, K, exact=True)
            print(name, "f32", rep, flush=True)
            assert rep["ok"], (name, rep)


@pytest.mark.parametrize("K", [1, 7, 8, 17, 63, 65, 200])
def test_ragged_k(K):
    """K not a multiple of 8 (a 16-byte chunk straddles K) and not of 64;
    the padding of A and B holds NaN, which must never be read."""
    M, N = 70, 90
    lda = ldb = ((K + 7) // 8) * 8 + 8
    A = np.full((M, lda), 0x7FC0, np.uint16)
    B = np.full((N, ldb), 0x7FC0, np.uint16)
    A[:, :K] = int_bf16(M, K, seed=200 + K)
    B[:, :K] = int_bf16(N, K, seed=300 + K)
    ref16, ref64 = _oracle().gemm(A, B, K=K)
    got = run_gemm(A, B, K=K)
    rep = check_bf16(got, ref16, None, K, exact=True)
    assert rep["ok"], rep
    got32 = run_gemm(A, B, K=K, out_f32=True)
    assert check_f32(got32, ref64, K, exact=True)["ok"]


@pytest.mark.parametrize("N", [8, 24, 8200, 1000])
def test_ragged_n_and_small_m(N):
    A = normal_bf16(17, 264, seed=400)
    B = normal_bf16(N, 264, seed=401)
    ref16, ref64 = _oracle().gemm(A, B)
    got = run_gemm(A, B)
    rep = check_bf16(got, ref16, ref64, 264)
    assert rep["ok"], rep


def test_no_writes_outside_c():
    """C sits inside a canary-filled buffer with ldc > N and a spare row on
    each side; only the M x N window may change."""
    M, N, K = 130, 200, 96
    A = int_bf16(M, K, seed=500)
    B = int_bf16(N, K, seed=501)
    ref16, _ = _oracle().gemm(A, B)
    canary = 0x5A5A
    buf = run_gemm(A, B, ldc=216, canary=canary)
    assert buf.shape == (M + 2, 216)
    assert np.all(buf[0] == canary) and np.all(buf[-1] == canary)
    assert np.all(buf[1:-1, N:] == canary)
    assert np.array_equal(buf[1:-1, :N], ref16)


BIG = "t256x256x64_w2x2_s2_x3_p10"
# A 256-row tile's operand rows, plus the 4 KB a load's resource base may be
# moved back by, must stay below 2^31 bytes (a 32-bit buffer offset with the
# top bit marking an absent chunk): the largest row stride the 256-row tile
# takes is the largest multiple of 8 elements below that.
LD_MAX_256 = ((((1 << 31) - 4096) - 1) // (256 * 2)) // 8 * 8


@pytest.mark.parametrize("plan", [BIG + "_k1_g4", BIG + "_k2_g4"])
def test_largest_accepted_strides(plan):
    """lda and ldb at the largest value the 256 x 256 tile accepts (2 GiB
    per operand, NaN everywhere but the first K columns) and ldc = 2^23, so
    C's byte offsets pass 2^32; the result is exact and nothing beyond the
    first N columns of C changes.  One element more of lda or ldb is refused
    before anything is enqueued."""
    import torch

    import dense_gemm_bf16_amd as g

    M, N, K = 256, 256, 200
    lda = ldb = LD_MAX_256
    assert 256 * (lda + 8) * 2 >= (1 << 31) - 4096 > 256 * lda * 2
    ldc = 1 << 23
    A = int_bf16(M, K, seed=560)
    B = int_bf16(N, K, seed=561)
    ref16, _ = _oracle().gemm(A, B)
    nan = np.array([0x7FC0], np.uint16).view(np.int16)[0]
    dA = torch.full((M, lda), int(nan), dtype=torch.int16, device="cuda")
    dB = torch.full((N, ldb), int(nan), dtype=torch.int16, device="cuda")
    dA[:, :K].copy_(torch.from_numpy(A.view(np.int16)))
    dB[:, :K].copy_(torch.from_numpy(B.view(np.int16)))
    canary = 0x5A5A
    dC = torch.full((M, ldc), canary, dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    print(plan, "lda", lda, "ldc", ldc, flush=True)
    g.gemm_bf16_ex(plan, M, N, K, dA, lda, dB, ldb, dC, ldc)
    torch.cuda.synchronize()
    got = dC[:, :N].cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref16), int(np.count_nonzero(got != ref16))
    assert np.all(dC[:, N:N + 512].cpu().numpy() == canary)
    assert np.all(dC[:, ldc - 64:].cpu().numpy() == canary)
    for la, lb in [(lda + 8, ldb), (lda, ldb + 8)]:
        rc = g.gemm_bf16_status(M, N, K, dA, la, dB, lb, dC, ldc, config=plan)
        assert rc == g.GEMM_ERR_UNSUPPORTED, (la, lb, rc)
    del dA, dB, dC
    torch.cuda.empty_cache()


def test_k_zero_gives_zeros():
    import torch

    import dense_gemm_bf16_amd as g

    C = torch.full((5, 16), 1234, dtype=torch.int16, device="cuda")
    g.gemm_bf16(5, 16, 0, None, 8, None, 8, C, 16)
    torch.cuda.synchronize()
    assert not C.cpu().numpy().any()


def test_empty_m_or_n_is_noop():
    import dense_gemm_bf16_amd as g

    g.gemm_bf16(0, 16, 8, None, 8, None, 8, None, 16)
    g.gemm_bf16(4, 0, 8, None, 8, None, 8, None, 8)


def test_split_k_matches_unsplit_on_integers():
    """Decode shape with integer inputs: split and unsplit both bit-exact,
    bf16 output and fp32 output (which equals the exact sum: every partial
    and every fixed-order slice sum is an integer below 2^24), for slice
    counts 1-8 and 16."""
    M, N, K = 256, 1024, 8192
    A = int_bf16(M, K, seed=600)
    B = int_bf16(N, K, seed=601)
    import dense_gemm_bf16_amd as g

    ref16, ref64 = _oracle().gemm(A, B)
    tile = g.config_name(M, N, K).split("_k")[0]
    for cfg in [f"{tile}_k{k}" for k in (1, 2, 3, 4, 5, 6, 7, 8, 16)]:
        got = run_gemm(A, B, config=cfg)
        assert check_bf16(got, ref16, None, K, exact=True)["ok"], cfg
        got32 = run_gemm(A, B, config=cfg, out_f32=True)
        rep = check_f32(got32, ref64, K, exact=True)
        assert rep["ok"], (cfg, rep)


def test_deterministic_repeat():
    """Two calls give identical bits (fixed summation order, split-K too)."""
    w = WORKLOADS["decode_attn_out"]
    A, B = w.make()
    a = run_gemm(A, B)
    b = run_gemm(A, B)
    assert np.array_equal(a, b)


def test_identity_and_k1_closed_forms():
    """A = I gives B^T exactly; K = 1 gives RNE(a*b) exactly, any bf16."""
    K = 64
    eye = np.zeros((K, K), np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    B = normal_bf16(40, K, seed=700)
    assert np.array_equal(run_gemm(eye, B), B.T)
    a = normal_bf16(50, 1, seed=701)
    b = normal_bf16(30, 1, seed=702)
    ref16, _ = _oracle().gemm(a, b)
    assert np.array_equal(run_gemm(a, b, K=1), ref16)


def test_random_shapes_automatic_plan_bit_exact():
    """Forty seeded random shapes (M, N log-uniform in [1, 3000], K in
    [1, 4000], almost all ragged), integer inputs, through the automatic
    plan: every shape rule, split count and edge path the choice reaches
    must be bit-exact."""
    import dense_gemm_bf16_amd as g

    rng = np.random.default_rng(4242)
    o = _oracle()
    plans = set()
    for i in range(40):
        M = int(np.exp(rng.uniform(0, np.log(3000))))
        N = int(np.exp(rng.uniform(0, np.log(3000))))
        K = int(np.exp(rng.uniform(0, np.log(4000))))
        A = int_bf16(M, K, seed=900 + 2 * i)
        B = int_bf16(N, K, seed=901 + 2 * i)
        ref16, _ = o.gemm(A, B)
        got = run_gemm(A, B)
        rep = check_bf16(got, ref16, None, K, exact=True)
        plan = g.config_name(M, N, K)
        plans.add(plan.split("_k")[0])
        print(i, (M, N, K), plan, rep, flush=True)
        assert rep["ok"], ((M, N, K), plan, rep)
    print("tiles used:", sorted(plans), flush=True)


def test_random_named_plans_bit_exact():
    """Thirty seeded random (plan, shape) pairs: a product tile, K split 1-4,
    K-step rotation on or off, non-temporal B on the tiles built with it,
    GROUP_M 4 or 8, M, N and K random and mostly ragged, A and B row strides
    padded by a random multiple of 8 elements (NaN in the padding), fp32
    output for one call in three; integer inputs, so every result is exact.
    Hybrid plans are named where the shape gives them a tail (three row tiles
    over a long N)."""
    import dense_gemm_bf16_amd as g

    rng = np.random.default_rng(5151)
    o = _oracle()
    tiles = sorted(PRODUCT_CONFIGS)
    stream = set(STREAM_TILES)
    for i in range(30):
        tile = tiles[int(rng.integers(len(tiles)))]
        bm, bn = int(tile[1:].split("x")[0]), int(tile.split("x")[1])
        hybrid = bm >= 128 and i % 5 == 0
        if hybrid:  # 3 rows of tiles x 90 columns: more than one pass of 256
            M = 2 * bm + int(rng.integers(1, bm))
            N = 89 * bn + int(rng.integers(1, bn))
            K = int(rng.integers(130, 400))
        else:
            M = int(rng.integers(1, 3 * bm + 1))
            N = int(rng.integers(1, 2000))
            K = int(rng.integers(1, 700))
        S = 1 if hybrid else int(rng.integers(1, 5))
        name = f"{tile}_k{S}_g{int(rng.choice([4, 8]))}"
        if rng.random() < 0.5:
            name += "_r1"
        if tile in stream and rng.random() < 0.5:
            name += "_n1"
        if hybrid:
            name += f"_h{int(rng.integers(2, 5))}"
        pad_a, pad_b = 8 * int(rng.integers(0, 3)), 8 * int(rng.integers(0, 3))
        kk = (K + 7) // 8 * 8
        A = np.full((M, kk + pad_a), 0x7FC0, np.uint16)
        B = np.full((N, kk + pad_b), 0x7FC0, np.uint16)
        A[:, :K] = int_bf16(M, K, seed=1600 + 2 * i)
        B[:, :K] = int_bf16(N, K, seed=1601 + 2 * i)
        ref16, ref64 = o.gemm(A, B, K=K)
        f32 = i % 3 == 0
        got = run_gemm(A, B, K=K, config=name, out_f32=f32)
        if f32:
            rep = check_f32(got, ref64, K, exact=True)
        else:
            rep = check_bf16(got, ref16, None, K, exact=True)
        print(i, name, (M, N, K), "f32" if f32 else "bf16", rep, flush=True)
        assert rep["ok"], (name, (M, N, K), rep)


PRODUCT_CONFIGS = {
    "t256x256x64_w2x2_s2_x3_p10", "t256x128x64_w2x2_s3_x3_p10", "t128x128x64_w2x2_s4_x3_p10",
    "t32x32x64_w1x1_s8_x2_p9", "t64x32x64_w1x1_s6_x2_p9", "t64x128x64_w1x4_s6_x2_p0",
    "t32x128x64_w1x4_s6_x2_p0",
}


def test_ablation_configurations_when_built():
    """The configurations of csrc/ablation (the kernel families and LDS
    layouts the product choices were measured against) exist only in
    build(ablation=True); there they must be as exact as the product ones,
    plain and split, bf16 and fp32 output."""
    import dense_gemm_bf16_amd as g

    names = set(g.config_names())
    assert PRODUCT_CONFIGS <= names, sorted(PRODUCT_CONFIGS - names)
    extra = sorted(names - PRODUCT_CONFIGS)
    if not extra:
        pytest.skip("ablation build absent: the default build holds only the product "
                    "configurations; build(ablation=True) adds csrc/ablation's")
    M, N, K = 300, 520, 456
    A = int_bf16(M, K, seed=105)
    B = int_bf16(N, K, seed=106)
    ref16, ref64 = _oracle().gemm(A, B)
    for cfg in extra:
        for suffix in ("_k1", "_k3"):
            got = run_gemm(A, B, config=cfg + suffix)
            assert check_bf16(got, ref16, None, K, exact=True)["ok"], cfg + suffix
            got32 = run_gemm(A, B, config=cfg + suffix, out_f32=True)
            assert check_f32(got32, ref64, K, exact=True)["ok"], cfg + suffix


# ------------------------------------------------------ persistent grid

BIG = "t256x256x64_w2x2_s2_x3_p10"


@pytest.mark.parametrize("shape,plan", [
    ((1024, 1024, 512), "_k1_g4_P8"),        # 16 tiles on 8 workgroups: 2 each
    ((600, 1100, 456), "_k1_g4_P8"),         # ragged M, N, K: edge tiles in the walk
    ((1100, 2100, 520), "_k1_g8_r1_P16"),    # rotation, GROUP_M 8, 45 tiles on 16
])
def test_persistent_plan_bit_exact(shape, plan):
    """A persistent grid (each workgroup walks several tiles; C of one tile
    drains through one LDS slot while the next tile's first K-steps land in
    the others) on integer inputs: bf16 bit-exact, and the fp32 debug output
    (the ordinary kernel, same per-tile order) exact."""
    M, N, K = shape
    A = int_bf16(M, K, seed=1300 + M)
    B = int_bf16(N, K, seed=1301 + N)
    ref16, ref64 = _oracle().gemm(A, B)
    name = BIG + plan
    got = run_gemm(A, B, config=name)
    rep = check_bf16(got, ref16, None, K, exact=True)
    print(shape, name, rep, flush=True)
    assert rep["ok"], rep
    got32 = run_gemm(A, B, config=name, out_f32=True)
    assert check_f32(got32, ref64, K, exact=True)["ok"]


def test_persistent_plan_k_not_multiple_of_8():
    """K = 203 with NaN in the padding: the tail chunk is trimmed in the slot
    its step lands in, which the persistent grid shifts by one."""
    M, N, K = 520, 600, 203
    ld = 216
    A = np.full((M, ld), 0x7FC0, np.uint16)
    B = np.full((N, ld), 0x7FC0, np.uint16)
    A[:, :K] = int_bf16(M, K, seed=1310)
    B[:, :K] = int_bf16(N, K, seed=1311)
    ref16, _ = _oracle().gemm(A, B, K=K)
    got = run_gemm(A, B, K=K, config=BIG + "_k1_g4_P8")
    assert check_bf16(got, ref16, None, K, exact=True)["ok"]


def test_persistent_plan_matches_one_tile_per_workgroup_on_prefill():
    """M = 8192 prefill attention-out (1024 tiles, 4 per workgroup on a grid
    of 256): the same bits as the ordinary plan on N(0,1) data, since each
    tile sums its K-steps in the same order; sampled rows against the
    oracle."""
    w = WORKLOADS["prefill_attn_out"]
    A, B = w.make()
    got = run_gemm(A, B, config=BIG + "_k1_g4_P256")
    ref = run_gemm(A, B, config=BIG + "_k1_g4")
    assert np.array_equal(got, ref), int(np.count_nonzero(got != ref))
    rows = np.array([0, 1, 255, 256, 4095, 4096, 8191])
    r16, r64 = _oracle().gemm(np.ascontiguousarray(A[rows]), B, K=w.K)
    rep = check_bf16(got[rows], r16, r64, w.K, w.sigma_a, w.sigma_b)
    assert rep["ok"], rep


def test_persistent_plan_k_zero():
    import torch

    import dense_gemm_bf16_amd as g

    C = torch.full((300, 600), 1234, dtype=torch.int16, device="cuda")
    dummy = torch.zeros(8, dtype=torch.int16, device="cuda")
    g.gemm_bf16_ex(BIG + "_k1_g4_P8", 300, 600, 0, dummy, 8, dummy, 8, C, 600)
    torch.cuda.synchronize()
    assert not C.cpu().numpy().any()


# ------------------------------------------------------ non-temporal B loads

# The configurations built with non-temporal B loads ("_n1"), by tile height.
STREAM_TILES = {
    "t256x128x64_w2x2_s3_x3_p10": 256,
    "t32x32x64_w1x1_s8_x2_p9": 32,
    "t64x32x64_w1x1_s6_x2_p9": 64,
    "t64x128x64_w1x4_s6_x2_p0": 64,
    "t32x128x64_w1x4_s6_x2_p0": 32,
}


@pytest.mark.parametrize("tile", sorted(STREAM_TILES))
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_stream_b_plans_bit_exact(tile, fmt):
    """_n1 changes only the cache policy of B's loads: on integer inputs with
    one row of tiles (ragged M and N), plain and split K, the result is
    bit-exact and the same bits as the plan without _n1; with fp32 output and
    with K % 64 != 0 (no such kernel: the ordinary one runs) it is exact
    too."""
    bm = STREAM_TILES[tile]
    M, N = bm - 3, 1000
    o = _oracle()
    for K, plans in ((1024, ("_k1_g4_n1", "_k3_g4_r1_n1")), (1000, ("_k2_g4_n1",))):
        A = int_bf16(M, K, seed=1400 + bm + K, fmt=fmt)
        B = int_bf16(N, K, seed=1401 + bm + K, fmt=fmt)
        ref16, ref64 = o.gemm(A, B, fmt=fmt)
        for plan in plans:
            name = tile + plan
            got = run_gemm(A, B, config=name, fmt=fmt)
            rep = check_bf16(got, ref16, None, K, exact=True, fmt=fmt)
            print(fmt, K, name, rep, flush=True)
            assert rep["ok"], (name, rep)
            plain = run_gemm(A, B, config=name[: -len("_n1")], fmt=fmt)
            assert np.array_equal(got, plain), name
            got32 = run_gemm(A, B, config=name, out_f32=True, fmt=fmt)
            assert check_f32(got32, ref64, K, exact=True)["ok"], name


def test_stream_b_with_several_tile_rows_is_still_exact():
    """_n1 where rows of tiles share B (M = 600 on the 256-row tile): slower,
    never wrong."""
    M, N, K = 600, 700, 512
    A = int_bf16(M, K, seed=1450)
    B = int_bf16(N, K, seed=1451)
    ref16, _ = _oracle().gemm(A, B)
    got = run_gemm(A, B, config="t256x128x64_w2x2_s3_x3_p10_k2_g4_n1")
    assert check_bf16(got, ref16, None, K, exact=True)["ok"]


# ------------------------------------------------------------ hybrid plans
# "_h<S>": the tile columns that fill whole passes over the 256 CUs run
# unsplit, the columns after them as a second call with K split S ways.
# Each shape below has a little more than one pass of tiles of its
# configuration (3 rows of tiles x 90 columns, the last column ragged), so
# the hybrid splits at column 85 of 90.
HYBRID_CASES = [  # (tile, M, N)
    ("t256x256x64_w2x2_s2_x3_p10", 520, 22920),
    ("t256x128x64_w2x2_s3_x3_p10", 520, 11460),
    ("t128x128x64_w2x2_s4_x3_p10", 300, 11460),
]


@pytest.mark.parametrize("tile,M,N", HYBRID_CASES)
def test_hybrid_plans_bit_exact(tile, M, N):
    """Integer inputs with K = 456 (a partial last K-step): the hybrid plan
    with the tail split 2 and 3 ways is bit-exact in bf16 and fp32 output,
    and so is the no-allocation entry point with it."""
    import torch

    import dense_gemm_bf16_amd as g

    K = 456
    A = int_bf16(M, K, seed=1500 + M)
    B = int_bf16(N, K, seed=1501 + N)
    ref16, ref64 = _oracle().gemm(A, B)
    for plan in (tile + "_k1_g4_h2", tile + "_k1_g4_h3"):
        got = run_gemm(A, B, config=plan)
        rep = check_bf16(got, ref16, None, K, exact=True)
        print(plan, M, N, rep, flush=True)
        assert rep["ok"], (plan, rep)
        got32 = run_gemm(A, B, config=plan, out_f32=True)
        assert check_f32(got32, ref64, K, exact=True)["ok"], plan
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dB = torch.from_numpy(B.view(np.int16)).cuda()
    ldc = (N + 7) // 8 * 8
    dC = torch.zeros((M, ldc), dtype=torch.int16, device="cuda")
    g.gemm_bf16_ex_noalloc(tile + "_k1_g4_h3", M, N, K, dA, K, dB, K, dC, ldc)
    torch.cuda.synchronize()
    assert np.array_equal(dC[:, :N].cpu().numpy().view(np.uint16), ref16)


@pytest.mark.parametrize("tile,M,N", HYBRID_CASES[:1])
def test_hybrid_head_matches_plain_plan_on_normal_inputs(tile, M, N):
    """N(0,1) inputs: the unsplit head columns are the plain plan's bits (same
    tiles, same summation order), and the whole result meets the ulp
    criterion against the oracle."""
    K = 1000
    A = normal_bf16(M, K, seed=1510)
    B = normal_bf16(N, K, seed=1511)
    hyb = run_gemm(A, B, config=tile + "_k1_g4_h3")
    plain = run_gemm(A, B, config=tile + "_k1_g4")
    hyb32 = run_gemm(A, B, config=tile + "_k1_g4_h3", out_f32=True)
    plain32 = run_gemm(A, B, config=tile + "_k1_g4", out_f32=True)
    bm, bn = int(tile[1:].split("x")[0]), int(tile.split("x")[1])
    tiles_m, tiles_n = -(-M // bm), -(-N // bn)
    n1 = (tiles_m * tiles_n // 256) * 256 // tiles_m * bn
    assert 0 < n1 < N
    assert np.array_equal(hyb[:, :n1], plain[:, :n1])
    assert np.array_equal(hyb32[:, :n1], plain32[:, :n1])
    # the tail's sums run in another order (split K)
    assert np.count_nonzero(hyb32[:, n1:] != plain32[:, n1:]) > 0
    ref16, ref64 = _oracle().gemm(A, B)
    rep = check_bf16(hyb, ref16, ref64, K)
    print(tile, "hybrid", rep, flush=True)
    assert rep["ok"], rep
    assert check_f32(hyb32, ref64, K)["ok"]


def test_hybrid_f16_bit_exact():
    """The hybrid plan over fp16 operands (integers in [-16, 16], so fp16
    rounding of sums above 2048 happens in both parts' epilogues)."""
    tile, M, N = HYBRID_CASES[2]
    K = 456
    A = int_bf16(M, K, seed=1520, lo=-16, hi=16, fmt="f16")
    B = int_bf16(N, K, seed=1521, lo=-16, hi=16, fmt="f16")
    ref16, ref64 = _oracle().gemm(A, B, fmt="f16")
    got = run_gemm(A, B, config=tile + "_k1_g4_h3", fmt="f16")
    rep = check_bf16(got, ref16, None, K, exact=True, fmt="f16")
    print("f16 hybrid", rep, flush=True)
    assert rep["ok"], rep


# ------------------------------------------------------------ mixed plans
# "_m1" / "_m2": the tile columns that fill whole passes run on 256 x 256
# tiles, the columns after them unsplit on 256 x 128 / 128 x 128 tiles.
# 520 x 22920: 3 rows x 90 columns of 256 x 256 tiles, so the head is 85
# columns (21760) and the tail 1160 columns (3 x 10 tiles of 256 x 128, or
# 5 x 10 of 128 x 128; the last column ragged).
MIXED_PLANS = ["t256x256x64_w2x2_s2_x3_p10_k1_g4_m1", "t256x256x64_w2x2_s2_x3_p10_k1_g4_m2"]


@pytest.mark.parametrize("MIXED", MIXED_PLANS)
def test_mixed_plan_bit_exact(MIXED):
    """Integer inputs, K = 456 (a partial last K-step): the mixed plan is
    bit-exact in bf16 and fp32 output, over fp16 operands and through the
    no-allocation entry point."""
    import torch

    import dense_gemm_bf16_amd as g

    M, N, K = 520, 22920, 456
    A = int_bf16(M, K, seed=1540)
    B = int_bf16(N, K, seed=1541)
    ref16, ref64 = _oracle().gemm(A, B)
    rep = check_bf16(run_gemm(A, B, config=MIXED), ref16, None, K, exact=True)
    print("bf16", rep, flush=True)
    assert rep["ok"], rep
    assert check_f32(run_gemm(A, B, config=MIXED, out_f32=True), ref64, K, exact=True)["ok"]
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dB = torch.from_numpy(B.view(np.int16)).cuda()
    ldc = (N + 7) // 8 * 8
    dC = torch.zeros((M, ldc), dtype=torch.int16, device="cuda")
    g.gemm_bf16_ex_noalloc(MIXED, M, N, K, dA, K, dB, K, dC, ldc)
    torch.cuda.synchronize()
    assert np.array_equal(dC[:, :N].cpu().numpy().view(np.uint16), ref16)
    A16 = int_bf16(M, K, seed=1542, lo=-16, hi=16, fmt="f16")
    B16 = int_bf16(N, K, seed=1543, lo=-16, hi=16, fmt="f16")
    r16, _ = _oracle().gemm(A16, B16, fmt="f16")
    rep = check_bf16(run_gemm(A16, B16, config=MIXED, fmt="f16"), r16, None, K, exact=True,
                     fmt="f16")
    print("f16", rep, flush=True)
    assert rep["ok"], rep


@pytest.mark.parametrize("MIXED", MIXED_PLANS)
def test_mixed_plan_is_the_plain_plans_bits(MIXED):
    """N(0,1) inputs: the mixed plan gives the plain 256 x 256 plan's bits in
    every column (both tiles add the same K-steps in the same order), in
    bf16 and fp32 output, and meets the ulp criterion against the oracle."""
    M, N, K = 520, 22920, 1000
    A = normal_bf16(M, K, seed=1550)
    B = normal_bf16(N, K, seed=1551)
    plain = "t256x256x64_w2x2_s2_x3_p10_k1_g4"
    got = run_gemm(A, B, config=MIXED)
    assert np.array_equal(got, run_gemm(A, B, config=plain))
    got32 = run_gemm(A, B, config=MIXED, out_f32=True)
    assert np.array_equal(got32, run_gemm(A, B, config=plain, out_f32=True))
    ref16, ref64 = _oracle().gemm(A, B)
    rep = check_bf16(got, ref16, ref64, K)
    print(rep, flush=True)
    assert rep["ok"], rep


def test_random_mixed_plans_bit_exact():
    """Six seeded random mixed plans on shapes with a tail: 3 rows of 256 x
    256 tiles over 90 columns, M, N and K ragged, the tail on 256 x 128 or
    128 x 128 tiles, rotation and GROUP_M random, row strides padded with
    NaN, fp32 output for one call in three; integer inputs, bit-exact."""
    rng = np.random.default_rng(6161)
    o = _oracle()
    for i in range(6):
        M = 512 + int(rng.integers(1, 256))
        N = 89 * 256 + int(rng.integers(1, 256))
        K = int(rng.integers(130, 500))
        name = f"t256x256x64_w2x2_s2_x3_p10_k1_g{int(rng.choice([4, 8]))}"
        if rng.random() < 0.5:
            name += "_r1"
        name += f"_m{1 + i % 2}"
        pad_a, pad_b = 8 * int(rng.integers(0, 3)), 8 * int(rng.integers(0, 3))
        kk = (K + 7) // 8 * 8
        A = np.full((M, kk + pad_a), 0x7FC0, np.uint16)
        B = np.full((N, kk + pad_b), 0x7FC0, np.uint16)
        A[:, :K] = int_bf16(M, K, seed=1700 + 2 * i)
        B[:, :K] = int_bf16(N, K, seed=1701 + 2 * i)
        ref16, ref64 = o.gemm(A, B, K=K)
        f32 = i % 3 == 0
        got = run_gemm(A, B, K=K, config=name, out_f32=f32)
        if f32:
            rep = check_f32(got, ref64, K, exact=True)
        else:
            rep = check_bf16(got, ref16, None, K, exact=True)
        print(i, name, (M, N, K), "f32" if f32 else "bf16", rep, flush=True)
        assert rep["ok"], (name, (M, N, K), rep)


@pytest.mark.parametrize("M,N,K,kind,n1", [(2048, 5376, 8192, "_h", 4096),
                                           (2048, 10240, 8192, "_m2", 8192)])
def test_automatic_split_plans_on_a_qkv_shape(M, N, K, kind, n1):
    """Shapes whose tiles make 1.31 and 1.25 passes over the CUs (the second
    a 70B-class fused QKV projection at 2048 tokens): the automatic plan is a
    hybrid (256 x 128 tiles, the tail from column n1 split along K) or a
    mixed one (256 x 256 tiles, the tail on 128 x 128 tiles); full rows and
    columns on both sides of the split column are checked against the
    oracle."""
    import dense_gemm_bf16_amd as g

    plan = g.config_name(M, N, K)
    print("plan", plan, flush=True)
    assert kind in plan, plan
    A = normal_bf16(M, K, seed=1530)
    B = normal_bf16(N, K, seed=1531, std=K ** -0.5)
    got = run_gemm(A, B)
    o = _oracle()
    rows = np.array([0, 1, 255, 256, M // 2 + 3, M - 1])
    cols = np.array([0, n1 - 1, n1, n1 + 1, (n1 + N) // 2, N - 1])
    r16, r64 = o.gemm(np.ascontiguousarray(A[rows]), B)
    rep = check_bf16(got[rows], r16, r64, K, 1.0, K ** -0.5)
    print("rows", rep, flush=True)
    assert rep["ok"], rep
    c16, c64 = o.gemm(A, np.ascontiguousarray(B[cols]))
    rep = check_bf16(got[:, cols], c16, c64, K, 1.0, K ** -0.5)
    print("cols", rep, flush=True)
    assert rep["ok"], rep


@pytest.mark.parametrize("M,N,K,rot", [(200, 11008, 4096, True), (224, 4096, 11008, True),
                                       (192, 4096, 4096, False)])
def test_two_rows_of_128_tiles_automatic_plan(M, N, K, rot):
    """128 < M <= 256 on two rows of 128 x 128 tiles: the automatic plan
    rotates the K order exactly on long K loops; either way every element
    is bit-exact on integers (full check)."""
    import dense_gemm_bf16_amd as g

    plan = g.config_name(M, N, K)
    print("plan", plan, flush=True)
    assert plan.startswith("t128x128") and ("_r1" in plan) == rot, plan
    A = int_bf16(M, K, seed=1600 + M)
    B = int_bf16(N, K, seed=1601 + M)
    ref16, _ = _oracle().gemm(A, B)
    rep = check_bf16(run_gemm(A, B), ref16, None, K, exact=True)
    print(rep, flush=True)
    assert rep["ok"], rep
