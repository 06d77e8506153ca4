"""GPU parity over the number formats' special codes.

Every E4M3FN scale byte (zero, -0, the subnormals 0x01..0x07, negatives, the
NaNs 0x7F and 0xFF) and every E2M1 code (including -0) goes through the FP4
GEMM, its split-K form and W4A16; BF16 +-Inf, NaN and subnormal values go
through the dense, order-preserving and fused-fold kernels. Inputs are built
so that every FP32 partial sum is exact whatever the summation order, so the
oracle fixes each output uniquely and the comparison is by value (NaN matches
NaN, -0 matches +0: the sign of an exact zero sum depends on the order).

Scale decoding follows the kernelbot NVFP4 GEMM page's "SCALE FACTORS"
section (one E4M3 scale per 16 K elements, applied to every element of its
group); the BF16 cases follow the IEEE arithmetic the FP32 accumulation of
the sm121a_matmul.py page's kernel implies.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
import synthetic
from gpu_util import assert_values_equal, bits_of, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu


def _all_scale_rows(rows, k, seed, tid):
    """[rows, k/16] scale bytes, one byte per row repeated over its groups:
    row r takes byte perm[r % 256] (every byte appears once per 256 rows)."""
    perm = np.random.default_rng(seed).permutation(256).astype(np.uint8)
    return np.repeat(perm[np.arange(rows) % 256][:, None], k // 16, axis=1)


def _fp4_specials(k=64, seed=0):
    """A, B: 256 rows each, every nibble code uniform, every scale byte once on
    each side (per row). Each dot product is s_i * t_j * T with 4*T an integer
    below 2^14 (K = 64) or 2^16 (K = 256): exact in FP32 in any order."""
    a = synthetic.fp4_packed(256, k, 900 + seed, 0)
    b = synthetic.fp4_packed(256, k, 900 + seed, 1)
    sfa = _all_scale_rows(256, k, 910 + seed, 4)
    sfb = _all_scale_rows(256, k, 920 + seed, 5)
    return a, sfa, b, sfb


def _want_fp4(a, sfa, b, sfb):
    ref = oracle.gemm_fp4_ref(a, sfa, b, sfb)
    fin = np.isfinite(ref)
    assert np.array_equal(ref[fin], ref[fin].astype(np.float32).astype(np.float64)), "not exact in FP32"
    return oracle.f32_to_bf16(ref.astype(np.float32))


@pytest.mark.parametrize("cfg", [-1, 0, 2, 10, 11])
def test_every_scale_byte_and_code_fp4(cfg, force):
    if cfg >= 0:
        force(bg.TUNE_FP4_TILE, cfg)
    a, sfa, b, sfb = _fp4_specials()
    # the construction covers every byte on both sides and every nibble code
    assert set(np.unique(sfa)) == set(range(256)) and set(np.unique(sfb)) == set(range(256))
    assert set(np.unique(oracle.unpack_e2m1(a))) == set(range(16))
    want = _want_fp4(a, sfa, b, sfb)
    assert np.isnan(oracle.bf16_to_f64(want)).any() and (oracle.bf16_to_f64(want) == 0).any()
    c = bg.gemm_fp4_blockscaled(to_dev_u8(a), to_dev_u8(sfa), to_dev_u8(b), to_dev_u8(sfb))
    torch.cuda.synchronize()
    assert_values_equal(bits_of(c), want, "fp4 special codes")


@pytest.mark.parametrize("ks,tile", [(2, -1), (4, -1), (4, 0), (2, 1), (4, 7), (3, 7), (3, 8), (3, 9)])
def test_every_scale_byte_and_code_fp4_splitk(ks, tile, force):
    if tile >= 0:
        force(bg.TUNE_FP4_SPLITK_TILE, tile)
    a, sfa, b, sfb = _fp4_specials(k=256, seed=1)
    want = _want_fp4(a, sfa, b, sfb)
    c = bg.gemm_fp4_blockscaled_splitk(to_dev_u8(a), to_dev_u8(sfa), to_dev_u8(b), to_dev_u8(sfb), ks)
    torch.cuda.synchronize()
    assert_values_equal(bits_of(c), want, f"fp4 split-K {ks} special codes")


@pytest.mark.parametrize("s2,cfg", [(1.0, -1), (0.0123, -1), (-3.0, -1), (0.0123, 0), (-3.0, 2)])
def test_every_weight_scale_byte_and_code_w4a16(s2, cfg, force):
    """Grid activations j * 2^-5 (|j| <= 8) times weights with every scale
    byte: each dot product is t_j * T with 64*T an integer below 2^13, exact
    in FP32; C = bf16(fl32(s2 * acc)), NaN rows where the scale is NaN."""
    if cfg >= 0:
        force(bg.TUNE_W4A16_TILE, cfg)
    k = 64
    a = synthetic.grid_bf16((96, k), -8, 8, -5, 930, 0)
    _, _, b, sfb = _fp4_specials(k=k, seed=2)
    nan_rows = np.isnan(oracle.e4m3fn_to_f64(sfb[:, 0]))
    want = np.empty((96, 256), np.uint16)
    ok = ~nan_rows
    want[:, ok] = oracle.gemm_w4a16_exact(a, b[ok], sfb[ok], s2)
    want[:, nan_rows] = 0x7FC0
    c = bg.gemm_w4a16(to_dev_bf16(a), to_dev_u8(b), to_dev_u8(sfb), s2)
    torch.cuda.synchronize()
    assert_values_equal(bits_of(c), want, f"w4a16 special codes s2={s2}")


def _bf16_specials(m, k, seed):
    """Grid values j * 2^-5 with BF16 specials planted: +-Inf, NaN, and
    subnormals (2^-130, -3 * 2^-133)."""
    a = synthetic.grid_bf16((m, k), -8, 8, -5, seed, 0).copy()
    g = np.random.default_rng(seed)
    flat = a.reshape(-1)
    for code, count in ((0x7F80, 3), (0xFF80, 3), (0x7FC0, 2), (0x0020, 6), (0x8006, 6)):
        flat[g.choice(flat.size, count, replace=False)] = code
    return a


@pytest.mark.parametrize("k", [64, 67])
def test_bf16_specials_dense_identity(k):
    """B = identity (N = K): C[i, j] = A[i, j] exactly where row i is finite;
    a row holding +-Inf at k0 gives NaN (Inf * 0) in every other column and
    the infinity in column k0; subnormal inputs come out unchanged."""
    a = _bf16_specials(40, k, 940 + k)
    eye = oracle.f32_to_bf16(np.eye(k, dtype=np.float32))
    want = oracle.f32_to_bf16(oracle.gemm_bf16_ref(a, eye).astype(np.float32))
    assert np.isinf(oracle.bf16_to_f64(want)).any() and np.isnan(oracle.bf16_to_f64(want)).any()
    c = bg.gemm_bf16(to_dev_bf16(a), to_dev_bf16(eye))
    torch.cuda.synchronize()
    assert_values_equal(bits_of(c), want, f"dense specials k={k}")


def test_bf16_specials_ordered():
    x = _bf16_specials(70, 300, 950)
    w = synthetic.grid_bf16((33, 300), -8, 8, -5, 951, 1)
    c32 = bg.gemm_bf16_ordered_f32(to_dev_bf16(x), to_dev_bf16(w))
    c16 = bg.gemm_bf16_ordered(to_dev_bf16(x), to_dev_bf16(w))
    torch.cuda.synchronize()
    want32 = oracle.gemm_ordered_f32(x, w)
    got32 = c32.cpu().numpy()
    same = (np.isnan(got32) & np.isnan(want32)) | (got32.view(np.uint32) == want32.view(np.uint32))
    assert same.all(), f"{int((~same).sum())} FP32 sums differ"
    assert_values_equal(bits_of(c16), oracle.f32_to_bf16(want32), "ordered specials")


def test_bf16_specials_fold():
    """Specials in `out` (Inf + 2 d = Inf, NaN stays NaN, subnormal + 2 d in
    FP32) and in X (an infinite or NaN delta)."""
    m, n, k = 64, 96, 64
    out = _bf16_specials(m, n, 960)
    x = _bf16_specials(m, k, 961)
    b = synthetic.grid_bf16((n, k), -8, 8, -5, 962, 1)
    want = oracle.gemm_scaled_acc_exact(out, x, b, 2.0)
    o = to_dev_bf16(out)
    bg.gemm_bf16_scaled_acc(to_dev_bf16(x), to_dev_bf16(b), o, 2.0)
    torch.cuda.synchronize()
    assert_values_equal(bits_of(o), want, "fold specials")


def test_every_weight_scale_byte_and_code_w4a16_transposed():
    """The transposed-weight entry point on the same special-code weights,
    stored [K/2, ldb] with an odd stride (byte loads) and a multiple of 4."""
    k = 64
    a = synthetic.grid_bf16((96, k), -8, 8, -5, 931, 0)
    _, _, b, sfb = _fp4_specials(k=k, seed=3)
    nan_rows = np.isnan(oracle.e4m3fn_to_f64(sfb[:, 0]))
    want = np.empty((96, 256), np.uint16)
    want[:, ~nan_rows] = oracle.gemm_w4a16_exact(a, b[~nan_rows], sfb[~nan_rows], 0.75)
    want[:, nan_rows] = 0x7FC0
    for ldb in (257, 260):
        bt = np.zeros((k // 2, ldb), np.uint8)
        bt[:, :256] = b.T
        sfbt = np.zeros((k // 16, ldb), np.uint8)
        sfbt[:, :256] = sfb.T
        c = bg.gemm_w4a16_t(to_dev_bf16(a), to_dev_u8(bt), to_dev_u8(sfbt), 256, 0.75)
        torch.cuda.synchronize()
        assert_values_equal(bits_of(c), want, f"w4a16_t special codes ldb={ldb}")
