"""GPU parity of gemm_w4a16 (BF16 activations x NVFP4 weights, per-tensor scale)."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
import synthetic
from gpu_util import assert_bits_equal, bits_of, check_close, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu

S2 = synthetic.W4A16_SCALE_2


def _run(a, b, sfb, s2):
    c = bg.gemm_w4a16(to_dev_bf16(a), to_dev_u8(b), to_dev_u8(sfb), s2)
    torch.cuda.synchronize()
    return bits_of(c)


def _check(a, b, sfb, s2, rows=None, what=""):
    got = _run(a, b, sfb, s2)
    k = a.shape[1]
    sel = slice(None) if rows is None else rows
    ref = oracle.gemm_w4a16_ref(a[sel], b, sfb, s2)
    sig_b = oracle.rms(oracle.dequant_fp4(b, sfb)) * abs(float(np.float32(s2)))
    check_close(got[sel], ref, k, oracle.rms(oracle.bf16_to_f64(a)), sig_b, what)


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (65, 129, 48), (7, 300, 64), (130, 66, 272),
                                   (257, 255, 1040), (33, 17, 528), (300, 520, 2048),
                                   (65, 129, 96), (300, 200, 1056)])
def test_w4a16_edge_shapes(m, n, k):
    print(f"w4a16 edge m={m} n={n} k={k}", flush=True)
    a = synthetic.normal_bf16((m, k), 1.0, 100 + m, 0)
    b = synthetic.fp4_packed(n, k, 100 + n, 1)
    sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 100, 5)
    _check(a, b, sfb, S2, what=f"w4a16 {m}x{n}x{k}")


@pytest.mark.parametrize("s2", [S2, 1.0, -3.0, 2.0 ** -20])
@pytest.mark.parametrize("m,n,k", [(96, 80, 3008), (257, 131, 512), (5, 600, 64)])
def test_w4a16_exactly_summable_bit_exact(m, n, k, s2):
    """Grid activations and weight scales in {1, 2}: the FP32 dot products are
    exact in any order, so C = bf16(fl32(s2 * acc)) is unique."""
    a = synthetic.grid_bf16((m, k), -8, 8, -5, 101, 0)
    b = synthetic.fp4_packed(n, k, 101, 1)
    sfb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40], 101, 5)
    assert_bits_equal(_run(a, b, sfb, s2), oracle.gemm_w4a16_exact(a, b, sfb, s2), f"w4a16 exact s2={s2}")


def test_w4a16_qkvz_workload_all_rows():
    print("w4a16 1016x12288x2048", flush=True)
    a, b, sfb, s2 = synthetic.w4a16_gemm()
    _check(a, b, sfb, s2, what="w4a16 qkvz")


# K % 32 == 16 takes 16-element FP4 staging units and the default tiles;
# K % 32 == 0 takes 32-element units and every forced tile (the K = 96,
# 224 and 1056 cases end in half a 64-wide step)
FP4_TILE_SHAPES = [(1, 1, 16), (65, 129, 48), (257, 255, 1040), (300, 520, 208),
                   (1, 1, 32), (65, 129, 96), (257, 255, 1056), (300, 520, 224)]


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5, 6, 7, 9])
def test_every_w4a16_tile_config(cfg, force):
    """Each W4A16 tile variant (the BG_TUNE_W4A16_TILE override) on ragged shapes."""
    force(bg.TUNE_W4A16_TILE, cfg)
    for m, n, k in FP4_TILE_SHAPES:
        a = synthetic.normal_bf16((m, k), 1.0, 110 + cfg, 0)
        b = synthetic.fp4_packed(n, k, 110 + cfg, 1)
        sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 110, 5)
        _check(a, b, sfb, S2, what=f"w4a16 cfg {cfg} {m}x{n}x{k}")
        ga = synthetic.grid_bf16((m, k), -8, 8, -5, 111, 0)
        eb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40], 111, 5)
        assert_bits_equal(_run(ga, b, eb, 0.75), oracle.gemm_w4a16_exact(ga, b, eb, 0.75),
                          f"w4a16 cfg {cfg} exact {m}x{n}x{k}")


def test_w4a16_equals_fp4_gemm_on_fp4_valued_activations():
    """A holding exact E2M1 values (unit scales) and s2 = 1: both entry points
    compute the same exact sums, so their outputs agree bit for bit."""
    m, n, k = 200, 136, 512
    qa = synthetic.fp4_packed(m, k, 112, 0)
    one = np.full((m, k // 16), 0x38, np.uint8)
    a = oracle.f32_to_bf16(oracle.dequant_fp4(qa, one).astype(np.float32))
    b = synthetic.fp4_packed(n, k, 112, 1)
    sfb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40], 112, 5)
    w = _run(a, b, sfb, 1.0)
    c = bg.gemm_fp4_blockscaled(to_dev_u8(qa), to_dev_u8(one), to_dev_u8(b), to_dev_u8(sfb))
    torch.cuda.synchronize()
    assert_bits_equal(w, bits_of(c), "w4a16 vs fp4")


# ---------------------------------------------------------------------------
# transposed weights with an explicit row stride (gemm_w4a16_t)
# ---------------------------------------------------------------------------

def _transposed(n, k, ldb, seed, scale_choice=None):
    """Bt [K/2, ldb] and SFBt [K/16, ldb], pad columns zero-filled (the page's
    convention), plus the same weights in gemm_w4a16's [N, K/2] layout."""
    b = synthetic.fp4_packed(n, k, seed, 1)
    if scale_choice is None:
        sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, seed, 5)
    else:
        sfb = synthetic.e4m3_choice(n, k // 16, scale_choice, seed, 5)
    bt = np.zeros((k // 2, ldb), np.uint8)
    bt[:, :n] = b.T
    sfbt = np.zeros((k // 16, ldb), np.uint8)
    sfbt[:, :n] = sfb.T
    return b, sfb, bt, sfbt


def _run_t(a, bt, sfbt, n, s2):
    c = bg.gemm_w4a16_t(to_dev_bf16(a), to_dev_u8(bt), to_dev_u8(sfbt), n, s2)
    torch.cuda.synchronize()
    return bits_of(c)


@pytest.mark.parametrize("ldb", [248192, 248077])
def test_w4a16_t_lm_head_odd_vocab(ldb):
    """lm_head-like: N = 248077 (odd), ldb = align_up(N, 128) with zero pad
    (4-byte column loads) and ldb = N (byte loads); every output against the
    oracle's transposed-layout definition."""
    m, n, k = 37, 248077, 512
    print(f"w4a16_t lm_head m={m} n={n} k={k} ldb={ldb}", flush=True)
    a = synthetic.normal_bf16((m, k), 1.0, 120, 0)
    bt = np.zeros((k // 2, ldb), np.uint8)
    bt[:, :n] = synthetic.fp4_packed(k // 2, 2 * n, 120, 1)
    sfbt = np.zeros((k // 16, ldb), np.uint8)
    sfbt[:, :n] = synthetic.e4m3_uniform(k // 16, n, 2 ** -4, 2 ** 4, 120, 5)
    got = _run_t(a, bt, sfbt, n, S2)
    ref = oracle.gemm_w4a16_t_ref(a, bt, sfbt, n, S2)
    sig_b = oracle.rms(oracle.dequant_fp4_t(bt, sfbt, n)) * abs(float(np.float32(S2)))
    check_close(got, ref, k, oracle.rms(oracle.bf16_to_f64(a)), sig_b, f"w4a16_t lm_head ldb={ldb}")


T_SHAPES = [(130, 1001, 256, 1004), (7, 300, 64, 301), (64, 257, 160, 257), (200, 4099, 512, 4224),
            (1, 1, 16, 1), (33, 130, 48, 133), (300, 520, 224, 520)]


@pytest.mark.parametrize("cfg", [-1, 0, 1, 2])
def test_w4a16_t_exact_and_equal_to_w4a16(cfg, force):
    """Grid activations and scales in {1, 2}: exact FP32 sums, so every output
    is unique (bit-exact against the oracle), and with the same tile the
    transposed entry point equals gemm_w4a16 on the same weights bit for bit."""
    if cfg >= 0:
        force(bg.TUNE_W4A16_TILE, cfg)
    for m, n, k, ldb in T_SHAPES:
        print(f"w4a16_t cfg={cfg} m={m} n={n} k={k} ldb={ldb}", flush=True)
        a = synthetic.grid_bf16((m, k), -8, 8, -5, 121, 0)
        b, sfb, bt, sfbt = _transposed(n, k, ldb, 121, [0x38, 0x40])
        got = _run_t(a, bt, sfbt, n, 0.75)
        assert_bits_equal(got, oracle.gemm_w4a16_exact(a, b, sfb, 0.75), f"w4a16_t exact {m}x{n}x{k} ldb={ldb}")
        if cfg >= 0:
            assert_bits_equal(got, _run(a, b, sfb, 0.75), f"w4a16_t vs w4a16 cfg {cfg}")
        # random data within the tolerance
        ar = synthetic.normal_bf16((m, k), 1.0, 122, 0)
        b2, sfb2, bt2, sfbt2 = _transposed(n, k, ldb, 122)
        ref = oracle.gemm_w4a16_t_ref(ar, bt2, sfbt2, n, S2)
        check_close(_run_t(ar, bt2, sfbt2, n, S2), ref, k, oracle.rms(oracle.bf16_to_f64(ar)),
                    oracle.rms(oracle.dequant_fp4_t(bt2, sfbt2, n)) * abs(S2), f"w4a16_t {m}x{n}x{k} ldb={ldb}")
