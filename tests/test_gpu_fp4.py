"""GPU parity of the block-scaled FP4 GEMM."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
import synthetic
from gpu_util import assert_bits_equal, bits_of, check_close, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu


def _run(a, sfa, b, sfb):
    c = bg.gemm_fp4_blockscaled(to_dev_u8(a), to_dev_u8(sfa), to_dev_u8(b), to_dev_u8(sfb))
    torch.cuda.synchronize()
    return bits_of(c)


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (65, 129, 48), (7, 300, 64), (130, 66, 272),
                                   (257, 255, 1040), (128, 128, 128), (33, 17, 16 * 33)])
def test_fp4_edge_shapes(m, n, k):
    print(f"fp4 edge m={m} n={n} k={k}", flush=True)
    a, b = synthetic.fp4_packed(m, k, 60, 0), synthetic.fp4_packed(n, k, 60, 1)
    sfa = synthetic.e4m3_uniform(m, k // 16, 2 ** -4, 2 ** 4, 60, 4)
    sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 60, 5)
    got = _run(a, sfa, b, sfb)
    ref = oracle.gemm_fp4_ref(a, sfa, b, sfb)
    check_close(got, ref, k, oracle.rms(oracle.dequant_fp4(a, sfa)), oracle.rms(oracle.dequant_fp4(b, sfb)),
                f"fp4 {m}x{n}x{k}")


def test_fp4_unit_scales_equal_dense_path_on_dequantized_operands():
    m, n, k = 200, 136, 512
    a, b = synthetic.fp4_packed(m, k, 61, 0), synthetic.fp4_packed(n, k, 61, 1)
    one_a = np.full((m, k // 16), 0x38, np.uint8)
    one_b = np.full((n, k // 16), 0x38, np.uint8)
    got = _run(a, one_a, b, one_b)
    ab = oracle.f32_to_bf16(oracle.dequant_fp4(a, one_a).astype(np.float32))
    bb = oracle.f32_to_bf16(oracle.dequant_fp4(b, one_b).astype(np.float32))
    dense = bg.gemm_bf16(to_dev_bf16(ab), to_dev_bf16(bb))
    torch.cuda.synchronize()
    # FP4 products are multiples of 1/4 bounded by 36: sums over 512 terms are exact in FP32
    assert_bits_equal(got, bits_of(dense), "fp4 vs dense")


def test_fp4_full_size_power_of_two_scales_bit_exact():
    """Scales in {1, 2}: every partial sum is exact in FP32, so C is unique."""
    print("fp4 4096x4096x8192 exact scales", flush=True)
    m = n = 4096
    k = 8192
    a, b = synthetic.fp4_packed(m, k, 4, 0), synthetic.fp4_packed(n, k, 4, 1)
    sfa = synthetic.e4m3_choice(m, k // 16, [0x38, 0x40], 4, 4)
    sfb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40], 4, 5)
    got = _run(a, sfa, b, sfb)
    want = oracle.f32_to_bf16(oracle.gemm_fp4_ref(a, sfa, b, sfb).astype(np.float32))
    assert_bits_equal(got, want, "fp4 full exact")


def test_fp4_config_sampled_rows():
    print("fp4 config sampled rows", flush=True)
    a, sfa, b, sfb = synthetic.fp4_gemm()
    got = _run(a, sfa, b, sfb)
    rows = synthetic.sample_rows(a.shape[0], 1024, 1004)
    ref = oracle.gemm_fp4_ref(a[rows], sfa[rows], b, sfb)
    check_close(got[rows], ref, 8192, oracle.rms(oracle.dequant_fp4(a, sfa)),
                oracle.rms(oracle.dequant_fp4(b, sfb)), "fp4 config")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_every_fp4_tile_config(cfg, monkeypatch):
    """Each FP4 tile variant (BLOCKGEMM_FP4_TILE, a tuning hook) on ragged shapes."""
    monkeypatch.setenv("BLOCKGEMM_FP4_TILE", str(cfg))
    for m, n, k in [(1, 1, 16), (65, 129, 48), (257, 255, 1040), (300, 520, 208)]:
        a, b = synthetic.fp4_packed(m, k, 70 + cfg, 0), synthetic.fp4_packed(n, k, 70 + cfg, 1)
        sfa = synthetic.e4m3_uniform(m, k // 16, 2 ** -4, 2 ** 4, 70, 4)
        sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 70, 5)
        got = _run(a, sfa, b, sfb)
        check_close(got, oracle.gemm_fp4_ref(a, sfa, b, sfb), k, oracle.rms(oracle.dequant_fp4(a, sfa)),
                    oracle.rms(oracle.dequant_fp4(b, sfb)), f"fp4 cfg {cfg} {m}x{n}x{k}")
        # power-of-two scales: exact in FP32, so bit-exact
        ea = synthetic.e4m3_choice(m, k // 16, [0x38, 0x40], 71, 4)
        eb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40], 71, 5)
        want = oracle.f32_to_bf16(oracle.gemm_fp4_ref(a, ea, b, eb).astype(np.float32))
        assert_bits_equal(_run(a, ea, b, eb), want, f"fp4 cfg {cfg} exact {m}x{n}x{k}")
