"""GPU checks of gemm_bf16_strided (row-strided operands and output).

Strides that are multiples of 8 elements keep the direct-load kernels and
must give exactly the contiguous result (same tiles, same K order); other
strides take the guarded element-wise path. C's padding elements between
rows are never written.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
import synthetic
from gpu_util import assert_bits_equal, bits_of, check_close, to_dev_bf16

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1   # a NaN pattern no product writes


def _padded(bits, ld):
    """Device tensor of shape [rows, ld] holding `bits` in its first columns, and the view."""
    rows, cols = bits.shape
    buf = np.full((rows, ld), SENTINEL, np.uint16)
    buf[:, :cols] = bits
    dev = to_dev_bf16(buf)
    return dev, dev[:, :cols]


def _strided(a, b, lda, ldb, ldc):
    m, n = a.shape[0], b.shape[0]
    _, av = _padded(a, lda)
    _, bv = _padded(b, ldb)
    cbuf, cv = _padded(np.full((m, n), SENTINEL, np.uint16), ldc)
    bg.gemm_bf16_strided(av, bv, cv)
    torch.cuda.synchronize()
    full = bits_of(cbuf)
    assert (full[:, n:] == SENTINEL).all(), "padding of C was written"
    return full[:, :n]


@pytest.mark.parametrize("m,n,k,lda,ldb,ldc", [
    (200, 136, 2000, 2064, 2008, 160),     # aligned strides: direct-load kernels
    (1, 1, 64, 72, 64, 8),
    (257, 255, 1040, 1040, 1104, 256),
    (300, 200, 1000, 1003, 1005, 201),     # unaligned strides: guarded path
    (65, 129, 72, 77, 73, 130),
])
def test_strided_matches_contiguous_and_oracle(m, n, k, lda, ldb, ldc):
    print(f"strided m={m} n={n} k={k} lda={lda} ldb={ldb} ldc={ldc}", flush=True)
    a = synthetic.normal_bf16((m, k), 1.0, 120, 0)
    b = synthetic.normal_bf16((n, k), 0.05, 120, 1)
    got = _strided(a, b, lda, ldb, ldc)
    check_close(got, oracle.gemm_bf16_ref(a, b), k, oracle.rms(oracle.bf16_to_f64(a)),
                oracle.rms(oracle.bf16_to_f64(b)), f"strided {m}x{n}x{k}")
    if lda % 8 == 0 and ldb % 8 == 0:
        c = bg.gemm_bf16(to_dev_bf16(a), to_dev_bf16(b))
        torch.cuda.synchronize()
        assert_bits_equal(got, bits_of(c), "strided vs contiguous")
    ga = synthetic.grid_bf16((m, k), -8, 8, -5, 121, 0)
    gb = synthetic.grid_bf16((n, k), -8, 8, -5, 121, 1)
    want = oracle.f32_to_bf16(oracle.gemm_bf16_ref(ga, gb).astype(np.float32))
    assert_bits_equal(_strided(ga, gb, lda, ldb, ldc), want, "strided grid")


def test_gate_and_up_into_one_fused_buffer():
    """The MLP gate and up projections written side by side into one
    [5120, 22016] buffer (ldc = 22016); each half equals its own gemm_bf16."""
    a, wg = synthetic.mlp_gate_up()
    wu = synthetic.normal_bf16((11008, 2048), 0.02, 2, synthetic.TID_B2 + 10)
    da, dg, du = to_dev_bf16(a), to_dev_bf16(wg), to_dev_bf16(wu)
    fused = torch.empty((5120, 22016), dtype=torch.bfloat16, device="cuda")
    bg.gemm_bf16_strided(da, dg, fused[:, :11008])
    bg.gemm_bf16_strided(da, du, fused[:, 11008:])
    g = bg.gemm_bf16(da, dg)
    u = bg.gemm_bf16(da, du)
    torch.cuda.synchronize()
    assert_bits_equal(bits_of(fused[:, :11008].contiguous()), bits_of(g), "gate half")
    assert_bits_equal(bits_of(fused[:, 11008:].contiguous()), bits_of(u), "up half")


def test_odd_vocab_n_with_padded_output():
    """An lm_head-like odd N (32771) with a 16-element-padded C row stride."""
    m, n, k = 64, 32771, 2048
    a = synthetic.normal_bf16((m, k), 1.0, 122, 0)
    b = synthetic.normal_bf16((n, k), 0.02, 122, 1)
    got = _strided(a, b, k, k, 32784)
    check_close(got, oracle.gemm_bf16_ref(a, b), k, oracle.rms(oracle.bf16_to_f64(a)),
                oracle.rms(oracle.bf16_to_f64(b)), "odd vocab")
