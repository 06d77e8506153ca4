"""K = 0 on every GEMM entry point: each output element is the empty sum.

Empty operands arrive with NULL data pointers, and every output starts filled
with a nonzero pattern, so a launch that skips its stores, or one that treats
the missing pointer as a reason to do nothing, fails here. The expected
values are the oracle's on the same empty operands: +0 for the plain
products (a scale of the empty sum keeps the scale's sign for W4A16), and
out + scale * bf16(+0) for the fused fold.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
import synthetic
from gpu_util import DEV, assert_bits_equal, bits_of, empty_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu

# one tile and a ragged grid of several tiles (the FP4 tile choice changes at
# M = 192, the split-K planes at the same point)
SHAPES = [(70, 40), (300, 260)]
FILL = 0x3F80   # bf16 1.0


def _bf16_of(ref):
    return oracle.f32_to_bf16(np.asarray(ref, dtype=np.float64).astype(np.float32))


def _empty_bf16(rows):
    return torch.empty((rows, 0), dtype=torch.bfloat16, device=DEV)


def _empty_u8(rows):
    return torch.empty((rows, 0), dtype=torch.uint8, device=DEV)


def _host_bf16(rows):
    return np.zeros((rows, 0), np.uint16)


def _host_u8(rows):
    return np.zeros((rows, 0), np.uint8)


@pytest.mark.parametrize("m,n", SHAPES)
def test_strided_k_zero(m, n):
    print(f"gemm_bf16_strided K=0 {m}x{n}", flush=True)
    c = empty_bf16(m, n, FILL)
    bg.gemm_bf16_strided(_empty_bf16(m), _empty_bf16(n), c)
    torch.cuda.synchronize()
    assert_bits_equal(bits_of(c), _bf16_of(oracle.gemm_bf16_ref(_host_bf16(m), _host_bf16(n))), "strided")


@pytest.mark.parametrize("scale", [0.75, -1.5])
@pytest.mark.parametrize("m,n", SHAPES)
def test_scaled_acc_k_zero_leaves_out_plus_zero(m, n, scale):
    """out + scale * bf16(+0): every value of out survives, except that a -0
    in out becomes +0 when scale is positive (-0 + +0 = +0)."""
    print(f"gemm_bf16_scaled_acc K=0 {m}x{n} scale={scale}", flush=True)
    out0 = synthetic.normal_bf16((m, n), 1.0, 11, 0)
    out0.reshape(-1)[::7] = 0x8000   # some -0
    out0.reshape(-1)[3::7] = 0x0000  # some +0
    out = to_dev_bf16(out0)
    bg.gemm_bf16_scaled_acc(_empty_bf16(m), _empty_bf16(n), out, scale)
    torch.cuda.synchronize()
    delta = _bf16_of(oracle.gemm_bf16_ref(_host_bf16(m), _host_bf16(n)))
    assert_bits_equal(bits_of(out), oracle.scaled_acc_epilogue(out0, delta, scale), "scaled_acc")


@pytest.mark.parametrize("k_splits", [1, 2, 5])
@pytest.mark.parametrize("m,n", SHAPES)
def test_splitk_k_zero(m, n, k_splits):
    print(f"gemm_bf16_splitk K=0 {m}x{n} splits={k_splits}", flush=True)
    c = empty_bf16(m, n, FILL)
    ws = None
    if k_splits > 1:
        ws = torch.full((k_splits, m, n), 3.0, dtype=torch.float32, device=DEV)
    bg.gemm_bf16_splitk(_empty_bf16(m), _empty_bf16(n), k_splits, workspace=ws, out=c)
    torch.cuda.synchronize()
    planes = oracle.gemm_splitk_planes_ref(_host_bf16(m), _host_bf16(n), k_splits)
    assert_bits_equal(bits_of(c), oracle.splitk_reduce(planes), "splitk")
    if ws is not None:
        got = ws.cpu().numpy().view(np.uint32)
        assert not got.any(), "every workspace plane holds the empty partial sum, +0"


@pytest.mark.parametrize("m,n", SHAPES)
def test_ordered_k_zero(m, n):
    print(f"gemm_bf16_ordered(_f32) K=0 {m}x{n}", flush=True)
    c = empty_bf16(m, n, FILL)
    c32 = torch.full((m, n), -2.0, dtype=torch.float32, device=DEV)
    a, b = _empty_bf16(m), _empty_bf16(n)
    bg.gemm_bf16_ordered(a, b, out=c)
    bg.gemm_bf16_ordered_f32(a, b, out=c32)
    torch.cuda.synchronize()
    ha, hb = _host_bf16(m), _host_bf16(n)
    assert_bits_equal(bits_of(c), oracle.gemm_ordered(ha, hb), "ordered")
    ref32 = oracle.gemm_ordered_f32(ha, hb)
    assert np.array_equal(c32.cpu().numpy().view(np.uint32), ref32.view(np.uint32))


@pytest.mark.parametrize("m,n", SHAPES)
def test_fp4_k_zero(m, n):
    print(f"gemm_fp4_blockscaled K=0 {m}x{n}", flush=True)
    c = empty_bf16(m, n, FILL)
    bg.gemm_fp4_blockscaled(_empty_u8(m), _empty_u8(m), _empty_u8(n), _empty_u8(n), out=c)
    torch.cuda.synchronize()
    ref = oracle.gemm_fp4_ref(_host_u8(m), _host_u8(m), _host_u8(n), _host_u8(n))
    assert_bits_equal(bits_of(c), _bf16_of(ref), "fp4")


def test_fp4_batched_k_zero():
    l, m, n = 3, 130, 70
    print(f"gemm_fp4_blockscaled_batched K=0 {l}x{m}x{n}", flush=True)
    e = lambda r: torch.empty((l, r, 0), dtype=torch.uint8, device=DEV)
    c = torch.full((l, m, n), 1.0, dtype=torch.bfloat16, device=DEV)
    bg.gemm_fp4_blockscaled_batched(e(m), e(m), e(n), e(n), out=c)
    torch.cuda.synchronize()
    ref = oracle.gemm_fp4_ref(_host_u8(m), _host_u8(m), _host_u8(n), _host_u8(n))
    for i in range(l):
        assert_bits_equal(bits_of(c[i]), _bf16_of(ref), f"fp4 batched [{i}]")


@pytest.mark.parametrize("k_splits", [2, 4])
@pytest.mark.parametrize("m,n", SHAPES)
def test_fp4_splitk_k_zero(m, n, k_splits):
    print(f"gemm_fp4_blockscaled_splitk K=0 {m}x{n} splits={k_splits}", flush=True)
    c = empty_bf16(m, n, FILL)
    ws = torch.full((k_splits, m, n), 3.0, dtype=torch.float32, device=DEV)
    bg.gemm_fp4_blockscaled_splitk(_empty_u8(m), _empty_u8(m), _empty_u8(n), _empty_u8(n), k_splits,
                                   workspace=ws, out=c)
    torch.cuda.synchronize()
    planes = oracle.gemm_fp4_splitk_planes_ref(_host_u8(m), _host_u8(m), _host_u8(n), _host_u8(n), k_splits)
    assert_bits_equal(bits_of(c), oracle.splitk_reduce(planes), "fp4 splitk")
    assert not ws.cpu().numpy().view(np.uint32).any()


@pytest.mark.parametrize("scale_2", [0.5, -3.0])
@pytest.mark.parametrize("m,n", SHAPES)
def test_w4a16_k_zero(m, n, scale_2):
    print(f"gemm_w4a16 K=0 {m}x{n} scale_2={scale_2}", flush=True)
    c = empty_bf16(m, n, FILL)
    bg.gemm_w4a16(_empty_bf16(m), _empty_u8(n), _empty_u8(n), scale_2, out=c)
    torch.cuda.synchronize()
    ref = oracle.gemm_w4a16_ref(_host_bf16(m), _host_u8(n), _host_u8(n), scale_2)
    assert_bits_equal(bits_of(c), _bf16_of(ref), "w4a16")
