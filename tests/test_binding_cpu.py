"""The Python binding's argument checks and the host-side helpers (CPU only).

Every wrapper must reject what the pointer-only C ABI cannot see (tensor kind,
element size, operand and output shapes, host tensors) before the library is
called. The library is replaced by a stub that fails the test if any entry
point is reached, so nothing here can launch a kernel.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg


class _NoLib:
    def __getattr__(self, name):
        def called(*a, **k):
            raise AssertionError(f"library entry point {name} was called")
        return called


@pytest.fixture
def nolib(monkeypatch):
    monkeypatch.setattr(bg, "lib", _NoLib())


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


BAD_SHAPES = [
    # (call, exception)
    (lambda: bg.gemm_bf16(bf(4, 8), bf(5, 9)), ValueError),                       # K mismatch
    (lambda: bg.gemm_bf16(bf(4, 8), bf(5, 8), out=bf(4, 6)), ValueError),         # out shape
    (lambda: bg.gemm_bf16(bf(4, 8), bf(5, 8), out=torch.zeros(4, 5)), TypeError),  # out dtype
    (lambda: bg.gemm_bf16(torch.zeros(4, 8), bf(5, 8)), TypeError),               # A dtype
    (lambda: bg.gemm_bf16(bf(4, 8, 1), bf(5, 8)), ValueError),                    # A rank
    (lambda: bg.gemm_bf16_dual(bf(4, 8), bf(5, 8), bf(6, 8)), ValueError),
    (lambda: bg.gemm_bf16_dual(bf(4, 8), bf(5, 8), bf(5, 8), out1=bf(5, 4)), ValueError),
    (lambda: bg.gemm_bf16_scaled_acc(bf(4, 8), bf(5, 8), bf(4, 4), 2.0), ValueError),
    (lambda: bg.gemm_bf16_scaled_acc(bf(4, 8), bf(5, 7), bf(4, 5), 2.0), ValueError),
    (lambda: bg.gemm_bf16_splitk(bf(4, 8), bf(5, 8), 2, workspace=torch.zeros(2 * 4 * 5 - 1)), ValueError),
    (lambda: bg.gemm_bf16_splitk(bf(4, 8), bf(5, 8), 2, workspace=torch.zeros(40, dtype=torch.float64)),
     TypeError),
    (lambda: bg.gemm_bf16_splitk(bf(4, 8), bf(5, 8), 2, out=bf(5, 4)), ValueError),
    (lambda: bg.gemm_bf16_ordered(bf(4, 8), bf(5, 8), out=bf(4, 4)), ValueError),
    (lambda: bg.gemm_bf16_ordered_f32(bf(4, 8), bf(5, 8), out=bf(4, 5)), TypeError),
    (lambda: bg.gemm_bf16_strided(bf(4, 8), bf(5, 8), bf(4, 4)), ValueError),
    (lambda: bg.gemm_fp4_blockscaled(u8(4, 16), u8(4, 2), u8(5, 16), u8(5, 3)), ValueError),     # SFB
    (lambda: bg.gemm_fp4_blockscaled(u8(4, 16), u8(4, 1), u8(5, 16), u8(5, 2)), ValueError),     # SFA
    (lambda: bg.gemm_fp4_blockscaled(u8(4, 16), u8(4, 2), u8(5, 12), u8(5, 2)), ValueError),     # B
    (lambda: bg.gemm_fp4_blockscaled(u8(4, 12), u8(4, 1), u8(5, 12), u8(5, 1)), ValueError),     # K % 16
    (lambda: bg.gemm_fp4_blockscaled(bf(4, 16), u8(4, 2), u8(5, 16), u8(5, 2)), TypeError),
    (lambda: bg.gemm_fp4_blockscaled(u8(4, 16), u8(4, 2), u8(5, 16), u8(5, 2), out=bf(5, 4)), ValueError),
    (lambda: bg.gemm_fp4_blockscaled_batched(u8(2, 4, 16), u8(2, 4, 2), u8(3, 5, 16), u8(3, 5, 2)), ValueError),
    (lambda: bg.gemm_fp4_blockscaled_batched(u8(4, 16), u8(4, 2), u8(5, 16), u8(5, 2)), ValueError),
    (lambda: bg.gemm_fp4_blockscaled_splitk(u8(4, 16), u8(4, 2), u8(5, 16), u8(5, 2), 4,
                                            workspace=torch.zeros(4 * 4 * 5 - 1)), ValueError),
    (lambda: bg.fp4_scales_from_blocked(u8(128 * 4 - 1), 128, 4), ValueError),
    (lambda: bg.fp4_scales_from_blocked(u8(128 * 4), 128, 4, out=u8(1, 128, 5)), ValueError),
    (lambda: bg.gemm_w4a16(bf(4, 32), u8(5, 15), u8(5, 2), 1.0), ValueError),
    (lambda: bg.gemm_w4a16(bf(4, 32), u8(5, 16), u8(5, 3), 1.0), ValueError),
    (lambda: bg.gemm_w4a16(bf(4, 24), u8(5, 12), u8(5, 1), 1.0), ValueError),                   # K % 16
    (lambda: bg.gemm_w4a16(bf(4, 32), u8(5, 16), u8(5, 2), 1.0, out=bf(4, 4)), ValueError),
    (lambda: bg.gemm_w4a16_t(bf(4, 32), u8(16, 9), u8(2, 9), 10, 1.0), ValueError),        # ldb < N
    (lambda: bg.gemm_w4a16_t(bf(4, 32), u8(15, 11), u8(2, 11), 10, 1.0), ValueError),      # K/2 rows
    (lambda: bg.gemm_w4a16_t(bf(4, 32), u8(16, 11), u8(2, 10), 10, 1.0), ValueError),      # SFBt
    (lambda: bg.bf16_scaled_add(bf(8), bf(9), 1.0), ValueError),
    (lambda: bg.bf16_scaled_add(bf(8), torch.zeros(8), 1.0), TypeError),
]


@pytest.mark.parametrize("i", range(len(BAD_SHAPES)))
def test_bad_arguments_raise_before_the_library(i, nolib):
    call, exc = BAD_SHAPES[i]
    with pytest.raises(exc):
        call()


GOOD_HOST = [
    lambda: bg.gemm_bf16(bf(4, 8), bf(5, 8)),
    lambda: bg.gemm_bf16_dual(bf(4, 8), bf(5, 8), bf(5, 8)),
    lambda: bg.gemm_bf16_scaled_acc(bf(4, 8), bf(5, 8), bf(4, 5), 2.0),
    lambda: bg.gemm_bf16_splitk(bf(4, 8), bf(5, 8), 2),
    lambda: bg.gemm_bf16_ordered(bf(4, 8), bf(5, 8)),
    lambda: bg.gemm_bf16_ordered_f32(bf(4, 8), bf(5, 8)),
    lambda: bg.gemm_bf16_strided(bf(4, 8), bf(5, 8), bf(4, 5)),
    lambda: bg.gemm_fp4_blockscaled(u8(4, 16), u8(4, 2), u8(5, 16), u8(5, 2)),
    lambda: bg.gemm_fp4_blockscaled_batched(u8(2, 4, 16), u8(2, 4, 2), u8(2, 5, 16), u8(2, 5, 2)),
    lambda: bg.gemm_fp4_blockscaled_splitk(u8(4, 16), u8(4, 2), u8(5, 16), u8(5, 2), 2),
    lambda: bg.fp4_scales_from_blocked(u8(128 * 4), 128, 4),
    lambda: bg.gemm_w4a16(bf(4, 32), u8(5, 16), u8(5, 2), 1.0),
    lambda: bg.bf16_scaled_add(bf(8), bf(8), 1.0),
    lambda: bg.gemm_w4a16_t(bf(4, 32), u8(16, 11), u8(2, 11), 10, 1.0),
]


@pytest.mark.parametrize("i", range(len(GOOD_HOST)))
def test_host_tensors_are_rejected(i, nolib):
    """Well-shaped operands in host memory: the device check in the binding
    raises before any pointer reaches the library."""
    with pytest.raises(ValueError, match="device"):
        GOOD_HOST[i]()


def test_tuning_overrides_set_get_reset():
    for key in range(7):
        assert bg.tune_get(key) == -1
    with bg.tuned(bg.TUNE_TILE, 3):
        assert bg.tune_get(bg.TUNE_TILE) == 3
        with bg.tuned(bg.TUNE_TILE, 1):
            assert bg.tune_get(bg.TUNE_TILE) == 1
        assert bg.tune_get(bg.TUNE_TILE) == 3
    assert bg.tune_get(bg.TUNE_TILE) == -1
    with pytest.raises(bg.BlockGemmError):
        bg.tune_set(7, 0)
    with pytest.raises(bg.BlockGemmError):
        bg.tune_set(bg.TUNE_TILE, -2)
    assert bg.tune_get(99) == -1


def test_tuning_is_not_read_from_the_environment(monkeypatch):
    monkeypatch.setenv("BLOCKGEMM_TILE", "3")
    assert bg.tune_get(bg.TUNE_TILE) == -1
