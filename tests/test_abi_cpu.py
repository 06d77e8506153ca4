"""C-ABI checks that need no GPU: the library loads, exports every function
include/blockgemm.h declares, and rejects bad arguments before touching the
device.

Fake device addresses are used only with arguments that fail validation, so no
kernel is ever launched on them; the single valid-argument call is skipped when
a GPU is present.
"""
import ctypes
import os
import re

import pytest
import torch

import block_scaled_fp4_gemm_amd as bg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blockgemm.h")

# fake, 16-byte aligned, far-apart addresses (never dereferenced)
A, B, C, W, S1, S2 = (0x10000000 * i for i in range(1, 7))


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"if", "sizeof"})


def test_header_and_binding_agree():
    names = declared_functions()
    assert set(names) == set(bg.EXPORTS)


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports_symbol(name):
    lib = ctypes.CDLL(bg._LIB_PATH)
    assert hasattr(lib, name)


def test_status_strings():
    for s in range(8):
        assert bg.bg_status_string(s)
    assert bg.bg_status_string(99) == "unknown status"


def test_workspace_bytes():
    assert bg.gemm_bf16_splitk_workspace_bytes(5120, 2048, 8) == 8 * 5120 * 2048 * 4
    assert bg.gemm_bf16_splitk_workspace_bytes(0, 7, 3) == 0


def test_empty_problems_are_ok_without_pointers():
    L = bg.lib
    assert L.gemm_bf16(None, None, None, 0, 5, 7, None) == bg.BG_OK
    assert L.gemm_bf16(None, None, None, 5, 0, 7, None) == bg.BG_OK
    assert L.gemm_bf16_strided(None, 9, None, 9, None, 3, 0, 3, 7, None) == bg.BG_OK
    assert L.gemm_bf16_scaled_acc(None, None, None, 0, 0, 0, 1.0, None) == bg.BG_OK
    assert L.gemm_bf16_ordered(None, None, None, 0, 3, 3, None) == bg.BG_OK
    assert L.gemm_fp4_blockscaled(None, None, None, None, None, 0, 4, 32, None) == bg.BG_OK
    assert L.gemm_w4a16(None, None, None, 1.0, None, 3, 0, 32, None) == bg.BG_OK
    assert L.gemm_fp4_blockscaled_batched(None, None, None, None, None, 4, 4, 32, 0, None) == bg.BG_OK
    assert L.gemm_fp4_blockscaled_splitk(None, None, None, None, None, None, 0, 0, 4, 32, 4, None) == bg.BG_OK
    assert L.fp4_scales_from_blocked(None, None, 128, 4, 0, None) == bg.BG_OK
    assert L.bf16_scaled_add(None, None, 0, 1.0, None) == bg.BG_OK
    assert L.gemm_bf16_splitk(None, None, None, None, 0, 0, 4, 64, 4, None) == bg.BG_OK
    assert L.gemm_bf16_dual(None, None, None, None, None, 0, 4, 64, None) == bg.BG_OK


def test_null_pointers():
    L = bg.lib
    assert L.gemm_bf16(None, B, C, 4, 4, 4, None) == bg.BG_ERR_NULL
    assert L.gemm_bf16(A, None, C, 4, 4, 4, None) == bg.BG_ERR_NULL
    assert L.gemm_bf16(A, B, None, 4, 4, 4, None) == bg.BG_ERR_NULL
    assert L.gemm_bf16_strided(A, 8, B, 8, None, 8, 4, 4, 4, None) == bg.BG_ERR_NULL
    assert L.gemm_bf16_ordered_f32(A, B, None, 4, 4, 4, None) == bg.BG_ERR_NULL
    assert L.gemm_fp4_blockscaled(A, None, B, S2, C, 4, 4, 32, None) == bg.BG_ERR_NULL
    assert L.gemm_w4a16(A, B, None, 1.0, C, 4, 4, 32, None) == bg.BG_ERR_NULL
    assert L.gemm_w4a16(None, B, S2, 1.0, C, 4, 4, 32, None) == bg.BG_ERR_NULL
    assert L.gemm_fp4_blockscaled_batched(A, S1, B, None, C, 4, 4, 32, 2, None) == bg.BG_ERR_NULL
    assert L.fp4_scales_from_blocked(S1, None, 128, 4, 1, None) == bg.BG_ERR_NULL
    assert L.bf16_scaled_add(None, B, 8, 1.0, None) == bg.BG_ERR_NULL
    assert L.gemm_bf16_dual(A, B, None, C, W, 4, 4, 8, None) == bg.BG_ERR_NULL
    assert L.gemm_bf16_dual(A, B, S1, C, None, 4, 4, 8, None) == bg.BG_ERR_NULL


def test_misaligned_pointers():
    L = bg.lib
    assert L.gemm_bf16(A + 2, B, C, 4, 4, 8, None) == bg.BG_ERR_ALIGN
    assert L.gemm_bf16(A, B, C + 8, 4, 4, 8, None) == bg.BG_ERR_ALIGN
    assert L.gemm_bf16_strided(A, 9, B + 2, 9, C, 4, 4, 4, 8, None) == bg.BG_ERR_ALIGN
    assert L.gemm_bf16_scaled_acc(A, B + 4, C, 4, 4, 8, 2.0, None) == bg.BG_ERR_ALIGN
    assert L.gemm_fp4_blockscaled(A, S1 + 1, B, S2, C, 4, 4, 32, None) == bg.BG_ERR_ALIGN
    assert L.gemm_w4a16(A, B + 8, S2, 1.0, C, 4, 4, 32, None) == bg.BG_ERR_ALIGN
    assert L.gemm_w4a16(A, B, S2, 1.0, C + 2, 4, 4, 32, None) == bg.BG_ERR_ALIGN
    assert L.fp4_scales_from_blocked(S1 + 4, S2, 128, 4, 1, None) == bg.BG_ERR_ALIGN
    assert L.gemm_fp4_blockscaled_splitk(A, S1, B, S2, C, W + 4, 1 << 20, 4, 4, 128, 2, None) == bg.BG_ERR_ALIGN
    assert L.gemm_bf16_splitk(A, B, C, W + 4, 1 << 20, 4, 4, 128, 2, None) == bg.BG_ERR_ALIGN
    assert L.gemm_bf16_dual(A, B, S1 + 2, C, W, 4, 4, 8, None) == bg.BG_ERR_ALIGN
    assert L.gemm_bf16_dual(A, B, S1, C, W + 8, 4, 4, 8, None) == bg.BG_ERR_ALIGN


def test_aliasing_outputs():
    L = bg.lib
    # C overlaps A
    assert L.gemm_bf16(A, B, A + 16, 4, 4, 64, None) == bg.BG_ERR_ALIAS
    # out overlaps B
    assert L.gemm_bf16_scaled_acc(A, B, B, 4, 4, 64, 2.0, None) == bg.BG_ERR_ALIAS
    # strided C spans (M-1)*ldc + N elements; the B operand lies inside that span
    assert L.gemm_bf16_strided(A, 64, B - 4 * 100 * 2 + 16, 64, B - 4 * 100 * 2, 100, 5, 4, 64, None) == bg.BG_ERR_ALIAS
    # split-K workspace overlaps C
    assert L.gemm_bf16_splitk(A, B, C, C, 1 << 20, 4, 4, 128, 2, None) == bg.BG_ERR_ALIAS
    # FP4 C overlaps a scale tensor
    assert L.gemm_fp4_blockscaled(A, S1, B, S2, S1, 4, 4, 32, None) == bg.BG_ERR_ALIAS
    # W4A16 C overlaps the activations or the weight scales
    assert L.gemm_w4a16(A, B, S2, 1.0, A + 64, 4, 4, 32, None) == bg.BG_ERR_ALIAS
    assert L.gemm_w4a16(A, B, S2, 1.0, S2, 4, 4, 32, None) == bg.BG_ERR_ALIAS
    # batched: the second problem's C (C + 4*4*2) runs into SFB placed right after the first
    assert L.gemm_fp4_blockscaled_batched(A, S1, B, C + 32, C, 4, 4, 32, 2, None) == bg.BG_ERR_ALIAS
    assert L.gemm_fp4_blockscaled_splitk(A, S1, B, S2, C, C, 1 << 20, 4, 4, 128, 2, None) == bg.BG_ERR_ALIAS
    assert L.fp4_scales_from_blocked(S1, S1 + 256, 128, 4, 1, None) == bg.BG_ERR_ALIAS
    assert L.bf16_scaled_add(A, A + 16, 64, 1.0, None) == bg.BG_ERR_ALIAS
    # dual: the two outputs overlap each other, or one output overlaps the other product's weights
    assert L.gemm_bf16_dual(A, B, S1, C, C + 16, 4, 4, 64, None) == bg.BG_ERR_ALIAS
    assert L.gemm_bf16_dual(A, B, S1, S1 + 16, W, 4, 4, 64, None) == bg.BG_ERR_ALIAS
    assert L.gemm_bf16_dual(A, B, S1, C, B, 4, 4, 64, None) == bg.BG_ERR_ALIAS
    # adjacent but disjoint ranges are fine up to the device check
    if torch.cuda.device_count() == 0:
        assert L.gemm_bf16(A, A + 4 * 64 * 2, A + 2 * 4 * 64 * 2, 4, 4, 64, None) == bg.BG_ERR_DEVICE


def test_shape_rules():
    L = bg.lib
    # transposed W4A16: N <= ldb, K % 16 == 0
    assert L.gemm_w4a16_t(A, B, S2, 9, 1.0, C, 4, 10, 32, None) == bg.BG_ERR_SHAPE
    assert L.gemm_w4a16_t(A, B, S2, 10, 1.0, C, 4, 10, 40, None) == bg.BG_ERR_SHAPE
    assert L.gemm_w4a16_t(A, B, S2, 1 << 31, 1.0, C, 4, 10, 32, None) == bg.BG_ERR_SHAPE
    assert L.gemm_w4a16_t(A, None, S2, 11, 1.0, C, 4, 10, 32, None) == bg.BG_ERR_NULL
    assert L.gemm_w4a16_t(A, B + 4, S2, 11, 1.0, C, 4, 10, 32, None) == bg.BG_ERR_ALIGN
    # C overlaps the last scale row: SFBt spans (K/16) * ldb bytes
    assert L.gemm_w4a16_t(A, B, S2, 11, 1.0, S2 + 16, 4, 10, 32, None) == bg.BG_ERR_ALIAS
    assert L.gemm_w4a16_t(None, None, None, 5, 1.0, None, 0, 5, 32, None) == bg.BG_OK
    assert L.gemm_fp4_blockscaled(A, S1, B, S2, C, 4, 4, 40, None) == bg.BG_ERR_SHAPE   # K % 16
    assert L.gemm_w4a16(A, B, S2, 1.0, C, 4, 4, 40, None) == bg.BG_ERR_SHAPE             # K % 16
    assert L.gemm_w4a16(A, B, S2, 1.0, C, 4, 1 << 31, 32, None) == bg.BG_ERR_SHAPE
    assert L.gemm_fp4_blockscaled_batched(A, S1, B, S2, C, 4, 4, 40, 2, None) == bg.BG_ERR_SHAPE
    assert L.gemm_fp4_blockscaled_batched(A, S1, B, S2, C, 4, 4, 32, 70000, None) == bg.BG_ERR_SHAPE
    assert L.gemm_fp4_blockscaled_splitk(A, S1, B, S2, C, W, 1 << 20, 4, 4, 40, 2, None) == bg.BG_ERR_SHAPE
    assert L.gemm_fp4_blockscaled_splitk(A, S1, B, S2, C, W, 1 << 20, 4, 4, 32, 0, None) == bg.BG_ERR_SHAPE
    assert L.fp4_scales_from_blocked(S1, S2, 100, 4, 1, None) == bg.BG_ERR_SHAPE      # rows % 128
    assert L.fp4_scales_from_blocked(S1, S2, 128, 6, 1, None) == bg.BG_ERR_SHAPE      # k_groups % 4
    assert L.gemm_bf16_splitk(A, B, C, W, 1 << 30, 4, 4, 128, 0, None) == bg.BG_ERR_SHAPE
    assert L.gemm_bf16_splitk(A, B, C, W, 1 << 30, 4, 4, 128, 65, None) == bg.BG_ERR_SHAPE
    assert L.gemm_bf16(A, B, C, 1 << 31, 4, 4, None) == bg.BG_ERR_SHAPE
    assert L.gemm_bf16_dual(A, B, S1, C, W, 4, 1 << 31, 4, None) == bg.BG_ERR_SHAPE
    assert L.gemm_bf16_strided(A, 7, B, 8, C, 4, 4, 4, 8, None) == bg.BG_ERR_SHAPE    # lda < K
    assert L.gemm_bf16_strided(A, 8, B, 7, C, 4, 4, 4, 8, None) == bg.BG_ERR_SHAPE    # ldb < K
    assert L.gemm_bf16_strided(A, 8, B, 8, C, 3, 4, 4, 8, None) == bg.BG_ERR_SHAPE    # ldc < N
    assert L.gemm_bf16_strided(A, 1 << 31, B, 8, C, 4, 4, 4, 8, None) == bg.BG_ERR_SHAPE


def test_workspace_rules():
    L = bg.lib
    # the allocation-free split-K: k_splits * M * N * 4 must fit the 32 MiB scratch
    assert L.gemm_bf16_splitk_noalloc(A, B, C, 1024, 2048, 256, 5, None) == bg.BG_ERR_WORKSPACE
    assert L.gemm_bf16_splitk_noalloc(A, B, C, 1024, 2048, 256, 0, None) == bg.BG_ERR_SHAPE
    assert L.gemm_bf16_splitk_noalloc(A, B, C, 1024, 2048, 256, 65, None) == bg.BG_ERR_SHAPE
    assert L.gemm_bf16_splitk_noalloc(A, B, None, 4, 4, 8, 2, None) == bg.BG_ERR_NULL
    assert L.gemm_bf16_splitk_noalloc(A, B, A + 16, 4, 4, 64, 2, None) == bg.BG_ERR_ALIAS
    assert L.gemm_bf16_splitk_noalloc(None, None, None, 0, 4, 64, 2, None) == bg.BG_OK
    need = 2 * 4 * 4 * 4
    assert L.gemm_bf16_splitk(A, B, C, None, need, 4, 4, 128, 2, None) == bg.BG_ERR_WORKSPACE
    assert L.gemm_bf16_splitk(A, B, C, W, need - 1, 4, 4, 128, 2, None) == bg.BG_ERR_WORKSPACE
    assert L.gemm_fp4_blockscaled_splitk(A, S1, B, S2, C, W, need - 1, 4, 4, 128, 2, None) == bg.BG_ERR_WORKSPACE
    assert L.gemm_fp4_blockscaled_splitk(A, S1, B, S2, C, None, need, 4, 4, 128, 2, None) == bg.BG_ERR_WORKSPACE


def test_streamk_argument_rules():
    L = bg.lib
    assert L.gemm_bf16_streamk(None, None, None, None, 0, 0, 4, 64, None) == bg.BG_OK
    assert L.gemm_bf16_streamk(None, None, None, None, 0, 4, 0, 64, None) == bg.BG_OK
    assert L.gemm_bf16_streamk(A, B, None, W, 1 << 20, 4, 4, 64, None) == bg.BG_ERR_NULL
    assert L.gemm_bf16_streamk(A, B, A + 16, W, 1 << 20, 4, 4, 64, None) == bg.BG_ERR_ALIAS
    assert L.gemm_bf16_streamk(A + 2, B, C, W, 1 << 20, 4, 4, 64, None) == bg.BG_ERR_ALIGN
    # the stream-K kernel takes K % 8 == 0: it needs a workspace, 16-byte aligned
    assert L.gemm_bf16_streamk(A, B, C, None, 1 << 20, 4, 4, 64, None) == bg.BG_ERR_WORKSPACE
    assert L.gemm_bf16_streamk(A, B, C, W + 8, 1 << 20, 4, 4, 64, None) == bg.BG_ERR_ALIGN
    assert L.gemm_bf16_streamk(A, B, C, None, 0, 4, 4, 2 ** 32 - 1, None) == bg.BG_ERR_SHAPE
    n = ctypes.c_size_t(7)
    assert L.gemm_bf16_streamk_workspace(4, 4, 64, None) == bg.BG_ERR_NULL
    assert L.gemm_bf16_streamk_workspace(4, 4, 2 ** 32 - 1, ctypes.byref(n)) == bg.BG_ERR_SHAPE
    rows = ctypes.c_size_t(0)
    assert L.bg_streamk_plan(160, 32, 32, None, 0, None) == bg.BG_ERR_NULL
    assert L.bg_streamk_plan(160, 32, 0, None, 0, ctypes.byref(rows)) == bg.BG_ERR_SHAPE
    assert L.bg_streamk_plan(160, 32, 32, None, 0, ctypes.byref(rows)) == bg.BG_OK and rows.value == 384
    buf = (ctypes.c_int32 * 6)()
    assert L.bg_streamk_plan(160, 32, 32, buf, 1, ctypes.byref(rows)) == bg.BG_ERR_WORKSPACE


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="valid call would launch on fake pointers")
def test_valid_arguments_reach_the_device_check():
    L = bg.lib
    assert L.gemm_bf16(A, B, C, 4, 4, 8, None) == bg.BG_ERR_DEVICE
    assert L.gemm_bf16_splitk(A, B, C, None, 0, 4, 4, 8, 1, None) == bg.BG_ERR_DEVICE
    assert L.gemm_w4a16(A, B, S2, 0.5, C, 4, 4, 32, None) == bg.BG_ERR_DEVICE
    assert L.gemm_bf16_strided(A, 13, B, 8, C, 5, 4, 4, 8, None) == bg.BG_ERR_DEVICE
    assert L.gemm_bf16_dual(A, B, S1, C, W, 4, 4, 8, None) == bg.BG_ERR_DEVICE
    assert L.gemm_w4a16_t(A, B, S2, 248077, 0.5, C, 4, 248077, 32, None) == bg.BG_ERR_DEVICE
    assert L.gemm_bf16_splitk_noalloc(A, B, C, 1024, 2048, 256, 4, None) == bg.BG_ERR_DEVICE
    assert L.gemm_bf16_streamk(A, B, C, W, 1 << 20, 4, 4, 64, None) == bg.BG_ERR_DEVICE
    assert L.gemm_bf16_streamk(A, B, C, None, 0, 4, 4, 100, None) == bg.BG_ERR_DEVICE
    n = ctypes.c_size_t(0)
    assert L.gemm_bf16_streamk_workspace(5120, 512, 2048, ctypes.byref(n)) == bg.BG_ERR_DEVICE


def test_python_binding_raises_on_status():
    with pytest.raises(bg.BlockGemmError) as e:
        bg._check(bg.BG_ERR_SHAPE, "x")
    assert e.value.status == bg.BG_ERR_SHAPE
