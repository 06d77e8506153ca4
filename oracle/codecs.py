"""Number-format definitions used by the oracle (test infrastructure only).

Plain textbook definitions, written out on bit fields with numpy. Nothing here
is shared with, or imported by, the HIP library.

  - BF16: the upper 16 bits of an IEEE binary32; narrowing rounds to nearest,
    ties to even.  The pages never state the rounding mode of their FP32 -> BF16
    casts (sm121a_matmul.py page, the accumulator cast at the end of the kernel;
    gemm_dense.rs page, "bf16(...)" in the dense_gemm_tc_scaled_acc doc); this
    oracle reads it as round-to-nearest-even with NaN kept NaN.
  - E2M1 (FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit, no Inf/NaN
    (OCP Microscaling Formats v1.0, FP4 element type).  Two codes per byte; the
    kernelbot NVFP4 page packs K as K/2 bytes without naming the nibble order,
    and this oracle reads the low nibble as the even K element.
  - E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, NaN = S.1111.111,
    no Inf (OCP 8-bit floating point v1.0).  The kernelbot NVFP4 page's
    custom_kernel docstring prints the scale dtype as float8_e4m3fnuz; the
    NVFP4 format it implements uses E4M3FN, which is the reading taken here.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening: BF16 bits become the high half of an FP32 pattern."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def f32_to_bf16(x) -> np.ndarray:
    """FP32 -> BF16 bits, round to nearest, ties to even; NaN -> quiet NaN, same sign."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    is_nan = np.isnan(f)
    quiet = ((u >> np.uint64(16)).astype(np.uint32) | np.uint32(0x0040))
    out = np.where(is_nan, quiet, rounded) & np.uint32(0xFFFF)
    return out.astype(np.uint16)


def e2m1_to_f64(codes) -> np.ndarray:
    """Value of 4-bit E2M1 codes: s = bit3, e = bits 2..1, m = bit0.

    e == 0: (-1)^s * m * 0.5 ; else (-1)^s * (1 + m/2) * 2^(e-1).
    """
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m * 0.5) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def e4m3fn_to_f64(b) -> np.ndarray:
    """Value of E4M3FN bytes: s = bit7, e = bits 6..3, m = bits 2..0, bias 7.

    e == 0: (-1)^s * m * 2^-9 ; e == 15 and m == 7: NaN ;
    else (-1)^s * (1 + m/8) * 2^(e-7).
    """
    v = np.asarray(b, dtype=np.int64)
    s = (v >> 7) & 1
    e = (v >> 3) & 15
    m = v & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def unpack_e2m1(packed) -> np.ndarray:
    """[R, K/2] bytes -> [R, K] codes; element 2t is the low nibble of byte t."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequant_fp4(packed, scales) -> np.ndarray:
    """Block-scaled FP4 operand as exact FP64 values.

    Element [i, k] is e2m1(code[i, k]) * e4m3fn(scales[i, k // 16]): one scale per
    16 consecutive K elements of a row, in the plain [rows, K/16] layout (the
    kernelbot NVFP4 page, "SCALE FACTORS": scale[i, j // group_sz] with
    group_sz = 16, multiplied into A[i, j]).
    """
    codes = unpack_e2m1(packed)
    k = codes.shape[-1]
    sc = np.asarray(scales, dtype=np.uint8)
    assert sc.shape[-1] * 16 == k, "one scale per 16 K elements"
    vals = e2m1_to_f64(codes)
    per_elem = np.repeat(e4m3fn_to_f64(sc), 16, axis=-1)
    return vals * per_elem


def scales_from_blocked(blocked, rows: int, k_groups: int, batch: int = 1) -> np.ndarray:
    """Plain [L, rows, K/16] E4M3 scale bytes from NVIDIA's blocked layout.

    kernelbot NVFP4 GEMM page, "SCALE FACTORS": the hardware layout has shape
    [32, 4, rest_m, 4, rest_k, L] (dims g_m, i_m, tile_m, i_k, tile_k, l) and
    is stored in memory in the order l, tile_m, tile_k, g_m, i_m, i_k. Plain
    row i = tile_m*128 + i_m*32 + g_m and group j = tile_k*4 + i_k. `blocked`
    is the flat byte buffer in that memory order; rows % 128 == 0 and
    k_groups % 4 == 0.
    """
    tm, tk = rows // 128, k_groups // 4
    assert tm * 128 == rows and tk * 4 == k_groups
    src = np.asarray(blocked, dtype=np.uint8).reshape(-1)
    assert src.size == batch * rows * k_groups
    out = np.empty((batch, rows, k_groups), np.uint8)
    pos = 0
    for l in range(batch):
        for tile_m in range(tm):
            for tile_k in range(tk):
                for g_m in range(32):
                    for i_m in range(4):
                        for i_k in range(4):
                            out[l, tile_m * 128 + i_m * 32 + g_m, tile_k * 4 + i_k] = src[pos]
                            pos += 1
    return out


def dequant_fp4_t(bt, sfbt, n: int) -> np.ndarray:
    """Weights stored transposed, as exact FP64 values in [n, K] (row j = weight row j).

    gemm_dense.rs page, doc comments of the `_ldb` W4A16 launchers: the
    transposed weight has one row per k pair at a row stride ldb >= N (pad
    columns unused). Byte (r, j) = bt[r, j] holds weight row j's codes for
    k = 2r (low nibble) and k = 2r + 1 (high nibble); the E4M3 scale of k in
    [16g, 16g + 16) of row j is sfbt[g, j].
    """
    b = np.asarray(bt, dtype=np.uint8)[:, :n]
    sf = np.asarray(sfbt, dtype=np.uint8)[:, :n]
    k = 2 * b.shape[0]
    assert sf.shape[0] * 16 == k, "one scale row per 16 K elements"
    codes = np.empty((k, n), dtype=np.uint8)
    codes[0::2] = b & 0x0F
    codes[1::2] = b >> 4
    vals = e2m1_to_f64(codes) * np.repeat(e4m3fn_to_f64(sf), 16, axis=0)
    return vals.T
