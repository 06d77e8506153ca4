"""Pins for the oracle's number-format codecs (CPU only).

Each codec is checked against something other than itself: the textbook
format tables under tests/golden/ and torch's own dtype conversions.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden
import oracle
from oracle import codecs


def test_e2m1_matches_ocp_table():
    rows = [ln.split() for ln in read_golden("e2m1_table.txt")]
    assert len(rows) == 16
    codes = np.array([int(r[0]) for r in rows])
    want = np.array([float(r[1]) for r in rows])
    got = oracle.e2m1_to_f64(codes)
    assert np.array_equal(got, want)
    # sign of zero: code 8 is -0.0
    assert math.copysign(1.0, got[8]) == -1.0 and math.copysign(1.0, got[0]) == 1.0


def test_e4m3fn_pins():
    for ln in read_golden("e4m3fn_pins.txt"):
        byte_s, val_s = ln.split()
        got = float(oracle.e4m3fn_to_f64(np.array([int(byte_s, 16)]))[0])
        if val_s == "nan":
            assert math.isnan(got), byte_s
        else:
            assert got == float(val_s) and math.copysign(1, got) == math.copysign(1, float(val_s)), byte_s


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_bf16_rne_vectors():
    for ln in read_golden("bf16_rne.txt"):
        src, want = (int(t, 16) for t in ln.split())
        f = np.array([src], dtype=np.uint32).view(np.float32)
        got = int(oracle.f32_to_bf16(f)[0])
        assert got == want, f"{src:#010x}: got {got:#06x} want {want:#06x}"


def test_bf16_rne_matches_torch_on_random_and_ties():
    g = np.random.default_rng(12345)
    bits = g.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # force a third of them onto exact ties and near-ties
    bits[::3] = (bits[::3] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    bits[1::3] = (bits[1::3] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    f = bits.view(np.float32)
    finite = np.isfinite(f)
    ref = torch.from_numpy(f[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(f[finite])
    assert np.array_equal(ref, got)
    # NaNs stay NaN with their sign
    nan_out = oracle.bf16_to_f32(oracle.f32_to_bf16(f[np.isnan(f)]))
    assert np.all(np.isnan(nan_out))
    assert np.array_equal(np.signbit(nan_out), np.signbit(f[np.isnan(f)]))


def test_bf16_widening_is_exact():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.bf16_to_f32(bits)
    same = (ref.view(np.uint32) == got.view(np.uint32)) | (np.isnan(ref) & np.isnan(got))
    assert same.all()
    # round trip of every non-NaN pattern is the identity
    nn = ~np.isnan(got)
    assert np.array_equal(oracle.f32_to_bf16(got[nn]), bits[nn])


def test_unpack_low_nibble_is_even_k():
    packed = np.array([[0x21, 0xF0, 0x8A]], dtype=np.uint8)
    assert oracle.unpack_e2m1(packed).tolist() == [[1, 2, 0, 15, 10, 8]]


def _table():
    return {int(r.split()[0]): Fraction(r.split()[1]) for r in read_golden("e2m1_table.txt")}


def test_dequant_group_index_brute_force():
    """Element [i,k] = table[code] * scale[i, k//16], checked by plain loops."""
    tab = _table()
    g = np.random.default_rng(7)
    rows, k = 3, 64
    packed = g.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    # distinct scales per group so a wrong group index shows up
    scales = np.array([[0x30, 0x38, 0x40, 0x48], [0x18, 0x58, 0x3C, 0x44], [0x7E, 0x01, 0x38, 0xB8]], dtype=np.uint8)
    sc_val = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.dequant_fp4(packed, scales)
    for i in range(rows):
        for kk in range(k):
            byte = int(packed[i, kk // 2])
            code = (byte & 0xF) if kk % 2 == 0 else (byte >> 4)
            want = float(tab[code]) * sc_val[i, kk // 16]
            assert got[i, kk] == want, (i, kk)


def test_e2m1_times_e4m3_is_exact_in_bf16():
    """Every dequantized value fits BF16 exactly (<= 6 significant bits)."""
    codes = np.arange(16)
    scales = np.arange(256, dtype=np.uint8)
    sv = oracle.e4m3fn_to_f64(scales)
    sv = sv[np.isfinite(sv)]
    prod = (oracle.e2m1_to_f64(codes)[:, None] * sv[None, :]).astype(np.float64).ravel()
    as_bf16 = oracle.bf16_to_f64(oracle.f32_to_bf16(prod.astype(np.float32)))
    assert np.array_equal(prod, as_bf16)


def test_oracle_does_not_import_the_library():
    src = open(codecs.__file__).read() + open(oracle.gemm.__file__).read()
    assert "block_scaled_fp4_gemm_amd" not in src


# NVIDIA blocked scale layout (kernelbot NVFP4 page, "SCALE FACTORS")

@pytest.mark.parametrize("rows,k_groups,batch", [(128, 4, 1), (256, 12, 1), (384, 8, 3)])
def test_scales_from_blocked_matches_grouped_reshape(rows, k_groups, batch):
    """The element loop equals the page's grouping
    'g_m i_m tile_m i_k tile_k l -> (tile_m i_m g_m) (tile_k i_k) l' applied to
    the stored order (l, tile_m, tile_k, g_m, i_m, i_k) by reshape/transpose."""
    rng = np.random.default_rng(rows + k_groups + batch)
    flat = rng.integers(0, 256, size=batch * rows * k_groups, dtype=np.uint8)
    tm, tk = rows // 128, k_groups // 4
    stored = flat.reshape(batch, tm, tk, 32, 4, 4)             # l tile_m tile_k g_m i_m i_k
    grouped = stored.transpose(0, 1, 4, 3, 2, 5).reshape(batch, rows, k_groups)
    assert np.array_equal(oracle.scales_from_blocked(flat, rows, k_groups, batch), grouped)


def test_scales_from_blocked_closed_form_positions():
    """One 128 x 4 block whose bytes hold their own offset g_m*16 + i_m*4 + i_k:
    plain[i, j] = (i % 32)*16 + (i // 32)*4 + j, from i = i_m*32 + g_m, j = i_k."""
    flat = np.arange(512, dtype=np.int64).astype(np.uint8)     # offsets mod 256
    got = oracle.scales_from_blocked(flat, 128, 4, 1)[0]
    i = np.arange(128)[:, None]
    j = np.arange(4)[None, :]
    assert np.array_equal(got, ((i % 32) * 16 + (i // 32) * 4 + j).astype(np.uint8))
