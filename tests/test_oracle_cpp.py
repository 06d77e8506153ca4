"""Pins for the plain C++17 oracle (oracle/cpu_oracle.cpp), CPU only.

The C++ oracle is pinned the same way as the numpy one, against things other
than itself: the textbook tables and hand-worked rounding cases under
tests/golden/, torch's dtype conversions, exact rational brute force, a
pure-Python IEEE-single emulation, and identities exact in any order. The two
oracles are written independently and are also compared with each other.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden
import oracle
from oracle import cpp
import synthetic
from test_oracle_gemm import _ordered_pure_python, _unfused_pure_python, bf16_exact, f32_bits, f32r, torch_bf16_bits


def _parse_row(s):
    return np.array([float(t) for t in s.split()], dtype=np.float32)


def _e2m1_table():
    return {int(r.split()[0]): Fraction(r.split()[1]) for r in read_golden("e2m1_table.txt")}


def test_library_builds_and_loads():
    cpp.build()
    assert cpp.hardware_threads() >= 1


# ---- codecs -----------------------------------------------------------------------

def test_e2m1_matches_ocp_table():
    rows = [ln.split() for ln in read_golden("e2m1_table.txt")]
    got = cpp.e2m1_to_f64(np.array([int(r[0]) for r in rows]))
    assert np.array_equal(got, np.array([float(r[1]) for r in rows]))
    assert math.copysign(1.0, got[8]) == -1.0


def test_e4m3fn_pins_and_all_codes_match_torch():
    for ln in read_golden("e4m3fn_pins.txt"):
        byte_s, val_s = ln.split()
        got = float(cpp.e4m3fn_to_f64(np.array([int(byte_s, 16)]))[0])
        if val_s == "nan":
            assert math.isnan(got), byte_s
        else:
            assert got == float(val_s) and math.copysign(1, got) == math.copysign(1, float(val_s)), byte_s
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = cpp.e4m3fn_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan]) and np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_bf16_rne_vectors_and_torch():
    for ln in read_golden("bf16_rne.txt"):
        src, want = (int(t, 16) for t in ln.split())
        got = int(cpp.f32_to_bf16(np.array([src], np.uint32).view(np.float32))[0])
        assert got == want, f"{src:#010x}: got {got:#06x} want {want:#06x}"
    g = np.random.default_rng(54321)
    bits = g.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    bits[::3] = (bits[::3] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    bits[1::3] = (bits[1::3] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    f = bits.view(np.float32)
    fin = np.isfinite(f)
    ref = torch.from_numpy(f[fin].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(cpp.f32_to_bf16(f[fin]), ref)
    nan_out = cpp.f32_to_bf16(f[np.isnan(f)])
    assert np.all((nan_out & 0x7F80) == 0x7F80) and np.all(nan_out & 0x7F)
    assert np.array_equal(nan_out >> 15, (f[np.isnan(f)].view(np.uint32) >> 31).astype(np.uint16))


def test_bf16_widening_is_exact():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    got = cpp.bf16_to_f32(bits)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))


def test_dequant_low_nibble_is_even_k_and_group_index():
    tab = _e2m1_table()
    k = 64
    packed = synthetic.fp4_packed(3, k, 7, 0)
    scales = synthetic.e4m3_uniform(3, k // 16, 2 ** -4, 2 ** 4, 7, 1)
    sv = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = cpp.dequant_fp4(packed, scales)
    for r in range(3):
        for kk in range(k):
            byte = int(packed[r, kk // 2])
            code = byte & 0xF if kk % 2 == 0 else byte >> 4
            assert Fraction(got[r, kk]) == tab[code] * Fraction(sv[r, kk // 16])


# ---- dense -----------------------------------------------------------------------------

@pytest.mark.parametrize("m,n,k", [(3, 5, 7), (1, 1, 1), (4, 2, 19)])
def test_dense_brute_force_exact_rationals(m, n, k):
    a = synthetic.normal_bf16((m, k), 1.0, 10 + k, 0)
    b = synthetic.normal_bf16((n, k), 0.5, 20 + k, 1)
    got = cpp.gemm_bf16_ref(a, b)
    for i in range(m):
        for j in range(n):
            exact = sum(bf16_exact(int(a[i, kk])) * bf16_exact(int(b[j, kk])) for kk in range(k))
            assert abs(Fraction(got[i, j]) - exact) <= Fraction(k) * Fraction(2) ** -52 * abs(exact) + Fraction(2) ** -1000


def test_dense_identity_permutation_and_exact_grid():
    a = synthetic.normal_bf16((6, 24), 1.0, 30, 0)
    eye = torch_bf16_bits(np.eye(24, dtype=np.float32))
    assert np.array_equal(cpp.gemm_bf16_ref(a, eye), oracle.bf16_to_f64(a))
    perm = np.random.default_rng(3).permutation(24)
    pm = torch_bf16_bits(np.eye(24, dtype=np.float32)[perm])
    assert np.array_equal(cpp.gemm_bf16_ref(a, pm), oracle.bf16_to_f64(a)[:, perm])
    x = synthetic.grid_bf16((16, 64), -8, 8, -5, 31, 0)
    w = synthetic.grid_bf16((12, 64), -8, 8, -5, 31, 1)
    xi = np.rint(oracle.bf16_to_f64(x) * 32).astype(np.int64)
    wi = np.rint(oracle.bf16_to_f64(w) * 32).astype(np.int64)
    assert np.array_equal(cpp.gemm_bf16_ref(x, w), (xi @ wi.T).astype(np.float64) / 1024.0)


def test_dense_rows_sample_equals_full_and_threads_do_not_change_results():
    a = synthetic.normal_bf16((37, 96), 1.0, 32, 0)
    b = synthetic.normal_bf16((29, 96), 0.02, 32, 1)
    full1 = cpp.gemm_bf16_ref(a, b, threads=1)
    full4 = cpp.gemm_bf16_ref(a, b, threads=4)
    assert np.array_equal(full1, full4)
    rows = np.array([0, 5, 36, 17])
    assert np.array_equal(cpp.gemm_bf16_ref_rows(a, b, rows, threads=3), full1[rows])


def test_dense_agrees_with_numpy_oracle():
    a = synthetic.normal_bf16((64, 320), 1.0, 33, 0)
    b = synthetic.normal_bf16((96, 320), 0.02, 33, 1)
    got, ref = cpp.gemm_bf16_ref(a, b), oracle.gemm_bf16_ref(a, b)
    bound = 320 * 2.0 ** -52 * (np.abs(oracle.bf16_to_f64(a)) @ np.abs(oracle.bf16_to_f64(b)).T)
    assert (np.abs(got - ref) <= 2 * bound).all()


# ---- ordered ------------------------------------------------------------------------

def test_ordered_worked_cases():
    for ln in read_golden("ordered_worked.txt"):
        fields = [f.strip() for f in ln.split(";")]
        name, arow, brow, want = fields[0], _parse_row(fields[1]), _parse_row(fields[2]), int(fields[3], 16)
        a = torch_bf16_bits(arow[None, :])
        b = torch_bf16_bits(brow[None, :])
        assert f32_bits(float(cpp.gemm_ordered_f32(a, b)[0, 0])) == want, name
        if name == "cancel":
            rev = cpp.gemm_ordered_f32(a[:, ::-1].copy(), b[:, ::-1].copy())
            assert f32_bits(float(rev[0, 0])) == 0x3F800000


@pytest.mark.parametrize("seed", [0, 1])
def test_ordered_matches_pure_python_ieee_single(seed):
    a = synthetic.normal_bf16((4, 37), 3.0, 100 + seed, 0)
    b = synthetic.normal_bf16((5, 37), 7.0, 200 + seed, 1)
    want = _ordered_pure_python(a, b)
    assert np.array_equal(cpp.gemm_ordered_f32(a, b).view(np.uint32), want.view(np.uint32))
    assert np.array_equal(cpp.gemm_ordered(a, b), torch_bf16_bits(want))


def test_ordered_bit_identical_to_numpy_oracle_and_empty_k():
    a = synthetic.normal_bf16((45, 700), 1.0, 110, 0)
    b = synthetic.normal_bf16((33, 700), 0.02, 110, 1)
    assert np.array_equal(cpp.gemm_ordered_f32(a, b, threads=3).view(np.uint32),
                          oracle.gemm_ordered_f32(a, b).view(np.uint32))
    z = cpp.gemm_ordered_f32(np.zeros((2, 0), np.uint16), np.zeros((3, 0), np.uint16))
    assert np.array_equal(z.view(np.uint32), np.zeros((2, 3), np.uint32))


# ---- fold epilogue --------------------------------------------------------------------

def test_scaled_acc_worked_cases():
    for ln in read_golden("scaled_acc_worked.txt"):
        f = [t.strip() for t in ln.split(";")]
        out = np.array([[int(f[1], 16)]], np.uint16)
        x = torch_bf16_bits(_parse_row(f[2])[None, :])
        b = torch_bf16_bits(_parse_row(f[3])[None, :])
        scale = struct.unpack("<f", struct.pack("<I", int(f[4], 16)))[0]
        delta = cpp.f32_to_bf16(cpp.gemm_bf16_ref(x, b).astype(np.float32))
        got = int(cpp.scaled_acc_epilogue(out, delta, scale)[0, 0])
        assert got == int(f[5], 16), (f[0], hex(got))


@pytest.mark.parametrize("scale", [2.0, 0.7, -1.3])
def test_scaled_acc_equals_unfused_pair(scale):
    out = synthetic.normal_bf16((6, 9), 1.0, 40, 0)
    x = synthetic.grid_bf16((6, 16), -8, 8, -5, 41, 0)
    b = synthetic.grid_bf16((9, 16), -8, 8, -5, 41, 1)
    delta = cpp.gemm_bf16_ref(x, b).astype(np.float32)
    got = cpp.scaled_acc_epilogue(out, cpp.f32_to_bf16(delta), scale)
    assert np.array_equal(got, _unfused_pure_python(out, delta, scale))
    assert np.array_equal(got, oracle.scaled_acc_epilogue(out, oracle.f32_to_bf16(delta), scale))


# ---- split-K -----------------------------------------------------------------------------

def test_splitk_chunk_table():
    for k, ks, want in [(11008, 8, 1408), (11008, 1, 11008), (2048, 4, 512), (100, 8, 64), (1, 4, 64)]:
        assert cpp.splitk_chunk(k, ks) == want
    with pytest.raises(ValueError):
        cpp.splitk_chunk(64, 0)


@pytest.mark.parametrize("k,ks", [(200, 3), (130, 8), (64, 2)])
def test_splitk_planes_brute_force_and_distributivity(k, ks):
    a = synthetic.grid_bf16((3, k), -8, 8, -5, 70 + k, 0)
    b = synthetic.grid_bf16((4, k), -8, 8, -5, 70 + k, 1)
    planes = cpp.gemm_splitk_planes_ref(a, b, ks)
    kc = cpp.splitk_chunk(k, ks)
    for s in range(ks):
        lo, hi = min(k, s * kc), min(k, (s + 1) * kc)
        for i in range(3):
            for j in range(4):
                exact = sum(bf16_exact(int(a[i, kk])) * bf16_exact(int(b[j, kk])) for kk in range(lo, hi))
                assert Fraction(planes[s, i, j]) == exact
    assert np.array_equal(planes.sum(axis=0), cpp.gemm_bf16_ref(a, b))


def test_splitk_reduce_is_ascending_fp32():
    p = np.array([[[2.0 ** 24]], [[1.0]], [[-(2.0 ** 24)]]], np.float32)
    # ((2^24 + 1) - 2^24) in FP32 ascending order is 0; descending gives 1
    assert int(cpp.splitk_reduce(p)[0, 0]) == 0
    assert int(cpp.splitk_reduce(p[::-1].copy())[0, 0]) == 0x3F80
    g = np.random.default_rng(5)
    q = g.standard_normal((4, 7, 9)).astype(np.float32)
    want = np.zeros((7, 9), np.float32)
    for idx in np.ndindex(7, 9):
        acc = float(q[0][idx])
        for s in range(1, 4):
            acc = f32r(acc + float(q[s][idx]))
        want[idx] = acc
    assert np.array_equal(cpp.splitk_reduce(q), torch_bf16_bits(want))


# ---- FP4 and W4A16 ------------------------------------------------------------------------

def test_fp4_brute_force_exact():
    tab = _e2m1_table()
    m, n, k = 3, 4, 48
    a = synthetic.fp4_packed(m, k, 80, 0)
    b = synthetic.fp4_packed(n, k, 80, 1)
    sfa = synthetic.e4m3_uniform(m, k // 16, 2 ** -4, 2 ** 4, 80, 4)
    sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 80, 5)
    sa = torch.from_numpy(sfa).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sb = torch.from_numpy(sfb).view(torch.float8_e4m3fn).to(torch.float64).numpy()

    def elem(packed, scales, r, kk):
        byte = int(packed[r, kk // 2])
        return tab[byte & 0xF if kk % 2 == 0 else byte >> 4] * Fraction(scales[r, kk // 16])

    got = cpp.gemm_fp4_ref(a, sfa, b, sfb)
    for i in range(m):
        for j in range(n):
            assert Fraction(got[i, j]) == sum(elem(a, sa, i, kk) * elem(b, sb, j, kk) for kk in range(k))


def test_fp4_agrees_with_numpy_oracle_and_splitk_planes_sum():
    m, n, k = 9, 11, 512
    a = synthetic.fp4_packed(m, k, 85, 0)
    b = synthetic.fp4_packed(n, k, 85, 1)
    sfa = synthetic.e4m3_uniform(m, k // 16, 2 ** -4, 2 ** 4, 85, 4)
    sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 85, 5)
    got, ref = cpp.gemm_fp4_ref(a, sfa, b, sfb), oracle.gemm_fp4_ref(a, sfa, b, sfb)
    da, db = oracle.dequant_fp4(a, sfa), oracle.dequant_fp4(b, sfb)
    bound = k * 2.0 ** -52 * (np.abs(da) @ np.abs(db).T)
    assert (np.abs(got - ref) <= 2 * bound).all()
    planes = cpp.gemm_fp4_splitk_planes_ref(a, sfa, b, sfb, 3)
    assert (np.abs(planes.sum(axis=0) - got) <= 4 * bound).all()


def test_w4a16_brute_force_exact_rationals():
    tab = _e2m1_table()
    m, n, k = 3, 5, 48
    a = synthetic.normal_bf16((m, k), 1.0, 90, 0)
    b = synthetic.fp4_packed(n, k, 90, 1)
    sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 90, 5)
    sb = torch.from_numpy(sfb).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    s2 = 0.0123
    s2f = Fraction(float(np.float32(s2)))
    got = cpp.gemm_w4a16_ref(a, b, sfb, s2)
    for i in range(m):
        for j in range(n):
            dot = sum(bf16_exact(int(a[i, kk])) *
                      tab[int(b[j, kk // 2]) & 0xF if kk % 2 == 0 else int(b[j, kk // 2]) >> 4] *
                      Fraction(sb[j, kk // 16]) for kk in range(k))
            exact = s2f * dot
            assert abs(Fraction(got[i, j]) - exact) <= Fraction(2) ** -50 * (abs(exact) + Fraction(2) ** -200)
