"""Pins for the oracle's GEMM definitions (CPU only).

The oracle is checked against things other than itself: exact rational brute
force written independently here, closed-form identities that hold exactly in
any summation order, hand-worked rounding cases under tests/golden/, and a
pure-Python IEEE-single emulation of the order-preserving recurrence.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden
import oracle
import synthetic


# ---------------------------------------------------------------------------
# independent helpers (exact rationals, pure-Python single precision)
# ---------------------------------------------------------------------------

def bf16_exact(bits: int) -> Fraction:
    """Exact value of a BF16 bit pattern from its fields (finite only)."""
    s, e, m = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    assert e != 0xFF
    v = Fraction(m, 128) * Fraction(2) ** -126 if e == 0 else Fraction(128 + m, 128) * Fraction(2) ** (e - 127)
    return -v if s else v


def f32r(x: float) -> float:
    """Round a Python float (binary64) to binary32, nearest-even.

    Correct for one +, -, * of binary32 operands computed in binary64, since
    53 >= 2*24 + 2 (double rounding is then innocuous).
    """
    return struct.unpack("<f", struct.pack("<f", x))[0]


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def torch_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x_f32, np.float32).copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rand_bf16(shape, seed, std=1.0):
    return synthetic.normal_bf16(shape, std, seed, 0)


# ---------------------------------------------------------------------------
# dense GEMM
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,n,k", [(3, 5, 7), (1, 1, 1), (4, 2, 19), (2, 6, 33)])
def test_dense_brute_force_exact_rationals(m, n, k):
    a = rand_bf16((m, k), 10 + k)
    b = synthetic.normal_bf16((n, k), 0.5, 20 + k, 1)
    got = oracle.gemm_bf16_ref(a, b)
    assert got.shape == (m, n)
    for i in range(m):
        for j in range(n):
            exact = sum(bf16_exact(int(a[i, kk])) * bf16_exact(int(b[j, kk])) for kk in range(k))
            absum = sum(abs(bf16_exact(int(a[i, kk])) * bf16_exact(int(b[j, kk]))) for kk in range(k))
            assert abs(Fraction(got[i, j]) - exact) <= Fraction(k) * Fraction(2) ** -52 * absum


def test_dense_exactly_summable_is_exact():
    a = synthetic.grid_bf16((9, 40), -8, 8, -5, 1, 0)
    b = synthetic.grid_bf16((11, 40), -8, 8, -5, 1, 1)
    got = oracle.gemm_bf16_ref(a, b)
    for i in range(9):
        for j in range(11):
            exact = sum(bf16_exact(int(a[i, kk])) * bf16_exact(int(b[j, kk])) for kk in range(40))
            assert Fraction(got[i, j]) == exact


def test_dense_identity_and_permutation():
    k = 24
    a = rand_bf16((5, k), 3)
    eye = torch_bf16_bits(np.eye(k, dtype=np.float32))
    assert np.array_equal(oracle.gemm_bf16_ref(a, eye), oracle.bf16_to_f64(a))
    perm = np.random.default_rng(5).permutation(k)
    p = np.zeros((k, k), np.float32)
    p[np.arange(k), perm] = 1.0          # row j of B selects column perm[j] of A
    got = oracle.gemm_bf16_ref(a, torch_bf16_bits(p))
    assert np.array_equal(got, oracle.bf16_to_f64(a)[:, perm])
    # power-of-two diagonal scales columns exactly
    d = np.diag(np.exp2(np.arange(k) % 5 - 2).astype(np.float32))
    got = oracle.gemm_bf16_ref(a, torch_bf16_bits(d))
    assert np.array_equal(got, oracle.bf16_to_f64(a) * np.exp2(np.arange(k) % 5 - 2)[None, :])


def test_dense_transpose_symmetry_and_zero_k_padding():
    a = synthetic.grid_bf16((7, 29), -6, 6, -4, 2, 0)
    b = synthetic.grid_bf16((13, 29), -6, 6, -4, 2, 1)
    c = oracle.gemm_bf16_ref(a, b)
    assert np.array_equal(c, oracle.gemm_bf16_ref(b, a).T)
    pad = np.zeros((7, 35), np.uint16)
    pad[:, :29] = a
    padb = np.zeros((13, 35), np.uint16)
    padb[:, :29] = b
    assert np.array_equal(c, oracle.gemm_bf16_ref(pad, padb))


def test_dense_empty_k_is_zero():
    a = np.zeros((3, 0), np.uint16)
    b = np.zeros((4, 0), np.uint16)
    assert np.array_equal(oracle.gemm_bf16_ref(a, b), np.zeros((3, 4)))


def test_tolerance_closed_form():
    ref = np.array([0.0, 1.0, -2.0])
    t = oracle.tolerance(ref, 400, 1.0, 0.02)
    assert np.allclose(t, 8e-3 * np.abs(ref) + 4e-3 * 20.0 * 0.02)


# ---------------------------------------------------------------------------
# order-preserving mode
# ---------------------------------------------------------------------------

def _parse_row(s):
    return np.array([float(t) for t in s.split()], dtype=np.float32)


def test_ordered_worked_cases():
    for ln in read_golden("ordered_worked.txt"):
        fields = [f.strip() for f in ln.split(";")]
        name, arow, brow, want = fields[0], _parse_row(fields[1]), _parse_row(fields[2]), int(fields[3], 16)
        a = torch_bf16_bits(arow[None, :])
        b = torch_bf16_bits(brow[None, :])
        assert np.array_equal(oracle.bf16_to_f32(a)[0], arow), name     # inputs exact in BF16
        got = oracle.gemm_ordered_f32(a, b)
        assert f32_bits(float(got[0, 0])) == want, name
        if name == "cancel":
            # reversed order differs, so the test pins the direction
            rev = oracle.gemm_ordered_f32(a[:, ::-1].copy(), b[:, ::-1].copy())
            assert f32_bits(float(rev[0, 0])) == 0x3F800000


def _ordered_pure_python(a_bits, b_bits):
    m, k = a_bits.shape
    n = b_bits.shape[0]
    a = [[float(bf16_exact(int(v))) for v in row] for row in a_bits]
    b = [[float(bf16_exact(int(v))) for v in row] for row in b_bits]
    out = np.zeros((m, n), np.float32)
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                acc = f32r(acc + f32r(a[i][kk] * b[j][kk]))
            out[i, j] = acc
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_ordered_matches_pure_python_ieee_single(seed):
    a = rand_bf16((4, 37), 100 + seed, 3.0)
    b = synthetic.normal_bf16((5, 37), 7.0, 200 + seed, 1)
    got = oracle.gemm_ordered_f32(a, b)
    want = _ordered_pure_python(a, b)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(oracle.gemm_ordered(a, b), torch_bf16_bits(want))


def test_ordered_empty_k_is_positive_zero():
    got = oracle.gemm_ordered_f32(np.zeros((2, 0), np.uint16), np.zeros((3, 0), np.uint16))
    assert np.array_equal(got.view(np.uint32), np.zeros((2, 3), np.uint32))


# ---------------------------------------------------------------------------
# fused LoRA fold
# ---------------------------------------------------------------------------

def test_scaled_acc_worked_cases():
    for ln in read_golden("scaled_acc_worked.txt"):
        f = [t.strip() for t in ln.split(";")]
        name = f[0]
        out = np.array([[int(f[1], 16)]], np.uint16)
        x = torch_bf16_bits(_parse_row(f[2])[None, :])
        b = torch_bf16_bits(_parse_row(f[3])[None, :])
        scale = struct.unpack("<f", struct.pack("<I", int(f[4], 16)))[0]
        want = int(f[5], 16)
        got = int(oracle.gemm_scaled_acc_exact(out, x, b, scale)[0, 0])
        assert got == want, (name, hex(got))


def _unfused_pure_python(out_bits, delta_f32, scale):
    """BF16 scratch of delta (torch RNE), then a scaled add in IEEE single."""
    scratch = torch_bf16_bits(delta_f32)
    res = np.zeros(out_bits.shape, np.float32)
    for idx in np.ndindex(out_bits.shape):
        d = float(bf16_exact(int(scratch[idx])))
        o = float(bf16_exact(int(out_bits[idx])))
        res[idx] = f32r(o + f32r(f32r(scale) * d))
    return torch_bf16_bits(res)


@pytest.mark.parametrize("scale", [2.0, 0.7, -1.3])
def test_scaled_acc_equals_unfused_pair(scale):
    out = rand_bf16((6, 9), 40)
    x = synthetic.grid_bf16((6, 16), -8, 8, -5, 41, 0)
    b = synthetic.grid_bf16((9, 16), -8, 8, -5, 41, 1)
    delta = oracle.gemm_bf16_ref(x, b).astype(np.float32)      # exact for grid inputs
    got = oracle.gemm_scaled_acc_exact(out, x, b, scale)
    assert np.array_equal(got, _unfused_pure_python(out, delta, scale))


def test_scaled_acc_scale_zero_keeps_values_and_unit_rows_add():
    out = rand_bf16((5, 8), 50)
    x = rand_bf16((5, 8), 51)
    b = rand_bf16((8, 8), 52)
    kept = oracle.gemm_scaled_acc_exact(out, x, b, 0.0)
    assert np.array_equal(oracle.bf16_to_f32(kept), oracle.bf16_to_f32(out))
    # X = identity rows, scale 1: out + B^T as a BF16 add (exact sum rounded once via FP32)
    eye = torch_bf16_bits(np.eye(8, dtype=np.float32)[:5])
    got = oracle.gemm_scaled_acc_exact(out, eye, b, 1.0)
    for i in range(5):
        for j in range(8):
            s = bf16_exact(int(out[i, j])) + bf16_exact(int(b[j, i]))
            want = torch_bf16_bits(np.array([f32r(float(s))], np.float32))[0]
            assert got[i, j] == want


def _bits_of_values(vals):
    return torch_bf16_bits(np.asarray(vals, np.float32)[None, :])


def test_candidate_deltas_one_when_far_from_a_rounding_midpoint():
    # exact delta 1.5 (a BF16 value), bound 4 * 2^-24 * 1.5: one candidate
    lo, hi, n = oracle.scaled_acc_candidate_deltas(_bits_of_values([1.0, 0.0]), _bits_of_values([1.5, 0.0]))
    assert int(n[0, 0]) == 1 and int(lo[0, 0]) == int(hi[0, 0]) == 0x3FC0


def test_candidate_deltas_exactly_two_at_a_midpoint():
    # exact delta 1 + 2^-8 lies halfway between the BF16 values 1.0 (0x3F80)
    # and 1 + 2^-7 (0x3F81): any nonzero error bound admits both, and a bound
    # of a few FP32 ulps admits nothing else
    lo, hi, n = oracle.scaled_acc_candidate_deltas(_bits_of_values([1.0, 2.0 ** -8]), _bits_of_values([1.0, 1.0]))
    assert (int(lo[0, 0]), int(hi[0, 0]), int(n[0, 0])) == (0x3F80, 0x3F81, 2)


def test_candidate_bound_size_pinned_from_both_sides():
    """K = 3, sum|x*b| = 1 + 2^-8 + e, so Bd = 2 * 3 * 2^-24 * (1 + 2^-8 + e)
    = 3.58e-7 (to 3 digits). The exact delta is the midpoint 1 + 2^-8 plus e:
    e = 2^-23 (1.19e-7, inside Bd) keeps the midpoint reachable (two
    candidates); e = 2^-21 (4.77e-7, outside Bd) does not (one candidate,
    0x3F81). A bound too small by 3x or too large by 1.4x fails one case."""
    b = _bits_of_values([1.0, 1.0, 1.0])
    _, _, n_in = oracle.scaled_acc_candidate_deltas(_bits_of_values([1.0, 2.0 ** -8, 2.0 ** -23]), b)
    lo, hi, n_out = oracle.scaled_acc_candidate_deltas(_bits_of_values([1.0, 2.0 ** -8, 2.0 ** -21]), b)
    assert int(n_in[0, 0]) == 2
    assert int(n_out[0, 0]) == 1 and int(lo[0, 0]) == 0x3F81
    # the same exact delta with a bound of 1/3 or 1.4x the default
    _, _, n_small = oracle.scaled_acc_candidate_deltas(_bits_of_values([1.0, 2.0 ** -8, 2.0 ** -23]), b,
                                                       depth_factor=2.0 / 3.5)
    _, _, n_big = oracle.scaled_acc_candidate_deltas(_bits_of_values([1.0, 2.0 ** -8, 2.0 ** -21]), b,
                                                     depth_factor=2.0 * 1.4)
    assert int(n_small[0, 0]) == 1 and int(n_big[0, 0]) == 2


def test_admissible_requires_a_candidate_output_not_the_range():
    """Candidates delta in {1.0, 1 + 2^-7}, out = 0, scale 3: the outputs are
    bf16(3.0) = 0x4040 and bf16(3.0234375) = 0x4042 (a tie rounded to even).
    0x4041 lies between them but no candidate produces it."""
    x, b = _bits_of_values([1.0, 2.0 ** -8]), _bits_of_values([1.0, 1.0])
    out = np.zeros((1, 1), np.uint16)
    for got, want in ((0x4040, True), (0x4041, False), (0x4042, True), (0x403F, False), (0x4043, False)):
        ok, n = oracle.scaled_acc_admissible(np.array([[got]], np.uint16), out, x, b, 3.0)
        assert bool(ok[0, 0]) == want, hex(got)
        assert int(n[0, 0]) == 2


def test_admissible_accepts_the_exact_result_and_rejects_neighbours():
    out = rand_bf16((8, 32), 60)
    x = synthetic.normal_bf16((8, 64), 0.1, 61, 0)
    b = synthetic.normal_bf16((32, 64), 0.1, 61, 1)
    exact = oracle.scaled_acc_epilogue(out, oracle.f32_to_bf16(oracle.gemm_bf16_ref(x, b).astype(np.float32)), 2.0)
    ok, n = oracle.scaled_acc_admissible(exact, out, x, b, 2.0)
    assert ok.all()
    # near-zero deltas may admit several BF16 values; most admit exactly one
    assert (n >= 1).all() and (n == 1).mean() > 0.8
    # one BF16 step away from the exact output is rejected wherever only one
    # candidate exists and the output is not zero
    one = (n == 1) & ((exact & 0x7FFF) != 0)
    ok_up, _ = oracle.scaled_acc_admissible((exact + 1).astype(np.uint16), out, x, b, 2.0)
    assert not ok_up[one].any()


def test_admissible_zero_delta_tries_both_signs():
    # out = -0, delta = exactly zero: -0 + 2*(+0) = +0 and -0 + 2*(-0) = -0 are both admissible
    x, b = _bits_of_values([0.0]), _bits_of_values([1.0])
    out = np.array([[0x8000]], np.uint16)
    for got in (0x0000, 0x8000):
        ok, _ = oracle.scaled_acc_admissible(np.array([[got]], np.uint16), out, x, b, 2.0)
        assert ok[0, 0]


# ---------------------------------------------------------------------------
# RMS (the sigma of the tolerance)
# ---------------------------------------------------------------------------

def test_rms_closed_forms():
    assert oracle.rms(np.array([3.0, 4.0])) == np.sqrt(12.5)
    assert oracle.rms(np.array([[1.0, -1.0], [-1.0, 1.0]])) == 1.0
    assert oracle.rms(np.full((7, 3), -0.25)) == 0.25
    assert oracle.rms(np.zeros((0, 5))) == 0.0
    # sqrt(mean): one large value among n zeros gives |v| / sqrt(n)
    v = np.zeros(16)
    v[5] = 8.0
    assert oracle.rms(v) == 2.0


def test_rms_of_the_config_weights_matches_their_standard_deviation():
    """N(0, 0.02) weights of the Q/O projection, 2048 x 2048 draws: the RMS of
    the stored BF16 values is 0.02 up to sampling error (relative standard
    error 1/sqrt(2n) = 3.5e-4) and BF16 rounding (relative 2^-9 per value,
    zero-mean)."""
    _, w = synthetic.attn_proj(n=2048)
    r = oracle.rms(oracle.bf16_to_f64(w))
    assert abs(r / 0.02 - 1.0) < 2e-3
    a, _ = synthetic.mlp_gate_up(m=256)
    assert abs(oracle.rms(oracle.bf16_to_f64(a)) - 1.0) < 5e-3


# ---------------------------------------------------------------------------
# split-K
# ---------------------------------------------------------------------------

def test_splitk_chunk_table():
    assert oracle.splitk_chunk(2048, 1) == 2048
    assert oracle.splitk_chunk(2048, 8) == 256
    assert oracle.splitk_chunk(11008, 2) == 5504
    assert oracle.splitk_chunk(11008, 4) == 2752
    assert oracle.splitk_chunk(11008, 8) == 1408
    assert oracle.splitk_chunk(100, 8) == 64
    assert oracle.splitk_chunk(0, 3) == 0


@pytest.mark.parametrize("k,ks", [(200, 3), (130, 8), (64, 2), (1, 4)])
def test_splitk_planes_brute_force_and_distributivity(k, ks):
    a = synthetic.grid_bf16((3, k), -8, 8, -5, 70, 0)
    b = synthetic.grid_bf16((4, k), -8, 8, -5, 70, 1)
    planes = oracle.gemm_splitk_planes_ref(a, b, ks)
    kc = oracle.splitk_chunk(k, ks)
    for s in range(ks):
        lo, hi = min(k, s * kc), min(k, (s + 1) * kc)
        for i in range(3):
            for j in range(4):
                exact = sum((bf16_exact(int(a[i, kk])) * bf16_exact(int(b[j, kk])) for kk in range(lo, hi)), Fraction(0))
                assert Fraction(planes[s, i, j]) == exact
    assert np.array_equal(planes.sum(axis=0), oracle.gemm_bf16_ref(a, b))


def test_splitk_reduce_is_ascending_fp32():
    planes = np.array([[[2.0 ** 24]], [[1.0]], [[-(2.0 ** 24)]]], np.float32)
    assert int(oracle.splitk_reduce(planes)[0, 0]) == 0x0000
    assert int(oracle.splitk_reduce(planes[::-1])[0, 0]) == 0x3F80
    # one plane: the value itself (sign of zero kept)
    neg0 = np.array([[[-0.0]]], np.float32)
    assert int(oracle.splitk_reduce(neg0)[0, 0]) == 0x8000


# ---------------------------------------------------------------------------
# block-scaled FP4
# ---------------------------------------------------------------------------

def _e2m1_table():
    return {int(r.split()[0]): Fraction(r.split()[1]) for r in read_golden("e2m1_table.txt")}


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
        code = byte & 0xF if kk % 2 == 0 else byte >> 4
        return tab[code] * Fraction(scales[r, kk // 16])

    got = oracle.gemm_fp4_ref(a, sfa, b, sfb)
    for i in range(m):
        for j in range(n):
            exact = sum(elem(a, sa, i, kk) * elem(b, sb, j, kk) for kk in range(k))
            assert Fraction(got[i, j]) == exact


def test_fp4_unit_scales_reduce_to_dense_on_dequantized_operands():
    m, n, k = 5, 6, 64
    a = synthetic.fp4_packed(m, k, 81, 0)
    b = synthetic.fp4_packed(n, k, 81, 1)
    one = np.full((m, k // 16), 0x38, np.uint8)
    oneb = np.full((n, k // 16), 0x38, np.uint8)
    tab = np.array([float(_e2m1_table()[c]) for c in range(16)], np.float32)
    ab = torch_bf16_bits(tab[oracle.unpack_e2m1(a)])
    bb = torch_bf16_bits(tab[oracle.unpack_e2m1(b)])
    assert np.array_equal(oracle.gemm_fp4_ref(a, one, b, oneb), oracle.gemm_bf16_ref(ab, bb))


def test_fp4_power_of_two_scales_exact_in_fp32():
    """Scales in {1, 2}: every partial sum is a multiple of 1/4 below 2^21."""
    m, n, k = 4, 4, 8192
    a = synthetic.fp4_packed(m, k, 82, 0)
    b = synthetic.fp4_packed(n, k, 82, 1)
    sfa = synthetic.e4m3_choice(m, k // 16, [0x38, 0x40], 82, 4)
    sfb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40], 82, 5)
    ref = oracle.gemm_fp4_ref(a, sfa, b, sfb)
    assert np.array_equal(ref, ref.astype(np.float32).astype(np.float64))
    assert np.array_equal(ref * 4, np.round(ref * 4))


# ---------------------------------------------------------------------------
# W4A16 (BF16 activations x NVFP4 weights with a per-tensor scale)
# ---------------------------------------------------------------------------

def _e4m3_exact(byte: int) -> Fraction:
    """E4M3FN from its bit fields (bias 7, subnormal m * 2^-9); finite codes only."""
    s, e, m = byte >> 7, (byte >> 3) & 15, byte & 7
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return -v if s else v


def test_w4a16_brute_force_exact_rationals():
    tab = _e2m1_table()
    m, n, k = 3, 5, 48
    a = rand_bf16((m, k), 90)
    b = synthetic.fp4_packed(n, k, 90, 1)
    sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 90, 5)
    s2 = 0.0123
    s2_exact = Fraction(struct.unpack("<f", struct.pack("<f", s2))[0])
    got = oracle.gemm_w4a16_ref(a, b, sfb, s2)
    for i in range(m):
        for j in range(n):
            dot = Fraction(0)
            for kk in range(k):
                byte = int(b[j, kk // 2])
                code = byte & 0xF if kk % 2 == 0 else byte >> 4
                dot += bf16_exact(int(a[i, kk])) * tab[code] * _e4m3_exact(int(sfb[j, kk // 16]))
            exact = s2_exact * dot
            # the FP64 dot product is exact here; only the final product rounds
            assert abs(Fraction(got[i, j]) - exact) <= abs(exact) * Fraction(2) ** -52


def test_w4a16_identity_weights_with_group_scales():
    """B = identity (code 0x2 = 1.0 on the diagonal), scale 2 on even 16-groups
    of each row and 1 on odd ones: C[:, j] = s2 * A[:, j] * (2 if (j // 16) even)."""
    k = n = 64
    a = rand_bf16((7, k), 91)
    codes = np.zeros((n, k), np.uint8)
    codes[np.arange(n), np.arange(n)] = 0x2
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sfb = np.where((np.arange(k // 16)[None, :] % 2) == 0, 0x40, 0x38).astype(np.uint8).repeat(n, 0)
    s2 = 0.75
    got = oracle.gemm_w4a16_ref(a, packed, sfb, s2)
    af = oracle.bf16_to_f64(a)
    factor = np.where((np.arange(n) // 16) % 2 == 0, 2.0, 1.0)
    assert np.array_equal(got, 0.75 * af * factor[None, :])


def test_w4a16_exact_output_rounds_once_in_fp32_then_bf16():
    """Grid activations and scales in {1, 2}: every dot product is exact in FP32,
    so C = bf16(fl32(s2 * acc)) is unique; checked by exact rationals and a
    pure-Python single-precision multiply."""
    tab = _e2m1_table()
    m, n, k = 4, 6, 256
    a = synthetic.grid_bf16((m, k), -8, 8, -5, 92, 0)
    b = synthetic.fp4_packed(n, k, 92, 1)
    sfb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40], 92, 5)
    for s2 in (0.0123, 1.0, 3.0, -0.3):
        got = oracle.gemm_w4a16_exact(a, b, sfb, s2)
        s2f = struct.unpack("<f", struct.pack("<f", s2))[0]
        for i in range(m):
            for j in range(n):
                dot = Fraction(0)
                for kk in range(k):
                    byte = int(b[j, kk // 2])
                    code = byte & 0xF if kk % 2 == 0 else byte >> 4
                    dot += bf16_exact(int(a[i, kk])) * tab[code] * _e4m3_exact(int(sfb[j, kk // 16]))
                prod = f32r(float(Fraction(s2f) * dot))      # exact in a double, one FP32 rounding
                want = torch_bf16_bits(np.array([prod], np.float32))[0]
                assert int(got[i, j]) == int(want)


def test_w4a16_exact_rejects_inexact_sums():
    a = rand_bf16((2, 64), 93)
    b = synthetic.fp4_packed(3, 64, 93, 1)
    sfb = synthetic.e4m3_uniform(3, 4, 2 ** -4, 2 ** 4, 93, 5)
    with pytest.raises(ValueError):
        oracle.gemm_w4a16_exact(a, b, sfb, 1.0)


def test_w4a16_on_dequantized_activations_equals_fp4_times_scale():
    """With A holding exact FP4 values (unit scales), W4A16 is the FP4 GEMM times s2."""
    m, n, k = 5, 4, 64
    qa = synthetic.fp4_packed(m, k, 94, 0)
    one = np.full((m, k // 16), 0x38, np.uint8)
    tab = np.array([float(_e2m1_table()[c]) for c in range(16)], np.float32)
    a = torch_bf16_bits(tab[oracle.unpack_e2m1(qa)])
    b = synthetic.fp4_packed(n, k, 94, 1)
    sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 94, 5)
    assert np.array_equal(oracle.gemm_w4a16_ref(a, b, sfb, 0.5), 0.5 * oracle.gemm_fp4_ref(qa, one, b, sfb))


@pytest.mark.parametrize("k,ks", [(1024, 4), (4096, 8), (160, 3)])
def test_fp4_splitk_planes_sum_and_slices(k, ks):
    """FP4 split-K planes: each is the FP4 definition on its K slice of the
    packed bytes and scales, and they sum exactly to the full FP4 result."""
    m, n = 3, 5
    a = synthetic.fp4_packed(m, k, 95, 0)
    b = synthetic.fp4_packed(n, k, 95, 1)
    sfa = synthetic.e4m3_choice(m, k // 16, [0x38, 0x40, 0x30], 95, 4)
    sfb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40, 0x30], 95, 5)
    planes = oracle.gemm_fp4_splitk_planes_ref(a, sfa, b, sfb, ks)
    kc = oracle.splitk_chunk(k, ks)
    for s in range(ks):
        lo, hi = min(k, s * kc), min(k, (s + 1) * kc)
        if hi == lo:
            assert not planes[s].any()
            continue
        want = oracle.gemm_fp4_ref(a[:, lo // 2:hi // 2], sfa[:, lo // 16:hi // 16],
                                   b[:, lo // 2:hi // 2], sfb[:, lo // 16:hi // 16])
        assert np.array_equal(planes[s], want)
    assert np.array_equal(planes.sum(axis=0), oracle.gemm_fp4_ref(a, sfa, b, sfb))


# ---------------------------------------------------------------------------
# W4A16 with transposed weights (row stride ldb >= N)
# ---------------------------------------------------------------------------

def test_w4a16_t_brute_force_exact_rationals():
    """Bytes read straight from the transposed layout by index: byte (k // 2, j)
    of Bt, low nibble for even k; scale byte (k // 16, j) of SFBt; pad columns
    j >= N hold junk that must not matter."""
    tab = _e2m1_table()
    m, n, k, ldb = 3, 5, 48, 7
    a = rand_bf16((m, k), 96)
    bt = synthetic.fp4_packed(k // 2, 2 * ldb, 96, 1)            # [K/2, ldb] bytes
    sfbt = synthetic.e4m3_uniform(k // 16, ldb, 2 ** -4, 2 ** 4, 96, 5)
    s2 = 0.0123
    s2_exact = Fraction(struct.unpack("<f", struct.pack("<f", s2))[0])
    got = oracle.gemm_w4a16_t_ref(a, bt, sfbt, n, s2)
    assert got.shape == (m, n)
    for i in range(m):
        for j in range(n):
            dot = Fraction(0)
            for kk in range(k):
                byte = int(bt[kk // 2, j])
                code = byte & 0xF if kk % 2 == 0 else byte >> 4
                dot += bf16_exact(int(a[i, kk])) * tab[code] * _e4m3_exact(int(sfbt[kk // 16, j]))
            exact = s2_exact * dot
            assert abs(Fraction(got[i, j]) - exact) <= abs(exact) * Fraction(2) ** -52


def test_w4a16_t_equals_w4a16_on_the_same_weights():
    """The same weights in both layouts give the same FP64 result: B[j, t] =
    Bt[t, j] and SFB[j, g] = SFBt[g, j], built with explicit loops."""
    m, n, k, ldb = 4, 9, 64, 12
    a = rand_bf16((m, k), 97)
    bt = synthetic.fp4_packed(k // 2, 2 * ldb, 97, 1)
    sfbt = synthetic.e4m3_uniform(k // 16, ldb, 2 ** -4, 2 ** 4, 97, 5)
    b = np.zeros((n, k // 2), np.uint8)
    sfb = np.zeros((n, k // 16), np.uint8)
    for j in range(n):
        for t in range(k // 2):
            b[j, t] = bt[t, j]
        for g in range(k // 16):
            sfb[j, g] = sfbt[g, j]
    assert np.array_equal(oracle.gemm_w4a16_t_ref(a, bt, sfbt, n, 0.7), oracle.gemm_w4a16_ref(a, b, sfb, 0.7))
    # the pad columns are ignored
    bt2, sfbt2 = bt.copy(), sfbt.copy()
    bt2[:, n:] = 0xFF
    sfbt2[:, n:] = 0x7F
    assert np.array_equal(oracle.gemm_w4a16_t_ref(a, bt2, sfbt2, n, 0.7), oracle.gemm_w4a16_t_ref(a, bt, sfbt, n, 0.7))
