"""Plain CPU definitions of what each library entry point computes.

Test infrastructure only (see the package docstring). Every routine is the
definition of its operation written out directly: decode the stored inputs
exactly, then form the sums. FP64 is used wherever the pages leave the
accumulation order open; the order-preserving mode is written as the literal
FP32 recurrence. numpy's float64 matrix product serves as the dot-product step
of the FP64 definitions (BF16 x BF16 and E2M1*E4M3 x E2M1*E4M3 products are
exact in FP64, and the FP64 sum's error is far below every tolerance used).

Layout throughout: A is [M, K], B is [N, K] (both K-contiguous), C is [M, N];
C = A * B^T (gemm_dense.rs page, doc comment of the dense BF16 GEMM: A [M, K]
activations, B [N, K] weights in HuggingFace layout, C [M, N]).
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import bf16_to_f32, bf16_to_f64, dequant_fp4, dequant_fp4_t, f32_to_bf16


# ---------------------------------------------------------------------------
# dense BF16 GEMM (gemm_bf16)
# ---------------------------------------------------------------------------

def gemm_bf16_ref(a_bits, b_bits) -> np.ndarray:
    """ref[i, j] = sum_k A[i, k] * B[j, k], exact BF16 operands, FP64 sum.

    sm121a_matmul.py page, the kernel body: FP32 accumulator over K blocks with
    the K tail masked to zero, cast to BF16 at the store; gemm_dense.rs page,
    dense BF16 GEMM doc: C = A @ B^T. The reference is left unrounded; the BF16
    output rounding is covered by the tolerance.
    """
    a = bf16_to_f64(a_bits)
    b = bf16_to_f64(b_bits)
    assert a.shape[1] == b.shape[1], "A and B share K"
    return a @ b.T


def rms(values_f64) -> float:
    """Root mean square sqrt(mean(v^2)) of a decoded input tensor, in FP64
    (0 for an empty one): the sigma_A, sigma_B of the tolerance below, taken
    from the stored values rather than the nominal standard deviation."""
    v = np.asarray(values_f64, dtype=np.float64)
    return float(np.sqrt(np.mean(v * v))) if v.size else 0.0


def tolerance(ref, k: int, sigma_a: float, sigma_b: float) -> np.ndarray:
    """Admissible |c - ref| for the MFMA paths: 8e-3*|ref| + 4e-3*sqrt(K)*sA*sB."""
    return 8e-3 * np.abs(ref) + 4e-3 * math.sqrt(max(k, 0)) * sigma_a * sigma_b


# ---------------------------------------------------------------------------
# order-preserving mode (gemm_bf16_ordered)
# ---------------------------------------------------------------------------

def gemm_ordered_f32(a_bits, b_bits) -> np.ndarray:
    """Strict k = 0..K-1 FP32 recurrence, one rounding per operation, no FMA.

    gemm_dense.rs page, doc comment of dense_gemm_router: the same math and the
    same per-output accumulation order (strict k = 0..K-1) as the scalar dense
    kernel, built without FMA contraction. Read here as: acc starts at +0.0f;
    for each k in ascending order, p = fl32(a*b) and acc = fl32(acc + p).
    numpy float32 ufuncs round once per operation and never fuse.
    """
    a = bf16_to_f32(a_bits)
    b = bf16_to_f32(b_bits)
    m, k = a.shape
    n = b.shape[0]
    acc = np.zeros((m, n), dtype=np.float32)
    prod = np.empty((m, n), dtype=np.float32)
    for kk in range(k):
        np.multiply(a[:, kk, None], b[None, :, kk], out=prod)
        np.add(acc, prod, out=acc)
    return acc


def gemm_ordered(a_bits, b_bits) -> np.ndarray:
    """BF16 output of the order-preserving mode: bf16(strict FP32 sum)."""
    return f32_to_bf16(gemm_ordered_f32(a_bits, b_bits))


# ---------------------------------------------------------------------------
# fused LoRA fold (gemm_bf16_scaled_acc)
# ---------------------------------------------------------------------------

def scaled_acc_epilogue(out_bits, delta_bf16_bits, scale) -> np.ndarray:
    """out_new = bf16(fl32(f32(out) + fl32(scale * f32(bf16(delta))))).

    gemm_dense.rs page, doc comment of dense_gemm_tc_scaled_acc: the fused
    epilogue must equal the unfused pair, i.e. the delta is first stored as a
    BF16 tensor and then a BF16 scaled add reads it. Read here as one FP32
    multiply, then one FP32 add (no FMA), then one FP32 -> BF16 rounding.
    """
    d = bf16_to_f32(delta_bf16_bits)
    p = np.multiply(np.float32(scale), d, dtype=np.float32)
    s = np.add(bf16_to_f32(out_bits), p, dtype=np.float32)
    return f32_to_bf16(s)


def gemm_scaled_acc_exact(out_bits, x_bits, b_bits, scale) -> np.ndarray:
    """Fused fold for inputs whose FP32 accumulation is exact in any order.

    The delta is the exact product sum (FP64, then FP32: exact by assumption),
    rounded to BF16, then the epilogue above.
    """
    delta = gemm_bf16_ref(x_bits, b_bits).astype(np.float32)
    return scaled_acc_epilogue(out_bits, f32_to_bf16(delta), scale)


def _f32_ceil(x) -> np.ndarray:
    """Smallest FP32 value >= x (elementwise, x finite FP64)."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    return np.where(f.astype(np.float64) < x, np.nextafter(f, np.float32(np.inf)), f).astype(np.float32)


def _f32_floor(x) -> np.ndarray:
    """Largest FP32 value <= x (elementwise, x finite FP64)."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    return np.where(f.astype(np.float64) > x, np.nextafter(f, np.float32(-np.inf)), f).astype(np.float32)


def _bf16_order_key(bits) -> np.ndarray:
    """Monotone integer key of BF16 bit patterns (-0 and +0 share key 0)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    return np.where(u & 0x8000, -(u & 0x7FFF), u)


def _bf16_from_key(key) -> np.ndarray:
    """Inverse of _bf16_order_key (key 0 gives +0)."""
    k = np.asarray(key, dtype=np.int64)
    return np.where(k < 0, 0x8000 | (-k), k).astype(np.uint16)


def scaled_acc_candidate_deltas(x_bits, b_bits, depth_factor: float = 2.0):
    """The BF16 deltas a correct FP32 accumulation of X * B^T may round to.

    The MFMA summation order is not specified, so the FP32 accumulator of a
    K-term dot product is only known to lie within
        Bd = depth_factor * K * 2^-24 * sum_k |x_k * b_k|
    of the exact sum (the classical bound for recursive summation with unit
    roundoff 2^-24 is (K-1) * 2^-24 * sum|x*b| to first order; depth_factor = 2
    doubles it to cover accumulators that truncate). The reachable FP32 values
    are those in [exact - Bd, exact + Bd]; BF16 rounding is monotone and moves
    at most one BF16 step between adjacent FP32 values, so the candidate
    deltas are every BF16 value from bf16(lowest reachable) to
    bf16(highest reachable).

    Returns (lo_bits, hi_bits, n_candidates): the extreme candidate deltas as
    BF16 bits and the number of distinct candidate values (1 where the
    rounding is unambiguous).
    """
    x = bf16_to_f64(x_bits)
    b = bf16_to_f64(b_bits)
    k = x.shape[1]
    exact = x @ b.T
    bound = depth_factor * k * 2.0 ** -24 * (np.abs(x) @ np.abs(b).T)
    lo_d = f32_to_bf16(_f32_ceil(exact - bound))
    hi_d = f32_to_bf16(_f32_floor(exact + bound))
    n_cand = _bf16_order_key(hi_d) - _bf16_order_key(lo_d) + 1
    return lo_d, hi_d, n_cand


def scaled_acc_admissible(got_bits, out_bits, x_bits, b_bits, scale, depth_factor: float = 2.0):
    """Which fused-fold outputs equal the epilogue at one candidate delta.

    For each element, got is admissible when
        got == scaled_acc_epilogue(out, d, scale)
    for some d among scaled_acc_candidate_deltas (both zeros are tried where
    the candidates include zero). Every candidate is enumerated: the output
    must be exactly one candidate's result, not merely lie between the
    extreme candidates' results. Returns (ok_mask, n_candidates).
    """
    got = np.asarray(got_bits, dtype=np.uint16)
    out = np.asarray(out_bits, dtype=np.uint16)
    lo_d, hi_d, n_cand = scaled_acc_candidate_deltas(x_bits, b_bits, depth_factor)
    lo_key = _bf16_order_key(lo_d)
    ok = np.zeros(got.shape, dtype=bool)
    idx = np.arange(got.size)
    flat_n = n_cand.reshape(-1)
    c = 0
    while idx.size:
        d = _bf16_from_key(lo_key.reshape(-1)[idx] + c)
        o = out.reshape(-1)[idx]
        hit = scaled_acc_epilogue(o, d, scale) == got.reshape(-1)[idx]
        zero = d == 0
        if zero.any():   # -0 as well as +0
            neg = scaled_acc_epilogue(o[zero], np.full(int(zero.sum()), 0x8000, np.uint16), scale)
            hit[zero] |= neg == got.reshape(-1)[idx][zero]
        ok.reshape(-1)[idx[hit]] = True
        c += 1
        idx = idx[~hit & (flat_n[idx] > c)]
    return ok, n_cand


# ---------------------------------------------------------------------------
# split-K (gemm_bf16_splitk)
# ---------------------------------------------------------------------------

SPLITK_ALIGN = 64


def splitk_chunk(k: int, k_splits: int) -> int:
    """Length of each contiguous K chunk: ceil(K / k_splits) rounded up to 64.

    gemm_dense.rs page, dense_gemm_splitk: K is cut into k_splits partial
    products written to a k_splits*M*N FP32 workspace, then reduced. The page
    does not give the chunking; this library fixes contiguous chunks of this
    length (split s covers [s*Kc, min(K, (s+1)*Kc)); trailing chunks may be
    empty and then contribute +0).
    """
    if k_splits <= 0:
        raise ValueError("k_splits >= 1")
    c = -(-k // k_splits)
    return -(-c // SPLITK_ALIGN) * SPLITK_ALIGN


def gemm_splitk_planes_ref(a_bits, b_bits, k_splits: int) -> np.ndarray:
    """FP64 partial sums per chunk: planes[s] = sum over k in chunk s of A*B."""
    a = bf16_to_f64(a_bits)
    b = bf16_to_f64(b_bits)
    k = a.shape[1]
    kc = splitk_chunk(k, k_splits)
    planes = np.zeros((k_splits, a.shape[0], b.shape[0]), dtype=np.float64)
    for s in range(k_splits):
        lo, hi = min(k, s * kc), min(k, (s + 1) * kc)
        if hi > lo:
            planes[s] = a[:, lo:hi] @ b[:, lo:hi].T
    return planes


def splitk_reduce(planes_f32) -> np.ndarray:
    """C = bf16(((p0 + p1) + p2) + ...): planes summed in ascending split order in FP32."""
    p = np.asarray(planes_f32, dtype=np.float32)
    acc = p[0].copy()
    for s in range(1, p.shape[0]):
        acc = np.add(acc, p[s], dtype=np.float32)
    return f32_to_bf16(acc)


# ---------------------------------------------------------------------------
# block-scaled FP4 GEMM (gemm_fp4_blockscaled)
# ---------------------------------------------------------------------------

def gemm_fp4_ref(a_packed, sfa, b_packed, sfb) -> np.ndarray:
    """ref[i, j] = sum_k deq(A)[i, k] * deq(B)[j, k] in FP64.

    kernelbot NVFP4 page: the "SCALE FACTORS" loop (each element times the
    scale of its 16-element K group, plain [rows, K/16] layout) applied to both
    operands, then a dot product accumulated in FP32 (tl.dot_scaled in the
    persistent kernel). Every dequantized element and every product is exact
    in FP64.
    """
    a = dequant_fp4(a_packed, sfa)
    b = dequant_fp4(b_packed, sfb)
    return a @ b.T


def gemm_w4a16_ref(a_bits, b_packed, sfb, scale_2) -> np.ndarray:
    """ref[i, j] = s2 * sum_k A[i, k] * deq(B)[j, k] in FP64, s2 = fl32(scale_2).

    gemm_dense.rs page, w4a16_gemm doc comment: C = A @ dequant(B) with A
    [M, K] BF16 activations and B NVFP4 weights: E2M1 values, one FP8 (E4M3)
    scale per 16 K elements and one FP32 per-tensor scale. The page's
    lossless BF16-MMA variant forms each dequantized weight exactly in BF16,
    which fixes the reading: deq(B) = e2m1 * e4m3 (exact, the same per-group
    dequantization as the FP4 GEMM), and the per-tensor scale multiplies the
    FP32 dot product once, before the BF16 output rounding. B is [N, K/2]
    bytes (low nibble = even k), its scales [N, K/16].
    """
    s2 = float(np.float32(scale_2))
    return s2 * (bf16_to_f64(a_bits) @ dequant_fp4(b_packed, sfb).T)


def gemm_w4a16_exact(a_bits, b_packed, sfb, scale_2) -> np.ndarray:
    """BF16 C = bf16(fl32(s2 * acc)) for inputs whose dot products acc are
    exact in FP32 whatever the summation order (the caller picks such data,
    e.g. grid activations and power-of-two scales). Raises ValueError if a
    dot product is not even representable in FP32."""
    acc = bf16_to_f64(a_bits) @ dequant_fp4(b_packed, sfb).T
    acc32 = acc.astype(np.float32)
    if not np.array_equal(acc32.astype(np.float64), acc):
        raise ValueError("dot products are not exact in FP32")
    prod = np.float32(scale_2) * acc32        # one IEEE single multiply, RNE
    return f32_to_bf16(prod.astype(np.float32))


def gemm_w4a16_t_ref(a_bits, bt, sfbt, n: int, scale_2) -> np.ndarray:
    """gemm_w4a16_ref for weights in the transposed layout (dequant_fp4_t):
    ref[i, j] = s2 * sum_k A[i, k] * w[j, k] in FP64, s2 = fl32(scale_2)."""
    s2 = float(np.float32(scale_2))
    return s2 * (bf16_to_f64(a_bits) @ dequant_fp4_t(bt, sfbt, n).T)


def gemm_fp4_splitk_planes_ref(a_packed, sfa, b_packed, sfb, k_splits: int) -> np.ndarray:
    """FP64 partial sums per K chunk of the FP4 GEMM (chunk rule of
    splitk_chunk): planes[s] = sum over k in chunk s of deq(A) * deq(B).
    Each plane is the FP4 definition (gemm_fp4_ref) on its own K range."""
    a = dequant_fp4(a_packed, sfa)
    b = dequant_fp4(b_packed, sfb)
    k = a.shape[1]
    kc = splitk_chunk(k, k_splits)
    planes = np.zeros((k_splits, a.shape[0], b.shape[0]), np.float64)
    for s in range(k_splits):
        lo, hi = min(k, s * kc), min(k, (s + 1) * kc)
        planes[s] = a[:, lo:hi] @ b[:, lo:hi].T
    return planes
