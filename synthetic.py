"""Seeded synthetic inputs shared by the tests, the bench and smoke().

This module draws random numbers and stores them in the input formats the
library consumes (BF16 bits, packed E2M1 bytes, E4M3FN scale bytes). It holds
none of the GEMM arithmetic: narrowing a drawn float to BF16 or E4M3FN is done
by torch's own dtype conversion (round to nearest even), so neither the oracle
nor the HIP path supplies any of it.

Every tensor is a function of (seed, tensor id) only: a Philox-4x64 counter
generator (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3",
SC'11) keyed by that pair, so both sides of a parity check see identical bytes.

The workloads below are the shapes and value distributions of the GEMMs the
pages measure:
  - sm121a_matmul.py page, module docstring: the per-step shape list of a
    2B-class decoder (MLP gate/up, MLP down, Q/O and GQA K/V projections);
  - gemm_dense.rs page, doc comments of dense_gemm_tc_scaled_acc (LoRA fold at
    n = 17408) and dense_gemm_router (router at M = 4510 and 2255, [M,2048] x
    [2048,256]);
  - kernelbot NVFP4 GEMM page (submission 123329), "SCALE FACTORS" section:
    E2M1 elements with one E4M3 scale per 16 K elements;
  - gemm_dense.rs page, w4a16_gemm doc comments: BF16 activations times NVFP4
    weights, measured at the qkvz projection (K = 2048, N = 12288, ISL 1016).
"""
from __future__ import annotations

import numpy as np
import torch

# tensor ids inside one workload
TID_A, TID_B, TID_OUT, TID_B2, TID_SFA, TID_SFB = 0, 1, 2, 3, 4, 5


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    key = np.array([seed & 0xFFFFFFFFFFFFFFFF, tensor_id & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def _to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, std: float, seed: int, tensor_id: int) -> np.ndarray:
    """BF16 bit patterns of N(0, std^2) draws (std is the standard deviation)."""
    g = _rng(seed, tensor_id)
    x = g.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(std)
    return _to_bf16_bits(x)


def grid_bf16(shape, lo: int, hi: int, exp2: int, seed: int, tensor_id: int) -> np.ndarray:
    """BF16 bits of j * 2**exp2 with j uniform over the integers lo..hi.

    With |j| <= 255 every value is exact in BF16; with small |j| and exponents,
    sums of their products are exact in FP32 in any order.
    """
    g = _rng(seed, tensor_id)
    j = g.integers(lo, hi + 1, size=shape, dtype=np.int64)
    x = (j.astype(np.float64) * (2.0 ** exp2)).astype(np.float32)
    return _to_bf16_bits(x)


def fp4_packed(rows: int, k: int, seed: int, tensor_id: int) -> np.ndarray:
    """[rows, k/2] bytes, each uniform over 0..255 (both nibbles uniform over 16 codes)."""
    assert k % 2 == 0
    g = _rng(seed, tensor_id)
    return g.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)


def e4m3_uniform(rows: int, groups: int, lo: float, hi: float, seed: int, tensor_id: int) -> np.ndarray:
    """[rows, groups] E4M3FN bytes of u ~ U(lo, hi), narrowed by torch (RNE)."""
    g = _rng(seed, tensor_id)
    u = g.uniform(lo, hi, size=(rows, groups)).astype(np.float32)
    return torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_choice(rows: int, groups: int, choices, seed: int, tensor_id: int) -> np.ndarray:
    """[rows, groups] bytes drawn uniformly from the given E4M3FN byte codes."""
    g = _rng(seed, tensor_id)
    c = np.asarray(choices, dtype=np.uint8)
    return c[g.integers(0, len(c), size=(rows, groups))]


def sample_rows(m: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct row indices: always 0 and m-1, and count-2 more drawn
    uniformly without replacement from 1..m-2 (all rows when m <= count)."""
    if m <= count:
        return np.arange(m, dtype=np.int64)
    g = _rng(seed, 99)
    mid = g.choice(np.arange(1, m - 1, dtype=np.int64), size=count - 2, replace=False)
    return np.concatenate([[0], np.sort(mid), [m - 1]]).astype(np.int64)


# ---------------------------------------------------------------------------
# Workload recipes (shapes, distributions, seeds).  Workload i uses seed i.
# ---------------------------------------------------------------------------

def dense_small(seed: int = 0):
    """A[128,512], B[256,512] ~ N(0,1)/sqrt(512); C[128,256]."""
    s = 1.0 / np.sqrt(512.0)
    return normal_bf16((128, 512), s, seed, TID_A), normal_bf16((256, 512), s, seed, TID_B)


def attn_proj(seed: int = 1, n: int = 2048, m: int = 5120, k: int = 2048):
    """Activations A[m,k] ~ N(0,1), weights B[n,k] ~ N(0,0.02) (Q/O: n=2048, K/V: n=512)."""
    return normal_bf16((m, k), 1.0, seed, TID_A), normal_bf16((n, k), 0.02, seed, TID_B if n != 512 else TID_B2)


def mlp_gate_up(seed: int = 2, m: int = 5120, n: int = 11008, k: int = 2048):
    return normal_bf16((m, k), 1.0, seed, TID_A), normal_bf16((n, k), 0.02, seed, TID_B)


def mlp_down(seed: int = 2, m: int = 5120, n: int = 2048, k: int = 11008):
    return normal_bf16((m, k), 1.0, seed, TID_OUT), normal_bf16((n, k), 0.02, seed, TID_B2)


def lora_fold(seed: int = 3, m: int = 2048, n: int = 17408, r: int = 64):
    """out[m,n] ~ N(0,1); X[m,r], Bl[n,r] ~ N(0,0.1); scale 2.0."""
    out = normal_bf16((m, n), 1.0, seed, TID_OUT)
    x = normal_bf16((m, r), 0.1, seed, TID_A)
    bl = normal_bf16((n, r), 0.1, seed, TID_B)
    return out, x, bl, 2.0


def router(seed: int = 3, m: int = 4510, n: int = 256, k: int = 2048):
    """X[m,k] ~ N(0,1), W[n,k] ~ N(0,0.02)."""
    return normal_bf16((m, k), 1.0, seed, 10 + TID_A), normal_bf16((n, k), 0.02, seed, 10 + TID_B)


def fp4_gemm(seed: int = 4, m: int = 4096, n: int = 4096, k: int = 8192):
    """Packed E2M1 A[m,k/2], B[n,k/2] (uniform bytes); E4M3FN scales U(2^-4, 2^4)."""
    a = fp4_packed(m, k, seed, TID_A)
    b = fp4_packed(n, k, seed, TID_B)
    sfa = e4m3_uniform(m, k // 16, 2.0 ** -4, 2.0 ** 4, seed, TID_SFA)
    sfb = e4m3_uniform(n, k // 16, 2.0 ** -4, 2.0 ** 4, seed, TID_SFB)
    return a, sfa, b, sfb


# Per-tensor FP32 scale of the W4A16 weights (an arbitrary non-power-of-two
# value of the size an NVFP4 global scale takes).
W4A16_SCALE_2 = 0.0123


def w4a16_gemm(seed: int = 5, m: int = 1016, n: int = 12288, k: int = 2048):
    """W4A16: BF16 activations A[m,k] ~ N(0,1); NVFP4 weights B[n,k/2]
    (uniform bytes) with E4M3FN scales U(2^-4, 2^4) per 16 K elements, and the
    per-tensor FP32 scale W4A16_SCALE_2. Default shape: the gemm_dense.rs
    page's qkvz projection (K = 2048, N = 12288) at ISL = 1016."""
    a = normal_bf16((m, k), 1.0, seed, TID_A)
    b = fp4_packed(n, k, seed, TID_B)
    sfb = e4m3_uniform(n, k // 16, 2.0 ** -4, 2.0 ** 4, seed, TID_SFB)
    return a, b, sfb, W4A16_SCALE_2


def fp4_decode(seed: int = 6, m: int = 128, n: int = 7168, k: int = 16384):
    """The kernelbot NVFP4 page's decode-sized problems (L=1, M=128; N, K =
    7168, 16384 or 4096, 7168): operands and scales drawn as for fp4_gemm."""
    return fp4_gemm(seed=seed, m=m, n=n, k=k)
