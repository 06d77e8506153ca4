// Plain C++17 CPU oracle of every operation the GEMM library computes.
//
// TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the tests, the smoke
// check and the benchmark's CPU-baseline leg load this library. It shares no
// code, header, table or constant with the HIP library and includes none of
// its files; both sides receive the same seeded input bytes.
//
// Built with `g++ -O2 -std=c++17 -ffp-contract=off` and no fast-math, for
// x86-64 SSE scalar arithmetic: every float operation written below is one
// IEEE binary32 operation rounded to nearest even, and no multiply is fused
// with an add.
//
// Every routine is the definition of its operation written out as loops:
// decode each stored input from its bit fields, then sum products in
// ascending k. Where the pages leave the accumulation order open the sum is
// taken in FP64 (every BF16 x BF16 and every dequantized E2M1*E4M3 product is
// exact in FP64); the order-preserving mode is the literal FP32 recurrence.
// Layout: A [M, K], B [N, K] (both K-contiguous), C [M, N], C = A * B^T
// (gemm_dense.rs page, doc comment of the dense BF16 GEMM).
//
// `threads` splits the output rows into contiguous ranges, one std::thread
// each (0 = one per hardware thread); the work of each output is unchanged.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

// BF16 is the upper half of an IEEE binary32 pattern: widening is exact.
float bf16_bits_to_f32(uint16_t h) {
    const uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// FP32 -> BF16 bits, round to nearest, ties to even; NaN -> quiet NaN of the
// same sign (the pages state no mode for their BF16 casts; this is the
// reading taken throughout).
uint16_t f32_to_bf16_bits(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) return (uint16_t)((u >> 16) | 0x0040u);
    const uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

// E2M1 (OCP microscaling FP4): sign bit 3, exponent bits 2..1 (bias 1),
// mantissa bit 0; exponent 0 is the subnormal m * 0.5. No Inf or NaN.
double e2m1_value(unsigned code) {
    const unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    const double mag = e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * std::ldexp(1.0, (int)e - 1);
    return s ? -mag : mag;
}

// E4M3FN (OCP FP8): sign bit 7, exponent bits 6..3 (bias 7), mantissa bits
// 2..0; exponent 0 is the subnormal m * 2^-9; S.1111.111 is NaN; no Inf.
double e4m3fn_value(unsigned byte) {
    const unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
    double mag;
    if (e == 15 && m == 7)
        mag = std::numeric_limits<double>::quiet_NaN();
    else if (e == 0)
        mag = m * std::ldexp(1.0, -9);
    else
        mag = (1.0 + m / 8.0) * std::ldexp(1.0, (int)e - 7);
    return s ? -mag : mag;
}

// Block-scaled FP4 element k of a row: the E2M1 code in nibble k of the packed
// bytes (element 2t in the LOW nibble of byte t) times the E4M3FN scale of its
// 16-element group k / 16 (kernelbot NVFP4 page, "SCALE FACTORS").
double fp4_element(const uint8_t* packed_row, const uint8_t* scale_row, int64_t k) {
    const uint8_t byte = packed_row[k / 2];
    const unsigned code = (k % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
    return e2m1_value(code) * e4m3fn_value(scale_row[k / 16]);
}

// Runs body(row) for rows [0, rows) over `threads` contiguous ranges.
template <class F>
void for_rows(int64_t rows, int threads, F body) {
    int t = threads > 0 ? threads : (int)std::max(1u, std::thread::hardware_concurrency());
    t = (int)std::min<int64_t>(t, std::max<int64_t>(rows, 1));
    if (t <= 1) {
        for (int64_t i = 0; i < rows; ++i) body(i);
        return;
    }
    std::vector<std::thread> pool;
    for (int w = 0; w < t; ++w) {
        const int64_t lo = rows * w / t, hi = rows * (w + 1) / t;
        pool.emplace_back([=]() {
            for (int64_t i = lo; i < hi; ++i) body(i);
        });
    }
    for (auto& th : pool) th.join();
}

// Decoded FP64 copy of a BF16 matrix (every value exact).
std::vector<double> decode_bf16(const uint16_t* x, int64_t rows, int64_t k) {
    std::vector<double> out((size_t)(rows * k));
    for (int64_t i = 0; i < rows * k; ++i) out[(size_t)i] = (double)bf16_bits_to_f32(x[i]);
    return out;
}

// Decoded FP64 copy of a block-scaled FP4 matrix (every value exact).
std::vector<double> decode_fp4(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t k) {
    std::vector<double> out((size_t)(rows * k));
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t kk = 0; kk < k; ++kk)
            out[(size_t)(i * k + kk)] = fp4_element(packed + i * (k / 2), scales + i * (k / 16), kk);
    return out;
}

// C[i, j] = sum over k in [k0, k1) of a[i, k] * b[j, k] in FP64, ascending k.
void dot_rows_f64(const double* a, const double* b, double* c, int64_t m, int64_t n, int64_t k, int64_t k0,
                  int64_t k1, int threads) {
    for_rows(m, threads, [&](int64_t i) {
        const double* ar = a + i * k;
        for (int64_t j = 0; j < n; ++j) {
            const double* br = b + j * k;
            double s = 0.0;
            for (int64_t kk = k0; kk < k1; ++kk) s += ar[kk] * br[kk];
            c[i * n + j] = s;
        }
    });
}

}  // namespace

extern "C" {

// ---- codecs (exposed for the pins) -----------------------------------------

float orc_bf16_to_f32(uint16_t h) { return bf16_bits_to_f32(h); }
uint16_t orc_f32_to_bf16(float f) { return f32_to_bf16_bits(f); }
double orc_e2m1(unsigned code) { return e2m1_value(code & 15u); }
double orc_e4m3fn(unsigned byte) { return e4m3fn_value(byte & 255u); }

void orc_bf16_to_f32_array(const uint16_t* x, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits_to_f32(x[i]);
}

void orc_f32_to_bf16_array(const float* x, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_bits(x[i]);
}

void orc_dequant_fp4(const uint8_t* packed, const uint8_t* scales, double* out, int64_t rows, int64_t k) {
    const std::vector<double> v = decode_fp4(packed, scales, rows, k);
    std::copy(v.begin(), v.end(), out);
}

int orc_hardware_threads() { return (int)std::max(1u, std::thread::hardware_concurrency()); }

// ---- dense BF16 GEMM ----------------------------------------------------------

// ref[i, j] = sum_k A[i, k] * B[j, k] in FP64 (sm121a_matmul.py page, kernel
// body: FP32 accumulator over K blocks, K tail masked to zero; gemm_dense.rs
// page, dense BF16 GEMM doc: C = A @ B^T). Left unrounded; the BF16 output
// rounding is inside the tolerance.
void orc_gemm_bf16_f64(const uint16_t* A, const uint16_t* B, double* C, int64_t M, int64_t N, int64_t K,
                       int threads) {
    const std::vector<double> a = decode_bf16(A, M, K), b = decode_bf16(B, N, K);
    dot_rows_f64(a.data(), b.data(), C, M, N, K, 0, K, threads);
}

// Row sample of the same definition: output rows rows[0..nrows) only (used to
// time the oracle on a bounded part of a large problem).
void orc_gemm_bf16_f64_rows(const uint16_t* A, const uint16_t* B, const int64_t* rows, double* C, int64_t nrows,
                            int64_t N, int64_t K, int threads) {
    const std::vector<double> b = decode_bf16(B, N, K);
    for_rows(nrows, threads, [&](int64_t r) {
        std::vector<double> ar((size_t)K);
        const uint16_t* src = A + rows[r] * K;
        for (int64_t kk = 0; kk < K; ++kk) ar[(size_t)kk] = (double)bf16_bits_to_f32(src[kk]);
        for (int64_t j = 0; j < N; ++j) {
            const double* br = b.data() + j * K;
            double s = 0.0;
            for (int64_t kk = 0; kk < K; ++kk) s += ar[(size_t)kk] * br[kk];
            C[r * N + j] = s;
        }
    });
}

// ---- order-preserving mode --------------------------------------------------

// gemm_dense.rs page, doc comment of dense_gemm_router: the scalar kernel's
// math and per-output order (strict k = 0..K-1), built without FMA. For each
// output: acc = +0.0f; for k ascending, p = fl32(a * b), acc = fl32(acc + p).
// C32 receives the FP32 sums; C16 (if not null) their BF16 rounding.
void orc_gemm_ordered(const uint16_t* A, const uint16_t* B, float* C32, uint16_t* C16, int64_t M, int64_t N,
                      int64_t K, int threads) {
    for_rows(M, threads, [&](int64_t i) {
        for (int64_t j = 0; j < N; ++j) {
            float acc = 0.0f;
            for (int64_t kk = 0; kk < K; ++kk) {
                const float p = bf16_bits_to_f32(A[i * K + kk]) * bf16_bits_to_f32(B[j * K + kk]);
                acc = acc + p;
            }
            C32[i * N + j] = acc;
            if (C16) C16[i * N + j] = f32_to_bf16_bits(acc);
        }
    });
}

// ---- fused LoRA fold epilogue -------------------------------------------------

// gemm_dense.rs page, doc comment of dense_gemm_tc_scaled_acc: the delta is
// rounded to BF16 before the scale, as a BF16 scratch tensor followed by a
// BF16 scaled add would: out_new = bf16(fl32(f32(out) + fl32(scale * f32(d)))),
// one FP32 multiply, one FP32 add, one BF16 rounding.
void orc_scaled_acc_epilogue(const uint16_t* out, const uint16_t* delta_bf16, float scale, uint16_t* out_new,
                             int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        const float p = scale * bf16_bits_to_f32(delta_bf16[i]);
        const float s = bf16_bits_to_f32(out[i]) + p;
        out_new[i] = f32_to_bf16_bits(s);
    }
}

// ---- split-K -------------------------------------------------------------------

// Chunk length: ceil(K / k_splits) rounded up to a multiple of 64; split s
// covers [s*Kc, min(K, (s+1)*Kc)) (gemm_dense.rs page, dense_gemm_splitk gives
// k_splits FP32 partial planes but not the chunking; this is the reading).
int64_t orc_splitk_chunk(int64_t K, int64_t k_splits) {
    if (k_splits <= 0) return -1;
    const int64_t c = (K + k_splits - 1) / k_splits;
    return (c + 63) / 64 * 64;
}

// planes[s][i][j] = FP64 sum over chunk s (empty chunks give +0).
void orc_splitk_planes_f64(const uint16_t* A, const uint16_t* B, double* planes, int64_t M, int64_t N, int64_t K,
                           int64_t k_splits, int threads) {
    const std::vector<double> a = decode_bf16(A, M, K), b = decode_bf16(B, N, K);
    const int64_t kc = orc_splitk_chunk(K, k_splits);
    for (int64_t s = 0; s < k_splits; ++s) {
        const int64_t lo = std::min(K, s * kc), hi = std::min(K, (s + 1) * kc);
        dot_rows_f64(a.data(), b.data(), planes + s * M * N, M, N, K, lo, hi, threads);
    }
}

// C = bf16(((p0 + p1) + p2) + ...): FP32 planes summed in ascending split order.
void orc_splitk_reduce(const float* planes, int64_t k_splits, int64_t count, uint16_t* C) {
    for (int64_t e = 0; e < count; ++e) {
        float acc = planes[e];
        for (int64_t s = 1; s < k_splits; ++s) acc = acc + planes[s * count + e];
        C[e] = f32_to_bf16_bits(acc);
    }
}

// ---- block-scaled FP4 and W4A16 ----------------------------------------------

// ref[i, j] = sum_k deq(A)[i, k] * deq(B)[j, k] in FP64 over [k0, k1)
// (kernelbot NVFP4 page: each E2M1 element times the E4M3 scale of its
// 16-element group, then an FP32-accumulated dot product). A [M, K/2] bytes,
// SFA [M, K/16], B [N, K/2], SFB [N, K/16].
void orc_gemm_fp4_f64(const uint8_t* Aq, const uint8_t* SFA, const uint8_t* Bq, const uint8_t* SFB, double* C,
                      int64_t M, int64_t N, int64_t K, int64_t k0, int64_t k1, int threads) {
    const std::vector<double> a = decode_fp4(Aq, SFA, M, K), b = decode_fp4(Bq, SFB, N, K);
    dot_rows_f64(a.data(), b.data(), C, M, N, K, k0, k1, threads);
}

// gemm_dense.rs page, w4a16_gemm doc: BF16 activations times NVFP4 weights
// (E2M1, an E4M3 scale per 16 K elements, an FP32 per-tensor scale). Each
// weight is dequantized exactly (e2m1 * e4m3, what the page's lossless
// BF16-MMA variant needs); s2 = fl32(scale_2) multiplies the dot product once.
// ref[i, j] = s2 * sum_k A[i, k] * deq(B)[j, k], in FP64.
void orc_gemm_w4a16_f64(const uint16_t* A, const uint8_t* Bq, const uint8_t* SFB, float scale_2, double* C,
                        int64_t M, int64_t N, int64_t K, int threads) {
    const std::vector<double> a = decode_bf16(A, M, K), b = decode_fp4(Bq, SFB, N, K);
    dot_rows_f64(a.data(), b.data(), C, M, N, K, 0, K, threads);
    const double s2 = (double)scale_2;
    for (int64_t e = 0; e < M * N; ++e) C[e] = s2 * C[e];
}

}  // extern "C"
