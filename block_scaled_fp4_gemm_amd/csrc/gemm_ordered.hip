// Order-preserving GEMM (router logits) on the FP32 vector ALU.
//
// gemm_dense.rs page, doc comment of dense_gemm_router: each output is the
// strict k = 0..K-1 FP32 recurrence of the scalar dense kernel, built without
// FMA contraction (bit-identical to it), made faster by register blocking and
// vectorized staging; matrix cores reassociate and are not allowed here.
//
// Per output: acc = +0.0f; for k ascending: acc = fl32(acc + fl32(a*b)).
// This file is compiled with FP contraction off and, in addition, every
// product and sum goes through __fmul_rn / __fadd_rn, so no multiply-add can
// be fused. FP32 denormals are kept (the library is built without flushing).
//
// Design (CDNA4), two forms. Tile form: a workgroup of 16x16 threads owns a
// (16*RM) x (16*RN) output tile; each thread keeps an RM x RN block of
// accumulators. K is walked in steps of KT; each step stages A and B rows as
// FP32 into LDS, row-major with a padded pitch. Scalar-A form (K % 8 == 0):
// only B goes through LDS; A's values come through scalar loads into SGPRs,
// which every lane of a wave reads as a broadcast operand. In both the
// per-output k order is untouched by the tiling: steps are visited in
// ascending k and, inside a step, k ascends.
#include <cmath>

#include "bg_internal.hpp"
#include "tile_order.hpp"

#pragma clang fp contract(off)

namespace bg {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int KT = 32;   // K elements per LDS step

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __builtin_bit_cast(float, h << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);   // v_cvt_pk_bf16_f32, nearest even
}

// Stage rows [row0, row0+ROWS) x k in [k0, k0+KT) of a [nrows, K] BF16 matrix
// into lds[row][LDK] as FP32 (row-major, LDK = KT + 4 floats per row).
// Positions with k >= K, or rows >= nrows, get 0. A unit is 8 consecutive k
// of one row, written as two 16-byte stores; consecutive threads take
// consecutive rows.
template <int ROWS, int NT, int LDK>
__device__ __forceinline__ void stage(float* lds, const uint16_t* src, int row0, int nrows,
                                      int K, int k0, bool vec, int tid) {
    constexpr int UNITS = ROWS * (KT / 8);
#pragma unroll
    for (int i = 0; i < (UNITS + NT - 1) / NT; ++i) {
        const int u = tid + i * NT;
        if (UNITS % NT != 0 && u >= UNITS) break;
        const int row = u % ROWS, c = u / ROWS;
        const int grow = row0 + row, gk = k0 + c * 8;
        uint32_t h[8];
        if (vec && grow < nrows && gk + 7 < K) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(src + (int64_t)grow * K + gk);
            h[0] = w.x & 0xFFFFu; h[1] = w.x >> 16; h[2] = w.y & 0xFFFFu; h[3] = w.y >> 16;
            h[4] = w.z & 0xFFFFu; h[5] = w.z >> 16; h[6] = w.w & 0xFFFFu; h[7] = w.w >> 16;
        } else {
#pragma unroll
            for (int x = 0; x < 8; ++x)
                h[x] = (grow < nrows && gk + x < K) ? (uint32_t)src[(int64_t)grow * K + gk + x] : 0u;
        }
        float* dst = lds + row * LDK + c * 8;
        *reinterpret_cast<f32x4*>(dst) = f32x4{bf16_bits_to_f32(h[0]), bf16_bits_to_f32(h[1]),
                                               bf16_bits_to_f32(h[2]), bf16_bits_to_f32(h[3])};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{bf16_bits_to_f32(h[4]), bf16_bits_to_f32(h[5]),
                                                   bf16_bits_to_f32(h[6]), bf16_bits_to_f32(h[7])};
    }
}

// A workgroup of 16 x 16 threads owns a (16*RM) x (16*RN) output tile; thread
// (tx, ty) keeps outputs rows ty + 16*i (i < RM) x cols tx + 16*j (j < RN).
// Each 16-byte LDS read brings four consecutive k of one row, so a thread
// reads RM + RN vectors per four k and then runs the 4*RM*RN multiply-add
// pairs in ascending k. With a 36-float row pitch the 16 rows that the 16
// lanes of a row group read start in 16 disjoint groups of four banks (A
// rows are shared by 16 lanes and broadcast). The register block size is
// chosen per shape so the number of waves lands just below a multiple of the
// SIMD count: the work is pure VALU, and a SIMD holding one wave more than
// the others sets the runtime.
template <int RM, int RN, bool F32_OUT>
__global__ void __launch_bounds__(256)
gemm_ordered_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* C,
                    int M, int N, int K, int tiles_n) {
    constexpr int TM = 16 * RM, TN = 16 * RN;
    constexpr int LDK = KT + 4;
    __shared__ __attribute__((aligned(16))) float sA[TM * LDK];
    __shared__ __attribute__((aligned(16))) float sB[TN * LDK];

    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    // Dispatch places workgroup b on XCD b % 8; renumbered so each XCD holds
    // one contiguous range of tiles, the column tiles of a row block (which
    // share its A rows) run on the same XCD and hit in its L2.
    int tm, tn;
    tile_of<ORDER_ROWS>((int)blockIdx.x, (int)gridDim.x / tiles_n, tiles_n, tm, tn);
    const int m0 = tm * TM, n0 = tn * TN;
    const bool vec = (K & 7) == 0;

    float acc[RM][RN];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j) acc[i][j] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += KT) {
        __syncthreads();
        stage<TM, 256, LDK>(sA, A, m0, M, K, k0, vec, tid);
        stage<TN, 256, LDK>(sB, B, n0, N, K, k0, vec, tid);
        __syncthreads();
        // Groups of four k; past K the staged values are zero, and adding the
        // product +0 leaves every accumulator unchanged (an accumulator that
        // starts at +0 never becomes -0 under round to nearest).
        const int kn = min(KT, K - k0);
#pragma unroll 2
        for (int kc = 0; kc < kn; kc += 4) {
            f32x4 a[RM], b[RN];
#pragma unroll
            for (int i = 0; i < RM; ++i) a[i] = *reinterpret_cast<const f32x4*>(&sA[(ty + 16 * i) * LDK + kc]);
#pragma unroll
            for (int j = 0; j < RN; ++j) b[j] = *reinterpret_cast<const f32x4*>(&sB[(tx + 16 * j) * LDK + kc]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < RM; ++i)
#pragma unroll
                    for (int j = 0; j < RN; ++j)
                        acc[i][j] = __fadd_rn(acc[i][j], __fmul_rn(a[i][q], b[j][q]));
        }
    }

#pragma unroll
    for (int i = 0; i < RM; ++i) {
        const int m = m0 + ty + 16 * i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < RN; ++j) {
            const int n = n0 + tx + 16 * j;
            if (n >= N) continue;
            if constexpr (F32_OUT)
                reinterpret_cast<float*>(C)[(int64_t)m * N + n] = acc[i][j];
            else
                reinterpret_cast<uint16_t*>(C)[(int64_t)m * N + n] = f32_to_bf16_rne(acc[i][j]);
        }
    }
}

// Second form, for K % 8 == 0: A's rows through the scalar unit. A wave owns
// RM output rows and 64 columns (one per lane); the four waves of a
// workgroup take 4*RM consecutive rows and share one 64-column B block in LDS
// (FP32, the same padded pitch as above). A's values arrive by scalar loads
// and are widened in scalar registers, so the 64 lanes multiply one SGPR
// operand (a broadcast that costs no LDS bandwidth): per four k a lane reads
// one 16-byte B vector from LDS, where the tile form reads RM + RN. Each
// thread loads its 8-element B unit one step ahead into registers and writes
// it to LDS at the start of the next step, so that load's latency is covered
// by a step of arithmetic; the B block alternates between two LDS buffers, so
// each step needs one barrier. The order per output is the same strict
// ascending k.
//
// Measured on MI355X against the tile form's best block (same bits), RM = 3:
// 4510 x 256 x 2048 142 -> 116 us, 2255 x 256 x 2048 104 -> 68 us (one B
// buffer and two barriers per step: 121 and 73 us; B loaded at the start of
// its own step as well: 126 and 79 us). Two columns per lane (half the
// scalar widening per multiply), 16-wide K steps with RM = 4..6, and a form
// that also prefetched A's words a step ahead were all slower; RM = 4 runs
// out of SGPRs (spills to VGPR lanes).
template <int RM, bool F32_OUT>
__global__ void __launch_bounds__(256)
gemm_ordered_sa_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* C,
                       int M, int N, int K, int tiles_n) {
    constexpr int TN = 64;
    constexpr int LDK = KT + 4;
    constexpr int W = KT / 2;   // 32-bit words of one A row per step
    __shared__ __attribute__((aligned(16))) float sBuf[2 * TN * LDK];   // two B buffers: one barrier per step

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_of<ORDER_ROWS>((int)blockIdx.x, (int)gridDim.x / tiles_n, tiles_n, tm, tn);
    const int r0 = tm * 4 * RM + wave * RM, n0 = tn * TN;

    // rows past M read row M - 1 (in bounds) and are not stored
    const uint32_t* arow[RM];
#pragma unroll
    for (int i = 0; i < RM; ++i)
        arow[i] = reinterpret_cast<const uint32_t*>(A + (int64_t)min(r0 + i, M - 1) * K);

    float acc[RM];
#pragma unroll
    for (int i = 0; i < RM; ++i) acc[i] = 0.0f;

    // this thread's B unit: k0 + 8*bc .. k0 + 8*bc + 7 of column n0 + brow,
    // zero past N or K (K % 8 == 0: a unit lies wholly inside or past K)
    const int brow = tid % TN, bc = tid / TN;
    const int bn = n0 + brow;
    const uint16_t* bsrc = B + (int64_t)min(bn, N - 1) * K + bc * 8;
    auto load_b = [&](int kk) -> u32x4 {
        if (bn < N && kk + bc * 8 < K) return *reinterpret_cast<const u32x4*>(bsrc + kk);
        return u32x4{0u, 0u, 0u, 0u};
    };
    u32x4 bw = load_b(0);
    int buf = 0;
    for (int k0 = 0; k0 < K; k0 += KT, buf ^= 1) {
        // buffer `buf` was last read in the step before the previous one,
        // which every wave finished before the previous step's barrier
        float* sB = sBuf + buf * TN * LDK;
        // this step's A words (two k each), zero past K; issued before the
        // barrier so they arrive while B is written to LDS
        uint32_t aw[RM][W];
        const int kw = k0 >> 1;
        if (k0 + KT <= K) {
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < W; ++j) aw[i][j] = arow[i][kw + j];
        } else {
            const int nw = (K - k0) >> 1;
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < W; ++j) aw[i][j] = j < nw ? arow[i][kw + j] : 0u;
        }
        {
            float* dst = &sB[brow * LDK + bc * 8];
            *reinterpret_cast<f32x4*>(dst) = f32x4{bf16_bits_to_f32(bw.x & 0xFFFFu), bf16_bits_to_f32(bw.x >> 16),
                                                   bf16_bits_to_f32(bw.y & 0xFFFFu), bf16_bits_to_f32(bw.y >> 16)};
            *reinterpret_cast<f32x4*>(dst + 4) = f32x4{bf16_bits_to_f32(bw.z & 0xFFFFu), bf16_bits_to_f32(bw.z >> 16),
                                                       bf16_bits_to_f32(bw.w & 0xFFFFu), bf16_bits_to_f32(bw.w >> 16)};
        }
        __syncthreads();
        if (k0 + KT < K) bw = load_b(k0 + KT);
        // past K both operands are zero: the products are +0 and leave every
        // accumulator unchanged
#pragma unroll
        for (int kc = 0; kc < KT; kc += 4) {
            const f32x4 b = *reinterpret_cast<const f32x4*>(&sB[lane * LDK + kc]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < RM; ++i) {
                    const uint32_t w = aw[i][(kc + q) >> 1];
                    const float a = __builtin_bit_cast(float, ((kc + q) & 1) ? (w & 0xFFFF0000u) : (w << 16));
                    acc[i] = __fadd_rn(acc[i], __fmul_rn(a, b[q]));
                }
        }
    }

    const int n = n0 + lane;
    if (n >= N) return;
#pragma unroll
    for (int i = 0; i < RM; ++i) {
        const int m = r0 + i;
        if (m >= M) break;
        if constexpr (F32_OUT)
            reinterpret_cast<float*>(C)[(int64_t)m * N + n] = acc[i];
        else
            reinterpret_cast<uint16_t*>(C)[(int64_t)m * N + n] = f32_to_bf16_rne(acc[i]);
    }
}

template <int RM>
hipError_t launch_ordered_sa(const uint16_t* A, const uint16_t* B, void* C, bool f32_out, int M, int N,
                             int K, hipStream_t stream) {
    const int tiles_m = (M + 4 * RM - 1) / (4 * RM);
    const int tiles_n = (N + 63) / 64;
    dim3 grid((unsigned)(tiles_m * tiles_n));
    if (f32_out)
        hipLaunchKernelGGL((gemm_ordered_sa_kernel<RM, true>), grid, dim3(256), 0, stream, A, B, C, M, N,
                           K, tiles_n);
    else
        hipLaunchKernelGGL((gemm_ordered_sa_kernel<RM, false>), grid, dim3(256), 0, stream, A, B, C, M, N,
                           K, tiles_n);
    return hipGetLastError();
}

template <int RM, int RN>
hipError_t launch_ordered_cfg(const uint16_t* A, const uint16_t* B, void* C, bool f32_out, int M,
                              int N, int K, hipStream_t stream) {
    const int tiles_m = (M + 16 * RM - 1) / (16 * RM);
    const int tiles_n = (N + 16 * RN - 1) / (16 * RN);
    dim3 grid((unsigned)(tiles_m * tiles_n));
    if (f32_out)
        hipLaunchKernelGGL((gemm_ordered_kernel<RM, RN, true>), grid, dim3(256), 0, stream, A, B, C,
                           M, N, K, tiles_n);
    else
        hipLaunchKernelGGL((gemm_ordered_kernel<RM, RN, false>), grid, dim3(256), 0, stream, A, B,
                           C, M, N, K, tiles_n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K reduction: C = bf16(((P0 + P1) + P2) + ...), one FP32 add per plane
// in ascending split order (gemm_dense.rs page, dense_gemm_splitk phase 2:
// reduce the FP32 workspace and write BF16). Four columns per thread.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ ws, uint16_t* __restrict__ C, int64_t count,
                     int splits, bool vec) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t e0 = q * 4;
    if (e0 >= count) return;
    if (vec && e0 + 3 < count) {
        f32x4 s = *reinterpret_cast<const f32x4*>(ws + e0);
        // four planes' loads in flight before their adds (same ascending
        // order): 128 x 4096 x 7168 FP4 decode at k_splits 12, 25.9 -> 25.1 us
        int p = 1;
        for (; p + 3 < splits; p += 4) {
            f32x4 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const f32x4*>(ws + (int64_t)(p + q) * count + e0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s.x = __fadd_rn(s.x, v[q].x);
                s.y = __fadd_rn(s.y, v[q].y);
                s.z = __fadd_rn(s.z, v[q].z);
                s.w = __fadd_rn(s.w, v[q].w);
            }
        }
        for (; p < splits; ++p) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(ws + (int64_t)p * count + e0);
            s.x = __fadd_rn(s.x, v.x);
            s.y = __fadd_rn(s.y, v.y);
            s.z = __fadd_rn(s.z, v.z);
            s.w = __fadd_rn(s.w, v.w);
        }
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(s.x) | ((uint32_t)f32_to_bf16_rne(s.y) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(s.z) | ((uint32_t)f32_to_bf16_rne(s.w) << 16);
        *reinterpret_cast<uint2*>(C + e0) = make_uint2(lo, hi);
    } else {
        for (int64_t e = e0; e < count && e < e0 + 4; ++e) {
            float s = ws[e];
            for (int p = 1; p < splits; ++p) s = __fadd_rn(s, ws[(int64_t)p * count + e]);
            C[e] = f32_to_bf16_rne(s);
        }
    }
}

// ---------------------------------------------------------------------------
// Unfused second half of the LoRA fold: out = bf16(out + fl32(scale*delta)).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
scaled_add_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ delta, int64_t count,
                  float scale) {
    const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (e0 >= count) return;
    if (e0 + 8 <= count) {   // base pointers are 16-byte aligned, so is every 8-element group
        const u32x4 o = *reinterpret_cast<const u32x4*>(out + e0);
        const u32x4 d = *reinterpret_cast<const u32x4*>(delta + e0);
        const uint32_t o4[4] = {o.x, o.y, o.z, o.w}, d4[4] = {d.x, d.y, d.z, d.w};
        uint32_t r4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = __fadd_rn(bf16_bits_to_f32(o4[e] & 0xFFFFu), __fmul_rn(scale, bf16_bits_to_f32(d4[e] & 0xFFFFu)));
            const float hi = __fadd_rn(bf16_bits_to_f32(o4[e] >> 16), __fmul_rn(scale, bf16_bits_to_f32(d4[e] >> 16)));
            r4[e] = (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
        }
        *reinterpret_cast<u32x4*>(out + e0) = u32x4{r4[0], r4[1], r4[2], r4[3]};
    } else {
        for (int64_t e = e0; e < count; ++e) {
            const float o = bf16_bits_to_f32(out[e]);
            const float d = bf16_bits_to_f32(delta[e]);
            out[e] = f32_to_bf16_rne(__fadd_rn(o, __fmul_rn(scale, d)));
        }
    }
}

}  // namespace

// Variant choice. With K % 8 == 0 the scalar-A form runs, with the most rows
// per wave (up to 3) that still gives every SIMD two waves: 4510 x 256 x 2048
// and 2255 x 256 x 2048 both take 3 (120 and 78 us). Otherwise the tile form
// runs with a register block fitted to MI355X measurements: the VALU loop
// needs four to five waves per SIMD to hide LDS and dependency latency (one
// wave per SIMD runs at roughly half speed), single-column blocks amortize
// their A reads worst, and a larger block reuses its operands better. Score =
// min(waves per SIMD, 4.5) x column factor x (outputs per thread)^(1/4); the
// highest score wins (those two shapes picked 2x2, 142 us, and 2x1, 104 us).
namespace {
// rn == 0: the scalar-A form with rm rows per wave (K % 8 == 0 only)
struct OrdChoice {
    int rm, rn;
};
constexpr OrdChoice kOrdChoices[] = {{4, 4}, {2, 2}, {2, 4}, {6, 2}, {5, 2}, {4, 2}, {3, 2}, {9, 1},
                                     {6, 1}, {4, 1}, {2, 1}, {1, 1}, {1, 0}, {2, 0}, {3, 0}};

template <int RM, int RN>
hipError_t run_ordered(const uint16_t* A, const uint16_t* B, void* C, bool f32_out, int M, int N,
                       int K, hipStream_t stream) {
    return launch_ordered_cfg<RM, RN>(A, B, C, f32_out, M, N, K, stream);
}
}  // namespace

hipError_t launch_ordered(const uint16_t* A, const uint16_t* B, void* C, bool f32_out, uint32_t M,
                          uint32_t N, uint32_t K, uint32_t cus, hipStream_t stream) {
    const int simds = 4 * (cus > 0 ? (int)cus : 256);
    int pick = tune(BG_TUNE_ORDERED);   // forced register-block variant, or -1
    constexpr int kChoices = (int)(sizeof(kOrdChoices) / sizeof(kOrdChoices[0]));
    if ((pick < 0 || pick >= kChoices) && K % 8 == 0) {
        pick = 12;   // scalar-A form, one row per wave
        for (int c = kChoices - 1; c >= 12; --c) {
            const int rm = kOrdChoices[c].rm;
            const double waves = 4.0 * ((M + 4 * rm - 1) / (4 * rm)) * (double)((N + 63) / 64);
            if (waves >= 2.0 * simds) {
                pick = c;
                break;
            }
        }
    }
    if (pick < 0 || pick >= kChoices) {
        double best = -1.0;
        for (int c = 0; c < kChoices; ++c) {
            const int rm = kOrdChoices[c].rm, rn = kOrdChoices[c].rn;
            if (rn == 0) continue;
            const double waves = 4.0 * ((M + 16 * rm - 1) / (16 * rm)) * (double)((N + 16 * rn - 1) / (16 * rn));
            const double per_simd = waves / simds;
            const double col = rn == 2 ? 1.0 : (rn == 4 ? 0.9 : 0.85);
            const double score = (per_simd < 4.5 ? per_simd : 4.5) * col * std::sqrt(std::sqrt((double)(rm * rn)));
            if (score > best) {
                best = score;
                pick = c;
            }
        }
    }
    const int m = (int)M, n = (int)N, k = (int)K;
    if (kOrdChoices[pick].rn == 0 && k % 8 != 0) pick = 10;   // the scalar-A form needs K % 8 == 0
    switch (pick) {
        case 0: return run_ordered<4, 4>(A, B, C, f32_out, m, n, k, stream);
        case 1: return run_ordered<2, 2>(A, B, C, f32_out, m, n, k, stream);
        case 2: return run_ordered<2, 4>(A, B, C, f32_out, m, n, k, stream);
        case 3: return run_ordered<6, 2>(A, B, C, f32_out, m, n, k, stream);
        case 4: return run_ordered<5, 2>(A, B, C, f32_out, m, n, k, stream);
        case 5: return run_ordered<4, 2>(A, B, C, f32_out, m, n, k, stream);
        case 6: return run_ordered<3, 2>(A, B, C, f32_out, m, n, k, stream);
        case 7: return run_ordered<9, 1>(A, B, C, f32_out, m, n, k, stream);
        case 8: return run_ordered<6, 1>(A, B, C, f32_out, m, n, k, stream);
        case 9: return run_ordered<4, 1>(A, B, C, f32_out, m, n, k, stream);
        case 10: return run_ordered<2, 1>(A, B, C, f32_out, m, n, k, stream);
        case 11: return run_ordered<1, 1>(A, B, C, f32_out, m, n, k, stream);
        case 12: return launch_ordered_sa<1>(A, B, C, f32_out, m, n, k, stream);
        case 13: return launch_ordered_sa<2>(A, B, C, f32_out, m, n, k, stream);
        default: return launch_ordered_sa<3>(A, B, C, f32_out, m, n, k, stream);
    }
}

hipError_t launch_splitk_reduce(const float* ws, uint16_t* C, uint32_t M, uint32_t N,
                                uint32_t splits, hipStream_t stream) {
    const int64_t count = (int64_t)M * N;
    const int64_t threads = (count + 3) / 4;
    dim3 grid((unsigned)((threads + 255) / 256));
    const bool vec = (count % 4) == 0;   // every plane then starts 16-byte aligned
    hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(256), 0, stream, ws, C, count, (int)splits,
                       vec);
    return hipGetLastError();
}

hipError_t launch_scaled_add(uint16_t* out, const uint16_t* delta, size_t count, float scale,
                             hipStream_t stream) {
    const int64_t threads = ((int64_t)count + 7) / 8;
    dim3 grid((unsigned)((threads + 255) / 256));
    hipLaunchKernelGGL(scaled_add_kernel, grid, dim3(256), 0, stream, out, delta, (int64_t)count,
                       scale);
    return hipGetLastError();
}

}  // namespace bg
