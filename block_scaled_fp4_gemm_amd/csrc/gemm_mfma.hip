// MFMA GEMM core for gfx950: C[M,N] = A[M,K] * B[N,K]^T with FP32 accumulation,
// BF16 or dequantized-FP4 operands, and three epilogues.
//
// Design (CDNA4, wave64):
//  - A workgroup owns a BM x BN output tile and walks K in steps of BK = 64.
//  - Operand tiles are staged global -> registers -> LDS, double-buffered:
//    the global loads for step t+1 are in flight while the MFMAs of step t
//    run, and one barrier per step separates the two LDS buffers.
//  - Tiles are stored K-contiguous (64 BF16 = eight 16-byte chunks per row)
//    with the chunk index XOR-swizzled by row, so both the 16-byte staging
//    writes and the 16-byte operand reads of v_mfma_f32_32x32x16_bf16 are
//    spread over all LDS banks.
//  - Each wave owns a (BM/WM) x (BN/WN) sub-tile as a grid of 32x32 MFMA
//    blocks. The MFMA is issued with the B tile as its first operand, so the
//    accumulator holds C^T: each lane ends up with four consecutive N
//    columns of one M row, stored as one 8-byte (BF16) or 16-byte (FP32)
//    write.
//  - Workgroups are numbered so that consecutive logical tiles share an XCD
//    (dispatch is round-robin over the 8 XCDs), and logical tiles follow a
//    grouped order (GROUP_M tile-rows at a time) for L2 reuse of B.
//
// Method semantics: sm121a_matmul.py page (kernel body: FP32 accumulator over
// K blocks, K tail contributes zeros, BF16 cast at the masked store; grouped
// program order for L2 reuse); gemm_dense.rs page (A [M,K], B [N,K], C [M,N];
// dense_gemm_tc_scaled_acc's delta rounded to BF16 before the scale;
// dense_gemm_splitk's FP32 partial planes); kernelbot NVFP4 GEMM page
// ("SCALE FACTORS": one E4M3 scale per 16 K elements multiplied into each
// E2M1 element, then an FP32-accumulated dot product).
#include "bg_internal.hpp"

#pragma clang fp contract(off)

namespace bg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;       // K elements per pipeline step
constexpr int GROUP_M = 8;   // tile-rows per group in the grouped order

enum Source : int { SRC_BF16_VEC = 0, SRC_BF16_SCALAR = 1, SRC_FP4 = 2 };

struct KParams {
    const uint16_t* A;     // bf16 [M,K]            (SRC_BF16_*)
    const uint16_t* B;     // bf16 [N,K]
    const uint8_t* Aq;     // packed e2m1 [M,K/2]   (SRC_FP4)
    const uint8_t* SFA;    // e4m3fn [M,K/16]
    const uint8_t* Bq;
    const uint8_t* SFB;
    void* C;               // bf16 [M,N] or f32 planes [splits][M][N]
    int M, N, K;
    int k_chunk;           // K elements per split (blockIdx.y)
    int tiles_m, tiles_n;
    float scale;
};

// Swizzled 16-byte chunk slot of logical chunk c in tile row `row`.
// Any 8 consecutive rows, and the 8 even (or odd) rows of any 16 consecutive
// rows, map one logical chunk to 8 distinct slots.
__device__ __forceinline__ int chunk_slot(int row, int c) {
    return c ^ ((row ^ (row >> 3)) & 7);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// E4M3FN byte -> FP32 (exact): bias 7, subnormal m*2^-9, S.1111.111 = NaN.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float mag = (e == 0) ? (float)m * 0x1p-9f
                         : __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
    if (e == 15u && m == 7u) mag = __builtin_nanf("");
    return (b & 0x80u) ? -mag : mag;
}

// Workgroup -> (tile_m, tile_n). Dispatch places workgroup b on XCD b % 8;
// logical ids are assigned so each XCD receives one contiguous range, and the
// range is walked in grouped order (GROUP_M tile-rows, m fastest).
__device__ __forceinline__ void tile_of_block(int tiles_m, int tiles_n, int& tm, int& tn) {
    const int nblocks = tiles_m * tiles_n;
    const int b = blockIdx.x;
    const int per = nblocks >> 3, rem = nblocks & 7;
    const int x = b & 7, j = b >> 3;
    const int logical = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + j;
    const int width = GROUP_M * tiles_n;
    const int g = logical / width;
    const int first_m = g * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int r = logical - g * width;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

// ---------------------------------------------------------------------------
// Operand staging: one BK-wide K step of a ROWS x BK tile into registers, then
// into LDS. Rows beyond the matrix are clamped to its last row (their results
// are never stored); K positions at or beyond k_end are zero.
// ---------------------------------------------------------------------------

template <int ROWS, int NT, int SRC>
struct Stager;

// BF16 rows whose pitch is a multiple of 16 bytes (K % 8 == 0): one 16-byte
// chunk per load, eight threads per 128-byte row segment.
template <int ROWS, int NT>
struct Stager<ROWS, NT, SRC_BF16_VEC> {
    static constexpr int PER = ROWS * (BK / 8) / NT;
    static_assert(PER * NT == ROWS * (BK / 8), "tile not divisible among threads");
    u32x4 r[PER];

    __device__ __forceinline__ void load(const uint16_t* base, int row0, int nrows, int K,
                                         int k0, int k_end, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * NT;
            const int row = q >> 3, c = q & 7;
            const int grow = min(row0 + row, nrows - 1);
            const int gk = k0 + c * 8;
            if (gk < k_end)
                r[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)grow * K + gk);
            else
                r[i] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * NT;
            const int row = q >> 3, c = q & 7;
            *reinterpret_cast<u32x4*>(lds + row * BK + chunk_slot(row, c) * 8) = r[i];
        }
    }
};

// BF16 rows with an unaligned pitch: element-wise guarded loads.
template <int ROWS, int NT>
struct Stager<ROWS, NT, SRC_BF16_SCALAR> {
    static constexpr int PER = ROWS * (BK / 8) / NT;
    u32x4 r[PER];

    __device__ __forceinline__ void load(const uint16_t* base, int row0, int nrows, int K,
                                         int k0, int k_end, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * NT;
            const int row = q >> 3, c = q & 7;
            const int grow = min(row0 + row, nrows - 1);
            const uint16_t* src = base + (int64_t)grow * K;
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int gk = k0 + c * 8 + e;
                h[e] = gk < k_end ? (uint32_t)src[gk] : 0u;
            }
            r[i] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                         h[6] | (h[7] << 16)};
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * NT;
            const int row = q >> 3, c = q & 7;
            *reinterpret_cast<u32x4*>(lds + row * BK + chunk_slot(row, c) * 8) = r[i];
        }
    }
};

// Block-scaled FP4: a unit is one 16-element scale group of one row (8 packed
// bytes + 1 scale byte); it is dequantized exactly to BF16 while being written
// to LDS as two 16-byte chunks. e2m1 * e4m3 has at most 6 significant bits,
// so the FP32 product and its BF16 conversion are exact.
template <int ROWS, int NT>
struct Stager<ROWS, NT, SRC_FP4> {
    static constexpr int PER = ROWS * (BK / 16) / NT;
    static_assert(PER * NT == ROWS * (BK / 16), "tile not divisible among threads");
    u32x2 w[PER];
    uint32_t s[PER];

    __device__ __forceinline__ void load(const uint8_t* q, const uint8_t* sf, int row0,
                                         int nrows, int K, int k0, int k_end, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            const int row = u >> 2, g = u & 3;
            const int grow = min(row0 + row, nrows - 1);
            const int gk = k0 + g * 16;
            if (gk < k_end) {
                w[i] = *reinterpret_cast<const u32x2*>(q + (int64_t)grow * (K >> 1) + (gk >> 1));
                s[i] = sf[(int64_t)grow * (K >> 4) + (gk >> 4)];
            } else {
                w[i] = u32x2{0u, 0u};
                s[i] = 0u;
            }
        }
    }

    __device__ __forceinline__ static uint32_t deq2(uint32_t word, float sc, int byte) {
        f32x2 v;
        switch (byte) {   // byte select must be an immediate
            case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0); break;
            case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1); break;
            case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2); break;
            default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3); break;
        }
        return pack_bf16x2(v.x * sc, v.y * sc);
    }

    __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            const int row = u >> 2, g = u & 3;
            const float sc = e4m3fn_to_f32(s[i]);
            const u32x4 lo = {deq2(w[i].x, sc, 0), deq2(w[i].x, sc, 1), deq2(w[i].x, sc, 2),
                              deq2(w[i].x, sc, 3)};
            const u32x4 hi = {deq2(w[i].y, sc, 0), deq2(w[i].y, sc, 1), deq2(w[i].y, sc, 2),
                              deq2(w[i].y, sc, 3)};
            *reinterpret_cast<u32x4*>(lds + row * BK + chunk_slot(row, 2 * g) * 8) = lo;
            *reinterpret_cast<u32x4*>(lds + row * BK + chunk_slot(row, 2 * g + 1) * 8) = hi;
        }
    }
};

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

template <int BM, int BN, int WM, int WN, int EPI, int SRC>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_mfma_kernel(KParams p) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;   // wave sub-tile
    constexpr int FM = TM / 32, FN = TN / 32;   // 32x32 MFMA blocks per wave
    static_assert(FM * 32 * WM == BM && FN * 32 * WN == BN, "bad tile split");
    constexpr int STAGE = (BM + BN) * BK;       // BF16 elements per LDS stage

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int tm, tn;
    tile_of_block(p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int split = blockIdx.y;
    const int kb = (int)min((int64_t)p.K, (int64_t)split * p.k_chunk);
    const int ke = (int)min((int64_t)p.K, (int64_t)kb + p.k_chunk);
    const int nk = (ke - kb + BK - 1) / BK;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    Stager<BM, NT, SRC> sa;
    Stager<BN, NT, SRC> sb;
    auto load_step = [&](int k0) {
        if constexpr (SRC == SRC_FP4) {
            sa.load(p.Aq, p.SFA, m0, p.M, p.K, k0, ke, tid);
            sb.load(p.Bq, p.SFB, n0, p.N, p.K, k0, ke, tid);
        } else {
            sa.load(p.A, m0, p.M, p.K, k0, ke, tid);
            sb.load(p.B, n0, p.N, p.K, k0, ke, tid);
        }
    };

    if (nk > 0) {
        load_step(kb);
        sa.store(smem, tid);
        sb.store(smem + BM * BK, tid);
    }
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        if (t + 1 < nk) load_step(kb + (t + 1) * BK);

        const uint16_t* sA = smem + cur * STAGE;
        const uint16_t* sB = sA + BM * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = kk * 2 + (lane >> 5);
            bf16x8 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * TM + i * 32 + (lane & 31);
                fa[i] = *reinterpret_cast<const bf16x8*>(sA + row * BK + chunk_slot(row, c) * 8);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * TN + j * 32 + (lane & 31);
                fb[j] = *reinterpret_cast<const bf16x8*>(sB + row * BK + chunk_slot(row, c) * 8);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }

        if (t + 1 < nk) {
            uint16_t* nxt = smem + (cur ^ 1) * STAGE;
            sa.store(nxt, tid);
            sb.store(nxt + BM * BK, tid);
        }
        __syncthreads();
    }

    // Epilogue. acc[i][j][4g + e] is C[m][n + e] with
    //   m = m0 + wm*TM + i*32 + lane%32,  n = n0 + wn*TN + j*32 + 8g + 4*(lane/32).
    const int M = p.M, N = p.N;
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * TM + i * 32 + (lane & 31);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * TN + j * 32 + g * 8 + (lane >> 5) * 4;
                const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
                const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
                const int64_t off = (int64_t)m * N + n;
                if constexpr (EPI == EPI_STORE_F32) {
                    float* plane = reinterpret_cast<float*>(p.C) + (int64_t)split * M * N;
                    if (vec_ok && n + 3 < N) {
                        *reinterpret_cast<f32x4*>(plane + off) = f32x4{v0, v1, v2, v3};
                    } else {
                        const float v[4] = {v0, v1, v2, v3};
                        for (int e = 0; e < 4; ++e)
                            if (n + e < N) plane[off + e] = v[e];
                    }
                } else if constexpr (EPI == EPI_STORE_BF16) {
                    uint16_t* C = reinterpret_cast<uint16_t*>(p.C);
                    const uint32_t w0 = pack_bf16x2(v0, v1), w1 = pack_bf16x2(v2, v3);
                    if (vec_ok && n + 3 < N) {
                        *reinterpret_cast<u32x2*>(C + off) = u32x2{w0, w1};
                    } else {
                        const uint16_t h[4] = {(uint16_t)w0, (uint16_t)(w0 >> 16), (uint16_t)w1,
                                               (uint16_t)(w1 >> 16)};
                        for (int e = 0; e < 4; ++e)
                            if (n + e < N) C[off + e] = h[e];
                    }
                } else {  // EPI_SCALED_ACC: out = bf16(out + scale * bf16(delta))
                    uint16_t* O = reinterpret_cast<uint16_t*>(p.C);
                    const uint32_t d0 = pack_bf16x2(v0, v1), d1 = pack_bf16x2(v2, v3);
                    const float s = p.scale;
                    if (vec_ok && n + 3 < N) {
                        const u32x2 o = *reinterpret_cast<const u32x2*>(O + off);
                        const float r0 = bf16_lo(o.x) + s * bf16_lo(d0);
                        const float r1 = bf16_hi(o.x) + s * bf16_hi(d0);
                        const float r2 = bf16_lo(o.y) + s * bf16_lo(d1);
                        const float r3 = bf16_hi(o.y) + s * bf16_hi(d1);
                        *reinterpret_cast<u32x2*>(O + off) = u32x2{pack_bf16x2(r0, r1), pack_bf16x2(r2, r3)};
                    } else {
                        const float d[4] = {bf16_lo(d0), bf16_hi(d0), bf16_lo(d1), bf16_hi(d1)};
                        for (int e = 0; e < 4; ++e) {
                            if (n + e < N) {
                                const float o = __builtin_bit_cast(float, (uint32_t)O[off + e] << 16);
                                const float r = o + s * d[e];
                                O[off + e] = (uint16_t)pack_bf16x2(r, 0.0f);
                            }
                        }
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, int EPI, int SRC>
hipError_t launch_cfg(const KParams& kp, int splits, hipStream_t stream) {
    KParams q = kp;
    q.tiles_m = (kp.M + BM - 1) / BM;
    q.tiles_n = (kp.N + BN - 1) / BN;
    dim3 grid((unsigned)(q.tiles_m * q.tiles_n), (unsigned)splits, 1);
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN, EPI, SRC>), grid, dim3(WM * WN * 64), 0,
                       stream, q);
    return hipGetLastError();
}

template <int EPI, int SRC>
hipError_t launch_dense_src(const KParams& kp, int splits, hipStream_t stream) {
    return launch_cfg<128, 128, 2, 2, EPI, SRC>(kp, splits, stream);
}

}  // namespace

hipError_t launch_dense(const DenseProblem& p, Epilogue epi, hipStream_t stream) {
    KParams kp{};
    kp.A = p.A;
    kp.B = p.B;
    kp.C = p.C;
    kp.M = (int)p.M;
    kp.N = (int)p.N;
    kp.K = (int)p.K;
    kp.k_chunk = (int)p.k_chunk;
    kp.scale = p.scale;
    const bool vec = (p.K % 8) == 0;
    const int splits = (int)p.splits;
    switch (epi) {
        case EPI_STORE_BF16:
            return vec ? launch_dense_src<EPI_STORE_BF16, SRC_BF16_VEC>(kp, splits, stream)
                       : launch_dense_src<EPI_STORE_BF16, SRC_BF16_SCALAR>(kp, splits, stream);
        case EPI_SCALED_ACC:
            return vec ? launch_dense_src<EPI_SCALED_ACC, SRC_BF16_VEC>(kp, splits, stream)
                       : launch_dense_src<EPI_SCALED_ACC, SRC_BF16_SCALAR>(kp, splits, stream);
        case EPI_STORE_F32:
            return vec ? launch_dense_src<EPI_STORE_F32, SRC_BF16_VEC>(kp, splits, stream)
                       : launch_dense_src<EPI_STORE_F32, SRC_BF16_SCALAR>(kp, splits, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fp4(const Fp4Problem& p, hipStream_t stream) {
    KParams kp{};
    kp.Aq = p.A;
    kp.SFA = p.SFA;
    kp.Bq = p.B;
    kp.SFB = p.SFB;
    kp.C = p.C;
    kp.M = (int)p.M;
    kp.N = (int)p.N;
    kp.K = (int)p.K;
    kp.k_chunk = (int)p.K;
    return launch_cfg<128, 128, 2, 2, EPI_STORE_BF16, SRC_FP4>(kp, 1, stream);
}

}  // namespace bg
