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
#include <type_traits>

#include "bg_internal.hpp"
#include "streamk_plan.hpp"
#include "tile_order.hpp"

#pragma clang fp contract(off)

namespace bg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;       // K elements per pipeline step

// Operand sources. A kernel's SRC names both operands: SRC_W4A16 is BF16 A
// (SRC_BF16_VEC staging) with FP4 B dequantized to BF16 (SRC_FP4_BF16).
enum Source : int {
    SRC_BF16_VEC = 0,
    SRC_BF16_SCALAR = 1,
    SRC_FP4 = 2,        // both operands FP4, dequantized to FP16
    SRC_W4A16 = 3,
    SRC_FP4_BF16 = 4,   // staging only: FP4 dequantized to BF16
    // the same with 32-element staging units (K % 32 == 0)
    SRC_FP4W = 5,
    SRC_W4A16W = 6,
    SRC_FP4W_BF16 = 7,
    // W4A16 with the weights in the transposed layout [K/2, ldb] bytes (byte
    // (r, n) holds k = 2r and 2r+1 of weight row n) and scales [K/16, ldb]:
    // 4-byte loads where ldb % 4 == 0, byte loads otherwise
    SRC_W4A16T4 = 8,
    SRC_W4A16T1 = 9,
    SRC_FP4T4_BF16 = 10,   // staging only
    SRC_FP4T1_BF16 = 11,
};

constexpr bool src_fp4(int src) { return src == SRC_FP4 || src == SRC_FP4W; }
constexpr bool src_w4a16t(int src) { return src == SRC_W4A16T4 || src == SRC_W4A16T1; }
constexpr bool src_w4a16(int src) { return src == SRC_W4A16 || src == SRC_W4A16W || src_w4a16t(src); }
constexpr bool src_fp4t(int src) { return src == SRC_FP4T4_BF16 || src == SRC_FP4T1_BF16; }
// K elements per staging unit of an FP4 operand of `rows` tile rows staged by
// nt threads (0: not FP4). The 32-element units are taken only where they
// divide evenly among the threads: otherwise some waves would convert twice
// as many elements as others, and every step waits for the slowest.
constexpr int fp4_unit(int src, int rows, int nt) {
    return src == SRC_FP4 || src == SRC_FP4_BF16                      ? 16
           : (src == SRC_FP4W || src == SRC_FP4W_BF16) && rows * 2 % nt == 0 ? 32
           : src == SRC_FP4W || src == SRC_FP4W_BF16                  ? 16
                                                                      : 0;
}

struct KParams {
    const uint16_t* A;     // bf16 [M,K]            (SRC_BF16_*)
    const uint16_t* B;     // bf16 [N,K]
    const uint8_t* Aq;     // packed e2m1 [M,K/2]   (SRC_FP4)
    const uint8_t* SFA;    // e4m3fn [M,K/16]
    const uint8_t* Bq;
    const uint8_t* SFB;
    void* C;               // bf16 [M,N] or f32 planes [splits][M][N], rows ldc elements apart
    int M, N, K;
    int lda, ldb;          // elements between consecutive rows of A and B (BF16 operands; >= K)
    int ldc;               // elements between consecutive rows of C (N, or more for a column range)
    int ldbt;              // bytes between rows of transposed FP4 weights and of their scales
    int k_chunk;           // K elements per split (blockIdx.y)
    int tiles_m, tiles_n;
    float scale;
    int cus;               // compute units of the device (tile choice)
    // batched FP4 (blockIdx.z = batch index): per-batch strides of Aq, SFA,
    // Bq, SFB (bytes) and C (elements); zero for one problem
    int64_t bs_a, bs_sa, bs_b, bs_sb, bs_c;
    // two products of the same A in one launch (direct kernels, BF16 store):
    // `dual` requests it (B1 may be NULL when K = 0); the launcher then sets
    // dual_tiles_n, and column tiles [dual_tiles_n, 2*dual_tiles_n) of the
    // grid compute C1 = A * B1^T; 0 for a single problem
    const uint16_t* B1;
    void* C1;
    int dual;
    int dual_tiles_n;
};

// Swizzled 16-byte chunk slot of logical chunk c in a tile row of CPR chunks
// (CPR = BK/8). The XOR keeps the eight (CPR = 8) or four (CPR = 4) chunks of a
// row in distinct slots, and gives one logical chunk distinct banks across the
// 8 consecutive rows (or the 16 rows, for 256-byte bank windows) that the
// lanes of one 16-byte LDS read touch. It is an involution in c.
template <int CPR>
__device__ __forceinline__ int chunk_slot(int row, int c) {
    if constexpr (CPR == 8)
        return c ^ ((row ^ (row >> 3)) & 7);
    else
        return c ^ (((row >> 1) ^ (row >> 3)) & 3);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS only. __syncthreads() would also wait for
// every outstanding global load of the wave (its release fence covers global
// memory), which would drain the direct-load ring at every step. Before the
// barrier this wave's LDS reads and writes are complete; the direct loads
// the caller needs are covered by its own vmcnt wait.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// One workgroup per tile: workgroup -> (tile_m, tile_n).
__device__ __forceinline__ void tile_of_block(int tiles_m, int tiles_n, int& tm, int& tn) {
    tile_of<ORDER_GEMM>((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
}

// ---------------------------------------------------------------------------
// Operand staging: one BK-wide K step of a ROWS x BK tile into registers, then
// into LDS. Rows beyond the matrix are clamped to its last row (their results
// are never stored); K positions at or beyond k_end are zero.
// ---------------------------------------------------------------------------

template <int ROWS, int NT, int SRC, int BKS = BK>
struct Stager;

// BF16 rows whose pitch is a multiple of 16 bytes (K % 8 == 0): one 16-byte
// chunk per load, eight threads per 128-byte row segment.
template <int ROWS, int NT, int BKS>
struct Stager<ROWS, NT, SRC_BF16_VEC, BKS> {
    static constexpr int CPR = BKS / 8;
    static constexpr int PER = (ROWS * CPR + NT - 1) / NT;
    u32x4 r[PER];
    uint32_t valid;   // bit i: chunk i lies inside the K range (applied when storing)

    // ld: elements between consecutive rows (a multiple of 8). Every lane
    // loads (a chunk past k_end re-reads the row's last chunk before k_end
    // and is stored as zeros), so the load has no branch around it, nothing
    // reads its result before the store, and the wait counts are exact.
    // k_end >= 8 whenever a step exists.
    __device__ __forceinline__ void load(const uint16_t* base, int row0, int nrows, int ld,
                                         int k0, int k_end, int tid) {
        valid = 0u;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * NT;
            if (PER * NT != ROWS * CPR && q >= ROWS * CPR) break;
            const int row = q / CPR, c = q % CPR;
            const int grow = min(row0 + row, nrows - 1);
            const int gk = k0 + c * 8;
            const int gkc = gk < k_end ? gk : max(k_end - 8, 0);
            r[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)grow * ld + gkc);
            valid |= (gk < k_end ? 1u : 0u) << i;
        }
    }
    // writes the chunks with lo <= i < hi
    __device__ __forceinline__ void store_units(uint16_t* lds, int tid, int lo, int hi) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (i < lo || i >= hi) continue;
            const int q = tid + i * NT;
            if (PER * NT != ROWS * CPR && q >= ROWS * CPR) break;
            const int row = q / CPR, c = q % CPR;
            const bool in = (valid >> i) & 1u;
            *reinterpret_cast<u32x4*>(lds + row * BKS + chunk_slot<CPR>(row, c) * 8) =
                in ? r[i] : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int tid) const { store_units(lds, tid, 0, PER); }
};

// BF16 rows with an unaligned pitch: element-wise guarded loads.
template <int ROWS, int NT, int BKS>
struct Stager<ROWS, NT, SRC_BF16_SCALAR, BKS> {
    static constexpr int CPR = BKS / 8;
    static constexpr int PER = (ROWS * CPR + NT - 1) / NT;
    u32x4 r[PER];

    __device__ __forceinline__ void load(const uint16_t* base, int row0, int nrows, int ld,
                                         int k0, int k_end, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = tid + i * NT;
            if (PER * NT != ROWS * CPR && q >= ROWS * CPR) break;
            const int row = q / CPR, c = q % CPR;
            const int grow = min(row0 + row, nrows - 1);
            const uint16_t* src = base + (int64_t)grow * ld;
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
    __device__ __forceinline__ void store_units(uint16_t* lds, int tid, int lo, int hi) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (i < lo || i >= hi) continue;
            const int q = tid + i * NT;
            if (PER * NT != ROWS * CPR && q >= ROWS * CPR) break;
            const int row = q / CPR, c = q % CPR;
            *reinterpret_cast<u32x4*>(lds + row * BKS + chunk_slot<CPR>(row, c) * 8) = r[i];
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int tid) const { store_units(lds, tid, 0, PER); }
};

// Block-scaled FP4: a unit is UE consecutive K elements of one row (UE / 2
// packed bytes and UE / 16 scale bytes); it is dequantized exactly while being
// written to LDS as UE / 8 16-byte chunks. Every e2m1 value, every e4m3 scale
// and their product (at most 6 significant bits, magnitude between 2^-10 and
// 2688, or zero, or NaN from a NaN scale) is exact in FP16 and in BF16.
//  - F16OUT (both operands FP4, FP16 MFMA): FP16 convert, then half a packed
//    FP16 multiply per element; the multiply rounds nothing.
//  - BF16 (W4A16 weights next to BF16 activations, BF16 MFMA): FP32 convert,
//    FP32 multiply (exact), BF16 pack (exact).
// UE = 32 (K % 32 == 0): one 16-byte load and one 2-byte scale load per unit,
// two lanes per 32-byte row step: a quarter of the load instructions of
// UE = 16 (an 8-byte and a 1-byte load per 16 elements) and fewer registers
// per held step, so the 256 x 256 FP16 tile holds two steps without spilling.
// UE = 16 serves K % 32 == 16, where a 32-element unit would straddle the end
// of K, and operands whose 32-element units do not divide evenly among the
// threads.
template <int ROWS, int NT, bool F16OUT, int UE = 16>
struct Fp4Stager {
    static_assert(UE == 16 || UE == 32, "unit of one or two scale groups");
    static constexpr int UPR = BK / UE;                  // units per row step
    static constexpr int UNITS = ROWS * UPR;
    static constexpr int PER = (UNITS + NT - 1) / NT;    // surplus slots (u >= UNITS) do nothing
    static constexpr int WORDS = UE / 8;                 // 32-bit words of packed data per unit
    typedef uint32_t Words __attribute__((ext_vector_type(WORDS)));
    Words w[PER];
    uint32_t s[PER];
    uint32_t valid;   // bit i: unit i lies inside the K range (applied when converting)

    __device__ __forceinline__ void load(const uint8_t* q, const uint8_t* sf, int row0,
                                         int nrows, int K, int k0, int k_end, int tid) {
        valid = 0u;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            if (PER * NT != UNITS && u >= UNITS) break;
            const int row = u / UPR, g = u % UPR;
            const int grow = min(row0 + row, nrows - 1);
            const int gk = k0 + g * UE;
            // always load from a valid unit (K >= UE whenever a step exists:
            // K is a multiple of UE), then zero what lies past the end of this
            // K range (k_end is a multiple of UE too)
            const int gkc = min(gk, K - UE);
            w[i] = *reinterpret_cast<const Words*>(q + (int64_t)grow * (K >> 1) + (gkc >> 1));
            if constexpr (UE == 16)
                s[i] = sf[(int64_t)grow * (K >> 4) + (gkc >> 4)];
            else
                s[i] = *reinterpret_cast<const uint16_t*>(sf + (int64_t)grow * (K >> 4) + (gkc >> 4));
            valid |= (gk < k_end ? 1u : 0u) << i;
        }
    }

    // Eight e2m1 values (word: low nibble first) times the scale, as four
    // packed 16-bit pairs. sc16 holds the scale in both halves.
    __device__ __forceinline__ static u32x4 deq8(uint32_t word, f16x2 sc16, float sc32) {
        u32x4 r;
        if constexpr (F16OUT) {
            r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * sc16);
            r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * sc16);
            r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * sc16);
            r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * sc16);
        } else {
            f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
            r.x = pack_bf16x2(v.x * sc32, v.y * sc32);
            v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
            r.y = pack_bf16x2(v.x * sc32, v.y * sc32);
            v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
            r.z = pack_bf16x2(v.x * sc32, v.y * sc32);
            v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
            r.w = pack_bf16x2(v.x * sc32, v.y * sc32);
        }
        return r;
    }

    __device__ __forceinline__ void store(uint16_t* lds, int tid) const { store_units(lds, tid, 0, PER); }

    // converts and writes the units with lo <= i < hi
    __device__ __forceinline__ void store_units(uint16_t* lds, int tid, int lo, int hi) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (i < lo || i >= hi) continue;
            const int u = tid + i * NT;
            if (PER * NT != UNITS && u >= UNITS) break;
            const int row = u / UPR, g = u % UPR;
            const bool in = (valid >> i) & 1u;
            // e4m3fn bytes -> FP16 or FP32 (exact, NaN stays NaN); a unit past
            // the K range gets scale 0 and zero data
            const uint32_t sb = in ? s[i] : 0u;
            f16x2 sc16 = {};
            f32x2 sc32 = {};
            if constexpr (F16OUT)
                sc16 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
            else
                sc32 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sb, 1.0f, false);
            uint16_t* dst = lds + row * BK;
#pragma unroll
            for (int c = 0; c < WORDS; ++c) {
                // word c holds elements 8c .. 8c+7 of the unit: scale group c / 2
                const uint32_t wc = in ? w[i][c] : 0u;
                const f16x2 s16 = c < 2 ? f16x2{sc16.x, sc16.x} : f16x2{sc16.y, sc16.y};
                const float s32 = c < 2 ? sc32.x : sc32.y;
                *reinterpret_cast<u32x4*>(dst + chunk_slot<8>(row, WORDS * g + c) * 8) = deq8(wc, s16, s32);
            }
        }
    }
};

template <int ROWS, int NT>
struct Stager<ROWS, NT, SRC_FP4, BK> : Fp4Stager<ROWS, NT, true> {};

template <int ROWS, int NT>
struct Stager<ROWS, NT, SRC_FP4_BF16, BK> : Fp4Stager<ROWS, NT, false> {};

template <int ROWS, int NT>
struct Stager<ROWS, NT, SRC_FP4W, BK> : Fp4Stager<ROWS, NT, true, fp4_unit(SRC_FP4W, ROWS, NT)> {};

template <int ROWS, int NT>
struct Stager<ROWS, NT, SRC_FP4W_BF16, BK> : Fp4Stager<ROWS, NT, false, fp4_unit(SRC_FP4W_BF16, ROWS, NT)> {};

// NVFP4 weights in the transposed layout of the gemm_dense.rs page's `_ldb`
// W4A16 launchers: byte (r, n) at Bt + r*ldb + n holds the E2M1 codes of
// weight row n at k = 2r (low nibble) and k = 2r + 1 (high nibble), and the
// E4M3 scale of group g of row n is at SFBt + g*ldb + n; ldb >= N may be any
// value (odd for a vocabulary-sized N). A unit is TW consecutive weight rows
// (n) times one 16-element scale group: 8 loads of TW bytes (one per k-pair
// row) and one TW-byte scale load, transposed in registers into each weight
// row's 8 packed bytes (the K-contiguous form), then dequantized exactly to
// BF16 as in Fp4Stager and written as two 16-byte chunks per weight row.
// Columns past the last valid one are clamped to it (their outputs are never
// stored); with TW = 4 a unit starts at a multiple of 4 below ldb, so every
// 4-byte load stays inside its row of ldb bytes.
template <int ROWS, int NT, int TW>
struct Fp4TStager {
    static_assert(TW == 1 || TW == 4, "1- or 4-byte column loads");
    static constexpr int CPU_ = 4;                        // weight rows per unit (TW = 1: 4 byte loads)
    static constexpr int UNITS = (ROWS / CPU_) * (BK / 16);
    static constexpr int PER = (UNITS + NT - 1) / NT;
    uint32_t d[PER][8];   // d[i][r]: bytes of k-pair row r, weight rows c = 0..3 in bytes c
    uint32_t s[PER];      // scale bytes of the unit's 4 weight rows
    uint32_t valid;

    __device__ __forceinline__ void load(const uint8_t* bt, const uint8_t* sft, int n0, int N, int ldb,
                                         int K, int k0, int k_end, int tid) {
        valid = 0u;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            if (PER * NT != UNITS && u >= UNITS) break;
            const int quad = u / (BK / 16), g = u % (BK / 16);
            const int gk = k0 + g * 16;
            const int gkc = min(gk, K - 16);             // K >= 16 whenever a step exists
            const uint8_t* rowp = bt + (int64_t)(gkc >> 1) * ldb;
            const uint8_t* srow = sft + (int64_t)(gkc >> 4) * ldb;
            if constexpr (TW == 4) {
                const int n = min(n0 + quad * 4, ldb - 4);   // ldb % 4 == 0, so n % 4 == 0
#pragma unroll
                for (int r = 0; r < 8; ++r) d[i][r] = *reinterpret_cast<const uint32_t*>(rowp + (int64_t)r * ldb + n);
                s[i] = *reinterpret_cast<const uint32_t*>(srow + n);
            } else {
                int n[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) n[c] = min(n0 + quad * 4 + c, N - 1);
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const uint8_t* q = rowp + (int64_t)r * ldb;
                    d[i][r] = (uint32_t)q[n[0]] | ((uint32_t)q[n[1]] << 8) | ((uint32_t)q[n[2]] << 16) |
                              ((uint32_t)q[n[3]] << 24);
                }
                s[i] = (uint32_t)srow[n[0]] | ((uint32_t)srow[n[1]] << 8) | ((uint32_t)srow[n[2]] << 16) |
                       ((uint32_t)srow[n[3]] << 24);
            }
            valid |= (gk < k_end ? 1u : 0u) << i;
        }
    }

    // byte c of each of four words, gathered into one word (word r -> byte r)
    __device__ __forceinline__ static uint32_t column(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, int c) {
        const int sh = 8 * c;
        return ((w0 >> sh) & 0xFFu) | (((w1 >> sh) & 0xFFu) << 8) | (((w2 >> sh) & 0xFFu) << 16) |
               (((w3 >> sh) & 0xFFu) << 24);
    }

    __device__ __forceinline__ void store(uint16_t* lds, int tid) const { store_units(lds, tid, 0, PER); }

    __device__ __forceinline__ void store_units(uint16_t* lds, int tid, int lo, int hi) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (i < lo || i >= hi) continue;
            const int u = tid + i * NT;
            if (PER * NT != UNITS && u >= UNITS) break;
            const int quad = u / (BK / 16), g = u % (BK / 16);
            const bool in = (valid >> i) & 1u;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int row = quad * 4 + c;
                // the 16 elements of weight row n0+row in this group, K-contiguous:
                // k-pair rows 0..3 in the low word, 4..7 in the high word
                const uint32_t lo_w = in ? column(d[i][0], d[i][1], d[i][2], d[i][3], c) : 0u;
                const uint32_t hi_w = in ? column(d[i][4], d[i][5], d[i][6], d[i][7], c) : 0u;
                const uint32_t sb = in ? (s[i] >> (8 * c)) & 0xFFu : 0u;
                const f32x2 sc32 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sb, 1.0f, false);
                uint16_t* dst = lds + row * BK;
                *reinterpret_cast<u32x4*>(dst + chunk_slot<8>(row, 2 * g) * 8) =
                    Fp4Stager<ROWS, NT, false>::deq8(lo_w, f16x2{}, sc32.x);
                *reinterpret_cast<u32x4*>(dst + chunk_slot<8>(row, 2 * g + 1) * 8) =
                    Fp4Stager<ROWS, NT, false>::deq8(hi_w, f16x2{}, sc32.x);
            }
        }
    }
};

template <int ROWS, int NT>
struct Stager<ROWS, NT, SRC_FP4T4_BF16, BK> : Fp4TStager<ROWS, NT, 4> {};

template <int ROWS, int NT>
struct Stager<ROWS, NT, SRC_FP4T1_BF16, BK> : Fp4TStager<ROWS, NT, 1> {};

// ---------------------------------------------------------------------------
// Direct global -> LDS staging (buffer_load_dwordx4 ... lds) for BF16 rows
// with a 16-byte-multiple pitch. One instruction moves 64 lanes x 16 bytes
// into one contiguous 1 KB LDS segment (lane i lands at byte 16*i), i.e.
// 512/BKS tile rows of 2*BKS bytes. The XOR swizzle is applied on the global
// side: the lane that lands in slot s of row r fetches logical chunk
// chunk_slot(r, s) (an involution). The lanes of one row still read that
// row's whole 2*BKS-byte segment. Only whole BKS steps use this path; rows
// beyond the matrix are clamped to its last row.
// ---------------------------------------------------------------------------
// A pointer every lane holds the same value of, stated as such so that a
// buffer resource built from it stays in scalar registers (the inline-asm
// loads need it there) whatever the compiler's divergence analysis concludes.
__device__ __forceinline__ void* uniform_ptr(const void* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

template <int ROWS, int NT, int BKS>
struct DirectStager {
    static constexpr int CPR = BKS / 8;          // 16-byte chunks per row
    static constexpr int RPS = 64 / CPR;         // rows per 1 KB segment
    static constexpr int NW = NT / 64;
    static constexpr int SEGS = ROWS / RPS;
    // Instructions per wave. When the segments do not divide evenly, the
    // surplus slots re-load the last segment (the same bytes to the same LDS
    // place), so every wave issues the same count for the vmcnt bookkeeping.
    static constexpr int PER = (SEGS + NW - 1) / NW;
    static_assert(SEGS * RPS == ROWS && RPS * CPR == 64, "whole 1 KB segments");

    // Buffer form: the tile's rows are addressed through a buffer resource
    // based at row row0, so each lane's offset (its row and swizzled chunk)
    // is a 32-bit constant for the whole K walk and the K position is a
    // scalar offset: no per-step vector address arithmetic. Needs
    // ROWS * ld * 2 < 2^32 (checked by the host).
    uint32_t voff[PER];
    __amdgpu_buffer_rsrc_t rsrc;

    __device__ __forceinline__ void init(const uint16_t* base, int row0, int nrows, int ld, int wave, int lane) {
        rsrc = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(base + (int64_t)row0 * ld), (short)0, 0x7FFFFFFF,
                                                 0x00020000);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int seg = min(wave + j * NW, SEGS - 1);
            const int row = seg * RPS + lane / CPR;
            const int c = chunk_slot<CPR>(row, lane % CPR);
            const int lrow = min(row0 + row, nrows - 1) - row0;
            voff[j] = (uint32_t)(lrow * ld + c * 8) * 2u;
        }
    }

    __device__ __forceinline__ void issue_buf(int k0, uint16_t* lds_tile, int wave) const {
        issue_range(k0, lds_tile, wave, 0, PER);
    }

    // the loads j with lo <= j < hi (all of them: issue_buf)
    __device__ __forceinline__ void issue_range(int k0, uint16_t* lds_tile, int wave, int lo, int hi) const {
        const uint32_t soff = (uint32_t)k0 * 2u;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if (j < lo || j >= hi) continue;
            const int seg = min(wave + j * NW, SEGS - 1);
            const uint32_t l = (uint32_t)(uintptr_t)(
                (__attribute__((address_space(3))) uint16_t*)(lds_tile + seg * 512));
            // Emitted as inline assembly on purpose: the compiler's wait
            // insertion cannot tell the ring buffers apart and would make every
            // later LDS read wait for these loads. Their completion is tracked
            // explicitly with s_waitcnt vmcnt before each step barrier.
            asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff[j]), "s"(rsrc), "s"(soff),
                         "{m0}"(l));
        }
    }

};

// ---------------------------------------------------------------------------
// Shared pieces of the kernels: MFMAs over one LDS stage, and the epilogue.
// ---------------------------------------------------------------------------

template <int FM, int FN, int TM, int TN, int BKS>
__device__ __forceinline__ void mma_stage(const uint16_t* sA, const uint16_t* sB, int wm, int wn,
                                          int lane, f32x16 (&acc)[FM][FN]) {
    constexpr int CPR = BKS / 8;
#pragma unroll
    for (int kk = 0; kk < BKS / 16; ++kk) {
        const int c = kk * 2 + (lane >> 5);
        bf16x8 fa[FM], fb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * TM + i * 32 + (lane & 31);
            fa[i] = *reinterpret_cast<const bf16x8*>(sA + row * BKS + chunk_slot<CPR>(row, c) * 8);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wn * TN + j * 32 + (lane & 31);
            fb[j] = *reinterpret_cast<const bf16x8*>(sB + row * BKS + chunk_slot<CPR>(row, c) * 8);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
}

template <int FM, int FN, int TM, int TN, int BKS>
__device__ __forceinline__ void load_frags(const uint16_t* sA, const uint16_t* sB, int wm, int wn,
                                           int lane, int kk, bf16x8 (&fa)[FM], bf16x8 (&fb)[FN]) {
    constexpr int CPR = BKS / 8;
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = wm * TM + i * 32 + (lane & 31);
        fa[i] = *reinterpret_cast<const bf16x8*>(sA + row * BKS + chunk_slot<CPR>(row, c) * 8);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int row = wn * TN + j * 32 + (lane & 31);
        fb[j] = *reinterpret_cast<const bf16x8*>(sB + row * BKS + chunk_slot<CPR>(row, c) * 8);
    }
}

// Fragment addresses for 64-wide K steps, precomputed. With rows of eight
// 16-byte chunks swizzled by chunk_slot<8>, the chunk a lane reads for
// fragment i at sub-step kk is (2kk + h) ^ s(row), and since every fragment
// starts on a 32-row boundary, s(row of fragment i) = s0 ^ 4(i & 1) with s0
// the swizzle of the lane's row in fragment 0. Hence the byte offset is
// v[kk ^ 2(i & 1)] + 4096 i with four per-lane values v[j] (one table for the
// A fragments, one for B): the per-read work is an immediate offset instead
// of a shift-xor-add chain. (Checked exhaustively against chunk_slot<8> for
// every lane, fragment, sub-step and 32-row-aligned origin.)
struct FragAddr64 {
    uint32_t va[4], vb[4];   // byte offsets from the stage's first A row

    __device__ __forceinline__ static void table(uint32_t (&v)[4], int row0, int lane, uint32_t base) {
        const int row = row0 + (lane & 31), h = lane >> 5;
        const int s0 = (row ^ (row >> 3)) & 7;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = base + (uint32_t)(row * 128 + 16 * (h ^ (s0 & 1)) + 32 * (j ^ (s0 >> 1)));
    }

    template <int BM, int TM, int TN>
    __device__ __forceinline__ void init(int wm, int wn, int lane) {
        table(va, wm * TM, lane, 0u);
        table(vb, wn * TN, lane, (uint32_t)BM * 128u);
    }
};

template <int FM, int FN>
__device__ __forceinline__ void load_frags64(const uint16_t* sA, const FragAddr64& fa_addr, int kk,
                                             bf16x8 (&fa)[FM], bf16x8 (&fb)[FN]) {
    const char* base = reinterpret_cast<const char*>(sA);
#pragma unroll
    for (int i = 0; i < FM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(base + fa_addr.va[kk ^ (2 * (i & 1))] + 4096 * i);
#pragma unroll
    for (int j = 0; j < FN; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(base + fa_addr.vb[kk ^ (2 * (j & 1))] + 4096 * j);
}

// F16: the fragments hold FP16 bit patterns (dequantized FP4), multiplied with
// the FP16 MFMA of the same shape and rate.
template <int FM, int FN, bool F16 = false>
__device__ __forceinline__ void mfma_block(const bf16x8 (&fa)[FM], const bf16x8 (&fb)[FN],
                                           f32x16 (&acc)[FM][FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if constexpr (F16)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fb[j]),
                                                                   __builtin_bit_cast(f16x8, fa[i]), acc[i][j], 0,
                                                                   0, 0);
            else
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }
}

// Scheduling groups for one sub-step: NM MFMAs, ND LDS reads and NV direct
// (VMEM) loads, issued as MFMA, LDS read, VMEM, MFMA, ... until the memory
// instructions run out, then the remaining MFMAs.
template <int NM, int ND, int NV>
__device__ __forceinline__ void interleave_mfma() {
#pragma unroll
    for (int q = 0; q < NM; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                     // MFMA
        if (q < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // LDS read
        if (q < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);         // VMEM read
    }
    if (NV > NM) __builtin_amdgcn_sched_group_barrier(0x020, NV - NM, 0);
    if (ND > NM) __builtin_amdgcn_sched_group_barrier(0x100, ND - NM, 0);
}

// Sub-step schedule with operand conversion: NM MFMAs, each followed by an
// LDS read (while ND last), up to NV VALU and up to NW LDS writes (spread
// evenly), so the conversion's VALU work issues under the matrix core's
// busy cycles.
template <int NM, int ND, int NV, int NW>
__device__ __forceinline__ void interleave_mfma_cvt() {
    constexpr int V = (NV + NM - 1) / NM, W = (NW + NM - 1) / NM;
#pragma unroll
    for (int q = 0; q < NM; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                     // MFMA
        if (q < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // LDS read
        if (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);          // VALU
        if (W > 0 && q * W < NW) __builtin_amdgcn_sched_group_barrier(0x200, W, 0);   // LDS write
    }
    if (ND > NM) __builtin_amdgcn_sched_group_barrier(0x100, ND - NM, 0);
}

// Epilogue through LDS: each wave writes its accumulator tile into LDS, then
// the whole workgroup streams complete rows to memory, 16 contiguous bytes
// per lane (a wave covers 1 KB of consecutive row bytes per store), instead
// of each lane scattering 8-byte pieces over 32 rows. 16-byte chunks are
// rotated by row within LDS. When the tile does not fit the LDS
// capacity (FP32 planes), rows are staged in passes of whole wave rows.
template <int EPI, int BM, int BN, int WM, int WN, int FM, int FN, int NT, int CAP, int NPRE = 0>
__device__ __forceinline__ void staged_epilogue(const KParams& p, const f32x16 (&acc)[FM][FN],
                                                uint8_t* lds, int m0, int n0, int wm, int wn,
                                                int lane, int tid, int split,
                                                const u32x4* pre = nullptr, void* c_base = nullptr,
                                                bool writer = true) {
    // `writer` false: this wave holds no part of the tile (the second K half
    // of a sliced-K workgroup) and only helps stream the staged rows
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int ELEM = (EPI == EPI_STORE_F32) ? 4 : 2;
    constexpr int ROWB = BN * ELEM;            // bytes per staged row
    constexpr int CPR16 = ROWB / 16;           // 16-byte chunks per row
    constexpr int ROWS_FIT = CAP / ROWB;
    constexpr int RP = (ROWS_FIT >= BM) ? BM : (ROWS_FIT / 32) * 32;   // rows per pass
    static_assert(RP >= 32, "a pass holds at least one 32-row MFMA block");
    constexpr int NPASS = (BM + RP - 1) / RP;
    constexpr int EPC = 16 / ELEM;             // elements per chunk
    const int M = p.M, N = p.N, ldc = p.ldc;
    void* const Cb = c_base != nullptr ? c_base : p.C;   // the output (a dual launch's second one)
    const bool vec_ok = (N % EPC) == 0 && (ldc % EPC) == 0;

    // chunks rotate by the row index, so the 32 rows one store instruction
    // covers spread over the banks for any row length
    auto slot = [](int row, int chunk) { return row * ROWB + (((chunk + row) % CPR16) << 4); };

#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        lds_barrier();   // previous users of LDS (main loop or previous pass) are done
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int blk = wm * TM + i * 32;            // first row of this MFMA row block
            if (!writer || blk < pass * RP || blk >= (pass + 1) * RP) continue;
            const int row = blk + (lane & 31) - pass * RP;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n_local = wn * TN + j * 32 + g * 8 + (lane >> 5) * 4;
                    const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
                    const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
                    if constexpr (EPI == EPI_STORE_F32) {
                        *reinterpret_cast<f32x4*>(lds + slot(row, n_local >> 2)) = f32x4{v0, v1, v2, v3};
                    } else if constexpr (EPI == EPI_SCALE_BF16) {
                        const float sc = p.scale;   // one FP32 multiply, then the BF16 rounding
                        *reinterpret_cast<u32x2*>(lds + slot(row, n_local >> 3) + (lane >> 5) * 8) =
                            u32x2{pack_bf16x2(v0 * sc, v1 * sc), pack_bf16x2(v2 * sc, v3 * sc)};
                    } else {
                        *reinterpret_cast<u32x2*>(lds + slot(row, n_local >> 3) + (lane >> 5) * 8) =
                            u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                    }
                }
            }
        }
        lds_barrier();
        const int rows_here = min(RP, BM - pass * RP);
        constexpr int ITER = (RP * CPR16 + NT - 1) / NT;
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int q = tid + it * NT;
            if (q >= rows_here * CPR16) break;
            const int row = q / CPR16, chunk = q % CPR16;
            const int m = m0 + pass * RP + row;
            const int n = n0 + chunk * EPC;
            if (m >= M || n >= N) continue;
            const u32x4 w = *reinterpret_cast<const u32x4*>(lds + slot(row, chunk));
            const int64_t off = (int64_t)m * ldc + n;
            const bool full = vec_ok && n + EPC <= N;
            if constexpr (EPI == EPI_STORE_F32) {
                float* plane = reinterpret_cast<float*>(Cb) + (int64_t)split * M * ldc;
                if (full) {
                    *reinterpret_cast<u32x4*>(plane + off) = w;
                } else {
                    const uint32_t e4[4] = {w.x, w.y, w.z, w.w};
                    for (int e = 0; e < 4 && n + e < N; ++e) plane[off + e] = __builtin_bit_cast(float, e4[e]);
                }
            } else if constexpr (EPI == EPI_STORE_BF16 || EPI == EPI_SCALE_BF16) {
                uint16_t* C = reinterpret_cast<uint16_t*>(Cb);
                if (full) {
                    // Non-temporal: the output does not displace operands
                    // (this GEMM's or the next one's) from the L2s and the
                    // Infinity Cache. MLP step 586.5 -> 571.9 us, Q/O 39.0 ->
                    // 37.8 us, down 185.7 -> 184.1 us in an interleaved A/B.
                    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(C + off));
                } else {
                    const uint32_t e4[4] = {w.x, w.y, w.z, w.w};
                    for (int e = 0; e < 8 && n + e < N; ++e) C[off + e] = (uint16_t)(e4[e >> 1] >> ((e & 1) * 16));
                }
            } else {  // EPI_SCALED_ACC: out = bf16(out + scale * delta), delta already BF16
                uint16_t* O = reinterpret_cast<uint16_t*>(Cb);
                const float sc = p.scale;
                const uint32_t d4[4] = {w.x, w.y, w.z, w.w};
                if (full) {
                    u32x4 o;
                    if constexpr (NPRE > 0)
                        o = pre[it];   // loaded at kernel start (single pass)
                    else
                        o = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(O + off));
                    const uint32_t o4[4] = {o.x, o.y, o.z, o.w};
                    uint32_t r4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = bf16_lo(o4[e]) + sc * bf16_lo(d4[e]);
                        const float hi = bf16_hi(o4[e]) + sc * bf16_hi(d4[e]);
                        r4[e] = pack_bf16x2(lo, hi);
                    }
                    // `out` is streamed once: non-temporal, so it does not displace cached data
                    __builtin_nontemporal_store(u32x4{r4[0], r4[1], r4[2], r4[3]}, reinterpret_cast<u32x4*>(O + off));
                } else {
                    for (int e = 0; e < 8 && n + e < N; ++e) {
                        const uint32_t dh = (d4[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
                        const float o = __builtin_bit_cast(float, (uint32_t)O[off + e] << 16);
                        const float r = o + sc * __builtin_bit_cast(float, dh << 16);
                        O[off + e] = (uint16_t)pack_bf16x2(r, 0.0f);
                    }
                }
            }
        }
    }
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 in order.
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

template <int FM, int FN>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[FM][FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// ---------------------------------------------------------------------------
// Kernel 1: register-staged operands (FP4 with in-register dequantization,
// and BF16 rows whose pitch is not a multiple of 16 bytes). Global loads go
// to registers two steps ahead (two register sets, loop unrolled by two);
// during step t the set holding step t+1 is converted (FP4 -> exact FP16)
// and written into the LDS buffer that step t-1 released, interleaved with
// step t's MFMAs. Same MFMA / LDS-read interleave, step barrier placement
// and LDS-staged epilogue as kernel 2.
// ---------------------------------------------------------------------------

template <int BM, int BN, int WM, int WN, int EPI, int SRC, int RSETS = 2>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_mfma_kernel(KParams p) {
    if constexpr (src_fp4(SRC)) {
        const int64_t l = blockIdx.z;   // batch index (0 for one problem)
        p.Aq += l * p.bs_a;
        p.SFA += l * p.bs_sa;
        p.Bq += l * p.bs_b;
        p.SFB += l * p.bs_sb;
        p.C = reinterpret_cast<uint16_t*>(p.C) + l * p.bs_c;
    }
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;   // wave sub-tile
    constexpr int FM = TM / 32, FN = TN / 32;   // 32x32 MFMA blocks per wave
    static_assert(FM * 32 * WM == BM && FN * 32 * WN == BN, "bad tile split");
    constexpr int STAGE = (BM + BN) * BK;       // BF16 elements per LDS stage
    constexpr int KK = BK / 16;
    constexpr int LAST = (KK - 1) & 1;

    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int tm, tn;
    tile_of_block(p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int split = blockIdx.y;
    const int kb = (int)min((int64_t)p.K, (int64_t)split * p.k_chunk);
    const int ke = (int)min((int64_t)p.K, (int64_t)kb + p.k_chunk);
    const int nsteps = (ke - kb + BK - 1) / BK;   // the last step may be ragged (masked loads)

    f32x16 acc[FM][FN];
    zero_acc(acc);

    constexpr int SRC_A = src_w4a16(SRC) ? SRC_BF16_VEC : SRC;
    constexpr int SRC_B = SRC == SRC_W4A16    ? SRC_FP4_BF16
                          : SRC == SRC_W4A16W   ? SRC_FP4W_BF16
                          : SRC == SRC_W4A16T4  ? SRC_FP4T4_BF16
                          : SRC == SRC_W4A16T1  ? SRC_FP4T1_BF16
                                                : SRC;
    // RSETS register sets form a ring: set r holds the steps t with t % RSETS == r
    constexpr int NSETS = RSETS > 1 ? RSETS : 1;
    Stager<BM, NT, SRC_A> sa[NSETS];
    Stager<BN, NT, SRC_B> sb[NSETS];
    Stager<BM, NT, SRC_A>& sa0 = sa[0];
    Stager<BN, NT, SRC_B>& sb0 = sb[0];
    auto load = [&](auto& sa, auto& sb, int k0) {
        if constexpr (src_fp4(SRC)) {
            sa.load(p.Aq, p.SFA, m0, p.M, p.K, k0, ke, tid);
            sb.load(p.Bq, p.SFB, n0, p.N, p.K, k0, ke, tid);
        } else if constexpr (src_w4a16t(SRC)) {
            sa.load(p.A, m0, p.M, p.lda, k0, ke, tid);
            sb.load(p.Bq, p.SFB, n0, p.N, p.ldbt, p.K, k0, ke, tid);
        } else if constexpr (src_w4a16(SRC)) {
            sa.load(p.A, m0, p.M, p.lda, k0, ke, tid);
            sb.load(p.Bq, p.SFB, n0, p.N, p.K, k0, ke, tid);
        } else {
            sa.load(p.A, m0, p.M, p.lda, k0, ke, tid);
            sb.load(p.B, n0, p.N, p.ldb, k0, ke, tid);
        }
    };
    auto store = [&](auto& sa, auto& sb, uint16_t* buf) {
        sa.store(buf, tid);
        sb.store(buf + BM * BK, tid);
    };

    if (nsteps > 0) {
        load(sa0, sb0, kb);
        store(sa0, sb0, smem);
        // the other sets are loaded even past the end (clamped, zero-masked
        // loads), so the loop below is one basic block with exact waits
#pragma unroll
        for (int r = 1; r < NSETS; ++r) load(sa[r], sb[r], kb + r * BK);
    }
    lds_barrier();

    bf16x8 fa[2][FM], fb[2][FN];
    FragAddr64 fadr;
    fadr.init<BM, TM, TN>(wm, wn, lane);
    if (nsteps > 0) load_frags64<FM, FN>(smem, fadr, 0, fa[0], fb[0]);

    // Conversion of the held set is spread over the KK-1 leading sub-steps:
    // part kk covers units [U*kk/(KK-1), U*(kk+1)/(KK-1)) of the U = PA + PB
    // units (A's first), interleaved with that sub-step's MFMAs.
    constexpr int PA = Stager<BM, NT, SRC_A>::PER, PB = Stager<BN, NT, SRC_B>::PER, U = PA + PB;
    // approximate VALU instructions and LDS writes per unit, for the schedule
    // (per 16 FP4 elements: 24 to FP16, 32 to BF16, and two 16-byte writes)
    constexpr int UEA = fp4_unit(SRC_A, BM, NT), UEB = fp4_unit(SRC_B, BN, NT);
    constexpr int VU_A = src_fp4(SRC_A) ? 24 * UEA / 16 : 0;
    // (a transposed-weight unit: 64 elements, about 150 VALU, eight writes)
    constexpr int VU_B = src_fp4t(SRC_B) ? 150 : src_fp4(SRC_B) ? 24 * UEB / 16 : UEB * 2;
    constexpr int WU_A = UEA ? UEA / 8 : 1;
    constexpr int WU_B = src_fp4t(SRC_B) ? 8 : UEB ? UEB / 8 : 1;
    constexpr int CVT_VALU = (PA * VU_A + PB * VU_B + KK - 2) / (KK - 1);
    constexpr int CVT_DSW = (PA * WU_A + PB * WU_B + KK - 2) / (KK - 1);
    auto store_part = [&](auto& sa, auto& sb, uint16_t* buf, int part) {
        const int lo = U * part / (KK - 1), hi = U * (part + 1) / (KK - 1);
        sa.store_units(buf, tid, lo, min(hi, PA));
        sb.store_units(buf + BM * BK, tid, max(lo - PA, 0), hi - PA);
    };

    // One K step. `held` carries step t+1 (loaded RSETS-1 steps ago), `next`
    // (step t's set, converted during step t-1) receives step t+RSETS. Loads
    // past the last step read clamped addresses and convert to zeros, so
    // nothing here branches.
    auto step = [&](int t, auto& held_a, auto& held_b, auto& next_a, auto& next_b) {
        const uint16_t* sA = smem + (t & 1) * STAGE;
        uint16_t* dst = smem + ((t + 1) & 1) * STAGE;
        load(next_a, next_b, kb + (t + NSETS) * BK);
        __builtin_amdgcn_sched_barrier(0);   // the loads lead the step: a whole step covers their latency
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
            const int cur = kk & 1;
            load_frags64<FM, FN>(sA, fadr, kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
            store_part(held_a, held_b, dst, kk);
            mfma_block<FM, FN, src_fp4(SRC)>(fa[cur], fb[cur], acc);
            interleave_mfma_cvt<FM * FN, FM + FN, CVT_VALU, CVT_DSW>();
        }
        // step t+1 is in LDS for every wave; step t's buffer is free. Past the
        // last step this reads a buffer of zeros (harmless).
        lds_barrier();
        const uint16_t* nA = smem + ((t + 1) & 1) * STAGE;
        load_frags64<FM, FN>(nA, fadr, 0, fa[LAST ^ 1], fb[LAST ^ 1]);
        mfma_block<FM, FN, src_fp4(SRC)>(fa[LAST], fb[LAST], acc);
        interleave_mfma<FM * FN, FM + FN, 0>();
    };

    // One register set: step t+1 is loaded at the start of step t and
    // converted / stored before step t's last sub-step (less latency cover,
    // fewer registers).
    auto step1 = [&](int t) {
        const uint16_t* sA = smem + (t & 1) * STAGE;
        // Past the last step the masked loads return zeros without touching
        // memory and the store lands in a buffer nobody reads again, so both
        // run unconditionally and stay in one basic block with the MFMAs.
        load(sa0, sb0, kb + (t + 1) * BK);
        __builtin_amdgcn_sched_barrier(0);   // keep the loads at the top: their latency spans the step
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
            const int cur = kk & 1;
            load_frags64<FM, FN>(sA, fadr, kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
            if (kk == KK - 2) {
                // not earlier: hoisted conversions would wait for the loads
                // just issued
                __builtin_amdgcn_sched_barrier(0);
                store(sa0, sb0, smem + ((t + 1) & 1) * STAGE);
                mfma_block<FM, FN, src_fp4(SRC)>(fa[cur], fb[cur], acc);
                interleave_mfma_cvt<FM * FN, FM + FN, CVT_VALU * (KK - 1), CVT_DSW * (KK - 1)>();
            } else {
                mfma_block<FM, FN, src_fp4(SRC)>(fa[cur], fb[cur], acc);
                interleave_mfma<FM * FN, FM + FN, 0>();
            }
        }
        if (t + 1 < nsteps) {
            lds_barrier();
            const uint16_t* nA = smem + ((t + 1) & 1) * STAGE;
            load_frags64<FM, FN>(nA, fadr, 0, fa[LAST ^ 1], fb[LAST ^ 1]);
        }
        mfma_block<FM, FN, src_fp4(SRC)>(fa[LAST], fb[LAST], acc);
        interleave_mfma<FM * FN, FM + FN, 0>();
    };

    if constexpr (RSETS > 1) {
        // whole rounds of RSETS steps: steps past the end multiply zeros
        for (int t = 0; t < nsteps; t += NSETS)
            static_for<NSETS>([&](auto rc) {
                constexpr int r = decltype(rc)::value;
                step(t + r, sa[(r + 1) % NSETS], sb[(r + 1) % NSETS], sa[r], sb[r]);
            });
    } else {
        for (int t = 0; t < nsteps; ++t) step1(t);
    }

    staged_epilogue<EPI, BM, BN, WM, WN, FM, FN, NT, 2 * STAGE * 2>(
        p, acc, reinterpret_cast<uint8_t*>(smem), m0, n0, wm, wn, lane, tid, split);
}

// ---------------------------------------------------------------------------
// Kernel 1b: FP4 x FP4 for few rows (decode shapes), K % 64 == 0, one
// problem. A 128 x 256 tile, four waves of 128 x 64 (WM = 1: every wave
// covers all the rows, so each weight column belongs to one wave) or eight
// waves of 64 x 64 (WM = 2: the two row halves each dequantize the weight
// columns they share, so that a second wave per SIMD overlaps one wave's
// dequantization with the other's MFMAs; the default). BN = 128 halves the
// tile's columns (eight waves of 64 x 32), for split counts that leave CUs
// idle with 256 columns.
//
// The register-staged kernel at these shapes sends about 770 L1-to-L2
// requests per 64-wide step (32 bytes of packed data and 4 scale bytes from
// each of the tile's 384 rows, one request each) and runs at about 64 in
// flight per CU at ~300 cycles each. Here the packed bytes and scales of
// four steps (one 128-byte line of data per row) go straight to LDS rings
// with direct loads whose 64 lanes cover 8 whole rows: about 190 requests
// per step. (Measured on MI355X: the rings alone gained 7% on 128 x 7168 x
// 16384; the second wave per SIMD of WM = 2 most of the rest.)
//
//   raw rings (two groups of 4 steps): A 128 x 128 B, B 256 x 128 B, their
//     scales 16 B per row; the lane that lands in slot c of a row fetches the
//     row's logical 16-byte chunk chunk_slot<8>(row, c)
//   A: each thread dequantizes one 32-element (WM = 1) or 16-element unit per
//     step from the raw ring into an FP16 stage (two stages), read as MFMA
//     fragments as elsewhere
//   B: each lane reads its column's 16 bytes and 2 scale bytes of the step
//     from the ring and dequantizes them into its MFMA operand registers
//
// K order inside a step: at sub-step kk, lane half h holds k = 32h + 8kk ..
// 32h + 8kk + 7 in both operands, so a lane's four sub-steps of B are one
// 16-byte read. The MFMA sums the same products over the step, in its own
// order, as with the natural order.
// ---------------------------------------------------------------------------
template <int EPI, int WM, int BN = 256>
__global__ void __launch_bounds__(256 * WM)
gemm_fp4_dec_kernel(KParams p) {
    constexpr int BM = 128, WN = 4, NW = WM * WN, NT = 64 * NW;
    constexpr int TM = BM / WM, TN = BN / WN;     // 128 (or 64) x 64 per wave
    constexpr int FM = TM / 32, FN = TN / 32;     // 4 (or 2) x 2 MFMA blocks
    static_assert(WM == 1 || WM == 2, "one or two row halves");
    constexpr int G = 4;                          // steps per raw group (one 128-byte line per row)
    constexpr int R = 2 * G;                      // steps per loop round (both raw buffers)
    // LDS map (bytes)
    constexpr int RAW_B = 0;                              // [2][256][128]
    constexpr int RAW_A = RAW_B + 2 * BN * 128;           // [2][128][128]
    constexpr int SC_B = RAW_A + 2 * BM * 128;            // [2][256][16]
    constexpr int SC_A = SC_B + 2 * BN * 16;              // [2][128][16]
    constexpr int F16_A = SC_A + 2 * BM * 16;             // [2][128][64] FP16
    constexpr int LDS_BYTES = F16_A + 2 * BM * BK * 2;    // 143360
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, h = lane >> 5;
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_of_block(p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int split = blockIdx.y;
    const int kb = (int)min((int64_t)p.K, (int64_t)split * p.k_chunk);
    const int ke = (int)min((int64_t)p.K, (int64_t)kb + p.k_chunk);
    const int nsteps = (ke - kb) / BK;            // whole steps: K and the chunk are multiples of 64

    f32x16 acc[FM][FN];
    zero_acc(acc);

    if (nsteps > 0) {
        const int kh = p.K >> 1, ks = p.K >> 4;   // bytes per row: packed data, scales
        // Buffer resources from the tile's first row to the end of each
        // matrix: a lane reading past the end (a group that runs past K on
        // the last row) gets zeros. Rows past M or N are clamped.
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(p.Aq + (int64_t)m0 * kh), (short)0, (p.M - m0) * kh, 0x00020000);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(p.Bq + (int64_t)n0 * kh), (short)0, (p.N - n0) * kh, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(p.SFA + (int64_t)m0 * ks), (short)0, (p.M - m0) * ks, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(p.SFB + (int64_t)n0 * ks), (short)0, (p.N - n0) * ks, 0x00020000);
        const uint32_t zero = __builtin_amdgcn_readfirstlane(0u);

        // Per-lane row offsets of this wave's direct loads: data segments of
        // 8 rows (B: 32 segments, A: 16, dealt out evenly), scale segments of
        // 64 rows (B: segment `wave` of waves 0-3; A: segments 0 and 1, from
        // waves 0-1 with four waves, 4-5 with eight)
        constexpr int SB = BN / 8 / NW, SA = 16 / NW;   // data segments per wave
        const int asw = NW == 8 ? wave - 4 : wave;   // A-scale segment of this wave (0 or 1 loads)
        uint32_t vb[SB], va[SA];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int row = (wave * SB + j) * 8 + lane / 8;
            const int lrow = min(n0 + row, p.N - 1) - n0;
            vb[j] = (uint32_t)(lrow * kh + chunk_slot<8>(row, lane % 8) * 16);
        }
#pragma unroll
        for (int j = 0; j < SA; ++j) {
            const int row = (wave * SA + j) * 8 + lane / 8;
            const int lrow = min(m0 + row, p.M - 1) - m0;
            va[j] = (uint32_t)(lrow * kh + chunk_slot<8>(row, lane % 8) * 16);
        }
        const uint32_t vsb = (uint32_t)((min(n0 + (wave & 3) * 64 + lane, p.N - 1) - n0) * ks);
        const uint32_t vsa = (uint32_t)((min(m0 + (asw & 1) * 64 + lane, p.M - 1) - m0) * ks);

        // group g (steps 4g .. 4g+3 of this split) into raw buffer g % 2
        auto load_group = [&](int g) {
            const int k = kb + g * G * BK;
            const uint32_t kd = (uint32_t)(k >> 1), kss = (uint32_t)(k >> 4);
            const int buf = g & 1;
            // Inline assembly: the compiler's wait insertion cannot tell the
            // ring buffers apart; completion is waited for explicitly (vmcnt)
            // before the barrier that publishes the group.
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const uint32_t l = (uint32_t)(uintptr_t)(
                    (__attribute__((address_space(3))) uint8_t*)(lds + RAW_B + buf * BN * 128 + (wave * SB + j) * 1024));
                asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(vb[j] + kd), "s"(rb), "s"(zero),
                             "{m0}"(l));
            }
#pragma unroll
            for (int j = 0; j < SA; ++j) {
                const uint32_t l = (uint32_t)(uintptr_t)(
                    (__attribute__((address_space(3))) uint8_t*)(lds + RAW_A + buf * BM * 128 + (wave * SA + j) * 1024));
                asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(va[j] + kd), "s"(ra), "s"(zero),
                             "{m0}"(l));
            }
            if (wave < BN / 64) {
                const uint32_t l = (uint32_t)(uintptr_t)(
                    (__attribute__((address_space(3))) uint8_t*)(lds + SC_B + buf * BN * 16 + wave * 1024));
                asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(vsb + kss), "s"(rsb), "s"(zero),
                             "{m0}"(l));
            }
            if (asw >= 0 && asw < 2) {
                const uint32_t l = (uint32_t)(uintptr_t)(
                    (__attribute__((address_space(3))) uint8_t*)(lds + SC_A + buf * BM * 16 + asw * 1024));
                asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(vsa + kss), "s"(rsa), "s"(zero),
                             "{m0}"(l));
            }
        };

        // B: this lane's column of each column block, its step-s chunk (2s + h)
        const int brow0 = wn * TN + (lane & 31);
        uint32_t boff[FN][G], bsoff[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = brow0 + j * 32;
#pragma unroll
            for (int st = 0; st < G; ++st) boff[j][st] = (uint32_t)(row * 128 + chunk_slot<8>(row, 2 * st + h) * 16);
            bsoff[j] = (uint32_t)(row * 16 + 2 * h);
        }
        auto read_b = [&](int buf, int st, u32x4 (&w)[FN], uint32_t (&sc)[FN]) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                w[j] = *reinterpret_cast<const u32x4*>(lds + RAW_B + buf * BN * 128 + boff[j][st]);
                sc[j] = *reinterpret_cast<const uint16_t*>(lds + SC_B + buf * BN * 16 + bsoff[j] + 4 * st);
            }
        };
        using Deq = Fp4Stager<BM, 256, true, 32>;
        auto deq_b = [&](const u32x4 (&w)[FN], const uint32_t (&sc)[FN], int kk, bf16x8 (&fb)[FN]) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const f16x2 s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[j], 1.0f, false);
                const f16x2 s16 = kk < 2 ? f16x2{s2.x, s2.x} : f16x2{s2.y, s2.y};
                fb[j] = __builtin_bit_cast(bf16x8, Deq::deq8(w[j][kk], s16, 0.0f));
            }
        };

        // A: thread tid's unit is row tid / UPR, elements UE*u .. UE*u + UE - 1
        // (u = tid % UPR): 32 elements with four waves, 16 with eight
        constexpr int UE = 32 / WM, UPR = BK / UE;
        const int arow = tid / UPR, au = tid % UPR;
        uint32_t aroff[G];
#pragma unroll
        for (int st = 0; st < G; ++st)
            // step st's packed bytes of the row start at 32 st; the unit's at
            // 32 st + UE*au/2: 16-byte chunk 2 st + UE*au/32, byte (UE*au/2) % 16
            aroff[st] = (uint32_t)(arow * 128 + chunk_slot<8>(arow, 2 * st + (UE * au) / 32) * 16 + ((UE * au) / 2) % 16);
        const uint32_t asoff = (uint32_t)(arow * 16 + (UE * au) / 16);
        uint32_t adst[UE / 8];   // FP16 stage byte offsets of the unit's 8-element chunks
#pragma unroll
        for (int c = 0; c < UE / 8; ++c) adst[c] = (uint32_t)(arow * 128 + chunk_slot<8>(arow, (UE / 8) * au + c) * 16);
        typedef uint32_t AWords __attribute__((ext_vector_type(UE / 8)));
        auto read_a = [&](int buf, int st, AWords& w, uint32_t& sc) {
            w = *reinterpret_cast<const AWords*>(lds + RAW_A + buf * BM * 128 + aroff[st]);
            if constexpr (UE == 32)
                sc = *reinterpret_cast<const uint16_t*>(lds + SC_A + buf * BM * 16 + asoff + 4 * st);
            else
                sc = *(lds + SC_A + buf * BM * 16 + asoff + 4 * st);
        };
        auto store_a = [&](int stage, const AWords& w, uint32_t sc) {
            const f16x2 s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false);
#pragma unroll
            for (int c = 0; c < UE / 8; ++c) {
                const f16x2 s16 = c < 2 ? f16x2{s2.x, s2.x} : f16x2{s2.y, s2.y};
                *reinterpret_cast<u32x4*>(lds + F16_A + stage * BM * BK * 2 + adst[c]) = Deq::deq8(w[c], s16, 0.0f);
            }
        };

        // A fragment byte offsets within an FP16 stage: row-block i, sub-step
        // kk reads chunk 4h + kk of row 32i + (lane & 31); the swizzle of row
        // 32i + r is that of r with bit 2 flipped for odd i
        uint32_t aoff[2][4];
        {
            const int r = lane & 31;
#pragma unroll
            for (int par = 0; par < 2; ++par)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    aoff[par][kk] = (uint32_t)((32 * par + r) * 128 + chunk_slot<8>(32 * par + r, 4 * h + kk) * 16);
        }
        auto load_fa = [&](int stage, int kk, bf16x8 (&fa)[FM]) {
            const uint8_t* base = lds + F16_A + stage * BM * BK * 2 + 4096 * FM * wm;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const bf16x8*>(base + aoff[i & 1][kk] + 4096 * (i & ~1));
        };

        // prologue: group 0 in raw buffer 0, step 0's A in FP16 stage 0 and
        // its B in registers
        load_group(0);
        wait_vmcnt<0>();
        lds_barrier();
        u32x4 bw[2][FN];
        AWords aw;
        uint32_t bsc[2][FN], asc;
        read_a(0, 0, aw, asc);
        store_a(0, aw, asc);
        read_b(0, 0, bw[0], bsc[0]);
        lds_barrier();
        bf16x8 fa[2][FM], fb[2][FN];
        load_fa(0, 0, fa[0]);
        deq_b(bw[0], bsc[0], 0, fb[0]);

        // step t = round start + r: raw buffer (r / G), step-in-group r % G,
        // FP16 stage t % 2, B registers r % 2 (the next step's in (r+1) % 2).
        // Each sub-step fetches the next one's A fragments and dequantizes
        // its B operands while its own 8 MFMAs (8 accumulators) run; a
        // scheduling boundary after each sub-step keeps the MFMAs on one
        // accumulator 8 apart.
        // One barrier per step, after sub-step 2: it publishes step t+1's
        // FP16 stage (written in sub-step 2), so sub-step 3 fetches that
        // step's first fragments under its own MFMAs. Stage (t+1) % 2 was last
        // read in sub-step 2 of step t-1, before that step's barrier; a raw
        // buffer is last read two barriers before its next group is loaded.
        auto step = [&](int t, auto rc) {
            constexpr int r = decltype(rc)::value;
            constexpr int st = r % G, cur = r % 2, nx = (r + 1) % 2;
            constexpr int nbuf = ((r + 1) % R) / G, nst = (r + 1) % G;   // where step t+1 lives
            if constexpr (st == 0) load_group(t / G + 1);   // the next group, 4 steps ahead
            __builtin_amdgcn_sched_barrier(0);
            static_for<4>([&](auto kc) {
                constexpr int kk = decltype(kc)::value;
                if constexpr (kk == 0) read_a(nbuf, nst, aw, asc);           // step t+1's A unit
                if constexpr (kk == 1) read_b(nbuf, nst, bw[nx], bsc[nx]);   // step t+1's B
                if constexpr (kk == 2) store_a(nx, aw, asc);
                if constexpr (kk + 1 < 4) {
                    load_fa(cur, kk + 1, fa[(kk + 1) & 1]);
                    deq_b(bw[cur], bsc[cur], kk + 1, fb[(kk + 1) & 1]);
                } else {
                    load_fa(nx, 0, fa[0]);                  // sub-step 0 of step t+1
                    deq_b(bw[nx], bsc[nx], 0, fb[0]);
                }
                mfma_block<FM, FN, true>(fa[kk & 1], fb[kk & 1], acc);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (kk == 2) {
                    // the next group's loads are complete for this wave
                    // before the barrier that precedes the first read of that
                    // group (sub-step 0 of the group's last step)
                    if constexpr (st == G - 2) wait_vmcnt<0>();
                    lds_barrier();
                }
            });
        };
        // whole rounds of R steps, then the remaining steps one by one (no
        // work past the last step)
        int t = 0;
        for (; t + R <= nsteps; t += R)
            static_for<R>([&](auto rc) { step(t + decltype(rc)::value, rc); });
        if (t < nsteps)
            static_for<R - 1>([&](auto rc) {
                if (t + decltype(rc)::value < nsteps) step(t + decltype(rc)::value, rc);
            });
        // direct loads still in flight (a group past the last step) must land
        // before the epilogue reuses LDS
        wait_vmcnt<0>();
    }

    staged_epilogue<EPI, BM, BN, WM, WN, FM, FN, NT, 65536>(p, acc, lds, m0, n0, wm, wn, lane, tid, split);
}

// ---------------------------------------------------------------------------
// Kernel 2: BF16 operands with K % 8 == 0. Whole BKS steps are loaded straight
// into LDS (no VGPR round trip, no LDS write instructions) through a ring of
// STAGES buffers: the loads for step t + STAGES - 1 are issued while step t
// is multiplied, so STAGES - 1 steps of MFMA work cover the load latency.
// ---------------------------------------------------------------------------

// Multiplies the K range [kb, ke) of the BM x BN tile at (m0, n0) into acc.
// LDS must be free on entry (the caller's barrier); on return every direct
// load has landed and LDS may be reused once the workgroup has passed a
// barrier. `extra` runs right after the prologue's loads are issued and may
// issue up to NEXTRA more vector load instructions per wave; it returns true
// (uniformly) only when every wave issued exactly NEXTRA, which lets the
// first wait leave them in flight. Otherwise the first wait counts none of
// them and so also waits for whichever were issued.
template <int BM, int BN, int BKS, int WM, int WN, int STAGES, int NEXTRA, class Extra>
__device__ __forceinline__ void direct_mainloop(const KParams& p, const uint16_t* Bop, uint16_t* smem, int m0,
                                                int n0, int kb, int ke, int wave, int lane, int tid,
                                                f32x16 (&acc)[BM / WM / 32][BN / WN / 32], Extra&& extra) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int STAGE = (BM + BN) * BKS;
    // direct-load instructions one wave issues per step
    constexpr int L = DirectStager<BM, NT, BKS>::PER + DirectStager<BN, NT, BKS>::PER;
    const int wm = wave / WN, wn = wave % WN;

    // A ragged K remainder (length not a multiple of BKS) is taken as the
    // FIRST step, through the guarded register path; every later step is a
    // whole BKS step loaded directly. The FP32 summation order inside the
    // MFMAs is unspecified, so visiting the remainder first changes nothing
    // the interface promises.
    const int ragged = (ke - kb) % BKS;
    const int nsteps = (ke - kb) / BKS + (ragged ? 1 : 0);

    DirectStager<BM, NT, BKS> dsa;
    DirectStager<BN, NT, BKS> dsb;
    dsa.init(p.A, m0, p.M, p.lda, wave, lane);
    dsb.init(Bop, n0, p.N, p.ldb, wave, lane);
    auto issue = [&](int k0, uint16_t* buf) {
        dsa.issue_buf(k0, buf, wave);
        dsb.issue_buf(k0, buf + BM * BKS, wave);
    };
    // Part q of KK of one stage's loads (A's first, then B's): a stage
    // refilled inside the loop is issued over KK sub-steps instead of at once,
    // which spreads the chip's L2 requests over the whole step.
    constexpr int PA = DirectStager<BM, NT, BKS>::PER;
    auto issue_part = [&](int k0, uint16_t* buf, int q) {
        constexpr int NP = BKS / 16;
        const int lo = L * q / NP, hi = L * (q + 1) / NP;
        dsa.issue_range(k0, buf, wave, lo, min(hi, PA));
        dsb.issue_range(k0, buf + BM * BKS, wave, max(lo - PA, 0), hi - PA);
    };

    // Direct loads are issued at a uniform rate: STAGES stages in the
    // prologue and exactly one per loop iteration, so "stage t+1 has landed"
    // is always "at most (STAGES-2)*L direct loads are still in flight".
    // Stages past the end re-load the last whole step (a valid address whose
    // buffer is never read again) instead of branching.
    const bool has_full = (ke - kb) >= BKS;
    const int k_last = ke - BKS;   // start of the last whole step (valid when has_full)
    int k_next = kb;
    if (ragged) {
        Stager<BM, NT, SRC_BF16_VEC, BKS> sa;
        Stager<BN, NT, SRC_BF16_VEC, BKS> sb;
        sa.load(p.A, m0, p.M, p.lda, kb, kb + ragged, tid);
        sb.load(Bop, n0, p.N, p.ldb, kb, kb + ragged, tid);
        sa.store(smem, tid);
        sb.store(smem + BM * BKS, tid);
        k_next = kb + ragged;
    } else if (has_full) {
        issue(k_next, smem);
        k_next += BKS;
    }
    if (has_full) {
#pragma unroll
        for (int st = 1; st < STAGES; ++st) {
            issue(min(k_next, k_last), smem + st * STAGE);
            k_next += BKS;
        }
    }
    if (extra())
        wait_vmcnt<(STAGES - 1) * L + NEXTRA>();
    else
        wait_vmcnt<(STAGES - 1) * L>();
    lds_barrier();

    // Sub-step kk of a step multiplies fragments loaded during sub-step kk-1
    // while the fragments of kk+1 are read; MFMAs and LDS reads alternate.
    // The barrier that retires step t sits before its LAST sub-step's MFMAs
    // (their fragments are already in registers), so the matrix core has work
    // while the freed buffer is refilled and step t+1's first fragments are
    // fetched.
    constexpr int KK = BKS / 16;
    static_assert(KK % 2 == 0, "fragment double buffer assumes an even sub-step count");
    constexpr int LAST = (KK - 1) & 1;
    bf16x8 fa[2][FM], fb[2][FN];
    FragAddr64 fadr;
    if constexpr (BKS == 64) fadr.init<BM, TM, TN>(wm, wn, lane);
    // fragments of sub-step kk of the stage at sA
    auto frags = [&](const uint16_t* sA, int kk, bf16x8 (&a)[FM], bf16x8 (&b)[FN]) {
        if constexpr (BKS == 64)
            load_frags64<FM, FN>(sA, fadr, kk, a, b);
        else
            load_frags<FM, FN, TM, TN, BKS>(sA, sA + BM * BKS, wm, wn, lane, kk, a, b);
    };
    if (nsteps > 0) frags(smem, 0, fa[0], fb[0]);

    // The stage refilled after a step's barrier: part 0 right after the
    // barrier, parts 1..KK-1 at the starts of the next step's leading
    // sub-steps, all before that step's wait, so the wait count below still
    // holds (every stage up to t+STAGES-1 fully issued at step t's wait).
    bool pend = false;
    int pk = 0;
    uint16_t* pbuf = smem;
    auto leading_substeps = [&](const uint16_t* sA, bool parts) {
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
            const int cur = kk & 1;
            if (parts) issue_part(pk, pbuf, kk + 1);
            frags(sA, kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
            mfma_block<FM, FN>(fa[cur], fb[cur], acc);
            interleave_mfma<FM * FN, FM + FN, 0>();
        }
    };

    for (int t = 0; t + 1 < nsteps; ++t) {
        leading_substeps(smem + (t % STAGES) * STAGE, pend);
        wait_vmcnt<(STAGES >= 2 ? (STAGES - 2) * L : 0)>();   // stage t+1 landed for this wave
        lds_barrier();                    // ... and for every wave; stage t is free
        pend = true;
        pk = min(k_next, k_last);
        pbuf = smem + (t % STAGES) * STAGE;
        k_next += BKS;
        issue_part(pk, pbuf, 0);
        const uint16_t* nA = smem + ((t + 1) % STAGES) * STAGE;
        frags(nA, 0, fa[LAST ^ 1], fb[LAST ^ 1]);
        mfma_block<FM, FN>(fa[LAST], fb[LAST], acc);
        interleave_mfma<FM * FN, FM + FN, 0>();
    }
    if (nsteps > 0) {
        // the stage pending here lies past the end (never read): its other
        // parts are not issued
        leading_substeps(smem + ((nsteps - 1) % STAGES) * STAGE, false);
        mfma_block<FM, FN>(fa[LAST], fb[LAST], acc);
    }
    wait_vmcnt<0>();   // drain the re-loads past the end before LDS is reused or the wave exits
}

template <int BM, int BN, int BKS, int WM, int WN, int STAGES, int EPI, bool PREF = false>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_mfma_direct_kernel(KParams p) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    static_assert(FM * 32 * WM == BM && FN * 32 * WN == BN, "bad tile split");
    static_assert(STAGES >= 1, "at least one LDS stage");
    constexpr int STAGE = (BM + BN) * BKS;

    // the prefetching fold stages its whole BF16 tile in one epilogue pass
    constexpr int SMEM_ELEMS = (PREF && BM * BN > STAGES * STAGE) ? BM * BN : STAGES * STAGE;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    int tm, tn;
    if constexpr (PREF) {
        // The fold streams `out` once: in dispatch order, adjacent tiles run
        // on different XCDs at the same time (7% faster on 2048 x 17408 than
        // the XCD-contiguous order, which serves L2 reuse of the operands).
        tile_of<ORDER_FOLD>((int)blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    } else {
        tile_of_block(p.tiles_m, p.tiles_n, tm, tn);
    }
    // the second problem of a dual launch: same A and shape, its own B and C
    // (uniform per workgroup)
    const uint16_t* Bop = p.B;
    void* Cop = p.C;
    if (p.dual_tiles_n > 0 && tn >= p.dual_tiles_n) {
        tn -= p.dual_tiles_n;
        Bop = p.B1;
        Cop = p.C1;
    }
    const int m0 = tm * BM, n0 = tn * BN;

    const int split = blockIdx.y;
    const int kb = (int)min((int64_t)p.K, (int64_t)split * p.k_chunk);
    const int ke = (int)min((int64_t)p.K, (int64_t)kb + p.k_chunk);

    f32x16 acc[FM][FN];
    zero_acc(acc);

    // Fused fold with a short K: the workgroup's `out` tile is fetched while
    // the operand loads are in flight, in the same 16-byte pieces the
    // epilogue's row-streaming assigns to this thread, so its HBM latency
    // overlaps the operand loads and MFMAs.
    constexpr int PCPR = BN * 2 / 16;
    constexpr int NPRE = PREF ? BM * PCPR / NT : 0;
    static_assert(!PREF || EPI == EPI_SCALED_ACC, "prefetch is for the fold epilogue");
    // every thread has a piece in every prefetch round, so on an interior
    // tile each wave issues exactly NPRE loads
    static_assert(!PREF || NPRE * NT == BM * PCPR, "prefetch rounds cover the tile exactly");
    u32x4 pre[NPRE > 0 ? NPRE : 1];
    direct_mainloop<BM, BN, BKS, WM, WN, STAGES, NPRE>(
        p, Bop, smem, m0, n0, kb, ke, wave, lane, tid, acc, [&]() {
            if constexpr (PREF) {
                const uint16_t* O = reinterpret_cast<const uint16_t*>(Cop);
                const bool vec_ok = (p.N & 7) == 0 && (p.ldc & 7) == 0;
#pragma unroll
                for (int it = 0; it < NPRE; ++it) {
                    const int piece = tid + it * NT;
                    const int row = piece / PCPR, chunk = piece % PCPR;
                    const int m = m0 + row, n = n0 + chunk * 8;
                    if (m < p.M && vec_ok && n + 8 <= p.N)
                        pre[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(O + (int64_t)m * p.ldc + n));
                }
                // edge tiles skip some prefetch loads: uniform per workgroup
                return vec_ok && m0 + BM <= p.M && n0 + BN <= p.N;
            }
            return true;
        });

    staged_epilogue<EPI, BM, BN, WM, WN, FM, FN, NT, SMEM_ELEMS * 2, NPRE>(
        p, acc, reinterpret_cast<uint8_t*>(smem), m0, n0, wm, wn, lane, tid, split, pre, Cop);
}

// ---------------------------------------------------------------------------
// Stream-K: K steps dealt out evenly over one workgroup per CU slot instead
// of whole tiles (streamk_plan.hpp has the plan). Each piece of a workgroup's
// range runs the direct main loop over its K steps. An unfinished tile's
// piece is written to the workgroup's FP32 partial slot and published with
// the call's epoch in its flag; the workgroup that runs a tile's last step
// adds the partials of the lower workgroups that ran its earlier steps
// (fixed order, so repeated calls give identical bits) and stores BF16.
// ---------------------------------------------------------------------------

struct SkArgs {
    float* ws;            // partial slots: one BM x BN FP32 tile per workgroup
    uint64_t* flags;      // one per workgroup: the epoch of its last published partial
    uint64_t epoch;       // unique per call
    int steps;            // K steps per tile
    int wgs_per_xcd;      // workgroups per XCD (the grid is 8 times this)
    int tiles;
};

// polls of a flag before a wait gives up (about a second): the output of a
// tile whose partials never arrive is NaN instead of a hang
constexpr int kSkSpinLimit = 1 << 20;

// Owner epilogue of a tile whose earlier K steps other workgroups ran: the
// FP32 accumulator tile is staged in LDS (in passes of whole rows when it
// does not fit), and the threads streaming each row add the sources'
// row-major FP32 partials to it, nearest source first, then round to BF16
// and store. `src` is the nearest source's slot, the others lie
// `src_stride` floats apart below it.
template <int BM, int BN, int WM, int WN, int FM, int FN, int NT, int CAP>
__device__ __forceinline__ void sk_fixup_epilogue(const KParams& p, const f32x16 (&acc)[FM][FN], uint8_t* lds,
                                                  int m0, int n0, int wm, int wn, int lane, int tid,
                                                  const float* src, int64_t src_stride, int nsrc, bool late) {
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int ROWB = BN * 4;
    constexpr int CPR16 = ROWB / 16;   // four FP32 values per chunk
    constexpr int ROWS_FIT = CAP / ROWB;
    constexpr int RP = (ROWS_FIT >= BM) ? BM : (ROWS_FIT / 32) * 32;
    static_assert(RP >= 32, "a pass holds at least one 32-row MFMA block");
    constexpr int NPASS = (BM + RP - 1) / RP;
    const int M = p.M, N = p.N, ldc = p.ldc;
    uint16_t* C = reinterpret_cast<uint16_t*>(p.C);
    const bool vec_ok = (N % 4) == 0 && (ldc % 4) == 0;
    auto slot = [](int row, int chunk) { return row * ROWB + (((chunk + row) % CPR16) << 4); };

#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        lds_barrier();
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int blk = wm * TM + i * 32;
            if (blk < pass * RP || blk >= (pass + 1) * RP) continue;
            const int row = blk + (lane & 31) - pass * RP;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n_local = wn * TN + j * 32 + g * 8 + (lane >> 5) * 4;
                    *reinterpret_cast<f32x4*>(lds + slot(row, n_local >> 2)) =
                        f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                }
        }
        lds_barrier();
        // groups of GRP chunks per thread: the group's chunks, then one
        // uniform loop over the sources (no loop inside lane-dependent
        // control flow); a partial slot holds the whole tile, so its reads
        // need no bound
        const int lim = min(RP, BM - pass * RP) * CPR16;
        constexpr int ITER = (RP * CPR16 + NT - 1) / NT;
        constexpr int GRP = ITER < 4 ? ITER : 4;
        static_assert(ITER % GRP == 0, "whole groups");
        const float* srcp0 = src + (int64_t)pass * RP * BN;
#pragma unroll
        for (int g0 = 0; g0 < ITER; g0 += GRP) {
            f32x4 v[GRP];
#pragma unroll
            for (int g = 0; g < GRP; ++g) {
                const int qi = tid + (g0 + g) * NT;
                if (qi < lim) v[g] = *reinterpret_cast<const f32x4*>(lds + slot(qi / CPR16, qi % CPR16));
            }
            const float* srcp = srcp0;
            for (int k = 0; k < nsrc; ++k, srcp -= src_stride) {
#pragma unroll
                for (int g = 0; g < GRP; ++g) {
                    const int qi = tid + (g0 + g) * NT;
                    if (qi < lim) {
                        const f32x4 w =
                            *reinterpret_cast<const f32x4*>(srcp + (qi / CPR16) * BN + (qi % CPR16) * 4);
                        v[g][0] += w[0];
                        v[g][1] += w[1];
                        v[g][2] += w[2];
                        v[g][3] += w[3];
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < GRP; ++g) {
                const int qi = tid + (g0 + g) * NT;
                const int row = qi / CPR16, chunk = qi % CPR16;
                const int m = m0 + pass * RP + row;
                const int n = n0 + chunk * 4;
                if (qi >= lim || m >= M || n >= N) continue;
                const f32x4 r = late ? f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                             __builtin_nanf("")}
                                     : v[g];
                const int64_t off = (int64_t)m * ldc + n;
                const uint32_t lo = pack_bf16x2(r[0], r[1]), hi = pack_bf16x2(r[2], r[3]);
                if (vec_ok && n + 4 <= N) {
                    *reinterpret_cast<u32x2*>(C + off) = u32x2{lo, hi};
                } else {
                    const uint32_t e2[2] = {lo, hi};
                    for (int e = 0; e < 4 && n + e < N; ++e) C[off + e] = (uint16_t)(e2[e >> 1] >> ((e & 1) * 16));
                }
            }
        }
    }
}

template <int BM, int BN, int BKS, int WM, int WN, int STAGES>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_streamk_kernel(KParams p, SkArgs q) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    static_assert(FM * 32 * WM == BM && FN * 32 * WN == BN, "bad tile split");
    constexpr int STAGE = (BM + BN) * BKS;
    constexpr int SMEM_ELEMS = STAGES * STAGE;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM_ELEMS];
    __shared__ int s_late;

    const int tid0 = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int b = blockIdx.x;
    const int x = b % SK_XCDS, u = b / SK_XCDS;

    SkWorkgroup wg;
    wg.init(q.tiles, q.steps, q.wgs_per_xcd, x, u);
    const int pieces = wg.count();
    // a partial slot is one BM x BN FP32 tile, row-major
    KParams ps = p;
    ps.M = BM;
    ps.N = BN;
    ps.ldc = BN;

    for (int pi = 0; pi < pieces; ++pi) {
        // the thread index plus an opaque (uniform) zero: otherwise the
        // compiler hoists every lane-dependent LDS and global offset of the
        // main loop and the epilogues out of the piece loop and keeps them
        // all live at once (up to 256 VGPRs with scratch spills)
        int opaque_zero = 0;
        asm volatile("" : "+s"(opaque_zero));
        const int tid = tid0 + opaque_zero;
        const int lane = tid & 63;
        const SkPiece pc = wg.piece(pi);
        int tm, tn;
        grouped_tile(wg.t0 + pc.tile, p.tiles_m, p.tiles_n, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const int kb = sk_kpos(pc.s_begin, p.K, q.steps), ke = sk_kpos(pc.s_end, p.K, q.steps);

        f32x16 acc[FM][FN];
        zero_acc(acc);
        if (pi > 0) lds_barrier();   // the previous piece's epilogue is done with LDS
        direct_mainloop<BM, BN, BKS, WM, WN, STAGES, 0>(p, p.B, smem, m0, n0, kb, ke, wave, lane, tid, acc,
                                                        []() { return true; });

        if (pc.partial) {
            staged_epilogue<EPI_STORE_F32, BM, BN, WM, WN, FM, FN, NT, SMEM_ELEMS * 2>(
                ps, acc, reinterpret_cast<uint8_t*>(smem), 0, 0, wm, wn, lane, tid, 0, nullptr,
                q.ws + (int64_t)b * (BM * BN));
            // Each wave waits until its stores are performed; after the
            // barrier one device-scope release (one L2 writeback for the
            // workgroup instead of one per wave: 60 -> 35 us on 5120 x 512 x
            // 2048) publishes the whole tile with the flag.
            wait_vmcnt<0>();
            __syncthreads();
            if (tid == 0) __hip_atomic_store(q.flags + b, q.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else if (pc.src_first >= 0) {
            if (wave == 0) {
                // the whole wave polls (one request per poll) and takes the
                // loaded value from lane 0, so the loop is uniform
                int late = 0;
                for (int su = pc.src_first; su < u; ++su) {
                    const uint64_t* f = q.flags + su * SK_XCDS + x;
                    for (int polls = 0;; ++polls) {
                        const uint64_t v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
                        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
                        if ((((uint64_t)hi << 32) | lo) == q.epoch) break;
                        if (polls >= kSkSpinLimit) {
                            late = 1;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                }
                s_late = late;
                // one device-scope acquire for the workgroup (the CU's L1 and
                // the XCD's L2 are shared by its waves), ordered before the
                // other waves' reads by the barrier
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            __syncthreads();
            const int late = s_late;
            sk_fixup_epilogue<BM, BN, WM, WN, FM, FN, NT, SMEM_ELEMS * 2>(
                p, acc, reinterpret_cast<uint8_t*>(smem), m0, n0, wm, wn, lane, tid,
                q.ws + (int64_t)((u - 1) * SK_XCDS + x) * (BM * BN), (int64_t)SK_XCDS * BM * BN,
                u - pc.src_first, late != 0);
        } else {
            staged_epilogue<EPI_STORE_BF16, BM, BN, WM, WN, FM, FN, NT, SMEM_ELEMS * 2>(
                p, acc, reinterpret_cast<uint8_t*>(smem), m0, n0, wm, wn, lane, tid, 0, nullptr, p.C);
        }
    }
}

// ---------------------------------------------------------------------------
// Sliced K: two groups of WM x WN waves share one BM x BN tile, group g
// walking the g-th half of K through its own ring of LDS stages, so each SIMD
// holds one wave of each group and the two overlap each other's waits (a
// problem with no more tiles than CUs runs one workgroup per CU, and a single
// wave per SIMD leaves the matrix core idle during its barriers and loads).
// Both halves have the same number of steps, so every wave passes the same
// barriers. The second group's FP32 sums are then added to the first's
// through LDS (always first half + second half) and the workgroup stores the
// tile. K must be a multiple of 128.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int STAGES, int BKS = BK>
__global__ void __launch_bounds__(2 * WM * WN * 64)
gemm_slicedk_kernel(KParams p) {
    constexpr int NTG = WM * WN * 64;   // threads per group
    constexpr int NT = 2 * NTG;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    static_assert(FM * 32 * WM == BM && FN * 32 * WN == BN, "bad tile split");
    constexpr int STAGE = (BM + BN) * BKS;
    constexpr int SMEM_ELEMS = 2 * STAGES * STAGE;
    // the exchange moves PB accumulator blocks (of every wave of the group)
    // per pass through the stages
    constexpr int NB = FM * FN;
    constexpr int PB = (SMEM_ELEMS * 2) / (NTG * 16 * 4) < NB ? (SMEM_ELEMS * 2) / (NTG * 16 * 4) : NB;
    static_assert(PB >= 1, "one accumulator block of the group fits the stages");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave / (WM * WN);                  // K half of this wave
    const int gw = wave % (WM * WN), gtid = tid % NTG;
    const int wm = gw / WN, wn = gw % WN;

    int tm, tn;
    tile_of_block(p.tiles_m, p.tiles_n, tm, tn);
    // the second problem of a dual launch (uniform per workgroup)
    const uint16_t* Bop = p.B;
    void* Cop = p.C;
    if (p.dual_tiles_n > 0 && tn >= p.dual_tiles_n) {
        tn -= p.dual_tiles_n;
        Bop = p.B1;
        Cop = p.C1;
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int half = p.K / 2;

    f32x16 acc[FM][FN];
    zero_acc(acc);
    direct_mainloop<BM, BN, BKS, WM, WN, STAGES, 0>(p, Bop, smem + g * STAGES * STAGE, m0, n0, g * half,
                                                    (g + 1) * half, gw, lane, gtid, acc, []() { return true; });

    // second half -> LDS in each lane's accumulator order, first half adds it
    float* xs = reinterpret_cast<float*>(smem);
    static_for<(NB + PB - 1) / PB>([&](auto pc) {
        constexpr int b0 = decltype(pc)::value * PB;
        lds_barrier();
        if (g == 1) {
            static_for<(NB - b0 < PB ? NB - b0 : PB)>([&](auto qc) {
                constexpr int q = b0 + decltype(qc)::value, i = q / FN, j = q % FN;
                float* dst = xs + ((int64_t)(q - b0) * (WM * WN) + gw) * (16 * 64);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<f32x4*>(dst + c * 256 + lane * 4) =
                        f32x4{acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2], acc[i][j][4 * c + 3]};
            });
        }
        lds_barrier();
        if (g == 0) {
            static_for<(NB - b0 < PB ? NB - b0 : PB)>([&](auto qc) {
                constexpr int q = b0 + decltype(qc)::value, i = q / FN, j = q % FN;
                const float* src = xs + ((int64_t)(q - b0) * (WM * WN) + gw) * (16 * 64);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(src + c * 256 + lane * 4);
                    acc[i][j][4 * c] += v[0];
                    acc[i][j][4 * c + 1] += v[1];
                    acc[i][j][4 * c + 2] += v[2];
                    acc[i][j][4 * c + 3] += v[3];
                }
            });
        }
    });
    staged_epilogue<EPI_STORE_BF16, BM, BN, WM, WN, FM, FN, NT, SMEM_ELEMS * 2>(
        p, acc, reinterpret_cast<uint8_t*>(smem), m0, n0, wm, wn, lane, tid, 0, nullptr, Cop, g == 0);
}

template <int BM, int BN, int WM, int WN, int STAGES, int BKS = BK>
hipError_t launch_slicedk(const KParams& kp, hipStream_t stream) {
    KParams q = kp;
    q.tiles_m = (kp.M + BM - 1) / BM;
    q.tiles_n = (kp.N + BN - 1) / BN;
    q.dual_tiles_n = 0;
    if (kp.dual) {   // dual launch: the second product's tiles follow the first's
        q.dual_tiles_n = q.tiles_n;
        q.tiles_n *= 2;
    }
    hipLaunchKernelGGL((gemm_slicedk_kernel<BM, BN, WM, WN, STAGES, BKS>), dim3((unsigned)(q.tiles_m * q.tiles_n)),
                       dim3(2 * WM * WN * 64), 0, stream, q);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int EPI, int SRC, int RSETS = 2>
hipError_t launch_cfg(const KParams& kp, int splits, hipStream_t stream, int batch = 1) {
    KParams q = kp;
    q.tiles_m = (kp.M + BM - 1) / BM;
    q.tiles_n = (kp.N + BN - 1) / BN;
    dim3 grid((unsigned)(q.tiles_m * q.tiles_n), (unsigned)splits, (unsigned)batch);
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN, EPI, SRC, RSETS>), grid, dim3(WM * WN * 64), 0,
                       stream, q);
    return hipGetLastError();
}

template <int BM, int BN, int BKS, int WM, int WN, int STAGES, int EPI, bool PREF = false>
hipError_t launch_direct(const KParams& kp, int splits, hipStream_t stream) {
    // A single LDS stage only works when the whole K chunk is one step.
    if constexpr (STAGES == 1) {
        if (kp.k_chunk > BKS) return launch_direct<BM, BN, BKS, WM, WN, 2, EPI, PREF>(kp, splits, stream);
    }
    KParams q = kp;
    q.tiles_m = (kp.M + BM - 1) / BM;
    q.tiles_n = (kp.N + BN - 1) / BN;
    q.dual_tiles_n = 0;
    if (kp.dual) {   // dual launch: the second product's tiles follow the first's
        q.dual_tiles_n = q.tiles_n;
        q.tiles_n *= 2;
    }
    dim3 grid((unsigned)(q.tiles_m * q.tiles_n), (unsigned)splits, 1);
    hipLaunchKernelGGL((gemm_mfma_direct_kernel<BM, BN, BKS, WM, WN, STAGES, EPI, PREF>), grid,
                       dim3(WM * WN * 64), 0, stream, q);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_tile_cfg(const KParams& kp, int splits, int cfg, hipStream_t stream) {
    switch (cfg) {
        //                                  BM   BN  BK WM WN ST
        case 0: return launch_cfg<128, 128, 2, 2, EPI, SRC_BF16_VEC>(kp, splits, stream);
        case 1: return launch_direct<256, 256, 64, 2, 2, 2, EPI>(kp, splits, stream);
        case 2: return launch_direct<256, 256, 64, 2, 4, 2, EPI>(kp, splits, stream);
        case 3: return launch_direct<160, 256, 64, 1, 4, 3, EPI>(kp, splits, stream);
        case 4: return launch_direct<128, 64, 64, 2, 1, 2, EPI>(kp, splits, stream);
        case 5: return launch_direct<256, 224, 64, 4, 1, 2, EPI>(kp, splits, stream);
        case 6: return launch_direct<128, 128, 64, 2, 2, 2, EPI>(kp, splits, stream);
        case 7: return launch_direct<224, 256, 64, 1, 4, 2, EPI>(kp, splits, stream);
        case 8: return launch_direct<160, 256, 64, 1, 4, 2, EPI>(kp, splits, stream);
        case 9: return launch_direct<160, 128, 64, 1, 4, 2, EPI>(kp, splits, stream);
        case 11:
            if constexpr (EPI == EPI_SCALED_ACC)
                return launch_direct<160, 128, 64, 1, 4, 2, EPI, true>(kp, splits, stream);
            else
                return launch_direct<160, 128, 64, 1, 4, 2, EPI>(kp, splits, stream);
        case 12:
            if constexpr (EPI == EPI_SCALED_ACC)
                return launch_direct<128, 128, 64, 2, 2, 2, EPI, true>(kp, splits, stream);
            else
                return launch_direct<128, 128, 64, 2, 2, 2, EPI>(kp, splits, stream);
        case 13:
            if constexpr (EPI == EPI_SCALED_ACC)
                return launch_direct<160, 128, 64, 1, 4, 1, EPI, true>(kp, splits, stream);
            else
                return launch_direct<160, 128, 64, 1, 4, 1, EPI>(kp, splits, stream);
        case 14:
            if constexpr (EPI == EPI_SCALED_ACC)
                return launch_direct<128, 128, 64, 2, 2, 1, EPI, true>(kp, splits, stream);
            else
                return launch_direct<128, 128, 64, 2, 2, 1, EPI>(kp, splits, stream);
        case 18:
        case 19:
        case 20:
        case 21:
        case 22:
            // single-stage prefetching tiles for the fold (K of one step)
            if constexpr (EPI == EPI_SCALED_ACC) {
                if (cfg == 18) return launch_direct<64, 128, 64, 2, 2, 1, EPI, true>(kp, splits, stream);
                if (cfg == 19) return launch_direct<64, 256, 64, 1, 4, 1, EPI, true>(kp, splits, stream);
                if (cfg == 20) return launch_direct<32, 256, 64, 1, 4, 1, EPI, true>(kp, splits, stream);
                if (cfg == 21) return launch_direct<128, 256, 64, 2, 4, 1, EPI, true>(kp, splits, stream);
                return launch_direct<64, 128, 64, 1, 2, 1, EPI, true>(kp, splits, stream);
            } else {
                return launch_direct<160, 128, 64, 1, 4, 2, EPI>(kp, splits, stream);
            }
        case 15: return launch_direct<160, 256, 64, 1, 8, 2, EPI>(kp, splits, stream);
        case 16: return launch_direct<320, 128, 64, 2, 2, 2, EPI>(kp, splits, stream);
        case 17: return launch_direct<160, 128, 64, 1, 4, 3, EPI>(kp, splits, stream);
        case 23: return launch_direct<128, 128, 64, 2, 2, 3, EPI>(kp, splits, stream);
        case 24: return launch_direct<96, 128, 64, 1, 4, 3, EPI>(kp, splits, stream);
        case 27:
        case 28:
            // sliced K (two K halves per tile): BF16 stores (one problem or a
            // dual launch) with K % 128 == 0; anything else takes the 128 x 128
            // three-stage tile
            if constexpr (EPI == EPI_STORE_BF16) {
                if (splits == 1 && kp.k_chunk == kp.K && kp.K % 128 == 0) {
                    if (cfg == 27) return launch_slicedk<128, 128, 2, 2, 2>(kp, stream);
                    return launch_slicedk<64, 128, 2, 2, 3>(kp, stream);
                }
            }
            return launch_direct<128, 128, 64, 2, 2, 3, EPI>(kp, splits, stream);
        default: return launch_direct<256, 128, 64, 4, 2, 3, EPI>(kp, splits, stream);   // 10
    }
}

// Shape -> schedule. Time estimates in microseconds use the measured
// sustained rate of each configuration with every CU busy (TFLOP/s on
// MI355X, random BF16 operands); tiles run in rounds of (CUs x blocks per
// CU). Problems with a tiny K are bound by the output traffic.
//
// Column split: when the last round of 256x256 tiles would be poorly filled
// (860 tiles on 256 CUs: the fourth round a third full), the first n1 columns
// run as whole rounds of 256x256 tiles and the remaining columns as a second
// launch with the tile that finishes them fastest (usually one round of a
// half-size tile). Every output is still produced by one tile walking K in
// the same order, so the result is bit-identical to the unsplit launch.
// `rate` holds with occ blocks on every CU; `rate1` with one block per CU
// (problems of at most one tile per CU), lower for the two-block tiles,
// whose latency the second block hides.
struct TileChoice {
    int cfg, bm, bn, occ;
    double rate, rate1;
};
constexpr TileChoice kTileChoices[] = {
    {2, 256, 256, 1, 1096.0, 1096.0},
    // three stages (159744 bytes of LDS): 6-8% ahead of two stages on the
    // 5120x2048 outputs (down, Q/O) in interleaved same-GPU runs
    {3, 160, 256, 1, 1050.0, 1050.0},
    {10, 256, 128, 1, 900.0, 900.0},
    {9, 160, 128, 2, 884.0, 819.0},
    {6, 128, 128, 2, 808.0, 671.0},
    {23, 128, 128, 1, 763.0, 763.0},   // three stages
    // 96 x 128 with three stages (four waves of 96 x 32): 5120 x 512 x 2048 is
    // one round of 216 tiles instead of 160, 15.6 us against 16.6 us
    {24, 96, 128, 1, 608.0, 608.0},
    // 160 x 128 with three stages (one block per CU): 5120 x 1024 x 2048 is one
    // round of 256 tiles, 23.9 us against 28.7 us for the two-block 160 x 128
    {17, 160, 128, 1, 880.0, 900.0},
    // sliced K, 64 x 128 (two K halves per tile, rates counted on the whole
    // K): deep-K problems with few tiles, e.g. 1024 x 1024 x 8192 33.5 us
    // against 50.0 us for the 128 x 128 tile. BF16 store of one problem
    // with K % 128 == 0 only (kSlicedCfg).
    {28, 64, 128, 1, 700.0, 950.0},
};
constexpr int kSlicedCfg = 28;
constexpr double kLaunchGapUs = 2.0;   // second launch of a column split

struct Schedule {
    int cfg;       // configuration of columns [0, n1)
    int n1;        // == N: no split
    int cfg2;      // configuration of columns [n1, N)
};

double dp_us(const TileChoice& c, int M, int N, int K, int splits, int cus) {
    const double tiles = (double)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn) * splits;
    const double slots = (double)cus * c.occ;
    const double rounds = tiles <= cus ? 1.0 : (double)(int64_t)((tiles + slots - 1) / slots);
    const double occ = tiles <= cus ? 1.0 : c.occ;
    const double rate = tiles <= cus ? c.rate1 : c.rate;
    return rounds * occ * 2.0 * c.bm * c.bn * ((double)K / splits) * cus / (rate * 1e6);
}

const TileChoice* best_single(int M, int N, int K, int splits, int cus, double* t_out, bool sliced_ok = false) {
    const TileChoice* best = &kTileChoices[0];
    double best_t = 1e300;
    for (const TileChoice& c : kTileChoices) {
        if (c.cfg == kSlicedCfg && !sliced_ok) continue;
        const double t = dp_us(c, M, N, K, splits, cus);
        if (t < best_t) {
            best_t = t;
            best = &c;
        }
    }
    *t_out = best_t;
    return best;
}

Schedule choose_schedule(int M, int N, int K, int splits, int cus, int epi) {
    if (K <= 128) {
        // Output-bound: the fold streams `out` best with small single-stage
        // prefetching tiles (64x128: up to six workgroups per CU), a plain
        // short-K product with the narrow 160x128 tile.
        const int cfg = epi == EPI_SCALED_ACC ? 18 : 9;
        return {cfg, N, cfg};
    }
    double best_t;
    const bool sliced_ok = epi == EPI_STORE_BF16 && splits == 1 && K % 128 == 0;
    const TileChoice* one = best_single(M, N, K, splits, cus, &best_t, sliced_ok);
    Schedule best{one->cfg, N, one->cfg};
    if (epi != EPI_STORE_BF16 || splits != 1) return best;
    const TileChoice& big = kTileChoices[0];
    for (int c1 = 1; c1 * big.bn < N; ++c1) {
        const int n1 = c1 * big.bn;
        double t2;
        const TileChoice* rest = best_single(M, N - n1, K, 1, cus, &t2);
        const double t = dp_us(big, M, n1, K, 1, cus) + t2 + kLaunchGapUs;
        if (t < best_t) {
            best_t = t;
            best = {big.cfg, n1, rest->cfg};
        }
    }
    return best;
}

template <int EPI>
hipError_t launch_dense_vec(const KParams& kp, int splits, hipStream_t stream) {
    const int forced = tune(BG_TUNE_TILE);
    if (forced >= 0) return launch_tile_cfg<EPI>(kp, splits, forced, stream);
    Schedule sch = choose_schedule(kp.M, kp.N, kp.K, splits, kp.cus, EPI);
    if (tune(BG_TUNE_COLSPLIT) == 0 && sch.n1 < kp.N) {
        double t;
        sch = {best_single(kp.M, kp.N, kp.K, splits, kp.cus, &t)->cfg, kp.N, 0};
    }
    if (sch.n1 >= kp.N) return launch_tile_cfg<EPI>(kp, splits, sch.cfg, stream);
    // columns [0, n1), then [n1, N) of the same C (row stride ldc)
    KParams left = kp;
    left.N = sch.n1;
    hipError_t e = launch_tile_cfg<EPI>(left, splits, sch.cfg, stream);
    if (e != hipSuccess) return e;
    KParams right = kp;
    right.B = kp.B + (int64_t)sch.n1 * kp.ldb;
    right.C = reinterpret_cast<uint16_t*>(kp.C) + sch.n1;
    right.N = kp.N - sch.n1;
    return launch_tile_cfg<EPI>(right, splits, sch.cfg2, stream);
}

template <int BM, int BN, int BKS, int WM, int WN, int STAGES>
hipError_t launch_sk(const KParams& kp, SkArgs q, hipStream_t stream) {
    KParams p = kp;
    p.tiles_m = (kp.M + BM - 1) / BM;
    p.tiles_n = (kp.N + BN - 1) / BN;
    p.dual_tiles_n = 0;
    q.tiles = p.tiles_m * p.tiles_n;
    q.steps = (kp.K + 63) / 64;
    const int grid = SK_XCDS * q.wgs_per_xcd;
    q.flags = reinterpret_cast<uint64_t*>(q.ws + (int64_t)grid * BM * BN);
    hipLaunchKernelGGL((gemm_streamk_kernel<BM, BN, BKS, WM, WN, STAGES>), dim3((unsigned)grid),
                       dim3(WM * WN * 64), 0, stream, p, q);
    return hipGetLastError();
}

template <int EPI, int SRC>
hipError_t launch_dense_src(const KParams& kp, int splits, hipStream_t stream) {
    if constexpr (SRC == SRC_BF16_VEC) return launch_dense_vec<EPI>(kp, splits, stream);
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
    kp.lda = (int)p.lda;
    kp.ldb = (int)p.ldb;
    kp.ldc = (int)p.ldc;
    kp.k_chunk = (int)p.k_chunk;
    kp.scale = p.scale;
    kp.cus = p.cus > 0 ? (int)p.cus : 256;
    // whole 16-byte chunks on 16-byte-aligned rows (the base pointers are),
    // and row pitches whose largest tile (320 rows) spans less than 2 GB, the
    // range of the direct kernels' 32-bit buffer offsets
    const bool vec = (p.K % 8) == 0 && (p.lda % 8) == 0 && (p.ldb % 8) == 0 &&
                     (int64_t)p.lda * 640 < (int64_t(1) << 31) && (int64_t)p.ldb * 640 < (int64_t(1) << 31);
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
        case EPI_SCALE_BF16:   // W4A16 only (launch_w4a16)
            break;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_streamk(const DenseProblem& p, void* ws, int cfg, uint64_t epoch, hipStream_t stream) {
    KParams kp{};
    kp.A = p.A;
    kp.B = p.B;
    kp.C = p.C;
    kp.M = (int)p.M;
    kp.N = (int)p.N;
    kp.K = (int)p.K;
    kp.lda = kp.ldb = (int)p.K;
    kp.ldc = (int)p.N;
    kp.k_chunk = (int)p.K;
    kp.cus = p.cus > 0 ? (int)p.cus : 256;
    SkArgs q{};
    q.ws = static_cast<float*>(ws);
    q.epoch = epoch;
    q.wgs_per_xcd = sk_wgs_per_xcd((uint32_t)kp.cus);
    //                                       BM   BN  BK WM WN ST
    if (cfg == 10) return launch_sk<256, 128, 64, 4, 2, 3>(kp, q, stream);
    return launch_sk<128, 128, 64, 2, 2, 3>(kp, q, stream);   // 23
}

// Two products of one A: the second problem's column tiles follow the first's
// in one grid, so the two share the rounds of one launch instead of each
// leaving its own last round partly empty (5120 x 11008 x 2048 twice: 1720
// tiles of 256 x 256, 6.7 rounds, against 2 x 3.4). The tile is the one the
// cost model picks for the combined problem (M, 2N, K); no column split.
// Operands outside the direct kernels' reach (K % 8 != 0, or a forced
// register-staged tile) run as two ordinary launches.
hipError_t launch_dense_dual(const DenseProblem& p, const uint16_t* B1, uint16_t* C1, hipStream_t stream) {
    const bool vec = (p.K % 8) == 0 && (int64_t)p.K * 640 < (int64_t(1) << 31);
    const int forced = tune(BG_TUNE_TILE);
    if (!vec || forced == 0) {
        hipError_t e = launch_dense(p, EPI_STORE_BF16, stream);
        if (e != hipSuccess) return e;
        DenseProblem p1 = p;
        p1.B = B1;
        p1.C = C1;
        return launch_dense(p1, EPI_STORE_BF16, stream);
    }
    KParams kp{};
    kp.A = p.A;
    kp.B = p.B;
    kp.C = p.C;
    kp.B1 = B1;
    kp.C1 = C1;
    kp.dual = 1;
    kp.M = (int)p.M;
    kp.N = (int)p.N;
    kp.K = (int)p.K;
    kp.lda = kp.ldb = (int)p.K;
    kp.ldc = (int)p.N;
    kp.k_chunk = (int)p.K;
    kp.cus = p.cus > 0 ? (int)p.cus : 256;
    int cfg = forced;
    if (cfg < 0) {
        if (p.K <= 128) {
            cfg = 9;
        } else if (choose_schedule(kp.M, kp.N, kp.K, 1, kp.cus, EPI_STORE_BF16).cfg == kSlicedCfg) {
            // gemm_bf16 sums these outputs in two K halves; so must the dual
            // launch, whose outputs equal gemm_bf16's bit for bit
            cfg = kSlicedCfg;
        } else {
            double t;
            cfg = best_single(kp.M, 2 * kp.N, kp.K, 1, kp.cus, &t)->cfg;
        }
    }
    return launch_tile_cfg<EPI_STORE_BF16>(kp, 1, cfg, stream);
}

// W4A16 tile choices (register-staged kernel; the BG_TUNE_W4A16_TILE override
// forces one). The estimate is rounds x blocks per CU x tile area /
// measured rate, as for the BF16 tiles.
struct W4a16Choice {
    int cfg, bm, bn, occ;
    double rate;
};
constexpr W4a16Choice kW4a16Choices[] = {
    {0, 256, 256, 1, 985.0},
    {6, 128, 384, 1, 810.0},   // 1016 x 12288: 256 tiles, exactly one round
    {1, 128, 256, 1, 850.0},
    {2, 128, 128, 2, 800.0},
};

int choose_w4a16(int M, int N, int cus) {
    int best = 0;
    double best_t = 1e300;
    for (const W4a16Choice& c : kW4a16Choices) {
        const double tiles = (double)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
        const double slots = (double)cus * c.occ;
        const double rounds = tiles <= cus ? 1.0 : (double)(int64_t)((tiles + slots - 1) / slots);
        const double occ = tiles <= cus ? 1.0 : c.occ;
        const double t = rounds * occ * c.bm * c.bn / c.rate;
        if (t < best_t) {
            best_t = t;
            best = c.cfg;
        }
    }
    return best;
}

// FP4 tile choices (the BG_TUNE_FP4_TILE and BG_TUNE_FP4_SPLITK_TILE
// overrides force one when `tuned`).
template <int EPI, int WM = 1, int BN = 256>
hipError_t launch_fp4_dec(const KParams& kp, int splits, hipStream_t stream) {
    KParams q = kp;
    q.tiles_m = (kp.M + 127) / 128;
    q.tiles_n = (kp.N + BN - 1) / BN;
    dim3 grid((unsigned)(q.tiles_m * q.tiles_n), (unsigned)splits, 1u);
    hipLaunchKernelGGL((gemm_fp4_dec_kernel<EPI, WM, BN>), grid, dim3(256 * WM), 0, stream, q);
    return hipGetLastError();
}

template <int SRC>
hipError_t launch_fp4_src(const KParams& kp, int M, int splits, int batch, bool tuned, hipStream_t stream) {
    // the decode kernel: one problem, K and the split chunk whole 64-wide steps
    // (buffer records: each operand's packed bytes below 2^31)
    const bool dec_ok = SRC == SRC_FP4W && batch == 1 && kp.K % 64 == 0 && kp.k_chunk % 64 == 0 &&
                        (int64_t)kp.M * (kp.K / 2) < (int64_t(1) << 31) &&
                        (int64_t)kp.N * (kp.K / 2) < (int64_t(1) << 31);
    // FP32 planes (split-K) for the small-M decode shapes
    if (splits > 1) {
        int sk = tuned ? tune(BG_TUNE_FP4_SPLITK_TILE) : -1;
        // the decode kernel with eight waves for M <= 128 (measured on MI355X,
        // interleaved, against the register-staged 128 x 256 tile: 128 x 7168 x
        // 16384 at k_splits 8 43.8 against 49.5 us, 128 x 4096 x 7168 at 12
        // 25.6 against 26.7 us; ahead at every k_splits from 4 to 16), with
        // 128-column tiles when twice as many tiles still fit one round: 128 x
        // 4096 x 7168 20.7-21.3 us at k_splits 6-8 against 22.8-22.9 us for the
        // best 256-column split (12-14), 128 x 7168 x 16384 a tie (44.5 at 4
        // against 44.0 us at 8)
        if (sk < 0) {
            const int64_t t128 = (int64_t)((M + 127) / 128) * ((kp.N + 127) / 128) * splits;
            sk = dec_ok && M <= 128 ? (t128 <= kp.cus ? 9 : 8) : M <= 192 ? 3 : 2;
        }
        if (dec_ok && sk == 7) return launch_fp4_dec<EPI_STORE_F32>(kp, splits, stream);
        if (dec_ok && sk == 8) return launch_fp4_dec<EPI_STORE_F32, 2>(kp, splits, stream);
        if (dec_ok && sk == 9) return launch_fp4_dec<EPI_STORE_F32, 2, 128>(kp, splits, stream);
        if constexpr (SRC == SRC_FP4W) {
            switch (sk) {
                case 0: return launch_cfg<128, 128, 2, 2, EPI_STORE_F32, SRC, 2>(kp, splits, stream);
                case 1: return launch_cfg<128, 256, 2, 4, EPI_STORE_F32, SRC, 1>(kp, splits, stream);
                case 4: return launch_cfg<128, 256, 2, 4, EPI_STORE_F32, SRC, 3>(kp, splits, stream);
                case 5: return launch_cfg<128, 256, 2, 4, EPI_STORE_F32, SRC, 4>(kp, splits, stream);
                case 6: return launch_cfg<128, 128, 2, 2, EPI_STORE_F32, SRC, 4>(kp, splits, stream);
                default: break;
            }
        }
        if (sk == 3) return launch_cfg<128, 256, 2, 4, EPI_STORE_F32, SRC, 2>(kp, splits, stream);
        return launch_cfg<256, 256, 2, 4, EPI_STORE_F32, SRC, 1>(kp, splits, stream);
    }
    int cfg = tuned ? tune(BG_TUNE_FP4_TILE) : -1;
    // 256 x 256 tiles with two register sets where the 32-element units
    // leave room for them (3% ahead of one set on 4096 x 4096 x 8192)
    if (cfg < 0) cfg = M <= 192 ? 2 : SRC == SRC_FP4W ? 1 : 0;
    if (dec_ok && cfg == 10) return launch_fp4_dec<EPI_STORE_BF16>(kp, 1, stream);
    if (dec_ok && cfg == 11) return launch_fp4_dec<EPI_STORE_BF16, 2>(kp, 1, stream);
    if constexpr (SRC == SRC_FP4W) {
        switch (cfg) {
            case 1: return launch_cfg<256, 256, 2, 4, EPI_STORE_BF16, SRC, 2>(kp, 1, stream, batch);
            case 3: return launch_cfg<256, 256, 2, 2, EPI_STORE_BF16, SRC, 1>(kp, 1, stream, batch);
            case 5: return launch_cfg<128, 256, 2, 4, EPI_STORE_BF16, SRC, 2>(kp, 1, stream, batch);
            case 6: return launch_cfg<256, 128, 4, 2, EPI_STORE_BF16, SRC, 2>(kp, 1, stream, batch);
            case 7: return launch_cfg<128, 256, 2, 4, EPI_STORE_BF16, SRC, 3>(kp, 1, stream, batch);
            case 8: return launch_cfg<256, 128, 4, 2, EPI_STORE_BF16, SRC, 3>(kp, 1, stream, batch);
            case 9: return launch_cfg<128, 256, 2, 4, EPI_STORE_BF16, SRC, 4>(kp, 1, stream, batch);
            default: break;
        }
    }
    if (cfg == 2) return launch_cfg<128, 128, 2, 2, EPI_STORE_BF16, SRC, 2>(kp, 1, stream, batch);
    return launch_cfg<256, 256, 2, 4, EPI_STORE_BF16, SRC, 1>(kp, 1, stream, batch);
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
    kp.lda = kp.ldb = (int)p.K;
    kp.ldc = (int)p.N;
    kp.k_chunk = (int)p.k_chunk;
    kp.cus = p.cus > 0 ? (int)p.cus : 256;
    const int splits = (int)p.splits, batch = (int)p.batch;
    if (batch > 1) {
        kp.bs_a = (int64_t)p.M * (p.K / 2);
        kp.bs_sa = (int64_t)p.M * (p.K / 16);
        kp.bs_b = (int64_t)p.N * (p.K / 2);
        kp.bs_sb = (int64_t)p.N * (p.K / 16);
        kp.bs_c = (int64_t)p.M * p.N;
    }
    // 32-element staging units when no unit can straddle the end of K; the
    // 16-element units (K % 32 == 16) take the default tiles only
    if (p.K % 32 == 0) return launch_fp4_src<SRC_FP4W>(kp, (int)p.M, splits, batch, true, stream);
    return launch_fp4_src<SRC_FP4>(kp, (int)p.M, splits, batch, false, stream);
}

// Blocked (NVIDIA hardware) scale layout -> plain [L, rows, k_groups]: the
// stored order is (l, tile_m, tile_k, g_m[32], i_m[4], i_k[4]); thread q
// moves the 4 bytes of one (l, tile_m, tile_k, g_m, i_m) to plain row
// tile_m*128 + i_m*32 + g_m, groups tile_k*4 .. tile_k*4 + 3.
__global__ void __launch_bounds__(256)
scales_from_blocked_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, int rows,
                           int k_groups, int64_t words) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= words) return;
    const int tk = k_groups / 4, tm = rows / 128;
    const int i_m = (int)(q & 3);
    const int g_m = (int)((q >> 2) & 31);
    int64_t r = q >> 7;                      // (l, tile_m, tile_k)
    const int tile_k = (int)(r % tk);
    r /= tk;
    const int tile_m = (int)(r % tm);
    const int64_t l = r / tm;
    const int row = tile_m * 128 + i_m * 32 + g_m;
    dst[(l * rows + row) * tk + tile_k] = src[q];
}

hipError_t launch_scales_from_blocked(const uint8_t* src, uint8_t* dst, uint32_t rows, uint32_t k_groups,
                                      uint32_t batch, hipStream_t stream) {
    const int64_t words = (int64_t)batch * rows * (k_groups / 4);
    const int64_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(scales_from_blocked_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(dst), (int)rows,
                       (int)k_groups, words);
    return hipGetLastError();
}

// Transposed-weight W4A16 (weights [K/2, ldb] bytes, scales [K/16, ldb]):
// three tiles, chosen by the W4A16 cost model; 4-byte column loads when ldb
// is a multiple of 4, byte loads otherwise.
template <int S>
hipError_t launch_w4a16_t(const KParams& kp, int cus, hipStream_t stream) {
    int cfg = tune(BG_TUNE_W4A16_TILE);
    if (cfg < 0) {
        double best_t = 1e300;
        for (const W4a16Choice& c : kW4a16Choices) {
            if (c.cfg > 2) continue;
            const double tiles = (double)((kp.M + c.bm - 1) / c.bm) * ((kp.N + c.bn - 1) / c.bn);
            const double slots = (double)cus * c.occ;
            const double rounds = tiles <= cus ? 1.0 : (double)(int64_t)((tiles + slots - 1) / slots);
            const double t = rounds * (tiles <= cus ? 1.0 : c.occ) * c.bm * c.bn / c.rate;
            if (t < best_t) {
                best_t = t;
                cfg = c.cfg;
            }
        }
    }
    switch (cfg) {
        case 1: return launch_cfg<128, 256, 2, 4, EPI_SCALE_BF16, S, 2>(kp, 1, stream);
        case 2: return launch_cfg<128, 128, 2, 2, EPI_SCALE_BF16, S, 2>(kp, 1, stream);
        default: return launch_cfg<256, 256, 2, 4, EPI_SCALE_BF16, S, 1>(kp, 1, stream);
    }
}

hipError_t launch_w4a16(const W4a16Problem& p, hipStream_t stream) {
    KParams kp{};
    kp.A = p.A;
    kp.Bq = p.B;
    kp.SFB = p.SFB;
    kp.C = p.C;
    kp.M = (int)p.M;
    kp.N = (int)p.N;
    kp.K = (int)p.K;
    kp.lda = kp.ldb = (int)p.K;
    kp.ldc = (int)p.N;
    kp.k_chunk = (int)p.K;
    kp.scale = p.scale_2;
    if (p.ldbt > 0) {
        kp.ldbt = (int)p.ldbt;
        const int cus = p.cus > 0 ? (int)p.cus : 256;
        return p.ldbt % 4 == 0 ? launch_w4a16_t<SRC_W4A16T4>(kp, cus, stream)
                               : launch_w4a16_t<SRC_W4A16T1>(kp, cus, stream);
    }
    int cfg = tune(BG_TUNE_W4A16_TILE);
    if (cfg < 0) cfg = choose_w4a16(kp.M, kp.N, p.cus > 0 ? (int)p.cus : 256);
    // 32-element weight units when no unit can straddle the end of K; the
    // 16-element units (K % 32 == 16) take the 256 x 256 tile
    if (p.K % 32 != 0) return launch_cfg<256, 256, 2, 4, EPI_SCALE_BF16, SRC_W4A16, 1>(kp, 1, stream);
    constexpr int S = SRC_W4A16W;
    switch (cfg) {
        case 1: return launch_cfg<128, 256, 2, 4, EPI_SCALE_BF16, S, 1>(kp, 1, stream);
        case 2: return launch_cfg<128, 128, 2, 2, EPI_SCALE_BF16, S, 2>(kp, 1, stream);
        case 3: return launch_cfg<256, 256, 2, 2, EPI_SCALE_BF16, S, 1>(kp, 1, stream);
        case 4: return launch_cfg<128, 384, 2, 4, EPI_SCALE_BF16, S, 1>(kp, 1, stream);
        case 5: return launch_cfg<256, 192, 2, 3, EPI_SCALE_BF16, S, 1>(kp, 1, stream);
        case 6: return launch_cfg<128, 384, 2, 4, EPI_SCALE_BF16, S, 2>(kp, 1, stream);
        case 7: return launch_cfg<128, 256, 2, 4, EPI_SCALE_BF16, S, 2>(kp, 1, stream);
        case 9: return launch_cfg<128, 256, 2, 4, EPI_SCALE_BF16, S, 3>(kp, 1, stream);
        default: return launch_cfg<256, 256, 2, 4, EPI_SCALE_BF16, S, 1>(kp, 1, stream);
    }
}

}  // namespace bg
