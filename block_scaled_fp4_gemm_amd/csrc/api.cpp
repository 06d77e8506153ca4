// C ABI entry points: argument validation, device check, kernel dispatch.
//
// Validation is plain host code that touches no HIP API, so every error path
// is reachable without a GPU; the device check runs only once the arguments
// are known to be good. Nothing is enqueued unless every check passes.
#include <atomic>
#include <chrono>
#include <cstring>
#include <random>

#include "bg_internal.hpp"
#include "streamk_plan.hpp"
#include "tile_order.hpp"

namespace {

constexpr uint32_t kMaxDim = 0x7FFFFFFFu;   // kernels index rows and K with int32
constexpr uint32_t kMaxSplits = 64;

struct Range {
    uintptr_t lo, hi;   // [lo, hi), empty when lo == hi
};

Range range_of(const void* p, uint64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + (uintptr_t)bytes};
}

bool overlap(Range x, Range y) {
    if (x.lo == x.hi || y.lo == y.hi) return false;
    return x.lo < y.hi && y.lo < x.hi;
}

bool misaligned(const void* p, uint64_t bytes) {
    return bytes != 0 && (reinterpret_cast<uintptr_t>(p) & 15u) != 0;
}

bool missing(const void* p, uint64_t bytes) { return bytes != 0 && p == nullptr; }

bool dims_ok(uint32_t M, uint32_t N, uint32_t K) {
    return M <= kMaxDim && N <= kMaxDim && K <= kMaxDim;
}

// Per-device cache: 0 unknown, 2 not gfx950, otherwise 2 + compute-unit count.
std::atomic<int> g_dev_info[64];

// Checks the current device and reports its compute-unit count.
bg_status check_device(uint32_t* cus) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return BG_ERR_DEVICE;
    if (dev < 64) {
        const int cached = g_dev_info[dev].load(std::memory_order_relaxed);
        if (cached == 2) return BG_ERR_DEVICE;
        if (cached > 2) {
            *cus = (uint32_t)(cached - 2);
            return BG_OK;
        }
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BG_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    const int n = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
    if (dev < 64) g_dev_info[dev].store(ok ? 2 + n : 2, std::memory_order_relaxed);
    *cus = (uint32_t)n;
    return ok ? BG_OK : BG_ERR_DEVICE;
}

bg_status check_device() {
    uint32_t cus = 0;
    return check_device(&cus);
}

bg_status launched(hipError_t e) { return e == hipSuccess ? BG_OK : BG_ERR_LAUNCH; }

std::atomic<int> g_tune[BG_TUNE_COUNT] = {{-1}, {-1}, {-1}, {-1}, {-1}, {-1}, {-1}};

// Stream-K call numbers: a random 64-bit start per process, then one per
// call, so a flag left in reused memory by another call or process matches
// the current call's number only by a 2^-64 chance.
uint64_t next_epoch() {
    static std::atomic<uint64_t> counter{[] {
        std::random_device rd;
        const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
        return (((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ (t * 0x9E3779B97F4A7C15ull)) | 1u;
    }()};
    uint64_t e = counter.fetch_add(1, std::memory_order_relaxed);
    return e != 0 ? e : counter.fetch_add(1, std::memory_order_relaxed);
}

// Common checks of a dense BF16 problem A[M,K], B[N,K] -> out[M,N] of
// `out_elem` bytes per element.
bg_status check_dense(const void* A, const void* B, const void* out, uint32_t M, uint32_t N,
                      uint32_t K, uint64_t out_elem) {
    if (!dims_ok(M, N, K)) return BG_ERR_SHAPE;
    const uint64_t a_bytes = (uint64_t)M * K * 2, b_bytes = (uint64_t)N * K * 2;
    const uint64_t o_bytes = (uint64_t)M * N * out_elem;
    if (M == 0 || N == 0) return BG_OK;
    if (missing(A, a_bytes) || missing(B, b_bytes) || missing(out, o_bytes)) return BG_ERR_NULL;
    if (misaligned(A, a_bytes) || misaligned(B, b_bytes) || misaligned(out, o_bytes))
        return BG_ERR_ALIGN;
    const Range ro = range_of(out, o_bytes);
    if (overlap(ro, range_of(A, a_bytes)) || overlap(ro, range_of(B, b_bytes))) return BG_ERR_ALIAS;
    return BG_OK;
}

// Common checks of an FP4 problem with `batch` problems stored one after
// another: A [M,K/2], SFA [M,K/16], B [N,K/2], SFB [N,K/16], out of
// out_bytes per problem.
bg_status check_fp4(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                    const void* out, uint64_t out_bytes, uint32_t M, uint32_t N, uint32_t K,
                    uint32_t batch) {
    const uint64_t a_bytes = (uint64_t)batch * M * (K / 2), sa_bytes = (uint64_t)batch * M * (K / 16);
    const uint64_t b_bytes = (uint64_t)batch * N * (K / 2), sb_bytes = (uint64_t)batch * N * (K / 16);
    const uint64_t c_bytes = (uint64_t)batch * out_bytes;
    if (missing(A, a_bytes) || missing(SFA, sa_bytes) || missing(B, b_bytes) || missing(SFB, sb_bytes) ||
        missing(out, c_bytes))
        return BG_ERR_NULL;
    if (misaligned(A, a_bytes) || misaligned(SFA, sa_bytes) || misaligned(B, b_bytes) ||
        misaligned(SFB, sb_bytes) || misaligned(out, c_bytes))
        return BG_ERR_ALIGN;
    const Range rc = range_of(out, c_bytes);
    if (overlap(rc, range_of(A, a_bytes)) || overlap(rc, range_of(SFA, sa_bytes)) ||
        overlap(rc, range_of(B, b_bytes)) || overlap(rc, range_of(SFB, sb_bytes)))
        return BG_ERR_ALIAS;
    return BG_OK;
}

}  // namespace

namespace bg {
int tune(int key) {
    return key >= 0 && key < BG_TUNE_COUNT ? g_tune[key].load(std::memory_order_relaxed) : -1;
}
}  // namespace bg

extern "C" {

bg_status bg_tune_set(int key, int value) {
    if (key < 0 || key >= BG_TUNE_COUNT || value < -1) return BG_ERR_SHAPE;
    g_tune[key].store(value, std::memory_order_relaxed);
    return BG_OK;
}

int bg_tune_get(int key) { return bg::tune(key); }

bg_status bg_tile_map(int order, uint32_t tiles_m, uint32_t tiles_n, int32_t* tm, int32_t* tn) {
    const uint64_t n = (uint64_t)tiles_m * tiles_n;
    if (order < 0 || order > 2 || n >= (uint64_t(1) << 31)) return BG_ERR_SHAPE;
    if (n == 0) return BG_OK;
    if (tm == nullptr || tn == nullptr) return BG_ERR_NULL;
    for (uint64_t b = 0; b < n; ++b) {
        int r = 0, c = 0;
        if (order == bg::ORDER_GEMM)
            bg::tile_of<bg::ORDER_GEMM>((int)b, (int)tiles_m, (int)tiles_n, r, c);
        else if (order == bg::ORDER_FOLD)
            bg::tile_of<bg::ORDER_FOLD>((int)b, (int)tiles_m, (int)tiles_n, r, c);
        else
            bg::tile_of<bg::ORDER_ROWS>((int)b, (int)tiles_m, (int)tiles_n, r, c);
        tm[b] = r;
        tn[b] = c;
    }
    return BG_OK;
}

const char* bg_status_string(bg_status s) {
    switch (s) {
        case BG_OK: return "ok";
        case BG_ERR_NULL: return "a required pointer is NULL";
        case BG_ERR_SHAPE: return "invalid dimensions for this operation";
        case BG_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
        case BG_ERR_WORKSPACE: return "workspace (or output rows) missing or too small";
        case BG_ERR_ALIAS: return "an output overlaps an input";
        case BG_ERR_DEVICE: return "no current HIP device, or it is not gfx950";
        case BG_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

bg_status gemm_bf16(const uint16_t* A, const uint16_t* B, uint16_t* C, uint32_t M, uint32_t N,
                    uint32_t K, void* stream) {
    bg_status s = check_dense(A, B, C, M, N, K, 2);
    if (s != BG_OK || M == 0 || N == 0) return s;
    uint32_t cus = 0;
    if ((s = check_device(&cus)) != BG_OK) return s;
    bg::DenseProblem p{A, B, C, M, N, K, K, K, N, K, 1, 0.0f, cus};
    return launched(bg::launch_dense(p, bg::EPI_STORE_BF16, (hipStream_t)stream));
}

bg_status gemm_bf16_dual(const uint16_t* A, const uint16_t* B0, const uint16_t* B1, uint16_t* C0,
                         uint16_t* C1, uint32_t M, uint32_t N, uint32_t K, void* stream) {
    bg_status s = check_dense(A, B0, C0, M, N, K, 2);
    if (s != BG_OK) return s;
    if ((s = check_dense(A, B1, C1, M, N, K, 2)) != BG_OK) return s;
    if (M == 0 || N == 0) return BG_OK;
    const uint64_t b_bytes = (uint64_t)N * K * 2, c_bytes = (uint64_t)M * N * 2;
    const Range r0 = range_of(C0, c_bytes), r1 = range_of(C1, c_bytes);
    if (overlap(r0, r1) || overlap(r0, range_of(B1, b_bytes)) || overlap(r1, range_of(B0, b_bytes)))
        return BG_ERR_ALIAS;
    uint32_t cus = 0;
    if ((s = check_device(&cus)) != BG_OK) return s;
    bg::DenseProblem p{A, B0, C0, M, N, K, K, K, N, K, 1, 0.0f, cus};
    return launched(bg::launch_dense_dual(p, B1, C1, (hipStream_t)stream));
}

bg_status gemm_bf16_strided(const uint16_t* A, uint32_t lda, const uint16_t* B, uint32_t ldb,
                            uint16_t* C, uint32_t ldc, uint32_t M, uint32_t N, uint32_t K,
                            void* stream) {
    if (!dims_ok(M, N, K) || lda > kMaxDim || ldb > kMaxDim || ldc > kMaxDim) return BG_ERR_SHAPE;
    if (lda < K || ldb < K || ldc < N) return BG_ERR_SHAPE;
    if (M == 0 || N == 0) return BG_OK;
    // bytes spanned: every row but the last is a full stride
    const uint64_t a_bytes = K == 0 ? 0 : ((uint64_t)(M - 1) * lda + K) * 2;
    const uint64_t b_bytes = K == 0 ? 0 : ((uint64_t)(N - 1) * ldb + K) * 2;
    const uint64_t c_bytes = ((uint64_t)(M - 1) * ldc + N) * 2;
    if (missing(A, a_bytes) || missing(B, b_bytes) || missing(C, c_bytes)) return BG_ERR_NULL;
    if (misaligned(A, a_bytes) || misaligned(B, b_bytes) || misaligned(C, c_bytes)) return BG_ERR_ALIGN;
    const Range rc = range_of(C, c_bytes);
    if (overlap(rc, range_of(A, a_bytes)) || overlap(rc, range_of(B, b_bytes))) return BG_ERR_ALIAS;
    uint32_t cus = 0;
    bg_status s = check_device(&cus);
    if (s != BG_OK) return s;
    bg::DenseProblem p{A, B, C, M, N, K, lda, ldb, ldc, K, 1, 0.0f, cus};
    return launched(bg::launch_dense(p, bg::EPI_STORE_BF16, (hipStream_t)stream));
}

bg_status gemm_bf16_scaled_acc(const uint16_t* X, const uint16_t* B, uint16_t* out, uint32_t M,
                               uint32_t N, uint32_t K, float scale, void* stream) {
    bg_status s = check_dense(X, B, out, M, N, K, 2);
    if (s != BG_OK || M == 0 || N == 0) return s;
    uint32_t cus = 0;
    if ((s = check_device(&cus)) != BG_OK) return s;
    bg::DenseProblem p{X, B, out, M, N, K, K, K, N, K, 1, scale, cus};
    return launched(bg::launch_dense(p, bg::EPI_SCALED_ACC, (hipStream_t)stream));
}

size_t gemm_bf16_splitk_workspace_bytes(uint32_t M, uint32_t N, uint32_t k_splits) {
    return (size_t)k_splits * (size_t)M * (size_t)N * sizeof(float);
}

bg_status gemm_bf16_splitk(const uint16_t* A, const uint16_t* B, uint16_t* C, float* workspace,
                           size_t workspace_bytes, uint32_t M, uint32_t N, uint32_t K,
                           uint32_t k_splits, void* stream) {
    if (k_splits == 0 || k_splits > kMaxSplits) return BG_ERR_SHAPE;
    bg_status s = check_dense(A, B, C, M, N, K, 2);
    if (s != BG_OK || M == 0 || N == 0) return s;
    // chunk = ceil(K / k_splits) rounded up to a multiple of 64
    const uint64_t per = ((uint64_t)K + k_splits - 1) / k_splits;
    const uint32_t chunk = (uint32_t)((per + 63) / 64 * 64);
    if (k_splits > 1) {
        const uint64_t need = (uint64_t)k_splits * M * N * 4;
        if (workspace == nullptr || workspace_bytes < need) return BG_ERR_WORKSPACE;
        if (misaligned(workspace, need)) return BG_ERR_ALIGN;
        const Range rw = range_of(workspace, need);
        if (overlap(rw, range_of(A, (uint64_t)M * K * 2)) ||
            overlap(rw, range_of(B, (uint64_t)N * K * 2)) ||
            overlap(rw, range_of(C, (uint64_t)M * N * 2)))
            return BG_ERR_ALIAS;
    }
    uint32_t cus = 0;
    if ((s = check_device(&cus)) != BG_OK) return s;
    const hipStream_t st = (hipStream_t)stream;
    if (k_splits == 1) {
        bg::DenseProblem p{A, B, C, M, N, K, K, K, N, K, 1, 0.0f, cus};
        return launched(bg::launch_dense(p, bg::EPI_STORE_BF16, st));
    }
    bg::DenseProblem p{A, B, workspace, M, N, K, K, K, N, chunk, k_splits, 0.0f, cus};
    hipError_t e = bg::launch_dense(p, bg::EPI_STORE_F32, st);
    if (e != hipSuccess) return BG_ERR_LAUNCH;
    return launched(bg::launch_splitk_reduce(workspace, C, M, N, k_splits, st));
}

bg_status gemm_bf16_splitk_noalloc(const uint16_t* A, const uint16_t* B, uint16_t* C, uint32_t M,
                                   uint32_t N, uint32_t K, uint32_t k_splits, void* stream) {
    if (k_splits == 0 || k_splits > kMaxSplits) return BG_ERR_SHAPE;
    bg_status s = check_dense(A, B, C, M, N, K, 2);
    if (s != BG_OK || M == 0 || N == 0) return s;
    const uint64_t need = (uint64_t)k_splits * M * N * 4;
    if (k_splits > 1 && need > bg::kNoallocScratchBytes) return BG_ERR_WORKSPACE;
    uint32_t cus = 0;
    if ((s = check_device(&cus)) != BG_OK) return s;
    const hipStream_t st = (hipStream_t)stream;
    if (k_splits == 1) {
        bg::DenseProblem p{A, B, C, M, N, K, K, K, N, K, 1, 0.0f, cus};
        return launched(bg::launch_dense(p, bg::EPI_STORE_BF16, st));
    }
    void* ws = nullptr;
    if (bg::noalloc_scratch(&ws) != hipSuccess) return BG_ERR_DEVICE;
    const uint64_t per = ((uint64_t)K + k_splits - 1) / k_splits;
    const uint32_t chunk = (uint32_t)((per + 63) / 64 * 64);
    bg::DenseProblem p{A, B, ws, M, N, K, K, K, N, chunk, k_splits, 0.0f, cus};
    hipError_t e = bg::launch_dense(p, bg::EPI_STORE_F32, st);
    if (e != hipSuccess) return BG_ERR_LAUNCH;
    return launched(bg::launch_splitk_reduce(static_cast<const float*>(ws), C, M, N, k_splits, st));
}

bg_status gemm_bf16_streamk_workspace(uint32_t M, uint32_t N, uint32_t K, size_t* bytes) {
    if (bytes == nullptr) return BG_ERR_NULL;
    if (!dims_ok(M, N, K)) return BG_ERR_SHAPE;
    uint32_t cus = 0;
    bg_status s = check_device(&cus);
    if (s != BG_OK) return s;
    bg::streamk_choose(M, N, K, cus, bg::tune(BG_TUNE_STREAMK_TILE), bytes);
    return BG_OK;
}

bg_status gemm_bf16_streamk(const uint16_t* A, const uint16_t* B, uint16_t* C, void* workspace,
                            size_t workspace_bytes, uint32_t M, uint32_t N, uint32_t K, void* stream) {
    bg_status s = check_dense(A, B, C, M, N, K, 2);
    if (s != BG_OK || M == 0 || N == 0) return s;
    const bool sk = bg::streamk_applies(M, N, K);
    if (sk && workspace == nullptr) return BG_ERR_WORKSPACE;
    if (sk && misaligned(workspace, 1)) return BG_ERR_ALIGN;
    uint32_t cus = 0;
    if ((s = check_device(&cus)) != BG_OK) return s;
    bg::DenseProblem p{A, B, C, M, N, K, K, K, N, K, 1, 0.0f, cus};
    if (!sk) return launched(bg::launch_dense(p, bg::EPI_STORE_BF16, (hipStream_t)stream));
    size_t need = 0;
    const int cfg = bg::streamk_choose(M, N, K, cus, bg::tune(BG_TUNE_STREAMK_TILE), &need);
    if (workspace_bytes < need) return BG_ERR_WORKSPACE;
    const Range rw = range_of(workspace, need);
    if (overlap(rw, range_of(A, (uint64_t)M * K * 2)) || overlap(rw, range_of(B, (uint64_t)N * K * 2)) ||
        overlap(rw, range_of(C, (uint64_t)M * N * 2)))
        return BG_ERR_ALIAS;
    return launched(bg::launch_streamk(p, workspace, cfg, next_epoch(), (hipStream_t)stream));
}

bg_status bg_streamk_plan(uint32_t tiles, uint32_t steps, uint32_t wgs_per_xcd, int32_t* rows,
                          size_t max_rows, size_t* n_rows) {
    if (n_rows == nullptr) return BG_ERR_NULL;
    if (tiles >= (1u << 30) || steps >= (1u << 30) || wgs_per_xcd == 0 || wgs_per_xcd > 4096 ||
        (uint64_t)(tiles / bg::SK_XCDS + 1) * steps >= (uint64_t(1) << 30))
        return BG_ERR_SHAPE;
    size_t n = 0;
    for (uint32_t b = 0; b < bg::SK_XCDS * wgs_per_xcd; ++b) {
        bg::SkWorkgroup wg;
        wg.init((int)tiles, (int)steps, (int)wgs_per_xcd, (int)(b % bg::SK_XCDS), (int)(b / bg::SK_XCDS));
        for (int q = 0; q < wg.count(); ++q, ++n) {
            if (rows == nullptr || n >= max_rows) continue;
            const bg::SkPiece pc = wg.piece(q);
            int32_t* r = rows + 6 * n;
            r[0] = (int32_t)b;
            r[1] = wg.t0 + pc.tile;
            r[2] = pc.s_begin;
            r[3] = pc.s_end;
            r[4] = pc.partial;
            r[5] = pc.src_first;
        }
    }
    *n_rows = n;
    return rows != nullptr && n > max_rows ? BG_ERR_WORKSPACE : BG_OK;
}

bg_status gemm_bf16_ordered(const uint16_t* A, const uint16_t* B, uint16_t* C, uint32_t M,
                            uint32_t N, uint32_t K, void* stream) {
    bg_status s = check_dense(A, B, C, M, N, K, 2);
    if (s != BG_OK || M == 0 || N == 0) return s;
    uint32_t cus = 0;
    if ((s = check_device(&cus)) != BG_OK) return s;
    return launched(bg::launch_ordered(A, B, C, false, M, N, K, cus, (hipStream_t)stream));
}

bg_status gemm_bf16_ordered_f32(const uint16_t* A, const uint16_t* B, float* C32, uint32_t M,
                                uint32_t N, uint32_t K, void* stream) {
    bg_status s = check_dense(A, B, C32, M, N, K, 4);
    if (s != BG_OK || M == 0 || N == 0) return s;
    uint32_t cus = 0;
    if ((s = check_device(&cus)) != BG_OK) return s;
    return launched(bg::launch_ordered(A, B, C32, true, M, N, K, cus, (hipStream_t)stream));
}

bg_status gemm_fp4_blockscaled(const uint8_t* A, const uint8_t* SFA, const uint8_t* B,
                               const uint8_t* SFB, uint16_t* C, uint32_t M, uint32_t N, uint32_t K,
                               void* stream) {
    return gemm_fp4_blockscaled_batched(A, SFA, B, SFB, C, M, N, K, 1, stream);
}

bg_status gemm_fp4_blockscaled_batched(const uint8_t* A, const uint8_t* SFA, const uint8_t* B,
                                       const uint8_t* SFB, uint16_t* C, uint32_t M, uint32_t N,
                                       uint32_t K, uint32_t L, void* stream) {
    if (!dims_ok(M, N, K) || (K % 16) != 0 || L > 65535) return BG_ERR_SHAPE;
    if (M == 0 || N == 0 || L == 0) return BG_OK;
    bg_status s = check_fp4(A, SFA, B, SFB, C, (uint64_t)M * N * 2, M, N, K, L);
    if (s != BG_OK) return s;
    uint32_t cus = 0;
    if ((s = check_device(&cus)) != BG_OK) return s;
    bg::Fp4Problem p{A, SFA, B, SFB, C, M, N, K, K, 1, L, cus};
    return launched(bg::launch_fp4(p, (hipStream_t)stream));
}

bg_status gemm_fp4_blockscaled_splitk(const uint8_t* A, const uint8_t* SFA, const uint8_t* B,
                                      const uint8_t* SFB, uint16_t* C, float* workspace,
                                      size_t workspace_bytes, uint32_t M, uint32_t N, uint32_t K,
                                      uint32_t k_splits, void* stream) {
    if (k_splits == 0 || k_splits > kMaxSplits) return BG_ERR_SHAPE;
    if (!dims_ok(M, N, K) || (K % 16) != 0) return BG_ERR_SHAPE;
    if (M == 0 || N == 0) return BG_OK;
    bg_status s = check_fp4(A, SFA, B, SFB, C, (uint64_t)M * N * 2, M, N, K, 1);
    if (s != BG_OK) return s;
    uint32_t cus = 0;
    if (k_splits == 1) {
        if ((s = check_device(&cus)) != BG_OK) return s;
        bg::Fp4Problem p{A, SFA, B, SFB, C, M, N, K, K, 1, 1, cus};
        return launched(bg::launch_fp4(p, (hipStream_t)stream));
    }
    const uint64_t per = ((uint64_t)K + k_splits - 1) / k_splits;
    const uint32_t chunk = (uint32_t)((per + 63) / 64 * 64);
    const uint64_t need = (uint64_t)k_splits * M * N * 4;
    if (workspace == nullptr || workspace_bytes < need) return BG_ERR_WORKSPACE;
    if (misaligned(workspace, need)) return BG_ERR_ALIGN;
    const Range rw = range_of(workspace, need);
    if (overlap(rw, range_of(A, (uint64_t)M * (K / 2))) || overlap(rw, range_of(SFA, (uint64_t)M * (K / 16))) ||
        overlap(rw, range_of(B, (uint64_t)N * (K / 2))) || overlap(rw, range_of(SFB, (uint64_t)N * (K / 16))) ||
        overlap(rw, range_of(C, (uint64_t)M * N * 2)))
        return BG_ERR_ALIAS;
    if ((s = check_device(&cus)) != BG_OK) return s;
    const hipStream_t st = (hipStream_t)stream;
    bg::Fp4Problem p{A, SFA, B, SFB, workspace, M, N, K, chunk, k_splits, 1, cus};
    hipError_t e = bg::launch_fp4(p, st);
    if (e != hipSuccess) return BG_ERR_LAUNCH;
    return launched(bg::launch_splitk_reduce(workspace, C, M, N, k_splits, st));
}

bg_status fp4_scales_from_blocked(const uint8_t* blocked, uint8_t* plain, uint32_t rows,
                                  uint32_t k_groups, uint32_t batch, void* stream) {
    if (rows % 128 != 0 || k_groups % 4 != 0 || rows > kMaxDim || k_groups > kMaxDim || batch > 65535)
        return BG_ERR_SHAPE;
    const uint64_t bytes = (uint64_t)batch * rows * k_groups;
    if (bytes == 0) return BG_OK;
    if (missing(blocked, bytes) || missing(plain, bytes)) return BG_ERR_NULL;
    if (misaligned(blocked, bytes) || misaligned(plain, bytes)) return BG_ERR_ALIGN;
    if (overlap(range_of(blocked, bytes), range_of(plain, bytes))) return BG_ERR_ALIAS;
    bg_status s = check_device();
    if (s != BG_OK) return s;
    return launched(bg::launch_scales_from_blocked(blocked, plain, rows, k_groups, batch, (hipStream_t)stream));
}

bg_status gemm_w4a16(const uint16_t* A, const uint8_t* B, const uint8_t* SFB, float scale_2,
                     uint16_t* C, uint32_t M, uint32_t N, uint32_t K, void* stream) {
    if (!dims_ok(M, N, K) || (K % 16) != 0) return BG_ERR_SHAPE;
    if (M == 0 || N == 0) return BG_OK;
    const uint64_t a_bytes = (uint64_t)M * K * 2;
    const uint64_t b_bytes = (uint64_t)N * (K / 2), sb_bytes = (uint64_t)N * (K / 16);
    const uint64_t c_bytes = (uint64_t)M * N * 2;
    if (missing(A, a_bytes) || missing(B, b_bytes) || missing(SFB, sb_bytes) || missing(C, c_bytes))
        return BG_ERR_NULL;
    if (misaligned(A, a_bytes) || misaligned(B, b_bytes) || misaligned(SFB, sb_bytes) ||
        misaligned(C, c_bytes))
        return BG_ERR_ALIGN;
    const Range rc = range_of(C, c_bytes);
    if (overlap(rc, range_of(A, a_bytes)) || overlap(rc, range_of(B, b_bytes)) ||
        overlap(rc, range_of(SFB, sb_bytes)))
        return BG_ERR_ALIAS;
    uint32_t cus = 0;
    bg_status s = check_device(&cus);
    if (s != BG_OK) return s;
    bg::W4a16Problem p{A, B, SFB, C, M, N, K, scale_2, cus, 0};
    return launched(bg::launch_w4a16(p, (hipStream_t)stream));
}

bg_status gemm_w4a16_t(const uint16_t* A, const uint8_t* Bt, const uint8_t* SFBt, uint32_t ldb, float scale_2,
                       uint16_t* C, uint32_t M, uint32_t N, uint32_t K, void* stream) {
    if (!dims_ok(M, N, K) || (K % 16) != 0 || ldb > kMaxDim || ldb < N || ldb == 0) return BG_ERR_SHAPE;
    if (M == 0 || N == 0) return BG_OK;
    const uint64_t a_bytes = (uint64_t)M * K * 2;
    const uint64_t b_bytes = (uint64_t)(K / 2) * ldb, sb_bytes = (uint64_t)(K / 16) * ldb;
    const uint64_t c_bytes = (uint64_t)M * N * 2;
    if (missing(A, a_bytes) || missing(Bt, b_bytes) || missing(SFBt, sb_bytes) || missing(C, c_bytes))
        return BG_ERR_NULL;
    if (misaligned(A, a_bytes) || misaligned(Bt, b_bytes) || misaligned(SFBt, sb_bytes) || misaligned(C, c_bytes))
        return BG_ERR_ALIGN;
    const Range rc = range_of(C, c_bytes);
    if (overlap(rc, range_of(A, a_bytes)) || overlap(rc, range_of(Bt, b_bytes)) ||
        overlap(rc, range_of(SFBt, sb_bytes)))
        return BG_ERR_ALIAS;
    uint32_t cus = 0;
    bg_status s = check_device(&cus);
    if (s != BG_OK) return s;
    bg::W4a16Problem p{A, Bt, SFBt, C, M, N, K, scale_2, cus, ldb};
    return launched(bg::launch_w4a16(p, (hipStream_t)stream));
}

bg_status bf16_scaled_add(uint16_t* out, const uint16_t* delta, size_t count, float scale,
                          void* stream) {
    if (count == 0) return BG_OK;
    if (count > ((size_t)1 << 62)) return BG_ERR_SHAPE;
    const uint64_t bytes = (uint64_t)count * 2;
    if (missing(out, bytes) || missing(delta, bytes)) return BG_ERR_NULL;
    if (misaligned(out, bytes) || misaligned(delta, bytes)) return BG_ERR_ALIGN;
    if (overlap(range_of(out, bytes), range_of(delta, bytes))) return BG_ERR_ALIAS;
    bg_status s = check_device();
    if (s != BG_OK) return s;
    return launched(bg::launch_scaled_add(out, delta, count, scale, (hipStream_t)stream));
}

}  // extern "C"
