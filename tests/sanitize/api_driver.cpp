// Sanitizer driver for the C-ABI validation layer (api.cpp), built for the
// host with -fsanitize=address,undefined against hip_stub/. The kernel
// launchers are replaced by recorders that check what validation hands them;
// the device query is a stub (device 0: gfx950 with 256 CUs, device 1: another
// architecture). Fake device addresses are never dereferenced.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../block_scaled_fp4_gemm_amd/csrc/bg_internal.hpp"
#include "../../block_scaled_fp4_gemm_amd/csrc/streamk_plan.hpp"

static int g_dev = 0;
static int g_sk_cfg = -1;
static size_t g_sk_need = 0;
static int g_launches = 0;
static bg::DenseProblem g_last{};

hipError_t hipGetDevice(int* dev) {
    *dev = g_dev;
    return hipSuccess;
}

hipError_t hipGetDeviceProperties(hipDeviceProp_t* prop, int dev) {
    std::memset(prop, 0, sizeof(*prop));
    std::strcpy(prop->gcnArchName, dev == 0 ? "gfx950:sramecc+:xnack-" : "gfx942");
    prop->multiProcessorCount = 256;
    return hipSuccess;
}

#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            std::exit(1);                                                    \
        }                                                                    \
    } while (0)

namespace bg {
static void record_dense(const DenseProblem& p) {
    CHECK(p.M > 0 && p.N > 0);
    CHECK(p.splits >= 1 && p.splits <= 64);
    CHECK((uint64_t)p.k_chunk * p.splits >= p.K);
    CHECK(p.lda >= p.K && p.ldb >= p.K && p.ldc >= p.N);
    CHECK(p.cus == 256);
    g_last = p;
    ++g_launches;
}
hipError_t launch_dense(const DenseProblem& p, Epilogue, hipStream_t) {
    record_dense(p);
    return hipSuccess;
}
hipError_t launch_dense_dual(const DenseProblem& p, const uint16_t* B1, uint16_t* C1, hipStream_t) {
    CHECK(B1 != nullptr || p.K == 0);
    CHECK(C1 != nullptr);
    record_dense(p);
    return hipSuccess;
}
hipError_t launch_fp4(const Fp4Problem& p, hipStream_t) {
    CHECK(p.M > 0 && p.N > 0 && p.K % 16 == 0 && p.batch >= 1);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_scales_from_blocked(const uint8_t*, uint8_t*, uint32_t rows, uint32_t k_groups, uint32_t,
                                      hipStream_t) {
    CHECK(rows % 128 == 0 && k_groups % 4 == 0);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_w4a16(const W4a16Problem& p, hipStream_t) {
    CHECK(p.M > 0 && p.N > 0 && p.K % 16 == 0);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_ordered(const uint16_t*, const uint16_t*, void*, bool, uint32_t M, uint32_t N, uint32_t,
                          uint32_t cus, hipStream_t) {
    CHECK(M > 0 && N > 0 && cus == 256);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_splitk_reduce(const float* ws, uint16_t* C, uint32_t M, uint32_t N, uint32_t splits,
                                hipStream_t) {
    CHECK(ws != nullptr && C != nullptr && M > 0 && N > 0 && splits >= 2);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_scaled_add(uint16_t* out, const uint16_t* delta, size_t count, float, hipStream_t) {
    CHECK(out != nullptr && delta != nullptr && count > 0);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_streamk(const DenseProblem& p, void* ws, int cfg, uint64_t epoch, hipStream_t) {
    CHECK(ws != nullptr && epoch != 0 && (cfg == 23 || cfg == 10));
    CHECK(p.K > 0 && p.K % 8 == 0 && p.lda == p.K && p.ldb == p.K && p.ldc == p.N);
    size_t need = 0;
    CHECK(streamk_choose(p.M, p.N, p.K, p.cus, -1, &need) == cfg || g_sk_cfg >= 0);
    g_sk_cfg = cfg;
    g_sk_need = need;
    record_dense(p);
    return hipSuccess;
}
static float g_fake_scratch[4];
hipError_t noalloc_scratch(void** ptr) {
    *ptr = g_fake_scratch;
    return hipSuccess;
}
}  // namespace bg

template <class T>
static T* at(uintptr_t a) {
    return reinterpret_cast<T*>(a);
}

int main() {
    const uintptr_t A = 0x10000000, B = 0x20000000, C = 0x30000000, W = 0x40000000, S1 = 0x50000000,
                    S2 = 0x60000000;
    auto u16 = at<uint16_t>;
    auto u8 = at<uint8_t>;
    auto f32 = at<float>;

    // valid calls reach the launcher with consistent problems
    CHECK(gemm_bf16(u16(A), u16(B), u16(C), 5120, 11008, 2048, nullptr) == BG_OK);
    CHECK(g_last.M == 5120 && g_last.N == 11008 && g_last.k_chunk == 2048);
    CHECK(gemm_bf16_splitk(u16(A), u16(B), u16(C), f32(W), (size_t)8 * 5120 * 2048 * 4, 5120, 2048, 11008, 8,
                           nullptr) == BG_OK);
    CHECK(g_last.splits == 8 && g_last.k_chunk == 1408);
    CHECK(gemm_bf16_splitk_noalloc(u16(A), u16(B), u16(C), 128, 2048, 11008, 8, nullptr) == BG_OK);
    CHECK(gemm_bf16_splitk_noalloc(u16(A), u16(B), u16(C), 1024, 2048, 11008, 8, nullptr) == BG_ERR_WORKSPACE);
    CHECK(gemm_bf16_dual(u16(A), u16(B), u16(S1), u16(C), u16(W), 5120, 11008, 2048, nullptr) == BG_OK);
    CHECK(gemm_bf16_strided(u16(A), 4099, u16(B), 2048, u16(C), 11008, 17, 11008, 2048, nullptr) == BG_OK);
    CHECK(gemm_bf16_scaled_acc(u16(A), u16(B), u16(C), 2048, 17408, 64, 2.0f, nullptr) == BG_OK);
    CHECK(gemm_bf16_ordered(u16(A), u16(B), u16(C), 4510, 256, 2048, nullptr) == BG_OK);
    CHECK(gemm_bf16_ordered_f32(u16(A), u16(B), f32(C), 4510, 256, 2048, nullptr) == BG_OK);
    CHECK(gemm_fp4_blockscaled(u8(A), u8(S1), u8(B), u8(S2), u16(C), 4096, 4096, 8192, nullptr) == BG_OK);
    CHECK(gemm_fp4_blockscaled_batched(u8(A), u8(S1), u8(B), u8(S2), u16(C), 128, 256, 512, 3, nullptr) == BG_OK);
    CHECK(gemm_fp4_blockscaled_splitk(u8(A), u8(S1), u8(B), u8(S2), u16(C), f32(W), (size_t)8 * 128 * 7168 * 4,
                                      128, 7168, 16384, 8, nullptr) == BG_OK);
    CHECK(fp4_scales_from_blocked(u8(S1), u8(S2), 256, 64, 2, nullptr) == BG_OK);
    CHECK(gemm_w4a16(u16(A), u8(B), u8(S2), 0.5f, u16(C), 1016, 12288, 2048, nullptr) == BG_OK);
    CHECK(bf16_scaled_add(u16(A), u16(B), 1000, 0.5f, nullptr) == BG_OK);
    CHECK(gemm_w4a16_t(u16(A), u8(B), u8(S2), 248192, 0.5f, u16(C), 37, 248077, 2048, nullptr) == BG_OK);
    size_t sk_need = 0;
    CHECK(gemm_bf16_streamk_workspace(5120, 512, 2048, &sk_need) == BG_OK);
    CHECK(sk_need == (size_t)256 * (128 * 128 * 4 + 8) || sk_need == (size_t)256 * (256 * 128 * 4 + 8));
    CHECK(gemm_bf16_streamk(u16(A), u16(B), u16(C), u8(W), sk_need, 5120, 512, 2048, nullptr) == BG_OK);
    CHECK(g_sk_need == sk_need);
    CHECK(gemm_bf16_streamk(u16(A), u16(B), u16(C), nullptr, 0, 70, 90, 100, nullptr) == BG_OK);   // K % 8
    CHECK(gemm_bf16_streamk(u16(A), u16(B), u16(C), nullptr, 0, 40, 30, 0, nullptr) == BG_OK);     // K == 0
    for (uint32_t m : {0u, 1u, 40u, 5120u})
        for (uint32_t k : {0u, 1u, 8u, 64u, 2048u}) CHECK(gemm_bf16_streamk_workspace(m, 30, k, &sk_need) == BG_OK);
    CHECK(gemm_bf16_streamk_workspace(5120, 512, 2048, &sk_need) == BG_OK);
    {
        size_t rows = 0;
        CHECK(bg_streamk_plan(160, 32, 32, nullptr, 0, &rows) == BG_OK && rows == 384);
        std::vector<int32_t> plan(6 * rows);
        CHECK(bg_streamk_plan(160, 32, 32, plan.data(), rows, &rows) == BG_OK);
        CHECK(bg_streamk_plan(1720, 32, 32, nullptr, 0, &rows) == BG_OK);
        std::vector<int32_t> big_plan(6 * rows);
        CHECK(bg_streamk_plan(1720, 32, 32, big_plan.data(), rows, &rows) == BG_OK);
        CHECK(bg_streamk_plan(3, 100, 1, nullptr, 0, &rows) == BG_OK);
        CHECK(bg_streamk_plan(7, 1, 32, nullptr, 0, &rows) == BG_OK && rows == 7);
    }
    const int valid = g_launches;

    // invalid calls return their status and launch nothing
    const uint32_t big = 0xFFFFFFFFu;
    CHECK(gemm_bf16(u16(A), u16(B), u16(C), big, big, big, nullptr) == BG_ERR_SHAPE);
    CHECK(gemm_bf16(u16(A), u16(B), u16(C), 0x7FFFFFFFu, 0x7FFFFFFFu, 0x7FFFFFFFu, nullptr) == BG_ERR_ALIAS);
    CHECK(gemm_bf16(nullptr, u16(B), u16(C), 4, 4, 4, nullptr) == BG_ERR_NULL);
    CHECK(gemm_bf16(u16(A + 2), u16(B), u16(C), 4, 4, 4, nullptr) == BG_ERR_ALIGN);
    CHECK(gemm_bf16(u16(A), u16(B), u16(A + 16), 4, 4, 64, nullptr) == BG_ERR_ALIAS);
    CHECK(gemm_bf16_splitk(u16(A), u16(B), u16(C), f32(W), 10, 4, 4, 128, 2, nullptr) == BG_ERR_WORKSPACE);
    CHECK(gemm_bf16_splitk(u16(A), u16(B), u16(C), f32(W), 1 << 20, 4, 4, 128, 65, nullptr) == BG_ERR_SHAPE);
    CHECK(gemm_bf16_splitk_noalloc(u16(A), u16(B), u16(C), big, 4, 4, 2, nullptr) == BG_ERR_SHAPE);
    CHECK(gemm_bf16_strided(u16(A), big, u16(B), 8, u16(C), 4, 4, 4, 8, nullptr) == BG_ERR_SHAPE);
    CHECK(gemm_bf16_strided(u16(A), 0x7FFFFFFFu, u16(B), 0x7FFFFFFFu, u16(C), 0x7FFFFFFFu, 0x7FFFFFFFu,
                            0x7FFFFFFFu, 8, nullptr) == BG_ERR_ALIAS);
    CHECK(gemm_fp4_blockscaled(u8(A), u8(S1), u8(B), u8(S2), u16(C), 4, 4, 40, nullptr) == BG_ERR_SHAPE);
    CHECK(gemm_fp4_blockscaled_batched(u8(A), u8(S1), u8(B), u8(S2), u16(C), 0x7FFFFFFFu, 0x7FFFFFFFu, 0x7FFFFFF0u,
                                       65535, nullptr) != BG_OK);
    CHECK(fp4_scales_from_blocked(u8(S1), u8(S2), 100, 4, 1, nullptr) == BG_ERR_SHAPE);
    CHECK(gemm_w4a16(u16(A), u8(B), u8(S2), 1.0f, u16(C), 4, big, 32, nullptr) == BG_ERR_SHAPE);
    CHECK(gemm_w4a16_t(u16(A), u8(B), u8(S2), 100, 1.0f, u16(C), 4, 101, 32, nullptr) == BG_ERR_SHAPE);
    CHECK(gemm_w4a16_t(u16(A), u8(B), u8(S2), 0x7FFFFFFFu, 1.0f, u16(C), 4, 101, 0x7FFFFFF0u, nullptr) == BG_ERR_ALIAS);
    CHECK(bf16_scaled_add(u16(A), u16(A + 16), 64, 1.0f, nullptr) == BG_ERR_ALIAS);
    CHECK(bf16_scaled_add(u16(A), u16(B), (size_t)1 << 63, 1.0f, nullptr) == BG_ERR_SHAPE);
    CHECK(gemm_bf16_streamk(u16(A), u16(B), u16(C), u8(W), sk_need - 1, 5120, 512, 2048, nullptr) == BG_ERR_WORKSPACE);
    CHECK(gemm_bf16_streamk(u16(A), u16(B), u16(C), nullptr, sk_need, 5120, 512, 2048, nullptr) == BG_ERR_WORKSPACE);
    CHECK(gemm_bf16_streamk(u16(A), u16(B), u16(C), u8(A + 16), sk_need, 5120, 512, 2048, nullptr) == BG_ERR_ALIAS);
    CHECK(gemm_bf16_streamk(u16(A), u16(B), u16(C), u8(W + 4), sk_need, 5120, 512, 2048, nullptr) == BG_ERR_ALIGN);
    CHECK(gemm_bf16_streamk_workspace(4, 4, big, &sk_need) == BG_ERR_SHAPE);
    {
        size_t rows = 0;
        int32_t one[6];
        CHECK(bg_streamk_plan(160, 32, 32, one, 1, &rows) == BG_ERR_WORKSPACE && rows == 384);
        CHECK(bg_streamk_plan(1u << 30, 1, 32, nullptr, 0, &rows) == BG_ERR_SHAPE);
        CHECK(bg_streamk_plan(4, 4, 0, nullptr, 0, &rows) == BG_ERR_SHAPE);
    }
    CHECK(g_launches == valid);

    // a device of another architecture is refused
    g_dev = 1;
    CHECK(gemm_bf16(u16(A), u16(B), u16(C), 4, 4, 8, nullptr) == BG_ERR_DEVICE);
    CHECK(gemm_bf16(u16(A), u16(B), u16(C), 4, 4, 8, nullptr) == BG_ERR_DEVICE);   // cached
    g_dev = 0;
    CHECK(g_launches == valid);

    // tuning overrides
    CHECK(bg_tune_set(BG_TUNE_TILE, 3) == BG_OK && bg_tune_get(BG_TUNE_TILE) == 3);
    CHECK(bg_tune_set(BG_TUNE_TILE, -1) == BG_OK && bg_tune_get(BG_TUNE_TILE) == -1);
    CHECK(bg_tune_set(BG_TUNE_COUNT, 0) == BG_ERR_SHAPE && bg_tune_set(-1, 0) == BG_ERR_SHAPE);
    CHECK(bg_tune_get(1000) == -1 && bg_tune_get(-5) == -1);

    // every tile order is a bijection onto its grid
    const int grids[][2] = {{20, 86}, {20, 37}, {32, 8}, {40, 4}, {32, 136}, {1, 1}, {1, 7}, {7, 1},
                            {9, 13}, {41, 41}, {1, 255}, {255, 1}, {33, 65}, {5, 3}};
    for (const auto& g : grids) {
        const int n = g[0] * g[1];
        std::vector<int32_t> tm(n), tn(n);
        std::vector<int> seen(n);
        for (int order = 0; order < 3; ++order) {
            CHECK(bg_tile_map(order, g[0], g[1], tm.data(), tn.data()) == BG_OK);
            std::fill(seen.begin(), seen.end(), 0);
            for (int b = 0; b < n; ++b) {
                CHECK(tm[b] >= 0 && tm[b] < g[0] && tn[b] >= 0 && tn[b] < g[1]);
                CHECK(++seen[tm[b] * g[1] + tn[b]] == 1);
            }
        }
    }
    CHECK(bg_tile_map(3, 2, 2, nullptr, nullptr) == BG_ERR_SHAPE);
    CHECK(bg_tile_map(0, 65536, 32768, nullptr, nullptr) == BG_ERR_SHAPE);
    CHECK(bg_tile_map(0, 2, 2, nullptr, nullptr) == BG_ERR_NULL);
    for (int s = 0; s <= 8; ++s) CHECK(bg_status_string((bg_status)s)[0] != 0);
    std::printf("api sanitizer driver: ok (%d launches recorded)\n", g_launches);
    return 0;
}
