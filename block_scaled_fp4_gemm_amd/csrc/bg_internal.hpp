// Internal host-side declarations shared by the C-ABI layer and the kernel
// translation units. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/blockgemm.h"

namespace bg {

// Epilogue applied to the FP32 accumulator tile of the MFMA core.
enum Epilogue : int {
    EPI_STORE_BF16 = 0,   // C = bf16(acc)
    EPI_SCALED_ACC = 1,   // out = bf16(out + scale * bf16(acc)), in place
    EPI_STORE_F32 = 2,    // plane[blockIdx.z] = acc (split-K partials)
    EPI_SCALE_BF16 = 3,   // C = bf16(fl32(scale * acc))  (W4A16 per-tensor scale)
};

struct DenseProblem {
    const uint16_t* A;   // [M, K] bf16
    const uint16_t* B;   // [N, K] bf16
    void* C;             // [M, N] bf16, or [splits][M][N] f32 planes
    uint32_t M, N, K;
    uint32_t lda, ldb;   // elements between rows of A and of B (>= K)
    uint32_t ldc;        // elements between rows of C (>= N; N for split-K planes)
    uint32_t k_chunk;    // K elements per split (multiple of 64, or K)
    uint32_t splits;
    float scale;
    uint32_t cus;        // compute units of the current device (tile choice), 0 = unknown
};

struct Fp4Problem {
    const uint8_t* A;    // [batch][M, K/2]
    const uint8_t* SFA;  // [batch][M, K/16]
    const uint8_t* B;    // [batch][N, K/2]
    const uint8_t* SFB;  // [batch][N, K/16]
    void* C;             // [batch][M, N] bf16, or [splits][M][N] f32 planes
    uint32_t M, N, K;
    uint32_t k_chunk;    // K elements per split (multiple of 64, or K)
    uint32_t splits;     // > 1: FP32 planes (batch must be 1)
    uint32_t batch;
    uint32_t cus;        // compute units of the device (0: 256)
};

struct W4a16Problem {
    const uint16_t* A;   // [M, K] bf16 activations
    const uint8_t* B;    // [N, K/2] packed e2m1 weights
    const uint8_t* SFB;  // [N, K/16] e4m3fn
    uint16_t* C;         // [M, N] bf16
    uint32_t M, N, K;
    float scale_2;       // per-tensor weight scale
    uint32_t cus;        // compute units of the current device (tile choice)
    uint32_t ldbt;       // 0: B [N, K/2], SFB [N, K/16]; else B [K/2, ldbt], SFB [K/16, ldbt] (transposed)
};

// Size of the library-owned split-K scratch of gemm_bf16_splitk_noalloc, per
// device (noalloc.hip).
constexpr size_t kNoallocScratchBytes = BG_NOALLOC_SCRATCH_BYTES;
// Device address of the current device's scratch (taken once per device).
hipError_t noalloc_scratch(void** ptr);

// Current tuning override of a bg_tune_key (-1: automatic choice).
int tune(int key);

// Kernel launchers (defined in the .hip files). They enqueue on `stream` and
// return hipGetLastError() of the launch. Shapes are already validated and
// non-empty (M > 0, N > 0).
hipError_t launch_dense(const DenseProblem& p, Epilogue epi, hipStream_t stream);
// C0 = bf16(A * B^T) (the problem p, BF16 store) and C1 = bf16(A * B1^T) of the
// same shape, in one launch when the direct kernels apply.
hipError_t launch_dense_dual(const DenseProblem& p, const uint16_t* B1, uint16_t* C1, hipStream_t stream);
hipError_t launch_fp4(const Fp4Problem& p, hipStream_t stream);
// Stream-K (gemm_bf16_streamk; the plan and the tile choice are in
// streamk_plan.hpp): p.C is the BF16 output, ws the workspace of
// streamk_choose's size for configuration cfg.
hipError_t launch_streamk(const DenseProblem& p, void* ws, int cfg, uint64_t epoch, hipStream_t stream);
hipError_t launch_scales_from_blocked(const uint8_t* src, uint8_t* dst, uint32_t rows, uint32_t k_groups,
                                      uint32_t batch, hipStream_t stream);
hipError_t launch_w4a16(const W4a16Problem& p, hipStream_t stream);
hipError_t launch_ordered(const uint16_t* A, const uint16_t* B, void* C, bool f32_out,
                          uint32_t M, uint32_t N, uint32_t K, uint32_t cus, hipStream_t stream);
hipError_t launch_splitk_reduce(const float* ws, uint16_t* C, uint32_t M, uint32_t N,
                                uint32_t splits, hipStream_t stream);
hipError_t launch_scaled_add(uint16_t* out, const uint16_t* delta, size_t count, float scale,
                             hipStream_t stream);

}  // namespace bg
