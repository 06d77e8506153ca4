/*
 * blockgemm.h - C ABI of the MI355X (gfx950) dense-BF16 / block-scaled-FP4
 * GEMM library.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Layout: A is [M, K], B is [N, K], C is [M, N], all row-major and densely
 *    packed, so both operands are K-contiguous and C = A * B^T. This is the
 *    layout of the gemm_dense.rs page (doc comment of the dense BF16 GEMM:
 *    A [M, K] activations, B [N, K] weights in HuggingFace layout, C [M, N]).
 *  - BF16 values travel as their raw 16-bit patterns (uint16_t).
 *  - Every data pointer is a DEVICE pointer on the current HIP device. The
 *    caller allocates and owns every buffer (including the split-K and
 *    stream-K workspaces);
 *    the library never allocates, frees or retains device memory and never
 *    synchronizes. Buffers must stay alive until the enqueued work finishes.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *    All work is enqueued on that stream in order.
 *  - Every FP32 -> BF16 conversion rounds to nearest, ties to even; NaN stays
 *    NaN. Accumulation is FP32.
 *  - Return value: BG_OK, or the first failed check. Arguments are validated
 *    completely before anything is enqueued, so a failing call enqueues
 *    nothing. Device-side faults surface at the caller's next synchronization.
 *  - M == 0 or N == 0 is a valid empty problem (BG_OK, nothing enqueued).
 *    K == 0 is the empty sum: C = +0 (gemm_bf16_scaled_acc then leaves the
 *    values of `out` unchanged).
 *  - Base pointers of non-empty tensors must be 16-byte aligned
 *    (BG_ERR_ALIGN otherwise). Row pitches need no alignment: shapes whose rows
 *    are not a multiple of 16 bytes take a slower guarded load path.
 *  - An output may not overlap any input (BG_ERR_ALIAS).
 *  - The current device must be gfx950 (BG_ERR_DEVICE). Kernels are compiled
 *    into the library; there is no runtime compilation.
 *  - Calls on different streams are thread-safe. A workspace must not be
 *    shared by calls that may run concurrently.
 */
#ifndef BLOCKGEMM_H
#define BLOCKGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bg_status {
    BG_OK = 0,
    BG_ERR_NULL = 1,      /* a required pointer is NULL                         */
    BG_ERR_SHAPE = 2,     /* dimensions invalid for this entry point            */
    BG_ERR_ALIGN = 3,     /* a base pointer is not 16-byte aligned              */
    BG_ERR_WORKSPACE = 4, /* workspace (or output rows) missing or too small    */
    BG_ERR_ALIAS = 5,     /* an output overlaps an input                        */
    BG_ERR_DEVICE = 6,    /* no current HIP device, or it is not gfx950         */
    BG_ERR_LAUNCH = 7     /* the HIP runtime rejected a kernel launch           */
} bg_status;

/*
 * gemm_bf16: C[M,N] = bf16( sum_k A[i,k] * B[j,k] ), FP32 accumulation.
 *
 * The plain BF16 matmul of the sm121a_matmul.py page (module docstring and
 * kernel: FP32 accumulator, K tail contributes zeros, cast to BF16 at the
 * masked store), in the A * B^T layout of the gemm_dense.rs page's dense BF16
 * GEMM. Summation order inside the FP32 accumulator is unspecified (MFMA).
 *
 *  A: [M, K] BF16, read only.   B: [N, K] BF16, read only.
 *  C: [M, N] BF16, written.     Dimensions: any M, N, K (M*K, N*K, M*N < 2^63).
 */
bg_status gemm_bf16(const uint16_t* A, const uint16_t* B, uint16_t* C,
                    uint32_t M, uint32_t N, uint32_t K, void* stream);

/*
 * gemm_bf16_dual: two products of the same activations in one launch,
 *   C0 = bf16(A * B0^T) and C1 = bf16(A * B1^T),
 * each exactly what gemm_bf16 returns for it (bit-identical: every output is
 * one tile's FP32 sum over K in the same order).
 *
 * sm121a_matmul.py page, module docstring: the MLP gate and up projections
 * are two GEMMs of one activation matrix with N = 11008 weights each (M =
 * 5120, K = 2048). Launched separately, each pays its own partly filled
 * last round of tiles on the 256 compute units; scheduled together their
 * tiles fill the rounds of one launch.
 *
 *  A: [M, K] BF16.  B0, B1: [N, K] BF16.  C0, C1: [M, N] BF16, written.
 *  Same shape rules, alignment and errors as gemm_bf16 for each pair; C0 and
 *  C1 must not overlap each other, A, B0 or B1 (BG_ERR_ALIAS).
 */
bg_status gemm_bf16_dual(const uint16_t* A, const uint16_t* B0, const uint16_t* B1, uint16_t* C0,
                         uint16_t* C1, uint32_t M, uint32_t N, uint32_t K, void* stream);

/*
 * gemm_bf16_strided: gemm_bf16 on operands and an output that are row ranges
 * of larger row-major buffers. Row i of A starts lda elements after row i-1,
 * row j of B ldb elements after row j-1, row i of C ldc elements after row
 * i-1; only the first K (A, B) or N (C) elements of each row are read or
 * written, and C's padding elements are left untouched.
 *
 * gemm_dense.rs page, doc comments of w4a16_gemm_n128_ldb and
 * w4a16_gemm_n128_m128_bf16_ldb: the weight rows are addressed through an
 * explicit row stride, so that padded or sub-matrix operands (the odd vocab
 * N of lm_head) are neither copied nor misaddressed. Strides that are not a
 * multiple of 8 elements (16 bytes) are legal and take a guarded
 * element-wise load path; they never fault.
 *
 *  lda >= K, ldb >= K, ldc >= N (BG_ERR_SHAPE otherwise); all at most 2^31-1.
 *  Base pointers 16-byte aligned (BG_ERR_ALIGN). C's spanned bytes
 *  [C, C + 2*((M-1)*ldc + N)) must not overlap A's or B's (BG_ERR_ALIAS).
 *  With lda = ldb = K and ldc = N this is exactly gemm_bf16.
 */
bg_status gemm_bf16_strided(const uint16_t* A, uint32_t lda, const uint16_t* B, uint32_t ldb,
                            uint16_t* C, uint32_t ldc, uint32_t M, uint32_t N, uint32_t K,
                            void* stream);

/*
 * gemm_bf16_scaled_acc: fused LoRA expand+fold, in place on `out`:
 *   out[i,j] = bf16( f32(out[i,j]) + fl32( scale * f32(bf16(delta[i,j])) ) ),
 *   delta = X * B^T accumulated in FP32.
 *
 * gemm_dense.rs page, doc comment of dense_gemm_tc_scaled_acc: the delta is
 * rounded to BF16 before the scale is applied, so the result is bit-identical
 * to writing bf16(X * B^T) to a scratch tensor and then running a BF16 scaled
 * add over it; fusing removes that scratch round trip. The multiply and the
 * add are separate FP32 operations (no FMA contraction).
 *
 *  X: [M, K] BF16.  B: [N, K] BF16.  out: [M, N] BF16, read and written.
 *  `out` must not overlap X or B.
 */
bg_status gemm_bf16_scaled_acc(const uint16_t* X, const uint16_t* B, uint16_t* out,
                               uint32_t M, uint32_t N, uint32_t K, float scale,
                               void* stream);

/*
 * gemm_bf16_splitk: C = bf16( sum_s P_s ), P_s[i,j] = FP32 partial sum of
 * A[i,k] * B[j,k] over K chunk s, planes added in ascending s in FP32.
 *
 * gemm_dense.rs page, dense_gemm_splitk: phase 1 writes k_splits partial
 * products into an FP32 workspace of k_splits * M * N * 4 bytes, phase 2
 * reduces them and writes BF16; both phases go on the same stream. Chunking
 * (the page leaves it open): chunk length Kc = ceil(K / k_splits) rounded up
 * to a multiple of 64; split s covers k in [s*Kc, min(K, (s+1)*Kc)); empty
 * chunks contribute +0. The reduction is deterministic (no atomics).
 *
 *  workspace: device FP32 buffer of at least
 *             gemm_bf16_splitk_workspace_bytes(M, N, k_splits) bytes, laid out
 *             as planes [k_splits][M][N]; on return (after the stream runs)
 *             plane s holds P_s. It may be NULL when k_splits == 1, in which
 *             case the result is computed without it and is bit-identical.
 *  k_splits:  1 .. 64 (BG_ERR_SHAPE otherwise).
 */
bg_status gemm_bf16_splitk(const uint16_t* A, const uint16_t* B, uint16_t* C,
                           float* workspace, size_t workspace_bytes,
                           uint32_t M, uint32_t N, uint32_t K, uint32_t k_splits,
                           void* stream);

/* Bytes of FP32 workspace gemm_bf16_splitk needs: k_splits * M * N * 4. */
size_t gemm_bf16_splitk_workspace_bytes(uint32_t M, uint32_t N, uint32_t k_splits);

/*
 * gemm_bf16_splitk_noalloc: gemm_bf16_splitk without a caller workspace and
 * without any allocation, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The FP32 planes go to a library-owned static device buffer of
 * BG_NOALLOC_SCRATCH_BYTES (32 MiB) that each device holds from the first
 * call on it until the process ends.
 *
 * Same result, chunking and reduction order as gemm_bf16_splitk (bit-identical
 * for the same arguments). Limit: k_splits * M * N * 4 <=
 * BG_NOALLOC_SCRATCH_BYTES, else BG_ERR_WORKSPACE (nothing is enqueued).
 * k_splits == 1 writes C directly and uses no scratch.
 *
 * Every call on one device shares that device's buffer, which keeps the last
 * call's planes: calls that may overlap on one device (other streams, other
 * threads) race on it and must be ordered by the caller. Nothing in the buffer
 * needs clearing: every plane element is written before the reduce reads it.
 * Other rules as gemm_bf16_splitk.
 */
#define BG_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
bg_status gemm_bf16_splitk_noalloc(const uint16_t* A, const uint16_t* B, uint16_t* C,
                                   uint32_t M, uint32_t N, uint32_t K, uint32_t k_splits,
                                   void* stream);

/*
 * gemm_bf16_streamk: C = bf16(A * B^T), FP32 accumulation, computed with a
 * stream-K schedule for problems whose tiles do not fill the compute units in
 * whole rounds (5120 x 512 x 2048: 160 tiles of 128 x 128 on 256 CUs).
 *
 * Prior art: the kernelbot NVFP4 GEMM page's persistent kernel (one program
 * per SM walking the tiles in a grouped order) and the gemm_dense.rs page's
 * dense_gemm_splitk (FP32 partial sums over K ranges combined into BF16).
 * Here one workgroup per compute unit takes an equal share of the problem's
 * (tile, 64-wide K step) pairs: the 8 XCDs each take a contiguous share of
 * the tiles in the grouped order, and the workgroups of an XCD split its
 * steps evenly, so a tile's steps may be spread over neighbouring workgroups.
 * A workgroup that runs the first steps of a tile without its last writes
 * the FP32 partial sum of its steps to its workspace slot; the workgroup that
 * runs the tile's last step adds those partials to its own sum in a fixed
 * order and stores the BF16 tile. The plan depends only on (M, N, K), the
 * tile configuration and the device's compute-unit count, so repeated calls
 * return identical bits. The FP32 sum is split differently from gemm_bf16's,
 * so the two agree to FP32 rounding, not bit for bit (exactly where every
 * partial sum is exact).
 *
 *  A: [M, K] BF16.  B: [N, K] BF16.  C: [M, N] BF16, written.
 *  workspace: device buffer of at least gemm_bf16_streamk_workspace(M, N, K)
 *             bytes (BG_ERR_WORKSPACE otherwise), 16-byte aligned, not
 *             overlapping A, B or C. It needs no initialization: the call
 *             marks each partial it publishes with a number unique to the
 *             call. Calls that may run concurrently need separate workspaces.
 *  K == 0, K not a multiple of 8, K >= 2^31 / 640 (beyond the kernel's
 *  32-bit operand offsets), or 2^30 or more 128 x 128 tiles or (tile, K step)
 *  pairs per XCD (beyond its 32-bit step ids): the data-parallel kernel of
 *  gemm_bf16 computes C (the same bits gemm_bf16 returns) and the workspace
 *  is unused (it may be NULL); otherwise a NULL workspace is BG_ERR_WORKSPACE.
 *  Other rules as gemm_bf16. The tile configuration is chosen from the shape
 *  (bg_tune_set(BG_TUNE_STREAMK_TILE, ...) overrides it); the workspace size
 *  depends on it, so query the size after any override.
 */
bg_status gemm_bf16_streamk(const uint16_t* A, const uint16_t* B, uint16_t* C,
                            void* workspace, size_t workspace_bytes,
                            uint32_t M, uint32_t N, uint32_t K, void* stream);

/* Bytes of workspace gemm_bf16_streamk needs for (M, N, K) on the current
 * device (one partial tile and one 8-byte flag per workgroup, one workgroup
 * per compute unit), in *bytes. BG_ERR_DEVICE without a gfx950 device. */
bg_status gemm_bf16_streamk_workspace(uint32_t M, uint32_t N, uint32_t K, size_t* bytes);

/*
 * bg_streamk_plan: the stream-K plan as the kernel computes it (the same host
 * and device code), for `tiles` output tiles of `steps` K steps each and
 * `wgs_per_xcd` workgroups on each of the 8 XCDs (workgroup b = u * 8 + x
 * runs on XCD x). Writes one row of 6 int32 per piece of work, workgroups in
 * ascending b, each workgroup's pieces in the order it runs them:
 *   b, grid tile index (grouped order), first step, end step (within the
 *   tile), 1 if the piece is published as a partial else 0, and for a tile
 *   whose earlier steps other workgroups ran, the lowest such workgroup's u
 *   (the sources are u' = that .. u-1 on the same XCD), else -1.
 * *n_rows receives the number of pieces; rows may be NULL to count only, else
 * it holds max_rows rows (BG_ERR_WORKSPACE if fewer than needed). Host only.
 */
bg_status bg_streamk_plan(uint32_t tiles, uint32_t steps, uint32_t wgs_per_xcd, int32_t* rows,
                          size_t max_rows, size_t* n_rows);

/*
 * gemm_bf16_ordered: order-preserving GEMM for router logits.
 *   acc = +0.0f; for k = 0, 1, ..., K-1: acc = fl32(acc + fl32(A[i,k] * B[j,k]));
 *   C[i,j] = bf16(acc).
 *
 * gemm_dense.rs page, doc comment of dense_gemm_router: same math and the
 * same strict k = 0..K-1 per-output FP32 order as the scalar dense kernel,
 * built without FMA contraction, so the output is bit-identical to it; matrix
 * cores reassociate and are not used. Computed with FP32 vector ALU only.
 *
 *  A: [M, K] BF16.  B: [N, K] BF16.  C: [M, N] BF16.
 */
bg_status gemm_bf16_ordered(const uint16_t* A, const uint16_t* B, uint16_t* C,
                            uint32_t M, uint32_t N, uint32_t K, void* stream);

/*
 * gemm_bf16_ordered_f32: as gemm_bf16_ordered but stores the FP32 sums
 * (C32: [M, N] float) instead of rounding them to BF16. Same kernel, same
 * order; exists so tests can compare the accumulator bit for bit.
 */
bg_status gemm_bf16_ordered_f32(const uint16_t* A, const uint16_t* B, float* C32,
                                uint32_t M, uint32_t N, uint32_t K, void* stream);

/*
 * gemm_fp4_blockscaled: C[i,j] = bf16( sum_k a[i,k] * b[j,k] ), FP32 accumulation,
 *   a[i,k] = e2m1(A nibble [i,k]) * e4m3fn(SFA[i, k/16]),
 *   b[j,k] = e2m1(B nibble [j,k]) * e4m3fn(SFB[j, k/16]).
 *
 * kernelbot NVFP4 GEMM page (submission 123329): the "SCALE FACTORS" loop
 * (one scale per 16 K elements, plain [rows, K/16] layout) applied to both
 * operands, followed by a block-scaled dot product with FP32 accumulation.
 * Each dequantized element is exact in FP16 (at most 6 significant bits,
 * magnitude 2^-10..2688) and is fed to FP16 matrix cores.
 *
 *  A:   [M, K/2] bytes, two E2M1 codes per byte, element 2t in the LOW nibble
 *       of byte t (sign bit 3, exponent bits 2..1, mantissa bit 0).
 *  SFA: [M, K/16] E4M3FN bytes (bias 7, 0x7F/0xFF = NaN), row-major.
 *  B:   [N, K/2] bytes; SFB: [N, K/16] bytes; same encodings.
 *  C:   [M, N] BF16, written.
 *  K must be a multiple of 16 (BG_ERR_SHAPE otherwise).
 */
bg_status gemm_fp4_blockscaled(const uint8_t* A, const uint8_t* SFA,
                               const uint8_t* B, const uint8_t* SFB, uint16_t* C,
                               uint32_t M, uint32_t N, uint32_t K, void* stream);

/*
 * gemm_fp4_blockscaled_batched: L independent gemm_fp4_blockscaled problems
 * of one shape, stored one after another (problem l of A at A + l*M*K/2, of
 * SFA at SFA + l*M*K/16, of B and SFB likewise with N, of C at C + l*M*N).
 *
 * kernelbot NVFP4 GEMM page, custom_kernel docstring: a, b, the scales and c
 * carry a batch dimension l, and the tensors are allocated l-major. The
 * page's kernel asserts L == 1; the method does not need it.
 *
 *  L <= 65535 (BG_ERR_SHAPE otherwise); L == 0 is a no-op. Other rules as
 *  gemm_fp4_blockscaled, over all L problems' bytes.
 */
bg_status gemm_fp4_blockscaled_batched(const uint8_t* A, const uint8_t* SFA,
                                       const uint8_t* B, const uint8_t* SFB, uint16_t* C,
                                       uint32_t M, uint32_t N, uint32_t K, uint32_t L,
                                       void* stream);

/*
 * gemm_fp4_blockscaled_splitk: gemm_fp4_blockscaled through k_splits FP32
 * partial planes, for shapes with few output tiles (the kernelbot page's
 * decode-sized problems, M = 128).
 *
 *  Phase 1: workspace[s][i][j] = FP32 sum of deq(A)[i,k]*deq(B)[j,k] over
 *           chunk s of K, chunks of ceil(K/k_splits) rounded up to 64.
 *  Phase 2: C = bf16( ((ws[0] + ws[1]) + ...) ), planes added in ascending s.
 *
 * The split is gemm_dense.rs's dense_gemm_splitk (FP32 workspace of
 * k_splits*M*N*4 bytes, then a BF16 reduce) applied to the block-scaled
 * product. workspace_bytes >= k_splits*M*N*4 (gemm_bf16_splitk_workspace_bytes
 * gives it) unless k_splits == 1, which writes C directly and ignores the
 * workspace. 1 <= k_splits <= 64.
 */
bg_status gemm_fp4_blockscaled_splitk(const uint8_t* A, const uint8_t* SFA,
                                      const uint8_t* B, const uint8_t* SFB, uint16_t* C,
                                      float* workspace, size_t workspace_bytes,
                                      uint32_t M, uint32_t N, uint32_t K, uint32_t k_splits,
                                      void* stream);

/*
 * fp4_scales_from_blocked: plain [L, rows, k_groups] E4M3 scale bytes (the
 * layout every FP4 entry point here takes) from NVIDIA's blocked hardware
 * layout.
 *
 * kernelbot NVFP4 GEMM page, "SCALE FACTORS": the blocked tensor has shape
 * [32, 4, rest_m, 4, rest_k, L] (dims g_m, i_m, tile_m, i_k, tile_k, l) and is
 * stored in the order (l, tile_m, tile_k, g_m, i_m, i_k): 512-byte blocks of
 * 128 rows x 4 groups. Plain row = tile_m*128 + i_m*32 + g_m, group =
 * tile_k*4 + i_k.
 *
 *  blocked: batch*rows*k_groups bytes in that order (read).
 *  plain:   [batch, rows, k_groups] bytes (written); must not overlap blocked.
 *  rows % 128 == 0 and k_groups % 4 == 0 (BG_ERR_SHAPE otherwise).
 */
bg_status fp4_scales_from_blocked(const uint8_t* blocked, uint8_t* plain, uint32_t rows,
                                  uint32_t k_groups, uint32_t batch, void* stream);

/*
 * gemm_w4a16: C[i,j] = bf16( fl32( s2 * sum_k A[i,k] * w[j,k] ) ), FP32
 *   accumulation, w[j,k] = e2m1(B nibble [j,k]) * e4m3fn(SFB[j, k/16]),
 *   s2 = scale_2.
 *
 * gemm_dense.rs page, doc comments of w4a16_gemm and its lossless BF16-MMA
 * variant: BF16 activations times NVFP4 weights (E2M1 values, one FP8 E4M3
 * scale per 16 K elements, one FP32 per-tensor scale). Each weight is
 * dequantized exactly (it is exact in BF16) and fed with A to BF16 matrix
 * cores; the per-tensor scale multiplies the FP32 dot product once, before
 * the BF16 rounding of C.
 *
 *  A:   [M, K] BF16 activations, row-major.
 *  B:   [N, K/2] bytes, two E2M1 codes per byte, element 2t in the LOW nibble
 *       of byte t (the weight rows, K contiguous).
 *  SFB: [N, K/16] E4M3FN bytes.
 *  scale_2: the per-tensor FP32 weight scale (any finite value).
 *  C:   [M, N] BF16, written.
 *  K must be a multiple of 16 (BG_ERR_SHAPE otherwise); C must not overlap
 *  A, B or SFB (BG_ERR_ALIAS).
 */
bg_status gemm_w4a16(const uint16_t* A, const uint8_t* B, const uint8_t* SFB, float scale_2,
                     uint16_t* C, uint32_t M, uint32_t N, uint32_t K, void* stream);

/*
 * gemm_w4a16_t: gemm_w4a16 with the weights in the transposed layout and an
 * explicit row stride, for weight matrices whose N is not a multiple of 16
 * (the vocabulary-sized lm_head).
 *
 * gemm_dense.rs page, doc comments of w4a16_gemm_n128_ldb and
 * w4a16_gemm_n128_m128_bf16_ldb: the transposed weight is addressed through
 * a row stride; with the odd vocabulary size 248077 as the stride, most rows
 * start off a 16-byte boundary and 16-byte loads fault, so the page pads the
 * stride to a multiple of 128 with zero-filled columns. Here any ldb >= N is
 * accepted: ldb % 4 == 0 takes 4-byte column loads, any other stride byte
 * loads; neither faults.
 *
 *  A:    [M, K] BF16 activations.
 *  Bt:   [K/2, ldb] bytes: byte (r, n) holds weight row n's E2M1 codes for
 *        k = 2r (LOW nibble) and k = 2r + 1 (high nibble); columns N..ldb-1
 *        are padding (read, never used). The whole (K/2) * ldb bytes must be
 *        readable.
 *  SFBt: [K/16, ldb] E4M3FN bytes: byte (g, n) scales k in [16g, 16g + 16) of
 *        weight row n (the scale tensor transposed with the same stride).
 *  C:    [M, N] BF16, C[i,j] = bf16(fl32(s2 * sum_k A[i,k] * w[j,k])) exactly
 *        as gemm_w4a16 with the same weights in its [N, K/2] layout.
 *  K % 16 == 0 and N <= ldb <= 2^31 - 1 (BG_ERR_SHAPE otherwise); C must not
 *  overlap A, Bt or SFBt (BG_ERR_ALIAS).
 */
bg_status gemm_w4a16_t(const uint16_t* A, const uint8_t* Bt, const uint8_t* SFBt, uint32_t ldb, float scale_2,
                       uint16_t* C, uint32_t M, uint32_t N, uint32_t K, void* stream);

/*
 * bf16_scaled_add: out[i] = bf16( f32(out[i]) + fl32(scale * f32(delta[i])) )
 * over `count` BF16 elements. The second half of the unfused LoRA fold that
 * gemm_bf16_scaled_acc must equal bit for bit (gemm_dense.rs page, doc comment
 * of dense_gemm_tc_scaled_acc); kept so the identity can be tested on the GPU.
 */
bg_status bf16_scaled_add(uint16_t* out, const uint16_t* delta, size_t count,
                          float scale, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* bg_status_string(bg_status status);

/*
 * Tuning overrides: each key names one automatic choice the library makes
 * per call. bg_tune_set(key, v) with v >= 0 forces that choice for every
 * later call in the process (any device, any thread); v = -1, the initial
 * state, restores the automatic choice. Nothing is read from the
 * environment. Meant for tests that must cover every tile configuration and
 * for tile sweeps; a forced choice changes speed only, never the promised
 * result (bit-identical where an entry point promises it, within the FP32
 * summation-order tolerance otherwise).
 *
 *  BG_TUNE_TILE:       dense tile configuration (gemm_bf16 and the entry
 *                      points built on it: dual, strided, scaled_acc,
 *                      split-K planes), an index into the library's tile table
 *  BG_TUNE_COLSPLIT:   0 turns the column split of gemm_bf16 off
 *  BG_TUNE_ORDERED:    variant of gemm_bf16_ordered (0-11 register blocks of
 *                      the tile form, 12-14 the scalar-A form with 1-3 rows
 *                      per wave, which needs K % 8 == 0: other K take the
 *                      tile form's 2 x 1 block)
 *  BG_TUNE_FP4_TILE:   tile of gemm_fp4_blockscaled(_batched) (10, 11: the
 *                      decode kernel with four or eight waves, one problem
 *                      with K % 64 == 0)
 *  BG_TUNE_FP4_SPLITK_TILE: tile of gemm_fp4_blockscaled_splitk's planes (7, 8:
 *                      the decode kernel with four or eight waves and 256
 *                      columns, 9: eight waves and 128 columns; K % 64 == 0)
 *  BG_TUNE_W4A16_TILE: tile of gemm_w4a16
 *  BG_TUNE_STREAMK_TILE: tile of gemm_bf16_streamk (23: 128 x 128, 10: 256 x 128;
 *                      other values select 128 x 128)
 * Returns BG_ERR_SHAPE for an unknown key or v < -1; an index past a table
 * selects that table's default entry.
 */
typedef enum bg_tune_key {
    BG_TUNE_TILE = 0,
    BG_TUNE_COLSPLIT = 1,
    BG_TUNE_ORDERED = 2,
    BG_TUNE_FP4_TILE = 3,
    BG_TUNE_FP4_SPLITK_TILE = 4,
    BG_TUNE_W4A16_TILE = 5,
    BG_TUNE_STREAMK_TILE = 6,
    BG_TUNE_COUNT = 7
} bg_tune_key;

bg_status bg_tune_set(int key, int value);

/* The current override of `key` (-1: automatic; also -1 for an unknown key). */
int bg_tune_get(int key);

/*
 * bg_tile_map: the workgroup -> output tile mapping of the GEMM kernels,
 * evaluated on the host by the same code the kernels run (no device needed).
 * For every workgroup b of a tiles_m x tiles_n grid it writes the tile row
 * tm[b] and tile column tn[b]; each mapping is a bijection onto the grid.
 *
 *  order 0: the GEMM kernels (the sm121a_matmul.py page's grouped program
 *           order, 4 tile-rows per group, applied to ids renumbered so each
 *           of the 8 XCDs holds one contiguous range);
 *  order 1: the LoRA fold (grouped order on the raw dispatch index);
 *  order 2: the order-preserving kernel (XCD-contiguous ids, row-major).
 *  tm, tn: host arrays of tiles_m * tiles_n int32 each.
 * BG_ERR_SHAPE for another order or tiles_m * tiles_n >= 2^31; BG_ERR_NULL
 * for a NULL array of a non-empty grid.
 */
bg_status bg_tile_map(int order, uint32_t tiles_m, uint32_t tiles_n, int32_t* tm, int32_t* tn);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKGEMM_H */
