// Work plan of the stream-K GEMM: which K steps of which output tiles each
// workgroup computes, who stores each tile, and whose partial sums it adds.
// Host and device share this code: the kernel calls it with blockIdx.x, and
// the library's bg_streamk_plan export runs the very same functions on
// the host, so tests can check on the CPU that the plan covers every K step
// of every tile exactly once and that every wait is on a workgroup that
// publishes without waiting.
//
// Prior art: the kernelbot NVFP4 GEMM page's persistent tile loop (one
// program per SM walking linear tile ids) and the gemm_dense.rs page's
// dense_gemm_splitk (FP32 partial sums combined after the K loop). Here the
// unit of work is one 64-wide K step of one tile, the steps are dealt out
// evenly instead of whole tiles, and the split is MI355X-specific: each of
// the 8 XCDs (workgroup b runs on XCD b % 8) takes a contiguous share of the
// tiles, and its workgroups split that share's steps among themselves, so
// the partial sums a tile needs come from workgroups on the same XCD.
//
//   tiles of XCD x         [t0, t0 + nt), in the grouped tile order
//   steps of XCD x         nt * S   (S = K steps per tile, local ids)
//   workgroup u of XCD x   steps [u*I/A, (u+1)*I/A) with I = nt * S and
//                          A = min(W, I) active workgroups (the others idle)
//
// A workgroup's range ends in at most one unfinished tile: it computes that
// head or middle piece FIRST and publishes it as an FP32 partial. It then
// stores every tile whose last step lies in its range, the first of them
// (possibly begun by lower workgroups) last: that one adds the partials of
// the workgroups u_a .. u-1 whose ranges hold its earlier steps. Every wait
// is on a lower-numbered workgroup of the same XCD, whose partial is its
// first piece of work and needs no wait.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bg {

constexpr int SK_XCDS = 8;

// Tiles [t0, t0 + nt) of XCD x: an even split, the first tiles % 8 XCDs one more.
__host__ __device__ inline void sk_xcd_tiles(int tiles, int x, int& t0, int& nt) {
    const int per = tiles / SK_XCDS, rem = tiles % SK_XCDS;
    nt = per + (x < rem ? 1 : 0);
    t0 = x * per + (x < rem ? x : rem);
}

// First step of active workgroup u (0 <= u <= active) of a share of `iters` steps.
__host__ __device__ inline int sk_start(int iters, int active, int u) {
    return (int)(((int64_t)u * iters) / active);
}

// The active workgroup whose range holds step i (0 <= i < iters): the largest
// u with sk_start(u) <= i.
__host__ __device__ inline int sk_wg_of(int iters, int active, int i) {
    return (int)((((int64_t)i + 1) * active - 1) / iters);
}

// One piece of a workgroup's work: K steps [s_begin, s_end) of local tile t
// (0-based within the XCD's share), as step ids relative to the tile.
struct SkPiece {
    int tile;          // local tile index; the grid tile is t0 + tile
    int s_begin, s_end;
    int partial;       // 1: unfinished tile, published as an FP32 partial
    int src_first;     // owner of a tile begun below: sources src_first .. u-1; else -1
};

// Workgroup (x, u)'s plan: the number of pieces (0 when idle) and piece q in
// processing order (q = 0 .. count-1).
struct SkWorkgroup {
    int t0, nt, iters, active;
    int s, e;          // local step range
    int steps;         // K steps per tile
    int has_partial, n_owned;

    __host__ __device__ void init(int tiles, int steps_per_tile, int wgs_per_xcd, int x, int u) {
        steps = steps_per_tile;
        sk_xcd_tiles(tiles, x, t0, nt);
        iters = nt * steps;
        active = iters < wgs_per_xcd ? iters : wgs_per_xcd;
        if (u >= active || iters == 0) {
            s = e = 0;
            has_partial = n_owned = 0;
            return;
        }
        s = sk_start(iters, active, u);
        e = sk_start(iters, active, u + 1);
        has_partial = (e % steps) != 0;
        n_owned = e / steps - s / steps;
    }
    __host__ __device__ int count() const { return has_partial + n_owned; }

    __host__ __device__ SkPiece piece(int q) const {
        SkPiece pc;
        if (has_partial && q == 0) {
            pc.tile = e / steps;
            const int first = pc.tile * steps;
            pc.s_begin = (s > first ? s : first) - first;
            pc.s_end = e - first;
            pc.partial = 1;
            pc.src_first = -1;
            return pc;
        }
        // owned tiles from the last to the first, so the one begun below
        // (the only one that waits) comes last
        const int k = q - has_partial;
        pc.tile = e / steps - 1 - k;
        const int first = pc.tile * steps;
        pc.s_begin = (s > first ? s : first) - first;
        pc.s_end = steps;
        pc.partial = 0;
        pc.src_first = s > first ? sk_wg_of(iters, active, first) : -1;
        return pc;
    }
};

// K element offset of step j of a tile (0 <= j <= steps): the first step is
// the ragged one when K is not a multiple of 64 (the main loop takes a
// ragged remainder as its first step).
__host__ __device__ inline int sk_kpos(int j, int K, int steps) {
    if (j <= 0) return 0;
    const int r = K - (steps - 1) * 64;   // 1 .. 64
    const int k = r + (j - 1) * 64;
    return k < K ? k : K;
}

// ---------------------------------------------------------------------------
// Host side: the tile configuration of a call and the workspace it needs.
// ---------------------------------------------------------------------------

// Tile choices. Every workgroup runs about the same number of K steps, so
// the estimate is the busiest workgroup's steps x the step's flops at the
// tile's rate with one workgroup per CU, plus a fixed cost per piece of work
// (pipeline fill and epilogue) and, when tiles are split, the partial-tile
// exchange (it grows with the partial's bytes). Rates and costs were measured
// on MI355X with the stream-K kernel itself (5120 x 512 x 2048, 5120 x 2048 x
// 2048 and 5120 x 2048 x 11008). Both tiles hold one workgroup per CU. Wider
// tiles (160 x 256, 256 x 256) do not keep their partial and fix-up epilogues
// beside the piece loop in registers (scratch spills), so they are not
// offered.
struct SkChoice {
    int cfg, bm, bn;
    double rate1;   // TFLOP/s on the whole chip
};
constexpr SkChoice kSkChoices[] = {
    {23, 128, 128, 763.0},
    {10, 256, 128, 1130.0},
};
constexpr double kSkPieceUs = 2.0;          // per piece of work
constexpr double kSkExchangeUsPerKB = 0.2;  // per KB of partial tile

inline double sk_us(const SkChoice& c, int64_t M, int64_t N, int64_t K, int cus) {
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const int64_t steps = (K + 63) / 64;
    if (tiles == 0 || steps == 0) return 0.0;   // empty: nothing to run
    const int64_t w = cus / SK_XCDS > 0 ? cus / SK_XCDS : 1;
    const int64_t share = (tiles + SK_XCDS - 1) / SK_XCDS * steps;
    const int64_t per_wg = (share + w - 1) / w;
    const bool split = share % w != 0 || per_wg % steps != 0;
    const double pieces = (double)((per_wg + steps - 1) / steps) + (split ? 1.0 : 0.0);
    return (double)per_wg * 2.0 * c.bm * c.bn * 64 * cus / (c.rate1 * 1e6) + pieces * kSkPieceUs +
           (split ? kSkExchangeUsPerKB * c.bm * c.bn * 4 / 1024.0 : 0.0);
}

// Workgroups per XCD on a device of `cus` compute units (one per CU).
inline int sk_wgs_per_xcd(uint32_t cus) {
    const int c = cus > 0 ? (int)cus : 256;
    return c / SK_XCDS > 0 ? c / SK_XCDS : 1;
}

// The tile configuration (`forced` >= 0 picks that table entry, the first
// when none matches) and the workspace bytes: one BM x BN FP32 partial and
// one 8-byte flag per workgroup.
inline int streamk_choose(uint32_t M, uint32_t N, uint32_t K, uint32_t cus, int forced, size_t* ws_bytes) {
    const SkChoice* pick = &kSkChoices[0];
    if (forced >= 0) {
        for (const SkChoice& ch : kSkChoices)
            if (ch.cfg == forced) pick = &ch;
    } else {
        double best = 1e300;
        for (const SkChoice& ch : kSkChoices) {
            const double t = sk_us(ch, M, N, K, cus > 0 ? (int)cus : 256);
            if (t < best) {
                best = t;
                pick = &ch;
            }
        }
    }
    const uint64_t grid = (uint64_t)SK_XCDS * sk_wgs_per_xcd(cus);
    *ws_bytes = (size_t)(grid * ((uint64_t)pick->bm * pick->bn * 4 + 8));
    return pick->cfg;
}

// Whether the stream-K kernel takes the shape: the direct loads' 16-byte
// rows and 32-bit buffer offsets, and int32 step ids (counted for the
// smallest tile, which has the most tiles).
inline bool streamk_applies(uint32_t M, uint32_t N, uint32_t K) {
    const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
    const int64_t steps = ((int64_t)K + 63) / 64;
    return K > 0 && (K % 8) == 0 && (int64_t)K * 640 < (int64_t(1) << 31) && tiles < (int64_t(1) << 30) &&
           (tiles + SK_XCDS - 1) / SK_XCDS * steps < (int64_t(1) << 30);
}

}  // namespace bg
