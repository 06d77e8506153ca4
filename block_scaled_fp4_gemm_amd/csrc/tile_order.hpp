// Workgroup -> output tile mappings of the GEMM kernels. Host and device
// share this code: the kernels call it with blockIdx.x, and the library's
// bg_tile_map export runs the very same functions on the host so that tests
// can check each mapping is a bijection onto the tile grid.
//
// The grouped order follows the sm121a_matmul.py page's kernel (program ids
// walk GROUP_M tile-rows at a time, m fastest, so the tiles that run together
// share B columns in L2). The XCD renumbering is MI355X-specific: dispatch
// places workgroup b of a grid on XCD b % 8, and each XCD has its own L2.
#pragma once

#include <hip/hip_runtime.h>

namespace bg {

// tile-rows per group in the grouped order. With 32 CUs per XCD, 4 gives the
// concurrent tiles of an XCD a 4 x 8 block (4 A panels, 8 B panels): measured
// against 2, 3, 5, 6, 8 and 16 on the MLP and attention shapes, 4 ran the
// gate+up dual call 1.6% and Q/O 5.4% faster than 8, other rows within 2%.
constexpr int GROUP_M = 4;

// Workgroup b of an n-workgroup grid -> a logical id such that each of the 8
// XCDs holds one contiguous range of ids (the first n % 8 XCDs one more).
__host__ __device__ inline int xcd_order(int b, int n) {
    const int per = n >> 3, rem = n & 7;
    const int x = b & 7, j = b >> 3;
    return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + j;
}

// Logical tile id -> (tile_m, tile_n) in grouped order: GROUP_M tile-rows at
// a time (the last group may be shorter), m fastest inside a group.
__host__ __device__ inline void grouped_tile(int logical, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int width = GROUP_M * tiles_n;
    const int g = logical / width;
    const int first_m = g * GROUP_M;
    const int gsize = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
    const int r = logical - g * width;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

// Tile orders of the kernels (compile-time; bg_tile_map's `order` argument
// selects the same instances on the host):
//   ORDER_GEMM (0): XCD-contiguous ids, then grouped: workgroups that share an
//      XCD share operand panels in its L2;
//   ORDER_FOLD (1): grouped on the raw dispatch index: adjacent tiles of the
//      fold's `out` stream on different XCDs at the same time;
//   ORDER_ROWS (2): XCD-contiguous ids, row-major tiles (the order-preserving
//      kernel: the column tiles of a row block share its A rows in one L2).
enum TileOrder : int { ORDER_GEMM = 0, ORDER_FOLD = 1, ORDER_ROWS = 2 };

template <int ORDER>
__host__ __device__ inline void tile_of(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
    if constexpr (ORDER == ORDER_FOLD) {
        grouped_tile(b, tiles_m, tiles_n, tm, tn);
    } else if constexpr (ORDER == ORDER_ROWS) {
        const int l = xcd_order(b, tiles_m * tiles_n);
        tm = l / tiles_n;
        tn = l % tiles_n;
    } else {
        grouped_tile(xcd_order(b, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
    }
}

}  // namespace bg
