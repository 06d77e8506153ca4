"""Workgroup -> tile mappings of the GEMM kernels, run on the host through the
library's bg_tile_map export (the same functions the kernels call): each must
be a bijection onto the tile grid for every grid the tests and the benchmark
launch, including grids whose tile-row count is not a multiple of the group
size and whose workgroup count is not a multiple of the 8 XCDs."""
import numpy as np
import pytest

import block_scaled_fp4_gemm_amd as bg


def tiles(m, n, bm, bn, dual=False):
    return -(-m // bm), -(-n // bn) * (2 if dual else 1)


GRIDS = sorted(set([
    # benchmark rows
    tiles(5120, 11008, 256, 256, dual=True),     # gate+up dual call: 20 x 86
    tiles(5120, 9472, 256, 256), tiles(5120, 1536, 256, 128),   # gate/up column split
    tiles(5120, 2048, 160, 256),                 # down and Q/O
    tiles(5120, 512, 96, 128),                   # K/V
    tiles(5120, 512, 128, 128),                  # K/V, the previous tile
    tiles(2048, 17408, 64, 128),                 # LoRA fold
    tiles(4096, 4096, 256, 256),                 # FP4
    tiles(128, 7168, 128, 256), tiles(128, 4096, 128, 256),   # FP4 decode
    tiles(1016, 12288, 128, 384),                # W4A16
    tiles(4510, 256, 32, 32), tiles(2255, 256, 32, 16),       # router register blocks
    tiles(128, 256, 128, 128),                   # small dense
    # edge counts
    (1, 1), (1, 7), (7, 1), (3, 5), (5, 3), (9, 13), (13, 9), (4, 2), (17, 1), (2, 33), (6, 86),
    (41, 41), (1, 255), (255, 1), (33, 65),
]))


@pytest.mark.parametrize("order", [0, 1, 2])
@pytest.mark.parametrize("tm_,tn_", GRIDS)
def test_every_tile_exactly_once(order, tm_, tn_):
    tm, tn = bg.tile_map(order, tm_, tn_)
    assert (tm >= 0).all() and (tm < tm_).all() and (tn >= 0).all() and (tn < tn_).all()
    ids = tm.astype(np.int64) * tn_ + tn
    assert np.array_equal(np.sort(ids), np.arange(tm_ * tn_))


def test_grouped_order_walks_four_tile_rows_m_fastest():
    # fold order (no renumbering): workgroups 0..3 take tile rows 0..3 of column 0
    tm, tn = bg.tile_map(1, 10, 5)
    assert list(zip(tm[:6], tn[:6])) == [(0, 0), (1, 0), (2, 0), (3, 0), (0, 1), (1, 1)]
    # the last group has 10 % 4 = 2 tile rows
    assert list(zip(tm[40:44], tn[40:44])) == [(8, 0), (9, 0), (8, 1), (9, 1)]


def test_xcd_renumbering_gives_each_xcd_a_contiguous_range():
    # 20 workgroups on 8 XCDs: XCD x runs workgroups x, x+8, x+16; the first
    # 4 XCDs hold 3 ids, the rest 2, and each XCD's ids are consecutive
    tm, tn = bg.tile_map(2, 4, 5)
    logical = tm * 5 + tn
    for x in range(8):
        ids = logical[x::8]
        assert (np.diff(ids) == 1).all()
    assert sorted(logical[0::8]) == [0, 1, 2]


def test_bad_orders_and_sizes():
    with pytest.raises(bg.BlockGemmError):
        bg.tile_map(3, 2, 2)
    with pytest.raises(bg.BlockGemmError):
        bg.tile_map(0, 1 << 16, 1 << 15)
    tm, tn = bg.tile_map(0, 0, 5)
    assert tm.size == 0
