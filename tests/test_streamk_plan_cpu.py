"""The stream-K plan (bg_streamk_plan: the same host-and-device code the
kernel runs) checked on the CPU for every grid the GPU tests and the
benchmark launch, and for degenerate ones: every K step of every tile is
computed exactly once, each tile is stored by exactly one workgroup, and every
wait is on a lower-numbered workgroup of the same XCD whose first piece of
work is the partial it waits for (so no wait depends on another wait, and a
workgroup never waits on one dispatched after it)."""
import collections

import pytest

import block_scaled_fp4_gemm_amd as bg

XCDS = 8


def _tiles(m, n, bm, bn):
    return -(-m // bm) * -(-n // bn)


# (tiles, steps, workgroups per XCD): the GPU tests' shapes for both tiles on
# 256 CUs, the benchmark's attention and MLP shapes, and degenerate grids
GRIDS = sorted({
    *((_tiles(m, n, bm, bn), -(-k // 64), 32)
      for m, n, k in [(5120, 512, 2048), (5120, 2048, 2048), (5120, 2048, 11008), (5120, 11008, 2048),
                      (1, 1, 8), (65, 129, 72), (300, 200, 1000), (257, 255, 1040), (130, 1001, 256),
                      (1000, 700, 4096), (64, 64, 6400), (33, 17, 528), (2048, 2048, 64)]
      for bm, bn in [(128, 128), (256, 128)]),
    (1, 1, 1), (1, 1, 32), (7, 1, 32), (8, 1, 32), (9, 3, 32), (3, 100, 1), (17, 33, 5), (160, 32, 31),
    (1720, 32, 32), (5, 7, 3), (8, 4, 32), (100, 1, 32),
})


@pytest.mark.parametrize("tiles,steps,w", GRIDS)
def test_plan_covers_every_step_once_and_waits_are_safe(tiles, steps, w):
    rows = bg.streamk_plan(tiles, steps, w)
    assert rows.ndim == 2 and rows.shape[1] == 6
    by_wg = collections.defaultdict(list)
    for r in rows:
        by_wg[int(r[0])].append(tuple(int(v) for v in r[1:]))
    assert all(0 <= b < XCDS * w for b in by_wg), "workgroup index outside the grid"

    covered = collections.defaultdict(list)    # tile -> [(begin, end, b, partial)]
    for b, pieces in by_wg.items():
        partials = [i for i, p in enumerate(pieces) if p[3] == 1]
        assert partials in ([], [0]), f"wg {b}: a partial must be its single first piece"
        waits = [i for i, p in enumerate(pieces) if p[4] >= 0]
        assert waits in ([], [len(pieces) - 1]), f"wg {b}: only its last piece may wait"
        for t, s0, s1, part, src in pieces:
            assert 0 <= t < tiles and 0 <= s0 < s1 <= steps
            assert (s1 < steps) == (part == 1), "a piece is published exactly when it ends before the tile"
            covered[t].append((s0, s1, b, part))
    assert sorted(covered) == list(range(tiles)), "every tile has pieces"
    for t, pcs in covered.items():
        pcs.sort()
        assert pcs[0][0] == 0 and pcs[-1][1] == steps
        assert all(a[1] == b[0] for a, b in zip(pcs, pcs[1:])), f"tile {t}: steps missing or computed twice"
        owners = [p for p in pcs if p[3] == 0]
        assert len(owners) == 1 and owners[0] is pcs[-1], f"tile {t}: one store, by the last steps' workgroup"
        # the pieces of one tile come from consecutive workgroups of one XCD, in K order
        wgs = [p[2] for p in pcs]
        assert len({b % XCDS for b in wgs}) == 1
        assert [b // XCDS for b in wgs] == list(range(wgs[0] // XCDS, wgs[0] // XCDS + len(wgs)))

    for b, pieces in by_wg.items():
        t, s0, s1, part, src = pieces[-1]
        if src < 0:
            assert part == 1 or s0 == 0, "a stored tile that starts mid-way must name its sources"
            continue
        x, u = b % XCDS, b // XCDS
        assert 0 <= src < u, "sources are lower-numbered workgroups"
        for su in range(src, u):
            first = by_wg[su * XCDS + x][0]
            assert first[0] == t and first[3] == 1, "each source publishes this tile as its first piece"
        assert by_wg[src * XCDS + x][0][1] == 0, "the lowest source holds the tile's first step"


@pytest.mark.parametrize("tiles,steps,w", [(160, 32, 32), (1720, 32, 32), (80, 32, 32), (13, 7, 32)])
def test_plan_balances_steps_within_one_per_xcd(tiles, steps, w):
    rows = bg.streamk_plan(tiles, steps, w)
    load = collections.Counter()
    for r in rows:
        load[int(r[0])] += int(r[3]) - int(r[2])
    for x in range(XCDS):
        per = [load.get(u * XCDS + x, 0) for u in range(w)]
        active = [v for v in per if v > 0]
        if active:
            assert max(active) - min(active) <= 1
        assert sum(per) == (tiles // XCDS + (x < tiles % XCDS)) * steps


def test_attention_kv_plan_shape():
    """5120 x 512 x 2048 with 128 x 128 tiles: 160 tiles of 32 steps, 20 per
    XCD, 20 steps per workgroup on 256 CUs."""
    rows = bg.streamk_plan(160, 32, 32)
    load = collections.Counter()
    for r in rows:
        load[int(r[0])] += int(r[3]) - int(r[2])
    assert set(load.values()) == {20} and len(load) == 256
    assert sum(1 for r in rows if r[4] == 1) == 224   # published partials
    assert sum(1 for r in rows if r[4] == 0) == 160   # one store per tile


def test_plan_rejects_bad_arguments():
    with pytest.raises(bg.BlockGemmError):
        bg.streamk_plan(4, 4, 0)
    with pytest.raises(bg.BlockGemmError):
        bg.streamk_plan(1 << 30, 1, 32)
    assert bg.streamk_plan(0, 5, 32).shape == (0, 6)
    assert bg.streamk_plan(5, 0, 32).shape == (0, 6)
