"""GPU parity of the block-scaled FP4 GEMM."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
import synthetic
from gpu_util import assert_bits_equal, bits_of, check_close, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu


def _run(a, sfa, b, sfb):
    c = bg.gemm_fp4_blockscaled(to_dev_u8(a), to_dev_u8(sfa), to_dev_u8(b), to_dev_u8(sfb))
    torch.cuda.synchronize()
    return bits_of(c)


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (65, 129, 48), (7, 300, 64), (130, 66, 272),
                                   (257, 255, 1040), (128, 128, 128), (33, 17, 16 * 33),
                                   (1, 1, 32), (65, 129, 96), (300, 200, 1056)])
def test_fp4_edge_shapes(m, n, k):
    print(f"fp4 edge m={m} n={n} k={k}", flush=True)
    a, b = synthetic.fp4_packed(m, k, 60, 0), synthetic.fp4_packed(n, k, 60, 1)
    sfa = synthetic.e4m3_uniform(m, k // 16, 2 ** -4, 2 ** 4, 60, 4)
    sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 60, 5)
    got = _run(a, sfa, b, sfb)
    ref = oracle.gemm_fp4_ref(a, sfa, b, sfb)
    check_close(got, ref, k, oracle.rms(oracle.dequant_fp4(a, sfa)), oracle.rms(oracle.dequant_fp4(b, sfb)),
                f"fp4 {m}x{n}x{k}")


def test_fp4_unit_scales_equal_dense_path_on_dequantized_operands():
    m, n, k = 200, 136, 512
    a, b = synthetic.fp4_packed(m, k, 61, 0), synthetic.fp4_packed(n, k, 61, 1)
    one_a = np.full((m, k // 16), 0x38, np.uint8)
    one_b = np.full((n, k // 16), 0x38, np.uint8)
    got = _run(a, one_a, b, one_b)
    ab = oracle.f32_to_bf16(oracle.dequant_fp4(a, one_a).astype(np.float32))
    bb = oracle.f32_to_bf16(oracle.dequant_fp4(b, one_b).astype(np.float32))
    dense = bg.gemm_bf16(to_dev_bf16(ab), to_dev_bf16(bb))
    torch.cuda.synchronize()
    # FP4 products are multiples of 1/4 bounded by 36: sums over 512 terms are exact in FP32
    assert_bits_equal(got, bits_of(dense), "fp4 vs dense")


def test_fp4_full_size_power_of_two_scales_bit_exact():
    """Scales in {1, 2}: every partial sum is exact in FP32, so C is unique."""
    print("fp4 4096x4096x8192 exact scales", flush=True)
    m = n = 4096
    k = 8192
    a, b = synthetic.fp4_packed(m, k, 4, 0), synthetic.fp4_packed(n, k, 4, 1)
    sfa = synthetic.e4m3_choice(m, k // 16, [0x38, 0x40], 4, 4)
    sfb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40], 4, 5)
    got = _run(a, sfa, b, sfb)
    want = oracle.f32_to_bf16(oracle.gemm_fp4_ref(a, sfa, b, sfb).astype(np.float32))
    assert_bits_equal(got, want, "fp4 full exact")


def test_fp4_config_sampled_rows():
    print("fp4 config sampled rows", flush=True)
    a, sfa, b, sfb = synthetic.fp4_gemm()
    got = _run(a, sfa, b, sfb)
    rows = synthetic.sample_rows(a.shape[0], 1024, 1004)
    ref = oracle.gemm_fp4_ref(a[rows], sfa[rows], b, sfb)
    check_close(got[rows], ref, 8192, oracle.rms(oracle.dequant_fp4(a, sfa)),
                oracle.rms(oracle.dequant_fp4(b, sfb)), "fp4 config")


# K % 32 == 16 takes 16-element FP4 staging units and the default tiles;
# K % 32 == 0 takes 32-element units and every forced tile (the K = 96,
# 224 and 1056 cases end in half a 64-wide step)
FP4_TILE_SHAPES = [(1, 1, 16), (65, 129, 48), (257, 255, 1040), (300, 520, 208),
                   (1, 1, 32), (65, 129, 96), (257, 255, 1056), (300, 520, 224)]


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 5, 6, 7, 8, 9, 10, 11])
def test_every_fp4_tile_config(cfg, force):
    """Each FP4 tile variant (the BG_TUNE_FP4_TILE override) on ragged shapes.
    10 and 11 are the decode kernel with four or eight waves (raw FP4 rings in
    LDS, weights dequantized in registers), which takes K % 64 == 0 (the last
    four shapes); other K fall back to the default tiles."""
    force(bg.TUNE_FP4_TILE, cfg)
    for m, n, k in FP4_TILE_SHAPES + [(1, 1, 64), (65, 129, 128), (129, 300, 1024), (128, 520, 320)]:
        a, b = synthetic.fp4_packed(m, k, 70 + cfg, 0), synthetic.fp4_packed(n, k, 70 + cfg, 1)
        sfa = synthetic.e4m3_uniform(m, k // 16, 2 ** -4, 2 ** 4, 70, 4)
        sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 70, 5)
        got = _run(a, sfa, b, sfb)
        check_close(got, oracle.gemm_fp4_ref(a, sfa, b, sfb), k, oracle.rms(oracle.dequant_fp4(a, sfa)),
                    oracle.rms(oracle.dequant_fp4(b, sfb)), f"fp4 cfg {cfg} {m}x{n}x{k}")
        # power-of-two scales: exact in FP32, so bit-exact
        ea = synthetic.e4m3_choice(m, k // 16, [0x38, 0x40], 71, 4)
        eb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40], 71, 5)
        want = oracle.f32_to_bf16(oracle.gemm_fp4_ref(a, ea, b, eb).astype(np.float32))
        assert_bits_equal(_run(a, ea, b, eb), want, f"fp4 cfg {cfg} exact {m}x{n}x{k}")


# ---------------------------------------------------------------------------
# batched FP4, FP4 split-K (decode shapes) and the blocked-scale importer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("L,m,n,k", [(3, 130, 66, 272), (3, 130, 66, 288), (2, 260, 70, 288)])
def test_fp4_batched_equals_per_problem_calls(L, m, n, k):
    print(f"fp4 batched L={L} m={m} n={n} k={k}", flush=True)
    a = np.stack([synthetic.fp4_packed(m, k, 130 + l, 0) for l in range(L)])
    b = np.stack([synthetic.fp4_packed(n, k, 130 + l, 1) for l in range(L)])
    sfa = np.stack([synthetic.e4m3_uniform(m, k // 16, 2 ** -4, 2 ** 4, 130 + l, 4) for l in range(L)])
    sfb = np.stack([synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 130 + l, 5) for l in range(L)])
    c = bg.gemm_fp4_blockscaled_batched(to_dev_u8(a), to_dev_u8(sfa), to_dev_u8(b), to_dev_u8(sfb))
    torch.cuda.synchronize()
    got = bits_of(c)
    for l in range(L):
        one = _run(a[l], sfa[l], b[l], sfb[l])
        assert_bits_equal(got[l], one, f"batch {l} vs single call")
        check_close(got[l], oracle.gemm_fp4_ref(a[l], sfa[l], b[l], sfb[l]), k,
                    oracle.rms(oracle.dequant_fp4(a[l], sfa[l])), oracle.rms(oracle.dequant_fp4(b[l], sfb[l])),
                    f"batch {l}")


@pytest.mark.parametrize("m,n,k,ks", [(128, 512, 4096, 4), (65, 300, 1040, 3), (128, 256, 16384, 16)])
def test_fp4_splitk_planes_and_result(m, n, k, ks):
    print(f"fp4 splitk m={m} n={n} k={k} ks={ks}", flush=True)
    a, b = synthetic.fp4_packed(m, k, 140, 0), synthetic.fp4_packed(n, k, 140, 1)
    sfa = synthetic.e4m3_uniform(m, k // 16, 2 ** -4, 2 ** 4, 140, 4)
    sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 140, 5)
    ws = torch.full((ks, m, n), float("nan"), dtype=torch.float32, device="cuda")
    c = bg.gemm_fp4_blockscaled_splitk(to_dev_u8(a), to_dev_u8(sfa), to_dev_u8(b), to_dev_u8(sfb), ks, workspace=ws)
    torch.cuda.synchronize()
    planes = ws.cpu().numpy()
    ref_planes = oracle.gemm_fp4_splitk_planes_ref(a, sfa, b, sfb, ks)
    kc = oracle.splitk_chunk(k, ks)
    sa, sb = oracle.rms(oracle.dequant_fp4(a, sfa)), oracle.rms(oracle.dequant_fp4(b, sfb))
    for s in range(ks):
        klen = max(0, min(k, (s + 1) * kc) - min(k, s * kc))
        assert (np.abs(planes[s] - ref_planes[s]) <= oracle.tolerance(ref_planes[s], klen, sa, sb)).all(), f"plane {s}"
    assert_bits_equal(bits_of(c), oracle.splitk_reduce(planes), "reduce")
    check_close(bits_of(c), oracle.gemm_fp4_ref(a, sfa, b, sfb), k, sa, sb, "fp4 splitk result")


def test_fp4_splitk_power_of_two_scales_bit_exact():
    m, n, k = 128, 384, 8192
    a, b = synthetic.fp4_packed(m, k, 141, 0), synthetic.fp4_packed(n, k, 141, 1)
    sfa = synthetic.e4m3_choice(m, k // 16, [0x38, 0x40], 141, 4)
    sfb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40], 141, 5)
    want = oracle.f32_to_bf16(oracle.gemm_fp4_ref(a, sfa, b, sfb).astype(np.float32))
    for ks in (1, 2, 8):
        c = bg.gemm_fp4_blockscaled_splitk(to_dev_u8(a), to_dev_u8(sfa), to_dev_u8(b), to_dev_u8(sfb), ks)
        torch.cuda.synchronize()
        assert_bits_equal(bits_of(c), want, f"fp4 splitk exact ks={ks}")


@pytest.mark.parametrize("n,k", [(7168, 16384), (4096, 7168)])
def test_fp4_decode_shapes_sampled_columns(n, k):
    """The kernelbot page's decode shapes (M = 128): all rows, 512 sampled
    output columns, plain call and split-K."""
    print(f"fp4 decode 128x{n}x{k}", flush=True)
    m = 128
    a, b = synthetic.fp4_packed(m, k, 142, 0), synthetic.fp4_packed(n, k, 142, 1)
    sfa = synthetic.e4m3_uniform(m, k // 16, 2 ** -4, 2 ** 4, 142, 4)
    sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 142, 5)
    cols = synthetic.sample_rows(n, 512, 1030)
    ref = oracle.gemm_fp4_ref(a, sfa, b[cols], sfb[cols])
    sa, sb = oracle.rms(oracle.dequant_fp4(a, sfa)), oracle.rms(oracle.dequant_fp4(b[cols], sfb[cols]))
    da, dsa, db, dsb = to_dev_u8(a), to_dev_u8(sfa), to_dev_u8(b), to_dev_u8(sfb)
    for ks in (1, 8):
        c = bg.gemm_fp4_blockscaled_splitk(da, dsa, db, dsb, ks)
        torch.cuda.synchronize()
        check_close(bits_of(c)[:, cols], ref, k, sa, sb, f"decode 128x{n}x{k} ks={ks}")


@pytest.mark.parametrize("rows,k_groups,batch", [(128, 4, 1), (256, 512, 1), (384, 12, 2)])
def test_scales_from_blocked_bit_exact(rows, k_groups, batch):
    rng = np.random.default_rng(rows + k_groups)
    blocked = rng.integers(0, 256, size=batch * rows * k_groups, dtype=np.uint8)
    got = bg.fp4_scales_from_blocked(to_dev_u8(blocked), rows, k_groups, batch)
    torch.cuda.synchronize()
    want = oracle.scales_from_blocked(blocked, rows, k_groups, batch)
    assert np.array_equal(got.cpu().numpy(), want)


def test_gemm_on_imported_scales_equals_plain_scales():
    """Scales handed over in the blocked layout, imported on the GPU, give
    the same product as the plain scales (inverse layout written here from
    the page's row/group formula)."""
    m, n, k = 256, 384, 1024
    a, b = synthetic.fp4_packed(m, k, 143, 0), synthetic.fp4_packed(n, k, 143, 1)
    sfa = synthetic.e4m3_uniform(m, k // 16, 2 ** -4, 2 ** 4, 143, 4)
    sfb = synthetic.e4m3_uniform(n, k // 16, 2 ** -4, 2 ** 4, 143, 5)

    def to_blocked(plain):
        rows, groups = plain.shape
        out = np.empty(rows * groups, np.uint8)
        pos = 0
        for tile_m in range(rows // 128):
            for tile_k in range(groups // 4):
                for g_m in range(32):
                    for i_m in range(4):
                        for i_k in range(4):
                            out[pos] = plain[tile_m * 128 + i_m * 32 + g_m, tile_k * 4 + i_k]
                            pos += 1
        return out

    isa = bg.fp4_scales_from_blocked(to_dev_u8(to_blocked(sfa)), m, k // 16)[0]
    isb = bg.fp4_scales_from_blocked(to_dev_u8(to_blocked(sfb)), n, k // 16)[0]
    c1 = bg.gemm_fp4_blockscaled(to_dev_u8(a), isa, to_dev_u8(b), isb)
    c2 = bg.gemm_fp4_blockscaled(to_dev_u8(a), to_dev_u8(sfa), to_dev_u8(b), to_dev_u8(sfb))
    torch.cuda.synchronize()
    assert_bits_equal(bits_of(c1), bits_of(c2), "imported vs plain scales")


def _decode_sweep_cases():
    """Seeded (M, N, K, k_splits) draws for the decode kernel: M up to 128
    (one row tile) and a few past it, N around the 128- and 256-column tiles, K a
    multiple of 64 (1 to 40 steps), splits from 1 to 9 (short, partial-group
    and empty splits)."""
    rng = np.random.default_rng(2024)
    cases = []
    for _ in range(24):
        m = int(rng.choice([1, 2, 31, 32, 33, 64, 95, 127, 128, 129, 200]))
        n = int(rng.choice([1, 16, 63, 127, 128, 129, 200, 255, 256, 257, 511, 700]))
        k = 64 * int(rng.integers(1, 41))
        ks = int(rng.integers(1, 10))
        cases.append((m, n, k, ks))
    return cases


@pytest.mark.parametrize("tile", [7, 8, 9])
def test_decode_kernel_shape_sweep_bit_exact(tile, force):
    """The decode kernel (split-K tiles 7, 8 and 9, forced) over 24 seeded shapes,
    on power-of-two scales (every product and sum exact in FP32): each output
    bit-identical to the oracle's."""
    force(bg.TUNE_FP4_SPLITK_TILE, tile)
    for i, (m, n, k, ks) in enumerate(_decode_sweep_cases()):
        print(f"decode sweep tile={tile} m={m} n={n} k={k} ks={ks}", flush=True)
        a, b = synthetic.fp4_packed(m, k, 1700 + i, 0), synthetic.fp4_packed(n, k, 1700 + i, 1)
        sfa = synthetic.e4m3_choice(m, k // 16, [0x30, 0x38, 0x40], 1700 + i, 4)
        sfb = synthetic.e4m3_choice(n, k // 16, [0x30, 0x38, 0x40], 1700 + i, 5)
        c = bg.gemm_fp4_blockscaled_splitk(to_dev_u8(a), to_dev_u8(sfa), to_dev_u8(b), to_dev_u8(sfb), ks)
        torch.cuda.synchronize()
        want = oracle.f32_to_bf16(oracle.gemm_fp4_ref(a, sfa, b, sfb).astype(np.float32))
        assert_bits_equal(bits_of(c), want, f"decode sweep tile {tile} {m}x{n}x{k} ks={ks}")


@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5, 6, 7, 8, 9])
def test_every_fp4_splitk_tile(tile, force):
    """Each FP4 split-K tile (the BG_TUNE_FP4_SPLITK_TILE override): planes
    summed in order equal the exact result on power-of-two scales. 7 and 8
    are the decode kernel with four or eight waves, 9 with eight waves and
    128 columns (K % 64 == 0 only: 1040 and 1056 fall back); its shapes
    cover splits of 1-4 steps (a partial last ring round), chunks that start
    mid-line (448 / 6 = 128-element chunks of a 448-long K), an empty last
    split and rows past 128."""
    force(bg.TUNE_FP4_SPLITK_TILE, tile)
    for m, n, k, ks in [(128, 384, 4096, 8), (65, 129, 1040, 3), (300, 520, 2048, 5), (65, 129, 1056, 3),
                        (1, 1, 64, 2), (33, 257, 640, 4), (128, 300, 1280, 3), (100, 70, 448, 6)]:
        a, b = synthetic.fp4_packed(m, k, 150 + tile, 0), synthetic.fp4_packed(n, k, 150 + tile, 1)
        sfa = synthetic.e4m3_choice(m, k // 16, [0x38, 0x40], 150, 4)
        sfb = synthetic.e4m3_choice(n, k // 16, [0x38, 0x40], 150, 5)
        c = bg.gemm_fp4_blockscaled_splitk(to_dev_u8(a), to_dev_u8(sfa), to_dev_u8(b), to_dev_u8(sfb), ks)
        torch.cuda.synchronize()
        want = oracle.f32_to_bf16(oracle.gemm_fp4_ref(a, sfa, b, sfb).astype(np.float32))
        assert_bits_equal(bits_of(c), want, f"fp4 splitk tile {tile} {m}x{n}x{k} ks={ks}")
