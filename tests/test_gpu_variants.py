"""GPU parity of split-K, the fused LoRA fold and the order-preserving mode."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
from oracle import cpp
import synthetic
from gpu_util import assert_bits_equal, bits_of, check_close, empty_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# split-K
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,n,k,ks", [(65, 129, 1000, 3), (128, 128, 4096, 8), (7, 300, 130, 8),
                                      (257, 63, 2056, 2), (33, 40, 17, 4), (100, 72, 11008, 8)])
def test_splitk_planes_and_result(m, n, k, ks):
    print(f"splitk m={m} n={n} k={k} ks={ks}", flush=True)
    a = synthetic.normal_bf16((m, k), 1.0, 30 + ks, 0)
    b = synthetic.normal_bf16((n, k), 0.02, 30 + ks, 1)
    ws = torch.full((ks, m, n), float("nan"), dtype=torch.float32, device="cuda")
    c = bg.gemm_bf16_splitk(to_dev_bf16(a), to_dev_bf16(b), ks, workspace=ws)
    torch.cuda.synchronize()
    planes = ws.cpu().numpy()
    ref_planes = oracle.gemm_splitk_planes_ref(a, b, ks)
    kc = oracle.splitk_chunk(k, ks)
    sa, sb = oracle.rms(oracle.bf16_to_f64(a)), oracle.rms(oracle.bf16_to_f64(b))
    for s in range(ks):
        klen = max(0, min(k, (s + 1) * kc) - min(k, s * kc))
        tol = oracle.tolerance(ref_planes[s], klen, sa, sb)
        assert (np.abs(planes[s] - ref_planes[s]) <= tol).all(), f"plane {s}"
    # the reduction is exactly the ascending FP32 sum of the planes the GPU wrote
    assert_bits_equal(bits_of(c), oracle.splitk_reduce(planes), "reduce")
    check_close(bits_of(c), oracle.gemm_bf16_ref(a, b), k, sa, sb, "splitk result")


def test_splitk_one_equals_gemm_bf16():
    a, b = synthetic.normal_bf16((200, 520), 1.0, 5, 0), synthetic.normal_bf16((136, 520), 1.0, 5, 1)
    da, db = to_dev_bf16(a), to_dev_bf16(b)
    c1 = bg.gemm_bf16_splitk(da, db, 1)
    c0 = bg.gemm_bf16(da, db)
    torch.cuda.synchronize()
    assert_bits_equal(bits_of(c1), bits_of(c0), "k_splits=1")


@pytest.mark.parametrize("ks", [1, 2, 4, 8])
def test_splitk_exactly_summable_bit_exact(ks):
    a = synthetic.grid_bf16((96, 3000), -8, 8, -5, 6, 0)
    b = synthetic.grid_bf16((80, 3000), -8, 8, -5, 6, 1)
    c = bg.gemm_bf16_splitk(to_dev_bf16(a), to_dev_bf16(b), ks)
    torch.cuda.synchronize()
    want = oracle.f32_to_bf16(oracle.gemm_bf16_ref(a, b).astype(np.float32))
    assert_bits_equal(bits_of(c), want, f"grid ks={ks}")


@pytest.mark.parametrize("ks", [1, 2, 4, 8])
def test_mlp_down_sampled_rows(ks):
    print(f"mlp down ks={ks}", flush=True)
    a, b = synthetic.mlp_down()
    c = bg.gemm_bf16_splitk(to_dev_bf16(a), to_dev_bf16(b), ks)
    torch.cuda.synchronize()
    got = bits_of(c)
    rows = synthetic.sample_rows(a.shape[0], 1024, 1002)
    ref = oracle.gemm_bf16_ref(a[rows], b)
    check_close(got[rows], ref, a.shape[1], oracle.rms(oracle.bf16_to_f64(a)),
                oracle.rms(oracle.bf16_to_f64(b)), f"down ks={ks}")


# ---------------------------------------------------------------------------
# fused LoRA fold
# ---------------------------------------------------------------------------

def _fold(out_bits, x_bits, b_bits, scale):
    out = to_dev_bf16(out_bits)
    bg.gemm_bf16_scaled_acc(to_dev_bf16(x_bits), to_dev_bf16(b_bits), out, scale)
    torch.cuda.synchronize()
    return bits_of(out)


@pytest.mark.parametrize("m,n,k", [(2048, 17408, 64), (65, 129, 40), (7, 300, 64), (130, 66, 200)])
def test_scaled_acc_exact_inputs_bit_exact(m, n, k):
    print(f"scaled_acc exact m={m} n={n} k={k}", flush=True)
    out = synthetic.normal_bf16((m, n), 1.0, 3, 2)
    x = synthetic.grid_bf16((m, k), -8, 8, -5, 3, 0)
    b = synthetic.grid_bf16((n, k), -8, 8, -5, 3, 1)
    got = _fold(out, x, b, 2.0)
    assert_bits_equal(got, oracle.gemm_scaled_acc_exact(out, x, b, 2.0), f"fold {m}x{n}x{k}")


def test_scaled_acc_config_data_equals_one_candidate_every_row():
    """LoRA fold workload, full output (2048 x 17408): every element must equal
    the epilogue evaluated at one of the BF16 deltas an FP32 accumulation of
    X * Bl^T can round to (the MFMA order is unspecified); all candidates are
    enumerated, so an output between two candidates' results fails."""
    print("scaled_acc config data, all rows", flush=True)
    out, x, bl, scale = synthetic.lora_fold()
    got = _fold(out, x, bl, scale)
    bad = 0
    multi = 0
    for r0 in range(0, out.shape[0], 256):
        r1 = r0 + 256
        ok, ncand = oracle.scaled_acc_admissible(got[r0:r1], out[r0:r1], x[r0:r1], bl, scale)
        bad += int((~ok).sum())
        multi += int((ncand > 1).sum())
        if not ok.all():
            i, j = np.argwhere(~ok)[0]
            print(f"first inadmissible output at ({r0 + i}, {j}): {int(got[r0 + i, j]):#x}", flush=True)
    print(f"elements with more than one candidate delta: {multi} of {out.size}", flush=True)
    assert bad == 0, f"{bad} outputs equal no candidate's epilogue"


def test_scaled_acc_equals_unfused_pair_on_gpu():
    out, x, bl, scale = synthetic.lora_fold(m=512, n=4096)
    dx, db = to_dev_bf16(x), to_dev_bf16(bl)
    fused = to_dev_bf16(out)
    bg.gemm_bf16_scaled_acc(dx, db, fused, scale)
    unfused = to_dev_bf16(out)
    delta = bg.gemm_bf16(dx, db)
    bg.bf16_scaled_add(unfused, delta, scale)
    torch.cuda.synchronize()
    assert_bits_equal(bits_of(fused), bits_of(unfused), "fused vs unfused")


def test_scaled_acc_worked_cases_on_gpu():
    # delta = 1 + 2^-8 must be rounded to BF16 before the add (result 1.0)
    out = np.array([[0x3B80]], np.uint16)
    x = oracle.f32_to_bf16(np.array([[1.0, 2.0 ** -8]], np.float32))
    b = oracle.f32_to_bf16(np.array([[1.0, 1.0]], np.float32))
    assert int(_fold(out, x, b, 1.0)[0, 0]) == 0x3F80
    # scale*delta added in FP32 then rounded (result 1.0, not 0x3F81)
    out = np.array([[0x3F80]], np.uint16)
    x = oracle.f32_to_bf16(np.array([[2.0 ** -8]], np.float32))
    b = oracle.f32_to_bf16(np.array([[1.0]], np.float32))
    assert int(_fold(out, x, b, float(np.float32(1 + 2.0 ** -22)))[0, 0]) == 0x3F80


FOLD_PREFETCH_CFGS = [11, 12, 13, 14, 18, 19, 20, 21, 22]


@pytest.mark.parametrize("cfg", FOLD_PREFETCH_CFGS)
def test_fold_edge_tiles_every_prefetch_config(cfg, force):
    """Edge tiles (rows past M, N not a multiple of 8, ragged columns) skip
    part of the early `out` prefetch; the operand tiles must still be in LDS
    before the MFMAs read them. Each case runs ten times, and every result
    must equal the exact one (grid inputs: the delta is exact in FP32)."""
    force(bg.TUNE_TILE, cfg)
    for m, n, k in [(33, 70, 64), (7, 300, 64), (130, 66, 64), (100, 1000, 32), (65, 136, 128)]:
        print(f"fold cfg={cfg} m={m} n={n} k={k}", flush=True)
        out = synthetic.normal_bf16((m, n), 1.0, 80 + cfg, 2)
        x = synthetic.grid_bf16((m, k), -8, 8, -5, 81, 0)
        b = synthetic.grid_bf16((n, k), -8, 8, -5, 81, 1)
        want = oracle.gemm_scaled_acc_exact(out, x, b, 2.0)
        dx, db = to_dev_bf16(x), to_dev_bf16(b)
        outs = [to_dev_bf16(out) for _ in range(10)]
        for o in outs:
            bg.gemm_bf16_scaled_acc(dx, db, o, 2.0)
        torch.cuda.synchronize()
        for r, o in enumerate(outs):
            assert_bits_equal(bits_of(o), want, f"fold cfg {cfg} {m}x{n}x{k} run {r}")


# ---------------------------------------------------------------------------
# order-preserving mode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m", [4510, 2255])
def test_router_bit_exact(m):
    print(f"router m={m}", flush=True)
    x, w = synthetic.router(m=m)
    dx, dw = to_dev_bf16(x), to_dev_bf16(w)
    c = bg.gemm_bf16_ordered(dx, dw)
    c32 = bg.gemm_bf16_ordered_f32(dx, dw)
    torch.cuda.synchronize()
    want32 = oracle.gemm_ordered_f32(x, w)
    got32 = c32.cpu().numpy()
    assert_bits_equal(got32.view(np.uint32), want32.view(np.uint32), "fp32 sums")
    assert_bits_equal(bits_of(c), oracle.f32_to_bf16(want32), "bf16 out")
    # the plain C++ oracle's strict FP32 recurrence gives the same bits
    want16 = cpp.gemm_ordered(x, w, threads=16)
    assert_bits_equal(bits_of(c), want16, "bf16 out vs C++ oracle")


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (65, 129, 33), (17, 7, 300), (130, 257, 64), (3, 70, 2049)])
def test_ordered_edge_shapes(m, n, k):
    x = synthetic.normal_bf16((m, k), 1.0, 50 + k, 0)
    w = synthetic.normal_bf16((n, k), 0.5, 50 + k, 1)
    c32 = bg.gemm_bf16_ordered_f32(to_dev_bf16(x), to_dev_bf16(w))
    torch.cuda.synchronize()
    assert_bits_equal(c32.cpu().numpy().view(np.uint32), oracle.gemm_ordered_f32(x, w).view(np.uint32),
                      f"ordered {m}x{n}x{k}")


def test_ordered_worked_cases_on_gpu():
    # strict ascending order: 2^24 + 1 - 2^24 -> 0
    x = oracle.f32_to_bf16(np.array([[4096.0, 1.0, 4096.0]], np.float32))
    w = oracle.f32_to_bf16(np.array([[4096.0, 1.0, -4096.0]], np.float32))
    c32 = bg.gemm_bf16_ordered_f32(to_dev_bf16(x), to_dev_bf16(w))
    # separate multiply and add on subnormal products: 3 * 2^-149 (a fused multiply-add gives 2)
    x2 = oracle.f32_to_bf16(np.array([[2.0 ** -75, 1.5 * 2.0 ** -75]], np.float32))
    w2 = oracle.f32_to_bf16(np.array([[2.0 ** -74, 2.0 ** -74]], np.float32))
    d32 = bg.gemm_bf16_ordered_f32(to_dev_bf16(x2), to_dev_bf16(w2))
    torch.cuda.synchronize()
    assert int(c32.cpu().numpy().view(np.uint32)[0, 0]) == 0
    assert int(d32.cpu().numpy().view(np.uint32)[0, 0]) == 3


@pytest.mark.parametrize("choice", list(range(15)))
def test_every_ordered_register_block_bit_exact(choice, force):
    """Each register-block variant (the BG_TUNE_ORDERED override) keeps the strict order.
    Choices 12-14 are the scalar-A form with 1-3 rows per wave (K % 8 == 0;
    other K run the tile form): the shapes with K % 8 == 0 cover a ragged last
    K step (264, 40, 8), rows that do not fill a workgroup's row block, and
    N % 64 != 0."""
    force(bg.TUNE_ORDERED, choice)
    for m, n, k in [(1, 1, 1), (37, 70, 300), (150, 33, 65), (145, 256, 2048), (37, 70, 264), (150, 33, 40),
                    (5, 200, 8), (1, 65, 96)]:
        x = synthetic.normal_bf16((m, k), 1.0, 90 + choice, 0)
        w = synthetic.normal_bf16((n, k), 0.5, 90 + choice, 1)
        dx, dw = to_dev_bf16(x), to_dev_bf16(w)
        c32 = bg.gemm_bf16_ordered_f32(dx, dw)
        c16 = bg.gemm_bf16_ordered(dx, dw)
        torch.cuda.synchronize()
        want = oracle.gemm_ordered_f32(x, w)
        assert_bits_equal(c32.cpu().numpy().view(np.uint32), want.view(np.uint32), f"ord {choice} {m}x{n}x{k}")
        assert_bits_equal(bits_of(c16), oracle.f32_to_bf16(want), f"ord bf16 {choice} {m}x{n}x{k}")


@pytest.mark.parametrize("choice", [-1, 12, 13, 14])
def test_ordered_scalar_a_shape_sweep(choice, force):
    """The scalar-A form (forced, and the automatic choice) over 16 seeded
    shapes with K % 8 == 0: rows that do not fill a workgroup's 4*RM rows,
    N % 64 != 0, and ragged last K steps (K % 32 in 8, 16, 24); FP32 sums
    bit-identical to the strict-order oracle."""
    if choice >= 0:
        force(bg.TUNE_ORDERED, choice)
    rng = np.random.default_rng(77)
    for i in range(16):
        m = int(rng.integers(1, 300))
        n = int(rng.integers(1, 200))
        k = 8 * int(rng.integers(1, 90))
        x = synthetic.normal_bf16((m, k), 1.0, 400 + i, 0)
        w = synthetic.normal_bf16((n, k), 0.5, 400 + i, 1)
        c32 = bg.gemm_bf16_ordered_f32(to_dev_bf16(x), to_dev_bf16(w))
        torch.cuda.synchronize()
        want = oracle.gemm_ordered_f32(x, w)
        assert_bits_equal(c32.cpu().numpy().view(np.uint32), want.view(np.uint32),
                          f"ordered sweep {choice} {m}x{n}x{k}")


@pytest.mark.parametrize("count", [1, 7, 8, 9, 1000, 4099])
def test_bf16_scaled_add_matches_epilogue_definition(count):
    out = synthetic.normal_bf16((count,), 1.0, 11, 2)
    d = synthetic.normal_bf16((count,), 0.3, 11, 3)
    o = to_dev_bf16(out)
    bg.bf16_scaled_add(o, to_dev_bf16(d), 0.7)
    torch.cuda.synchronize()
    assert_bits_equal(bits_of(o), oracle.scaled_acc_epilogue(out, d, 0.7), f"scaled_add {count}")
