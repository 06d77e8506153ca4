"""GPU parity of gemm_bf16 against the oracle (C-ABI through the binding)."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
import synthetic
from gpu_util import assert_bits_equal, bits_of, check_close, empty_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu

EDGE = [1, 2, 7, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 257]
EDGE_SHAPES = sorted({(v, 129, 65) for v in EDGE} | {(65, v, 129) for v in EDGE}
                     | {(129, 65, v) for v in EDGE} | {(300, 200, 1000), (257, 255, 136), (33, 520, 64)})


def _run(a_bits, b_bits):
    a, b = to_dev_bf16(a_bits), to_dev_bf16(b_bits)
    c = bg.gemm_bf16(a, b)
    torch.cuda.synchronize()
    return bits_of(c)


@pytest.mark.parametrize("m,n,k", EDGE_SHAPES)
def test_edge_shapes(m, n, k):
    print(f"gemm_bf16 edge m={m} n={n} k={k}", flush=True)
    a = synthetic.normal_bf16((m, k), 1.0, 1000 + m, 0)
    b = synthetic.normal_bf16((n, k), 0.5, 2000 + n, 1)
    got = _run(a, b)
    ref = oracle.gemm_bf16_ref(a, b)
    check_close(got, ref, k, oracle.rms(oracle.bf16_to_f64(a)), oracle.rms(oracle.bf16_to_f64(b)),
                f"edge {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(200, 136, 2000), (129, 255, 1032), (64, 64, 64), (5, 3, 9)])
def test_exactly_summable_is_bit_exact(m, n, k):
    a = synthetic.grid_bf16((m, k), -8, 8, -5, 3, 0)
    b = synthetic.grid_bf16((n, k), -8, 8, -5, 3, 1)
    got = _run(a, b)
    want = oracle.f32_to_bf16(oracle.gemm_bf16_ref(a, b).astype(np.float32))
    assert_bits_equal(got, want, f"grid {m}x{n}x{k}")


def test_k_zero_gives_positive_zero():
    a = np.zeros((70, 0), np.uint16)
    c = empty_bf16(70, 40, fill_bits=0x3F80)
    bg.gemm_bf16(torch.empty((70, 0), dtype=torch.bfloat16, device="cuda"),
                 torch.empty((40, 0), dtype=torch.bfloat16, device="cuda"), out=c)
    torch.cuda.synchronize()
    assert not bits_of(c).any()
    del a


def test_identity_and_permutation_weights_are_exact():
    k = 256
    a = synthetic.normal_bf16((300, k), 1.0, 7, 0)
    eye = oracle.f32_to_bf16(np.eye(k, dtype=np.float32))
    assert_bits_equal(_run(a, eye), a, "identity")
    perm = np.random.default_rng(1).permutation(k)
    p = np.zeros((k, k), np.float32)
    p[np.arange(k), perm] = 1.0
    assert_bits_equal(_run(a, oracle.f32_to_bf16(p)), a[:, perm], "permutation")


def test_config_dense_small_full_output():
    a, b = synthetic.dense_small()
    got = _run(a, b)
    ref = oracle.gemm_bf16_ref(a, b)
    check_close(got, ref, 512, oracle.rms(oracle.bf16_to_f64(a)), oracle.rms(oracle.bf16_to_f64(b)),
                "128x256x512")


def _sampled_check(a_bits, b_bits, got_bits, seed, what):
    rows = synthetic.sample_rows(a_bits.shape[0], 1024, 1000 + seed)
    ref = oracle.gemm_bf16_ref(a_bits[rows], b_bits)
    return check_close(got_bits[rows], ref, a_bits.shape[1], oracle.rms(oracle.bf16_to_f64(a_bits)),
                       oracle.rms(oracle.bf16_to_f64(b_bits)), what)


@pytest.mark.parametrize("n", [2048, 512])
def test_attention_projections_sampled_rows(n):
    print(f"attn proj n={n}", flush=True)
    a, b = synthetic.attn_proj(n=n)
    got = _run(a, b)
    _sampled_check(a, b, got, 1, f"attn n={n}")


def test_mlp_gate_up_sampled_rows_and_determinism():
    print("mlp gate/up", flush=True)
    a, b = synthetic.mlp_gate_up()
    da, db = to_dev_bf16(a), to_dev_bf16(b)
    c1 = bg.gemm_bf16(da, db)
    c2 = bg.gemm_bf16(da, db)
    torch.cuda.synchronize()
    g1, g2 = bits_of(c1), bits_of(c2)
    assert_bits_equal(g1, g2, "repeat run")
    _sampled_check(a, b, g1, 2, "gate/up")


# every entry of the tile table (the BG_TUNE_TILE override forces one)
TILE_CFGS = list(range(0, 25)) + [27, 28]
CFG_SHAPES = [(1, 1, 8), (65, 129, 72), (161, 257, 136), (257, 225, 1000), (320, 448, 520), (33, 70, 64)]


@pytest.mark.parametrize("cfg", TILE_CFGS)
def test_every_tile_config_edge_shapes(cfg, force):
    force(bg.TUNE_TILE, cfg)
    for m, n, k in CFG_SHAPES:
        a = synthetic.normal_bf16((m, k), 1.0, 3000 + m, 0)
        b = synthetic.normal_bf16((n, k), 0.5, 3000 + n, 1)
        got = _run(a, b)
        check_close(got, oracle.gemm_bf16_ref(a, b), k, oracle.rms(oracle.bf16_to_f64(a)),
                    oracle.rms(oracle.bf16_to_f64(b)), f"cfg {cfg} {m}x{n}x{k}")
        ga = synthetic.grid_bf16((m, k), -8, 8, -5, 5, 0)
        gb = synthetic.grid_bf16((n, k), -8, 8, -5, 5, 1)
        want = oracle.f32_to_bf16(oracle.gemm_bf16_ref(ga, gb).astype(np.float32))
        assert_bits_equal(_run(ga, gb), want, f"cfg {cfg} grid {m}x{n}x{k}")
        # fused fold and split-K planes through the same tile
        out = synthetic.normal_bf16((m, n), 1.0, 7, 2)
        o = to_dev_bf16(out)
        bg.gemm_bf16_scaled_acc(to_dev_bf16(ga), to_dev_bf16(gb), o, 2.0)
        c3 = bg.gemm_bf16_splitk(to_dev_bf16(ga), to_dev_bf16(gb), 3)
        torch.cuda.synchronize()
        assert_bits_equal(bits_of(o), oracle.gemm_scaled_acc_exact(out, ga, gb, 2.0), f"cfg {cfg} fold")
        assert_bits_equal(bits_of(c3), want, f"cfg {cfg} splitk3")


# sliced K (cfg 27: 128 x 128, cfg 28: 64 x 128; two K halves per tile, added
# in a fixed order) takes K % 128 == 0; ragged M and N, one and many steps per half
SLICED_SHAPES = [(1, 1, 128), (65, 129, 128), (161, 257, 1024), (300, 200, 2048), (33, 70, 256), (257, 513, 640)]


@pytest.mark.parametrize("cfg", [27, 28])
def test_slicedk_tiles(cfg, force):
    force(bg.TUNE_TILE, cfg)
    for m, n, k in SLICED_SHAPES:
        print(f"slicedk cfg={cfg} m={m} n={n} k={k}", flush=True)
        a = synthetic.normal_bf16((m, k), 1.0, 3500 + m, 0)
        b = synthetic.normal_bf16((n, k), 0.5, 3500 + n, 1)
        got = _run(a, b)
        check_close(got, oracle.gemm_bf16_ref(a, b), k, oracle.rms(oracle.bf16_to_f64(a)),
                    oracle.rms(oracle.bf16_to_f64(b)), f"slicedk cfg {cfg} {m}x{n}x{k}")
        assert_bits_equal(_run(a, b), got, f"slicedk repeat cfg {cfg} {m}x{n}x{k}")
        ga = synthetic.grid_bf16((m, k), -8, 8, -5, 3501, 0)
        gb = synthetic.grid_bf16((n, k), -8, 8, -5, 3501, 1)
        want = oracle.f32_to_bf16(oracle.gemm_bf16_ref(ga, gb).astype(np.float32))
        assert_bits_equal(_run(ga, gb), want, f"slicedk exact cfg {cfg} {m}x{n}x{k}")

