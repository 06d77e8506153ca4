"""GPU parity of gemm_bf16_dual (two products of one A in one launch).

Each output must equal the oracle within the tolerance, and must be
bit-identical to an ordinary gemm_bf16 call on the same operands: every
output element is one tile's FP32 sum over K in the same order whichever
launch computes it.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
import synthetic
from gpu_util import assert_bits_equal, bits_of, check_close, to_dev_bf16

pytestmark = pytest.mark.gpu

# the last three take gemm_bf16's sliced-K tile (deep K, few tiles): the dual
# launch must then sum each output in the same two K halves
SHAPES = [(1, 1, 8), (7, 129, 65), (65, 257, 136), (300, 200, 1000), (257, 255, 2000), (129, 520, 64),
          (513, 384, 72), (33, 70, 9), (260, 300, 127), (128, 256, 512), (300, 200, 2048), (512, 1024, 4096)]


def _inputs(m, n, k, seed):
    a = synthetic.normal_bf16((m, k), 1.0, seed, 0)
    b0 = synthetic.normal_bf16((n, k), 0.5, seed, 1)
    b1 = synthetic.normal_bf16((n, k), 0.25, seed, 3)
    return a, b0, b1


def _check(a, b0, b1, what):
    m, k = a.shape
    da, db0, db1 = to_dev_bf16(a), to_dev_bf16(b0), to_dev_bf16(b1)
    c0, c1 = bg.gemm_bf16_dual(da, db0, db1)
    s0, s1 = bg.gemm_bf16(da, db0), bg.gemm_bf16(da, db1)
    torch.cuda.synchronize()
    g0, g1 = bits_of(c0), bits_of(c1)
    sa = oracle.rms(oracle.bf16_to_f64(a))
    check_close(g0, oracle.gemm_bf16_ref(a, b0), k, sa, oracle.rms(oracle.bf16_to_f64(b0)), what + " C0")
    check_close(g1, oracle.gemm_bf16_ref(a, b1), k, sa, oracle.rms(oracle.bf16_to_f64(b1)), what + " C1")
    assert_bits_equal(g0, bits_of(s0), what + " C0 vs gemm_bf16")
    assert_bits_equal(g1, bits_of(s1), what + " C1 vs gemm_bf16")


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_dual_matches_oracle_and_single_calls(m, n, k):
    print(f"gemm_bf16_dual m={m} n={n} k={k}", flush=True)
    _check(*_inputs(m, n, k, 4000 + m + n + k), f"dual {m}x{n}x{k}")


# every direct tile configuration of the dense table, forced through the
# tuning hook (0 is the register-staged tile: the dual call then runs two
# ordinary launches)
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 6, 8, 9, 10, 12, 14, 17, 23, 24, 27, 28])
def test_dual_every_tile_config(cfg, force):
    force(bg.TUNE_TILE, cfg)
    for m, n, k in [(65, 257, 136), (257, 300, 520), (33, 70, 64), (130, 260, 512)]:
        _check(*_inputs(m, n, k, 5000 + cfg), f"cfg {cfg} dual {m}x{n}x{k}")


def test_dual_exactly_summable_is_bit_exact():
    m, n, k = 300, 260, 1000
    a = synthetic.grid_bf16((m, k), -8, 8, -5, 11, 0)
    b0 = synthetic.grid_bf16((n, k), -8, 8, -5, 11, 1)
    b1 = synthetic.grid_bf16((n, k), -8, 8, -5, 11, 3)
    c0, c1 = bg.gemm_bf16_dual(to_dev_bf16(a), to_dev_bf16(b0), to_dev_bf16(b1))
    torch.cuda.synchronize()
    assert_bits_equal(bits_of(c0), oracle.f32_to_bf16(oracle.gemm_bf16_ref(a, b0).astype(np.float32)), "C0")
    assert_bits_equal(bits_of(c1), oracle.f32_to_bf16(oracle.gemm_bf16_ref(a, b1).astype(np.float32)), "C1")


def test_dual_mlp_gate_up_shape():
    """5120 x 11008 x 2048 twice (the gate and up projections), in the launch
    configuration bench.py times: both outputs bit-identical to single calls
    over the whole output, and 256 seeded rows of each against the oracle."""
    print("gemm_bf16_dual gate/up 5120x11008x2048", flush=True)
    x, wg = synthetic.mlp_gate_up()
    wu = synthetic.normal_bf16((11008, 2048), 0.02, 2, synthetic.TID_B2 + 10)
    dx, dg, du = to_dev_bf16(x), to_dev_bf16(wg), to_dev_bf16(wu)
    g, u = bg.gemm_bf16_dual(dx, dg, du)
    g1, u1 = bg.gemm_bf16(dx, dg), bg.gemm_bf16(dx, du)
    torch.cuda.synchronize()
    assert torch.equal(g.view(torch.int16), g1.view(torch.int16))
    assert torch.equal(u.view(torch.int16), u1.view(torch.int16))
    rows = synthetic.sample_rows(5120, 256, 1002)
    sx = oracle.rms(oracle.bf16_to_f64(x))
    for w, c, name in ((wg, g, "gate"), (wu, u, "up")):
        got = bits_of(c[torch.from_numpy(rows).to(c.device)])
        check_close(got, oracle.gemm_bf16_ref(x[rows], w), 2048, sx, oracle.rms(oracle.bf16_to_f64(w)),
                    f"dual {name} rows")


def test_dual_repeat_runs_are_identical():
    a, b0, b1 = _inputs(520, 700, 300, 77)
    da, db0, db1 = to_dev_bf16(a), to_dev_bf16(b0), to_dev_bf16(b1)
    outs = [bg.gemm_bf16_dual(da, db0, db1) for _ in range(3)]
    torch.cuda.synchronize()
    for c0, c1 in outs[1:]:
        assert_bits_equal(bits_of(c0), bits_of(outs[0][0]), "repeat C0")
        assert_bits_equal(bits_of(c1), bits_of(outs[0][1]), "repeat C1")


def test_dual_k_zero_gives_positive_zero():
    """K = 0: both outputs are the empty sum, +0, over their whole extent."""
    dev = "cuda"
    a = torch.empty((70, 0), dtype=torch.bfloat16, device=dev)
    b = torch.empty((40, 0), dtype=torch.bfloat16, device=dev)
    c0 = torch.full((70, 40), 1.0, dtype=torch.bfloat16, device=dev)
    c1 = torch.full((70, 40), -1.0, dtype=torch.bfloat16, device=dev)
    bg.gemm_bf16_dual(a, b, b.clone(), out0=c0, out1=c1)
    torch.cuda.synchronize()
    assert not bits_of(c0).any() and not bits_of(c1).any()
