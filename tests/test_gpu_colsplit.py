"""GPU checks of gemm_bf16's column split.

When the last round of 256x256 tiles would be poorly filled, gemm_bf16 runs
the first n1 columns as whole rounds of 256x256 tiles and the remaining
columns as a second launch with a smaller tile, writing into the same C
(row stride N). Each output is still one tile's FP32 sum over K in the same
order, so the split result must equal the unsplit one (the BG_TUNE_COLSPLIT override set to 0, a
tuning hook) bit for bit, and the oracle within the GEMM tolerance.

With 256 CUs the shapes below split as noted (first part, second tile).
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
import synthetic
from gpu_util import assert_bits_equal, bits_of, check_close, to_dev_bf16

pytestmark = pytest.mark.gpu

SPLIT_SHAPES = [
    (5120, 11008, 2048),   # 9472 columns, then 256x128 tiles (the MLP gate/up shape)
    (5000, 7000, 3000),    # 6400, then 128x128; ragged M, ragged remainder, ragged K step
    (4096, 10472, 1024),   # 8192, then 160x256; ragged remainder
    (2500, 10000, 512),    # 6144, then 160x256
    (1000, 20000, 256),    # 16128, then 128x128
    (6000, 6100, 1000),    # 5376, then 160x128
]


def _both(a_bits, b_bits, force):
    da, db = to_dev_bf16(a_bits), to_dev_bf16(b_bits)
    split = bits_of(bg.gemm_bf16(da, db))
    force(bg.TUNE_COLSPLIT, 0)
    whole = bits_of(bg.gemm_bf16(da, db))
    force(bg.TUNE_COLSPLIT, -1)
    torch.cuda.synchronize()
    return split, whole


@pytest.mark.parametrize("m,n,k", SPLIT_SHAPES)
def test_column_split_equals_unsplit_bitwise(m, n, k, force):
    print(f"column split m={m} n={n} k={k}", flush=True)
    a = synthetic.normal_bf16((m, k), 1.0, 70, 0)
    b = synthetic.normal_bf16((n, k), 0.05, 70, 1)
    split, whole = _both(a, b, force)
    assert_bits_equal(split, whole, f"split vs unsplit {m}x{n}x{k}")
    rows = synthetic.sample_rows(m, min(m, 256), 1020)
    check_close(split[rows], oracle.gemm_bf16_ref(a[rows], b), k, oracle.rms(oracle.bf16_to_f64(a)),
                oracle.rms(oracle.bf16_to_f64(b)), f"split {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(5000, 7000, 3000), (6000, 6100, 1000)])
def test_column_split_exactly_summable_matches_oracle(m, n, k):
    a = synthetic.grid_bf16((m, k), -8, 8, -5, 71, 0)
    b = synthetic.grid_bf16((n, k), -8, 8, -5, 71, 1)
    got = bits_of(bg.gemm_bf16(to_dev_bf16(a), to_dev_bf16(b)))
    want = oracle.f32_to_bf16(oracle.gemm_bf16_ref(a, b).astype(np.float32))
    assert_bits_equal(got, want, f"split grid {m}x{n}x{k}")


def test_column_split_leaves_nothing_outside_c():
    """C is written exactly: a guard band around it keeps its sentinel."""
    m, n, k = 6000, 6100, 1000
    a = synthetic.grid_bf16((m, k), -8, 8, -5, 72, 0)
    b = synthetic.grid_bf16((n, k), -8, 8, -5, 72, 1)
    guard = 4096
    buf = torch.full((guard + m * n + guard,), 0x7FC1, dtype=torch.int16, device="cuda")
    c = buf[guard:guard + m * n].view(torch.bfloat16).view(m, n)
    bg.gemm_bf16(to_dev_bf16(a), to_dev_bf16(b), out=c)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert (host[:guard] == 0x7FC1).all() and (host[guard + m * n:] == 0x7FC1).all()
    want = oracle.f32_to_bf16(oracle.gemm_bf16_ref(a, b).astype(np.float32))
    assert_bits_equal(host[guard:guard + m * n].view(np.uint16).reshape(m, n), want, "guarded split")
