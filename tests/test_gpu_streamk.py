"""GPU parity of gemm_bf16_streamk against the oracle (C-ABI through the binding).

The stream-K schedule splits some tiles' K sums over several workgroups and
adds their FP32 partials, so random data is compared within the FP32
tolerance and exactly summable data (every partial sum exact) bit for bit.
The plan is fixed by the shape, so repeated calls must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
import synthetic
from gpu_util import assert_bits_equal, bits_of, check_close, empty_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu

# ragged M, N and K (K % 64 != 0 takes a ragged first step), fewer tiles than
# XCDs, fewer steps than workgroups, several tiles per workgroup, deep K
SHAPES = [(1, 1, 8), (5, 3, 16), (65, 129, 72), (129, 65, 64), (33, 17, 528), (300, 200, 1000),
          (257, 255, 1040), (130, 1001, 256), (64, 64, 6400), (1000, 700, 4096), (2048, 2048, 64)]


def _run(a_bits, b_bits, ws=None):
    c = bg.gemm_bf16_streamk(to_dev_bf16(a_bits), to_dev_bf16(b_bits), workspace=ws)
    torch.cuda.synchronize()
    return bits_of(c)


@pytest.mark.parametrize("cfg", [-1, 23, 10])
def test_streamk_shapes_against_oracle(cfg, force):
    if cfg >= 0:
        force(bg.TUNE_STREAMK_TILE, cfg)
    for m, n, k in SHAPES:
        print(f"streamk cfg={cfg} m={m} n={n} k={k}", flush=True)
        a = synthetic.normal_bf16((m, k), 1.0, 3000 + m, 0)
        b = synthetic.normal_bf16((n, k), 0.5, 3000 + n, 1)
        check_close(_run(a, b), oracle.gemm_bf16_ref(a, b), k, oracle.rms(oracle.bf16_to_f64(a)),
                    oracle.rms(oracle.bf16_to_f64(b)), f"streamk cfg {cfg} {m}x{n}x{k}")
        ga = synthetic.grid_bf16((m, k), -8, 8, -5, 3001, 0)
        gb = synthetic.grid_bf16((n, k), -8, 8, -5, 3001, 1)
        want = oracle.f32_to_bf16(oracle.gemm_bf16_ref(ga, gb).astype(np.float32))
        assert_bits_equal(_run(ga, gb), want, f"streamk exact cfg {cfg} {m}x{n}x{k}")


@pytest.mark.parametrize("cfg", [23, 10])
def test_streamk_attention_kv_sampled_rows_and_repeatable(cfg, force):
    """5120 x 512 x 2048 (160 tiles of 128 x 128 on 256 CUs: every tile's K
    split over two or three workgroups): sampled rows against the oracle;
    three calls, one with a workspace full of random bytes, give identical
    bits."""
    force(bg.TUNE_STREAMK_TILE, cfg)
    a, b = synthetic.attn_proj(n=512)
    print(f"streamk kv cfg={cfg}", flush=True)
    A, B = to_dev_bf16(a), to_dev_bf16(b)
    need = bg.gemm_bf16_streamk_workspace(5120, 512, 2048)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    first = bits_of(bg.gemm_bf16_streamk(A, B, workspace=ws))
    second = bits_of(bg.gemm_bf16_streamk(A, B, workspace=ws))
    noise = torch.randint(0, 256, (need,), dtype=torch.uint8, generator=torch.Generator().manual_seed(5)).cuda()
    third = bits_of(bg.gemm_bf16_streamk(A, B, workspace=noise))
    torch.cuda.synchronize()
    assert_bits_equal(second, first, "repeat")
    assert_bits_equal(third, first, "workspace of random bytes")
    rows = synthetic.sample_rows(5120, 1024, 3100)
    check_close(first[rows], oracle.gemm_bf16_ref(a[rows], b), 2048, oracle.rms(oracle.bf16_to_f64(a)),
                oracle.rms(oracle.bf16_to_f64(b)), f"streamk kv cfg {cfg}")


def test_streamk_workspace_reused_across_shapes():
    """One workspace, calls of different shapes back to back (flags left by
    the previous call belong to another call and must not be taken)."""
    need = max(bg.gemm_bf16_streamk_workspace(m, n, k) for m, n, k in SHAPES)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for i, (m, n, k) in enumerate(SHAPES + SHAPES[::-1]):
        a = synthetic.grid_bf16((m, k), -8, 8, -5, 3200 + i, 0)
        b = synthetic.grid_bf16((n, k), -8, 8, -5, 3200 + i, 1)
        want = oracle.f32_to_bf16(oracle.gemm_bf16_ref(a, b).astype(np.float32))
        assert_bits_equal(_run(a, b, ws), want, f"reuse {m}x{n}x{k}")


def test_streamk_fallback_shapes_equal_gemm_bf16():
    """K % 8 != 0 runs gemm_bf16's kernel (no workspace needed: NULL is
    accepted); K == 0 gives +0."""
    L = bg.lib
    for m, n, k in [(70, 90, 100), (129, 3, 9), (1, 1, 1)]:
        a = synthetic.normal_bf16((m, k), 1.0, 3300 + k, 0)
        b = synthetic.normal_bf16((n, k), 0.5, 3300 + k, 1)
        A, B = to_dev_bf16(a), to_dev_bf16(b)
        c = empty_bf16(m, n)
        st = torch.cuda.current_stream().cuda_stream
        assert L.gemm_bf16_streamk(A.data_ptr(), B.data_ptr(), c.data_ptr(), None, 0, m, n, k, st) == bg.BG_OK
        ref = bg.gemm_bf16(A, B)
        torch.cuda.synchronize()
        assert_bits_equal(bits_of(c), bits_of(ref), f"fallback {m}x{n}x{k}")
    c = empty_bf16(40, 30, fill_bits=0x3F80)
    bg.gemm_bf16_streamk(torch.empty((40, 0), dtype=torch.bfloat16, device="cuda"),
                         torch.empty((30, 0), dtype=torch.bfloat16, device="cuda"), out=c)
    torch.cuda.synchronize()
    assert not bits_of(c).any()


def test_streamk_workspace_rules_on_device(force):
    m, n, k = 300, 200, 1000
    need = bg.gemm_bf16_streamk_workspace(m, n, k)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = 8 * (cus // 8)
    force(bg.TUNE_STREAMK_TILE, 23)
    assert bg.gemm_bf16_streamk_workspace(m, n, k) == grid * (128 * 128 * 4 + 8)
    force(bg.TUNE_STREAMK_TILE, 10)
    assert bg.gemm_bf16_streamk_workspace(m, n, k) == grid * (256 * 128 * 4 + 8)
    force(bg.TUNE_STREAMK_TILE, -1)
    assert bg.gemm_bf16_streamk_workspace(m, n, k) == need
    a = to_dev_bf16(synthetic.normal_bf16((m, k), 1.0, 1, 0))
    b = to_dev_bf16(synthetic.normal_bf16((n, k), 1.0, 1, 1))
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(bg.BlockGemmError) as e:
        bg.gemm_bf16_streamk(a, b, workspace=small)
    assert e.value.status == bg.BG_ERR_WORKSPACE
    c = empty_bf16(m, n)
    L = bg.lib
    st = torch.cuda.current_stream().cuda_stream
    assert L.gemm_bf16_streamk(a.data_ptr(), b.data_ptr(), c.data_ptr(), None, need, m, n, k, st) == \
        bg.BG_ERR_WORKSPACE
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [23, 10])
def test_streamk_exchange_repeated_calls(cfg, force):
    """100 calls back to back on exactly summable data (every output unique
    whatever the split), alternating two workspaces: each result compared
    bit for bit on the device with the oracle's, so a partial read before
    its flag, or a flag taken from another call, shows up as a difference."""
    force(bg.TUNE_STREAMK_TILE, cfg)
    m, n, k = 5120, 512, 2048
    print(f"streamk repeated cfg={cfg}", flush=True)
    a = synthetic.grid_bf16((m, k), -8, 8, -5, 3400, 0)
    b = synthetic.grid_bf16((n, k), -8, 8, -5, 3400, 1)
    want = to_dev_bf16(oracle.f32_to_bf16(oracle.gemm_bf16_ref(a, b).astype(np.float32))).view(torch.int16)
    A, B = to_dev_bf16(a), to_dev_bf16(b)
    need = bg.gemm_bf16_streamk_workspace(m, n, k)
    wss = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
    outs = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for i in range(100):
        c = bg.gemm_bf16_streamk(A, B, workspace=wss[i % 2], out=outs[i % 2])
        bad += (c.view(torch.int16) != want).sum()
    torch.cuda.synchronize()
    assert int(bad) == 0, f"{int(bad)} differing elements over 100 calls"
