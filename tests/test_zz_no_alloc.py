"""gemm_bf16_splitk_noalloc (the entry point for callers that cannot
allocate) against gemm_bf16_splitk with a caller workspace: same kernels,
chunking and reduction order, so the outputs must be bit-identical. Two calls
in a row, the second with a smaller problem (the shared scratch keeps the
first call's planes, which the second must not read), then limits."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_fp4_gemm_amd as bg
import oracle
import synthetic
from gpu_util import assert_bits_equal, bits_of, check_close, to_dev_bf16

pytestmark = pytest.mark.gpu


def _pair(m, n, k, ks, seed):
    a = synthetic.normal_bf16((m, k), 1.0, seed, 0)
    b = synthetic.normal_bf16((n, k), 0.02, seed, 1)
    da, db = to_dev_bf16(a), to_dev_bf16(b)
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    # through the C ABI directly (the binding only marshals)
    st = bg.lib.gemm_bf16_splitk_noalloc(da.data_ptr(), db.data_ptr(), out.data_ptr(), m, n, k, ks,
                                         torch.cuda.current_stream().cuda_stream)
    assert st == bg.BG_OK, bg.bg_status_string(st)
    ref = bg.gemm_bf16_splitk(da, db, ks)
    torch.cuda.synchronize()
    return a, b, bits_of(out), bits_of(ref)


@pytest.mark.parametrize("first,second", [((1024, 2048, 11008, 4), (128, 2048, 11008, 8)),
                                          ((600, 1000, 3000, 8), (7, 300, 130, 3))])
def test_noalloc_equals_workspace_splitk_twice(first, second):
    for (m, n, k, ks), seed in ((first, 1100), (second, 1101)):
        print(f"noalloc splitk m={m} n={n} k={k} ks={ks}", flush=True)
        a, b, got, ref = _pair(m, n, k, ks, seed)
        assert_bits_equal(got, ref, f"noalloc vs workspace {m}x{n}x{k} ks={ks}")
        rows = synthetic.sample_rows(m, min(m, 64), seed)
        check_close(got[rows], oracle.gemm_bf16_ref(a[rows], b), k, oracle.rms(oracle.bf16_to_f64(a)),
                    oracle.rms(oracle.bf16_to_f64(b)), f"noalloc vs oracle {m}x{n}x{k}")


def test_noalloc_limits_and_k_splits_one():
    da = to_dev_bf16(synthetic.normal_bf16((1024, 256), 1.0, 1102, 0))
    db = to_dev_bf16(synthetic.normal_bf16((2048, 256), 1.0, 1102, 1))
    out = torch.empty((1024, 2048), dtype=torch.bfloat16, device="cuda")
    # 5 * 1024 * 2048 * 4 bytes = 40 MiB > 32 MiB: rejected, nothing enqueued
    with pytest.raises(bg.BlockGemmError) as e:
        bg.gemm_bf16_splitk_noalloc(da, db, 5, out)
    assert e.value.status == bg.BG_ERR_WORKSPACE
    # exactly the limit is accepted
    bg.gemm_bf16_splitk_noalloc(da, db, 4, out)
    four = bits_of(out)
    ref = bits_of(bg.gemm_bf16_splitk(da, db, 4))
    assert_bits_equal(four, ref, "at the limit")
    # k_splits = 1 uses no scratch and equals gemm_bf16
    bg.gemm_bf16_splitk_noalloc(da, db, 1, out)
    assert_bits_equal(bits_of(out), bits_of(bg.gemm_bf16(da, db)), "k_splits = 1")
