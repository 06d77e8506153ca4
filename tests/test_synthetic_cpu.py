"""The seeded input generators (CPU only): determinism and the row sample."""
import numpy as np
import pytest

import synthetic


@pytest.mark.parametrize("m,count,seed", [(5120, 1024, 1002), (4096, 1024, 1004), (2048, 512, 1003),
                                          (5120, 256, 1002), (300, 64, 7)])
def test_sample_rows_spans_every_quarter(m, count, seed):
    rows = synthetic.sample_rows(m, count, seed)
    assert rows.size == count and np.unique(rows).size == count
    assert rows[0] == 0 and rows[-1] == m - 1 and (np.diff(rows) > 0).all()
    # uniform over the rows: each quarter holds count/4 rows up to sampling noise
    q = np.bincount(np.minimum(rows * 4 // m, 3), minlength=4)
    assert (np.abs(q - count / 4) < 4 * np.sqrt(count / 4) + 2).all(), q
    assert rows[-2] > m * (1 - 8.0 / count)


def test_sample_rows_small_m_is_every_row_and_deterministic():
    assert np.array_equal(synthetic.sample_rows(100, 128, 1), np.arange(100))
    assert np.array_equal(synthetic.sample_rows(5000, 100, 3), synthetic.sample_rows(5000, 100, 3))
    assert not np.array_equal(synthetic.sample_rows(5000, 100, 3), synthetic.sample_rows(5000, 100, 4))


def test_generators_are_functions_of_seed_and_tensor_id():
    a = synthetic.normal_bf16((4, 8), 1.0, 5, 0)
    assert np.array_equal(a, synthetic.normal_bf16((4, 8), 1.0, 5, 0))
    assert not np.array_equal(a, synthetic.normal_bf16((4, 8), 1.0, 5, 1))
    assert not np.array_equal(a, synthetic.normal_bf16((4, 8), 1.0, 6, 0))
