"""CPU checks of the full-size tests' helpers against the oracle they stand
in for (no GPU)."""
import numpy as np

import oracle
from tests import fullsize_util as FU


def test_row_chunked_quantization_equals_the_oracle():
    r = np.random.default_rng(3)
    w = r.standard_normal((1000, 96)) * np.exp(r.uniform(-4, 4, (1000, 96)))
    s = np.float32(448.0) / np.float32(np.abs(w).max())
    np.testing.assert_array_equal(FU.quantize_e4m3_rows(w, s, chunk=37),
                                  oracle.quantize_e4m3(w, s))


def test_fp8_matmul_with_prequantized_weights_equals_the_oracle():
    r = np.random.default_rng(4)
    a = r.standard_normal((5, 64))
    b = r.standard_normal((40, 64)) * 0.1
    sa, sb = np.float32(448.0 / 4.0), np.float32(448.0) / np.float32(np.abs(b).max())
    np.testing.assert_array_equal(FU.fp8_matmul_q(a, sa, FU.quantize_e4m3_rows(b, sb, 7), sb),
                                  oracle.fp8_matmul(a, b, sa, sb))


def test_sample_rows_cover_every_block_boundary():
    r = np.random.default_rng(5)
    for a, b in ((0, 1), (10, 42), (100, 1124), (7, 7 + 32 * 5)):
        rows = FU.sample_rows(a, b, r)
        assert rows.min() >= a and rows.max() < b
        for s in range(a, b, FU.BLOCK):
            assert s in rows and min(s + FU.BLOCK - 1, b - 1) in rows


def test_choose_experts_takes_the_hottest_and_ragged_ones():
    r = np.random.default_rng(6)
    counts = np.array([0, 5, 64, 700, 33, 31, 32, 9000, 96, 1, 0, 65])
    hot, other = FU.choose_experts(counts, 2, 3, r)
    assert hot.tolist() == [3, 7]
    assert len(other) == 3 and all(counts[e] % 32 != 0 and e not in (3, 7) for e in other)
