"""Host checks of the parity helpers the GPU tests use (tolerance metric and tie band)."""
import numpy as np
import pytest

from helpers import rel_rowmax, topk_valid


def test_rel_rowmax_is_per_row_max_norm():
    ref = np.array([[1.0, -2.0, 0.5], [0.0, 0.0, 0.0]])
    got = np.array([[1.1, -2.0, 0.5], [0.0, 1e-9, 0.0]])
    err = rel_rowmax(got, ref)
    assert np.allclose(err, [0.05, 1e-9])


def test_rel_rowmax_requires_minus_inf_where_the_reference_is_masked():
    ref = np.array([[1.0, -np.inf, 2.0]])
    assert rel_rowmax(np.array([[1.0, -np.inf, 2.0]]), ref).max() == 0.0
    for bad in (np.inf, np.nan, 3.0):
        with pytest.raises(AssertionError):
            rel_rowmax(np.array([[1.0, bad, 2.0]]), ref)
    with pytest.raises(AssertionError):  # -inf where the reference is finite
        rel_rowmax(np.array([[-np.inf, -np.inf, 2.0]]), ref)
    with pytest.raises(AssertionError):  # NaN in the finite part
        rel_rowmax(np.array([[np.nan, -np.inf, 2.0]]), ref)


def test_rel_rowmax_does_not_warn_on_masked_entries():
    ref = np.array([[1.0, -np.inf]])
    with np.errstate(all="raise"):
        rel_rowmax(np.array([[1.0, -np.inf]]), ref)


def test_topk_valid_tie_band():
    sc = np.array([5.0, 4.0, 4.0 + 1e-5, 1.0, 0.0])
    assert topk_valid([0, 1, -1], sc, p=4, K=2) is None          # 1 and 2 tie within the band
    assert topk_valid([0, 2, -1], sc, p=4, K=2) is None
    assert topk_valid([0, 3, -1], sc, p=4, K=2) is not None      # below the band
    assert topk_valid([1, 2, -1], sc, p=4, K=2) is not None      # misses 0, above the band
    assert topk_valid([0, 0, -1], sc, p=4, K=2) is not None      # duplicate
    assert topk_valid([0, 1, 3], sc, p=4, K=2) is not None       # padding not -1
