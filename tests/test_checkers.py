"""CPU checks of the parity helpers themselves: each planted mistake in an
index set or an attention output must be caught (so that a GPU result the
helpers accept is really correct)."""
import numpy as np
import pytest
import torch

from parity_checks import check_attention, check_topk_properties


def _check(scores, idx, offset, k):
    s = torch.tensor(scores, dtype=torch.float32)
    i = torch.tensor(idx, dtype=torch.int32)
    check_topk_properties(torch, s, i, offset, k, "case")


def test_topk_checker_accepts_the_top_k():
    _check([[5, 4, 3, 3]], [[0, 1]], 3, 2)
    _check([[5, 3, 3, 3]], [[0, 1]], 3, 2)
    _check([[1, 7, 7, 2]], [[1, 2]], 3, 2)
    # fewer causal keys than k: all of them, then -1
    _check([[2, 9, -np.inf, -np.inf]], [[0, 1, -1]], 1, 3)


def test_topk_checker_rejects_a_left_out_larger_score():
    # [5, 4, 3, 3], k = 2: keeping the tied 3 instead of the 4 is wrong
    with pytest.raises(AssertionError, match="larger score"):
        _check([[5, 4, 3, 3]], [[0, 2]], 3, 2)


def test_topk_checker_rejects_the_wrong_tie():
    with pytest.raises(AssertionError, match="tie rule"):
        _check([[5, 3, 3, 3]], [[0, 2]], 3, 2)


def test_topk_checker_rejects_bad_layouts():
    with pytest.raises(AssertionError, match="ascending"):
        _check([[5, 4, 3, 3]], [[1, 0]], 3, 2)
    with pytest.raises(AssertionError, match="count"):
        _check([[5, 4, 3, 3]], [[0, -1]], 3, 2)
    with pytest.raises(AssertionError, match="non-causal"):
        _check([[5, 4, 3, 9]], [[0, 3]], 2, 2)


def test_attention_checker_tolerances():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((3, 2, 8))
    lse = rng.standard_normal((3, 2))
    check_attention((ref + 3e-3).astype(np.float32), lse.astype(np.float32) + 5e-4, ref, lse, "ok")
    bad = ref.copy()
    bad[1, 1, 3] += 5e-3
    with pytest.raises(AssertionError, match="max abs"):
        check_attention(bad.astype(np.float32), None, ref, lse, "max")
    with pytest.raises(AssertionError, match="lse"):
        check_attention(ref.astype(np.float32), lse.astype(np.float32) + 2e-3, ref, lse, "lse")
    neg = lse.copy()
    neg[0, 0] = -np.inf
    with pytest.raises(AssertionError, match="finiteness"):
        check_attention(ref.astype(np.float32), lse.astype(np.float32), ref, neg, "inf")
