"""The relaxed index-set rule used for the matrix-core scorer accepts swaps at
the K-th score and rejects anything else (checked on the CPU with the oracle's
scores; the planted mistakes are made on the CPU side)."""
import numpy as np
import pytest

from oracle import csa2 as O
from oracle import formats as F
from gpu_util import relaxed_topk_check


def _case(seed, n=3000, k=200):
    rng = np.random.default_rng(seed)
    q = F.e4m3_value(F.e4m3_encode(rng.standard_normal((8, 64)))).astype(np.float32)
    keys = F.e4m3_value(F.e4m3_encode(rng.standard_normal((n, 8, 64)))).astype(np.float32)
    cand = np.arange(n)
    canon = O.index_scores(q, keys)
    exact, mag = O.index_scores_exact(q, keys)
    want = O.topk_select(canon, cand, k)
    return cand, canon, exact, mag, want, k


def test_identical_sets_pass():
    cand, canon, exact, mag, want, k = _case(1)
    assert relaxed_topk_check(want, want, cand, canon, exact, mag) == 0


def test_exact_score_ranking_passes():
    # the Top-K of the exact scores differs from the fp32 one only at the boundary
    cand, canon, exact, mag, want, k = _case(2)
    got = O.topk_select(exact.astype(np.float32), cand, k)
    relaxed_topk_check(got, want, cand, canon, exact, mag)


def test_boundary_swap_passes_but_far_swap_fails():
    cand, canon, exact, mag, want, k = _case(3)
    w = want[want >= 0]
    order = np.argsort(-exact, kind="stable")
    outside = order[k + 50]                    # well below the K-th score
    got = np.sort(np.concatenate([w[w != w[np.argmax(exact[w])]], [outside]]))
    with pytest.raises(AssertionError):
        relaxed_topk_check(got, want, cand, canon, exact, mag)


def test_boundary_swap_within_tolerance_passes():
    # swap the K-th element for an outside candidate whose exact score is made
    # (by editing the scores) equal to the K-th one's
    cand, canon, exact, mag, want, k = _case(4)
    w = want[want >= 0]
    kth = w[np.lexsort((-w, canon[w]))[0]]
    outside = np.setdiff1d(cand, w)[0]
    exact = exact.copy()
    exact[outside] = exact[kth]
    got = np.sort(np.concatenate([w[w != kth], [outside]]))
    assert relaxed_topk_check(got, want, cand, canon, exact, mag) == 1


def test_wrong_size_or_order_fails():
    cand, canon, exact, mag, want, k = _case(5)
    with pytest.raises(AssertionError):
        relaxed_topk_check(np.concatenate([want[:-1], [-1]]), want, cand, canon, exact, mag)
    with pytest.raises(AssertionError):
        relaxed_topk_check(want[::-1], want, cand, canon, exact, mag)
