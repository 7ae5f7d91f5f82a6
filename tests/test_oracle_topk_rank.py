"""Pins of the oracle's rank-component top-k proxy update (the reading of the
pages' top-k as a selection over the r rank components of the adapter).

  * a component's score is the largest |element| of its rank-1 term, checked
    against the explicit outer product;
  * the selection is the k largest scores, ties to the lower index (planted
    ties, brute force over all subsets for a tiny r);
  * k = r reduces to the plain row-wise proxy update (same chain order);
  * k = 0 merges nothing; merged rows zero only the selected components;
  * the merged delta equals the explicit sum over the selected components.
"""
import itertools

import numpy as np

import oracle
from oracle import e4m3


def small(seed, d_out=24, d_in=32, r=6):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    wq, s_w, _, _ = oracle.fp8_quantize(W)
    A = (rng.standard_normal((r, d_in)) / np.sqrt(r)).astype(np.float32)
    B = (rng.standard_normal((d_out, r)) * 10.0 ** rng.uniform(-5, -2, r)).astype(np.float32)
    return wq, s_w, A, B


def test_scores_are_the_largest_element_of_each_rank1_term():
    _, _, A, B = small(1)
    c = oracle.component_scores(A, B)
    for j in range(A.shape[0]):
        term = np.outer(B[:, j].astype(np.float64), A[j].astype(np.float64))
        assert c[j] == np.max(np.abs(term))


def test_selection_brute_force_and_ties():
    _, _, A, B = small(2, r=5)
    B[:, 3] = B[:, 1] * 1.0          # planted tie between components 1 and 3
    A[3] = A[1]
    c = oracle.component_scores(A, B)
    assert c[1] == c[3]
    for k in range(6):
        K = oracle.select_components(A, B, k)
        best = None
        for sub in itertools.combinations(range(5), k):
            key = (sorted((-c[j], j) for j in sub))
            if best is None or key < best[0]:
                best = (key, sub)
        assert tuple(K) == tuple(sorted(best[1])), (k, K, best)
    K2 = oracle.select_components(A, B, 2)
    if 1 in K2 or 3 in K2:
        assert not (3 in K2 and 1 not in K2)    # the lower index wins the tie


def test_k_equals_r_is_the_plain_update():
    wq, s_w, A, B = small(3)
    ref = oracle.rowwise_proxy_update(wq, s_w, A, B, 0.5, 0)
    got = oracle.rowwise_proxy_update_topk_rank(wq, s_w, A, B, A.shape[0], 0.5, 0)
    for a, b in zip(ref, got[:4]):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    assert np.array_equal(got[4], np.arange(A.shape[0]))


def test_k_zero_merges_nothing():
    wq, s_w, A, B = small(4)
    wq2, B2, sel, rho, K = oracle.rowwise_proxy_update_topk_rank(wq, s_w, A, B, 0, 0.5, 0)
    assert K.size == 0 and sel.size == 0 and not rho.any()
    assert np.array_equal(wq2, wq) and np.array_equal(B2, B)


def test_merged_rows_and_delta_use_only_the_selected_components():
    wq, s_w, A, B = small(5, d_out=40, r=8)
    k = 3
    wq2, B2, sel, rho, K = oracle.rowwise_proxy_update_topk_rank(wq, s_w, A, B, k, 0.25, 0)
    assert sel.size > 0
    rest = np.setdiff1d(np.arange(A.shape[0]), K)
    # selected rows: components K zeroed, the others untouched; other rows untouched
    assert not B2[np.ix_(sel, K)].any()
    assert np.array_equal(B2[:, rest], B[:, rest])
    unsel = np.setdiff1d(np.arange(B.shape[0]), sel)
    assert np.array_equal(B2[unsel], B[unsel]) and np.array_equal(wq2[unsel], wq[unsel])
    # the merged value is dec + fl(s_w * u) with u the sum over K, to one code
    u = (B[sel][:, K].astype(np.float64) @ A[K].astype(np.float64))
    v = e4m3.decode(wq[sel]) + float(s_w) * u
    back = e4m3.decode(wq2[sel])
    assert np.all(np.abs(back - v) <= e4m3.step_of(np.abs(v)) * 0.5 + 1e-3 * np.abs(v) + 1e-6)
