"""Pins for the oracle's router scores and top-k selection (CPU only)."""
import numpy as np
import pytest

from oracle import msa_oracle as O
from tests import brute


def _tiny(seed, T=3, H=2, D=8, n_chunks=(2, 1, 3, 1)):
    rng = np.random.default_rng(seed)
    C = sum(n_chunks)
    Qr = rng.standard_normal((T, H, D))
    Kb = rng.standard_normal((C, H, D))
    off = np.concatenate([[0], np.cumsum(n_chunks)])
    return Qr, Kb, off


def test_doc_scores_match_brute_force():
    for seed in range(5):
        Qr, Kb, off = _tiny(seed)
        got = O.doc_scores_one(Qr, Kb, off)
        ref = brute.doc_scores_brute(Qr, Kb, off)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_cosine_range_and_aligned_extremes():
    Qr, Kb, off = _tiny(20, T=4, H=3, D=16, n_chunks=(3, 2, 5))
    s = O.token_chunk_scores(Qr, Kb)
    assert np.all(s <= 1 + 1e-12) and np.all(s >= -1 - 1e-12)
    # Query token 2 equal to +lambda times chunk 4 in every head: score exactly 1 there,
    # and the document owning chunk 4 ranks first.
    Q2 = Qr.copy()
    Q2[2] = 3.5 * Kb[4]
    s2 = O.token_chunk_scores(Q2, Kb)
    assert abs(s2[2, 4] - 1.0) < 1e-14
    D = O.doc_scores_one(Q2, Kb, off)
    assert O.topk_docs(D, 1)[0][0] == 1
    Q3 = Qr.copy()
    Q3[1] = -0.25 * Kb[0]
    assert abs(O.token_chunk_scores(Q3, Kb)[1, 0] + 1.0) < 1e-14


def test_zero_norm_gives_zero_cosine():
    Qr, Kb, off = _tiny(21, H=2)
    Kb[1, 0] = 0.0                  # head 0 of chunk 1 is a zero vector
    cos = O.head_cosines(Qr, Kb)
    assert np.all(cos[:, 1, 0] == 0.0)
    Qr[0, 1] = 0.0
    assert np.all(O.head_cosines(Qr, Kb)[0, :, 1] == 0.0)
    assert np.all(np.isfinite(O.doc_scores_one(Qr, Kb, off)))


def test_score_invariances():
    rng = np.random.default_rng(22)
    Qr, Kb, off = _tiny(22, T=5, H=4, D=8, n_chunks=(2, 3, 1, 4))
    D0 = O.doc_scores_one(Qr, Kb, off)
    # positive rescaling of any single head vector
    Kb2 = Kb * rng.uniform(0.1, 10.0, size=Kb.shape[:2])[..., None]
    Qr2 = Qr * rng.uniform(0.1, 10.0, size=Qr.shape[:2])[..., None]
    np.testing.assert_allclose(O.doc_scores_one(Qr2, Kb2, off), D0, atol=1e-13)
    # joint permutation of heads, permutation of query tokens
    ph = rng.permutation(4)
    np.testing.assert_allclose(O.doc_scores_one(Qr[:, ph], Kb[:, ph], off), D0, atol=1e-13)
    np.testing.assert_allclose(O.doc_scores_one(Qr[rng.permutation(5)], Kb, off), D0, atol=1e-13)
    # permuting chunks inside a document does not change its score
    Kb3 = Kb.copy()
    Kb3[off[1]:off[2]] = Kb[off[1]:off[2]][::-1]
    np.testing.assert_allclose(O.doc_scores_one(Qr, Kb3, off), D0, atol=1e-13)


def test_head_mean_not_concatenated_cosine():
    # The router averages per-head cosines; the cosine of the concatenated heads is a
    # different number when head norms differ.
    Qr, Kb, off = _tiny(23, T=1, H=2, D=4, n_chunks=(1,))
    Kb[0, 1] *= 100.0
    s = O.token_chunk_scores(Qr, Kb)[0, 0]
    q, k = Qr[0].ravel(), Kb[0].ravel()
    concat = q @ k / np.linalg.norm(q) / np.linalg.norm(k)
    assert abs(s - concat) > 1e-3
    per = [Qr[0, h] @ Kb[0, h] / np.linalg.norm(Qr[0, h]) / np.linalg.norm(Kb[0, h]) for h in range(2)]
    assert abs(s - np.mean(per)) < 1e-14


def test_topk_matches_lexsort_and_rank_counting():
    rng = np.random.default_rng(24)
    for trial in range(20):
        N = int(rng.integers(1, 40))
        sc = np.round(rng.standard_normal(N), 1)        # rounding creates ties
        k = int(rng.integers(1, 45))
        ids, vals = O.topk_docs(sc, k)
        order = np.lexsort((np.arange(N), -sc))
        keff = min(k, N)
        assert list(ids[:keff]) == list(order[:keff])
        assert list(ids) == brute.topk_brute(list(sc), k)
        assert np.all(ids[keff:] == -1) and np.all(np.isneginf(vals[keff:]))
        np.testing.assert_array_equal(vals[:keff], sc[order[:keff]])


def test_topk_ties_lowest_id_and_permutation_equivariance():
    sc = np.array([0.5, 0.9, 0.5, 0.9, 0.1])
    ids, _ = O.topk_docs(sc, 3)
    assert list(ids) == [1, 3, 0]
    rng = np.random.default_rng(25)
    sc = rng.standard_normal(30)                         # distinct scores
    perm = rng.permutation(30)
    ids, _ = O.topk_docs(sc, 7)
    ids_p, _ = O.topk_docs(sc[perm], 7)                  # document i of the new order is perm[i]
    assert list(perm[ids_p]) == list(ids)
    with pytest.raises(ValueError):
        O.topk_docs(sc, 0)


def test_route_duplicate_documents_tie_to_lower_id():
    Qr, Kb, off = _tiny(26, n_chunks=(2, 3, 2))
    Kb[5:7] = Kb[0:2]                                    # document 2 duplicates document 0
    ids, vals, D = O.route(Qr, np.array([0, 3]), Kb, off, k=3)
    assert D[0, 0] == D[0, 2]
    assert list(ids[0]).index(0) < list(ids[0]).index(2)


def test_route_blocking_is_exact():
    rng = np.random.default_rng(27)
    lens = rng.integers(1, 9, size=40)
    off = np.concatenate([[0], np.cumsum(lens)])
    Kb = rng.standard_normal((off[-1], 2, 8))
    Qr = rng.standard_normal((7, 2, 8))
    q_off = np.array([0, 3, 7])
    a = O.route_doc_scores(Qr, q_off, Kb, off)
    b = O.route_doc_scores(Qr, q_off, Kb, off, block=13)
    assert np.array_equal(a, b)


def test_empty_query_is_the_identity_of_the_token_max():
    # Scores of a token set are the max over its tokens, so scores(A u B) = max(scores(A),
    # scores(B)) for any split; with B empty this forces scores(empty) = -inf (R25), and the
    # top-k of an all -inf row is the k lowest ids by the tie rule.
    Qr, Kb, off = _tiny(28, T=5, n_chunks=(2, 1, 3, 1, 2))
    whole = O.doc_scores_one(Qr, Kb, off)
    for cut in range(0, 6):
        a = O.doc_scores_one(Qr[:cut], Kb, off)
        b = O.doc_scores_one(Qr[cut:], Kb, off)
        assert np.array_equal(np.maximum(a, b), whole)
    empty = O.doc_scores_one(Qr[:0], Kb, off)
    assert np.all(np.isneginf(empty))
    q_off = np.array([0, 2, 2, 5])                         # the middle query has no tokens
    ids, vals, D = O.route(Qr, q_off, Kb, off, k=3)
    assert list(ids[1]) == [0, 1, 2] and np.all(np.isneginf(vals[1]))
    assert np.array_equal(D[0], O.doc_scores_one(Qr[:2], Kb, off))
    assert np.array_equal(D[2], O.doc_scores_one(Qr[2:], Kb, off))
