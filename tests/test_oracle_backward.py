"""Pins for the oracle's backward of step D and of the router (CPU only).

The gradients are checked against central finite differences of the forward oracle (which
is pinned on its own), element by element, on tiny inputs, plus closed forms."""
import numpy as np

from oracle import msa_oracle as O

EPS = 1e-6


def _fd(f, args, i, idx):
    ap = [a.copy() for a in args]
    am = [a.copy() for a in args]
    ap[i][idx] += EPS
    am[i][idx] -= EPS
    return (f(*ap) - f(*am)) / (2 * EPS)


def _attn_case(seed, Lq=3, Lkv=5, Hq=4, Hkv=2, D=8, M=6):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((Lq, Hq, D)), rng.standard_normal((Lkv, Hkv, D)),
            rng.standard_normal((Lkv, Hkv, D)), rng.standard_normal((M, Hkv, D)),
            rng.standard_normal((M, Hkv, D)), rng.standard_normal((Lq, Hq, D)))


def test_attention_backward_matches_finite_differences_everywhere():
    for seed, keff, base, scale in ((40, 2, 1e4, None), (41, 7, 1e6, 0.3)):
        Q, Kl, Vl, Km, Vm, dO = _attn_case(seed)
        grads = O.sparse_attention_backward_one(Q, Kl, Vl, Km, Vm, keff, base, dO, scale)

        def loss(Q, Kl, Vl, Km, Vm):
            return float(np.sum(dO * O.sparse_attention_one(Q, Kl, Vl, Km, Vm, keff, base, scale)))

        args = [Q, Kl, Vl, Km, Vm]
        for i, (a, g) in enumerate(zip(args, grads)):
            assert g.shape == a.shape
            for idx in np.ndindex(a.shape):
                assert abs(_fd(loss, args, i, idx) - g[idx]) < 1e-7, (seed, i, idx)


def test_attention_backward_single_visible_key():
    # One local key and no memory: P = 1, so O = V, dV = dO and no gradient reaches Q or K.
    rng = np.random.default_rng(42)
    Q, K, V, dO = (rng.standard_normal(s) for s in ((1, 4, 8), (1, 2, 8), (1, 2, 8), (1, 4, 8)))
    empty = np.zeros((0, 2, 8))
    dQ, dK, dV, dKm, dVm = O.sparse_attention_backward_one(Q, K, V, empty, empty, 3, 1e4, dO)
    assert np.allclose(dQ, 0, atol=1e-15) and np.allclose(dK, 0, atol=1e-15)
    assert np.allclose(dV[0, 0], dO[0, 0] + dO[0, 1]) and np.allclose(dV[0, 1], dO[0, 2] + dO[0, 3])
    assert dKm.shape == (0, 2, 8) and dVm.shape == (0, 2, 8)


def test_attention_backward_bank_rows_sum_over_queries():
    # Two queries both select document 1; the bank gradient is checked by finite differences
    # of the batched forward, so a row used by both queries must receive both contributions.
    rng = np.random.default_rng(43)
    H, Hq, D = 2, 4, 8
    coff = np.array([0, 2, 5, 7])
    Kb, Vb = rng.standard_normal((7, H, D)), rng.standard_normal((7, H, D))
    q_off, kv_off = [0, 2, 5], [0, 3, 7]
    Q, dO = rng.standard_normal((5, Hq, D)), rng.standard_normal((5, Hq, D))
    Kl, Vl = rng.standard_normal((7, H, D)), rng.standard_normal((7, H, D))
    ids = np.array([[1, 0], [2, 1]])
    grads = O.sparse_attn_backward(Q, Kl, Vl, q_off, kv_off, ids, coff, Kb, Vb, 1e4, dO)

    def loss(Q, Kl, Vl, Kb, Vb):
        return float(np.sum(dO * O.sparse_attn(Q, Kl, Vl, q_off, kv_off, ids, coff, Kb, Vb, 1e4)))

    args = [Q, Kl, Vl, Kb, Vb]
    for i, (a, g) in enumerate(zip(args, grads)):
        for idx in np.ndindex(a.shape):
            assert abs(_fd(loss, args, i, idx) - g[idx]) < 1e-7, (i, idx)


def test_route_backward_matches_finite_differences_everywhere():
    rng = np.random.default_rng(44)
    H, D = 3, 6
    coff = np.array([0, 2, 3, 6, 7])
    Kb = rng.standard_normal((7, H, D))
    Qr = rng.standard_normal((5, H, D))
    q_off = [0, 2, 5]
    dD = rng.standard_normal((2, 4))
    dD[1, 2] = 0.0
    dQr, dKb = O.route_backward(Qr, q_off, Kb, coff, dD)

    def loss(Qr, Kb):
        return float(np.sum(dD * O.route_doc_scores(Qr, q_off, Kb, coff)))

    for i, (a, g) in enumerate(zip([Qr, Kb], [dQr, dKb])):
        for idx in np.ndindex(a.shape):
            assert abs(_fd(loss, [Qr, Kb], i, idx) - g[idx]) < 1e-7, (i, idx)


def test_route_backward_reaches_only_the_maximising_pair_and_skips_zero_vectors():
    rng = np.random.default_rng(45)
    H, D = 2, 8
    Kb = rng.standard_normal((4, H, D))
    Kb[3, 1] = 0.0                                   # a zero head vector: cosine 0, no gradient
    Qr = rng.standard_normal((3, H, D))
    coff = np.array([0, 4])
    dQr, dKb = O.route_backward(Qr, [0, 3], Kb, coff, np.array([[2.0]]))
    s = O.token_chunk_scores(Qr, Kb)
    t, c = np.unravel_index(np.argmax(s), s.shape)
    assert np.count_nonzero(np.abs(dQr).sum(axis=(1, 2))) == 1 and np.abs(dQr[t]).sum() > 0
    assert np.count_nonzero(np.abs(dKb).sum(axis=(1, 2))) == 1 and np.abs(dKb[c]).sum() > 0
    if c == 3:
        assert np.all(dKb[3, 1] == 0)
    # a gradient orthogonal to its own vector: scale invariance of the cosine
    for h in range(H):
        assert abs(dQr[t, h] @ Qr[t, h]) < 1e-12
        assert abs(dKb[c, h] @ Kb[c, h]) < 1e-12
