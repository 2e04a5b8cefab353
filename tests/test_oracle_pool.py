"""Pins for the oracle's chunk-mean pooling with document-wise RoPE (CPU only)."""
import numpy as np
import pytest

from oracle import msa_oracle as O
from tests import brute


def _bank(rng, lens, H, D):
    T = int(sum(lens))
    return rng.standard_normal((T, H, D)), rng.standard_normal((T, H, D)), rng.standard_normal((T, H + 1, D))


@pytest.mark.parametrize("mask", [O.ROPE_K, 0, O.ROPE_K | O.ROPE_V | O.ROPE_KR])
def test_pool_matches_brute_force(mask):
    rng = np.random.default_rng(10)
    lens = [1, 5, 9, 17, 4]          # chunk 8: full, partial and single-token chunks
    H, D, chunk, base = 2, 8, 8, 1e4
    K, V, Kr = _bank(rng, lens, H, D)
    off = np.concatenate([[0], np.cumsum(lens)])
    Kb, Vb, Krb, coff = O.pool(K, V, Kr, off, chunk=chunk, base=base, rope_mask=mask)
    assert list(coff) == [0, 1, 2, 4, 7, 8]
    for X, got, bit in ((K, Kb, O.ROPE_K), (V, Vb, O.ROPE_V), (Kr, Krb, O.ROPE_KR)):
        ref = np.array(brute.pool_brute(X, lens, chunk, base, bool(mask & bit)))
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_constant_chunk_is_identity_bit_exact():
    # A chunk whose tokens are all equal pools to that value exactly (V, Kr, and K with
    # no rotation), including after rounding to bf16.
    rng = np.random.default_rng(11)
    v = O.round_to_bf16(rng.standard_normal((1, 2, 16)))
    for L in (1, 3, 64, 100, 128):
        X = np.repeat(v, L, axis=0)
        off = np.array([0, L])
        Kb, Vb, Krb, _ = O.pool(X, X, X[:, :1], off, chunk=64, base=1e6, rope_mask=0)
        for got in (Kb, Vb):
            assert np.array_equal(got, np.repeat(v, got.shape[0], axis=0))
            assert np.array_equal(O.round_to_bf16(got), got)


def test_single_token_document_keeps_k():
    rng = np.random.default_rng(12)
    K = rng.standard_normal((1, 2, 16))
    Kb, _, _, _ = O.pool(K, K, K, np.array([0, 1]), chunk=64, base=1e6, rope_mask=O.ROPE_K)
    assert np.array_equal(Kb, K)


def test_document_wise_positions_restart():
    # The same token content placed as document 0 and as document 3 pools to identical
    # rows: positions restart at 0 in every document.
    rng = np.random.default_rng(13)
    H, D = 2, 16
    docA = rng.standard_normal((150, H, D))
    other = [rng.standard_normal((n, H, D)) for n in (70, 33)]
    K = np.concatenate([docA, other[0], other[1], docA])
    lens = [150, 70, 33, 150]
    off = np.concatenate([[0], np.cumsum(lens)])
    Kb, _, _, coff = O.pool(K, K, K, off, chunk=64, base=1e6, rope_mask=O.ROPE_K)
    assert np.array_equal(Kb[coff[0]:coff[1]], Kb[coff[3]:coff[4]])
    # ...whereas a shared position counter would rotate document 3 differently:
    glob = O.rope_rotate(K, np.arange(len(K)), 1e6)
    assert not np.allclose(glob[off[3]:off[3] + 64].mean(0), Kb[coff[3]])


def test_pool_rotation_before_pooling():
    # Mean of rotated tokens, not rotation of the mean: with two tokens, the pooled K
    # equals (R_0 x0 + R_1 x1)/2.
    rng = np.random.default_rng(14)
    x = rng.standard_normal((2, 1, 8))
    Kb, _, _, _ = O.pool(x, x, x, np.array([0, 2]), chunk=64, base=100.0, rope_mask=O.ROPE_K)
    ref = (np.array(brute.rope_pairs(x[0, 0], 0, 100.0)) + np.array(brute.rope_pairs(x[1, 0], 1, 100.0))) / 2
    np.testing.assert_allclose(Kb[0, 0], ref, atol=1e-14)
