"""Pins for the oracle's context assembly and sparse attention (CPU only)."""
import numpy as np
import torch

from oracle import msa_oracle as O
from tests import brute


def _rot(x, pos, base):
    return np.array([[brute.rope_pairs(x[t, h], int(pos[t]), base) for h in range(x.shape[1])]
                     for t in range(x.shape[0])])


def test_attention_matches_brute_force():
    rng = np.random.default_rng(30)
    Lq, Lkv, Hq, Hkv, D, M = 3, 5, 4, 2, 8, 6
    Q = rng.standard_normal((Lq, Hq, D))
    Kl, Vl = rng.standard_normal((Lkv, Hkv, D)), rng.standard_normal((Lkv, Hkv, D))
    Km, Vm = rng.standard_normal((M, Hkv, D)), rng.standard_normal((M, Hkv, D))
    got = O.sparse_attention_one(Q, Kl, Vl, Km, Vm, 2, 1e4)
    ref = np.array(brute.attention_brute(Q, Kl, Vl, Km, Vm, 2, 1e4))
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_empty_memory_equals_torch_sdpa():
    # With no memory rows the step is causal GQA attention over the rotated local context
    # (query rows aligned to the end of the local keys), checked against PyTorch's SDPA
    # in float64 on the CPU, with the rotation done by the complex-number brute force.
    rng = np.random.default_rng(31)
    Lq, Lkv, Hq, Hkv, D, base, keff = 4, 7, 8, 2, 16, 1e6, 3
    Q = rng.standard_normal((Lq, Hq, D))
    Kl, Vl = rng.standard_normal((Lkv, Hkv, D)), rng.standard_normal((Lkv, Hkv, D))
    empty = np.zeros((0, Hkv, D))
    got = O.sparse_attention_one(Q, Kl, Vl, empty, empty, keff, base)
    qr = _rot(Q, keff + Lkv - Lq + np.arange(Lq), base)
    kr = _rot(Kl, keff + np.arange(Lkv), base)
    mask = torch.tensor(np.arange(Lkv)[None, :] <= (Lkv - Lq + np.arange(Lq))[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(qr).permute(1, 0, 2)[None], torch.tensor(kr).permute(1, 0, 2)[None],
        torch.tensor(Vl).permute(1, 0, 2)[None], attn_mask=mask, enable_gqa=True)
    np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)
    # only relative positions matter once the memory is empty
    got2 = O.sparse_attention_one(Q, Kl, Vl, empty, empty, 40, base)
    np.testing.assert_allclose(got, got2, atol=1e-10)


def test_single_key_and_uniform_weights():
    rng = np.random.default_rng(32)
    D = 8
    Q = rng.standard_normal((1, 2, D))
    Kl, Vl = rng.standard_normal((1, 1, D)), rng.standard_normal((1, 1, D))
    empty = np.zeros((0, 1, D))
    out = O.sparse_attention_one(Q, Kl, Vl, empty, empty, 5, 1e6)
    np.testing.assert_allclose(out[0, 0], Vl[0, 0], atol=1e-15)
    np.testing.assert_allclose(out[0, 1], Vl[0, 0], atol=1e-15)
    # all keys zero -> every logit is 0 -> output is the mean of the visible values
    Lq, Lkv, M = 2, 3, 4
    Q = rng.standard_normal((Lq, 2, D))
    Kl = np.zeros((Lkv, 1, D))
    Vl = rng.standard_normal((Lkv, 1, D))
    Km = np.zeros((M, 1, D))
    Vm = rng.standard_normal((M, 1, D))
    out = O.sparse_attention_one(Q, Kl, Vl, Km, Vm, 1, 1e6)
    for t in range(Lq):
        vis = np.concatenate([Vm[:, 0], Vl[: Lkv - Lq + t + 1, 0]])
        np.testing.assert_allclose(out[t, 0], vis.mean(0), atol=1e-14)


def test_memory_order_invariance_and_assembly():
    rng = np.random.default_rng(33)
    lens = [3, 1, 4, 2]
    coff = np.concatenate([[0], np.cumsum(lens)])
    Hkv, D = 2, 8
    Kb, Vb = rng.standard_normal((10, Hkv, D)), rng.standard_normal((10, Hkv, D))
    Km, Vm = O.assemble_memory(np.array([2, 0, -1]), coff, Kb, Vb)
    assert np.array_equal(Km, np.concatenate([Kb[4:8], Kb[0:3]]))
    Q = rng.standard_normal((2, 4, D))
    Kl, Vl = rng.standard_normal((2, Hkv, D)), rng.standard_normal((2, Hkv, D))
    a = O.sparse_attention_one(Q, Kl, Vl, Km, Vm, 2, 1e6)
    Km2, Vm2 = O.assemble_memory(np.array([0, 2, -1]), coff, Kb, Vb)
    b = O.sparse_attention_one(Q, Kl, Vl, Km2, Vm2, 2, 1e6)
    np.testing.assert_allclose(a, b, atol=1e-13)


def test_gqa_mapping_contiguous_groups():
    # Query heads 0..G-1 read kv head 0, G..2G-1 kv head 1: swapping the two kv heads'
    # inputs swaps the two groups' outputs.
    rng = np.random.default_rng(34)
    Q = rng.standard_normal((2, 4, 8))
    Kl, Vl = rng.standard_normal((2, 2, 8)), rng.standard_normal((2, 2, 8))
    Km, Vm = rng.standard_normal((3, 2, 8)), rng.standard_normal((3, 2, 8))
    a = O.sparse_attention_one(Q, Kl, Vl, Km, Vm, 1, 1e6)
    sw = [1, 0]
    b = O.sparse_attention_one(Q[:, [2, 3, 0, 1]], Kl[:, sw], Vl[:, sw], Km[:, sw], Vm[:, sw], 1, 1e6)
    np.testing.assert_allclose(a[:, [2, 3, 0, 1]], b, atol=1e-13)


def test_sparse_attn_multi_query_offsets():
    rng = np.random.default_rng(35)
    lens = [2, 3, 1]
    coff = np.concatenate([[0], np.cumsum(lens)])
    Kb, Vb = rng.standard_normal((6, 1, 8)), rng.standard_normal((6, 1, 8))
    q_off, kv_off = np.array([0, 2, 3]), np.array([0, 4, 6])
    Q = rng.standard_normal((3, 2, 8))
    Kl, Vl = rng.standard_normal((6, 1, 8)), rng.standard_normal((6, 1, 8))
    ids = np.array([[2, 0], [1, -1]])
    out = O.sparse_attn(Q, Kl, Vl, q_off, kv_off, ids, coff, Kb, Vb, 1e6)
    Km, Vm = O.assemble_memory(ids[1], coff, Kb, Vb)
    ref = O.sparse_attention_one(Q[2:3], Kl[4:6], Vl[4:6], Km, Vm, 1, 1e6)
    np.testing.assert_allclose(out[2:3], ref, atol=0)


def test_lse_matches_brute_force():
    # each row's log-sum-exp of its logits against the explicit-loop attention
    rng = np.random.default_rng(34)
    Lq, Lkv, Hq, Hkv, D, M = 3, 6, 4, 2, 8, 5
    Q = rng.standard_normal((Lq, Hq, D))
    Kl, Vl = rng.standard_normal((Lkv, Hkv, D)), rng.standard_normal((Lkv, Hkv, D))
    Km, Vm = rng.standard_normal((M, Hkv, D)), rng.standard_normal((M, Hkv, D))
    out, lse = O.sparse_attention_one(Q, Kl, Vl, Km, Vm, 3, 1e4, with_lse=True)
    ref_out, ref_lse = brute.attention_brute(Q, Kl, Vl, Km, Vm, 3, 1e4, with_lse=True)
    np.testing.assert_allclose(lse, np.array(ref_lse), atol=1e-12)
    np.testing.assert_allclose(out, np.array(ref_out), atol=1e-12)


def test_lse_closed_forms():
    rng = np.random.default_rng(35)
    D = 16
    empty = np.zeros((0, 1, D))
    # one query token that sees only its own key: query and key are rotated by the same
    # angles, so the single logit, and hence the log-sum-exp, is scale * q . k
    Q = rng.standard_normal((1, 2, D))
    Kl, Vl = rng.standard_normal((1, 1, D)), rng.standard_normal((1, 1, D))
    _, lse = O.sparse_attention_one(Q, Kl, Vl, empty, empty, 7, 1e6, with_lse=True)
    for h in range(2):
        assert abs(lse[0, h] - float(Q[0, h] @ Kl[0, 0]) / np.sqrt(D)) < 1e-12
    # all keys zero: every logit is 0, so the log-sum-exp is log(number of visible keys)
    Lq, Lkv, M = 3, 5, 4
    Q = rng.standard_normal((Lq, 1, D))
    _, lse = O.sparse_attention_one(Q, np.zeros((Lkv, 1, D)), rng.standard_normal((Lkv, 1, D)),
                                    np.zeros((M, 1, D)), rng.standard_normal((M, 1, D)), 2, 1e6, with_lse=True)
    for t in range(Lq):
        assert abs(lse[t, 0] - np.log(M + Lkv - Lq + t + 1)) < 1e-12


def test_sparse_attn_lse_per_query():
    # the batched form equals the per-query one, memory assembled from each query's ids
    rng = np.random.default_rng(36)
    q_len, kv_len, Hq, Hkv, D = [2, 3], [4, 3], 4, 2, 8
    q_off, kv_off = np.array([0, 2, 5]), np.array([0, 4, 7])
    coff = np.array([0, 2, 3, 6])
    Q = rng.standard_normal((5, Hq, D))
    Kl, Vl = rng.standard_normal((7, Hkv, D)), rng.standard_normal((7, Hkv, D))
    Kb, Vb = rng.standard_normal((6, Hkv, D)), rng.standard_normal((6, Hkv, D))
    ids = np.array([[2, -1], [0, 1]])
    got = O.sparse_attn_lse(Q, Kl, Vl, q_off, kv_off, ids, coff, Kb, Vb, 1e6)
    for b, rows in enumerate(([3, 4, 5], [0, 1, 2])):
        _, ref = brute.attention_brute(Q[q_off[b]:q_off[b + 1]], Kl[kv_off[b]:kv_off[b + 1]],
                                       Vl[kv_off[b]:kv_off[b + 1]], Kb[rows], Vb[rows], 1 + b, 1e6, with_lse=True)
        np.testing.assert_allclose(got[q_off[b]:q_off[b + 1]], np.array(ref), atol=1e-12)
