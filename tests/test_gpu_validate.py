"""Opt-in validation of the device index arrays (MSA_DEBUG_VALIDATE=1).

With validation on, valid inputs give the same bits as without it, and each kind of bad
offset or id array is refused with MSA_ERR_INVALID_ARG and a message naming the entry.
Every bad case here would also be harmless if a kernel did run on it (short or empty
ranges, ids that read as unused), so a validation bug cannot turn into a bad access."""
import numpy as np
import pytest
import torch

import latent_memory_long_amd as M
from tests.helpers import as_keys, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("MSA_DEBUG_VALIDATE", "1")


def _i64(x):
    return torch.tensor(np.asarray(x, dtype=np.int64), device=DEV)


def _i32(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), device=DEV)


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16).to(DEV)


def _refused(fn, needle):
    with pytest.raises(M.MsaError) as e:
        fn()
    assert e.value.status == M.MSA_ERR_INVALID_ARG, e.value
    assert needle in e.value.message, e.value.message
    say(f"  refused: {e.value.message}")


def _setup():
    lens = [70, 5, 130]
    off = np.concatenate([[0], np.cumsum(lens)])
    coff = M.msa_chunk_offsets(off, 64)
    K, V, Kr = _rand((off[-1], 2, 64), 1), _rand((off[-1], 2, 64), 2), _rand((off[-1], 4, 64), 3)
    return lens, off, coff, K, V, Kr


def test_valid_inputs_unchanged(validate, monkeypatch):
    say("case validation on: valid inputs give the same bits")
    lens, off, coff, K, V, Kr = _setup()
    C = int(coff[-1])
    on = M.msa_pool(K, V, Kr, _i64(off), _i64(coff), C)
    Qr = _rand((9, 4, 64), 4)
    q_off = _i32([0, 6, 9])
    ids_on, sc_on, ds_on = M.msa_route_topk(Qr, q_off, 6, on[2], _i64(coff), 2, want_doc_scores=True)
    Q, Kl, Vl = _rand((9, 8, 64), 5), _rand((12, 2, 64), 6), _rand((12, 2, 64), 7)
    kv_off = _i32([0, 8, 12])
    o_on = M.msa_sparse_attn(Q, Kl, Vl, q_off, kv_off, 6, ids_on, _i64(coff), on[0], on[1])
    monkeypatch.delenv("MSA_DEBUG_VALIDATE")
    off_ = M.msa_pool(K, V, Kr, _i64(off), _i64(coff), C)
    ids, sc, ds = M.msa_route_topk(Qr, q_off, 6, off_[2], _i64(coff), 2, want_doc_scores=True)
    o = M.msa_sparse_attn(Q, Kl, Vl, q_off, kv_off, 6, ids, _i64(coff), off_[0], off_[1])
    torch.cuda.synchronize()
    for a, b in zip(on + (ids_on, sc_on, ds_on, o_on), off_ + (ids, sc, ds, o)):
        assert a.equal(b) if isinstance(a, M.RouteKeys) else torch.equal(a, b)


def test_pool_offsets_refused(validate):
    say("case validation: bad pool offsets")
    lens, off, coff, K, V, Kr = _setup()
    C = int(coff[-1])
    # a document without tokens (its row range is empty too)
    off0 = np.array([0, 70, 70, 205])
    coff0 = np.array([0, 2, 2, 5])
    _refused(lambda: M.msa_pool(K, V, Kr, _i64(off0), _i64(coff0), 5), "doc_tok_off[2]")
    # offsets that stop short of the token count
    short = np.array([0, 70, 75, 200])
    _refused(lambda: M.msa_pool(K, V, Kr, _i64(short), _i64(M.msa_chunk_offsets(short, 64)), C),
             "doc_tok_off[3] is 200, not 205")


def test_route_offsets_refused(validate):
    say("case validation: bad routing offsets")
    lens, off, coff, K, V, Kr = _setup()
    Krb = as_keys(_rand((int(coff[-1]), 4, 64), 8))
    Qr = _rand((9, 4, 64), 9)
    # a query longer than max_q_len
    _refused(lambda: M.msa_route_scan(Qr, _i32([0, 6, 9]), 4, Krb, _i64(coff)), "more than max_q_len 4")
    # query offsets that stop short of total_q
    _refused(lambda: M.msa_route_scan(Qr, _i32([0, 3, 8]), 6, Krb, _i64(coff)), "q_off[2] is 8, not 9")
    # a document without rows
    _refused(lambda: M.msa_route_topk(Qr, _i32([0, 6, 9]), 6, Krb, _i64([0, 2, 2, 6]), 2), "chunk_off[2]")


def test_attention_inputs_refused(validate):
    say("case validation: bad attention inputs")
    lens, off, coff, K, V, Kr = _setup()
    C = int(coff[-1])
    Kb, Vb = _rand((C, 2, 64), 10), _rand((C, 2, 64), 11)
    Q, Kl, Vl = _rand((9, 8, 64), 12), _rand((12, 2, 64), 13), _rand((12, 2, 64), 14)
    q_off, kv_off = _i32([0, 6, 9]), _i32([0, 8, 12])
    # an id below -1 (a kernel reads any negative id as an unused slot)
    _refused(lambda: M.msa_sparse_attn(Q, Kl, Vl, q_off, kv_off, 6, _i32([[0, 2], [1, -2]]), _i64(coff), Kb, Vb),
             "topk_ids[1][1] = -2")
    # fewer local tokens than query tokens
    _refused(lambda: M.msa_sparse_attn(Q, Kl, Vl, q_off, _i32([0, 5, 12]), 6, _i32([[0, 2], [1, -1]]), _i64(coff),
                                       Kb, Vb), "query 0: 5 local tokens")
