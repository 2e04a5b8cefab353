"""The router entry point for callers that cannot allocate (msa_route_topk_noalloc, scratch in
the library's per-device array) gives the results of msa_route_topk with a workspace: twice
in a row on the same device, the second call with a smaller input, and it refuses inputs
whose scratch would not fit."""
import numpy as np
import pytest
import torch

import latent_memory_long_amd as M
from oracle import msa_oracle as O
from tests.helpers import as_keys, assert_scores_close, assert_topk_consistent, assert_topk_valid, f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bank(n_docs, heads, d, seed):
    rng = np.random.default_rng(seed)
    counts = rng.integers(1, 30, size=n_docs)
    coff = np.concatenate([[0], np.cumsum(counts)])
    g = torch.Generator().manual_seed(seed)
    mu = torch.randn((n_docs, heads, d), generator=g) * 0.5
    rows = torch.randn((int(coff[-1]), heads, d), generator=g) * 0.125
    rows += torch.repeat_interleave(mu, torch.as_tensor(counts), dim=0)
    return coff, rows.to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("want_doc_scores", [False, True], ids=["scores-in-scratch", "scores-given"])
def test_noalloc_matches_route_topk(want_doc_scores):
    cases = [(3000, [64, 17, 1], 16, 401), (700, [5], 8, 402)]   # the second call: a smaller input
    for n_docs, q_lens, k, seed in cases:
        say(f"case no-alloc router: {n_docs} docs, queries {q_lens}, k {k}, doc scores given {want_doc_scores}")
        coff, rows = _bank(n_docs, 8, 128, seed)
        keys = as_keys(rows)
        Qr = torch.randn((sum(q_lens), 8, 128), generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
        q_off = np.concatenate([[0], np.cumsum(q_lens)])
        q_off_d = torch.tensor(q_off, dtype=torch.int32, device=DEV)
        coff_d = torch.tensor(coff, device=DEV)
        Qd = Qr.to(DEV)
        ids_a, sc_a, ds_a = M.msa_route_topk(Qd, q_off_d, max(q_lens), keys, coff_d, k, want_doc_scores=True)
        ids_b, sc_b, ds_b = M.msa_route_topk_noalloc(Qd, q_off_d, max(q_lens), keys, coff_d, k,
                                                     want_doc_scores=want_doc_scores)
        torch.cuda.synchronize()
        assert torch.equal(ids_a, ids_b) and torch.equal(sc_a, sc_b), "top-k differs from msa_route_topk"
        if want_doc_scores:
            assert torch.equal(ds_a, ds_b), "document scores differ from msa_route_topk"
        o = O.route_doc_scores(f64(Qr), q_off, f64(rows), coff)
        for b in range(len(q_lens)):
            assert_scores_close(ds_a.cpu().numpy()[b], o[b], "bf16", f"query {b}")
            assert_topk_consistent(ids_b.cpu().numpy()[b], sc_b.cpu().numpy()[b], ds_a.cpu().numpy()[b], k, f"query {b}")
            assert_topk_valid(ids_b.cpu().numpy()[b], o[b], k, f"query {b}")


def test_noalloc_refuses_inputs_beyond_its_scratch():
    # 8 queries x 600,000 one-row documents need 19.2 MB of document scores: refused on the
    # host before any kernel runs
    say("case no-alloc router: input beyond the scratch array")
    n_docs, B = 600_000, 8
    coff = torch.arange(n_docs + 1, dtype=torch.int64, device=DEV)
    keys = M.RouteKeys.empty(n_docs, 1, 32, torch.bfloat16, DEV, zero=True)
    Qr = torch.zeros((B, 1, 32), dtype=torch.bfloat16, device=DEV)
    q_off = torch.arange(B + 1, dtype=torch.int32, device=DEV)
    with pytest.raises(M.MsaError) as e:
        M.msa_route_topk_noalloc(Qr, q_off, 1, keys, coff, 4)
    assert e.value.status == M.MSA_ERR_WORKSPACE and "more than the" in e.value.message
    # with the scores given, only the top-k candidates use the scratch: accepted
    ids, sc, ds = M.msa_route_topk_noalloc(Qr, q_off, 1, keys, coff, 4, want_doc_scores=True)
    torch.cuda.synchronize()
    assert ids.shape == (B, 4)
