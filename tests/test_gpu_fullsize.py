"""GPU parity at the full workload sizes, in the launch configurations the benchmark uses.

Every document score of the 10M- and 100M-token banks (and of eight of the 32 batched
queries, the longest among them) is compared with the oracle, scored on host threads
group by group, and the top-k set with the oracle's full ranking.  Pooled rows are
compared for sampled documents (pooling 10M tokens in float64 would take minutes), and
attention for every query.  Exact properties are checked as well: the top-k is the
(score desc, id asc) order of the GPU's own document scores, and planted needles are
recalled (10M-token bank, and the 100M-token bank's routing keys).
"""
import gc

import numpy as np
import pytest
import torch

import latent_memory_long_amd as M
from oracle import msa_oracle as O
from synth import workloads as W
from tests.helpers import (as_keys, assert_attn_close, assert_pool_close, key_rows, pool_error_bound,
                           assert_scores_close, assert_topk_consistent, assert_topk_valid, f64,
                           oracle_doc_scores_all, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def sample_docs(n_docs, seed, extra=()):
    rng = np.random.default_rng(seed)
    pick = set([0, 1, 2, n_docs - 3, n_docs - 2, n_docs - 1])
    pick |= set(int(x) for x in rng.choice(n_docs, size=min(n_docs, 40), replace=False))
    pick |= set(int(x) for x in extra)
    return sorted(d for d in pick if 0 <= d < n_docs)


def check_pool_sample(K, V, Kr, off, coff, Kb, Vb, Krb, docs, chunk, base, what):
    """Pool the sampled documents with the oracle and compare their bank rows."""
    Krb = key_rows(Krb)
    for d in docs:
        t0, t1 = int(off[d]), int(off[d + 1])
        c0, c1 = int(coff[d]), int(coff[d + 1])
        xs = (f64(K[t0:t1]), f64(V[t0:t1]), f64(Kr[t0:t1]))
        oK, oV, oKr, _ = O.pool(*xs, [0, t1 - t0], chunk, base, O.ROPE_K)
        for g, o, x, rot, n in ((Kb[c0:c1], oK, xs[0], True, "Kbar"), (Vb[c0:c1], oV, xs[1], False, "Vbar"),
                                (Krb[c0:c1], oKr, xs[2], False, "Krbar")):
            assert_pool_close(g, o, "bf16", f"{what} doc {d} {n}", pool_error_bound(x, [0, t1 - t0], chunk, rot))


def token_bank(wl, needle_q=None):
    sh = wl.shape
    lens = W.doc_lengths(wl)
    off = W.token_offsets(lens)
    coff = M.msa_chunk_offsets(off, sh.chunk)
    needle_ids = None
    dirs = None
    if needle_q is not None:
        needle_ids, dirs = W.plant_needles(wl, len(lens), needle_q)
    K, V, Kr = W.gen_token_states(wl, lens, DEV, needle_dirs=dirs, needle_ids=needle_ids)
    return lens, off, coff, K, V, Kr, needle_ids


def run_pool(wl, off, coff, K, V, Kr):
    sh = wl.shape
    return M.msa_pool(K, V, Kr, torch.tensor(off, device=DEV), torch.tensor(coff, device=DEV),
                      int(coff[-1]), sh.chunk, sh.rope_base)


def run_route(q, coff, Krb, k, ws=None):
    q_len = q["q_len"]
    steps = q["decode_steps"]
    B = len(q_len)
    # prefill rows of every query (decode rows, if any, follow each query's prefill rows)
    rows, q_off = [], [0]
    start = 0
    for b in range(B):
        rows.append(q["Qr"][start:start + int(q_len[b])])
        q_off.append(q_off[-1] + int(q_len[b]))
        start += int(q_len[b]) + steps
    Qr = torch.cat(rows).contiguous()
    q_off_d = torch.tensor(q_off, dtype=torch.int32, device=DEV)
    ids, sc, ds = M.msa_route_topk(Qr, q_off_d, int(max(q_len)), Krb, torch.tensor(coff, device=DEV), k,
                                   want_doc_scores=True)
    torch.cuda.synchronize()
    return Qr, np.array(q_off), ids, sc.cpu().numpy(), ds.cpu().numpy()


def attn_check(q, ids, coff, Kb, Vb, rope_base, queries, what):
    """Attention of the prefill rows (local context = the query itself) vs the oracle."""
    q_len = q["q_len"]
    kv_len = q["kv_len"]
    B = len(q_len)
    # per query: its prefill rows of Q (Q holds prefill then decode rows) and the first
    # q_len rows of its local K/V, so the local context is the query's own tokens
    q_src = np.concatenate([[0], np.cumsum(kv_len)])
    rows_q, rows_k, rows_v, q_off = [], [], [], [0]
    for b in range(B):
        L = int(q_len[b])
        s0 = int(q_src[b])
        rows_q.append(q["Q"][s0:s0 + L])
        rows_k.append(q["Kloc"][s0:s0 + L])
        rows_v.append(q["Vloc"][s0:s0 + L])
        q_off.append(q_off[-1] + L)
    Q = torch.cat(rows_q).contiguous()
    Kl = torch.cat(rows_k).contiguous()
    Vl = torch.cat(rows_v).contiguous()
    q_off_d = torch.tensor(q_off, dtype=torch.int32, device=DEV)
    out = M.msa_sparse_attn(Q, Kl, Vl, q_off_d, q_off_d, int(max(q_len)), ids, torch.tensor(coff, device=DEV),
                            Kb, Vb, rope_base=rope_base)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    # the oracle sees only the selected documents' rows: gather them into a compact bank
    for b in queries:
        sel = [int(d) for d in ids_h[b] if d >= 0]
        idx = np.concatenate([np.arange(coff[d], coff[d + 1]) for d in sel])
        kb = f64(Kb[torch.as_tensor(idx, device=Kb.device)])
        vb = f64(Vb[torch.as_tensor(idx, device=Vb.device)])
        cnt = [int(coff[d + 1] - coff[d]) for d in sel]
        coff_c = np.concatenate([[0], np.cumsum(cnt)])
        ids_c = np.arange(len(sel), dtype=np.int32)[None]
        ref = O.sparse_attn(f64(Q[q_off[b]:q_off[b + 1]]), f64(Kl[q_off[b]:q_off[b + 1]]),
                            f64(Vl[q_off[b]:q_off[b + 1]]), [0, int(q_len[b])], [0, int(q_len[b])],
                            ids_c, coff_c, kb, vb, rope_base)
        err = assert_attn_close(out[q_off[b]:q_off[b + 1]], ref, "bf16", f"{what} query {b}")
        say(f"  {what} query {b}: attention max abs err {err:.3g}")
    return out


def test_bank1m_full():
    say("case full-size bank1m: pool, route (all documents), attention")
    wl = W.workload("bank1m")
    sh = wl.shape
    lens, off, coff, K, V, Kr, _ = token_bank(wl)
    Kb, Vb, Krb = run_pool(wl, off, coff, K, V, Kr)
    torch.cuda.synchronize()
    check_pool_sample(K, V, Kr, off, coff, Kb, Vb, Krb, sample_docs(len(lens), 1)[:12], sh.chunk,
                      sh.rope_base, "bank1m")
    q = W.gen_queries(wl, DEV)
    Qr, q_off, ids, sc, ds = run_route(q, coff, Krb, wl.k)
    o = O.route_doc_scores(f64(Qr), q_off, f64(Krb), coff, block=8192)[0]
    err = assert_scores_close(ds[0], o, "bf16", "bank1m all doc scores")
    say(f"  bank1m: {len(lens)} docs, score max rel err {err:.3g}")
    assert_topk_consistent(ids.cpu().numpy()[0], sc[0], ds[0], wl.k, "bank1m")
    assert_topk_valid(ids.cpu().numpy()[0], o, wl.k, "bank1m")
    attn_check(q, ids, coff, Kb, Vb, sh.rope_base, [0], "bank1m")


def test_bank10m_needles_full():
    say("case full-size bank10m_needles: pool sample, route sample, needle recall, attention")
    wl = W.workload("bank10m_needles")
    sh = wl.shape
    q = W.gen_queries(wl, DEV)
    Lq = int(q["q_len"][0])
    lens, off, coff, K, V, Kr, needles = token_bank(wl, needle_q=q["Qr"][:Lq])
    Kb, Vb, Krb = run_pool(wl, off, coff, K, V, Kr)
    torch.cuda.synchronize()
    docs = sample_docs(len(lens), 2, extra=needles)
    check_pool_sample(K, V, Kr, off, coff, Kb, Vb, Krb, docs[:10] + list(needles), sh.chunk, sh.rope_base,
                      "bank10m")
    del K, V, Kr
    gc.collect()
    torch.cuda.empty_cache()
    Qr, q_off, ids, sc, ds = run_route(q, coff, Krb, wl.k)
    ids_h = ids.cpu().numpy()[0]
    assert_topk_consistent(ids_h, sc[0], ds[0], wl.k, "bank10m")
    o = oracle_doc_scores_all(Qr, q_off, Krb, coff, what="bank10m")[0]
    err = assert_scores_close(ds[0], o, "bf16", "bank10m every document score")
    assert_topk_valid(ids_h, o, wl.k, "bank10m top-k vs the oracle's ranking")
    recalled = set(int(x) for x in needles) & set(int(x) for x in ids_h)
    say(f"  bank10m: needles {list(needles)} recalled {len(recalled)}/5; every score, max rel err {err:.3g}")
    assert len(recalled) == len(needles)
    attn_check(q, ids, coff, Kb, Vb, sh.rope_base, [0], "bank10m")


def test_bank100m_host_full():
    say("case full-size bank100m_host: pooled bank, route sample, host-sourced attention, decode")
    wl = W.workload("bank100m_host")
    sh = wl.shape
    lens = W.doc_lengths(wl)
    off = W.token_offsets(lens)
    coff = M.msa_chunk_offsets(off, sh.chunk)
    Krb_rows, Kb, Vb = W.gen_pooled_bank(wl, coff, DEV, kv_device="cpu-pinned")
    assert Kb.is_pinned() and not Kb.is_cuda
    Krb = as_keys(Krb_rows)
    Krb_rows = Krb_rows.cpu()   # the oracle's copy of the rows, in host memory
    torch.cuda.empty_cache()
    q = W.gen_queries(wl, DEV)
    Qr, q_off, ids, sc, ds = run_route(q, coff, Krb, wl.k)
    ids_h = ids.cpu().numpy()[0]
    assert_topk_consistent(ids_h, sc[0], ds[0], wl.k, "bank100m")
    o = oracle_doc_scores_all(Qr, q_off, Krb_rows, coff, what="bank100m")[0]
    err = assert_scores_close(ds[0], o, "bf16", "bank100m every document score")
    assert_topk_valid(ids_h, o, wl.k, "bank100m top-k vs the oracle's ranking")
    say(f"  bank100m: {len(lens)} docs, {int(coff[-1])} rows; every score, max rel err {err:.3g}")
    attn_check(q, ids, coff, Kb, Vb, sh.rope_base, [0], "bank100m host")
    # two routed decode steps (single-token queries pad one 16-row tile of the MFMA scan)
    coff_d = torch.tensor(coff, device=DEV)
    Lq = int(q["q_len"][0])
    for s in (0, 5):
        r = Lq + s
        one = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
        ids1, sc1, ds1 = M.msa_route_topk(q["Qr"][r:r + 1].contiguous(), one, 1, Krb, coff_d, wl.k,
                                          want_doc_scores=True)
        kvo = torch.tensor([0, r + 1], dtype=torch.int32, device=DEV)
        out1 = M.msa_sparse_attn(q["Q"][r:r + 1].contiguous(), q["Kloc"][:r + 1].contiguous(),
                                 q["Vloc"][:r + 1].contiguous(), one, kvo, 1, ids1, coff_d, Kb, Vb,
                                 rope_base=sh.rope_base)
        torch.cuda.synchronize()
        i1 = ids1.cpu().numpy()[0]
        d1 = ds1.cpu().numpy()[0]
        assert_topk_consistent(i1, sc1.cpu().numpy()[0], d1, wl.k, f"decode {s}")
        o1 = oracle_doc_scores_all(q["Qr"][r:r + 1], [0, 1], Krb_rows, coff, what=f"decode {s}")[0]
        assert_scores_close(d1, o1, "bf16", f"decode {s} every document score")
        assert_topk_valid(i1, o1, wl.k, f"decode {s} top-k vs the oracle's ranking")
        sel = [int(d) for d in i1 if d >= 0]
        idx = np.concatenate([np.arange(coff[d], coff[d + 1]) for d in sel])
        kb, vb = f64(Kb[torch.as_tensor(idx)]), f64(Vb[torch.as_tensor(idx)])
        coff_c = np.concatenate([[0], np.cumsum([int(coff[d + 1] - coff[d]) for d in sel])])
        ref = O.sparse_attn(f64(q["Q"][r:r + 1]), f64(q["Kloc"][:r + 1]), f64(q["Vloc"][:r + 1]), [0, 1],
                            [0, r + 1], np.arange(len(sel), dtype=np.int32)[None], coff_c, kb, vb, sh.rope_base)
        e = assert_attn_close(out1, ref, "bf16", f"decode step {s}")
        say(f"  decode step {s}: attention max abs err {e:.3g}")


def test_bank100m_needles():
    # the headline bank (routing keys only) with five needle documents whose rows make cosine
    # 0.9 with the query's mean routing direction: all five are routed into the top-16, and
    # their scores and those of sampled documents agree with the oracle
    say("case full-size bank100m with 5 planted needles: recall and sampled scores")
    wl = W.workload("bank100m_host", needles=5)
    sh = wl.shape
    lens = W.doc_lengths(wl)
    off = W.token_offsets(lens)
    coff = M.msa_chunk_offsets(off, sh.chunk)
    q = W.gen_queries(wl, DEV)
    Lq = int(q["q_len"][0])
    needles, dirs = W.plant_needles(wl, len(lens), q["Qr"][:Lq])
    Krb_rows, _, _ = W.gen_pooled_bank(wl, coff, DEV, needle_dirs=dirs, needle_ids=needles, krbar_only=True)
    Qr, q_off, ids, sc, ds = run_route(q, coff, as_keys(Krb_rows), wl.k)
    ids_h = ids.cpu().numpy()[0]
    assert_topk_consistent(ids_h, sc[0], ds[0], wl.k, "bank100m needles")
    docs = sample_docs(len(lens), 4, extra=needles)
    Qh = f64(Qr[:Lq])
    o = np.array([O.doc_scores_one(Qh, f64(Krb_rows[int(coff[d]):int(coff[d + 1])]), [0, int(coff[d + 1] - coff[d])])[0]
                  for d in docs])
    err = assert_scores_close(ds[0][docs], o, "bf16", "bank100m needles: sampled document scores")
    recalled = set(int(x) for x in needles) & set(int(x) for x in ids_h)
    say(f"  bank100m: needles {list(needles)} recalled {len(recalled)}/5; {len(docs)} scores, max rel err {err:.3g}")
    assert len(recalled) == len(needles)


def test_batch32_bank10m_full():
    say("case full-size batch32_bank10m: pool, batched route sample, attention sample")
    wl = W.workload("batch32_bank10m")
    sh = wl.shape
    lens, off, coff, K, V, Kr, _ = token_bank(wl)
    Kb, Vb, Krb = run_pool(wl, off, coff, K, V, Kr)
    torch.cuda.synchronize()
    check_pool_sample(K, V, Kr, off, coff, Kb, Vb, Krb, sample_docs(len(lens), 5)[:10], sh.chunk,
                      sh.rope_base, "batch32")
    del K, V, Kr
    gc.collect()
    torch.cuda.empty_cache()
    q = W.gen_queries(wl, DEV)
    Qr, q_off, ids, sc, ds = run_route(q, coff, Krb, wl.k)
    ids_h = ids.cpu().numpy()
    B = len(q["q_len"])
    longest, shortest = int(np.argmax(q["q_len"])), int(np.argmin(q["q_len"]))
    for b in range(B):
        assert_topk_consistent(ids_h[b], sc[b], ds[b], wl.k, f"batch query {b}")
    # eight queries, the longest and the shortest among them: every document score
    rng = np.random.default_rng(31)
    picked = {0, 7, B - 1, longest, shortest}
    while len(picked) < 8:
        picked.add(int(rng.integers(0, B)))
    picked = sorted(picked)
    sub_rows = [Qr[q_off[b]:q_off[b + 1]] for b in picked]
    sub_off = np.concatenate([[0], np.cumsum([int(q_off[b + 1] - q_off[b]) for b in picked])])
    o = oracle_doc_scores_all(torch.cat(sub_rows), sub_off, Krb.rows(), coff, what="batch32")
    for i, b in enumerate(picked):
        err = assert_scores_close(ds[b], o[i], "bf16", f"batch query {b} every document score")
        assert_topk_valid(ids_h[b], o[i], wl.k, f"batch query {b} top-k vs the oracle's ranking")
        say(f"  batch query {b} ({int(q['q_len'][b])} tokens): every score, max rel err {err:.3g}")
    attn_check(q, ids, coff, Kb, Vb, sh.rope_base, list(range(B)), "batch32")


def test_batch32_bank10m_training_full():
    """The training backward of the 32-query batch over the 10M-token bank, in the bench's
    launch configuration (forward log-sum-exp and scan rows reused).  One sampled query
    carries the only nonzero dO and dL/dS, so every gradient it produces (its dQ and local
    dK/dV rows, the bank rows of its documents, its dQr rows and the maximising rows' dKrbar)
    can be checked against the oracle run on that query alone, and every other query's
    gradients must be exactly zero."""
    say("case full-size batch32_bank10m training backward, one sampled query")
    wl = W.workload("batch32_bank10m")
    sh = wl.shape
    lens = W.doc_lengths(wl)
    coff = M.msa_chunk_offsets(W.token_offsets(lens), sh.chunk)
    N, C = len(lens), int(coff[-1])
    Krb_rows, Kb, Vb = W.gen_pooled_bank(wl, coff, DEV)
    Krb = as_keys(Krb_rows)
    coff_d = torch.tensor(coff, device=DEV)
    q = W.gen_queries(wl, DEV)
    q_len = q["q_len"]
    B = len(q_len)
    q_off = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32)
    q_off_d = torch.tensor(q_off, device=DEV)
    Lmax = int(q_len.max())
    Qr, Q, Kl, Vl = q["Qr"], q["Q"], q["Kloc"], q["Vloc"]
    tq = int(q_off[-1])
    # forward: scan with row outputs, top-k, attention with log-sum-exp
    rows = (torch.empty((B, C), dtype=torch.float32, device=DEV), torch.empty((B, C), dtype=torch.int32, device=DEV))
    ds = M.msa_route_scan(Qr, q_off_d, Lmax, Krb, coff_d, rows=rows)
    ids, sc = M.msa_topk(ds, wl.k)
    lse = torch.empty((tq, sh.hq), dtype=torch.float32, device=DEV)
    out = M.msa_sparse_attn(Q, Kl, Vl, q_off_d, q_off_d, Lmax, ids, coff_d, Kb, Vb, rope_base=sh.rope_base, lse=lse)
    b = 7
    r0, r1 = int(q_off[b]), int(q_off[b + 1])
    g = torch.Generator(device=DEV).manual_seed(11)
    dO = torch.zeros_like(Q)
    dO[r0:r1] = torch.randn((r1 - r0,) + tuple(Q.shape[1:]), generator=g, device=DEV).to(torch.bfloat16)
    # dL/dS on sampled documents of query b whose best (token, row) pair is clear of the runner-up
    Qb64 = f64(Qr[r0:r1])
    cand = sample_docs(N, 21)[:30]
    keep = []
    for d in cand:
        s = np.sort(O.token_chunk_scores(Qb64, f64(Krb_rows[int(coff[d]):int(coff[d + 1])])).ravel())[::-1]
        if s.size == 1 or s[0] - s[1] >= 5e-3:
            keep.append(d)
    assert len(keep) >= 10, keep
    dD = torch.zeros((B, N), dtype=torch.float32, device=DEV)
    dvals = torch.randn(len(keep), generator=torch.Generator().manual_seed(12))
    dD[b, torch.tensor(keep, device=DEV)] = dvals.to(DEV)
    f32 = torch.float32
    dKb, dVb = torch.zeros(Kb.shape, dtype=f32, device=DEV), torch.zeros(Vb.shape, dtype=f32, device=DEV)
    gq = M.msa_sparse_attn_backward(Q, Kl, Vl, q_off_d, q_off_d, Lmax, ids, coff_d, Kb, Vb, out, dO,
                                    rope_base=sh.rope_base, dbank=(dKb, dVb), lse=lse)
    dKr = torch.zeros(Krb.shape, dtype=f32, device=DEV)
    dQr, _ = M.msa_route_backward(Qr, q_off_d, Lmax, Krb, coff_d, dD, dKrbar=dKr, rows=rows)
    torch.cuda.synchronize()
    # every other query: exactly zero gradients
    for t in (gq[0], gq[1], gq[2], dQr):
        assert torch.count_nonzero(t[:r0]) == 0 and torch.count_nonzero(t[r1:]) == 0
    # attention backward of query b against the oracle on its own compact bank
    sel = [int(d) for d in ids[b].cpu().numpy() if d >= 0]
    idx = np.concatenate([np.arange(coff[d], coff[d + 1]) for d in sel])
    cnt = [int(coff[d + 1] - coff[d]) for d in sel]
    coff_c = np.concatenate([[0], np.cumsum(cnt)])
    idx_d = torch.as_tensor(idx, device=DEV)
    L = r1 - r0
    ref = O.sparse_attn_backward(f64(Q[r0:r1]), f64(Kl[r0:r1]), f64(Vl[r0:r1]), [0, L], [0, L],
                                 np.arange(len(sel), dtype=np.int32)[None], coff_c, f64(Kb[idx_d]), f64(Vb[idx_d]),
                                 sh.rope_base, f64(dO[r0:r1]))
    got = (gq[0][r0:r1], gq[1][r0:r1], gq[2][r0:r1], dKb[idx_d], dVb[idx_d])
    for gg, oo, n in zip(got, ref, ("dQ", "dKloc", "dVloc", "dKbar", "dVbar")):
        gg = f64(gg)
        top = float(np.max(np.abs(oo)))
        err = float(np.max(np.abs(gg - oo)))
        say(f"  query {b} {n}: max err {err:.3g}, oracle max {top:.3g}")
        assert err <= 2.0 ** -6 * top + 1e-4, n
    # router backward of query b on the sampled documents
    cnt_r = [int(coff[d + 1] - coff[d]) for d in keep]
    coff_r = np.concatenate([[0], np.cumsum(cnt_r)])
    idx_r = torch.as_tensor(np.concatenate([np.arange(coff[d], coff[d + 1]) for d in keep]), device=DEV)
    rq, rk = O.route_backward(Qb64, [0, L], f64(Krb_rows[idx_r]), coff_r, dvals.double().numpy()[None])
    for gg, oo, n in ((f64(dQr[r0:r1]), rq, "dQr"), (f64(dKr[idx_r]), rk, "dKrbar")):
        top = float(np.max(np.abs(oo)))
        err = float(np.max(np.abs(gg - oo)))
        say(f"  query {b} {n}: max err {err:.3g}, oracle max {top:.3g}")
        assert err <= 1e-4 * top + 1e-7, n
    # rows of the bank no sampled document owns get no router gradient
    mask = torch.ones(C, dtype=torch.bool, device=DEV)
    mask[idx_r] = False
    assert torch.count_nonzero(dKr[mask]) == 0
