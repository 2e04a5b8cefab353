"""GPU parity of the backward of step D against the oracle's float64 gradients.

Inputs are bf16 (the GPU products run in bf16 on MFMA with float32 sums; the probabilities
and dS enter the second products rounded to bf16), the oracle runs in float64 on the same
bf16 values and on the GPU's selected documents.  Each gradient tensor is compared as a
whole: max |gpu - oracle| <= GRAD_RTOL * max |oracle| + GRAD_ATOL."""
import numpy as np
import pytest
import torch

import latent_memory_long_amd as M
from oracle import msa_oracle as O
from tests.helpers import f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

# Three roundings to bf16 (unit roundoff u = 2^-8) enter every gradient term: the rotated
# Q / local K operands, the probabilities' dS operand, and the forward output O inside
# rowsum(dO * O).  Emulating those three roundings in float64 on the CPU reproduces the GPU's
# errors to three digits (about 1.1 u x max |gradient| on the decode case), so the bar is
# 4 u = 2^-6 of the tensor's largest oracle value.
GRAD_RTOL = 2.0 ** -6
GRAD_ATOL = 1e-4

# The forward's per-row log-sum-exp: the GPU's logits use the rotated Q and local K rounded
# to bf16 (unit roundoff u = 2^-8 each), so every logit is off by at most
# scale * 2u * |q| * |k| (Cauchy-Schwarz), and so is the log-sum-exp; float32 sums and
# exp2/log2 add about 1e-4 at most at these sizes.
LSE_U = 2.0 ** -8
LSE_ATOL = 1e-4


def _randn(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def _case(q_lens, extra_kv, hq, h_kv, d, counts, ids, seed, host=False, use_lse=False):
    """Runs the GPU forward then backward, and the oracle backward, on one batch.  With
    use_lse the forward also returns each row's log-sum-exp, which the backward reuses; it
    is checked against the oracle's here."""
    B = len(q_lens)
    kv_lens = [q + e for q, e in zip(q_lens, extra_kv)]
    q_off = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kv_off = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    coff = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    C = int(coff[-1])
    Q = _randn((int(q_off[-1]), hq, d), seed)
    Kl = _randn((int(kv_off[-1]), h_kv, d), seed + 1)
    Vl = _randn((int(kv_off[-1]), h_kv, d), seed + 2)
    Kb = _randn((C, h_kv, d), seed + 3, 0.6)
    Vb = _randn((C, h_kv, d), seed + 4)
    dO = _randn((int(q_off[-1]), hq, d), seed + 5)
    ids_t = torch.tensor(np.asarray(ids, dtype=np.int32), device=DEV)
    args = dict(q_off=torch.tensor(q_off, device=DEV), kv_off=torch.tensor(kv_off, device=DEV),
                max_q_len=int(max(q_lens)), topk_ids=ids_t, chunk_off=torch.tensor(coff, device=DEV))
    Kb_d = Kb.pin_memory() if host else Kb.to(DEV)
    Vb_d = Vb.pin_memory() if host else Vb.to(DEV)
    Qd, Kld, Vld = Q.to(DEV), Kl.to(DEV), Vl.to(DEV)
    lse = torch.full((int(q_off[-1]), hq), float("nan"), device=DEV) if use_lse else None
    Out = M.msa_sparse_attn(Qd, Kld, Vld, args["q_off"], args["kv_off"], args["max_q_len"], ids_t,
                            args["chunk_off"], Kb_d, Vb_d, rope_base=1e6, lse=lse)
    grads = M.msa_sparse_attn_backward(Qd, Kld, Vld, args["q_off"], args["kv_off"], args["max_q_len"], ids_t,
                                       args["chunk_off"], Kb_d, Vb_d, Out, dO.to(DEV), rope_base=1e6, lse=lse)
    torch.cuda.synchronize()
    if use_lse:
        _check_lse(lse, Q, Kl, Kb, q_off, kv_off, np.asarray(ids), coff, d)
    ref = O.sparse_attn_backward(f64(Q), f64(Kl), f64(Vl), q_off, kv_off, np.asarray(ids), coff, f64(Kb),
                                 f64(Vb), 1e6, f64(dO))
    return grads, ref, coff


def _check_lse(lse, Q, Kl, Kb, q_off, kv_off, ids, coff, d):
    ref = O.sparse_attn_lse(f64(Q), f64(Kl), f64(Kl), q_off, kv_off, ids, coff, f64(Kb), f64(Kb), 1e6)
    got = lse.cpu().double().numpy()
    assert np.all(np.isfinite(got)), "lse: non-finite or unwritten rows"
    # per-row bound: the row's |q| times the largest |k| of its query's keys
    qn = np.linalg.norm(f64(Q), axis=-1)
    G = Q.shape[1] // Kl.shape[1]
    for b in range(len(q_off) - 1):
        if q_off[b + 1] == q_off[b]:
            continue  # a query without tokens has no rows
        rows = [r for dd in ids[b] if dd >= 0 for r in range(int(coff[dd]), int(coff[dd + 1]))]
        kn = np.linalg.norm(f64(Kl)[kv_off[b]:kv_off[b + 1]], axis=-1).max(axis=0)
        if rows:
            kn = np.maximum(kn, np.linalg.norm(f64(Kb)[rows], axis=-1).max(axis=0))
        tol = 2 * LSE_U / np.sqrt(d) * qn[q_off[b]:q_off[b + 1]] * np.repeat(kn, G)[None, :] + LSE_ATOL
        err = np.abs(got[q_off[b]:q_off[b + 1]] - ref[q_off[b]:q_off[b + 1]])
        say(f"  lse query {b}: max err {err.max():.3g}, smallest bound {tol.min():.3g}")
        assert np.all(err <= tol), f"lse query {b}: max err {err.max():.3g}"


def _check(grads, ref, what):
    names = ("dQ", "dKloc", "dVloc", "dKbar", "dVbar")
    for g, o, n in zip(grads, ref, names):
        g = g.detach().cpu().double().numpy()
        assert g.shape == o.shape, (what, n)
        assert np.all(np.isfinite(g)), f"{what} {n}: non-finite"
        top = float(np.max(np.abs(o))) if o.size else 0.0
        err = float(np.max(np.abs(g - o))) if o.size else 0.0
        say(f"  {what} {n}: max err {err:.3g}, oracle max {top:.3g}, ratio {err / max(top, 1e-30):.3g}")
        assert err <= GRAD_RTOL * top + GRAD_ATOL, f"{what} {n}: max err {err:.3g} vs max {top:.3g}"


_MAXK_RNG = np.random.default_rng(101)
_MAXK_COUNTS = [int(x) for x in _MAXK_RNG.integers(1, 3, size=1100)]
_MAXK_IDS = [[int(x) for x in _MAXK_RNG.choice(1100, size=1024, replace=False)],
             [int(x) for x in _MAXK_RNG.choice(1100, size=924, replace=False)] + [-1] * 100]

CASES = [
    # name, q_lens, extra kv (decode cache), hq, h_kv, d, chunk counts per doc, ids per query
    ("prefill64_gqa4_d128", [64], [0], 32, 8, 128, [3, 17, 1, 40, 9, 2], [[3, 1, 4, 0]]),
    ("decode_d128", [1], [36], 32, 8, 128, [5, 12, 7], [[1, 2]]),
    ("gqa2_d64_ragged", [5, 33, 17], [0, 2, 40], 8, 4, 64, [4, 1, 9, 30, 2, 6, 3],
     [[2, 4, -1], [4, 0, 3], [6, 5, 4]]),
    ("few_docs_k_gt_n", [20], [3], 16, 4, 128, [2, 5], [[1, 0, -1, -1]]),
    # dQ row blocks of 32 and 64 query rows (2 and 4 waves)
    ("rows32_d128", [8], [2], 32, 8, 128, [4, 9, 2], [[2, 0]]),
    ("rows64_d128", [16, 5], [0, 3], 32, 8, 128, [4, 9, 2, 6], [[3, 1], [0, 2]]),
    # 8 queries x 8 kv heads fill the GPU without splitting the keys: the forward writes O
    # and the log-sum-exp straight from the attention kernel instead of the split merge
    ("batch8_unsplit", [12, 3, 20, 7, 1, 16, 9, 5], [0, 4, 0, 2, 30, 0, 1, 0], 32, 8, 128,
     [3, 8, 1, 5, 12, 2, 6], [[0, 4], [2, 1], [6, 5], [3, -1], [4, 0], [1, 2], [5, 6], [0, 3]]),
    # k = 1024, the largest the library takes: 1,100 documents of one or two rows, the two
    # queries sharing many of them (their rows' gradients collect both shares); the second
    # leaves its last 100 slots unused
    ("k1024_max", [7, 3], [2, 0], 8, 2, 64, _MAXK_COUNTS, _MAXK_IDS),
    # a query with no tokens between two others: its local keys get zero gradients
    ("empty_query", [5, 0, 7], [0, 2, 1], 8, 2, 64, [3, 2, 4, 1], [[0, 2], [1, 3], [3, -1]]),
]


@pytest.mark.parametrize("use_lse", [False, True], ids=["recompute_lse", "forward_lse"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_backward(case, use_lse):
    name, q_lens, extra, hq, h_kv, d, counts, ids = case
    say(f"case attention backward {name} lse {'from the forward' if use_lse else 'recomputed'}")
    grads, ref, coff = _case(q_lens, extra, hq, h_kv, d, counts, ids, seed=len(name), use_lse=use_lse)
    _check(grads, ref, name)
    # bank rows no query selected keep their (zero) initial value
    used = set(int(x) for row in ids for x in row if x >= 0)
    for dd in range(len(coff) - 1):
        if dd not in used:
            r0, r1 = int(coff[dd]), int(coff[dd + 1])
            assert torch.count_nonzero(grads[3][r0:r1]) == 0 and torch.count_nonzero(grads[4][r0:r1]) == 0


def test_attention_backward_host_bank():
    say("case attention backward, bank content in pinned host memory")
    grads, ref, coff = _case([16, 9], [4, 0], 16, 4, 128, [6, 3, 11, 2], [[2, 0], [2, 3]], seed=77, host=True,
                             use_lse=True)
    _check(grads, ref, "host bank")


def test_forward_lse_fp32():
    say("case forward log-sum-exp, float32 inputs")
    rng = np.random.default_rng(90)
    q_lens, kv_lens, hq, h_kv, d = [6, 2], [9, 2], 8, 2, 64
    q_off = np.array([0, 6, 8], dtype=np.int32)
    kv_off = np.array([0, 9, 11], dtype=np.int32)
    coff = np.array([0, 3, 4, 9], dtype=np.int64)
    Q = torch.tensor(rng.standard_normal((8, hq, d)), dtype=torch.float32)
    Kl = torch.tensor(rng.standard_normal((11, h_kv, d)), dtype=torch.float32)
    Vl = torch.tensor(rng.standard_normal((11, h_kv, d)), dtype=torch.float32)
    Kb = torch.tensor(rng.standard_normal((9, h_kv, d)) * 0.6, dtype=torch.float32)
    Vb = torch.tensor(rng.standard_normal((9, h_kv, d)), dtype=torch.float32)
    ids = np.array([[2, 0], [1, -1]], dtype=np.int32)
    lse = torch.full((8, hq), float("nan"), device=DEV)
    M.msa_sparse_attn(Q.to(DEV), Kl.to(DEV), Vl.to(DEV), torch.tensor(q_off, device=DEV),
                      torch.tensor(kv_off, device=DEV), max(q_lens), torch.tensor(ids, device=DEV),
                      torch.tensor(coff, device=DEV), Kb.to(DEV), Vb.to(DEV), rope_base=1e6, lse=lse)
    torch.cuda.synchronize()
    ref = O.sparse_attn_lse(f64(Q), f64(Kl), f64(Vl), q_off, kv_off, ids, coff, f64(Kb), f64(Vb), 1e6)
    # float32 rotation and dot products: errors of order 1e-6 relative to |q||k| / sqrt(d)
    err = float(np.max(np.abs(lse.cpu().double().numpy() - ref)))
    say(f"  fp32 lse max err {err:.3g}")
    assert err < 1e-4
