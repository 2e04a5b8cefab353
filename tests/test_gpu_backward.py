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


def _randn(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def _case(q_lens, extra_kv, hq, h_kv, d, counts, ids, seed, host=False):
    """Runs the GPU forward then backward, and the oracle backward, on one batch."""
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
    Out = M.msa_sparse_attn(Qd, Kld, Vld, args["q_off"], args["kv_off"], args["max_q_len"], ids_t,
                            args["chunk_off"], Kb_d, Vb_d, rope_base=1e6)
    grads = M.msa_sparse_attn_backward(Qd, Kld, Vld, args["q_off"], args["kv_off"], args["max_q_len"], ids_t,
                                       args["chunk_off"], Kb_d, Vb_d, Out, dO.to(DEV), rope_base=1e6)
    torch.cuda.synchronize()
    ref = O.sparse_attn_backward(f64(Q), f64(Kl), f64(Vl), q_off, kv_off, np.asarray(ids), coff, f64(Kb),
                                 f64(Vb), 1e6, f64(dO))
    return grads, ref, coff


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


CASES = [
    # name, q_lens, extra kv (decode cache), hq, h_kv, d, chunk counts per doc, ids per query
    ("prefill64_gqa4_d128", [64], [0], 32, 8, 128, [3, 17, 1, 40, 9, 2], [[3, 1, 4, 0]]),
    ("decode_d128", [1], [36], 32, 8, 128, [5, 12, 7], [[1, 2]]),
    ("gqa2_d64_ragged", [5, 33, 17], [0, 2, 40], 8, 4, 64, [4, 1, 9, 30, 2, 6, 3],
     [[2, 4, -1], [4, 0, 3], [6, 5, 4]]),
    ("few_docs_k_gt_n", [20], [3], 16, 4, 128, [2, 5], [[1, 0, -1, -1]]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_backward(case):
    name, q_lens, extra, hq, h_kv, d, counts, ids = case
    say(f"case attention backward {name}")
    grads, ref, coff = _case(q_lens, extra, hq, h_kv, d, counts, ids, seed=len(name))
    _check(grads, ref, name)
    # bank rows no query selected keep their (zero) initial value
    used = set(int(x) for row in ids for x in row if x >= 0)
    for dd in range(len(coff) - 1):
        if dd not in used:
            r0, r1 = int(coff[dd]), int(coff[dd + 1])
            assert torch.count_nonzero(grads[3][r0:r1]) == 0 and torch.count_nonzero(grads[4][r0:r1]) == 0


def test_attention_backward_host_bank():
    say("case attention backward, bank content in pinned host memory")
    grads, ref, coff = _case([16, 9], [4, 0], 16, 4, 128, [6, 3, 11, 2], [[2, 0], [2, 3]], seed=77, host=True)
    _check(grads, ref, "host bank")
