"""GPU parity of the router's backward against the oracle's float64 gradients.

A document score is a maximum, so its gradient lands on one (token, bank row) pair.  Where
the best and second-best pair of a (query, document) lie closer than the forward scan's
error bound, the float32 GPU and the float64 oracle may pick different pairs, both correct;
those entries of dL/dS are set to zero, so the comparison covers only well-defined choices
(the tests check that at least a third of the entries remain).  The gradient formulas then
run in float32 on the same bf16 / float32 inputs the oracle reads exactly:
max |gpu - oracle| <= RTOL x max |oracle| per tensor."""
import os

import numpy as np
import pytest
import torch

import latent_memory_long_amd as M
from oracle import msa_oracle as O
from tests.helpers import f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

GAP = 5e-3      # above twice the scan's score bound (bf16 scores: 2e-3 relative, 1e-3 floor)
RTOL = 1e-4     # float32 sums of at most a few thousand terms
ATOL = 1e-7


@pytest.fixture(autouse=True)
def _reset_env():
    yield
    os.environ.pop("MSA_ROUTE_PATH", None)


def _randn(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g) * std


def _mask_near_ties(Qr64, q_off, Kb64, coff, dD):
    """Zeroes dD where the top two (token, row) pairs of a (query, document) are within GAP."""
    kept = 0
    for b in range(len(q_off) - 1):
        Qb = Qr64[q_off[b]:q_off[b + 1]]
        for d in range(len(coff) - 1):
            if len(Qb) == 0:
                continue
            s = np.sort(O.token_chunk_scores(Qb, Kb64[coff[d]:coff[d + 1]]).ravel())[::-1]
            if s.size > 1 and s[0] - s[1] < GAP:
                dD[b, d] = 0.0
            elif dD[b, d] != 0:
                kept += 1
    return kept


def _run(q_lens, counts, H, D, dtype, seed, path="auto", zero_heads=False, dKinit=False):
    torch_dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q_off = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    coff = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    B, N, C = len(q_lens), len(counts), int(coff[-1])
    # documents share a mean direction so that several of them compete for each token
    mu = _randn((N, H, D), seed, 0.5)
    Kb = _randn((C, H, D), seed + 1) + torch.repeat_interleave(mu, torch.as_tensor(counts), dim=0)
    Qr = _randn((int(q_off[-1]), H, D), seed + 2)
    if zero_heads:
        Kb[::3, 0] = 0.0      # a zero routing key head: cosine 0, no gradient for that head
        Qr[1::4, H - 1] = 0.0
    Kb, Qr = Kb.to(torch_dt), Qr.to(torch_dt)
    dD = _randn((B, N), seed + 3).double().numpy()
    dD[:, ::5] = 0.0
    kept = _mask_near_ties(f64(Qr), q_off, f64(Kb), coff, dD)
    if path != "auto":
        os.environ["MSA_ROUTE_PATH"] = path
    init = _randn((C, H, D), seed + 4) if dKinit else torch.zeros((C, H, D))
    dK = init.to(DEV)
    dQr, dK = M.msa_route_backward(Qr.to(DEV), torch.tensor(q_off, dtype=torch.int32, device=DEV),
                                   int(max(max(q_lens), 1)), Kb.to(DEV),
                                   torch.tensor(coff, dtype=torch.int64, device=DEV),
                                   torch.tensor(dD, dtype=torch.float32, device=DEV), dKrbar=dK)
    torch.cuda.synchronize()
    rq, rk = O.route_backward(f64(Qr), q_off, f64(Kb), coff, dD)
    rk = rk + init.double().numpy()
    return (f64(dQr), f64(dK)), (rq, rk), kept


def _check(got, ref, what):
    for g, o, n in zip(got, ref, ("dQr", "dKrbar")):
        assert g.shape == o.shape and np.all(np.isfinite(g)), (what, n)
        top = float(np.max(np.abs(o), initial=0.0))
        err = float(np.max(np.abs(g - o), initial=0.0))
        say(f"  {what} {n}: max err {err:.3g}, oracle max {top:.3g}")
        assert err <= RTOL * top + ATOL, f"{what} {n}: max err {err:.3g} vs max {top:.3g}"


CASES = [
    # name, q_lens, H, D, dtype, path
    ("bf16_h4_d128_auto", [1, 7, 40], 4, 128, "bf16", "auto"),
    ("bf16_h4_d128_dot", [1, 7, 40], 4, 128, "bf16", "dot"),
    ("bf16_h8_d64_mfma", [3, 17], 8, 64, "bf16", "mfma"),
    ("f32_h16_d32", [2, 9, 1], 16, 32, "f32", "auto"),
    ("bf16_h16_d128", [5, 12], 16, 128, "bf16", "auto"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_route_backward(case):
    name, q_lens, H, D, dtype, path = case
    say(f"case route backward {name}")
    counts = np.random.default_rng(len(name)).integers(1, 13, size=37)
    got, ref, kept = _run(q_lens, counts, H, D, dtype, seed=len(name) * 7, path=path, zero_heads=True)
    assert kept >= len(q_lens) * 37 // 3, kept
    _check(got, ref, name)
    # rows no maximum reached keep their initial (zero) value
    used = np.abs(ref[1]).sum(axis=(1, 2)) > 0
    assert np.all(got[1][~used] == 0)


def test_route_backward_long_query_and_accumulation():
    # 1500 tokens: more than the token grid, so workgroups stride over tokens; dKrbar starts
    # from a nonzero array and is added to
    say("case route backward long query, accumulated dKrbar")
    counts = np.random.default_rng(3).integers(1, 9, size=40)
    got, ref, kept = _run([1500, 4], counts, 8, 128, "bf16", seed=90, dKinit=True)
    assert kept >= 2 * 40 // 3, kept
    _check(got, ref, "long")


def test_route_backward_empty_query():
    # a query with no tokens contributes nothing, whatever dL/dS holds for it
    say("case route backward with an empty query")
    counts = np.random.default_rng(4).integers(1, 6, size=20)
    got, ref, kept = _run([6, 0, 3], counts, 4, 64, "bf16", seed=91)
    _check(got, ref, "empty")
