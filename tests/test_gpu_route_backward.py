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
from tests.helpers import SCORE_FLOOR, SCORE_RTOL, as_keys, assert_scores_close, f64, say

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


def _scan_rows(Qr_d, q_off_d, max_q_len, Kb_d, coff_d, B, N, C):
    """The forward scan with its row outputs: (doc scores, row scores, row args)."""
    rows = (torch.empty((B, C), dtype=torch.float32, device=DEV), torch.empty((B, C), dtype=torch.int32, device=DEV))
    ds = M.msa_route_scan(Qr_d, q_off_d, max_q_len, Kb_d, coff_d, rows=rows)
    return ds, rows


def _run(q_lens, counts, H, D, dtype, seed, path="auto", zero_heads=False, dKinit=False, use_rows=False):
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
    args = (Qr.to(DEV), torch.tensor(q_off, dtype=torch.int32, device=DEV), int(max(max(q_lens), 1)), as_keys(Kb.to(DEV)),
            torch.tensor(coff, dtype=torch.int64, device=DEV))
    rows = _scan_rows(*args, B, N, C)[1] if use_rows else None
    dQr, dK = M.msa_route_backward(*args, torch.tensor(dD, dtype=torch.float32, device=DEV), dKrbar=dK, rows=rows)
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
    ("bf16_h8_d128_batch", [3, 40, 130], 8, 128, "bf16", "batch"),
    ("bf16_h4_d128_batch", [1, 7, 40], 4, 128, "bf16", "batch"),
]


@pytest.mark.parametrize("use_rows", [False, True], ids=["rescan", "forward_rows"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_route_backward(case, use_rows):
    name, q_lens, H, D, dtype, path = case
    say(f"case route backward {name}, rows {'from the forward scan' if use_rows else 'rescanned'}")
    counts = np.random.default_rng(len(name)).integers(1, 13, size=37)
    got, ref, kept = _run(q_lens, counts, H, D, dtype, seed=len(name) * 7, path=path, zero_heads=True,
                          use_rows=use_rows)
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
    for use_rows in (False, True):
        got, ref, kept = _run([6, 0, 3], counts, 4, 64, "bf16", seed=91, use_rows=use_rows)
        _check(got, ref, "empty")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_scan_row_outputs(case):
    # every bank row's best token score and the first token reaching it, from each scan path;
    # the document scores come out bit-identical to a scan without row outputs
    name, q_lens, H, D, dtype, path = case
    say(f"case scan row outputs {name}")
    q_lens = list(q_lens) + [0]                      # and a query without tokens
    counts = np.random.default_rng(len(name) + 1).integers(1, 13, size=31)
    torch_dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q_off = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    coff = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    B, N, C = len(q_lens), len(counts), int(coff[-1])
    Kb = _randn((C, H, D), len(name) + 5).to(torch_dt)
    Qr = _randn((int(q_off[-1]), H, D), len(name) + 6).to(torch_dt)
    if path != "auto":
        os.environ["MSA_ROUTE_PATH"] = path
    args = (Qr.to(DEV), torch.tensor(q_off, dtype=torch.int32, device=DEV), int(max(q_lens)), as_keys(Kb.to(DEV)),
            torch.tensor(coff, dtype=torch.int64, device=DEV))
    ds_rows, (rs, ra) = _scan_rows(*args, B, N, C)
    ds = M.msa_route_scan(*args)
    torch.cuda.synchronize()
    assert torch.equal(ds_rows, ds), "document scores differ with row outputs"
    rs, ra = rs.cpu().numpy(), ra.cpu().numpy()
    assert np.all(rs[B - 1] == -np.inf), "rows of a query without tokens"
    Q64, K64 = f64(Qr), f64(Kb)
    for b in range(B - 1):
        ts = O.token_chunk_scores(Q64[q_off[b]:q_off[b + 1]], K64)          # [Lq, C]
        best = ts.max(axis=0)
        assert_scores_close(rs[b], best, dtype, f"{name} query {b} row scores")
        assert np.all((ra[b] >= 0) & (ra[b] < q_lens[b])), f"{name} query {b}: row arg out of range"
        # the chosen token reaches the row's maximum up to the scores' error; where the best
        # token leads the runner-up by more than that, it is the oracle's first maximum
        picked = ts[ra[b], np.arange(C)]
        tol = SCORE_RTOL[dtype] * np.maximum(np.abs(best), SCORE_FLOOR)
        assert np.all(best - picked <= 2 * tol), f"{name} query {b}: row arg misses the maximum"
        if q_lens[b] > 1:
            srt = np.sort(ts, axis=0)
            clear = srt[-1] - srt[-2] > 2 * tol
            assert np.array_equal(ra[b][clear], np.argmax(ts, axis=0)[clear]), f"{name} query {b}: row arg"


# ------------------------------------------------------------------ routing auxiliary loss

AUX_RTOL = 1e-6   # double sums, one rounding to float32 at the end


def _aux_case(kind, B, N, seed, tau):
    rng = np.random.default_rng(seed)
    S = rng.uniform(-1, 1, size=(B, N)).astype(np.float32)
    if kind == O.AUX_BCE:
        Y = rng.random((B, N)).astype(np.float32)
    else:
        Y = (rng.random((B, N)) < 0.05).astype(np.float32)
        Y[:, 0] = 1.0
    return S, Y


@pytest.mark.parametrize("kind", [O.AUX_BCE, O.AUX_INFONCE], ids=["bce", "infonce"])
@pytest.mark.parametrize("B,N,tau", [(1, 1, 1.0), (3, 7, 0.1), (32, 4747, 0.05), (2, 47343, 1.0)])
def test_aux_loss(kind, B, N, tau):
    say(f"case routing aux loss kind={kind} B={B} N={N} tau={tau}")
    S, Y = _aux_case(kind, B, N, B * 1000 + N, tau)
    if B > 1:
        S[1, N // 2] = -np.inf          # a query without tokens: skipped
    if kind == O.AUX_INFONCE and B > 2:
        Y[2] = 0.0                      # no positive label: skipped
    loss, dD = M.msa_route_aux_loss(torch.tensor(S, device=DEV), torch.tensor(Y, device=DEV), kind, tau)
    torch.cuda.synchronize()
    rl, rd = O.route_aux_loss(kind, S.astype(np.float64), Y.astype(np.float64), tau)
    gl, gd = f64(loss), f64(dD)
    assert np.all(np.abs(gl - rl) <= AUX_RTOL * np.abs(rl) + 1e-12), (gl, rl)
    err = np.abs(gd - rd) - (AUX_RTOL * np.abs(rd) + 1e-12)
    assert err.max() <= 0, float(np.abs(gd - rd).max())
    if B > 1:
        assert gl[1] == 0 and not gd[1].any()


def test_route_training_chain():
    # scan -> auxiliary loss -> router backward on the GPU against the same chain in the
    # oracle, on data whose maximising (token, row) pairs are all well separated
    say("case router training chain: scan, InfoNCE, backward")
    H, D = 8, 128
    q_lens, counts = [1, 3, 2], np.array([2, 1, 4, 3, 1, 2, 5, 1])
    q_off = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    coff = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    Kb = _randn((int(coff[-1]), H, D), 518).to(torch.bfloat16)   # seed chosen for separated maxima
    Qr = _randn((int(q_off[-1]), H, D), 519).to(torch.bfloat16)
    for b in range(len(q_lens)):
        for d in range(len(counts)):
            s = np.sort(O.token_chunk_scores(f64(Qr)[q_off[b]:q_off[b + 1]],
                                             f64(Kb)[coff[d]:coff[d + 1]]).ravel())[::-1]
            assert s.size == 1 or s[0] - s[1] >= GAP, (b, d)
    Y = np.zeros((len(q_lens), len(counts)), dtype=np.float32)
    Y[[0, 1, 2], [3, 0, 6]] = 1.0
    qo = torch.tensor(q_off, dtype=torch.int32, device=DEV)
    co = torch.tensor(coff, dtype=torch.int64, device=DEV)
    Qd, Kd = Qr.to(DEV), as_keys(Kb.to(DEV))
    S = M.msa_route_scan(Qd, qo, max(q_lens), Kd, co)
    loss, dD = M.msa_route_aux_loss(S, torch.tensor(Y, device=DEV), M.MSA_AUX_INFONCE, 0.1)
    dQr, dK = M.msa_route_backward(Qd, qo, max(q_lens), Kd, co, dD)
    torch.cuda.synchronize()
    rS = O.route_doc_scores(f64(Qr), q_off, f64(Kb), coff)
    rl, rd = O.route_aux_loss(O.AUX_INFONCE, rS, Y.astype(np.float64), 0.1)
    rq, rk = O.route_backward(f64(Qr), q_off, f64(Kb), coff, rd)
    assert np.allclose(f64(loss), rl, rtol=1e-4, atol=1e-6)
    _check((f64(dQr), f64(dK)), (rq, rk), "chain")


def test_route_backward_many_queries_shared_rows():
    # 1,032 queries over 6 short documents: every bank row maximises many queries' scores, so
    # its gradient gathers hundreds of atomic additions.  The query gradient has a fixed
    # summation order: two runs give the same bits.
    say("case route backward, 1032 queries sharing 6 documents' rows, run twice")
    counts = np.array([1, 3, 2, 4, 1, 2])
    q_lens = [1] * 1030 + [3, 2]
    got, ref, kept = _run(q_lens, counts, 4, 64, "bf16", seed=92)
    assert kept >= len(q_lens) * len(counts) // 3, kept
    _check(got, ref, "shared rows")
    again, _, _ = _run(q_lens, counts, 4, 64, "bf16", seed=92)
    assert np.array_equal(got[0], again[0]), "dQr differs between two identical runs"
