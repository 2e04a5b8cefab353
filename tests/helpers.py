"""Comparison helpers for the GPU parity tests (tolerances as stated in the design notes)."""
from __future__ import annotations

import concurrent.futures
import os
import sys
import time

import numpy as np
import torch

import latent_memory_long_amd as M
from oracle import msa_oracle as O

# floating-point bars
SCORE_RTOL = {"f32": 1e-5, "bf16": 2e-3}       # doc scores, relative, floor 1e-3
SCORE_FLOOR = 1e-3
ATTN_ATOL = {"f32": 1e-5, "bf16": 1e-2}        # attention output, absolute
TIE_RTOL = 1e-4                                  # top-k boundary tie window, relative


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def key_rows(t):
    """Routing keys as a row-major [C, h_r, d] tensor (RouteKeys are unpacked on the GPU)."""
    return t.rows() if isinstance(t, M.RouteKeys) else t


def as_keys(t):
    """Routing keys in the library's bank layout, from a row-major [C, h_r, d] tensor."""
    return t if isinstance(t, M.RouteKeys) else M.RouteKeys.from_rows(t)


def f64(t) -> np.ndarray:
    """Exact float64 copy of a float32 / bf16 tensor (device or host) or of RouteKeys' rows."""
    return key_rows(t).detach().float().cpu().double().numpy()


U32 = 2.0 ** -24                                 # unit roundoff of float32


def pool_error_bound(X, doc_tok_off, chunk: int, rotated: bool) -> np.ndarray:
    """Per element of every pooled row, a bound on |float32 mean - exact mean| for the GPU's
    arithmetic: each chunk's tokens are summed in float32 in token order, the sum divided
    by the token count with one IEEE division; a rotated tensor is first rotated token by
    token by R(r) (float32 cos/sin, r the position in the chunk) and its chunk sum by R(s)
    (float32 cos/sin, s the chunk's first position).  With u = 2^-24, n tokens, and
    a_i = |x_i| (+ |y_i|, the rotation partner, when rotated):
      summation of n terms (sequential, Higham's bound)   gamma_{n-1} * sum a_i
      each token's rotation x c - y s (c, s rounded)      3u * a_i
      the chunk-start rotation of the sum                 3u * sum a_i
      the division                                        u * |mean|
    so, at the mean's scale, |m_gpu - m| <= u |m| + (gamma_{n-1} + 6u [rotated]) mean_i a_i.
    X: float64 [T, H, D] token states of the pooled tensor.  Returns float64 [C, H, D]."""
    X = np.asarray(X, dtype=np.float64)
    off = np.asarray(doc_tok_off, dtype=np.int64)
    A = np.abs(X)
    if rotated:
        h = X.shape[-1] // 2
        A = A + np.concatenate([np.abs(X[..., h:]), np.abs(X[..., :h])], axis=-1)
    out = []
    for d in range(len(off) - 1):
        for t0 in range(int(off[d]), int(off[d + 1]), chunk):
            t1 = min(t0 + chunk, int(off[d + 1]))
            n = t1 - t0
            gamma = (n - 1) * U32 / (1.0 - (n - 1) * U32)
            mean_a = A[t0:t1].sum(axis=0) / n
            # u |m|: for a rotated tensor |m| <= mean a_i
            m_abs = mean_a if rotated else np.abs(X[t0:t1].sum(axis=0) / n)
            out.append(U32 * m_abs + (gamma + (6 * U32 if rotated else 0.0)) * mean_a)
    return np.stack(out)


def _half_ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of the storage type's numbers in the binade of |v| (normal range)."""
    mant = 7 if dtype == "bf16" else 23
    _, e = np.frexp(np.maximum(np.abs(v), 2.0 ** -126))
    return np.ldexp(0.5, e - 1 - mant)


def assert_pool_close(gpu, oracle64: np.ndarray, dtype: str, what: str, bound: np.ndarray):
    """|gpu - exact mean| <= B + (for bf16) half a bf16 spacing at |mean| + B, with B the
    float32 arithmetic's bound from pool_error_bound: the GPU rounds its float32 mean m~
    (|m~ - m| <= B) once to bf16, landing within half a spacing of m~."""
    g = f64(gpu)
    B = np.asarray(bound, dtype=np.float64)
    err = np.abs(g - oracle64)
    allow = B + (_half_ulp(np.abs(oracle64) + B, "bf16") if dtype == "bf16" else 0.0)
    bad = err > allow
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the bound (worst error "
                           f"{err[bad].max():.3g}, allowed {allow[bad][np.argmax(err[bad])]:.3g})")
    return float(np.max(err / np.maximum(allow, 1e-300), initial=0.0))


def assert_scores_close(gpu_scores: np.ndarray, oracle_scores: np.ndarray, dtype: str, what: str):
    err = np.abs(gpu_scores - oracle_scores) / np.maximum(np.abs(oracle_scores), SCORE_FLOOR)
    assert err.max(initial=0) <= SCORE_RTOL[dtype], f"{what}: score rel err {err.max():.3g}"
    return float(err.max(initial=0))


def assert_topk_valid(ids_g: np.ndarray, oracle_scores: np.ndarray, k: int, what: str):
    """GPU ids vs the oracle's scores of every document: same set except documents whose
    oracle score lies within TIE_RTOL of the k-th best; order non-increasing in oracle
    score up to the same window; unused slots -1."""
    N = len(oracle_scores)
    keff = min(k, N)
    oid, ov = O.topk_docs(oracle_scores, k)
    kth = ov[keff - 1]
    win = TIE_RTOL * max(abs(kth), SCORE_FLOOR)
    g = [int(x) for x in ids_g[:keff]]
    assert len(set(g)) == keff and all(0 <= x < N for x in g), f"{what}: bad ids {g}"
    assert np.all(ids_g[keff:] == -1), f"{what}: unused slots {ids_g[keff:]}"
    for d in set(g) ^ set(int(x) for x in oid[:keff]):
        assert abs(oracle_scores[d] - kth) <= win, \
            f"{what}: id {d} (score {oracle_scores[d]:.7g}) differs from oracle set, k-th {kth:.7g}"
    s = oracle_scores[g]
    for i in range(keff - 1):
        assert s[i] >= s[i + 1] - TIE_RTOL * max(abs(s[i]), SCORE_FLOOR), f"{what}: order at {i}"
    return list(oid[:keff])


def assert_topk_consistent(ids_g: np.ndarray, sc_g: np.ndarray, doc_scores_g: np.ndarray, k: int,
                           what: str):
    """Exact integer check: the GPU's top-k equals the (score desc, id asc) order of the GPU's
    own float32 document scores."""
    N = len(doc_scores_g)
    order = np.lexsort((np.arange(N), -doc_scores_g.astype(np.float64)))
    keff = min(k, N)
    assert np.array_equal(ids_g[:keff], order[:keff]), f"{what}: top-k not the order of doc scores"
    assert np.array_equal(sc_g[:keff], doc_scores_g[order[:keff]]), f"{what}: top-k scores"


def assert_attn_close(gpu: torch.Tensor, oracle64: np.ndarray, dtype: str, what: str):
    g = f64(gpu)
    rows = ~np.isnan(oracle64[:, 0, 0])
    err = np.abs(g[rows] - oracle64[rows])
    assert np.all(np.isfinite(g[rows])), f"{what}: non-finite output"
    assert err.max(initial=0) <= ATTN_ATOL[dtype], f"{what}: max abs err {err.max():.3g}"
    return float(err.max(initial=0))


def host_threads() -> int:
    """Host threads for oracle work: the cores this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def doc_groups(coff: np.ndarray, block: int):
    """Consecutive document ranges [d0, d1) of about ``block`` bank rows each (a document
    larger than the block is a group of its own)."""
    coff = np.asarray(coff, dtype=np.int64)
    N = len(coff) - 1
    out, d0 = [], 0
    while d0 < N:
        d1 = int(np.searchsorted(coff, coff[d0] + block, side="right")) - 1
        d1 = min(max(d1, d0 + 1), N)
        out.append((d0, d1))
        d0 = d1
    return out


def oracle_doc_scores_all(Qr: torch.Tensor, q_off, Krb: torch.Tensor, coff, block: int = 8192,
                          what: str = "") -> np.ndarray:
    """The oracle's score of every document for every query, [B, N] float64.

    Each group of whole documents is scored by the unchanged oracle (``doc_scores_one``
    on its rows, from an exact float64 copy of the bank), so the result equals one call
    of ``route_doc_scores`` on the whole bank.  The groups run on host threads: NumPy
    leaves the interpreter lock while it evaluates the oracle's products.  Prints its
    progress, since a 100M-token bank takes tens of seconds."""
    q_off = np.asarray(q_off, dtype=np.int64)
    coff = np.asarray(coff, dtype=np.int64)
    B, N = len(q_off) - 1, len(coff) - 1
    Kh = key_rows(Krb).detach().cpu()
    Qs = [f64(Qr[int(q_off[b]):int(q_off[b + 1])]) for b in range(B)]
    groups = doc_groups(coff, block)
    out = np.empty((B, N), dtype=np.float64)

    def work(g):
        d0, d1 = g
        sub = Kh[int(coff[d0]):int(coff[d1])].float().double().numpy()
        loc = coff[d0:d1 + 1] - coff[d0]
        for b in range(B):
            out[b, d0:d1] = O.doc_scores_one(Qs[b], sub, loc)
        return d1 - d0

    t0 = time.time()
    nthr = host_threads()
    done, next_mark = 0, 0.1
    with concurrent.futures.ThreadPoolExecutor(nthr) as ex:
        for n in ex.map(work, groups):
            done += n
            if done >= next_mark * N:
                say(f"  oracle scores {what}: {done}/{N} documents, {time.time() - t0:.1f} s, {nthr} threads")
                next_mark += 0.1
    return out
