"""Comparison helpers for the GPU parity tests (tolerances as stated in the design notes)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import msa_oracle as O

# floating-point bars
SCORE_RTOL = {"f32": 1e-5, "bf16": 2e-3}       # doc scores, relative, floor 1e-3
SCORE_FLOOR = 1e-3
ATTN_ATOL = {"f32": 1e-5, "bf16": 1e-2}        # attention output, absolute
TIE_RTOL = 1e-4                                  # top-k boundary tie window, relative
POOL_F32_RTOL = 1e-6                             # pooled rows, relative to max(|o|, rms)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a float32 / bf16 tensor (device or host)."""
    return t.detach().float().cpu().double().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


POOL_ACC_ABS = 2.0 ** -20                        # float32 accumulation bound, x input RMS


def assert_pool_close(gpu: torch.Tensor, oracle64: np.ndarray, dtype: str, what: str,
                      input_rms: float = 1.0):
    """bf16: within 1 ulp of the exact mean, or -- for means that cancel to near zero,
    where a bf16 ulp is far below float32 summation error -- within 2^-20 x the RMS of
    the pooled inputs in absolute terms.  float32: relative 1e-6 of max(|o|, rms)."""
    if dtype == "bf16":
        ref = O.f64_to_bf16_bits(oracle64)
        d = np.abs(_ordered(bf16_bits(gpu)) - _ordered(ref))
        absdiff = np.abs(f64(gpu) - oracle64)
        bad = (d > 1) & (absdiff > POOL_ACC_ABS * input_rms)
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond 1 bf16 ulp and the "
                               f"accumulation bound (max {int(d.max())} ulp, {absdiff[bad].max():.3g} abs)")
    else:
        g = f64(gpu)
        scale = max(float(np.sqrt(np.mean(oracle64 ** 2))), 1e-30)
        err = np.abs(g - oracle64) / np.maximum(np.abs(oracle64), scale)
        assert err.max(initial=0) <= POOL_F32_RTOL, f"{what}: rel err {err.max():.3g}"


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
