"""Seeded synthetic workloads shaped like the pages' memory banks and queries.

The pages evaluate on question-answering banks of 277K-10M tokens and a needle test of
32K-1M tokens, and run a 100M-token bank for throughput ([hysenlabs] "Quality is measured
on 9 QA sets ..." and "The 100M-token setup depends on host memory ...").  None of those
datasets is used: the inputs here are random tensors with the layer shapes, bank sizes
and document-length mixes of those workloads.

Everything is drawn from seeded generators:
  * NumPy ``default_rng(seed)`` for document lengths, needle ids and the tiny float32
    workload;
  * ``torch.Generator(device).manual_seed(seed * 1000 + stream)`` for bulk tensors, one
    stream per tensor so the draw order of one tensor does not shift another.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

__all__ = [
    "LayerShape", "Workload", "WORKLOADS", "workload", "layer",
    "doc_lengths", "token_offsets", "gen_token_states", "gen_queries", "plant_needles",
    "gen_pooled_bank", "torch_gen", "STREAM",
]


@dataclass(frozen=True)
class LayerShape:
    hq: int      # query heads
    h_kv: int    # key/value heads
    h_r: int     # routing heads (Qr / Kr)
    d: int       # head dim
    chunk: int = 64
    rope_base: float = 1e6


QWEN3_4B_LIKE = LayerShape(hq=32, h_kv=8, h_r=8, d=128)
TINY_LAYER = LayerShape(hq=4, h_kv=2, h_r=2, d=32)


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                   # "f32" or "bf16": storage / arithmetic type of the run
    shape: LayerShape
    len_dist: tuple              # ("uniform" | "loguniform", lo, hi), inclusive bounds
    bank_tokens: Optional[int] = None   # total bank tokens (documents drawn until reached)
    n_docs: Optional[int] = None        # or a fixed document count
    doc_offset_std: float = 0.0  # std of the per-document mean offset added to K, V, Kr
    q_offset_std: float = 0.0    # std of the per-query, per-head offset added to Qr
    n_queries: int = 1
    lq: tuple = (64, 64)         # query length range, inclusive
    k: int = 16
    needles: int = 0             # documents whose Kr is aligned with the query's Qr mean
    needle_cos: float = 0.9
    kv_source: str = "hbm"       # where K-bar / V-bar live: "hbm" or "host" (pinned)
    pooled_direct: bool = False  # bank drawn already pooled (token level would not fit)
    decode_steps: int = 0        # single-token steps after the prefill query
    n_layers: int = 1            # routed layers, each with its own bank and query tensors
    seed: int = 0


WORKLOADS = {
    # 16 documents, fp32, two KV/routing heads of dim 32; 8-token query, k = 2.
    "tiny_fp32": Workload("tiny_fp32", "f32", TINY_LAYER, ("uniform", 100, 512), n_docs=16,
                          lq=(8, 8), k=2),
    # 1M-token bank, bf16, Qwen3-4B-like upper layer; 64-token query, k = 16.
    "bank1m": Workload("bank1m", "bf16", QWEN3_4B_LIKE, ("loguniform", 200, 4000),
                       bank_tokens=1_000_000, doc_offset_std=0.5, q_offset_std=0.5),
    # 10M-token bank with 5 planted needle documents.
    "bank10m_needles": Workload("bank10m_needles", "bf16", QWEN3_4B_LIKE,
                                ("loguniform", 200, 8000), bank_tokens=10_000_000,
                                doc_offset_std=0.5, q_offset_std=0.5, needles=5),
    # 100M-token bank: routing keys in HBM, content K/V in pinned host memory, plus decode.
    "bank100m_host": Workload("bank100m_host", "bf16", QWEN3_4B_LIKE, ("loguniform", 200, 8000),
                              bank_tokens=100_000_000, doc_offset_std=0.5, q_offset_std=0.5,
                              kv_source="host", pooled_direct=True, decode_steps=32),
    # 18 routed (upper) layers of a 36-layer Qwen3-4B-like model over one 10M-token corpus:
    # a bank per layer, all resident in HBM, one 64-token query routed in every layer.
    "layers18_bank10m": Workload("layers18_bank10m", "bf16", QWEN3_4B_LIKE, ("loguniform", 200, 8000),
                                 bank_tokens=10_000_000, doc_offset_std=0.5, q_offset_std=0.5,
                                 pooled_direct=True, n_layers=18),
    # Encode 10M tokens, then a batch of 32 queries of 16-256 tokens, k = 32.
    "batch32_bank10m": Workload("batch32_bank10m", "bf16", QWEN3_4B_LIKE,
                                ("loguniform", 200, 8000), bank_tokens=10_000_000,
                                doc_offset_std=0.5, q_offset_std=0.5, n_queries=32,
                                lq=(16, 256), k=32),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (e.g. a smaller bank)."""
    return replace(WORKLOADS[name], **overrides) if overrides else WORKLOADS[name]


def layer(wl: Workload, l: int) -> Workload:
    """The tensor streams of routed layer l.  Every layer sees the same documents and
    query lengths: take those from the base workload (``doc_lengths(wl)``, and pass the
    base query lengths to ``gen_queries`` as ``lq_override``), and draw layer l's banks and
    query tensors from ``layer(wl, l)``."""
    return replace(wl, seed=wl.seed + 1000 * (l + 1))


# Independent generator streams, one per tensor.
STREAM = {"K": 1, "V": 2, "Kr": 3, "doc_off_K": 4, "doc_off_V": 5, "doc_off_Kr": 6,
          "Qr": 7, "q_off_Qr": 8, "Q": 9, "Kloc": 10, "Vloc": 11, "Kbar": 12, "Vbar": 13,
          "Krbar": 14}


def torch_gen(device, seed: int, stream: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + STREAM[stream])
    return g


def doc_lengths(wl: Workload) -> np.ndarray:
    """Document lengths (int64, every length >= 1).

    uniform:    integers in [lo, hi];
    loguniform: floor(exp(U(ln lo, ln(hi + 1)))), so values lie in [lo, hi].
    With ``bank_tokens`` set, documents are drawn until the total reaches the bank size
    and the last one is cut so the total is exact.
    """
    rng = np.random.default_rng(wl.seed)
    kind, lo, hi = wl.len_dist

    def draw(m):
        if kind == "uniform":
            return rng.integers(lo, hi + 1, size=m).astype(np.int64)
        if kind == "loguniform":
            u = rng.uniform(math.log(lo), math.log(hi + 1), size=m)
            return np.minimum(np.floor(np.exp(u)).astype(np.int64), hi)
        raise ValueError(kind)

    if wl.n_docs is not None:
        return draw(wl.n_docs)
    total = int(wl.bank_tokens)
    parts, acc = [], 0
    while acc < total:
        est = max(64, int(1.2 * (total - acc) / max(1.0, (lo + hi) / 4)))
        b = draw(est)
        parts.append(b)
        acc += int(b.sum())
    lens = np.concatenate(parts)
    cs = np.cumsum(lens)
    n = int(np.searchsorted(cs, total)) + 1          # first prefix reaching the total
    lens = lens[:n].copy()
    lens[-1] -= int(cs[n - 1]) - total
    if lens[-1] < 1:                                  # cannot happen: cs[n-2] < total
        raise AssertionError("length recipe produced an empty document")
    return lens


def token_offsets(lens: np.ndarray) -> np.ndarray:
    off = np.zeros(len(lens) + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens)
    return off


def _torch_dtype(dt: str):
    return torch.float32 if dt == "f32" else torch.bfloat16


def gen_token_states(wl: Workload, lens: np.ndarray, device, slice_tokens: int = 1 << 20,
                     needle_dirs: Optional[torch.Tensor] = None,
                     needle_ids: Optional[np.ndarray] = None):
    """Token-level document states K, V [T, H_kv, D] and Kr [T, H_r, D].

    Each token is N(0, 1) plus its document's offset, a vector drawn once per document
    and tensor from N(0, doc_offset_std^2).  Needle documents get the Kr offset
    a * needle_dirs[h] instead, with a chosen so that a full 64-token chunk mean makes
    cosine ``needle_cos`` with that direction: a^2 / (a^2 + D/64) = needle_cos^2.
    Generated on ``device`` in slices of ``slice_tokens`` tokens.
    """
    sh = wl.shape
    T = int(lens.sum())
    N = len(lens)
    dt = _torch_dtype(wl.dtype)
    doc_of_tok = torch.repeat_interleave(torch.arange(N, device=device),
                                         torch.as_tensor(lens, device=device))
    out = {}
    for name, heads in (("K", sh.h_kv), ("V", sh.h_kv), ("Kr", sh.h_r)):
        offs = None
        if wl.doc_offset_std > 0:
            offs = torch.randn((N, heads, sh.d), generator=torch_gen(device, wl.seed, "doc_off_" + name),
                               device=device, dtype=torch.float32) * wl.doc_offset_std
        if name == "Kr" and needle_ids is not None and len(needle_ids):
            if offs is None:
                offs = torch.zeros((N, heads, sh.d), device=device, dtype=torch.float32)
            c2 = wl.needle_cos ** 2
            a = math.sqrt(c2 * (sh.d / sh.chunk) / (1.0 - c2))
            ids_t = torch.as_tensor(needle_ids, device=device, dtype=torch.long)
            offs[ids_t] = a * needle_dirs.to(device=device, dtype=torch.float32)[None]
        X = torch.empty((T, heads, sh.d), device=device, dtype=dt)
        g = torch_gen(device, wl.seed, name)
        for t0 in range(0, T, slice_tokens):
            t1 = min(T, t0 + slice_tokens)
            x = torch.randn((t1 - t0, heads, sh.d), generator=g, device=device, dtype=torch.float32)
            if offs is not None:
                x += offs[doc_of_tok[t0:t1]]
            X[t0:t1].copy_(x)
        out[name] = X
    return out["K"], out["V"], out["Kr"]


def gen_queries(wl: Workload, device, lq_override: Optional[list] = None):
    """Query-side tensors for ``wl.n_queries`` queries.

    Returns dict with q_len (host int64 [B]), Qr [sum Lq, H_r, D], Q [sum Lq, Hq, D],
    Kloc / Vloc [sum Lkv, H_kv, D] with Lkv = Lq + decode_steps (the query's own tokens,
    then the decode tokens), and for decode the extra Qr / Q rows of the decode tokens.
    Qr is N(0, 1) plus a per-query, per-head offset from N(0, q_offset_std^2); the rest
    is N(0, 1).
    """
    sh = wl.shape
    rng = np.random.default_rng(wl.seed + 7)
    if lq_override is not None:
        q_len = np.asarray(lq_override, dtype=np.int64)
    else:
        q_len = rng.integers(wl.lq[0], wl.lq[1] + 1, size=wl.n_queries).astype(np.int64)
    B = len(q_len)
    steps = wl.decode_steps
    kv_len = q_len + steps
    Tq = int(q_len.sum()) + B * steps
    dt = _torch_dtype(wl.dtype)

    def randn(shape, stream):
        return torch.randn(shape, generator=torch_gen(device, wl.seed, stream), device=device,
                           dtype=torch.float32)

    qr = randn((Tq, sh.h_r, sh.d), "Qr")
    if wl.q_offset_std > 0:
        qoff = randn((B, sh.h_r, sh.d), "q_off_Qr") * wl.q_offset_std
        owner = torch.repeat_interleave(torch.arange(B, device=device),
                                        torch.as_tensor(q_len + steps, device=device))
        qr += qoff[owner]
    q = randn((Tq, sh.hq, sh.d), "Q")
    kl = randn((int(kv_len.sum()), sh.h_kv, sh.d), "Kloc")
    vl = randn((int(kv_len.sum()), sh.h_kv, sh.d), "Vloc")
    # Row layout of Qr / Q: query b's prefill rows, then its decode rows, query after query.
    return {"q_len": q_len, "kv_len": kv_len, "decode_steps": steps,
            "Qr": qr.to(dt), "Q": q.to(dt), "Kloc": kl.to(dt), "Vloc": vl.to(dt)}


def plant_needles(wl: Workload, n_docs: int, qr_prefill: torch.Tensor):
    """Needle document ids (distinct, seeded) and the per-head unit direction of the mean
    of the query's routing vectors over its tokens."""
    rng = np.random.default_rng(wl.seed + 11)
    ids = np.sort(rng.choice(n_docs, size=wl.needles, replace=False)).astype(np.int64)
    m = qr_prefill.float().mean(dim=0)                      # [H_r, D]
    dirs = m / m.norm(dim=-1, keepdim=True)
    return ids, dirs


def gen_pooled_bank(wl: Workload, chunk_off: np.ndarray, device, kv_device=None,
                    slice_rows: int = 1 << 16, needle_dirs: Optional[torch.Tensor] = None,
                    needle_ids: Optional[np.ndarray] = None, krbar_only: bool = False):
    """A bank drawn directly at chunk level (for banks whose token states exceed memory).

    Row c of document d is mu_d + 0.125 * eps with mu_d ~ N(0, doc_offset_std^2) per
    document and tensor and eps ~ N(0, 1) per element: 0.125 = 1/sqrt(64) is the spread
    of the mean of a full chunk of unit-variance tokens.  ``chunk_off`` ([N+1]) gives each
    document's rows.  Krbar is placed on ``device``; Kbar / Vbar on ``kv_device``
    ("cpu-pinned" for page-locked host memory, else a torch device), or not drawn at all
    with ``krbar_only`` (then None).  Needle documents get the Krbar offset
    a * needle_dirs[h] instead of mu_d, with a chosen as in ``gen_token_states``: a row
    then makes cosine ``needle_cos`` with that direction, a^2 / (a^2 + D/64) = needle_cos^2.
    """
    sh = wl.shape
    N = len(chunk_off) - 1
    C = int(chunk_off[-1])
    dt = _torch_dtype(wl.dtype)
    counts = torch.as_tensor(np.diff(chunk_off), device=device)
    doc_of_row = torch.repeat_interleave(torch.arange(N, device=device), counts)
    kv_device = device if kv_device is None else kv_device
    out = {"Kbar": None, "Vbar": None}
    tensors = (("Krbar", sh.h_r, device),) if krbar_only else (
        ("Krbar", sh.h_r, device), ("Kbar", sh.h_kv, kv_device), ("Vbar", sh.h_kv, kv_device))
    for name, heads, where in tensors:
        mu = torch.randn((N, heads, sh.d), generator=torch_gen(device, wl.seed, name),
                         device=device, dtype=torch.float32) * wl.doc_offset_std
        if name == "Krbar" and needle_ids is not None and len(needle_ids):
            c2 = wl.needle_cos ** 2
            a = math.sqrt(c2 * (sh.d / sh.chunk) / (1.0 - c2))
            ids_t = torch.as_tensor(needle_ids, device=device, dtype=torch.long)
            mu[ids_t] = a * needle_dirs.to(device=device, dtype=torch.float32)[None]
        g = torch_gen(device, wl.seed + 500, name)
        if where == "cpu-pinned":
            X = torch.empty((C, heads, sh.d), dtype=dt, pin_memory=True)
        else:
            X = torch.empty((C, heads, sh.d), dtype=dt, device=where)
        for r0 in range(0, C, slice_rows):
            r1 = min(C, r0 + slice_rows)
            x = torch.randn((r1 - r0, heads, sh.d), generator=g, device=device,
                            dtype=torch.float32) * 0.125
            x += mu[doc_of_row[r0:r1]]
            X[r0:r1].copy_(x.to(dt))
        out[name] = X
    return out["Krbar"], out["Kbar"], out["Vbar"]
