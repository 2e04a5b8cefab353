"""CPU oracle (NumPy, float64) for Memory Sparse Attention's routing + sparse-attention path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the HIP product path, with which it
shares no code.

Sources (the web pages this project is built from; cited by page and section):

* [hysenlabs] hysenlabs.com, "EverMind-AI/MSA: routing top-k compressed documents
  inside attention, and where the 100M-token claim stops", editorial sections
  "Routing happens inside attention ...", "Document-wise RoPE resets every document
  to position zero", "Memory must be encoded offline before a query can reach it",
  "The 100M-token setup depends on host memory as well as two GPUs".
* [yeyulingfeng] yeyulingfeng.com, "深度分析MSA：把超长文档组织成可检索内部记忆的工程路径",
  sections 三 (how documents become memory: chunk compression), 四 (training: the
  language-model loss and the routing auxiliary loss) and 五 (inference: routing
  retrieval, local generation).
* [github-wiki] github-wiki.com project 250, "MSA 记忆稀疏注意力框架 ...",
  section 6 (implementation features).

Each function states which passage it follows.  Where the pages leave a step open
the function implements the declared reading (R-number) listed in the design notes;
those readings are:

  R1  document-wise RoPE rotates K only (V and Kr are not rotated) unless a mask says so;
  R2  rotate-half pairing (i, i + D/2), theta_i = base^(-2i/D);
  R4  a document of L tokens has ceil(L/chunk) chunks; the last one is the mean of its
      real tokens only;
  R5  chunks never span two documents;
  R6  per-head cosine, then mean over heads, then max over query tokens;
  R7  a zero-norm vector has cosine 0 with everything;
  R8  document score = max over the document's chunk scores   (parity unpinned by the
      pages: the rule is a declaration, the code is pinned against brute force);
  R9  top-k order is (score descending, document id ascending), k_eff = min(k, N),
      unused slots hold id -1;
  R11 memory keys keep the document-wise rotation they got before pooling and are
      not rotated again                                       (parity unpinned by the
      pages: a declaration, pinned against brute force);
  R12 local token j of the active context sits at global position k_eff + j;
  R13 every query token sees all memory keys; local keys are causal;
  R14 GQA: query head hq uses kv head hq // (Hq / H_kv);
  R15 softmax scale 1/sqrt(D), no extras;
  R16 bf16 values are produced by one round-to-nearest-even from float64;
  R25 a query with no tokens scores -inf on every document (the maximum over an empty set
      of tokens), so its top-k is the k_eff lowest ids;
  R26 backward of step D: the gradient of sum(dO * O) through the same computation
      (softmax, GQA, global RoPE of the local context); memory rows' gradients are summed
      into bank-shaped arrays over every query that selected them;
  R27 backward of the router: a document score is one maximum over (query token, bank
      row), so its gradient reaches only the maximising pair -- the first in row-major
      order over (bank row, token) -- through that pair's head-mean of cosines; a zero
      vector has cosine 0 and gets no gradient;
  R28 the routing auxiliary loss supervises the document scores S in one of the two forms
      the training section names, on logits z = S / temperature, averaged over queries:
      BCE: the mean over documents of binary cross-entropy with logits against labels y
      in [0, 1]; InfoNCE: -log of the label-weighted share of softmax(z) (y >= 0; one
      positive gives the usual cross-entropy).  A query with a non-finite score (a query
      without tokens) or, for InfoNCE, without a positive label contributes nothing.

Precision: every computation is float64.  Inputs given as bf16 are decoded exactly.
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np

ROPE_K = 1
ROPE_V = 2
ROPE_KR = 4

__all__ = [
    "ROPE_K", "ROPE_V", "ROPE_KR",
    "bf16_bits_to_f64", "f64_to_bf16_bits", "round_to_bf16", "round_to_f32", "round_to",
    "chunk_counts", "chunk_offsets",
    "rope_inv_freq", "rope_rotate",
    "pool",
    "head_cosines", "token_chunk_scores", "chunk_scores", "doc_scores_one", "route_doc_scores",
    "topk_docs", "route",
    "assemble_memory", "sparse_attention_one", "sparse_attn",
    "sparse_attention_backward_one", "sparse_attn_backward", "route_backward",
    "AUX_BCE", "AUX_INFONCE", "route_aux_loss",
]


# ---------------------------------------------------------------------------------------
# bf16 encoding (R16).  bf16 = the top 16 bits of an IEEE float32: 1 sign, 8 exponent,
# 7 stored mantissa bits.
# ---------------------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) exactly into float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, in one step (R16).

    A finite x = m * 2**e with 0.5 <= |m| < 1 has bf16 neighbours spaced 2**(e-8)
    apart (8 significant bits).  Below the normal range the spacing is fixed at
    2**-133.  np.rint rounds half to even.  Values beyond the largest bf16 become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(xf, -q)), q)
    bf16_max = float(np.ldexp(255.0, 120))           # (2 - 2**-7) * 2**127
    r = np.where(np.abs(r) > bf16_max, np.copysign(np.inf, r), r)
    out[finite] = r
    out[~finite] = x[~finite]
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """Encode float64 values as bf16 bit patterns (uint16) with one RNE rounding."""
    r = round_to_bf16(x).astype(np.float32)  # exact: every bf16 value is a float32 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_to_f32(x) -> np.ndarray:
    """Round float64 to float32 (NumPy's cast is a single round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, dtype: str) -> np.ndarray:
    """Round to the run's storage type: "f32" or "bf16"."""
    if dtype == "f32":
        return round_to_f32(x)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------------------
# Chunking ([yeyulingfeng] section 三.2: every 64 tokens become one chunk; its worked
# example turns 180 tokens into 3 chunks, which fixes rounding up, R4).
# ---------------------------------------------------------------------------------------

def chunk_counts(doc_lens: Sequence[int], chunk: int = 64) -> np.ndarray:
    """Number of chunks of each document: ceil(L / chunk) (R4)."""
    lens = np.asarray(doc_lens, dtype=np.int64)
    if chunk < 1 or np.any(lens < 1):
        raise ValueError("chunk >= 1 and every document needs >= 1 token")
    return (lens + chunk - 1) // chunk


def chunk_offsets(doc_lens: Sequence[int], chunk: int = 64) -> np.ndarray:
    """Exclusive prefix sum of chunk counts: document d owns bank rows
    [off[d], off[d+1]) (R5: chunks never span documents)."""
    n = chunk_counts(doc_lens, chunk)
    off = np.zeros(len(n) + 1, dtype=np.int64)
    off[1:] = np.cumsum(n)
    return off


# ---------------------------------------------------------------------------------------
# Rotary position embedding.  Document-wise use: [hysenlabs] "Document-wise RoPE resets
# every document to position zero".  Global use for the active context: same section,
# second paragraph (query start offset by the number of retrieved blocks).
# ---------------------------------------------------------------------------------------

def rope_inv_freq(d: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d) for i in [0, d/2)  (R2)."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def rope_rotate(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate x[t, h, :] by angle pos[t] * theta_i on the pair (i, i + D/2) (R2).

    x'_i       = x_i cos(a) - x_{i+D/2} sin(a)
    x'_{i+D/2} = x_{i+D/2} cos(a) + x_i sin(a),   a = pos * theta_i
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("head dim must be even")
    a = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(d, base)[None, :]
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    lo, hi = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# ---------------------------------------------------------------------------------------
# Step A: offline memory encoding by chunk-mean pooling.
# [yeyulingfeng] section 三.1-三.3 (token-level K, V, K_r per document; mean pooling per
# 64-token chunk; the bank holds K-bar, V-bar, K_r-bar); [hysenlabs] "Routing happens
# inside attention" (chunk-mean pooling of K, V, Kr) and "Document-wise RoPE resets ...".
# ---------------------------------------------------------------------------------------

def pool(K, V, Kr, doc_tok_off, chunk: int = 64, base: float = 1e6, rope_mask: int = ROPE_K):
    """Pool token-level document states into bank rows.

    K, V: [T, H_kv, D];  Kr: [T, H_r, D];  doc_tok_off: [N+1] token offsets.
    Returns (Kbar, Vbar, Krbar, chunk_off), float64, rows ordered by document then chunk.

    For each document d and in-document position p (restarting at 0, R3), the tensors
    selected by rope_mask are rotated at p; then chunk j of d is the plain mean of the
    rotated/raw rows of tokens [j*chunk, min((j+1)*chunk, L_d)) (R4, R5).
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Kr = np.asarray(Kr, dtype=np.float64)
    off = np.asarray(doc_tok_off, dtype=np.int64)
    lens = np.diff(off)
    coff = chunk_offsets(lens, chunk)
    C = int(coff[-1])
    outs = []
    for X, bit in ((K, ROPE_K), (V, ROPE_V), (Kr, ROPE_KR)):
        Y = np.zeros((C,) + X.shape[1:], dtype=np.float64)
        for d in range(len(lens)):
            t0, t1 = int(off[d]), int(off[d + 1])
            rows = X[t0:t1]
            if rope_mask & bit:
                rows = rope_rotate(rows, np.arange(t1 - t0), base)
            for j in range(int(coff[d + 1] - coff[d])):
                seg = rows[j * chunk: min((j + 1) * chunk, t1 - t0)]
                Y[coff[d] + j] = seg.sum(axis=0) / seg.shape[0]
        outs.append(Y)
    return outs[0], outs[1], outs[2], coff


# ---------------------------------------------------------------------------------------
# Step B: router relevance.  [hysenlabs] "Routing happens inside attention": cosine
# similarity between the query's routing vectors and the pooled routing keys, averaged
# over heads, then the maximum over the query's tokens (R6); [yeyulingfeng] section 五
# step 2 (Q_r against K_r-bar gives a document score, then top-k).
# ---------------------------------------------------------------------------------------

def head_cosines(Qr_q: np.ndarray, Krbar: np.ndarray) -> np.ndarray:
    """cos[t, c, h] between Qr_q[t, h] and Krbar[c, h]; 0 where either norm is 0 (R7)."""
    Q = np.asarray(Qr_q, dtype=np.float64)
    Kb = np.asarray(Krbar, dtype=np.float64)
    dots = np.einsum("thd,chd->tch", Q, Kb)
    qn = np.sqrt(np.einsum("thd,thd->th", Q, Q))
    kn = np.sqrt(np.einsum("chd,chd->ch", Kb, Kb))
    den = qn[:, None, :] * kn[None, :, :]
    out = np.zeros_like(dots)
    nz = den > 0
    out[nz] = dots[nz] / den[nz]
    return out


def token_chunk_scores(Qr_q, Krbar) -> np.ndarray:
    """s[t, c] = mean over heads of the per-head cosine (R6)."""
    return head_cosines(Qr_q, Krbar).mean(axis=2)


def chunk_scores(Qr_q, Krbar) -> np.ndarray:
    """S[c] = max over query tokens t of s[t, c] (R6); -inf for a query with no tokens (R25)."""
    if np.asarray(Qr_q).shape[0] == 0:
        return np.full(np.asarray(Krbar).shape[0], -np.inf)
    return token_chunk_scores(Qr_q, Krbar).max(axis=0)


def doc_scores_one(Qr_q, Krbar, chunk_off) -> np.ndarray:
    """D[d] = max over the chunks of document d of S[c] (R8)."""
    S = chunk_scores(Qr_q, Krbar)
    off = np.asarray(chunk_off, dtype=np.int64)
    return np.array([S[off[d]:off[d + 1]].max() for d in range(len(off) - 1)], dtype=np.float64)


def route_doc_scores(Qr, q_off, Krbar, chunk_off, block: int = 0) -> np.ndarray:
    """Doc scores for every query b (rows [q_off[b], q_off[b+1]) of Qr): [B, N].

    ``block`` > 0 evaluates the documents in groups of about that many bank rows to bound
    memory; each document's score is computed whole inside one group, so the result is
    the same as with block = 0.
    """
    q_off = np.asarray(q_off, dtype=np.int64)
    coff = np.asarray(chunk_off, dtype=np.int64)
    N = len(coff) - 1
    out = np.zeros((len(q_off) - 1, N), dtype=np.float64)
    groups = [(0, N)]
    if block > 0:
        groups, d0 = [], 0
        while d0 < N:
            d1 = d0 + 1
            while d1 < N and coff[d1 + 1] - coff[d0] <= block:
                d1 += 1
            groups.append((d0, d1))
            d0 = d1
    for b in range(len(q_off) - 1):
        Qb = np.asarray(Qr[q_off[b]:q_off[b + 1]], dtype=np.float64)
        for d0, d1 in groups:
            sub = np.asarray(Krbar[coff[d0]:coff[d1]], dtype=np.float64)
            out[b, d0:d1] = doc_scores_one(Qb, sub, coff[d0:d1 + 1] - coff[d0])
    return out


# ---------------------------------------------------------------------------------------
# Step C: top-k document selection ([github-wiki] section 6 item 1; [yeyulingfeng] section
# 五 step 2; [hysenlabs] "Routing happens inside attention").  Order (R9).
# ---------------------------------------------------------------------------------------

def topk_docs(scores: np.ndarray, k: int):
    """The k_eff = min(k, N) documents with the largest score, ties to the lower id.

    Returns (ids[k] int32, vals[k] float64); unused slots hold id -1 and score -inf.
    """
    if k < 1:
        raise ValueError("k must be >= 1")
    sc = np.asarray(scores, dtype=np.float64)
    order = sorted(range(len(sc)), key=lambda d: (-sc[d], d))
    keff = min(k, len(sc))
    ids = np.full(k, -1, dtype=np.int32)
    vals = np.full(k, -np.inf, dtype=np.float64)
    ids[:keff] = order[:keff]
    vals[:keff] = sc[order[:keff]]
    return ids, vals


def route(Qr, q_off, Krbar, chunk_off, k: int, block: int = 0):
    """Steps B + C for every query: (ids [B,k], top scores [B,k], doc scores [B,N])."""
    D = route_doc_scores(Qr, q_off, Krbar, chunk_off, block=block)
    ids = np.zeros((D.shape[0], k), dtype=np.int32)
    vals = np.zeros((D.shape[0], k), dtype=np.float64)
    for b in range(D.shape[0]):
        ids[b], vals[b] = topk_docs(D[b], k)
    return ids, vals, D


# ---------------------------------------------------------------------------------------
# Step D: context assembly and sparse attention.
# [hysenlabs] "Routing happens inside attention" (the selected documents' compressed K/V
# are concatenated with the query's local K/V) and "Document-wise RoPE ..." second
# paragraph (global RoPE on the active context, query start offset by k, causal order
# memory -> query -> generation); [yeyulingfeng] section 五 step 3 (the generation context
# is the query's local states plus the top-k memory).
# ---------------------------------------------------------------------------------------

def assemble_memory(ids_b, chunk_off, Kbar, Vbar):
    """Concatenate, in rank order, every bank row of each selected document (R11)."""
    coff = np.asarray(chunk_off, dtype=np.int64)
    rows = [np.arange(coff[d], coff[d + 1]) for d in ids_b if d >= 0]
    idx = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return (np.asarray(Kbar[idx], dtype=np.float64), np.asarray(Vbar[idx], dtype=np.float64))


def sparse_attention_one(Q_b, Kloc_b, Vloc_b, Kmem, Vmem, k_eff: int, base: float,
                         scale: float | None = None, with_lse: bool = False):
    """Attention of one query's tokens over [memory ; causal local context].

    Q_b: [Lq, Hq, D]; Kloc_b, Vloc_b: [Lkv, H_kv, D] (Lkv >= Lq; the query's tokens are
    the last Lq local tokens); Kmem, Vmem: [M, H_kv, D].
    Local token j is rotated at global position k_eff + j (R12), memory keys are used as
    pooled (R11); query token t is local token Lkv - Lq + t and sees every memory key and
    local keys j <= Lkv - Lq + t (R13).  kv head of hq = hq // (Hq/H_kv) (R14).
    with_lse also returns [Lq, Hq]: the natural log of each row's softmax normaliser,
    log sum_j exp(logit_j) over the keys the row sees (what a backward pass reuses).
    """
    Q_b = np.asarray(Q_b, dtype=np.float64)
    Kl = np.asarray(Kloc_b, dtype=np.float64)
    Vl = np.asarray(Vloc_b, dtype=np.float64)
    Lq, Hq, D = Q_b.shape
    Lkv, Hkv, _ = Kl.shape
    if Lkv < Lq or Hq % Hkv:
        raise ValueError("need Lkv >= Lq and Hq % H_kv == 0")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    G = Hq // Hkv
    Qr_ = rope_rotate(Q_b, k_eff + (Lkv - Lq) + np.arange(Lq), base)
    Klr = rope_rotate(Kl, k_eff + np.arange(Lkv), base)
    M = Kmem.shape[0]
    qpos = (Lkv - Lq) + np.arange(Lq)
    mask = np.arange(Lkv)[None, :] <= qpos[:, None]           # [Lq, Lkv]
    out = np.zeros((Lq, Hq, D), dtype=np.float64)
    lse = np.zeros((Lq, Hq), dtype=np.float64)
    for hq in range(Hq):
        g = hq // G
        keys = np.concatenate([Kmem[:, g, :], Klr[:, g, :]], axis=0)   # [M+Lkv, D]
        vals = np.concatenate([Vmem[:, g, :], Vl[:, g, :]], axis=0)
        logits = scale * (Qr_[:, hq, :] @ keys.T)                       # [Lq, M+Lkv]
        logits[:, M:][~mask] = -np.inf
        mx = logits.max(axis=1, keepdims=True)
        logits -= mx
        p = np.exp(logits)
        z = p.sum(axis=1, keepdims=True)
        lse[:, hq] = (mx + np.log(z))[:, 0]
        p /= z
        out[:, hq, :] = p @ vals
    return (out, lse) if with_lse else out


def sparse_attn(Q, Kloc, Vloc, q_off, kv_off, ids, chunk_off, Kbar, Vbar, base: float,
                scale: float | None = None, queries: Sequence[int] | None = None) -> np.ndarray:
    """Step D for every query (or the listed ones): O [total_q, Hq, D] float64.

    Rows of queries that are not listed are left as NaN.
    """
    q_off = np.asarray(q_off, dtype=np.int64)
    kv_off = np.asarray(kv_off, dtype=np.int64)
    ids = np.asarray(ids)
    out = np.full(np.asarray(Q).shape, np.nan, dtype=np.float64)
    todo = range(len(q_off) - 1) if queries is None else queries
    for b in todo:
        Km, Vm = assemble_memory(ids[b], chunk_off, Kbar, Vbar)
        keff = int(np.sum(ids[b] >= 0))
        out[q_off[b]:q_off[b + 1]] = sparse_attention_one(
            Q[q_off[b]:q_off[b + 1]], Kloc[kv_off[b]:kv_off[b + 1]],
            Vloc[kv_off[b]:kv_off[b + 1]], Km, Vm, keff, base, scale)
    return out


def sparse_attn_lse(Q, Kloc, Vloc, q_off, kv_off, ids, chunk_off, Kbar, Vbar, base: float,
                    scale: float | None = None) -> np.ndarray:
    """Each row's log-sum-exp of its logits over the keys it sees, [total_q, Hq] float64
    (natural log), as returned alongside O by sparse_attention_one."""
    q_off = np.asarray(q_off, dtype=np.int64)
    kv_off = np.asarray(kv_off, dtype=np.int64)
    ids = np.asarray(ids)
    out = np.zeros(np.asarray(Q).shape[:2], dtype=np.float64)
    for b in range(len(q_off) - 1):
        Km, Vm = assemble_memory(ids[b], chunk_off, Kbar, Vbar)
        keff = int(np.sum(ids[b] >= 0))
        out[q_off[b]:q_off[b + 1]] = sparse_attention_one(
            Q[q_off[b]:q_off[b + 1]], Kloc[kv_off[b]:kv_off[b + 1]],
            Vloc[kv_off[b]:kv_off[b + 1]], Km, Vm, keff, base, scale, with_lse=True)[1]
    return out


# ---------------------------------------------------------------------------------------
# Backward of step D and of the router (training: [yeyulingfeng] section 四 -- the
# language-model loss reaches Q, K/V and Q_r/K_r through the selected memory, and a routing
# auxiliary loss supervises the document scores; [github-wiki] section 6 item 1 -- the
# layer stays differentiable end to end).  Readings R26, R27.
# ---------------------------------------------------------------------------------------

def sparse_attention_backward_one(Q_b, Kloc_b, Vloc_b, Kmem, Vmem, k_eff: int, base: float, dO_b,
                                  scale: float | None = None):
    """Gradients of L = sum(dO_b * O_b), O_b = sparse_attention_one(...), with respect to
    Q_b, Kloc_b, Vloc_b (un-rotated inputs), Kmem and Vmem: a tuple of float64 arrays of
    their shapes.  Per query head: dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(dO O)),
    dQ~ = scale dS K, dK~ = scale dS^T Q~; the rotations of Q and the local K are undone by
    rotating the gradient by the negative angle; kv head g sums over its query heads."""
    Q_b = np.asarray(Q_b, dtype=np.float64)
    Kl = np.asarray(Kloc_b, dtype=np.float64)
    Vl = np.asarray(Vloc_b, dtype=np.float64)
    Km = np.asarray(Kmem, dtype=np.float64)
    Vm = np.asarray(Vmem, dtype=np.float64)
    dO = np.asarray(dO_b, dtype=np.float64)
    Lq, Hq, D = Q_b.shape
    Lkv, Hkv, _ = Kl.shape
    M = Km.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    G = Hq // Hkv
    qpos = k_eff + (Lkv - Lq) + np.arange(Lq)
    kpos = k_eff + np.arange(Lkv)
    Qr_ = rope_rotate(Q_b, qpos, base)
    Klr = rope_rotate(Kl, kpos, base)
    mask = np.arange(Lkv)[None, :] <= ((Lkv - Lq) + np.arange(Lq))[:, None]
    dQr = np.zeros_like(Qr_)
    dKall = np.zeros((M + Lkv, Hkv, D))
    dVall = np.zeros((M + Lkv, Hkv, D))
    for hq in range(Hq):
        g = hq // G
        keys = np.concatenate([Km[:, g, :], Klr[:, g, :]], axis=0)
        vals = np.concatenate([Vm[:, g, :], Vl[:, g, :]], axis=0)
        logits = scale * (Qr_[:, hq, :] @ keys.T)
        logits[:, M:][~mask] = -np.inf
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        o = p @ vals
        do = dO[:, hq, :]
        dVall[:, g, :] += p.T @ do
        dp = do @ vals.T
        ds = p * (dp - np.sum(do * o, axis=1, keepdims=True))
        dQr[:, hq, :] = scale * (ds @ keys)
        dKall[:, g, :] += scale * (ds.T @ Qr_[:, hq, :])
    dQ = rope_rotate(dQr, -qpos, base)
    dKl = rope_rotate(dKall[M:], -kpos, base)
    return dQ, dKl, dVall[M:], dKall[:M], dVall[:M]


def sparse_attn_backward(Q, Kloc, Vloc, q_off, kv_off, ids, chunk_off, Kbar, Vbar, base: float, dO,
                         scale: float | None = None):
    """Backward of step D for every query: (dQ, dKloc, dVloc, dKbar, dVbar), float64, with
    dKbar / dVbar shaped like the bank and summed over the queries that selected a row."""
    q_off = np.asarray(q_off, dtype=np.int64)
    kv_off = np.asarray(kv_off, dtype=np.int64)
    coff = np.asarray(chunk_off, dtype=np.int64)
    ids = np.asarray(ids)
    dQ = np.zeros(np.asarray(Q).shape)
    dKl = np.zeros(np.asarray(Kloc).shape)
    dVl = np.zeros(np.asarray(Vloc).shape)
    dKb = np.zeros(np.asarray(Kbar).shape)
    dVb = np.zeros(np.asarray(Vbar).shape)
    for b in range(len(q_off) - 1):
        Km, Vm = assemble_memory(ids[b], chunk_off, Kbar, Vbar)
        keff = int(np.sum(ids[b] >= 0))
        q0, q1, k0, k1 = q_off[b], q_off[b + 1], kv_off[b], kv_off[b + 1]
        gq, gk, gv, gkm, gvm = sparse_attention_backward_one(
            Q[q0:q1], Kloc[k0:k1], Vloc[k0:k1], Km, Vm, keff, base, dO[q0:q1], scale)
        dQ[q0:q1] = gq
        dKl[k0:k1] = gk
        dVl[k0:k1] = gv
        idx = np.concatenate([np.arange(coff[d], coff[d + 1]) for d in ids[b] if d >= 0]
                             + [np.zeros(0, dtype=np.int64)])
        np.add.at(dKb, idx, gkm)
        np.add.at(dVb, idx, gvm)
    return dQ, dKl, dVl, dKb, dVb


def route_backward(Qr, q_off, Krbar, chunk_off, dD):
    """Gradients of L = sum(dD * D) with D = route_doc_scores(Qr, q_off, Krbar, chunk_off),
    with respect to Qr and Krbar (R27): (dQr, dKrbar), float64.  For query b and document d
    with dD[b, d] != 0, the maximising pair (t*, c*) receives
        dQr[t*, h]    += dD[b, d] / H * (khat - cos_h qhat) / |q|
        dKrbar[c*, h] += dD[b, d] / H * (qhat - cos_h khat) / |k|
    with qhat, khat the unit vectors of Qr[t*, h] and Krbar[c*, h] (no gradient to a zero
    vector)."""
    Qr = np.asarray(Qr, dtype=np.float64)
    Kb = np.asarray(Krbar, dtype=np.float64)
    q_off = np.asarray(q_off, dtype=np.int64)
    coff = np.asarray(chunk_off, dtype=np.int64)
    dD = np.asarray(dD, dtype=np.float64)
    H = Qr.shape[1]
    dQr = np.zeros_like(Qr)
    dKb = np.zeros_like(Kb)
    for b in range(len(q_off) - 1):
        Qb = Qr[q_off[b]:q_off[b + 1]]
        if len(Qb) == 0:
            continue
        for d in range(len(coff) - 1):
            gd = dD[b, d]
            if gd == 0:
                continue
            s = token_chunk_scores(Qb, Kb[coff[d]:coff[d + 1]])        # [T, rows]
            j = int(np.argmax(s.T))                                     # row-major over (row, t)
            c = int(coff[d] + j // s.shape[0])
            t = int(j % s.shape[0])
            for h in range(H):
                q, k = Qb[t, h], Kb[c, h]
                nq, nk = np.linalg.norm(q), np.linalg.norm(k)
                if nq == 0 or nk == 0:
                    continue
                qh, kh = q / nq, k / nk
                cs = float(qh @ kh)
                dQr[q_off[b] + t, h] += gd / H * (kh - cs * qh) / nq
                dKb[c, h] += gd / H * (qh - cs * kh) / nk
    return dQr, dKb


# ---------------------------------------------------------------------------------------
# Routing auxiliary loss ([yeyulingfeng] section 四, training signal 2: the document scores
# are supervised, commonly with BCE or InfoNCE).  Reading R28.
# ---------------------------------------------------------------------------------------

AUX_BCE = 0
AUX_INFONCE = 1


def _softplus(z):
    """log(1 + e^z), evaluated without overflow."""
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def _sigmoid(z):
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def route_aux_loss(kind: int, scores, labels, temperature: float = 1.0):
    """Per-query losses l[b] and the gradient dD = dL/dS of L = mean_b l[b] (R28), float64.

    BCE:     l[b] = (1/N) sum_d [softplus(z) - y z],   dl/dz = (sigmoid(z) - y) / N
    InfoNCE: l[b] = log sum_d e^z - log sum_d y e^z,   dl/dz = softmax(z) - y e^z / sum y e^z
    with z = S[b] / temperature; a skipped query has l[b] = 0 and a zero gradient row."""
    S = np.asarray(scores, dtype=np.float64)
    Y = np.asarray(labels, dtype=np.float64)
    B, N = S.shape
    loss = np.zeros(B)
    dD = np.zeros((B, N))
    for b in range(B):
        if not np.all(np.isfinite(S[b])):
            continue
        z = S[b] / temperature
        y = Y[b]
        if kind == AUX_BCE:
            loss[b] = float(np.mean(_softplus(z) - y * z))
            dz = (_sigmoid(z) - y) / N
        elif kind == AUX_INFONCE:
            if not np.any(y > 0):
                continue
            # each log-sum-exp shifted by its own maximum, so neither sum underflows
            m = z.max()
            mp = z[y > 0].max()
            e, ep = np.exp(z - m), np.zeros_like(z)
            ep[y > 0] = np.exp(z[y > 0] - mp)
            tot, pos = e.sum(), (y * ep).sum()
            loss[b] = float((m + np.log(tot)) - (mp + np.log(pos)))
            dz = e / tot - y * ep / pos
        else:
            raise ValueError(f"unknown loss kind {kind}")
        dD[b] = dz / temperature / B
    return loss, dD
