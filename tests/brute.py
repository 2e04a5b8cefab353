"""Pure-Python brute force for tiny inputs: the oracle's oracle.

Written independently of ``oracle.msa_oracle`` (different formulation where one exists:
RoPE through complex multiplication, top-k through rank counting, softmax through
explicit sums) so that a mistake in either one shows up as a disagreement.
Inputs are nested lists or NumPy arrays; everything is Python floats.
"""
from __future__ import annotations

import cmath
import math


def rope_pairs(vec, pos, base):
    """Rotate one head vector with complex numbers: z_i = x_i + j*x_{i+D/2},
    z_i' = z_i * exp(j * pos * base**(-2i/D))."""
    D = len(vec)
    h = D // 2
    out = [0.0] * D
    for i in range(h):
        z = complex(float(vec[i]), float(vec[i + h])) * cmath.exp(1j * pos * base ** (-2.0 * i / D))
        out[i] = z.real
        out[i + h] = z.imag
    return out


def pool_brute(X, doc_lens, chunk, base, rotate):
    """Chunk means of X [T][H][D] per document, rotating each token at its in-document
    position first when ``rotate``."""
    rows = []
    t = 0
    for L in doc_lens:
        j = 0
        while j * chunk < L:
            lo, hi = j * chunk, min((j + 1) * chunk, L)
            H = len(X[t])
            D = len(X[t][0])
            acc = [[0.0] * D for _ in range(H)]
            for p in range(lo, hi):
                for h in range(H):
                    v = rope_pairs(X[t + p][h], p, base) if rotate else [float(a) for a in X[t + p][h]]
                    for e in range(D):
                        acc[h][e] += v[e]
            n = hi - lo
            rows.append([[a / n for a in acc[h]] for h in range(H)])
            j += 1
        t += L
    return rows


def doc_scores_brute(Qr, Krbar, chunk_off):
    """Doc score = max over (token, chunk of the doc) of the head-mean cosine."""
    T = len(Qr)
    H = len(Qr[0])
    out = []
    for d in range(len(chunk_off) - 1):
        best = -math.inf
        for c in range(int(chunk_off[d]), int(chunk_off[d + 1])):
            for t in range(T):
                tot = 0.0
                for h in range(H):
                    q = [float(a) for a in Qr[t][h]]
                    k = [float(a) for a in Krbar[c][h]]
                    qq = math.sqrt(sum(a * a for a in q))
                    kk = math.sqrt(sum(a * a for a in k))
                    dot = sum(a * b for a, b in zip(q, k))
                    tot += 0.0 if qq == 0 or kk == 0 else dot / (qq * kk)
                best = max(best, tot / H)
        out.append(best)
    return out


def topk_brute(scores, k):
    """Rank of d = number of documents that beat it (higher score, or equal score and
    lower id); the top-k are the documents of rank < k, listed by rank."""
    N = len(scores)
    rank = []
    for d in range(N):
        r = 0
        for e in range(N):
            if scores[e] > scores[d] or (scores[e] == scores[d] and e < d):
                r += 1
        rank.append(r)
    by_rank = sorted(range(N), key=lambda d: rank[d])
    keff = min(k, N)
    return by_rank[:keff] + [-1] * (k - keff)


def attention_brute(Q, Kloc, Vloc, Kmem, Vmem, k_eff, base, scale=None, with_lse=False):
    """Explicit loops: rotate local query/keys at k_eff + local index, softmax over
    every memory key and the causal local keys, weighted sum of values.  with_lse also
    returns each row's log of the softmax normaliser, log sum_j exp(logit_j)."""
    Lq, Hq, D = len(Q), len(Q[0]), len(Q[0][0])
    Lkv, Hkv = len(Kloc), len(Kloc[0])
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(Lq)]
    lse = [[0.0] * Hq for _ in range(Lq)]
    for t in range(Lq):
        i = Lkv - Lq + t
        for hq in range(Hq):
            g = hq // G
            q = rope_pairs(Q[t][hq], k_eff + i, base)
            keys, vals = [], []
            for m in range(len(Kmem)):
                keys.append([float(a) for a in Kmem[m][g]])
                vals.append([float(a) for a in Vmem[m][g]])
            for j in range(i + 1):
                keys.append(rope_pairs(Kloc[j][g], k_eff + j, base))
                vals.append([float(a) for a in Vloc[j][g]])
            logits = [scale * sum(a * b for a, b in zip(q, kv)) for kv in keys]
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            z = sum(w)
            lse[t][hq] = mx + math.log(z)
            for e in range(D):
                out[t][hq][e] = sum(w[n] * vals[n][e] for n in range(len(w))) / z
    return (out, lse) if with_lse else out
