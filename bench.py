"""Benchmark of the MSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload bank100m_host]

One step is one query through the router and the sparse attention: the routing scan of
every bank row (msa_route_scan), top-k document selection (msa_topk), and sparse attention
over the selected documents' pooled K/V plus the query's local K/V (msa_sparse_attn).
The timed steps run one query at a time.  A second run, reported apart as serving
throughput, keeps --inflight queries in flight on separate streams (default 3), so one
query's top-k and host-link-bound attention overlap other queries' HBM-bound scans, as
concurrent requests do on a serving GPU.
On the 100M-token bank the routing keys (3.25 GB) are in HBM and the content K/V are in
pinned host memory, read over the host link when selected.  Inputs are resident before
the timed region starts.  The pooling step (offline memory encoding) cannot run on the
100M-token bank itself (its token states would take 614 GB), so it is measured on the
10M-token encode workload and reported next to the step figures.

Prints one JSON line.  The CPU baseline runs the NumPy oracle on a bounded sample of the
same bank on the host's cores (up to 16 threads) and scales it to the same unit.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from dataclasses import replace

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import latent_memory_long_amd as M  # noqa: E402
from synth import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_BF16_TFLOPS = 2500.0   # dense bf16 matrix-core peak
METRIC = "routed bank tokens/s & % HBM peak; p50 route+attend latency, 100M-token bank"
SCAN_KERNEL = "route_scan_mfma"

# HBM traffic of the scan kernel per launch, from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# on this workload (scaled by the counters' reading of a copy kernel of known size).  It is
# reported only while the kernel source still has the digest it was measured with.
TRAFFIC = {"route_sha": "8980c242f2a1ffd2",
           # FETCH_SIZE 1,594,751 KiB per launch x 1.99993 (a 1 GiB copy reads 524,306 KiB)
           "fetch_bytes": 3265940121,
           # WRITE_SIZE 214.8 KiB per launch x 1.0 (a 1 GiB copy writes 1,048,576 KiB)
           "write_bytes": 219968}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def pct(a, q):
    return float(np.percentile(np.asarray(a), q))


def source_sha(name):
    with open(os.path.join(ROOT, "latent_memory_long_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def make_bank(wl, dev):
    lens = W.doc_lengths(wl)
    off = W.token_offsets(lens)
    coff = M.msa_chunk_offsets(off, wl.shape.chunk)
    kv_dev = "cpu-pinned" if wl.kv_source == "host" else dev
    log(f"bank: {len(lens)} documents, {int(coff[-1])} rows, content K/V on {kv_dev}")
    Krb_rows, Kb, Vb = W.gen_pooled_bank(wl, coff, dev, kv_device=kv_dev)
    Krb = M.RouteKeys.from_rows(Krb_rows)   # the routing keys in the library's bank layout
    return lens, off, coff, Krb, Krb_rows, Kb, Vb


def make_queries(wl, dev, n):
    qs = []
    for i in range(n):
        q = W.gen_queries(replace(wl, seed=wl.seed + 1 + i), dev)
        qs.append(q)
    return qs


def time_pool(dev, reps=3):
    """Pool a 10M-token bank (the batched encode workload) and time msa_pool.  Returns the
    figures and the pooled bank, which the batched route + attend stage then queries."""
    wl = W.workload("batch32_bank10m")
    sh = wl.shape
    lens = W.doc_lengths(wl)
    off = W.token_offsets(lens)
    coff = M.msa_chunk_offsets(off, sh.chunk)
    C = int(coff[-1])
    K, V, Kr = W.gen_token_states(wl, lens, dev)
    off_d = torch.tensor(off, device=dev)
    coff_d = torch.tensor(coff, device=dev)
    outs = (torch.empty((C, sh.h_kv, sh.d), dtype=torch.bfloat16, device=dev),
            torch.empty((C, sh.h_kv, sh.d), dtype=torch.bfloat16, device=dev),
            M.RouteKeys.empty(C, sh.h_r, sh.d, torch.bfloat16, dev))
    M.msa_pool(K, V, Kr, off_d, coff_d, C, sh.chunk, sh.rope_base, out=outs)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        M.msa_pool(K, V, Kr, off_d, coff_d, C, sh.chunk, sh.rope_base, out=outs)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    T = int(off[-1])
    row = (2 * sh.h_kv + sh.h_r) * sh.d * 2
    nbytes = T * row + C * row
    t = float(np.median(ms)) / 1e3
    del K, V, Kr
    torch.cuda.empty_cache()
    fig = {"workload": "batch32_bank10m (encode stage)", "tokens": T, "bank_rows": C,
           "ms": round(t * 1e3, 3), "tokens_per_s": T / t, "algorithmic_bytes": nbytes,
           "gbps": nbytes / t / 1e9, "frac_hbm_peak": nbytes / t / 1e9 / HBM_PEAK_GBPS}
    return fig, (wl, lens, coff, coff_d) + outs


def time_batch(dev, bank, reps=20):
    """Route + attend a batch of 32 queries (16-256 tokens each) against the pooled 10M-token
    bank: one msa_route_scan over all queries, msa_topk, one msa_sparse_attn."""
    wl, lens, coff, coff_d, Kb, Vb, Krb = bank
    sh = wl.shape
    N, C = len(lens), int(coff[-1])
    q = W.gen_queries(wl, dev)
    q_len = q["q_len"]
    B = len(q_len)
    q_off = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32)
    q_off_d = torch.tensor(q_off, device=dev)
    Qr, Q, Kl, Vl = q["Qr"], q["Q"], q["Kloc"], q["Vloc"]      # no decode rows: prefill only
    Lmax = int(q_len.max())
    tq = int(q_off[-1])
    ds = torch.empty((B, N), dtype=torch.float32, device=dev)
    ids = torch.empty((B, wl.k), dtype=torch.int32, device=dev)
    sc = torch.empty((B, wl.k), dtype=torch.float32, device=dev)
    out = torch.empty_like(Q)
    tws = torch.empty(max(M.msa_topk_workspace(B, N, wl.k), 256), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(M.msa_sparse_attn_workspace(M.MSA_BF16, B, tq, tq, Lmax, sh.hq, sh.h_kv, sh.d), 256),
                     dtype=torch.uint8, device=dev)
    lse = torch.empty((tq, sh.hq), dtype=torch.float32, device=dev)   # kept for the backward

    def run(ev):
        ev[0].record()
        M.msa_route_scan(Qr, q_off_d, Lmax, Krb, coff_d, out=ds)
        ev[1].record()
        M.msa_topk(ds, wl.k, out=(ids, sc), workspace=tws)
        ev[2].record()
        M.msa_sparse_attn(Q, Kl, Vl, q_off_d, q_off_d, Lmax, ids, coff_d, Kb, Vb, rope_base=sh.rope_base,
                          out=out, workspace=ws, lse=lse)
        ev[3].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps + 2)]
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    evs = evs[2:]
    scan = [e[0].elapsed_time(e[1]) for e in evs]
    topk = [e[1].elapsed_time(e[2]) for e in evs]
    attn = [e[2].elapsed_time(e[3]) for e in evs]
    tot = [e[0].elapsed_time(e[3]) for e in evs]
    # algorithmic scan flops: one dot product of D per (query token, bank row, routing head)
    flops = 2.0 * tq * C * sh.h_r * sh.d
    t_scan = float(np.mean(scan)) / 1e3
    fig = {"workload": "batch32_bank10m (route + attend)", "queries": B, "query_tokens": tq,
           "k": wl.k, "bank_rows": C, "route_attend_p50_ms": round(pct(tot, 50), 4),
           "scan_p50_ms": round(pct(scan, 50), 4), "topk_p50_ms": round(pct(topk, 50), 4),
           "attend_p50_ms": round(pct(attn, 50), 4), "scan_tflops": flops / t_scan / 1e12,
           "scan_mfma_util": flops / t_scan / 1e12 / MFMA_PEAK_BF16_TFLOPS,
           "routed_bank_tokens_per_s": B * int(np.sum(lens)) / (pct(tot, 50) / 1e3)}

    # ---- training step of the same batch: the attention's and the router's backward ----
    dO = torch.randn(Q.shape, generator=torch.Generator(device=dev).manual_seed(7), device=dev,
                     dtype=torch.float32).to(torch.bfloat16)
    dD = torch.randn((B, N), generator=torch.Generator(device=dev).manual_seed(8), device=dev)
    f32 = torch.float32
    gq = (torch.empty(Q.shape, dtype=f32, device=dev), torch.empty(Kl.shape, dtype=f32, device=dev),
          torch.empty(Vl.shape, dtype=f32, device=dev))
    gb = (torch.zeros((C, sh.h_kv, sh.d), dtype=f32, device=dev), torch.zeros((C, sh.h_kv, sh.d), dtype=f32, device=dev))
    bws = torch.empty(max(M.msa_sparse_attn_backward_workspace(tq, tq, sh.hq, sh.h_kv, sh.d), 256),
                      dtype=torch.uint8, device=dev)
    dQr = torch.empty(Qr.shape, dtype=f32, device=dev)
    dKr = torch.zeros(Krb.shape, dtype=f32, device=dev)
    rws = torch.empty(max(M.msa_route_backward_workspace(B, N, C, sh.h_r), 256), dtype=torch.uint8, device=dev)
    # a training step's forward scan keeps every bank row's best token for the backward
    rows = (torch.empty((B, C), dtype=torch.float32, device=dev), torch.empty((B, C), dtype=torch.int32, device=dev))
    ds_rows = torch.empty_like(ds)
    ev_rows = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps + 2)]
    for e in ev_rows:
        e[0].record()
        M.msa_route_scan(Qr, q_off_d, Lmax, Krb, coff_d, out=ds_rows, rows=rows)
        e[1].record()
    torch.cuda.synchronize()
    scan_rows = [e[0].elapsed_time(e[1]) for e in ev_rows[2:]]

    def run_bwd(ev):
        ev[0].record()
        M.msa_sparse_attn_backward(Q, Kl, Vl, q_off_d, q_off_d, Lmax, ids, coff_d, Kb, Vb, out, dO,
                                   rope_base=sh.rope_base, dbank=gb, out=gq, workspace=bws, lse=lse)
        ev[1].record()
        M.msa_route_backward(Qr, q_off_d, Lmax, Krb, coff_d, dD, dKrbar=dKr, out=dQr, workspace=rws, rows=rows)
        ev[2].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps + 2)]
    for e in evs:
        run_bwd(e)
    torch.cuda.synchronize()
    evs = evs[2:]
    abwd = [e[0].elapsed_time(e[1]) for e in evs]
    rbwd = [e[1].elapsed_time(e[2]) for e in evs]
    # algorithmic attention flops: (query, key) pairs x heads x d, 4 per pair forward and
    # 10 per pair backward (S recomputed, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q)
    sel = ids.cpu().numpy()
    pairs = 0
    for b in range(B):
        m = int(sum(coff[d + 1] - coff[d] for d in sel[b] if d >= 0))
        L = int(q_len[b])
        pairs += L * m + L * (L + 1) // 2
    bflops = 10.0 * pairs * sh.hq * sh.d
    t_abwd = pct(abwd, 50) / 1e3
    bwd = {"workload": "batch32_bank10m (training backward)", "attend_pairs": pairs,
           "attend_backward_p50_ms": round(pct(abwd, 50), 4), "attend_backward_lse": "from the forward",
           "attend_backward_tflops": bflops / t_abwd / 1e12,
           "attend_backward_mfma_util": bflops / t_abwd / 1e12 / MFMA_PEAK_BF16_TFLOPS,
           "attend_forward_tflops": 0.4 * bflops / (pct(attn, 50) / 1e3) / 1e12,
           "scan_with_rows_p50_ms": round(pct(scan_rows, 50), 4),
           "route_backward_p50_ms": round(pct(rbwd, 50), 4), "route_backward_rows": "from the forward scan",
           "route_backward_over_scan": pct(rbwd, 50) / pct(scan, 50)}
    return fig, bwd


def time_layers(dev, reps=20):
    """One 64-token query routed and attended in each of 18 upper layers, every layer with
    its own 10M-token bank (K-bar, V-bar, Kr-bar all in HBM: 17.5 GB).  The step runs the
    layers in order, eagerly and as one captured HIP graph."""
    wl = W.workload("layers18_bank10m")
    sh = wl.shape
    lens = W.doc_lengths(wl)
    coff = M.msa_chunk_offsets(W.token_offsets(lens), sh.chunk)
    N, C, L, k = len(lens), int(coff[-1]), wl.n_layers, wl.k
    lq = 64
    banks = []
    for l in range(L):
        Krb, Kb, Vb = W.gen_pooled_bank(W.layer(wl, l), coff, dev)
        banks.append((M.RouteKeys.from_rows(Krb), Kb, Vb))
        del Krb
    qs = [W.gen_queries(W.layer(wl, l), dev, lq_override=[lq]) for l in range(L)]
    q_off = torch.tensor([0, lq], dtype=torch.int32, device=dev)
    coff_d = torch.tensor(coff, device=dev)
    ds = torch.empty((L, 1, N), dtype=torch.float32, device=dev)
    ids = torch.empty((L, 1, k), dtype=torch.int32, device=dev)
    sc = torch.empty((L, 1, k), dtype=torch.float32, device=dev)
    out = torch.empty((L, lq, sh.hq, sh.d), dtype=torch.bfloat16, device=dev)
    tws = torch.empty(max(M.msa_topk_workspace(1, N, k), 256), dtype=torch.uint8, device=dev)
    aws = torch.empty(max(M.msa_sparse_attn_workspace(M.MSA_BF16, 1, lq, lq, lq, sh.hq, sh.h_kv, sh.d), 256),
                      dtype=torch.uint8, device=dev)

    def step():
        for l in range(L):
            Krb, Kb, Vb = banks[l]
            q = qs[l]
            M.msa_route_scan(q["Qr"], q_off, lq, Krb, coff_d, out=ds[l])
            M.msa_topk(ds[l], k, out=(ids[l], sc[l]), workspace=tws)
            M.msa_sparse_attn(q["Q"], q["Kloc"], q["Vloc"], q_off, q_off, lq, ids[l], coff_d, Kb, Vb,
                              rope_base=sh.rope_base, out=out[l], workspace=aws)

    def timed(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in ev]

    eager = timed(step)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.synchronize()
    replay = timed(graph.replay)
    scan_bytes = L * C * sh.h_r * sh.d * 2
    t = pct(replay, 50) / 1e3
    del banks, qs, graph
    torch.cuda.empty_cache()
    return {"workload": "layers18_bank10m", "layers": L, "bank_tokens_per_layer": int(lens.sum()),
            "bank_rows": C, "documents": N, "query_tokens": lq, "k": k, "banks_gb_in_hbm": round(3 * scan_bytes / 1e9, 2),
            "eager_step_p50_ms": round(pct(eager, 50), 4), "graph_step_p50_ms": round(pct(replay, 50), 4),
            "graph_per_layer_ms": round(pct(replay, 50) / L, 4),
            "routed_bank_tokens_per_s": L * int(lens.sum()) / t,
            "krbar_gbps_over_step": scan_bytes / t / 1e9}


def time_banks(dev, reps=50):
    """Route + attend one 64-token query against the 1M- and 10M-token banks (drawn pooled,
    everything in HBM).  The 1M bank's routing keys (33 MB) stay in the last-level cache
    between steps; the 10M bank (325 MB) is timed warm (back to back) and cold (a 1 GiB
    buffer is rewritten between steps)."""
    out = {}
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    for name in ("bank1m", "bank10m_needles"):
        wl = W.workload(name)
        sh = wl.shape
        lens = W.doc_lengths(wl)
        off = W.token_offsets(lens)
        coff = M.msa_chunk_offsets(off, sh.chunk)
        N, C, T = len(lens), int(coff[-1]), int(off[-1])
        Krb, Kb, Vb = W.gen_pooled_bank(wl, coff, dev)
        Krb = M.RouteKeys.from_rows(Krb)
        coff_d = torch.tensor(coff, device=dev)
        q = W.gen_queries(wl, dev)
        Lq = int(q["q_len"][0])
        q_off = torch.tensor([0, Lq], dtype=torch.int32, device=dev)
        Qr, Q, Kl, Vl = (q[x][:Lq].contiguous() for x in ("Qr", "Q", "Kloc", "Vloc"))
        ds = torch.empty((1, N), dtype=torch.float32, device=dev)
        ids = torch.empty((1, wl.k), dtype=torch.int32, device=dev)
        sc = torch.empty((1, wl.k), dtype=torch.float32, device=dev)
        o = torch.empty_like(Q)
        tws = torch.empty(max(M.msa_topk_workspace(1, N, wl.k), 256), dtype=torch.uint8, device=dev)
        ws = torch.empty(max(M.msa_sparse_attn_workspace(M.MSA_BF16, 1, Lq, Lq, Lq, sh.hq, sh.h_kv, sh.d), 256),
                         dtype=torch.uint8, device=dev)

        def step():
            M.msa_route_scan(Qr, q_off, Lq, Krb, coff_d, out=ds)
            M.msa_topk(ds, wl.k, out=(ids, sc), workspace=tws)
            M.msa_sparse_attn(Q, Kl, Vl, q_off, q_off, Lq, ids, coff_d, Kb, Vb, rope_base=sh.rope_base,
                              out=o, workspace=ws)

        res = {"bank_tokens": T, "bank_rows": C, "documents": N, "krbar_mb": round(C * sh.h_r * sh.d * 2 / 1e6, 1)}
        for mode in ("warm", "cold") if name != "bank1m" else ("warm",):
            ms = []
            for i in range(reps + 3):
                if mode == "cold":
                    flush.fill_(i & 255)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                step()
                e1.record()
                torch.cuda.synchronize()
                if i >= 3:
                    ms.append(e0.elapsed_time(e1))
            p50 = pct(ms, 50)
            res[mode] = {"route_attend_p50_ms": round(p50, 4), "routed_bank_tokens_per_s": T / (p50 / 1e3)}
        out[name] = res
        del Krb, Kb, Vb
        torch.cuda.empty_cache()
    return out


def host_threads():
    """Host threads for the oracle: the cores this process may run on, at most 16 (a GPU's
    share of its host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def blas_backend():
    from threadpoolctl import threadpool_info
    libs = [f"{x.get('internal_api')} {x.get('version')}" for x in threadpool_info() if x.get("user_api") == "blas"]
    return ", ".join(libs) or "none found"


def cpu_baseline(wl, lens, off, coff, Krb, Kb, Vb, q, target_s, runs=3):
    """The oracle, as it stands, on a bounded sample (the first documents of the bank) for
    one query: every document scored (the oracle's per-document scoring, groups of whole
    documents spread over the host threads: NumPy leaves the interpreter lock inside its
    products), its top-k, then its attention over the selected documents.  The sample is
    sized so that one run takes about target_s / runs; the median of `runs` runs is kept."""
    import concurrent.futures
    from threadpoolctl import threadpool_limits
    from oracle import msa_oracle as O

    nthr = host_threads()
    Lq = int(q["q_len"][0])
    Lkv = int(q["kv_len"][0])
    Qr = q["Qr"][:Lq].float().cpu().double().numpy()
    Q = q["Q"][:Lq].float().cpu().double().numpy()
    Kl = q["Kloc"][:Lkv].float().cpu().double().numpy()
    Vl = q["Vloc"][:Lkv].float().cpu().double().numpy()
    Kr_host = Krb.cpu()      # the bank's routing keys, row-major, in host memory (bf16)

    def groups(n_docs, block=4096):
        out, d0 = [], 0
        while d0 < n_docs:
            d1 = int(np.searchsorted(coff, coff[d0] + block, side="right")) - 1
            d1 = min(max(d1, d0 + 1), n_docs)
            out.append((d0, d1))
            d0 = d1
        return out

    def run(n_docs):
        scores = np.empty(n_docs)

        def work(g):
            d0, d1 = g
            kb = Kr_host[int(coff[d0]):int(coff[d1])].float().double().numpy()
            scores[d0:d1] = O.doc_scores_one(Qr, kb, coff[d0:d1 + 1] - coff[d0])

        t0 = time.perf_counter()
        with threadpool_limits(limits=1), concurrent.futures.ThreadPoolExecutor(nthr) as ex:
            list(ex.map(work, groups(n_docs)))
        ids, _ = O.topk_docs(scores, wl.k)
        t1 = time.perf_counter()
        sel = [int(d) for d in ids if d >= 0]
        idx = np.concatenate([np.arange(coff[d], coff[d + 1]) for d in sel])
        Kb_s = Kb[torch.as_tensor(idx)].float().double().numpy()
        Vb_s = Vb[torch.as_tensor(idx)].float().double().numpy()
        # the selected documents' rows, gathered in rank order, form a compact bank
        coff_c = np.concatenate([[0], np.cumsum([int(coff[d + 1] - coff[d]) for d in sel])])
        t2 = time.perf_counter()
        with threadpool_limits(limits=nthr):
            O.sparse_attn(Q, Kl, Vl, [0, Lq], [0, Lkv], np.arange(len(sel), dtype=np.int32)[None], coff_c, Kb_s,
                          Vb_s, wl.shape.rope_base)
        t3 = time.perf_counter()
        return (t1 - t0) + (t3 - t2), t1 - t0, t3 - t2

    # size the sample from a short run: one run takes about target_s / runs
    n1 = min(max(int(np.searchsorted(coff, 65536)), 1), len(lens))
    t_small = run(n1)[0]
    per_row = t_small / max(int(coff[n1]), 1)
    rows_target = int((target_s / runs) / max(per_row, 1e-12))
    n_docs = int(min(len(lens), max(1, np.searchsorted(coff, rows_target))))
    res = [run(n_docs) for _ in range(runs)]
    t, t_route, t_attn = (float(np.median([r[i] for r in res])) for i in range(3))
    tokens = int(off[n_docs])
    rows = int(coff[n_docs])
    pool = cpu_pool_sample()
    return {"value": tokens / t, "unit": "tokens/s", "cores": nthr, "kind": "oracle",
            "sample": (f"first {n_docs} of {len(lens)} documents ({rows} bank rows, {tokens} tokens) "
                       f"of the 100M-token bank: oracle route (every document scored, top-k) and "
                       f"attention for one {Lq}-token query, float64 NumPy, document groups over "
                       f"{nthr} host threads; median of {runs} runs of {t:.1f} s"),
            "blas": blas_backend(), "runs": runs,
            "route_tokens_per_s": tokens / t_route, "route_s": round(t_route, 3),
            "attend_s": round(t_attn, 3), "pool": pool}


def cpu_pool_sample(n_docs=64):
    """The oracle's pooling on the first documents of the 10M-token encode workload (token
    states drawn on the host with the same recipe), in tokens/s."""
    from oracle import msa_oracle as O

    wl = W.workload("batch32_bank10m")
    lens = W.doc_lengths(wl)[:n_docs]
    off = W.token_offsets(lens)
    K, V, Kr = W.gen_token_states(wl, lens, "cpu")
    K64, V64, Kr64 = (x.float().double().numpy() for x in (K, V, Kr))
    t0 = time.perf_counter()
    O.pool(K64, V64, Kr64, off, wl.shape.chunk, wl.shape.rope_base, O.ROPE_K)
    t = time.perf_counter() - t0
    T = int(off[-1])
    return {"value": T / t, "unit": "tokens/s", "cores": 1,
            "sample": f"first {n_docs} documents ({T} tokens) of the 10M-token encode workload, one "
                      f"thread (the oracle's pooling loops over chunks in Python), {t:.1f} s"}


def batch_scan_only(dev, n):
    """The batched router scan of the 32-query batch, n launches over the 10M-token bank drawn
    already pooled: a short program for hardware counter runs of that one kernel."""
    wl = W.workload("batch32_bank10m")
    sh = wl.shape
    lens = W.doc_lengths(wl)
    coff = M.msa_chunk_offsets(W.token_offsets(lens), sh.chunk)
    Krb, Kb, Vb = W.gen_pooled_bank(wl, coff, dev, krbar_only=True)
    Krb = M.RouteKeys.from_rows(Krb)
    q = W.gen_queries(wl, dev)
    q_len = q["q_len"]
    q_off = torch.tensor(np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32), device=dev)
    ds = torch.empty((len(q_len), len(lens)), dtype=torch.float32, device=dev)
    coff_d = torch.tensor(coff, device=dev)
    for _ in range(n):
        M.msa_route_scan(q["Qr"], q_off, int(q_len.max()), Krb, coff_d, out=ds)
    torch.cuda.synchronize()
    log(f"batched scan: {n} launches")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bank100m_host")
    ap.add_argument("--queries", type=int, default=8, help="distinct queries cycled by the steps")
    ap.add_argument("--inflight", type=int, default=3,
                    help="queries in flight on separate streams for the extra serving-throughput run (1: none)")
    ap.add_argument("--decode-steps", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=24.0, help="oracle time for the CPU baseline's runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pool", action="store_true", help="skip the 10M-token encode and batch stages")
    ap.add_argument("--no-layers", action="store_true", help="skip the 18-layer stage")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device to device 3 times: a kernel of known traffic "
                         "against which hardware byte counters are scaled")
    ap.add_argument("--batch-scan-launches", type=int, default=0, metavar="N",
                    help="only launch the 32-query batched scan N times over the 10M-token bank drawn "
                         "pooled (for counter runs), then exit")
    args = ap.parse_args()
    if args.batch_scan_launches:
        batch_scan_only(torch.device("cuda:0"), args.batch_scan_launches)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "sharded multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = W.workload(args.workload)
    sh = wl.shape
    lens, off, coff, Krb, Krb_rows, Kb, Vb = make_bank(wl, dev)
    N, C = len(lens), int(coff[-1])
    T = int(off[-1])
    coff_d = torch.tensor(coff, device=dev)
    if args.copy_calibration:
        # kernels of known traffic for scaling hardware byte counters: a device-to-device
        # copy (the runtime's copy kernel) and an elementwise kernel (read n, write n bytes)
        n = args.copy_calibration << 20
        src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies and 3 elementwise negations of {n} bytes")
        del src, dst
    qs = make_queries(wl, dev, args.queries)
    Lq = int(qs[0]["q_len"][0])
    k = wl.k

    # buffers, allocated once per in-flight query slot
    q_off = torch.tensor([0, Lq], dtype=torch.int32, device=dev)
    kv_off = torch.tensor([0, Lq], dtype=torch.int32, device=dev)

    def slot_buffers():
        return {"ds": torch.empty((1, N), dtype=torch.float32, device=dev),
                "ids": torch.empty((1, k), dtype=torch.int32, device=dev),
                "sc": torch.empty((1, k), dtype=torch.float32, device=dev),
                "out": torch.empty((Lq, sh.hq, sh.d), dtype=torch.bfloat16, device=dev),
                "tws": torch.empty(max(M.msa_topk_workspace(1, N, k), 256), dtype=torch.uint8, device=dev),
                "ws": torch.empty(max(M.msa_sparse_attn_workspace(M.MSA_BF16, 1, 200, 200, 200, sh.hq, sh.h_kv,
                                                                  sh.d), 256), dtype=torch.uint8, device=dev)}

    pre = [(q["Qr"][:Lq].contiguous(), q["Q"][:Lq].contiguous(), q["Kloc"][:Lq].contiguous(),
            q["Vloc"][:Lq].contiguous()) for q in qs]

    def run(n_slots, steps, sync_each=False, instrument=True):
        """`steps` timed steps, query i on stream i mod n_slots (default priority).  With one
        slot the queries run one at a time.  With several, queries are in flight together
        as concurrent requests are on a serving GPU: one query's top-k and host-link-bound
        attention overlap other queries' HBM-bound scans, and scans overlap one another.
        Per-step events are recorded on the step's own stream; without `instrument` a step
        records none (each event leaves the GPU idle for a few microseconds)."""
        streams = [torch.cuda.current_stream()] if n_slots == 1 else [torch.cuda.Stream() for _ in range(n_slots)]
        slots = [slot_buffers() for _ in range(n_slots)]

        def step(i, ev):
            Qr, Q, Kl, Vl = pre[i % len(pre)]
            st, b = streams[i % n_slots], slots[i % n_slots]
            if ev is not None:
                ev[0].record(st)
            M.msa_route_scan(Qr, q_off, Lq, Krb, coff_d, out=b["ds"], stream=st)
            if ev is not None:
                ev[1].record(st)
            M.msa_topk(b["ds"], k, out=(b["ids"], b["sc"]), workspace=b["tws"], stream=st)
            if ev is not None:
                ev[2].record(st)
            M.msa_sparse_attn(Q, Kl, Vl, q_off, kv_off, Lq, b["ids"], coff_d, Kb, Vb, rope_base=sh.rope_base,
                              out=b["out"], workspace=b["ws"], stream=st)
            if ev is not None:
                ev[3].record(st)

        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        wev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for i in range(args.warmup):
            step(i, wev)
        torch.cuda.synchronize()
        if sync_each:  # host wall time of a step that waits for its own result
            host = []
            for i in range(steps):
                t0 = time.perf_counter()
                step(i, evs[i])
                torch.cuda.synchronize()
                host.append((time.perf_counter() - t0) * 1e3)
            return host
        t0 = time.perf_counter()
        for i in range(steps):
            step(i, evs[i] if instrument else None)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, evs, slots[(steps - 1) % n_slots]["ids"]

    log(f"timing {args.steps} steps, one query at a time")
    # per-step events: the latencies, the phase split and the scan's roofline
    wall_ev, evs, ids = run(1, args.steps)
    host_sync_ms = run(1, min(args.steps, 50), sync_each=True)
    # the same steps back to back without per-step events: the throughput (`value`)
    log(f"timing {args.steps} steps without per-step events")
    wall, _, _ = run(1, args.steps, instrument=False)
    serving = None
    if args.inflight > 1:
        log(f"serving throughput: {args.steps} steps with {args.inflight} queries in flight")
        wall_n, _, _ = run(args.inflight, args.steps)
        t_n = wall_n / args.steps
        serving = {"queries_in_flight": args.inflight, "ms_per_step": t_n * 1e3, "tokens_per_s": T / t_n,
                   "krbar_tb_per_s": C * sh.h_r * sh.d * 2 / t_n / 1e12}
    # bytes the attention reads over the host link: K-bar and V-bar rows of the selected
    # documents (the last step's selection; the cycled queries select alike)
    sel = [int(d) for d in ids[0].cpu().numpy() if d >= 0]
    mem_rows = int(sum(coff[d + 1] - coff[d] for d in sel))
    host_bytes = mem_rows * sh.h_kv * sh.d * 2 * 2
    scan_ms = [e[0].elapsed_time(e[1]) for e in evs]
    topk_ms = [e[1].elapsed_time(e[2]) for e in evs]
    attn_ms = [e[2].elapsed_time(e[3]) for e in evs]
    step_ms = [e[0].elapsed_time(e[3]) for e in evs]
    ms_per_step = wall / args.steps * 1e3
    ms_per_step_events = wall_ev / args.steps * 1e3

    # roofline of the scan kernel: algorithmic bytes per launch / its average duration
    scan_bytes = C * sh.h_r * sh.d * 2 + Lq * sh.h_r * sh.d * 2 + (N + 1) * 8 + N * 4
    scan_s = float(np.mean(scan_ms)) / 1e3
    achieved = scan_bytes / scan_s / 1e9
    traffic = None
    if TRAFFIC and TRAFFIC.get("route_sha") == source_sha("route.hip"):
        traffic = TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]
    out = torch.empty((Lq, sh.hq, sh.d), dtype=torch.bfloat16, device=dev)
    ds = torch.empty((1, N), dtype=torch.float32, device=dev)
    sc = torch.empty((1, k), dtype=torch.float32, device=dev)
    ids = torch.empty((1, k), dtype=torch.int32, device=dev)
    tws = torch.empty(max(M.msa_topk_workspace(1, N, k), 256), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(M.msa_sparse_attn_workspace(M.MSA_BF16, 1, 200, 200, 200, sh.hq, sh.h_kv, sh.d), 256),
                     dtype=torch.uint8, device=dev)

    # decode: single-token steps after the prefill, routed again each step or reusing ids
    dec = {}
    if wl.decode_steps and args.decode_steps:
        q = qs[0]
        steps = min(args.decode_steps, wl.decode_steps)
        M.msa_route_topk(pre[0][0], q_off, Lq, Krb, coff_d, k, out=(ids, sc, ds), workspace=tws)
        fixed_ids = ids.clone()
        one = torch.tensor([0, 1], dtype=torch.int32, device=dev)
        routed, fixed = [], []
        for s in range(steps):
            r = Lq + s
            kvo = torch.tensor([0, r + 1], dtype=torch.int32, device=dev)
            Qr1, Q1 = q["Qr"][r:r + 1], q["Q"][r:r + 1]
            Kl, Vl = q["Kloc"][:r + 1], q["Vloc"][:r + 1]
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            M.msa_route_scan(Qr1, one, 1, Krb, coff_d, out=ds)
            M.msa_topk(ds, k, out=(ids, sc), workspace=tws)
            M.msa_sparse_attn(Q1, Kl, Vl, one, kvo, 1, ids, coff_d, Kb, Vb, rope_base=sh.rope_base,
                              out=out[:1], workspace=ws)
            e[1].record()
            M.msa_sparse_attn(Q1, Kl, Vl, one, kvo, 1, fixed_ids, coff_d, Kb, Vb,
                              rope_base=sh.rope_base, out=out[:1], workspace=ws)
            e[2].record()
            torch.cuda.synchronize()
            if s >= 2:
                routed.append(e[0].elapsed_time(e[1]))
                fixed.append(e[1].elapsed_time(e[2]))
        dec = {"steps": steps, "routed_p50_ms": round(pct(routed, 50), 4),
               "routed_p90_ms": round(pct(routed, 90), 4), "fixed_ids_p50_ms": round(pct(fixed, 50), 4),
               "routed_bank_tokens_per_s": T / (pct(routed, 50) / 1e3)}

    banks = None
    if not args.no_pool:
        log("1M- and 10M-token banks")
        banks = time_banks(dev)
    pool = batch = backward = layers = None
    if not args.no_pool:
        del qs
        torch.cuda.empty_cache()
        log("pool on the 10M-token encode workload")
        pool, bank10m = time_pool(dev)
        log("batched route + attend and its backward: 32 queries against the pooled 10M-token bank")
        batch, backward = time_batch(dev, bank10m)
        del bank10m
        torch.cuda.empty_cache()
    if not args.no_layers:
        log("18 routed layers, a 10M-token bank each, eager and graph-captured")
        layers = time_layers(dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        q0 = W.gen_queries(replace(wl, seed=wl.seed + 1), dev)
        cpu = cpu_baseline(wl, lens, off, coff, Krb_rows, Kb, Vb, q0, args.cpu_seconds)

    value = T / (ms_per_step / 1e3)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "bank_tokens": T, "documents": N, "bank_rows": C,
                   "query_tokens": Lq, "k": k, "heads_q_kv_r": [sh.hq, sh.h_kv, sh.h_r],
                   "head_dim": sh.d, "content_kv": "pinned host" if wl.kv_source == "host" else "hbm",
                   "distinct_queries": len(pre)},
        "latency_ms": {"route_attend_p50": round(pct(step_ms, 50), 4),
                       "route_attend_p90": round(pct(step_ms, 90), 4),
                       "scan_p50": round(pct(scan_ms, 50), 4), "topk_p50": round(pct(topk_ms, 50), 4),
                       "attend_p50": round(pct(attn_ms, 50), 4),
                       "route_attend_host_sync_p50": round(pct(host_sync_ms, 50), 4),
                       "ms_per_step_with_step_events": round(ms_per_step_events, 4)},
        "serving": serving,
        "roofline": {"kernel": SCAN_KERNEL, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": scan_bytes,
                     "avg_launch_ms": scan_s * 1e3},
        "attend_memory": {"rows": mem_rows, "kv_bytes": host_bytes,
                          "source": "pinned host" if wl.kv_source == "host" else "hbm",
                          "gbps_at_p50": host_bytes / (pct(attn_ms, 50) / 1e3) / 1e9},
        "scan_routed_bank_tokens_per_s": T / scan_s,
        "scan_mfma_util": 2.0 * Lq * C * sh.h_r * sh.d / scan_s / 1e12 / MFMA_PEAK_BF16_TFLOPS,
        "decode": dec or None,
        "banks": banks,
        "pool": pool,
        "batch": batch,
        "backward": backward,
        "layers": layers,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
