"""Routing in several upper layers: one bank per layer over the same documents, one query
routed and attended in every layer, and the whole multi-layer step captured in a HIP graph.

Each layer is checked against the oracle applied to that layer's tensors; graph replays are
checked bit for bit against eager runs of the same step, several times, with eager work and
new inputs between the replays."""
import numpy as np
import pytest
import torch

import latent_memory_long_amd as M
from oracle import msa_oracle as O
from synth import workloads as W
from tests.helpers import (as_keys, assert_attn_close, assert_scores_close, assert_topk_consistent,
                           assert_topk_valid, f64, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layers(n_layers, n_docs, lq, seed=5):
    wl = W.workload("layers18_bank10m", bank_tokens=None, n_docs=n_docs, n_layers=n_layers,
                    len_dist=("loguniform", 64, 900), seed=seed, k=4)
    lens = W.doc_lengths(wl)
    coff = M.msa_chunk_offsets(W.token_offsets(lens), wl.shape.chunk)
    banks, queries = [], []
    for l in range(n_layers):
        wl_l = W.layer(wl, l)
        Krb, Kb, Vb = W.gen_pooled_bank(wl_l, coff, DEV)
        banks.append((as_keys(Krb), Kb, Vb))
        queries.append(W.gen_queries(wl_l, DEV, lq_override=[lq]))
    return wl, coff, banks, queries


class Step:
    """One routed step through every layer with preallocated outputs and workspaces, so it
    can run eagerly or be captured."""

    def __init__(self, wl, coff, banks, queries):
        sh = wl.shape
        self.wl, self.banks, self.q = wl, banks, queries
        lq = int(queries[0]["q_len"][0])
        N, k = len(coff) - 1, wl.k
        self.lq = lq
        self.q_off = torch.tensor([0, lq], dtype=torch.int32, device=DEV)
        self.coff = torch.tensor(coff, device=DEV)
        L = len(banks)
        self.ds = torch.empty((L, 1, N), dtype=torch.float32, device=DEV)
        self.ids = torch.empty((L, 1, k), dtype=torch.int32, device=DEV)
        self.sc = torch.empty((L, 1, k), dtype=torch.float32, device=DEV)
        self.out = torch.empty((L, lq, sh.hq, sh.d), dtype=torch.bfloat16, device=DEV)
        self.tws = torch.empty(max(M.msa_topk_workspace(1, N, k), 256), dtype=torch.uint8, device=DEV)
        self.aws = torch.empty(max(M.msa_sparse_attn_workspace(M.MSA_BF16, 1, lq, lq, lq, sh.hq, sh.h_kv, sh.d),
                                   256), dtype=torch.uint8, device=DEV)

    def __call__(self):
        for l, ((Krb, Kb, Vb), q) in enumerate(zip(self.banks, self.q)):
            M.msa_route_scan(q["Qr"], self.q_off, self.lq, Krb, self.coff, out=self.ds[l])
            M.msa_topk(self.ds[l], self.wl.k, out=(self.ids[l], self.sc[l]), workspace=self.tws)
            M.msa_sparse_attn(q["Q"], q["Kloc"], q["Vloc"], self.q_off, self.q_off, self.lq, self.ids[l], self.coff,
                              Kb, Vb, rope_base=self.wl.shape.rope_base, out=self.out[l], workspace=self.aws)

    def snapshot(self):
        return self.ds.clone(), self.ids.clone(), self.out.clone()


def test_every_layer_matches_the_oracle():
    say("case three routed layers, one bank each, against the oracle")
    wl, coff, banks, queries = _layers(3, 40, 20)
    step = Step(wl, coff, banks, queries)
    step()
    torch.cuda.synchronize()
    q_off = np.array([0, step.lq])
    for l, ((Krb, Kb, Vb), q) in enumerate(zip(banks, queries)):
        o = O.route_doc_scores(f64(q["Qr"]), q_off, f64(Krb), coff)[0]
        ds, ids, sc = (x[l, 0].cpu().numpy() for x in (step.ds, step.ids, step.sc))
        assert_scores_close(ds, o, "bf16", f"layer {l} scores")
        assert_topk_consistent(ids, sc, ds, wl.k, f"layer {l}")
        assert_topk_valid(ids, o, wl.k, f"layer {l}")
        ref = O.sparse_attn(f64(q["Q"]), f64(q["Kloc"]), f64(q["Vloc"]), q_off, q_off, ids[None], coff,
                            f64(Kb), f64(Vb), wl.shape.rope_base)
        assert_attn_close(step.out[l], ref, "bf16", f"layer {l} attention")
    # the layers route differently: their banks and queries are independent draws
    assert not torch.equal(step.ids[0], step.ids[1]) or not torch.equal(step.ids[1], step.ids[2])


def test_graph_replays_match_eager():
    say("case multi-layer step captured in a graph, replayed against eager runs")
    wl, coff, banks, queries = _layers(4, 60, 48)
    step = Step(wl, coff, banks, queries)
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                    # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV)
    for rep in range(3):
        # new query inputs, written in place into the captured tensors
        gen.manual_seed(100 + rep)
        for q in queries:
            for name in ("Qr", "Q", "Kloc", "Vloc"):
                q[name].copy_(torch.randn(q[name].shape, generator=gen, device=DEV).to(q[name].dtype))
        step()                                    # eager reference on the same inputs
        torch.cuda.synchronize()
        ref = step.snapshot()
        step.out.zero_()
        step.ds.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = step.snapshot()
        for a, b, name in zip(got, ref, ("scores", "ids", "output")):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager run"
