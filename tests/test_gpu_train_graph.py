"""A whole training step of the routed layer captured in a HIP graph.

Forward (scan with row outputs, top-k, attention with log-sum-exp), the routing loss and
both backward passes, all into preallocated outputs and workspaces, run eagerly and then
replayed from a graph several times with new inputs written in place between replays.
Every replay must reproduce the eager step bit for bit, except the bank-row gradients,
whose atomic additions may round differently from run to run (checked to a float32
tolerance instead)."""
import numpy as np
import pytest
import torch

import latent_memory_long_amd as M
from synth import workloads as W
from tests.helpers import as_keys, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


class TrainStep:
    def __init__(self, wl):
        sh = wl.shape
        self.sh, self.k = sh, wl.k
        lens = W.doc_lengths(wl)
        coff = M.msa_chunk_offsets(W.token_offsets(lens), sh.chunk)
        self.N, self.C = len(lens), int(coff[-1])
        self.coff = torch.tensor(coff, device=DEV)
        Krb, self.Kb, self.Vb = W.gen_pooled_bank(wl, coff, DEV)
        self.Krb = as_keys(Krb)
        q = W.gen_queries(wl, DEV)
        self.q = q
        q_len = q["q_len"]
        self.B = B = len(q_len)
        self.q_off = torch.tensor(np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32), device=DEV)
        self.Lmax = int(q_len.max())
        tq = int(self.q_off[-1])
        N, C, f32 = self.N, self.C, torch.float32
        self.labels = (torch.rand((B, N), generator=torch.Generator().manual_seed(3)) < 0.05).float().to(DEV)
        self.dO = torch.zeros_like(q["Q"])
        # outputs and workspaces
        self.ds = torch.empty((B, N), dtype=f32, device=DEV)
        self.rows = (torch.empty((B, C), dtype=f32, device=DEV), torch.empty((B, C), dtype=torch.int32, device=DEV))
        self.ids = torch.empty((B, wl.k), dtype=torch.int32, device=DEV)
        self.sc = torch.empty((B, wl.k), dtype=f32, device=DEV)
        self.out = torch.empty_like(q["Q"])
        self.lse = torch.empty((tq, sh.hq), dtype=f32, device=DEV)
        self.loss = torch.empty(B, dtype=f32, device=DEV)
        self.dD = torch.empty((B, N), dtype=f32, device=DEV)
        self.gq = (torch.empty(q["Q"].shape, dtype=f32, device=DEV), torch.empty(q["Kloc"].shape, dtype=f32, device=DEV),
                   torch.empty(q["Vloc"].shape, dtype=f32, device=DEV))
        self.gb = (torch.empty(self.Kb.shape, dtype=f32, device=DEV), torch.empty(self.Vb.shape, dtype=f32, device=DEV))
        self.dQr = torch.empty(q["Qr"].shape, dtype=f32, device=DEV)
        self.dKr = torch.empty(self.Krb.shape, dtype=f32, device=DEV)
        u8 = torch.uint8
        self.tws = torch.empty(max(M.msa_topk_workspace(B, N, wl.k), 256), dtype=u8, device=DEV)
        self.aws = torch.empty(max(M.msa_sparse_attn_workspace(M.MSA_BF16, B, tq, tq, self.Lmax, sh.hq, sh.h_kv, sh.d),
                                   256), dtype=u8, device=DEV)
        self.bws = torch.empty(max(M.msa_sparse_attn_backward_workspace(tq, tq, sh.hq, sh.h_kv, sh.d), 256), dtype=u8,
                               device=DEV)
        self.rws = torch.empty(max(M.msa_route_backward_workspace(B, N, C, sh.h_r), 256), dtype=u8, device=DEV)

    def __call__(self):
        q, sh = self.q, self.sh
        M.msa_route_scan(q["Qr"], self.q_off, self.Lmax, self.Krb, self.coff, out=self.ds, rows=self.rows)
        M.msa_topk(self.ds, self.k, out=(self.ids, self.sc), workspace=self.tws)
        M.msa_sparse_attn(q["Q"], q["Kloc"], q["Vloc"], self.q_off, self.q_off, self.Lmax, self.ids, self.coff,
                          self.Kb, self.Vb, rope_base=sh.rope_base, out=self.out, workspace=self.aws, lse=self.lse)
        M.msa_route_aux_loss(self.ds, self.labels, M.MSA_AUX_BCE, 0.5, out=(self.loss, self.dD))
        # the gradient arrays that are added to start from zero (a fill kernel, capturable)
        for t in self.gb + (self.dKr,):
            t.zero_()
        self.dO.copy_(self.out)   # dL/dO for L = sum(O^2) / 2
        M.msa_sparse_attn_backward(q["Q"], q["Kloc"], q["Vloc"], self.q_off, self.q_off, self.Lmax, self.ids,
                                   self.coff, self.Kb, self.Vb, self.out, self.dO, rope_base=sh.rope_base,
                                   dbank=self.gb, out=self.gq, workspace=self.bws, lse=self.lse)
        M.msa_route_backward(q["Qr"], self.q_off, self.Lmax, self.Krb, self.coff, self.dD, dKrbar=self.dKr,
                             out=self.dQr, workspace=self.rws, rows=self.rows)

    def exact(self):
        return (self.ds, self.ids, self.out, self.lse, self.loss, self.dD) + self.gq + (self.dQr,)

    def atomic(self):
        return self.gb + (self.dKr,)


def test_training_step_graph_replays_match_eager():
    say("case training step (forward, routing loss, both backward passes) captured in a graph")
    wl = W.workload("batch32_bank10m", bank_tokens=None, n_docs=300, n_queries=6, lq=(5, 70), k=8,
                    len_dist=("loguniform", 64, 2000), seed=4)
    step = TrainStep(wl)
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV)
    for rep in range(3):
        gen.manual_seed(200 + rep)
        for name in ("Qr", "Q", "Kloc", "Vloc"):
            t = step.q[name]
            t.copy_(torch.randn(t.shape, generator=gen, device=DEV).to(t.dtype))
        step()                               # eager reference on the new inputs
        torch.cuda.synchronize()
        ref_x = [t.clone() for t in step.exact()]
        ref_a = [t.clone() for t in step.atomic()]
        for t in step.exact() + step.atomic():
            t.fill_(0) if t.dtype != torch.int32 else t.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(step.exact(), ref_x)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager step"
        for i, (a, b) in enumerate(zip(step.atomic(), ref_a)):
            err = float((a - b).abs().max())
            top = float(b.abs().max())
            assert err <= 1e-5 * top + 1e-9, f"replay {rep}: bank gradient {i} differs by {err:.3g} (max {top:.3g})"
        say(f"  replay {rep}: exact outputs equal, bank gradients within {1e-5:.0e} of the eager step")
