"""The attention backward's side stream in a fresh process whose first backward call is made
under graph capture.

With the forward's log-sum-exp the backward forks its key-side gradients onto a stream the
library creates on the first such call outside capture.  A first call inside a capture must
not create it (it runs its kernels in order on the captured stream); the eager call after
it creates the stream and forks.  The graph's replay (in order) and the eager step (forked)
must give the same gradients: bit for bit except the bank rows' atomic additions."""
import os
import subprocess
import sys

import pytest

from tests.helpers import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys, torch
sys.path.insert(0, sys.argv[1])
from synth import workloads as W
from tests.test_gpu_train_graph import TrainStep
wl = W.workload("batch32_bank10m", bank_tokens=None, n_docs=200, n_queries=4, lq=(5, 60), k=8,
                len_dist=("loguniform", 64, 1500), seed=9)
step = TrainStep(wl)
torch.cuda.synchronize()
graph = torch.cuda.CUDAGraph()
s = torch.cuda.Stream()
s.wait_stream(torch.cuda.current_stream())
with torch.cuda.stream(s):
    with torch.cuda.graph(graph, stream=s):
        step()                      # the process's first backward call: under capture
torch.cuda.synchronize()
graph.replay()
torch.cuda.synchronize()
rx = [t.clone() for t in step.exact()]
ra = [t.clone() for t in step.atomic()]
step()                              # eager: creates the side stream and forks
torch.cuda.synchronize()
for i, (a, b) in enumerate(zip(step.exact(), rx)):
    assert torch.equal(a, b), f"output {i}: replay (in order) and eager (forked) differ"
for i, (a, b) in enumerate(zip(step.atomic(), ra)):
    err = float((a - b).abs().max()); top = float(b.abs().max())
    assert err <= 1e-5 * top + 1e-9, f"bank gradient {i} differs by {err:.3g} (max {top:.3g})"
print("capture-first ok", flush=True)
'''


def test_first_backward_call_under_capture():
    say("case fresh process: first attention backward captured in a graph, then eager with the side stream")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "capture-first ok" in r.stdout, (r.stdout + r.stderr)[-3000:]
