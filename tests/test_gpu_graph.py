"""The calls capture into a HIP graph (torch.cuda.graph over the library's stream
argument) and the replays compute what eager calls compute.

A full W-worker step (W = 3 compress-only workers with fp16 gradients, the server
stage, the masked finish) over a plan with a two-pass chunk is captured once on one
set of buffers; the same step runs eagerly on a copy.  Four rounds: new gradients
are copied into both sets (eager work between replays), the graph is replayed, the
eager step is run, and every buffer is compared bit for bit.  The quantizers (QSDP
quantize and dequantize, three workers' QSGD streams and their decode-and-average, a
LoCo step whose error average carries over) are checked the same way.
"""
import numpy as np
import pytest
import torch

from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import workloads as W
from gpu_helpers import DEV
from parity import say

pytestmark = pytest.mark.gpu


class StepState:
    def __init__(self, plan, n, words, nch, workers, seed):
        rng = np.random.default_rng(seed)
        npad = (n + 7) // 8 * 8            # fp16 and fp32 worker rows start 16-byte aligned
        self.g = torch.zeros((workers, npad), dtype=torch.float16, device=DEV)
        self.m = torch.zeros(n, device=DEV)
        self.e = torch.zeros((workers, npad), device=DEV)
        self.es = torch.zeros(n, device=DEV)
        self.v = torch.from_numpy((rng.uniform(0.5, 2, n) * 1e-6).astype(np.float32)).to(DEV)
        self.x = torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)).to(DEV)
        self.mask = torch.from_numpy((rng.random(n) < 0.9).astype(np.uint8)).to(DEV)
        self.wb = torch.zeros((workers, words), dtype=torch.int32, device=DEV)
        self.wsc = torch.zeros((workers, nch), device=DEV)
        self.sb = torch.zeros(words, dtype=torch.int32, device=DEV)
        self.ss = torch.zeros(nch, device=DEV)
        self.ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
        self.n, self.workers = n, workers

    def step(self, plan, stream=None):
        n = self.n
        for w in range(self.workers):
            ob.onebit_compress_update(plan, self.g[w, :n], self.m, self.e[w, :n], None, None, None, self.wb[w],
                                      self.wsc[w], lr=0.0, beta1=0.9, eps=1e-8, weight_decay=0.0,
                                      workspace=self.ws, stream=stream)
        ob.onebit_server_reduce(plan, self.wb, self.wsc, self.es, self.sb, self.ss, self.m, self.ws, stream=stream)
        ob.onebit_momentum_update(self.m, self.mask, self.v, self.x, None, lr=1e-3, eps=1e-8, weight_decay=0.01,
                                  stream=stream)

    def buffers(self):
        return [self.m, self.e, self.es, self.x, self.wb, self.wsc, self.sb, self.ss]


def test_graph_replays_match_eager_steps():
    big = max(ob.onebit_onepass_max_elements(), 1) + 4097
    off = W.offsets_from_sizes([5000, big, 33, 70001])
    n = int(off[-1])
    plan = ob.onebit_plan_create(off)
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    A = StepState(plan, n, words, nch, 3, seed=5)     # replayed
    B = StepState(plan, n, words, nch, 3, seed=5)     # eager
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        A.step(plan, stream=s)
    torch.cuda.synchronize()
    for t in range(4):
        g = torch.from_numpy((np.random.default_rng(70 + t).standard_normal((3, n)) * 1e-3).astype(np.float16)).to(DEV)
        A.g[:, :n].copy_(g)
        B.g[:, :n].copy_(g)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        B.step(plan)
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(A.buffers(), B.buffers())):
            assert torch.equal(a, b), f"round {t}: buffer {k} differs between the replay and the eager step"
        say(f"  graph replay {t}: all buffers identical to the eager step")
    assert ob.onebit_workspace_status(A.ws) == 0 and ob.onebit_workspace_status(B.ws) == 0


class QuantState:
    """Inputs and outputs of one round of the quantizers: QSDP quantize + dequantize
    of bf16 weights (4- and 8-bit), QSGD quantize of three workers' bf16 gradients and
    the decode-and-average of their streams, and a LoCo step whose error average
    carries over from round to round."""

    def __init__(self, n, workers):
        self.n, self.workers = n, workers
        nb = (n + 1023) // 1024
        self.x = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
        self.g = torch.zeros((workers, (n + 15) // 16 * 16), dtype=torch.bfloat16, device=DEV)   # rows 32-byte aligned
        self.codes = {b: torch.zeros(n if b == 8 else (n + 1) // 2, dtype=torch.uint8, device=DEV) for b in (4, 8)}
        self.bmin = {b: torch.zeros(nb, device=DEV) for b in (4, 8)}
        self.bmax = {b: torch.zeros(nb, device=DEV) for b in (4, 8)}
        self.y = {b: torch.zeros(n, dtype=torch.bfloat16, device=DEV) for b in (4, 8)}
        stride = ((n + 1) // 2 + 15) // 16 * 16
        self.qc = torch.zeros((workers, stride), dtype=torch.uint8, device=DEV)
        self.qn = torch.zeros((workers, nb), device=DEV)
        self.avg = torch.zeros(n, device=DEV)
        self.err = torch.zeros(n, device=DEV)
        self.lc = torch.zeros((n + 1) // 2, dtype=torch.uint8, device=DEV)
        self.ln = torch.zeros(nb, device=DEV)

    def run(self, stream=None):
        n = self.n
        for b in (4, 8):
            ob.qsdp_quantize(self.x, 1024, b, 17 + b, self.codes[b], self.bmin[b], self.bmax[b], stream=stream)
            ob.qsdp_dequantize(self.codes[b], self.bmin[b], self.bmax[b], n, 1024, b, self.y[b], stream=stream)
        for w in range(self.workers):
            ob.qsgd_quantize(self.g[w, :n], 1024, 4, 300 + w, self.qc[w], self.qn[w], stream=stream)
        ob.qsgd_reduce(self.qc, self.qn, n, 1024, 4, out_f32=self.avg, stream=stream)
        ob.loco_quantize(self.g[0, :n], self.err, 1024, 4, 0.9, 5, self.lc, self.ln, stream=stream)

    def buffers(self):
        return ([self.codes[b] for b in (4, 8)] + [self.bmin[b] for b in (4, 8)] + [self.bmax[b] for b in (4, 8)] +
                [self.y[b] for b in (4, 8)] + [self.qc, self.qn, self.avg, self.err, self.lc, self.ln])


def test_quantizer_graph_replays_match_eager_calls():
    n, workers = 3 * 1024 * 7 + 333, 3
    A, B = QuantState(n, workers), QuantState(n, workers)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        A.run(stream=s)
    torch.cuda.synchronize()
    for t in range(4):
        rng = np.random.default_rng(500 + t)
        x = torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)).to(DEV).to(torch.bfloat16)
        g = torch.from_numpy((rng.standard_normal((workers, n)) * 1e-3).astype(np.float32)).to(DEV).to(torch.bfloat16)
        for S in (A, B):
            S.x.copy_(x)
            S.g[:, :n].copy_(g)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        B.run()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(A.buffers(), B.buffers())):
            assert torch.equal(a, b), f"round {t}: quantizer buffer {k} differs between the replay and the eager calls"
        say(f"  quantizer graph replay {t}: all buffers identical to the eager calls")
