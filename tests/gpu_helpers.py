"""Device-side drivers shared by the GPU parity tests: one compressed step, one
server step, their oracle counterparts on host copies of the same inputs."""
import numpy as np
import torch

import oracle
from error_compensated_bit_amd import onebit as ob

DEV = "cuda:0"
H = dict(lr=1e-3, beta1=0.9, eps=1e-8, weight_decay=0.0)


class CompressBuffers:
    """Device state and outputs for one plan."""

    def __init__(self, chunk_off, tensor_off=None, tensor_keep=None, x_bf16=False, workspace=None):
        self.chunk_off = np.asarray(chunk_off, np.int64)
        self.tensor_off = tensor_off
        self.tensor_keep = tensor_keep
        self.plan = ob.onebit_plan_create(self.chunk_off, tensor_off, tensor_keep)
        self.n = ob.onebit_plan_elements(self.plan)
        self.words = ob.onebit_plan_words(self.plan)
        self.n_chunks = ob.onebit_plan_chunks(self.plan)
        self.bits = torch.zeros(max(self.words, 1), dtype=torch.int32, device=DEV)
        self.scales = torch.zeros(max(self.n_chunks, 1), dtype=torch.float32, device=DEV)
        self.xb = torch.zeros(max(self.n, 1), dtype=torch.bfloat16, device=DEV) if x_bf16 else None
        wsb = ob.onebit_plan_workspace_bytes(self.plan)
        if workspace is None:
            self.ws = torch.zeros(wsb // 8, dtype=torch.int64, device=DEV)
        else:
            assert workspace.numel() * 8 >= wsb
            self.ws = workspace

    def step(self, g, m, e, v=None, x=None, **h):
        hh = dict(H)
        hh.update(h)
        ob.onebit_compress_update(self.plan, g, m, e, v, x, self.xb, self.bits, self.scales, workspace=self.ws, **hh)

    def out_bits(self):
        return self.bits.cpu().numpy().view(np.uint32)[:self.words]

    def out_scales(self):
        return self.scales.cpu().numpy()[:self.n_chunks]

    def ws_status(self):
        return ob.onebit_workspace_status(self.ws)


def host(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).copy()
    return t.detach().cpu().numpy().copy()


def oracle_compress(chunk_off, g, m, e, v=None, x=None, tensor_off=None, tensor_keep=None, want_bf16=False, **h):
    hh = dict(H)
    hh.update(h)
    return oracle.compress_update(chunk_off, g, m, e, v, x, tensor_off=tensor_off, tensor_keep=tensor_keep,
                                  want_bf16=want_bf16, **hh)
