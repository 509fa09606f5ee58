"""Phase control of 1-bit Adam over one flat fp32 parameter vector.

What it follows (DeepSpeed 1-bit Adam configuration guide, yfxerp.com):
  sec. 3.4  the optimizer's parameters: lr, betas, eps, weight_decay,
            bias_correction, freeze_step;
  sec. 4    steps 1..freeze_step are full-precision Adam (m and v both updated);
            every later step keeps v fixed and runs the error-compensated 1-bit
            compressed momentum step, whose decompressed result becomes m;
  sec. 3.5  tensors whose gradient is always zero carry a mask that keeps their
            momentum (and compression error) at zero;
  sec. 7    a checkpoint keeps m and v; the compression error is discarded when one
            is loaded.
1-bit Adam review (nubint.ai), "proposed method": the variance stops changing after
the warmup and then serves as a fixed preconditioner.

Host logic only: each step is one call of the library (onebit_adam_warmup_step or
onebit_compress_update); m, v, the error, the packed words, the scales and the
workspace are device tensors this object allocates next to x.  Bias correction,
when enabled, applies to the warmup steps only (the compressed phase never
corrects), so it is off by default, as in every configuration the guide prints
(sec. 6.2): with it on, the step size changes by about (1 - b1^T) / sqrt(1 - b2^T)
at the switch to compression, T = freeze_step.

Failure detection: the compressed step's cross-workgroup waits are bounded; a wait
that gives up records an error in the workspace and the step's outputs are not
valid.  The error stays set until the workspace is re-initialized, and while it is
set every later wait gives up at once, so the driver reads it (a synchronizing
8-byte copy) after every `check_every`-th compressed step; when it is set the driver
re-initializes the workspace and raises WaitTimeout.
"""
from __future__ import annotations

import numpy as np
import torch

from . import onebit as ob


class WaitTimeout(RuntimeError):
    """A cross-workgroup wait of a compressed step gave up; that step's m, e and x
    are not valid (restore them, e.g. from a checkpoint, before continuing)."""


class OneBitAdam:
    """1-bit Adam on the flat fp32 vector `x` (updated in place).

    chunk_offsets   chunk table (one scale per chunk); default: the tensor table if
                    given, else the whole vector as one chunk;
    tensor_offsets, tensor_keep
                    tensor table and keep flags (0 = masked: m and the error pinned
                    at zero in the compressed phase);
    freeze_step     number of full-precision warmup steps;
    check_every     read the workspace's error word after every check_every-th
                    compressed step (0: never).
    """

    def __init__(self, x, *, chunk_offsets=None, tensor_offsets=None, tensor_keep=None, lr=1e-3,
                 betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, bias_correction=False, freeze_step=100000,
                 check_every=1):
        if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.dim() != 1:
            raise TypeError("x must be a one-dimensional float32 tensor")
        if freeze_step < 0:
            raise ValueError("freeze_step must be >= 0")
        n = x.numel()
        if chunk_offsets is None:
            chunk_offsets = tensor_offsets if tensor_offsets is not None else [0, n]
        co = np.asarray(chunk_offsets, dtype=np.int64)
        if co.ndim != 1 or co.size < 2 or co[0] != 0 or co[-1] != n:
            raise ValueError("chunk_offsets must start at 0 and end at x.numel()")
        if tensor_offsets is not None and int(np.asarray(tensor_offsets)[-1]) != n:
            raise ValueError("tensor_offsets must end at x.numel()")
        self.x = x
        self.lr, self.beta1, self.beta2 = float(lr), float(betas[0]), float(betas[1])
        self.eps, self.weight_decay = float(eps), float(weight_decay)
        self.bias_correction = bool(bias_correction)
        self.freeze_step = int(freeze_step)
        self.check_every = int(check_every)
        self.step_count = 0
        self.compressed_steps = 0
        self.m = torch.zeros_like(x)
        self.v = torch.zeros_like(x)
        self.e = torch.zeros_like(x)
        self.plan = ob.onebit_plan_create(co, tensor_offsets, tensor_keep)
        words, chunks = ob.onebit_plan_words(self.plan), ob.onebit_plan_chunks(self.plan)
        self.bits = torch.zeros(max(words, 1), dtype=torch.int32, device=x.device)
        self.scales = torch.zeros(max(chunks, 1), dtype=torch.float32, device=x.device)
        self.workspace = torch.zeros(max(ob.onebit_plan_workspace_bytes(self.plan) // 8, 1), dtype=torch.int64,
                                     device=x.device)

    @property
    def frozen(self) -> bool:
        """True once the next step is a compressed one (v no longer changes)."""
        return self.step_count >= self.freeze_step

    def step(self, g, stream=None):
        """One optimizer step with gradient g (fp32, bf16 or fp16, same length as x)."""
        if g.numel() != self.x.numel():
            raise ValueError("gradient and parameters differ in length")
        t = self.step_count + 1
        if t <= self.freeze_step:
            ob.onebit_adam_warmup_step(self.x, self.m, self.v, g, lr=self.lr, beta1=self.beta1, beta2=self.beta2,
                                       eps=self.eps, weight_decay=self.weight_decay,
                                       bias_correction=self.bias_correction, step=t, stream=stream)
        else:
            ob.onebit_compress_update(self.plan, g, self.m, self.e, self.v, self.x, None, self.bits, self.scales,
                                      lr=self.lr, beta1=self.beta1, eps=self.eps, weight_decay=self.weight_decay,
                                      workspace=self.workspace, stream=stream)
            self.compressed_steps += 1
        self.step_count = t
        if t > self.freeze_step and self.check_every > 0 and self.compressed_steps % self.check_every == 0:
            self.check(stream)

    def check(self, stream=None):
        """Raise WaitTimeout (after re-initializing the workspace) if a bounded wait of a
        compressed step since the last check gave up."""
        status = ob.onebit_workspace_status(self.workspace, stream)
        if status != 0:
            ob.onebit_workspace_init(self.workspace, stream)
            raise WaitTimeout(f"a cross-workgroup wait gave up (code {status}) during the compressed steps up to "
                              f"step {self.step_count}; their outputs are not valid")

    def state_dict(self) -> dict:
        """Step count, momentum and variance (the compression error is not kept)."""
        return {"step": self.step_count, "exp_avg": self.m.clone(), "exp_avg_sq": self.v.clone()}

    def load_state_dict(self, state: dict):
        """Restore step, m and v; the compression error restarts from zero."""
        self.step_count = int(state["step"])
        self.m.copy_(state["exp_avg"])
        self.v.copy_(state["exp_avg_sq"])
        self.e.zero_()
