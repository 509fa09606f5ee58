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
onebit_compress_update; OneBitAdamWorkers below makes the W workers' calls of the
simulated all-reduce); m, v, the errors, the packed words, the scales and the
workspace are device tensors these objects allocate next to x.  Bias correction,
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


def _check_workspace(opt, stream):
    """Raise WaitTimeout (after re-initializing the workspace) if a bounded wait of a
    compressed step since the last check gave up."""
    status = ob.onebit_workspace_status(opt.workspace, stream)
    if status != 0:
        ob.onebit_workspace_init(opt.workspace, stream)
        raise WaitTimeout(f"a cross-workgroup wait gave up (code {status}) during the compressed steps up to "
                          f"step {opt.step_count}; their outputs are not valid")


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
        _check_workspace(self, stream)

    def state_dict(self) -> dict:
        """Step count, momentum and variance (the compression error is not kept)."""
        return {"step": self.step_count, "exp_avg": self.m.clone(), "exp_avg_sq": self.v.clone()}

    def load_state_dict(self, state: dict):
        """Restore step, m and v; the compression error restarts from zero."""
        self.step_count = int(state["step"])
        self.m.copy_(state["exp_avg"])
        self.v.copy_(state["exp_avg_sq"])
        self.e.zero_()


class OneBitAdamWorkers:
    """1-bit Adam over W data-parallel workers whose buffers share one GPU's memory:
    the compressed all-reduce of the guide's sec. 4 with a worker error per worker and
    one server error, simulated in place of the exchange between GPUs.

    Every worker holds the same x, m and v (the all-reduce makes them equal), so one
    copy of each is kept; each worker has its own gradient and its own compression
    error.  step(grads) takes the W workers' gradients as one [W, n] tensor (fp32,
    bf16 or fp16):
      warmup (steps 1..freeze_step)  the gradients are averaged at full precision
          (onebit_average_rows, the warmup phase's all-reduce) and the Adam step runs
          on the average (onebit_adam_warmup_step);
      compressed (later steps)  every worker compresses beta1 m + (1 - beta1) g_w plus
          its error (onebit_compress_update, compress-only), the server stage averages
          the W decompressed streams and compresses again with the server error
          (onebit_server_reduce), and the finish multiplies the result by exp_avg_mask
          and takes the frozen-v step (onebit_momentum_update).
    With packed_momentum the momentum is kept, after the first compressed step, as
    the server's sign words and chunk scales (times the mask) instead of an fp32
    array: the workers read it through onebit_compress_update_packed and the finish
    through onebit_momentum_update_packed, with every result identical.

    chunk_offsets   the all-reduce's chunk table (one scale per worker and chunk and
                    one per server chunk); default: the whole vector as one chunk;
    exp_avg_mask    uint8 or bool [n] device tensor, 0 = the momentum is zeroed there
                    after the all-reduce (guide sec. 3.5); None: no mask.
    The checkpoint (state_dict) keeps the step, m (decompressed in packed mode) and v;
    load_state_dict restarts both errors from zero (guide sec. 7).  Errors of bounded
    waits are checked as in OneBitAdam.
    """

    def __init__(self, x, workers, *, chunk_offsets=None, exp_avg_mask=None, lr=1e-3, betas=(0.9, 0.999),
                 eps=1e-8, weight_decay=0.0, bias_correction=False, freeze_step=100000, packed_momentum=False,
                 check_every=1):
        if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.dim() != 1:
            raise TypeError("x must be a one-dimensional float32 tensor")
        if int(workers) < 1:
            raise ValueError("workers must be >= 1")
        if freeze_step < 0:
            raise ValueError("freeze_step must be >= 0")
        n = x.numel()
        co = np.asarray(chunk_offsets if chunk_offsets is not None else [0, n], dtype=np.int64)
        if co.ndim != 1 or co.size < 2 or co[0] != 0 or co[-1] != n:
            raise ValueError("chunk_offsets must start at 0 and end at x.numel()")
        if exp_avg_mask is not None:
            if exp_avg_mask.numel() != n or exp_avg_mask.dtype not in (torch.uint8, torch.bool):
                raise ValueError("exp_avg_mask must be a uint8 or bool tensor with one entry per parameter")
            exp_avg_mask = exp_avg_mask.to(torch.uint8).contiguous()
        self.x, self.W, self.mask = x, int(workers), exp_avg_mask
        self.lr, self.beta1, self.beta2 = float(lr), float(betas[0]), float(betas[1])
        self.eps, self.weight_decay = float(eps), float(weight_decay)
        self.bias_correction = bool(bias_correction)
        self.freeze_step = int(freeze_step)
        self.packed = bool(packed_momentum)
        self.check_every = int(check_every)
        self.step_count = 0
        self.compressed_steps = 0
        dev = x.device
        self.m = torch.zeros_like(x)
        self.v = torch.zeros_like(x)
        # rows padded to 64 elements, so every worker's row starts on a 256-byte boundary
        self.row_stride = (n + 63) // 64 * 64
        self.worker_error = torch.zeros((self.W, self.row_stride), dtype=torch.float32, device=dev)[:, :n]
        self.server_error = torch.zeros_like(x)
        self.g_avg = torch.zeros_like(x)
        self.plan = ob.onebit_plan_create(co)
        words, chunks = max(ob.onebit_plan_words(self.plan), 1), max(ob.onebit_plan_chunks(self.plan), 1)
        self.worker_bits = torch.zeros((self.W, words), dtype=torch.int32, device=dev)
        self.worker_scales = torch.zeros((self.W, chunks), dtype=torch.float32, device=dev)
        # two (words, scales) pairs: the server writes one while the workers read the other
        self.server_bits = [torch.zeros(words, dtype=torch.int32, device=dev) for _ in range(2)]
        self.server_scales = [torch.zeros(chunks, dtype=torch.float32, device=dev) for _ in range(2)]
        self.current = None      # index of the pair that holds m in packed form, None: m is the fp32 array
        self.workspace = torch.zeros(max(ob.onebit_plan_workspace_bytes(self.plan) // 8, 1), dtype=torch.int64,
                                     device=dev)

    @property
    def frozen(self) -> bool:
        return self.step_count >= self.freeze_step

    def gradient_buffer(self, dtype=torch.float32):
        """A [W, n] device tensor whose rows start on 256-byte boundaries (a view of a
        row-padded allocation), for the workers' gradients."""
        return torch.zeros((self.W, self.row_stride), dtype=dtype, device=self.x.device)[:, :self.x.numel()]

    def step(self, grads, stream=None):
        """One step with the W workers' gradients: a [W, n] tensor (fp32, bf16 or fp16)
        whose rows are contiguous and start on 16-byte boundaries, e.g. one from
        gradient_buffer()."""
        if grads.dim() != 2 or grads.shape[0] != self.W or grads.shape[1] != self.x.numel():
            raise ValueError(f"grads must be a [{self.W}, {self.x.numel()}] tensor")
        if grads.stride(1) != 1 or (grads.data_ptr() | grads.stride(0) * grads.element_size()) % 16 != 0:
            raise ValueError("every gradient row must be contiguous and start on a 16-byte boundary "
                             "(use gradient_buffer())")
        t = self.step_count + 1
        hp = dict(lr=self.lr, eps=self.eps, weight_decay=self.weight_decay, stream=stream)
        if t <= self.freeze_step:
            ob.onebit_average_rows(grads, self.g_avg, stream=stream)
            ob.onebit_adam_warmup_step(self.x, self.m, self.v, self.g_avg, beta1=self.beta1, beta2=self.beta2,
                                       bias_correction=self.bias_correction, step=t, **hp)
        elif self.current is None:
            nxt = 0
            for w in range(self.W):
                ob.onebit_compress_update(self.plan, grads[w], self.m, self.worker_error[w], None, None, None,
                                          self.worker_bits[w], self.worker_scales[w], lr=0.0, beta1=self.beta1,
                                          eps=self.eps, weight_decay=0.0, workspace=self.workspace, stream=stream)
            ob.onebit_server_reduce(self.plan, self.worker_bits, self.worker_scales, self.server_error,
                                    self.server_bits[nxt], self.server_scales[nxt], self.m, self.workspace,
                                    stream=stream)
            ob.onebit_momentum_update(self.m, self.mask, self.v, self.x, None, **hp)
            if self.packed:
                self.current = nxt
        else:
            cur, nxt = self.current, 1 - self.current
            for w in range(self.W):
                ob.onebit_compress_update_packed(self.plan, grads[w], self.server_bits[cur], self.server_scales[cur],
                                                 self.worker_error[w], None, None, None, self.worker_bits[w],
                                                 self.worker_scales[w], lr=0.0, beta1=self.beta1, eps=self.eps,
                                                 weight_decay=0.0, workspace=self.workspace, m_mask=self.mask,
                                                 stream=stream)
            ob.onebit_server_reduce(self.plan, self.worker_bits, self.worker_scales, self.server_error,
                                    self.server_bits[nxt], self.server_scales[nxt], None, self.workspace,
                                    stream=stream)
            ob.onebit_momentum_update_packed(self.plan, self.server_bits[nxt], self.server_scales[nxt], self.mask,
                                             self.v, self.x, None, **hp)
            self.current = nxt
        if t > self.freeze_step:
            self.compressed_steps += 1
        self.step_count = t
        if t > self.freeze_step and self.check_every > 0 and self.compressed_steps % self.check_every == 0:
            _check_workspace(self, stream)

    def check(self, stream=None):
        """Raise WaitTimeout (after re-initializing the workspace) if a bounded wait of a
        compressed step since the last check gave up."""
        _check_workspace(self, stream)

    def exp_avg(self, stream=None):
        """The momentum as an fp32 [n] tensor (decompressed from the packed form)."""
        if self.current is None:
            return self.m.clone()
        out = torch.empty_like(self.x)
        ob.onebit_decompress(self.plan, self.server_bits[self.current], self.server_scales[self.current], self.mask,
                             out, stream=stream)
        return out

    def state_dict(self) -> dict:
        """Step count, momentum and variance (the worker and server errors are not kept)."""
        return {"step": self.step_count, "exp_avg": self.exp_avg(), "exp_avg_sq": self.v.clone()}

    def load_state_dict(self, state: dict):
        """Restore step, m and v; the worker and server errors restart from zero."""
        self.step_count = int(state["step"])
        self.m.copy_(state["exp_avg"])
        self.v.copy_(state["exp_avg_sq"])
        self.current = None
        self.worker_error.zero_()
        self.server_error.zero_()


def variance_update_steps(var_freeze_step, var_update_scaler):
    """The steps (1-based) at which 0/1 Adam's adaptive variance freezing updates v.

    The DeepSpeed guide (sec. 8, from 1-bit Adam to 0/1 Adam) names the method's
    adaptive variance freezing and its parameters var_freeze_step and
    var_update_scaler, but gives no rule.  Reading taken here: v is updated at step 1;
    the spacing between consecutive updates starts at 1 step and doubles after every
    var_update_scaler updates (var_update_scaler spacings of 1, then as many of 2,
    then of 4, ...); no update comes after var_freeze_step, from which on v stays
    frozen.
    """
    if var_update_scaler < 1 or var_freeze_step < 0:
        raise ValueError("var_update_scaler must be >= 1 and var_freeze_step >= 0")
    steps, t = [], 1
    while t <= var_freeze_step:
        # after update j (0-based) the next one is 2^(j // var_update_scaler) steps later
        t_next = t + (1 << (len(steps) // var_update_scaler))
        steps.append(t)
        t = t_next
    return steps


class ZeroOneAdam(OneBitAdam):
    """0/1 Adam's adaptive variance freezing over one flat vector (a reading: the
    guide names the method and its parameters only; see variance_update_steps).

    At the variance-update steps the step is full-precision Adam (m and v updated,
    onebit_adam_warmup_step); every other step is the error-compensated 1-bit
    compressed momentum step with the current v held fixed (onebit_compress_update),
    and after var_freeze_step v never changes again.  The compression error carries
    over the full-precision steps unchanged.  With var_update_scaler large enough that
    the spacing never doubles before var_freeze_step, every step up to it updates v
    and this is 1-bit Adam with freeze_step = var_freeze_step.  The guide's local
    steps (local_step_scaler, local_step_clipper) skip the synchronization between
    GPUs and are not modelled on one GPU.
    """

    def __init__(self, x, *, var_freeze_step=100000, var_update_scaler=16, **kw):
        if "freeze_step" in kw:
            raise TypeError("ZeroOneAdam takes var_freeze_step, not freeze_step")
        super().__init__(x, freeze_step=var_freeze_step, **kw)
        self.var_update_scaler = int(var_update_scaler)
        self._var_steps = set(variance_update_steps(self.freeze_step, self.var_update_scaler))

    def is_variance_step(self, t: int) -> bool:
        return t in self._var_steps

    def step(self, g, stream=None):
        if g.numel() != self.x.numel():
            raise ValueError("gradient and parameters differ in length")
        t = self.step_count + 1
        if self.is_variance_step(t):
            ob.onebit_adam_warmup_step(self.x, self.m, self.v, g, lr=self.lr, beta1=self.beta1, beta2=self.beta2,
                                       eps=self.eps, weight_decay=self.weight_decay,
                                       bias_correction=self.bias_correction, step=t, stream=stream)
            self.step_count = t
            return
        ob.onebit_compress_update(self.plan, g, self.m, self.e, self.v, self.x, None, self.bits, self.scales,
                                  lr=self.lr, beta1=self.beta1, eps=self.eps, weight_decay=self.weight_decay,
                                  workspace=self.workspace, stream=stream)
        self.compressed_steps += 1
        self.step_count = t
        if self.check_every > 0 and self.compressed_steps % self.check_every == 0:
            _check_workspace(self, stream)
