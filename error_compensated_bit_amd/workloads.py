"""Seeded synthetic inputs for the 1-bit Adam hot path and the QSDP quantizer.

This module only draws random numbers and builds offset tables; it holds none of
the method's arithmetic.  The same inputs are handed to the HIP library and to the
CPU oracle, so parity never depends on how they were drawn.

Workloads (all synthetic; the pages' datasets and weights are not used):
  tiny        n = 1,048,576 fp32, one chunk: 5 Adam warmup steps, then 5
              compressed steps.
  bert_large  335,143,938 fp32 params in the 393 tensors of BERT-Large (HF
              BertModel order plus the next-sentence head), one chunk per tensor,
              per-tensor gradient std log-uniform in [1e-4, 1e-1], 8 tensors with
              all-zero gradients and masked, v = std^2 * U(0.5, 2).
  allreduce   W = 16 worker buffers of 64M fp32, 16 chunks of 4M per buffer,
              gradients N(0, 1e-3) with per-worker seeds, 3 steps.
  gpt2_xl     1,557,611,200 params (GPT-2 XL), fp32 x/m/v/e, bf16 gradients with
              std 1e-3 and 0.1% outliers with std 0.1, chunks of 2^20 (the last one
              ragged), bf16 copy of x, 3 steps.
  qsdp        1.3e9 bf16 weights ~ N(0, 0.02), buckets of 1024, 4- and 8-bit codes,
              64 seeds.
  qsgd        the gradients of the same 1.3e9-parameter model, bf16, N(0, 1) scaled
              per block of 2^20 elements by 10^U(-4, -2) (layers differ in gradient
              scale), one vector per worker; W = 8 workers, each owning a
              bucket-aligned shard of ceil(n / 8 / 1024) buckets; 4- and 8-bit codes.
"N(mu, s)" means standard deviation s.

Seeds: workload k uses base seed 1000*k; step t adds t; worker w adds 100*w.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

HYPER = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, bias_correction=False)

SEED_TINY, SEED_BERT, SEED_ALLREDUCE, SEED_GPT2, SEED_QSDP, SEED_QSGD = 0, 1000, 2000, 3000, 4000, 5000


# ----------------------------------------------------------------- tables

def bert_tensor_shapes(hidden=1024, ffn=4096, layers=24, vocab=30522, max_pos=512, type_vocab=2,
                       nsp_head=True) -> List[Tuple[str, Tuple[int, ...]]]:
    """Parameter tensors of a BERT encoder in HF BertModel order, plus the NSP head."""
    h, f = hidden, ffn
    t = [("embeddings.word_embeddings.weight", (vocab, h)),
         ("embeddings.position_embeddings.weight", (max_pos, h)),
         ("embeddings.token_type_embeddings.weight", (type_vocab, h)),
         ("embeddings.LayerNorm.weight", (h,)),
         ("embeddings.LayerNorm.bias", (h,))]
    for i in range(layers):
        p = f"encoder.layer.{i}."
        t += [(p + "attention.self.query.weight", (h, h)), (p + "attention.self.query.bias", (h,)),
              (p + "attention.self.key.weight", (h, h)), (p + "attention.self.key.bias", (h,)),
              (p + "attention.self.value.weight", (h, h)), (p + "attention.self.value.bias", (h,)),
              (p + "attention.output.dense.weight", (h, h)), (p + "attention.output.dense.bias", (h,)),
              (p + "attention.output.LayerNorm.weight", (h,)), (p + "attention.output.LayerNorm.bias", (h,)),
              (p + "intermediate.dense.weight", (f, h)), (p + "intermediate.dense.bias", (f,)),
              (p + "output.dense.weight", (h, f)), (p + "output.dense.bias", (h,)),
              (p + "output.LayerNorm.weight", (h,)), (p + "output.LayerNorm.bias", (h,))]
    t += [("pooler.dense.weight", (h, h)), ("pooler.dense.bias", (h,))]
    if nsp_head:
        t += [("cls.seq_relationship.weight", (2, h)), ("cls.seq_relationship.bias", (2,))]
    return t


def gpt2_param_count(d=1600, layers=48, vocab=50257, ctx=1024) -> int:
    """GPT-2 parameter count (tied LM head): wte, wpe, per block ln_1, attn, ln_2, mlp; ln_f."""
    per_block = 2 * d + (d * 3 * d + 3 * d) + (d * d + d) + 2 * d + (d * 4 * d + 4 * d) + (4 * d * d + d)
    return vocab * d + ctx * d + layers * per_block + 2 * d


def offsets_from_sizes(sizes) -> np.ndarray:
    off = np.zeros(len(sizes) + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(sizes, dtype=np.int64))
    return off


def fixed_chunks(n: int, chunk: int) -> np.ndarray:
    """Offsets of fixed-size chunks over [0, n); the last chunk holds the remainder."""
    if n == 0:
        return np.zeros(1, dtype=np.int64)
    k = (n + chunk - 1) // chunk
    off = np.arange(k + 1, dtype=np.int64) * chunk
    off[-1] = n
    return off


# ----------------------------------------------------------- descriptors

@dataclass
class CompressWorkload:
    """A flat parameter vector with its chunk table and (optional) tensor/mask table."""
    name: str
    n: int
    chunk_off: np.ndarray
    tensor_off: Optional[np.ndarray] = None
    tensor_keep: Optional[np.ndarray] = None
    tensor_std: Optional[np.ndarray] = None     # per-tensor gradient std (None: grad_std everywhere)
    grad_std: float = 1e-3
    outlier_p: float = 0.0                      # probability of a heavy-tail element
    outlier_std: float = 0.0
    grad_bf16: bool = False
    x_bf16_copy: bool = False
    base_seed: int = 0
    hyper: dict = field(default_factory=lambda: dict(HYPER))

    @property
    def n_chunks(self) -> int:
        return int(self.chunk_off.size - 1)

    @property
    def plan_words(self) -> int:
        lens = np.diff(self.chunk_off)
        return int(((lens + 31) // 32).sum())


def tiny(n: int = 1 << 20) -> CompressWorkload:
    return CompressWorkload("tiny", n, fixed_chunks(n, max(n, 1)), base_seed=SEED_TINY)


def bert_like(shapes=None, n_masked=8, seed=SEED_BERT, name="bert_large") -> CompressWorkload:
    """One chunk per tensor; per-tensor gradient std 10^U(-4,-1); n_masked tensors masked."""
    shapes = shapes if shapes is not None else bert_tensor_shapes()
    sizes = [int(np.prod(s)) for _, s in shapes]
    off = offsets_from_sizes(sizes)
    rng = np.random.Generator(np.random.Philox(seed))
    std = (10.0 ** rng.uniform(-4.0, -1.0, size=len(sizes))).astype(np.float64)
    keep = np.ones(len(sizes), dtype=np.uint8)
    if n_masked:
        keep[rng.choice(len(sizes), size=n_masked, replace=False)] = 0
    return CompressWorkload(name, int(off[-1]), off.copy(), off.copy(), keep, std, base_seed=seed)


def bert_small(seed=SEED_BERT + 1) -> CompressWorkload:
    """A scaled-down BERT table (mixed tensor sizes, several masked tensors) for quick parity runs."""
    shapes = bert_tensor_shapes(hidden=96, ffn=384, layers=2, vocab=997, max_pos=64, type_vocab=2)
    return bert_like(shapes, n_masked=4, seed=seed, name="bert_small")


def gpt2_like(n: int = None, chunk: int = 1 << 20, seed=SEED_GPT2) -> CompressWorkload:
    n = gpt2_param_count() if n is None else n
    return CompressWorkload("gpt2_xl" if n == gpt2_param_count() else f"gpt2_like_{n}", n,
                            fixed_chunks(n, chunk), grad_std=1e-3, outlier_p=1e-3, outlier_std=0.1,
                            grad_bf16=True, x_bf16_copy=True, base_seed=seed)


@dataclass
class AllreduceWorkload:
    W: int = 16
    n: int = 64 << 20
    chunk: int = 4 << 20
    grad_std: float = 1e-3
    steps: int = 3
    base_seed: int = SEED_ALLREDUCE

    @property
    def chunk_off(self) -> np.ndarray:
        return fixed_chunks(self.n, self.chunk)


@dataclass
class QsdpWorkload:
    n: int = 1_300_000_000
    bucket: int = 1024
    std: float = 0.02
    seeds: int = 64
    base_seed: int = SEED_QSDP


@dataclass
class QsgdWorkload:
    n: int = 1_300_000_000
    bucket: int = 1024
    W: int = 8
    block: int = 1 << 20
    base_seed: int = SEED_QSGD

    @property
    def shard(self) -> int:
        """Elements per worker's shard: a whole number of buckets."""
        return -(-self.n // self.W // self.bucket) * self.bucket if self.n >= self.W * self.bucket else self.n


# -------------------------------------------------------------- generators

def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _per_element(values: np.ndarray, off: np.ndarray, device) -> torch.Tensor:
    sizes = torch.as_tensor(np.diff(off), dtype=torch.int64, device=device)
    return torch.repeat_interleave(torch.as_tensor(values, dtype=torch.float32, device=device), sizes)


def init_state(wl: CompressWorkload, device="cpu"):
    """x ~ N(0, 0.02); m = e = 0; v = std^2 * U(0.5, 2) (zero for the tiny workload, which warms up)."""
    gen = _gen(device, wl.base_seed + 999)
    x = torch.randn(wl.n, generator=gen, device=device, dtype=torch.float32).mul_(0.02)
    m = torch.zeros(wl.n, device=device, dtype=torch.float32)
    e = torch.zeros(wl.n, device=device, dtype=torch.float32)
    if wl.name == "tiny":
        v = torch.zeros(wl.n, device=device, dtype=torch.float32)
    else:
        u = torch.rand(wl.n, generator=gen, device=device, dtype=torch.float32).mul_(1.5).add_(0.5)
        if wl.tensor_std is not None:
            s = _per_element(wl.tensor_std, wl.tensor_off, device)
            v = u.mul_(s * s)
        else:
            v = u.mul_(wl.grad_std * wl.grad_std)
    return x, m, e, v


def gradient(wl: CompressWorkload, step: int, device="cpu", worker: int = 0) -> torch.Tensor:
    """Gradient for step t (1-based) of worker w: fp32, or bf16 (round-to-nearest-even) when requested."""
    gen = _gen(device, wl.base_seed + step + 100 * worker)
    g = torch.randn(wl.n, generator=gen, device=device, dtype=torch.float32)
    if wl.tensor_std is not None:
        g.mul_(_per_element(wl.tensor_std, wl.tensor_off, device))
    else:
        g.mul_(wl.grad_std)
    if wl.outlier_p > 0:
        hit = torch.rand(wl.n, generator=gen, device=device) < wl.outlier_p
        big = torch.randn(wl.n, generator=gen, device=device, dtype=torch.float32).mul_(wl.outlier_std)
        g = torch.where(hit, big, g)
    if wl.tensor_keep is not None:
        masked = _per_element((wl.tensor_keep == 0).astype(np.float32), wl.tensor_off, device) > 0
        g.masked_fill_(masked, 0.0)
    if wl.grad_bf16:
        g = g.to(torch.bfloat16)
    return g


def allreduce_gradient(wl: AllreduceWorkload, step: int, worker: int, device="cpu") -> torch.Tensor:
    gen = _gen(device, wl.base_seed + step + 100 * worker)
    return torch.randn(wl.n, generator=gen, device=device, dtype=torch.float32).mul_(wl.grad_std)


def qsdp_weights(wl: QsdpWorkload, device="cpu") -> torch.Tensor:
    """bf16 weights ~ N(0, std), returned as a bfloat16 tensor."""
    gen = _gen(device, wl.base_seed)
    return torch.randn(wl.n, generator=gen, device=device, dtype=torch.float32).mul_(wl.std).to(torch.bfloat16)


def qsgd_gradient(wl: QsgdWorkload, worker: int, device="cpu", n: Optional[int] = None) -> torch.Tensor:
    """bf16 gradient of one worker: N(0, 1) times a per-block scale 10^U(-4, -2)."""
    n = wl.n if n is None else n
    gen = _gen(device, wl.base_seed + 100 * worker)
    nblk = -(-n // wl.block)
    scale = torch.pow(10.0, torch.rand(nblk, generator=gen, device=device) * 2.0 - 4.0)
    g = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
    g.view(-1)[: (n // wl.block) * wl.block].view(-1, wl.block).mul_(scale[: n // wl.block, None])
    if n % wl.block:
        g[(n // wl.block) * wl.block:].mul_(scale[-1])
    return g.to(torch.bfloat16)


def as_u16(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
