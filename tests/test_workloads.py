"""Host-side checks of the synthetic workloads: table sizes, chunk histograms, seeding."""
import collections

import numpy as np
import torch

from error_compensated_bit_amd import workloads as W


def test_bert_large_table():
    shapes = W.bert_tensor_shapes()
    assert len(shapes) == 393
    sizes = [int(np.prod(s)) for _, s in shapes]
    assert sum(sizes) == 335_143_938
    hist = collections.Counter(sizes)
    assert hist == {1024: 219, 4096: 24, 2048: 2, 2: 1, 1 << 20: 97, 4 << 20: 48, 524_288: 1, 31_254_528: 1}
    wl = W.bert_like()
    assert wl.plan_words == 10_473_249
    assert int((wl.tensor_keep == 0).sum()) == 8
    # every tensor but the last starts on a multiple of 4 elements
    assert np.all(wl.chunk_off[:-1] % 4 == 0)


def test_gpt2_and_qsdp_sizes():
    assert W.gpt2_param_count() == 1_557_611_200
    wl = W.gpt2_like()
    assert wl.n_chunks == 1486
    assert int(wl.chunk_off[-1] - wl.chunk_off[-2]) == 475_840
    assert wl.plan_words == 48_675_350
    q = W.QsdpWorkload()
    assert (q.n + q.bucket - 1) // q.bucket == 1_269_532 and q.n % q.bucket == 256
    a = W.AllreduceWorkload()
    assert a.chunk_off.size == 17 and a.n == 67_108_864


def test_generators_are_seeded_and_masked():
    wl = W.bert_small()
    g1 = W.gradient(wl, 2)
    g2 = W.gradient(wl, 2)
    assert torch.equal(g1, g2) and not torch.equal(g1, W.gradient(wl, 3))
    masked = np.repeat(wl.tensor_keep == 0, np.diff(wl.tensor_off))
    assert torch.all(g1[torch.from_numpy(masked)] == 0)
    x, m, e, v = W.init_state(wl)
    assert torch.all(m == 0) and torch.all(e == 0) and torch.all(v > 0)
    gw = W.gpt2_like(n=100_003)
    gb = W.gradient(gw, 1)
    assert gb.dtype == torch.bfloat16 and gb.numel() == 100_003
    big = (gb.float().abs() > 0.02).sum().item()
    assert 20 <= big <= 200           # about 0.1 % heavy-tail elements


def test_fixed_chunks_ragged_tail():
    off = W.fixed_chunks(10, 4)
    assert off.tolist() == [0, 4, 8, 10]
    assert W.fixed_chunks(0, 4).tolist() == [0]
