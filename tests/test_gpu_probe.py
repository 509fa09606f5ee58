"""The streaming probe (diagnostics) writes out_k = sum of its inputs + k, for every
supported read/write mix and both cache policies, and with the loads staged in LDS
(ragged lengths, fewer chunks than waves, grids that leave waves idle or give each
wave many chunks); the read-only mix leaves its input unchanged; unsupported mixes,
workgroup sizes and policies are refused.  The Philox probe's per-thread words
equal the XOR of the oracle generator's blocks."""
import numpy as np
import pytest
import torch

import oracle

from error_compensated_bit_amd import onebit as ob
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu

MIXES = [(1, 0), (0, 1), (1, 1), (2, 1), (3, 1), (1, 2), (2, 2), (4, 2), (5, 3)]


@pytest.mark.parametrize("nontemporal", [True, False])
@pytest.mark.parametrize("block", [256, 1024])
@pytest.mark.parametrize("reads,writes", MIXES)
def test_stream_probe_values(reads, writes, block, nontemporal):
    n = 1024 * 4 * 4 * 3 + 44                   # several grid-stride spans and a ragged last one
    ins = [torch.randn(n, device=DEV) for _ in range(reads)]
    before = [t.clone() for t in ins]
    outs = [torch.zeros(n, device=DEV) for _ in range(writes)]
    keep = ob.onebit_stream_probe(ins, outs, 2, block, 1 if nontemporal else 0)
    torch.cuda.synchronize()
    s = torch.zeros(n, device=DEV)
    for t in ins:
        s = s + t
    for k, o in enumerate(outs):
        assert torch.equal(o, s + float(k))
    for a, b in zip(ins, before):
        assert torch.equal(a, b)
    del keep


@pytest.mark.parametrize("n,grid", [(4, 1), (516, 3), (1024 * 4 * 4 * 3 + 44, 2), (1 << 20, 7), ((1 << 20) + 12, 300)])
@pytest.mark.parametrize("reads,writes", [m for m in MIXES if m[0] > 0])
def test_stream_probe_lds_staged_values(reads, writes, n, grid):
    ins = [torch.randn(n, device=DEV) for _ in range(reads)]
    before = [t.clone() for t in ins]
    outs = [torch.zeros(n, device=DEV) for _ in range(writes)]
    keep = ob.onebit_stream_probe(ins, outs, grid, 256, 2)
    torch.cuda.synchronize()
    s = torch.zeros(n, device=DEV)
    for t in ins:
        s = s + t
    for k, o in enumerate(outs):
        assert torch.equal(o, s + float(k)), (reads, writes, n, grid, k)
    for a, b in zip(ins, before):
        assert torch.equal(a, b)
    del keep


@pytest.mark.parametrize("seed,n_blocks,grid,block", [(0, 0, 1, 256), (7, 1, 1, 256), (12345, 1000, 2, 256),
                                                      ((1 << 40) + 7, 3001, 3, 512), (99, 700, 1, 1024)])
def test_philox_probe_matches_the_oracle_generator(seed, n_blocks, grid, block):
    """Every thread's word is the XOR of the four words of its blocks, drawn with the
    oracle's own Philox4x32-10 (key = the seed's low / high words, counter = block)."""
    T = grid * block
    out = torch.full((T,), -1, dtype=torch.int32, device=DEV)
    ob.onebit_philox_probe(seed, n_blocks, out, grid, block)
    torch.cuda.synchronize()
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32)
    want = np.zeros(T, np.uint32)
    for blk in range(n_blocks):
        r = oracle.philox4x32_10(key, np.array([blk & 0xFFFFFFFF, blk >> 32, 0, 0], np.uint32))
        want[blk % T] ^= r[0] ^ r[1] ^ r[2] ^ r[3]
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)


def test_stream_probe_refusals():
    n = 4096
    ins = [torch.zeros(n, device=DEV) for _ in range(3)]
    outs = [torch.zeros(n, device=DEV) for _ in range(2)]
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_stream_probe(ins, outs, 2)                  # 3 + 2 is not a supported mix
    assert ei.value.status == ob.ONEBIT_ERR_UNSUPPORTED
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_stream_probe(ins[:1], outs[:1], 2, 300)
    assert ei.value.status == ob.ONEBIT_ERR_INVALID
    for args in [(ins[:1], outs[:1], 2, 1024, 2), ([], outs[:1], 2, 256, 2), (ins[:1], outs[:1], 2, 256, 3),
                 (ins[:1], outs[:1], 2, 256, -1)]:
        with pytest.raises(ob.OnebitError) as ei:
            ob.onebit_stream_probe(*args)
        assert ei.value.status == ob.ONEBIT_ERR_INVALID
    w = torch.zeros(256, dtype=torch.int32, device=DEV)
    for args in [(1, -1, w, 1, 256), (1, 10, w[:0], 0, 256), (1, 10, w[:128], 1, 128)]:
        with pytest.raises(ob.OnebitError) as ei:
            ob.onebit_philox_probe(*args)
        assert ei.value.status == ob.ONEBIT_ERR_INVALID
