"""The streaming probe (diagnostics) writes out_k = sum of its inputs + k."""
import pytest
import torch

from error_compensated_bit_amd import onebit as ob
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("block", [256, 1024])
@pytest.mark.parametrize("reads,writes", [(5, 3), (1, 1)])
def test_stream_probe_values(reads, writes, block):
    n = 1024 * 4 * 4 * 3 + 44                   # several grid-stride spans and a ragged last one
    ins = [torch.randn(n, device=DEV) for _ in range(reads)]
    outs = [torch.zeros(n, device=DEV) for _ in range(writes)]
    keep = ob.onebit_stream_probe(ins, outs, 2, block)
    torch.cuda.synchronize()
    s = torch.zeros(n, device=DEV)
    for t in ins:
        s = s + t
    for k, o in enumerate(outs):
        assert torch.equal(o, s + float(k))
    del keep
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_stream_probe(ins[:1], outs, 2) if writes == 3 else ob.onebit_stream_probe(ins * 2, outs, 2)
    assert ei.value.status == ob.ONEBIT_ERR_UNSUPPORTED
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_stream_probe(ins, outs, 2, 300)
    assert ei.value.status == ob.ONEBIT_ERR_INVALID
