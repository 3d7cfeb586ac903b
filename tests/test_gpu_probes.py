"""GPU checks of the measurement probes (qa_probe.h): the streaming read
returns the exact XOR of what thread 0 of each workgroup visits, and every
matrix- and vector-throughput kind runs and leaves finite values."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


def test_stream_read_visits_every_element():
    from quantized_attention_quantize_amd import probes
    wgs, n16 = 8, 8 * 256 * 3 + 100            # a ragged grid-stride tail
    data = (np.arange(n16 * 4, dtype=np.int64) * 2654435761 % (1 << 31)).astype(np.int32)
    src = torch.from_numpy(data).cuda()
    sink = torch.full((wgs,), -1, dtype=torch.int32, device="cuda")
    say("probe stream_read", n16 * 16, "bytes,", wgs, "workgroups")
    probes.stream_read(src, wgs, sink, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    v = data.reshape(n16, 4)
    want = []
    for b in range(wgs):
        idx = np.arange(b * 256, n16, wgs * 256)      # the int4 elements thread 0 of workgroup b reads
        w = np.bitwise_xor.reduce(v[idx].reshape(-1)) if idx.size else 0
        want.append(int(w))
    assert sink.cpu().numpy().tolist() == want


@pytest.mark.parametrize("kind", list(range(9)))
def test_mfma_probe_runs(kind):
    from quantized_attention_quantize_amd import probes
    sink = torch.full((4 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    say("probe mfma kind", kind)
    ops = probes.mfma(kind, 10, 4, sink, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert ops == probes.MFMA_KINDS[kind][1] * 10 * 4 * 4
    assert torch.isfinite(sink).all()


@pytest.mark.parametrize("kind", [0, 1])
def test_valu_probe_runs(kind):
    from quantized_attention_quantize_amd import probes
    sink = torch.full((4 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    say("probe valu kind", kind)
    ops = probes.valu(kind, 10, 4, sink, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert ops == 8 * 10 * 256 * 4
    s = sink.cpu()
    assert torch.isfinite(s).all()
    if kind == 0:
        assert ((s > 8 * 0.5) & (s <= 8.0)).all()     # eight values of 2^-x, each in (0.5, 1]
