"""The measurement probes behind bench.py --microbench: they run, leave their sinks alone
(the sink is written only on values that never occur, so the work cannot be dropped), and
report plausible shader-clock cycles; bad arguments are refused on the host."""
import pytest
import torch

import mixture_experts_ffn_03_amd as M

pytestmark = pytest.mark.gpu


def test_stream_read_probe():
    print("case: stream read probe", flush=True)
    src = torch.ones(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(M.PROBE_READ_BLOCKS, dtype=torch.float32, device="cuda")
    M.probe_stream_read(src, sink)
    M.probe_stream_read(src[: (1 << 20) + 48], sink)  # a ragged tail of 16-byte pieces
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0
    with pytest.raises(M.MoeError):
        M.probe_stream_read(src[:20], sink)  # not a multiple of 16 bytes


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_mfma_probe(kind):
    print("case: mfma probe", kind, flush=True)
    blocks = M.probe_mfma_blocks(2)
    assert blocks == 2 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(blocks, dtype=torch.float32, device="cuda")
    cycles = torch.zeros(blocks, dtype=torch.int64, device="cuda")
    M.probe_mfma(kind, 256, 2, sink, cycles)
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0
    # 256 rounds of 8 MFMAs of at least 16 cycles each, two waves sharing each SIMD
    assert cycles.min().item() >= 256 * 8 * 16
    with pytest.raises(M.MoeError):
        M.probe_mfma(3, 256, 2, sink, cycles)
