"""GPU check of the measurement entry point tq_stream_read: the per-workgroup words it writes
fold back to the XOR of every 32-bit word of the buffer (so every byte was read)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 64 << 20])
def test_stream_read_covers_the_buffer(nbytes):
    import compressed_key_attention_amd as tq
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    buf = host.cuda()
    n = 64 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(n, dtype=torch.int32, device="cuda")
    tq.stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


def test_stream_read_rejects_a_small_sink():
    import compressed_key_attention_amd as tq
    buf = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(tq.TqError):
        tq.stream_read(buf, sink)
