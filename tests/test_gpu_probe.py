"""The streaming-read measurement aid (w12_read_probe) reads every byte: a
zero buffer with one word set to the probe's marker value makes the xor of
all words equal the marker, and only then is the sink written -- wherever
the word sits and whatever the buffer size."""
import pytest
import torch

from lossless_bit_weight_amd import w12

MARK = 0x9E3779B9

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1000 * 16, (1 << 20) + 48, 55375872, 270061568])
def test_probe_reads_every_word(nbytes):
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    n = nbytes // 4
    for pos in sorted({0, n // 3, n // 2 + 1, n - 1}):
        print("probe %d bytes, marker at word %d" % (nbytes, pos), flush=True)
        buf.zero_()
        sink.zero_()
        buf[pos] = MARK - (1 << 32)          # the same 32 bits as an int32
        w12.w12_read_probe(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) & 0xFFFFFFFF == MARK, (nbytes, pos)
    buf.zero_()
    sink.zero_()
    w12.w12_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
