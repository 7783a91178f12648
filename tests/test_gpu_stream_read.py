"""The bare read the bench sets beside each HBM-bound point (a measurement
aid, not a step of the decode path) reads every byte of its buffer once: the
XOR of the per-thread words it leaves equals the XOR of the buffer's 32-bit
words, at work-group counts below, at and above the number of 16 KiB tiles."""
import numpy as np
import pytest
import torch

from paged_attention_fp8_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("tiles", [0, 1, 7, 300])
@pytest.mark.parametrize("work_groups", [1, 3, 256, 1000])
def test_stream_read_reads_every_word(tiles, work_groups):
    print(f"stream_read: tiles={tiles} work_groups={work_groups}", flush=True)
    g = np.random.default_rng(1000 * tiles + work_groups)
    words = g.integers(0, 2**32, tiles * ops.STREAM_READ_TILE // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(DEV)
    sink = torch.full((work_groups * ops.STREAM_READ_THREADS + 5,), 7, dtype=torch.int32, device=DEV)
    ops.stream_read(buf, work_groups, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(words) if words.size else np.uint32(0)
    assert np.bitwise_xor.reduce(got[:work_groups * ops.STREAM_READ_THREADS]) == want
    assert (got[work_groups * ops.STREAM_READ_THREADS:] == 7).all()      # nothing past the sink's range


def test_stream_read_errors():
    buf = torch.zeros(ops.STREAM_READ_TILE + 4, dtype=torch.uint8, device=DEV)
    with pytest.raises(ops.Pafp8Error, match="16384"):
        ops.stream_read(buf, 4)
