"""The bare streams the bench sets beside each HBM-bound point (measurement
aids, not steps of the decode path).  The read touches every byte of its
buffer once: the XOR of the per-thread words it leaves equals the XOR of the
buffer's 32-bit words.  The read-write writes every byte of its output from
the words its layout names.  Both at work-group counts below, at and above
the number of 16 KiB tiles."""
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


@pytest.mark.parametrize("ratio", [1, 2, 4])
@pytest.mark.parametrize("tiles,work_groups", [(1, 1), (7, 3), (300, 256), (5, 1000)])
def test_stream_read_write_layout(ratio, tiles, work_groups):
    print(f"stream_read_write: R={ratio} tiles={tiles} work_groups={work_groups}", flush=True)
    g = np.random.default_rng(100 * tiles + 10 * ratio + work_groups)
    src = g.integers(0, 256, tiles * ops.STREAM_READ_TILE, dtype=np.uint8)
    out = torch.full((tiles * ops.STREAM_READ_TILE // ratio + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    ops.stream_read_write(torch.from_numpy(src).to(DEV), out[:-64], work_groups)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # tile t, store k, lane l, 16 bytes = XOR over q < R of load kR + q
    want = np.bitwise_xor.reduce(src.reshape(tiles, 16 // ratio, ratio, 64, 16), axis=2).reshape(-1)
    assert np.array_equal(got[:-64], want)
    assert (got[-64:] == 0xA5).all()        # nothing past dst
