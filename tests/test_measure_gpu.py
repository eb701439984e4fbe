"""The streaming references (include/w4a16_measure.h) read and copy exactly the bytes
they are given: the read's per-workgroup XORs against NumPy's, the copy byte for byte
with canaries past the end."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    import w4a16_int4_weight_amd as mod
    return mod


@pytest.mark.parametrize("nbytes", [16, 32768, 32768 + 48, (1 << 20) + 4096 + 16, 14_194_688, (80 << 20) + 48])
def test_stream_read_xors_every_chunk(w, nbytes):
    rng = np.random.default_rng(nbytes % 1000)
    host = rng.integers(0, 2**32, size=nbytes // 4 + 64, dtype=np.uint32)   # extra words past the end
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = w.w4a16_stream_read(src, nbytes)
    torch.cuda.synchronize()
    chunks = host[:nbytes // 4].reshape(-1, 4)
    C = chunks.shape[0]
    blocks = w.w4a16_stream_sink_bytes(nbytes) // 16
    want = np.stack([np.bitwise_xor.reduce(chunks[b * C // blocks:(b + 1) * C // blocks], axis=0)
                     if (b + 1) * C // blocks > b * C // blocks else np.zeros(4, np.uint32) for b in range(blocks)])
    got = sink[:blocks * 16].cpu().numpy().view(np.uint32).reshape(blocks, 4)
    assert np.array_equal(got, want)
    assert np.array_equal(np.bitwise_xor.reduce(got, axis=0), np.bitwise_xor.reduce(chunks, axis=0))


@pytest.mark.parametrize("nbytes", [16, 32768 + 48, (1 << 20) + 4096 + 16])
def test_stream_copy_is_exact_and_in_bounds(w, nbytes):
    rng = np.random.default_rng(7)
    src = torch.from_numpy(rng.integers(0, 256, size=nbytes + 256, dtype=np.uint8)).to(DEV)
    dst = torch.full((nbytes + 256,), 0xA5, dtype=torch.uint8, device=DEV)
    w.w4a16_stream_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert torch.all(dst[nbytes:] == 0xA5)


def test_clock_stamps_bracket_captured_work(w):
    """Two stamps captured around four 64 MiB reads in one graph: later than each other,
    by at least what the reads take at 10 TB/s and at most the events around the replay
    (which also hold the host's graph-launch latency); only dst[index] is written."""
    hz = w.w4a16_wall_clock_hz()
    assert hz > 0
    src = torch.ones(64 << 20, dtype=torch.uint8, device=DEV)
    sink = torch.empty(w.w4a16_stream_sink_bytes(src.numel()), dtype=torch.uint8, device=DEV)
    stamps = torch.full((4,), -1, dtype=torch.int64, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w.w4a16_clock_stamp(stamps, 1)
        for _ in range(4):
            w.w4a16_stream_read(src, sink=sink)
        w.w4a16_clock_stamp(stamps, 2)
    for _ in range(3):
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        v = stamps.cpu().tolist()
        assert v[0] == -1 and v[3] == -1
        span_us = (v[2] - v[1]) * 1e6 / hz
        assert 4 * (64 << 20) / 10e12 * 1e6 <= span_us <= start.elapsed_time(end) * 1e3 + 1.0, span_us
