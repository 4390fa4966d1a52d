"""The streaming-read probe that bench.py times for the GPU's read ceiling:
it must read every 16-byte word of the buffer, whatever the grid.  Each
thread folds the words it reads by XOR and writes the result only when it
equals a marker, so a marker word anywhere in the buffer must come back,
and a buffer without one must leave the output alone."""
import pytest

from test_gpu_parity import announce, pkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MARKER = 0x9E3779B9 - (1 << 32)  # as int32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv().library()
    torch.cuda.set_device(0)


@pytest.mark.parametrize("work_groups", [1, 7, 64, 1000, 4096])
def test_probe_reads_every_word(work_groups):
    m = pkv()
    n = 3 * (1 << 20) + 12  # int32 words: shares that do not divide evenly
    announce(f"stream probe: {n * 4} bytes, {work_groups} work-groups")
    buf = torch.zeros(n, dtype=torch.int32, device="cuda")
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    n16 = n // 4
    per = -(-n16 // work_groups)  # 16-byte words per work-group share
    # both sides of every share boundary (at most 64 of them), the ends and the middle
    edges = [4 * k * per + d for k in range(1, min(work_groups, 64)) if 4 * k * per < n for d in (-1, 0)]
    for pos in [0, n // 2 + 5, n - 1] + edges:
        buf.zero_()
        buf[pos] = MARKER
        out.zero_()
        m.probe_stream_read(buf, out, work_groups)
        torch.cuda.synchronize()
        assert int(out[0]) == MARKER, f"word {pos} not read"
    buf.zero_()
    out.zero_()
    m.probe_stream_read(buf, out, work_groups)
    torch.cuda.synchronize()
    assert int(out[0]) == 0


@pytest.mark.parametrize("tile_bytes,work_groups", [(1024, 1), (1024, 64), (4096, 3), (16384, 1000)])
def test_gather_probe_reads_every_listed_tile(tile_bytes, work_groups):
    # Tiles at shuffled, non-overlapping places of two buffers (even list
    # entries in the first, odd in the second), plus entries the probe must
    # skip (negative, misaligned, reaching past the end): a marker at the
    # first or last word of any listed tile must come back.
    import numpy as np

    m = pkv()
    words = (1 << 20) // 4  # 1 MiB per buffer
    slots = (words * 4) // tile_bytes
    rng = np.random.default_rng(tile_bytes + work_groups)
    n_each = min(slots, 96)
    offs0 = rng.permutation(slots)[:n_each] * tile_bytes
    offs1 = rng.permutation(slots)[:n_each] * tile_bytes
    offs = np.empty(2 * n_each, np.int64)
    offs[0::2], offs[1::2] = offs0, offs1
    bad = np.array([-tile_bytes, 8, words * 4, words * 4 - 16], np.int64)  # skipped
    listed = np.concatenate([offs, bad])
    announce(f"gather probe: {len(listed)} tiles of {tile_bytes} B, {work_groups} work-groups")
    bufs = [torch.zeros(words, dtype=torch.int32, device="cuda") for _ in range(2)]
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    t_offs = torch.from_numpy(listed).cuda()
    for t in range(len(offs)):
        for pos in (offs[t] // 4, (offs[t] + tile_bytes) // 4 - 1):
            b = bufs[t % 2]
            b[pos] = MARKER
            out.zero_()
            m.probe_gather_read(bufs[0], bufs[1], t_offs, tile_bytes, out, work_groups)
            torch.cuda.synchronize()
            assert int(out[0]) == MARKER, f"tile {t} word {pos} not read"
            b[pos] = 0
    out.zero_()
    m.probe_gather_read(bufs[0], bufs[1], t_offs, tile_bytes, out, work_groups)
    torch.cuda.synchronize()
    assert int(out[0]) == 0
