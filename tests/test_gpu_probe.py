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
