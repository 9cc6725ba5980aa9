"""The HBM probes beside the decode kernels (include/fd_probe.h): the copy
moves exactly the bytes it is given; the row probe, in every pattern, runs
over whole and ragged chunks and only reads; the streaming read folds every
16-byte unit into its work-group's sink value exactly once."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SENTINEL = -12345.0


@pytest.mark.parametrize("nbytes", [16, 48, 4096 + 16, (1 << 20) + 16 * 7])
def test_copy_moves_exact_bytes(fd, nbytes):
    dev = torch.device("cuda", 0)
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).to(dev)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device=dev)
    fd.fd_probe_copy(dst[:nbytes], src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].count_nonzero()) == 0  # nothing past the end


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("rows,chunk", [(2048, 128), (1000, 64), (4096, 512), (37, 16)])
def test_row_probes_only_read(fd, mode, rows, chunk):
    """Modes: 0 head rows, 1 head columns (8 KB blocks), 2 head rows from
    rotated starts (chunks of 128 and 512 rows are whole multiples of the
    eight waves' 4-row stages; 1000 and 37 rows leave a ragged last chunk)."""
    dev = torch.device("cuda", 0)
    row_bytes = 8192
    g = torch.Generator(device="cpu").manual_seed(rows * 10 + mode)
    a = torch.randint(-1000, 1000, (rows, row_bytes // 2), dtype=torch.int16, generator=g).to(dev)
    b = torch.randint(-1000, 1000, (rows, row_bytes // 2), dtype=torch.int16, generator=g).to(dev)
    a0, b0 = a.clone(), b.clone()
    sink = torch.full((fd.PROBE_SINK_FLOATS,), SENTINEL, dtype=torch.float32, device=dev)
    fd.fd_probe_read_rows(a, b, row_bytes, chunk, mode, sink)
    torch.cuda.synchronize()
    assert torch.equal(a, a0) and torch.equal(b, b0)
    # the row probe stores to the sink only for a data pattern these inputs do not make
    assert bool((sink == SENTINEL).all())


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, (3 << 20) + 16 * 5])
def test_stream_probe_reads_every_word_once(fd, nbytes):
    """Work-group w of the streaming read covers 16-byte units [w p, (w + 1) p)
    (p = ceil(units / work-groups)) and writes the XOR of their 32-bit words,
    low 16 bits, to sink[w]: recomputed here on the CPU, so a unit skipped or
    read twice shows."""
    dev = torch.device("cuda", 0)
    g = np.random.default_rng(nbytes)
    words = g.integers(0, 1 << 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32).copy()).to(dev)
    sink = torch.full((fd.PROBE_SINK_FLOATS,), SENTINEL, dtype=torch.float32, device=dev)
    fd.fd_probe_read(src, sink)
    torch.cuda.synchronize()
    units = nbytes // 16
    per = -(-units // fd.PROBE_SINK_FLOATS)
    want = np.zeros(fd.PROBE_SINK_FLOATS, dtype=np.float64)
    u = words.reshape(units, 4)
    for w in range(fd.PROBE_SINK_FLOATS):
        lo, hi = w * per, min((w + 1) * per, units)
        if lo < hi:
            want[w] = float(np.bitwise_xor.reduce(u[lo:hi].ravel()) & 0xFFFF)
    assert np.array_equal(sink.double().cpu().numpy(), want)
