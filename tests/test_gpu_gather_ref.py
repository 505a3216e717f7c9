"""The read-only gather reference (a measurement tool of bench.py): it reads
exactly the rows it is given, and clamps out-of-range indices to the last row.
The XOR of all its per-thread words must equal the XOR of every 32-bit word of
the rows read, computed on the host."""

import numpy as np
import pytest

import gpu_setup as gs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 7, 5000, 300001])
def test_gather_read_reference_reads_the_given_rows(n):
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    rng = np.random.default_rng(n)
    num_rows = 4096
    rows = rng.integers(0, 256, size=(num_rows, 768), dtype=np.uint8)
    idx = rng.integers(-3, num_rows + 3, size=n).astype(np.int32)       # a few out of range
    gs.say(f"gather reference n={n}")
    sink = torch.zeros(B.OSCAR_GATHER_REF_SINK_WORDS, dtype=torch.int32, device="cuda")
    B.oscar_gather_read_reference(gs.dev(rows), gs.dev(idx), sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    clamped = np.minimum(idx.astype(np.int64) & 0xFFFFFFFF, num_rows - 1)
    row_xor = np.bitwise_xor.reduce(rows.view(np.uint32), axis=1)
    want = np.bitwise_xor.reduce(row_xor[clamped])
    assert got == want
