"""GPU check of the streaming-read ceiling kernel (fp8_stream_read, through the
C ABI): the rate it reports is only a ceiling if every byte is really read.
The kernel folds each thread's loads into one 32-bit value and stores it only
when it equals 0x9E3779B9 (the header's contract), so a zero buffer holding
that word in one 16-byte element must leave exactly that value in the sink,
wherever the element is -- the first and last element, the first element
after every workgroup's share boundary, random elements -- for every grid
size and both load kinds; an all-zero buffer must leave the sink untouched."""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_quantize_amd as fp8
from tests._gpu import DEV, log

pytestmark = pytest.mark.gpu

MAGIC = np.array([0x9E3779B9], dtype=np.uint32).view(np.int32)[0]
THREADS, UNROLL = 256, 8          # the kernel's block size and loads per thread per round


def _shares(n16, workgroups):
    """First 16-byte element of each workgroup's share (the launcher's split:
    equal shares rounded up to whole rounds of the block)."""
    rnd = THREADS * UNROLL
    per = -(-n16 // workgroups)
    per = -(-per // rnd) * rnd
    return list(range(0, n16, per))


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 7, 24 << 20])
@pytest.mark.parametrize("workgroups", [1, 7, 256, 2048])
@pytest.mark.parametrize("nontemporal", [False, True])
def test_every_element_is_read(nbytes, workgroups, nontemporal):
    n16 = nbytes // 16
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    fp8.fp8_stream_read(buf, workgroups=workgroups, nontemporal=nontemporal, sink=sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0, "sink written for an all-zero buffer"
    rng = np.random.default_rng(n16 + workgroups)
    pos = {0, n16 - 1}
    for s in _shares(n16, workgroups):
        pos.update({s, max(0, s - 1)})
    pos.update(int(p) for p in rng.integers(0, n16, 8))
    log(f"stream_read bytes={nbytes} workgroups={workgroups} nt={nontemporal}: {len(pos)} positions")
    for p in sorted(pos):
        buf[4 * p] = int(MAGIC)
        sink.zero_()
        fp8.fp8_stream_read(buf, workgroups=workgroups, nontemporal=nontemporal, sink=sink)
        torch.cuda.synchronize()
        assert int(sink.item()) == int(MAGIC), f"element {p} of {n16} not read"
        buf[4 * p] = 0
