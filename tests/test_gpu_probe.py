"""The bandwidth probe (sk_stream_read) reads every byte it is given: the
XOR of its per-workgroup checksums equals the XOR of all 32-bit words of the buffer,
computed on the host. Sizes cover an empty buffer, less than one wave, a ragged tail
past the four-loads-per-lane loop and a multi-GiB buffer."""

import numpy as np
import pytest
import torch

from tests.helpers import requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


# 32 KiB rounds per workgroup of 256: a partial round, one workgroup's range plus a ragged
# tail, ranges of several rounds that end mid-round, and an exact multiple
@pytest.mark.parametrize("nbytes", [0, 16, 1008, 16 * (2048 * 3 + 777), 16 * (256 * 2048 * 5 + 12345),
                                    16 * 256 * 2048 * 4])
def test_stream_read_checksum(nbytes):
    from sparse_kv_recall_amd import ops
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence([950, nbytes])))
    words = gen.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    data = torch.as_tensor(words.view(np.int32), device="cuda")
    sink = ops.stream_read(data)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(words) if nbytes else np.uint32(0)
    assert int(got) == int(want)


def test_stream_read_large_buffer():
    """Just over 4 GiB (64-bit offsets), random words made on the device."""
    from sparse_kv_recall_amd import ops
    n = (1 << 30) + 12
    g = torch.Generator(device="cuda")
    g.manual_seed(951)
    data = torch.randint(-(1 << 31), (1 << 31) - 1, (n,), dtype=torch.int32, device="cuda", generator=g)
    sink = ops.stream_read(data)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    want = int(np.bitwise_xor.reduce(data.cpu().numpy().view(np.uint32)))
    assert got == want
