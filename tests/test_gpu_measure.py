"""The streaming-read measurement kernel (qsa_stream_read) reads exactly the
bytes it is asked to: each workgroup's XOR checksum equals a CPU XOR of its
share of the footprint, wrap-around included."""
import numpy as np
import pytest
import torch

import top_sparse_attention_amd as qsa

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("footprint,per_wg,wgs", [(240 << 10, 48 << 10, 11),
                                                  (4096, 4096, 3), (1 << 20, 16, 70),
                                                  (96 << 10, 80 << 10, 5)])
def test_stream_read_checksums(footprint, per_wg, wgs):
    rng = np.random.Generator(np.random.PCG64(footprint + wgs))
    host = rng.integers(0, 2**32, size=(footprint + 4096) // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV).view(torch.uint8)
    sink = qsa.stream_read(buf, footprint, per_wg, wgs)
    torch.cuda.synchronize()
    words = host[: footprint // 4]
    n, m = footprint // 4, per_wg // 4
    want = []
    for w in range(wgs):
        start = (w * m) % n
        idx = (start + np.arange(m)) % n
        want.append(np.bitwise_xor.reduce(words[idx]))
    got = sink.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, np.array(want, dtype=np.uint32))
