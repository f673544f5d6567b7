"""GPU: the streaming-read reference kernel (w4ec_stream_read) reads every
byte it is given: each workgroup's word is the XOR of the 32-bit words of
its share of the 16-byte chunks (workgroup w: chunks [w c, (w + 1) c), c =
ceil(chunks / 512)), checked against numpy on ragged buffers."""
import numpy as np
import pytest

import w4_gemm_error_amd as w4

from gpu_util import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, (3 << 20) + 16 * 777])
def test_stream_read_visits_every_chunk(nbytes):
    print(f"stream read {nbytes} bytes", flush=True)
    t = torch()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = t.from_numpy(host.view(np.int32).copy()).cuda()
    sink = t.full((512,), -1, dtype=t.int32, device="cuda")
    w4.w4ec_stream_read(src, sink)
    t.cuda.synchronize()
    words = host.reshape(-1, 4)
    c = -(-words.shape[0] // 512)
    wg = np.arange(words.shape[0]) // c
    want = np.zeros(512, dtype=np.uint32)
    per_chunk = np.bitwise_xor.reduce(words, axis=1)
    np.bitwise_xor.at(want, wg, per_chunk)
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want)
