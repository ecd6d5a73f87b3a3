"""GPU check of the streaming-read measuring kernel: it reads every word of
the buffer once (the XOR of its per-wavefront words equals the XOR of the
buffer), whatever the grid.  Needs an MI355X and libpagedkv.so."""
import numpy as np
import pytest
import torch

from paged_kv_cache_97_amd import ops

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,sink_len", [(16, 4), (4096 + 48, 4), (64 * 2**20 + 16 * 7, 8192),
                                             (3 * 2**20, 262144)])
def test_stream_read_touches_every_word_once(nbytes, sink_len):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(sink_len, dtype=torch.int32, device="cuda")
    ops.stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
