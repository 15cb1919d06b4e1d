"""The streaming-read measurement helper on the GPU: every byte is read (the
XOR of all 32-bit words comes back exactly) for a buffer of one 16-byte
chunk, one below a workgroup's 16 KB step, one whose last workgroup range
holds a single chunk (1 MiB + 16: 65 ranges), and one of 821 ranges of
80 KB with a two-chunk last range (on 256 compute units)."""
import numpy as np
import pytest
import torch

import kv_cache_decode_attn_amd as K

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16, (64 << 20) + 4096 * 16 + 32])
def test_stream_read_xors_every_word(nbytes):
    g = torch.Generator().manual_seed(nbytes)
    words = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int64, generator=g).to(torch.int32)
    want = np.bitwise_xor.reduce(words.numpy().view(np.uint32))
    x = words.to("cuda")
    sink = K.stream_read(x)
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
    # the sink accumulates: a second pass cancels the first
    K.stream_read(x, sink)
    assert int(sink.cpu()[0]) == 0
