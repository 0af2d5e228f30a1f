"""The streaming-read probe (a measurement aid): its sink partials XOR to the XOR of
every 32-bit word of the buffer, so every byte was read exactly once."""
import numpy as np
import pytest
import torch

import decode_attention_shared_amd as hp
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, (1 << 20) + 16, 64 << 20])
def test_read_probe_reads_every_word_once(nbytes):
    say(f"read probe {nbytes} bytes")
    g = torch.Generator().manual_seed(nbytes)
    words = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int64)
    host = words.to(torch.int32)
    buf = host.to(DEV)
    sink = torch.full((hp.HP_READ_PROBE_WGS,), 7, dtype=torch.int32, device=DEV)
    hp.read_probe(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32)) if nbytes else np.uint32(0)
    assert got == want
