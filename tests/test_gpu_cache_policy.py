"""GPU: the cache policy of the K/V loads never changes a result.

The paged suffix pass marks its K/V loads non-temporal when the footprint its
block tables can reach (or the pool, if smaller) reaches the 256 MiB last-level
cache.  The same step gathered once from a large pool (non-temporal loads) and
once from a compact copy of the referenced blocks (ordinary loads) must give
bit-identical outputs, and both must match the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import decode_attention_shared_amd as hp
import oracle
from gpu_util import DEV, compare, say

pytestmark = pytest.mark.gpu

BLOCK = 16
LLC_BYTES = 256 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X (no GPU visible)")
    hp.lib()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_suffix_loads_policy_does_not_change_results(dtype):
    B, Hq, Hkv, d = 4, 16, 8, 128
    big_blocks, wide = 4200, 1100  # footprint min(4200, 4 * 1100) blocks of 64 KiB: 275 MB
    block_bytes = BLOCK * Hkv * d * 2 * 2
    assert min(big_blocks, B * wide) * block_bytes >= LLC_BYTES
    g = torch.Generator().manual_seed(7)
    lens = torch.randint(20, 97, (B,), generator=g, dtype=torch.int32)
    nblk = [(int(n) + BLOCK - 1) // BLOCK for n in lens]
    ids = torch.randperm(big_blocks, generator=g)[: sum(nblk)].to(torch.int32)
    say(f"cache policy {dtype}: pool {big_blocks} blocks, lens {lens.tolist()}")

    gd = torch.Generator(device=DEV).manual_seed(11)
    k_big = torch.randn(big_blocks, BLOCK, Hkv, d, generator=gd, device=DEV).to(dtype)
    v_big = torch.randn(big_blocks, BLOCK, Hkv, d, generator=gd, device=DEV).to(dtype)
    q = torch.randn(B, Hq, d, generator=gd, device=DEV).to(dtype)

    table_big = torch.zeros(B, wide, dtype=torch.int32)
    table_small = torch.zeros(B, max(nblk), dtype=torch.int32)
    pos = 0
    for b in range(B):
        table_big[b, : nblk[b]] = ids[pos: pos + nblk[b]]
        table_small[b, : nblk[b]] = torch.arange(pos, pos + nblk[b], dtype=torch.int32)
        pos += nblk[b]
    idx = ids.to(DEV, torch.int64)
    k_small = k_big.index_select(0, idx).contiguous()
    v_small = v_big.index_select(0, idx).contiguous()
    assert min(k_small.shape[0], B * table_small.shape[1]) * block_bytes < LLC_BYTES
    lens_d = lens.to(DEV)

    scale = 1.0 / np.sqrt(d)
    o_nt, l_nt = hp.suffix_decode(q, k_big, v_big, table_big.to(DEV), lens_d, scale)
    o_c, l_c = hp.suffix_decode(q, k_small, v_small, table_small.to(DEV), lens_d, scale)
    torch.cuda.synchronize()
    assert torch.equal(o_nt, o_c) and torch.equal(l_nt, l_c)

    # against the oracle: each sequence's keys in order, from the compact pool
    kc = k_small.cpu()
    vc = v_small.cpu()
    segs = []
    pos = 0
    for b in range(B):
        n = int(lens[b])
        kb = kc[pos: pos + nblk[b]].reshape(-1, Hkv, d)[:n]
        vb = vc[pos: pos + nblk[b]].reshape(-1, Hkv, d)[:n]
        segs.append([(kb, vb)])
        pos += nblk[b]
    o_ref, l_ref = oracle.attention(q.cpu(), segs, Hkv, scale)
    compare(o_nt, l_nt, o_ref, l_ref, "bf16" if dtype == torch.bfloat16 else "f16",
            "suffix, non-temporal loads")
