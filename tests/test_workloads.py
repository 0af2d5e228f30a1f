"""The seeded generator: layout invariants of the paged pool, traps, determinism, and the
byte model against the pages' own arithmetic."""
import json
import math
import os

import pytest
import torch

import workloads
from workloads import BLOCK_SIZE

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _small(paged=True, levels=(((70, 0, 5),),), lo=1, hi=40, dtype="bf16"):
    return workloads.custom("small", B=5, Hq=4, Hkv=2, d=16, dtype=dtype, levels=levels,
                            suffix_lo=lo, suffix_hi=hi, paged=paged)


@pytest.mark.parametrize("paged", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_pool_holds_logical_suffix(paged, dtype):
    step = workloads.generate(_small(paged, dtype=dtype), seed=4)
    tbl = step.block_table
    for b in range(step.cfg.B):
        k, v = step.suffix(b)
        s = int(step.seq_lens[b])
        assert k.shape[0] == s
        for t in range(s):
            blk = int(tbl[b, t // BLOCK_SIZE])
            assert torch.equal(step.k_pool[blk, t % BLOCK_SIZE], k[t])
            assert torch.equal(step.v_pool[blk, t % BLOCK_SIZE], v[t])
        if s % BLOCK_SIZE:
            blk = int(tbl[b, s // BLOCK_SIZE])
            assert torch.all(step.k_pool[blk, s % BLOCK_SIZE:].float() == workloads.TAIL_K)
            assert torch.all(step.v_pool[blk, s % BLOCK_SIZE:].float() == workloads.TAIL_V)


def test_unreferenced_blocks_are_nan_and_blocks_unique():
    step = workloads.generate(_small(True), seed=5)
    used = set()
    for b in range(step.cfg.B):
        nb = -(-int(step.seq_lens[b]) // BLOCK_SIZE)
        ids = [int(x) for x in step.block_table[b, :nb]]
        assert not used.intersection(ids), "a block is owned by two sequences"
        used.update(ids)
    for b in range(step.cfg.B):                    # table padding points at a trap block
        nb = -(-int(step.seq_lens[b]) // BLOCK_SIZE)
        for j in range(nb, step.cfg.max_blocks):
            assert int(step.block_table[b, j]) not in used
    spare = [i for i in range(step.num_blocks) if i not in used]
    assert spare, "need at least one spare block"
    for i in spare:
        assert torch.isnan(step.k_pool[i].float()).all() and torch.isnan(step.v_pool[i].float()).all()
    assert step.num_blocks >= len(used) * (1 + workloads.SPARE_FRACTION) - 1


def test_determinism_and_seed_dependence():
    cfg = _small(True, levels=(((30, 0, 5),), ((7, 0, 2), (9, 2, 5))))
    a = workloads.generate(cfg, seed=9).digest()
    b = workloads.generate(cfg, seed=9).digest()
    c = workloads.generate(cfg, seed=10).digest()
    assert a == b and a != c


def test_seq_lens_drawn_inclusive_range():
    cfg = workloads.custom("r", B=400, Hq=1, Hkv=1, d=8, dtype="bf16", levels=(((4, 0, 400),),),
                           suffix_lo=3, suffix_hi=6)
    lens = workloads.generate(cfg, seed=1).seq_lens
    assert int(lens.min()) == 3 and int(lens.max()) == 6


def test_seq_lens_override_and_empty():
    cfg = _small(True)
    step = workloads.generate(cfg, seed=2, seq_lens=[0, 1, 16, 17, 40])
    assert step.seq_lens.tolist() == [0, 1, 16, 17, 40]
    assert step.suffix(0)[0].shape[0] == 0


def test_scale_is_float32_of_inverse_sqrt():
    assert workloads.scale_for(128) == float(torch.tensor(1 / math.sqrt(128), dtype=torch.float32))
    assert workloads.scale_for(64) == 0.125


def test_config_shapes():
    cfgs = {c.name: c for c in workloads.all_configs()}
    assert set(cfgs) == {"tiny_f32", "llama3_8b_gqa", "codellama13b_mha_p16384",
                         "docqa_codellama7b", "two_level_gqa"}
    t = cfgs["two_level_gqa"]
    assert len(t.levels) == 2 and len(t.levels[1]) == 8 and t.G == 4
    assert [n[1] for n in t.levels[1]] == list(range(0, 256, 32))
    assert cfgs["docqa_codellama7b"].max_blocks == 32


def test_kv_bytes_against_pages():
    with open(os.path.join(GOLDEN, "kv_bytes.json")) as f:
        cases = json.load(f)["cases"]
    blog, hyd = cases
    per_tok = workloads.kv_bytes_per_token(blog["Hkv"], blog["d"], blog["esize"], blog["layers"])
    assert per_tok == blog["bytes_per_token"]
    assert per_tok * blog["prefix_tokens"] == blog["prefix_bytes"]
    elems = hyd["tokens"] * hyd["Hkv"] * hyd["d"]
    assert elems == hyd["elements"]
    assert abs(elems * 2 - hyd["half_precision_bytes_approx"]) / hyd["half_precision_bytes_approx"] < 0.05


def test_algorithmic_bytes_headline():
    cfg = workloads.codellama13b_mha(16384)
    lens = [64] * 256
    ab = workloads.algorithmic_bytes(cfg, lens)
    assert ab["prefix"] == 16384 * 40 * 128 * 2 * 2
    assert ab["suffix"] == 256 * 64 * 40 * 128 * 2 * 2
    assert ab["q"] == 256 * 40 * 128 * 2
    assert ab["out"] == 256 * 40 * 128 * 4 + 256 * 40 * 4
    assert workloads.prefix_flops(cfg) == 4 * 256 * 40 * 16384 * 128
