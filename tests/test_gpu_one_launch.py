"""GPU parity of the cascade step with both passes in one launch (hp_cascade_step_overlap
mode 3, and mode 1 where the plan picks it): the prefix pass's workgroups and suffix
workgroups of the same shape share one kernel, each suffix wave walking its own units
as a stream of 16-token blocks, then one merge.  Results against the fp64 oracle
(tolerances in gpu_util.TOL) for one, two and four query heads per KV head, both block
layouts, empty and block-edge suffixes, NaN rows for bad metadata, graph replays with
suffix lengths changed between them, and run-to-run identity."""
import numpy as np
import pytest
import torch

import decode_attention_shared_amd as hp
import oracle
import workloads
from gpu_util import DEV, compare, dev_step, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X (no GPU visible)")


# Shapes the one-launch plan takes: 129 or more stacked query rows per KV head (the
# prefix pass's 256-row kernel), d = 128, 16-bit, K/V within the last-level cache.
ONE = [
    workloads.custom("gqa4_b64", B=64, Hq=32, Hkv=8, d=128, dtype="bf16",
                     levels=(((1000, 0, 64),),), suffix_lo=1, suffix_hi=256),
    workloads.custom("gqa2_b96", B=96, Hq=16, Hkv=8, d=128, dtype="f16",
                     levels=(((700, 0, 96),),), suffix_lo=1, suffix_hi=200),
    workloads.custom("mha_b160", B=160, Hq=8, Hkv=8, d=128, dtype="f16",
                     levels=(((900, 0, 160),),), suffix_lo=0, suffix_hi=130),
]


def _call(ds, scale, layout="NHD", mode=3):
    return hp.CascadeCall(ds["q"], ds["levels"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                          ds["seq_lens"], scale, overlap=mode, kv_layout=layout)


@pytest.mark.parametrize("cfg", ONE, ids=lambda c: c.name)
@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("seed", [0, 1])
def test_one_launch_matches_oracle(cfg, layout, seed):
    say(f"one launch {cfg.name} {layout} seed {seed}")
    step = workloads.generate(cfg, seed=seed)
    ds = dev_step(step, kv_layout=layout)
    call = _call(ds, step.scale, layout)
    assert call.one_launch, "mode 3 must put both passes in one launch for this shape"
    out, lse = call()
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "all")
    compare(out, lse, ref_o, ref_l, cfg.dtype, f"one launch {cfg.name} {layout}")


def test_one_launch_block_edges_and_empty_suffixes():
    """Suffix lengths 0, 1, 15, 16, 17, 31, 32, 33 and the table's capacity."""
    cfg = ONE[2]
    edges = [0, 1, 15, 16, 17, 31, 32, 33, cfg.max_blocks * 16]
    lens = [edges[b % len(edges)] for b in range(cfg.B)]
    step = workloads.generate(cfg, seed=5, seq_lens=lens)
    ds = dev_step(step, kv_layout="HND")
    out, lse = _call(ds, step.scale, "HND")()
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "all")
    compare(out, lse, ref_o, ref_l, cfg.dtype, "one launch, block-edge suffixes")


def test_one_launch_bad_metadata_gives_nan_rows_only():
    cfg = ONE[0]
    step = workloads.generate(cfg, seed=8)
    ds = dev_step(step)
    ds["block_table"][3, 0] = step.num_blocks
    ds["block_table"][5, 0] = -1
    ds["seq_lens"][9] = cfg.max_blocks * 16 + 1
    call = _call(ds, step.scale)
    assert call.one_launch
    out, lse = call()
    torch.cuda.synchronize()
    bad = [3, 5, 9]
    assert torch.isnan(out[bad]).all() and torch.isnan(lse[bad]).all()
    good = [b for b in range(cfg.B) if b not in bad]
    rows = np.array([b * cfg.Hq + h for b in good for h in range(cfg.Hq)])
    ref_o, ref_l = oracle.step_attention(step, "all", rows=rows)
    compare(out, lse, ref_o, ref_l, cfg.dtype, "one launch good rows", rows=rows)


def test_one_launch_graph_replay_follows_lengths():
    """Captured into a HIP graph: every replay equals an eager step on the same inputs,
    with eager work between replays, also after the suffix lengths change on the device."""
    cfg = ONE[1]
    step = workloads.generate(cfg, seed=11)
    ds = dev_step(step)
    call = _call(ds, step.scale)
    assert call.one_launch
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(stream=s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        g.capture_begin()
        call(stream=s)
        g.capture_end()
    torch.cuda.synchronize()
    for rep in range(4):
        if rep == 2:  # shorter suffixes from here on
            ds["seq_lens"].copy_(torch.clamp(ds["seq_lens"] - 37, min=0))
        call()
        torch.cuda.synchronize()
        eager_o, eager_l = call.out.clone(), call.lse.clone()
        call.out.fill_(3.0)
        call.lse.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.out, eager_o) and torch.equal(call.lse, eager_l), f"replay {rep}"
    # the last replay against the oracle on the shortened suffixes (the pool is unchanged,
    # so each suffix is its first seq_lens[b] tokens)
    lens = ds["seq_lens"].cpu().tolist()
    segs = [[(nd.k, nd.v) for nd in step.nodes_of(b)] +
            [tuple(t[:lens[b]] for t in step.suffix(b))] for b in range(cfg.B)]
    ref_o, ref_l = oracle.attention(step.q, segs, cfg.Hkv, step.scale)
    compare(call.out, call.lse, ref_o, ref_l, cfg.dtype, "one launch replay, shorter suffixes")


def test_one_launch_deterministic():
    cfg = ONE[0]
    step = workloads.generate(cfg, seed=2)
    ds = dev_step(step, kv_layout="HND")
    call = _call(ds, step.scale, "HND")
    o1, l1 = [t.clone() for t in call()]
    o2, l2 = call()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_auto_policy_takes_one_launch_for_small_steps():
    """Mode 1 (the default) puts both passes in one launch for a small MHA step, keeps a
    small GQA step serial and keeps the second stream for a large MHA one."""
    small = workloads.generate(ONE[2], seed=0)
    ds = dev_step(small)
    assert _call(ds, small.scale, mode=1).one_launch
    gqa = workloads.generate(ONE[0], seed=0)
    ds = dev_step(gqa)
    assert not _call(ds, gqa.scale, mode=1).concurrent
    big = workloads.custom("mha_big", B=256, Hq=40, Hkv=40, d=128, dtype="f16",
                           levels=(((8192, 0, 256),),), suffix_lo=1, suffix_hi=128)
    q = torch.zeros(256, 40, 128, dtype=torch.float16, device=DEV)
    kv = torch.zeros(8192, 40, 128, dtype=torch.float16, device=DEV)
    pool = torch.zeros(256 * 8 + 1, 16, 40, 128, dtype=torch.float16, device=DEV)
    table = torch.arange(256 * 8, dtype=torch.int32, device=DEV).view(256, 8)
    lens = torch.full((256,), 100, dtype=torch.int32, device=DEV)
    call = hp.CascadeCall(q, [[(kv, kv, 0, 256)]], pool, pool, table, lens, 0.088, overlap=1)
    assert call.concurrent and not call.one_launch, big.name


NEG = -16384.0  # exact in bf16 and fp16; scale * NEG underflows exp to exactly 0


@pytest.mark.parametrize("shape", [(160, 8, 8, "f16"), (64, 16, 4, "bf16")],
                         ids=["G1", "G4"])
def test_one_launch_needles_every_position(shape):
    """Every logical suffix position found exactly by the one-launch suffix waves (their
    step tables walk the block table in items of 4 blocks): one needle key per (sequence,
    KV head) scores 0 and every other key, prefix included, scores far below, so the
    output is the needle's value row exactly and the LSE exactly 0."""
    B, Hq, Hkv, dt = shape
    cfg = workloads.custom(f"needle_one_{Hq // Hkv}", B=B, Hq=Hq, Hkv=Hkv, d=128, dtype=dt,
                           levels=(((600, 0, B),),), suffix_lo=1, suffix_hi=70)
    step = workloads.generate(cfg, seed=21)
    ds = dev_step(step)
    ds["q"].zero_()
    ds["q"][:, :, 0] = 1.0
    pk = ds["k_pool"]
    for lvl in ds["levels"]:
        for (k, v, _, _) in lvl:
            k[:, :, 0] = NEG
    lens = step.seq_lens.tolist()
    tbl = step.block_table
    valid = torch.zeros(pk.shape[:3], dtype=torch.bool)
    for b in range(B):
        for t in range(lens[b]):
            valid[int(tbl[b, t // 16]), t % 16, :] = True
    pk[..., 0][valid.to(DEV)] = NEG
    call = _call(ds, step.scale)
    assert call.one_launch
    suf_v = step.suf_v.float()
    offs = step.suf_offsets.tolist()
    G = Hq // Hkv
    for r in range(max(lens)):
        blks, slots, heads, want_rows = [], [], [], []
        for b in range(B):
            for g in range(Hkv):
                t = (r + 3 * g) % lens[b]
                blks.append(int(tbl[b, t // 16]))
                slots.append(t % 16)
                heads.append(g)
                want_rows.append(suf_v[offs[b] + t, g])
        idx = (torch.tensor(blks, device=DEV), torch.tensor(slots, device=DEV),
               torch.tensor(heads, device=DEV))
        pk[idx + (0,)] = 0.0
        out, lse = call()
        got = out.cpu()
        want = torch.stack(want_rows).view(B, Hkv, 1, 128).expand(B, Hkv, G, 128).reshape(
            B, Hq, 128)
        assert torch.equal(got, want), f"needle run {r}: wrong key picked"
        assert torch.all(lse.cpu() == 0.0), f"needle run {r}: LSE must be exactly 0"
        pk[idx + (0,)] = NEG
    say(f"  one-launch suffix needles (G = {G}): {max(lens)} runs")
