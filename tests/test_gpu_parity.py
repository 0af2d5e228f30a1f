"""GPU parity: every pass of the HIP path against the fp64 oracle, through the C ABI.

Tolerances (written in gpu_util.TOL): fp32 inputs max-abs 1e-5; bf16/fp16 inputs
max-abs 1e-2, mean-abs 1e-3, LSE max-abs 1e-3.  Block-table indexing is checked
bit-exactly with needles (one key scores 0, every other key scores about -1450,
so softmax puts weight exactly 1 on it and O must equal that key's value row).
"""
import ctypes

import numpy as np
import pytest
import torch

import decode_attention_shared_amd as hp
import oracle
import workloads
from gpu_util import DEV, cascade, compare, dev_step, sample_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X (no GPU visible)")
    hp.lib()


def _one_level(name, dtype, d, B, Hq, Hkv, P, b0, b1, lo=1, hi=1, paged=True):
    return workloads.custom(name, B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype,
                            levels=(((P, b0, b1),),), suffix_lo=lo, suffix_hi=hi, paged=paged)


# ------------------------------------------------------------------ prefix pass

PREFIX_CASES = [
    # dtype, d, B, Hq, Hkv, P, seq_begin, seq_end
    ("bf16", 128, 75, 8, 2, 1000, 0, 75),     # 300 rows per KV head: 2 row blocks, key splits
    ("f16", 128, 5, 8, 2, 65, 1, 4),          # 12 rows, a sub-range of sequences, ragged tile
    ("bf16", 64, 12, 4, 1, 2500, 0, 12),      # d=64, 48 rows, many splits
    ("f16", 64, 30, 8, 8, 1, 0, 30),          # a single key
    ("bf16", 128, 32, 4, 4, 64, 0, 32),       # exactly one tile of keys
    ("f16", 128, 100, 1, 1, 3000, 0, 100),    # 100 rows, one head
    ("bf16", 128, 130, 8, 1, 700, 0, 130),    # MQA-like group of 8: 1040 rows, 5 row blocks
    ("f16", 64, 150, 2, 1, 900, 0, 150),      # d=64 in the 256-row kernel: 300 rows, ragged tile
    ("bf16", 64, 140, 1, 1, 1111, 3, 140),    # d=64, 137 rows from sequence 3 on, ragged tile
    ("f32", 64, 4, 1, 1, 512, 0, 4),          # the tiny fp32 shape
    ("f32", 128, 9, 4, 2, 777, 0, 9),         # fp32, d=128, GQA
    ("f32", 64, 70, 2, 1, 300, 5, 70),        # fp32, 130 rows
]


@pytest.mark.parametrize("case", PREFIX_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefix_pass(case):
    dtype, d, B, Hq, Hkv, P, b0, b1 = case
    say(f"prefix {case}")
    step = workloads.generate(_one_level("pfx", dtype, d, B, Hq, Hkv, P, b0, b1), seed=1)
    node = step.levels[0][0]
    q = step.q.to(DEV)
    out = torch.full((B, Hq, d), 7.0, device=DEV)
    lse = torch.full((B, Hq), 7.0, device=DEV)
    hp.prefix_attn(q, node.k.to(DEV), node.v.to(DEV), b0, b1, step.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    rows = np.arange(b0 * Hq, b1 * Hq)
    ref_o, ref_l = oracle.step_attention(step, "prefix", rows=rows)
    compare(out, lse, ref_o, ref_l, dtype, "prefix", rows=rows)
    outside = torch.ones(B, dtype=torch.bool)
    outside[b0:b1] = False
    assert torch.all(out.cpu()[outside] == 7.0) and torch.all(lse.cpu()[outside] == 7.0), \
        "rows outside the node were written"


def test_prefix_empty_node():
    step = workloads.generate(_one_level("e", "bf16", 128, 4, 4, 2, 0, 0, 4), seed=0)
    q = step.q.to(DEV)
    k = torch.zeros(0, 2, 128, dtype=torch.bfloat16, device=DEV)
    out, lse = hp.prefix_attn(q, k, k, 0, 4, step.scale)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == -float("inf"))


# ------------------------------------------------------------------ suffix pass

SUFFIX_CASES = [
    # dtype, d, B, Hq, Hkv, lo, hi
    ("bf16", 128, 40, 32, 8, 1, 300),    # group 4, suffixes split over 3 work items
    ("f16", 128, 20, 40, 40, 1, 128),    # MHA
    ("bf16", 64, 16, 16, 2, 0, 40),      # group 8, d=64, empty suffixes included
    ("f32", 64, 4, 1, 1, 1, 64),         # tiny fp32
    ("f32", 128, 6, 4, 2, 1, 200),       # fp32 group 2 with splits
    ("f16", 64, 33, 2, 1, 16, 17),       # block boundaries
    ("bf16", 128, 8, 8, 4, 300, 512),    # long suffixes, 4 splits
]


@pytest.mark.parametrize("case", SUFFIX_CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("layout", ["NHD", "HND", "contiguous"])
def test_suffix_pass(case, layout):
    """Paged suffixes in both block layouts (token-major NHD, head-major HND), and
    suffixes stored contiguously (an identity block table)."""
    dtype, d, B, Hq, Hkv, lo, hi = case
    paged = layout != "contiguous"
    say(f"suffix {case} layout={layout}")
    step = workloads.generate(_one_level("suf", dtype, d, B, Hq, Hkv, 0, 0, B, lo, hi, paged),
                              seed=2)
    ds = dev_step(step, kv_layout="HND" if layout == "HND" else "NHD")
    out, lse = hp.suffix_decode(ds["q"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                                ds["seq_lens"], step.scale, kv_layout=ds["kv_layout"])
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "suffix")
    compare(out, lse, ref_o, ref_l, dtype, "suffix")


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_suffix_lengths_at_block_edges(layout):
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 127, 128, 129, 255, 256, 300]
    cfg = _one_level("edges", "bf16", 128, len(lens), 8, 2, 0, 0, len(lens), 0, 300)
    step = workloads.generate(cfg, seed=3, seq_lens=lens)
    ds = dev_step(step, kv_layout=layout)
    out, lse = hp.suffix_decode(ds["q"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                                ds["seq_lens"], step.scale, kv_layout=layout)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "suffix")
    compare(out, lse, ref_o, ref_l, "bf16", "suffix edges")
    assert torch.all(out[0] == 0) and torch.all(lse[0] == -float("inf"))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_single_suffix_token_returns_value_exactly(dtype):
    cfg = _one_level("one", dtype, 128, 10, 8, 2, 0, 0, 10, 1, 1)
    step = workloads.generate(cfg, seed=4)
    ds = dev_step(step)
    out, lse = hp.suffix_decode(ds["q"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                                ds["seq_lens"], step.scale)
    torch.cuda.synchronize()
    G = 4
    want = step.suf_v.float().repeat_interleave(G, dim=1)  # [B][Hq][d]: token 0 of each sequence
    assert torch.equal(out.cpu(), want), "one key: O must equal its value row exactly"


# ------------------------------------------------------------------ merge

@pytest.mark.parametrize("n", [1, 2, 3, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_lse_merge(n, d):
    g = torch.Generator().manual_seed(n * 100 + d)
    rows = 1000
    os_ = [torch.randn(rows, d, generator=g) for _ in range(n)]
    ls_ = [torch.randn(rows, generator=g) * 5 for _ in range(n)]
    for i in range(n):                       # some empty partials, and some all-empty rows
        ls_[i][i::7] = -float("inf")
        os_[i][i::7] = 0.0
    for i in range(n):
        ls_[i][::97] = -float("inf")
        os_[i][::97] = 0.0
    out, lse = hp.lse_merge([o.to(DEV) for o in os_], [l.to(DEV) for l in ls_])
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge([o.numpy() for o in os_], [l.numpy() for l in ls_])
    go, gl = out.double().cpu().numpy(), lse.double().cpu().numpy()
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.all(go[~fin] == 0)
    # fp32 arithmetic on fp32 partials: the fp32 tolerance of this path (1e-5)
    assert np.abs(go - ref_o).max() <= 1e-5 * max(1.0, np.abs(ref_o).max())
    assert np.abs(gl[fin] - ref_l[fin]).max() <= 1e-5 * max(1.0, np.abs(ref_l[fin]).max())
    if n == 1:
        assert np.array_equal(go[fin], os_[0].double().numpy()[fin]), "one part passes through"


# ------------------------------------------------------------------ whole step, reduced sizes

REDUCED = [
    workloads.tiny_f32(),
    workloads.custom("llama3_8b_gqa_small", B=16, Hq=32, Hkv=8, d=128, dtype="bf16",
                     levels=(((1000, 0, 16),),), suffix_lo=1, suffix_hi=256),
    workloads.custom("codellama13b_small", B=24, Hq=40, Hkv=40, d=128, dtype="f16",
                     levels=(((1500, 0, 24),),), suffix_lo=1, suffix_hi=128),
    workloads.custom("docqa_small", B=12, Hq=32, Hkv=32, d=128, dtype="bf16",
                     levels=(((2000, 0, 12),),), suffix_lo=64, suffix_hi=512),
    workloads.custom("two_level_small", B=24, Hq=32, Hkv=8, d=128, dtype="bf16",
                     levels=(((700, 0, 24),), ((300, 0, 8), (300, 8, 16), (300, 16, 24))),
                     suffix_lo=1, suffix_hi=128),
    workloads.custom("forest_gaps", B=20, Hq=8, Hkv=8, d=64, dtype="f16",
                     levels=(((129, 2, 20),), ((64, 2, 5), (17, 9, 14)), ((5, 10, 12),)),
                     suffix_lo=0, suffix_hi=70),
]


@pytest.mark.parametrize("cfg", REDUCED, ids=lambda c: c.name)
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("share_min,layout", [(0, "NHD"), (1, "NHD"), (0, "HND")],
                         ids=["policy", "batch_all", "policy_hnd"])
def test_cascade_reduced(cfg, seed, share_min, layout):
    """Every reduced shape, with the batching policy (short or narrowly shared nodes are
    read by each sequence in the suffix pass) and with every node batched; the paged
    suffix in token-major and head-major blocks."""
    say(f"cascade {cfg.name} seed {seed} share_min {share_min} {layout}")
    step = workloads.generate(cfg, seed=seed)
    ds = dev_step(step, kv_layout=layout)
    out, lse = cascade(ds, step.scale, share_min=share_min)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "all")
    compare(out, lse, ref_o, ref_l, cfg.dtype, f"{cfg.name} share_min {share_min} {layout}")


def test_cascade_peaky_scores():
    """Q scaled by 8: a wide score range exercises large online-softmax rescales."""
    cfg = REDUCED[1]
    step = workloads.generate(cfg, seed=5, q_mult=8.0)
    ds = dev_step(step)
    out, lse = cascade(ds, step.scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "all")
    compare(out, lse, ref_o, ref_l, cfg.dtype, "peaky")


def _prefix_splits(q, k, b0, b1):
    """Key-range splits the library plans for one node (from its workspace size)."""
    L = hp.lib()
    qs = hp.make_query(q, k.shape[1])
    node = hp.make_node(k, k, b0, b1)
    nbytes = ctypes.c_size_t(0)
    assert L.hp_prefix_attn_workspace_size(ctypes.byref(qs), ctypes.byref(node),
                                           ctypes.byref(nbytes)) == 0
    rows, d = (b1 - b0) * q.shape[1], q.shape[2]
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for n in range(1, 257):
        if (n == 1 and nbytes.value == 0) or nbytes.value == up(n * rows * d * 4) + up(n * rows * 4):
            return n
    raise AssertionError(f"unexpected workspace size {nbytes.value}")


def _late_rescales(step, node, nsplit):
    """(row, tile) pairs, over all splits of the node, where a tile that is not the first
    of its split has a row max more than 8 log2 units above the row's max over the
    split's earlier tiles: the kernel's running max (which moves lazily, so it is never
    above that max) must then move, and the accumulated O is rescaled by a factor
    strictly between 0 and 1."""
    c = float(np.float32(step.scale)) / np.log(2.0)
    K = node.k.double()
    G = step.cfg.Hq // step.cfg.Hkv
    P = K.shape[0]
    tiles = -(-P // 64)
    tps = -(-tiles // nsplit)
    count = 0
    for h in range(step.cfg.Hq):
        S = (step.q[node.seq_begin:node.seq_end, h, :].double() @ K[:, h // G, :].T) * c
        for t0 in range(0, tiles, tps):
            run = S[:, t0 * 64:(t0 + 1) * 64].max(dim=1).values
            for t in range(t0 + 1, min(t0 + tps, tiles)):
                tm = S[:, t * 64:min((t + 1) * 64, P)].max(dim=1).values
                count += int((tm > run + 8.0).sum())
                run = torch.maximum(run, tm)
    return count


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("P", [4000, 16384], ids=["p4000", "p16384_nontemporal"])
def test_prefix_256row_rescale_mid_split(dtype, P):
    """The 256-row (ping-pong) prefix kernel with peaky scores: Q scaled by 8 and one key
    in the middle of the prefix scaled by 6, so that tiles inside a split raise the row
    max by more than the lazy threshold (checked on the inputs) and O is rescaled by a
    factor strictly between 0 and 1 mid-split.  160 rows per KV head (more than 128
    selects the 256-row kernel).  At P = 16384 the launch's K/V reach 256 MiB, so the
    non-temporal variant of the kernel runs."""
    B, Hq, Hkv, d = 160, 32, 32, 128
    cfg = workloads.custom(f"peaky256_{dtype}_{P}", B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype,
                           levels=(((P, 0, B),),), suffix_lo=1, suffix_hi=20)
    step = workloads.generate(cfg, seed=21, q_mult=8.0)
    node = step.levels[0][0]
    node.k[P // 2 + 37] *= 6.0
    if P * Hkv * d * 2 * 2 >= 256 << 20:
        say("  K/V of the launch reach 256 MiB: non-temporal transfers")
    q = step.q.to(DEV)
    kd, vd = node.k.to(DEV), node.v.to(DEV)
    nsplit = _prefix_splits(q, kd, 0, B)
    late = _late_rescales(step, node, nsplit)
    say(f"peaky 256-row prefix {dtype} P={P}: {nsplit} splits, {late} mid-split rescales")
    assert late >= 100, "the inputs must force rescales inside splits"
    out = torch.zeros(B, Hq, d, device=DEV)
    lse = torch.zeros(B, Hq, device=DEV)
    hp.prefix_attn(q, kd, vd, 0, B, step.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    rows = None if P <= 4000 else sample_rows(B, Hq, 320, seed=3)
    ref_o, ref_l = oracle.step_attention(step, "prefix", rows=rows)
    compare(out, lse, ref_o, ref_l, dtype, f"peaky prefix {dtype} P={P}", rows=rows)
    # and through the whole step (prefix, suffix and merge)
    ds = dev_step(step)
    out2, lse2 = cascade(ds, step.scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "all", rows=rows)
    compare(out2, lse2, ref_o, ref_l, dtype, f"peaky step {dtype} P={P}", rows=rows)


@pytest.mark.parametrize("share_min", [0, 1, 1000], ids=["policy", "batch_all", "none_batched"])
def test_cascade_prefix_only_and_suffix_only(share_min):
    """No paged suffix: the tree alone, its nodes batched, left to the policy (the group
    nodes are read privately: the suffix pass runs on them alone) or all private."""
    cfg = REDUCED[4]
    step = workloads.generate(cfg, seed=6)
    ds = dev_step(step)
    out, lse = cascade(ds, step.scale, paged=False, share_min=share_min)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "prefix")
    compare(out, lse, ref_o, ref_l, cfg.dtype, f"tree only share_min {share_min}")
    out, lse = cascade(ds, step.scale, levels=[])
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "suffix")
    compare(out, lse, ref_o, ref_l, cfg.dtype, "suffix only")


def test_cascade_deterministic():
    cfg = REDUCED[3]
    step = workloads.generate(cfg, seed=7)
    ds = dev_step(step)
    call = hp.CascadeCall(ds["q"], ds["levels"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                          ds["seq_lens"], step.scale)
    o1, l1 = [t.clone() for t in call()]
    o2, l2 = [t.clone() for t in call()]
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bad_metadata_gives_nan_rows_only():
    cfg = REDUCED[1]
    step = workloads.generate(cfg, seed=8)
    ds = dev_step(step)
    ds["block_table"][3, 0] = step.num_blocks          # block id out of range
    ds["block_table"][5, 0] = -1
    ds["seq_lens"][9] = cfg.max_blocks * 16 + 1        # longer than the table
    out, lse = cascade(ds, step.scale)
    torch.cuda.synchronize()
    bad = [3, 5, 9]
    assert torch.isnan(out[bad]).all() and torch.isnan(lse[bad]).all()
    good = [b for b in range(cfg.B) if b not in bad]
    rows = np.array([b * cfg.Hq + h for b in good for h in range(cfg.Hq)])
    ref_o, ref_l = oracle.step_attention(step, "all", rows=rows)
    compare(out, lse, ref_o, ref_l, cfg.dtype, "good rows", rows=rows)


# ------------------------------------------------------------------ needles: bit-exact indexing

NEG = -16384.0   # exact in bf16 and fp16; scale * NEG ~ -1448 underflows exp to exactly 0


def _needle_q(step):
    """q[b][h] = e_c with c = (b*G + h%G) % d: every (KV head, dim) pair has its rows."""
    cfg = step.cfg
    q = torch.zeros_like(step.q)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            q[b, h, (b * cfg.G + h % cfg.G) % cfg.d] = 1.0
    return q


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_needles_suffix_every_position(layout):
    """Every logical suffix position found exactly, through the block table, in both
    block layouts (the needles are placed in the token-major pool, which is copied to
    a head-major one before each call for HND)."""
    cfg = workloads.custom("needle_suf", B=24, Hq=8, Hkv=4, d=128, dtype="bf16",
                           levels=(((200, 0, 24),),), suffix_lo=1, suffix_hi=100)
    step = workloads.generate(cfg, seed=9)
    ds = dev_step(step)
    ds["q"].zero_()
    ds["q"][:, :, 0] = 1.0
    pk = ds["k_pool"]
    for lvl in ds["levels"]:
        for (k, v, _, _) in lvl:
            k[:, :, 0] = NEG
    valid = torch.zeros(pk.shape[:3], dtype=torch.bool)   # (block, slot, head) holding a token
    lens = step.seq_lens.tolist()
    tbl = step.block_table
    for b in range(cfg.B):
        for t in range(lens[b]):
            valid[int(tbl[b, t // 16]), t % 16, :] = True
    pk[..., 0][valid.to(DEV)] = NEG
    if layout == "HND":
        pk_call = pk.permute(0, 2, 1, 3).contiguous()
        pv_call = ds["v_pool"].permute(0, 2, 1, 3).contiguous()
    else:
        pk_call, pv_call = pk, ds["v_pool"]
    call = hp.CascadeCall(ds["q"], ds["levels"], pk_call, pv_call, ds["block_table"],
                          ds["seq_lens"], step.scale, kv_layout=layout)
    suf_v = step.suf_v.float()
    offs = step.suf_offsets.tolist()
    G = cfg.G
    for r in range(max(lens)):
        blks, slots, heads, want_rows = [], [], [], []
        for b in range(cfg.B):
            for g in range(cfg.Hkv):
                t = (r + g) % lens[b]
                blks.append(int(tbl[b, t // 16]))
                slots.append(t % 16)
                heads.append(g)
                want_rows.append(suf_v[offs[b] + t, g])
        idx = (torch.tensor(blks, device=DEV), torch.tensor(slots, device=DEV),
               torch.tensor(heads, device=DEV))
        pk[idx + (0,)] = 0.0
        if layout == "HND":
            pk_call.copy_(pk.permute(0, 2, 1, 3))
        out, lse = call()
        got = out.cpu()
        want = torch.stack(want_rows).view(cfg.B, cfg.Hkv, 1, cfg.d).expand(
            cfg.B, cfg.Hkv, G, cfg.d).reshape(cfg.B, cfg.Hq, cfg.d)
        assert torch.equal(got, want), f"needle run {r}: wrong key picked"
        assert torch.all(lse.cpu() == 0.0), f"needle run {r}: LSE must be exactly 0"
        pk[idx + (0,)] = NEG
    say(f"  suffix needles: {max(lens)} runs, every logical position of every sequence")


@pytest.mark.parametrize("level", [0, 1])
@pytest.mark.parametrize("share_min", [0, 1], ids=["policy", "batch_all"])
def test_needles_prefix_nodes(level, share_min):
    """Every key position of the level's nodes found exactly.  Under the policy the
    root (1000 tokens, 64 sequences) is batched and the level-1 nodes (300 and 260
    tokens, 32 sequences each) are read by each sequence in the suffix pass."""
    cfg = workloads.custom("needle_pfx", B=64, Hq=8, Hkv=2, d=128, dtype="f16",
                           levels=(((1000, 0, 64),), ((300, 0, 32), (260, 32, 64))),
                           suffix_lo=1, suffix_hi=40)
    step = workloads.generate(cfg, seed=10)
    ds = dev_step(step)
    q = _needle_q(step)
    ds["q"].copy_(q.to(DEV))
    for lvl in ds["levels"]:
        for (k, v, _, _) in lvl:
            k.fill_(NEG)
    ds["k_pool"].fill_(NEG)
    call = hp.CascadeCall(ds["q"], ds["levels"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                          ds["seq_lens"], step.scale, share_min=share_min)
    if share_min == 0:
        assert hp.share_decision(cfg.Hq, cfg.Hkv, 1000, 64, d=cfg.d, dtype=torch.float16)
        assert not hp.share_decision(cfg.Hq, cfg.Hkv, 300, 32, d=cfg.d, dtype=torch.float16)
    d, G = cfg.d, cfg.G
    nodes = ds["levels"][level]
    cpu_nodes = step.levels[level]
    P = max(n[0].shape[0] for n in nodes)
    runs = -(-P // d)
    for r in range(runs):
        want = torch.empty(cfg.B, cfg.Hq, d)
        for (k, v, b0, b1), cn in zip(nodes, cpu_nodes):
            L = k.shape[0]
            for g in range(cfg.Hkv):
                for c in range(d):
                    k[(r * d + c + 7 * g) % L, g, c] = 0.0
            for b in range(b0, b1):
                for h in range(cfg.Hq):
                    g, c = h // G, (b * G + h % G) % d
                    want[b, h] = cn.v[(r * d + c + 7 * g) % L, g].float()
        out, lse = call()
        assert torch.equal(out.cpu(), want), f"prefix needle run {r} (level {level}) wrong key"
        assert torch.all(lse.cpu() == 0.0)
        for (k, v, b0, b1) in nodes:
            k.fill_(NEG)
    say(f"  prefix needles level {level}: {runs} runs cover every key of every node")


# ------------------------------------------------------------------ full sizes, sampled rows

FULL = [(workloads.tiny_f32(), "HND"), (workloads.llama3_8b_gqa(), "HND"),
        (workloads.codellama13b_mha(1024), "HND"), (workloads.codellama13b_mha(16384), "HND"),
        (workloads.docqa_codellama7b(), "HND"), (workloads.two_level_gqa(), "HND"),
        (workloads.codellama13b_mha_share(8), "HND"), (workloads.codellama13b_mha(16384), "NHD")]


@pytest.mark.parametrize("cfg,layout", FULL, ids=lambda c: c.name if hasattr(c, "name") else c)
def test_cascade_full_size_every_row(cfg, layout):
    """Each benchmark shape at full size, in the launch configuration bench.py times
    (CascadeCall with the batching policy, head-major paged blocks, passes side by side
    where the plan picks it), and the 16K step with token-major blocks: every row against
    the oracle."""
    say(f"full {cfg.name} {layout}: generating")
    step = workloads.generate(cfg, seed=0)
    ds = dev_step(step, kv_layout=layout)
    say(f"full {cfg.name} {layout}: running")
    call = hp.CascadeCall(ds["q"], ds["levels"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                          ds["seq_lens"], step.scale, kv_layout=layout)
    out, lse = call()
    torch.cuda.synchronize()
    say(f"full {cfg.name}: oracle over {cfg.B * cfg.Hq} rows (side by side: {call.concurrent})")
    ref_o, ref_l = oracle.step_attention(step, "all")
    compare(out, lse, ref_o, ref_l, cfg.dtype, f"{cfg.name} (all rows)")
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


# ------------------------------------------------------------------ graph capture, timed entry

def test_cascade_graph_replay_matches_eager():
    """The whole step captured into a HIP graph: every replay, with eager work and
    synchronisations between replays and changed suffix lengths before one of them,
    equals the eager call on the same inputs."""
    cfg = REDUCED[4]
    step = workloads.generate(cfg, seed=11)
    ds = dev_step(step)
    call = hp.CascadeCall(ds["q"], ds["levels"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                          ds["seq_lens"], step.scale)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(stream=s)
        torch.cuda.synchronize()
        eager_o, eager_l = call.out.clone(), call.lse.clone()
        g = torch.cuda.CUDAGraph()
        g.capture_begin()
        call(stream=s)
        g.capture_end()
    for rep in range(4):
        call.out.fill_(3.0)
        call.lse.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.out, eager_o) and torch.equal(call.lse, eager_l), f"replay {rep}"
    # lengths live in device memory: shortening them changes the replayed step
    new_lens = (step.seq_lens // 2).to(torch.int32)
    ds["seq_lens"].copy_(new_lens.to(DEV))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    segs = []
    for b in range(cfg.B):
        k, v = step.suffix(b)
        n = int(new_lens[b])
        segs.append([(nd.k, nd.v) for nd in step.nodes_of(b)] + [(k[:n], v[:n])])
    ref_o, ref_l = oracle.attention(step.q, segs, cfg.Hkv, step.scale)
    compare(call.out, call.lse, ref_o, ref_l, cfg.dtype, "replay with new lengths")


def test_calls_on_a_stream_that_is_not_current():
    """Every entry point called with stream=s while another stream is current: the
    binding's temporaries (workspace, outputs) must stay reserved until s has run, so
    allocations made on the current stream right after each call (filled with NaN) may
    not land on them."""
    cfg = REDUCED[4]
    step = workloads.generate(cfg, seed=21)
    ds = dev_step(step)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    spin = torch.ones(1 << 26, device=DEV)   # keeps s busy while the current stream allocates
    junk = []
    with torch.cuda.stream(s):
        for _ in range(4):
            spin.mul_(1.0)
    out, lse = hp.cascade_step(ds["q"], ds["levels"], ds["k_pool"], ds["v_pool"],
                               ds["block_table"], ds["seq_lens"], step.scale, stream=s)
    junk += [torch.full((1 << 22,), float("nan"), device=DEV) for _ in range(8)]
    k, v, b0, b1 = ds["levels"][0][0]
    p_out, p_lse = hp.prefix_attn(ds["q"], k, v, b0, b1, step.scale, stream=s)
    junk += [torch.full((1 << 22,), float("nan"), device=DEV) for _ in range(8)]
    s_out, s_lse = hp.suffix_decode(ds["q"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                                    ds["seq_lens"], step.scale, stream=s)
    junk += [torch.full((1 << 22,), float("nan"), device=DEV) for _ in range(8)]
    s.synchronize()
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "all")
    compare(out, lse, ref_o, ref_l, cfg.dtype, "cascade on a non-current stream")
    ref_o, ref_l = oracle.step_attention(step, "suffix")
    compare(s_out, s_lse, ref_o, ref_l, cfg.dtype, "suffix on a non-current stream")
    node = step.levels[0][0]
    segs = [[(node.k, node.v)] if b0 <= b < b1 else [] for b in range(cfg.B)]
    ref_o, ref_l = oracle.attention(step.q, segs, cfg.Hkv, step.scale)
    compare(p_out, p_lse, ref_o, ref_l, cfg.dtype, "prefix on a non-current stream")
    del junk


def test_cascade_timed_records_events_and_matches():
    cfg = REDUCED[2]
    step = workloads.generate(cfg, seed=12)
    ds = dev_step(step)
    call = hp.CascadeCall(ds["q"], ds["levels"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                          ds["seq_lens"], step.scale)
    o1, l1 = [t.clone() for t in call()]
    torch.cuda.synchronize()
    rt = ctypes.CDLL("libamdhip64.so")
    raw = []
    for _ in range(4):
        h = ctypes.c_void_p()
        assert rt.hipEventCreate(ctypes.byref(h)) == 0
        raw.append(h.value)
    o2, l2 = call.timed(raw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ms = []
    for a, b in zip(raw[:-1], raw[1:]):
        t = ctypes.c_float()
        assert rt.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        ms.append(t.value)
    assert all(m >= 0 for m in ms) and ms[0] > 0, ms
    for h in raw:
        rt.hipEventDestroy(ctypes.c_void_p(h))
