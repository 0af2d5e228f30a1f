"""hp_cascade_step_noalloc: the cascade step whose workspace is the library's fixed
per-GPU scratch array.  Its results must be those of hp_cascade_step with a
caller-allocated workspace (same plan, same kernels: the same bits), call after call,
whatever an earlier call left in the array."""
import ctypes
import os

import pytest
import torch

import decode_attention_shared_amd as hp
import oracle
import workloads
from decode_attention_shared_amd import PagedKV, PrefixNode, PrefixTree, Query, HP_BF16
from gpu_util import compare

CAPACITY = 6
FAKE = 0x10000  # an aligned non-null address; validation never dereferences it


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hp.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return hp.lib()


def _fake_step(B, Hq, Hkv, d, P):
    q = Query(FAKE, B, Hq, Hkv, d, HP_BF16, 0.088)
    nodes = (PrefixNode * 1)(PrefixNode(FAKE, FAKE, Hkv * d, d, P, 0, B))
    tree = PrefixTree(1, (ctypes.c_int32 * 4)(1, 0, 0, 0),
                      ctypes.cast(nodes, ctypes.POINTER(PrefixNode)))
    kv = PagedKV(FAKE, FAKE, FAKE, FAKE, 8, 16, B * 8)
    return q, tree, kv, nodes


def test_noalloc_rejects_steps_beyond_the_scratch(L):
    """A step whose workspace exceeds HP_NOALLOC_SCRATCH_BYTES is refused on the host
    before anything is looked up or enqueued (no GPU is needed to see it)."""
    q, tree, kv, keep = _fake_step(4096, 64, 8, 128, 131072)
    need = ctypes.c_size_t(0)
    assert L.hp_cascade_workspace_size(ctypes.byref(q), ctypes.byref(tree), ctypes.byref(kv),
                                       ctypes.byref(need)) == 0
    assert need.value > hp.HP_NOALLOC_SCRATCH_BYTES
    st = L.hp_cascade_step_noalloc(ctypes.byref(q), ctypes.byref(tree), ctypes.byref(kv),
                                   FAKE, FAKE, None)
    assert st == CAPACITY
    assert b"scratch" in L.hp_status_string(st)


def test_noalloc_validates_like_cascade_step(L):
    q, tree, kv, keep = _fake_step(8, 8, 2, 128, 100)
    assert L.hp_cascade_step_noalloc(None, ctypes.byref(tree), ctypes.byref(kv), FAKE, FAKE,
                                     None) == 1
    bad = Query(FAKE, 8, 8, 2, 96, HP_BF16, 0.088)  # d = 96
    assert L.hp_cascade_step_noalloc(ctypes.byref(bad), ctypes.byref(tree), ctypes.byref(kv),
                                     FAKE, FAKE, None) == 3
    neg = Query(FAKE, 8, 8, 2, 128, HP_BF16, -1.0)
    assert L.hp_cascade_step_noalloc(ctypes.byref(neg), ctypes.byref(tree), ctypes.byref(kv),
                                     FAKE, FAKE, None) == 2
    assert L.hp_cascade_step_noalloc(ctypes.byref(q), ctypes.byref(tree), ctypes.byref(kv),
                                     None, FAKE, None) == 1


def _dev(step):
    dev = "cuda:0"
    levels = [[(n.k.to(dev), n.v.to(dev), n.seq_begin, n.seq_end) for n in lvl]
              for lvl in step.levels]
    return dict(q=step.q.to(dev), levels=levels, k_pool=step.k_pool.to(dev),
                v_pool=step.v_pool.to(dev), block_table=step.block_table.to(dev),
                seq_lens=step.seq_lens.to(dev))


def _reference(ds, scale):
    """hp_cascade_step (one stream, caller workspace) on the same inputs."""
    call = hp.CascadeCall(ds["q"], ds["levels"], ds["k_pool"], ds["v_pool"],
                          ds["block_table"], ds["seq_lens"], scale, overlap=0)
    o, l = call()
    torch.cuda.synchronize()
    return o.clone(), l.clone()


def _noalloc(ds, scale):
    out = torch.full(ds["q"].shape, float("nan"), dtype=torch.float32, device="cuda:0")
    lse = torch.full(ds["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda:0")
    o, l = hp.cascade_step_noalloc(ds["q"], ds["levels"], ds["k_pool"], ds["v_pool"],
                                   ds["block_table"], ds["seq_lens"], scale, out=out, lse=lse)
    assert o.data_ptr() == out.data_ptr() and l.data_ptr() == lse.data_ptr()
    torch.cuda.synchronize()
    return o.clone(), l.clone()


def _same_bits(a, b, what):
    assert torch.equal(a.view(torch.int32), b.view(torch.int32)), what


@pytest.mark.gpu
def test_noalloc_matches_cascade_step_call_after_call():
    """Three calls in a row on the one scratch array: the 16K-token document step
    (B=256, MHA 32, bf16, about 30 MiB of partials), then a smaller two-level GQA
    step, then a step whose root node has no keys (its partial slot still holds the
    earlier calls' values, so a kernel that skipped writing it would show here).
    Each result must equal hp_cascade_step's bit for bit; the small ones are also
    checked against the oracle."""
    torch.manual_seed(0)
    big_cfg = workloads.docqa_codellama7b()
    small_cfg = workloads.custom("noalloc_small", B=24, Hq=16, Hkv=4, d=128, dtype="bf16",
                                 levels=[[(300, 0, 24)], [(70, 0, 10), (129, 10, 24)]],
                                 suffix_lo=1, suffix_hi=40)
    empty_cfg = workloads.custom("noalloc_empty_root", B=12, Hq=8, Hkv=8, d=64, dtype="f16",
                                 levels=[[(0, 0, 12)], [(65, 0, 5), (3, 5, 12)]],
                                 suffix_lo=0, suffix_hi=33)
    steps = [workloads.generate(c, seed=s) for c, s in
             ((big_cfg, 11), (small_cfg, 12), (empty_cfg, 13))]
    devs = [_dev(s) for s in steps]

    outs = []
    for st, ds in zip(steps, devs):  # the no-allocation calls, back to back
        print(f"noalloc call: {st.cfg.name} B={st.cfg.B} Hq={st.cfg.Hq} d={st.cfg.d}",
              flush=True)
        outs.append(_noalloc(ds, st.scale))
    for st, ds, (o, l) in zip(steps, devs, outs):
        ro, rl = _reference(ds, st.scale)
        _same_bits(o, ro, f"{st.cfg.name}: O differs from hp_cascade_step")
        _same_bits(l, rl, f"{st.cfg.name}: LSE differs from hp_cascade_step")
    for st, (o, l) in zip(steps[1:], outs[1:]):
        ref_o, ref_l = oracle.step_attention(st, "all")
        compare(o, l, ref_o, ref_l, st.cfg.dtype, f"noalloc {st.cfg.name}")
