"""Seeded synthetic inputs for one decode step of shared-prefix attention.

This module only draws random numbers and lays them out in memory: the
logical (unpaged) key/value arrays that the fp64 oracle reads, and the
shuffled paged pool plus block table that the GPU path reads.  It contains
none of the attention arithmetic.  It is the only code that the oracle side
and the GPU side share.

Workload shapes follow the pages' own setups:
  * "Hydragen: High-Throughput LLM Inference with Shared Prefixes" --
    CodeLlama-13b end-to-end sweep of the shared prefix from 1K to 16K tokens
    at a large batch (section "Estimating Throughput Improvements" and the
    evaluation it summarises), and the two-level few-shot/problem/solution
    tree (section "Hierarchical Sharing").
  * "Read Once, Answer Many: Parallel Prompting for Shared-Context LLM
    Inference" -- one long document read by many question streams with
    CodeLlama-7B (its evaluation setup).
  * "Shared Prefix KV Caching, in depth" -- the Llama-3-8B-shaped cache
    (8 KV heads, head dim 128) and its paged block layout (section "The
    arithmetic of a decode step").

The datasets those pages measure on are not used: every tensor here is drawn
from N(0, 1) with a seeded torch CPU generator, at the pages' shapes.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

BLOCK_SIZE = 16          # tokens per paged KV block
SPARE_FRACTION = 0.125   # extra never-referenced pool blocks (NaN-filled traps)
TAIL_K = 0.0             # key value stored in slots past a sequence's end
TAIL_V = 8192.0          # value stored there (exact in fp32, fp16 and bf16): a read of a tail slot shows up as a large error

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_ESIZE = {"f32": 4, "f16": 2, "bf16": 2}


@dataclasses.dataclass(frozen=True)
class Config:
    """Shape of one decode step.

    ``levels`` is a tuple of tree levels; each level is a tuple of prefix nodes
    ``(len, seq_begin, seq_end)``: sequences ``[seq_begin, seq_end)`` attend
    that node's ``len`` keys.  Suffix lengths are drawn uniformly from the
    inclusive integer range ``[suffix_lo, suffix_hi]``.
    """
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    dtype: str
    levels: Tuple[Tuple[Tuple[int, int, int], ...], ...]
    suffix_lo: int
    suffix_hi: int
    paged: bool = True
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_blocks(self) -> int:
        return max(1, -(-self.suffix_hi // BLOCK_SIZE))

    @property
    def esize(self) -> int:
        return _ESIZE[self.dtype]

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[self.dtype]


def tiny_f32() -> Config:
    return Config("tiny_f32", B=4, Hq=1, Hkv=1, d=64, dtype="f32",
                  levels=(((512, 0, 4),),), suffix_lo=1, suffix_hi=64, paged=False,
                  description="tiny fp32 cascade, prefix 512, suffix U[1,64], contiguous suffix")


def llama3_8b_gqa() -> Config:
    return Config("llama3_8b_gqa", B=64, Hq=32, Hkv=8, d=128, dtype="bf16",
                  levels=(((4096, 0, 64),),), suffix_lo=1, suffix_hi=256,
                  description="Llama-3-8B-shaped layer, GQA 32/8, prefix 4096, B=64, suffix U[1,256]")


def codellama13b_mha(prefix: int = 16384) -> Config:
    return Config(f"codellama13b_mha_p{prefix}", B=256, Hq=40, Hkv=40, d=128, dtype="f16",
                  levels=(((prefix, 0, 256),),), suffix_lo=1, suffix_hi=128,
                  description=f"CodeLlama-13B-shaped layer, MHA 40, fp16, prefix {prefix}, "
                              f"B=256, suffix U[1,128]")


CODELLAMA13B_SWEEP = (1024, 2048, 4096, 8192, 16384)


def codellama13b_mha_share(ways: int = 8, prefix: int = 16384) -> Config:
    """One GPU's share of the CodeLlama-13B shape when its 40 heads are split over
    `ways` GPUs by KV head (40 / ways heads each, no exchange between them)."""
    h = 40 // ways
    return Config(f"codellama13b_mha_p{prefix}_share{ways}", B=256, Hq=h, Hkv=h, d=128,
                  dtype="f16", levels=(((prefix, 0, 256),),), suffix_lo=1, suffix_hi=128,
                  description=f"one {ways}-way head share of CodeLlama-13B: MHA {h}, fp16, "
                              f"prefix {prefix}, B=256, suffix U[1,128]")


def docqa_codellama7b() -> Config:
    return Config("docqa_codellama7b", B=256, Hq=32, Hkv=32, d=128, dtype="bf16",
                  levels=(((16384, 0, 256),),), suffix_lo=64, suffix_hi=512,
                  description="shared 16384-token document, 256 question streams, "
                              "CodeLlama-7B-shaped MHA 32, suffix U[64,512]")


def two_level_gqa() -> Config:
    groups = tuple((1024, 32 * g, 32 * g + 32) for g in range(8))
    return Config("two_level_gqa", B=256, Hq=32, Hkv=8, d=128, dtype="bf16",
                  levels=(((2048, 0, 256),), groups), suffix_lo=1, suffix_hi=128,
                  description="two-level tree: global prefix 2048, 8 groups x sub-prefix 1024, "
                              "32 sequences per group, GQA 32/8, suffix U[1,128]")


def all_configs() -> List[Config]:
    """The five workload shapes, with the CodeLlama-13B sweep at its largest prefix."""
    return [tiny_f32(), llama3_8b_gqa(), codellama13b_mha(16384), docqa_codellama7b(),
            two_level_gqa()]


def custom(name: str, B: int, Hq: int, Hkv: int, d: int, dtype: str, levels, suffix_lo: int,
           suffix_hi: int, paged: bool = True) -> Config:
    """A reduced shape for tests (same structure, smaller sizes)."""
    lv = tuple(tuple(tuple(int(x) for x in node) for node in level) for level in levels)
    return Config(name, B, Hq, Hkv, d, dtype, lv, suffix_lo, suffix_hi, paged)


@dataclasses.dataclass
class Node:
    k: torch.Tensor        # [len][Hkv][d]
    v: torch.Tensor        # [len][Hkv][d]
    seq_begin: int
    seq_end: int

    @property
    def length(self) -> int:
        return int(self.k.shape[0])


@dataclasses.dataclass
class Step:
    """All inputs of one decode step, on the CPU.

    Logical suffix: token ``t`` of sequence ``b`` is row ``suf_offsets[b] + t``
    of ``suf_k`` / ``suf_v`` (the oracle reads these).  Paged suffix: the same
    bytes sit at ``k_pool[block_table[b][t // 16]][t % 16]`` (the GPU reads
    these).  Unreferenced pool blocks are NaN; slots past a sequence's end in
    its last block hold key 0 and value 8192.
    """
    cfg: Config
    seed: int
    scale: float
    q: torch.Tensor
    levels: List[List[Node]]
    seq_lens: torch.Tensor
    suf_offsets: torch.Tensor
    suf_k: torch.Tensor
    suf_v: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_table: torch.Tensor

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    def suffix(self, b: int) -> Tuple[torch.Tensor, torch.Tensor]:
        lo, hi = int(self.suf_offsets[b]), int(self.suf_offsets[b + 1])
        return self.suf_k[lo:hi], self.suf_v[lo:hi]

    def nodes_of(self, b: int) -> List[Node]:
        """Prefix nodes sequence ``b`` attends, root level first."""
        out = []
        for level in self.levels:
            for n in level:
                if n.seq_begin <= b < n.seq_end:
                    out.append(n)
        return out

    def digest(self) -> str:
        """Hash of every generated byte (detects generator drift)."""
        h = hashlib.sha256()
        for t in [self.q, self.seq_lens, self.suf_k, self.suf_v, self.k_pool, self.v_pool,
                  self.block_table]:
            h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
        for level in self.levels:
            for n in level:
                h.update(n.k.contiguous().view(torch.uint8).numpy().tobytes())
                h.update(n.v.contiguous().view(torch.uint8).numpy().tobytes())
        return h.hexdigest()


def pool_in_layout(pool: torch.Tensor, kv_layout: str) -> torch.Tensor:
    """A paged pool [blocks][16][Hkv][d] (NHD, as generated) in the given layout: NHD
    as is, HND as [blocks][Hkv][16][d] (the same values, each block's rows of one KV
    head contiguous)."""
    if kv_layout == "NHD":
        return pool
    if kv_layout == "HND":
        return pool.permute(0, 2, 1, 3).contiguous()
    raise ValueError(f"unknown layout {kv_layout}")


def scale_for(d: int) -> float:
    """The float32 value of 1/sqrt(d), as the kernels receive it."""
    return float(np.float32(1.0 / math.sqrt(d)))


def _randn(g: torch.Generator, shape, dtype: torch.dtype, mult: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if mult != 1.0:
        x.mul_(mult)
    return x.to(dtype)  # round to nearest even


def _validate_config(cfg: Config) -> None:
    if cfg.Hq % cfg.Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    for level in cfg.levels:
        prev_end = 0
        for (ln, b0, b1) in level:
            if not (0 <= b0 < b1 <= cfg.B) or b0 < prev_end or ln < 0:
                raise ValueError(f"bad prefix node {(ln, b0, b1)} in {cfg.name}")
            prev_end = b1
    if not (0 <= cfg.suffix_lo <= cfg.suffix_hi):
        raise ValueError("bad suffix range")


def generate(cfg: Config, seed: int = 0, q_mult: float = 1.0,
             seq_lens: Optional[Sequence[int]] = None) -> Step:
    """Draw one decode step's inputs.

    Draw order (all from one ``torch.Generator`` seeded with ``seed``): suffix
    lengths, Q, each prefix node's K then V (root level first), the logical
    suffix K then V, then a permutation of the pool blocks.  ``q_mult``
    scales Q before rounding (a "peaky" variant with a wider score range).
    ``seq_lens`` overrides the drawn suffix lengths (the draw still happens,
    so the rest of the stream is unchanged).
    """
    _validate_config(cfg)
    g = torch.Generator().manual_seed(int(seed))
    dt = cfg.torch_dtype
    drawn = torch.randint(cfg.suffix_lo, cfg.suffix_hi + 1, (cfg.B,), generator=g,
                          dtype=torch.int64)
    if seq_lens is not None:
        lst = [int(x) for x in seq_lens]
        if len(lst) != cfg.B or any(x < 0 or x > cfg.max_blocks * BLOCK_SIZE for x in lst):
            raise ValueError("seq_lens override out of range")
        drawn = torch.as_tensor(lst, dtype=torch.int64)
    lens = drawn
    q = _randn(g, (cfg.B, cfg.Hq, cfg.d), dt, q_mult)
    levels: List[List[Node]] = []
    for level in cfg.levels:
        nodes = []
        for (ln, b0, b1) in level:
            k = _randn(g, (ln, cfg.Hkv, cfg.d), dt)
            v = _randn(g, (ln, cfg.Hkv, cfg.d), dt)
            nodes.append(Node(k, v, b0, b1))
        levels.append(nodes)
    total = int(lens.sum())
    offsets = torch.zeros(cfg.B + 1, dtype=torch.int64)
    offsets[1:] = torch.cumsum(lens, 0)
    suf_k = _randn(g, (total, cfg.Hkv, cfg.d), dt)
    suf_v = _randn(g, (total, cfg.Hkv, cfg.d), dt)

    nblk = (lens + BLOCK_SIZE - 1) // BLOCK_SIZE
    used = int(nblk.sum())
    mb = cfg.max_blocks
    if cfg.paged:
        spare = max(1, int(math.ceil(used * SPARE_FRACTION)))
        num_blocks = used + spare
        perm = torch.randperm(num_blocks, generator=g).to(torch.int64)
        table = torch.empty(cfg.B, mb, dtype=torch.int64)
        pad_block = perm[used] if used < num_blocks else perm[0]
        table.fill_(int(pad_block))
        starts = torch.zeros(cfg.B + 1, dtype=torch.int64)
        starts[1:] = torch.cumsum(nblk, 0)
        for b in range(cfg.B):
            n = int(nblk[b])
            table[b, :n] = perm[int(starts[b]):int(starts[b]) + n]
    else:
        # identity table: sequence b owns blocks [b*mb, (b+1)*mb), one contiguous
        # [mb*16][Hkv][d] suffix region per sequence; unused blocks are the traps.
        num_blocks = cfg.B * mb + 1
        torch.randperm(num_blocks, generator=g)  # keep the draw stream uniform
        table = torch.arange(cfg.B * mb, dtype=torch.int64).view(cfg.B, mb)
    k_pool = torch.full((num_blocks, BLOCK_SIZE, cfg.Hkv, cfg.d), float("nan"), dtype=dt)
    v_pool = torch.full((num_blocks, BLOCK_SIZE, cfg.Hkv, cfg.d), float("nan"), dtype=dt)
    if total:
        seq_of_tok = torch.repeat_interleave(torch.arange(cfg.B), lens)
        pos = torch.arange(total) - offsets[seq_of_tok]
        dest = table[seq_of_tok, pos // BLOCK_SIZE] * BLOCK_SIZE + pos % BLOCK_SIZE
        k_pool.view(-1, cfg.Hkv, cfg.d)[dest] = suf_k
        v_pool.view(-1, cfg.Hkv, cfg.d)[dest] = suf_v
    # finite sentinels in the tail slots of each sequence's last block
    for b in range(cfg.B):
        s = int(lens[b])
        if s % BLOCK_SIZE:
            blk = int(table[b, s // BLOCK_SIZE])
            k_pool[blk, s % BLOCK_SIZE:] = TAIL_K
            v_pool[blk, s % BLOCK_SIZE:] = TAIL_V
    return Step(cfg=cfg, seed=int(seed), scale=scale_for(cfg.d), q=q, levels=levels,
                seq_lens=lens.to(torch.int32), suf_offsets=offsets, suf_k=suf_k, suf_v=suf_v,
                k_pool=k_pool, v_pool=v_pool, block_table=table.to(torch.int32))


# ----------------------------------------------------------------------------------------
# Byte and FLOP accounting (what one step must move / compute; no attention arithmetic)
# ----------------------------------------------------------------------------------------

def kv_bytes_per_token(Hkv: int, d: int, esize: int, layers: int = 1) -> int:
    """K and V bytes of one token: 2 (K and V) x layers x Hkv x d x element size."""
    return 2 * layers * Hkv * d * esize


def algorithmic_bytes(cfg: Config, seq_lens: Sequence[int]) -> dict:
    """Bytes one step must move: every prefix node's KV once, each sequence's suffix KV,
    Q in, and fp32 O and LSE out.  Partials and metadata are excluded."""
    tok = kv_bytes_per_token(cfg.Hkv, cfg.d, cfg.esize)
    prefix = sum(ln for level in cfg.levels for (ln, _, _) in level) * tok
    suffix = int(sum(int(s) for s in seq_lens)) * tok
    q = cfg.B * cfg.Hq * cfg.d * cfg.esize
    out = cfg.B * cfg.Hq * cfg.d * 4 + cfg.B * cfg.Hq * 4
    return {"prefix": prefix, "suffix": suffix, "q": q, "out": out,
            "total": prefix + suffix + q + out}


def prefix_flops(cfg: Config) -> int:
    """Dense-product FLOPs of the prefix pass: 2 products (QK^T and PV) x 2 FLOP per MAC x
    rows x keys x d, with rows = sequences of the node x query heads."""
    total = 0
    for level in cfg.levels:
        for (ln, b0, b1) in level:
            total += 4 * (b1 - b0) * cfg.Hq * ln * cfg.d
    return total


# ----------------------------------------------------------------------------------------
# Chunk-tree steps: keys in a pool of rows named by (C, i, j) descriptors
# ----------------------------------------------------------------------------------------

CHUNK = 64  # tokens per pool chunk


@dataclasses.dataclass
class ChunkTreeStep:
    """One decode step over chunk descriptors, on the CPU.

    ``descs[k] = (row, count, seq_begin, seq_end)``: sequences [seq_begin,
    seq_end) attend pool rows row .. row + count - 1.  Sequence b attends the
    rows of every descriptor holding b, in descriptor order, up to
    ``seq_lens[b]`` rows in total (a sequence's last descriptor may name rows
    past that: room to append into, NaN-filled).  Rows no descriptor names are
    NaN too.
    """
    B: int
    Hq: int
    Hkv: int
    d: int
    dtype: str
    scale: float
    q: torch.Tensor            # [B][Hq][d]
    k_pool: torch.Tensor       # [rows][Hkv][d]
    v_pool: torch.Tensor
    descs: np.ndarray          # [n][4] int32
    seq_lens: np.ndarray       # [B] int32: rows each sequence attends

    @property
    def pool_rows(self) -> int:
        return int(self.k_pool.shape[0])

    def rows_of(self, b: int) -> List[int]:
        rows: List[int] = []
        for (r, c, b0, b1) in self.descs.tolist():
            if b0 <= b < b1:
                rows.extend(range(r, r + c))
        return rows[:int(self.seq_lens[b])]

    def keys_of(self, b: int) -> List[Tuple[torch.Tensor, torch.Tensor]]:
        idx = torch.as_tensor(self.rows_of(b), dtype=torch.int64)
        return [(self.k_pool[idx], self.v_pool[idx])]


def _pool_from_descs(g: torch.Generator, num_chunks: int, Hkv: int, d: int, dt: torch.dtype,
                     live_rows: Sequence[int]) -> Tuple[torch.Tensor, torch.Tensor]:
    rows = num_chunks * CHUNK
    k_pool = torch.full((rows, Hkv, d), float("nan"), dtype=dt)
    v_pool = torch.full((rows, Hkv, d), float("nan"), dtype=dt)
    idx = torch.as_tensor(list(live_rows), dtype=torch.int64)
    if idx.numel():
        k_pool[idx] = _randn(g, (idx.numel(), Hkv, d), dt)
        v_pool[idx] = _randn(g, (idx.numel(), Hkv, d), dt)
    return k_pool, v_pool


def random_chunk_tree(seed: int, B: int, Hq: int, Hkv: int, d: int, dtype: str,
                      depth: int = 4, max_chunks: int = 3, root_chunks: int = 4,
                      p_partial: float = 0.3, p_gap: float = 0.2, private_chunks: int = 2,
                      room: bool = True, q_mult: float = 1.0) -> ChunkTreeStep:
    """A random forest of chunk descriptors in tree pre-order.

    Every node covers a contiguous sequence range and holds 1..max_chunks
    pieces (root_chunks at depth 0), each a full 64-row chunk or, with
    probability p_partial, a run of 1..64 rows at a random offset inside one.
    A range of several sequences is cut into 1..4 contiguous parts; each part
    gets a child subtree, or with probability p_gap nothing.  Single sequences
    get 0..private_chunks private pieces.  With ``room``, each sequence's
    last private piece names the rest of its chunk (NaN rows past the
    sequence's length).  Chunks are placed at a random permutation of the
    pool.  Draw order: structure (torch.randint), chunk permutation, Q, then
    K and V of every named row in row order.
    """
    g = torch.Generator().manual_seed(int(seed))
    dt = _TORCH_DTYPES[dtype]

    def ri(lo: int, hi: int) -> int:  # inclusive
        return int(torch.randint(lo, hi + 1, (1,), generator=g))

    def rf() -> float:
        return float(torch.rand((1,), generator=g))

    # (chunk placeholder, slot, count, b0, b1, is_private_leaf_piece)
    pieces: List[List[int]] = []

    def piece(b0: int, b1: int, private: bool) -> None:
        if rf() < p_partial:
            cnt = ri(1, CHUNK)
            slot = ri(0, CHUNK - cnt)
        else:
            cnt, slot = CHUNK, 0
        pieces.append([len(pieces), slot, cnt, b0, b1, int(private)])

    def node(b0: int, b1: int, level: int) -> None:
        n = root_chunks if level == 0 else ri(1, max_chunks)
        for _ in range(n):
            piece(b0, b1, False)
        if b1 - b0 == 1:
            for _ in range(ri(0, private_chunks)):
                piece(b0, b1, True)
            return
        if level + 1 > depth:
            return
        parts = min(b1 - b0, ri(1, 4))
        cuts = sorted(set([b0, b1] + [ri(b0 + 1, b1 - 1) for _ in range(parts - 1)]))
        for lo, hi in zip(cuts[:-1], cuts[1:]):
            if rf() < p_gap:
                continue
            node(lo, hi, level + 1)

    node(0, B, 0)
    num_chunks = len(pieces) + max(1, len(pieces) // 8)
    perm = torch.randperm(num_chunks, generator=g).tolist()
    q = _randn(g, (B, Hq, d), dt, q_mult)

    descs = []
    real = np.zeros(B, dtype=np.int64)
    last_private = {}
    for p in pieces:
        chunk, slot, cnt, b0, b1, priv = p
        row = perm[chunk] * CHUNK + slot
        descs.append([row, cnt, b0, b1])
        for b in range(b0, b1):
            real[b] += cnt
        if b1 - b0 == 1:
            last_private[b0] = len(descs) - 1
    live = sorted({r for (r, c, _, _) in descs for r in range(r, r + c)})
    k_pool, v_pool = _pool_from_descs(g, num_chunks, Hkv, d, dt, live)
    if room:
        for b, k in last_private.items():
            r, c, b0, b1 = descs[k]
            descs[k][1] = CHUNK - (r % CHUNK)  # the rest of the chunk: not yet written
    return ChunkTreeStep(B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, scale=scale_for(d), q=q,
                         k_pool=k_pool, v_pool=v_pool,
                         descs=np.asarray(descs, dtype=np.int32).reshape(-1, 4),
                         seq_lens=real.astype(np.int32))


def chunked_config(cfg: Config, seed: int = 0, seq_lens: Optional[Sequence[int]] = None
                   ) -> ChunkTreeStep:
    """A Config's step laid out as chunk descriptors: every prefix node's keys in
    full 64-row chunks (one descriptor per chunk over the node's range, root
    level first), then each sequence's suffix in private chunks, the last one
    named whole (room to append).  Chunks sit at a random permutation of the
    pool.  Suffix lengths are drawn as in ``generate``; draw order: lengths, Q,
    chunk permutation, K and V of every named row in row order."""
    _validate_config(cfg)
    g = torch.Generator().manual_seed(int(seed))
    dt = cfg.torch_dtype
    lens = torch.randint(cfg.suffix_lo, cfg.suffix_hi + 1, (cfg.B,), generator=g,
                         dtype=torch.int64)
    if seq_lens is not None:
        lens = torch.as_tensor([int(x) for x in seq_lens], dtype=torch.int64)
    q = _randn(g, (cfg.B, cfg.Hq, cfg.d), dt)
    plan = []  # (b0, b1, count, real)
    for level in cfg.levels:
        for (ln, b0, b1) in level:
            for t in range(0, ln, CHUNK):
                c = min(CHUNK, ln - t)
                plan.append((b0, b1, c, c))
    for b in range(cfg.B):
        s = int(lens[b])
        for t in range(0, s, CHUNK):
            c = min(CHUNK, s - t)
            last = t + CHUNK >= s
            plan.append((b, b + 1, CHUNK if last else c, c))
    num_chunks = len(plan) + max(1, len(plan) // 8)
    perm = torch.randperm(num_chunks, generator=g).tolist()
    descs, live = [], []
    real = np.zeros(cfg.B, dtype=np.int64)
    for i, (b0, b1, cnt, rl) in enumerate(plan):
        row = perm[i] * CHUNK
        descs.append([row, cnt, b0, b1])
        live.extend(range(row, row + rl))
        real[b0:b1] += rl
    k_pool, v_pool = _pool_from_descs(g, num_chunks, cfg.Hkv, cfg.d, dt, sorted(live))
    return ChunkTreeStep(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, dtype=cfg.dtype,
                         scale=scale_for(cfg.d), q=q, k_pool=k_pool, v_pool=v_pool,
                         descs=np.asarray(descs, dtype=np.int32).reshape(-1, 4),
                         seq_lens=real.astype(np.int32))


# ----------------------------------------------------------------------------------------
# Shared-context requests: P streams per request, stream-id tagged KV rows
# ----------------------------------------------------------------------------------------

@dataclasses.dataclass
class StreamStep:
    """One decode step of shared-context requests, on the CPU.

    The B queries are the streams: query b is stream ``q_sid[b]`` of request
    ``q_req[b]`` (requests hold P consecutive queries; the last may hold
    fewer).  Every query attends the document nodes ``levels`` (as a Step's
    prefix) and the positions of its request's KV row whose stream id is -1
    or its own.  Request r's row, position i < row_len[r]: stream id
    ``row_sid[r][i]``, logical key/value ``row_k[r][i]`` / ``row_v[r][i]`` (the
    oracle reads these), stored at pool row ``row_slots[r][i]`` of
    ``k_pool`` / ``v_pool`` (the GPU reads these).  Row layout, as the
    Parallel Prompting page lays a request out: ``shared_len`` tokens every
    stream sees (id -1), then each stream's question tokens, then the
    streams' answer tokens interleaved step by step.  Unused pool rows are
    NaN; row padding points at a NaN row with id -3 (never visible).
    """
    cfg: Config
    P: int
    seed: int
    scale: float
    q: torch.Tensor            # [B][Hq][d]
    levels: List[List[Node]]
    q_req: torch.Tensor        # [B] int32
    q_sid: torch.Tensor        # [B] int32
    own_lens: torch.Tensor     # [B] int64: question + answer tokens of each stream
    answer_len: int
    shared_len: int
    row_len: torch.Tensor      # [R] int32
    row_sid: torch.Tensor      # [R][row_cap] int32
    row_slots: torch.Tensor    # [R][row_cap] int32
    row_k: List[torch.Tensor]  # per request [row_len][Hkv][d]
    row_v: List[torch.Tensor]
    k_pool: torch.Tensor       # [pool_rows][Hkv][d]
    v_pool: torch.Tensor

    @property
    def R(self) -> int:
        return int(self.row_len.shape[0])

    @property
    def row_cap(self) -> int:
        return int(self.row_sid.shape[1])

    def own_positions(self, b: int) -> List[int]:
        """Row positions of stream b's own tokens and the shared tokens, from the
        layout rule (not from the ids): what the stream would hold if decoded alone."""
        r, s = int(self.q_req[b]), int(self.q_sid[b])
        b0 = r * self.P
        n = min(self.P, self.cfg.B - b0)
        qlens = [int(self.own_lens[x]) - self.answer_len for x in range(b0, b0 + n)]
        pos = list(range(self.shared_len))
        start = self.shared_len + sum(qlens[:s])
        pos += list(range(start, start + qlens[s]))
        ans0 = self.shared_len + sum(qlens)
        pos += [ans0 + t * n + s for t in range(self.answer_len)]
        return pos


def docqa_streams(P: int = 32) -> Config:
    """Parallel Prompting's shared-document workload at the docqa_codellama7b shape: one
    16384-token document, 256 question streams in requests of P, each stream with
    question + answer tokens U[64, 512]."""
    base = docqa_codellama7b()
    return dataclasses.replace(base, name=f"docqa_streams_p{P}",
                               description=base.description + f", requests of {P} streams, "
                               "stream-id tagged rows")


def stream_step(cfg: Config, P: int, seed: int = 0, answer_len: int = 32, shared_len: int = 0,
                q_mult: float = 1.0) -> StreamStep:
    """Draw one shared-context step: cfg.B streams in requests of P, document = cfg's
    prefix nodes, each stream's own token count (question + answer) drawn from
    U[cfg.suffix_lo, cfg.suffix_hi] (at least answer_len).  Draw order: own token
    counts, Q, each prefix node's K then V, each request's row K then V in row
    order, then a permutation of the pool rows."""
    _validate_config(cfg)
    if P < 1 or answer_len < 0 or shared_len < 0 or cfg.suffix_lo < answer_len:
        raise ValueError("need P >= 1 and suffix_lo >= answer_len >= 0")
    g = torch.Generator().manual_seed(int(seed))
    dt = cfg.torch_dtype
    B = cfg.B
    own = torch.randint(cfg.suffix_lo, cfg.suffix_hi + 1, (B,), generator=g, dtype=torch.int64)
    q = _randn(g, (B, cfg.Hq, cfg.d), dt, q_mult)
    levels: List[List[Node]] = []
    for level in cfg.levels:
        nodes = []
        for (ln, b0, b1) in level:
            nodes.append(Node(_randn(g, (ln, cfg.Hkv, cfg.d), dt),
                              _randn(g, (ln, cfg.Hkv, cfg.d), dt), b0, b1))
        levels.append(nodes)
    R = -(-B // P)
    sids, row_k, row_v = [], [], []
    for r in range(R):
        b0 = r * P
        n = min(P, B - b0)
        qlens = [int(own[b]) - answer_len for b in range(b0, b0 + n)]
        sid = [-1] * shared_len
        for s in range(n):
            sid += [s] * qlens[s]
        for _ in range(answer_len):
            sid += list(range(n))
        sids.append(sid)
        row_k.append(_randn(g, (len(sid), cfg.Hkv, cfg.d), dt))
        row_v.append(_randn(g, (len(sid), cfg.Hkv, cfg.d), dt))
    lens = [len(s) for s in sids]
    cap = max(1, max(lens))
    used = sum(lens)
    pool_rows = used + max(1, int(math.ceil(used * SPARE_FRACTION)))
    perm = torch.randperm(pool_rows, generator=g).to(torch.int64)
    pad_row = int(perm[used])
    k_pool = torch.full((pool_rows, cfg.Hkv, cfg.d), float("nan"), dtype=dt)
    v_pool = torch.full((pool_rows, cfg.Hkv, cfg.d), float("nan"), dtype=dt)
    row_sid = torch.full((R, cap), -3, dtype=torch.int32)
    row_slots = torch.full((R, cap), pad_row, dtype=torch.int32)
    off = 0
    for r in range(R):
        n = lens[r]
        dest = perm[off:off + n]
        off += n
        row_sid[r, :n] = torch.as_tensor(sids[r], dtype=torch.int32)
        row_slots[r, :n] = dest.to(torch.int32)
        if n:
            k_pool[dest] = row_k[r]
            v_pool[dest] = row_v[r]
    q_req = (torch.arange(B) // P).to(torch.int32)
    q_sid = (torch.arange(B) % P).to(torch.int32)
    return StreamStep(cfg=cfg, P=P, seed=int(seed), scale=scale_for(cfg.d), q=q, levels=levels,
                      q_req=q_req, q_sid=q_sid, own_lens=own, answer_len=answer_len,
                      shared_len=shared_len, row_len=torch.as_tensor(lens, dtype=torch.int32),
                      row_sid=row_sid, row_slots=row_slots, row_k=row_k, row_v=row_v,
                      k_pool=k_pool, v_pool=v_pool)


def stream_bytes(step: StreamStep) -> dict:
    """Bytes a shared-context step must move: each document node's KV once, each
    stream's visible row tokens (its own and the shared ones), the stream ids of
    every row position each query's selection reads, Q in, fp32 O and LSE out."""
    cfg = step.cfg
    tok = kv_bytes_per_token(cfg.Hkv, cfg.d, cfg.esize)
    prefix = sum(ln for level in cfg.levels for (ln, _, _) in level) * tok
    visible = sum(len(step.own_positions(b)) for b in range(cfg.B))
    q = cfg.B * cfg.Hq * cfg.d * cfg.esize
    out = cfg.B * cfg.Hq * cfg.d * 4 + cfg.B * cfg.Hq * 4
    return {"prefix": prefix, "streams": visible * tok, "q": q, "out": out,
            "total": prefix + visible * tok + q + out}
