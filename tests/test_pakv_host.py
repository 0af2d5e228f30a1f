"""Host tests of the prefix-aware KV cache manager (no GPU).

The manager (hp_pakv_*) is checked against brute force over the live
sequences' token lists ("ChunkAttention: Efficient Self-Attention with
Prefix-Aware KV Cache and Two-Phase Partition", section "Prefix-Aware KV Cache
(PAKV): The Prefix Tree Structure"):
  * insert shares exactly the longest common prefix with any live sequence;
  * rows it calls shared already hold the right token, rows it hands out are
    referenced by no other live sequence (a simulated token pool records what
    was written where, so a row reused while still referenced corrupts some
    sequence's read-back);
  * every live sequence reads back its own tokens;
  * the context's descriptors, taken per batch row in order and cut at the
    row's length, give exactly that sequence's rows, and every descriptor's
    rows lie in one chunk (the contiguity of the ranges is what makes this
    possible);
  * with inserts only, every distinct prefix is stored once (the tree holds
    one row per trie node);
  * freed chunks return to the free list and are reused before fresh ones.
"""
import numpy as np
import pytest

import decode_attention_shared_amd as hp

CHUNK = hp.HP_CHUNK


def _lcp(a, b):
    n = 0
    for x, y in zip(a, b):
        if x != y:
            break
        n += 1
    return n


class Model:
    def __init__(self, num_chunks):
        self.P = hp.Pakv(num_chunks)
        self.seqs = {}          # id -> token list
        self.pool = {}          # row -> token written there

    def live_rows(self, exclude=None):
        out = set()
        for sid in self.seqs:
            if sid != exclude:
                out.update(self.P.seq_rows(sid).tolist())
        return out

    def insert(self, sid, toks):
        expect = max([_lcp(toks, t) for t in self.seqs.values()] + [0])
        others = self.live_rows()
        rows, matched = self.P.insert(sid, toks)
        assert matched == expect, (matched, expect)
        for t in range(len(toks)):
            r = int(rows[t])
            if t < matched:
                assert self.pool.get(r) == toks[t], "shared row holds another token"
            else:
                assert r not in others, "fresh row still referenced by a live sequence"
                self.pool[r] = toks[t]
        self.seqs[sid] = list(toks)

    def append(self, sid, tok):
        others = self.live_rows(exclude=sid)
        own = self.P.seq_rows(sid).tolist()
        r, changed = self.P.append(sid, tok)
        assert r not in others and r not in own
        if not changed:  # grown in place: the row after the sequence's last one
            assert own and r == own[-1] + 1
        self.pool[r] = tok
        self.seqs[sid].append(tok)

    def remove(self, sid):
        self.P.remove(sid)
        del self.seqs[sid]

    def check(self):
        for sid, toks in self.seqs.items():
            rows = self.P.seq_rows(sid)
            assert [self.pool[int(r)] for r in rows] == toks
        order, lens, descs = self.P.context()
        assert sorted(order.tolist()) == sorted(self.seqs)
        for b, sid in enumerate(order.tolist()):
            assert lens[b] == len(self.seqs[sid])
            rows = []
            for (r, c, b0, b1) in descs.tolist():
                assert 1 <= c <= CHUNK and r // CHUNK == (r + c - 1) // CHUNK
                assert 0 <= b0 < b1 <= len(order)
                if b0 <= b < b1:
                    rows.extend(range(r, r + c))
            assert rows[:lens[b]] == self.P.seq_rows(sid).tolist()
            # only the last descriptor may name rows past the sequence's end
            assert len(rows) - lens[b] < CHUNK
        st = self.P.stats()
        assert st.seqs == len(self.seqs)
        assert st.tokens_logical == sum(len(t) for t in self.seqs.values())
        assert st.chunks_used + st.chunks_free + st.chunks_fresh == st.num_chunks
        assert st.nodes == len(descs)


def _random_tokens(rng, model, vocab):
    if model.seqs and rng.random() < 0.7:
        base = list(model.seqs.values())[rng.integers(len(model.seqs))]
        k = int(rng.integers(0, len(base) + 1))
        return base[:k] + [int(x) for x in rng.integers(0, vocab, int(rng.integers(0, 150)))]
    return [int(x) for x in rng.integers(0, vocab, int(rng.integers(0, 200)))]


@pytest.mark.parametrize("seed", range(6))
def test_random_insert_append_remove(seed):
    rng = np.random.default_rng(seed)
    m = Model(4000)
    next_id = 0
    for step in range(220):
        op = rng.random()
        if op < 0.35 or not m.seqs:
            m.insert(next_id, _random_tokens(rng, m, vocab=3 if seed % 2 else 50))
            next_id += 1
        elif op < 0.8:
            for sid in list(m.seqs):
                if rng.random() < 0.5:
                    m.append(sid, int(rng.integers(0, 4)))
        else:
            m.remove(list(m.seqs)[rng.integers(len(m.seqs))])
        if step % 5 == 0:
            m.check()
    m.check()
    for sid in list(m.seqs):
        m.remove(sid)
    st = m.P.stats()
    assert st.chunks_used == 0 and st.nodes == 0 and st.tokens_stored == 0


@pytest.mark.parametrize("seed", range(4))
def test_inserts_store_each_prefix_once(seed):
    rng = np.random.default_rng(100 + seed)
    m = Model(4000)
    for sid in range(40):
        m.insert(sid, _random_tokens(rng, m, vocab=4))
        if sid % 7 == 6:
            m.remove(int(rng.choice(list(m.seqs))))
        prefixes = {tuple(t[:k + 1]) for t in m.seqs.values() for k in range(len(t))}
        assert m.P.stats().tokens_stored == len(prefixes)
    m.check()


def test_split_shares_rows_without_copy():
    m = Model(16)
    m.insert(1, list(range(100)))
    r1 = m.P.seq_rows(1)
    m.insert(2, list(range(70)) + [7, 7])
    assert m.P.seq_rows(2)[:70].tolist() == r1[:70].tolist()
    # the first sequence keeps its rows and can still grow in place
    assert m.P.seq_rows(1).tolist() == r1.tolist()
    row, changed = m.P.append(1, 5)
    assert not changed and row == r1[-1] + 1
    # a strict prefix of a live sequence ends at a split and appends elsewhere
    m.insert(3, list(range(30)))
    assert m.P.seq_rows(3).tolist() == r1[:30].tolist()
    row, changed = m.P.append(3, 9)
    assert changed and row % CHUNK == 0
    m.pool[row] = 9
    m.seqs[3].append(9)
    m.seqs[1].append(5)
    m.pool[r1[-1] + 1] = 5
    m.check()


def test_free_list_reuse_and_capacity():
    m = Model(4)
    m.insert(1, list(range(128)))          # chunks 0, 1
    m.insert(2, [9] * 64)                  # chunk 2
    st = m.P.stats()
    assert (st.chunks_used, st.chunks_free, st.chunks_fresh) == (3, 0, 1)
    m.remove(1)
    st = m.P.stats()
    assert (st.chunks_used, st.chunks_free, st.chunks_fresh) == (1, 2, 1)
    m.insert(3, [5] * 100)                 # reuses the two freed chunks, not the fresh one
    st = m.P.stats()
    assert (st.chunks_used, st.chunks_free, st.chunks_fresh) == (3, 0, 1)
    before = (st.chunks_used, st.nodes, st.tokens_stored)
    with pytest.raises(hp.HpError) as e:   # needs 2 chunks, 1 left: nothing changes
        m.P.insert(4, [1] * 65)
    assert e.value.status == 6
    st = m.P.stats()
    assert (st.chunks_used, st.nodes, st.tokens_stored) == before
    m.check()


def test_errors():
    P = hp.Pakv(2)
    P.insert(1, [1, 2, 3])
    with pytest.raises(hp.HpError) as e:
        P.insert(1, [4])
    assert e.value.status == 2
    for call in (lambda: P.append(9, 1), lambda: P.remove(9), lambda: P.seq_rows(9)):
        with pytest.raises(hp.HpError) as e:
            call()
        assert e.value.status == 2
    with pytest.raises(hp.HpError):
        hp.Pakv(-1)
