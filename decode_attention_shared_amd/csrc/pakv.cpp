// Prefix-aware KV cache manager ("ChunkAttention: Efficient Self-Attention
// with Prefix-Aware KV Cache and Two-Phase Partition", section "Prefix-Aware
// KV Cache (PAKV): The Prefix Tree Structure": the prefix tree, its Insert,
// Append and Delete operations and its chunk allocator; section "Context
// Generation and GPU-CPU Coordination": the (C, i, j) context).  Host only:
// it hands out pool rows; the caller's device pool holds the K/V.
//
// A node holds a run of 1..64 tokens stored in rows slot0 .. slot0 + n - 1 of
// one chunk.  Splitting a node at a token keeps both halves in the same chunk
// (the second half starts at slot0 + k), so a partly matched node is shared
// without copying.  A chunk is free when no node uses it.  A node's tokens can
// grow in place only while it is the leaf of exactly one sequence and ends at
// the chunk's last written slot; otherwise a new token starts a new node in a
// new chunk.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <memory>
#include <unordered_map>
#include <vector>

#include "guard.hpp"
#include "hp_attn.h"

namespace {

struct Node {
    int32_t chunk = -1;
    int32_t slot0 = 0;
    std::vector<int32_t> tokens;
    Node *parent = nullptr;
    std::vector<Node *> children;  // in creation order: the context's pre-order
    std::vector<int64_t> ending;   // sequences whose path ends here
    int32_t refs = 0;              // live sequences whose path holds this node
};

struct Seq {
    Node *leaf;
    int64_t len;
};

}  // namespace

struct hp_pakv {
    int32_t num_chunks = 0;
    int32_t fresh = 0;                 // chunks [fresh, num_chunks) never handed out
    std::vector<int32_t> chunk_nodes;  // nodes using each chunk
    std::vector<int32_t> chunk_used;   // slots written in each chunk (its tail)
    std::vector<int32_t> free_list;    // freed chunks, reused last-in first-out
    Node root;
    int32_t nodes = 0;
    std::unordered_map<int64_t, Seq> seqs;

    int32_t available() const { return (int32_t)free_list.size() + (num_chunks - fresh); }

    int32_t alloc_chunk() {
        int32_t c;
        if (!free_list.empty()) {
            c = free_list.back();
            free_list.pop_back();
        } else {
            c = fresh++;
        }
        chunk_nodes[c] = 0;
        chunk_used[c] = 0;
        return c;
    }
    void release_chunk(int32_t c) {
        if (--chunk_nodes[c] == 0) {
            chunk_used[c] = 0;
            free_list.push_back(c);
        }
    }
    Node *new_node(Node *parent, int32_t chunk, int32_t slot0) {
        Node *n = new Node;
        n->parent = parent;
        n->chunk = chunk;
        n->slot0 = slot0;
        chunk_nodes[chunk]++;
        parent->children.push_back(n);
        ++nodes;
        return n;
    }
    static bool owns_tail(const hp_pakv &p, const Node *n) {
        return p.chunk_used[n->chunk] == n->slot0 + (int32_t)n->tokens.size();
    }

    // Longest match of tokens[pos..n) below `node`: every child whose first
    // token matches is explored, so duplicate-start siblings are handled.
    struct Match {
        int64_t total;  // tokens matched from the root
        Node *node;     // node holding the last matched token (root if none)
        int32_t k;      // tokens of `node` matched (== its size unless partial)
    };
    Match best_match(Node *node, const int32_t *tokens, int64_t n, int64_t pos) {
        Match best{pos, node, (int32_t)node->tokens.size()};
        for (Node *c : node->children) {
            int32_t k = 0;
            const int32_t cn = (int32_t)c->tokens.size();
            while (k < cn && pos + k < n && c->tokens[k] == tokens[pos + k]) ++k;
            if (k == 0) continue;
            Match m = (k == cn) ? best_match(c, tokens, n, pos + k) : Match{pos + k, c, k};
            if (m.total > best.total) best = m;
        }
        return best;
    }

    // Cut `x` after its first k tokens; the rest becomes its only child.
    void split(Node *x, int32_t k) {
        Node *y = new Node;
        y->chunk = x->chunk;
        y->slot0 = x->slot0 + k;
        y->tokens.assign(x->tokens.begin() + k, x->tokens.end());
        x->tokens.resize(k);
        y->parent = x;
        y->children.swap(x->children);
        for (Node *c : y->children) c->parent = y;
        y->ending.swap(x->ending);
        for (int64_t id : y->ending) seqs[id].leaf = y;
        y->refs = x->refs;
        x->children.push_back(y);
        chunk_nodes[x->chunk]++;
        ++nodes;
    }

    void rows_of(const Seq &s, int32_t *rows) const {
        std::vector<const Node *> path;
        for (const Node *n = s.leaf; n && n != &root; n = n->parent) path.push_back(n);
        int64_t t = 0;
        for (auto it = path.rbegin(); it != path.rend(); ++it)
            for (size_t i = 0; i < (*it)->tokens.size(); ++i)
                rows[t++] = (*it)->chunk * HP_CHUNK + (*it)->slot0 + (int32_t)i;
    }

    void free_subtree(Node *n) {
        for (Node *c : n->children) {
            free_subtree(c);
            delete c;
        }
        n->children.clear();
    }
    ~hp_pakv() { free_subtree(&root); }
};

extern "C" {

hp_status hp_pakv_create(int32_t num_chunks, hp_pakv **out) {
    return hp::guarded([&]() -> hp_status {
        if (!out) return HP_ERR_NULL;
        *out = nullptr;
        if (num_chunks < 0 || (int64_t)num_chunks * HP_CHUNK > INT32_MAX) return HP_ERR_INVALID_ARG;
        std::unique_ptr<hp_pakv> p(new hp_pakv);
        p->num_chunks = num_chunks;
        p->chunk_nodes.assign(num_chunks, 0);
        p->chunk_used.assign(num_chunks, 0);
        *out = p.release();
        return HP_OK;
    });
}

void hp_pakv_destroy(hp_pakv *p) {
    try {
        delete p;
    } catch (...) {
    }
}

hp_status hp_pakv_insert(hp_pakv *p, int64_t seq_id, const int32_t *tokens, int32_t n,
                         int32_t *rows, int32_t *matched) {
    return hp::guarded([&]() -> hp_status {
        if (!p) return HP_ERR_NULL;
        if (n < 0) return HP_ERR_INVALID_ARG;
        if (n > 0 && !tokens) return HP_ERR_NULL;
        if (p->seqs.count(seq_id)) return HP_ERR_INVALID_ARG;
        hp_pakv::Match m = p->best_match(&p->root, tokens, n, 0);
        const int64_t rest = n - m.total;
        if ((rest + HP_CHUNK - 1) / HP_CHUNK > p->available()) return HP_ERR_CAPACITY;

        Node *end = m.node;
        if (end != &p->root && m.k < (int32_t)end->tokens.size()) p->split(end, m.k);
        for (Node *x = end; x; x = x->parent) x->refs++;
        Node *leaf = end;
        for (int64_t t = m.total; t < n;) {
            const int32_t c = p->alloc_chunk();
            Node *nn = p->new_node(leaf, c, 0);
            const int64_t take = std::min<int64_t>(HP_CHUNK, n - t);
            nn->tokens.assign(tokens + t, tokens + t + take);
            p->chunk_used[c] = (int32_t)take;
            nn->refs = 1;
            leaf = nn;
            t += take;
        }
        leaf->ending.push_back(seq_id);
        Seq s{leaf, n};
        p->seqs[seq_id] = s;
        if (rows) p->rows_of(s, rows);
        if (matched) *matched = (int32_t)m.total;
        return HP_OK;
    });
}

hp_status hp_pakv_append(hp_pakv *p, int64_t seq_id, int32_t token, int32_t *row,
                         int32_t *changed) {
    return hp::guarded([&]() -> hp_status {
        if (!p) return HP_ERR_NULL;
        auto it = p->seqs.find(seq_id);
        if (it == p->seqs.end()) return HP_ERR_INVALID_ARG;
        Seq &s = it->second;
        Node *L = s.leaf;
        const int32_t end = L->slot0 + (int32_t)L->tokens.size();
        const bool grow = L != &p->root && L->refs == 1 && L->children.empty() && end < HP_CHUNK &&
                          hp_pakv::owns_tail(*p, L);
        int32_t r;
        if (grow) {
            r = L->chunk * HP_CHUNK + end;
            L->tokens.push_back(token);
            p->chunk_used[L->chunk]++;
        } else {
            if (p->available() < 1) return HP_ERR_CAPACITY;
            const int32_t c = p->alloc_chunk();
            Node *nn = p->new_node(L, c, 0);
            nn->tokens.push_back(token);
            nn->refs = 1;
            p->chunk_used[c] = 1;
            L->ending.erase(std::find(L->ending.begin(), L->ending.end(), seq_id));
            nn->ending.push_back(seq_id);
            s.leaf = nn;
            r = c * HP_CHUNK;
        }
        s.len++;
        if (row) *row = r;
        if (changed) *changed = grow ? 0 : 1;
        return HP_OK;
    });
}

hp_status hp_pakv_remove(hp_pakv *p, int64_t seq_id) {
    return hp::guarded([&]() -> hp_status {
        if (!p) return HP_ERR_NULL;
        auto it = p->seqs.find(seq_id);
        if (it == p->seqs.end()) return HP_ERR_INVALID_ARG;
        Node *n = it->second.leaf;
        n->ending.erase(std::find(n->ending.begin(), n->ending.end(), seq_id));
        while (n != &p->root) {
            Node *parent = n->parent;
            if (--n->refs == 0) {  // no live sequence passes here: nor below
                auto &sib = parent->children;
                sib.erase(std::find(sib.begin(), sib.end(), n));
                p->release_chunk(n->chunk);
                delete n;
                --p->nodes;
            }
            n = parent;
        }
        p->root.refs--;
        p->seqs.erase(it);
        return HP_OK;
    });
}

hp_status hp_pakv_context(hp_pakv *p, int64_t *seq_order, int32_t *seq_lens,
                          int32_t seq_capacity, hp_chunk_desc *descs, int32_t desc_capacity,
                          int32_t *num_seqs, int32_t *num_descs) {
    return hp::guarded([&]() -> hp_status {
        if (!p || !num_seqs || !num_descs) return HP_ERR_NULL;
        const int32_t ns = (int32_t)p->seqs.size(), nd = p->nodes;
        *num_seqs = ns;
        *num_descs = nd;
        if (seq_capacity < ns || desc_capacity < nd) return HP_ERR_CAPACITY;
        if ((ns > 0 && (!seq_order || !seq_lens)) || (nd > 0 && !descs)) return HP_ERR_NULL;
        int32_t b = 0, k = 0;
        // Pre-order: a node's own sequences first, then its children's, so the
        // sequences under every node are the contiguous batch rows [i, j).
        struct Frame {
            Node *n;
            size_t next;
            int32_t desc;
        };
        std::vector<Frame> stack;
        auto enter = [&](Node *n) {
            int32_t di = -1;
            if (n != &p->root) {
                di = k++;
                const bool grow = n->refs == 1 && n->children.empty() && hp_pakv::owns_tail(*p, n);
                descs[di].row = n->chunk * HP_CHUNK + n->slot0;
                descs[di].count = grow ? HP_CHUNK - n->slot0 : (int32_t)n->tokens.size();
                descs[di].seq_begin = b;
            }
            for (int64_t id : n->ending) {
                seq_order[b] = id;
                seq_lens[b] = (int32_t)p->seqs[id].len;
                ++b;
            }
            stack.push_back(Frame{n, 0, di});
        };
        enter(&p->root);
        while (!stack.empty()) {
            Frame &f = stack.back();
            if (f.next < f.n->children.size()) {
                Node *c = f.n->children[f.next++];
                enter(c);
            } else {
                if (f.desc >= 0) descs[f.desc].seq_end = b;
                stack.pop_back();
            }
        }
        return HP_OK;
    });
}

hp_status hp_pakv_seq_rows(hp_pakv *p, int64_t seq_id, int32_t *rows, int32_t capacity,
                           int32_t *n) {
    return hp::guarded([&]() -> hp_status {
        if (!p || !n) return HP_ERR_NULL;
        auto it = p->seqs.find(seq_id);
        if (it == p->seqs.end()) return HP_ERR_INVALID_ARG;
        *n = (int32_t)it->second.len;
        if (capacity < it->second.len) return HP_ERR_CAPACITY;
        if (it->second.len > 0 && !rows) return HP_ERR_NULL;
        p->rows_of(it->second, rows);
        return HP_OK;
    });
}

hp_status hp_pakv_get_stats(hp_pakv *p, hp_pakv_stats *st) {
    return hp::guarded([&]() -> hp_status {
        if (!p || !st) return HP_ERR_NULL;
        std::memset(st, 0, sizeof *st);
        st->num_chunks = p->num_chunks;
        for (int32_t c = 0; c < p->fresh; ++c) st->chunks_used += p->chunk_nodes[c] > 0;
        st->chunks_free = (int32_t)p->free_list.size();
        st->chunks_fresh = p->num_chunks - p->fresh;
        st->nodes = p->nodes;
        st->seqs = (int32_t)p->seqs.size();
        std::vector<Node *> todo{&p->root};
        while (!todo.empty()) {
            Node *n = todo.back();
            todo.pop_back();
            st->tokens_stored += (int64_t)n->tokens.size();
            for (Node *c : n->children) todo.push_back(c);
        }
        for (auto &kv : p->seqs) st->tokens_logical += kv.second.len;
        return HP_OK;
    });
}

}  // extern "C"
