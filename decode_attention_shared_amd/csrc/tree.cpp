// Host side of the chunk-tree step ("ChunkAttention: Efficient Self-Attention
// with Prefix-Aware KV Cache and Two-Phase Partition", sections "Two-Phase
// Partition (TPP): Algorithm Overview", "The Chunk-First Phase Kernel in
// Detail", "The Sequence-First Phase Kernel in Detail" and "Context
// Generation and GPU-CPU Coordination"): the plan image built from (C, i, j)
// descriptors, the launches of one step, and the KV append entry point.
//
// Plan.  Descriptors covering at least share_min sequences are batched; a run
// of consecutive batched descriptors with one range [i, j) is a segment, whose
// pieces (one per descriptor, up to 64 rows each) are the key tiles of one
// online softmax on the matrix cores, split over workgroups like a prefix
// node.  Segments are launched by row-block width (1, 2, 4 or 8 waves of 32
// rows), each launch reading its workgroup -> segment table from the image.
// Every other descriptor is private: its rows are appended to the row list of
// every sequence it covers.  Per sequence the image holds that row list, the
// number of batched rows it attends, and the (segment, split) partials the
// sequence-first pass merges with its private attention.
#include <algorithm>
#include <cstring>
#include <vector>

#include "guard.hpp"
#include "host.hpp"

using namespace hp;
using namespace hp::host;

namespace hp {
namespace host {

// Batching policy: read a run of `tokens` shared keys once for its `nseq`
// sequences (the chunk-first phase, plus the partial merge) only when that is
// faster than every sequence reading the run in its own pass.  Under a few
// hundred shared tokens, or with few sequences, the extra launch and merge
// cost more than the shared read saves ("Shared Prefix KV Caching, in depth",
// section "Trade-offs"; the boundary conditions listed in "Hydragen:
// High-Throughput LLM Inference with Shared Prefixes", section "How Hydragen
// Positions Itself": long shared prefixes and large batches).
//
// The thresholds are fitted to timings of both ways on MI355X: bf16 and fp16
// (one table: they measure alike), and fp32, each at d = 128 and d = 64; 32
// query heads with 32 KV heads (the column for one query head per KV head)
// or 8 (every larger group); 2, 4, ..., 256 sequences, each with 64 private
// rows; run lengths 64, 128, ..., 4096 and 16384.  Per (type, d, group) the
// thresholds are the smallest that classify every measured point where one
// way beat the other by at least 5 % and that never rise with the number of
// sequences.  A sequence count between two measured ones takes the lower
// one's threshold.  With one query head per KV head the private pass keeps
// up longer (each (sequence, KV head) workgroup streams its keys for a
// single query); fp32 keys favour it longer still (the batched pass then
// runs on the fp32 matrix path).
bool share_decision(int dtype, int d, int G, int64_t tokens, int64_t nseq) {
    if (nseq < 2 || tokens <= 0) return false;
    // [16-bit d128, 16-bit d64, fp32 d128, fp32 d64][G == 1, G > 1][2, 4, ..., 256 sequences]
    static constexpr int32_t kThreshold[4][2][8] = {
        {{2048, 1024, 512, 512, 256, 256, 128, 128}, {512, 512, 512, 512, 512, 512, 256, 128}},
        {{1024, 1024, 1024, 512, 512, 256, 256, 128}, {1024, 1024, 1024, 1024, 1024, 1024, 256, 128}},
        {{2048, 2048, 2048, 1024, 512, 256, 128, 128}, {1024, 1024, 1024, 1024, 1024, 1024, 512, 256}},
        {{2048, 2048, 2048, 2048, 1024, 512, 256, 256}, {1024, 1024, 1024, 1024, 1024, 1024, 512, 256}},
    };
    const int kind = (dtype == HP_F32 ? 2 : 0) + (d == 64 ? 1 : 0);
    int bucket = 0;  // largest measured count (2 << bucket) not above nseq
    while (bucket < 7 && (int64_t(2) << (bucket + 1)) <= nseq) ++bucket;
    return tokens >= kThreshold[kind][G > 1 ? 1 : 0][bucket];
}

}  // namespace host
}  // namespace hp

namespace {

struct Image {
    std::vector<TreeSeg> segs;
    std::vector<TreePiece> pieces;
    std::vector<int32_t> wgseg;
    std::vector<int32_t> seq_tok, tok_rows, seq_src, shared;
    std::vector<TreeSrc> srcs;
};

hp_status check_descs(const hp_query &g, const hp_chunk_desc *descs, int32_t n,
                      int64_t pool_rows) {
    if (n < 0 || pool_rows < 0 || pool_rows > INT32_MAX) return HP_ERR_INVALID_ARG;
    if (n > 0 && !descs) return HP_ERR_NULL;
    for (int32_t k = 0; k < n; ++k) {
        const hp_chunk_desc &c = descs[k];
        if (c.count < 1 || c.count > HP_CHUNK) return HP_ERR_INVALID_ARG;
        if (c.row < 0 || (int64_t)c.row + c.count > pool_rows) return HP_ERR_INVALID_ARG;
        if (c.seq_begin < 0 || c.seq_begin >= c.seq_end || c.seq_end > g.B)
            return HP_ERR_INVALID_ARG;
    }
    return HP_OK;
}

// Everything of the plan but the image bytes; fills `plan` and `img`.
hp_status build(const hp_query &g, const hp_chunk_desc *descs, int32_t n, int32_t share_min,
                int64_t pool_rows, hp_tree_plan &plan, Image &img) {
    const int G = g.Hq / g.Hkv;
    const int B = g.B;
    std::memset(&plan, 0, sizeof plan);
    plan.B = g.B;
    plan.Hq = g.Hq;
    plan.Hkv = g.Hkv;
    plan.d = g.d;
    plan.dtype = g.dtype;
    plan.share_min = share_min;
    plan.num_descs = n;
    plan.pool_rows = pool_rows;

    // Which descriptors are batched: by range size (share_min >= 2), or, with
    // share_min == 0, run by run (consecutive descriptors with one range of at
    // least two sequences) by the measured batching policy on the run's
    // total rows.
    std::vector<char> is_batched(n > 0 ? n : 1, 0);
    for (int32_t k = 0; k < n;) {
        int32_t e = k + 1;
        while (e < n && descs[e].seq_begin == descs[k].seq_begin &&
               descs[e].seq_end == descs[k].seq_end)
            ++e;
        const int32_t nseq = descs[k].seq_end - descs[k].seq_begin;
        bool batch;
        if (share_min == 0) {
            int64_t tokens = 0;
            for (int32_t j = k; j < e; ++j) tokens += descs[j].count;
            batch = share_decision(g.dtype, g.d, G, tokens, nseq);
        } else {
            batch = nseq >= share_min;
        }
        for (int32_t j = k; j < e; ++j) is_batched[j] = batch;
        k = e;
    }

    // Segments: runs of consecutive batched descriptors with one range.
    std::vector<int64_t> seg_tokens;
    bool open = false;
    for (int32_t k = 0; k < n; ++k) {
        const hp_chunk_desc &c = descs[k];
        const bool batched = is_batched[k];
        if (!batched) {
            open = false;
            continue;
        }
        if (!open || img.segs.back().seq_begin != c.seq_begin ||
            img.segs.back().seq_end != c.seq_end) {
            TreeSeg s;
            std::memset(&s, 0, sizeof s);
            s.piece_begin = (int32_t)img.pieces.size();
            s.seq_begin = c.seq_begin;
            s.seq_end = c.seq_end;
            img.segs.push_back(s);
            seg_tokens.push_back(0);
            open = true;
        }
        img.pieces.push_back(TreePiece{c.row, c.count});
        img.segs.back().ntiles++;
        seg_tokens.back() += c.count;
    }
    const int nseg = (int)img.segs.size();

    // Splits, by row-block width; workgroup table entries launch by launch.
    int64_t part_rows = 0;
    const int widths[HP_TREE_MAX_LAUNCHES] = {1, 2, 4, 8};
    for (int wi = 0; wi < HP_TREE_MAX_LAUNCHES; ++wi) {
        const int nw = widths[wi];
        std::vector<int> members;
        std::vector<SplitItem> items;
        for (int s = 0; s < nseg; ++s) {
            const int64_t nseq = img.segs[s].seq_end - img.segs[s].seq_begin;
            if (choose_nw(nseq * G) != nw) continue;
            members.push_back(s);
            items.push_back(SplitItem{nseq * G, nseq * g.Hq, img.segs[s].ntiles});
        }
        if (members.empty()) continue;
        std::vector<SplitPlan> sp(members.size());
        plan_splits(items.data(), (int)items.size(), g.Hkv, g.d, nw, kTreeMaxTilesPerSplit,
                    sp.data());
        const int li = plan.num_launches++;
        plan.launch_nw[li] = nw;
        plan.launch_wg0[li] = (int32_t)img.wgseg.size();
        int64_t wg = 0;
        for (size_t m = 0; m < members.size(); ++m) {
            TreeSeg &sg = img.segs[members[m]];
            sg.nsplit = sp[m].nsplit;
            sg.tiles_per_split = sp[m].tiles_per_split;
            sg.rowblocks = sp[m].rowblocks;
            sg.units_padded = sp[m].units_padded;
            sg.wg_begin = (int32_t)wg;
            for (int w = 0; w < sp[m].wgs; ++w) img.wgseg.push_back(members[m]);
            wg += sp[m].wgs;
        }
        if (wg > INT32_MAX) return HP_ERR_UNSUPPORTED;
        plan.launch_wgs[li] = (int32_t)wg;
    }
    for (int s = 0; s < nseg; ++s) {
        TreeSeg &sg = img.segs[s];
        sg.part_row0 = (int32_t)part_rows;
        part_rows += (int64_t)sg.nsplit * (sg.seq_end - sg.seq_begin);
        if (part_rows > INT32_MAX) return HP_ERR_UNSUPPORTED;
    }

    // Per sequence: partial sources (segment order = tree order, root first)
    // and the batched row count.
    std::vector<int64_t> nsrc(B + 1, 0), shared(B, 0);
    for (int s = 0; s < nseg; ++s)
        for (int b = img.segs[s].seq_begin; b < img.segs[s].seq_end; ++b) {
            nsrc[b + 1]++;
            shared[b] += seg_tokens[s];
        }
    for (int b = 0; b < B; ++b) nsrc[b + 1] += nsrc[b];
    if (nsrc[B] > INT32_MAX) return HP_ERR_UNSUPPORTED;
    img.srcs.assign((size_t)nsrc[B], TreeSrc{0, 0, 0, 0});
    {
        std::vector<int64_t> fill(nsrc.begin(), nsrc.end() - 1);
        for (int s = 0; s < nseg; ++s) {
            const TreeSeg &sg = img.segs[s];
            for (int b = sg.seq_begin; b < sg.seq_end; ++b)
                img.srcs[(size_t)fill[b]++] =
                    TreeSrc{sg.part_row0 + (b - sg.seq_begin), sg.nsplit,
                            sg.seq_end - sg.seq_begin, 0};
        }
    }
    img.seq_src.resize(B + 1);
    img.shared.resize(B);
    for (int b = 0; b <= B; ++b) img.seq_src[b] = (int32_t)nsrc[b];
    for (int b = 0; b < B; ++b) {
        if (shared[b] > INT32_MAX) return HP_ERR_UNSUPPORTED;
        img.shared[b] = (int32_t)shared[b];
    }

    // Private rows: every other descriptor, appended to each sequence it covers.
    std::vector<int64_t> ntok(B + 1, 0);
    for (int32_t k = 0; k < n; ++k) {
        const hp_chunk_desc &c = descs[k];
        if (is_batched[k]) continue;
        for (int b = c.seq_begin; b < c.seq_end; ++b) ntok[b + 1] += c.count;
    }
    int64_t max_private = 0;
    for (int b = 0; b < B; ++b) {
        max_private = std::max(max_private, ntok[b + 1]);
        ntok[b + 1] += ntok[b];
    }
    if (ntok[B] > INT32_MAX) return HP_ERR_UNSUPPORTED;
    img.tok_rows.assign((size_t)ntok[B], 0);
    {
        std::vector<int64_t> fill(ntok.begin(), ntok.end() - 1);
        for (int32_t k = 0; k < n; ++k) {
            const hp_chunk_desc &c = descs[k];
            if (is_batched[k]) continue;
            for (int b = c.seq_begin; b < c.seq_end; ++b)
                for (int r = 0; r < c.count; ++r) img.tok_rows[(size_t)fill[b]++] = c.row + r;
        }
    }
    img.seq_tok.resize(B + 1);
    for (int b = 0; b <= B; ++b) img.seq_tok[b] = (int32_t)ntok[b];

    plan.num_segs = nseg;
    plan.num_pieces = (int32_t)img.pieces.size();
    plan.num_srcs = (int32_t)img.srcs.size();
    plan.num_tok_rows = (int32_t)img.tok_rows.size();
    plan.max_private = (int32_t)max_private;
    plan.part_rows = part_rows;
    const TreeLayout L = tree_layout(nseg, plan.num_pieces, (int64_t)img.wgseg.size(), B,
                                     plan.num_tok_rows, plan.num_srcs);
    plan.blob_bytes = (size_t)L.words * 4;
    plan.workspace_bytes =
        part_rows == 0 ? 0
                       : round_up((size_t)part_rows * g.Hq * g.d * sizeof(float), kWsAlign) +
                             round_up((size_t)part_rows * g.Hq * sizeof(float), kWsAlign);
    return HP_OK;
}

void write_image(const hp_tree_plan &plan, const Image &img, void *blob) {
    const TreeLayout L = tree_layout(plan.num_segs, plan.num_pieces, (int64_t)img.wgseg.size(),
                                     plan.B, plan.num_tok_rows, plan.num_srcs);
    int32_t *w = (int32_t *)blob;
    std::memset(blob, 0, (size_t)L.words * 4);
    auto put = [&](int64_t off, const void *src, size_t bytes) {
        if (bytes) std::memcpy(w + off, src, bytes);
    };
    put(L.segs, img.segs.data(), img.segs.size() * sizeof(TreeSeg));
    put(L.pieces, img.pieces.data(), img.pieces.size() * sizeof(TreePiece));
    put(L.wgseg, img.wgseg.data(), img.wgseg.size() * 4);
    put(L.seq_tok, img.seq_tok.data(), img.seq_tok.size() * 4);
    put(L.tok_rows, img.tok_rows.data(), img.tok_rows.size() * 4);
    put(L.seq_src, img.seq_src.data(), img.seq_src.size() * 4);
    put(L.srcs, img.srcs.data(), img.srcs.size() * sizeof(TreeSrc));
    put(L.shared, img.shared.data(), img.shared.size() * 4);
}

int64_t total_wgs(const hp_tree_plan &p) {
    int64_t w = 0;
    for (int i = 0; i < p.num_launches; ++i) w += p.launch_wgs[i];
    return w;
}

}  // namespace

extern "C" {

hp_status hp_tree_plan_build(const hp_query *geom, const hp_chunk_desc *descs, int32_t n,
                             int32_t share_min, int64_t pool_rows, void *blob,
                             size_t blob_capacity, hp_tree_plan *plan) {
    return hp::guarded([&]() -> hp_status {
        if (!plan) return HP_ERR_NULL;
        hp_status st = check_geometry(geom, false);
        if (st != HP_OK) return st;
        if (share_min != 0 && share_min < 2) return HP_ERR_INVALID_ARG;
        st = check_descs(*geom, descs, n, pool_rows);
        if (st != HP_OK) return st;
        hp_tree_plan p;
        Image img;
        st = build(*geom, descs, n, share_min, pool_rows, p, img);
        if (st != HP_OK) return st;
        if (blob) {
            if (blob_capacity < p.blob_bytes) return HP_ERR_CAPACITY;
            write_image(p, img, blob);
        }
        *plan = p;
        return HP_OK;
    });
}

hp_status hp_share_decision(const hp_query *geom, int64_t tokens, int32_t nseq,
                            int32_t *batch) {
    return hp::guarded([&]() -> hp_status {
        if (!batch) return HP_ERR_NULL;
        hp_status st = check_geometry(geom, false);
        if (st != HP_OK) return st;
        if (tokens < 0 || nseq < 0 || nseq > geom->B) return HP_ERR_INVALID_ARG;
        *batch = share_decision(geom->dtype, geom->d, geom->Hq / geom->Hkv, tokens, nseq) ? 1 : 0;
        return HP_OK;
    });
}

hp_status hp_tree_step(const hp_query *q, const hp_tree_plan *plan, const void *blob_dev,
                       const void *k_pool, const void *v_pool, const int32_t *seq_lens,
                       float *o, float *lse, void *ws, size_t ws_bytes, void *stream) {
    return hp::guarded([&]() -> hp_status {
        hp_status st = check_geometry(q, true);
        if (st != HP_OK) return st;
        if (!plan || !o) return HP_ERR_NULL;
        if (plan->B != q->B || plan->Hq != q->Hq || plan->Hkv != q->Hkv || plan->d != q->d ||
            plan->dtype != q->dtype)
            return HP_ERR_INVALID_ARG;
        if (plan->num_launches < 0 || plan->num_launches > HP_TREE_MAX_LAUNCHES)
            return HP_ERR_INVALID_ARG;
        if (!aligned16(o) || ((uintptr_t)lse & 3u) || ((uintptr_t)seq_lens & 3u))
            return HP_ERR_INVALID_ARG;
        if (q->B == 0) return HP_OK;
        if (!blob_dev) return HP_ERR_NULL;
        if (!aligned16(blob_dev)) return HP_ERR_INVALID_ARG;
        const bool reads_pool = plan->num_pieces > 0 || plan->num_tok_rows > 0;
        if (reads_pool && (!k_pool || !v_pool)) return HP_ERR_NULL;
        if (reads_pool && (!aligned16(k_pool) || !aligned16(v_pool))) return HP_ERR_INVALID_ARG;
        const int64_t row_stride = (int64_t)q->Hkv * q->d;
        if ((int64_t)kTileKeys * row_stride + q->d > (int64_t)INT32_MAX) return HP_ERR_UNSUPPORTED;
        if (plan->workspace_bytes > 0 && (!ws || ws_bytes < plan->workspace_bytes || !aligned16(ws)))
            return HP_ERR_WORKSPACE;

        const TreeLayout L = tree_layout(plan->num_segs, plan->num_pieces, total_wgs(*plan), q->B,
                                         plan->num_tok_rows, plan->num_srcs);
        float *part_o = (float *)ws;
        float *part_lse = plan->part_rows == 0
                              ? nullptr
                              : (float *)((char *)ws + round_up((size_t)plan->part_rows * q->Hq *
                                                                    q->d * sizeof(float),
                                                                kWsAlign));
        hipStream_t s = (hipStream_t)stream;
        const float scale_log2 = (float)((double)q->scale * 1.4426950408889634);

        // Chunk-first phase: every segment, one launch per row-block width.
        for (int li = 0; li < plan->num_launches; ++li) {
            if (plan->launch_wgs[li] <= 0) continue;
            PrefixArgs a;
            std::memset(&a, 0, sizeof a);
            a.q = q->q;
            a.B = q->B;
            a.Hq = q->Hq;
            a.Hkv = q->Hkv;
            a.G = q->Hq / q->Hkv;
            a.scale_log2 = scale_log2;
            a.tree = (const int32_t *)blob_dev;
            a.seg_off = L.segs;
            a.piece_off = L.pieces;
            a.wgseg_off = L.wgseg;
            a.wg0 = plan->launch_wg0[li];
            a.k_pool = k_pool;
            a.v_pool = v_pool;
            a.row_stride = row_stride;
            a.d = q->d;
            a.part_o = part_o;
            a.part_lse = part_lse;
            hipError_t e = launch_tree_prefix(a, q->dtype, q->d, plan->launch_nw[li],
                                              plan->launch_wgs[li], s);
            if (e != hipSuccess) return fail_hip(e);
        }

        // Sequence-first phase: private rows plus the merge of the partials.
        SuffixArgs a;
        std::memset(&a, 0, sizeof a);
        a.q = q->q;
        a.k_pool = k_pool;
        a.v_pool = v_pool;
        a.lens = seq_lens;
        a.B = q->B;
        a.Hq = q->Hq;
        a.Hkv = q->Hkv;
        a.has_suffix = 1;
        a.scale_log2 = scale_log2;
        a.dest = RowDest{o, lse, 0, 0, 0};
        a.tree = (const int32_t *)blob_dev;
        a.seq_tok_off = L.seq_tok;
        a.tok_rows_off = L.tok_rows;
        a.seq_src_off = L.seq_src;
        a.srcs_off = L.srcs;
        a.shared_off = L.shared;
        a.pool_rows = plan->pool_rows;
        a.part_o = part_o;
        a.part_lse = part_lse;
        const int64_t mb = cdiv(plan->max_private, HP_BLOCK_SIZE);
        const int nws = mb <= 2 ? 1 : mb <= 16 ? 2 : 4;
        hipError_t e = launch_tree_suffix(a, q->dtype, q->d, q->Hq / q->Hkv, nws, s);
        return e == hipSuccess ? HP_OK : fail_hip(e);
    });
}

hp_status hp_kv_append(const void *k_new, const void *v_new, const int32_t *rows, int32_t n,
                       int32_t Hkv, int32_t d, int32_t dtype, void *k_pool, void *v_pool,
                       int64_t pool_rows, int32_t *seq_lens, const int32_t *seq_idx,
                       int32_t num_seqs, void *stream) {
    return hp::guarded([&]() -> hp_status {
        if (n < 0 || Hkv <= 0 || d <= 0 || pool_rows < 0 || num_seqs < 0) return HP_ERR_INVALID_ARG;
        if (dtype < HP_F32 || dtype > HP_BF16) return HP_ERR_INVALID_ARG;
        if ((seq_lens == nullptr) != (seq_idx == nullptr)) return HP_ERR_INVALID_ARG;
        const int64_t row_bytes = (int64_t)Hkv * d * esize(dtype);
        if (row_bytes % 16) return HP_ERR_INVALID_ARG;
        if (n == 0) return HP_OK;
        if (!k_new || !v_new || !rows || !k_pool || !v_pool) return HP_ERR_NULL;
        if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) ||
            ((uintptr_t)rows & 3u) || ((uintptr_t)seq_lens & 3u) || ((uintptr_t)seq_idx & 3u))
            return HP_ERR_INVALID_ARG;
        if (cdiv(row_bytes / 16, 256) > 65535) return HP_ERR_UNSUPPORTED;
        hipError_t e = launch_kv_append(k_new, v_new, rows, n, row_bytes, k_pool, v_pool, pool_rows,
                                        seq_lens, seq_idx, num_seqs, (hipStream_t)stream);
        return e == hipSuccess ? HP_OK : fail_hip(e);
    });
}

}  // extern "C"
