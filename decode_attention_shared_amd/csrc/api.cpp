// Host side of the C ABI declared in hp_attn.h: argument and tree
// validation, work partitioning, workspace layout and kernel launches.
// No allocation, no synchronisation, no host-to-device copies: everything a
// kernel needs goes in its by-value arguments, so every entry point can be
// captured into a HIP graph.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <utility>
#include <cstdint>
#include <cstring>

#include "guard.hpp"
#include "host.hpp"

namespace {
thread_local int32_t g_last_hip_error = 0;
}  // namespace

namespace hp {
namespace host {

hp_status fail_hip(hipError_t e) {
    g_last_hip_error = (int32_t)e;
    return HP_ERR_HIP;
}

void plan_splits(const SplitItem *items, int count, int Hkv, int d, int nw, int64_t max_T,
                 SplitPlan *out, int cus) {
    const int64_t rows_per_wg = 32 * nw;
    const int64_t slots = (int64_t)cus * kWavesPerCU / nw;
    int64_t max_tiles = 0;
    for (int i = 0; i < count; ++i) {
        max_tiles = std::max<int64_t>(max_tiles, items[i].tiles);
        out[i].rowblocks = (int)cdiv(std::max<int64_t>(items[i].M, 1), rows_per_wg);
    }
    const int64_t T_hi = std::max<int64_t>(1, std::min<int64_t>(max_T, max_tiles));
    int64_t best_T = T_hi;
    double best_cost = 1e300;
    for (int64_t T = 1; T <= T_hi; ++T) {
        int64_t wgs = 0;
        double pbytes = 0;
        for (int i = 0; i < count; ++i) {
            const int64_t tiles = items[i].tiles;
            const int64_t ns = tiles ? cdiv(tiles, T) : 1;
            const int64_t units = (int64_t)Hkv * ns;
            const int64_t rb = out[i].rowblocks;
            wgs += (rb > 1 ? (int64_t)round_up(units, 8) : units) * rb;
            pbytes += (double)ns * items[i].rows * (d + 1) * 4.0 * 2.0;
        }
        const double cost = (double)cdiv(wgs, slots) * T + kPartialByteCost * pbytes;
        if (cost < best_cost) {
            best_cost = cost;
            best_T = T;
        }
    }
    for (int i = 0; i < count; ++i) {
        SplitPlan &sp = out[i];
        const int64_t tiles = items[i].tiles;
        const int64_t ns = tiles ? cdiv(tiles, best_T) : 1;
        sp.tiles_per_split = tiles ? (int)cdiv(tiles, ns) : 0;
        sp.nsplit = tiles ? (int)cdiv(tiles, sp.tiles_per_split) : 1;
        const int64_t units = (int64_t)Hkv * sp.nsplit;
        sp.units_padded = (int)(sp.rowblocks > 1 ? round_up(units, 8) : units);
        sp.wgs = sp.units_padded * sp.rowblocks;
    }
}

}  // namespace host
}  // namespace hp

namespace {

using namespace hp;
using namespace hp::host;

hp_status check_query(const hp_query *q) { return check_geometry(q, true); }

hp_status check_node(const hp_query *q, const hp_prefix_node *n) {
    if (!n) return HP_ERR_NULL;
    if (n->len < 0) return HP_ERR_INVALID_ARG;
    if (n->seq_begin < 0 || n->seq_begin >= n->seq_end || n->seq_end > q->B)
        return HP_ERR_INVALID_ARG;
    if (n->len == 0) return HP_OK;
    if (!n->k || !n->v) return HP_ERR_NULL;
    if (!aligned16(n->k) || !aligned16(n->v)) return HP_ERR_INVALID_ARG;
    const int64_t vec = 16 / esize(q->dtype);  // elements per 16 bytes
    if (n->stride_tok <= 0 || n->stride_head <= 0 || n->stride_tok % vec || n->stride_head % vec)
        return HP_ERR_INVALID_ARG;
    if (q->Hkv > 1 && n->stride_head < q->d) return HP_ERR_INVALID_ARG;  // heads would overlap
    return HP_OK;
}

hp_status check_tree(const hp_query *q, const hp_prefix_tree *t, int *total_nodes) {
    *total_nodes = 0;
    if (!t) return HP_OK;
    if (t->num_levels < 0 || t->num_levels > HP_MAX_LEVELS) return HP_ERR_UNSUPPORTED;
    int total = 0;
    for (int l = 0; l < t->num_levels; ++l) {
        if (t->nodes_per_level[l] < 0) return HP_ERR_INVALID_ARG;
        total += t->nodes_per_level[l];
        if (total > HP_MAX_NODES) return HP_ERR_UNSUPPORTED;
    }
    if (total > 0 && !t->nodes) return HP_ERR_NULL;
    int idx = 0;
    for (int l = 0; l < t->num_levels; ++l) {
        int prev_end = 0;
        for (int i = 0; i < t->nodes_per_level[l]; ++i, ++idx) {
            const hp_prefix_node *n = &t->nodes[idx];
            hp_status st = check_node(q, n);
            if (st != HP_OK) return st;
            if (n->seq_begin < prev_end) return HP_ERR_INVALID_ARG;  // unsorted or overlapping
            prev_end = n->seq_end;
        }
    }
    *total_nodes = total;
    return HP_OK;
}

hp_status check_kv(const hp_query *q, const hp_paged_kv *kv) {
    if (!kv) return HP_ERR_NULL;
    if (kv->block_size != HP_BLOCK_SIZE) return HP_ERR_UNSUPPORTED;
    if (kv->layout != HP_KV_NHD && kv->layout != HP_KV_HND) return HP_ERR_INVALID_ARG;
    if (kv->max_blocks < 1 || kv->num_blocks < 1) return HP_ERR_INVALID_ARG;
    if ((int64_t)kv->max_blocks * HP_BLOCK_SIZE > INT32_MAX) return HP_ERR_INVALID_ARG;
    if (!kv->k_pool || !kv->v_pool || !kv->block_table || !kv->seq_lens) return HP_ERR_NULL;
    if (!aligned16(kv->k_pool) || !aligned16(kv->v_pool)) return HP_ERR_INVALID_ARG;
    if (((uintptr_t)kv->block_table & 3u) || ((uintptr_t)kv->seq_lens & 3u))
        return HP_ERR_INVALID_ARG;
    return HP_OK;
}

hp_status check_out(const float *o, const float *lse) {
    if (!o) return HP_ERR_NULL;
    if (!aligned16(o) || ((uintptr_t)lse & 3u)) return HP_ERR_INVALID_ARG;
    return HP_OK;
}

// ---------------------------------------------------------------------------
// Work partitioning
// ---------------------------------------------------------------------------

struct NodePlan {
    int nsplit = 1, tiles_per_split = 0, rowblocks = 1, units_padded = 0, wgs = 0;
    int64_t rows = 0;  // (seq_end - seq_begin) * Hq output rows
};

// Plan of every node of one launch (a tree level).
struct LevelPlan {
    int nw = 1;
    int first = 0, count = 0;
    NodePlan nodes[HP_MAX_NODES];
};

// Splits of every node of one level (one launch): plan_splits over the nodes.
void plan_level(const hp_query &q, const hp_prefix_node *nodes, int count, LevelPlan &lp,
                int cus = kCUs) {
    const int G = q.Hq / q.Hkv;
    SplitItem items[HP_MAX_NODES];
    SplitPlan sp[HP_MAX_NODES];
    int64_t maxM = 1;
    for (int i = 0; i < count; ++i) {
        const int64_t nseq = nodes[i].seq_end - nodes[i].seq_begin;
        items[i] = SplitItem{nseq * G, nseq * q.Hq, cdiv(nodes[i].len, kTileKeys)};
        maxM = std::max<int64_t>(maxM, nseq * G);
    }
    lp.nw = choose_nw(maxM);
    plan_splits(items, count, q.Hkv, q.d, lp.nw, INT64_MAX, sp, cus);
    for (int i = 0; i < count; ++i) {
        NodePlan &np = lp.nodes[i];
        np.nsplit = sp[i].nsplit;
        np.tiles_per_split = sp[i].tiles_per_split;
        np.rowblocks = sp[i].rowblocks;
        np.units_padded = sp[i].units_padded;
        np.wgs = sp[i].wgs;
        np.rows = items[i].rows;
    }
    lp.count = count;
}

size_t node_ws_bytes(const NodePlan &np, int d) {
    return round_up((size_t)np.nsplit * np.rows * d * sizeof(float), kWsAlign) +
           round_up((size_t)np.nsplit * np.rows * sizeof(float), kWsAlign);
}

// Dynamic LDS (floats) for the suffix pass to stage the partials of the row
// that merges the most (0 when more than 32 KB or 64 LSEs would be needed):
// its 16-byte chunks rounded up to whole wave-wide transfers.
int32_t stage_floats(const MergeSrc *src, int nsrc, int G, int d) {
    if (nsrc <= 0) return 0;
    std::pair<int64_t, int64_t> ev[2 * kMaxMergeSrc];
    int ne = 0;
    for (int i = 0; i < nsrc; ++i) {
        ev[ne++] = {src[i].b0, src[i].nsplit};
        ev[ne++] = {src[i].b1, -(int64_t)src[i].nsplit};
    }
    std::sort(ev, ev + ne);  // at equal b the ends (negative) come first
    int64_t cur = 0, most = 0;
    for (int i = 0; i < ne; ++i) most = std::max(most, cur += ev[i].second);
    const int64_t chunks = most * G * d / 4;
    const int64_t floats = (chunks + 63) / 64 * 64 * 4;
    if (most * G > 64 || floats > 8192) return 0;
    return (int32_t)floats;
}

// Waves per (sequence, KV head) workgroup of the suffix pass.  More waves
// shorten each sequence's walk but leave more of them idle on short
// sequences; two waves measured best for suffixes of up to 16 blocks.
int suffix_waves(const hp_query &q, int64_t max_blocks) {
    const int64_t units = (int64_t)q.B * q.Hkv;
    if (max_blocks <= 2) return 1;
    // Few (sequence, KV head) units: more waves per unit keep enough blocks in
    // flight (measured: 512 units of up to 16 blocks run 30% faster on four).
    if (units <= 1024 && max_blocks > 4) return 4;
    return max_blocks <= 16 ? 2 : 4;
}

PrefixArgs base_prefix_args(const hp_query &q) {
    PrefixArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q.q;
    a.B = q.B;
    a.Hq = q.Hq;
    a.Hkv = q.Hkv;
    a.G = q.Hq / q.Hkv;
    a.scale_log2 = (float)((double)q.scale * 1.4426950408889634);
    return a;
}

PrefixNodeArg node_arg(const hp_prefix_node &n, const NodePlan &np, int wg_begin, RowDest dest) {
    PrefixNodeArg na;
    std::memset(&na, 0, sizeof na);
    na.k = n.k;
    na.v = n.v;
    na.stride_tok = n.stride_tok;
    na.stride_head = n.stride_head;
    na.len = n.len;
    na.seq_begin = n.seq_begin;
    na.seq_end = n.seq_end;
    na.nsplit = np.nsplit;
    na.tiles_per_split = np.tiles_per_split;
    na.rowblocks = np.rowblocks;
    na.units_padded = np.units_padded;
    na.wg_begin = wg_begin;
    na.dest = dest;
    return na;
}

// Launch the prefix pass for nodes [0, count) of one level, at most
// kMaxLaunchNodes per launch.  dests[i] is where node i's results go.
hp_status run_level(const hp_query &q, const hp_prefix_node *nodes, const LevelPlan &lp,
                    const RowDest *dests, hipStream_t s) {
    for (int c0 = 0; c0 < lp.count; c0 += kMaxLaunchNodes) {
        PrefixArgs a = base_prefix_args(q);
        int wg = 0;
        int64_t kv_bytes = 0;  // the launch's K/V (each node's keys and values once)
        const int c1 = std::min(lp.count, c0 + kMaxLaunchNodes);
        for (int i = c0; i < c1; ++i) {
            a.nodes[a.num_nodes++] = node_arg(nodes[i], lp.nodes[i], wg, dests[i]);
            wg += lp.nodes[i].wgs;
            kv_bytes += (int64_t)nodes[i].len * q.Hkv * q.d * esize(q.dtype) * 2;
        }
        if (wg == 0) continue;
        a.stream_kv = kv_bytes >= kLlcBytes ? 1 : 0;
        hipError_t e = launch_prefix(a, q.dtype, q.d, lp.nw, wg, s);
        if (e != hipSuccess) return fail_hip(e);
    }
    return HP_OK;
}

// kv may be NULL: no paged suffix (only private prefix nodes and partials).
SuffixArgs suffix_args(const hp_query &q, const hp_paged_kv *kv, RowDest dest) {
    SuffixArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q.q;
    a.B = q.B;
    a.Hq = q.Hq;
    a.Hkv = q.Hkv;
    a.scale_log2 = (float)((double)q.scale * 1.4426950408889634);
    a.dest = dest;
    if (!kv) return a;
    a.k_pool = kv->k_pool;
    a.v_pool = kv->v_pool;
    a.table = kv->block_table;
    a.lens = kv->seq_lens;
    a.max_blocks = kv->max_blocks;
    a.num_blocks = kv->num_blocks;
    a.kv_hnd = kv->layout == HP_KV_HND ? 1 : 0;
    a.has_suffix = 1;
    // K/V footprint: the pool, or what the block tables can reach if less.
    const int64_t blocks = std::min<int64_t>(kv->num_blocks, (int64_t)q.B * kv->max_blocks);
    const int64_t kv_bytes = blocks * kBlock * q.Hkv * q.d * esize(q.dtype) * 2;
    a.stream_kv = kv_bytes >= kLlcBytes ? 1 : 0;
    return a;
}

// Plan of a whole cascade step (shared by the size query and the run).
struct CascadePlan {
    int total_nodes = 0;  // nodes of the prefix pass (batched)
    int num_levels = 0;  // launch groups: tree levels, or one group holding every node
    LevelPlan levels[HP_MAX_LEVELS];
    bool has_suffix = false;
    bool conc = false;   // suffix pass beside the prefix pass, then one merge
    bool one_launch = false;  // conc, with both passes in one launch (step_pp_kernel)
    size_t node_off[HP_MAX_NODES];
    size_t suf_off = 0;  // concurrent plan: the suffix pass's (O, LSE) rows
    size_t bytes = 0;
    // The tree as the prefix pass sees it (the batched nodes, level-major) and
    // the nodes that each of their sequences reads in its suffix pass instead.
    int tree_levels = 0;
    int32_t batched_per_level[HP_MAX_LEVELS] = {};
    hp_prefix_node batched[HP_MAX_NODES];
    int nseg = 0;
    PrivSeg seg[HP_MAX_NODES];
    int64_t seg_blocks = 0;  // blocks of private nodes a sequence reads, at most
    hp_prefix_tree view() const {
        hp_prefix_tree t;
        std::memset(&t, 0, sizeof t);
        t.num_levels = tree_levels;
        for (int l = 0; l < tree_levels; ++l) t.nodes_per_level[l] = batched_per_level[l];
        t.nodes = batched;
        t.share_min = 1;
        return t;
    }
    bool suffix_pass() const { return has_suffix || nseg > 0; }
};

// The suffix pass's arguments for the plan: the paged suffix (if any) and
// the private prefix nodes.
SuffixArgs plan_suffix_args(const hp_query &q, const hp_paged_kv *kv, const CascadePlan &cp,
                            RowDest dest) {
    SuffixArgs a = suffix_args(q, kv, dest);
    a.nseg = cp.nseg;
    for (int i = 0; i < cp.nseg; ++i) a.seg[i] = cp.seg[i];
    return a;
}

int plan_suffix_waves(const hp_query &q, const hp_paged_kv *kv, const CascadePlan &cp) {
    return suffix_waves(q, (kv ? kv->max_blocks : 0) + cp.seg_blocks);
}

// Lay out the prefix launches of the tree for `cus` compute units; returns
// the workspace bytes of their partials.
size_t plan_prefix(const hp_query *q, const hp_prefix_tree *tree, CascadePlan &cp, int cus) {
    size_t off = 0;
    int idx = 0;
    const int levels = tree ? tree->num_levels : 0;
    // The levels' prefix passes are independent (only the merge needs them
    // all): launch every node together when their stacked row counts call
    // for row blocks within a factor of two of each other, so one launch
    // fills the GPU instead of one per level (each with its own pipeline
    // fill and partial write-out); otherwise one launch per level.
    bool joint = levels > 1 && cp.total_nodes <= kMaxLaunchNodes;
    if (joint) {
        const int G = q->Hq / q->Hkv;
        int nw_max = 1, nw_min = 8;
        for (int i = 0; i < cp.total_nodes; ++i) {
            const hp_prefix_node &n = tree->nodes[i];
            const int nw = choose_nw((int64_t)(n.seq_end - n.seq_begin) * G);
            nw_max = std::max(nw_max, nw);
            nw_min = std::min(nw_min, nw);
        }
        joint = nw_min * 2 >= nw_max;
    }
    cp.num_levels = joint ? 1 : levels;  // launch groups
    for (int l = 0; l < cp.num_levels; ++l) {
        LevelPlan &lp = cp.levels[l];
        lp.first = idx;
        plan_level(*q, tree->nodes + idx, joint ? cp.total_nodes : tree->nodes_per_level[l], lp,
                   cus);
        for (int i = 0; i < lp.count; ++i) {
            cp.node_off[idx + i] = off;
            off += node_ws_bytes(lp.nodes[i], q->d);
        }
        idx += lp.count;
    }
    return off;
}

// Plan of a whole cascade step (shared by the size query and the run).
// mode: 0 the passes one after the other on one stream; 1 side by side when
// the plan expects a gain; 2 side by side whenever there is a prefix and a
// suffix.
// Both passes in one launch (step_pp_kernel) for a plan whose prefix is laid
// out for kConcCUs: one prefix launch of the ping-pong kernel, no private
// nodes, G in {1, 2, 4}, 16-bit, d = 128, K/V of both passes within the
// last-level cache (the kernel's loads are plain), and every suffix wave's
// units and blocks within its LDS tables (kFatMaxRows, kFatMaxSteps).
int one_launch_suffix_wgs(const CascadePlan &cp) {
    int wg = 0;
    const LevelPlan &lp = cp.levels[0];
    for (int i = 0; i < lp.count; ++i) wg += lp.nodes[i].wgs;
    return kCUs - wg;
}

bool one_launch_ok(const hp_query *q, const hp_paged_kv *kv, const CascadePlan &cp) {
    if (!kv || cp.nseg > 0 || cp.num_levels != 1 || q->B <= 0) return false;
    const int G = q->Hq / q->Hkv;
    const LevelPlan &lp = cp.levels[0];
    if (lp.count < 1 || lp.count > kMaxLaunchNodes || !step_supported(q->dtype, q->d, G, lp.nw))
        return false;
    if (kv->max_blocks < 1 || kv->num_blocks < 1) return false;
    if ((int64_t)q->B * q->Hq >= (int64_t(1) << 24)) return false;
    const hp_prefix_tree view = cp.view();
    int64_t kv_bytes = 0;
    for (int i = 0; i < lp.count; ++i) {
        const hp_prefix_node &n = view.nodes[lp.first + i];
        if ((int64_t)kTileKeys * n.stride_tok + q->d > (int64_t)INT32_MAX) return false;
        kv_bytes += (int64_t)n.len * q->Hkv * q->d * esize(q->dtype) * 2;
    }
    if (kv_bytes >= kLlcBytes) return false;
    if (suffix_args(*q, kv, RowDest{}).stream_kv) return false;
    const int swgs = one_launch_suffix_wgs(cp);
    if (swgs < 32) return false;
    const int64_t nsp = cdiv(kv->max_blocks, kFatSplitBlocks);
    if ((int64_t)q->B * q->Hq * nsp >= (int64_t(1) << 24)) return false;
    const int64_t per_wave = cdiv((int64_t)q->B * q->Hkv * nsp, (int64_t)swgs * 8);
    return per_wave * G <= kFatMaxRows && per_wave * kFatSplitBlocks <= kFatMaxSteps - 4;
}

// The one-launch plan's suffix items per (sequence, KV head): each covers
// kFatSplitBlocks blocks and has its own slot of (O, LSE) rows.
int64_t one_launch_splits(const hp_paged_kv *kv) { return cdiv(kv->max_blocks, kFatSplitBlocks); }

// The prefix pass's compute units beside the suffix pass: kConcCUs, or
// kConcCUsHeavy when the suffix pass's K/V bound (suffix_kv bytes) is at least
// kConcHeavyRatio times the batched nodes' K/V.
int conc_prefix_cus(const hp_query *q, const CascadePlan &cp, int64_t suffix_kv) {
    int64_t prefix_kv = 0;
    for (int i = 0; i < cp.total_nodes; ++i)
        prefix_kv += (int64_t)cp.batched[i].len * q->Hkv * q->d * esize(q->dtype) * 2;
    return suffix_kv >= kConcHeavyRatio * prefix_kv ? kConcCUsHeavy : kConcCUs;
}

hp_status plan_cascade(const hp_query *q, const hp_prefix_tree *tree, const hp_paged_kv *kv,
                       int mode, CascadePlan &cp, bool batch_all = false) {
    if (mode < 0 || mode > 3) return HP_ERR_INVALID_ARG;
    hp_status st = check_query(q);
    if (st != HP_OK) return st;
    int total = 0;
    st = check_tree(q, tree, &total);
    if (st != HP_OK) return st;
    if (tree && tree->share_min < 0) return HP_ERR_INVALID_ARG;
    if (kv) {
        st = check_kv(q, kv);
        if (st != HP_OK) return st;
    }
    cp.has_suffix = kv != nullptr;
    // Which nodes the prefix pass batches (the rest are read by each of their
    // sequences in the suffix pass): share_min 0 asks the batching policy per
    // node, k >= 1 batches the nodes over at least k sequences.
    if (tree) {
        const int G = q->Hq / q->Hkv;
        cp.tree_levels = tree->num_levels;
        for (int l = 0, idx = 0; l < tree->num_levels; ++l) {
            int64_t level_blocks = 0;
            for (int i = 0; i < tree->nodes_per_level[l]; ++i, ++idx) {
                const hp_prefix_node &n = tree->nodes[idx];
                const int64_t nseq = (int64_t)n.seq_end - n.seq_begin;
                const bool batch = batch_all ||
                    (tree->share_min == 0 ? share_decision(q->dtype, q->d, G, n.len, nseq)
                                          : nseq >= tree->share_min);
                if (batch) {
                    cp.batched[cp.total_nodes++] = n;
                    ++cp.batched_per_level[l];
                } else if (n.len > 0 && nseq > 0) {
                    cp.seg[cp.nseg++] = PrivSeg{n.k, n.v, n.stride_tok, n.stride_head,
                                                n.len, n.seq_begin, n.seq_end, 0};
                    level_blocks = std::max<int64_t>(level_blocks, cdiv(n.len, kBlock));
                }
            }
            cp.seg_blocks += level_blocks;
        }
    }
    (void)total;
    const hp_prefix_tree bt = cp.view();
    cp.bytes = plan_prefix(q, tree ? &bt : nullptr, cp, kCUs);
    // The suffix pass beside the prefix pass: the prefix is planned for
    // kConcCUs compute units, the suffix writes its own (O, LSE) rows and one
    // merge combines them with the prefix partials.
    if (cp.has_suffix && cp.total_nodes > 0 && q->B > 0 && mode != 0) {
        CascadePlan alt = cp;
        size_t pbytes = plan_prefix(q, tree ? &bt : nullptr, alt, kConcCUs);
        bool pays = (int64_t)q->B * q->Hkv >= kConcMinUnits;
        for (int l = 0; l < alt.num_levels && pays; ++l)
            for (int i = 0; i < alt.levels[l].count; ++i)
                pays = pays && alt.levels[l].nodes[i].tiles_per_split >= kConcMinTiles;
        // Both passes in one launch (no second stream): in mode 1 for MHA steps
        // whose suffix is too small for the second stream's fork and join to pay
        // (with several query heads per KV head a suffix wave's unit is too much
        // work for one wave, and the serial plan is faster).
        const bool want_one = mode == 3 || (mode == 1 && !pays && q->Hq == q->Hkv &&
                                            (int64_t)q->B * q->Hkv < kConcMinUnits);
        CascadePlan one_plan = cp;
        size_t one_pbytes = 0;
        bool one = false;
        if (want_one) {
            one_pbytes = plan_prefix(q, tree ? &bt : nullptr, one_plan, kOneLaunchCUs);
            one = one_launch_ok(q, kv, one_plan);
        }
        if (one) {
            alt = one_plan;
            pbytes = one_pbytes;
        } else {
            const int64_t suffix_kv =
                (int64_t)q->B * kv->max_blocks * kBlock * q->Hkv * q->d * esize(q->dtype) * 2;
            const int cus = conc_prefix_cus(q, cp, suffix_kv);
            if (cus != kConcCUs) {  // the gain test above stays the one at kConcCUs
                alt = cp;
                pbytes = plan_prefix(q, tree ? &bt : nullptr, alt, cus);
            }
        }
        if (mode == 2 || (mode == 1 && pays) || one) {
            // the suffix rows: one slot (second stream) or one per item split
            const size_t nsp = one ? (size_t)one_launch_splits(kv) : 1;
            cp = alt;
            cp.conc = true;
            cp.one_launch = one;
            cp.suf_off = pbytes;
            cp.bytes = pbytes +
                       round_up(nsp * q->B * q->Hq * q->d * sizeof(float), kWsAlign) +
                       round_up(nsp * q->B * q->Hq * sizeof(float), kWsAlign);
        }
    }
    return HP_OK;
}

// Workspace that serves every mode: the largest of the serial plan, the
// always-side-by-side plan and the one-launch plan.
hp_status cascade_ws_bytes(const hp_query *q, const hp_prefix_tree *tree, const hp_paged_kv *kv,
                           size_t *bytes) {
    CascadePlan serial, conc, one;
    hp_status st = plan_cascade(q, tree, kv, 0, serial);
    if (st != HP_OK) return st;
    st = plan_cascade(q, tree, kv, 2, conc);
    if (st != HP_OK) return st;
    st = plan_cascade(q, tree, kv, 3, one);
    if (st != HP_OK) return st;
    *bytes = std::max({serial.bytes, conc.bytes, one.bytes});
    return HP_OK;
}

}  // namespace

extern "C" {

static_assert(sizeof(hp_status) == sizeof(int32_t), "hp_status is a 32-bit int at the ABI");

const char *hp_status_string(hp_status s) {
    // A C caller may pass any int; read it as one (a C++ load of an enum value
    // outside its enumerators' range is undefined).
    int32_t v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
    case HP_OK: return "ok";
    case HP_ERR_NULL: return "a required pointer is NULL";
    case HP_ERR_INVALID_ARG: return "invalid argument (size, range, stride or alignment)";
    case HP_ERR_UNSUPPORTED: return "unsupported (outside the implemented domain)";
    case HP_ERR_WORKSPACE: return "workspace missing or too small";
    case HP_ERR_HIP: return "HIP launch failed";
    case HP_ERR_CAPACITY:
        return "capacity exceeded (pool, plan buffer, output array or fixed scratch too small)";
    case HP_ERR_HOST: return "host-side failure (out of host memory)";
    default: return "unknown status";
    }
}

int32_t hp_last_hip_error(void) { return g_last_hip_error; }

const char *hp_version(void) { return "hp_attn 0.1 gfx950"; }

// ------------------------------- prefix -----------------------------------

hp_status hp_prefix_attn_workspace_size(const hp_query *q, const hp_prefix_node *node,
                                        size_t *bytes) {
    return hp::guarded([&]() -> hp_status {
        if (!bytes) return HP_ERR_NULL;
        hp_status st = check_query(q);
        if (st != HP_OK) return st;
        st = check_node(q, node);
        if (st != HP_OK) return st;
        LevelPlan lp;
        plan_level(*q, node, 1, lp);
        *bytes = lp.nodes[0].nsplit > 1 ? node_ws_bytes(lp.nodes[0], q->d) : 0;
        return HP_OK;
    });
}

hp_status hp_prefix_attn(const hp_query *q, const hp_prefix_node *node, float *o, float *lse,
                         void *ws, size_t ws_bytes, void *stream) {
    return hp::guarded([&]() -> hp_status {
        hp_status st = check_query(q);
        if (st != HP_OK) return st;
        st = check_node(q, node);
        if (st != HP_OK) return st;
        st = check_out(o, lse);
        if (st != HP_OK) return st;
        LevelPlan lp;
        plan_level(*q, node, 1, lp);
        const NodePlan &np = lp.nodes[0];
        hipStream_t s = (hipStream_t)stream;
        if (np.nsplit == 1) {
            const RowDest dest{o, lse, 0, 0, 0};
            return run_level(*q, node, lp, &dest, s);
        }
        const size_t need = node_ws_bytes(np, q->d);
        if (!ws || ws_bytes < need || !aligned16(ws)) return HP_ERR_WORKSPACE;
        float *wo = (float *)ws;
        float *wl =
            (float *)((char *)ws + round_up((size_t)np.nsplit * np.rows * q->d * 4, kWsAlign));
        const RowDest dest{wo, wl, np.rows * q->d, np.rows, node->seq_begin};
        st = run_level(*q, node, lp, &dest, s);
        if (st != HP_OK) return st;
        MergeArgs m;
        std::memset(&m, 0, sizeof m);
        m.src[0] = MergeSrc{wo, wl, np.rows * q->d, np.rows, np.nsplit, 0, node->seq_begin,
                            node->seq_end};
        m.nsrc = 1;
        m.Hq = q->Hq;
        m.row_b0 = node->seq_begin;
        m.row_b1 = node->seq_end;
        m.o = o;
        m.lse = lse;
        hipError_t e = launch_merge(m, q->d, s);
        return e == hipSuccess ? HP_OK : fail_hip(e);
    });
}

// ------------------------------- suffix -----------------------------------

hp_status hp_suffix_decode_workspace_size(const hp_query *q, const hp_paged_kv *kv,
                                          size_t *bytes) {
    return hp::guarded([&]() -> hp_status {
        if (!bytes) return HP_ERR_NULL;
        hp_status st = check_query(q);
        if (st != HP_OK) return st;
        st = check_kv(q, kv);
        if (st != HP_OK) return st;
        *bytes = 0;  // the waves of one (sequence, KV head) combine in LDS
        return HP_OK;
    });
}

hp_status hp_suffix_decode(const hp_query *q, const hp_paged_kv *kv, float *o, float *lse,
                           void *ws, size_t ws_bytes, void *stream) {
    return hp::guarded([&]() -> hp_status {
        (void)ws;
        (void)ws_bytes;
        hp_status st = check_query(q);
        if (st != HP_OK) return st;
        st = check_kv(q, kv);
        if (st != HP_OK) return st;
        st = check_out(o, lse);
        if (st != HP_OK) return st;
        if (q->B == 0) return HP_OK;
        const SuffixArgs a = suffix_args(*q, kv, RowDest{o, lse, 0, 0, 0});
        hipError_t e = launch_suffix(a, q->dtype, q->d, q->Hq / q->Hkv,
                                     suffix_waves(*q, kv->max_blocks), (hipStream_t)stream);
        return e == hipSuccess ? HP_OK : fail_hip(e);
    });
}

// -------------------------------- merge -----------------------------------

hp_status hp_lse_merge(int32_t n, const float *const *o_in, const float *const *lse_in, float *o,
                       float *lse, int64_t rows, int32_t d, void *stream) {
    return hp::guarded([&]() -> hp_status {
        if (!o_in || !lse_in || !o) return HP_ERR_NULL;
        if (n < 1 || n > HP_MAX_MERGE || rows < 0) return HP_ERR_INVALID_ARG;
        if (d != 64 && d != 128) return HP_ERR_UNSUPPORTED;
        if (!aligned16(o) || ((uintptr_t)lse & 3u)) return HP_ERR_INVALID_ARG;
        const uintptr_t olo = (uintptr_t)o, ohi = olo + (uintptr_t)rows * d * sizeof(float);
        const uintptr_t llo = (uintptr_t)lse, lhi = llo + (uintptr_t)rows * sizeof(float);
        for (int i = 0; i < n; ++i) {
            if (!o_in[i] || !lse_in[i]) return HP_ERR_NULL;
            if (!aligned16(o_in[i]) || ((uintptr_t)lse_in[i] & 3u)) return HP_ERR_INVALID_ARG;
            const uintptr_t a0 = (uintptr_t)o_in[i], a1 = a0 + (uintptr_t)rows * d * sizeof(float);
            const uintptr_t b0 = (uintptr_t)lse_in[i], b1 = b0 + (uintptr_t)rows * sizeof(float);
            auto overlap = [](uintptr_t x0, uintptr_t x1, uintptr_t y0, uintptr_t y1) {
                return x0 < y1 && y0 < x1;
            };
            if (rows > 0 && (overlap(olo, ohi, a0, a1) || overlap(olo, ohi, b0, b1) ||
                             (lse && (overlap(llo, lhi, a0, a1) || overlap(llo, lhi, b0, b1)))))
                return HP_ERR_INVALID_ARG;
        }
        if (rows == 0) return HP_OK;
        MergeArgs m;
        std::memset(&m, 0, sizeof m);
        for (int i = 0; i < n; ++i) m.src[i] = MergeSrc{o_in[i], lse_in[i], 0, 0, 1, 0, 0, rows};
        m.nsrc = n;
        m.Hq = 1;
        m.row_b0 = 0;
        m.row_b1 = rows;
        m.o = o;
        m.lse = lse;
        hipError_t e = launch_merge(m, d, (hipStream_t)stream);
        return e == hipSuccess ? HP_OK : fail_hip(e);
    });
}

// ------------------------------- cascade ----------------------------------

hp_status hp_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
    return hp::guarded([&]() -> hp_status {
        if (!sink || (!buf && bytes > 0)) return HP_ERR_NULL;
        if (bytes % 16 || !aligned16(buf) || ((uintptr_t)sink & 3u)) return HP_ERR_INVALID_ARG;
        if (bytes > (size_t)INT64_MAX) return HP_ERR_INVALID_ARG;
        hipError_t e = launch_read_probe(buf, (int64_t)bytes, sink, HP_READ_PROBE_WGS,
                                         (hipStream_t)stream);
        return e == hipSuccess ? HP_OK : fail_hip(e);
    });
}

hp_status hp_cascade_overlap_plan(const hp_query *q, const hp_prefix_tree *tree,
                                  const hp_paged_kv *kv, int32_t mode, int32_t *overlapped) {
    return hp::guarded([&]() -> hp_status {
        if (!overlapped) return HP_ERR_NULL;
        CascadePlan cp;
        hp_status st = plan_cascade(q, tree, kv, mode, cp);
        if (st != HP_OK) return st;
        *overlapped = cp.one_launch ? 2 : cp.conc ? 1 : 0;
        return HP_OK;
    });
}

hp_status hp_cascade_workspace_size(const hp_query *q, const hp_prefix_tree *tree,
                                    const hp_paged_kv *kv, size_t *bytes) {
    return hp::guarded([&]() -> hp_status {
        if (!bytes) return HP_ERR_NULL;
        return cascade_ws_bytes(q, tree, kv, bytes);
    });
}

}  // extern "C"

namespace {

hp_status record(void *const *events, int i, hipStream_t s) {
    if (!events || !events[i]) return HP_OK;
    hipError_t e = hipEventRecord((hipEvent_t)events[i], s);
    return e == hipSuccess ? HP_OK : fail_hip(e);
}

hp_status run_prefix_levels(const hp_query *q, const CascadePlan &cp, char *base, MergeArgs &m,
                            hipStream_t s);

// Both passes in one launch on s (step_pp_kernel: the prefix workgroups of
// the plan's single prefix launch, then one suffix workgroup per compute
// unit they leave free), then one merge of every prefix partial with the
// suffix rows on s.
hp_status cascade_one_launch(const hp_query *q, const hp_paged_kv *kv, const CascadePlan &cp,
                             float *o, float *lse, char *base, hipStream_t s,
                             void *const *events) {
    const int64_t nsp = one_launch_splits(kv);
    float *so = (float *)(base + cp.suf_off);
    float *sl = (float *)((char *)so + round_up((size_t)nsp * q->B * q->Hq * q->d * sizeof(float),
                                                kWsAlign));
    const hp_prefix_tree view = cp.view();
    const LevelPlan &lp = cp.levels[0];
    MergeArgs m;
    std::memset(&m, 0, sizeof m);
    PrefixArgs a = base_prefix_args(*q);
    int wg = 0;
    for (int i = 0; i < lp.count; ++i) {
        const NodePlan &np = lp.nodes[i];
        const hp_prefix_node &nd = view.nodes[lp.first + i];
        float *wo = (float *)(base + cp.node_off[lp.first + i]);
        float *wl = (float *)((char *)wo +
                              round_up((size_t)np.nsplit * np.rows * q->d * 4, kWsAlign));
        a.nodes[a.num_nodes++] =
            node_arg(nd, np, wg, RowDest{wo, wl, np.rows * q->d, np.rows, nd.seq_begin});
        m.src[m.nsrc++] = MergeSrc{wo, wl, np.rows * q->d, np.rows, np.nsplit, 0,
                                   nd.seq_begin, nd.seq_end};
        wg += np.wgs;
    }
    a.stream_kv = 0;  // one_launch_ok: the launch's K/V are within the last-level cache
    const SuffixArgs sa = suffix_args(*q, kv, RowDest{so, sl, 0, 0, 0});
    FatSuffixArgs f;
    std::memset(&f, 0, sizeof f);
    f.q = q->q;
    f.k_pool = kv->k_pool;
    f.v_pool = kv->v_pool;
    f.table = kv->block_table;
    f.lens = kv->seq_lens;
    f.o = so;
    f.lse = sl;
    f.B = q->B;
    f.Hq = q->Hq;
    f.Hkv = q->Hkv;
    f.max_blocks = kv->max_blocks;
    f.num_blocks = kv->num_blocks;
    f.kv_hnd = sa.kv_hnd;
    f.scale_log2 = sa.scale_log2;
    f.prefix_wgs = wg;
    f.nsplit = (int32_t)nsp;
    hp_status st = record(events, 0, s);
    if (st != HP_OK) return st;
    if ((st = record(events, 4, s)) != HP_OK) return st;
    hipError_t e = launch_step(a, wg, f, one_launch_suffix_wgs(cp), q->dtype, q->d,
                               q->Hq / q->Hkv, s);
    if (e != hipSuccess) return fail_hip(e);
    if ((st = record(events, 1, s)) != HP_OK) return st;
    if ((st = record(events, 2, s)) != HP_OK) return st;
    // the items' rows: only the splits that hold blocks of the sequence are read,
    // and a length out of range makes the row NaN
    const int64_t bhq = (int64_t)q->B * q->Hq;
    m.src[m.nsrc++] = MergeSrc{so, sl, bhq * q->d, bhq, (int32_t)nsp, kFatSplitBlocks, 0, q->B};
    m.lens = kv->seq_lens;
    m.max_len = kv->max_blocks * kBlock;
    m.Hq = q->Hq;
    m.row_b0 = 0;
    m.row_b1 = q->B;
    m.o = o;
    m.lse = lse;
    if ((e = launch_merge(m, q->d, s)) != hipSuccess) return fail_hip(e);
    return record(events, 3, s);
}

// Suffix pass beside the prefix pass: fork the caller's side stream from s,
// prefix launches on s, the suffix pass (its own (O, LSE) rows, no merge) on
// the side stream, join, then one merge of every prefix partial with the
// suffix rows on s.
hp_status cascade_concurrent(const hp_query *q, const hp_prefix_tree *tree,
                             const hp_paged_kv *kv, const CascadePlan &cp, float *o, float *lse,
                             char *base, hipStream_t s, const hp_overlap &ov, void *const *events) {
    float *so = (float *)(base + cp.suf_off);
    float *sl = (float *)((char *)so +
                          round_up((size_t)q->B * q->Hq * q->d * sizeof(float), kWsAlign));
    const hipStream_t ss = (hipStream_t)ov.side_stream;
    const hipEvent_t fork = (hipEvent_t)ov.fork_event, join = (hipEvent_t)ov.join_event;
    hipError_t e;
    if ((e = hipEventRecord(fork, s)) != hipSuccess) return fail_hip(e);
    if ((e = hipStreamWaitEvent(ss, fork, 0)) != hipSuccess) return fail_hip(e);
    hp_status st = record(events, 0, s);  // right before the first prefix launch
    if (st != HP_OK) return st;
    MergeArgs m;
    std::memset(&m, 0, sizeof m);
    if ((st = run_prefix_levels(q, cp, base, m, s)) != HP_OK) return st;
    if ((st = record(events, 1, s)) != HP_OK) return st;
    SuffixArgs a = plan_suffix_args(*q, kv, cp, RowDest{so, sl, 0, 0, 0});
    if ((st = record(events, 4, ss)) != HP_OK) return st;
    e = launch_suffix(a, q->dtype, q->d, q->Hq / q->Hkv, plan_suffix_waves(*q, kv, cp), ss);
    if (e != hipSuccess) return fail_hip(e);
    if ((st = record(events, 2, ss)) != HP_OK) return st;
    if ((e = hipEventRecord(join, ss)) != hipSuccess) return fail_hip(e);
    if ((e = hipStreamWaitEvent(s, join, 0)) != hipSuccess) return fail_hip(e);
    m.src[m.nsrc++] = MergeSrc{so, sl, 0, 0, 1, 0, 0, q->B};
    m.Hq = q->Hq;
    m.row_b0 = 0;
    m.row_b1 = q->B;
    m.o = o;
    m.lse = lse;
    if ((e = launch_merge(m, q->d, s)) != hipSuccess) return fail_hip(e);
    return record(events, 3, s);
}

// Prefix pass of every tree level (root first), results into the cascade
// plan's workspace slots; m receives one merge source per node.
hp_status run_prefix_levels(const hp_query *q, const CascadePlan &cp, char *base, MergeArgs &m,
                            hipStream_t s) {
    const hp_prefix_tree view = cp.view();
    const hp_prefix_tree *tree = &view;
    for (int l = 0; l < cp.num_levels; ++l) {
        const LevelPlan &lp = cp.levels[l];
        RowDest dests[HP_MAX_NODES];
        for (int i = 0; i < lp.count; ++i) {
            const NodePlan &np = lp.nodes[i];
            const hp_prefix_node &nd = tree->nodes[lp.first + i];
            float *wo = (float *)(base + cp.node_off[lp.first + i]);
            float *wl = (float *)((char *)wo +
                                  round_up((size_t)np.nsplit * np.rows * q->d * 4, kWsAlign));
            dests[i] = RowDest{wo, wl, np.rows * q->d, np.rows, nd.seq_begin};
            m.src[m.nsrc++] = MergeSrc{wo, wl, np.rows * q->d, np.rows, np.nsplit, 0,
                                       nd.seq_begin, nd.seq_end};
        }
        hp_status st = run_level(*q, tree->nodes + lp.first, lp, dests, s);
        if (st != HP_OK) return st;
    }
    return HP_OK;
}

hp_status cascade_impl(const hp_query *q, const hp_prefix_tree *tree, const hp_paged_kv *kv,
                       float *o, float *lse, void *ws, size_t ws_bytes, void *stream,
                       const hp_overlap *ov, void *const *events) {
    CascadePlan cp;
    hp_status st = plan_cascade(q, tree, kv, ov ? ov->mode : 0, cp);
    if (st != HP_OK) return st;
    st = check_out(o, lse);
    if (st != HP_OK) return st;
    if (cp.conc && !cp.one_launch) {
        if (!ov->side_stream || !ov->fork_event || !ov->join_event) return HP_ERR_NULL;
        if (ov->side_stream == stream) return HP_ERR_INVALID_ARG;
    }
    if (q->B == 0) return HP_OK;
    if (cp.bytes > 0 && (!ws || ws_bytes < cp.bytes || !aligned16(ws))) return HP_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char *base = (char *)ws;
    if (cp.one_launch) return cascade_one_launch(q, kv, cp, o, lse, base, s, events);
    if (cp.conc) return cascade_concurrent(q, tree, kv, cp, o, lse, base, s, *ov, events);
    if ((st = record(events, 0, s)) != HP_OK) return st;

    MergeArgs m;
    std::memset(&m, 0, sizeof m);
    if ((st = run_prefix_levels(q, cp, base, m, s)) != HP_OK) return st;
    if ((st = record(events, 1, s)) != HP_OK) return st;
    if (cp.suffix_pass()) {
        // Suffix pass (paged suffix and private prefix nodes) with the merge of
        // every level's partials fused in.
        SuffixArgs a = plan_suffix_args(*q, kv, cp, RowDest{o, lse, 0, 0, 0});
        a.nsrc = m.nsrc;
        for (int i = 0; i < m.nsrc; ++i) a.src[i] = m.src[i];
        a.stage_floats = stage_floats(m.src, m.nsrc, q->Hq / q->Hkv, q->d);
        if ((st = record(events, 4, s)) != HP_OK) return st;
        hipError_t e = launch_suffix(a, q->dtype, q->d, q->Hq / q->Hkv,
                                     plan_suffix_waves(*q, kv, cp), s);
        if (e != hipSuccess) return fail_hip(e);
        if ((st = record(events, 2, s)) != HP_OK) return st;
    } else {
        // Prefix only: one n-way merge of every level's splits.
        if ((st = record(events, 2, s)) != HP_OK) return st;
        m.Hq = q->Hq;
        m.row_b0 = 0;
        m.row_b1 = q->B;
        m.o = o;
        m.lse = lse;
        hipError_t e = launch_merge(m, q->d, s);
        if (e != hipSuccess) return fail_hip(e);
    }
    return record(events, 3, s);
}

// ------------------------- shared-context streams -------------------------

hp_status check_stream_rows(const hp_query *q, const hp_stream_rows *r) {
    if (!r) return HP_ERR_NULL;
    if (r->num_requests < 1 || r->row_cap < 1 || r->pool_rows < 1) return HP_ERR_INVALID_ARG;
    if (r->pool_rows > INT32_MAX) return HP_ERR_INVALID_ARG;  // pool rows are int32 entries
    if (!r->k_pool || !r->v_pool || !r->row_slots || !r->slot_sid || !r->row_len || !r->q_req ||
        !r->q_sid)
        return HP_ERR_NULL;
    if (!aligned16(r->k_pool) || !aligned16(r->v_pool)) return HP_ERR_INVALID_ARG;
    for (const void *p : {(const void *)r->row_slots, (const void *)r->slot_sid,
                          (const void *)r->row_len, (const void *)r->q_req,
                          (const void *)r->q_sid})
        if ((uintptr_t)p & 3u) return HP_ERR_INVALID_ARG;
    (void)q;
    return HP_OK;
}

// Workspace of a stream step: the cascade plan's prefix partials, then the
// per-query visible-row counts and tables.
struct StreamPlan {
    CascadePlan cp;
    bool conc = false;      // the stream pass beside the document's prefix pass
    size_t suf_off = 0;     // conc: the stream pass's own (O, LSE) rows
    size_t len_off = 0, table_off = 0, bytes = 0;
};

// mode as hp_overlap.mode 0-2: the stream selection and the stream pass run
// on the second stream beside the prefix pass (planned for kConcCUs) by the
// same rule as the cascade step's.
hp_status plan_stream(const hp_query *q, const hp_prefix_tree *doc, const hp_stream_rows *r,
                      StreamPlan &sp, int mode = 0) {
    if (mode < 0 || mode > 2) return HP_ERR_INVALID_ARG;
    hp_status st = plan_cascade(q, doc, nullptr, 0, sp.cp, /*batch_all=*/true);
    if (st != HP_OK) return st;
    if ((st = check_stream_rows(q, r)) != HP_OK) return st;
    if (mode != 0 && sp.cp.total_nodes > 0 && q->B > 0) {
        CascadePlan alt = sp.cp;
        const hp_prefix_tree bt = alt.view();
        size_t pbytes = plan_prefix(q, &bt, alt, kConcCUs);
        bool pays = (int64_t)q->B * q->Hkv >= kConcMinUnits;
        for (int l = 0; l < alt.num_levels && pays; ++l)
            for (int i = 0; i < alt.levels[l].count; ++i)
                pays = pays && alt.levels[l].nodes[i].tiles_per_split >= kConcMinTiles;
        const int64_t stream_kv =
            (int64_t)q->B * r->row_cap * q->Hkv * q->d * esize(q->dtype) * 2;
        const int cus = conc_prefix_cus(q, sp.cp, stream_kv);
        if (cus != kConcCUs) {  // the gain test above stays the one at kConcCUs
            alt = sp.cp;
            pbytes = plan_prefix(q, &bt, alt, cus);
        }
        if (mode == 2 || pays) {
            sp.cp = alt;
            sp.conc = true;
            sp.suf_off = pbytes;
            sp.cp.bytes = pbytes + round_up((size_t)q->B * q->Hq * q->d * sizeof(float), kWsAlign) +
                          round_up((size_t)q->B * q->Hq * sizeof(float), kWsAlign);
        }
    }
    sp.len_off = round_up(sp.cp.bytes, kWsAlign);
    sp.table_off = sp.len_off + round_up((size_t)q->B * 4, kWsAlign);
    sp.bytes = sp.table_off + round_up((size_t)q->B * (size_t)r->row_cap * 4, kWsAlign);
    return HP_OK;
}

// One stream-decode step (hp_stream_decode, or _overlap with ov).
hp_status stream_impl(const hp_query *q, const hp_prefix_tree *doc, const hp_stream_rows *rows,
                      float *o, float *lse, void *ws, size_t ws_bytes, void *stream,
                      const hp_overlap *ov) {
    StreamPlan sp;
    hp_status st = plan_stream(q, doc, rows, sp, ov ? ov->mode : 0);
    if (st != HP_OK) return st;
    if ((st = check_out(o, lse)) != HP_OK) return st;
    if (sp.conc) {
        if (!ov->side_stream || !ov->fork_event || !ov->join_event) return HP_ERR_NULL;
        if (ov->side_stream == stream) return HP_ERR_INVALID_ARG;
    }
    if (q->B == 0) return HP_OK;
    if (!ws || ws_bytes < sp.bytes || !aligned16(ws)) return HP_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char *base = (char *)ws;
    int32_t *tok_len = (int32_t *)(base + sp.len_off);
    int32_t *tok_table = (int32_t *)(base + sp.table_off);
    hipError_t e;
    // side by side: the selection and the stream pass wait for everything
    // before the call on `stream`, and run on the second stream
    const hipStream_t ss = sp.conc ? (hipStream_t)ov->side_stream : s;
    if (sp.conc) {
        if ((e = hipEventRecord((hipEvent_t)ov->fork_event, s)) != hipSuccess) return fail_hip(e);
        if ((e = hipStreamWaitEvent(ss, (hipEvent_t)ov->fork_event, 0)) != hipSuccess)
            return fail_hip(e);
    }

    MergeArgs m;
    std::memset(&m, 0, sizeof m);
    if ((st = run_prefix_levels(q, sp.cp, base, m, s)) != HP_OK) return st;

    StreamSelectArgs sel;
    std::memset(&sel, 0, sizeof sel);
    sel.row_slots = rows->row_slots;
    sel.slot_sid = rows->slot_sid;
    sel.row_len = rows->row_len;
    sel.q_req = rows->q_req;
    sel.q_sid = rows->q_sid;
    sel.B = q->B;
    sel.R = rows->num_requests;
    sel.row_cap = rows->row_cap;
    sel.tok_table = tok_table;
    sel.tok_len = tok_len;
    if ((e = launch_stream_select(sel, ss)) != hipSuccess) return fail_hip(e);

    float *so = (float *)(base + sp.suf_off);
    float *sl = (float *)((char *)so +
                          round_up((size_t)q->B * q->Hq * q->d * sizeof(float), kWsAlign));
    SuffixArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q->q;
    a.k_pool = rows->k_pool;
    a.v_pool = rows->v_pool;
    a.table = tok_table;
    a.lens = tok_len;
    a.B = q->B;
    a.Hq = q->Hq;
    a.Hkv = q->Hkv;
    a.max_blocks = rows->row_cap;  // capacity of each query's table
    a.has_suffix = 1;
    a.scale_log2 = (float)((double)q->scale * 1.4426950408889634);
    a.dest = sp.conc ? RowDest{so, sl, 0, 0, 0} : RowDest{o, lse, 0, 0, 0};
    a.pool_rows = rows->pool_rows;
    // K/V footprint: the pool rows, or what the token tables can reach if less.
    const int64_t kv_rows = std::min<int64_t>(rows->pool_rows, (int64_t)q->B * rows->row_cap);
    a.stream_kv = kv_rows * q->Hkv * q->d * esize(q->dtype) * 2 >= kLlcBytes ? 1 : 0;
    if (!sp.conc) {  // the document partials merged in the stream pass's epilogue
        a.nsrc = m.nsrc;
        for (int i = 0; i < m.nsrc; ++i) a.src[i] = m.src[i];
        a.stage_floats = stage_floats(m.src, m.nsrc, q->Hq / q->Hkv, q->d);
    }
    const int blocks = (int)cdiv(rows->row_cap, HP_BLOCK_SIZE);
    const int nws = blocks <= 2 ? 1 : blocks <= 16 ? 2 : 4;
    if ((e = launch_token_suffix(a, q->dtype, q->d, q->Hq / q->Hkv, nws, ss)) != hipSuccess)
        return fail_hip(e);
    if (!sp.conc) return HP_OK;

    // join, then one merge of the document partials with the stream rows
    if ((e = hipEventRecord((hipEvent_t)ov->join_event, ss)) != hipSuccess) return fail_hip(e);
    if ((e = hipStreamWaitEvent(s, (hipEvent_t)ov->join_event, 0)) != hipSuccess)
        return fail_hip(e);
    m.src[m.nsrc++] = MergeSrc{so, sl, 0, 0, 1, 0, 0, q->B};
    m.Hq = q->Hq;
    m.row_b0 = 0;
    m.row_b1 = q->B;
    m.o = o;
    m.lse = lse;
    if ((e = launch_merge(m, q->d, s)) != hipSuccess) return fail_hip(e);
    return HP_OK;
}

}  // namespace

namespace hp {
namespace host {

hp_status cascade_serial_plan(const hp_query *q, const hp_prefix_tree *tree,
                              const hp_paged_kv *kv, const float *o, const float *lse,
                              size_t *bytes) {
    CascadePlan cp;
    hp_status st = plan_cascade(q, tree, kv, 0, cp);
    if (st != HP_OK) return st;
    if ((st = check_out(o, lse)) != HP_OK) return st;
    *bytes = cp.bytes;
    return HP_OK;
}

hp_status cascade_serial(const hp_query *q, const hp_prefix_tree *tree, const hp_paged_kv *kv,
                         float *o, float *lse, void *ws, size_t ws_bytes, void *stream) {
    return cascade_impl(q, tree, kv, o, lse, ws, ws_bytes, stream, nullptr, nullptr);
}

}  // namespace host
}  // namespace hp

extern "C" {

hp_status hp_stream_decode_workspace_size(const hp_query *q, const hp_prefix_tree *doc,
                                          const hp_stream_rows *rows, size_t *bytes) {
    return hp::guarded([&]() -> hp_status {
        if (!bytes) return HP_ERR_NULL;
        StreamPlan serial, conc;  // one size for every mode
        hp_status st = plan_stream(q, doc, rows, serial, 0);
        if (st != HP_OK) return st;
        if ((st = plan_stream(q, doc, rows, conc, 2)) != HP_OK) return st;
        *bytes = std::max(serial.bytes, conc.bytes);
        return HP_OK;
    });
}

hp_status hp_stream_overlap_plan(const hp_query *q, const hp_prefix_tree *doc,
                                 const hp_stream_rows *rows, int32_t mode, int32_t *overlapped) {
    return hp::guarded([&]() -> hp_status {
        if (!overlapped) return HP_ERR_NULL;
        StreamPlan sp;
        hp_status st = plan_stream(q, doc, rows, sp, mode);
        if (st != HP_OK) return st;
        *overlapped = sp.conc ? 1 : 0;
        return HP_OK;
    });
}

hp_status hp_stream_decode(const hp_query *q, const hp_prefix_tree *doc,
                           const hp_stream_rows *rows, float *o, float *lse, void *ws,
                           size_t ws_bytes, void *stream) {
    return hp::guarded([&]() -> hp_status {
        return stream_impl(q, doc, rows, o, lse, ws, ws_bytes, stream, nullptr);
    });
}

hp_status hp_stream_decode_overlap(const hp_query *q, const hp_prefix_tree *doc,
                                   const hp_stream_rows *rows, float *o, float *lse, void *ws,
                                   size_t ws_bytes, void *stream, const hp_overlap *overlap) {
    return hp::guarded([&]() -> hp_status {
        if (!overlap) return HP_ERR_NULL;
        return stream_impl(q, doc, rows, o, lse, ws, ws_bytes, stream, overlap);
    });
}

hp_status hp_cascade_step(const hp_query *q, const hp_prefix_tree *tree, const hp_paged_kv *kv,
                          float *o, float *lse, void *ws, size_t ws_bytes, void *stream) {
    return hp::guarded([&]() -> hp_status {
        return cascade_impl(q, tree, kv, o, lse, ws, ws_bytes, stream, nullptr, nullptr);
    });
}

hp_status hp_cascade_step_overlap(const hp_query *q, const hp_prefix_tree *tree,
                                  const hp_paged_kv *kv, float *o, float *lse, void *ws,
                                  size_t ws_bytes, void *stream, const hp_overlap *overlap) {
    return hp::guarded([&]() -> hp_status {
        if (!overlap) return HP_ERR_NULL;
        return cascade_impl(q, tree, kv, o, lse, ws, ws_bytes, stream, overlap, nullptr);
    });
}

hp_status hp_cascade_step_timed(const hp_query *q, const hp_prefix_tree *tree,
                                const hp_paged_kv *kv, float *o, float *lse, void *ws,
                                size_t ws_bytes, void *stream, const hp_overlap *overlap,
                                void *const *events, int32_t n_events) {
    return hp::guarded([&]() -> hp_status {
        if (n_events != 0 && n_events != 4 && n_events != 5) return HP_ERR_INVALID_ARG;
        if (n_events == 0)
            return cascade_impl(q, tree, kv, o, lse, ws, ws_bytes, stream, overlap, nullptr);
        if (!events) return HP_ERR_NULL;
        void *ev[5] = {events[0], events[1], events[2], events[3],
                       n_events == 5 ? events[4] : nullptr};
        return cascade_impl(q, tree, kv, o, lse, ws, ws_bytes, stream, overlap, ev);
    });
}

}  // extern "C"
