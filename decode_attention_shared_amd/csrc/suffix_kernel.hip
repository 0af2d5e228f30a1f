// Suffix pass: per-sequence paged decode attention, with the final merge of
// the prefix passes' partials fused into its epilogue.
//
// Each sequence's private keys cannot be shared with any other query, so this
// pass is a plain single-query attention per (sequence, KV head), streaming
// the sequence's 16-token blocks through its block table ("Hydragen:
// High-Throughput LLM Inference with Shared Prefixes", section "Inter-Sequence
// Batched Prefix Attention", on suffix attention; "ChunkAttention: Efficient
// Self-Attention with Prefix-Aware KV Cache and Two-Phase Partition", section
// "The Sequence-First Phase Kernel in Detail": per sequence, reduce the saved
// partials of the shared chunks, then walk the private chunks).  Its
// arithmetic intensity is at most G FLOP per byte, so it is bound by HBM: the
// vector ALUs do the dot products and the matrix cores are not used.
//
// One workgroup owns one (sequence, KV head) and the G query heads of that KV
// head.  Its waves take the sequence's blocks in turn (wave w: blocks w,
// w+W, ...), each keeping the next block's loads in flight while it computes
// the current one.  A token's d values are spread over 16-byte lane slices (16
// lanes per token for 16-bit d = 128), so one load instruction covers several
// whole rows; partial dot products are summed inside each 16-lane row with
// DPP.  The waves' online-softmax states meet in LDS, and one pass merges them
// with every prefix partial of the row's tree levels, in the exp2 domain:
// O = sum_i w_i O_i / sum_i w_i, w_i = 2^(L_i - max L) (the Hydragen page's
// "Attention Decomposition Across Subsequences", Eq. 5, over all parts).
#include "common.hpp"

namespace hp {

template <int kDt>
struct Elem;
// get: element e of a lane's 16-byte slice, widened to fp32.  dot: the dot
// product of two such slices in fp32 (16-bit pairs through v_dot2 with fp32
// accumulation; every product of two 16-bit values is exact in fp32).  The
// pairs are taken from a whole-vector cast by shuffles: this toolchain
// miscompiles __builtin_bit_cast of a single vector element (it reads element
// 0 whatever the index).
typedef _Float16 sf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 sbf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 sf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 sbf16x8 __attribute__((ext_vector_type(8)));
template <>
struct Elem<HP_F32> {
    static constexpr int kSize = 4;
    __device__ static float get(const u32x4 &w, int e) { return __uint_as_float(w[e]); }
    __device__ static float dot(const u32x4 &a, const u32x4 &b) {
        const f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
        float s = x[0] * y[0];
        s = fmaf(x[1], y[1], s);
        s = fmaf(x[2], y[2], s);
        return fmaf(x[3], y[3], s);
    }
};
template <>
struct Elem<HP_F16> {
    static constexpr int kSize = 2;
    __device__ static float get(const u32x4 &w, int e) {
        return f16_bits_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    }
    __device__ static float dot(const u32x4 &a, const u32x4 &b) {
        const sf16x8 x = __builtin_bit_cast(sf16x8, a), y = __builtin_bit_cast(sf16x8, b);
        float s0 = __builtin_amdgcn_fdot2(__builtin_shufflevector(x, x, 0, 1),
                                          __builtin_shufflevector(y, y, 0, 1), 0.f, false);
        float s1 = __builtin_amdgcn_fdot2(__builtin_shufflevector(x, x, 2, 3),
                                          __builtin_shufflevector(y, y, 2, 3), 0.f, false);
        s0 = __builtin_amdgcn_fdot2(__builtin_shufflevector(x, x, 4, 5),
                                    __builtin_shufflevector(y, y, 4, 5), s0, false);
        s1 = __builtin_amdgcn_fdot2(__builtin_shufflevector(x, x, 6, 7),
                                    __builtin_shufflevector(y, y, 6, 7), s1, false);
        return s0 + s1;
    }
};
template <>
struct Elem<HP_BF16> {
    static constexpr int kSize = 2;
    __device__ static float get(const u32x4 &w, int e) {
        return bf16_bits_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    }
    __device__ static float dot(const u32x4 &a, const u32x4 &b) {
        const sbf16x8 x = __builtin_bit_cast(sbf16x8, a), y = __builtin_bit_cast(sbf16x8, b);
        float s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1),
                                                   __builtin_shufflevector(y, y, 0, 1), 0.f,
                                                   false);
        float s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3),
                                                   __builtin_shufflevector(y, y, 2, 3), 0.f,
                                                   false);
        s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5),
                                             __builtin_shufflevector(y, y, 4, 5), s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7),
                                             __builtin_shufflevector(y, y, 6, 7), s1, false);
        return s0 + s1;
    }
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xf, 0xf, true));
}

// Sum over aligned groups of kWidth consecutive lanes; every lane of a group
// ends with the group's sum.  Within a 16-lane row: quad swaps, then the
// half-row mirror (lane i <-> 7-i) and the row mirror (i <-> 15-i), each of
// which pairs every lane with one from the other half of its group.
template <int kWidth>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (kWidth >= 2) x += dpp<0xb1>(x);   // quad_perm [1,0,3,2]
    if constexpr (kWidth >= 4) x += dpp<0x4e>(x);   // quad_perm [2,3,0,1]
    if constexpr (kWidth >= 8) x += dpp<0x141>(x);  // row_half_mirror
    if constexpr (kWidth >= 16) x += dpp<0x140>(x); // row_mirror
    if constexpr (kWidth >= 32) x += __shfl_xor(x, 16, kWave);
    return x;
}

// Where a sequence's keys are (kMode):
//   kBlocks  paged: token t in slot t % 16 of block table[b][t / 16];
//   kTree    chunk-tree: pool row tok_rows[seq_tok[b] + t] (one row per token:
//            tree pieces start at any row), partials from the plan's source
//            list instead of the by-value sources;
//   kTokens  token table: pool row table[b * cap + t] (cap = max_blocks) for
//            t < lens[b] (the visible positions of a stream of a
//            shared-context request, gathered by the stream selection
//            kernel; its document is merged in as a by-value source).
constexpr int kBlocks = 0, kTree = 1, kTokens = 2;

template <int kDt, int D, int G, int NWS, int kMode, bool kNT>
__global__ __launch_bounds__(64 * NWS) void suffix_kernel(SuffixArgs a) {
    constexpr bool kRows = kMode != kBlocks;  // one pool row per token
    using E = Elem<kDt>;
    constexpr int kEpl = 16 / E::kSize;  // elements per lane per token
    constexpr int kLpt = D / kEpl;       // lanes per token
    constexpr int kTpp = kWave / kLpt;   // tokens per wave-wide load
    constexpr int kPasses = kBlock / kTpp;
    constexpr int kThreads = 64 * NWS;
    static_assert(kLpt <= kWave && kPasses >= 1, "layout");
    __shared__ float sm_acc[NWS][G][D];
    __shared__ float sm_m[NWS][G], sm_l[NWS][G];
    __shared__ int sm_bad[NWS];

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int g = (int)(blockIdx.x % a.Hkv);
    const int b = (int)(blockIdx.x / a.Hkv);
    const int tg = lane / kLpt;  // token slot within a load
    const int li = lane % kLpt;  // lane within the token's group
    const int d0 = li * kEpl;

    // The G query rows of this KV head, this lane's 16-byte slice of each.
    u32x4 qraw[G];

    int len = 0;
    bool bad = false;
    const int *trow;
    int row_cap = a.max_blocks;  // entries of this sequence's table row
    if constexpr (kMode == kTree) {
        const int tok0 = a.tree[a.seq_tok_off + b];
        const int cap = a.tree[a.seq_tok_off + b + 1] - tok0;
        trow = a.tree + a.tok_rows_off + tok0;
        row_cap = cap;
        len = cap;
        if (a.lens != nullptr) {
            len = a.lens[b] - a.tree[a.shared_off + b];
            bad = len < 0 || len > cap;
        }
    } else if constexpr (kMode == kTokens) {
        trow = a.table + (int64_t)b * a.max_blocks;
        len = a.lens[b];
        bad = len < 0 || len > a.max_blocks;
    } else {
        trow = a.table + (int64_t)b * a.max_blocks;
    }
    if (kMode == kBlocks && a.has_suffix) {
        len = a.lens[b];
        bad = len < 0 || len > a.max_blocks * kBlock;
    }
    // Paged mode: the prefix nodes this sequence reads privately come first,
    // as blocks [sb[i], sb[i + 1]) of node sid[i] (at most one per level).
    // (Indexed by constants only, so the arrays stay in registers.)
    int sid[HP_MAX_LEVELS], sb[HP_MAX_LEVELS + 1];
#pragma unroll
    for (int j = 0; j < HP_MAX_LEVELS; ++j) sid[j] = 0;
#pragma unroll
    for (int j = 0; j <= HP_MAX_LEVELS; ++j) sb[j] = 0;
    int nps = 0;
    if constexpr (kMode == kBlocks) {
#pragma unroll 1
        for (int si = 0; si < a.nseg; ++si) {
            const PrivSeg &sg = a.seg[si];
            if (b < sg.b0 || b >= sg.b1 || sg.len <= 0) continue;
            const int nb = (sg.len + kBlock - 1) / kBlock;
#pragma unroll
            for (int j = 0; j < HP_MAX_LEVELS; ++j)
                if (j == nps) {
                    sid[j] = si;
                    sb[j + 1] = sb[j] + nb;
                }
            nps = min(nps + 1, HP_MAX_LEVELS);
        }
    }
    int nsb = 0;  // blocks over the private prefix nodes
#pragma unroll
    for (int j = 1; j <= HP_MAX_LEVELS; ++j)
        if (j == nps) nsb = sb[j];
    const int nblk = bad ? 0 : nsb + (len + kBlock - 1) / kBlock;

    // The prefix partials this row merges (splits of the by-value sources
    // covering sequence b) are copied into LDS by DMA right away, so their
    // latency hides behind the suffix stream and the epilogue reads them
    // from LDS.  Part p holds G rows of D floats and G LSEs; rows whose
    // parts do not fit the stage are read from memory in the epilogue.
    // The stage is the launch's dynamic LDS (a.stage_floats floats, sized by
    // the host for the rows with the most partials; 0 when they do not fit).
    constexpr int kCpp = G * D / 4;  // 16-byte chunks per part
    extern __shared__ __attribute__((aligned(16))) float sm_po[];
    __shared__ float sm_pl[kWave];
    int nparts = 0;
    if constexpr (kMode != kTree) {
#pragma unroll 1
        for (int si = 0; si < a.nsrc; ++si)
            if (b >= a.src[si].b0 && b < a.src[si].b1) nparts += a.src[si].nsplit;
    }
    const bool staged = kMode != kTree && nparts > 0 && nparts * G <= kWave &&
                        (nparts * kCpp + kWave - 1) / kWave * kWave * 4 <= a.stage_floats;
    // Copies the row's partials into LDS.  The global-to-LDS loads are the
    // compiler-tracked form, so its waits for later register loads stay exact.
    auto stage = [&]() {
        if constexpr (kMode != kTree) {
            if (!staged) return;
            // Lane p < nparts holds the base pointers of part p (uniform walk
            // over the sources); each transfer picks its part's base by shuffle.
            const float *pbo = a.src[0].o, *pbl = a.src[0].lse;
            int pb = 0;
#pragma unroll 1
            for (int si = 0; si < a.nsrc; ++si) {
                const MergeSrc &sr = a.src[si];
                if (b < sr.b0 || b >= sr.b1) continue;
                const int i = lane - pb;
                if (i >= 0 && i < sr.nsplit) {
                    const int64_t ri = (b - sr.b0) * a.Hq + (int64_t)g * G;
                    pbo = sr.o + (int64_t)i * sr.o_split + ri * D;
                    pbl = sr.lse + (int64_t)i * sr.lse_split + ri;
                }
                pb += sr.nsplit;
            }
            const int chunks = nparts * kCpp;
#pragma unroll 1
            for (int c0 = wave * kWave; c0 < chunks; c0 += NWS * kWave) {
                const int c = min(c0 + lane, chunks - 1);  // lanes past the end re-read the last chunk
                const float *po = (const float *)__shfl((long long)(intptr_t)pbo, c / kCpp, kWave);
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(po + (c % kCpp) * 4),
                    (__attribute__((address_space(3))) void *)&sm_po[c0 * 4], 16, 0, 0);
            }
            if (wave == 0) {
                const int e = min(lane, nparts * G - 1);
                const float *pl = (const float *)__shfl((long long)(intptr_t)pbl, e / G, kWave);
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(pl + e % G),
                    (__attribute__((address_space(3))) void *)sm_pl, 4, 0, 0);
            }
        }
    };

    float m[G], l[G], acc[G][kEpl];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < kEpl; ++e) acc[j][e] = 0.f;
    }

    // Paged blocks: bytes between a block's tokens and offset of this KV head
    // (token-major [16][Hkv][D] or head-major [Hkv][16][D] blocks).
    const int64_t tok_stride = a.kv_hnd ? (int64_t)D * E::kSize : (int64_t)a.Hkv * D * E::kSize;
    const int64_t head_off = (int64_t)g * D * E::kSize * (a.kv_hnd ? kBlock : 1);
    const char *kp = (const char *)a.k_pool;
    const char *vp = (const char *)a.v_pool;

    // Where a block's keys are: its block id (block table), or in chunk-tree
    // mode the pool row of each token this lane loads.  Read one block-step
    // ahead of the K/V loads, so the lookup's latency never sits in front of
    // a block's loads.  The lookup is bounded by the row's capacity, not by
    // the sequence length, so the first ones go out together with the length
    // read instead of after it; entries past the length are never used (only
    // blocks below nblk are fetched, and their ids are checked there).
    struct Ref {
        int v[kRows ? kPasses : 1];
    };
    auto table_id = [&](int blk) {
        Ref r;
        if constexpr (kRows) {
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const int t = blk * kBlock + p * kTpp + tg;
                r.v[p] = t < row_cap ? trow[t] : 0;
            }
        } else {
            const int pb = blk - nsb;  // block of the paged suffix
            r.v[0] = pb >= 0 && pb < row_cap ? trow[pb] : 0;
        }
        return r;
    };
    // 16 bytes of one K or V row; kNT marks the load non-temporal (the data is
    // read once per step and would not survive in the cache until the next).
    auto load16 = [](const char *p) -> u32x4 {
        if constexpr (kNT) return __builtin_nontemporal_load((const u32x4 *)p);
        else return *(const u32x4 *)p;
    };
    // Issue the loads of one block (keys past the sequence's end and blocks
    // with an out-of-range id are never read).
    auto fetch = [&](int blk, const Ref &ref, u32x4 (&kr)[kPasses], u32x4 (&vr)[kPasses],
                     int &valid) {
        if constexpr (kRows) {
            valid = min(kBlock, len - blk * kBlock);
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const int t = p * kTpp + tg;
                const int row = ref.v[p];
                const bool row_ok = row >= 0 && row < a.pool_rows;
                bad |= t < valid && !row_ok;
                const bool ok = t < valid && row_ok;
                const int64_t off = ((int64_t)(ok ? row : 0) * a.Hkv + g) * D * E::kSize +
                                    d0 * E::kSize;
                kr[p] = ok ? load16(kp + off) : u32x4{0, 0, 0, 0};
                vr[p] = ok ? load16(vp + off) : u32x4{0, 0, 0, 0};
            }
        } else if (blk < nsb) {
            // a block of a private prefix node: contiguous rows, plain loads
            // (the node's other sequences read the same rows in this step)
            int si = sid[0], s0 = 0;
#pragma unroll
            for (int j = 1; j < HP_MAX_LEVELS; ++j)
                if (j < nps && blk >= sb[j]) {
                    si = sid[j];
                    s0 = sb[j];
                }
            const PrivSeg &sg = a.seg[si];
            const int t0 = (blk - s0) * kBlock;
            valid = min(kBlock, sg.len - t0);
            const int64_t base = ((int64_t)t0 * sg.stride_tok + (int64_t)g * sg.stride_head + d0) *
                                 E::kSize;
            const char *ks = (const char *)sg.k + base;
            const char *vs = (const char *)sg.v + base;
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const int t = p * kTpp + tg;
                const bool ok = t < valid;
                const int64_t off = (int64_t)t * sg.stride_tok * E::kSize;
                kr[p] = ok ? *(const u32x4 *)(ks + off) : u32x4{0, 0, 0, 0};
                vr[p] = ok ? *(const u32x4 *)(vs + off) : u32x4{0, 0, 0, 0};
            }
        } else {
            const int id = ref.v[0];
            const bool id_ok = id >= 0 && id < a.num_blocks;
            bad |= !id_ok;
            valid = id_ok ? min(kBlock, len - (blk - nsb) * kBlock) : 0;
            const int64_t base = (int64_t)(id_ok ? id : 0) * kBlock * a.Hkv * D * E::kSize +
                                 head_off + d0 * E::kSize;
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const int t = p * kTpp + tg;
                const bool ok = t < valid;
                const int64_t off = base + t * tok_stride;
                kr[p] = ok ? load16(kp + off) : u32x4{0, 0, 0, 0};
                vr[p] = ok ? load16(vp + off) : u32x4{0, 0, 0, 0};
            }
        }
    };
    // Online-softmax update with one block (exp2 domain, scale folded in).
    auto process = [&](const u32x4 (&kr)[kPasses], const u32x4 (&vr)[kPasses], int valid) {
        float x[kPasses][G];
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const bool ok = p * kTpp + tg < valid;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float dot = group_sum<kLpt>(E::dot(kr[p], qraw[j]));
                x[p][j] = ok ? dot * a.scale_log2 : -INFINITY;
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float bm = x[0][j];
#pragma unroll
            for (int p = 1; p < kPasses; ++p) bm = fmaxf(bm, x[p][j]);
            bm = xor_max_from<kLpt>(bm);  // max over the block's 16 tokens
            const float mn = fmaxf(m[j], bm);
            const float alpha = fast_exp2(m[j] - mn);
            l[j] *= alpha;
#pragma unroll
            for (int e = 0; e < kEpl; ++e) acc[j][e] *= alpha;
            m[j] = mn;
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const float pw = fast_exp2(x[p][j] - mn);
                l[j] += pw;
#pragma unroll
                for (int e = 0; e < kEpl; ++e) acc[j][e] = fmaf(pw, E::get(vr[p], e), acc[j][e]);
            }
        }
    };

    // Blocks wave, wave + NWS, ...: two register sets, the next block's loads
    // are in flight while the current block is computed.
    {
        u32x4 k0[kPasses], v0[kPasses], k1[kPasses], v1[kPasses];
        int n0 = 0, n1 = 0;
        int blk = wave;
        Ref id0 = table_id(blk), id1 = table_id(blk + NWS);
#pragma unroll
        for (int j = 0; j < G; ++j)
            qraw[j] = *(const u32x4 *)((const char *)a.q +
                                       (((int64_t)b * a.Hq + g * G + j) * D + d0) * E::kSize);
        if (blk < nblk) fetch(blk, id0, k0, v0, n0);
        stage();
#pragma unroll 1
        for (; blk < nblk; blk += 2 * NWS) {
            const int b1 = blk + NWS, b2 = blk + 2 * NWS, b3 = blk + 3 * NWS;
            id0 = table_id(b2);
            if (b1 < nblk) fetch(b1, id1, k1, v1, n1);
            if (n0 > 0) process(k0, v0, n0);
            id1 = table_id(b3);
            if (b2 < nblk) fetch(b2, id0, k0, v0, n0);
            if (b1 < nblk && n1 > 0) process(k1, v1, n1);
        }
    }

    // This wave's state: sum the token groups, publish to LDS.
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const float lt = xor_sum_from<kLpt>(l[j]);
#pragma unroll
        for (int e = 0; e < kEpl; ++e) {
            const float s = xor_sum_from<kLpt>(acc[j][e]);
            if (tg == 0) sm_acc[wave][j][d0 + e] = s;
        }
        if (lane == 0) {
            sm_m[wave][j] = m[j];
            sm_l[wave][j] = lt;
        }
    }
    // A bad pool row is seen by the lanes that hold its token (row modes): any lane
    // of the wave marks it.
    const bool wave_bad = __any(bad);
    if (lane == 0) sm_bad[wave] = wave_bad ? 1 : 0;
    __syncthreads();

    // Final merge: this row's suffix (the waves' states) and every prefix
    // partial of the tree levels covering sequence b.
    bool any_bad = false;
#pragma unroll
    for (int w = 0; w < NWS; ++w) any_bad |= sm_bad[w] != 0;
#pragma unroll 1
    for (int t = tid; t < G * (D / 4); t += kThreads) {
        const int j = t / (D / 4);
        const int c4 = (t % (D / 4)) * 4;
        const int h = g * G + j;
        // suffix part, unnormalised: (sum_w 2^(m_w - Ms) acc_w, sum_w 2^(m_w - Ms) l_w)
        float ms = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWS; ++w) ms = fmaxf(ms, sm_m[w][j]);
        f32x4 so = {0.f, 0.f, 0.f, 0.f};
        float sl = 0.f;
        if (ms > -INFINITY) {
#pragma unroll
            for (int w = 0; w < NWS; ++w) {
                const float f = fast_exp2(sm_m[w][j] - ms);
                sl += f * sm_l[w][j];
                so += f * *(const f32x4 *)&sm_acc[w][j][c4];
            }
        }
        // prefix parts: normalised O_i with natural-log LSE_i
        float mx = sl > 0.f ? ms : -INFINITY;
        bool nan_seen = false;
        if constexpr (kMode == kTree) {
            const int s0 = a.tree[a.seq_src_off + b], s1 = a.tree[a.seq_src_off + b + 1];
#pragma unroll 1
            for (int si = s0; si < s1; ++si) {
                const TreeSrc sr = *(const TreeSrc *)(a.tree + a.srcs_off + 4 * (int64_t)si);
#pragma unroll 4
                for (int i = 0; i < sr.nsplit; ++i) {
                    const float L =
                        a.part_lse[((int64_t)sr.part_row + (int64_t)i * sr.split_rows) * a.Hq + h] *
                        kLog2e;
                    nan_seen |= (L != L);
                    mx = fmaxf(mx, L);
                }
            }
        } else if (staged) {
#pragma unroll 4
            for (int p = 0; p < nparts; ++p) {
                const float L = sm_pl[p * G + j] * kLog2e;
                nan_seen |= (L != L);
                mx = fmaxf(mx, L);
            }
        } else {
#pragma unroll 1
            for (int si = 0; si < a.nsrc; ++si) {
                const MergeSrc &s = a.src[si];
                if (b < s.b0 || b >= s.b1) continue;
                const int64_t ri = (b - s.b0) * a.Hq + h;
#pragma unroll 4
                for (int i = 0; i < s.nsplit; ++i) {
                    const float L = s.lse[(int64_t)i * s.lse_split + ri] * kLog2e;
                    nan_seen |= (L != L);
                    mx = fmaxf(mx, L);
                }
            }
        }
        f32x4 out;
        float lse;
        if (any_bad || nan_seen) {
            out = f32x4{NAN, NAN, NAN, NAN};
            lse = NAN;
        } else if (!(mx > -INFINITY)) {
            out = f32x4{0.f, 0.f, 0.f, 0.f};
            lse = -INFINITY;
        } else {
            float den = 0.f;
            f32x4 num = {0.f, 0.f, 0.f, 0.f};
            if (sl > 0.f) {
                const float f = fast_exp2(ms - mx);
                den = sl * f;
                num = so * f;
            }
            if constexpr (kMode == kTree) {
                const int s0 = a.tree[a.seq_src_off + b], s1 = a.tree[a.seq_src_off + b + 1];
#pragma unroll 1
                for (int si = s0; si < s1; ++si) {
                    const TreeSrc sr = *(const TreeSrc *)(a.tree + a.srcs_off + 4 * (int64_t)si);
#pragma unroll 4
                    for (int i = 0; i < sr.nsplit; ++i) {
                        const int64_t ri =
                            ((int64_t)sr.part_row + (int64_t)i * sr.split_rows) * a.Hq + h;
                        const float w = fast_exp2(a.part_lse[ri] * kLog2e - mx);
                        num += w * *(const f32x4 *)(a.part_o + ri * D + c4);
                        den += w;
                    }
                }
            } else if (staged) {
#pragma unroll 4
                for (int p = 0; p < nparts; ++p) {
                    const float w = fast_exp2(sm_pl[p * G + j] * kLog2e - mx);
                    num += w * *(const f32x4 *)&sm_po[(p * G + j) * D + c4];
                    den += w;
                }
            } else {
#pragma unroll 1
                for (int si = 0; si < a.nsrc; ++si) {
                    const MergeSrc &s = a.src[si];
                    if (b < s.b0 || b >= s.b1) continue;
                    const int64_t ri = (b - s.b0) * a.Hq + h;
#pragma unroll 4
                    for (int i = 0; i < s.nsplit; ++i) {
                        const float w =
                            fast_exp2(s.lse[(int64_t)i * s.lse_split + ri] * kLog2e - mx);
                        num += w * *(const f32x4 *)(s.o + (int64_t)i * s.o_split + ri * D + c4);
                        den += w;
                    }
                }
            }
            out = num * (1.f / den);
            lse = (mx + fast_log2(den)) * kLn2;
        }
        const int64_t orow = ((int64_t)b - a.dest.row_base) * a.Hq + h;
        *(f32x4 *)(a.dest.o + orow * D + c4) = out;
        if (c4 == 0 && a.dest.lse != nullptr) a.dest.lse[orow] = lse;
    }
}

template <int kDt, int D, int NWS, int kMode, bool kNT>
static void launch_g(const SuffixArgs &a, int G, dim3 grid, hipStream_t s) {
    constexpr int T = 64 * NWS;
    const size_t lds = (size_t)a.stage_floats * sizeof(float);
    switch (G) {
    case 1: suffix_kernel<kDt, D, 1, NWS, kMode, kNT><<<grid, T, lds, s>>>(a); break;
    case 2: suffix_kernel<kDt, D, 2, NWS, kMode, kNT><<<grid, T, lds, s>>>(a); break;
    case 4: suffix_kernel<kDt, D, 4, NWS, kMode, kNT><<<grid, T, lds, s>>>(a); break;
    default: suffix_kernel<kDt, D, 8, NWS, kMode, kNT><<<grid, T, lds, s>>>(a); break;
    }
}

template <int kDt, int NWS, int kMode, bool kNT>
static void launch_d(const SuffixArgs &a, int d, int G, dim3 grid, hipStream_t s) {
    if (d == 128) launch_g<kDt, 128, NWS, kMode, kNT>(a, G, grid, s);
    else launch_g<kDt, 64, NWS, kMode, kNT>(a, G, grid, s);
}

template <int kDt, int kMode, bool kNT>
static void launch_dt(const SuffixArgs &a, int d, int G, int nws, dim3 grid, hipStream_t s) {
    switch (nws) {
    case 1: launch_d<kDt, 1, kMode, kNT>(a, d, G, grid, s); break;
    case 2: launch_d<kDt, 2, kMode, kNT>(a, d, G, grid, s); break;
    default: launch_d<kDt, 4, kMode, kNT>(a, d, G, grid, s); break;
    }
}

template <int kMode, bool kNT = false>
static hipError_t launch_mode(const SuffixArgs &a, int dtype, int d, int G, int nws,
                              hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)a.B * a.Hkv));
    if (dtype == HP_BF16) launch_dt<HP_BF16, kMode, kNT>(a, d, G, nws, grid, s);
    else if (dtype == HP_F16) launch_dt<HP_F16, kMode, kNT>(a, d, G, nws, grid, s);
    else launch_dt<HP_F32, kMode, kNT>(a, d, G, nws, grid, s);
    return hipGetLastError();
}

hipError_t launch_suffix(const SuffixArgs &a, int dtype, int d, int G, int nws, hipStream_t s) {
    return a.stream_kv ? launch_mode<kBlocks, true>(a, dtype, d, G, nws, s)
                       : launch_mode<kBlocks, false>(a, dtype, d, G, nws, s);
}

// Sequence-first pass of a chunk-tree step (a.tree set).
hipError_t launch_tree_suffix(const SuffixArgs &a, int dtype, int d, int G, int nws,
                              hipStream_t s) {
    return launch_mode<kTree>(a, dtype, d, G, nws, s);
}

// Per-stream token tables of a shared-context request (a.table [B][cap]).
hipError_t launch_token_suffix(const SuffixArgs &a, int dtype, int d, int G, int nws,
                               hipStream_t s) {
    return a.stream_kv ? launch_mode<kTokens, true>(a, dtype, d, G, nws, s)
                       : launch_mode<kTokens, false>(a, dtype, d, G, nws, s);
}

}  // namespace hp
