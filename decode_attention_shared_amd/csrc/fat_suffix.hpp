// Suffix pass for workgroups shaped like the prefix pass's (512 threads, all
// of its registers and LDS), so that both passes can share one launch.
//
// Each sequence's private keys are read by a plain decode attention per
// (sequence, KV head) and its G query heads ("Hydragen: High-Throughput LLM
// Inference with Shared Prefixes", section "Inter-Sequence Batched Prefix
// Attention", on suffix attention), written as those rows' own (O, LSE) for
// the merge (section "Attention Decomposition Across Subsequences", Eq. 5).
//
// A workgroup of the prefix pass's shape is the only one on its compute
// unit, so its 8 waves must keep that unit's loads in flight on their own.
// The work is split into items: block range s of (sequence, KV head) unit u
// (blocks [s * split_blocks, (s + 1) * split_blocks) of the sequence), each
// with its own (O, LSE) rows in split slot s, which the merge combines like
// any other partial (items past a sequence's blocks hold nothing and are
// neither computed nor read).  Every wave walks a fixed list of items as one
// stream of steps, one 16-token block per step: before the first step the
// wave gathers its items' lengths and block ids into a table of steps in
// LDS, then keeps the loads of the next kRing - 1 steps in flight while it
// computes the current one.  Every step issues the
// same loads (a step without a block loads one that exists and masks it) and
// no vector-memory store sits in the loop (finished rows wait in LDS and are
// written after it), so the compiler's waits for the ring are exact counts
// rather than full drains.  Each token group of lanes keeps its own running
// max; the groups are combined once per item.
//
// 16-bit K/V, d = 128: a token's d values are spread over 16 lanes of 16-byte
// slices, one load instruction covers 4 tokens, and partial dot products are
// summed inside each 16-lane row with DPP.
#pragma once

#include "common.hpp"

namespace hp {

// Steps (16-token blocks) one suffix wave may take: the wave's table of them
// lives in LDS beside the prefix pass's ring.
constexpr int kFatMaxSteps = 504;
// Rows (items x G) of one suffix wave, whose finished (O, LSE) wait in the
// wave's kFatStageBytes share of the prefix pass's LDS ring until the wave
// writes them all out at its end.
constexpr int kFatMaxRows = 31;
constexpr int kFatStageBytes = 16384;
// Blocks of one item (64 keys): a long suffix is spread over several waves.
constexpr int kFatSplitBlocks = 4;

struct FatSuffixArgs {
    const void *q;          // [B][Hq][d]
    const void *k_pool;     // paged blocks, token-major [16][Hkv][d] or head-major [Hkv][16][d]
    const void *v_pool;
    const int32_t *table;   // [B][max_blocks]
    const int32_t *lens;    // [B]
    float *o;               // [nsplit][B][Hq][d] the items' rows, normalised
    float *lse;             // [nsplit][B][Hq] natural-log LSE
    int32_t B, Hq, Hkv;
    int32_t max_blocks, num_blocks;
    int32_t kv_hnd;
    float scale_log2;
    int32_t prefix_wgs;     // workgroups of the launch before the suffix ones
    int32_t nsplit;         // items per unit: ceil(max_blocks / kFatSplitBlocks)
};

namespace fs {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// Dot product of two 16-byte slices (8 16-bit values) in fp32.
template <bool kBf16>
__device__ __forceinline__ float dot8(const u32x4 &a, const u32x4 &b) {
    if constexpr (kBf16) {
        const b8 x = __builtin_bit_cast(b8, a), y = __builtin_bit_cast(b8, b);
        float s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1),
                                                   __builtin_shufflevector(y, y, 0, 1), 0.f, false);
        float s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3),
                                                   __builtin_shufflevector(y, y, 2, 3), 0.f, false);
        s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5),
                                             __builtin_shufflevector(y, y, 4, 5), s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7),
                                             __builtin_shufflevector(y, y, 6, 7), s1, false);
        return s0 + s1;
    } else {
        const h8 x = __builtin_bit_cast(h8, a), y = __builtin_bit_cast(h8, b);
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
}

// Element e of a 16-byte slice, widened to fp32.
template <bool kBf16>
__device__ __forceinline__ float elem(const u32x4 &w, int e) {
    const uint32_t bits = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
    return kBf16 ? bf16_bits_to_float(bits) : f16_bits_to_float(bits);
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xf, 0xf, true));
}

// Sum over each 16-lane row: quad swaps, then the half-row and row mirrors.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0xb1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4e>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0x140>(x);  // row_mirror
    return x;
}

__device__ __forceinline__ int lane_read(int v, int i) { return __builtin_amdgcn_readlane(v, i); }

}  // namespace fs

// Wave `sw` of `S` suffix waves: items sw, sw + S, ... of the B * Hkv * nsplit
// items (item i: unit i / nsplit, split i % nsplit), each with the G query
// heads of its KV head.  The host keeps a wave's items within kFatMaxRows / G
// and their blocks within kFatMaxSteps; `stage` is the wave's kFatStageBytes
// of LDS.
template <bool kBf16, int D, int G, bool kNT>
__device__ __forceinline__ void fat_suffix_wave(const FatSuffixArgs &a, int sw, int S,
                                                char *stage) {
    static_assert(D == 128, "16 lanes of 8 values per token");
    constexpr int kEpl = 8;             // 16-bit elements per lane slice
    constexpr int kLpt = D / kEpl;      // lanes per token (16)
    constexpr int kTpp = kWave / kLpt;  // tokens per load (4)
    constexpr int kPasses = kBlock / kTpp;
    constexpr int kRing = G >= 4 ? 3 : 4;  // steps whose registers the ring holds
    constexpr int kMaxItems = kFatMaxRows / G;
    static_assert(kFatMaxSteps % 12 == 0, "table a multiple of every ring depth");
    static_assert(kFatMaxRows * (D + 2) * 4 <= kFatStageBytes, "staging");
    float *st_o = (float *)stage;                   // [kFatMaxRows][D]
    float *st_lse = st_o + kFatMaxRows * D;         // [kFatMaxRows]
    int *st_row = (int *)(st_lse + kFatMaxRows);    // [kFatMaxRows]

    const int lane = threadIdx.x % kWave;
    const int tg = lane / kLpt;
    const int d0 = (lane % kLpt) * kEpl;
    const int items = a.B * a.Hkv * a.nsplit;
    if (sw >= items) return;
    // (the clamp only keeps a violated host bound inside the staging area)
    const int K = min((items - sw + S - 1) / S, kMaxItems);

    // Item k of this wave in lane k: sequence, head, split, length, its blocks
    // [j0, j1).  A sequence whose length is out of range gets no item: the
    // merge, which checks the same length, makes its rows NaN.
    const bool has = lane < K;
    const int it = has ? sw + lane * S : sw;
    const int u = it / a.nsplit, sp = it % a.nsplit;
    const int ub = u / a.Hkv, ug = u % a.Hkv;
    const int len = a.lens[ub];
    const bool ubad = len < 0 || len > a.max_blocks * kBlock;
    const int nblk = ubad ? 0 : (len + kBlock - 1) / kBlock;
    const int j0 = sp * kFatSplitBlocks;
    const int nit = has ? max(min(nblk - j0, kFatSplitBlocks), 0) : 0;  // steps
    int incl = nit;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_up(incl, off, kWave);
        incl += lane >= off ? t : 0;
    }
    const int excl = incl - nit;
    const int T = fs::lane_read(incl, kWave - 1);
    if (T == 0) return;  // no item of this wave holds a key
    const int Tpad = min((T + kRing - 1) / kRing * kRing, kFatMaxSteps);

    // The wave's table of steps in LDS, one 8-byte entry per step:
    //   x: the block to load (0 when the step has none: a block that exists)
    //   y: the item's first output row split * B * Hq + b * Hq + g * G (bits
    //      0-23), valid keys (bits 24-28), first step of its item (bit 29), a
    //      block id out of range (bit 30), last step of its item (bit 31)
    // Steps past the last item (up to a multiple of kRing) repeat a row with
    // no keys and no flags, which changes nothing.
    __shared__ uint2 steps[8][kFatMaxSteps];
    uint2 *tab = steps[threadIdx.x / kWave];
#pragma unroll 1
    for (int w0 = 0; w0 < Tpad; w0 += kWave) {
        const int s = w0 + lane;
        int k = 0;
#pragma unroll 1
        for (int kk = 0; kk < K; ++kk) k += fs::lane_read(incl, kk) <= s ? 1 : 0;
        const bool pad = k >= K;
        const int kc = pad ? K - 1 : k;
        const int ex = __shfl(excl, kc, kWave);
        const int n = __shfl(nit, kc, kWave);
        const int ln = __shfl(len, kc, kWave);
        const int bb = __shfl(ub, kc, kWave);
        const int gg = __shfl(ug, kc, kWave);
        const int spl = __shfl(sp, kc, kWave);
        const int i = s - ex;  // step within the item
        const bool real = !pad && i < n;
        const int j = spl * kFatSplitBlocks + (real ? i : 0);  // block of the sequence
        const int bid = a.table[(int64_t)bb * a.max_blocks + min(j, a.max_blocks - 1)];
        const bool id_ok = bid >= 0 && bid < a.num_blocks;
        const int valid = real && id_ok ? min(kBlock, ln - j * kBlock) : 0;
        const bool bad = real && !id_ok;
        const uint32_t y = (uint32_t)((spl * a.B + bb) * a.Hq + gg * G) |
                           ((uint32_t)valid << 24) | ((real && i == 0) ? (1u << 29) : 0u) |
                           (bad ? (1u << 30) : 0u) | ((real && i == n - 1) ? (1u << 31) : 0u);
        if (s < Tpad) tab[s] = uint2{(uint32_t)(real && id_ok ? bid : 0), y};
    }

    const int64_t blk_bytes = (int64_t)kBlock * a.Hkv * D * 2;
    const int64_t tok_stride = a.kv_hnd ? (int64_t)D * 2 : (int64_t)a.Hkv * D * 2;
    const int64_t head_mul = (int64_t)D * 2 * (a.kv_hnd ? kBlock : 1);
    const char *kp = (const char *)a.k_pool;
    const char *vp = (const char *)a.v_pool;
    const char *qp = (const char *)a.q;

    auto load16 = [](const char *p) -> u32x4 {
        if constexpr (kNT) return __builtin_nontemporal_load((const u32x4 *)p);
        else return *(const u32x4 *)p;
    };

    u32x4 kb[kRing][kPasses], vb[kRing][kPasses], qb[kRing][G];
    uint32_t r_y[kRing];

    // Loads of step t (clamped to the last step) into slot r.
    auto issue = [&](int r, int t) {
        const uint2 e = tab[min(t, Tpad - 1)];
        const uint32_t id = __builtin_amdgcn_readfirstlane(e.x);
        const uint32_t y = __builtin_amdgcn_readfirstlane(e.y);
        r_y[r] = y;
        const int row = (int)(y & 0xffffffu) % (a.B * a.Hq);  // the query row
        const int g = (row % a.Hq) / G;
        const int64_t base = (int64_t)id * blk_bytes + g * head_mul + d0 * 2;
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const int64_t off = base + (int64_t)(p * kTpp + tg) * tok_stride;
            kb[r][p] = load16(kp + off);
            vb[r][p] = load16(vp + off);
        }
#pragma unroll
        for (int j = 0; j < G; ++j)
            qb[r][j] = *(const u32x4 *)(qp + ((int64_t)(row + j) * D + d0) * 2);
    };

    float m[G], l[G], acc[G][kEpl];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < kEpl; ++e) acc[j][e] = 0.f;
    }
    bool sbad = false;
    int ku = -1;  // the item of the step being computed (this wave's count)

    // One block of slot r into the running state of its item; at the item's
    // last step the token groups are combined (weights 2^(m_group - M)) and
    // the item's G rows go to their staging slots.
    auto compute = [&](int r) {
        const uint32_t y = r_y[r];
        const int valid = (int)((y >> 24) & 31u);
        if (y & (1u << 29)) {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                m[j] = -INFINITY;
                l[j] = 0.f;
#pragma unroll
                for (int e = 0; e < kEpl; ++e) acc[j][e] = 0.f;
            }
            sbad = false;
            ++ku;
        }
        sbad |= (y & (1u << 30)) != 0;
        // keys past the valid ones may hold anything: zero their values
        u32x4 vv[kPasses];
        bool ok[kPasses];
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            ok[p] = p * kTpp + tg < valid;
#pragma unroll
            for (int w = 0; w < 4; ++w) vv[p][w] = ok[p] ? vb[r][p][w] : 0u;
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float x[kPasses];
            float bm = -INFINITY;
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const float dsum = fs::row_sum16(fs::dot8<kBf16>(kb[r][p], qb[r][j]));
                x[p] = ok[p] ? dsum * a.scale_log2 : -INFINITY;
                bm = fmaxf(bm, x[p]);
            }
            const float mn = fmaxf(m[j], bm);
            const float alpha = mn > -INFINITY ? fast_exp2(m[j] - mn) : 1.f;
            l[j] *= alpha;
#pragma unroll
            for (int e = 0; e < kEpl; ++e) acc[j][e] *= alpha;
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                // a NaN key of a valid token stays NaN, as in the scores
                const float pw = ok[p] ? fast_exp2(x[p] - mn) : 0.f;
                l[j] += pw;
#pragma unroll
                for (int e = 0; e < kEpl; ++e)
                    acc[j][e] = fmaf(pw, fs::elem<kBf16>(vv[p], e), acc[j][e]);
            }
            m[j] = mn;
        }
        if (y & (1u << 31)) {
            const int row = (int)(y & 0xffffffu);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float M = xor_max_from<kLpt>(m[j]);
                const float f = M > -INFINITY ? fast_exp2(m[j] - M) : 0.f;
                const float lt = xor_sum_from<kLpt>(l[j] * f);
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                f32x4 o0, o1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o0[e] = xor_sum_from<kLpt>(acc[j][e] * f) * inv;
                    o1[e] = xor_sum_from<kLpt>(acc[j][4 + e] * f) * inv;
                }
                float lse = lt > 0.f ? (M + fast_log2(lt)) * kLn2 : -INFINITY;
                if (sbad) {
                    o0 = f32x4{NAN, NAN, NAN, NAN};
                    o1 = o0;
                    lse = NAN;
                }
                const int slot = ku * G + j;
                if (tg == 0) {
                    *(f32x4 *)&st_o[slot * D + d0] = o0;
                    *(f32x4 *)&st_o[slot * D + d0 + 4] = o1;
                }
                if (lane == 0) {
                    st_lse[slot] = lse;
                    st_row[slot] = row + j;
                }
            }
        }
    };

    // (the prologue's loads in the loop's order: the waits in the loop are
    // counted along both the entry and the back edge)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
        issue(r, r);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll 1
    for (int t = 0; t < Tpad; t += kRing) {
#pragma unroll
        for (int r = 0; r < kRing; ++r) {
            // the scheduler must not reorder the steps: slot r's loads are
            // waited for by count, which holds only in program order
            compute(r);
            __builtin_amdgcn_sched_barrier(0);
            issue(r, t + r + kRing);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // The finished rows, two per pass (32 lanes x 4 floats each).
    const int rows = (ku + 1) * G;
#pragma unroll 1
    for (int k0 = 0; k0 < rows; k0 += 2) {
        const int k = k0 + lane / 32;
        if (k < rows) {
            const int row = st_row[k];
            const int c = (lane % 32) * 4;
            *(f32x4 *)(a.o + (int64_t)row * D + c) = *(const f32x4 *)&st_o[k * D + c];
            if (c == 0) a.lse[row] = st_lse[k];
        }
    }
}

}  // namespace hp
