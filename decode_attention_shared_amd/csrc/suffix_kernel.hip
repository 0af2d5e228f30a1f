// Suffix pass: per-sequence paged decode attention.
//
// Each sequence's private keys cannot be shared with any other query, so this
// pass is a plain single-query attention per (sequence, KV head), streaming
// the sequence's 16-token blocks through its block table ("Hydragen:
// High-Throughput LLM Inference with Shared Prefixes", section "Inter-Sequence
// Batched Prefix Attention", on suffix attention; "ChunkAttention: Efficient
// Self-Attention with Prefix-Aware KV Cache and Two-Phase Partition", section
// "The Sequence-First Phase Kernel in Detail", for the per-sequence walk over
// private chunks with an online-softmax reduce).  Its arithmetic intensity is
// G FLOP per byte at most, so it is bound by HBM: the vector ALUs do the dot
// products and the matrix cores are not used.
//
// One wave owns one (sequence, KV head, block range) work item and the G
// query heads of that KV head.  A token's d values are spread over d*size/16
// lanes (16 bytes per lane, one coalesced row per lane group), so a wave
// covers 64*16/(d*size) tokens per load; the partial dot products are summed
// across the lane group, and the online-softmax state is kept per query head.
// A long suffix is split into fixed ranges of blocks across waves; each range
// writes its own normalised (O, LSE) partial for the merge.
#include "common.hpp"

namespace hp {

template <int kDt>
struct Elem;
template <>
struct Elem<HP_F32> {
    static constexpr int kSize = 4;
    __device__ static float get(const u32x4 &w, int e) { return __uint_as_float(w[e]); }
};
template <>
struct Elem<HP_F16> {
    static constexpr int kSize = 2;
    __device__ static float get(const u32x4 &w, int e) {
        return f16_bits_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    }
};
template <>
struct Elem<HP_BF16> {
    static constexpr int kSize = 2;
    __device__ static float get(const u32x4 &w, int e) {
        return bf16_bits_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    }
};

template <int kDt, int D, int G>
__global__ __launch_bounds__(256) void suffix_kernel(SuffixArgs a) {
    using E = Elem<kDt>;
    constexpr int kEpl = 16 / E::kSize;  // elements per lane per token
    constexpr int kLpt = D / kEpl;       // lanes per token
    constexpr int kTpp = kWave / kLpt;   // tokens per wave-wide load
    constexpr int kPasses = kBlock / kTpp;
    static_assert(kLpt <= kWave && kPasses >= 1, "layout");

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    const int64_t total = (int64_t)a.B * a.Hkv * a.nsplit;
    if (item >= total) return;
    const int split = (int)(item % a.nsplit);
    const int64_t bg = item / a.nsplit;
    const int g = (int)(bg % a.Hkv);
    const int b = (int)(bg / a.Hkv);
    const int tg = lane / kLpt;  // token slot within a load
    const int li = lane % kLpt;  // lane within the token's group
    const int d0 = li * kEpl;

    // The G query rows of this KV head, in fp32.
    float qf[G][kEpl];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const u32x4 w = *(const u32x4 *)((const char *)a.q +
                                         (((int64_t)b * a.Hq + g * G + j) * D + d0) * E::kSize);
#pragma unroll
        for (int e = 0; e < kEpl; ++e) qf[j][e] = E::get(w, e);
    }

    const int len = a.lens[b];
    bool bad = len < 0 || len > a.max_blocks * kBlock;
    const int nblk = bad ? 0 : (len + kBlock - 1) / kBlock;
    const int blk0 = split * a.blocks_per_split;
    const int blk1 = min(blk0 + a.blocks_per_split, nblk);

    float m[G], l[G], acc[G][kEpl];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < kEpl; ++e) acc[j][e] = 0.f;
    }

    const int64_t tok_stride = (int64_t)a.Hkv * D * E::kSize;  // bytes between tokens of a block
    const char *kp = (const char *)a.k_pool;
    const char *vp = (const char *)a.v_pool;

#pragma unroll 1
    for (int blk = blk0; blk < blk1; ++blk) {
        const int id = a.table[(int64_t)b * a.max_blocks + blk];
        if (id < 0 || id >= a.num_blocks) {  // never dereferenced; the row becomes NaN
            bad = true;
            continue;
        }
        const int64_t base = ((int64_t)id * kBlock * a.Hkv + g) * D * E::kSize + d0 * E::kSize;
        u32x4 kr[kPasses], vr[kPasses];
        bool ok[kPasses];
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const int t = p * kTpp + tg;
            ok[p] = blk * kBlock + t < len;
            const int64_t off = base + t * tok_stride;
            kr[p] = ok[p] ? *(const u32x4 *)(kp + off) : u32x4{0, 0, 0, 0};
            vr[p] = ok[p] ? *(const u32x4 *)(vp + off) : u32x4{0, 0, 0, 0};
        }
        float x[kPasses][G];
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            float kf[kEpl];
#pragma unroll
            for (int e = 0; e < kEpl; ++e) kf[e] = E::get(kr[p], e);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < kEpl; ++e) dot = fmaf(qf[j][e], kf[e], dot);
                dot = xor_sum<kLpt>(dot);
                x[p][j] = ok[p] ? dot * a.scale_log2 : -INFINITY;
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
    }

    // Sum the token groups' partial denominators and value sums.
    float *obase = a.dest.o + (int64_t)split * a.dest.o_split;
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const float lt = xor_sum_from<kLpt>(l[j]);
        float out[kEpl];
#pragma unroll
        for (int e = 0; e < kEpl; ++e) out[e] = xor_sum_from<kLpt>(acc[j][e]);
        const bool empty = !(lt > 0.f);
        const float inv = empty ? 0.f : 1.f / lt;
        float lse = empty ? -INFINITY : (m[j] + fast_log2(lt)) * kLn2;
        if (bad) lse = NAN;
        if (tg == 0) {
            const int64_t ri = ((int64_t)(b - a.dest.row_base)) * a.Hq + g * G + j;
            float *op = obase + ri * D + d0;
#pragma unroll
            for (int e = 0; e < kEpl; e += 4) {
                f32x4 v;
                v.x = bad ? NAN : out[e + 0] * inv;
                v.y = bad ? NAN : out[e + 1] * inv;
                v.z = bad ? NAN : out[e + 2] * inv;
                v.w = bad ? NAN : out[e + 3] * inv;
                *(f32x4 *)(op + e) = v;
            }
            if (li == 0 && a.dest.lse != nullptr)
                a.dest.lse[(int64_t)split * a.dest.lse_split + ri] = lse;
        }
    }
}

template <int kDt, int D>
static void launch_g(const SuffixArgs &a, int G, dim3 grid, hipStream_t s) {
    switch (G) {
    case 1: suffix_kernel<kDt, D, 1><<<grid, 256, 0, s>>>(a); break;
    case 2: suffix_kernel<kDt, D, 2><<<grid, 256, 0, s>>>(a); break;
    case 4: suffix_kernel<kDt, D, 4><<<grid, 256, 0, s>>>(a); break;
    default: suffix_kernel<kDt, D, 8><<<grid, 256, 0, s>>>(a); break;
    }
}

template <int kDt>
static void launch_dt(const SuffixArgs &a, int d, int G, dim3 grid, hipStream_t s) {
    if (d == 128) launch_g<kDt, 128>(a, G, grid, s);
    else launch_g<kDt, 64>(a, G, grid, s);
}

hipError_t launch_suffix(const SuffixArgs &a, int dtype, int d, int G, hipStream_t s) {
    const int64_t items = (int64_t)a.B * a.Hkv * a.nsplit;
    const dim3 grid((unsigned)((items + 3) / 4));
    if (dtype == HP_BF16) launch_dt<HP_BF16>(a, d, G, grid, s);
    else if (dtype == HP_F16) launch_dt<HP_F16>(a, d, G, grid, s);
    else launch_dt<HP_F32>(a, d, G, grid, s);
    return hipGetLastError();
}

}  // namespace hp
