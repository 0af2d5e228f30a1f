// Exact n-way merge of (O, LSE) partials over disjoint key sets.
//
// For the partials i of one row: m = max_i LSE_i, w_i = e^{LSE_i - m},
// O = sum_i w_i O_i / sum_i w_i, LSE = m + ln sum_i w_i.  This is the
// two-part recombination of "Hydragen: High-Throughput LLM Inference with
// Shared Prefixes" (section "Attention Decomposition Across Subsequences",
// Eq. 5, with the max subtracted as its combine_lse description gives)
// applied to all parts at once: the weights of the two-part form, composed
// over a left-to-right chain, multiply out to exactly these.  The same pass
// reduces the key-range splits of the prefix and suffix passes (the
// attn_reduce update of "ChunkAttention: Efficient Self-Attention with
// Prefix-Aware KV Cache and Two-Phase Partition", Eq. 2, with LSE = m + ln n).
//
// One thread owns 4 consecutive output elements of one row; the row's
// partial list comes from the source descriptors (tree nodes covering the
// row's sequence, and the suffix splits that hold keys).  A NaN LSE (a row
// whose device-side metadata was out of range) makes the row NaN.
#include "common.hpp"

namespace hp {

__device__ __forceinline__ int src_count(const MergeSrc &s, int64_t b, const MergeArgs &a,
                                         bool &bad) {
    if (b < s.b0 || b >= s.b1) return 0;
    if (s.split_blocks <= 0) return s.nsplit;
    const int len = a.lens[b];
    if (len < 0 || len > a.max_len) {
        bad = true;
        return 0;
    }
    const int nblk = (len + kBlock - 1) / kBlock;
    return min(s.nsplit, (nblk + s.split_blocks - 1) / s.split_blocks);
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
    constexpr int kTpr = D / 4;         // threads per row
    constexpr int kRpb = 256 / kTpr;    // rows per block
    const int64_t r = (int64_t)blockIdx.x * kRpb + threadIdx.x / kTpr;
    const int c4 = (threadIdx.x % kTpr) * 4;
    const int64_t nrows = (int64_t)(a.row_b1 - a.row_b0) * a.Hq;
    if (r >= nrows) return;
    const int64_t b = a.row_b0 + r / a.Hq;
    const int h = (int)(r % a.Hq);

    // One pass with a running max, the sum so far rescaled when a larger LSE
    // arrives; the result is the same weighted mean up to rounding order.  The
    // update has no branch, so every load of a group of partials (its LSEs and
    // its O rows) is issued before the first of them is used: one memory round
    // trip per group instead of two per partial.  An empty part (LSE -inf)
    // gets weight 0; its O row is the zero row every pass writes for it.
    bool bad = false;
    float mx = -INFINITY;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
#pragma unroll 1
    for (int si = 0; si < a.nsrc; ++si) {
        const MergeSrc &s = a.src[si];
        const int n = src_count(s, b, a, bad);
        const int64_t ri = (b - s.b0) * a.Hq + h;
#pragma unroll 4
        for (int i = 0; i < n; ++i) {
            const float L = s.lse[(int64_t)i * s.lse_split + ri];
            const f32x4 v = *(const f32x4 *)(s.o + (int64_t)i * s.o_split + ri * D + c4);
            bad |= (L != L);
            const bool live = L > -INFINITY;  // false for an empty part (and NaN, flagged)
            const float m_new = live ? fmaxf(mx, L) : mx;
            // 0 while mx = -inf (acc and wsum are 0 then); 1 when the max stays
            const float rs = m_new > mx ? fast_exp2((mx - m_new) * kLog2e) : 1.f;
            const float w = live ? fast_exp2((L - m_new) * kLog2e) : 0.f;
            acc = acc * rs + w * v;
            wsum = wsum * rs + w;
            mx = m_new;
        }
    }
    f32x4 out;
    float lse;
    if (bad) {
        out = f32x4{NAN, NAN, NAN, NAN};
        lse = NAN;
    } else if (!(mx > -INFINITY)) {
        out = f32x4{0.f, 0.f, 0.f, 0.f};
        lse = -INFINITY;
    } else {
        out = acc * (1.f / wsum);
        lse = mx + fast_log2(wsum) * kLn2;
    }
    const int64_t orow = b * a.Hq + h;
    *(f32x4 *)(a.o + orow * D + c4) = out;
    if (c4 == 0 && a.lse != nullptr) a.lse[orow] = lse;
}

hipError_t launch_merge(const MergeArgs &a, int d, hipStream_t s) {
    const int64_t nrows = (int64_t)(a.row_b1 - a.row_b0) * a.Hq;
    if (nrows <= 0) return hipSuccess;
    const int rpb = 256 / (d / 4);
    const dim3 grid((unsigned)((nrows + rpb - 1) / rpb));
    if (d == 128) merge_kernel<128><<<grid, 256, 0, s>>>(a);
    else merge_kernel<64><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace hp
