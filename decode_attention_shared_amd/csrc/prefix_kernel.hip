// Prefix pass on the gfx950 matrix cores.
//
// All query rows that share a prefix node are stacked into one matrix per KV
// head: with G = Hq/Hkv query heads per KV head, the node's sequences
// [seq_begin, seq_end) give M = (seq_end - seq_begin) * G rows, and the node's
// keys are read once for all of them ("Hydragen: High-Throughput LLM Inference
// with Shared Prefixes", section "Inter-Sequence Batched Prefix Attention";
// "Shared Prefix KV Caching, in depth", section "Splitting attention at the
// prefix boundary", on the group multiplying the rows).  Keys are consumed in
// 64-key tiles with an online softmax: per tile a row max, rescale of the
// running state, exponentials, row sum and the value product ("ChunkAttention:
// Efficient Self-Attention with Prefix-Aware KV Cache and Two-Phase
// Partition", sections "The partial_attn Function", Eq. 1, and "The
// attn_reduce Function", Eq. 2, applied tile by tile).  The key range can be
// split across workgroups (that page's chunk-parallel third axis, section "The
// Chunk-First Phase Kernel in Detail"); each split writes its own normalised
// (O, LSE) partial with no atomics, merged later by the LSE merge.
//
// Layout on the matrix cores.  A wave owns 32 query rows.  It computes
// S^T = K Q^T (keys x queries) so that each lane ends up holding the scores
// of one query (lane % 32) for 16 keys per 32-key block; those probabilities
// feed O^T = V^T P^T directly as the B operand, with V staged transposed in
// LDS as the A operand.  Scores stay in fp32 and go to the exp2 domain by
// folding log2(e) into the scale; P is rounded to the input type for the
// second product, as the matrix cores require.
#include "common.hpp"

namespace hp {

constexpr int kTile = 64;  // keys per LDS tile

template <bool kBf16>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (kBf16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Which node, (KV head, split) unit and row block this workgroup owns.
// Workgroups of one unit that differ only in row block are 8 apart in the
// launch, so they land on the same XCD (dispatch is round-robin over the 8
// XCDs) and the second read of the unit's K/V tiles can hit that XCD's L2.
struct WgTask {
    int node, g, split, rb;
    bool valid;
};

__device__ __forceinline__ WgTask decode_wg(const PrefixArgs &args) {
    WgTask t;
    const int wg = blockIdx.x;
    int ni = 0;
#pragma unroll 1
    for (int i = 1; i < args.num_nodes; ++i)
        if (wg >= args.nodes[i].wg_begin) ni = i;
    const PrefixNodeArg &nd = args.nodes[ni];
    const int local = wg - nd.wg_begin;
    int unit, rb;
    if (nd.rowblocks == 1) {
        unit = local;
        rb = 0;
    } else {
        const int chunk = local / (8 * nd.rowblocks);
        const int rem = local % (8 * nd.rowblocks);
        rb = rem / 8;
        unit = chunk * 8 + rem % 8;
    }
    t.node = ni;
    t.g = unit / nd.nsplit;
    t.split = unit % nd.nsplit;
    t.rb = rb;
    t.valid = unit < args.Hkv * nd.nsplit;
    return t;
}

// Online-softmax update for one 64-key tile held as two 32x32 score blocks.
// x0/x1 hold scores already scaled to the exp2 domain (masked keys = -inf).
// Returns alpha (the rescale factor of the old state) and leaves p in x.
__device__ __forceinline__ float softmax_tile(float (&x)[32], float &m_run, float &l_run) {
    float mt = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mt = fmaxf(mt, x[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));  // the other half-wave holds the other keys of this query
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile (m_run = -inf)
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        x[i] = fast_exp2(x[i] - m_new);
        sum += x[i];
    }
    l_run = l_run * alpha + sum;
    m_run = m_new;
    return alpha;
}

template <int D>
__device__ __forceinline__ void write_row(const RowDest &dest, int split, int64_t row_index,
                                          const f32x16 (&oacc)[D / 32], int hi, float m_run,
                                          float l_run) {
    const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    float *op = dest.o + (int64_t)split * dest.o_split + row_index * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v;
            v.x = oacc[db][4 * q4 + 0] * inv;
            v.y = oacc[db][4 * q4 + 1] * inv;
            v.z = oacc[db][4 * q4 + 2] * inv;
            v.w = oacc[db][4 * q4 + 3] * inv;
            *(f32x4 *)(op + db * 32 + 8 * q4 + 4 * hi) = v;
        }
    }
    if (hi == 0 && dest.lse != nullptr)
        dest.lse[(int64_t)split * dest.lse_split + row_index] =
            empty ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// 16-bit inputs: v_mfma_f32_32x32x16_{bf16,f16}
// ---------------------------------------------------------------------------
template <bool kBf16, int D, int NW>
__global__ __launch_bounds__(64 * NW) void prefix_mfma16_kernel(PrefixArgs args) {
    constexpr int kThreads = 64 * NW;
    constexpr int kKStride = D + 8;      // halves per K row in LDS (16-byte pad)
    constexpr int kVStride = kTile + 4;  // halves per transposed V row (8-byte pad)
    constexpr int kDSteps = D / 16;
    constexpr int kDBlocks = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t ks[kTile * kKStride];
    __shared__ __attribute__((aligned(16))) uint16_t vt[D * kVStride];

    const WgTask task = decode_wg(args);
    if (!task.valid) return;
    const PrefixNodeArg &nd = args.nodes[task.node];
    const int G = args.G;
    const int M = (nd.seq_end - nd.seq_begin) * G;
    const int ntiles = (nd.len + kTile - 1) / kTile;
    const int tile_begin = task.split * nd.tiles_per_split;
    const int tile_end = min(tile_begin + nd.tiles_per_split, ntiles);

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int n = lane & 31;   // query column of this lane
    const int hi = lane >> 5;  // which half of the k-slice this lane supplies
    const int row = task.rb * 32 * NW + wave * 32 + n;
    const bool row_ok = row < M;
    const int b = nd.seq_begin + (row_ok ? row / G : 0);
    const int h = task.g * G + (row_ok ? row % G : 0);

    // Q as the B operand of S^T = K Q^T: lane holds 8 consecutive dims per k-step.
    u32x4 qf[kDSteps];
    {
        const uint16_t *qp =
            (const uint16_t *)args.q + ((int64_t)b * args.Hq + h) * D + hi * 8;
#pragma unroll
        for (int kk = 0; kk < kDSteps; ++kk)
            qf[kk] = row_ok ? *(const u32x4 *)(qp + kk * 16) : u32x4{0, 0, 0, 0};
    }

    f32x16 oacc[kDBlocks];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    const uint16_t *kbase = (const uint16_t *)nd.k + (int64_t)task.g * nd.stride_head;
    const uint16_t *vbase = (const uint16_t *)nd.v + (int64_t)task.g * nd.stride_head;

#pragma unroll 1
    for (int tile = tile_begin; tile < tile_end; ++tile) {
        const int key0 = tile * kTile;
        __syncthreads();  // the previous tile's LDS reads are done
        // Stage K (row-major) and V (transposed) for 64 keys.  Keys past the
        // node's end are zero-filled, never read.
        static_assert((kTile * D / 8) % kThreads == 0, "tile chunks must divide evenly");
#pragma unroll
        for (int it = 0; it < kTile * D / 8 / kThreads; ++it) {
            const int c = threadIdx.x + it * kThreads;
            const int key = c / (D / 8);
            const int dc = c % (D / 8);
            const int t = key0 + key;
            u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
            if (t < nd.len) {
                const int64_t off = (int64_t)t * nd.stride_tok + dc * 8;
                kv = *(const u32x4 *)(kbase + off);
                vv = *(const u32x4 *)(vbase + off);
            }
            *(u32x4 *)&ks[key * kKStride + dc * 8] = kv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vt[(dc * 8 + 2 * j) * kVStride + key] = (uint16_t)(vv[j] & 0xffffu);
                vt[(dc * 8 + 2 * j + 1) * kVStride + key] = (uint16_t)(vv[j] >> 16);
            }
        }
        __syncthreads();

        // S^T for keys [0,32) and [32,64) of the tile.
        f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
        for (int kk = 0; kk < kDSteps; ++kk) {
            const u32x4 a0 = *(const u32x4 *)&ks[n * kKStride + kk * 16 + hi * 8];
            const u32x4 a1 = *(const u32x4 *)&ks[(32 + n) * kKStride + kk * 16 + hi * 8];
            s0 = mfma32x32x16<kBf16>(a0, qf[kk], s0);
            s1 = mfma32x32x16<kBf16>(a1, qf[kk], s1);
        }
        // Accumulator i of a 32x32 block holds key 8*(i/4) + 4*hi + i%4.
        float x[32];
        const int valid = nd.len - key0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kr = 8 * (i / 4) + 4 * hi + (i % 4);
            x[i] = kr < valid ? s0[i] * args.scale_log2 : -INFINITY;
            x[16 + i] = 32 + kr < valid ? s1[i] * args.scale_log2 : -INFINITY;
        }
        const float alpha = softmax_tile(x, m_run, l_run);
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) oacc[db] *= alpha;

        // O^T += V^T P^T in four 16-key steps.  Step u takes accumulators
        // 8*(u%2) .. +8 of block u/2, i.e. keys 16u + 8*(j/4) + 4*hi + j%4 for
        // j = 0..7; the A operand reads V^T at the same keys.
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            u32x4 bop;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float p0 = x[(u / 2) * 16 + (u % 2) * 8 + 2 * w];
                const float p1 = x[(u / 2) * 16 + (u % 2) * 8 + 2 * w + 1];
                bop[w] = float_to_half_bits<kBf16>(p0) | (float_to_half_bits<kBf16>(p1) << 16);
            }
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) {
                const uint16_t *vr = &vt[(db * 32 + n) * kVStride + u * 16 + 4 * hi];
                const u32x2 lo = *(const u32x2 *)vr;
                const u32x2 up = *(const u32x2 *)(vr + 8);
                const u32x4 aop = {lo.x, lo.y, up.x, up.y};
                oacc[db] = mfma32x32x16<kBf16>(aop, bop, oacc[db]);
            }
        }
    }

    if (row_ok) {
        const int64_t ri = ((int64_t)(b - nd.dest.row_base)) * args.Hq + h;
        write_row<D>(nd.dest, task.split, ri, oacc, hi, m_run, l_run);
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs: v_mfma_f32_32x32x2f32 (no down-conversion anywhere)
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void prefix_mfma32_kernel(PrefixArgs args) {
    constexpr int kThreads = 64 * NW;
    constexpr int kKStride = D + 1;  // odd stride: rows fall in different banks
    constexpr int kDBlocks = D / 32;
    __shared__ float ks[kTile * kKStride];
    __shared__ __attribute__((aligned(16))) float vs[kTile * D];

    const WgTask task = decode_wg(args);
    if (!task.valid) return;
    const PrefixNodeArg &nd = args.nodes[task.node];
    const int G = args.G;
    const int M = (nd.seq_end - nd.seq_begin) * G;
    const int ntiles = (nd.len + kTile - 1) / kTile;
    const int tile_begin = task.split * nd.tiles_per_split;
    const int tile_end = min(tile_begin + nd.tiles_per_split, ntiles);

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int n = lane & 31;
    const int hi = lane >> 5;
    const int row = task.rb * 32 * NW + wave * 32 + n;
    const bool row_ok = row < M;
    const int b = nd.seq_begin + (row_ok ? row / G : 0);
    const int h = task.g * G + (row_ok ? row % G : 0);

    // Q as the B operand of the K=2 products: dims 2kk + hi.
    float qf[D / 2];
    {
        const float *qp = (const float *)args.q + ((int64_t)b * args.Hq + h) * D + hi;
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk) qf[kk] = row_ok ? qp[2 * kk] : 0.f;
    }
    f32x16 oacc[kDBlocks];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    const float *kbase = (const float *)nd.k + (int64_t)task.g * nd.stride_head;
    const float *vbase = (const float *)nd.v + (int64_t)task.g * nd.stride_head;

#pragma unroll 1
    for (int tile = tile_begin; tile < tile_end; ++tile) {
        const int key0 = tile * kTile;
        __syncthreads();
        static_assert((kTile * D / 4) % kThreads == 0, "tile chunks must divide evenly");
#pragma unroll
        for (int it = 0; it < kTile * D / 4 / kThreads; ++it) {
            const int c = threadIdx.x + it * kThreads;
            const int key = c / (D / 4);
            const int dc = c % (D / 4);
            const int t = key0 + key;
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (t < nd.len) {
                const int64_t off = (int64_t)t * nd.stride_tok + dc * 4;
                kv = *(const f32x4 *)(kbase + off);
                vv = *(const f32x4 *)(vbase + off);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) ks[key * kKStride + dc * 4 + j] = kv[j];
            *(f32x4 *)&vs[key * D + dc * 4] = vv;
        }
        __syncthreads();

        f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk) {
            s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[n * kKStride + 2 * kk + hi], qf[kk], s0,
                                                      0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[(32 + n) * kKStride + 2 * kk + hi],
                                                      qf[kk], s1, 0, 0, 0);
        }
        float x[32];
        const int valid = nd.len - key0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kr = 8 * (i / 4) + 4 * hi + (i % 4);
            x[i] = kr < valid ? s0[i] * args.scale_log2 : -INFINITY;
            x[16 + i] = 32 + kr < valid ? s1[i] * args.scale_log2 : -INFINITY;
        }
        const float alpha = softmax_tile(x, m_run, l_run);
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) oacc[db] *= alpha;
        // O^T += V^T P^T, one K=2 product per accumulator: k = hi selects key
        // 8*(i/4) + 4*hi + i%4 of the block, which is exactly the key this lane's
        // accumulator i holds.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kb * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
#pragma unroll
                for (int db = 0; db < kDBlocks; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        vs[key * D + db * 32 + n], x[kb * 16 + i], oacc[db], 0, 0, 0);
            }
        }
    }

    if (row_ok) {
        const int64_t ri = ((int64_t)(b - nd.dest.row_base)) * args.Hq + h;
        write_row<D>(nd.dest, task.split, ri, oacc, hi, m_run, l_run);
    }
}

template <int NW>
static hipError_t launch_nw(const PrefixArgs &a, int dtype, int d, int wgs, hipStream_t s) {
    const dim3 grid(wgs), block(64 * NW);
    if (dtype == HP_BF16) {
        if (d == 128) prefix_mfma16_kernel<true, 128, NW><<<grid, block, 0, s>>>(a);
        else prefix_mfma16_kernel<true, 64, NW><<<grid, block, 0, s>>>(a);
    } else if (dtype == HP_F16) {
        if (d == 128) prefix_mfma16_kernel<false, 128, NW><<<grid, block, 0, s>>>(a);
        else prefix_mfma16_kernel<false, 64, NW><<<grid, block, 0, s>>>(a);
    } else {
        if (d == 128) prefix_mfma32_kernel<128, NW><<<grid, block, 0, s>>>(a);
        else prefix_mfma32_kernel<64, NW><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_prefix(const PrefixArgs &a, int dtype, int d, int nw, int wgs, hipStream_t s) {
    switch (nw) {
    case 1: return launch_nw<1>(a, dtype, d, wgs, s);
    case 2: return launch_nw<2>(a, dtype, d, wgs, s);
    case 4: return launch_nw<4>(a, dtype, d, wgs, s);
    default: return launch_nw<8>(a, dtype, d, wgs, s);
    }
}

}  // namespace hp
