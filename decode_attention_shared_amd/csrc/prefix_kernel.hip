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
// feed O^T = V^T P^T directly as the B operand.  V is staged row-major in
// LDS like K; its transpose for the A operand comes from gfx950's
// transposing LDS read (ds_read_b64_tr_b16).  Scores stay in fp32 and go to the exp2 domain by
// folding log2(e) into the scale; P is rounded to the input type for the
// second product, as the matrix cores require.
#include "common.hpp"
#include "fat_suffix.hpp"

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

// gfx950 transposing LDS read of 4 x 16-bit: within each 16-lane group, lane i
// receives element i%4 of the 8-byte chunks read by lanes 4j + i/4, j = 0..3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t *p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(u32x2, r);
}

// Which node, (KV head, split) unit and row block this workgroup owns.
// Workgroups of one unit that differ only in row block are 8 apart in the
// launch, so they land on the same XCD (dispatch is round-robin over the 8
// XCDs) and the second read of the unit's K/V tiles can hit that XCD's L2.
struct WgTask {
    int node, g, split, rb;
    bool valid;
};

__device__ __forceinline__ WgTask decode_local(const PrefixNodeArg &nd, int local, int Hkv) {
    WgTask t;
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
    t.node = 0;
    t.g = unit / nd.nsplit;
    t.split = unit % nd.nsplit;
    t.rb = rb;
    t.valid = unit < Hkv * nd.nsplit;
    return t;
}

__device__ __forceinline__ WgTask decode_wg(const PrefixArgs &args) {
    const int wg = blockIdx.x;
    int ni = 0;
#pragma unroll 1
    for (int i = 1; i < args.num_nodes; ++i)
        if (wg >= args.nodes[i].wg_begin) ni = i;
    WgTask t = decode_local(args.nodes[ni], wg - args.nodes[ni].wg_begin, args.Hkv);
    t.node = ni;
    return t;
}

// Chunk-tree launches: the workgroup table of the plan image names this
// workgroup's segment; the segment record gives the same fields as a node
// (its keys are pool rows, its results go to the partial buffers).
__device__ __forceinline__ WgTask decode_tree_wg(const PrefixArgs &args, PrefixNodeArg &nd,
                                                 int &piece_begin) {
    const int32_t *tr = args.tree;
    const int si = tr[args.wgseg_off + args.wg0 + blockIdx.x];
    const TreeSeg sg = *(const TreeSeg *)(tr + args.seg_off + (int64_t)si * (sizeof(TreeSeg) / 4));
    const int64_t nseq = sg.seq_end - sg.seq_begin;
    nd.k = args.k_pool;
    nd.v = args.v_pool;
    nd.stride_tok = args.row_stride;
    nd.stride_head = args.d;
    nd.len = sg.ntiles * kTile;
    nd.seq_begin = sg.seq_begin;
    nd.seq_end = sg.seq_end;
    nd.nsplit = sg.nsplit;
    nd.tiles_per_split = sg.tiles_per_split;
    nd.rowblocks = sg.rowblocks;
    nd.units_padded = sg.units_padded;
    nd.wg_begin = sg.wg_begin;
    nd.dest.o = args.part_o + (int64_t)sg.part_row0 * args.Hq * args.d;
    nd.dest.lse = args.part_lse + (int64_t)sg.part_row0 * args.Hq;
    nd.dest.o_split = nseq * args.Hq * args.d;
    nd.dest.lse_split = nseq * args.Hq;
    nd.dest.row_base = sg.seq_begin;
    piece_begin = sg.piece_begin;
    return decode_local(nd, (int)blockIdx.x - sg.wg_begin, args.Hkv);
}

// Where the keys of a tile come from.  key0(t): row offset of tile t's first
// key from the node's base (in rows of stride_tok); valid(t): keys the tile
// holds (values of 64 or more mean a full tile).
//
// A node stored contiguously: tile t holds keys 64t .. 64t + 63, and only the
// node's last tile can be partial.
struct ContigTiles {
    int len;
    __device__ __forceinline__ int key0(int tile) const { return tile * kTile; }
    __device__ __forceinline__ int valid(int tile) const { return len - tile * kTile; }
};
// A chunk-tree segment: tile t is one piece (up to 64 consecutive pool rows),
// and any piece may be partial.  Lane l holds piece tb + l of this split;
// a tile's fields are read from that lane into scalar registers.
struct ChunkTiles {
    int tb;
    int row_l, cnt_l;
    __device__ __forceinline__ int key0(int tile) const {
        return __builtin_amdgcn_readlane(row_l, tile - tb);
    }
    __device__ __forceinline__ int valid(int tile) const {
        return __builtin_amdgcn_readlane(cnt_l, tile - tb);
    }
};

__device__ __forceinline__ ChunkTiles load_pieces(const PrefixArgs &args, int piece_begin, int tb,
                                                  int te) {
    ChunkTiles src;
    src.tb = tb;
    const int l = threadIdx.x % kWave;
    src.row_l = 0;
    src.cnt_l = 0;
    if (tb + l < te) {
        const TreePiece p =
            *(const TreePiece *)(args.tree + args.piece_off + 2 * ((int64_t)piece_begin + tb + l));
        src.row_l = p.row;
        src.cnt_l = p.count;
    }
    return src;
}

// Max of x over this lane and the lane 32 apart (the other half-wave), with
// gfx950's v_permlane32_swap: the exchange stays in the vector ALU instead of
// queueing on the LDS crossbar (as ds_bpermute would) behind the operand
// reads of the other waves.  The two results hold x of lane l and of lane
// l ^ 32 in some order, so their max is the same on both halves.
__device__ __forceinline__ float max_across_halves(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// Online-softmax update for one 64-key tile held as two 32x32 score blocks.
// x0/x1 hold scores already scaled to the exp2 domain (masked keys = -inf).
// Returns alpha (the rescale factor of the old state) and leaves p in x.
__device__ __forceinline__ float softmax_tile(float (&x)[32], float &m_run, float &l_run) {
    float mt = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mt = fmaxf(mt, x[i]);
    mt = max_across_halves(mt);  // the other half-wave holds the other keys of this query
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
                                          float l_run, float l_lse) {
    const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
    const float l_lse_tot = l_lse + __shfl_xor(l_lse, 32, kWave);
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
            empty ? -INFINITY : (m_run + fast_log2(l_lse_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// 16-bit inputs: v_mfma_f32_32x32x16_{bf16,f16}
// ---------------------------------------------------------------------------

// Lazy rescaling threshold (log2 units).  The running max only moves when a
// row's tile max exceeds it by more than this; until then probabilities may
// reach 2^8, which the fp32 accumulators and the 16-bit P operand hold with
// their usual relative precision, and the per-tile rescale of the O
// accumulators is skipped.  The result is the same softmax: O / l and
// m + log2 l do not depend on which shift m was used.
constexpr float kLazy = 8.f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 probabilities rounded (nearest even) to the 16-bit type, packed
// (one v_cvt_pk_{f16,bf16}_f32).
template <bool kBf16>
__device__ __forceinline__ uint32_t pack_p(float a, float b) {
    const f32x2 v = {a, b};
    if constexpr (kBf16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// sum + (the two packed 16-bit values), accumulated in fp32 (v_dot2c with ones).
template <bool kBf16>
__device__ __forceinline__ float add_packed(uint32_t pk, float sum) {
    if constexpr (kBf16) {
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), ones, sum, false);
    } else {
        const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), ones, sum, false);
    }
}

// Running softmax denominators of one row (this lane's keys).  `o` sums the
// probabilities after rounding to the 16-bit P operand, so that the weights
// O is divided by are the ones the value product used.  The log-sum-exp needs
// the sum before rounding: rounding each term moves the log of the sum by at
// most the type's unit roundoff, 2^-11 (4.9e-4) for fp16 but 2^-8 (3.9e-3) for
// bf16, so bf16 keeps the unrounded sum as well.
template <bool kBf16>
struct RowSum {
    float o = 0.f;
    float x = 0.f;  // bf16 only: the probabilities before rounding
    __device__ __forceinline__ void scale(float a) {
        o *= a;
        if constexpr (kBf16) x *= a;
    }
    __device__ __forceinline__ float lse() const { return kBf16 ? x : o; }
};

// Online softmax for one 64-key tile of raw scores q.k (masked keys are
// -inf), in two halves.  softmax_max: the tile's row max (both half-waves hold
// keys of the same query) and, when it exceeds the running max by more than
// kLazy, the new max and the factor alpha by which the running state must be
// rescaled (the return value, wave-uniform).  softmax_exp: the probabilities
// 2^(s*c - m) with c = scale * log2(e), packed into 16 pairs of the 16-bit
// type (the B operand of the value product), and the row sums.
template <bool kBf16>
__device__ __forceinline__ bool softmax_max(const f32x16 &s0, const f32x16 &s1, float c,
                                            float &m_run, RowSum<kBf16> &l, float &alpha) {
    // maximum (not fmaxf): no NaN canonicalisation of every input, and
    // v_maximum3 takes two new scores per instruction.
    // four independent chains, then a short tree (latency, not op count)
    float mq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) mq[r] = __builtin_elementwise_maximum(s0[r], s1[r]);
#pragma unroll
    for (int i = 4; i < 16; ++i)
        mq[i % 4] = __builtin_elementwise_maximum(mq[i % 4],
                                                  __builtin_elementwise_maximum(s0[i], s1[i]));
    float mt = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mq[0], mq[1]),
                                             __builtin_elementwise_maximum(mq[2], mq[3]));
    mt = max_across_halves(mt);  // the other half-wave: the other keys of this query
    const float mts = mt * c;  // c > 0: the max commutes with the scaling
    const bool rescale = __any(mts > m_run + kLazy);
    alpha = 1.f;
    if (rescale) {
        const float m_new = fmaxf(m_run, mts);
        alpha = fast_exp2(m_run - m_new);  // 0 on the first tile (m_run = -inf)
        l.scale(alpha);
        m_run = m_new;
    }
    return rescale;
}

template <bool kBf16>
__device__ __forceinline__ void softmax_exp(const f32x16 &s0, const f32x16 &s1, float c,
                                            float m_run, RowSum<kBf16> &l, uint32_t (&pk)[16]) {
    const float neg_m = -m_run;
    float sq[4] = {0.f, 0.f, 0.f, 0.f};  // independent accumulation chains
    float sx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const f32x16 &s = i < 8 ? s0 : s1;
        const int j = 2 * (i % 8);
        const float a = fast_exp2(fmaf(s[j], c, neg_m));
        const float b = fast_exp2(fmaf(s[j + 1], c, neg_m));
        pk[i] = pack_p<kBf16>(a, b);
        sq[i % 4] = add_packed<kBf16>(pk[i], sq[i % 4]);
        if constexpr (kBf16) sx[i % 4] += a + b;
    }
    l.o += (sq[0] + sq[1]) + (sq[2] + sq[3]);
    if constexpr (kBf16) l.x += (sx[0] + sx[1]) + (sx[2] + sx[3]);
}

// Position of a V row's 16-byte chunks in LDS: chunk c of row r sits at
// c ^ v_swizzle(r).  The transposing read of one half-wave touches 4 rows x
// 4 consecutive chunks; spreading rows 4 chunks apart within each 256-byte
// bank line puts those 256 bytes on distinct banks.
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
    return 4 * ((r / (128 / D)) % (D / 32));
}

// Workgroup barrier that the compiler may not move memory accesses across
// (LDS is written by DMA outside its view), taken after this wave's own LDS
// reads have returned.
__device__ __forceinline__ void block_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <bool kBf16, int D, int NW, class Tiles>
__device__ __forceinline__ void mfma16_body(const PrefixArgs &args, const WgTask &task,
                                            const PrefixNodeArg &nd, const Tiles &src, int tb,
                                            int te) {
    constexpr int kDSteps = D / 16;
    constexpr int kDBlocks = D / 32;
    constexpr int kRowChunks = D / 8;                     // 16-byte chunks per K/V row
    constexpr int kRowsPerDma = kWave / kRowChunks;       // rows one wave-wide DMA fills
    constexpr int kDmas = kTile / kRowsPerDma / NW;       // DMAs per tensor per wave per tile
    static_assert(kDmas >= 1 && kTile % (kRowsPerDma * NW) == 0, "tile split");
    constexpr int kPerTile = 2 * kDmas;                   // K and V DMAs per wave per tile
    // K/V tiles stream through a ring of LDS stages, filled by DMA (no
    // registers involved), several tiles ahead of the math: each CU needs
    // tens of KB in flight to cover HBM latency.  Iteration i computes
    // S(i+1) = K(i+1) Q^T on the matrix cores interleaved with the softmax of
    // tile i on the vector ALUs, then O += V(i) P(i), and issues tile
    // i + kStages - 1 into the stage tile i-1 used.
    constexpr int kStages = NW >= 4 ? 4 : 3;
    constexpr int kAhead = kStages - 3;  // tiles issued beyond i+1 when waiting for i+1
    static_assert(kPerTile * (kStages - 2) < 64, "vmcnt range");
    constexpr int kTileElems = kTile * D;
    // Rows are unpadded; 16-byte chunk c of row r sits at position c ^ swz(r).
    // K: 16 consecutive rows hit 16 different chunk positions (the 32 lanes of
    // an operand read take 32 different rows).  V: the four rows one 16-lane
    // group of the transposing read touches land 2 chunks apart.
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kStages][2][kTileElems];

    const int G = args.G;
    const int M = (nd.seq_end - nd.seq_begin) * G;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int n = lane & 31;   // query column of this lane
    const int hi = lane >> 5;  // which half of the k-slice this lane supplies
    const int row = task.rb * 32 * NW + wave * 32 + n;
    const bool row_ok = row < M;
    const int b = nd.seq_begin + (row_ok ? row / G : 0);
    const int h = task.g * G + (row_ok ? row % G : 0);
    const float c = args.scale_log2;

    // Q as the B operand of S^T = K Q^T: lane holds 8 consecutive dims per k-step.
    // Loaded once the first tiles' transfers are issued (below), then waited for
    // together with them: the compiler does not count the transfers, so a wait
    // for Q inside the tile loop would drain every transfer in flight.
    u32x4 qf[kDSteps];
    const uint16_t *qp = (const uint16_t *)args.q + ((int64_t)b * args.Hq + h) * D + hi * 8;
    auto load_q = [&]() {
#pragma unroll
        for (int kk = 0; kk < kDSteps; ++kk)
            qf[kk] = row_ok ? *(const u32x4 *)(qp + kk * 16) : u32x4{0, 0, 0, 0};
        wait_vmcnt<0>();
    };

    f32x16 oacc[kDBlocks];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;
    RowSum<kBf16> l;

    const uint16_t *kbase = (const uint16_t *)nd.k + (int64_t)task.g * nd.stride_head;
    const uint16_t *vbase = (const uint16_t *)nd.v + (int64_t)task.g * nd.stride_head;

    // DMA j of this wave fills rows rj .. rj + kRowsPerDma of a tile; lane
    // `lane` lands at row rj + lane / kRowChunks, position lane % kRowChunks,
    // so it fetches the logical chunk that belongs there.
    int dma_row[kDmas], dma_ck[kDmas], dma_cv[kDmas];
#pragma unroll
    for (int j = 0; j < kDmas; ++j) {
        const int r = (wave * kDmas + j) * kRowsPerDma + lane / kRowChunks;
        const int pos = lane % kRowChunks;
        dma_row[j] = r;
        dma_ck[j] = (pos ^ (r % kRowChunks)) * 8;
        dma_cv[j] = (pos ^ (2 * (r % (kRowChunks / 2)))) * 8;
    }
    auto issue = [&](int tile) {
        const int st = (tile - tb) % kStages;
        const int key0 = src.key0(tile);
        const int valid = src.valid(tile);
        const bool full = valid >= kTile;
#pragma unroll
        for (int j = 0; j < kDmas; ++j) {
            // keys past the tile's end re-read its last key (finite data whose
            // scores are masked to -inf)
            const int t = key0 + (full ? dma_row[j] : min(dma_row[j], valid - 1));
            const int64_t off = (int64_t)t * nd.stride_tok;
            uint16_t *dst = &lds[st][0][(wave * kDmas + j) * kRowsPerDma * D];
            dma16(kbase + off + dma_ck[j], dst);
            dma16(vbase + off + dma_cv[j], dst + kTileElems);
        }
    };

    // Operand reads.  K: rows n and 32+n (same swizzle), logical chunk 2kk+hi.
    const int k_swz = n % kRowChunks;
    auto qk = [&](int st, f32x16 &s0, f32x16 &s1) {
        const uint16_t *kb = &lds[st][0][n * D];
        s0 = f32x16{};
        s1 = f32x16{};
#pragma unroll
        for (int kk = 0; kk < kDSteps; ++kk) {
            const int col = ((2 * kk + hi) ^ k_swz) * 8;
            const u32x4 a0 = *(const u32x4 *)&kb[col];
            const u32x4 a1 = *(const u32x4 *)&kb[32 * D + col];
            s0 = mfma32x32x16<kBf16>(a0, qf[kk], s0);
            s1 = mfma32x32x16<kBf16>(a1, qf[kk], s1);
        }
    };
    // V^T operand: 16-lane group gi covers 16 consecutive d rows; within it
    // lane 4j + q reads 4 dims of key j, and the transposing read hands lane i
    // the value of each of the 4 keys at dim (group base + i).  Keys 16u + 4hi
    // + li/4 (and + 8) share the swizzle 2*(key % (kRowChunks/2)).
    const int gi = lane >> 4, li = lane & 15;
    const int v_key = 4 * hi + (li >> 2);
    const int v_swz = 2 * (v_key % (kRowChunks / 2));
    int v_col[kDBlocks];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
        v_col[db] = v_key * D + ((4 * db + 2 * (gi & 1) + ((li & 3) >> 1)) ^ v_swz) * 8 +
                    (li & 1) * 4;
    auto pv = [&](const uint32_t (&pk)[16], int st) {
        const uint16_t *vb = &lds[st][1][0];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 bop = {pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]};
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) {
                const uint16_t *vr = vb + 16 * u * D + v_col[db];
                const u32x2 lo = lds_read_tr16(vr);           // keys 16u + 4hi + 0..3
                const u32x2 up = lds_read_tr16(vr + 8 * D);   // keys 16u + 8 + 4hi + 0..3
                const u32x4 aop = {lo.x, lo.y, up.x, up.y};
                oacc[db] = mfma32x32x16<kBf16>(aop, bop, oacc[db]);
            }
        }
    };
    // One tile: softmax of `tile` (scores sc) interleaved with S(tile+1) -> sn,
    // then the value product.  On a split's last tile the next-S product reads
    // a stale (in-bounds) stage and is discarded.
    auto step = [&](int tile, f32x16 &sc0, f32x16 &sc1, f32x16 &sn0, f32x16 &sn1) {
        // wait for this wave's DMAs of tile+1, then for everyone's
        if constexpr (kAhead > 0) {
            if (tile + 2 < te) wait_vmcnt<kAhead * kPerTile>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        block_sync();
        if (tile + kStages - 1 < te) issue(tile + kStages - 1);

        // Accumulator i of a 32x32 block holds key 8*(i/4) + 4*hi + i%4.
        const int valid = src.valid(tile);
        if (valid < kTile) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kr = 8 * (i / 4) + 4 * hi + (i % 4);
                if (kr >= valid) sc0[i] = -INFINITY;
                if (32 + kr >= valid) sc1[i] = -INFINITY;
            }
        }
        float alpha;
        if (softmax_max<kBf16>(sc0, sc1, c, m_run, l, alpha)) {
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) oacc[db] *= alpha;
        }
        qk((tile + 1 - tb) % kStages, sn0, sn1);
        uint32_t pk[16];
        softmax_exp<kBf16>(sc0, sc1, c, m_run, l, pk);
        pv(pk, (tile - tb) % kStages);
#pragma unroll
        for (int k = 0; k < 2 * kDSteps + 4 * kDBlocks; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
        }
    };

    if (tb < te) {
        // Prologue: tiles tb .. tb + kStages - 2 in flight, wait for tb, S(tb).
#pragma unroll
        for (int k = 0; k < kStages - 1; ++k)
            if (tb + k < te) issue(tb + k);
        load_q();  // also lands the prologue tiles
        const int younger = min(kStages - 2, te - tb - 1);
        if constexpr (kStages >= 4) {
            if (younger >= 2) wait_vmcnt<2 * kPerTile>();
            else if (younger == 1) wait_vmcnt<kPerTile>();
            else wait_vmcnt<0>();
        } else {
            if (younger >= 1) wait_vmcnt<kPerTile>();
            else wait_vmcnt<0>();
        }
        block_sync();
        f32x16 sa0, sa1, sb0, sb1;
        qk(0, sa0, sa1);
        int tile = tb;
#pragma unroll 1
        for (; tile + 1 < te; tile += 2) {  // two tiles per trip: the S sets alternate
            step(tile, sa0, sa1, sb0, sb1);
            step(tile + 1, sb0, sb1, sa0, sa1);
        }
        if (tile < te) step(tile, sa0, sa1, sb0, sb1);
    }

    if (row_ok) {
        const int64_t ri = ((int64_t)(b - nd.dest.row_base)) * args.Hq + h;
        write_row<D>(nd.dest, task.split, ri, oacc, hi, m_run, l.o, l.lse());
    }
}

template <bool kBf16, int D, int NW>
__global__ __launch_bounds__(64 * NW) void prefix_mfma16_kernel(PrefixArgs args) {
    const WgTask task = decode_wg(args);
    if (!task.valid) return;
    const PrefixNodeArg &nd = args.nodes[task.node];
    const int ntiles = (nd.len + kTile - 1) / kTile;
    const int tb = task.split * nd.tiles_per_split;  // first tile of this split
    const int te = min(tb + nd.tiles_per_split, ntiles);
    mfma16_body<kBf16, D, NW>(args, task, nd, ContigTiles{nd.len}, tb, te);
}

template <bool kBf16, int D, int NW>
__global__ __launch_bounds__(64 * NW) void tree_mfma16_kernel(PrefixArgs args) {
    PrefixNodeArg nd;
    int piece_begin;
    const WgTask task = decode_tree_wg(args, nd, piece_begin);
    if (!task.valid) return;
    const int ntiles = nd.len / kTile;
    const int tb = task.split * nd.tiles_per_split;
    const int te = min(tb + nd.tiles_per_split, ntiles);
    mfma16_body<kBf16, D, NW>(args, task, nd, load_pieces(args, piece_begin, tb, te), tb, te);
}

// ---------------------------------------------------------------------------
// Ping-pong variant for 256 rows per workgroup: 8 waves of 32 rows.  Waves w
// and w+4 of a workgroup share a SIMD, so waves 0-3 and 4-7 form two groups
// with one wave on every SIMD.  The groups run half a tile apart: while one
// wave of a SIMD issues its matrix products (scores of tile u and the value
// product of tile u-1) the other runs the softmax of its latest tile on the
// vector ALUs, and the two swap roles at every workgroup barrier, so the
// matrix core and the vector ALUs of a SIMD can work at the same time.
// ---------------------------------------------------------------------------

// The LDS ring is the body's own static array, or (kExtLds) the one a
// kernel that also runs other work passes in (ext_lds, kStages x 2 tiles).
template <bool kBf16, int D, bool kNT, class Tiles, bool kExtLds = false>
__device__ __forceinline__ void pp_body(const PrefixArgs &args, const WgTask &task,
                                        const PrefixNodeArg &nd, const Tiles &src, int tb,
                                        int te, uint16_t *ext_lds = nullptr) {
    constexpr int NW = 8;
    constexpr int kDSteps = D / 16;
    constexpr int kDBlocks = D / 32;
    constexpr int kRowChunks = D / 8;
    constexpr int kRowsPerDma = kWave / kRowChunks;
    constexpr int kDmas = kTile / kRowsPerDma / NW;
    static_assert(kDmas >= 1 && kTile % (kRowsPerDma * NW) == 0, "tile split");
    constexpr int kPerTile = 2 * kDmas;
    // Tile u+2 is issued once both groups are past the value product of
    // tile u-2, whose stage it takes: four stages, two tiles in flight.
    constexpr int kStages = 4;
    constexpr int kTileElems = kTile * D;
    using Ring = uint16_t[kStages][2][kTileElems];
    __shared__ __attribute__((aligned(1024)))
    uint16_t own_lds[kExtLds ? 1 : kStages][2][kExtLds ? 1 : kTileElems];
    Ring &lds = *reinterpret_cast<Ring *>(kExtLds ? ext_lds : &own_lds[0][0][0]);

    const int G = args.G;
    const int M = (nd.seq_end - nd.seq_begin) * G;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int grp = wave >> 2;
    const int n = lane & 31;
    const int hi = lane >> 5;
    const int row = task.rb * 32 * NW + wave * 32 + n;
    const bool row_ok = row < M;
    const int b = nd.seq_begin + (row_ok ? row / G : 0);
    const int h = task.g * G + (row_ok ? row % G : 0);
    const float c = args.scale_log2;

    // Q (B operand of the score product), loaded after the first two tiles'
    // transfers are issued and waited for with them (see the 32-row body).
    u32x4 qf[kDSteps];
    const uint16_t *qp = (const uint16_t *)args.q + ((int64_t)b * args.Hq + h) * D + hi * 8;
    f32x16 oacc[kDBlocks];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;
    RowSum<kBf16> l;

    // Node fields the loop needs, read once (the compiler would otherwise
    // reload them from the argument segment, a scalar-memory round trip, at
    // every tile).
    const int64_t stride_tok = nd.stride_tok;
    const uint16_t *kbase = (const uint16_t *)nd.k + (int64_t)task.g * nd.stride_head;
    const uint16_t *vbase = (const uint16_t *)nd.v + (int64_t)task.g * nd.stride_head;
    // Per-lane element offsets of this wave's DMAs within a tile, in 32 bits
    // (the launch picks this kernel only when kTile * stride_tok + d fits in
    // int32); per tile only a wave-uniform tile offset is added.
    int dma_row[kDmas];
    uint32_t koff[kDmas], voff[kDmas];  // bytes
#pragma unroll
    for (int j = 0; j < kDmas; ++j) {
        const int r = (wave * kDmas + j) * kRowsPerDma + lane / kRowChunks;
        const int pos = lane % kRowChunks;
        dma_row[j] = r;
        koff[j] = 2u * ((uint32_t)(r * stride_tok) + (pos ^ (r % kRowChunks)) * 8);
        voff[j] = 2u * ((uint32_t)(r * stride_tok) + (pos ^ v_swizzle<D>(r)) * 8);
    }
    // The transfers are issued with scalar instructions only: the wave index
    // and the LDS destinations live in scalar registers (the vector ALU is
    // held by the other group's matrix products while this runs).
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)&lds[0][0][0];
    auto issue = [&](int tile) {
        const int st = (tile - tb) % kStages;
        const int key0 = __builtin_amdgcn_readfirstlane(src.key0(tile));
        const int valid = __builtin_amdgcn_readfirstlane(src.valid(tile));  // a scalar branch
        const int64_t tile_off = (int64_t)key0 * stride_tok;
        const uint16_t *kt = kbase + tile_off;
        const uint16_t *vt = vbase + tile_off;
        const uint32_t kdst = lds0 + 2u * (uint32_t)(st * 2 * kTileElems +
                                                     wave_s * kDmas * kRowsPerDma * D);
        const uint32_t vdst = kdst + 2u * kTileElems;
        // element offsets below kTile * stride_tok + d < 2^31: the byte offsets fit
        if (valid >= kTile) {
#pragma unroll
            for (int j = 0; j < kDmas; ++j) {
                dma16_s<kNT>(kt, koff[j], kdst + 2u * j * kRowsPerDma * D);
                dma16_s<kNT>(vt, voff[j], vdst + 2u * j * kRowsPerDma * D);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kDmas; ++j) {
                uint32_t ko = koff[j], vo = voff[j];
                if (dma_row[j] >= valid) {
                    // keys past the tile's end re-read its last key (masked to -inf)
                    const uint32_t back = 2u * (uint32_t)((dma_row[j] - (valid - 1)) * stride_tok);
                    ko -= back;
                    vo -= back;
                }
                dma16_s<kNT>(kt, ko, kdst + 2u * j * kRowsPerDma * D);
                dma16_s<kNT>(vt, vo, vdst + 2u * j * kRowsPerDma * D);
            }
        }
    };
    const int k_swz = n % kRowChunks;
    f32x16 s0, s1;  // scores of the latest tile (keys 0-31, 32-63)
    const int gi = lane >> 4, li = lane & 15;
    const int v_key = 4 * hi + (li >> 2);
    const int v_swz = v_swizzle<D>(v_key);
    int v_col[kDBlocks];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
        v_col[db] = v_key * D + ((4 * db + 2 * (gi & 1) + ((li & 3) >> 1)) ^ v_swz) * 8 +
                    (li & 1) * 4;
    uint32_t pk[16];  // probabilities of the latest softmaxed tile
    // V operands stream two key-steps ahead of the products that use them.
    auto pv = [&](int st) {
        const uint16_t *vb = &lds[st][1][0];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 bop = {pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]};
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) {
                const uint16_t *vr = vb + 16 * u * D + v_col[db];
                const u32x2 lo = lds_read_tr16(vr);
                const u32x2 up = lds_read_tr16(vr + 8 * D);
                const u32x4 aop = {lo.x, lo.y, up.x, up.y};
                oacc[db] = mfma32x32x16<kBf16>(aop, bop, oacc[db]);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * kDBlocks, 0);  // reads of steps 0, 1
        __builtin_amdgcn_sched_group_barrier(0x008, kDBlocks, 0);      // products of step 0
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kDBlocks, 0);  // reads of step 2
        __builtin_amdgcn_sched_group_barrier(0x008, kDBlocks, 0);      // products of step 1
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kDBlocks, 0);  // reads of step 3
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * kDBlocks, 0);  // products of steps 2, 3
    };
    // K operands of this wave's next matrix phase: the first kPre k-steps are
    // read during its vector phase (LDS reads take no vector-ALU issue slots,
    // so their latency hides behind the softmax and the score products start
    // with operands in hand), the rest at the start of the matrix phase,
    // behind the first products.  Prefetching all of them would not fit in
    // the registers beside the softmax.
    constexpr int kPre = kDSteps / 4;
    u32x4 kpre[kDSteps][2];
    auto load_k_steps = [&](int st, int k0, int k1) {
        const uint16_t *kb = &lds[st][0][n * D];
#pragma unroll
        for (int kk = k0; kk < k1; ++kk) {
            const int col = ((2 * kk + hi) ^ k_swz) * 8;
            kpre[kk][0] = *(const u32x4 *)&kb[col];
            kpre[kk][1] = *(const u32x4 *)&kb[32 * D + col];
        }
    };
    auto load_k = [&](int st) { load_k_steps(st, 0, kPre); };
    int kst = 0;  // stage of the tile whose K is (partly) prefetched
    auto qk_pre = [&]() {
        load_k_steps(kst, kPre, kDSteps);
        s0 = f32x16{};
        s1 = f32x16{};
#pragma unroll
        for (int kk = 0; kk < kDSteps; ++kk) {
            s0 = mfma32x32x16<kBf16>(kpre[kk][0], qf[kk], s0);
            s1 = mfma32x32x16<kBf16>(kpre[kk][1], qf[kk], s1);
        }
    };
    // Both products of one matrix phase: the V operands (transposing reads,
    // slower than 16-byte ones) are read while the score products run, a
    // quarter after each pair of them, into the registers the consumed K
    // operands free; the value product then starts with its operands in hand.
    auto qkpv_pre = [&](int stv) {
        const uint16_t *vb = &lds[stv][1][0];
        u32x4 va[4][kDBlocks];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) {
                const uint16_t *vr = vb + 16 * u * D + v_col[db];
                const u32x2 lo = lds_read_tr16(vr);
                const u32x2 up = lds_read_tr16(vr + 8 * D);
                va[u][db] = u32x4{lo.x, lo.y, up.x, up.y};
            }
        qk_pre();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 bop = {pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]};
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) oacc[db] = mfma32x32x16<kBf16>(va[u][db], bop, oacc[db]);
        }
        constexpr int kVReadsPerPair = 8 * kDBlocks / kDSteps;
        static_assert(kVReadsPerPair * kDSteps == 8 * kDBlocks, "V reads spread over the pairs");
#pragma unroll
        for (int kk = 0; kk < kDSteps; ++kk) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);               // two score products
            __builtin_amdgcn_sched_group_barrier(0x100, kVReadsPerPair, 0);  // a share of V
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * kDBlocks, 0);  // the value products
    };
    const int T = te - tb;
    // Vector phase: online softmax of tile u (scores in s0/s1) into pk.  O
    // already holds every earlier tile, so a rescale applies to all of it.
    auto vphase = [&](int u) {
        const int valid = src.valid(tb + u);
        if (valid < kTile) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kr = 8 * (i / 4) + 4 * hi + (i % 4);
                if (kr >= valid) s0[i] = -INFINITY;
                if (32 + kr >= valid) s1[i] = -INFINITY;
            }
        }
        float alpha;
        if (softmax_max<kBf16>(s0, s1, c, m_run, l, alpha)) {
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) oacc[db] *= alpha;
        }
        softmax_exp<kBf16>(s0, s1, c, m_run, l, pk);
    };

    if (T > 0) {
        issue(tb);
        if (T > 1) issue(tb + 1);
#pragma unroll
        for (int kk = 0; kk < kDSteps; ++kk)
            qf[kk] = row_ok ? *(const u32x4 *)(qp + kk * 16) : u32x4{0, 0, 0, 0};
        wait_vmcnt<0>();  // Q and the first two tiles
        block_sync();
        if (grp == 0) load_k(0);  // kst = 0
        // Vector phase of tile x with the K prefetch of tile x + 1.
        auto vp = [&](int x) {
            if (x + 1 < T) {
                kst = (x + 1) % kStages;
                load_k(kst);
            }
            if (x >= 0 && x < T) vphase(x);
        };
        // Step u: group 0 takes the matrix phase of u (S(u), O += V(u-1)
        // P(u-1)) then the vector phase of u; group 1 the vector phase of u-1
        // then the matrix phase of u.  Tile u+1 is waited for at the middle
        // barrier, since its K operands are read in the second half.  Tile
        // u+2 goes into the stage of tile u-2, whose last reads (K prefetches
        // in the step before last, the value products in the last step) are
        // behind the step's first barrier.  The first and last steps (a lone
        // score or value product) are peeled off so that the loop body holds
        // only the fused phase.
        auto step = [&](int u, auto &&mphase) {
            if (u > 0) block_sync();
            if (u + 2 < T) issue(tb + u + 2);
            if (grp == 0) mphase(u);
            else vp(u - 1);
            if (u + 1 < T) {
                if (u + 2 < T) wait_vmcnt<kPerTile>();
                else wait_vmcnt<0>();
            }
            block_sync();
            if (grp == 0) vp(u);
            else mphase(u);
        };
        step(0, [&](int) { qk_pre(); });
#pragma unroll 1
        for (int u = 1; u < T; ++u) step(u, [&](int w) { qkpv_pre((w - 1) % kStages); });
        step(T, [&](int w) { pv((w - 1) % kStages); });
    }

    if (row_ok) {
        const int64_t ri = ((int64_t)(b - nd.dest.row_base)) * args.Hq + h;
        write_row<D>(nd.dest, task.split, ri, oacc, hi, m_run, l.o, l.lse());
    }
}

template <bool kBf16, int D, bool kNT>
__global__ __launch_bounds__(512) void prefix_mfma16_pp_kernel(PrefixArgs args) {
    const WgTask task = decode_wg(args);
    if (!task.valid) return;
    const PrefixNodeArg &nd = args.nodes[task.node];
    const int ntiles = (nd.len + kTile - 1) / kTile;
    const int tb = task.split * nd.tiles_per_split;
    const int te = min(tb + nd.tiles_per_split, ntiles);
    pp_body<kBf16, D, kNT>(args, task, nd, ContigTiles{nd.len}, tb, te);
}

template <bool kBf16, int D>
__global__ __launch_bounds__(512) void tree_mfma16_pp_kernel(PrefixArgs args) {
    PrefixNodeArg nd;
    int piece_begin;
    const WgTask task = decode_tree_wg(args, nd, piece_begin);
    if (!task.valid) return;
    const int ntiles = nd.len / kTile;
    const int tb = task.split * nd.tiles_per_split;
    const int te = min(tb + nd.tiles_per_split, ntiles);
    pp_body<kBf16, D, false>(args, task, nd, load_pieces(args, piece_begin, tb, te), tb, te);
}

// ---------------------------------------------------------------------------
// fp32 inputs: v_mfma_f32_32x32x2f32 (no down-conversion anywhere)
// ---------------------------------------------------------------------------
template <int D, int NW, class Tiles>
__device__ __forceinline__ void mfma32_body(const PrefixArgs &args, const WgTask &task,
                                            const PrefixNodeArg &nd, const Tiles &src,
                                            int tile_begin, int tile_end) {
    constexpr int kThreads = 64 * NW;
    constexpr int kKStride = D + 1;  // odd stride: rows fall in different banks
    constexpr int kDBlocks = D / 32;
    __shared__ float ks[kTile * kKStride];
    __shared__ __attribute__((aligned(16))) float vs[kTile * D];

    const int G = args.G;
    const int M = (nd.seq_end - nd.seq_begin) * G;

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
        const int key0 = src.key0(tile);
        const int valid = src.valid(tile);
        __syncthreads();
        static_assert((kTile * D / 4) % kThreads == 0, "tile chunks must divide evenly");
#pragma unroll
        for (int it = 0; it < kTile * D / 4 / kThreads; ++it) {
            const int c = threadIdx.x + it * kThreads;
            const int key = c / (D / 4);
            const int dc = c % (D / 4);
            const int t = key0 + key;
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (key < valid) {
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
        write_row<D>(nd.dest, task.split, ri, oacc, hi, m_run, l_run, l_run);
    }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void prefix_mfma32_kernel(PrefixArgs args) {
    const WgTask task = decode_wg(args);
    if (!task.valid) return;
    const PrefixNodeArg &nd = args.nodes[task.node];
    const int ntiles = (nd.len + kTile - 1) / kTile;
    const int tb = task.split * nd.tiles_per_split;
    const int te = min(tb + nd.tiles_per_split, ntiles);
    mfma32_body<D, NW>(args, task, nd, ContigTiles{nd.len}, tb, te);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void tree_mfma32_kernel(PrefixArgs args) {
    PrefixNodeArg nd;
    int piece_begin;
    const WgTask task = decode_tree_wg(args, nd, piece_begin);
    if (!task.valid) return;
    const int ntiles = nd.len / kTile;
    const int tb = task.split * nd.tiles_per_split;
    const int te = min(tb + nd.tiles_per_split, ntiles);
    mfma32_body<D, NW>(args, task, nd, load_pieces(args, piece_begin, tb, te), tb, te);
}

constexpr bool kPingPongEnabled = true;

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
    bool fits32 = true;  // per-lane DMA offsets within a tile fit in int32
    for (int i = 0; i < a.num_nodes; ++i)
        fits32 = fits32 && (int64_t)kTile * a.nodes[i].stride_tok + d <= (int64_t)INT32_MAX;
    if (kPingPongEnabled && fits32 && nw == 8 && dtype != HP_F32) {
        const dim3 grid(wgs), block(512);
        if (a.stream_kv) {
            if (dtype == HP_BF16) {
                if (d == 128) prefix_mfma16_pp_kernel<true, 128, true><<<grid, block, 0, s>>>(a);
                else prefix_mfma16_pp_kernel<true, 64, true><<<grid, block, 0, s>>>(a);
            } else {
                if (d == 128) prefix_mfma16_pp_kernel<false, 128, true><<<grid, block, 0, s>>>(a);
                else prefix_mfma16_pp_kernel<false, 64, true><<<grid, block, 0, s>>>(a);
            }
        } else {
            if (dtype == HP_BF16) {
                if (d == 128) prefix_mfma16_pp_kernel<true, 128, false><<<grid, block, 0, s>>>(a);
                else prefix_mfma16_pp_kernel<true, 64, false><<<grid, block, 0, s>>>(a);
            } else {
                if (d == 128) prefix_mfma16_pp_kernel<false, 128, false><<<grid, block, 0, s>>>(a);
                else prefix_mfma16_pp_kernel<false, 64, false><<<grid, block, 0, s>>>(a);
            }
        }
        return hipGetLastError();
    }
    switch (nw) {
    case 1: return launch_nw<1>(a, dtype, d, wgs, s);
    case 2: return launch_nw<2>(a, dtype, d, wgs, s);
    case 4: return launch_nw<4>(a, dtype, d, wgs, s);
    default: return launch_nw<8>(a, dtype, d, wgs, s);
    }
}

template <int NW>
static hipError_t launch_tree_nw(const PrefixArgs &a, int dtype, int d, int wgs, hipStream_t s) {
    const dim3 grid(wgs), block(64 * NW);
    if (dtype == HP_BF16) {
        if (d == 128) tree_mfma16_kernel<true, 128, NW><<<grid, block, 0, s>>>(a);
        else tree_mfma16_kernel<true, 64, NW><<<grid, block, 0, s>>>(a);
    } else if (dtype == HP_F16) {
        if (d == 128) tree_mfma16_kernel<false, 128, NW><<<grid, block, 0, s>>>(a);
        else tree_mfma16_kernel<false, 64, NW><<<grid, block, 0, s>>>(a);
    } else {
        if (d == 128) tree_mfma32_kernel<128, NW><<<grid, block, 0, s>>>(a);
        else tree_mfma32_kernel<64, NW><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

// Chunk-tree segments of one row-block width (the caller checks that
// kTile * row_stride + d fits in int32).
hipError_t launch_tree_prefix(const PrefixArgs &a, int dtype, int d, int nw, int wgs,
                              hipStream_t s) {
    if (kPingPongEnabled && nw == 8 && dtype != HP_F32) {
        const dim3 grid(wgs), block(512);
        if (dtype == HP_BF16) {
            if (d == 128) tree_mfma16_pp_kernel<true, 128><<<grid, block, 0, s>>>(a);
            else tree_mfma16_pp_kernel<true, 64><<<grid, block, 0, s>>>(a);
        } else {
            if (d == 128) tree_mfma16_pp_kernel<false, 128><<<grid, block, 0, s>>>(a);
            else tree_mfma16_pp_kernel<false, 64><<<grid, block, 0, s>>>(a);
        }
        return hipGetLastError();
    }
    switch (nw) {
    case 1: return launch_tree_nw<1>(a, dtype, d, wgs, s);
    case 2: return launch_tree_nw<2>(a, dtype, d, wgs, s);
    case 4: return launch_tree_nw<4>(a, dtype, d, wgs, s);
    default: return launch_tree_nw<8>(a, dtype, d, wgs, s);
    }
}

// Both passes of a cascade step in one launch: workgroups [0, prefix_wgs)
// are the ping-pong prefix pass (as prefix_mfma16_pp_kernel), the rest run
// the suffix pass, each of their 8 waves its own list of (sequence, KV head)
// units.  No workgroup waits for another, so the two passes share the chip
// without a second stream; the merge follows on the same stream.  For steps
// whose K/V stay within the last-level cache (plain loads in both passes).
template <bool kBf16, int G>
__global__ __launch_bounds__(512) void step_pp_kernel(PrefixArgs args, FatSuffixArgs fa) {
    constexpr int D = 128;
    // the prefix pass's ring; a suffix workgroup stages its rows there
    __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * 2 * kTile * D];
    static_assert(sizeof(lds) >= 8 * kFatStageBytes, "suffix staging");
    if ((int)blockIdx.x >= fa.prefix_wgs) {
        const int S = ((int)gridDim.x - fa.prefix_wgs) * 8;
        const int wave = (int)threadIdx.x / kWave;
        const int sw = ((int)blockIdx.x - fa.prefix_wgs) * 8 + wave;
        fat_suffix_wave<kBf16, D, G, false>(fa, sw, S, (char *)lds + wave * kFatStageBytes);
        return;
    }
    const WgTask task = decode_wg(args);
    if (!task.valid) return;
    const PrefixNodeArg &nd = args.nodes[task.node];
    const int ntiles = (nd.len + kTile - 1) / kTile;
    const int tb = task.split * nd.tiles_per_split;
    const int te = min(tb + nd.tiles_per_split, ntiles);
    pp_body<kBf16, D, false, ContigTiles, true>(args, task, nd, ContigTiles{nd.len}, tb, te, lds);
}

template <bool kBf16>
static hipError_t launch_step_dt(const PrefixArgs &a, const FatSuffixArgs &f, int G, dim3 grid,
                                 hipStream_t s) {
    switch (G) {
    case 1: step_pp_kernel<kBf16, 1><<<grid, 512, 0, s>>>(a, f); break;
    case 2: step_pp_kernel<kBf16, 2><<<grid, 512, 0, s>>>(a, f); break;
    default: step_pp_kernel<kBf16, 4><<<grid, 512, 0, s>>>(a, f); break;
    }
    return hipGetLastError();
}

bool step_supported(int dtype, int d, int G, int nw) {
    return kPingPongEnabled && nw == 8 && d == 128 && (G == 1 || G == 2 || G == 4) &&
           (dtype == HP_F16 || dtype == HP_BF16);
}

hipError_t launch_step(const PrefixArgs &a, int prefix_wgs, const FatSuffixArgs &f,
                       int suffix_wgs, int dtype, int d, int G, hipStream_t s) {
    bool fits32 = true;
    for (int i = 0; i < a.num_nodes; ++i)
        fits32 = fits32 && (int64_t)kTile * a.nodes[i].stride_tok + d <= (int64_t)INT32_MAX;
    if (!step_supported(dtype, d, G, 8) || !fits32 || a.stream_kv || prefix_wgs < 0 ||
        suffix_wgs < 1 || f.prefix_wgs != prefix_wgs)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(prefix_wgs + suffix_wgs));
    return dtype == HP_BF16 ? launch_step_dt<true>(a, f, G, grid, s)
                            : launch_step_dt<false>(a, f, G, grid, s);
}

}  // namespace hp
