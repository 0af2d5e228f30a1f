// Device helpers and launch-argument structs shared by the gfx950 kernels and
// the host entry points.  Internal to the library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hp_attn.h"

namespace hp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;
constexpr int kBlock = HP_BLOCK_SIZE;

// ---------------------------------------------------------------------------
// Launch arguments.  Everything a kernel needs travels by value, so a launch
// reads no host memory and needs no host-to-device copy (graph-capture safe).
// ---------------------------------------------------------------------------

// Destination of a pass's per-row results: normalised O and natural-log LSE.
// Row (b, h) of split s lands at o + s*o_split + ((b - row_base)*Hq + h)*d.
struct RowDest {
    float *o;
    float *lse;          // may be null only for direct writes with lse == NULL
    int64_t o_split;     // elements between splits
    int64_t lse_split;
    int32_t row_base;
};

constexpr int kMaxLaunchNodes = 16;

struct PrefixNodeArg {
    const void *k;
    const void *v;
    int64_t stride_tok;
    int64_t stride_head;
    int32_t len;
    int32_t seq_begin;
    int32_t seq_end;
    int32_t nsplit;           // key-range splits
    int32_t tiles_per_split;  // 64-key tiles per split
    int32_t rowblocks;        // row blocks per (KV head, split)
    int32_t units_padded;     // (KV head, split) units, rounded up to a multiple of 8 when rowblocks > 1
    int32_t wg_begin;         // first workgroup of this node in the launch
    RowDest dest;
};

// ---------------------------------------------------------------------------
// Chunked-tree plan image: int32 arrays built on the host, copied to device
// memory once per tree shape.  Word offsets of each array come from
// tree_layout() (same on both sides).
// ---------------------------------------------------------------------------
struct TreeSeg {               // a run of batched descriptors sharing one range
    int32_t piece_begin;       // first key tile in the piece table
    int32_t ntiles;
    int32_t seq_begin, seq_end;
    int32_t nsplit, tiles_per_split, rowblocks, units_padded;
    int32_t wg_begin;          // first workgroup of the segment in its launch
    int32_t part_row0;         // first (sequence, split) partial row of the segment
    int32_t pad0, pad1;
};
struct TreePiece {             // one key tile: `count` pool rows from `row`
    int32_t row, count;
};
struct TreeSrc {               // one segment a sequence reads the partials of
    int32_t part_row;          // partial row of (this sequence, split 0)
    int32_t nsplit;
    int32_t split_rows;        // partial rows between splits (= the segment's sequences)
    int32_t pad;
};
constexpr int kTreeMaxTilesPerSplit = 64;  // one piece per lane of a wave

struct TreeLayout {            // word offsets into the image
    int64_t segs, pieces, wgseg, seq_tok, tok_rows, seq_src, srcs, shared, words;
};

__host__ __device__ inline int64_t tree_align4(int64_t w) { return (w + 3) & ~(int64_t)3; }

__host__ __device__ inline TreeLayout tree_layout(int64_t num_segs, int64_t num_pieces,
                                                  int64_t num_wgs, int64_t B,
                                                  int64_t num_tok_rows, int64_t num_srcs) {
    TreeLayout L;
    int64_t w = 0;
    L.segs = w;     w = tree_align4(w + num_segs * (int64_t)(sizeof(TreeSeg) / 4));
    L.pieces = w;   w = tree_align4(w + num_pieces * 2);
    L.wgseg = w;    w = tree_align4(w + num_wgs);
    L.seq_tok = w;  w = tree_align4(w + B + 1);
    L.tok_rows = w; w = tree_align4(w + num_tok_rows);
    L.seq_src = w;  w = tree_align4(w + B + 1);
    L.srcs = w;     w = tree_align4(w + num_srcs * 4);
    L.shared = w;   w = tree_align4(w + B);
    L.words = w;
    return L;
}

struct PrefixArgs {
    const void *q;
    int32_t B, Hq, Hkv, G;
    float scale_log2;         // scale * log2(e): scores go straight to the exp2 domain
    int32_t num_nodes;
    PrefixNodeArg nodes[kMaxLaunchNodes];
    // Chunk-tree launches only: segments come from the plan image.
    const int32_t *tree;      // plan image (device)
    int64_t seg_off, piece_off, wgseg_off;  // word offsets of its arrays
    int32_t wg0;              // this launch's first entry of the workgroup table
    const void *k_pool, *v_pool;
    int64_t row_stride;       // elements between pool rows (Hkv * d)
    int32_t d;
    float *part_o, *part_lse; // partial results, [part_rows][Hq][d] and [part_rows][Hq]
    int32_t stream_kv;        // node launches: K/V transfers marked non-temporal (the launch's
                              // K/V exceed the last-level cache)
};

constexpr int kMaxMergeSrc = HP_MAX_NODES + 1;

// One source of partials for the merge.  Row (b, h) reads split s at
// o + s*o_split + ((b - b0)*Hq + h)*d when b in [b0, b1).  When
// split_blocks > 0 the source is a suffix pass: only the first
// ceil(ceil(len_b / 16) / split_blocks) splits hold keys.
struct MergeSrc {
    const float *o;
    const float *lse;
    int64_t o_split;
    int64_t lse_split;
    int32_t nsplit;
    int32_t split_blocks;
    int64_t b0, b1;
};

// A prefix node that each of its sequences reads in its own suffix pass (the
// batching policy found the node too short, or shared by too few sequences,
// for the batched pass to pay).  Key of token t, KV head g at
// k + t*stride_tok + g*stride_head (elements); sequences [b0, b1).
struct PrivSeg {
    const void *k, *v;
    int64_t stride_tok, stride_head;
    int32_t len, b0, b1, pad;
};

// Suffix pass with the final merge fused in: every row (b, h) merges its
// suffix attention with the partials of the sources covering sequence b.
struct SuffixArgs {
    const void *q;
    const void *k_pool;
    const void *v_pool;
    const int32_t *table;     // block table; chunk-tree mode: unused
    const int32_t *lens;      // chunk-tree mode: total tokens of each sequence, may be null
    int32_t B, Hq, Hkv;
    int32_t max_blocks, num_blocks;
    int32_t kv_hnd;           // paged mode: blocks are [Hkv][16][d] (else [16][Hkv][d])
    int32_t has_suffix;       // 0: no paged suffix (only the sources are merged)
    float scale_log2;
    RowDest dest;             // final O and LSE (o_split, lse_split unused)
    int32_t nsrc;
    MergeSrc src[kMaxMergeSrc];
    // Chunk-tree mode: private rows and segment partials from the plan image.
    const int32_t *tree;
    int64_t seq_tok_off, tok_rows_off, seq_src_off, srcs_off, shared_off;
    int64_t pool_rows;
    const float *part_o, *part_lse;
    int32_t stage_floats;     // dynamic LDS for staged partials (0: read them from memory)
    int32_t stream_kv;        // paged and token-table modes: K/V loads marked non-temporal
                              // (footprint beyond the last-level cache, so nothing of it would be
                              // found there next step)
    // Paged mode: prefix nodes read privately, before the paged suffix.  At
    // most one per tree level covers a sequence (a level's ranges are disjoint).
    int32_t nseg;
    PrivSeg seg[HP_MAX_NODES];
};

// Stream selection of a shared-context step: query b (request q_req[b],
// stream q_sid[b]) gets the pool rows of the visible positions of its
// request's KV row, in row order.
struct StreamSelectArgs {
    const int32_t *row_slots;  // [R][row_cap] pool row of each position
    const int32_t *slot_sid;   // [R][row_cap] stream id of each position (-1: every stream)
    const int32_t *row_len;    // [R]
    const int32_t *q_req;      // [B]
    const int32_t *q_sid;      // [B]
    int32_t B, R, row_cap;
    int32_t *tok_table;        // [B][row_cap] out: visible pool rows
    int32_t *tok_len;          // [B] out: their count, -1 when the metadata is out of range
};

struct MergeArgs {
    MergeSrc src[kMaxMergeSrc];
    int32_t nsrc;
    const int32_t *lens;      // suffix lengths (for suffix sources), may be null otherwise
    int32_t max_len;          // capacity check for lens
    int32_t Hq;
    int64_t row_b0, row_b1;   // sequences whose rows are written
    float *o;                 // [B][Hq][d], indexed by absolute b
    float *lse;               // may be null
};

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t bits16) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
    return (float)h;
}

template <bool kBf16>
__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    if constexpr (kBf16) return bf16_bits_to_float(bits16);
    else return f16_bits_to_float(bits16);
}

// Round fp32 to the 16-bit type (nearest even), returned as raw bits.
template <bool kBf16>
__device__ __forceinline__ uint32_t float_to_half_bits(float x) {
    if constexpr (kBf16) {
        __bf16 b = (__bf16)x;
        return __builtin_bit_cast(uint16_t, b);
    } else {
        _Float16 h = (_Float16)x;
        return __builtin_bit_cast(uint16_t, h);
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

template <int kWidth>
__device__ __forceinline__ float xor_sum(float x) {
#pragma unroll
    for (int off = 1; off < kWidth; off <<= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Max over lanes that differ only in the bits [from, 64): lanes l, l^from, l^2from, ...
template <int kFrom>
__device__ __forceinline__ float xor_max_from(float x) {
#pragma unroll
    for (int off = kFrom; off < kWave; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
    return x;
}

template <int kFrom>
__device__ __forceinline__ float xor_sum_from(float x) {
#pragma unroll
    for (int off = kFrom; off < kWave; off <<= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Global memory straight into LDS (gfx950 global_load_lds_dword{,x4}): lane i
// writes lds_base + 16*i (dma16) or lds_base + 4*i (dma4); lds_base is
// wave-uniform (M0).  Issued as inline assembly so that the compiler does not
// track it: it cannot prove that later LDS reads do not alias a transfer in
// flight, and would otherwise wait for every transfer before each of them.
// Completion is the caller's business: a vmcnt wait, then a barrier.
template <int kBytes>
__device__ __forceinline__ void lds_dma(const void *g, void *lds_base) {
    static_assert(kBytes == 4 || kBytes == 16, "dword or dwordx4");
    const uint32_t l = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds_base);
    uint32_t saved;  // M0 is reserved by the compiler: restore it
    if constexpr (kBytes == 16)
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"(g), "s"(l)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"(g), "s"(l)
            : "memory");
}
__device__ __forceinline__ void dma16(const void *g, void *lds_base) { lds_dma<16>(g, lds_base); }

// The same 16-byte transfer with every wave-uniform part in scalar
// registers: the global base, and the LDS destination as an LDS byte address
// (M0); only the per-lane unsigned 32-bit byte offset is a vector register.
// No vector instruction is needed to issue it.
// kNT marks the load non-temporal (data read once per step that would not
// survive in the last-level cache until the next).
template <bool kNT = false>
__device__ __forceinline__ void dma16_s(const void *base, uint32_t byte_off, uint32_t lds_addr) {
    uint32_t saved;
    if constexpr (kNT) {
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"(byte_off), "s"(base), "s"(lds_addr)
            : "memory");
    } else {
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"(byte_off), "s"(base), "s"(lds_addr)
            : "memory");
    }
}

// s_waitcnt with only vmcnt = n (expcnt and lgkmcnt left unconstrained).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

}  // namespace hp
