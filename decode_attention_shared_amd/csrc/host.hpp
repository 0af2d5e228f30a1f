// Host-side helpers shared by the C-ABI translation units (validation,
// sizes and the split planner).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "common.hpp"
#include "fat_suffix.hpp"
#include "hp_attn.h"

namespace hp {

hipError_t launch_prefix(const PrefixArgs &a, int dtype, int d, int nw, int wgs, hipStream_t s);
hipError_t launch_tree_prefix(const PrefixArgs &a, int dtype, int d, int nw, int wgs,
                              hipStream_t s);
hipError_t launch_suffix(const SuffixArgs &a, int dtype, int d, int G, int nws, hipStream_t s);
hipError_t launch_tree_suffix(const SuffixArgs &a, int dtype, int d, int G, int nws,
                              hipStream_t s);
hipError_t launch_merge(const MergeArgs &a, int d, hipStream_t s);
hipError_t launch_token_suffix(const SuffixArgs &a, int dtype, int d, int G, int nws,
                               hipStream_t s);
hipError_t launch_stream_select(const StreamSelectArgs &a, hipStream_t s);
bool step_supported(int dtype, int d, int G, int nw);
hipError_t launch_step(const PrefixArgs &a, int prefix_wgs, const FatSuffixArgs &f,
                       int suffix_wgs, int dtype, int d, int G, hipStream_t s);
hipError_t launch_read_probe(const void *buf, int64_t bytes, uint32_t *sink, int wgs,
                             hipStream_t s);
hipError_t launch_kv_append(const void *k_new, const void *v_new, const int32_t *rows, int32_t n,
                            int64_t row_bytes, void *k_pool, void *v_pool, int64_t pool_rows,
                            int32_t *seq_lens, const int32_t *seq_idx, int32_t num_seqs,
                            hipStream_t s);

namespace host {

constexpr int kTileKeys = 64;           // keys per prefix tile (matches the kernels)
constexpr int kCUs = 256;               // MI355X compute units
constexpr int kWavesPerCU = 8;          // two waves per SIMD at the prefix kernels' register use
// Cost of one byte of split partials (written once, read once by the merge),
// in units of one 64-key tile of prefix work per resident workgroup (about
// 2.5 us on MI355X; a byte at ~5 TB/s effective is 2e-13 s): used to trade
// scheduling rounds against partial traffic.
constexpr double kPartialByteCost = 8e-8;
constexpr size_t kWsAlign = 256;
// MI355X's last-level (Infinity) cache.  K/V that a prefix launch or a paged
// suffix reads and that are at least this large cannot be found there on the
// next step, so their loads are marked non-temporal; smaller ones are left to
// stay cached.
constexpr int64_t kLlcBytes = int64_t(256) << 20;

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline int esize(int dtype) { return dtype == HP_F32 ? 4 : 2; }

// hipError_t of the calling thread's last failed launch.
hp_status fail_hip(hipError_t e);

// Geometry checks of a query (q may be NULL when need_q is false).
inline hp_status check_geometry(const hp_query *q, bool need_q) {
    if (!q) return HP_ERR_NULL;
    if (q->B < 0 || q->Hq <= 0 || q->Hkv <= 0 || q->Hq % q->Hkv != 0) return HP_ERR_INVALID_ARG;
    if (q->dtype < HP_F32 || q->dtype > HP_BF16) return HP_ERR_INVALID_ARG;
    // scale >= 0: the 16-bit prefix kernels take the row max of the raw dot
    // products and scale it afterwards, which is the max of the scaled scores
    // only when the scale is not negative.
    if (need_q && !(std::isfinite(q->scale) && q->scale >= 0.f)) return HP_ERR_INVALID_ARG;
    if (q->d != 64 && q->d != 128) return HP_ERR_UNSUPPORTED;
    const int G = q->Hq / q->Hkv;
    if (G > 8 || (G & (G - 1)) != 0) return HP_ERR_UNSUPPORTED;
    if (need_q && q->B > 0 && !q->q) return HP_ERR_NULL;
    if (need_q && q->B > 0 && !aligned16(q->q)) return HP_ERR_INVALID_ARG;
    return HP_OK;
}

inline int choose_nw(int64_t M) { return M <= 32 ? 1 : M <= 64 ? 2 : M <= 128 ? 4 : 8; }

// One unit of prefix work for the split planner: M stacked query rows per
// KV head, `rows` output rows ((sequences) * Hq) and `tiles` 64-key tiles.
struct SplitItem {
    int64_t M, rows, tiles;
};
struct SplitPlan {
    int nsplit = 1, tiles_per_split = 0, rowblocks = 1, units_padded = 0, wgs = 0;
};

// Splits of the key range for items launched together (one row-block width
// nw): every item gets splits of (about) the same number of tiles T <= max_T,
// chosen to minimise
//     rounds(T) * T + kPartialByteCost * partial_bytes(T)
// where rounds(T) is how many times the launch fills the GPU's workgroup slots
// (a partly filled last round costs a full round) and partial_bytes(T) the
// split results written and read back by the merge.
// `cus` is the number of compute units the launch may fill.
void plan_splits(const SplitItem *items, int count, int Hkv, int d, int nw, int64_t max_T,
                 SplitPlan *out, int cus = kCUs);

// Running the suffix pass beside the prefix pass (see the cascade step): the
// prefix is then planned for kConcCUs compute units, where alone it takes
// 1.15-1.28x the time of its all-CU plan (less than the CU ratio), leaving
// the rest to the memory-bound suffix.
// Used when every prefix split keeps at least kConcMinTiles tiles under that
// plan and the suffix has at least kConcMinUnits (sequence, KV head) units.
// Measured on MI355X with the caches flushed before every step (as a layer's
// attention finds them in a model): MHA steps with 10 240 units and 1K-16K
// prefixes (4-64 tiles per split) gain 3-8 %, a two-level GQA step with 2 048
// units gains 5 %; with 512 (Llama-3-8B shape) or 1 280 units (one 8-way head
// share of the 16K MHA shape) the side-by-side step loses 13-16 %.
constexpr int kConcCUs = 160;
// Both passes in one launch: the prefix plan's compute units (the rest host
// one suffix workgroup each).  Measured on the one-GPU head share of the 16K
// MHA shape: 160 units 52.5 us per step, 192 or 208 units 56.8.
constexpr int kOneLaunchCUs = 160;
// Suffix-heavy steps (a bound on the suffix pass's K/V bytes, B * max_blocks
// blocks, at least kConcHeavyRatio times the batched prefix's K/V bytes) plan
// the prefix for kConcCUsHeavy units instead, leaving more to the suffix pass.
constexpr int kConcCUsHeavy = 96;
constexpr int64_t kConcHeavyRatio = 6;
constexpr int kConcMinTiles = 4;
constexpr int64_t kConcMinUnits = 2048;

// Batching policy (hp_share_decision): whether `tokens` keys shared by `nseq`
// sequences are better read once for all of them than by each sequence.
bool share_decision(int dtype, int d, int G, int64_t tokens, int64_t nseq);

// The cascade step on one stream (hp_cascade_step), for entry points that
// supply the workspace themselves: cascade_serial_plan validates every
// argument of the step (outputs included) and gives the workspace bytes.
hp_status cascade_serial_plan(const hp_query *q, const hp_prefix_tree *tree,
                              const hp_paged_kv *kv, const float *o, const float *lse,
                              size_t *bytes);
hp_status cascade_serial(const hp_query *q, const hp_prefix_tree *tree, const hp_paged_kv *kv,
                         float *o, float *lse, void *ws, size_t ws_bytes, void *stream);

}  // namespace host
}  // namespace hp
