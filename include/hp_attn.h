/*
 * hp_attn.h -- shared-prefix ("cascade") decode attention for AMD Instinct
 * MI355X (gfx950).  C ABI: plain pointers and sizes, no C++ or framework types.
 *
 * One decode step has B sequences, each with one new query token carrying Hq
 * query heads of dimension d.  All sequences (or contiguous ranges of them)
 * share prefix keys/values; each sequence also owns a private suffix held in a
 * paged pool.  The step is computed in passes whose (O, LSE) results merge
 * exactly:
 *
 *   prefix pass   every query row of the sequences under a prefix node attends
 *                 that node's keys in one batched matrix-matrix product, so the
 *                 node's K/V cross HBM once per step ("Hydragen: High-Throughput
 *                 LLM Inference with Shared Prefixes", section "Inter-Sequence
 *                 Batched Prefix Attention"; "ChunkAttention: Efficient
 *                 Self-Attention with Prefix-Aware KV Cache and Two-Phase
 *                 Partition", section "The Chunk-First Phase Kernel in Detail");
 *   suffix pass   ordinary per-sequence decode over each paged suffix (Hydragen
 *                 page, same section, on why suffixes cannot be batched;
 *                 ChunkAttention page, "The Sequence-First Phase Kernel in
 *                 Detail");
 *   merge         O = sum_i e^{LSE_i} O_i / sum_i e^{LSE_i}, LSE = ln sum_i
 *                 e^{LSE_i} (Hydragen page, "Attention Decomposition Across
 *                 Subsequences", Eq. 5, generalised to n parts by applying it
 *                 repeatedly; ChunkAttention page, "The attn_reduce Function",
 *                 Eq. 2 is the same update in (O, m, n) form).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Types.       Q, K and V share one storage type (hp_dtype).  Outputs are
 *              always fp32: O [B][Hq][d] and LSE [B][Hq] (natural log).  Scores
 *              are scale * q.k with no mask, softcap or positional term.
 * GQA.         Query head h reads KV head h / (Hq / Hkv).
 * Memory.      Every tensor pointer is a device pointer the caller owns.  The
 *              library allocates nothing, frees nothing and never synchronises;
 *              scratch space comes from the caller's workspace.  Q, K, V and O
 *              pointers must be 16-byte aligned and every stride a multiple of
 *              16 bytes; d elements of one (token, head) are contiguous.
 * Streams.     `stream` is a hipStream_t (NULL = the null stream).  Work is
 *              enqueued asynchronously; calls are graph-capture safe (no
 *              allocation, host sync, memset or host-to-device copy).
 * Errors.      Every argument is validated on the host before anything is
 *              enqueued; on an error nothing is enqueued and nothing is written.
 *              A failed launch returns HP_ERR_HIP (hp_last_hip_error() has the
 *              hipError_t).  Device-side metadata (block table entries, suffix
 *              lengths) cannot be checked on the host: an entry out of range
 *              makes that row's O and LSE NaN and is never dereferenced.
 * Empty sets.  A row with no keys gets O = 0 and LSE = -inf.  Merging with an
 *              empty part returns the other part.
 * Determinism. No atomics: the same inputs on the same GPU and build give the
 *              same bits.
 * Domain (v1). d in {64, 128}; block_size 16; 1 <= Hq/Hkv <= 8 and a power of
 *              two; at most HP_MAX_LEVELS tree levels and HP_MAX_NODES nodes.
 *              Anything else returns HP_ERR_UNSUPPORTED.
 */
#ifndef HP_ATTN_H
#define HP_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HP_MAX_LEVELS 4   /* prefix tree depth */
#define HP_MAX_NODES 32   /* prefix nodes per call, all levels together */
#define HP_MAX_MERGE 16   /* partials per hp_lse_merge call */
#define HP_BLOCK_SIZE 16  /* tokens per paged KV block */

typedef enum hp_dtype { HP_F32 = 0, HP_F16 = 1, HP_BF16 = 2 } hp_dtype;

typedef enum hp_status {
    HP_OK = 0,
    HP_ERR_NULL = 1,        /* a required pointer is NULL */
    HP_ERR_INVALID_ARG = 2, /* sizes, ranges or alignment are inconsistent */
    HP_ERR_UNSUPPORTED = 3, /* valid, but outside the implemented domain */
    HP_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than the size query's answer */
    HP_ERR_HIP = 5          /* a HIP launch failed; see hp_last_hip_error() */
} hp_status;

/* The query side of one decode step. */
typedef struct hp_query {
    const void *q;      /* device [B][Hq][d] of dtype */
    int32_t B;          /* sequences, >= 0 */
    int32_t Hq, Hkv;    /* query and KV heads; Hq % Hkv == 0 */
    int32_t d;          /* head dimension */
    int32_t dtype;      /* hp_dtype of q, k and v */
    float scale;        /* score = scale * q.k (normally 1/sqrt(d)) */
} hp_query;

/*
 * One shared prefix: `len` tokens attended by sequences [seq_begin, seq_end)
 * (the contiguous descriptor (C, i, j) of the ChunkAttention page, section
 * "Context Generation and GPU-CPU Coordination").  Key of token t, KV head g
 * is at k + t*stride_tok + g*stride_head (elements); same for v.
 */
typedef struct hp_prefix_node {
    const void *k, *v;
    int64_t stride_tok, stride_head;
    int32_t len;        /* >= 0; k and v may be NULL when 0 */
    int32_t seq_begin, seq_end;
} hp_prefix_node;

/*
 * A prefix tree by levels (Hydragen page, section "Hierarchical Sharing"):
 * level 0 is the root (normally one node over all sequences), deeper levels
 * hold narrower shared ranges.  Within a level, nodes are sorted by seq_begin
 * and their ranges are disjoint; a sequence may have no node at a level.
 * `nodes` is a host array, level-major, sum(nodes_per_level) entries.
 */
typedef struct hp_prefix_tree {
    int32_t num_levels;
    int32_t nodes_per_level[HP_MAX_LEVELS];
    const hp_prefix_node *nodes;
} hp_prefix_tree;

/*
 * Paged private suffixes ("Shared Prefix KV Caching, in depth", sections
 * "Storing once is not reading once" and "Splitting attention at the prefix
 * boundary": ordinary paged decode over each sequence's own blocks).  Token t
 * of sequence b is slot t % block_size of block block_table[b*max_blocks +
 * t / block_size]; its key for KV head g is at
 * k_pool + ((blk*block_size + slot)*Hkv + g)*d.  seq_lens may change between
 * graph replays (it is read on the device).
 */
typedef struct hp_paged_kv {
    const void *k_pool, *v_pool;   /* device [num_blocks][block_size][Hkv][d] of dtype */
    const int32_t *block_table;    /* device [B][max_blocks] */
    const int32_t *seq_lens;       /* device [B], each in [0, max_blocks*block_size] */
    int32_t max_blocks;            /* >= 1 */
    int32_t block_size;            /* HP_BLOCK_SIZE */
    int32_t num_blocks;            /* >= 1 */
} hp_paged_kv;

/*
 * Prefix pass over one node: for rows (b, h) with b in [seq_begin, seq_end),
 * O = softmax(scale * q K^T) V over the node's keys and LSE = ln sum exp(scale
 * * q K^T).  The (seq_end - seq_begin) * Hq/Hkv query rows of each KV head are
 * stacked into one matrix and multiplied against the node's keys on the
 * matrix cores (Hydragen page, "Inter-Sequence Batched Prefix Attention";
 * ChunkAttention page, "The partial_attn Function", Eq. 1, evaluated as an
 * online softmax over key tiles).  Rows outside the node are not written.
 * lse may be NULL.  Workspace: hp_prefix_attn_workspace_size().
 */
hp_status hp_prefix_attn_workspace_size(const hp_query *query, const hp_prefix_node *node,
                                        size_t *bytes);
hp_status hp_prefix_attn(const hp_query *query, const hp_prefix_node *node, float *o,
                         float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Suffix pass: for every row (b, h), attention over sequence b's seq_lens[b]
 * paged suffix tokens (Hydragen page, "Inter-Sequence Batched Prefix
 * Attention", on per-sequence suffix attention; ChunkAttention page, "The
 * Sequence-First Phase Kernel in Detail").  lse may be NULL.
 */
hp_status hp_suffix_decode_workspace_size(const hp_query *query, const hp_paged_kv *kv,
                                          size_t *bytes);
hp_status hp_suffix_decode(const hp_query *query, const hp_paged_kv *kv, float *o, float *lse,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * n-way exact merge of n (1..HP_MAX_MERGE) partial results over disjoint key
 * sets (Hydragen page, "Attention Decomposition Across Subsequences", Eq. 5,
 * max-subtracted as its combine_lse description gives).  o_in and lse_in are
 * host arrays of n device pointers: o_in[i] [rows][d] fp32, lse_in[i] [rows]
 * fp32.  Outputs o [rows][d] and lse [rows] (lse may be NULL) must not
 * overlap any input.  d in {64, 128}.
 */
hp_status hp_lse_merge(int32_t n, const float *const *o_in, const float *const *lse_in,
                       float *o, float *lse, int64_t rows, int32_t d, void *stream);

/*
 * One whole decode step: every row (b, h) attends the keys of every tree node
 * covering b (root level first) followed by its paged suffix.  Runs the prefix
 * pass for every node, the suffix pass, and one n-way merge, in that order on
 * `stream` (Hydragen page, "Hierarchical Sharing": decomposition at every
 * tree vertex, recombined with the stored LSE of each level).  tree may be
 * NULL (suffix only); kv may be NULL (prefix only).  lse may be NULL.
 */
hp_status hp_cascade_workspace_size(const hp_query *query, const hp_prefix_tree *tree,
                                    const hp_paged_kv *kv, size_t *bytes);
hp_status hp_cascade_step(const hp_query *query, const hp_prefix_tree *tree,
                          const hp_paged_kv *kv, float *o, float *lse, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * hp_cascade_step plus per-pass timing: records events[0] on `stream` before
 * the first launch, events[1] after the prefix pass (all levels), events[2]
 * after the suffix pass and events[3] after the merge.  events is a host
 * array of n_events (0 or 4) hipEvent_t handles created by the caller; NULL
 * entries are skipped.  Otherwise identical to hp_cascade_step.  For
 * measurement harnesses; the computation is the one described above.
 */
hp_status hp_cascade_step_timed(const hp_query *query, const hp_prefix_tree *tree,
                                const hp_paged_kv *kv, float *o, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream, void *const *events,
                                int32_t n_events);

/* Static description of a status code. */
const char *hp_status_string(hp_status status);
/* hipError_t of the calling thread's last HP_ERR_HIP (0 if none). */
int32_t hp_last_hip_error(void);
/* Library version string. */
const char *hp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HP_ATTN_H */
