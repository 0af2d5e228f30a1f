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
 *              scratch space comes from the caller's workspace (for
 *              hp_cascade_step_noalloc, from a fixed array in the library's
 *              device image).  Q, K, V and O
 *              pointers must be 16-byte aligned and every stride a multiple of
 *              16 bytes; d elements of one (token, head) are contiguous.
 *              K/V that a prefix launch, a paged suffix or a token-table pass
 *              reads and that reach 256 MiB (MI355X's last-level cache) are
 *              loaded non-temporal; results do not depend on it.
 * Streams.     `stream` is a hipStream_t (NULL = the null stream).  Work is
 *              enqueued asynchronously; calls are graph-capture safe (no
 *              allocation, host sync, memset or host-to-device copy).  The
 *              library holds no state of its own: no streams, events, buffers
 *              or settings; a second stream, when a step uses one, is the
 *              caller's (hp_cascade_step_overlap).  The one exception is the
 *              per-GPU scratch array of hp_cascade_step_noalloc.
 * Errors.      Every argument is validated on the host before anything is
 *              enqueued; on an error nothing is enqueued and nothing is written.
 *              A failed launch returns HP_ERR_HIP (hp_last_hip_error() has the
 *              hipError_t).  Device-side metadata (block table entries, suffix
 *              lengths) cannot be checked on the host: an entry out of range
 *              makes that row's O and LSE NaN and is never dereferenced.
 * Empty sets.  A row with no keys gets O = 0 and LSE = -inf.  Merging with an
 *              empty part returns the other part.
 * Determinism. The attention kernels use no atomics and no order-dependent
 *              reduction: the same inputs on the same GPU and build give the same
 *              bits.  (hp_kv_append's optional length advance uses integer atomic
 *              adds, whose result does not depend on their order.)
 * Exceptions.  None crosses the boundary: a host-side failure inside an entry
 *              point (out of host memory) returns HP_ERR_HOST.
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
#define HP_CHUNK 64       /* tokens per chunk of the prefix-tree KV pool */

typedef enum hp_dtype { HP_F32 = 0, HP_F16 = 1, HP_BF16 = 2 } hp_dtype;

typedef enum hp_status {
    HP_OK = 0,
    HP_ERR_NULL = 1,        /* a required pointer is NULL */
    HP_ERR_INVALID_ARG = 2, /* sizes, ranges or alignment are inconsistent */
    HP_ERR_UNSUPPORTED = 3, /* valid, but outside the implemented domain */
    HP_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than the size query's answer */
    HP_ERR_HIP = 5,         /* a HIP launch failed; see hp_last_hip_error() */
    HP_ERR_CAPACITY = 6,    /* a pool, plan buffer, output array or fixed scratch array
                               is too small */
    HP_ERR_HOST = 7         /* host-side failure (out of host memory); nothing was enqueued */
} hp_status;

/* The query side of one decode step. */
typedef struct hp_query {
    const void *q;      /* device [B][Hq][d] of dtype */
    int32_t B;          /* sequences, >= 0 */
    int32_t Hq, Hkv;    /* query and KV heads; Hq % Hkv == 0 */
    int32_t d;          /* head dimension */
    int32_t dtype;      /* hp_dtype of q, k and v */
    float scale;        /* score = scale * q.k (normally 1/sqrt(d)); finite and >= 0,
                           else HP_ERR_INVALID_ARG */
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
 *
 * share_min chooses which nodes a cascade step reads once for all their
 * sequences (the batched prefix pass) and which each of their sequences reads
 * in its own suffix pass, as keys before its paged suffix.  Under a few
 * hundred shared tokens, or with few sharing sequences, the batched pass and
 * its merge cost more than they save ("Shared Prefix KV Caching, in depth",
 * section "Trade-offs"):
 *   0      per node, by hp_share_decision() on its length and number of
 *          sequences (the automatic policy);
 *   k >= 1 batch the nodes over at least k sequences (1: every node).
 * Negative values are HP_ERR_INVALID_ARG.  The result is the same attention
 * either way (up to rounding); hp_stream_decode batches every node of its
 * documents whatever the value.
 */
typedef struct hp_prefix_tree {
    int32_t num_levels;
    int32_t nodes_per_level[HP_MAX_LEVELS];
    const hp_prefix_node *nodes;
    int32_t share_min;
} hp_prefix_tree;

/*
 * Paged private suffixes ("Shared Prefix KV Caching, in depth", sections
 * "Storing once is not reading once" and "Splitting attention at the prefix
 * boundary": ordinary paged decode over each sequence's own blocks).  Token t
 * of sequence b is slot t % block_size of block block_table[b*max_blocks +
 * t / block_size]; its key for KV head g is at
 *   HP_KV_NHD  k_pool + ((blk*block_size + slot)*Hkv + g)*d   (token-major)
 *   HP_KV_HND  k_pool + ((blk*Hkv + g)*block_size + slot)*d   (head-major)
 * and likewise in v_pool.  Head-major blocks keep the block_size rows one
 * (sequence, KV head) reads contiguous: the suffix pass reads them measurably
 * faster (3-9 % on the 16K-prefix shapes).  seq_lens may change between graph
 * replays (it is read on the device).
 */
#define HP_KV_NHD 0
#define HP_KV_HND 1

typedef struct hp_paged_kv {
    const void *k_pool, *v_pool;   /* device, num_blocks blocks of block_size*Hkv*d of dtype */
    const int32_t *block_table;    /* device [B][max_blocks] */
    const int32_t *seq_lens;       /* device [B], each in [0, max_blocks*block_size] */
    int32_t max_blocks;            /* >= 1 */
    int32_t block_size;            /* HP_BLOCK_SIZE */
    int32_t num_blocks;            /* >= 1 */
    int32_t layout;                /* HP_KV_NHD or HP_KV_HND, else HP_ERR_INVALID_ARG */
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
 * pass for every batched node (tree->share_min), then the suffix pass --
 * each sequence's private nodes and paged suffix -- with one n-way merge
 * fused into its epilogue (Hydragen page, "Hierarchical Sharing":
 * decomposition at every tree vertex, recombined with the stored LSE of each
 * level), all on `stream`.  tree may be NULL (suffix only); kv may be NULL
 * (prefix only).  lse may be NULL.  Workspace: hp_cascade_workspace_size()
 * for the same tree (its share_min included), which covers
 * hp_cascade_step_overlap() too.
 */
hp_status hp_cascade_workspace_size(const hp_query *query, const hp_prefix_tree *tree,
                                    const hp_paged_kv *kv, size_t *bytes);
hp_status hp_cascade_step(const hp_query *query, const hp_prefix_tree *tree,
                          const hp_paged_kv *kv, float *o, float *lse, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Running the prefix and suffix passes side by side.  They depend on nothing
 * but the inputs (only the merge needs both; Hydragen page, "Attention
 * Decomposition Across Subsequences", Eq. 5), so a step may launch the
 * suffix pass on a second stream while the prefix pass, planned for fewer
 * compute units, runs on `stream`; one merge on `stream` then combines every
 * partial.  The caller owns the second stream and both events (the library
 * creates, keeps and synchronises nothing):
 *   side_stream  a hipStream_t of the same device as `stream`, not `stream`
 *                itself (a stream that does not synchronise with the null
 *                stream, at default priority, is what this path is made for);
 *   fork_event, join_event  hipEvent_t handles created by the caller
 *                (hipEventDisableTiming suffices), recorded and waited on by
 *                the step: fork on `stream` before any launch and waited on by
 *                side_stream, join on side_stream after the suffix pass and
 *                waited on by `stream` before the merge.  They only order
 *                two streams of one device, so events created with
 *                hipEventDisableSystemFence as well serve (the kernels' own
 *                device-scope release and acquire carry the data); under
 *                graph capture the events become graph edges either way;
 *   mode         0: never (exactly hp_cascade_step); 1: when the plan expects
 *                a gain, that is when, with the prefix pass planned for 160 of
 *                the 256 compute units, every prefix split still covers at
 *                least 4 tiles of 64 keys and the suffix has at least 2048
 *                (sequence, KV head) units (second stream), or, for a step
 *                with one query head per KV head that qualifies for one
 *                launch (below) and has fewer units, in one launch; 2: on the
 *                second stream whenever the step has both a prefix and a
 *                suffix; 3: in one launch whenever the step qualifies, else
 *                as mode 0.
 * One launch: the prefix pass's workgroups and suffix workgroups of the same
 * shape (one per compute unit the prefix plan leaves free) share a kernel,
 * so no second stream or event is used (side_stream and the events may then
 * be NULL), then one merge on `stream`.  A step qualifies when its batched
 * nodes form one prefix launch of the 256-row kernel (at least 129 stacked
 * query rows per KV head), the dtype is 16-bit, d = 128, Hq/Hkv is 1, 2 or 4,
 * no node is read privately, the K/V of both passes stay under 256 MiB, and
 * each suffix wave's share fits its tables (at most 31 query rows and 500
 * blocks; the suffix work goes to the waves in items of 4 blocks).
 * Side by side, the prefix pass is planned for 160 compute units, or for 96
 * when B * max_blocks suffix blocks hold at least 6 times the K/V bytes of
 * the batched nodes (the test of mode 1 is made on the 160-unit plan).  The
 * host cannot read the lengths, so max_blocks stands for the suffix size: a
 * table cut to the batch's longest suffix (as the workloads here use) keeps
 * the estimate within about twice the mean; a table far wider than any
 * suffix can make a prefix-bound step take the 96-unit plan, which is slower
 * for it (an 8K-token prefix over 256 MHA sequences: 170 against 123 us).
 * Everything enqueued on `stream` before the call is ordered before both
 * passes and everything after it after the merge, eagerly and under graph
 * capture alike (the events become the graph's fork and join).  Calls that
 * share the same events or side stream must not run concurrently from
 * several host threads.  HP_ERR_NULL when the plan uses the second stream
 * and a handle is NULL; HP_ERR_INVALID_ARG for side_stream == stream (the
 * second stream used) or another mode.
 */
typedef struct hp_overlap {
    void *side_stream;
    void *fork_event;
    void *join_event;
    int32_t mode;
} hp_overlap;

hp_status hp_cascade_step_overlap(const hp_query *query, const hp_prefix_tree *tree,
                                  const hp_paged_kv *kv, float *o, float *lse, void *workspace,
                                  size_t workspace_bytes, void *stream, const hp_overlap *overlap);

/*
 * *overlapped = 1 when hp_cascade_step_overlap with these arguments and this
 * mode would run the passes side by side on the second stream, 2 when in one
 * launch, else 0.  Validates the arguments like hp_cascade_workspace_size.
 */
hp_status hp_cascade_overlap_plan(const hp_query *query, const hp_prefix_tree *tree,
                                  const hp_paged_kv *kv, int32_t mode, int32_t *overlapped);

/*
 * hp_cascade_step (overlap NULL) or hp_cascade_step_overlap plus per-pass
 * timing: records events[0] on `stream` right before the first prefix launch
 * (after the fork when the passes run side by side), events[1] after the
 * prefix pass (all levels), events[2] after the suffix pass (on the side
 * stream when the passes run side by side) and events[3] after the merge;
 * with n_events = 5, events[4] on the suffix pass's stream right before its
 * launch (so that the suffix pass can be timed from its own start when it
 * does not follow the prefix pass).  events is a host array of n_events (0, 4
 * or 5) hipEvent_t handles created by the caller; NULL entries are skipped; a
 * NULL array with n_events > 0 is HP_ERR_NULL.  For measurement harnesses;
 * the computation is the one described above.
 */
hp_status hp_cascade_step_timed(const hp_query *query, const hp_prefix_tree *tree,
                                const hp_paged_kv *kv, float *o, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream, const hp_overlap *overlap,
                                void *const *events, int32_t n_events);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid
 * it): hp_cascade_step with its workspace taken from a fixed array of
 * HP_NOALLOC_SCRATCH_BYTES in the library's device image instead of a
 * caller-allocated one.  The caller still passes every input and the outputs;
 * the step allocates and frees nothing (host or device) and computes exactly
 * what hp_cascade_step computes, on `stream` alone.
 *   The array exists once per GPU, from when the library's code object is
 * loaded on that GPU until the process ends.  Its device address is looked up
 * on the first call for a GPU (the GPU `stream` belongs to; the current device
 * for the null stream), with that device made current for the lookup and the
 * caller's current device restored.  Every call on a GPU uses that GPU's one
 * array: calls that may overlap on one GPU (several streams, several host
 * threads, a graph replayed beside an eager call) race on it and must be
 * ordered by the caller.  The array keeps what the last call left in it;
 * no call depends on those contents.
 *   Returns HP_ERR_CAPACITY, enqueuing nothing, when the step's workspace
 * (hp_cascade_workspace_size reports at least that much) exceeds
 * HP_NOALLOC_SCRATCH_BYTES; HP_ERR_UNSUPPORTED for a device ordinal of 64 or
 * more; otherwise the errors of hp_cascade_step.
 */
#define HP_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

hp_status hp_cascade_step_noalloc(const hp_query *query, const hp_prefix_tree *tree,
                                  const hp_paged_kv *kv, float *o, float *lse, void *stream);

/* ------------------------------------------------------------------------
 * Shared-context requests: stream-id masked decode
 * ------------------------------------------------------------------------
 * A request decodes P independent questions about one document as P streams
 * of one KV row ("Read Once, Answer Many: Parallel Prompting for
 * Shared-Context LLM Inference", section "Parallel Prompting").  The document
 * is a prefix node (read once for every stream of every request that shares
 * it, by the prefix pass).  The rest of a request's row -- its questions and
 * the streams' answer tokens, in whatever order the engine appends them --
 * lives in a pool with one token per row, each position tagged with a stream
 * id; -1 marks a position every stream of the request sees.  Query b, of
 * stream q_sid[b] in request q_req[b], attends the document and exactly the
 * positions of its request's row whose id is -1 or q_sid[b] (the page's
 * Eq. 2 and Figure 2: the answer of a stream depends only on the document and
 * its own question), in row order.
 *
 * Key of pool row p, KV head g at k_pool + (p*Hkv + g)*d (elements).
 * row_slots / slot_sid: device [num_requests][row_cap]; row_len: device
 * [num_requests]; q_req / q_sid: device [B].  All are read on the device, so
 * they may change between graph replays.  A request index or row length out
 * of range, or a visible position whose pool row is outside [0, pool_rows),
 * makes that query's O and LSE NaN (nothing out of range is dereferenced).
 */
typedef struct hp_stream_rows {
    const void *k_pool, *v_pool;   /* device [pool_rows][Hkv][d] of dtype */
    const int32_t *row_slots;      /* device [num_requests][row_cap] */
    const int32_t *slot_sid;       /* device [num_requests][row_cap] */
    const int32_t *row_len;        /* device [num_requests], each in [0, row_cap] */
    const int32_t *q_req;          /* device [B] */
    const int32_t *q_sid;          /* device [B] */
    int32_t num_requests;          /* >= 1 */
    int32_t row_cap;               /* >= 1 */
    int64_t pool_rows;             /* >= 1 */
} hp_stream_rows;

/*
 * One decode step of shared-context requests: the prefix pass over every node
 * of `doc` (a prefix tree as in hp_cascade_step; NULL for none), the stream
 * selection (the mask of Eq. 2 evaluated on the stream ids, writing each
 * query's visible pool rows into the workspace), and the sequence-first pass
 * over those rows with the merge of the document partials fused in.  lse may
 * be NULL.  Workspace: hp_stream_decode_workspace_size().
 */
hp_status hp_stream_decode_workspace_size(const hp_query *query, const hp_prefix_tree *doc,
                                          const hp_stream_rows *rows, size_t *bytes);
hp_status hp_stream_decode(const hp_query *query, const hp_prefix_tree *doc,
                           const hp_stream_rows *rows, float *o, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * hp_stream_decode with the stream selection and the stream pass on a second
 * stream beside the document's prefix pass, as hp_cascade_step_overlap does
 * for the suffix pass: the stream pass then writes its own (O, LSE) rows to
 * the workspace and one merge on `stream` combines them with the document
 * partials.  overlap->mode: 0 serial (hp_stream_decode); 1 side by side by
 * the cascade step's rule (the prefix pass planned for 160 compute units,
 * every prefix split at least 4 tiles of 64 keys, at least 2048 (query, KV
 * head) units), else serial; 2 side by side whenever the document has a node.
 * The prefix pass then runs on 96 compute units when B * row_cap row
 * positions hold at least 6 times the document's K/V bytes, else on 160.  One launch (mode 3) is
 * not offered here.  Ordering, event and stream rules, and errors as for
 * hp_cascade_step_overlap (HP_ERR_INVALID_ARG for mode 3).  The workspace
 * size from hp_stream_decode_workspace_size serves every mode.
 */
hp_status hp_stream_decode_overlap(const hp_query *query, const hp_prefix_tree *doc,
                                   const hp_stream_rows *rows, float *o, float *lse,
                                   void *workspace, size_t workspace_bytes, void *stream,
                                   const hp_overlap *overlap);

/* *overlapped = 1 when hp_stream_decode_overlap with these arguments and this
 * mode would run the stream pass on the second stream, else 0.  Validates the
 * arguments like hp_stream_decode_workspace_size. */
hp_status hp_stream_overlap_plan(const hp_query *query, const hp_prefix_tree *doc,
                                 const hp_stream_rows *rows, int32_t mode, int32_t *overlapped);

/* ------------------------------------------------------------------------
 * Chunked prefix tree: device-resident (C, i, j) plans
 * ------------------------------------------------------------------------
 * Keys and values live in a pool of rows: row r holds one token, its key for
 * KV head g at k_pool + (r*Hkv + g)*d (elements); same for v_pool.  A chunk
 * is HP_CHUNK consecutive rows.  A descriptor names `count` consecutive rows
 * and the sequences [seq_begin, seq_end) that attend them: the chunk
 * descriptor (C, i, j) of the ChunkAttention page, section "Context
 * Generation and GPU-CPU Coordination".  Any set of descriptors is a valid
 * step (a tree of any depth, a forest, or ranges that cover only some
 * sequences); sequence b attends the union of the rows of every descriptor
 * whose range holds b.
 */
typedef struct hp_chunk_desc {
    int32_t row;        /* first pool row */
    int32_t count;      /* rows, 1..HP_CHUNK */
    int32_t seq_begin, seq_end;
} hp_chunk_desc;

/*
 * Host summary of a plan built by hp_tree_plan_build().  The plan itself is a
 * byte image ("blob") that the caller copies to device memory and passes to
 * hp_tree_step(); it only changes when the descriptors change, so a caller
 * copies it again only then (the page's lazy context copy, same section).
 * Every field is written by hp_tree_plan_build(); pass the struct unchanged.
 */
#define HP_TREE_MAX_LAUNCHES 4
typedef struct hp_tree_plan {
    int32_t B, Hq, Hkv, d, dtype;
    int32_t share_min;          /* descriptors with seq_end - seq_begin >= share_min are batched */
    int32_t num_descs;
    int32_t num_segs;           /* batched segments (runs of descriptors with one range) */
    int32_t num_pieces;         /* key tiles of the segments */
    int32_t num_srcs;           /* (sequence, segment) pairs */
    int32_t num_tok_rows;       /* private rows over all sequences */
    int32_t max_private;        /* longest private row list of one sequence */
    int32_t num_launches;       /* chunk-first launches (one per row-block width) */
    int32_t launch_nw[HP_TREE_MAX_LAUNCHES];   /* waves per workgroup */
    int32_t launch_wgs[HP_TREE_MAX_LAUNCHES];  /* workgroups */
    int32_t launch_wg0[HP_TREE_MAX_LAUNCHES];  /* first entry of the launch in the blob's workgroup table */
    int64_t part_rows;          /* (sequence, split) partial rows of all segments */
    int64_t pool_rows;          /* rows the descriptors were checked against */
    size_t blob_bytes;          /* size of the device image */
    size_t workspace_bytes;     /* workspace hp_tree_step needs */
} hp_tree_plan;

/*
 * Plan one decode step over chunk descriptors (ChunkAttention page, sections
 * "Two-Phase Partition (TPP): Algorithm Overview" and "The Chunk-First Phase
 * Kernel in Detail").  Descriptors with seq_end - seq_begin >= share_min
 * (>= 2) are batched: consecutive ones with the same range form a segment
 * whose keys stream once through the matrix cores for all the range's query
 * rows (chunk-first phase).  The others are private: each sequence they cover
 * reads them in the per-sequence pass (sequence-first phase).  share_min = 0
 * decides run by run (consecutive descriptors with one range) with
 * hp_share_decision() on the run's total rows and range size.  Descriptors are
 * given in tree pre-order, as hp_pakv_context() emits them, so that a path of
 * chunks shared by one range is one segment; any order is still correct.
 *
 * geom: B, Hq, Hkv, d, dtype (geom->q and geom->scale are not used).  descs:
 * host array of n descriptors.  pool_rows: rows of the pool the step will
 * read (every descriptor must lie inside it).  blob: host buffer of
 * blob_capacity bytes that receives the device image, or NULL to only fill
 * `plan` (the size query).  Returns HP_ERR_CAPACITY when blob is too small.
 */
hp_status hp_tree_plan_build(const hp_query *geom, const hp_chunk_desc *descs, int32_t n,
                             int32_t share_min, int64_t pool_rows, void *blob,
                             size_t blob_capacity, hp_tree_plan *plan);

/*
 * Batching policy: *batch = 1 when `tokens` keys shared by `nseq` sequences
 * are better read once for all of them (prefix pass plus merge) than by each
 * sequence in its own pass, else 0 ("Shared Prefix KV Caching, in depth",
 * section "Trade-offs": under a few hundred shared tokens or with few
 * sequences the extra launch and merge cost more than they save; Hydragen
 * page, section "How Hydragen Positions Itself", on its boundary conditions).  The rule is
 * a threshold on `tokens` that falls as `nseq` grows, fitted to timings of
 * both passes on MI355X; it depends on geom's dtype, d and Hq / Hkv (geom->q
 * and geom->scale are not used).  nseq in [0, geom->B], tokens >= 0.
 */
hp_status hp_share_decision(const hp_query *geom, int64_t tokens, int32_t nseq, int32_t *batch);

/*
 * One decode step over a plan: every row (b, h) attends the rows of every
 * descriptor covering b.  Runs the chunk-first launches (MFMA, one per
 * row-block width), then the sequence-first pass, which walks each sequence's
 * private rows and merges them with the partials of its segments in one
 * epilogue (ChunkAttention page, "The Sequence-First Phase Kernel in
 * Detail" and "The attn_reduce Function", Eq. 2, in LSE form).
 *
 * blob_dev: the plan's image in device memory (16-byte aligned).  k_pool,
 * v_pool: device [pool_rows][Hkv][d].  seq_lens: device [B] total tokens of
 * each sequence (batched + private), or NULL to read every private row the
 * descriptors give.  With seq_lens, a sequence reads the first seq_lens[b] -
 * (its batched rows) of its private rows, so the last private descriptor of a
 * sequence may name rows not yet written (room to append into without a new
 * plan); a length outside [batched rows, batched + private rows] makes the
 * row's O and LSE NaN.  q must match the plan's geometry.  lse may be NULL.
 */
hp_status hp_tree_step(const hp_query *q, const hp_tree_plan *plan, const void *blob_dev,
                       const void *k_pool, const void *v_pool, const int32_t *seq_lens,
                       float *o, float *lse, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * Decode-step KV append: token i's key and value rows (k_new, v_new: device
 * [n][Hkv][d]) are copied to pool row rows[i] (ChunkAttention page, section
 * "Prefix-Aware KV Cache (PAKV): The Prefix Tree Structure", the Append
 * operation: the new token's K/V
 * go into its sequence's leaf chunk).  rows: device [n]; an entry outside
 * [0, pool_rows) is skipped (nothing written, no length advanced).  If seq_idx
 * is not NULL, seq_lens[seq_idx[i]] is incremented for every token that was
 * written (device arrays; an index outside [0, num_seqs) is skipped), so a
 * captured step can advance its lengths without a host copy.  Rows of one
 * call must be distinct.  Exact copy.
 */
hp_status hp_kv_append(const void *k_new, const void *v_new, const int32_t *rows, int32_t n,
                       int32_t Hkv, int32_t d, int32_t dtype, void *k_pool, void *v_pool,
                       int64_t pool_rows, int32_t *seq_lens, const int32_t *seq_idx,
                       int32_t num_seqs, void *stream);

/*
 * Measurement aid (no part of the attention): reads `bytes` of device memory
 * at `buf` once, front to back, with 16-byte non-temporal loads, and writes
 * the XOR of all its 32-bit words, one partial per workgroup, to
 * sink[0 .. HP_READ_PROBE_WGS) (device memory; the XOR of the sink words is
 * the XOR of the buffer's words, so the loads cannot be elided).  A caller
 * times it to learn the device's streaming-read rate, reported beside the 8
 * TB/s specification.  buf 16-byte aligned, bytes a multiple of 16 (0 is
 * allowed: every sink word is then 0); HP_ERR_NULL for a NULL buf (bytes > 0)
 * or sink, HP_ERR_INVALID_ARG for misalignment.  Enqueued on `stream`.
 */
#define HP_READ_PROBE_WGS 512
hp_status hp_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/*
 * Prefix-aware KV cache manager (host only; ChunkAttention page, section
 * "Prefix-Aware KV Cache (PAKV): The Prefix Tree Structure", its Insert,
 * Append and Delete operations and its memory allocator; section "Design
 * Choices and Their Justifications" on the pool): a prefix tree whose nodes
 * hold token runs of at most HP_CHUNK tokens, each in one pool chunk, plus a
 * chunk allocator with a free list (freed chunks are reused, never returned).  It owns chunk
 * ids only; the caller owns the device pool of num_chunks * HP_CHUNK rows and
 * writes K/V where the manager says (hp_kv_append).
 *
 *   insert  the longest prefix of `tokens` already in the tree is shared (a
 *           node matched part-way is split, without copying); the remaining
 *           tokens get new chunks.  rows[t] receives the pool row of token t;
 *           rows of tokens >= *matched must be written by the caller.
 *   append  one new token at the end of a sequence: into its leaf chunk when
 *           the sequence alone owns that chunk's tail, else into a new chunk.
 *           *changed is 1 when the tree's shape changed (a new plan is due).
 *   remove  the sequence leaves; nodes no sequence passes through are freed
 *           and chunks no node uses return to the free list.
 *   context the (C, i, j) descriptors of the live tree in pre-order, with
 *           sequences numbered so that every node covers a contiguous range
 *           (the page's contiguity property); seq_order[b] is the id of batch
 *           row b and seq_lens[b] its token count.  A sequence's leaf chunk is
 *           reported with its remaining room, so the plan stays valid while
 *           tokens are appended into it.
 * Sequence ids are caller-chosen int64 values.  A handle is not thread-safe.
 * After HP_ERR_HOST (host memory exhausted part-way) a handle may be left
 * inconsistent and must only be destroyed.
 */
typedef struct hp_pakv hp_pakv;
typedef struct hp_pakv_stats {
    int32_t num_chunks;     /* capacity */
    int32_t chunks_used;    /* referenced by a node */
    int32_t chunks_free;    /* on the free list */
    int32_t chunks_fresh;   /* never handed out */
    int32_t nodes;          /* tree nodes, root excluded */
    int32_t seqs;           /* live sequences */
    int64_t tokens_stored;  /* tokens held by nodes (shared tokens once) */
    int64_t tokens_logical; /* sum of sequence lengths */
} hp_pakv_stats;

hp_status hp_pakv_create(int32_t num_chunks, hp_pakv **out);
void hp_pakv_destroy(hp_pakv *p);
hp_status hp_pakv_insert(hp_pakv *p, int64_t seq_id, const int32_t *tokens, int32_t n,
                         int32_t *rows, int32_t *matched);
hp_status hp_pakv_append(hp_pakv *p, int64_t seq_id, int32_t token, int32_t *row,
                         int32_t *changed);
hp_status hp_pakv_remove(hp_pakv *p, int64_t seq_id);
hp_status hp_pakv_context(hp_pakv *p, int64_t *seq_order, int32_t *seq_lens,
                          int32_t seq_capacity, hp_chunk_desc *descs, int32_t desc_capacity,
                          int32_t *num_seqs, int32_t *num_descs);
/* Pool rows of every token of one sequence, in order (n = its length). */
hp_status hp_pakv_seq_rows(hp_pakv *p, int64_t seq_id, int32_t *rows, int32_t capacity,
                           int32_t *n);
hp_status hp_pakv_get_stats(hp_pakv *p, hp_pakv_stats *stats);

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
