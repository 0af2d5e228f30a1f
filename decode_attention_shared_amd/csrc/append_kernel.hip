// Decode-step KV append: scatter each new token's key and value rows into its
// pool row ("ChunkAttention: Efficient Self-Attention with Prefix-Aware KV
// Cache and Two-Phase Partition", section "Prefix-Aware KV Cache (PAKV): The
// Prefix Tree Structure", the Append operation: every sequence's new token
// goes into its leaf chunk).  A pure copy bound by HBM: 16 bytes per lane,
// one workgroup column per token row, so a row's Hkv*d elements are read and
// written with full 64-byte-per-quad-lane coalescing.
#include "common.hpp"

namespace hp {

__global__ __launch_bounds__(256) void kv_append_kernel(const u32x4 *__restrict__ k_new,
                                                        const u32x4 *__restrict__ v_new,
                                                        const int32_t *__restrict__ rows,
                                                        int64_t row_vecs, u32x4 *k_pool,
                                                        u32x4 *v_pool, int64_t pool_rows,
                                                        int32_t *seq_lens,
                                                        const int32_t *seq_idx, int32_t num_seqs) {
    const int64_t i = blockIdx.x;  // token
    const int64_t c = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;  // 16-byte column
    const int32_t r = rows[i];
    if (r < 0 || r >= pool_rows) return;  // never written: the row is skipped
    if (c < row_vecs) {
        k_pool[(int64_t)r * row_vecs + c] = k_new[i * row_vecs + c];
        v_pool[(int64_t)r * row_vecs + c] = v_new[i * row_vecs + c];
    }
    if (seq_lens != nullptr && blockIdx.y == 0 && threadIdx.x == 0) {
        const int32_t b = seq_idx[i];
        if (b >= 0 && b < num_seqs) atomicAdd(&seq_lens[b], 1);
    }
}

hipError_t launch_kv_append(const void *k_new, const void *v_new, const int32_t *rows, int32_t n,
                            int64_t row_bytes, void *k_pool, void *v_pool, int64_t pool_rows,
                            int32_t *seq_lens, const int32_t *seq_idx, int32_t num_seqs,
                            hipStream_t s) {
    const int64_t row_vecs = row_bytes / 16;
    const dim3 grid((unsigned)n, (unsigned)((row_vecs + 255) / 256));
    kv_append_kernel<<<grid, 256, 0, s>>>((const u32x4 *)k_new, (const u32x4 *)v_new, rows,
                                          row_vecs, (u32x4 *)k_pool, (u32x4 *)v_pool, pool_rows,
                                          seq_lens, seq_idx, num_seqs);
    return hipGetLastError();
}

}  // namespace hp
