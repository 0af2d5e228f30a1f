// Stream-id mask of shared-context decode, evaluated on the device.
//
// A shared-context request decodes P independent streams at once; its KV row
// holds every stream's tokens (questions, then the streams' answer tokens
// interleaved step by step), each position tagged with the id of the stream
// it belongs to, or -1 for tokens every stream may see.  A query of stream s
// attends a position only when that position's id is -1 or s: the other
// streams' tokens never enter its softmax, so its result equals that of a
// request holding only the shared tokens and its own ("Read Once, Answer
// Many: Parallel Prompting for Shared-Context LLM Inference", section
// "Parallel Prompting", Eq. 2 and Figure 2; its document is a shared prefix
// read once for all streams by the prefix pass).
//
// Instead of streaming every position's keys and discarding the masked ones
// (the page's kernel scans the whole row), this kernel evaluates the mask on
// the stream ids alone (4 bytes per position) and writes, per query, the
// pool rows of its visible positions in row order; the sequence-first pass
// then reads only those keys.  One workgroup per query: each thread tests 8
// consecutive positions, a workgroup prefix sum of the counts gives every
// visible position its output slot, so the order is the row order and the
// result is deterministic.
#include "common.hpp"

namespace hp {

constexpr int kSelThreads = 256;
constexpr int kSelPer = 8;  // consecutive positions per thread per pass

__global__ __launch_bounds__(kSelThreads) void stream_select_kernel(StreamSelectArgs a) {
    __shared__ int sm_wave[kSelThreads / kWave];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int r = a.q_req[b];
    const int s = a.q_sid[b];
    int len = -1;
    if (r >= 0 && r < a.R) len = a.row_len[r];
    if (len < 0 || len > a.row_cap) {  // uniform over the workgroup
        if (tid == 0) a.tok_len[b] = -1;
        return;
    }
    const int32_t *sid = a.slot_sid + (int64_t)r * a.row_cap;
    const int32_t *slot = a.row_slots + (int64_t)r * a.row_cap;
    int32_t *out = a.tok_table + (int64_t)b * a.row_cap;
    int n = 0;
#pragma unroll 1
    for (int base = 0; base < len; base += kSelThreads * kSelPer) {
        const int p0 = base + tid * kSelPer;
        unsigned vis = 0;
#pragma unroll
        for (int k = 0; k < kSelPer; ++k) {
            const int p = p0 + k;
            if (p < len) {
                const int sd = sid[p];
                if (sd == -1 || sd == s) vis |= 1u << k;
            }
        }
        const int c = __popc(vis);
        int x = c;  // inclusive prefix sum of the counts within the wave
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_up(x, off, kWave);
            if (lane >= off) x += y;
        }
        if (lane == kWave - 1) sm_wave[wave] = x;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kSelThreads / kWave; ++w) {
            const int t = sm_wave[w];
            before += w < wave ? t : 0;
            total += t;
        }
        __syncthreads();  // sm_wave is rewritten by the next pass
        int o = n + before + x - c;
#pragma unroll
        for (int k = 0; k < kSelPer; ++k)
            if ((vis >> k) & 1u) out[o++] = slot[p0 + k];
        n += total;
    }
    if (tid == 0) a.tok_len[b] = n;
}

hipError_t launch_stream_select(const StreamSelectArgs &a, hipStream_t s) {
    if (a.B <= 0) return hipSuccess;
    stream_select_kernel<<<a.B, kSelThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace hp
