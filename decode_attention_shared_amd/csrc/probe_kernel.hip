// Streaming-read probe: the rate at which this device's HBM delivers a plain
// sequential read, measured beside the specification's 8 TB/s so that a
// step's effective bandwidth can be read against both.  Every lane streams
// 16-byte non-temporal loads (four independent ones in flight per lane and
// iteration) over a grid-stride range and folds them with XOR, one word per
// workgroup goes to `sink` so that no load can be elided.  Two 256-thread
// workgroups per CU (the host launches HP_READ_PROBE_WGS = 512) read a 4 GiB
// buffer at 6.8-7.1 TB/s on MI355X; 2 048 or 8 192 workgroups, or eight loads
// per lane, reach only 6.1-6.8.
#include "common.hpp"

namespace hp {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *__restrict__ buf,
                                                                   int64_t nvec,
                                                                   uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t acc = 0;
#pragma unroll 1
    for (; i + 3 * stride < nvec; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(buf + i);
        const u32x4 b = __builtin_nontemporal_load(buf + i + stride);
        const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * stride);
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^
               (d.x ^ d.y ^ d.z ^ d.w);
    }
#pragma unroll 1
    for (; i < nvec; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(buf + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // workgroup XOR: within each wave by shuffles, then across the 4 waves in LDS
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, kWave);
    __shared__ uint32_t part[kProbeThreads / kWave];
    if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
#pragma unroll
        for (int w = 0; w < kProbeThreads / kWave; ++w) x ^= part[w];
        sink[blockIdx.x] = x;
    }
}

hipError_t launch_read_probe(const void *buf, int64_t bytes, uint32_t *sink, int wgs,
                             hipStream_t s) {
    read_probe_kernel<<<wgs, kProbeThreads, 0, s>>>((const u32x4 *)buf, bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace hp
