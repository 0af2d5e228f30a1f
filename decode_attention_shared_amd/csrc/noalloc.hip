// hp_cascade_step_noalloc: the one-stream cascade step with its workspace in
// a fixed device array of the library instead of caller-allocated memory, for
// callers that cannot allocate device memory.
#include <hip/hip_runtime.h>

#include <mutex>

#include "guard.hpp"
#include "host.hpp"

namespace {

using namespace hp::host;

// The workspace of every hp_cascade_step_noalloc call on a GPU: one copy per
// GPU, loaded with the library's code object and held until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: it is
// never passed to a kernel or a copy.  Its device address comes from
// hipGetSymbolAddress, once per device (scratch_on).
static __device__ __align__(256) unsigned char scratch[HP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device ordinal, once looked up

// The device that work enqueued on `stream` runs on.
hp_status stream_device(void *stream, int *dev) {
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, dev) : hipGetDevice(dev);
    return e == hipSuccess ? HP_OK : fail_hip(e);
}

// Device address of `scratch` on device `dev`, looked up with that device
// current on the first call for it (the caller's current device is restored).
hp_status scratch_on(int dev, void **out) {
    if (dev < 0 || dev >= kMaxDevices) return HP_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return fail_hip(e);
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return fail_hip(e);
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return fail_hip(e);
        if (back != hipSuccess) return fail_hip(back);
        if (!p) return HP_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return HP_OK;
}

}  // namespace

extern "C" hp_status hp_cascade_step_noalloc(const hp_query *q, const hp_prefix_tree *tree,
                                             const hp_paged_kv *kv, float *o, float *lse,
                                             void *stream) {
    return hp::guarded([&]() -> hp_status {
        size_t need = 0;
        hp_status st = cascade_serial_plan(q, tree, kv, o, lse, &need);
        if (st != HP_OK) return st;
        if (need > (size_t)HP_NOALLOC_SCRATCH_BYTES) return HP_ERR_CAPACITY;
        int dev = -1;
        if ((st = stream_device(stream, &dev)) != HP_OK) return st;
        void *ws = nullptr;
        if ((st = scratch_on(dev, &ws)) != HP_OK) return st;
        // Nothing in the workspace has to start at zero: every partial the
        // merge reads is written earlier in the same step.
        return cascade_serial(q, tree, kv, o, lse, ws, HP_NOALLOC_SCRATCH_BYTES, stream);
    });
}
