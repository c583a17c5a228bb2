// fa_fwd_splitkv_noalloc: the key-split forward on a fixed scratch array of
// the library instead of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The fp32 partial results of the key splits live in `scratch`, a
// file-scope device array of kScratchBytes.  Each GPU the library runs on
// holds its own copy at its own address until the process ends.  Host code
// never passes the array's name to a kernel (in host code it is only a
// stand-in for the symbol): on the first call on a device, with that device
// current, hipGetSymbolAddress yields the device address, which is kept per
// device and passed on as the workspace of the ordinary key-split path.
// Nothing is allocated or freed per call.  Every call on one GPU shares that
// GPU's array: calls that overlap in time on one GPU race (their partials
// collide).  The split kernels write every partial element they merge, so
// nothing in the array needs to start at zero.

#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)40 << 20;   // 40 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up once per
// device, with that device current); nullptr if the lookup fails.
void* scratch_address(int dev) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t fa_noalloc_scratch_bytes(void) { return kScratchBytes; }

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Lq, int Lk, int d, int causal, float scale,
                           int num_splits, hipStream_t stream) {
    // every argument check first, on the host; then the partials must fit
    // the fixed array
    const int st = fa::splitkv_check(q, k, v, o, lse, B, H, Lq, Lk, d, causal, scale,
                                     num_splits);
    if (st != FA_OK) return st;
    if (fa_splitkv_workspace_size(B, H, Lq, d, num_splits) > kScratchBytes) return FA_ERR_SCRATCH;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
    void* ws = scratch_address(dev);
    if (!ws) return FA_ERR_LAUNCH;
    return fa_fwd_splitkv(q, k, v, o, lse, B, H, Lq, Lk, d, causal, scale, num_splits, ws,
                          kScratchBytes, stream);
}

}  // extern "C"
