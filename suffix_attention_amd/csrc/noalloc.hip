// Scratch memory of the no-allocation forward (ls_replay_fwd_noalloc), for callers that cannot
// allocate device memory.  The forward's per-part results (o_parts, lse_parts) live in one
// fixed array per GPU instead of a caller's workspace.  The array is a device global: every GPU
// the library runs on holds its own copy, at its own address, until the process ends.  Host
// code never uses the array's name as an address.  Its device address comes from
// hipGetSymbolAddress, taken once per device with that device current and kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/longstraw.h"
#include "launch.hpp"

namespace ls {

// 256 MiB: the forward workspace of a 1,024-row block over 8 prompt shards at hq = 24, d = 256
// (227 MB) fits.
constexpr size_t kNoAllocScratchBytes = LS_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) __attribute__((used)) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once set up
}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    *bytes = kNoAllocScratchBytes;
    return hipSuccess;
}

}  // namespace ls
