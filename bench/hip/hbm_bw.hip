// HBM ceilings as this code can reach them: a streaming read, a streaming write and a copy of a
// buffer much larger than the last-level caches, each with 16-byte accesses by every lane of a
// full grid, timed with HIP events.  The read is also run over random bits and over zeros, since
// the rate a memory-bound pass reaches was seen to depend on the data it reads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kUnroll = 4;  // 16-byte loads in flight per lane per iteration

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, size_t n16, uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = {0, 0, 0, 0};
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; u++) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= src[i];
    const uint32_t s = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (s == 0x9e3779b9u) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the loads live
}

__global__ __launch_bounds__(256) void write_kernel(u32x4* __restrict__ dst, size_t n16, uint32_t seed) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const uint32_t x = (uint32_t)i * 0x9e3779b9u ^ seed;
        dst[i] = u32x4{x, x ^ 0x85ebca6bu, x ^ 0xc2b2ae35u, x ^ 0x27d4eb2fu};
    }
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Fill with random bits (an integer hash of the index: every bit toggles) or zeros.
__global__ __launch_bounds__(256) void fill_kernel(u32x4* __restrict__ dst, size_t n16, int random) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        if (!random) {
            dst[i] = u32x4{0, 0, 0, 0};
            continue;
        }
        u32x4 v;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            uint64_t z = (uint64_t)(4 * i + k) + 0x9e3779b97f4a7c15ull;
            z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
            z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
            v[k] = (uint32_t)(z ^ (z >> 31));
        }
        dst[i] = v;
    }
}

}  // namespace

extern "C" {

// mode 0: read `bytes`; 1: write `bytes`; 2: copy `bytes` (read + write, counted as 2 * bytes).
// fill: the buffer read holds random bits (1) or zeros (0).  `blocks` workgroups of 256 lanes
// (a few per CU).  Writes the best rate over `reps` timed launches (after one warm-up) in GB/s
// of HBM traffic.  Allocates its own buffers.  Returns 0, or the HIP error code.
int mb_hbm(int mode, size_t bytes, int fill, int blocks, int reps, double* gbs) {
    const size_t n16 = bytes / 16;
    u32x4 *a = nullptr, *b = nullptr;
    uint32_t* sink = nullptr;
    hipError_t e = hipMalloc(&a, n16 * 16);
    if (e == hipSuccess && mode == 2) e = hipMalloc(&b, n16 * 16);
    if (e == hipSuccess) e = hipMalloc(&sink, (size_t)blocks * 256 * sizeof(uint32_t));
    if (e == hipSuccess) fill_kernel<<<2048, 256>>>(a, n16, fill);
    hipEvent_t t0, t1;
    hipEventCreate(&t0);
    hipEventCreate(&t1);
    double best = 0.0;
    for (int r = -1; r < reps && e == hipSuccess; r++) {
        hipEventRecord(t0, nullptr);
        if (mode == 0) read_kernel<<<blocks, 256>>>(a, n16, sink);
        else if (mode == 1) write_kernel<<<blocks, 256>>>(a, n16, (uint32_t)r);
        else copy_kernel<<<blocks, 256>>>(a, b, n16);
        hipEventRecord(t1, nullptr);
        e = hipEventSynchronize(t1);
        float ms = 0.f;
        hipEventElapsedTime(&ms, t0, t1);
        const double moved = (mode == 2 ? 2.0 : 1.0) * (double)(n16 * 16);
        if (r >= 0 && ms > 0.f && moved / (ms * 1e-3) / 1e9 > best) best = moved / (ms * 1e-3) / 1e9;
    }
    hipEventDestroy(t0);
    hipEventDestroy(t1);
    hipFree(a);
    if (b) hipFree(b);
    hipFree(sink);
    *gbs = best;
    return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
