// Matrix-core ceiling of the chip as this code can reach it: every wave of a full grid runs
// independent chains of v_mfma_f32_32x32x16_bf16 (the instruction every matrix kernel of the
// library uses) with no memory traffic, and the rate is timed with HIP events.  The published
// dense bf16 peak assumes the 2.4 GHz peak engine clock; under sustained matrix load the clock
// is lower, and this measures what is left.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;  // independent accumulators per wave: enough to keep the pipe full

__global__ __launch_bounds__(256) void mfma_chain_kernel(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
        b[i] = (__bf16)(0.002f * (float)((lane * 3 + i) & 7));
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; c++) acc[c] = f32x16{};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int c = 0; c < kChains; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; c++)
#pragma unroll
        for (int i = 0; i < 16; i++) s += acc[c][i];
    if (s == 123456.789f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the chains live
}

}  // namespace

extern "C" {

// Runs the chain kernel on the current device over `blocks` workgroups of 4 waves (blocks = 256
// puts one wave on every SIMD of a 256-CU part, 512 two) for `iters` iterations of kChains matrix
// instructions per wave, `reps` times after one warm-up launch.  Writes the best rate over the
// repetitions in TFLOP/s (dense: 2 * 32 * 32 * 16 flops per instruction).  Returns 0, or the HIP
// error code.
int mb_mfma_peak(int blocks, int iters, int reps, double* tflops) {
    float* sink = nullptr;
    hipError_t e = hipMalloc(&sink, (size_t)blocks * 256 * sizeof(float));
    if (e != hipSuccess) return (int)e;
    hipEvent_t t0, t1;
    hipEventCreate(&t0);
    hipEventCreate(&t1);
    double best = 0.0;
    for (int r = -1; r < reps && e == hipSuccess; r++) {
        hipEventRecord(t0, nullptr);
        mfma_chain_kernel<<<blocks, 256, 0, nullptr>>>(iters, sink);
        hipEventRecord(t1, nullptr);
        e = hipEventSynchronize(t1);
        float ms = 0.f;
        hipEventElapsedTime(&ms, t0, t1);
        const double flops = 2.0 * 32 * 32 * 16 * kChains * (double)iters * blocks * 4;
        if (r >= 0 && ms > 0.f) best = flops / (ms * 1e-3) / 1e12 > best ? flops / (ms * 1e-3) / 1e12 : best;
    }
    hipEventDestroy(t0);
    hipEventDestroy(t1);
    hipFree(sink);
    *tflops = best;
    return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
