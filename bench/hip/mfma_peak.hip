// Matrix-core ceiling of the chip as this code can reach it: every wave of a full grid runs
// independent chains of v_mfma_f32_32x32x16_bf16 (the instruction every matrix kernel of the
// library uses) with no memory traffic, and the rate is timed with HIP events.  The published
// dense bf16 peak assumes the 2.4 GHz peak engine clock; under sustained matrix load the clock
// is lower, and this measures what is left.  With constant operands the chip holds about the
// peak clock; with random operands (sixteen operand registers of random bf16 of magnitude 1/4
// to 2, rotated so that consecutive instructions see different bits, as real data do) the
// switching power of the matrix cores alone lowers the clock, and that rate is the realistic
// ceiling for kernels on N(0, 1)-like data.  A second kernel runs the same on the 16x16x32
// instruction, to compare the two shapes' rate and power on random data.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kChains = 4;  // independent accumulators per wave: enough to keep the pipe full

__device__ __forceinline__ uint32_t mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    return x ^ (x >> 16);
}

// a bf16 of random sign and mantissa with exponent 125..128 (magnitude 1/4 to 2)
__device__ __forceinline__ uint32_t rand_bf16(uint32_t h) { return (h & 0x807fu) | ((125u + ((h >> 8) & 3u)) << 7); }

template <bool RANDOM>
__global__ __launch_bounds__(256) void mfma_chain_kernel(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    constexpr int NOP = RANDOM ? 8 : 1;  // operand registers of each side
    bf16x8 a[NOP], b[NOP];
#pragma unroll
    for (int k = 0; k < NOP; k++) {
        if (RANDOM) {
            u32x4 ua, ub;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t h1 = mix((uint32_t)(lane * 131 + k * 17 + j + 1) + blockIdx.x * 7919u);
                const uint32_t h2 = mix(h1 + 99991u);
                ua[j] = rand_bf16(h1) | (rand_bf16(h1 >> 16) << 16);
                ub[j] = rand_bf16(h2) | (rand_bf16(h2 >> 16) << 16);
            }
            a[k] = __builtin_bit_cast(bf16x8, ua);
            b[k] = __builtin_bit_cast(bf16x8, ub);
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++) {
                a[k][i] = (__bf16)(0.001f * (float)((lane + i) & 7));
                b[k][i] = (__bf16)(0.002f * (float)((lane * 3 + i) & 7));
            }
        }
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; c++) acc[c] = f32x16{};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int k = 0; k < 16; k++)
            acc[k % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k % NOP], b[(k * 3 + (k >> 3)) % NOP],
                                                                       acc[k % kChains], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; c++)
#pragma unroll
        for (int i = 0; i < 16; i++) s += acc[c][i];
    if (s == 123456.789f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the chains live
}
// The same on v_mfma_f32_16x16x32_bf16 (half the flops per instruction, a quarter of the
// accumulator), random operands only: twice the instructions per iteration, so an iteration is
// the same 2^19 flops per wave, over eight independent accumulators.  For the choice of shape:
// the larger one does more work per unit of energy on such data.
__global__ __launch_bounds__(256) void mfma16_chain_kernel(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    constexpr int NOP = 8;
    bf16x8 a[NOP], b[NOP];
#pragma unroll
    for (int k = 0; k < NOP; k++) {
        u32x4 ua, ub;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t h1 = mix((uint32_t)(lane * 131 + k * 17 + j + 1) + blockIdx.x * 7919u);
            const uint32_t h2 = mix(h1 + 99991u);
            ua[j] = rand_bf16(h1) | (rand_bf16(h1 >> 16) << 16);
            ub[j] = rand_bf16(h2) | (rand_bf16(h2 >> 16) << 16);
        }
        a[k] = __builtin_bit_cast(bf16x8, ua);
        b[k] = __builtin_bit_cast(bf16x8, ub);
    }
    constexpr int kChains16 = 8;
    f32x4 acc[kChains16];
#pragma unroll
    for (int c = 0; c < kChains16; c++) acc[c] = f32x4{};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int k = 0; k < 32; k++)
            acc[k % kChains16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k % NOP], b[(k * 3 + (k >> 3)) % NOP],
                                                                         acc[k % kChains16], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains16; c++)
#pragma unroll
        for (int i = 0; i < 4; i++) s += acc[c][i];
    if (s == 123456.789f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
}  // namespace

extern "C" {

// Runs the chain kernel on the current device over `blocks` workgroups of 4 waves (blocks = 256
// puts one wave on every SIMD of a 256-CU part, 512 two) for `iters` iterations of 16 matrix
// instructions per wave, with constant (random_operands = 0) or random operands, `reps` times
// after one warm-up launch.  Writes the best rate over the repetitions in TFLOP/s (dense:
// 2 * 32 * 32 * 16 flops per instruction).  Returns 0, or the HIP error code.
int mb_mfma_peak(int blocks, int iters, int reps, int random_operands, double* tflops) {
    float* sink = nullptr;
    hipError_t e = hipMalloc(&sink, (size_t)blocks * 256 * sizeof(float));
    if (e != hipSuccess) return (int)e;
    hipEvent_t t0, t1;
    hipEventCreate(&t0);
    hipEventCreate(&t1);
    double best = 0.0;
    for (int r = -1; r < reps && e == hipSuccess; r++) {
        hipEventRecord(t0, nullptr);
        if (random_operands)
            mfma_chain_kernel<true><<<blocks, 256, 0, nullptr>>>(iters, sink);
        else
            mfma_chain_kernel<false><<<blocks, 256, 0, nullptr>>>(iters, sink);
        hipEventRecord(t1, nullptr);
        e = hipEventSynchronize(t1);
        float ms = 0.f;
        hipEventElapsedTime(&ms, t0, t1);
        const double flops = 2.0 * 32 * 32 * 16 * 16 * (double)iters * blocks * 4;
        if (r >= 0 && ms > 0.f) best = flops / (ms * 1e-3) / 1e12 > best ? flops / (ms * 1e-3) / 1e12 : best;
    }
    hipEventDestroy(t0);
    hipEventDestroy(t1);
    hipFree(sink);
    *tflops = best;
    return e == hipSuccess ? 0 : (int)e;
}


// The 16x16x32 chains (random operands) in the same way: `blocks` workgroups of 4 waves for
// `iters` iterations of 32 instructions (the same flops per iteration as above), `reps` timed
// launches after a warm-up; best rate in TFLOP/s.  Returns 0, or the HIP error code.
int mb_mfma_peak_16x16x32(int blocks, int iters, int reps, double* tflops) {
    float* sink = nullptr;
    hipError_t e = hipMalloc(&sink, (size_t)blocks * 256 * sizeof(float));
    if (e != hipSuccess) return (int)e;
    hipEvent_t t0, t1;
    hipEventCreate(&t0);
    hipEventCreate(&t1);
    double best = 0.0;
    for (int r = -1; r < reps && e == hipSuccess; r++) {
        hipEventRecord(t0, nullptr);
        mfma16_chain_kernel<<<blocks, 256, 0, nullptr>>>(iters, sink);
        hipEventRecord(t1, nullptr);
        e = hipEventSynchronize(t1);
        float ms = 0.f;
        hipEventElapsedTime(&ms, t0, t1);
        const double flops = 2.0 * 16 * 16 * 32 * 32 * (double)iters * blocks * 4;
        if (r >= 0 && ms > 0.f) best = flops / (ms * 1e-3) / 1e12 > best ? flops / (ms * 1e-3) / 1e12 : best;
    }
    hipEventDestroy(t0);
    hipEventDestroy(t1);
    hipFree(sink);
    *tflops = best;
    return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
