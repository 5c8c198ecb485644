// LDS ceilings as this code can reach them: the aggregate read rate of ds_read_b128 and of the
// transposing ds_read_b64_tr_b16 (conflict-free addresses, every CU, 4 or 8 waves per CU), and
// the rate of a chain of v_mfma_f32_32x32x16_bf16 whose B operand is a fresh 1 KiB LDS read per
// instruction (the operand pattern of the library's matrix kernels), per two instructions, or
// two 512-byte transposed reads per instruction (the accumulation pattern of the dK/dV pass).
//
// Every LDS address is formed from the buffer's own address: a buffer reached only through
// integer addresses is dropped by the compiler (no LDS is allocated), and reads past a
// workgroup's allocation return zeros without touching the banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS __attribute__((address_space(3)))

constexpr int kLdsBytes = 64 * 1024;

__device__ __forceinline__ uint32_t lds_base(const char* buf) { return (uint32_t)(uintptr_t)(const LDS char*)buf; }

// mode 0: ds_read_b128, mode 1: ds_read_b64_tr_b16; 8 reads in flight per wave
template <int MODE>
__global__ void lds_read_kernel(int iters, uint32_t* __restrict__ sink) {
    __shared__ __attribute__((aligned(1024))) char buf[kLdsBytes];
    for (int i = threadIdx.x * 16; i < kLdsBytes; i += blockDim.x * 16)
        *(u32x4*)(buf + i) = u32x4{(uint32_t)i, 1u, 2u, 3u};
    __syncthreads();
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    // each wave walks its own 8 KiB window of 1 KiB blocks; lane l reads 16 (or 8) consecutive bytes
    const uint32_t base = lds_base(buf) + (uint32_t)((w * 8192) % kLdsBytes);
    u32x4 acc = {0, 0, 0, 0};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            // the block read rotates with the iteration, so no read is loop-invariant
            const uint32_t off = base + (uint32_t)(((it + j) & 7) * 1024);
            if (MODE == 0) {
                acc ^= *(const LDS u32x4*)(uintptr_t)(off + lane * 16);
            } else {
                const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (LDS i16x4*)(uintptr_t)(off + lane * 8));
                acc.x ^= (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
                acc.y ^= (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
            }
        }
    }
    const uint32_t s = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (s == 0x12345678u) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// A chain of matrix instructions over 4 accumulators, B read from LDS: one 1 KiB read per
// instruction (PER = 1) or per two instructions (PER = 2), prefetched 4 reads ahead; PER = 0:
// two 512-byte transposed reads per instruction, prefetched 4 instructions ahead.
template <int PER>
__global__ void lds_mfma_kernel(int iters, float* __restrict__ sink) {
    __shared__ __attribute__((aligned(1024))) char buf[kLdsBytes];
    for (int i = threadIdx.x * 16; i < kLdsBytes; i += blockDim.x * 16)
        *(u32x4*)(buf + i) = u32x4{0x3c003c00u, 0x3c003c00u, 0u, 0u};
    __syncthreads();
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t base = lds_base(buf) + (uint32_t)((w * 8192) % kLdsBytes);
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; i++) a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; c++) acc[c] = f32x16{};
    if constexpr (PER == 0) {
        auto tr = [&](uint32_t off) {
            return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(uintptr_t)(off + lane * 8));
        };
        i16x4 b[4][2];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            b[j][0] = tr(base + j * 1024);
            b[j][1] = tr(base + j * 1024 + 512);
        }
        for (int it = 0; it < iters; it++) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const bf16x8 bj = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(b[j][0], b[j][1], 0, 1, 2, 3, 4, 5, 6, 7));
                const uint32_t next = base + ((it * 4 + j + 4) & 7) * 1024;
                b[j][0] = tr(next);
                b[j][1] = tr(next + 512);
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bj, acc[j], 0, 0, 0);
            }
        }
    } else {
        bf16x8 b[4];
#pragma unroll
        for (int j = 0; j < 4; j++) b[j] = *(const LDS bf16x8*)(uintptr_t)(base + j * 1024 + lane * 16);
        for (int it = 0; it < iters; it++) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const bf16x8 bj = b[j];
                b[j] = *(const LDS bf16x8*)(uintptr_t)(base + ((it * 4 + j + 4) & 7) * 1024 + lane * 16);
#pragma unroll
                for (int r = 0; r < PER; r++)
                    acc[(j * PER + r) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bj, acc[(j * PER + r) & 3], 0, 0, 0);
            }
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
        for (int i = 0; i < 16; i++) s += acc[c][i];
    if (s == 123456.789f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <typename Launch>
double best_ms(int reps, Launch&& launch, hipError_t* err) {
    hipEvent_t t0, t1;
    hipEventCreate(&t0);
    hipEventCreate(&t1);
    double best = 1e30;
    for (int r = -1; r < reps && *err == hipSuccess; r++) {
        hipEventRecord(t0, nullptr);
        launch();
        hipEventRecord(t1, nullptr);
        *err = hipEventSynchronize(t1);
        float ms = 0.f;
        hipEventElapsedTime(&ms, t0, t1);
        if (r >= 0 && ms > 0.f && ms < best) best = ms;
    }
    hipEventDestroy(t0);
    hipEventDestroy(t1);
    return best;
}

}  // namespace

extern "C" {

// mode 0 / 1: LDS read rate in TB/s of ds_read_b128 / ds_read_b64_tr_b16 over `blocks`
// workgroups of `waves` waves (one workgroup per CU at 64 KiB of LDS each).
// mode 2 / 3: TFLOP/s of the LDS-fed matrix chain with one 1 KiB read per one / two
// instructions; mode 4: with two 512-byte transposed reads per instruction.  Writes the best of `reps` timed launches.  Returns 0 or the HIP error code.
int mb_lds(int mode, int blocks, int waves, int iters, int reps, double* rate) {
    uint32_t* sink = nullptr;
    hipError_t e = hipMalloc(&sink, (size_t)blocks * waves * 64 * sizeof(float));
    if (e != hipSuccess) return (int)e;
    const int threads = waves * 64;
    const double ms = best_ms(reps, [&] {
        if (mode == 0) lds_read_kernel<0><<<blocks, threads>>>(iters, sink);
        else if (mode == 1) lds_read_kernel<1><<<blocks, threads>>>(iters, sink);
        else if (mode == 2) lds_mfma_kernel<1><<<blocks, threads>>>(iters, (float*)sink);
        else if (mode == 3) lds_mfma_kernel<2><<<blocks, threads>>>(iters, (float*)sink);
        else lds_mfma_kernel<0><<<blocks, threads>>>(iters, (float*)sink);
    }, &e);
    hipFree(sink);
    if (e != hipSuccess) return (int)e;
    const double per_wave_iter = mode == 0 ? 8.0 * 1024 : mode == 1 ? 8.0 * 512 : 2.0 * 32 * 32 * 16 * 4 * (mode == 3 ? 2 : 1);
    const double total = per_wave_iter * (double)iters * blocks * waves;
    *rate = total / (ms * 1e-3) / 1e12;  // TB/s or TFLOP/s
    return 0;
}

}  // extern "C"
