// Row-wise float32 kernels around the attention passes: the LSE merge of local softmax
// results, delta = rowsum(dO * O) for the backward, the sum of per-part dQ, and zeroing.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

// Composition of local softmax results into the global one (LongStraw digest, "Method",
// Qwen implementation: global LSE/output merge; here numerator and weights are float32):
//   L = m + log sum_p exp(L_p - m), m = max_p L_p;  O = sum_p exp(L_p - L) O_p.
// BF16NUM is the pages' own variant, whose numerator is BF16 (explainer, "The fine print"):
// each term exp(L_p - m) O_p is rounded to bf16 and so is the running sum after every
// addition, in part order (a bf16 reduction over the owners); the denominator and L stay
// float32, and O = numerator / sum_p exp(L_p - m).
// Each thread owns 4 consecutive elements of one row.
template <typename OutT, bool BF16NUM>
__global__ __launch_bounds__(256) void lse_merge_kernel(int n_parts, int64_t n_rows, int d,
                                                        const float* __restrict__ o_parts,
                                                        const float* __restrict__ lse_parts,
                                                        OutT* __restrict__ o_out,
                                                        float* __restrict__ lse_out) {
    const int vecs = d / 4;
    const int rows_per_block = 256 / vecs;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / vecs;
    const int c = threadIdx.x % vecs;
    if (threadIdx.x >= rows_per_block * vecs || row >= n_rows) return;
    // the largest part LSE, NaN if any part is NaN (a NaN input then gives a NaN row rather
    // than one that looks empty)
    float m = -INFINITY;
    for (int p = 0; p < n_parts; p++) {
        const float lp = lse_parts[(int64_t)p * n_rows + row];
        m = (lp > m || lp != lp) ? lp : m;
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float L = -INFINITY;
    if (m != -INFINITY) {
        float ssum = 0.f;
        for (int p = 0; p < n_parts; p++) ssum += expf(lse_parts[(int64_t)p * n_rows + row] - m);
        L = m + logf(ssum);
        for (int p = 0; p < n_parts; p++) {
            const float lp = lse_parts[(int64_t)p * n_rows + row];
            if (lp == -INFINITY) continue;
            const float4 v = *reinterpret_cast<const float4*>(o_parts + ((int64_t)p * n_rows + row) * d + 4 * c);
            const float ve[4] = {v.x, v.y, v.z, v.w};
            if (BF16NUM) {
                const float w = expf(lp - m);
                auto rb = [](float x) { return bf16_to_f32(f32_to_bf16(x)); };
#pragma unroll
                for (int e = 0; e < 4; e++) acc[e] = rb(acc[e] + rb(w * ve[e]));
            } else {
                const float w = expf(lp - L);
#pragma unroll
                for (int e = 0; e < 4; e++) acc[e] += w * ve[e];
            }
        }
        if (BF16NUM) {
#pragma unroll
            for (int e = 0; e < 4; e++) acc[e] /= ssum;
        }
    }
    OutT* dst = o_out + row * d + 4 * c;
#pragma unroll
    for (int e = 0; e < 4; e++) store_f32<OutT>(dst + e, acc[e]);
    if (c == 0) lse_out[row] = L;
}

// delta[row] = sum_k dO[row, k] * O[row, k]; one wave per row, 4 rows per block.
template <typename T>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                    int64_t n_rows, int d, float* __restrict__ delta) {
    const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    if (row >= n_rows) return;
    float s = 0.f;
    for (int k = lane; k < d; k += 64) s += load_f32<T>(o + row * d + k) * load_f32<T>(dout + row * d + k);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) delta[row] = s;
}

__global__ __launch_bounds__(256) void sum_parts_kernel(int n_parts, int64_t n4, const float4* __restrict__ parts,
                                                        float4* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    float4 a = parts[i];
    for (int p = 1; p < n_parts; p++) {
        const float4 b = parts[(int64_t)p * n4 + i];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    out[i] = a;
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

}  // namespace

hipError_t launch_lse_merge(int n_parts, int64_t n_rows, int d, const float* o_parts,
                            const float* lse_parts, void* o_out, int out_dtype, float* lse_out,
                            hipStream_t s, bool bf16_numerator) {
    if (n_rows == 0) return hipSuccess;
    const int rows_per_block = 256 / (d / 4);
    const unsigned grid = (unsigned)((n_rows + rows_per_block - 1) / rows_per_block);
    KernelTimer kt("lse_merge", s);
    if (bf16_numerator) {
        if (out_dtype == 0)
            lse_merge_kernel<float, true><<<grid, 256, 0, s>>>(n_parts, n_rows, d, o_parts, lse_parts, (float*)o_out,
                                                               lse_out);
        else
            lse_merge_kernel<bf16_t, true><<<grid, 256, 0, s>>>(n_parts, n_rows, d, o_parts, lse_parts,
                                                                (bf16_t*)o_out, lse_out);
    } else if (out_dtype == 0) {
        lse_merge_kernel<float, false><<<grid, 256, 0, s>>>(n_parts, n_rows, d, o_parts, lse_parts, (float*)o_out,
                                                            lse_out);
    } else {
        lse_merge_kernel<bf16_t, false><<<grid, 256, 0, s>>>(n_parts, n_rows, d, o_parts, lse_parts, (bf16_t*)o_out,
                                                             lse_out);
    }
    return hipGetLastError();
}

hipError_t launch_delta(const void* o, const void* dout, int dtype, int64_t n_rows, int d,
                        float* delta, hipStream_t s) {
    if (n_rows == 0) return hipSuccess;
    const unsigned grid = (unsigned)((n_rows + 3) / 4);
    KernelTimer kt("delta", s);
    if (dtype == 0)
        delta_kernel<float><<<grid, 256, 0, s>>>((const float*)o, (const float*)dout, n_rows, d, delta);
    else
        delta_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)o, (const bf16_t*)dout, n_rows, d, delta);
    return hipGetLastError();
}

hipError_t launch_sum_parts(int n_parts, int64_t n, const float* parts, float* out, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int64_t n4 = n / 4;
    KernelTimer kt("dq_sum_parts", s);
    sum_parts_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(n_parts, n4, (const float4*)parts, (float4*)out);
    return hipGetLastError();
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    KernelTimer kt("zero", s);
    zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n);
    return hipGetLastError();
}

}  // namespace ls
