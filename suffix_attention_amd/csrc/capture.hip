// Page capture and gather: the page-table walk between logical prompt order and the
// physical page pools (LongStraw digest, "Method", step 1: the captured prompt keeps its
// KV pages).  Logical token t lives in row t % 64 of physical page table[t / 64]; a pool
// is [n_phys, hkv, 64, d], so one (page, kv head) tile is a contiguous 64 x d block.
#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

// One thread moves one 8-element chunk of one (token, head) row.
template <typename SrcT, typename DstT>
__global__ __launch_bounds__(256) void capture_kernel(const SrcT* __restrict__ ks,
                                                      const SrcT* __restrict__ vs,
                                                      int64_t n_tok, int64_t first_tok,
                                                      const int32_t* __restrict__ table,
                                                      DstT* __restrict__ kp, DstT* __restrict__ vp,
                                                      int64_t n_phys, int hkv, int d) {
    const int chunks = d / 8;
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n_items = n_tok * hkv * chunks;
    if (item >= n_items) return;
    const int c = (int)(item % chunks);
    const int64_t th = item / chunks;
    const int h = (int)(th % hkv);
    const int64_t t = th / hkv;
    const int64_t T = first_tok + t;
    const int32_t phys = table[T / kPage];
    if (phys < 0 || phys >= n_phys) return;  // invalid table entry: write nothing
    const int64_t src = (t * hkv + h) * d + c * 8;
    const int64_t dst = (((int64_t)phys * hkv + h) * kPage + (T % kPage)) * d + c * 8;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        store_f32<DstT>(kp + dst + e, load_f32<SrcT>(ks + src + e));
        store_f32<DstT>(vp + dst + e, load_f32<SrcT>(vs + src + e));
    }
}

// Bit copies (same dtype) use 16-byte moves.
__global__ __launch_bounds__(256) void capture_copy_kernel(const uint4* __restrict__ ks,
                                                           const uint4* __restrict__ vs,
                                                           int64_t n_tok, int64_t first_tok,
                                                           const int32_t* __restrict__ table,
                                                           uint4* __restrict__ kp,
                                                           uint4* __restrict__ vp, int64_t n_phys,
                                                           int hkv, int row_vecs) {
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n_items = n_tok * hkv * row_vecs;
    if (item >= n_items) return;
    const int c = (int)(item % row_vecs);
    const int64_t th = item / row_vecs;
    const int h = (int)(th % hkv);
    const int64_t t = th / hkv;
    const int64_t T = first_tok + t;
    const int32_t phys = table[T / kPage];
    if (phys < 0 || phys >= n_phys) return;
    const int64_t src = (t * hkv + h) * row_vecs + c;
    const int64_t dst = (((int64_t)phys * hkv + h) * kPage + (T % kPage)) * row_vecs + c;
    kp[dst] = ks[src];
    vp[dst] = vs[src];
}

__global__ __launch_bounds__(256) void gather_copy_kernel(const uint4* __restrict__ pages,
                                                          const int32_t* __restrict__ table,
                                                          int64_t n_phys, int64_t first_tok,
                                                          int64_t n_tok, int hkv, int row_vecs,
                                                          uint4* __restrict__ dst) {
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n_items = n_tok * hkv * row_vecs;
    if (item >= n_items) return;
    const int c = (int)(item % row_vecs);
    const int64_t th = item / row_vecs;
    const int h = (int)(th % hkv);
    const int64_t t = th / hkv;
    const int64_t T = first_tok + t;
    int32_t phys = table[T / kPage];
    const int64_t o = (t * hkv + h) * row_vecs + c;
    if (phys < 0 || phys >= n_phys) {
        dst[o] = make_uint4(0, 0, 0, 0);
        return;
    }
    dst[o] = pages[(((int64_t)phys * hkv + h) * kPage + (T % kPage)) * row_vecs + c];
}

inline int elem_bytes(int dtype) { return dtype == 0 ? 4 : 2; }

}  // namespace

hipError_t launch_capture(const void* k_src, const void* v_src, int src_dtype, int64_t n_tok,
                          int64_t first_tok, const int32_t* table, void* k_pages, void* v_pages,
                          int page_dtype, int64_t n_phys, int hkv, int d, hipStream_t s) {
    if (n_tok == 0) return hipSuccess;
    if (src_dtype == page_dtype) {
        const int row_vecs = d * elem_bytes(src_dtype) / 16;
        const int64_t n = n_tok * hkv * row_vecs;
        KernelTimer kt("capture", s);
        capture_copy_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            (const uint4*)k_src, (const uint4*)v_src, n_tok, first_tok, table, (uint4*)k_pages,
            (uint4*)v_pages, n_phys, hkv, row_vecs);
    } else {  // f32 -> bf16
        const int64_t n = n_tok * hkv * (d / 8);
        KernelTimer kt("capture", s);
        capture_kernel<float, bf16_t><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            (const float*)k_src, (const float*)v_src, n_tok, first_tok, table,
            (bf16_t*)k_pages, (bf16_t*)v_pages, n_phys, hkv, d);
    }
    return hipGetLastError();
}

hipError_t launch_gather(const void* pages, int dtype, const int32_t* table, int64_t n_phys,
                         int64_t first_tok, int64_t n_tok, int hkv, int d, void* dst,
                         hipStream_t s) {
    if (n_tok == 0) return hipSuccess;
    const int row_vecs = d * elem_bytes(dtype) / 16;
    const int64_t n = n_tok * hkv * row_vecs;
    KernelTimer kt("gather", s);
    gather_copy_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
        (const uint4*)pages, table, n_phys, first_tok, n_tok, hkv, row_vecs, (uint4*)dst);
    return hipGetLastError();
}

}  // namespace ls
