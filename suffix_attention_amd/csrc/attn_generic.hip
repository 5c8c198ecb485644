// Replay attention on the vector ALUs: LDS-tiled kernels used for float32 inputs (the exact
// f32 path).  Three passes, each a plain tiling of the definition of softmax attention over
// the prompt pages plus the causal response keys:
//   forward   (query tile, part, kv head): online softmax over the part's keys, writing the
//             part's normalised output and LSE (one owner's local softmax statistics,
//             LongStraw digest "Method", Qwen implementation);
//   dK/dV     (key tile, kv head): loops over every query row that sees the tile and writes
//             that tile's gradient rows (one writer, no atomics);
//   dQ        (query tile, part, kv head): per-part dQ, summed afterwards.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int TR = 16;   // query rows per tile
constexpr int TK = 32;   // keys per tile (a page holds two)
constexpr int NT = 256;  // threads per block

template <typename T>
__device__ __forceinline__ const T* key_row(const AttnArgs& a, bool resp, int kvh, int64_t key,
                                            const void* pages, const void* resp_src) {
    if (!resp) {
        int32_t phys = a.table[key / kPage];
        phys = phys < 0 ? 0 : (phys >= a.n_phys ? (int32_t)(a.n_phys - 1) : phys);
        return (const T*)pages + (((int64_t)phys * a.hkv + kvh) * kPage + key % kPage) * a.d;
    }
    return (const T*)resp_src + (key * a.hkv + kvh) * a.d;
}

// Key range [lo, hi) of a part for a query tile whose largest token is tok_max.
__device__ __forceinline__ void part_keys(const AttnArgs& a, int part, int64_t tok_max, int64_t& lo,
                                          int64_t& hi) {
    if (part < a.n_shards) {
        lo = a.shard_lo[part] * kPage;
        hi = a.shard_lo[part + 1] * kPage;
        if (hi > a.prefix_len) hi = a.prefix_len;
        if (hi < lo) hi = lo;
    } else {
        lo = 0;
        hi = a.q_start + tok_max + 1;
        if (hi > a.key_end) hi = a.key_end;
    }
}

template <typename T, int D>
__global__ __launch_bounds__(NT) void fwd_generic_kernel(AttnArgs a) {
    constexpr int OC = D / 16;
    __shared__ float qs[TR][D];
    __shared__ float ks[TK][D + 1];
    __shared__ float vs[TK][D];
    __shared__ float ps[TR][TK + 1];
    __shared__ float m_s[TR], l_s[TR], al_s[TR];
    const int kvh = blockIdx.z, part = blockIdx.y, t = threadIdx.x;
    const bool resp = part == a.n_shards;
    const int64_t rows_total = a.n_rows * a.g;
    const int64_t r0 = (int64_t)blockIdx.x * TR;
    const T* Q = (const T*)a.q;
    for (int e = t; e < TR * D; e += NT) {
        const int rr = e / D, c = e % D;
        const int64_t r = r0 + rr;
        float v = 0.f;
        if (r < rows_total) v = load_f32<T>(Q + ((r / a.g) * a.hq + kvh * a.g + r % a.g) * D + c);
        qs[rr][c] = v;
    }
    if (t < TR) {
        m_s[t] = -INFINITY;
        l_s[t] = 0.f;
    }
    int64_t tok_max = (r0 + TR - 1) / a.g;
    if (tok_max > a.n_rows - 1) tok_max = a.n_rows - 1;
    int64_t k_lo, k_hi;
    part_keys(a, part, tok_max, k_lo, k_hi);
    const int orow = t / 16, oc0 = t % 16;
    float o[OC];
#pragma unroll
    for (int j = 0; j < OC; j++) o[j] = 0.f;
    __syncthreads();
    for (int64_t kb = k_lo; kb < k_hi; kb += TK) {
        for (int e = t; e < TK * D; e += NT) {
            const int kk = e / D, c = e % D;
            const int64_t key = kb + kk;
            float kx = 0.f, vx = 0.f;
            if (key < k_hi) {
                kx = load_f32<T>(key_row<T>(a, resp, kvh, key, a.k_pages, a.k_resp) + c);
                vx = load_f32<T>(key_row<T>(a, resp, kvh, key, a.v_pages, a.v_resp) + c);
            }
            ks[kk][c] = kx;
            vs[kk][c] = vx;
        }
        __syncthreads();
        for (int e = t; e < TR * TK; e += NT) {
            const int rr = e / TK, kk = e % TK;
            const int64_t key = kb + kk, r = r0 + rr;
            float s = 0.f;
            for (int c = 0; c < D; c++) s += qs[rr][c] * ks[kk][c];
            bool vis = key < k_hi;
            if (resp) vis = vis && key <= a.q_start + r / a.g;
            ps[rr][kk] = vis ? s * a.scale : -INFINITY;
        }
        __syncthreads();
        if (t < TR) {
            float mx = -INFINITY;
            for (int kk = 0; kk < TK; kk++) mx = fmaxf(mx, ps[t][kk]);
            const float m_old = m_s[t];
            const float m_new = fmaxf(m_old, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = expf(m_old - m_use);
            float sum = 0.f;
            for (int kk = 0; kk < TK; kk++) {
                const float p = expf(ps[t][kk] - m_use);
                ps[t][kk] = p;
                sum += p;
            }
            l_s[t] = l_s[t] * alpha + sum;
            m_s[t] = m_new;
            al_s[t] = alpha;
        }
        __syncthreads();
        const float al = al_s[orow];
#pragma unroll
        for (int j = 0; j < OC; j++) {
            const int c = oc0 + 16 * j;
            float acc = o[j] * al;
            for (int kk = 0; kk < TK; kk++) acc += ps[orow][kk] * vs[kk][c];
            o[j] = acc;
        }
        __syncthreads();
    }
    const int64_t r = r0 + orow;
    if (r < rows_total) {
        const int64_t tok = r / a.g;
        const int h = kvh * a.g + (int)(r % a.g);
        const float l = l_s[orow];
        const float inv = l != 0.f ? 1.f / l : 0.f;  // 0: no key seen; NaN inputs stay NaN
        const int64_t prow = (int64_t)part * a.part_rows + a.row0 + tok;
        float* dst = a.o_parts + (prow * a.hq + h) * D;
#pragma unroll
        for (int j = 0; j < OC; j++) dst[oc0 + 16 * j] = o[j] * inv;
        if (oc0 == 0) a.lse_parts[prow * a.hq + h] = l != 0.f ? m_s[orow] + logf(l) : -INFINITY;
    }
}

// dK/dV for one tile of TK keys (half a page, or response keys), over every row seeing it.
template <typename T, int D>
__global__ __launch_bounds__(NT) void dkdv_generic_kernel(AttnArgs a) {
    constexpr int KC = D / 8;
    __shared__ float ks[TK][D + 1];
    __shared__ float vs[TK][D + 1];
    __shared__ float qs[TR][D + 1];
    __shared__ float dos[TR][D + 1];
    __shared__ float ps[TR][TK + 1];
    __shared__ float dss[TR][TK + 1];
    __shared__ float lse_s[TR], dl_s[TR];
    const int kvh = blockIdx.y, t = threadIdx.x;
    const int64_t n_pt = a.n_logical_pages * (kPage / TK);
    const int64_t tile = blockIdx.x;
    const bool resp = tile >= n_pt;
    const int64_t key0 = (resp ? tile - n_pt : tile) * TK;
    const int64_t kend = resp ? a.key_end : a.prefix_len;
    const int64_t rows_total = a.n_rows * a.g;
    for (int e = t; e < TK * D; e += NT) {
        const int kk = e / D, c = e % D;
        const int64_t key = key0 + kk;
        float kx = 0.f, vx = 0.f;
        if (key < kend) {
            kx = load_f32<T>(key_row<T>(a, resp, kvh, key, a.k_pages, a.k_resp) + c);
            vx = load_f32<T>(key_row<T>(a, resp, kvh, key, a.v_pages, a.v_resp) + c);
        }
        ks[kk][c] = kx;
        vs[kk][c] = vx;
    }
    int64_t r_begin = 0;
    if (resp && key0 > a.q_start) r_begin = (key0 - a.q_start) * a.g;
    const T* Q = (const T*)a.q;
    const T* DO = (const T*)a.dout;
    float dk[KC], dv[KC];
#pragma unroll
    for (int j = 0; j < KC; j++) dk[j] = dv[j] = 0.f;
    const int mykey = t / 8, mc0 = t % 8;
    for (int64_t rb = r_begin; rb < rows_total; rb += TR) {
        __syncthreads();
        for (int e = t; e < TR * D; e += NT) {
            const int rr = e / D, c = e % D;
            const int64_t r = rb + rr;
            float qv = 0.f, dv_ = 0.f;
            if (r < rows_total) {
                const int64_t off = ((r / a.g) * a.hq + kvh * a.g + r % a.g) * D + c;
                qv = load_f32<T>(Q + off);
                dv_ = load_f32<T>(DO + off);
            }
            qs[rr][c] = qv;
            dos[rr][c] = dv_;
        }
        if (t < TR) {
            const int64_t r = rb + t;
            float l = 0.f, dl = 0.f;
            if (r < rows_total) {
                const int64_t off = (r / a.g) * a.hq + kvh * a.g + r % a.g;
                l = a.lse[off];
                dl = a.delta[off];
            }
            lse_s[t] = l;
            dl_s[t] = dl;
        }
        __syncthreads();
        for (int e = t; e < TR * TK; e += NT) {
            const int rr = e / TK, kk = e % TK;
            const int64_t r = rb + rr, key = key0 + kk;
            bool vis = r < rows_total && key < kend;
            if (resp) vis = vis && key <= a.q_start + r / a.g;
            float s = 0.f, dp = 0.f;
            for (int c = 0; c < D; c++) {
                s += qs[rr][c] * ks[kk][c];
                dp += dos[rr][c] * vs[kk][c];
            }
            const float p = vis ? expf(s * a.scale - lse_s[rr]) : 0.f;
            ps[rr][kk] = p;
            dss[rr][kk] = p * (dp - dl_s[rr]);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KC; j++) {
            const int c = mc0 + 8 * j;
            float av = dv[j], ak = dk[j];
            for (int rr = 0; rr < TR; rr++) {
                av += ps[rr][mykey] * dos[rr][c];
                ak += dss[rr][mykey] * qs[rr][c];
            }
            dv[j] = av;
            dk[j] = ak;
        }
    }
    const int64_t key = key0 + mykey;
    float *gk, *gv;
    bool first;
    if (!resp) {
        const int64_t lp = key / kPage;
        int32_t phys = a.table[lp];
        if (phys < 0 || phys >= a.n_phys) return;
        int s = 0;
        while (s + 1 < a.n_shards && lp >= a.shard_lo[s + 1]) s++;
        first = (a.first_touch_mask >> s) & 1ull;
        const int64_t off = (((int64_t)phys * a.hkv + kvh) * kPage + key % kPage) * D;
        gk = a.dk_pages + off;
        gv = a.dv_pages + off;
        if (key >= kend) {  // padding rows of a partial last page
            if (first)
                for (int j = 0; j < KC; j++) gk[mc0 + 8 * j] = gv[mc0 + 8 * j] = 0.f;
            return;
        }
    } else {
        if (key >= kend) return;
        first = a.resp_first_touch != 0;
        const int64_t off = (key * a.hkv + kvh) * D;
        gk = a.dk_resp + off;
        gv = a.dv_resp + off;
    }
#pragma unroll
    for (int j = 0; j < KC; j++) {
        const int c = mc0 + 8 * j;
        const float k_add = a.scale * dk[j];
        gk[c] = first ? k_add : gk[c] + k_add;
        gv[c] = first ? dv[j] : gv[c] + dv[j];
    }
}

template <typename T, int D>
__global__ __launch_bounds__(NT) void dq_generic_kernel(AttnArgs a) {
    constexpr int OC = D / 16;
    __shared__ float qs[TR][D + 1];
    __shared__ float dos[TR][D + 1];
    __shared__ float ks[TK][D + 1];
    __shared__ float vs[TK][D + 1];
    __shared__ float dss[TR][TK + 1];
    __shared__ float lse_s[TR], dl_s[TR];
    const int kvh = blockIdx.z, part = blockIdx.y, t = threadIdx.x;
    const bool resp = part == a.n_shards;
    const int64_t rows_total = a.n_rows * a.g;
    const int64_t r0 = (int64_t)blockIdx.x * TR;
    const T* Q = (const T*)a.q;
    const T* DO = (const T*)a.dout;
    for (int e = t; e < TR * D; e += NT) {
        const int rr = e / D, c = e % D;
        const int64_t r = r0 + rr;
        float qv = 0.f, dv_ = 0.f;
        if (r < rows_total) {
            const int64_t off = ((r / a.g) * a.hq + kvh * a.g + r % a.g) * D + c;
            qv = load_f32<T>(Q + off);
            dv_ = load_f32<T>(DO + off);
        }
        qs[rr][c] = qv;
        dos[rr][c] = dv_;
    }
    if (t < TR) {
        const int64_t r = r0 + t;
        float l = 0.f, dl = 0.f;
        if (r < rows_total) {
            const int64_t off = (r / a.g) * a.hq + kvh * a.g + r % a.g;
            l = a.lse[off];
            dl = a.delta[off];
        }
        lse_s[t] = l;
        dl_s[t] = dl;
    }
    int64_t tok_max = (r0 + TR - 1) / a.g;
    if (tok_max > a.n_rows - 1) tok_max = a.n_rows - 1;
    int64_t k_lo, k_hi;
    part_keys(a, part, tok_max, k_lo, k_hi);
    const int orow = t / 16, oc0 = t % 16;
    float acc[OC];
#pragma unroll
    for (int j = 0; j < OC; j++) acc[j] = 0.f;
    for (int64_t kb = k_lo; kb < k_hi; kb += TK) {
        __syncthreads();
        for (int e = t; e < TK * D; e += NT) {
            const int kk = e / D, c = e % D;
            const int64_t key = kb + kk;
            float kx = 0.f, vx = 0.f;
            if (key < k_hi) {
                kx = load_f32<T>(key_row<T>(a, resp, kvh, key, a.k_pages, a.k_resp) + c);
                vx = load_f32<T>(key_row<T>(a, resp, kvh, key, a.v_pages, a.v_resp) + c);
            }
            ks[kk][c] = kx;
            vs[kk][c] = vx;
        }
        __syncthreads();
        for (int e = t; e < TR * TK; e += NT) {
            const int rr = e / TK, kk = e % TK;
            const int64_t key = kb + kk, r = r0 + rr;
            bool vis = r < rows_total && key < k_hi;
            if (resp) vis = vis && key <= a.q_start + r / a.g;
            float s = 0.f, dp = 0.f;
            for (int c = 0; c < D; c++) {
                s += qs[rr][c] * ks[kk][c];
                dp += dos[rr][c] * vs[kk][c];
            }
            const float p = vis ? expf(s * a.scale - lse_s[rr]) : 0.f;
            dss[rr][kk] = p * (dp - dl_s[rr]);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < OC; j++) {
            const int c = oc0 + 16 * j;
            float x = acc[j];
            for (int kk = 0; kk < TK; kk++) x += dss[orow][kk] * ks[kk][c];
            acc[j] = x;
        }
    }
    const int64_t r = r0 + orow;
    if (r < rows_total) {
        const int64_t tok = r / a.g;
        const int h = kvh * a.g + (int)(r % a.g);
        float* dst = a.dq_parts + (((int64_t)part * a.n_rows + tok) * a.hq + h) * D;
#pragma unroll
        for (int j = 0; j < OC; j++) dst[oc0 + 16 * j] = a.scale * acc[j];
    }
}

template <typename T>
hipError_t fwd_dispatch(const AttnArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.n_rows * a.g + TR - 1) / TR), a.n_parts, a.hkv);
    if (a.n_rows == 0) return hipSuccess;
    KernelTimer kt("fwd_generic", s);
    switch (a.d) {
        case 64: fwd_generic_kernel<T, 64><<<grid, NT, 0, s>>>(a); break;
        case 128: fwd_generic_kernel<T, 128><<<grid, NT, 0, s>>>(a); break;
        case 256: fwd_generic_kernel<T, 256><<<grid, NT, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t bwd_dispatch(const AttnArgs& a, hipStream_t s) {
    const int64_t n_tiles = a.n_logical_pages * (kPage / TK) + (a.key_end + TK - 1) / TK;
    const dim3 g1((unsigned)n_tiles, a.hkv);
    const dim3 g2((unsigned)((a.n_rows * a.g + TR - 1) / TR), a.n_parts, a.hkv);
    const bool k_work = n_tiles > 0, q_work = a.n_rows > 0;
    switch (a.d) {
        case 64:
            if (k_work) { KernelTimer kt("dkdv_generic", s); dkdv_generic_kernel<T, 64><<<g1, NT, 0, s>>>(a); }
            if (q_work) { KernelTimer kt("dq_generic", s); dq_generic_kernel<T, 64><<<g2, NT, 0, s>>>(a); }
            break;
        case 128:
            if (k_work) { KernelTimer kt("dkdv_generic", s); dkdv_generic_kernel<T, 128><<<g1, NT, 0, s>>>(a); }
            if (q_work) { KernelTimer kt("dq_generic", s); dq_generic_kernel<T, 128><<<g2, NT, 0, s>>>(a); }
            break;
        case 256:
            if (k_work) { KernelTimer kt("dkdv_generic", s); dkdv_generic_kernel<T, 256><<<g1, NT, 0, s>>>(a); }
            if (q_work) { KernelTimer kt("dq_generic", s); dq_generic_kernel<T, 256><<<g2, NT, 0, s>>>(a); }
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_generic(const AttnArgs& a, hipStream_t s) { return fwd_dispatch<float>(a, s); }

hipError_t launch_bwd_generic(const AttnArgs& a, hipStream_t s) { return bwd_dispatch<float>(a, s); }

}  // namespace ls
