// Split-prefix replay-attention forward on gfx950 bf16 matrix cores.
//
// One workgroup handles BM = 32 * NW query rows of one kv head's group against the keys of
// one part: a prompt shard (a contiguous range of logical pages, walked through the page
// table) or the response keys the rows see (causal).  It writes the part's normalised
// output and LSE, the owner-local softmax statistics that the merge composes into the exact
// result (LongStraw digest, "Method", Qwen implementation; explainer, "Two incompatible
// architectures, same transaction").
//
// Per wave (32 rows), per 64-key page:
//   S^T[64 x 32] = K[64 x D] . Q^T        v_mfma_f32_32x32x16_bf16, K from LDS, Q in VGPRs
//   online softmax in base 2               each lane owns one row: in-lane max/sum, one
//                                          cross-half exchange (v_permlane32_swap)
//   O^T[D x 32] += V^T[D x 64] . P^T       V read transposed from LDS (ds_read_b64_tr_b16),
//                                          P^T taken straight from the S^T accumulators
// Keys are permuted inside each 16-key MFMA step so that P^T needs no data movement: the
// order is the same on both operands, so the sum is unchanged.
//
// K/V pages (64 x D bf16 each, one contiguous tile per (page, kv head)) are copied into a
// double-buffered LDS stage by direct global->LDS loads, issued one page ahead.  A 16-byte
// chunk c of LDS row r holds logical chunk c ^ (r & 15) to spread rows over the banks.
#include <math.h>

#include "mfma_tiles.hpp"

namespace ls {
namespace {

template <int D>
struct WaveState {
    bf16x8 qb[TileShape<D>::KS];   // Q^T operand: row lane%32, d = 16ks + 8(lane/32) .. +8
    f32x16 o[TileShape<D>::DT];    // O^T accumulators: col = row, rows = d
    float m;                      // running max (base-2 scaled scores)
    float l;                      // running sum of this lane's half of the keys
};

template <int D>
__device__ __forceinline__ void compute_tile(WaveState<D>& ws, const LS_LDS char* lds_k,
                                             const LS_LDS char* lds_v, LaneAddr<D> la,
                                             const TileSrc& src, bool resp, bool need_mask,
                                             int64_t vis_limit, float scale_log2, int lane) {
    using F = TileShape<D>;
    const int h = lane >> 5;
    // keep the per-lane offsets from being hoisted out of the page loop as many registers
    asm volatile("" : "+v"(la.k), "+v"(la.v));
    // ---- S^T = K Q^T for the two 32-key halves of the page
    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
    // LDS operands are read PD k-steps ahead of the MFMAs that use them; each sched_barrier
    // keeps that order.
    constexpr int PD = 3;
    bf16x8 kbuf[PD][2];
#pragma unroll
    for (int j = 0; j < PD; j++) {
        const LS_LDS char* pk = lds_k + (la.k ^ (uint32_t)(j << 5));
        kbuf[j][0] = *(const LS_LDS bf16x8*)(pk);
        kbuf[j][1] = *(const LS_LDS bf16x8*)(pk + 32 * 2 * D);
    }
#pragma unroll
    for (int ks = 0; ks < F::KS; ks++) {
        const bf16x8 k0 = kbuf[ks % PD][0], k1 = kbuf[ks % PD][1];
        if (ks + PD < F::KS) {
            const LS_LDS char* pk = lds_k + (la.k ^ (uint32_t)((ks + PD) << 5));
            kbuf[ks % PD][0] = *(const LS_LDS bf16x8*)(pk);
            kbuf[ks % PD][1] = *(const LS_LDS bf16x8*)(pk + 32 * 2 * D);
        }
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, ws.qb[ks], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, ws.qb[ks], s[1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    // ---- mask and running max on the raw scores (scale_log2 > 0 commutes with max).
    // Element i of tile kt is key 32kt + 8(i/4) + 4h + i%4 of the page; the mask compares
    // its lane-free part with two per-lane limits.
    if (need_mask) {
        const int lim_valid = src.valid - 4 * h;  // keys < valid exist
        int lim_causal = 64;                      // response keys <= vis_limit are visible
        if (resp) {
            const int64_t c = vis_limit - src.key0 - 4 * h;
            lim_causal = c < -1 ? -1 : (c > 64 ? 64 : (int)c);
        }
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int kc = 32 * kt + 8 * (i >> 2) + (i & 3);
                s[kt][i] = (kc < lim_valid && kc <= lim_causal) ? s[kt][i] : -INFINITY;
            }
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[kt][i], s[kt][i + 1]));
    }
    mx = fmaxf(mx, other_half(mx)) * scale_log2;
    const float m_new = fmaxf(ws.m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(ws.m - m_use);
    ws.m = m_new;
    // ---- P = exp2(S * scale_log2 - m), packed to bf16 as the P^T operand
    bf16x8 pb[2][2];
    float lsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
            uint32_t w4[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const float p0 = fast_exp2(__builtin_fmaf(s[kt][8 * u + 2 * t], scale_log2, -m_use));
                const float p1 = fast_exp2(__builtin_fmaf(s[kt][8 * u + 2 * t + 1], scale_log2, -m_use));
                lsum += p0 + p1;
                w4[t] = pack_bf16x2(p0, p1);
            }
            pb[kt][u] = __builtin_bit_cast(bf16x8, (u32x4{w4[0], w4[1], w4[2], w4[3]}));
        }
    }
    ws.l = ws.l * alpha + lsum;
    if (!__all(alpha == 1.f)) {
#pragma unroll
        for (int dt = 0; dt < F::DT; dt++) ws.o[dt] *= alpha;
    }
    // ---- O^T += V^T P^T.  Step st = (kt, u, dt) with dt fastest, so consecutive MFMAs
    // accumulate into different tiles; V^T fragments (rows 32kt + 16u + 8e) are read PV
    // steps ahead.
    constexpr int NST = 4 * F::DT;
    constexpr int PV = 4;
    i16x4 vlo[PV], vhi[PV];
    auto read_v = [&](int st, i16x4& lo, i16x4& hi) {
        const int dt = st % F::DT, ku = st / F::DT;
        const int R = 32 * (ku >> 1) + 16 * (ku & 1);
        lo = lds_read_tr4(lds_v + (la.v ^ tr_x<D>(dt, R)) + R * 2 * D);
        hi = lds_read_tr4(lds_v + (la.v ^ tr_x<D>(dt, R + 8)) + (R + 8) * 2 * D);
    };
#pragma unroll
    for (int j = 0; j < PV; j++) read_v(j, vlo[j], vhi[j]);
#pragma unroll
    for (int st = 0; st < NST; st++) {
        const int dt = st % F::DT, ku = st / F::DT;
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[st % PV], vhi[st % PV], 0, 1, 2, 3, 4, 5, 6, 7));
        if (st + PV < NST) read_v(st + PV, vlo[st % PV], vhi[st % PV]);
        ws.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ku >> 1][ku & 1], ws.o[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One pipeline step: start copying the next page into the other LDS stage, then compute on
// the current one.  The stages are passed as restrict pointers so that, once inlined, the
// compiler knows the copies cannot alias the reads and does not wait for them.
template <int D, int NW>
__device__ __forceinline__ void fwd_step(WaveState<D>& ws, const char* __restrict__ cur,
                                         char* __restrict__ nxt, bool has_next,
                                         const TileSrc& next_src, const TileSrc& src,
                                         LaneAddr<D> la, bool resp, bool need_mask,
                                         int64_t vis_limit, float scale_log2, int w, int lane) {
    using F = TileShape<D>;
    if (has_next) issue_tile<D, NW>(next_src, nxt, nxt + F::TILE, w, lane);
    compute_tile<D>(ws, (const LS_LDS char*)cur, (const LS_LDS char*)(cur + F::TILE), la, src, resp,
                    need_mask, vis_limit, scale_log2, lane);
}

template <int D, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(1, 1)))
void fwd_mfma_kernel(AttnArgs a, int n_qtiles, int n_blocks) {
    using F = TileShape<D>;
    constexpr int BM = 32 * NW;
    __shared__ __attribute__((aligned(1024))) char st0[2 * F::TILE];
    __shared__ __attribute__((aligned(1024))) char st1[2 * F::TILE];

    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    if (lb >= n_blocks) return;
    const int qtile = lb % n_qtiles;
    const int part = (lb / n_qtiles) % a.n_parts;
    const int kvh = lb / (n_qtiles * a.n_parts);
    const bool resp = part == a.n_shards;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int n = lane & 31;
    const int64_t rows_total = a.n_rows * a.g;
    const int64_t r0 = (int64_t)qtile * BM;
    const int64_t my_row = r0 + 32 * w + n;
    const bool row_ok = my_row < rows_total;
    const int64_t my_tok = my_row / a.g;
    const int my_head = kvh * a.g + (int)(my_row % a.g);

    WaveState<D> ws;
    {
        // rows past the block (a partial last tile) read a valid row and are never stored
        const int64_t ld_row = row_ok ? my_row : rows_total - 1;
        const int64_t ld_tok = ld_row / a.g;
        const int ld_head = kvh * a.g + (int)(ld_row % a.g);
        const bf16_t* qrow = (const bf16_t*)a.q + (ld_tok * a.hq + ld_head) * (int64_t)D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < F::KS; ks++) {
            ws.qb[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * ks));
            asm volatile("" : "+a"(ws.qb[ks]));  // read-only MFMA operand: keep it in AGPRs
        }
#pragma unroll
        for (int dt = 0; dt < F::DT; dt++) ws.o[dt] = f32x16{};
        ws.m = -INFINITY;
        ws.l = 0.f;
    }
    const LaneAddr<D> la(lane);

    // number of key tiles of this part for this query tile
    int64_t n_tiles;
    const int64_t tok_min = r0 / a.g;
    if (!resp) {
        n_tiles = a.shard_lo[part + 1] - a.shard_lo[part];
    } else {
        int64_t tok_max = (r0 + BM - 1) / a.g;
        if (tok_max > a.n_rows - 1) tok_max = a.n_rows - 1;
        n_tiles = (a.q_start + tok_max + 1 + kPage - 1) / kPage;
    }
    const int64_t vis_limit = a.q_start + my_tok;  // last response key this row sees
    // Page-table entries are read one tile ahead of their copy, so the lookup latency hides
    // behind the current tile's compute.
    int32_t phys_cur = (!resp && n_tiles > 0) ? phys_page(a, part, 0) : 0;
    int32_t phys_next = (!resp && n_tiles > 1) ? phys_page(a, part, 1) : 0;
    TileSrc src = part_tile(a, resp, part, kvh, 0, __builtin_amdgcn_readfirstlane(phys_cur));
    if (n_tiles > 0) issue_tile<D, NW>(src, st0, st0 + F::TILE, w, lane);
    for (int64_t t = 0; t < n_tiles; t++) {
        wait_vm_all();
        __syncthreads();
        const bool has_next = t + 1 < n_tiles;
        const TileSrc next_src =
            part_tile(a, resp, part, kvh, has_next ? t + 1 : t, __builtin_amdgcn_readfirstlane(phys_next));
        if (!resp && t + 2 < n_tiles) phys_next = phys_page(a, part, t + 2);
        const bool need_mask = src.valid < kPage || (resp && src.key0 + kPage - 1 > a.q_start + tok_min);
        char* cur = (t & 1) ? st1 : st0;
        char* nxt = (t & 1) ? st0 : st1;
        fwd_step<D, NW>(ws, cur, nxt, has_next, next_src, src, la, resp, need_mask, vis_limit, a.scale_log2, w,
                        lane);
        src = next_src;
    }

    // ---- normalise and write this part's output and LSE
    const float l = ws.l + other_half(ws.l);
    if (!row_ok) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst = a.o_parts + (((int64_t)part * a.n_rows + my_tok) * a.hq + my_head) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < F::DT; dt++) {
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
            const int dd = dt * 32 + 8 * q4 + 4 * h;
            float4 v = make_float4(ws.o[dt][4 * q4] * inv, ws.o[dt][4 * q4 + 1] * inv,
                                   ws.o[dt][4 * q4 + 2] * inv, ws.o[dt][4 * q4 + 3] * inv);
            *(float4*)(dst + dd) = v;
        }
    }
    if (h == 0)
        a.lse_parts[((int64_t)part * a.n_rows + my_tok) * a.hq + my_head] =
            l > 0.f ? (ws.m + fast_log2(l)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
    constexpr int NW = 4;
    constexpr int BM = 32 * NW;
    const int64_t n_qtiles = (a.n_rows * a.g + BM - 1) / BM;
    const int64_t n_blocks = n_qtiles * a.n_parts * a.hkv;
    if (n_blocks == 0) return hipSuccess;
    const int grid = pad_grid((int)n_blocks);
    KernelTimer kt("fwd_mfma", s);
    fwd_mfma_kernel<D, NW><<<grid, NW * 64, 0, s>>>(a, (int)n_qtiles, (int)n_blocks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t s) {
    switch (a.d) {
        case 64: return launch_d<64>(a, s);
        case 128: return launch_d<128>(a, s);
        case 256: return launch_d<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ls
