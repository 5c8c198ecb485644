// dQ pass of the replay-attention backward on gfx950 bf16 matrix cores.
//
// (query tile, part, kv head), like the forward: per 64-key page, S^T = K Q^T and
// dP^T = V dO^T (Q, dO in AGPRs as the B operands, K, V from LDS), dS^T = P^T (dP^T - delta)
// with P recomputed from the forward's LSE, dQ^T += K^T dS^T (K read transposed).  Writes
// one dQ part per key part; the parts are summed afterwards.  Built with its accumulators in
// VGPRs: the S and dP tiles feed vector-ALU work every page.
#include <math.h>

#include "mfma_bwd.hpp"

namespace ls {
namespace {

// ---------------------------------------------------------------------------------------
// dQ pass
// ---------------------------------------------------------------------------------------
template <int D>
struct DqState {
    bf16x8 qb[TileShape<D>::KS];    // Q^T operand (row lane%32)
    bf16x8 dob[TileShape<D>::KS];   // dO^T operand
    f32x16 dq[TileShape<D>::DT];    // dQ^T accumulators: col = row, rows = d
    float lse2;                     // LSE * log2 e of this lane's row
    float dlt;                      // delta of this lane's row
};

template <int D>
__device__ __forceinline__ void dq_tile(DqState<D>& st, const LS_LDS char* lds_k, const LS_LDS char* lds_v,
                                        LaneAddr<D> la, int valid, int64_t key0, bool resp, bool need_mask,
                                        int64_t vis_limit, float scale_log2, int lane) {
    using F = TileShape<D>;
    const int h = lane >> 5;
    asm volatile("" : "+v"(la.k), "+v"(la.v));
    f32x16 s[2], dp[2];
    s[0] = s[1] = dp[0] = dp[1] = f32x16{};
    // K and V fragments are read PD k-steps ahead of their MFMAs
    constexpr int PD = 2;
    bf16x8 kb[PD][4];
    auto read_kv = [&](int ks, bf16x8* b) {
        const uint32_t o = la.k ^ (uint32_t)(ks << 5);
        b[0] = *(const LS_LDS bf16x8*)(lds_k + o);
        b[1] = *(const LS_LDS bf16x8*)(lds_k + o + 32 * 2 * D);
        b[2] = *(const LS_LDS bf16x8*)(lds_v + o);
        b[3] = *(const LS_LDS bf16x8*)(lds_v + o + 32 * 2 * D);
    };
#pragma unroll
    for (int j = 0; j < PD; j++) read_kv(j, kb[j]);
#pragma unroll
    for (int ks = 0; ks < F::KS; ks++) {
        const bf16x8 k0 = kb[ks % PD][0], k1 = kb[ks % PD][1], v0 = kb[ks % PD][2], v1 = kb[ks % PD][3];
        if (ks + PD < F::KS) read_kv(ks + PD, kb[ks % PD]);
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, st.qb[ks], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, st.qb[ks], s[1], 0, 0, 0);
        dp[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, st.dob[ks], dp[0], 0, 0, 0);
        dp[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, st.dob[ks], dp[1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    int lim_valid = valid - 4 * h;
    int lim_causal = 64;
    if (resp) {
        const int64_t c = vis_limit - key0 - 4 * h;
        lim_causal = c < -1 ? -1 : (c > 64 ? 64 : (int)c);
    }
    bf16x8 db[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
            uint32_t w4[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                float d2[2];
#pragma unroll
                for (int e = 0; e < 2; e++) {
                    const int i = 8 * u + 2 * t + e;
                    float p = fast_exp2(__builtin_fmaf(s[kt][i], scale_log2, -st.lse2));
                    if (need_mask) {
                        const int kc = 32 * kt + 8 * (i >> 2) + (i & 3);
                        p = (kc < lim_valid && kc <= lim_causal) ? p : 0.f;
                    }
                    d2[e] = p * (dp[kt][i] - st.dlt);
                }
                w4[t] = pack_bf16x2(d2[0], d2[1]);
            }
            db[kt][u] = __builtin_bit_cast(bf16x8, (u32x4{w4[0], w4[1], w4[2], w4[3]}));
        }
    }
    // dQ^T += K^T dS^T.  Step st = (kt, u, dt), dt fastest; K^T fragments read PV steps ahead.
    constexpr int NST = 4 * F::DT;
    constexpr int PV = 4;
    i16x4 tlo[PV], thi[PV];
    auto read_kt = [&](int st_, i16x4& lo, i16x4& hi) {
        const int dt = st_ % F::DT, ku = st_ / F::DT;
        const int R = 32 * (ku >> 1) + 16 * (ku & 1);
        lo = lds_read_tr4(lds_k + (la.v ^ tr_x<D>(dt, R)) + R * 2 * D);
        hi = lds_read_tr4(lds_k + (la.v ^ tr_x<D>(dt, R + 8)) + (R + 8) * 2 * D);
    };
#pragma unroll
    for (int j = 0; j < PV; j++) read_kt(j, tlo[j], thi[j]);
#pragma unroll
    for (int st_ = 0; st_ < NST; st_++) {
        const int dt = st_ % F::DT, ku = st_ / F::DT;
        const bf16x8 ka = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tlo[st_ % PV], thi[st_ % PV], 0, 1, 2, 3, 4, 5, 6, 7));
        if (st_ + PV < NST) read_kt(st_ + PV, tlo[st_ % PV], thi[st_ % PV]);
        st.dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, db[ku >> 1][ku & 1], st.dq[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One page: issue the copies of page t+1 (K and V into nxt), then the tile on cur.  The two
// stages are restrict pointers so that, once inlined, the compiler knows the copies in flight
// cannot alias the tile being read and does not wait for them.
template <int D, int NW>
__device__ __forceinline__ void dq_step(DqState<D>& st, const char* __restrict__ cur, char* __restrict__ nxt,
                                        const KeyTiles<D, NW>& kt, bool has_next, int32_t e_next, int64_t t,
                                        int valid, int64_t key0, LaneAddr<D> la, bool resp, bool need_mask,
                                        int64_t vis_limit, float scale_log2, int w, int lane) {
    using F = TileShape<D>;
    if (has_next) {
        const int vn = kt.valid(t + 1);
        kt.copy(kt.tile(e_next, t + 1, false), vn, nxt, w);
        kt.copy(kt.tile(e_next, t + 1, true), vn, nxt + F::TILE, w);
    }
    dq_tile<D>(st, (const LS_LDS char*)cur, (const LS_LDS char*)(cur + F::TILE), la, valid, key0, resp, need_mask,
               vis_limit, scale_log2, lane);
}

template <int D, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(1, 1)))
void dq_mfma_kernel(AttnArgs a, GroupRows gr, int n_qtiles, int n_blocks) {
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

    DqState<D> st;
    {
        const int64_t ld_row = row_ok ? my_row : rows_total - 1;
        const int64_t th = (ld_row / a.g) * a.hq + kvh * a.g + ld_row % a.g;
        const bf16_t* qrow = (const bf16_t*)a.q + th * (int64_t)D + 8 * h;
        const bf16_t* drow = (const bf16_t*)a.dout + th * (int64_t)D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < F::KS; ks++) {
            st.qb[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * ks));
            st.dob[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(drow + 16 * ks));
            asm volatile("" : "+a"(st.qb[ks]), "+a"(st.dob[ks]));  // read-only MFMA operands
        }
#pragma unroll
        for (int dt = 0; dt < F::DT; dt++) st.dq[dt] = f32x16{};
        const f32x2 ld = gr.lsed[kvh * gr.rows_pad + (row_ok ? my_row : rows_total - 1)];
        st.lse2 = ld[0];
        st.dlt = ld[1];
    }
    const LaneAddr<D> la(lane);
    int64_t n_tiles;
    const int64_t tok_min = r0 / a.g;
    if (!resp) {
        n_tiles = a.shard_lo[part + 1] - a.shard_lo[part];
    } else {
        int64_t tok_max = (r0 + BM - 1) / a.g;
        if (tok_max > a.n_rows - 1) tok_max = a.n_rows - 1;
        n_tiles = (a.q_start + tok_max + 1 + kPage - 1) / kPage;
    }
    const int64_t vis_limit = a.q_start + my_tok;

    const int64_t lp0 = resp ? 0 : a.shard_lo[part];
    const KeyTiles<D, NW> kt(a, resp, lp0, kvh, w, lane);
    // page-table entries are read through the scalar cache one page before their copies and
    // clamped where they are used
    int32_t e_next = n_tiles > 1 ? kt.entry(1) : 0;
    if (n_tiles > 0) {
        const int32_t e0 = kt.entry(0);
        kt.copy(kt.tile(e0, 0, false), kt.valid(0), st0, w);
        kt.copy(kt.tile(e0, 0, true), kt.valid(0), st0 + F::TILE, w);
    }
    for (int64_t t = 0; t < n_tiles; t++) {
        const int32_t e_after = t + 2 < n_tiles ? kt.entry(t + 2) : 0;
        wait_vm_all();
        __syncthreads();
        const int valid = kt.valid(t);
        const int64_t key0 = (lp0 + t) * kPage;
        const bool need_mask = valid < kPage || (resp && key0 + kPage - 1 > a.q_start + tok_min);
        char* cur = (t & 1) ? st1 : st0;
        char* nxt = (t & 1) ? st0 : st1;
        dq_step<D, NW>(st, cur, nxt, kt, t + 1 < n_tiles, e_next, t, valid, key0, la, resp, need_mask, vis_limit,
                       a.scale_log2, w, lane);
        e_next = e_after;
    }
    if (!row_ok) return;
    float* dst = a.dq_parts + (((int64_t)part * a.n_rows + my_tok) * a.hq + my_head) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < F::DT; dt++) {
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
            const int dd = dt * 32 + 8 * q4 + 4 * h;
            *(float4*)(dst + dd) = make_float4(a.scale * st.dq[dt][4 * q4], a.scale * st.dq[dt][4 * q4 + 1],
                                               a.scale * st.dq[dt][4 * q4 + 2], a.scale * st.dq[dt][4 * q4 + 3]);
        }
    }
}

}  // namespace

hipError_t launch_dq_mfma(const AttnArgs& a, const GroupRows& gr, hipStream_t s) {
    constexpr int NW = 4;
    constexpr int BM = 32 * NW;
    const int64_t rows_total = a.n_rows * a.g;
    const int64_t n_qtiles = (rows_total + BM - 1) / BM;
    const int64_t nb_q = n_qtiles * a.n_parts * a.hkv;
    if (nb_q == 0) return hipSuccess;
    KernelTimer kt("dq_mfma", s);
    switch (a.d) {
        case 64: dq_mfma_kernel<64, NW><<<pad_grid((int)nb_q), NW * 64, 0, s>>>(a, gr, (int)n_qtiles, (int)nb_q); break;
        case 128: dq_mfma_kernel<128, NW><<<pad_grid((int)nb_q), NW * 64, 0, s>>>(a, gr, (int)n_qtiles, (int)nb_q); break;
        case 256: dq_mfma_kernel<256, NW><<<pad_grid((int)nb_q), NW * 64, 0, s>>>(a, gr, (int)n_qtiles, (int)nb_q); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ls
