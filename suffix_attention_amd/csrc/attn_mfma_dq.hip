// dQ pass of the replay-attention backward on gfx950 bf16 matrix cores.
//
// (query tile, part, kv head), like the forward: per 64-key page, S^T = K Q^T and
// dP^T = V dO^T (Q, dO in AGPRs as the B operands, K, V from LDS), dS^T = P^T (dP^T - delta)
// with P recomputed from the forward's LSE, dQ^T += K^T dS^T (K read transposed).  Writes
// one dQ part per key part; the parts are summed afterwards.
//
// Software pipeline over pages, so that the vector work (P and dS) of one tile runs between the
// matrix instructions of another: iteration t computes S and dP of page t+1 and accumulates dQ
// for page t, with dS of page t's second key tile and page t+1's first formed beside them.  That
// needs K of three pages (t for dQ, t+1 for S, t+2 in flight) and V of two in LDS: 5 x 32 KiB
// at d = 256.  Built with VGPR-form matrix
// instructions (the S and dP tiles feed vector-ALU work); the dQ accumulators stay in AGPRs
// through explicit AGPR-form instructions.
#include <math.h>

#include "mfma_bwd.hpp"

namespace ls {
namespace {

template <int D>
struct DqState {
    bf16x8 qb[TileShape<D>::KS];    // Q^T operand (row lane%32)
    bf16x8 dob[TileShape<D>::KS];   // dO^T operand
    f32x16 dq[TileShape<D>::DT];    // dQ^T accumulators (AGPRs): col = row, rows = d
    float lse2;                     // LSE * log2 e of this lane's row
    float dlt;                      // delta of this lane's row
};

// Phase 1 of one 32-key tile of a page: S^T = K Q^T and dP^T = V dO^T (ak, av: LDS address of
// the tile's first key row in the K and V buffers plus the lane's natural-read offset), 16
// k-steps of two matrix instructions; K and V fragments are read PD steps ahead.  beside(ks)
// runs after step ks's matrix instructions: vector work or copies that overlap them.
template <int D, typename Beside>
__device__ __forceinline__ void tile_scores(const DqState<D>& st, uint32_t ak, uint32_t av, f32x16& s, f32x16& dp,
                                            Beside&& beside) {
    using F = TileShape<D>;
    s = dp = f32x16{};
    constexpr int PD = 3;
    bf16x8 kb[PD][2];
    auto read_kv = [&](int ks, bf16x8* b) {
        b[0] = lds_b128(ak ^ (uint32_t)(ks << 5));
        b[1] = lds_b128(av ^ (uint32_t)(ks << 5));
    };
#pragma unroll
    for (int j = 0; j < PD; j++)
        if (j < F::KS) read_kv(j, kb[j]);
#pragma unroll
    for (int ks = 0; ks < F::KS; ks++) {
        const bf16x8 k0 = kb[ks % PD][0], v0 = kb[ks % PD][1];
        if (ks + PD < F::KS) read_kv(ks + PD, kb[ks % PD]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, st.qb[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, st.dob[ks], dp, 0, 0, 0);
        beside(ks);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Masking limit of one page for this lane's row: element i of key tile kt is key
// 32kt + 8(i/4) + 4h + i%4 of the page, and gets P = 0 unless that key is below the page's
// valid keys and, for response keys, at most the row's own position.  Both conditions fold into
// one bound on 32kt + 8(i/4) + i%4 (the lane's 4h is taken out of it).
struct PageMask {
    int lim;
};

__device__ __forceinline__ PageMask page_mask(int valid, int64_t key0, bool resp, int64_t vis_limit, int h) {
    PageMask m;
    m.lim = valid - 4 * h;
    if (resp) {
        const int64_t c = vis_limit - key0 - 4 * h + 1;
        const int lc = c < 0 ? 0 : (c > 65 ? 65 : (int)c);
        m.lim = lc < m.lim ? lc : m.lim;
    }
    return m;
}

// Phase 2, one unit (u, t) of two elements of key tile kt: P = exp2(S scale log2e - LSE log2e),
// dS = P (dP - delta), packed as word t of the bf16 dS^T operand of key step 2kt + u.  Units are
// small so that they fit between consecutive matrix instructions; the masked form is only
// instantiated for pages that need it.
template <bool MASK, int D>
__device__ __forceinline__ void ds_unit(int unit, int kt, const f32x16& s, const f32x16& dp, int lim,
                                        const DqState<D>& st, float scale_log2, u32x4 (&out)[4]) {
    const int u = unit >> 2, t = unit & 3;
    float d2[2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
        const int i = 8 * u + 2 * t + e;
        float p = fast_exp2(__builtin_fmaf(s[i], scale_log2, -st.lse2));
        if (MASK) p = (32 * kt + 8 * (i >> 2) + (i & 3)) < lim ? p : 0.f;
        d2[e] = p * (dp[i] - st.dlt);
    }
    uint32_t word = pack_bf16x2(d2[0], d2[1]);
    // pinned here: otherwise the compiler sinks the unit past the branches of the copies that
    // share its stretch, next to its use, where no matrix work is left to hide it
    asm volatile("" : "+v"(word));
    out[2 * kt + u][t] = word;
}

// Phase 3 of page t: dQ^T += K^T dS^T (K read transposed; sv: LDS address of page t's K tile
// plus the lane's transposed-read offset).  Step st = (ku, dt), dt fastest; K^T fragments read
// PV steps ahead; beside(st) runs after each step's matrix instruction.
template <int D, typename Beside>
__device__ __forceinline__ void page_accumulate(DqState<D>& st, const u32x4 (&ds)[4], uint32_t sv, Beside&& beside) {
    using F = TileShape<D>;
    bf16x8 db[4];
#pragma unroll
    for (int ku = 0; ku < 4; ku++) db[ku] = __builtin_bit_cast(bf16x8, ds[ku]);
    constexpr int NST = 4 * F::DT;
    constexpr int PV = 4;
    i16x4 tlo[PV], thi[PV];
    auto read_kt = [&](int st_, i16x4& lo, i16x4& hi) {
        const int dt = st_ % F::DT, ku = st_ / F::DT;
        const int R = 32 * (ku >> 1) + 16 * (ku & 1);
        lo = lds_tr4((sv ^ tr_x<D>(dt, R)) + R * 2 * D);
        hi = lds_tr4((sv ^ tr_x<D>(dt, R + 8)) + (R + 8) * 2 * D);
    };
#pragma unroll
    for (int j = 0; j < PV; j++) read_kt(j, tlo[j], thi[j]);
    // two steps (dt, dt + 1 of one key step) per matrix-instruction pair
#pragma unroll
    for (int st_ = 0; st_ < NST; st_ += 2) {
        const int dt = st_ % F::DT, ku = st_ / F::DT;
        const bf16x8 ka0 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tlo[st_ % PV], thi[st_ % PV], 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 ka1 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tlo[(st_ + 1) % PV], thi[(st_ + 1) % PV], 0, 1, 2, 3, 4, 5, 6, 7));
        if (st_ + PV < NST) read_kt(st_ + PV, tlo[st_ % PV], thi[st_ % PV]);
        if (st_ + 1 + PV < NST) read_kt(st_ + 1 + PV, tlo[(st_ + 1) % PV], thi[(st_ + 1) % PV]);
        mfma32_agpr2(st.dq[dt], ka0, db[ku], st.dq[dt + 1], ka1, db[ku]);
        beside(st_);
        beside(st_ + 1);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Run the units [n * k / steps, n * (k + 1) / steps) of n at step k, with constant loop bounds so
// that every unit index is a constant after unrolling.
template <int N, int STEPS, typename F>
__device__ __forceinline__ void units_at(int k, F&& f) {
#pragma unroll
    for (int un = 0; un < N; un++)
        if (un >= k * N / STEPS && un < (k + 1) * N / STEPS) f(un);
}

// Iteration t, three stretches of matrix work, each with vector work beside it:
//   1. S, dP of key tile 0 of page t+1, beside dS of key tile 1 of page t and the copies of
//      page t+2;
//   2. dQ += K^T dS^T of page t, beside dS of key tile 0 of page t+1;
//   3. S, dP of key tile 1 of page t+1.
// ds holds page t's dS operand words (key tile 0 on entry, both on leaving stretch 1) and page
// t+1's key tile 0 on return; s1, dp1 hold key tile 1 of page t on entry and of page t+1 on
// return.  The LDS tiles are restrict pointers so that, once inlined, the compiler knows the
// copies in flight cannot alias the tiles being read.
template <bool MASK, int D, int NW>
__device__ __forceinline__ void dq_iter(DqState<D>& st, const KeyTiles<D, NW>& kt, int64_t t, int64_t last, bool copy,
                                        int32_t e2,
                                        uint32_t k_dst, uint32_t v_dst, uint32_t k_n, uint32_t v_n, uint32_t k_t,
                                        u32x4 (&ds)[4], f32x16& s1, f32x16& dp1,
                                        int lim_t, int lim_n, LaneAddr<D> la, float scale_log2, int w) {
    constexpr int PW = KeyTiles<D, NW>::PER_WAVE;
    constexpr int KS = TileShape<D>::KS;
    constexpr int NST = 4 * TileShape<D>::DT;
    // Near the end there is no page t+2: the last page is copied again instead, into buffers
    // that nothing reads, so that the stretch has no branch (a branch would let the compiler
    // move the vector work out of it)
    const int64_t tc = copy ? t + 2 : last;
    const int vn = kt.valid(tc);
    const char* ksrc = kt.tile(e2, tc, false);
    const char* vsrc = kt.tile(e2, tc, true);
    uint32_t lk = la.k, lv = la.v;
    asm volatile("" : "+v"(lk), "+v"(lv));
    f32x16 s0, dp0;
    tile_scores<D>(st, k_n + lk, v_n + lk, s0, dp0, [&](int ks) {
        units_at<8, KS>(ks, [&](int un) { ds_unit<MASK>(un, 1, s1, dp1, lim_t, st, scale_log2, ds); });
        units_at<2 * PW, KS>(ks, [&](int p) {
                if (p < PW) kt.copy_piece(ksrc, vn, k_dst, w, p);
                else kt.copy_piece(vsrc, vn, v_dst, w, p - PW);
            });
    });
    u32x4 nxt[4];
    page_accumulate<D>(st, ds, k_t + lv, [&](int k) {
        units_at<8, NST>(k, [&](int un) { ds_unit<MASK>(un, 0, s0, dp0, lim_n, st, scale_log2, nxt); });
    });
    tile_scores<D>(st, k_n + lk + 32 * 2 * D, v_n + lk + 32 * 2 * D, s1, dp1, [](int) {});
    ds[0] = nxt[0];
    ds[1] = nxt[1];
}

// Every page of the part through the pipeline, with or without the per-element mask.
template <bool MASK, int D, int NW, typename MaskOf>
__device__ __forceinline__ void dq_pages(DqState<D>& st, const KeyTiles<D, NW>& kt, int64_t n_tiles, MaskOf&& mask_of,
                                         uint32_t kb0, uint32_t vb0, LaneAddr<D> la, float scale_log2, int w) {
    using F = TileShape<D>;
    // prologue: pages 0 and 1 in LDS; S, dP of page 0 and dS of its key tile 0
    const int32_t e0 = kt.entry(0);
    kt.copy(kt.tile(e0, 0, false), kt.valid(0), kb0, w);
    kt.copy(kt.tile(e0, 0, true), kt.valid(0), vb0, w);
    if (n_tiles > 1) {
        const int32_t e1 = kt.entry(1);
        kt.copy(kt.tile(e1, 1, false), kt.valid(1), kb0 + F::TILE, w);
        kt.copy(kt.tile(e1, 1, true), kt.valid(1), vb0 + F::TILE, w);
    }
    // page-table entries are read through the scalar cache one iteration before their
    // copies and clamped where they are used
    int32_t e2 = n_tiles > 2 ? kt.entry(2) : 0;
    wait_vm_all();
    __syncthreads();
    u32x4 ds[4];
    f32x16 s1, dp1;
    PageMask m_t = mask_of(0);
    {
        f32x16 s0, dp0;
        tile_scores<D>(st, kb0 + la.k, vb0 + la.k, s0, dp0, [](int) {});
        tile_scores<D>(st, kb0 + la.k + 32 * 2 * D, vb0 + la.k + 32 * 2 * D, s1, dp1, [&](int ks) {
                           units_at<8, F::KS>(ks, [&](int un) {
                               ds_unit<MASK>(un, 0, s0, dp0, m_t.lim, st, scale_log2, ds);
                           });
                       });
    }
    for (int64_t t = 0; t < n_tiles; t++) {
        // K(t+1), V(t+1) have landed; K buffer (t+2) % 3 and V buffer t % 2 were last read
        // in iteration t-1.  The last iteration runs phase 1 on stale tiles; that result is
        // never used.
        const int32_t e3 = t + 3 < n_tiles ? kt.entry(t + 3) : 0;
        wait_vm_all();
        __syncthreads();
        const int k0 = (int)(t % 3), k1 = k0 == 2 ? 0 : k0 + 1, k2 = k0 == 0 ? 2 : k0 - 1;
        const int v0 = (int)(t & 1), v1 = v0 ^ 1;
        const PageMask m_n = mask_of(t + 1);
        dq_iter<MASK, D, NW>(st, kt, t, n_tiles - 1, t + 2 < n_tiles, e2, kb0 + k2 * F::TILE, vb0 + v0 * F::TILE,
                             kb0 + k1 * F::TILE, vb0 + v1 * F::TILE, kb0 + k0 * F::TILE, ds,
                             s1, dp1, m_t.lim, m_n.lim, la, scale_log2, w);
        m_t = m_n;
        e2 = e3;
    }
    wait_vm_all();  // the last iterations' copies land before the workgroup's LDS is released
    mfma_drain();
}

// Blocks (query tile, part, kv head) over parts [part0, part0 + n_parts_l).  MASK selects the
// per-element mask, needed only in the response part and at a partial last prompt page; the
// host launches the two kinds of parts separately, so that each kernel holds one pipeline.
template <int D, int NW, bool MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(1, 1)))
void dq_mfma_kernel(AttnArgs a, GroupRows gr, int n_qtiles, int part0, int n_parts_l, int n_blocks) {
    using F = TileShape<D>;
    constexpr int BM = 32 * NW;
    __shared__ __attribute__((aligned(1024))) char kbuf[3][F::TILE];
    __shared__ __attribute__((aligned(1024))) char vbuf[2][F::TILE];

    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    if (lb >= n_blocks) return;
    const int qtile = lb % n_qtiles;
    const int part = part0 + (lb / n_qtiles) % n_parts_l;
    const int kvh = lb / (n_qtiles * n_parts_l);
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
        }
        // read-only MFMA operands (after all loads are in flight), and the accumulators: AGPRs
#pragma unroll
        for (int ks = 0; ks < F::KS; ks++) asm volatile("" : "+a"(st.qb[ks]), "+a"(st.dob[ks]));
#pragma unroll
        for (int dt = 0; dt < F::DT; dt++) {
            st.dq[dt] = f32x16{};
            asm volatile("" : "+a"(st.dq[dt]));
        }
        agpr_write_gap();
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
    auto mask_of = [&](int64_t t) { return page_mask(kt.valid(t), (lp0 + t) * kPage, resp, vis_limit, h); };

    const uint32_t kb0 = lds_addr(kbuf[0]), vb0 = lds_addr(vbuf[0]);
    clear_lds(&kbuf[0][0], sizeof(kbuf), threadIdx.x, NW * 64);
    clear_lds(&vbuf[0][0], sizeof(vbuf), threadIdx.x, NW * 64);
    __syncthreads();
    if (n_tiles > 0) dq_pages<MASK, D, NW>(st, kt, n_tiles, mask_of, kb0, vb0, la, a.scale_log2, w);
    mfma_drain();
    if (!row_ok) return;
    float* dst = a.dq_parts + (((int64_t)part * a.n_rows + my_tok) * a.hq + my_head) * (int64_t)D;
    if (a.owner && h == 0)  // debug run: this lane pair writes the row
        atomicAdd(a.owner + a.owner_dq0 + ((int64_t)part * a.n_rows + my_tok) * a.hq + my_head, 1u);
#pragma unroll
    for (int dt = 0; dt < F::DT; dt++) {
        // scale in place in the AGPRs; the stores read them from there
#pragma unroll
        for (int i = 0; i < 16; i++) st.dq[dt][i] = agpr_scaled(st.dq[dt][i], a.scale);
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
            const int dd = dt * 32 + 8 * q4 + 4 * h;
            *(float4*)(dst + dd) = make_float4(st.dq[dt][4 * q4], st.dq[dt][4 * q4 + 1], st.dq[dt][4 * q4 + 2],
                                               st.dq[dt][4 * q4 + 3]);
        }
    }
}

template <int D, int NW>
hipError_t launch_dq_d(const AttnArgs& a, const GroupRows& gr, int64_t n_qtiles, hipStream_t s) {
    // prompt shards (masked only when the last prompt page is partial), then the response part
    if (a.n_shards > 0) {
        const int nb = (int)(n_qtiles * a.n_shards * a.hkv);
        if (a.prefix_len % kPage != 0)
            dq_mfma_kernel<D, NW, true><<<pad_grid(nb), NW * 64, 0, s>>>(a, gr, (int)n_qtiles, 0, a.n_shards, nb);
        else
            dq_mfma_kernel<D, NW, false><<<pad_grid(nb), NW * 64, 0, s>>>(a, gr, (int)n_qtiles, 0, a.n_shards, nb);
    }
    const int nb = (int)(n_qtiles * a.hkv);
    dq_mfma_kernel<D, NW, true><<<pad_grid(nb), NW * 64, 0, s>>>(a, gr, (int)n_qtiles, a.n_shards, 1, nb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dq_mfma(const AttnArgs& a, const GroupRows& gr, hipStream_t s) {
    constexpr int NW = 4;
    constexpr int BM = 32 * NW;
    const int64_t rows_total = a.n_rows * a.g;
    const int64_t n_qtiles = (rows_total + BM - 1) / BM;
    if (n_qtiles * a.n_parts * a.hkv == 0) return hipSuccess;
    KernelTimer kt("dq_mfma", s);
    switch (a.d) {
        case 64: return launch_dq_d<64, NW>(a, gr, n_qtiles, s);
        case 128: return launch_dq_d<128, NW>(a, gr, n_qtiles, s);
        case 256: return launch_dq_d<256, NW>(a, gr, n_qtiles, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ls
