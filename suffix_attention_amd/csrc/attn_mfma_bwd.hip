// Replay-attention backward on gfx950 bf16 matrix cores, for the loss sum(O * dO).
//
// P is recomputed from the forward's LSE, so the backward runs as two passes over the same
// keys (a dQ row sum over 2M keys cannot be gathered by a key-stationary kernel):
//
//  dq_mfma_kernel   (query tile, part, kv head), like the forward: per 64-key page,
//                   S^T = K Q^T and dP^T = V dO^T (Q, dO in VGPRs, K, V from LDS),
//                   dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T (K read transposed).
//                   Writes one dQ part per key part; the parts are summed afterwards.
//  dkdv_mfma_kernel (two pages, kv head): each wave keeps 32 keys of K and V in VGPRs and
//                   their dK, dV accumulators in AGPRs, and streams every query row of the
//                   group that sees them through LDS, 32 rows at a time:
//                   S = Q K^T, dP = dO V^T, P, dS = P (dP - delta),
//                   dV += P^T dO, dK += dS^T Q (dO, Q read transposed).
//                   The result is written to the gradient pages (first touch) or added to
//                   them; each element has exactly one writer, so no atomics are needed.
//
// A prep kernel first writes, per kv head and group row r = token * g + j,
// (LSE * log2 e, delta = rowsum(dO * O)) and group-major copies of the Q and dO rows, so the
// dK/dV pass streams each kv head's rows as one contiguous array.  Rows padded up to a
// multiple of 64 get (+inf, 0) and zero Q/dO, so their P is exactly 0 wherever they are read.
#include <math.h>

#include "mfma_bwd.hpp"

namespace ls {
namespace {

// ---------------------------------------------------------------------------------------
// prep: delta, log2-scaled LSE and group-major Q / dO rows; also delta in [n_rows, hq] order
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(AttnArgs a, GroupRows gr, float* __restrict__ delta_th) {
    static_assert(D % 64 == 0, "4 bf16 per lane per pass");
    const int64_t gw = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;  // one wave per (kvh, r)
    const int lane = threadIdx.x % 64;
    const int64_t rows_total = a.n_rows * a.g;
    if (gw >= gr.rows_pad * a.hkv) return;
    const int kvh = (int)(gw / gr.rows_pad);
    const int64_t r = gw % gr.rows_pad;
    uint2* qd = (uint2*)(gr.q + gw * D);
    uint2* dd = (uint2*)(gr.dout + gw * D);
    if (r >= rows_total) {
#pragma unroll
        for (int k = lane; k < D / 4; k += 64) qd[k] = dd[k] = make_uint2(0, 0);
        if (lane == 0) gr.lsed[gw] = f32x2{INFINITY, 0.f};
        return;
    }
    const int64_t th = (r / a.g) * a.hq + kvh * a.g + r % a.g;
    const uint2* o = (const uint2*)((const bf16_t*)a.o + th * D);
    const uint2* dout = (const uint2*)((const bf16_t*)a.dout + th * D);
    const uint2* q = (const uint2*)((const bf16_t*)a.q + th * D);
    float s = 0.f;
#pragma unroll
    for (int k = lane; k < D / 4; k += 64) {
        const uint2 ov = o[k], dv = dout[k];
        qd[k] = q[k];
        dd[k] = dv;
        s += bf16_to_f32((bf16_t)(ov.x & 0xffff)) * bf16_to_f32((bf16_t)(dv.x & 0xffff)) +
             bf16_to_f32((bf16_t)(ov.x >> 16)) * bf16_to_f32((bf16_t)(dv.x >> 16)) +
             bf16_to_f32((bf16_t)(ov.y & 0xffff)) * bf16_to_f32((bf16_t)(dv.y & 0xffff)) +
             bf16_to_f32((bf16_t)(ov.y >> 16)) * bf16_to_f32((bf16_t)(dv.y >> 16));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) {
        gr.lsed[gw] = f32x2{a.lse[th] * kLog2e, s};
        delta_th[th] = s;
    }
}

// ---------------------------------------------------------------------------------------
// dK/dV pass
// ---------------------------------------------------------------------------------------
constexpr int kRows = 32;  // query rows per LDS stage

template <int D>
struct RowStage {
    static constexpr int QBYTES = kRows * D * 2;            // one Q or dO row tile
    static constexpr int BYTES = 2 * QBYTES + kRows * 8;    // Q, dO, (lse2, delta) per row
};

// Copy group rows [r0, r0 + 32) of Q and dO (group-major, zero padded) and their
// (lse2, delta) into an LDS stage.
template <int D>
__device__ __forceinline__ void issue_rows(const GroupRows& gr, int kvh, int64_t r0, uint32_t stage, int w, int lane) {
    const int64_t base = ((int64_t)kvh * gr.rows_pad + r0) * D;
    dma_rows<D, 4, kRows>(gr.q + base, gr.dout + base, D, stage, stage + RowStage<D>::QBYTES, w, lane);
    if (w == 0 && lane < kRows * 8 / 16)
        dma16(gr.lsed + kvh * gr.rows_pad + r0, kRows * 8, lane * 16, stage + 2 * RowStage<D>::QBYTES);
}

// The same copy in pieces, so that a caller can spread it over its compute steps: piece p of
// 2 * PER_WAVE copies block p % PER_WAVE of Q (p < PER_WAVE) or dO; piece 0 also carries the
// (lse2, delta) pairs (wave 0).
template <int D>
struct RowCopy {
    static constexpr int RPK = 512 / D;
    static constexpr int PER_WAVE = kRows * D * 2 / 1024 / 4;
    static constexpr int JROWS = 4 * RPK;
    static constexpr int PIECES = 2 * PER_WAVE;
    uint32_t off[PER_WAVE];  // this lane's byte offset inside the Q (or dO) row tile, copy j

    __device__ __forceinline__ RowCopy(int w, int lane) {
        using F = TileShape<D>;
        const int low = w * RPK + lane / F::KCH;
        const int lane_x = (lane % F::KCH) ^ swz<D>(low);
#pragma unroll
        for (int j = 0; j < PER_WAVE; j++)
            off[j] = (uint32_t)(j * JROWS + low) * (D * 2) + (uint32_t)((lane_x ^ swz<D>(j * JROWS)) << 4);
    }

    __device__ __forceinline__ void piece(const GroupRows& gr, int kvh, int64_t r0, uint32_t stage, int w, int lane,
                                          int p) const {
        const int64_t base = ((int64_t)kvh * gr.rows_pad + r0) * D * 2;
        const int j = p % PER_WAVE;
        const char* src = (const char*)(p < PER_WAVE ? gr.q : gr.dout) + base;
        const uint32_t dst = stage + (p < PER_WAVE ? 0 : RowStage<D>::QBYTES);
        dma16(src, RowStage<D>::QBYTES, off[j], dst + (j * 4 + w) * 1024);
        if (p == 0 && w == 0 && lane < kRows * 8 / 16)
            dma16(gr.lsed + kvh * gr.rows_pad + r0, kRows * 8, lane * 16, stage + 2 * RowStage<D>::QBYTES);
    }
};

template <int D>
struct DkvState {
    bf16x8 kb[TileShape<D>::KS];   // K^T operand: key lane%32, d = 16ks + 8(lane/32) .. +8
    bf16x8 vb[TileShape<D>::KS];   // V^T operand
    f32x16 dk[TileShape<D>::DT];   // dK accumulators: col = d, rows = keys
    f32x16 dv[TileShape<D>::DT];
};

// Phase 1 of a row tile: S = Q K^T and dP = dO V^T for 32 rows x 32 keys (element i is row
// 8(i/4) + 4h + i%4 of the tile, key lane%32).  Q and dO fragments are read PD k-steps ahead;
// sk is the stage's LDS address plus the lane's natural-read offset.
template <int D, typename Copy, typename Tail>
__device__ __forceinline__ void tile_scores(const DkvState<D>& st, uint32_t sk, f32x16& s, f32x16& dp,
                                            Copy&& copy_step, Tail&& tail_read) {
    using F = TileShape<D>;
    s = f32x16{};
    dp = f32x16{};
    constexpr int PD = 3;
    bf16x8 qd[PD][2];
#pragma unroll
    for (int j = 0; j < PD; j++) {
        const uint32_t o = sk ^ (uint32_t)(j << 5);
        qd[j][0] = lds_b128(o);
        qd[j][1] = lds_b128(o + RowStage<D>::QBYTES);
    }
#pragma unroll
    for (int ks = 0; ks < F::KS; ks++) {
        const bf16x8 qa = qd[ks % PD][0], da = qd[ks % PD][1];
        if (ks + PD < F::KS) {
            const uint32_t o = sk ^ (uint32_t)((ks + PD) << 5);
            qd[ks % PD][0] = lds_b128(o);
            qd[ks % PD][1] = lds_b128(o + RowStage<D>::QBYTES);
        }
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, st.kb[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, st.vb[ks], dp, 0, 0, 0);
        copy_step(ks);  // this step's share of a later tile's copies, beside the matrix work
        tail_read(ks);  // the last steps, which read nothing of their own: phase 3's first reads
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Phase 2, one unit (u, hb, j2) of two elements: P = exp2(S log2e/sqrt(d) - LSE log2e) (0 for
// rows that precede the key when masked) and dS = P (dP - delta), packed as bf16 operand
// word 2hb + j2 of key step u.  Units are small so that they fit between consecutive matrix
// instructions.
struct Prob {
    uint32_t wp[2][4], wd[2][4];  // [u][word]
};

template <bool MASK>
__device__ __forceinline__ void prob_unit(int unit, const f32x16& s, const f32x16& dp, f32x4 l, int rmh,
                                          float scale_log2, Prob& pr) {
    const int u = unit >> 2, hb = (unit >> 1) & 1, j2 = unit & 1;
    float pv[2], dv[2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
        const int j = 2 * j2 + e;
        const int i = 8 * u + 4 * hb + j;
        float p = fast_exp2(__builtin_fmaf(s[i], scale_log2, -l[2 * e]));
        if (MASK) p = (16 * u + 8 * hb + j) >= rmh ? p : 0.f;  // rmh <= 0 where no row precedes the key
        pv[e] = p;
        dv[e] = p * (dp[i] - l[2 * e + 1]);
    }
    pr.wp[u][2 * hb + j2] = pack_bf16x2(pv[0], pv[1]);
    pr.wd[u][2 * hb + j2] = pack_bf16x2(dv[0], dv[1]);
}

// (LSE log2e, delta) of the two rows of unit `unit` (rows 16u + 8hb + 4h + 2j2, +1); lsd_h is
// the LDS address of the stage's pairs plus 8 bytes per row of the lane's 4h.
__device__ __forceinline__ f32x4 unit_lsd(int unit, uint32_t lsd_h) {
    const int u = unit >> 2, hb = (unit >> 1) & 1, j2 = unit & 1;
    return lds_f32x4(lsd_h + (16 * u + 8 * hb + 2 * j2) * 8);
}

// Phase 3 of row tile t: dV += P^T dO, dK += dS^T Q (dO, Q read transposed: rows are the
// contraction), with phase 2 of row tile t+1 (its S, dP already computed) spread over the
// steps so that its vector work runs while the matrix core is busy.  Step st = (u, dt), dt
// fastest; fragments read PT steps ahead.  sv is the stage's LDS address plus the lane's
// transposed-read offset.
constexpr int kPT = 2;  // phase-3 fragment reads in flight (steps ahead)

// Fragment st of phase 3 (dO^T and Q^T of key step u = st / DT, d tile st % DT): four
// transposing reads.  sv is the stage's LDS address plus the lane's transposed-read offset.
template <int D>
__device__ __forceinline__ void read_accumulate_frag(uint32_t sv, int st_, i16x4* f) {
    const int dt = st_ % TileShape<D>::DT, u = st_ / TileShape<D>::DT;
    const int R = 16 * u;
    const uint32_t a0 = (sv ^ tr_x<D>(dt, R)) + R * 2 * D;
    const uint32_t a1 = (sv ^ tr_x<D>(dt, R + 8)) + (R + 8) * 2 * D;
    f[0] = lds_tr4(a0 + RowStage<D>::QBYTES);
    f[1] = lds_tr4(a1 + RowStage<D>::QBYTES);
    f[2] = lds_tr4(a0);
    f[3] = lds_tr4(a1);
}

template <bool MASK, int D>
__device__ __forceinline__ void tile_accumulate(DkvState<D>& st, const Prob& cur, uint32_t sv, const f32x16& s_n,
                                                const f32x16& dp_n, uint32_t lsd_n, int rmh_n, float scale_log2,
                                                Prob& nxt, i16x4 (&fr)[kPT][4]) {
    using F = TileShape<D>;
    bf16x8 pa[2], sa[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
        pa[u] = __builtin_bit_cast(bf16x8, (u32x4{cur.wp[u][0], cur.wp[u][1], cur.wp[u][2], cur.wp[u][3]}));
        sa[u] = __builtin_bit_cast(bf16x8, (u32x4{cur.wd[u][0], cur.wd[u][1], cur.wd[u][2], cur.wd[u][3]}));
    }
    constexpr int NST = 2 * F::DT;
    constexpr int PT = kPT;
    constexpr int NU = 8;  // phase-2 units of the next tile
    // fragments 0 .. PT-1 were read at the end of phase 1 (fr)
    auto read_t = [&](int st_, i16x4* f) { read_accumulate_frag<D>(sv, st_, f); };
    // each unit's (LSE, delta) pair is read one unit ahead: a read issued just before its use
    // would make the wait for it (LDS returns in order) drain the prefetched operand reads too
    f32x4 lb[2];
    lb[0] = unit_lsd(0, lsd_n);
#pragma unroll
    for (int st_ = 0; st_ < NST; st_++) {
        const int dt = st_ % F::DT, u = st_ / F::DT;
        i16x4* f = fr[st_ % PT];
        const bf16x8 dob = __builtin_bit_cast(bf16x8, __builtin_shufflevector(f[0], f[1], 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 qbt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(f[2], f[3], 0, 1, 2, 3, 4, 5, 6, 7));
        if (st_ + PT < NST) read_t(st_ + PT, f);
        mfma32_agpr2(st.dv[dt], pa[u], dob, st.dk[dt], sa[u], qbt);
        // units [st*NU/NST, (st+1)*NU/NST) of the next tile's phase 2 run beside this step;
        // constant loop bounds so that every unit index is a constant after unrolling
#pragma unroll
        for (int un = 0; un < NU; un++)
            if (un >= st_ * NU / NST && un < (st_ + 1) * NU / NST) {
                if (un + 1 < NU) lb[(un + 1) & 1] = unit_lsd(un + 1, lsd_n);
                prob_unit<MASK>(un, s_n, dp_n, lb[un & 1], rmh_n, scale_log2, nxt);
            }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Row tile t of the pipeline: phase 1 of tile t+1, then phase 3 of tile t with phase 2 of
// tile t+1 beside it.  The LDS stages are restrict pointers so that, once inlined, the
// compiler knows the copy in flight (into `dst`) cannot alias the stages being read and does
// not wait for it.
template <bool MASK, int D>
__device__ __forceinline__ void dkdv_step(DkvState<D>& st, uint32_t stage_t, uint32_t stage_n, uint32_t dst,
                                          const GroupRows& gr, const RowCopy<D>& rc, int kvh, int64_t copy_r0,
                                          const Prob& cur, Prob& nxt,
                                          LaneAddr<D> la, int rmh_n, float scale_log2, int w, int lane) {
    // the copies of the tile two ahead are spread over the S / dP steps, so that issuing them
    // never stalls the wave for long and they overlap the matrix work (near the end the caller
    // passes the last tile again, into a stage nothing reads, so that there is no branch here)
    auto copy_step = [&](int ks) {
#pragma unroll
        for (int p = 0; p < RowCopy<D>::PIECES; p++)
            if (p * TileShape<D>::KS / RowCopy<D>::PIECES == ks) rc.piece(gr, kvh, copy_r0, dst, w, lane, p);
    };
    uint32_t lk = la.k, lv = la.v;
    asm volatile("" : "+v"(lk), "+v"(lv));
    f32x16 s_n, dp_n;
    // phase 3's first fragments (tile t, whose stage has landed) are read in phase 1's last
    // steps, so that phase 3 does not start by waiting for them
    i16x4 fr[kPT][4];
    const uint32_t sv = stage_t + lv;
    tile_scores<D>(st, stage_n + lk, s_n, dp_n, copy_step, [&](int ks) {
        const int j = ks - (TileShape<D>::KS - kPT);
        if (j >= 0) read_accumulate_frag<D>(sv, j, fr[j]);
    });
    tile_accumulate<MASK, D>(st, cur, sv, s_n, dp_n, stage_n + 2 * RowStage<D>::QBYTES + (lane >> 5) * 32, rmh_n,
                             scale_log2, nxt, fr);
}

// One workgroup: 4 waves over two consecutive 64-key pages (wave w: page w/2, keys
// 32 (w%2) .. +32).  Pairs [0, n_pp) are prompt page pairs, the rest response pairs; a launch
// covers pairs [pair0, pair0 + n_pairs_l) of every kv head.  MASK selects the causal mask, which
// only response pairs need; the host launches the two kinds separately.  DS also stores every
// row tile's dS (a.ds), for the dQ pass to read; response pairs then walk every row tile, so
// that the masked (row, key) pairs are stored as 0 too.
template <int D, bool MASK, bool DS>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void dkdv_mfma_kernel(AttnArgs a, GroupRows gr, int n_pp, int pair0, int n_pairs_l, int n_blocks) {
    using F = TileShape<D>;
    constexpr int kStage = (RowStage<D>::BYTES + 1023) / 1024 * 1024;
    __shared__ __attribute__((aligned(1024))) char stg[3][kStage];

    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    if (lb >= n_blocks) return;
    const int kvh = (DS ? a.ds_kvh0 : 0) + lb / n_pairs_l;
    const int pair = pair0 + lb % n_pairs_l;
    const bool resp = pair >= n_pp;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int n = lane & 31;
    const int64_t rows_total = a.n_rows * a.g;

    // ---- this wave's 32 keys
    const int64_t page = 2 * (int64_t)(resp ? pair - n_pp : pair) + (w >> 1);  // logical or response page
    const int64_t n_pages_here = resp ? (a.key_end + kPage - 1) / kPage : a.n_logical_pages;
    const bool page_exists = page < n_pages_here;
    // the wave writes its page's gradients only if the launch owns the page (a chunk of key
    // parts owns its shards' pages; a pair cut by the chunk's edge has one page of each chunk)
    const bool page_ok = page_exists && (resp || (page >= a.pg_lo && page < a.pg_hi));
    const int64_t src_page = page_exists ? page : page - 1;  // an existing page to read
    const int kh = w & 1;
    int32_t phys = 0;
    int valid;
    const bf16_t *ksrc, *vsrc;
    int64_t stride;
    if (!resp) {
        phys = a.table[src_page];
        phys = phys < 0 ? 0 : (phys >= a.n_phys ? (int32_t)(a.n_phys - 1) : phys);
        const int64_t off = ((int64_t)phys * a.hkv + kvh) * kPage * D;
        ksrc = (const bf16_t*)a.k_pages + off;
        vsrc = (const bf16_t*)a.v_pages + off;
        stride = D;
        const int64_t left = a.prefix_len - src_page * kPage;
        valid = left < kPage ? (int)left : kPage;
    } else {
        const int64_t off = (src_page * kPage * a.hkv + kvh) * D;
        ksrc = (const bf16_t*)a.k_resp + off;
        vsrc = (const bf16_t*)a.v_resp + off;
        stride = (int64_t)a.hkv * D;
        const int64_t left = a.key_end - src_page * kPage;
        valid = left < kPage ? (int)left : kPage;
    }
    DkvState<D> st;
    {
        int kr = 32 * kh + n;
        if (kr >= valid) kr = valid - 1;  // keys past the end: any finite row, never written
        const bf16_t* krow = ksrc + kr * stride + 8 * h;
        const bf16_t* vrow = vsrc + kr * stride + 8 * h;
#pragma unroll
        for (int ks = 0; ks < F::KS; ks++) {
            st.kb[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(krow + 16 * ks));
            st.vb[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(vrow + 16 * ks));
        }
#pragma unroll
        for (int dt = 0; dt < F::DT; dt++) {
            st.dk[dt] = st.dv[dt] = f32x16{};
            asm volatile("" : "+a"(st.dk[dt]), "+a"(st.dv[dt]));  // accumulators live in AGPRs
        }
        agpr_write_gap();
    }

    // ---- rows that see these keys: all rows for the prompt; for response keys the rows
    // whose token is at least (first key of the pair) - q_start
    const int64_t key0_pair = 2 * (int64_t)(resp ? pair - n_pp : pair) * kPage;
    int64_t r_begin = 0;
    if (!DS && resp && key0_pair > a.q_start) r_begin = (key0_pair - a.q_start) * a.g / kRows * kRows;
    const int64_t n_stages = rows_total > r_begin ? (rows_total - r_begin + kRows - 1) / kRows : 0;
    // causal limit of this lane's key: visible to group rows >= (key - q_start) * g
    const int64_t my_key = page * kPage + 32 * kh + n;
    const int64_t row_min = resp ? (my_key - a.q_start) * a.g : 0;

    // Causal mask of row tile t: rmh is the number of its rows (without the 4h of this lane's
    // half) that precede this lane's key; it is <= 0 wherever no row does (all prompt keys).
    auto rmh_of = [&](int64_t t) {
        const int64_t rm = row_min - (r_begin + t * kRows);
        return (rm < 0 ? 0 : (rm > kRows ? kRows : (int)rm)) - 4 * h;
    };

    // Pipeline over row tiles (three LDS stages): iteration t copies tile t+2, computes
    // S and dP of tile t+1, and accumulates tile t with tile t+1's P and dS formed beside it.
    const LaneAddr<D> la(lane);
    const RowCopy<D> rc(w, lane);
    const uint32_t stg0 = lds_addr(stg[0]);
    if (n_stages > 0) {
        issue_rows<D>(gr, kvh, r_begin, stg0, w, lane);
        if (n_stages > 1) issue_rows<D>(gr, kvh, r_begin + kRows, stg0 + kStage, w, lane);
        wait_vm_all();
        __syncthreads();
        Prob cur;
        {
            f32x16 s0, dp0;
            tile_scores<D>(st, stg0 + la.k, s0, dp0, [](int) {}, [](int) {});
            const int rmh0 = rmh_of(0);
            const uint32_t lsd0 = stg0 + 2 * RowStage<D>::QBYTES + h * 32;
#pragma unroll
            for (int un = 0; un < 8; un++) prob_unit<MASK>(un, s0, dp0, unit_lsd(un, lsd0), rmh0, a.scale_log2, cur);
        }
        // stage t % 3 is kept as a rotating counter (no 64-bit division in the loop)
        const int n_st = (int)n_stages;
        int it = 0;
        // stored dS of this lane: row tile t (r_begin = 0 here), key slot of its key, the 16
        // positions of its lane half
        u32x4* ds_p = nullptr;
        int64_t ds_step = 0;
        if (DS) {
            const int64_t slot = (resp ? a.ds_resp_slot0 + 128 * (int64_t)(pair - n_pp) : 128 * ((int64_t)pair - a.ds_pair0)) +
                                 64 * (w >> 1) + 32 * kh + n;
            ds_p = (u32x4*)(a.ds + ((int64_t)(kvh - a.ds_kvh0) * a.ds_rt * a.ds_kslots + slot) * 32 + 16 * h);
            ds_step = a.ds_kslots * 32 * 2 / 16;
        }
        for (int t = 0; t < n_st; t++) {
            // tile t+1 has landed; stage (t+2) % 3 was last read in iteration t-1
            wait_vm_all();
            __syncthreads();
            if (DS) {
                // tile t's dS words, in register order: [key step u][word]; issued here so that
                // they drain during the iteration, before the next wait for the copies
                ds_p[0] = u32x4{cur.wd[0][0], cur.wd[0][1], cur.wd[0][2], cur.wd[0][3]};
                ds_p[1] = u32x4{cur.wd[1][0], cur.wd[1][1], cur.wd[1][2], cur.wd[1][3]};
                ds_p += ds_step;
            }
            // the last iteration runs phases 1-2 on a stale stage; that result is never used
            const int rmhn = rmh_of(t + 1);
            Prob nxt;
            const int it1 = it == 2 ? 0 : it + 1, it2 = it == 0 ? 2 : it - 1;
            dkdv_step<MASK, D>(st, stg0 + it * kStage, stg0 + it1 * kStage, stg0 + it2 * kStage,
                         gr, rc, kvh, r_begin + (int64_t)(t + 2 < n_st ? t + 2 : n_st - 1) * kRows, cur, nxt, la,
                         rmhn, a.scale_log2, w, lane);
            cur = nxt;
            it = it1;
        }
        wait_vm_all();  // the last iterations' copies land before the workgroup's LDS is released
    }

    // ---- write this wave's keys: dK (scaled) and dV, element i is key 8(i/4) + 4h + i%4
    mfma_drain();
    if (!page_ok) return;
    if (a.owner && lane == 0)  // debug run: this wave writes its half of the page
        atomicAdd(a.owner + (resp ? a.owner_resp0 + (page * a.hkv + kvh) * 2 + kh
                                  : ((int64_t)phys * a.hkv + kvh) * 2 + kh), 1u);
    bool first;
    float *gk, *gv;
    int64_t key_stride;
    if (!resp) {
        int s = 0;
        while (s + 1 < a.n_shards && page >= a.shard_lo[s + 1]) s++;
        first = (a.first_touch_mask >> s) & 1ull;
        const int64_t off = ((int64_t)phys * a.hkv + kvh) * kPage * D;
        gk = a.dk_pages + off;
        gv = a.dv_pages + off;
        key_stride = D;
    } else {
        first = a.resp_first_touch != 0;
        const int64_t off = (page * kPage * a.hkv + kvh) * D;
        gk = a.dk_resp + off;
        gv = a.dv_resp + off;
        key_stride = (int64_t)a.hkv * D;
    }
    // Four key rows at a time: all their old values are loaded before any is used, so the
    // read-modify-writes of an accumulating pass overlap instead of waiting one by one.  Keys
    // past the block are skipped, except that a first touch writes the padding rows of a prompt
    // page as 0; their loads read row 0 (always a key) and are discarded.
#pragma unroll
    for (int ib = 0; ib < 16; ib += 4) {
        float old_k[4][F::DT], old_v[4][F::DT];
        if (!first) {
#pragma unroll
            for (int ii = 0; ii < 4; ii++) {
                const int i = ib + ii;
                const int kr = 32 * kh + 8 * (i >> 2) + 4 * h + (i & 3);
                const int rr = kr < valid ? kr : 0;
#pragma unroll
                for (int dt = 0; dt < F::DT; dt++) {
                    old_k[ii][dt] = gk[rr * key_stride + n + 32 * dt];
                    old_v[ii][dt] = gv[rr * key_stride + n + 32 * dt];
                }
            }
        }
#pragma unroll
        for (int ii = 0; ii < 4; ii++) {
            const int i = ib + ii;
            const int kr = 32 * kh + 8 * (i >> 2) + 4 * h + (i & 3);  // key row within the page
            const bool key_ok = kr < valid;
            if (!key_ok && (resp || !first)) continue;  // response keys past the block / kept padding
            float* pk = gk + kr * key_stride + n;
            float* pv = gv + kr * key_stride + n;
#pragma unroll
            for (int dt = 0; dt < F::DT; dt++) {
                const float vk = key_ok ? a.scale * st.dk[dt][i] : 0.f;
                const float vv = key_ok ? st.dv[dt][i] : 0.f;
                pk[32 * dt] = first ? vk : old_k[ii][dt] + vk;
                pv[32 * dt] = first ? vv : old_v[ii][dt] + vv;
            }
        }
    }
}

template <int D>
hipError_t launch_bwd_d(const AttnArgs& a, hipStream_t s) {
    const int64_t rows_total = a.n_rows * a.g;
    const int64_t rows_pad = rows_padded(rows_total);
    const GroupRows gr = group_rows(a.dq_parts + (int64_t)a.n_parts * a.n_rows * a.hq * D, rows_pad, a.hkv, D);
    float* delta_th = const_cast<float*>(a.delta);
    if (rows_total > 0) {
        const int64_t waves = rows_pad * a.hkv;
        KernelTimer kt("bwd_prep", s);
        bwd_prep_kernel<D><<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(a, gr, delta_th);
    }
    // dK / dV
    const int n_pp = (int)((a.n_logical_pages + 1) / 2);
    const int n_rp = (int)((resp_tiles(a.key_end) + 1) / 2);
    if (a.ds) {
        // stored dS, a chunk at a time (ds_heads kv heads by ds_parts consecutive key parts):
        // dK/dV writes the chunk's dS, then dQ reads it for the chunk's parts
        const int n_all = a.n_shards + 1;
        for (int k0 = 0; k0 < a.hkv; k0 += a.ds_heads) {
            const int nh = a.hkv - k0 < a.ds_heads ? a.hkv - k0 : a.ds_heads;
            for (int p0 = 0; p0 < n_all; p0 += a.ds_parts) {
                const int p1 = p0 + a.ds_parts < n_all ? p0 + a.ds_parts : n_all;
                const PartChunk pc = part_chunk(a.shard_lo, a.n_shards, a.key_end, p0, p1);
                AttnArgs c = a;
                c.ds_kvh0 = k0;
                c.pg_lo = pc.pg_lo;
                c.pg_hi = pc.pg_hi;
                c.ds_pair0 = pc.pair_lo;
                c.ds_resp_slot0 = 128 * pc.n_pairs;
                const int nbp = (int)pc.n_pairs * nh, nbr = pc.resp ? n_rp * nh : 0;
                if (nbp + nbr > 0) {
                    KernelTimer kt("dkdv_mfma", s);
                    if (nbp > 0)
                        dkdv_mfma_kernel<D, false, true><<<pad_grid(nbp), 256, 0, s>>>(c, gr, n_pp, (int)pc.pair_lo,
                                                                                        (int)pc.n_pairs, nbp);
                    if (nbr > 0) dkdv_mfma_kernel<D, true, true><<<pad_grid(nbr), 256, 0, s>>>(c, gr, n_pp, n_pp, n_rp, nbr);
                }
                hipError_t e = hipGetLastError();
                const int s1 = p1 < a.n_shards ? p1 : a.n_shards;
                if (e == hipSuccess && a.dq_sub_k > 1 && p0 == 0 && p1 == n_all) {
                    // a small block: the dQ pass over k sub-ranges of every shard, into dq_sub
                    AttnArgs r = c;
                    r.n_shards = a.n_shards * a.dq_sub_k;
                    r.n_parts = r.n_shards + 1;
                    split_bounds(a.shard_lo, a.n_shards, a.dq_sub_k, r.shard_lo);
                    r.dq_parts = a.dq_sub;
                    e = launch_dqs_mfma(r, nh, 0, r.n_shards, true, s);
                } else if (e == hipSuccess) {
                    e = launch_dqs_mfma(c, nh, p0 < s1 ? p0 : 0, p0 < s1 ? s1 - p0 : 0, pc.resp, s);
                }
                if (e != hipSuccess) return e;
            }
        }
        return hipSuccess;
    }
    if ((int64_t)(n_pp + n_rp) * a.hkv > 0) {
        KernelTimer kt("dkdv_mfma", s);
        const int nbp = n_pp * a.hkv, nbr = n_rp * a.hkv;
        if (nbp > 0) dkdv_mfma_kernel<D, false, false><<<pad_grid(nbp), 256, 0, s>>>(a, gr, n_pp, 0, n_pp, nbp);
        if (nbr > 0) dkdv_mfma_kernel<D, true, false><<<pad_grid(nbr), 256, 0, s>>>(a, gr, n_pp, n_pp, n_rp, nbr);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.skip_dq) return e;
    // dQ parts recomputed (attn_mfma_dq.hip)
    return launch_dq_mfma(a, gr, s);
}

}  // namespace

hipError_t launch_bwd_mfma(const AttnArgs& a, hipStream_t s) {
    switch (a.d) {
        case 64: return launch_bwd_d<64>(a, s);
        case 128: return launch_bwd_d<128>(a, s);
        case 256: return launch_bwd_d<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ls
