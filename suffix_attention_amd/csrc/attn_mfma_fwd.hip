// Split-prefix replay-attention forward on gfx950 bf16 matrix cores.
//
// One workgroup handles BM = 128 query rows of one kv head's group against the keys of one
// part: a prompt shard (a contiguous range of logical pages, walked through the page table)
// or the response keys the rows see (causal).  It writes the part's normalised output and
// LSE, the owner-local softmax statistics that the merge composes into the exact result
// (LongStraw digest, "Method", Qwen implementation; explainer, "Two incompatible
// architectures, same transaction").
//
// Eight waves, two per SIMD, in two roles over the same four 32-row groups:
//   score wave g   S^T(t)[64 x 32] = K(t) . Q^T     v_mfma_f32_32x32x16_bf16, K from LDS,
//                                                  Q and S in VGPRs
//                  online softmax of page t - 1     each lane owns one row; P(t-1) goes to LDS
//                                                  already in the layout of an MFMA operand
//   output wave g  O^T[D x 32] += V(t-2)^T P(t-2)^T V read transposed from LDS
//                                                  (ds_read_b64_tr_b16), O in VGPRs
// The work runs in slots with two barriers each: between them the output waves fetch
// P(t-2) from LDS into registers; after the second the score waves compute S(t) with the
// softmax of page t - 1 interleaved step by step (its vector work issues while the matrix
// core runs the products), and the output waves issue the slot's copies and multiply
// V(t-2) P(t-2), so both waves of a SIMD keep its matrix core busy at once.  The copies sit
// with the output waves because a wave issues at most about one instruction per four cycles
// and the score wave's stream is the longer one.  Splitting the roles also halves the
// registers a wave needs (the 32 x D output tile alone is 128 registers at D = 256), which is
// what lets two waves share a SIMD.
//
// Keys are permuted inside each 16-key MFMA step so that P^T needs no data movement: the
// order is the same on both operands, so the sum is unchanged.
//
// The softmax keeps a running reference m for each row and moves it only when the page max
// exceeds it by more than kLazyLog2 (base 2); probabilities are then at most 2^kLazyLog2,
// which bf16 and the fp32 sums hold exactly as well as values below 1, and the output
// rescale is skipped on almost every page.  The result is the same softmax: every term and
// the sum are taken relative to the same m.
#include <math.h>

#include <type_traits>

#include "mfma_tiles.hpp"

namespace ls {
namespace {

constexpr float kLazyLog2 = 8.f;
constexpr int kNW = 8;           // waves per workgroup
constexpr int kGroups = 4;       // 32-row groups per workgroup
constexpr int kBM = 32 * kGroups;
static_assert(kBM == kFwdTileRows, "the host's sub-part split assumes this tile");

template <int D>
struct FwdLds {
    static constexpr int TILE = TileShape<D>::TILE;
    static constexpr int P_BYTES = 4 * 64 * 16;   // one group's P^T operands: 4 key steps x 64 lanes x 16 B
    char kb[2][TILE];
    char vb[2][TILE];
    char p[kGroups][P_BYTES];
    float alpha[kGroups][32];
    float fin_l[kGroups][32];
};

// Raw s_barrier after this wave's LDS accesses have completed.  The direct-to-LDS copies in
// flight are left alone (a workgroup fence would wait for them too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Copy addressing of the four output waves, which do all the copying: the score waves'
// instruction stream (scores, softmax) is the longer one.
template <int D>
using OutTiles = KeyTiles<D, kGroups>;

// Where the keys of the workgroup's part come from, and the rows it serves.
template <int D>
struct PartInfo {
    OutTiles<D> kt;     // copy addressing of the output waves (valid() serves both roles)
    bool resp;
    int64_t lp0;        // first logical page (prompt shard)
    int64_t n_tiles;
    int64_t tok_min;    // first token of the workgroup's rows
};

// ---------------------------------------------------------------------------------------
// score role
// ---------------------------------------------------------------------------------------

// The score wave's work per slot: the products S^T(t) = K(t) Q^T of page t for its 32 rows (two
// 32-key tiles, KS k-steps each, K fragments read PD steps ahead) and the online softmax of
// page t - 1, whose scores it holds from the slot before.  The softmax is cut into units
// that are spread over the k-steps, so that its vector work issues while the matrix core
// runs the products: a wave issues about one instruction per four cycles, and the product of
// one k-step keeps the matrix core busy for 64.  Each k-step is fenced off with a scheduling
// barrier so the compiler keeps that interleave (and the operand prefetch) as written.
template <int D>
struct ScoreStep {
    static constexpr int KS = TileShape<D>::KS;
    static constexpr int PD = 2;
};

// Mask page t's scores: element i of tile kt is key 32kt + 8(i/4) + 4h + i%4 of the page; the
// mask compares its lane-free part with two per-lane limits (valid keys of the page and, for
// response keys, the causal limit of this lane's row).
__device__ __forceinline__ void mask_scores(f32x16 (&s)[2], int valid, int64_t key0, bool resp, int64_t vis_limit,
                                            int h) {
    const int lim_valid = valid - 4 * h;
    int lim_causal = 64;
    if (resp) {
        const int64_t c = vis_limit - key0 - 4 * h;
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

// IEEE maximum (NaN-propagating): maps to v_maximum3_f32 without operand canonicalisation.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}

// Online softmax of one page for this lane's row, in units.  Score x (0..31) of the lane is
// element x % 16 of tile x / 16.  Units 0-15 take the raw maximum two scores at a time; unit
// 16 combines the two half-waves' maxima and moves the row's reference if the page exceeds it
// by more than kLazyLog2; units 17-32 exponentiate two scores each and pack them to bf16;
// units 33-36 store P^T (MFMA B-operand layout: key step ku at [ku][lane]); unit 37 updates
// the row sum and publishes the rescale factor.
constexpr int kSoftmaxUnits = 38;

struct SoftmaxState {
    float mx, alpha, m_use, lsum;
    uint32_t wd[16];
};

__device__ __forceinline__ float score_at(const f32x16 (&s)[2], int x) { return s[x >> 4][x & 15]; }

__device__ __forceinline__ void softmax_unit(int u, const f32x16 (&s)[2], SoftmaxState& st, float& m_ref, float& l,
                                             float scale_log2, LS_LDS char* p_out, LS_LDS float* alpha_out,
                                             int lane) {
    if (u < 16) {
        st.mx = max3f(st.mx, score_at(s, 2 * u), score_at(s, 2 * u + 1));
    } else if (u == 16) {
        // max on raw scores: scale_log2 > 0 commutes with max
        const float mx = __builtin_elementwise_maximum(st.mx, other_half(st.mx)) * scale_log2;
        st.alpha = 1.f;
        if (mx > m_ref + kLazyLog2) {  // false for a fully masked page (mx = -inf)
            st.alpha = fast_exp2(m_ref - mx);  // 0 on the first page (m_ref = -inf)
            m_ref = mx;
        }
        st.m_use = m_ref == -INFINITY ? 0.f : m_ref;
        st.lsum = 0.f;
    } else if (u < 33) {
        const int j = u - 17;
        const float p0 = fast_exp2(__builtin_fmaf(score_at(s, 2 * j), scale_log2, -st.m_use));
        const float p1 = fast_exp2(__builtin_fmaf(score_at(s, 2 * j + 1), scale_log2, -st.m_use));
        st.lsum += p0 + p1;
        st.wd[j] = pack_bf16x2(p0, p1);
    } else if (u < 37) {
        const int ku = u - 33;
        *(LS_LDS u32x4*)(p_out + (ku * 64 + lane) * 16) =
            u32x4{st.wd[4 * ku], st.wd[4 * ku + 1], st.wd[4 * ku + 2], st.wd[4 * ku + 3]};
    } else {
        l = l * st.alpha + st.lsum;
        if (lane < 32) alpha_out[lane] = st.alpha;
    }
}

// One slot of the score wave: S(t) into sn when SCORE, the softmax of the page held in sp when
// SOFTMAX (writing P and its rescale factor), interleaved step by step.
template <int D, bool SCORE, bool SOFTMAX>
__device__ __forceinline__ void score_slot_work(const bf16x8 (&qb)[TileShape<D>::KS], f32x16 (&sn)[2], uint32_t ak,
                                                const f32x16 (&sp)[2], float& m_ref, float& l, float scale_log2,
                                                LS_LDS char* p_out, LS_LDS float* alpha_out, int lane) {
    constexpr int KS = ScoreStep<D>::KS, PD = ScoreStep<D>::PD;
    SoftmaxState st;
    st.mx = -INFINITY;
    bf16x8 kbuf[PD][2];
    if constexpr (SCORE) {
        sn[0] = f32x16{};
        sn[1] = f32x16{};
#pragma unroll
        for (int j = 0; j < PD; j++) {
            const uint32_t pk = ak ^ (uint32_t)(j << 5);
            kbuf[j][0] = lds_b128(pk);
            kbuf[j][1] = lds_b128(pk + 32 * 2 * D);
        }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        if constexpr (SCORE) {
            const bf16x8 k0 = kbuf[ks % PD][0], k1 = kbuf[ks % PD][1];
            if (ks + PD < KS) {
                const uint32_t pk = ak ^ (uint32_t)((ks + PD) << 5);
                kbuf[ks % PD][0] = lds_b128(pk);
                kbuf[ks % PD][1] = lds_b128(pk + 32 * 2 * D);
            }
            sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qb[ks], sn[0], 0, 0, 0);
            sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qb[ks], sn[1], 0, 0, 0);
        }
        if constexpr (SOFTMAX) {
#pragma unroll
            for (int u = ks * kSoftmaxUnits / KS; u < (ks + 1) * kSoftmaxUnits / KS; u++)
                softmax_unit(u, sp, st, m_ref, l, scale_log2, p_out, alpha_out, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Score slot t (0 .. n_tiles + 1): scores of page t (t < n_tiles) and softmax of page t - 1
// (1 <= t <= n_tiles), after the two barriers: the first publishes K(t), the second tells
// that the output waves hold P(t - 2) in registers, so P(t - 1) may be written.
template <int D, bool SCORE, bool SOFTMAX>
__device__ __forceinline__ void score_slot(const AttnArgs& a, const PartInfo<D>& pi, int64_t t, uint32_t k_cur,
                                           char* __restrict__ p_out, float* __restrict__ alpha_out,
                                           const bf16x8 (&qb)[TileShape<D>::KS], f32x16 (&sn)[2], f32x16 (&sp)[2],
                                           float& m_ref, float& l, int64_t vis_limit, uint32_t lk, int lane) {
    wait_vm_all();
    lds_barrier();
    lds_barrier();
    if constexpr (SOFTMAX) {
        const int64_t tp = t - 1;
        const int valid = pi.kt.valid(tp);
        const int64_t key0 = (pi.lp0 + tp) * kPage;
        if (valid < kPage || (pi.resp && key0 + kPage - 1 > a.q_start + pi.tok_min))
            mask_scores(sp, valid, key0, pi.resp, vis_limit, lane >> 5);
    }
    score_slot_work<D, SCORE, SOFTMAX>(qb, sn, k_cur + lk, sp, m_ref, l, a.scale_log2, (LS_LDS char*)p_out,
                                       (LS_LDS float*)alpha_out, lane);
}

// ---------------------------------------------------------------------------------------
// output role
// ---------------------------------------------------------------------------------------

// O^T += V^T P^T over one page.  Step st = (ku, dt) with dt fastest, so consecutive MFMAs
// accumulate into different tiles; V^T fragments (rows 32kt + 16u + 8e) are read PV steps
// ahead.
template <int D, typename Beside>
__device__ __forceinline__ void accumulate_pv(f32x16 (&o)[TileShape<D>::DT], const bf16x8 (&pb)[4], uint32_t sv,
                                              Beside&& beside) {
    using F = TileShape<D>;
    constexpr int NST = 4 * F::DT;
    constexpr int PV = 4;
    i16x4 vlo[PV], vhi[PV];
    auto read_v = [&](int st, i16x4& lo, i16x4& hi) {
        const int dt = st % F::DT, ku = st / F::DT;
        const int R = 32 * (ku >> 1) + 16 * (ku & 1);
        lo = lds_tr4((sv ^ tr_x<D>(dt, R)) + R * 2 * D);
        hi = lds_tr4((sv ^ tr_x<D>(dt, R + 8)) + (R + 8) * 2 * D);
    };
#pragma unroll
    for (int j = 0; j < PV; j++) read_v(j, vlo[j], vhi[j]);
#pragma unroll
    for (int st = 0; st < NST; st++) {
        const int dt = st % F::DT, ku = st / F::DT;
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[st % PV], vhi[st % PV], 0, 1, 2, 3, 4, 5, 6, 7));
        if (st + PV < NST) read_v(st + PV, vlo[st % PV], vhi[st % PV]);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ku], o[dt], 0, 0, 0);
        beside(st);  // this step's share of the copies, beside the matrix work
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Output slot u (0 .. n_tiles + 1): after the first barrier fetch P(u - 2) (u >= 2); after the
// second, rescale O if a row's reference moved and accumulate V(u - 2) P(u - 2), with the
// slot's copies K(u + 1) and V(u - 1) issued one piece per step over the first steps.  Copies
// past either end repeat a tile of the part into a buffer nothing reads, so the steps carry no
// branch; slots 0 and 1 only copy.  Every pointer to LDS is restrict-qualified so that, once
// inlined, the compiler knows the copies just issued cannot alias the tiles being read.
template <int D>
__device__ __forceinline__ void slot_copies(const PartInfo<D>& pi, int64_t u, int32_t e_k, int32_t e_v,
                                            const char*& ksrc, const char*& vsrc, int& vk, int& vv) {
    const int64_t last = pi.n_tiles - 1;
    const int64_t tk = u + 1 < last ? u + 1 : last;
    const int64_t tv = u - 1 < 0 ? 0 : (u - 1 < last ? u - 1 : last);
    ksrc = pi.kt.tile(e_k, tk, false);
    vsrc = pi.kt.tile(e_v, tv, true);
    vk = pi.kt.valid(tk);
    vv = pi.kt.valid(tv);
}

template <int D>
__device__ __forceinline__ void output_slot(const AttnArgs& a, const PartInfo<D>& pi, int64_t u, int32_t e_k,
                                            int32_t e_v, uint32_t k_dst, uint32_t v_dst, uint32_t v_src,
                                            const char* __restrict__ p_in, const float* __restrict__ alpha_in,
                                            f32x16 (&o)[TileShape<D>::DT], uint32_t lv, int w, int lane) {
    using F = TileShape<D>;
    constexpr int PW = OutTiles<D>::PER_WAVE;
    wait_vm_all();
    lds_barrier();
    bf16x8 pb[4];
#pragma unroll
    for (int ku = 0; ku < 4; ku++) pb[ku] = *(const LS_LDS bf16x8*)((const LS_LDS char*)p_in + (ku * 64 + lane) * 16);
    const float alpha = ((const LS_LDS float*)alpha_in)[lane & 31];
    lds_barrier();  // P(u - 2) is in registers: the score waves may overwrite it
    if (!__all(alpha == 1.f)) {
#pragma unroll
        for (int dt = 0; dt < F::DT; dt++)
#pragma unroll
            for (int i = 0; i < 16; i++) o[dt][i] *= alpha;
    }
    const char *ksrc, *vsrc;
    int vk, vv;
    slot_copies<D>(pi, u, e_k, e_v, ksrc, vsrc, vk, vv);
    accumulate_pv<D>(o, pb, v_src + lv, [&](int st) {
        if (st < PW) pi.kt.copy_piece(ksrc, vk, k_dst, w, st);
        else if (st < 2 * PW) pi.kt.copy_piece(vsrc, vv, v_dst, w, st - PW);
    });
}

// Slots 0 and 1 of an output wave: the copies only.
template <int D>
__device__ __forceinline__ void output_copy_slot(const PartInfo<D>& pi, int64_t u, int32_t e_k, int32_t e_v,
                                                 uint32_t k_dst, uint32_t v_dst, int w) {
    constexpr int PW = OutTiles<D>::PER_WAVE;
    wait_vm_all();
    lds_barrier();
    lds_barrier();
    if (pi.n_tiles > 0) {
        const char *ksrc, *vsrc;
        int vk, vv;
        slot_copies<D>(pi, u, e_k, e_v, ksrc, vsrc, vk, vv);
#pragma unroll
        for (int st = 0; st < PW; st++) pi.kt.copy_piece(ksrc, vk, k_dst, w, st);
#pragma unroll
        for (int st = 0; st < PW; st++) pi.kt.copy_piece(vsrc, vv, v_dst, w, st);
    }
}

// Blocks (query tile, part, kv head); the query tiles of each member (pre-step scoring runs
// several members' blocks at once) are numbered member-major, n_qtiles_m per member.  They
// reach the XCDs as deal_block() orders them (long prompt-shard blocks first, evenly).
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kNW * 64, kNW * 64), amdgpu_waves_per_eu(2, 2)))
void fwd_mfma_kernel(AttnArgs a, int n_qtiles_m, int n_qtiles) {
    using F = TileShape<D>;
    __shared__ __attribute__((aligned(1024))) FwdLds<D> L;

    const XcdBlock blk = deal_block(blockIdx.x, n_qtiles, a.n_shards, a.n_parts, a.hkv);
    if (blk.qtile_g < 0) return;
    const int qtile_g = blk.qtile_g;
    const int member = qtile_g / n_qtiles_m;
    const int qtile = qtile_g % n_qtiles_m;
    const int part = blk.part;
    const int kvh = blk.kvh;
    const bool resp = part == a.n_shards;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g = w & (kGroups - 1);
    const bool score_role = w < kGroups;
    const int h = lane >> 5;
    const int n = lane & 31;
    const int64_t rows_total = a.n_rows * a.g;
    const int64_t r0 = (int64_t)qtile * kBM;
    const int64_t my_row = r0 + 32 * g + n;
    const bool row_ok = my_row < rows_total;
    const int64_t my_tok = my_row / a.g;
    const int my_head = kvh * a.g + (int)(my_row % a.g);
    const int64_t tok_base = (int64_t)member * a.n_rows;          // the member's first row in q
    const int64_t out_row0 = a.row0 + tok_base;                     // ... and in the parts arrays

    // keys of this part
    const int64_t lp0 = resp ? 0 : a.shard_lo[part];
    int64_t n_tiles;
    if (!resp) {
        n_tiles = a.shard_lo[part + 1] - a.shard_lo[part];
    } else {
        int64_t tok_max = (r0 + kBM - 1) / a.g;
        if (tok_max > a.n_rows - 1) tok_max = a.n_rows - 1;
        n_tiles = (a.q_start + tok_max + 1 + kPage - 1) / kPage;
    }

    // output wave g copies share g of every tile; the score waves use kt only for valid()
    PartInfo<D> pi{OutTiles<D>(a, resp, lp0, kvh, g, lane, (int64_t)member * a.resp_member_elems * 2)};
    const OutTiles<D>& kt = pi.kt;
    pi.resp = resp;
    pi.lp0 = lp0;
    pi.n_tiles = n_tiles;
    pi.tok_min = r0 / a.g;

    clear_lds(&L.kb[0][0], sizeof(L.kb), threadIdx.x, kNW * 64);
    clear_lds(&L.vb[0][0], sizeof(L.vb), threadIdx.x, kNW * 64);
    lds_barrier();
    char* p_grp = L.p[g];
    float* alpha_grp = L.alpha[g];
    LS_LDS float* fin_grp = (LS_LDS float*)L.fin_l[g];
    const LaneAddr<D> la(lane);

    // Slot t (0 .. n_tiles + 1): the score waves compute S(t) and the softmax of page t - 1,
    // the output waves accumulate page t - 2.  The lane's base offsets are re-materialised
    // opaquely each slot so that their xor variants are formed next to their reads instead of
    // all being held across the loop.
    if (score_role) {
        bf16x8 qb[F::KS];
        {
            // rows past the block (a partial last tile) read a valid row; their output is never stored
            const int64_t ld_row = row_ok ? my_row : rows_total - 1;
            const int64_t ld_tok = ld_row / a.g;
            const int ld_head = kvh * a.g + (int)(ld_row % a.g);
            const bf16_t* qrow = (const bf16_t*)a.q + ((tok_base + ld_tok) * a.hq + ld_head) * (int64_t)D + 8 * h;
#pragma unroll
            for (int ks = 0; ks < F::KS; ks++) qb[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * ks));
        }
        const int64_t vis_limit = a.q_start + my_tok;  // last response key this row sees
        float m_ref = -INFINITY, l = 0.f;
        f32x16 sa[2], sb[2];
        const uint32_t kb0 = lds_addr(L.kb[0]);
        auto slot = [&](auto score, auto softmax, int64_t t, f32x16(&sn)[2], f32x16(&sp)[2]) {
            uint32_t lk = la.k;
            asm volatile("" : "+v"(lk));
            score_slot<D, decltype(score)::value, decltype(softmax)::value>(
                a, pi, t, kb0 + (t & 1) * F::TILE, p_grp, alpha_grp, qb, sn, sp, m_ref, l, vis_limit, lk, lane);
        };
        using Y = std::true_type;
        using N = std::false_type;
        // slot 0: S(0) into sa; then pairs of slots alternate the two score buffers
        if (n_tiles > 0) slot(Y{}, N{}, 0, sa, sb);
        else slot(N{}, N{}, 0, sa, sb);
        int64_t t = 1;
        for (; t + 1 < n_tiles; t += 2) {
            slot(Y{}, Y{}, t, sb, sa);
            slot(Y{}, Y{}, t + 1, sa, sb);
        }
        if (t < n_tiles) {  // t = n_tiles - 1: S(t) into sb, then page t alone
            slot(Y{}, Y{}, t, sb, sa);
            slot(N{}, Y{}, t + 1, sa, sb);
        } else if (t == n_tiles) {  // page n_tiles - 1 is in sa
            slot(N{}, Y{}, t, sb, sa);
        }
        // slot n_tiles + 1: the output waves' last page; nothing left to score
        slot(N{}, N{}, n_tiles + 1, sa, sb);
        // final statistics for the output waves, and this part's LSE
        const float l_tot = l + other_half(l);
        if (lane < 32) fin_grp[lane] = l_tot;
        lds_barrier();
        // l_tot is 0 exactly when the row sees no key of the part (LSE -inf, O 0); a NaN in the
        // row's inputs leaves it NaN, and NaN is what the row's LSE and O then hold
        if (row_ok && h == 0)
            a.lse_parts[((int64_t)part * a.part_rows + out_row0 + my_tok) * a.hq + my_head] =
                l_tot != 0.f ? (m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
    } else {
        f32x16 o[F::DT];
#pragma unroll
        for (int dt = 0; dt < F::DT; dt++) o[dt] = f32x16{};
        // Page-table entries are read through the scalar cache a slot before their copies and
        // clamped where they are used; e_m1, e_0, e_p1 are the entries of tiles u - 1, u, u + 1.
        auto entry = [&](int64_t i) { return i >= 0 && i < n_tiles ? kt.entry(i) : 0; };
        int32_t e_m1 = 0, e_0 = entry(0), e_p1 = entry(1);
        // prologue: K(0) in flight
        if (n_tiles > 0) kt.copy(kt.tile(e_0, 0, false), kt.valid(0), lds_addr(L.kb[0]), g);
        const uint32_t kb0 = lds_addr(L.kb[0]), vb0 = lds_addr(L.vb[0]);
        // slots 0 and 1: only the copies (no page has been through the softmax yet)
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int32_t e_p2 = entry(u + 2);
            output_copy_slot<D>(pi, u, e_p1, e_m1, kb0 + ((u + 1) & 1) * F::TILE, vb0 + ((u + 1) & 1) * F::TILE, g);
            e_m1 = e_0;
            e_0 = e_p1;
            e_p1 = e_p2;
        }
        for (int64_t u = 2; u <= n_tiles + 1; u++) {
            const int32_t e_p2 = entry(u + 2);
            uint32_t lv = la.v;
            asm volatile("" : "+v"(lv));
            output_slot<D>(a, pi, u, e_p1, e_m1, kb0 + ((u + 1) & 1) * F::TILE, vb0 + ((u + 1) & 1) * F::TILE,
                           vb0 + (u & 1) * F::TILE, p_grp, alpha_grp, o, lv, g, lane);
            e_m1 = e_0;
            e_0 = e_p1;
            e_p1 = e_p2;
        }
        wait_vm_all();  // the last iterations' copies land before the workgroup's LDS is released
        lds_barrier();
        const float l_tot = fin_grp[n];
        if (row_ok) {
            const float inv = l_tot != 0.f ? 1.f / l_tot : 0.f;
            float* dst = a.o_parts + (((int64_t)part * a.part_rows + out_row0 + my_tok) * a.hq + my_head) * (int64_t)D;
#pragma unroll
            for (int dt = 0; dt < F::DT; dt++) {
#pragma unroll
                for (int i = 0; i < 16; i++) o[dt][i] *= inv;
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++) {
                    const int dd = dt * 32 + 8 * q4 + 4 * h;
                    *(float4*)(dst + dd) = make_float4(o[dt][4 * q4], o[dt][4 * q4 + 1], o[dt][4 * q4 + 2],
                                                       o[dt][4 * q4 + 3]);
                }
            }
        }
    }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
    const int64_t n_qtiles_m = (a.n_rows * a.g + kBM - 1) / kBM;
    const int64_t n_qtiles = n_qtiles_m * a.n_members;
    const int64_t n_blocks = n_qtiles * a.n_parts * a.hkv;
    if (n_blocks == 0) return hipSuccess;
    const int grid = deal_grid(n_qtiles, a.n_shards, a.n_parts, a.hkv);
    KernelTimer kt("fwd_mfma", s);
    fwd_mfma_kernel<D><<<grid, kNW * 64, 0, s>>>(a, (int)n_qtiles_m, (int)n_qtiles);
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
