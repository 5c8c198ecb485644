// Split-prefix replay-attention forward on gfx950 bf16 matrix cores: one wave per SIMD, 64
// query rows per wave.
//
// One workgroup handles 256 query rows of one kv head's group against the keys of one part (a
// prompt shard walked through the page table, or the response keys the rows see) and writes
// the part's normalised output and LSE, the owner-local statistics that the merge composes
// into the exact result (LongStraw digest, "Method", Qwen implementation; explainer, "Two
// incompatible architectures, same transaction").
//
// Each of the four waves owns two 32-row tiles and keeps their Q (the B operands of
// S^T = K Q^T, 2 x D/2 registers) and their O^T accumulators (AGPRs) for the whole part.  Every
// operand fragment read from LDS therefore feeds two matrix instructions, one per row tile: a
// K fragment (32 keys x 16 d) both tiles' scores, a V^T fragment (32 d x 16 keys) both tiles'
// outputs.  P never leaves the registers: keys are permuted inside each 16-key step
// identically on both operands of O^T += V^T P^T, so the score accumulators are, once
// exponentiated and packed, already the B operand.
//
// A page (64 keys) runs in four phases of 2 * D/16 matrix instructions:
//   1  S^T of keys 0-31                     beside: the copies of the next page
//   2  S^T of keys 32-63                    beside: the softmax of keys 0-31
//   3  O^T += V^T P^T over keys 0-31        beside: the softmax of keys 32-63
//   4  O^T += V^T P^T over keys 32-63
// so the vector work of each half-page's softmax issues while the matrix core runs the other
// half's products.  K and V pages are double-buffered in LDS (one barrier per page).
//
// The softmax keeps one running reference m per row and moves it only when a half-page's
// maximum exceeds it by more than kLazyLog2 (base 2), so probabilities stay below 2^kLazyLog2
// and the output is almost never rescaled; when it is, O is scaled in place (in the AGPRs)
// after the products already taken relative to the old reference, before any taken relative
// to the new one.  Every term and the sum are relative to the same m, so the result is the
// same softmax.
#include <math.h>

#include "mfma_tiles.hpp"

namespace ls {
namespace {

constexpr float kLazyLog2 = 8.f;
constexpr int kW = 4;               // waves per workgroup, one per SIMD
constexpr int kRT = 2;              // 32-row tiles per wave
constexpr int kBM = 32 * kRT * kW;  // query rows per workgroup
static_assert(kBM == kFwdTileRows, "the host's sub-part split assumes this tile");

template <int D>
struct FwdLds {
    char kb[2][TileShape<D>::TILE];
    char vb[2][TileShape<D>::TILE];
};

// Raw s_barrier after this wave's LDS accesses have completed; the direct-to-LDS copies in
// flight are left alone (a workgroup fence would wait for them too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// IEEE maximum (NaN-propagating): maps to v_maximum3_f32.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}

// Mask one 32-key tile of scores of one row tile: element i is key 32kt + 8(i/4) + 4h + i%4 of
// the page; keys at or past `valid` go to -inf, and so do keys past `causal` (the last key of
// the page this lane's row sees, counted from the page's first key; 64 or more: all).
__device__ __forceinline__ void mask_tile(f32x16& s, int kt, int valid, int causal, int h) {
    const int lim_valid = valid - 4 * h - 32 * kt;
    const int lim_causal = causal - 4 * h - 32 * kt;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int kc = 8 * (i >> 2) + (i & 3);
        s[i] = (kc < lim_valid && kc <= lim_causal) ? s[i] : -INFINITY;
    }
}

// The softmax of one 32-key tile for both row tiles, in units spread over a phase's steps.
// Units 0-7 take the maximum of four scores of each row tile; unit 8 combines the two
// half-waves' maxima and moves a row's reference if the tile exceeds it by more than
// kLazyLog2; units 9-16 exponentiate and pack four scores of each row tile; unit 17 updates the
// row sums.
constexpr int kSmUnits = 18;

struct SmState {
    float mx[kRT], alpha[kRT], m_use[kRT], lsum[kRT];
};

// Each unit ends by pinning its results with an empty asm statement: without it, the compiler
// sinks the exponentials into the block that first uses them (past the rescale branch, into the
// next phase), where no matrix work hides them.
__device__ __forceinline__ void sm_unit(int u, const f32x16 (&s)[kRT], SmState& st, float (&m_ref)[kRT],
                                        float (&l)[kRT], uint32_t (&wd)[kRT][8], float scale_log2) {
    if (u < 8) {
#pragma unroll
        for (int rt = 0; rt < kRT; rt++) {
            st.mx[rt] = max3f(st.mx[rt], s[rt][2 * u], s[rt][2 * u + 1]);
            asm volatile("" : "+v"(st.mx[rt]));
        }
    } else if (u == 8) {
#pragma unroll
        for (int rt = 0; rt < kRT; rt++) {
            // max on raw scores: scale_log2 > 0 commutes with max
            const float mx = __builtin_elementwise_maximum(st.mx[rt], other_half(st.mx[rt])) * scale_log2;
            st.alpha[rt] = 1.f;
            if (mx > m_ref[rt] + kLazyLog2) {  // false for a fully masked tile (mx = -inf) and for NaN
                // while the row has seen nothing its O and sum are exactly 0: nothing to rescale
                st.alpha[rt] = m_ref[rt] == -INFINITY ? 1.f : fast_exp2(m_ref[rt] - mx);
                m_ref[rt] = mx;
            }
            st.m_use[rt] = m_ref[rt] == -INFINITY ? 0.f : m_ref[rt];
            st.lsum[rt] = 0.f;
            asm volatile("" : "+v"(st.alpha[rt]), "+v"(st.m_use[rt]), "+v"(m_ref[rt]));
        }
    } else if (u < 17) {
        const int j = u - 9;
#pragma unroll
        for (int rt = 0; rt < kRT; rt++) {
            const float p0 = fast_exp2(__builtin_fmaf(s[rt][2 * j], scale_log2, -st.m_use[rt]));
            const float p1 = fast_exp2(__builtin_fmaf(s[rt][2 * j + 1], scale_log2, -st.m_use[rt]));
            st.lsum[rt] += p0 + p1;
            wd[rt][j] = pack_bf16x2(p0, p1);
            asm volatile("" : "+v"(wd[rt][j]), "+v"(st.lsum[rt]));
        }
    } else {
#pragma unroll
        for (int rt = 0; rt < kRT; rt++) {
            l[rt] = l[rt] * st.alpha[rt] + st.lsum[rt];
            asm volatile("" : "+v"(l[rt]));
        }
    }
}

// O *= alpha per row (the lane's row of each row tile), in place in the AGPRs, if any row's
// reference moved.  The products that used the old reference must have retired first.
template <int DT>
__device__ __forceinline__ void rescale_o(f32x16 (&o)[DT][kRT], const float (&alpha)[kRT]) {
    if (__all(alpha[0] == 1.f && alpha[1] == 1.f)) return;
    mfma_drain();
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int rt = 0; rt < kRT; rt++)
#pragma unroll
            for (int i = 0; i < 16; i++) o[dt][rt][i] = agpr_scaled(o[dt][rt][i], alpha[rt]);
    agpr_write_gap();
}

// Phase 1 / 2: S^T of the 32 keys of tile kt for both row tiles.  K fragments (rows 32kt..,
// d step ks) are read PD steps ahead; beside(ks) runs that step's share of the other work.
template <int D, typename Beside>
__device__ __forceinline__ void score_tile(f32x16 (&s)[kRT], const bf16x8 (&qb)[kRT][TileShape<D>::KS], uint32_t ak,
                                           Beside&& beside) {
    constexpr int KS = TileShape<D>::KS, PD = 2;
    bf16x8 kbuf[PD];
#pragma unroll
    for (int j = 0; j < PD; j++) kbuf[j] = lds_b128(ak ^ (uint32_t)(j << 5));
#pragma unroll
    for (int rt = 0; rt < kRT; rt++) s[rt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        const bf16x8 kf = kbuf[ks % PD];
        if (ks + PD < KS) kbuf[ks % PD] = lds_b128(ak ^ (uint32_t)((ks + PD) << 5));
#pragma unroll
        for (int rt = 0; rt < kRT; rt++) s[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qb[rt][ks], s[rt], 0, 0, 0);
        beside(ks);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Phase 3 / 4: O^T += V^T P^T over the 32 keys of tile kt (key steps ku = 2kt, 2kt + 1) for
// both row tiles.  Step st = (ku, dt) with dt fastest; V^T fragments (rows 32kt + 16(ku&1) +
// 0..7 and + 8..15 of d tile dt, through the transposing read) are read PV steps ahead.
template <int D, typename Beside>
__device__ __forceinline__ void output_tile(f32x16 (&o)[TileShape<D>::DT][kRT], const uint32_t (&wd)[kRT][8], int kt,
                                            uint32_t sv, Beside&& beside) {
    using F = TileShape<D>;
    constexpr int NST = 2 * F::DT, PV = 2;
    i16x4 vlo[PV], vhi[PV];
    auto read_v = [&](int st, i16x4& lo, i16x4& hi) {
        const int dt = st % F::DT, j = st / F::DT;
        const int R = 32 * kt + 16 * j;
        lo = lds_tr4((sv ^ tr_x<D>(dt, R)) + R * 2 * D);
        hi = lds_tr4((sv ^ tr_x<D>(dt, R + 8)) + (R + 8) * 2 * D);
    };
    bf16x8 pb[kRT][2];
#pragma unroll
    for (int rt = 0; rt < kRT; rt++)
#pragma unroll
        for (int j = 0; j < 2; j++)
            pb[rt][j] = __builtin_bit_cast(bf16x8, u32x4{wd[rt][4 * j], wd[rt][4 * j + 1], wd[rt][4 * j + 2],
                                                         wd[rt][4 * j + 3]});
#pragma unroll
    for (int j = 0; j < PV; j++) read_v(j, vlo[j], vhi[j]);
#pragma unroll
    for (int st = 0; st < NST; st++) {
        const int dt = st % F::DT, j = st / F::DT;
        const bf16x8 va =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[st % PV], vhi[st % PV], 0, 1, 2, 3, 4, 5, 6, 7));
        if (st + PV < NST) read_v(st + PV, vlo[st % PV], vhi[st % PV]);
        mfma32_agpr2(o[dt][0], va, pb[0][j], o[dt][1], va, pb[1][j]);
        beside(st);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Blocks (query tile, part, kv head), dealt to the XCDs as deal_block() orders them; the query
// tiles of each member (pre-step scoring runs several members at once) are numbered
// member-major, n_qtiles_m per member.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kW * 64, kW * 64), amdgpu_waves_per_eu(1, 1)))
void fwd_mfma_kernel(AttnArgs a, int n_qtiles_m, int n_qtiles) {
    using F = TileShape<D>;
    using Tiles = KeyTiles<D, kW>;
    constexpr int PW = Tiles::PER_WAVE;
    __shared__ __attribute__((aligned(1024))) FwdLds<D> L;

    const XcdBlock blk = deal_block(blockIdx.x, n_qtiles, a.n_shards, a.n_parts, a.hkv);
    if (blk.qtile_g < 0) return;
    const int member = blk.qtile_g / n_qtiles_m;
    const int qtile = blk.qtile_g % n_qtiles_m;
    const int part = blk.part;
    const int kvh = blk.kvh;
    const bool resp = part == a.n_shards;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int n = lane & 31;
    const int64_t rows_total = a.n_rows * a.g;
    const int64_t r0 = (int64_t)qtile * kBM;
    const int64_t tok_base = (int64_t)member * a.n_rows;  // the member's first row in q
    const int64_t out_row0 = a.row0 + tok_base;            // ... and in the parts arrays

    // keys of this part; pages from t_mask on need a mask (a partial last page, or response keys
    // past the first row's causal limit)
    const int64_t lp0 = resp ? 0 : a.shard_lo[part];
    int64_t n_tiles, t_mask;
    if (!resp) {
        n_tiles = a.shard_lo[part + 1] - a.shard_lo[part];
        const int64_t keys = a.prefix_len - lp0 * kPage;
        t_mask = keys < n_tiles * kPage ? n_tiles - 1 : n_tiles;
    } else {
        int64_t tok_max = (r0 + kBM - 1) / a.g;
        if (tok_max > a.n_rows - 1) tok_max = a.n_rows - 1;
        n_tiles = (a.q_start + tok_max + 1 + kPage - 1) / kPage;
        t_mask = (a.q_start + r0 / a.g + 1) / kPage;  // first page with a key past the first row's limit
    }
    const int nt = __builtin_amdgcn_readfirstlane((int)n_tiles);
    const int tm = __builtin_amdgcn_readfirstlane((int)t_mask);
    const Tiles kt(a, resp, lp0, kvh, w, lane, (int64_t)member * a.resp_member_elems * 2);

    clear_lds(&L.kb[0][0], sizeof(L.kb), threadIdx.x, kW * 64);
    clear_lds(&L.vb[0][0], sizeof(L.vb), threadIdx.x, kW * 64);
    lds_barrier();

    // this lane's rows: 32rt + n of the wave's 64; rows past the block (a partial last tile)
    // read a valid row, and their output is never stored
    auto lane_row = [&](int rt) {
        const int64_t row = r0 + 64 * w + 32 * rt + n;
        return row < rows_total ? row : rows_total - 1;
    };
    bf16x8 qb[kRT][F::KS];
#pragma unroll
    for (int rt = 0; rt < kRT; rt++) {
        const int64_t row = lane_row(rt);
        const int64_t tok = row / a.g;
        const int head = kvh * a.g + (int)(row % a.g);
        const bf16_t* qrow = (const bf16_t*)a.q + ((tok_base + tok) * a.hq + head) * (int64_t)D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < F::KS; ks++) qb[rt][ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * ks));
    }
    // Wait for the Q loads here, with the wait the compiler sees (vmcnt(0), no other counter):
    // otherwise it guards Q's first uses inside the page loop on every page, and those waits
    // would also wait for the page copies, which share the counter but which it does not see.
    __builtin_amdgcn_s_waitcnt(0x0F70);

    float m_ref[kRT] = {-INFINITY, -INFINITY}, l[kRT] = {0.f, 0.f};
    f32x16 o[F::DT][kRT];
#pragma unroll
    for (int dt = 0; dt < F::DT; dt++)
#pragma unroll
        for (int rt = 0; rt < kRT; rt++) {
            o[dt][rt] = f32x16{};
            asm volatile("" : "+a"(o[dt][rt]));  // the accumulators live in AGPRs
        }

    const uint32_t kb0 = lds_addr(L.kb[0]), vb0 = lds_addr(L.vb[0]);
    // Copy j of this wave's share of a tile: 1 KiB block j * kW + w, rows j * JROWS + low.  The
    // lane's byte offset is (base ^ chunk constant) + row constant, since the swizzle is linear
    // over xor and the row part leaves the chunk bits alone.
    constexpr int RPK = Tiles::RPK, JROWS = Tiles::JROWS;
    const int low = w * RPK + lane / F::KCH;
    const uint32_t cp_base = (uint32_t)low * kt.row_bytes + ((uint32_t)((lane % F::KCH) ^ swz<D>(low)) << 4);
    auto copy_piece = [&](const char* src, int valid_rows, uint32_t lds, int j) {
        const uint32_t off = (cp_base ^ ((uint32_t)swz<D>(j * JROWS) << 4)) + (uint32_t)(j * JROWS) * kt.row_bytes;
        dma16(src, kt.bytes_of(valid_rows), off, lds + (j * kW + w) * 1024);
    };
    // page-table entries are read through the scalar cache a page before their copies
    auto entry = [&](int i) { return i < nt ? kt.entry(i) : 0; };
    if (nt > 0) {
        const int32_t e0 = entry(0);
#pragma unroll
        for (int j = 0; j < PW; j++) {
            copy_piece(kt.tile(e0, 0, false), kt.valid(0), kb0, j);
            copy_piece(kt.tile(e0, 0, true), kt.valid(0), vb0, j);
        }
    }
    int32_t e_next = entry(1);

    for (int t = 0; t < nt; t++) {
        const uint32_t kcur = kb0 + (uint32_t)(t & 1) * F::TILE, vcur = vb0 + (uint32_t)(t & 1) * F::TILE;
        const uint32_t knext = kb0 + (uint32_t)((t + 1) & 1) * F::TILE, vnext = vb0 + (uint32_t)((t + 1) & 1) * F::TILE;
        // the next page's copies; past the last page they repeat it into the free buffer
        const int tn = t + 1 < nt ? t + 1 : nt - 1;
        const int32_t e_cp = t + 1 < nt ? e_next : entry(tn);
        const char* ksrc = kt.tile(e_cp, tn, false);
        const char* vsrc = kt.tile(e_cp, tn, true);
        const int vn = kt.valid(tn);
        e_next = entry(t + 2);
        wait_vm_all();
        lds_barrier();  // page t is in LDS; every wave is done with page t - 1's buffers

        const bool masked = t >= tm;
        const int valid = kt.valid(t);
        // the row's causal limit relative to the page's first key (response keys; else all)
        int causal[kRT] = {kPage, kPage};
        // Lane-dependent values are re-formed from an opaque lane id each page rather than held
        // (or spilled) across the loop: every register is taken by Q, S, P and the fragments.
        int ln = __lane_id();
        asm volatile("" : "+v"(ln));
        if (masked && resp) {
            int64_t d = a.q_start - (int64_t)t * kPage;
            d = d < -(1 << 30) ? -(1 << 30) : (d > (1 << 30) ? (1 << 30) : d);
#pragma unroll
            for (int rt = 0; rt < kRT; rt++) {
                int64_t row = r0 + 64 * w + 32 * rt + (ln & 31);
                row = row < rows_total ? row : rows_total - 1;
                causal[rt] = (int)d + (int)(row / a.g);
            }
        }
        const LaneAddr<D> la(ln);
        const uint32_t lk = la.k, lv = la.v;

        f32x16 s0[kRT], s1[kRT];
        uint32_t wd0[kRT][8], wd1[kRT][8];
        SmState st0, st1;
        st0.mx[0] = st0.mx[1] = st1.mx[0] = st1.mx[1] = -INFINITY;

        // 1: scores of keys 0-31, the next page's copies beside
        score_tile<D>(s0, qb, kcur + lk, [&](int ks) {
            if (ks < PW) copy_piece(ksrc, vn, knext, ks);
            else if (ks < 2 * PW) copy_piece(vsrc, vn, vnext, ks - PW);
        });
        if (masked) {
#pragma unroll
            for (int rt = 0; rt < kRT; rt++) mask_tile(s0[rt], 0, valid, causal[rt], ln >> 5);
        }
        // 2: scores of keys 32-63, the softmax of keys 0-31 beside
        score_tile<D>(s1, qb, kcur + lk + 32 * 2 * D, [&](int ks) {
#pragma unroll
            for (int u = ks * kSmUnits / F::KS; u < (ks + 1) * kSmUnits / F::KS; u++)
                sm_unit(u, s0, st0, m_ref, l, wd0, a.scale_log2);
        });
        if (masked) {
#pragma unroll
            for (int rt = 0; rt < kRT; rt++) mask_tile(s1[rt], 1, valid, causal[rt], ln >> 5);
        }
        // 3: output over keys 0-31 (after any rescale the softmax of keys 0-31 asked for), the
        // softmax of keys 32-63 beside
        rescale_o<F::DT>(o, st0.alpha);
        output_tile<D>(o, wd0, 0, vcur + lv, [&](int step) {
#pragma unroll
            for (int u = step * kSmUnits / (2 * F::DT); u < (step + 1) * kSmUnits / (2 * F::DT); u++)
                sm_unit(u, s1, st1, m_ref, l, wd1, a.scale_log2);
        });
        // 4: output over keys 32-63
        rescale_o<F::DT>(o, st1.alpha);
        output_tile<D>(o, wd1, 1, vcur + lv, [&](int) {});
    }
    wait_vm_all();  // the last copies land before the workgroup's LDS is released
    mfma_drain();

    // LSE and the normalised output of each row tile
#pragma unroll
    for (int rt = 0; rt < kRT; rt++) {
        const float l_tot = l[rt] + other_half(l[rt]);
        const int64_t row = r0 + 64 * w + 32 * rt + n;
        if (row >= rows_total) continue;
        const int64_t orow = ((int64_t)part * a.part_rows + out_row0 + row / a.g) * a.hq + kvh * a.g + row % a.g;
        // l_tot is 0 exactly when the row sees no key of the part (LSE -inf, O 0); a NaN in the
        // row's inputs leaves it NaN, and NaN is what the row's LSE and O then hold
        if (h == 0) a.lse_parts[orow] = l_tot != 0.f ? (m_ref[rt] + fast_log2(l_tot)) * kLn2 : -INFINITY;
        const float inv = l_tot != 0.f ? 1.f / l_tot : 0.f;
        float* dst = a.o_parts + orow * (int64_t)D;
#pragma unroll
        for (int dt = 0; dt < F::DT; dt++) {
            f32x16 v = o[dt][rt];
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                const int dd = dt * 32 + 8 * q4 + 4 * h;
                *(float4*)(dst + dd) = make_float4(v[4 * q4] * inv, v[4 * q4 + 1] * inv, v[4 * q4 + 2] * inv,
                                                   v[4 * q4 + 3] * inv);
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
    fwd_mfma_kernel<D><<<grid, kW * 64, 0, s>>>(a, (int)n_qtiles_m, (int)n_qtiles);
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
