// Split-prefix replay-attention forward on gfx950 bf16 matrix cores: one wave per SIMD, 64
// query rows per wave (32 for small blocks).
//
// One workgroup handles 256 query rows (128 for blocks under 512 group rows) of one kv head's
// group against the keys of one part (a prompt shard walked through the page table, or the
// response keys the rows see) and writes the part's normalised output and LSE, the owner-local
// statistics that the merge composes into the exact result (LongStraw digest, "Method", Qwen
// implementation; explainer, "Two incompatible architectures, same transaction").
//
// Each of the four waves owns RT = 2 (or 1) 32-row tiles and keeps their Q (the B operands of
// S^T = K Q^T, RT x D/4 registers) and their O^T accumulators (AGPRs) for the whole part.
// With two tiles every operand fragment read from LDS feeds two matrix instructions, one per
// row tile: a K fragment (32 keys x 16 d) both tiles' scores, a V^T fragment (32 d x 16 keys)
// both tiles' outputs.  P never leaves the registers: keys are permuted inside each 16-key step
// identically on both operands of O^T += V^T P^T, so the score accumulators are, once
// exponentiated and packed, already the B operand.
//
// A page (64 keys) runs in four phases of D/16 steps, each step one operand fragment and RT
// matrix instructions:
//   1  S^T of keys 0-31                     beside: the copies of the next page
//   2  S^T of keys 32-63                    beside: the softmax of keys 0-31
//   3  O^T += V^T P^T over keys 0-31        beside: the softmax of keys 32-63
//   4  O^T += V^T P^T over keys 32-63       beside: the page's row sums
// so the vector work of each half-page's softmax issues while the matrix core runs the other
// half's products.  The fragments are read two steps ahead across the phase boundaries.  K and
// V pages are double-buffered in LDS (one barrier per page).
//
// The softmax keeps one running reference m per row and moves it only when a half-page's
// maximum exceeds it by more than kLazyLog2 (base 2), so probabilities stay below 2^kLazyLog2
// and the output is almost never rescaled; when it is, O is scaled in place (in the AGPRs)
// after the products already taken relative to the old reference, before any taken relative
// to the new one.  Every term and the sum are relative to the same m, so the result is the
// same softmax.  The row sums add the bf16 words of P that the products use, so the weights O
// is normalised by are exactly those it summed.
#include <math.h>

#include <type_traits>

#include "mfma_tiles.hpp"

namespace ls {
namespace {

constexpr float kLazyLog2 = 8.f;
constexpr int kW = 4;  // waves per workgroup, one per SIMD
// RT (template parameter below) is the number of 32-row tiles per wave: 2 (256 rows per
// workgroup), or 1 (128 rows) for small blocks, which 256-row tiles would mostly pad
// (fwd_tile_rows, shared with the host's sub-range split).

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
// kLazyLog2; units 9-16 exponentiate and pack four scores of each row tile.  The row sums are
// taken later from the packed words (row_sums), beside matrix work that has no vector work of
// its own.
constexpr int kSmUnits = 17;

template <int RT>
struct SmState {
    float mx[RT], alpha[RT], m_use[RT];
};

// Each unit ends by pinning its results with an empty asm statement: without it, the compiler
// sinks the exponentials into the block that first uses them (past the rescale branch, into the
// next phase), where no matrix work hides them.
template <int RT>
__device__ __forceinline__ void sm_unit(int u, const f32x16 (&s)[RT], SmState<RT>& st, float (&m_ref)[RT],
                                        float (&l)[RT], uint32_t (&wd)[RT][8], float scale_log2) {
    if (u < 8) {
#pragma unroll
        for (int rt = 0; rt < RT; rt++) {
            st.mx[rt] = max3f(st.mx[rt], s[rt][2 * u], s[rt][2 * u + 1]);
            asm volatile("" : "+v"(st.mx[rt]));
        }
    } else if (u == 8) {
#pragma unroll
        for (int rt = 0; rt < RT; rt++) {
            // max on raw scores: scale_log2 > 0 commutes with max
            const float mx = __builtin_elementwise_maximum(st.mx[rt], other_half(st.mx[rt])) * scale_log2;
            st.alpha[rt] = 1.f;
            if (mx > m_ref[rt] + kLazyLog2) {  // false for a fully masked tile (mx = -inf) and for NaN
                // while the row has seen nothing its O and sum are exactly 0: nothing to rescale
                st.alpha[rt] = m_ref[rt] == -INFINITY ? 1.f : fast_exp2(m_ref[rt] - mx);
                m_ref[rt] = mx;
            }
            st.m_use[rt] = m_ref[rt] == -INFINITY ? 0.f : m_ref[rt];
            asm volatile("" : "+v"(st.alpha[rt]), "+v"(st.m_use[rt]), "+v"(m_ref[rt]));
        }
    } else {
        const int j = u - 9;
#pragma unroll
        for (int rt = 0; rt < RT; rt++) {
            const float p0 = fast_exp2(__builtin_fmaf(s[rt][2 * j], scale_log2, -st.m_use[rt]));
            const float p1 = fast_exp2(__builtin_fmaf(s[rt][2 * j + 1], scale_log2, -st.m_use[rt]));
            wd[rt][j] = pack_bf16x2(p0, p1);
            asm volatile("" : "+v"(wd[rt][j]));
        }
    }
}

// The row sums of one page: l = (l alpha0 + sum P0) alpha1 + sum P1, in the order the
// reference moved, from the bf16 words the products used (v_dot2c_f32_bf16 against (1, 1), one
// instruction per pair), so the weights O is normalised by are exactly those it summed.
template <int RT>
__device__ __forceinline__ void row_sums(float (&l)[RT], const uint32_t (&wd0)[RT][8], const uint32_t (&wd1)[RT][8],
                                         const SmState<RT>& st0, const SmState<RT>& st1, int step, int n_steps) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const bf16x2v one = {(__bf16)1.f, (__bf16)1.f};
    // 2 x RT chains of 8 words, spread over the steps; each chain starts from its scaled l
#pragma unroll
    for (int c = step * 2 * RT / n_steps; c < (step + 1) * 2 * RT / n_steps; c++) {
        const int half = c / RT, rt = c % RT;
        const uint32_t(&wd)[RT][8] = half ? wd1 : wd0;
        float acc = l[rt] * (half ? st1.alpha[rt] : st0.alpha[rt]);
#pragma unroll
        for (int j = 0; j < 8; j++) acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, wd[rt][j]), one, acc, false);
        l[rt] = acc;
        asm volatile("" : "+v"(l[rt]));
    }
}

// O *= alpha per row (the lane's row of each row tile), in place in the AGPRs, if any row's
// reference moved.  The products that used the old reference must have retired first.
template <int DT, int RT>
__device__ __forceinline__ void rescale_o(f32x16 (&o)[DT][RT], const float (&alpha)[RT]) {
    bool same = true;
#pragma unroll
    for (int rt = 0; rt < RT; rt++) same = same && alpha[rt] == 1.f;
    if (__all(same)) return;
    mfma_drain();
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int i = 0; i < 16; i++) o[dt][rt][i] = agpr_scaled(o[dt][rt][i], alpha[rt]);
    agpr_write_gap();
}

// The LDS operand fragments of one page, as one stream over its four phases of NS = D/16 steps
// each: step i of phase 0 / 1 reads the K fragment of keys 32kt.. (kt = phase) at d step i
// (natural read); step i = (j, dt) of phase 2 / 3 reads the V^T fragment of d tile dt and keys
// 32kt + 16j + 0..15 (two transposing reads, the key order permuted inside the 16 as on P).
// The page is walked with the stream read PF steps ahead across the phase boundaries, so only
// the first read after the page's barrier is waited for.
template <int D>
struct PageFrags {
    static constexpr int NS = TileShape<D>::KS;  // steps per phase (= 2 * DT)
    uint32_t ak, sv;                             // lane bases of this page's K and V tiles
    __device__ __forceinline__ bf16x8 read(int step) const {
        const int ph = step / NS, i = step % NS;
        if (ph < 2) {
            uint32_t b = ak;  // formed per read (one xor) rather than held as 2 * NS addresses
            asm volatile("" : "+v"(b));
            return lds_b128((b + ph * 32 * 2 * D) ^ (uint32_t)(i << 5));
        }
        const int dt = i % TileShape<D>::DT, R = 32 * (ph - 2) + 16 * (i / TileShape<D>::DT);
        const i16x4 lo = lds_tr4((sv ^ tr_x<D>(dt, R)) + R * 2 * D);
        const i16x4 hi = lds_tr4((sv ^ tr_x<D>(dt, R + 8)) + (R + 8) * 2 * D);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// P^T operands of one 32-key tile: key steps j = 0, 1 of both row tiles, from the packed words.
template <int RT>
__device__ __forceinline__ void p_operands(bf16x8 (&pb)[RT][2], const uint32_t (&wd)[RT][8]) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int j = 0; j < 2; j++)
            pb[rt][j] =
                __builtin_bit_cast(bf16x8, u32x4{wd[rt][4 * j], wd[rt][4 * j + 1], wd[rt][4 * j + 2], wd[rt][4 * j + 3]});
}

// Blocks (query tile, part, kv head), dealt to the XCDs as deal_block() orders them; the query
// tiles of each member (pre-step scoring runs several members at once) are numbered
// member-major, n_qtiles_m per member.
template <int D, int RT>
__global__ __attribute__((amdgpu_flat_work_group_size(kW * 64, kW * 64), amdgpu_waves_per_eu(1, 1)))
void fwd_mfma_kernel(AttnArgs a, int n_qtiles_m, int n_qtiles) {
    constexpr int kRT = RT;
    constexpr int kBM = 32 * RT * kW;  // query rows per workgroup
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
        const int64_t row = r0 + 32 * kRT * w + 32 * rt + n;
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

    float m_ref[kRT], l[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; rt++) {
        m_ref[rt] = -INFINITY;
        l[rt] = 0.f;
    }
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
    auto copy_piece = [&](const i32x4& rsrc, uint32_t lds, int j) {
        const uint32_t off = (cp_base ^ ((uint32_t)swz<D>(j * JROWS) << 4)) + (uint32_t)(j * JROWS) * kt.row_bytes;
        dma16r(rsrc, off, lds + (j * kW + w) * 1024);
    };
    // page-table entries are read through the scalar cache a page before their copies
    auto entry = [&](int i) { return i < nt ? kt.entry(i) : 0; };
    if (nt > 0) {
        const int32_t e0 = entry(0);
        const i32x4 rk = buffer_rsrc(kt.tile(e0, 0, false), kt.bytes_of(kt.valid(0)));
        const i32x4 rv = buffer_rsrc(kt.tile(e0, 0, true), kt.bytes_of(kt.valid(0)));
#pragma unroll
        for (int j = 0; j < PW; j++) {
            copy_piece(rk, kb0, j);
            copy_piece(rv, vb0, j);
        }
    }
    int32_t e_next = entry(1);

    // One page; MASKED (pages from tm on) adds the masks.  The pages before tm run without any
    // mask code, so the hot loop carries neither its branches nor its registers.
    auto page = [&](int t, auto mtag) {
        constexpr bool MASKED = decltype(mtag)::value;
        const uint32_t kcur = kb0 + (uint32_t)(t & 1) * F::TILE, vcur = vb0 + (uint32_t)(t & 1) * F::TILE;
        const uint32_t knext = kb0 + (uint32_t)((t + 1) & 1) * F::TILE, vnext = vb0 + (uint32_t)((t + 1) & 1) * F::TILE;
        // the next page's copies; past the last page they repeat it into the free buffer
        const int tn = t + 1 < nt ? t + 1 : nt - 1;
        const int32_t e_cp = t + 1 < nt ? e_next : entry(tn);
        const int vn = kt.valid(tn);
        const i32x4 rk = buffer_rsrc(kt.tile(e_cp, tn, false), kt.bytes_of(vn));
        const i32x4 rv = buffer_rsrc(kt.tile(e_cp, tn, true), kt.bytes_of(vn));
        e_next = entry(t + 2);
        wait_vm_all();
        lds_barrier();  // page t is in LDS; every wave is done with page t - 1's buffers

        const int valid = kt.valid(t);
        // the row's causal limit relative to the page's first key (response keys; else all)
        int causal[kRT];
#pragma unroll
        for (int rt = 0; rt < kRT; rt++) causal[rt] = kPage;
        // Lane-dependent values are re-formed from an opaque lane id each page rather than held
        // (or spilled) across the loop: every register is taken by Q, S, P and the fragments.
        int ln = __lane_id();
        asm volatile("" : "+v"(ln));
        if (MASKED && resp) {
            int64_t d = a.q_start - (int64_t)t * kPage;
            d = d < -(1 << 30) ? -(1 << 30) : (d > (1 << 30) ? (1 << 30) : d);
#pragma unroll
            for (int rt = 0; rt < kRT; rt++) {
                int64_t row = r0 + 32 * kRT * w + 32 * rt + (ln & 31);
                row = row < rows_total ? row : rows_total - 1;
                causal[rt] = (int)d + (int)(row / a.g);
            }
        }
        const LaneAddr<D> la(ln);
        const uint32_t lk = la.k, lv = la.v;

        f32x16 s0[kRT], s1[kRT];
        uint32_t wd0[kRT][8], wd1[kRT][8];
        bf16x8 pb[kRT][2];
        SmState<kRT> st0, st1;
#pragma unroll
        for (int rt = 0; rt < kRT; rt++) st0.mx[rt] = st1.mx[rt] = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < kRT; rt++) s0[rt] = s1[rt] = f32x16{};

        // The page in four phases (see the top of the file), one step = one fragment feeding two
        // matrix instructions and a share of the phase's vector or copy work:
        //   0  S^T of keys 0-31             beside: the next page's copies
        //   1  S^T of keys 32-63            beside: the softmax of keys 0-31
        //   2  O^T += V^T P^T, keys 0-31    beside: the softmax of keys 32-63
        //   3  O^T += V^T P^T, keys 32-63   beside: the page's row sums
        constexpr int NS = PageFrags<D>::NS, PF = 2;
        const PageFrags<D> pg{kcur + lk, vcur + lv};
        bf16x8 fb[PF];
#pragma unroll
        for (int j = 0; j < PF; j++) fb[j] = pg.read(j);
        // step `step` of the page (phase step / NS): its fragment, the next read, its matrix
        // instructions and its share of the phase's other work
        auto one_step = [&](int step) {
            const int ph = step / NS, i = step % NS;
            const bf16x8 f = fb[step % PF];
            if (step + PF < 4 * NS) fb[step % PF] = pg.read(step + PF);
            if (ph == 0) {
#pragma unroll
                for (int rt = 0; rt < kRT; rt++) s0[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qb[rt][i], s0[rt], 0, 0, 0);
                // the copy's LDS base passes through an empty asm so that the 2 * PW bases are
                // formed one by one rather than all held in scalar registers across the phase
                uint32_t kn = knext, vnx = vnext;
                asm volatile("" : "+s"(kn), "+s"(vnx));
                if (i < PW) copy_piece(rk, kn, i);
                else if (i < 2 * PW) copy_piece(rv, vnx, i - PW);
            } else if (ph == 1) {
#pragma unroll
                for (int rt = 0; rt < kRT; rt++) s1[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qb[rt][i], s1[rt], 0, 0, 0);
#pragma unroll
                for (int u = i * kSmUnits / NS; u < (i + 1) * kSmUnits / NS; u++)
                    sm_unit(u, s0, st0, m_ref, l, wd0, a.scale_log2);
            } else {
                const int dt = i % F::DT, j = i / F::DT;
                if constexpr (kRT == 2) mfma32_agpr2(o[dt][0], f, pb[0][j], o[dt][1], f, pb[1][j]);
                else mfma32_agpr(o[dt][0], f, pb[0][j]);
                if (ph == 2) {
#pragma unroll
                    for (int u = i * kSmUnits / NS; u < (i + 1) * kSmUnits / NS; u++)
                        sm_unit(u, s1, st1, m_ref, l, wd1, a.scale_log2);
                } else {
                    row_sums(l, wd0, wd1, st0, st1, i, NS);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        // each phase is its own loop (a loop over the whole page is too large to be unrolled),
        // with the masks and rescales between them; the reads run ahead across the boundaries
#pragma unroll
        for (int step = 0; step < NS; step++) one_step(step);
        if constexpr (MASKED) {
#pragma unroll
            for (int rt = 0; rt < kRT; rt++) mask_tile(s0[rt], 0, valid, causal[rt], ln >> 5);
        }
#pragma unroll
        for (int step = NS; step < 2 * NS; step++) one_step(step);
        if constexpr (MASKED) {
#pragma unroll
            for (int rt = 0; rt < kRT; rt++) mask_tile(s1[rt], 1, valid, causal[rt], ln >> 5);
        }
        rescale_o<F::DT>(o, st0.alpha);  // any move the softmax of keys 0-31 made
        p_operands(pb, wd0);
#pragma unroll
        for (int step = 2 * NS; step < 3 * NS; step++) one_step(step);
        rescale_o<F::DT>(o, st1.alpha);  // any move the softmax of keys 32-63 made
        p_operands(pb, wd1);
#pragma unroll
        for (int step = 3 * NS; step < 4 * NS; step++) one_step(step);
    };
    const int t_split = tm < nt ? tm : nt;
    int t = 0;
    for (; t < t_split; t++) page(t, std::false_type{});
    for (; t < nt; t++) page(t, std::true_type{});
    wait_vm_all();  // the last copies land before the workgroup's LDS is released
    mfma_drain();

    // LSE and the normalised output of each row tile
#pragma unroll
    for (int rt = 0; rt < kRT; rt++) {
        const float l_tot = l[rt] + other_half(l[rt]);
        const int64_t row = r0 + 32 * kRT * w + 32 * rt + n;
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

template <int D, int RT>
hipError_t launch_rt(const AttnArgs& a, hipStream_t s) {
    constexpr int BM = 32 * RT * kW;
    const int64_t n_qtiles_m = (a.n_rows * a.g + BM - 1) / BM;
    const int64_t n_qtiles = n_qtiles_m * a.n_members;
    const int64_t n_blocks = n_qtiles * a.n_parts * a.hkv;
    if (n_blocks == 0) return hipSuccess;
    const int grid = deal_grid(n_qtiles, a.n_shards, a.n_parts, a.hkv);
    KernelTimer kt("fwd_mfma", s);
    fwd_mfma_kernel<D, RT><<<grid, kW * 64, 0, s>>>(a, (int)n_qtiles_m, (int)n_qtiles);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
    static_assert(32 * 1 * kW == 128 && 32 * 2 * kW == 256, "fwd_tile_rows names these tiles");
    return fwd_tile_rows(a.n_rows * a.g) == 128 ? launch_rt<D, 1>(a, s) : launch_rt<D, 2>(a, s);
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
