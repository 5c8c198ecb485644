// Fused replay-attention forward and dQ pass, for a dO that is known before the forward, on
// gfx950 bf16 matrix cores.
//
// The exact attention of a response row (LongStraw explainer, "Two incompatible architectures,
// same transaction": the owners' softmax statistics compose into the exact global output)
// and the gradient of sum(O * dO) with respect to its query:
//   dQ_i = scale sum_j P_ij (dP_ij - delta_i) K_j,  dP_ij = dO_i . V_j,
//   delta_i = dO_i . O_i = sum_j P_ij dP_ij.
// delta is only known once every key has been seen, so one pass over the keys keeps, per row
// and relative to the online softmax's running reference m (p_ij = exp(s_ij - m)),
//   O~ = sum p V,  A = sum p dP K,  B = sum p K,  l = sum p,  delta~ = sum p dP,
// all rescaled together when m moves.  Then O = O~ / l, delta = delta~ / l and
// dQ = scale (A / l - delta B / l).  Each of O~ / l, A / l, B / l and delta~ / l is an average
// under the part's softmax, so parts merge exactly as O does: weighted by exp(LSE_p - LSE).
// The kernel writes them per part (prompt shards and the response part, as the forward), the
// LSE merge composes O and the LSE, and fwd_dq_merge_kernel composes dQ.
//
// Registers decide the shape.  Three d-wide fp32 accumulators per row (O~, A, B) at d = 256
// leave room for 16 rows per wave, so the products are v_mfma_f32_16x16x32_bf16 (a 16-key by
// 16-row score tile, a 16-d by 16-row accumulator tile).  A workgroup of 4 waves takes 64 group
// rows of one kv head against one part; K and V pages are double-buffered in LDS.  Per page:
//   S^T = K Q^T and dP^T = V dO^T  (K, V natural reads; Q and dO in registers)
//   the softmax of the page's 64 keys (one reference move at most)
//   O~^T += V^T P^T, A^T += K^T (P o dP)^T, B^T += K^T P^T  (V^T, K^T transposed reads)
// Keys are permuted inside each 32-key step identically on both operands of the accumulating
// products, so the score accumulators, exponentiated and packed, are already their B operands:
// lane group G (lanes 16G..16G+15) holds keys 4G..4G+3 of the step's two 16-key score tiles.
#include <math.h>

#include "mfma_tiles.hpp"

namespace ls {
namespace {

constexpr int kFW = 4;               // waves per workgroup, one per SIMD
constexpr int kFRows = 16;           // query rows per wave
constexpr int kFBM = kFW * kFRows;   // query rows per workgroup
constexpr float kFLazyLog2 = 8.f;    // the reference moves when a page's maximum exceeds it by this
constexpr int kPF = 3;               // operand fragments read this many steps ahead

template <int D>
struct FdqLds {
    char kb[2][TileShape<D>::TILE];
    char vb[2][TileShape<D>::TILE];
};

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc += A B with the accumulator held in AGPRs (the score accumulators, which vector code
// reads, stay in VGPRs).  As for mfma32_agpr (common.hpp): the compiler does not see this as a
// matrix instruction, so the two wait states ahead of it cover a vector-ALU write of A or B just
// before it, a chain on one accumulator needs none, and mfma_drain() comes before anything reads
// the accumulator.
__device__ __forceinline__ void mfma16_agpr(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// The four lanes n, n + 16, n + 32, n + 48 hold one row: maximum (NaN-propagating) and sum.
__device__ __forceinline__ float row4_max(float x) {
    x = __builtin_elementwise_maximum(x, __shfl_xor(x, 16, 64));
    return __builtin_elementwise_maximum(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float row4_sum(float x) {
    x += __shfl_xor(x, 16, 64);
    return x + __shfl_xor(x, 32, 64);
}

struct FdqOut {
    float* a_parts;      // [n_parts, n_rows, hq, d]  A / l per part
    float* b_parts;      // [n_parts, n_rows, hq, d]  B / l per part
    float* delta_parts;  // [n_parts, n_rows, hq]     delta~ / l per part
};

// Blocks (64-row query tile, part, kv head), dealt to the XCDs by deal_block().
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kFW * 64, kFW * 64), amdgpu_waves_per_eu(1, 1)))
void fwd_dq_mfma_kernel(AttnArgs a, FdqOut out, int n_qtiles) {
    using F = TileShape<D>;
    using Tiles = KeyTiles<D, kFW>;
    constexpr int KS = D / 32;  // 32-wide steps of the score products over d
    constexpr int DT = D / 16;  // 16-wide d tiles of the accumulators
    __shared__ __attribute__((aligned(1024))) FdqLds<D> L;

    const XcdBlock blk = deal_block(blockIdx.x, n_qtiles, a.n_shards, a.n_parts, a.hkv);
    if (blk.qtile_g < 0) return;
    const int part = blk.part, kvh = blk.kvh;
    const bool resp = part == a.n_shards;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, n16 = lane & 15;
    const int64_t rows_total = a.n_rows * a.g;
    const int64_t r0 = (int64_t)blk.qtile_g * kFBM;
    // this lane's row (n16 of the wave's 16); rows past the block read a valid row and are never
    // stored
    const int64_t row_raw = r0 + kFRows * w + n16;
    const bool row_ok = row_raw < rows_total;
    const int64_t row = row_ok ? row_raw : rows_total - 1;
    const int64_t tok = row / a.g;
    const int head = kvh * a.g + (int)(row % a.g);

    // keys of the part: a prompt shard's pages, or the response keys the tile's last row sees
    const int64_t lp0 = resp ? 0 : a.shard_lo[part];
    int64_t n_tiles;
    if (!resp) {
        n_tiles = a.shard_lo[part + 1] - lp0;
    } else {
        int64_t tok_max = (r0 + kFBM - 1) / a.g;
        if (tok_max > a.n_rows - 1) tok_max = a.n_rows - 1;
        n_tiles = (a.q_start + tok_max + 1 + kPage - 1) / kPage;
    }
    const int nt = __builtin_amdgcn_readfirstlane((int)n_tiles);
    const Tiles kt(a, resp, lp0, kvh, w, lane);

    clear_lds(&L.kb[0][0], sizeof(L.kb), threadIdx.x, kFW * 64);
    clear_lds(&L.vb[0][0], sizeof(L.vb), threadIdx.x, kFW * 64);

    // Q and dO of this lane's row, d = 32 ks + 8 G .. + 8: the B operands of the score products
    bf16x8 qf[KS], df[KS];
    {
        const int64_t off = (tok * a.hq + head) * (int64_t)D + 8 * G;
        const bf16_t* qrow = (const bf16_t*)a.q + off;
        const bf16_t* drow = (const bf16_t*)a.dout + off;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            qf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 32 * ks));
            df[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(drow + 32 * ks));
        }
    }
    // Wait for these loads here, with a wait the compiler sees: otherwise it guards their first
    // uses inside the page loop on every page, and those waits would also wait for the page
    // copies, which share the counter but which it does not see.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) only
    f32x4 oc[DT], ac[DT], bc[DT];  // element i of tile dt: d = 16 dt + 4 G + i of row n16
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
        oc[dt] = ac[dt] = bc[dt] = f32x4{};
        asm volatile("" : "+a"(oc[dt]), "+a"(ac[dt]), "+a"(bc[dt]));  // the accumulators live in AGPRs
    }
    agpr_write_gap();
    float m_ref = -INFINITY;  // the row's reference (log2 units), the same in its four lanes
    float l = 0.f, dl = 0.f;  // this lane's share of the row's l and delta~
    // the last response key the row sees (inclusive); prompt keys are all visible
    const int64_t causal_key = a.q_start + tok;

    const uint32_t kb0 = lds_addr(L.kb[0]), vb0 = lds_addr(L.vb[0]);
    __syncthreads();  // the cleared buffers, before any copy into them
    auto issue = [&](int t) {
        const int32_t e = kt.entry(t);
        const int v = kt.valid(t);
        const uint32_t buf = (uint32_t)(t & 1) * F::TILE;
        kt.copy(kt.tile(e, t, false), v, kb0 + buf, w);
        kt.copy(kt.tile(e, t, true), v, vb0 + buf, w);
    };
    if (nt > 0) issue(0);
    for (int t = 0; t < nt; t++) {
        wait_vm_all();
        // page t is in LDS for every wave, and every wave is done with page t - 1's buffers
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (t + 1 < nt) issue(t + 1);
        const uint32_t kc = kb0 + (uint32_t)(t & 1) * F::TILE, vc = vb0 + (uint32_t)(t & 1) * F::TILE;
        // Lane bases of the page's reads, formed each page from an opaque lane id rather than
        // held across the loop (every register is taken by the operands and accumulators).  The
        // tile swizzle (swz, mfma_tiles.hpp) is linear over xor and depends only on a row's low
        // four bits, so a read is (lane base ^ step constant) + row constant (the constant goes
        // into its immediate):
        //  natural, rows 16 kb + n16, chunk 4 ks + G:     (nat ^ (ks << 6)) + 32 kb D
        //  transposed, rows 32 js + 4 G + n16 / 4 (+16),
        //  elements 16 dt + 4 (n16 % 4):                  (tr ^ (dt << 5)) + 64 js D (+32 D)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lg = ln >> 4, ln16 = ln & 15, rq = 4 * lg + (ln16 >> 2);
        const uint32_t nat = (uint32_t)ln16 * (2 * D) + ((uint32_t)(lg ^ swz<D>(ln16)) << 4);
        const uint32_t tr = (uint32_t)rq * (2 * D) + ((uint32_t)(((ln16 & 3) >> 1) ^ swz<D>(rq)) << 4) + 8u * (ln16 & 1);

        // S^T and dP^T of the page's four 16-key tiles: element i of tile kb is key 16 kb + 4 G + i.
        // Step i = (ks, kb), kb fastest; its K and V fragments are read kPF steps ahead.
        constexpr int NS1 = 4 * KS;
        bf16x8 kfb[kPF + 1], vfb[kPF + 1];
        auto sread = [&](int i) {
            const uint32_t off = (nat ^ (uint32_t)((i / 4) << 6)) + (uint32_t)(32 * (i % 4) * D);
            kfb[i % (kPF + 1)] = lds_b128(kc + off);
            vfb[i % (kPF + 1)] = lds_b128(vc + off);
        };
#pragma unroll
        for (int i = 0; i < kPF; i++) sread(i);
        f32x4 s[4], dp[4];
#pragma unroll
        for (int kb = 0; kb < 4; kb++) s[kb] = dp[kb] = f32x4{};
#pragma unroll
        for (int i = 0; i < NS1; i++) {
            if (i + kPF < NS1) sread(i + kPF);
            const int ks = i / 4, kb = i % 4;
            s[kb] = mfma16(kfb[i % (kPF + 1)], qf[ks], s[kb]);
            dp[kb] = mfma16(vfb[i % (kPF + 1)], df[ks], dp[kb]);
            // the step's reads and products stay in place: hoisting every step's reads would need
            // more registers than the accumulators leave
            __builtin_amdgcn_sched_barrier(0);
        }

        // The accumulate phase's fragments: step i = (js, dt), dt fastest, four transposing reads
        // each (V^T and K^T, low and high rows); the first kPF are issued here so that the softmax
        // below runs while they are in flight.
        constexpr int NS2 = 2 * DT;
        i16x4 fr[kPF + 1][4];
        auto aread = [&](int i) {
            const uint32_t olo = (tr ^ (uint32_t)((i % DT) << 5)) + (uint32_t)(64 * (i / DT) * D), ohi = olo + 32 * D;
            i16x4(&f)[4] = fr[i % (kPF + 1)];
            f[0] = lds_tr4(vc + olo);
            f[1] = lds_tr4(vc + ohi);
            f[2] = lds_tr4(kc + olo);
            f[3] = lds_tr4(kc + ohi);
        };
#pragma unroll
        for (int i = 0; i < kPF; i++) aread(i);

        // keys past the part's end or past the row's causal limit
        const int valid = kt.valid(t);
        int lim = valid - 1;  // the last key of the page the row sees
        if (resp) {
            const int64_t c = causal_key - (int64_t)t * kPage;
            if (c < lim) lim = c < -1 ? -1 : (int)c;
        }
        if (lim < kPage - 1) {
#pragma unroll
            for (int kb = 0; kb < 4; kb++)
#pragma unroll
                for (int i = 0; i < 4; i++) s[kb][i] = (16 * kb + 4 * G + i) <= lim ? s[kb][i] : -INFINITY;
        }

        // the page's maximum; the reference moves (and everything is rescaled) only when the page
        // exceeds it by more than kFLazyLog2, so that p stays below 2^kFLazyLog2
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; kb++)
            mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(
                                                       __builtin_elementwise_maximum(s[kb][0], s[kb][1]),
                                                       __builtin_elementwise_maximum(s[kb][2], s[kb][3])));
        mx = row4_max(mx) * a.scale_log2;  // scale_log2 > 0 commutes with max
        float alpha = 1.f;
        if (mx > m_ref + kFLazyLog2) {  // false for a fully masked page (-inf) and for NaN
            alpha = m_ref == -INFINITY ? 1.f : fast_exp2(m_ref - mx);
            m_ref = mx;
        }
        if (__any(alpha != 1.f)) {
            // in place in the AGPRs, after the products taken relative to the old reference
            mfma_drain();
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    oc[dt][i] = agpr_scaled(oc[dt][i], alpha);
                    ac[dt][i] = agpr_scaled(ac[dt][i], alpha);
                    bc[dt][i] = agpr_scaled(bc[dt][i], alpha);
                }
            agpr_write_gap();
            l *= alpha;
            dl *= alpha;
        }
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;

        // p and p dP as the operands of the two 32-key steps: slots 0-3 keys 32 js + 4 G + i,
        // slots 4-7 keys 32 js + 16 + 4 G + i.  l adds the bf16 p the products use.
        bf16x8 pb[2], pdb[2];
#pragma unroll
        for (int js = 0; js < 2; js++) {
            uint32_t wp[4], wq[4];
#pragma unroll
            for (int hb = 0; hb < 2; hb++)
#pragma unroll
                for (int i2 = 0; i2 < 2; i2++) {
                    const f32x4& sv = s[2 * js + hb];
                    const f32x4& dv = dp[2 * js + hb];
                    const float p0 = fast_exp2(__builtin_fmaf(sv[2 * i2], a.scale_log2, -m_use));
                    const float p1 = fast_exp2(__builtin_fmaf(sv[2 * i2 + 1], a.scale_log2, -m_use));
                    const uint32_t wpp = pack_bf16x2(p0, p1);
                    l += __uint_as_float(wpp << 16) + __uint_as_float(wpp & 0xffff0000u);
                    const float q0 = p0 * dv[2 * i2], q1 = p1 * dv[2 * i2 + 1];
                    dl += q0 + q1;
                    wp[2 * hb + i2] = wpp;
                    wq[2 * hb + i2] = pack_bf16x2(q0, q1);
                }
            pb[js] = __builtin_bit_cast(bf16x8, (u32x4{wp[0], wp[1], wp[2], wp[3]}));
            pdb[js] = __builtin_bit_cast(bf16x8, (u32x4{wq[0], wq[1], wq[2], wq[3]}));
        }

        // O~^T += V^T P^T, A^T += K^T (P o dP)^T, B^T += K^T P^T.  The A operands are two
        // transposing reads each: lane n16 of group G gives the address of row 4 G + n16 / 4 (+16)
        // of the step and elements 16 dt + 4 (n16 % 4) .. + 4, and receives d = 16 dt + n16 of the
        // group's four rows.
#pragma unroll
        for (int i = 0; i < NS2; i++) {
            if (i + kPF < NS2) aread(i + kPF);
            const int js = i / DT, dt = i % DT;
            const i16x4(&f)[4] = fr[i % (kPF + 1)];
            const bf16x8 vt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(f[0], f[1], 0, 1, 2, 3, 4, 5, 6, 7));
            const bf16x8 kt8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(f[2], f[3], 0, 1, 2, 3, 4, 5, 6, 7));
            mfma16_agpr(oc[dt], vt, pb[js]);
            mfma16_agpr(ac[dt], kt8, pdb[js]);
            mfma16_agpr(bc[dt], kt8, pb[js]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_vm_all();  // the last copies land before the workgroup's LDS is released
    mfma_drain();   // the accumulators are read below

    l = row4_sum(l);
    dl = row4_sum(dl);
    if (!row_ok) return;
    const int64_t orow = ((int64_t)part * a.n_rows + tok) * a.hq + head;
    const float inv = l != 0.f ? 1.f / l : 0.f;  // l = 0: the row sees no key of the part
    if (G == 0) {
        a.lse_parts[orow] = l != 0.f ? (m_ref + fast_log2(l)) * kLn2 : -INFINITY;
        out.delta_parts[orow] = dl * inv;
    }
    float* po = a.o_parts + orow * D + 4 * G;
    float* pa = out.a_parts + orow * D + 4 * G;
    float* pbp = out.b_parts + orow * D + 4 * G;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
        *(f32x4*)(po + 16 * dt) = oc[dt] * inv;
        *(f32x4*)(pa + 16 * dt) = ac[dt] * inv;
        *(f32x4*)(pbp + 16 * dt) = bc[dt] * inv;
    }
}

// dQ of each (row, head) from the parts: with w_p = exp(LSE_p - LSE) (LSE the merged one),
// delta = sum_p w_p delta_p and dQ = scale (sum_p w_p A_p - delta sum_p w_p B_p).  Each thread
// owns 4 consecutive elements of one row.
__global__ __launch_bounds__(256) void fwd_dq_merge_kernel(int n_parts, int64_t n_rows, int d,
                                                           const float* __restrict__ lse_parts,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ a_parts,
                                                           const float* __restrict__ b_parts,
                                                           const float* __restrict__ delta_parts, float scale,
                                                           float* __restrict__ dq) {
    const int vecs = d / 4;
    const int rows_per_block = 256 / vecs;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / vecs;
    const int c = threadIdx.x % vecs;
    if (threadIdx.x >= rows_per_block * vecs || row >= n_rows) return;
    const float L = lse[row];
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    if (L != -INFINITY) {
        float delta = 0.f;
        for (int p = 0; p < n_parts; p++) {
            const float lp = lse_parts[(int64_t)p * n_rows + row];
            if (lp != -INFINITY) delta += expf(lp - L) * delta_parts[(int64_t)p * n_rows + row];
        }
        float4 sa = make_float4(0.f, 0.f, 0.f, 0.f), sb = sa;
        for (int p = 0; p < n_parts; p++) {
            const float lp = lse_parts[(int64_t)p * n_rows + row];
            if (lp == -INFINITY) continue;
            const float wgt = expf(lp - L);
            const float4 va = *reinterpret_cast<const float4*>(a_parts + ((int64_t)p * n_rows + row) * d + 4 * c);
            const float4 vb = *reinterpret_cast<const float4*>(b_parts + ((int64_t)p * n_rows + row) * d + 4 * c);
            sa.x += wgt * va.x; sa.y += wgt * va.y; sa.z += wgt * va.z; sa.w += wgt * va.w;
            sb.x += wgt * vb.x; sb.y += wgt * vb.y; sb.z += wgt * vb.z; sb.w += wgt * vb.w;
        }
        r = make_float4(scale * (sa.x - delta * sb.x), scale * (sa.y - delta * sb.y), scale * (sa.z - delta * sb.z),
                        scale * (sa.w - delta * sb.w));
    }
    *reinterpret_cast<float4*>(dq + row * d + 4 * c) = r;
}

template <int D>
hipError_t launch_fwd_dq_d(const AttnArgs& a, const FdqOut& out, hipStream_t s) {
    const int64_t n_qtiles = (a.n_rows * a.g + kFBM - 1) / kFBM;
    if (n_qtiles == 0 || a.n_parts == 0) return hipSuccess;
    const int grid = deal_grid(n_qtiles, a.n_shards, a.n_parts, a.hkv);
    KernelTimer kt("fwd_dq_mfma", s);
    fwd_dq_mfma_kernel<D><<<grid, kFW * 64, 0, s>>>(a, out, (int)n_qtiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_dq_mfma(const AttnArgs& a, float* a_parts, float* b_parts, float* delta_parts, hipStream_t s) {
    const FdqOut out{a_parts, b_parts, delta_parts};
    switch (a.d) {
        case 64: return launch_fwd_dq_d<64>(a, out, s);
        case 128: return launch_fwd_dq_d<128>(a, out, s);
        case 256: return launch_fwd_dq_d<256>(a, out, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fwd_dq_merge(int n_parts, int64_t n_rows, int d, const float* lse_parts, const float* lse,
                               const float* a_parts, const float* b_parts, const float* delta_parts, float scale,
                               float* dq, hipStream_t s) {
    if (n_rows == 0) return hipSuccess;
    const int rows_per_block = 256 / (d / 4);
    const unsigned grid = (unsigned)((n_rows + rows_per_block - 1) / rows_per_block);
    KernelTimer kt("fwd_dq_merge", s);
    fwd_dq_merge_kernel<<<grid, 256, 0, s>>>(n_parts, n_rows, d, lse_parts, lse, a_parts, b_parts, delta_parts, scale,
                                             dq);
    return hipGetLastError();
}

}  // namespace ls
