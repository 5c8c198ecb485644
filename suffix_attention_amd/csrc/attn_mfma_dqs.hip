// dQ pass of the replay-attention backward from the dS that the dK/dV pass stored.
//
// dQ = scale * sum over visible keys of dS K, with dS = P (dP - delta) formed by the
// key-stationary dK/dV pass (rounded to bf16 there, as its matrix instructions take it) and
// written out per (group row, key) pair.  Reading it back turns the dQ pass into a single
// contraction per pair, where recomputing needs three (S, dP and the dQ product itself).
// Pairs that the causal mask hides were stored as dS = 0, so nothing here is masked: a key row
// past the end of a partial page is zero in LDS (the copy's range stops at the last key), and
// its stored dS is finite, so it adds nothing.
//
// Blocks (256-row block of a kv head's group rows, part, kv head).  Wave w owns group rows
// 64w .. 64w + 63 of the block, i.e. two 32-row tiles, and keeps dQ^T (d x 64 rows, fp32) in
// AGPRs.  Per 64-key page, K is copied once into LDS for the workgroup and each wave copies its
// own two 4 KiB dS tiles, all by direct-to-LDS copies.  K^T is read transposed and feeds two
// matrix instructions (one per row tile); dS^T is read transposed once per 16-key step.
// Pipeline: K double-buffered, copied one page ahead; dS triple-buffered, copied two pages ahead
// (it comes from HBM, K mostly from L2).
#include "mfma_bwd.hpp"

namespace ls {
namespace {

constexpr int kDsTile = kPage * 32 * 2;  // bytes of one 32-row tile's dS over one page: 4 KiB
constexpr int kDsWave = 2 * kDsTile;     // one wave's two row tiles

// This lane's byte offset for a transposed read of a dS tile (rows = keys, 64 bytes of 32 bf16
// rows each, no swizzle): the 64 lanes read 8 key rows x 64 bytes, contiguously.  The lane
// pattern is the one LaneAddr::v uses for a 32-wide d tile.
__device__ __forceinline__ uint32_t ds_lane_off(int lane) {
    const int G = lane >> 4, i16 = lane & 15;
    const int c = 4 * (G >> 1) + (i16 >> 2);        // key row within an 8-row group
    const int l = 2 * (G & 1) + ((i16 & 3) >> 1);   // 16-byte chunk within the row
    return (uint32_t)(c * 64 + l * 16 + (i16 & 1) * 8);
}

template <int D>
struct DqsState {
    f32x16 dq[2][TileShape<D>::DT];  // dQ^T accumulators per row tile: col = stored position, rows = d
};

// One page: dQ^T[rt] += K^T dS^T[rt] for the wave's two row tiles.  kv: LDS address of the
// page's K tile plus the lane's transposed-read offset; dsb: LDS address of the wave's two dS
// tiles plus ds_lane_off.  Steps (ku, dt), dt fastest; K^T fragments read PV steps ahead, the
// dS^T fragments of the whole page first.  beside(st) runs after step st's matrix instructions.
template <int D, typename Beside>
__device__ __forceinline__ void dqs_page(DqsState<D>& st, uint32_t kv, uint32_t dsb, Beside&& beside) {
    using F = TileShape<D>;
    constexpr int NST = 4 * F::DT;
    constexpr int PV = 4;
    bf16x8 db[4][2];
#pragma unroll
    for (int ku = 0; ku < 4; ku++)
#pragma unroll
        for (int rt = 0; rt < 2; rt++) {
            const uint32_t b = dsb + rt * kDsTile + 16 * ku * 64;
            const i16x4 lo = lds_tr4(b), hi = lds_tr4(b + 8 * 64);
            db[ku][rt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    i16x4 tlo[PV], thi[PV];
    auto read_kt = [&](int st_, i16x4& lo, i16x4& hi) {
        const int dt = st_ % F::DT, ku = st_ / F::DT;
        const int R = 16 * ku;
        lo = lds_tr4((kv ^ tr_x<D>(dt, R)) + R * 2 * D);
        hi = lds_tr4((kv ^ tr_x<D>(dt, R + 8)) + (R + 8) * 2 * D);
    };
#pragma unroll
    for (int j = 0; j < PV; j++) read_kt(j, tlo[j], thi[j]);
#pragma unroll
    for (int st_ = 0; st_ < NST; st_++) {
        const int dt = st_ % F::DT, ku = st_ / F::DT;
        const bf16x8 ka = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tlo[st_ % PV], thi[st_ % PV], 0, 1, 2, 3, 4, 5, 6, 7));
        if (st_ + PV < NST) read_kt(st_ + PV, tlo[st_ % PV], thi[st_ % PV]);
        mfma32_agpr2(st.dq[0][dt], ka, db[ku][0], st.dq[1][dt], ka, db[ku][1]);
        beside(st_);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Run the units [n * k / steps, n * (k + 1) / steps) of n at step k, with constant loop bounds so
// that every unit index is a constant after unrolling.
template <int N, int STEPS, typename Fn>
__device__ __forceinline__ void units_at(int k, Fn&& f) {
#pragma unroll
    for (int un = 0; un < N; un++)
        if (un >= k * N / STEPS && un < (k + 1) * N / STEPS) f(un);
}

// Blocks (256-row block, part, kv head), dealt to the XCDs by deal_block(): every XCD gets an
// equal run of the long prompt-shard blocks, then of the short response-part blocks.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void dqs_mfma_kernel(AttnArgs a, int n_rblocks, int n_kvh, int part0, int n_sp, int n_rp) {
    using F = TileShape<D>;
    constexpr int NW = 4;
    constexpr int PW = KeyTiles<D, NW>::PER_WAVE;  // K copies per wave per page
    constexpr int PD = kDsWave / 1024;             // dS copies per wave per page
    constexpr int NST = 4 * F::DT;
    __shared__ __attribute__((aligned(1024))) char kbuf[2][F::TILE];
    __shared__ __attribute__((aligned(1024))) char dbuf[3][NW][kDsWave];

    const XcdBlock blk = deal_block(blockIdx.x, n_rblocks, n_sp, n_sp + n_rp, n_kvh);
    if (blk.qtile_g < 0) return;
    const int rblock = blk.qtile_g;
    const int part = blk.part < n_sp ? part0 + blk.part : a.n_shards;
    const int kvh = a.ds_kvh0 + blk.kvh;  // the stored dS holds kv heads from ds_kvh0 on
    const bool resp = part == a.n_shards;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int n = lane & 31;
    const int64_t rows_total = a.n_rows * a.g;
    const int64_t r0 = (int64_t)rblock * kDqsTileRows;
    const int64_t rt0 = r0 / 32 + 2 * w;  // the wave's first row tile

    // pages of the part: a prompt shard's pages, or the response pages up to the last key the
    // block's last row sees
    int64_t n_tiles;
    int64_t lp0 = 0, slot0;
    if (!resp) {
        lp0 = a.shard_lo[part];
        n_tiles = a.shard_lo[part + 1] - lp0;
        slot0 = lp0 * kPage - 128 * a.ds_pair0;  // the chunk's key slots start at its first page pair
    } else {
        int64_t tok_max = (r0 + 255) / a.g;
        if (tok_max > a.n_rows - 1) tok_max = a.n_rows - 1;
        n_tiles = (a.q_start + tok_max + 1 + kPage - 1) / kPage;
        slot0 = a.ds_resp_slot0;
    }
    const KeyTiles<D, NW> kt(a, resp, lp0, kvh, w, lane);
    // the wave's dS source: row tile rt0 (rt0 + 1 is ds_rt_bytes further), from key slot0 on
    const char* ds0 = (const char*)(a.ds + (((int64_t)blk.kvh * a.ds_rt + rt0) * a.ds_kslots + slot0) * 32);
    const int64_t ds_rt_bytes = a.ds_kslots * 64;
    // copy j of the wave's dS for page t: row tile j / 4, keys 16 (j % 4) .. +16 (1 KiB)
    auto ds_piece = [&](int64_t t, uint32_t dst, int j) {
        const char* src = ds0 + (j >> 2) * ds_rt_bytes + t * kDsTile;
        dma16(src, kDsTile, (uint32_t)((j & 3) * 1024 + lane * 16), dst + j * 1024);
    };

    DqsState<D> st;
#pragma unroll
    for (int rt = 0; rt < 2; rt++)
#pragma unroll
        for (int dt = 0; dt < F::DT; dt++) {
            st.dq[rt][dt] = f32x16{};
            asm volatile("" : "+a"(st.dq[rt][dt]));  // accumulators live in AGPRs
        }
    agpr_write_gap();

    const LaneAddr<D> la(lane);
    const uint32_t kb0 = lds_addr(kbuf[0]);
    const uint32_t db0 = lds_addr(dbuf[0][w]);
    constexpr uint32_t kDbStage = NW * kDsWave;
    const uint32_t dlo = ds_lane_off(lane);
    clear_lds(&kbuf[0][0], sizeof(kbuf), threadIdx.x, NW * 64);
    __syncthreads();
    if (n_tiles > 0) {
        // prologue: K(0), dS(0), dS(1) (the last page again if there is none: nothing reads it)
        const int32_t e0 = kt.entry(0);
        kt.copy(kt.tile(e0, 0, false), kt.valid(0), kb0, w);
#pragma unroll
        for (int j = 0; j < PD; j++) ds_piece(0, db0, j);
        const int64_t t1 = n_tiles > 1 ? 1 : 0;
#pragma unroll
        for (int j = 0; j < PD; j++) ds_piece(t1, db0 + kDbStage, j);
        int32_t e1 = n_tiles > 1 ? kt.entry(1) : e0;
        int kb = 0, dsb = 0;
        for (int64_t t = 0; t < n_tiles; t++) {
            // K(t) and dS(t) have landed (dS(t+1), issued after K(t), may still be in flight);
            // K buffer (t+1) % 2 and dS buffer (t+2) % 3 were last read in iteration t-1
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PD) : "memory");
            __syncthreads();
            const int32_t e2 = t + 2 < n_tiles ? kt.entry(t + 2) : 0;
            // copies beside the matrix steps: K(t+1) first, then dS(t+2), so that at the top of
            // the next iteration a wait leaving PD copies in flight covers K(t+1)
            const int64_t tk = t + 1 < n_tiles ? t + 1 : t;
            const int64_t td = t + 2 < n_tiles ? t + 2 : n_tiles - 1;
            const char* ksrc = kt.tile(e1, tk, false);
            const int vk = kt.valid(tk);
            const int kbn = kb ^ 1;
            const int dsn = dsb == 0 ? 2 : dsb - 1;  // (t + 2) % 3
            uint32_t kv = la.v;
            asm volatile("" : "+v"(kv));
            dqs_page<D>(st, kb0 + kb * F::TILE + kv, db0 + dsb * kDbStage + dlo, [&](int s_) {
                units_at<PW + PD, NST>(s_, [&](int p) {
                    if (p < PW) kt.copy_piece(ksrc, vk, kb0 + kbn * F::TILE, w, p);
                    else ds_piece(td, db0 + dsn * kDbStage, p - PW);
                });
            });
            kb = kbn;
            dsb = dsb == 2 ? 0 : dsb + 1;
            e1 = e2;
        }
        wait_vm_all();  // the last iterations' copies land before the workgroup's LDS is released
    }
    mfma_drain();

    // stored position p = n of row tile rt0 + rt is group row 32 (rt0 + rt) + ds_row_of(n);
    // element i of d tile dt is d = 32 dt + 8 (i / 4) + 4 h + i % 4
#pragma unroll
    for (int rt = 0; rt < 2; rt++) {
        const int64_t row = 32 * (rt0 + rt) + ds_row_of(n);
        if (row >= rows_total) continue;
        const int64_t tok = row / a.g;
        const int head = kvh * a.g + (int)(row % a.g);
        float* dst = a.dq_parts + (((int64_t)part * a.n_rows + tok) * a.hq + head) * (int64_t)D;
        if (a.owner && h == 0)  // debug run: this lane pair writes the row
            atomicAdd(a.owner + a.owner_dq0 + ((int64_t)part * a.n_rows + tok) * a.hq + head, 1u);
#pragma unroll
        for (int dt = 0; dt < F::DT; dt++) {
#pragma unroll
            for (int i = 0; i < 16; i++) st.dq[rt][dt][i] = agpr_scaled(st.dq[rt][dt][i], a.scale);
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                const int dd = dt * 32 + 8 * q4 + 4 * h;
                *(float4*)(dst + dd) = make_float4(st.dq[rt][dt][4 * q4], st.dq[rt][dt][4 * q4 + 1],
                                                   st.dq[rt][dt][4 * q4 + 2], st.dq[rt][dt][4 * q4 + 3]);
            }
        }
    }
}

template <int D>
hipError_t launch_dqs_d(const AttnArgs& a, int n_kvh, int part0, int n_sp, int n_rp, hipStream_t s) {
    const int64_t rows_total = a.n_rows * a.g;
    const int n_rblocks = (int)((rows_total + kDqsTileRows - 1) / kDqsTileRows);
    if (n_rblocks == 0 || n_kvh == 0 || n_sp + n_rp == 0) return hipSuccess;
    dqs_mfma_kernel<D><<<deal_grid(n_rblocks, n_sp, n_sp + n_rp, n_kvh), 256, 0, s>>>(a, n_rblocks, n_kvh, part0,
                                                                                      n_sp, n_rp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dqs_mfma(const AttnArgs& a, int n_kvh, int part0, int n_sp, bool resp, hipStream_t s) {
    KernelTimer kt("dqs_mfma", s);
    const int n_rp = resp ? 1 : 0;
    switch (a.d) {
        case 64: return launch_dqs_d<64>(a, n_kvh, part0, n_sp, n_rp, s);
        case 128: return launch_dqs_d<128>(a, n_kvh, part0, n_sp, n_rp, s);
        case 256: return launch_dqs_d<256>(a, n_kvh, part0, n_sp, n_rp, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ls
