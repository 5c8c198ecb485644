// Tiles of keys (prompt pages or response positions) staged in LDS for the bf16
// matrix-core kernels, and the per-lane LDS addressing of their operands.
//
// A tile is 64 rows x D bf16 (one page of one kv head, or 64 consecutive response keys,
// or 64 query rows).  In LDS, 16-byte chunk c of row r holds logical chunk c ^ swz(r)
// (below), which spreads both operand read patterns over the banks.  Tiles are filled by
// direct global->LDS copies (16 bytes per lane, 1 KiB per wave instruction).
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace ls {

template <int D>
struct TileShape {
    static constexpr int KCH = D / 8;                        // 16-byte chunks per row
    static constexpr int KS = D / 16;                        // k-steps of S over d
    static constexpr int DT = D / 32;                        // 32-wide d tiles of O
    static constexpr int TILE = kPage * D * 2;               // bytes of one K or V page tile
};

// LDS swizzle: 16-byte chunk c of tile row r is stored at chunk c ^ swz(r).  swz is a bit
// permutation of the row's low bits (so swz(a ^ b) = swz(a) ^ swz(b)) chosen so that
//  - the 16 rows of one half of a natural operand read (32 rows, one chunk) hit 16 distinct
//    bank groups, and
//  - a transposed read (4 consecutive rows x 4 consecutive chunks per 32 lanes) hits 16
//    distinct bank groups.
template <int D>
__host__ __device__ constexpr int swz(int r) {
    return TileShape<D>::KCH >= 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : (((r & 1) << 2) | ((r >> 1) & 3));
}

// The key tiles of one part (a prompt shard: logical pages lp0.., walked through the page
// table; or the response keys as 64-key "virtual pages"), with everything that does not change
// from page to page computed once per workgroup, so that a page costs one page-table entry,
// a few scalar operations and PER_WAVE direct-to-LDS copies per tile.
//
// Wave w's j-th copy fills 1 KiB block j*NW + w of an LDS tile, i.e. RPK = 512/D whole rows
// starting at row j*JROWS + low; lane l writes 16-byte slot l of the block, so it fetches the
// logical chunk that the swizzle puts there (swz is linear over xor and low < JROWS, a power
// of two, so the chunk index splits into a lane part and a j part).
template <int D, int NW>
struct KeyTiles {
    using F = TileShape<D>;
    static constexpr int RPK = 512 / D;
    static constexpr int PER_WAVE = F::TILE / 1024 / NW;
    static constexpr int JROWS = NW * RPK;
    static_assert(PER_WAVE * NW * 1024 == F::TILE, "a tile must split evenly over the waves");

    const char* kbase;      // K of this kv head: physical page 0 (prompt) or response key 0
    const char* vbase;
    int64_t tile_bytes;     // bytes between physical pages (prompt) or 64-key tiles (response)
    const __attribute__((address_space(4))) int32_t* table;  // entries from logical page lp0 on
    int64_t keys;           // keys of the part counted from tile 0
    int32_t n_phys;
    uint32_t row_bytes;     // bytes between key rows inside a tile
    bool resp;
    uint32_t off[PER_WAVE]; // this lane's byte offset in a full tile, copy j

    // resp_off: bytes from the response keys of the launch to those of this workgroup's member
    __device__ __forceinline__ KeyTiles(const AttnArgs& a, bool resp_, int64_t lp0, int kvh, int w, int lane,
                                        int64_t resp_off = 0) {
        resp = resp_;
        n_phys = (int32_t)a.n_phys;
        if (!resp) {
            kbase = (const char*)a.k_pages + (int64_t)kvh * kPage * D * 2;
            vbase = (const char*)a.v_pages + (int64_t)kvh * kPage * D * 2;
            tile_bytes = (int64_t)a.hkv * kPage * D * 2;
            row_bytes = D * 2;
            keys = a.prefix_len - lp0 * kPage;
        } else {
            kbase = (const char*)a.k_resp + resp_off + (int64_t)kvh * D * 2;
            vbase = (const char*)a.v_resp + resp_off + (int64_t)kvh * D * 2;
            tile_bytes = (int64_t)kPage * a.hkv * D * 2;
            row_bytes = (uint32_t)a.hkv * D * 2;
            keys = a.key_end;
        }
        table = (const __attribute__((address_space(4))) int32_t*)a.table + (resp ? 0 : lp0);
        const int low = w * RPK + lane / F::KCH;      // first row of this lane's copies
        const int lane_x = (lane % F::KCH) ^ swz<D>(low);
#pragma unroll
        for (int j = 0; j < PER_WAVE; j++)
            off[j] = (uint32_t)(j * JROWS + low) * row_bytes + (uint32_t)((lane_x ^ swz<D>(j * JROWS)) << 4);
    }

    // Raw page-table entry of tile t (scalar load; 0 for the response).  Clamp it with tile()
    // where it is used, so that the load's latency is not waited for where it is issued.
    __device__ __forceinline__ int32_t entry(int64_t t) const { return resp ? 0 : table[t]; }

    // Base of tile t of K (v = false) or V; `raw` is entry(t).  A bad table entry is clamped
    // into the pool, so it cannot fault.
    __device__ __forceinline__ const char* tile(int32_t raw, int64_t t, bool v) const {
        const int32_t phys = raw < 0 ? 0 : (raw >= n_phys ? n_phys - 1 : raw);
        return (v ? vbase : kbase) + (resp ? t : (int64_t)phys) * tile_bytes;
    }

    // Rows of tile t that hold keys of the part.
    __device__ __forceinline__ int valid(int64_t t) const {
        const int64_t left = keys - t * kPage;
        return left < kPage ? (int)left : kPage;
    }

    // Bytes of a tile's source that hold its valid_rows (>= 1) keys.  Copies of rows past them
    // fall outside the copy's buffer range and read as zero; the kernels also clear their key
    // buffers once at the start (clear_lds), so those rows are finite either way (masked by the
    // caller).
    __device__ __forceinline__ uint32_t bytes_of(int valid_rows) const {
        return (uint32_t)(valid_rows - 1) * row_bytes + D * 2;
    }

    // Copy j (0 <= j < PER_WAVE) of this wave's share of one tile, so that a caller can spread
    // a tile's copies over its compute steps.
    __device__ __forceinline__ void copy_piece(const char* src, int valid_rows, uint32_t lds, int w, int j) const {
        dma16(src, bytes_of(valid_rows), off[j], lds + (j * NW + w) * 1024);
    }

    // Copy one tile into LDS (all NW waves together).
    __device__ __forceinline__ void copy(const char* src, int valid_rows, uint32_t lds, int w) const {
#pragma unroll
        for (int j = 0; j < PER_WAVE; j++) copy_piece(src, valid_rows, lds, w, j);
    }
};

// Zero `bytes` (a multiple of 16) of LDS from p, by all `nthreads` threads of the workgroup;
// the caller puts a barrier between this and any copy into the same memory.
__device__ __forceinline__ void clear_lds(char* p, int bytes, int tid, int nthreads) {
    for (int i = tid * 16; i < bytes; i += nthreads * 16) *(LS_LDS u32x4*)((LS_LDS char*)p + i) = u32x4{0, 0, 0, 0};
}

// Direct-to-LDS copy of ROWS full rows (D bf16 each, rows `stride` elements apart) from two
// sources a, b into two LDS tiles, by all NW waves together.  Wave w's j-th copy fills 1 KiB
// block j*NW + w of a tile, i.e. RPK = 512/D whole rows; lane l writes 16-byte slot l of the
// block, so it fetches the logical chunk that the swizzle puts there.  `w` must be
// wave-uniform.
template <int D, int NW, int ROWS>
__device__ __forceinline__ void dma_rows(const bf16_t* a, const bf16_t* b, int64_t stride, uint32_t lds_a,
                                         uint32_t lds_b, int w, int lane) {
    using F = TileShape<D>;
    constexpr int RPK = 512 / D;                 // rows per 1 KiB block
    constexpr int PER_WAVE = ROWS * D * 2 / 1024 / NW;
    constexpr int JROWS = NW * RPK;              // rows advanced per j (a power of two)
    static_assert(PER_WAVE * NW * 1024 == ROWS * D * 2, "tile must split evenly over the waves");
    const int low = w * RPK + lane / F::KCH;     // row inside the j-th group of JROWS rows
    const int pc = lane % F::KCH;                // 16-byte slot inside the row
    const int lane_x = pc ^ swz<D>(low);
#pragma unroll
    for (int j = 0; j < PER_WAVE; j++) {
        const int lc = lane_x ^ swz<D>(j * JROWS);
        const uint32_t off = (uint32_t)((j * JROWS + low) * (int)stride + lc * 8) * 2u;
        const uint32_t bytes = (uint32_t)((ROWS - 1) * stride + D) * 2u;
        const int blk = j * NW + w;
        dma16(a, bytes, off, lds_a + blk * 1024);
        dma16(b, bytes, off, lds_b + blk * 1024);
    }
}

// Per-lane LDS byte offsets inside a tile.  Splitting the row and chunk of every operand read
// into lane-fixed and step-varying parts turns its address into (lane base ^ constant) +
// constant, because swz is linear over xor.
//  - natural reads (an MFMA operand whose contraction runs along a row): lane reads row
//    lane%32 (+32kt), chunk 2ks + lane/32:  (k ^ (ks << 5)) + 32kt * 2D;
//  - transposed reads (ds_read_b64_tr_b16; contraction down the rows): for rows R + 0..7
//    (R a multiple of 8) and 32-wide d tile dt:  (v ^ tr_x(dt, R)) + R * 2D.
template <int D>
struct LaneAddr {
    uint32_t k;
    uint32_t v;
    __device__ __forceinline__ LaneAddr(int lane) {
        const int h = lane >> 5, n = lane & 31;
        k = n * 2 * D + ((h ^ swz<D>(n)) << 4);
        const int G = lane >> 4, i16 = lane & 15;
        const int c_lane = 4 * (G >> 1) + (i16 >> 2);          // row within an 8-row group
        const int l_lane = 2 * (G & 1) + ((i16 & 3) >> 1);     // chunk within a 32-wide d tile
        const int half8 = (i16 & 1) * 8;                       // byte inside the 16-byte chunk
        v = c_lane * 2 * D + half8 + ((l_lane ^ swz<D>(c_lane)) << 4);
    }
};

// xor constant of a transposed read of rows R.. (R % 8 == 0) in d tile dt
template <int D>
__host__ __device__ constexpr uint32_t tr_x(int dt, int R) {
    return (uint32_t)(((4 * dt) ^ swz<D>(R)) << 4);
}

// Blocks (query tile, part, kv head) of the matrix-core kernels that walk a part's keys for a
// tile of query rows (the forward, the dQ passes).
//
// Only one block fits on a compute unit, and a prompt-shard block runs for thousands of pages
// while a response-part block runs for a few, so the order in which blocks reach the XCDs
// decides the balance.  The hardware deals block ids round-robin to the eight XCDs; each XCD
// takes an equal, contiguous run of the prompt-shard blocks (kv head, shard, query tile
// order: the query tiles that read the same pages share that XCD's L2) and then an equal run
// of the response-part blocks, which fill in behind the long ones.  Padding ids return.
struct XcdBlock {
    int qtile_g, part, kvh;  // qtile_g < 0: padding
};

__device__ __forceinline__ XcdBlock deal_block(int b, int n_qtiles, int n_shards, int n_parts, int hkv) {
    const int x = b % kXcds, slot = b / kXcds;
    const int n_long = n_qtiles * n_shards * hkv;
    const int lq = n_long / kXcds, lr = n_long % kXcds;
    const int cnt_l = lq + (x < lr ? 1 : 0);
    if (slot < cnt_l) {
        const int item = x * lq + (x < lr ? x : lr) + slot;
        return {item % n_qtiles, (item / n_qtiles) % n_shards, item / (n_qtiles * n_shards)};
    }
    // short runs are dealt from the other end, so that the XCDs holding an extra long block
    // are the last to hold an extra short one
    const int n_rp = n_parts - n_shards;
    const int n_short = n_qtiles * n_rp * hkv;
    const int xr = kXcds - 1 - x;
    const int sq = n_short / kXcds, sr = n_short % kXcds;
    const int s2 = slot - cnt_l;
    if (s2 >= sq + (xr < sr ? 1 : 0)) return {-1, 0, 0};
    const int item = xr * sq + (xr < sr ? xr : sr) + s2;
    return {item % n_qtiles, n_shards + (item / n_qtiles) % n_rp, item / (n_qtiles * n_rp)};
}

inline int deal_grid(int64_t n_qtiles, int n_shards, int n_parts, int hkv) {
    const int64_t n_long = n_qtiles * n_shards * hkv, n_short = n_qtiles * (n_parts - n_shards) * hkv;
    return (int)(kXcds * ((n_long + kXcds - 1) / kXcds + (n_short + kXcds - 1) / kXcds));
}

}  // namespace ls
