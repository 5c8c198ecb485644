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

struct TileSrc {
    const bf16_t* k;
    const bf16_t* v;
    int64_t stride;  // elements between consecutive key rows
    int valid;       // rows [0, valid) hold keys; the rest repeat the last valid row
    int64_t key0;    // first key: logical prompt token, or response position
};

// Physical page of tile t of a prompt part (clamped so that a bad table cannot fault).
__device__ __forceinline__ int32_t phys_page(const AttnArgs& a, int part, int64_t t) {
    int32_t phys = a.table[a.shard_lo[part] + t];
    return phys < 0 ? 0 : (phys >= a.n_phys ? (int32_t)(a.n_phys - 1) : phys);
}

// Scalar pieces of tile t of a part starting at logical page lp0 (prompt) or key 0 (response):
// its physical page, base pointer of K or V, row stride and number of valid rows.
__device__ __forceinline__ int32_t page_phys(const AttnArgs& a, bool resp, int64_t lp0, int64_t t) {
    if (resp) return 0;
    const int32_t phys = a.table[lp0 + t];
    return phys < 0 ? 0 : (phys >= a.n_phys ? (int32_t)(a.n_phys - 1) : phys);
}

// Raw page-table entry of tile t of a prompt part (0 for response tiles), read through the
// scalar cache: the table is never written while a kernel runs.  Clamp it with clamp_phys()
// where it is used, so that the load's latency is not waited for where it is issued.
__device__ __forceinline__ int32_t page_entry(const AttnArgs& a, bool resp, int64_t lp0, int64_t t) {
    if (resp) return 0;
    const __attribute__((address_space(4))) int32_t* tab = (const __attribute__((address_space(4))) int32_t*)a.table;
    return tab[lp0 + t];
}

// A physical page index that is always inside the pool (a bad table cannot fault).
__device__ __forceinline__ int32_t clamp_phys(const AttnArgs& a, int32_t phys) {
    return phys < 0 ? 0 : (phys >= a.n_phys ? (int32_t)(a.n_phys - 1) : phys);
}

template <int D>
__device__ __forceinline__ const bf16_t* tile_ptr(const AttnArgs& a, bool resp, int64_t lp0, int64_t t, int32_t phys,
                                                  int kvh, bool v) {
    if (!resp) return (const bf16_t*)(v ? a.v_pages : a.k_pages) + ((int64_t)phys * a.hkv + kvh) * kPage * D;
    return (const bf16_t*)(v ? a.v_resp : a.k_resp) + (t * kPage * a.hkv + kvh) * D;
}

template <int D>
__device__ __forceinline__ int64_t tile_stride(const AttnArgs& a, bool resp) {
    return resp ? (int64_t)a.hkv * D : D;
}

__device__ __forceinline__ int tile_valid(const AttnArgs& a, bool resp, int64_t lp0, int64_t t) {
    const int64_t left = resp ? a.key_end - t * kPage : a.prefix_len - (lp0 + t) * kPage;
    return left < kPage ? (int)left : kPage;
}

// Source of tile t of a part; `phys` is its physical page (prompt parts only).
__device__ __forceinline__ TileSrc part_tile(const AttnArgs& a, bool resp, int part, int kvh,
                                             int64_t t, int32_t phys) {
    TileSrc s;
    if (!resp) {
        const int64_t lp = a.shard_lo[part] + t;
        const int64_t off = ((int64_t)phys * a.hkv + kvh) * kPage * a.d;
        s.k = (const bf16_t*)a.k_pages + off;
        s.v = (const bf16_t*)a.v_pages + off;
        s.stride = a.d;
        s.key0 = lp * kPage;
        const int64_t left = a.prefix_len - s.key0;
        s.valid = left < kPage ? (int)left : kPage;
    } else {
        s.key0 = t * kPage;
        const int64_t off = (s.key0 * a.hkv + kvh) * a.d;
        s.k = (const bf16_t*)a.k_resp + off;
        s.v = (const bf16_t*)a.v_resp + off;
        s.stride = (int64_t)a.hkv * a.d;
        const int64_t left = a.key_end - s.key0;
        s.valid = left < kPage ? (int)left : kPage;
    }
    return s;
}

// Direct-to-LDS copy of ROWS full rows (D bf16 each, rows `stride` elements apart) from two
// sources a, b into two LDS tiles, by all NW waves together.  Wave w's j-th copy fills 1 KiB
// block j*NW + w of a tile, i.e. RPK = 512/D whole rows; lane l writes 16-byte slot l of the
// block, so it fetches the logical chunk that the swizzle puts there.  `w` must be
// wave-uniform.
template <int D, int NW, int ROWS>
__device__ __forceinline__ void dma_rows(const bf16_t* a, const bf16_t* b, int64_t stride, char* lds_a,
                                         char* lds_b, int w, int lane) {
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
        const uint32_t off = (uint32_t)(low * (int)stride + lc * 8) * 2u;
        const int64_t rowj = (int64_t)(j * JROWS) * stride * 2;
        const int blk = j * NW + w;
        dma16((const char*)a + rowj + off, (LS_LDS void*)(lds_a + blk * 1024));
        dma16((const char*)b + rowj + off, (LS_LDS void*)(lds_b + blk * 1024));
    }
}

// Copy one 64-row tile from one source (K or V of a page, or 64 response keys) into LDS;
// rows past `valid` repeat the last valid row (finite, masked later).
template <int D, int NW>
__device__ __forceinline__ void issue_one(const bf16_t* src, int64_t stride, int valid, char* lds, int w,
                                          int lane) {
    using F = TileShape<D>;
    constexpr int RPK = 512 / D;
    constexpr int PER_WAVE = F::TILE / 1024 / NW;
    constexpr int JROWS = NW * RPK;
    const int low = w * RPK + lane / F::KCH;
    const int pc = lane % F::KCH;
    const int lane_x = pc ^ swz<D>(low);
    if (valid == kPage) {
#pragma unroll
        for (int j = 0; j < PER_WAVE; j++) {
            const int lc = lane_x ^ swz<D>(j * JROWS);
            const uint32_t off = (uint32_t)(low * (int)stride + lc * 8) * 2u;
            const int64_t rowj = (int64_t)(j * JROWS) * stride * 2;
            dma16((const char*)src + rowj + off, (LS_LDS void*)(lds + (j * NW + w) * 1024));
        }
    } else {
#pragma unroll
        for (int j = 0; j < PER_WAVE; j++) {
            const int r = j * JROWS + low;
            const int lc = lane_x ^ swz<D>(j * JROWS);
            const int rs = r < valid ? r : valid - 1;
            const uint32_t off = (uint32_t)(rs * (int)stride + lc * 8) * 2u;
            dma16((const char*)src + off, (LS_LDS void*)(lds + (j * NW + w) * 1024));
        }
    }
}

// Issue the direct-to-LDS copies of one K and one V page tile (all waves together).
template <int D, int NW>
__device__ __forceinline__ void issue_tile(const TileSrc& s, char* lds_k, char* lds_v, int w,
                                           int lane) {
    using F = TileShape<D>;
    if (s.valid == kPage) {
        dma_rows<D, NW, kPage>(s.k, s.v, s.stride, lds_k, lds_v, w, lane);
        return;
    }
    // a partial tile: rows past `valid` repeat the last valid row (finite, masked later)
    constexpr int RPK = 512 / D;
    constexpr int PER_WAVE = F::TILE / 1024 / NW;
    constexpr int JROWS = NW * RPK;
    const int low = w * RPK + lane / F::KCH;
    const int pc = lane % F::KCH;
    const int lane_x = pc ^ swz<D>(low);
#pragma unroll
    for (int j = 0; j < PER_WAVE; j++) {
        const int r = j * JROWS + low;
        const int lc = lane_x ^ swz<D>(j * JROWS);
        const int rs = r < s.valid ? r : s.valid - 1;
        const uint32_t off = (uint32_t)(rs * (int)s.stride + lc * 8) * 2u;
        const int blk = j * NW + w;
        dma16((const char*)s.k + off, (LS_LDS void*)(lds_k + blk * 1024));
        dma16((const char*)s.v + off, (LS_LDS void*)(lds_v + blk * 1024));
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

}  // namespace ls
