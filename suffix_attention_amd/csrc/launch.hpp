// Internal interface between the C ABI front end (abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ls {

constexpr int kMaxShards = 64;     // prompt shards a caller may use
constexpr int kMaxSubParts = 256;  // key ranges a launch may split the prompt into (below)
constexpr int kDqsTileRows = 256;  // group rows per workgroup of the stored-dS dQ pass
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPage = 64;  // tokens per KV page

// Everything one replay-attention launch needs, passed by value to the kernels.
struct AttnArgs {
    // captured prompt (pages)
    const void* k_pages;
    const void* v_pages;
    const int32_t* table;
    int64_t prefix_len;
    int64_t n_logical_pages;
    int64_t n_phys;
    int hq, hkv, g, d;
    float scale;       // softmax scale
    float scale_log2;  // scale * log2(e)
    // response block: rows are response positions [q_start, q_start + n_rows)
    const void* q;
    const void* k_resp;
    const void* v_resp;
    int64_t n_rows;
    int64_t q_start;
    int64_t key_end;  // q_start + n_rows: response keys [0, key_end) are visible at most
    // parts: shard s = logical pages [shard_lo[s], shard_lo[s+1]); part n_shards = response
    int n_shards;
    int n_parts;
    int64_t shard_lo[kMaxSubParts + 1];
    // Pre-step scoring runs the blocks of n_members members in one forward (1 for a replay):
    // member m's rows follow member m-1's in q; its response keys start resp_member_elems
    // elements after member m-1's.
    int64_t n_members;
    int64_t resp_member_elems;
    // forward products; part p holds rows [p * part_rows, (p + 1) * part_rows), of which this
    // launch writes part_rows from row0 on (part_rows = n_members * n_rows, row0 = 0, unless a
    // host loop runs the members one launch at a time)
    int64_t part_rows;
    int64_t row0;
    float* o_parts;    // [n_parts, part_rows, hq, d]
    float* lse_parts;  // [n_parts, part_rows, hq]
    // backward
    const void* o;
    const void* dout;
    const float* lse;    // [n_rows, hq]
    const float* delta;  // [n_rows, hq]
    float* dq_parts;     // [n_parts, n_rows, hq, d]
    float* dk_pages;
    float* dv_pages;
    uint64_t first_touch_mask;  // bit s: shard s's gradient pages are written, not added to
    float* dk_resp;
    float* dv_resp;
    int resp_first_touch;
    // stored dS (bf16), or null: the dK/dV pass then also writes dS = P (dP - delta) of every
    // (group row, key) pair it forms, and the dQ pass reads it instead of recomputing S and dP.
    // Layout [hkv][ds_rt][ds_kslots][32] bf16: for kv head h, 32-row tile rt of its group rows
    // and key slot k, the 32 rows in the order of ds_row_of(); key slots are 128 per page pair,
    // prompt pairs first (slot = logical key), the response pairs from ds_resp_slot0 on.
    // When the workspace holds dS for only some kv heads, the backward runs in chunks of
    // ds_heads kv heads (dK/dV, then dQ, per chunk); ds_kvh0 is the first kv head of the chunk
    // being launched, and the stored dS is indexed by kv head - ds_kvh0.  When it holds less
    // than one kv head's dS over all keys, the chunks are one kv head by ds_parts consecutive
    // key parts (shards in order, then the response): a chunk's prompt page pairs start at
    // ds_pair0 (its key slot 0) and its response pairs, if it has the response part, at
    // ds_resp_slot0.
    uint16_t* ds;
    int64_t ds_rt;
    int64_t ds_kslots;
    int64_t ds_resp_slot0;
    int64_t ds_pair0;
    int ds_heads;
    int ds_parts;
    int ds_kvh0;
    // prompt pages [pg_lo, pg_hi) are the ones whose K/V gradients a dK/dV launch writes (all
    // logical pages, except in a chunk of key parts: the chunk's shards)
    int64_t pg_lo, pg_hi;
    // One-writer counters of a debug run (null: off).  Every writer of a gradient half-page or
    // of a dQ part row adds 1 to its slot: prompt half-pages at ((phys * hkv + kv) * 2 + half),
    // response half-pages from owner_resp0 on at ((page * hkv + kv) * 2 + half), dQ part rows
    // from owner_dq0 on at ((part * n_rows + token) * hq + head).
    uint32_t* owner;
    int64_t owner_resp0, owner_dq0;
    // The stored-dS dQ pass over shard sub-ranges (dq_sub_k > 1, a chunk over all key parts
    // only): its per-range dQ partials [n_shards * dq_sub_k + 1, n_rows, hq, d], summed instead
    // of dq_parts.
    float* dq_sub;
    int dq_sub_k;
    // The backward stops after dK/dV (the caller formed dQ elsewhere, e.g. in the fused
    // forward + dQ pass); no stored dS then.
    bool skip_dq;
};

// Sub-parts.  The forward and the stored-dS dQ pass run one workgroup per (query tile, part,
// kv head); a small block has few query tiles, so with the shards as parts most compute units
// would idle (a 16-row block at 8 shards and 4 kv heads: 36 workgroups for 256 compute units).
// Such a pass splits each shard into k contiguous page ranges, enough for about three
// workgroups per compute unit but at least 64 pages a range on average, and merges (forward)
// or sums (dQ) what the ranges give.
inline int sub_split(int64_t n_qtiles, int n_shards, int hkv, int64_t n_logical_pages) {
    constexpr int64_t kTarget = 3 * 256;
    const int64_t base = n_qtiles * n_shards * hkv;
    if (base <= 0 || base >= kTarget) return 1;
    int64_t k = (kTarget + base - 1) / base;
    const int64_t by_pages = n_logical_pages / ((int64_t)n_shards * 64);
    if (k > by_pages) k = by_pages;
    if (k > kMaxSubParts / n_shards) k = kMaxSubParts / n_shards;
    return k < 1 ? 1 : (int)k;
}
// Group rows per forward workgroup for a block (per member) of `group_rows`: 256 (two 32-row
// tiles per wave), or 128 (one) for blocks under 512 group rows, which 256-row tiles would
// mostly pad.
inline int fwd_tile_rows(int64_t group_rows) { return group_rows < 512 ? 128 : 256; }
inline int fwd_split(int64_t n_rows, int g, int n_shards, int hkv, int64_t n_logical_pages) {
    const int tr = fwd_tile_rows(n_rows * g);
    return sub_split((n_rows * g + tr - 1) / tr, n_shards, hkv, n_logical_pages);
}
inline int dqs_split(int64_t n_rows, int g, int n_shards, int hkv, int64_t n_logical_pages) {
    return sub_split((n_rows * g + kDqsTileRows - 1) / kDqsTileRows, n_shards, hkv, n_logical_pages);
}
// Page bounds of the k ranges of every shard: out[s * k + j] = lo[s] + (lo[s+1] - lo[s]) j / k,
// out[n_shards * k] = lo[n_shards] (ranges of a short shard may be empty).
inline void split_bounds(const int64_t* lo, int n_shards, int k, int64_t* out) {
    for (int s = 0; s < n_shards; s++)
        for (int j = 0; j < k; j++) out[s * k + j] = lo[s] + (lo[s + 1] - lo[s]) * j / k;
    out[n_shards * k] = lo[n_shards];
}

// Slots of the one-writer counters for a block of n_rows rows whose response keys end at key_end.
inline int64_t owner_resp0(int64_t n_phys, int hkv) { return n_phys * hkv * 2; }
inline int64_t owner_dq0(int64_t n_phys, int hkv, int64_t key_end) {
    return owner_resp0(n_phys, hkv) + (key_end + 63) / 64 * hkv * 2;
}
inline int64_t owner_slots(int64_t n_phys, int hkv, int hq, int n_dq_parts, int64_t n_rows, int64_t key_end) {
    return owner_dq0(n_phys, hkv, key_end) + (int64_t)n_dq_parts * n_rows * hq;
}

// Row (0..31) inside a 32-row tile of the stored-dS position p (0..31): the positions are in
// the order the dK/dV pass holds dS in its registers (lane half h = p / 16, key step
// u = (p / 8) % 2, word half hb = (p / 4) % 2).
__host__ __device__ constexpr int ds_row_of(int p) {
    return 16 * ((p >> 3) & 1) + 8 * ((p >> 2) & 1) + 4 * (p >> 4) + (p & 3);
}

// Stored-dS sizes for a block of rows_total group rows per kv head whose response keys end
// at key_end: row tiles cover the rows padded to 256 (the dQ pass's row block), key slots
// cover prompt and response pages rounded up to pairs (the dK/dV pass's unit).
inline int64_t ds_row_tiles(int64_t rows_total) { return (rows_total + 255) / 256 * 8; }
inline int64_t ds_key_slots(int64_t n_logical_pages, int64_t key_end, int64_t* resp_slot0) {
    const int64_t pp = (n_logical_pages + 1) / 2, rp = ((key_end + 63) / 64 + 1) / 2;
    if (resp_slot0) *resp_slot0 = 128 * pp;
    return 128 * (pp + rp);
}

// A chunk of consecutive key parts [p0, p1) (parts 0 .. n_shards - 1 are the prompt shards,
// part n_shards the response): its prompt pages [pg_lo, pg_hi), the page pairs that cover them
// (pairs are the dK/dV pass's unit; a pair cut by the chunk's edge is walked by both chunks, each
// writing only its own page), and its key slots (prompt pairs first, then the response pairs).
struct PartChunk {
    int p0, p1;
    int64_t pg_lo, pg_hi;      // prompt pages (pg_lo == pg_hi: none)
    int64_t pair_lo, n_pairs;  // prompt page pairs [pair_lo, pair_lo + n_pairs)
    bool resp;                 // the chunk holds the response part
    int64_t n_resp_pairs;
    int64_t slots() const { return 128 * (n_pairs + (resp ? n_resp_pairs : 0)); }
};

inline PartChunk part_chunk(const int64_t* shard_lo, int n_shards, int64_t key_end, int p0, int p1) {
    PartChunk c;
    c.p0 = p0;
    c.p1 = p1;
    const int s1 = p1 < n_shards ? p1 : n_shards;
    c.pg_lo = p0 < n_shards ? shard_lo[p0] : shard_lo[n_shards];
    c.pg_hi = p0 < n_shards ? shard_lo[s1] : c.pg_lo;
    c.pair_lo = c.pg_lo / 2;
    c.n_pairs = c.pg_hi > c.pg_lo ? (c.pg_hi + 1) / 2 - c.pair_lo : 0;
    c.resp = p1 > n_shards;
    c.n_resp_pairs = ((key_end + 63) / 64 + 1) / 2;
    return c;
}

// Key slots per kv head that the stored dS needs for chunks of `parts` consecutive key parts:
// the largest chunk's.
inline int64_t ds_chunk_slots(const int64_t* shard_lo, int n_shards, int64_t key_end, int parts) {
    int64_t m = 0;
    for (int p0 = 0; p0 < n_shards + 1; p0 += parts) {
        const int p1 = p0 + parts < n_shards + 1 ? p0 + parts : n_shards + 1;
        const int64_t sl = part_chunk(shard_lo, n_shards, key_end, p0, p1).slots();
        m = sl > m ? sl : m;
    }
    return m;
}

// Brackets one kernel launch with HIP events on its stream while profiling is on
// (ls_profile_begin / ls_profile_end); does nothing otherwise.
class KernelTimer {
  public:
    KernelTimer(const char* name, hipStream_t s);
    ~KernelTimer();
    KernelTimer(const KernelTimer&) = delete;
    KernelTimer& operator=(const KernelTimer&) = delete;

  private:
    const char* name_;
    hipStream_t stream_;
    hipEvent_t start_ = nullptr;
};

// Rows of one kv head's group are numbered r = token * g + j (query head kv * g + j).
// Key-range helpers shared by host launch code.
inline int64_t resp_tiles(int64_t key_end) { return (key_end + 63) / 64; }

// noalloc.hip: this device's fixed scratch array for ls_replay_fwd_noalloc (its device address,
// set up on the first call with this device current) and its size
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// capture.hip
hipError_t launch_capture(const void* k_src, const void* v_src, int src_dtype, int64_t n_tok,
                          int64_t first_tok, const int32_t* table, void* k_pages, void* v_pages,
                          int page_dtype, int64_t n_phys, int hkv, int d, hipStream_t s);
hipError_t launch_gather(const void* pages, int dtype, const int32_t* table, int64_t n_phys,
                         int64_t first_tok, int64_t n_tok, int hkv, int d, void* dst,
                         hipStream_t s);

// reduce.hip
hipError_t launch_lse_merge(int n_parts, int64_t n_rows, int d, const float* o_parts,
                            const float* lse_parts, void* o_out, int out_dtype, float* lse_out,
                            hipStream_t s, bool bf16_numerator = false);
hipError_t launch_delta(const void* o, const void* dout, int dtype, int64_t n_rows, int d,
                        float* delta, hipStream_t s);
hipError_t launch_sum_parts(int n_parts, int64_t n, const float* parts, float* out,
                            hipStream_t s);
hipError_t launch_zero(float* p, int64_t n, hipStream_t s);

// attn_generic.hip: LDS-tiled kernels on the vector ALUs (the exact float32 path)
hipError_t launch_fwd_generic(const AttnArgs& a, hipStream_t s);
hipError_t launch_bwd_generic(const AttnArgs& a, hipStream_t s);

// attn_mfma_fwd.hip / attn_mfma_bwd.hip: bf16 matrix-core kernels
hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t s);
// Fused forward + dQ for a dO known up front (a.dout): writes a.o_parts / a.lse_parts as the
// forward does, and per part A / l, B / l ([n_parts, n_rows, hq, d]) and delta~ / l
// ([n_parts, n_rows, hq]); launch_fwd_dq_merge then forms dQ from them and the merged LSE.
hipError_t launch_fwd_dq_mfma(const AttnArgs& a, float* a_parts, float* b_parts, float* delta_parts, hipStream_t s);
hipError_t launch_fwd_dq_merge(int n_parts, int64_t n_rows, int d, const float* lse_parts, const float* lse,
                               const float* a_parts, const float* b_parts, const float* delta_parts, float scale,
                               float* dq, hipStream_t s);
hipError_t launch_bwd_mfma(const AttnArgs& a, hipStream_t s);
// bytes the matrix-core backward keeps after the dQ parts: (LSE * log2 e, delta) float32 pairs
// and the bf16 Q and dO rows of every kv head's group, group-major and padded to a multiple of
// 64 rows
constexpr int kRowPad = 64;
inline int64_t rows_padded(int64_t rows) { return (rows + kRowPad - 1) / kRowPad * kRowPad; }
inline size_t mfma_bwd_extra_bytes(int64_t n_rows, int g, int hkv, int d) {
    return (2 * sizeof(float) + 2 * sizeof(uint16_t) * (size_t)d) * (size_t)rows_padded(n_rows * g) * (size_t)hkv;
}

// Backward workspace layout (float32 elements from the start): delta [n_rows * hq] padded to a
// multiple of 64, then dq_parts [n_parts, n_rows, hq, d], then the matrix-core extra.
inline int64_t bwd_delta_elems(int64_t n_rows, int hq) { return (n_rows * hq + 63) / 64 * 64; }

}  // namespace ls
