// C ABI front end of the replay-attention library: argument checks (all before any launch),
// workspace sizing, kernel dispatch and the per-thread error message.  No exception crosses
// the boundary and nothing here allocates device memory or synchronises with the host.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/longstraw.h"
#include "launch.hpp"

namespace {

thread_local std::string g_err;
thread_local uint32_t* g_owner = nullptr;  // one-writer counters of this thread's debug runs
thread_local size_t g_owner_slots = 0;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(LS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool d_supported(int d) { return d == 64 || d == 128 || d == 256; }

int64_t logical_pages(int64_t n_tok, int page_size) { return (n_tok + page_size - 1) / page_size; }

int check_prefix(const ls_prefix_t* p) {
    if (!p) return fail(LS_ERR_INVALID, "prefix descriptor is NULL");
    if (p->hq < 1 || p->hkv < 1 || p->hq % p->hkv != 0)
        return fail(LS_ERR_INVALID, "hq (%d) must be a positive multiple of hkv (%d)", p->hq, p->hkv);
    if (!d_supported(p->d)) return fail(LS_ERR_UNSUPPORTED, "head dim d=%d not in {64,128,256}", p->d);
    if (p->page_size != ls::kPage) return fail(LS_ERR_UNSUPPORTED, "page_size=%d, only 64 is built", p->page_size);
    if (p->dtype != LS_DTYPE_F32 && p->dtype != LS_DTYPE_BF16)
        return fail(LS_ERR_UNSUPPORTED, "dtype %d unknown", p->dtype);
    if (p->n_shards < 1 || p->n_shards > ls::kMaxShards)
        return fail(LS_ERR_INVALID, "n_shards=%d outside [1, %d]", p->n_shards, ls::kMaxShards);
    if (p->prefix_len < 0) return fail(LS_ERR_INVALID, "prefix_len=%lld < 0", (long long)p->prefix_len);
    if (!std::isfinite(p->softmax_scale) || !(p->softmax_scale > 0.f))
        return fail(LS_ERR_INVALID, "softmax_scale must be finite and > 0");
    const int64_t nlp = logical_pages(p->prefix_len, p->page_size);
    if (nlp > 0) {
        if (!p->page_table || !p->k_pages || !p->v_pages)
            return fail(LS_ERR_INVALID, "page_table/k_pages/v_pages must be non-NULL for a non-empty prompt");
        if (p->n_phys_pages < 1) return fail(LS_ERR_INVALID, "n_phys_pages=%lld < 1", (long long)p->n_phys_pages);
        if (nlp > (int64_t)INT32_MAX) return fail(LS_ERR_INVALID, "too many logical pages");
    }
    if (!p->shard_page_bounds) return fail(LS_ERR_INVALID, "shard_page_bounds is NULL");
    const int64_t* b = p->shard_page_bounds;
    if (b[0] != 0 || b[p->n_shards] != nlp)
        return fail(LS_ERR_INVALID, "shard bounds must run from 0 to %lld logical pages (got %lld..%lld)",
                    (long long)nlp, (long long)b[0], (long long)b[p->n_shards]);
    for (int s = 0; s < p->n_shards; s++)
        if (b[s + 1] < b[s]) return fail(LS_ERR_INVALID, "shard bounds decrease at shard %d", s);
    return LS_OK;
}

int check_block(const ls_prefix_t* p, const void* q, int64_t n_rows, int64_t q_start, const void* k_resp,
                const void* v_resp, int64_t n_resp_keys) {
    if (n_rows < 0 || q_start < 0) return fail(LS_ERR_INVALID, "n_rows=%lld, q_start=%lld must be >= 0",
                                               (long long)n_rows, (long long)q_start);
    if (n_resp_keys < q_start + n_rows)
        return fail(LS_ERR_INVALID, "n_resp_keys=%lld < q_start + n_rows = %lld", (long long)n_resp_keys,
                    (long long)(q_start + n_rows));
    if (n_rows > 0 && !q) return fail(LS_ERR_INVALID, "q is NULL");
    if (q_start + n_rows > 0 && (!k_resp || !v_resp)) return fail(LS_ERR_INVALID, "k_resp/v_resp is NULL");
    const int64_t rows_g = n_rows * (p->hq / p->hkv);
    if (rows_g > (int64_t)1 << 30) return fail(LS_ERR_INVALID, "block too large (%lld group rows)", (long long)rows_g);
    // kernels address one block's rows with 32-bit byte offsets
    if ((n_rows + 64) * (int64_t)p->hq * p->d * 4 >= ((int64_t)1 << 32))
        return fail(LS_ERR_INVALID, "block of %lld rows too large: split it into smaller blocks", (long long)n_rows);
    return LS_OK;
}

ls::AttnArgs make_args(const ls_prefix_t* p, const void* q, int64_t n_rows, int64_t q_start, const void* k_resp,
                       const void* v_resp) {
    ls::AttnArgs a;
    std::memset(&a, 0, sizeof a);
    a.k_pages = p->k_pages;
    a.v_pages = p->v_pages;
    a.table = p->page_table;
    a.prefix_len = p->prefix_len;
    a.n_logical_pages = logical_pages(p->prefix_len, p->page_size);
    a.n_phys = p->n_phys_pages;
    a.hq = p->hq;
    a.hkv = p->hkv;
    a.g = p->hq / p->hkv;
    a.d = p->d;
    a.scale = p->softmax_scale;
    a.scale_log2 = p->softmax_scale * ls::kLog2e;
    a.q = q;
    a.k_resp = k_resp;
    a.v_resp = v_resp;
    a.n_rows = n_rows;
    a.q_start = q_start;
    a.key_end = q_start + n_rows;
    a.n_shards = p->n_shards;
    a.n_parts = p->n_shards + 1;
    for (int s = 0; s <= p->n_shards; s++) a.shard_lo[s] = p->shard_page_bounds[s];
    a.n_members = 1;
    a.part_rows = n_rows;
    a.pg_lo = 0;
    a.pg_hi = a.n_logical_pages;
    a.ds_parts = a.n_parts;
    return a;
}

// Sub-range splits of a small block's shards (bf16 matrix-core passes only; launch.hpp).
int fwd_k(const ls_prefix_t* p, int64_t n_rows) {
    if (p->dtype != LS_DTYPE_BF16) return 1;
    return ls::fwd_split(n_rows, p->hq / p->hkv, p->n_shards, p->hkv, logical_pages(p->prefix_len, p->page_size));
}
int dqs_k(const ls_prefix_t* p, int64_t n_rows) {
    if (p->dtype != LS_DTYPE_BF16) return 1;
    return ls::dqs_split(n_rows, p->hq / p->hkv, p->n_shards, p->hkv, logical_pages(p->prefix_len, p->page_size));
}

// Forward workspace: the parts [n_parts, rows, d] float32 and their LSE [n_parts, rows], then,
// when the block's shards are split, the same for the n_shards * k + 1 sub-ranges.
size_t fwd_parts_bytes(const ls_prefix_t* p, int64_t n_rows, int64_t n_parts) {
    return sizeof(float) * (size_t)n_parts * (size_t)n_rows * (size_t)p->hq * (size_t)(p->d + 1);
}
size_t fwd_ws_k(const ls_prefix_t* p, int64_t rows, int k) {
    size_t b = fwd_parts_bytes(p, rows, p->n_shards + 1);
    if (k > 1) b += fwd_parts_bytes(p, rows, (int64_t)p->n_shards * k + 1);
    return b;
}
size_t fwd_ws(const ls_prefix_t* p, int64_t n_rows) { return fwd_ws_k(p, n_rows, fwd_k(p, n_rows)); }

// The matrix-core forward over the parts of `a` (its o_parts / lse_parts hold part_rows_hq rows
// of (row, head) per part).  With k > 1 it runs over k page ranges of every shard, writing their
// results after the parts, and then merges each shard's ranges into the shard's part (the
// response part is copied by a one-part merge, which is exact).
hipError_t fwd_mfma_parts(const ls::AttnArgs& a, int n_shards, int k, int64_t part_rows_hq, int d, hipStream_t s) {
    if (k <= 1) return ls::launch_fwd_mfma(a, s);
    ls::AttnArgs b = a;
    b.n_shards = n_shards * k;
    b.n_parts = b.n_shards + 1;
    ls::split_bounds(a.shard_lo, n_shards, k, b.shard_lo);
    b.o_parts = a.lse_parts + (size_t)a.n_parts * part_rows_hq;
    b.lse_parts = b.o_parts + (size_t)b.n_parts * part_rows_hq * d;
    hipError_t e = ls::launch_fwd_mfma(b, s);
    for (int sh = 0; sh <= n_shards && e == hipSuccess; sh++)
        e = ls::launch_lse_merge(sh < n_shards ? k : 1, part_rows_hq, d, b.o_parts + (size_t)sh * k * part_rows_hq * d,
                                 b.lse_parts + (size_t)sh * k * part_rows_hq, a.o_parts + (size_t)sh * part_rows_hq * d,
                                 LS_DTYPE_F32, a.lse_parts + (size_t)sh * part_rows_hq, s);
    return e;
}

// Backward workspace: delta, the dQ parts, the matrix-core passes' row copies, then, when the
// dQ pass of a small block splits its shards, the sub-ranges' dQ partials at a 256-byte boundary.
size_t bwd_base(const ls_prefix_t* p, int64_t n_rows) {
    return sizeof(float) * ((size_t)ls::bwd_delta_elems(n_rows, p->hq) + (size_t)(p->n_shards + 1) * n_rows * p->hq * p->d) +
           ls::mfma_bwd_extra_bytes(n_rows, p->hq / p->hkv, p->hkv, p->d);
}
size_t dq_sub_offset(const ls_prefix_t* p, int64_t n_rows) { return (bwd_base(p, n_rows) + 255) / 256 * 256; }
size_t bwd_ws(const ls_prefix_t* p, int64_t n_rows) {
    const int k = dqs_k(p, n_rows);
    if (k <= 1) return bwd_base(p, n_rows);
    return dq_sub_offset(p, n_rows) +
           sizeof(float) * ((size_t)p->n_shards * k + 1) * (size_t)n_rows * (size_t)p->hq * (size_t)p->d;
}
// dQ partials the stored-dS backward forms (shards and response, or their sub-ranges)
int dq_parts_formed(const ls_prefix_t* p, int64_t n_rows) {
    const int k = dqs_k(p, n_rows);
    return k > 1 ? p->n_shards * k + 1 : p->n_shards + 1;
}

// Bytes of the stored dS (bf16, one per group row and key slot) of a block whose response keys
// end at key_end, placed after the recompute workspace at a 256-byte boundary: per kv head, for
// chunks of `parts` consecutive key parts (n_shards + 1: all keys at once).
size_t ds_offset(const ls_prefix_t* p, int64_t n_rows) { return (bwd_ws(p, n_rows) + 255) / 256 * 256; }
size_t ds_head_bytes(const ls_prefix_t* p, int64_t n_rows, int64_t key_end, int parts) {
    const int64_t rows_total = n_rows * (p->hq / p->hkv);
    return (size_t)ls::ds_row_tiles(rows_total) *
           (size_t)ls::ds_chunk_slots(p->shard_page_bounds, p->n_shards, key_end, parts) * 64;
}
size_t ds_bytes(const ls_prefix_t* p, int64_t n_rows, int64_t key_end) {
    return (size_t)p->hkv * ds_head_bytes(p, n_rows, key_end, p->n_shards + 1);
}

}  // namespace

extern "C" {

int ls_version(void) { return LS_VERSION; }

const char* ls_last_error(void) { return g_err.c_str(); }

int ls_capture_pages(const void* k_src, const void* v_src, int src_dtype, int64_t n_tok, int64_t first_tok,
                     const int32_t* page_table, int64_t n_logical_pages, void* k_pages, void* v_pages,
                     int page_dtype, int64_t n_phys_pages, int hkv, int d, int page_size, ls_stream_t stream) {
    g_err.clear();
    if (n_tok < 0 || first_tok < 0) return fail(LS_ERR_INVALID, "n_tok and first_tok must be >= 0");
    if (hkv < 1) return fail(LS_ERR_INVALID, "hkv=%d < 1", hkv);
    if (!d_supported(d)) return fail(LS_ERR_UNSUPPORTED, "head dim d=%d not in {64,128,256}", d);
    if (page_size != ls::kPage) return fail(LS_ERR_UNSUPPORTED, "page_size=%d, only 64 is built", page_size);
    const bool same = src_dtype == page_dtype && (src_dtype == LS_DTYPE_F32 || src_dtype == LS_DTYPE_BF16);
    const bool down = src_dtype == LS_DTYPE_F32 && page_dtype == LS_DTYPE_BF16;
    if (!same && !down) return fail(LS_ERR_UNSUPPORTED, "capture from dtype %d into dtype %d", src_dtype, page_dtype);
    if (first_tok % page_size != 0) return fail(LS_ERR_INVALID, "first_tok=%lld is not page aligned", (long long)first_tok);
    if (n_tok == 0) return LS_OK;
    if (!k_src || !v_src || !page_table || !k_pages || !v_pages) return fail(LS_ERR_INVALID, "NULL pointer argument");
    if (n_phys_pages < 1) return fail(LS_ERR_INVALID, "n_phys_pages=%lld < 1", (long long)n_phys_pages);
    if (logical_pages(first_tok + n_tok, page_size) > n_logical_pages)
        return fail(LS_ERR_INVALID, "tokens up to %lld need more than %lld logical pages", (long long)(first_tok + n_tok),
                    (long long)n_logical_pages);
    hipError_t e = ls::launch_capture(k_src, v_src, src_dtype, n_tok, first_tok, page_table, k_pages, v_pages, page_dtype,
                                      n_phys_pages, hkv, d, (hipStream_t)stream);
    return e == hipSuccess ? LS_OK : hip_fail(e, "capture kernel");
}

int ls_check_page_table(const int32_t* page_table_host, int64_t n_logical_pages, int64_t n_phys_pages) {
    g_err.clear();
    if (n_logical_pages < 0) return fail(LS_ERR_INVALID, "n_logical_pages=%lld < 0", (long long)n_logical_pages);
    if (n_logical_pages == 0) return LS_OK;
    if (!page_table_host) return fail(LS_ERR_INVALID, "page_table_host is NULL");
    if (n_phys_pages < n_logical_pages)
        return fail(LS_ERR_INVALID, "%lld logical pages cannot map one to one into %lld physical pages",
                    (long long)n_logical_pages, (long long)n_phys_pages);
    std::vector<uint8_t> seen((size_t)n_phys_pages, 0);
    for (int64_t i = 0; i < n_logical_pages; i++) {
        const int32_t e = page_table_host[i];
        if (e < 0 || e >= n_phys_pages)
            return fail(LS_ERR_INVALID, "page_table[%lld] = %d is outside [0, %lld)", (long long)i, e,
                        (long long)n_phys_pages);
        if (seen[(size_t)e])
            return fail(LS_ERR_INVALID, "page_table[%lld] = %d: physical page already mapped by an earlier logical page",
                        (long long)i, e);
        seen[(size_t)e] = 1;
    }
    return LS_OK;
}

int ls_gather_pages(const void* pages, int dtype, const int32_t* page_table, int64_t n_logical_pages,
                    int64_t n_phys_pages, int64_t first_tok, int64_t n_tok, int hkv, int d, int page_size, void* dst,
                    ls_stream_t stream) {
    g_err.clear();
    if (n_tok < 0 || first_tok < 0) return fail(LS_ERR_INVALID, "n_tok and first_tok must be >= 0");
    if (hkv < 1) return fail(LS_ERR_INVALID, "hkv=%d < 1", hkv);
    if (!d_supported(d)) return fail(LS_ERR_UNSUPPORTED, "head dim d=%d not in {64,128,256}", d);
    if (page_size != ls::kPage) return fail(LS_ERR_UNSUPPORTED, "page_size=%d, only 64 is built", page_size);
    if (dtype != LS_DTYPE_F32 && dtype != LS_DTYPE_BF16) return fail(LS_ERR_UNSUPPORTED, "dtype %d unknown", dtype);
    if (n_tok == 0) return LS_OK;
    if (!pages || !page_table || !dst) return fail(LS_ERR_INVALID, "NULL pointer argument");
    if (n_phys_pages < 1) return fail(LS_ERR_INVALID, "n_phys_pages=%lld < 1", (long long)n_phys_pages);
    if (logical_pages(first_tok + n_tok, page_size) > n_logical_pages)
        return fail(LS_ERR_INVALID, "tokens up to %lld need more than %lld logical pages", (long long)(first_tok + n_tok),
                    (long long)n_logical_pages);
    hipError_t e = ls::launch_gather(pages, dtype, page_table, n_phys_pages, first_tok, n_tok, hkv, d, dst,
                                     (hipStream_t)stream);
    return e == hipSuccess ? LS_OK : hip_fail(e, "gather kernel");
}

size_t ls_fwd_workspace_bytes(const ls_prefix_t* pre, int64_t n_rows) {
    g_err.clear();
    if (check_prefix(pre) != LS_OK) return 0;
    if (n_rows < 0) {
        fail(LS_ERR_INVALID, "n_rows < 0");
        return 0;
    }
    return fwd_ws(pre, n_rows);
}

size_t ls_bwd_workspace_bytes(const ls_prefix_t* pre, int64_t n_rows) {
    g_err.clear();
    if (check_prefix(pre) != LS_OK) return 0;
    if (n_rows < 0) {
        fail(LS_ERR_INVALID, "n_rows < 0");
        return 0;
    }
    return bwd_ws(pre, n_rows);
}

size_t ls_bwd_ds_workspace_bytes(const ls_prefix_t* pre, int64_t n_rows, int64_t key_end) {
    g_err.clear();
    if (check_prefix(pre) != LS_OK) return 0;
    if (n_rows < 0 || key_end < n_rows) {
        fail(LS_ERR_INVALID, "n_rows=%lld, key_end=%lld: need 0 <= n_rows <= key_end", (long long)n_rows,
             (long long)key_end);
        return 0;
    }
    if (pre->dtype != LS_DTYPE_BF16) return bwd_ws(pre, n_rows);  // the float32 path stores no dS
    return ds_offset(pre, n_rows) + ds_bytes(pre, n_rows, key_end);
}

size_t ls_bwd_ds_chunk_workspace_bytes(const ls_prefix_t* pre, int64_t n_rows, int64_t key_end, int heads,
                                       int parts) {
    g_err.clear();
    if (check_prefix(pre) != LS_OK) return 0;
    if (n_rows < 0 || key_end < n_rows) {
        fail(LS_ERR_INVALID, "n_rows=%lld, key_end=%lld: need 0 <= n_rows <= key_end", (long long)n_rows,
             (long long)key_end);
        return 0;
    }
    const int n_all = pre->n_shards + 1;
    if (heads < 1 || heads > pre->hkv || parts < 1 || parts > n_all || (heads > 1 && parts < n_all)) {
        fail(LS_ERR_INVALID, "chunks of %d kv heads by %d key parts: need 1 <= heads <= hkv (%d), 1 <= parts <= %d, "
             "and all parts when heads > 1", heads, parts, pre->hkv, n_all);
        return 0;
    }
    if (pre->dtype != LS_DTYPE_BF16) return bwd_ws(pre, n_rows);
    return ds_offset(pre, n_rows) + (size_t)heads * ds_head_bytes(pre, n_rows, key_end, parts);
}

// Checks of a forward call, before any launch (shared by ls_replay_fwd and the no-allocation
// variant): LS_OK with nothing to do for an empty block is reported through *empty.
static int check_fwd(const ls_prefix_t* pre, const void* q, int64_t n_rows, int64_t q_start, const void* k_resp,
                     const void* v_resp, int64_t n_resp_keys, void* o, float* lse, bool* empty) {
    int rc = check_prefix(pre);
    if (rc != LS_OK) return rc;
    rc = check_block(pre, q, n_rows, q_start, k_resp, v_resp, n_resp_keys);
    if (rc != LS_OK) return rc;
    *empty = n_rows == 0;
    if (*empty) return LS_OK;
    if (!o || !lse) return fail(LS_ERR_INVALID, "o/lse is NULL");
    return LS_OK;
}

static int run_fwd(const ls_prefix_t* pre, const void* q, int64_t n_rows, int64_t q_start, const void* k_resp,
                   const void* v_resp, void* o, float* lse, void* workspace, ls_stream_t stream);

int ls_replay_fwd(const ls_prefix_t* pre, const void* q, int64_t n_rows, int64_t q_start, const void* k_resp,
                  const void* v_resp, int64_t n_resp_keys, void* o, float* lse, void* workspace, size_t ws_bytes,
                  ls_stream_t stream) {
    g_err.clear();
    bool empty = false;
    const int rc = check_fwd(pre, q, n_rows, q_start, k_resp, v_resp, n_resp_keys, o, lse, &empty);
    if (rc != LS_OK || empty) return rc;
    const size_t need = fwd_ws(pre, n_rows);
    if (!workspace || ws_bytes < need)
        return fail(LS_ERR_WORKSPACE, "forward workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
    return run_fwd(pre, q, n_rows, q_start, k_resp, v_resp, o, lse, workspace, stream);
}

int ls_replay_fwd_noalloc(const ls_prefix_t* pre, const void* q, int64_t n_rows, int64_t q_start, const void* k_resp,
                          const void* v_resp, int64_t n_resp_keys, void* o, float* lse, ls_stream_t stream) {
    g_err.clear();
    bool empty = false;
    const int rc = check_fwd(pre, q, n_rows, q_start, k_resp, v_resp, n_resp_keys, o, lse, &empty);
    if (rc != LS_OK || empty) return rc;
    const size_t need = fwd_ws(pre, n_rows);
    if (need > (size_t)LS_NOALLOC_SCRATCH_BYTES) {
        const size_t per_row = fwd_ws(pre, 1);
        return fail(LS_ERR_WORKSPACE,
                    "a block of %lld rows needs %zu bytes of forward scratch; the no-allocation forward holds %zu "
                    "(at most %zu rows at this shape): split the block",
                    (long long)n_rows, need, (size_t)LS_NOALLOC_SCRATCH_BYTES,
                    per_row ? (size_t)LS_NOALLOC_SCRATCH_BYTES / per_row : 0);
    }
    void* scratch = nullptr;
    size_t scratch_bytes = 0;
    const hipError_t e = ls::noalloc_scratch(&scratch, &scratch_bytes);
    if (e != hipSuccess) return hip_fail(e, "scratch set-up (hipGetSymbolAddress)");
    if (scratch_bytes < need) return fail(LS_ERR_WORKSPACE, "scratch of %zu bytes, %zu needed", scratch_bytes, need);
    return run_fwd(pre, q, n_rows, q_start, k_resp, v_resp, o, lse, scratch, stream);
}

// Fused forward + dQ workspace (float32): o, A / l and B / l parts [n_parts, n_rows, hq, d] each,
// then the LSE and delta parts [n_parts, n_rows, hq] each.
static size_t fwd_dq_ws(const ls_prefix_t* p, int64_t n_rows) {
    return sizeof(float) * (size_t)(p->n_shards + 1) * (size_t)n_rows * (size_t)p->hq * (3 * (size_t)p->d + 2);
}

size_t ls_fwd_dq_workspace_bytes(const ls_prefix_t* pre, int64_t n_rows) {
    g_err.clear();
    if (check_prefix(pre) != LS_OK) return 0;
    if (n_rows < 0) {
        fail(LS_ERR_INVALID, "n_rows=%lld < 0", (long long)n_rows);
        return 0;
    }
    return fwd_dq_ws(pre, n_rows);
}

int ls_replay_fwd_dq(const ls_prefix_t* pre, const void* q, int64_t n_rows, int64_t q_start, const void* k_resp,
                     const void* v_resp, int64_t n_resp_keys, const void* dout, void* o, float* lse, float* dq,
                     void* workspace, size_t ws_bytes, ls_stream_t stream) {
    g_err.clear();
    bool empty = false;
    const int rc = check_fwd(pre, q, n_rows, q_start, k_resp, v_resp, n_resp_keys, o, lse, &empty);
    if (rc != LS_OK || empty) return rc;
    if (!dout || !dq) return fail(LS_ERR_INVALID, "dout/dq is NULL");
    if (pre->dtype != LS_DTYPE_BF16) return fail(LS_ERR_UNSUPPORTED, "the fused forward + dQ pass takes bf16 pages only");
    const size_t need = fwd_dq_ws(pre, n_rows);
    if (!workspace || ws_bytes < need)
        return fail(LS_ERR_WORKSPACE, "fused forward + dQ workspace of %zu bytes needed, %zu given", need,
                    workspace ? ws_bytes : 0);
    ls::AttnArgs a = make_args(pre, q, n_rows, q_start, k_resp, v_resp);
    a.dout = dout;
    const int64_t rows = n_rows * pre->hq;
    const size_t part_elems = (size_t)a.n_parts * rows * pre->d;
    a.o_parts = (float*)workspace;
    float* a_parts = a.o_parts + part_elems;
    float* b_parts = a_parts + part_elems;
    a.lse_parts = b_parts + part_elems;
    float* delta_parts = a.lse_parts + (size_t)a.n_parts * rows;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = ls::launch_fwd_dq_mfma(a, a_parts, b_parts, delta_parts, s);
    if (e != hipSuccess) return hip_fail(e, "fused forward + dQ kernel");
    e = ls::launch_lse_merge(a.n_parts, rows, pre->d, a.o_parts, a.lse_parts, o, pre->dtype, lse, s);
    if (e != hipSuccess) return hip_fail(e, "LSE merge kernel");
    e = ls::launch_fwd_dq_merge(a.n_parts, rows, pre->d, a.lse_parts, lse, a_parts, b_parts, delta_parts, a.scale, dq,
                                s);
    return e == hipSuccess ? LS_OK : hip_fail(e, "dQ merge kernel");
}

static int run_fwd(const ls_prefix_t* pre, const void* q, int64_t n_rows, int64_t q_start, const void* k_resp,
                   const void* v_resp, void* o, float* lse, void* workspace, ls_stream_t stream) {
    ls::AttnArgs a = make_args(pre, q, n_rows, q_start, k_resp, v_resp);
    const int64_t rows = n_rows * pre->hq;
    a.o_parts = (float*)workspace;
    a.lse_parts = a.o_parts + (size_t)a.n_parts * rows * pre->d;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = pre->dtype == LS_DTYPE_BF16 ? fwd_mfma_parts(a, pre->n_shards, fwd_k(pre, n_rows), rows, pre->d, s)
                                               : ls::launch_fwd_generic(a, s);
    if (e != hipSuccess) return hip_fail(e, "forward kernel");
    e = ls::launch_lse_merge(a.n_parts, rows, pre->d, a.o_parts, a.lse_parts, o, pre->dtype, lse, s);
    return e == hipSuccess ? LS_OK : hip_fail(e, "LSE merge kernel");
}

size_t ls_score_workspace_bytes(const ls_prefix_t* pre, int64_t n_members, int64_t n_rows) {
    g_err.clear();
    if (check_prefix(pre) != LS_OK) return 0;
    if (n_members < 0 || n_rows < 0) {
        fail(LS_ERR_INVALID, "n_members=%lld, n_rows=%lld must be >= 0", (long long)n_members, (long long)n_rows);
        return 0;
    }
    // the page-range split follows each member's block size, as ls_replay_fwd would choose it
    return fwd_ws_k(pre, n_members * n_rows, fwd_k(pre, n_rows));
}

int ls_score_fwd(const ls_prefix_t* pre, int64_t n_members, const void* q, int64_t n_rows, const void* k_resp,
                 const void* v_resp, void* o, float* lse, void* workspace, size_t ws_bytes, ls_stream_t stream) {
    g_err.clear();
    int rc = check_prefix(pre);
    if (rc != LS_OK) return rc;
    if (n_members < 0) return fail(LS_ERR_INVALID, "n_members=%lld < 0", (long long)n_members);
    // the members' rows together must fit one block's limits
    rc = check_block(pre, q, n_members * n_rows, 0, k_resp, v_resp, n_members * n_rows);
    if (rc != LS_OK) return rc;
    if (n_members * n_rows == 0) return LS_OK;
    if (!o || !lse) return fail(LS_ERR_INVALID, "o/lse is NULL");
    const size_t need = fwd_ws_k(pre, n_members * n_rows, fwd_k(pre, n_rows));
    if (!workspace || ws_bytes < need)
        return fail(LS_ERR_WORKSPACE, "scoring workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
    ls::AttnArgs a = make_args(pre, q, n_rows, 0, k_resp, v_resp);
    const int64_t all_rows = n_members * n_rows;
    a.part_rows = all_rows;
    a.resp_member_elems = n_rows * pre->hkv * pre->d;
    a.o_parts = (float*)workspace;
    a.lse_parts = a.o_parts + (size_t)a.n_parts * all_rows * pre->hq * pre->d;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (pre->dtype == LS_DTYPE_BF16) {
        // one launch over every member's rows, split into the page ranges that each member's
        // own replay would use, so that a member scores bit for bit as it replays
        a.n_members = n_members;
        e = fwd_mfma_parts(a, pre->n_shards, fwd_k(pre, n_rows), all_rows * pre->hq, pre->d, s);
    } else {
        // the exact f32 path runs the members one launch at a time into the same parts
        const size_t esz = 4;
        for (int64_t m = 0; m < n_members && e == hipSuccess; m++) {
            ls::AttnArgs am = a;
            am.q = (const char*)q + (size_t)(m * n_rows * pre->hq * pre->d) * esz;
            am.k_resp = (const char*)k_resp + (size_t)(m * a.resp_member_elems) * esz;
            am.v_resp = (const char*)v_resp + (size_t)(m * a.resp_member_elems) * esz;
            am.row0 = m * n_rows;
            e = ls::launch_fwd_generic(am, s);
        }
    }
    if (e != hipSuccess) return hip_fail(e, "scoring forward kernel");
    e = ls::launch_lse_merge(a.n_parts, all_rows * pre->hq, pre->d, a.o_parts, a.lse_parts, o, pre->dtype, lse, s);
    return e == hipSuccess ? LS_OK : hip_fail(e, "LSE merge kernel");
}

int ls_replay_bwd(const ls_prefix_t* pre, const void* q, int64_t n_rows, int64_t q_start, const void* k_resp,
                  const void* v_resp, int64_t n_resp_keys, const void* o, const float* lse, const void* dout, float* dq,
                  float* dk_resp, float* dv_resp, int resp_first_touch, float* dk_pages, float* dv_pages,
                  const uint8_t* shard_first_touch, void* workspace, size_t ws_bytes, ls_stream_t stream) {
    g_err.clear();
    int rc = check_prefix(pre);
    if (rc != LS_OK) return rc;
    rc = check_block(pre, q, n_rows, q_start, k_resp, v_resp, n_resp_keys);
    if (rc != LS_OK) return rc;
    if (n_rows > 0 && (!o || !lse || !dout)) return fail(LS_ERR_INVALID, "o/lse/dout is NULL");
    const bool skip_dq = dq == nullptr;  // dK/dV only
    if (n_resp_keys > 0 && (!dk_resp || !dv_resp)) return fail(LS_ERR_INVALID, "dk_resp/dv_resp is NULL");
    if (pre->prefix_len > 0 && (!dk_pages || !dv_pages)) return fail(LS_ERR_INVALID, "dk_pages/dv_pages is NULL");
    const size_t need = bwd_ws(pre, n_rows);
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(LS_ERR_WORKSPACE, "backward workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
    ls::AttnArgs a = make_args(pre, q, n_rows, q_start, k_resp, v_resp);
    int64_t owner_slots = 0;
    if (g_owner) {
        if (pre->dtype != LS_DTYPE_BF16)
            return fail(LS_ERR_UNSUPPORTED, "one-writer counters cover the bf16 matrix-core kernels only");
        if (skip_dq) return fail(LS_ERR_UNSUPPORTED, "one-writer counters cover backward calls that form dQ");
        owner_slots = ls::owner_slots(pre->n_phys_pages, pre->hkv, pre->hq, dq_parts_formed(pre, n_rows), n_rows,
                                      a.key_end);
        if (g_owner_slots < (size_t)owner_slots)
            return fail(LS_ERR_INVALID, "one-writer counters: %lld slots needed, %zu registered", (long long)owner_slots,
                        g_owner_slots);
        a.owner = g_owner;
        a.owner_resp0 = ls::owner_resp0(pre->n_phys_pages, pre->hkv);
        a.owner_dq0 = ls::owner_dq0(pre->n_phys_pages, pre->hkv, a.key_end);
    }
    const int64_t rows = n_rows * pre->hq;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.delta = (float*)workspace;
    a.dq_parts = (float*)workspace + ls::bwd_delta_elems(n_rows, pre->hq);
    a.dk_pages = dk_pages;
    a.dv_pages = dv_pages;
    a.dk_resp = dk_resp;
    a.dv_resp = dv_resp;
    a.resp_first_touch = resp_first_touch != 0;
    a.skip_dq = skip_dq;
    a.first_touch_mask = 0;
    if (shard_first_touch)
        for (int s = 0; s < pre->n_shards; s++)
            if (shard_first_touch[s]) a.first_touch_mask |= 1ull << s;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (owner_slots > 0) {  // zero bits are the same for uint32 and float32
        e = ls::launch_zero((float*)a.owner, owner_slots, s);
        if (e != hipSuccess) return hip_fail(e, "zero kernel");
    }
    if (pre->dtype == LS_DTYPE_BF16) {
        // A workspace that also holds some stored dS selects the stored-dS dQ pass: with room
        // for every key's dS of at least one kv head, in chunks of as many kv heads as it holds;
        // otherwise one kv head at a time by the largest number of consecutive key parts whose
        // dS it holds.  With room for none, the dQ pass recomputes.
        const int n_all = pre->n_shards + 1;
        const size_t off = ds_offset(pre, n_rows);
        const size_t room = ws_bytes > off ? ws_bytes - off : 0;
        const size_t per_head = ds_head_bytes(pre, n_rows, a.key_end, n_all);
        int heads = 0, parts = n_all;
        if (skip_dq) {
            // no dQ pass: nothing reads a stored dS
        } else if (n_rows > 0 && per_head > 0 && room >= per_head) {
            const size_t fit = room / per_head;
            heads = fit < (size_t)pre->hkv ? (int)fit : pre->hkv;
        } else if (n_rows > 0) {
            for (int k = n_all - 1; k >= 1 && heads == 0; k--)
                if (room >= ds_head_bytes(pre, n_rows, a.key_end, k)) {
                    heads = 1;
                    parts = k;
                }
        }
        if (heads > 0) {
            a.ds = (uint16_t*)((char*)workspace + off);
            a.ds_rt = ls::ds_row_tiles(n_rows * a.g);
            a.ds_kslots = ls::ds_chunk_slots(pre->shard_page_bounds, pre->n_shards, a.key_end, parts);
            a.ds_heads = heads;
            a.ds_parts = parts;
            const int k = dqs_k(pre, n_rows);
            if (k > 1 && parts == n_all) {  // a small block: the dQ pass over shard sub-ranges
                a.dq_sub = (float*)((char*)workspace + dq_sub_offset(pre, n_rows));
                a.dq_sub_k = k;
            }
        }
        e = ls::launch_bwd_mfma(a, s);  // its prep kernel also writes delta
    } else {
        e = ls::launch_delta(o, dout, pre->dtype, rows, pre->d, (float*)a.delta, s);
        if (e == hipSuccess) e = ls::launch_bwd_generic(a, s);
    }
    if (e != hipSuccess) return hip_fail(e, "backward kernels");
    if (skip_dq)
        e = hipSuccess;
    else if (a.dq_sub_k > 1)
        e = ls::launch_sum_parts(pre->n_shards * a.dq_sub_k + 1, rows * pre->d, a.dq_sub, dq, s);
    else
        e = ls::launch_sum_parts(a.n_parts, rows * pre->d, a.dq_parts, dq, s);
    if (e != hipSuccess) return hip_fail(e, "dQ part sum kernel");
    if (resp_first_touch && n_resp_keys > a.key_end) {
        const int64_t off = a.key_end * pre->hkv * pre->d;
        const int64_t cnt = (n_resp_keys - a.key_end) * pre->hkv * pre->d;
        e = ls::launch_zero(dk_resp + off, cnt, s);
        if (e == hipSuccess) e = ls::launch_zero(dv_resp + off, cnt, s);
        if (e != hipSuccess) return hip_fail(e, "zero kernel");
    }
    return LS_OK;
}

size_t ls_debug_owner_slots(const ls_prefix_t* pre, int64_t n_rows, int64_t key_end) {
    g_err.clear();
    if (check_prefix(pre) != LS_OK) return 0;
    if (n_rows < 0 || key_end < n_rows) {
        fail(LS_ERR_INVALID, "n_rows=%lld, key_end=%lld", (long long)n_rows, (long long)key_end);
        return 0;
    }
    return (size_t)ls::owner_slots(pre->n_phys_pages, pre->hkv, pre->hq, dq_parts_formed(pre, n_rows), n_rows,
                                   key_end);
}

int ls_debug_set_owner_counts(uint32_t* counts, size_t n_slots) {
    g_err.clear();
    if (counts && n_slots == 0) return fail(LS_ERR_INVALID, "n_slots is 0");
    g_owner = counts;
    g_owner_slots = counts ? n_slots : 0;
    return LS_OK;
}

static int lse_merge_impl(int n_parts, int64_t n_rows, int d, const float* o_parts, const float* lse_parts,
                          void* o_out, int out_dtype, float* lse_out, ls_stream_t stream, bool bf16_numerator) {
    g_err.clear();
    if (n_parts < 1) return fail(LS_ERR_INVALID, "n_parts=%d < 1", n_parts);
    if (n_rows < 0) return fail(LS_ERR_INVALID, "n_rows < 0");
    if (d < 4 || d % 4 != 0 || d > 1024) return fail(LS_ERR_UNSUPPORTED, "d=%d must be a multiple of 4 in [4, 1024]", d);
    if (out_dtype != LS_DTYPE_F32 && out_dtype != LS_DTYPE_BF16) return fail(LS_ERR_UNSUPPORTED, "dtype %d", out_dtype);
    if (n_rows == 0) return LS_OK;
    if (!o_parts || !lse_parts || !o_out || !lse_out) return fail(LS_ERR_INVALID, "NULL pointer argument");
    hipError_t e = ls::launch_lse_merge(n_parts, n_rows, d, o_parts, lse_parts, o_out, out_dtype, lse_out,
                                        (hipStream_t)stream, bf16_numerator);
    return e == hipSuccess ? LS_OK : hip_fail(e, "LSE merge kernel");
}

int ls_lse_merge(int n_parts, int64_t n_rows, int d, const float* o_parts, const float* lse_parts, void* o_out,
                 int out_dtype, float* lse_out, ls_stream_t stream) {
    return lse_merge_impl(n_parts, n_rows, d, o_parts, lse_parts, o_out, out_dtype, lse_out, stream, false);
}

int ls_lse_merge_bf16num(int n_parts, int64_t n_rows, int d, const float* o_parts, const float* lse_parts,
                         void* o_out, int out_dtype, float* lse_out, ls_stream_t stream) {
    return lse_merge_impl(n_parts, n_rows, d, o_parts, lse_parts, o_out, out_dtype, lse_out, stream, true);
}

}  // extern "C"
