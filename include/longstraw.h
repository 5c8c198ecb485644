/*
 * longstraw.h -- C ABI of the replay-attention library for AMD MI355X (gfx950).
 *
 * The operation: exact attention of a short block of response rows over a long prompt
 * whose keys and values were captured once, without gradients, into pages, plus the
 * response itself under a causal mask; forward and backward.  This is the attention
 * slice of LongStraw's capture-once / replay-suffix GRPO step ("LongStraw: Long-Context
 * RL Beyond 2M Tokens under a Fixed GPU Budget"; paper digest, section "Method", steps 1
 * and 3; explainer, sections "The move: change the graph boundary" and "Two incompatible
 * architectures, same transaction").
 *
 * Conventions for every entry point:
 *  - All functions are callable from C, return int (LS_OK == 0 on success, a negative
 *    LS_ERR_* code otherwise) and never throw.  On failure ls_last_error() returns a
 *    message for the calling thread.  Every argument check happens before the first
 *    launch: a call that returns an error has enqueued nothing.
 *  - Pointers named *device* point to GPU memory of the current device; pointers named
 *    *host* point to host memory that is read during the call only.  The caller owns
 *    all memory.  The library allocates no device memory, keeps no pointer after
 *    returning and does not synchronise with the host: work is enqueued on `stream` (a
 *    hipStream_t; NULL is the null stream) and buffers must stay alive until it is done.
 *    Device faults caused by bad pointers surface at the caller's next synchronisation.
 *  - Dense tensors are contiguous, row-major, with the shapes given below.
 *  - Element types: LS_DTYPE_F32 (IEEE binary32) or LS_DTYPE_BF16 (bfloat16).  Softmax
 *    statistics, gradients, partial results and merges are always float32.  bf16
 *    outputs are rounded to nearest-even from float32.
 *  - Scores are s = softmax_scale * q.k.  LSE values are natural logarithms of
 *    sum exp(s).  Query head h reads kv head h / (hq / hkv).
 *
 * Supported shapes: hq % hkv == 0; d in {64, 128, 256}; page_size == 64;
 * 1 <= n_shards <= 64.  The bf16 path runs on matrix cores; the f32 path is exact f32 on the
 * vector ALUs.
 */
#ifndef LONGSTRAW_H
#define LONGSTRAW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LS_VERSION 100 /* 1.0.0 */

#define LS_OK 0
#define LS_ERR_INVALID (-1)     /* a null pointer, a bad size, a range or a layout      */
#define LS_ERR_UNSUPPORTED (-2) /* a dtype / head-dim / page-size combination not built */
#define LS_ERR_WORKSPACE (-3)   /* workspace missing or smaller than the query says     */
#define LS_ERR_HIP (-4)         /* a HIP launch failed; the message names the kernel    */

#define LS_DTYPE_F32 0
#define LS_DTYPE_BF16 1

typedef void* ls_stream_t; /* a hipStream_t */

/*
 * The captured prompt: paged keys and values of one attention layer (digest, "Method",
 * step 1: the retained conditional state holds KV pages; explainer, "The move": a
 * read-only resident state).
 *
 *   page_table      device int32 [ceil(prefix_len / page_size)]: logical page -> physical
 *                   page.  Must be injective with entries in [0, n_phys_pages).
 *   k_pages/v_pages device [n_phys_pages, hkv, page_size, d] of `dtype`: row r of physical
 *                   page table[i] holds logical prompt token i * page_size + r.  Rows of a
 *                   last, partial page past prefix_len are never read.
 *   n_shards, shard_page_bounds
 *                   host int64 [n_shards + 1], non-decreasing, from 0 to the number of
 *                   logical pages: shard s owns logical pages [b[s], b[s+1]).  The shards
 *                   are the context-parallel owners whose local softmax statistics are
 *                   merged into the exact result (digest, "Method", Qwen implementation;
 *                   explainer, "Two incompatible architectures").  Empty shards are allowed.
 *   softmax_scale   > 0, usually 1 / sqrt(d).
 */
typedef struct ls_prefix {
    int hq;
    int hkv;
    int d;
    int page_size;
    int dtype;
    int n_shards;
    int64_t prefix_len;
    int64_t n_phys_pages;
    const int32_t* page_table;
    const void* k_pages;
    const void* v_pages;
    const int64_t* shard_page_bounds;
    float softmax_scale;
} ls_prefix_t;

/* Library version (LS_VERSION of the build). */
int ls_version(void);

/* Message of the calling thread's last failure ("" if none).  Valid until its next call. */
const char* ls_last_error(void);

/*
 * ls_capture_pages -- write captured prompt keys and values into page pools (digest,
 * "Method", step 1: the prompt is evaluated once without autograd and its KV pages are
 * kept).  Chunked capture is allowed: tokens [first_tok, first_tok + n_tok) of the prompt
 * are written, so a prompt can be captured in pieces.
 *
 *   k_src, v_src    device [n_tok, hkv, d] of src_dtype, logical token order.
 *   first_tok       multiple of page_size.
 *   page_table      device int32 [n_logical_pages]; must cover the written tokens.
 *   k_pages,v_pages device [n_phys_pages, hkv, page_size, d] of page_dtype.
 *   page_dtype      equal to src_dtype (a bit copy) or BF16 from an F32 source (rounded to
 *                   nearest-even).
 * Rows of a partial last page past the written tokens are left untouched.
 * Errors: LS_ERR_INVALID (null pointer, negative size, misaligned first_tok, a page index
 * past n_logical_pages), LS_ERR_UNSUPPORTED (dtype pair, d, page_size).
 */
int ls_capture_pages(const void* k_src, const void* v_src, int src_dtype, int64_t n_tok,
                     int64_t first_tok, const int32_t* page_table, int64_t n_logical_pages,
                     void* k_pages, void* v_pages, int page_dtype, int64_t n_phys_pages,
                     int hkv, int d, int page_size, ls_stream_t stream);

/*
 * ls_check_page_table -- host-side check of the caller contract on a page table: every entry
 * of page_table_host (host int32 [n_logical_pages]) lies in [0, n_phys_pages) and no two
 * logical pages share a physical page.  The kernels do not check the table (a bad entry is
 * clamped into the pool so that it cannot fault, and two logical pages on one physical page
 * would give that page two writers of its gradient), so a caller that builds its own table can
 * run this once per capture, before the table is uploaded.  Runs on the host only; it reads the
 * table and nothing else.
 * Errors: LS_ERR_INVALID (NULL table, an entry out of range, a repeated entry; the message
 * names the first offending logical page).
 */
int ls_check_page_table(const int32_t* page_table_host, int64_t n_logical_pages, int64_t n_phys_pages);

/*
 * ls_gather_pages -- read tokens [first_tok, first_tok + n_tok) of a pool back into logical
 * order: dst device [n_tok, hkv, d] of `dtype`, a bit copy.  The inverse of capture, for
 * checking the page-table walk.  Errors as for ls_capture_pages.
 */
int ls_gather_pages(const void* pages, int dtype, const int32_t* page_table,
                    int64_t n_logical_pages, int64_t n_phys_pages, int64_t first_tok,
                    int64_t n_tok, int hkv, int d, int page_size, void* dst,
                    ls_stream_t stream);

/*
 * Workspace bytes that ls_replay_fwd / ls_replay_bwd need for a block of n_rows response
 * rows (0 on invalid arguments, with ls_last_error set).
 *
 * Forward workspace layout (float32, from offset 0; n_parts = n_shards + 1):
 *   o_parts   [n_parts, n_rows, hq, d]   part p < n_shards: shard p; last: response keys
 *   lse_parts [n_parts, n_rows, hq]      -inf where a part has no key (O part = 0 there)
 * so that callers may inspect each owner's local result; for a bf16 block whose shards are
 * split into k page ranges (see ls_replay_fwd), the same two arrays for the n_shards * k + 1
 * ranges follow.
 * Backward workspace layout (from offset 0):
 *   delta     float32 [n_rows, hq], padded to a multiple of 64 elements: rowsum(dO * O)
 *   dq_parts  float32 [n_parts, n_rows, hq, d]
 *   then, for bf16, per kv head and query row of its group (padded to a multiple of 64
 *   rows): (LSE * log2 e, delta) float32 pairs, then the Q rows and the dO rows (bf16);
 *   then, for a bf16 block whose stored-dS dQ pass splits its shards into k page ranges, at a
 *   256-byte boundary, float32 dQ partials [n_shards * k + 1, n_rows, hq, d].
 * A block may have at most about 2^32 / (16 * hq * d) rows (174,000 at hq = 24, d = 256).
 */
size_t ls_fwd_workspace_bytes(const ls_prefix_t* pre, int64_t n_rows);
size_t ls_bwd_workspace_bytes(const ls_prefix_t* pre, int64_t n_rows);

/*
 * ls_bwd_ds_workspace_bytes -- backward workspace that also holds the block's dS, for a block
 * of n_rows rows whose response keys end at key_end = q_start + n_rows (0 on invalid
 * arguments, with ls_last_error set).  Equal to ls_bwd_workspace_bytes for float32.
 *
 * The backward's dQ is scale * sum_j dS_ij K_j with dS = P (dP - delta) (the softmax gradient
 * of exact attention, explainer "Serial replay makes G a schedule").  When ls_replay_bwd is
 * given at least this many bytes (bf16 only), the key-stationary dK/dV pass also writes dS,
 * rounded to bf16 as its matrix instructions take it, and the dQ pass reads it back, so the
 * dQ pass multiplies once per (row, key) pair instead of recomputing S and dP.  With fewer
 * bytes (but at least ls_bwd_workspace_bytes) the dQ pass recomputes them.  Both give dQ
 * within the bf16 rounding of dS of each other; dK, dV, delta are the same either way.
 *
 * Chunks.  A smaller workspace still selects the stored-dS pass if it holds the dS of part of
 * the block; the block is then run a chunk at a time (dK/dV of the chunk, which writes its dS,
 * then dQ of the chunk, which reads it; the same space serves each chunk in turn).  Kv heads
 * are independent and key parts (the n_shards prompt shards in order, then the response keys)
 * give separate dQ parts, so every chunking gives the same results bit for bit.  The chunking
 * a workspace of ws_bytes selects:
 *   - if it holds every key's dS of at least one kv head: chunks of as many kv heads as it
 *     holds (at most hkv), each over all keys;
 *   - otherwise one kv head at a time, by the largest number k of consecutive key parts such
 *     that it holds the dS of the largest chunk of k parts;
 *   - otherwise none: the dQ pass recomputes.
 * ls_bwd_ds_chunk_workspace_bytes gives the exact size for a chosen chunking, so that a caller
 * can pin the chunking for every block of a response.
 *
 * Layout: the recompute workspace, then from the next 256-byte boundary the stored dS, bf16
 * [kv heads of the chunk][row tiles][key slots][32]: row tiles of 32 group rows (r = token * g +
 * j for query head kv * g + j) padded to a multiple of 256 rows, key slots 128 per page pair of
 * the chunk (its prompt pairs first, then its response pairs).  Over all keys the size is
 * hkv * ceil(n_rows * g / 256) * 8 * 128 * (ceil(pages / 2) + ceil(ceil(key_end / 64) / 2)) * 64
 * bytes: 103 GB for 1,024 rows over a 2,097,152-token prompt with hq = 24, hkv = 4.  A workspace
 * sized for the largest key_end serves every block of a member.
 */
size_t ls_bwd_ds_workspace_bytes(const ls_prefix_t* pre, int64_t n_rows, int64_t key_end);

/*
 * ls_bwd_ds_chunk_workspace_bytes -- the backward workspace with which ls_replay_bwd runs the
 * stored-dS pass in chunks of `heads` kv heads by `parts` consecutive key parts (see
 * ls_bwd_ds_workspace_bytes): heads in [1, hkv] with parts == n_shards + 1 (all keys), or
 * heads == 1 with parts in [1, n_shards + 1].  (heads = hkv, parts = n_shards + 1) equals
 * ls_bwd_ds_workspace_bytes.  Returns 0 on invalid arguments, with ls_last_error set; for
 * float32 it equals ls_bwd_workspace_bytes.
 */
size_t ls_bwd_ds_chunk_workspace_bytes(const ls_prefix_t* pre, int64_t n_rows, int64_t key_end, int heads,
                                       int parts);

/*
 * ls_replay_fwd -- forward of one replayed response block (digest, "Method", step 3:
 * serial response replay; explainer, "Serial replay makes G a schedule": exact attention;
 * "Two incompatible architectures": local softmax statistics composed into the exact
 * global output).
 *
 * Rows are response positions [q_start, q_start + n_rows).  Row i sees every prompt key
 * and response keys [0, q_start + i] (the response follows the prompt).  Each shard and
 * the response keys give one local (O, LSE) written to the workspace, then the parts are
 * merged in float32 as by ls_lse_merge.
 *
 *   q               device [n_rows, hq, d] of pre->dtype.
 *   k_resp, v_resp  device [n_resp_keys, hkv, d] of pre->dtype; n_resp_keys >=
 *                   q_start + n_rows.  Keys at or past q_start + n_rows are never read.
 *   o               device [n_rows, hq, d] of pre->dtype (written).
 *   lse             device float32 [n_rows, hq] (written).
 *   workspace       device, ws_bytes >= ls_fwd_workspace_bytes(pre, n_rows).
 * Inputs are not checked for NaN: a NaN in a row's query (or in a key or value it sees) makes
 * that row's O and LSE NaN, and leaves every other row exactly as without it.
 * A small block has too few query tiles to fill the GPU with one workgroup per (query tile,
 * part, kv head); its shards are then split into k contiguous page ranges (up to 256 ranges,
 * at least 64 pages each on average), and the ranges' results merged into their shard's part
 * before the final merge, so the parts in the workspace keep the layout above and the
 * workspace size (ls_fwd_workspace_bytes) includes the ranges' results.  The stored-dS dQ pass
 * does the same (ls_bwd_workspace_bytes).
 * Errors: LS_ERR_INVALID, LS_ERR_UNSUPPORTED, LS_ERR_WORKSPACE, LS_ERR_HIP.
 */
int ls_replay_fwd(const ls_prefix_t* pre, const void* q, int64_t n_rows, int64_t q_start,
                  const void* k_resp, const void* v_resp, int64_t n_resp_keys, void* o,
                  float* lse, void* workspace, size_t ws_bytes, ls_stream_t stream);

/*
 * ls_replay_fwd_noalloc -- ls_replay_fwd for callers that cannot allocate device memory (code
 * under stream capture, tight serving loops, harnesses that forbid allocation).  The per-part
 * results live in a fixed scratch array of LS_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on, until the process ends, instead of in a caller's workspace.  Arguments,
 * results and errors are those of ls_replay_fwd without the workspace; a block whose forward
 * workspace (ls_fwd_workspace_bytes) exceeds LS_NOALLOC_SCRATCH_BYTES fails with
 * LS_ERR_WORKSPACE before any launch (split it into smaller blocks).  Nothing is allocated: the
 * first call on a device looks up that device's array (hipGetSymbolAddress); a failure there is
 * LS_ERR_HIP.  Every call on one GPU uses that GPU's one array, which keeps the last call's
 * contents, so calls that overlap on one GPU (on other streams or from other threads) race;
 * calls ordered on the device give exactly ls_replay_fwd's results.
 */
#define LS_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int ls_replay_fwd_noalloc(const ls_prefix_t* pre, const void* q, int64_t n_rows, int64_t q_start,
                          const void* k_resp, const void* v_resp, int64_t n_resp_keys, void* o,
                          float* lse, ls_stream_t stream);

/*
 * ls_score_fwd -- forward-only scoring of several members' whole responses against the same
 * captured prompt, in one launch (digest, "Method", step 2, pre-step scoring; explainer, "The
 * move: change the graph boundary": the old- and reference-policy passes need no autograd
 * graph, so nothing is kept for a backward and the members' rows can share every pass over
 * the prompt pages).
 *
 * Member m's row i (response position i) sees every prompt key and the member's own response
 * keys [0, i].  Each member's result equals ls_replay_fwd of its rows with q_start = 0 (the
 * matrix-core path gives the same bits).
 *
 *   n_members       >= 0.
 *   q               device [n_members, n_rows, hq, d] of pre->dtype.
 *   k_resp, v_resp  device [n_members, n_rows, hkv, d] of pre->dtype.
 *   o               device [n_members, n_rows, hq, d] of pre->dtype (written).
 *   lse             device float32 [n_members, n_rows, hq] (written).
 *   workspace       device, ws_bytes >= ls_score_workspace_bytes(pre, n_members, n_rows); its
 *                   layout is the forward one for n_members * n_rows rows, member-major, with
 *                   the shards split into page ranges as a replay block of n_rows rows would
 *                   be (see ls_replay_fwd), so that each member's O and LSE equal those of its
 *                   own ls_replay_fwd bit for bit.
 * The members' rows together obey the block-size limit of ls_fwd_workspace_bytes.
 * Errors as for ls_replay_fwd.
 */
size_t ls_score_workspace_bytes(const ls_prefix_t* pre, int64_t n_members, int64_t n_rows);
int ls_score_fwd(const ls_prefix_t* pre, int64_t n_members, const void* q, int64_t n_rows,
                 const void* k_resp, const void* v_resp, void* o, float* lse, void* workspace,
                 size_t ws_bytes, ls_stream_t stream);

/*
 * ls_replay_bwd -- backward of one replayed response block for the loss sum(O * dO)
 * (digest, "Method", step 3: backpropagate and accumulate; explainer, "Two incompatible
 * architectures": response blocks replayed in reverse, K/V gradient pages allocated when
 * a response backward touches them).  P is recomputed from the stored LSE.
 *
 *   q, k_resp, v_resp, n_resp_keys, q_start, n_rows   as for ls_replay_fwd.
 *   o               device [n_rows, hq, d] of pre->dtype: the forward's output.
 *   lse             device float32 [n_rows, hq]: the forward's LSE.
 *   dout            device [n_rows, hq, d] of pre->dtype: dL/dO.
 *   dq              device float32 [n_rows, hq, d]: overwritten with dL/dq; or NULL, for the
 *                   gradients of the keys and values only (no dQ pass and no stored dS: the
 *                   caller formed dQ with ls_replay_fwd_dq).
 *   dk_resp,dv_resp device float32 [n_resp_keys, hkv, d]: gradients of response keys
 *                   [0, q_start + n_rows) are added in (written instead when
 *                   resp_first_touch != 0, in which case keys past that range are set
 *                   to zero).
 *   dk_pages,dv_pages
 *                   device float32 [n_phys_pages, hkv, page_size, d], indexed like the
 *                   pools: prompt-key gradients are added in, or written for shards whose
 *                   shard_first_touch[s] != 0 (rows past prefix_len in a partial last
 *                   page are then written as zero).  Physical pages that no logical page
 *                   maps to are left untouched.
 *   shard_first_touch  host uint8 [n_shards], or NULL for "accumulate everywhere".
 *   workspace       device, ws_bytes >= ls_bwd_workspace_bytes(pre, n_rows); with
 *                   room for the block's dS, or for a chunk of it (bf16; see
 *                   ls_bwd_ds_workspace_bytes), dQ is formed from the stored dS instead of
 *                   a recompute.
 * Each gradient element has one writer per call (no atomics); results are
 * deterministic.  Errors as for ls_replay_fwd.
 */
int ls_replay_bwd(const ls_prefix_t* pre, const void* q, int64_t n_rows, int64_t q_start,
                  const void* k_resp, const void* v_resp, int64_t n_resp_keys,
                  const void* o, const float* lse, const void* dout, float* dq,
                  float* dk_resp, float* dv_resp, int resp_first_touch, float* dk_pages,
                  float* dv_pages, const uint8_t* shard_first_touch, void* workspace,
                  size_t ws_bytes, ls_stream_t stream);

/*
 * ls_replay_fwd_dq -- the forward of one replayed response block and its dQ in one pass over
 * the keys, for a dL/dO known before the forward (bf16 pages only).  O and LSE are those of
 * ls_replay_fwd (exact attention; explainer "Two incompatible architectures, same transaction":
 * the owners' softmax statistics compose into the exact global output), and dQ is that of
 * ls_replay_bwd for the loss sum(O * dO):
 *   dQ_i = scale sum_j P_ij (dP_ij - delta_i) K_j,  dP_ij = dO_i . V_j,  delta_i = dO_i . O_i.
 * delta needs every key, so the pass keeps, relative to the online softmax's reference,
 * sum p V, sum p dP K, sum p K, sum p and sum p dP per row and part, and forms
 * dQ = scale (A / l - delta B / l) after the parts are merged.  The keys' and values'
 * gradients then come from ls_replay_bwd with dq = NULL.  The results agree with
 * ls_replay_fwd + ls_replay_bwd to rounding, not bit for bit: the products run on the
 * 16x16x32 instruction, 16 rows per wave.
 *
 *   pre, q, n_rows, q_start, k_resp, v_resp, n_resp_keys, o, lse   as for ls_replay_fwd.
 *   dout            device [n_rows, hq, d] bf16: dL/dO.
 *   dq              device float32 [n_rows, hq, d]: overwritten with dL/dq.
 *   workspace       device, ws_bytes >= ls_fwd_dq_workspace_bytes(pre, n_rows); layout
 *                   (float32, n_parts = n_shards + 1): o_parts, A / l parts, B / l parts
 *                   [n_parts, n_rows, hq, d] each, then lse_parts and delta parts
 *                   [n_parts, n_rows, hq] each (delta part = sum p dP / sum p).
 * The caller owns every buffer; nothing is retained.  Errors: as for ls_replay_fwd, and
 * LS_ERR_INVALID for a NULL dout or dq, LS_ERR_UNSUPPORTED for float32 pages.
 */
size_t ls_fwd_dq_workspace_bytes(const ls_prefix_t* pre, int64_t n_rows);
int ls_replay_fwd_dq(const ls_prefix_t* pre, const void* q, int64_t n_rows, int64_t q_start,
                     const void* k_resp, const void* v_resp, int64_t n_resp_keys, const void* dout,
                     void* o, float* lse, float* dq, void* workspace, size_t ws_bytes,
                     ls_stream_t stream);

/*
 * ls_lse_merge -- compose local softmax results into the global one in float32 (digest,
 * "Method", Qwen implementation: global LSE/output merge; the pages keep a BF16 numerator,
 * explainer "The fine print", here every step is float32):
 *   L = m + log sum_p exp(L_p - m), m = max_p L_p;  O = sum_p exp(L_p - L) O_p.
 * A part with L_p = -inf adds nothing; a row where every part is -inf gets L = -inf and
 * O = 0; a row with a NaN L_p gets NaN.  With n_parts == 1 the result equals the input exactly.
 *
 *   o_parts   device float32 [n_parts, n_rows, d]
 *   lse_parts device float32 [n_parts, n_rows]
 *   o_out     device [n_rows, d] of out_dtype;  lse_out device float32 [n_rows].
 * Errors: LS_ERR_INVALID, LS_ERR_UNSUPPORTED (d not a multiple of 4 or > 1024, dtype).
 */
int ls_lse_merge(int n_parts, int64_t n_rows, int d, const float* o_parts,
                 const float* lse_parts, void* o_out, int out_dtype, float* lse_out,
                 ls_stream_t stream);

/*
 * ls_lse_merge_bf16num -- the same merge with the pages' BF16 numerator (explainer, "The fine
 * print": the prototype's global attention merge keeps its numerator in BF16), to measure the
 * error that choice adds.  Each term exp(L_p - m) O_p is rounded to bf16 and so is the running
 * sum after every addition, in part order; L and the denominator sum_p exp(L_p - m) stay
 * float32; O = numerator / denominator.  Arguments and errors as for ls_lse_merge.
 */
int ls_lse_merge_bf16num(int n_parts, int64_t n_rows, int d, const float* o_parts,
                         const float* lse_parts, void* o_out, int out_dtype, float* lse_out,
                         ls_stream_t stream);

/*
 * One-writer counters, a debug check of the backward's ownership rule (each gradient element
 * has exactly one writer per call, which is why the kernels need no atomics: digest,
 * "Method", step 3 accumulates every member's K/V gradients into the same pages, and the
 * explainer, "Two incompatible architectures, same transaction", writes them per page).
 * While counters are registered on the calling thread (ls_debug_set_owner_counts with a
 * non-NULL buffer), every ls_replay_bwd call on that thread first zeroes them on its stream
 * and then every writer adds 1 to the slot of what it writes:
 *   slot (phys * hkv + kv) * 2 + half                    prompt gradient half-page (keys
 *                                                        32 half .. +32 of physical page phys);
 *   R + (page * hkv + kv) * 2 + half                     response gradient half-page, with
 *                                                        R = n_phys_pages * hkv * 2;
 *   Q + (part * n_rows + token) * hq + head              dQ partial row, with
 *                                                        Q = R + ceil(key_end / 64) * hkv * 2:
 *                                                        part < n_shards a shard, n_shards the
 *                                                        response; when the stored-dS dQ pass of
 *                                                        a small block splits every shard into k
 *                                                        page ranges (see ls_replay_fwd), part
 *                                                        < n_shards * k a range, n_shards * k
 *                                                        the response.
 * After a correct call every slot holds 1 if the call writes it and 0 otherwise; a slot above
 * 1 is a second writer.  The caller reads the counters back (the library never synchronises).
 * Counting uses device atomics and costs time; it is for tests and debugging.
 *
 * ls_debug_owner_slots -- slots needed for a block of n_rows rows whose response keys end at
 *   key_end (= q_start + n_rows); 0 (with an error message) for an invalid descriptor.
 * ls_debug_set_owner_counts -- register `counts` (device uint32 [n_slots], owned by the
 *   caller, which keeps it alive while registered) for this thread's backward calls; NULL
 *   turns the counting off.  A registered ls_replay_bwd call fails with LS_ERR_INVALID if
 *   n_slots is below ls_debug_owner_slots for its block, and with LS_ERR_UNSUPPORTED for
 *   float32 descriptors (the counters cover the bf16 matrix-core kernels) and for dq = NULL
 *   (the dQ part rows are among the counted slots).
 */
size_t ls_debug_owner_slots(const ls_prefix_t* pre, int64_t n_rows, int64_t key_end);
int ls_debug_set_owner_counts(uint32_t* counts, size_t n_slots);

/*
 * Kernel timing, for diagnostics and benchmarks.  Between ls_profile_begin() and
 * ls_profile_end(), every kernel the library launches (from any thread, on any stream) is
 * bracketed by a pair of HIP events recorded on that kernel's stream, so each record is the
 * kernel's own duration on the device.  ls_profile_end() waits for the recorded events (a
 * host synchronisation), sums the durations per kernel name and writes up to max_entries
 * records, in name order, to `out` (host memory); *n_entries receives the number of
 * distinct kernels seen.  Recording adds one event pair per launch and nothing else.
 * Errors: LS_ERR_INVALID (NULL pointers, end without begin), LS_ERR_HIP.
 */
typedef struct ls_kernel_stat {
    char name[48];
    int64_t launches;
    double total_ms;
} ls_kernel_stat_t;

int ls_profile_begin(void);
int ls_profile_end(ls_kernel_stat_t* out, int max_entries, int* n_entries);

#ifdef __cplusplus
}
#endif

#endif /* LONGSTRAW_H */
