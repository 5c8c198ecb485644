// Host-only checks of the C ABI front end (abi.cpp), built with the host compiler's address and
// undefined-behaviour sanitizers against stand-in kernel launchers (abi_stubs.cpp): argument
// validation, workspace sizing, the stored-dS chunk plan, the small-block split, the page-table check
// and the per-thread error message.  Device pointers are fake and never dereferenced (no launch happens).  Prints
// one line per check and exits non-zero on the first failure.
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/longstraw.h"
#include "abi_stubs.hpp"

namespace {

int g_failed = 0;

void expect(bool ok, const char* what) {
    std::printf("%s %s\n", ok ? "ok" : "FAIL", what);
    if (!ok) g_failed++;
}

void* fake(uintptr_t i) { return (void*)(0x100000 + 0x1000 * i); }

struct Prefix {
    std::vector<int64_t> bounds;
    ls_prefix_t p{};
    Prefix(int hq, int hkv, int d, int dtype, int64_t prefix_len, std::vector<int64_t> b) : bounds(std::move(b)) {
        p.hq = hq;
        p.hkv = hkv;
        p.d = d;
        p.page_size = 64;
        p.dtype = dtype;
        p.n_shards = (int)bounds.size() - 1;
        p.prefix_len = prefix_len;
        p.n_phys_pages = (prefix_len + 63) / 64 + 3;
        p.page_table = (const int32_t*)fake(1);
        p.k_pages = fake(2);
        p.v_pages = fake(3);
        p.shard_page_bounds = bounds.data();
        p.softmax_scale = 0.0625f;
    }
};

std::vector<int64_t> even(int64_t pages, int s) {
    std::vector<int64_t> b;
    for (int i = 0; i <= s; i++) b.push_back(i * pages / s);
    return b;
}

int bwd(const ls_prefix_t* p, int64_t n, int64_t q0, size_t ws_bytes, int first = 1) {
    return ls_replay_bwd(p, fake(4), n, q0, fake(5), fake(6), q0 + n + 5, fake(7), (const float*)fake(8), fake(9),
                         (float*)fake(10), (float*)fake(11), (float*)fake(12), first, (float*)fake(13),
                         (float*)fake(14), nullptr, fake(15), ws_bytes, nullptr);
}

void page_table_checks() {
    const int32_t good[5] = {4, 0, 2, 1, 3};
    expect(ls_check_page_table(good, 5, 5) == LS_OK, "page table: a permutation");
    expect(ls_check_page_table(good, 3, 7) == LS_OK, "page table: injective into a larger pool");
    const int32_t dup[4] = {0, 2, 2, 1};
    expect(ls_check_page_table(dup, 4, 4) == LS_ERR_INVALID &&
               std::strstr(ls_last_error(), "page_table[2]") != nullptr,
           "page table: a repeated entry names its logical page");
    const int32_t out[3] = {0, -1, 1};
    expect(ls_check_page_table(out, 3, 3) == LS_ERR_INVALID && std::strstr(ls_last_error(), "outside") != nullptr,
           "page table: a negative entry");
    const int32_t big[3] = {0, 1, 3};
    expect(ls_check_page_table(big, 3, 3) == LS_ERR_INVALID, "page table: an entry past the pool");
    expect(ls_check_page_table(good, 5, 4) == LS_ERR_INVALID, "page table: more logical than physical pages");
    expect(ls_check_page_table(nullptr, 0, 0) == LS_OK, "page table: empty");
    expect(ls_check_page_table(nullptr, 2, 2) == LS_ERR_INVALID, "page table: NULL");
    std::vector<int32_t> large(1 << 16);
    for (uint32_t i = 0; i < (1u << 16); i++) large[i] = (int32_t)((i * 40503u) & 0xffffu);  // odd multiplier: a permutation
    expect(ls_check_page_table(large.data(), 1 << 16, 1 << 16) == LS_OK, "page table: 65,536 pages");
}

void prefix_checks() {
    Prefix ok(24, 4, 256, LS_DTYPE_BF16, 2000, {0, 5, 19, 32});
    expect(ls_fwd_workspace_bytes(&ok.p, 100) == 4ull * 4 * 100 * 24 * 257, "forward workspace size");
    Prefix bad = ok;
    bad.p.shard_page_bounds = bad.bounds.data();
    bad.bounds[3] = 31;
    expect(ls_fwd_workspace_bytes(&bad.p, 10) == 0 && std::strstr(ls_last_error(), "shard bounds"),
           "bounds must end at the number of logical pages");
    Prefix many(8, 2, 64, LS_DTYPE_BF16, 64 * 640, even(640, 64));
    expect(ls_fwd_workspace_bytes(&many.p, 16) > 0, "64 shards accepted");
    Prefix too_many(8, 2, 64, LS_DTYPE_BF16, 64 * 650, even(650, 65));
    expect(ls_fwd_workspace_bytes(&too_many.p, 16) == 0, "65 shards rejected");
    Prefix empty(8, 2, 64, LS_DTYPE_BF16, 0, {0, 0});
    empty.p.page_table = nullptr;
    empty.p.k_pages = empty.p.v_pages = nullptr;
    expect(ls_fwd_workspace_bytes(&empty.p, 16) > 0, "an empty prompt needs no pages");
    expect(ls_replay_fwd(&ok.p, fake(4), int64_t(1) << 40, 0, fake(5), fake(6), int64_t(1) << 41, fake(7),
                         (float*)fake(8), fake(9), ~size_t(0), nullptr) == LS_ERR_INVALID,
           "a block too large for the kernels' 32-bit offsets is rejected");
}

void dispatch_checks() {
    Prefix pb(24, 4, 256, LS_DTYPE_BF16, 2000, {0, 5, 19, 32});
    const size_t fw = ls_fwd_workspace_bytes(&pb.p, 100);
    stub::last = stub::Record();
    int rc = ls_replay_fwd(&pb.p, fake(4), 100, 44, fake(5), fake(6), 144, fake(7), (float*)fake(8), fake(9), fw,
                           nullptr);
    expect(rc == LS_OK && std::string(stub::last.name) == "lse_merge" && stub::last.calls == 2,
           "bf16 forward: matrix-core forward, then the merge");
    expect(stub::last.args.key_end == 144 && stub::last.args.n_parts == 4 && stub::last.args.shard_lo[2] == 19 &&
               stub::last.args.o_parts == (float*)fake(9),
           "forward arguments: key range, parts, shard bounds, workspace");
    expect(ls_replay_fwd(&pb.p, fake(4), 100, 44, fake(5), fake(6), 144, fake(7), (float*)fake(8), fake(9), fw - 1,
                         nullptr) == LS_ERR_WORKSPACE,
           "a short forward workspace is rejected");
    Prefix pf(4, 1, 64, LS_DTYPE_F32, 4096, {0, 32, 64});
    stub::last = stub::Record();
    rc = ls_replay_fwd(&pf.p, fake(4), 256, 0, fake(5), fake(6), 256, fake(7), (float*)fake(8), fake(9),
                       ls_fwd_workspace_bytes(&pf.p, 256), nullptr);
    expect(rc == LS_OK && stub::last.calls == 2, "f32 forward: the vector-ALU forward, then the merge");
}

void noalloc_checks() {
    Prefix pb(24, 4, 256, LS_DTYPE_BF16, 64 * 80, even(80, 8));
    const int64_t per_row = (int64_t)ls_fwd_workspace_bytes(&pb.p, 1);
    const int64_t max_rows = (int64_t)(LS_NOALLOC_SCRATCH_BYTES / per_row);
    stub::last = stub::Record();
    int rc = ls_replay_fwd_noalloc(&pb.p, fake(4), max_rows + 1, 0, fake(5), fake(6), max_rows + 1, fake(7),
                                   (float*)fake(8), nullptr);
    expect(rc == LS_ERR_WORKSPACE && stub::last.calls == 0 && std::strstr(ls_last_error(), "split the block"),
           "no-allocation forward: one row past the scratch is refused before any launch");
    stub::last = stub::Record();
    rc = ls_replay_fwd_noalloc(&pb.p, fake(4), max_rows, 0, fake(5), fake(6), max_rows, fake(7), (float*)fake(8),
                               nullptr);
    expect(rc == LS_OK && stub::last.args.o_parts == (float*)0x7000000 && std::string(stub::last.name) == "lse_merge",
           "no-allocation forward: the largest block runs in the scratch array");
    stub::last = stub::Record();
    rc = ls_replay_fwd_noalloc(&pb.p, fake(4), 0, 0, fake(5), fake(6), 0, fake(7), (float*)fake(8), nullptr);
    expect(rc == LS_OK && stub::last.calls == 0, "no-allocation forward: an empty block does nothing");
}

void chunk_plan_checks() {
    // 2,000-token prompt in 3 uneven shards, 24/4 heads, a 128-row block at rows [128, 256)
    Prefix pb(24, 4, 256, LS_DTYPE_BF16, 2000, {0, 5, 19, 32});
    const int64_t n = 128, q0 = 128, kend = q0 + n;
    const size_t rec = ls_bwd_workspace_bytes(&pb.p, n);
    stub::last = stub::Record();
    expect(bwd(&pb.p, n, q0, rec) == LS_OK && stub::last.bwd.ds == nullptr, "recompute workspace: no stored dS");
    const size_t all = ls_bwd_ds_workspace_bytes(&pb.p, n, kend);
    expect(all == ls_bwd_ds_chunk_workspace_bytes(&pb.p, n, kend, 4, 4), "chunk size of (all heads, all parts)");
    stub::last = stub::Record();
    expect(bwd(&pb.p, n, q0, all) == LS_OK && stub::last.bwd.ds != nullptr && stub::last.bwd.ds_heads == 4 &&
               stub::last.bwd.ds_parts == 4,
           "full workspace: every kv head over all keys");
    for (int h = 1; h <= 3; h++) {
        const size_t ws = ls_bwd_ds_chunk_workspace_bytes(&pb.p, n, kend, h, 4);
        stub::last = stub::Record();
        const bool ok = bwd(&pb.p, n, q0, ws) == LS_OK && stub::last.bwd.ds_heads == h && stub::last.bwd.ds_parts == 4;
        expect(ok, ("exact workspace of " + std::to_string(h) + " kv head(s) selects that chunk").c_str());
    }
    for (int k = 1; k <= 3; k++) {
        const size_t ws = ls_bwd_ds_chunk_workspace_bytes(&pb.p, n, kend, 1, k);
        stub::last = stub::Record();
        const bool ok = bwd(&pb.p, n, q0, ws) == LS_OK && stub::last.bwd.ds_heads == 1 &&
                        stub::last.bwd.ds_parts >= k && stub::last.bwd.ds_parts < 4 &&
                        stub::last.bwd.ds_kslots ==
                            ls::ds_chunk_slots(pb.bounds.data(), 3, kend, stub::last.bwd.ds_parts);
        expect(ok, ("exact workspace of 1 kv head x " + std::to_string(k) + " part(s) selects a part chunk").c_str());
    }
    const size_t one = ls_bwd_ds_chunk_workspace_bytes(&pb.p, n, kend, 1, 1);
    stub::last = stub::Record();
    expect(bwd(&pb.p, n, q0, one - 1) == LS_OK && stub::last.bwd.ds == nullptr,
           "one byte short of the smallest chunk: recompute");
    expect(ls_bwd_ds_chunk_workspace_bytes(&pb.p, n, kend, 2, 3) == 0, "several kv heads need all key parts");
    expect(ls_bwd_ds_chunk_workspace_bytes(&pb.p, n, kend, 0, 4) == 0, "zero heads rejected");
    expect(ls_bwd_ds_chunk_workspace_bytes(&pb.p, n, kend, 1, 5) == 0, "more parts than there are rejected");
    // the chunks: odd page bounds put a page pair in two chunks; the response is the last part
    const ls::PartChunk c0 = ls::part_chunk(pb.bounds.data(), 3, kend, 0, 1);
    const ls::PartChunk c1 = ls::part_chunk(pb.bounds.data(), 3, kend, 1, 2);
    const ls::PartChunk c3 = ls::part_chunk(pb.bounds.data(), 3, kend, 3, 4);
    expect(c0.pg_lo == 0 && c0.pg_hi == 5 && c0.pair_lo == 0 && c0.n_pairs == 3 && !c0.resp, "chunk of shard 0");
    expect(c1.pg_lo == 5 && c1.pg_hi == 19 && c1.pair_lo == 2 && c1.n_pairs == 8 && !c1.resp, "chunk of shard 1");
    expect(c3.n_pairs == 0 && c3.resp && c3.n_resp_pairs == 2, "chunk of the response keys");
    // first touch past the block: the response gradients past key_end are zeroed
    stub::last = stub::Record();
    expect(bwd(&pb.p, n, q0, rec, 1) == LS_OK && std::string(stub::last.name) == "zero",
           "first touch zeroes response gradients past the block");
    Prefix pf(4, 1, 64, LS_DTYPE_F32, 4096, {0, 32, 64});
    expect(ls_bwd_ds_workspace_bytes(&pf.p, 64, 64) == ls_bwd_workspace_bytes(&pf.p, 64),
           "f32 stores no dS");
}

// The sub-range split of a small block's shards (launch.hpp): how many ranges, their page
// bounds, and what the front end launches and sizes for them.
void split_checks() {
    bool ok = true;
    const int64_t tiles[] = {1, 2, 3, 5, 12, 48, 96, 200};
    const int shards[] = {1, 2, 3, 8, 17, 64};
    const int heads[] = {1, 2, 4, 8};
    const int64_t pages[] = {0, 63, 64, 640, 1024, 32768, int64_t(1) << 20};
    for (int64_t t : tiles)
        for (int s : shards)
            for (int h : heads)
                for (int64_t pg : pages) {
                    const int k = ls::sub_split(t, s, h, pg);
                    const int64_t wg = t * s * h;  // workgroups with one range per shard
                    bool c = k >= 1 && (int64_t)k * s <= ls::kMaxSubParts;
                    if (wg >= 768) c = c && k == 1;                          // the chip is already full
                    if (k > 1) c = c && (int64_t)k * s * 64 <= pg;            // >= 64 pages a range on average
                    if (k > 1) c = c && (int64_t)(k - 1) * wg < 768;          // no more ranges than it takes
                    if (wg < 768 && (int64_t)k * wg < 768)                    // short of the target only when capped
                        c = c && ((int64_t)(k + 1) * s * 64 > pg || (k + 1) * s > ls::kMaxSubParts);
                    if (!c) {
                        std::printf("  sub_split(%lld, %d, %d, %lld) = %d\n", (long long)t, s, h, (long long)pg, k);
                        ok = false;
                    }
                }
    expect(ok, "sub_split: fills the chip, at least 64 pages a range, at most 256 ranges");
    expect(ls::fwd_split(16, 6, 8, 4, 32832) > 1 && ls::fwd_split(1024, 6, 8, 4, 32832) == 1,
           "a 16-row block splits, a 1,024-row block does not (8 shards, 4 kv heads)");

    ok = true;
    const std::vector<std::vector<int64_t>> cases = {{0, 5, 19, 32}, {0, 0, 3, 3, 10}, {0, 1}, {0, 1000}};
    for (const auto& lo : cases)
        for (int k = 1; k <= 8; k++) {
            const int s = (int)lo.size() - 1;
            int64_t out[ls::kMaxSubParts + 1];
            ls::split_bounds(lo.data(), s, k, out);
            for (int i = 0; i <= s; i++) ok = ok && out[i * k] == lo[i];  // the shard bounds stay bounds
            for (int i = 0; i < s; i++)
                for (int j = 0; j < k; j++) {
                    const int64_t len = out[i * k + j + 1] - out[i * k + j], shard = lo[i + 1] - lo[i];
                    ok = ok && len >= shard / k && len <= (shard + k - 1) / k;  // as even as pages allow
                }
        }
    expect(ok, "split_bounds: keeps the shard bounds, ranges differ by at most one page");

    // 16 rows over a 65,536-token prompt in two shards, 24 / 4 heads, d = 256: eight ranges a shard
    Prefix big(24, 4, 256, LS_DTYPE_BF16, 65536, {0, 512, 1024});
    const int64_t n = 16, rows_hq = n * 24;
    const int k = ls::fwd_split(n, 6, 2, 4, 1024);
    const size_t fw = ls_fwd_workspace_bytes(&big.p, n);
    expect(k == 8 && fw == sizeof(float) * (size_t)rows_hq * 257 * (3 + 2 * 8 + 1),
           "split forward workspace: the parts, then the ranges' results");
    stub::last = stub::Record();
    int rc = ls_replay_fwd(&big.p, fake(4), n, 0, fake(5), fake(6), n, fake(7), (float*)fake(8), fake(9), fw, nullptr);
    bool bounds_ok = true;
    for (int j = 0; j <= 16; j++) bounds_ok = bounds_ok && stub::last.args.shard_lo[j] == 64 * j;
    expect(rc == LS_OK && stub::last.args.n_shards == 16 && stub::last.args.n_parts == 17 && bounds_ok &&
               stub::last.args.o_parts == (float*)fake(9) + rows_hq * 257 * 3,
           "split forward: one launch over 16 ranges and the response, after the parts");
    const int* mp = stub::last.merge_parts;
    expect(stub::last.merges == 4 && mp[0] == 8 && mp[1] == 8 && mp[2] == 1 && mp[3] == 3 && stub::last.calls == 5,
           "split forward: a merge per shard, one for the response, then the final merge");
    expect(ls_replay_fwd(&big.p, fake(4), n, 0, fake(5), fake(6), n, fake(7), (float*)fake(8), fake(9), fw - 1,
                         nullptr) == LS_ERR_WORKSPACE,
           "split forward: a workspace without the ranges' area is rejected");
    Prefix big_f32(24, 4, 256, LS_DTYPE_F32, 65536, {0, 512, 1024});
    expect(ls_fwd_workspace_bytes(&big_f32.p, n) == sizeof(float) * (size_t)rows_hq * 257 * 3,
           "the vector-ALU forward does not split");

    // the stored-dS dQ pass of the same block: eight ranges a shard, summed from their own area
    const int64_t q0 = 0, kend = q0 + n;
    const int kq = ls::dqs_split(n, 6, 2, 4, 1024);
    const size_t rec = ls_bwd_workspace_bytes(&big.p, n);
    const size_t all = ls_bwd_ds_workspace_bytes(&big.p, n, kend);
    stub::last = stub::Record();
    rc = bwd(&big.p, n, q0, all, 0);
    const float* sub = stub::last.bwd.dq_sub;
    const size_t sub_bytes = sizeof(float) * (size_t)(2 * kq + 1) * rows_hq * 256;
    expect(rc == LS_OK && kq == 8 && stub::last.bwd.ds != nullptr && stub::last.bwd.dq_sub_k == kq &&
               (char*)sub + sub_bytes == (char*)fake(15) + rec && ((char*)sub - (char*)fake(15)) % 256 == 0,
           "split dQ pass: sub-range partials at the end of the backward workspace, 256-byte aligned");
    expect(stub::last.sum_n == 2 * kq + 1 && stub::last.sum_src == sub, "split dQ pass: the sum reads the sub-ranges");
    expect(ls_debug_owner_slots(&big.p, n, kend) ==
               (size_t)ls::owner_slots(big.p.n_phys_pages, 4, 24, 2 * kq + 1, n, kend),
           "split dQ pass: a counter slot per sub-range partial row");
    stub::last = stub::Record();
    rc = bwd(&big.p, n, q0, rec, 0);
    expect(rc == LS_OK && stub::last.bwd.ds == nullptr && stub::last.bwd.dq_sub_k == 0 && stub::last.sum_n == 3,
           "recomputing dQ pass: no split, the sum over the shard parts");
    const size_t part_chunk = ls_bwd_ds_chunk_workspace_bytes(&big.p, n, kend, 1, 2);
    stub::last = stub::Record();
    rc = bwd(&big.p, n, q0, part_chunk, 0);
    expect(rc == LS_OK && stub::last.bwd.ds != nullptr && stub::last.bwd.ds_parts < 3 &&
               stub::last.bwd.dq_sub_k == 0 && stub::last.sum_n == 3,
           "stored dS in key-part chunks: no split");
}

void thread_checks() {
    // the error message belongs to the calling thread
    const int32_t dup[2] = {1, 1};
    ls_check_page_table(dup, 2, 2);
    std::string other;
    std::thread t([&] {
        const int32_t good[2] = {1, 0};
        ls_check_page_table(good, 2, 2);
        other = ls_last_error();
    });
    t.join();
    expect(other.empty() && std::strstr(ls_last_error(), "already mapped") != nullptr, "per-thread error message");
}

// The fused forward + dQ pass: validation, the workspace layout it hands the kernels, and the
// backward that then forms the key and value gradients only.
void fused_checks() {
    Prefix pb(24, 4, 256, LS_DTYPE_BF16, 2000, {0, 5, 19, 32});
    const int64_t n = 100, rows = n * 24;
    const size_t ws = ls_fwd_dq_workspace_bytes(&pb.p, n);
    expect(ws == sizeof(float) * 4 * rows * (3 * 256 + 2), "fused workspace: three d-wide and two scalar parts");
    auto call = [&](const void* dout, float* dq, size_t bytes) {
        return ls_replay_fwd_dq(&pb.p, fake(4), n, 44, fake(5), fake(6), 144, dout, fake(7), (float*)fake(8), dq,
                                fake(9), bytes, nullptr);
    };
    stub::last = stub::Record();
    int rc = call(fake(16), (float*)fake(17), ws);
    const float* base = (const float*)fake(9);
    const size_t pe = (size_t)4 * rows * 256;
    expect(rc == LS_OK && stub::last.calls == 3 && std::string(stub::last.name) == "fwd_dq_merge" &&
               stub::last.merges == 1 && stub::last.merge_parts[0] == 4,
           "fused: kernel, LSE merge, dQ merge");
    expect(stub::last.args.o_parts == base && stub::last.fdq_a == base + pe && stub::last.fdq_b == base + 2 * pe &&
               stub::last.args.lse_parts == base + 3 * pe && stub::last.fdq_delta == base + 3 * pe + 4 * rows &&
               stub::last.args.dout == fake(16) && stub::last.args.key_end == 144 && stub::last.args.n_parts == 4,
           "fused: workspace layout and arguments");
    expect(stub::last.dqm_parts == 4 && stub::last.dqm_rows == rows && stub::last.dqm_dq == (float*)fake(17) &&
               stub::last.dqm_lse == (const float*)fake(8) && stub::last.dqm_a == base + pe &&
               stub::last.dqm_b == base + 2 * pe && stub::last.dqm_lse_parts == base + 3 * pe &&
               stub::last.dqm_delta == base + 3 * pe + 4 * rows && stub::last.dqm_scale == 0.0625f,
           "dQ merge: parts, merged LSE, output, scale");
    stub::last = stub::Record();
    expect(call(fake(16), (float*)fake(17), ws - 1) == LS_ERR_WORKSPACE && stub::last.calls == 0,
           "fused: a short workspace is rejected before any launch");
    expect(call(nullptr, (float*)fake(17), ws) == LS_ERR_INVALID && call(fake(16), nullptr, ws) == LS_ERR_INVALID,
           "fused: NULL dout or dq is rejected");
    Prefix pf(4, 1, 64, LS_DTYPE_F32, 4096, {0, 32, 64});
    expect(ls_replay_fwd_dq(&pf.p, fake(4), 256, 0, fake(5), fake(6), 256, fake(16), fake(7), (float*)fake(8),
                            (float*)fake(17), fake(9), ls_fwd_dq_workspace_bytes(&pf.p, 256), nullptr) ==
               LS_ERR_UNSUPPORTED,
           "fused: float32 pages are unsupported");
    stub::last = stub::Record();
    expect(ls_replay_fwd_dq(&pb.p, fake(4), 0, 44, fake(5), fake(6), 144, fake(16), fake(7), (float*)fake(8),
                            (float*)fake(17), nullptr, 0, nullptr) == LS_OK &&
               stub::last.calls == 0,
           "fused: an empty block launches nothing");
    // the backward without dQ: no stored dS even with room for it, no part sum
    const size_t ds_ws = ls_bwd_ds_workspace_bytes(&pb.p, n, 144);
    stub::last = stub::Record();
    rc = ls_replay_bwd(&pb.p, fake(4), n, 44, fake(5), fake(6), 149, fake(7), (const float*)fake(8), fake(16),
                       nullptr, (float*)fake(11), (float*)fake(12), 1, (float*)fake(13), (float*)fake(14), nullptr,
                       fake(15), ds_ws, nullptr);
    expect(rc == LS_OK && stub::last.bwd.skip_dq && stub::last.bwd.ds == nullptr && stub::last.sum_n == 0,
           "backward with dq = NULL: key and value gradients only");
    stub::last = stub::Record();
    rc = bwd(&pb.p, n, 44, ds_ws);
    expect(rc == LS_OK && !stub::last.bwd.skip_dq && stub::last.bwd.ds != nullptr && stub::last.sum_n > 0,
           "backward with dq: the stored-dS dQ pass and its part sum, as before");
}

}  // namespace

int main() {
    page_table_checks();
    prefix_checks();
    dispatch_checks();
    noalloc_checks();
    chunk_plan_checks();
    split_checks();
    fused_checks();
    thread_checks();
    std::printf("%s: %d failure(s)\n", g_failed ? "FAILED" : "PASSED", g_failed);
    return g_failed ? 1 : 0;
}
