// Shared by the two halves of the matrix-core backward (dK/dV in attn_mfma_bwd.hip, dQ in
// attn_mfma_dq.hip): the group-major per-kv-head view of one block that the prep kernel
// writes.
#pragma once

#include "mfma_tiles.hpp"

namespace ls {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Per-kv-head, group-major views of the block: row r of kv head h is (token r / g, query head
// h * g + r % g); rows_pad rows per head.
struct GroupRows {
    f32x2* lsed;     // [hkv][rows_pad] (LSE * log2 e, delta)
    bf16_t* q;       // [hkv][rows_pad][D]
    bf16_t* dout;    // [hkv][rows_pad][D]
    int64_t rows_pad;
};

inline GroupRows group_rows(void* base, int64_t rows_pad, int hkv, int d) {
    GroupRows g;
    g.rows_pad = rows_pad;
    g.lsed = (f32x2*)base;
    g.q = (bf16_t*)(g.lsed + (int64_t)hkv * rows_pad);
    g.dout = g.q + (int64_t)hkv * rows_pad * d;
    return g;
}

hipError_t launch_dq_mfma(const AttnArgs& a, const GroupRows& gr, hipStream_t s);
// dQ parts of kv heads [a.ds_kvh0, a.ds_kvh0 + n_kvh) from the dS that the dK/dV pass stored
// for them (a.ds): shard parts [part0, part0 + n_sp), and the response part if `resp`
hipError_t launch_dqs_mfma(const AttnArgs& a, int n_kvh, int part0, int n_sp, bool resp, hipStream_t s);

}  // namespace ls
