// Host-only stand-ins for the kernel launchers that the C ABI front end (abi.cpp) calls, so that
// the front end can be built with the host compiler and its sanitizers, without a GPU.  Each
// records the arguments of its last call and returns hipSuccess; nothing is launched.
#include "abi_stubs.hpp"

#include "../../include/longstraw.h"

namespace stub {
Record last;
}

namespace ls {

static hipError_t note(const char* name, const AttnArgs* a = nullptr) {
    stub::last.calls++;
    stub::last.name = name;
    if (a) stub::last.args = *a;
    return hipSuccess;
}

hipError_t launch_capture(const void*, const void*, int, int64_t, int64_t, const int32_t*, void*, void*, int, int64_t,
                          int, int, hipStream_t) {
    return note("capture");
}
hipError_t launch_gather(const void*, int, const int32_t*, int64_t, int64_t, int64_t, int, int, void*, hipStream_t) {
    return note("gather");
}
hipError_t launch_lse_merge(int n_parts, int64_t, int, const float*, const float*, void*, int, float*, hipStream_t,
                            bool) {
    if (stub::last.merges < 8) stub::last.merge_parts[stub::last.merges] = n_parts;
    stub::last.merges++;
    return note("lse_merge");
}
hipError_t launch_delta(const void*, const void*, int, int64_t, int, float*, hipStream_t) { return note("delta"); }
hipError_t launch_sum_parts(int n_parts, int64_t, const float* src, float*, hipStream_t) {
    stub::last.sum_n = n_parts;
    stub::last.sum_src = src;
    return note("sum_parts");
}
hipError_t launch_zero(float*, int64_t, hipStream_t) { return note("zero"); }
hipError_t launch_fwd_generic(const AttnArgs& a, hipStream_t) { return note("fwd_generic", &a); }
hipError_t launch_bwd_generic(const AttnArgs& a, hipStream_t) { return note("bwd_generic", &a); }
hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t) { return note("fwd_mfma", &a); }
hipError_t launch_fwd_dq_mfma(const AttnArgs& a, float* a_parts, float* b_parts, float* delta_parts, hipStream_t) {
    stub::last.fdq_a = a_parts;
    stub::last.fdq_b = b_parts;
    stub::last.fdq_delta = delta_parts;
    return note("fwd_dq_mfma", &a);
}
hipError_t launch_fwd_dq_merge(int n_parts, int64_t n_rows, int, const float* lse_parts, const float* lse,
                               const float* a_parts, const float* b_parts, const float* delta_parts, float scale,
                               float* dq, hipStream_t) {
    stub::last.dqm_parts = n_parts;
    stub::last.dqm_rows = n_rows;
    stub::last.dqm_lse_parts = lse_parts;
    stub::last.dqm_lse = lse;
    stub::last.dqm_a = a_parts;
    stub::last.dqm_b = b_parts;
    stub::last.dqm_delta = delta_parts;
    stub::last.dqm_scale = scale;
    stub::last.dqm_dq = dq;
    return note("fwd_dq_merge");
}
hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
    stub::last.calls++;
    stub::last.name = "noalloc_scratch";
    *ptr = (void*)0x7000000;
    *bytes = LS_NOALLOC_SCRATCH_BYTES;
    return hipSuccess;
}
hipError_t launch_bwd_mfma(const AttnArgs& a, hipStream_t) {
    // the stored-dS chunk plan the front end chose is what a test checks, so keep it apart from
    // the merge / sum launches that follow
    stub::last.bwd = a;
    return note("bwd_mfma", &a);
}

}  // namespace ls
