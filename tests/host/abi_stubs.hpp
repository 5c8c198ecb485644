// Records of the stand-in kernel launchers (abi_stubs.cpp) for the host-only build of abi.cpp.
#pragma once

#include <hip/hip_runtime.h>

#include "../../suffix_attention_amd/csrc/launch.hpp"

namespace stub {
struct Record {
    int calls = 0;
    const char* name = "";
    ls::AttnArgs args{};
    ls::AttnArgs bwd{};
    int merges = 0;                   // LSE merge launches, and the parts of the first eight
    int merge_parts[8] = {};
    int sum_n = 0;                    // parts and source of the last dQ part sum
    const float* sum_src = nullptr;
    float *fdq_a = nullptr, *fdq_b = nullptr, *fdq_delta = nullptr;  // fused forward + dQ partials
    int dqm_parts = 0;                // the dQ merge: parts, rows, inputs, output, scale
    int64_t dqm_rows = 0;
    const float *dqm_lse_parts = nullptr, *dqm_lse = nullptr, *dqm_a = nullptr, *dqm_b = nullptr,
                *dqm_delta = nullptr;
    float* dqm_dq = nullptr;
    float dqm_scale = 0.f;
};
extern Record last;
}  // namespace stub
