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
};
extern Record last;
}  // namespace stub
