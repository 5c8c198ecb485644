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
};
extern Record last;
}  // namespace stub
