// Internal helpers shared by the library's translation units (host side).
#pragma once

#include <stdint.h>

#include <string>

#include "pagedkv.h"

namespace pkv {

// Records msg as this thread's last error and returns code.
int fail(int code, const std::string& msg);
// Clears the last error and returns PKV_OK.
int ok();

inline int esize_of(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kBlockSize = 16;

}  // namespace pkv
