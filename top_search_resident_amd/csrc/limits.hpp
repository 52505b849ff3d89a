// limits.hpp -- the engine limits of the C ABI (include/resident_topk.h), host
// and device independent so that the argument checks also build as plain C++.
#pragma once
#include <stdint.h>

namespace rt {

constexpr int64_t kMaxN = 2147483647LL;  // row / element indices are int32
constexpr int32_t kMaxD = 65536;
constexpr int32_t kMaxK = 1024;
constexpr int32_t kMaxQ = 32;

}  // namespace rt
