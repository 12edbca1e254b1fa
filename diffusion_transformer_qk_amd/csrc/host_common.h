// host_common.h -- host-side argument checks shared by the library's entry
// points.  Internal header (not part of the C ABI).
#pragma once

#include <stdint.h>

namespace qkr_host {

inline bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// True when the byte ranges [a, a + na) and [b, b + nb) share a byte.
inline bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na != 0 && nb != 0 && x < y + nb && y < x + na;
}

}  // namespace qkr_host
