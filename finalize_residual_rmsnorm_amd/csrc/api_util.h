// Host-side helpers shared by the C-ABI sources: argument checks and launch bookkeeping.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "mf.h"

namespace mf {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Do [a, a+na) and [b, b+nb) share a byte?
inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

inline int pow2_at_least(int n) {
    int p = 1;
    while (p < n) p *= 2;
    return p;
}

// AMD grids count work-items in 32 bits per dimension.
inline bool grid_fits(int64_t blocks, int threads) {
    return blocks >= 1 && blocks * int64_t(threads) <= int64_t(UINT32_MAX);
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MF_OK : MF_ERR_HIP; }

}  // namespace mf
