// Host side: the launch shape of the token-row kernels (finalize and gated norms) and the
// width limits they share.
#pragma once

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "api_util.h"
#include "row_norm.h"

namespace mf {

constexpr int32_t kMaxH = 32768;   // 64 slots of 512 values
constexpr int kMaxWaves = 16;           // waves per workgroup (1024 threads)
constexpr int kMaxVpl = 4;              // plain finalize and gated kernels: 4 x 16 x 512 = 32768

inline bool eps_ok(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

inline bool row_width_supported(int32_t H) { return H >= 8 && H <= kMaxH && H % 8 == 0; }

// Launch shape of the token-row kernels: one workgroup per token, `wpt` waves holding `vpl`
// slots each.  It depends on H only, so a token's result never depends on the batch.
struct RowShape {
    int tail;       // RowTail: how the row's last slot meets H
    int vpl;        // slots per wave (kernel instantiation)
    int wpt;        // waves per token = per workgroup
    int block;      // threads per workgroup
    int64_t grid;   // workgroups = tokens
    int nr;         // row sums per reduction barrier
    int nl = 0;     // slots per wave staged in LDS (the slot-serial kernel of wide rows)
    size_t lds;     // dynamic LDS bytes
};

// One slot of 512 values per wave, unless the row needs more than max_waves waves; never more
// than max_vpl slots per wave (the widest compiled instantiation).
inline RowShape row_shape(int64_t T, int32_t H, int max_waves, int max_vpl) {
    const int ns = (H + kSlot - 1) / kSlot;
    // Waves per token are a power of two (measured faster on MI355X than an odd wave count;
    // spare waves hold slots past H and skip their loads).  Among the slots-per-wave values
    // that fit in 16 waves, take the one that leaves the fewest spare slots, then the
    // smallest.
    const int vmin = (ns + max_waves - 1) / max_waves;
    int best_v = vmin, best_waste = 1 << 30;
    for (int v = vmin; v <= std::min(vmin + 2, max_vpl); ++v) {
        const int waste = pow2_at_least((ns + v - 1) / v) * v - ns;
        if (waste < best_waste) {
            best_v = v;
            best_waste = waste;
        }
    }
    RowShape s;
    s.vpl = best_v;
    s.wpt = pow2_at_least((ns + s.vpl - 1) / s.vpl);
    s.tail = H != ns * kSlot ? kRowRagged : (ns == s.wpt * s.vpl ? kRowFull : kRowWhole);
    s.block = kWave * s.wpt;
    s.grid = T;
    s.nr = 1;
    s.lds = token_sum_lds_bytes(s.wpt, 1);
    return s;
}

// Kernel of the gated-residual RMSNorm for a shape (single or dual output), or nullptr.
const void* gated_kernel_for(const RowShape& s, bool dual);

}  // namespace mf
