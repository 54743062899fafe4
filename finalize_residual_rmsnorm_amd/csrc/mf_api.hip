// Host side of the C ABI declared in include/mf.h: argument checks (before any HIP call),
// launch-shape selection and kernel dispatch.  Stateless and allocation-free.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "api_util.h"
#include "finalize_kernel.h"
#include "mf.h"
#include "norm_kernels.h"

namespace {

using namespace mf;

constexpr int32_t kMaxH = 32768;   // 64 slots of 512 values
constexpr int32_t kMaxK = 64;
constexpr int kMaxWaves = 16;           // waves per workgroup (1024 threads)
constexpr int kMaxWavesPerExpert = 8;   // the per-expert variant reduces a batch of row sums
                                        // per barrier; 8 waves keep that LDS under 64 KiB
constexpr int kMaxVpl = 4;              // plain finalize and gated kernels: 4 x 16 x 512 = 32768
constexpr int kMaxVplPerExpert = 8;     // per-expert finalize: 8 x 8 x 512 = 32768
constexpr int kPerHeadGroupsPerWave = 2;

bool eps_ok(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

bool row_width_supported(int32_t H) { return H >= 8 && H <= kMaxH && H % 8 == 0; }

// Launch shape of the token-row kernels: one workgroup per token, `wpt` waves holding `vpl`
// slots each.  It depends on H only, so a token's result never depends on the batch.
struct RowShape {
    int tail;       // RowTail: how the row's last slot meets H
    int vpl;        // slots per wave (kernel instantiation)
    int wpt;        // waves per token = per workgroup
    int block;      // threads per workgroup
    int64_t grid;   // workgroups = tokens
    int nr;         // row sums per reduction barrier
    size_t lds;     // dynamic LDS bytes
};

// One slot of 512 values per wave, unless the row needs more than max_waves waves; never more
// than max_vpl slots per wave (the widest compiled instantiation).
RowShape row_shape(int64_t T, int32_t H, int max_waves, int max_vpl) {
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

// The top-k the finalize kernels are specialised for (all loads of a token issued at once).
constexpr int kCompiledTopK = 8;

constexpr bool uses_compiled_topk(int vpl, bool per_expert);

RowShape finalize_shape(int64_t T, int32_t H, int32_t k, bool per_expert) {
    RowShape s = per_expert ? row_shape(T, H, kMaxWavesPerExpert, kMaxVplPerExpert)
                            : row_shape(T, H, kMaxWaves, kMaxVpl);
    const int kc = k == kCompiledTopK && uses_compiled_topk(s.vpl, per_expert) ? kCompiledTopK : 0;
    s.nr = per_expert ? batch_rows(s.vpl, kc, true) : 1;
    s.lds = token_sum_lds_bytes(s.wpt, s.nr);
    return s;
}

template <int VPL, int KC, bool PE>
const void* finalize_fn(int tail) {
    switch (tail) {
        case kRowFull: return reinterpret_cast<const void*>(&moe_finalize_kernel<VPL, KC, PE, kRowFull>);
        case kRowWhole: return reinterpret_cast<const void*>(&moe_finalize_kernel<VPL, KC, PE, kRowWhole>);
        default: return reinterpret_cast<const void*>(&moe_finalize_kernel<VPL, KC, PE, kRowRagged>);
    }
}

// The fully unrolled top-k keeps every row of a token in flight; it fits in registers up to
// two slots per wave (one for the per-expert variant, which also holds a gamma row per
// gathered row).  Wider slices keep the batched loop.
constexpr bool uses_compiled_topk(int vpl, bool per_expert) { return vpl <= (per_expert ? 1 : 2); }

template <int VPL, bool PE>
const void* finalize_fn(int tail, int k) {
    if constexpr (uses_compiled_topk(VPL, PE)) {
        if (k == kCompiledTopK) return finalize_fn<VPL, kCompiledTopK, PE>(tail);
    }
    return finalize_fn<VPL, 0, PE>(tail);
}

const void* finalize_kernel_for(const RowShape& s, int k, bool per_expert) {
    if (per_expert) {
        switch (s.vpl) {
            case 1: return finalize_fn<1, true>(s.tail, k);
            case 2: return finalize_fn<2, true>(s.tail, k);
            case 3: return finalize_fn<3, true>(s.tail, k);
            case 4: return finalize_fn<4, true>(s.tail, k);
            case 5: return finalize_fn<5, true>(s.tail, k);
            case 6: return finalize_fn<6, true>(s.tail, k);
            case 7: return finalize_fn<7, true>(s.tail, k);
            case 8: return finalize_fn<8, true>(s.tail, k);
            default: return nullptr;
        }
    }
    switch (s.vpl) {
        case 1: return finalize_fn<1, false>(s.tail, k);
        case 2: return finalize_fn<2, false>(s.tail, k);
        case 3: return finalize_fn<3, false>(s.tail, k);
        case 4: return finalize_fn<4, false>(s.tail, k);
        default: return nullptr;
    }
}

template <int VPL>
const void* gated_fn(int tail) {
    switch (tail) {
        case kRowFull: return reinterpret_cast<const void*>(&gated_residual_rmsnorm_kernel<VPL, kRowFull>);
        case kRowWhole: return reinterpret_cast<const void*>(&gated_residual_rmsnorm_kernel<VPL, kRowWhole>);
        default: return reinterpret_cast<const void*>(&gated_residual_rmsnorm_kernel<VPL, kRowRagged>);
    }
}

const void* gated_kernel_for(const RowShape& s) {
    switch (s.vpl) {
        case 1: return gated_fn<1>(s.tail);
        case 2: return gated_fn<2>(s.tail);
        case 3: return gated_fn<3>(s.tail);
        case 4: return gated_fn<4>(s.tail);
        default: return nullptr;
    }
}

}  // namespace

extern "C" {

int mf_moe_finalize_supported(int32_t H, int32_t k, int per_expert) {
    (void)per_expert;
    return row_width_supported(H) && k >= 1 && k <= kMaxK;
}

int mf_gated_residual_rmsnorm_supported(int32_t H) { return row_width_supported(H); }

int mf_rmsnorm_sigmoid_gate_supported(int32_t head_dim) { return head_dim == kHeadDim; }

int mf_launch_shape(int kind, int64_t T, int32_t H, int32_t k, int32_t* waves_per_token,
                    int32_t* vectors_per_lane, int32_t* block_threads, int64_t* grid_blocks) {
    if (kind < 0 || kind > 2 || T < 0) return MF_ERR_SHAPE;
    if (kind <= 1 ? !mf_moe_finalize_supported(H, k, kind) : !row_width_supported(H))
        return MF_ERR_UNSUPPORTED;
    const RowShape s = kind <= 1 ? finalize_shape(T, H, k, kind == 1) : row_shape(T, H, kMaxWaves, kMaxVpl);
    if (T > 0 && !grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
    // the same kernel lookup as the launch itself
    const void* fn = kind <= 1 ? finalize_kernel_for(s, k, kind == 1) : gated_kernel_for(s);
    if (!fn || (kind <= 1 && s.block > finalize_block_max(kind == 1))) return MF_ERR_UNSUPPORTED;
    if (waves_per_token) *waves_per_token = s.wpt;
    if (vectors_per_lane) *vectors_per_lane = s.vpl;
    if (block_threads) *block_threads = s.block;
    if (grid_blocks) *grid_blocks = s.grid;
    return MF_OK;
}

int mf_moe_finalize(const uint16_t* expert_rows, int64_t num_rows, const int32_t* idx,
                    const float* weights, const int32_t* expert_ids,
                    const uint16_t* expert_gamma, int32_t num_experts, const float* residual,
                    float* residual_out, const uint16_t* gamma, float eps, uint16_t* out,
                    int64_t T, int32_t H, int32_t k, void* stream) {
    if (T < 0 || num_rows < 0) return MF_ERR_SHAPE;
    const bool per_expert = expert_ids != nullptr || expert_gamma != nullptr;
    if (!mf_moe_finalize_supported(H, k, per_expert)) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    const RowShape s = finalize_shape(T, H, k, per_expert);
    if (!grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
    const void* fn = finalize_kernel_for(s, k, per_expert);
    if (!fn || s.block > finalize_block_max(per_expert)) return MF_ERR_UNSUPPORTED;
    if (!expert_rows || !idx || !weights || !residual || !residual_out || !gamma || !out)
        return MF_ERR_NULL;
    if (per_expert && (!expert_ids || !expert_gamma)) return MF_ERR_NULL;
    if (num_rows < 1 || (per_expert && num_experts < 1)) return MF_ERR_SHAPE;
    if (!eps_ok(eps)) return MF_ERR_VALUE;
    if (!aligned(expert_rows, 16) || !aligned(residual, 16) || !aligned(residual_out, 16) ||
        !aligned(gamma, 16) || !aligned(out, 16) || !aligned(idx, 4) || !aligned(weights, 4) ||
        (per_expert && (!aligned(expert_gamma, 16) || !aligned(expert_ids, 4))))
        return MF_ERR_ALIGN;
    const size_t th = size_t(T) * H;
    const size_t tk = size_t(T) * k;
    const size_t nr = size_t(num_rows) * H * 2;
    // residual_out may be residual itself; any other overlap of an output with anything is
    // rejected.
    if (residual_out != residual && overlap(residual_out, th * 4, residual, th * 4))
        return MF_ERR_ALIAS;
    const void* ins[] = {expert_rows, idx, weights, gamma, expert_ids, expert_gamma};
    const size_t in_bytes[] = {nr, tk * 4, tk * 4, size_t(H) * 2, per_expert ? tk * 4 : 0,
                               per_expert ? size_t(num_experts) * H * 2 : 0};
    for (int i = 0; i < 6; ++i) {
        if (overlap(residual_out, th * 4, ins[i], in_bytes[i]) ||
            overlap(out, th * 2, ins[i], in_bytes[i]))
            return MF_ERR_ALIAS;
    }
    if (overlap(out, th * 2, residual, th * 4) || overlap(out, th * 2, residual_out, th * 4))
        return MF_ERR_ALIAS;

    FinalizeArgs a;
    a.rows = expert_rows;
    a.idx = idx;
    a.w = weights;
    a.eids = expert_ids;
    a.egamma = expert_gamma;
    a.residual = residual;
    a.residual_out = residual_out;
    a.gamma = gamma;
    a.out = out;
    a.T = T;
    a.num_rows = num_rows;
    a.H = H;
    a.k = k;
    a.num_experts = per_expert ? num_experts : 0;
    a.eps = eps;
    void* args[] = {&a};
    return hip_status(hipLaunchKernel(fn, dim3((unsigned)s.grid), dim3(s.block), args, s.lds,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int mf_gated_residual_rmsnorm(const uint16_t* x, const uint16_t* gate, const float* residual,
                              float* residual_out, const uint16_t* gamma, float eps,
                              uint16_t* out, int64_t T, int32_t H, void* stream) {
    if (T < 0) return MF_ERR_SHAPE;
    if (!row_width_supported(H)) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    const RowShape s = row_shape(T, H, kMaxWaves, kMaxVpl);
    if (!grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
    const void* fn = gated_kernel_for(s);
    if (!fn) return MF_ERR_UNSUPPORTED;
    if (!x || !gate || !residual || !residual_out || !gamma || !out) return MF_ERR_NULL;
    if (!eps_ok(eps)) return MF_ERR_VALUE;
    if (!aligned(x, 16) || !aligned(gate, 16) || !aligned(residual, 16) ||
        !aligned(residual_out, 16) || !aligned(gamma, 16) || !aligned(out, 16))
        return MF_ERR_ALIGN;
    const size_t th = size_t(T) * H;
    if (residual_out != residual && overlap(residual_out, th * 4, residual, th * 4))
        return MF_ERR_ALIAS;
    const void* ins[] = {x, gate, gamma};
    const size_t in_bytes[] = {th * 2, th * 2, size_t(H) * 2};
    for (int i = 0; i < 3; ++i) {
        if (overlap(residual_out, th * 4, ins[i], in_bytes[i]) ||
            overlap(out, th * 2, ins[i], in_bytes[i]))
            return MF_ERR_ALIAS;
    }
    if (overlap(out, th * 2, residual, th * 4) || overlap(out, th * 2, residual_out, th * 4))
        return MF_ERR_ALIAS;

    GatedArgs a;
    a.x = x;
    a.gate = gate;
    a.residual = residual;
    a.residual_out = residual_out;
    a.gamma = gamma;
    a.out = out;
    a.T = T;
    a.H = H;
    a.eps = eps;
    void* args[] = {&a};
    return hip_status(hipLaunchKernel(fn, dim3((unsigned)s.grid), dim3(s.block), args, s.lds,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int mf_rmsnorm_sigmoid_gate(const uint16_t* x, const uint16_t* gate, const uint16_t* gamma,
                            float eps, uint16_t* out, int64_t T, int32_t num_heads,
                            int32_t head_dim, void* stream) {
    if (T < 0 || num_heads < 1) return MF_ERR_SHAPE;
    if (!mf_rmsnorm_sigmoid_gate_supported(head_dim)) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    constexpr int G = kPerHeadGroupsPerWave;
    const int64_t nh = T * num_heads;
    const int64_t groups = (nh + kHeadsPerWaveLoad - 1) / kHeadsPerWaveLoad;
    const int64_t waves = (groups + G - 1) / G;
    const int64_t blocks = (waves + 3) / 4;
    if (!grid_fits(blocks, 256)) return MF_ERR_SHAPE;
    if (!x || !gate || !gamma || !out) return MF_ERR_NULL;
    if (!eps_ok(eps)) return MF_ERR_VALUE;
    if (!aligned(x, 16) || !aligned(gate, 16) || !aligned(gamma, 16) || !aligned(out, 16))
        return MF_ERR_ALIGN;
    const size_t bytes = size_t(nh) * head_dim * 2;
    if (overlap(out, bytes, x, bytes) || overlap(out, bytes, gate, bytes) ||
        overlap(out, bytes, gamma, size_t(head_dim) * 2))
        return MF_ERR_ALIAS;

    PerHeadArgs a;
    a.x = x;
    a.gate = gate;
    a.gamma = gamma;
    a.out = out;
    a.num_heads_total = nh;
    a.eps = eps;
    void* args[] = {&a};
    return hip_status(hipLaunchKernel(reinterpret_cast<const void*>(&rmsnorm_sigmoid_gate_kernel<G>),
                                      dim3((unsigned)blocks), dim3(256), args, 0,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int mf_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16 != 0) return MF_ERR_SHAPE;
    if (bytes == 0) return MF_OK;
    if (!src || !dst) return MF_ERR_NULL;
    if (!aligned(src, 16) || !aligned(dst, 16)) return MF_ERR_ALIGN;
    if (overlap(src, size_t(bytes), dst, size_t(bytes))) return MF_ERR_ALIAS;
    constexpr int U = 4;
    const int64_t n = bytes / 16;
    const int64_t blocks = (n + 256 * U - 1) / (256 * U);
    if (!grid_fits(blocks, 256)) return MF_ERR_SHAPE;
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    void* args[] = {&s, &d, const_cast<int64_t*>(&n)};
    return hip_status(hipLaunchKernel(reinterpret_cast<const void*>(&stream_copy_kernel<U>),
                                      dim3((unsigned)blocks), dim3(256), args, 0,
                                      reinterpret_cast<hipStream_t>(stream)));
}

const char* mf_status_string(int status) {
    switch (status) {
        case MF_OK: return "MF_OK: success";
        case MF_ERR_NULL: return "MF_ERR_NULL: a required pointer is NULL";
        case MF_ERR_SHAPE: return "MF_ERR_SHAPE: a size is negative or inconsistent";
        case MF_ERR_UNSUPPORTED: return "MF_ERR_UNSUPPORTED: width, expert count or top-k not supported";
        case MF_ERR_ALIGN: return "MF_ERR_ALIGN: a pointer is misaligned";
        case MF_ERR_ALIAS: return "MF_ERR_ALIAS: an output overlaps an input";
        case MF_ERR_VALUE: return "MF_ERR_VALUE: eps must be finite and >= 0";
        case MF_ERR_HIP: return "MF_ERR_HIP: the HIP runtime rejected the launch";
        default: return "unknown mf_status";
    }
}

}  // extern "C"
