// Host side of the C ABI declared in include/mf.h: argument checks (before any HIP call),
// launch-shape selection and kernel dispatch.  Stateless and allocation-free.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "finalize_kernel.h"
#include "mf.h"
#include "norm_kernels.h"

namespace {

using namespace mf;

constexpr int32_t kMaxH = 32768;       // 64 slots of 512 values
constexpr int32_t kMaxK = 64;
constexpr int kMaxVpl = 16;
constexpr int kMaxVplPerExpert = 8;  // the per-expert variant also holds a batch of gamma rows
constexpr int kMaxWptPerExpert = 8;  // keeps its LDS (a batch of sums per wave) under 64 KiB
constexpr int kMaxWpt = 16;
// Waves that keep all 256 CUs of an MI355X busy (8 per CU); smaller token counts spread
// each row over more waves instead.
constexpr int64_t kFillWaves = 2048;
constexpr int kPerHeadGroupsPerWave = 2;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Do [a, a+na) and [b, b+nb) share a byte?
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool eps_ok(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

struct RowShape {
    int wpt;        // waves per token (power of two)
    int spw;        // slots per wave
    int vpl;        // slots held per lane (kernel instantiation)
    int block;      // threads per workgroup
    int64_t grid;   // workgroups
    size_t lds;     // dynamic LDS bytes
};

bool row_shape_supported(int32_t H) { return H >= 8 && H <= kMaxH && H % 8 == 0; }

// Launch shape of the token-row kernels.  The per-expert variant reduces one row sum per
// gathered row of a batch at each barrier, so its LDS holds a batch of sums per wave.
RowShape row_shape(int64_t T, int32_t H, bool per_expert) {
    const int ns = (H + kSlot - 1) / kSlot;
    int nsp = 1;
    while (nsp < ns) nsp *= 2;
    int wpt = 1;
    const int max_vpl = per_expert ? kMaxVplPerExpert : kMaxVpl;
    while (nsp / wpt > max_vpl) wpt *= 2;                   // the row must fit in registers
    const int wpt_cap = per_expert ? kMaxWptPerExpert : kMaxWpt;
    while (wpt < nsp && wpt < wpt_cap && T * wpt < kFillWaves) wpt *= 2;  // fill the chip
    RowShape s;
    s.wpt = wpt;
    s.spw = nsp / wpt;
    s.vpl = wpt == 1 ? ns : s.spw;
    const int tpb = wpt >= 4 ? 1 : 4 / wpt;
    s.block = kWave * wpt * tpb;
    s.grid = (T + tpb - 1) / tpb;
    const int nr = per_expert ? gather_batch_for(s.vpl, true) : 1;
    s.lds = wpt > 1 ? token_sum_lds_bytes(s.block / kWave, nr) : 0;
    return s;
}

template <int VPL, bool PE>
hipError_t launch_finalize_vpl(const FinalizeArgs& a, const RowShape& s, hipStream_t st) {
    void* args[] = {const_cast<FinalizeArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&moe_finalize_kernel<VPL, PE>),
                           dim3((unsigned)s.grid), dim3(s.block), args, s.lds, st);
}

hipError_t launch_finalize(bool per_expert, const FinalizeArgs& a, const RowShape& s,
                           hipStream_t st) {
#define MF_CASE(V, PE) \
    case V: return launch_finalize_vpl<V, PE>(a, s, st);
    if (per_expert) {
        switch (s.vpl) {
            MF_CASE(1, true) MF_CASE(2, true) MF_CASE(3, true) MF_CASE(4, true)
            MF_CASE(5, true) MF_CASE(6, true) MF_CASE(7, true) MF_CASE(8, true)
            default: return hipErrorInvalidValue;
        }
    }
    switch (s.vpl) {
        MF_CASE(1, false) MF_CASE(2, false) MF_CASE(3, false) MF_CASE(4, false)
        MF_CASE(5, false) MF_CASE(6, false) MF_CASE(7, false) MF_CASE(8, false)
        MF_CASE(9, false) MF_CASE(10, false) MF_CASE(11, false) MF_CASE(12, false)
        MF_CASE(13, false) MF_CASE(14, false) MF_CASE(15, false) MF_CASE(16, false)
        default: return hipErrorInvalidValue;
    }
#undef MF_CASE
}

template <int VPL>
hipError_t launch_gated_vpl(const GatedArgs& a, const RowShape& s, hipStream_t st) {
    void* args[] = {const_cast<GatedArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gated_residual_rmsnorm_kernel<VPL>),
                           dim3((unsigned)s.grid), dim3(s.block), args, s.lds, st);
}

hipError_t launch_gated(const GatedArgs& a, const RowShape& s, hipStream_t st) {
    switch (s.vpl) {
#define MF_CASE(V) \
    case V: return launch_gated_vpl<V>(a, s, st);
        MF_CASE(1) MF_CASE(2) MF_CASE(3) MF_CASE(4) MF_CASE(5) MF_CASE(6) MF_CASE(7) MF_CASE(8)
        MF_CASE(9) MF_CASE(10) MF_CASE(11) MF_CASE(12) MF_CASE(13) MF_CASE(14) MF_CASE(15)
        MF_CASE(16)
#undef MF_CASE
        default: return hipErrorInvalidValue;
    }
}

// AMD grids count work-items in 32 bits per dimension.
bool grid_fits(int64_t blocks, int threads) {
    return blocks >= 1 && blocks * int64_t(threads) <= int64_t(UINT32_MAX);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MF_OK : MF_ERR_HIP; }

}  // namespace

extern "C" {

int mf_moe_finalize_supported(int32_t H, int32_t k, int per_expert) {
    (void)per_expert;
    return row_shape_supported(H) && k >= 1 && k <= kMaxK;
}

int mf_gated_residual_rmsnorm_supported(int32_t H) { return row_shape_supported(H); }

int mf_rmsnorm_sigmoid_gate_supported(int32_t head_dim) { return head_dim == kHeadDim; }

int mf_launch_shape(int kind, int64_t T, int32_t H, int32_t k, int32_t* waves_per_token,
                    int32_t* vectors_per_lane, int32_t* block_threads, int64_t* grid_blocks) {
    if (kind < 0 || kind > 2 || T < 0) return MF_ERR_SHAPE;
    if (kind <= 1 ? !mf_moe_finalize_supported(H, k, kind) : !row_shape_supported(H))
        return MF_ERR_UNSUPPORTED;
    const RowShape s = row_shape(T, H, kind == 1);
    if (T > 0 && !grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
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
    const RowShape s = row_shape(T, H, per_expert);
    if (!grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
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
    a.wpt = s.wpt;
    a.spw = s.spw;
    a.eps = eps;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    return hip_status(launch_finalize(per_expert, a, s, st));
}

int mf_gated_residual_rmsnorm(const uint16_t* x, const uint16_t* gate, const float* residual,
                              float* residual_out, const uint16_t* gamma, float eps,
                              uint16_t* out, int64_t T, int32_t H, void* stream) {
    if (T < 0) return MF_ERR_SHAPE;
    if (!row_shape_supported(H)) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    const RowShape s = row_shape(T, H, false);
    if (!grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
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
    a.wpt = s.wpt;
    a.spw = s.spw;
    a.eps = eps;
    return hip_status(launch_gated(a, s, reinterpret_cast<hipStream_t>(stream)));
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
        case MF_ERR_UNSUPPORTED: return "MF_ERR_UNSUPPORTED: width or top-k not supported";
        case MF_ERR_ALIGN: return "MF_ERR_ALIGN: a pointer is misaligned";
        case MF_ERR_ALIAS: return "MF_ERR_ALIAS: an output overlaps an input";
        case MF_ERR_VALUE: return "MF_ERR_VALUE: eps must be finite and >= 0";
        case MF_ERR_HIP: return "MF_ERR_HIP: the HIP runtime rejected the launch";
        default: return "unknown mf_status";
    }
}

}  // extern "C"
