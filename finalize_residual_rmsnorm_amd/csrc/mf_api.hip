// Host side of the MoE finalize entry points declared in include/mf.h (and the shared
// launch-shape query and status strings): argument checks before any HIP call, launch-shape
// selection and kernel dispatch.  Stateless and allocation-free.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "api_util.h"
#include "finalize_kernel.h"
#include "mf.h"
#include "row_shape.h"

namespace {

using namespace mf;

constexpr int32_t kMaxK = 64;
constexpr int kMaxWavesPerExpert = 8;   // the per-expert variant reduces a batch of row sums
                                        // per barrier; 8 waves keep that LDS under 64 KiB
constexpr int kMaxVplPerExpert = 8;     // per-expert finalize: 8 x 8 x 512 = 32768

// The top-k the finalize kernels are specialised for (all loads of a token issued at once).
constexpr int kCompiledTopK = 8;

constexpr bool uses_compiled_topk(int vpl, bool per_expert);

// The combine runs at most 8 waves per token (two slots per wave at H = 7168): measured 2%
// faster than 16 waves.  Rows too wide for 8 waves of kMaxVpl slots take 16.
constexpr int kCombineWaves = 8;
RowShape combine_shape(int64_t T, int32_t H) {
    const RowShape s = row_shape(T, H, kCombineWaves, kMaxVpl);
    return s.vpl <= kMaxVpl ? s : row_shape(T, H, kMaxWaves, kMaxVpl);
}

// Rows too wide for one or two slots per wave (H > 8192) take the slot-serial kernel
// (moe_finalize_wide_kernel) at the compiled top-k when its shape fills whole waves of slots:
// 8 waves per token of 3 or 5 to 8 slots each (H = 12288, 20480, 24576, 28672, 32768), of which
// wide_staged_slots wait in LDS.  H = 16384, which 16 waves of two slots would fill, keeps
// moe_finalize_kernel at 8 waves of 4 (74.7% of 8 TB/s against 72.5% for this kernel at that
// shape, T = 8192), as do the other wide shapes (a row that is not whole waves of whole slots,
// another top-k).
constexpr int kWideMaxVpl = 8;
constexpr int wide_staged_slots(int vpl) { return vpl >= 6 ? 3 : 0; }

RowShape wide_shape(int64_t T, int32_t H) {
    const int ns = (H + kSlot - 1) / kSlot;
    RowShape s;
    s.vpl = (ns + kWideWaves - 1) / kWideWaves;
    s.wpt = kWideWaves;
    s.tail = ns == s.wpt * s.vpl && H == ns * kSlot ? kRowFull : kRowWhole;
    s.block = kWave * s.wpt;
    s.grid = T;
    s.nr = 1;
    s.nl = wide_staged_slots(s.vpl);
    s.lds = wide_lds_bytes(s.wpt, s.nl);
    return s;
}

bool uses_wide_kernel(int64_t T, int32_t H, int32_t k, bool per_expert) {
    if (per_expert || k != kCompiledTopK || row_shape(1, H, kMaxWaves, kMaxVpl).vpl <= 2) return false;
    const RowShape s = wide_shape(T, H);
    return s.tail == kRowFull && s.vpl >= 3 && s.vpl <= kWideMaxVpl;
}

// The finalize without per-expert norm (and its partial and MXFP4 forms), rather than the fewest
// spare slots:
//  - a row of up to 16 slots takes one slot per wave over a power-of-two count of waves, the
//    spare waves idle.  Measured on MI355X (T = 16384, k = 8, one GPU, interleaved rounds):
//    H = 1536 79.8% of 8 TB/s against 75.9% for 1 wave of 3 slots; 2560 81.3% against 78.1%
//    (2 x 3); 3072 80.8% against 76.2% (2 x 3); 5120 81.3% against 79.0% (4 x 3); 6144 81.1%
//    against 77.7% (4 x 3).  Exactly one wave per slot (3, 5, 6, 10, 12, 14 or 15 waves) came
//    between the two, and below the power of two at H = 7168 (77.1% against 78.7%).
//  - 14 to 16 slots (H = 6657 to 8192) take 8 waves of 2 instead, except in the expert-parallel
//    partial: the prefill finalize (H = 7168) 480.9-482.3 us against 484.5-486.5 us for 16 waves
//    of 1 (79.3% against 78.8%, on two GPUs), H = 8192 0.9% faster, the MXFP4 form 0.2% faster; the
//    partial 2.5% slower, and 13 slots or fewer equal or slower.
//  - 17 to 32 slots take 8 waves of 3 or 4: at H = 13312, 14336 and 16384 (T = 8192) 75.5%,
//    75.5% and 74.7% against 73.6%, 74.3% and 73.2% for 16 waves of 2 (one GPU, every variant
//    writing the same buffers); 9216 and 10240 at 8 waves of 3 77.8% against 70-72% for 16 x 2.
RowShape plain_finalize_shape(int64_t T, int32_t H, bool partial) {
    const int ns = (H + kSlot - 1) / kSlot;
    if (ns > 2 * kMaxWaves) return row_shape(T, H, kMaxWaves, kMaxVpl);
    const bool two = ns > kMaxWaves || (ns >= 14 && !partial);
    RowShape s;
    s.vpl = ns > kMaxWaves ? (ns + 7) / 8 : (two ? 2 : 1);
    s.wpt = two ? 8 : pow2_at_least(ns);
    s.tail = H != ns * kSlot ? kRowRagged : (ns == s.wpt * s.vpl ? kRowFull : kRowWhole);
    s.block = kWave * s.wpt;
    s.grid = T;
    s.nr = 1;
    s.lds = token_sum_lds_bytes(s.wpt, 1);
    return s;
}

// Launch shape of the finalize kernels; `wide` selects the slot-serial kernel's (the bf16-output
// finalize of wide rows only), `partial` the expert-parallel partial's.
RowShape finalize_shape(int64_t T, int32_t H, int32_t k, bool per_expert, bool wide = false,
                        bool partial = false) {
    if (wide) return wide_shape(T, H);
    RowShape s = per_expert ? row_shape(T, H, kMaxWavesPerExpert, kMaxVplPerExpert)
                            : plain_finalize_shape(T, H, partial);
    const int kc = k == kCompiledTopK && uses_compiled_topk(s.vpl, per_expert) ? kCompiledTopK : 0;
    s.nr = per_expert ? batch_rows(s.vpl, kc, true) : 1;
    s.lds = token_sum_lds_bytes(s.wpt, s.nr);
    return s;
}

template <int VPL, int KC, bool PE, bool PARTIAL, bool OUT_MX = false>
const void* finalize_fn(int tail) {
    switch (tail) {
        case kRowFull: return reinterpret_cast<const void*>(&moe_finalize_kernel<VPL, KC, PE, kRowFull, PARTIAL, OUT_MX>);
        case kRowWhole: return reinterpret_cast<const void*>(&moe_finalize_kernel<VPL, KC, PE, kRowWhole, PARTIAL, OUT_MX>);
        default: return reinterpret_cast<const void*>(&moe_finalize_kernel<VPL, KC, PE, kRowRagged, PARTIAL, OUT_MX>);
    }
}

// The fully unrolled top-k keeps every row of a token in flight; it fits in registers up to
// two slots per wave (one for the per-expert variant, which also holds a gamma row per
// gathered row).  Wider slices keep the batched loop.
constexpr bool uses_compiled_topk(int vpl, bool per_expert) { return vpl <= (per_expert ? 1 : 2); }

template <int VPL, bool PE, bool PARTIAL>
const void* finalize_fn(int tail, int k) {
    if constexpr (uses_compiled_topk(VPL, PE)) {
        if (k == kCompiledTopK) return finalize_fn<VPL, kCompiledTopK, PE, PARTIAL>(tail);
    }
    return finalize_fn<VPL, 0, PE, PARTIAL>(tail);
}

template <bool PARTIAL>
const void* finalize_kernel_for_mode(const RowShape& s, int k, bool per_expert) {
    if (per_expert) {
        switch (s.vpl) {
            case 1: return finalize_fn<1, true, PARTIAL>(s.tail, k);
            case 2: return finalize_fn<2, true, PARTIAL>(s.tail, k);
            case 3: return finalize_fn<3, true, PARTIAL>(s.tail, k);
            case 4: return finalize_fn<4, true, PARTIAL>(s.tail, k);
            case 5: return finalize_fn<5, true, PARTIAL>(s.tail, k);
            case 6: return finalize_fn<6, true, PARTIAL>(s.tail, k);
            case 7: return finalize_fn<7, true, PARTIAL>(s.tail, k);
            case 8: return finalize_fn<8, true, PARTIAL>(s.tail, k);
            default: return nullptr;
        }
    }
    switch (s.vpl) {
        case 1: return finalize_fn<1, false, PARTIAL>(s.tail, k);
        case 2: return finalize_fn<2, false, PARTIAL>(s.tail, k);
        case 3: return finalize_fn<3, false, PARTIAL>(s.tail, k);
        case 4: return finalize_fn<4, false, PARTIAL>(s.tail, k);
        default: return nullptr;
    }
}

template <int VPL>
const void* wide_fn() {
    return reinterpret_cast<const void*>(
        &moe_finalize_wide_kernel<VPL, wide_staged_slots(VPL), kCompiledTopK>);
}

const void* wide_kernel_for(const RowShape& s) {
    switch (s.vpl) {
        case 3: return wide_fn<3>();
        case 5: return wide_fn<5>();
        case 6: return wide_fn<6>();
        case 7: return wide_fn<7>();
        case 8: return wide_fn<8>();
        default: return nullptr;
    }
}

// The finalize kernel for a shape (wide: the slot-serial kernel of wide rows), or its
// expert-parallel partial.
const void* finalize_kernel_for(const RowShape& s, int k, bool per_expert, bool partial = false,
                                bool wide = false) {
    if (wide) return wide_kernel_for(s);
    return partial ? finalize_kernel_for_mode<true>(s, k, per_expert)
                   : finalize_kernel_for_mode<false>(s, k, per_expert);
}

// The MXFP4 epilogue is built for the plain finalize (no per-expert norm).
template <int VPL>
const void* finalize_mx_fn(int tail, int k) {
    if constexpr (uses_compiled_topk(VPL, false)) {
        if (k == kCompiledTopK) return finalize_fn<VPL, kCompiledTopK, false, false, true>(tail);
    }
    return finalize_fn<VPL, 0, false, false, true>(tail);
}

const void* finalize_mx_kernel_for(const RowShape& s, int k) {
    switch (s.vpl) {
        case 1: return finalize_mx_fn<1>(s.tail, k);
        case 2: return finalize_mx_fn<2>(s.tail, k);
        case 3: return finalize_mx_fn<3>(s.tail, k);
        case 4: return finalize_mx_fn<4>(s.tail, k);
        default: return nullptr;
    }
}

template <int VPL>
const void* combine_fn(int tail) {
    switch (tail) {
        case kRowFull: return reinterpret_cast<const void*>(&moe_finalize_combine_kernel<VPL, kRowFull>);
        case kRowWhole: return reinterpret_cast<const void*>(&moe_finalize_combine_kernel<VPL, kRowWhole>);
        default: return reinterpret_cast<const void*>(&moe_finalize_combine_kernel<VPL, kRowRagged>);
    }
}

const void* combine_kernel_for(const RowShape& s) {
    switch (s.vpl) {
        case 1: return combine_fn<1>(s.tail);
        case 2: return combine_fn<2>(s.tail);
        case 3: return combine_fn<3>(s.tail);
        case 4: return combine_fn<4>(s.tail);
        default: return nullptr;
    }
}

constexpr int32_t kMaxRanks = 1024;

}  // namespace

extern "C" {

int mf_moe_finalize_supported(int32_t H, int32_t k, int per_expert) {
    (void)per_expert;
    return row_width_supported(H) && k >= 1 && k <= kMaxK;
}

int mf_launch_shape(int kind, int64_t T, int32_t H, int32_t k, int32_t* waves_per_token,
                    int32_t* vectors_per_lane, int32_t* block_threads, int64_t* grid_blocks) {
    if (kind < 0 || kind > 4 || T < 0) return MF_ERR_SHAPE;
    const bool finalize = kind <= 1 || kind == 4;
    if (finalize ? !mf_moe_finalize_supported(H, k, kind == 1) : !row_width_supported(H))
        return MF_ERR_UNSUPPORTED;
    const bool wide = kind <= 1 && uses_wide_kernel(T, H, k, kind == 1);
    const RowShape s = kind <= 1   ? finalize_shape(T, H, k, kind == 1, wide)
                       : kind == 2 ? row_shape(T, H, kMaxWaves, kMaxVpl)
                       : kind == 3 ? combine_shape(T, H)
                                   : finalize_shape(T, H, k, false, false, true);
    if (T > 0 && !grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
    // the same kernel lookup as the launch itself
    const void* fn = kind <= 1   ? finalize_kernel_for(s, k, kind == 1, false, wide)
                     : kind == 2 ? gated_kernel_for(s, false)
                     : kind == 3 ? combine_kernel_for(s)
                                 : finalize_kernel_for(s, k, false, true);
    if (!fn || (finalize && s.block > finalize_block_max(kind == 1))) return MF_ERR_UNSUPPORTED;
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
    const bool wide = uses_wide_kernel(T, H, k, per_expert);
    const RowShape s = finalize_shape(T, H, k, per_expert, wide);
    if (!grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
    const void* fn = finalize_kernel_for(s, k, per_expert, false, wide);
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
    a.q = nullptr;
    a.scales = nullptr;
    void* args[] = {&a};
    return hip_status(hipLaunchKernel(fn, dim3((unsigned)s.grid), dim3(s.block), args, s.lds,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int mf_moe_finalize_mxfp4(const uint16_t* expert_rows, int64_t num_rows, const int32_t* idx,
                          const float* weights, const float* residual, float* residual_out,
                          const uint16_t* gamma, float eps, uint8_t* q, uint8_t* scales,
                          int64_t T, int32_t H, int32_t k, void* stream) {
    if (T < 0 || num_rows < 0) return MF_ERR_SHAPE;
    if (!mf_moe_finalize_supported(H, k, 0) || H % 32 != 0) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    const RowShape s = finalize_shape(T, H, k, false);
    if (!grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
    const void* fn = finalize_mx_kernel_for(s, k);
    if (!fn || s.block > finalize_block_max(false)) return MF_ERR_UNSUPPORTED;
    if (!expert_rows || !idx || !weights || !residual || !residual_out || !gamma || !q || !scales)
        return MF_ERR_NULL;
    if (num_rows < 1) return MF_ERR_SHAPE;
    if (!eps_ok(eps)) return MF_ERR_VALUE;
    if (!aligned(expert_rows, 16) || !aligned(residual, 16) || !aligned(residual_out, 16) ||
        !aligned(gamma, 16) || !aligned(q, 4) || !aligned(idx, 4) || !aligned(weights, 4))
        return MF_ERR_ALIGN;
    const size_t th = size_t(T) * H;
    const size_t tk = size_t(T) * k;
    if (residual_out != residual && overlap(residual_out, th * 4, residual, th * 4))
        return MF_ERR_ALIAS;
    const void* ins[] = {expert_rows, idx, weights, gamma, residual};
    const size_t in_bytes[] = {size_t(num_rows) * H * 2, tk * 4, tk * 4, size_t(H) * 2, th * 4};
    for (int i = 0; i < 5; ++i) {
        if ((i < 4 && overlap(residual_out, th * 4, ins[i], in_bytes[i])) ||
            overlap(q, th / 2, ins[i], in_bytes[i]) || overlap(scales, th / 32, ins[i], in_bytes[i]))
            return MF_ERR_ALIAS;
    }
    if (overlap(q, th / 2, residual_out, th * 4) || overlap(scales, th / 32, residual_out, th * 4) ||
        overlap(q, th / 2, scales, th / 32))
        return MF_ERR_ALIAS;

    FinalizeArgs a;
    a.rows = expert_rows;
    a.idx = idx;
    a.w = weights;
    a.eids = nullptr;
    a.egamma = nullptr;
    a.residual = residual;
    a.residual_out = residual_out;
    a.gamma = gamma;
    a.out = nullptr;
    a.q = q;
    a.scales = scales;
    a.T = T;
    a.num_rows = num_rows;
    a.H = H;
    a.k = k;
    a.num_experts = 0;
    a.eps = eps;
    void* args[] = {&a};
    return hip_status(hipLaunchKernel(fn, dim3((unsigned)s.grid), dim3(s.block), args, s.lds,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int mf_moe_finalize_ep_partial(const uint16_t* expert_rows, int64_t num_rows,
                               const int32_t* idx, const float* weights,
                               const int32_t* expert_ids, const uint16_t* expert_gamma,
                               int32_t num_experts, float eps, float* partial, int64_t T,
                               int32_t H, int32_t k, void* stream) {
    if (T < 0 || num_rows < 0) return MF_ERR_SHAPE;
    const bool per_expert = expert_ids != nullptr || expert_gamma != nullptr;
    if (!mf_moe_finalize_supported(H, k, per_expert)) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    const RowShape s = finalize_shape(T, H, k, per_expert, false, true);
    if (!grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
    const void* fn = finalize_kernel_for(s, k, per_expert, true);
    if (!fn || s.block > finalize_block_max(per_expert)) return MF_ERR_UNSUPPORTED;
    if (!expert_rows || !idx || !weights || !partial) return MF_ERR_NULL;
    if (per_expert && (!expert_ids || !expert_gamma)) return MF_ERR_NULL;
    if (num_rows < 1 || (per_expert && num_experts < 1)) return MF_ERR_SHAPE;
    if (!eps_ok(eps)) return MF_ERR_VALUE;
    if (!aligned(expert_rows, 16) || !aligned(partial, 16) || !aligned(idx, 4) ||
        !aligned(weights, 4) ||
        (per_expert && (!aligned(expert_gamma, 16) || !aligned(expert_ids, 4))))
        return MF_ERR_ALIGN;
    const size_t th = size_t(T) * H;
    const size_t tk = size_t(T) * k;
    const void* ins[] = {expert_rows, idx, weights, expert_ids, expert_gamma};
    const size_t in_bytes[] = {size_t(num_rows) * H * 2, tk * 4, tk * 4, per_expert ? tk * 4 : 0,
                               per_expert ? size_t(num_experts) * H * 2 : 0};
    for (int i = 0; i < 5; ++i)
        if (overlap(partial, th * 4, ins[i], in_bytes[i])) return MF_ERR_ALIAS;

    FinalizeArgs a;
    a.rows = expert_rows;
    a.idx = idx;
    a.w = weights;
    a.eids = expert_ids;
    a.egamma = expert_gamma;
    a.residual = nullptr;
    a.residual_out = partial;
    a.gamma = nullptr;
    a.out = nullptr;
    a.T = T;
    a.num_rows = num_rows;
    a.H = H;
    a.k = k;
    a.num_experts = per_expert ? num_experts : 0;
    a.eps = eps;
    a.q = nullptr;
    a.scales = nullptr;
    void* args[] = {&a};
    return hip_status(hipLaunchKernel(fn, dim3((unsigned)s.grid), dim3(s.block), args, s.lds,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int mf_moe_finalize_ep_combine(const float* partials, int32_t num_ranks, const float* residual,
                               float* residual_out, const uint16_t* gamma, float eps,
                               uint16_t* out, int64_t T, int32_t H, void* stream) {
    if (T < 0 || num_ranks < 1 || num_ranks > kMaxRanks) return MF_ERR_SHAPE;
    if (!row_width_supported(H)) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    const RowShape s = combine_shape(T, H);
    if (!grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
    const void* fn = combine_kernel_for(s);
    if (!fn) return MF_ERR_UNSUPPORTED;
    if (!partials || !residual || !residual_out || !gamma || !out) return MF_ERR_NULL;
    if (!eps_ok(eps)) return MF_ERR_VALUE;
    if (!aligned(partials, 16) || !aligned(residual, 16) || !aligned(residual_out, 16) ||
        !aligned(gamma, 16) || !aligned(out, 16))
        return MF_ERR_ALIGN;
    const size_t th = size_t(T) * H;
    if (residual_out != residual && overlap(residual_out, th * 4, residual, th * 4))
        return MF_ERR_ALIAS;
    const void* ins[] = {partials, gamma};
    const size_t in_bytes[] = {size_t(num_ranks) * th * 4, size_t(H) * 2};
    for (int i = 0; i < 2; ++i) {
        if (overlap(residual_out, th * 4, ins[i], in_bytes[i]) ||
            overlap(out, th * 2, ins[i], in_bytes[i]))
            return MF_ERR_ALIAS;
    }
    if (overlap(out, th * 2, residual, th * 4) || overlap(out, th * 2, residual_out, th * 4))
        return MF_ERR_ALIAS;

    CombineArgs a;
    a.partials = partials;
    a.residual = residual;
    a.residual_out = residual_out;
    a.gamma = gamma;
    a.out = out;
    a.T = T;
    a.H = H;
    a.G = num_ranks;
    a.eps = eps;
    void* args[] = {&a};
    return hip_status(hipLaunchKernel(fn, dim3((unsigned)s.grid), dim3(s.block), args, s.lds,
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
        case MF_ERR_HIP: return "MF_ERR_HIP: the HIP runtime rejected the launch";
        case MF_ERR_VALUE: return "MF_ERR_VALUE: eps must be finite and >= 0";
        case MF_ERR_SCRATCH:
            return "MF_ERR_SCRATCH: the problem needs more scratch than the library's static buffer holds";
        default: return "unknown mf_status";
    }
}

}  // extern "C"
