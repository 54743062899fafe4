// Host side of the fused-norm entry points declared in include/mf.h (gated-residual RMSNorm,
// its dual-output form, per-head RMSNorm with a sigmoid gate) and the copy kernel: argument
// checks before any HIP call, launch-shape selection and kernel dispatch.  Stateless and
// allocation-free.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "api_util.h"
#include "mf.h"
#include "norm_kernels.h"
#include "row_shape.h"

namespace {

using namespace mf;

// One group of 8 heads per wave and one wave per workgroup: measured 7% faster on MI355X than
// two groups per wave in 4-wave workgroups (every other combination of 1-2 groups and 64-1024
// threads was within 1% of the latter).

template <int VPL, bool DUAL>
const void* gated_fn(int tail) {
    switch (tail) {
        case kRowFull: return reinterpret_cast<const void*>(&gated_residual_rmsnorm_kernel<VPL, kRowFull, DUAL>);
        case kRowWhole: return reinterpret_cast<const void*>(&gated_residual_rmsnorm_kernel<VPL, kRowWhole, DUAL>);
        default: return reinterpret_cast<const void*>(&gated_residual_rmsnorm_kernel<VPL, kRowRagged, DUAL>);
    }
}

template <bool DUAL>
const void* gated_kernel_for_vpl(int vpl, int tail) {
    switch (vpl) {
        case 1: return gated_fn<1, DUAL>(tail);
        case 2: return gated_fn<2, DUAL>(tail);
        case 3: return gated_fn<3, DUAL>(tail);
        case 4: return gated_fn<4, DUAL>(tail);
        default: return nullptr;
    }
}

// Checks and launch shared by the single- and dual-output gated norms (gamma_next and out_next
// NULL for the single output).
int launch_gated(const uint16_t* x, const uint16_t* gate, const float* residual,
                 float* residual_out, const uint16_t* gamma, const uint16_t* gamma_next,
                 float eps, uint16_t* out, uint16_t* out_next, int64_t T, int32_t H, bool dual,
                 void* stream) {
    if (T < 0) return MF_ERR_SHAPE;
    if (!row_width_supported(H)) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    const RowShape s = row_shape(T, H, kMaxWaves, kMaxVpl);
    if (!grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
    const void* fn = gated_kernel_for(s, dual);
    if (!fn) return MF_ERR_UNSUPPORTED;
    if (!x || !gate || !residual || !residual_out || !gamma || !out) return MF_ERR_NULL;
    if (dual && (!gamma_next || !out_next)) return MF_ERR_NULL;
    if (!eps_ok(eps)) return MF_ERR_VALUE;
    if (!aligned(x, 16) || !aligned(gate, 16) || !aligned(residual, 16) ||
        !aligned(residual_out, 16) || !aligned(gamma, 16) || !aligned(out, 16) ||
        (dual && (!aligned(gamma_next, 16) || !aligned(out_next, 16))))
        return MF_ERR_ALIGN;
    const size_t th = size_t(T) * H;
    if (residual_out != residual && overlap(residual_out, th * 4, residual, th * 4))
        return MF_ERR_ALIAS;
    // residual_out may be residual itself; any other overlap of an output with anything is
    // rejected.
    const void* ins[] = {x, gate, gamma, dual ? gamma_next : nullptr, residual};
    const size_t in_bytes[] = {th * 2, th * 2, size_t(H) * 2, size_t(H) * 2, th * 4};
    uint16_t* bf_outs[] = {out, dual ? out_next : nullptr};
    for (int i = 0; i < 5; ++i) {
        if (i < 4 && overlap(residual_out, th * 4, ins[i], in_bytes[i])) return MF_ERR_ALIAS;
        for (uint16_t* o : bf_outs)
            if (overlap(o, th * 2, ins[i], in_bytes[i])) return MF_ERR_ALIAS;
    }
    for (uint16_t* o : bf_outs)
        if (overlap(o, th * 2, residual_out, th * 4)) return MF_ERR_ALIAS;
    if (dual && overlap(out, th * 2, out_next, th * 2)) return MF_ERR_ALIAS;

    GatedArgs a;
    a.x = x;
    a.gate = gate;
    a.residual = residual;
    a.residual_out = residual_out;
    a.gamma = gamma;
    a.out = out;
    a.gamma_next = dual ? gamma_next : nullptr;
    a.out_next = dual ? out_next : nullptr;
    a.T = T;
    a.H = H;
    a.eps = eps;
    void* args[] = {&a};
    return hip_status(hipLaunchKernel(fn, dim3((unsigned)s.grid), dim3(s.block), args, s.lds,
                                      reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

namespace mf {

const void* gated_kernel_for(const RowShape& s, bool dual) {
    return dual ? gated_kernel_for_vpl<true>(s.vpl, s.tail) : gated_kernel_for_vpl<false>(s.vpl, s.tail);
}

}  // namespace mf

extern "C" {

int mf_gated_residual_rmsnorm_supported(int32_t H) { return row_width_supported(H); }

int mf_gated_residual_next_rmsnorm_supported(int32_t H) { return row_width_supported(H); }

int mf_rmsnorm_sigmoid_gate_supported(int32_t head_dim) { return head_dim == kHeadDim; }

int mf_gated_residual_rmsnorm(const uint16_t* x, const uint16_t* gate, const float* residual,
                              float* residual_out, const uint16_t* gamma, float eps,
                              uint16_t* out, int64_t T, int32_t H, void* stream) {
    return launch_gated(x, gate, residual, residual_out, gamma, nullptr, eps, out, nullptr, T, H,
                        false, stream);
}

int mf_gated_residual_next_rmsnorm(const uint16_t* x, const uint16_t* gate,
                                   const float* residual, float* residual_out,
                                   const uint16_t* gamma, const uint16_t* gamma_next, float eps,
                                   uint16_t* out, uint16_t* out_next, int64_t T, int32_t H,
                                   void* stream) {
    return launch_gated(x, gate, residual, residual_out, gamma, gamma_next, eps, out, out_next, T,
                        H, true, stream);
}

int mf_rmsnorm_sigmoid_gate(const uint16_t* x, const uint16_t* gate, const uint16_t* gamma,
                            float eps, uint16_t* out, int64_t T, int32_t num_heads,
                            int32_t head_dim, void* stream) {
    if (T < 0 || num_heads < 1) return MF_ERR_SHAPE;
    if (!mf_rmsnorm_sigmoid_gate_supported(head_dim)) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    const int64_t nh = T * num_heads;
    const int64_t groups = (nh + kHeadsPerWaveLoad - 1) / kHeadsPerWaveLoad;
    if (!grid_fits(groups, kPerHeadBlock)) return MF_ERR_SHAPE;
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
    // the full-tile kernel when the heads fill whole waves, else the one with the tail handling
    const void* fn = nh % kHeadsPerWaveLoad == 0
                         ? reinterpret_cast<const void*>(&rmsnorm_sigmoid_gate_kernel<false>)
                         : reinterpret_cast<const void*>(&rmsnorm_sigmoid_gate_kernel<true>);
    return hip_status(hipLaunchKernel(fn, dim3((unsigned)groups), dim3(kPerHeadBlock), args, 0,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int mf_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16 != 0) return MF_ERR_SHAPE;
    if (bytes == 0) return MF_OK;
    if (!src || !dst) return MF_ERR_NULL;
    if (!aligned(src, 16) || !aligned(dst, 16)) return MF_ERR_ALIGN;
    if (overlap(src, size_t(bytes), dst, size_t(bytes))) return MF_ERR_ALIAS;
    const int64_t n = bytes / 16;
    const int64_t blocks = (n + kCopyBlock - 1) / kCopyBlock;
    if (!grid_fits(blocks, kCopyBlock)) return MF_ERR_SHAPE;
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    void* args[] = {&s, &d, const_cast<int64_t*>(&n)};
    return hip_status(hipLaunchKernel(reinterpret_cast<const void*>(&stream_copy_kernel),
                                      dim3((unsigned)blocks), dim3(kCopyBlock), args, 0,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int mf_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    if (bytes < 0 || bytes % 16 != 0) return MF_ERR_SHAPE;
    if (bytes == 0) return MF_OK;
    if (!src || !sink) return MF_ERR_NULL;
    if (!aligned(src, 16) || !aligned(sink, 4)) return MF_ERR_ALIGN;
    constexpr int U = 4;
    const int64_t n = bytes / 16;
    const int64_t blocks = (n + 256 * U - 1) / (256 * U);
    static_assert(256 * U * 16 == MF_STREAM_READ_CHUNK, "one workgroup per chunk");
    if (overlap(src, size_t(bytes), sink, size_t(blocks) * 4)) return MF_ERR_ALIAS;
    if (!grid_fits(blocks, 256)) return MF_ERR_SHAPE;
    const u32x4* s = static_cast<const u32x4*>(src);
    void* args[] = {&s, &sink, const_cast<int64_t*>(&n)};
    return hip_status(hipLaunchKernel(reinterpret_cast<const void*>(&stream_read_kernel<U>),
                                      dim3((unsigned)blocks), dim3(256), args, 0,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int mf_empty_grid(int64_t workgroups, int32_t threads, void* stream) {
    if (workgroups < 1 || threads < 1 || threads > 1024) return MF_ERR_SHAPE;
    if (!grid_fits(workgroups, threads)) return MF_ERR_SHAPE;
    return hip_status(hipLaunchKernel(reinterpret_cast<const void*>(&empty_grid_kernel),
                                      dim3((unsigned)workgroups), dim3(threads), nullptr, 0,
                                      reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
