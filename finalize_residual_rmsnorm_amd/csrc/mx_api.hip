// Host side of the MXFP4 entry points declared in include/mf.h: argument checks before any HIP
// call, launch-shape selection and kernel dispatch.  Stateless and allocation-free.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "api_util.h"
#include "mf.h"
#include "mx_kernels.h"
#include "row_shape.h"

namespace {

using namespace mf;

bool mx_width_supported(int32_t H) { return H >= 32 && H <= kMaxH && H % 32 == 0; }

// A token moves only 2.5 bytes per value here, so few waves per token, each with several slots
// in flight, keep more tokens resident per CU: 4 waves (unless the row needs more) measured 33%
// faster than one slot on each of 16 waves at H = 8192.
int rms_mx_waves(int32_t H) {
    const int ns = (H + kSlot - 1) / kSlot;
    const int need = pow2_at_least((ns + kMaxVpl - 1) / kMaxVpl);
    return need > 4 ? need : 4;
}

template <int VPL>
const void* rms_mx_fn(int tail) {
    switch (tail) {
        case kRowFull: return reinterpret_cast<const void*>(&rmsnorm_mxfp4_kernel<VPL, kRowFull>);
        case kRowWhole: return reinterpret_cast<const void*>(&rmsnorm_mxfp4_kernel<VPL, kRowWhole>);
        default: return reinterpret_cast<const void*>(&rmsnorm_mxfp4_kernel<VPL, kRowRagged>);
    }
}

const void* rms_mx_kernel_for(const RowShape& s) {
    switch (s.vpl) {
        case 1: return rms_mx_fn<1>(s.tail);
        case 2: return rms_mx_fn<2>(s.tail);
        case 3: return rms_mx_fn<3>(s.tail);
        case 4: return rms_mx_fn<4>(s.tail);
        default: return nullptr;
    }
}

}  // namespace

extern "C" {

int mf_mxfp4_supported(int32_t H) { return mx_width_supported(H); }

int mf_mxfp4_quantize(const float* x, int64_t T, int32_t H, uint8_t* q, uint8_t* scales,
                      void* stream) {
    if (T < 0) return MF_ERR_SHAPE;
    if (!mx_width_supported(H)) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    const int64_t chunks = T * (H / 8);
    const int64_t blocks = (chunks + kMxThreads - 1) / kMxThreads;
    if (!grid_fits(blocks, kMxThreads)) return MF_ERR_SHAPE;
    if (!x || !q || !scales) return MF_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q, 4)) return MF_ERR_ALIGN;
    const size_t n = size_t(T) * H;
    if (overlap(q, n / 2, x, n * 4) || overlap(scales, n / 32, x, n * 4) ||
        overlap(q, n / 2, scales, n / 32))
        return MF_ERR_ALIAS;
    MxArgs a;
    a.x = x;
    a.q = q;
    a.scales = scales;
    a.chunks = chunks;
    void* args[] = {&a};
    return hip_status(hipLaunchKernel(reinterpret_cast<const void*>(&mxfp4_quantize_kernel),
                                      dim3(unsigned(blocks)), dim3(kMxThreads), args, 0,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int mf_rmsnorm_mxfp4_quantize(const uint16_t* x, const uint16_t* gamma, float eps, uint8_t* q,
                              uint8_t* scales, int64_t T, int32_t H, void* stream) {
    if (T < 0) return MF_ERR_SHAPE;
    if (!mx_width_supported(H)) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    const RowShape s = row_shape(T, H, rms_mx_waves(H), kMaxVpl);
    if (!grid_fits(s.grid, s.block)) return MF_ERR_SHAPE;
    const void* fn = rms_mx_kernel_for(s);
    if (!fn) return MF_ERR_UNSUPPORTED;
    if (!x || !gamma || !q || !scales) return MF_ERR_NULL;
    if (!eps_ok(eps)) return MF_ERR_VALUE;
    if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(q, 4)) return MF_ERR_ALIGN;
    const size_t n = size_t(T) * H;
    const void* ins[] = {x, gamma};
    const size_t in_bytes[] = {n * 2, size_t(H) * 2};
    for (int i = 0; i < 2; ++i)
        if (overlap(q, n / 2, ins[i], in_bytes[i]) || overlap(scales, n / 32, ins[i], in_bytes[i]))
            return MF_ERR_ALIAS;
    if (overlap(q, n / 2, scales, n / 32)) return MF_ERR_ALIAS;
    RmsMxArgs a;
    a.x = x;
    a.gamma = gamma;
    a.q = q;
    a.scales = scales;
    a.T = T;
    a.H = H;
    a.eps = eps;
    void* args[] = {&a};
    return hip_status(hipLaunchKernel(fn, dim3(unsigned(s.grid)), dim3(s.block), args, s.lds,
                                      reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
