// MXFP4 block quantisation on gfx950, alone and after an RMSNorm.
//
// What it computes (page "FlashInfer: fused norms and TP/EP MoE for Muse-Spark-Open", PR #6544,
// section 2.3: RMSNorm + block-scaled FP4 quantisation, NVFP4 there; retargeted to the OCP
// Microscaling MXFP4 format, from its published definition): blocks of 32 consecutive values of
// a row share one E8M0 scale X = 2^e, e = floor(log2(max|v|)) - 2 clamped to [-127, 127] (an
// all-zero block takes -127); each value is stored as the E2M1 code nearest to v / X (ties to
// the even code, saturating at 6, the sign kept for zeros), two codes per byte with the
// even-indexed value in the low nibble.
//
// How it maps onto CDNA4:
//  - A lane holds 8 consecutive values, so a block of 32 is one quad of lanes; the block maximum
//    is a DPP max over the quad.
//  - e + 127 is the biased exponent of the block maximum minus 2 (floor(log2) of a float is its
//    exponent field), clamped at 0.
//  - The conversion is gfx950's v_cvt_scalef32_pk_fp4_f32: two fp32 values divided by the
//    power-of-two scale, rounded to nearest even and saturated, into one byte; four of them
//    fill the lane's 32-bit word of codes.
#pragma once

#include "mx_device.h"
#include "row_norm.h"

namespace mf {

// ---------------------------------------------------------------------------------------
// fp32 [T, H] -> codes [T, H/2], scales [T, H/32] (H % 32 == 0).  Flat over 8-value chunks:
// chunk c covers values [8c, 8c + 8) of the flattened array; a block never crosses a row
// because H / 8 is a multiple of 4.  Chunks past the end (whole quads, since the chunk count
// is a multiple of 4) load a clamped chunk and store nothing.
struct MxArgs {
    const float* x;
    uint8_t* q;
    uint8_t* scales;
    int64_t chunks;  // T * H / 8
};

constexpr int kMxThreads = 256;

__global__ void __launch_bounds__(kMxThreads) mxfp4_quantize_kernel(const MxArgs a) {
    const int64_t c = int64_t(blockIdx.x) * kMxThreads + threadIdx.x;
    const int64_t cl = c < a.chunks ? c : a.chunks - 1;
    const f32x4 lo = ld_stream(reinterpret_cast<const f32x4*>(a.x + cl * 8));
    const f32x4 hi = ld_stream(reinterpret_cast<const f32x4*>(a.x + cl * 8 + 4));
    const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const uint32_t code = mx_scale_code(mx_block_max(v));
    const uint32_t w = mx_pack8(v, mx_scale_value(code));
    if (c < a.chunks) {
        reinterpret_cast<uint32_t*>(a.q)[c] = w;
        if ((threadIdx.x & 3) == 0) a.scales[c / 4] = uint8_t(code);
    }
}

// ---------------------------------------------------------------------------------------
// RMSNorm of bf16 rows, then MXFP4: the row framework of the fused norms (one workgroup per
// token), y = (x * inv) * gamma in fp32 exactly as the bf16 RMSNorm output is formed, then the
// quantisation above per slot.  H % 32 == 0, so a quad is wholly inside or wholly past the row.
struct RmsMxArgs {
    const uint16_t* x;      // bf16 [T, H]
    const uint16_t* gamma;  // bf16 [H]
    uint8_t* q;             // [T, H/2]
    uint8_t* scales;        // [T, H/32]
    int64_t T;
    int32_t H;
    float eps;
};

template <int VPL, int TAIL>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(VPL == 1 ? 8 : 4, 8)))
rmsnorm_mxfp4_kernel(const RmsMxArgs a) {
    extern __shared__ float lds[];
    const RowMap m = row_map();
    const int H = a.H;
    const Slots<VPL, TAIL> sl = slot_offsets<VPL, TAIL>(m, H);
    const uint16_t* xr = a.x + m.t * H;

    u32x4 xv[VPL], gm[VPL];
#pragma unroll
    for (int s = 0; s < VPL; ++s)
        xv[s] = sl.suni[s] ? ld_stream(at<u32x4>(xr, sl.eoff[s] * 2u)) : u32x4{0u, 0u, 0u, 0u};
    load_gamma(gm, a.gamma, sl);
    float x[VPL][8];
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        widen8(xv[s], x[s]);
        if (!sl.sval[s]) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[s][i] = 0.0f;
        }
    }
    float ss[1] = {lane_sumsq(x, sl)};
    TokenLds L = token_lds(lds, m.wpt, 1);
    token_sum<1>(ss, L, m);
    const float inv = rms_scale(ss[0], 1.0f / (float)H, a.eps);
    mx_store_normed(x, gm, sl, inv, m.lane, a.q + m.t * (H / 2), a.scales + m.t * (H / 32));
}

}  // namespace mf
