// MXFP4 helpers shared by the quantisation kernels and the finalize's MXFP4 epilogue: the OCP
// Microscaling rule (blocks of 32 values, E8M0 scale 2^(floor(log2 max|v|) - 2), E2M1
// elements nearest with ties to even, saturating at 6) mapped onto quads of lanes that hold 8
// consecutive values each, with gfx950's v_cvt_scalef32_pk_fp4_f32 for the elements.
#pragma once

#include "mf_device.h"

namespace mf {

// The E8M0 scale code of a block from its maximum magnitude (>= 0), and the scale as an fp32
// power of two (2^-127, code 0, is a denormal: the conversion takes it as 2^-127).
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
    const int be = int((__float_as_uint(amax) >> 23) & 0xFFu);
    return uint32_t(be > 2 ? be - 2 : 0);
}

__device__ __forceinline__ float mx_scale_value(uint32_t code) {
    return __uint_as_float(code > 0 ? code << 23 : 0x00400000u);
}

// Maximum of |v| over the lane's 8 values and its quad (lanes 4q .. 4q+3, all active).
__device__ __forceinline__ float mx_block_max(const float (&v)[8]) {
    float m = __builtin_fabsf(v[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
    m = __builtin_fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
    m = __builtin_fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
    return m;
}

// The lane's 8 codes, value 2i in the low nibble of byte i.
__device__ __forceinline__ uint32_t mx_pack8(const float (&v)[8], float scale) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], scale, 3);
    return w;
}

// RMSNorm of a row held as r[VPL][8] (fp32), quantised to MXFP4 instead of rounded to bf16:
// y = (r * inv) * gamma exactly as the bf16 output would be formed, then per slot the block
// scale and codes.  q_row / scale_row: the token's [H/2] codes and [H/32] scales.  H % 32 == 0,
// so a quad is wholly inside or wholly past the row; every lane of the wave must be active.
template <int VPL, class SlotsT>
__device__ __forceinline__ void mx_store_normed(const float (&r)[VPL][8], const u32x4 (&g)[VPL],
                                                const SlotsT& sl, float inv, int lane,
                                                uint8_t* q_row, uint8_t* scale_row) {
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        float gf[8], y[8];
        widen8(g[s], gf);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = (r[s][i] * inv) * gf[i];
        const uint32_t code = mx_scale_code(mx_block_max(y));
        const uint32_t w = mx_pack8(y, mx_scale_value(code));
        if (sl.sval[s]) {
            *at<uint32_t>(q_row, sl.eoff[s] / 2u) = w;
            if ((lane & 3) == 0) scale_row[sl.eoff[s] / 32u] = uint8_t(code);
        }
        // one slot at a time: interleaving them only adds register pressure here
        if constexpr (VPL > 1) __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace mf
