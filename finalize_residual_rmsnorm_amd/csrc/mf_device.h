// Device helpers for the gfx950 kernels: vector types, bf16 conversion, streaming
// loads/stores and fixed-order reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mf {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;                      // lanes per wavefront (CDNA)
constexpr int kVec = 8;                        // bf16 values in one 16-byte vector
constexpr int kSlot = kWave * kVec;            // 512 values: one 16-byte vector per lane

constexpr int next_pow2(int n) { return n <= 1 ? 1 : 2 * next_pow2((n + 1) / 2); }

// bf16 -> fp32 is exact: a bf16 is the upper half of a binary32.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ void widen8(const u32x4 v, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(v[i]);
        x[2 * i + 1] = bf16_hi(v[i]);
    }
}

// Two fp32 -> packed bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Address `base + byte_off` with a 32-bit unsigned offset: with a wave-uniform base this allows
// the SGPR-base + VGPR-offset form of global loads/stores (no 64-bit address per lane; the
// compiler may still form per-lane addresses, e.g. when it shares `base + offset` between
// several uniform bases).
template <class T>
__device__ __forceinline__ const T* at(const void* base, uint32_t byte_off) {
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}
template <class T>
__device__ __forceinline__ T* at(void* base, uint32_t byte_off) {
    return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off);
}

// Single-use streams (gathered rows, residual in/out) bypass cache retention.
template <class T>
__device__ __forceinline__ T ld_stream(const T* p) { return __builtin_nontemporal_load(p); }
template <class T>
__device__ __forceinline__ void st_stream(T v, T* p) { __builtin_nontemporal_store(v, p); }

// A load whose cache policy is a compile-time choice (nontemporal or default).
template <bool NT, class T>
__device__ __forceinline__ T ld_policy(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each group of 8 consecutive lanes, returned to all 8 (quad swaps, then the
// half-row mirror).  Every lane of a group gets the bit-identical value.
__device__ __forceinline__ float sum8_lanes(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    return v;
}

// Sum over all 64 lanes in one fixed order; every lane gets the same value.
// Within each row of 16 lanes: a butterfly through DPP; then the four row sums are added as
// (row0 + row1) + (row2 + row3).  Must be called with all 64 lanes active.
__device__ __forceinline__ float wave_sum(float v) {
    v = sum8_lanes(v);
    v += dpp<0x140>(v);  // row_mirror
    float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// The RMSNorm scale (mean + eps)^-1/2 of a row sum of squares: the mean as ss * (1/n) and the
// hardware reciprocal square root.  Both are within a few fp32 ulps of the exact value, far
// below half an ulp of the bf16 (or MXFP4) outputs the scale feeds, and a fixed function of ss:
// the same ss always gives the same scale.
__device__ __forceinline__ float rms_scale(float ss, float inv_n, float eps) {
    return __builtin_amdgcn_rsqf(__builtin_fmaf(ss, inv_n, eps));
}

// Sum of squares of eight values in index order.
__device__ __forceinline__ float sumsq8(const float (&x)[8]) {
    float s = x[0] * x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) s = __builtin_fmaf(x[i], x[i], s);
    return s;
}

}  // namespace mf
