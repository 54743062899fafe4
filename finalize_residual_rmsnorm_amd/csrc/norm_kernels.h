// The two fused norms that sit beside the MoE finalize, and a streaming copy used to
// measure the achievable HBM bandwidth.
#pragma once

#include "row_norm.h"

namespace mf {

// ---------------------------------------------------------------------------------------
// Gated-residual RMSNorm (page "FlashInfer: fused norms and TP/EP MoE for Muse-Spark-Open",
// PR #6544, section 1.1, and its "Fixed-Width Fused Norms" docs at hidden size 8192):
//   residual_out = residual + sigmoid(gate) * x      (fp32 stream, one rounding via fma)
//   out = bf16(residual_out * (mean(residual_out^2) + eps)^-1/2 * gamma)
// Same row mapping and fixed reduction tree as the finalize kernel.  The sigmoid uses the
// hardware exp2 and an IEEE division so that residual_out stays within a few fp32 ulps of
// the exact value; that keeps the kernel bound by HBM rather than by the transcendental.
// Cache policies, measured on MI355X with inputs and outputs rotated past the Infinity Cache:
// the single-output form is fastest with every stream nontemporal except the bf16 out store;
// the dual form with default-policy residual loads and nontemporal stores of both bf16
// outputs (6% faster than the single form's policy).
//
// DUAL: the dual-output form (gated_residual_next_rmsnorm, named by the same page's docs and
// its section 2.2 "gated residual dual norm", not defined there).  Reading taken: the one
// gated residual and its one mean square feed two outputs, this layer's RMSNorm (gamma) and
// the next layer's (gamma_next):
//   out_next = bf16(residual_out * (mean(residual_out^2) + eps)^-1/2 * gamma_next)
// out is computed exactly as without DUAL, so it is bit-identical to the single-output form.
struct GatedArgs {
    const uint16_t* x;           // bf16 [T, H]
    const uint16_t* gate;        // bf16 [T, H]
    const float* residual;       // [T, H]
    float* residual_out;         // [T, H], may equal residual
    const uint16_t* gamma;       // bf16 [H]
    uint16_t* out;               // bf16 [T, H]
    const uint16_t* gamma_next;  // bf16 [H] (DUAL only)
    uint16_t* out_next;          // bf16 [T, H] (DUAL only)
    int64_t T;
    int32_t H;
    float eps;
};

// The final RMSNorm of a row into two bf16 outputs with one mean square: the same arithmetic
// as rmsnorm_store, applied with each gamma.
template <int VPL, int TAIL>
__device__ __forceinline__ void rmsnorm_store_dual(const float (&r)[VPL][8], const u32x4 (&g)[VPL],
                                                   const u32x4 (&gn)[VPL],
                                                   const Slots<VPL, TAIL>& sl, uint16_t* out_row,
                                                   uint16_t* next_row, int H, float eps,
                                                   TokenLds& L, const RowMap& m) {
    float ss[1] = {lane_sumsq(r, sl)};
    token_sum<1>(ss, L, m);
    const float inv = 1.0f / __builtin_sqrtf(ss[0] / (float)H + eps);
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        float gf[8], gnf[8];
        widen8(g[s], gf);
        widen8(gn[s], gnf);
        u32x4 o, on;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float y0 = r[s][2 * i] * inv, y1 = r[s][2 * i + 1] * inv;
            o[i] = pack_bf16x2(y0 * gf[2 * i], y1 * gf[2 * i + 1]);
            on[i] = pack_bf16x2(y0 * gnf[2 * i], y1 * gnf[2 * i + 1]);
        }
        if (sl.sval[s]) {
            st_stream(o, at<u32x4>(out_row, sl.eoff[s] * 2u));
            st_stream(on, at<u32x4>(next_row, sl.eoff[s] * 2u));
        }
    }
}

__device__ __forceinline__ float sigmoid_accurate(float g) {
    return 1.0f / (1.0f + __expf(-g));
}

template <int VPL, int TAIL, bool DUAL>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(VPL == 1 ? 7 : 4, 8)))
gated_residual_rmsnorm_kernel(const GatedArgs a) {
    extern __shared__ float lds[];
    const RowMap m = row_map();
    const int H = a.H;
    const Slots<VPL, TAIL> sl = slot_offsets<VPL, TAIL>(m, H);
    const int64_t row = m.t * H;
    const uint16_t* xr = a.x + row;
    const uint16_t* gr = a.gate + row;
    const float* res = a.residual + row;

    u32x4 xv[VPL], gv[VPL], gm[VPL], gn[VPL];
    f32x4 rv[VPL][2];
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        xv[s] = ld_stream(at<u32x4>(xr, sl.eoff[s] * 2u));
        gv[s] = ld_stream(at<u32x4>(gr, sl.eoff[s] * 2u));
        rv[s][0] = ld_policy<!DUAL>(at<f32x4>(res, sl.eoff[s] * 4u));
        rv[s][1] = ld_policy<!DUAL>(at<f32x4>(res, sl.eoff[s] * 4u + 16u));
    }
    load_gamma(gm, a.gamma, sl);
    if constexpr (DUAL) load_gamma(gn, a.gamma_next, sl);
    float r[VPL][8];
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        float x[8], g[8];
        widen8(xv[s], x);
        widen8(gv[s], g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r[s][i] = __builtin_fmaf(sigmoid_accurate(g[i]), x[i], rv[s][0][i]);
            r[s][4 + i] = __builtin_fmaf(sigmoid_accurate(g[4 + i]), x[4 + i], rv[s][1][i]);
        }
    }
    store_residual(r, sl, m, H, a.residual_out + row);
    TokenLds L = token_lds(lds, m.wpt, 1);
    if constexpr (DUAL)
        rmsnorm_store_dual(r, gm, gn, sl, a.out + row, a.out_next + row, H, a.eps, L, m);
    else
        rmsnorm_store(r, gm, sl, a.out + row, H, a.eps, L, m);
}

// ---------------------------------------------------------------------------------------
// Per-head RMSNorm with a sigmoid gate (PR #6544 page, section 1.2; head dim 64):
//   out[t,n,:] = bf16(((x * (mean(x^2) + eps)^-1/2) * gamma) * sigmoid(gate))
// One head is 64 bf16 = 128 bytes = 8 lanes x 16 bytes, so a wave covers 8 heads per
// instruction; the sum of squares is reduced in fp32 across the 8 lanes of the head with
// DPP.  Each wave handles GPW groups of 8 heads, all loads issued before use.  The output is
// bf16, so a hardware reciprocal is ample for the sigmoid here.
struct PerHeadArgs {
    const uint16_t* x;      // bf16 [T*heads, 64]
    const uint16_t* gate;   // bf16 [T*heads, 64]
    const uint16_t* gamma;  // bf16 [64]
    uint16_t* out;          // bf16 [T*heads, 64]
    int64_t num_heads_total;
    float eps;
};

constexpr int kHeadDim = 64;
constexpr int kHeadsPerWaveLoad = kWave * kVec / kHeadDim;  // 8

constexpr int kPerHeadBlock = 64;  // threads per workgroup

template <int GPW>
__global__ void __launch_bounds__(kPerHeadBlock) rmsnorm_sigmoid_gate_kernel(const PerHeadArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int d0 = (lane & 7) * kVec;
    const int64_t last = a.num_heads_total - 1;

    float gm[8];
    widen8(*reinterpret_cast<const u32x4*>(a.gamma + d0), gm);

    u32x4 xv[GPW], gv[GPW];
    int64_t head[GPW];
#pragma unroll
    for (int g = 0; g < GPW; ++g) {
        head[g] = (wave * GPW + g) * kHeadsPerWaveLoad + (lane >> 3);
        const int64_t hc = head[g] < last ? head[g] : last;
        xv[g] = ld_stream(reinterpret_cast<const u32x4*>(a.x + hc * kHeadDim + d0));
        gv[g] = ld_stream(reinterpret_cast<const u32x4*>(a.gate + hc * kHeadDim + d0));
    }
#pragma unroll
    for (int g = 0; g < GPW; ++g) {
        float x[8], gt[8];
        widen8(xv[g], x);
        widen8(gv[g], gt);
        const float ss = sum8_lanes(sumsq8(x));
        const float inv = 1.0f / __builtin_sqrtf(ss * (1.0f / kHeadDim) + a.eps);
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s0 = __builtin_amdgcn_rcpf(1.0f + __expf(-gt[2 * i]));
            const float s1 = __builtin_amdgcn_rcpf(1.0f + __expf(-gt[2 * i + 1]));
            o[i] = pack_bf16x2(((x[2 * i] * inv) * gm[2 * i]) * s0,
                               ((x[2 * i + 1] * inv) * gm[2 * i + 1]) * s1);
        }
        if (head[g] <= last) st_stream(o, reinterpret_cast<u32x4*>(a.out + head[g] * kHeadDim + d0));
    }
}

// ---------------------------------------------------------------------------------------
// Streaming copy with 16-byte vectors, U vectors in flight per lane.
template <int U>
__global__ void __launch_bounds__(256) stream_copy_kernel(const u32x4* src, u32x4* dst, int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * (blockDim.x * U) + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * blockDim.x;
        if (i < n) v[u] = ld_stream(src + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * blockDim.x;
        if (i < n) st_stream(v[u], dst + i);
    }
}

}  // namespace mf
