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
// Same row mapping and fixed reduction tree as the finalize kernel.  The sigmoid is formed in
// fp32 from the hardware exp (sigmoid_f32).
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
    const float inv = rms_scale(ss[0], 1.0f / (float)H, eps);
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

// sigmoid(g) = 1 / (1 + e^-g) in fp32: the hardware exp2 of -g*log2(e) (its error is a few ulp,
// growing with |g| through the rounding of the scaled argument) and an IEEE division.  The
// rounding of the fp32 sigmoid itself is what makes the gated residual differ from the exactly
// rounded one in about a quarter of the elements (by one ulp or so): on MI355X the library expf
// raised the bit-identical fraction only from 0.754 to 0.768, at 1% more kernel time.
__device__ __forceinline__ float sigmoid_f32(float g) {
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
            r[s][i] = __builtin_fmaf(sigmoid_f32(g[i]), x[i], rv[s][0][i]);
            r[s][4 + i] = __builtin_fmaf(sigmoid_f32(g[4 + i]), x[4 + i], rv[s][1][i]);
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
// One head is 64 bf16 = 128 bytes = 8 lanes x 16 bytes, so one wave covers 8 consecutive heads:
// one contiguous 1 KiB of x, of gate and of out, addressed as a wave-uniform base plus the lane's
// 16-byte offset.  The sum of squares is reduced in fp32 across the 8 lanes of a head with DPP.
// The output is bf16, so the hardware reciprocal square root and reciprocal are ample for the
// scale and the sigmoid (their few-ulp fp32 error is far below half a bf16 ulp).
// TAIL = false is the full-tile kernel (the head count is a multiple of 8: no clamp, no
// predicate); TAIL = true also handles a last wave whose heads end inside it, with the same
// arithmetic on every head that exists (bit-identical to the full-tile kernel there).
// Measured on MI355X at 4096 tokens x 64 heads (cold inputs): the kernel runs in 16.7-17.1 us,
// 96-99% of the rate of stream_copy_kernel moving the same 100.7 MB (16.5 us), while an empty
// kernel of the same 32768 one-wave workgroups already takes 7.7 us to dispatch.  Issuing the
// gate load only after the x load has returned measured 1% faster than issuing both at once;
// 4-wave workgroups (5%) and persistent waves that prefetch their next group (11%) measured
// slower.
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

constexpr int kPerHeadBlock = 64;  // threads per workgroup: one wave, one group of 8 heads

template <bool TAIL>
__global__ void __launch_bounds__(kPerHeadBlock) rmsnorm_sigmoid_gate_kernel(const PerHeadArgs a) {
    const int lane = threadIdx.x;
    const int64_t group = blockIdx.x;
    const uint32_t off = uint32_t(lane) * 16u;            // byte offset of the lane's 8 values
    const int64_t first = group * (kHeadsPerWaveLoad * kHeadDim);  // first value of the wave
    const uint16_t* xw = a.x + first;
    const uint16_t* gw = a.gate + first;
    uint16_t* ow = a.out + first;
    // TAIL: lanes whose head lies past the last one load nothing and store nothing
    const bool live = !TAIL || group * kHeadsPerWaveLoad + (lane >> 3) < a.num_heads_total;

    float gm[8];
    widen8(*at<u32x4>(a.gamma, uint32_t(lane & 7) * 16u), gm);
    u32x4 xv = u32x4{0u, 0u, 0u, 0u}, gv = u32x4{0u, 0u, 0u, 0u};
    if (live) xv = ld_stream(at<u32x4>(xw, off));
    float x[8], gt[8];
    widen8(xv, x);
    const float ss = sum8_lanes(sumsq8(x));
    // the gate load is issued after the x load has returned (see above)
    __builtin_amdgcn_sched_barrier(0);
    if (live) gv = ld_stream(at<u32x4>(gw, off));
    widen8(gv, gt);
    const float inv = rms_scale(ss, 1.0f / kHeadDim, a.eps);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float s0 = __builtin_amdgcn_rcpf(1.0f + __expf(-gt[2 * i]));
        const float s1 = __builtin_amdgcn_rcpf(1.0f + __expf(-gt[2 * i + 1]));
        o[i] = pack_bf16x2(((x[2 * i] * inv) * gm[2 * i]) * s0,
                           ((x[2 * i + 1] * inv) * gm[2 * i + 1]) * s1);
    }
    if (live) st_stream(o, at<u32x4>(ow, off));
}

// ---------------------------------------------------------------------------------------
// An empty kernel: the dispatch floor of a grid shape (a measurement aid).
__global__ void empty_grid_kernel() {}

// ---------------------------------------------------------------------------------------
// Streaming copy: one 16-byte vector per lane, one wave per workgroup (kCopyBlock threads).
// Measured on MI355X, cold, the fastest simple copy at every size tried: 83.7% of 8 TB/s for
// 2 GiB moved, against 81.2% with 256-thread workgroups and 77.5% with four vectors per lane in
// 256-thread workgroups; 82.5% at 470 MB, 73.6% at 101 MB, 71.8% at 85 MB (3-8 points above
// the others).
constexpr int kCopyBlock = 64;
__global__ void __launch_bounds__(kCopyBlock) stream_copy_kernel(const u32x4* src, u32x4* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kCopyBlock + threadIdx.x;
    if (i < n) st_stream(ld_stream(src + i), dst + i);
}

// Streaming read with 16-byte vectors, U vectors in flight per lane (a measurement aid: the HBM
// read rate with nothing written but one word per chunk).  Each workgroup reads one chunk of
// 256 * U vectors and writes the xor of its 32-bit words to sink[blockIdx.x].
// A chunk wholly inside the source is read with no per-vector test: guarding each load
// separately made the compiler wait for every other load before issuing the next.
template <int U>
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* src, uint32_t* sink, int64_t n) {
    __shared__ uint32_t part[256 / kWave];
    const int64_t chunk = (int64_t)blockDim.x * U;
    const int64_t base = (int64_t)blockIdx.x * chunk + threadIdx.x;
    u32x4 v[U];
    if ((int64_t)(blockIdx.x + 1) * chunk <= n) {
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld_stream(src + base + (int64_t)u * blockDim.x);
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * blockDim.x;
            v[u] = i < n ? ld_stream(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    uint32_t x = 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
#pragma unroll
    for (int d = kWave / 2; d >= 1; d /= 2) x ^= uint32_t(__shfl_xor(int(x), d, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0u;
        for (int w = 0; w < int(blockDim.x / kWave); ++w) r ^= part[w];
        sink[blockIdx.x] = r;
    }
}

}  // namespace mf
