// Row mapping and the fixed-order row reduction shared by the token-row kernels (MoE
// finalize and gated-residual RMSNorm).
//
// One workgroup handles one token row of H values.  The row is cut into slots of 512 values
// (one 16-byte vector per lane of a wavefront, 1 KiB of bf16 or 2 KiB of fp32); the
// workgroup's `wpt` waves own VPL consecutive slots each: wave w holds slots
// [w*VPL, w*VPL + VPL), lane l the values [slot*512 + 8l, +8) of each.  The shape depends on H
// only, never on the token count, so every token is computed the same way whatever the
// batch: results are bit-identical for a token alone or inside any batch.
//
// Sums over the row have one fixed order: per lane, its slots in order; then, per lane
// position, the waves in order (through LDS); then the fixed 64-lane order of wave_sum.
#pragma once

#include "mf_device.h"

namespace mf {

struct RowMap {
    int lane;   // lane in the wave
    int wave;   // wave in the workgroup = wave in the token (uniform)
    int wpt;    // waves per token = waves per workgroup
    int64_t t;  // token
};

__device__ __forceinline__ RowMap row_map() {
    RowMap m;
    m.lane = threadIdx.x & (kWave - 1);
    m.wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    m.wpt = blockDim.x / kWave;
    m.t = blockIdx.x;
    return m;
}

// How a row's slots meet its end:
//   kRowFull   - H = wpt * VPL * 512: every slot of every wave is inside the row;
//   kRowWhole  - H is a multiple of 512: a slot is entirely inside or entirely past the row,
//                so validity is uniform per wave and slot;
//   kRowRagged - the last slot is cut inside, so validity is per lane.
enum RowTail { kRowFull = 0, kRowWhole = 1, kRowRagged = 2 };

// Offsets of the slots a lane holds.  eoff[s]: element offset of its 8 values (0 when they
// lie past H); sval[s]: they lie inside the row; suni[s] (wave-uniform): the slot starts
// inside the row.
template <int VPL, int TAIL>
struct Slots {
    uint32_t eoff[VPL];
    bool sval[VPL];
    bool suni[VPL];
};

template <int VPL, int TAIL>
__device__ __forceinline__ Slots<VPL, TAIL> slot_offsets(const RowMap& m, int H) {
    Slots<VPL, TAIL> sl;
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        const int slot = m.wave * VPL + s;
        const uint32_t e = uint32_t(slot * kSlot + m.lane * kVec);
        sl.suni[s] = TAIL == kRowFull || slot * kSlot < H;
        sl.sval[s] = TAIL == kRowRagged ? e < uint32_t(H) : sl.suni[s];
        sl.eoff[s] = sl.sval[s] ? e : 0u;
    }
    return sl;
}

// Cross-wave reductions of a token go through LDS in two alternating halves, each sized
// for the largest number of sums (NRMAX) any call of the kernel reduces at once: a half holds
// [wpt][NR][64] lane partials followed by [NR] totals.  Consecutive calls use different
// halves, and a half is only rewritten two calls later, after every wave has passed the
// barrier of the call in between, i.e. after every wave has finished reading it.
struct TokenLds {
    float* base;
    int half;    // floats per half
    int parity;  // half the next call uses
};

__device__ __forceinline__ TokenLds token_lds(float* lds, int wpt, int nr_max) {
    return TokenLds{lds, wpt * nr_max * kWave + nr_max, 0};
}

// Reduce NR row sums over the token (NR <= the NRMAX the LDS was sized for).  On entry v[n]
// is this lane's partial; on exit every lane of every wave holds the token total.  With
// wpt > 1 the waves meet at workgroup barriers, so all waves must make the same calls.
//  - NR == 1: one barrier; every wave adds the wpt partials of its lane position in order.
//  - NR > 1: wave w finishes rows w, w + wpt, ... and publishes them; a second barrier, then
//    every wave reads the NR totals.
// Sum, in wave order, of the wpt partials held at part[w * stride + lane] (all reads issued
// together; trailing zeros for w >= wpt leave the sum unchanged: a sum of squares is never -0).
__device__ __forceinline__ float sum_waves(const float* part, int stride, int wpt, int lane) {
    constexpr int kMaxWaves = 16;
    float c[kMaxWaves];
#pragma unroll
    for (int w = 0; w < kMaxWaves; ++w) c[w] = w < wpt ? part[w * stride + lane] : 0.0f;
    float s = c[0];
#pragma unroll
    for (int w = 1; w < kMaxWaves; ++w) s += c[w];
    return s;
}

template <int NR>
__device__ __forceinline__ void token_sum(float (&v)[NR], TokenLds& L, const RowMap& m) {
    if (m.wpt == 1) {
#pragma unroll
        for (int n = 0; n < NR; ++n) v[n] = wave_sum(v[n]);
        return;
    }
    float* part = L.base + (size_t)L.parity * L.half;
    float* tot = part + m.wpt * NR * kWave;
    L.parity ^= 1;
#pragma unroll
    for (int n = 0; n < NR; ++n) part[(m.wave * NR + n) * kWave + m.lane] = v[n];
    __syncthreads();
    if constexpr (NR == 1) {
        v[0] = wave_sum(sum_waves(part, kWave, m.wpt, m.lane));
    } else {
        for (int n = m.wave; n < NR; n += m.wpt) {
            const float s = wave_sum(sum_waves(part + n * kWave, NR * kWave, m.wpt, m.lane));
            if (m.lane == 0) tot[n] = s;
        }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < NR; ++n) v[n] = tot[n];
    }
}

// LDS bytes for `wpt` waves reducing at most nr_max sums per call.
constexpr size_t token_sum_lds_bytes(int wpt, int nr_max) {
    return wpt > 1 ? size_t(2) * (wpt * nr_max * kWave + nr_max) * sizeof(float) : 0;
}

// Sum of squares of the lane's valid values, its slots in order.
template <int VPL, int TAIL>
__device__ __forceinline__ float lane_sumsq(const float (&r)[VPL][8], const Slots<VPL, TAIL>& sl) {
    float p = 0.0f;
#pragma unroll
    for (int s = 0; s < VPL; ++s) p += sl.sval[s] ? sumsq8(r[s]) : 0.0f;
    return p;
}

// Store of the updated fp32 residual row (after every residual load of the row).  A lane holds
// 8 consecutive values (32 bytes), so storing them directly would make each wave instruction
// write every other 16 bytes of a 2 KiB span; on MI355X such half-line nontemporal stores run
// at about two thirds of the rate of contiguous ones.  So the lanes first exchange halves with
// ds_bpermute: for the first store lane l takes slot elements 4l..4l+3 (the first or second
// half of lane l/2's values), for the second 256+4l..256+4l+3 (from lane 32 + l/2), and each
// store instruction writes 1 KiB contiguous.  A store is valid exactly when its source lane's
// values are, since H % 8 == 0.  Every lane of the wave must be active.  Used for every fp32
// row the kernels write (the residual, the expert-parallel partial).  Measured: the finalize
// 1.5% and the gated-residual norm 7% faster than the direct stores, results identical.
// (The slots argument only selects the tail handling.)
// One slot (the 512 values from slot * 512) of the row, held as 8 values per lane.
template <int TAIL>
__device__ __forceinline__ void store_residual_slot(const float (&v)[8], int slot, const RowMap& m,
                                                    int H, float* row) {
    const int l = m.lane;
    const int a0 = (l >> 1) << 2, a1 = (32 + (l >> 1)) << 2;  // source lanes, as byte addresses
    const bool odd = l & 1;
    const uint32_t base = uint32_t(slot * kSlot);
    float t0[4], t1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int lo = __float_as_int(v[i]), hi = __float_as_int(v[4 + i]);
        const float x0 = __int_as_float(__builtin_amdgcn_ds_bpermute(a0, lo));
        const float y0 = __int_as_float(__builtin_amdgcn_ds_bpermute(a0, hi));
        const float x1 = __int_as_float(__builtin_amdgcn_ds_bpermute(a1, lo));
        const float y1 = __int_as_float(__builtin_amdgcn_ds_bpermute(a1, hi));
        t0[i] = odd ? y0 : x0;
        t1[i] = odd ? y1 : x1;
    }
    const uint32_t e0 = base + 4u * l, e1 = base + 256u + 4u * l;
    bool v0, v1;
    if constexpr (TAIL == kRowFull) {
        v0 = v1 = true;
    } else if constexpr (TAIL == kRowWhole) {
        v0 = v1 = base < uint32_t(H);
    } else {
        v0 = e0 < uint32_t(H);
        v1 = e1 < uint32_t(H);
    }
    if (v0) st_stream(f32x4{t0[0], t0[1], t0[2], t0[3]}, at<f32x4>(row, e0 * 4u));
    if (v1) st_stream(f32x4{t1[0], t1[1], t1[2], t1[3]}, at<f32x4>(row, e1 * 4u));
}

template <int VPL, int TAIL>
__device__ __forceinline__ void store_residual(const float (&r)[VPL][8], const Slots<VPL, TAIL>&,
                                               const RowMap& m, int H, float* row) {
#pragma unroll
    for (int s = 0; s < VPL; ++s) store_residual_slot<TAIL>(r[s], m.wave * VPL + s, m, H, row);
}

// gamma slice of the lane (bf16, loaded early so that its latency overlaps other work).
template <int VPL, int TAIL>
__device__ __forceinline__ void load_gamma(u32x4 (&g)[VPL], const uint16_t* gamma,
                                           const Slots<VPL, TAIL>& sl) {
#pragma unroll
    for (int s = 0; s < VPL; ++s) g[s] = *at<u32x4>(gamma, sl.eoff[s] * 2u);
}

// Final RMSNorm of a row held as r[VPL][8] (fp32) and the bf16 store of out:
//   out = bf16((r * (sum(r^2)/H + eps)^-1/2) * gamma).
// OUT_NT selects the cache policy of the out stores, which was measured per kernel on MI355X:
// the finalize and the gated-residual norm are faster with the default policy (4% for the
// finalize; each wave instruction writes whole 128-byte lines), the expert-parallel combine
// 3% faster with nontemporal stores.
// (lane_ss: the lane's sum of squares of its valid values, its slots in order, if the caller
// has already formed it as lane_sumsq would; else it is formed here.)
// The bf16 out of one slot's 8 values of a lane: bf16((v * inv) * gamma), stored at dst.
template <bool OUT_NT = false>
__device__ __forceinline__ void norm_store_slot(const float (&v)[8], const u32x4& g, float inv,
                                                uint16_t* dst) {
    float gf[8];
    widen8(g, gf);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2((v[2 * i] * inv) * gf[2 * i], (v[2 * i + 1] * inv) * gf[2 * i + 1]);
    if constexpr (OUT_NT)
        st_stream(o, reinterpret_cast<u32x4*>(dst));
    else
        *reinterpret_cast<u32x4*>(dst) = o;
}

template <bool OUT_NT = false, int VPL, int TAIL>
__device__ __forceinline__ void rmsnorm_store(const float (&r)[VPL][8], const u32x4 (&g)[VPL],
                                              const Slots<VPL, TAIL>& sl, uint16_t* out_row,
                                              int H, float eps, TokenLds& L, const RowMap& m,
                                              const float* lane_ss = nullptr) {
    float ss[1] = {lane_ss ? *lane_ss : lane_sumsq(r, sl)};
    token_sum<1>(ss, L, m);
    const float inv = rms_scale(ss[0], 1.0f / (float)H, eps);
#pragma unroll
    for (int s = 0; s < VPL; ++s)
        if (sl.sval[s]) norm_store_slot<OUT_NT>(r[s], g[s], inv, at<uint16_t>(out_row, sl.eoff[s] * 2u));
}

}  // namespace mf
