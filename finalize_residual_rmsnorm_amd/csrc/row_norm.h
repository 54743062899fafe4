// Row mapping and the fixed-order row reduction shared by the token-row kernels
// (MoE finalize and gated-residual RMSNorm).
//
// A token row of H values is cut into slots of 512 values (one 16-byte vector per lane of a
// wavefront).  A token is handled by `wpt` waves (a power of two); wave w of the token owns
// the `spw` consecutive slots starting at w * spw, and each lane holds VPL <= spw of them in
// registers.  Sums over a row always follow one tree, whatever wpt is:
//   per lane, a pairwise tree over the slot partials (padded to a power of two),
//   then a pairwise tree over the waves of the token (through LDS),
//   then the fixed 64-lane order of wave_sum.
// The launch shape therefore never changes a result bit, which keeps outputs independent of
// the token count (a different T can pick a different wpt).
#pragma once

#include "mf_device.h"

namespace mf {

struct RowMap {
    int lane;        // lane in the wave
    int wave;        // wave in the workgroup (uniform)
    int tok_in_blk;  // token slot within the workgroup (uniform)
    int wit;         // wave index within the token (uniform)
    int wpt;         // waves per token
    int64_t t;       // token (clamped to T-1 for the spare waves of the last workgroup)
    bool valid;      // false for spare waves: they compute but store nothing
};

__device__ __forceinline__ RowMap row_map(int64_t T, int wpt) {
    RowMap m;
    m.lane = threadIdx.x & (kWave - 1);
    m.wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    m.wpt = wpt;
    m.tok_in_blk = m.wave / wpt;
    m.wit = m.wave - m.tok_in_blk * wpt;
    const int tpb = (int)(blockDim.x / kWave) / wpt;
    int64_t t = (int64_t)blockIdx.x * tpb + m.tok_in_blk;
    m.valid = t < T;
    m.t = m.valid ? t : T - 1;
    return m;
}

// Reduce NR row sums.  On entry v[n] is this lane's tree root over its slots; on exit every
// lane of every wave of the token holds the token total.  With wpt > 1 the waves of a token
// meet at workgroup barriers, so every wave of the workgroup must make the same calls.
// Layout of `lds` (floats): two halves, each [waves per workgroup][NR][64] lane partials
// followed by [waves per workgroup][NR] totals; `parity` alternates the halves so that no
// extra barrier is needed before a half is reused.
//  - NR == 1: one barrier; every wave combines the wpt partials of its lane itself.
//  - NR > 1: wave w of the token finishes rows w, w + wpt, ... and publishes the totals;
//    a second barrier, then every wave reads the NR totals.  This keeps the registers at
//    WPT_MAX per row instead of NR * WPT_MAX.
template <int NR, int WPT_MAX>
__device__ __forceinline__ void token_sum(float (&v)[NR], float* lds, int& parity,
                                          const RowMap& m) {
    if (m.wpt > 1) {
        const int nw = blockDim.x / kWave;
        float* part = lds + (size_t)parity * nw * NR * (kWave + 1);
        float* tot = part + nw * NR * kWave;
#pragma unroll
        for (int n = 0; n < NR; ++n) part[(m.wave * NR + n) * kWave + m.lane] = v[n];
        __syncthreads();
        const int base = m.tok_in_blk * m.wpt;
        parity ^= 1;
        if constexpr (NR == 1) {
            float c[WPT_MAX];
#pragma unroll
            for (int w = 0; w < WPT_MAX; ++w)
                c[w] = (w < m.wpt) ? part[(base + w) * kWave + m.lane] : 0.0f;
            v[0] = wave_sum(tree_sum<WPT_MAX>(c));
        } else {
            for (int n = m.wit; n < NR; n += m.wpt) {
                float c[WPT_MAX];
#pragma unroll
                for (int w = 0; w < WPT_MAX; ++w)
                    c[w] = (w < m.wpt) ? part[((base + w) * NR + n) * kWave + m.lane] : 0.0f;
                const float q = wave_sum(tree_sum<WPT_MAX>(c));
                if (m.lane == 0) tot[m.tok_in_blk * NR + n] = q;
            }
            __syncthreads();
#pragma unroll
            for (int n = 0; n < NR; ++n) v[n] = tot[m.tok_in_blk * NR + n];
        }
        return;
    }
#pragma unroll
    for (int n = 0; n < NR; ++n) v[n] = wave_sum(v[n]);
}

// LDS bytes token_sum needs for a workgroup of `waves` waves reducing NR sums per call.
constexpr size_t token_sum_lds_bytes(int waves, int nr) {
    return size_t(2) * waves * nr * (kWave + 1) * sizeof(float);
}

// Largest waves-per-token a VPL instantiation is launched with, and the matching workgroup
// bound: the row slice in registers shrinks as the token is spread over more waves.
constexpr int wpt_max_for(int vpl) { return vpl <= 4 ? 16 : (vpl <= 8 ? 8 : 4); }
constexpr int block_max_for(int vpl) { return vpl <= 4 ? 1024 : (vpl <= 8 ? 512 : 256); }

// Final RMSNorm of a row held as r[VPL][8] (fp32) and the bf16 store of out:
//   out = bf16((r * (sum(r^2)/H + eps)^-1/2) * gamma).
// `eoff[s]` is the element offset of slot s (0 for slots past H), `sval[s]` its validity.
template <int VPL>
__device__ __forceinline__ void rmsnorm_store(float (&r)[VPL][8], const int (&eoff)[VPL],
                                              const bool (&sval)[VPL], const uint16_t* gamma,
                                              uint16_t* out_row, int H, float eps, float* lds,
                                              int& parity, const RowMap& m) {
    constexpr int NP = next_pow2(VPL);
    float p[NP];
#pragma unroll
    for (int s = 0; s < NP; ++s) p[s] = 0.0f;
#pragma unroll
    for (int s = 0; s < VPL; ++s) p[s] = sval[s] ? sumsq8(r[s]) : 0.0f;
    float ss[1] = {tree_sum<NP>(p)};
    token_sum<1, wpt_max_for(VPL)>(ss, lds, parity, m);
    const float inv = 1.0f / __builtin_sqrtf(ss[0] / (float)H + eps);
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        const u32x4 g = *reinterpret_cast<const u32x4*>(gamma + eoff[s]);
        float gf[8];
        widen8(g, gf);
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = pack_bf16x2((r[s][2 * i] * inv) * gf[2 * i],
                               (r[s][2 * i + 1] * inv) * gf[2 * i + 1]);
        if (m.valid && sval[s]) st_stream(o, reinterpret_cast<u32x4*>(out_row + eoff[s]));
    }
}

}  // namespace mf
