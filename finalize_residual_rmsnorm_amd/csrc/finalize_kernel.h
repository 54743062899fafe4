// MoE finalize fused with the residual add and RMSNorm, for gfx950.
//
// What it computes (page "FlashInfer MoE performance: improving the deterministic finalize
// with CuTe DSL", PR #5319, section 1; page "FlashInfer: fused norms and TP/EP MoE for
// Muse-Spark-Open", PR #6544, sections 2.1 and 2.4; page "MoE all-reduce fusion for
// Blackwell: FlashInfer's Cake backend", PR #4730, section 2, fusion strategy): per token,
// gather its k rows of the permuted GEMM2 output, optionally RMSNorm each row with its
// expert's gamma, accumulate w_j * row_j with fp32 FMAs in ascending j from +0, add the fp32
// residual, store it, and emit bf16(RMSNorm(residual_out) * gamma).
//
// How it maps onto CDNA4 (the pages' kernels are CuTe-DSL / cluster designs for other
// hardware; none of that carries over):
//  - One token row per `wpt` wavefronts (wpt = 1 when there are enough tokens to fill the
//    chip); each lane keeps its slice of the row in fp32 registers from the first FMA to the
//    bf16 store, so the residual is read once and written once, and nothing is re-read.
//  - Gathers are 16-byte loads, a full 1 KiB per wave instruction, contiguous within a row.
//    All loads of a batch of JB rows are issued before any is consumed (JB * VPL vectors in
//    flight per lane).
//  - The token's idx / weight / expert id are wave-uniform scalar loads.
//  - No MFMA: the arithmetic intensity is below 1 flop per byte; the kernel is bound by HBM.
//  - No atomics and a fixed reduction tree: results are bit-deterministic and do not depend
//    on the launch shape.
#pragma once

#include "row_norm.h"

namespace mf {

struct FinalizeArgs {
    const uint16_t* rows;        // bf16 [num_rows, H]
    const int32_t* idx;          // [T, k]
    const float* w;              // [T, k]
    const int32_t* eids;         // [T, k] or null
    const uint16_t* egamma;      // bf16 [E, H] or null
    const float* residual;       // [T, H]
    float* residual_out;         // [T, H], may equal residual
    const uint16_t* gamma;       // bf16 [H]
    uint16_t* out;               // bf16 [T, H]
    int64_t T;
    int64_t num_rows;
    int32_t H;
    int32_t k;
    int32_t num_experts;
    int32_t wpt;                 // waves per token (power of two)
    int32_t spw;                 // slots per wave
    float eps;
};

// Rows per gather batch: enough 16-byte loads in flight per lane without spilling.  The
// per-expert variant also holds the batch's gamma rows, so it batches less at larger VPL.
constexpr int gather_batch_for(int vpl, bool per_expert) {
    return vpl >= 8 ? 1 : (vpl >= 4 ? (per_expert ? 1 : 2) : (vpl >= 2 ? 4 : 8));
}

// The per-expert variant is launched with at most 8 waves per token (512 threads).
constexpr int finalize_block_max(int vpl, bool per_expert) {
    return per_expert && block_max_for(vpl) > 512 ? 512 : block_max_for(vpl);
}

template <int VPL, bool PER_EXPERT>
__global__ void __launch_bounds__(finalize_block_max(VPL, PER_EXPERT))
moe_finalize_kernel(const FinalizeArgs a) {
    constexpr int JB = gather_batch_for(VPL, PER_EXPERT);
    constexpr int NP = next_pow2(VPL);
    constexpr int WPT_MAX = wpt_max_for(VPL);
    extern __shared__ float lds[];

    const RowMap m = row_map(a.T, a.wpt);
    if (a.wpt == 1 && !m.valid) return;  // no barriers when wpt == 1

    const int H = a.H;
    int eoff[VPL];
    bool sval[VPL];
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        const int e = (m.wit * a.spw + s) * kSlot + m.lane * kVec;
        sval[s] = e < H;
        eoff[s] = sval[s] ? e : 0;
    }

    const int64_t tk = m.t * a.k;
    const int64_t last_row = a.num_rows - 1;
    float acc[VPL][8];
#pragma unroll
    for (int s = 0; s < VPL; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[s][i] = 0.0f;

    int parity = 0;
    for (int jb = 0; jb < a.k; jb += JB) {
        u32x4 xv[JB][VPL];
#pragma unroll
        for (int u = 0; u < JB; ++u) {
            // Past the last j of a partial batch, reload row k-1 (same cache lines; unused).
            const int j = min(jb + u, a.k - 1);
            int64_t row = a.idx[tk + j];
            row = row < 0 ? 0 : (row > last_row ? last_row : row);
            const uint16_t* rp = a.rows + row * H;
#pragma unroll
            for (int s = 0; s < VPL; ++s)
                xv[u][s] = ld_stream(reinterpret_cast<const u32x4*>(rp + eoff[s]));
        }
        if constexpr (PER_EXPERT) {
            // RMSNorm of each gathered row with its expert's gamma, before the weighted sum.
            u32x4 gv[JB][VPL];
            float ps[JB];
#pragma unroll
            for (int u = 0; u < JB; ++u) {
                const int j = min(jb + u, a.k - 1);
                int e = a.eids[tk + j];
                e = e < 0 ? 0 : (e >= a.num_experts ? a.num_experts - 1 : e);
                const uint16_t* gp = a.egamma + (int64_t)e * H;
#pragma unroll
                for (int s = 0; s < VPL; ++s)
                    gv[u][s] = *reinterpret_cast<const u32x4*>(gp + eoff[s]);
                float p[NP];
#pragma unroll
                for (int s = 0; s < NP; ++s) p[s] = 0.0f;
#pragma unroll
                for (int s = 0; s < VPL; ++s) {
                    float x[8];
                    widen8(xv[u][s], x);
                    p[s] = sval[s] ? sumsq8(x) : 0.0f;
                }
                ps[u] = tree_sum<NP>(p);
            }
            token_sum<JB, WPT_MAX>(ps, lds, parity, m);
#pragma unroll
            for (int u = 0; u < JB; ++u) {
                if (jb + u < a.k) {
                    const float inv = 1.0f / __builtin_sqrtf(ps[u] / (float)H + a.eps);
                    const float wj = a.w[tk + jb + u];
#pragma unroll
                    for (int s = 0; s < VPL; ++s) {
                        float x[8], g[8];
                        widen8(xv[u][s], x);
                        widen8(gv[u][s], g);
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            acc[s][i] = __builtin_fmaf(wj, (x[i] * inv) * g[i], acc[s][i]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < JB; ++u) {
                if (jb + u < a.k) {
                    const float wj = a.w[tk + jb + u];
#pragma unroll
                    for (int s = 0; s < VPL; ++s) {
                        float x[8];
                        widen8(xv[u][s], x);
#pragma unroll
                        for (int i = 0; i < 8; ++i) acc[s][i] = __builtin_fmaf(wj, x[i], acc[s][i]);
                    }
                }
            }
        }
    }

    // Residual add (one fp32 add after the k-term sum), then the store of the updated
    // residual.  Every residual load precedes every residual_out store in program order, so
    // the in-place case (residual_out == residual) never orders a load behind a store.
    const float* res = a.residual + m.t * H;
    float* res_out = a.residual_out + m.t * H;
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        const f32x4 r0 = ld_stream(reinterpret_cast<const f32x4*>(res + eoff[s]));
        const f32x4 r1 = ld_stream(reinterpret_cast<const f32x4*>(res + eoff[s] + 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[s][i] = r0[i] + acc[s][i];
            acc[s][4 + i] = r1[i] + acc[s][4 + i];
        }
    }
    if (m.valid) {
#pragma unroll
        for (int s = 0; s < VPL; ++s) {
            if (sval[s]) {
                st_stream(f32x4{acc[s][0], acc[s][1], acc[s][2], acc[s][3]},
                          reinterpret_cast<f32x4*>(res_out + eoff[s]));
                st_stream(f32x4{acc[s][4], acc[s][5], acc[s][6], acc[s][7]},
                          reinterpret_cast<f32x4*>(res_out + eoff[s] + 4));
            }
        }
    }

    rmsnorm_store<VPL>(acc, eoff, sval, a.gamma, a.out + m.t * H, H, a.eps, lds, parity, m);
}

}  // namespace mf
