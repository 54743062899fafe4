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
//  - One workgroup per token; its waves split the row into 1 KiB slots (row_norm.h) and keep
//    their part of the row in fp32 registers from the first FMA to the bf16 store, so the
//    residual is read once and written once and nothing is re-read.
//  - Gathers are 16-byte loads, a full contiguous 1 KiB per wave instruction.  A batch of
//    rows is issued in full before any of it is used; with the compile-time top-k (k = 8)
//    the token's indices and weights come in a few wide scalar loads, and the residual, gamma
//    and all k rows are then in flight at once, so a token costs the index loads and about
//    one more memory round trip.
//  - No MFMA: the arithmetic intensity is below 1 flop per byte; the kernel is bound by HBM.
//  - No atomics and a fixed reduction order: results are bit-deterministic and identical for
//    a token whatever batch it is in.
//
// Expert-parallel split (PR #6544 page, section 2.4: finalize + RMSNorm + all-reduce, the
// slots of non-local experts skipping normalisation; PR #4730 page, section 2: the
// all-reduce's sum fused with the residual add and RMSNorm):
//  - PARTIAL mode of moe_finalize_kernel: one GPU's share.  idx < 0 marks a slot whose expert
//    lives on another GPU; it is skipped (no row read, no norm, no FMA; the test is on a
//    wave-uniform scalar, so it is a branch, not a mask).  The fp32 accumulator is stored as
//    the token's partial; no residual, no norm.
//  - moe_finalize_combine_kernel: the token owner adds the ranks' partials in ascending rank
//    order from +0, then the residual add and the final RMSNorm as above.
#pragma once

#include "mx_device.h"
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
    uint8_t* q;                  // MXFP4 output: codes [T, H/2] (OUT_MX only)
    uint8_t* scales;             // MXFP4 output: scales [T, H/32] (OUT_MX only)
    int64_t T;
    int64_t num_rows;
    int32_t H;
    int32_t k;
    int32_t num_experts;
    float eps;
};

// Rows gathered per batch: up to 16 vectors per lane in flight (fewer for wider slices and
// for the per-expert variant, which also loads each row's expert gamma), at most the
// compile-time top-k.
constexpr int batch_rows(int vpl, int kc, bool per_expert) {
    const int vectors = per_expert ? (vpl == 1 && kc > 0 ? 8 : 4) : (vpl <= 2 ? 16 : 8);
    const int jb = vectors / vpl;
    const int j1 = jb < 1 ? 1 : (jb > 8 ? 8 : jb);
    return kc > 0 && j1 > kc ? kc : j1;
}

// Workgroup bound (16 waves; 8 for the per-expert variant) and the minimum waves per SIMD
// the register allocation must allow.  One slot per wave keeps the plain kernel within 64
// VGPRs, so two workgroups of 16 waves share a CU.
constexpr int finalize_block_max(bool per_expert) { return per_expert ? 512 : 1024; }
constexpr int finalize_min_waves(int vpl, bool per_expert) {
    return per_expert ? 2 : (vpl == 1 ? 8 : 4);
}

// The slot-serial kernel of wide rows: 8 waves per token, NL of each wave's VPL slots staged in
// LDS after the reduction area (16-byte aligned).
constexpr int kWideWaves = 8;
__host__ __device__ constexpr int wide_stage_offset(int wpt) {
    return (int(token_sum_lds_bytes(wpt, 1) / sizeof(float)) + 3) & ~3;
}
constexpr size_t wide_lds_bytes(int wpt, int nl) {
    return size_t(wide_stage_offset(wpt)) * sizeof(float) + size_t(wpt) * nl * kSlot * sizeof(float);
}

// One gather batch: JB rows (and, per-expert, their gamma rows) of the lane's slots; with
// SKIP, which of them are local (live).
template <int VPL, int JB, bool PER_EXPERT, bool SKIP = false>
struct GatherBatch {
    u32x4 x[JB][VPL];
    u32x4 g[PER_EXPERT ? JB : 1][VPL];
    bool live[SKIP ? JB : 1];
};

template <int VPL, int JB, bool PER_EXPERT, int TAIL, bool SKIP>
__device__ __forceinline__ void issue_batch(GatherBatch<VPL, JB, PER_EXPERT, SKIP>& b,
                                            const FinalizeArgs& a, int64_t tk, int jb, int k,
                                            const Slots<VPL, TAIL>& sl) {
    const int64_t last_row = a.num_rows - 1;
    // Every index of the batch first (one wide scalar load), then every row load: reading an
    // index right before its row's load serialises the index loads.
    // Past the last j of a partial batch, row k-1 is loaded again (same cache lines; unused).
    int32_t rid[JB], eid[PER_EXPERT ? JB : 1];
#pragma unroll
    for (int u = 0; u < JB; ++u) {
        rid[u] = a.idx[tk + min(jb + u, k - 1)];
        if constexpr (PER_EXPERT) eid[u] = a.eids[tk + min(jb + u, k - 1)];
    }
#pragma unroll
    for (int u = 0; u < JB; ++u) {
        int64_t row = rid[u];
        if constexpr (SKIP) {
            // another GPU's expert: nothing is read for it (a wave-uniform branch)
            b.live[u] = row >= 0;
            if (row < 0) {
#pragma unroll
                for (int s = 0; s < VPL; ++s) b.x[u][s] = u32x4{0u, 0u, 0u, 0u};
                if constexpr (PER_EXPERT) {
#pragma unroll
                    for (int s = 0; s < VPL; ++s) b.g[u][s] = u32x4{0u, 0u, 0u, 0u};
                }
                continue;
            }
        }
        row = row < 0 ? 0 : (row > last_row ? last_row : row);
        const uint16_t* rp = a.rows + row * a.H;
#pragma unroll
        for (int s = 0; s < VPL; ++s)
            b.x[u][s] = sl.suni[s] ? ld_stream(at<u32x4>(rp, sl.eoff[s] * 2u)) : u32x4{0u, 0u, 0u, 0u};
        if constexpr (PER_EXPERT) {
            int e = eid[u];
            e = e < 0 ? 0 : (e >= a.num_experts ? a.num_experts - 1 : e);
            const uint16_t* gp = a.egamma + (int64_t)e * a.H;
#pragma unroll
            for (int s = 0; s < VPL; ++s) b.g[u][s] = *at<u32x4>(gp, sl.eoff[s] * 2u);
        }
    }
}

// acc += w_j * row_j for the batch's rows in ascending j (per-expert: row_j normalised with
// its own mean square and multiplied by its expert's gamma first).
template <int VPL, int JB, bool PER_EXPERT, int TAIL, bool SKIP>
__device__ __forceinline__ void consume_batch(const GatherBatch<VPL, JB, PER_EXPERT, SKIP>& b,
                                              float (&acc)[VPL][8], const FinalizeArgs& a,
                                              int64_t tk, int jb, int k,
                                              const Slots<VPL, TAIL>& sl, TokenLds& L,
                                              const RowMap& m) {
    // Per-expert: the row's scale inv = (mean(x_j^2) + eps)^-1/2, and the row enters the sum as
    // fma(w_j * inv, x * gamma_e, acc): the product of two bf16 values is exact in fp32, so the
    // only roundings are the scale's, its product with the weight and the fma's.
    float inv[JB];
    if constexpr (PER_EXPERT) {
#pragma unroll
        for (int u = 0; u < JB; ++u) {
            float x[VPL][8];
#pragma unroll
            for (int s = 0; s < VPL; ++s) widen8(b.x[u][s], x[s]);
            inv[u] = lane_sumsq(x, sl);
        }
        token_sum<JB>(inv, L, m);
        const float inv_h = 1.0f / (float)a.H;
#pragma unroll
        for (int u = 0; u < JB; ++u) inv[u] = rms_scale(inv[u], inv_h, a.eps);
    }
#pragma unroll
    for (int u = 0; u < JB; ++u) {
        bool use = jb + u < k;
        if constexpr (SKIP) use = use && b.live[u];
        if (use) {
            // (a skipped slot's weight is never read)
            const float wj = PER_EXPERT ? a.w[tk + jb + u] * inv[u] : a.w[tk + jb + u];
#pragma unroll
            for (int s = 0; s < VPL; ++s) {
                float x[8];
                widen8(b.x[u][s], x);
                if constexpr (PER_EXPERT) {
                    float g[8];
                    widen8(b.g[u][s], g);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[s][i] = __builtin_fmaf(wj, x[i] * g[i], acc[s][i]);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[s][i] = __builtin_fmaf(wj, x[i], acc[s][i]);
                }
            }
        }
    }
}

// KC: the top-k fixed at compile time (8), or 0 for a runtime k.  PARTIAL: this GPU's share
// of the expert-parallel split (slots with idx < 0 skipped; the fp32 accumulator is stored to
// residual_out, which then holds the [T, H] partial; residual, gamma and out are unused).
// OUT_MX: the MXFP4 epilogue: the normalised output is quantised to MXFP4 (q, scales) instead
// of rounded to bf16 (page "FlashInfer: fused norms and TP/EP MoE for Muse-Spark-Open",
// PR #6544, section 2.3: RMSNorm + block-scaled FP4 quantisation; the OCP MXFP4 format).
template <int VPL, int KC, bool PER_EXPERT, int TAIL, bool PARTIAL = false, bool OUT_MX = false>
__global__ void __launch_bounds__(finalize_block_max(PER_EXPERT))
__attribute__((amdgpu_waves_per_eu(OUT_MX && KC == 0 ? (VPL == 1 ? 6 : 4)
                                                     : finalize_min_waves(VPL, PER_EXPERT), 8)))
moe_finalize_kernel(const FinalizeArgs a) {
    // (the MXFP4 epilogue keeps its store addresses live across the loop: with two or more
    // slots and a runtime k, half the batch keeps it out of scratch)
    constexpr int JB = OUT_MX && VPL >= 2 && KC == 0 ? (batch_rows(VPL, KC, PER_EXPERT) + 1) / 2
                                                     : batch_rows(VPL, KC, PER_EXPERT);
    // With small row slices the residual and gamma ride along with the first batch.
    constexpr bool EARLY = VPL <= 2;
    extern __shared__ float lds[];

    const RowMap m = row_map();
    const int H = a.H;
    const int k = KC > 0 ? KC : a.k;
    const Slots<VPL, TAIL> sl = slot_offsets<VPL, TAIL>(m, H);
    const int64_t tk = m.t * k;
    const float* res = a.residual + m.t * H;

    float acc[VPL][8];
#pragma unroll
    for (int s = 0; s < VPL; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[s][i] = 0.0f;
    f32x4 rv[VPL][2];
    u32x4 g[VPL];
    auto load_res_gamma = [&]() {
#pragma unroll
        for (int s = 0; s < VPL; ++s) {
            rv[s][0] = ld_stream(at<f32x4>(res, sl.eoff[s] * 4u));
            rv[s][1] = ld_stream(at<f32x4>(res, sl.eoff[s] * 4u + 16u));
        }
        load_gamma(g, a.gamma, sl);
    };

    TokenLds L = token_lds(lds, m.wpt, PER_EXPERT ? JB : 1);
    // The residual and gamma do not depend on the indices: in flight while they arrive.
    if (!PARTIAL && EARLY) load_res_gamma();
    constexpr int UNROLL = KC > 0 ? (KC + JB - 1) / JB : 1;
#pragma unroll UNROLL
    for (int jb = 0; jb < k; jb += JB) {
        GatherBatch<VPL, JB, PER_EXPERT, PARTIAL> b;
        issue_batch(b, a, tk, jb, k, sl);
        consume_batch(b, acc, a, tk, jb, k, sl, L, m);
    }
    if constexpr (PARTIAL) {
        // the token's partial, written like the residual (contiguous 1 KiB per store
        // instruction, nontemporal): measured 6% faster than direct stores of the lanes' halves
        store_residual(acc, sl, m, H, a.residual_out + m.t * H);
        return;
    }
    if (!EARLY) load_res_gamma();

    // Residual add (one fp32 add after the k-term sum), then the store of the updated
    // residual.  Every residual load precedes every residual_out store in program order, so
    // the in-place case (residual_out == residual) never orders a load behind a store.
#pragma unroll
    for (int s = 0; s < VPL; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[s][i] = rv[s][0][i] + acc[s][i];
            acc[s][4 + i] = rv[s][1][i] + acc[s][4 + i];
        }
    store_residual(acc, sl, m, H, a.residual_out + m.t * H);
    if constexpr (OUT_MX) {
        float ss[1] = {lane_sumsq(acc, sl)};
        token_sum<1>(ss, L, m);
        const float inv = rms_scale(ss[0], 1.0f / (float)H, a.eps);
        mx_store_normed(acc, g, sl, inv, m.lane, a.q + m.t * (H / 2), a.scales + m.t * (H / 32));
    } else {
        rmsnorm_store(acc, g, sl, a.out + m.t * H, H, a.eps, L, m);
    }
}

// Wide rows (several 512-value slots per wave, compile-time top-k of at most 8): the same
// arithmetic as moe_finalize_kernel, with the gather run slot by slot.  A slot's k rows and its
// residual are loaded together, and the next slot's are issued before this slot's are summed, so
// two slots' rows are in flight while only the finished fp32 values of earlier slots wait for
// the norm.  Per slot the rows are summed in ascending j and the lane's sum of squares runs over
// its slots in order, exactly as there: on the same launch shape the results are bit-identical to
// it.  Measured on MI355X at 3 and 5 slots (8 waves, T = 4096-8192, k = 8, cold): H = 12288 77.3%
// of 8 TB/s (77.6% for moe_finalize_kernel), H = 20480 74.5% (72.4%).  Not taken: 4-row batches
// with a 64-VGPR cap for two 16-wave workgroups per CU (spills; 34-62%), per-slot residual stores
// (1-3% slower), and a persistent form whose lookahead crosses into the next token (spills at
// every width).
//
// The finished fp32 row waits in registers for the norm: 8 values per slot and lane, 64 at
// H = 32768 with 8 waves, more than the registers of two workgroups per CU allow.  So the first NL
// slots of each wave wait in LDS instead (2 KiB per slot and wave, lane-major: each 16-byte access
// of a wave is 1 KiB contiguous, free of bank conflicts) and are read back for the residual store
// and the norm; only the last VPL - NL stay in VGPRs.  At 6 to 8 slots per wave three are staged
// (52 KiB per workgroup): two 8-wave workgroups per CU, no spills.
// Measured on MI355X (T = 4096, k = 8, cold; one GPU, interleaved rounds, every variant writing
// the same output buffers):
//  - equal within noise to 16 waves of 4 or 3 slots in registers: 71.9% against 72.1% of 8 TB/s at
//    H = 32768, 72.1% against 72.3% at 24576; at 28672 71.9% against 71.3% for moe_finalize_kernel.
//  - Not taken: staging at 5 slots for three workgroups per CU at H = 20480 (70.1% against 73.9%),
//    one staged slot at H = 12288 (71.9% against 77.2%): capped at 80 VGPRs, the waves keep fewer
//    loads in flight.  Slots interleaved across waves (s * 8 + w, so that the workgroup reads 8 KiB
//    of each row contiguously at each step): 70.5% at H = 32768.  The residual's loads issued
//    ahead of the rows': within 0.5% either way.
//
// Every residual load of the token precedes its residual_out stores: the in-place case is safe.
template <int VPL, int NL, int KC>
__global__ void __launch_bounds__(kWideWaves * kWave) __attribute__((amdgpu_waves_per_eu(4, 8)))
moe_finalize_wide_kernel(const FinalizeArgs a) {
    static_assert(KC > 0 && KC <= 8, "one batch of rows per slot");
    static_assert(NL >= 0 && NL < VPL, "at least one slot stays in registers");
    constexpr int TAIL = kRowFull;
    constexpr int NREG = VPL - NL;
    extern __shared__ float lds[];
    const RowMap m = row_map();
    const int H = a.H;
    const Slots<VPL, TAIL> sl = slot_offsets<VPL, TAIL>(m, H);
    const int64_t tk = m.t * KC;
    const float* res = a.residual + m.t * H;
    TokenLds L = token_lds(lds, m.wpt, 1);
    // this lane's staged values: slot s, half h at stage[(s * 2 + h) * 64]
    f32x4* stage = reinterpret_cast<f32x4*>(lds + wide_stage_offset(m.wpt)) +
                   m.wave * NL * 2 * kWave + m.lane;

    auto slot_of = [&](int s) {
        Slots<1, TAIL> one;
        one.eoff[0] = sl.eoff[s];
        one.sval[0] = sl.sval[s];
        one.suni[0] = sl.suni[s];
        return one;
    };
    auto staged = [&](int s, float (&v)[8]) {
        const f32x4 lo = stage[(s * 2) * kWave], hi = stage[(s * 2 + 1) * kWave];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = lo[i];
            v[4 + i] = hi[i];
        }
    };
    float r[NREG][8];
    float lane_ss = 0.0f;   // the lane's sum of squares, its slots in order
    f32x4 rv[2][2];
    GatherBatch<1, KC, false> b[2];
    auto issue = [&](int buf, int s) {
        issue_batch(b[buf], a, tk, 0, KC, slot_of(s));
        rv[buf][0] = ld_stream(at<f32x4>(res, sl.eoff[s] * 4u));
        rv[buf][1] = ld_stream(at<f32x4>(res, sl.eoff[s] * 4u + 16u));
    };
    issue(0, 0);
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        if (s + 1 < VPL) issue((s + 1) & 1, s + 1);
        float acc[1][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[0][i] = 0.0f;
        consume_batch(b[s & 1], acc, a, tk, 0, KC, slot_of(s), L, m);
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = rv[s & 1][0][i] + acc[0][i];
            v[4 + i] = rv[s & 1][1][i] + acc[0][4 + i];
        }
        if (s < NL) {
            lane_ss += sumsq8(v);
            stage[(s * 2) * kWave] = f32x4{v[0], v[1], v[2], v[3]};
            stage[(s * 2 + 1) * kWave] = f32x4{v[4], v[5], v[6], v[7]};
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) r[s - NL][i] = v[i];
        }
    }
    u32x4 g[VPL];
    load_gamma(g, a.gamma, sl);
    float* res_out = a.residual_out + m.t * H;
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        if (s < NL) {
            float v[8];
            staged(s, v);
            store_residual_slot<TAIL>(v, m.wave * VPL + s, m, H, res_out);
        } else {
            store_residual_slot<TAIL>(r[s - NL], m.wave * VPL + s, m, H, res_out);
        }
    }
#pragma unroll
    for (int s = 0; s < NREG; ++s) lane_ss += sumsq8(r[s]);
    float ss[1] = {lane_ss};
    token_sum<1>(ss, L, m);
    const float inv = rms_scale(ss[0], 1.0f / (float)H, a.eps);
    uint16_t* out_row = a.out + m.t * H;
#pragma unroll
    for (int s = 0; s < VPL; ++s) {
        uint16_t* dst = at<uint16_t>(out_row, sl.eoff[s] * 2u);
        if (s < NL) {
            float v[8];
            staged(s, v);
            norm_store_slot(v, g[s], inv, dst);
        } else {
            norm_store_slot(r[s - NL], g[s], inv, dst);
        }
    }
}

// The token owner's combine of the expert-parallel split.
struct CombineArgs {
    const float* partials;   // [G, T, H]: rank g's partial of token t at (g*T + t)*H
    const float* residual;   // [T, H]
    float* residual_out;     // [T, H], may equal residual
    const uint16_t* gamma;   // bf16 [H]
    uint16_t* out;           // bf16 [T, H]
    int64_t T;
    int32_t H;
    int32_t G;
    float eps;
};

// Ranks whose partial rows are in flight together: 32 fp32 values per lane, so that two
// 16-wave workgroups fit on a CU at one slot per wave.
constexpr int combine_batch(int vpl) { return vpl == 1 ? 4 : (vpl == 2 ? 2 : 1); }

template <int VPL, int TAIL>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(VPL == 1 ? 8 : 4, 8)))
moe_finalize_combine_kernel(const CombineArgs a) {
    constexpr int kCombineBatch = combine_batch(VPL);
    extern __shared__ float lds[];
    const RowMap m = row_map();
    const int H = a.H;
    const Slots<VPL, TAIL> sl = slot_offsets<VPL, TAIL>(m, H);
    const int64_t row = m.t * H;
    const int64_t rank_stride = a.T * H;

    float acc[VPL][8];
#pragma unroll
    for (int s = 0; s < VPL; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[s][i] = 0.0f;
    f32x4 rv[VPL][2];
    u32x4 g[VPL];
    auto load_res_gamma = [&]() {
#pragma unroll
        for (int s = 0; s < VPL; ++s) {
            rv[s][0] = ld_stream(at<f32x4>(a.residual + row, sl.eoff[s] * 4u));
            rv[s][1] = ld_stream(at<f32x4>(a.residual + row, sl.eoff[s] * 4u + 16u));
        }
        load_gamma(g, a.gamma, sl);
    };
    // With small row slices the residual and gamma ride along with the first ranks.
    constexpr bool EARLY = VPL <= 2;
    // Rotating pipeline over the ranks: rank g sits in buffer g % B, and as soon as a buffer has
    // been added into the sum it is reloaded with the rank B further on, so B ranks stay in
    // flight throughout (measured 2% faster than loading B ranks, adding them, then loading the
    // next B).  The default cache policy measured 12% faster than nontemporal loads here.
    constexpr int B = kCombineBatch;
    f32x4 p[B][VPL][2];
    auto issue = [&](int u, int gr) {
        const float* pr = a.partials + gr * rank_stride + row;
#pragma unroll
        for (int s = 0; s < VPL; ++s) {
            p[u][s][0] = *at<f32x4>(pr, sl.eoff[s] * 4u);
            p[u][s][1] = *at<f32x4>(pr, sl.eoff[s] * 4u + 16u);
        }
    };
    // A wave whose first slot lies past the row (a spare wave) loads nothing.  A slot past the
    // row in a live wave reads the row's first values (eoff = 0) and is never stored or summed.
    const bool live = sl.suni[0];
    if (live) {
#pragma unroll
        for (int u = 0; u < B; ++u) issue(u, u < a.G ? u : a.G - 1);
    }
    if (EARLY) load_res_gamma();
    if (live) {
        // ascending rank order: acc = acc + partial_g
        for (int g0 = 0; g0 < a.G; g0 += B) {
#pragma unroll
            for (int u = 0; u < B; ++u) {
                if (g0 + u < a.G) {
#pragma unroll
                    for (int s = 0; s < VPL; ++s)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[s][i] = acc[s][i] + p[u][s][0][i];
                            acc[s][4 + i] = acc[s][4 + i] + p[u][s][1][i];
                        }
                }
                if (g0 + B + u < a.G) issue(u, g0 + B + u);
            }
        }
    }
    if (!EARLY) load_res_gamma();
    // residual add, then the store (every residual load precedes it: in-place is safe)
#pragma unroll
    for (int s = 0; s < VPL; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[s][i] = rv[s][0][i] + acc[s][i];
            acc[s][4 + i] = rv[s][1][i] + acc[s][4 + i];
        }
    store_residual(acc, sl, m, H, a.residual_out + row);
    TokenLds L = token_lds(lds, m.wpt, 1);
    rmsnorm_store<true>(acc, g, sl, a.out + row, H, a.eps, L, m);
}

}  // namespace mf
