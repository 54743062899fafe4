// MoE routing and the expert-sorted permutation on gfx950: the producer of the finalize's
// gather indices and weights.
//
// For T tokens with router logits [T, E] (fp32):
//   expert_ids[t, j]  the experts of the k largest logits, largest first; among equal logits
//                     the lower expert id first
//   weights[t, j]     softmax over those k logits: exp(l_j - l_0) / sum_i exp(l_i - l_0), the
//                     sum taken in j order (fp32)
//   offsets[e]        slots routed to experts below e, offsets[E] = T*k: the per-expert row
//                     ranges of the grouped GEMM (its m_indptr / token_offset argument, page
//                     "FlashInfer: fused kernels and an optimised scheduler for MoE" (PR #4130),
//                     code analysis items 1 and 2)
//   perm[p]           the slot s = t*k + j stored at permuted row p: rows grouped by expert,
//                     slots ascending within an expert (a stable sort of the slots by expert)
//   idx[t, j]         the permuted row of slot (t, j), idx[perm[p]] = p: what the finalize
//                     gathers with
//
// Three launches:
//  1. route_select_kernel: one wave per run of `tpw` consecutive tokens, 16 waves per block.
//     Top-k in k rounds over the order-preserving 32-bit image of the logits, each round a
//     wave-wide maximum (DPP max within rows of 16 lanes, then across the four rows) and an
//     exact tie-break to the lowest expert id: up to 4 logits per lane (E <= 256), every lane
//     keeps its logits sorted and a round pops the head of the lowest lane holding the maximum;
//     beyond that, a ballot per logit register finds the lowest id, whose logit is retired; the
//     softmax; then each wave ranks its own slots (contiguous, in
//     slot order) by expert in 64-slot chunks: a slot's rank among the earlier slots of its chunk with the same
//     expert comes from ballots over the bits of the expert id (the ballot / prefix-count
//     technique of the PR #4130 page's warp-cooperative scheduler, "why is this good" item 2),
//     added to the wave's running per-expert count in LDS.  The waves' counts are scanned in
//     wave order; the workspace receives the block's per-expert counts, and at the very end
//     expert_ids, weights and idx (each slot's rank within its block) are stored, coalesced.
//  2. route_scan_kernel: per expert, the exclusive scan of the block counts over the blocks
//     (in place) and the expert's total.
//  3. route_scatter_kernel: one thread per expert: offsets = exclusive scan of the totals over
//     the experts, and a per-block LDS table offsets[e] + block prefix[e]; then for every slot
//     p = table[e] + rank: idx[s] = p, perm[p] = s.
// Small calls (decode sizes) replace kernels 2 and 3 by route_finish_kernel, one workgroup that
// does both: two launches instead of three.
// Everything but the weights is integer work, exact and independent of the launch shape.
#pragma once

#include "mf_device.h"

namespace mf {

struct RouteArgs {
    const float* logits;   // [T, E]
    int32_t* expert_ids;   // [T, k]
    float* weights;        // [T, k]
    int32_t* idx;          // [T, k]: rank within the block after kernel 1, the row after kernel 3
    int32_t* perm;         // [T*k]
    int32_t* offsets;      // [E + 1]
    int32_t* counts;       // workspace [nblocks, E]: block counts, then their prefix over blocks
    int32_t* totals;       // workspace [E]
    int64_t T;
    int32_t E;
    int32_t k;
    int32_t tpw;           // tokens per wave in kernel 1 (tpw * k <= kRouteSlotsPerWave)
    int32_t nblocks;       // blocks of kRouteWaves * tpw tokens
    int32_t id_bits;       // 2^id_bits >= E
};

constexpr int kRouteMaxK = 16;
constexpr int kRouteMaxE = 1024;
constexpr int kRouteWaves = 16;          // waves per block of kernels 1 and 2
constexpr int kRouteSlotsPerWave = 256;  // 4 chunks of 64 slots
constexpr int kRouteChunks = kRouteSlotsPerWave / kWave;
constexpr int kRouteScatterThreads = kRouteMaxE;  // one thread per expert
constexpr int kRouteScatterSlots = kRouteWaves * kRouteSlotsPerWave / kRouteScatterThreads;

// LDS of kernel 1: the wave's weights in slot order (fp32), then per-wave per-expert counts and
// the wave's expert ids in slot order (both 16-bit: a wave holds at most 256 slots and a block
// 4096).
constexpr size_t route_select_lds_bytes(int E) {
    return size_t(kRouteWaves) * kRouteSlotsPerWave * sizeof(float) +
           size_t(kRouteWaves) * (E + kRouteSlotsPerWave) * sizeof(uint16_t);
}

// Orders the program-order LDS accesses of one wave's lanes (no hardware wait needed:
// a wave's LDS instructions complete in order).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Order-preserving map of a float to uint32 (-0 is taken as +0, so it ties with +0).  Every
// non-NaN value maps to 1 or more (the one NaN pattern that would map to 0 is raised to 1), so
// 0 can mark "no expert": retired logits and lanes past E.
__device__ __forceinline__ uint32_t ordered_bits(float v) {
    const uint32_t b = __float_as_uint(v + 0.0f);
    const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return o > 1u ? o : 1u;
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Maximum over the 64 lanes (every lane active), wave-uniform: within each row of 16 lanes
// through DPP (quad swaps, half-row mirror, row mirror), then across the rows with the row
// broadcasts (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3), leaving the maximum in
// lane 63.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_rows_u32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROWS, 0xF, false));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = umax(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
    v = umax(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
    v = umax(v, dpp_u32<0x141>(v));  // row_half_mirror
    v = umax(v, dpp_u32<0x140>(v));  // row_mirror
    v = umax(v, dpp_rows_u32<0x142, 0xA>(v));  // row_bcast:15 (disabled rows take 0: no change)
    v = umax(v, dpp_rows_u32<0x143, 0xC>(v));  // row_bcast:31
    return __builtin_amdgcn_readlane(v, kWave - 1);
}

// Logits of one token.  LANE_MAJOR: lane l holds experts l*EPL + q; otherwise experts q*64 + l.
// The loads are unconditional (experts past E read expert E-1 and their value is ignored): with
// no branch around them the compiler can wait for exactly the loads a use needs, so the next
// token's loads stay in flight.
// VEC (lane-major, E a multiple of EPL, rows aligned to EPL floats): one EPL-wide load per lane,
// lanes past E reading the last group.
template <int EPL, bool LANE_MAJOR, bool VEC>
__device__ __forceinline__ void load_logits(float (&x)[EPL], const float* row, int E, int lane) {
    if constexpr (VEC && EPL == 4) {
        const int g = lane * 4 < E ? lane : E / 4 - 1;
        const f32x4 v = ld_stream(reinterpret_cast<const f32x4*>(row) + g);
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = v[q];
    } else if constexpr (VEC && EPL == 2) {
        const int g = lane * 2 < E ? lane : E / 2 - 1;
        const f32x2 v = ld_stream(reinterpret_cast<const f32x2*>(row) + g);
        x[0] = v[0];
        x[1] = v[1];
    } else {
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            const int e = LANE_MAJOR ? lane * EPL + q : q * kWave + lane;
            x[q] = ld_stream(row + (e < E ? e : E - 1));
        }
    }
}

// Largest number of logits per lane that the sorted selection handles (sorting more per lane
// costs more than it saves).
constexpr int kSortedMaxEpl = 4;

// Top-k with experts laid out lane-major (lane l holds l*EPL .. l*EPL + EPL-1).  Each lane sorts
// its logits once, largest first and equal logits by lower expert id; a round is then the wave
// maximum of the lanes' heads, the lowest lane whose head holds it (a ballot: lanes hold
// ascending id ranges, and a lane's head is its lowest id with that value), that head's id, and
// a pop of that lane's list.  Exact and tie-correct, like the strided form below, with a fraction
// of its scalar work per round.  Lane j < k receives selection j.
template <int EPL>
__device__ __forceinline__ void select_sorted(const float (&x)[EPL], int lane, int E, int k,
                                              int& my_e, float& my_v, float& top) {
    uint32_t s[EPL], my_o = 0, top_o = 0;
    int sq[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
        s[q] = lane * EPL + q < E ? ordered_bits(x[q]) : 0u;  // 0: no expert
        sq[q] = q;
    }
    // sorting network on (value descending, position ascending): a total order, so the
    // network's result is the sorted list whatever the order of its exchanges
    auto cx = [&](int i, int j) {
        const bool sw = s[j] > s[i] || (s[j] == s[i] && sq[j] < sq[i]);
        const uint32_t si = s[i], sj = s[j];
        const int qi = sq[i], qj = sq[j];
        s[i] = sw ? sj : si;
        s[j] = sw ? si : sj;
        sq[i] = sw ? qj : qi;
        sq[j] = sw ? qi : qj;
    };
    if constexpr (EPL == 2) cx(0, 1);
    if constexpr (EPL == 4) {
        cx(0, 1);
        cx(2, 3);
        cx(0, 2);
        cx(1, 3);
        cx(1, 2);
    }
#pragma unroll
    for (int j = 0; j < kRouteMaxK; ++j) {
        if (j < k) {
            // m >= 1: k <= E leaves an unretired expert in every round
            const uint32_t m = wave_max_u32(s[0]);
            const int wl = __builtin_ctzll(__builtin_amdgcn_ballot_w64(s[0] == m));
            const int e = wl * EPL + __builtin_amdgcn_readlane(sq[0], wl);
            const bool mine = lane == wl;
#pragma unroll
            for (int q = 0; q + 1 < EPL; ++q) {
                s[q] = mine ? s[q + 1] : s[q];
                sq[q] = mine ? sq[q + 1] : sq[q];
            }
            s[EPL - 1] = mine ? 0u : s[EPL - 1];
            if (j == 0) top_o = m;
            if (lane == j) {
                my_e = e;
                my_o = m;
            }
        }
    }
    my_v = from_ordered_bits(my_o);
    top = from_ordered_bits(top_o);
}

// Top-k with experts strided over the lanes (lane l holds experts q*64 + l): each round takes
// the wave maximum of the lanes' maxima, then one ballot per logit register finds the lowest
// expert id holding it (the first register with a match, then its lowest lane), which is
// retired.  Used where a lane holds too many logits to sort.
template <int EPL>
__device__ __forceinline__ void select_strided(const float (&x)[EPL], int lane, int E, int k,
                                               int& my_e, float& my_v, float& top) {
    uint32_t o[EPL], my_o = 0, top_o = 0;
#pragma unroll
    for (int q = 0; q < EPL; ++q) o[q] = q * kWave + lane < E ? ordered_bits(x[q]) : 0u;
#pragma unroll
    for (int j = 0; j < kRouteMaxK; ++j) {
        if (j < k) {
            uint32_t lm = o[0];
#pragma unroll
            for (int q = 1; q < EPL; ++q) lm = umax(lm, o[q]);
            const uint32_t m = wave_max_u32(lm);
            int wq = 0;
            uint64_t hit = 0;
#pragma unroll
            for (int q = EPL - 1; q >= 0; --q) {
                const uint64_t bq = __builtin_amdgcn_ballot_w64(o[q] == m);
                if (bq) {
                    wq = q;
                    hit = bq;
                }
            }
            const int wl = __builtin_ctzll(hit);
#pragma unroll
            for (int q = 0; q < EPL; ++q)
                if (q == wq && lane == wl) o[q] = 0u;  // retired
            if (j == 0) top_o = m;
            if (lane == j) {
                my_e = wq * kWave + wl;
                my_o = m;
            }
        }
    }
    my_v = from_ordered_bits(my_o);
    top = from_ordered_bits(top_o);
}

// One token's top-k and softmax over its logits x (laid out for EPL): lane j < k receives the
// j-th expert and its weight exp(l_j - l_0) / sum_i exp(l_i - l_0) (fp32, the sum in j order).
template <int EPL>
__device__ __forceinline__ void route_token(const float (&x)[EPL], int lane, int E, int k,
                                            int& my_e, float& w) {
    float my_v = 0.0f, top = 0.0f;
    my_e = 0;
    if constexpr (EPL <= kSortedMaxEpl) select_sorted<EPL>(x, lane, E, k, my_e, my_v, top);
    else select_strided<EPL>(x, lane, E, k, my_e, my_v, top);
    const float ex = expf(my_v - top);
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
    w = ex / sum;
}

// EPL: logits per lane, E <= 64 * EPL.  VEC: vector loads of the logits (see load_logits).
template <int EPL, bool VEC>
__global__ void __launch_bounds__(kRouteWaves * kWave) route_select_kernel(const RouteArgs a) {
    extern __shared__ float route_lds_f[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int E = a.E, k = a.k;
    float* wstage = route_lds_f + wave * kRouteSlotsPerWave;       // [kRouteWaves][256] weights
    uint16_t* route_lds = reinterpret_cast<uint16_t*>(route_lds_f + kRouteWaves * kRouteSlotsPerWave);
    uint16_t* cnt = route_lds;                                     // [kRouteWaves][E]
    uint16_t* mycnt = cnt + wave * E;
    uint16_t* stage = route_lds + kRouteWaves * E + wave * kRouteSlotsPerWave;

    const int64_t tw0 = (int64_t(blockIdx.x) * kRouteWaves + wave) * a.tpw;
    const int ntok = a.T - tw0 <= 0 ? 0 : (a.T - tw0 < a.tpw ? int(a.T - tw0) : a.tpw);
    for (int e = lane; e < E; e += kWave) mycnt[e] = 0;

    // --- top-k and softmax, one token at a time; the next token's logits are in flight ---
    // The results are staged in LDS and stored at the end of the kernel: a global store inside
    // the loop (under lane < k) made every iteration's wait for the next logits also wait for
    // the previous token's stores to complete (loads and stores share one counter on gfx950).
    constexpr bool kLaneMajor = EPL <= kSortedMaxEpl;
    float x[EPL], xn[EPL];
    if (ntok > 0) load_logits<EPL, kLaneMajor, VEC>(x, a.logits + tw0 * E, E, lane);
    for (int i = 0; i < ntok; ++i) {
        const int64_t t = tw0 + i;
        // the next token's logits (the last token re-reads its own row: no branch, in bounds)
        load_logits<EPL, kLaneMajor, VEC>(xn, a.logits + (i + 1 < ntok ? t + 1 : t) * E, E, lane);
        int my_e;
        float w;
        route_token<EPL>(x, lane, E, k, my_e, w);
        if (lane < k) {
            wstage[i * k + lane] = w;
            stage[i * k + lane] = uint16_t(my_e);
        }
#pragma unroll
        for (int q = 0; q < EPL; ++q) x[q] = xn[q];
    }
    wave_sync();

    // --- rank of each slot among the wave's earlier slots of the same expert ---
    const int ns = ntok * k;
    int rank[kRouteChunks], ce[kRouteChunks];
    float cw[kRouteChunks];
#pragma unroll
    for (int c = 0; c < kRouteChunks; ++c) {
        rank[c] = 0;
        ce[c] = 0;
        cw[c] = 0.0f;
        if (c * kWave < ns) {
            const int sl = c * kWave + lane;
            const bool valid = sl < ns;
            const int e = valid ? stage[sl] : 0;
            cw[c] = valid ? wstage[sl] : 0.0f;
            // m: the chunk's lanes whose expert has every id bit equal to this lane's
            uint64_t m = __builtin_amdgcn_ballot_w64(valid);
            for (int b = 0; b < a.id_bits; ++b) {
                const bool bit = (e >> b) & 1;
                const uint64_t bb = __builtin_amdgcn_ballot_w64(bit);
                m &= bit ? bb : ~bb;
            }
            const int below = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0));
            const int base = valid ? mycnt[e] : 0;
            rank[c] = base + below;
            ce[c] = e;
            wave_sync();
            if (valid && (m >> lane) == 1) mycnt[e] = uint16_t(base + below + 1);  // last of its expert
            wave_sync();
        }
    }
    __syncthreads();
    // waves' counts -> exclusive prefix over the waves, in wave order; block totals out
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int c[kRouteWaves];
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) c[w] = cnt[w * E + e];
        int run = 0;
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) {
            cnt[w * E + e] = uint16_t(run);
            run += c[w];
        }
        a.counts[int64_t(blockIdx.x) * E + e] = run;
    }
    __syncthreads();
    // Every global store of the wave's slots comes last: a store before a barrier or a wave
    // fence would be waited for there.  A wave's slots are contiguous, so these are coalesced.
#pragma unroll
    for (int c = 0; c < kRouteChunks; ++c) {
        const int sl = c * kWave + lane;
        if (sl < ns) {
            a.expert_ids[tw0 * k + sl] = ce[c];
            a.weights[tw0 * k + sl] = cw[c];
            a.idx[tw0 * k + sl] = rank[c] + mycnt[ce[c]];
        }
    }
}

// Grid: ceil(E / 64) blocks of kRouteWaves waves; lane = expert, wave = a run of blocks.  Runs
// of up to kScanRegs blocks stay in registers between the sum and the rewrite.
constexpr int kScanRegs = 16;

__global__ void __launch_bounds__(kRouteWaves * kWave) route_scan_kernel(const RouteArgs a) {
    __shared__ int32_t wsum[kRouteWaves][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int E = a.E, nb = a.nblocks;
    const int e = blockIdx.x * kWave + lane;
    const bool valid = e < E;
    const int per = (nb + kRouteWaves - 1) / kRouteWaves;
    const int b0 = wave * per < nb ? wave * per : nb;
    const int b1 = b0 + per < nb ? b0 + per : nb;
    int32_t* col = a.counts + (valid ? e : E - 1);
    int v[kScanRegs];
    int sum = 0;
    if (per <= kScanRegs) {
        // unconditional loads (clamped into the wave's run) so that all are in flight at once
        if (b0 < b1) {
#pragma unroll
            for (int i = 0; i < kScanRegs; ++i) v[i] = col[int64_t(b0 + i < b1 ? b0 + i : b1 - 1) * E];
        }
#pragma unroll
        for (int i = 0; i < kScanRegs; ++i) {
            v[i] = valid && b0 + i < b1 ? v[i] : 0;
            sum += v[i];
        }
    } else if (valid) {
#pragma unroll 8
        for (int b = b0; b < b1; ++b) sum += col[int64_t(b) * E];
    }
    wsum[wave][lane] = sum;
    __syncthreads();
    int run = 0;
    for (int w = 0; w < wave; ++w) run += wsum[w][lane];
    if (per <= kScanRegs) {
#pragma unroll
        for (int i = 0; i < kScanRegs; ++i) {
            if (valid && b0 + i < b1) col[int64_t(b0 + i) * E] = run;
            run += v[i];
        }
    } else if (valid) {
        for (int b = b0; b < b1; ++b) {
            const int c = col[int64_t(b) * E];
            col[int64_t(b) * E] = run;
            run += c;
        }
    }
    if (valid && wave == kRouteWaves - 1) a.totals[e] = run;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(v, d);
        if (lane >= d) v += y;
    }
    return v;
}

// Grid: max(nblocks, 1) blocks of kRouteScatterThreads (one thread per expert).
__global__ void __launch_bounds__(kRouteScatterThreads) route_scatter_kernel(const RouteArgs a) {
    __shared__ int32_t tab[kRouteMaxE];
    __shared__ int32_t wtot[kRouteScatterThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int E = a.E, k = a.k;
    const int64_t total = a.T * k;
    const int64_t per = int64_t(kRouteWaves) * a.tpw * k;
    const int64_t s0 = int64_t(blockIdx.x) * per;
    const int64_t s1 = s0 + per < total ? s0 + per : total;
    // the block's slots: loaded first, they depend on nothing below
    // (unconditional loads, clamped into range, so that all are in flight at once)
    int se[kRouteScatterSlots], sr[kRouteScatterSlots];
    const int e = tid;
    const int ec = e < E ? e : E - 1;
    int v = a.totals[ec];
    int c = 0;
    if (s0 < s1) {  // false only for the single block of T == 0
#pragma unroll
        for (int i = 0; i < kRouteScatterSlots; ++i) {
            const int64_t s = s0 + tid + int64_t(i) * kRouteScatterThreads;
            se[i] = a.expert_ids[s < s1 ? s : s1 - 1];
            sr[i] = a.idx[s < s1 ? s : s1 - 1];
        }
        c = a.counts[int64_t(blockIdx.x) * E + ec];
    }
    v = e < E ? v : 0;
    c = e < E ? c : 0;
    const int incl = wave_inclusive_scan(v, lane);
    if (lane == kWave - 1) wtot[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    const int off = before + incl - v;  // slots routed to experts below e
    if (e < E) tab[e] = off + c;
    if (blockIdx.x == 0 && e < E) {
        a.offsets[e] = off;
        if (e == E - 1) a.offsets[E] = off + v;  // the total T*k
    }
    __syncthreads();
    if (s0 >= s1) return;
#pragma unroll
    for (int i = 0; i < kRouteScatterSlots; ++i) {
        const int64_t s = s0 + tid + int64_t(i) * kRouteScatterThreads;
        const int ex = se[i];
        if (s >= s1 || ex < 0 || ex >= E) continue;  // ids are always below E
        const int64_t p = int64_t(tab[ex]) + sr[i];
        if (p < 0 || p >= total) continue;  // never taken: the ranks of an expert are distinct
        a.idx[s] = int32_t(p);
        a.perm[p] = int32_t(s);
    }
}

// ---------------------------------------------------------------------------------------
// Small calls (a per-block count table of at most kRouteFinishCells entries and at most
// kRouteFinishSlots slots, e.g. decode): kernels 2 and 3 in one workgroup of 1024 threads,
// which saves a launch (about the floor of a small kernel).  Same results as kernels 2 and 3.
//  1. one thread per expert: the exclusive prefix of its block counts over the blocks (in
//     LDS) and its total;
//  2. offsets = exclusive scan of the totals over the experts, added to every block prefix;
//  3. every slot s of block b: p = offsets[e] + prefix[b][e] + (its rank within the block,
//     left in idx by kernel 1); idx[s] = p, perm[p] = s.
constexpr int kRouteFinishCells = 8192;
constexpr int kRouteFinishSlots = 16384;
static_assert(kRouteScatterThreads == kRouteMaxE, "one thread per expert in the finish kernel");

__global__ void __launch_bounds__(kRouteScatterThreads) route_finish_kernel(const RouteArgs a) {
    __shared__ int32_t pre[kRouteFinishCells];  // [nblocks][E]
    __shared__ int32_t wtot[kRouteScatterThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int E = a.E, k = a.k, nb = a.nblocks;
    const int e = tid;
    int run = 0;
    if (e < E) {
        for (int b = 0; b < nb; ++b) {
            const int c = a.counts[int64_t(b) * E + e];
            pre[b * E + e] = run;
            run += c;
        }
    }
    const int incl = wave_inclusive_scan(run, lane);
    if (lane == kWave - 1) wtot[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    const int off = before + incl - run;  // slots routed to experts below e
    if (e < E) {
        a.offsets[e] = off;
        if (e == E - 1) a.offsets[E] = off + run;  // the total T*k
        for (int b = 0; b < nb; ++b) pre[b * E + e] += off;
    }
    __syncthreads();
    const int total = int(a.T) * k;
    const int per = kRouteWaves * a.tpw * k;  // slots per block of kernel 1
    for (int s = tid; s < total; s += kRouteScatterThreads) {
        const int ex = a.expert_ids[s];
        const int b = s / per;
        if (ex < 0 || ex >= E || b >= nb) continue;  // never taken: ids are below E
        const int p = pre[b * E + ex] + a.idx[s];
        if (p < 0 || p >= total) continue;  // never taken: the ranks of an expert are distinct
        a.idx[s] = p;
        a.perm[p] = s;
    }
}

}  // namespace mf
