// Host side of the routing entry points declared in include/mf.h: argument checks (before any
// HIP call), the launch plan and the launches (two for small calls, three otherwise).
// mf_moe_route allocates nothing and keeps no state: the caller passes the workspace.
// mf_moe_route_noalloc runs on a static per-device scratch array instead (below).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "api_util.h"
#include "mf.h"
#include "route_kernels.h"

namespace {

using namespace mf;

// Routing launch plan.  Kernel 1 runs one wave per `tpw` consecutive tokens, 16 waves per
// block: tpw grows with T (a power of two, up to 16, and tpw * k <= 256 slots per wave) so that
// about 4096 waves share the work and the per-block count table stays small.
struct RoutePlan {
    int tpw;
    int64_t nblocks;
    int id_bits;
    int epl;  // logits per lane: E <= 64 * epl
};

bool route_supported(int32_t E, int32_t k) {
    return E >= 1 && E <= kRouteMaxE && k >= 1 && k <= kRouteMaxK && k <= E;
}

RoutePlan route_plan(int64_t T, int32_t E, int32_t k) {
    RoutePlan p;
    const int64_t want = (T + 4095) / 4096;
    p.tpw = 1;
    while (p.tpw < want && p.tpw < 16) p.tpw *= 2;
    while (p.tpw * k > kRouteSlotsPerWave) p.tpw /= 2;
    const int64_t tpb = int64_t(kRouteWaves) * p.tpw;
    p.nblocks = (T + tpb - 1) / tpb;
    p.id_bits = 0;
    while ((1 << p.id_bits) < E) ++p.id_bits;
    p.epl = pow2_at_least((E + kWave - 1) / kWave);
    return p;
}

int64_t route_workspace_bytes(const RoutePlan& p, int32_t E) {
    return (p.nblocks + 1) * int64_t(E) * int64_t(sizeof(int32_t));
}

// The select kernel for a logits-per-lane count; vec: E a multiple of it and the logits
// aligned to it (only the lane-major widths 2 and 4 have a vector form).
const void* route_select_fn(int epl, bool vec) {
    switch (epl) {
        case 1: return reinterpret_cast<const void*>(&route_select_kernel<1, false>);
        case 2: return vec ? reinterpret_cast<const void*>(&route_select_kernel<2, true>)
                           : reinterpret_cast<const void*>(&route_select_kernel<2, false>);
        case 4: return vec ? reinterpret_cast<const void*>(&route_select_kernel<4, true>)
                           : reinterpret_cast<const void*>(&route_select_kernel<4, false>);
        case 8: return reinterpret_cast<const void*>(&route_select_kernel<8, false>);
        case 16: return reinterpret_cast<const void*>(&route_select_kernel<16, false>);
        default: return nullptr;
    }
}

// Checks of mf_moe_route's arguments (all before any HIP call) and its launch plan.  Without a
// caller workspace (caller_ws false) the call runs on the library's own scratch: workspace is
// then NULL, takes no part in the null, alignment and overlap checks, and workspace_bytes is
// the scratch's size.
int route_check(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* expert_ids,
                float* weights, int32_t* idx, int32_t* perm, int32_t* expert_offsets,
                const void* workspace, int64_t workspace_bytes, bool caller_ws, RoutePlan* plan) {
    if (T < 0 || workspace_bytes < 0) return MF_ERR_SHAPE;
    if (!route_supported(E, k)) return MF_ERR_UNSUPPORTED;
    if (T > INT32_MAX / k) return MF_ERR_SHAPE;  // T * k slots are indexed in int32
    const RoutePlan p = route_plan(T, E, k);
    if (p.nblocks > INT32_MAX || !grid_fits(std::max<int64_t>(p.nblocks, 1), kRouteWaves * kWave))
        return MF_ERR_SHAPE;
    if (workspace_bytes < route_workspace_bytes(p, E)) return MF_ERR_SHAPE;
    if (!expert_offsets || (caller_ws && !workspace)) return MF_ERR_NULL;
    if (T > 0 && (!logits || !expert_ids || !weights || !idx || !perm)) return MF_ERR_NULL;
    const void* ptrs[] = {logits, expert_ids, weights, idx, perm, expert_offsets, workspace};
    for (const void* q : ptrs)
        if (!aligned(q, 4)) return MF_ERR_ALIGN;
    const size_t tk = size_t(T) * k * 4;
    const size_t ws = caller_ws ? size_t(route_workspace_bytes(p, E)) : 0;
    const size_t sizes[] = {size_t(T) * E * 4, tk, tk, tk, tk, size_t(E + 1) * 4, ws};
    for (int i = 0; i < 7; ++i)
        for (int j = i + 1; j < 7; ++j)
            if (overlap(ptrs[i], sizes[i], ptrs[j], sizes[j])) return MF_ERR_ALIAS;
    *plan = p;
    return MF_OK;
}

// The launches of one routing call (two for small calls, three otherwise); `counts` is the
// workspace: [nblocks, E] block counts followed by [E] totals.  Every entry is written by the
// select kernel before it is read, so nothing needs clearing beforehand.
int route_launch(const RoutePlan& p, const float* logits, int64_t T, int32_t E, int32_t k,
                 int32_t* expert_ids, float* weights, int32_t* idx, int32_t* perm,
                 int32_t* expert_offsets, int32_t* counts, void* stream) {
    RouteArgs a;
    a.logits = logits;
    a.expert_ids = expert_ids;
    a.weights = weights;
    a.idx = idx;
    a.perm = perm;
    a.offsets = expert_offsets;
    a.counts = counts;
    a.totals = a.counts + p.nblocks * E;
    a.T = T;
    a.E = E;
    a.k = k;
    a.tpw = p.tpw;
    a.nblocks = int32_t(p.nblocks);
    a.id_bits = p.id_bits;
    void* args[] = {&a};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p.nblocks > 0) {
        const bool vec = (p.epl == 2 || p.epl == 4) && E % p.epl == 0 && aligned(logits, 4 * p.epl);
        const hipError_t e = hipLaunchKernel(route_select_fn(p.epl, vec), dim3(unsigned(p.nblocks)),
                                             dim3(kRouteWaves * kWave), args,
                                             route_select_lds_bytes(E), s);
        if (e != hipSuccess) return MF_ERR_HIP;
    }
    if (p.nblocks * E <= kRouteFinishCells && T * k <= kRouteFinishSlots) {
        // small calls: the scan and the scatter in one workgroup
        return hip_status(hipLaunchKernel(reinterpret_cast<const void*>(&route_finish_kernel),
                                          dim3(1), dim3(kRouteScatterThreads), args, 0, s));
    }
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&route_scan_kernel),
                                   dim3(unsigned((E + kWave - 1) / kWave)),
                                   dim3(kRouteWaves * kWave), args, 0, s);
    if (e != hipSuccess) return MF_ERR_HIP;
    e = hipLaunchKernel(reinterpret_cast<const void*>(&route_scatter_kernel),
                        dim3(unsigned(std::max<int64_t>(p.nblocks, 1))),
                        dim3(kRouteScatterThreads), args, 0, s);
    return hip_status(e);
}

}  // namespace

// ---------------------------------------------------------------------------------------
// The allocation-free routing call (mf_moe_route_noalloc) runs on this file-scope device
// array instead of a caller workspace.  Every GPU the library runs on holds its own copy until
// the process ends.  On the host, `scratch` names a host-side stand-in, not device memory:
// only the address hipGetSymbolAddress returns, looked up once per device with that device
// current, is ever passed to a kernel or used by host code.
static constexpr int64_t kRouteScratchBytes = MF_ROUTE_SCRATCH_BYTES;
static __device__ __align__(256) int32_t scratch[kRouteScratchBytes / sizeof(int32_t)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on that device).
int scratch_on_current_device(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MF_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MF_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MF_OK;
}

// Does a supported call need more workspace than the scratch holds?
bool route_needs_scratch(int64_t T, int32_t E, int32_t k) {
    if (T < 0 || !route_supported(E, k) || T > INT32_MAX / k) return false;
    return route_workspace_bytes(route_plan(T, E, k), E) > kRouteScratchBytes;
}

}  // namespace

extern "C" {

int mf_moe_route_supported(int32_t num_experts, int32_t k) { return route_supported(num_experts, k); }

int64_t mf_moe_route_workspace_bytes(int64_t T, int32_t num_experts, int32_t k) {
    if (T < 0) return MF_ERR_SHAPE;
    if (!route_supported(num_experts, k)) return MF_ERR_UNSUPPORTED;
    if (T > INT32_MAX / k) return MF_ERR_SHAPE;  // T * k slots are indexed in int32
    return route_workspace_bytes(route_plan(T, num_experts, k), num_experts);
}

int mf_moe_route(const float* logits, int64_t T, int32_t num_experts, int32_t k,
                 int32_t* expert_ids, float* weights, int32_t* idx, int32_t* perm,
                 int32_t* expert_offsets, void* workspace, int64_t workspace_bytes,
                 void* stream) {
    RoutePlan p;
    const int st = route_check(logits, T, num_experts, k, expert_ids, weights, idx, perm,
                               expert_offsets, workspace, workspace_bytes, true, &p);
    if (st != MF_OK) return st;
    return route_launch(p, logits, T, num_experts, k, expert_ids, weights, idx, perm,
                        expert_offsets, static_cast<int32_t*>(workspace), stream);
}

int mf_moe_route_noalloc(const float* logits, int64_t T, int32_t num_experts, int32_t k,
                         int32_t* expert_ids, float* weights, int32_t* idx, int32_t* perm,
                         int32_t* expert_offsets, void* stream) {
    // every argument check first, then the one HIP query of the set-up
    if (route_needs_scratch(T, num_experts, k)) return MF_ERR_SCRATCH;
    RoutePlan p;
    const int st = route_check(logits, T, num_experts, k, expert_ids, weights, idx, perm,
                               expert_offsets, nullptr, kRouteScratchBytes, false, &p);
    if (st != MF_OK) return st;
    void* ws = nullptr;
    const int sst = scratch_on_current_device(&ws);
    if (sst != MF_OK) return sst;
    return route_launch(p, logits, T, num_experts, k, expert_ids, weights, idx, perm,
                        expert_offsets, static_cast<int32_t*>(ws), stream);
}

}  // extern "C"
