/*
 * mf.h - C ABI of the MI355X (gfx950) MoE finalize library, its sibling fused norms and the
 * routing producer of its inputs.
 *
 * Sources of the operations (pages on FlashInfer pull requests; section names as on each page):
 *  [PR5319] "FlashInfer MoE performance: improving the deterministic finalize with CuTe DSL",
 *           section 1 (the new CuTe DSL finalize kernel and its _fma_rn helper).
 *  [PR6544] "FlashInfer: fused norms and TP/EP MoE for Muse-Spark-Open", sections 1.1
 *           (gated residual RMSNorm), 1.2 (RMSNorm + sigmoid gate), 2.1 (TP MoE finalize),
 *           2.4 (MoE finalize + RMSNorm + all-reduce) and the "Fixed-Width Fused Norms" docs.
 *  [PR4730] "MoE all-reduce fusion for Blackwell: FlashInfer's Cake backend", section 2
 *           (fusion strategy: expert sum, residual add and RMSNorm in one launch).
 *  [PR4130] "FlashInfer: fused kernels and an optimised scheduler for MoE", code analysis
 *           items 1-3 (grouped GEMM over m_indptr rows; the warp-cooperative scheduler).
 *  OCP Microscaling Formats (MX) specification: the MXFP4 format (E8M0 block scales over
 *           32 values, E2M1 elements) used for the FP4 quantisation.
 *
 * Conventions for every entry point:
 *  - Tensors are dense and row-major.  bfloat16 data is passed as raw 16-bit patterns
 *    (uint16_t).  All tensor pointers are device pointers on the current HIP device.
 *  - The caller owns every buffer.  The library allocates nothing, keeps no state between
 *    calls and is safe to call from several threads (mf_moe_route_noalloc alone keeps a static
 *    per-GPU scratch array; see its declaration).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the null stream).
 *    The library never synchronizes.
 *  - Arguments are checked on the host before any HIP call.  On a failed check the function
 *    returns a negative mf_status and launches nothing.  A zero token count returns MF_OK
 *    without a launch (mf_moe_route still writes its expert_offsets).
 *  - Row pointers (bf16 and fp32 tensors with H or head_dim columns) must be 16-byte
 *    aligned; idx, weights and expert_ids 4-byte aligned.
 *  - Results are deterministic: the same inputs give bit-identical outputs, whatever the
 *    token count, the stream or the launch shape chosen for it.
 *  - Preconditions that are not checked (the kernels stay memory-safe if they are broken,
 *    but the affected outputs are unspecified): indices lie in range, pointers are device
 *    memory of the stated size.
 */
#ifndef MF_H
#define MF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mf_status {
    MF_OK = 0,
    MF_ERR_NULL = -1,        /* a required pointer is NULL */
    MF_ERR_SHAPE = -2,       /* a size is negative or inconsistent */
    MF_ERR_UNSUPPORTED = -3, /* a width or top-k outside what the *_supported queries accept */
    MF_ERR_ALIGN = -4,       /* a pointer is not aligned as stated above */
    MF_ERR_ALIAS = -5,       /* an output overlaps an input (except residual_out == residual) */
    MF_ERR_HIP = -6,         /* the HIP runtime reported an error for the launch */
    MF_ERR_VALUE = -7,       /* eps is negative, NaN or infinite */
    MF_ERR_SCRATCH = -8      /* the problem needs more scratch than the library's static
                                buffer holds (mf_moe_route_noalloc only) */
} mf_status;

/*
 * MoE finalize fused with the residual add and RMSNorm ([PR5319] section 1; [PR6544]
 * sections 2.1 and 2.4; [PR4730] section 2).
 *
 * For every token t in [0, T):
 *   acc = +0 (fp32, H values)
 *   for j = 0 .. k-1, in this order:
 *       x = widen(expert_rows[idx[t,j], :])                               (bf16 -> fp32, exact)
 *       if per-expert: x = x * (mean(x^2) + eps)^-1/2 * expert_gamma[expert_ids[t,j], :]
 *       acc = fma(weights[t,j], x, acc)                      (fp32 fused multiply-add, RNE)
 *   residual_out[t,:] = residual[t,:] + acc                                         (fp32)
 *   out[t,:] = bf16_rne(residual_out[t,:] * (mean(residual_out[t,:]^2) + eps)^-1/2 * gamma)
 *
 *  expert_rows   bf16 [num_rows, H]: the permuted GEMM2 (FC2) output, one row per (t, j).
 *  idx           int32 [T, k]: the row of expert_rows holding slot (t, j).  A gather: rows
 *                may be in any order (e.g. grouped by expert); each is read where it lies.
 *  weights       fp32 [T, k]: routing weights.
 *  expert_ids    int32 [T, k] and expert_gamma bf16 [num_experts, H]: both NULL for the plain
 *                finalize; both set for the per-expert-RMSNorm variant ([PR6544] 2.1).
 *  residual      fp32 [T, H] in; residual_out fp32 [T, H] out.  residual_out may equal
 *                residual (in-place update of the residual stream); partial overlap is
 *                rejected.
 *  gamma         bf16 [H]; eps >= 0; out bf16 [T, H].
 * Supported: H % 8 == 0 and 8 <= H <= 32768; 1 <= k <= 64 (both variants).  Out-of-range
 * idx or expert_ids are clamped into range (memory-safe, result unspecified for that token).
 */
int mf_moe_finalize(const uint16_t* expert_rows, int64_t num_rows, const int32_t* idx,
                    const float* weights, const int32_t* expert_ids,
                    const uint16_t* expert_gamma, int32_t num_experts, const float* residual,
                    float* residual_out, const uint16_t* gamma, float eps, uint16_t* out,
                    int64_t T, int32_t H, int32_t k, void* stream);

/*
 * mf_moe_finalize with an MXFP4 epilogue ([PR6544] section 2.3: RMSNorm + block-scaled FP4
 * quantisation; the MXFP4 format as for mf_mxfp4_quantize below): residual_out as in
 * mf_moe_finalize, and instead of the bf16 out the normalised row
 *   y = fp32((residual_out * (mean(residual_out^2) + eps)^-1/2) * gamma)
 * quantised to MXFP4: q uint8 [T, H/2] (4-byte aligned) and scales uint8 [T, H/32].  The plain
 * finalize only (no per-expert norm); H % 32 == 0; other arguments and checks as
 * mf_moe_finalize's.
 */
int mf_moe_finalize_mxfp4(const uint16_t* expert_rows, int64_t num_rows, const int32_t* idx,
                          const float* weights, const float* residual, float* residual_out,
                          const uint16_t* gamma, float eps, uint8_t* q, uint8_t* scales,
                          int64_t T, int32_t H, int32_t k, void* stream);

/*
 * The expert-parallel split of the finalize ([PR6544] section 2.4: finalize + RMSNorm +
 * all-reduce, where the slots of non-local experts skip normalisation; [PR4730] section 2: the
 * all-reduce's sum fused with the residual add and RMSNorm).  Between the two calls the
 * caller exchanges the partials (a reduce-scatter by token owner), which is not part of this
 * library; on one GPU the partials of every rank can be computed and combined in place.
 *
 * mf_moe_finalize_ep_partial: this GPU's share.  For every token t:
 *   partial[t,:] = +0; for j = 0..k-1 in order, skipping every slot with idx[t,j] < 0 (an
 *   expert on another GPU: its row, expert id and weight are not read):
 *       partial[t,:] = fma(weights[t,j], x_j, partial[t,:])      (x_j as in mf_moe_finalize)
 *  Arguments as mf_moe_finalize's; partial fp32 [T, H] (16-byte aligned, overlapping no
 *  input).  A token with no local slot gets +0.  num_rows >= 1 (pass any one-row buffer when
 *  no expert is local).  idx >= num_rows is clamped (memory-safe, result unspecified).
 *
 * mf_moe_finalize_ep_combine: the token owner's step.  For every token t of its T tokens:
 *   acc = +0; for g = 0..num_ranks-1 in order: acc = acc + partials[g, t, :]      (fp32)
 *   residual_out[t,:] = residual[t,:] + acc
 *   out[t,:] = bf16_rne(residual_out * (mean(residual_out^2) + eps)^-1/2 * gamma)
 *  partials fp32 [num_ranks, T, H] (rank-major), 1 <= num_ranks <= 1024; the other arguments
 *  and their checks as mf_moe_finalize's (residual_out may equal residual).
 * With one rank holding every expert, partial + combine give mf_moe_finalize's residual_out bit
 * for bit, and its out within one bf16 ulp (the combine's final RMSNorm may reduce the mean
 * square in another wave layout).
 */
int mf_moe_finalize_ep_partial(const uint16_t* expert_rows, int64_t num_rows,
                               const int32_t* idx, const float* weights,
                               const int32_t* expert_ids, const uint16_t* expert_gamma,
                               int32_t num_experts, float eps, float* partial, int64_t T,
                               int32_t H, int32_t k, void* stream);
int mf_moe_finalize_ep_combine(const float* partials, int32_t num_ranks, const float* residual,
                               float* residual_out, const uint16_t* gamma, float eps,
                               uint16_t* out, int64_t T, int32_t H, void* stream);

/*
 * Gated-residual RMSNorm ([PR6544] section 1.1; fixed hidden size 8192 there, any
 * supported H here):
 *   residual_out = residual + sigmoid(gate) * x                 (fp32, sigmoid = 1/(1+e^-g))
 *   out = bf16_rne(residual_out * (mean(residual_out^2) + eps)^-1/2 * gamma)
 *  x, gate bf16 [T, H]; residual, residual_out fp32 [T, H] (may be equal); gamma bf16 [H];
 *  out bf16 [T, H].  Supported: H % 8 == 0 and 8 <= H <= 32768.
 */
int mf_gated_residual_rmsnorm(const uint16_t* x, const uint16_t* gate, const float* residual,
                              float* residual_out, const uint16_t* gamma, float eps,
                              uint16_t* out, int64_t T, int32_t H, void* stream);

/*
 * Gated-residual dual RMSNorm ("gated_residual_next_rmsnorm": named by [PR6544]'s fixed-width
 * norm docs and its section 2.2 "gated residual dual norm", not defined there).  Reading taken:
 * the gated residual above feeds two RMSNorm outputs that share one mean square, this layer's
 * and the next layer's pre-norm:
 *   residual_out = residual + sigmoid(gate) * x                                     (fp32)
 *   out      = bf16_rne(residual_out * (mean(residual_out^2) + eps)^-1/2 * gamma)
 *   out_next = bf16_rne(residual_out * (mean(residual_out^2) + eps)^-1/2 * gamma_next)
 *  Arguments as for mf_gated_residual_rmsnorm, plus gamma_next bf16 [H] and out_next bf16 [T, H]
 *  (16-byte aligned; out_next may overlap nothing).  residual_out and out are bit-identical to
 *  what mf_gated_residual_rmsnorm returns for the same inputs.  Supported: as that function.
 */
int mf_gated_residual_next_rmsnorm(const uint16_t* x, const uint16_t* gate,
                                   const float* residual, float* residual_out,
                                   const uint16_t* gamma, const uint16_t* gamma_next, float eps,
                                   uint16_t* out, uint16_t* out_next, int64_t T, int32_t H,
                                   void* stream);

/*
 * Per-head RMSNorm with a sigmoid gate ([PR6544] section 1.2; head dim 64):
 *   out[t,n,:] = bf16_rne(x[t,n,:] * (mean(x[t,n,:]^2) + eps)^-1/2 * gamma * sigmoid(gate[t,n,:]))
 *  x, gate, out bf16 [T, num_heads, head_dim]; gamma bf16 [head_dim], shared by all heads.
 *  The sum of squares is reduced in fp32.  Supported: head_dim == 64, num_heads >= 1.
 */
int mf_rmsnorm_sigmoid_gate(const uint16_t* x, const uint16_t* gate, const uint16_t* gamma,
                            float eps, uint16_t* out, int64_t T, int32_t num_heads,
                            int32_t head_dim, void* stream);

/*
 * MXFP4 block quantisation ([PR6544] section 2.3: RMSNorm + block-scaled FP4 quantisation,
 * NVFP4 there; here the OCP Microscaling MXFP4 format, from its published definition).  Along
 * each row, blocks of 32 consecutive values share one E8M0 scale X = 2^e,
 *   e = floor(log2(max |v|)) - 2, clamped to [-127, 127] (an all-zero block takes -127),
 *   scales[t, b] = e + 127
 * and every value is stored as the E2M1 code (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 the
 * sign, kept for zeros) nearest to v / X, ties to the even code, magnitudes above 6 saturating
 * to 6.  q[t, i] holds the codes of values 2i (low nibble) and 2i+1 (high nibble).
 *
 * mf_mxfp4_quantize: x fp32 [T, H] (16-byte aligned) -> q uint8 [T, H/2] (4-byte aligned),
 *   scales uint8 [T, H/32].
 * mf_rmsnorm_mxfp4_quantize: x bf16 [T, H], gamma bf16 [H] (16-byte aligned), eps >= 0:
 *   y = fp32((x * (mean(x^2) + eps)^-1/2) * gamma) (as the bf16 RMSNorm outputs above, before
 *   their rounding), then q, scales = MXFP4(y).
 * Supported: H % 32 == 0 and 32 <= H <= 32768.  No output may overlap an input or the other
 * output.  Inputs must be finite (other values give unspecified codes).
 */
int mf_mxfp4_quantize(const float* x, int64_t T, int32_t H, uint8_t* q, uint8_t* scales,
                      void* stream);
int mf_rmsnorm_mxfp4_quantize(const uint16_t* x, const uint16_t* gamma, float eps, uint8_t* q,
                              uint8_t* scales, int64_t T, int32_t H, void* stream);

/*
 * MoE routing and the expert-sorted permutation: the producer of the finalize's idx and
 * weights, and of the per-expert row ranges of the grouped GEMM that writes expert_rows
 * ([PR4130] code analysis items 1-3: the m_indptr / token_offset layout of the grouped GEMM
 * and its warp-cooperative prefix-count scheduler; the finalize gathers through idx, [PR5319]
 * section 1).
 *
 * For every token t in [0, T), with logits fp32 [T, E]:
 *   expert_ids[t, 0..k-1] = the experts of the k largest logits of row t, largest first; equal
 *                           logits go to the lower expert id first (-0 equals +0)
 *   weights[t, j]         = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0)   (fp32; the softmax over
 *                           the k selected logits, l_j = logits[t, expert_ids[t, j]])
 * and over the T*k slots s = t*k + j:
 *   expert_offsets[e]     = number of slots routed to experts below e; expert_offsets[E] = T*k
 *   perm[p]               = the slot at permuted row p: slots grouped by expert in expert
 *                           order, ascending slot order within an expert (a stable sort)
 *   idx[t, j]             = the permuted row of slot (t, j); idx[perm[p]] = p
 *
 *  logits        fp32 [T, E], finite (NaN logits give in-range experts, otherwise unspecified).
 *  expert_ids    int32 [T, k], weights fp32 [T, k], idx int32 [T, k], perm int32 [T*k],
 *                expert_offsets int32 [E + 1]: outputs, all written by the call.
 *  workspace     device memory of at least mf_moe_route_workspace_bytes(T, E, k) bytes,
 *                4-byte aligned, owned by the caller; its contents on entry do not matter and
 *                on exit are unspecified.  Calls that share a workspace must not overlap.
 * Supported: 1 <= E <= 1024 and 1 <= k <= min(E, 16); T * k < 2^31.  Everything but the
 * weights is exact integer work; the weights are fp32 (expf, a sum in j order, a division).
 * T == 0 writes expert_offsets (all zero) and nothing else.  No output may overlap another,
 * the logits or the workspace.
 */
int mf_moe_route(const float* logits, int64_t T, int32_t num_experts, int32_t k,
                 int32_t* expert_ids, float* weights, int32_t* idx, int32_t* perm,
                 int32_t* expert_offsets, void* workspace, int64_t workspace_bytes,
                 void* stream);

/*
 * Workspace bytes mf_moe_route needs: 4 * E * (nblocks + 1), a per-block table of per-expert
 * counts and the per-expert totals.  nblocks = ceil(T / (16 * tpw)), where tpw (tokens per
 * wave) is the smallest power of two >= T / 4096, capped at 16 and at 256 / k.  Returns a
 * negative mf_status for unsupported arguments.
 */
int64_t mf_moe_route_workspace_bytes(int64_t T, int32_t num_experts, int32_t k);

/*
 * mf_moe_route without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * results as mf_moe_route, bit for bit, with the per-block count table kept in a static device
 * array of the library, MF_ROUTE_SCRATCH_BYTES (4 MiB) per GPU, held until the process ends.
 *  - Arguments, outputs and checks as mf_moe_route's, less the workspace.  A call whose
 *    mf_moe_route_workspace_bytes exceeds MF_ROUTE_SCRATCH_BYTES returns MF_ERR_SCRATCH and
 *    launches nothing (at E = 256, k = 8 that is T above about a million tokens).
 *  - Calls nothing that allocates (no hipMalloc, hipFree or allocating library routine).  The
 *    first call on a device looks up that device's copy of the array (hipGetSymbolAddress);
 *    a failure there returns MF_ERR_HIP.
 *  - Every call on one GPU shares that GPU's array, and nothing in it needs to start at zero.
 *    Calls that may overlap on one GPU (different streams, or several host threads) race on
 *    it: the caller must order them, or use mf_moe_route with workspaces of its own.
 */
#define MF_ROUTE_SCRATCH_BYTES (4 << 20)
int mf_moe_route_noalloc(const float* logits, int64_t T, int32_t num_experts, int32_t k,
                         int32_t* expert_ids, float* weights, int32_t* idx, int32_t* perm,
                         int32_t* expert_offsets, void* stream);

/*
 * Capability queries (the fixed-width contract of [PR6544]'s "Fixed-Width Fused Norms":
 * check before calling and fall back otherwise).  Return 1 if supported, else 0.
 */
int mf_moe_finalize_supported(int32_t H, int32_t k, int per_expert);
int mf_gated_residual_rmsnorm_supported(int32_t H);
int mf_gated_residual_next_rmsnorm_supported(int32_t H);
int mf_rmsnorm_sigmoid_gate_supported(int32_t head_dim);
int mf_moe_route_supported(int32_t num_experts, int32_t k);
int mf_mxfp4_supported(int32_t H);

/*
 * Launch shape that mf_moe_finalize / mf_gated_residual_rmsnorm / mf_moe_finalize_ep_combine /
 * mf_moe_finalize_ep_partial use for a problem size: waves per token row, 16-byte vectors per
 * lane (the row slice each lane holds), workgroup size and grid size.  Any output pointer may be
 * NULL.  Returns MF_OK or MF_ERR_UNSUPPORTED.  (kind: 0 = finalize, 1 = finalize with
 * per-expert RMSNorm, 2 = gated-residual RMSNorm, 3 = expert-parallel combine, 4 =
 * expert-parallel partial without per-expert RMSNorm (with it, kind 1's shape); k is ignored for
 * kinds 2 and 3.)
 */
int mf_launch_shape(int kind, int64_t T, int32_t H, int32_t k, int32_t* waves_per_token,
                    int32_t* vectors_per_lane, int32_t* block_threads, int64_t* grid_blocks);

/*
 * Streaming copy of `bytes` bytes (a multiple of 16, at most 64 GiB; both pointers 16-byte
 * aligned, not overlapping) with the same 16-byte nontemporal loads and stores as the kernels
 * above, one per lane in one-wave workgroups.  A measurement aid: it gives the achievable HBM
 * copy bandwidth and calibrates the HBM byte counters.  MF_ERR_SHAPE for a bad or oversized
 * byte count.
 */
int mf_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * Streaming read of `bytes` bytes (a multiple of 16; src 16-byte aligned) with the same
 * 16-byte nontemporal loads.  A measurement aid: it gives the achievable HBM read bandwidth.
 * Nothing is written but sink[c] = the xor of the 32-bit words of chunk c, for each chunk of
 * MF_STREAM_READ_CHUNK bytes (the last one may be short): sink holds
 * ceil(bytes / MF_STREAM_READ_CHUNK) words (4-byte aligned, not overlapping src).
 */
#define MF_STREAM_READ_CHUNK 16384
int mf_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/*
 * An empty kernel of `workgroups` workgroups of `threads` threads (1..1024): a measurement aid
 * giving the dispatch floor of a grid shape, e.g. the per-head norm's 32768 one-wave
 * workgroups.  Returns MF_ERR_SHAPE for an empty or oversized grid.
 */
int mf_empty_grid(int64_t workgroups, int32_t threads, void* stream);

/* Human-readable name of a status code (never NULL). */
const char* mf_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MF_H */
