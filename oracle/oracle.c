/*
 * Plain CPU oracle for the MoE finalize path (and its expert-parallel split into a partial
 * sum per GPU and a combine on the token's owner), its sibling fused norms (gated residual
 * RMSNorm, the dual-output gated residual norm, per-head RMSNorm with a sigmoid gate), the
 * MXFP4 block quantisation of a normalised row, and the routing that produces the finalize's
 * gather indices and weights.
 *
 * Parity unpinned, as to meaning only: the dual-output gated residual norm is named by the
 * pages but not defined; the reading taken is stated at its function, whose arithmetic the
 * tests pin.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark may load this library.  It shares no code, header, table or helper with
 * the GPU library; the two are independent implementations of the same definitions.
 *
 * Every function is the plain definition, written out with one loop per step and no
 * blocking, fusion or reordering:
 *
 *  - The weighted accumulation is the one place where the pages fix the precision: the
 *    deterministic finalize (page "FlashInfer MoE performance: improving the deterministic
 *    finalize with CuTe DSL", PR #5319, section 1, the _fma_rn listing and the paragraph
 *    after it) accumulates the gathered expert rows with FP32 fused multiply-adds, rounded
 *    to nearest, in a fixed order, and converts to BF16 only at the end.  Here that is
 *    fmaf() for j = 0..k-1, starting from +0.  The flush-to-zero in that listing is there to
 *    match an older fast-math kernel and only changes values below 2^-126; this oracle
 *    keeps denormals.
 *  - The residual add is one float32 addition after the k-term sum (page "MoE all-reduce
 *    fusion for Blackwell: FlashInfer's Cake backend", PR #4730, section 2, fusion
 *    strategy: the expert outputs are summed, the residual added and RMSNorm applied in one
 *    launch; the residual stream stays FP32 per page "FlashInfer fused norms and TP/EP MoE
 *    for Muse-Spark-Open", PR #6544, section 1.1).
 *  - Everything the pages leave open is computed in float64: sums of squares, the RMSNorm
 *    scale (mean(x^2) + eps)^-1/2, the sigmoid 1/(1+e^-g), and products with gamma.  A
 *    float64 value is rounded once, to nearest-even, to the stored type (float32 or bf16).
 *
 * bfloat16 values are passed as their raw 16-bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Exact widening of a bfloat16 bit pattern: it is the upper half of a binary32. */
static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a float64 to the nearest bfloat16 (8 significant bits, ties to even), once. */
static uint16_t bf16_round(double v) {
    if (isnan(v)) return 0x7FC0;
    if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    double r;
    if (fabs(v) < 0x1p-126) {
        /* subnormal range of bfloat16: a fixed spacing of 2^-133 */
        r = ldexp(nearbyint(ldexp(v, 133)), -133);
    } else {
        int e;
        double m = frexp(v, &e);                      /* v = m * 2^e, 0.5 <= |m| < 1 */
        r = ldexp(nearbyint(ldexp(m, 8)), e - 8);     /* keep 8 significant bits */
    }
    float f = (float)r; /* exact (8 significant bits), or +-inf past the bf16 range */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* RMSNorm scale of n values: (sum(x^2)/n + eps)^(-1/2), all in float64. */
static double rms_scale_f32(const float* x, int64_t n, float eps) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
    return 1.0 / sqrt(ss / (double)n + (double)eps);
}

static double rms_scale_bf16(const uint16_t* x, int64_t n, float eps) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double v = bf16_value(x[i]);
        ss += v * v;
    }
    return 1.0 / sqrt(ss / (double)n + (double)eps);
}

static double sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }

/*
 * MoE finalize with a residual add and a final RMSNorm.
 *
 * For token t, slot j's expert output is row idx[t,j] of expert_rows, the permuted GEMM2
 * output that the TP MoE finalize reads directly (PR #6544 page, section 2.1).  If
 * expert_gamma is given, each gathered row is first RMSNormed over H with the gamma of its
 * expert expert_ids[t,j] (the per-expert RMSNorm of that section); the normalised row is
 * rounded to float32.  Then
 *     acc = +0;  acc = fmaf(w[t,j], row_j, acc) for j = 0..k-1
 *     residual_out[t] = residual[t] + acc                              (float32)
 *     out[t] = bf16(residual_out[t] * rms_scale(residual_out[t]) * gamma)
 *
 * Returns 0, -1 if an index is out of range, -2 if scratch memory cannot be allocated.
 * residual_out may be the same array as residual.
 */
int oracle_moe_finalize(const uint16_t* expert_rows, int64_t num_rows, const int32_t* idx,
                        const float* weights, const int32_t* expert_ids,
                        const uint16_t* expert_gamma, int32_t num_experts, const float* residual,
                        float* residual_out, const uint16_t* gamma, float eps, uint16_t* out,
                        int64_t T, int32_t H, int32_t k) {
    float* acc = (float*)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
    float* row = (float*)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
    int status = 0;
    if (!acc || !row) {
        status = -2;
        goto done;
    }
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) acc[h] = 0.0f;
        for (int32_t j = 0; j < k; ++j) {
            int64_t p = idx[t * k + j];
            if (p < 0 || p >= num_rows) {
                status = -1;
                goto done;
            }
            const uint16_t* x = expert_rows + p * (int64_t)H;
            if (expert_gamma) {
                int32_t e = expert_ids[t * k + j];
                if (e < 0 || e >= num_experts) {
                    status = -1;
                    goto done;
                }
                const uint16_t* ge = expert_gamma + (int64_t)e * H;
                double s = rms_scale_bf16(x, H, eps);
                for (int32_t h = 0; h < H; ++h)
                    row[h] = (float)(bf16_value(x[h]) * s * bf16_value(ge[h]));
            } else {
                for (int32_t h = 0; h < H; ++h) row[h] = (float)bf16_value(x[h]);
            }
            float wj = weights[t * k + j];
            for (int32_t h = 0; h < H; ++h) acc[h] = fmaf(wj, row[h], acc[h]);
        }
        const float* res = residual + t * (int64_t)H;
        float* r = residual_out + t * (int64_t)H;
        for (int32_t h = 0; h < H; ++h) r[h] = res[h] + acc[h];
        double s = rms_scale_f32(r, H, eps);
        uint16_t* o = out + t * (int64_t)H;
        for (int32_t h = 0; h < H; ++h) o[h] = bf16_round((double)r[h] * s * bf16_value(gamma[h]));
    }
done:
    free(acc);
    free(row);
    return status;
}

/*
 * The MoE finalize split for expert parallelism (page "FlashInfer: fused norms and TP/EP MoE
 * for Muse-Spark-Open", PR #6544, section 2.4: finalize + RMSNorm + all-reduce, where the
 * slots of non-local experts skip the per-expert normalisation; page "MoE all-reduce fusion
 * for Blackwell: FlashInfer's Cake backend", PR #4730, section 2: the all-reduce's sum of the
 * expert outputs is fused with the residual add and RMSNorm).  Two steps:
 *
 *  ep_partial (on every GPU, over its local slots): idx[t,j] < 0 marks a slot whose expert
 *  lives on another GPU; it is skipped entirely (no row read, no normalisation, no FMA).
 *      partial[t,:] = +0; for j ascending with idx[t,j] >= 0:
 *          partial = fmaf(w[t,j], row_j (per-expert normalised as in the finalize), partial)
 *
 *  ep_combine (on the token's owner, after the exchange): the G ranks' partials of a token
 *  are added in ascending rank order from +0 (fixed order, so the result is deterministic),
 *  then the residual add and the final RMSNorm exactly as in the finalize:
 *      acc = +0; for g = 0..G-1: acc = acc + partials[g][t,:]        (float32 adds)
 *      residual_out = residual + acc;  out = bf16(residual_out * rms_scale * gamma)
 * With one rank holding every expert, the two steps give exactly the finalize's results.
 */
int oracle_moe_finalize_ep_partial(const uint16_t* expert_rows, int64_t num_rows,
                                   const int32_t* idx, const float* weights,
                                   const int32_t* expert_ids, const uint16_t* expert_gamma,
                                   int32_t num_experts, float eps, float* partial, int64_t T,
                                   int32_t H, int32_t k) {
    float* row = (float*)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
    if (!row) return -2;
    int status = 0;
    for (int64_t t = 0; t < T; ++t) {
        float* acc = partial + t * (int64_t)H;
        for (int32_t h = 0; h < H; ++h) acc[h] = 0.0f;
        for (int32_t j = 0; j < k; ++j) {
            int64_t p = idx[t * k + j];
            if (p < 0) continue; /* another GPU's expert */
            if (p >= num_rows) {
                status = -1;
                goto done;
            }
            const uint16_t* x = expert_rows + p * (int64_t)H;
            if (expert_gamma) {
                int32_t e = expert_ids[t * k + j];
                if (e < 0 || e >= num_experts) {
                    status = -1;
                    goto done;
                }
                const uint16_t* ge = expert_gamma + (int64_t)e * H;
                double s = rms_scale_bf16(x, H, eps);
                for (int32_t h = 0; h < H; ++h)
                    row[h] = (float)(bf16_value(x[h]) * s * bf16_value(ge[h]));
            } else {
                for (int32_t h = 0; h < H; ++h) row[h] = (float)bf16_value(x[h]);
            }
            float wj = weights[t * k + j];
            for (int32_t h = 0; h < H; ++h) acc[h] = fmaf(wj, row[h], acc[h]);
        }
    }
done:
    free(row);
    return status;
}

int oracle_moe_finalize_ep_combine(const float* partials, int32_t num_ranks,
                                   const float* residual, float* residual_out,
                                   const uint16_t* gamma, float eps, uint16_t* out, int64_t T,
                                   int32_t H) {
    float* acc = (float*)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
    if (!acc) return -2;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) acc[h] = 0.0f;
        for (int32_t g = 0; g < num_ranks; ++g) {
            const float* pg = partials + ((int64_t)g * T + t) * (int64_t)H;
            for (int32_t h = 0; h < H; ++h) acc[h] = acc[h] + pg[h];
        }
        const float* res = residual + t * (int64_t)H;
        float* r = residual_out + t * (int64_t)H;
        for (int32_t h = 0; h < H; ++h) r[h] = res[h] + acc[h];
        double s = rms_scale_f32(r, H, eps);
        uint16_t* o = out + t * (int64_t)H;
        for (int32_t h = 0; h < H; ++h) o[h] = bf16_round((double)r[h] * s * bf16_value(gamma[h]));
    }
    free(acc);
    return 0;
}

/*
 * Gated-residual RMSNorm (PR #6544 page, section 1.1): gating, the residual add and
 * RMSNorm in one pass over an FP32 residual stream.
 *     residual_out = float32(residual + sigmoid(gate) * x)     (one rounding)
 *     out = bf16(residual_out * rms_scale(residual_out) * gamma)
 */
int oracle_gated_residual_rmsnorm(const uint16_t* x, const uint16_t* gate, const float* residual,
                                  float* residual_out, const uint16_t* gamma, float eps,
                                  uint16_t* out, int64_t T, int32_t H) {
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* xt = x + t * (int64_t)H;
        const uint16_t* gt = gate + t * (int64_t)H;
        const float* res = residual + t * (int64_t)H;
        float* r = residual_out + t * (int64_t)H;
        for (int32_t h = 0; h < H; ++h)
            r[h] = (float)((double)res[h] + sigmoid(bf16_value(gt[h])) * bf16_value(xt[h]));
        double s = rms_scale_f32(r, H, eps);
        uint16_t* o = out + t * (int64_t)H;
        for (int32_t h = 0; h < H; ++h) o[h] = bf16_round((double)r[h] * s * bf16_value(gamma[h]));
    }
    return 0;
}

/*
 * Gated-residual dual RMSNorm, "gated_residual_next_rmsnorm": the PR #6544 page names it in its
 * Fixed-Width Fused Norms docs and calls it a "gated residual dual norm" in section 2.2, but
 * never defines it.  Reading taken: the gated residual of section 1.1 feeds two RMSNorm outputs
 * that share one mean square, this layer's (gamma) and the next layer's pre-norm (gamma_next):
 *     r        = fp32(residual + sigmoid(gate) * x)                  (one rounding, as above)
 *     out      = bf16(r * rms_scale(r) * gamma)
 *     out_next = bf16(r * rms_scale(r) * gamma_next)
 * The arithmetic under this reading is pinned by the tests; the reading itself is not fixed by
 * the pages (parity unpinned as to what the pages mean).
 */
int oracle_gated_residual_next_rmsnorm(const uint16_t* x, const uint16_t* gate,
                                       const float* residual, float* residual_out,
                                       const uint16_t* gamma, const uint16_t* gamma_next,
                                       float eps, uint16_t* out, uint16_t* out_next, int64_t T,
                                       int32_t H) {
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* xt = x + t * (int64_t)H;
        const uint16_t* gt = gate + t * (int64_t)H;
        const float* res = residual + t * (int64_t)H;
        float* r = residual_out + t * (int64_t)H;
        for (int32_t h = 0; h < H; ++h)
            r[h] = (float)((double)res[h] + sigmoid(bf16_value(gt[h])) * bf16_value(xt[h]));
        double s = rms_scale_f32(r, H, eps);
        uint16_t* o = out + t * (int64_t)H;
        uint16_t* on = out_next + t * (int64_t)H;
        for (int32_t h = 0; h < H; ++h) {
            o[h] = bf16_round((double)r[h] * s * bf16_value(gamma[h]));
            on[h] = bf16_round((double)r[h] * s * bf16_value(gamma_next[h]));
        }
    }
    return 0;
}

/*
 * MXFP4 block quantisation: the PR #6544 page's RMSNorm + block-scaled FP4 quantisation
 * (section 2.3; NVFP4 there), retargeted to the OCP Microscaling (MX) format, whose published
 * definition is taken here because the pages do not define the format: blocks of 32
 * consecutive values along a row share one E8M0 scale X = 2^e; each value is stored as
 * E2M1 (sign, 2 exponent bits, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
 *     e = floor(log2(max_i |v_i|)) - 2         (2 = the largest E2M1 exponent), clamped to
 *                                               [-127, 127]; an all-zero block takes e = -127
 *     scale code = e + 127                      (one byte per block)
 *     code_i = E2M1 nearest to v_i / 2^e, ties to the even code, |.| above 6 saturating to 6;
 *              the sign bit follows v_i, also for zeros
 * Two codes per byte, the even-indexed value in the low nibble.
 */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static uint8_t e2m1_code(double v) {
    const uint8_t sign = signbit(v) ? 8 : 0;
    const double m = fabs(v);
    if (m >= 6.0) return sign | 7;
    uint8_t best = 0;
    for (uint8_t c = 1; c < 8; ++c) {
        const double d = fabs(m - kE2M1[c]), db = fabs(m - kE2M1[best]);
        if (d < db || (d == db && (c & 1) == 0)) best = c; /* ties: the even code */
    }
    return sign | best;
}

static int mx_block_exponent(const double* v) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[i]));
    if (amax == 0.0) return -127;
    int e2;
    frexp(amax, &e2); /* amax = m * 2^e2, m in [0.5, 1): floor(log2(amax)) = e2 - 1 */
    int e = e2 - 1 - 2;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

static void mx_quantize_row(const double* v, int32_t H, uint8_t* q, uint8_t* scales) {
    for (int32_t b = 0; b < H / 32; ++b) {
        const double* blk = v + b * 32;
        const int e = mx_block_exponent(blk);
        scales[b] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; i += 2) {
            const uint8_t lo = e2m1_code(ldexp(blk[i], -e)); /* exact: a power-of-two scale */
            const uint8_t hi = e2m1_code(ldexp(blk[i + 1], -e));
            q[(b * 32 + i) / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

/* fp32 values [T, H] (H a multiple of 32) -> codes [T, H/2] and scale codes [T, H/32]. */
int oracle_mxfp4_quantize(const float* x, int64_t T, int32_t H, uint8_t* q, uint8_t* scales) {
    double* v = (double*)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
    if (!v) return -2;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) v[h] = (double)x[t * (int64_t)H + h];
        mx_quantize_row(v, H, q + t * (int64_t)(H / 2), scales + t * (int64_t)(H / 32));
    }
    free(v);
    return 0;
}

/*
 * RMSNorm, then MXFP4 (the same page's section 2.3 without the all-gather):
 *     y = fp32(x * rms_scale(x) * gamma)   (float64, rounded once to float32: the quantisation
 *                                           decision is taken on float32 values, the
 *                                           precision the kernel works in)
 *     (q, scales) = mxfp4(y)
 */
int oracle_rmsnorm_mxfp4_quantize(const uint16_t* x, const uint16_t* gamma, float eps,
                                  uint8_t* q, uint8_t* scales, int64_t T, int32_t H) {
    double* v = (double*)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
    if (!v) return -2;
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* xt = x + t * (int64_t)H;
        double s = rms_scale_bf16(xt, H, eps);
        for (int32_t h = 0; h < H; ++h)
            v[h] = (double)(float)(bf16_value(xt[h]) * s * bf16_value(gamma[h]));
        mx_quantize_row(v, H, q + t * (int64_t)(H / 2), scales + t * (int64_t)(H / 32));
    }
    free(v);
    return 0;
}

/*
 * The same on fp32 rows (the finalize's residual_out): the MXFP4 epilogue of the finalize,
 * whose normalised output is quantised instead of rounded to bf16.
 *     y = fp32(r * rms_scale(r) * gamma);   (q, scales) = mxfp4(y)
 */
int oracle_rmsnorm_f32_mxfp4_quantize(const float* r, const uint16_t* gamma, float eps,
                                      uint8_t* q, uint8_t* scales, int64_t T, int32_t H) {
    double* v = (double*)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
    if (!v) return -2;
    for (int64_t t = 0; t < T; ++t) {
        const float* rt = r + t * (int64_t)H;
        double s = rms_scale_f32(rt, H, eps);
        for (int32_t h = 0; h < H; ++h)
            v[h] = (double)(float)((double)rt[h] * s * bf16_value(gamma[h]));
        mx_quantize_row(v, H, q + t * (int64_t)(H / 2), scales + t * (int64_t)(H / 32));
    }
    free(v);
    return 0;
}

/*
 * Per-head RMSNorm with a sigmoid gate (same page, section 1.2): every head of every token
 * is normalised over its D values with one gamma[D] shared by all heads, then multiplied by
 * the sigmoid of the gate element.
 *     out[t,n,d] = bf16(x[t,n,d] * rms_scale(x[t,n,:]) * gamma[d] * sigmoid(gate[t,n,d]))
 */
int oracle_rmsnorm_sigmoid_gate(const uint16_t* x, const uint16_t* gate, const uint16_t* gamma,
                                float eps, uint16_t* out, int64_t T, int32_t num_heads,
                                int32_t D) {
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t n = 0; n < num_heads; ++n) {
            int64_t base = (t * num_heads + n) * (int64_t)D;
            double s = rms_scale_bf16(x + base, D, eps);
            for (int32_t d = 0; d < D; ++d)
                out[base + d] = bf16_round(bf16_value(x[base + d]) * s * bf16_value(gamma[d]) *
                                           sigmoid(bf16_value(gate[base + d])));
        }
    }
    return 0;
}

/* Round float64 values to bfloat16 bit patterns; lets the tests pin the rounding itself. */
void oracle_bf16_round(const double* v, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(v[i]);
}

/*
 * MoE routing and the expert-sorted permutation: the inputs the finalize consumes.
 *
 * Per token t (logits[t, 0..E-1]):
 *   expert_ids[t, j], j = 0..k-1: the experts of the k largest logits, largest first; equal
 *     logits go to the lower expert id;
 *   weights[t, j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected logits (a
 *     softmax over the top k), in float64, rounded once to float32.
 * Over all slots s = t*k + j (the flattened order), a stable sort by expert id gives the
 * contiguous grouped-GEMM layout (page "FlashInfer: fused kernels and an optimised scheduler
 * for MoE", PR #4130, the m_indptr / token_offset arguments of its grouped GEMM):
 *   offsets[e] = number of slots routed to experts < e, offsets[E] = T*k;
 *   perm[p] = the slot stored at permuted row p (rows grouped by expert, slots ascending);
 *   idx[s] = the permuted row of slot s, so idx[perm[p]] = p.
 * Returns 0, or -2 if scratch memory cannot be allocated.
 */
int oracle_moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* expert_ids,
                     float* weights, int32_t* idx, int32_t* perm, int32_t* offsets) {
    unsigned char* taken = (unsigned char*)malloc((size_t)(E > 0 ? E : 1));
    int64_t* cursor = (int64_t*)malloc(sizeof(int64_t) * (size_t)(E > 0 ? E : 1));
    double* ex = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    if (!taken || !cursor || !ex) {
        free(taken);
        free(cursor);
        free(ex);
        return -2;
    }
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * (int64_t)E;
        for (int32_t e = 0; e < E; ++e) taken[e] = 0;
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;  /* ties keep the lower id */
            taken[best] = 1;
            expert_ids[t * k + j] = best;
        }
        double top = (double)l[expert_ids[t * k]];
        double sum = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            ex[j] = exp((double)l[expert_ids[t * k + j]] - top);
            sum += ex[j];
        }
        for (int32_t j = 0; j < k; ++j) weights[t * k + j] = (float)(ex[j] / sum);
    }
    /* counting sort of the slots by expert id, stable in slot order */
    for (int32_t e = 0; e < E; ++e) cursor[e] = 0;
    for (int64_t s = 0; s < T * k; ++s) cursor[expert_ids[s]] += 1;
    int64_t run = 0;
    for (int32_t e = 0; e < E; ++e) {
        int64_t c = cursor[e];
        offsets[e] = (int32_t)run;
        cursor[e] = run;
        run += c;
    }
    offsets[E] = (int32_t)run;
    for (int64_t s = 0; s < T * k; ++s) {
        int64_t p = cursor[expert_ids[s]]++;
        idx[s] = (int32_t)p;
        perm[p] = (int32_t)s;
    }
    free(taken);
    free(cursor);
    free(ex);
    return 0;
}
