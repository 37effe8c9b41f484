/*
 * adaln.h -- C ABI of libadaln: fused adaLN normalisation for AMD MI355X (gfx950).
 *
 * Five compute entry points fuse a row normalisation (LayerNorm without
 * affine parameters, or RMSNorm with an optional weight) with the adaLN
 * modulate epilogue  y = norm(x) * (1 + scale[b]) + shift[b]  that diffusion
 * transformers run at every adaLN site, optionally preceded by the residual-gate
 * prologue  r = res + gate[b] * x (for both norms), or followed, for the
 * LayerNorm, by a static FP8 quantisation of y.  A sixth normalises the attention
 * heads of Q and K and applies the rotary embedding (adaln_qk_rmsnorm_rope); a
 * seventh applies the residual gate to a channel-first residual stream.
 *
 * Sources, cited by page title and section:
 *  - FLUX.1 PR report "route the adaLN LN+modulate sites through the bit-exact
 *    fused LayerNorm+modulate kernel" (sglang #34126): the LayerNorm+modulate
 *    operation (source snippet of flux.py), its eager semantics (test snippet,
 *    `_eager`: LayerNorm(hidden, eps=1e-6, elementwise_affine=False), then
 *    norm(x) * (1 + scale[:, None]) + shift[:, None]), the site shapes and the
 *    strided `emb.chunk` modulation views, and the kernel contract
 *    (implementation item 4; related PRs: hidden % 4 == 0, hidden <= 8192).
 *  - ERNIE-Image PR report "fused RMSNorm+scale/shift bit-exact kernel"
 *    (sglang #33854): the RMSNorm+scale/shift operation and its residual-gate
 *    variant that also returns the residual stream (implementation items 1-2).
 *  - sglang diffusion kernels guide, "selection matrix / Norm + scale/shift":
 *    the rounding points of the chain and of the residual variant; "directory
 *    layout / kernel registry": the scale_residual_norm_scale_shift operator
 *    (residual gate + norm + scale/shift) that the LayerNorm gated entry point
 *    provides; "entry-point protocol": unsupported input raises (here: returns
 *    a status), it never degrades silently.
 *  - FLUX.1 PR report, related PRs: the FLUX.1 bit-exact residual-gate fast path
 *    (#33819) beside the LN+modulate sites.
 *  - kernels guide, "data movement and quantised layout producers":
 *    fused_layernorm_modulate_fp8_quant_raw folds FLUX.2's LayerNorm, adaLN
 *    modulate and static FP8 quantisation into one kernel; Qwen PR report
 *    (modelopt_quant.py snippet): ModelOpt FP8 checkpoints use E4M3 (e4m3fn) with
 *    a per-tensor static input scale.
 *  - Batch-invariance article (vLLM), section 3 (RMSNorm): the reduction layout
 *    depends on the hidden size only, never on the number of rows.
 *
 * Numerics (identical bits on every call, for every batch composition):
 *   every binary32 operation is rounded to nearest-even with no FMA
 *   contraction; sqrt and divide are correctly rounded; denormals are kept.
 *   The reduction order is a function of H only:
 *     W = 1 wave (64 lanes) per row if H < 2048, 2 waves if H < 4096, else 4;
 *     P = 64W lanes; C = ceil(H / 8P) chunks; lane t owns the columns
 *     b*8P + 8t + v (b < C, v < 8) and visits them b-major, v-minor;
 *     lane partials are folded by a butterfly over the lane index with distances
 *     1, 2, ..., P/2, each step combining (partial of lane t&~k, partial of
 *     lane t|k) in that order.
 *   RMS statistic: s = s + RN(x*x) per lane, fold by +; rstd =
 *     RN(1 / RN(sqrt(RN(RN(S / H) + eps)))).
 *   LN statistic: per-lane Welford with the count's rounded reciprocal
 *     (mean += RN(d * RN(1/n)), M2 += RN(d * RN(x - mean))), folded by the
 *     Chan pairwise combine; var = RN(M2 / H); rstd as for RMS.
 *   Norm output (bf16, rounded once): LN RN(RN(x - mean) * rstd);
 *     RMS RN(RN(x * rstd) * RN(w + 0)).
 *   Modulate: a = bf16(1 + scale); p = bf16(yn * a); y = bf16(p + shift).
 *   Residual gate: g = bf16(gate * x); r = bf16(res + g); r feeds the norm.
 *   FP8 quantisation: inv = RN(1 / qscale); q = E4M3(clamp(RN(y * inv), -448, 448))
 *     with nearest-even rounding into the OCP E4M3 format (bias 7, subnormals, no
 *     infinity, largest finite 448); a NaN y gives a NaN code.
 *
 * Conventions shared by all entry points:
 *  - Tensors are raw bf16 bit patterns (adaln_bf16).  x, res, y, r are
 *    contiguous row-major [B, T, H]; row index = b*T + t.
 *  - Per-batch vectors scale / shift / gate have unit inner stride; row b starts
 *    at ptr + b * <name>_bstride elements.  A batch stride of 0 shares one
 *    vector across the batch; otherwise it must be >= H.  Views such as
 *    emb.chunk(k, dim=1) of a [B, k*H] embedding are accepted without a copy.
 *    weight is a contiguous [H] vector; NULL means a weight of one.
 *  - Requirements: 8 <= H <= 8192, H % 8 == 0 (16-byte vectors of 8 bf16);
 *    every pointer 16-byte aligned; batch strides >= 0 and % 8 == 0; B, T >= 0;
 *    eps finite and >= 0.  B*T == 0 is a successful no-op (pointers unchecked).
 *  - Outputs (y, r, q) may not overlap any input or each other.
 *  - Ownership: the caller owns every buffer; the library never allocates,
 *    frees or synchronises.  Work is enqueued on `hip_stream` (a hipStream_t;
 *    NULL = the null stream) of the current device; pointers must be device
 *    memory of that device.
 *  - Errors: a non-OK status is returned before anything is launched, so the
 *    outputs are untouched.  ADALN_ERR_LAUNCH reports a failed launch (for
 *    example no gfx950 device).  Thread-safe and reentrant: the only global state
 *    is a mutex-guarded cache of occupancy queries per kernel and device.
 */
#ifndef ADALN_H
#define ADALN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ADALN_ABI_VERSION 11 /* 2: two waves per row for 2048 <= H < 4096;
                              3: residual-gate LayerNorm, stream copy;
                              4: LayerNorm + modulate + FP8 quantisation;
                              5: per-head QK RMSNorm + RoPE;
                              6: channel-first residual gating;
                              7: launch-plan diagnostic;
                              8: the plan takes T and gives row blocks; the finalize
                                 diagnostic takes H;
                              9: streaming read / fill / copy measurement kernels;
                                 the plan diagnostic takes every resident count and
                                 the CU count and reports the ring; the device's own
                                 plan;
                             10: the plan diagnostics take and report a fourth
                                 resident count, of the one-slot ring on interleaved
                                 rows that large RMS launches take;
                             11: large launches take a one-shot grid; the plan
                                 diagnostics take and report three resident counts
                                 again, ring kinds 0-2 */

typedef uint16_t adaln_bf16; /* raw bfloat16 bits */

typedef enum adaln_status {
    ADALN_OK = 0,
    ADALN_ERR_NULL = 1,    /* a required pointer is NULL */
    ADALN_ERR_SHAPE = 2,   /* H outside [8, 8192] or H % 8 != 0, B < 0, T < 0, size overflow */
    ADALN_ERR_ALIGN = 3,   /* a pointer is not 16-byte aligned */
    ADALN_ERR_STRIDE = 4,  /* a batch stride is negative, not % 8, or in (0, H) */
    ADALN_ERR_OVERLAP = 5, /* an output overlaps an input or the other output */
    ADALN_ERR_VALUE = 6,   /* eps is negative or not finite */
    ADALN_ERR_LAUNCH = 7   /* the HIP launch failed */
} adaln_status;

/* y = LayerNorm(x) * (1 + scale[b]) + shift[b]; LayerNorm without affine
 * parameters, biased variance (FLUX.1 PR report, flux.py and test snippets). */
adaln_status adaln_layernorm_modulate(const adaln_bf16* x, const adaln_bf16* scale,
                                      const adaln_bf16* shift, adaln_bf16* y, int64_t B, int64_t T,
                                      int64_t H, int64_t scale_bstride, int64_t shift_bstride,
                                      float eps, void* hip_stream);

/* y = RMSNorm(x) * (1 + scale[b]) + shift[b]; RMSNorm(x) = x * rstd * w, with
 * weight NULL meaning w = 1 (ERNIE-Image PR report, kernel snippet). */
adaln_status adaln_rmsnorm_scale_shift(const adaln_bf16* x, const adaln_bf16* weight,
                                       const adaln_bf16* scale, const adaln_bf16* shift,
                                       adaln_bf16* y, int64_t B, int64_t T, int64_t H,
                                       int64_t scale_bstride, int64_t shift_bstride, float eps,
                                       void* hip_stream);

/* r = res + gate[b] * x (written to r_out), then
 * y = RMSNorm(r) * (1 + scale[b]) + shift[b] (ERNIE-Image PR report,
 * implementation item 2: the gated site returns the bit-identical residual). */
adaln_status adaln_residual_gate_rmsnorm_scale_shift(
    const adaln_bf16* res, const adaln_bf16* x, const adaln_bf16* gate, const adaln_bf16* weight,
    const adaln_bf16* scale, const adaln_bf16* shift, adaln_bf16* r_out, adaln_bf16* y, int64_t B,
    int64_t T, int64_t H, int64_t gate_bstride, int64_t scale_bstride, int64_t shift_bstride,
    float eps, void* hip_stream);

/* r = res + gate[b] * x (written to r_out), then
 * y = LayerNorm(r) * (1 + scale[b]) + shift[b] with the LayerNorm of
 * adaln_layernorm_modulate (kernels guide: the residual variant feeds the rounded
 * r to the same norm; scale_residual_norm_scale_shift in the kernel registry). */
adaln_status adaln_residual_gate_layernorm_modulate(
    const adaln_bf16* res, const adaln_bf16* x, const adaln_bf16* gate, const adaln_bf16* scale,
    const adaln_bf16* shift, adaln_bf16* r_out, adaln_bf16* y, int64_t B, int64_t T, int64_t H,
    int64_t gate_bstride, int64_t scale_bstride, int64_t shift_bstride, float eps,
    void* hip_stream);

/* q = E4M3(clamp(RN(y * RN(1 / *qscale)), -448, 448)) with y the output of
 * adaln_layernorm_modulate (bf16, never written to memory): one byte per element,
 * q contiguous [B, T, H], 16-byte aligned.  qscale points to one float in device
 * memory (the static per-tensor input scale of an FP8 checkpoint), 4-byte aligned;
 * it is read on the device, so its value is not validated: a zero, negative or
 * non-finite scale gives whatever the formula gives.  (kernels guide:
 * fused_layernorm_modulate_fp8_quant_raw) */
adaln_status adaln_layernorm_modulate_fp8_quant(const adaln_bf16* x, const adaln_bf16* scale,
                                                const adaln_bf16* shift, const float* qscale,
                                                uint8_t* q, int64_t B, int64_t T, int64_t H,
                                                int64_t scale_bstride, int64_t shift_bstride,
                                                float eps, void* hip_stream);

/* Per-head QK RMSNorm + interleaved (non-NeoX) rotary embedding, head_dim 128
 * (kernels guide, RoPE / QK-norm; Qwen PR report, implementation item 3 and the
 * qwen_image.py snippet: Q/K RMSNorm with their weights, then RoPE from an fp32
 * cos/sin cache, Q/K as strided views of the packed QKV projection).  Per head
 * vector x of Q (weight q_weight) or K (weight k_weight):
 *   yn = bf16(RN(RN(x * rstd) * RN(w + 0))), rstd the RMS statistic above with H = 128;
 *   out[2i]   = bf16(RN(RN(a*c) - RN(b*s))), out[2i+1] = bf16(RN(RN(b*c) + RN(a*s)))
 *   with a = yn[2i], b = yn[2i+1], c = cos_sin[t][i], s = cos_sin[t][64 + i].
 * Layout: Q head h of token t at q + t*q_token_stride + h*128 (elements; heads
 * contiguous, token stride >= heads_q*128 and % 8 == 0 when tokens > 1); K likewise;
 * cos_sin fp32 [tokens, 128] contiguous (cos of the 64 pairs, then their sin);
 * q_out [tokens, heads_q, 128] and k_out [tokens, heads_k, 128] contiguous; weights
 * [128] bf16 or NULL (one).  head_dim other than 128, or more than 2^23 - 8 heads
 * on a side, is ADALN_ERR_SHAPE; heads_q or heads_k may be 0 (that tensor's pointers
 * are then unused). */
adaln_status adaln_qk_rmsnorm_rope(const adaln_bf16* q, const adaln_bf16* k,
                                   const adaln_bf16* q_weight, const adaln_bf16* k_weight,
                                   const float* cos_sin, adaln_bf16* q_out, adaln_bf16* k_out,
                                   int64_t tokens, int64_t heads_q, int64_t heads_k,
                                   int64_t head_dim, int64_t q_token_stride,
                                   int64_t k_token_stride, float eps, void* hip_stream);

/* Residual gating on the channel-first layout (kernels guide, norm variants /
 * residual gating: the transposed dense path keeps the residual and the output in
 * their [B, hidden, tokens] layout and reads the update in its row-major order,
 * with no .contiguous() copy):
 *   out[b][h][t] = bf16(res[b][h][t] + bf16(gate[b][h] * update[b][t][h]))
 * res, out: contiguous [B, H, T]; update: contiguous [B, T, H]; gate row b at
 * gate + b*gate_bstride (0 shares one vector; else >= H and % 8 == 0).  Any T >= 0;
 * H % 8 == 0; one workgroup of 256 per tile of 64 hidden rows and 64 tokens (each
 * row's tiles start on a 128-byte line of the flat tensor, so with T % 64 != 0 they
 * cover T + 63 tokens), at most 2^24 - 8 tiles (ADALN_ERR_SHAPE otherwise);
 * pointers 16-byte aligned.  out may be
 * res itself (in-place update); any other overlap is ADALN_ERR_OVERLAP. */
adaln_status adaln_residual_gate_channel_first(const adaln_bf16* res, const adaln_bf16* update,
                                               const adaln_bf16* gate, adaln_bf16* out, int64_t B,
                                               int64_t T, int64_t H, int64_t gate_bstride,
                                               void* hip_stream);

/* Predicates: the validation of the entry point of the same name, without a
 * launch (the `can_use_*` predicate of the kernels guide's entry-point protocol).
 * They never touch the GPU. */
adaln_status adaln_check_layernorm_modulate(const adaln_bf16* x, const adaln_bf16* scale,
                                            const adaln_bf16* shift, const adaln_bf16* y,
                                            int64_t B, int64_t T, int64_t H,
                                            int64_t scale_bstride, int64_t shift_bstride,
                                            float eps);
adaln_status adaln_check_rmsnorm_scale_shift(const adaln_bf16* x, const adaln_bf16* weight,
                                             const adaln_bf16* scale, const adaln_bf16* shift,
                                             const adaln_bf16* y, int64_t B, int64_t T, int64_t H,
                                             int64_t scale_bstride, int64_t shift_bstride,
                                             float eps);
adaln_status adaln_check_residual_gate_rmsnorm_scale_shift(
    const adaln_bf16* res, const adaln_bf16* x, const adaln_bf16* gate, const adaln_bf16* weight,
    const adaln_bf16* scale, const adaln_bf16* shift, const adaln_bf16* r_out,
    const adaln_bf16* y, int64_t B, int64_t T, int64_t H, int64_t gate_bstride,
    int64_t scale_bstride, int64_t shift_bstride, float eps);

adaln_status adaln_check_residual_gate_layernorm_modulate(
    const adaln_bf16* res, const adaln_bf16* x, const adaln_bf16* gate, const adaln_bf16* scale,
    const adaln_bf16* shift, const adaln_bf16* r_out, const adaln_bf16* y, int64_t B, int64_t T,
    int64_t H, int64_t gate_bstride, int64_t scale_bstride, int64_t shift_bstride, float eps);

adaln_status adaln_check_layernorm_modulate_fp8_quant(const adaln_bf16* x, const adaln_bf16* scale,
                                                      const adaln_bf16* shift, const float* qscale,
                                                      const uint8_t* q, int64_t B, int64_t T,
                                                      int64_t H, int64_t scale_bstride,
                                                      int64_t shift_bstride, float eps);

adaln_status adaln_check_qk_rmsnorm_rope(const adaln_bf16* q, const adaln_bf16* k,
                                         const adaln_bf16* q_weight, const adaln_bf16* k_weight,
                                         const float* cos_sin, const adaln_bf16* q_out,
                                         const adaln_bf16* k_out, int64_t tokens,
                                         int64_t heads_q, int64_t heads_k, int64_t head_dim,
                                         int64_t q_token_stride, int64_t k_token_stride,
                                         float eps);

adaln_status adaln_check_residual_gate_channel_first(const adaln_bf16* res,
                                                     const adaln_bf16* update,
                                                     const adaln_bf16* gate, const adaln_bf16* out,
                                                     int64_t B, int64_t T, int64_t H,
                                                     int64_t gate_bstride);

/* The fixed reduction layout for H: waves per row, lanes per row, chunks per
 * lane.  ADALN_ERR_SHAPE for an unsupported H; out-pointers may be NULL. */
adaln_status adaln_reduction_layout(int64_t H, int* waves_per_row, int* lanes_per_row,
                                    int* chunks_per_lane);

/* Static English text for a status (never NULL). */
const char* adaln_status_string(adaln_status status);

/* ADALN_ABI_VERSION of the built library. */
int adaln_abi_version(void);

/* Diagnostics: run the exact device steps the kernels use, elementwise, so that
 * tests can check them exhaustively against host IEEE arithmetic.
 *  - adaln_diag_round_bf16: out[i] = bf16(in[i]) (nearest-even).
 *  - adaln_diag_finalize:   out[i] = RN(1 / RN(sqrt(RN(RN(in[i] / H) + eps)))), the
 *    rstd of a row of H elements whose statistic (sum of squares or M2) is in[i],
 *    by the kernels' own code (including its shortcuts for in-range waves);
 *    1 <= H <= 8192 (else ADALN_ERR_SHAPE).
 * n >= 0 elements of device memory, 4-byte aligned; ADALN_ERR_* as above.  out may
 * not overlap in (ADALN_ERR_OVERLAP), except that finalize may run in place. */
adaln_status adaln_diag_round_bf16(const float* in, adaln_bf16* out, int64_t n, void* hip_stream);
adaln_status adaln_diag_finalize(const float* in, float* out, int64_t n, int64_t H, float eps,
                                 void* hip_stream);

/* Diagnostic: the FP8 kernel's quantisation step on binary32 inputs,
 * out[i] = E4M3(clamp(RN(in[i] * RN(1 / *qscale)), -448, 448)).  n >= 0 and
 * n % 4 == 0 (ADALN_ERR_SHAPE); in 16-byte aligned, out and qscale 4-byte aligned;
 * device memory; out may not overlap in or *qscale (ADALN_ERR_OVERLAP). */
adaln_status adaln_diag_quant_fp8(const float* in, uint8_t* out, int64_t n, const float* qscale,
                                  void* hip_stream);

/* Diagnostic: the row-group plan of one launch of a fused entry point, computed on
 * the host with no device work, for given counts of what fits on the device at once.
 * op: 0 LayerNorm+modulate, 1 RMSNorm+scale/shift, 2 residual gate + RMSNorm,
 * 3 residual gate + LayerNorm, 4 LayerNorm+modulate+FP8.  resident[3]: row groups
 * resident at once with the default ring, with the one-slot ring and with the
 * two-row ring (0: not available; resident[0] >= 1); cus: compute units (0: unknown;
 * the two-row ring is chosen only with it).  rows = B*T >= 1 with 1 <= T <= rows and
 * rows % T == 0 (else ADALN_ERR_SHAPE, also for a plan whose grid would pass 2^32
 * work-items, which needs rows of more than 2^55 bytes), H as for the entry points.
 * out[11] receives {one-slot ring (0/1), ring slots, ring kind (0 default depth,
 * 1 one slot, 2 two rows), groups, groups per block, rows per block, group stride,
 * step, span, workgroups, threads per workgroup}: with k = g / (groups per block) and
 * first =
 * k * (rows per block) + (g % groups per block) * stride, group g takes the rows
 * first + i*step below min(first + span, (k + 1) * (rows per block), rows).  A launch
 * of at least 2^25 elements (rows * H) of ops 0-3 takes a one-shot grid: the default
 * ring, group g the rows g*span .. g*span + span - 1, span the ring depth (or a
 * multiple of it when the grid would otherwise pass 2^32 work-items), and as many
 * groups as that takes, whatever the resident counts.
 * ADALN_ERR_VALUE for an unknown op or a resident count or cus below 0 or above
 * 2^31 - 1 (resident[0] below 1); ADALN_ERR_NULL for a NULL resident or out. */
adaln_status adaln_diag_launch_plan(int op, int64_t rows, int64_t H, int64_t T,
                                    const int64_t* resident, int64_t cus, int64_t* out);

/* Diagnostic: the plan a launch takes on the current device, from the same
 * occupancy queries (cached per kernel and device), with nothing launched; weight:
 * nonzero when the RMS weight is given (ops 1 and 2; it selects the kernel whose
 * occupancy is queried).  out[11] as above; resident_out[3] and *cus_out (each may be
 * NULL) receive the counts it used.  ADALN_ERR_LAUNCH when the queries fail (for
 * example no gfx950 device). */
adaln_status adaln_diag_device_plan(int op, int64_t rows, int64_t H, int64_t T, int weight,
                                    int64_t* out, int64_t* resident_out, int64_t* cus_out);

/* Measurement aid: copy `bytes` bytes of device memory from src to dst with the
 * fused kernels' access style (16-byte non-temporal loads and stores), so that the
 * attainable streaming rate of the device can be timed beside the fused kernels.
 * bytes >= 0 and % 16 == 0 (else ADALN_ERR_SHAPE); both pointers 16-byte aligned
 * (ADALN_ERR_ALIGN); the ranges may not overlap (ADALN_ERR_OVERLAP).  The same as
 * adaln_diag_stream(0, src, dst, bytes, 8, hip_stream). */
adaln_status adaln_diag_stream_copy(const void* src, void* dst, int64_t bytes, void* hip_stream);

/* Measurement aid: the streaming kernels behind the measured ceilings, with
 * vectors_per_thread (1, 2, 4, 8 or 16; else ADALN_ERR_VALUE) 16-byte vectors in
 * flight per thread, one-shot grids of 256 threads.
 *  kind 0 (copy): dst[0, bytes) = src[0, bytes);
 *  kind 1 (read): reads src[0, bytes) and writes 4 bytes per 1024*vectors_per_thread
 *                 bytes read (a fold of the data, so that no load is dropped) to the
 *                 start of dst, which must hold `bytes` bytes;
 *  kind 2 (fill): writes a fixed pattern to dst[0, bytes); src is unused.
 * bytes >= 0 and % 16 == 0 (ADALN_ERR_SHAPE); pointers used are non-NULL and
 * 16-byte aligned; the bytes written may not overlap src (ADALN_ERR_OVERLAP);
 * kind outside 0..2 is ADALN_ERR_VALUE.  Device memory of the current device. */
adaln_status adaln_diag_stream(int kind, const void* src, void* dst, int64_t bytes,
                               int vectors_per_thread, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* ADALN_H */
