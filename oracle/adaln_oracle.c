/*
 * adaln_oracle.c -- plain, slow CPU oracle for the fused adaLN normalisation path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file defines, one scalar operation at a time,
 * the exact bits the HIP library must produce.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the product path never
 * does.  It shares no code, header, table or helper with the HIP library.
 *
 * Sources (cited by page title and section; the pages are sglang / vLLM write-ups):
 *  - "FLUX.1: route the adaLN LN+modulate sites through the bit-exact fused
 *    LayerNorm+modulate kernel" (sglang PR #34126 report), test snippet `_eager`
 *    and the LayerNorm module it builds: LayerNorm without affine parameters,
 *    eps 1e-6, then norm(x) * (1 + scale[:, None]) + shift[:, None] in bf16 eager ops.
 *  - "sglang.kernels.ops.diffusion complete guide", section "selection matrix /
 *    Norm + scale/shift": per-thread column ownership with v fastest then b, each
 *    square rounded on its own (no FMA), an ordered add chain, an adjacent-pair
 *    butterfly fold, the RMS output rounded once to bf16, then round(1+scale),
 *    round(y*that), round(prod+shift); the residual variant rounds gate*update and
 *    residual+that before the norm.
 *  - "ERNIE-Image fused RMSNorm+scale/shift bit-exact kernel" (sglang PR #33854
 *    report), key source snippet: the same rounding points, the gated variant
 *    returning the residual stream, and 64-bit row addressing.
 *  - Batch-invariance article (vLLM), section 3.1: RMS(x) = sqrt(mean(x^2) + eps);
 *    the reduction layout must depend on the hidden size only, never on the
 *    number of rows.
 *  - FLUX PR report, motivation: LayerNorm statistics by per-element Welford
 *    updates and a count-weighted combine (Welford 1962; Chan, Golub & LeVeque
 *    1979 for the pairwise combine).
 *
 * The fixed order (a function of H only):
 *   W waves of 64 lanes per row: W = 1 if H < 2048, W = 2 if H < 4096, else W = 4.
 *   P = 64*W lanes, C = ceil(H / (8*P)) chunks.  Lane t owns the columns
 *   b*8P + 8t + v (b < C, v < 8, column < H) and visits them b-major, v-minor.
 *   Lane partials are folded by a butterfly over the lane index with distances
 *   1, 2, 4, ..., P/2: at distance k every lane combines the partial of lane
 *   (t & ~k) with the partial of lane (t | k) in that order, so all lanes end
 *   with identical bits.  Distances 64 and 128 are the cross-wave combine
 *   (w0 (+) w1) for two waves, ((w0 (+) w1) (+) (w2 (+) w3)) for four.
 *
 * Every arithmetic step below is one IEEE-754 binary32 operation rounded to
 * nearest-even.  The file must be compiled with -ffp-contract=off and without
 * -ffast-math; the entry points also clear FTZ/DAZ in MXCSR for their duration,
 * so denormals are kept.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>
#include <float.h>
#include <xmmintrin.h>

#if FLT_EVAL_METHOD != 0
#error "the oracle needs float expressions evaluated in binary32"
#endif

#define ORACLE_MAX_LANES 256
#define ORACLE_MAX_H 8192

/* ------------------------------------------------------------------------ */
/* floating-point environment: round to nearest-even, no flush-to-zero       */
/* ------------------------------------------------------------------------ */
static unsigned int fp_enter(void) {
    unsigned int saved = _mm_getcsr();
    /* bit 15 FTZ, bit 6 DAZ, bits 13-14 rounding control (00 = nearest-even) */
    _mm_setcsr(saved & ~(0x8000u | 0x0040u | 0x6000u));
    return saved;
}
static void fp_leave(unsigned int saved) { _mm_setcsr(saved); }

/* ------------------------------------------------------------------------ */
/* bfloat16 <-> binary32                                                     */
/* ------------------------------------------------------------------------ */
/* Exact widening: a bf16 value is the upper half of a binary32 pattern. */
static float widen(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 value to the nearest bf16, ties to even (IEEE-754 RNE on
 * the 8-bit significand).  Working on the magnitude bits: the kept upper half
 * is the value truncated toward zero, the dropped lower half is the remainder
 * in units of 2^-16 of one bf16 ulp; add one ulp when the remainder is above
 * one half, or exactly one half and the kept significand is odd.  A carry into
 * the exponent field is the correct next binade (or infinity).  NaN maps to a
 * quiet NaN with the same sign. */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t sign = u & 0x80000000u;
    uint32_t mag = u & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return (uint16_t)((sign >> 16) | 0x7FC0u);
    uint32_t keep = mag >> 16;
    uint32_t rest = mag & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)((sign >> 16) | keep);
}

/* ------------------------------------------------------------------------ */
/* layout                                                                    */
/* ------------------------------------------------------------------------ */
static int valid_h(int64_t H) { return H >= 8 && H <= ORACLE_MAX_H && (H % 8) == 0; }

int oracle_layout(int64_t H, int* waves, int* lanes, int* chunks) {
    if (!valid_h(H)) return -1;
    int W = (H < 2048) ? 1 : (H < 4096) ? 2 : 4;
    int P = 64 * W;
    int C = (int)((H + 8 * P - 1) / (8 * P));
    if (waves) *waves = W;
    if (lanes) *lanes = P;
    if (chunks) *chunks = C;
    return 0;
}

/* Column owned by lane t at chunk b, element v (may be >= H: not owned). */
static int64_t owned_col(int P, int t, int b, int v) { return (int64_t)b * 8 * P + 8 * (int64_t)t + v; }

/* ------------------------------------------------------------------------ */
/* finalize: rstd = RN(1 / RN(sqrt(RN(stat + eps))))                         */
/* ------------------------------------------------------------------------ */
/* The pages print rsqrt(mean + eps); here the reciprocal square root is a
 * correctly rounded sqrt followed by a correctly rounded divide. */
static void finalize(float mean_like, float eps, float* v_out, float* root_out, float* rstd_out) {
    float v = mean_like + eps;
    float root = sqrtf(v);
    float rstd = 1.0f / root;
    *v_out = v;
    *root_out = root;
    *rstd_out = rstd;
}

/* ------------------------------------------------------------------------ */
/* RMS statistic                                                             */
/* ------------------------------------------------------------------------ */
/* Returns 0, or 1 when the butterfly left lanes with different bits (which
 * would be a bug in this file).  st[0]=sum of squares S, st[1]=RN(S/H),
 * st[2]=RN(st[1]+eps), st[3]=RN(sqrt(st[2])), st[4]=rstd. */
static int rms_stat(const float* xr, int64_t H, float eps, float* st) {
    int W, P, C;
    oracle_layout(H, &W, &P, &C);
    float part[ORACLE_MAX_LANES];
    memset(part, 0, sizeof part);
    for (int t = 0; t < P; t++) {
        float s = 0.0f;
        for (int b = 0; b < C; b++) {
            for (int v = 0; v < 8; v++) {
                int64_t col = owned_col(P, t, b, v);
                if (col >= H) continue;
                float sq = xr[col] * xr[col];
                s = s + sq;
            }
        }
        part[t] = s;
    }
    for (int k = 1; k < P; k <<= 1) {
        float next[ORACLE_MAX_LANES];
        for (int t = 0; t < P; t++) next[t] = part[t & ~k] + part[t | k];
        memcpy(part, next, sizeof(float) * (size_t)P);
    }
    int bad = 0;
    for (int t = 1; t < P; t++)
        if (memcmp(&part[t], &part[0], sizeof(float)) != 0) bad = 1;
    float S = part[0];
    float ms = S / (float)H;
    float v, root, rstd;
    finalize(ms, eps, &v, &root, &rstd);
    st[0] = S;
    st[1] = ms;
    st[2] = v;
    st[3] = root;
    st[4] = rstd;
    return bad;
}

/* ------------------------------------------------------------------------ */
/* LayerNorm statistic: per-lane Welford, pairwise Chan combine              */
/* ------------------------------------------------------------------------ */
typedef struct {
    int64_t n;
    float mean;
    float m2;
} welford_t;

/* One Welford update with the count's correctly rounded reciprocal
 * rho_n = RN(1/n):  d = x - mean; mean += d*rho_n; M2 += d*(x - mean). */
static void welford_push(welford_t* s, float x) {
    s->n += 1;
    float rho = 1.0f / (float)s->n;
    float d = x - s->mean;
    float step = d * rho;
    s->mean = s->mean + step;
    float e = x - s->mean;
    float q = d * e;
    s->m2 = s->m2 + q;
}

/* Chan et al. pairwise combine of (lo, hi), in that operand order:
 *   n = na + nb, delta = mean_b - mean_a, wb = nb/n,
 *   mean = mean_a + delta*wb,  M2 = (M2a + M2b) + (delta*delta)*(na*wb).
 * An empty side returns the other side unchanged. */
static welford_t welford_combine(welford_t lo, welford_t hi) {
    if (hi.n == 0) return lo;
    if (lo.n == 0) return hi;
    welford_t o;
    o.n = lo.n + hi.n;
    float delta = hi.mean - lo.mean;
    float wb = (float)hi.n / (float)o.n;
    float step = delta * wb;
    o.mean = lo.mean + step;
    float msum = lo.m2 + hi.m2;
    float dd = delta * delta;
    float nw = (float)lo.n * wb;
    float corr = dd * nw;
    o.m2 = msum + corr;
    return o;
}

/* st[0]=mean, st[1]=M2, st[2]=RN(M2/H), st[3]=RN(st[2]+eps), st[4]=RN(sqrt),
 * st[5]=rstd.  Returns 0, or 1 on a lane disagreement (a bug in this file). */
static int ln_stat(const float* xr, int64_t H, float eps, float* st) {
    int W, P, C;
    oracle_layout(H, &W, &P, &C);
    welford_t part[ORACLE_MAX_LANES];
    memset(part, 0, sizeof part);
    for (int t = 0; t < P; t++) {
        welford_t s = {0, 0.0f, 0.0f};
        for (int b = 0; b < C; b++) {
            for (int v = 0; v < 8; v++) {
                int64_t col = owned_col(P, t, b, v);
                if (col >= H) continue;
                welford_push(&s, xr[col]);
            }
        }
        part[t] = s;
    }
    for (int k = 1; k < P; k <<= 1) {
        welford_t next[ORACLE_MAX_LANES];
        for (int t = 0; t < P; t++) next[t] = welford_combine(part[t & ~k], part[t | k]);
        memcpy(part, next, sizeof(welford_t) * (size_t)P);
    }
    int bad = 0;
    for (int t = 1; t < P; t++) {
        if (part[t].n != part[0].n || memcmp(&part[t].mean, &part[0].mean, sizeof(float)) != 0 ||
            memcmp(&part[t].m2, &part[0].m2, sizeof(float)) != 0)
            bad = 1;
    }
    if (part[0].n != H) bad = 1;
    float var = part[0].m2 / (float)H;
    float v, root, rstd;
    finalize(var, eps, &v, &root, &rstd);
    st[0] = part[0].mean;
    st[1] = part[0].m2;
    st[2] = var;
    st[3] = v;
    st[4] = root;
    st[5] = rstd;
    return bad;
}

/* ------------------------------------------------------------------------ */
/* modulate and residual-gate steps (eager bf16 chain, one rounding per op)  */
/* ------------------------------------------------------------------------ */
static uint16_t modulate(uint16_t yn, uint16_t scale, uint16_t shift) {
    uint16_t a = to_bf16(1.0f + widen(scale));   /* round(1 + scale) */
    uint16_t p = to_bf16(widen(yn) * widen(a));  /* round(y * that)  */
    return to_bf16(widen(p) + widen(shift));     /* round(p + shift) */
}

static uint16_t gate_residual(uint16_t res, uint16_t upd, uint16_t gate) {
    uint16_t g = to_bf16(widen(gate) * widen(upd)); /* round(gate * update) */
    return to_bf16(widen(res) + widen(g));          /* round(residual + that) */
}

/* ------------------------------------------------------------------------ */
/* static FP8 quantisation (OCP E4M3, "e4m3fn")                              */
/* ------------------------------------------------------------------------ */
/* The format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
 * field 0 holds the subnormals m * 2^-9; there is no infinity; S.1111.111 is NaN,
 * so the largest finite value is 1.75 * 2^8 = 448.  The format has two NaN codes
 * and no page says which one a conversion writes (nor does IEEE 754 interpret the
 * sign of a NaN): this library writes 0xFF for every NaN.  Rounding to nearest-even from
 * the definition: the spacing of representable values around |v| is 2^(E-3) for
 * |v| in [2^E, 2^(E+1)) with E >= -6, and 2^-9 below 2^-6. */
static uint8_t to_e4m3fn(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return 0xFF;
    double a = fabs((double)v);
    if (a == 0.0) return sign;
    int e2;
    (void)frexp(a, &e2);        /* a = f * 2^e2, f in [0.5, 1): floor(log2 a) = e2 - 1 */
    int E = e2 - 1;
    if (E < -6) E = -6;         /* subnormal range shares the spacing of [2^-6, 2^-5) */
    double units = ldexp(a, 3 - E);    /* a / spacing, exact (power-of-two scaling) */
    double r = nearbyint(units);       /* round half to even (default rounding mode) */
    /* r in [8, 16] for the normal range (16: carry into the next binade), in [0, 8]
     * below 2^-6 (8: the smallest normal); the encoding is continuous across both */
    int code;
    if (r >= 8.0) {
        int e = E, m = (int)r - 8;
        if (r == 16.0) { e = E + 1; m = 0; }
        code = ((e + 7) << 3) | m;
    } else {
        code = (int)r;  /* exponent field 0: m * 2^-9 */
    }
    if (code >= 0x7F) return 0xFF;  /* beyond 448: NaN (the caller clamps first) */
    return sign | (uint8_t)code;
}

/* q = e4m3fn(clamp(RN(f(y) * inv), -448, 448)); NaN stays NaN. */
static uint8_t quant_fp8(uint16_t y, float inv) {
    float v = widen(y) * inv;
    if (!isnan(v)) {
        if (v > 448.0f) v = 448.0f;
        if (v < -448.0f) v = -448.0f;
    }
    return to_e4m3fn(v);
}

/* ------------------------------------------------------------------------ */
/* entry points                                                              */
/* ------------------------------------------------------------------------ */
#define STATS_PER_ROW 6

static int check_common(int64_t B, int64_t T, int64_t H) {
    if (B < 0 || T < 0) return -1;
    if (!valid_h(H)) return -1;
    return 0;
}

/* y = LN(x) * (1 + scale[b]) + shift[b], LayerNorm without affine parameters.
 * x, y: [B,T,H] contiguous bf16 bits; scale/shift: row b at ptr + b*bstride.
 * yn_out (nullable): the bf16 norm output before modulate, [B,T,H].
 * stats_out (nullable): STATS_PER_ROW floats per row, see ln_stat.
 * Returns 0, -1 for bad arguments, or the number of rows whose lanes disagreed. */
/* Shared LN tail: statistic of the fp32 row xr, then normalise and modulate. */
static int ln_row(const float* xr, const uint16_t* sc, const uint16_t* sh, int64_t H, float eps,
                  uint16_t* yrow, uint16_t* ynrow, float* strow) {
    float st[STATS_PER_ROW];
    int bad = ln_stat(xr, H, eps, st);
    float mean = st[0], rstd = st[5];
    for (int64_t c = 0; c < H; c++) {
        float d = xr[c] - mean;
        float p = d * rstd;
        uint16_t yn = to_bf16(p);
        if (ynrow) ynrow[c] = yn;
        yrow[c] = modulate(yn, sc[c], sh[c]);
    }
    if (strow) memcpy(strow, st, sizeof st);
    return bad;
}

int oracle_layernorm_modulate(const uint16_t* x, const uint16_t* scale, const uint16_t* shift,
                              uint16_t* y, int64_t B, int64_t T, int64_t H, int64_t scale_bstride,
                              int64_t shift_bstride, float eps, uint16_t* yn_out, float* stats_out) {
    if (check_common(B, T, H)) return -1;
    unsigned int env = fp_enter();
    float xr[ORACLE_MAX_H];
    int bad = 0;
    for (int64_t row = 0; row < B * T; row++) {
        int64_t b = row / T;
        const uint16_t* xp = x + row * H;
        for (int64_t c = 0; c < H; c++) xr[c] = widen(xp[c]);
        bad += ln_row(xr, scale + b * scale_bstride, shift + b * shift_bstride, H, eps, y + row * H,
                      yn_out ? yn_out + row * H : NULL,
                      stats_out ? stats_out + row * STATS_PER_ROW : NULL);
    }
    fp_leave(env);
    return bad;
}

/* Shared RMS tail: statistic of the fp32 row xr, then normalise, weight,
 * modulate.  weight NULL means a weight of one. */
static int rms_row(const float* xr, const uint16_t* weight, const uint16_t* sc, const uint16_t* sh,
                   int64_t H, float eps, uint16_t* yrow, uint16_t* ynrow, float* strow) {
    float st[STATS_PER_ROW] = {0};
    int bad = rms_stat(xr, H, eps, st);
    float rstd = st[4];
    for (int64_t c = 0; c < H; c++) {
        float n = xr[c] * rstd;
        float wf = weight ? (widen(weight[c]) + 0.0f) : 1.0f; /* (w + 0.0) maps -0 to +0 */
        float p = n * wf;
        uint16_t yn = to_bf16(p);
        if (ynrow) ynrow[c] = yn;
        yrow[c] = modulate(yn, sc[c], sh[c]);
    }
    if (strow) memcpy(strow, st, sizeof st);
    return bad;
}

/* y = RMSNorm(x) * (1 + scale[b]) + shift[b]; RMSNorm(x) = x * rstd * w. */
int oracle_rmsnorm_scale_shift(const uint16_t* x, const uint16_t* weight, const uint16_t* scale,
                               const uint16_t* shift, uint16_t* y, int64_t B, int64_t T, int64_t H,
                               int64_t scale_bstride, int64_t shift_bstride, float eps,
                               uint16_t* yn_out, float* stats_out) {
    if (check_common(B, T, H)) return -1;
    unsigned int env = fp_enter();
    float xr[ORACLE_MAX_H];
    int bad = 0;
    for (int64_t row = 0; row < B * T; row++) {
        int64_t b = row / T;
        const uint16_t* xp = x + row * H;
        for (int64_t c = 0; c < H; c++) xr[c] = widen(xp[c]);
        bad += rms_row(xr, weight, scale + b * scale_bstride, shift + b * shift_bstride, H, eps,
                       y + row * H, yn_out ? yn_out + row * H : NULL,
                       stats_out ? stats_out + row * STATS_PER_ROW : NULL);
    }
    fp_leave(env);
    return bad;
}

/* r = res + gate[b]*x (two roundings), returned; y = RMSNorm(r)*(1+scale[b])+shift[b]. */
int oracle_residual_gate_rmsnorm_scale_shift(const uint16_t* res, const uint16_t* x,
                                             const uint16_t* gate, const uint16_t* weight,
                                             const uint16_t* scale, const uint16_t* shift,
                                             uint16_t* r_out, uint16_t* y, int64_t B, int64_t T,
                                             int64_t H, int64_t gate_bstride,
                                             int64_t scale_bstride, int64_t shift_bstride,
                                             float eps, uint16_t* yn_out, float* stats_out) {
    if (check_common(B, T, H)) return -1;
    unsigned int env = fp_enter();
    float xr[ORACLE_MAX_H];
    int bad = 0;
    for (int64_t row = 0; row < B * T; row++) {
        int64_t b = row / T;
        const uint16_t* rp = res + row * H;
        const uint16_t* up = x + row * H;
        const uint16_t* gp = gate + b * gate_bstride;
        for (int64_t c = 0; c < H; c++) {
            uint16_t r = gate_residual(rp[c], up[c], gp[c]);
            r_out[row * H + c] = r;
            xr[c] = widen(r);
        }
        bad += rms_row(xr, weight, scale + b * scale_bstride, shift + b * shift_bstride, H, eps,
                       y + row * H, yn_out ? yn_out + row * H : NULL,
                       stats_out ? stats_out + row * STATS_PER_ROW : NULL);
    }
    fp_leave(env);
    return bad;
}

/* The LayerNorm member of the residual-gate family (the operator the kernels
 * guide registers as scale_residual_norm_scale_shift, and the FLUX.1 residual-gate
 * fast path the FLUX PR report relates to): r = res + gate[b]*x with the same two
 * roundings as above, returned; y = LN(r)*(1+scale[b])+shift[b] with the LN of
 * oracle_layernorm_modulate. */
int oracle_residual_gate_layernorm_modulate(const uint16_t* res, const uint16_t* x,
                                            const uint16_t* gate, const uint16_t* scale,
                                            const uint16_t* shift, uint16_t* r_out, uint16_t* y,
                                            int64_t B, int64_t T, int64_t H, int64_t gate_bstride,
                                            int64_t scale_bstride, int64_t shift_bstride, float eps,
                                            uint16_t* yn_out, float* stats_out) {
    if (check_common(B, T, H)) return -1;
    unsigned int env = fp_enter();
    float xr[ORACLE_MAX_H];
    int bad = 0;
    for (int64_t row = 0; row < B * T; row++) {
        int64_t b = row / T;
        const uint16_t* rp = res + row * H;
        const uint16_t* up = x + row * H;
        const uint16_t* gp = gate + b * gate_bstride;
        for (int64_t c = 0; c < H; c++) {
            uint16_t r = gate_residual(rp[c], up[c], gp[c]);
            r_out[row * H + c] = r;
            xr[c] = widen(r);
        }
        bad += ln_row(xr, scale + b * scale_bstride, shift + b * shift_bstride, H, eps, y + row * H,
                      yn_out ? yn_out + row * H : NULL,
                      stats_out ? stats_out + row * STATS_PER_ROW : NULL);
    }
    fp_leave(env);
    return bad;
}

/* LayerNorm + modulate + static FP8 quantisation (kernels guide, data movement and
 * quantised layout producers: fused_layernorm_modulate_fp8_quant_raw folds FLUX.2's
 * LayerNorm, adaLN modulate and static FP8 quantisation into one kernel):
 * y = LN(x)*(1+scale[b])+shift[b] exactly as oracle_layernorm_modulate (bf16), then
 * q = e4m3fn(clamp(RN(f(y) * RN(1/qscale)), -448, 448)), one byte per element.
 * y_out (nullable) receives the bf16 y. */
int oracle_layernorm_modulate_fp8(const uint16_t* x, const uint16_t* scale, const uint16_t* shift,
                                  float qscale, uint8_t* q, int64_t B, int64_t T, int64_t H,
                                  int64_t scale_bstride, int64_t shift_bstride, float eps,
                                  uint16_t* y_out, float* stats_out) {
    if (check_common(B, T, H)) return -1;
    unsigned int env = fp_enter();
    float xr[ORACLE_MAX_H];
    uint16_t yr[ORACLE_MAX_H];
    const float inv = 1.0f / qscale;  /* correctly rounded */
    int bad = 0;
    for (int64_t row = 0; row < B * T; row++) {
        int64_t b = row / T;
        const uint16_t* xp = x + row * H;
        for (int64_t c = 0; c < H; c++) xr[c] = widen(xp[c]);
        bad += ln_row(xr, scale + b * scale_bstride, shift + b * shift_bstride, H, eps, yr, NULL,
                      stats_out ? stats_out + row * STATS_PER_ROW : NULL);
        for (int64_t c = 0; c < H; c++) {
            q[row * H + c] = quant_fp8(yr[c], inv);
            if (y_out) y_out[row * H + c] = yr[c];
        }
    }
    fp_leave(env);
    return bad;
}

/* Per-head QK RMSNorm + interleaved RoPE (kernels guide, RoPE / QK-norm: the
 * QK-norm chain fused into the rotary embedding; Qwen PR report, implementation
 * item 3 and the qwen_image.py snippet: per-head RMSNorm of Q and K with their
 * weights, then interleaved (non-NeoX) RoPE from an fp32 cos/sin cache,
 * head_dim 128).  Per head vector x (head_dim values):
 *   yn[c] = bf16(RN(RN(x[c] * rstd) * RN(w[c] + 0))), with rstd the RMS statistic
 *           of this library for H = head_dim (same fixed order);
 *   for i < head_dim/2, with a = f(yn[2i]), b = f(yn[2i+1]), c = cs[i],
 *   s = cs[head_dim/2 + i] (cs: the token's cache row, cos half then sin half):
 *     out[2i]   = bf16(RN(RN(a*c) - RN(b*s)))
 *     out[2i+1] = bf16(RN(RN(b*c) + RN(a*s)))
 * q: token t, head h at q + t*q_tstride + h*head_dim; k likewise; outputs are
 * contiguous [tokens, heads, head_dim].  weight NULL means one.  yn_q/yn_k
 * (nullable) receive the normalised values before the rotation. */
#define ORACLE_MAX_HEAD_DIM 256
static int qk_head(const uint16_t* x, const uint16_t* w, const float* cs, int64_t D, float eps,
                   uint16_t* out, uint16_t* yn_out) {
    float xr[ORACLE_MAX_HEAD_DIM] = {0};
    uint16_t yn[ORACLE_MAX_HEAD_DIM] = {0};
    for (int64_t c = 0; c < D; c++) xr[c] = widen(x[c]);
    float st[STATS_PER_ROW];
    int bad = rms_stat(xr, D, eps, st);
    const float rstd = st[4];
    for (int64_t c = 0; c < D; c++) {
        float n = xr[c] * rstd;
        float wf = w ? (widen(w[c]) + 0.0f) : 1.0f;
        float p = n * wf;
        yn[c] = to_bf16(p);
        if (yn_out) yn_out[c] = yn[c];
    }
    for (int64_t i = 0; i < D / 2; i++) {
        float a = widen(yn[2 * i]), b = widen(yn[2 * i + 1]);
        float co = cs[i], si = cs[D / 2 + i];
        float ac = a * co, bs = b * si, bc = b * co, as = a * si;
        float o1 = ac - bs;
        float o2 = bc + as;
        out[2 * i] = to_bf16(o1);
        out[2 * i + 1] = to_bf16(o2);
    }
    return bad;
}

int oracle_qk_rmsnorm_rope(const uint16_t* q, const uint16_t* k, const uint16_t* q_weight,
                           const uint16_t* k_weight, const float* cos_sin, uint16_t* q_out,
                           uint16_t* k_out, int64_t tokens, int64_t heads_q, int64_t heads_k,
                           int64_t head_dim, int64_t q_tstride, int64_t k_tstride, float eps,
                           uint16_t* yn_q, uint16_t* yn_k) {
    if (tokens < 0 || heads_q < 0 || heads_k < 0 || !valid_h(head_dim) ||
        head_dim > ORACLE_MAX_HEAD_DIM)
        return -1;
    unsigned int env = fp_enter();
    int bad = 0;
    for (int64_t t = 0; t < tokens; t++) {
        const float* cs = cos_sin + t * head_dim;
        for (int64_t h = 0; h < heads_q; h++) {
            int64_t o = (t * heads_q + h) * head_dim;
            bad += qk_head(q + t * q_tstride + h * head_dim, q_weight, cs, head_dim, eps,
                           q_out + o, yn_q ? yn_q + o : NULL);
        }
        for (int64_t h = 0; h < heads_k; h++) {
            int64_t o = (t * heads_k + h) * head_dim;
            bad += qk_head(k + t * k_tstride + h * head_dim, k_weight, cs, head_dim, eps,
                           k_out + o, yn_k ? yn_k + o : NULL);
        }
    }
    fp_leave(env);
    return bad;
}

/* Residual gating on the channel-first layout (kernels guide, norm variants /
 * residual gating: the transposed dense path reads `update` in its logical
 * row-major order while the residual and the output stay in their [B, hidden,
 * tokens] layout, with no .contiguous() copy):
 *   out[b][h][t] = bf16(res[b][h][t] + bf16(gate[b][h] * update[b][t][h]))
 * res, out: [B, H, T] contiguous; update: [B, T, H] contiguous; gate row b at
 * gate + b*gate_bstride.  out may be res itself. */
int oracle_residual_gate_channel_first(const uint16_t* res, const uint16_t* update,
                                       const uint16_t* gate, uint16_t* out, int64_t B, int64_t T,
                                       int64_t H, int64_t gate_bstride) {
    if (B < 0 || T < 0 || H < 0) return -1;
    unsigned int env = fp_enter();
    for (int64_t b = 0; b < B; b++)
        for (int64_t h = 0; h < H; h++)
            for (int64_t t = 0; t < T; t++) {
                int64_t i = (b * H + h) * T + t;
                out[i] = gate_residual(res[i], update[(b * T + t) * H + h], gate[b * gate_bstride + h]);
            }
    fp_leave(env);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* elementwise helpers exposed for the pins                                  */
/* ------------------------------------------------------------------------ */
void oracle_round_bf16(const float* in, uint16_t* out, int64_t n) {
    unsigned int env = fp_enter();
    for (int64_t i = 0; i < n; i++) out[i] = to_bf16(in[i]);
    fp_leave(env);
}

void oracle_modulate(const uint16_t* yn, const uint16_t* scale, const uint16_t* shift, uint16_t* out,
                     int64_t n) {
    unsigned int env = fp_enter();
    for (int64_t i = 0; i < n; i++) out[i] = modulate(yn[i], scale[i], shift[i]);
    fp_leave(env);
}

void oracle_gate_residual(const uint16_t* res, const uint16_t* x, const uint16_t* gate,
                          uint16_t* out, int64_t n) {
    unsigned int env = fp_enter();
    for (int64_t i = 0; i < n; i++) out[i] = gate_residual(res[i], x[i], gate[i]);
    fp_leave(env);
}

void oracle_to_e4m3fn(const float* in, uint8_t* out, int64_t n) {
    unsigned int env = fp_enter();
    for (int64_t i = 0; i < n; i++) out[i] = to_e4m3fn(in[i]);
    fp_leave(env);
}

void oracle_quant_fp8(const uint16_t* y, uint8_t* q, int64_t n, float qscale) {
    unsigned int env = fp_enter();
    const float inv = 1.0f / qscale;
    for (int64_t i = 0; i < n; i++) q[i] = quant_fp8(y[i], inv);
    fp_leave(env);
}

int oracle_stats_per_row(void) { return STATS_PER_ROW; }
