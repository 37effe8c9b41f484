// adaln_api.cpp -- the C ABI of libadaln (include/adaln.h): argument validation,
// status codes, and the launch on the caller's stream.
//
// Unsupported input is rejected with a status before anything is launched, so
// outputs are never half-written and the path never degrades silently (kernels
// guide, "entry-point protocol": a kernel raises on unsupported input and never
// returns a silent None).  Validation touches no GPU state, so the `adaln_check_*`
// predicates and every rejection path run on a machine without a GPU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/adaln.h"
#include "adaln_internal.hpp"

namespace {

constexpr int64_t kMaxH = 8192;

struct Span {
    uintptr_t lo, hi;  // [lo, hi) in bytes; empty when lo == hi
};

bool overlaps(const Span& a, const Span& b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

Span act_span(const void* p, int64_t rows, int64_t H) {
    uintptr_t lo = (uintptr_t)p;
    return Span{lo, lo + (uintptr_t)(rows * H * 2)};
}

Span vec_span(const void* p, int64_t B, int64_t H, int64_t bstride) {
    uintptr_t lo = (uintptr_t)p;
    int64_t elems = (B > 1 ? (B - 1) * bstride : 0) + H;
    return Span{lo, lo + (uintptr_t)(elems * 2)};
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by all entry points; *rows receives B*T.
adaln_status check_shape(int64_t B, int64_t T, int64_t H, float eps, int64_t* rows) {
    if (B < 0 || T < 0) return ADALN_ERR_SHAPE;
    if (H < 8 || H > kMaxH || (H % 8) != 0) return ADALN_ERR_SHAPE;
    if (T != 0 && B > INT64_MAX / T) return ADALN_ERR_SHAPE;
    const int64_t r = B * T;
    if (r != 0 && r > INT64_MAX / (2 * H)) return ADALN_ERR_SHAPE;  // byte size must fit
    if (!(eps >= 0.0f) || !isfinite(eps)) return ADALN_ERR_VALUE;
    *rows = r;
    return ADALN_OK;
}

adaln_status check_vec(const void* p, int64_t B, int64_t H, int64_t bstride) {
    if (!p) return ADALN_ERR_NULL;
    if (!aligned16(p)) return ADALN_ERR_ALIGN;
    if (B > 1) {
        if (bstride < 0 || (bstride % 8) != 0) return ADALN_ERR_STRIDE;
        if (bstride != 0 && bstride < H) return ADALN_ERR_STRIDE;
        if (bstride != 0 && (B - 1) > (INT64_MAX / 2 - H) / bstride) return ADALN_ERR_SHAPE;
    }
    return ADALN_OK;
}

#define ADALN_TRY(expr)                  \
    do {                                 \
        adaln_status s_ = (expr);        \
        if (s_ != ADALN_OK) return s_;   \
    } while (0)

// Validation of the compute entry points.  res/gate/r are required by the gated
// ops (RG, RGLN) and ignored by the others; y is the bf16 output, or for LNQ the
// one-byte E4M3 output, whose scale qscale (one float) is then an input.
adaln_status validate(int op, const void* res, const void* x, const void* gate,
                      const void* weight, const void* scale, const void* shift, const void* r,
                      const void* y, int64_t B, int64_t T, int64_t H, int64_t gate_bs,
                      int64_t scale_bs, int64_t shift_bs, float eps, int64_t* rows_out,
                      const void* qscale = nullptr) {
    int64_t rows = 0;
    ADALN_TRY(check_shape(B, T, H, eps, &rows));
    *rows_out = rows;
    if (rows == 0) return ADALN_OK;
    const bool gated = adaln::op_gated(op);
    const bool fp8 = adaln::op_fp8(op);
    if (!x || !y || (gated && (!res || !r)) || (fp8 && !qscale)) return ADALN_ERR_NULL;
    if (!aligned16(x) || !aligned16(y)) return ADALN_ERR_ALIGN;
    if (fp8 && ((uintptr_t)qscale & 3u)) return ADALN_ERR_ALIGN;
    if (gated && (!aligned16(res) || !aligned16(r))) return ADALN_ERR_ALIGN;
    if (weight && !aligned16(weight)) return ADALN_ERR_ALIGN;
    ADALN_TRY(check_vec(scale, B, H, scale_bs));
    ADALN_TRY(check_vec(shift, B, H, shift_bs));
    if (gated) ADALN_TRY(check_vec(gate, B, H, gate_bs));

    // outputs may not overlap any input or each other
    Span in[7];
    int n_in = 0;
    in[n_in++] = act_span(x, rows, H);
    in[n_in++] = vec_span(scale, B, H, scale_bs);
    in[n_in++] = vec_span(shift, B, H, shift_bs);
    if (weight) in[n_in++] = Span{(uintptr_t)weight, (uintptr_t)weight + (uintptr_t)(2 * H)};
    if (gated) {
        in[n_in++] = act_span(res, rows, H);
        in[n_in++] = vec_span(gate, B, H, gate_bs);
    }
    if (fp8) in[n_in++] = Span{(uintptr_t)qscale, (uintptr_t)qscale + 4};
    const Span ys = fp8 ? Span{(uintptr_t)y, (uintptr_t)y + (uintptr_t)(rows * H)}
                        : act_span(y, rows, H);
    for (int i = 0; i < n_in; ++i)
        if (overlaps(ys, in[i])) return ADALN_ERR_OVERLAP;
    if (gated) {
        const Span rs = act_span(r, rows, H);
        if (overlaps(rs, ys)) return ADALN_ERR_OVERLAP;
        for (int i = 0; i < n_in; ++i)
            if (overlaps(rs, in[i])) return ADALN_ERR_OVERLAP;
    }
    return ADALN_OK;
}

adaln_status run(adaln::Op op, const adaln_bf16* res, const adaln_bf16* x, const adaln_bf16* gate,
                 const adaln_bf16* weight, const adaln_bf16* scale, const adaln_bf16* shift,
                 adaln_bf16* r, void* y, int64_t B, int64_t T, int64_t H, int64_t gate_bs,
                 int64_t scale_bs, int64_t shift_bs, float eps, void* stream,
                 const float* qscale = nullptr) {
    int64_t rows = 0;
    ADALN_TRY(validate(op, res, x, gate, weight, scale, shift, r, y, B, T, H, gate_bs, scale_bs,
                       shift_bs, eps, &rows, qscale));
    if (rows == 0) return ADALN_OK;
    adaln::Params p{};
    p.x = x;
    p.res = res;
    p.gate = gate;
    p.weight = weight;
    p.scale = scale;
    p.shift = shift;
    if (adaln::op_fp8(op)) {
        p.q = static_cast<uint8_t*>(y);
        p.qscale = qscale;
    } else {
        p.y = static_cast<uint16_t*>(y);
    }
    p.r = r;
    p.rows = rows;
    p.T = T;
    p.H = H;
    p.gate_bs = B > 1 ? gate_bs : 0;
    p.scale_bs = B > 1 ? scale_bs : 0;
    p.shift_bs = B > 1 ? shift_bs : 0;
    p.eps = eps;
    hipError_t e = adaln::launch(op, p, (hipStream_t)stream);
    return e == hipSuccess ? ADALN_OK : ADALN_ERR_LAUNCH;
}

// Validation of the QK RMSNorm + RoPE entry point.
adaln_status validate_qk(const void* q, const void* k, const void* q_weight, const void* k_weight,
                         const void* cos_sin, const void* q_out, const void* k_out, int64_t tokens,
                         int64_t heads_q, int64_t heads_k, int64_t head_dim, int64_t q_tstride,
                         int64_t k_tstride, float eps, bool* empty) {
    *empty = true;
    if (head_dim != 128) return ADALN_ERR_SHAPE;
    if (tokens < 0 || heads_q < 0 || heads_k < 0) return ADALN_ERR_SHAPE;
    if (!(eps >= 0.0f) || !isfinite(eps)) return ADALN_ERR_VALUE;
    // a token's row of heads is addressed with 32-bit byte offsets
    const int64_t max_heads = (int64_t(1) << 23) - 8;
    if (heads_q > max_heads || heads_k > max_heads) return ADALN_ERR_SHAPE;
    const int64_t lim = INT64_MAX / 4 / 128;
    if (tokens != 0 && (heads_q + heads_k > lim / tokens)) return ADALN_ERR_SHAPE;
    if (tokens == 0 || heads_q + heads_k == 0) return ADALN_OK;
    *empty = false;
    if (!cos_sin) return ADALN_ERR_NULL;
    if ((heads_q > 0 && (!q || !q_out)) || (heads_k > 0 && (!k || !k_out))) return ADALN_ERR_NULL;
    const void* ptrs[] = {heads_q > 0 ? q : nullptr, heads_k > 0 ? k : nullptr, q_weight,
                          k_weight, cos_sin, heads_q > 0 ? q_out : nullptr,
                          heads_k > 0 ? k_out : nullptr};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return ADALN_ERR_ALIGN;
    // token strides (elements): rows of heads*128 values, 16-byte aligned
    if (tokens > 1) {
        if (heads_q > 0 && (q_tstride < heads_q * 128 || (q_tstride % 8) != 0 ||
                            q_tstride > INT64_MAX / 2 / tokens))
            return ADALN_ERR_STRIDE;
        if (heads_k > 0 && (k_tstride < heads_k * 128 || (k_tstride % 8) != 0 ||
                            k_tstride > INT64_MAX / 2 / tokens))
            return ADALN_ERR_STRIDE;
    }
    auto strided = [&](const void* p, int64_t tstride, int64_t heads) {
        const int64_t elems = (tokens > 1 ? (tokens - 1) * tstride : 0) + heads * 128;
        return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(2 * elems)};
    };
    Span in[5];
    int n_in = 0;
    if (heads_q > 0) in[n_in++] = strided(q, q_tstride, heads_q);
    if (heads_k > 0) in[n_in++] = strided(k, k_tstride, heads_k);
    in[n_in++] = Span{(uintptr_t)cos_sin, (uintptr_t)cos_sin + (uintptr_t)(tokens * 128 * 4)};
    if (q_weight) in[n_in++] = Span{(uintptr_t)q_weight, (uintptr_t)q_weight + 256};
    if (k_weight) in[n_in++] = Span{(uintptr_t)k_weight, (uintptr_t)k_weight + 256};
    Span outs[2];
    int n_out = 0;
    if (heads_q > 0) outs[n_out++] = act_span(q_out, tokens, heads_q * 128);
    if (heads_k > 0) outs[n_out++] = act_span(k_out, tokens, heads_k * 128);
    for (int o = 0; o < n_out; ++o) {
        for (int i = 0; i < n_in; ++i)
            if (overlaps(outs[o], in[i])) return ADALN_ERR_OVERLAP;
        for (int o2 = o + 1; o2 < n_out; ++o2)
            if (overlaps(outs[o], outs[o2])) return ADALN_ERR_OVERLAP;
    }
    return ADALN_OK;
}

// Validation of the channel-first residual gate.
adaln_status validate_cf(const void* res, const void* update, const void* gate, const void* out,
                         int64_t B, int64_t T, int64_t H, int64_t gate_bs, bool* empty) {
    *empty = true;
    if (B < 0 || T < 0 || H < 0 || (H % 8) != 0) return ADALN_ERR_SHAPE;
    if (B == 0 || T == 0 || H == 0) return ADALN_OK;
    if (B > INT64_MAX / T || B * T > INT64_MAX / 2 / H) return ADALN_ERR_SHAPE;
    // one workgroup of 256 per tile (adaln::cf_tiles), and a grid holds fewer than 2^32
    // work-items; the bound on B first keeps the tile count itself in range
    const int64_t per_b = adaln::cf_tiles(1, H, T);
    if (B > (int64_t(0xFFFFFFFF) / 256) / per_b) return ADALN_ERR_SHAPE;
    if (adaln::cf_grid(adaln::cf_tiles(B, H, T)) > int64_t(0xFFFFFFFF) / 256) return ADALN_ERR_SHAPE;
    *empty = false;
    if (!res || !update || !out) return ADALN_ERR_NULL;
    if (!aligned16(res) || !aligned16(update) || !aligned16(out)) return ADALN_ERR_ALIGN;
    ADALN_TRY(check_vec(gate, B, H, gate_bs));
    const Span os = act_span(out, B * T, H);
    // out may be res itself (an in-place residual update), never a partial overlap
    if (out != res && overlaps(os, act_span(res, B * T, H))) return ADALN_ERR_OVERLAP;
    if (overlaps(os, act_span(update, B * T, H)) || overlaps(os, vec_span(gate, B, H, gate_bs)))
        return ADALN_ERR_OVERLAP;
    return ADALN_OK;
}

}  // namespace

extern "C" {

adaln_status adaln_residual_gate_channel_first(const adaln_bf16* res, const adaln_bf16* update,
                                               const adaln_bf16* gate, adaln_bf16* out, int64_t B,
                                               int64_t T, int64_t H, int64_t gate_bstride,
                                               void* hip_stream) {
    bool empty = true;
    ADALN_TRY(validate_cf(res, update, gate, out, B, T, H, gate_bstride, &empty));
    if (empty) return ADALN_OK;
    adaln::CFParams p{res, update, gate, out, B, T, H, B > 1 ? gate_bstride : 0};
    hipError_t e = adaln::launch_cf(p, (hipStream_t)hip_stream);
    return e == hipSuccess ? ADALN_OK : ADALN_ERR_LAUNCH;
}

adaln_status adaln_check_residual_gate_channel_first(const adaln_bf16* res,
                                                     const adaln_bf16* update,
                                                     const adaln_bf16* gate, const adaln_bf16* out,
                                                     int64_t B, int64_t T, int64_t H,
                                                     int64_t gate_bstride) {
    bool empty = true;
    return validate_cf(res, update, gate, out, B, T, H, gate_bstride, &empty);
}

adaln_status adaln_qk_rmsnorm_rope(const adaln_bf16* q, const adaln_bf16* k,
                                   const adaln_bf16* q_weight, const adaln_bf16* k_weight,
                                   const float* cos_sin, adaln_bf16* q_out, adaln_bf16* k_out,
                                   int64_t tokens, int64_t heads_q, int64_t heads_k,
                                   int64_t head_dim, int64_t q_token_stride,
                                   int64_t k_token_stride, float eps, void* hip_stream) {
    bool empty = true;
    ADALN_TRY(validate_qk(q, k, q_weight, k_weight, cos_sin, q_out, k_out, tokens, heads_q,
                          heads_k, head_dim, q_token_stride, k_token_stride, eps, &empty));
    if (empty) return ADALN_OK;
    adaln::QKParams p{};
    p.q = q;
    p.k = k;
    p.q_weight = q_weight;
    p.k_weight = k_weight;
    p.cos_sin = cos_sin;
    p.q_out = q_out;
    p.k_out = k_out;
    p.tokens = tokens;
    p.heads_q = heads_q;
    p.heads_k = heads_k;
    p.q_tstride = q_token_stride;
    p.k_tstride = k_token_stride;
    p.eps = eps;
    hipError_t e = adaln::launch_qk(p, (hipStream_t)hip_stream);
    return e == hipSuccess ? ADALN_OK : ADALN_ERR_LAUNCH;
}

adaln_status adaln_check_qk_rmsnorm_rope(const adaln_bf16* q, const adaln_bf16* k,
                                         const adaln_bf16* q_weight, const adaln_bf16* k_weight,
                                         const float* cos_sin, const adaln_bf16* q_out,
                                         const adaln_bf16* k_out, int64_t tokens,
                                         int64_t heads_q, int64_t heads_k, int64_t head_dim,
                                         int64_t q_token_stride, int64_t k_token_stride,
                                         float eps) {
    bool empty = true;
    return validate_qk(q, k, q_weight, k_weight, cos_sin, q_out, k_out, tokens, heads_q, heads_k,
                       head_dim, q_token_stride, k_token_stride, eps, &empty);
}

adaln_status adaln_layernorm_modulate(const adaln_bf16* x, const adaln_bf16* scale,
                                      const adaln_bf16* shift, adaln_bf16* y, int64_t B, int64_t T,
                                      int64_t H, int64_t scale_bstride, int64_t shift_bstride,
                                      float eps, void* hip_stream) {
    return run(adaln::OP_LN, nullptr, x, nullptr, nullptr, scale, shift, nullptr, y, B, T, H, 0,
               scale_bstride, shift_bstride, eps, hip_stream);
}

adaln_status adaln_rmsnorm_scale_shift(const adaln_bf16* x, const adaln_bf16* weight,
                                       const adaln_bf16* scale, const adaln_bf16* shift,
                                       adaln_bf16* y, int64_t B, int64_t T, int64_t H,
                                       int64_t scale_bstride, int64_t shift_bstride, float eps,
                                       void* hip_stream) {
    return run(adaln::OP_RMS, nullptr, x, nullptr, weight, scale, shift, nullptr, y, B, T, H, 0,
               scale_bstride, shift_bstride, eps, hip_stream);
}

adaln_status adaln_residual_gate_rmsnorm_scale_shift(
    const adaln_bf16* res, const adaln_bf16* x, const adaln_bf16* gate, const adaln_bf16* weight,
    const adaln_bf16* scale, const adaln_bf16* shift, adaln_bf16* r_out, adaln_bf16* y, int64_t B,
    int64_t T, int64_t H, int64_t gate_bstride, int64_t scale_bstride, int64_t shift_bstride,
    float eps, void* hip_stream) {
    return run(adaln::OP_RG, res, x, gate, weight, scale, shift, r_out, y, B, T, H, gate_bstride,
               scale_bstride, shift_bstride, eps, hip_stream);
}

adaln_status adaln_residual_gate_layernorm_modulate(
    const adaln_bf16* res, const adaln_bf16* x, const adaln_bf16* gate, const adaln_bf16* scale,
    const adaln_bf16* shift, adaln_bf16* r_out, adaln_bf16* y, int64_t B, int64_t T, int64_t H,
    int64_t gate_bstride, int64_t scale_bstride, int64_t shift_bstride, float eps,
    void* hip_stream) {
    return run(adaln::OP_RGLN, res, x, gate, nullptr, scale, shift, r_out, y, B, T, H,
               gate_bstride, scale_bstride, shift_bstride, eps, hip_stream);
}

adaln_status adaln_layernorm_modulate_fp8_quant(const adaln_bf16* x, const adaln_bf16* scale,
                                                const adaln_bf16* shift, const float* qscale,
                                                uint8_t* q, int64_t B, int64_t T, int64_t H,
                                                int64_t scale_bstride, int64_t shift_bstride,
                                                float eps, void* hip_stream) {
    return run(adaln::OP_LNQ, nullptr, x, nullptr, nullptr, scale, shift, nullptr, q, B, T, H, 0,
               scale_bstride, shift_bstride, eps, hip_stream, qscale);
}

adaln_status adaln_check_layernorm_modulate(const adaln_bf16* x, const adaln_bf16* scale,
                                            const adaln_bf16* shift, const adaln_bf16* y,
                                            int64_t B, int64_t T, int64_t H,
                                            int64_t scale_bstride, int64_t shift_bstride,
                                            float eps) {
    int64_t rows;
    return validate(adaln::OP_LN, nullptr, x, nullptr, nullptr, scale, shift, nullptr, y, B, T, H,
                    0, scale_bstride, shift_bstride, eps, &rows);
}

adaln_status adaln_check_rmsnorm_scale_shift(const adaln_bf16* x, const adaln_bf16* weight,
                                             const adaln_bf16* scale, const adaln_bf16* shift,
                                             const adaln_bf16* y, int64_t B, int64_t T, int64_t H,
                                             int64_t scale_bstride, int64_t shift_bstride,
                                             float eps) {
    int64_t rows;
    return validate(adaln::OP_RMS, nullptr, x, nullptr, weight, scale, shift, nullptr, y, B, T, H,
                    0, scale_bstride, shift_bstride, eps, &rows);
}

adaln_status adaln_check_residual_gate_rmsnorm_scale_shift(
    const adaln_bf16* res, const adaln_bf16* x, const adaln_bf16* gate, const adaln_bf16* weight,
    const adaln_bf16* scale, const adaln_bf16* shift, const adaln_bf16* r_out,
    const adaln_bf16* y, int64_t B, int64_t T, int64_t H, int64_t gate_bstride,
    int64_t scale_bstride, int64_t shift_bstride, float eps) {
    int64_t rows;
    return validate(adaln::OP_RG, res, x, gate, weight, scale, shift, r_out, y, B, T, H,
                    gate_bstride, scale_bstride, shift_bstride, eps, &rows);
}

adaln_status adaln_check_residual_gate_layernorm_modulate(
    const adaln_bf16* res, const adaln_bf16* x, const adaln_bf16* gate, const adaln_bf16* scale,
    const adaln_bf16* shift, const adaln_bf16* r_out, const adaln_bf16* y, int64_t B, int64_t T,
    int64_t H, int64_t gate_bstride, int64_t scale_bstride, int64_t shift_bstride, float eps) {
    int64_t rows;
    return validate(adaln::OP_RGLN, res, x, gate, nullptr, scale, shift, r_out, y, B, T, H,
                    gate_bstride, scale_bstride, shift_bstride, eps, &rows);
}

adaln_status adaln_check_layernorm_modulate_fp8_quant(const adaln_bf16* x, const adaln_bf16* scale,
                                                      const adaln_bf16* shift, const float* qscale,
                                                      const uint8_t* q, int64_t B, int64_t T,
                                                      int64_t H, int64_t scale_bstride,
                                                      int64_t shift_bstride, float eps) {
    int64_t rows;
    return validate(adaln::OP_LNQ, nullptr, x, nullptr, nullptr, scale, shift, nullptr, q, B, T, H,
                    0, scale_bstride, shift_bstride, eps, &rows, qscale);
}

adaln_status adaln_reduction_layout(int64_t H, int* waves_per_row, int* lanes_per_row,
                                    int* chunks_per_lane) {
    if (H < 8 || H > kMaxH || (H % 8) != 0) return ADALN_ERR_SHAPE;
    const adaln::Layout L = adaln::layout_of(H);
    if (waves_per_row) *waves_per_row = L.waves;
    if (lanes_per_row) *lanes_per_row = L.lanes;
    if (chunks_per_lane) *chunks_per_lane = L.chunks;
    return ADALN_OK;
}

const char* adaln_status_string(adaln_status status) {
    switch (status) {
        case ADALN_OK: return "success";
        case ADALN_ERR_NULL: return "a required pointer is NULL";
        case ADALN_ERR_SHAPE:
            return "unsupported shape: sizes >= 0; row ops need 8 <= H <= 8192 and H % 8 == 0; "
                   "QK-norm needs head_dim 128; the channel-first op needs H % 8 == 0 (any T) "
                   "and fewer than 2^24 tiles of 64x64";
        case ADALN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case ADALN_ERR_STRIDE: return "a batch stride is negative, not a multiple of 8, or in (0, H)";
        case ADALN_ERR_OVERLAP: return "an output overlaps an input or the other output";
        case ADALN_ERR_VALUE: return "eps must be finite and >= 0";
        case ADALN_ERR_LAUNCH: return "the HIP kernel launch failed";
    }
    return "unknown status";
}

int adaln_abi_version(void) { return ADALN_ABI_VERSION; }

}  // extern "C"

namespace {

// plan arguments shared by the two plan diagnostics
adaln_status check_plan_args(int op, int64_t rows, int64_t H, int64_t T, const int64_t* out) {
    if (!out) return ADALN_ERR_NULL;
    if (op < adaln::OP_LN || op > adaln::OP_LNQ) return ADALN_ERR_VALUE;
    if (rows < 1 || H < 8 || H > kMaxH || (H % 8) != 0) return ADALN_ERR_SHAPE;
    if (rows > INT64_MAX / (2 * H)) return ADALN_ERR_SHAPE;
    if (T < 1 || T > rows || rows % T != 0) return ADALN_ERR_SHAPE;
    return ADALN_OK;
}

void write_plan(const adaln::Plan& pl, int64_t* out) {
    out[0] = pl.shallow ? 1 : 0;
    out[1] = pl.slots;
    out[2] = pl.ring;
    out[3] = pl.groups;
    out[4] = pl.gpb;
    out[5] = pl.blk_rows;
    out[6] = pl.group_stride;
    out[7] = pl.step;
    out[8] = pl.span;
    out[9] = pl.blocks;
    out[10] = pl.block_threads;
}

}  // namespace

extern "C" {

adaln_status adaln_diag_launch_plan(int op, int64_t rows, int64_t H, int64_t T,
                                    const int64_t* resident, int64_t cus, int64_t* out) {
    ADALN_TRY(check_plan_args(op, rows, H, T, out));
    if (!resident) return ADALN_ERR_NULL;
    // resident counts of a real device are far below 2^31; the plan's products of
    // them stay in range only below that
    constexpr int64_t kMaxResident = 0x7FFFFFFF;
    if (resident[0] < 1) return ADALN_ERR_VALUE;
    for (int i = 0; i < 3; ++i)
        if (resident[i] < 0 || resident[i] > kMaxResident) return ADALN_ERR_VALUE;
    if (cus < 0 || cus > kMaxResident) return ADALN_ERR_VALUE;
    const adaln::Plan pl = adaln::decide(static_cast<adaln::Op>(op), rows, H, T, resident, cus);
    // a launch whose grid would pass 2^32 work-items is refused (rows past 2^55 bytes)
    if (pl.blocks * pl.block_threads > int64_t(0xFFFFFFFF)) return ADALN_ERR_SHAPE;
    write_plan(pl, out);
    return ADALN_OK;
}

adaln_status adaln_diag_device_plan(int op, int64_t rows, int64_t H, int64_t T, int weight,
                                    int64_t* out, int64_t* resident_out, int64_t* cus_out) {
    ADALN_TRY(check_plan_args(op, rows, H, T, out));
    adaln::Plan pl;
    int64_t resident[3], cus = 0;
    if (!adaln::device_plan(static_cast<adaln::Op>(op), rows, H, T, weight != 0, &pl, resident,
                            &cus))
        return ADALN_ERR_LAUNCH;
    write_plan(pl, out);
    if (resident_out)
        for (int i = 0; i < 3; ++i) resident_out[i] = resident[i];
    if (cus_out) *cus_out = cus;
    return ADALN_OK;
}

adaln_status adaln_diag_round_bf16(const float* in, adaln_bf16* out, int64_t n, void* hip_stream) {
    if (n < 0) return ADALN_ERR_SHAPE;
    if (n == 0) return ADALN_OK;
    if (!in || !out) return ADALN_ERR_NULL;
    if (((uintptr_t)in & 3u) || ((uintptr_t)out & 1u)) return ADALN_ERR_ALIGN;
    if (overlaps(Span{(uintptr_t)out, (uintptr_t)out + (uintptr_t)(2 * n)},
                 Span{(uintptr_t)in, (uintptr_t)in + (uintptr_t)(4 * n)}))
        return ADALN_ERR_OVERLAP;
    return adaln::launch_diag_round(in, out, n, (hipStream_t)hip_stream) == hipSuccess
               ? ADALN_OK
               : ADALN_ERR_LAUNCH;
}

adaln_status adaln_diag_finalize(const float* in, float* out, int64_t n, int64_t H, float eps,
                                 void* hip_stream) {
    if (n < 0 || H < 1 || H > kMaxH) return ADALN_ERR_SHAPE;
    if (!(eps >= 0.0f) || !isfinite(eps)) return ADALN_ERR_VALUE;
    if (n == 0) return ADALN_OK;
    if (!in || !out) return ADALN_ERR_NULL;
    if (((uintptr_t)in & 3u) || ((uintptr_t)out & 3u)) return ADALN_ERR_ALIGN;
    // elementwise: in place is fine, a shifted overlap is not
    if ((const void*)in != (const void*)out &&
        overlaps(Span{(uintptr_t)out, (uintptr_t)out + (uintptr_t)(4 * n)},
                 Span{(uintptr_t)in, (uintptr_t)in + (uintptr_t)(4 * n)}))
        return ADALN_ERR_OVERLAP;
    return adaln::launch_diag_finalize(in, out, n, H, eps, (hipStream_t)hip_stream) == hipSuccess
               ? ADALN_OK
               : ADALN_ERR_LAUNCH;
}

adaln_status adaln_diag_quant_fp8(const float* in, uint8_t* out, int64_t n, const float* qscale,
                                  void* hip_stream) {
    if (n < 0 || (n % 4) != 0) return ADALN_ERR_SHAPE;
    if (n == 0) return ADALN_OK;
    if (!in || !out || !qscale) return ADALN_ERR_NULL;
    if (!aligned16(in) || ((uintptr_t)out & 3u) || ((uintptr_t)qscale & 3u)) return ADALN_ERR_ALIGN;
    const Span o{(uintptr_t)out, (uintptr_t)out + (uintptr_t)n};
    if (overlaps(o, Span{(uintptr_t)in, (uintptr_t)in + (uintptr_t)(4 * n)}) ||
        overlaps(o, Span{(uintptr_t)qscale, (uintptr_t)qscale + 4}))
        return ADALN_ERR_OVERLAP;
    return adaln::launch_diag_quant(in, out, n, qscale, (hipStream_t)hip_stream) == hipSuccess
               ? ADALN_OK
               : ADALN_ERR_LAUNCH;
}

adaln_status adaln_diag_stream_copy(const void* src, void* dst, int64_t bytes,
                                    void* hip_stream) {
    return adaln_diag_stream(0, src, dst, bytes, 8, hip_stream);
}

adaln_status adaln_diag_stream(int kind, const void* src, void* dst, int64_t bytes,
                               int vectors_per_thread, void* hip_stream) {
    if (kind < adaln::STREAM_COPY || kind > adaln::STREAM_FILL) return ADALN_ERR_VALUE;
    const int per = vectors_per_thread;
    if (per != 1 && per != 2 && per != 4 && per != 8 && per != 16) return ADALN_ERR_VALUE;
    if (bytes < 0 || (bytes % 16) != 0) return ADALN_ERR_SHAPE;
    if (bytes == 0) return ADALN_OK;
    const bool reads = kind != adaln::STREAM_FILL;
    if ((reads && !src) || !dst) return ADALN_ERR_NULL;
    if ((reads && !aligned16(src)) || !aligned16(dst)) return ADALN_ERR_ALIGN;
    // copy: dst receives `bytes`; read: the waves' folds, a prefix of dst
    const int64_t n16 = bytes / 16;
    const int64_t written = kind == adaln::STREAM_READ ? adaln::stream_sink_bytes(n16, per) : bytes;
    if (written > bytes) return ADALN_ERR_SHAPE;
    if (reads && overlaps(Span{(uintptr_t)src, (uintptr_t)src + (uintptr_t)bytes},
                          Span{(uintptr_t)dst, (uintptr_t)dst + (uintptr_t)written}))
        return ADALN_ERR_OVERLAP;
    return adaln::launch_stream(kind, src, dst, n16, per, (hipStream_t)hip_stream) == hipSuccess
               ? ADALN_OK
               : ADALN_ERR_LAUNCH;
}

}  // extern "C"
