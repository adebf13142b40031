// C-ABI entry points: argument validation (no HIP call before it passes),
// kernel selection, launch.
#include "cattn.h"
#include "cattn_internal.h"

#include <math.h>
#include <stdint.h>

namespace {

using cattn::Problem;

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates a call and fills `p`.  Returns CATTN_OK, or the first error found.
// `empty` is set when B*H*T == 0 (valid, nothing to do).
cattn_status validate(int op, int layout, const void *q_re, const void *q_im, const void *k_re,
                      const void *k_im, const void *v_re, const void *v_im, void *o_re, void *o_im,
                      int64_t B, int64_t H, int64_t T, int64_t d_h, int causal, float eps, float bias,
                      float *row_den, void *stream, Problem *p, bool *empty) {
    if (layout != CATTN_LAYOUT_C64 && layout != CATTN_LAYOUT_BF16_PLANES) return CATTN_E_LAYOUT;
    if (op == cattn::OP_BORN && (!isfinite(eps) || eps < 0.f)) return CATTN_E_ARG;
    if (op == cattn::OP_PCT && !isfinite(bias)) return CATTN_E_ARG;
    if (B < 0 || H < 0 || T < 0 || d_h < 0) return CATTN_E_SHAPE;
    if (d_h < 1 || d_h > CATTN_MAX_DH) return CATTN_E_UNSUPPORTED;
    if (T > INT32_MAX || H > INT32_MAX || B > INT32_MAX) return CATTN_E_SHAPE;
    const int64_t BH = B * H;  // both <= 2^31, no overflow
    if (BH > INT32_MAX) return CATTN_E_SHAPE;
    const int64_t elem = layout == CATTN_LAYOUT_C64 ? 8 : 2;  // bytes per element per pointer
    // rows * d_h * elem must fit comfortably in int64
    if (BH != 0 && T > (int64_t)(INT64_MAX / 16) / BH / d_h / elem) return CATTN_E_SHAPE;
    *empty = BH == 0 || T == 0;
    if (*empty) return CATTN_OK;

    const void *ins[6] = {q_re, q_im, k_re, k_im, v_re, v_im};
    if (!q_re || !k_re || !v_re || !o_re) return CATTN_E_NULL;
    if (layout == CATTN_LAYOUT_C64) {
        if (q_im || k_im || v_im || o_im) return CATTN_E_NULL;
    } else {
        if (!q_im || !k_im || !v_im || !o_im) return CATTN_E_NULL;
    }
    for (const void *x : ins)
        if (x && !aligned16(x)) return CATTN_E_ALIGN;
    if (!aligned16(o_re) || (o_im && !aligned16(o_im))) return CATTN_E_ALIGN;
    if (row_den && !aligned16(row_den)) return CATTN_E_ALIGN;

    const uintptr_t bytes = (uintptr_t)(BH * T * d_h * elem);
    auto span = [bytes](const void *x) { return Span{(uintptr_t)x, (uintptr_t)x + bytes}; };
    const void *outs[2] = {o_re, o_im};
    for (const void *o : outs) {
        if (!o) continue;
        for (const void *x : ins)
            if (x && overlaps(span(o), span(x))) return CATTN_E_ALIAS;
    }
    if (o_im && overlaps(span(o_re), span(o_im))) return CATTN_E_ALIAS;
    if (row_den) {
        const Span rd{(uintptr_t)row_den, (uintptr_t)row_den + (uintptr_t)(BH * T * 4)};
        for (const void *x : ins)
            if (x && overlaps(rd, span(x))) return CATTN_E_ALIAS;
        for (const void *o : outs)
            if (o && overlaps(rd, span(o))) return CATTN_E_ALIAS;
    }

    p->op = op;
    p->layout = layout == CATTN_LAYOUT_C64 ? cattn::LAYOUT_C64 : cattn::LAYOUT_BF16;
    p->q_re = q_re; p->q_im = q_im;
    p->k_re = k_re; p->k_im = k_im;
    p->v_re = v_re; p->v_im = v_im;
    p->o_re = o_re; p->o_im = o_im;
    p->row_den = row_den;
    p->BH = (int)BH;
    p->T = (int)T;
    p->d = (int)d_h;
    p->causal = causal != 0;
    p->eps = eps;
    p->bias = bias;
    p->stream = reinterpret_cast<hipStream_t>(stream);
    return CATTN_OK;
}

cattn_status run(const Problem &p) {
    hipError_t e;
    if (cattn::supports_born_bf16_d64(p))
        e = cattn::launch_born_bf16_d64(p);
    else if (cattn::supports_born_bf16_mfma(p))
        e = cattn::launch_born_bf16_mfma(p);
    else if (cattn::supports_f32_mfma(p))
        e = cattn::launch_f32_mfma(p);
    else
        e = cattn::launch_generic(p);
    return e == hipSuccess ? CATTN_OK : CATTN_E_LAUNCH;
}

}  // namespace

extern "C" {

cattn_status cattn_born_fwd(int layout, const void *q_re, const void *q_im, const void *k_re, const void *k_im,
                            const void *v_re, const void *v_im, void *o_re, void *o_im, int64_t B, int64_t H,
                            int64_t T, int64_t d_h, int causal, float eps, float *row_den, void *stream) {
    Problem p{};
    bool empty = false;
    const cattn_status s = validate(cattn::OP_BORN, layout, q_re, q_im, k_re, k_im, v_re, v_im, o_re, o_im, B, H,
                                    T, d_h, causal, eps, 0.f, row_den, stream, &p, &empty);
    if (s != CATTN_OK || empty) return s;
    return run(p);
}

cattn_status cattn_pct_fwd(int layout, const void *q_re, const void *q_im, const void *k_re, const void *k_im,
                           const void *v_re, const void *v_im, void *o_re, void *o_im, int64_t B, int64_t H,
                           int64_t T, int64_t d_h, int causal, float bias, void *stream) {
    Problem p{};
    bool empty = false;
    const cattn_status s = validate(cattn::OP_PCT, layout, q_re, q_im, k_re, k_im, v_re, v_im, o_re, o_im, B, H,
                                    T, d_h, causal, 0.f, bias, nullptr, stream, &p, &empty);
    if (s != CATTN_OK || empty) return s;
    return run(p);
}

const char *cattn_status_str(int status) {
    switch (status) {
        case CATTN_OK: return "ok";
        case CATTN_E_NULL: return "required pointer is NULL (or an imaginary-plane pointer was given for complex64)";
        case CATTN_E_SHAPE: return "negative or too large size";
        case CATTN_E_LAYOUT: return "unknown layout";
        case CATTN_E_ALIGN: return "pointer not 16-byte aligned";
        case CATTN_E_ALIAS: return "output overlaps an input or another output";
        case CATTN_E_UNSUPPORTED: return "head width d_h outside 1..128";
        case CATTN_E_LAUNCH: return "HIP kernel launch failed";
        case CATTN_E_ARG: return "eps negative or not finite, or bias not finite";
        default: return "unknown status";
    }
}

int cattn_abi_version(void) { return 1; }

}  // extern "C"
