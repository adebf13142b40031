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
bool aligned_to(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

// Resolves one operand's strides (0 -> dense) and its extent in elements
// (largest element offset + 1).  False if a stride is negative or the extent
// overflows.
bool resolve_strides(const cattn_stride *in, int64_t B, int64_t H, int64_t T, int64_t d, cattn::Str3 *out,
                     int64_t *extent) {
    cattn::Str3 s{in ? in->b : 0, in ? in->h : 0, in ? in->t : 0};
    if (s.b < 0 || s.h < 0 || s.t < 0) return false;
    if (s.t == 0) s.t = d;
    if (s.h == 0) s.h = T * d;          // T * d and H * T * d are bounded by the caller's size check
    if (s.b == 0) s.b = H * T * d;
    const int64_t n[3] = {B, H, T}, st[3] = {s.b, s.h, s.t};
    int64_t e = d;
    for (int i = 0; i < 3; ++i) {
        int64_t m;
        if (__builtin_mul_overflow(n[i] - 1, st[i], &m) || __builtin_add_overflow(e, m, &e)) return false;
    }
    if (e > INT64_MAX / 16) return false;   // byte extents stay far from overflow
    *out = s;
    *extent = e;
    return true;
}

// True when no two (b, h, t) rows of an operand share an element: with the
// dimensions of size > 1 sorted by stride, each stride reaches past the span
// of the dimensions inside it.
bool rows_disjoint(const cattn::Str3 &s, int64_t B, int64_t H, int64_t T, int64_t d) {
    int64_t n[3] = {B, H, T}, st[3] = {s.b, s.h, s.t};
    for (int i = 0; i < 3; ++i)        // sort by stride, ascending
        for (int j = i + 1; j < 3; ++j)
            if (st[j] < st[i]) {
                int64_t a = st[i]; st[i] = st[j]; st[j] = a;
                a = n[i]; n[i] = n[j]; n[j] = a;
            }
    int64_t ext = d;
    for (int i = 0; i < 3; ++i) {
        if (n[i] <= 1) continue;
        if (st[i] < ext) return false;
        ext += st[i] * (n[i] - 1);     // bounded by the operand's extent
    }
    return true;
}

// Reads a host decay table of H values into `out` (lg2 = log2 gamma in
// double precision).  NULL: no decay.
cattn_status resolve_decay(const float *decay, int64_t H, int causal, cattn::Decay *out) {
    out->on = 0;
    if (!decay) return CATTN_OK;
    if (!causal) return CATTN_E_ARG;
    if (H > CATTN_MAX_DECAY_HEADS) return CATTN_E_UNSUPPORTED;
    for (int64_t h = 0; h < H; ++h) {
        const float g = decay[h];
        if (!(g > 0.f) || !(g <= 1.f)) return CATTN_E_ARG;   // NaN fails both
        out->lg2[h] = (float)log2((double)g);
    }
    out->on = 1;
    return CATTN_OK;
}

// Validates a call and fills `p`.  Returns CATTN_OK, or the first error found.
// `empty` is set when B*H*T == 0 (valid, nothing to do).
cattn_status validate(int op, int layout, const void *q_re, const void *q_im, const void *k_re,
                      const void *k_im, const void *v_re, const void *v_im, void *o_re, void *o_im,
                      int64_t B, int64_t H, int64_t T, int64_t d_h, const cattn_strides *strides, int causal,
                      float eps, float bias, float *row_den, void *stream, Problem *p, bool *empty,
                      float gate_r = 0.f, float gate_t = 0.f) {
    if (layout != CATTN_LAYOUT_C64 && layout != CATTN_LAYOUT_BF16_PLANES) return CATTN_E_LAYOUT;
    if (op == cattn::OP_BORN && (!isfinite(eps) || eps < 0.f)) return CATTN_E_ARG;
    if (op == cattn::OP_PCT && !isfinite(bias)) return CATTN_E_ARG;
    if (op == cattn::OP_PCT_SCREEN && (!isfinite(gate_r) || !isfinite(gate_t))) return CATTN_E_ARG;
    if (B < 0 || H < 0 || T < 0 || d_h < 0) return CATTN_E_SHAPE;
    if (d_h < 1 || d_h > CATTN_MAX_DH) return CATTN_E_UNSUPPORTED;
    if (T > CATTN_MAX_T || H > INT32_MAX || B > INT32_MAX) return CATTN_E_SHAPE;
    const int64_t BH = B * H;  // both <= 2^31, no overflow
    if (BH > INT32_MAX) return CATTN_E_SHAPE;
    const int64_t elem = layout == CATTN_LAYOUT_C64 ? 8 : 2;  // bytes per element per pointer
    // rows * d_h * elem must fit comfortably in int64
    if (BH != 0 && T > (int64_t)(INT64_MAX / 16) / BH / d_h / elem) return CATTN_E_SHAPE;
    *empty = BH == 0 || T == 0;
    if (*empty) return CATTN_OK;

    cattn::Str3 st[4];
    int64_t ext[4];
    const cattn_stride *given[4] = {strides ? &strides->q : nullptr, strides ? &strides->k : nullptr,
                                    strides ? &strides->v : nullptr, strides ? &strides->o : nullptr};
    for (int i = 0; i < 4; ++i)
        if (!resolve_strides(given[i], B, H, T, d_h, &st[i], &ext[i])) return CATTN_E_SHAPE;

    const void *ins[6] = {q_re, q_im, k_re, k_im, v_re, v_im};
    if (!q_re || !k_re || !v_re || !o_re) return CATTN_E_NULL;
    if (layout == CATTN_LAYOUT_C64) {
        if (q_im || k_im || v_im || o_im) return CATTN_E_NULL;
    } else {
        if (!q_im || !k_im || !v_im || !o_im) return CATTN_E_NULL;
    }
    // element alignment is required; the matrix-core kernels also want 16 bytes (below)
    for (const void *x : ins)
        if (x && !aligned_to(x, elem)) return CATTN_E_ALIGN;
    if (!aligned_to(o_re, elem) || (o_im && !aligned_to(o_im, elem))) return CATTN_E_ALIGN;
    if (row_den && !aligned_to(row_den, 4)) return CATTN_E_ALIGN;
    if (!rows_disjoint(st[3], B, H, T, d_h)) return CATTN_E_ALIAS;

    // input i (pointer slot) belongs to operand i / 2
    auto span = [&](const void *x, int operand) {
        return Span{(uintptr_t)x, (uintptr_t)x + (uintptr_t)(ext[operand] * elem)};
    };
    const void *outs[2] = {o_re, o_im};
    for (const void *o : outs) {
        if (!o) continue;
        for (int i = 0; i < 6; ++i)
            if (ins[i] && overlaps(span(o, 3), span(ins[i], i / 2))) return CATTN_E_ALIAS;
    }
    if (o_im && overlaps(span(o_re, 3), span(o_im, 3))) return CATTN_E_ALIAS;
    if (row_den) {
        const Span rd{(uintptr_t)row_den, (uintptr_t)row_den + (uintptr_t)(BH * T * 4)};
        for (int i = 0; i < 6; ++i)
            if (ins[i] && overlaps(rd, span(ins[i], i / 2))) return CATTN_E_ALIAS;
        for (const void *o : outs)
            if (o && overlaps(rd, span(o, 3))) return CATTN_E_ALIAS;
    }

    p->op = op;
    p->layout = layout == CATTN_LAYOUT_C64 ? cattn::LAYOUT_C64 : cattn::LAYOUT_BF16;
    p->q_re = q_re; p->q_im = q_im;
    p->k_re = k_re; p->k_im = k_im;
    p->v_re = v_re; p->v_im = v_im;
    p->o_re = o_re; p->o_im = o_im;
    p->row_den = row_den;
    p->sq = st[0]; p->sk = st[1]; p->sv = st[2]; p->so = st[3];
    p->aligned16 = true;
    for (const void *x : ins)
        if (x && !aligned16(x)) p->aligned16 = false;
    if (!aligned16(o_re) || (o_im && !aligned16(o_im))) p->aligned16 = false;
    for (int i = 0; i < 4; ++i) {
        const int64_t n[3] = {B, H, T}, v[3] = {st[i].b, st[i].h, st[i].t};
        for (int j = 0; j < 3; ++j) {
            if (n[j] <= 1) continue;   // the stride of a dimension of size 1 is never used
            if ((v[j] * elem) % 16 != 0) p->aligned16 = false;
        }
    }
    p->BH = (int)BH;
    p->H = (int)H;
    p->T = (int)T;
    p->d = (int)d_h;
    p->causal = causal != 0;
    p->eps = eps;
    p->bias = bias;
    p->gate_r = gate_r;
    p->gate_t = gate_t;
    p->stream = reinterpret_cast<hipStream_t>(stream);
    return CATTN_OK;
}

cattn_status run(const Problem &p) {
    hipError_t e;
    if (cattn::supports_born_bf16_d64(p))
        e = cattn::launch_born_bf16_d64(p);
    else if (cattn::supports_born_bf16_q16<128>(p))
        e = cattn::launch_born_bf16_q16<128>(p);
    else if (cattn::supports_born_bf16_q16<32>(p))
        e = cattn::launch_born_bf16_q16<32>(p);
    else if (cattn::supports_born_bf16_mfma(p))
        e = cattn::launch_born_bf16_mfma(p);
    else if (cattn::supports_f32_mfma16(p))
        e = cattn::launch_f32_mfma16(p);
    else
        e = cattn::launch_generic(p);
    return e == hipSuccess ? CATTN_OK : CATTN_E_LAUNCH;
}

// Validates a backward call and fills `p` (same rules as the forward: layout,
// sizes, NULLs, 16-byte alignment, and no output overlapping an input or
// another output).
cattn_status validate_bwd(int op, int layout, const void *const in_re[5], const void *const in_im[5],
                          const float *row_den, void *const out_re[3], void *const out_im[3], float *db_rows,
                          int64_t B, int64_t H, int64_t T, int64_t d_h, int causal, float bias, void *stream,
                          cattn::BwdProblem *p, bool *empty) {
    // in: q, k, v, o (Born only), g
    if (layout != CATTN_LAYOUT_C64 && layout != CATTN_LAYOUT_BF16_PLANES) return CATTN_E_LAYOUT;
    if (op == cattn::OP_PCT && !isfinite(bias)) return CATTN_E_ARG;
    if (B < 0 || H < 0 || T < 0 || d_h < 0) return CATTN_E_SHAPE;
    if (d_h < 1 || d_h > CATTN_MAX_DH) return CATTN_E_UNSUPPORTED;
    if (T > CATTN_MAX_T || H > INT32_MAX || B > INT32_MAX) return CATTN_E_SHAPE;
    const int64_t BH = B * H;
    if (BH > INT32_MAX) return CATTN_E_SHAPE;
    const int64_t elem = layout == CATTN_LAYOUT_C64 ? 8 : 2;
    if (BH != 0 && T > (int64_t)(INT64_MAX / 16) / BH / d_h / elem) return CATTN_E_SHAPE;
    *empty = BH == 0 || T == 0;
    if (*empty) return CATTN_OK;

    const bool born = op == cattn::OP_BORN;
    const bool c64 = layout == CATTN_LAYOUT_C64;
    for (int i = 0; i < 5; ++i) {
        if (i == 3 && !born) continue;   // PCT takes no O
        if (!in_re[i] || (c64 ? in_im[i] != nullptr : in_im[i] == nullptr)) return CATTN_E_NULL;
    }
    for (int i = 0; i < 3; ++i)
        if (!out_re[i] || (c64 ? out_im[i] != nullptr : out_im[i] == nullptr)) return CATTN_E_NULL;
    if (born && !row_den) return CATTN_E_NULL;

    for (int i = 0; i < 5; ++i)
        if ((in_re[i] && !aligned16(in_re[i])) || (in_im[i] && !aligned16(in_im[i]))) return CATTN_E_ALIGN;
    for (int i = 0; i < 3; ++i)
        if (!aligned16(out_re[i]) || (out_im[i] && !aligned16(out_im[i]))) return CATTN_E_ALIGN;
    if ((row_den && !aligned16(row_den)) || (db_rows && !aligned16(db_rows))) return CATTN_E_ALIGN;

    const uintptr_t bytes = (uintptr_t)(BH * T * d_h * elem);
    const uintptr_t rbytes = (uintptr_t)(BH * T * 4);
    Span ins[11];
    int ni = 0;
    for (int i = 0; i < 5; ++i) {
        if (in_re[i]) ins[ni++] = Span{(uintptr_t)in_re[i], (uintptr_t)in_re[i] + bytes};
        if (in_im[i]) ins[ni++] = Span{(uintptr_t)in_im[i], (uintptr_t)in_im[i] + bytes};
    }
    if (row_den) ins[ni++] = Span{(uintptr_t)row_den, (uintptr_t)row_den + rbytes};
    Span outs[7];
    int no = 0;
    for (int i = 0; i < 3; ++i) {
        outs[no++] = Span{(uintptr_t)out_re[i], (uintptr_t)out_re[i] + bytes};
        if (out_im[i]) outs[no++] = Span{(uintptr_t)out_im[i], (uintptr_t)out_im[i] + bytes};
    }
    if (db_rows) outs[no++] = Span{(uintptr_t)db_rows, (uintptr_t)db_rows + rbytes};
    for (int a = 0; a < no; ++a) {
        for (int b = 0; b < ni; ++b)
            if (overlaps(outs[a], ins[b])) return CATTN_E_ALIAS;
        for (int b = a + 1; b < no; ++b)
            if (overlaps(outs[a], outs[b])) return CATTN_E_ALIAS;
    }

    p->op = op;
    p->layout = c64 ? cattn::LAYOUT_C64 : cattn::LAYOUT_BF16;
    p->q_re = in_re[0]; p->q_im = in_im[0];
    p->k_re = in_re[1]; p->k_im = in_im[1];
    p->v_re = in_re[2]; p->v_im = in_im[2];
    p->o_re = in_re[3]; p->o_im = in_im[3];
    p->g_re = in_re[4]; p->g_im = in_im[4];
    p->row_den = row_den;
    p->dq_re = out_re[0]; p->dq_im = out_im[0];
    p->dk_re = out_re[1]; p->dk_im = out_im[1];
    p->dv_re = out_re[2]; p->dv_im = out_im[2];
    p->db_rows = db_rows;
    p->BH = (int)BH;
    p->H = (int)H;
    p->T = (int)T;
    p->d = (int)d_h;
    p->causal = causal != 0;
    p->bias = bias;
    p->stream = reinterpret_cast<hipStream_t>(stream);
    return CATTN_OK;
}

cattn_status run_bwd(const cattn::BwdProblem &p) {
    hipError_t e;
    if (cattn::supports_born_bf16_d64_bwd(p)) {
        e = cattn::launch_born_bf16_d64_bwd_dkdv(p);
        if (e == hipSuccess) e = cattn::launch_born_bf16_d64_bwd_dq(p);
    } else if (cattn::supports_bwd_f32_mfma16(p)) {
        e = cattn::launch_bwd_f32_mfma16(p);
    } else if (cattn::supports_bwd_f32_mfma(p)) {
        e = cattn::launch_bwd_f32_mfma(p);
    } else {
        e = cattn::launch_bwd_generic(p);
    }
    return e == hipSuccess ? CATTN_OK : CATTN_E_LAUNCH;
}

}  // namespace

extern "C" {

cattn_status cattn_born_fwd(int layout, const void *q_re, const void *q_im, const void *k_re, const void *k_im,
                            const void *v_re, const void *v_im, void *o_re, void *o_im, int64_t B, int64_t H,
                            int64_t T, int64_t d_h, const cattn_strides *strides, int causal, float eps,
                            float *row_den, const cattn_born_opts *opts, void *stream) {
    Problem p{};
    bool empty = false;
    cattn_status s = validate(cattn::OP_BORN, layout, q_re, q_im, k_re, k_im, v_re, v_im, o_re, o_im, B, H, T,
                              d_h, strides, causal, eps, 0.f, row_den, stream, &p, &empty);
    if (s != CATTN_OK) return s;
    if (opts) {
        if (!isfinite(opts->rotary_base) || opts->rotary_base < 0.f) return CATTN_E_ARG;
        if (opts->rotary_pos0 < 0 || opts->rotary_pos0 > ((int64_t)1 << 40)) return CATTN_E_ARG;
        s = resolve_decay(opts->decay, H, causal, &p.decay);
        if (s != CATTN_OK) return s;
        if (opts->rotary_base > 0.f) {
            p.rot = 1;
            p.rot_pos0 = opts->rotary_pos0;
            p.rot_log_base = log((double)opts->rotary_base);
        }
    }
    if (empty) return CATTN_OK;
    return run(p);
}

cattn_status cattn_pct_fwd(int layout, const void *q_re, const void *q_im, const void *k_re, const void *k_im,
                           const void *v_re, const void *v_im, void *o_re, void *o_im, int64_t B, int64_t H,
                           int64_t T, int64_t d_h, const cattn_strides *strides, int causal, float bias,
                           void *stream) {
    Problem p{};
    bool empty = false;
    const cattn_status s = validate(cattn::OP_PCT, layout, q_re, q_im, k_re, k_im, v_re, v_im, o_re, o_im, B, H,
                                    T, d_h, strides, causal, 0.f, bias, nullptr, stream, &p, &empty);
    if (s != CATTN_OK || empty) return s;
    return run(p);
}

cattn_status cattn_pct_gate_fwd(int layout, const void *q_re, const void *q_im, const void *k_re,
                                const void *k_im, const void *v_re, const void *v_im, void *o_re, void *o_im,
                                int64_t B, int64_t H, int64_t T, int64_t d_h, const cattn_strides *strides,
                                int causal, int gate, float a, float b, void *stream) {
    int op;
    switch (gate) {
        case CATTN_GATE_SIGMOID: op = cattn::OP_PCT; break;
        case CATTN_GATE_SOFTMAX: op = cattn::OP_PCT_SOFTMAX; break;
        case CATTN_GATE_SCREEN: op = cattn::OP_PCT_SCREEN; break;
        default: return CATTN_E_ARG;
    }
    Problem p{};
    bool empty = false;
    const cattn_status s = validate(op, layout, q_re, q_im, k_re, k_im, v_re, v_im, o_re, o_im, B, H, T, d_h, strides,
                                    causal, 0.f, gate == CATTN_GATE_SIGMOID ? a : 0.f, nullptr, stream, &p, &empty,
                                    gate == CATTN_GATE_SCREEN ? a : 0.f, gate == CATTN_GATE_SCREEN ? b : 0.f);
    if (s != CATTN_OK || empty) return s;
    return run(p);
}

cattn_status cattn_born_bwd(int layout, const void *q_re, const void *q_im, const void *k_re, const void *k_im,
                            const void *v_re, const void *v_im, const void *o_re, const void *o_im,
                            const void *g_re, const void *g_im, const float *row_den, void *dq_re, void *dq_im,
                            void *dk_re, void *dk_im, void *dv_re, void *dv_im, int64_t B, int64_t H, int64_t T,
                            int64_t d_h, int causal, const float *decay, void *stream) {
    const void *const in_re[5] = {q_re, k_re, v_re, o_re, g_re};
    const void *const in_im[5] = {q_im, k_im, v_im, o_im, g_im};
    void *const out_re[3] = {dq_re, dk_re, dv_re};
    void *const out_im[3] = {dq_im, dk_im, dv_im};
    cattn::BwdProblem p{};
    bool empty = false;
    cattn_status s = validate_bwd(cattn::OP_BORN, layout, in_re, in_im, row_den, out_re, out_im, nullptr, B, H,
                                  T, d_h, causal, 0.f, stream, &p, &empty);
    if (s != CATTN_OK) return s;
    s = resolve_decay(decay, H, causal, &p.decay);
    if (s != CATTN_OK || empty) return s;
    return run_bwd(p);
}

cattn_status cattn_pct_bwd(int layout, const void *q_re, const void *q_im, const void *k_re, const void *k_im,
                           const void *v_re, const void *v_im, const void *g_re, const void *g_im, void *dq_re,
                           void *dq_im, void *dk_re, void *dk_im, void *dv_re, void *dv_im, int64_t B, int64_t H,
                           int64_t T, int64_t d_h, int causal, float bias, float *db_rows, void *stream) {
    const void *const in_re[5] = {q_re, k_re, v_re, nullptr, g_re};
    const void *const in_im[5] = {q_im, k_im, v_im, nullptr, g_im};
    void *const out_re[3] = {dq_re, dk_re, dv_re};
    void *const out_im[3] = {dq_im, dk_im, dv_im};
    cattn::BwdProblem p{};
    bool empty = false;
    const cattn_status s = validate_bwd(cattn::OP_PCT, layout, in_re, in_im, nullptr, out_re, out_im, db_rows, B, H,
                                        T, d_h, causal, bias, stream, &p, &empty);
    if (s != CATTN_OK || empty) return s;
    return run_bwd(p);
}

cattn_status cattn_rotary(int layout, const void *x_re, const void *x_im, void *y_re, void *y_im, int64_t B,
                          int64_t H, int64_t T, int64_t d_h, int64_t pos0, float base, void *stream) {
    if (layout != CATTN_LAYOUT_C64 && layout != CATTN_LAYOUT_BF16_PLANES) return CATTN_E_LAYOUT;
    if (!isfinite(base) || !(base > 0.f)) return CATTN_E_ARG;
    if (pos0 < 0 || pos0 > ((int64_t)1 << 40)) return CATTN_E_ARG;
    if (B < 0 || H < 0 || T < 0 || d_h < 0) return CATTN_E_SHAPE;
    if (d_h < 1 || d_h > CATTN_MAX_DH) return CATTN_E_UNSUPPORTED;
    if (T > CATTN_MAX_T || H > INT32_MAX || B > INT32_MAX) return CATTN_E_SHAPE;
    const int64_t BH = B * H;
    const int64_t elem = layout == CATTN_LAYOUT_C64 ? 8 : 2;
    if (BH != 0 && T > (int64_t)(INT64_MAX / 16) / BH / d_h / elem) return CATTN_E_SHAPE;
    if (BH == 0 || T == 0) return CATTN_OK;
    const bool c64 = layout == CATTN_LAYOUT_C64;
    if (!x_re || !y_re || (c64 ? (x_im || y_im) : (!x_im || !y_im))) return CATTN_E_NULL;
    for (const void *q : {(const void *)x_re, (const void *)x_im, (const void *)y_re, (const void *)y_im})
        if (q && !aligned16(q)) return CATTN_E_ALIGN;
    // the output either is the input (in place, plane by plane) or overlaps nothing
    const uintptr_t bytes = (uintptr_t)(BH * T * d_h * elem);
    auto span = [bytes](const void *q) { return Span{(uintptr_t)q, (uintptr_t)q + bytes}; };
    const void *xs[2] = {x_re, x_im};
    const void *ys[2] = {y_re, y_im};
    for (int a = 0; a < 2; ++a) {
        if (!ys[a]) continue;
        for (int b = 0; b < 2; ++b)
            if (xs[b] && overlaps(span(ys[a]), span(xs[b])) && !(a == b && ys[a] == xs[b])) return CATTN_E_ALIAS;
    }
    if (y_im && overlaps(span(y_re), span(y_im))) return CATTN_E_ALIAS;
    cattn::RotaryProblem p{};
    p.layout = c64 ? cattn::LAYOUT_C64 : cattn::LAYOUT_BF16;
    p.x_re = x_re; p.x_im = x_im; p.y_re = y_re; p.y_im = y_im;
    p.rows = BH * T;
    p.BH = BH;
    p.T = (int)T;
    p.d = (int)d_h;
    p.pos0 = pos0;
    p.log_base = log((double)base);
    p.stream = reinterpret_cast<hipStream_t>(stream);
    return cattn::launch_rotary(p) == hipSuccess ? CATTN_OK : CATTN_E_LAUNCH;
}

namespace {

// Shared checks of the carried-state calls: layout, sizes (d_h <= 64), the
// complex operands (NULL and alignment rules of the forward), the state and
// row_den buffers, and that no written buffer overlaps another buffer.
struct Buf {
    const void *p;
    uintptr_t bytes;
    bool written;
};

cattn_status check_linear(int layout, int64_t B, int64_t H, int64_t T, int64_t d_h, const void *const *cre,
                          const void *const *cim, const bool *cwritten, int nc, const Buf *extra, int ne,
                          cattn::LinearProblem *p, bool *empty) {
    if (layout != CATTN_LAYOUT_C64 && layout != CATTN_LAYOUT_BF16_PLANES) return CATTN_E_LAYOUT;
    if (B < 0 || H < 0 || T < 0 || d_h < 0) return CATTN_E_SHAPE;
    if (d_h < 1 || d_h > CATTN_LIN_MAXD) return CATTN_E_UNSUPPORTED;
    if (T > CATTN_MAX_T || H > INT32_MAX || B > INT32_MAX) return CATTN_E_SHAPE;
    const int64_t BH = B * H;
    if (BH > INT32_MAX) return CATTN_E_SHAPE;
    const int64_t elem = layout == CATTN_LAYOUT_C64 ? 8 : 2;
    if (BH != 0 && T > (int64_t)(INT64_MAX / 16) / BH / d_h / elem) return CATTN_E_SHAPE;
    *empty = BH == 0 || T == 0;
    if (*empty) return CATTN_OK;
    const bool c64 = layout == CATTN_LAYOUT_C64;
    Buf all[16];
    int n = 0;
    for (int i = 0; i < nc; ++i) {
        if (!cre[i] || (c64 ? cim[i] != nullptr : cim[i] == nullptr)) return CATTN_E_NULL;
        if (!aligned16(cre[i]) || (cim[i] && !aligned16(cim[i]))) return CATTN_E_ALIGN;
        const uintptr_t bytes = (uintptr_t)(BH * T * d_h * elem);
        all[n++] = Buf{cre[i], bytes, cwritten[i]};
        if (cim[i]) all[n++] = Buf{cim[i], bytes, cwritten[i]};
    }
    for (int i = 0; i < ne; ++i) {
        if (!extra[i].p) return CATTN_E_NULL;
        if (!aligned16(extra[i].p)) return CATTN_E_ALIGN;
        all[n++] = extra[i];
    }
    for (int a = 0; a < n; ++a)
        for (int b = a + 1; b < n; ++b)
            if ((all[a].written || all[b].written) &&
                overlaps(Span{(uintptr_t)all[a].p, (uintptr_t)all[a].p + all[a].bytes},
                         Span{(uintptr_t)all[b].p, (uintptr_t)all[b].p + all[b].bytes}))
                return CATTN_E_ALIAS;
    p->layout = c64 ? cattn::LAYOUT_C64 : cattn::LAYOUT_BF16;
    p->BH = (int)BH;
    p->H = (int)H;
    p->T = (int)T;
    p->d = (int)d_h;
    return CATTN_OK;
}

uintptr_t s_bytes(int64_t B, int64_t H, int64_t d) { return (uintptr_t)(B * H * (2 * d + 1) * d * d * 4); }

}  // namespace

cattn_status cattn_born_state(int layout, const void *k_re, const void *k_im, const void *v_re, const void *v_im,
                              int64_t B, int64_t H, int64_t T, int64_t d_h, float *S, int accumulate,
                              const float *decay, void *stream) {
    const void *cre[2] = {k_re, v_re}, *cim[2] = {k_im, v_im};
    const bool cw[2] = {false, false};
    const Buf extra[1] = {{S, s_bytes(B, H, d_h), true}};
    cattn::LinearProblem p{};
    bool empty = false;
    if (H >= 0) {
        const cattn_status s = resolve_decay(decay, H, 1, &p.decay);
        if (s != CATTN_OK) return s;
    }
    if (T == 0 && !accumulate) {
        // no tokens, overwrite: the state becomes zero (k and v are not read)
        const cattn_status s = check_linear(layout, B, H, 1, d_h, nullptr, nullptr, nullptr, 0, extra, 1, &p, &empty);
        if (s != CATTN_OK || empty) return s;
        p.T = 0;
    } else {
        const cattn_status s = check_linear(layout, B, H, T, d_h, cre, cim, cw, 2, extra, 1, &p, &empty);
        if (s != CATTN_OK || empty) return s;
    }
    p.k_re = k_re; p.k_im = k_im; p.v_re = v_re; p.v_im = v_im;
    p.S = S;
    p.accumulate = accumulate != 0;
    p.stream = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = cattn::supports_born_linear_bf16_d64(p) ? cattn::launch_born_state_bf16_d64(p)
                         : cattn::supports_born_linear_f32(p)     ? cattn::launch_born_state_f32(p)
                                                                  : cattn::launch_born_state(p);
    return e == hipSuccess ? CATTN_OK : CATTN_E_LAUNCH;
}

cattn_status cattn_born_merge(int layout, const void *q_re, const void *q_im, const float *S, void *o_re,
                              void *o_im, float *row_den, int64_t B, int64_t H, int64_t T, int64_t d_h,
                              const float *decay, void *stream) {
    const void *cre[2] = {q_re, o_re}, *cim[2] = {q_im, o_im};
    const bool cw[2] = {false, true};
    const Buf extra[2] = {{S, s_bytes(B, H, d_h), false}, {row_den, (uintptr_t)(B * H * T * 4), true}};
    cattn::LinearProblem p{};
    bool empty = false;
    if (H >= 0) {
        const cattn_status s = resolve_decay(decay, H, 1, &p.decay);
        if (s != CATTN_OK) return s;
    }
    const cattn_status s = check_linear(layout, B, H, T, d_h, cre, cim, cw, 2, extra, 2, &p, &empty);
    if (s != CATTN_OK || empty) return s;
    p.q_re = q_re; p.q_im = q_im; p.o_re = o_re; p.o_im = o_im;
    p.S = const_cast<float *>(S);   // read only in this call
    p.row_den = row_den;
    p.stream = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = cattn::supports_born_linear_bf16_d64(p) ? cattn::launch_born_merge_bf16_d64(p)
                         : cattn::supports_born_linear_f32(p)     ? cattn::launch_born_merge_f32(p)
                                                                  : cattn::launch_born_merge(p);
    return e == hipSuccess ? CATTN_OK : CATTN_E_LAUNCH;
}

cattn_status cattn_born_step(int layout, const void *q_re, const void *q_im, const void *k_re, const void *k_im,
                             const void *v_re, const void *v_im, void *o_re, void *o_im, float *S,
                             float *row_den, int64_t B, int64_t H, int64_t d_h, float eps, const float *decay,
                             void *stream) {
    if (!isfinite(eps) || eps < 0.f) return CATTN_E_ARG;
    cattn::LinearProblem p{};
    if (H >= 0) {
        const cattn_status s = resolve_decay(decay, H, 1, &p.decay);
        if (s != CATTN_OK) return s;
    }
    const void *cre[4] = {q_re, k_re, v_re, o_re}, *cim[4] = {q_im, k_im, v_im, o_im};
    const bool cw[4] = {false, false, false, true};
    const Buf extra[2] = {{S, s_bytes(B, H, d_h), true}, {row_den, (uintptr_t)(B * H * 4), true}};
    bool empty = false;
    const cattn_status s = check_linear(layout, B, H, 1, d_h, cre, cim, cw, 4, extra, 2, &p, &empty);
    if (s != CATTN_OK || empty) return s;
    p.q_re = q_re; p.q_im = q_im; p.k_re = k_re; p.k_im = k_im; p.v_re = v_re; p.v_im = v_im;
    p.o_re = o_re; p.o_im = o_im;
    p.S = S; p.row_den = row_den;
    p.eps = eps;
    p.stream = reinterpret_cast<hipStream_t>(stream);
    return cattn::launch_born_step(p) == hipSuccess ? CATTN_OK : CATTN_E_LAUNCH;
}

const char *cattn_status_str(cattn_status status) {
    switch (status) {
        case CATTN_OK: return "ok";
        case CATTN_E_NULL: return "required pointer is NULL (or an imaginary-plane pointer was given for complex64)";
        case CATTN_E_SHAPE: return "negative or too large size";
        case CATTN_E_LAYOUT: return "unknown layout";
        case CATTN_E_ALIGN: return "pointer not 16-byte aligned";
        case CATTN_E_ALIAS: return "an output overlaps an input or another output";
        case CATTN_E_UNSUPPORTED: return "head width d_h outside 1..128 (1..64 for the carried-state calls), or too many heads for a decay table";
        case CATTN_E_LAUNCH: return "HIP kernel launch failed";
        case CATTN_E_ARG: return "a scalar argument out of range (eps, bias, gate parameters, rotary base or position, a decay value), decay on a non-causal call, or an unknown gate";
        default: return "unknown status";
    }
}

int cattn_abi_version(void) { return 8; }

}  // extern "C"
