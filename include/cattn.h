/*
 * cattn.h -- fused forward and backward passes of complex-valued attention on
 * AMD Instinct gfx950 (CDNA4).  C ABI: plain pointers and sizes, no C++ or
 * framework types.
 *
 * Two operators, both ending in O = W V over complex values V:
 *
 *   Born-rule attention ("CNet: A Complex-Valued Deep Learning Framework with
 *   Wirtinger Autodifferentiation and FFT-Hadamard Convolution", section 11.2,
 *   paragraph "Closing it: Born-rule attention", Figure 2):
 *       S[k,j] = sum_m Q[k,m] conj(K[j,m])          (Hermitian inner product)
 *       w[k,j] = |S[k,j]|^2
 *       O[k]   = sum_{j in J(k)} w[k,j] V[j] / (sum_{j in J(k)} w[k,j] + eps)
 *   A row whose denominator is 0 is written as 0.
 *
 *   Phase-coherent (PCT) attention ("Complex-valued Phase-Coherent
 *   Transformers", section 1 and Appendix D.2, the PCT cell):
 *       s[i,j] = sqrt(d_h) Re < q_i/||q_i||, k_j/||k_j|| >
 *       w[i,j] = sigmoid(s[i,j] + bias)
 *       O[i]   = sum_{j in J(i)} w[i,j] V[j]             (no row normalisation)
 *   A zero-norm q or k contributes score 0 (weight sigmoid(bias)).
 *
 * J(k) = {0..k} if causal != 0, else {0..T-1}.
 *
 * Tensors.  Q, K, V and O are [B, H, T, d_h] in DEVICE memory owned by the
 * caller; the library allocates nothing and keeps no state.  The d_h
 * components of a row are contiguous.  The forward calls take element
 * strides for the batch, head and token dimensions of each operand
 * (cattn_strides below), so Q, K and V may be views into one fused
 * projection output; every other call takes dense row-major tensors.  Two
 * layouts:
 *   CATTN_LAYOUT_C64        interleaved complex64 (float re, float im); pass
 *                           the tensor in the *_re argument, *_im must be NULL.
 *   CATTN_LAYOUT_BF16_PLANES two bf16 tensors per operand, real plane in *_re
 *                           and imaginary plane in *_im.
 * O is written in the layout of the inputs and fully overwritten.
 * Arithmetic: bf16 planes use bf16 matrix-core products with fp32
 * accumulation; complex64 uses fp32 throughout.
 *
 * Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 * stream of the current device) and run on the current HIP device.
 *
 * Errors.  All argument checks happen before any HIP call; on an argument
 * error nothing is enqueued and a status other than CATTN_OK is returned.
 * A failed kernel launch returns CATTN_E_LAUNCH.  Faults inside a kernel
 * surface at the caller's next synchronisation.  Sizes B, H or T equal to 0
 * are an empty problem: CATTN_OK, nothing enqueued.
 */
#ifndef CATTN_H
#define CATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CATTN_OK = 0,
    CATTN_E_NULL = 1,        /* a required pointer is NULL, or *_im is non-NULL for C64 */
    CATTN_E_SHAPE = 2,       /* a size is negative, or the byte size overflows int64 */
    CATTN_E_LAYOUT = 3,      /* unknown layout value */
    CATTN_E_ALIGN = 4,       /* a pointer is misaligned: forward calls need element alignment, other calls 16 bytes */
    CATTN_E_ALIAS = 5,       /* an output overlaps an input or another output */
    CATTN_E_UNSUPPORTED = 6, /* d_h outside 1..128 (1..64 for the carried-state calls), or H above
                                CATTN_MAX_DECAY_HEADS with a decay table */
    CATTN_E_LAUNCH = 7,      /* the HIP kernel launch failed */
    CATTN_E_ARG = 8          /* a scalar out of range: eps, bias, a gate parameter, rotary base or position,
                                a decay value; decay on a non-causal call; or an unknown gate */
} cattn_status;

/* Gates on the PCT score path ("Complex-valued Phase-Coherent Transformers",
 * Appendix D.2, the family's cells). */
typedef enum {
    CATTN_GATE_SIGMOID = 0,  /* w = sigmoid(s + a): the PCT cell (as cattn_pct_fwd, bias a) */
    CATTN_GATE_SOFTMAX = 1,  /* w = exp(s) / sum_{j in J(i)} exp(s): the L2-softmax cell */
    CATTN_GATE_SCREEN = 2    /* w = a^2 max(s - b, 0)^2: the screening gate (r = a, t = b) */
} cattn_gate;

typedef enum {
    CATTN_LAYOUT_C64 = 0,
    CATTN_LAYOUT_BF16_PLANES = 1
} cattn_layout;

/* Largest head width accepted. */
#define CATTN_MAX_DH 128

/* Largest sequence length accepted (2^30), so that token indices plus a tile
 * never overflow 32-bit arithmetic inside the kernels. */
#define CATTN_MAX_T (1 << 30)

/*
 * Element strides of one [B, H, T, d_h] operand: how far apart, in elements
 * of the layout, consecutive batches (b), heads (h) and tokens (t) sit.  An
 * element is one complex64 value for CATTN_LAYOUT_C64 and one bf16 value of
 * a plane for CATTN_LAYOUT_BF16_PLANES (both planes of an operand share the
 * strides).  The d_h components of a row are always contiguous.  A stride of
 * 0 stands for the dense value (b: H*T*d_h, h: T*d_h, t: d_h); a negative
 * stride is CATTN_E_SHAPE.
 *
 * Example: the pages' BornAttention layer ("Show HN: CNET", BornAttention)
 * takes Q, K and V as one concatenated input.  From a complex64 projection
 * output P laid out [B, T, 3, H, d_h], the views are q = P + 0*H*d_h,
 * k = P + 1*H*d_h, v = P + 2*H*d_h, each with strides
 * {b = 3*T*H*d_h, h = d_h, t = 3*H*d_h}, and no copy is needed.
 */
typedef struct {
    int64_t b, h, t;
} cattn_stride;

/* Strides of the four operands of a forward call (12 consecutive int64). */
typedef struct {
    cattn_stride q, k, v, o;
} cattn_strides;

/* Largest head count H for which a per-head decay table is accepted. */
#define CATTN_MAX_DECAY_HEADS 256

/*
 * Per-head decay (a reading of "Show HN: CNET", BornAttention: a fixed
 * per-head decay that multiplies the score, the page's best fix for long
 * contexts, run together with the linear mode; the page's formula is lost in
 * its text).  For causal attention and gamma_h in (0, 1] the weight of key j
 * for query k of head h becomes
 *     w[k,j] = gamma_h^(k-j) |S[k,j]|^2,   j <= k,
 * the one fixed per-head factor that a carried state reproduces by
 * Z <- gamma_h Z + k k^H (cattn_born_state, _merge, _step below).  gamma_h = 1
 * is plain Born attention.
 * A decay table is a HOST array of H floats, read during the call and not
 * kept; NULL means no decay.  Errors: CATTN_E_ARG if the call is not causal
 * or a value lies outside (0, 1] (NaN included); CATTN_E_UNSUPPORTED if
 * H > CATTN_MAX_DECAY_HEADS.
 */

/*
 * Options of cattn_born_fwd (NULL: none of them).
 *   decay         NULL or a decay table (above).
 *   rotary_base   0: Q is used as given.  > 0 and finite: each query row t
 *                 is rotated as it is loaded, q[t,m] exp(i (rotary_pos0 + t)
 *                 theta_m) with theta_m = rotary_base^(-m/d_h), the
 *                 arithmetic of cattn_rotary ("Show HN: CNET", RotaryEmbed);
 *                 K is taken as given, i.e. already rotated (as a key cache
 *                 holds it), so this replaces a cattn_rotary pass over Q.
 *   rotary_pos0   absolute position of token 0, 0 <= rotary_pos0 <= 2^40.
 * Errors: CATTN_E_ARG for a negative or non-finite rotary_base or a
 * rotary_pos0 out of range.
 */
typedef struct {
    const float *decay;
    float rotary_base;
    int64_t rotary_pos0;
} cattn_born_opts;

/*
 * Born-rule attention forward (definition above).
 *   layout        CATTN_LAYOUT_C64 or CATTN_LAYOUT_BF16_PLANES.
 *   q_*, k_*, v_* inputs, o_* output (device pointers, see "Tensors").
 *   B, H, T, d_h  batch, heads, sequence length, head width (complex
 *                 components per token); 1 <= d_h <= CATTN_MAX_DH,
 *                 T <= CATTN_MAX_T.
 *   strides       NULL (every operand dense) or the element strides of
 *                 Q, K, V and O (see cattn_strides).  Rows of O must not
 *                 share memory (CATTN_E_ALIAS).  Each operand spans the bytes
 *                 from its base to the end of its last row; O's span must
 *                 not overlap an input's or row_den's, while the inputs'
 *                 spans may overlap each other (views of one buffer).
 *                 Pointers must be aligned to their element (8 bytes for
 *                 complex64, 2 for bf16, 4 for row_den); strides need no
 *                 alignment.  The matrix-core kernels run when every base
 *                 pointer and every stride is a multiple of 16 bytes (always
 *                 so for dense tensors from a 16-byte aligned allocation),
 *                 an element-wise kernel otherwise.
 *   causal        non-zero: query k sees keys 0..k; zero: all keys.
 *   eps           added to each row denominator; >= 0 and finite.
 *   row_den       optional (NULL allowed) device float[B*H*T]: receives each
 *                 row's denominator sum_j w + eps.
 *   opts          NULL or the decay and rotary options (cattn_born_opts).
 *   stream        hipStream_t to enqueue on.
 */
cattn_status cattn_born_fwd(int layout,
                            const void *q_re, const void *q_im,
                            const void *k_re, const void *k_im,
                            const void *v_re, const void *v_im,
                            void *o_re, void *o_im,
                            int64_t B, int64_t H, int64_t T, int64_t d_h,
                            const cattn_strides *strides,
                            int causal, float eps, float *row_den,
                            const cattn_born_opts *opts, void *stream);

/*
 * Phase-coherent (PCT) attention forward (definition above).  Arguments as
 * for cattn_born_fwd; `bias` is the gate bias b (finite; the pages
 * initialise it to -log N, 0 gives a plain sigmoid of the score).
 */
cattn_status cattn_pct_fwd(int layout,
                           const void *q_re, const void *q_im,
                           const void *k_re, const void *k_im,
                           const void *v_re, const void *v_im,
                           void *o_re, void *o_im,
                           int64_t B, int64_t H, int64_t T, int64_t d_h,
                           const cattn_strides *strides,
                           int causal, float bias, void *stream);

/*
 * PCT-family forward with a choice of gate on the same scaled cosine score
 * s[i,j] = sqrt(d_h) Re < q_i/||q_i||, k_j/||k_j|| >  (|s| <= sqrt(d_h)):
 *   gate CATTN_GATE_SIGMOID  O[i] = sum_j sigmoid(s[i,j] + a) V[j]
 *   gate CATTN_GATE_SOFTMAX  O[i] = sum_j exp(s[i,j]) V[j] / sum_j exp(s[i,j])
 *                            (a and b unused; the score bound keeps exp finite)
 *   gate CATTN_GATE_SCREEN   O[i] = sum_j a^2 max(s[i,j] - b, 0)^2 V[j]
 * with j over J(i).  The screening cell's TanhNorm of the aggregate and its
 * modReLU gate act after this sum and are not part of it.  Other arguments
 * as for cattn_pct_fwd; a and b must be finite where used; an unknown gate
 * is CATTN_E_ARG.
 */
cattn_status cattn_pct_gate_fwd(int layout,
                                const void *q_re, const void *q_im,
                                const void *k_re, const void *k_im,
                                const void *v_re, const void *v_im,
                                void *o_re, void *o_im,
                                int64_t B, int64_t H, int64_t T, int64_t d_h,
                                const cattn_strides *strides,
                                int causal, int gate, float a, float b, void *stream);

/*
 * Backward passes.  Gradients follow the Wirtinger convention of "CNet ..."
 * (section 3, the accumulation rule (2) and the CModulus2 worked example):
 * for a real loss L the caller passes G = dL/d(conj O) and receives
 * dL/d(conj q), dL/d(conj k), dL/d(conj v).  The map is linear in G, so
 * passing the real-pair gradient dL/dRe O + i dL/dIm O (the convention of
 * torch's complex autograd) returns real-pair gradients.  The closed forms
 * (derived from the forward definitions; section 11.2 of the same page states
 * that Born attention's backward exists in closed form):
 *
 *   Born, with l = row_den, delta[k] = Re(G[k]^H O[k]) and, for j in J(k),
 *   D[k,j] = (Re(G[k]^H V[j]) - delta[k]) / l[k]:
 *       dV[j] = sum_k w[k,j] / l[k] G[k]
 *       dQ[k] = sum_j 2 D[k,j] S[k,j] K[j]
 *       dK[j] = sum_k 2 D[k,j] conj(S[k,j]) Q[k]
 *   A row with l[k] == 0 contributes nothing.
 *
 *   PCT, with qh, kh the unit rows and ds[i,j] = Re(G[i]^H V[j]) w (1 - w):
 *       dV[j] = sum_i w[i,j] G[i]
 *       dq[i] = P(qh[i], sqrt(d_h) sum_j ds[i,j] kh[j]) / ||q[i]||
 *       dk[j] = P(kh[j], sqrt(d_h) sum_i ds[i,j] qh[i]) / ||k[j]||
 *   where P(u, x) = x - Re(x^H u) u; a zero-norm row gets gradient 0.
 *
 * Arguments as for the forward, plus:
 *   o_*        Born: the forward output O (same layout).
 *   g_*        the incoming gradient G (same layout).
 *   row_den    Born: device float[B*H*T], the forward's row denominators
 *              (sum_j w + eps), required.
 *   decay      Born: NULL or the forward's decay table (see "Per-head
 *              decay"); every w[k,j] above, in dV and in D alike, then
 *              carries the factor gamma_h^(k-j).
 *   dq_*, dk_*, dv_*  outputs (same layout), fully overwritten.
 *   db_rows    PCT: optional (NULL allowed) device float[B*H*T], receives
 *              sum_j ds[i,j] per query row; their sum is dL/d(bias).
 * The outputs must not overlap any input or each other.  The arithmetic is
 * fp32 for both layouts (bf16 inputs are widened, outputs rounded to bf16).
 * Each call enqueues two kernels (key-side and query-side gradients), and on
 * the bf16 Born path at d_h = 64 and the Born path at d_h = 128 (either
 * layout) a third before them that writes per-query scalars into the dq_re
 * buffer for the key-side kernel (the query-side kernel then overwrites it);
 * it allocates nothing, uses no atomics and is deterministic.
 */
cattn_status cattn_born_bwd(int layout,
                            const void *q_re, const void *q_im,
                            const void *k_re, const void *k_im,
                            const void *v_re, const void *v_im,
                            const void *o_re, const void *o_im,
                            const void *g_re, const void *g_im,
                            const float *row_den,
                            void *dq_re, void *dq_im,
                            void *dk_re, void *dk_im,
                            void *dv_re, void *dv_im,
                            int64_t B, int64_t H, int64_t T, int64_t d_h,
                            int causal, const float *decay, void *stream);

cattn_status cattn_pct_bwd(int layout,
                           const void *q_re, const void *q_im,
                           const void *k_re, const void *k_im,
                           const void *v_re, const void *v_im,
                           const void *g_re, const void *g_im,
                           void *dq_re, void *dq_im,
                           void *dk_re, void *dk_im,
                           void *dv_re, void *dv_im,
                           int64_t B, int64_t H, int64_t T, int64_t d_h,
                           int causal, float bias, float *db_rows, void *stream);

/*
 * Rotary phase embedding ("Show HN: CNET", the RotaryEmbed layer: position
 * as a complex phase rotation, base 10000, an absolute position for the
 * one-token step mode):
 *     y[b,h,t,m] = x[b,h,t,m] * exp(i (pos0 + t) theta_m),  theta_m = base^(-m/d_h)
 * over [B, H, T, d_h] tensors in either layout.  y may be x itself (in
 * place, same pointers) or must not overlap it.  base > 0 and finite;
 * 0 <= pos0 <= 2^40.  The angle is reduced modulo 2 pi in fp64, so long
 * positions keep full fp32 accuracy.  Allocates nothing; asynchronous on
 * stream.
 */
cattn_status cattn_rotary(int layout,
                          const void *x_re, const void *x_im,
                          void *y_re, void *y_im,
                          int64_t B, int64_t H, int64_t T, int64_t d_h,
                          int64_t pos0, float base, void *stream);

/*
 * Born attention with a carried density state ("Show HN: CNET",
 * BornAttention's linear and step modes: each key lifted to its outer
 * product, a running state, constant-memory decoding; "The Quantum Shortcut",
 * section 2: the Born rule as q^H rho q with rho = k k^H).  Per head:
 *     Z    = sum_j k_j k_j^H            (d_h x d_h)
 *     M[c] = sum_j V[j,c] k_j k_j^H      (d_h x d_h per value channel c)
 *     O[t,c] = q_t^H M_t[c] q_t / (q_t^H Z_t q_t + eps)
 * where the states at token t hold the carried keys and every key of the
 * sequence up to t.  This is exactly Born attention (the feature map is
 * finite), with O(1) memory per decoded token.
 *
 * State layout (device, caller-owned, fp32): S [B, H, 2 d_h + 1, d_h, d_h],
 * 2 d_h + 1 real matrices per head, each the packed form of a Hermitian
 * matrix X_n:
 *     X_c        = sum_j Re V[j,c] k_j k_j^H     (n = c < d_h)
 *     X_{d_h+c}  = sum_j Im V[j,c] k_j k_j^H     (so M[c] = X_c + i X_{d_h+c})
 *     X_{2 d_h}  = Z
 * packed as S[n][a][b] = Re X_n[a][b] for a <= b and Im X_n[b][a] for a > b.
 * The state is (2 d_h + 1) d_h^2 floats per head: 2.02 MiB at d_h = 64.
 * The carried-state calls take 1 <= d_h <= 64.
 *
 * cattn_born_state: S over the T tokens of k, v; accumulate != 0 adds to the
 *     buffer's contents, 0 overwrites it (T = 0 then zeroes the state, and
 *     k, v may be NULL).
 * cattn_born_merge: prefill with an incoming state.  Given the output O and
 *     row denominators l of cattn_born_fwd (causal) over this call's tokens,
 *     folds in the incoming state:
 *         O <- (O l + q^H M q) / (l + q^H Z q),   l <- l + q^H Z q.
 *     Then cattn_born_state(accumulate = 1) carries the call's own tokens out.
 * cattn_born_step: one token per head (q, k, v, o are [B, H, 1, d_h]): adds
 *     (k, v) to the state in place, then writes o and row_den[b*H + h] =
 *     q^H Z q + eps.  For bf16 the numerator is rounded once to bf16 before
 *     the division (a second rounding of o).
 * Decay: each of these calls takes a decay table (NULL: none; see "Per-head
 *     decay"), under which every token first scales the state by gamma_h and
 *     then adds its own terms, so the state after token t holds
 *     sum_{j <= t} gamma_h^(t-j) (...):
 *     cattn_born_state  S <- gamma_h^T S + sum_t gamma_h^(T-1-t) (terms of t)
 *                       (with accumulate = 0 the old contents count as 0);
 *     cattn_born_merge  the incoming state counts gamma_h^(t+1) at token t:
 *                       O <- (O l + g q^H M q) / (l + g q^H Z q), g = gamma_h^(t+1),
 *                       which needs O and l from cattn_born_fwd with the same table;
 *     cattn_born_step   S <- gamma_h S + (terms of the token), then the read-out.
 * Written buffers must not overlap any other buffer of the call.
 */
cattn_status cattn_born_state(int layout,
                              const void *k_re, const void *k_im,
                              const void *v_re, const void *v_im,
                              int64_t B, int64_t H, int64_t T, int64_t d_h,
                              float *S, int accumulate, const float *decay, void *stream);

cattn_status cattn_born_merge(int layout,
                              const void *q_re, const void *q_im,
                              const float *S,
                              void *o_re, void *o_im, float *row_den,
                              int64_t B, int64_t H, int64_t T, int64_t d_h,
                              const float *decay, void *stream);

cattn_status cattn_born_step(int layout,
                             const void *q_re, const void *q_im,
                             const void *k_re, const void *k_im,
                             const void *v_re, const void *v_im,
                             void *o_re, void *o_im,
                             float *S, float *row_den,
                             int64_t B, int64_t H, int64_t d_h, float eps,
                             const float *decay, void *stream);

/* Static, NUL-terminated description of a status value (never NULL; an
 * unknown value gives "unknown status"). */
const char *cattn_status_str(cattn_status status);

/* ABI version of this header: 8 (2 added the backward, 3 the PCT gates, 4 rotary, 5 the carried state,
   6 its packed real layout, 7 strided operands in the forward calls, 8 per-head decay and rotary Q
   at load). */
int cattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CATTN_H */
