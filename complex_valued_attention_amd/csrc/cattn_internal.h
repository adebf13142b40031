// Internal launch interface shared by the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace cattn {

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per device (the limit is a per-device property of the function; `done`
// holds one bit per device id, and a repeated set is harmless).
inline hipError_t set_dynamic_lds(const void *kern, int bytes, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

// OP_PCT is the sigmoid cell; the two siblings share its scaled cosine score
// ("Complex-valued Phase-Coherent Transformers", Appendix D.2): the
// L2-softmax cell and the screening gate r^2 relu(s - t)^2.
enum Op : int { OP_BORN = 0, OP_PCT = 1, OP_PCT_SOFTMAX = 2, OP_PCT_SCREEN = 3 };

// Operators on the PCT score path, and operators whose weights are row-normalised.
__host__ __device__ inline bool op_pct_score(int op) { return op != OP_BORN; }
__host__ __device__ inline bool op_row_norm(int op) { return op == OP_BORN || op == OP_PCT_SOFTMAX; }
enum Layout : int { LAYOUT_C64 = 0, LAYOUT_BF16 = 1 };

// Element strides of one [B, H, T, d] operand (batch, head, token), resolved
// (never 0 for a dimension of size > 1); d is contiguous.
struct Str3 {
    int64_t b, h, t;
};

// Element offset of head bh = b * H + h.
__host__ __device__ inline int64_t head_offset(const Str3 &s, int bh, int H) {
    return (int64_t)(bh / H) * s.b + (int64_t)(bh % H) * s.h;
}

// Per-head decay of the causal Born weights, w[k, j] = gamma_h^(k - j) |S|^2:
// lg2[h] = log2(gamma_h) <= 0 (formed on the host in double precision) for
// the H heads of the call; on == 0 means no decay.  Powers are formed as
// exp2(n * lg2[h]).  Passed by value in the kernel arguments.
#define CATTN_DECAY_MAXH 256
struct Decay {
    int on;
    float lg2[CATTN_DECAY_MAXH];
};

// gamma_h^n, n >= 0
__device__ inline float decay_pow(float lg2, int n) { return __builtin_amdgcn_exp2f(lg2 * (float)n); }

// One validated forward call.  Pointers are device pointers; operand x of
// head bh, token t starts at x + head_offset(sx, bh, H) + t * sx.t (in
// elements of the layout).  B and H are folded into BH; heads never interact.
struct Problem {
    int op;
    int layout;
    const void *q_re, *q_im, *k_re, *k_im, *v_re, *v_im;
    void *o_re, *o_im;
    float *row_den;     // Born only, may be null; dense [BH, T]
    Str3 sq, sk, sv, so;
    int BH;
    int H;
    int T;
    int d;
    bool aligned16;     // every base pointer and every stride is a multiple of 16 bytes
    int causal;
    float eps;          // Born
    float bias;         // PCT sigmoid cell
    float gate_r;       // screening gate: r
    float gate_t;       // screening gate: t
    hipStream_t stream;
    // Born options (kept last: large and rarely read)
    int rot;            // rotate Q at load (the rotary phase of cattn_rotary)
    int64_t rot_pos0;
    double rot_log_base;
    Decay decay;
};

// Each launcher enqueues the whole forward for `p` and returns the launch
// status.  `supports_*` say whether a specialised kernel covers `p`.
hipError_t launch_generic(const Problem &p);

bool supports_born_bf16_d64(const Problem &p);
hipError_t launch_born_bf16_d64(const Problem &p);

// Width D (128 or 32), one translation unit each.
template <int D> bool supports_born_bf16_q16(const Problem &p);
template <int D> hipError_t launch_born_bf16_q16(const Problem &p);

bool supports_born_bf16_mfma(const Problem &p);
hipError_t launch_born_bf16_mfma(const Problem &p);

// complex64 on 16 x 16 fp32 matrix tiles, pairs of 64-query row blocks
bool supports_f32_mfma16(const Problem &p);
hipError_t launch_f32_mfma16(const Problem &p);

// One validated backward call (same [BH, T, d] layout).  G = dL/d(conj O);
// the outputs are dL/d(conj q), dL/d(conj k), dL/d(conj v).
struct BwdProblem {
    int op;
    int layout;
    const void *q_re, *q_im, *k_re, *k_im, *v_re, *v_im;
    const void *o_re, *o_im;     // Born: the forward output
    const void *g_re, *g_im;     // incoming gradient
    const float *row_den;        // Born: the forward's row denominators
    void *dq_re, *dq_im, *dk_re, *dk_im, *dv_re, *dv_im;
    float *db_rows;              // PCT: per-row bias gradient, may be null
    int BH;
    int T;
    int d;
    int causal;
    float bias;                  // PCT
    hipStream_t stream;
    int H;
    Decay decay;                 // Born
};

hipError_t launch_bwd_generic(const BwdProblem &p);        // both kernels
hipError_t launch_bwd_generic_dkdv(const BwdProblem &p);   // key-side gradients only
hipError_t launch_bwd_generic_dq(const BwdProblem &p);     // query-side gradients only

bool supports_born_bf16_d64_bwd(const BwdProblem &p);
bool supports_bwd_f32_mfma16(const BwdProblem &p);        // width 128, 16 x 16 fp32 tiles
hipError_t launch_bwd_f32_mfma16(const BwdProblem &p);    // all its kernels
bool supports_bwd_f32_mfma(const BwdProblem &p);          // complex64, widths 16/32/64
hipError_t launch_bwd_f32_mfma(const BwdProblem &p);      // both kernels
hipError_t launch_born_bf16_d64_bwd_dq(const BwdProblem &p);
hipError_t launch_born_bf16_d64_bwd_dkdv(const BwdProblem &p);

// One validated rotary call over rows = B*H*T rows of d complex channels.
struct RotaryProblem {
    int layout;
    const void *x_re, *x_im;
    void *y_re, *y_im;
    int64_t rows;      // BH * T
    int64_t BH;
    int T;
    int d;
    int64_t pos0;
    double log_base;
    hipStream_t stream;
};

hipError_t launch_rotary(const RotaryProblem &p);

// Born attention with a carried density state (state build, merge, step).
#define CATTN_LIN_MAXD 64
struct LinearProblem {
    int layout;
    const void *q_re, *q_im, *k_re, *k_im, *v_re, *v_im;
    void *o_re, *o_im;
    float *S;          // packed state [BH, 2d + 1, d, d] fp32
    float *row_den;    // merge: [BH * T] in/out; step: [BH] out
    int BH;
    int T;
    int d;
    int accumulate;    // state build: add to the state instead of overwriting it
    float eps;         // step
    hipStream_t stream;
    int H;
    Decay decay;
};

hipError_t launch_born_state(const LinearProblem &p);
hipError_t launch_born_merge(const LinearProblem &p);
hipError_t launch_born_step(const LinearProblem &p);
// matrix-core versions for bf16 planes at head width 64
bool supports_born_linear_bf16_d64(const LinearProblem &p);
hipError_t launch_born_merge_bf16_d64(const LinearProblem &p);
hipError_t launch_born_state_bf16_d64(const LinearProblem &p);
// fp32 matrix-core versions for complex64 at head widths 16, 32, 64
bool supports_born_linear_f32(const LinearProblem &p);
hipError_t launch_born_state_f32(const LinearProblem &p);
hipError_t launch_born_merge_f32(const LinearProblem &p);

}  // namespace cattn
