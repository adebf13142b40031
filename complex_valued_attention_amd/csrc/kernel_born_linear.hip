// Born attention with a carried density state ("Show HN: CNET",
// BornAttention's linear and step modes: each key lifted to its outer
// product, a running state, constant-memory decoding; "The Quantum
// Shortcut", section 2: the Born rule as q^H rho q with rho = k k^H).
//
// The state of a head is 2d + 1 Hermitian d x d matrices,
//     X_c      = sum_j Re V[j, c] k_j k_j^H        (c < d)
//     X_{d+c}  = sum_j Im V[j, c] k_j k_j^H
//     X_{2d}   = Z = sum_j k_j k_j^H
// (so M[c] = sum_j V[j, c] k_j k_j^H = X_c + i X_{d+c}), each stored as the
// real d x d matrix P with P[a][b] = Re X[a][b] for a <= b and Im X[b][a]
// for a > b.  With the real features of a vector u,
//     phi_ab(u) = Re(u_a conj u_b)  (a <= b),   Im(u_b conj u_a)  (a > b),
// the packed outer product is P(u u^H) = phi(u), and the quadratic form is
//     q^H X q = sum_ab psi_ab(q) P[a][b],   psi = phi times 1 on the diagonal, 2 off it.
// So the state update is P_n += w_n phi(k) and the readout of matrix n is
// psi(q) . P_n: real dot products over d^2 features.
//
// Kernels here run fp32 arithmetic on either input layout:
//  * state build: P over a token range (overwrite or accumulate); one
//    workgroup per (head, group of 4 matrices), a thread per (row a, 16
//    columns), phi formed once per token and entry for the 4 matrices;
//  * merge: fold an incoming state into a causal forward's output over the
//    call's tokens, O <- (O l + num) / (l + den); one workgroup per (head,
//    64-token tile), a thread per (token, group of matrices);
//  * step: one token per head, HBM-bound (the state read and written once);
//    then the division by the denominator.
// With a per-head decay gamma every token first scales the state by gamma:
// the state build weighs token t of T by gamma^(T-1-t) and an accumulated
// state by gamma^T, the merge counts the incoming state gamma^(t+1) at token
// t, and the step scales the state by gamma before adding the token.
#include "cattn_internal.h"

namespace cattn {
namespace {

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ inline uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ inline float2 ld(int layout, const void *re, const void *im, int64_t idx) {
    if (layout == LAYOUT_C64) return reinterpret_cast<const float2 *>(re)[idx];
    return make_float2(bf16_to_f32(reinterpret_cast<const uint16_t *>(re)[idx]),
                       bf16_to_f32(reinterpret_cast<const uint16_t *>(im)[idx]));
}

__device__ inline void st(int layout, void *re, void *im, int64_t idx, float2 x) {
    if (layout == LAYOUT_C64) {
        reinterpret_cast<float2 *>(re)[idx] = x;
    } else {
        reinterpret_cast<uint16_t *>(re)[idx] = f32_to_bf16(x.x);
        reinterpret_cast<uint16_t *>(im)[idx] = f32_to_bf16(x.y);
    }
}

// One real component (0: real, 1: imaginary) of element idx.
__device__ inline void st_part(int layout, void *re, void *im, int64_t idx, int part, float x) {
    if (layout == LAYOUT_C64)
        reinterpret_cast<float *>(re)[2 * idx + part] = x;
    else
        reinterpret_cast<uint16_t *>(part ? im : re)[idx] = f32_to_bf16(x);
}

// phi_ab(u) from u_a and u_b
__device__ inline float phi(float2 ua, float2 ub, bool upper) {
    return upper ? ua.x * ub.x + ua.y * ub.y      // Re(u_a conj u_b)
                 : ub.y * ua.x - ub.x * ua.y;     // Im(u_b conj u_a)
}

// weight of state matrix n for a token's value row: Re V, Im V, or 1 for Z
__device__ inline float col_weight(int layout, const void *v_re, const void *v_im, int64_t row, int n, int d) {
    if (n == 2 * d) return 1.f;
    const float2 v = ld(layout, v_re, v_im, row + (n < d ? n : n - d));
    return n < d ? v.x : v.y;
}

constexpr int NT = 256;
constexpr int TT = 64;   // tokens per LDS tile

__device__ inline float *state_matrix(const LinearProblem &p, int64_t bh, int n) {
    const int64_t dd = (int64_t)p.d * p.d;
    return p.S + (bh * (2 * p.d + 1) + n) * dd;
}

// ---------------------------------------------------------------------------- state build
// Workgroup (head, matrices n0 .. n0 + G - 1).  Thread owns row a = tid / 4
// and columns b = 16 (tid % 4) + j, j < 16; whether an entry is above the
// diagonal is fixed per thread and column, so the pair (Re k, Im k) or the
// rotated pair (Im k, -Re k) is picked by address, once.
constexpr int SG_G = 4;

__global__ __launch_bounds__(NT) void born_state_kernel(LinearProblem p) {
    __shared__ float2 Kp[TT][CATTN_LIN_MAXD + 1];   // (Re k, Im k)
    __shared__ float2 Ka[TT][CATTN_LIN_MAXD + 1];   // (Im k, -Re k): phi below the diagonal
    __shared__ float wv[TT][SG_G];
    const int tid = threadIdx.x;
    const int d = p.d;
    const int ngroups = (2 * d + 1 + SG_G - 1) / SG_G;
    const int64_t bh = blockIdx.x / ngroups;
    const int n0 = (int)(blockIdx.x % ngroups) * SG_G;
    const int a = tid / 4, b0 = 16 * (tid % 4);
    const bool active = a < d && b0 < d;
    const int64_t base = bh * p.T * d;
    const float lg2 = p.decay.on ? p.decay.lg2[bh % p.H] : 0.f;
    const float carry = p.decay.on ? decay_pow(lg2, p.T) : 1.f;   // gamma^T on the old state

    float acc[SG_G][16];
#pragma unroll
    for (int g = 0; g < SG_G; ++g)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int n = n0 + g, b = b0 + j;
            acc[g][j] = (p.accumulate && active && n <= 2 * d && b < d) ? carry * state_matrix(p, bh, n)[a * d + b]
                                                                        : 0.f;
        }
    // which table each column reads: the pair on or above the diagonal, the rotated pair below
    const float2(*tab[16]);
#pragma unroll
    for (int j = 0; j < 16; ++j) tab[j] = a <= b0 + j ? &Kp[0][0] : &Ka[0][0];

    for (int t0 = 0; t0 < p.T; t0 += TT) {
        __syncthreads();
        for (int i = tid; i < TT * d; i += NT) {
            const int r = i / d, m = i % d;
            float2 kx = make_float2(0.f, 0.f);
            if (t0 + r < p.T) kx = ld(p.layout, p.k_re, p.k_im, base + (int64_t)(t0 + r) * d + m);
            Kp[r][m] = kx;
            Ka[r][m] = make_float2(kx.y, -kx.x);
        }
        for (int i = tid; i < TT * SG_G; i += NT) {
            const int r = i / SG_G, g = i % SG_G;
            const int n = n0 + g;
            float w = (t0 + r < p.T && n <= 2 * d)
                          ? col_weight(p.layout, p.v_re, p.v_im, base + (int64_t)(t0 + r) * d, n, d) : 0.f;
            if (p.decay.on && t0 + r < p.T) w *= decay_pow(lg2, p.T - 1 - (t0 + r));
            wv[r][g] = w;
        }
        __syncthreads();
        if (!active) continue;
        const int nr = min(TT, p.T - t0);
        for (int r = 0; r < nr; ++r) {
            const float2 ka = Kp[r][a];
            float w[SG_G];
#pragma unroll
            for (int g = 0; g < SG_G; ++g) w[g] = wv[r][g];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int b = min(b0 + j, d - 1);   // columns past d compute a discarded value
                const float2 u = tab[j][r * (CATTN_LIN_MAXD + 1) + b];
                const float f = ka.x * u.x + ka.y * u.y;
#pragma unroll
                for (int g = 0; g < SG_G; ++g) acc[g][j] += w[g] * f;
            }
        }
    }
    if (!active) return;
#pragma unroll
    for (int g = 0; g < SG_G; ++g) {
        const int n = n0 + g;
        if (n > 2 * d) break;
        float *X = state_matrix(p, bh, n);
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (b0 + j < d) X[a * d + b0 + j] = acc[g][j];
    }
}

// ---------------------------------------------------------------------------- merge
// Workgroup (head, 64-token tile); thread (token t = tid % 64, group g = tid /
// 64) accumulates psi(q_t) . P_n for its group's matrices n = g NG + i.  Row a
// of every matrix is staged per step as Ps[b][n]; all lanes of a wave share
// g, so the state reads are broadcasts.
constexpr int MG_NG = 36;                  // matrices per group (4 groups cover 2d + 1 <= 129)
constexpr int MG_LD = 4 * MG_NG;           // Ps row length

__global__ __launch_bounds__(NT) void born_merge_kernel(LinearProblem p) {
    // the per-token results reuse the staging space once the feature loop is done
    constexpr int QS_BYTES = TT * (CATTN_LIN_MAXD + 1) * 8, PS_BYTES = CATTN_LIN_MAXD * MG_LD * 4;
    constexpr int RES_BYTES = TT * (MG_LD + 1) * 4;
    __shared__ __align__(16) char smem[(QS_BYTES + PS_BYTES) > RES_BYTES ? QS_BYTES + PS_BYTES : RES_BYTES];
    auto Qs = reinterpret_cast<float2(*)[CATTN_LIN_MAXD + 1]>(smem);
    auto Ps = reinterpret_cast<float(*)[MG_LD]>(smem + QS_BYTES);
    auto res = reinterpret_cast<float(*)[MG_LD + 1]>(smem);
    const int tid = threadIdx.x;
    const int t = tid % TT, g = tid / TT;
    const int d = p.d, nm = 2 * d + 1;
    const int nt = (p.T + TT - 1) / TT;
    const int64_t bh = blockIdx.x / nt;
    const int t0 = (int)(blockIdx.x % nt) * TT;
    const int64_t base = bh * p.T * d;
    const float *S = p.S + bh * (int64_t)nm * d * d;

    for (int i = tid; i < TT * d; i += NT) {
        const int r = i / d, m = i % d;
        float2 qx = make_float2(0.f, 0.f);
        if (t0 + r < p.T) qx = ld(p.layout, p.q_re, p.q_im, base + (int64_t)(t0 + r) * d + m);
        Qs[r][m] = qx;
    }
    float acc[MG_NG];
#pragma unroll
    for (int i = 0; i < MG_NG; ++i) acc[i] = 0.f;

    for (int a = 0; a < d; ++a) {
        __syncthreads();   // Qs ready; the previous row consumed
        for (int i = tid; i < MG_LD * d; i += NT) {
            const int n = i / d, b = i % d;
            Ps[b][n] = n < nm ? S[((int64_t)n * d + a) * d + b] : 0.f;
        }
        __syncthreads();
        const float2 qa = Qs[t][a];
        for (int b = 0; b < d; ++b) {
            const float2 qb = Qs[t][b];
            const float f = (a == b ? 1.f : 2.f) * phi(qa, qb, a <= b);
            const float4 *row = reinterpret_cast<const float4 *>(&Ps[b][g * MG_NG]);
#pragma unroll
            for (int i = 0; i < MG_NG / 4; ++i) {
                const float4 s4 = row[i];
                acc[4 * i + 0] += f * s4.x;
                acc[4 * i + 1] += f * s4.y;
                acc[4 * i + 2] += f * s4.z;
                acc[4 * i + 3] += f * s4.w;
            }
        }
    }
    __syncthreads();   // every thread done with Qs and Ps
#pragma unroll
    for (int i = 0; i < MG_NG; ++i) res[t][g * MG_NG + i] = acc[i];
    __syncthreads();
    // with decay the incoming state counts gamma^(t+1) at token t
    const float lg2 = p.decay.on ? p.decay.lg2[bh % p.H] : 0.f;
    auto carry = [&](int tq) { return p.decay.on ? decay_pow(lg2, tq + 1) : 1.f; };
    // O <- (O l + num) / (l + den); l from the forward (eps included)
    for (int i = tid; i < TT * d; i += NT) {
        const int r = i / d, c = i % d;
        const int tq = t0 + r;
        if (tq >= p.T) continue;
        const float g = carry(tq);
        const float l = p.row_den[bh * p.T + tq];
        const float D = l + g * res[r][2 * d];
        const float inv = D != 0.f ? 1.f / D : 0.f;
        const int64_t idx = base + (int64_t)tq * d + c;
        const float2 o = ld(p.layout, p.o_re, p.o_im, idx);
        st(p.layout, p.o_re, p.o_im, idx,
           make_float2((o.x * l + g * res[r][c]) * inv, (o.y * l + g * res[r][d + c]) * inv));
    }
    __syncthreads();
    for (int r = tid; r < TT; r += NT) {
        const int tq = t0 + r;
        if (tq < p.T) p.row_den[bh * p.T + tq] += carry(tq) * res[r][2 * d];
    }
}

// ---------------------------------------------------------------------------- step
// One token per head.  Workgroup (head, SGN consecutive matrices); thread
// owns PER groups of VW consecutive entries of a matrix (the same entries in
// every matrix), forms phi(k) and psi(q) for them once, then per matrix:
// P += w phi(k), r += psi(q) . P.  The numerators (real part from matrix c,
// imaginary part from matrix d + c) go to O and the denominator to row_den;
// a second kernel divides.
template <int VW, int PER, int SGN>
__global__ __launch_bounds__(NT) void born_step_kernel(LinearProblem p) {
    __shared__ float2 q[CATTN_LIN_MAXD], k[CATTN_LIN_MAXD];
    __shared__ float wn[SGN];
    __shared__ float red[SGN][NT / 64];
    const int tid = threadIdx.x;
    const int d = p.d, nm = 2 * d + 1, dd = d * d;
    const int ng = (nm + SGN - 1) / SGN;
    const int64_t bh = blockIdx.x / ng;
    const int n0 = (int)(blockIdx.x % ng) * SGN;
    const int64_t row = bh * d;   // the single token of this head
    for (int m = tid; m < d; m += NT) {
        q[m] = ld(p.layout, p.q_re, p.q_im, row + m);
        k[m] = ld(p.layout, p.k_re, p.k_im, row + m);
    }
    if (tid < SGN) wn[tid] = n0 + tid < nm ? col_weight(p.layout, p.v_re, p.v_im, row, n0 + tid, d) : 0.f;
    __syncthreads();

    float fk[PER][VW], fq[PER][VW];
#pragma unroll
    for (int i = 0; i < PER; ++i)
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            const int x = (tid + i * NT) * VW + e;
            fk[i][e] = fq[i][e] = 0.f;
            if (x < dd) {
                const int a = x / d, b = x % d;
                fk[i][e] = phi(k[a], k[b], a <= b);
                fq[i][e] = (a == b ? 1.f : 2.f) * phi(q[a], q[b], a <= b);
            }
        }
    const float gam = p.decay.on ? decay_pow(p.decay.lg2[bh % p.H], 1) : 1.f;   // the state's scale per token
    float r[SGN];
#pragma unroll
    for (int s = 0; s < SGN; ++s) {
        r[s] = 0.f;
        const int n = n0 + s;
        if (n >= nm) continue;   // uniform: the last group may be short
        const float w = wn[s];
        float *X = state_matrix(p, bh, n);
        float e[PER][VW];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = tid + i * NT;
            if (v * VW >= dd) continue;
            if (VW == 4) {
                const float4 x4 = reinterpret_cast<const float4 *>(X)[v];
                e[i][0] = x4.x; e[i][1] = x4.y; e[i][2] = x4.z; e[i][3] = x4.w;
            } else {
                e[i][0] = X[v];
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = tid + i * NT;
            if (v * VW >= dd) continue;
#pragma unroll
            for (int c = 0; c < VW; ++c) {
                e[i][c] = fmaf(w, fk[i][c], gam * e[i][c]);
                r[s] += fq[i][c] * e[i][c];
            }
            if (VW == 4)
                reinterpret_cast<float4 *>(X)[v] = make_float4(e[i][0], e[i][1], e[i][2], e[i][3]);
            else
                X[v] = e[i][0];
        }
    }
#pragma unroll
    for (int s = 0; s < SGN; ++s) {
        for (int o = 32; o > 0; o >>= 1) r[s] += __shfl_xor(r[s], o);
        if ((tid & 63) == 0) red[s][tid >> 6] = r[s];
    }
    __syncthreads();
    if (tid < SGN && n0 + tid < nm) {
        float tot = 0.f;
        for (int i = 0; i < NT / 64; ++i) tot += red[tid][i];
        const int n = n0 + tid;
        if (n < 2 * d)
            st_part(p.layout, p.o_re, p.o_im, row + (n < d ? n : n - d), n < d ? 0 : 1, tot);   // numerator for now
        else
            p.row_den[bh] = tot + p.eps;
    }
}

__global__ __launch_bounds__(NT) void born_step_divide_kernel(LinearProblem p) {
    const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (i >= (int64_t)p.BH * p.d) return;
    const int64_t bh = i / p.d;
    const float D = p.row_den[bh];
    const float inv = D != 0.f ? 1.f / D : 0.f;
    const float2 o = ld(p.layout, p.o_re, p.o_im, i);
    // the numerator was rounded to the layout once already; for bf16 that is
    // a second rounding of the output
    st(p.layout, p.o_re, p.o_im, i, make_float2(o.x * inv, o.y * inv));
}

template <int VW, int PER, int SGN>
hipError_t launch_step_cfg(const LinearProblem &p) {
    const int64_t blocks = (int64_t)p.BH * ((2 * p.d + 1 + SGN - 1) / SGN);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((born_step_kernel<VW, PER, SGN>), dim3((unsigned)blocks), dim3(NT), 0, p.stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_born_state(const LinearProblem &p) {
    const int64_t blocks = (int64_t)p.BH * ((2 * p.d + 1 + SG_G - 1) / SG_G);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(born_state_kernel, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p);
    return hipGetLastError();
}

hipError_t launch_born_merge(const LinearProblem &p) {
    const int64_t blocks = (int64_t)p.BH * ((p.T + TT - 1) / TT);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(born_merge_kernel, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p);
    return hipGetLastError();
}

hipError_t launch_born_step(const LinearProblem &p) {
    hipError_t e;
    // float4 entries when rows hold a multiple of 4; matrices per workgroup
    // sized so that a workgroup moves tens of KiB
    if (p.d == 64)
        e = launch_step_cfg<4, 4, 3>(p);          // 43 groups of 3 matrices (16 KiB each)
    else if (p.d % 4 == 0 && p.d > 32)
        e = launch_step_cfg<4, 4, 5>(p);
    else if (p.d % 4 == 0)
        e = launch_step_cfg<4, 1, 11>(p);         // d <= 32: d^2 / 4 <= 256 float4
    else
        e = launch_step_cfg<1, 16, 5>(p);         // any d <= 64: d^2 <= 4096 = 16 x 256
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)p.BH * p.d;
    hipLaunchKernelGGL(born_step_divide_kernel, dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, p.stream, p);
    return hipGetLastError();
}

}  // namespace cattn
