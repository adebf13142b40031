// Born attention with a carried density state ("Show HN: CNET",
// BornAttention's linear and step modes: each key lifted to its outer
// product, a running state, constant-memory decoding; "The Quantum
// Shortcut", section 2: the Born rule as q^H rho q with rho = k k^H).  Per
// head the state is
//     Z    = sum_j k_j k_j^H            (d x d)
//     M[c] = sum_j V[j, c] k_j k_j^H    (d x d per value channel, M[c][a][b])
// stored as interleaved complex64, and a query reads it as
//     O[c] = q^H M[c] q / (q^H Z q + eps).
// Three kernels, fp32 arithmetic, inputs in either layout:
//  * state build: Z, M over a token range (overwrite or accumulate); one
//    workgroup per (head, matrix), the matrix index d standing for Z;
//  * merge: fold an incoming state into a forward's output over the call's
//    own tokens, O <- (O l + q^H M q) / (l + q^H Z q) with l the forward's row
//    denominators (eps included), one workgroup per (head, 64-token tile);
//  * step: add one token to the state and read it out, HBM-bound; then the
//    division by the denominator.
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

constexpr int NT = 256;
constexpr int TT = 64;   // tokens per LDS tile

// Matrix x of head bh: x == d is Z, else M[x].
__device__ inline float2 *state_matrix(const LinearProblem &p, int64_t bh, int x) {
    const int64_t dd = (int64_t)p.d * p.d;
    return x == p.d ? reinterpret_cast<float2 *>(p.Z) + bh * dd
                    : reinterpret_cast<float2 *>(p.M) + (bh * p.d + x) * dd;
}

// ---------------------------------------------------------------------------- state build
// DP: head width rounded up to a multiple of 16; thread (ta, tb) of a 16 x 16
// grid owns the (DP/16) x (DP/16) block of entries a = ta + 16 i, b = tb + 16 j.
template <int DP>
__global__ __launch_bounds__(NT) void born_state_kernel(LinearProblem p) {
    constexpr int R = DP / 16;
    __shared__ float2 Ks[TT][DP + 1];
    __shared__ float2 wv[TT];   // per token: V[j, x] for M[x], 1 for Z
    const int tid = threadIdx.x;
    const int ta = tid / 16, tb = tid % 16;
    const int64_t bh = blockIdx.x / (p.d + 1);
    const int x = (int)(blockIdx.x % (p.d + 1));
    const int d = p.d;
    const int64_t base = bh * p.T * d;
    float2 *X = state_matrix(p, bh, x);

    float2 acc[R][R];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int a = ta + 16 * i, b = tb + 16 * j;
            acc[i][j] = (p.accumulate && a < d && b < d) ? X[a * d + b] : make_float2(0.f, 0.f);
        }

    for (int t0 = 0; t0 < p.T; t0 += TT) {
        __syncthreads();
        for (int i = tid; i < TT * DP; i += NT) {
            const int r = i / DP, m = i % DP;
            float2 kx = make_float2(0.f, 0.f);
            if (m < d && t0 + r < p.T) kx = ld(p.layout, p.k_re, p.k_im, base + (int64_t)(t0 + r) * d + m);
            Ks[r][m] = kx;
        }
        if (tid < TT) {
            float2 w = make_float2(0.f, 0.f);
            if (t0 + tid < p.T)
                w = x == d ? make_float2(1.f, 0.f) : ld(p.layout, p.v_re, p.v_im, base + (int64_t)(t0 + tid) * d + x);
            wv[tid] = w;
        }
        __syncthreads();
        for (int r = 0; r < TT && t0 + r < p.T; ++r) {
            const float2 wc = wv[r];
            float2 u[R], kb[R];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const float2 ka = Ks[r][ta + 16 * i];
                u[i] = make_float2(wc.x * ka.x - wc.y * ka.y, wc.x * ka.y + wc.y * ka.x);   // w k_a
                kb[i] = Ks[r][tb + 16 * i];
            }
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    // += (w k_a) conj(k_b)
                    acc[i][j].x += u[i].x * kb[j].x + u[i].y * kb[j].y;
                    acc[i][j].y += u[i].y * kb[j].x - u[i].x * kb[j].y;
                }
        }
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int a = ta + 16 * i, b = tb + 16 * j;
            if (a < d && b < d) X[a * d + b] = acc[i][j];
        }
}

// ---------------------------------------------------------------------------- merge
// Thread (token t = tid % 64, quarter g = tid / 64) forms the part of
// q_t^H X q_t over rows a = g, g + 4, ...; the quarters are summed in LDS.
template <int DP>
__global__ __launch_bounds__(NT) void born_merge_kernel(LinearProblem p) {
    __shared__ float2 Qs[TT][DP + 1];
    __shared__ float2 Xs[DP][DP + 1];
    __shared__ float2 part[4][TT];
    __shared__ float2 num[TT][DP + 1];
    __shared__ float den[TT];
    const int tid = threadIdx.x;
    const int t = tid % TT, g = tid / TT;
    const int nt = (p.T + TT - 1) / TT;
    const int64_t bh = blockIdx.x / nt;
    const int t0 = (int)(blockIdx.x % nt) * TT;
    const int d = p.d;
    const int64_t base = bh * p.T * d;

    for (int i = tid; i < TT * DP; i += NT) {
        const int r = i / DP, m = i % DP;
        float2 qx = make_float2(0.f, 0.f);
        if (m < d && t0 + r < p.T) qx = ld(p.layout, p.q_re, p.q_im, base + (int64_t)(t0 + r) * d + m);
        Qs[r][m] = qx;
    }
    for (int x = 0; x <= d; ++x) {
        __syncthreads();   // Qs ready; the previous matrix fully consumed
        const float2 *X = state_matrix(p, bh, x);
        for (int i = tid; i < d * d; i += NT) Xs[i / d][i % d] = X[i];
        __syncthreads();
        float2 s = make_float2(0.f, 0.f);
        for (int a = g; a < d; a += 4) {
            float2 y = make_float2(0.f, 0.f);   // (X q)_a
            for (int b = 0; b < d; ++b) {
                const float2 xa = Xs[a][b], qb = Qs[t][b];
                y.x += xa.x * qb.x - xa.y * qb.y;
                y.y += xa.x * qb.y + xa.y * qb.x;
            }
            const float2 qa = Qs[t][a];   // conj(q_a) y
            s.x += qa.x * y.x + qa.y * y.y;
            s.y += qa.x * y.y - qa.y * y.x;
        }
        part[g][t] = s;
        __syncthreads();
        if (tid < TT) {
            const float2 a0 = part[0][tid], a1 = part[1][tid], a2 = part[2][tid], a3 = part[3][tid];
            const float2 tot = make_float2(a0.x + a1.x + a2.x + a3.x, a0.y + a1.y + a2.y + a3.y);
            if (x < d)
                num[tid][x] = tot;
            else
                den[tid] = tot.x;   // q^H Z q is real
        }
    }
    __syncthreads();
    // O <- (O l + num) / (l + den); l from the forward (eps included)
    for (int i = tid; i < TT * d; i += NT) {
        const int r = i / d, c = i % d;
        const int tq = t0 + r;
        if (tq >= p.T) continue;
        const int64_t row = bh * p.T + tq;
        const float l = p.row_den[row];
        const float D = l + den[r];
        const float2 o = ld(p.layout, p.o_re, p.o_im, base + (int64_t)tq * d + c);
        const float inv = D != 0.f ? 1.f / D : 0.f;
        const float2 nm = num[r][c];
        st(p.layout, p.o_re, p.o_im, base + (int64_t)tq * d + c,
           make_float2((o.x * l + nm.x) * inv, (o.y * l + nm.y) * inv));
    }
    __syncthreads();
    for (int r = tid; r < TT; r += NT) {
        const int tq = t0 + r;
        if (tq < p.T) p.row_den[bh * p.T + tq] += den[r];
    }
}

// ---------------------------------------------------------------------------- step
// One token per head.  Workgroup (head, group of SG matrices): X += w k k^H,
// then q^H X q.  Numerators go to O, the denominator (matrix d) to row_den;
// a second kernel divides.
constexpr int SG = 4;

__global__ __launch_bounds__(NT) void born_step_kernel(LinearProblem p) {
    __shared__ float2 q[CATTN_LIN_MAXD], k[CATTN_LIN_MAXD];
    __shared__ float2 red[NT / 64];
    const int tid = threadIdx.x;
    const int d = p.d;
    const int ngroups = (d + 1 + SG - 1) / SG;
    const int64_t bh = blockIdx.x / ngroups;
    const int x0 = (int)(blockIdx.x % ngroups) * SG;
    const int64_t row = bh * d;   // the single token of this head
    for (int m = tid; m < d; m += NT) {
        q[m] = ld(p.layout, p.q_re, p.q_im, row + m);
        k[m] = ld(p.layout, p.k_re, p.k_im, row + m);
    }
    __syncthreads();
    for (int x = x0; x < x0 + SG && x <= d; ++x) {
        const float2 w = x == d ? make_float2(1.f, 0.f) : ld(p.layout, p.v_re, p.v_im, row + x);
        float2 *X = state_matrix(p, bh, x);
        float2 s = make_float2(0.f, 0.f);
        for (int i = tid; i < d * d; i += NT) {
            const int a = i / d, b = i % d;
            const float2 ka = k[a], kb = k[b];
            const float2 u = make_float2(w.x * ka.x - w.y * ka.y, w.x * ka.y + w.y * ka.x);
            float2 e = X[i];
            e.x += u.x * kb.x + u.y * kb.y;   // += w k_a conj(k_b)
            e.y += u.y * kb.x - u.x * kb.y;
            X[i] = e;
            // conj(q_a) e q_b
            const float2 qa = q[a], qb = q[b];
            const float2 eq = make_float2(e.x * qb.x - e.y * qb.y, e.x * qb.y + e.y * qb.x);
            s.x += qa.x * eq.x + qa.y * eq.y;
            s.y += qa.x * eq.y - qa.y * eq.x;
        }
        for (int o = 32; o > 0; o >>= 1) {
            s.x += __shfl_xor(s.x, o);
            s.y += __shfl_xor(s.y, o);
        }
        if ((tid & 63) == 0) red[tid >> 6] = s;
        __syncthreads();
        if (tid == 0) {
            float2 tot = make_float2(0.f, 0.f);
            for (int i = 0; i < NT / 64; ++i) {
                tot.x += red[i].x;
                tot.y += red[i].y;
            }
            if (x < d)
                st(p.layout, p.o_re, p.o_im, row + x, tot);   // numerator for now
            else
                p.row_den[bh] = tot.x + p.eps;
        }
        __syncthreads();
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
    // a second rounding of the output (documented)
    st(p.layout, p.o_re, p.o_im, i, make_float2(o.x * inv, o.y * inv));
}

template <int DP>
hipError_t launch_state_dp(const LinearProblem &p) {
    const int64_t blocks = (int64_t)p.BH * (p.d + 1);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(born_state_kernel<DP>, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p);
    return hipGetLastError();
}

template <int DP>
hipError_t launch_merge_dp(const LinearProblem &p) {
    const int64_t blocks = (int64_t)p.BH * ((p.T + TT - 1) / TT);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(born_merge_kernel<DP>, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_born_state(const LinearProblem &p) {
    if (p.d <= 16) return launch_state_dp<16>(p);
    if (p.d <= 32) return launch_state_dp<32>(p);
    return launch_state_dp<64>(p);
}

hipError_t launch_born_merge(const LinearProblem &p) {
    if (p.d <= 16) return launch_merge_dp<16>(p);
    if (p.d <= 32) return launch_merge_dp<32>(p);
    return launch_merge_dp<64>(p);
}

hipError_t launch_born_step(const LinearProblem &p) {
    const int ngroups = (p.d + 1 + SG - 1) / SG;
    const int64_t blocks = (int64_t)p.BH * ngroups;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(born_step_kernel, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)p.BH * p.d;
    hipLaunchKernelGGL(born_step_divide_kernel, dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, p.stream, p);
    return hipGetLastError();
}

}  // namespace cattn
