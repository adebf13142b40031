// Generic backward of Born and phase-coherent attention: any head width
// 1..128, both layouts, fp32 vector arithmetic.
//
// Gradients are dL/d(conj z) for a real loss L given G = dL/d(conj O)
// ("CNet ...", section 3, the Wirtinger accumulation rule (2)); the map is
// linear in G, so real-pair gradients in give real-pair gradients out.
//
// Born ("CNet ...", section 11.2, "Closing it: Born-rule attention"), with
// S = Q K^H, w = |S|^2, l the forward's row denominators, delta = Re(G^H O)
// per row and D = (Re(G^H V) - delta) / l on the causal support:
//     dV = (w / l)^T G,   dQ = (2 D o S) K,   dK = (2 D o S)^H Q.
// Under a per-head decay every w and D on the causal support carries the
// factor gamma^(k - j) of the forward's weight.
// PCT ("Complex-valued Phase-Coherent Transformers", section 1 and Appendix
// D.2), with qh, kh the unit-normalised rows, s = sqrt(d_h) Re(qh kh^H),
// w = sigmoid(s + b), ds = Re(G^H V) w (1 - w):
//     dV = w^T G,  dq = P_q(sqrt(d_h) ds kh) / ||q||,  dk = P_k(sqrt(d_h) ds^T qh) / ||k||
// where P_x removes the component along the unit vector x, and the per-row
// bias gradient is sum_j ds.
//
// Two kernels, each recomputing the scores: one workgroup of the first owns a
// tile of keys and streams the query tiles that see them (dK, dV); one
// workgroup of the second owns a tile of queries and streams their keys (dQ,
// and the bias gradient).  Nothing is written twice, so there are no atomics
// and the result is deterministic.  delta comes from O and G as each query
// tile is loaded, so no workspace is needed.
#include "cattn_internal.h"

namespace cattn {
namespace {

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ inline uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // keep NaN a NaN
    u += 0x7fffu + ((u >> 16) & 1u);                                             // round to nearest even
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

template <int DP>
struct BwdTile {
    static constexpr int B = DP == 128 ? 16 : 32;   // query rows and key rows per tile
    static constexpr int NG = NT / B;               // threads per row (8 or 16)
    static constexpr int NC = DP / NG;              // components per thread in the accumulation
    static constexpr int PPT = B * B / NT;          // (query, key) pairs per thread
};

// Reduction over the NG consecutive lanes that share a row.
template <int NG>
__device__ inline float row_sum(float x) {
#pragma unroll
    for (int o = 1; o < NG; o <<= 1) x += __shfl_xor(x, o);
    return x;
}

// Shared per-tile state.  Rows (queries or keys) beyond T are zero.
template <int DP>
struct BwdSmem {
    static constexpr int B = BwdTile<DP>::B;
    float2 Qs[B][DP + 1];   // query tile (raw q)
    float2 Gs[B][DP + 1];   // incoming gradient rows
    float2 Ks[B][DP + 1];   // key tile (raw k)
    float2 Vs[B][DP + 1];   // value tile
    float qa[B], qb[B];     // per query: Born 1/l, delta; PCT sqrt(d)/||q||, 1/||q||
    float ka[B];            // per key: PCT 1/||k||
    float Ws[B][B + 1];     // [query][key]: Born w/l, PCT w
    float2 Ps[B][B + 1];    // [query][key]: Born 2 D S, PCT (ds, 0)
};

// Loads rows r0 .. r0+B-1 of x (zero beyond T or d) into dst[B][DP+1]; the
// NG threads of row i also return sum |x|^2 over the row in `ss` (for PCT norms).
template <int DP>
__device__ inline void load_rows(const BwdProblem &p, const void *re, const void *im, int64_t base, int r0,
                                 float2 (*dst)[DP + 1], float &ss) {
    constexpr int B = BwdTile<DP>::B, NG = BwdTile<DP>::NG;
    const int tid = threadIdx.x;
    const int r = tid / NG, c0 = tid % NG;
    float acc = 0.f;
#pragma unroll
    for (int m = c0; m < DP; m += NG) {
        float2 x = make_float2(0.f, 0.f);
        if (m < p.d && r0 + r < p.T) x = ld(p.layout, re, im, base + (int64_t)(r0 + r) * p.d + m);
        dst[r][m] = x;
        acc += x.x * x.x + x.y * x.y;
    }
    ss = row_sum<NG>(acc);
    (void)B;
}

// Per query tile: loads Q and G, and forms the per-query scalars.
template <int DP>
__device__ inline void load_query_tile(const BwdProblem &p, BwdSmem<DP> &s, int64_t base, int q0) {
    constexpr int NG = BwdTile<DP>::NG;
    const int tid = threadIdx.x;
    const int r = tid / NG, c0 = tid % NG;
    float ssq, ssg;
    load_rows<DP>(p, p.q_re, p.q_im, base, q0, s.Qs, ssq);
    load_rows<DP>(p, p.g_re, p.g_im, base, q0, s.Gs, ssg);
    const int q = q0 + r;
    if (p.op == OP_BORN) {
        // delta = Re(G^H O) from the forward output, this thread's components
        float dl = 0.f;
        if (q < p.T) {
            for (int m = c0; m < p.d; m += NG) {
                const float2 o = ld(p.layout, p.o_re, p.o_im, base + (int64_t)q * p.d + m);
                const float2 g = s.Gs[r][m];
                dl += g.x * o.x + g.y * o.y;
            }
        }
        dl = row_sum<NG>(dl);
        if (c0 == 0) {
            float inv = 0.f;
            if (q < p.T) {
                const float l = p.row_den[(int64_t)(base / p.d) + q];
                inv = l != 0.f ? 1.f / l : 0.f;   // a zero denominator: O = 0, no gradient
            }
            s.qa[r] = inv;
            s.qb[r] = dl;
        }
    } else if (c0 == 0) {
        const float inv = ssq > 0.f ? 1.f / sqrtf(ssq) : 0.f;
        s.qa[r] = sqrtf((float)p.d) * inv;
        s.qb[r] = inv;
    }
}

// Loads the key/value tile; PCT also forms 1/||k||.
template <int DP>
__device__ inline void load_key_tile(const BwdProblem &p, BwdSmem<DP> &s, int64_t base, int k0) {
    constexpr int NG = BwdTile<DP>::NG;
    const int tid = threadIdx.x;
    float ssk, ssv;
    load_rows<DP>(p, p.k_re, p.k_im, base, k0, s.Ks, ssk);
    load_rows<DP>(p, p.v_re, p.v_im, base, k0, s.Vs, ssv);
    if (p.op == OP_PCT && tid % NG == 0) s.ka[tid / NG] = ssk > 0.f ? 1.f / sqrtf(ssk) : 0.f;
}

// Pair tile: for every (query r, key c) of the current tiles forms Ws and Ps.
// Returns this thread's sum of ds over its pairs (PCT bias gradient; the
// pairs of one thread share a query row).
template <int DP>
__device__ inline float pair_tile(const BwdProblem &p, BwdSmem<DP> &s, int q0, int k0, int bh) {
    constexpr int B = BwdTile<DP>::B, PPT = BwdTile<DP>::PPT;
    constexpr int TPR = B / PPT;   // threads per query row in the pair tile
    const int tid = threadIdx.x;
    const int r = tid / TPR;
    const int cb = tid % TPR;      // keys cb, cb + TPR, ...
    float2 S[PPT];
    float E[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        S[i] = make_float2(0.f, 0.f);
        E[i] = 0.f;
    }
#pragma unroll 4
    for (int m = 0; m < DP; ++m) {
        const float2 q = s.Qs[r][m], g = s.Gs[r][m];
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const float2 k = s.Ks[cb + TPR * i][m], v = s.Vs[cb + TPR * i][m];
            // S += q conj(k);  E += Re(conj(g) v)
            S[i].x += q.x * k.x + q.y * k.y;
            S[i].y += q.y * k.x - q.x * k.y;
            E[i] += g.x * v.x + g.y * v.y;
        }
    }
    const int qi = q0 + r;
    float dsum = 0.f;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int c = cb + TPR * i;
        const int kj = k0 + c;
        const bool live = qi < p.T && kj < p.T && (!p.causal || kj <= qi);
        float a = 0.f;
        float2 pp = make_float2(0.f, 0.f);
        if (live) {
            if (p.op == OP_BORN) {
                // 1 / l, times gamma^(k - j) under the decay: both the weight and D carry it
                float inv = s.qa[r];
                if (p.decay.on) inv *= decay_pow(p.decay.lg2[bh % p.H], qi - kj);
                const float w = S[i].x * S[i].x + S[i].y * S[i].y;
                a = w * inv;
                const float D2 = 2.f * (E[i] - s.qb[r]) * inv;
                pp = make_float2(D2 * S[i].x, D2 * S[i].y);
            } else {
                const float sc = S[i].x * s.qa[r] * s.ka[c];   // sqrt(d) Re<qh, kh>
                const float w = 1.f / (1.f + __expf(-(sc + p.bias)));
                a = w;
                pp.x = E[i] * w * (1.f - w);
                dsum += pp.x;
            }
        }
        s.Ws[r][c] = a;
        s.Ps[r][c] = pp;
    }
    return dsum;
}

template <int DP>
__global__ __launch_bounds__(NT) void bwd_dkdv_kernel(BwdProblem p) {
    constexpr int B = BwdTile<DP>::B, NG = BwdTile<DP>::NG, NC = BwdTile<DP>::NC;
    __shared__ BwdSmem<DP> s;
    const int tid = threadIdx.x;
    const int nkb = (p.T + B - 1) / B;
    const int bh = blockIdx.x / nkb;
    const int k0 = (blockIdx.x % nkb) * B;
    const int64_t base = (int64_t)bh * p.T * p.d;
    const bool pct = p.op == OP_PCT;

    load_key_tile<DP>(p, s, base, k0);

    // accumulation ownership: key row j, components c0 + NG e
    const int j = tid / NG, c0 = tid % NG;
    float2 dk[NC], dv[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) dk[e] = dv[e] = make_float2(0.f, 0.f);

    const int qstart = p.causal ? (k0 / B) * B : 0;
    for (int q0 = qstart; q0 < p.T; q0 += B) {
        __syncthreads();   // previous tile fully consumed
        load_query_tile<DP>(p, s, base, q0);
        __syncthreads();
        pair_tile<DP>(p, s, q0, k0, bh);
        __syncthreads();
#pragma unroll 2
        for (int r = 0; r < B; ++r) {
            const float a = s.Ws[r][j];
            float2 pp = s.Ps[r][j];
            if (pct) pp.x *= s.qa[r];   // sqrt(d) ds / ||q||: multiplies raw q to give sqrt(d) ds qh
#pragma unroll
            for (int e = 0; e < NC; ++e) {
                const int m = c0 + NG * e;
                const float2 g = s.Gs[r][m], q = s.Qs[r][m];
                dv[e].x += a * g.x;
                dv[e].y += a * g.y;
                // dK += conj(P) q  (PCT: P real)
                dk[e].x += pp.x * q.x + pp.y * q.y;
                dk[e].y += pp.x * q.y - pp.y * q.x;
            }
        }
    }

    const int kj = k0 + j;
    if (pct) {
        // dk = (gkh - Re(gkh^H kh) kh) / ||k||, kh = k / ||k||
        const float rk = s.ka[j];
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            const float2 k = s.Ks[j][c0 + NG * e];
            dot += dk[e].x * k.x + dk[e].y * k.y;
        }
        dot = row_sum<NG>(dot) * rk * rk;   // Re(gkh^H kh) / ||k||
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            const float2 k = s.Ks[j][c0 + NG * e];
            dk[e].x = (dk[e].x - dot * k.x) * rk;
            dk[e].y = (dk[e].y - dot * k.y) * rk;
        }
    }
    if (kj < p.T) {
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            const int m = c0 + NG * e;
            if (m < p.d) {
                st(p.layout, p.dk_re, p.dk_im, base + (int64_t)kj * p.d + m, dk[e]);
                st(p.layout, p.dv_re, p.dv_im, base + (int64_t)kj * p.d + m, dv[e]);
            }
        }
    }
}

template <int DP>
__global__ __launch_bounds__(NT) void bwd_dq_kernel(BwdProblem p) {
    constexpr int B = BwdTile<DP>::B, NG = BwdTile<DP>::NG, NC = BwdTile<DP>::NC;
    constexpr int PPT = BwdTile<DP>::PPT, TPR = B / PPT;
    __shared__ BwdSmem<DP> s;
    __shared__ float dbs[B];
    const int tid = threadIdx.x;
    const int nqb = (p.T + B - 1) / B;
    const int bh = blockIdx.x / nqb;
    const int q0 = (blockIdx.x % nqb) * B;
    const int64_t base = (int64_t)bh * p.T * p.d;
    const bool pct = p.op == OP_PCT;

    load_query_tile<DP>(p, s, base, q0);

    const int r = tid / NG, c0 = tid % NG;
    float2 dq[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) dq[e] = make_float2(0.f, 0.f);
    float dsum = 0.f;

    const int kend = p.causal ? min(p.T, q0 + B) : p.T;
    for (int k0 = 0; k0 < kend; k0 += B) {
        __syncthreads();
        load_key_tile<DP>(p, s, base, k0);
        __syncthreads();
        dsum += pair_tile<DP>(p, s, q0, k0, bh);
        __syncthreads();
#pragma unroll 2
        for (int c = 0; c < B; ++c) {
            float2 pp = s.Ps[r][c];
            if (pct) pp.x *= s.ka[c];   // multiplies raw k to give ds kh
#pragma unroll
            for (int e = 0; e < NC; ++e) {
                const float2 k = s.Ks[c][c0 + NG * e];
                // dQ += P k  (PCT: P real)
                dq[e].x += pp.x * k.x - pp.y * k.y;
                dq[e].y += pp.x * k.y + pp.y * k.x;
            }
        }
    }

    const int qi = q0 + r;
    if (pct) {
        // dq = (gqh - Re(gqh^H qh) qh) / ||q||, gqh = sqrt(d) sum ds kh
        const float sq = sqrtf((float)p.d);
        const float rq = s.qb[r];
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            dq[e].x *= sq;
            dq[e].y *= sq;
            const float2 q = s.Qs[r][c0 + NG * e];
            dot += dq[e].x * q.x + dq[e].y * q.y;
        }
        dot = row_sum<NG>(dot) * rq * rq;
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            const float2 q = s.Qs[r][c0 + NG * e];
            dq[e].x = (dq[e].x - dot * q.x) * rq;
            dq[e].y = (dq[e].y - dot * q.y) * rq;
        }
        // per-row bias gradient: the pair-tile threads of one query row are
        // TPR consecutive lanes
        dsum = row_sum<TPR>(dsum);
        if (tid % TPR == 0) dbs[tid / TPR] = dsum;
        __syncthreads();
        if (p.db_rows && c0 == 0 && qi < p.T) p.db_rows[(int64_t)(base / p.d) + qi] = dbs[r];
    }
    if (qi < p.T) {
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            const int m = c0 + NG * e;
            if (m < p.d) st(p.layout, p.dq_re, p.dq_im, base + (int64_t)qi * p.d + m, dq[e]);
        }
    }
}

template <int DP>
hipError_t launch_dp(const BwdProblem &p, bool dkdv, bool dq) {
    constexpr int B = BwdTile<DP>::B;
    const int64_t nt = (p.T + B - 1) / B;
    const int64_t blocks = (int64_t)p.BH * nt;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (dkdv) {
        hipLaunchKernelGGL(bwd_dkdv_kernel<DP>, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (dq) {
        hipLaunchKernelGGL(bwd_dq_kernel<DP>, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_parts(const BwdProblem &p, bool dkdv, bool dq) {
    if (p.d <= 16) return launch_dp<16>(p, dkdv, dq);
    if (p.d <= 32) return launch_dp<32>(p, dkdv, dq);
    if (p.d <= 64) return launch_dp<64>(p, dkdv, dq);
    return launch_dp<128>(p, dkdv, dq);
}

}  // namespace

hipError_t launch_bwd_generic(const BwdProblem &p) { return launch_parts(p, true, true); }
hipError_t launch_bwd_generic_dkdv(const BwdProblem &p) { return launch_parts(p, true, false); }
hipError_t launch_bwd_generic_dq(const BwdProblem &p) { return launch_parts(p, false, true); }

}  // namespace cattn
