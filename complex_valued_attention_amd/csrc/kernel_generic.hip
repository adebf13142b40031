// Generic complex-valued attention forward: any head width 1..128, both
// operators, both layouts, fp32 vector arithmetic.
//
// This is the plain tiled kernel that covers every shape the specialised
// matrix-core kernels do not (odd head widths, bf16 PCT).  One workgroup owns
// BQ query rows of one (batch, head); key/value tiles of BK rows are staged
// in LDS as fp32 (re, im) pairs, the BQ x BK weights are formed in LDS, and
// each thread accumulates a few output components in registers.
//
// Born options: the per-head decay multiplies each causal weight by
// gamma_h^(k - j); a rotary Q is rotated as it is staged (the arithmetic of
// the rotary pass, rounded to bf16 for bf16 planes as that pass would store
// it).
#include "cattn_internal.h"
#include "rotary_math.h"

namespace cattn {
namespace {

__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ inline uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // keep NaN a NaN
    u += 0x7fffu + ((u >> 16) & 1u);                                             // round to nearest even
    return (uint16_t)(u >> 16);
}

__device__ inline float2 load_c(int layout, const void *re, const void *im, int64_t idx) {
    if (layout == LAYOUT_C64) return reinterpret_cast<const float2 *>(re)[idx];
    return make_float2(bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(re)[idx]),
                       bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(im)[idx]));
}

__device__ inline void store_c(int layout, void *re, void *im, int64_t idx, float2 x) {
    if (layout == LAYOUT_C64) {
        reinterpret_cast<float2 *>(re)[idx] = x;
    } else {
        reinterpret_cast<uint16_t *>(re)[idx] = f32_to_bf16_bits(x.x);
        reinterpret_cast<uint16_t *>(im)[idx] = f32_to_bf16_bits(x.y);
    }
}

constexpr int NT = 256;

template <int DP>
struct GenericTile {
    static constexpr int BQ = DP == 128 ? 16 : 32;  // query rows per workgroup
    static constexpr int BK = BQ;                   // key rows per LDS tile
};

// DP: head width rounded up to 16/32/64/128; components d..DP-1 are zero.
template <int DP>
__global__ __launch_bounds__(NT) void generic_fwd_kernel(Problem p) {
    constexpr int BQ = GenericTile<DP>::BQ;
    constexpr int BK = GenericTile<DP>::BK;
    constexpr int NG = NT / BQ;               // threads sharing one query row
    constexpr int NC = (DP + NG - 1) / NG;    // output components per thread

    __shared__ float2 Qs[BQ][DP + 1];
    __shared__ float2 Ks[BK][DP + 1];
    __shared__ float2 Vs[BK][DP];
    __shared__ float Ws[BQ][BK + 1];
    __shared__ float rq[BQ], rk[BK], dens[BQ];

    const int tid = threadIdx.x;
    const int d = p.d;
    const int nqb = (p.T + BQ - 1) / BQ;
    const int bh = blockIdx.x / nqb;
    const int q0 = (blockIdx.x % nqb) * BQ;
    // head bases and token strides (elements) of each operand
    const int64_t bq = head_offset(p.sq, bh, p.H), bk = head_offset(p.sk, bh, p.H);
    const int64_t bv = head_offset(p.sv, bh, p.H), bo = head_offset(p.so, bh, p.H);
    const bool pct = op_pct_score(p.op);
    const bool norm = op_row_norm(p.op);

    for (int i = tid; i < BQ * DP; i += NT) {
        const int r = i / DP, m = i % DP;
        float2 x = make_float2(0.f, 0.f);
        if (m < d && q0 + r < p.T) {
            x = load_c(p.layout, p.q_re, p.q_im, bq + (int64_t)(q0 + r) * p.sq.t + m);
            if (p.rot) {
                float c, sn;
                rotary_phase((double)(p.rot_pos0 + q0 + r), rotary_theta(m, p.rot_log_base, d), c, sn);
                rotary_apply(x.x, x.y, c, sn, x.x, x.y);
                if (p.layout == LAYOUT_BF16)
                    x = make_float2(bf16_bits_to_f32(rotary_bf16(x.x)), bf16_bits_to_f32(rotary_bf16(x.y)));
            }
        }
        Qs[r][m] = x;
    }
    __syncthreads();
    if (pct && tid < BQ) {
        float ss = 0.f;
        for (int m = 0; m < DP; ++m) ss += Qs[tid][m].x * Qs[tid][m].x + Qs[tid][m].y * Qs[tid][m].y;
        rq[tid] = ss > 0.f ? sqrtf((float)d) / sqrtf(ss) : 0.f;   // sqrt(d_h) / ||q||, 0 for a zero row
    }

    const int oq = tid % BQ;
    const int og = tid / BQ;
    float2 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = make_float2(0.f, 0.f);
    float den = 0.f;

    const int qlast = min(q0 + BQ, p.T) - 1;
    const int kend = p.causal ? qlast + 1 : p.T;
    for (int k0 = 0; k0 < kend; k0 += BK) {
        __syncthreads();                      // previous tile fully consumed
        for (int i = tid; i < BK * DP; i += NT) {
            const int r = i / DP, m = i % DP;
            float2 kx = make_float2(0.f, 0.f), vx = make_float2(0.f, 0.f);
            if (m < d && k0 + r < p.T) {
                kx = load_c(p.layout, p.k_re, p.k_im, bk + (int64_t)(k0 + r) * p.sk.t + m);
                vx = load_c(p.layout, p.v_re, p.v_im, bv + (int64_t)(k0 + r) * p.sv.t + m);
            }
            Ks[r][m] = kx;
            Vs[r][m] = vx;
        }
        __syncthreads();
        if (pct && tid < BK) {
            float ss = 0.f;
            for (int m = 0; m < DP; ++m) ss += Ks[tid][m].x * Ks[tid][m].x + Ks[tid][m].y * Ks[tid][m].y;
            rk[tid] = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
        }
        __syncthreads();
        for (int i = tid; i < BQ * BK; i += NT) {
            const int r = i / BK, c = i % BK;
            float sr = 0.f, si = 0.f;               // S = sum_m q_m conj(k_m)
            for (int m = 0; m < DP; ++m) {
                const float2 a = Qs[r][m], b = Ks[c][m];
                sr += a.x * b.x + a.y * b.y;
                si += a.y * b.x - a.x * b.y;
            }
            const int qi = q0 + r, kj = k0 + c;
            const bool valid = kj < p.T && (!p.causal || kj <= qi);
            float w;
            if (!pct) {
                w = sr * sr + si * si;
                if (p.decay.on && valid) w *= decay_pow(p.decay.lg2[bh % p.H], qi - kj);
            } else {
                const float x = sr * rq[r] * rk[c];   // sqrt(d_h) Re<qh, kh>, |x| <= sqrt(d_h)
                if (p.op == OP_PCT) {
                    w = 1.f / (1.f + __expf(-(x + p.bias)));
                } else if (p.op == OP_PCT_SOFTMAX) {
                    w = __expf(x);                    // bounded by e^sqrt(d_h): no shift needed
                } else {
                    const float y = fmaxf(x - p.gate_t, 0.f);
                    w = p.gate_r * p.gate_r * y * y;
                }
            }
            Ws[r][c] = valid ? w : 0.f;
        }
        __syncthreads();
        for (int j = 0; j < BK; ++j) {
            const float w = Ws[oq][j];
            den += w;
#pragma unroll
            for (int ci = 0; ci < NC; ++ci) {
                const int c = og + ci * NG;
                if (c < DP) {
                    const float2 vv = Vs[j][c];
                    acc[ci].x += w * vv.x;
                    acc[ci].y += w * vv.y;
                }
            }
        }
    }

    if (og == 0) dens[oq] = den + p.eps;
    __syncthreads();
    const int qi = q0 + oq;
    if (qi >= p.T) return;
    const float D = dens[oq];
    const float inv = (norm && D != 0.f) ? 1.f / D : 0.f;
#pragma unroll
    for (int ci = 0; ci < NC; ++ci) {
        const int c = og + ci * NG;
        if (c < d) {
            float2 o = acc[ci];
            if (norm) o = make_float2(o.x * inv, o.y * inv);
            store_c(p.layout, p.o_re, p.o_im, bo + (int64_t)qi * p.so.t + c, o);
        }
    }
    if (!pct && og == 0 && p.row_den) p.row_den[(int64_t)bh * p.T + qi] = D;
}

template <int DP>
hipError_t launch_dp(const Problem &p) {
    const int nqb = (p.T + GenericTile<DP>::BQ - 1) / GenericTile<DP>::BQ;
    const int64_t blocks = (int64_t)p.BH * nqb;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(generic_fwd_kernel<DP>, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_generic(const Problem &p) {
    if (p.d <= 16) return launch_dp<16>(p);
    if (p.d <= 32) return launch_dp<32>(p);
    if (p.d <= 64) return launch_dp<64>(p);
    return launch_dp<128>(p);
}

}  // namespace cattn
