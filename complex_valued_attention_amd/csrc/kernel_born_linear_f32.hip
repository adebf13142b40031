// Carried-state Born attention on gfx950 fp32 matrix cores
// (v_mfma_f32_32x32x2_f32), interleaved complex64 or bf16 planes (widened to
// fp32 on load, rounded back on store), head widths 16, 32, 64
// ("Show HN: CNET", BornAttention's linear mode: the key lifted to its outer
// product, a running state; "The Quantum Shortcut", section 2: the Born rule
// q^H rho q as a linear functional of rho = k k^H).
//
// The packed state of a head is S[n][f], n < 2d + 1 matrices (Re V channels,
// Im V channels, Z), f = a d + b over the d^2 real features
//     phi_ab(u) = Re(u_a conj u_b) (a <= b),  Im(u_b conj u_a) (a > b),
// and a query reads q^H X_n q = sum_f psi_f(q) S[n][f] with psi = phi times 1
// on the diagonal and 2 off it.  Both directions are real products with fp32
// accumulation:
//  * state build: S[n][f] (+)= sum_j W[j][n] phi_f(k_j), W[j] = (Re V[j], Im V[j], 1):
//    MFMA rows are the matrices (tiles of 32; the last tile holds Z, whose
//    operand is the constant 1 in its first row), columns are features, the
//    reduction runs over tokens two at a time;
//  * readout (merge): R[t][n] = sum_f psi_f(q_t) S[n][f]: rows are the
//    matrices, columns are tokens, the reduction runs over features.
// A lane forms its feature of one token with two multiply-adds from the
// (Re, Im) pairs of u_a and u_b: phi = x . u_b with x = u_a on and above the
// diagonal, x = (-Im u_a, Re u_a) below it.
#include "cattn_internal.h"

namespace cattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NW = 4;
constexpr int NT = 64 * NW;

template <int D>
struct LCfg {
    static constexpr int NM = 2 * D + 1;        // packed matrices per head
    static constexpr int NTI = 2 * D / 32 + 1;  // 32-row tiles: the value channels, then Z (+ zero rows)
    static constexpr int F = D * D;             // features
};

__device__ inline void mfma(float a, float b, f32x16 &c) { c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0); }

// workgroups of one head on one XCD when the grid is a multiple of 8
__device__ inline int xcd_order(int x, int nblk) { return (nblk % 8 == 0) ? (x % 8) * (nblk / 8) + x / 8 : x; }

// ---------------------------------------------------------------------------- state build
// Workgroup: 4 waves x FT feature tiles of 32 (features f0 .. f0 + 32 NW FT - 1 of one head).
constexpr int SFT = 2;          // feature tiles per wave
constexpr int STS = 32;         // tokens per LDS stage

template <int D>
struct StateSmem {
    float2 Kp[STS][D];          // (Re k, Im k)
    float2 Kr[STS][D];          // (-Im k, Re k)
    float W[STS][2 * D];        // Re V channels, then Im V channels
};


// One complex element i (counted from the start of the tensor): interleaved
// complex64, or two bf16 planes widened on load and rounded (nearest even) on
// store; the arithmetic is fp32 either way.
template <int LAY>
__device__ inline float2 ld2(const void *re, const void *im, int64_t i) {
    if constexpr (LAY == LAYOUT_C64) {
        return reinterpret_cast<const float2 *>(re)[i];
    } else {
        return make_float2(__uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(re)[i] << 16),
                           __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(im)[i] << 16));
    }
}

template <int LAY>
__device__ inline void st2(void *re, void *im, int64_t i, float2 v) {
    if constexpr (LAY == LAYOUT_C64) {
        reinterpret_cast<float2 *>(re)[i] = v;
    } else {
        reinterpret_cast<uint16_t *>(re)[i] = __builtin_bit_cast(uint16_t, (__bf16)v.x);
        reinterpret_cast<uint16_t *>(im)[i] = __builtin_bit_cast(uint16_t, (__bf16)v.y);
    }
}

// DECAY: token t of T weighs gamma^(T-1-t) (on the feature operand, so the
// value rows and the constant row of Z alike) and an accumulated state
// gamma^T.
template <int D, int LAY, bool DECAY>
__global__ __launch_bounds__(NT) void born_state_f32_kernel(LinearProblem p, int groups) {
    using C = LCfg<D>;
    __shared__ __align__(16) StateSmem<D> sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
    const int T = p.T;
    const int lin = xcd_order(blockIdx.x, gridDim.x);
    const int64_t bh = lin / groups;
    const int f0 = (lin % groups) * (32 * NW * SFT) + wave * 32 * SFT;   // this wave's first feature
    const int64_t base = bh * (int64_t)T * D;

    // this lane's features (a, b) and which pair table its first operand reads
    int fa[SFT], fb[SFT];
    bool upper[SFT];
#pragma unroll
    for (int ft = 0; ft < SFT; ++ft) {
        const int f = f0 + 32 * ft + l32;
        fa[ft] = f / D;
        fb[ft] = f % D;
        upper[ft] = fa[ft] <= fb[ft];
    }

    f32x16 acc[C::NTI][SFT];
#pragma unroll
    for (int ti = 0; ti < C::NTI; ++ti)
#pragma unroll
        for (int ft = 0; ft < SFT; ++ft) acc[ti][ft] = f32x16{};
    const float zrow = l32 == 0 ? 1.f : 0.f;   // Z tile: the constant 1 in its first row
    const float lg2 = DECAY ? p.decay.lg2[bh % p.H] : 0.f;

    // a stage's (k, v) pairs go global -> registers one stage ahead, then
    // registers -> LDS once the previous stage is consumed
    constexpr int PK = STS * D / NT;   // pairs per thread
    float2 pk[PK], pv[PK];
    auto load = [&](int t0) {
#pragma unroll
        for (int j = 0; j < PK; ++j) {
            const int i = tid + j * NT;
            const int r = i / D, m = i % D;
            pk[j] = pv[j] = make_float2(0.f, 0.f);
            if (t0 + r < T) {
                pk[j] = ld2<LAY>(p.k_re, p.k_im, base + (int64_t)(t0 + r) * D + m);
                pv[j] = ld2<LAY>(p.v_re, p.v_im, base + (int64_t)(t0 + r) * D + m);
            }
        }
    };
    load(0);
    for (int t0 = 0; t0 < T; t0 += STS) {
        __syncthreads();   // the previous stage is consumed
#pragma unroll
        for (int j = 0; j < PK; ++j) {
            const int i = tid + j * NT;
            const int r = i / D, m = i % D;
            sm.Kp[r][m] = pk[j];
            sm.Kr[r][m] = make_float2(-pk[j].y, pk[j].x);
            sm.W[r][m] = pv[j].x;
            sm.W[r][D + m] = pv[j].y;
        }
        __syncthreads();
        if (t0 + STS < T) load(t0 + STS);
        // tokens past T have zero keys: their features are zero
#pragma unroll 4
        for (int s = 0; s < STS / 2; ++s) {
            const int t = 2 * s + h;   // this lane's token of the step
            float w[C::NTI];
#pragma unroll
            for (int ti = 0; ti < C::NTI - 1; ++ti) w[ti] = sm.W[t][32 * ti + l32];
            w[C::NTI - 1] = zrow;
            // tokens past T have zero features; clamp their exponent
            const float fdec = DECAY ? decay_pow(lg2, max(T - 1 - (t0 + t), 0)) : 1.f;
#pragma unroll
            for (int ft = 0; ft < SFT; ++ft) {
                const float2 x = upper[ft] ? sm.Kp[t][fa[ft]] : sm.Kr[t][fa[ft]];
                const float2 kb = sm.Kp[t][fb[ft]];
                float phi = x.x * kb.x + x.y * kb.y;
                if (DECAY) phi *= fdec;
#pragma unroll
                for (int ti = 0; ti < C::NTI; ++ti) mfma(w[ti], phi, acc[ti][ft]);
            }
        }
    }

    // write S[n][f]: lane (feature column l32, half h) holds rows n = 32 ti + 8 (r/4) + 4 h + r % 4
    float *Sh = p.S + bh * (int64_t)C::NM * C::F;
    const float carry = DECAY ? decay_pow(lg2, T) : 1.f;
#pragma unroll
    for (int ti = 0; ti < C::NTI; ++ti)
#pragma unroll
        for (int ft = 0; ft < SFT; ++ft)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = 32 * ti + 8 * (r >> 2) + 4 * h + (r & 3);
                if (n >= C::NM) continue;
                float *dst = Sh + (int64_t)n * C::F + f0 + 32 * ft + l32;
                *dst = p.accumulate ? carry * *dst + acc[ti][ft][r] : acc[ti][ft][r];
            }
}

// ---------------------------------------------------------------------------- readout (merge)
// Workgroup: 32 TG tokens of one head.  Its 4 waves form TG token groups of
// 32 tokens times FG = 4 / TG feature groups: wave (tg, fg) accumulates every
// matrix for the tokens of tg over the features of fg, and the feature groups
// are summed through LDS at the end.  Few tokens (a short chunk) take TG = 1,
// so the grid still fills the chip; many take TG = 4, which reads the state
// once per 128 tokens.  The state streams through LDS in blocks of 32
// consecutive features (group fg takes columns fg 32/FG .. of each block),
// double buffered, with each block's global loads issued two blocks ahead.
constexpr int MBC = 32;         // staged features per block

template <int D, int TG>
struct MergeSmem {
    static constexpr int FG = NW / TG;
    static constexpr int NM = LCfg<D>::NM;
    static constexpr int PARK = (LCfg<D>::NTI - 1) * 16 + 1;   // accumulator floats a lane hands over
    static constexpr int SB_FLOATS = 2 * NM * (MBC + 1);
    static constexpr int RED_FLOATS = (FG - 1) * TG * PARK * 64;
    float buf[SB_FLOATS > RED_FLOATS ? SB_FLOATS : RED_FLOATS];   // state blocks, then the partial sums
    float2 Qs[32 * TG][D + 1];
};

template <int D, int TG, int LAY>
__global__ __launch_bounds__(NT) void born_merge_f32_kernel(LinearProblem p, int ntile_t) {
    using C = LCfg<D>;
    using M = MergeSmem<D, TG>;
    constexpr int FG = M::FG;
    constexpr int NM = C::NM;
    constexpr int LD = MBC + 1;          // floats per staged matrix row
    constexpr int GB = MBC / FG;         // features per group per block
    extern __shared__ __align__(16) float fsm[];
    M &sm = *reinterpret_cast<M *>(fsm);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
    const int tg = wave % TG, fg = wave / TG;
    const int T = p.T;
    const int lin = xcd_order(blockIdx.x, gridDim.x);
    const int64_t bh = lin / ntile_t;
    const int t0 = (lin % ntile_t) * 32 * TG;
    const int64_t base = bh * (int64_t)T * D;
    const float *S = p.S + bh * (int64_t)NM * C::F;
    auto Sb = [&](int b, int n, int c) -> float & { return sm.buf[(b * NM + n) * LD + c]; };

    for (int i = tid; i < 32 * TG * D; i += NT) {
        const int r = i / D, m = i % D;
        sm.Qs[r][m] = t0 + r < T ? ld2<LAY>(p.q_re, p.q_im, base + (int64_t)(t0 + r) * D + m) : make_float2(0.f, 0.f);
    }

    // block k: features k MBC .. k MBC + 31 of every matrix, one float4 per
    // (matrix, 4 features); a thread holds PF of them between load and store
    constexpr int V4 = NM * (MBC / 4);
    constexpr int PF = (V4 + NT - 1) / NT;
    float4 pre[PF];
    auto load = [&](int k) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int i = tid + j * NT;
            if (i < V4) pre[j] = *reinterpret_cast<const float4 *>(S + (int64_t)(i / (MBC / 4)) * C::F + k * MBC + 4 * (i % (MBC / 4)));
        }
    };
    auto store = [&](int b) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int i = tid + j * NT;
            if (i < V4) {
                const int n = i / (MBC / 4), c = 4 * (i % (MBC / 4));
                Sb(b, n, c) = pre[j].x;
                Sb(b, n, c + 1) = pre[j].y;
                Sb(b, n, c + 2) = pre[j].z;
                Sb(b, n, c + 3) = pre[j].w;
            }
        }
    };
    constexpr int NB = C::F / MBC;
    load(0);
    store(0);
    if (NB > 1) load(1);
    __syncthreads();

    f32x16 acc[C::NTI];
#pragma unroll
    for (int ti = 0; ti < C::NTI; ++ti) acc[ti] = f32x16{};
    // the last tile's rows past 2d hold nothing: those lanes feed zeros
    const int zl = NM - 1 - 32 * (C::NTI - 1);   // lanes 0 .. zl of the last tile are matrices
    const bool last_row = l32 <= zl;
    const int last_n = last_row ? 32 * (C::NTI - 1) + l32 : NM - 1;
    const float2 *qrow = sm.Qs[32 * tg + l32];

    for (int k = 0; k < NB; ++k) {
        const int b = k & 1;
        // block k + 1 into the other buffer (read last before the previous
        // barrier), then block k + 2's loads into the freed registers
        if (k + 1 < NB) store(b ^ 1);
        if (k + 2 < NB) load(k + 2);
#pragma unroll
        for (int s = 0; s < GB / 2; ++s) {
            const int col = fg * GB + 2 * s + h;          // this lane's feature of the step
            const int f = k * MBC + col;
            const int a = f / D, bb = f % D;
            const float2 qa = qrow[a], qb = qrow[bb];
            // psi: Re(q_a conj q_b) above the diagonal, Im(q_b conj q_a) below; x2 off it
            const float up = qa.x * qb.x + qa.y * qb.y;
            const float lo = qb.y * qa.x - qb.x * qa.y;
            const float psi = a == bb ? up : 2.f * (a < bb ? up : lo);
#pragma unroll
            for (int ti = 0; ti < C::NTI - 1; ++ti) mfma(Sb(b, 32 * ti + l32, col), psi, acc[ti]);
            const float zs = Sb(b, last_n, col);
            mfma(last_row ? zs : 0.f, psi, acc[C::NTI - 1]);
        }
        __syncthreads();
    }

    // sum the feature groups: groups 1 .. FG - 1 park their accumulators
    // (the value tiles, and the Z row of the last tile), group 0 adds them
    if constexpr (FG > 1) {
        if (fg > 0) {
            float *dst = sm.buf + ((fg - 1) * TG + tg) * M::PARK * 64 + lane;
#pragma unroll
            for (int ti = 0; ti < C::NTI - 1; ++ti)
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[(ti * 16 + r) * 64] = acc[ti][r];
            dst[(M::PARK - 1) * 64] = acc[C::NTI - 1][0];
        }
        __syncthreads();
        if (fg > 0) return;
#pragma unroll
        for (int g = 1; g < FG; ++g) {
            const float *src = sm.buf + ((g - 1) * TG + tg) * M::PARK * 64 + lane;
#pragma unroll
            for (int ti = 0; ti < C::NTI - 1; ++ti)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[ti][r] += src[(ti * 16 + r) * 64];
            acc[C::NTI - 1][0] += src[(M::PARK - 1) * 64];
        }
    }

    // epilogue: lane (token l32, half h) holds rows n = 32 ti + 8 (r/4) + 4 h + r % 4;
    // channel c's real part is row c, its imaginary part row d + c (same lane), Z is row 2d
    const float den_h0 = acc[C::NTI - 1][0];
    const float den = __shfl(den_h0, l32);
    const int tq = t0 + 32 * tg + l32;
    if (tq >= T) return;
    const int64_t rowi = bh * (int64_t)T + tq;
    const float l = p.row_den[rowi];
    // decay: the incoming state counts gamma^(t+1) at token t
    const float gc = p.decay.on ? decay_pow(p.decay.lg2[bh % p.H], tq + 1) : 1.f;
    const float Dn = l + gc * den;
    const float inv = Dn != 0.f ? 1.f / Dn : 0.f;
    const int64_t orow = base + (int64_t)tq * D;
#pragma unroll
    for (int ti = 0; ti < C::NTI - 1; ++ti)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = 32 * ti + 8 * (r >> 2) + 4 * h + (r & 3);
            if (c >= D) continue;
            // the imaginary row d + c sits D / 32 tiles (D >= 32) or 16 rows (D = 16) further on
            const float im = D >= 32 ? acc[ti + D / 32][r] : acc[ti][r + 8];
            const float2 o = ld2<LAY>(p.o_re, p.o_im, orow + c);
            st2<LAY>(p.o_re, p.o_im, orow + c,
                     make_float2((o.x * l + gc * acc[ti][r]) * inv, (o.y * l + gc * im) * inv));
        }
    if (h == 0) p.row_den[rowi] = Dn;
}

template <int D, int LAY>
hipError_t launch_state_d(const LinearProblem &p) {
    const int groups = LCfg<D>::F / (32 * NW * SFT);
    const int64_t blocks = (int64_t)p.BH * groups;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    auto kern = p.decay.on ? born_state_f32_kernel<D, LAY, true> : born_state_f32_kernel<D, LAY, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p, groups);
    return hipGetLastError();
}

template <int D, int TG, int LAY>
hipError_t launch_merge_tg(const LinearProblem &p) {
    static std::atomic<uint64_t> lds_set{0};
    const int bytes = (int)sizeof(MergeSmem<D, TG>);
    const hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(born_merge_f32_kernel<D, TG, LAY>), bytes, lds_set);
    if (e != hipSuccess) return e;
    const int ntile_t = (p.T + 32 * TG - 1) / (32 * TG);
    const int64_t blocks = (int64_t)p.BH * ntile_t;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((born_merge_f32_kernel<D, TG, LAY>), dim3((unsigned)blocks), dim3(NT), bytes, p.stream, p, ntile_t);
    return hipGetLastError();
}

// 128-token workgroups once they alone give two per compute unit, else 32
template <int D, int LAY>
hipError_t launch_merge_l(const LinearProblem &p) {
    const int64_t wide = (int64_t)p.BH * ((p.T + 127) / 128);
    return wide >= 512 ? launch_merge_tg<D, 4, LAY>(p) : launch_merge_tg<D, 1, LAY>(p);
}

template <int D>
hipError_t launch_merge_d(const LinearProblem &p) {
    return p.layout == LAYOUT_C64 ? launch_merge_l<D, LAYOUT_C64>(p) : launch_merge_l<D, LAYOUT_BF16>(p);
}

template <int D>
hipError_t launch_state_l(const LinearProblem &p) {
    return p.layout == LAYOUT_C64 ? launch_state_d<D, LAYOUT_C64>(p) : launch_state_d<D, LAYOUT_BF16>(p);
}

}  // namespace

// complex64 at widths 16/32/64, and bf16 planes at 16/32 (bf16 at 64 has its
// own bf16 matrix-core kernels, tried first)
bool supports_born_linear_f32(const LinearProblem &p) {
    return p.d == 16 || p.d == 32 || p.d == 64;
}

hipError_t launch_born_state_f32(const LinearProblem &p) {
    switch (p.d) {
        case 16: return launch_state_l<16>(p);
        case 32: return launch_state_l<32>(p);
        default: return launch_state_l<64>(p);
    }
}

hipError_t launch_born_merge_f32(const LinearProblem &p) {
    switch (p.d) {
        case 16: return launch_merge_d<16>(p);
        case 32: return launch_merge_d<32>(p);
        default: return launch_merge_d<64>(p);
    }
}

}  // namespace cattn
