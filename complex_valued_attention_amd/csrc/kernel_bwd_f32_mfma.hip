// Backward of Born and phase-coherent attention on interleaved complex64 (or
// bf16 planes, widened to the same fp32 rows on load and rounded back on
// store) with gfx950 fp32 matrix cores (v_mfma_f32_32x32x2_f32), fp32
// throughout; head width 16 (the wider heads run on the 16 x 16 kernels).
//
// Gradients are dL/d(conj z) for a real loss L given G = dL/d(conj O)
// ("CNet ...", section 3, the Wirtinger accumulation rule (2)).  Born ("CNet
// ...", section 11.2), with S = Q K^H, w = |S|^2, l the forward's row
// denominators, delta = Re(G^H O) per query and D = (Re(G V^H) - delta) / l:
//     dV = (w / l)^T G,   dQ = (2 D o S) K,   dK = (2 D o S)^H Q.
// PCT ("Complex-valued Phase-Coherent Transformers", section 1 and Appendix
// D.2), with s = sqrt(d_h) Re<qh, kh>, w = sigmoid(s + b), ds = Re(G V^H) w (1 - w):
//     dV = w^T G,  dq = P_q(sqrt(d_h) sum_j ds kh_j) / ||q||,  dk = P_k(sqrt(d_h) sum_i ds qh_i) / ||k||,
// P_x removing the component along the unit vector x; the bias gradient per
// query row is sum_j ds.
//
// Complex rows are handled as real interleaved rows x' = (Re x0, Im x0, ...),
// as in the forward: Re<q, k> = k' . q', Im<q, k> = k'' . q' with
// k'' = (-Im k0, Re k0, ...), and Re<g, v> = v' . g'.  A complex product
// P k accumulates as K'^T Re P + K''^T Im P, and conj(P) q as
// Q'^T Re P - Q''^T Im P; the partner component of a lane is the neighbouring
// lane (a DPP swap), the sign set by the component's parity.
//
// Two kernels, each recomputing the scores:
//  * dq: a wave owns 32 queries (Q', G' as register operands) and streams
//    32-key stages of K', V' through LDS; scores, E and the weights come out
//    transposed (lane = query, 16 keys), the shape of the weight operand of
//    dQ'^T += K'^T P^T;
//  * dkdv: a wave owns 32 keys (K' in registers, V' parked in the wave's own
//    LDS rows) and streams 32-query stages of Q', G' (and per query 1/l and
//    delta, or 1/||q||) through LDS; lane = key, 16 queries:
//    dV'^T += G'^T W, dK'^T += Q'^T P.
// Nothing is written twice: no atomics, deterministic results.
#include "cattn_internal.h"

namespace cattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int NW = 4;          // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int BM = 32 * NW;    // rows (queries or keys) owned per workgroup
constexpr int BN = 32;         // rows per LDS stage

template <int D>
struct BCfg {
    static constexpr int KD = 2 * D;                 // interleaved real width
    static constexpr int KCH = KD / 8;               // float4 chunks per lane half of a row
    static constexpr int CT = KD / 32;               // 32-row tiles of a gradient's transposed rows
    static constexpr int KROW = KD + 4;              // padded LDS row (floats)
    static constexpr int ROWS = BN * KROW;
    static constexpr int STAGE = 2 * ROWS + 2 * BN;  // two operands + two per-row scalars
    static constexpr int LDS_BYTES = 2 * STAGE * 4;
    static constexpr int VW_FLOATS = NW * 32 * KROW; // dkdv: each wave's V' rows (its own operand, not shared)
    static constexpr int LDS_BYTES_KV = LDS_BYTES + VW_FLOATS * 4;
    static constexpr int LPK = NT / BN;              // staging lanes per row (8)
    static constexpr int CPT = (KD / 4) / LPK;       // float4 chunks per staging lane
};

__device__ inline void mfma(float a, float b, f32x16 &c) { c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0); }

// value held by the neighbouring lane (l ^ 1): the partner component of an interleaved row
__device__ inline float swap_adj(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
}

// hardware reciprocal (1 ulp), not the IEEE division sequence
__device__ inline float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// Workgroup -> (head, owned block).  The blocks of a head go to one XCD when
// BH % 8 == 0 (workgroups are dealt to the 8 XCDs in turn).  `heavy_last`
// orders the owned blocks so that the causal heaviest come first: for the
// query side the last blocks see the most keys, for the key side the first
// blocks see the most queries.
__device__ inline void map_block(int BH, int nblk, bool heavy_last, int &bh, int &blk) {
    const int L = blockIdx.x;
    int j;
    if ((BH & 7) == 0) {
        const int x = L & 7;
        j = L >> 3;
        bh = x + 8 * (j / nblk);
    } else {
        bh = L / nblk;
        j = L;
    }
    blk = heavy_last ? nblk - 1 - (j % nblk) : j % nblk;
}


// A 16-byte chunk (4 floats: complex elements f/2, f/2 + 1) of the interleaved
// real row `row` (counted from the start of the tensor), at float offset f.
// LAYOUT_BF16: the two elements are read from the bf16 planes and widened, or
// rounded to bf16 (nearest even) and written to them.
template <int LAY, int D>
__device__ inline f32x4 load4(const void *re, const void *im, int64_t row, int f) {
    if constexpr (LAY == LAYOUT_C64) {
        return *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(re) + row * (2 * D) + f);
    } else {
        const int64_t el = row * D + f / 2;
        const uint32_t r2 = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(re) + el);
        const uint32_t i2 = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(im) + el);
        return f32x4{__uint_as_float(r2 << 16), __uint_as_float(i2 << 16), __uint_as_float(r2 & 0xffff0000u),
                     __uint_as_float(i2 & 0xffff0000u)};
    }
}

template <int LAY, int D>
__device__ inline void store4(void *re, void *im, int64_t row, int f, f32x4 v) {
    if constexpr (LAY == LAYOUT_C64) {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(re) + row * (2 * D) + f) = v;
    } else {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const int64_t el = row * D + f / 2;
        const f32x2 r = {v[0], v[2]}, i = {v[1], v[3]};
        *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(re) + el) =
            __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
        *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(im) + el) =
            __builtin_bit_cast(uint32_t, __builtin_convertvector(i, bf16x2_t));
    }
}

// ------------------------------------------------------------------------------ dQ (and db)
// DECAY (Born): every weight and D2 carries gamma^(query - key), one
// exponential per weight (the distance clamped at 0 where the mask zeroes it).
template <int D, int OP, int LAY, bool DECAY>
__global__ __launch_bounds__(NT) void bwd_dq_f32_kernel(BwdProblem p, int nrb) {
    using C = BCfg<D>;
    extern __shared__ __align__(16) float fsm[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int T = p.T;
    const bool born = OP == OP_BORN;

    int bh, rb;
    map_block(p.BH, nrb, true, bh, rb);
    const int m0 = rb * BM;
    const int64_t hrow = (int64_t)bh * T;   // this head's first row

    // Q', G' operands: lane (query l32, half h) holds x'[8 j + 4 h .. +3]
    const int qt0 = m0 + 32 * wave;
    const int qrow = qt0 + l32;
    f32x4 qb[C::KCH], gb[C::KCH];
    float dl = 0.f, ss = 0.f;
#pragma unroll
    for (int j = 0; j < C::KCH; ++j) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f}, g = x, o = x;
        if (qrow < T) {
            x = load4<LAY, D>(p.q_re, p.q_im, hrow + qrow, 8 * j + 4 * h);
            g = load4<LAY, D>(p.g_re, p.g_im, hrow + qrow, 8 * j + 4 * h);
            if (born) o = load4<LAY, D>(p.o_re, p.o_im, hrow + qrow, 8 * j + 4 * h);
        }
        qb[j] = x;
        gb[j] = g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dl += g[e] * o[e];   // Re(G^H O), this half's components
            ss += x[e] * x[e];
        }
    }
    dl += __shfl_xor(dl, 32);
    ss += __shfl_xor(ss, 32);
    float inv_l = 0.f;   // Born: 1 / l (0 for a zero denominator: O = 0, no gradient)
    if (born && qrow < T) {
        const float l = p.row_den[(int64_t)bh * T + qrow];
        inv_l = l != 0.f ? 1.f / l : 0.f;
    }
    const float iq = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;   // PCT: 1 / ||q|| (0 for a zero row)
    const float rq = sqrtf((float)D) * iq;

    f32x16 dq[C::CT];
#pragma unroll
    for (int c = 0; c < C::CT; ++c) dq[c] = f32x16{};
    float dsum = 0.f;

    const int kend = p.causal ? min(T, m0 + BM) : T;
    const int nstages = (kend + BN - 1) / BN;
    const int skey = tid / C::LPK;
    const int schunk = (tid % C::LPK) * C::CPT;
    f32x4 kreg[C::CPT], vreg[C::CPT];
    auto load_stage = [&](int k0) {
        const int kr = k0 + skey;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
            if (kr < T) {
                a = load4<LAY, D>(p.k_re, p.k_im, hrow + kr, 4 * (schunk + i));
                b = load4<LAY, D>(p.v_re, p.v_im, hrow + kr, 4 * (schunk + i));
            }
            kreg[i] = a;
            vreg[i] = b;
        }
    };
    auto store_stage = [&](int buf) {
        float *ks = fsm + buf * C::STAGE;
        float *vs = ks + C::ROWS;
        float *rk = vs + C::ROWS;
        float s2 = 0.f;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            *reinterpret_cast<f32x4 *>(ks + skey * C::KROW + 4 * (schunk + i)) = kreg[i];
            *reinterpret_cast<f32x4 *>(vs + skey * C::KROW + 4 * (schunk + i)) = vreg[i];
            s2 += kreg[i][0] * kreg[i][0] + kreg[i][1] * kreg[i][1] + kreg[i][2] * kreg[i][2] + kreg[i][3] * kreg[i][3];
        }
        if (!born) {
#pragma unroll
            for (int o = 1; o < C::LPK; o <<= 1) s2 += __shfl_xor(s2, o);
            if (tid % C::LPK == 0) rk[skey] = s2 > 0.f ? 1.f / sqrtf(s2) : 0.f;
        }
    };
    if (nstages > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();

    const float sgn = (l32 & 1) ? 1.f : -1.f;   // K''[n] = sgn(n) K'[n ^ 1]
    for (int st = 0; st < nstages; ++st) {
        const int k0 = st * BN;
        const int buf = st & 1;
        if (st + 1 < nstages) load_stage(k0 + BN);
        const bool live = k0 < T && (!p.causal || k0 <= qt0);
        if (live) {
            const bool diag = p.causal && k0 == qt0;
            const float *ks = fsm + buf * C::STAGE;
            const float *vs = ks + C::ROWS;
            const float *rk = vs + C::ROWS;
            // S^T, E^T for 32 keys x 32 queries
            f32x16 sr = f32x16{}, si = f32x16{}, ev = f32x16{};
#pragma unroll
            for (int j = 0; j < C::KCH; ++j) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(ks + l32 * C::KROW + 8 * j + 4 * h);
                const f32x4 v = *reinterpret_cast<const f32x4 *>(vs + l32 * C::KROW + 8 * j + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    mfma(a[e], qb[j][e], sr);
                    mfma(v[e], gb[j][e], ev);
                }
                if (born) {
                    const f32x4 b = {-a[1], a[0], -a[3], a[2]};
#pragma unroll
                    for (int e = 0; e < 4; ++e) mfma(b[e], qb[j][e], si);
                }
            }
            // register r of lane half h is key 8 (r/4) + 4 h + r % 4
            float pr[16], pi[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 rkv = {0.f, 0.f, 0.f, 0.f};
                if (!born) rkv = *reinterpret_cast<const f32x4 *>(rk + 8 * g + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    const int key = 8 * g + 4 * h + e;
                    const bool keep = !((diag && key > l32) || k0 + key >= T);
                    if (born) {
                        float d2 = keep ? 2.f * (ev[r] - dl) * inv_l : 0.f;
                        if (DECAY) d2 *= decay_pow(p.decay.lg2[bh % p.H], max(qrow - (k0 + key), 0));
                        pr[r] = d2 * sr[r];
                        pi[r] = d2 * si[r];
                    } else {
                        const float w = sigmoid(sr[r] * rq * rkv[e] + p.bias);
                        const float ds = keep ? ev[r] * w * (1.f - w) : 0.f;
                        dsum += ds;
                        pr[r] = ds * rkv[e];   // ds kh on the raw key row
                        pi[r] = 0.f;
                    }
                }
            }
            // dQ'^T += K'^T Re P^T (+ K''^T Im P^T); instruction r takes key 8 (r/4) + 4 h + r % 4
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
                for (int c = 0; c < C::CT; ++c) {
                    const float a = ks[key * C::KROW + 32 * c + l32];
                    mfma(a, pr[r], dq[c]);
                    if (born) mfma(sgn * swap_adj(a), pi[r], dq[c]);
                }
            }
        }
        if (st + 1 < nstages) store_stage(buf ^ 1);
        __syncthreads();
    }

    // lane (query l32, half h) holds components n = 32 c + 8 (r/4) + 4 h + r % 4 of dQ',
    // the components qb[4 c + r/4][r % 4] of Q'
    if (!born) {
        const float sq = sqrtf((float)D);
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < C::CT; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dq[c][r] *= sq;
                dot += dq[c][r] * qb[4 * c + (r >> 2)][r & 3];
            }
        dot += __shfl_xor(dot, 32);
        dot *= iq * iq;
#pragma unroll
        for (int c = 0; c < C::CT; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) dq[c][r] = (dq[c][r] - dot * qb[4 * c + (r >> 2)][r & 3]) * iq;
        const float db = dsum + __shfl_xor(dsum, 32);
        if (p.db_rows && h == 0 && qrow < T) p.db_rows[(int64_t)bh * T + qrow] = db;
    }
    if (qrow >= T) return;
#pragma unroll
    for (int c = 0; c < C::CT; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            store4<LAY, D>(p.dq_re, p.dq_im, hrow + qrow, 32 * c + 8 * g + 4 * h,
                           f32x4{dq[c][4 * g], dq[c][4 * g + 1], dq[c][4 * g + 2], dq[c][4 * g + 3]});
}

// ------------------------------------------------------------------------------ dK, dV
template <int D, int OP, int LAY, bool DECAY>
__global__ __launch_bounds__(NT) void bwd_dkdv_f32_kernel(BwdProblem p, int nkb) {
    using C = BCfg<D>;
    extern __shared__ __align__(16) float fsm[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int T = p.T;
    const bool born = OP == OP_BORN;

    int bh, kblk;
    map_block(p.BH, nkb, false, bh, kblk);
    const int kb0 = kblk * BM;
    const int64_t hrow = (int64_t)bh * T;   // this head's first row

    // K' operand of this wave's 32 keys in registers (K'' for Im S is formed from it); the
    // V' operand is parked in this wave's LDS rows, each lane reading back what it wrote
    const int kt0 = kb0 + 32 * wave;
    const int krow = kt0 + l32;
    float *vw = fsm + 2 * C::STAGE + wave * 32 * C::KROW + l32 * C::KROW;
    f32x4 kb[C::KCH];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < C::KCH; ++j) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f}, v = x;
        if (krow < T) {
            x = load4<LAY, D>(p.k_re, p.k_im, hrow + krow, 8 * j + 4 * h);
            v = load4<LAY, D>(p.v_re, p.v_im, hrow + krow, 8 * j + 4 * h);
        }
        kb[j] = x;
        *reinterpret_cast<f32x4 *>(vw + 8 * j + 4 * h) = v;
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += x[e] * x[e];
    }
    ss += __shfl_xor(ss, 32);
    const float rk = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;   // PCT: 1 / ||k||
    const float sqd = sqrtf((float)D);

    f32x16 dk[C::CT], dv[C::CT];
#pragma unroll
    for (int c = 0; c < C::CT; ++c) dk[c] = dv[c] = f32x16{};

    // query stages: with the causal mask only queries >= this workgroup's first key
    const int qstart = p.causal ? kb0 : 0;
    const int nstages = qstart < T ? (T - qstart + BN - 1) / BN : 0;
    const int sq = tid / C::LPK;
    const int schunk = (tid % C::LPK) * C::CPT;
    f32x4 qreg[C::CPT], greg[C::CPT], oreg[C::CPT];
    auto load_stage = [&](int q0) {
        const int qr = q0 + sq;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, g = a, o = a;
            if (qr < T) {
                a = load4<LAY, D>(p.q_re, p.q_im, hrow + qr, 4 * (schunk + i));
                g = load4<LAY, D>(p.g_re, p.g_im, hrow + qr, 4 * (schunk + i));
                if (born) o = load4<LAY, D>(p.o_re, p.o_im, hrow + qr, 4 * (schunk + i));
            }
            qreg[i] = a;
            greg[i] = g;
            oreg[i] = o;
        }
    };
    // per query: Born (1 / l, delta); PCT (1 / ||q||, unused)
    auto store_stage = [&](int buf, int q0) {
        float *qs = fsm + buf * C::STAGE;
        float *gs = qs + C::ROWS;
        float *sa = gs + C::ROWS;
        float *sb = sa + BN;
        float x2 = 0.f, gd = 0.f;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            *reinterpret_cast<f32x4 *>(qs + sq * C::KROW + 4 * (schunk + i)) = qreg[i];
            *reinterpret_cast<f32x4 *>(gs + sq * C::KROW + 4 * (schunk + i)) = greg[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x2 += qreg[i][e] * qreg[i][e];
                gd += greg[i][e] * oreg[i][e];
            }
        }
#pragma unroll
        for (int o = 1; o < C::LPK; o <<= 1) {
            x2 += __shfl_xor(x2, o);
            gd += __shfl_xor(gd, o);
        }
        if (tid % C::LPK == 0) {
            const int qr = q0 + sq;
            if (born) {
                float inv = 0.f;
                if (qr < T) {
                    const float l = p.row_den[(int64_t)bh * T + qr];
                    inv = l != 0.f ? 1.f / l : 0.f;
                }
                sa[sq] = inv;
                sb[sq] = gd;
            } else {
                sa[sq] = x2 > 0.f ? 1.f / sqrtf(x2) : 0.f;
                sb[sq] = 0.f;
            }
        }
    };
    if (nstages > 0) {
        load_stage(qstart);
        store_stage(0, qstart);
    }
    __syncthreads();

    const float nsgn = (l32 & 1) ? -1.f : 1.f;   // -Q''[n] = nsgn(n) Q'[n ^ 1]
    for (int st = 0; st < nstages; ++st) {
        const int q0 = qstart + st * BN;
        const int buf = st & 1;
        if (st + 1 < nstages) load_stage(q0 + BN);
        // this wave's keys see queries >= kt0
        const bool live = !p.causal || q0 + BN - 1 >= kt0;
        if (live && kt0 < T) {
            const bool diag = p.causal && q0 == kt0;
            const float *qs = fsm + buf * C::STAGE;
            const float *gs = qs + C::ROWS;
            const float *sa = gs + C::ROWS;
            const float *sb = sa + BN;
            // lane = key l32, registers = 16 queries
            f32x16 sr = f32x16{}, si = f32x16{}, ev = f32x16{};
#pragma unroll
            for (int j = 0; j < C::KCH; ++j) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(qs + l32 * C::KROW + 8 * j + 4 * h);
                const f32x4 g = *reinterpret_cast<const f32x4 *>(gs + l32 * C::KROW + 8 * j + 4 * h);
                const f32x4 vj = *reinterpret_cast<const f32x4 *>(vw + 8 * j + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    mfma(a[e], kb[j][e], sr);
                    mfma(g[e], vj[e], ev);
                }
                if (born) {
                    const f32x4 k2 = {-kb[j][1], kb[j][0], -kb[j][3], kb[j][2]};
#pragma unroll
                    for (int e = 0; e < 4; ++e) mfma(a[e], k2[e], si);
                }
            }
            // register r of lane half h is query 8 (r/4) + 4 h + r % 4 of the stage
            float wl[16], pr[16], pi[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 av = *reinterpret_cast<const f32x4 *>(sa + 8 * g + 4 * h);
                const f32x4 bv = *reinterpret_cast<const f32x4 *>(sb + 8 * g + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    const int qi = 8 * g + 4 * h + e;
                    const bool keep = !((diag && qi < l32) || q0 + qi >= T);
                    if (born) {
                        const float w = sr[r] * sr[r] + si[r] * si[r];
                        // DECAY: gamma^(query - key) on the weight and on D2
                        const float f = DECAY ? decay_pow(p.decay.lg2[bh % p.H], max(q0 + qi - (kt0 + l32), 0)) : 1.f;
                        wl[r] = keep ? w * av[e] * f : 0.f;
                        const float d2 = keep ? 2.f * (ev[r] - bv[e]) * av[e] * f : 0.f;
                        pr[r] = d2 * sr[r];
                        pi[r] = d2 * si[r];
                    } else {
                        const float w = sigmoid(sr[r] * sqd * av[e] * rk + p.bias);
                        wl[r] = keep ? w : 0.f;
                        const float ds = keep ? ev[r] * w * (1.f - w) : 0.f;
                        pr[r] = sqd * ds * av[e];   // sqrt(d) ds qh on the raw query row
                        pi[r] = 0.f;
                    }
                }
            }
            // dV'^T += G'^T W, dK'^T += Q'^T Re P (- Q''^T Im P); instruction r takes query 8 (r/4) + 4 h + r % 4
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qi = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
                for (int c = 0; c < C::CT; ++c) {
                    const float g = gs[qi * C::KROW + 32 * c + l32];
                    const float a = qs[qi * C::KROW + 32 * c + l32];
                    mfma(g, wl[r], dv[c]);
                    mfma(a, pr[r], dk[c]);
                    if (born) mfma(nsgn * swap_adj(a), pi[r], dk[c]);
                }
            }
        }
        if (st + 1 < nstages) store_stage(buf ^ 1, q0 + BN);
        __syncthreads();
    }

    // lane (key l32, half h) holds components n = 32 c + 8 (r/4) + 4 h + r % 4,
    // the components kb[4 c + r/4][r % 4] of K'
    if (!born) {
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < C::CT; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) dot += dk[c][r] * kb[4 * c + (r >> 2)][r & 3];
        dot += __shfl_xor(dot, 32);
        dot *= rk * rk;
#pragma unroll
        for (int c = 0; c < C::CT; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) dk[c][r] = (dk[c][r] - dot * kb[4 * c + (r >> 2)][r & 3]) * rk;
    }
    if (krow >= T) return;
#pragma unroll
    for (int c = 0; c < C::CT; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            store4<LAY, D>(p.dk_re, p.dk_im, hrow + krow, 32 * c + 8 * g + 4 * h,
                           f32x4{dk[c][4 * g], dk[c][4 * g + 1], dk[c][4 * g + 2], dk[c][4 * g + 3]});
            store4<LAY, D>(p.dv_re, p.dv_im, hrow + krow, 32 * c + 8 * g + 4 * h,
                           f32x4{dv[c][4 * g], dv[c][4 * g + 1], dv[c][4 * g + 2], dv[c][4 * g + 3]});
        }
}

template <int D, int OP, int LAY, bool DECAY = false>
hipError_t launch_cfg(const BwdProblem &p) {
    using C = BCfg<D>;
    static std::atomic<uint64_t> dq_set{0}, kv_set{0};
    const int nblk = (p.T + BM - 1) / BM;
    const int64_t blocks = (int64_t)p.BH * nblk;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    auto kkv = bwd_dkdv_f32_kernel<D, OP, LAY, DECAY>;
    auto kdq = bwd_dq_f32_kernel<D, OP, LAY, DECAY>;
    hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kkv), C::LDS_BYTES_KV, kv_set);
    if (e != hipSuccess) return e;
    e = set_dynamic_lds(reinterpret_cast<const void *>(kdq), C::LDS_BYTES, dq_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kkv, dim3((unsigned)blocks), dim3(NT), C::LDS_BYTES_KV, p.stream, p, nblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kdq, dim3((unsigned)blocks), dim3(NT), C::LDS_BYTES, p.stream, p, nblk);
    return hipGetLastError();
}

template <int D, int LAY>
hipError_t launch_op(const BwdProblem &p) {
    if (p.op == OP_BORN)
        return p.decay.on ? launch_cfg<D, OP_BORN, LAY, true>(p) : launch_cfg<D, OP_BORN, LAY>(p);
    return launch_cfg<D, OP_PCT, LAY>(p);
}

template <int D>
hipError_t launch_d(const BwdProblem &p) {
    return p.layout == LAYOUT_C64 ? launch_op<D, LAYOUT_C64>(p) : launch_op<D, LAYOUT_BF16>(p);
}

}  // namespace

bool supports_bwd_f32_mfma(const BwdProblem &p) {
    // complex64, or bf16 planes widened to fp32 on load, at width 16 (the
    // widths 32, 64 and 128 run on the 16 x 16 kernels, and bf16 Born at 64 on
    // its own bf16 pair)
    return (p.op == OP_BORN || p.op == OP_PCT) && p.d == 16;
}

hipError_t launch_bwd_f32_mfma(const BwdProblem &p) {
    return p.d == 16 ? launch_d<16>(p) : hipErrorNotSupported;
}

}  // namespace cattn
