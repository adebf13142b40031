// Born and phase-coherent attention forward on interleaved complex64 with
// gfx950 fp32 matrix cores (v_mfma_f32_32x32x2_f32), fp32 throughout.
//
// Complex contraction as real GEMMs in the interleaved order.  A complex64
// row x is the real row x' = (Re x0, Im x0, Re x1, Im x1, ...).  Then
//     Re <q, k> = sum_n k'[n] q'[n]
//     Im <q, k> = sum_n k''[n] q'[n],   k'' = (-Im k0, Re k0, -Im k1, Re k1, ...)
// (<q, k> = sum_m q_m conj(k_m)).  k'' is formed in registers from k' with
// two negations per four values, so the Q' operand is held once.  Scores are
// formed transposed (keys = MFMA rows, queries = MFMA columns); each lane then
// holds one query and 16 keys, the shape of the W^T operand of
//     O'^T = V'^T W^T
// with V' the interleaved value rows; the output rows come out interleaved.
//
// Born ("CNet ...", section 11.2, "Closing it: Born-rule attention"):
// w = |S|^2 with a running row sum (no running maximum: w >= 0), O = acc / sum.
// PCT ("Complex-valued Phase-Coherent Transformers", section 1, Appendix D.2):
// w = sigmoid(sqrt(d_h) Re<q,k> / (||q|| ||k||) + b), O = acc; the query norms
// come from the resident Q' operands, the key norms are reduced while a key
// tile is staged into LDS.
#include "cattn_internal.h"

namespace cattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 4;          // waves per workgroup
constexpr int NT = 64 * NW;    // threads
constexpr int BM = 32 * NW;    // query rows per workgroup (one 32-query tile per wave)
constexpr int BN = 32;         // keys per LDS stage

template <int D>
struct F32Cfg {
    static constexpr int KD = 2 * D;                 // interleaved real width of a row
    static constexpr int KSTEPS = KD / 2;            // MFMA k-steps (2 per instruction)
    static constexpr int KCH = KD / 8;               // float4 chunks per lane half of a row
    static constexpr int CT = KD / 32;               // 32-row tiles of O'^T
    static constexpr int KROW = KD + 4;              // padded LDS row of K' (floats)
    static constexpr int VROW = KD;                  // LDS row of V' (floats)
    static constexpr int K_ELEMS = BN * KROW;
    static constexpr int V_ELEMS = BN * VROW;
    static constexpr int STAGE = K_ELEMS + V_ELEMS + BN;   // + per-key inverse norms
    static constexpr int LDS_BYTES = 2 * STAGE * 4;
    static constexpr int LPK = NT / BN;              // staging lanes per key (8)
    static constexpr int CPT = (KD / 4) / LPK;       // float4 chunks per staging lane
};

template <int D, int OP>
__global__ __launch_bounds__(NT) void attn_f32_mfma_kernel(Problem p, int nrb) {
    using C = F32Cfg<D>;
    static_assert(C::CPT >= 1, "head width too small for this staging split");
    extern __shared__ __align__(16) float fsm[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int T = p.T;

    const int L = blockIdx.x;
    int bh, rb;
    if ((p.BH & 7) == 0) {       // all row blocks of a head on one XCD, heaviest first
        const int x = L & 7, j = L >> 3;
        bh = x + 8 * (j / nrb);
        rb = nrb - 1 - (j % nrb);
    } else {
        bh = L / nrb;
        rb = nrb - 1 - (L % nrb);
    }
    const int m0 = rb * BM;
    const int64_t head = (int64_t)bh * T * C::KD;      // in floats
    const float *qg = reinterpret_cast<const float *>(p.q_re) + head;
    const float *kg = reinterpret_cast<const float *>(p.k_re) + head;
    const float *vg = reinterpret_cast<const float *>(p.v_re) + head;

    // Q' operand: lane (q = l32, h) holds q'[8 j + 4 h .. +3] for chunk j; k-step
    // s uses element s % 4 of chunk s / 4, i.e. q'[8 (s/4) + 4 h + s % 4].
    const int qt0 = m0 + 32 * wave;
    const int qrow = qt0 + l32;
    f32x4 qb[C::KCH];
#pragma unroll
    for (int j = 0; j < C::KCH; ++j) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (qrow < T) x = *reinterpret_cast<const f32x4 *>(qg + (int64_t)qrow * C::KD + 8 * j + 4 * h);
        qb[j] = x;
    }
    float rq = 0.f;
    if (OP != OP_BORN) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < C::KCH; ++j) ss += qb[j][0] * qb[j][0] + qb[j][1] * qb[j][1] + qb[j][2] * qb[j][2] +
                                               qb[j][3] * qb[j][3];
        ss += __shfl_xor(ss, 32);
        rq = ss > 0.f ? sqrtf((float)D) / sqrtf(ss) : 0.f;   // sqrt(d_h) / ||q||, 0 for a zero row
    }

    f32x16 oacc[C::CT];
#pragma unroll
    for (int c = 0; c < C::CT; ++c) oacc[c] = f32x16{};
    float rsum = 0.f;

    const int kend = p.causal ? min(T, m0 + BM) : T;
    const int nstages = (kend + BN - 1) / BN;

    // staging: lane t holds CPT consecutive float4 chunks of key t / LPK
    const int skey = tid / C::LPK;
    const int schunk = (tid % C::LPK) * C::CPT;
    f32x4 kreg[C::CPT], vreg[C::CPT];

    auto load_stage = [&](int k0) {
        const int kr = k0 + skey;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
            if (kr < T) {
                a = *reinterpret_cast<const f32x4 *>(kg + (int64_t)kr * C::KD + 4 * (schunk + i));
                b = *reinterpret_cast<const f32x4 *>(vg + (int64_t)kr * C::KD + 4 * (schunk + i));
            }
            kreg[i] = a;
            vreg[i] = b;
        }
    };
    auto store_stage = [&](int buf) {
        float *ks = fsm + buf * C::STAGE;
        float *vs = ks + C::K_ELEMS;
        float *rk = vs + C::V_ELEMS;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            *reinterpret_cast<f32x4 *>(ks + skey * C::KROW + 4 * (schunk + i)) = kreg[i];
            *reinterpret_cast<f32x4 *>(vs + skey * C::VROW + 4 * (schunk + i)) = vreg[i];
        }
        if (OP != OP_BORN) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < C::CPT; ++i)
                ss += kreg[i][0] * kreg[i][0] + kreg[i][1] * kreg[i][1] + kreg[i][2] * kreg[i][2] +
                      kreg[i][3] * kreg[i][3];
#pragma unroll
            for (int o = 1; o < C::LPK; o <<= 1) ss += __shfl_xor(ss, o);
            if (tid % C::LPK == 0) rk[skey] = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
        }
    };

    if (nstages > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();

    for (int st = 0; st < nstages; ++st) {
        const int k0 = st * BN;
        const int buf = st & 1;
        if (st + 1 < nstages) load_stage(k0 + BN);

        const bool live = k0 < T && (!p.causal || k0 <= qt0);
        if (live) {
            const bool diag = p.causal && k0 == qt0;
            const float *ks = fsm + buf * C::STAGE;
            const float *vs = ks + C::K_ELEMS;
            const float *rk = vs + C::V_ELEMS;

            // S^T for 32 keys x 32 queries
            f32x16 sr = f32x16{}, si = f32x16{};
#pragma unroll
            for (int j = 0; j < C::KCH; ++j) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(ks + l32 * C::KROW + 8 * j + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) sr = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qb[j][e], sr, 0, 0, 0);
                if (OP == OP_BORN) {
                    // k'' = (-Im k, Re k) per complex element
                    const f32x4 b = {-a[1], a[0], -a[3], a[2]};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        si = __builtin_amdgcn_mfma_f32_32x32x2f32(b[e], qb[j][e], si, 0, 0, 0);
                }
            }

            // weights; register r of lane half h is key 8 (r/4) + 4 h + r % 4
            float w[16];
            if (OP == OP_BORN) {
#pragma unroll
                for (int r = 0; r < 16; ++r) w[r] = sr[r] * sr[r] + si[r] * si[r];
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 rkv = *reinterpret_cast<const f32x4 *>(rk + 8 * g + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = sr[4 * g + e] * rq * rkv[e];   // sqrt(d_h) Re<qh, kh>
                        if (OP == OP_PCT) {
                            w[4 * g + e] = 1.f / (1.f + __expf(-(x + p.bias)));
                        } else if (OP == OP_PCT_SOFTMAX) {
                            w[4 * g + e] = __expf(x);   // |x| <= sqrt(d_h): no shift needed
                        } else {
                            const float y = fmaxf(x - p.gate_t, 0.f);
                            w[4 * g + e] = p.gate_r * p.gate_r * y * y;
                        }
                    }
                }
            }
            const bool tail = k0 + BN > T;
            if (diag || tail) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 8 * (r >> 2) + 4 * h + (r & 3);
                    if ((diag && key > l32) || k0 + key >= T) w[r] = 0.f;
                }
            }
            if (OP == OP_BORN || OP == OP_PCT_SOFTMAX) {
#pragma unroll
                for (int r = 0; r < 16; ++r) rsum += w[r];
            }

            // O'^T += V'^T W^T: instruction r takes key 8 (r/4) + 4 h + r % 4 from lane half h
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
                for (int c = 0; c < C::CT; ++c) {
                    const float a = vs[key * C::VROW + 32 * c + l32];
                    oacc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, w[r], oacc[c], 0, 0, 0);
                }
            }
        }

        if (st + 1 < nstages) store_stage(buf ^ 1);
        __syncthreads();
    }

    // epilogue: rows of O'^T come out interleaved (re, im, re, im) in groups of 4
    float scale = 1.f;
    float den = 0.f;
    if (OP == OP_BORN || OP == OP_PCT_SOFTMAX) {
        den = rsum + __shfl_xor(rsum, 32) + (OP == OP_BORN ? p.eps : 0.f);
        scale = den != 0.f ? 1.f / den : 0.f;
    }
    if (qrow >= T) return;
    float *og = reinterpret_cast<float *>(p.o_re) + head + (int64_t)qrow * C::KD;
#pragma unroll
    for (int c = 0; c < C::CT; ++c) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 v = {oacc[c][4 * g] * scale, oacc[c][4 * g + 1] * scale, oacc[c][4 * g + 2] * scale,
                             oacc[c][4 * g + 3] * scale};
            *reinterpret_cast<f32x4 *>(og + 32 * c + 8 * g + 4 * h) = v;
        }
    }
    if (OP == OP_BORN && p.row_den && h == 0) p.row_den[(int64_t)bh * T + qrow] = den;
}

template <int D, int OP>
hipError_t launch_cfg(const Problem &p) {
    using C = F32Cfg<D>;
    auto kern = attn_f32_mfma_kernel<D, OP>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), C::LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
    const int nrb = (p.T + BM - 1) / BM;
    const int64_t blocks = (int64_t)p.BH * nrb;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), C::LDS_BYTES, p.stream, p, nrb);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Problem &p) {
    switch (p.op) {
        case OP_BORN: return launch_cfg<D, OP_BORN>(p);
        case OP_PCT: return launch_cfg<D, OP_PCT>(p);
        case OP_PCT_SOFTMAX: return launch_cfg<D, OP_PCT_SOFTMAX>(p);
        default: return launch_cfg<D, OP_PCT_SCREEN>(p);
    }
}

}  // namespace

bool supports_f32_mfma(const Problem &p) {
    return p.layout == LAYOUT_C64 && (p.d == 16 || p.d == 32 || p.d == 64);
}

hipError_t launch_f32_mfma(const Problem &p) {
    switch (p.d) {
        case 16: return launch_d<16>(p);
        case 32: return launch_d<32>(p);
        case 64: return launch_d<64>(p);
        default: return hipErrorNotSupported;
    }
}

}  // namespace cattn
