// Born and phase-coherent attention forward on interleaved complex64 with
// gfx950 fp32 matrix cores in their 16 x 16 form (v_mfma_f32_16x16x4_f32),
// fp32 throughout.
//
// Operators.  Born ("CNet: A Complex-Valued Deep Learning Framework ...",
// section 11.2, "Closing it: Born-rule attention", Figure 2): w = |<q, k>|^2
// with a running row sum (no running maximum: w >= 0), O = acc / sum.  PCT
// ("Complex-valued Phase-Coherent Transformers", section 1 and Appendix D.2):
// w = sigmoid(sqrt(d_h) Re<q,k> / (|q| |k|) + b), O = acc, and the cells of the
// same family on that score (L2-softmax, screening gate).  The query norms
// come from the resident query operands, the key norms are reduced while a
// key stage is staged into LDS.
//
// Why 16-query tiles.  With 32-query tiles a causal problem of B*H heads of T
// tokens has B*H*T/32 tiles, and the last tile of a head does twice the
// average work.  When that tile count is about the SIMD count (four heads of
// 1024 tokens times eight, for instance) the grid cannot be balanced: pairing
// a long tile with a short one halves the number of waves.  With 16-query
// tiles there are twice as many tiles.  A workgroup of eight waves takes a
// pair of 64-query row blocks of a head at once, one wave of each block per
// SIMD: causal, the mirrored pair (nrb - 1 - i, i), so every SIMD carries the
// same work; without a mask, two neighbouring blocks.  Two waves are resident
// per SIMD to hide each other's latency.
//
// Products.  A complex64 row x is the real row x' = (Re x0, Im x0, Re x1, ...)
// of width 2d.  With q''' = (Im q0, -Re q0, Im q1, -Re q1, ...),
//     Re <q, k> = sum_n k'[n] q'[n],   Im <q, k> = sum_n k'[n] q'''[n]
// (<q, k> = sum_m q_m conj(k_m)), so one K' operand read from LDS feeds both
// products and the two query operands q', q''' stay in registers.  Scores are
// formed transposed, S^T = K' Q'^T: keys are MFMA rows, queries columns.  The
// contraction index is visited in any order that the A and B operands share;
// lane group g = lane / 16 takes the contiguous quarter [g d/2, (g+1) d/2) of
// the row, so each lane reads its K' slice with wide LDS reads.
//
// Values.  O'^T += V'^T W^T over a 16-key block in 4 steps of 4 keys.  Lane
// (g, query j) holds S^T rows (keys) 4 g + r, r = 0..3; step t uses key 4 g + t
// from lane group g, which is its own register r = t, so the weights need no
// shuffle.  Output channel tile c, row i stands for real channel (d/8) i + c, so
// the V' slice a lane needs for one key is d/8 contiguous floats, and the output
// rows a lane ends with are 4 (d/8) contiguous floats of its query.  At d = 64
// rows i with ((i >> 2) ^ (i >> 3)) odd take the two halves of their slice in
// the other order (channel 8 i + (c ^ 4)): each 16-byte read of a slice then
// touches every LDS bank once, whether the hardware serves it 16 lanes over 64
// banks or 8 lanes over 32, instead of hitting half of them twice.
//
// LDS banks.  Rows are padded by 4 floats (K' reads conflict-free).  A staging
// lane writes its key row's 16-byte chunks c + 8 i, rotated by 7 chunks on odd
// key rows, so the 16 lanes of one write, two key rows, cover all 64 banks
// (widths 32 and 64; at 16 the writes stay two-way).
//
// Born options.  A per-head decay multiplies each weight by gamma^(k - j),
// formed per weight as exp2((k - j) log2 gamma) (the diagonal block's masked
// weights are zeroed after it).  A rotary Q is rotated as its operands are
// loaded, with the arithmetic of the rotary pass (rotary_math.h).
#include "cattn_internal.h"
#include "rotary_math.h"

namespace cattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int NW = 8;          // waves per workgroup: two row blocks of four tiles
constexpr int NT = 64 * NW;    // threads
constexpr int NST = 256;       // threads that stage K and V (the first four waves; all eight at d = 128)
constexpr int TQ = 16;         // queries per wave tile
constexpr int BM = TQ * 4;     // queries per row block
constexpr int BN = 32;         // keys per LDS stage (two 16-key blocks)

template <int D>
struct Cfg16 {
    static constexpr int KD = 2 * D;        // real width of a row
    static constexpr int KQ = KD / 4;       // contraction floats per lane group (= k-steps)
    static constexpr int NC = KD / 16;      // 16-row channel tiles of O'^T
    static constexpr int CPL = KD / 16;     // channels per lane per key in the value operand
    static constexpr int ROW = KD + 4;      // padded LDS row (floats) of K' and V'
    static constexpr int STAGE = 2 * BN * ROW + BN;   // K', V', per-key inverse norms
    static constexpr int LDS_BYTES = 2 * STAGE * 4;
    static constexpr int NSTG = D >= 128 ? 2 * NST : NST;   // staging threads
    static constexpr int LPK = NSTG / BN;             // staging lanes per key (8; 16 at d = 128)
    static constexpr int CPT = (KD / 4) / LPK;        // float4 chunks per staging lane
    // d = 128: the (Im, -Re) query operand is formed as it is used rather than
    // held (64 more registers), and a lane's K' slice is read in pieces of 16
    static constexpr bool QIM = D < 128;
    static constexpr int KP = D < 128 ? KQ : 16;      // K' floats per LDS read batch
};

// n floats from LDS into registers with the widest reads that fit
template <int N>
__device__ inline void lds_row(const float *p, float (&out)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const f32x4 x = *reinterpret_cast<const f32x4 *>(p + 4 * i);
            out[4 * i] = x[0];
            out[4 * i + 1] = x[1];
            out[4 * i + 2] = x[2];
            out[4 * i + 3] = x[3];
        }
    } else {
        static_assert(N % 2 == 0, "even slices only");
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const f32x2 x = *reinterpret_cast<const f32x2 *>(p + 2 * i);
            out[2 * i] = x[0];
            out[2 * i + 1] = x[1];
        }
    }
}

__device__ inline f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// LAY = LAYOUT_C64: interleaved complex64 in and out.  LAY = LAYOUT_BF16: two
// bf16 planes per operand, widened to the same interleaved fp32 rows while K
// and V are staged and Q is loaded, and rounded back to bf16 planes on store
// (round to nearest even); all arithmetic stays fp32.
// OPT: the Born options (decay, rotary Q) may be on; a separate instance, so
// the plain kernel carries none of their registers.
template <int D, int OP, int LAY, bool OPT>
__global__ __launch_bounds__(NT) void attn_f32_mfma16_kernel(Problem p, int nrb, int nwork) {
    using C = Cfg16<D>;
    static_assert(C::CPT >= 1, "head width too small for this staging split");
    extern __shared__ __align__(16) float fsm[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j16 = lane & 15;   // query column (scores, values) / key row (K' operand)
    const int g = lane >> 4;     // lane group
    const int T = p.T;

    // Workgroup -> (head, item); all items of a head on one XCD when BH % 8 == 0
    const int L = blockIdx.x;
    int bh, item;
    if ((p.BH & 7) == 0) {
        const int x = L & 7, jj = L >> 3;
        bh = x + 8 * (jj / nwork);
        item = jj % nwork;
    } else {
        bh = L / nwork;
        item = L % nwork;
    }
    // head bases (elements: complex64 values, or bf16 values of a plane) and
    // token strides of each operand; a complex64 element is two floats
    const int64_t hq = head_offset(p.sq, bh, p.H), hk = head_offset(p.sk, bh, p.H);
    const int64_t hv = head_offset(p.sv, bh, p.H), ho = head_offset(p.so, bh, p.H);
    const int64_t rsq = p.sq.t, rsk = p.sk.t, rsv = p.sv.t, rso = p.so.t;
    const float lg2 = OPT && p.decay.on ? p.decay.lg2[bh % p.H] : 0.f;
    const float *qg = reinterpret_cast<const float *>(p.q_re) + 2 * hq;
    const float *kg = reinterpret_cast<const float *>(p.k_re) + 2 * hk;
    const float *vg = reinterpret_cast<const float *>(p.v_re) + 2 * hv;
    float *og = reinterpret_cast<float *>(p.o_re) + 2 * ho;
    auto plane = [&](const void *x, int64_t off) { return reinterpret_cast<const uint16_t *>(x) + off; };
    const uint16_t *bq_re = plane(p.q_re, hq), *bq_im = plane(p.q_im, hq), *bk_re = plane(p.k_re, hk),
                   *bk_im = plane(p.k_im, hk), *bv_re = plane(p.v_re, hv), *bv_im = plane(p.v_im, hv);
    uint16_t *ore = reinterpret_cast<uint16_t *>(p.o_re) + ho;
    uint16_t *oim = reinterpret_cast<uint16_t *>(p.o_im) + ho;
    // complex elements 2 e, 2 e + 1 of a row as the interleaved fp32 chunk
    auto widen2 = [&](const uint16_t *re, const uint16_t *im, int64_t el) {
        const uint32_t r2 = *reinterpret_cast<const uint32_t *>(re + el);
        const uint32_t i2 = *reinterpret_cast<const uint32_t *>(im + el);
        return f32x4{bf_lo(r2), bf_lo(i2), bf_hi(r2), bf_hi(i2)};
    };

    // Waves 0-3 take the four tiles of the first row block of the item, waves
    // 4-7 those of the second, at the same time: a SIMD holds one wave of each.
    // Causal: the mirrored pair nrb-1-item (long) and item (short), whose key
    // range is a prefix of the long one's, so both read the same stages.  The
    // middle block of an odd count has no partner.  Without a mask: the row
    // blocks 2 item and 2 item + 1.
    const int half = wave >> 2;
    int rb;
    if (p.causal)
        rb = half == 0 ? nrb - 1 - item : (item != nrb - 1 - item ? item : -1);
    else
        rb = 2 * item + half < nrb ? 2 * item + half : -1;
    const int m0 = rb * BM;
    const int qt0 = m0 + TQ * (wave & 3);   // first query of this wave's tile
    const int qrow = qt0 + j16;
    const bool live = rb >= 0 && qt0 < T;
    const bool stager = tid < C::NSTG;       // wave-uniform
    // d = 64: value rows i with ((i >> 2) ^ (i >> 3)) odd take their slice's
    // halves swapped; as A operand row i = j16, as output row i = 4 g + r
    const int vsw = C::CPL == 8 ? 4 * (((j16 >> 2) ^ (j16 >> 3)) & 1) : 0;
    const int osw = C::CPL == 8 ? 4 * ((g ^ (g >> 1)) & 1) : 0;

    // staging: thread t holds CPT 16-byte chunks of key row t / LPK, chunk
    // (t % LPK) + LPK i rotated by 7 on odd rows (see the LDS note above)
    const int skey = tid / C::LPK;
    const int sc = tid % C::LPK;
    constexpr int NCH = C::KD / 4;                 // 16-byte chunks per row
    constexpr int ROT = D >= 32 ? 7 : 0;           // odd key rows: chunk rotation
    auto chunk_of = [&](int i) { return (sc + C::LPK * i + ROT * (skey & 1)) % NCH; };
    f32x4 kreg[C::CPT], vreg[C::CPT];
    auto load_stage = [&](int k0) {
        const int kr = k0 + skey;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
            if (kr < T) {
                if constexpr (LAY == LAYOUT_C64) {
                    a = *reinterpret_cast<const f32x4 *>(kg + 2 * (int64_t)kr * rsk + 4 * chunk_of(i));
                    b = *reinterpret_cast<const f32x4 *>(vg + 2 * (int64_t)kr * rsv + 4 * chunk_of(i));
                } else {
                    a = widen2(bk_re, bk_im, (int64_t)kr * rsk + 2 * chunk_of(i));
                    b = widen2(bv_re, bv_im, (int64_t)kr * rsv + 2 * chunk_of(i));
                }
            }
            kreg[i] = a;
            vreg[i] = b;
        }
    };
    auto store_stage = [&](int buf) {
        float *ks = fsm + buf * C::STAGE;
        float *vs = ks + BN * C::ROW;
        float *rk = vs + BN * C::ROW;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            *reinterpret_cast<f32x4 *>(ks + skey * C::ROW + 4 * chunk_of(i)) = kreg[i];
            *reinterpret_cast<f32x4 *>(vs + skey * C::ROW + 4 * chunk_of(i)) = vreg[i];
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

    // query operands q', q''' over this lane group's quarter of the row, and
    // PCT's sqrt(d_h) / |q| (0 for a zero row)
    float qre[C::KQ], qim[C::QIM ? C::KQ : 1];
    float rq = 0.f;
    auto load_q = [&](int qt, bool ok) {
        const int qr = qt + j16;
        f32x4 x[C::KQ / 4];
#pragma unroll
        for (int i = 0; i < C::KQ / 4; ++i) {
            x[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (ok && qr < T) {
                if constexpr (LAY == LAYOUT_C64)
                    x[i] = *reinterpret_cast<const f32x4 *>(qg + 2 * (int64_t)qr * rsq + g * C::KQ + 4 * i);
                else
                    x[i] = widen2(bq_re, bq_im, (int64_t)qr * rsq + g * (C::KQ / 2) + 2 * i);
            }
        }
        if (OPT && p.rot && ok && qr < T) {
            // complex channels g KQ / 2 + 2 i + e of query qr
            const double pos = (double)(p.rot_pos0 + qr);
#pragma unroll
            for (int i = 0; i < C::KQ / 4; ++i)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    float c, sn;
                    rotary_phase(pos, rotary_theta(g * (C::KQ / 2) + 2 * i + e, p.rot_log_base, D), c, sn);
                    float yr, yi;
                    rotary_apply(x[i][2 * e], x[i][2 * e + 1], c, sn, yr, yi);
                    x[i][2 * e] = yr;
                    x[i][2 * e + 1] = yi;
                }
        }
#pragma unroll
        for (int i = 0; i < C::KQ / 4; ++i) {
            qre[4 * i] = x[i][0];
            qre[4 * i + 1] = x[i][1];
            qre[4 * i + 2] = x[i][2];
            qre[4 * i + 3] = x[i][3];
            // (Im, -Re) per complex element; a quarter starts on an element boundary
            if constexpr (C::QIM) {
                qim[4 * i] = x[i][1];
                qim[4 * i + 1] = -x[i][0];
                qim[4 * i + 2] = x[i][3];
                qim[4 * i + 3] = -x[i][2];
            }
        }
        if (OP != OP_BORN) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < C::KQ; ++i) ss += qre[i] * qre[i];
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            rq = ss > 0.f ? sqrtf((float)D) / sqrtf(ss) : 0.f;
        }
    };

    f32x4 oacc[C::NC];
    float rsum = 0.f;
    auto reset = [&]() {
#pragma unroll
        for (int c = 0; c < C::NC; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        rsum = 0.f;
    };

    // epilogue: lane (g, query j16) holds O'^T rows 4 g + r of tile c, i.e.
    // real channel CPL (4 g + r) + (c ^ osw) of its query: 4 CPL contiguous
    // floats.
    auto write_out = [&](int qt) {
        const int qr = qt + j16;
        float scale = 1.f;
        float den = 0.f;
        if (OP == OP_BORN || OP == OP_PCT_SOFTMAX) {
            den = rsum + __shfl_xor(rsum, 16);
            den += __shfl_xor(den, 32);
            if (OP == OP_BORN) den += p.eps;
            scale = den != 0.f ? 1.f / den : 0.f;
        }
        if (qr < T) {
            float *orow = og + 2 * (int64_t)qr * rso + 4 * C::CPL * g;
            // bf16 planes: real channel n is element n / 2 of the Re (n even) or Im plane
            const int64_t brow = (int64_t)qr * rso + 2 * C::CPL * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (C::CPL % 4 == 0) {
#pragma unroll
                    for (int c = 0; c < C::NC; c += 4) {
                        const f32x4 v = {oacc[c][r] * scale, oacc[c + 1][r] * scale, oacc[c + 2][r] * scale,
                                         oacc[c + 3][r] * scale};
                        const int ch = C::CPL * r + (c ^ osw);   // first of 4 channels, relative to the lane's run
                        if constexpr (LAY == LAYOUT_C64) {
                            *reinterpret_cast<f32x4 *>(orow + ch) = v;
                        } else {
                            *reinterpret_cast<uint32_t *>(ore + brow + ch / 2) = pack_bf16x2(v[0], v[2]);
                            *reinterpret_cast<uint32_t *>(oim + brow + ch / 2) = pack_bf16x2(v[1], v[3]);
                        }
                    }
                } else {
                    const f32x2 v = {oacc[0][r] * scale, oacc[1][r] * scale};
                    if constexpr (LAY == LAYOUT_C64) {
                        *reinterpret_cast<f32x2 *>(orow + C::CPL * r) = v;
                    } else {
                        const uint32_t pk = pack_bf16x2(v[0], v[1]);
                        ore[brow + r] = (uint16_t)(pk & 0xffffu);
                        oim[brow + r] = (uint16_t)(pk >> 16);
                    }
                }
            }
            if (OP == OP_BORN && p.row_den && g == 0) p.row_den[(int64_t)bh * T + qr] = den;
        }
    };

    // Causal: a wave of the short block, once past its own diagonal, helps the
    // long tile of its SIMD partner (wave - 4).  From stage st_switch on, the
    // partner keeps the first 16-key block of each stage and the helper takes
    // the second; at the end the helper's partial sums are added to the
    // partner's through LDS, in a fixed order, so the result does not depend on
    // timing.  Without a short block (the middle block of an odd count) the
    // helpers start at once.  Without a mask nothing is shared.
    const int tq = wave & 3;
    const int rbL = nrb - 1 - item;
    const int qtL = rbL * BM + TQ * tq;          // the long tile of this SIMD slot
    const bool liveL = p.causal && qtL < T;
    int st_switch = 0x7fffffff;
    if (p.causal) st_switch = item != rbL ? (item * BM + TQ * tq) / BN + 1 : 0;

    // keys for both row blocks: the first (long) one's range
    const int kend = p.causal ? min(T, rbL * BM + BM) : T;
    const int nstages = (kend + BN - 1) / BN;

    int qt_cur = qt0;
    bool live_cur = live;
    bool helping = false;
    load_q(qt0, live);
    reset();

    if (stager && nstages > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();

    for (int st = 0; st < nstages; ++st) {
        const int k0 = st * BN;
        const int buf = st & 1;
        if (half == 1 && st == st_switch) {   // wave-uniform
            if (live) write_out(qt0);
            helping = true;
            qt_cur = qtL;
            live_cur = liveL;
            load_q(qtL, liveL);
            reset();
        }
        const bool split = st >= st_switch;
        if (stager && st + 1 < nstages) load_stage(k0 + BN);
        const float *ks = fsm + buf * C::STAGE;
        const float *vs = ks + BN * C::ROW;
        const float *rk = vs + BN * C::ROW;

#pragma unroll
        for (int sb = 0; sb < BN / 16; ++sb) {
            if (split && sb != half) continue;   // long wave: block 0, helper: block 1
            const int kb0 = k0 + 16 * sb;
            if (!live_cur || kb0 >= T || (p.causal && kb0 > qt_cur)) continue;
            const bool diag = p.causal && kb0 == qt_cur;

            // S^T for 16 keys x 16 queries
            f32x4 sr = {0.f, 0.f, 0.f, 0.f}, si = {0.f, 0.f, 0.f, 0.f};
            // d = 128: the sign flip of -Re q made opaque here, so that it is
            // applied per product and not hoisted into 32 more registers
            uint32_t sgn = 0x80000000u;
            if constexpr (!C::QIM) __asm__ __volatile__("" : "+v"(sgn));
#pragma unroll
            for (int p0 = 0; p0 < C::KQ; p0 += C::KP) {
                float ka[C::KP];
                lds_row<C::KP>(ks + (16 * sb + j16) * C::ROW + g * C::KQ + p0, ka);
#pragma unroll
                for (int s3 = 0; s3 < C::KP; ++s3) {
                    const int s2 = p0 + s3;
                    sr = mfma16(ka[s3], qre[s2], sr);
                    if (OP == OP_BORN) {
                        float qi;
                        if constexpr (C::QIM)
                            qi = qim[s2];
                        else   // (Im, -Re): element s2 + 1 (even s2), or minus element s2 - 1 (odd)
                            qi = (s2 & 1) ? __uint_as_float(__float_as_uint(qre[s2 - 1]) ^ sgn) : qre[s2 + 1];
                        si = mfma16(ka[s3], qi, si);
                    }
                }
            }

            // weights: register r is key 4 g + r of the block
            float w[4];
            if (OP == OP_BORN) {
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = sr[r] * sr[r] + si[r] * si[r];
                if (OPT && p.decay.on) {   // gamma^(k - j); negative distances only on masked keys
#pragma unroll
                    for (int r = 0; r < 4; ++r) w[r] *= decay_pow(lg2, max(qt_cur + j16 - kb0 - 4 * g - r, 0));
                }
            } else {
                const f32x4 rkv = *reinterpret_cast<const f32x4 *>(rk + 16 * sb + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = sr[r] * rq * rkv[r];   // sqrt(d_h) Re<qh, kh>
                    if (OP == OP_PCT) {
                        // hardware reciprocal (1 ulp), not the IEEE division sequence
                        w[r] = __builtin_amdgcn_rcpf(1.f + __expf(-(x + p.bias)));
                    } else if (OP == OP_PCT_SOFTMAX) {
                        w[r] = __expf(x);   // |x| <= sqrt(d_h): no shift needed
                    } else {
                        const float y = fmaxf(x - p.gate_t, 0.f);
                        w[r] = p.gate_r * p.gate_r * y * y;
                    }
                }
            }
            if (diag || kb0 + 16 > T) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = 4 * g + r;
                    if ((diag && key > j16) || kb0 + key >= T) w[r] = 0.f;
                }
            }
            if (OP == OP_BORN || OP == OP_PCT_SOFTMAX) rsum += (w[0] + w[1]) + (w[2] + w[3]);

            // O'^T += V'^T W^T: step t takes key 4 g + t from lane group g
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float va[C::CPL];
                const float *vrow = vs + (16 * sb + 4 * g + t) * C::ROW + C::CPL * j16;
                if constexpr (C::CPL == 8) {   // halves in the order of this row's channels
                    const f32x4 x0 = *reinterpret_cast<const f32x4 *>(vrow + vsw);
                    const f32x4 x1 = *reinterpret_cast<const f32x4 *>(vrow + (4 ^ vsw));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        va[e] = x0[e];
                        va[4 + e] = x1[e];
                    }
                } else {
                    lds_row<C::CPL>(vrow, va);
                }
#pragma unroll
                for (int c = 0; c < C::NC; ++c) oacc[c] = mfma16(va[c], w[t], oacc[c]);
            }
        }

        if (stager && st + 1 < nstages) store_stage(buf ^ 1);
        __syncthreads();
    }

    // merge the helpers' partial sums (the stage buffers are free now)
    if (p.causal) {
        constexpr int PW = 4 * C::NC + 1;   // floats per lane of one partial
        static_assert(4 * PW * 64 <= 2 * C::STAGE, "partials fit in the stage buffers");
        float *part = fsm + tq * PW * 64 + lane;
        if (helping && liveL) {
#pragma unroll
            for (int c = 0; c < C::NC; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) part[(4 * c + r) * 64] = oacc[c][r];
            part[4 * C::NC * 64] = rsum;
        }
        __syncthreads();
        if (half == 0 && st_switch < nstages && liveL) {
#pragma unroll
            for (int c = 0; c < C::NC; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) oacc[c][r] += part[(4 * c + r) * 64];
            rsum += part[4 * C::NC * 64];
        }
    }
    if (!helping && live_cur) write_out(qt_cur);
}

template <int D, int OP, int LAY, bool OPT = false>
hipError_t launch_cfg16(const Problem &p) {
    using C = Cfg16<D>;
    auto kern = attn_f32_mfma16_kernel<D, OP, LAY, OPT>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), C::LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
    const int nrb = (p.T + BM - 1) / BM;
    const int nwork = (nrb + 1) / 2;   // row blocks in pairs, causal or not
    const int64_t blocks = (int64_t)p.BH * nwork;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), C::LDS_BYTES, p.stream, p, nrb, nwork);
    return hipGetLastError();
}

template <int D, int LAY>
hipError_t launch_op16(const Problem &p) {
    switch (p.op) {
        case OP_BORN:   // bf16 Born runs on the bf16 matrix-core kernels
            if constexpr (LAY == LAYOUT_C64) {
                if (p.decay.on || p.rot) return launch_cfg16<D, OP_BORN, LAY, true>(p);
                return launch_cfg16<D, OP_BORN, LAY>(p);
            }
            return hipErrorNotSupported;
        case OP_PCT: return launch_cfg16<D, OP_PCT, LAY>(p);
        case OP_PCT_SOFTMAX: return launch_cfg16<D, OP_PCT_SOFTMAX, LAY>(p);
        default: return launch_cfg16<D, OP_PCT_SCREEN, LAY>(p);
    }
}

template <int D>
hipError_t launch_d16(const Problem &p) {
    return p.layout == LAYOUT_C64 ? launch_op16<D, LAYOUT_C64>(p) : launch_op16<D, LAYOUT_BF16>(p);
}

}  // namespace

// complex64 (every operator) and bf16 planes (the PCT cells: bf16 Born has
// its own bf16 matrix-core kernels) at widths 16, 32, 64 and 128
bool supports_f32_mfma16(const Problem &p) {
    return (p.d == 16 || p.d == 32 || p.d == 64 || p.d == 128) && (p.layout == LAYOUT_C64 || p.op != OP_BORN) &&
           p.aligned16;
}

hipError_t launch_f32_mfma16(const Problem &p) {
    switch (p.d) {
        case 16: return launch_d16<16>(p);
        case 32: return launch_d16<32>(p);
        case 64: return launch_d16<64>(p);
        case 128: return launch_d16<128>(p);
        default: return hipErrorNotSupported;
    }
}

}  // namespace cattn
