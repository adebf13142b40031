// Backward of Born and phase-coherent attention at head widths 32, 64 and 128
// on interleaved complex64 (or bf16 planes, widened to the same fp32 rows on
// load and rounded back on store) with gfx950 fp32 matrix cores in their
// 16 x 16 form (v_mfma_f32_16x16x4_f32), fp32 throughout.
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
// Why the 16 x 16 form.  A complex row of d channels is a real row
// x' = (Re x0, Im x0, ...) of KD = 2 d floats.  A wave that owns rows as a
// register operand holds (rows x KD) / 64 floats per lane, and each kernel
// holds two such operands (Q', G' or K', V') beside gradient accumulators of
// the same size.  With 32-row tiles that is 128 floats per operand at d = 128,
// more than a lane has, and at d = 64 it allows one wave per SIMD; with 16-row
// tiles it is KD / 4 floats: two waves per SIMD at 64 and 32.  At 128 Born
// splits each row tile over two waves, each holding one half of the channels
// of every owned row and of every gradient row; the two add their partial
// scores through LDS (one more barrier per block), and two waves per SIMD fit.
// PCT at 128 (fewer products per block to amortise that exchange) keeps one
// wave per SIMD with whole rows.
//
// Products (lane l: j16 = l % 16, lane group g = l / 16; an A operand row and
// a B operand column are j16, the contraction index of a step is g; a result
// lane holds rows 4 g + r of column j16).
//  * Scores: the contraction runs over the real row (over the wave's channel
//    group when a row tile is split) in any order both operands share; lane
//    group g takes the contiguous quarter [KQ g, KQ g + KQ), KQ = KDC / 4, of
//    it, so a lane reads its slice of a streamed row
//    with 16-byte LDS reads.  Re <q, k> = k' . q' and Im <q, k> = k'' . q'
//    with k'' = (-Im k0, Re k0, ...) (equally q''' . k' with
//    q''' = (Im q0, -Re q0, ...)): the swapped, sign-flipped partner is formed
//    from the streamed operand as it is read, and the owned operand is used as
//    it stands.
//  * Gradients: over a 16-row block in 4 steps of 4 rows; step t takes row
//    4 g + t from lane group g, which is its own result register r = t, so the
//    weights need no shuffle.  With NC = KDC / 16 tiles, channel tile c, row i
//    stands for real channel NC i + 4 ((c / 4 + rho(i)) mod (NC / 4)) + c mod 4,
//    rho(i) = (i / (32 / NC) + i / 8) mod (NC / 4): the streamed operand a lane
//    needs for one row is NC contiguous floats (NC / 4 16-byte reads, taken in
//    an order rotated by rho(i) so that each bank is touched once by every 16
//    lanes of a read over 64 banks and by every 8 over 32), and the
//    gradient a lane ends with is the KQ contiguous channels of its quarter.  The imaginary part of a complex product uses
//    the partner channel (c ^ 1, the same rotation) with the sign on the weight.
//
// Three kernels:
//  * Born only: per query, 1 / l and delta, written as float pairs into the
//    dq buffer (it holds B H T 8 bytes many times over, and nothing reads it
//    until the dq kernel overwrites it);
//  * dkdv: a wave owns 16 keys (K', V' in registers) and streams stages of
//    32 queries (16 with split row tiles) of Q', G' (with the pairs, or
//    1 / ||q||) through LDS, in 16-query blocks: lane = key, registers =
//    queries; dV'^T += G'^T W, dK'^T += Q'^T P;
//  * dq: a wave owns 16 queries (Q', G' in registers) and streams stages of K',
//    V' the same way: lane = query, registers = keys; dQ'^T += K'^T P^T.
// Every wave runs every stage of its workgroup with no branch around the
// products: the causal mask, applied per weight, zeroes the blocks above a
// wave's diagonal.  (A branch there made the compiler copy the loop-carried
// gradient accumulators between register files at every stage; the few
// wasted blocks cost less.)
// Nothing is written twice: no atomics, deterministic results.
#include "cattn_internal.h"

namespace cattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int TR = 16;             // rows owned per row tile
constexpr int NW = 4;              // waves per workgroup

template <int D, int CH_ = 1>
struct B16 {
    // Channel groups per row tile: at width 128 two waves share a row tile,
    // each holding one half of every owned row and of every gradient row
    // (about 250 registers a wave instead of 450: two waves per SIMD), and
    // they add their partial scores through LDS.
    static constexpr int CH = CH_;
    static constexpr int NRT = NW / CH;       // row tiles per workgroup
    static constexpr int BM = TR * NRT;       // rows owned per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int BN = CH > 1 ? 16 : 32;   // streamed rows per LDS stage (16-row blocks)
    static constexpr int LPK = NT / BN;       // staging lanes per row
    static constexpr int KD = 2 * D;          // real width of a row (floats)
    static constexpr int KDC = KD / CH;       // real channels of a wave's group
    static constexpr int KQ = KDC / 4;        // contraction floats per lane group
    static constexpr int NC = KDC / 16;       // 16-row tiles of a gradient; also the floats of a lane's run
    static constexpr int NCK = NC / 4;        // 16-byte reads per run
    static constexpr int RDIV = 8 / NCK;      // a run's reads are rotated by (row / RDIV + row / 8) mod NCK
    static constexpr int ROW = KD + 4;        // padded LDS row (floats): a 16-lane read of 16 rows covers every bank once
    static constexpr int NCH = KD / 4;        // 16-byte chunks per row
    static constexpr int CPT = NCH / LPK;     // chunks per staging lane and operand
    static constexpr int STAGE = 2 * BN * ROW + 2 * BN;   // two operands and two per-row scalars (floats)
    static constexpr int XCH = CH > 1 ? NW * 12 * 64 : 0;  // per wave, 12 partial sums a lane
    static constexpr int LDS_BYTES = (2 * STAGE + XCH) * 4;
    static constexpr int KP = KQ < 16 ? KQ : 16;          // contraction floats per LDS read batch of the scores
    // waves per SIMD: two, except at width 128 without channel groups (about
    // 450 registers a wave)
    static constexpr int WPE = D >= 128 && CH == 1 ? 1 : 2;
    static_assert(CPT * LPK == NCH && NCK >= 1 && NC % 4 == 0, "width");
};

__device__ inline f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// hardware reciprocal (1 ulp), not the IEEE division sequence
__device__ inline float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Floats f .. f + 3 (complex elements f / 2, f / 2 + 1) of dense row `row`;
// LAYOUT_BF16 reads the two planes and widens.
template <int D, int LAY>
__device__ inline f32x4 load4(const void *re, const void *im, int64_t row, int f) {
    if constexpr (LAY == LAYOUT_C64) {
        return *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(re) + row * (2 * D) + f);
    } else {
        const int64_t el = row * D + f / 2;
        const uint32_t r2 = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(re) + el);
        const uint32_t i2 = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(im) + el);
        return f32x4{bf_lo(r2), bf_lo(i2), bf_hi(r2), bf_hi(i2)};
    }
}

// LAYOUT_BF16 rounds to bf16 (nearest even) and writes the two planes.
template <int D, int LAY>
__device__ inline void store4(void *re, void *im, int64_t row, int f, f32x4 v) {
    if constexpr (LAY == LAYOUT_C64) {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(re) + row * (2 * D) + f) = v;
    } else {
        const int64_t el = row * D + f / 2;
        const f32x2 r = {v[0], v[2]}, i = {v[1], v[3]};
        *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(re) + el) =
            __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
        *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(im) + el) =
            __builtin_bit_cast(uint32_t, __builtin_convertvector(i, bf16x2));
    }
}

// Channel groups per row tile: two for Born at width 128 (its products per
// block amortise the score exchange); PCT there keeps one wave per SIMD.
constexpr int ch_of(int D, int OP) { return D >= 128 && OP == OP_BORN ? 2 : 1; }

// n floats from LDS with 16-byte reads
template <int N>
__device__ inline void lds_row(const float *p, float (&out)[N]) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(p + 4 * i);
        out[4 * i] = x[0];
        out[4 * i + 1] = x[1];
        out[4 * i + 2] = x[2];
        out[4 * i + 3] = x[3];
    }
}

// The run of NC floats NC j16 .. NC j16 + NC - 1 of a streamed LDS row as the
// gradient products' operand: out[4 p + e] is float 4 ((p + rho) mod NCK) + e
// of the run, rho = rho_of(j16).
template <class C>
__device__ inline int rho_of(int i) { return (i / C::RDIV + i / 8) % C::NCK; }
template <class C>
__device__ inline void lds_run(const float *rowp, int j16, float (&out)[C::NC]) {
    const float *run = rowp + C::NC * j16;
    const int rho = rho_of<C>(j16);
#pragma unroll
    for (int p = 0; p < C::NCK; ++p) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(run + 4 * ((p + rho) % C::NCK));
        out[4 * p] = x[0];
        out[4 * p + 1] = x[1];
        out[4 * p + 2] = x[2];
        out[4 * p + 3] = x[3];
    }
}

// Gradient tile c, register r of lane group g is row i = 4 g + r, real channel
// NC i + 4 ((c / 4 + rho_of(i)) mod NCK) + c mod 4: in the lane's quarter of
// the row, float own_idx = NC r + 4 m + c mod 4.
template <class C>
__device__ inline int run_rot(int g, int r) { return rho_of<C>(4 * g + r); }
// The owned operand's float at gradient tile c, register r, selected with
// compile-time indices (c and r unrolled) so that the array stays in registers.
template <class C>
__device__ inline float own_of(const float (&x)[C::KQ], int g, int c, int r) {
    const int m = ((c >> 2) + run_rot<C>(g, r)) % C::NCK;
    float v = x[C::NC * r + (c & 3)];
#pragma unroll
    for (int j = 1; j < C::NCK; ++j) v = m == j ? x[C::NC * r + 4 * j + (c & 3)] : v;
    return v;
}

// Workgroup -> (head, owned block).  The blocks of a head go to one XCD when
// BH % 8 == 0 (workgroups are dealt to the 8 XCDs in turn).  `heavy_last`:
// the query side, whose last blocks see the most keys under the causal mask,
// takes them first; the key side takes its first blocks first.
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

// Streamed rows: thread t stages row t / LPK, chunks t % LPK + LPK i of each
// operand, rotated by 7 chunks on odd rows: the 16 lanes of one LDS write,
// two rows, then cover every bank once.
template <int NCH, int LPK>
struct Stager {
    int row, sc, rot;
    __device__ Stager(int tid) : row(tid / LPK), sc(tid % LPK), rot(7 * ((tid / LPK) & 1)) {}
    __device__ int chunk(int i) const { return (sc + LPK * i + rot) % NCH; }
};

// CH > 1: the sum of value x over the waves of a row tile, through the
// exchange area (slot k of 12), the same in every wave of the tile; a
// workgroup barrier makes the partners' values visible and another frees the
// slot again (all waves reach both).
template <class C>
__device__ inline float tile_sum(float *xch, int wave, int lane, int k, float x) {
    const int w0 = wave - wave % C::CH;
    xch[(wave * 12 + k) * 64 + lane] = x;
    __syncthreads();
    float t = xch[(w0 * 12 + k) * 64 + lane];
#pragma unroll
    for (int c = 1; c < C::CH; ++c) t += xch[((w0 + c) * 12 + k) * 64 + lane];
    __syncthreads();
    return t;
}

// ------------------------------------------------------------------------------ per-query scalars (Born)
// 16 lanes per query row: 1 / l (0 for a zero denominator: O = 0, no gradient)
// and delta = Re(G^H O), as a float pair at index row of the dq buffer.
template <int D, int LAY>
__global__ __launch_bounds__(256) void bwd16_scal_kernel(BwdProblem p, int64_t rows) {
    using C = B16<D>;
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sp = threadIdx.x & 15;
    float dl = 0.f;
    constexpr int PER = C::KD / 16;   // floats of the row per lane
    if (row < rows) {
#pragma unroll
        for (int i = 0; i < PER / 4; ++i) {
            const f32x4 gg = load4<D, LAY>(p.g_re, p.g_im, row, PER * sp + 4 * i);
            const f32x4 o = load4<D, LAY>(p.o_re, p.o_im, row, PER * sp + 4 * i);
            dl += gg[0] * o[0] + gg[1] * o[1] + gg[2] * o[2] + gg[3] * o[3];
        }
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) dl += __shfl_xor(dl, o);
    if (sp == 0 && row < rows) {
        const float l = p.row_den[row];
        reinterpret_cast<f32x2 *>(p.dq_re)[row] = f32x2{l != 0.f ? 1.f / l : 0.f, dl};
    }
}

// ------------------------------------------------------------------------------ dK, dV
// DECAY (Born): every weight and D2 carries gamma^(query - key), one
// exponential per weight (the distance clamped at 0 where the mask zeroes it).
template <int D, int OP, int LAY, bool DECAY>
__global__ __launch_bounds__((B16<D, ch_of(D, OP)>::NT))
__attribute__((amdgpu_waves_per_eu((B16<D, ch_of(D, OP)>::WPE), (B16<D, ch_of(D, OP)>::WPE))))
void bwd16_dkdv_kernel(BwdProblem p, int nkb) {
    using C = B16<D, ch_of(D, OP)>;
    extern __shared__ __align__(16) float fsm[];
    constexpr bool born = OP == OP_BORN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j16 = lane & 15;
    const int g = lane >> 4;
    const int T = p.T;
    const int rt = wave / C::CH, hc = wave % C::CH;   // row tile, channel group
    const int cg0 = C::KDC * hc;                      // first real channel of the group
    float *xch = fsm + 2 * C::STAGE;                  // CH > 1: the exchange area

    int bh, kblk;
    map_block(p.BH, nkb, false, bh, kblk);
    const int kb0 = kblk * C::BM;
    const int64_t hrow = (int64_t)bh * T;   // this head's first row
    const float lg2 = DECAY ? p.decay.lg2[bh % p.H] : 0.f;

    // K', V' of this wave's 16 keys over the lane group's quarter of its channel group
    const int kt0 = kb0 + TR * rt;
    const int krow = kt0 + j16;
    float kre[C::KQ], vre[C::KQ];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < C::KQ / 4; ++i) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f}, v = x;
        if (krow < T) {
            x = load4<D, LAY>(p.k_re, p.k_im, hrow + krow, cg0 + g * C::KQ + 4 * i);
            v = load4<D, LAY>(p.v_re, p.v_im, hrow + krow, cg0 + g * C::KQ + 4 * i);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kre[4 * i + e] = x[e];
            vre[4 * i + e] = v[e];
            ss += x[e] * x[e];
        }
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if constexpr (C::CH > 1) ss = tile_sum<C>(xch, wave, lane, 0, ss);
    const float rk = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;   // PCT: 1 / ||k||
    const float sqd = sqrtf((float)D);

    f32x4 dk[C::NC], dv[C::NC];
#pragma unroll
    for (int c = 0; c < C::NC; ++c) dk[c] = dv[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // query stages: with the causal mask only queries >= this workgroup's first key
    const int qstart = p.causal ? kb0 : 0;
    const int nst = qstart < T ? (T - qstart + C::BN - 1) / C::BN : 0;
    const Stager<C::NCH, C::LPK> stg(tid);
    f32x4 qreg[C::CPT], greg[C::CPT];
    f32x2 tab = {0.f, 0.f};
    auto load_stage = [&](int q0) {
        const int qr = q0 + stg.row;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
            if (qr < T) {
                a = load4<D, LAY>(p.q_re, p.q_im, hrow + qr, 4 * stg.chunk(i));
                b = load4<D, LAY>(p.g_re, p.g_im, hrow + qr, 4 * stg.chunk(i));
            }
            qreg[i] = a;
            greg[i] = b;
        }
        if (born) {
            tab = f32x2{0.f, 0.f};
            if (stg.sc == 0 && qr < T) tab = reinterpret_cast<const f32x2 *>(p.dq_re)[hrow + qr];
        }
    };
    // per query: Born (1 / l, delta); PCT (1 / ||q||, unused)
    auto store_stage = [&](int buf) {
        float *qs = fsm + buf * C::STAGE;
        float *gs = qs + C::BN * C::ROW;
        float *sa = gs + C::BN * C::ROW;
        float *sb = sa + C::BN;
        float x2 = 0.f;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            *reinterpret_cast<f32x4 *>(qs + stg.row * C::ROW + 4 * stg.chunk(i)) = qreg[i];
            *reinterpret_cast<f32x4 *>(gs + stg.row * C::ROW + 4 * stg.chunk(i)) = greg[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) x2 += qreg[i][e] * qreg[i][e];
        }
        if (!born) {
#pragma unroll
            for (int o = 1; o < C::LPK; o <<= 1) x2 += __shfl_xor(x2, o);
        }
        if (stg.sc == 0) {
            if (born) {
                sa[stg.row] = tab[0];
                sb[stg.row] = tab[1];
            } else {
                sa[stg.row] = x2 > 0.f ? 1.f / sqrtf(x2) : 0.f;
                sb[stg.row] = 0.f;
            }
        }
    };
    if (nst > 0) {
        load_stage(qstart);
        store_stage(0);
    }
    __syncthreads();

    for (int st = 0; st < nst; ++st) {
        const int qb0s = qstart + st * C::BN;
        const int buf = st & 1;
        if (st + 1 < nst) load_stage(qb0s + C::BN);
#pragma unroll
        for (int sbk = 0; sbk < C::BN / 16; ++sbk) {   // every wave, every block: the mask zeroes queries before a lane's key
            const float *qs = fsm + buf * C::STAGE + 16 * sbk * C::ROW;
            const float *gs = fsm + buf * C::STAGE + C::BN * C::ROW + 16 * sbk * C::ROW;
            const float *sa = fsm + buf * C::STAGE + 2 * C::BN * C::ROW + 16 * sbk;
            const float *sb = sa + C::BN;
            const int qb0 = qb0s + 16 * sbk;
            // S, E for 16 queries x 16 keys: lane = key j16, registers = queries 4 g + r
            f32x4 sr = {0.f, 0.f, 0.f, 0.f}, si = sr, ev = sr;
#pragma unroll
            for (int p0 = 0; p0 < C::KQ; p0 += C::KP) {
                float qa[C::KP], ga[C::KP];
                lds_row<C::KP>(qs + j16 * C::ROW + cg0 + g * C::KQ + p0, qa);
                lds_row<C::KP>(gs + j16 * C::ROW + cg0 + g * C::KQ + p0, ga);
#pragma unroll
                for (int s = 0; s < C::KP; ++s) {
                    sr = mfma16(qa[s], kre[p0 + s], sr);
                    ev = mfma16(ga[s], vre[p0 + s], ev);
                    // Im <q, k> = sum_n q'''[n] k'[n] with q''' = (Im q0, -Re q0, ...): the sign
                    // and the swap on the streamed operand (a quarter starts on an even index)
                    if (born) si = mfma16((s & 1) ? -qa[s - 1] : qa[s + 1], kre[p0 + s], si);
                }
            }
            if constexpr (C::CH > 1) {   // the partial sums of the tile's channel groups
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    xch[(wave * 12 + r) * 64 + lane] = sr[r];
                    xch[(wave * 12 + 4 + r) * 64 + lane] = si[r];
                    xch[(wave * 12 + 8 + r) * 64 + lane] = ev[r];
                }
                __syncthreads();
                const int w0 = C::CH * rt;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sr[r] = xch[(w0 * 12 + r) * 64 + lane];
                    si[r] = xch[(w0 * 12 + 4 + r) * 64 + lane];
                    ev[r] = xch[(w0 * 12 + 8 + r) * 64 + lane];
#pragma unroll
                    for (int c = 1; c < C::CH; ++c) {
                        sr[r] += xch[((w0 + c) * 12 + r) * 64 + lane];
                        si[r] += xch[((w0 + c) * 12 + 4 + r) * 64 + lane];
                        ev[r] += xch[((w0 + c) * 12 + 8 + r) * 64 + lane];
                    }
                }
            }
            const f32x4 av = *reinterpret_cast<const f32x4 *>(sa + 4 * g);
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(sb + 4 * g);
            float wl[4], pr[4], pi[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int qi = 4 * g + r;
                const bool keep = (!p.causal || qb0 + qi >= krow) && qb0 + qi < T;
                if (born) {
                    const float w = sr[r] * sr[r] + si[r] * si[r];
                    const float f = DECAY ? decay_pow(lg2, max(qb0 + qi - krow, 0)) : 1.f;
                    wl[r] = keep ? w * av[r] * f : 0.f;
                    const float d2 = keep ? 2.f * (ev[r] - bv[r]) * av[r] * f : 0.f;
                    pr[r] = d2 * sr[r];
                    pi[r] = d2 * si[r];
                } else {
                    const float w = sigmoid(sr[r] * sqd * av[r] * rk + p.bias);
                    wl[r] = keep ? w : 0.f;
                    const float ds = keep ? ev[r] * w * (1.f - w) : 0.f;
                    pr[r] = sqd * ds * av[r];   // sqrt(d) ds qh on the raw query row
                    pi[r] = 0.f;
                }
            }
            // dV'^T += G'^T W, dK'^T += Q'^T Re P - Q''^T Im P; step t takes query 4 g + t
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float ga2[C::NC], qa2[C::NC];
                lds_run<C>(gs + (4 * g + t) * C::ROW + cg0, j16, ga2);
                lds_run<C>(qs + (4 * g + t) * C::ROW + cg0, j16, qa2);
#pragma unroll
                for (int c = 0; c < C::NC; ++c) {
                    dv[c] = mfma16(ga2[c], wl[t], dv[c]);
                    dk[c] = mfma16(qa2[c], pr[t], dk[c]);
                }
                if (born) {
                    // -q''[n]: q'[n + 1] on even n, -q'[n - 1] on odd n
                    const float npi = -pi[t];
#pragma unroll
                    for (int c = 0; c < C::NC; ++c) dk[c] = mfma16(qa2[c ^ 1], (c & 1) ? npi : pi[t], dk[c]);
                }
            }
        }
        if (st + 1 < nst) store_stage(buf ^ 1);
        __syncthreads();
    }

    // lane (key j16, group g), tile c, register r: the owned float own_of(kre, c, r)
    if (!born) {
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < C::NC; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) dot += dk[c][r] * own_of<C>(kre, g, c, r);
        dot += __shfl_xor(dot, 16);
        dot += __shfl_xor(dot, 32);
        if constexpr (C::CH > 1) dot = tile_sum<C>(xch, wave, lane, 0, dot);
        dot *= rk * rk;
#pragma unroll
        for (int c = 0; c < C::NC; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) dk[c][r] = (dk[c][r] - dot * own_of<C>(kre, g, c, r)) * rk;
    }
    if (krow >= T) return;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < C::NCK; ++q) {
            const int f = cg0 + g * C::KQ + C::NC * r + 4 * ((q + run_rot<C>(g, r)) % C::NCK);
            store4<D, LAY>(p.dk_re, p.dk_im, hrow + krow, f,
                        f32x4{dk[4 * q][r], dk[4 * q + 1][r], dk[4 * q + 2][r], dk[4 * q + 3][r]});
            store4<D, LAY>(p.dv_re, p.dv_im, hrow + krow, f,
                        f32x4{dv[4 * q][r], dv[4 * q + 1][r], dv[4 * q + 2][r], dv[4 * q + 3][r]});
        }
}

// ------------------------------------------------------------------------------ dQ (and db)
template <int D, int OP, int LAY, bool DECAY>
__global__ __launch_bounds__((B16<D, ch_of(D, OP)>::NT))
__attribute__((amdgpu_waves_per_eu((B16<D, ch_of(D, OP)>::WPE), (B16<D, ch_of(D, OP)>::WPE))))
void bwd16_dq_kernel(BwdProblem p, int nrb) {
    using C = B16<D, ch_of(D, OP)>;
    extern __shared__ __align__(16) float fsm[];
    constexpr bool born = OP == OP_BORN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j16 = lane & 15;
    const int g = lane >> 4;
    const int T = p.T;
    const int rt = wave / C::CH, hc = wave % C::CH;   // row tile, channel group
    const int cg0 = C::KDC * hc;                      // first real channel of the group
    float *xch = fsm + 2 * C::STAGE;                  // CH > 1: the exchange area

    int bh, rb;
    map_block(p.BH, nrb, true, bh, rb);
    const int m0 = rb * C::BM;
    const int64_t hrow = (int64_t)bh * T;
    const float lg2 = DECAY ? p.decay.lg2[bh % p.H] : 0.f;

    // Q', G' of this wave's 16 queries over the lane group's quarter of its channel group
    const int qt0 = m0 + TR * rt;
    const int qrow = qt0 + j16;
    float qre[C::KQ], gre[C::KQ];
    float dl = 0.f, ss = 0.f;
#pragma unroll
    for (int i = 0; i < C::KQ / 4; ++i) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f}, gg = x, o = x;
        if (qrow < T) {
            x = load4<D, LAY>(p.q_re, p.q_im, hrow + qrow, cg0 + g * C::KQ + 4 * i);
            gg = load4<D, LAY>(p.g_re, p.g_im, hrow + qrow, cg0 + g * C::KQ + 4 * i);
            if (born) o = load4<D, LAY>(p.o_re, p.o_im, hrow + qrow, cg0 + g * C::KQ + 4 * i);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qre[4 * i + e] = x[e];
            gre[4 * i + e] = gg[e];
            dl += gg[e] * o[e];   // Re(G^H O), this quarter's components
            ss += x[e] * x[e];
        }
    }
    dl += __shfl_xor(dl, 16);
    dl += __shfl_xor(dl, 32);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if constexpr (C::CH > 1) {
        dl = tile_sum<C>(xch, wave, lane, 0, dl);
        ss = tile_sum<C>(xch, wave, lane, 1, ss);
    }
    float inv_l = 0.f;   // Born: 1 / l (0 for a zero denominator: O = 0, no gradient)
    if (born && qrow < T) {
        const float l = p.row_den[hrow + qrow];
        inv_l = l != 0.f ? 1.f / l : 0.f;
    }
    const float iq = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;   // PCT: 1 / ||q|| (0 for a zero row)
    const float rq = sqrtf((float)D) * iq;

    f32x4 dq[C::NC];
#pragma unroll
    for (int c = 0; c < C::NC; ++c) dq[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dsum = 0.f;

    const int kend = p.causal ? min(T, m0 + C::BM) : T;
    const int nst = (kend + C::BN - 1) / C::BN;
    const Stager<C::NCH, C::LPK> stg(tid);
    f32x4 kreg[C::CPT], vreg[C::CPT];
    auto load_stage = [&](int k0) {
        const int kr = k0 + stg.row;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
            if (kr < T) {
                a = load4<D, LAY>(p.k_re, p.k_im, hrow + kr, 4 * stg.chunk(i));
                b = load4<D, LAY>(p.v_re, p.v_im, hrow + kr, 4 * stg.chunk(i));
            }
            kreg[i] = a;
            vreg[i] = b;
        }
    };
    auto store_stage = [&](int buf) {
        float *ks = fsm + buf * C::STAGE;
        float *vs = ks + C::BN * C::ROW;
        float *rks = vs + C::BN * C::ROW;
        float s2 = 0.f;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            *reinterpret_cast<f32x4 *>(ks + stg.row * C::ROW + 4 * stg.chunk(i)) = kreg[i];
            *reinterpret_cast<f32x4 *>(vs + stg.row * C::ROW + 4 * stg.chunk(i)) = vreg[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) s2 += kreg[i][e] * kreg[i][e];
        }
        if (!born) {
#pragma unroll
            for (int o = 1; o < C::LPK; o <<= 1) s2 += __shfl_xor(s2, o);
            if (stg.sc == 0) rks[stg.row] = s2 > 0.f ? 1.f / sqrtf(s2) : 0.f;
        }
    };
    if (nst > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();

    for (int st = 0; st < nst; ++st) {
        const int kb0s = st * C::BN;
        const int buf = st & 1;
        if (st + 1 < nst) load_stage(kb0s + C::BN);
#pragma unroll
        for (int sbk = 0; sbk < C::BN / 16; ++sbk) {   // every wave, every block: the mask zeroes keys past a lane's query
            const float *ks = fsm + buf * C::STAGE + 16 * sbk * C::ROW;
            const float *vs = fsm + buf * C::STAGE + C::BN * C::ROW + 16 * sbk * C::ROW;
            const float *rks = fsm + buf * C::STAGE + 2 * C::BN * C::ROW + 16 * sbk;
            const int kb0 = kb0s + 16 * sbk;
            // S^T, E^T for 16 keys x 16 queries: lane = query j16, registers = keys 4 g + r
            f32x4 sr = {0.f, 0.f, 0.f, 0.f}, si = sr, ev = sr;
#pragma unroll
            for (int p0 = 0; p0 < C::KQ; p0 += C::KP) {
                float ka[C::KP], va[C::KP];
                lds_row<C::KP>(ks + j16 * C::ROW + cg0 + g * C::KQ + p0, ka);
                lds_row<C::KP>(vs + j16 * C::ROW + cg0 + g * C::KQ + p0, va);
#pragma unroll
                for (int s = 0; s < C::KP; ++s) {
                    sr = mfma16(ka[s], qre[p0 + s], sr);
                    ev = mfma16(va[s], gre[p0 + s], ev);
                    // Im <q, k> = sum_n k''[n] q'[n] with k'' = (-Im k0, Re k0, ...): the sign and
                    // the swap on the streamed operand
                    if (born) si = mfma16((s & 1) ? ka[s - 1] : -ka[s + 1], qre[p0 + s], si);
                }
            }
            if constexpr (C::CH > 1) {   // the partial sums of the tile's channel groups
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    xch[(wave * 12 + r) * 64 + lane] = sr[r];
                    xch[(wave * 12 + 4 + r) * 64 + lane] = si[r];
                    xch[(wave * 12 + 8 + r) * 64 + lane] = ev[r];
                }
                __syncthreads();
                const int w0 = C::CH * rt;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sr[r] = xch[(w0 * 12 + r) * 64 + lane];
                    si[r] = xch[(w0 * 12 + 4 + r) * 64 + lane];
                    ev[r] = xch[(w0 * 12 + 8 + r) * 64 + lane];
#pragma unroll
                    for (int c = 1; c < C::CH; ++c) {
                        sr[r] += xch[((w0 + c) * 12 + r) * 64 + lane];
                        si[r] += xch[((w0 + c) * 12 + 4 + r) * 64 + lane];
                        ev[r] += xch[((w0 + c) * 12 + 8 + r) * 64 + lane];
                    }
                }
            }
            f32x4 rkv = {0.f, 0.f, 0.f, 0.f};
            if (!born) rkv = *reinterpret_cast<const f32x4 *>(rks + 4 * g);
            float pr[4], pi[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = 4 * g + r;
                const bool keep = (!p.causal || kb0 + key <= qrow) && kb0 + key < T;
                if (born) {
                    float d2 = keep ? 2.f * (ev[r] - dl) * inv_l : 0.f;
                    if (DECAY) d2 *= decay_pow(lg2, max(qrow - (kb0 + key), 0));
                    pr[r] = d2 * sr[r];
                    pi[r] = d2 * si[r];
                } else {
                    const float w = sigmoid(sr[r] * rq * rkv[r] + p.bias);
                    const float ds = keep ? ev[r] * w * (1.f - w) : 0.f;
                    dsum += ds;
                    pr[r] = ds * rkv[r];   // ds kh on the raw key row
                    pi[r] = 0.f;
                }
            }
            // dQ'^T += K'^T Re P^T + K''^T Im P^T; step t takes key 4 g + t
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float a[C::NC];
                lds_run<C>(ks + (4 * g + t) * C::ROW + cg0, j16, a);
#pragma unroll
                for (int c = 0; c < C::NC; ++c) dq[c] = mfma16(a[c], pr[t], dq[c]);
                if (born) {
                    // k''[n]: -k'[n + 1] on even n, k'[n - 1] on odd n
                    const float npi = -pi[t];
#pragma unroll
                    for (int c = 0; c < C::NC; ++c) dq[c] = mfma16(a[c ^ 1], (c & 1) ? pi[t] : npi, dq[c]);
                }
            }
        }
        if (st + 1 < nst) store_stage(buf ^ 1);
        __syncthreads();
    }

    // lane (query j16, group g), tile c, register r: the owned float own_of(qre, c, r)
    if (!born) {
        const float sq = sqrtf((float)D);
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < C::NC; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dq[c][r] *= sq;
                dot += dq[c][r] * own_of<C>(qre, g, c, r);
            }
        dot += __shfl_xor(dot, 16);
        dot += __shfl_xor(dot, 32);
        if constexpr (C::CH > 1) dot = tile_sum<C>(xch, wave, lane, 0, dot);
        dot *= iq * iq;
#pragma unroll
        for (int c = 0; c < C::NC; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) dq[c][r] = (dq[c][r] - dot * own_of<C>(qre, g, c, r)) * iq;
        float db = dsum + __shfl_xor(dsum, 16);
        db += __shfl_xor(db, 32);
        if (p.db_rows && g == 0 && hc == 0 && qrow < T) p.db_rows[hrow + qrow] = db;
    }
    if (qrow >= T) return;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < C::NCK; ++q)
            store4<D, LAY>(p.dq_re, p.dq_im, hrow + qrow, cg0 + g * C::KQ + C::NC * r + 4 * ((q + run_rot<C>(g, r)) % C::NCK),
                        f32x4{dq[4 * q][r], dq[4 * q + 1][r], dq[4 * q + 2][r], dq[4 * q + 3][r]});
}

template <int D, int OP, int LAY, bool DECAY = false>
hipError_t launch_cfg(const BwdProblem &p) {
    using C = B16<D, ch_of(D, OP)>;
    static std::atomic<uint64_t> dq_set{0}, kv_set{0};
    const int nblk = (p.T + C::BM - 1) / C::BM;
    const int64_t blocks = (int64_t)p.BH * nblk;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    auto kkv = bwd16_dkdv_kernel<D, OP, LAY, DECAY>;
    auto kdq = bwd16_dq_kernel<D, OP, LAY, DECAY>;
    hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kkv), C::LDS_BYTES, kv_set);
    if (e != hipSuccess) return e;
    e = set_dynamic_lds(reinterpret_cast<const void *>(kdq), C::LDS_BYTES, dq_set);
    if (e != hipSuccess) return e;
    if (OP == OP_BORN) {
        const int64_t rows = (int64_t)p.BH * p.T;
        const int64_t sblocks = (rows + 15) / 16;
        if (sblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((bwd16_scal_kernel<D, LAY>), dim3((unsigned)sblocks), dim3(256), 0, p.stream, p, rows);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kkv, dim3((unsigned)blocks), dim3(C::NT), C::LDS_BYTES, p.stream, p, nblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kdq, dim3((unsigned)blocks), dim3(C::NT), C::LDS_BYTES, p.stream, p, nblk);
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

bool supports_bwd_f32_mfma16(const BwdProblem &p) {
    return (p.op == OP_BORN || p.op == OP_PCT) && (p.d == 32 || p.d == 64 || p.d == 128);
}

hipError_t launch_bwd_f32_mfma16(const BwdProblem &p) {
    switch (p.d) {
        case 32: return launch_d<32>(p);
        case 64: return launch_d<64>(p);
        default: return launch_d<128>(p);
    }
}

}  // namespace cattn
