// Carried-state Born attention on gfx950 matrix cores, bf16 real/imag planes,
// head width 64 ("Show HN: CNET", BornAttention's linear mode: the key lifted
// to its outer product, a running state; "The Quantum Shortcut", section 2:
// the Born rule q^H rho q as a linear functional of rho = k k^H).
//
// Readout of the packed state (the merge of an incoming state into a causal
// forward): with the real features phi(q) of a token (d^2 = 4096 of them) and
// the packed state S[n][f] (2d + 1 = 129 matrices),
//     R[t][n] = sum_f psi_f(q_t) S[n][f],   psi = phi times 1 (diagonal) or 2,
// a real product [129 x 4096] x [4096 x T] per head, on v_mfma_f32_32x32x16_bf16
// with fp32 accumulation.  MFMA rows are the state matrices (five tiles of 32:
// Re V, Im V, and Z with zero rows), columns are tokens, the reduction runs
// over features.  The state operand is staged per feature row a (64 features)
// from fp32 to bf16 in LDS, the factor 2 of off-diagonal features folded in
// (exact).  The token operand is formed in registers: lane (token t, half h)
// holds the (Re, Im) bf16 pairs of the 32 channels b = 16 m + 8 h + e it ever
// needs, and per feature row a one pair q_a from LDS; each feature is one
// v_dot2_f32_bf16:
//     phi_ab = Re(q_a conj q_b) = dot((Re q_a, Im q_a), (Re q_b, Im q_b))   (a <= b)
//            = Im(q_b conj q_a) = dot((-Im q_a, Re q_a), (Re q_b, Im q_b))  (a > b).
// Workgroup: 4 waves, 64 tokens per wave (two column tiles), one head.
//
// State build: S[n][f] (+)= sum_j W[j][n] phi_f(k_j) with W[j] = (Re V[j],
// Im V[j], 1), a real product [129 x T] x [T x 4096] per head.  MFMA rows are
// the state matrices (the Z tile takes a constant operand: ones in row 128),
// columns are features, the reduction runs over tokens.  Per 64-token stage
// the values are staged transposed (VT[n][token], bf16) and the keys as
// transposed (Re, Im) pairs (KT[channel][token]), with the rotated pairs
// (-Im, Re) of the workgroup's four feature rows for the features below the
// diagonal.  Workgroup: 4 waves, wave w owns feature row a = 4 g + w (64
// features, two column tiles).
#include "cattn_internal.h"

namespace cattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 64;
constexpr int NM = 2 * D + 1;           // packed matrices per head
constexpr int NW = 4;                   // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int TPW = 2;                  // 32-token column tiles per wave
constexpr int TOK = 32 * TPW * NW;      // tokens per workgroup
constexpr int NTILE = 5;                // 32-row tiles of state matrices (129 rows used)
constexpr int SROW = 72;                // bf16 per staged state row (64 + 8: conflict-free 16-byte reads)
constexpr int QROW = D + 1;             // dwords per staged token row
constexpr int SLOADS = (NM * D / 4 + NT - 1) / NT;   // float4 state loads per thread per feature row

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ inline float dot2(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), 0.f, false);
}

// (Re, Im) -> (-Im, Re) on a bf16 pair (low half Re)
__device__ inline uint32_t rot_pair(uint32_t x) { return ((x >> 16) | (x << 16)) ^ 0x8000u; }

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(NT) void born_merge_bf16_d64_kernel(LinearProblem p, int ntile_t) {
    __shared__ __align__(16) uint16_t Sb[2][NM][SROW];   // staged state rows (bf16), double buffered
    __shared__ uint32_t Qs[TOK][QROW];                   // (Re, Im) bf16 pairs of the tile's tokens

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int T = p.T;

    // blocks of one head on one XCD (workgroups are dealt to the 8 XCDs in turn)
    const int nblk = gridDim.x;
    const int x = blockIdx.x;
    const int lin = (nblk % 8 == 0) ? (x % 8) * (nblk / 8) + x / 8 : x;
    const int64_t bh = lin / ntile_t;
    const int t0 = (lin % ntile_t) * TOK;
    const int64_t base = bh * (int64_t)T * D;
    const float *S = p.S + bh * (int64_t)NM * D * D;
    const uint16_t *qre = reinterpret_cast<const uint16_t *>(p.q_re);
    const uint16_t *qim = reinterpret_cast<const uint16_t *>(p.q_im);

    // ---- stage the tile's queries as (Re, Im) pairs; rows past T are zero
    for (int i = tid; i < TOK * (D / 8); i += NT) {
        const int r = i / (D / 8), c8 = (i % (D / 8)) * 8;
        u32x4 re = {0, 0, 0, 0}, im = {0, 0, 0, 0};
        if (t0 + r < T) {
            re = *reinterpret_cast<const u32x4 *>(qre + base + (int64_t)(t0 + r) * D + c8);
            im = *reinterpret_cast<const u32x4 *>(qim + base + (int64_t)(t0 + r) * D + c8);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            Qs[r][c8 + 2 * e] = (re[e] & 0xffffu) | (im[e] << 16);
            Qs[r][c8 + 2 * e + 1] = (re[e] >> 16) | (im[e] & 0xffff0000u);
        }
    }

    // ---- state staging: feature row a of all 129 matrices, fp32 -> bf16, x2 off the diagonal
    float4 sreg[SLOADS];
    auto load_rows = [&](int a) {
#pragma unroll
        for (int i = 0; i < SLOADS; ++i) {
            const int idx = tid + i * NT;
            if (idx < NM * D / 4) {
                const int n = idx / (D / 4), q4 = idx % (D / 4);
                sreg[i] = *reinterpret_cast<const float4 *>(S + ((int64_t)n * D + a) * D + 4 * q4);
            }
        }
    };
    auto store_rows = [&](int a, int buf) {
#pragma unroll
        for (int i = 0; i < SLOADS; ++i) {
            const int idx = tid + i * NT;
            if (idx < NM * D / 4) {
                const int n = idx / (D / 4), q4 = idx % (D / 4);
                const int b = 4 * q4;
                const float4 v = sreg[i];
                const float w0 = b + 0 == a ? 1.f : 2.f, w1 = b + 1 == a ? 1.f : 2.f;
                const float w2 = b + 2 == a ? 1.f : 2.f, w3 = b + 3 == a ? 1.f : 2.f;
                uint2 pk;
                pk.x = pack_bf16x2(v.x * w0, v.y * w1);
                pk.y = pack_bf16x2(v.z * w2, v.w * w3);
                *reinterpret_cast<uint2 *>(&Sb[buf][n][b]) = pk;
            }
        }
    };
    load_rows(0);
    store_rows(0, 0);
    __syncthreads();

    // ---- this lane's token pairs for the channels b = 16 m + 8 h + e
    int tl[TPW];
    uint32_t qb[TPW][32];
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
        tl[s] = 64 * wave + 32 * s + l32;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) qb[s][8 * m + e] = Qs[tl[s]][16 * m + 8 * h + e];
    }

    f32x16 acc[TPW][NTILE];
#pragma unroll
    for (int s = 0; s < TPW; ++s)
#pragma unroll
        for (int ti = 0; ti < NTILE; ++ti)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[s][ti][r] = 0.f;

    const u32x4 zero4 = {0, 0, 0, 0};
    for (int a = 0; a < D; ++a) {
        const int buf = a & 1;
        if (a + 1 < D) load_rows(a + 1);
        uint32_t qa[TPW], qr[TPW];
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            qa[s] = Qs[tl[s]][a];
            qr[s] = rot_pair(qa[s]);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // state operand: rows 32 ti + l32, features 16 m + 8 h .. + 7 of row a
            bf16x8 sa[NTILE];
#pragma unroll
            for (int ti = 0; ti < NTILE - 1; ++ti)
                sa[ti] = *reinterpret_cast<const bf16x8 *>(&Sb[buf][32 * ti + l32][16 * m + 8 * h]);
            sa[NTILE - 1] = l32 == 0 ? *reinterpret_cast<const bf16x8 *>(&Sb[buf][2 * D][16 * m + 8 * h])
                                     : as_bf16x8(zero4);
            const int b0 = 16 * m + 8 * h;   // this lane's first channel of the step
#pragma unroll
            for (int s = 0; s < TPW; ++s) {
                uint32_t pk[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const uint32_t x0 = a <= b0 + e ? qa[s] : qr[s];
                    const uint32_t x1 = a <= b0 + e + 1 ? qa[s] : qr[s];
                    pk[e >> 1] = pack_bf16x2(dot2(x0, qb[s][8 * m + e]), dot2(x1, qb[s][8 * m + e + 1]));
                }
                const bf16x8 fq = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
                for (int ti = 0; ti < NTILE; ++ti) acc[s][ti] = mfma(sa[ti], fq, acc[s][ti]);
            }
        }
        if (a + 1 < D) store_rows(a + 1, buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane (token, half h) holds rows n = 32 ti + 8 (r / 4) + 4 h + r % 4
    uint16_t *ore = reinterpret_cast<uint16_t *>(p.o_re);
    uint16_t *oim = reinterpret_cast<uint16_t *>(p.o_im);
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
        // q^H Z q is row 128: tile 4, register 0, lanes of half 0
        const float den_h0 = acc[s][NTILE - 1][0];
        const float den = __shfl(den_h0, l32);
        const int tq = t0 + tl[s];
        if (tq >= T) continue;
        const int64_t rowi = bh * (int64_t)T + tq;
        const float l = p.row_den[rowi];
        const float Dn = l + den;
        const float inv = Dn != 0.f ? 1.f / Dn : 0.f;
        const int64_t ob = base + (int64_t)tq * D;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = 32 * ti + 8 * g + 4 * h;   // four consecutive channels
                const uint2 ur = *reinterpret_cast<const uint2 *>(ore + ob + c0);
                const uint2 ui = *reinterpret_cast<const uint2 *>(oim + ob + c0);
                const uint32_t wr[2] = {ur.x, ur.y}, wi[2] = {ui.x, ui.y};
                float vr[4], vi[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float o_r = __uint_as_float((e & 1 ? wr[e >> 1] >> 16 : wr[e >> 1] & 0xffffu) << 16);
                    const float o_i = __uint_as_float((e & 1 ? wi[e >> 1] >> 16 : wi[e >> 1] & 0xffffu) << 16);
                    vr[e] = (o_r * l + acc[s][ti][4 * g + e]) * inv;
                    vi[e] = (o_i * l + acc[s][ti + 2][4 * g + e]) * inv;
                }
                *reinterpret_cast<uint2 *>(ore + ob + c0) = make_uint2(pack_bf16x2(vr[0], vr[1]), pack_bf16x2(vr[2], vr[3]));
                *reinterpret_cast<uint2 *>(oim + ob + c0) = make_uint2(pack_bf16x2(vi[0], vi[1]), pack_bf16x2(vi[2], vi[3]));
            }
        if (h == 0) p.row_den[rowi] = Dn;
    }
}

constexpr int ST_TOK = 64;               // tokens per stage
constexpr int KROW = ST_TOK + 4;         // dwords per staged key row (16-byte aligned, offset banks)
constexpr int VROW = ST_TOK + 8;         // bf16 per staged value row
constexpr int ROWS_PER_WG = NW;          // feature rows per workgroup

struct StateStage {
    uint32_t KT[D][KROW];                // (Re k, Im k) pairs, [channel][token]
    uint32_t KR[ROWS_PER_WG][KROW];      // (-Im k, Re k) of this workgroup's feature rows
    uint16_t VT[2 * D][VROW];            // Re V channels then Im V channels, [n][token]
};

__global__ __launch_bounds__(NT) void born_state_bf16_d64_kernel(LinearProblem p) {
    __shared__ __align__(16) StateStage st[2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int T = p.T;
    constexpr int GROUPS = D / ROWS_PER_WG;   // workgroups per head

    const int nblk = gridDim.x;
    const int x = blockIdx.x;
    const int lin = (nblk % 8 == 0) ? (x % 8) * (nblk / 8) + x / 8 : x;
    const int64_t bh = lin / GROUPS;
    const int a0 = (lin % GROUPS) * ROWS_PER_WG;
    const int a = a0 + wave;                  // this wave's feature row
    const int64_t base = bh * (int64_t)T * D;
    const uint16_t *kre = reinterpret_cast<const uint16_t *>(p.k_re);
    const uint16_t *kim = reinterpret_cast<const uint16_t *>(p.k_im);
    const uint16_t *vre = reinterpret_cast<const uint16_t *>(p.v_re);
    const uint16_t *vim = reinterpret_cast<const uint16_t *>(p.v_im);

    // staging: thread -> (token, 8-channel group); two K groups and four V groups per stage
    u32x4 kr_reg[2], ki_reg[2], v_reg[4];
    auto load_stage = [&](int t0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int g = tid + i * NT;                 // 512 (token, channel group) of K
            const int r = g / (D / 8), c8 = (g % (D / 8)) * 8;
            kr_reg[i] = ki_reg[i] = u32x4{0, 0, 0, 0};
            if (t0 + r < T) {
                kr_reg[i] = *reinterpret_cast<const u32x4 *>(kre + base + (int64_t)(t0 + r) * D + c8);
                ki_reg[i] = *reinterpret_cast<const u32x4 *>(kim + base + (int64_t)(t0 + r) * D + c8);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = tid + i * NT;                 // 1024 (plane, token, channel group) of V
            const int pl = g / (ST_TOK * D / 8), rem = g % (ST_TOK * D / 8);
            const int r = rem / (D / 8), c8 = (rem % (D / 8)) * 8;
            v_reg[i] = u32x4{0, 0, 0, 0};
            if (t0 + r < T)
                v_reg[i] = *reinterpret_cast<const u32x4 *>((pl ? vim : vre) + base + (int64_t)(t0 + r) * D + c8);
        }
    };
    auto store_stage = [&](StateStage &S_) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int g = tid + i * NT;
            const int r = g / (D / 8), c8 = (g % (D / 8)) * 8;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t p0 = (kr_reg[i][e] & 0xffffu) | (ki_reg[i][e] << 16);
                const uint32_t p1 = (kr_reg[i][e] >> 16) | (ki_reg[i][e] & 0xffff0000u);
                S_.KT[c8 + 2 * e][r] = p0;
                S_.KT[c8 + 2 * e + 1][r] = p1;
                const int c0 = c8 + 2 * e - a0;
                if (c0 >= 0 && c0 < ROWS_PER_WG) S_.KR[c0][r] = rot_pair(p0);
                if (c0 + 1 >= 0 && c0 + 1 < ROWS_PER_WG) S_.KR[c0 + 1][r] = rot_pair(p1);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = tid + i * NT;
            const int pl = g / (ST_TOK * D / 8), rem = g % (ST_TOK * D / 8);
            const int r = rem / (D / 8), c8 = (rem % (D / 8)) * 8;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S_.VT[pl * D + c8 + 2 * e][r] = (uint16_t)(v_reg[i][e] & 0xffffu);
                S_.VT[pl * D + c8 + 2 * e + 1][r] = (uint16_t)(v_reg[i][e] >> 16);
            }
        }
    };

    f32x16 acc[2][NTILE];
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int ti = 0; ti < NTILE; ++ti)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ft][ti][r] = 0.f;

    // the Z tile's row operand: ones in row 128 (lane 0 of each half), zero elsewhere
    const uint32_t one2 = 0x3f803f80u;
    const bf16x8 zrow = l32 == 0 ? as_bf16x8(u32x4{one2, one2, one2, one2}) : as_bf16x8(u32x4{0, 0, 0, 0});
    // features of column tile ft: (a, b = 32 ft + l32); on or above the diagonal reads KT[a], below KR
    bool upper[2];
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) upper[ft] = a <= 32 * ft + l32;

    const int nst = (T + ST_TOK - 1) / ST_TOK;
    if (nst > 0) {
        load_stage(0);
        store_stage(st[0]);
    }
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        StateStage &cur = st[s & 1];
        if (s + 1 < nst) load_stage((s + 1) * ST_TOK);
#pragma unroll
        for (int ks = 0; ks < ST_TOK / 16; ++ks) {
            const int tk = 16 * ks + 8 * h;   // this lane's first token of the step
            bf16x8 wa[NTILE];
#pragma unroll
            for (int ti = 0; ti < NTILE - 1; ++ti)
                wa[ti] = *reinterpret_cast<const bf16x8 *>(&cur.VT[32 * ti + l32][tk]);
            wa[NTILE - 1] = zrow;
            const u32x4 ka0 = *reinterpret_cast<const u32x4 *>(&cur.KT[a][tk]);
            const u32x4 ka1 = *reinterpret_cast<const u32x4 *>(&cur.KT[a][tk + 4]);
            const u32x4 kq0 = *reinterpret_cast<const u32x4 *>(&cur.KR[wave][tk]);
            const u32x4 kq1 = *reinterpret_cast<const u32x4 *>(&cur.KR[wave][tk + 4]);
#pragma unroll
            for (int ft = 0; ft < 2; ++ft) {
                const int b = 32 * ft + l32;
                const u32x4 kb0 = *reinterpret_cast<const u32x4 *>(&cur.KT[b][tk]);
                const u32x4 kb1 = *reinterpret_cast<const u32x4 *>(&cur.KT[b][tk + 4]);
                const u32x4 x0 = upper[ft] ? ka0 : kq0, x1 = upper[ft] ? ka1 : kq1;
                uint32_t pk[4];
                pk[0] = pack_bf16x2(dot2(x0[0], kb0[0]), dot2(x0[1], kb0[1]));
                pk[1] = pack_bf16x2(dot2(x0[2], kb0[2]), dot2(x0[3], kb0[3]));
                pk[2] = pack_bf16x2(dot2(x1[0], kb1[0]), dot2(x1[1], kb1[1]));
                pk[3] = pack_bf16x2(dot2(x1[2], kb1[2]), dot2(x1[3], kb1[3]));
                const bf16x8 fk = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
                for (int ti = 0; ti < NTILE; ++ti) acc[ft][ti] = mfma(wa[ti], fk, acc[ft][ti]);
            }
        }
        if (s + 1 < nst) store_stage(st[(s + 1) & 1]);
        __syncthreads();
    }

    // write S[n][a * 64 + b]: lane (column b = 32 ft + l32, half h) holds rows n = 32 ti + 8 (r / 4) + 4 h + r % 4
    float *Sh = p.S + bh * (int64_t)NM * D * D;
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int ti = 0; ti < NTILE; ++ti)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = 32 * ti + 8 * (r >> 2) + 4 * h + (r & 3);
                if (n >= NM) continue;
                float *dst = Sh + ((int64_t)n * D + a) * D + 32 * ft + l32;
                *dst = p.accumulate ? *dst + acc[ft][ti][r] : acc[ft][ti][r];
            }
}

}  // namespace

bool supports_born_linear_bf16_d64(const LinearProblem &p) {
    return p.layout == LAYOUT_BF16 && p.d == D;
}

hipError_t launch_born_merge_bf16_d64(const LinearProblem &p) {
    const int ntile_t = (p.T + TOK - 1) / TOK;
    const int64_t blocks = (int64_t)p.BH * ntile_t;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(born_merge_bf16_d64_kernel, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p, ntile_t);
    return hipGetLastError();
}

}  // namespace cattn

namespace cattn {

hipError_t launch_born_state_bf16_d64(const LinearProblem &p) {
    const int64_t blocks = (int64_t)p.BH * (D / ROWS_PER_WG);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(born_state_bf16_d64_kernel, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p);
    return hipGetLastError();
}

}  // namespace cattn
