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
// from fp32 to bf16 in LDS; the factor 2 of off-diagonal features is put on
// the token side (the doubled pairs of q_b, the diagonal feature halved).  The token operand is formed in registers: lane (token t, half h)
// holds the (Re, Im) bf16 pairs of the 32 channels b = 16 m + 8 h + e it ever
// needs, and per feature row a one pair q_a from LDS; each feature is one
// v_dot2_f32_bf16:
//     phi_ab = Re(q_a conj q_b) = dot((Re q_a, Im q_a), (Re q_b, Im q_b))   (a <= b)
//            = Im(q_b conj q_a) = dot((-Im q_a, Re q_a), (Re q_b, Im q_b))  (a > b).
// Workgroup: 8 waves (two per SIMD, so one wave's feature formation overlaps
// the other's matrix products), 32 tokens per wave, one head.
//
// State build: S[n][f] (+)= sum_j W[j][n] phi_f(k_j) with W[j] = (Re V[j],
// Im V[j], 1), a real product [129 x T] x [T x 4096] per head.  The value
// rows (Re V, Im V: four tiles of 32) run on matrix cores, MFMA rows the state
// matrices, columns the features, the reduction over tokens; the Z row (the
// plain sum of the features over tokens) is summed per lane from the fp32
// features.  Per 64-token stage the key and value planes are copied
// token-major into LDS (LDS-direct loads, no registers) and read through the
// transposing LDS read: the values as the row operand, the keys so that lane
// l32 receives channel b of its eight tokens, whose (Re, Im) pairs two byte
// permutes form.  The pairs of the workgroup's four feature rows, and their
// rotations (-Im, Re) for the features below the diagonal, are staged
// [row][token] through one wave's registers.  Workgroup: feature rows
// 4 g .. 4 g + 3 of one head (256 features), 8 waves in two token groups of
// four: wave w of a group owns the two rows 4 g + 2 (w / 2) + {0, 1} over the
// column tile w % 2 (32 features each), so the key pairs of its columns are
// formed once per token step for both rows.  The even stages go to group 0
// and the odd ones to group 1, so two waves share each SIMD and hide each
// other's operand latency; at the end each group finishes half the state
// rows, adding the other group's partial sums through LDS in a fixed order.
//
// Decay (per head gamma): the state build weighs token t of T by
// gamma^(T-1-t) on the feature operand (a per-stage table of the 64 token
// factors in LDS; an instance of its own) and an accumulated state by
// gamma^T; the merge counts the incoming state gamma^(t+1) at token t.
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
constexpr int NW = 4;                   // waves per workgroup (state build)
constexpr int NT = 64 * NW;
constexpr int MNW = 8;                  // waves per workgroup (readout): two per SIMD
constexpr int MNT = 64 * MNW;
constexpr int TPW = 1;                  // 32-token column tiles per wave (readout)
constexpr int TOK = 32 * TPW * MNW;     // tokens per workgroup (readout)
constexpr int NTILE = 5;                // 32-row tiles of state matrices (129 rows used)
constexpr int SROW = 72;                // bf16 per staged state row (64 + 8: conflict-free 16-byte reads)
constexpr int QROW = D + 1;             // dwords per staged token row
constexpr int SLOADS = (NM * D / 4 + MNT - 1) / MNT;   // float4 state loads per thread per feature row

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

__global__ __launch_bounds__(MNT) void born_merge_bf16_d64_kernel(LinearProblem p, int ntile_t) {
    // staged state rows (bf16), double buffered; rows NM .. 32 NTILE - 1 stay zero, so
    // the Z tile (row 128 and 31 zero rows) is read like the others
    __shared__ __align__(16) uint16_t Sb[2][32 * NTILE][SROW];
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

    for (int i = tid; i < 2 * (32 * NTILE - NM) * (SROW / 2); i += MNT) {
        const int b = i / ((32 * NTILE - NM) * (SROW / 2)), j = i % ((32 * NTILE - NM) * (SROW / 2));
        reinterpret_cast<uint32_t *>(&Sb[b][NM][0])[j] = 0u;
    }
    // ---- stage the tile's queries as (Re, Im) pairs; rows past T are zero
    for (int i = tid; i < TOK * (D / 8); i += MNT) {
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

    // ---- state staging: feature row a of all 129 matrices, fp32 -> bf16.  Rows
    // are loaded two iterations ahead into alternating register sets (row r in
    // set r % 2), so a row's load latency spans two feature rows of products.
    float4 sreg0[SLOADS], sreg1[SLOADS];
    // 2064 float4 per row: four full passes of the workgroup and a 16-thread tail
    static_assert(NM * D / 4 == (SLOADS - 1) * MNT + 16, "state row split");
    auto load_rows = [&](int a, float4 (&sreg)[SLOADS]) {
#pragma unroll
        for (int i = 0; i < SLOADS; ++i) {
            const int idx = tid + i * MNT;
            const int n = idx / (D / 4), q4 = idx % (D / 4);
            if (i < SLOADS - 1 || tid < 16)
                sreg[i] = *reinterpret_cast<const float4 *>(S + ((int64_t)n * D + a) * D + 4 * q4);
        }
    };
    auto store_rows = [&](int buf, const float4 (&sreg)[SLOADS]) {
#pragma unroll
        for (int i = 0; i < SLOADS; ++i) {
            const int idx = tid + i * MNT;
            const int n = idx / (D / 4), q4 = idx % (D / 4);
            const float4 v = sreg[i];
            uint2 pk;
            pk.x = pack_bf16x2(v.x, v.y);
            pk.y = pack_bf16x2(v.z, v.w);
            if (i < SLOADS - 1 || tid < 16) *reinterpret_cast<uint2 *>(&Sb[buf][n][4 * q4]) = pk;
        }
    };
    load_rows(0, sreg0);
    store_rows(0, sreg0);
    load_rows(1, sreg1);
    __syncthreads();

    // ---- this lane's token pairs for the channels b = 16 m + 8 h + e, doubled by
    // one on the exponent (psi = 2 phi off the diagonal; exact for normal values;
    // zero, subnormal, infinite and NaN halves are left as they are)
    int tl[TPW];
    uint32_t qb[TPW][32];
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
        tl[s] = 32 * TPW * wave + 32 * s + l32;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t x = Qs[tl[s]][16 * m + 8 * h + e];
                const uint32_t lo = x & 0x7f80u, hi = x & 0x7f800000u;   // exponent fields
                qb[s][8 * m + e] = x + (lo != 0u && lo != 0x7f80u ? 0x0080u : 0u)
                                     + (hi != 0u && hi != 0x7f800000u ? 0x00800000u : 0u);
            }
    }

    f32x16 acc[TPW][NTILE];
#pragma unroll
    for (int s = 0; s < TPW; ++s)
#pragma unroll
        for (int ti = 0; ti < NTILE; ++ti)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[s][ti][r] = 0.f;

    // feature row a: products from Sb[a % 2]; rows a + 2 load into the set that held
    // row a, rows a + 1 (loaded an iteration ago) go to the other buffer
    // feature row a of the 16-row block MB (a = 16 MB + 0 .. 15): steps m < MB lie
    // wholly below the diagonal, steps m > MB wholly above it, step MB holds it
    auto feature_row = [&](auto MB, int a, float4 (&ld)[SLOADS], const float4 (&sv)[SLOADS]) {
        constexpr int mb = decltype(MB)::value;
        const int buf = a & 1;
        if (a + 2 < D) load_rows(a + 2, ld);
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
            for (int ti = 0; ti < NTILE; ++ti)
                sa[ti] = *reinterpret_cast<const bf16x8 *>(&Sb[buf][32 * ti + l32][16 * m + 8 * h]);
            // steps wholly above (a < 16 m) or below (a > 16 m + 15) the diagonal take one
            // operand for all their features; in the step holding the diagonal (at position
            // rd = a - 16 m) the lane's feature 8 h + e lies above it when 8 h + e > rd, and
            // the diagonal feature itself takes half the upper value (q_b is doubled)
            const int rd = a - 16 * m;
            const bool mixed = m == mb;
#pragma unroll
            for (int s = 0; s < TPW; ++s) {
                float f[8];
                if (!mixed) {
                    const uint32_t xs = m > mb ? qa[s] : qr[s];
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = dot2(xs, qb[s][8 * m + e]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float up = dot2(qa[s], qb[s][8 * m + e]);
                        const float lo = dot2(qr[s], qb[s][8 * m + e]);
                        f[e] = 8 * h + e > rd ? up : lo;
                        if (e == (rd & 7)) f[e] = h == (rd >> 3) ? 0.5f * up : f[e];
                    }
                }
                uint32_t pk[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) pk[e >> 1] = pack_bf16x2(f[e], f[e + 1]);
                const bf16x8 fq = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
                for (int ti = 0; ti < NTILE; ++ti) acc[s][ti] = mfma(sa[ti], fq, acc[s][ti]);
            }
        }
        if (a + 1 < D) store_rows(buf ^ 1, sv);
        __syncthreads();
    };
    auto block16 = [&](auto MB) {
        constexpr int mb = decltype(MB)::value;
        for (int a = 16 * mb; a < 16 * mb + 16; a += 2) {
            feature_row(MB, a, sreg0, sreg1);
            feature_row(MB, a + 1, sreg1, sreg0);
        }
    };
    block16(std::integral_constant<int, 0>{});
    block16(std::integral_constant<int, 1>{});
    block16(std::integral_constant<int, 2>{});
    block16(std::integral_constant<int, 3>{});

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
        // decay: the incoming state counts gamma^(t+1) at token t
        const float gc = p.decay.on ? decay_pow(p.decay.lg2[bh % p.H], tq + 1) : 1.f;
        const float Dn = l + gc * den;
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
                    vr[e] = (o_r * l + gc * acc[s][ti][4 * g + e]) * inv;
                    vi[e] = (o_i * l + gc * acc[s][ti + 2][4 * g + e]) * inv;
                }
                *reinterpret_cast<uint2 *>(ore + ob + c0) = make_uint2(pack_bf16x2(vr[0], vr[1]), pack_bf16x2(vr[2], vr[3]));
                *reinterpret_cast<uint2 *>(oim + ob + c0) = make_uint2(pack_bf16x2(vi[0], vi[1]), pack_bf16x2(vi[2], vi[3]));
            }
        if (h == 0) p.row_den[rowi] = Dn;
    }
}

constexpr int ST_TOK = 64;               // tokens per stage
constexpr int KROW = ST_TOK + 4;         // dwords per staged key row (16-byte aligned, offset banks)
constexpr int ROWS_PER_WG = NW;          // feature rows per workgroup
constexpr int VROWB = 2 * D;             // bytes per token row of a value plane
constexpr int VREGION = ST_TOK * VROWB;  // 8 KiB per plane and stage
constexpr int VRPT = VREGION / 16 / NT;  // 16-byte LDS-direct loads per thread per plane
static_assert(VRPT * 16 * NT == VREGION, "value staging split");

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))
typedef __bf16 bf16x4v __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct StateStage {
    char K[2][VREGION];                  // key planes, token-major, 16-byte chunks swizzled by token
    char V[2][VREGION];                  // value planes, the same layout
    uint32_t KA[ROWS_PER_WG][KROW];      // (Re k, Im k) of this workgroup's feature rows, [row][token]
    uint32_t KR[ROWS_PER_WG][KROW];      // (-Im k, Re k) of the same rows
    float F[ST_TOK];                     // decay: gamma^(T-1-t) of the stage's tokens
};

__device__ inline int swz_v(int row) { return (row & 3) << 1; }

// (Re, Im) bf16 pairs from two words of one plane each: the low halves, the high halves
__device__ inline uint32_t pair_lo(uint32_t re, uint32_t im) { return __builtin_amdgcn_perm(im, re, 0x05040100u); }
__device__ inline uint32_t pair_hi(uint32_t re, uint32_t im) { return __builtin_amdgcn_perm(im, re, 0x07060302u); }

__device__ inline u32x2 ds_read_tr(const char *p) {
    const bf16x4v r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4v *)(p));
    return __builtin_bit_cast(u32x2, r);
}

// All of this wave's LDS-direct loads have landed; then workgroup barrier.
__device__ inline void loads_done_barrier() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

constexpr int SNT = 2 * NT;   // threads per state-build workgroup: two token groups

template <bool DECAY>
__global__ __launch_bounds__(SNT) void born_state_bf16_d64_kernel(LinearProblem p) {
    // the two stage buffers, each [token group], as two LDS variables: every
    // access names its buffer at compile time, so the reads of one buffer wait
    // only for the loads into it, not for the next stage's loads into the other
    __shared__ __align__(16) StateStage stA[2];
    __shared__ __align__(16) StateStage stB[2];

    const int lane = threadIdx.x & 63;
    const int grp = threadIdx.x / NT;         // token group: even (0) or odd (1) stages
    const int tid = threadIdx.x % NT;         // thread within the group
    const int wave = tid >> 6;                // wave within the group
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int T = p.T;
    constexpr int GROUPS = D / ROWS_PER_WG;   // workgroups per head

    const int nblk = gridDim.x;
    const int x = blockIdx.x;
    const int lin = (nblk % 8 == 0) ? (x % 8) * (nblk / 8) + x / 8 : x;
    const int64_t bh = lin / GROUPS;
    const int a0 = (lin % GROUPS) * ROWS_PER_WG;
    const int ftw = wave & 1;                 // this wave's column tile: features b = 32 ftw + l32
    const int ar0 = a0 + 2 * (wave >> 1);     // and its feature rows ar0, ar0 + 1 (both groups alike)
    const int64_t base = bh * (int64_t)T * D;
    const uint16_t *kre = reinterpret_cast<const uint16_t *>(p.k_re) + base;
    const uint16_t *kim = reinterpret_cast<const uint16_t *>(p.k_im) + base;
    const uint16_t *vpl[4] = {kre, kim, reinterpret_cast<const uint16_t *>(p.v_re) + base,
                              reinterpret_cast<const uint16_t *>(p.v_im) + base};

    // the workgroup's four feature rows through registers: lane t of the
    // group's first wave holds channels a0 .. a0 + 3 of token t of a stage
    // (zero past T, which makes every feature of such a token zero)
    u32x2 rr_reg, ri_reg;
    auto load_rows = [&](int t0) {
        rr_reg = ri_reg = u32x2{0u, 0u};
        if (tid < ST_TOK && t0 + tid < T) {
            rr_reg = *reinterpret_cast<const u32x2 *>(kre + (int64_t)(t0 + tid) * D + a0);
            ri_reg = *reinterpret_cast<const u32x2 *>(kim + (int64_t)(t0 + tid) * D + a0);
        }
    };
    const float lg2 = DECAY ? p.decay.lg2[bh % p.H] : 0.f;
    auto store_rows = [&](StateStage &S_, int t0) {
        if (tid < ST_TOK) {
            if (DECAY) S_.F[tid] = t0 + tid < T ? decay_pow(lg2, T - 1 - (t0 + tid)) : 0.f;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t p0 = pair_lo(rr_reg[i], ri_reg[i]), p1 = pair_hi(rr_reg[i], ri_reg[i]);
                S_.KA[2 * i][tid] = p0;
                S_.KA[2 * i + 1][tid] = p1;
                S_.KR[2 * i][tid] = rot_pair(p0);
                S_.KR[2 * i + 1][tid] = rot_pair(p1);
            }
        }
    };
    // values straight to LDS: chunk NT e + tid is token tid / 8 + 32 e, physical slot tid % 8,
    // holding logical chunk slot ^ swz(token); tokens past T repeat the last one (their keys are zero)
    const int srow = tid >> 3, sslot = tid & 7;
    const int lcv = sslot ^ swz_v(srow);
    auto issue_values = [&](int t0, StateStage &S_) {
#pragma unroll
        for (int i = 0; i < 4 * VRPT; ++i) {
            const int pl = i / VRPT, e = i % VRPT;
            const int row = min(t0 + srow + (NT / 8) * e, T - 1);
            char *dst = pl < 2 ? S_.K[pl] : S_.V[pl - 2];
            __builtin_amdgcn_global_load_lds((GLB_AS void *)(vpl[pl] + (int64_t)row * D + 8 * lcv),
                                             (LDS_AS void *)(dst + e * (NT * 16) + wave * 1024), 16, 0, 0);
        }
    };
    // V^T operand through the transposing read (k-step of 16 tokens): lane 16 G + 4 r + c4
    // points at token 4 h + r, channels 16 (G & 1) + 4 c4 of the 32-channel tile; its
    // element e then belongs to token 8 (e / 4) + 4 h + e % 4 of the step.
    int voff[2];
    {
        const int G = lane >> 4, r = (lane >> 2) & 3, c4 = lane & 3;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int lc = 4 * cc + 2 * (G & 1) + (c4 >> 1);
            voff[cc] = (4 * h + r) * VROWB + ((lc ^ (r << 1)) << 4) + ((c4 & 1) << 3);
        }
    }

    // value rows (tiles 0-3: Re V, Im V) on matrix cores; the Z row (the plain
    // sum of the features over tokens) as per-lane sums of the fp32 features
    f32x16 acc[2][NTILE - 1];
    float zs[2] = {0.f, 0.f};
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int ti = 0; ti < NTILE - 1; ++ti)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ft][ti][r] = 0.f;
    // row i of the wave holds features (a = ar0 + i, b = 32 ftw + l32): on or above the
    // diagonal the first operand is the pair of k_a (KA row a - a0), below it the rotated
    // pair (KR row a - a0); the second is the pair of k_b, formed from the two key planes
    // (read like the value operand: lane l32 gets channel b for its eight tokens)
    int xoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int ai = ar0 + i, b = 32 * ftw + l32;
        xoff[i] = ai <= b ? (int)offsetof(StateStage, KA) + (ai - a0) * KROW * 4
                          : (int)offsetof(StateStage, KR) + (ai - a0) * KROW * 4;
    }

    // pair pr: stage 2 pr for group 0, 2 pr + 1 for group 1.  A stage past the
    // end (group 1 in the last pair of an odd count) is staged harmlessly (its
    // keys are zero, its value rows clamped to T - 1) and not multiplied.
    const int nst = (T + ST_TOK - 1) / ST_TOK;
    const int npair = (nst + 1) / 2;
    auto t0_of = [&](int pr) { return (2 * pr + grp) * ST_TOK; };
    if (npair > 0) {
        issue_values(t0_of(0), stA[grp]);
        load_rows(t0_of(0));
        store_rows(stA[grp], t0_of(0));
    }
    loads_done_barrier();
    // pair pr reads buffer pr % 2 and stages pair pr + 1 into the other
    auto pair_step = [&](StateStage (&cur_buf)[2], StateStage (&nxt_buf)[2], int pr) {
        StateStage &cur = cur_buf[grp];
        const char *cb = reinterpret_cast<const char *>(&cur);
        if (pr + 1 < npair) {
            issue_values(t0_of(pr + 1), nxt_buf[grp]);
            load_rows(t0_of(pr + 1));
        }
        const bool live = t0_of(pr) < T;   // wave-uniform
#pragma unroll
        for (int ks = 0; ks < ST_TOK / 16; ++ks) {
            if (!live) break;
            bf16x8 wa[NTILE - 1];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const char *vb = cur.V[c >> 1] + 16 * ks * VROWB + voff[c & 1];
                const u32x2 lo = ds_read_tr(vb);
                const u32x2 hi = ds_read_tr(vb + 8 * VROWB);
                wa[c] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
            const int tb = (16 * ks + 4 * h) * 4;   // byte offset of this lane's first token in a key row
            // decay: the factors of the lane's tokens 16 ks + 4 h + e and 16 ks + 8 + 4 h + e
            float4 fa = make_float4(1.f, 1.f, 1.f, 1.f), fb = fa;
            if (DECAY) {
                fa = *reinterpret_cast<const float4 *>(&cur.F[16 * ks + 4 * h]);
                fb = *reinterpret_cast<const float4 *>(&cur.F[16 * ks + 8 + 4 * h]);
            }
            u32x4 kb0, kb1;
            {
                const char *kb = cur.K[0] + 16 * ks * VROWB + voff[ftw];
                const u32x2 rlo = ds_read_tr(kb), rhi = ds_read_tr(kb + 8 * VROWB);
                const u32x2 ilo = ds_read_tr(kb + VREGION), ihi = ds_read_tr(kb + VREGION + 8 * VROWB);
                kb0 = u32x4{pair_lo(rlo[0], ilo[0]), pair_hi(rlo[0], ilo[0]), pair_lo(rlo[1], ilo[1]), pair_hi(rlo[1], ilo[1])};
                kb1 = u32x4{pair_lo(rhi[0], ihi[0]), pair_hi(rhi[0], ihi[0]), pair_lo(rhi[1], ihi[1]), pair_hi(rhi[1], ihi[1])};
            }
#pragma unroll
            for (int ft = 0; ft < 2; ++ft) {   // ft: the wave's row ar0 + ft
                const u32x4 x0 = *reinterpret_cast<const u32x4 *>(cb + xoff[ft] + tb);
                const u32x4 x1 = *reinterpret_cast<const u32x4 *>(cb + xoff[ft] + tb + 32);
                float f[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[e] = dot2(x0[e], kb0[e]);
                    f[4 + e] = dot2(x1[e], kb1[e]);
                }
                if (DECAY) {
                    f[0] *= fa.x, f[1] *= fa.y, f[2] *= fa.z, f[3] *= fa.w;
                    f[4] *= fb.x, f[5] *= fb.y, f[6] *= fb.z, f[7] *= fb.w;
                }
                zs[ft] += ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
                const bf16x8 fk = as_bf16x8(u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                                  pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])});
#pragma unroll
                for (int ti = 0; ti < NTILE - 1; ++ti) acc[ft][ti] = mfma(wa[ti], fk, acc[ft][ti]);
            }
        }
        if (pr + 1 < npair) store_rows(nxt_buf[grp], t0_of(pr + 1));
        loads_done_barrier();
    };
    for (int pr = 0; pr < npair; pr += 2) {
        pair_step(stA, stB, pr);
        if (pr + 1 < npair) pair_step(stB, stA, pr + 1);
    }

    // Epilogue, split over the two token groups: group 0 finishes the value
    // tiles 0-1 (rows n < 64) and Z, group 1 the tiles 2-3 (64 <= n < 128).
    // Each sends the other's tiles of its partial sums through LDS (the stage
    // buffers are free: every read ended before the last barrier), and in
    // accumulate mode the old state of its own rows is in flight meanwhile.
    // Lane (l32, half h) holds rows n = 32 ti + 8 (r / 4) + 4 h + r % 4 of
    // S[n][a * 64 + b], a = ar0 + ft, b = 32 ftw + l32; an accumulated state
    // first decays by gamma^T.
    constexpr int PX = 2 * 2 * 16 + 2;   // floats per lane sent: two tiles of both rows, and Z
    static_assert((size_t)NW * PX * 64 * 4 <= sizeof(stA), "a group's partials fit in one stage buffer pair");
    float *xsend = reinterpret_cast<float *>(grp == 0 ? &stA[0] : &stB[0]) + (size_t)wave * PX * 64 + lane;
    const float *xrecv = reinterpret_cast<const float *>(grp == 0 ? &stB[0] : &stA[0]) + (size_t)wave * PX * 64 + lane;
    // the two halves of a wave summed different tokens of the same feature
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) zs[ft] += __shfl_xor(zs[ft], 32);
    auto send = [&](auto SEND) {
        constexpr int t0 = decltype(SEND)::value;
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) xsend[((ft * 2 + i) * 16 + r) * 64] = acc[ft][t0 + i][r];
    };
    if (grp == 0) {
        send(std::integral_constant<int, 2>{});
    } else {
        send(std::integral_constant<int, 0>{});
#pragma unroll
        for (int ft = 0; ft < 2; ++ft) xsend[(64 + ft) * 64] = zs[ft];
    }

    float *Sh = p.S + bh * (int64_t)NM * D * D;
    float *col[2];
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) col[ft] = Sh + (int64_t)(ar0 + ft) * D + 32 * ftw + l32;   // row n at col + n D^2
    const int keep = 2 * grp;                 // first kept tile
    const bool acc_mode = p.accumulate;       // uniform
    const bool zlane = grp == 0 && h == 0;    // lanes that write Z (row 128)
    float old[2][2][16], oldz[2] = {0.f, 0.f};
    if (acc_mode) {
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = 32 * (keep + i) + 8 * (r >> 2) + 4 * h + (r & 3);
                    old[ft][i][r] = col[ft][(int64_t)n * D * D];
                }
        if (zlane) {
#pragma unroll
            for (int ft = 0; ft < 2; ++ft) oldz[ft] = col[ft][(int64_t)(NM - 1) * D * D];
        }
    } else {
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) old[ft][i][r] = 0.f;
    }
    __syncthreads();
    const float carry = !acc_mode ? 0.f : DECAY ? decay_pow(lg2, T) : 1.f;
    auto finish = [&](auto KEEP) {
        constexpr int t0 = decltype(KEEP)::value;
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = 32 * (t0 + i) + 8 * (r >> 2) + 4 * h + (r & 3);
                    const float v = acc[ft][t0 + i][r] + xrecv[((ft * 2 + i) * 16 + r) * 64];
                    col[ft][(int64_t)n * D * D] = fmaf(carry, old[ft][i][r], v);
                }
    };
    if (grp == 0) {
        finish(std::integral_constant<int, 0>{});
        if (zlane) {
#pragma unroll
            for (int ft = 0; ft < 2; ++ft)
                col[ft][(int64_t)(NM - 1) * D * D] = fmaf(carry, oldz[ft], zs[ft] + xrecv[(64 + ft) * 64]);
        }
    } else {
        finish(std::integral_constant<int, 2>{});
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
    hipLaunchKernelGGL(born_merge_bf16_d64_kernel, dim3((unsigned)blocks), dim3(MNT), 0, p.stream, p, ntile_t);
    return hipGetLastError();
}

}  // namespace cattn

namespace cattn {

hipError_t launch_born_state_bf16_d64(const LinearProblem &p) {
    const int64_t blocks = (int64_t)p.BH * (D / ROWS_PER_WG);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    auto kern = p.decay.on ? born_state_bf16_d64_kernel<true> : born_state_bf16_d64_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(SNT), 0, p.stream, p);
    return hipGetLastError();
}

}  // namespace cattn
