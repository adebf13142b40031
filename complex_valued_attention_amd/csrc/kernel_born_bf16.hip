// Born-rule attention forward on bf16 real/imaginary planes with gfx950
// matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// The operator ("CNet: A Complex-Valued Deep Learning Framework ...",
// section 11.2, "Closing it: Born-rule attention", Figure 2) needs no running
// maximum: the weights |<q,k>|^2 are non-negative, so one pass accumulates the
// numerator sum_j w V_j and the denominator sum_j w side by side.
//
// Complex contraction as real GEMMs.  With Q' = [Re Q | Im Q] and
// K' = [Re K | Im K] (2 d_h real columns),
//     Re S^T = K' [Re Q | Im Q]^T,     Im S^T = K' [Im Q | -Re Q]^T,
// both with the same A operand K'.  Scores are formed transposed (keys are
// MFMA rows, queries MFMA columns) so that every lane of the 32x32 result
// holds one query and 16 keys -- exactly the shape the next product needs:
//     O^T = V'^T W^T,   V' = [Re V | Im V]  (2 d_h rows of O^T),
// where W^T enters as the B operand straight from registers (after packing to
// bf16), with the key order permuted consistently on both operands.
//
// Work split.  A workgroup of NW waves owns BM = 32 * NQT * NW query rows of
// one (batch, head); each wave owns NQT tiles of 32 queries whose Q' operands
// stay in registers for the whole kernel.  Keys stream in stages of BN = 64
// through double-buffered LDS: K' row-major (padded rows), V' transposed to
// [2 d_h][BN] with the key order the W^T operand uses, so both are read with
// one 16-byte LDS load per lane per MFMA.  Stages above a tile's causal
// diagonal are skipped; the diagonal 32x32 block is masked in registers.
//
// Born options (instances of their own): a per-head decay multiplies each
// weight by gamma^(k - j), formed per weight; a rotary Q is rotated as it is
// loaded, with the arithmetic of the rotary pass (rotary_math.h).
#include "cattn_internal.h"
#include "rotary_math.h"

namespace cattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int PAD = 8;   // bf16 padding per LDS row (16 bytes): conflict-free 16-byte lane reads

template <int D, int NQT, int NW, int BN>
struct BornCfg {
    static constexpr int KD = 2 * D;             // real contraction width of S
    static constexpr int KSTEPS = KD / 16;       // MFMA k-steps for S
    static constexpr int CT = KD / 32;           // 32-row tiles of O^T
    static constexpr int BM = 32 * NQT * NW;     // query rows per workgroup
    static constexpr int NT = 64 * NW;           // threads
    static constexpr int KROW = KD + PAD;        // LDS row length of K' (bf16)
    static constexpr int VROW = BN + PAD;        // LDS row length of V'^T (bf16)
    static constexpr int KS_ELEMS = BN * KROW;
    static constexpr int VT_ELEMS = KD * VROW;
    static constexpr int STAGE_ELEMS = KS_ELEMS + VT_ELEMS;
    static constexpr int LDS_BYTES = 2 * STAGE_ELEMS * 2;
    static constexpr int KCHUNKS = BN * KD / 8;  // 16-byte chunks of a K' stage
    static constexpr int VUNITS = D * (BN / 8);  // (column pair, 8-key group) units of a V' stage
    static constexpr int K_PER_T = (KCHUNKS + NT - 1) / NT;
    static constexpr int V_PER_T = (VUNITS + NT - 1) / NT;
};

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ inline u32x4 as_u32x4(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Key (within a 32-key sub-block) whose weight sits in accumulator register r of
// lane half h of the 32x32 MFMA result: rows 8*(r/4) + 4*h + r%4.
// The same key goes to LDS position 16*(r/8) + 8*h + r%8 of V'^T, so that
// lane half h reading 8 consecutive positions from 16*m + 8*h feeds the
// W^T operand registers 8m..8m+7.
__device__ inline int vt_key_of_pos(int pos) {   // pos in 0..31 -> key in 0..31
    const int m = pos >> 4, h = (pos >> 3) & 1, s = pos & 7;
    return 16 * m + 8 * (s >> 2) + 4 * h + (s & 3);
}

template <int D, int NQT, int NW, int BN, bool OPT>
__global__ __launch_bounds__(64 * NW) void born_bf16_mfma_kernel(Problem p, int nrb) {
    using C = BornCfg<D, NQT, NW, BN>;
    extern __shared__ __align__(16) __bf16 smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int T = p.T;

    // Workgroup -> (head, row block).  Heaviest causal row blocks first; with
    // BH % 8 == 0 all row blocks of a head land on one XCD (workgroups are
    // dealt to the 8 XCDs round-robin), so its K/V stay in that XCD's L2.
    const int L = blockIdx.x;
    int bh, rb;
    if ((p.BH & 7) == 0) {
        const int x = L & 7, j = L >> 3;
        bh = x + 8 * (j / nrb);
        rb = nrb - 1 - (j % nrb);
    } else {
        bh = L / nrb;
        rb = nrb - 1 - (L % nrb);
    }
    const int m0 = rb * C::BM;
    // head bases and token strides (elements) of each operand
    const int64_t hq = head_offset(p.sq, bh, p.H), hk = head_offset(p.sk, bh, p.H);
    const int64_t hv = head_offset(p.sv, bh, p.H);
    const int64_t tq = p.sq.t, tk = p.sk.t, tv = p.sv.t;

    const uint16_t *qre = reinterpret_cast<const uint16_t *>(p.q_re) + hq;
    const uint16_t *qim = reinterpret_cast<const uint16_t *>(p.q_im) + hq;
    const uint16_t *kre = reinterpret_cast<const uint16_t *>(p.k_re) + hk;
    const uint16_t *kim = reinterpret_cast<const uint16_t *>(p.k_im) + hk;
    const uint16_t *vre = reinterpret_cast<const uint16_t *>(p.v_re) + hv;
    const uint16_t *vim = reinterpret_cast<const uint16_t *>(p.v_im) + hv;

    // ---- Q' operands, resident for the whole kernel ------------------------
    // B operand of k-step ks, lane (q = l32, h): Q'[q][16 ks + 8 h .. +8].
    bf16x8 qb[NQT][C::KSTEPS];
    bf16x8 qneg[NQT][C::KSTEPS / 2];   // -Re Q chunks: the second half of [Im Q | -Re Q]
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
        const int q = m0 + 32 * (NQT * wave + t) + l32;
        u32x4 x[C::KSTEPS];
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            const int col = 16 * ks + 8 * h;
            x[ks] = u32x4{0u, 0u, 0u, 0u};
            if (q < T) {
                const uint16_t *src = col < D ? qre + (int64_t)q * tq + col : qim + (int64_t)q * tq + (col - D);
                x[ks] = *reinterpret_cast<const u32x4 *>(src);
            }
        }
        if (OPT && p.rot && q < T) {
            // chunk ks < KSTEPS / 2 holds Re of channels 16 ks + 8 h + e, chunk ks + KSTEPS / 2 their Im
            const double pos = (double)(p.rot_pos0 + q);
#pragma unroll
            for (int ks = 0; ks < C::KSTEPS / 2; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int sh = 16 * (e & 1);
                    const uint32_t rw = x[ks][e >> 1], iw = x[ks + C::KSTEPS / 2][e >> 1];
                    float c, sn, yr, yi;
                    rotary_phase(pos, rotary_theta(16 * ks + 8 * h + e, p.rot_log_base, D), c, sn);
                    rotary_apply(__uint_as_float(((rw >> sh) & 0xffffu) << 16),
                                 __uint_as_float(((iw >> sh) & 0xffffu) << 16), c, sn, yr, yi);
                    x[ks][e >> 1] = (rw & ~(0xffffu << sh)) | ((uint32_t)rotary_bf16(yr) << sh);
                    x[ks + C::KSTEPS / 2][e >> 1] = (iw & ~(0xffffu << sh)) | ((uint32_t)rotary_bf16(yi) << sh);
                }
        }
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            qb[t][ks] = as_bf16x8(x[ks]);
            if (ks < C::KSTEPS / 2) qneg[t][ks] = as_bf16x8(x[ks] ^ 0x80008000u);
        }
    }
    const float lg2 = OPT && p.decay.on ? p.decay.lg2[bh % p.H] : 0.f;

    f32x16 oacc[NQT][C::CT];
    float rsum[NQT];
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
        rsum[t] = 0.f;
#pragma unroll
        for (int c = 0; c < C::CT; ++c) oacc[t][c] = f32x16{};
    }

    const int kend = p.causal ? min(T, m0 + C::BM) : T;
    const int nstages = (kend + BN - 1) / BN;

    // ---- global -> register staging of one K'/V' stage ----------------------
    u32x4 kreg[C::K_PER_T];
    uint32_t vreg[C::V_PER_T][8];

    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < C::K_PER_T; ++i) {
            const int ci = tid + i * C::NT;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (ci < C::KCHUNKS) {
                const int key = ci / (C::KD / 8), part = ci % (C::KD / 8);
                const int col = part * 8;
                const int kg = k0 + key;
                if (kg < T) {
                    const uint16_t *src = col < D ? kre + (int64_t)kg * tk + col : kim + (int64_t)kg * tk + (col - D);
                    x = *reinterpret_cast<const u32x4 *>(src);
                }
            }
            kreg[i] = x;
        }
#pragma unroll
        for (int i = 0; i < C::V_PER_T; ++i) {
            const int u = tid + i * C::NT;
            const int cp = u % D, grp = u / D;              // column pair over [Re V | Im V], 8-key group
            const int plane = cp / (D / 2), cc = 2 * (cp % (D / 2));
            const uint16_t *src = plane == 0 ? vre : vim;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int pos = 8 * grp + s;                // LDS position within the stage
                const int key = 32 * (pos >> 5) + vt_key_of_pos(pos & 31);
                const int kg = k0 + key;
                uint32_t x = 0u;
                if (u < C::VUNITS && kg < T) x = *reinterpret_cast<const uint32_t *>(src + (int64_t)kg * tv + cc);
                vreg[i][s] = x;
            }
        }
    };

    auto store_stage = [&](int buf) {
        __bf16 *ks = smem + buf * C::STAGE_ELEMS;
        __bf16 *vt = ks + C::KS_ELEMS;
#pragma unroll
        for (int i = 0; i < C::K_PER_T; ++i) {
            const int ci = tid + i * C::NT;
            if (ci < C::KCHUNKS) {
                const int key = ci / (C::KD / 8), part = ci % (C::KD / 8);
                *reinterpret_cast<u32x4 *>(ks + key * C::KROW + part * 8) = kreg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < C::V_PER_T; ++i) {
            const int u = tid + i * C::NT;
            if (u < C::VUNITS) {
                const int cp = u % D, grp = u / D;
                const int c = 2 * cp;                       // row of V'^T (Re V columns then Im V columns)
                u32x4 lo, hi;                               // column c and c + 1, 8 keys each
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint32_t a = vreg[i][2 * s], b = vreg[i][2 * s + 1];
                    lo[s] = (a & 0xffffu) | (b << 16);
                    hi[s] = (a >> 16) | (b & 0xffff0000u);
                }
                *reinterpret_cast<u32x4 *>(vt + c * C::VROW + 8 * grp) = lo;
                *reinterpret_cast<u32x4 *>(vt + (c + 1) * C::VROW + 8 * grp) = hi;
            }
        }
    };

    if (nstages > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();

    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    for (int st = 0; st < nstages; ++st) {
        const int k0 = st * BN;
        const int buf = st & 1;
        if (st + 1 < nstages) load_stage(k0 + BN);

        const __bf16 *ks = smem + buf * C::STAGE_ELEMS;
        const __bf16 *vt = ks + C::KS_ELEMS;

#pragma unroll
        for (int sb = 0; sb < BN / 32; ++sb) {
            const int kb0 = k0 + 32 * sb;
            bool live[NQT], diag[NQT];
            bool any = false;
#pragma unroll
            for (int t = 0; t < NQT; ++t) {
                const int qt0 = m0 + 32 * (NQT * wave + t);
                live[t] = kb0 < T && (!p.causal || kb0 <= qt0);
                diag[t] = p.causal && kb0 == qt0;
                any = any || live[t];
            }
            if (!any) continue;

            // S^T = K' Q'^H for this 32-key sub-block
            f32x16 sr[NQT], si[NQT];
#pragma unroll
            for (int t = 0; t < NQT; ++t) { sr[t] = f32x16{}; si[t] = f32x16{}; }
#pragma unroll
            for (int kk = 0; kk < C::KSTEPS; ++kk) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ks + (32 * sb + l32) * C::KROW + 16 * kk + 8 * h);
#pragma unroll
                for (int t = 0; t < NQT; ++t) {
                    if (!live[t]) continue;
                    const bf16x8 b2 = kk < C::KSTEPS / 2 ? qb[t][kk + C::KSTEPS / 2] : qneg[t][kk - C::KSTEPS / 2];
                    sr[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[t][kk], sr[t], 0, 0, 0);
                    si[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b2, si[t], 0, 0, 0);
                }
            }

            // w = |S|^2 (masked on the diagonal block), packed to bf16 as the W^T operand
            bf16x8 wop[NQT][2];
#pragma unroll
            for (int t = 0; t < NQT; ++t) {
                if (!live[t]) continue;
                uint32_t packed[8];
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float w0 = sr[t][r] * sr[t][r] + si[t][r] * si[t][r];
                    float w1 = sr[t][r + 1] * sr[t][r + 1] + si[t][r + 1] * si[t][r + 1];
                    if (OPT && p.decay.on) {
                        // gamma^(k - j); negative distances only on keys the mask zeroes
                        const int n = m0 + 32 * (NQT * wave + t) + l32 - kb0 - (8 * (r >> 2) + 4 * h + (r & 3));
                        w0 *= decay_pow(lg2, max(n, 0));
                        w1 *= decay_pow(lg2, max(n - 1, 0));
                    }
                    if (diag[t]) {
                        const int key0 = 8 * (r >> 2) + 4 * h + (r & 3);   // key row of register r
                        if (key0 > l32) w0 = 0.f;
                        if (key0 + 1 > l32) w1 = 0.f;
                    }
                    packed[r >> 1] = pack_bf16x2(w0, w1);
                    rsum[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed[r >> 1]), ones,
                                                             rsum[t], false);
                }
                wop[t][0] = as_bf16x8(u32x4{packed[0], packed[1], packed[2], packed[3]});
                wop[t][1] = as_bf16x8(u32x4{packed[4], packed[5], packed[6], packed[7]});
            }

            // O^T += V'^T W^T
#pragma unroll
            for (int c = 0; c < C::CT; ++c) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const bf16x8 a =
                        *reinterpret_cast<const bf16x8 *>(vt + (32 * c + l32) * C::VROW + 32 * sb + 16 * m + 8 * h);
#pragma unroll
                    for (int t = 0; t < NQT; ++t) {
                        if (!live[t]) continue;
                        oacc[t][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wop[t][m], oacc[t][c], 0, 0, 0);
                    }
                }
            }
        }

        if (st + 1 < nstages) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = acc / (sum w + eps), stored as bf16 planes ------------
    const int64_t ho = head_offset(p.so, bh, p.H), to = p.so.t;
    uint16_t *ore = reinterpret_cast<uint16_t *>(p.o_re) + ho;
    uint16_t *oim = reinterpret_cast<uint16_t *>(p.o_im) + ho;
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
        const float den = rsum[t] + __shfl_xor(rsum[t], 32) + p.eps;   // both lane halves hold this query
        const float inv = den != 0.f ? 1.f / den : 0.f;
        const int q = m0 + 32 * (NQT * wave + t) + l32;
        if (q >= T) continue;
#pragma unroll
        for (int c = 0; c < C::CT; ++c) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 32 * c + 8 * g + 4 * h;     // rows col..col+3 of O^T
                const u32x2 v = {pack_bf16x2(oacc[t][c][4 * g] * inv, oacc[t][c][4 * g + 1] * inv),
                                 pack_bf16x2(oacc[t][c][4 * g + 2] * inv, oacc[t][c][4 * g + 3] * inv)};
                uint16_t *dst = col < D ? ore + (int64_t)q * to + col : oim + (int64_t)q * to + (col - D);
                *reinterpret_cast<u32x2 *>(dst) = v;
            }
        }
        if (p.row_den && h == 0) p.row_den[(int64_t)bh * T + q] = den;
    }
}

template <int D, int NQT, int NW, int BN>
hipError_t launch_cfg(const Problem &p) {
    using C = BornCfg<D, NQT, NW, BN>;
    const bool opt = p.decay.on || p.rot;
    auto kern = opt ? born_bf16_mfma_kernel<D, NQT, NW, BN, true> : born_bf16_mfma_kernel<D, NQT, NW, BN, false>;
    static std::atomic<uint64_t> lds_set[2] = {{0}, {0}};   // per instance
    const hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), C::LDS_BYTES, lds_set[opt]);
    if (e != hipSuccess) return e;
    const int nrb = (p.T + C::BM - 1) / C::BM;
    const int64_t blocks = (int64_t)p.BH * nrb;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(C::NT), C::LDS_BYTES, p.stream, p, nrb);
    return hipGetLastError();
}

}  // namespace

bool supports_born_bf16_mfma(const Problem &p) {
    return p.op == OP_BORN && p.layout == LAYOUT_BF16 && p.d == 16 && p.aligned16;
}

hipError_t launch_born_bf16_mfma(const Problem &p) {
    switch (p.d) {
        case 16: return launch_cfg<16, 1, 8, 64>(p);
        default: return hipErrorNotSupported;
    }
}

}  // namespace cattn
