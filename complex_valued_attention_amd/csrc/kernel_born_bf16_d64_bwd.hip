// Born-rule attention backward, head width 64, bf16 real/imaginary planes,
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
//
// Gradients ("CNet ...", section 3, the Wirtinger accumulation rule (2)):
// given G = dL/d(conj O), the forward's output O and row denominators l, and
// per query row delta = Re(G^H O), with E = Re(G V^H) and, on the causal
// support, D2 = 2 (E - delta) / l and P = D2 o S (S = Q K^H):
//     dV = (w / l)^T G,   dQ = P K,   dK = P^H Q.
// Real forms used below, with a prime for the real width-128 row [Re | Im]:
//     Re S = Q' . K',   Im S = Re Q . (-Im K) + Im Q . Re K,   E = G' . V'
//     Re dQ = P_r K_r - P_i K_i,  Im dQ = P_r K_i + P_i K_r
//     Re dK = P_r Q_r + P_i Q_i,  Im dK = P_r Q_i - P_i Q_r
//     dV'   = (w / l) G'
//
// Two kernels share the forward's building blocks: swizzled 64-row stages of
// one plane per 8 KiB region, staged straight from global memory into LDS,
// A operands of row-major tiles read as 16-byte chunks, and the transposing
// LDS read (ds_read_b64_tr_b16) for tiles used with their rows as the
// contraction index.  Every tile is staged once, in a swizzle that keeps
// both kinds of read free of bank conflicts (swz_b), whether a kernel reads
// it one way (V in the dQ kernel) or both (K; Q and G).  Products are
// formed with the streamed rows along the MFMA's k-dimension's partner, so
// each lane's 16 accumulator values are directly the bf16 B operand of the
// next product (no shuffles).
//
//  * dQ kernel: a workgroup of 4 waves owns 128 queries (32 per wave, the
//    wave's Q' and G' in registers) and streams K and V; two workgroups per
//    compute unit.  Per 32-key block:
//    S^T and E^T (keys x queries), P^T, then dQ^T += K^T P^T.
//  * dK/dV kernel: a workgroup owns 128 keys (K' and V' in registers) and
//    streams Q and G with the per-query 1/l and delta/l (formed once per
//    query by a small kernel before it, see born_bf16_d64_bwd_scal_kernel,
//    and copied into LDS with each stage).  Per 32-query
//    block: S and E (queries x keys), w/l and P, then dV^T += G^T (w/l) and
//    dK^T += Q^T P.
// Causal work is balanced by mirrored pairs of tiles, as in the forward.
//
// Per-head decay (DECAY instances): every weight w and D2 on the causal
// support carries gamma^(k - j) (query k, key j).  In the dQ kernel, on a
// block with no mask, the factor splits into a part per lane and register
// group (one exponential each) and a part per register within its group
// (gamma^0..3, per kernel); the dK/dV kernel, at its register limit, and
// masked blocks form it per weight, the distance clamped at 0 where the mask
// zeroes the weight anyway.
#include "cattn_internal.h"

namespace cattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4v __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

constexpr int D = 64;
constexpr int NW = 4;                   // waves per workgroup, one per SIMD
constexpr int NT = 64 * NW;
constexpr int BT = 32 * NW;             // rows owned by a workgroup (queries or keys)
constexpr int BS = 64;                  // streamed rows per LDS stage
constexpr int ROWB = 2 * D;             // bytes per row of one plane
constexpr int REGION = BS * ROWB;       // 8 KiB

// One swizzle for a tile read both ways, free of bank conflicts for the
// row-major operand reads (16 lanes on 16 rows, one chunk) and for the
// transposing reads (rows 4 q .. 4 q + 3, four chunks): the even rows of
// 16 take eight distinct slots, and so do the odd ones, and rows 4 q and
// 4 q + 2 (likewise 4 q + 1 and 4 q + 3) differ in bit 2 of the slot.
__device__ inline int swz_b(int row) {
    const int i = (row >> 1) & 7;
    return (((i & 1) << 2) | (i >> 1)) ^ ((row & 1) << 1);
}

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ inline u32x2 ds_read_tr(const char *p) {
    const bf16x4v r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4v *)(p));
    return __builtin_bit_cast(u32x2, r);
}

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane,
// as a buffer load: the resource (SGPRs) holds the stage's first row as its
// base and the 8 KiB a stage spans as its extent, and each lane supplies a
// 32-bit byte offset (one VGPR, where a plain global address takes two).  The
// compiler sets M0 from the LDS pointer itself.  Completion is tracked by
// hand (vmcnt(0) before the barrier that publishes a stage).
__device__ inline void dma16(uint32_t lds, __amdgpu_buffer_rsrc_t rsrc, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(uintptr_t)lds, 16, voff, 0, 0, 0);
}

// All of this wave's loads have landed; then workgroup barrier.
__device__ inline void loads_done_barrier() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

// Rows r0 .. r0 + 63 of one plane into one LDS region, chunk c of row r at
// slot c ^ swz_b(r).  Rows past T repeat row T - 1 (they are masked later).
// NTH threads of the workgroup share the copy.
template <int NTH>
__device__ inline void stage_region(uint32_t region, const uint16_t *plane, int r0, int T, int tid, int wave) {
    constexpr int C = REGION / 16 / NTH;   // 16-byte chunks per thread
    static_assert(C * 16 * NTH == REGION, "staging split");
    // the stage's first row as the uniform base (64-bit arithmetic, any T);
    // dword 3 is the gfx9 raw-buffer format word
    const char *sbase = reinterpret_cast<const char *>(plane) + (int64_t)r0 * ROWB;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)sbase, 0, REGION, 0x00020000);
    const int slot = tid & 7;
#pragma unroll
    for (int e = 0; e < C; ++e) {
        const int row = (tid >> 3) + (NTH / 8) * e;
        const int lc = slot ^ swz_b(row);
        const int g = min(row, T - 1 - r0);   // row within the stage; < 64, so the offset is < 8 KiB
        const uint32_t dst = __builtin_amdgcn_readfirstlane(region + (uint32_t)(e * NTH * 16 + wave * 1024));
        dma16(dst, rsrc, (uint32_t)(g * ROWB + 16 * lc));
    }
}

// B-operand rows: lane (row l32, half h) holds X'[row][16 kk + 8 h .. + 8] of
// X' = [Re X | Im X]; zero for rows past T.
__device__ inline void load_rows_b(const uint16_t *re, const uint16_t *im, int row, int T, int h, u32x4 (&x)[8]) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < T) v = *reinterpret_cast<const u32x4 *>((kk < 4 ? re : im) + (int64_t)row * D + 16 * (kk & 3) + 8 * h);
        x[kk] = v;
    }
}

// Per-lane LDS offsets in a swz_b tile: the A operand of k-step kk of a
// row-major tile (row l32, logical chunk 2 (kk % 4) + h), and the two
// transposing reads of a tile whose rows are the contraction index (rows
// 0-7 and 8-15 of a 16-row step: the slot depends on bit 3 of the row, so
// the second read has offsets of its own).
struct Offsets {
    int koff[4];
    int voff[2];
    int voffh[2];
};

__device__ inline Offsets lane_offsets_b(int lane) {
    Offsets o;
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int j = 0; j < 4; ++j) o.koff[j] = l32 * ROWB + (((2 * j + h) ^ swz_b(l32)) << 4);
    const int G = lane >> 4, r = (lane >> 2) & 3, c4 = lane & 3;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
        const int lc = 4 * cc + 2 * (G & 1) + (c4 >> 1);
        o.voff[cc] = (4 * h + r) * ROWB + ((lc ^ swz_b(4 * h + r)) << 4) + ((c4 & 1) << 3);
        o.voffh[cc] = (4 * h + r + 8) * ROWB + ((lc ^ swz_b(4 * h + r + 8)) << 4) + ((c4 & 1) << 3);
    }
    return o;
}

// 32 channels x 16 rows A operand through two transposing reads, rows 0-7
// and 8-15 of the step at their own offsets.
__device__ inline bf16x8 tr_operand_b(const char *base, int lo_off, int hi_off) {
    const u32x2 lo = ds_read_tr(base + lo_off);
    const u32x2 hi = ds_read_tr(base + hi_off);
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Stores a (channels x rows) accumulator set as bf16 planes: acc[c], c < 2 real
// plane, c >= 2 imaginary plane, channel tile c & 1; lane row = l32.
__device__ inline void store_rows(uint16_t *re, uint16_t *im, int row, int h, const f32x16 (&acc)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int col = 32 * (c & 1) + 8 * g + 4 * h;
            const u32x2 v = {pack_bf16x2(acc[c][4 * g], acc[c][4 * g + 1]),
                             pack_bf16x2(acc[c][4 * g + 2], acc[c][4 * g + 3])};
            *reinterpret_cast<u32x2 *>((c < 2 ? re : im) + (int64_t)row * D + col) = v;
        }
    }
}

__device__ inline void work_item(const BwdProblem &p, int nwork, int &bh, int &item) {
    const int L = blockIdx.x;
    if ((p.BH & 7) == 0) {   // all items of a head on one XCD
        const int x = L & 7, j = L >> 3;
        bh = x + 8 * (j / nwork);
        item = j % nwork;
    } else {
        bh = L / nwork;
        item = L % nwork;
    }
}

// ---------------------------------------------------------------------------- dQ
constexpr int QREG = 4;   // K re, K im, V re, V im, each staged once (swizzle swz_b)
// The dQ kernel runs two waves per SIMD (256 registers) from two workgroups
// of 4 waves over 128 queries each: one wave's waits, barriers included, are
// filled by a wave of the other workgroup.
constexpr int QNW = 4;
constexpr int QNT = 64 * QNW;
constexpr int QBT = 32 * QNW;

template <bool DECAY>
__global__ __launch_bounds__(QNT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void born_bf16_d64_bwd_dq_kernel(BwdProblem p, int nrb, int nwork) {
    __shared__ __align__(16) char lds[2 * QREG * REGION];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int T = p.T;
    int bh, item;
    work_item(p, nwork, bh, item);

    const int64_t head = (int64_t)bh * T * D;
    auto plane = [&](const void *x) { return reinterpret_cast<const uint16_t *>(x) + head; };
    const uint16_t *stage_planes[QREG] = {plane(p.k_re), plane(p.k_im), plane(p.v_re), plane(p.v_im)};
    const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char *)lds;
    const Offsets off = lane_offsets_b(lane);

    auto issue_stage = [&](int s) {
        const uint32_t base = lds0 + (uint32_t)((s & 1) * QREG * REGION);
#pragma unroll
        for (int r = 0; r < QREG; ++r)
            stage_region<QNT>(base + r * REGION, stage_planes[r], s * BS, T, tid, wave);
    };

    const int nblocks = p.causal && item != nrb - 1 - item ? 2 : 1;
    for (int blk = 0; blk < nblocks; ++blk) {
        const int rb = p.causal ? (blk == 0 ? nrb - 1 - item : item) : item;
        const int m0 = rb * QBT;
        const int qt0 = m0 + 32 * wave;
        const int q = qt0 + l32;

        // Q' and G' of this lane's query as B operands; delta and 2/l
        u32x4 x[8];
        bf16x8 qb[8], gb[8];
        load_rows_b(plane(p.q_re), plane(p.q_im), q, T, h, x);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qb[kk] = as_bf16x8(x[kk]);
        load_rows_b(plane(p.g_re), plane(p.g_im), q, T, h, x);
        u32x4 ox[8];
        load_rows_b(plane(p.o_re), plane(p.o_im), q, T, h, ox);
        float dl = 0.f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            gb[kk] = as_bf16x8(x[kk]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dl += bf_lo(x[kk][e]) * bf_lo(ox[kk][e]) + bf_hi(x[kk][e]) * bf_hi(ox[kk][e]);
        }
        dl += __shfl_xor(dl, 32);   // both lane halves hold this query
        float inv2 = 0.f;
        if (q < T) {
            const float l = p.row_den[(int64_t)bh * T + q];
            inv2 = l != 0.f ? 2.f / l : 0.f;   // a zero denominator: no gradient
        }
        const float dinv2 = dl * inv2;
        // DECAY: gamma^(3 - b) for register b = r % 4 of a group
        const float lg2 = DECAY ? p.decay.lg2[bh % p.H] : 0.f;
        float sig[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) sig[b] = DECAY ? decay_pow(lg2, 3 - b) : 1.f;

        f32x16 acc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = f32x16{};

        auto key_block = [&](const char *st, int sb, bool masked, int lim, int kb0) {
            f32x16 sr = f32x16{}, si = f32x16{}, e = f32x16{};
            // the sign mask made opaque here, so that -Re Q is formed in the
            // block rather than hoisted into 16 registers for the whole loop
            uint32_t sgn = 0x80008000u;
            __asm__ __volatile__("" : "+s"(sgn));
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int o = (kk >> 2) * REGION + sb * 32 * ROWB + off.koff[kk & 3];
                const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(st + o);
                sr = mfma(ak, qb[kk], sr);
                // -Re Q formed as it is used (sign bits flipped), not held in 16 more registers
                si = mfma(ak, kk < 4 ? qb[kk + 4] : as_bf16x8(__builtin_bit_cast(u32x4, qb[kk - 4]) ^ sgn), si);
                const bf16x8 av = *reinterpret_cast<const bf16x8 *>(st + 2 * REGION + o);
                e = mfma(av, gb[kk], e);
            }
            // P^T = D2 S^T; register r of lane half h is key 8 (r/4) + 4 h + r % 4
            // DECAY, no mask: gamma^(q - key) = mu[r / 4] sigma[r % 4] (all <= 1)
            float mu[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) mu[a] = DECAY && !masked ? decay_pow(lg2, q - kb0 - 8 * a - 4 * h - 3) : 1.f;
            uint32_t pr[8], pi[8];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float d0 = e[r] * inv2 - dinv2, d1 = e[r + 1] * inv2 - dinv2;
                if (DECAY) {
                    const int n0 = q - kb0 - (8 * (r >> 2) + 4 * h + (r & 3));
                    d0 *= masked ? decay_pow(lg2, max(n0, 0)) : mu[r >> 2] * sig[r & 3];
                    d1 *= masked ? decay_pow(lg2, max(n0 - 1, 0)) : mu[r >> 2] * sig[(r & 3) + 1];
                }
                if (masked) {
                    const int key0 = 8 * (r >> 2) + 4 * h + (r & 3);
                    d0 = key0 > lim ? 0.f : d0;
                    d1 = key0 + 1 > lim ? 0.f : d1;
                }
                pr[r >> 1] = pack_bf16x2(d0 * sr[r], d1 * sr[r + 1]);
                pi[r >> 1] = pack_bf16x2(d0 * si[r], d1 * si[r + 1]);
            }
            bf16x8 prb[2], pib[2], pnb[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const u32x4 a = {pr[4 * m], pr[4 * m + 1], pr[4 * m + 2], pr[4 * m + 3]};
                const u32x4 b = {pi[4 * m], pi[4 * m + 1], pi[4 * m + 2], pi[4 * m + 3]};
                prb[m] = as_bf16x8(a);
                pib[m] = as_bf16x8(b);
                pnb[m] = as_bf16x8(b ^ 0x80008000u);
            }
            // dQ^T += K^T P^T:  Re += K_r P_r - K_i P_i,  Im += K_i P_r + K_r P_i
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const char *b = st + (32 * sb + 16 * m) * ROWB;
                    const bf16x8 krt = tr_operand_b(b, off.voff[ct], off.voffh[ct]);
                    const bf16x8 kit = tr_operand_b(b + REGION, off.voff[ct], off.voffh[ct]);
                    acc[ct] = mfma(krt, prb[m], acc[ct]);
                    acc[ct] = mfma(kit, pnb[m], acc[ct]);
                    acc[2 + ct] = mfma(kit, prb[m], acc[2 + ct]);
                    acc[2 + ct] = mfma(krt, pib[m], acc[2 + ct]);
                }
            }
        };

        const int kend = p.causal ? min(T, m0 + QBT) : T;
        const int nstages = (kend + BS - 1) / BS;
        const bool wave_live = qt0 < T;

        loads_done_barrier();   // the previous row block is done with both buffers
        issue_stage(0);
        // Stages whose key blocks are full for every wave (below the row
        // block's diagonal region, inside T) run in a loop with no mask or
        // skip branch, so the accumulators stay in place across it; a wave past
        // T computes on zero operands there and stores nothing.
        const int nfull = (p.causal ? min(m0, T) : T) / BS;
        int s = 0;
        for (; s < nfull; ++s) {
            loads_done_barrier();
            if (s + 1 < nstages) issue_stage(s + 1);
            const char *st = lds + (s & 1) * QREG * REGION;
#pragma unroll
            for (int sb = 0; sb < BS / 32; ++sb) key_block(st, sb, false, 31, s * BS + 32 * sb);
        }
        for (; s < nstages; ++s) {
            loads_done_barrier();
            if (s + 1 < nstages) issue_stage(s + 1);
            if (!wave_live) continue;
            const char *st = lds + (s & 1) * QREG * REGION;
#pragma unroll
            for (int sb = 0; sb < BS / 32; ++sb) {
                const int kb0 = s * BS + 32 * sb;
                const bool skip = kb0 >= T || (p.causal && kb0 > qt0);
                const bool full = (!p.causal || kb0 + 32 <= qt0) && kb0 + 32 <= T;
                if (full)
                    key_block(st, sb, false, 31, kb0);
                else if (!skip)
                    key_block(st, sb, true, min(p.causal ? qt0 + l32 - kb0 : 31, T - 1 - kb0), kb0);
            }
        }
        if (q < T) store_rows(reinterpret_cast<uint16_t *>(p.dq_re) + head, reinterpret_cast<uint16_t *>(p.dq_im) + head,
                              q, h, acc);
    }
}

// ---------------------------------------------------------------------------- dK, dV
constexpr int KREG = 4;   // Q re, Q im, G re, G im, each staged once (swizzle swz_b)

// Per-query scalars of the key-side kernel, (1 / l, delta / l) as a float
// pair per row, formed once before it (four threads per query, the
// channels split as 4 x 16) rather than in every workgroup of keys.  They
// are written into the dq_re buffer, which the query-side kernel, run after
// the key-side one, then overwrites.
__global__ __launch_bounds__(256) void born_bf16_d64_bwd_scal_kernel(BwdProblem p, int64_t rows) {
    const int64_t row = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
    const int sp = threadIdx.x & 3;
    const uint16_t *src[4] = {reinterpret_cast<const uint16_t *>(p.g_re), reinterpret_cast<const uint16_t *>(p.g_im),
                              reinterpret_cast<const uint16_t *>(p.o_re), reinterpret_cast<const uint16_t *>(p.o_im)};
    u32x4 sx[8];   // G re, G im, O re, O im: two 16-byte chunks each
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < rows) v = *reinterpret_cast<const u32x4 *>(src[i >> 1] + row * D + 16 * sp + 8 * (i & 1));
        sx[i] = v;
    }
    float dl = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dl += bf_lo(sx[i][e]) * bf_lo(sx[4 + i][e]) + bf_hi(sx[i][e]) * bf_hi(sx[4 + i][e]) +
                  bf_lo(sx[2 + i][e]) * bf_lo(sx[6 + i][e]) + bf_hi(sx[2 + i][e]) * bf_hi(sx[6 + i][e]);
    dl += __shfl_xor(dl, 1);
    dl += __shfl_xor(dl, 2);
    if (sp == 0 && row < rows) {
        const float l = p.row_den[row];
        const float inv = l != 0.f ? 1.f / l : 0.f;
        reinterpret_cast<f32x2 *>(p.dq_re)[row] = f32x2{inv, dl * inv};
    }
}

template <bool DECAY>
__global__ __launch_bounds__(NT) void born_bf16_d64_bwd_dkdv_kernel(BwdProblem p, int nkt, int nwork) {
    __shared__ __align__(16) char lds[2 * KREG * REGION];
    __shared__ __align__(16) float scal[2][2 * BS];   // [buffer][(1/l, delta/l) of each query of the stage]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int T = p.T;
    int bh, item;
    work_item(p, nwork, bh, item);

    const int64_t head = (int64_t)bh * T * D;
    auto plane = [&](const void *x) { return reinterpret_cast<const uint16_t *>(x) + head; };
    const uint16_t *stage_planes[KREG] = {plane(p.q_re), plane(p.q_im), plane(p.g_re), plane(p.g_im)};
    const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char *)lds;
    const Offsets off = lane_offsets_b(lane);

    // the stage's per-query scalars (64 float pairs, 512 bytes) from the pairs
    // written before this kernel, by waves 0 and 1 (64 lanes x 4 bytes each);
    // pairs past T read as zero
    const char *scal_src = reinterpret_cast<const char *>(p.dq_re) + (int64_t)bh * T * 8;
    auto scal_issue = [&](int q0, int buf) {
        if (wave < 2) {
            const int64_t left = (int64_t)(T - q0) * 8;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(scal_src + (int64_t)q0 * 8), 0, (int)(left < 512 ? left : 512), 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(&scal[buf][0] + 64 * wave), 4,
                                                     (uint32_t)(256 * wave + 4 * lane), 0, 0, 0);
        }
    };

    const int nblocks = p.causal && item != nkt - 1 - item ? 2 : 1;
    for (int blk = 0; blk < nblocks; ++blk) {
        const int kt = p.causal ? (blk == 0 ? item : nkt - 1 - item) : item;   // long tile first
        const int k0 = kt * BT;
        const int kw0 = k0 + 32 * wave;
        const int key = kw0 + l32;

        // K' and V' of this lane's key as B operands
        u32x4 x[8];
        bf16x8 kb[8], kni[4], vb[8];
        load_rows_b(plane(p.k_re), plane(p.k_im), key, T, h, x);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            kb[kk] = as_bf16x8(x[kk]);
            if (kk >= 4) kni[kk - 4] = as_bf16x8(x[kk] ^ 0x80008000u);   // -Im K
        }
        load_rows_b(plane(p.v_re), plane(p.v_im), key, T, h, x);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) vb[kk] = as_bf16x8(x[kk]);

        f32x16 dk[4], dv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) dk[c] = dv[c] = f32x16{};
        // DECAY: the head's log2 gamma (this kernel is at its register limit: each
        // factor is one exponential, formed as it is used)
        const float lg2 = DECAY ? p.decay.lg2[bh % p.H] : 0.f;

        // The work of one 32-query block sb, in steps that a full stage
        // interleaves across its two blocks.
        // S^T and E = Re(G V^H)^T, contraction step kk (three products)
        auto score_step = [&](const char *st, int sb, int kk, f32x16 &sr, f32x16 &si, f32x16 &e) {
            const int o = (kk >> 2) * REGION + sb * 32 * ROWB + off.koff[kk & 3];
            const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(st + o);
            sr = mfma(aq, kb[kk], sr);
            si = mfma(aq, kk < 4 ? kni[kk] : kb[kk - 4], si);
            const bf16x8 ag = *reinterpret_cast<const bf16x8 *>(st + 2 * REGION + o);
            e = mfma(ag, vb[kk], e);
        };
        // weights of register group g: register r of lane half h is query
        // 8 (r/4) + 4 h + r % 4 of the block
        // DECAY: qb0 is the block's first query; the factor gamma^(query - key)
        auto weight_group = [&](const float *sc, int sb, int g, bool masked, int lo,
                                int hi, const f32x16 &sr, const f32x16 &si, const f32x16 &e, uint32_t (&aw)[8],
                                uint32_t (&pr)[8], uint32_t (&pi)[8], int qb0) {
            // (1/l, delta/l) of queries 32 sb + 8 g + 4 h + c, c = 0 .. 3
            const f32x4 x0 = *reinterpret_cast<const f32x4 *>(sc + 2 * (32 * sb + 8 * g + 4 * h));
            const f32x4 x1 = *reinterpret_cast<const f32x4 *>(sc + 2 * (32 * sb + 8 * g + 4 * h) + 4);
            const f32x4 iv = {x0[0], x0[2], x1[0], x1[2]};
            const f32x4 di = {x0[1], x0[3], x1[1], x1[3]};
            const int n0 = qb0 + 8 * g + 4 * h - key;   // distance of register c = 0
            float a[4], d2[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int r = 4 * g + c;
                // w/l, and half of dL/ds (2 (e - delta)/l); dK is doubled on store
                a[c] = iv[c] * (sr[r] * sr[r] + si[r] * si[r]);
                d2[c] = e[r] * iv[c] - di[c];
                if (DECAY) {   // distances are >= 0 where the mask keeps the weight
                    const float f = decay_pow(lg2, max(n0 + c, 0));
                    a[c] *= f;
                    d2[c] *= f;
                }
                if (masked) {
                    const int qi = 8 * g + 4 * h + c;
                    const bool ok = qi >= lo && qi <= hi;
                    a[c] = ok ? a[c] : 0.f;
                    d2[c] = ok ? d2[c] : 0.f;
                }
            }
#pragma unroll
            for (int c = 0; c < 4; c += 2) {
                const int r = 4 * g + c;
                aw[r >> 1] = pack_bf16x2(a[c], a[c + 1]);
                pr[r >> 1] = pack_bf16x2(d2[c] * sr[r], d2[c + 1] * sr[r + 1]);
                pi[r >> 1] = pack_bf16x2(d2[c] * si[r], d2[c + 1] * si[r + 1]);
            }
        };
        // the packed weights as B operands: w/l, Re P, Im P, -Im P
        struct GradOps {
            bf16x8 ab[2], prb[2], pib[2], pnb[2];
        };
        auto grad_ops = [&](const uint32_t (&aw)[8], const uint32_t (&pr)[8], const uint32_t (&pi)[8]) {
            GradOps o;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const u32x4 w4 = {aw[4 * m], aw[4 * m + 1], aw[4 * m + 2], aw[4 * m + 3]};
                const u32x4 a4 = {pr[4 * m], pr[4 * m + 1], pr[4 * m + 2], pr[4 * m + 3]};
                const u32x4 b4 = {pi[4 * m], pi[4 * m + 1], pi[4 * m + 2], pi[4 * m + 3]};
                o.ab[m] = as_bf16x8(w4);
                o.prb[m] = as_bf16x8(a4);
                o.pib[m] = as_bf16x8(b4);
                o.pnb[m] = as_bf16x8(b4 ^ 0x80008000u);
            }
            return o;
        };
        // gradient products of step j (query half m = j / 2, channel tile ct = j % 2):
        // dV^T += G'^T (w/l);  dK^T: Re += Q_r P_r + Q_i P_i,  Im += Q_i P_r - Q_r P_i
        auto grad_step = [&](const char *st, int sb, int j, const GradOps &w) {
            const int m = j >> 1, ct = j & 1;
            const char *b = st + (32 * sb + 16 * m) * ROWB;
            const int lo = off.voff[ct], hi = off.voffh[ct];
            const bf16x8 grt = tr_operand_b(b + 2 * REGION, lo, hi);
            const bf16x8 git = tr_operand_b(b + 3 * REGION, lo, hi);
            dv[ct] = mfma(grt, w.ab[m], dv[ct]);
            dv[2 + ct] = mfma(git, w.ab[m], dv[2 + ct]);
            const bf16x8 qrt = tr_operand_b(b, lo, hi);
            const bf16x8 qit = tr_operand_b(b + REGION, lo, hi);
            dk[ct] = mfma(qrt, w.prb[m], dk[ct]);
            dk[ct] = mfma(qit, w.pib[m], dk[ct]);
            dk[2 + ct] = mfma(qit, w.prb[m], dk[2 + ct]);
            dk[2 + ct] = mfma(qrt, w.pnb[m], dk[2 + ct]);
        };
        auto query_block = [&](const char *st, const float *sc, int sb, int qb0, bool masked,
                               int lo, int hi) {
            f32x16 sr = f32x16{}, si = f32x16{}, e = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) score_step(st, sb, kk, sr, si, e);
            uint32_t aw[8], pr[8], pi[8];
#pragma unroll
            for (int g = 0; g < 4; ++g)
                weight_group(sc, sb, g, masked, lo, hi, sr, si, e, aw, pr, pi, qb0);
            const GradOps w = grad_ops(aw, pr, pi);
#pragma unroll
            for (int j = 0; j < 4; ++j) grad_step(st, sb, j, w);
        };
        // both blocks of a stage with no mask: block 1's score products run
        // beside block 0's weight arithmetic, and block 0's gradient products
        // beside block 1's weight arithmetic
        auto full_stage = [&](const char *st, const float *sc, int qbase) {
            f32x16 sr0 = f32x16{}, si0 = f32x16{}, e0 = f32x16{};
            f32x16 sr1 = f32x16{}, si1 = f32x16{}, e1 = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) score_step(st, 0, kk, sr0, si0, e0);
            uint32_t aw0[8], pr0[8], pi0[8], aw1[8], pr1[8], pi1[8];
            // Issue is in order: a run of products holds the vector
            // instructions behind it. The scheduling groups below ask for the
            // two streams to alternate, one product then four vector
            // instructions, with each step's LDS reads ahead of its products
            // (the scheduler follows the pattern only in part).
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                score_step(st, 1, 2 * g, sr1, si1, e1);
                score_step(st, 1, 2 * g + 1, sr1, si1, e1);
                weight_group(sc, 0, g, false, 0, 31, sr0, si0, e0, aw0, pr0, pi0, qbase);
            }
            const GradOps w0 = grad_ops(aw0, pr0, pi0);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // product
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // vector ALU
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                grad_step(st, 0, j, w0);
                weight_group(sc, 1, j, false, 0, 31, sr1, si1, e1, aw1, pr1, pi1, qbase + 32);
            }
            const GradOps w1 = grad_ops(aw1, pr1, pi1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // LDS reads
#pragma unroll
                for (int i = 0; i < 6; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 4; ++j) grad_step(st, 1, j, w1);
        };

        const int qs = p.causal ? k0 : 0;   // earlier queries see none of these keys
        const int nstages = qs < T ? (T - qs + BS - 1) / BS : 0;
        auto issue_stage = [&](int s) {
            const uint32_t base = lds0 + (uint32_t)((s & 1) * KREG * REGION);
#pragma unroll
            for (int r = 0; r < KREG; ++r)
                stage_region<NT>(base + r * REGION, stage_planes[r], qs + s * BS, T, tid, wave);
            scal_issue(qs + s * BS, s & 1);
        };

        loads_done_barrier();   // the previous key tile is done with both buffers
        if (nstages > 0) {
            issue_stage(0);
        }
        // One stage: wait for it, issue the next one, run its two query blocks.
        // ALL_FULL drops the mask and skip branches (see below).
        auto stage = [&](int s, bool all_full) {
            loads_done_barrier();   // stage s and its scalars are visible
            const bool next = s + 1 < nstages;
            if (next) {
                issue_stage(s + 1);
            }
            const char *st = lds + (s & 1) * KREG * REGION;
            const float *sc = scal[s & 1];
            if (all_full) full_stage(st, sc, qs + s * BS);
#pragma unroll
            for (int sb = 0; sb < BS / 32; ++sb) {
                if (all_full) continue;
                const int qb0 = qs + s * BS + 32 * sb;
                const bool skip = qb0 >= T || kw0 >= T || (p.causal && qb0 + 31 < kw0);
                const bool full = (!p.causal || qb0 >= kw0 + 31) && qb0 + 32 <= T && kw0 + 32 <= T;
                if (full) {
                    query_block(st, sc, sb, qb0, false, 0, 31);
                } else if (!skip) {
                    const int lo = p.causal ? key - qb0 : 0;
                    const int hi = key < T ? T - 1 - qb0 : -1;
                    query_block(st, sc, sb, qb0, true, lo, hi);
                }
            }
        };
        // Stages [s_lo, s_hi) hold only queries inside T that see every key of
        // the tile (causal: at least BT - 1 past its first key), so they run in
        // a loop with no mask or skip branch and the accumulators stay in
        // place. A lane whose key is past T has zero K' and V' there, so its
        // sums stay zero, and it stores nothing.
        const int s_lo = min(p.causal ? (BT - 1 + BS - 1) / BS : 0, nstages);
        const int s_hi = max(s_lo, nstages > 0 ? (T - qs) / BS : 0);
        int s = 0;
        for (; s < s_lo; ++s) stage(s, false);
        for (; s < s_hi; ++s) stage(s, true);
        for (; s < nstages; ++s) stage(s, false);
        if (key < T) {
#pragma unroll
            for (int c = 0; c < 4; ++c) dk[c] *= 2.f;   // the weights carried half of dL/ds
            store_rows(reinterpret_cast<uint16_t *>(p.dk_re) + head, reinterpret_cast<uint16_t *>(p.dk_im) + head,
                       key, h, dk);
            store_rows(reinterpret_cast<uint16_t *>(p.dv_re) + head, reinterpret_cast<uint16_t *>(p.dv_im) + head,
                       key, h, dv);
        }
    }
}

}  // namespace

bool supports_born_bf16_d64_bwd(const BwdProblem &p) {
    return p.op == OP_BORN && p.layout == LAYOUT_BF16 && p.d == D;
}

hipError_t launch_born_bf16_d64_bwd_dq(const BwdProblem &p) {
    const int nrb = (p.T + QBT - 1) / QBT;
    const int nwork = p.causal ? (nrb + 1) / 2 : nrb;
    const int64_t blocks = (int64_t)p.BH * nwork;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    auto kern = p.decay.on ? born_bf16_d64_bwd_dq_kernel<true> : born_bf16_d64_bwd_dq_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(QNT), 0, p.stream, p, nrb, nwork);
    return hipGetLastError();
}

hipError_t launch_born_bf16_d64_bwd_dkdv(const BwdProblem &p) {
    const int64_t rows = (int64_t)p.BH * p.T;
    if (rows > 0) {
        if ((rows + 63) / 64 > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(born_bf16_d64_bwd_scal_kernel, dim3((unsigned)((rows + 63) / 64)), dim3(256), 0, p.stream, p,
                           rows);
    }
    const int nkt = (p.T + BT - 1) / BT;
    const int nwork = p.causal ? (nkt + 1) / 2 : nkt;
    const int64_t blocks = (int64_t)p.BH * nwork;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    auto kern = p.decay.on ? born_bf16_d64_bwd_dkdv_kernel<true> : born_bf16_d64_bwd_dkdv_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p, nkt, nwork);
    return hipGetLastError();
}

}  // namespace cattn
