// Born-rule attention forward at head width Q16_D (128 or 32), bf16
// real/imaginary planes, gfx950 matrix cores (v_mfma_f32_16x16x32_bf16) with
// fp32 accumulation.  Included once per width by kernel_born_bf16_q16*.hip,
// each defining Q16_D first.
//
// Operator ("CNet: A Complex-Valued Deep Learning Framework ...", section
// 11.2, "Closing it: Born-rule attention", Figure 2): w = |<q, k>|^2 and the
// output row is sum_j w_j v_j / (sum_j w_j + eps), in one pass with no running
// maximum (the weights are never negative).
//
// Why tiles of 16 queries.  At width 128 a tile of 32 queries needs 128 fp32
// output accumulators and 64 registers of query operands per lane: one wave
// per SIMD.  With 16 queries per wave the output takes 64 registers, Q' 32
// and -Re Q 16, so two waves per SIMD fit in 256 registers with no
// accumulation registers to copy scores out of.
//
// Products, 16 x 16 x 32 (A row i = lane % 16 with k = 8 (lane / 16) .. + 7,
// B column j = lane % 16 with the same k, result rows 4 (lane / 16) + r of
// column j).  Scores are formed transposed, keys along the rows:
//     Re S^T = K' [Re Q | Im Q]^T,   Im S^T = K' [Im Q | -Re Q]^T,
// K' = [Re K | Im K] from LDS, 8 steps of 32 real channels, for the two
// 16-key tiles of a 32-key block.  Lane (j, g) ends with keys 4 g + r of both
// tiles for its query j: packed to bf16, these 8 weights are already its B
// operand of
//     O^T += [Re V | Im V]^T W^T,
// with the block's keys taken in the order 4 g .. 4 g + 3, 16 + 4 g ..
// 16 + 4 g + 3 for k = 8 g .. 8 g + 7.  The V^T operand takes the same order
// from the row-major V tile through two transposing LDS reads
// (ds_read_b64_tr_b16: lane i of a 16-lane group receives column i of a
// 4 x 16 block), one for keys 4 g .., one for 16 + 4 g ...  Output tile c then
// holds four consecutive channels of the lane's query in rows 4 g + r.
//
// LDS.  A stage of 64 keys holds four 16 KiB regions (Re K, Im K, Re V, Im V),
// rows of 256 bytes = 16 chunks of 16 bytes, chunk c of row r stored at slot
// c ^ swz(r): at width 128 K takes swz = r mod 16, so the 16 rows that one
// operand read touches at one chunk fall on 16 distinct slots, and V takes
// swz = 2 (r mod 8), so the 8 rows x 2 chunks of two groups' transposing reads
// fall on 16 distinct slots; at width 32 (4 chunks a row, four rows to a
// 256-byte bank window) K takes h = ((r >> 1) ^ (r >> 2)) mod 4 and V 2 (h mod 2).  Stages go from global memory straight into LDS (buffer
// loads to LDS: each lane's 16 bytes land at base + 16 lane, so the swizzle is
// applied by choosing which chunk a lane fetches).  Rows past T read as zero.
// Two stage buffers, each its own LDS variable named at compile time: the
// loads of stage s + 1 are issued when stage s begins and are the only ones in
// flight while it runs, so the compiler knows they never touch the buffer
// being read and holds no read back for them.
//
// Pipeline.  A stage is two 32-key blocks.  When neither needs a mask, the
// second block's score products run beside the first block's weights, and
// the first block's value product beside the second block's weights (one
// stretch of code, so the matrix products fill the vector work's gaps).
//
// Work split.  8 waves (two per SIMD at width 128, four at 32), 16 queries each: row blocks of 128
// queries.  Causal: a workgroup takes the mirrored row blocks nrb-1-i and i,
// so every workgroup carries the same number of key blocks.  All items of a
// head go to one XCD when BH % 8 == 0 (workgroups are dealt to the XCDs in
// turn), so its K and V stay in that XCD's L2.  A 32-key block entirely below
// a wave's queries runs without mask arithmetic, one that crosses the
// diagonal or T is masked, one above the wave's last query is skipped.
//
// Born options, in instances of their own: decay multiplies each weight by
// gamma^(k - j) (formed per weight); rotary Q rotates each query operand as it
// is loaded, with the arithmetic of the rotary pass (rotary_math.h).
#ifndef Q16_D
#error "define Q16_D (the head width) before including this file"
#endif
#include "cattn_internal.h"
#include "rotary_math.h"

namespace cattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4v __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int D = Q16_D;
static_assert(D == 128 || D == 32, "widths 128 and 32");
constexpr int NW = 8;                 // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int QT = 16;                // queries per wave
constexpr int BM = QT * NW;           // query rows per row block
constexpr int BN = 64;                // keys per stage: two blocks of two 16-key tiles
constexpr int ROWB = 2 * D;           // bytes per row of one plane region
constexpr int REGION = BN * ROWB;     // 16 KiB
constexpr int STAGE = 4 * REGION;     // Re K, Im K, Re V, Im V
constexpr int TILEB = 16 * ROWB;      // bytes of 16 rows
constexpr int BLKB = 32 * ROWB;       // bytes of a 32-key block
constexpr int KSTEPS = 2 * D / 32;    // score k-steps of 32 real channels
constexpr int KH = KSTEPS / 2;        // k-steps per plane
constexpr int CT = 2 * D / 16;        // 16-channel tiles of O^T (Re, then Im)
constexpr int CH = CT / 2;            // tiles per plane
constexpr int NBUF = 2;               // stage buffers
constexpr int NCR = ROWB / 16;        // 16-byte chunks per row
constexpr int RPL = 1024 / ROWB;      // rows of one wave-wide load (64 lanes x 16 bytes)
constexpr int LPR = REGION / 1024;    // wave-wide loads per region
constexpr int LPW = 4 * LPR / NW;     // wave-wide loads per wave and stage
constexpr int NP = LPR > NW ? LPR / NW : 1;   // period in i of load i's rows
constexpr int WPE = D >= 128 ? 2 : 4;         // waves per SIMD
static_assert(LPW * NW == 4 * LPR, "whole loads per wave");

// gfx9 raw-buffer descriptor format word (dword 3)
constexpr int RSRC_WORD3 = 0x00020000;

__device__ inline int swz_k(int row) {
    if constexpr (D == 128) return row & 15;
    else return ((row >> 1) ^ (row >> 2)) & 3;
}
__device__ inline int swz_v(int row) {
    if constexpr (D == 128) return (row & 7) << 1;
    else return (((row >> 1) ^ (row >> 2)) & 1) << 1;
}

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ inline u32x2 ds_read_tr(const char *ptr) {
    const bf16x4v r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4v *)(ptr));
    return __builtin_bit_cast(u32x2, r);
}

__device__ inline f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <bool DECAY, bool ROT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void born_bf16_q16_kernel(Problem p, int nrb, int nwork) {
    __shared__ __align__(16) char buf0[STAGE];
    __shared__ __align__(16) char buf1[STAGE];
    char *const bufs[NBUF] = {buf0, buf1};
    // ROT: theta_m of the D channels
    __shared__ double rtheta[D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int j16 = lane & 15;
    const int g = lane >> 4;
    const int T = p.T;

    // Workgroup -> (head, work item)
    const int L = blockIdx.x;
    int bh, item;
    if ((p.BH & 7) == 0) {
        const int x = L & 7, j = L >> 3;
        bh = x + 8 * (j / nwork);
        item = j % nwork;
    } else {
        bh = L / nwork;
        item = L % nwork;
    }
    const int64_t hq = head_offset(p.sq, bh, p.H), hk = head_offset(p.sk, bh, p.H);
    const int64_t hv = head_offset(p.sv, bh, p.H), ho = head_offset(p.so, bh, p.H);
    const int64_t tq = p.sq.t, to = p.so.t;
    const uint16_t *qre = reinterpret_cast<const uint16_t *>(p.q_re) + hq;
    const uint16_t *qim = reinterpret_cast<const uint16_t *>(p.q_im) + hq;
    const char *planes[4] = {reinterpret_cast<const char *>(reinterpret_cast<const uint16_t *>(p.k_re) + hk),
                             reinterpret_cast<const char *>(reinterpret_cast<const uint16_t *>(p.k_im) + hk),
                             reinterpret_cast<const char *>(reinterpret_cast<const uint16_t *>(p.v_re) + hv),
                             reinterpret_cast<const char *>(reinterpret_cast<const uint16_t *>(p.v_im) + hv)};
    uint16_t *ore = reinterpret_cast<uint16_t *>(p.o_re) + ho;
    uint16_t *oim = reinterpret_cast<uint16_t *>(p.o_im) + ho;

    // ---- staging: global -> LDS, no registers ------------------------------
#if Q16_D == 128
    // Load h (0, 1) of lane (j16, g) of wave w covers row 8 w + 4 h + g of
    // each region and physical slot j16, and fetches logical chunk
    // j16 ^ swz(row) of that row.  The descriptor's base is the stage's first
    // key row and its extent ends at row T; each lane adds a 32-bit offset
    // below 64 rows.
    const int64_t rbk = 2 * p.sk.t, rbv = 2 * p.sv.t;   // bytes from one key row to the next
    uint32_t offk[2], offv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int srow = 8 * wave + 4 * h + g;
        offk[h] = (uint32_t)(srow * rbk) + 16u * (uint32_t)(j16 ^ swz_k(srow));
        offv[h] = (uint32_t)(srow * rbv) + 16u * (uint32_t)(j16 ^ swz_v(srow));
    }
    // live = false: an extent of 0, so the loads touch no memory (they fill
    // the buffer with zeros).
    auto dma_stage = [&](int k0, char *buf, bool live) {
        char *dst = buf + wave * 2048;
        const int64_t left = live ? T - k0 : 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t rb = r < 2 ? rbk : rbv;
            const int64_t ext = left * rb;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(planes[r] + (int64_t)k0 * rb), 0, (int)(uint32_t)(ext < 0xffffffffll ? ext : 0xffffffffll),
                RSRC_WORD3);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(dst + r * REGION + h * 1024), 16,
                                                         r < 2 ? offk[h] : offv[h], 0, 0, 0);
        }
    };
#else
    // Wave-wide load i of wave w is load L = NW i + w of the stage: region
    // L / LPR (Re K, Im K, Re V, Im V), rows RPL (L mod LPR) .. of it, one
    // 1 KiB stretch of LDS.  Lane l covers row RPL (L mod LPR) + l / NCR and
    // physical slot l mod NCR, and fetches logical chunk slot ^ swz(row) of
    // that row.  The rows of load i repeat with period NP in i: one K and one
    // V offset per residue.  The descriptor's base is the stage's first key
    // row and its extent ends at row T; each lane adds a 32-bit offset below
    // 64 rows.
    const int64_t rbk = 2 * p.sk.t, rbv = 2 * p.sv.t;   // bytes from one key row to the next
    uint32_t offk[NP], offv[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int L = NW * i + wave;
        const int row = RPL * (L % LPR) + lane / NCR, slot = lane % NCR;
        offk[i] = (uint32_t)(row * rbk) + 16u * (uint32_t)(slot ^ swz_k(row));
        offv[i] = (uint32_t)(row * rbv) + 16u * (uint32_t)(slot ^ swz_v(row));
    }
    // live = false: an extent of 0, so the loads touch no memory (they fill
    // the buffer with zeros).
    auto dma_stage = [&](int k0, char *buf, bool live) {
        const int64_t left = live ? T - k0 : 0;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int L = NW * i + wave, r = L / LPR;
            const int64_t rb = r < 2 ? rbk : rbv;
            const int64_t ext = left * rb;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(planes[r] + (int64_t)k0 * rb), 0, (int)(uint32_t)(ext < 0xffffffffll ? ext : 0xffffffffll),
                RSRC_WORD3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(buf + r * REGION + (L % LPR) * 1024), 16,
                                                     r < 2 ? offk[i % NP] : offv[i % NP], 0, 0, 0);
        }
    };
#endif

    // ---- per-lane LDS read offsets ----------------------------------------
    // K' A operand, block sb, k-step ks, tile kt: row 32 sb + 16 kt + j16,
    // logical chunk 4 (ks % KH) + g of the Re K (ks < KH) or Im K region.
    int koff[KH];
#pragma unroll
    for (int i = 0; i < KH; ++i) koff[i] = j16 * ROWB + 16 * ((4 * i + g) ^ swz_k(j16));
    // V^T A operand of channel tile c (16 channels of the Re V or Im V region
    // from 16 (c % CH)): lane 4 r + c4 of group g points at row 4 g + r,
    // channels 16 (c % CH) + 4 c4 .. + 3, i.e. logical chunk 2 (c % CH) + c4 / 2,
    // half c4 % 2, of block sb; the second read is 16 rows further.
    int voff[CH];
    {
        const int r = (lane >> 2) & 3, c4 = lane & 3;
        const int row = 4 * g + r;
#pragma unroll
        for (int m = 0; m < CH; ++m) voff[m] = row * ROWB + 16 * ((2 * m + (c4 >> 1)) ^ swz_v(row)) + 8 * (c4 & 1);
    }

    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    const float lg2 = DECAY ? p.decay.lg2[bh % p.H] : 0.f;

    // ---- query operands -----------------------------------------------------
    // k-step ks, lane (query j16, group g): Q'[q][32 ks + 8 g .. + 8], i.e.
    // channels 32 (ks % KH) + 8 g .. of Re Q (ks < KH) or Im Q; qn = -Re Q.
    bf16x8 qb[KSTEPS], qn[KH];
    auto load_q = [&](int qt0) {
        const int q = qt0 + j16;
        u32x4 x[KSTEPS];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            x[ks] = u32x4{0u, 0u, 0u, 0u};
            if (q < T) {
                const uint16_t *src = (ks < KH ? qre : qim) + (int64_t)q * tq + 32 * (ks % KH) + 8 * g;
                x[ks] = *reinterpret_cast<const u32x4 *>(src);
            }
        }
        if (ROT && q < T) {
            // (Re, Im) of channel 32 ks + 8 g + e: element e of chunks ks and ks + KH
            const double pos = (double)(p.rot_pos0 + q);
#pragma unroll
            for (int ks = 0; ks < KH; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int sh = 16 * (e & 1);
                    const uint32_t rw = x[ks][e >> 1], iw = x[ks + KH][e >> 1];
                    float c, sn, yr, yi;
                    rotary_phase(pos, rtheta[32 * ks + 8 * g + e], c, sn);
                    rotary_apply(__uint_as_float(((rw >> sh) & 0xffffu) << 16),
                                 __uint_as_float(((iw >> sh) & 0xffffu) << 16), c, sn, yr, yi);
                    x[ks][e >> 1] = (rw & ~(0xffffu << sh)) | ((uint32_t)rotary_bf16(yr) << sh);
                    x[ks + KH][e >> 1] = (iw & ~(0xffffu << sh)) | ((uint32_t)rotary_bf16(yi) << sh);
                }
        }
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) qb[ks] = as_bf16x8(x[ks]);
#pragma unroll
        for (int ks = 0; ks < KH; ++ks) qn[ks] = as_bf16x8(x[ks] ^ 0x80008000u);
    };

    f32x4 oacc[CT];
    // the row sum of the packed weights in four independent partial sums
    float rsum[4];

    // Score products of 32-key block sb of stage buffer st.
    auto scores = [&](const char *st, int sb, f32x4 (&sr)[2], f32x4 (&si)[2]) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sr[kt] = si[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(st + (ks / KH) * REGION + sb * BLKB + kt * TILEB +
                                                                   koff[ks % KH]);
                sr[kt] = mfma(a, qb[ks], sr[kt]);
                si[kt] = mfma(a, ks < KH ? qb[ks + KH] : qn[ks - KH], si[kt]);
            }
    };
    // The block's weights (first key kb0; the wave's first query qt0), packed
    // to bf16 as the B operand of its value product and added to the row sums.
    // Register r of tile kt is key kb0 + 16 kt + 4 g + r.  masked: keys above
    // the query or at or past T get weight 0.
    auto weights = [&](const f32x4 (&sr)[2], const f32x4 (&si)[2], int kb0, int qt0, bool masked) {
        const int q = qt0 + j16;
        uint32_t pk[4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int rp = 0; rp < 2; ++rp) {
                const int r = 2 * rp;
                float w0 = sr[kt][r] * sr[kt][r] + si[kt][r] * si[kt][r];
                float w1 = sr[kt][r + 1] * sr[kt][r + 1] + si[kt][r + 1] * si[kt][r + 1];
                const int key0 = kb0 + 16 * kt + 4 * g + r;
                if (DECAY) {   // distances are >= 0 where the mask keeps the weight
                    w0 *= decay_pow(lg2, max(q - key0, 0));
                    w1 *= decay_pow(lg2, max(q - key0 - 1, 0));
                }
                if (masked) {
                    const int lim = min(p.causal ? q : T - 1, T - 1);
                    w0 = key0 > lim ? 0.f : w0;
                    w1 = key0 + 1 > lim ? 0.f : w1;
                }
                pk[2 * kt + rp] = pack_bf16x2(w0, w1);
                rsum[2 * kt + rp] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[2 * kt + rp]), ones,
                                                                    rsum[2 * kt + rp], false);
            }
        return as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
    };
    // The value product of block sb: its packed weights wop against its V
    // tile in stage buffer st.
    auto values = [&](const char *st, int sb, bf16x8 wop) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const char *vb = st + (2 + c / CH) * REGION + sb * BLKB + voff[c % CH];
            const u32x2 lo = ds_read_tr(vb);
            const u32x2 hi = ds_read_tr(vb + TILEB);
            oacc[c] = mfma(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), wop, oacc[c]);
        }
    };
    // ---- the workgroup's row blocks and their key stages --------------------
    const int nblocks = p.causal && item != nrb - 1 - item ? 2 : 1;
    auto row_block = [&](int blk) { return p.causal ? (blk == 0 ? nrb - 1 - item : item) : item; };
    auto stages_of = [&](int blk) {
        const int kend = p.causal ? min(T, row_block(blk) * BM + BM) : T;
        return (kend + BN - 1) / BN;
    };
    const int nst0 = stages_of(0);
    const int nst1 = nblocks > 1 ? stages_of(1) : 0;
    const int total = nst0 + nst1;
    // the workgroup's stages form one stream, row blocks in order; stage gs
    // lives in buffer gs % 2
    auto stage_k0 = [&](int gs) { return (gs < nst0 ? gs : gs - nst0) * BN; };

    auto epilogue = [&](int qt0) {
        const float rs = (rsum[0] + rsum[1]) + (rsum[2] + rsum[3]);
        const float r2 = rs + __shfl_xor(rs, 16);
        const float den = (r2 + __shfl_xor(r2, 32)) + p.eps;   // the four lane groups hold this query
        const float inv = den != 0.f ? 1.f / den : 0.f;
        const int q = qt0 + j16;
        if (q < T) {
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                const int col = 16 * (c % CH) + 4 * g;   // channel of row 4 g in its plane
                const u32x2 v = {pack_bf16x2(oacc[c][0] * inv, oacc[c][1] * inv),
                                 pack_bf16x2(oacc[c][2] * inv, oacc[c][3] * inv)};
                *reinterpret_cast<u32x2 *>((c < CH ? ore : oim) + (int64_t)q * to + col) = v;
            }
            if (p.row_den && g == 0) p.row_den[(int64_t)bh * T + q] = den;
        }
    };

    // One stage: every wave's loads of it have landed and every wave is past
    // the previous stage (whose buffer the loads of stage gs + 1 now fill).
    auto step = [&](auto J, int gs) {
        constexpr int j = decltype(J)::value;
        __asm__ __volatile__("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
        __builtin_amdgcn_s_barrier();
        __asm__ __volatile__("" ::: "memory");
        const int blk = gs < nst0 ? 0 : 1;
        const int s = gs - (blk ? nst0 : 0);
        const int qt0 = row_block(blk) * BM + QT * wave;
        if (s == 0) {
            // before the stage loads, so that waiting for Q leaves them in flight
            load_q(qt0);
#pragma unroll
            for (int c = 0; c < CT; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
            rsum[0] = rsum[1] = rsum[2] = rsum[3] = 0.f;
        }
        dma_stage(stage_k0(gs + 1), bufs[(j + 1) % NBUF], gs + 1 < total);
        const char *st = bufs[j];
        const int kb0 = s * BN;
        bool skip[2], full[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int kb = kb0 + 32 * sb;
            skip[sb] = qt0 >= T || kb >= T || (p.causal && kb > qt0 + QT - 1);
            full[sb] = (!p.causal || kb + 31 <= qt0) && kb + 32 <= T;
        }
        if (full[0] && full[1]) {
            f32x4 sr0[2], si0[2], sr1[2], si1[2];
            scores(st, 0, sr0, si0);
            const bf16x8 w0 = weights(sr0, si0, kb0, qt0, false);
            scores(st, 1, sr1, si1);
            values(st, 0, w0);
            const bf16x8 w1 = weights(sr1, si1, kb0 + 32, qt0, false);
            values(st, 1, w1);
        } else {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                if (!skip[sb]) {
                    f32x4 sr[2], si[2];
                    scores(st, sb, sr, si);
                    const bf16x8 w = full[sb] ? weights(sr, si, kb0 + 32 * sb, qt0, false)
                                              : weights(sr, si, kb0 + 32 * sb, qt0, true);
                    values(st, sb, w);
                }
            }
        }
        if (s == (blk ? nst1 : nst0) - 1) epilogue(qt0);
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    if (ROT) {
        if (tid < D) rtheta[tid] = rotary_theta(tid, p.rot_log_base, D);
        __syncthreads();
    }
    dma_stage(stage_k0(0), buf0, total > 0);
    for (int gs = 0; gs < total; gs += NBUF) {
        // The read offsets are loop-invariant, and so is every address of a
        // statically named buffer: left alone, the compiler holds one register
        // per address across the loop.  Made opaque here, they are formed
        // inside the loop, with the constant part in the instruction's offset.
#pragma unroll
        for (int i = 0; i < KH; ++i) __asm__ __volatile__("" : "+v"(koff[i]));
#pragma unroll
        for (int m = 0; m < CH; ++m) __asm__ __volatile__("" : "+v"(voff[m]));
        step(I0{}, gs);
        if (gs + 1 < total) step(I1{}, gs + 1);
    }
    // Loads past the stream's end (extent 0) still write zeros into LDS: let
    // them land before the workgroup's LDS can be handed to another.
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
}

}  // namespace

template <>
bool supports_born_bf16_q16<D>(const Problem &p) {
    return p.op == OP_BORN && p.layout == LAYOUT_BF16 && p.d == D && p.aligned16;
}

template <>
hipError_t launch_born_bf16_q16<D>(const Problem &p) {
    const int nrb = (p.T + BM - 1) / BM;
    const int nwork = p.causal ? (nrb + 1) / 2 : nrb;   // causal: mirrored pairs of row blocks
    const int64_t blocks = (int64_t)p.BH * nwork;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    auto kern = p.decay.on ? (p.rot ? born_bf16_q16_kernel<true, true> : born_bf16_q16_kernel<true, false>)
                           : (p.rot ? born_bf16_q16_kernel<false, true> : born_bf16_q16_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p, nrb, nwork);
    return hipGetLastError();
}

}  // namespace cattn
