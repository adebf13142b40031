// Born-rule attention forward, head width 64, bf16 real/imaginary planes,
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
//
// Operator ("CNet: A Complex-Valued Deep Learning Framework ...", section
// 11.2, "Closing it: Born-rule attention", Figure 2): w = |<q, k>|^2, and the
// output row is sum_j w_j v_j / (sum_j w_j + eps).  The weights are never
// negative, so one pass carries the numerator and the denominator side by side
// with no running maximum and no rescaling.
//
// Products.  With Q' = [Re Q | Im Q], K' = [Re K | Im K] (128 real columns)
//     Re S^T = K' [Re Q | Im Q]^T,   Im S^T = K' [Im Q | -Re Q]^T
// share the A operand K' (read from LDS); both Q operands stay in registers.
// Scores are formed transposed, keys along MFMA rows, so each lane ends up
// with one query and 16 keys: after w = Re^2 + Im^2 and packing to bf16 that
// is already the B operand of
//     O^T += [Re V | Im V]^T W^T.
// The V^T operand comes straight from the row-major V tile in LDS through the
// transposing LDS read (ds_read_b64_tr_b16): each 16-lane group receives the
// columns of a 4 x 16 block, so nothing is transposed while staging.
//
// LDS.  A stage of 64 keys holds four 8 KiB regions (Re K, Im K, Re V, Im V),
// rows of 128 bytes = eight 16-byte chunks, chunk c of row r stored at slot
// c ^ swz(r).  The K swizzle spreads the 32 rows read by one A operand fetch
// over all banks; the V swizzle does the same for the 4-key x 2-chunk
// footprint of a transposing read.  Stages go from global memory straight
// into LDS (global_load_lds_dwordx4: each lane's 16 bytes land at base +
// 16 * lane, so the swizzle is applied by choosing which chunk a lane fetches),
// into two stage buffers that alternate: the loads of stage s + 1 are in
// flight while stage s is multiplied.  The two buffers are separate LDS
// variables, which lets the compiler see that the transposing reads of one
// never alias the loads into the other.
//
// Work split.  A workgroup of 8 waves (two per SIMD) covers row blocks of
// 256 queries of one (batch, head), one 32-query tile per wave.  For causal
// attention a workgroup takes the mirrored pair of row blocks nrb-1-i and i,
// so every workgroup carries the same number of key blocks and the grid
// drains evenly.  Key blocks of 32 strictly below a tile's diagonal take a
// path with no mask arithmetic; the diagonal block (and a ragged tail) is
// masked; blocks above the diagonal are skipped.
//
// Born options, in instances of their own (the plain kernel carries none of
// their registers).  Decay (causal): the weight of key j for query k is
// multiplied by gamma^(k - j).  On a full block the distance of register r
// (key 8 (r/4) + 4 h + r%4 of the block) splits into a part fixed per lane,
// block and group of four registers (query offset, lane half, block start,
// r/4) and a part fixed per register within its group (r%4):
// gamma^(k - j) = mu[r/4] * sigma[r%4], all at most 1 on a full block; mu is
// formed per block and lane (four exponentials), sigma once per kernel, so
// each weight takes two extra multiplies.  Masked blocks
// form gamma^(k - j) per weight.  Rotary Q: each query operand is rotated as it is loaded (the
// arithmetic of the rotary pass, rotary_math.h), with the channel
// frequencies in a small LDS table formed once per workgroup.
#include "cattn_internal.h"
#include "rotary_math.h"



namespace cattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4v __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

constexpr int D = 64;
constexpr int NW = 8;                 // waves per workgroup, two per SIMD
constexpr int NT = 64 * NW;
constexpr int BM = 32 * NW;           // query rows per row block
constexpr int BN = 64;                // keys per stage
constexpr int ROWB = 2 * D;           // bytes per row of one plane region
constexpr int REGION = BN * ROWB;     // 8 KiB
constexpr int STAGE = 4 * REGION;     // Re K, Im K, Re V, Im V
constexpr int NSB = BN / 32;          // 32-key blocks per stage
constexpr int RPT = REGION / 16 / NT; // 16-byte chunks per thread per region per stage
constexpr int LOADS_PER_T = 4 * RPT;  // LDS-direct loads per thread per stage
static_assert(RPT * 16 * NT == REGION, "staging split");

__device__ inline int swz_k(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }
__device__ inline int swz_v(int row) { return (row & 3) << 1; }

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ inline u32x2 ds_read_tr(const char *p) {
    const bf16x4v r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4v *)(p));
    return __builtin_bit_cast(u32x2, r);
}

// All of this wave's LDS-direct loads have landed; then workgroup barrier.  A
// bare s_barrier is used (the fence of __syncthreads adds nothing here).
__device__ inline void loads_done_barrier() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// gfx9 raw-buffer descriptor format word (dword 3)
constexpr int RSRC_WORD3 = 0x00020000;

template <bool DECAY, bool ROT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void born_bf16_d64_kernel(Problem p, int nrb, int nwork) {
    // Four stage buffers, each its own LDS variable: every access names its
    // buffer at compile time, so the compiler can tell the transposing and
    // operand reads of one buffer from the LDS-direct loads into another and
    // waits only for the loads a read depends on.
    __shared__ __align__(16) char buf0[STAGE];
    __shared__ __align__(16) char buf1[STAGE];
    __shared__ __align__(16) char buf2[STAGE];
    __shared__ __align__(16) char buf3[STAGE];
    char *const bufs[4] = {buf0, buf1, buf2, buf3};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int T = p.T;

    // Workgroup -> (head, work item).  When BH % 8 == 0 all items of a head go
    // to one XCD (workgroups are dealt to the 8 XCDs round-robin), so its K/V
    // stay in that XCD's L2.
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
    // head bases and token strides (elements) of each operand
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
    // Thread t covers key row t / 8 of the stage and physical chunk slot t % 8
    // of each region, and fetches logical chunk slot ^ swz(row) of that row.
    // A wave's 64 chunks of one region are 1 KiB of LDS.  Each plane's load is
    // a buffer load: the descriptor's base is the stage's first key row and
    // its extent ends at row T, so rows past T read as zero (zero keys carry
    // zero weight, zero values add nothing); each lane adds a 32-bit offset.
    const int srow = tid >> 3;
    const int sslot = tid & 7;
    const int64_t rbk = 2 * p.sk.t, rbv = 2 * p.sv.t;   // bytes from one key row to the next (K, V planes)
    const uint32_t offk = (uint32_t)(srow * rbk) + 16u * (uint32_t)(sslot ^ swz_k(srow));
    const uint32_t offv = (uint32_t)(srow * rbv) + 16u * (uint32_t)(sslot ^ swz_v(srow));

    // live = false: an extent of 0, so the loads touch no memory (they fill
    // the buffer with zeros); it keeps the caller free of branches.
    auto dma_stage = [&](int k0, char *buf, bool live) {
        char *dst = buf + wave * 1024;
        const int64_t left = live ? T - k0 : 0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int64_t rb = g < 2 ? rbk : rbv;
            const int64_t ext = left * rb;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(planes[g] + (int64_t)k0 * rb), 0, (int)(uint32_t)(ext < 0xffffffffll ? ext : 0xffffffffll),
                RSRC_WORD3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(dst + g * REGION), 16,
                                                     g < 2 ? offk : offv, 0, 0, 0);
        }
    };

    // ---- per-lane LDS read offsets ----------------------------------------
    // K' A operand, k-step kk: row 32 sb + l32, logical chunk 2 (kk % 4) + h.
    int koff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) koff[j] = l32 * ROWB + (((2 * j + h) ^ swz_k(l32)) << 4);
    // V^T A operand through the transposing read: lane 16 G + 4 r + c4 points
    // at key 4 h + r (+ block offsets), columns 16 (G & 1) + 4 c4 of the tile.
    int voff[2];
    {
        const int G = lane >> 4, r = (lane >> 2) & 3, c4 = lane & 3;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int lc = 4 * cc + 2 * (G & 1) + (c4 >> 1);
            voff[cc] = (4 * h + r) * ROWB + ((lc ^ (r << 1)) << 4) + ((c4 & 1) << 3);
        }
    }

    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // ---- the workgroup's row blocks and their key stages --------------------
    const int nblocks = p.causal && item != nrb - 1 - item ? 2 : 1;
    auto row_block = [&](int blk) { return p.causal ? (blk == 0 ? nrb - 1 - item : item) : item; };
    auto stages_of = [&](int blk) {
        const int kend = p.causal ? min(T, row_block(blk) * BM + BM) : T;
        return (kend + BN - 1) / BN;
    };
    const int nst0 = stages_of(0);
    const int nst1 = nblocks > 1 ? stages_of(1) : 0;
    // Stage s of a row block lives in buffer s % 4.  When the first row block
    // has a multiple of 4 stages the stream runs on into the second with no
    // break; otherwise (a ragged last row block) the second restarts it.
    const bool seamless = (nst0 & 3) == 0;
    // Loads of the workgroup's stage gs (row blocks in order) into buffer buf;
    // past the stream's end they load nothing.  A restarted stream loads the
    // second row block's first two stages itself, at the restart.
    auto dma_global = [&](int gs, char *buf) {
        const bool first = gs < nst0;
        const int s = first ? gs : gs - nst0;
        // no short-circuit evaluation: no branch inside the pipeline
        dma_stage(s * BN, buf, first | ((s < nst1) & (seamless | (s >= 2))));
    };
    // This wave's stage loads have landed, and every wave is past the barrier.
    auto stage_barrier = [&]() {
        __asm__ __volatile__("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
        __builtin_amdgcn_s_barrier();
        __asm__ __volatile__("" ::: "memory");
    };

    // Q operands (B operand of the score products): k-step kk, lane
    // (query l32, half h) holds Q'[q][16 kk + 8 h .. + 8].
    bf16x8 qb[8];
    // ROT: theta_m of the 64 channels
    __shared__ double rtheta[D];
    auto load_q = [&](int qt0) {
        const int q = qt0 + l32;
        u32x4 x[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            x[kk] = u32x4{0u, 0u, 0u, 0u};
            if (q < T) {
                const uint16_t *src = (kk < 4 ? qre : qim) + (int64_t)q * tq + 16 * (kk & 3) + 8 * h;
                x[kk] = *reinterpret_cast<const u32x4 *>(src);
            }
        }
        if (ROT && q < T) {
            // (Re, Im) of channel 16 kk + 8 h + e: element e of chunks kk and kk + 4
            const double pos = (double)(p.rot_pos0 + q);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int sh = 16 * (e & 1);
                    const uint32_t rw = x[kk][e >> 1], iw = x[kk + 4][e >> 1];
                    float c, sn, yr, yi;
                    rotary_phase(pos, rtheta[16 * kk + 8 * h + e], c, sn);
                    rotary_apply(__uint_as_float(((rw >> sh) & 0xffffu) << 16),
                                 __uint_as_float(((iw >> sh) & 0xffffu) << 16), c, sn, yr, yi);
                    x[kk][e >> 1] = (rw & ~(0xffffu << sh)) | ((uint32_t)rotary_bf16(yr) << sh);
                    x[kk + 4][e >> 1] = (iw & ~(0xffffu << sh)) | ((uint32_t)rotary_bf16(yi) << sh);
                }
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qb[kk] = as_bf16x8(x[kk]);
    };

    // DECAY: log2 gamma of the head, sigma[b] = gamma^(3 - b), and per row
    // block the lane's part of the exponent of mu (see the note at the top).
    const float lg2 = DECAY ? p.decay.lg2[bh % p.H] : 0.f;
    float sig[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        sig[b] = 1.f;
        if (DECAY) {
            const float x = decay_pow(lg2, 3 - b);
            sig[b] = x;
        }
    }
    int dq0 = 0;     // qt0 + l32 - 4 h - 3 of the current row block
    int gbase = 0;   // the workgroup's stage index of this row block's stage 0

    f32x16 oacc[4];
    // The row sum of the weights in four independent partial sums: one
    // accumulator would chain every pair's dot2 on the previous one, and at
    // that instruction's latency the chain stalls the wave (products included).
    float rsum[4];

    // -Re Q chunk kk: the second half of [Im Q | -Re Q], formed as it is
    // needed (one exclusive-or per register, in the issue slots between
    // products) rather than held in 16 more registers.
    auto neg_req = [&](int kk) { return as_bf16x8(__builtin_bit_cast(u32x4, qb[kk]) ^ 0x80008000u); };
    // Scores S^T of a block from K' operands held in registers.
    auto scores_reg = [&](const bf16x8 (&ka)[8], f32x16 &sr, f32x16 &si) {
        sr = f32x16{};
        si = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            sr = mfma(ka[kk], qb[kk], sr);
            si = mfma(ka[kk], kk < 4 ? qb[kk + 4] : neg_req(kk - 4), si);
        }
    };
    auto read_k = [&](const char *st, int sb, bf16x8 (&ka)[8]) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            ka[kk] = *reinterpret_cast<const bf16x8 *>(st + (kk >> 2) * REGION + sb * 32 * ROWB + koff[kk & 3]);
    };
    // The same products for the pipeline, with fewer live registers: the Re K
    // half of K' (k-steps 0-3) arrives prefetched; the Im K half is read here
    // and lands while the first eight products run.
    auto read_k_re = [&](const char *st, int sb, bf16x8 (&kre)[4]) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            kre[kk] = *reinterpret_cast<const bf16x8 *>(st + sb * 32 * ROWB + koff[kk]);
    };
    auto scores_pipe = [&](const char *st, int sb, const bf16x8 (&kre)[4], f32x16 &sr, f32x16 &si) {
        bf16x8 kim[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            kim[kk] = *reinterpret_cast<const bf16x8 *>(st + REGION + sb * 32 * ROWB + koff[kk]);
        sr = f32x16{};
        si = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            sr = mfma(kre[kk], qb[kk], sr);
            si = mfma(kre[kk], qb[kk + 4], si);
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            sr = mfma(kim[kk], qb[kk + 4], sr);
            si = mfma(kim[kk], neg_req(kk), si);
        }
    };
    // V^T operand halves of a block: vt[2 c + m] = (lo, hi) of output tile c, keys 16 m .. 16 m + 15
    auto read_v = [&](const char *st, int sb, u32x4 (&vt)[8]) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const char *vb = st + (2 + (c >> 1)) * REGION + (32 * sb + 16 * m) * ROWB + voff[c & 1];
                const u32x2 lo = ds_read_tr(vb);
                const u32x2 hi = ds_read_tr(vb + 8 * ROWB);
                vt[2 * c + m] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
    };
    // w = |S|^2 of one pair of keys packed to bf16, added to the row sum;
    // register r of lane half h is key 8 (r/4) + 4 h + r % 4.  DECAY: times
    // the factors f0, f1 of the two keys.
    auto weight_pair = [&](const f32x16 &sr, const f32x16 &si, int r, bool masked, int lim, float f0, float f1) {
        float w0 = sr[r] * sr[r] + si[r] * si[r];
        float w1 = sr[r + 1] * sr[r + 1] + si[r + 1] * si[r + 1];
        if (DECAY) {
            w0 *= f0;
            w1 *= f1;
        }
        if (masked) {
            const int key0 = 8 * (r >> 2) + 4 * h + (r & 3);
            w0 = key0 > lim ? 0.f : w0;
            w1 = key0 + 1 > lim ? 0.f : w1;
        }
        const uint32_t pk = pack_bf16x2(w0, w1);
        rsum[(r >> 1) & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), ones, rsum[(r >> 1) & 3], false);
        return pk;
    };
    // The value product of the previous block (operands vt, wprev) interleaved
    // with the weights of this block (scores sr, si -> wop): one product, then
    // the vector work of one pair of keys.
    // DECAY: kb0 is the block's first key (a full block: every factor <= 1).
    auto values_and_weights = [&](const u32x4 (&vt)[8], const bf16x8 (&wprev)[2], const f32x16 &sr,
                                  const f32x16 &si, bf16x8 (&wop)[2], int kb0) {
        float mu[4];   // gamma^(qt0 + l32 - kb0 - 8 a - 4 h - 3) for register group a
#pragma unroll
        for (int a = 0; a < 4; ++a) mu[a] = DECAY ? decay_pow(lg2, dq0 - kb0 - 8 * a) : 1.f;
        uint32_t pk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            oacc[i >> 1] = mfma(as_bf16x8(vt[i]), wprev[i & 1], oacc[i >> 1]);
            // registers 2 i, 2 i + 1: group i / 2, places 2 (i % 2) and 2 (i % 2) + 1
            pk[i] = weight_pair(sr, si, 2 * i, false, 31, mu[i >> 1] * sig[2 * (i & 1)],
                                mu[i >> 1] * sig[2 * (i & 1) + 1]);
        }
        wop[0] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
        wop[1] = as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]});
    };

    // Software pipeline over the key blocks of full stages (no mask: every
    // key of the stage is visible to every query of the row block).  Per block
    // b: the scores of b, the Re K reads of b + 1, the value product of b - 1
    // beside the weights of b, the V^T reads of b.  The stage's barrier sits
    // after the scores of its second block: past it the next stage is
    // readable, and the stage two ahead is loaded into the buffer that was
    // read two stages back.  Entry: ka holds K' of the stage's first block,
    // vt and wprev the previous block's value operands.
    bf16x8 ka[4];
    u32x4 vt[8];
    bf16x8 wprev[2];
    auto main_stage = [&](auto J, int gs) {
        constexpr int j = decltype(J)::value;
        const char *st = bufs[j];
        const int k0 = (gs - gbase) * BN;   // the stage's first key
        f32x16 sr, si;
        bf16x8 wop[2];
        // block 0
        scores_pipe(st, 0, ka, sr, si);
        read_k_re(st, 1, ka);
        values_and_weights(vt, wprev, sr, si, wop, k0);
        wprev[0] = wop[0];
        wprev[1] = wop[1];
        read_v(st, 0, vt);
        // block 1
        scores_pipe(st, 1, ka, sr, si);
        stage_barrier();
        dma_global(gs + 2, bufs[(j + 2) & 3]);
        read_k_re(bufs[(j + 1) & 3], 0, ka);   // the next stage's first block (unused past the last full stage)
        values_and_weights(vt, wprev, sr, si, wop, k0 + 32);
        wprev[0] = wop[0];
        wprev[1] = wop[1];
        read_v(st, 1, vt);
    };

    // Stages with a mask or skipped blocks (the causal diagonal region, a
    // ragged tail), one block after another straight from LDS; then the
    // stage's barrier and the loads two stages ahead.
    auto rest_stage = [&](auto J, int gs, int s, int qt0, bool wave_live) {
        constexpr int j = decltype(J)::value;
        const char *st = bufs[j];
        if (wave_live) {
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int kb0 = s * BN + 32 * sb;
                const bool skip = kb0 >= T || (p.causal && kb0 > qt0);
                const bool full = (!p.causal || kb0 + 32 <= qt0) && kb0 + 32 <= T;
                if (!skip) {
                    const int lim = full ? 31 : min(p.causal ? qt0 + l32 - kb0 : 31, T - 1 - kb0);
                    bf16x8 kb[8];
                    read_k(st, sb, kb);
                    f32x16 sr, si;
                    scores_reg(kb, sr, si);
                    u32x4 vb[8];
                    read_v(st, sb, vb);
                    bf16x8 wop[2];
                    uint32_t pk[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        // DECAY: gamma^(k - j) per weight; masked keys (negative distance) are zeroed
                        const int key0 = 8 * (i >> 1) + 4 * h + 2 * (i & 1);
                        const int n0 = qt0 + l32 - kb0 - key0;
                        const float f0 = DECAY ? decay_pow(lg2, max(n0, 0)) : 1.f;
                        const float f1 = DECAY ? decay_pow(lg2, max(n0 - 1, 0)) : 1.f;
                        pk[i] = weight_pair(sr, si, 2 * i, !full, lim, f0, f1);
                    }
                    wop[0] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
                    wop[1] = as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]});
#pragma unroll
                    for (int i = 0; i < 8; ++i) oacc[i >> 1] = mfma(as_bf16x8(vb[i]), wop[i & 1], oacc[i >> 1]);
                }
            }
        }
        stage_barrier();
        dma_global(gs + 2, bufs[(j + 2) & 3]);
    };

    // ---- the row blocks ---------------------------------------------------
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    if (ROT) {
        if (tid < D) rtheta[tid] = rotary_theta(tid, p.rot_log_base, D);
        __syncthreads();
    }
    load_q(row_block(0) * BM + 32 * wave);
    dma_stage(0, buf0, true);
    dma_stage(BN, buf1, nst0 > 1);
    stage_barrier();
    gbase = 0;
    for (int blk = 0; blk < nblocks; ++blk) {
        const int m0 = row_block(blk) * BM;
        const int qt0 = m0 + 32 * wave;   // first query of this wave's tile
        dq0 = qt0 + l32 - 4 * h - 3;
        const int nst = blk == 0 ? nst0 : nst1;
        // full stages: causal, every key below the row block; otherwise every
        // stage inside T.  They run in the pipeline in groups of four; the rest
        // (at most four stages) take the masked path.
        const int nfull = p.causal ? m0 / BN : T / BN;
        const int nmain = nfull & ~3;

#pragma unroll
        for (int c = 0; c < 4; ++c) oacc[c] = f32x16{};
        rsum[0] = rsum[1] = rsum[2] = rsum[3] = 0.f;
        if (nmain > 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) vt[i] = u32x4{0u, 0u, 0u, 0u};   // no previous block: 0 x 0
            wprev[0] = wprev[1] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
            read_k_re(buf0, 0, ka);
            for (int s = 0; s < nmain; s += 4) {
                // The read offsets are loop-invariant, and so is every address
                // of a statically named buffer: left alone, the compiler hoists
                // one register per address out of the loop.  Made opaque here,
                // they are formed inside the loop, with the constant part in
                // the instruction's offset field.
                __asm__ __volatile__("" : "+v"(koff[0]), "+v"(koff[1]), "+v"(koff[2]), "+v"(koff[3]),
                                     "+v"(voff[0]), "+v"(voff[1]));
                main_stage(I0{}, gbase + s);
                main_stage(I1{}, gbase + s + 1);
                main_stage(I2{}, gbase + s + 2);
                main_stage(I3{}, gbase + s + 3);
            }
            // the last block's value product
#pragma unroll
            for (int i = 0; i < 8; ++i) oacc[i >> 1] = mfma(as_bf16x8(vt[i]), wprev[i & 1], oacc[i >> 1]);
        }
        const bool wave_live = qt0 < T;
        if (nmain < nst) rest_stage(I0{}, gbase + nmain, nmain, qt0, wave_live);
        if (nmain + 1 < nst) rest_stage(I1{}, gbase + nmain + 1, nmain + 1, qt0, wave_live);
        if (nmain + 2 < nst) rest_stage(I2{}, gbase + nmain + 2, nmain + 2, qt0, wave_live);
        if (nmain + 3 < nst) rest_stage(I3{}, gbase + nmain + 3, nmain + 3, qt0, wave_live);

        if (blk + 1 < nblocks) {
            load_q(row_block(blk + 1) * BM + 32 * wave);   // in flight during the epilogue
            if (!seamless) {
                // restart the stream: every wave is past its last read (the
                // barrier ending the last stage), so buffers 0 and 1 are free
                dma_stage(0, buf0, true);
                dma_stage(BN, buf1, nst1 > 1);
            }
        }

        // ---- epilogue: O = acc / (sum w + eps), bf16 planes ----------------
        const float rs = (rsum[0] + rsum[1]) + (rsum[2] + rsum[3]);
        const float den = rs + __shfl_xor(rs, 32) + p.eps;   // both lane halves hold this query
        const float inv = den != 0.f ? 1.f / den : 0.f;
        const int q = qt0 + l32;
        if (q < T) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = 32 * (c & 1) + 8 * g + 4 * h;   // channel of register 4 g in its plane
                    const u32x2 v = {pack_bf16x2(oacc[c][4 * g] * inv, oacc[c][4 * g + 1] * inv),
                                     pack_bf16x2(oacc[c][4 * g + 2] * inv, oacc[c][4 * g + 3] * inv)};
                    *reinterpret_cast<u32x2 *>((c < 2 ? ore : oim) + (int64_t)q * to + col) = v;
                }
            }
            if (p.row_den && h == 0) p.row_den[(int64_t)bh * T + q] = den;
        }
        if (blk + 1 < nblocks && !seamless) stage_barrier();   // the restarted stream's first stage
        gbase += nst;
    }
    // Loads past the stream's end (extent 0) still write zeros into LDS: let
    // them land before the workgroup's LDS can be handed to another.
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
}

}  // namespace

bool supports_born_bf16_d64(const Problem &p) {
    return p.op == OP_BORN && p.layout == LAYOUT_BF16 && p.d == D && p.aligned16;
}

hipError_t launch_born_bf16_d64(const Problem &p) {
    const int nrb = (p.T + BM - 1) / BM;
    const int nwork = p.causal ? (nrb + 1) / 2 : nrb;   // causal: mirrored pairs of row blocks
    const int64_t blocks = (int64_t)p.BH * nwork;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    auto kern = p.decay.on ? (p.rot ? born_bf16_d64_kernel<true, true> : born_bf16_d64_kernel<true, false>)
                           : (p.rot ? born_bf16_d64_kernel<false, true> : born_bf16_d64_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p, nrb, nwork);
    return hipGetLastError();
}

}  // namespace cattn
