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
#include "cattn_internal.h"



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

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void born_bf16_d64_kernel(Problem p, int nrb, int nwork) {
    __shared__ __align__(16) char stage_a[STAGE];   // even stages
    __shared__ __align__(16) char stage_b[STAGE];   // odd stages

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
    const int64_t tkv[2] = {p.sk.t, p.sv.t};
    const uint16_t *qre = reinterpret_cast<const uint16_t *>(p.q_re) + hq;
    const uint16_t *qim = reinterpret_cast<const uint16_t *>(p.q_im) + hq;
    const uint16_t *planes[4] = {reinterpret_cast<const uint16_t *>(p.k_re) + hk,
                                 reinterpret_cast<const uint16_t *>(p.k_im) + hk,
                                 reinterpret_cast<const uint16_t *>(p.v_re) + hv,
                                 reinterpret_cast<const uint16_t *>(p.v_im) + hv};
    uint16_t *ore = reinterpret_cast<uint16_t *>(p.o_re) + ho;
    uint16_t *oim = reinterpret_cast<uint16_t *>(p.o_im) + ho;

    // ---- staging: global -> LDS, no registers ------------------------------
    // Within a region, chunk id = NT e + t (e < RPT) covers row id / 8 and
    // physical slot t % 8, and receives logical chunk slot ^ swz(row) of that
    // key row.  A wave's 64 chunks of one (region, e) are 1 KiB of LDS.
    const int srow = tid >> 3;
    const int sslot = tid & 7;
    const int lck = sslot ^ swz_k(srow);   // swizzles depend on row % 16 only
    const int lcv = sslot ^ swz_v(srow);

    auto issue_stage = [&](int k0, char *buf) {
        const bool tail = k0 + BN > T;
        char *dst = buf + wave * 1024;
#pragma unroll
        for (int i = 0; i < LOADS_PER_T; ++i) {
            const int g = i / RPT, e = i % RPT;
            int row = k0 + srow + (NT / 8) * e;
            if (tail) row = min(row, T - 1);   // rows past T are masked out of the weights
            const int lc = g < 2 ? lck : lcv;
            __builtin_amdgcn_global_load_lds((GLB_AS void *)(planes[g] + (int64_t)row * tkv[g >> 1] + 8 * lc),
                                             (LDS_AS void *)(dst + g * REGION + e * (NT * 16)), 16, 0, 0);
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

    const int nblocks = p.causal && item != nrb - 1 - item ? 2 : 1;
    auto row_block = [&](int blk) { return p.causal ? (blk == 0 ? nrb - 1 - item : item) : item; };
    auto tile_of = [&](int blk) { return row_block(blk) * BM + 32 * wave; };   // this wave's first query

    // Q operands (B operand of the score products): k-step kk, lane
    // (query l32, half h) holds Q'[q][16 kk + 8 h .. + 8].
    bf16x8 qb[8];
    bf16x8 qneg[4];   // -Re Q chunks: second half of [Im Q | -Re Q]
    auto load_q = [&](int qt0) {
        const int q = qt0 + l32;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (q < T) {
                const uint16_t *src = (kk < 4 ? qre : qim) + (int64_t)q * tq + 16 * (kk & 3) + 8 * h;
                x = *reinterpret_cast<const u32x4 *>(src);
            }
            qb[kk] = as_bf16x8(x);
            if (kk < 4) qneg[kk] = as_bf16x8(x ^ 0x80008000u);
        }
    };
    load_q(tile_of(0));
    bool stage0_issued = false;   // the next row block's first stage is already in flight

    for (int blk = 0; blk < nblocks; ++blk) {
        const int rb = row_block(blk);
        const int m0 = rb * BM;
        const int qt0 = tile_of(blk);   // first query of this wave's tile

        f32x16 oacc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) oacc[c] = f32x16{};
        float rsum = 0.f;

        // Scores S^T of 32-key block sb of LDS stage st
        auto scores = [&](const char *st, int sb, f32x16 &sr, f32x16 &si) {
            sr = f32x16{};
            si = f32x16{};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(st + (kk >> 2) * REGION + sb * 32 * ROWB + koff[kk & 3]);
                sr = mfma(a, qb[kk], sr);
                si = mfma(a, kk < 4 ? qb[kk + 4] : qneg[kk - 4], si);
            }
        };
        // w = |S|^2 packed to bf16; register r of lane half h is key 8 (r/4) + 4 h + r % 4.
        // MASKED zeroes keys past `lim` (per lane): the causal diagonal, a ragged tail.
        auto weights = [&](const f32x16 &sr, const f32x16 &si, bf16x8 (&wop)[2], bool masked, int lim) {
            uint32_t pk[8];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float w0 = sr[r] * sr[r] + si[r] * si[r];
                float w1 = sr[r + 1] * sr[r + 1] + si[r + 1] * si[r + 1];
                if (masked) {
                    const int key0 = 8 * (r >> 2) + 4 * h + (r & 3);
                    w0 = key0 > lim ? 0.f : w0;
                    w1 = key0 + 1 > lim ? 0.f : w1;
                }
                pk[r >> 1] = pack_bf16x2(w0, w1);
                rsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[r >> 1]), ones, rsum, false);
            }
            wop[0] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
            wop[1] = as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]});
        };
        // O^T += V'^T W^T for block sb
        auto values = [&](const char *st, int sb, const bf16x8 (&wop)[2]) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const char *vb = st + (2 + (c >> 1)) * REGION + (32 * sb + 16 * m) * ROWB + voff[c & 1];
                    const u32x2 lo = ds_read_tr(vb);
                    const u32x2 hi = ds_read_tr(vb + 8 * ROWB);
                    oacc[c] = mfma(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), wop[m], oacc[c]);
                }
            }
        };
        auto key_block = [&](const char *st, int sb, bool masked, int lim) {
            f32x16 sr, si;
            bf16x8 wop[2];
            scores(st, sb, sr, si);
            weights(sr, si, wop, masked, lim);
            values(st, sb, wop);
        };

        const int kend = p.causal ? min(T, m0 + BM) : T;
        const int nstages = (kend + BN - 1) / BN;

        const bool wave_live = qt0 < T;
        auto compute_stage = [&](int k0, const char *st) {
            if (!wave_live) return;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int kb0 = k0 + 32 * sb;
                const bool skip = kb0 >= T || (p.causal && kb0 > qt0);
                const bool full = (!p.causal || kb0 + 32 <= qt0) && kb0 + 32 <= T;
                if (full) {
                    key_block(st, sb, false, 31);
                } else if (!skip) {
                    key_block(st, sb, true, min(p.causal ? qt0 + l32 - kb0 : 31, T - 1 - kb0));
                }
            }
        };

        // Stage s lives in stage_a (s even) or stage_b (s odd).  At the top of
        // stage s its loads have landed for every wave (barrier), and every
        // wave is done reading the other buffer, which then takes stage s + 1.
        if (!stage0_issued) {
            loads_done_barrier();   // the previous row block is done with both buffers
            issue_stage(0, stage_a);
        }
        // with an even stage count the last stage sits in stage_b; from its top
        // on stage_a is free and takes the next row block's first stage
        const bool prefetch_next = blk + 1 < nblocks && (nstages & 1) == 0;
        for (int s = 0; s < nstages; s += 2) {
            loads_done_barrier();
            if (s + 1 < nstages) issue_stage((s + 1) * BN, stage_b);
            compute_stage(s * BN, stage_a);
            if (s + 1 < nstages) {
                loads_done_barrier();
                if (s + 2 < nstages)
                    issue_stage((s + 2) * BN, stage_a);
                else if (prefetch_next)
                    issue_stage(0, stage_a);
                compute_stage((s + 1) * BN, stage_b);
            }
        }
        stage0_issued = prefetch_next;
        if (blk + 1 < nblocks) load_q(tile_of(blk + 1));   // in flight during the epilogue

        // ---- epilogue: O = acc / (sum w + eps), bf16 planes ----------------
        const float den = rsum + __shfl_xor(rsum, 32) + p.eps;   // both lane halves hold this query
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
    }
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
    hipLaunchKernelGGL(born_bf16_d64_kernel, dim3((unsigned)blocks), dim3(NT), 0, p.stream, p, nrb, nwork);
    return hipGetLastError();
}

}  // namespace cattn
