// Rotary phase embedding ("Show HN: CNET", the RotaryEmbed layer: position as
// a complex phase rotation, base 10000, absolute position for step mode):
//     y[t, m] = x[t, m] * exp(i (p0 + t) theta_m),   theta_m = base^(-m / d_h).
//
// An elementwise pass bound by HBM bandwidth.  The phase depends on the
// position and the channel only, so each thread forms it once and applies it
// to a chunk of heads.  The phase arithmetic (angle reduced in fp64) lives in
// rotary_math.h, shared with the forward kernels that rotate Q at load.  In
// place (y == x) is allowed: every element is read and written by one thread.
#include "cattn_internal.h"
#include "rotary_math.h"

namespace cattn {
namespace {

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// VEC: channels per thread (2 complex64 values = 16 bytes; 8 bf16 per plane =
// 16 bytes; 1 = scalar).  Thread g of a head covers row t = g / L, channels
// VEC (g % L) ..; it forms the phases of its channels once and applies them to
// every head of its chunk (blockIdx.y), since the rotation does not depend on
// the head.  Consecutive threads cover consecutive 16-byte pieces of a row.
template <int LAYOUT, int VEC>
__global__ __launch_bounds__(256) void rotary_kernel(RotaryProblem p, int L, int hc) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= (int64_t)p.T * L) return;
    const int t = (int)(g / L), mg = (int)(g % L);
    const double pos = (double)(p.pos0 + t);
    float c[VEC], sn[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const int m = mg * VEC + e;
        const double theta = m < p.d ? rotary_theta(m, p.log_base, p.d) : 0.0;
        rotary_phase(pos, theta, c[e], sn[e]);
    }
    const int64_t bh0 = (int64_t)blockIdx.y * hc;
    const int64_t bh1 = bh0 + hc < p.BH ? bh0 + hc : p.BH;
    const int64_t head = (int64_t)p.T * p.d;                      // elements per head
    const int64_t off = (int64_t)t * p.d + (int64_t)mg * VEC;    // this thread's piece of a head
    // UH heads at a time: every load of the group is issued before any store
    // (each element belongs to this thread alone, so in place is safe)
    constexpr int UH = 4;
    for (int64_t b0 = bh0; b0 < bh1; b0 += UH) {
        const int nh = bh1 - b0 < UH ? (int)(bh1 - b0) : UH;
        if (LAYOUT == LAYOUT_C64) {
            float xv[UH][2 * VEC];
#pragma unroll
            for (int u = 0; u < UH; ++u) {
                if (u >= nh) break;
                const float2 *src = reinterpret_cast<const float2 *>(p.x_re) + (b0 + u) * head + off;
                if (VEC == 2) {
                    const float4 x4 = *reinterpret_cast<const float4 *>(src);
                    xv[u][0] = x4.x; xv[u][1] = x4.y; xv[u][2] = x4.z; xv[u][3] = x4.w;
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float2 x2 = src[e];
                        xv[u][2 * e] = x2.x; xv[u][2 * e + 1] = x2.y;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < UH; ++u) {
                if (u >= nh) break;
                float yv[2 * VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) rotary_apply(xv[u][2 * e], xv[u][2 * e + 1], c[e], sn[e], yv[2 * e], yv[2 * e + 1]);
                float2 *dst = reinterpret_cast<float2 *>(p.y_re) + (b0 + u) * head + off;
                if (VEC == 2) {
                    *reinterpret_cast<float4 *>(dst) = make_float4(yv[0], yv[1], yv[2], yv[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) dst[e] = make_float2(yv[2 * e], yv[2 * e + 1]);
                }
            }
        } else {
            uint16_t xr[UH][VEC], xi[UH][VEC];
#pragma unroll
            for (int u = 0; u < UH; ++u) {
                if (u >= nh) break;
                const uint16_t *sr = reinterpret_cast<const uint16_t *>(p.x_re) + (b0 + u) * head + off;
                const uint16_t *si = reinterpret_cast<const uint16_t *>(p.x_im) + (b0 + u) * head + off;
                if (VEC == 8) {
                    const uint4 r4 = *reinterpret_cast<const uint4 *>(sr);
                    const uint4 i4 = *reinterpret_cast<const uint4 *>(si);
                    const uint32_t rw[4] = {r4.x, r4.y, r4.z, r4.w}, iw[4] = {i4.x, i4.y, i4.z, i4.w};
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        xr[u][e] = (uint16_t)(rw[e >> 1] >> (16 * (e & 1)));
                        xi[u][e] = (uint16_t)(iw[e >> 1] >> (16 * (e & 1)));
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        xr[u][e] = sr[e];
                        xi[u][e] = si[e];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < UH; ++u) {
                if (u >= nh) break;
                uint16_t yr[VEC], yi[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float a, b;
                    rotary_apply(bf16_to_f32(xr[u][e]), bf16_to_f32(xi[u][e]), c[e], sn[e], a, b);
                    yr[e] = rotary_bf16(a);
                    yi[e] = rotary_bf16(b);
                }
                uint16_t *dr = reinterpret_cast<uint16_t *>(p.y_re) + (b0 + u) * head + off;
                uint16_t *di = reinterpret_cast<uint16_t *>(p.y_im) + (b0 + u) * head + off;
                if (VEC == 8) {
                    uint32_t rw[4], iw[4];
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        rw[w] = (uint32_t)yr[2 * w] | ((uint32_t)yr[2 * w + 1] << 16);
                        iw[w] = (uint32_t)yi[2 * w] | ((uint32_t)yi[2 * w + 1] << 16);
                    }
                    *reinterpret_cast<uint4 *>(dr) = make_uint4(rw[0], rw[1], rw[2], rw[3]);
                    *reinterpret_cast<uint4 *>(di) = make_uint4(iw[0], iw[1], iw[2], iw[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        dr[e] = yr[e];
                        di[e] = yi[e];
                    }
                }
            }
        }
    }
}

template <int LAYOUT, int VEC>
hipError_t launch_vec(const RotaryProblem &p) {
    const int L = p.d / VEC;                              // channel groups per row
    const int64_t per_head = (int64_t)p.T * L;            // threads per head
    const int64_t bx = (per_head + 255) / 256;
    if (bx > 0x7fffffff) return hipErrorInvalidConfiguration;
    // head chunks: enough workgroups to fill the chip (about 2048), each thread
    // reusing its phases over hc heads
    int64_t chunks = (2048 + bx - 1) / bx;
    chunks = chunks < p.BH ? chunks : p.BH;
    chunks = chunks < 65535 ? chunks : 65535;
    const int hc = (int)((p.BH + chunks - 1) / chunks);
    chunks = (p.BH + hc - 1) / hc;
    hipLaunchKernelGGL((rotary_kernel<LAYOUT, VEC>), dim3((unsigned)bx, (unsigned)chunks), dim3(256), 0, p.stream, p, L, hc);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rotary(const RotaryProblem &p) {
    if (p.layout == LAYOUT_C64)
        return p.d % 2 == 0 ? launch_vec<LAYOUT_C64, 2>(p) : launch_vec<LAYOUT_C64, 1>(p);
    return p.d % 8 == 0 ? launch_vec<LAYOUT_BF16, 8>(p) : launch_vec<LAYOUT_BF16, 1>(p);
}

}  // namespace cattn
