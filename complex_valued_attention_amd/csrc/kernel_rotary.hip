// Rotary phase embedding ("Show HN: CNET", the RotaryEmbed layer: position as
// a complex phase rotation, base 10000, absolute position for step mode):
//     y[t, m] = x[t, m] * exp(i (p0 + t) theta_m),   theta_m = base^(-m / d_h).
//
// An elementwise pass bound by HBM bandwidth.  The phase depends on the
// position and the channel only, so each thread forms it once and applies it
// to a chunk of heads.
// The angle (p0 + t) theta_m is formed and reduced modulo 2 pi in fp64: at
// t ~ 1e4 an fp32 product would already carry ~1e-3 rad of error.  The
// reduced angle lies in [-pi, pi], where the fp32 hardware sine and cosine are
// accurate to ~1e-6.  In place (y == x) is allowed: every element is read and
// written by one thread.
#include "cattn_internal.h"

namespace cattn {
namespace {

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ inline uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// cos and sin of (p0 + t) theta, reduced in fp64
__device__ inline void phase(double pos, double theta, float &c, float &s) {
    const double a = pos * theta;
    const double k = rint(a * 0.15915494309189535);                  // a / (2 pi), nearest integer
    const double r = fma(-k, 2.4492935982947064e-16, fma(-k, 6.283185307179586, a));   // a - 2 pi k
    __sincosf((float)r, &s, &c);
}

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
        const double theta = m < p.d ? exp(-(double)m * p.log_base / (double)p.d) : 0.0;
        phase(pos, theta, c[e], sn[e]);
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
                for (int e = 0; e < VEC; ++e) {
                    yv[2 * e] = xv[u][2 * e] * c[e] - xv[u][2 * e + 1] * sn[e];
                    yv[2 * e + 1] = xv[u][2 * e] * sn[e] + xv[u][2 * e + 1] * c[e];
                }
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
                    const float a = bf16_to_f32(xr[u][e]), b = bf16_to_f32(xi[u][e]);
                    yr[e] = f32_to_bf16(a * c[e] - b * sn[e]);
                    yi[e] = f32_to_bf16(a * sn[e] + b * c[e]);
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
