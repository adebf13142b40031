// Rotary phase embedding ("Show HN: CNET", the RotaryEmbed layer: position as
// a complex phase rotation, base 10000, absolute position for step mode):
//     y[t, m] = x[t, m] * exp(i (p0 + t) theta_m),   theta_m = base^(-m / d_h).
//
// An elementwise pass bound by HBM bandwidth.  Each thread keeps one group of
// VEC consecutive channels for its whole grid-stride loop (the block size is
// a multiple of the groups per row), so theta_m is formed once per thread.
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

// VEC: channels per thread-group (2 complex64 values = 16 bytes; 8 bf16 per plane = 16 bytes; 1 = scalar)
template <int LAYOUT, int VEC>
__global__ __launch_bounds__(256) void rotary_kernel(RotaryProblem p, int L) {
    const int mg = threadIdx.x % L;              // this thread's channel group, fixed (blockDim % L == 0)
    double theta[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const int m = mg * VEC + e;
        theta[e] = m < p.d ? exp(-(double)m * p.log_base / (double)p.d) : 0.0;
    }
    const int64_t ngroups = p.rows * (int64_t)L;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < ngroups; g += stride) {
        const int64_t row = g / L;
        const double pos = (double)(p.pos0 + row % p.T);
        const int64_t idx = row * p.d + (int64_t)mg * VEC;
        if (LAYOUT == LAYOUT_C64) {
            float xv[2 * VEC], yv[2 * VEC];
            if (VEC == 2) {
                const float4 x4 = *reinterpret_cast<const float4 *>(reinterpret_cast<const float2 *>(p.x_re) + idx);
                xv[0] = x4.x; xv[1] = x4.y; xv[2] = x4.z; xv[3] = x4.w;
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float2 x2 = reinterpret_cast<const float2 *>(p.x_re)[idx + e];
                    xv[2 * e] = x2.x; xv[2 * e + 1] = x2.y;
                }
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float c, s;
                phase(pos, theta[e], c, s);
                yv[2 * e] = xv[2 * e] * c - xv[2 * e + 1] * s;
                yv[2 * e + 1] = xv[2 * e] * s + xv[2 * e + 1] * c;
            }
            if (VEC == 2) {
                *reinterpret_cast<float4 *>(reinterpret_cast<float2 *>(p.y_re) + idx) = make_float4(yv[0], yv[1], yv[2], yv[3]);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    reinterpret_cast<float2 *>(p.y_re)[idx + e] = make_float2(yv[2 * e], yv[2 * e + 1]);
            }
        } else {
            uint16_t xr[VEC], xi[VEC], yr[VEC], yi[VEC];
            if (VEC == 8) {
                const uint4 r4 = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.x_re) + idx);
                const uint4 i4 = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.x_im) + idx);
                const uint32_t rw[4] = {r4.x, r4.y, r4.z, r4.w}, iw[4] = {i4.x, i4.y, i4.z, i4.w};
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    xr[e] = (uint16_t)(rw[e >> 1] >> (16 * (e & 1)));
                    xi[e] = (uint16_t)(iw[e >> 1] >> (16 * (e & 1)));
                }
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    xr[e] = reinterpret_cast<const uint16_t *>(p.x_re)[idx + e];
                    xi[e] = reinterpret_cast<const uint16_t *>(p.x_im)[idx + e];
                }
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float c, s;
                phase(pos, theta[e], c, s);
                const float a = bf16_to_f32(xr[e]), b = bf16_to_f32(xi[e]);
                yr[e] = f32_to_bf16(a * c - b * s);
                yi[e] = f32_to_bf16(a * s + b * c);
            }
            if (VEC == 8) {
                uint32_t rw[4], iw[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    rw[w] = (uint32_t)yr[2 * w] | ((uint32_t)yr[2 * w + 1] << 16);
                    iw[w] = (uint32_t)yi[2 * w] | ((uint32_t)yi[2 * w + 1] << 16);
                }
                *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(p.y_re) + idx) = make_uint4(rw[0], rw[1], rw[2], rw[3]);
                *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(p.y_im) + idx) = make_uint4(iw[0], iw[1], iw[2], iw[3]);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    reinterpret_cast<uint16_t *>(p.y_re)[idx + e] = yr[e];
                    reinterpret_cast<uint16_t *>(p.y_im)[idx + e] = yi[e];
                }
            }
        }
    }
}

template <int LAYOUT, int VEC>
hipError_t launch_vec(const RotaryProblem &p) {
    const int L = p.d / VEC;                        // channel groups per row
    const int nb = L * (256 / L);                   // block size: a multiple of L, at most 256
    const int64_t ngroups = p.rows * (int64_t)L;
    int64_t blocks = (ngroups + nb - 1) / nb;
    blocks = blocks < 8192 ? blocks : 8192;         // grid-stride beyond 32 blocks per CU
    hipLaunchKernelGGL((rotary_kernel<LAYOUT, VEC>), dim3((unsigned)blocks), dim3(nb), 0, p.stream, p, L);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rotary(const RotaryProblem &p) {
    if (p.layout == LAYOUT_C64)
        return p.d % 2 == 0 ? launch_vec<LAYOUT_C64, 2>(p) : launch_vec<LAYOUT_C64, 1>(p);
    return p.d % 8 == 0 ? launch_vec<LAYOUT_BF16, 8>(p) : launch_vec<LAYOUT_BF16, 1>(p);
}

}  // namespace cattn
