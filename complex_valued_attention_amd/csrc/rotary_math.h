// Rotary phase arithmetic shared by the rotary pass and the forward kernels
// that rotate Q as they load it ("Show HN: CNET", the RotaryEmbed layer:
// position as a complex phase rotation):
//     y[t, m] = x[t, m] * exp(i pos theta_m),  theta_m = base^(-m / d_h).
// One definition of every step, so a fused rotation gives the same bits as
// the separate pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cattn {

// theta_m = base^(-m / d) in double precision (log_base = ln base)
__device__ inline double rotary_theta(int m, double log_base, int d) { return exp(-(double)m * log_base / (double)d); }

// cos and sin of pos * theta.  The angle is formed and reduced modulo 2 pi in
// double precision (two-part 2 pi, a Cody-Waite style split), since at pos ~
// 1e4 an fp32 product would already be off by ~1e-3 rad; the reduced angle
// lies in [-pi, pi], where the fp32 hardware sine and cosine are accurate to
// ~1e-6.
__device__ inline void rotary_phase(double pos, double theta, float &c, float &s) {
    const double a = pos * theta;
    const double k = rint(a * 0.15915494309189535);                                   // a / (2 pi), nearest integer
    const double r = fma(-k, 2.4492935982947064e-16, fma(-k, 6.283185307179586, a));   // a - 2 pi k
    __sincosf((float)r, &s, &c);
}

// (a + i b) (c + i s), with the fused multiply-adds written out so that every
// caller rounds alike
__device__ inline void rotary_apply(float a, float b, float c, float s, float &yr, float &yi) {
    yr = fmaf(a, c, -(b * s));
    yi = fmaf(a, s, b * c);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept a NaN)
__device__ inline uint16_t rotary_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace cattn
