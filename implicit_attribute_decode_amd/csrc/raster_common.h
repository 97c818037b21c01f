// Per-pixel splat arithmetic shared by the forward raster and its backward
// pass, so that both take exactly the same compositing decisions ("SPIN-4DGS"
// §3.1, Eq. 1 and Eq. 4).  The kernels work with the exponent in base 2: the
// conic is staged pre-scaled by -log2(e)/2, -log2(e), -log2(e)/2 (one fp32
// rounding each), gz = -A log2(e)/2, gw = -B log2(e), gbx = -C log2(e)/2, so
// that p2 = (gz dx^2 + gbx dy^2) + gw dx dy = log2(e) power, with power =
// -0.5 (A dx^2 + C dy^2) - B dx dy and d = pixel centre - mean, and
// exp(power) = 2^p2 is one hardware exp2.  The 3-sigma bound power >= -4.5 is
// p2 >= -4.5 log2(e).
#pragma once

#include <hip/hip_runtime.h>

namespace ia {

constexpr float kLog2e = 1.44269504088896341f;
constexpr float kConicScaleA = -0.5f * kLog2e;  // staged A and C factor
constexpr float kConicScaleB = -kLog2e;          // staged B factor
constexpr float kPower2Min = -4.5f * kLog2e;     // 3 sigma in base-2 units

// Terms of power that depend on dx only.
__device__ __forceinline__ void splat_dx_terms(float gz, float gw, float dx, float& ta, float& tb) {
#pragma clang fp contract(fast)
    ta = gz * dx * dx;
    tb = gw * dx;
}

// p2 = log2(e) power from the dx terms and dy.
__device__ __forceinline__ float splat_power(float ta, float tb, float gbx, float dy) {
#pragma clang fp contract(fast)
    return (ta + gbx * dy * dy) + tb * dy;
}

// exp(power) = 2^p2.
__device__ __forceinline__ float splat_gauss(float p2) { return __builtin_amdgcn_exp2f(p2); }

// alpha = min(0.99, o exp(power)) before the skip rule.
__device__ __forceinline__ float splat_alpha(float opacity, float p2) {
#pragma clang fp contract(fast)
    return fminf(0.99f, opacity * splat_gauss(p2));
}

// Composited unless outside 3 sigma (power outside [-4.5, 0]) or alpha < 1/255.
__device__ __forceinline__ bool splat_takes(float p2, float a0) {
    return p2 >= kPower2Min && p2 <= 0.0f && a0 >= (1.0f / 255.0f);
}

// Degree-3 real spherical harmonics (orthonormal, l-major, m = -l..l, the
// Condon-Shortley sign convention) at unit direction (x, y, z).
__device__ __forceinline__ void sh_basis16(float x, float y, float z, float Y[16]) {
    const float xx = x * x, yy = y * y, zz = z * z;
    Y[0] = 0.28209479177387814f;
    Y[1] = -0.48860251190291992f * y;
    Y[2] = 0.48860251190291992f * z;
    Y[3] = -0.48860251190291992f * x;
    Y[4] = 1.0925484305920792f * x * y;
    Y[5] = -1.0925484305920792f * y * z;
    Y[6] = 0.31539156525252005f * (2.0f * zz - xx - yy);
    Y[7] = -1.0925484305920792f * x * z;
    Y[8] = 0.54627421529603959f * (xx - yy);
    Y[9] = -0.59004358992664352f * y * (3.0f * xx - yy);
    Y[10] = 2.8906114426405538f * x * y * z;
    Y[11] = -0.45704579946446572f * y * (4.0f * zz - xx - yy);
    Y[12] = 0.37317633259011546f * z * (2.0f * zz - 3.0f * xx - 3.0f * yy);
    Y[13] = -0.45704579946446572f * x * (4.0f * zz - xx - yy);
    Y[14] = 1.4453057213202769f * z * (xx - yy);
    Y[15] = -0.59004358992664352f * x * (xx - 3.0f * yy);
}

// sum_k w_k grad Y_k at unit direction (x, y, z): the derivatives of the
// basis polynomials of sh_basis16 in (x, y, z) (the caller projects the
// result onto the sphere).
__device__ __forceinline__ void sh_basis16_grad(float x, float y, float z, const float w[16], float g[3]) {
    const float k1 = 0.48860251190291992f, k2a = 1.0925484305920792f, k2b = 0.31539156525252005f,
                k2c = 0.54627421529603959f, k3a = 0.59004358992664352f, k3b = 2.8906114426405538f,
                k3c = 0.45704579946446572f, k3d = 0.37317633259011546f, k3e = 1.4453057213202769f;
    const float xx = x * x, yy = y * y, zz = z * z;
    g[0] = -k1 * w[3] + k2a * y * w[4] - 2.0f * k2b * x * w[6] - k2a * z * w[7] + 2.0f * k2c * x * w[8] -
           6.0f * k3a * x * y * w[9] + k3b * y * z * w[10] + 2.0f * k3c * x * y * w[11] - 6.0f * k3d * x * z * w[12] -
           k3c * (4.0f * zz - 3.0f * xx - yy) * w[13] + 2.0f * k3e * x * z * w[14] - k3a * (3.0f * xx - 3.0f * yy) * w[15];
    g[1] = -k1 * w[1] + k2a * x * w[4] - k2a * z * w[5] - 2.0f * k2b * y * w[6] - 2.0f * k2c * y * w[8] -
           k3a * (3.0f * xx - 3.0f * yy) * w[9] + k3b * x * z * w[10] - k3c * (4.0f * zz - xx - 3.0f * yy) * w[11] -
           6.0f * k3d * y * z * w[12] + 2.0f * k3c * x * y * w[13] - 2.0f * k3e * y * z * w[14] + 6.0f * k3a * x * y * w[15];
    g[2] = k1 * w[2] - k2a * y * w[5] + 4.0f * k2b * z * w[6] - k2a * x * w[7] + k3b * x * y * w[10] -
           8.0f * k3c * y * z * w[11] + k3d * (6.0f * zz - 3.0f * xx - 3.0f * yy) * w[12] - 8.0f * k3c * x * z * w[13] +
           k3e * (xx - yy) * w[14];
}

}  // namespace ia
