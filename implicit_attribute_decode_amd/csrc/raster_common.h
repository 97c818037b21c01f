// Per-pixel splat arithmetic shared by the forward raster and its backward
// pass, so that both take exactly the same compositing decisions ("SPIN-4DGS"
// §3.1, Eq. 1 and Eq. 4).  The conic is pre-scaled by -1/2, -1, -1/2:
// gz = -A/2, gw = -B, gbx = -C/2, so power = -0.5 (A dx^2 + C dy^2) - B dx dy
// = (gz dx^2 + gbx dy^2) + gw dx dy with d = pixel centre - mean.
#pragma once

#include <hip/hip_runtime.h>

namespace ia {

// Terms of power that depend on dx only.
__device__ __forceinline__ void splat_dx_terms(float gz, float gw, float dx, float& ta, float& tb) {
#pragma clang fp contract(fast)
    ta = gz * dx * dx;
    tb = gw * dx;
}

__device__ __forceinline__ float splat_power(float ta, float tb, float gbx, float dy) {
#pragma clang fp contract(fast)
    return (ta + gbx * dy * dy) + tb * dy;
}

// alpha = min(0.99, o exp(power)) before the skip rule.
__device__ __forceinline__ float splat_alpha(float opacity, float power) {
#pragma clang fp contract(fast)
    return fminf(0.99f, opacity * __expf(power));
}

// Composited unless outside 3 sigma (power outside [-4.5, 0]) or alpha < 1/255.
__device__ __forceinline__ bool splat_takes(float power, float a0) {
    return power >= -4.5f && power <= 0.0f && a0 >= (1.0f / 255.0f);
}

}  // namespace ia
