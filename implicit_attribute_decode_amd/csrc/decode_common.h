// Device helpers shared by the decode (decode.hip) and its backward
// (decode_bwd.hip): position normalisation and the cell decision of the hash
// encoding (SPIN-4DGS §3.3 Eq. 7-9), the fp16-path GELU, and the fp16 operand
// packing of v_mfma_f32_16x16x32_f16.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ia {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kP1 = 1u, kP2 = 2654435761u, kP3 = 805459861u, kP4 = 3674653429u;

// Eq. 7 (contraction with the L2 norm, mapped to [0,1]^3) and Eq. 8.
__device__ __forceinline__ void normalize_pos(float x, float y, float z, float t, float t_min, float t_max,
                                              float xt[4]) {
    float n2 = x * x + y * y;
    n2 = n2 + z * z;
    float n = sqrtf(n2);
    float c0 = x, c1 = y, c2 = z;
    if (!(n <= 1.0f)) {
        float k = 2.0f - 1.0f / n;
        k = k / n;
        c0 = x * k;
        c1 = y * k;
        c2 = z * k;
    }
    float tn = (t - t_min) / (t_max - t_min);
    tn = tn < 0.0f ? 0.0f : (tn > 1.0f ? 1.0f : tn);
    float a0 = 0.25f * c0, a1 = 0.25f * c1, a2 = 0.25f * c2;
    xt[0] = a0 + 0.5f;
    xt[1] = a1 + 0.5f;
    xt[2] = a2 + 0.5f;
    xt[3] = tn;
}

// Per-axis cell: p = x*(res-1), i = clamp(floor p, 0, res-2), f = p - i.
__device__ __forceinline__ void cell_axis(float x, int res, int& i, float& f) {
    float p = x * (float)(res - 1);
    int c = (int)floorf(p);
    c = c < 0 ? 0 : (c > res - 2 ? res - 2 : c);
    i = c;
    f = p - (float)c;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

// GELU for the fp16 path, whose hidden activations are rounded to fp16
// (relative step 2^-11) right after: erf from Abramowitz & Stegun, Handbook
// of Mathematical Functions, formula 7.1.26, |error| <= 1.5e-7:
//   erf(u) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-u^2),
//   t = 1 / (1 + p u), u >= 0, erf odd.
__device__ __forceinline__ float gelu_fp16path(float x) {
    const float u = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, u, 1.0f));
    float poly = fmaf(t, 1.061405429f, -1.453152027f);
    poly = fmaf(t, poly, 1.421413741f);
    poly = fmaf(t, poly, -0.284496736f);
    poly = fmaf(t, poly, 0.254829592f);
    const float e = __expf(-(u * u));
    const float erf_u = fmaf(-(poly * t), e, 1.0f);
    return 0.5f * x * (1.0f + copysignf(erf_u, x));
}

__device__ __forceinline__ half4_t load_h4(const _Float16* p) {
    return *reinterpret_cast<const half4_t*>(p);
}

__device__ __forceinline__ half4_t unpack2(uint32_t a, uint32_t b) {
    half4_t r;
    r[0] = __builtin_bit_cast(_Float16, (uint16_t)(a & 0xffffu));
    r[1] = __builtin_bit_cast(_Float16, (uint16_t)(a >> 16));
    r[2] = __builtin_bit_cast(_Float16, (uint16_t)(b & 0xffffu));
    r[3] = __builtin_bit_cast(_Float16, (uint16_t)(b >> 16));
    return r;
}

__device__ __forceinline__ half8_t cat8(half4_t lo, half4_t hi) {
    return half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// A operand of v_mfma_f32_16x16x32_f16 for row block rb, 32-wide k-block m of
// a row-major [rows][in] fp16 matrix: slots e < 4 hold inputs 32 m + 4 q + e,
// slots e >= 4 inputs 32 m + 16 + 4 q + (e - 4); rows >= `rows` are zero.
__device__ __forceinline__ half8_t a_tile32(const _Float16* W, int in_dim, int rows, int rb, int m, int q, int c) {
    const int row = 16 * rb + c;
    if (row >= rows) return half8_t{0, 0, 0, 0, 0, 0, 0, 0};
    const _Float16* r = W + (size_t)row * in_dim + 32 * m + 4 * q;
    return cat8(load_h4(r), load_h4(r + 16));
}

}  // namespace ia
