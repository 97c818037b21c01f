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

// Buffer resources (raw, stride 0, range-checked in bytes): word 3 of the
// descriptor for untyped 32-bit loads on this architecture, and an offset past
// any table, whose loads return zero and touch no memory.
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kBufferNone = 0x80000000u;

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
// (relative step 2^-11) right after.  GELU(x) = x Phi(x) = max(x, 0) - |x| Q
// with Q = 1 - Phi(|x|) the upper tail of the standard normal distribution.
// Writing the negative half as -|x| Q (instead of x (1 - erf)) avoids the
// cancellation 1 - erf(u) for large |x|.  Q(w) is evaluated as 2^P(min(w, 6))
// with P a degree-7 polynomial fitted to log2 Q on [0, 6] (gen_gelu_tail.py,
// least squares refined towards the minimax error): relative error of Q at
// most 3.9e-6 for w < 4.3 (where |x| Q is above fp16's smallest normal) and
// 4.6e-6 on [0, 6], in fp32 with fused multiply-adds, under a hundredth of an
// fp16 step of the result; beyond 6, |x| Q(6) < 1e-9 |x| is far below what
// the fp16 result can hold.  One exponential per value and no reciprocal.
// The clamps are v_med3_f32 (for finite inputs: min(|x|, 6) and max(x, 0))
// rather than fminf / fmaxf, which add a NaN-quieting instruction each.
__device__ __forceinline__ float normal_tail(float w) {
#pragma clang fp contract(fast)
    const float v = __builtin_amdgcn_fmed3f(w, 0.0f, 6.0f);
    float p = -1.845025508e-06f;
    p = fmaf(p, v, 6.177832256e-05f);
    p = fmaf(p, v, -9.317235090e-04f);
    p = fmaf(p, v, 8.511628956e-03f);
    p = fmaf(p, v, -5.396552756e-02f);
    p = fmaf(p, v, -4.584611952e-01f);
    p = fmaf(p, v, -1.151251435e+00f);
    p = fmaf(p, v, -9.999952912e-01f);
    return __builtin_amdgcn_exp2f(p);
}

// max(x, 0) for finite x in one instruction.
__device__ __forceinline__ float relu_med3(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.402823466e+38f); }

__device__ __forceinline__ float gelu_fp16path(float x) {
    const float q = normal_tail(fabsf(x));
    return fmaf(-fabsf(x), q, relu_med3(x));
}

// Q = 1 - Phi(|x|) as gelu_fp16path computes it, and e = exp(-x^2 / 2) (for
// GELU' = Phi(x) + x phi(x) in the backward).
__device__ __forceinline__ float gelu_tail(float x, float& e) {
    e = __builtin_amdgcn_exp2f(-(x * x) * 0.72134752044448170f);  // log2(e) / 2
    return normal_tail(fabsf(x));
}

// The hidden activation of the fp16 path: GELU (erf form) or ReLU.
template <bool GELU>
__device__ __forceinline__ float hidden_act(float v) {
    if constexpr (GELU)
        return gelu_fp16path(v);
    else
        return v > 0.0f ? v : 0.0f;
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
