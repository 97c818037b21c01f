// Paper-scale decoder (SPIN-4DGS §3.3 Eq. 9-11 with the §4 implementation
// details: 16 levels of F = 4 features, 2^21-entry tables, hidden width 64,
// GELU, one decoder branch per attribute reading the shared encoding z):
//
//   gather_f4_kernel   level-major quadrilinear interpolation as the F = 2
//       gather, with 8-byte table entries (four fp16 features) and z written
//       as four fp16 per (level, Gaussian).
//   mlp_branch_kernel  four MLPs 64 -> 64 -> 64 -> out_a (scale 3, rotation 4,
//       colour 3 or 48 SH coefficients, opacity 1) on
//       v_mfma_f32_16x16x32_f16 with fp32 accumulation, hidden activations
//       rounded to fp16, then Eq. 11.  All branch weights (72 or 76 A tiles
//       of 1 KiB, laid out once per parameter set) stay in LDS for the whole
//       persistent kernel; each tile read feeds four MFMAs (64 Gaussians per
//       wave, as four 16-column groups).
//
// MFMA layout as in the shared decoder: lane l = 16 q + c, Gaussians are the
// columns, neurons the rows; slot (q, e) of k-block m stands for input
// 32 m + 4 q + e (e < 4) or 32 m + 16 + 4 q + (e - 4) (e >= 4).  With F = 4
// the four features of level 8 m + q (e < 4) and 8 m + 4 + q (e >= 4) are
// exactly a lane's B slots of layer 1.
#include <hip/hip_runtime.h>

#include "decode_common.h"
#include "ia_internal.h"

namespace ia {
namespace {

constexpr int kBr = 4;        // branches: scale, rotation, colour, opacity
constexpr int kBrG = 4;       // 16-Gaussian column groups per wave
constexpr int kTile = 64;     // half8 per A tile (64 lanes x 16 B)

__host__ __device__ constexpr int colour_rb(bool sh) { return sh ? 3 : 1; }
// last-layer row blocks of branch br
__host__ __device__ constexpr int branch_rb(int br, bool sh) { return br == 2 ? colour_rb(sh) : 1; }
// tiles of branch br: layer 1 and 2 (4 row blocks x 2 k-blocks each) + layer 3
__host__ __device__ constexpr int branch_tiles(int br, bool sh) { return 16 + 2 * branch_rb(br, sh); }
__host__ __device__ constexpr int branch_tile_off(int br, bool sh) {
    int o = 0;
    for (int b = 0; b < br; ++b) o += branch_tiles(b, sh);
    return o;
}
__host__ __device__ constexpr int total_tiles(bool sh) { return branch_tile_off(kBr, sh); }
// packed biases of branch br: [64 layer 1][64 layer 2][16 rb layer 3, zero padded]
__host__ __device__ constexpr int branch_bias_off(int br, bool sh) {
    int o = 0;
    for (int b = 0; b < br; ++b) o += 128 + 16 * branch_rb(b, sh);
    return o;
}
__host__ __device__ constexpr int total_bias(bool sh) { return branch_bias_off(kBr, sh); }

// Tile t of the packed buffer: lane (q, c) holds row 16 rb + c of its matrix
// at the k-slots of block m (zero beyond the matrix's rows).
__global__ void branch_tiles_kernel(const _Float16* W0, const _Float16* W1, const _Float16* W2, const _Float16* W3,
                                    const _Float16* W4, const _Float16* W5, const _Float16* W6, const _Float16* W7,
                                    const _Float16* W8, const _Float16* W9, const _Float16* W10, const _Float16* W11,
                                    int sh, half8_t* Wt) {
    const _Float16* W[12] = {W0, W1, W2, W3, W4, W5, W6, W7, W8, W9, W10, W11};
    const bool s = sh != 0;
    const int tile = blockIdx.x, lane = threadIdx.x;
    const int q = lane >> 4, c = lane & 15;
    int br = 0;
    while (br + 1 < kBr && tile >= branch_tile_off(br + 1, s)) ++br;
    const int t = tile - branch_tile_off(br, s);
    const int layer = t < 8 ? 0 : (t < 16 ? 1 : 2);
    const int rb = ((t - 8 * layer) >> 1), m = t & 1;
    const int outs[kBr] = {3, 4, s ? 48 : 3, 1};
    const int rows = layer < 2 ? 64 : outs[br];
    const _Float16* M = W[br * 3 + layer];
    const int row = 16 * rb + c;
    half8_t v = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
    if (row < rows) v = cat8(load_h4(M + (size_t)row * 64 + 32 * m + 4 * q), load_h4(M + (size_t)row * 64 + 32 * m + 16 + 4 * q));
    Wt[tile * kTile + lane] = v;
}

__global__ void branch_bias_kernel(const float* b0, const float* b1, const float* b2, const float* b3, const float* b4,
                                   const float* b5, const float* b6, const float* b7, const float* b8, const float* b9,
                                   const float* b10, const float* b11, int sh, float* out) {
    const float* B[12] = {b0, b1, b2, b3, b4, b5, b6, b7, b8, b9, b10, b11};
    const bool s = sh != 0;
    const int br = blockIdx.x;
    const int outs[kBr] = {3, 4, s ? 48 : 3, 1};
    float* o = out + branch_bias_off(br, s);
    for (int i = threadIdx.x; i < 128 + 16 * branch_rb(br, s); i += blockDim.x) {
        float v;
        if (i < 64)
            v = B[br * 3][i];
        else if (i < 128)
            v = B[br * 3 + 1][i - 64];
        else
            v = i - 128 < outs[br] ? B[br * 3 + 2][i - 128] : 0.0f;
        o[i] = v;
    }
}

// As gather_f16_kernel, with four fp16 features (8 bytes) per table entry.
__global__ void __launch_bounds__(256) gather_f4_kernel(const float4* xt, int64_t n, int nchunk, HashLevels h,
                                                        const uint2* tables, uint2* zbuf, int64_t zstride) {
#pragma clang fp contract(fast)
    const int level = blockIdx.x / nchunk;
    const int64_t first = (int64_t)(blockIdx.x % nchunk) * 256;
    const int res = h.res_s[level], res_t = h.res_t[level];
    const bool dense = h.dense[level] != 0;
    const uint2* tab = tables + (size_t)level * h.T;
    uint2* zl = zbuf + (size_t)level * zstride;
    const int s = threadIdx.x & 3;
    const int bx = s & 1, by = s >> 1;
    const int sub = threadIdx.x >> 2;
    const uint32_t r = (uint32_t)res, r2 = r * r, r3 = r2 * r;
    // Every corner load of the four passes is issued before any is used; a
    // skipped corner or a lane past the end reads past the table (zero, no
    // memory request), as in the F = 2 gather.
    const __amdgpu_buffer_rsrc_t rt =
        __builtin_amdgcn_make_buffer_rsrc((void*)tab, (short)0, (int)(h.T * 8u), kBufferWord3);
    float4 P[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t i = first + j * 64 + sub;
        P[j] = xt[i < n ? i : n - 1];
    }
    uint2 raw[4][4];
    float wc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool valid = first + j * 64 + sub < n;
        int cx, cy, cz, ct;
        float fx, fy, fz, ft;
        cell_axis(P[j].x, res, cx, fx);
        cell_axis(P[j].y, res, cy, fy);
        cell_axis(P[j].z, res, cz, fz);
        cell_axis(P[j].w, res_t, ct, ft);
        const uint32_t ux = (uint32_t)(cx + bx), uy = (uint32_t)(cy + by);
        uint32_t txy, tz[2], tt[2];
        if (dense) {
            txy = ux + uy * r;
            tz[0] = (uint32_t)cz * r2;
            tz[1] = tz[0] + r2;
            tt[0] = (uint32_t)ct * r3;
            tt[1] = tt[0] + r3;
        } else {
            txy = (ux * kP1) ^ (uy * kP2);
            tz[0] = (uint32_t)cz * kP3;
            tz[1] = (uint32_t)(cz + 1) * kP3;
            tt[0] = (uint32_t)ct * kP4;
            tt[1] = (uint32_t)(ct + 1) * kP4;
        }
        const float wxy = (bx ? fx : 1.0f - fx) * (by ? fy : 1.0f - fy);
        const float wz[2] = {1.0f - fz, fz}, wt[2] = {1.0f - ft, ft};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int bz = k & 1, bt = k >> 1;
            const uint32_t idx = (dense ? (txy + tz[bz] + tt[bt]) : (txy ^ tz[bz] ^ tt[bt])) & h.mask;
            wc[j][k] = (wxy * wz[bz]) * wt[bt];
            // a corner of zero weight adds exactly zero: not fetched
            const uint32_t off = (valid && wc[j][k] != 0.0f) ? idx * 8u : kBufferNone;
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rt, off, 0, 0);
            raw[j][k] = make_uint2(v[0], v[1]);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float w = wc[j][k];
            acc[0] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j][k].x & 0xffffu));
            acc[1] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j][k].x >> 16));
            acc[2] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j][k].y & 0xffffu));
            acc[3] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j][k].y >> 16));
        }
        // sums over the four lanes of the (Gaussian, level): xor 1, then xor 2
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            acc[f] += __builtin_bit_cast(
                float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc[f]), 0xB1, 0xF, 0xF, true));
            acc[f] += __builtin_bit_cast(
                float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc[f]), 0x4E, 0xF, 0xF, true));
        }
        const int64_t i = first + j * 64 + sub;
        if (s == 0 && i < n) {
            uint2 o;
            o.x = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)acc[0]) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)acc[1]) << 16);
            o.y = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)acc[2]) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)acc[3]) << 16);
            zl[i] = o;
        }
    }
}

__device__ __forceinline__ half4_t unpack4(uint2 v) { return unpack2(v.x, v.y); }

// Bias + activation of one 16-row D tile, rounded to fp16 (rows 16 rb + 4 q + e).
template <bool GELU>
__device__ __forceinline__ half4_t act4(floatx4 acc) {
    half4_t h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (_Float16)hidden_act<GELU>(acc[e]);
    return h;
}

// Four biases of a lane (rows 4 q .. 4 q + 3 of a tile) as an initial MFMA
// accumulator: the products then start from the bias, one add fewer per value.
__device__ __forceinline__ floatx4 bias4(const float* b) { return *reinterpret_cast<const floatx4*>(b); }

// Eq. 11 activations from the hardware's one-ulp exp2, rcp and rsq (see the
// shared-trunk decoder); the clamps are v_med3_f32.
__device__ __forceinline__ float exp_clip20_b(float x) {
    return __builtin_amdgcn_exp2f(__builtin_amdgcn_fmed3f(x, -3.402823466e+38f, 20.0f) * 1.44269504088896341f);
}
__device__ __forceinline__ float sigmoid_b(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}

// One hidden layer (64 -> 64) of a branch for kBrG column groups: the output
// k-block mo collects row blocks 2 mo and 2 mo + 1.
template <bool GELU>
__device__ __forceinline__ void hidden_layer(const half8_t* W, const float* bias, const half8_t (&X)[2][kBrG],
                                             half8_t (&Y)[2][kBrG], int lane, int q) {
#pragma unroll
    for (int mo = 0; mo < 2; ++mo) {
        floatx4 lo[kBrG], hi[kBrG];
        const floatx4 b_lo = bias4(bias + 16 * (2 * mo) + 4 * q), b_hi = bias4(bias + 16 * (2 * mo + 1) + 4 * q);
#pragma unroll
        for (int g = 0; g < kBrG; ++g) {
            lo[g] = b_lo;
            hi[g] = b_hi;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const half8_t a_lo = W[(2 * (2 * mo) + m) * kTile + lane];
            const half8_t a_hi = W[(2 * (2 * mo + 1) + m) * kTile + lane];
#pragma unroll
            for (int g = 0; g < kBrG; ++g) {
                lo[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, X[m][g], lo[g], 0, 0, 0);
                hi[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, X[m][g], hi[g], 0, 0, 0);
            }
        }
#pragma unroll
        for (int g = 0; g < kBrG; ++g)
            Y[mo][g] = cat8(act4<GELU>(lo[g]), act4<GELU>(hi[g]));
    }
}

// One branch for kBrG column groups: two hidden layers, the output layer and
// its part of Eq. 11.  The scheduling barriers keep the compiler from
// interleaving branches (their live ranges would not fit the register file).
template <int BR, bool SH, bool GELU>
__device__ __forceinline__ void run_branch(const DecodeArgs& a, const half8_t* s_w, const float* s_b,
                                           const half8_t (&Z)[2][kBrG], int64_t base, int64_t n, int64_t out_off,
                                           int lane, int q, int c) {
    __builtin_amdgcn_sched_barrier(0);
    const half8_t* W = s_w + branch_tile_off(BR, SH) * kTile;
    const float* bias = s_b + branch_bias_off(BR, SH);
    half8_t H1[2][kBrG], H2[2][kBrG];
    hidden_layer<GELU>(W, bias, Z, H1, lane, q);
    __builtin_amdgcn_sched_barrier(0);
    hidden_layer<GELU>(W + 8 * kTile, bias + 64, H1, H2, lane, q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < branch_rb(BR, SH); ++rb) {
        const half8_t a0 = W[(16 + 2 * rb) * kTile + lane], a1 = W[(16 + 2 * rb + 1) * kTile + lane];
#pragma unroll
        for (int g = 0; g < kBrG; ++g) {
            floatx4 acc = bias4(bias + 128 + 16 * rb + 4 * q);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, H2[0][g], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, H2[1][g], acc, 0, 0, 0);
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = acc[e];
            const int64_t gl = base + 16 * g + c;
            if (gl >= n) continue;
            const int64_t gi = out_off + gl;
            // Eq. 11 per branch (rows 16 rb + 4 q + e of the branch output)
            if (BR == 0) {
                if (q == 0)
#pragma unroll
                    for (int e = 0; e < 3; ++e) a.scales[gi * 3 + e] = exp_clip20_b(o[e]);
            } else if (BR == 1) {
                if (q == 0) {
                    const float sq = o[0] * o[0] + (o[1] * o[1] + o[2] * o[2] + o[3] * o[3]);
                    const float inv = __builtin_amdgcn_fmed3f(__builtin_amdgcn_rsqf(sq), 0.0f, 1e12f);
#pragma unroll
                    for (int e = 0; e < 4; ++e) a.quats[gi * 4 + e] = o[e] * inv;
                }
            } else if (BR == 2) {
                if (SH) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) a.sh[gi * 48 + 16 * rb + 4 * q + e] = o[e];
                } else if (q == 0) {
#pragma unroll
                    for (int e = 0; e < 3; ++e) a.colors[gi * 3 + e] = sigmoid_b(o[e]);
                }
            } else if (q == 0) {
                a.opacity[gi] = sigmoid_b(o[0]);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <bool SH, bool GELU>
__global__ void __launch_bounds__(256, 2) mlp_branch_kernel(DecodeArgs a, const uint2* z, int64_t zstride, int64_t n,
                                                            int64_t out_off) {
    constexpr int kT = total_tiles(SH), kB = total_bias(SH);
    __shared__ half8_t s_w[kT * kTile];
    __shared__ __attribute__((aligned(16))) float s_b[kB];
    const half8_t* Wt = (const half8_t*)a.Wt;
    for (int i = threadIdx.x; i < kT * kTile; i += 256) s_w[i] = Wt[i];
    for (int i = threadIdx.x; i < kB; i += 256) s_b[i] = a.bpack[i];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, c = lane & 15;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t base = wave * 16 * kBrG; base < n; base += nwaves * 16 * kBrG) {
        half8_t Z[2][kBrG];
#pragma unroll
        for (int g = 0; g < kBrG; ++g) {
            int64_t gi = base + 16 * g + c;
            if (gi >= n) gi = n - 1;
#pragma unroll
            for (int m = 0; m < 2; ++m)
                Z[m][g] = cat8(unpack4(z[(size_t)(8 * m + q) * zstride + gi]),
                               unpack4(z[(size_t)(8 * m + 4 + q) * zstride + gi]));
        }
        run_branch<0, SH, GELU>(a, s_w, s_b, Z, base, n, out_off, lane, q, c);
        run_branch<1, SH, GELU>(a, s_w, s_b, Z, base, n, out_off, lane, q, c);
        run_branch<2, SH, GELU>(a, s_w, s_b, Z, base, n, out_off, lane, q, c);
        run_branch<3, SH, GELU>(a, s_w, s_b, Z, base, n, out_off, lane, q, c);
    }
}

int grid_cap(int64_t n, int per, int cap) {
    int64_t b = (n + per - 1) / per;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (int)b;
}

}  // namespace

size_t branch_tile_bytes(bool sh) { return (size_t)total_tiles(sh) * kTile * sizeof(half8_t); }
size_t branch_bias_bytes(bool sh) { return (size_t)total_bias(sh) * sizeof(float); }

hipError_t launch_branch_pack(const _Float16* const* W, const float* const* b, bool sh, void* Wt, float* bpack,
                              hipStream_t s) {
    IA_LAUNCH("branch_tiles_kernel", branch_tiles_kernel, dim3(total_tiles(sh)), dim3(64), 0, s, W[0], W[1], W[2],
              W[3], W[4], W[5], W[6], W[7], W[8], W[9], W[10], W[11], sh ? 1 : 0, (half8_t*)Wt);
    IA_LAUNCH("branch_bias_kernel", branch_bias_kernel, dim3(kBr), dim3(64), 0, s, b[0], b[1], b[2], b[3], b[4], b[5],
              b[6], b[7], b[8], b[9], b[10], b[11], sh ? 1 : 0, bpack);
    return hipGetLastError();
}

hipError_t launch_gather_f4(const float4* xt, int64_t n, const HashLevels& h, const void* tables, uint32_t* z,
                            int64_t zstride, hipStream_t s) {
    const int nchunk = (int)((n + 255) / 256);
    IA_LAUNCH("gather_f4_kernel", gather_f4_kernel, dim3((unsigned)(h.L * nchunk)), dim3(256), 0, s, xt, n, nchunk, h,
              (const uint2*)tables, (uint2*)z, zstride);
    return hipGetLastError();
}

hipError_t launch_mlp_branch(const DecodeArgs& a, const uint32_t* z, int64_t zstride, int64_t n, int64_t off,
                             hipStream_t s) {
    // 4 waves x 64 Gaussians per block; the weights fill most of the LDS: two blocks per CU
    const int grid = grid_cap(n, 256, 256 * 2);
    const bool gelu = a.act == IA_ACT_GELU;
    auto k = a.sh_head ? (gelu ? mlp_branch_kernel<true, true> : mlp_branch_kernel<true, false>)
                       : (gelu ? mlp_branch_kernel<false, true> : mlp_branch_kernel<false, false>);
    IA_LAUNCH("mlp_branch_kernel", k, dim3(grid), dim3(256), 0, s, a, (const uint2*)z, zstride, n, off);
    return hipGetLastError();
}

}  // namespace ia
