// HexPlane deformation of canonical Gaussians ("4D Gaussian Splatting详解：
// 动态场景实时渲染的范式突破", §3.1 six feature planes, §3.2 deformation MLP
// predicting position, rotation, scale and SH increments, §6.1 opacity kept).
//
// Per Gaussian: positions map to [0,1] through the box [-aabb, aabb]^3, time
// t in [0,1]; six planes XY XZ YZ (res_xyz^2) and XT YT ZT (res_xyz x res_t)
// of 32 fp16 channels are sampled bilinearly and concatenated (192 features);
// an MLP 192 -> 256 -> 256 -> 58 (ReLU, fp16 MFMA, fp32 accumulation, hidden
// activations rounded to fp16) gives [dpos 3 | dquat 4 | dlog-scale 3 | dSH 48].
//
// MFMA layout (v_mfma_f32_16x16x32_f16, wave64, lane l, q = l/16, c = l%16):
// Gaussians are the columns, neurons the rows; A supplies row c and B column c
// for the same eight k-slots of each lane, D holds rows 4q..4q+3 of column c.
// Slot (q, e) of a 32-wide k-block m stands for input 32 m + 4 q + e (e < 4)
// or 32 m + 16 + 4 q + (e - 4) (e >= 4).  With that assignment the outputs of
// two consecutive 16-row D tiles are exactly the next layer's B operand for
// one 32-wide k-block, and one plane's 32 channels are one k-block of layer 1.
#include <hip/hip_runtime.h>

#include "ia_internal.h"

namespace ia {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half4_t ld4(const _Float16* p) { return *reinterpret_cast<const half4_t*>(p); }

__device__ __forceinline__ half8_t cat8(half4_t lo, half4_t hi) {
    return half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

constexpr int kG = 3;          // 16-Gaussian column groups per wave
constexpr int kHexWaves = 4;   // waves per block (two blocks per CU)
constexpr int kHexThreads = 64 * kHexWaves;
constexpr int kTileHalf8 = 64;  // one A tile = 64 lanes x 8 fp16 = 1 KiB

// Tiled weight buffer (built once per parameter set): A tiles of the three
// layers in the order the kernel streams them through LDS.
//   layer 1: tile (rb, m), rb in 0..15, m in 0..5, at rb * 6 + m
//   layer 2: tile (rb, m), rb in 0..15, m in 0..7, at 96 + rb * 8 + m
//   layer 3: tile (m, rb), m in 0..7, rb in 0..3 (rows >= 58 zero), at 224 + m * 4 + rb
// Tile content: lane (q, c) holds row 16 rb + c at the k-slots of block m.
constexpr int kL1Tiles = 96, kL2Tiles = 128, kL3Tiles = 32;
constexpr int kTiles = kL1Tiles + kL2Tiles + kL3Tiles;

__global__ void tile_weights_kernel(const _Float16* W1, const _Float16* W2, const _Float16* W3, half8_t* Wt) {
    const int tile = blockIdx.x, lane = threadIdx.x;
    const int q = lane >> 4, c = lane & 15;
    const _Float16* W;
    int in_dim, rows, rb, m;
    if (tile < kL1Tiles) {
        W = W1, in_dim = 192, rows = 256, rb = tile / 6, m = tile % 6;
    } else if (tile < kL1Tiles + kL2Tiles) {
        const int t = tile - kL1Tiles;
        W = W2, in_dim = 256, rows = 256, rb = t / 8, m = t % 8;
    } else {
        const int t = tile - kL1Tiles - kL2Tiles;
        W = W3, in_dim = 256, rows = 58, m = t / 4, rb = t % 4;
    }
    const int row = 16 * rb + c;
    half8_t v = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
    if (row < rows) {
        const _Float16* r = W + (size_t)row * in_dim + 32 * m + 4 * q;
        v = cat8(ld4(r), ld4(r + 16));
    }
    Wt[tile * kTileHalf8 + lane] = v;
}

__device__ __forceinline__ void axis_cell(float u, int res, int& i, float& f) {
    float p = u * (float)(res - 1);
    int c = (int)floorf(p);
    c = c < 0 ? 0 : (c > res - 2 ? res - 2 : c);
    i = c;
    f = p - (float)c;
}

// Copy tiles [first, first + N) of the tiled weights into s[0, N) and, with
// N2 > 0, tiles [first2, first2 + N2) into s[N, N + N2) (all threads): every
// load is issued before the first store, so a stage costs one L2 round trip
// rather than one per 4 KiB.
template <int N, int N2 = 0>
__device__ __forceinline__ void stage_tiles(half8_t* s, const half8_t* Wt, int first, int first2 = 0) {
    constexpr int kPer = N * kTileHalf8 / kHexThreads, kPer2 = N2 * kTileHalf8 / kHexThreads;
    static_assert(N * kTileHalf8 % kHexThreads == 0 && N2 * kTileHalf8 % kHexThreads == 0, "whole rounds");
    half8_t v[kPer + kPer2];
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = Wt[first * kTileHalf8 + k * kHexThreads + threadIdx.x];
#pragma unroll
    for (int k = 0; k < kPer2; ++k) v[kPer + k] = Wt[first2 * kTileHalf8 + k * kHexThreads + threadIdx.x];
#pragma unroll
    for (int k = 0; k < kPer + kPer2; ++k) s[k * kHexThreads + threadIdx.x] = v[k];
}

// One block = kHexWaves waves x 16 kG Gaussians.  The weights pass through LDS
// in eight chunks of four row blocks (layer 1: 24 tiles; layer 2: 32 tiles
// plus the 8 layer-3 tiles that consume those rows); each 1 KiB A tile read
// from LDS feeds kG MFMAs (one per 16-Gaussian column group), and row blocks
// go in pairs so that a wave has 2 kG independent accumulation chains.
// Features, hidden layers and accumulators stay in registers; two blocks per
// CU overlap one block's staging with the other's MFMAs.
__global__ void __launch_bounds__(kHexThreads, 2) hexplane_kernel(HexArgs a, const half8_t* Wt) {
#pragma clang fp contract(fast)
    __shared__ half8_t s_w[40 * kTileHalf8];
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, c = lane & 15;
    const int64_t base = ((int64_t)blockIdx.x * kHexWaves + (threadIdx.x >> 6)) * 16 * kG;
    const int C = 32;
    const float t = a.t < 0.0f ? 0.0f : (a.t > 1.0f ? 1.0f : a.t);

    // ---- six bilinear plane lookups -> layer-1 B operand
    half8_t X[6][kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
        int64_t gi = base + 16 * g + c;
        if (gi >= a.N) gi = a.N - 1;
        float u[4];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            float v = a.means[gi * 3 + k] + a.aabb;
            v = v / (2.0f * a.aabb);
            u[k] = v < 0.0f ? 0.0f : (v > 1.0f ? 1.0f : v);
        }
        u[3] = t;
#pragma unroll
        for (int p = 0; p < 6; ++p) {
            const int ax = p == 2 ? 1 : (p == 4 ? 1 : (p == 5 ? 2 : 0));
            const int bx = p == 0 ? 1 : (p == 1 || p == 2 ? 2 : 3);
            const int ra = a.res_xyz, rb = bx == 3 ? a.res_t : a.res_xyz;
            int ia, ib;
            float fa, fb;
            axis_cell(u[ax], ra, ia, fa);
            axis_cell(u[bx], rb, ib, fb);
            const _Float16* P = a.planes[p];
            const _Float16* t00 = P + ((size_t)ib * ra + ia) * C + 4 * q;
            const _Float16* t01 = t00 + C;
            const _Float16* t10 = t00 + (size_t)ra * C;
            const _Float16* t11 = t10 + C;
            const float w00 = (1.0f - fa) * (1.0f - fb), w01 = fa * (1.0f - fb);
            const float w10 = (1.0f - fa) * fb, w11 = fa * fb;
            half8_t out;
#pragma unroll
            for (int hsel = 0; hsel < 2; ++hsel) {
                const int o = 16 * hsel;
                half4_t v00 = ld4(t00 + o), v01 = ld4(t01 + o), v10 = ld4(t10 + o), v11 = ld4(t11 + o);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float s = w00 * (float)v00[e] + w01 * (float)v01[e] + w10 * (float)v10[e] + w11 * (float)v11[e];
                    out[4 * hsel + e] = (_Float16)s;
                }
            }
            X[p][g] = out;
        }
        // materialise this column group's features here (its 48 corner loads
        // are in flight together): left to the compiler, the interpolation
        // sinks to its first use and the raw corner loads of every group stay
        // live across the staging barriers
#pragma unroll
        for (int p = 0; p < 6; ++p) asm volatile("" : "+v"(X[p][g]));
    }

    // ---- layer 1: 192 -> 256, ReLU, fp16; H1[m][g] = k-block m of layer 2's B operand
    half8_t H1[8][kG];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        __syncthreads();
        stage_tiles<24>(s_w, Wt, 24 * r);
        __syncthreads();
        const half8_t* sw = s_w;
        // two row blocks at a time: 2 kG independent accumulation chains,
        // together one k-block of layer 2's B operand
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int rb = 4 * r + 2 * i;
            floatx4 acc0[kG], acc1[kG];
#pragma unroll
            for (int g = 0; g < kG; ++g) acc0[g] = acc1[g] = floatx4{0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < 6; ++m) {
                const half8_t A0 = sw[((2 * i) * 6 + m) * kTileHalf8 + lane];
                const half8_t A1 = sw[((2 * i + 1) * 6 + m) * kTileHalf8 + lane];
#pragma unroll
                for (int g = 0; g < kG; ++g) {
                    acc0[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, X[m][g], acc0[g], 0, 0, 0);
                    acc1[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, X[m][g], acc1[g], 0, 0, 0);
                }
            }
#pragma unroll
            for (int g = 0; g < kG; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v0 = acc0[g][e] + a.b[0][16 * rb + 4 * q + e];
                    const float v1 = acc1[g][e] + a.b[0][16 * (rb + 1) + 4 * q + e];
                    H1[2 * r + i][g][e] = (_Float16)(v0 > 0.0f ? v0 : 0.0f);
                    H1[2 * r + i][g][4 + e] = (_Float16)(v1 > 0.0f ? v1 : 0.0f);
                }
            // convert now (fp32 accumulators would otherwise stay live until
            // layer 2) and keep later row blocks' loads from being hoisted
#pragma unroll
            for (int g = 0; g < kG; ++g) asm volatile("" : "+v"(H1[2 * r + i][g]));
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- layer 2 (256 -> 256, ReLU) streamed into layer 3 (256 -> 58)
    floatx4 acc3[4][kG];
#pragma unroll
    for (int r3 = 0; r3 < 4; ++r3)
#pragma unroll
        for (int g = 0; g < kG; ++g) acc3[r3][g] = floatx4{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        __syncthreads();
        stage_tiles<32, 8>(s_w, Wt, kL1Tiles + 32 * r, kL1Tiles + kL2Tiles + 8 * r);
        __syncthreads();
        const half8_t* sw = s_w;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            // the two row blocks of this k-block of layer 3 together
            const int rb = 4 * r + 2 * half;
            floatx4 acc0[kG], acc1[kG];
#pragma unroll
            for (int g = 0; g < kG; ++g) acc0[g] = acc1[g] = floatx4{0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const half8_t A0 = sw[((2 * half) * 8 + m) * kTileHalf8 + lane];
                const half8_t A1 = sw[((2 * half + 1) * 8 + m) * kTileHalf8 + lane];
#pragma unroll
                for (int g = 0; g < kG; ++g) {
                    acc0[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, H1[m][g], acc0[g], 0, 0, 0);
                    acc1[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, H1[m][g], acc1[g], 0, 0, 0);
                }
            }
            half8_t H2[kG];
#pragma unroll
            for (int g = 0; g < kG; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v0 = acc0[g][e] + a.b[1][16 * rb + 4 * q + e];
                    const float v1 = acc1[g][e] + a.b[1][16 * (rb + 1) + 4 * q + e];
                    H2[g][e] = (_Float16)(v0 > 0.0f ? v0 : 0.0f);
                    H2[g][4 + e] = (_Float16)(v1 > 0.0f ? v1 : 0.0f);
                }
#pragma unroll
            for (int r3 = 0; r3 < 4; ++r3) {
                const half8_t A = sw[(32 + 4 * half + r3) * kTileHalf8 + lane];
#pragma unroll
                for (int g = 0; g < kG; ++g)
                    acc3[r3][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, H2[g], acc3[r3][g], 0, 0, 0);
            }
        }
    }

    // ---- apply the deltas: output o = 16 r3 + 4 q + e
#pragma unroll
    for (int g = 0; g < kG; ++g) {
        const int64_t gi = base + 16 * g + c;
        float d0[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) d0[e] = acc3[0][g][e] + a.b[2][4 * q + e];
        // quaternion: output 3 on q = 0 (e = 3), outputs 4..6 on q = 1 (e = 0..2)
        const int64_t gq = gi < a.N ? gi : a.N - 1;
        float qv[4];
        if (q == 0) {
            qv[0] = a.quats[gq * 4 + 0] + d0[3];
            qv[1] = qv[2] = qv[3] = 0.0f;
        } else if (q == 1) {
            qv[0] = 0.0f;
            qv[1] = a.quats[gq * 4 + 1] + d0[0];
            qv[2] = a.quats[gq * 4 + 2] + d0[1];
            qv[3] = a.quats[gq * 4 + 3] + d0[2];
        } else {
            qv[0] = qv[1] = qv[2] = qv[3] = 0.0f;
        }
        const float part = qv[0] * qv[0] + qv[1] * qv[1] + qv[2] * qv[2] + qv[3] * qv[3];
        const float other = __shfl_xor(part, 16);
        const float inv = 1.0f / fmaxf(sqrtf(part + other), 1e-12f);
        if (gi < a.N) {
            if (q == 0) {
                a.o_means[gi * 3 + 0] = a.means[gi * 3 + 0] + d0[0];
                a.o_means[gi * 3 + 1] = a.means[gi * 3 + 1] + d0[1];
                a.o_means[gi * 3 + 2] = a.means[gi * 3 + 2] + d0[2];
                a.o_quats[gi * 4 + 0] = qv[0] * inv;
                a.o_opacity[gi] = a.opacity[gi];
            } else if (q == 1) {
                a.o_quats[gi * 4 + 1] = qv[1] * inv;
                a.o_quats[gi * 4 + 2] = qv[2] * inv;
                a.o_quats[gi * 4 + 3] = qv[3] * inv;
                a.o_scales[gi * 3 + 0] = a.scales[gi * 3 + 0] * expf(d0[3]);
            } else if (q == 2) {
                a.o_scales[gi * 3 + 1] = a.scales[gi * 3 + 1] * expf(d0[0]);
                a.o_scales[gi * 3 + 2] = a.scales[gi * 3 + 2] * expf(d0[1]);
                a.o_sh[gi * 48 + 0] = a.sh[gi * 48 + 0] + d0[2];
                a.o_sh[gi * 48 + 1] = a.sh[gi * 48 + 1] + d0[3];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) a.o_sh[gi * 48 + 2 + e] = a.sh[gi * 48 + 2 + e] + d0[e];
            }
#pragma unroll
            for (int r3 = 1; r3 < 4; ++r3)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int o = 16 * r3 + 4 * q + e;
                    if (o < 58) a.o_sh[gi * 48 + (o - 10)] = a.sh[gi * 48 + (o - 10)] + acc3[r3][g][e] + a.b[2][o];
                }
        }
    }
}

}  // namespace

hipError_t launch_hexplane_tiles(const _Float16* const W[3], void* Wt, hipStream_t s) {
    IA_LAUNCH("tile_weights_kernel", tile_weights_kernel, dim3(kTiles), dim3(64), 0, s, W[0], W[1], W[2],
              static_cast<half8_t*>(Wt));
    return hipGetLastError();
}

hipError_t launch_hexplane(const HexArgs& a, const void* Wt, hipStream_t s) {
    if (a.N <= 0) return hipSuccess;
    const int64_t per_block = kHexWaves * 16 * kG;
    const int64_t grid = (a.N + per_block - 1) / per_block;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    IA_LAUNCH("hexplane_kernel", hexplane_kernel, dim3((unsigned)grid), dim3(kHexThreads), 0, s, a,
              static_cast<const half8_t*>(Wt));
    return hipGetLastError();
}

}  // namespace ia
