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
// In layers 2 and 3, slot (q, e) of a 32-wide k-block m stands for input
// 32 m + 4 q + e (e < 4) or 32 m + 16 + 4 q + (e - 4) (e >= 4): with that
// assignment the outputs of two consecutive 16-row D tiles are exactly the
// next layer's B operand for one 32-wide k-block.  In layer 1, one plane's 32
// channels are one k-block and slot (q, e) stands for channel 8 q + e, so that
// a lane's eight features come from one 16-byte load per plane corner.
#include <hip/hip_runtime.h>

#include "ia_internal.h"

namespace ia {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half4_t ld4(const _Float16* p) { return *reinterpret_cast<const half4_t*>(p); }
__device__ __forceinline__ half8_t ld8(const _Float16* p) { return *reinterpret_cast<const half8_t*>(p); }

__device__ __forceinline__ half8_t cat8(half4_t lo, half4_t hi) {
    return half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

constexpr int kG = 3;          // 16-Gaussian column groups per wave
constexpr int kHexWaves = 4;   // waves per block (two blocks per CU, one wave of each per SIMD)
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
        if (tile < kL1Tiles) {  // layer 1: slot e of lane group q is input 32 m + 8 q + e
            v = *reinterpret_cast<const half8_t*>(W + (size_t)row * in_dim + 32 * m + 8 * q);
        } else {
            const _Float16* r = W + (size_t)row * in_dim + 32 * m + 4 * q;
            v = cat8(ld4(r), ld4(r + 16));
        }
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

// The weights pass through LDS in twelve stages: layer 1 in four of four row
// blocks (24 tiles), layer 2 in eight of two row blocks (16 tiles) with the 4
// layer-3 tiles of the k-block those rows form.  Stage st's tiles are copied
// global -> LDS by the LDS-DMA loads (one 1 KiB tile per wave instruction, no
// registers) into buffer st % 3, two stages ahead of their use: the copy has
// two stages' time to land.  Twelve stages keep st % 3 the same in every
// sub-batch.
constexpr int kStages = 12;
constexpr int kStageTiles = 24;

__device__ __forceinline__ int stage_tiles_of(int st) { return st < 4 ? 24 : 20; }

__device__ __forceinline__ int stage_tile(int st, int j) {
    if (st < 4) return 24 * st + j;
    const int r = st - 4;
    return j < 16 ? kL1Tiles + 16 * r + j : kL1Tiles + kL2Tiles + 4 * r + (j - 16);
}

// Issue the copies of stage st into buf (wave w copies tiles w, w + kHexWaves,
// ...; every wave issues stage_tiles_of(st) / kHexWaves of them).
__device__ __forceinline__ void issue_stage(half8_t* buf, const half8_t* Wt, int st, int wave, int lane) {
    const int n = stage_tiles_of(st);
    for (int j = wave; j < n; j += kHexWaves)
        __builtin_amdgcn_global_load_lds((const void*)(Wt + stage_tile(st, j) * kTileHalf8 + lane),
                                         (__attribute__((address_space(3))) void*)(buf + j * kTileHalf8), 16, 0, 0);
}

// LDS written by the lanes of one wave is read back by other lanes of the same
// wave: order the accesses at wavefront scope.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kEpiStride = 61;  // floats per LDS row of deltas (58 used; odd: fewer bank conflicts)
static_assert(kHexWaves * 16 * kEpiStride * 4 <= kStageTiles * kTileHalf8 * 16, "delta rows fit a stage buffer");

// The LDS-DMA copies of this wave are done (vmcnt counts them in issue order).
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// All but the last `later` vector-memory operations of this wave are done
// (the copies of a stage issued after those being waited for).
__device__ __forceinline__ void wait_copies_but(int later) {
    if (later == 6)
        asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if (later == 5)
        asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

struct HexShared {
    half8_t* w0;
    half8_t* w1;
    half8_t* w2;
    const float* sb1;
    const float* sb2;
    const float* sb3;
};

__device__ __forceinline__ half8_t* stage_buf(const HexShared& sh, int st) {
    const int b = st % 3;
    return b == 0 ? sh.w0 : (b == 1 ? sh.w1 : sh.w2);
}

// One sub-batch of one wave: K (0..3) 16-Gaussian column groups starting at
// Gaussian g0.  Every wave of the block runs the same sequence of stage
// copies and barriers whatever its K (K = 0 only takes part in them), so
// waves with different amounts of work stay in step.  Each 1 KiB A tile read
// from LDS feeds K MFMAs (one per column group), and row blocks go in pairs
// so that a wave has 2 K independent accumulation chains.  Features, hidden
// layers and accumulators stay in registers.  The compute phases issue no
// global loads, so waiting for a stage's copies never waits for anything
// issued after them.  With `more`, stage 0 of the block's next sub-batch is
// copied during the last stage.
template <int K>
__device__ __forceinline__ void hex_sub_batch(const HexArgs& a, const half8_t* Wt, const HexShared& sh, int64_t g0,
                                              bool more, int wave, int lane, float t_raw) {
#pragma clang fp contract(fast)
    constexpr int KK = K > 0 ? K : 1;  // array extents
    const int q = lane >> 4, c = lane & 15;
    const int C = 32;
    const float t = t_raw < 0.0f ? 0.0f : (t_raw > 1.0f ? 1.0f : t_raw);

    // ---- six bilinear plane lookups -> layer-1 B operand.  The positions of
    // all groups are loaded first, then each group's 24 corner loads are
    // issued together (one round trip per group).
    float u[KK][3];
#pragma unroll
    for (int g = 0; g < K; ++g) {
        int64_t gi = g0 + 16 * g + c;
        if (gi >= a.N) gi = a.N - 1;
#pragma unroll
        for (int k = 0; k < 3; ++k) u[g][k] = a.means[gi * 3 + k];
    }
    half8_t X[6][KK];
#pragma unroll
    for (int g = 0; g < K; ++g) {
        float uu[4];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            float v = u[g][k] + a.aabb;
            v = v / (2.0f * a.aabb);
            uu[k] = v < 0.0f ? 0.0f : (v > 1.0f ? 1.0f : v);
        }
        uu[3] = t;
        half8_t raw[6][4];
        float wgt[6][4];
#pragma unroll
        for (int p = 0; p < 6; ++p) {
            const int ax = p == 2 ? 1 : (p == 4 ? 1 : (p == 5 ? 2 : 0));
            const int bx = p == 0 ? 1 : (p == 1 || p == 2 ? 2 : 3);
            const int ra = a.res_xyz, rb = bx == 3 ? a.res_t : a.res_xyz;
            int ia, ib;
            float fa, fb;
            axis_cell(uu[ax], ra, ia, fa);
            axis_cell(uu[bx], rb, ib, fb);
            const _Float16* t00 = a.planes[p] + ((size_t)ib * ra + ia) * C + 8 * q;
            raw[p][0] = ld8(t00);
            raw[p][1] = ld8(t00 + C);
            raw[p][2] = ld8(t00 + (size_t)ra * C);
            raw[p][3] = ld8(t00 + (size_t)ra * C + C);
            wgt[p][0] = (1.0f - fa) * (1.0f - fb);
            wgt[p][1] = fa * (1.0f - fb);
            wgt[p][2] = (1.0f - fa) * fb;
            wgt[p][3] = fa * fb;
        }
        // every corner load of the group is issued before any is used (the
        // memory clobber keeps them above this point)
        asm volatile("" : "+v"(raw[0][0]), "+v"(raw[0][1]), "+v"(raw[0][2]), "+v"(raw[0][3])::"memory");
#pragma unroll
        for (int p = 1; p < 6; ++p)
            asm volatile("" : "+v"(raw[p][0]), "+v"(raw[p][1]), "+v"(raw[p][2]), "+v"(raw[p][3]));
#pragma unroll
        for (int p = 0; p < 6; ++p) {
            half8_t out;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float s = wgt[p][0] * (float)raw[p][0][e] + wgt[p][1] * (float)raw[p][1][e] +
                          wgt[p][2] * (float)raw[p][2][e] + wgt[p][3] * (float)raw[p][3][e];
                out[e] = (_Float16)s;
            }
            X[p][g] = out;
        }
        // materialise this column group's features here: left to the
        // compiler, the interpolation sinks to its first use and the raw
        // corner values of every group stay live across the stage barriers
#pragma unroll
        for (int p = 0; p < 6; ++p) asm volatile("" : "+v"(X[p][g]));
    }
    wait_copies();
    __syncthreads();

    // ---- layer 1: 192 -> 256, ReLU, fp16; H1[m][g] = k-block m of layer 2's B
    // operand (row blocks 2 m, 2 m + 1)
    half8_t H1[8][KK];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        // stage st + 2 copies while this one computes
        issue_stage(stage_buf(sh, st + 2), Wt, st + 2, wave, lane);
        const half8_t* sw = stage_buf(sh, st);
        if constexpr (K > 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                // row blocks in pairs: 2 K independent accumulation chains
                const int rb = 4 * st + 2 * i;
                floatx4 acc0[KK], acc1[KK];
#pragma unroll
                for (int g = 0; g < K; ++g) acc0[g] = acc1[g] = floatx4{0, 0, 0, 0};
                // the next k-block's A tiles are read while this one's MFMAs run
                half8_t A0 = sw[((2 * i) * 6) * kTileHalf8 + lane];
                half8_t A1 = sw[((2 * i + 1) * 6) * kTileHalf8 + lane];
#pragma unroll
                for (int m = 0; m < 6; ++m) {
                    half8_t N0 = A0, N1 = A1;
                    if (m < 5) {
                        N0 = sw[((2 * i) * 6 + m + 1) * kTileHalf8 + lane];
                        N1 = sw[((2 * i + 1) * 6 + m + 1) * kTileHalf8 + lane];
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int g = 0; g < K; ++g) {
                        acc0[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, X[m][g], acc0[g], 0, 0, 0);
                        acc1[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, X[m][g], acc1[g], 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    A0 = N0;
                    A1 = N1;
                }
#pragma unroll
                for (int g = 0; g < K; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v0 = acc0[g][e] + sh.sb1[16 * rb + 4 * q + e];
                        const float v1 = acc1[g][e] + sh.sb1[16 * (rb + 1) + 4 * q + e];
                        H1[rb >> 1][g][e] = (_Float16)(v0 > 0.0f ? v0 : 0.0f);
                        H1[rb >> 1][g][4 + e] = (_Float16)(v1 > 0.0f ? v1 : 0.0f);
                    }
                // convert now (fp32 accumulators would otherwise stay live until
                // layer 2) and keep later row blocks' loads from being hoisted
#pragma unroll
                for (int g = 0; g < K; ++g) asm volatile("" : "+v"(H1[rb >> 1][g]));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // stage st + 1's copies have landed (st + 2's may still be in flight)
        wait_copies_but(stage_tiles_of(st + 2) / kHexWaves);
        __syncthreads();
    }

    // ---- layer 2 (256 -> 256, ReLU) streamed into layer 3 (256 -> 58): stage
    // 4 + r gives row blocks 2 r, 2 r + 1 of layer 2, i.e. k-block r of layer 3
    floatx4 acc3[4][KK];
#pragma unroll
    for (int r3 = 0; r3 < 4; ++r3)
#pragma unroll
        for (int g = 0; g < K; ++g) acc3[r3][g] = floatx4{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int st = 4 + r;
        // stage st + 2 (or, past the end, the next sub-batch's stage 0 or 1)
        // copies while this one computes
        if (st + 2 < kStages)
            issue_stage(stage_buf(sh, st + 2), Wt, st + 2, wave, lane);
        else if (more)
            issue_stage(stage_buf(sh, st + 2), Wt, st + 2 - kStages, wave, lane);
        const half8_t* sw = stage_buf(sh, st);
        if constexpr (K > 0) {
            const int rb = 2 * r;
            floatx4 acc0[KK], acc1[KK];
#pragma unroll
            for (int g = 0; g < K; ++g) acc0[g] = acc1[g] = floatx4{0, 0, 0, 0};
            half8_t A0 = sw[0 * kTileHalf8 + lane];
            half8_t A1 = sw[8 * kTileHalf8 + lane];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                half8_t N0 = A0, N1 = A1;
                if (m < 7) {
                    N0 = sw[(m + 1) * kTileHalf8 + lane];
                    N1 = sw[(8 + m + 1) * kTileHalf8 + lane];
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < K; ++g) {
                    acc0[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, H1[m][g], acc0[g], 0, 0, 0);
                    acc1[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, H1[m][g], acc1[g], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                A0 = N0;
                A1 = N1;
            }
            half8_t H2[KK];
#pragma unroll
            for (int g = 0; g < K; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v0 = acc0[g][e] + sh.sb2[16 * rb + 4 * q + e];
                    const float v1 = acc1[g][e] + sh.sb2[16 * (rb + 1) + 4 * q + e];
                    H2[g][e] = (_Float16)(v0 > 0.0f ? v0 : 0.0f);
                    H2[g][4 + e] = (_Float16)(v1 > 0.0f ? v1 : 0.0f);
                }
#pragma unroll
            for (int r3 = 0; r3 < 4; ++r3) {
                const half8_t A = sw[(16 + r3) * kTileHalf8 + lane];
#pragma unroll
                for (int g = 0; g < K; ++g)
                    acc3[r3][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, H2[g], acc3[r3][g], 0, 0, 0);
            }
        }
        // stage st + 1's copies have landed (st + 2's may still be in flight)
        if (st + 1 < kStages) {
            if (st + 2 < kStages)
                wait_copies_but(stage_tiles_of(st + 2) / kHexWaves);
            else
                wait_copies_but(more ? stage_tiles_of(0) / kHexWaves : 0);
            __syncthreads();
        }
    }

    // ---- apply the deltas.  Lane (q, c) holds outputs o = 16 r3 + 4 q + e of
    // Gaussian c of a column group; they go through this wave's LDS rows (one
    // per Gaussian), so that the canonical values are read and the deformed
    // ones written with consecutive lanes on consecutive addresses (a group's
    // 16 Gaussians are consecutive in every array).  The canonical values of
    // all of the wave's groups are loaded first, in flight together.
    // The last stage's buffer is free until the next sub-batch's stage 2 is
    // copied into it: every wave is done reading it after this barrier.
    __syncthreads();
    float* sE = reinterpret_cast<float*>(stage_buf(sh, kStages - 1)) + wave * (16 * kEpiStride);
    float csh[KK][12], cm[KK], cs[KK], cq[KK], co[KK];
#pragma unroll
    for (int g = 0; g < K; ++g) {
        const int64_t b0 = g0 + 16 * g;
        const int nv = a.N - b0 < 16 ? (int)(a.N - b0) : 16;  // Gaussians of the group that exist
#pragma unroll
        for (int j = 0; j < 12; ++j) csh[g][j] = lane + 64 * j < nv * 48 ? a.sh[b0 * 48 + lane + 64 * j] : 0.0f;
        cm[g] = lane < nv * 3 ? a.means[b0 * 3 + lane] : 0.0f;
        cs[g] = lane < nv * 3 ? a.scales[b0 * 3 + lane] : 0.0f;
        cq[g] = lane < nv * 4 ? a.quats[b0 * 4 + lane] : 0.0f;
        co[g] = lane < nv ? a.opacity[b0 + lane] : 0.0f;
    }
#pragma unroll
    for (int g = 0; g < K; ++g) {
        const int64_t b0 = g0 + 16 * g;
        const int nv = a.N - b0 < 16 ? (int)(a.N - b0) : 16;
#pragma unroll
        for (int r3 = 0; r3 < 4; ++r3)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int o = 16 * r3 + 4 * q + e;
                if (o < 58) sE[c * kEpiStride + o] = acc3[r3][g][e] + sh.sb3[o];
            }
        wave_lds_sync();
        // SH: 16 x 48 consecutive floats
#pragma unroll
        for (int j = 0; j < 12; ++j) {
            const int k = lane + 64 * j;
            if (k < nv * 48) {
                const int r = k / 48;
                a.o_sh[b0 * 48 + k] = csh[g][j] + sE[r * kEpiStride + 10 + (k - 48 * r)];
            }
        }
        // means, scales: 16 x 3 consecutive floats each
        if (lane < nv * 3) {
            const int r = lane / 3, i = lane - 3 * r;
            a.o_means[b0 * 3 + lane] = cm[g] + sE[r * kEpiStride + i];
            a.o_scales[b0 * 3 + lane] = cs[g] * expf(sE[r * kEpiStride + 7 + i]);
        }
        // rotation normalize(q + dq): lanes 4 r .. 4 r + 3 hold Gaussian r's
        // four components; the squared norm is summed over the four lanes
        {
            const int r = lane >> 2, i = lane & 3;
            const float v = cq[g] + (r < nv ? sE[r * kEpiStride + 3 + i] : 0.0f);
            float n2 = v * v;
            n2 += __shfl_xor(n2, 1);
            n2 += __shfl_xor(n2, 2);
            const float inv = 1.0f / fmaxf(sqrtf(n2), 1e-12f);
            if (lane < nv * 4) a.o_quats[b0 * 4 + lane] = v * inv;
        }
        if (lane < nv) a.o_opacity[b0 + lane] = co[g];  // opacity kept
        wave_lds_sync();  // this wave's rows are rewritten by the next group
    }
    // the next sub-batch's first two stages are in this wave's queue: they and
    // every wave's copies land before that sub-batch's layer 1 reads them
    wait_copies();
    __syncthreads();
}

// Two blocks per compute unit, persistent over an equal share each of the
// 16-Gaussian column groups (block b: groups [b G / B, (b + 1) G / B)).  The
// share goes in sub-batches of up to kHexWaves * kG groups; in each, wave w
// takes a contiguous run of floor or ceil (groups / kHexWaves) of them, so the
// last, partial sub-batch is spread over the waves instead of falling to a
// few of them, and no block has more than one partial sub-batch.
__global__ void __launch_bounds__(kHexThreads, 2) hexplane_kernel(HexArgs a, const half8_t* Wt) {
    // three distinct LDS objects (not one array): the compiler can then tell
    // that one stage's reads do not touch the buffers later stages are copied into
    __shared__ half8_t s_w0[kStageTiles * kTileHalf8];
    __shared__ half8_t s_w1[kStageTiles * kTileHalf8];
    __shared__ half8_t s_w2[kStageTiles * kTileHalf8];
    __shared__ float s_b[256 + 256 + 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int k = threadIdx.x; k < 256 + 256 + 64; k += kHexThreads)
        s_b[k] = k < 256 ? a.b[0][k] : (k < 512 ? a.b[1][k - 256] : (k - 512 < 58 ? a.b[2][k - 512] : 0.0f));
    const HexShared sh{s_w0, s_w1, s_w2, s_b, s_b + 256, s_b + 512};

    const int64_t groups = (a.N + 15) / 16;
    const int64_t lo = groups * blockIdx.x / gridDim.x, hi = groups * (blockIdx.x + 1) / gridDim.x;
    if (hi > lo) {
        issue_stage(s_w0, Wt, 0, wave, lane);
        issue_stage(s_w1, Wt, 1, wave, lane);
    }
    // The second half of the grid (the other block on a compute unit, as the
    // blocks are dispatched) starts with a half sub-batch: the two blocks of a
    // compute unit are then out of phase, and one's plane lookups and stores
    // overlap the other's MFMAs instead of competing with them.
    const bool shifted = gridDim.x > 1 && blockIdx.x >= gridDim.x / 2;
    for (int64_t first = lo; first < hi;) {
        const int cap = first == lo && shifted ? kHexWaves * kG / 2 : kHexWaves * kG;
        const int n = (int)(hi - first < cap ? hi - first : cap);
        const int k = n / kHexWaves + (wave < n % kHexWaves ? 1 : 0);
        const int64_t g0 = 16 * (first + (int64_t)wave * (n / kHexWaves) + (wave < n % kHexWaves ? wave : n % kHexWaves));
        first += n;
        const bool more = first < hi;
        // opaque copies of the lane and wave indices and of t: what derives
        // from them (corner, tile and bias addresses, the time cell) is then
        // recomputed per sub-batch instead of being hoisted out of this loop
        // and held in registers across it
        int ln = lane, wv = wave;
        float tv = a.t;
        asm volatile("" : "+v"(ln), "+v"(wv), "+v"(tv));
        if (k == 3)
            hex_sub_batch<3>(a, Wt, sh, g0, more, wv, ln, tv);
        else if (k == 2)
            hex_sub_batch<2>(a, Wt, sh, g0, more, wv, ln, tv);
        else if (k == 1)
            hex_sub_batch<1>(a, Wt, sh, g0, more, wv, ln, tv);
        else
            hex_sub_batch<0>(a, Wt, sh, g0, more, wv, ln, tv);
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
    // two blocks per compute unit (fewer when there are fewer than
    // 2 kHexWaves groups per compute unit), each over an equal share of groups;
    // one block's lookups and stores overlap the other's MFMAs
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    const int64_t groups = (a.N + 15) / 16;
    const int64_t want = (groups + kHexWaves - 1) / kHexWaves;
    const int64_t grid = want < 2 * cus ? want : 2 * cus;
    IA_LAUNCH("hexplane_kernel", hexplane_kernel, dim3((unsigned)grid), dim3(kHexThreads), 0, s, a,
              static_cast<const half8_t*>(Wt));
    return hipGetLastError();
}

}  // namespace ia
