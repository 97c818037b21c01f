// Implicit attribute decode (SPIN-4DGS, "Implicit 4D Gaussian Splatting for
// Fast Motion with Large Inter-Frame Displacements", §3.3 Eq. 7-11):
//   position + t -> contraction / normalisation (Eq. 7-8)
//               -> 4D multiresolution hash encoding, 16-corner quadrilinear
//                  interpolation per level, levels concatenated (Eq. 9)
//               -> shared MLP trunk + linear head block (Eq. 10)
//               -> exp / normalise / sigmoid activations (Eq. 11).
//
// Paths:
//   decode_f32_kernel : fp32 VALU, one thread per Gaussian, weights in LDS
//                       (small tables: the 4-level fp32 grid).
//   fp16 path         : 16 levels x 2 features, 32->64->64->11 decoder.  A
//                       level-major gather kernel (one level's table resident
//                       in L2 at a time) writes the features to a scratch
//                       buffer owned by the decoder handle; an MLP kernel runs
//                       the decoder on v_mfma_f32_16x16x32_f16 with fp32
//                       accumulation and applies Eq. 11.
//
// Position normalisation and the per-axis cell decision are computed one IEEE
// fp32 operation at a time in the order written (the library is built with
// -ffp-contract=off), so the chosen cell matches any other implementation of
// the same formula bit for bit; interpolation and the MLP allow contraction.
#include <hip/hip_runtime.h>

#include "decode_common.h"
#include "ia_internal.h"

namespace ia {
namespace {

// Quadrilinear interpolation of one level with F = 2 features.  The table of
// the level starts at `tab` (T entries of 2 features).  Index per corner is
// a separable combination of per-axis terms: sum (dense, row-major x fastest)
// or XOR of coordinate * prime (hashed), then mod T.
template <bool F16>
__device__ __forceinline__ void interp_level2(const void* tab, const float xt[4], int res, int res_t, int dense,
                                              uint32_t mask, float& z0, float& z1) {
#pragma clang fp contract(fast)
    int ci[4];
    float f[4];
    cell_axis(xt[0], res, ci[0], f[0]);
    cell_axis(xt[1], res, ci[1], f[1]);
    cell_axis(xt[2], res, ci[2], f[2]);
    cell_axis(xt[3], res_t, ci[3], f[3]);
    uint32_t tx[2], ty[2], tz[2], tt[2];
    if (dense) {
        uint32_t r = (uint32_t)res, r2 = r * r, r3 = r2 * r;
        tx[0] = (uint32_t)ci[0];
        tx[1] = tx[0] + 1u;
        ty[0] = (uint32_t)ci[1] * r;
        ty[1] = ty[0] + r;
        tz[0] = (uint32_t)ci[2] * r2;
        tz[1] = tz[0] + r2;
        tt[0] = (uint32_t)ci[3] * r3;
        tt[1] = tt[0] + r3;
    } else {
        tx[0] = (uint32_t)ci[0] * kP1;
        tx[1] = (uint32_t)(ci[0] + 1) * kP1;
        ty[0] = (uint32_t)ci[1] * kP2;
        ty[1] = (uint32_t)(ci[1] + 1) * kP2;
        tz[0] = (uint32_t)ci[2] * kP3;
        tz[1] = (uint32_t)(ci[2] + 1) * kP3;
        tt[0] = (uint32_t)ci[3] * kP4;
        tt[1] = (uint32_t)(ci[3] + 1) * kP4;
    }
    float wx[2] = {1.0f - f[0], f[0]}, wy[2] = {1.0f - f[1], f[1]};
    float wz[2] = {1.0f - f[2], f[2]}, wt[2] = {1.0f - f[3], f[3]};
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        int bx = c & 1, by = (c >> 1) & 1, bz = (c >> 2) & 1, bt = (c >> 3) & 1;
        uint32_t idx = dense ? (tx[bx] + ty[by] + tz[bz] + tt[bt]) : (tx[bx] ^ ty[by] ^ tz[bz] ^ tt[bt]);
        idx &= mask;
        float w = ((wx[bx] * wy[by]) * wz[bz]) * wt[bt];
        float v0, v1;
        if (F16) {
            uint32_t raw = reinterpret_cast<const uint32_t*>(tab)[idx];
            _Float16 h0 = __builtin_bit_cast(_Float16, (uint16_t)(raw & 0xffffu));
            _Float16 h1 = __builtin_bit_cast(_Float16, (uint16_t)(raw >> 16));
            v0 = (float)h0;
            v1 = (float)h1;
        } else {
            float2 v = reinterpret_cast<const float2*>(tab)[idx];
            v0 = v.x;
            v1 = v.y;
        }
        a0 += w * v0;
        a1 += w * v1;
    }
    z0 = a0;
    z1 = a1;
}

__device__ __forceinline__ float act_fn(int act, float x) {
    if (act == IA_ACT_RELU) return x > 0.0f ? x : 0.0f;
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}


// ---------------------------------------------------------------- fp32 path

constexpr int kF32MaxIn = 32, kF32MaxH = 64;

template <int LF, int H1, int H2>
__global__ void __launch_bounds__(256, 2) decode_f32_kernel(DecodeArgs a) {
    // weights: W1 [H1][LF], W2 [H2][H1] (if H2 > 0), Wh [11][HL]
    constexpr int HL = H2 > 0 ? H2 : H1;
    __shared__ float sW1[H1 * LF];
    __shared__ float sW2[H2 > 0 ? H2 * H1 : 1];
    __shared__ float sWh[11 * HL];
    __shared__ float sb1[H1], sb2[H2 > 0 ? H2 : 1], sbh[11];
    const float* W1 = (const float*)a.W[0];
    const float* W2 = (const float*)a.W[1];
    const float* Wh = (const float*)a.W[H2 > 0 ? 2 : 1];
    for (int k = threadIdx.x; k < H1 * LF; k += blockDim.x) sW1[k] = W1[k];
    if (H2 > 0)
        for (int k = threadIdx.x; k < H2 * H1; k += blockDim.x) sW2[k] = W2[k];
    for (int k = threadIdx.x; k < 11 * HL; k += blockDim.x) sWh[k] = Wh[k];
    for (int k = threadIdx.x; k < H1; k += blockDim.x) sb1[k] = a.b[0][k];
    if (H2 > 0)
        for (int k = threadIdx.x; k < H2; k += blockDim.x) sb2[k] = a.b[1][k];
    for (int k = threadIdx.x; k < 11; k += blockDim.x) sbh[k] = a.b[H2 > 0 ? 2 : 1][k];
    __syncthreads();

    const int L = LF / 2;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < a.N) {
        const float* p = a.pos + i * a.stride;
        float xt[4];
        normalize_pos(p[0], p[1], p[2], a.stride == 4 ? p[3] : a.t_scalar, a.h.t_min, a.h.t_max, xt);
        float z[LF];
#pragma unroll
        for (int l = 0; l < L; ++l) {
            const size_t off = (size_t)l * a.h.T * 2;
            if (a.h.table_f16)
                interp_level2<true>((const _Float16*)a.tables + off, xt, a.h.res_s[l], a.h.res_t[l], a.h.dense[l],
                                    a.h.mask, z[2 * l], z[2 * l + 1]);
            else
                interp_level2<false>((const float*)a.tables + off, xt, a.h.res_s[l], a.h.res_t[l], a.h.dense[l],
                                     a.h.mask, z[2 * l], z[2 * l + 1]);
        }
        float h1[H1];
#pragma unroll
        for (int o = 0; o < H1; ++o) {
            float s = 0.0f;
#pragma unroll
            for (int k = 0; k < LF; ++k) s = fmaf(sW1[o * LF + k], z[k], s);
            h1[o] = act_fn(a.act, s + sb1[o]);
        }
        float hl[HL];
        if (H2 > 0) {
#pragma unroll
            for (int o = 0; o < HL; ++o) {
                float s = 0.0f;
#pragma unroll
                for (int k = 0; k < H1; ++k) s = fmaf(sW2[o * H1 + k], h1[k], s);
                hl[o] = act_fn(a.act, s + sb2[o]);
            }
        } else {
#pragma unroll
            for (int o = 0; o < HL; ++o) hl[o] = h1[o];
        }
        float r[11];
#pragma unroll
        for (int o = 0; o < 11; ++o) {
            float s = 0.0f;
#pragma unroll
            for (int k = 0; k < HL; ++k) s = fmaf(sWh[o * HL + k], hl[k], s);
            r[o] = s + sbh[o];
        }
        // Eq. 11
        a.scales[i * 3 + 0] = expf(fminf(r[0], 20.0f));
        a.scales[i * 3 + 1] = expf(fminf(r[1], 20.0f));
        a.scales[i * 3 + 2] = expf(fminf(r[2], 20.0f));
        float n = sqrtf(r[3] * r[3] + r[4] * r[4] + r[5] * r[5] + r[6] * r[6]);
        n = fmaxf(n, 1e-12f);
        a.quats[i * 4 + 0] = r[3] / n;
        a.quats[i * 4 + 1] = r[4] / n;
        a.quats[i * 4 + 2] = r[5] / n;
        a.quats[i * 4 + 3] = r[6] / n;
        a.colors[i * 3 + 0] = sigmoidf_(r[7]);
        a.colors[i * 3 + 1] = sigmoidf_(r[8]);
        a.colors[i * 3 + 2] = sigmoidf_(r[9]);
        a.opacity[i] = sigmoidf_(r[10]);
    }
}

// ---------------------------------------------------------------- fp16 path
//
// Two kernels per chunk of at most zcap Gaussians:
//
// normalize_kernel: Eq. 7-8 once per Gaussian -> x~ (fp32 x4) in the scratch.
//
// gather_f16_kernel: level-major.  Block b handles level b / nchunk and
// Gaussians [256 (b % nchunk), +256).  Blocks are dispatched in index order
// and spread round-robin over the XCDs, so at any moment all XCDs work on the
// same level and that level's 2^log2T x 4-byte table stays resident in every
// XCD's L2 instead of being fetched line by line from HBM / Infinity Cache.
// Four lanes share one (Gaussian, level): lane s takes the x-corner s & 1 and
// the y-corner s >> 1 and loops over the four (z, t) corners.  Under the hash
// (first prime 1) the two x-corners differ only in their low index bits, so
// neighbouring lanes usually hit the same cache line inside one load
// instruction, halving the distinct lines each gather touches.  Two quad
// shuffles sum the four partial results.  Output z[level][i] = two fp16
// features packed in 32 bits (RNE).
//
// mlp_f16_kernel: the 32 -> 64 -> 64 -> 11 (or 56, SH colour) decoder on
// v_mfma_f32_16x16x32_f16.
// Register layout (wave64, lane l, q = l/16, c = l%16): A supplies row c and
// B column c, each with eight k-slots per lane that A and B share; D holds
// rows 4q..4q+3 of column c.  Gaussians are the columns and neurons the rows.

constexpr int kGatherPerBlock = 256;  // Gaussians per gather block (64 per pass x 4 passes)
constexpr int kMlpCusPerBlock = 2;    // MLP beside a gather: one block per this many CUs
constexpr int kNormBlocksPerCu = 2;   // normalisation beside a gather: blocks per CU

__global__ void __launch_bounds__(256) normalize_kernel(DecodeArgs a, const float* pos, int64_t n, float4* xt) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const float* p = pos + i * a.stride;
        float v[4];
        normalize_pos(p[0], p[1], p[2], a.stride == 4 ? p[3] : a.t_scalar, a.h.t_min, a.h.t_max, v);
        xt[i] = make_float4(v[0], v[1], v[2], v[3]);
    }
}

__global__ void __launch_bounds__(256) gather_f16_kernel(const float4* xt, int64_t n, int nchunk, HashLevels h,
                                                         const uint32_t* tables, uint32_t* zbuf, int64_t zstride) {
#pragma clang fp contract(fast)
    const int level = blockIdx.x / nchunk;
    const int64_t first = (int64_t)(blockIdx.x % nchunk) * kGatherPerBlock;
    const int res = h.res_s[level], res_t = h.res_t[level];
    const bool dense = h.dense[level] != 0;
    const uint32_t* tab = tables + (size_t)level * h.T;
    uint32_t* zl = zbuf + (size_t)level * zstride;
    const int s = threadIdx.x & 3;           // corner pair this lane takes
    const int bx = s & 1, by = s >> 1;
    const int sub = threadIdx.x >> 2;        // Gaussian slot within a pass (0..63)
    const uint32_t r = (uint32_t)res, r2 = r * r, r3 = r2 * r;
#pragma unroll 2
    for (int j = 0; j < kGatherPerBlock / 64; ++j) {
        const int64_t i = first + j * 64 + sub;
        if (i >= n) break;  // uniform across each group of four lanes
        const float4 p = xt[i];
        int cx, cy, cz, ct;
        float fx, fy, fz, ft;
        cell_axis(p.x, res, cx, fx);
        cell_axis(p.y, res, cy, fy);
        cell_axis(p.z, res, cz, fz);
        cell_axis(p.w, res_t, ct, ft);
        const uint32_t ux = (uint32_t)(cx + bx), uy = (uint32_t)(cy + by);
        uint32_t txy, tz0, tz1, tt0, tt1;
        if (dense) {
            txy = ux + uy * r;
            tz0 = (uint32_t)cz * r2;
            tz1 = tz0 + r2;
            tt0 = (uint32_t)ct * r3;
            tt1 = tt0 + r3;
        } else {
            txy = (ux * kP1) ^ (uy * kP2);
            tz0 = (uint32_t)cz * kP3;
            tz1 = (uint32_t)(cz + 1) * kP3;
            tt0 = (uint32_t)ct * kP4;
            tt1 = (uint32_t)(ct + 1) * kP4;
        }
        const float wxy = (bx ? fx : 1.0f - fx) * (by ? fy : 1.0f - fy);
        const float wz[2] = {1.0f - fz, fz}, wt[2] = {1.0f - ft, ft};
        const uint32_t tz[2] = {tz0, tz1}, tt[2] = {tt0, tt1};
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int bz = c & 1, bt = c >> 1;
            const uint32_t idx = (dense ? (txy + tz[bz] + tt[bt]) : (txy ^ tz[bz] ^ tt[bt])) & h.mask;
            const float w = (wxy * wz[bz]) * wt[bt];
            // A corner of exactly zero weight adds exactly zero (finite table
            // entries): it is not fetched.  This happens whenever a coordinate
            // sits on a grid vertex, e.g. frames whose time is a temporal vertex.
            if (w != 0.0f) {
                const uint32_t raw = tab[idx];
                a0 += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw & 0xffffu));
                a1 += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw >> 16));
            }
        }
        a0 += __shfl_xor(a0, 1, 4);
        a1 += __shfl_xor(a1, 1, 4);
        a0 += __shfl_xor(a0, 2, 4);
        a1 += __shfl_xor(a1, 2, 4);
        if (s == 0) {
            const uint16_t h0 = __builtin_bit_cast(uint16_t, (_Float16)a0);
            const uint16_t h1 = __builtin_bit_cast(uint16_t, (_Float16)a1);
            zl[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        }
    }
}

// The same gather for a launch with nothing beside it: all 16 corner loads of
// a thread's four passes are issued before any is used (46 VGPRs), which a
// lone launch needs to cover the L2 latency; beside the MLP the kernel above
// leaves that MLP more room.  The loads are range-checked buffer loads over
// the level's table: a skipped corner or a lane past the last Gaussian reads
// past the end (zero, no memory request) instead of branching.
__global__ void __launch_bounds__(256) gather_f16_batched_kernel(const float4* xt, int64_t n, int nchunk,
                                                                 HashLevels h, const uint32_t* tables,
                                                                 uint32_t* zbuf, int64_t zstride) {
#pragma clang fp contract(fast)
    const int level = blockIdx.x / nchunk;
    const int64_t first = (int64_t)(blockIdx.x % nchunk) * kGatherPerBlock;
    const int res = h.res_s[level], res_t = h.res_t[level];
    const bool dense = h.dense[level] != 0;
    const uint32_t* tab = tables + (size_t)level * h.T;
    uint32_t* zl = zbuf + (size_t)level * zstride;
    const int s = threadIdx.x & 3;
    const int bx = s & 1, by = s >> 1;
    const int sub = threadIdx.x >> 2;
    const uint32_t r = (uint32_t)res, r2 = r * r, r3 = r2 * r;
    constexpr int kPasses = kGatherPerBlock / 64;
    const __amdgpu_buffer_rsrc_t rt =
        __builtin_amdgcn_make_buffer_rsrc((void*)tab, (short)0, (int)(h.T * 4u), kBufferWord3);
    float4 P[kPasses];
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
        const int64_t i = first + j * 64 + sub;
        P[j] = xt[i < n ? i : n - 1];
    }
    uint32_t raw[kPasses][4];
    float wc[kPasses][4];
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
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
        for (int c = 0; c < 4; ++c) {
            const int bz = c & 1, bt = c >> 1;
            const uint32_t idx = (dense ? (txy + tz[bz] + tt[bt]) : (txy ^ tz[bz] ^ tt[bt])) & h.mask;
            wc[j][c] = (wxy * wz[bz]) * wt[bt];
            // a corner of zero weight adds exactly zero: not fetched (zero bits stand in)
            const uint32_t off = (valid && wc[j][c] != 0.0f) ? idx * 4u : kBufferNone;
            raw[j][c] = __builtin_amdgcn_raw_buffer_load_b32(rt, off, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            a0 += wc[j][c] * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j][c] & 0xffffu));
            a1 += wc[j][c] * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j][c] >> 16));
        }
        // the same sums over the four lanes as the kernel above: xor 1, then xor 2
        a0 += __shfl_xor(a0, 1, 4);
        a1 += __shfl_xor(a1, 1, 4);
        a0 += __shfl_xor(a0, 2, 4);
        a1 += __shfl_xor(a1, 2, 4);
        const int64_t i = first + j * 64 + sub;
        if (s == 0 && i < n) {
            const uint16_t h0 = __builtin_bit_cast(uint16_t, (_Float16)a0);
            const uint16_t h1 = __builtin_bit_cast(uint16_t, (_Float16)a1);
            zl[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        }
    }
}

// Bias + activation of one 16x16 D tile (rows 16 rb + 4 q + e), rounded to fp16.
template <bool GELU>
__device__ __forceinline__ half4_t act_tile(floatx4 acc, const float* bias) {
    half4_t h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (_Float16)hidden_act<GELU>(acc[e] + bias[e]);
    return h;
}

// Head block of the SH colour decoder for one 16-Gaussian column group, and
// Eq. 11: rows 0-2 scale, 3-6 rotation (normalised), 7-54 the 48 SH
// coefficients (no activation), 55 opacity (sigmoid); rows 56-63 are zero.
// Lane (q, c) holds rows 16 hb + 4 q + e of Gaussian gl.
__device__ __forceinline__ void sh_head_out(const DecodeArgs& a, const half8_t (&A3)[4][2], const float (&B3)[4][4],
                                            half8_t h0, half8_t h1, int64_t gl, int64_t n, int64_t out_off, int q) {
    float o[4][4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
        floatx4 acc = {0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3[hb][0], h0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3[hb][1], h1, acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[hb][e] = acc[e] + B3[hb][e];
    }
    // rotation rows 3 (q = 0) and 4-6 (q = 1) of the first tile
    const float part = q == 0 ? o[0][3] * o[0][3] : (q == 1 ? o[0][0] * o[0][0] + o[0][1] * o[0][1] + o[0][2] * o[0][2] : 0.0f);
    const float other = __shfl_xor(part, 16);
    const float nrm = fmaxf(sqrtf(part + other), 1e-12f);
    if (gl >= n) return;
    const int64_t gi = out_off + gl;
    float* sh = a.sh + gi * 48;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * hb + 4 * q + e;
            const float v = o[hb][e];
            if (row < 3)
                a.scales[gi * 3 + row] = expf(fminf(v, 20.0f));
            else if (row < 7)
                a.quats[gi * 4 + (row - 3)] = v / nrm;
            else if (row < 55)
                sh[row - 7] = v;
            else if (row == 55)
                a.opacity[gi] = sigmoidf_(v);
        }
}

// The decoder on v_mfma_f32_16x16x32_f16: a 32-wide k-block's slots (q, e)
// map to inputs 32 m + 4 q + e and 32 m + 16 + 4 q + (e - 4), so the rows a
// lane holds in two consecutive 16-row D tiles are exactly its B slots for
// the next layer, and the features of levels {2q, 2q+1, 8+2q, 9+2q} the lane
// loads are exactly its B slots of layer 1.  SH: the head block has 56 rows
// (four 16-row tiles) with the 48 SH coefficients in place of the RGB rows.
template <bool SH, bool GELU>
__global__ void __launch_bounds__(256, SH ? 1 : 2) mlp_f16_kernel(DecodeArgs a, const uint32_t* zbuf,
                                                                  int64_t zstride, int64_t n, int64_t out_off) {
    constexpr int NH = SH ? 4 : 1, kHeadRows = SH ? 56 : 11;
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, c = lane & 15;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const _Float16* W1 = (const _Float16*)a.W[0];  // [64][32]
    const _Float16* W2 = (const _Float16*)a.W[1];  // [64][64]
    const _Float16* Wh = (const _Float16*)a.W[2];  // [kHeadRows][64]

    half8_t A1[4], A2[4][2], A3[NH][2];
    float B1[4][4], B2[4][4], B3[NH][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        A1[rb] = a_tile32(W1, 32, 64, rb, 0, q, c);
#pragma unroll
        for (int m = 0; m < 2; ++m) A2[rb][m] = a_tile32(W2, 64, 64, rb, m, q, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            B1[rb][e] = a.b[0][16 * rb + 4 * q + e];
            B2[rb][e] = a.b[1][16 * rb + 4 * q + e];
        }
    }
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
#pragma unroll
        for (int m = 0; m < 2; ++m) A3[hb][m] = a_tile32(Wh, 64, kHeadRows, hb, m, q, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * hb + 4 * q + e;
            B3[hb][e] = row < kHeadRows ? a.b[2][row] : 0.0f;
        }
    }

    // features of the next 64 Gaussians are loaded while this tile computes
    auto load_z = [&](int64_t b0, half8_t (&Zo)[4]) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            int64_t gi = b0 + 16 * g + c;
            if (gi >= n) gi = n - 1;
            const int l = 2 * q;
            Zo[g] = cat8(unpack2(zbuf[(size_t)l * zstride + gi], zbuf[(size_t)(l + 1) * zstride + gi]),
                         unpack2(zbuf[(size_t)(l + 8) * zstride + gi], zbuf[(size_t)(l + 9) * zstride + gi]));
        }
    };
    half8_t Zn[4];
    if (wave * 64 < n) load_z(wave * 64, Zn);
    for (int64_t base = wave * 64; base < n; base += nwaves * 64) {
        half8_t Z[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) Z[g] = Zn[g];
        if (base + nwaves * 64 < n) load_z(base + nwaves * 64, Zn);
        // ---- trunk layer 1: 32 -> 64
        half8_t H1[2][4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                floatx4 z0 = {0, 0, 0, 0};
                const floatx4 lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[2 * m], Z[g], z0, 0, 0, 0);
                const floatx4 hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[2 * m + 1], Z[g], z0, 0, 0, 0);
                H1[m][g] = cat8(act_tile<GELU>(lo, B1[2 * m]), act_tile<GELU>(hi, B1[2 * m + 1]));
            }
        // ---- trunk layer 2: 64 -> 64
        half8_t H2[2][4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                floatx4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2[2 * m][k], H1[k][g], lo, 0, 0, 0);
                    hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2[2 * m + 1][k], H1[k][g], hi, 0, 0, 0);
                }
                H2[m][g] = cat8(act_tile<GELU>(lo, B2[2 * m]), act_tile<GELU>(hi, B2[2 * m + 1]));
            }
        // ---- head block 64 -> 11 (rows 11..15 are zero) and Eq. 11
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if constexpr (SH) {
                sh_head_out(a, A3, B3, H2[0][g], H2[1][g], base + 16 * g + c, n, out_off, q);
                continue;
            }
            floatx4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int k = 0; k < 2; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3[0][k], H2[k][g], acc, 0, 0, 0);
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = acc[e] + B3[0][e];
            // lane q = 0: s0 s1 s2 rw | q = 1: rx ry rz c0 | q = 2: c1 c2 op - | q = 3: -
            float part = q == 0 ? o[3] * o[3] : (q == 1 ? o[0] * o[0] + o[1] * o[1] + o[2] * o[2] : 0.0f);
            float other = __shfl_xor(part, 16);
            float nrm = fmaxf(sqrtf(part + other), 1e-12f);
            const int64_t gl = base + 16 * g + c;
            if (gl < n) {
                const int64_t gi = out_off + gl;
                if (q == 0) {
                    a.scales[gi * 3 + 0] = expf(fminf(o[0], 20.0f));
                    a.scales[gi * 3 + 1] = expf(fminf(o[1], 20.0f));
                    a.scales[gi * 3 + 2] = expf(fminf(o[2], 20.0f));
                    a.quats[gi * 4 + 0] = o[3] / nrm;
                } else if (q == 1) {
                    a.quats[gi * 4 + 1] = o[0] / nrm;
                    a.quats[gi * 4 + 2] = o[1] / nrm;
                    a.quats[gi * 4 + 3] = o[2] / nrm;
                    a.colors[gi * 3 + 0] = sigmoidf_(o[3]);
                } else if (q == 2) {
                    a.colors[gi * 3 + 1] = sigmoidf_(o[0]);
                    a.colors[gi * 3 + 2] = sigmoidf_(o[1]);
                    a.opacity[gi] = sigmoidf_(o[2]);
                }
            }
        }
    }
}

// Compute units of the current device (cached per device; 256 if the
// runtime cannot tell).
int device_cus() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] > 0) return cached[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
    cached[dev] = cus;
    return cus;
}

int grid_for(int64_t items_per_block, int64_t N, int cap_blocks) {
    int64_t b = (N + items_per_block - 1) / items_per_block;
    if (b < 1) b = 1;
    if (b > cap_blocks) b = cap_blocks;
    return (int)b;
}

}  // namespace

hipError_t launch_decode_features(const DecodeArgs& a, int64_t off, int64_t n, float4* xt, uint32_t* z,
                                  int64_t zstride, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int nchunk = (int)((n + kGatherPerBlock - 1) / kGatherPerBlock);
    IA_LAUNCH("normalize_kernel", normalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a,
              a.pos + off * a.stride, n, xt);
    if (!z) return hipGetLastError();  // features kept by the forward: normalisation only
    IA_LAUNCH("gather_f16_kernel", gather_f16_batched_kernel, dim3((unsigned)(a.h.L * nchunk)), dim3(256), 0, s, xt, n,
              nchunk, a.h, (const uint32_t*)a.tables, z, zstride);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s) {
    if (a.N <= 0) return hipSuccess;
    if (dtype == IA_DTYPE_F16) {
        if (!a.zbuf || a.zcap <= 0) return hipErrorInvalidValue;
        // Chunks of at most zcap Gaussians.  With a side stream, the MLP of
        // chunk k and the normalisation of chunk k + 1 run there while chunk
        // k is gathered on s, so s gathers back to back:
        //   s:    N0 G0 | G1 | G2 ...         (G k+1 waits for N k+1)
        //   side:    N1 | M0 N2 | M1 N3 ...   (M k waits for G k)
        // The feature scratch and the normalised positions are
        // double-buffered; N k+2 follows M k on the side stream, which
        // follows G k, the last reader of position slot k & 1.
        const size_t zslot = (size_t)a.h.L * a.zcap * (a.h.F / 2);  // 32-bit words per scratch slot
        float4* xtb[2] = {reinterpret_cast<float4*>(a.zbuf + 2 * zslot),
                          reinterpret_cast<float4*>(a.zbuf + 2 * zslot) + a.zcap};
        // features go to the caller's buffer ([L][N], kept for a backward) or to the
        // double-buffered scratch ([L][zcap] per slot)
        const int64_t zstride = a.features ? a.N : a.zcap;
        const bool overlap = a.side != nullptr && a.N > a.zcap;
        auto mlp = [&](hipStream_t st, const uint32_t* zb, int64_t n, int64_t off, bool beside) -> hipError_t {
            if (a.branches) return launch_mlp_branch(a, zb, zstride, n, off, st);
            // 256 threads = 4 waves x 64 Gaussians.  Beside a gather, one block
            // per kMlpCusPerBlock CUs: the MLP still finishes within the gather
            // and takes fewer wave slots from it; the last chunk's MLP, which
            // runs alone, takes the whole chip.
            const int grid = grid_for(256, n, beside ? device_cus() / kMlpCusPerBlock : 256 * 8);
            const bool gelu = a.act == IA_ACT_GELU;
            auto k = a.sh_head ? (gelu ? mlp_f16_kernel<true, true> : mlp_f16_kernel<true, false>)
                               : (gelu ? mlp_f16_kernel<false, true> : mlp_f16_kernel<false, false>);
            IA_LAUNCH("mlp_f16_kernel", k, dim3(grid), dim3(256), 0, st, a, zb, zstride, n, off);
            return hipGetLastError();
        };
        // Chunk length at offset off: zcap, except that with the side stream
        // the last two chunks split what is left about 2 : 1, so that the
        // MLP of the second-last chunk hides under the last gather and the
        // MLP left exposed at the end is short.  Every chunk but the last is
        // a multiple of 256 Gaussians: the MFMA rounding of a Gaussian's
        // decode depends on the column it occupies (its index mod 64 in the
        // chunk), so aligned chunks make the result independent of chunking.
        auto chunk_len = [&](int64_t off) -> int64_t {
            const int64_t left = a.N - off;
            if (left <= a.zcap) return left;
            if (overlap && left < 2 * a.zcap) {
                const int64_t two_thirds = ((2 * left + 2) / 3 + 255) & ~(int64_t)255;
                return two_thirds < a.zcap ? two_thirds : a.zcap;
            }
            return a.zcap;
        };
        auto normalize = [&](hipStream_t st, int64_t off, float4* xt) -> hipError_t {
            const int64_t n = chunk_len(off);
            // beside a gather (side stream) a few blocks per CU are enough
            const int grid = grid_for(256, n, st == s ? 1 << 30 : kNormBlocksPerCu * device_cus());
            IA_LAUNCH("normalize_kernel", normalize_kernel, dim3(grid), dim3(256), 0, st, a, a.pos + off * a.stride, n,
                      xt);
            return hipGetLastError();
        };
        hipError_t e = normalize(s, 0, xtb[0]);
        if (e != hipSuccess) return e;
        if (overlap) {
            // the side stream starts after everything already queued on s
            // (the caller's writes of the positions, earlier readers of the scratch)
            if ((e = hipEventRecord(a.ev_norm[0], s)) != hipSuccess) return e;
            if ((e = hipStreamWaitEvent(a.side, a.ev_norm[0], 0)) != hipSuccess) return e;
        }
        int k = 0;
        for (int64_t off = 0, n = 0; off < a.N; off += n, ++k) {
            n = chunk_len(off);
            const int nchunk = (int)((n + kGatherPerBlock - 1) / kGatherPerBlock);
            uint32_t* zb = a.features ? a.features + (size_t)off * (a.h.F / 2) : a.zbuf + (size_t)(k & 1) * zslot;
            float4* xt = xtb[overlap ? (k & 1) : 0];
            if (overlap && k >= 1 && (e = hipStreamWaitEvent(s, a.ev_norm[k & 1], 0)) != hipSuccess) return e;
            if (overlap && k >= 2 && (e = hipStreamWaitEvent(s, a.ev_mlp[k & 1], 0)) != hipSuccess) return e;
            if (!overlap && k >= 1 && (e = normalize(s, off, xt)) != hipSuccess) return e;
            if (a.h.F == 4) {
                if ((e = launch_gather_f4(xt, n, a.h, a.tables, zb, zstride, s)) != hipSuccess) return e;
            } else {
                // beside an MLP (every chunk but the first of an overlapped decode)
                // the lean gather, alone the batched one
                if (overlap && k >= 1)
                    IA_LAUNCH("gather_f16_kernel", gather_f16_kernel, dim3((unsigned)(a.h.L * nchunk)), dim3(256), 0,
                              s, xt, n, nchunk, a.h, (const uint32_t*)a.tables, zb, zstride);
                else
                    IA_LAUNCH("gather_f16_kernel", gather_f16_batched_kernel, dim3((unsigned)(a.h.L * nchunk)),
                              dim3(256), 0, s, xt, n, nchunk, a.h, (const uint32_t*)a.tables, zb, zstride);
            }
            if (overlap) {
                if ((e = hipEventRecord(a.ev_gather[k & 1], s)) != hipSuccess) return e;
                const int64_t noff = off + n;
                if (noff < a.N) {
                    if ((e = normalize(a.side, noff, xtb[(k + 1) & 1])) != hipSuccess) return e;
                    if ((e = hipEventRecord(a.ev_norm[(k + 1) & 1], a.side)) != hipSuccess) return e;
                }
                if ((e = hipStreamWaitEvent(a.side, a.ev_gather[k & 1], 0)) != hipSuccess) return e;
                if ((e = mlp(a.side, zb, n, off, noff < a.N)) != hipSuccess) return e;
                if ((e = hipEventRecord(a.ev_mlp[k & 1], a.side)) != hipSuccess) return e;
            } else {
                if ((e = mlp(s, zb, n, off, false)) != hipSuccess) return e;
            }
        }
        if (overlap) {
            // the caller's stream resumes after the last MLPs (the side stream
            // is in order, so the last event covers every earlier chunk)
            e = hipStreamWaitEvent(s, a.ev_mlp[(k - 1) & 1], 0);
            if (e != hipSuccess) return e;
        }
        return hipGetLastError();
    }
    int grid = grid_for(256, a.N, 1 << 30);
    const int LF = a.in_dim, H1 = a.hidden[0], H2 = a.n_hidden > 1 ? a.hidden[1] : 0;
    if (LF == 8 && H1 == 32 && H2 == 0)
        IA_LAUNCH("decode_f32_kernel", (decode_f32_kernel<8, 32, 0>), dim3(grid), dim3(256), 0, s, a);
    else if (LF == 32 && H1 == 64 && H2 == 64)
        IA_LAUNCH("decode_f32_kernel", (decode_f32_kernel<32, 64, 64>), dim3(grid), dim3(256), 0, s, a);
    else if (LF == 32 && H1 == 64 && H2 == 0)
        IA_LAUNCH("decode_f32_kernel", (decode_f32_kernel<32, 64, 0>), dim3(grid), dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ia
