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
// gather_f16_kernel: level-major.  Block b handles level group b / nchunk and
// Gaussians [256 (b % nchunk), +256), one lane per Gaussian.  Blocks are
// dispatched in index order and spread round-robin over the XCDs, so at any
// moment all XCDs work on the same level and that level's 2^log2T x 4-byte
// table stays resident in every XCD's L2 instead of being fetched line by
// line from HBM / Infinity Cache.  The eight coarsest levels go four to a
// block: their Gaussians touch few table lines (the four levels' working
// sets share L2), and one load of the normalised position (a 16-byte read,
// mostly from the Infinity Cache) then serves four levels instead of one.
// A lane computes its Gaussian's cell once and issues all its corner loads
// before using any (range-checked buffer loads; the corners of a temporal
// vertex no lane of the wave weights are not loaded).  Consecutive
// lanes hold consecutive Gaussians, so when the positions of a frame are
// stored in spatial order the lanes of a wave share the coarse levels' cache
// lines.  Output z[level][i] = two fp16 features packed in 32 bits (RNE).
//
// mlp_f16_kernel: the 32 -> 64 -> 64 -> 11 (or 56, SH colour) decoder on
// v_mfma_f32_16x16x32_f16.
// Register layout (wave64, lane l, q = l/16, c = l%16): A supplies row c and
// B column c, each with eight k-slots per lane that A and B share; D holds
// rows 4q..4q+3 of column c.  Gaussians are the columns and neurons the rows.

constexpr int kGatherPerBlock = 256;  // Gaussians per gather block, one lane each
// Levels [0, kGroupedLevels) go kLevelGroup to a block (one position load for
// all of them); the finer levels one to a block.
constexpr int kGroupedLevels = 8;
constexpr int kLevelGroup = 4;

// Gather blocks per chunk of kGatherPerBlock Gaussians for L levels.
int gather_groups(int L) {
    const int gl = L < kGroupedLevels ? L : kGroupedLevels;
    return (gl + kLevelGroup - 1) / kLevelGroup + (L - gl);
}
constexpr int kMlpBlocksPerCu = 1;    // MLP beside a gather: blocks per CU
constexpr int kMlpAhead = 4;          // MLP: 16-Gaussian groups whose features load ahead
constexpr int kNormBlocksPerCu = 2;   // normalisation beside a gather: blocks per CU

__global__ void __launch_bounds__(256) normalize_kernel(DecodeArgs a, const float* pos, int64_t n, float4* xt) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const float* p = pos + i * a.stride;
        float v[4];
        normalize_pos(p[0], p[1], p[2], a.stride == 4 ? p[3] : a.t_scalar, a.h.t_min, a.h.t_max, v);
        xt[i] = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// One lane's gather of one level (see gather_f16_kernel).  DENSE: corner
// index = sum of the per-axis terms (row-major, x fastest); else their XOR
// (the hash), modulo T.
template <bool DENSE>
__device__ __forceinline__ void gather_lane(const float4 p, bool valid, int res, int res_t, uint32_t mask,
                                            const __amdgpu_buffer_rsrc_t rt, float& a0, float& a1) {
#pragma clang fp contract(fast)
    int cx, cy, cz, ct;
    float fx, fy, fz, ft;
    cell_axis(p.x, res, cx, fx);
    cell_axis(p.y, res, cy, fy);
    cell_axis(p.z, res, cz, fz);
    cell_axis(p.w, res_t, ct, ft);
    // per-axis index terms in bytes (4 per entry): the factor distributes over
    // the sum and, before the mask, over the XOR of the hash
    uint32_t tx[2], ty[2], tz[2], tt[2];
    if (DENSE) {
        const uint32_t r = (uint32_t)res, r2 = r * r, r3 = r2 * r;
        tx[0] = (uint32_t)cx * 4u;
        tx[1] = tx[0] + 4u;
        ty[0] = (uint32_t)cy * (r * 4u);
        ty[1] = ty[0] + r * 4u;
        tz[0] = (uint32_t)cz * (r2 * 4u);
        tz[1] = tz[0] + r2 * 4u;
        tt[0] = (uint32_t)ct * (r3 * 4u);
        tt[1] = tt[0] + r3 * 4u;
    } else {
        tx[0] = (uint32_t)cx * (kP1 * 4u);
        tx[1] = (uint32_t)(cx + 1) * (kP1 * 4u);
        ty[0] = (uint32_t)cy * (kP2 * 4u);
        ty[1] = (uint32_t)(cy + 1) * (kP2 * 4u);
        tz[0] = (uint32_t)cz * (kP3 * 4u);
        tz[1] = (uint32_t)(cz + 1) * (kP3 * 4u);
        tt[0] = (uint32_t)ct * (kP4 * 4u);
        tt[1] = (uint32_t)(ct + 1) * (kP4 * 4u);
    }
    const uint32_t mask4 = mask * 4u;
    auto comb = [](uint32_t u, uint32_t v) { return DENSE ? u + v : u ^ v; };
    const float wx[2] = {1.0f - fx, fx}, wy[2] = {1.0f - fy, fy}, wz[2] = {1.0f - fz, fz}, wt[2] = {1.0f - ft, ft};
    float wxyz[8];
    uint32_t txyz[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int bx = c & 1, by = (c >> 1) & 1, bz = (c >> 2) & 1;
        wxyz[c] = (wx[bx] * wy[by]) * wz[bz];
        txyz[c] = comb(comb(tx[bx], ty[by]), tz[bz]);
    }
    // The corners of one temporal vertex are fetched only when some lane of
    // the wave gives them a non-zero weight (a frame's Gaussians share one
    // time, and on a temporal vertex half the corners weigh exactly zero).
    // A lane past the last Gaussian gathers the last one's corners, unused.
    const bool need_t[2] = {__ballot(valid && wt[0] != 0.0f) != 0ull, __ballot(valid && wt[1] != 0.0f) != 0ull};
    uint32_t raw[16];
    float w[16];
#pragma unroll
    for (int bt = 0; bt < 2; ++bt) {
        if (need_t[bt]) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                w[8 * bt + c] = wxyz[c] * wt[bt];
                raw[8 * bt + c] = __builtin_amdgcn_raw_buffer_load_b32(rt, comb(txyz[c], tt[bt]) & mask4, 0, 0);
            }
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                w[8 * bt + c] = 0.0f;
                raw[8 * bt + c] = 0u;
            }
        }
    }
    // sum over the 16 corners in corner order of w_c * table entry
    a0 = 0.0f;
    a1 = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        a0 += w[c] * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[c] & 0xffffu));
        a1 += w[c] * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[c] >> 16));
    }
}

// One lane's gather of one level, stored as two packed fp16 features.
__device__ __forceinline__ void gather_store(const float4 p, bool valid, int64_t i, int level, const HashLevels& h,
                                             const uint32_t* tables, uint32_t* zbuf, int64_t zstride) {
    const __amdgpu_buffer_rsrc_t rt =
        __builtin_amdgcn_make_buffer_rsrc((void*)(tables + (size_t)level * h.T), (short)0, (int)(h.T * 4u),
                                          kBufferWord3);
    float a0, a1;
    if (h.dense[level])
        gather_lane<true>(p, valid, h.res_s[level], h.res_t[level], h.mask, rt, a0, a1);
    else
        gather_lane<false>(p, valid, h.res_s[level], h.res_t[level], h.mask, rt, a0, a1);
    if (valid) {
        const uint16_t h0 = __builtin_bit_cast(uint16_t, (_Float16)a0);
        const uint16_t h1 = __builtin_bit_cast(uint16_t, (_Float16)a1);
        zbuf[(size_t)level * zstride + i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    }
}

// A full group of coarse levels L0 .. L0 + kLevelGroup - 1, compiled with its
// level indices: all of its loads can be in flight together.
template <int L0>
__device__ __forceinline__ void gather_group(const float4 p, bool valid, int64_t i, const HashLevels& h,
                                             const uint32_t* tables, uint32_t* zbuf, int64_t zstride) {
#pragma unroll
    for (int k = 0; k < kLevelGroup; ++k) gather_store(p, valid, i, L0 + k, h, tables, zbuf, zstride);
}
static_assert(kGroupedLevels == 2 * kLevelGroup, "two groups of coarse levels");

__global__ void __launch_bounds__(kGatherPerBlock) gather_f16_kernel(const float4* xt, int64_t n, int nchunk,
                                                                     HashLevels h, const uint32_t* tables,
                                                                     uint32_t* zbuf, int64_t zstride) {
    const int gl = h.L < kGroupedLevels ? h.L : kGroupedLevels;
    const int ng = (gl + kLevelGroup - 1) / kLevelGroup;
    const int grp = blockIdx.x / nchunk;
    const int64_t i = (int64_t)(blockIdx.x % nchunk) * kGatherPerBlock + threadIdx.x;
    const bool valid = i < n;
    const float4 p = xt[valid ? i : n - 1];
    if (grp < ng) {
        // kLevelGroup coarse levels from one position load
        if (gl == kGroupedLevels) {
            if (grp == 0)
                gather_group<0>(p, valid, i, h, tables, zbuf, zstride);
            else
                gather_group<kLevelGroup>(p, valid, i, h, tables, zbuf, zstride);
        } else {  // fewer levels than two full groups
            const int l1 = grp * kLevelGroup + kLevelGroup < gl ? grp * kLevelGroup + kLevelGroup : gl;
            for (int l = grp * kLevelGroup; l < l1; ++l) gather_store(p, valid, i, l, h, tables, zbuf, zstride);
        }
    } else {
        gather_store(p, valid, i, grp - ng + gl, h, tables, zbuf, zstride);
    }
}

// Activation of one 16x16 D tile (rows 16 rb + 4 q + e; the MFMA started
// from the bias, so acc = W x + b), rounded to fp16.
template <bool GELU>
__device__ __forceinline__ half4_t act_tile(floatx4 acc) {
    half4_t h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (_Float16)hidden_act<GELU>(acc[e]);
    return h;
}

// Eq. 11 activations of the fp16 path from the hardware's one-ulp exp2, rcp
// and rsq (the full-precision expf and the IEEE division take several times
// the instructions, and every lane of a wave runs each lane's branch):
//   scale     exp(min(x, 20)) = 2^(min(x, 20) log2 e)
//   colour    1 / (1 + 2^(-x log2 e))      (0 and 1 at the extremes)
//   rotation  r / max(|r|, 1e-12) = r min(rsq(|r|^2), 1e12)
// The clamps are v_med3_f32 (fminf adds a NaN-quieting instruction).
__device__ __forceinline__ float exp_clip20(float x) {
    return __builtin_amdgcn_exp2f(__builtin_amdgcn_fmed3f(x, -3.402823466e+38f, 20.0f) * 1.44269504088896341f);
}
__device__ __forceinline__ float sigmoid_fast(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}
__device__ __forceinline__ float inv_norm(float sq) {
    return __builtin_amdgcn_fmed3f(__builtin_amdgcn_rsqf(sq), 0.0f, 1e12f);
}

// Head block of the SH colour decoder for one 16-Gaussian column group, and
// Eq. 11: rows 0-2 scale, 3-6 rotation (normalised), 7-54 the 48 SH
// coefficients (no activation), 55 opacity (sigmoid); rows 56-63 are zero.
// Lane (q, c) holds rows 16 hb + 4 q + e of Gaussian gl.
__device__ __forceinline__ void sh_head_out(const DecodeArgs& a, const half8_t (*sA3)[64], const floatx4 (*sB3)[64],
                                            half8_t h0, half8_t h1, int64_t gl, int64_t n, int64_t out_off, int lane,
                                            int q) {
    float o[4][4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
        floatx4 acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sA3[2 * hb][lane], h0, sB3[hb][lane], 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sA3[2 * hb + 1][lane], h1, acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[hb][e] = acc[e];
    }
    // rotation rows 3 (q = 0) and 4-6 (q = 1) of the first tile
    const float part = q == 0 ? o[0][3] * o[0][3] : (q == 1 ? o[0][0] * o[0][0] + o[0][1] * o[0][1] + o[0][2] * o[0][2] : 0.0f);
    const float other = __shfl_xor(part, 16);
    const float inv = inv_norm(part + other);
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
                a.scales[gi * 3 + row] = exp_clip20(v);
            else if (row < 7)
                a.quats[gi * 4 + (row - 3)] = v * inv;
            else if (row < 55)
                sh[row - 7] = v;
            else if (row == 55)
                a.opacity[gi] = sigmoid_fast(v);
        }
}

// The decoder on v_mfma_f32_16x16x32_f16: a 32-wide k-block's slots (q, e)
// map to inputs 32 m + 4 q + e and 32 m + 16 + 4 q + (e - 4), so the rows a
// lane holds in two consecutive 16-row D tiles are exactly its B slots for
// the next layer, and the features of levels {2q, 2q+1, 8+2q, 9+2q} the lane
// loads are exactly its B slots of layer 1.  SH: the head block has 56 rows
// (four 16-row tiles) with the 48 SH coefficients in place of the RGB rows.
// Each lane's A operands (the weights) and initial accumulators (the biases)
// are staged once per block in LDS, indexed by lane, and every 16-Gaussian
// column group goes through all layers before the next, so a wave holds few
// registers and more waves (of this kernel, or of the gather beside it) fit.
template <bool SH, bool GELU>
__global__ void __launch_bounds__(256) mlp_f16_kernel(DecodeArgs a, const uint32_t* zbuf, int64_t zstride, int64_t n,
                                                      int64_t out_off) {
    constexpr int NH = SH ? 4 : 1, kHeadRows = SH ? 56 : 11;
    // A tiles: layer 1 [rb] (4), layer 2 [rb][m] (8), head [hb][m] (2 NH);
    // bias tiles: layer 1 [rb], layer 2 [rb], head [hb]
    constexpr int kA2 = 4, kA3 = 12, kTilesA = 12 + 2 * NH;
    constexpr int kB2 = 4, kB3 = 8, kTilesB = 8 + NH;
    __shared__ half8_t sA[kTilesA][64];
    __shared__ floatx4 sB[kTilesB][64];
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, c = lane & 15;
    {
        const _Float16* W1 = (const _Float16*)a.W[0];  // [64][32]
        const _Float16* W2 = (const _Float16*)a.W[1];  // [64][64]
        const _Float16* Wh = (const _Float16*)a.W[2];  // [kHeadRows][64]
        for (int j = threadIdx.x >> 6; j < kTilesA; j += 4) {
            if (j < kA2)
                sA[j][lane] = a_tile32(W1, 32, 64, j, 0, q, c);
            else if (j < kA3)
                sA[j][lane] = a_tile32(W2, 64, 64, (j - kA2) >> 1, (j - kA2) & 1, q, c);
            else
                sA[j][lane] = a_tile32(Wh, 64, kHeadRows, (j - kA3) >> 1, (j - kA3) & 1, q, c);
        }
        for (int j = threadIdx.x >> 6; j < kTilesB; j += 4) {
            floatx4 b;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (j < kB2)
                    b[e] = a.b[0][16 * j + 4 * q + e];
                else if (j < kB3)
                    b[e] = a.b[1][16 * (j - kB2) + 4 * q + e];
                else {
                    const int row = 16 * (j - kB3) + 4 * q + e;
                    b[e] = row < kHeadRows ? a.b[2][row] : 0.0f;
                }
            }
            sB[j][lane] = b;
        }
    }
    __syncthreads();
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;

    // the features of one 16-Gaussian group (rows of the columns' B operand)
    auto load_z = [&](int64_t g0) {
        int64_t gi = g0 + c;
        if (gi >= n) gi = n - 1;
        const int l = 2 * q;
        return cat8(unpack2(zbuf[(size_t)l * zstride + gi], zbuf[(size_t)(l + 1) * zstride + gi]),
                    unpack2(zbuf[(size_t)(l + 8) * zstride + gi], zbuf[(size_t)(l + 9) * zstride + gi]));
    };
    // groups of this wave: 64 consecutive Gaussians per turn (four groups), turns nwaves apart
    auto group_at = [&](int64_t k) { return ((k >> 2) * nwaves + wave) * 64 + 16 * (k & 3); };
    // The features of the next kMlpAhead groups are in flight while a group
    // computes (beside a gather, loads wait behind its flood of L2 requests).
    // Slot i of the ring holds group k + i of the unrolled turn, so no
    // register is moved while its load is pending.
    // (load_z clamps its index, so every load is issued unconditionally.)
    half8_t Zr[kMlpAhead];
#pragma unroll
    for (int i = 0; i < kMlpAhead; ++i) Zr[i] = load_z(group_at(i));
    for (int64_t k0 = 0; group_at(k0) < n; k0 += kMlpAhead)
#pragma unroll
    for (int i = 0; i < kMlpAhead; ++i) {
        const int64_t k = k0 + i;
        const int64_t g0 = group_at(k);
        const half8_t Z = Zr[i];
        Zr[i] = load_z(group_at(k + kMlpAhead));
        if (g0 >= n) continue;  // wave-uniform
        // ---- trunk layer 1: 32 -> 64
        half8_t H1[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const floatx4 lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(sA[2 * m][lane], Z, sB[2 * m][lane], 0, 0, 0);
            const floatx4 hi =
                __builtin_amdgcn_mfma_f32_16x16x32_f16(sA[2 * m + 1][lane], Z, sB[2 * m + 1][lane], 0, 0, 0);
            H1[m] = cat8(act_tile<GELU>(lo), act_tile<GELU>(hi));
        }
        // ---- trunk layer 2: 64 -> 64
        half8_t H2[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            floatx4 lo = sB[kB2 + 2 * m][lane], hi = sB[kB2 + 2 * m + 1][lane];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(sA[kA2 + 2 * (2 * m) + kk][lane], H1[kk], lo, 0, 0, 0);
                hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(sA[kA2 + 2 * (2 * m + 1) + kk][lane], H1[kk], hi, 0, 0, 0);
            }
            H2[m] = cat8(act_tile<GELU>(lo), act_tile<GELU>(hi));
        }
        // ---- head block and Eq. 11
        const int64_t gl = g0 + c;
        if constexpr (SH) {
            sh_head_out(a, sA + kA3, sB + kB3, H2[0], H2[1], gl, n, out_off, lane, q);
            continue;
        }
        floatx4 acc = sB[kB3][lane];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sA[kA3 + kk][lane], H2[kk], acc, 0, 0, 0);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[e];
        // lane q = 0: s0 s1 s2 rw | q = 1: rx ry rz c0 | q = 2: c1 c2 op - | q = 3: -
        float part = q == 0 ? o[3] * o[3] : (q == 1 ? o[0] * o[0] + o[1] * o[1] + o[2] * o[2] : 0.0f);
        float other = __shfl_xor(part, 16);
        const float inv = inv_norm(part + other);
        if (gl < n) {
            const int64_t gi = out_off + gl;
            if (q == 0) {
                a.scales[gi * 3 + 0] = exp_clip20(o[0]);
                a.scales[gi * 3 + 1] = exp_clip20(o[1]);
                a.scales[gi * 3 + 2] = exp_clip20(o[2]);
                a.quats[gi * 4 + 0] = o[3] * inv;
            } else if (q == 1) {
                a.quats[gi * 4 + 1] = o[0] * inv;
                a.quats[gi * 4 + 2] = o[1] * inv;
                a.quats[gi * 4 + 3] = o[2] * inv;
                a.colors[gi * 3 + 0] = sigmoid_fast(o[3]);
            } else if (q == 2) {
                a.colors[gi * 3 + 1] = sigmoid_fast(o[0]);
                a.colors[gi * 3 + 2] = sigmoid_fast(o[1]);
                a.opacity[gi] = sigmoid_fast(o[2]);
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
    if (a.h.F == 4) return launch_gather_f4(xt, n, a.h, a.tables, z, zstride, s);
    IA_LAUNCH("gather_f16_kernel", gather_f16_kernel, dim3((unsigned)(gather_groups(a.h.L) * nchunk)), dim3(kGatherPerBlock), 0, s,
              xt, n, nchunk, a.h, (const uint32_t*)a.tables, z, zstride);
    return hipGetLastError();
}

namespace {

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Events of the side-stream overlap, one set per host thread and device.
// A stream wait takes the event's latest record at the time the wait is
// enqueued, so reusing a set across the calls of one thread is safe, and
// threads never share one.  Created on a thread's first overlapped decode on
// a device (no device memory) and kept until the process ends.
struct OverlapEvents {
    hipEvent_t gather[2], mlp[2], norm[2];
};

hipError_t overlap_events(OverlapEvents** out) {
    constexpr int kMaxDevices = 64;
    thread_local OverlapEvents* per_device[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!per_device[dev]) {
        OverlapEvents ev{};
        hipEvent_t* all[6] = {&ev.gather[0], &ev.gather[1], &ev.mlp[0], &ev.mlp[1], &ev.norm[0], &ev.norm[1]};
        for (int k = 0; k < 6; ++k) {
            e = hipEventCreateWithFlags(all[k], hipEventDisableTiming);
            if (e != hipSuccess) {
                for (int j = 0; j < k; ++j) (void)hipEventDestroy(*all[j]);
                return e;
            }
        }
        per_device[dev] = new OverlapEvents(ev);
    }
    *out = per_device[dev];
    return hipSuccess;
}

}  // namespace

DecodeLayout decode_layout(const HashLevels& h, int64_t N, int64_t max_chunk) {
    DecodeLayout L{};
    const int64_t n = N > 0 ? N : 1;
    int64_t zcap = (n + 255) / 256 * 256;
    if (zcap > max_chunk) zcap = max_chunk;
    L.zcap = zcap;
    L.slots = n > zcap ? 2 : 1;
    size_t off = 0;
    for (int k = 0; k < L.slots; ++k) {
        L.z[k] = off;
        off = align256(off + (size_t)h.L * (size_t)zcap * (size_t)(h.F / 2) * 4);
    }
    for (int k = 0; k < L.slots; ++k) {
        L.xt[k] = off;
        off = align256(off + (size_t)zcap * sizeof(float4));
    }
    if (L.slots == 1) {
        L.z[1] = L.z[0];
        L.xt[1] = L.xt[0];
    }
    L.total = off;
    return L;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s) {
    if (a.N <= 0) return hipSuccess;
    if (dtype == IA_DTYPE_F16) {
        if (!a.zslot[0] || !a.xt[0] || a.zcap <= 0) return hipErrorInvalidValue;
        // Chunks of at most zcap Gaussians.  With a side stream, the MLP of
        // chunk k and the normalisation of chunk k + 1 run there while chunk
        // k is gathered on s, so s gathers back to back:
        //   s:    N0 G0 | G1 | G2 ...         (G k+1 waits for N k+1)
        //   side:    N1 | M0 N2 | M1 N3 ...   (M k waits for G k)
        // The feature scratch and the normalised positions alternate between
        // two slots; N k+2 follows M k on the side stream, which follows G k,
        // the last reader of position slot k & 1.
        // features go to the caller's buffer ([L][N], kept for a backward) or to the
        // scratch slots ([L][zcap] each)
        const int64_t zstride = a.features ? a.N : a.zcap;
        const bool overlap = a.side != nullptr && a.side != s && a.N > a.zcap && a.zslot[1] != a.zslot[0] &&
                             a.xt[1] != a.xt[0];
        OverlapEvents* ev = nullptr;
        if (overlap) {
            hipError_t e = overlap_events(&ev);
            if (e != hipSuccess) return e;
        }
        auto mlp = [&](hipStream_t st, const uint32_t* zb, int64_t n, int64_t off, bool beside) -> hipError_t {
            if (a.branches) return launch_mlp_branch(a, zb, zstride, n, off, st);
            // 256 threads = 4 waves.  Beside a gather, kMlpBlocksPerCu blocks
            // per CU: the MLP finishes within the gather and leaves it most
            // wave slots; the last chunk's MLP, which runs alone, takes the
            // whole chip.
            const int grid = grid_for(256, n, beside ? device_cus() * kMlpBlocksPerCu : 256 * 8);
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
        hipError_t e = normalize(s, 0, a.xt[0]);
        if (e != hipSuccess) return e;
        if (overlap) {
            // the side stream starts after everything already queued on s
            // (the caller's writes of the positions, earlier readers of the scratch)
            if ((e = hipEventRecord(ev->norm[0], s)) != hipSuccess) return e;
            if ((e = hipStreamWaitEvent(a.side, ev->norm[0], 0)) != hipSuccess) return e;
        }
        int k = 0;
        for (int64_t off = 0, n = 0; off < a.N; off += n, ++k) {
            n = chunk_len(off);
            const int nchunk = (int)((n + kGatherPerBlock - 1) / kGatherPerBlock);
            const int slot = overlap ? (k & 1) : 0;
            uint32_t* zb = a.features ? a.features + (size_t)off * (a.h.F / 2) : a.zslot[slot];
            float4* xt = a.xt[slot];
            if (overlap && k >= 1 && (e = hipStreamWaitEvent(s, ev->norm[k & 1], 0)) != hipSuccess) return e;
            if (overlap && k >= 2 && (e = hipStreamWaitEvent(s, ev->mlp[k & 1], 0)) != hipSuccess) return e;
            if (!overlap && k >= 1 && (e = normalize(s, off, xt)) != hipSuccess) return e;
            if (a.h.F == 4) {
                if ((e = launch_gather_f4(xt, n, a.h, a.tables, zb, zstride, s)) != hipSuccess) return e;
            } else {
                IA_LAUNCH("gather_f16_kernel", gather_f16_kernel, dim3((unsigned)(gather_groups(a.h.L) * nchunk)),
                          dim3(kGatherPerBlock), 0, s, xt, n, nchunk, a.h, (const uint32_t*)a.tables, zb, zstride);
            }
            if (overlap) {
                if ((e = hipEventRecord(ev->gather[k & 1], s)) != hipSuccess) return e;
                const int64_t noff = off + n;
                if (noff < a.N) {
                    if ((e = normalize(a.side, noff, a.xt[(k + 1) & 1])) != hipSuccess) return e;
                    if ((e = hipEventRecord(ev->norm[(k + 1) & 1], a.side)) != hipSuccess) return e;
                }
                if ((e = hipStreamWaitEvent(a.side, ev->gather[k & 1], 0)) != hipSuccess) return e;
                if ((e = mlp(a.side, zb, n, off, noff < a.N)) != hipSuccess) return e;
                if ((e = hipEventRecord(ev->mlp[k & 1], a.side)) != hipSuccess) return e;
            } else {
                if ((e = mlp(s, zb, n, off, false)) != hipSuccess) return e;
            }
        }
        if (overlap) {
            // the caller's stream resumes after the last MLPs (the side stream
            // is in order, so the last event covers every earlier chunk)
            e = hipStreamWaitEvent(s, ev->mlp[(k - 1) & 1], 0);
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
