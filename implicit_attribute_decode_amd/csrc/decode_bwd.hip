// Backward of the fp16 decode path (SPIN-4DGS §3.3 Eq. 7-11) for upstream
// gradients of the decoded attributes: gradients of the hash tables, of every
// decoder weight and bias, and of the positions.
//
// Per chunk of at most 2^21 Gaussians:
//   features   the encoding z kept by the forward decode, or recomputed by the
//              forward's normalise + level-major gather kernels (fp16, as the
//              forward fed the MLP); x~ is renormalised either way.
//   compaction the Gaussians whose upstream gradient is not all zero (the
//              others have exactly zero decoder gradients), then ordered by a
//              key of 6 bits of time over a 24-bit Morton code of the
//              normalised position (stable radix sort: index order within a
//              key), so that the Gaussians of one block lie close together
//              and share the corners of the coarser levels; the two kernels
//              below work on that list only.
//   mlp_bwd_kernel  one wave per 16 Gaussians at a time (persistent grid):
//       forward  the decoder on v_mfma_f32_16x16x32_f16 exactly as the decode
//                runs it (same operands, same fp16 roundings), keeping the
//                activation derivative at both hidden layers' pre-activations
//                (GELU' shares the erf polynomial and exponential of GELU);
//       Eq. 11   dr from the upstream gradients: exp' = s below the clip,
//                (I - q q^T) / |r| for the normalisation, sigma' = c (1 - c);
//       Eq. 10   data gradients dx = W^T (dy act'(a)) on
//                v_mfma_f32_16x16x4_f32 with the fp32 weights in LDS (the k
//                order of each product is permuted so that the gradient a lane
//                holds in the output tile is its own operand slot for the next
//                product: no shuffles), and weight gradients
//                dW += dy x^T over the Gaussians on the same instruction, after
//                a per-wave LDS transpose that puts the Gaussians on the k
//                axis.  Each wave accumulates its weight and bias gradients in
//                registers over all its Gaussians and adds them to its own
//                slot of a partial buffer;
//       dz       written to the scratch, fp32, [level][Gaussian] x 2 features.
//   scatter_kernel  level-major like the gather, four lanes per (Gaussian,
//       level), each with four of the 16 corners: dtable[corner] += w dz with
//       float atomics; for positions dz/df_axis = sum_c (+-1) prod_{other
//       axes} w table[c] (time carries no gradient), times (res - 1), then the
//       Jacobian of Eq. 7: each level's share is stored (one 16-byte store per
//       Gaussian and level, in list order) and pos_reduce_kernel adds the
//       levels in a fixed order to the position gradient (no atomics).
//       On levels of at most kAggMaxRes vertices per axis, where the block's
//       Gaussians share corners, each block first adds its contributions per
//       table entry in an LDS hash table (open addressing, LDS atomics) and
//       then issues one pair of global atomics per distinct entry: global
//       float atomics are served far below L2 speed on this chip, LDS ones
//       are not.
// After the last chunk a two-stage reduction sums the partial buffer in a
// fixed order (deterministic weight and bias gradients).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "decode_common.h"
#include "ia_internal.h"

namespace ia {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kTS = 18;  // row stride (floats) of the per-wave transpose buffers: conflict-free column reads
// per lane: 4 head tiles + 16 W2 tiles + 8 W1 tiles (4 floats each) + 36 bias partials
constexpr int kTileSlots = (4 + 16 + 8) * 4;
constexpr int kBiasSlots = 4 + 16 + 16;
static_assert(kDecodeBwdBlocks * kBwdWaves % kDecodeBwdGroups == 0, "groups must split the waves evenly");

typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma4(float a, float b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS written by the lanes of one wave is read back by other lanes of the same
// wave: order the accesses at wavefront scope.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The hidden activation of the fp16 path (GELU computed exactly as
// gelu_fp16path, so the value is bit-identical to the forward's; ReLU
// otherwise) and its derivative; GELU' = Phi(x) + x phi(x) reuses the tail
// Q = 1 - Phi(|x|) and exp(-x^2 / 2).
template <bool GELU>
__device__ __forceinline__ float act_fwd_grad(float x, float& d) {
    if constexpr (!GELU) {
        d = x > 0.0f ? 1.0f : 0.0f;
        return x > 0.0f ? x : 0.0f;
    } else {
        float e;
        const float q = gelu_tail(x, e);
        d = fmaf(x * e, 0.39894228040143268f, x >= 0.0f ? 1.0f - q : q);
        return fmaf(-fabsf(x), q, fmaxf(x, 0.0f));
    }
}

__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

struct MlpBwdArgs {
    const _Float16* W[3];  // [64][32], [64][64], [11][64]
    const float* b[3];
    int gelu;
    const uint32_t* z;  // [L][zstride] fp16 pairs
    int64_t zstride;
    const uint32_t* list;   // chunk-local indices of the Gaussians with a non-zero upstream gradient
    const uint32_t* count;  // how many (device)
    int64_t off;  // index of the chunk's first Gaussian in the upstream gradients
    const float* gs;
    const float* gq;
    const float* gc;
    const float* go;
    float2* gz;      // [L][gzstride]
    int64_t gzstride;
    float* partial;  // [waves][kTileSlots + kBiasSlots][64]
    int first;       // 1: the partial slots start from zero
};

template <bool GELU>
__global__ void __launch_bounds__(kBwdThreads, 1) mlp_bwd_kernel(MlpBwdArgs a) {
#pragma clang fp contract(fast)
    // fp32 operands of the data-gradient products, lane-ordered:
    //   sWh[rb][e][lane] = Wh[4q+e][16rb+c], sW2[ob][rb][e][lane] = W2[16rb+4q+e][16ob+c],
    //   sW1[ob][rb][e][lane] = W1[16rb+4q+e][16ob+c]
    __shared__ float sWh[4 * 4 * 64];
    __shared__ float sW2[4 * 4 * 4 * 64];
    __shared__ float sW1[2 * 4 * 4 * 64];
    __shared__ float sT[kBwdWaves][2][64 * kTS];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int q = lane >> 4, c = lane & 15;
    const _Float16* W1 = a.W[0];
    const _Float16* W2 = a.W[1];
    const _Float16* Wh = a.W[2];
    for (int k = threadIdx.x; k < 4 * 4 * 64; k += kBwdThreads) {
        const int l = k & 63, e = (k >> 6) & 3, rb = k >> 8, qq = l >> 4, cc = l & 15;
        const int row = 4 * qq + e;
        sWh[k] = row < 11 ? (float)Wh[row * 64 + 16 * rb + cc] : 0.0f;
    }
    for (int k = threadIdx.x; k < 4 * 4 * 4 * 64; k += kBwdThreads) {
        const int l = k & 63, e = (k >> 6) & 3, rb = (k >> 8) & 3, ob = k >> 10, qq = l >> 4, cc = l & 15;
        sW2[k] = (float)W2[(16 * rb + 4 * qq + e) * 64 + 16 * ob + cc];
    }
    for (int k = threadIdx.x; k < 2 * 4 * 4 * 64; k += kBwdThreads) {
        const int l = k & 63, e = (k >> 6) & 3, rb = (k >> 8) & 3, ob = k >> 10, qq = l >> 4, cc = l & 15;
        sW1[k] = (float)W1[(16 * rb + 4 * qq + e) * 32 + 16 * ob + cc];
    }
    __syncthreads();

    // forward operands, as the decode holds them
    half8_t A1[4], A2[4][2], A3[2];
    float B1[4][4], B2[4][4], B3[4];
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
    for (int m = 0; m < 2; ++m) A3[m] = a_tile32(Wh, 64, 11, 0, m, q, c);
#pragma unroll
    for (int e = 0; e < 4; ++e) B3[e] = (4 * q + e) < 11 ? a.b[2][4 * q + e] : 0.0f;

    const int64_t wave = (int64_t)blockIdx.x * kBwdWaves + wv;
    const int64_t nwaves = (int64_t)gridDim.x * kBwdWaves;
    float* part = a.partial + wave * (int64_t)(kTileSlots + kBiasSlots) * 64 + lane;
    floatx4_t accH[4], accW2[4][4], accW1[4][2];
    float gbh[4], gb2[4][4], gb1[4][4];
    {
        int j = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) accH[t][e] = a.first ? 0.0f : part[64 * j++];
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) accW2[t >> 2][t & 3][e] = a.first ? 0.0f : part[64 * j++];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) accW1[t >> 1][t & 1][e] = a.first ? 0.0f : part[64 * j++];
#pragma unroll
        for (int e = 0; e < 4; ++e) gbh[e] = a.first ? 0.0f : part[64 * j++];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) gb2[t][e] = a.first ? 0.0f : part[64 * j++];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) gb1[t][e] = a.first ? 0.0f : part[64 * j++];
    }

    float* sG = sT[wv][0];
    float* sH = sT[wv][1];
    const int64_t n = *a.count;
    for (int64_t base = wave * 16; base < n; base += nwaves * 16) {
        const int64_t kc = base + c;  // compact index
        const bool valid = kc < n;
        const int64_t gi = a.list[valid ? kc : n - 1];  // chunk-local Gaussian
        // ---------------- forward (as the decode computes it)
        const int l0 = 2 * q;
        const half8_t Z = cat8(unpack2(a.z[(size_t)l0 * a.zstride + gi], a.z[(size_t)(l0 + 1) * a.zstride + gi]),
                               unpack2(a.z[(size_t)(l0 + 8) * a.zstride + gi], a.z[(size_t)(l0 + 9) * a.zstride + gi]));
        floatx4_t P1[4], P2[4];  // act' of the hidden pre-activations
        half8_t H1[2], H2[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const floatx4_t z0 = {0, 0, 0, 0};
            P1[2 * m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[2 * m], Z, z0, 0, 0, 0);
            P1[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[2 * m + 1], Z, z0, 0, 0, 0);
            half8_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float d0, d1;
                h[e] = (_Float16)act_fwd_grad<GELU>(P1[2 * m][e] + B1[2 * m][e], d0);
                h[4 + e] = (_Float16)act_fwd_grad<GELU>(P1[2 * m + 1][e] + B1[2 * m + 1][e], d1);
                P1[2 * m][e] = d0;  // from here on: act'(a1)
                P1[2 * m + 1][e] = d1;
            }
            H1[m] = h;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            floatx4_t lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2[2 * m][k], H1[k], lo, 0, 0, 0);
                hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2[2 * m + 1][k], H1[k], hi, 0, 0, 0);
            }
            half8_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float d0, d1;
                h[e] = (_Float16)act_fwd_grad<GELU>(lo[e] + B2[2 * m][e], d0);
                h[4 + e] = (_Float16)act_fwd_grad<GELU>(hi[e] + B2[2 * m + 1][e], d1);
                P2[2 * m][e] = d0;  // act'(a2)
                P2[2 * m + 1][e] = d1;
            }
            H2[m] = h;
        }
        floatx4_t accO = {0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < 2; ++k) accO = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3[k], H2[k], accO, 0, 0, 0);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = accO[e] + B3[e];

        // ---------------- Eq. 11 backward.  Rows 4q+e of column c:
        // q = 0: s0 s1 s2 rw | q = 1: rx ry rz c0 | q = 2: c1 c2 op - | q = 3: -
        float up[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (valid) {
            const int64_t u = a.off + gi;
            if (q == 0) {
                up[0] = a.gs[u * 3 + 0];
                up[1] = a.gs[u * 3 + 1];
                up[2] = a.gs[u * 3 + 2];
                up[3] = a.gq[u * 4 + 0];
            } else if (q == 1) {
                up[0] = a.gq[u * 4 + 1];
                up[1] = a.gq[u * 4 + 2];
                up[2] = a.gq[u * 4 + 3];
                up[3] = a.gc[u * 3 + 0];
            } else if (q == 2) {
                up[0] = a.gc[u * 3 + 1];
                up[1] = a.gc[u * 3 + 2];
                up[2] = a.go[u];
            }
        }
        const float part_n = q == 0 ? o[3] * o[3] : (q == 1 ? o[0] * o[0] + o[1] * o[1] + o[2] * o[2] : 0.0f);
        const float rn = sqrtf(part_n + __shfl_xor(part_n, 16));
        const float nrm = fmaxf(rn, 1e-12f);
        const float part_d = q == 0 ? up[3] * (o[3] / nrm)
                                    : (q == 1 ? up[0] * (o[0] / nrm) + up[1] * (o[1] / nrm) + up[2] * (o[2] / nrm) : 0.0f);
        const float dot = rn >= 1e-12f ? part_d + __shfl_xor(part_d, 16) : 0.0f;
        float go[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (q == 0) {
#pragma unroll
            for (int e = 0; e < 3; ++e) go[e] = o[e] < 20.0f ? up[e] * expf(o[e]) : 0.0f;
            go[3] = (up[3] - dot * (o[3] / nrm)) / nrm;
        } else if (q == 1) {
#pragma unroll
            for (int e = 0; e < 3; ++e) go[e] = (up[e] - dot * (o[e] / nrm)) / nrm;
            const float s = sigmoid_f(o[3]);
            go[3] = up[3] * s * (1.0f - s);
        } else if (q == 2) {
#pragma unroll
            for (int e = 0; e < 3; ++e) {
                const float s = sigmoid_f(o[e]);
                go[e] = up[e] * s * (1.0f - s);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) gbh[e] += go[e];

        // ---------------- head: dWh += go H2^T (Gaussians on k through LDS)
#pragma unroll
        for (int e = 0; e < 4; ++e) sG[(4 * q + e) * kTS + c] = go[e];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sH[(32 * m + 4 * q + e) * kTS + c] = (float)H2[m][e];
                sH[(32 * m + 16 + 4 * q + e) * kTS + c] = (float)H2[m][4 + e];
            }
        wave_lds_sync();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float ag = sG[c * kTS + 4 * s + q];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) accH[hb] = mfma4(ag, sH[(16 * hb + c) * kTS + 4 * s + q], accH[hb]);
        }
        wave_lds_sync();
        // dH2 = Wh^T go; da2 = dH2 act'(a2)
        floatx4_t D[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            D[rb] = floatx4_t{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) D[rb] = mfma4(sWh[(rb * 4 + e) * 64 + lane], go[e], D[rb]);
        }
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                D[rb][e] *= P2[rb][e];
                gb2[rb][e] += D[rb][e];
            }
        // ---------------- layer 2: dW2 += da2 H1^T
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) sG[(16 * rb + 4 * q + e) * kTS + c] = D[rb][e];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sH[(32 * m + 4 * q + e) * kTS + c] = (float)H1[m][e];
                sH[(32 * m + 16 + 4 * q + e) * kTS + c] = (float)H1[m][4 + e];
            }
        wave_lds_sync();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float bh[4];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) bh[hb] = sH[(16 * hb + c) * kTS + 4 * s + q];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const float ag = sG[(16 * rb + c) * kTS + 4 * s + q];
#pragma unroll
                for (int hb = 0; hb < 4; ++hb) accW2[rb][hb] = mfma4(ag, bh[hb], accW2[rb][hb]);
            }
        }
        wave_lds_sync();
        // dH1 = W2^T da2; da1 = dH1 act'(a1)
        floatx4_t E[4];
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) {
            E[ob] = floatx4_t{0, 0, 0, 0};
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int e = 0; e < 4; ++e) E[ob] = mfma4(sW2[((ob * 4 + rb) * 4 + e) * 64 + lane], D[rb][e], E[ob]);
        }
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                E[rb][e] *= P1[rb][e];
                gb1[rb][e] += E[rb][e];
            }
        // ---------------- layer 1: dW1 += da1 z^T
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) sG[(16 * rb + 4 * q + e) * kTS + c] = E[rb][e];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sH[(4 * q + e) * kTS + c] = (float)Z[e];
            sH[(16 + 4 * q + e) * kTS + c] = (float)Z[4 + e];
        }
        wave_lds_sync();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float b0 = sH[c * kTS + 4 * s + q], b1 = sH[(16 + c) * kTS + 4 * s + q];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const float ag = sG[(16 * rb + c) * kTS + 4 * s + q];
                accW1[rb][0] = mfma4(ag, b0, accW1[rb][0]);
                accW1[rb][1] = mfma4(ag, b1, accW1[rb][1]);
            }
        }
        wave_lds_sync();
        // dz = W1^T da1: rows 16 ob + 4 q + e = features (e & 1) of level 8 ob + 2 q + (e >> 1)
#pragma unroll
        for (int ob = 0; ob < 2; ++ob) {
            floatx4_t G = {0, 0, 0, 0};
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int e = 0; e < 4; ++e) G = mfma4(sW1[((ob * 4 + rb) * 4 + e) * 64 + lane], E[rb][e], G);
            if (valid) {
                const int lv = 8 * ob + 2 * q;
                a.gz[(size_t)lv * a.gzstride + kc] = make_float2(G[0], G[1]);
                a.gz[(size_t)(lv + 1) * a.gzstride + kc] = make_float2(G[2], G[3]);
            }
        }
    }
    {
        int j = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = accH[t][e];
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = accW2[t >> 2][t & 3][e];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = accW1[t >> 1][t & 1][e];
#pragma unroll
        for (int e = 0; e < 4; ++e) part[64 * j++] = gbh[e];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = gb2[t][e];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = gb1[t][e];
    }
}

// First stage of the partial sums: block (slot j, group g) adds the slot of
// waves [g W, (g + 1) W), W = waves / groups, in wave order, lane by lane.
__global__ void __launch_bounds__(64) mlp_bwd_group_kernel(const float* partial, int waves_per_group,
                                                           float* group_sums) {
    const int stride = (kTileSlots + kBiasSlots) * 64;
    const int j = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
    const float* src = partial + (size_t)g * waves_per_group * stride + j * 64 + lane;
    float s = 0.0f;
    for (int w = 0; w < waves_per_group; ++w) s += src[(size_t)w * stride];
    group_sums[(size_t)g * stride + j * 64 + lane] = s;
}

// Sum the per-wave (or per-group) partials in order.  Thread t < kTileSlots * 64 owns
// one (slot, lane) of the weight tiles; the next 36 * 4 threads own one bias
// slot of one lane group q (summed over its 16 lanes c).
__global__ void __launch_bounds__(256) mlp_bwd_reduce_kernel(const float* partial, int nwaves, float* gW1,
                                                             float* gW2, float* gWh, float* gb1, float* gb2,
                                                             float* gbh) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    const int stride = (kTileSlots + kBiasSlots) * 64;
    if (t < kTileSlots * 64) {
        const int j = t >> 6, lane = t & 63, q = lane >> 4, c = lane & 15, e = j & 3, tile = j >> 2;
        float s = 0.0f;
        for (int w = 0; w < nwaves; ++w) s += partial[(size_t)w * stride + t];
        if (tile < 4) {
            const int row = 4 * q + e;
            if (row < 11) gWh[row * 64 + 16 * tile + c] = s;
        } else if (tile < 20) {
            const int rb = (tile - 4) >> 2, hb = (tile - 4) & 3;
            gW2[(16 * rb + 4 * q + e) * 64 + 16 * hb + c] = s;
        } else {
            const int rb = (tile - 20) >> 1, kb = (tile - 20) & 1;
            gW1[(16 * rb + 4 * q + e) * 32 + 16 * kb + c] = s;
        }
        return;
    }
    const int u = t - kTileSlots * 64;
    if (u >= kBiasSlots * 4) return;
    const int jb = u >> 2, q = u & 3;
    float s = 0.0f;
    for (int w = 0; w < nwaves; ++w)
        for (int c = 0; c < 16; ++c) s += partial[(size_t)w * stride + (kTileSlots + jb) * 64 + 16 * q + c];
    if (jb < 4) {
        const int row = 4 * q + jb;
        if (row < 11) gbh[row] = s;
    } else if (jb < 20) {
        const int rb = (jb - 4) >> 2, e = (jb - 4) & 3;
        gb2[16 * rb + 4 * q + e] = s;
    } else {
        const int rb = (jb - 20) >> 2, e = (jb - 20) & 3;
        gb1[16 * rb + 4 * q + e] = s;
    }
}

// Per-block combining of table-gradient contributions (see the file header):
// kAggSlots entries of LDS, at most kAggProbes linear probes, then a direct
// global atomic.
constexpr int kAggBits = 11;
constexpr int kAggSlots = 1 << kAggBits;
constexpr int kAggProbes = 8;
constexpr uint32_t kAggEmpty = 0xffffffffu;  // table indices are < 2^24
constexpr int kAggMaxRes = 640;
// rounds of 64 Gaussians per combining block: 384 Gaussians share one
// 2048-slot LDS table (24 KiB, six blocks per CU); 768 Gaussians on 4096
// slots, 512 or 768 on 2048, and 192 on 1024 measured slower
constexpr int kAggRounds = 6;

__device__ __forceinline__ void agg_add(uint32_t* key, float* v0, float* v1, uint32_t idx, float a, float b,
                                        float* gt) {
    uint32_t slot = (idx * 2654435761u) >> (32 - kAggBits);
    for (int p = 0; p < kAggProbes; ++p) {
        // a set key never changes: a plain read settles most probes, the
        // compare-and-swap only claims an empty slot
        uint32_t old = key[slot];
        if (old == kAggEmpty) old = atomicCAS(&key[slot], kAggEmpty, idx);
        if (old == kAggEmpty || old == idx) {
            atomicAdd(&v0[slot], a);
            atomicAdd(&v1[slot], b);
            return;
        }
        slot = (slot + 1) & (kAggSlots - 1);
    }
    atomicAdd(gt + 2 * (size_t)idx, a);
    atomicAdd(gt + 2 * (size_t)idx + 1, b);
}

// Eq. 9 and Eq. 7 backward, level-major as the gather, levels level0 + 0, 1,
// ...  Lane s of a group of four takes the x/y corner (s & 1, s >> 1) and its
// four z/t corners.  AGG: combine per entry in LDS first (every thread of a
// block reaches the final barrier: the only early exit is block-uniform).
template <bool POS, bool AGG>
__global__ void __launch_bounds__(256) scatter_kernel(const float4* xt, const float* pos, int stride,
                                                      const uint32_t* list, const uint32_t* count, int nchunk,
                                                      int level0, HashLevels h, const uint32_t* tables,
                                                      const float2* gz, int64_t zstride, float* gtab,
                                                      float4* gpos_part) {
#pragma clang fp contract(fast)
    __shared__ uint32_t s_key[AGG ? kAggSlots : 1];
    __shared__ float s_v0[AGG ? kAggSlots : 1], s_v1[AGG ? kAggSlots : 1];
    const int level = level0 + (int)(blockIdx.x / nchunk);
    constexpr int kRounds = AGG ? kAggRounds : 4;
    const int64_t first = (int64_t)(blockIdx.x % nchunk) * (64 * kRounds);
    const int64_t n = *count;  // Gaussians with a gradient, compacted
    if (first >= n) return;
    if constexpr (AGG) {
        for (int k = threadIdx.x; k < kAggSlots; k += 256) {
            s_key[k] = kAggEmpty;
            s_v0[k] = 0.0f;
            s_v1[k] = 0.0f;
        }
        __syncthreads();
    }
    const int res = h.res_s[level], res_t = h.res_t[level];
    const bool dense = h.dense[level] != 0;
    const uint32_t* tab = tables + (size_t)level * h.T;
    float* gt = gtab + (size_t)level * h.T * 2;
    const int s = threadIdx.x & 3;
    const int bx = s & 1, by = s >> 1;
    const int sub = threadIdx.x >> 2;
    const uint32_t r = (uint32_t)res, r2 = r * r, r3 = r2 * r;
    for (int j = 0; j < kRounds; ++j) {
        const int64_t k = first + j * 64 + sub;  // compact index
        if (k >= n) break;  // uniform across each group of four lanes
        const int64_t i = list[k];  // chunk-local Gaussian
        const float4 p = xt[i];
        const float2 g = gz[(size_t)level * zstride + k];
        int cx, cy, cz, ct;
        float fx, fy, fz, ft;
        cell_axis(p.x, res, cx, fx);
        cell_axis(p.y, res, cy, fy);
        cell_axis(p.z, res, cz, fz);
        cell_axis(p.w, res_t, ct, ft);
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
        const float wx = bx ? fx : 1.0f - fx, wy = by ? fy : 1.0f - fy;
        const float sx = bx ? 1.0f : -1.0f, sy = by ? 1.0f : -1.0f;
        const float wxy = wx * wy;
        const float wz[2] = {1.0f - fz, fz}, wt[2] = {1.0f - ft, ft};
        // no gradient at this level: nothing to add, no position term (uniform over the four lanes)
        if (g.x == 0.0f && g.y == 0.0f) {
            if (POS && s == 0) gpos_part[(size_t)level * zstride + k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            continue;
        }
        float dx = 0.0f, dy = 0.0f, dz = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int bz = k & 1, bt = k >> 1;
            // a corner of zero time weight has zero weight and zero spatial derivatives
            if (wt[bt] == 0.0f) continue;
            const uint32_t idx = (dense ? (txy + tz[bz] + tt[bt]) : (txy ^ tz[bz] ^ tt[bt])) & h.mask;
            const float w = (wxy * wz[bz]) * wt[bt];
            if (w != 0.0f) {
                if constexpr (AGG) {
                    agg_add(s_key, s_v0, s_v1, idx, w * g.x, w * g.y, gt);
                } else {
                    atomicAdd(gt + 2 * (size_t)idx, w * g.x);
                    atomicAdd(gt + 2 * (size_t)idx + 1, w * g.y);
                }
            }
            if (POS) {
                const uint32_t raw = tab[idx];
                const float v0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw & 0xffffu));
                const float v1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw >> 16));
                const float tg = v0 * g.x + v1 * g.y;
                const float wzt = wz[bz] * wt[bt];
                dx += tg * (sx * wy) * wzt;
                dy += tg * (wx * sy) * wzt;
                dz += tg * wxy * ((bz ? 1.0f : -1.0f) * wt[bt]);
            }
        }
        if (POS) {
            dx += __shfl_xor(dx, 1, 4);
            dy += __shfl_xor(dy, 1, 4);
            dz += __shfl_xor(dz, 1, 4);
            dx += __shfl_xor(dx, 2, 4);
            dy += __shfl_xor(dy, 2, 4);
            dz += __shfl_xor(dz, 2, 4);
            if (s == 0) {
                const float sc = (float)(res - 1);
                const float gx[3] = {dx * sc, dy * sc, dz * sc};
                const float* mu = pos + i * stride;
                const float m0 = mu[0], m1 = mu[1], m2 = mu[2];
                const float nn = sqrtf(m0 * m0 + m1 * m1 + m2 * m2);
                float out[3];
                if (nn <= 1.0f) {
#pragma unroll
                    for (int k = 0; k < 3; ++k) out[k] = 0.25f * gx[k];
                } else {
                    // x~ = c(mu)/4 + 1/2, c = gn mu, gn = 2/n - 1/n^2: J = gn I + (gn'/n) mu mu^T
                    const float inv = 1.0f / nn;
                    const float gn = (2.0f - inv) * inv;
                    const float gp_n = (-2.0f + 2.0f * inv) * inv * inv * inv;
                    const float md = m0 * gx[0] + m1 * gx[1] + m2 * gx[2];
                    out[0] = 0.25f * (gn * gx[0] + gp_n * m0 * md);
                    out[1] = 0.25f * (gn * gx[1] + gp_n * m1 * md);
                    out[2] = 0.25f * (gn * gx[2] + gp_n * m2 * md);
                }
                // this level's share, summed over the levels by pos_reduce_kernel
                gpos_part[(size_t)level * zstride + k] = make_float4(out[0], out[1], out[2], 0.0f);
            }
        }
    }
    if constexpr (AGG) {
        __syncthreads();
        for (int k = threadIdx.x; k < kAggSlots; k += 256) {
            const uint32_t idx = s_key[k];
            if (idx != kAggEmpty) {
                atomicAdd(gt + 2 * (size_t)idx, s_v0[k]);
                atomicAdd(gt + 2 * (size_t)idx + 1, s_v1[k]);
            }
        }
    }
}

// Position gradient of the active Gaussians: the levels' shares added in level
// order (deterministic) to what the position gradient already holds.
__global__ void __launch_bounds__(256) pos_reduce_kernel(const uint32_t* list, const uint32_t* count, int L,
                                                         const float4* part, int64_t zstride, float* gpos) {
    const int64_t n = *count;
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < n; k += (int64_t)gridDim.x * 256) {
        float sx = 0.0f, sy = 0.0f, sz = 0.0f;
        for (int l = 0; l < L; ++l) {
            const float4 p = part[(size_t)l * zstride + k];
            sx += p.x;
            sy += p.y;
            sz += p.z;
        }
        float* dst = gpos + (size_t)list[k] * 3;
        dst[0] += sx;
        dst[1] += sy;
        dst[2] += sz;
    }
}

// Compaction of the chunk's Gaussians whose upstream gradient is not all zero
// (their decoder gradients are exactly zero otherwise), in index order:
// per-block counts, one exclusive scan, ordered writes.
constexpr int kCompactItems = 4096;  // per block: 256 threads x 16 rounds

__device__ __forceinline__ bool has_gradient(const float* gs, const float* gq, const float* gc, const float* go,
                                             int64_t u) {
    // all eleven values are loaded (no short circuit, so the loads overlap);
    // a value counts unless it is +0 or -0 (NaN counts)
    uint32_t bits = __float_as_uint(go[u]);
#pragma unroll
    for (int k = 0; k < 3; ++k) bits |= __float_as_uint(gs[u * 3 + k]) | __float_as_uint(gc[u * 3 + k]);
#pragma unroll
    for (int k = 0; k < 4; ++k) bits |= __float_as_uint(gq[u * 4 + k]);
    return (bits & 0x7fffffffu) != 0u;
}

__global__ void __launch_bounds__(256) active_count_kernel(const float* gs, const float* gq, const float* gc,
                                                           const float* go, int64_t off, int64_t n, uint32_t* bcount) {
    __shared__ uint32_t s_cnt[4];
    const int64_t b0 = (int64_t)blockIdx.x * kCompactItems;
    uint32_t cnt = 0;
    for (int r = 0; r < kCompactItems / 256; ++r) {
        const int64_t i = b0 + r * 256 + threadIdx.x;
        if (i < n && has_gradient(gs, gq, gc, go, off + i)) ++cnt;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
    if ((threadIdx.x & 63) == 0) s_cnt[threadIdx.x >> 6] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) bcount[blockIdx.x] = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
}

// Exclusive scan of nb <= 256 * 8 block counts in place; total into *count.
__global__ void __launch_bounds__(256) active_scan_kernel(uint32_t* bcount, int nb, uint32_t* count,
                                                          uint64_t* count64) {
    __shared__ uint32_t s_sum[256];
    constexpr int kPer = 8;
    uint32_t v[kPer], run = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = threadIdx.x * kPer + k;
        v[k] = i < nb ? bcount[i] : 0u;
        run += v[k];
    }
    s_sum[threadIdx.x] = run;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const uint32_t add = threadIdx.x >= (unsigned)o ? s_sum[threadIdx.x - o] : 0u;
        __syncthreads();
        s_sum[threadIdx.x] += add;
        __syncthreads();
    }
    uint32_t base = s_sum[threadIdx.x] - run;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = threadIdx.x * kPer + k;
        if (i < nb) bcount[i] = base;
        base += v[k];
    }
    if (threadIdx.x == 255) {
        *count = s_sum[255];
        *count64 = s_sum[255];
    }
}

// 8 bits of v in [0, 1] spread to every third bit (bits 0, 3, ..., 21)
__device__ __forceinline__ uint32_t spread3(float v) {
    uint32_t q = (uint32_t)(fminf(fmaxf(v, 0.0f), 1.0f) * 255.0f);
    q = (q | (q << 8)) & 0x0000f00fu;
    q = (q | (q << 4)) & 0x000c30c3u;
    q = (q | (q << 2)) & 0x00249249u;
    return q;
}

// sort key of a normalised position: 6 bits of time above the 24-bit Morton
// code of x, y, z (30 bits: three 10-bit radix passes)
__device__ __forceinline__ uint32_t spatial_key(float4 p) {
    const uint32_t tq = (uint32_t)(fminf(fmaxf(p.w, 0.0f), 1.0f) * 63.0f);
    return (tq << 24) | spread3(p.x) | (spread3(p.y) << 1) | (spread3(p.z) << 2);
}

__global__ void __launch_bounds__(256) active_write_kernel(const float* gs, const float* gq, const float* gc,
                                                           const float* go, int64_t off, int64_t n,
                                                           const uint32_t* boff, const float4* xt,
                                                           uint64_t* items) {
    __shared__ uint32_t s_w[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t b0 = (int64_t)blockIdx.x * kCompactItems;
    uint32_t pos = boff[blockIdx.x];
    for (int r = 0; r < kCompactItems / 256; ++r) {
        const int64_t i = b0 + r * 256 + threadIdx.x;
        const bool f = i < n && has_gradient(gs, gq, gc, go, off + i);
        const uint64_t m = __ballot(f);
        if (lane == 0) s_w[wv] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t before = 0;
        for (int w = 0; w < wv; ++w) before += s_w[w];
        const uint32_t rank = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
        if (f) items[pos + before + rank] = ((uint64_t)spatial_key(xt[i]) << 32) | (uint64_t)i;
        pos += s_w[0] + s_w[1] + s_w[2] + s_w[3];
        __syncthreads();
    }
}

// the chunk-local indices of the sorted (key, index) words
__global__ void __launch_bounds__(256) unpack_list_kernel(const uint64_t* items, const uint32_t* count,
                                                          uint32_t* list) {
    const int64_t n = *count;
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < n; k += (int64_t)gridDim.x * 256)
        list[k] = (uint32_t)items[k];
}

__global__ void fill_kernel(float* p, int64_t n, const float* src) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = src ? src[i] : 0.0f;
}

int blocks_for(int64_t n, int per, int cap) {
    int64_t b = (n + per - 1) / per;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (int)b;
}

constexpr int64_t kBwdChunk = kDecodeChunk / 2;

// the sort scratch: two buffers of kBwdChunk words, the radix counts, the
// digit totals and the item count
struct SortScratch {
    uint64_t* items[2];
    uint32_t* counts;
    uint32_t* digit_tot;
    uint64_t* count;
    int max_blocks;
};

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

SortScratch sort_scratch(void* base) {
    SortScratch t{};
    char* p = static_cast<char*>(base);
    t.max_blocks = radix_sort_blocks(kBwdChunk);
    t.items[0] = reinterpret_cast<uint64_t*>(p);
    p += align256(kBwdChunk * sizeof(uint64_t));
    t.items[1] = reinterpret_cast<uint64_t*>(p);
    p += align256(kBwdChunk * sizeof(uint64_t));
    t.counts = reinterpret_cast<uint32_t*>(p);
    p += align256(radix_sort_counts_bytes(t.max_blocks));
    t.digit_tot = reinterpret_cast<uint32_t*>(p);
    p += align256(4 * 1024);
    t.count = reinterpret_cast<uint64_t*>(p);
    return t;
}

}  // namespace

size_t decode_bwd_pos_bytes(int L) { return (size_t)L * kBwdChunk * sizeof(float4); }

size_t decode_bwd_sort_bytes() {
    return 2 * align256(kBwdChunk * sizeof(uint64_t)) + align256(radix_sort_counts_bytes(radix_sort_blocks(kBwdChunk))) +
           align256(4 * 1024) + 256;
}

hipError_t launch_decode_backward(const DecodeBwdArgs& b, hipStream_t s) {
    const DecodeArgs& a = b.fwd;
    const size_t tab_floats = (size_t)a.h.L * a.h.T * 2;
    IA_LAUNCH("decode_bwd_fill_kernel", fill_kernel, dim3(blocks_for((int64_t)tab_floats, 256, 8192)), dim3(256), 0,
              s, b.g_tables, (int64_t)tab_floats, (const float*)nullptr);
    if (b.g_pos && a.N > 0)
        IA_LAUNCH("decode_bwd_fill_kernel", fill_kernel, dim3(blocks_for(a.N * 3, 256, 8192)), dim3(256), 0, s,
                  b.g_pos, a.N * 3, b.g_means);
    const int64_t chunk = kBwdChunk;
    const SortScratch srt = sort_scratch(b.sort);
    const size_t zslot = (size_t)a.h.L * a.zcap;
    float4* xt = reinterpret_cast<float4*>(a.zbuf + 2 * zslot);
    uint32_t* z = a.zbuf;
    float2* gz = reinterpret_cast<float2*>(a.zbuf + (size_t)a.h.L * chunk);
    // after z and dz: the compacted list of a chunk, per-block offsets and the count
    uint32_t* list = a.zbuf + (size_t)3 * a.h.L * chunk;
    uint32_t* boff = list + chunk;
    const int nbc = (int)(chunk / kCompactItems);
    uint32_t* count = boff + nbc;
    MlpBwdArgs m{};
    for (int k = 0; k < 3; ++k) {
        m.W[k] = (const _Float16*)a.W[k];
        m.b[k] = a.b[k];
    }
    m.gelu = a.act == IA_ACT_GELU;
    m.gzstride = chunk;
    m.gs = b.g_scales;
    m.gq = b.g_quats;
    m.gc = b.g_colors;
    m.go = b.g_opacity;
    m.gz = gz;
    m.partial = b.partial;
    int first = 1;
    for (int64_t off = 0; off < a.N; off += chunk) {
        const int64_t n = a.N - off < chunk ? a.N - off : chunk;
        // features kept by the forward ([L][N]) or recomputed into the scratch ([L][chunk])
        hipError_t e = launch_decode_features(a, off, n, xt, a.features ? nullptr : z, chunk, s);
        if (e != hipSuccess) return e;
        m.z = a.features ? a.features + off : z;
        m.zstride = a.features ? a.N : chunk;
        const int nb = (int)((n + kCompactItems - 1) / kCompactItems);
        IA_LAUNCH("active_count_kernel", active_count_kernel, dim3(nb), dim3(256), 0, s, b.g_scales, b.g_quats,
                  b.g_colors, b.g_opacity, off, n, boff);
        IA_LAUNCH("active_scan_kernel", active_scan_kernel, dim3(1), dim3(256), 0, s, boff, nb, count, srt.count);
        IA_LAUNCH("active_write_kernel", active_write_kernel, dim3(nb), dim3(256), 0, s, b.g_scales, b.g_quats,
                  b.g_colors, b.g_opacity, off, n, boff, xt, srt.items[0]);
        // stable sort on the 30 key bits above the index
        const int cur = radix_sort_u64(srt.items, srt.count, (uint64_t)chunk, 32, 30, srt.max_blocks, srt.counts,
                                       srt.digit_tot, s);
        IA_LAUNCH("unpack_list_kernel", unpack_list_kernel, dim3(blocks_for(n, 256, 2048)), dim3(256), 0, s,
                  srt.items[cur], count, list);
        m.list = list;
        m.count = count;
        m.off = off;
        m.first = first;
        first = 0;
        IA_LAUNCH("mlp_bwd_kernel", m.gelu ? mlp_bwd_kernel<true> : mlp_bwd_kernel<false>, dim3(kDecodeBwdBlocks),
                  dim3(kBwdThreads), 0, s, m);
        const int nchunk = (int)((n + 255) / 256), nchunk_agg = (int)((n + 64 * kAggRounds - 1) / (64 * kAggRounds));
        const float* pos = a.pos + off * a.stride;
        float* gpos = b.g_pos ? b.g_pos + off * 3 : nullptr;
        // levels [0, nagg) combine in LDS first (resolution grows with the level)
        int nagg = 0;
        while (nagg < a.h.L && a.h.res_s[nagg] <= kAggMaxRes) ++nagg;
        auto scatter = [&](auto pos_t, auto agg_t, int level0, int levels) {
            constexpr bool P = decltype(pos_t)::value, G = decltype(agg_t)::value;
            const int nc = G ? nchunk_agg : nchunk;
            if (levels > 0)
                IA_LAUNCH(G ? "scatter_agg_kernel" : "scatter_kernel", (scatter_kernel<P, G>),
                          dim3((unsigned)(levels * nc)), dim3(256), 0,
                          s, xt, pos, a.stride, list, count, nc, level0, a.h, (const uint32_t*)a.tables, gz,
                          chunk, b.g_tables, b.pos_partial);
        };
        if (b.g_pos) {
            scatter(std::true_type{}, std::true_type{}, 0, nagg);
            scatter(std::true_type{}, std::false_type{}, nagg, a.h.L - nagg);
            IA_LAUNCH("pos_reduce_kernel", pos_reduce_kernel, dim3(blocks_for(n, 256, 4096)), dim3(256), 0, s, list,
                      count, a.h.L, (const float4*)b.pos_partial, chunk, gpos);
        } else {
            scatter(std::false_type{}, std::true_type{}, 0, nagg);
            scatter(std::false_type{}, std::false_type{}, nagg, a.h.L - nagg);
        }
    }
    if (first) {  // N = 0: the weight and bias gradients are zero
        const int64_t nf = (int64_t)kDecodeBwdBlocks * kBwdWaves * (kTileSlots + kBiasSlots) * 64;
        IA_LAUNCH("decode_bwd_fill_kernel", fill_kernel, dim3(blocks_for(nf, 256, 8192)), dim3(256), 0, s, b.partial,
                  nf, (const float*)nullptr);
    }
    // fixed-order two-stage sum of the per-wave partials (deterministic)
    const int nwaves = kDecodeBwdBlocks * kBwdWaves;
    float* groups = b.partial + (size_t)nwaves * (kTileSlots + kBiasSlots) * 64;
    IA_LAUNCH("mlp_bwd_group_kernel", mlp_bwd_group_kernel, dim3(kTileSlots + kBiasSlots, kDecodeBwdGroups), dim3(64),
              0, s, b.partial, nwaves / kDecodeBwdGroups, groups);
    const int nred = kTileSlots * 64 + kBiasSlots * 4;
    IA_LAUNCH("mlp_bwd_reduce_kernel", mlp_bwd_reduce_kernel, dim3((nred + 255) / 256), dim3(256), 0, s, groups,
              kDecodeBwdGroups, b.g_W[0], b.g_W[1], b.g_W[2], b.g_b[0], b.g_b[1], b.g_b[2]);
    return hipGetLastError();
}

}  // namespace ia
