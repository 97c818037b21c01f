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
//                (GELU' reuses GELU's normal tail Q);
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
//       dz       written to the scratch, fp32, [level][Gaussian] x F features.
//   mlp_bwd_branch_kernel  the same for one branch of the per-attribute
//       decoder (F = 4, 64 -> 64 -> 64 -> out), one launch per branch: the
//       branches' encoding gradients add up in dz, each branch's weight
//       gradients are reduced after its launch.
//   table and position gradients, level-major like the gather, four lanes
//       per (Gaussian, level), each with four of the 16 corners:
//       dtable[corner] += w dz (how it is summed: below); for positions dz/df_axis = sum_c (+-1) prod_{other
//       axes} w table[c] (time carries no gradient), times (res - 1), then the
//       Jacobian of Eq. 7: each level's share is stored (one 16-byte store per
//       Gaussian and level, in list order) and pos_reduce_kernel adds the
//       levels in a fixed order to the position gradient (no atomics).
//       Global float atomics are served far below L2 speed on this chip, LDS
//       ones are not.  scatter_kernel: on levels of at most kAggMaxRes
//       vertices per axis, where the block's Gaussians share corners, each
//       block first adds its contributions per table entry in an LDS hash
//       table (open addressing, LDS atomics), then issues one global atomic
//       per distinct entry and feature.  bucket_scatter_kernel and
//       bucket_add_kernel: on the finer levels the contributions go as
//       (entry, value) records into per-bucket runs (2^11 table entries a
//       bucket) and one block per bucket sums them in LDS and adds them to
//       the table's gradient with plain stores; with few Gaussians with a
//       gradient in the chunk, direct float atomics instead.
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
// The head block has HT row tiles of 16: 1 for the RGB head (11 rows), 4 for
// the SH colour head (56 rows: s | r | 48 SH | o).  Per lane of a wave's
// partial slot: 4 HT head tiles + 16 W2 tiles + 8 W1 tiles (4 floats each),
// then 4 HT + 16 + 16 bias partials.
template <int HT>
constexpr int tile_slots() { return (4 * HT + 16 + 8) * 4; }
template <int HT>
constexpr int bias_slots() { return 4 * HT + 16 + 16; }
template <int HT>
constexpr int head_rows() { return HT == 1 ? 11 : 56; }
static_assert(tile_slots<4>() + bias_slots<4>() <= kDecodeBwdSlotFloats / 64, "partial slots hold the SH head");
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
        return fmaf(-fabsf(x), q, relu_med3(x));
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
    const float* gc;  // [N,3] colours, or [N,48] SH coefficients (HT = 4)
    const float* go;
    float2* gz;      // [L][gzstride]
    int64_t gzstride;
    float* partial;  // [waves][kDecodeBwdSlotFloats]: tile_slots<HT>() + bias_slots<HT>() rows of 64
    int first;       // 1: the partial slots start from zero
};

template <bool GELU, int HT>
__global__ void __launch_bounds__(kBwdThreads, 1) mlp_bwd_kernel(MlpBwdArgs a) {
#pragma clang fp contract(fast)
    constexpr int HEAD = head_rows<HT>();
    constexpr bool SH = HT == 4;
    // fp32 operands of the data-gradient products, lane-ordered:
    //   sWh[ht][rb][e][lane] = Wh[16ht+4q+e][16rb+c], sW2[ob][rb][e][lane] = W2[16rb+4q+e][16ob+c],
    //   sW1[ob][rb][e][lane] = W1[16rb+4q+e][16ob+c]
    __shared__ float sWh[HT * 4 * 4 * 64];
    __shared__ float sW2[4 * 4 * 4 * 64];
    __shared__ float sW1[2 * 4 * 4 * 64];
    __shared__ float sT[kBwdWaves][2][64 * kTS];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int q = lane >> 4, c = lane & 15;
    const _Float16* W1 = a.W[0];
    const _Float16* W2 = a.W[1];
    const _Float16* Wh = a.W[2];
    for (int k = threadIdx.x; k < HT * 4 * 4 * 64; k += kBwdThreads) {
        const int l = k & 63, e = (k >> 6) & 3, rb = (k >> 8) & 3, ht = k >> 10, qq = l >> 4, cc = l & 15;
        const int row = 16 * ht + 4 * qq + e;
        sWh[k] = row < HEAD ? (float)Wh[row * 64 + 16 * rb + cc] : 0.0f;
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
    half8_t A1[4], A2[4][2], A3[HT][2];
    // biases as the recomputed forward's initial MFMA accumulators, as the decode does
    floatx4_t B1[4], B2[4], B3[HT];
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
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
        for (int m = 0; m < 2; ++m) A3[ht][m] = a_tile32(Wh, 64, HEAD, ht, m, q, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) B3[ht][e] = (16 * ht + 4 * q + e) < HEAD ? a.b[2][16 * ht + 4 * q + e] : 0.0f;
    }

    const int64_t wave = (int64_t)blockIdx.x * kBwdWaves + wv;
    const int64_t nwaves = (int64_t)gridDim.x * kBwdWaves;
    float* part = a.partial + wave * (int64_t)kDecodeBwdSlotFloats + lane;
    floatx4_t accH[HT][4], accW2[4][4], accW1[4][2];
    float gbh[HT][4], gb2[4][4], gb1[4][4];
    {
        int j = 0;
#pragma unroll
        for (int t = 0; t < 4 * HT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) accH[t >> 2][t & 3][e] = a.first ? 0.0f : part[64 * j++];
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) accW2[t >> 2][t & 3][e] = a.first ? 0.0f : part[64 * j++];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) accW1[t >> 1][t & 1][e] = a.first ? 0.0f : part[64 * j++];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) gbh[ht][e] = a.first ? 0.0f : part[64 * j++];
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
            P1[2 * m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[2 * m], Z, B1[2 * m], 0, 0, 0);
            P1[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[2 * m + 1], Z, B1[2 * m + 1], 0, 0, 0);
            half8_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float d0, d1;
                h[e] = (_Float16)act_fwd_grad<GELU>(P1[2 * m][e], d0);
                h[4 + e] = (_Float16)act_fwd_grad<GELU>(P1[2 * m + 1][e], d1);
                P1[2 * m][e] = d0;  // from here on: act'(a1)
                P1[2 * m + 1][e] = d1;
            }
            H1[m] = h;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            floatx4_t lo = B2[2 * m], hi = B2[2 * m + 1];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2[2 * m][k], H1[k], lo, 0, 0, 0);
                hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2[2 * m + 1][k], H1[k], hi, 0, 0, 0);
            }
            half8_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float d0, d1;
                h[e] = (_Float16)act_fwd_grad<GELU>(lo[e], d0);
                h[4 + e] = (_Float16)act_fwd_grad<GELU>(hi[e], d1);
                P2[2 * m][e] = d0;  // act'(a2)
                P2[2 * m + 1][e] = d1;
            }
            H2[m] = h;
        }
        float o[HT][4];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            floatx4_t accO = B3[ht];
#pragma unroll
            for (int k = 0; k < 2; ++k) accO = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3[ht][k], H2[k], accO, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[ht][e] = accO[e];
        }

        // ---------------- Eq. 11 backward.  Head row r = 16 ht + 4 q + e of
        // column c.  Tile 0: q = 0: s0 s1 s2 rw | q = 1: rx ry rz, then row 7
        // (RGB: c0 c1 c2 op; SH: the 48 coefficients up to row 54, opacity 55)
        float up[HT][4];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * ht + 4 * q + e;
                float v = 0.0f;
                if (valid) {
                    const int64_t u = a.off + gi;
                    if (r < 3)
                        v = a.gs[u * 3 + r];
                    else if (r < 7)
                        v = a.gq[u * 4 + (r - 3)];
                    else if (r < HEAD - 1)
                        v = a.gc[u * (HEAD - 8) + (r - 7)];
                    else if (r == HEAD - 1)
                        v = a.go[u];
                }
                up[ht][e] = v;
            }
        const float part_n =
            q == 0 ? o[0][3] * o[0][3] : (q == 1 ? o[0][0] * o[0][0] + o[0][1] * o[0][1] + o[0][2] * o[0][2] : 0.0f);
        const float rn = sqrtf(part_n + __shfl_xor(part_n, 16));
        const float nrm = fmaxf(rn, 1e-12f);
        const float part_d = q == 0 ? up[0][3] * (o[0][3] / nrm)
                                    : (q == 1 ? up[0][0] * (o[0][0] / nrm) + up[0][1] * (o[0][1] / nrm) +
                                                    up[0][2] * (o[0][2] / nrm)
                                              : 0.0f);
        const float dot = rn >= 1e-12f ? part_d + __shfl_xor(part_d, 16) : 0.0f;
        float go[HT][4];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * ht + 4 * q + e;
                const float x = o[ht][e], g = up[ht][e];
                float d = 0.0f;
                if (r < 3) {
                    d = x < 20.0f ? g * expf(x) : 0.0f;
                } else if (r < 7) {
                    d = (g - dot * (x / nrm)) / nrm;
                } else if (r < HEAD) {
                    if (SH && r < HEAD - 1) {
                        d = g;  // an SH coefficient is its head output
                    } else {
                        const float sg = sigmoid_f(x);
                        d = g * sg * (1.0f - sg);
                    }
                }
                go[ht][e] = d;
            }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) gbh[ht][e] += go[ht][e];

        // ---------------- head: dWh += go H2^T (Gaussians on k through LDS)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) sG[(16 * ht + 4 * q + e) * kTS + c] = go[ht][e];
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
            float bh[4];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) bh[hb] = sH[(16 * hb + c) * kTS + 4 * s + q];
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const float ag = sG[(16 * ht + c) * kTS + 4 * s + q];
#pragma unroll
                for (int hb = 0; hb < 4; ++hb) accH[ht][hb] = mfma4(ag, bh[hb], accH[ht][hb]);
            }
        }
        wave_lds_sync();
        // dH2 = Wh^T go; da2 = dH2 act'(a2)
        floatx4_t D[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            D[rb] = floatx4_t{0, 0, 0, 0};
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int e = 0; e < 4; ++e) D[rb] = mfma4(sWh[((ht * 4 + rb) * 4 + e) * 64 + lane], go[ht][e], D[rb]);
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
        for (int t = 0; t < 4 * HT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = accH[t >> 2][t & 3][e];
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = accW2[t >> 2][t & 3][e];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = accW1[t >> 1][t & 1][e];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = gbh[ht][e];
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

// ---------------------------------------------------------------- per-attribute branches
//
// The paper-scale decoder (F = 4 encoding of 64 features, one GELU MLP
// 64 -> 64 -> 64 -> out per attribute) differentiated one branch per launch:
// the forward of branch BR recomputed exactly as mlp_branch_kernel runs it
// (same A tiles, biases as the initial accumulators, fp16 hidden
// activations), Eq. 11 of its own rows, the data and weight gradients as in
// mlp_bwd_kernel, and its input gradient added into dz (branch 0 writes it).
// Lane (q, c): Z[m] slots e < 4 are the four features of level 8 m + q, e >= 4
// those of level 8 m + 4 + q; the dz tile ob holds inputs 16 ob + 4 q + e, the
// four features of level 4 ob + q.
__host__ __device__ constexpr int branch_out(int br, bool sh) { return br == 0 ? 3 : (br == 1 ? 4 : (br == 2 ? (sh ? 48 : 3) : 1)); }
__host__ __device__ constexpr int branch_head_tiles(int br, bool sh) { return br == 2 && sh ? 3 : 1; }
template <int HT>
constexpr int branch_tile_slots() { return (4 * HT + 16 + 16) * 4; }
template <int HT>
constexpr int branch_bias_slots() { return 4 * HT + 16 + 16; }
static_assert(branch_tile_slots<3>() + branch_bias_slots<3>() <= kDecodeBwdSlotFloats / 64, "partial slots hold a branch");

struct BranchBwdArgs {
    const _Float16* W[3];  // the branch's [64][64], [64][64], [out][64]
    const float* b[3];
    const uint2* z;        // [L][zstride] four fp16 per level
    int64_t zstride;
    const uint32_t* list;
    const uint32_t* count;
    int64_t off;
    const float* gup;      // the branch's upstream gradient, [N][out] (or opacity [N])
    float4* gz;            // [L][gzstride]
    int64_t gzstride;
    float* partial;        // [waves][kDecodeBwdSlotFloats]
};

__device__ __forceinline__ half4_t unpack4(uint2 v) { return unpack2(v.x, v.y); }

template <bool GELU, int BR, bool SH>
__global__ void __launch_bounds__(kBwdThreads, 1) mlp_bwd_branch_kernel(BranchBwdArgs a) {
#pragma clang fp contract(fast)
    constexpr int HT = branch_head_tiles(BR, SH), OUT = branch_out(BR, SH);
    __shared__ float sWh[HT * 4 * 4 * 64];
    __shared__ float sW2[4 * 4 * 4 * 64];
    __shared__ float sW1[4 * 4 * 4 * 64];
    __shared__ float sT[kBwdWaves][2][64 * kTS];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int q = lane >> 4, c = lane & 15;
    const _Float16* W1 = a.W[0];
    const _Float16* W2 = a.W[1];
    const _Float16* Wh = a.W[2];
    for (int k = threadIdx.x; k < HT * 4 * 4 * 64; k += kBwdThreads) {
        const int l = k & 63, e = (k >> 6) & 3, rb = (k >> 8) & 3, ht = k >> 10, qq = l >> 4, cc = l & 15;
        const int row = 16 * ht + 4 * qq + e;
        sWh[k] = row < OUT ? (float)Wh[row * 64 + 16 * rb + cc] : 0.0f;
    }
    for (int k = threadIdx.x; k < 4 * 4 * 4 * 64; k += kBwdThreads) {
        const int l = k & 63, e = (k >> 6) & 3, rb = (k >> 8) & 3, ob = k >> 10, qq = l >> 4, cc = l & 15;
        sW2[k] = (float)W2[(16 * rb + 4 * qq + e) * 64 + 16 * ob + cc];
        sW1[k] = (float)W1[(16 * rb + 4 * qq + e) * 64 + 16 * ob + cc];
    }
    __syncthreads();

    half8_t A1[4][2], A2[4][2], A3[HT][2];
    floatx4_t B1[4], B2[4], B3[HT];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            A1[rb][m] = a_tile32(W1, 64, 64, rb, m, q, c);
            A2[rb][m] = a_tile32(W2, 64, 64, rb, m, q, c);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            B1[rb][e] = a.b[0][16 * rb + 4 * q + e];
            B2[rb][e] = a.b[1][16 * rb + 4 * q + e];
        }
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
        for (int m = 0; m < 2; ++m) A3[ht][m] = a_tile32(Wh, 64, OUT, ht, m, q, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) B3[ht][e] = (16 * ht + 4 * q + e) < OUT ? a.b[2][16 * ht + 4 * q + e] : 0.0f;
    }

    const int64_t wave = (int64_t)blockIdx.x * kBwdWaves + wv;
    const int64_t nwaves = (int64_t)gridDim.x * kBwdWaves;
    float* part = a.partial + wave * (int64_t)kDecodeBwdSlotFloats + lane;
    floatx4_t accH[HT][4], accW2[4][4], accW1[4][4];
    float gbh[HT][4], gb2[4][4], gb1[4][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            accH[ht][t] = floatx4_t{0, 0, 0, 0};
            gbh[ht][t] = 0.0f;
        }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            accW2[r][t] = accW1[r][t] = floatx4_t{0, 0, 0, 0};
            gb2[r][t] = gb1[r][t] = 0.0f;
        }

    float* sG = sT[wv][0];
    float* sH = sT[wv][1];
    const int64_t n = *a.count;
    for (int64_t base = wave * 16; base < n; base += nwaves * 16) {
        const int64_t kc = base + c;
        const bool valid = kc < n;
        const int64_t gi = a.list[valid ? kc : n - 1];
        // ---------------- forward (as mlp_branch_kernel computes it)
        half8_t Z[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
            Z[m] = cat8(unpack4(a.z[(size_t)(8 * m + q) * a.zstride + gi]),
                        unpack4(a.z[(size_t)(8 * m + 4 + q) * a.zstride + gi]));
        floatx4_t P1[4], P2[4];
        half8_t H1[2], H2[2];
#pragma unroll
        for (int mo = 0; mo < 2; ++mo) {
            floatx4_t lo = B1[2 * mo], hi = B1[2 * mo + 1];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[2 * mo][m], Z[m], lo, 0, 0, 0);
                hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[2 * mo + 1][m], Z[m], hi, 0, 0, 0);
            }
            half8_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float d0, d1;
                h[e] = (_Float16)act_fwd_grad<GELU>(lo[e], d0);
                h[4 + e] = (_Float16)act_fwd_grad<GELU>(hi[e], d1);
                P1[2 * mo][e] = d0;
                P1[2 * mo + 1][e] = d1;
            }
            H1[mo] = h;
        }
#pragma unroll
        for (int mo = 0; mo < 2; ++mo) {
            floatx4_t lo = B2[2 * mo], hi = B2[2 * mo + 1];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2[2 * mo][m], H1[m], lo, 0, 0, 0);
                hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2[2 * mo + 1][m], H1[m], hi, 0, 0, 0);
            }
            half8_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float d0, d1;
                h[e] = (_Float16)act_fwd_grad<GELU>(lo[e], d0);
                h[4 + e] = (_Float16)act_fwd_grad<GELU>(hi[e], d1);
                P2[2 * mo][e] = d0;
                P2[2 * mo + 1][e] = d1;
            }
            H2[mo] = h;
        }
        float o[HT][4];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            floatx4_t acc = B3[ht];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3[ht][0], H2[0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3[ht][1], H2[1], acc, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[ht][e] = acc[e];
        }
        // ---------------- Eq. 11 backward of this branch's rows r = 16 ht + 4 q + e
        float go[HT][4];
        const int64_t u = a.off + gi;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * ht + 4 * q + e;
                go[ht][e] = valid && r < OUT ? a.gup[u * OUT + r] : 0.0f;
            }
        if constexpr (BR == 0) {  // scale: exp below the clip
#pragma unroll
            for (int e = 0; e < 4; ++e) go[0][e] = o[0][e] < 20.0f ? go[0][e] * expf(o[0][e]) : 0.0f;
        } else if constexpr (BR == 1) {  // rotation: rows 0-3 all in lane group q = 0
            const float rn = sqrtf(o[0][0] * o[0][0] + (o[0][1] * o[0][1] + o[0][2] * o[0][2] + o[0][3] * o[0][3]));
            const float nrm = fmaxf(rn, 1e-12f);
            float dot = 0.0f;
            if (rn >= 1e-12f)
#pragma unroll
                for (int e = 0; e < 4; ++e) dot += go[0][e] * (o[0][e] / nrm);
#pragma unroll
            for (int e = 0; e < 4; ++e) go[0][e] = (go[0][e] - dot * (o[0][e] / nrm)) / nrm;
        } else if constexpr (BR == 3 || (BR == 2 && !SH)) {  // sigmoid
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sg = sigmoid_f(o[0][e]);
                go[0][e] = go[0][e] * sg * (1.0f - sg);
            }
        }  // SH coefficients: the head outputs themselves
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (16 * ht + 4 * q + e >= OUT) go[ht][e] = 0.0f;
                gbh[ht][e] += go[ht][e];
            }
        // ---------------- head: dWh += go H2^T
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) sG[(16 * ht + 4 * q + e) * kTS + c] = go[ht][e];
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
            float bh[4];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) bh[hb] = sH[(16 * hb + c) * kTS + 4 * s + q];
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const float ag = sG[(16 * ht + c) * kTS + 4 * s + q];
#pragma unroll
                for (int hb = 0; hb < 4; ++hb) accH[ht][hb] = mfma4(ag, bh[hb], accH[ht][hb]);
            }
        }
        wave_lds_sync();
        floatx4_t D[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            D[rb] = floatx4_t{0, 0, 0, 0};
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int e = 0; e < 4; ++e) D[rb] = mfma4(sWh[((ht * 4 + rb) * 4 + e) * 64 + lane], go[ht][e], D[rb]);
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
        // ---------------- layer 1: dW1 += da1 z^T (64 inputs: four 16-wide k tiles)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) sG[(16 * rb + 4 * q + e) * kTS + c] = E[rb][e];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sH[(32 * m + 4 * q + e) * kTS + c] = (float)Z[m][e];
                sH[(32 * m + 16 + 4 * q + e) * kTS + c] = (float)Z[m][4 + e];
            }
        wave_lds_sync();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float bz[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) bz[kb] = sH[(16 * kb + c) * kTS + 4 * s + q];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const float ag = sG[(16 * rb + c) * kTS + 4 * s + q];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) accW1[rb][kb] = mfma4(ag, bz[kb], accW1[rb][kb]);
            }
        }
        wave_lds_sync();
        // dz = W1^T da1, added into this level's four features
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) {
            floatx4_t G = {0, 0, 0, 0};
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int e = 0; e < 4; ++e) G = mfma4(sW1[((ob * 4 + rb) * 4 + e) * 64 + lane], E[rb][e], G);
            if (valid) {
                float4* dst = a.gz + (size_t)(4 * ob + q) * a.gzstride + kc;
                float4 v = make_float4(G[0], G[1], G[2], G[3]);
                if (BR > 0) {
                    const float4 w = *dst;
                    v = make_float4(w.x + v.x, w.y + v.y, w.z + v.z, w.w + v.w);
                }
                *dst = v;
            }
        }
    }
    {
        int j = 0;
#pragma unroll
        for (int t = 0; t < 4 * HT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = accH[t >> 2][t & 3][e];
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = accW2[t >> 2][t & 3][e];
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = accW1[t >> 2][t & 3][e];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[64 * j++] = gbh[ht][e];
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

// As mlp_bwd_reduce_kernel for one branch (64 inputs, HT head tiles of which
// OUT rows are real); add != 0 adds into the outputs (later chunks) instead of
// overwriting them.
template <int HT, int OUT>
__global__ void __launch_bounds__(256) branch_bwd_reduce_kernel(const float* partial, int nwaves, float* gW1,
                                                                float* gW2, float* gWh, float* gb1, float* gb2,
                                                                float* gbh, int add) {
    constexpr int kT = branch_tile_slots<HT>(), kB = branch_bias_slots<HT>();
    const int t = blockIdx.x * 256 + threadIdx.x;
    const int stride = kDecodeBwdSlotFloats;
    float* dst = nullptr;
    float s = 0.0f;
    if (t < kT * 64) {
        const int j = t >> 6, lane = t & 63, q = lane >> 4, c = lane & 15, e = j & 3, tile = j >> 2;
        for (int w = 0; w < nwaves; ++w) s += partial[(size_t)w * stride + t];
        if (tile < 4 * HT) {
            const int row = 16 * (tile >> 2) + 4 * q + e;
            if (row < OUT) dst = gWh + row * 64 + 16 * (tile & 3) + c;
        } else if (tile < 4 * HT + 16) {
            const int rb = (tile - 4 * HT) >> 2, hb = (tile - 4 * HT) & 3;
            dst = gW2 + (16 * rb + 4 * q + e) * 64 + 16 * hb + c;
        } else {
            const int rb = (tile - 4 * HT - 16) >> 2, kb = (tile - 4 * HT - 16) & 3;
            dst = gW1 + (16 * rb + 4 * q + e) * 64 + 16 * kb + c;
        }
    } else {
        const int u = t - kT * 64;
        if (u >= kB * 4) return;
        const int jb = u >> 2, q = u & 3;
        for (int w = 0; w < nwaves; ++w)
            for (int c = 0; c < 16; ++c) s += partial[(size_t)w * stride + (kT + jb) * 64 + 16 * q + c];
        if (jb < 4 * HT) {
            const int row = 16 * (jb >> 2) + 4 * q + (jb & 3);
            if (row < OUT) dst = gbh + row;
        } else if (jb < 4 * HT + 16) {
            const int rb = (jb - 4 * HT) >> 2, e = (jb - 4 * HT) & 3;
            dst = gb2 + 16 * rb + 4 * q + e;
        } else {
            const int rb = (jb - 4 * HT - 16) >> 2, e = (jb - 4 * HT - 16) & 3;
            dst = gb1 + 16 * rb + 4 * q + e;
        }
    }
    if (dst) *dst = add ? *dst + s : s;
}

// First stage of the partial sums: block (slot j, group g) adds the slot of
// waves [g W, (g + 1) W), W = waves / groups, in wave order, lane by lane.
__global__ void __launch_bounds__(64) mlp_bwd_group_kernel(const float* partial, int waves_per_group,
                                                           float* group_sums) {
    const int stride = kDecodeBwdSlotFloats;
    const int j = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
    const float* src = partial + (size_t)g * waves_per_group * stride + j * 64 + lane;
    float s = 0.0f;
    for (int w = 0; w < waves_per_group; ++w) s += src[(size_t)w * stride];
    group_sums[(size_t)g * stride + j * 64 + lane] = s;
}

// Sum the per-wave (or per-group) partials in order.  Thread t < tile_slots * 64
// owns one (slot, lane) of the weight tiles; the next bias_slots * 4 threads own
// one bias slot of one lane group q (summed over its 16 lanes c).
template <int HT>
__global__ void __launch_bounds__(256) mlp_bwd_reduce_kernel(const float* partial, int nwaves, float* gW1,
                                                             float* gW2, float* gWh, float* gb1, float* gb2,
                                                             float* gbh) {
    constexpr int kT = tile_slots<HT>(), kB = bias_slots<HT>(), HEAD = head_rows<HT>();
    const int t = blockIdx.x * 256 + threadIdx.x;
    const int stride = kDecodeBwdSlotFloats;
    if (t < kT * 64) {
        const int j = t >> 6, lane = t & 63, q = lane >> 4, c = lane & 15, e = j & 3, tile = j >> 2;
        float s = 0.0f;
        for (int w = 0; w < nwaves; ++w) s += partial[(size_t)w * stride + t];
        if (tile < 4 * HT) {
            const int ht = tile >> 2, hb = tile & 3;
            const int row = 16 * ht + 4 * q + e;
            if (row < HEAD) gWh[row * 64 + 16 * hb + c] = s;
        } else if (tile < 4 * HT + 16) {
            const int rb = (tile - 4 * HT) >> 2, hb = (tile - 4 * HT) & 3;
            gW2[(16 * rb + 4 * q + e) * 64 + 16 * hb + c] = s;
        } else {
            const int rb = (tile - 4 * HT - 16) >> 1, kb = (tile - 4 * HT - 16) & 1;
            gW1[(16 * rb + 4 * q + e) * 32 + 16 * kb + c] = s;
        }
        return;
    }
    const int u = t - kT * 64;
    if (u >= kB * 4) return;
    const int jb = u >> 2, q = u & 3;
    float s = 0.0f;
    for (int w = 0; w < nwaves; ++w)
        for (int c = 0; c < 16; ++c) s += partial[(size_t)w * stride + (kT + jb) * 64 + 16 * q + c];
    if (jb < 4 * HT) {
        const int row = 16 * (jb >> 2) + 4 * q + (jb & 3);
        if (row < HEAD) gbh[row] = s;
    } else if (jb < 4 * HT + 16) {
        const int rb = (jb - 4 * HT) >> 2, e = (jb - 4 * HT) & 3;
        gb2[16 * rb + 4 * q + e] = s;
    } else {
        const int rb = (jb - 4 * HT - 16) >> 2, e = (jb - 4 * HT - 16) & 3;
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
constexpr int kAggMaxRes = 300;  // with the finer levels in buckets: 640 and 200 measured slower
// rounds of 64 Gaussians per combining block: 384 Gaussians share one
// 2048-slot LDS table (24 KiB, six blocks per CU); 768 Gaussians on 4096
// slots, 512 or 768 on 2048, and 192 on 1024 measured slower
constexpr int kAggRounds = 6;

// F features per entry: feature f of slot k at v[f * kAggSlots + k].
template <int F>
__device__ __forceinline__ void agg_add(uint32_t* key, float* v, uint32_t idx, const float (&a)[F], float* gt) {
    uint32_t slot = (idx * 2654435761u) >> (32 - kAggBits);
    for (int p = 0; p < kAggProbes; ++p) {
        // a set key never changes: a plain read settles most probes, the
        // compare-and-swap only claims an empty slot
        uint32_t old = key[slot];
        if (old == kAggEmpty) old = atomicCAS(&key[slot], kAggEmpty, idx);
        if (old == kAggEmpty || old == idx) {
#pragma unroll
            for (int f = 0; f < F; ++f) atomicAdd(&v[f * kAggSlots + slot], a[f]);
            return;
        }
        slot = (slot + 1) & (kAggSlots - 1);
    }
#pragma unroll
    for (int f = 0; f < F; ++f) atomicAdd(gt + F * (size_t)idx + f, a[f]);
}

// Eq. 9 and Eq. 7 backward of one (Gaussian, level) for lane s of its group
// of four: the lane takes the x/y corner (s & 1, s >> 1) and its four z/t
// corners; emit(idx, w) receives each corner of non-zero weight w (its
// contribution to table entry idx is w g[f] per feature f).  POS: this
// level's share of the position gradient, stored by lane 0 of the group.
// k is the Gaussian's compact index (its upstream gradient row), i its
// chunk-local index.
template <int F, bool POS, class Emit>
__device__ __forceinline__ void scatter_one(const float4 p, const float* pos, int stride, int64_t i, int64_t k,
                                            int level, const HashLevels& h, const uint32_t* tab, const float (&g)[F],
                                            int64_t zstride, float4* gpos_part, int s, Emit&& emit) {
#pragma clang fp contract(fast)
    const int res = h.res_s[level], res_t = h.res_t[level];
    const bool dense = h.dense[level] != 0;
    const int bx = s & 1, by = s >> 1;
    const uint32_t r = (uint32_t)res, r2 = r * r, r3 = r2 * r;
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
    bool none = true;
#pragma unroll
    for (int f = 0; f < F; ++f) none = none && g[f] == 0.0f;
    if (none) {
        if (POS && s == 0) gpos_part[(size_t)level * zstride + k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        return;
    }
    float dx = 0.0f, dy = 0.0f, dz = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int bz = c & 1, bt = c >> 1;
        // a corner of zero time weight has zero weight and zero spatial derivatives
        if (wt[bt] == 0.0f) continue;
        const uint32_t idx = (dense ? (txy + tz[bz] + tt[bt]) : (txy ^ tz[bz] ^ tt[bt])) & h.mask;
        const float w = (wxy * wz[bz]) * wt[bt];
        if (w != 0.0f) emit(idx, w);
        if (POS) {
            // the entry's features times the level's gradient
            float tg = 0.0f;
#pragma unroll
            for (int f = 0; f < F; f += 2) {
                const uint32_t raw = tab[(F / 2) * (size_t)idx + f / 2];
                const float v0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw & 0xffffu));
                const float v1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw >> 16));
                tg += v0 * g[f] + v1 * g[f + 1];
            }
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

// The upstream gradient of Gaussian k (compact index) at a level.
template <int F>
__device__ __forceinline__ void level_grad(const float* gz, int64_t zstride, int level, int64_t k, float (&g)[F]) {
    if constexpr (F == 2) {
        const float2 v = reinterpret_cast<const float2*>(gz)[(size_t)level * zstride + k];
        g[0] = v.x;
        g[1] = v.y;
    } else {
        const float4 v = reinterpret_cast<const float4*>(gz)[(size_t)level * zstride + k];
        g[0] = v.x;
        g[1] = v.y;
        g[2] = v.z;
        g[3] = v.w;
    }
}

// The coarse levels (at most kAggMaxRes vertices per axis), level-major as the
// gather, levels level0 + 0, 1, ...: each block adds its contributions per
// table entry in LDS first, then one global atomic per distinct entry and
// feature (every thread of a block reaches the final barrier: the only early
// exit is block-uniform).  F features per table entry (2, or 4 for the
// paper-scale encoder; gz holds F floats per level and Gaussian).
template <int F, bool POS>
__global__ void __launch_bounds__(256) scatter_kernel(const float4* xt, const float* pos, int stride,
                                                      const uint32_t* list, const uint32_t* count, int nchunk,
                                                      int level0, HashLevels h, const uint32_t* tables,
                                                      const float* gz, int64_t zstride, float* gtab,
                                                      float4* gpos_part) {
    static_assert(F == 2 || F == 4, "two or four features per entry");
    __shared__ uint32_t s_key[kAggSlots];
    __shared__ float s_v[F * kAggSlots];
    const int level = level0 + (int)(blockIdx.x / nchunk);
    const int64_t first = (int64_t)(blockIdx.x % nchunk) * (64 * kAggRounds);
    const int64_t n = *count;  // Gaussians with a gradient, compacted
    if (first >= n) return;
    for (int k = threadIdx.x; k < kAggSlots; k += 256) s_key[k] = kAggEmpty;
    for (int k = threadIdx.x; k < F * kAggSlots; k += 256) s_v[k] = 0.0f;
    __syncthreads();
    const uint32_t* tab = tables + (size_t)level * h.T * (F / 2);
    float* gt = gtab + (size_t)level * h.T * F;
    const int s = threadIdx.x & 3, sub = threadIdx.x >> 2;
    for (int j = 0; j < kAggRounds; ++j) {
        const int64_t k = first + j * 64 + sub;  // compact index
        if (k >= n) break;  // uniform across each group of four lanes
        const int64_t i = list[k];  // chunk-local Gaussian
        float g[F];
        level_grad<F>(gz, zstride, level, k, g);
        scatter_one<F, POS>(xt[i], pos, stride, i, k, level, h, tab, g, zstride, gpos_part, s,
                            [&](uint32_t idx, float w) {
                                float wg[F];
#pragma unroll
                                for (int f = 0; f < F; ++f) wg[f] = w * g[f];
                                agg_add<F>(s_key, s_v, idx, wg, gt);
                            });
    }
    __syncthreads();
    for (int k = threadIdx.x; k < kAggSlots; k += 256) {
        const uint32_t idx = s_key[k];
        if (idx != kAggEmpty)
#pragma unroll
            for (int f = 0; f < F; ++f) atomicAdd(gt + F * (size_t)idx + f, s_v[f * kAggSlots + k]);
    }
}

// The fine levels, where a block's Gaussians rarely share a corner, without
// global float atomics (served far below L2 speed on this chip): the table is
// cut into buckets of 2^shift entries, and the contributions to a level go
// as (entry, w g) records (1 + F consecutive words) into per-bucket runs of
// the record buffer, each
// then summed in LDS by one block of bucket_add_kernel.  One launch of each
// kernel covers a group of fine levels (all of them when their buckets fit
// kBktGroupBytes), each level with buckets of its own.
//   bucket_scatter_kernel (kBktRounds x 64 Gaussians of one level per block,
//     their inputs loaded once for both passes):
//     pass 1 counts the block's records per bucket in LDS; one global atomic
//     per bucket then reserves their places in the bucket's run; pass 2
//     recomputes the same records (the same arithmetic, so the same set) and
//     writes each at its bucket's reserved start plus its rank from an LDS
//     counter.  A record past the run's capacity is added to the table with
//     global float atomics instead (correct, slower; a run holds 5/4 of its
//     share of 16 corners per Gaussian, so only a skewed table needs it).
//     With few Gaussians with a gradient (kBktSparse) every contribution is
//     a direct float atomic and no bucket is used.
//   bucket_add_kernel (one block per bucket and level): adds the bucket's
//     records into an LDS copy of its 2^shift entries, then adds that copy to
//     the table's gradient (one owner per entry: plain read-modify-writes)
//     and clears the bucket's count for the next group.
constexpr int kBktRounds = 8;  // rounds of 64 Gaussians per scatter block: 512 Gaussians
constexpr int kBktMaxBuckets = 4096;
constexpr int kBktMaxEntries = 4096;

// Entries per bucket (log2) for a table of 2^log2T entries: 2^11, whole
// tables below that, and at most kBktMaxBuckets buckets.
int bucket_shift(uint32_t T) {
    int lg = 0;
    while ((1u << lg) < T) ++lg;
    int sh = lg < 11 ? lg : 11;
    if (lg - sh > 12) sh = lg - 12;
    return sh;
}

// Records per bucket run for a chunk of `chunk` Gaussians.
int64_t bucket_cap(uint32_t T, int64_t chunk) {
    const int64_t nb = (int64_t)(T >> bucket_shift(T));
    return (16 * chunk + nb - 1) / nb * 5 / 4 + 256;
}

// Bytes of one fine level's buckets (counts, entries, values) for a chunk.
size_t bucket_level_bytes(uint32_t T, int F, int64_t chunk) {
    const size_t nb = (size_t)(T >> bucket_shift(T));
    return nb * 4 + nb * (size_t)bucket_cap(T, chunk) * (size_t)(1 + F) * 4;
}

// Fine levels per bucket launch: all of them, or as many as fit
// kBktGroupBytes (at least one).
constexpr size_t kBktGroupBytes = (size_t)2 << 30;
int bucket_group_levels(const HashLevels& h, int64_t chunk) {
    int nagg = 0;
    while (nagg < h.L && h.res_s[nagg] <= kAggMaxRes) ++nagg;
    const int nfine = h.L - nagg;
    if (nfine <= 0) return 1;
    const size_t per = bucket_level_bytes(h.T, h.F, chunk);
    int g = (int)(kBktGroupBytes / per);
    if (g < 1) g = 1;
    return g < nfine ? g : nfine;
}

struct BucketArgs {
    uint32_t* count;  // [levels][nb] records per bucket (zero between groups)
    uint32_t* rec;    // [levels][nb][cap] records of 1 + F words: entry within the bucket, w g[f] (fp32 bits)
    int64_t cap;
    int shift;
    int nb;
};

// A chunk with at most kBktSparse Gaussians with a gradient adds its few
// fine-level contributions with direct float atomics (the buckets would cost
// more than they save); bucket_add_kernel then finds every bucket empty.
constexpr int64_t kBktSparse = 65536;

// One launch covers a group of consecutive fine levels level0 ... (block b:
// level level0 + b / nblk), each with its own buckets.
template <int F, bool POS>
__global__ void __launch_bounds__(256) bucket_scatter_kernel(const float4* xt, const float* pos, int stride,
                                                             const uint32_t* list, const uint32_t* count, int nblk,
                                                             int level0, HashLevels h, const uint32_t* tables,
                                                             const float* gz, int64_t zstride, float* gtab,
                                                             float4* gpos_part, BucketArgs bk) {
    static_assert(F == 2 || F == 4, "two or four features per entry");
    __shared__ uint32_t s_cnt[kBktMaxBuckets];
    __shared__ uint32_t s_base[kBktMaxBuckets];
    const int lg = (int)(blockIdx.x / nblk);  // level within the group
    const int level = level0 + lg;
    const int64_t first = (int64_t)(blockIdx.x % nblk) * (64 * kBktRounds);
    const int64_t n = *count;  // Gaussians with a gradient, compacted
    const uint32_t* tab = tables + (size_t)level * h.T * (F / 2);
    float* gt = gtab + (size_t)level * h.T * F;
    const int s = threadIdx.x & 3, sub = threadIdx.x >> 2;
    if (n <= kBktSparse) {
        // few Gaussians: direct atomics, one round of 64 at a time, spread
        // over all the level's blocks (no barrier on this path)
        for (int64_t r = blockIdx.x % nblk; r * 64 < n; r += nblk) {
            const int64_t k = r * 64 + sub;
            if (k >= n) break;
            const int64_t i = list[k];
            float g[F];
            level_grad<F>(gz, zstride, level, k, g);
            scatter_one<F, POS>(xt[i], pos, stride, i, k, level, h, tab, g, zstride, gpos_part, s,
                                [&](uint32_t idx, float w) {
#pragma unroll
                                    for (int f = 0; f < F; ++f) atomicAdd(gt + F * (size_t)idx + f, w * g[f]);
                                });
        }
        return;
    }
    if (first >= n) return;  // block-uniform
    for (int b = threadIdx.x; b < bk.nb; b += 256) s_cnt[b] = 0u;
    uint32_t* bcount = bk.count + (size_t)lg * bk.nb;
    uint32_t* brec = bk.rec + (size_t)lg * bk.nb * bk.cap * (1 + F);
    // the inputs of every round, loaded once (all in flight together) for both passes
    uint32_t gi[kBktRounds];
    float4 gp[kBktRounds];
    float gg[kBktRounds][F];
#pragma unroll
    for (int j = 0; j < kBktRounds; ++j) {
        int64_t k = first + j * 64 + sub;
        if (k >= n) k = n - 1;  // a clamped round is skipped below
        gi[j] = list[k];
    }
#pragma unroll
    for (int j = 0; j < kBktRounds; ++j) {
        const int64_t k = first + j * 64 + sub < n ? first + j * 64 + sub : n - 1;
        gp[j] = xt[gi[j]];
        level_grad<F>(gz, zstride, level, k, gg[j]);
    }
    __syncthreads();
    // pass 1: records per bucket
#pragma unroll
    for (int j = 0; j < kBktRounds; ++j) {
        const int64_t k = first + j * 64 + sub;
        if (k < n)  // uniform across each group of four lanes
            scatter_one<F, false>(gp[j], pos, stride, gi[j], k, level, h, tab, gg[j], zstride, gpos_part, s,
                                  [&](uint32_t idx, float) { atomicAdd(&s_cnt[idx >> bk.shift], 1u); });
    }
    __syncthreads();
    for (int b = threadIdx.x; b < bk.nb; b += 256) {
        const uint32_t c = s_cnt[b];
        s_base[b] = c ? atomicAdd(&bcount[b], c) : 0u;
        s_cnt[b] = 0u;
    }
    __syncthreads();
    // pass 2: the same records, each at its reserved place
#pragma unroll
    for (int j = 0; j < kBktRounds; ++j) {
        const int64_t k = first + j * 64 + sub;
        if (k < n)
            scatter_one<F, POS>(gp[j], pos, stride, gi[j], k, level, h, tab, gg[j], zstride, gpos_part, s,
                                [&](uint32_t idx, float w) {
                                    const uint32_t b = idx >> bk.shift;
                                    const uint64_t at = (uint64_t)s_base[b] + atomicAdd(&s_cnt[b], 1u);
                                    if (at < (uint64_t)bk.cap) {
                                        // one record: consecutive words, written together
                                        uint32_t* rp = brec + ((size_t)b * bk.cap + at) * (1 + F);
                                        rp[0] = idx & ((1u << bk.shift) - 1u);
#pragma unroll
                                        for (int f = 0; f < F; ++f) rp[1 + f] = __float_as_uint(w * gg[j][f]);
                                    } else {
#pragma unroll
                                        for (int f = 0; f < F; ++f) atomicAdd(gt + F * (size_t)idx + f, w * gg[j][f]);
                                    }
                                });
    }
}

// kBktAddThreads threads per bucket, kBktAddPer records per thread and step,
// loaded before any is added.  Block b: bucket b % nb of level level0 + b / nb.
constexpr int kBktAddThreads = 1024;
constexpr int kBktAddPer = 8;

template <int F>
__global__ void __launch_bounds__(kBktAddThreads) bucket_add_kernel(int level0, uint32_t T, float* gtab, BucketArgs bk) {
    __shared__ float s_acc[F * kBktMaxEntries];
    const int lg = (int)(blockIdx.x / bk.nb), b = (int)(blockIdx.x % bk.nb);
    uint32_t* cnt = bk.count + (size_t)lg * bk.nb + b;
    uint64_t c = *cnt;
    if (c == 0) return;  // nothing to add (block-uniform; the count stays zero)
    if (c > (uint64_t)bk.cap) c = (uint64_t)bk.cap;  // the rest went to the table directly
    const int E = 1 << bk.shift;  // entries per bucket
    for (int e = threadIdx.x; e < F * E; e += kBktAddThreads) s_acc[e] = 0.0f;
    __syncthreads();
    const uint32_t* rb = bk.rec + ((size_t)lg * bk.nb + b) * bk.cap * (1 + F);
    for (uint64_t r0 = 0; r0 < c; r0 += kBktAddThreads * kBktAddPer) {
        uint32_t e[kBktAddPer];
        float v[kBktAddPer][F];
#pragma unroll
        for (int u = 0; u < kBktAddPer; ++u) {
            uint64_t r = r0 + (uint64_t)u * kBktAddThreads + threadIdx.x;
            if (r >= c) r = c - 1;  // re-reads the last record, not added
            const uint32_t* rp = rb + r * (1 + F);
            e[u] = rp[0];
#pragma unroll
            for (int f = 0; f < F; ++f) v[u][f] = __uint_as_float(rp[1 + f]);
        }
#pragma unroll
        for (int u = 0; u < kBktAddPer; ++u)
            if (r0 + (uint64_t)u * kBktAddThreads + threadIdx.x < c)
#pragma unroll
                for (int f = 0; f < F; ++f) atomicAdd(&s_acc[f * E + e[u]], v[u][f]);
    }
    __syncthreads();
    float* gt = gtab + ((size_t)(level0 + lg) * T + (size_t)b * E) * F;
    for (int e = threadIdx.x; e < E; e += kBktAddThreads)
#pragma unroll
        for (int f = 0; f < F; ++f) gt[(size_t)e * F + f] += s_acc[f * E + e];
    if (threadIdx.x == 0) *cnt = 0u;  // every thread read the count before the first barrier
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

// ncol: colour values per Gaussian (3 RGB, or the 48 SH coefficients)
__device__ __forceinline__ bool has_gradient(const float* gs, const float* gq, const float* gc, const float* go,
                                             int ncol, int64_t u) {
    // every value is loaded (no short circuit, so the loads overlap); a
    // value counts unless it is +0 or -0 (NaN counts)
    uint32_t bits = __float_as_uint(go[u]);
#pragma unroll
    for (int k = 0; k < 3; ++k) bits |= __float_as_uint(gs[u * 3 + k]);
#pragma unroll
    for (int k = 0; k < 4; ++k) bits |= __float_as_uint(gq[u * 4 + k]);
    for (int k = 0; k < ncol; ++k) bits |= __float_as_uint(gc[u * ncol + k]);
    return (bits & 0x7fffffffu) != 0u;
}

__global__ void __launch_bounds__(256) active_count_kernel(const float* gs, const float* gq, const float* gc,
                                                           const float* go, int ncol, int64_t off, int64_t n,
                                                           uint32_t* bcount) {
    __shared__ uint32_t s_cnt[4];
    const int64_t b0 = (int64_t)blockIdx.x * kCompactItems;
    uint32_t cnt = 0;
    for (int r = 0; r < kCompactItems / 256; ++r) {
        const int64_t i = b0 + r * 256 + threadIdx.x;
        if (i < n && has_gradient(gs, gq, gc, go, ncol, off + i)) ++cnt;
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
                                                           const float* go, int ncol, int64_t off, int64_t n,
                                                           const uint32_t* boff, const float4* xt,
                                                           uint64_t* items) {
    __shared__ uint32_t s_w[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t b0 = (int64_t)blockIdx.x * kCompactItems;
    uint32_t pos = boff[blockIdx.x];
    for (int r = 0; r < kCompactItems / 256; ++r) {
        const int64_t i = b0 + r * 256 + threadIdx.x;
        const bool f = i < n && has_gradient(gs, gq, gc, go, ncol, off + i);
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

// the sort scratch: two buffers of `chunk` words, the radix counts, the
// digit totals and the item count
struct SortScratch {
    uint64_t* items[2];
    uint32_t* counts;
    uint32_t* digit_tot;
    uint64_t* count;
    int max_blocks;
};

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t sort_scratch_bytes(int64_t chunk) {
    return 2 * align256(chunk * sizeof(uint64_t)) + align256(radix_sort_counts_bytes(radix_sort_blocks(chunk))) +
           align256(4 * 1024) + 256;
}

SortScratch sort_scratch(void* base, int64_t chunk) {
    SortScratch t{};
    char* p = static_cast<char*>(base);
    t.max_blocks = radix_sort_blocks(chunk);
    t.items[0] = reinterpret_cast<uint64_t*>(p);
    p += align256(chunk * sizeof(uint64_t));
    t.items[1] = reinterpret_cast<uint64_t*>(p);
    p += align256(chunk * sizeof(uint64_t));
    t.counts = reinterpret_cast<uint32_t*>(p);
    p += align256(radix_sort_counts_bytes(t.max_blocks));
    t.digit_tot = reinterpret_cast<uint32_t*>(p);
    p += align256(4 * 1024);
    t.count = reinterpret_cast<uint64_t*>(p);
    return t;
}

// One branch: the fixed-order sum of its partials into its weight and bias
// gradients (added after the first chunk).
template <int BR, bool SH>
hipError_t reduce_branch(const DecodeBwdArgs& b, const float* partial, bool add, hipStream_t s) {
    constexpr int HT = branch_head_tiles(BR, SH), OUT = branch_out(BR, SH);
    constexpr int kSlots = branch_tile_slots<HT>() + branch_bias_slots<HT>();
    const int nwaves = kDecodeBwdBlocks * kBwdWaves;
    float* groups = const_cast<float*>(partial) + (size_t)nwaves * kDecodeBwdSlotFloats;
    IA_LAUNCH("mlp_bwd_group_kernel", mlp_bwd_group_kernel, dim3(kSlots, kDecodeBwdGroups), dim3(64), 0, s, partial,
              nwaves / kDecodeBwdGroups, groups);
    const int nred = branch_tile_slots<HT>() * 64 + branch_bias_slots<HT>() * 4;
    const int k = 3 * BR;
    IA_LAUNCH("branch_bwd_reduce_kernel", (branch_bwd_reduce_kernel<HT, OUT>), dim3((nred + 255) / 256), dim3(256),
              0, s, groups, kDecodeBwdGroups, b.g_W[k], b.g_W[k + 1], b.g_W[k + 2], b.g_b[k], b.g_b[k + 1],
              b.g_b[k + 2], add ? 1 : 0);
    return hipGetLastError();
}

template <bool SH>
hipError_t reduce_branches_t(const DecodeBwdArgs& b, const float* partial, bool add, hipStream_t s) {
    hipError_t e = reduce_branch<0, SH>(b, partial, add, s);
    if (e == hipSuccess) e = reduce_branch<1, SH>(b, partial, add, s);
    if (e == hipSuccess) e = reduce_branch<2, SH>(b, partial, add, s);
    if (e == hipSuccess) e = reduce_branch<3, SH>(b, partial, add, s);
    return e;
}

hipError_t reduce_branches(const DecodeBwdArgs& b, const float* partial, bool add, hipStream_t s) {
    return b.fwd.sh_head ? reduce_branches_t<true>(b, partial, add, s) : reduce_branches_t<false>(b, partial, add, s);
}

// Branch BR over a chunk's active list, then its reduction (each branch
// starts from zeroed partials: the kernel overwrites every slot).
template <int BR, bool SH>
hipError_t branch_bwd(const DecodeBwdArgs& b, BranchBwdArgs ba, float* partial, bool add, hipStream_t s) {
    const int k = 3 * BR;
    for (int l = 0; l < 3; ++l) {
        ba.W[l] = b.Wbr[k + l];
        ba.b[l] = b.bbr[k + l];
    }
    ba.gup = BR == 0 ? b.g_scales : (BR == 1 ? b.g_quats : (BR == 2 ? b.g_colors : b.g_opacity));
    ba.partial = partial;
    const bool gelu = b.fwd.act == IA_ACT_GELU;
    auto kernel = gelu ? mlp_bwd_branch_kernel<true, BR, SH> : mlp_bwd_branch_kernel<false, BR, SH>;
    IA_LAUNCH("mlp_bwd_branch_kernel", kernel, dim3(kDecodeBwdBlocks), dim3(kBwdThreads), 0, s, ba);
    return reduce_branch<BR, SH>(b, partial, add, s);
}

template <bool SH>
hipError_t branches_bwd_t(const DecodeBwdArgs& b, const BranchBwdArgs& ba, float* partial, bool add, hipStream_t s) {
    hipError_t e = branch_bwd<0, SH>(b, ba, partial, add, s);
    if (e == hipSuccess) e = branch_bwd<1, SH>(b, ba, partial, add, s);
    if (e == hipSuccess) e = branch_bwd<2, SH>(b, ba, partial, add, s);
    if (e == hipSuccess) e = branch_bwd<3, SH>(b, ba, partial, add, s);
    return e;
}

// The four branches of one chunk: their input gradients accumulate in gz
// (branch 0 first), their weight gradients are reduced per branch.
hipError_t launch_branches_bwd(const DecodeBwdArgs& b, const uint2* z, int64_t zstride, const uint32_t* list,
                               const uint32_t* count, int64_t off, float4* gz, int64_t gzstride, float* partial,
                               bool add, hipStream_t s) {
    BranchBwdArgs ba{};
    ba.z = z;
    ba.zstride = zstride;
    ba.list = list;
    ba.count = count;
    ba.off = off;
    ba.gz = gz;
    ba.gzstride = gzstride;
    return b.fwd.sh_head ? branches_bwd_t<true>(b, ba, partial, add, s) : branches_bwd_t<false>(b, ba, partial, add, s);
}

}  // namespace

DecodeBwdLayout decode_bwd_layout(const HashLevels& h, int64_t N) {
    DecodeBwdLayout L{};
    const int64_t n = N > 0 ? N : 1;
    // a multiple of the compaction's block size, at most kBwdChunk
    int64_t chunk = (n + kCompactItems - 1) / kCompactItems * kCompactItems;
    if (chunk > kBwdChunk) chunk = kBwdChunk;
    L.chunk = chunk;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    L.z = take((size_t)h.L * chunk * 2 * h.F);              // F fp16 per level
    L.gz = take((size_t)h.L * chunk * sizeof(float) * h.F);  // F fp32 per level
    L.list = take((size_t)chunk * 4);
    L.boff = take((size_t)(chunk / kCompactItems) * 4);
    L.count = take(16);
    L.xt = take((size_t)chunk * sizeof(float4));
    L.partial = take((size_t)kDecodeBwdPartialFloats * sizeof(float));
    L.sort = take(sort_scratch_bytes(chunk));
    L.pos = take((size_t)h.L * chunk * sizeof(float4));
    // fine-level buckets of one group of levels, reused group after group
    const int64_t nb = (int64_t)(h.T >> bucket_shift(h.T));
    const size_t G = (size_t)bucket_group_levels(h, chunk);
    L.bcap = bucket_cap(h.T, chunk);
    L.bcount = take(G * nb * 4);
    L.brec = take(G * nb * L.bcap * (1 + h.F) * 4);
    L.total = off;
    return L;
}

hipError_t launch_decode_backward(const DecodeBwdArgs& b, hipStream_t s) {
    const DecodeArgs& a = b.fwd;
    const int F = a.h.F;
    const size_t tab_floats = (size_t)a.h.L * a.h.T * F;
    IA_LAUNCH("decode_bwd_fill_kernel", fill_kernel, dim3(blocks_for((int64_t)tab_floats, 256, 8192)), dim3(256), 0,
              s, b.g_tables, (int64_t)tab_floats, (const float*)nullptr);
    if (b.g_pos && a.N > 0)
        IA_LAUNCH("decode_bwd_fill_kernel", fill_kernel, dim3(blocks_for(a.N * 3, 256, 8192)), dim3(256), 0, s,
                  b.g_pos, a.N * 3, b.g_means);
    const DecodeBwdLayout lay = decode_bwd_layout(a.h, a.N);
    const int64_t chunk = lay.chunk;
    const SortScratch srt = sort_scratch(b.ws + lay.sort, chunk);
    float4* xt = reinterpret_cast<float4*>(b.ws + lay.xt);
    uint32_t* z = reinterpret_cast<uint32_t*>(b.ws + lay.z);
    float* gz = reinterpret_cast<float*>(b.ws + lay.gz);
    // the compacted list of a chunk, per-block offsets and the count
    uint32_t* list = reinterpret_cast<uint32_t*>(b.ws + lay.list);
    uint32_t* boff = reinterpret_cast<uint32_t*>(b.ws + lay.boff);
    uint32_t* count = reinterpret_cast<uint32_t*>(b.ws + lay.count);
    float* partial = reinterpret_cast<float*>(b.ws + lay.partial);
    float4* pos_partial = reinterpret_cast<float4*>(b.ws + lay.pos);
    BucketArgs bk;
    bk.shift = bucket_shift(a.h.T);
    bk.nb = (int)(a.h.T >> bk.shift);
    bk.cap = lay.bcap;
    bk.count = reinterpret_cast<uint32_t*>(b.ws + lay.bcount);
    bk.rec = reinterpret_cast<uint32_t*>(b.ws + lay.brec);
    // the bucket counts start at zero (the workspace arrives uninitialised;
    // bucket_add_kernel leaves them zero after every group)
    const int bgroup = bucket_group_levels(a.h, lay.chunk);
    IA_LAUNCH("decode_bwd_fill_kernel", fill_kernel, dim3(blocks_for((int64_t)bgroup * bk.nb, 256, 8192)), dim3(256),
              0, s, reinterpret_cast<float*>(bk.count), (int64_t)bgroup * bk.nb, (const float*)nullptr);
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
    m.gz = reinterpret_cast<float2*>(gz);
    m.partial = partial;
    const int ncol = a.sh_head ? 48 : 3;
    int first = 1;
    for (int64_t off = 0; off < a.N; off += chunk) {
        const int64_t n = a.N - off < chunk ? a.N - off : chunk;
        // features kept by the forward ([L][N]) or recomputed into the scratch ([L][chunk])
        hipError_t e = launch_decode_features(a, off, n, xt, a.features ? nullptr : z, chunk, s);
        if (e != hipSuccess) return e;
        // F = 2: one word per (level, Gaussian); F = 4: two
        const uint32_t* zc = a.features ? a.features + off * (F / 2) : z;
        const int64_t zstride = a.features ? a.N : chunk;
        m.z = zc;
        m.zstride = zstride;
        const int nb = (int)((n + kCompactItems - 1) / kCompactItems);
        IA_LAUNCH("active_count_kernel", active_count_kernel, dim3(nb), dim3(256), 0, s, b.g_scales, b.g_quats,
                  b.g_colors, b.g_opacity, ncol, off, n, boff);
        IA_LAUNCH("active_scan_kernel", active_scan_kernel, dim3(1), dim3(256), 0, s, boff, nb, count, srt.count);
        IA_LAUNCH("active_write_kernel", active_write_kernel, dim3(nb), dim3(256), 0, s, b.g_scales, b.g_quats,
                  b.g_colors, b.g_opacity, ncol, off, n, boff, xt, srt.items[0]);
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
        if (a.branches) {
            hipError_t be = launch_branches_bwd(b, reinterpret_cast<const uint2*>(zc), zstride, list, count, off,
                                                reinterpret_cast<float4*>(gz), chunk, partial, off > 0, s);
            if (be != hipSuccess) return be;
        } else {
            auto kernel = a.sh_head ? (m.gelu ? mlp_bwd_kernel<true, 4> : mlp_bwd_kernel<false, 4>)
                                    : (m.gelu ? mlp_bwd_kernel<true, 1> : mlp_bwd_kernel<false, 1>);
            IA_LAUNCH("mlp_bwd_kernel", kernel, dim3(kDecodeBwdBlocks), dim3(kBwdThreads), 0, s, m);
        }
        const int nchunk_agg = (int)((n + 64 * kAggRounds - 1) / (64 * kAggRounds));
        const int nblk_bkt = (int)((n + 64 * kBktRounds - 1) / (64 * kBktRounds));
        const float* pos = a.pos + off * a.stride;
        float* gpos = b.g_pos ? b.g_pos + off * 3 : nullptr;
        // levels [0, nagg) combine in LDS first (resolution grows with the level),
        // the finer ones go through the buckets
        int nagg = 0;
        while (nagg < a.h.L && a.h.res_s[nagg] <= kAggMaxRes) ++nagg;
        auto scatter = [&](auto pos_t) {
            constexpr bool P = decltype(pos_t)::value;
            if (nagg > 0) {
                if (F == 4)
                    IA_LAUNCH("scatter_agg_kernel", (scatter_kernel<4, P>), dim3((unsigned)(nagg * nchunk_agg)),
                              dim3(256), 0, s, xt, pos, a.stride, list, count, nchunk_agg, 0, a.h,
                              (const uint32_t*)a.tables, gz, chunk, b.g_tables, pos_partial);
                else
                    IA_LAUNCH("scatter_agg_kernel", (scatter_kernel<2, P>), dim3((unsigned)(nagg * nchunk_agg)),
                              dim3(256), 0, s, xt, pos, a.stride, list, count, nchunk_agg, 0, a.h,
                              (const uint32_t*)a.tables, gz, chunk, b.g_tables, pos_partial);
            }
            for (int level0 = nagg; level0 < a.h.L; level0 += bgroup) {
                const int g = a.h.L - level0 < bgroup ? a.h.L - level0 : bgroup;
                if (F == 4) {
                    IA_LAUNCH("bucket_scatter_kernel", (bucket_scatter_kernel<4, P>), dim3((unsigned)(g * nblk_bkt)),
                              dim3(256), 0, s, xt, pos, a.stride, list, count, nblk_bkt, level0, a.h,
                              (const uint32_t*)a.tables, gz, chunk, b.g_tables, pos_partial, bk);
                    IA_LAUNCH("bucket_add_kernel", bucket_add_kernel<4>, dim3((unsigned)(g * bk.nb)),
                              dim3(kBktAddThreads), 0, s, level0, a.h.T, b.g_tables, bk);
                } else {
                    IA_LAUNCH("bucket_scatter_kernel", (bucket_scatter_kernel<2, P>), dim3((unsigned)(g * nblk_bkt)),
                              dim3(256), 0, s, xt, pos, a.stride, list, count, nblk_bkt, level0, a.h,
                              (const uint32_t*)a.tables, gz, chunk, b.g_tables, pos_partial, bk);
                    IA_LAUNCH("bucket_add_kernel", bucket_add_kernel<2>, dim3((unsigned)(g * bk.nb)),
                              dim3(kBktAddThreads), 0, s, level0, a.h.T, b.g_tables, bk);
                }
            }
        };
        if (b.g_pos) {
            scatter(std::true_type{});
            IA_LAUNCH("pos_reduce_kernel", pos_reduce_kernel, dim3(blocks_for(n, 256, 4096)), dim3(256), 0, s, list,
                      count, a.h.L, (const float4*)pos_partial, chunk, gpos);
        } else {
            scatter(std::false_type{});
        }
    }
    if (first) {  // N = 0: the weight and bias gradients are zero
        const int64_t nf = (int64_t)kDecodeBwdBlocks * kBwdWaves * kDecodeBwdSlotFloats;
        IA_LAUNCH("decode_bwd_fill_kernel", fill_kernel, dim3(blocks_for(nf, 256, 8192)), dim3(256), 0, s, partial,
                  nf, (const float*)nullptr);
        if (a.branches) return reduce_branches(b, partial, false, s);
    }
    if (a.branches) return hipGetLastError();  // reduced after every chunk
    // fixed-order two-stage sum of the per-wave partials (deterministic)
    const int nwaves = kDecodeBwdBlocks * kBwdWaves;
    float* groups = partial + (size_t)nwaves * kDecodeBwdSlotFloats;
    const int slots = a.sh_head ? tile_slots<4>() + bias_slots<4>() : tile_slots<1>() + bias_slots<1>();
    IA_LAUNCH("mlp_bwd_group_kernel", mlp_bwd_group_kernel, dim3(slots, kDecodeBwdGroups), dim3(64), 0, s, partial,
              nwaves / kDecodeBwdGroups, groups);
    if (a.sh_head) {
        const int nred = tile_slots<4>() * 64 + bias_slots<4>() * 4;
        IA_LAUNCH("mlp_bwd_reduce_kernel", mlp_bwd_reduce_kernel<4>, dim3((nred + 255) / 256), dim3(256), 0, s,
                  groups, kDecodeBwdGroups, b.g_W[0], b.g_W[1], b.g_W[2], b.g_b[0], b.g_b[1], b.g_b[2]);
    } else {
        const int nred = tile_slots<1>() * 64 + bias_slots<1>() * 4;
        IA_LAUNCH("mlp_bwd_reduce_kernel", mlp_bwd_reduce_kernel<1>, dim3((nred + 255) / 256), dim3(256), 0, s,
                  groups, kDecodeBwdGroups, b.g_W[0], b.g_W[1], b.g_W[2], b.g_b[0], b.g_b[1], b.g_b[2]);
    }
    return hipGetLastError();
}

}  // namespace ia
