// Backward pass of the tile rasteriser and of the EWA projection ("SPIN-4DGS"
// §3.1, Eq. 1-4; Eq. 2-3 differentiated by hand) for an image-space loss
// gradient dL/dimage, and the L1 image loss itself.
//
//   raster_backward_kernel  one block per tile (one or two pixels per
//       thread).  Each pixel walks its tile's list from the last composited
//       Gaussian (n_contrib) back to the first, re-deciding every step with
//       the forward's arithmetic (raster_common.h) and recovering
//       T_i = T_{i+1} / (1 - alpha_i) from T_final:
//         dL/dc_i     = g alpha_i T_i
//         dL/dalpha_i = g . (c_i T_i - S_i / (1 - alpha_i)),
//                       S_i = sum_{j>i} c_j alpha_j T_j + T_final bg
//         alpha = o exp(power) (constant where clamped at 0.99), power =
//         -0.5 (A dx^2 + C dy^2) - B dx dy, d = pixel centre - mean.
//       Per Gaussian nine partials (power moments gp (dx, dy, dx^2, dx dy,
//       dy^2), opacity, r, g, b) are summed over each quad of lanes with DPP
//       adds, buffered per wave in LDS and summed seven Gaussians at a time
//       (one lane per Gaussian and partial), gathered per block in LDS, turned
//       into d/d(u, v, A, B, C) and added once per (Gaussian, tile) to its
//       accumulator in global memory.
//   preprocess_backward_kernel  one thread per Gaussian: (u, v, A, B, C) ->
//       (mean, scale, quaternion) through the conic inverse, Sigma2D =
//       T Sigma T^T, T = J W and Sigma = (Rq S)(Rq S)^T; opacity and colour
//       partials are copied out.
#include <hip/hip_runtime.h>

#include "ia_internal.h"
#include "raster_common.h"

namespace ia {
namespace {

constexpr int kBwdBatch = 256;
constexpr int64_t kBwdTwoPixelTiles = 8192;

constexpr int kSlots = 7;  // Gaussians buffered per wave before their partials are summed (7 x 9 <= 64 lanes)

// Sum of v over the lane's quad (lanes 4i..4i+3), in every lane of the quad
// (two adds with a DPP quad permutation on their second operand).
__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    return v;
}

// LDS written by the lanes of one wave is read back by other lanes of the same
// wave: order the accesses at wavefront scope.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct RasterBwdArgs {
    const uint2* ranges;
    const uint32_t* vals;
    const float4* pa;
    const float4* pb;
    const float* pc;
    const DevCamera* cams;
    int W, H, tiles_x;
    uint32_t ntiles;
    uint64_t cap;
    int64_t N;
    const float* gimg;
    const float* T_final;
    const uint32_t* n_contrib;
    float* gacc;  // [N][9]
};

// Backward state of one pixel: transmittance recovered back to front,
// D = dL/dpixel . S where S is the colour lying behind the current Gaussian
// (starting at T_final bg), dL/dpixel and the number of Gaussians composited.
struct BPix {
    float T, D, g[3];
    uint32_t nc;
};

// Adds one pixel's partials for a Gaussian to gv (Eq. 4 and the splat of
// Eq. 3 differentiated), branch-free: a pixel that does not composite the
// Gaussian (tk false) adds zeros and keeps its state.
//   T_i = T_{i+1} / (1 - alpha), w = alpha T_i, dL/dc += g w,
//   dL/dalpha = T_i (g . c) - D / (1 - alpha), then D += w (g . c);
//   unless alpha is clamped at 0.99: dL/do += dL/dalpha G and, with
//   gp = dL/dalpha alpha = dL/dpower, the moments gp (dx, dy, dx^2, dx dy,
//   dy^2), from which the mean and conic gradients follow once per Gaussian.
template <bool FIRST>
__device__ __forceinline__ void pixel_grad(BPix& p, bool tk, float a0, float G, float dx, float dy, float c0,
                                           float c1, float c2, float gv[kGradPerGaussian]) {
#pragma clang fp contract(fast)
    const float ae = tk ? a0 : 0.0f;
    const float inv = __builtin_amdgcn_rcpf(1.0f - ae);
    const float Ti = p.T * inv;
    const float w = ae * Ti;
    const float gc = p.g[0] * c0 + p.g[1] * c1 + p.g[2] * c2;
    const float galpha = Ti * gc - inv * p.D;
    p.D += w * gc;
    p.T = tk ? Ti : p.T;
    const float gal = tk && a0 < 0.99f ? galpha : 0.0f;
    const float gp = gal * a0;
    const float t = gp * dx, u = gp * dy;
    const float add[kGradPerGaussian] = {t, u, t * dx, t * dy, u * dy, gal * G, p.g[0] * w, p.g[1] * w, p.g[2] * w};
#pragma unroll
    for (int k = 0; k < kGradPerGaussian; ++k) gv[k] = FIRST ? add[k] : gv[k] + add[k];
}

// One block per 16x16 tile.  PX = 2: 128 threads, thread (col, row) takes
// pixels (col, 2 row) and (col, 2 row + 1), sharing dx, the dx terms of the
// power and the per-Gaussian reductions; PX = 1: 256 threads, one pixel each.
template <int PX>
__global__ void __launch_bounds__(256 / PX) raster_backward_kernel(RasterBwdArgs a) {
#pragma clang fp contract(fast)
    constexpr int kThreads = 256 / PX, kWaves = kThreads / 64;
    __shared__ float4 s_a[kBwdBatch];  // u, v, -A log2(e)/2, -B log2(e)
    __shared__ float4 s_b[kBwdBatch];  // -C log2(e)/2, o, r, g
    __shared__ float s_c[kBwdBatch];   // b
    __shared__ uint32_t s_id[kBwdBatch];
    __shared__ float s_g[kBwdBatch][kGradPerGaussian];
    // per wave: quad partial sums of the buffered Gaussians [slot][partial][quad]
    __shared__ __align__(16) float s_q[kWaves][kSlots][kGradPerGaussian][16];
    __shared__ int s_slot[kWaves][kSlots];
    __shared__ uint32_t s_maxnc;
    const int f = blockIdx.z;
    const uint32_t tile = (uint32_t)f * a.ntiles + blockIdx.y * (uint32_t)a.tiles_x + blockIdx.x;
    uint2 rg = a.ranges[tile];
    if (rg.y > a.cap) rg.y = (uint32_t)a.cap;
    if (rg.x > rg.y) rg.x = rg.y;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int px = blockIdx.x * 16 + (threadIdx.x & 15);
    const int py0 = blockIdx.y * 16 + PX * (threadIdx.x >> 4);
    const size_t plane = (size_t)a.W * a.H;
    const DevCamera& cam = a.cams[f];
    BPix P[PX];
    uint32_t mine = 0;
#pragma unroll
    for (int k = 0; k < PX; ++k) {
        const int py = py0 + k;
        const bool in = px < a.W && py < a.H;
        const size_t pix = (size_t)py * a.W + px;
        P[k].nc = 0;
        P[k].T = 1.0f;
        for (int c = 0; c < 3; ++c) P[k].g[c] = 0.0f;
        if (in) {
            P[k].nc = a.n_contrib[(size_t)f * plane + pix];
            P[k].T = a.T_final[(size_t)f * plane + pix];
            for (int c = 0; c < 3; ++c) P[k].g[c] = a.gimg[((size_t)f * 3 + c) * plane + pix];
        }
        P[k].D = P[k].T * ((P[k].g[0] * cam.bg[0] + P[k].g[1] * cam.bg[1]) + P[k].g[2] * cam.bg[2]);
        mine = max(mine, P[k].nc);
    }
    if (threadIdx.x == 0) s_maxnc = 0;
    __syncthreads();
    if (mine) atomicMax(&s_maxnc, mine);
    // largest n_contrib of this wave: no pixel of the wave composites beyond it
    uint32_t wmax = mine;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wmax = max(wmax, (uint32_t)__shfl_xor((int)wmax, o, 64));
    __syncthreads();
    const uint32_t len = rg.y - rg.x;
    const int maxnc = (int)(s_maxnc < len ? s_maxnc : len);
    const float fx = (float)px + 0.5f;
    float* q = &s_q[wv][0][0][0];
    for (int end = maxnc; end > 0; end -= kBwdBatch) {
        const int start = end - kBwdBatch > 0 ? end - kBwdBatch : 0;
        const int n = end - start;
#pragma unroll
        for (int r = 0; r < PX; ++r) {
            const int slot = threadIdx.x + r * kThreads;
            if (slot < n) {
                uint32_t gid = a.vals[rg.x + start + slot];
                if ((int64_t)gid >= a.N) gid = 0;  // cannot happen for a valid sort; keeps reads in bounds
                const float4 pa = a.pa[gid], pb = a.pb[gid];
                s_a[slot] = make_float4(pa.x, pa.y, kConicScaleA * pa.z, kConicScaleB * pa.w);
                s_b[slot] = make_float4(kConicScaleA * pb.x, pb.y, pb.z, pb.w);
                s_c[slot] = a.pc[gid];
                s_id[slot] = gid;
            }
        }
        for (int k = threadIdx.x; k < kBwdBatch * kGradPerGaussian; k += kThreads) (&s_g[0][0])[k] = 0.0f;
        __syncthreads();
        // positions above the wave's largest n_contrib composite nothing here
        const int top = (int)wmax - start < n ? (int)wmax - start : n;
        int ns = 0;  // buffered Gaussians (wave-uniform)
        // sum the buffered quad partials: lane L < 9 m takes slot L / 9, partial L % 9
        auto flush = [&](int m) {
            wave_lds_sync();
            if (lane < kGradPerGaussian * m) {
                const int slot = lane / kGradPerGaussian, k = lane - slot * kGradPerGaussian;
                const float4* r = reinterpret_cast<const float4*>(q + (slot * kGradPerGaussian + k) * 16);
                const float4 v0 = r[0], v1 = r[1], v2 = r[2], v3 = r[3];
                const float sum = ((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w)) +
                                  ((v2.x + v2.y) + (v2.z + v2.w)) + ((v3.x + v3.y) + (v3.z + v3.w));
                if (sum != 0.0f) atomicAdd(&s_g[s_slot[wv][slot]][k], sum);
            }
            wave_lds_sync();
        };
        for (int j = top - 1; j >= 0; --j) {
            const uint32_t pos1 = (uint32_t)(start + j + 1);  // 1-based list position
            const float4 ga = s_a[j];
            const float4 gb = s_b[j];
            const float dx = fx - ga.x;
            float ta, tb;
            splat_dx_terms(ga.z, ga.w, dx, ta, tb);
            float pw[PX], al[PX], dy[PX];
            bool tk[PX];
            bool near = false;  // a superset of the composited pixels, before any exp
#pragma unroll
            for (int k = 0; k < PX; ++k) {
                dy[k] = (float)(py0 + k) + 0.5f - ga.y;
                pw[k] = splat_power(ta, tb, gb.x, dy[k]);
                near = near || (pos1 <= P[k].nc && pw[k] >= kPower2Min);
            }
            if (__ballot(near) == 0ull) continue;
            bool any = false;
#pragma unroll
            for (int k = 0; k < PX; ++k) {
                al[k] = splat_alpha(gb.y, pw[k]);
                tk[k] = pos1 <= P[k].nc && splat_takes(pw[k], al[k]);
                any = any || tk[k];
            }
            if (__ballot(any) == 0ull) continue;
            float gv[kGradPerGaussian];
            const float cb = s_c[j];
            pixel_grad<true>(P[0], tk[0], al[0], splat_gauss(pw[0]), dx, dy[0], gb.z, gb.w, cb, gv);
            // a further pixel row of the wave (PX > 1) is skipped when none of it composites
#pragma unroll
            for (int k = 1; k < PX; ++k)
                if (__ballot(tk[k]) != 0ull)
                    pixel_grad<false>(P[k], tk[k], al[k], splat_gauss(pw[k]), dx, dy[k], gb.z, gb.w, cb, gv);
#pragma unroll
            for (int k = 0; k < kGradPerGaussian; ++k) gv[k] = quad_sum(gv[k]);
            if ((lane & 3) == 0) {
#pragma unroll
                for (int k = 0; k < kGradPerGaussian; ++k) q[(ns * kGradPerGaussian + k) * 16 + (lane >> 2)] = gv[k];
            }
            if (lane == 0) s_slot[wv][ns] = j;
            if (++ns == kSlots) {
                flush(kSlots);
                ns = 0;
            }
        }
        if (ns) flush(ns);
        __syncthreads();
#pragma unroll
        for (int r = 0; r < PX; ++r) {
            const int slot = threadIdx.x + r * kThreads;
            if (slot < n) {
                // moments -> d/d(u, v, A, B, C) with power = -(A dx^2 + C dy^2)/2 - B dx dy
                float v[kGradPerGaussian];
#pragma unroll
                for (int k = 0; k < kGradPerGaussian; ++k) v[k] = s_g[slot][k];
                // the conic as projected (the staged copy is scaled to base 2)
                const float A = a.pa[s_id[slot]].z, B = a.pa[s_id[slot]].w, C = a.pb[s_id[slot]].x;
                const float mx = v[0], my = v[1], mxx = v[2], mxy = v[3], myy = v[4];
                v[0] = A * mx + B * my;
                v[1] = C * my + B * mx;
                v[2] = -0.5f * mxx;
                v[3] = -mxy;
                v[4] = -0.5f * myy;
                float* dst = a.gacc + (size_t)s_id[slot] * kGradPerGaussian;
#pragma unroll
                for (int k = 0; k < kGradPerGaussian; ++k)
                    if (v[k] != 0.0f) atomicAdd(dst + k, v[k]);
            }
        }
        __syncthreads();
    }
}

struct PreBwdArgs {
    const float* means;
    int stride;
    const float* scales;
    const float* quats;
    const DevCamera* cams;
    const int64_t* fo;
    int F;
    int64_t N;
    const uint32_t* tiles;
    const float* gacc;
    float* g_means;  // [N][3]
    float* g_scales;
    float* g_quats;
    float* g_opacity;
    float* g_colors;
    const float* sh;  // degree-3 SH colours, or null
    float* g_sh;
};

__device__ __forceinline__ int frame_index(const int64_t* fo, int F, int64_t i) {
    int lo = 0, hi = F - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (fo[mid] <= i)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

__global__ void __launch_bounds__(256) preprocess_backward_kernel(PreBwdArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.N) return;
    float gmu[3] = {0, 0, 0}, gs[3] = {0, 0, 0}, gq[4] = {0, 0, 0, 0};
    const float* gi = a.gacc + i * kGradPerGaussian;
    const bool vis = a.tiles[i] > 0;
    if (vis) {
        const DevCamera& cam = a.cams[frame_index(a.fo, a.F, i)];
        const float* R = cam.R;
        const float* mu = a.means + i * a.stride;
        const float* s = a.scales + i * 3;
        const float* q = a.quats + i * 4;
        float p[3];
        for (int k = 0; k < 3; ++k) p[k] = (R[k * 3] * mu[0] + R[k * 3 + 1] * mu[1]) + R[k * 3 + 2] * mu[2] + cam.t[k];
        const float qlen = sqrtf(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
        const float w = q[0] / qlen, x = q[1] / qlen, y = q[2] / qlen, z = q[3] / qlen;
        float Rq[9];
        Rq[0] = 1.0f - 2.0f * (y * y + z * z);
        Rq[1] = 2.0f * (x * y - w * z);
        Rq[2] = 2.0f * (x * z + w * y);
        Rq[3] = 2.0f * (x * y + w * z);
        Rq[4] = 1.0f - 2.0f * (x * x + z * z);
        Rq[5] = 2.0f * (y * z - w * x);
        Rq[6] = 2.0f * (x * z - w * y);
        Rq[7] = 2.0f * (y * z + w * x);
        Rq[8] = 1.0f - 2.0f * (x * x + y * y);
        float M[9], S[9];
        for (int r = 0; r < 3; ++r)
            for (int c = 0; c < 3; ++c) M[r * 3 + c] = Rq[r * 3 + c] * s[c];
        for (int r = 0; r < 3; ++r)
            for (int c = 0; c < 3; ++c) S[r * 3 + c] = M[r * 3] * M[c * 3] + M[r * 3 + 1] * M[c * 3 + 1] + M[r * 3 + 2] * M[c * 3 + 2];
        const float pz = p[2], pz2 = pz * pz;
        const float j00 = cam.fx / pz, j02 = -cam.fx * p[0] / pz2, j11 = cam.fy / pz, j12 = -cam.fy * p[1] / pz2;
        float T[6];
        for (int k = 0; k < 3; ++k) {
            T[k] = j00 * R[k] + j02 * R[6 + k];
            T[3 + k] = j11 * R[3 + k] + j12 * R[6 + k];
        }
        float TS[6];
        for (int r = 0; r < 2; ++r)
            for (int k = 0; k < 3; ++k) TS[r * 3 + k] = T[r * 3] * S[k] + T[r * 3 + 1] * S[3 + k] + T[r * 3 + 2] * S[6 + k];
        float c2[4];
        for (int r = 0; r < 2; ++r)
            for (int c = 0; c < 2; ++c) c2[r * 2 + c] = TS[r * 3] * T[c * 3] + TS[r * 3 + 1] * T[c * 3 + 1] + TS[r * 3 + 2] * T[c * 3 + 2];
        const float det = c2[0] * c2[3] - c2[1] * c2[1];
        const float Kc[4] = {c2[3] / det, -c2[1] / det, -c2[1] / det, c2[0] / det};
        // conic = Sigma2D^-1: dL/dSigma2D = -K G K (G: symmetric gradient of the conic matrix)
        const float G[4] = {gi[2], 0.5f * gi[3], 0.5f * gi[3], gi[4]};
        float KG[4], GS[4];
        for (int r = 0; r < 2; ++r)
            for (int c = 0; c < 2; ++c) KG[r * 2 + c] = Kc[r * 2] * G[c] + Kc[r * 2 + 1] * G[2 + c];
        for (int r = 0; r < 2; ++r)
            for (int c = 0; c < 2; ++c) GS[r * 2 + c] = -(KG[r * 2] * Kc[c] + KG[r * 2 + 1] * Kc[2 + c]);
        // Sigma2D = T Sigma T^T: dL/dT = 2 GS T Sigma, dL/dSigma = T^T GS T
        float GT[6];
        for (int r = 0; r < 2; ++r)
            for (int k = 0; k < 3; ++k) GT[r * 3 + k] = 2.0f * (GS[r * 2] * TS[k] + GS[r * 2 + 1] * TS[3 + k]);
        float GSig[9];
        for (int k = 0; k < 3; ++k)
            for (int l = 0; l < 3; ++l) {
                float acc = 0.0f;
                for (int r = 0; r < 2; ++r)
                    for (int c = 0; c < 2; ++c) acc += T[r * 3 + k] * GS[r * 2 + c] * T[c * 3 + l];
                GSig[k * 3 + l] = acc;
            }
        // T = J W: dL/dJ = GT W^T
        float gj00 = 0, gj02 = 0, gj11 = 0, gj12 = 0;
        for (int k = 0; k < 3; ++k) {
            gj00 += GT[k] * R[k];
            gj02 += GT[k] * R[6 + k];
            gj11 += GT[3 + k] * R[3 + k];
            gj12 += GT[3 + k] * R[6 + k];
        }
        const float gu = gi[0], gv = gi[1];
        const float pz3 = pz2 * pz;
        float gp[3];
        gp[0] = gu * cam.fx / pz - gj02 * cam.fx / pz2;
        gp[1] = gv * cam.fy / pz - gj12 * cam.fy / pz2;
        gp[2] = -gu * cam.fx * p[0] / pz2 - gv * cam.fy * p[1] / pz2 - gj00 * cam.fx / pz2 +
                gj02 * 2.0f * cam.fx * p[0] / pz3 - gj11 * cam.fy / pz2 + gj12 * 2.0f * cam.fy * p[1] / pz3;
        for (int k = 0; k < 3; ++k) gmu[k] = R[k] * gp[0] + R[3 + k] * gp[1] + R[6 + k] * gp[2];
        // Sigma = M M^T: dL/dM = 2 GSig M; M = Rq diag(s)
        float GR[9];
        for (int c = 0; c < 3; ++c) {
            float acc = 0.0f;
            for (int r = 0; r < 3; ++r) {
                const float gm = 2.0f * (GSig[r * 3] * M[c] + GSig[r * 3 + 1] * M[3 + c] + GSig[r * 3 + 2] * M[6 + c]);
                acc += gm * Rq[r * 3 + c];
                GR[r * 3 + c] = gm * s[c];
            }
            gs[c] = acc;
        }
        // Rq of the unit quaternion, then through q / |q|
        float gn[4];
        gn[0] = 2.0f * (-z * GR[1] + y * GR[2] + z * GR[3] - x * GR[5] - y * GR[6] + x * GR[7]);
        gn[1] = 2.0f * (y * GR[1] + z * GR[2] + y * GR[3] - 2.0f * x * GR[4] - w * GR[5] + z * GR[6] + w * GR[7] -
                        2.0f * x * GR[8]);
        gn[2] = 2.0f * (-2.0f * y * GR[0] + x * GR[1] + w * GR[2] + x * GR[3] + z * GR[5] - w * GR[6] + z * GR[7] -
                        2.0f * y * GR[8]);
        gn[3] = 2.0f * (-2.0f * z * GR[0] - w * GR[1] + x * GR[2] + w * GR[3] - 2.0f * z * GR[4] + y * GR[5] +
                        x * GR[6] + y * GR[7]);
        const float dot = gn[0] * w + gn[1] * x + gn[2] * y + gn[3] * z;
        gq[0] = (gn[0] - dot * w) / qlen;
        gq[1] = (gn[1] - dot * x) / qlen;
        gq[2] = (gn[2] - dot * y) / qlen;
        gq[3] = (gn[3] - dot * z) / qlen;
    }
    if (a.sh) {
        // colour = max(0, sum_k sh_k Y_k(dir) + 1/2), dir = normalize(mu - centre)
        // (as the forward evaluates it): dL/dsh_k = dL/dc Y_k where the sum is
        // positive, and the view direction's share of dL/dmu
        float* gsh = a.g_sh + i * 48;
        if (vis) {
            const DevCamera& cam = a.cams[frame_index(a.fo, a.F, i)];
            const float* mu = a.means + i * a.stride;
            const float d0 = mu[0] - cam.centre[0], d1 = mu[1] - cam.centre[1], d2 = mu[2] - cam.centre[2];
            const float inv = 1.0f / sqrtf(d0 * d0 + d1 * d1 + d2 * d2);
            const float x = d0 * inv, y = d1 * inv, z = d2 * inv;
            float Y[16];
            sh_basis16(x, y, z, Y);
            const float* shc = a.sh + i * 48;
            float acc[3] = {0.5f, 0.5f, 0.5f};
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                acc[0] += shc[k * 3 + 0] * Y[k];
                acc[1] += shc[k * 3 + 1] * Y[k];
                acc[2] += shc[k * 3 + 2] * Y[k];
            }
            float gc[3];
#pragma unroll
            for (int c = 0; c < 3; ++c) gc[c] = acc[c] > 0.0f ? gi[6 + c] : 0.0f;
            float wk[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                gsh[k * 3 + 0] = gc[0] * Y[k];
                gsh[k * 3 + 1] = gc[1] * Y[k];
                gsh[k * 3 + 2] = gc[2] * Y[k];
                wk[k] = (gc[0] * shc[k * 3 + 0] + gc[1] * shc[k * 3 + 1]) + gc[2] * shc[k * 3 + 2];
            }
            float gd[3];
            sh_basis16_grad(x, y, z, wk, gd);
            const float dot = (x * gd[0] + y * gd[1]) + z * gd[2];
            gmu[0] += (gd[0] - x * dot) * inv;
            gmu[1] += (gd[1] - y * dot) * inv;
            gmu[2] += (gd[2] - z * dot) * inv;
        } else {
            for (int k = 0; k < 48; ++k) gsh[k] = 0.0f;
        }
    }
    for (int k = 0; k < 3; ++k) {
        a.g_means[i * 3 + k] = gmu[k];
        a.g_scales[i * 3 + k] = gs[k];
        a.g_colors[i * 3 + k] = vis ? gi[6 + k] : 0.0f;
    }
    for (int k = 0; k < 4; ++k) a.g_quats[i * 4 + k] = gq[k];
    a.g_opacity[i] = vis ? gi[5] : 0.0f;
}

__global__ void fill_f32_kernel(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.0f;
}

__global__ void zero_f64_kernel(double* p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) p[0] = 0.0;
}

// L = mean |image - target|; dL/dimage = sign(image - target) / n (0 where equal).
__global__ void __launch_bounds__(256) l1_loss_kernel(const float* img, const float* tgt, int64_t n, double* loss,
                                                      float* grad) {
    __shared__ double s_sum[4];
    const float inv = 1.0f / (float)n;
    double local = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const float x = img[i], y = tgt[i];
        grad[i] = x > y ? inv : (x < y ? -inv : 0.0f);
        local += fabs((double)x - (double)y);  // exact in double
    }
    for (int o = 32; o > 0; o >>= 1) local += __shfl_xor(local, o, 64);
    if ((threadIdx.x & 63) == 0) s_sum[threadIdx.x >> 6] = local;
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(loss, (s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3]) / (double)n);
}

int blocks_for(int64_t n, int per, int cap) {
    int64_t b = (n + per - 1) / per;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (int)b;
}

}  // namespace

hipError_t launch_render_backward(const RenderBwdArgs& a, hipStream_t s) {
    const RenderLayout& L = a.lay;
    unsigned char* ws = a.ws;
    const int64_t N = L.N;
    float* gacc = reinterpret_cast<float*>(ws + L.gacc);
    const DevCamera* cams = reinterpret_cast<const DevCamera*>(ws + L.cams);
    const int64_t* fo = reinterpret_cast<const int64_t*>(ws + L.fo);
    if (N <= 0) return hipSuccess;
    IA_LAUNCH("fill_f32_kernel", fill_f32_kernel, dim3(blocks_for(N * kGradPerGaussian, 256, 8192)), dim3(256), 0, s,
              gacc, N * kGradPerGaussian);
    RasterBwdArgs rb{reinterpret_cast<const uint2*>(ws + L.ranges), reinterpret_cast<const uint32_t*>(ws + L.vals),
                     reinterpret_cast<const float4*>(ws + L.pa), reinterpret_cast<const float4*>(ws + L.pb),
                     reinterpret_cast<const float*>(ws + L.pc), cams, a.W, a.H, L.tiles_x,
                     (uint32_t)(L.tiles_x * L.tiles_y), (uint64_t)L.cap, N, a.grad_image, a.T_final, a.n_contrib,
                     gacc};
    // two pixels per thread when there are enough tiles to fill the chip twice
    // over (four per thread, one wave per tile, measured slower: 8.3 -> 9.2 ms
    // on Stress, as the block's LDS batch then caps a CU at six waves)
    if (L.ntiles_all >= kBwdTwoPixelTiles)
        IA_LAUNCH("raster_backward_kernel", raster_backward_kernel<2>, dim3(L.tiles_x, L.tiles_y, L.frames),
                  dim3(128), 0, s, rb);
    else
        IA_LAUNCH("raster_backward_kernel", raster_backward_kernel<1>, dim3(L.tiles_x, L.tiles_y, L.frames),
                  dim3(256), 0, s, rb);
    PreBwdArgs pb{a.means, a.means_stride, a.scales, a.quats, cams, fo, L.frames, N,
                  reinterpret_cast<const uint32_t*>(ws + L.tiles), gacc, a.g_means, a.g_scales, a.g_quats,
                  a.g_opacity, a.g_colors, a.sh, a.g_sh};
    IA_LAUNCH("preprocess_backward_kernel", preprocess_backward_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0,
              s, pb);
    return hipGetLastError();
}

hipError_t launch_l1_loss(const float* image, const float* target, int64_t n, double* loss, float* grad,
                          hipStream_t s) {
    IA_LAUNCH("zero_f64_kernel", zero_f64_kernel, dim3(1), dim3(64), 0, s, loss);
    if (n > 0)
        IA_LAUNCH("l1_loss_kernel", l1_loss_kernel, dim3(blocks_for(n, 256, 4096)), dim3(256), 0, s, image, target, n,
                  loss, grad);
    return hipGetLastError();
}

}  // namespace ia
