// Refinement of the positions, SPIN-4DGS ("Implicit 4D Gaussian Splatting for
// Fast Motion with Large Inter-Frame Displacements") §3.2 Eq. 6: the rendering
// loss densifies salient points and prunes unnecessary ones.  The rule is the
// adaptive density control of 3D Gaussian Splatting on the trainable
// positions:
//   salient  mean norm of the position gradient over the iterations that gave
//            one >= grad_threshold;
//   prune    decoded opacity < min_opacity (takes precedence);
//   clone    salient and largest decoded scale <= scale_threshold: the
//            Gaussian and a copy at its position (the copy's Adam moments 0);
//   split    salient and larger: two Gaussians at mu + R(q) (s * n_j), the
//            normal draws n_j handed in by the caller, moments 0;
//   keep     everything else, with its moments.
// Outputs keep the input order: per-block output counts, one scan of the
// block counts, then each block writes its Gaussians' outputs after a
// block-level exclusive scan of their counts (0, 1 or 2).  The decisions
// compare fp32 values (the mean is one correctly rounded fp32 division).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ia_internal.h"

namespace ia {
namespace {

constexpr int kDT = 256;                   // threads per block
constexpr int kDRounds = 16;               // rounds of kDT Gaussians per block
constexpr int kDItems = kDT * kDRounds;    // 4096 Gaussians per block
constexpr int kScanThreads = 1024;

enum : int { kPrune = 0, kKeep = 1, kClone = 2, kSplit = 3 };

struct DensifyArgs {
    const float* xyzt;
    const float* grad_acc;
    const int32_t* grad_count;
    const float* scales;
    const float* quats;
    const float* opacity;
    const float* noise;  // [N][2][3]
    const float* m;      // [N][3]
    const float* v;
    int64_t N;
    float grad_threshold, scale_threshold, min_opacity;
    float* out_xyzt;  // [2N][4]
    float* out_m;     // [2N][3]
    float* out_v;
    int64_t* boff;    // per block: first output row
    int64_t* out_n;
};

__device__ __forceinline__ int decide(const DensifyArgs& a, int64_t i) {
    const float op = a.opacity[i];
    if (op < a.min_opacity) return kPrune;
    const int32_t cnt = a.grad_count[i];
    if (cnt <= 0) return kKeep;
    const float mean = a.grad_acc[i] / (float)cnt;
    if (!(mean >= a.grad_threshold)) return kKeep;
    const float smax = fmaxf(fmaxf(a.scales[i * 3], a.scales[i * 3 + 1]), a.scales[i * 3 + 2]);
    return smax <= a.scale_threshold ? kClone : kSplit;
}

__device__ __forceinline__ int outputs(int d) { return d == kPrune ? 0 : (d == kKeep ? 1 : 2); }

__global__ void __launch_bounds__(kDT) densify_count_kernel(DensifyArgs a, int64_t* bcount) {
    __shared__ int s_w[kDT / 64];
    const int64_t b0 = (int64_t)blockIdx.x * kDItems;
    int cnt = 0;
    for (int r = 0; r < kDRounds; ++r) {
        const int64_t i = b0 + r * kDT + threadIdx.x;
        if (i < a.N) cnt += outputs(decide(a, i));
    }
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) bcount[blockIdx.x] = (int64_t)s_w[0] + s_w[1] + s_w[2] + s_w[3];
}

// Exclusive scan of nb block counts in place (one block); the total into *out_n.
__global__ void __launch_bounds__(kScanThreads) densify_scan_kernel(int64_t* b, int64_t nb, int64_t* out_n) {
    __shared__ int64_t s[kScanThreads];
    const int64_t per = (nb + kScanThreads - 1) / kScanThreads;
    const int64_t lo = threadIdx.x * per, hi = lo + per < nb ? lo + per : nb;
    int64_t run = 0;
    for (int64_t k = lo; k < hi; ++k) run += b[k];
    s[threadIdx.x] = run;
    __syncthreads();
    for (int o = 1; o < kScanThreads; o <<= 1) {
        const int64_t add = threadIdx.x >= (unsigned)o ? s[threadIdx.x - o] : 0;
        __syncthreads();
        s[threadIdx.x] += add;
        __syncthreads();
    }
    int64_t base = s[threadIdx.x] - run;
    for (int64_t k = lo; k < hi; ++k) {
        const int64_t c = b[k];
        b[k] = base;
        base += c;
    }
    if (threadIdx.x == kScanThreads - 1) *out_n = s[kScanThreads - 1];
}

__device__ __forceinline__ void put(const DensifyArgs& a, int64_t o, float4 p, const float* m, const float* v) {
    reinterpret_cast<float4*>(a.out_xyzt)[o] = p;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        a.out_m[o * 3 + k] = m ? m[k] : 0.0f;
        a.out_v[o * 3 + k] = v ? v[k] : 0.0f;
    }
}

__global__ void __launch_bounds__(kDT) densify_write_kernel(DensifyArgs a) {
    __shared__ int s_w[kDT / 64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t b0 = (int64_t)blockIdx.x * kDItems;
    int64_t base = a.boff[blockIdx.x];
    for (int r = 0; r < kDRounds; ++r) {
        const int64_t i = b0 + r * kDT + threadIdx.x;
        const int d = i < a.N ? decide(a, i) : kPrune;
        const int k = outputs(d);
        // inclusive scan of k over the wave, then over the block's waves
        int inc = k;
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(inc, o, 64);
            if (lane >= o) inc += t;
        }
        if (lane == 63) s_w[wv] = inc;
        __syncthreads();
        int before = 0;
        for (int w = 0; w < wv; ++w) before += s_w[w];
        const int total = s_w[0] + s_w[1] + s_w[2] + s_w[3];
        const int64_t o = base + before + inc - k;
        if (d != kPrune) {
            const float4 p = reinterpret_cast<const float4*>(a.xyzt)[i];
            if (d == kKeep) {
                put(a, o, p, a.m + i * 3, a.v + i * 3);
            } else if (d == kClone) {
                put(a, o, p, a.m + i * 3, a.v + i * 3);
                put(a, o + 1, p, nullptr, nullptr);
            } else {
                // R(q) of the normalised quaternion (w, x, y, z)
                float qw = a.quats[i * 4], qx = a.quats[i * 4 + 1], qy = a.quats[i * 4 + 2], qz = a.quats[i * 4 + 3];
                const float inv = 1.0f / sqrtf(qw * qw + qx * qx + qy * qy + qz * qz);
                qw *= inv;
                qx *= inv;
                qy *= inv;
                qz *= inv;
                const float R[3][3] = {{1.0f - 2.0f * (qy * qy + qz * qz), 2.0f * (qx * qy - qw * qz),
                                        2.0f * (qx * qz + qw * qy)},
                                       {2.0f * (qx * qy + qw * qz), 1.0f - 2.0f * (qx * qx + qz * qz),
                                        2.0f * (qy * qz - qw * qx)},
                                       {2.0f * (qx * qz - qw * qy), 2.0f * (qy * qz + qw * qx),
                                        1.0f - 2.0f * (qx * qx + qy * qy)}};
                const float s[3] = {a.scales[i * 3], a.scales[i * 3 + 1], a.scales[i * 3 + 2]};
                for (int j = 0; j < 2; ++j) {
                    const float* n = a.noise + (i * 2 + j) * 3;
                    const float d0 = s[0] * n[0], d1 = s[1] * n[1], d2 = s[2] * n[2];
                    const float4 c = make_float4(p.x + (R[0][0] * d0 + R[0][1] * d1 + R[0][2] * d2),
                                                 p.y + (R[1][0] * d0 + R[1][1] * d1 + R[1][2] * d2),
                                                 p.z + (R[2][0] * d0 + R[2][1] * d1 + R[2][2] * d2), p.w);
                    put(a, o + j, c, nullptr, nullptr);
                }
            }
        }
        base += total;
        __syncthreads();
    }
}

__global__ void __launch_bounds__(256) densify_accumulate_kernel(const float* g, int64_t N, float* acc, int32_t* cnt) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < N; i += (int64_t)gridDim.x * 256) {
        const float x = g[i * 3], y = g[i * 3 + 1], z = g[i * 3 + 2];
        const float nrm = sqrtf((x * x + y * y) + z * z);
        if (nrm > 0.0f) {
            acc[i] += nrm;
            cnt[i] += 1;
        }
    }
}

int64_t densify_blocks(int64_t N) { return (N + kDItems - 1) / kDItems; }

}  // namespace

size_t densify_workspace(int64_t N) { return ((size_t)densify_blocks(N) * sizeof(int64_t) + 255) & ~(size_t)255; }

hipError_t launch_densify_accumulate(const float* g, int64_t N, float* acc, int32_t* cnt, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    int64_t blocks = (N + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    IA_LAUNCH("densify_accumulate_kernel", densify_accumulate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, g, N,
              acc, cnt);
    return hipGetLastError();
}

hipError_t launch_densify(const DensifyIn& in, void* ws, hipStream_t s) {
    DensifyArgs a{in.xyzt, in.grad_acc, in.grad_count, in.scales, in.quats, in.opacity, in.noise, in.m, in.v, in.N,
                  in.grad_threshold, in.scale_threshold, in.min_opacity, in.out_xyzt, in.out_m, in.out_v,
                  reinterpret_cast<int64_t*>(ws), in.out_n};
    const int64_t nb = densify_blocks(in.N);
    if (nb == 0) {
        IA_LAUNCH("densify_scan_kernel", densify_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a.boff, (int64_t)0,
                  a.out_n);
        return hipGetLastError();
    }
    IA_LAUNCH("densify_count_kernel", densify_count_kernel, dim3((unsigned)nb), dim3(kDT), 0, s, a, a.boff);
    IA_LAUNCH("densify_scan_kernel", densify_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a.boff, nb, a.out_n);
    IA_LAUNCH("densify_write_kernel", densify_write_kernel, dim3((unsigned)nb), dim3(kDT), 0, s, a);
    return hipGetLastError();
}

}  // namespace ia
