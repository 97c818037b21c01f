// Training objective and optimiser step of SPIN-4DGS ("Implicit 4D Gaussian
// Splatting for Fast Motion with Large Inter-Frame Displacements"):
//   image loss, §3.3 Eq. 12: L = (1 - lambda) L1 + lambda (1 - SSIM), with
//     SSIM the structural similarity of Wang et al. (2004), which the pages
//     cite for their metric: 11 x 11 Gaussian window (sigma 1.5), C1 = 0.01^2,
//     C2 = 0.03^2, per colour channel, window taps outside the image zero,
//     averaged over every pixel, channel and frame; and dL/dimage;
//   Adam (Kingma & Ba, 2015), the optimiser named in §4 implementation
//     details, one bias-corrected step over a parameter array.
//
// ssim_fwd_kernel: one 256-thread block per 16 x 16 output tile of one image
// plane.  The 26 x 26 halo of x and y is staged in LDS, the horizontal window
// sums of the five moments (x, y, x^2, y^2, xy) over the 26 rows are formed
// in LDS, and each thread sums 11 of them vertically: mu_x, mu_y, E[x^2],
// E[y^2], E[xy] of its pixel.  It writes S's derivatives with respect to
// mu_x, E[x^2] and E[xy] (the only moments that depend on x) and the block's
// sums of S and |x - y| (one pair per block; loss_finish_kernel adds them in
// a fixed order, so the loss is the same on every run).
// ssim_bwd_kernel: the same tiling applied to the three derivative maps (the
// window is symmetric, so its adjoint is the same zero-padded window sum),
// combined into dL/dx = (1 - lambda) sign(x - y) / n
//   - lambda (blur(dS/dmu_x) + 2 x blur(dS/dE[x^2]) + y blur(dS/dE[xy])) / n.
#include <hip/hip_runtime.h>

#include "ia_internal.h"

namespace ia {
namespace {

constexpr int kT = 16;                // output tile edge
constexpr int kR = 5;                 // window radius
constexpr int kHalo = kT + 2 * kR;    // 26
constexpr float kC1 = 0.01f * 0.01f;
constexpr float kC2 = 0.03f * 0.03f;

// 1-D window taps exp(-d^2 / (2 * 1.5^2)) for d = -5..5, normalised to sum 1
// (evaluated in double, rounded to float)
__constant__ float c_win[2 * kR + 1] = {0.001028380123898387f,  0.0075987582094967365f, 0.036000773310661316f,
                                        0.10936068743467331f,  0.21300554275512695f,   0.26601171493530273f,
                                        0.21300554275512695f,  0.10936068743467331f,   0.036000773310661316f,
                                        0.0075987582094967365f, 0.001028380123898387f};

struct LossArgs {
    const float* x;
    const float* y;
    int H, W;
    float lambda;
    double inv_n;
    float* d;       // [3][planes][H][W]: dS/dmu_x, dS/dE[x^2], dS/dE[xy]
    size_t plane_stride;  // floats between the three derivative maps
    double2* part;  // per block: sum S, sum |x - y|
    float* grad;
};

// Stage the 26 x 26 halo of `src` (one plane) around tile (tx, ty); zero outside.
__device__ __forceinline__ void stage_halo(const float* src, int H, int W, int x0, int y0, float* dst) {
    for (int k = threadIdx.x; k < kHalo * kHalo; k += 256) {
        const int r = k / kHalo, c = k - r * kHalo;
        const int yy = y0 + r - kR, xx = x0 + c - kR;
        dst[k] = (yy >= 0 && yy < H && xx >= 0 && xx < W) ? src[(size_t)yy * W + xx] : 0.0f;
    }
}

__global__ void __launch_bounds__(256) ssim_fwd_kernel(LossArgs a) {
    __shared__ float s_x[kHalo * kHalo], s_y[kHalo * kHalo];
    __shared__ float s_h[5][kHalo][kT];  // horizontal window sums of the moments
    __shared__ double s_red[2][4];
    const int plane = blockIdx.z;
    const int x0 = blockIdx.x * kT, y0 = blockIdx.y * kT;
    const size_t poff = (size_t)plane * a.H * a.W;
    stage_halo(a.x + poff, a.H, a.W, x0, y0, s_x);
    stage_halo(a.y + poff, a.H, a.W, x0, y0, s_y);
    __syncthreads();
    for (int k = threadIdx.x; k < kHalo * kT; k += 256) {
        const int r = k / kT, c = k - r * kT;
        float m[5] = {0, 0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t <= 2 * kR; ++t) {
            const float xv = s_x[r * kHalo + c + t], yv = s_y[r * kHalo + c + t], w = c_win[t];
            m[0] += w * xv;
            m[1] += w * yv;
            m[2] += w * (xv * xv);
            m[3] += w * (yv * yv);
            m[4] += w * (xv * yv);
        }
#pragma unroll
        for (int q = 0; q < 5; ++q) s_h[q][r][c] = m[q];
    }
    __syncthreads();
    const int c = threadIdx.x & (kT - 1), r = threadIdx.x / kT;
    const int px = x0 + c, py = y0 + r;
    const bool in = px < a.W && py < a.H;
    float m[5] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t <= 2 * kR; ++t) {
        const float w = c_win[t];
#pragma unroll
        for (int q = 0; q < 5; ++q) m[q] += w * s_h[q][r + t][c];
    }
    double s_sum = 0.0, l1_sum = 0.0;
    if (in) {
        const float mx = m[0], my = m[1];
        const float sxx = m[2] - mx * mx, syy = m[3] - my * my, sxy = m[4] - mx * my;
        const float a1 = 2.0f * mx * my + kC1, a2 = 2.0f * sxy + kC2;
        const float b1 = mx * mx + my * my + kC1, b2 = sxx + syy + kC2;
        const float S = (a1 * a2) / (b1 * b2);
        const size_t i = poff + (size_t)py * a.W + px;
        // terms paired by the moments that approach each other as x -> y, so
        // identical windows give exactly zero
        a.d[i] = S * ((2.0f * my / a1 - 2.0f * mx / b1) + (2.0f * mx / b2 - 2.0f * my / a2));
        a.d[a.plane_stride + i] = -S / b2;
        a.d[2 * a.plane_stride + i] = 2.0f * S / a2;
        s_sum = (double)S;
        const float xv = s_x[(r + kR) * kHalo + c + kR], yv = s_y[(r + kR) * kHalo + c + kR];
        l1_sum = fabs((double)xv - (double)yv);
    }
    for (int o = 32; o > 0; o >>= 1) {
        s_sum += __shfl_xor(s_sum, o, 64);
        l1_sum += __shfl_xor(l1_sum, o, 64);
    }
    if ((threadIdx.x & 63) == 0) {
        s_red[0][threadIdx.x >> 6] = s_sum;
        s_red[1][threadIdx.x >> 6] = l1_sum;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const size_t b = ((size_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
        a.part[b] = make_double2((s_red[0][0] + s_red[0][1]) + (s_red[0][2] + s_red[0][3]),
                                 (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]));
    }
}

__global__ void __launch_bounds__(256) ssim_bwd_kernel(LossArgs a) {
    __shared__ float s_d[3][kHalo * kHalo];
    __shared__ float s_h[3][kHalo][kT];
    const int plane = blockIdx.z;
    const int x0 = blockIdx.x * kT, y0 = blockIdx.y * kT;
    const size_t poff = (size_t)plane * a.H * a.W;
#pragma unroll
    for (int q = 0; q < 3; ++q) stage_halo(a.d + q * a.plane_stride + poff, a.H, a.W, x0, y0, s_d[q]);
    __syncthreads();
    for (int k = threadIdx.x; k < kHalo * kT; k += 256) {
        const int r = k / kT, c = k - r * kT;
        float m[3] = {0, 0, 0};
#pragma unroll
        for (int t = 0; t <= 2 * kR; ++t) {
            const float w = c_win[t];
#pragma unroll
            for (int q = 0; q < 3; ++q) m[q] += w * s_d[q][r * kHalo + c + t];
        }
#pragma unroll
        for (int q = 0; q < 3; ++q) s_h[q][r][c] = m[q];
    }
    __syncthreads();
    const int c = threadIdx.x & (kT - 1), r = threadIdx.x / kT;
    const int px = x0 + c, py = y0 + r;
    if (px >= a.W || py >= a.H) return;
    float m[3] = {0, 0, 0};
#pragma unroll
    for (int t = 0; t <= 2 * kR; ++t) {
        const float w = c_win[t];
#pragma unroll
        for (int q = 0; q < 3; ++q) m[q] += w * s_h[q][r + t][c];
    }
    const size_t i = poff + (size_t)py * a.W + px;
    const float xv = a.x[i], yv = a.y[i];
    const float inv_n = (float)a.inv_n;
    const float dssim = (m[0] + 2.0f * xv * m[1] + yv * m[2]) * inv_n;
    const float sgn = xv > yv ? 1.0f : (xv < yv ? -1.0f : 0.0f);
    a.grad[i] = (1.0f - a.lambda) * sgn * inv_n - a.lambda * dssim;
}

// One block of kFinish threads: the per-block sums added in a fixed order;
// loss[0] = (1 - lambda) L1 + lambda (1 - SSIM), loss[1] = L1, loss[2] = SSIM
constexpr int kFinish = 1024;
__global__ void __launch_bounds__(kFinish) loss_finish_kernel(const double2* part, int64_t nblocks, double inv_n,
                                                              double lambda, double* loss) {
    __shared__ double s_s[kFinish], s_l[kFinish];
    double ss = 0.0, sl = 0.0;
    for (int64_t b = threadIdx.x; b < nblocks; b += kFinish) {
        const double2 v = part[b];
        ss += v.x;
        sl += v.y;
    }
    s_s[threadIdx.x] = ss;
    s_l[threadIdx.x] = sl;
    __syncthreads();
    for (int w = kFinish / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            s_s[threadIdx.x] += s_s[threadIdx.x + w];
            s_l[threadIdx.x] += s_l[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double ssim = s_s[0] * inv_n, l1 = s_l[0] * inv_n;
        loss[0] = (1.0 - lambda) * l1 + lambda * (1.0 - ssim);
        loss[1] = l1;
        loss[2] = ssim;
    }
}

// p -= step_size * m / (sqrt(v * v_scale) + eps) after the moment updates;
// step_size = lr / (1 - b1^t), v_scale = 1 / (1 - b2^t) (host, double).
// g, m, v are dense [n]; with STRIDED the parameter is rows of `dim` values
// `stride` floats apart (element i at (i / dim) * stride + i % dim).
template <bool STRIDED>
__global__ void __launch_bounds__(256) adam_kernel(float* p, const float* g, float* m, float* v, int64_t n, int dim,
                                                   int stride, float b1, float b2, float eps, float step_size,
                                                   float v_scale, uint16_t* p16) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        int64_t j = i;
        if constexpr (STRIDED) {
            const int64_t row = i / dim;
            j = row * stride + (i - row * dim);
        }
        const float gi = g[i];
        const float mi = b1 * m[i] + (1.0f - b1) * gi;
        const float vi = b2 * v[i] + (1.0f - b2) * (gi * gi);
        m[i] = mi;
        v[i] = vi;
        const float pi = p[j] - step_size * mi / (sqrtf(vi * v_scale) + eps);
        p[j] = pi;
        if (p16) p16[i] = __builtin_bit_cast(uint16_t, (_Float16)pi);
    }
}

}  // namespace

// [3][planes][H][W] float derivative maps, then one double2 per SSIM block
size_t image_loss_workspace(int32_t frames, int32_t H, int32_t W) {
    const size_t maps = (size_t)3 * frames * 3 * (size_t)H * W * sizeof(float);
    const size_t blocks = (size_t)((W + kT - 1) / kT) * ((H + kT - 1) / kT) * frames * 3;
    return ((maps + 255) & ~(size_t)255) + blocks * sizeof(double2);
}

hipError_t launch_image_loss(const float* image, const float* target, int32_t frames, int32_t H, int32_t W,
                             float lambda, void* ws, double* loss, float* grad, hipStream_t s) {
    const int planes = frames * 3;
    const size_t n = (size_t)planes * H * W;
    const size_t maps = ((3 * n * sizeof(float)) + 255) & ~(size_t)255;
    double2* part = reinterpret_cast<double2*>((char*)ws + maps);
    LossArgs a{image, target, H, W, lambda, 1.0 / (double)n, reinterpret_cast<float*>(ws), n, part, grad};
    const dim3 grid((W + kT - 1) / kT, (H + kT - 1) / kT, planes);
    const int64_t nblocks = (int64_t)grid.x * grid.y * grid.z;
    IA_LAUNCH("ssim_fwd_kernel", ssim_fwd_kernel, grid, dim3(256), 0, s, a);
    IA_LAUNCH("ssim_bwd_kernel", ssim_bwd_kernel, grid, dim3(256), 0, s, a);
    IA_LAUNCH("loss_finish_kernel", loss_finish_kernel, dim3(1), dim3(kFinish), 0, s, part, nblocks,
              1.0 / (double)n, (double)lambda, loss);
    return hipGetLastError();
}

hipError_t launch_adam(float* p, const float* g, float* m, float* v, int64_t n, int32_t dim, int32_t stride,
                       float lr, float beta1, float beta2, float eps, int32_t step, uint16_t* p16, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const double step_size = (double)lr / (1.0 - pow((double)beta1, (double)step));
    const double v_scale = 1.0 / (1.0 - pow((double)beta2, (double)step));
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (dim == stride)
        IA_LAUNCH("adam_kernel", adam_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, p, g, m, v, n, dim,
                  stride, beta1, beta2, eps, (float)step_size, (float)v_scale, p16);
    else
        IA_LAUNCH("adam_kernel", adam_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, p, g, m, v, n, dim,
                  stride, beta1, beta2, eps, (float)step_size, (float)v_scale, p16);
    return hipGetLastError();
}

}  // namespace ia
