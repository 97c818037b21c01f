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
// ssim_fwd_kernel: one 256-thread block per strip of 256 columns x 64 output
// rows of one image plane, one column per thread.  The block walks the 74
// input rows the strip's windows cover: each row of x and y (with a 5-column
// margin, zero outside the image) is staged in LDS, every thread forms the
// horizontal window sums of the five moments (x, y, x^2, y^2, xy) for its
// column and keeps the last 11 rows of them in registers; once 11 rows are
// in, the vertical window sum gives mu_x, mu_y, E[x^2], E[y^2], E[xy] of one
// output pixel.  It writes S's derivatives with respect to mu_x, E[x^2] and
// E[xy] (the only moments that depend on x) and the block's sums of S and
// |x - y| (one pair per block; loss_finish_kernel adds them in a fixed order,
// so the loss is the same on every run).
// ssim_bwd_kernel: the same sliding window over the three derivative maps
// (the window is symmetric, so its adjoint is the same zero-padded window
// sum), combined into dL/dx = (1 - lambda) sign(x - y) / n
//   - lambda (blur(dS/dmu_x) + 2 x blur(dS/dE[x^2]) + y blur(dS/dE[xy])) / n.
#include <hip/hip_runtime.h>

#include "ia_internal.h"

namespace ia {
namespace {

constexpr int kR = 5;                  // window radius
constexpr int kWin = 2 * kR + 1;       // 11 taps
constexpr int kSW = 256;               // strip width: one column per thread
constexpr int kSH = 64;                // output rows per block
constexpr int kRowsIn = kSH + 2 * kR;  // input rows a block reads
constexpr int kRowW = kSW + 2 * kR;    // staged row width
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

// A thread's share of image row yy (columns x0 - kR .. x0 + kSW + kR - 1,
// zero outside the image) of plane `src`: staged column c, and c + kSW for
// the first 2 kR threads.  Loaded one row ahead of its use (registers), so
// the loads overlap the previous row's arithmetic.
struct RowVals {
    float v0, v1;
};

// Both loads are unconditional, from clamped (in-image) addresses, and the
// values outside the image are replaced by zero afterwards: a load under a
// branch would wait for its data inside the branch.
__device__ __forceinline__ RowVals load_row(const float* src, int H, int W, int x0, int yy) {
    const int xa = x0 - kR + (int)threadIdx.x, xb = xa + kSW;
    const float* row = src + (size_t)min(max(yy, 0), H - 1) * W;
    const float va = row[min(max(xa, 0), W - 1)];
    const float vb = row[min(max(xb, 0), W - 1)];
    const bool rin = yy >= 0 && yy < H;
    return RowVals{(rin && xa >= 0 && xa < W) ? va : 0.0f, (rin && xb < W && threadIdx.x < 2 * kR) ? vb : 0.0f};
}

__device__ __forceinline__ void store_row(float* dst, RowVals r) {
    dst[threadIdx.x] = r.v0;
    if (threadIdx.x < 2 * kR) dst[threadIdx.x + kSW] = r.v1;
}

__device__ __forceinline__ size_t block_index() {
    return ((size_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
}

__global__ void __launch_bounds__(kSW) ssim_fwd_kernel(LossArgs a) {
    __shared__ float s_x[2][kRowW], s_y[2][kRowW];
    __shared__ double s_red[2][kSW / 64];
    const int x0 = blockIdx.x * kSW, y0 = blockIdx.y * kSH;
    const size_t poff = (size_t)blockIdx.z * a.H * a.W;
    const int c = threadIdx.x, px = x0 + c;
    float ring[kWin][5];  // horizontal sums of the last 11 input rows, slot = row % 11
    double s_sum = 0.0, l1_sum = 0.0;
    const float* xs = a.x + poff;
    const float* ys = a.y + poff;
    RowVals nx = load_row(xs, a.H, a.W, x0, y0 - kR), ny = load_row(ys, a.H, a.W, x0, y0 - kR);
    for (int base = 0; base < kRowsIn; base += kWin) {
#pragma unroll
        for (int u = 0; u < kWin; ++u) {
            const int ri = base + u;  // input row of the block's window (uniform)
            if (ri < kRowsIn) {
                float* bx = s_x[ri & 1];
                float* by = s_y[ri & 1];
                store_row(bx, nx);
                store_row(by, ny);
                // one barrier per row: a buffer is rewritten two rows later,
                // after every thread has passed this barrier of the row between
                __syncthreads();
                if (ri + 1 < kRowsIn) {
                    nx = load_row(xs, a.H, a.W, x0, y0 - kR + ri + 1);
                    ny = load_row(ys, a.H, a.W, x0, y0 - kR + ri + 1);
                }
                float m[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t = 0; t < kWin; ++t) {
                    const float xv = bx[c + t], yv = by[c + t], w = c_win[t];
                    m[0] += w * xv;
                    m[1] += w * yv;
                    m[2] += w * (xv * xv);
                    m[3] += w * (yv * yv);
                    m[4] += w * (xv * yv);
                }
#pragma unroll
                for (int q = 0; q < 5; ++q) ring[u][q] = m[q];
                const int ro = ri - 2 * kR;  // output row whose window ends at this input row
                const int py = y0 + ro;
                if (ro >= 0 && px < a.W && py < a.H) {
                    float v[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int t = 0; t < kWin; ++t) {
                        // input row ro + t = ri - 10 + t sits in slot (u + 1 + t) % 11
                        const float w = c_win[t];
#pragma unroll
                        for (int q = 0; q < 5; ++q) v[q] += w * ring[(u + 1 + t) % kWin][q];
                    }
                    const float mx = v[0], my = v[1];
                    const float sxx = v[2] - mx * mx, syy = v[3] - my * my, sxy = v[4] - mx * my;
                    const float a1 = 2.0f * mx * my + kC1, a2 = 2.0f * sxy + kC2;
                    const float b1 = mx * mx + my * my + kC1, b2 = sxx + syy + kC2;
                    const float S = (a1 * a2) / (b1 * b2);
                    const size_t i = poff + (size_t)py * a.W + px;
                    // terms paired by the moments that approach each other as x -> y,
                    // so identical windows give exactly zero
                    a.d[i] = S * ((2.0f * my / a1 - 2.0f * mx / b1) + (2.0f * mx / b2 - 2.0f * my / a2));
                    a.d[a.plane_stride + i] = -S / b2;
                    a.d[2 * a.plane_stride + i] = 2.0f * S / a2;
                    const float xv = a.x[i], yv = a.y[i];  // staged kR rows ago: an L2 hit
                    s_sum += (double)S;
                    l1_sum += fabs((double)xv - (double)yv);
                }
            }
        }
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
    if (threadIdx.x == 0)
        a.part[block_index()] = make_double2((s_red[0][0] + s_red[0][1]) + (s_red[0][2] + s_red[0][3]),
                                             (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]));
}

__global__ void __launch_bounds__(kSW) ssim_bwd_kernel(LossArgs a) {
    __shared__ float s_d[2][3][kRowW];
    const int x0 = blockIdx.x * kSW, y0 = blockIdx.y * kSH;
    const size_t poff = (size_t)blockIdx.z * a.H * a.W;
    const int c = threadIdx.x, px = x0 + c;
    const float inv_n = (float)a.inv_n;
    float ring[kWin][3];
    const float* ds[3] = {a.d + poff, a.d + a.plane_stride + poff, a.d + 2 * a.plane_stride + poff};
    RowVals nd[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) nd[q] = load_row(ds[q], a.H, a.W, x0, y0 - kR);
    for (int base = 0; base < kRowsIn; base += kWin) {
#pragma unroll
        for (int u = 0; u < kWin; ++u) {
            const int ri = base + u;
            if (ri < kRowsIn) {
                float(*bd)[kRowW] = s_d[ri & 1];
#pragma unroll
                for (int q = 0; q < 3; ++q) store_row(bd[q], nd[q]);
                __syncthreads();
                if (ri + 1 < kRowsIn) {
#pragma unroll
                    for (int q = 0; q < 3; ++q) nd[q] = load_row(ds[q], a.H, a.W, x0, y0 - kR + ri + 1);
                }
                float m[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t = 0; t < kWin; ++t) {
                    const float w = c_win[t];
#pragma unroll
                    for (int q = 0; q < 3; ++q) m[q] += w * bd[q][c + t];
                }
#pragma unroll
                for (int q = 0; q < 3; ++q) ring[u][q] = m[q];
                const int ro = ri - 2 * kR;
                const int py = y0 + ro;
                if (ro >= 0 && px < a.W && py < a.H) {
                    float v[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int t = 0; t < kWin; ++t) {
                        const float w = c_win[t];
#pragma unroll
                        for (int q = 0; q < 3; ++q) v[q] += w * ring[(u + 1 + t) % kWin][q];
                    }
                    const size_t i = poff + (size_t)py * a.W + px;
                    const float xv = a.x[i], yv = a.y[i];
                    const float dssim = (v[0] + 2.0f * xv * v[1] + yv * v[2]) * inv_n;
                    const float sgn = xv > yv ? 1.0f : (xv < yv ? -1.0f : 0.0f);
                    a.grad[i] = (1.0f - a.lambda) * sgn * inv_n - a.lambda * dssim;
                }
            }
        }
    }
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
    const size_t blocks = (size_t)((W + kSW - 1) / kSW) * ((H + kSH - 1) / kSH) * frames * 3;
    return ((maps + 255) & ~(size_t)255) + blocks * sizeof(double2);
}

hipError_t launch_image_loss(const float* image, const float* target, int32_t frames, int32_t H, int32_t W,
                             float lambda, void* ws, double* loss, float* grad, hipStream_t s) {
    const int planes = frames * 3;
    const size_t n = (size_t)planes * H * W;
    const size_t maps = ((3 * n * sizeof(float)) + 255) & ~(size_t)255;
    double2* part = reinterpret_cast<double2*>((char*)ws + maps);
    LossArgs a{image, target, H, W, lambda, 1.0 / (double)n, reinterpret_cast<float*>(ws), n, part, grad};
    const dim3 grid((W + kSW - 1) / kSW, (H + kSH - 1) / kSH, planes);
    const int64_t nblocks = (int64_t)grid.x * grid.y * grid.z;
    IA_LAUNCH("ssim_fwd_kernel", ssim_fwd_kernel, grid, dim3(kSW), 0, s, a);
    IA_LAUNCH("ssim_bwd_kernel", ssim_bwd_kernel, grid, dim3(kSW), 0, s, a);
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
