// Spatial order of the positions of each frame (a storage layout, not a step
// of the method).  The position sets of a sequence are fixed once refined
// (SPIN-4DGS page, §3.2: every frame is its own set of positions), and the
// order of the Gaussians inside a frame changes neither a decoded attribute
// nor a composited pixel (compositing follows depth, with ties in index
// order).  It does change the hash gather's memory traffic: Gaussians that
// are close in space share grid cells on the coarse levels, and when they sit
// in the same wave their corner loads fall into the same cache lines.  This
// computes, for every frame, the order of its Gaussians along a Morton curve
// of the normalised positions x~ of Eq. 7 (the space the hash grid lives in).
//
// Key of Gaussian i of frame f, local index j = i - frame_offsets[f]:
//   (f << (3 a + l)) | (morton_a(x~) << l) | j
// with l bits for the largest frame, a bits per axis (10, fewer only when the
// three fields would not fit 64 bits).  A stable radix sort on the bits above
// j keeps frames contiguous and in order, and equal Morton cells in index
// order.
#include <hip/hip_runtime.h>

#include "decode_common.h"
#include "ia_internal.h"

namespace ia {
namespace {

constexpr int kOrderBlock = 256;

__device__ __forceinline__ int order_frame_of(const int64_t* fo, int F, int64_t i) {
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

// The low 10 bits of v spread to every third bit (bit k -> bit 3k).
__device__ __forceinline__ uint32_t spread3(uint32_t v) {
    v &= 0x3ffu;
    v = (v | (v << 16)) & 0x030000ffu;
    v = (v | (v << 8)) & 0x0300f00fu;
    v = (v | (v << 4)) & 0x030c30c3u;
    v = (v | (v << 2)) & 0x09249249u;
    return v;
}

struct OrderArgs {
    const float* pos;
    int stride;
    int64_t N;
    const int64_t* fo;
    int F;
    int lbits;  // bits of the local index
    int abits;  // bits per axis of the Morton code
    uint64_t* words;
};

__global__ void __launch_bounds__(kOrderBlock) order_keys_kernel(OrderArgs a) {
    for (int64_t i = (int64_t)blockIdx.x * kOrderBlock + threadIdx.x; i < a.N;
         i += (int64_t)gridDim.x * kOrderBlock) {
        const int f = order_frame_of(a.fo, a.F, i);
        const uint64_t local = (uint64_t)(i - a.fo[f]);
        const float* p = a.pos + i * a.stride;
        float xt[4];
        normalize_pos(p[0], p[1], p[2], 0.0f, 0.0f, 1.0f, xt);
        const float scale = (float)(1u << a.abits);
        const uint32_t top = (1u << a.abits) - 1u;
        uint32_t q[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const float v = xt[k] * scale;  // x~ in [0, 1] (non-finite input: cell 0)
            q[k] = v >= 1.0f ? min((uint32_t)v, top) : 0u;
        }
        const uint64_t morton = (uint64_t)spread3(q[0]) | ((uint64_t)spread3(q[1]) << 1) |
                                ((uint64_t)spread3(q[2]) << 2);
        a.words[i] = ((uint64_t)f << (3 * a.abits + a.lbits)) | (morton << a.lbits) | local;
    }
}

__global__ void __launch_bounds__(kOrderBlock) order_apply_kernel(const uint64_t* words, int64_t N, const int64_t* fo,
                                                                  int shift_f, int lbits, const float* pos,
                                                                  int stride, uint32_t* perm, float* pos_out) {
    for (int64_t i = (int64_t)blockIdx.x * kOrderBlock + threadIdx.x; i < N; i += (int64_t)gridDim.x * kOrderBlock) {
        const uint64_t w = words[i];
        const int f = (int)(w >> shift_f);
        const int64_t g = fo[f] + (int64_t)(w & ((1ull << lbits) - 1ull));
        perm[i] = (uint32_t)g;
        if (pos_out)
            for (int k = 0; k < stride; ++k) pos_out[i * stride + k] = pos[g * stride + k];
    }
}

int bits_for(int64_t n) {
    int b = 0;
    while (b < 63 && ((int64_t)1 << b) < n) ++b;
    return b;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct OrderLayout {
    size_t fo, count, w0, w1, counts, digit_tot, total;
    int max_blocks;
};

OrderLayout order_layout(int64_t N, int frames) {
    OrderLayout L{};
    const int64_t n = N > 0 ? N : 1;
    L.max_blocks = radix_sort_blocks(n);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    L.fo = take(sizeof(int64_t) * (size_t)(frames + 1));
    L.count = take(sizeof(uint64_t));
    L.w0 = take(sizeof(uint64_t) * (size_t)n);
    L.w1 = take(sizeof(uint64_t) * (size_t)n);
    L.counts = take(radix_sort_counts_bytes(L.max_blocks));
    L.digit_tot = take(4 * 1024);
    L.total = off;
    return L;
}

}  // namespace

size_t spatial_order_workspace(int64_t N, int frames) { return order_layout(N, frames).total; }

hipError_t launch_spatial_order(const float* pos, int stride, int64_t N, const int64_t* frame_offsets_host, int frames,
                                uint32_t* perm, float* pos_out, void* ws, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    const OrderLayout L = order_layout(N, frames);
    unsigned char* w = static_cast<unsigned char*>(ws);
    int64_t* fo = reinterpret_cast<int64_t*>(w + L.fo);
    uint64_t* count = reinterpret_cast<uint64_t*>(w + L.count);
    uint64_t* buf[2] = {reinterpret_cast<uint64_t*>(w + L.w0), reinterpret_cast<uint64_t*>(w + L.w1)};
    hipError_t e = upload(fo, frame_offsets_host, sizeof(int64_t) * (size_t)(frames + 1), s);
    if (e != hipSuccess) return e;
    const uint64_t n64 = (uint64_t)N;
    if ((e = upload(count, &n64, sizeof(n64), s)) != hipSuccess) return e;
    int64_t largest = 1;
    for (int f = 0; f < frames; ++f)
        largest = frame_offsets_host[f + 1] - frame_offsets_host[f] > largest
                      ? frame_offsets_host[f + 1] - frame_offsets_host[f]
                      : largest;
    const int lbits = bits_for(largest);
    const int fbits = bits_for(frames);
    int abits = (64 - lbits - fbits) / 3;
    if (abits > 10) abits = 10;
    if (abits < 1) return hipErrorInvalidValue;
    const int grid = (int)((N + kOrderBlock - 1) / kOrderBlock < 16384 ? (N + kOrderBlock - 1) / kOrderBlock : 16384);
    OrderArgs a{pos, stride, N, fo, frames, lbits, abits, buf[0]};
    IA_LAUNCH("order_keys_kernel", order_keys_kernel, dim3(grid), dim3(kOrderBlock), 0, s, a);
    const int cur = radix_sort_u64(buf, count, n64, lbits, 3 * abits + fbits, L.max_blocks,
                                   reinterpret_cast<uint32_t*>(w + L.counts), reinterpret_cast<uint32_t*>(w + L.digit_tot),
                                   s);
    IA_LAUNCH("order_apply_kernel", order_apply_kernel, dim3(grid), dim3(kOrderBlock), 0, s, buf[cur], N, fo,
              3 * abits + lbits, lbits, pos, stride, perm, pos_out);
    return hipGetLastError();
}

}  // namespace ia
