// Tile rasteriser for 3D Gaussians (SPIN-4DGS, "Implicit 4D Gaussian
// Splatting for Fast Motion with Large Inter-Frame Displacements", §3.1):
// Eq. 2 covariance from scale and quaternion, Eq. 3 EWA projection to a 2D
// conic, Eq. 1 / Eq. 4 front-to-back alpha compositing, on 16x16-pixel tiles.
//
// Pipeline for a batch of frames (all kernels on one stream, no host sync):
//   preprocess  one thread per Gaussian: project, cull, conic, 3-sigma tile
//               rect, tiles touched; per-block count of visible Gaussians
//   order       visible Gaussians compacted in index order and radix-sorted
//               (stable, four 8-bit digits) on their 31 depth bits
//   scan        two-level exclusive prefix sum of the tiles touched, in that
//               depth order; the total entry count stays in device memory
//   emit        each block spreads its Gaussians' entries over all its
//               threads: (frame*tiles + tile) << 32 | Gaussian index, in
//               depth order
//   sort        stable LSD radix sort of the entries on the tile bits only,
//               digits of up to 10 bits (two of 9 for 18 tile bits); per pass: per-block digit
//               histograms, a per-digit scan over blocks, and a stable
//               scatter ranked by wave ballots.  Because the input is in
//               (depth, index) order, the result is ordered by the key
//               (tile << 32 | depth bits) with ties in index order
//   ranges      [start, end) of every tile in the sorted list
//   raster      one 256-thread block per tile; Gaussians staged through LDS
//               in batches of 256; per pixel the 3-sigma test, alpha =
//               min(0.99, o G), skip alpha < 1/255, stop once T < 1e-4; a wave
//               whose pixels are all saturated skips the batch (ballot), and
//               the block stops once every pixel is.
//
// Projection runs one IEEE fp32 operation at a time in source order (the
// library is built with -ffp-contract=off, and '/' and sqrt are correctly
// rounded), which makes tile rects and depth keys reproducible bit for bit.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "ia_internal.h"
#include "raster_common.h"

namespace ia {
namespace {

constexpr int kBlock = 256;
constexpr int kSortItems = 16;                     // keys per thread per sort tile
constexpr int kSortTile = kBlock * kSortItems;     // 4096
constexpr int kScanChunk = 1024;                   // block sums per second-level group

// ---------------------------------------------------------------- helpers

struct Payload {
    uint32_t w[896];
};

__global__ void upload_kernel(uint32_t* dst, Payload p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = p.w[i];
}

}  // namespace

hipError_t upload(void* dst, const void* src, size_t bytes, hipStream_t s) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(src);
    size_t words = (bytes + 3) / 4;
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);
    for (size_t off = 0; off < words; off += 896) {
        Payload p;
        int n = (int)(words - off < 896 ? words - off : 896);
        for (int i = 0; i < n; ++i) p.w[i] = w[off + i];
        IA_LAUNCH("upload_kernel", upload_kernel, dim3(1), dim3(256), 0, s, d + off, p, n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

namespace {

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__device__ __forceinline__ int frame_of(const int64_t* fo, int F, int64_t i) {
    int lo = 0, hi = F - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (fo[mid] <= i)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Inclusive wave-level prefix sum (wave64).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        T o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

// Exclusive block-level prefix sum over 256 threads; returns the block total.
template <typename T>
__device__ __forceinline__ T block_excl_scan(T v, T& total) {
    __shared__ T s_w[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    T inc = wave_incl_scan(v);
    if (lane == 63) s_w[w] = inc;
    __syncthreads();
    T off = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        T x = s_w[k];
        if (k < w) off += x;
        tot += x;
    }
    __syncthreads();
    total = tot;
    return off + inc - v;
}

// ---------------------------------------------------------------- preprocess

struct PreArgs {
    const float* means;
    int stride;
    const float* scales;
    const float* quats;
    const float* colors;
    const float* sh;
    const float* opacity;
    int sh_degree;
    const DevCamera* cams;
    const int64_t* fo;
    int F;
    int64_t N;
    float4* pa;
    float4* pb;
    float* pc;
    float* depth;
    ushort4* rect;
    uint32_t* tiles;
    uint32_t* bsum;    // per block: visible Gaussians
    uint32_t* bsum_t;  // per block: tiles touched
};

__global__ void __launch_bounds__(kBlock) preprocess_kernel(PreArgs a) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    uint32_t ntouch = 0;
    if (i < a.N) {
        const DevCamera& cam = a.cams[frame_of(a.fo, a.F, i)];
        const float* mu = a.means + i * a.stride;
        const float* R = cam.R;
        const float m0 = mu[0], m1 = mu[1], m2 = mu[2];
        float px = R[0] * m0 + R[1] * m1;
        px = px + R[2] * m2;
        px = px + cam.t[0];
        float py = R[3] * m0 + R[4] * m1;
        py = py + R[5] * m2;
        py = py + cam.t[1];
        float pz = R[6] * m0 + R[7] * m1;
        pz = pz + R[8] * m2;
        pz = pz + cam.t[2];
        bool vis = pz > cam.near_z;
        float u = 0, v = 0, A = 0, B = 0, C = 0;
        int x0 = 0, x1 = -1, y0 = 0, y1 = -1;
        if (vis) {
            const float* q = a.quats + i * 4;
            const float* s = a.scales + i * 3;
            float qn = q[0] * q[0] + q[1] * q[1];
            qn = qn + q[2] * q[2];
            qn = qn + q[3] * q[3];
            qn = sqrtf(qn);
            const float w = q[0] / qn, x = q[1] / qn, y = q[2] / qn, z = q[3] / qn;
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
            float M[9];
#pragma unroll
            for (int r = 0; r < 3; ++r)
#pragma unroll
                for (int k = 0; k < 3; ++k) M[r * 3 + k] = Rq[r * 3 + k] * s[k];
            // Eq. 2: Sigma = (R S)(R S)^T
            float S[9];
#pragma unroll
            for (int r = 0; r < 3; ++r)
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    float acc = M[r * 3 + 0] * M[k * 3 + 0] + M[r * 3 + 1] * M[k * 3 + 1];
                    S[r * 3 + k] = acc + M[r * 3 + 2] * M[k * 3 + 2];
                }
            // Eq. 3: Sigma2D = J W Sigma W^T J^T with T = J W (2x3)
            const float zz = pz * pz;
            const float j00 = cam.fx / pz;
            const float j02 = -(cam.fx * px) / zz;
            const float j11 = cam.fy / pz;
            const float j12 = -(cam.fy * py) / zz;
            float T[6];
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                T[k] = j00 * R[k] + j02 * R[6 + k];
                T[3 + k] = j11 * R[3 + k] + j12 * R[6 + k];
            }
            float U[6];
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    float acc = T[r * 3 + 0] * S[0 * 3 + k] + T[r * 3 + 1] * S[1 * 3 + k];
                    U[r * 3 + k] = acc + T[r * 3 + 2] * S[2 * 3 + k];
                }
            float c2[4];
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    float acc = U[r * 3 + 0] * T[k * 3 + 0] + U[r * 3 + 1] * T[k * 3 + 1];
                    c2[r * 2 + k] = acc + U[r * 3 + 2] * T[k * 3 + 2];
                }
            const float ca = c2[0], cb = c2[1], cc = c2[3];
            const float det = ca * cc - cb * cb;
            vis = det > 0.0f;
            if (vis) {
                const float inv = 1.0f / det;
                A = cc * inv;
                B = -cb * inv;
                C = ca * inv;
                const float mid = 0.5f * (ca + cc);
                float disc = mid * mid - det;
                disc = disc > 0.0f ? disc : 0.0f;
                const float lam = mid + sqrtf(disc);
                const float rr = ceilf(3.0f * sqrtf(lam));
                u = (cam.fx * px) / pz + cam.cx;
                v = (cam.fy * py) / pz + cam.cy;
                vis = isfinite(u) && isfinite(v) && isfinite(A) && isfinite(B) && isfinite(C) && isfinite(rr);
                if (vis) {
                    float fx0 = ceilf((u - rr) - 0.5f), fx1 = floorf((u + rr) - 0.5f);
                    float fy0 = ceilf((v - rr) - 0.5f), fy1 = floorf((v + rr) - 0.5f);
                    fx0 = fx0 > 0.0f ? fx0 : 0.0f;
                    fy0 = fy0 > 0.0f ? fy0 : 0.0f;
                    fx1 = fx1 < (float)(cam.W - 1) ? fx1 : (float)(cam.W - 1);
                    fy1 = fy1 < (float)(cam.H - 1) ? fy1 : (float)(cam.H - 1);
                    vis = fx0 <= fx1 && fy0 <= fy1;
                    if (vis) {
                        x0 = (int)fx0 >> 4;
                        x1 = (int)fx1 >> 4;
                        y0 = (int)fy0 >> 4;
                        y1 = (int)fy1 >> 4;
                    }
                }
            }
        }
        float r = 0, g = 0, b = 0, o = 0;
        if (vis) {
            o = a.opacity[i];
            if (a.sh_degree == 3) {
                float d0 = m0 - cam.centre[0], d1 = m1 - cam.centre[1], d2 = m2 - cam.centre[2];
                const float inv = 1.0f / sqrtf(d0 * d0 + d1 * d1 + d2 * d2);
                float Y[16];
                sh_basis16(d0 * inv, d1 * inv, d2 * inv, Y);
                const float* shc = a.sh + i * 48;
                float acc[3] = {0.5f, 0.5f, 0.5f};
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    acc[0] += shc[k * 3 + 0] * Y[k];
                    acc[1] += shc[k * 3 + 1] * Y[k];
                    acc[2] += shc[k * 3 + 2] * Y[k];
                }
                r = fmaxf(acc[0], 0.0f);
                g = fmaxf(acc[1], 0.0f);
                b = fmaxf(acc[2], 0.0f);
            } else {
                r = a.colors[i * 3 + 0];
                g = a.colors[i * 3 + 1];
                b = a.colors[i * 3 + 2];
            }
            ntouch = (uint32_t)((x1 - x0 + 1) * (y1 - y0 + 1));
        }
        // the projection of a culled Gaussian is never read (every reader
        // starts from tiles > 0 or from a tile list): only its zero tile
        // count is written, which saves most of the stores of a frame
        if (vis) {
            a.pa[i] = make_float4(u, v, A, B);
            a.pb[i] = make_float4(C, o, r, g);
            a.pc[i] = b;
            a.depth[i] = pz;
            a.rect[i] = make_ushort4((unsigned short)x0, (unsigned short)y0, (unsigned short)x1, (unsigned short)y1);
        }
        a.tiles[i] = ntouch;
    }
    uint32_t total, total_t;
    block_excl_scan<uint32_t>(ntouch > 0 ? 1u : 0u, total);
    block_excl_scan<uint32_t>(ntouch, total_t);
    if (threadIdx.x == 0) {
        a.bsum[blockIdx.x] = total;
        a.bsum_t[blockIdx.x] = total_t;
    }
}

// ---------------------------------------------------------------- scan of block sums

__global__ void __launch_bounds__(kBlock) scan_reduce_kernel(const uint32_t* bsum, int nb1, uint64_t* bsum2) {
    uint64_t v = 0;
    const int base = blockIdx.x * kScanChunk;
#pragma unroll
    for (int k = 0; k < kScanChunk / kBlock; ++k) {
        int idx = base + k * kBlock + threadIdx.x;
        if (idx < nb1) v += bsum[idx];
    }
    uint64_t total;
    block_excl_scan<uint64_t>(v, total);
    if (threadIdx.x == 0) bsum2[blockIdx.x] = total;
}

__global__ void __launch_bounds__(kBlock) scan_top_kernel(uint64_t* bsum2, int nb2, uint64_t cap, uint64_t* nent,
                                                          uint64_t* nent_out, uint32_t* ovf_out) {
    uint64_t carry = 0;
    for (int base = 0; base < nb2; base += kBlock) {
        int idx = base + threadIdx.x;
        uint64_t v = idx < nb2 ? bsum2[idx] : 0;
        uint64_t total;
        uint64_t ex = block_excl_scan<uint64_t>(v, total);
        if (idx < nb2) bsum2[idx] = carry + ex;
        carry += total;
    }
    if (threadIdx.x == 0) {
        nent[0] = carry;
        nent[1] = carry > cap ? 1 : 0;
        if (nent_out) *nent_out = carry;
        if (ovf_out) *ovf_out = carry > cap ? 1u : 0u;
    }
}

__global__ void __launch_bounds__(kBlock) scan_down_kernel(const uint32_t* bsum, int nb1, const uint64_t* bsum2,
                                                           uint64_t* boff) {
    const int base = blockIdx.x * kScanChunk;
    uint64_t carry = bsum2[blockIdx.x];
#pragma unroll
    for (int k = 0; k < kScanChunk / kBlock; ++k) {
        int idx = base + k * kBlock + threadIdx.x;
        uint64_t v = idx < nb1 ? bsum[idx] : 0;
        uint64_t total;
        uint64_t ex = block_excl_scan<uint64_t>(v, total);
        if (idx < nb1) boff[idx] = carry + ex;
        carry += total;
    }
}

// ---------------------------------------------------------------- depth order of the visible Gaussians

// Visible Gaussians (tiles touched > 0) of block b land at boff[b] + their
// rank in the block, as the word depth_bits << 32 | index.  Depth is > 0, so
// its bit pattern orders like the float and bit 63 stays clear.
__global__ void __launch_bounds__(kBlock) compact_kernel(const uint32_t* tiles, const float* depth, int64_t N,
                                                         const uint64_t* boff, uint64_t* gkeys) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const bool vis = i < N && tiles[i] > 0;
    uint32_t total;
    const uint32_t ex = block_excl_scan<uint32_t>(vis ? 1u : 0u, total);
    if (vis) gkeys[boff[blockIdx.x] + ex] = ((uint64_t)__float_as_uint(depth[i]) << 32) | (uint32_t)i;
}

// ---------------------------------------------------------------- binning
//
// Two ways to turn the depth-ordered Gaussians into per-tile lists, chosen on
// the device from the mean number of tiles a visible Gaussian touches (or
// forced per call through ia_render_aux.binning):
//
// Tile sort (small footprints): one entry (frame*tiles + tile) << 32 | index
// per (Gaussian, tile), emitted in depth order, then a stable radix sort on
// the tile bits; tile ranges from the sorted keys.
//
// Regions (large footprints): a region is kRegion x kRegion tiles of one frame.  Every visible Gaussian
// gets one coarse entry per region its tile rect overlaps, emitted in depth
// order; a stable radix sort on the region index then lists, per region, its
// Gaussians in (depth, index) order.  Work items of kItemCoarse consecutive
// coarse entries of one region expand them into per-tile entries: one pass
// counts entries per (item, tile), scans give every tile its range and every
// item its offset inside each tile, a second pass writes each entry at its
// final position.  The tile lists come out in (depth, index) order without a
// sort over the per-tile entries.
constexpr int kRegion = 8;
constexpr int kRegionTiles = kRegion * kRegion;  // 64: one lane per tile of a region
constexpr int kItemCoarse = 256;                 // coarse entries per work item
constexpr uint64_t kRegionFootprint = 4;         // tiles per visible Gaussian from which regions are used

enum : uint64_t { kModeTiles = 0, kModeRegions = 1 };

__device__ __forceinline__ uint32_t region_span(uint32_t a0, uint32_t a1) { return a1 / kRegion - a0 / kRegion + 1; }

// mode[0] = binning used by this call (force: 0 automatic, 1 tile sort, 2 regions)
__global__ void binning_mode_kernel(const uint64_t* nent, const uint64_t* nvis, int force, uint64_t* mode) {
    if (threadIdx.x != 0) return;
    uint64_t m = nent[0] >= kRegionFootprint * nvis[0] ? kModeRegions : kModeTiles;
    if (force == 1) m = kModeTiles;
    if (force == 2) m = kModeRegions;
    mode[0] = m;
}

__device__ __forceinline__ uint32_t entries_of(ushort4 r, uint64_t mode) {
    return mode == kModeRegions ? region_span(r.x, r.z) * region_span(r.y, r.w)
                                : ((uint32_t)r.z - r.x + 1) * ((uint32_t)r.w - r.y + 1);
}

// Per block of 256 depth-ordered Gaussians: their tile rects in that order
// (one gather) and their entries (tiles touched, or regions overlapped).
__global__ void __launch_bounds__(kBlock) sorted_rects_kernel(const uint64_t* gkeys, const uint64_t* nvis,
                                                              const uint64_t* mode, const ushort4* rect,
                                                              ushort4* srect, uint32_t* bsum) {
    const uint64_t j = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    uint32_t n = 0;
    if (j < nvis[0]) {
        const ushort4 r = rect[(uint32_t)gkeys[j]];
        srect[j] = r;
        n = entries_of(r, mode[0]);
    }
    uint32_t total;
    block_excl_scan<uint32_t>(n, total);
    if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

// Entries are emitted `per` per block whatever the Gaussians' sizes
// (depth order groups the large near Gaussians).
constexpr int kEmitMax = 16384;  // entries per emission block, at most (at least kBlock)

struct GInfo {
    uint32_t off;  // first entry (clamped to the capacity)
    uint32_t idx;  // Gaussian index
    uint32_t lo;   // tile rect x0 | y0 << 16
    uint32_t hi;   // tile rect x1 | y1 << 16
};

struct OffsetArgs {
    const uint64_t* gkeys;
    const uint64_t* nvis;
    const uint64_t* mode;
    const ushort4* srect;
    const uint64_t* boff;
    uint64_t cap;
    uint32_t nemit;    // emission blocks
    uint32_t per;      // entries per emission block
    const int64_t* fo;
    int F;
    GInfo* info;
    uint32_t* frame;   // per depth-ordered Gaussian: its frame
    uint32_t* bstart;  // per emission block: the Gaussian holding its first entry
};

// Frame offsets searched in LDS (the depth-ordered Gaussians of a block come
// from any frame, so every lane searches on its own): up to this many frames,
// with offsets below 2^32; beyond, the search reads global memory.
constexpr int kLdsFrames = 2047;

__device__ __forceinline__ int frame_of_lds(const uint32_t* fo, int F, uint32_t i) {
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

__global__ void __launch_bounds__(kBlock) offsets_kernel(OffsetArgs a) {
    __shared__ uint32_t s_fo[kLdsFrames + 1];
    const bool lds_fo = a.F <= kLdsFrames && a.fo[a.F] <= (int64_t)0xffffffffu;
    if (lds_fo)
        for (int k = threadIdx.x; k <= a.F; k += kBlock) s_fo[k] = (uint32_t)a.fo[k];
    __syncthreads();
    const uint64_t j = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const bool live = j < a.nvis[0];
    ushort4 r = make_ushort4(0, 0, 0, 0);
    uint32_t n = 0;
    if (live) {
        r = a.srect[j];
        n = entries_of(r, a.mode[0]);
    }
    uint32_t total;
    const uint32_t ex = block_excl_scan<uint32_t>(n, total);
    if (!live) return;
    const uint64_t off = a.boff[blockIdx.x] + ex, stop = off + n;
    GInfo g;
    g.off = (uint32_t)(off < a.cap ? off : a.cap);
    g.idx = (uint32_t)a.gkeys[j];
    g.lo = (uint32_t)r.x | ((uint32_t)r.y << 16);
    g.hi = (uint32_t)r.z | ((uint32_t)r.w << 16);
    a.info[j] = g;
    a.frame[j] = (uint32_t)(lds_fo ? frame_of_lds(s_fo, a.F, g.idx) : frame_of(a.fo, a.F, g.idx));
    // emission blocks whose first entry lies in [off, stop)
    for (uint64_t b = (off + a.per - 1) / a.per; b * a.per < stop && b < a.nemit; ++b)
        a.bstart[b] = (uint32_t)j;
}

struct EmitArgs {
    const GInfo* info;
    const uint32_t* frame;
    const uint64_t* nvis;
    const uint64_t* mode;
    const uint32_t* bstart;
    const uint64_t* nsort;  // entries to emit
    uint64_t cap;
    uint32_t per;           // entries per block
    int tiles_x;
    uint32_t ntiles;
    uint32_t regions_x;
    uint32_t regions_per_frame;
    uint64_t* ents;  // tile sort: tile << 32 | Gaussian index; regions: region << 32 | depth-order position
};

__global__ void __launch_bounds__(kBlock) emit_kernel(EmitArgs a) {
    __shared__ uint32_t s_off[kBlock + 1];
    __shared__ uint32_t s_next;
    const bool regions = a.mode[0] == kModeRegions;
    uint64_t Ecap = a.nsort[0];
    if (Ecap > a.cap) Ecap = a.cap;
    const uint64_t e0 = (uint64_t)blockIdx.x * a.per;
    if (e0 >= Ecap) return;
    const uint64_t e1 = e0 + a.per < Ecap ? e0 + a.per : Ecap;
    const uint64_t nv = a.nvis[0];
    uint64_t jc = a.bstart[blockIdx.x];  // Gaussian holding entry ec
    for (uint64_t ec = e0; ec < e1; ec += kBlock) {
        // offsets of the (at most 257) Gaussians that can hold this chunk's entries
        for (int k = threadIdx.x; k <= kBlock; k += kBlock)
            s_off[k] = jc + k < nv ? a.info[jc + k].off : 0xffffffffu;
        __syncthreads();
        const uint32_t e = (uint32_t)(ec + threadIdx.x);
        if (ec + threadIdx.x < e1) {
            int lo = 0, hi = kBlock;  // last k with s_off[k] <= e
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_off[mid] <= e)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const uint64_t j = jc + lo;
            const GInfo g = a.info[j];
            const uint32_t f = a.frame[j];
            const uint32_t k = e - g.off;
            if (regions) {
                const uint32_t gx0 = (g.lo & 0xffffu) / kRegion, gy0 = (g.lo >> 16) / kRegion;
                const uint32_t w = (g.hi & 0xffffu) / kRegion - gx0 + 1;
                const uint32_t row = k / w, col = k - row * w;
                const uint64_t region = (uint64_t)f * a.regions_per_frame + (gy0 + row) * a.regions_x + gx0 + col;
                a.ents[e] = (region << 32) | (uint32_t)j;
            } else {
                const uint32_t x0 = g.lo & 0xffffu, y0 = g.lo >> 16;
                const uint32_t w = (g.hi & 0xffffu) - x0 + 1;
                const uint32_t row = k / w, col = k - row * w;
                const uint64_t tile = (uint64_t)f * a.ntiles + (y0 + row) * (uint32_t)a.tiles_x + x0 + col;
                a.ents[e] = (tile << 32) | g.idx;
            }
        }
        if (threadIdx.x == 0) {
            const uint32_t next = (uint32_t)(ec + kBlock);
            int lo = 0, hi = kBlock;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_off[mid] <= next)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            s_next = (uint32_t)lo;
        }
        __syncthreads();
        jc += s_next;
    }
}

// ---------------------------------------------------------------- radix sort

// One stable LSD pass over 64-bit words on the digit (word >> shift) &
// (2^bits - 1), bits <= 10.  Items: the first min(*count, cap) words.
constexpr int kMaxDigitBits = 10;
constexpr int kMaxBuckets = 1 << kMaxDigitBits;

struct SortPass {
    const uint64_t* in;
    uint64_t* out;
    const uint64_t* count;
    uint64_t cap;
    int shift;
    int bits;
    int nblocks;
    uint32_t* counts;     // [buckets][nblocks]
    uint32_t* digit_tot;  // [buckets]
};

__device__ __forceinline__ void sort_chunk(const SortPass& p, uint32_t& begin, uint32_t& end) {
    uint64_t E = p.count[0];
    if (E > p.cap) E = p.cap;
    uint64_t per = (E + p.nblocks - 1) / p.nblocks;
    per = (per + kSortTile - 1) / kSortTile * kSortTile;
    uint64_t b = (uint64_t)blockIdx.x * per, e = b + per;
    if (b > E) b = E;
    if (e > E) e = E;
    begin = (uint32_t)b;
    end = (uint32_t)e;
}

template <int MAXB>
__global__ void __launch_bounds__(kBlock) sort_upsweep_kernel(SortPass p) {
    // per-wave histograms, [4][nb] flat, and one spare slot that counts the
    // lanes past the end of the chunk
    __shared__ uint32_t hist[(4 << MAXB) + 1];
    const int w = threadIdx.x >> 6;
    const int nb = 1 << p.bits;
    const uint32_t mask = (uint32_t)nb - 1u;
    for (int k = threadIdx.x; k <= 4 * nb; k += kBlock) hist[k] = 0;
    __syncthreads();
    uint32_t begin, end;
    sort_chunk(p, begin, end);
    for (uint32_t tile = begin; tile < end; tile += kSortTile) {
        // all 16 loads are issued before the first count: the index is
        // clamped (tile < end) and every lane counts, the ones past the end
        // in the spare slot
        uint32_t slot[kSortItems];
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const uint32_t idx = tile + j * kBlock + threadIdx.x;
            const uint64_t v = p.in[idx < end ? idx : end - 1];
            const uint32_t d = (uint32_t)(v >> p.shift) & mask;
            // past the end: pushed to the spare slot by arithmetic, not by a
            // select on the loaded value (which the compiler would turn into
            // a branch around the load)
            const uint32_t past = idx < end ? 0u : 0x7fffffffu;
            slot[j] = min(w * nb + d + past, (uint32_t)(4 * nb));
        }
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            // a wave whose lanes all count the same slot (common for the top
            // digit of depth keys) adds its 64 with one atomic instead of 64
            // conflicting ones
            const uint32_t s0 = __builtin_amdgcn_readfirstlane(slot[j]);
            if (__ballot(slot[j] != s0) == 0ull) {
                if ((threadIdx.x & 63) == 0) atomicAdd(&hist[s0], 64u);
            } else {
                atomicAdd(&hist[slot[j]], 1u);
            }
        }
    }
    __syncthreads();
    for (int d = threadIdx.x; d < nb; d += kBlock)
        p.counts[d * p.nblocks + blockIdx.x] = hist[d] + hist[nb + d] + hist[2 * nb + d] + hist[3 * nb + d];
}

// One block per digit: exclusive scan of that digit's counts over blocks.
__global__ void __launch_bounds__(kBlock) sort_scan_kernel(SortPass p) {
    uint32_t* c = p.counts + blockIdx.x * p.nblocks;
    uint32_t carry = 0;
    for (int base = 0; base < p.nblocks; base += kBlock) {
        int idx = base + threadIdx.x;
        uint32_t v = idx < p.nblocks ? c[idx] : 0;
        uint32_t total;
        uint32_t ex = block_excl_scan<uint32_t>(v, total);
        if (idx < p.nblocks) c[idx] = carry + ex;
        carry += total;
    }
    if (threadIdx.x == 0) p.digit_tot[blockIdx.x] = carry;
}

// Stable scatter.  Sort tile = 4 waves x 16 steps x 64 lanes, item order
// wave-major then step then lane (the chunk order).  Per step each lane finds
// the lanes holding the same digit with one ballot per digit bit; its rank is
// the count of such lanes below it plus the wave's running count for the
// digit.  The tile is then laid out in LDS in digit order and written back
// with consecutive threads on consecutive destinations, so each digit's items
// leave as one contiguous run instead of one scattered word per lane.
// MAXB: the largest digit width the instance handles (sizes its LDS).  All
// 16 key loads of a thread are issued before the first is used; the grid is
// one round of resident blocks (three per CU), which the occupancy allows
// because the next tile's keys are not held in registers.
// Thread t owns digits [t kDPT, (t + 1) kDPT): it keeps their global
// destinations in registers and, per tile, turns the per-wave counts into
// tile-local starts (s_wc) and destination offsets (s_off = global
// destination - tile-local start), so placing an item in the tile and
// writing it out take one LDS lookup each.
template <int MAXB>
__global__ void __launch_bounds__(kBlock, 3) sort_downsweep_kernel(SortPass p) {
    constexpr int kNB = 1 << MAXB;
    constexpr int kDPT = kNB > kBlock ? kNB / kBlock : 1;  // digits per thread
    __shared__ uint64_t s_stage[kSortTile];
    __shared__ uint32_t s_off[kNB];
    __shared__ uint4 s_wc4[kNB];  // per-wave counters, [4][nb] flat
    uint32_t* s_wc = reinterpret_cast<uint32_t*>(s_wc4);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nb = 1 << p.bits;
    const uint32_t mask = (uint32_t)nb - 1u;
    const int d0 = threadIdx.x * kDPT;
    uint32_t base[kDPT];  // global destination of the next item of each owned digit
    {
        // exclusive scan of the digit totals + this block's offset within the digit
        uint32_t v[kDPT], sum = 0;
#pragma unroll
        for (int k = 0; k < kDPT; ++k) {
            v[k] = d0 + k < nb ? p.digit_tot[d0 + k] : 0u;
            sum += v[k];
        }
        uint32_t total;
        uint32_t run = block_excl_scan<uint32_t>(sum, total);
#pragma unroll
        for (int k = 0; k < kDPT; ++k) {
            base[k] = d0 + k < nb ? run + p.counts[(d0 + k) * p.nblocks + blockIdx.x] : 0u;
            run += v[k];
        }
    }
    uint32_t begin, end;
    sort_chunk(p, begin, end);
    const uint64_t end_all = p.count[0] < p.cap ? p.count[0] : p.cap;  // bound on every destination
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (uint32_t tile = begin; tile < end; tile += kSortTile) {
        uint64_t key[kSortItems];
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            // clamped so that every load is issued unconditionally (tile < end)
            const uint32_t idx = tile + w * (64 * kSortItems) + j * 64 + lane;
            key[j] = p.in[idx < end ? idx : end - 1];
        }
        for (int k = threadIdx.x; k < nb; k += kBlock) s_wc4[k] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
        // digit << 16 | rank within the wave's items of that digit (rank < 4096);
        // digit 0xffff marks an item past the end
        uint32_t dr[kSortItems];
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const uint32_t idx = tile + w * (64 * kSortItems) + j * 64 + lane;
            const bool valid = idx < end;
            const uint32_t d = (uint32_t)(key[j] >> p.shift) & mask;
            uint64_t peers = __ballot(valid);
            // bits at and above p.bits are zero in every lane's digit and
            // leave peers unchanged
#pragma unroll
            for (int bit = 0; bit < MAXB; ++bit) {
                const uint64_t b = __ballot((d >> bit) & 1u);
                peers &= ((d >> bit) & 1u) ? b : ~b;
            }
            uint32_t prior = 0;
            if (valid) prior = s_wc[w * nb + d];
            const uint32_t below = (uint32_t)__popcll(peers & lt_mask);
            // the lowest lane of each peer group advances the wave's counter
            if (valid && below == 0) s_wc[w * nb + d] = prior + (uint32_t)__popcll(peers);
            dr[j] = ((valid ? d : 0xffffu) << 16) | (prior + below);
        }
        __syncthreads();
        // per owned digit: the tile-local start of each wave's items (tile
        // start + counts of the waves before), and the destination offset
        {
            uint32_t c[kDPT][4], tc[kDPT], sum = 0;
#pragma unroll
            for (int k = 0; k < kDPT; ++k) {
                const int d = d0 + k;
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) c[k][ww] = d < nb ? s_wc[ww * nb + d] : 0u;
                tc[k] = c[k][0] + c[k][1] + c[k][2] + c[k][3];
                sum += tc[k];
            }
            uint32_t total;
            uint32_t run = block_excl_scan<uint32_t>(sum, total);
#pragma unroll
            for (int k = 0; k < kDPT; ++k) {
                const int d = d0 + k;
                if (d < nb) {
                    s_wc[d] = run;
                    s_wc[nb + d] = run + c[k][0];
                    s_wc[2 * nb + d] = run + c[k][0] + c[k][1];
                    s_wc[3 * nb + d] = run + c[k][0] + c[k][1] + c[k][2];
                    s_off[d] = base[k] - run;
                    base[k] += tc[k];
                }
                run += tc[k];
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kSortItems; ++j)
            if ((dr[j] >> 16) <= mask) s_stage[s_wc[w * nb + (dr[j] >> 16)] + (dr[j] & 0xffffu)] = key[j];
        __syncthreads();
        const uint32_t n = end - tile < (uint32_t)kSortTile ? end - tile : (uint32_t)kSortTile;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const uint32_t pos = j * kBlock + threadIdx.x;
            if (pos < n) {
                const uint64_t k = s_stage[pos];
                const uint32_t d = (uint32_t)(k >> p.shift) & mask;
                const uint32_t dst = s_off[d] + pos;
                if (dst < end_all) p.out[dst] = k;
            }
        }
    }
}

// ---------------------------------------------------------------- tile ranges

// A tile starts where its key differs from the previous one; the previous
// key comes from the neighbouring lane.
// Runs only when mode[0] == want; with vals, also splits off the low words.
__global__ void __launch_bounds__(kBlock) ranges_kernel(const uint64_t* keys, const uint64_t* nent, uint64_t cap,
                                                        uint2* ranges, uint32_t ntiles_all, uint32_t* vals,
                                                        const uint64_t* mode, uint64_t want) {
    if (mode[0] != want) return;
    uint64_t E = nent[0];
    if (E > cap) E = cap;
    const int lane = threadIdx.x & 63;
    for (uint64_t i0 = (uint64_t)blockIdx.x * kBlock; i0 < E; i0 += (uint64_t)gridDim.x * kBlock) {
        const uint64_t i = i0 + threadIdx.x;
        const bool valid = i < E;
        const uint64_t key = valid ? keys[i] : ~0ull;
        const uint32_t t = (uint32_t)(key >> 32);
        if (vals && valid) vals[i] = (uint32_t)key;
        uint32_t tp = __shfl_up(t, 1, 64);
        if (lane == 0) tp = (valid && i > 0) ? (uint32_t)(keys[i - 1] >> 32) : 0xffffffffu;
        if (valid && (i == 0 || t != tp)) {
            // t >= ntiles_all cannot happen for emitted keys; the checks keep a bad key in bounds
            if (t < ntiles_all) ranges[t].x = (uint32_t)i;
            if (i > 0 && tp < ntiles_all) ranges[tp].y = (uint32_t)i;
        }
        if (i + 1 == E && t < ntiles_all) ranges[t].y = (uint32_t)E;
    }
}

// ---------------------------------------------------------------- per-tile lists from regions

// Per block of 256 regions: work items (kItemCoarse coarse entries each).
__global__ void __launch_bounds__(kBlock) region_items_kernel(const uint64_t* mode, const uint2* rranges, uint32_t nreg, uint32_t* bsum) {
    if (mode[0] != kModeRegions) return;
    const uint32_t r = blockIdx.x * kBlock + threadIdx.x;
    uint32_t n = 0;
    if (r < nreg) {
        const uint2 rr = rranges[r];
        n = (rr.y - rr.x + kItemCoarse - 1) / kItemCoarse;
    }
    uint32_t total;
    block_excl_scan<uint32_t>(n, total);
    if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

// Item table: item -> (region, segment); per region its first item.
__global__ void __launch_bounds__(kBlock) region_expand_kernel(const uint64_t* mode, const uint2* rranges, uint32_t nreg,
                                                               const uint64_t* boff, uint64_t max_items,
                                                               uint2* items, uint32_t* rfirst) {
    if (mode[0] != kModeRegions) return;
    const uint32_t r = blockIdx.x * kBlock + threadIdx.x;
    uint32_t n = 0;
    if (r < nreg) {
        const uint2 rr = rranges[r];
        n = (rr.y - rr.x + kItemCoarse - 1) / kItemCoarse;
    }
    uint32_t total;
    const uint32_t ex = block_excl_scan<uint32_t>(n, total);
    if (r >= nreg) return;
    const uint64_t base = boff[blockIdx.x] + ex;
    rfirst[r] = (uint32_t)base;
    for (uint32_t s = 0; s < n && base + s < max_items; ++s) items[base + s] = make_uint2(r, s);
}

struct ExpandArgs {
    const uint64_t* mode;
    const uint2* items;
    const uint64_t* nitems;  // [0] = work items
    const uint2* rranges;
    const uint64_t* coarse;  // sorted coarse entries
    const GInfo* info;
    uint32_t regions_x;
    uint32_t regions_per_frame;
    int tiles_x, tiles_y;
    uint32_t ntiles;
    uint32_t* cnt;            // [item][64]: entries per tile, then the item's offset inside the tile
    const uint32_t* tstart;   // per tile: first entry
    uint64_t cap;
    uint32_t* vals;
};

// One wave per work item.  Its coarse entries are taken 64 at a time; lane l
// clips Gaussian l's tile rect to the region (w x h tiles), a wave scan
// flattens the chunk's entries (Gaussian-major, then rows, then columns) and
// each lane finds the owner of its entry by a binary search over the lanes'
// offsets (cross-lane reads).  WRITE = false counts entries per region tile;
// WRITE = true ranks each entry among the item's entries of the same tile
// (one ballot per bit of the 6-bit tile index) and stores the Gaussian index
// at its final position.
constexpr int kStage = 2048;  // entries staged per chunk of a work item (LDS, per wave)

// One work item on one wave.  Coarse entries are taken up to 64 at a time,
// as many as keep the chunk within kStage entries; lane l clips Gaussian l's
// tile rect to the region.  Eight ballots over the lanes whose clip covers a
// region column and eight over those covering a row give, intersected, the
// lanes covering each of the 64 region tiles: the tile's count in the chunk
// and, below each lane, that lane's rank among them (the lanes are in depth
// order), so no per-entry search is needed.
// WRITE = false: entries per region tile of the item.
// WRITE = true: the chunk's per-tile counts give each tile a segment of the
// stage; every (lane, tile) entry goes to its slot and the stage is written
// out with consecutive lanes on consecutive positions of a tile's list.
template <bool WRITE>
__device__ __forceinline__ void expand_item(const ExpandArgs& a, uint64_t item, int lane, uint32_t* stage,
                                            uint8_t* tof) {
    const uint2 it = a.items[item];
    const uint32_t r = it.x;
    const uint2 rr = a.rranges[r];
    const uint32_t cb = rr.x + it.y * kItemCoarse;
    const uint32_t ce = cb + kItemCoarse < rr.y ? cb + kItemCoarse : rr.y;
    const uint32_t f = r / a.regions_per_frame, rl = r - f * a.regions_per_frame;
    const uint32_t ox = (rl % a.regions_x) * kRegion, oy = (rl / a.regions_x) * kRegion;
    uint32_t basev = 0;  // lane t: next position of this item's entries of region tile t
    if (WRITE) {
        const uint32_t tx = ox + (lane % kRegion), ty = oy + (lane / kRegion);
        if (tx < (uint32_t)a.tiles_x && ty < (uint32_t)a.tiles_y)
            basev = a.tstart[f * a.ntiles + ty * (uint32_t)a.tiles_x + tx] + a.cnt[item * kRegionTiles + lane];
    }
    uint32_t total = 0;  // lane t: entries of region tile t in the item so far (count pass)
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (uint32_t k0 = cb; k0 < ce;) {
        const uint32_t k = k0 + lane;
        // clip [cx0, cx1] x [cy0, cy1] in region tile coordinates; empty for lanes past the item
        uint32_t cx0 = 1, cy0 = 1, cx1 = 0, cy1 = 0, n = 0, gidx = 0;
        if (k < ce) {
            const GInfo g = a.info[(uint32_t)a.coarse[k]];
            const uint32_t x0 = g.lo & 0xffffu, y0 = g.lo >> 16, x1 = g.hi & 0xffffu, y1 = g.hi >> 16;
            cx0 = (x0 > ox ? x0 : ox) - ox;
            cy0 = (y0 > oy ? y0 : oy) - oy;
            cx1 = (x1 < ox + kRegion - 1 ? x1 : ox + kRegion - 1) - ox;
            cy1 = (y1 < oy + kRegion - 1 ? y1 : oy + kRegion - 1) - oy;
            n = (cx1 - cx0 + 1) * (cy1 - cy0 + 1);
            gidx = g.idx;
        }
        uint32_t take = 64;
        if (WRITE) {
            // lanes [0, take) fit the stage (the inclusive count is non-decreasing; lane 0 always fits)
            const uint32_t incl = wave_incl_scan(n);
            take = (uint32_t)__popcll(__ballot(incl <= (uint32_t)kStage));
            if ((uint32_t)lane >= take) cx0 = 1, cx1 = 0;
        }
        // lanes whose clip covers region column x / row y; the lanes covering
        // tile (x, y) are the intersection of the two masks
        uint64_t colm[kRegion], rowm[kRegion];
#pragma unroll
        for (int x = 0; x < kRegion; ++x) colm[x] = __ballot(cx0 <= (uint32_t)x && (uint32_t)x <= cx1);
#pragma unroll
        for (int y = 0; y < kRegion; ++y) rowm[y] = __ballot(cy0 <= (uint32_t)y && (uint32_t)y <= cy1);
        // lane t: entries of region tile t in this chunk
        uint64_t cm = 0ull, rm = 0ull;
#pragma unroll
        for (int x = 0; x < kRegion; ++x) {
            cm = lane % kRegion == x ? colm[x] : cm;
            rm = lane / kRegion == x ? rowm[x] : rm;
        }
        const uint32_t c = (uint32_t)__popcll(cm & rm);
        if (!WRITE) {
            total += c;
        } else {
            const uint32_t choff = wave_incl_scan(c) - c;  // tile's segment in the stage
            const uint32_t m = __shfl(choff + c, 63, 64);
#pragma unroll 8
            for (int t = 0; t < kRegionTiles; ++t) {
                const uint64_t mk = colm[t % kRegion] & rowm[t / kRegion];
                if (mk == 0ull) continue;
                const uint32_t seg = __builtin_amdgcn_readlane(choff, t);
                if ((mk >> lane) & 1ull) {
                    // rank among the covering lanes below this one (depth order)
                    const uint32_t below =
                        __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
                    stage[seg + below] = gidx;
                    tof[seg + below] = (uint8_t)t;
                }
            }
            asm volatile("" ::: "memory");
            for (uint32_t s0 = 0; s0 < m; s0 += 64) {
                const uint32_t slot = s0 + lane;
                const int t = slot < m ? tof[slot] : 0;
                const uint32_t pos = __shfl(basev, t, 64) + (slot - __shfl(choff, t, 64));
                if (slot < m && pos < a.cap) a.vals[pos] = stage[slot];
            }
            basev += c;
            asm volatile("" ::: "memory");
        }
        k0 += take;
    }
    if (!WRITE) a.cnt[item * kRegionTiles + lane] = total;
}

template <bool WRITE>
__global__ void __launch_bounds__(kBlock) expand_kernel(ExpandArgs a) {
    if (a.mode[0] != kModeRegions) return;
    __shared__ uint32_t s_stage[WRITE ? 4 : 1][WRITE ? kStage : 1];
    __shared__ uint8_t s_tof[WRITE ? 4 : 1][WRITE ? kStage : 1];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t nitems = a.nitems[0];
    for (uint64_t item = (uint64_t)blockIdx.x * 4 + w; item < nitems; item += (uint64_t)gridDim.x * 4)
        expand_item<WRITE>(a, item, lane, s_stage[WRITE ? w : 0], s_tof[WRITE ? w : 0]);
}


// One wave per region: lane t turns the per-item counts of region tile t into
// the items' offsets inside the tile (exclusive scan over the region's items)
// and writes the tile's entry count.
__global__ void __launch_bounds__(kBlock) region_tiles_kernel(const uint64_t* mode, const uint2* rranges, const uint32_t* rfirst,
                                                              uint32_t nreg, uint32_t regions_x,
                                                              uint32_t regions_per_frame, int tiles_x, int tiles_y,
                                                              uint32_t ntiles, uint64_t max_items, uint32_t* cnt,
                                                              uint32_t* tcount) {
    if (mode[0] != kModeRegions) return;
    const int lane = threadIdx.x & 63;
    const uint32_t r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= nreg) return;
    const uint2 rr = rranges[r];
    const uint32_t n = (rr.y - rr.x + kItemCoarse - 1) / kItemCoarse;
    const uint64_t first = rfirst[r];
    uint32_t run = 0;
    for (uint32_t s = 0; s < n && first + s < max_items; ++s) {
        uint32_t* c = cnt + (first + s) * kRegionTiles + lane;
        const uint32_t v = *c;
        *c = run;
        run += v;
    }
    const uint32_t f = r / regions_per_frame, rl = r - f * regions_per_frame;
    const uint32_t tx = (rl % regions_x) * kRegion + (lane % kRegion);
    const uint32_t ty = (rl / regions_x) * kRegion + (lane / kRegion);
    if (tx < (uint32_t)tiles_x && ty < (uint32_t)tiles_y) tcount[f * ntiles + ty * (uint32_t)tiles_x + tx] = run;
}

// Per block of 256 tiles: entries.
__global__ void __launch_bounds__(kBlock) tile_sums_kernel(const uint64_t* mode, const uint32_t* tcount, int64_t ntiles_all, uint32_t* bsum) {
    if (mode[0] != kModeRegions) return;
    const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    uint32_t total;
    block_excl_scan<uint32_t>(t < ntiles_all ? tcount[t] : 0u, total);
    if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

// Tile ranges [start, start + count) (empty tiles [0, 0)) and first entries.
__global__ void __launch_bounds__(kBlock) tile_ranges_kernel(const uint64_t* mode, const uint32_t* tcount, int64_t ntiles_all,
                                                             const uint64_t* boff, uint64_t cap, uint32_t* tstart,
                                                             uint2* ranges) {
    if (mode[0] != kModeRegions) return;
    const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint32_t c = t < ntiles_all ? tcount[t] : 0u;
    uint32_t total;
    const uint32_t ex = block_excl_scan<uint32_t>(c, total);
    if (t >= ntiles_all) return;
    uint64_t s = boff[blockIdx.x] + ex, e = s + c;
    if (s > cap) s = cap;
    if (e > cap) e = cap;
    tstart[t] = (uint32_t)s;
    ranges[t] = c ? make_uint2((uint32_t)s, (uint32_t)e) : make_uint2(0u, 0u);
}

// Sorted (tile << 32 | depth bits) keys of the entries, one block per tile.
__global__ void __launch_bounds__(kBlock) unpack_kernel(const uint2* ranges, const uint32_t* vals, const float* depth,
                                                        int64_t N, uint64_t* keys) {
    const uint64_t t = blockIdx.x + (uint64_t)gridDim.x * blockIdx.y;
    const uint2 rg = ranges[t];
    for (uint32_t i = rg.x + threadIdx.x; i < rg.y; i += kBlock) {
        const uint32_t g = vals[i];
        keys[i] = (t << 32) | ((int64_t)g < N ? __float_as_uint(depth[g]) : 0u);
    }
}

// ---------------------------------------------------------------- raster

struct RasterArgs {
    const uint2* ranges;
    const uint32_t* vals;  // per-tile lists of Gaussian indices
    const float4* pa;
    const float4* pb;
    const float* pc;
    const DevCamera* cams;
    int W, H, tiles_x;
    uint32_t ntiles;
    uint64_t cap;
    int64_t N;
    float* image;
    float* T_final;
    uint32_t* n_contrib;
};

// Per-pixel compositing state and one front-to-back step (Eq. 4).  A
// Gaussian that is skipped (power outside [-4.5, 0] i.e. beyond 3 sigma,
// alpha below 1/255, or the pixel already saturated) contributes alpha = 0,
// which leaves C and T exactly unchanged, so the step has no branches.
// A pixel's compositing state.  It is saturated ("done") exactly when
// T < 1e-4: T only decreases, the step that takes T below the threshold is
// the last one composited, and a pixel outside the image starts at T = 0.
struct Pix {
    float T, r, g, b;
    uint32_t last;
};

__device__ __forceinline__ bool pix_done(const Pix& p) { return p.T < 1e-4f; }

// LAST: track the index of the last composited Gaussian (the n_contrib output).
template <bool LAST>
__device__ __forceinline__ void composite_step(Pix& p, float power, float opacity, float cr, float cg, float cb,
                                               uint32_t pos) {
#pragma clang fp contract(fast)
    const float a0 = splat_alpha(opacity, power);
    const bool take = !pix_done(p) && splat_takes(power, a0);
    const float alpha = take ? a0 : 0.0f;
    const float wgt = alpha * p.T;
    p.r += cr * wgt;
    p.g += cg * wgt;
    p.b += cb * wgt;
    p.T = p.T * (1.0f - alpha);
    if (LAST) p.last = take ? pos : p.last;
}

// Whether a staged Gaussian (ga = mean, A', B'; gbx = C'; p2 = A' dx^2 +
// C' dy^2 + B' dx dy, the base-2 power) can pass the per-pixel 3-sigma test
// p2 >= -4.5 log2(e) = -Q at some pixel centre of a wave, whose centres lie
// in [X0, X1] x [Y0, Y1].  q = -p2 is convex: its minimum over the box is 0
// when the box holds the mean, else it lies on an edge, where q is a parabola
// in the free coordinate, minimised at its vertex clamped to the edge.  The
// offsets a pixel computes lie in the box the offsets of its corners span
// (rounding is monotonic), so a pixel whose computed p2 is >= -Q has q <= Q +
// e there, and the computed minimum exceeds the exact one by at most e', with
// e, e' a few units of fp32 rounding of M = |A'| dx^2 + |C'| dy^2 + |B' dx dy|
// over the box (about 15 u M in all, u = 2^-24).  The test allows 4e-6 M +
// 1.5e-4: it never rejects a Gaussian the per-pixel test would take, only
// spares the wave the Gaussians that cannot reach it.  Degenerate or
// non-finite values pass.
__device__ __forceinline__ bool may_reach(float4 ga, float gbx, float X0, float X1, float Y0, float Y1) {
#pragma clang fp contract(fast)
    const float x0 = X0 - ga.x, x1 = X1 - ga.x, y0 = Y0 - ga.y, y1 = Y1 - ga.y;
    if (x0 <= 0.0f && x1 >= 0.0f && y0 <= 0.0f && y1 >= 0.0f) return true;
    const float a = -ga.z, b = -ga.w, c = -gbx;
    if (!(a > 1e-30f && c > 1e-30f)) return true;
    const float ia = 0.5f / a, ic = 0.5f / c;
    auto q = [&](float dx, float dy) { return (a * dx * dx + c * dy * dy) + b * dx * dy; };
    auto clampf = [](float v, float lo, float hi) { return fminf(fmaxf(v, lo), hi); };
    float m = q(x0, clampf(-b * x0 * ic, y0, y1));
    m = fminf(m, q(x1, clampf(-b * x1 * ic, y0, y1)));
    m = fminf(m, q(clampf(-b * y0 * ia, x0, x1), y0));
    m = fminf(m, q(clampf(-b * y1 * ia, x0, x1), y1));
    const float xm = fmaxf(fabsf(x0), fabsf(x1)), ym = fmaxf(fabsf(y0), fabsf(y1));
    const float M = (a * xm * xm + c * ym * ym) + fabsf(b) * xm * ym;
    return !(m > -kPower2Min + 4e-6f * M + 1.5e-4f);
}

// One block per 16x16 tile.  PX = 2: 128 threads, thread (col, row) shades
// pixels (col, 2 row) and (col, 2 row + 1), which share dx and the dx terms
// of power, so a wave covers a 16 x 8 pixel block; PX = 1: 256 threads, one
// pixel each (twice the waves, for launches with few tiles).
// Gaussians of the tile's list are staged in LDS 256 at a time with the
// conic pre-scaled to the base-2 power (kConicScaleA, kConicScaleB), so p2 =
// A' dx^2 + C' dy^2 + B' dx dy = log2(e) power.  After staging, each wave marks with may_reach the batch's
// Gaussians that can reach one of its pixels (four per lane, one ballot per
// 64) and visits only those, in list order.  A wave leaves a batch once all
// its pixels are saturated; the block stops once all 256 are.
constexpr int kRasterBatch = 256;
constexpr int kRasterCheck = 8;  // Gaussians between two saturation checks of a wave
constexpr int64_t kRasterTwoPixelTiles = 8192;  // tiles per launch from which two pixels per thread pay

template <int PX, bool LAST>
__global__ void __launch_bounds__(256 / PX) raster_kernel(RasterArgs a) {
#pragma clang fp contract(fast)
    constexpr int kThreads = 256 / PX;
    static_assert(kRasterBatch % kThreads == 0, "every thread stages the same number of Gaussians");
    __shared__ float4 s_a[kRasterBatch];
    __shared__ float4 s_b[kRasterBatch];
    // third colour channel, at the same 16-byte stride as s_a and s_b so that one
    // address serves all three reads of a Gaussian
    __shared__ float4 s_c[kRasterBatch];
    const int f = blockIdx.z;
    const uint32_t tile = (uint32_t)f * a.ntiles + blockIdx.y * (uint32_t)a.tiles_x + blockIdx.x;
    uint2 rg = a.ranges[tile];
    if (rg.y > a.cap) rg.y = (uint32_t)a.cap;
    if (rg.x > rg.y) rg.x = rg.y;
    const int px = blockIdx.x * 16 + (threadIdx.x & 15);
    const int py0 = blockIdx.y * 16 + PX * (threadIdx.x >> 4);
    const float fx = (float)px + 0.5f;
    // this wave's pixel centres: 16 columns, 4 PX rows
    const int lane = threadIdx.x & 63;
    const float wx0 = (float)(blockIdx.x * 16) + 0.5f, wx1 = wx0 + 15.0f;
    const float wy0 = (float)(blockIdx.y * 16 + 4 * PX * (int)(threadIdx.x >> 6)) + 0.5f, wy1 = wy0 + (float)(4 * PX - 1);
    Pix p[PX];
    bool in[PX];
#pragma unroll
    for (int k = 0; k < PX; ++k) {
        in[k] = px < a.W && py0 + k < a.H;
        p[k] = Pix{in[k] ? 1.0f : 0.0f, 0.0f, 0.0f, 0.0f, 0u};
    }
    auto all_done = [&]() {
        bool d = true;
#pragma unroll
        for (int k = 0; k < PX; ++k) d = d && pix_done(p[k]);
        return d;
    };
    for (uint32_t start = rg.x; start < rg.y; start += kRasterBatch) {
        if (__syncthreads_count(all_done()) == kThreads) break;
#pragma unroll
        for (int k = 0; k < kRasterBatch / kThreads; ++k) {
            const uint32_t slot = threadIdx.x + k * kThreads;
            const uint32_t idx = start + slot;
            if (idx < rg.y) {
                uint32_t gid = a.vals[idx];
                if ((int64_t)gid >= a.N) gid = 0;  // cannot happen for a valid sort; keeps reads in bounds
                const float4 pa = a.pa[gid], pb = a.pb[gid];
                s_a[slot] = make_float4(pa.x, pa.y, kConicScaleA * pa.z, kConicScaleB * pa.w);
                s_b[slot] = make_float4(kConicScaleA * pb.x, pb.y, pb.z, pb.w);
                s_c[slot].x = a.pc[gid];
            }
        }
        __syncthreads();
        const int n = (int)min((uint32_t)kRasterBatch, rg.y - start);
        const uint32_t pos0 = start - rg.x + 1u;
        uint64_t hit[kRasterBatch / 64];
#pragma unroll
        for (int r = 0; r < kRasterBatch / 64; ++r) {
            const int j = r * 64 + lane;
            hit[r] = r * 64 < n ? __ballot(j < n && may_reach(s_a[j], s_b[j].x, wx0, wx1, wy0, wy1)) : 0ull;
        }
        // A wave whose pixels are all saturated leaves the batch; that is
        // checked before every kRasterCheck-th Gaussian it visits
        // (compositing ignores saturated pixels, so the check only saves work).
        bool live = true;
        int since = 0;
#pragma unroll
        for (int r = 0; r < kRasterBatch / 64; ++r) {
            uint64_t mm = hit[r];
            while (live && mm != 0ull) {
                if (since == 0 && __ballot(!all_done()) == 0ull) {
                    live = false;
                    break;
                }
                since = since + 1 == kRasterCheck ? 0 : since + 1;
                const int j = r * 64 + (int)__builtin_ctzll(mm);
                mm &= mm - 1ull;
                const float4 ga = s_a[j];
                const float4 gb = s_b[j];
                const float gcb = s_c[j].x;
                const float dx = fx - ga.x;
                float ta, tb;
                splat_dx_terms(ga.z, ga.w, dx, ta, tb);
                float pw[PX];
#pragma unroll
                for (int k = 0; k < PX; ++k) {
                    const float dy = ((float)(py0 + k) + 0.5f) - ga.y;
                    pw[k] = splat_power(ta, tb, gb.x, dy);
                }
                // (no wave-wide test that some pixel is within 3 sigma before
                // compositing: the compositing step leaves a pixel outside
                // unchanged, and the branch cost more than the steps it saved)
#pragma unroll
                for (int k = 0; k < PX; ++k) composite_step<LAST>(p[k], pw[k], gb.y, gb.z, gb.w, gcb, pos0 + (uint32_t)j);
            }
        }
    }
    const DevCamera& cam = a.cams[f];
    const size_t plane = (size_t)a.W * a.H;
    float* img = a.image + (size_t)f * 3 * plane;
#pragma unroll
    for (int k = 0; k < PX; ++k) {
        if (!in[k]) continue;
        const size_t pix = (size_t)(py0 + k) * a.W + px;
        img[pix] = p[k].r + p[k].T * cam.bg[0];
        img[plane + pix] = p[k].g + p[k].T * cam.bg[1];
        img[2 * plane + pix] = p[k].b + p[k].T * cam.bg[2];
        if (a.T_final) a.T_final[(size_t)f * plane + pix] = p[k].T;
        if (LAST && a.n_contrib) a.n_contrib[(size_t)f * plane + pix] = p[k].last;
    }
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Blocks of the kBlock-thread kernel K the whole device holds at once (its
// occupancy times the CU count), cached per kernel; 1024 if the runtime
// cannot tell.
template <auto K>
int resident_blocks() {
    static int cached = 0;
    if (cached > 0) return cached;
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, K, kBlock, 0) != hipSuccess || cus <= 0 || per <= 0)
        return 1024;
    cached = cus * per;
    return cached;
}

int grid_cap(int64_t n, int per, int cap) {
    int64_t g = (n + per - 1) / per;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

}  // namespace

// LSD passes over bits [lo, lo + nbits) of the first min(*count, cap) 64-bit
// words of buf[0], digits of at most kMaxDigitBits bits, ping-ponging between
// buf[0] and buf[1]; returns the index of the buffer holding the result.
// counts: 4 * kMaxBuckets * max_blocks bytes, digit_tot: 4 * kMaxBuckets.
int radix_sort_u64(uint64_t* const* buf, const uint64_t* count, uint64_t cap, int lo, int nbits, int max_blocks,
                   uint32_t* counts, uint32_t* digit_tot, hipStream_t s) {
    const int passes = (nbits + kMaxDigitBits - 1) / kMaxDigitBits;
    const int bits = (nbits + passes - 1) / passes;
    int cur = 0;
    for (int pass = 0; pass < passes; ++pass) {
        SortPass sp{buf[cur], buf[cur ^ 1], count, cap, lo + pass * bits, bits, max_blocks, counts, digit_tot};
        auto run = [&](auto digit_bits) {
            constexpr int B = decltype(digit_bits)::value;
            // one round of resident blocks: every block takes an equal chunk
            const int r = resident_blocks<sort_downsweep_kernel<B>>();
            sp.nblocks = max_blocks < r ? max_blocks : r;
            IA_LAUNCH("sort_upsweep_kernel", sort_upsweep_kernel<B>, dim3(sp.nblocks), dim3(kBlock), 0, s, sp);
            IA_LAUNCH("sort_scan_kernel", sort_scan_kernel, dim3(1 << bits), dim3(kBlock), 0, s, sp);
            IA_LAUNCH("sort_downsweep_kernel", sort_downsweep_kernel<B>, dim3(sp.nblocks), dim3(kBlock), 0, s, sp);
        };
        if (bits <= 8)
            run(std::integral_constant<int, 8>{});
        else if (bits == 9)
            run(std::integral_constant<int, 9>{});
        else
            run(std::integral_constant<int, kMaxDigitBits>{});
        cur ^= 1;
    }
    return cur;
}

int radix_sort_blocks(int64_t items) {
    const int64_t b = (items + kSortTile - 1) / kSortTile;
    return (int)(b < 1 ? 1 : (b > 1024 ? 1024 : b));
}

size_t radix_sort_counts_bytes(int max_blocks) { return 4 * (size_t)kMaxBuckets * (size_t)max_blocks; }


RenderLayout render_layout(int64_t N, int frames, int W, int H, int64_t max_entries) {
    RenderLayout L{};
    L.N = N;
    L.cap = max_entries;
    L.frames = frames;
    L.tiles_x = (W + 15) / 16;
    L.tiles_y = (H + 15) / 16;
    L.ntiles_all = (int64_t)frames * L.tiles_x * L.tiles_y;
    L.regions_x = (L.tiles_x + kRegion - 1) / kRegion;
    L.regions_y = (L.tiles_y + kRegion - 1) / kRegion;
    L.nreg = (int64_t)frames * L.regions_x * L.regions_y;
    const int64_t n1 = N > 0 ? N : 1;
    const int64_t cap1 = max_entries > 0 ? max_entries : 1;
    L.nb1 = (int)((n1 + kBlock - 1) / kBlock);
    L.nbr = (int)((L.nreg + kBlock - 1) / kBlock);
    L.nbt = (int)((L.ntiles_all + kBlock - 1) / kBlock);
    int nbmax = L.nb1 > L.nbr ? L.nb1 : L.nbr;
    nbmax = nbmax > L.nbt ? nbmax : L.nbt;
    auto blocks = [](int64_t items) {
        int64_t b = (items + kSortTile - 1) / kSortTile;
        return (int)(b < 1 ? 1 : (b > 1024 ? 1024 : b));
    };
    L.sort_blocks_g = blocks(n1);
    L.sort_blocks_e = blocks(cap1);
    // about 65536 emission blocks of a power of two entries each, kBlock..kEmitMax:
    // a block's chunks of kBlock entries run one after another (each starts
    // with a global read of Gaussian offsets), so short blocks keep that
    // chain short (22.7M entries: 512 per block 0.157 ms, 2048 0.164 ms,
    // 16384 0.209 ms; 256 per block 0.173 ms)
    L.emit_per = kBlock;
    while (L.emit_per < kEmitMax && (int64_t)L.emit_per * 65536 < cap1) L.emit_per *= 2;
    L.nemit = (int)((cap1 + L.emit_per - 1) / L.emit_per);
    // coarse entries <= tile entries <= capacity, so items <= cap / kItemCoarse + regions
    L.max_items = (cap1 + kItemCoarse - 1) / kItemCoarse + L.nreg;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    L.cams = take(sizeof(DevCamera) * frames);
    L.fo = take(sizeof(int64_t) * (frames + 1));
    L.pa = take(16 * (size_t)n1);
    L.pb = take(16 * (size_t)n1);
    L.pc = take(4 * (size_t)n1);
    L.depth = take(4 * (size_t)n1);
    L.rect = take(8 * (size_t)n1);
    L.tiles = take(4 * (size_t)n1);
    L.bsum = take(4 * (size_t)nbmax);
    L.bsum_t = take(4 * (size_t)L.nb1);
    L.bsum2 = take(8 * (size_t)((nbmax + kScanChunk - 1) / kScanChunk));
    L.boff = take(8 * (size_t)nbmax);
    L.srect = take(8 * (size_t)n1);
    L.ginfo = take(sizeof(GInfo) * (size_t)n1);
    L.gframe = take(4 * (size_t)n1);
    L.bstart = take(4 * (size_t)L.nemit);
    L.gk0 = take(8 * (size_t)n1);
    L.gk1 = take(8 * (size_t)n1);
    L.ent0 = take(8 * (size_t)cap1);
    L.ent1 = take(8 * (size_t)cap1);
    L.vals = take(4 * (size_t)cap1);
    L.counts = take(4 * (size_t)kMaxBuckets *
                    (size_t)(L.sort_blocks_g > L.sort_blocks_e ? L.sort_blocks_g : L.sort_blocks_e));
    L.digit_tot = take(4 * (size_t)kMaxBuckets);
    L.rranges = take(8 * (size_t)L.nreg);
    L.rfirst = take(4 * (size_t)L.nreg);
    L.items = take(8 * (size_t)L.max_items);
    L.icnt = take(4 * (size_t)kRegionTiles * (size_t)L.max_items);
    L.tcount = take(4 * (size_t)L.ntiles_all);
    L.tstart = take(4 * (size_t)L.ntiles_all);
    L.ranges = take(8 * (size_t)L.ntiles_all);
    L.counters = take(128);
    L.gacc = take(4 * (size_t)kGradPerGaussian * (size_t)n1);
    L.total = off;
    return L;
}

hipError_t launch_render(const RenderArgs& a, hipStream_t s, const uint64_t** keys_out, const uint32_t** vals_out) {
    const RenderLayout& L = a.lay;
    unsigned char* ws = a.ws;
    DevCamera* cams = reinterpret_cast<DevCamera*>(ws + L.cams);
    int64_t* fo = reinterpret_cast<int64_t*>(ws + L.fo);
    hipError_t e = upload(cams, a.cams_host, sizeof(DevCamera) * a.frames, s);
    if (e != hipSuccess) return e;
    e = upload(fo, a.frame_offsets_host, sizeof(int64_t) * (a.frames + 1), s);
    if (e != hipSuccess) return e;

    float4* pa = reinterpret_cast<float4*>(ws + L.pa);
    float4* pb = reinterpret_cast<float4*>(ws + L.pb);
    float* pc = reinterpret_cast<float*>(ws + L.pc);
    float* depth = reinterpret_cast<float*>(ws + L.depth);
    ushort4* rect = reinterpret_cast<ushort4*>(ws + L.rect);
    uint32_t* tiles = reinterpret_cast<uint32_t*>(ws + L.tiles);
    uint32_t* bsum = reinterpret_cast<uint32_t*>(ws + L.bsum);
    uint32_t* bsum_t = reinterpret_cast<uint32_t*>(ws + L.bsum_t);
    uint64_t* bsum2 = reinterpret_cast<uint64_t*>(ws + L.bsum2);
    uint64_t* boff = reinterpret_cast<uint64_t*>(ws + L.boff);
    ushort4* srect = reinterpret_cast<ushort4*>(ws + L.srect);
    GInfo* ginfo = reinterpret_cast<GInfo*>(ws + L.ginfo);
    uint32_t* gframe = reinterpret_cast<uint32_t*>(ws + L.gframe);
    uint32_t* bstart = reinterpret_cast<uint32_t*>(ws + L.bstart);
    uint64_t* gk[2] = {reinterpret_cast<uint64_t*>(ws + L.gk0), reinterpret_cast<uint64_t*>(ws + L.gk1)};
    uint64_t* ent[2] = {reinterpret_cast<uint64_t*>(ws + L.ent0), reinterpret_cast<uint64_t*>(ws + L.ent1)};
    uint32_t* vals = reinterpret_cast<uint32_t*>(ws + L.vals);
    uint32_t* counts = reinterpret_cast<uint32_t*>(ws + L.counts);
    uint32_t* digit_tot = reinterpret_cast<uint32_t*>(ws + L.digit_tot);
    uint2* rranges = reinterpret_cast<uint2*>(ws + L.rranges);
    uint32_t* rfirst = reinterpret_cast<uint32_t*>(ws + L.rfirst);
    uint2* items = reinterpret_cast<uint2*>(ws + L.items);
    uint32_t* icnt = reinterpret_cast<uint32_t*>(ws + L.icnt);
    uint32_t* tcount = reinterpret_cast<uint32_t*>(ws + L.tcount);
    uint32_t* tstart = reinterpret_cast<uint32_t*>(ws + L.tstart);
    uint2* ranges = reinterpret_cast<uint2*>(ws + L.ranges);
    uint64_t* ctr = reinterpret_cast<uint64_t*>(ws + L.counters);
    uint64_t* nent = ctr;         // [0] tile entries, [1] overflow
    uint64_t* nvis = ctr + 2;     // visible Gaussians
    uint64_t* nsort = ctr + 4;    // entries emitted for sorting (tile or region entries)
    uint64_t* nitems = ctr + 6;   // work items
    uint64_t* mode = ctr + 10;    // binning of this call
    const int64_t N = L.N;
    const uint64_t cap = (uint64_t)L.cap;
    const uint32_t ntiles = (uint32_t)(L.tiles_x * L.tiles_y);
    const uint32_t rpf = (uint32_t)(L.regions_x * L.regions_y);
    constexpr uint64_t kNoCap = ~0ull;

    // exclusive scan of per-block sums: per-block offsets (when boff_out) and
    // the total (with the capacity check when outputs are given)
    auto scan = [&](const uint32_t* bs, int nb, uint64_t limit, uint64_t* total, uint64_t* total_out,
                    uint32_t* ovf_out, uint64_t* boff_out) {
        const int nb2 = (nb + kScanChunk - 1) / kScanChunk;
        IA_LAUNCH("scan_reduce_kernel", scan_reduce_kernel, dim3(nb2), dim3(kBlock), 0, s, bs, nb, bsum2);
        IA_LAUNCH("scan_top_kernel", scan_top_kernel, dim3(1), dim3(kBlock), 0, s, bsum2, nb2, limit, total,
                  total_out, ovf_out);
        if (boff_out)
            IA_LAUNCH("scan_down_kernel", scan_down_kernel, dim3(nb2), dim3(kBlock), 0, s, bs, nb, bsum2, boff_out);
    };
    auto radix = [&](uint64_t** buf, const uint64_t* count, uint64_t rcap, int lo, int nbits, int max_blocks) {
        return radix_sort_u64(buf, count, rcap, lo, nbits, max_blocks, counts, digit_tot, s);
    };
    auto bits_for = [](int64_t n) {
        int b = 1;
        while (((int64_t)1 << b) < n) ++b;
        return b;
    };

    IA_LAUNCH("fill_u32_kernel", fill_u32_kernel, dim3(grid_cap(2 * L.ntiles_all, kBlock, 4096)), dim3(kBlock), 0, s,
              reinterpret_cast<uint32_t*>(ranges), 0u, 2 * L.ntiles_all);
    if (N > 0) {
        // projection; per block: visible Gaussians and tiles touched
        PreArgs pre{a.means, a.means_stride, a.scales, a.quats, a.colors, a.sh, a.opacity, a.sh_degree,
                    cams, fo, a.frames, N, pa, pb, pc, depth, rect, tiles, bsum, bsum_t};
        IA_LAUNCH("preprocess_kernel", preprocess_kernel, dim3(L.nb1), dim3(kBlock), 0, s, pre);
        scan(bsum_t, L.nb1, cap, nent, a.n_entries_out, a.overflow_out, nullptr);
        scan(bsum, L.nb1, kNoCap, nvis, nullptr, nullptr, boff);
        // visible Gaussians in ascending depth, ties in index order (stable
        // sort of index-ordered input on the 31 depth bits above the index)
        IA_LAUNCH("compact_kernel", compact_kernel, dim3(L.nb1), dim3(kBlock), 0, s, tiles, depth, N, boff, gk[0]);
        const int gcur = radix(gk, nvis, (uint64_t)N, 32, 31, L.sort_blocks_g);
        IA_LAUNCH("binning_mode_kernel", binning_mode_kernel, dim3(1), dim3(64), 0, s, nent, nvis, a.binning, mode);
        // entries in depth order: one per (Gaussian, tile) or per (Gaussian, region)
        IA_LAUNCH("sorted_rects_kernel", sorted_rects_kernel, dim3(L.nb1), dim3(kBlock), 0, s, gk[gcur], nvis, mode,
                  rect, srect, bsum);
        scan(bsum, L.nb1, cap, nsort, nullptr, nullptr, boff);
        OffsetArgs oa{gk[gcur], nvis, mode, srect, boff, cap, (uint32_t)L.nemit, (uint32_t)L.emit_per, fo, a.frames,
                      ginfo, gframe, bstart};
        IA_LAUNCH("offsets_kernel", offsets_kernel, dim3(L.nb1), dim3(kBlock), 0, s, oa);
        EmitArgs em{ginfo, gframe, nvis, mode, bstart, nsort, cap, (uint32_t)L.emit_per, L.tiles_x, ntiles,
                    (uint32_t)L.regions_x, rpf, ent[0]};
        IA_LAUNCH("emit_kernel", emit_kernel, dim3(L.nemit), dim3(kBlock), 0, s, em);
        // stable sort on the tile (or region) index: per tile (region), its
        // Gaussians in (depth, index) order.  Region indices are below the
        // tile count, so the tile bits cover both.
        const int ecur = radix(ent, nsort, cap, 32, bits_for(L.ntiles_all), L.sort_blocks_e);
        // tile sort: ranges and values from the sorted entries
        IA_LAUNCH("ranges_kernel", ranges_kernel, dim3(grid_cap(L.cap, kBlock, 8192)), dim3(kBlock), 0, s,
                  ent[ecur], nsort, cap, ranges, (uint32_t)L.ntiles_all, vals, mode, (uint64_t)kModeTiles);
        // regions: ranges of the regions, work items, count, scan, write
        IA_LAUNCH("fill_u32_kernel", fill_u32_kernel, dim3(grid_cap(2 * L.nreg, kBlock, 4096)), dim3(kBlock), 0, s,
                  reinterpret_cast<uint32_t*>(rranges), 0u, 2 * L.nreg);
        IA_LAUNCH("ranges_kernel", ranges_kernel, dim3(grid_cap(L.cap, kBlock, 8192)), dim3(kBlock), 0, s,
                  ent[ecur], nsort, cap, rranges, (uint32_t)L.nreg, (uint32_t*)nullptr, mode,
                  (uint64_t)kModeRegions);
        IA_LAUNCH("region_items_kernel", region_items_kernel, dim3(L.nbr), dim3(kBlock), 0, s, mode, rranges,
                  (uint32_t)L.nreg, bsum);
        scan(bsum, L.nbr, kNoCap, nitems, nullptr, nullptr, boff);
        IA_LAUNCH("region_expand_kernel", region_expand_kernel, dim3(L.nbr), dim3(kBlock), 0, s, mode, rranges,
                  (uint32_t)L.nreg, boff, (uint64_t)L.max_items, items, rfirst);
        ExpandArgs xa{mode, items, nitems, rranges, ent[ecur], ginfo, (uint32_t)L.regions_x, rpf, L.tiles_x,
                      L.tiles_y, ntiles, icnt, tstart, cap, vals};
        const int xgrid = grid_cap((L.max_items + 3) / 4, 1, 16384);
        IA_LAUNCH("expand_count_kernel", expand_kernel<false>, dim3(xgrid), dim3(kBlock), 0, s, xa);
        IA_LAUNCH("region_tiles_kernel", region_tiles_kernel, dim3(grid_cap((L.nreg + 3) / 4, 1, 1 << 30)),
                  dim3(kBlock), 0, s, mode, rranges, rfirst, (uint32_t)L.nreg, (uint32_t)L.regions_x, rpf, L.tiles_x,
                  L.tiles_y, ntiles, (uint64_t)L.max_items, icnt, tcount);
        IA_LAUNCH("tile_sums_kernel", tile_sums_kernel, dim3(L.nbt), dim3(kBlock), 0, s, mode, tcount, L.ntiles_all,
                  bsum);
        scan(bsum, L.nbt, kNoCap, ctr + 8, nullptr, nullptr, boff);
        IA_LAUNCH("tile_ranges_kernel", tile_ranges_kernel, dim3(L.nbt), dim3(kBlock), 0, s, mode, tcount,
                  L.ntiles_all, boff, cap, tstart, ranges);
        IA_LAUNCH("expand_write_kernel", expand_kernel<true>, dim3(xgrid), dim3(kBlock), 0, s, xa);
    } else {
        IA_LAUNCH("scan_top_kernel", scan_top_kernel, dim3(1), dim3(kBlock), 0, s, bsum2, 0, cap, nent,
                  a.n_entries_out, a.overflow_out);
    }
    RasterArgs ra{ranges, vals, pa, pb, pc, cams, a.W, a.H, L.tiles_x, ntiles, cap, N, a.image, a.T_final,
                  a.n_contrib};
    // two pixels per thread when there are enough tiles to fill the chip twice over
    // (the index of the last composited Gaussian is tracked only for n_contrib)
    const dim3 tgrid(L.tiles_x, L.tiles_y, a.frames);
    // (four pixels per thread, one wave per tile, measured slower: sequence
    // raster 3.3 -> 5.4 ms, Stress 2.6 -> 3.3 ms)
    if (L.ntiles_all >= kRasterTwoPixelTiles) {
        if (a.n_contrib)
            IA_LAUNCH("raster_kernel", (raster_kernel<2, true>), tgrid, dim3(128), 0, s, ra);
        else
            IA_LAUNCH("raster_kernel", (raster_kernel<2, false>), tgrid, dim3(128), 0, s, ra);
    } else {
        if (a.n_contrib)
            IA_LAUNCH("raster_kernel", (raster_kernel<1, true>), tgrid, dim3(256), 0, s, ra);
        else
            IA_LAUNCH("raster_kernel", (raster_kernel<1, false>), tgrid, dim3(256), 0, s, ra);
    }
    *keys_out = nullptr;
    *vals_out = nullptr;
    if (a.unpack) {
        uint64_t* keys = ent[0];
        if (N > 0)
            IA_LAUNCH("unpack_kernel", unpack_kernel, dim3(ntiles, a.frames), dim3(kBlock), 0, s, ranges, vals, depth,
                      N, keys);
        *keys_out = keys;
        *vals_out = vals;
    }
    return hipGetLastError();
}

}  // namespace ia
