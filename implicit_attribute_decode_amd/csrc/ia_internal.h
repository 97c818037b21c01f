// Internal declarations shared by the translation units of libia.so.
// Kernels live in decode.hip, hexplane.hip and render.hip; each file exports
// host-side launchers that api.hip calls after validating arguments.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "ia.h"

namespace ia {

// Brackets one kernel launch with HIP events on its stream when profiling is
// enabled (ia_profile_enable); a no-op otherwise.
class ProfScope {
  public:
    ProfScope(const char* name, hipStream_t s);
    ~ProfScope();

  private:
    const char* name_;
    hipStream_t s_;
    hipEvent_t start_{}, stop_{};
    bool active_ = false;
};

#define IA_LAUNCH(name, kernel, grid, block, shmem, stream, ...)               \
    do {                                                                       \
        ::ia::ProfScope ia_prof_scope_(name, stream);                          \
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);   \
    } while (0)

constexpr int kMaxLevels = 32;
constexpr int kMaxDecoderMats = 12;  // per-attribute decoder: 4 branches x 3 layers

// Per-level geometry of the 4D hash encoder (SPIN-4DGS §3.3, Eq. 9).
struct HashLevels {
    int L;
    int F;
    uint32_t mask;  // 2^log2T - 1
    uint32_t T;     // 2^log2T
    int table_f16;
    float t_min, t_max;
    int res_s[kMaxLevels];  // vertices per spatial axis
    int res_t[kMaxLevels];  // vertices on the t axis
    int dense[kMaxLevels];  // 1: row-major dense indexing, 0: hashed
};

struct DecodeArgs {
    HashLevels h;
    const void* tables;
    const void* W[4];  // trunk layers then the 11-row head block, row-major [out][in]
    const float* b[4];
    int in_dim;
    int n_hidden;
    int hidden[4];
    int act;
    int sh_head;       // 1: the colour is 48 SH coefficients (head block of 56 rows, or a 48-row branch)
    int branches;      // 1: per-attribute fp16 decoder (F = 4), weights in Wt / bpack
    const void* Wt;    // branch weights in MFMA A-tile order (branch_tile_bytes)
    const float* bpack;  // branch biases, packed (branch_bias_bytes)
    const float* pos;  // [N, stride]
    int stride;        // 3 (scalar t) or 4 (per-point t)
    float t_scalar;
    int64_t N;
    float* scales;
    float* quats;
    float* colors;
    float* sh;  // [N][48] for the SH head
    float* opacity;
    uint32_t* features;  // fp16 path, or null: caller buffer [L][N] of packed fp16 features (F / 2 words each)
    // fp16 path scratch, carved from the caller's workspace (decode_layout)
    uint32_t* zslot[2];  // per slot: [L][zcap] packed fp16 features (F / 2 words each)
    float4* xt[2];       // per slot: [zcap] normalised positions
    int64_t zcap;        // Gaussians per chunk a slot holds
    hipStream_t side;    // caller's second stream for the MLP beside the next gather, or null
};

// Gaussians per fp16-decode chunk (one normalise / gather / MLP triple).
constexpr int64_t kDecodeChunk = int64_t(1) << 22;

// Byte offsets of the fp16 decode's scratch inside a workspace: chunks of
// zcap Gaussians (N rounded up to a multiple of 256, at most max_chunk), one
// slot, or two when N needs more than one chunk (consecutive chunks
// alternate, so the MLP of one can run beside the gather of the next).
struct DecodeLayout {
    size_t z[2], xt[2], total;
    int64_t zcap;
    int slots;
};
DecodeLayout decode_layout(const HashLevels& h, int64_t N, int64_t max_chunk = kDecodeChunk);

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s);

// Per-attribute fp16 decoder (64 -> 64 -> 64 -> out per branch): bytes of the
// tiled weights and packed biases, and the kernel that builds both from the
// 12 row-major matrices / bias vectors (branch by branch: scale, rotation,
// colour, opacity; three layers each).
size_t branch_tile_bytes(bool sh);
size_t branch_bias_bytes(bool sh);
hipError_t launch_branch_pack(const _Float16* const* W, const float* const* b, bool sh, void* Wt, float* bpack,
                              hipStream_t s);
// F = 4 level-major gather of n Gaussians (xt) into z ([L][zstride] x 8 bytes).
hipError_t launch_gather_f4(const float4* xt, int64_t n, const HashLevels& h, const void* tables, uint32_t* z,
                            int64_t zstride, hipStream_t s);
// Per-attribute MLPs and Eq. 11 for Gaussians [off, off + n) from z.
hipError_t launch_mlp_branch(const DecodeArgs& a, const uint32_t* z, int64_t zstride, int64_t n, int64_t off,
                             hipStream_t s);

// fp16 path: normalise Gaussians [off, off + n) of a.pos into xt and gather
// their features into z ([L][zstride] fp16 pairs), as the decode does; with z
// null, normalise only.
hipError_t launch_decode_features(const DecodeArgs& a, int64_t off, int64_t n, float4* xt, uint32_t* z,
                                  int64_t zstride, hipStream_t s);

// Backward of the fp16 decode: one persistent grid of kDecodeBwdBlocks blocks
// of four waves; each wave owns a slot of kDecodeBwdSlotFloats floats in the
// workspace's partials (148 x 64 used by the RGB head, 208 x 64 by the SH
// colour head, up to 220 x 64 by one branch of the per-attribute decoder),
// followed by kDecodeBwdGroups slots of group sums.
constexpr int kDecodeBwdBlocks = 256;
constexpr int kDecodeBwdGroups = 16;
constexpr int kDecodeBwdSlotFloats = 224 * 64;
constexpr int64_t kDecodeBwdPartialFloats = ((int64_t)kDecodeBwdBlocks * 4 + kDecodeBwdGroups) * kDecodeBwdSlotFloats;

// Byte offsets of the backward's scratch inside a workspace (chunks of at
// most 2^21 Gaussians): recomputed features z [L][chunk], their gradient
// [L][chunk] float2, the chunk's active list, block offsets and count,
// normalised positions, the weight-gradient partials, the spatial sort's
// buffers and the per-level position shares [L][chunk] float4.
struct DecodeBwdLayout {
    size_t z, gz, list, boff, count, xt, partial, sort, pos, bcount, brec, total;
    int64_t chunk;
    int64_t bcap;  // records per fine-level bucket
};
DecodeBwdLayout decode_bwd_layout(const HashLevels& h, int64_t N);

struct DecodeBwdArgs {
    DecodeArgs fwd;           // the decode being differentiated (parameters, positions)
    const float* g_scales;    // [N,3] upstream dL/dscales
    const float* g_quats;     // [N,4]
    const float* g_colors;    // [N,3], or the SH coefficients [N,48] (SH colour head)
    const float* g_opacity;   // [N]
    const float* g_means;     // [N,3] added into g_pos, or null
    float* g_pos;             // [N,3] out, or null (no position gradient)
    float* g_tables;          // [L][T][F] out
    // shared trunk: g_W[0..2] = [64][32], [64][64], [11 or 56][64]; per-attribute
    // branches: g_W[3 br + l] = [64][64], [64][64], [out_br][64]; the same for g_b
    float* g_W[kMaxDecoderMats];
    float* g_b[kMaxDecoderMats];
    const _Float16* Wbr[kMaxDecoderMats];  // per-attribute branches: the fp16 weights, branch-major
    const float* bbr[kMaxDecoderMats];
    unsigned char* ws;        // caller's workspace, decode_bwd_layout(h, N).total bytes
};

hipError_t launch_decode_backward(const DecodeBwdArgs& b, hipStream_t s);

struct HexArgs {
    int res_xyz, res_t, C;
    float aabb;
    const _Float16* planes[6];
    const _Float16* W[3];
    const float* b[3];
    const float* means;
    const float* scales;
    const float* quats;
    const float* sh;
    const float* opacity;
    float t;
    int64_t N;
    float* o_means;
    float* o_scales;
    float* o_quats;
    float* o_sh;
    float* o_opacity;
};

// Rearrange the three row-major fp16 weight matrices into the A-tile order the
// deformation kernel stages through LDS (256 tiles of 1 KiB, Wt owns 256 KiB).
constexpr size_t kHexTiledWeightBytes = 256 * 1024;
hipError_t launch_hexplane_tiles(const _Float16* const W[3], void* Wt, hipStream_t s);

hipError_t launch_hexplane(const HexArgs& a, const void* Wt, hipStream_t s);

// ---------------------------------------------------------------- render

// Camera in the device-side table.  centre = -R^T t (for SH view directions).
struct DevCamera {
    float R[9];
    float t[3];
    float fx, fy, cx, cy, near_z;
    float centre[3];
    float bg[3];
    int W, H;
};

// Byte offsets of every buffer inside the render workspace.
struct RenderLayout {
    size_t cams, fo, pa, pb, pc, depth, rect, tiles, bsum, bsum_t, bsum2, boff, srect, ginfo, gframe, bstart, gk0, gk1, ent0,
        ent1, vals, counts, digit_tot, rranges, rfirst, items, icnt, tcount, tstart, ranges, counters, gacc, total;
    int64_t N, cap, ntiles_all, nreg, max_items;
    int frames, tiles_x, tiles_y, regions_x, regions_y, nb1, nbr, nbt, nemit, emit_per;
    int sort_blocks_g, sort_blocks_e;  // radix-sort blocks over Gaussians / over coarse entries
};

RenderLayout render_layout(int64_t N, int frames, int W, int H, int64_t max_entries);

struct RenderArgs {
    const float* means;
    int means_stride;
    const float* scales;
    const float* quats;
    const float* colors;
    const float* sh;
    const float* opacity;
    int sh_degree;
    int frames, W, H;
    const int64_t* frame_offsets_host;
    const DevCamera* cams_host;
    unsigned char* ws;
    RenderLayout lay;
    float* image;
    float* T_final;
    uint32_t* n_contrib;
    uint64_t* n_entries_out;
    uint32_t* overflow_out;
    int unpack;  // write the sorted (tile << 32 | depth bits) keys and index values for inspection
    int binning; // 0 automatic, 1 tile sort, 2 regions
};

// Enqueue the whole render.  With unpack set, returns the sorted keys and
// values through keys_out / vals_out (else both are null).
hipError_t launch_render(const RenderArgs& a, hipStream_t s, const uint64_t** keys_out, const uint32_t** vals_out);

// Partials per Gaussian the raster backward accumulates in the workspace
// (gacc): d/d(u, v, A, B, C, opacity, r, g, b).
constexpr int kGradPerGaussian = 9;

struct RenderBwdArgs {
    unsigned char* ws;  // workspace of the forward render with the same arguments
    RenderLayout lay;
    int W, H;
    const float* means;
    int means_stride;
    const float* scales;
    const float* quats;
    const float* grad_image;  // [F,3,H,W]
    const float* T_final;     // [F,H,W]
    const uint32_t* n_contrib;
    float* g_means;  // [N,3]
    float* g_scales;
    float* g_quats;  // [N,4]
    float* g_opacity;
    float* g_colors;
    const float* sh;  // [N,16,3] when the colours are degree-3 SH, else null
    float* g_sh;      // [N,16,3] out with sh
};

hipError_t launch_render_backward(const RenderBwdArgs& a, hipStream_t s);

// L = mean |image - target| into *loss (device double); grad = dL/dimage.
hipError_t launch_l1_loss(const float* image, const float* target, int64_t n, double* loss, float* grad,
                          hipStream_t s);

// Eq. 12 image loss (L1 + D-SSIM) and its image gradient; workspace bytes for
// frames x 3 x H x W images.
size_t image_loss_workspace(int32_t frames, int32_t H, int32_t W);
hipError_t launch_image_loss(const float* image, const float* target, int32_t frames, int32_t H, int32_t W,
                             float lambda, void* ws, double* loss, float* grad, hipStream_t s);
// One bias-corrected Adam step over n fp32 parameters (optional fp16 copy).
// Densify / prune of the positions (densify.hip)
struct DensifyIn {
    const float* xyzt;        // [N][4]
    const float* grad_acc;    // [N]
    const int32_t* grad_count;
    const float* scales;      // [N][3] decoded
    const float* quats;       // [N][4] decoded
    const float* opacity;     // [N] decoded
    const float* noise;       // [N][2][3] standard normal draws
    const float* m;           // [N][3] Adam moments of the positions
    const float* v;
    int64_t N;
    float grad_threshold, scale_threshold, min_opacity;
    float* out_xyzt;          // [2N][4]
    float* out_m;             // [2N][3]
    float* out_v;
    int64_t* out_n;           // device: rows written
};
size_t densify_workspace(int64_t N);
hipError_t launch_densify(const DensifyIn& in, void* ws, hipStream_t s);
hipError_t launch_densify_accumulate(const float* g, int64_t N, float* acc, int32_t* cnt, hipStream_t s);

// Copy `bytes` of host memory to device memory through kernel arguments
// (stream-ordered, no host staging buffer that could outlive the call; the
// host source may be freed on return).
hipError_t upload(void* dst, const void* src, size_t bytes, hipStream_t s);

// Per-frame spatial order of positions (order.hip).
size_t spatial_order_workspace(int64_t N, int frames);
hipError_t launch_spatial_order(const float* pos, int stride, int64_t N, const int64_t* frame_offsets_host, int frames,
                                uint32_t* perm, float* pos_out, void* ws, hipStream_t s);

// Stable LSD radix sort of the first min(*count, cap) 64-bit words of buf[0]
// on bits [lo, lo + nbits) (render.hip); returns the index (0 or 1) of the
// buffer of buf that holds the result.  max_blocks <= radix_sort_blocks(cap);
// counts: radix_sort_counts_bytes(max_blocks) bytes; digit_tot: 4 KiB.
int radix_sort_u64(uint64_t* const* buf, const uint64_t* count, uint64_t cap, int lo, int nbits, int max_blocks,
                   uint32_t* counts, uint32_t* digit_tot, hipStream_t s);
int radix_sort_blocks(int64_t items);
size_t radix_sort_counts_bytes(int max_blocks);

// g, m, v dense [n]; the parameter is rows of `dim` values `stride` floats
// apart (dim == stride: dense); p16 (dense [n] fp16 copy of the result) or null
hipError_t launch_adam(float* p, const float* g, float* m, float* v, int64_t n, int32_t dim, int32_t stride,
                       float lr, float beta1, float beta2, float eps, int32_t step, uint16_t* p16, hipStream_t s);

}  // namespace ia
