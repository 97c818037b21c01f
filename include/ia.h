/*
 * ia.h - C ABI of libia.so: implicit attribute decode + tile rasterisation of
 * 4D Gaussian splats on AMD Instinct MI355X (gfx950).
 *
 * The operations follow two pages:
 *   [SPIN] "Implicit 4D Gaussian Splatting for Fast Motion with Large
 *          Inter-Frame Displacements" (SPIN-4DGS): §3.1 Eq. 1-4 (Gaussians,
 *          covariance, EWA projection, alpha compositing), §3.2 Eq. 6
 *          (refinement of the positions), §3.3 Eq. 7-12 (normalisation, 4D
 *          hash encoder, multibranch decoder, activations, training loss),
 *          §4 implementation details (Adam, per-group rates).
 *   [HEX]  "4D Gaussian Splatting详解：动态场景实时渲染的范式突破":
 *          §3.1 (HexPlane six-plane encoder), §3.2 (deformation MLP), §6.1
 *          (opacity is not deformed).
 *
 * Conventions for every entry point:
 *   - Device pointers point to memory the caller allocated on the current
 *     HIP device (e.g. torch tensors); host pointers are marked "host".
 *   - All floating-point buffers are fp32 unless stated; every [N,k] buffer is
 *     row-major and densely packed.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued on
 *     it and the call returns without waiting, except where stated.
 *   - Return value: IA_OK (0) or a negative ia_status.  Argument and size
 *     errors are detected before anything is enqueued; the message is
 *     available from ia_last_error() on the calling thread.  No C++
 *     exception crosses this boundary.
 *   - Handles own only their parameters (device memory allocated by
 *     set_params, freed by destroy) and change only through set_params and,
 *     for decoders, ia_decoder_update_params (stream-ordered).  Every other
 *     call reads a handle without modifying it, so calls on one handle from
 *     several streams or threads may overlap, each with its own workspace.
 *   - Scratch memory is the caller's: a workspace of the size the matching
 *     *_workspace_size call reports, 256-byte aligned, contents undefined
 *     between calls.  Calls that share a workspace must not overlap.  No entry
 *     point allocates device memory except set_params / create.
 */
#ifndef IA_H_
#define IA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IA_API __attribute__((visibility("default")))

typedef int32_t ia_status;
#define IA_OK 0
#define IA_ERR_INVALID_ARG (-1)        /* null/misaligned pointer, bad size, bad descriptor */
#define IA_ERR_UNSUPPORTED (-2)        /* valid but not implemented shape/dtype combination */
#define IA_ERR_WORKSPACE_TOO_SMALL (-3)
#define IA_ERR_DEVICE (-4)             /* a HIP call or kernel launch failed */
#define IA_ERR_OUT_OF_MEMORY (-5)

#define IA_DTYPE_F32 0
#define IA_DTYPE_F16 1

#define IA_ACT_RELU 0
#define IA_ACT_GELU 1 /* exact: 0.5 x (1 + erf(x / sqrt 2)) */

/* Colour head of the decoder ([SPIN] §3.3 Eq. 10-11) */
#define IA_COLOR_RGB 0 /* 3 outputs, sigmoid                                   */
#define IA_COLOR_SH3 1 /* 48 spherical-harmonic coefficients of degree 3, no
                          activation (the paper's colour decoder)              */

/* Decoder layout ([SPIN] §3.3 Eq. 10) */
#define IA_BRANCHES_SHARED 0        /* one trunk, one head block             */
#define IA_BRANCHES_PER_ATTRIBUTE 1 /* one MLP per attribute (scale, rotation,
                                       colour, opacity), all reading z       */

/* Message of the last non-OK status returned on this thread ("" if none). */
IA_API const char* ia_last_error(void);

/* ------------------------------------------------------------------------ */
/* Gaussian attribute buffers (structure of arrays, all device, fp32)        */
/* ------------------------------------------------------------------------ */
typedef struct {
    float* means;          /* [N, means_stride]: x, y, z (+ anything after)  */
    int32_t means_stride;  /* floats between consecutive means; 0 means 3    */
    float* scales;         /* [N,3] linear scales                            */
    float* quats;          /* [N,4] rotation (w, x, y, z), any non-zero norm */
    float* colors;         /* [N,3] RGB in [0,1] (sh_degree < 0)             */
    float* sh;             /* [N,16,3] SH coefficients, coefficient-major    */
    float* opacity;        /* [N]                                            */
    int32_t sh_degree;     /* -1: use colors; 3: evaluate sh (render only)   */
} ia_gaussians;

/* ------------------------------------------------------------------------ */
/* Decoder: [SPIN] §3.3 Eq. 7-11                                             */
/* ------------------------------------------------------------------------ */

/* 4D multiresolution hash encoder ([SPIN] §3.3 Eq. 9).  Level l has
 * floor(base_res * growth^l) vertices per spatial axis and temporal_res
 * vertices on t (0 = same as spatial).  A level is stored densely when
 * res^3 * res_t <= 2^log2T, otherwise it is hashed with
 * (ix*1 ^ iy*2654435761 ^ iz*805459861 ^ it*3674653429) mod 2^log2T. */
typedef struct {
    int32_t L;            /* levels: 4 or 16 (in_dim = 2 L)                 */
    int32_t F;            /* features per level: 2, or 4 (fp16 tables)      */
    int32_t log2T;        /* table entries per level = 2^log2T, 4..24       */
    double base_res;      /* vertices per axis at level 0, >= 2             */
    double growth;        /* per-level growth factor, >= 1                  */
    int32_t temporal_res; /* vertices on the t axis, 0 = spatial res        */
    int32_t table_dtype;  /* IA_DTYPE_F32 or IA_DTYPE_F16                   */
    float t_min, t_max;   /* time normalisation of Eq. 8, t_max > t_min     */
} ia_hash_desc;

/* Decoder MLP ([SPIN] §3.3 Eq. 10).  Outputs in the order
 * scale(3) | rotation(4: w,x,y,z) | colour | opacity(1), where colour is 3
 * RGB outputs (color = IA_COLOR_RGB: 11 outputs) or 48 SH coefficients,
 * coefficient-major [16][3] (IA_COLOR_SH3: 56 outputs).
 *   branches = IA_BRANCHES_SHARED: a trunk of n_hidden layers act(W x + b)
 *     and one linear head block of all outputs; weights[k], biases[k] for
 *     layer k (n_hidden + 1 layers).
 *   branches = IA_BRANCHES_PER_ATTRIBUTE: four MLPs in -> hidden -> out_a
 *     (out_a = 3, 4, 3 or 48, 1), each of n_hidden act layers and a linear
 *     last layer; weights / biases hold 4 (n_hidden + 1) pointers, branch by
 *     branch in the order scale, rotation, colour, opacity.
 * Supported:
 *   dtype F32: shared; (in_dim, hidden) = (8, {32}), (32, {64}) or
 *              (32, {64, 64}); RGB
 *   dtype F16: fp16 MFMA with fp32 accumulation, hidden activations rounded
 *              to fp16; shared with in_dim = 32 (F = 2), hidden = {64, 64},
 *              or per attribute with in_dim = 64 (F = 4), hidden = {64, 64};
 *              RGB or SH3. */
typedef struct {
    int32_t in_dim;
    int32_t n_hidden;
    int32_t hidden[4];
    int32_t activation; /* IA_ACT_RELU or IA_ACT_GELU */
    int32_t dtype;      /* IA_DTYPE_F32 or IA_DTYPE_F16 (weights and math) */
    int32_t color;      /* IA_COLOR_RGB or IA_COLOR_SH3                    */
    int32_t branches;   /* IA_BRANCHES_SHARED or IA_BRANCHES_PER_ATTRIBUTE */
} ia_mlp_desc;

typedef struct ia_decoder ia_decoder;

/* Validate the descriptors and create an empty handle (no device memory yet).
 * Errors: INVALID_ARG (null pointers, out-of-range fields), UNSUPPORTED. */
IA_API ia_status ia_decoder_create(const ia_hash_desc* hash, const ia_mlp_desc* mlp, ia_decoder** out);

/* Copy the parameters into device memory owned by the handle.
 *   tables : [L][2^log2T][F] of table_dtype
 *   weights: layer matrices row-major [out][in] of mlp dtype: n_hidden + 1
 *            (shared: the last one is the head block) or 4 (n_hidden + 1)
 *            (per attribute, see ia_mlp_desc)
 *   biases : fp32 [out], one per weight matrix
 * params_on_device: 1 if all the above are device pointers, 0 if host.
 * The copies are enqueued on `stream`; host sources may be freed on return
 * (host copies are synchronous).  May be called again to replace parameters
 * (waits for the device first).
 * Errors: INVALID_ARG, OUT_OF_MEMORY, DEVICE. */
IA_API ia_status ia_decoder_set_params(ia_decoder* dec, const void* tables, const void* const* weights,
                                const float* const* biases, int32_t params_on_device, void* stream);

/* Overwrite the parameter values of a decoder whose parameters are set, from
 * device memory in the layouts of ia_decoder_set_params, with copies enqueued
 * on `stream` (no allocation, no synchronisation): an optimiser's update
 * between training steps.  Decodes and backwards enqueued later on `stream`
 * see the new values; the caller orders other streams after it.
 * Errors: INVALID_ARG (null, parameters not set), DEVICE. */
IA_API ia_status ia_decoder_update_params(ia_decoder* dec, const void* tables, const void* const* weights,
                                          const float* const* biases, void* stream);

/* Bytes of workspace a decode of N Gaussians needs (ia_decode,
 * ia_decode_xyzt, ia_decode_keep): 0 for fp32 decoders; for fp16 decoders
 * (2 L F + 16) bytes per Gaussian of a chunk of min(N, 2^22) Gaussians
 * (rounded up to a multiple of 256), twice that when N > 2^22 (consecutive
 * chunks alternate between two halves).  Errors: INVALID_ARG. */
IA_API ia_status ia_decode_workspace_size(const ia_decoder* dec, int64_t N, size_t* bytes);

/* Decode N Gaussians at one time t ([SPIN] §3.3 Eq. 7-11):
 *   xyz : device [N,3] positions mu
 *   out : device scales[N,3] = exp(min(s_hat,20)), quats[N,4] = r_hat/|r_hat|,
 *         colors[N,3] = sigmoid(c_hat) (RGB head) or sh[N,16,3] = sh_hat
 *         (SH3 head; out->colors is then not used), opacity[N] =
 *         sigmoid(o_hat); out->means is not written (the input positions
 *         are the means).
 *   ws, ws_bytes: device workspace of ia_decode_workspace_size(dec, N) bytes
 *         (may be NULL when that is 0), 256-byte aligned.
 *   side_stream: a second hipStream_t of the caller, or NULL.  When N needs
 *         more than one chunk, the MLP of each chunk runs on it beside the
 *         gather of the next; otherwise it is not used.
 * N = 0 is a no-op.  Errors: INVALID_ARG (null, N < 0, params not set,
 * misaligned workspace), WORKSPACE_TOO_SMALL.
 * Asynchronous on stream: all of the call's work, including what it runs on
 * side_stream, starts after everything already queued on stream, and stream
 * continues only after all of it.  Results are deterministic and do not
 * depend on side_stream; with the fp16 decoder the rounding of a Gaussian
 * depends on its index modulo 64 (the matrix-core column it occupies), so
 * decoding a slice that starts at a multiple of 64 gives bit for bit the same
 * values as decoding it within a larger array. */
IA_API ia_status ia_decode(const ia_decoder* dec, const float* xyz, int64_t N, float t, const ia_gaussians* out,
                           void* ws, size_t ws_bytes, void* side_stream, void* stream);

/* As ia_decode with a per-Gaussian time: xyzt is device [N,4] (x, y, z, t).
 * One launch decodes any mix of frames (spatiotemporal slicing: every frame
 * is its own set of positions, [SPIN] §3.2). */
IA_API ia_status ia_decode_xyzt(const ia_decoder* dec, const float* xyzt, int64_t N, const ia_gaussians* out,
                                void* ws, size_t ws_bytes, void* side_stream, void* stream);

/* For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): ia_decode_xyzt (no second stream) with its scratch in a
 * file-scope device array of 20 MiB instead of a workspace.  Allocates
 * nothing; each GPU the library runs on holds its own copy of the array from
 * the first call on it until the process ends.
 *   N: at most floor(20 MiB / (2 L F + 16 bytes)) rounded down to a multiple
 *      of 256 for fp16 decoders (262,144 Gaussians for L = 16, F = 2;
 *      145,408 for L = 16, F = 4), else INVALID_ARG before anything is
 *      enqueued; any N for fp32 decoders, which use no scratch.
 * Results equal those of ia_decode_xyzt for the same N bit for bit.  Every
 * call on one GPU uses the same array: calls that overlap on one GPU (other
 * streams, other threads) race and must not be made; the array needs no
 * clearing between calls (each call overwrites what it reads).
 * Errors: INVALID_ARG, DEVICE. */
IA_API ia_status ia_decode_xyzt_noalloc(const ia_decoder* dec, const float* xyzt, int64_t N, const ia_gaussians* out,
                                        void* stream);

/* Bytes of the encoding z of N Gaussians (N x L x F fp16) that
 * ia_decode_keep stores and ia_decode_backward can reuse. */
IA_API ia_status ia_decode_feature_bytes(const ia_decoder* dec, int64_t N, size_t* bytes);

/* As ia_decode (pos_stride 3, time t) or ia_decode_xyzt (pos_stride 4), and
 * keep the hash encoding z of every Gaussian in `features` (device,
 * caller-owned, >= ia_decode_feature_bytes, 8-byte aligned; layout
 * [L][N] x F fp16) for a later ia_decode_backward of the same positions,
 * which then skips recomputing it.  fp16 decoders only; ws, side_stream as
 * ia_decode.  Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, DEVICE. */
IA_API ia_status ia_decode_keep(const ia_decoder* dec, const float* pos, int32_t pos_stride, int64_t N, float t,
                                const ia_gaussians* out, void* features, size_t features_bytes, void* ws,
                                size_t ws_bytes, void* side_stream, void* stream);

/* Gradients of the decoder parameters (device, fp32, overwritten), one per
 * weight matrix in the order ia_decoder_set_params takes them: the shared
 * trunk's n_hidden + 1 layers, or the per-attribute decoder's 12 (branch by
 * branch: scale, rotation, colour, opacity; three layers each). */
typedef struct {
    float* tables;      /* [L][2^log2T][F], whatever the table dtype         */
    float* weights[12]; /* matrix k: [out][in]                               */
    float* biases[12];  /* matrix k: [out]                                   */
} ia_decoder_grads;

/* Bytes of workspace ia_decode_backward needs for N Gaussians: per chunk of
 * min(N, 2^21) Gaussians (rounded up to a multiple of 4096) the recomputed
 * encoding, its gradient, the chunk's active list and spatial sort, the
 * normalised positions and the per-level position shares (484 bytes per
 * Gaussian at L = 16, F = 2; 676 at F = 4), plus 60 MB of weight-gradient
 * partials, plus the table-gradient buckets of the levels finer than 300
 * vertices per axis: per such level 20 (entry, value) records per Gaussian
 * of the chunk, 4 (1 + F) bytes each (240 bytes at F = 2), for as many of
 * those levels at a time as fit 2 GiB (at least one).
 * Errors: INVALID_ARG, UNSUPPORTED (decoders without a backward). */
IA_API ia_status ia_decode_backward_workspace_size(const ia_decoder* dec, int64_t N, size_t* bytes);

/* Backward of ia_decode (pos_stride 3, time t) or ia_decode_xyzt (pos_stride
 * 4) for upstream gradients of the decoded attributes ([SPIN] §3.3 Eq. 7-11
 * differentiated; positions are trainable, §3.3 Eq. 7).
 *   grad_attr: device dL/d scales [N,3], quats [N,4], colors [N,3] (RGB
 *              head) or sh [N,16,3] (SH colour head), opacity [N] (means
 *              and the other colour field are ignored).
 *   grad_means: device [N,3] or NULL; added into grad_pos (e.g. the render's
 *              position gradient, the positions being the means).
 *   grad_pos:  device [N,3] out, grad_means + dL/dposition through Eq. 7 and
 *              the corner weights of Eq. 9 (time carries none), the levels'
 *              shares added in a fixed order (the same on every run); NULL
 *              skips the position gradient.
 *   grads:     all outputs overwritten: table gradient (scatter-add of
 *              w_c dL/dz over the 16 corners of each level, float atomics,
 *              so the last bits vary from run to run), weight and bias
 *              gradients (summed in a fixed order: deterministic).
 *   features:  the encoding kept by ia_decode_keep for the same positions, or
 *              NULL (then recomputed).
 *   ws, ws_bytes: device workspace of ia_decode_backward_workspace_size(dec,
 *              N) bytes, 256-byte aligned.
 * The forward is recomputed exactly as the decode computes it (fp16 hidden
 * activations); the backward runs in fp32 (v_mfma_f32_16x16x4_f32), treating
 * the fp16 roundings as the identity.  Supported: every fp16 decoder -- the
 * shared trunk with the RGB head or the SH colour head ([SPIN] §3.3: the
 * colour decoder regresses the 48 coefficients, so their gradient passes
 * unchanged to the head outputs), and the per-attribute decoder of §3.3 (one
 * MLP per attribute over the F = 4 encoding; the encoding's gradient is the
 * sum of the four branches').
 * Errors: INVALID_ARG, UNSUPPORTED (other decoders), WORKSPACE_TOO_SMALL,
 * DEVICE. */
IA_API ia_status ia_decode_backward(const ia_decoder* dec, const float* pos, int32_t pos_stride, int64_t N, float t,
                                    const ia_gaussians* grad_attr, const float* grad_means, float* grad_pos,
                                    const ia_decoder_grads* grads, const void* features, size_t features_bytes,
                                    void* ws, size_t ws_bytes, void* stream);

IA_API void ia_decoder_destroy(ia_decoder* dec);

/* ------------------------------------------------------------------------ */
/* HexPlane deformation: [HEX] §3.1-3.2, §6.1                                */
/* ------------------------------------------------------------------------ */

/* Six planes XY, XZ, YZ ([res_xyz][res_xyz][C]) and XT, YT, ZT
 * ([res_t][res_xyz][C], time on the slow axis), fp16, bilinear with vertices
 * at 0..res-1, positions mapped to [0,1] by the box [-aabb, aabb]^3 (clamped),
 * concatenated to 6C features -> MLP 6C -> 256 -> 256 -> 58 (ReLU hidden,
 * fp16 MFMA, fp32 accumulate).  Supported: C = 32, res_xyz, res_t in 2..4096. */
typedef struct {
    int32_t res_xyz;
    int32_t res_t;
    int32_t channels;
    float aabb;
} ia_hexplane_desc;

typedef struct ia_hexplane ia_hexplane;

IA_API ia_status ia_hexplane_create(const ia_hexplane_desc* desc, ia_hexplane** out);

/* planes: 6 pointers (order XY XZ YZ XT YT ZT) to fp16 [res_b][res_a][C];
 * weights: 3 pointers to fp16 [256][6C], [256][256], [58][256];
 * biases: 3 pointers to fp32.  Same ownership rules as ia_decoder_set_params. */
IA_API ia_status ia_hexplane_set_params(ia_hexplane* hp, const void* const* planes, const void* const* weights,
                                 const float* const* biases, int32_t params_on_device, void* stream);

/* Deform N canonical Gaussians to time t in [0,1]:
 *   means' = means + dpos;  quats' = normalize(quats + dquat);
 *   scales' = scales * exp(dlog_scale);  sh' = sh + dsh;  opacity' = opacity.
 * canonical: means[N,3], scales, quats, sh[N,16,3], opacity (device);
 * out: the same fields (device, may not alias canonical).  means_stride must be
 * 0 or 3.  Errors: INVALID_ARG, params not set. */
IA_API ia_status ia_hexplane_deform(const ia_hexplane* hp, const ia_gaussians* canonical, int64_t N, float t,
                             const ia_gaussians* out, void* stream);

IA_API void ia_hexplane_destroy(ia_hexplane* hp);

/* ------------------------------------------------------------------------ */
/* Render: [SPIN] §3.1 Eq. 1-4, 16x16 tiles                                  */
/* ------------------------------------------------------------------------ */

/* Spatial order of the Gaussians of each frame (a storage layout, not a step
 * of the method).  Every frame is a fixed set of positions ([SPIN] §3.2), and
 * the order of a frame's Gaussians changes neither a decoded attribute nor a
 * composited pixel (compositing follows depth, ties in index order), but it
 * does change the hash gather's traffic: Gaussians close in space share the
 * coarse levels' grid cells, and cache lines when they sit in one wave.
 *   pos: device [N, pos_stride] (x, y, z first; e.g. xyzt rows, stride 4);
 *   frame_offsets: host [frames + 1], 0 = first, N = last, non-decreasing;
 *   perm: device uint32 [N] out: new position i holds old index perm[i];
 *         every frame's range maps onto itself, its Gaussians in the order of
 *         a Morton curve over the normalised positions of Eq. 7 (10 bits per
 *         axis; fewer only when frame, cell and index do not fit 64 bits),
 *         equal cells in index order;
 *   pos_out: device [N, pos_stride] or NULL: pos_out[i] = pos[perm[i]] (must
 *         not overlap pos);
 *   ws: ia_spatial_order_workspace_size bytes (16 per Gaussian + 8 per
 *         frame + radix counts), 256-byte aligned.
 * One-time data preparation: decode, render and their backwards take the
 * reordered positions as they are.
 * Errors: INVALID_ARG (N outside [0, 2^32), frames outside 1..65535, bad
 * offsets, null or overlapping buffers), WORKSPACE_TOO_SMALL, DEVICE. */
IA_API ia_status ia_spatial_order_workspace_size(int64_t N, int32_t frames, size_t* bytes);
IA_API ia_status ia_spatial_order(const float* pos, int32_t pos_stride, int64_t N, const int64_t* frame_offsets,
                                  int32_t frames, uint32_t* perm, float* pos_out, void* ws, size_t ws_bytes,
                                  void* stream);

/* Pinhole camera, OpenCV axes (x right, y down, z forward).
 * p_cam = R p_world + t; u = fx x/z + cx; v = fy y/z + cy; pixel (i, j) has
 * its centre at (i + 0.5, j + 0.5).  Gaussians with z <= near_z are culled. */
typedef struct {
    float R[9]; /* row-major world->camera rotation */
    float t[3];
    float fx, fy, cx, cy, near_z;
    int32_t W, H;
    float bg[3]; /* background colour added as T_final * bg */
} ia_camera;

/* Optional outputs of ia_render.  Device pointers may be NULL.  The view
 * fields are filled by ia_render (host-side) and point into the workspace;
 * they stay valid until the workspace is reused. */
typedef struct {
    float* T_final;      /* device [F,H,W] final transmittance, or NULL          */
    uint32_t* n_contrib; /* device [F,H,W] 1 + list position of the last
                            composited Gaussian (0 = none), or NULL               */
    uint64_t* n_entries; /* device [1] tile entries emitted (true count), or NULL */
    uint32_t* overflow;  /* device [1] 1 if n_entries > max_entries, or NULL       */
    /* views (written by ia_render) */
    const uint64_t* sorted_keys;  /* [min(E,max_entries)] (tile<<32 | depth bits);
                                     only with want_keys                        */
    const uint32_t* sorted_vals;  /* [min(E,max_entries)] Gaussian index          */
    const uint32_t* tile_ranges;  /* [F*tiles][2] [start,end), empty = [0,0)      */
    /* projections: defined where tiles_touched > 0 (a culled Gaussian's
       entries are not written)                                               */
    const float* proj_a;          /* [N][4] u, v, conic A, conic B                */
    const float* proj_b;          /* [N][4] conic C, opacity, red, green          */
    const float* proj_c;          /* [N] blue                                     */
    const float* depth;           /* [N] camera-space z                           */
    const uint32_t* tiles_touched;/* [N] 0 = culled                               */
    const uint16_t* tile_rect;    /* [N][4] tx0, ty0, tx1, ty1 (inclusive)        */
    /* inputs */
    int32_t want_keys;  /* nonzero: also fill sorted_keys / sorted_vals (one
                           extra pass over the entries); else both stay NULL */
    int32_t binning;    /* how depth-ordered Gaussians become per-tile lists;
                           both methods give the same lists, they differ in
                           speed (a NULL aux means IA_BINNING_AUTO):
      IA_BINNING_AUTO       regions when visible Gaussians touch 4 or more
                            tiles on average, else the tile sort;
      IA_BINNING_TILE_SORT  one entry per (Gaussian, tile), stable radix sort
                            on the tile index;
      IA_BINNING_REGIONS    one entry per (Gaussian, 8x8-tile region), stable
                            radix sort on the region index, then per region a
                            count pass and a write pass that place every
                            (Gaussian, tile) entry at its final position.
                            Other values: IA_ERR_INVALID_ARG. */
} ia_render_aux;

#define IA_BINNING_AUTO 0
#define IA_BINNING_TILE_SORT 1
#define IA_BINNING_REGIONS 2

/* Bytes of workspace ia_render needs for N_total Gaussians over `frames`
 * frames of W x H with room for max_entries tile entries.
 * Errors: INVALID_ARG (negative or zero sizes, max_entries >= 2^32). */
IA_API ia_status ia_render_workspace_size(int64_t N_total, int32_t frames, int32_t W, int32_t H,
                                   int64_t max_entries, size_t* bytes);

/* Render a batch of frames.  Gaussians [frame_offsets[f], frame_offsets[f+1])
 * of g belong to frame f and are seen by cams[f]; all cameras share W x H.
 *   frame_offsets: host [frames+1], frame_offsets[0] = 0, non-decreasing.
 *   cams: host [frames].  Both host arrays may be freed on return.
 *   ws: device workspace of ws_bytes >= ia_render_workspace_size(...).
 *   image: device [frames,3,H,W] = C + T_final * bg.
 * Steps: EWA projection -> tiles touched -> one entry per (Gaussian, tile),
 * ordered by the key (frame*tiles + tile) << 32 | depth bits with ties in
 * Gaussian-index order (stable radix sort of the visible Gaussians on depth,
 * then of the entries on the tile) -> per-tile ranges -> front-to-back
 * compositing per pixel with
 * a 3-sigma cutoff, alpha = min(0.99, o G), skip alpha < 1/255, stop once
 * T < 1e-4.  No host synchronisation: if more than max_entries entries are
 * needed, the surplus is dropped, aux->overflow is set to 1 and
 * aux->n_entries holds the needed count; the image is then incomplete and
 * the caller retries with a larger max_entries.
 * Errors: INVALID_ARG (also an unknown aux->binning), UNSUPPORTED (sh_degree
 * not -1/3), WORKSPACE_TOO_SMALL, DEVICE. */
IA_API ia_status ia_render(const ia_gaussians* g, const int64_t* frame_offsets, int32_t frames, const ia_camera* cams,
                    void* ws, size_t ws_bytes, int64_t max_entries, float* image, ia_render_aux* aux,
                    void* stream);

/* Per-Gaussian gradient buffers (device, float32, packed rows). */
typedef struct {
    float* means;   /* [N][3] dL/dmean                                   */
    float* scales;  /* [N][3] dL/dscale                                  */
    float* quats;   /* [N][4] dL/dquaternion (of the unnormalised input) */
    float* opacity; /* [N]    dL/dopacity                                */
    float* colors;  /* [N][3] dL/dcolour (the rendered colour)           */
    float* sh;      /* [N][16][3] dL/dsh when the render used sh_degree 3
                     * (then also added into means: the view direction's
                     * share); unused otherwise                           */
} ia_gaussian_grads;

/* Backward of ia_render for an image-space gradient ([SPIN] §3.1 Eq. 1-4,
 * and the EWA projection of Eq. 2-3 differentiated).  Takes exactly the
 * arguments of a preceding ia_render call (same g, frame_offsets, cams, ws,
 * max_entries) whose aux produced T_final and n_contrib, and which reported
 * no overflow; the workspace must not have been reused in between (the tile
 * lists and projections are read from it).
 *   grad_image: device [F,3,H,W] dL/dimage.
 *   T_final, n_contrib: device [F,H,W], as written by that ia_render.
 *   grads: device outputs, [N] rows each; overwritten (culled Gaussians get 0).
 * Per pixel the composited Gaussians are revisited from the last to the
 * first, recovering T_i = T_{i+1} / (1 - alpha_i); alpha clamped at 0.99
 * passes no gradient to opacity or position.  Per-Gaussian partials are
 * summed with float atomics, so results vary in the last bits from run to
 * run.  The chain to means, scales and quaternions is through the conic
 * inverse, Sigma2D = J W Sigma W^T J^T and Sigma = R S S^T R^T.  With
 * degree-3 SH colours (sh_degree 3, grads->sh required) the colour gradient
 * is chained through colour = max(0, sum_k sh_k Y_k(dir) + 1/2) to
 * grads->sh, and through dir = normalize(mu - camera centre) into
 * grads->means.
 * Errors: INVALID_ARG, WORKSPACE_TOO_SMALL, DEVICE. */
IA_API ia_status ia_render_backward(const ia_gaussians* g, const int64_t* frame_offsets, int32_t frames,
                                    const ia_camera* cams, void* ws, size_t ws_bytes, int64_t max_entries,
                                    const float* grad_image, const float* T_final, const uint32_t* n_contrib,
                                    const ia_gaussian_grads* grads, void* stream);

/* L1 image loss: *loss = mean |image - target| (device double, overwritten)
 * and grad_image = sign(image - target) / n (0 where they are equal), over n
 * floats of device memory.  Errors: INVALID_ARG, DEVICE. */
IA_API ia_status ia_l1_loss(const float* image, const float* target, int64_t n, double* loss, float* grad_image,
                            void* stream);

/* The training objective of [SPIN] §3.3 Eq. 12 on frames x 3 x H x W images
 * (device, planar, values nominally in [0, 1]):
 *   L = (1 - lambda) L1 + lambda (1 - SSIM),
 * L1 the mean absolute difference and SSIM the structural similarity of
 * Wang et al. (2004), the metric the pages cite: 11 x 11 Gaussian window of
 * standard deviation 1.5, C1 = 0.01^2, C2 = 0.03^2, per colour channel,
 * window taps outside the image counted as zero, averaged over every pixel,
 * channel and frame.  The pages set lambda = 0.2 (after 3DGS).
 *   loss       : device double[3], overwritten: {L, L1, SSIM}; the per-pixel
 *                terms are summed in a fixed order (the same on every run)
 *   grad_image : device float, like image: dL/dimage (the L1 part 0 where
 *                image == target)
 *   ws         : caller-owned device workspace of ia_image_loss_workspace_size
 *                bytes, 256-byte aligned; contents undefined between calls.
 * Asynchronous on stream; calls on one workspace must not overlap.
 * Errors: INVALID_ARG (null, sizes <= 0, lambda outside [0, 1], more than
 * 21845 frames), WORKSPACE_TOO_SMALL, DEVICE. */
IA_API ia_status ia_image_loss_workspace_size(int32_t frames, int32_t H, int32_t W, size_t* bytes);
IA_API ia_status ia_image_loss(const float* image, const float* target, int32_t frames, int32_t H, int32_t W,
                               float lambda, void* ws, size_t ws_bytes, double* loss, float* grad_image,
                               void* stream);

/* One Adam step (Kingma & Ba 2015; the optimiser of [SPIN] §4 implementation
 * details) over n fp32 parameters, in place, step >= 1:
 *   m = beta1 m + (1 - beta1) g,  v = beta2 v + (1 - beta2) g^2,
 *   param -= lr (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps).
 * param, grad, m, v are device float[n] (m and v zero before the first step);
 * param_f16 (nullable) receives the updated values rounded to fp16 (RNE), e.g.
 * for an fp16 hash table.  Per-group learning rates are the caller's (one
 * call per group, the rate from ia_lr_at).  Errors: INVALID_ARG, DEVICE. */
IA_API ia_status ia_adam_step(float* param, const float* grad, float* m, float* v, int64_t n, float lr, float beta1,
                              float beta2, float eps, int32_t step, uint16_t* param_f16, void* stream);

/* The learning-rate schedule of [SPIN] §4 implementation details: at
 * iteration `step` (0-based), a linear warm-up base (step + 1) / warmup over
 * the first `warmup` iterations, then a cosine decay from base_lr at
 * iteration warmup to final_lr at iteration total (and final_lr after it):
 *   lr = final + (base - final) (1 + cos(pi min(step - warmup, span) / span)) / 2,
 * span = max(total - warmup, 1), evaluated in double and rounded to float.
 * Host-only, no device work.  Errors: INVALID_ARG (null lr, step < 0,
 * warmup < 0, total < warmup, non-finite or negative rates). */
IA_API ia_status ia_lr_at(float base_lr, int32_t step, int32_t warmup, int32_t total, float final_lr, float* lr);

/* ia_adam_step for a parameter laid out as rows of `dim` values that sit
 * `param_stride` floats apart (dim <= param_stride), e.g. the x, y, z of
 * positions stored as [rows][4] (x, y, z, t), leaving the other values of a
 * row untouched.  grad, m, v are dense device float[rows][dim].
 * Errors: INVALID_ARG (rows < 0, dim < 1, param_stride < dim, ...), DEVICE. */
IA_API ia_status ia_adam_step_strided(float* param, int32_t param_stride, int32_t dim, const float* grad, float* m,
                                      float* v, int64_t rows, float lr, float beta1, float beta2, float eps,
                                      int32_t step, void* stream);

/* Refinement of the positions ([SPIN] §3.2 Eq. 6: the rendering loss
 * densifies salient points and prunes unnecessary ones; the rule is read as
 * 3D Gaussian Splatting's adaptive density control on the trainable
 * positions, the other attributes being decoded):
 *   prune  decoded opacity < min_opacity (first);
 *   salient  grad_count > 0 and grad_acc / grad_count >= grad_threshold
 *          (one fp32 division);
 *   clone  salient and max(scale) <= scale_threshold: the Gaussian (with its
 *          moments) and a copy at the same position (moments 0);
 *   split  salient and larger: two Gaussians at mu + R(q) (s * n_j), j = 0, 1,
 *          n = noise[i][j][0..2] (standard normal draws the caller supplies),
 *          time carried over, moments 0;
 *   keep   otherwise, with its moments.
 * Outputs keep the input order (a Gaussian's rows follow its predecessors').
 * All arrays are device memory:
 *   xyzt [N][4] (16-byte aligned), grad_acc [N], grad_count [N] (as left by
 *   ia_densify_accumulate), scales [N][3], quats [N][4] (w,x,y,z, any
 *   non-zero norm), opacity [N] (decoded), noise [N][2][3], m, v [N][3] (the
 *   positions' Adam moments);
 *   out_xyzt [out_capacity][4] (16-byte aligned), out_m, out_v
 *   [out_capacity][3], out_capacity >= 2 N; out_n: device int64, the rows
 *   written (no host synchronisation);
 *   ws: ia_densify_workspace_size bytes, contents undefined between calls.
 * The accumulators are not reset here (zero them after a densification).
 * Errors: INVALID_ARG (null, N < 0, out_capacity < 2 N, misalignment,
 * negative thresholds), WORKSPACE_TOO_SMALL, DEVICE. */
typedef struct {
    float grad_threshold;  /* mean position-gradient norm that makes a Gaussian salient */
    float scale_threshold; /* largest decoded scale up to which a salient one is cloned */
    float min_opacity;     /* decoded opacity below which a Gaussian is pruned        */
} ia_densify_params;

/* grad_acc[i] += |grad_pos[i]| and grad_count[i] += 1 for every Gaussian whose
 * position gradient (device [N][3]) is not zero; |.| is sqrtf((x^2 + y^2) + z^2).
 * Errors: INVALID_ARG, DEVICE. */
IA_API ia_status ia_densify_accumulate(const float* grad_pos, int64_t N, float* grad_acc, int32_t* grad_count,
                                       void* stream);
IA_API ia_status ia_densify_workspace_size(int64_t N, size_t* bytes);
IA_API ia_status ia_densify(const float* xyzt, const float* grad_acc, const int32_t* grad_count, const float* scales,
                            const float* quats, const float* opacity, const float* noise, const float* m,
                            const float* v, int64_t N, const ia_densify_params* params, float* out_xyzt,
                            float* out_m, float* out_v, int64_t out_capacity, int64_t* out_n, void* ws,
                            size_t ws_bytes, void* stream);


/* ------------------------------------------------------------------------ */
/* Diagnostics: per-kernel timing with HIP events                            */
/* ------------------------------------------------------------------------ */

/* Enable (on != 0) or disable timing.  While enabled, every kernel launch of
 * the library is bracketed by two HIP events recorded on its launch stream.
 * Process-wide; safe to call at any time.  Returns IA_OK. */
IA_API ia_status ia_profile_enable(int32_t on);

/* Wait for the recorded events and write a JSON object
 * {"kernel name": [calls, total milliseconds], ...} accumulated since the last
 * reset into buf (host, len bytes).  *needed (nullable) receives the size
 * required including the terminating zero.  Errors: INVALID_ARG if buf is
 * null or too small (needed is still set). */
IA_API ia_status ia_profile_report(char* buf, size_t len, size_t* needed);

/* Drop all recorded timings. */
IA_API void ia_profile_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* IA_H_ */
