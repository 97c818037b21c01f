// C ABI of libia.so (declared in include/ia.h): argument validation, handle
// management and launch orchestration.  Every check runs before the first
// HIP call of an entry point, so invalid arguments never enqueue work.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "ia_internal.h"

namespace {

thread_local std::string g_err;

ia_status fail(ia_status s, const std::string& msg) {
    g_err = msg;
    return s;
}

ia_status hip_fail(hipError_t e, const char* what) {
    return fail(IA_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Copy bytes into a fresh device allocation; host sources are copied
// synchronously so the caller may free them on return.
ia_status upload_param(void** dst, const void* src, size_t bytes, bool on_device, hipStream_t s) {
    void* d = nullptr;
    hipError_t e = hipMalloc(&d, bytes);
    if (e != hipSuccess) return fail(IA_ERR_OUT_OF_MEMORY, std::string("hipMalloc: ") + hipGetErrorString(e));
    if (on_device)
        e = hipMemcpyAsync(d, src, bytes, hipMemcpyDeviceToDevice, s);
    else
        e = hipMemcpy(d, src, bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return hip_fail(e, "parameter copy");
    }
    *dst = d;
    return IA_OK;
}

}  // namespace

// ============================================================== decoder

struct ia_decoder {
    ia_hash_desc hash;
    ia_mlp_desc mlp;
    ia::HashLevels lv;
    int n_layers;  // layers of one chain (trunk + head, or one attribute branch)
    int dims[6];   // shared: dims[0] = in, dims[k+1] = out of layer k; last = 11 (RGB) or 56 (SH3)
    int n_mats;    // weight matrices: n_layers (shared) or 4 n_layers (per attribute)
    int mat_in[ia::kMaxDecoderMats], mat_out[ia::kMaxDecoderMats];
    void* tables = nullptr;
    void* W[ia::kMaxDecoderMats] = {};
    float* b[ia::kMaxDecoderMats] = {};
    void* Wt = nullptr;         // per-attribute fp16 decoder: weights in MFMA A-tile order
    float* bpack = nullptr;     // per-attribute fp16 decoder: biases packed per branch
    bool ready = false;
};

namespace {

void free_decoder_params(ia_decoder* d) {
    if (d->tables) (void)hipFree(d->tables);
    for (int k = 0; k < ia::kMaxDecoderMats; ++k) {
        if (d->W[k]) (void)hipFree(d->W[k]);
        if (d->b[k]) (void)hipFree(d->b[k]);
        d->W[k] = nullptr;
        d->b[k] = nullptr;
    }
    if (d->Wt) (void)hipFree(d->Wt);
    if (d->bpack) (void)hipFree(d->bpack);
    d->Wt = nullptr;
    d->bpack = nullptr;
    d->tables = nullptr;
    d->ready = false;
}

ia_status check_hash(const ia_hash_desc* h, ia::HashLevels* lv) {
    if (h->L < 1 || h->L > ia::kMaxLevels) return fail(IA_ERR_INVALID_ARG, "hash.L must be in 1..32");
    if (h->F != 2 && h->F != 4) return fail(IA_ERR_UNSUPPORTED, "hash.F must be 2 or 4");
    if (h->F == 4 && h->table_dtype != IA_DTYPE_F16) return fail(IA_ERR_UNSUPPORTED, "hash.F = 4 needs an fp16 table");
    if (h->log2T < 4 || h->log2T > 24) return fail(IA_ERR_INVALID_ARG, "hash.log2T must be in 4..24");
    if (!(std::isfinite(h->base_res) && h->base_res >= 2.0)) return fail(IA_ERR_INVALID_ARG, "hash.base_res must be >= 2");
    if (!(std::isfinite(h->growth) && h->growth >= 1.0)) return fail(IA_ERR_INVALID_ARG, "hash.growth must be >= 1");
    if (h->temporal_res < 0 || h->temporal_res == 1) return fail(IA_ERR_INVALID_ARG, "hash.temporal_res must be 0 or >= 2");
    if (h->table_dtype != IA_DTYPE_F32 && h->table_dtype != IA_DTYPE_F16)
        return fail(IA_ERR_INVALID_ARG, "hash.table_dtype must be F32 or F16");
    if (!(std::isfinite(h->t_min) && std::isfinite(h->t_max) && h->t_max > h->t_min))
        return fail(IA_ERR_INVALID_ARG, "hash.t_max must exceed hash.t_min");
    lv->L = h->L;
    lv->F = h->F;
    lv->T = 1u << h->log2T;
    lv->mask = lv->T - 1u;
    lv->table_f16 = h->table_dtype == IA_DTYPE_F16;
    lv->t_min = h->t_min;
    lv->t_max = h->t_max;
    for (int l = 0; l < h->L; ++l) {
        double r = std::floor(h->base_res * std::pow(h->growth, (double)l));
        if (r > 1e6) return fail(IA_ERR_INVALID_ARG, "level resolution above 1e6");
        int res = (int)r;
        int rt = h->temporal_res > 0 ? h->temporal_res : res;
        lv->res_s[l] = res;
        lv->res_t[l] = rt;
        lv->dense[l] = ((double)res * res * res * rt) <= (double)lv->T;
    }
    return IA_OK;
}

ia_status check_mlp(const ia_hash_desc* h, const ia_mlp_desc* m) {
    if (m->in_dim != h->L * h->F) return fail(IA_ERR_INVALID_ARG, "mlp.in_dim must equal L*F");
    if (m->n_hidden < 1 || m->n_hidden > 2) return fail(IA_ERR_UNSUPPORTED, "mlp.n_hidden must be 1 or 2");
    if (m->activation != IA_ACT_RELU && m->activation != IA_ACT_GELU)
        return fail(IA_ERR_INVALID_ARG, "mlp.activation must be RELU or GELU");
    if (m->color != IA_COLOR_RGB && m->color != IA_COLOR_SH3)
        return fail(IA_ERR_INVALID_ARG, "mlp.color must be RGB or SH3");
    if (m->color == IA_COLOR_SH3 && m->dtype != IA_DTYPE_F16)
        return fail(IA_ERR_UNSUPPORTED, "the SH colour head is supported on the fp16 decoder");
    if (m->branches != IA_BRANCHES_SHARED && m->branches != IA_BRANCHES_PER_ATTRIBUTE)
        return fail(IA_ERR_INVALID_ARG, "mlp.branches must be SHARED or PER_ATTRIBUTE");
    if (m->branches == IA_BRANCHES_PER_ATTRIBUTE) {
        if (!(m->dtype == IA_DTYPE_F16 && h->F == 4 && m->in_dim == 64 && m->n_hidden == 2 && m->hidden[0] == 64 &&
              m->hidden[1] == 64))
            return fail(IA_ERR_UNSUPPORTED, "per-attribute decoders: fp16, F = 4, 64 -> 64 -> 64 -> out only");
        return IA_OK;
    }
    if (h->F != 2) return fail(IA_ERR_UNSUPPORTED, "shared-trunk decoders need F = 2");
    for (int k = 0; k < m->n_hidden; ++k)
        if (m->hidden[k] < 1 || m->hidden[k] > 1024) return fail(IA_ERR_INVALID_ARG, "mlp.hidden width out of range");
    if (m->dtype == IA_DTYPE_F16) {
        if (!(m->in_dim == 32 && m->n_hidden == 2 && m->hidden[0] == 64 && m->hidden[1] == 64))
            return fail(IA_ERR_UNSUPPORTED, "fp16 decoder supports a 32 -> 64 -> 64 trunk only");
        if (h->table_dtype != IA_DTYPE_F16) return fail(IA_ERR_UNSUPPORTED, "fp16 decoder needs an fp16 hash table");
        return IA_OK;
    }
    if (m->dtype != IA_DTYPE_F32) return fail(IA_ERR_INVALID_ARG, "mlp.dtype must be F32 or F16");
    const bool ok = (m->in_dim == 8 && m->n_hidden == 1 && m->hidden[0] == 32) ||
                    (m->in_dim == 32 && m->n_hidden == 1 && m->hidden[0] == 64) ||
                    (m->in_dim == 32 && m->n_hidden == 2 && m->hidden[0] == 64 && m->hidden[1] == 64);
    if (!ok) return fail(IA_ERR_UNSUPPORTED, "fp32 decoder supports 8->32->11, 32->64->11 and 32->64->64->11");
    return IA_OK;
}

bool outputs_ok(const ia_gaussians* o, bool sh) {
    return o && o->scales && o->quats && (sh ? o->sh != nullptr : o->colors != nullptr) && o->opacity;
}

// Launch arguments of a decode of N Gaussians (outputs left null).
ia::DecodeArgs decode_args(const ia_decoder* dec, const float* pos, int stride, float t, int64_t N) {
    ia::DecodeArgs a{};
    a.h = dec->lv;
    a.tables = dec->tables;
    if (dec->mlp.branches == IA_BRANCHES_SHARED)
        for (int k = 0; k < dec->n_layers; ++k) {
            a.W[k] = dec->W[k];
            a.b[k] = dec->b[k];
        }
    a.branches = dec->mlp.branches == IA_BRANCHES_PER_ATTRIBUTE;
    a.Wt = dec->Wt;
    a.bpack = dec->bpack;
    a.in_dim = dec->mlp.in_dim;
    a.n_hidden = dec->mlp.n_hidden;
    for (int k = 0; k < 4; ++k) a.hidden[k] = dec->mlp.hidden[k];
    a.act = dec->mlp.activation;
    a.sh_head = dec->mlp.color == IA_COLOR_SH3;
    a.pos = pos;
    a.stride = stride;
    a.t_scalar = t;
    a.N = N;
    return a;
}

size_t feature_bytes(const ia_decoder* dec, int64_t N) {
    return (size_t)(N > 0 ? N : 0) * (size_t)dec->hash.L * (size_t)dec->hash.F * 2;
}

// Checks a caller buffer for the decode's features (null allowed).
ia_status check_features(const ia_decoder* dec, int64_t N, const void* features, size_t bytes) {
    if (!features) return IA_OK;
    if (dec->mlp.dtype != IA_DTYPE_F16) return fail(IA_ERR_UNSUPPORTED, "features are kept by the fp16 decoder only");
    if (!aligned(features, 8)) return fail(IA_ERR_INVALID_ARG, "features must be 8-byte aligned");
    if (bytes < feature_bytes(dec, N))
        return fail(IA_ERR_INVALID_ARG, "features buffer too small: need " + std::to_string(feature_bytes(dec, N)) + " bytes");
    return IA_OK;
}

size_t decode_ws_bytes(const ia_decoder* dec, int64_t N) {
    if (dec->mlp.dtype != IA_DTYPE_F16 || N <= 0) return 0;
    return ia::decode_layout(dec->lv, N).total;
}

// Points the decode's scratch slots into a workspace laid out by decode_layout.
void set_scratch(ia::DecodeArgs& a, unsigned char* ws, const ia::DecodeLayout& lay) {
    for (int k = 0; k < 2; ++k) {
        a.zslot[k] = reinterpret_cast<uint32_t*>(ws + lay.z[k]);
        a.xt[k] = reinterpret_cast<float4*>(ws + lay.xt[k]);
    }
    a.zcap = lay.zcap;
}

ia_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return IA_OK;
    if (!ws || !aligned(ws, 256)) return fail(IA_ERR_INVALID_ARG, "workspace must be non-null and 256-byte aligned");
    if (ws_bytes < need)
        return fail(IA_ERR_WORKSPACE_TOO_SMALL, "workspace too small: need " + std::to_string(need) + " bytes");
    return IA_OK;
}

ia_status decode_common(const ia_decoder* dec, const float* pos, int stride, float t, int64_t N,
                        const ia_gaussians* out, void* features, size_t features_bytes, void* ws, size_t ws_bytes,
                        void* side_stream, void* stream) {
    if (!dec) return fail(IA_ERR_INVALID_ARG, "decoder is null");
    if (!dec->ready) return fail(IA_ERR_INVALID_ARG, "decoder parameters not set");
    if (N < 0) return fail(IA_ERR_INVALID_ARG, "N must be >= 0");
    if (N == 0) return IA_OK;
    if (!pos || !aligned(pos, 4)) return fail(IA_ERR_INVALID_ARG, "positions must be a non-null fp32 array");
    if (!outputs_ok(out, dec->mlp.color == IA_COLOR_SH3))
        return fail(IA_ERR_INVALID_ARG, "output scales/quats/colors (or sh)/opacity must be non-null");
    if (N > ((int64_t)1 << 40)) return fail(IA_ERR_INVALID_ARG, "N too large");
    ia_status fs = check_features(dec, N, features, features_bytes);
    if (fs != IA_OK) return fs;
    fs = check_ws(ws, ws_bytes, decode_ws_bytes(dec, N));
    if (fs != IA_OK) return fs;
    ia::DecodeArgs a = decode_args(dec, pos, stride, t, N);
    if (dec->mlp.dtype == IA_DTYPE_F16) set_scratch(a, static_cast<unsigned char*>(ws), ia::decode_layout(dec->lv, N));
    a.side = (hipStream_t)side_stream;
    a.features = static_cast<uint32_t*>(features);
    a.scales = out->scales;
    a.quats = out->quats;
    a.colors = out->colors;
    a.sh = out->sh;
    a.opacity = out->opacity;
    hipError_t e = ia::launch_decode(a, dec->mlp.dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return IA_OK;
}

}  // namespace

extern "C" {

const char* ia_last_error(void) { return g_err.c_str(); }

ia_status ia_decoder_create(const ia_hash_desc* hash, const ia_mlp_desc* mlp, ia_decoder** out) {
    if (!hash || !mlp || !out) return fail(IA_ERR_INVALID_ARG, "null argument");
    ia::HashLevels lv{};
    ia_status s = check_hash(hash, &lv);
    if (s != IA_OK) return s;
    s = check_mlp(hash, mlp);
    if (s != IA_OK) return s;
    ia_decoder* d = new (std::nothrow) ia_decoder();
    if (!d) return fail(IA_ERR_OUT_OF_MEMORY, "host allocation failed");
    d->hash = *hash;
    d->mlp = *mlp;
    d->lv = lv;
    d->n_layers = mlp->n_hidden + 1;
    d->dims[0] = mlp->in_dim;
    for (int k = 0; k < mlp->n_hidden; ++k) d->dims[k + 1] = mlp->hidden[k];
    d->dims[d->n_layers] = mlp->color == IA_COLOR_SH3 ? 56 : 11;
    if (mlp->branches == IA_BRANCHES_SHARED) {
        d->n_mats = d->n_layers;
        for (int k = 0; k < d->n_layers; ++k) {
            d->mat_in[k] = d->dims[k];
            d->mat_out[k] = d->dims[k + 1];
        }
    } else {
        // branch a: in -> hidden... -> out_a, out_a = scale 3, rotation 4, colour 3 / 48, opacity 1
        const int outs[4] = {3, 4, mlp->color == IA_COLOR_SH3 ? 48 : 3, 1};
        d->n_mats = 4 * d->n_layers;
        for (int br = 0; br < 4; ++br)
            for (int k = 0; k < d->n_layers; ++k) {
                d->mat_in[br * d->n_layers + k] = d->dims[k];
                d->mat_out[br * d->n_layers + k] = k + 1 < d->n_layers ? d->dims[k + 1] : outs[br];
            }
    }
    *out = d;
    return IA_OK;
}

ia_status ia_decoder_set_params(ia_decoder* dec, const void* tables, const void* const* weights,
                                const float* const* biases, int32_t params_on_device, void* stream) {
    if (!dec || !tables || !weights || !biases) return fail(IA_ERR_INVALID_ARG, "null argument");
    for (int k = 0; k < dec->n_mats; ++k)
        if (!weights[k] || !biases[k]) return fail(IA_ERR_INVALID_ARG, "null weight or bias pointer");
    const bool dev = params_on_device != 0;
    hipStream_t s = (hipStream_t)stream;
    if (dec->tables) {
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
        free_decoder_params(dec);
    }
    const size_t tsize = dec->hash.table_dtype == IA_DTYPE_F16 ? 2 : 4;
    const size_t tbytes = (size_t)dec->hash.L * dec->lv.T * dec->hash.F * tsize;
    ia_status st = upload_param(&dec->tables, tables, tbytes, dev, s);
    const size_t wsize = dec->mlp.dtype == IA_DTYPE_F16 ? 2 : 4;
    for (int k = 0; st == IA_OK && k < dec->n_mats; ++k) {
        const size_t nw = (size_t)dec->mat_out[k] * dec->mat_in[k];
        st = upload_param(&dec->W[k], weights[k], nw * wsize, dev, s);
        if (st == IA_OK) st = upload_param(reinterpret_cast<void**>(&dec->b[k]), biases[k], 4 * (size_t)dec->mat_out[k], dev, s);
    }
    if (st == IA_OK && dec->mlp.branches == IA_BRANCHES_PER_ATTRIBUTE) {
        const bool sh = dec->mlp.color == IA_COLOR_SH3;
        hipError_t e = hipMalloc(&dec->Wt, ia::branch_tile_bytes(sh));
        if (e == hipSuccess) e = hipMalloc(&dec->bpack, ia::branch_bias_bytes(sh));
        if (e != hipSuccess) {
            st = fail(IA_ERR_OUT_OF_MEMORY, std::string("hipMalloc: ") + hipGetErrorString(e));
        } else {
            e = ia::launch_branch_pack((const _Float16* const*)dec->W, (const float* const*)dec->b, sh, dec->Wt,
                                       dec->bpack, s);
            if (e != hipSuccess) st = hip_fail(e, "decoder weight tiling");
        }
    }
    if (st != IA_OK) {
        free_decoder_params(dec);
        return st;
    }
    dec->ready = true;
    return IA_OK;
}

ia_status ia_decoder_update_params(ia_decoder* dec, const void* tables, const void* const* weights,
                                   const float* const* biases, void* stream) {
    if (!dec || !tables || !weights || !biases) return fail(IA_ERR_INVALID_ARG, "null argument");
    if (!dec->ready) return fail(IA_ERR_INVALID_ARG, "decoder parameters not set");
    for (int k = 0; k < dec->n_mats; ++k)
        if (!weights[k] || !biases[k]) return fail(IA_ERR_INVALID_ARG, "null weight or bias pointer");
    hipStream_t s = (hipStream_t)stream;
    const size_t tsize = dec->hash.table_dtype == IA_DTYPE_F16 ? 2 : 4;
    const size_t wsize = dec->mlp.dtype == IA_DTYPE_F16 ? 2 : 4;
    hipError_t e = hipMemcpyAsync(dec->tables, tables, (size_t)dec->hash.L * dec->lv.T * dec->hash.F * tsize,
                                  hipMemcpyDeviceToDevice, s);
    for (int k = 0; e == hipSuccess && k < dec->n_mats; ++k) {
        e = hipMemcpyAsync(dec->W[k], weights[k], (size_t)dec->mat_out[k] * dec->mat_in[k] * wsize,
                           hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(dec->b[k], biases[k], 4 * (size_t)dec->mat_out[k], hipMemcpyDeviceToDevice, s);
    }
    if (e == hipSuccess && dec->mlp.branches == IA_BRANCHES_PER_ATTRIBUTE)
        e = ia::launch_branch_pack((const _Float16* const*)dec->W, (const float* const*)dec->b,
                                   dec->mlp.color == IA_COLOR_SH3, dec->Wt, dec->bpack, s);
    if (e != hipSuccess) return hip_fail(e, "decoder parameter update");
    return IA_OK;
}

ia_status ia_decode_workspace_size(const ia_decoder* dec, int64_t N, size_t* bytes) {
    if (!dec || !bytes) return fail(IA_ERR_INVALID_ARG, "null argument");
    if (N < 0) return fail(IA_ERR_INVALID_ARG, "N must be >= 0");
    *bytes = decode_ws_bytes(dec, N);
    return IA_OK;
}

ia_status ia_decode(const ia_decoder* dec, const float* xyz, int64_t N, float t, const ia_gaussians* out, void* ws,
                    size_t ws_bytes, void* side_stream, void* stream) {
    if (!std::isfinite(t)) return fail(IA_ERR_INVALID_ARG, "t must be finite");
    return decode_common(dec, xyz, 3, t, N, out, nullptr, 0, ws, ws_bytes, side_stream, stream);
}

ia_status ia_decode_xyzt(const ia_decoder* dec, const float* xyzt, int64_t N, const ia_gaussians* out, void* ws,
                         size_t ws_bytes, void* side_stream, void* stream) {
    return decode_common(dec, xyzt, 4, 0.0f, N, out, nullptr, 0, ws, ws_bytes, side_stream, stream);
}

ia_status ia_decode_feature_bytes(const ia_decoder* dec, int64_t N, size_t* bytes) {
    if (!dec || !bytes) return fail(IA_ERR_INVALID_ARG, "null argument");
    if (N < 0) return fail(IA_ERR_INVALID_ARG, "N must be >= 0");
    *bytes = feature_bytes(dec, N);
    return IA_OK;
}

ia_status ia_decode_keep(const ia_decoder* dec, const float* pos, int32_t pos_stride, int64_t N, float t,
                         const ia_gaussians* out, void* features, size_t features_bytes, void* ws, size_t ws_bytes,
                         void* side_stream, void* stream) {
    if (pos_stride != 3 && pos_stride != 4) return fail(IA_ERR_INVALID_ARG, "pos_stride must be 3 or 4");
    if (pos_stride == 3 && !std::isfinite(t)) return fail(IA_ERR_INVALID_ARG, "t must be finite");
    if (!features && N > 0) return fail(IA_ERR_INVALID_ARG, "features is null");
    return decode_common(dec, pos, pos_stride, t, N, out, features, features_bytes, ws, ws_bytes, side_stream, stream);
}

namespace {
// every fp16 decoder: the shared trunk (RGB or SH head) and the per-attribute branches
bool backward_supported(const ia_decoder* dec) { return dec->mlp.dtype == IA_DTYPE_F16; }
}  // namespace

ia_status ia_decode_backward_workspace_size(const ia_decoder* dec, int64_t N, size_t* bytes) {
    if (!dec || !bytes) return fail(IA_ERR_INVALID_ARG, "null argument");
    if (N < 0) return fail(IA_ERR_INVALID_ARG, "N must be >= 0");
    if (!backward_supported(dec))
        return fail(IA_ERR_UNSUPPORTED, "the decode backward supports the fp16 decoders");
    *bytes = ia::decode_bwd_layout(dec->lv, N).total;
    return IA_OK;
}

ia_status ia_decode_backward(const ia_decoder* dec, const float* pos, int32_t pos_stride, int64_t N, float t,
                             const ia_gaussians* grad_attr, const float* grad_means, float* grad_pos,
                             const ia_decoder_grads* grads, const void* features, size_t features_bytes, void* ws,
                             size_t ws_bytes, void* stream) {
    if (!dec) return fail(IA_ERR_INVALID_ARG, "decoder is null");
    if (!dec->ready) return fail(IA_ERR_INVALID_ARG, "decoder parameters not set");
    if (!backward_supported(dec))
        return fail(IA_ERR_UNSUPPORTED, "the decode backward supports the fp16 decoders");
    if (pos_stride != 3 && pos_stride != 4) return fail(IA_ERR_INVALID_ARG, "pos_stride must be 3 or 4");
    if (pos_stride == 3 && !std::isfinite(t)) return fail(IA_ERR_INVALID_ARG, "t must be finite");
    if (N < 0 || N > ((int64_t)1 << 40)) return fail(IA_ERR_INVALID_ARG, "N must be in [0, 2^40]");
    if (!grads || !grads->tables) return fail(IA_ERR_INVALID_ARG, "gradient outputs must be non-null");
    for (int k = 0; k < dec->n_mats; ++k)
        if (!grads->weights[k] || !grads->biases[k]) return fail(IA_ERR_INVALID_ARG, "null weight or bias gradient");
    if (N > 0) {
        if (!pos || !aligned(pos, 4)) return fail(IA_ERR_INVALID_ARG, "positions must be a non-null fp32 array");
        if (!outputs_ok(grad_attr, dec->mlp.color == IA_COLOR_SH3))
            return fail(IA_ERR_INVALID_ARG, "grad_attr scales/quats/colors (sh for the SH head)/opacity must be non-null");
    }
    ia_status fs = check_features(dec, N, features, features_bytes);
    if (fs != IA_OK) return fs;
    fs = check_ws(ws, ws_bytes, ia::decode_bwd_layout(dec->lv, N).total);
    if (fs != IA_OK) return fs;
    ia::DecodeBwdArgs b{};
    b.fwd = decode_args(dec, pos, pos_stride, t, N);
    b.fwd.features = const_cast<uint32_t*>(static_cast<const uint32_t*>(features));
    if (N > 0) {
        b.g_scales = grad_attr->scales;
        b.g_quats = grad_attr->quats;
        b.g_colors = dec->mlp.color == IA_COLOR_SH3 ? grad_attr->sh : grad_attr->colors;
        b.g_opacity = grad_attr->opacity;
    }
    b.g_means = grad_means;
    b.g_pos = grad_pos;
    b.g_tables = grads->tables;
    for (int k = 0; k < dec->n_mats; ++k) {
        b.g_W[k] = grads->weights[k];
        b.g_b[k] = grads->biases[k];
    }
    if (dec->mlp.branches == IA_BRANCHES_PER_ATTRIBUTE)
        for (int k = 0; k < dec->n_mats; ++k) {
            b.Wbr[k] = static_cast<const _Float16*>(dec->W[k]);
            b.bbr[k] = dec->b[k];
        }
    b.ws = static_cast<unsigned char*>(ws);
    hipError_t e = ia::launch_decode_backward(b, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode backward launch");
    return IA_OK;
}

}  // extern "C"

// ============================================================== decode without allocation

namespace {

// Scratch of ia_decode_xyzt_noalloc: a file-scope device array, so the call
// allocates nothing.  Every GPU the library runs on holds its own copy until
// the process ends, and every call on that GPU shares it.
constexpr size_t kNoAllocScratchBytes = size_t(20) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kNoAllocMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kNoAllocMaxDevices] = {};

// The device address of the current device's copy of `scratch`, looked up on
// the first call on that device (with it current) and kept.  In host code the
// array's name is a host-side stand-in, never a device address: only this
// pointer reaches the kernels.
ia_status noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kNoAllocMaxDevices) return fail(IA_ERR_DEVICE, "device index out of range");
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (!g_noalloc_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(IA_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned null");
        g_noalloc_ptr[dev] = p;
    }
    *out = g_noalloc_ptr[dev];
    return IA_OK;
}

// Largest N whose decode scratch (one slot: 2 L F + 16 bytes per Gaussian,
// a multiple of 256 Gaussians) fits the array.
int64_t noalloc_max_n(const ia_decoder* dec) {
    const int64_t per = 2 * (int64_t)dec->hash.L * dec->hash.F + 16;
    return ((int64_t)kNoAllocScratchBytes / per) & ~(int64_t)255;
}

}  // namespace

extern "C" {

ia_status ia_decode_xyzt_noalloc(const ia_decoder* dec, const float* xyzt, int64_t N, const ia_gaussians* out,
                                 void* stream) {
    if (!dec) return fail(IA_ERR_INVALID_ARG, "decoder is null");
    if (!dec->ready) return fail(IA_ERR_INVALID_ARG, "decoder parameters not set");
    if (N < 0) return fail(IA_ERR_INVALID_ARG, "N must be >= 0");
    if (N == 0) return IA_OK;
    const bool f16 = dec->mlp.dtype == IA_DTYPE_F16;  // the fp32 decoder uses no scratch
    if (f16 && N > noalloc_max_n(dec))
        return fail(IA_ERR_INVALID_ARG, "N = " + std::to_string(N) + " exceeds the " +
                                            std::to_string(noalloc_max_n(dec)) +
                                            " Gaussians the 20 MiB static scratch holds for this decoder");
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (f16) {
        if (ia::decode_layout(dec->lv, N).total > kNoAllocScratchBytes)
            return fail(IA_ERR_INVALID_ARG, "decode scratch exceeds the static array");
        ia_status st = noalloc_scratch(&ws);
        if (st != IA_OK) return st;
        ws_bytes = kNoAllocScratchBytes;
    }
    return decode_common(dec, xyzt, 4, 0.0f, N, out, nullptr, 0, ws, ws_bytes, nullptr, stream);
}

void ia_decoder_destroy(ia_decoder* dec) {
    if (!dec) return;
    if (dec->tables) (void)hipDeviceSynchronize();
    free_decoder_params(dec);
    delete dec;
}

}  // extern "C"

// ============================================================== HexPlane

struct ia_hexplane {
    ia_hexplane_desc d;
    void* planes[6] = {};
    void* W[3] = {};
    float* b[3] = {};
    void* Wt = nullptr;  // weights in the deformation kernel's A-tile order
    bool ready = false;
};

namespace {

void free_hex(ia_hexplane* h) {
    for (int k = 0; k < 6; ++k) {
        if (h->planes[k]) (void)hipFree(h->planes[k]);
        h->planes[k] = nullptr;
    }
    for (int k = 0; k < 3; ++k) {
        if (h->W[k]) (void)hipFree(h->W[k]);
        if (h->b[k]) (void)hipFree(h->b[k]);
        h->W[k] = nullptr;
        h->b[k] = nullptr;
    }
    if (h->Wt) (void)hipFree(h->Wt);
    h->Wt = nullptr;
    h->ready = false;
}

}  // namespace

extern "C" {

ia_status ia_hexplane_create(const ia_hexplane_desc* desc, ia_hexplane** out) {
    if (!desc || !out) return fail(IA_ERR_INVALID_ARG, "null argument");
    if (desc->channels != 32) return fail(IA_ERR_UNSUPPORTED, "HexPlane supports 32 channels per plane");
    if (desc->res_xyz < 2 || desc->res_xyz > 4096 || desc->res_t < 2 || desc->res_t > 4096)
        return fail(IA_ERR_INVALID_ARG, "plane resolutions must be in 2..4096");
    if (!(std::isfinite(desc->aabb) && desc->aabb > 0.0f)) return fail(IA_ERR_INVALID_ARG, "aabb must be > 0");
    ia_hexplane* h = new (std::nothrow) ia_hexplane();
    if (!h) return fail(IA_ERR_OUT_OF_MEMORY, "host allocation failed");
    h->d = *desc;
    *out = h;
    return IA_OK;
}

ia_status ia_hexplane_set_params(ia_hexplane* hp, const void* const* planes, const void* const* weights,
                                 const float* const* biases, int32_t params_on_device, void* stream) {
    if (!hp || !planes || !weights || !biases) return fail(IA_ERR_INVALID_ARG, "null argument");
    for (int k = 0; k < 6; ++k)
        if (!planes[k]) return fail(IA_ERR_INVALID_ARG, "null plane pointer");
    for (int k = 0; k < 3; ++k)
        if (!weights[k] || !biases[k]) return fail(IA_ERR_INVALID_ARG, "null weight or bias pointer");
    if (hp->ready) {
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
        free_hex(hp);
    }
    const bool dev = params_on_device != 0;
    hipStream_t s = (hipStream_t)stream;
    const int C = hp->d.channels;
    ia_status st = IA_OK;
    for (int k = 0; st == IA_OK && k < 6; ++k) {
        const size_t rb = k < 3 ? hp->d.res_xyz : hp->d.res_t;
        st = upload_param(&hp->planes[k], planes[k], rb * hp->d.res_xyz * C * 2, dev, s);
    }
    const int dims[4] = {6 * C, 256, 256, 58};
    for (int k = 0; st == IA_OK && k < 3; ++k) {
        st = upload_param(&hp->W[k], weights[k], (size_t)dims[k + 1] * dims[k] * 2, dev, s);
        if (st == IA_OK) st = upload_param(reinterpret_cast<void**>(&hp->b[k]), biases[k], 4 * (size_t)dims[k + 1], dev, s);
    }
    if (st == IA_OK) {
        hipError_t e = hipMalloc(&hp->Wt, ia::kHexTiledWeightBytes);
        if (e != hipSuccess) {
            hp->Wt = nullptr;
            st = hip_fail(e, "hipMalloc");
        } else {
            const _Float16* W[3] = {(const _Float16*)hp->W[0], (const _Float16*)hp->W[1], (const _Float16*)hp->W[2]};
            e = ia::launch_hexplane_tiles(W, hp->Wt, s);
            if (e != hipSuccess) st = hip_fail(e, "hexplane weight tiling");
        }
    }
    if (st != IA_OK) {
        free_hex(hp);
        return st;
    }
    hp->ready = true;
    return IA_OK;
}

ia_status ia_hexplane_deform(const ia_hexplane* hp, const ia_gaussians* cn, int64_t N, float t, const ia_gaussians* out,
                             void* stream) {
    if (!hp) return fail(IA_ERR_INVALID_ARG, "hexplane is null");
    if (!hp->ready) return fail(IA_ERR_INVALID_ARG, "hexplane parameters not set");
    if (N < 0) return fail(IA_ERR_INVALID_ARG, "N must be >= 0");
    if (!std::isfinite(t)) return fail(IA_ERR_INVALID_ARG, "t must be finite");
    if (N == 0) return IA_OK;
    if (!cn || !out) return fail(IA_ERR_INVALID_ARG, "null Gaussian buffers");
    if (!cn->means || !cn->scales || !cn->quats || !cn->sh || !cn->opacity)
        return fail(IA_ERR_INVALID_ARG, "canonical means/scales/quats/sh/opacity must be non-null");
    if (!out->means || !out->scales || !out->quats || !out->sh || !out->opacity)
        return fail(IA_ERR_INVALID_ARG, "output means/scales/quats/sh/opacity must be non-null");
    if ((cn->means_stride != 0 && cn->means_stride != 3) || (out->means_stride != 0 && out->means_stride != 3))
        return fail(IA_ERR_INVALID_ARG, "HexPlane means must be packed [N,3]");
    ia::HexArgs a{};
    a.res_xyz = hp->d.res_xyz;
    a.res_t = hp->d.res_t;
    a.C = hp->d.channels;
    a.aabb = hp->d.aabb;
    for (int k = 0; k < 6; ++k) a.planes[k] = (const _Float16*)hp->planes[k];
    for (int k = 0; k < 3; ++k) {
        a.W[k] = (const _Float16*)hp->W[k];
        a.b[k] = hp->b[k];
    }
    a.means = cn->means;
    a.scales = cn->scales;
    a.quats = cn->quats;
    a.sh = cn->sh;
    a.opacity = cn->opacity;
    a.t = t;
    a.N = N;
    a.o_means = out->means;
    a.o_scales = out->scales;
    a.o_quats = out->quats;
    a.o_sh = out->sh;
    a.o_opacity = out->opacity;
    hipError_t e = ia::launch_hexplane(a, hp->Wt, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "hexplane launch");
    return IA_OK;
}

void ia_hexplane_destroy(ia_hexplane* hp) {
    if (!hp) return;
    if (hp->ready) (void)hipDeviceSynchronize();
    free_hex(hp);
    delete hp;
}

// ============================================================== render

ia_status ia_render_workspace_size(int64_t N_total, int32_t frames, int32_t W, int32_t H, int64_t max_entries,
                                   size_t* bytes) {
    if (!bytes) return fail(IA_ERR_INVALID_ARG, "bytes is null");
    if (N_total < 0 || N_total >= ((int64_t)1 << 32)) return fail(IA_ERR_INVALID_ARG, "N_total must be in [0, 2^32)");
    if (frames < 1 || frames > 65535) return fail(IA_ERR_INVALID_ARG, "frames must be in 1..65535");
    if (W < 1 || H < 1 || W > 16 * 4096 || H > 16 * 4096) return fail(IA_ERR_INVALID_ARG, "W, H must be in 1..65536");
    if (max_entries < 1 || max_entries >= ((int64_t)1 << 32) - 1)
        return fail(IA_ERR_INVALID_ARG, "max_entries must be in [1, 2^32 - 1)");
    const int64_t tiles = (int64_t)frames * ((W + 15) / 16) * ((H + 15) / 16);
    if (tiles >= ((int64_t)1 << 32)) return fail(IA_ERR_INVALID_ARG, "frames * tiles must be below 2^32");
    *bytes = ia::render_layout(N_total, frames, W, H, max_entries).total;
    return IA_OK;
}

}  // extern "C"

namespace {

// Validates the arguments ia_render and ia_render_backward share; on success
// *N, *W, *H hold the Gaussian count and the common image size.
ia_status check_render_args(const ia_gaussians* g, const int64_t* frame_offsets, int32_t frames, const ia_camera* cams,
                            void* ws, size_t ws_bytes, int64_t max_entries, int64_t* N_out, int* W_out, int* H_out) {
    if (!g || !frame_offsets || !cams) return fail(IA_ERR_INVALID_ARG, "null argument");
    if (frames < 1 || frames > 65535) return fail(IA_ERR_INVALID_ARG, "frames must be in 1..65535");
    if (frame_offsets[0] != 0) return fail(IA_ERR_INVALID_ARG, "frame_offsets[0] must be 0");
    for (int f = 0; f < frames; ++f)
        if (frame_offsets[f + 1] < frame_offsets[f]) return fail(IA_ERR_INVALID_ARG, "frame_offsets must be non-decreasing");
    const int64_t N = frame_offsets[frames];
    const int W = cams[0].W, H = cams[0].H;
    for (int f = 0; f < frames; ++f) {
        const ia_camera& c = cams[f];
        if (c.W != W || c.H != H) return fail(IA_ERR_INVALID_ARG, "all cameras must share W and H");
        bool fin = std::isfinite(c.fx) && std::isfinite(c.fy) && std::isfinite(c.cx) && std::isfinite(c.cy) &&
                   std::isfinite(c.near_z);
        for (int k = 0; k < 9; ++k) fin = fin && std::isfinite(c.R[k]);
        for (int k = 0; k < 3; ++k) fin = fin && std::isfinite(c.t[k]) && std::isfinite(c.bg[k]);
        if (!fin) return fail(IA_ERR_INVALID_ARG, "camera parameters must be finite");
    }
    size_t need = 0;
    ia_status st = ia_render_workspace_size(N, frames, W, H, max_entries, &need);
    if (st != IA_OK) return st;
    if (N > 0) {
        if (!g->means || !g->scales || !g->quats || !g->opacity)
            return fail(IA_ERR_INVALID_ARG, "means/scales/quats/opacity must be non-null");
        if (g->sh_degree == -1) {
            if (!g->colors) return fail(IA_ERR_INVALID_ARG, "colors must be non-null when sh_degree = -1");
        } else if (g->sh_degree == 3) {
            if (!g->sh) return fail(IA_ERR_INVALID_ARG, "sh must be non-null when sh_degree = 3");
        } else {
            return fail(IA_ERR_UNSUPPORTED, "sh_degree must be -1 or 3");
        }
        if (g->means_stride != 0 && g->means_stride < 3) return fail(IA_ERR_INVALID_ARG, "means_stride must be 0 or >= 3");
    }
    if (!ws || !aligned(ws, 256)) return fail(IA_ERR_INVALID_ARG, "workspace must be non-null and 256-byte aligned");
    if (ws_bytes < need)
        return fail(IA_ERR_WORKSPACE_TOO_SMALL, "workspace too small: need " + std::to_string(need) + " bytes");
    *N_out = N;
    *W_out = W;
    *H_out = H;
    return IA_OK;
}

}  // namespace

extern "C" {

ia_status ia_render(const ia_gaussians* g, const int64_t* frame_offsets, int32_t frames, const ia_camera* cams,
                    void* ws, size_t ws_bytes, int64_t max_entries, float* image, ia_render_aux* aux, void* stream) {
    if (!image) return fail(IA_ERR_INVALID_ARG, "null argument");
    int64_t N = 0;
    int W = 0, H = 0;
    ia_status st = check_render_args(g, frame_offsets, frames, cams, ws, ws_bytes, max_entries, &N, &W, &H);
    if (st != IA_OK) return st;
    const int binning = aux ? aux->binning : IA_BINNING_AUTO;
    if (binning != IA_BINNING_AUTO && binning != IA_BINNING_TILE_SORT && binning != IA_BINNING_REGIONS)
        return fail(IA_ERR_INVALID_ARG, "aux->binning must be IA_BINNING_AUTO, _TILE_SORT or _REGIONS");

    // camera table (centre = -R^T t, for SH view directions)
    std::string err;
    ia::DevCamera* dc = new (std::nothrow) ia::DevCamera[frames];
    if (!dc) return fail(IA_ERR_OUT_OF_MEMORY, "host allocation failed");
    for (int f = 0; f < frames; ++f) {
        const ia_camera& c = cams[f];
        ia::DevCamera& d = dc[f];
        std::memcpy(d.R, c.R, sizeof(d.R));
        std::memcpy(d.t, c.t, sizeof(d.t));
        d.fx = c.fx;
        d.fy = c.fy;
        d.cx = c.cx;
        d.cy = c.cy;
        d.near_z = c.near_z;
        for (int k = 0; k < 3; ++k) {
            double s = 0.0;
            for (int r = 0; r < 3; ++r) s += (double)c.R[r * 3 + k] * (double)c.t[r];
            d.centre[k] = (float)(-s);
            d.bg[k] = c.bg[k];
        }
        d.W = c.W;
        d.H = c.H;
    }
    ia::RenderArgs a{};
    a.means = g->means;
    a.means_stride = g->means_stride == 0 ? 3 : g->means_stride;
    a.scales = g->scales;
    a.quats = g->quats;
    a.colors = g->colors;
    a.sh = g->sh;
    a.opacity = g->opacity;
    a.sh_degree = g->sh_degree;
    a.frames = frames;
    a.W = W;
    a.H = H;
    a.frame_offsets_host = frame_offsets;
    a.cams_host = dc;
    a.ws = static_cast<unsigned char*>(ws);
    a.lay = ia::render_layout(N, frames, W, H, max_entries);
    a.image = image;
    a.T_final = aux ? aux->T_final : nullptr;
    a.n_contrib = aux ? aux->n_contrib : nullptr;
    a.n_entries_out = aux ? aux->n_entries : nullptr;
    a.overflow_out = aux ? aux->overflow : nullptr;
    a.unpack = aux != nullptr && aux->want_keys != 0;
    a.binning = binning;
    const uint64_t* keys = nullptr;
    const uint32_t* vals = nullptr;
    hipError_t e = ia::launch_render(a, (hipStream_t)stream, &keys, &vals);
    delete[] dc;
    if (e != hipSuccess) return hip_fail(e, "render launch");
    if (aux) {
        unsigned char* w = static_cast<unsigned char*>(ws);
        aux->sorted_keys = keys;
        aux->sorted_vals = vals;
        aux->tile_ranges = reinterpret_cast<const uint32_t*>(w + a.lay.ranges);
        aux->proj_a = reinterpret_cast<const float*>(w + a.lay.pa);
        aux->proj_b = reinterpret_cast<const float*>(w + a.lay.pb);
        aux->proj_c = reinterpret_cast<const float*>(w + a.lay.pc);
        aux->depth = reinterpret_cast<const float*>(w + a.lay.depth);
        aux->tiles_touched = reinterpret_cast<const uint32_t*>(w + a.lay.tiles);
        aux->tile_rect = reinterpret_cast<const uint16_t*>(w + a.lay.rect);
    }
    return IA_OK;
}


ia_status ia_render_backward(const ia_gaussians* g, const int64_t* frame_offsets, int32_t frames, const ia_camera* cams,
                             void* ws, size_t ws_bytes, int64_t max_entries, const float* grad_image,
                             const float* T_final, const uint32_t* n_contrib, const ia_gaussian_grads* grads,
                             void* stream) {
    if (!grads) return fail(IA_ERR_INVALID_ARG, "null argument");
    int64_t N = 0;
    int W = 0, H = 0;
    ia_status st = check_render_args(g, frame_offsets, frames, cams, ws, ws_bytes, max_entries, &N, &W, &H);
    if (st != IA_OK) return st;
    if (N > 0 && g->sh_degree == 3 && !grads->sh)
        return fail(IA_ERR_INVALID_ARG, "grads->sh must be non-null when sh_degree = 3");
    if (!grad_image || !T_final || !n_contrib) return fail(IA_ERR_INVALID_ARG, "grad_image, T_final, n_contrib must be non-null");
    if (N > 0 && (!grads->means || !grads->scales || !grads->quats || !grads->opacity || !grads->colors))
        return fail(IA_ERR_INVALID_ARG, "every gradient buffer must be non-null");
    ia::RenderBwdArgs a{};
    a.ws = static_cast<unsigned char*>(ws);
    a.lay = ia::render_layout(N, frames, W, H, max_entries);
    a.W = W;
    a.H = H;
    a.means = g->means;
    a.means_stride = g->means_stride == 0 ? 3 : g->means_stride;
    a.scales = g->scales;
    a.quats = g->quats;
    a.grad_image = grad_image;
    a.T_final = T_final;
    a.n_contrib = n_contrib;
    a.g_means = grads->means;
    a.g_scales = grads->scales;
    a.g_quats = grads->quats;
    a.g_opacity = grads->opacity;
    a.g_colors = grads->colors;
    a.sh = g->sh_degree == 3 ? g->sh : nullptr;
    a.g_sh = g->sh_degree == 3 ? grads->sh : nullptr;
    hipError_t e = ia::launch_render_backward(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "render backward launch");
    return IA_OK;
}

ia_status ia_l1_loss(const float* image, const float* target, int64_t n, double* loss, float* grad_image,
                     void* stream) {
    if (n < 0) return fail(IA_ERR_INVALID_ARG, "n must be >= 0");
    if (!loss) return fail(IA_ERR_INVALID_ARG, "loss is null");
    if (n > 0 && (!image || !target || !grad_image)) return fail(IA_ERR_INVALID_ARG, "null argument");
    hipError_t e = ia::launch_l1_loss(image, target, n, loss, grad_image, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "l1 loss launch");
    return IA_OK;
}

ia_status ia_image_loss_workspace_size(int32_t frames, int32_t H, int32_t W, size_t* bytes) {
    if (!bytes) return fail(IA_ERR_INVALID_ARG, "bytes is null");
    if (frames <= 0 || H <= 0 || W <= 0) return fail(IA_ERR_INVALID_ARG, "frames, H and W must be > 0");
    *bytes = ia::image_loss_workspace(frames, H, W);
    return IA_OK;
}

ia_status ia_image_loss(const float* image, const float* target, int32_t frames, int32_t H, int32_t W, float lambda,
                        void* ws, size_t ws_bytes, double* loss, float* grad_image, void* stream) {
    if (frames <= 0 || H <= 0 || W <= 0) return fail(IA_ERR_INVALID_ARG, "frames, H and W must be > 0");
    if (!image || !target || !ws || !loss || !grad_image) return fail(IA_ERR_INVALID_ARG, "null argument");
    if (!(lambda >= 0.0f && lambda <= 1.0f)) return fail(IA_ERR_INVALID_ARG, "lambda must be in [0, 1]");
    if ((int64_t)frames * 3 > 65535) return fail(IA_ERR_INVALID_ARG, "at most 21845 frames per call");
    if (ws_bytes < ia::image_loss_workspace(frames, H, W))
        return fail(IA_ERR_WORKSPACE_TOO_SMALL, "image loss workspace too small");
    if (((uintptr_t)ws & 255) != 0) return fail(IA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    hipError_t e = ia::launch_image_loss(image, target, frames, H, W, lambda, ws, loss, grad_image,
                                         (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "image loss launch");
    return IA_OK;
}

ia_status ia_adam_step(float* param, const float* grad, float* m, float* v, int64_t n, float lr, float beta1,
                       float beta2, float eps, int32_t step, uint16_t* param_f16, void* stream) {
    if (n < 0) return fail(IA_ERR_INVALID_ARG, "n must be >= 0");
    if (n > 0 && (!param || !grad || !m || !v)) return fail(IA_ERR_INVALID_ARG, "null argument");
    if (step < 1) return fail(IA_ERR_INVALID_ARG, "step must be >= 1");
    if (!(beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f))
        return fail(IA_ERR_INVALID_ARG, "betas must be in [0, 1)");
    if (!(eps >= 0.0f) || !(lr >= 0.0f)) return fail(IA_ERR_INVALID_ARG, "lr and eps must be >= 0");
    hipError_t e =
        ia::launch_adam(param, grad, m, v, n, 1, 1, lr, beta1, beta2, eps, step, param_f16, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "adam launch");
    return IA_OK;
}

ia_status ia_lr_at(float base_lr, int32_t step, int32_t warmup, int32_t total, float final_lr, float* lr) {
    if (!lr) return fail(IA_ERR_INVALID_ARG, "lr is null");
    if (step < 0 || warmup < 0 || total < warmup)
        return fail(IA_ERR_INVALID_ARG, "need step >= 0, warmup >= 0 and total >= warmup");
    if (!(std::isfinite(base_lr) && base_lr >= 0.0f && std::isfinite(final_lr) && final_lr >= 0.0f))
        return fail(IA_ERR_INVALID_ARG, "rates must be finite and >= 0");
    const double base = base_lr, fin = final_lr;
    if (warmup > 0 && step < warmup) {
        *lr = (float)(base * (double)(step + 1) / (double)warmup);
        return IA_OK;
    }
    const int64_t span = total - warmup > 1 ? (int64_t)total - warmup : 1;
    int64_t k = (int64_t)step - warmup;
    if (k > span) k = span;
    const double frac = (double)k / (double)span;
    *lr = (float)(fin + 0.5 * (base - fin) * (1.0 + std::cos(M_PI * frac)));
    return IA_OK;
}

ia_status ia_adam_step_strided(float* param, int32_t param_stride, int32_t dim, const float* grad, float* m, float* v,
                               int64_t rows, float lr, float beta1, float beta2, float eps, int32_t step,
                               void* stream) {
    if (rows < 0 || dim < 1 || param_stride < dim)
        return fail(IA_ERR_INVALID_ARG, "need rows >= 0 and 1 <= dim <= param_stride");
    if (rows > 0 && (!param || !grad || !m || !v)) return fail(IA_ERR_INVALID_ARG, "null argument");
    if (step < 1) return fail(IA_ERR_INVALID_ARG, "step must be >= 1");
    if (!(beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f))
        return fail(IA_ERR_INVALID_ARG, "betas must be in [0, 1)");
    if (!(eps >= 0.0f) || !(lr >= 0.0f)) return fail(IA_ERR_INVALID_ARG, "lr and eps must be >= 0");
    hipError_t e = ia::launch_adam(param, grad, m, v, rows * dim, dim, param_stride, lr, beta1, beta2, eps, step,
                                   nullptr, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "adam launch");
    return IA_OK;
}

ia_status ia_spatial_order_workspace_size(int64_t N, int32_t frames, size_t* bytes) {
    if (!bytes) return fail(IA_ERR_INVALID_ARG, "bytes is null");
    if (N < 0 || N >= ((int64_t)1 << 32)) return fail(IA_ERR_INVALID_ARG, "N must be in [0, 2^32)");
    if (frames < 1 || frames > 65535) return fail(IA_ERR_INVALID_ARG, "frames must be in 1..65535");
    *bytes = ia::spatial_order_workspace(N, frames);
    return IA_OK;
}

ia_status ia_spatial_order(const float* pos, int32_t pos_stride, int64_t N, const int64_t* frame_offsets,
                           int32_t frames, uint32_t* perm, float* pos_out, void* ws, size_t ws_bytes, void* stream) {
    size_t need = 0;
    ia_status st = ia_spatial_order_workspace_size(N, frames, &need);
    if (st != IA_OK) return st;
    if (pos_stride < 3 || pos_stride > 64) return fail(IA_ERR_INVALID_ARG, "pos_stride must be in 3..64");
    if (!frame_offsets) return fail(IA_ERR_INVALID_ARG, "frame_offsets is null");
    if (frame_offsets[0] != 0) return fail(IA_ERR_INVALID_ARG, "frame_offsets[0] must be 0");
    for (int f = 0; f < frames; ++f)
        if (frame_offsets[f + 1] < frame_offsets[f]) return fail(IA_ERR_INVALID_ARG, "frame_offsets must be non-decreasing");
    if (frame_offsets[frames] != N) return fail(IA_ERR_INVALID_ARG, "frame_offsets[frames] must equal N");
    if (N == 0) return IA_OK;
    if (!pos || !perm || !aligned(pos, 4) || !aligned(perm, 4)) return fail(IA_ERR_INVALID_ARG, "null or misaligned pos / perm");
    if (pos_out) {
        const char* a = reinterpret_cast<const char*>(pos);
        const char* b = reinterpret_cast<const char*>(pos_out);
        const size_t bytes = (size_t)N * pos_stride * sizeof(float);
        if (!aligned(pos_out, 4)) return fail(IA_ERR_INVALID_ARG, "pos_out misaligned");
        if (a < b + bytes && b < a + bytes) return fail(IA_ERR_INVALID_ARG, "pos_out must not overlap pos");
    }
    st = check_ws(ws, ws_bytes, need);
    if (st != IA_OK) return st;
    hipError_t e = ia::launch_spatial_order(pos, pos_stride, N, frame_offsets, frames, perm, pos_out, ws,
                                            (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "spatial order launch");
    return IA_OK;
}

ia_status ia_densify_accumulate(const float* grad_pos, int64_t N, float* grad_acc, int32_t* grad_count,
                                void* stream) {
    if (N < 0) return fail(IA_ERR_INVALID_ARG, "N must be >= 0");
    if (N > 0 && (!grad_pos || !grad_acc || !grad_count)) return fail(IA_ERR_INVALID_ARG, "null argument");
    hipError_t e = ia::launch_densify_accumulate(grad_pos, N, grad_acc, grad_count, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "densify accumulate launch");
    return IA_OK;
}

ia_status ia_densify_workspace_size(int64_t N, size_t* bytes) {
    if (N < 0 || !bytes) return fail(IA_ERR_INVALID_ARG, "N must be >= 0 and bytes non-null");
    *bytes = ia::densify_workspace(N);
    return IA_OK;
}

ia_status ia_densify(const float* xyzt, const float* grad_acc, const int32_t* grad_count, const float* scales,
                     const float* quats, const float* opacity, const float* noise, const float* m, const float* v,
                     int64_t N, const ia_densify_params* params, float* out_xyzt, float* out_m, float* out_v,
                     int64_t out_capacity, int64_t* out_n, void* ws, size_t ws_bytes, void* stream) {
    if (N < 0 || !params || !out_n) return fail(IA_ERR_INVALID_ARG, "N must be >= 0; params, out_n non-null");
    if (N > 0 && (!xyzt || !grad_acc || !grad_count || !scales || !quats || !opacity || !noise || !m || !v ||
                  !out_xyzt || !out_m || !out_v))
        return fail(IA_ERR_INVALID_ARG, "null argument");
    if (N > ((int64_t)1 << 40)) return fail(IA_ERR_INVALID_ARG, "N too large");
    if (out_capacity < 2 * N) return fail(IA_ERR_INVALID_ARG, "out_capacity must be >= 2 N");
    if (N > 0 && (!aligned(xyzt, 16) || !aligned(out_xyzt, 16)))
        return fail(IA_ERR_INVALID_ARG, "xyzt and out_xyzt must be 16-byte aligned");
    if (N > 0 && (!ws || ws_bytes < ia::densify_workspace(N)))
        return fail(IA_ERR_WORKSPACE_TOO_SMALL, "densify workspace too small");
    if (!(params->grad_threshold >= 0.0f) || !(params->scale_threshold >= 0.0f) || !(params->min_opacity >= 0.0f))
        return fail(IA_ERR_INVALID_ARG, "thresholds must be >= 0");
    ia::DensifyIn in{xyzt, grad_acc, grad_count, scales, quats, opacity, noise, m, v, N, params->grad_threshold,
                     params->scale_threshold, params->min_opacity, out_xyzt, out_m, out_v, out_n};
    hipError_t e = ia::launch_densify(in, ws, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "densify launch");
    return IA_OK;
}

}  // extern "C"
