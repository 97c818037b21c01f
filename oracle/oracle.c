/*
 * CPU oracle for SPIN-4DGS-style decode + render.  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow definition that the HIP path is checked
 * against.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load it.  It shares no source, header, table or constant with the HIP
 * library; both sides are written independently from the pages:
 *
 *   [SPIN] "Implicit 4D Gaussian Splatting for Fast Motion with Large
 *          Inter-Frame Displacements" (SPIN-4DGS), §3.1 Eq. 1-4, §3.3 Eq. 7-11.
 *   [HEX]  "4D Gaussian Splatting详解：动态场景实时渲染的范式突破",
 *          §2.2, §3.1 (HexPlane six planes), §3.2 (deformation MLP), §6.1.
 *
 * Precision.  Interpolation, MLPs, activations and compositing run in fp64.
 * Two steps whose floating-point result decides an integer run in fp32 with a
 * fixed operation order (one IEEE op per step, left to right, no FMA,
 * correctly rounded '/' and sqrt), exactly as the kernels do:
 *   - position normalisation (decides the hash-grid cell), and
 *   - projection (decides the tile rectangle and the depth bits of the sort
 *     key).
 * Build with -ffp-contract=off and without fast-math.
 *
 * Parity status: every exported function is pinned by tests/test_oracle_*.py
 * (closed forms, library routines, brute force, invariants).  Agreement with
 * trained SPIN-4DGS images is "parity unpinned" (no data or weights exist).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the parallel loops of this file use (1 without OpenMP). */
EXPORT int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads later parallel loops use (n >= 1; no-op without OpenMP). */
EXPORT void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* IEEE binary16 <-> double, from the format definition                      */
/* ------------------------------------------------------------------------ */

EXPORT double orc_half_to_double(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* Round to nearest, ties to even. */
EXPORT uint16_t orc_double_to_half(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return 0x7e00;
    if (a >= 65520.0) return sign | 0x7c00; /* halfway above 65504 -> inf */
    if (a < ldexp(1.0, -14)) {              /* subnormal range, quantum 2^-24 */
        double m = nearbyint(a * 16777216.0);
        return (uint16_t)(sign | (uint16_t)m); /* m == 1024 encodes 2^-14 */
    }
    int e;
    frexp(a, &e);                    /* a in [2^(e-1), 2^e) */
    double m = nearbyint(ldexp(a, 11 - e)); /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; e += 1; }
    int E = e - 1 + 15;
    if (E >= 31) return sign | 0x7c00;
    return (uint16_t)(sign | (E << 10) | ((int)m - 1024));
}

static double round_f16(double x) { return orc_half_to_double(orc_double_to_half(x)); }

/* ------------------------------------------------------------------------ */
/* Hash encoder description ([SPIN] §3.3 Eq. 9; Instant-NGP extended by t)   */
/* ------------------------------------------------------------------------ */

typedef struct {
    int L, F, log2T;
    double base_res, growth;
    int temporal_res; /* 0: same as the level's spatial resolution */
    int table_f16;
    float t_min, t_max;
} orc_hash;

/* Level resolution res_l = floor(base * growth^l) (vertices per axis). */
EXPORT void orc_level_res(const orc_hash* h, int* res_s, int* res_t, int* dense) {
    double T = ldexp(1.0, h->log2T);
    for (int l = 0; l < h->L; ++l) {
        int r = (int)floor(h->base_res * pow(h->growth, (double)l));
        int rt = h->temporal_res > 0 ? h->temporal_res : r;
        res_s[l] = r;
        res_t[l] = rt;
        dense[l] = ((double)r * (double)r * (double)r * (double)rt) <= T;
    }
}

/*
 * Normalisation, [SPIN] §3.3 Eq. 7 (scene contraction, L2 norm) and Eq. 8
 * (time).  fp32, fixed order:
 *   n2 = (x*x + y*y) + z*z;  n = sqrt(n2)
 *   n <= 1: c = mu;  else k = (2 - 1/n) / n, c = mu * k
 *   mu_bar = 0.25*c + 0.5
 *   t_norm = clamp((t - t_min) / (t_max - t_min), 0, 1)
 * pos has `stride` floats per point (3: xyz with the scalar t, 4: xyzt).
 */
EXPORT void orc_normalize(const orc_hash* h, const float* pos, int stride, float t_scalar, long N,
                          float* xt) {
    for (long i = 0; i < N; ++i) {
        const float* p = pos + i * stride;
        float x = p[0], y = p[1], z = p[2];
        float n2 = x * x + y * y;
        n2 = n2 + z * z;
        float n = sqrtf(n2);
        float c0 = x, c1 = y, c2 = z;
        if (!(n <= 1.0f)) {
            float k = 2.0f - 1.0f / n;
            k = k / n;
            c0 = x * k;
            c1 = y * k;
            c2 = z * k;
        }
        float t = stride == 4 ? p[3] : t_scalar;
        float tn = (t - h->t_min) / (h->t_max - h->t_min);
        tn = tn < 0.0f ? 0.0f : (tn > 1.0f ? 1.0f : tn);
        float a0 = 0.25f * c0, a1 = 0.25f * c1, a2 = 0.25f * c2;
        xt[i * 4 + 0] = a0 + 0.5f;
        xt[i * 4 + 1] = a1 + 0.5f;
        xt[i * 4 + 2] = a2 + 0.5f;
        xt[i * 4 + 3] = tn;
    }
}

/* Spatial hash of a 4D vertex: XOR of coordinate * prime, mod T.  The first
 * three primes are Instant-NGP's; the fourth (time) is a fixed odd constant. */
static uint32_t hash4(uint32_t ix, uint32_t iy, uint32_t iz, uint32_t it, uint32_t mask) {
    uint32_t hsh = ix * 1u;
    hsh ^= iy * 2654435761u;
    hsh ^= iz * 805459861u;
    hsh ^= it * 3674653429u;
    return hsh & mask;
}

static double table_at(const orc_hash* h, const void* tables, long level, long idx, int k) {
    long T = 1L << h->log2T;
    long off = (level * T + idx) * h->F + k;
    if (h->table_f16) return orc_half_to_double(((const uint16_t*)tables)[off]);
    return (double)((const float*)tables)[off];
}

/*
 * 4D multiresolution hash encoding, [SPIN] §3.3 Eq. 9, with quadrilinear
 * interpolation over the 16 corners of the cell.  Per axis (fp32, the cell
 * decision): p = xt*(res-1), i = clamp(floor(p), 0, res-2), f = p - i.  The
 * corner weights and the weighted sum are fp64.  Corner c: bit k adds one on
 * axis k (x, y, z, t); weight = prod_k (bit ? f_k : 1 - f_k).  Level l is
 * dense (row-major x fastest) iff res^3 * res_t <= T, otherwise hashed.
 * z[l*F + k] = sum_c w_c * table[l][idx_c][k].
 */
EXPORT void orc_encode(const orc_hash* h, const void* tables, const float* xt, long N, double* z) {
    int res_s[64], res_t[64], dense[64];
    orc_level_res(h, res_s, res_t, dense);
    uint32_t mask = (uint32_t)((1UL << h->log2T) - 1);
#pragma omp parallel for schedule(static)
    for (long i = 0; i < N; ++i) {
        for (int l = 0; l < h->L; ++l) {
            int res[4] = {res_s[l], res_s[l], res_s[l], res_t[l]};
            int ci[4];
            double f[4];
            for (int a = 0; a < 4; ++a) {
                float p = xt[i * 4 + a] * (float)(res[a] - 1);
                float fl = floorf(p);
                int c = (int)fl;
                if (c < 0) c = 0;
                if (c > res[a] - 2) c = res[a] - 2;
                ci[a] = c;
                f[a] = (double)p - (double)c;
            }
            double acc[8] = {0};
            for (int corner = 0; corner < 16; ++corner) {
                double w = 1.0;
                uint32_t v[4];
                for (int a = 0; a < 4; ++a) {
                    int bit = (corner >> a) & 1;
                    v[a] = (uint32_t)(ci[a] + bit);
                    w *= bit ? f[a] : 1.0 - f[a];
                }
                long idx;
                if (dense[l])
                    idx = (long)v[0] + (long)res[0] * ((long)v[1] + (long)res[1] * ((long)v[2] + (long)res[2] * (long)v[3]));
                else
                    idx = (long)hash4(v[0], v[1], v[2], v[3], mask);
                for (int k = 0; k < h->F; ++k) acc[k] += w * table_at(h, tables, l, idx, k);
            }
            for (int k = 0; k < h->F; ++k) z[i * (long)(h->L * h->F) + l * h->F + k] = acc[k];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* MLP, [SPIN] §3.3 Eq. 10-11                                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
    int n_layers;  /* number of linear layers (the last one is the head block) */
    int dims[8];   /* dims[0] = input width, dims[l+1] = output width of layer l */
    int act;       /* hidden activation: 0 = ReLU, 1 = GELU (exact erf) */
    int w_f16;     /* weights stored as binary16 (else fp32) */
    int branches;  /* orc_decode_grad only: 1 = one MLP per attribute on the
                      same z ([SPIN] §3.3 Eq. 10, the per-head reading), dims
                      [in, hidden..., head] with each branch's last width
                      3, 4, head - 8, 1; weights and biases branch-major */
} orc_mlp;

static double act_fn(int act, double x) {
    if (act == 0) return x > 0.0 ? x : 0.0;
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

/*
 * y = act(W x + b) for every layer but the last, which stays linear.
 * W is row-major [out][in].  mode 0: fp64 throughout.  mode 1 ("fp16
 * emulation"): the input and every hidden activation are rounded to binary16
 * (RNE) before they enter the next layer, as an fp16-in/fp32-accumulate
 * device path does; sums stay fp64.
 */
EXPORT void orc_mlp_forward(const orc_mlp* m, const void* const* W, const float* const* b,
                            const double* in, long N, int mode, double* out) {
    int in_dim = m->dims[0], out_dim = m->dims[m->n_layers];
#pragma omp parallel for schedule(static)
    for (long i = 0; i < N; ++i) {
        double bufa[512], bufb[512];
        double* x = bufa;
        double* y = bufb;
        for (int k = 0; k < in_dim; ++k) x[k] = mode ? round_f16(in[i * in_dim + k]) : in[i * in_dim + k];
        for (int l = 0; l < m->n_layers; ++l) {
            int di = m->dims[l], dout = m->dims[l + 1];
            for (int o = 0; o < dout; ++o) {
                double s = 0.0;
                for (int k = 0; k < di; ++k) {
                    double w = m->w_f16 ? orc_half_to_double(((const uint16_t*)W[l])[(long)o * di + k])
                                        : (double)((const float*)W[l])[(long)o * di + k];
                    s += w * x[k];
                }
                s += (double)b[l][o];
                if (l + 1 < m->n_layers) {
                    s = act_fn(m->act, s);
                    if (mode) s = round_f16(s);
                }
                y[o] = s;
            }
            double* tmp = x; x = y; y = tmp;
        }
        for (int o = 0; o < out_dim; ++o) out[i * out_dim + o] = x[o];
    }
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/*
 * Eq. 11 activations on the 11 head outputs [s(3) | r(4) w,x,y,z | c(3) | o]:
 *   s = exp(min(s_hat, 20))   (the pre-activation clip at 20, §3.3 scale head)
 *   r = r_hat / max(||r_hat||, 1e-12)
 *   c = sigmoid(c_hat),  o = sigmoid(o_hat)
 */
EXPORT void orc_activate(const double* raw, long N, double* scales, double* quats, double* colors,
                         double* opacity) {
    for (long i = 0; i < N; ++i) {
        const double* r = raw + i * 11;
        for (int k = 0; k < 3; ++k) scales[i * 3 + k] = exp(r[k] < 20.0 ? r[k] : 20.0);
        double n = sqrt(r[3] * r[3] + r[4] * r[4] + r[5] * r[5] + r[6] * r[6]);
        if (n < 1e-12) n = 1e-12;
        for (int k = 0; k < 4; ++k) quats[i * 4 + k] = r[3 + k] / n;
        for (int k = 0; k < 3; ++k) colors[i * 3 + k] = sigmoid(r[7 + k]);
        opacity[i] = sigmoid(r[10]);
    }
}

/*
 * Eq. 11 with the SH colour decoder ([SPIN] §3.3: the colour head regresses
 * the SH coefficients directly) on the 56 head outputs
 * [s(3) | r(4) | sh(48, coefficient-major [16][3]) | o]:
 *   s = exp(min(s_hat, 20)), r = r_hat / max(||r_hat||, 1e-12),
 *   sh = sh_hat (no activation), o = sigmoid(o_hat).
 */
EXPORT void orc_activate_sh(const double* raw, long N, double* scales, double* quats, double* sh,
                            double* opacity) {
    for (long i = 0; i < N; ++i) {
        const double* r = raw + i * 56;
        for (int k = 0; k < 3; ++k) scales[i * 3 + k] = exp(r[k] < 20.0 ? r[k] : 20.0);
        double n = sqrt(r[3] * r[3] + r[4] * r[4] + r[5] * r[5] + r[6] * r[6]);
        if (n < 1e-12) n = 1e-12;
        for (int k = 0; k < 4; ++k) quats[i * 4 + k] = r[3 + k] / n;
        for (int k = 0; k < 48; ++k) sh[i * 48 + k] = r[7 + k];
        opacity[i] = sigmoid(r[55]);
    }
}

/* Full decode: normalise -> encode -> MLP -> activations.  raw is [N][11]. */
EXPORT void orc_decode(const orc_hash* h, const void* tables, const orc_mlp* m, const void* const* W,
                       const float* const* b, const float* pos, int stride, float t_scalar, long N,
                       int mode, double* raw, double* scales, double* quats, double* colors,
                       double* opacity) {
    long LF = (long)h->L * h->F;
    float* xt = (float*)malloc(sizeof(float) * 4 * (size_t)(N > 0 ? N : 1));
    double* z = (double*)malloc(sizeof(double) * (size_t)LF * (size_t)(N > 0 ? N : 1));
    orc_normalize(h, pos, stride, t_scalar, N, xt);
    orc_encode(h, tables, xt, N, z);
    orc_mlp_forward(m, W, b, z, N, mode, raw);
    orc_activate(raw, N, scales, quats, colors, opacity);
    free(xt);
    free(z);
}

/* ------------------------------------------------------------------------ */
/* Real spherical harmonics, degree 3 (16 functions, l-major, m = -l..l)      */
/* ------------------------------------------------------------------------ */

/* Orthonormal real basis built from the complex harmonics with the
 * Condon-Shortley phase: Y_l0, and sqrt(2) Re / Im of Y_l^|m| for m > 0 / m < 0.
 * Written as polynomials in the unit direction (x, y, z). */
EXPORT void orc_sh_basis(const double* dirs, long N, double* Y) {
    const double pi = 3.14159265358979323846;
    const double k00 = 0.5 * sqrt(1.0 / pi);
    const double k1 = sqrt(3.0 / (4.0 * pi));
    const double k2a = 0.5 * sqrt(15.0 / pi), k2b = 0.25 * sqrt(5.0 / pi), k2c = 0.25 * sqrt(15.0 / pi);
    const double k3a = 0.25 * sqrt(35.0 / (2.0 * pi)), k3b = 0.5 * sqrt(105.0 / pi);
    const double k3c = 0.25 * sqrt(21.0 / (2.0 * pi)), k3d = 0.25 * sqrt(7.0 / pi);
    const double k3e = 0.25 * sqrt(105.0 / pi);
    for (long i = 0; i < N; ++i) {
        double x = dirs[i * 3], y = dirs[i * 3 + 1], z = dirs[i * 3 + 2];
        double* o = Y + i * 16;
        double xx = x * x, yy = y * y, zz = z * z;
        o[0] = k00;
        o[1] = -k1 * y;
        o[2] = k1 * z;
        o[3] = -k1 * x;
        o[4] = k2a * x * y;
        o[5] = -k2a * y * z;
        o[6] = k2b * (2.0 * zz - xx - yy);
        o[7] = -k2a * x * z;
        o[8] = k2c * (xx - yy);
        o[9] = -k3a * y * (3.0 * xx - yy);
        o[10] = k3b * x * y * z;
        o[11] = -k3c * y * (4.0 * zz - xx - yy);
        o[12] = k3d * z * (2.0 * zz - 3.0 * xx - 3.0 * yy);
        o[13] = -k3c * x * (4.0 * zz - xx - yy);
        o[14] = k3e * z * (xx - yy);
        o[15] = -k3a * x * (xx - 3.0 * yy);
    }
}

/* ------------------------------------------------------------------------ */
/* HexPlane deformation, [HEX] §3.1-§3.2, §6.1                                */
/* ------------------------------------------------------------------------ */

typedef struct {
    int res_xyz, res_t, C;
    float aabb; /* positions map to [0,1] through [-aabb, aabb]^3, clamped */
} orc_hexplane;

/*
 * Features: six planes XY, XZ, YZ (res_xyz^2) and XT, YT, ZT (res_xyz x res_t,
 * time on the second axis), each [res_b][res_a][C] binary16; bilinear per
 * plane with vertices at 0..res-1; concatenated in that order (6*C values).
 * Cell decision in fp32: u = clamp((x + aabb) / (2 aabb), 0, 1),
 * p = u*(res-1), i = clamp(floor(p), 0, res-2), f = p - i.  t is used as is
 * (already in [0,1]).
 */
EXPORT void orc_hexplane_features(const orc_hexplane* hp, const uint16_t* const* planes,
                                  const float* means, float t, long N, double* feat) {
    static const int pa[6] = {0, 0, 1, 0, 1, 2}; /* first axis of each plane */
    static const int pb[6] = {1, 2, 2, 3, 3, 3}; /* second axis (3 = time) */
    float tt = t < 0.0f ? 0.0f : (t > 1.0f ? 1.0f : t);
#pragma omp parallel for schedule(static)
    for (long i = 0; i < N; ++i) {
        float u[4];
        for (int a = 0; a < 3; ++a) {
            float v = means[i * 3 + a] + hp->aabb;
            v = v / (2.0f * hp->aabb);
            u[a] = v < 0.0f ? 0.0f : (v > 1.0f ? 1.0f : v);
        }
        u[3] = tt;
        for (int p = 0; p < 6; ++p) {
            int ra = hp->res_xyz, rb = pb[p] == 3 ? hp->res_t : hp->res_xyz;
            float qa = u[pa[p]] * (float)(ra - 1), qb = u[pb[p]] * (float)(rb - 1);
            int ia = (int)floorf(qa), ib = (int)floorf(qb);
            if (ia < 0) ia = 0;
            if (ia > ra - 2) ia = ra - 2;
            if (ib < 0) ib = 0;
            if (ib > rb - 2) ib = rb - 2;
            double fa = (double)qa - ia, fb = (double)qb - ib;
            const uint16_t* P = planes[p];
            for (int c = 0; c < hp->C; ++c) {
                double v00 = orc_half_to_double(P[((long)ib * ra + ia) * hp->C + c]);
                double v01 = orc_half_to_double(P[((long)ib * ra + ia + 1) * hp->C + c]);
                double v10 = orc_half_to_double(P[((long)(ib + 1) * ra + ia) * hp->C + c]);
                double v11 = orc_half_to_double(P[((long)(ib + 1) * ra + ia + 1) * hp->C + c]);
                feat[i * 6L * hp->C + p * hp->C + c] = (1 - fa) * (1 - fb) * v00 + fa * (1 - fb) * v01 +
                                                       (1 - fa) * fb * v10 + fa * fb * v11;
            }
        }
    }
}

/*
 * Deform canonical Gaussians at time t: features -> MLP (ReLU hidden) -> 58
 * outputs [dpos(3) | dquat(4) | dlog_scale(3) | dsh(48)], then
 *   mu' = mu + dpos;  q' = (q + dq) / ||q + dq||;  s' = s * exp(dlog_scale)
 *   sh' = sh + dsh;   opacity unchanged ([HEX] §6.1).
 */
EXPORT void orc_hexplane_deform(const orc_hexplane* hp, const uint16_t* const* planes, const orc_mlp* m,
                                const void* const* W, const float* const* b, const float* means,
                                const float* scales, const float* quats, const float* sh, float t, long N,
                                int mode, double* o_means, double* o_scales, double* o_quats, double* o_sh) {
    long D = 6L * hp->C;
    double* feat = (double*)malloc(sizeof(double) * (size_t)D * (size_t)(N > 0 ? N : 1));
    double* raw = (double*)malloc(sizeof(double) * 58 * (size_t)(N > 0 ? N : 1));
    orc_hexplane_features(hp, planes, means, t, N, feat);
    orc_mlp_forward(m, W, b, feat, N, mode, raw);
    for (long i = 0; i < N; ++i) {
        const double* r = raw + i * 58;
        for (int k = 0; k < 3; ++k) o_means[i * 3 + k] = (double)means[i * 3 + k] + r[k];
        double q[4], n = 0.0;
        for (int k = 0; k < 4; ++k) { q[k] = (double)quats[i * 4 + k] + r[3 + k]; n += q[k] * q[k]; }
        n = sqrt(n);
        if (n < 1e-12) n = 1e-12;
        for (int k = 0; k < 4; ++k) o_quats[i * 4 + k] = q[k] / n;
        for (int k = 0; k < 3; ++k) o_scales[i * 3 + k] = (double)scales[i * 3 + k] * exp(r[7 + k]);
        for (int k = 0; k < 48; ++k) o_sh[i * 48 + k] = (double)sh[i * 48 + k] + r[10 + k];
    }
    free(feat);
    free(raw);
}

/* ------------------------------------------------------------------------ */
/* Projection, [SPIN] §3.1 Eq. 2-3 (EWA splatting)                            */
/* ------------------------------------------------------------------------ */

typedef struct {
    float R[9]; /* world -> camera rotation, row-major */
    float t[3];
    float fx, fy, cx, cy, near_z;
    int W, H;
    float bg[3];
} orc_camera;

/*
 * One Gaussian, fp32, one IEEE op per step in the order written:
 *   p = ((R_k0*mu0 + R_k1*mu1) + R_k2*mu2) + t_k;  cull unless p_z > near
 *   q /= sqrt(((w*w + x*x) + y*y) + z*z);  R_q from q (w,x,y,z)
 *   M = R_q diag(s);  Sigma_ij = (M_i0 M_j0 + M_i1 M_j1) + M_i2 M_j2          (Eq. 2)
 *   J = [[fx/z, 0, -(fx x)/(z z)], [0, fy/z, -(fy y)/(z z)]];  T = J R
 *   Sigma2D = T Sigma T^T  (U = T Sigma, then U T^T)                            (Eq. 3)
 *   det = a c - b b (cull det <= 0);  conic = (c, -b, a) / det
 *   lambda1 = mid + sqrt(max(0, mid*mid - det)), mid = 0.5 (a + c);  r = ceil(3 sqrt(lambda1))
 *   (u, v) = ((fx x)/z + cx, (fy y)/z + cy)
 *   pixel rect: x in [max(0, ceil((u - r) - 0.5)), min(W-1, floor((u + r) - 0.5))], same for y
 *   tile rect = pixel rect / 16;  tiles = tile-rect area; any non-finite value culls.
 * Returns 1 if visible.
 */
typedef struct {
    float u, v, A, B, C, depth;
    int px0, px1, py0, py1; /* pixel rect, inclusive */
    int tx0, tx1, ty0, ty1; /* tile rect, inclusive */
} orc_proj;

static int project_one(const orc_camera* cam, const float* mu, const float* s, const float* q,
                       orc_proj* o) {
    const float* R = cam->R;
    float px = R[0] * mu[0] + R[1] * mu[1];
    px = px + R[2] * mu[2];
    px = px + cam->t[0];
    float py = R[3] * mu[0] + R[4] * mu[1];
    py = py + R[5] * mu[2];
    py = py + cam->t[1];
    float pz = R[6] * mu[0] + R[7] * mu[1];
    pz = pz + R[8] * mu[2];
    pz = pz + cam->t[2];
    if (!(pz > cam->near_z)) return 0;

    float qn = q[0] * q[0] + q[1] * q[1];
    qn = qn + q[2] * q[2];
    qn = qn + q[3] * q[3];
    qn = sqrtf(qn);
    float w = q[0] / qn, x = q[1] / qn, y = q[2] / qn, z = q[3] / qn;
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
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) M[i * 3 + j] = Rq[i * 3 + j] * s[j];
    float S[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            float acc = M[i * 3 + 0] * M[j * 3 + 0] + M[i * 3 + 1] * M[j * 3 + 1];
            S[i * 3 + j] = acc + M[i * 3 + 2] * M[j * 3 + 2];
        }
    float zz = pz * pz;
    float j00 = cam->fx / pz;
    float j02 = -(cam->fx * px) / zz;
    float j11 = cam->fy / pz;
    float j12 = -(cam->fy * py) / zz;
    float T[6];
    for (int k = 0; k < 3; ++k) {
        T[k] = j00 * R[k] + j02 * R[6 + k];
        T[3 + k] = j11 * R[3 + k] + j12 * R[6 + k];
    }
    float U[6];
    for (int i = 0; i < 2; ++i)
        for (int k = 0; k < 3; ++k) {
            float acc = T[i * 3 + 0] * S[0 * 3 + k] + T[i * 3 + 1] * S[1 * 3 + k];
            U[i * 3 + k] = acc + T[i * 3 + 2] * S[2 * 3 + k];
        }
    float c2[4];
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) {
            float acc = U[i * 3 + 0] * T[j * 3 + 0] + U[i * 3 + 1] * T[j * 3 + 1];
            c2[i * 2 + j] = acc + U[i * 3 + 2] * T[j * 3 + 2];
        }
    float a = c2[0], b = c2[1], c = c2[3];
    float det = a * c - b * b;
    if (!(det > 0.0f)) return 0;
    float inv = 1.0f / det;
    float A = c * inv, B = -b * inv, C = a * inv;
    float mid = 0.5f * (a + c);
    float disc = mid * mid - det;
    disc = disc > 0.0f ? disc : 0.0f;
    float lam = mid + sqrtf(disc);
    float r = ceilf(3.0f * sqrtf(lam));
    float u = (cam->fx * px) / pz + cam->cx;
    float v = (cam->fy * py) / pz + cam->cy;
    if (!(isfinite(u) && isfinite(v) && isfinite(A) && isfinite(B) && isfinite(C) && isfinite(r))) return 0;
    float x0 = ceilf((u - r) - 0.5f), x1 = floorf((u + r) - 0.5f);
    float y0 = ceilf((v - r) - 0.5f), y1 = floorf((v + r) - 0.5f);
    x0 = x0 > 0.0f ? x0 : 0.0f;
    y0 = y0 > 0.0f ? y0 : 0.0f;
    x1 = x1 < (float)(cam->W - 1) ? x1 : (float)(cam->W - 1);
    y1 = y1 < (float)(cam->H - 1) ? y1 : (float)(cam->H - 1);
    if (!(x0 <= x1 && y0 <= y1)) return 0;
    o->u = u; o->v = v; o->A = A; o->B = B; o->C = C; o->depth = pz;
    o->px0 = (int)x0; o->px1 = (int)x1; o->py0 = (int)y0; o->py1 = (int)y1;
    o->tx0 = o->px0 / 16; o->tx1 = o->px1 / 16; o->ty0 = o->py0 / 16; o->ty1 = o->py1 / 16;
    return 1;
}

static int frame_of(const long* frame_offsets, int F, long i) {
    int lo = 0, hi = F - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (frame_offsets[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/*
 * Project a batch of frames.  Outputs (per Gaussian): mean2d[2], conic[3],
 * depth, pixel rect [x0,x1,y0,y1], tile rect [tx0,ty0,tx1,ty1], tiles
 * touched (0 = culled).
 */
EXPORT void orc_preprocess(const orc_camera* cams, int F, const long* frame_offsets, const float* means,
                           const float* scales, const float* quats, float* mean2d, float* conic,
                           float* depth, int* pix_rect, int* tile_rect, uint32_t* tiles) {
    long N = frame_offsets[F];
#pragma omp parallel for schedule(static)
    for (long i = 0; i < N; ++i) {
        int f = frame_of(frame_offsets, F, i);
        orc_proj o;
        int vis = project_one(&cams[f], means + i * 3, scales + i * 3, quats + i * 4, &o);
        if (!vis) {
            memset(&o, 0, sizeof(o));
            o.px0 = o.py0 = o.tx0 = o.ty0 = 0;
            o.px1 = o.py1 = o.tx1 = o.ty1 = -1;
        }
        mean2d[i * 2] = o.u; mean2d[i * 2 + 1] = o.v;
        conic[i * 3] = o.A; conic[i * 3 + 1] = o.B; conic[i * 3 + 2] = o.C;
        depth[i] = o.depth;
        pix_rect[i * 4] = o.px0; pix_rect[i * 4 + 1] = o.px1; pix_rect[i * 4 + 2] = o.py0; pix_rect[i * 4 + 3] = o.py1;
        tile_rect[i * 4] = o.tx0; tile_rect[i * 4 + 1] = o.ty0; tile_rect[i * 4 + 2] = o.tx1; tile_rect[i * 4 + 3] = o.ty1;
        tiles[i] = vis ? (uint32_t)((o.tx1 - o.tx0 + 1) * (o.ty1 - o.ty0 + 1)) : 0u;
    }
}

/*
 * Colour of each Gaussian seen from its frame's camera, degree-3 SH:
 * dir = normalize(mu - centre), centre = -R^T t;  rgb = max(0, sum_k sh_k Y_k(dir) + 0.5).
 */
EXPORT void orc_sh_colors(const orc_camera* cams, int F, const long* frame_offsets, const float* means,
                          const float* sh, double* rgb) {
    long N = frame_offsets[F];
#pragma omp parallel for schedule(static)
    for (long i = 0; i < N; ++i) {
        const orc_camera* c = &cams[frame_of(frame_offsets, F, i)];
        double ctr[3];
        for (int k = 0; k < 3; ++k)
            ctr[k] = -((double)c->R[0 * 3 + k] * c->t[0] + (double)c->R[1 * 3 + k] * c->t[1] +
                       (double)c->R[2 * 3 + k] * c->t[2]);
        double d[3], n = 0.0;
        for (int k = 0; k < 3; ++k) { d[k] = (double)means[i * 3 + k] - ctr[k]; n += d[k] * d[k]; }
        n = sqrt(n);
        for (int k = 0; k < 3; ++k) d[k] /= n;
        double Y[16];
        orc_sh_basis(d, 1, Y);
        for (int ch = 0; ch < 3; ++ch) {
            double s = 0.5;
            for (int k = 0; k < 16; ++k) s += (double)sh[i * 48 + k * 3 + ch] * Y[k];
            rgb[i * 3 + ch] = s > 0.0 ? s : 0.0;
        }
    }
}

/*
 * Backward of orc_sh_colors for a colour gradient gcol = dL/drgb [N][3]:
 *   dL/dsh_k,ch = gcol_ch Y_k(dir) where sum_k sh_k,ch Y_k + 0.5 > 0, else 0
 *   dL/dmean    = (I - dir dir^T) / |mu - centre| . sum_ch,k gcol_ch [>0] sh_k,ch grad Y_k
 * with grad Y_k the derivative of the basis polynomials of orc_sh_basis in
 * (x, y, z), projected onto the sphere by the normalisation's Jacobian.
 * Outputs gsh [N][48] (k-major like sh) and gmeans [N][3] (overwritten).
 */
EXPORT void orc_sh_colors_grad(const orc_camera* cams, int F, const long* frame_offsets, const float* means,
                               const float* sh, const double* gcol, double* gsh, double* gmeans) {
    const double pi = 3.14159265358979323846;
    const double k1 = sqrt(3.0 / (4.0 * pi));
    const double k2a = 0.5 * sqrt(15.0 / pi), k2b = 0.25 * sqrt(5.0 / pi), k2c = 0.25 * sqrt(15.0 / pi);
    const double k3a = 0.25 * sqrt(35.0 / (2.0 * pi)), k3b = 0.5 * sqrt(105.0 / pi);
    const double k3c = 0.25 * sqrt(21.0 / (2.0 * pi)), k3d = 0.25 * sqrt(7.0 / pi);
    const double k3e = 0.25 * sqrt(105.0 / pi);
    long N = frame_offsets[F];
#pragma omp parallel for schedule(static)
    for (long i = 0; i < N; ++i) {
        const orc_camera* c = &cams[frame_of(frame_offsets, F, i)];
        double ctr[3];
        for (int k = 0; k < 3; ++k)
            ctr[k] = -((double)c->R[0 * 3 + k] * c->t[0] + (double)c->R[1 * 3 + k] * c->t[1] +
                       (double)c->R[2 * 3 + k] * c->t[2]);
        double d[3], n = 0.0;
        for (int k = 0; k < 3; ++k) { d[k] = (double)means[i * 3 + k] - ctr[k]; n += d[k] * d[k]; }
        n = sqrt(n);
        for (int k = 0; k < 3; ++k) d[k] /= n;
        double Y[16];
        orc_sh_basis(d, 1, Y);
        const double x = d[0], y = d[1], z = d[2], xx = x * x, yy = y * y, zz = z * z;
        /* dY_k / d(x, y, z) */
        const double dY[16][3] = {
            {0, 0, 0},
            {0, -k1, 0},
            {0, 0, k1},
            {-k1, 0, 0},
            {k2a * y, k2a * x, 0},
            {0, -k2a * z, -k2a * y},
            {-2 * k2b * x, -2 * k2b * y, 4 * k2b * z},
            {-k2a * z, 0, -k2a * x},
            {2 * k2c * x, -2 * k2c * y, 0},
            {-6 * k3a * x * y, -k3a * (3 * xx - 3 * yy), 0},
            {k3b * y * z, k3b * x * z, k3b * x * y},
            {2 * k3c * x * y, -k3c * (4 * zz - xx - 3 * yy), -8 * k3c * y * z},
            {-6 * k3d * x * z, -6 * k3d * y * z, k3d * (6 * zz - 3 * xx - 3 * yy)},
            {-k3c * (4 * zz - 3 * xx - yy), 2 * k3c * x * y, -8 * k3c * x * z},
            {2 * k3e * x * z, -2 * k3e * y * z, k3e * (xx - yy)},
            {-k3a * (3 * xx - 3 * yy), 6 * k3a * x * y, 0}};
        double gd[3] = {0, 0, 0};
        for (int ch = 0; ch < 3; ++ch) {
            double s = 0.5;
            for (int k = 0; k < 16; ++k) s += (double)sh[i * 48 + k * 3 + ch] * Y[k];
            const double g = s > 0.0 ? gcol[i * 3 + ch] : 0.0;
            for (int k = 0; k < 16; ++k) {
                gsh[i * 48 + k * 3 + ch] = g * Y[k];
                for (int a = 0; a < 3; ++a) gd[a] += g * (double)sh[i * 48 + k * 3 + ch] * dY[k][a];
            }
        }
        const double dot = d[0] * gd[0] + d[1] * gd[1] + d[2] * gd[2];
        for (int a = 0; a < 3; ++a) gmeans[i * 3 + a] = (gd[a] - d[a] * dot) / n;
    }
}

/* ------------------------------------------------------------------------ */
/* Binning and sort (16x16 tiles)                                             */
/* ------------------------------------------------------------------------ */

typedef struct { uint64_t key; uint64_t seq; uint32_t val; } orc_entry;

static int cmp_entry(const void* a, const void* b) {
    const orc_entry* x = (const orc_entry*)a;
    const orc_entry* y = (const orc_entry*)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    if (x->seq != y->seq) return x->seq < y->seq ? -1 : 1;
    return 0;
}

static uint32_t float_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/*
 * Emit one entry per (visible Gaussian, touched tile): Gaussians in ascending
 * index, tiles by row then column; key = ((frame*ntiles + ty*tiles_x + tx) << 32)
 * | bits(depth), val = Gaussian index.  Stable ascending sort on the key (ties
 * keep emission order), then per-tile [start, end) ranges (empty = [0,0)).
 * Returns the entry count E; writes at most cap entries.
 */
EXPORT long orc_bin(int F, int W, int H, const long* frame_offsets, const float* depth, const int* tile_rect,
                    const uint32_t* tiles, long cap, uint64_t* keys, uint32_t* vals, uint32_t* ranges) {
    long N = frame_offsets[F];
    int tx_n = (W + 15) / 16, ty_n = (H + 15) / 16;
    long ntiles = (long)tx_n * ty_n;
    long E = 0;
    for (long i = 0; i < N; ++i) E += tiles[i];
    orc_entry* ent = (orc_entry*)malloc(sizeof(orc_entry) * (size_t)(E > 0 ? E : 1));
    long e = 0;
    for (long i = 0; i < N; ++i) {
        if (!tiles[i]) continue;
        long f = frame_of(frame_offsets, F, i);
        for (int ty = tile_rect[i * 4 + 1]; ty <= tile_rect[i * 4 + 3]; ++ty)
            for (int tx = tile_rect[i * 4 + 0]; tx <= tile_rect[i * 4 + 2]; ++tx) {
                uint64_t tile = (uint64_t)(f * ntiles + (long)ty * tx_n + tx);
                ent[e].key = (tile << 32) | float_bits(depth[i]);
                ent[e].seq = (uint64_t)e;
                ent[e].val = (uint32_t)i;
                ++e;
            }
    }
    qsort(ent, (size_t)E, sizeof(orc_entry), cmp_entry);
    for (long k = 0; k < (long)F * ntiles * 2; ++k) ranges[k] = 0;
    for (long k = 0; k < E; ++k) {
        if (k < cap) { keys[k] = ent[k].key; vals[k] = ent[k].val; }
        uint64_t tile = ent[k].key >> 32;
        if (k == 0 || (ent[k - 1].key >> 32) != tile) ranges[tile * 2] = (uint32_t)k;
        if (k == E - 1 || (ent[k + 1].key >> 32) != tile) ranges[tile * 2 + 1] = (uint32_t)(k + 1);
    }
    free(ent);
    return E;
}

/* ------------------------------------------------------------------------ */
/* Compositing, [SPIN] §3.1 Eq. 1 and Eq. 4                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float* mean2d;
    const float* conic;
    const float* opacity;
    const double* color;
} orc_splats;

/*
 * One pixel over an ordered list of Gaussians, fp64:
 *   d = (px + 0.5 - u, py + 0.5 - v);  power = -0.5 (A dx^2 + C dy^2) - B dx dy
 *   skip if power < -4.5 (outside 3 sigma) or power > 0
 *   alpha = min(0.99, o exp(power));  skip if alpha < 1/255
 *   C += c alpha T;  T *= 1 - alpha;  stop once T < 1e-4 (after compositing)
 * n_contrib = 1 + list position of the last composited Gaussian.
 * flag = 1 if any decision lies within its rounding band of a threshold, so
 * that an fp32 evaluation may legitimately decide it the other way.
 */
static void composite(const orc_splats* g, const uint32_t* list, long n, int px, int py, double out[3],
                      double* T_out, uint32_t* nc_out, int* flag) {
    double T = 1.0, C[3] = {0, 0, 0};
    double relT = 0.0; /* bound on the relative error an fp32 evaluation of T may carry */
    uint32_t last = 0;
    int fl = 0;
    for (long j = 0; j < n; ++j) {
        uint32_t i = list[j];
        double dx = (double)px + 0.5 - (double)g->mean2d[i * 2];
        double dy = (double)py + 0.5 - (double)g->mean2d[i * 2 + 1];
        double A = g->conic[i * 3], B = g->conic[i * 3 + 1], Cc = g->conic[i * 3 + 2];
        double quad = A * dx * dx + Cc * dy * dy;
        double cross = B * dx * dy;
        double power = -0.5 * quad - cross;
        /* Rounding bands of an fp32 evaluation (u = 2^-24), doubled for margin:
         *   power: six roundings of terms no larger than mag -> 6 u mag;
         *   alpha = o exp(power): exp2 of a rounded product plus one ulp,
         *     a further rounding for o *, and the power error -> (10 u + 6 u mag)
         *     relative;
         *   T *= 1 - alpha: two roundings, plus alpha's error scaled by
         *     alpha / (1 - alpha). */
        const double u = 5.9604644775390625e-08;
        double mag = 0.5 * fabs(quad) + fabs(cross);
        double err_p = 2.0 * 6.0 * u * mag;
        if (fabs(power + 4.5) <= err_p) fl = 1;
        if (fabs(power) <= err_p && mag > 0.0) fl = 1;
        if (power < -4.5 || power > 0.0) continue;
        double ga = (double)g->opacity[i] * exp(power);
        double rel_a = 2.0 * (10.0 * u + 6.0 * u * mag);
        if (fabs(ga - 0.99) <= rel_a * 0.99) fl = 1;
        double alpha = ga < 0.99 ? ga : 0.99;
        if (fabs(alpha - 1.0 / 255.0) <= rel_a / 255.0) fl = 1;
        if (alpha < 1.0 / 255.0) continue;
        for (int k = 0; k < 3; ++k) C[k] += g->color[i * 3 + k] * alpha * T;
        T = T * (1.0 - alpha);
        last = (uint32_t)(j + 1);
        relT += 2.0 * (2.0 * u + alpha / (1.0 - alpha) * rel_a * 0.5);
        if (fabs(T - 1e-4) <= relT * 1e-4) fl = 1;
        if (T < 1e-4) break;
    }
    for (int k = 0; k < 3; ++k) out[k] = C[k];
    *T_out = T;
    *nc_out = last;
    *flag = fl;
}

/* Tiled raster: each pixel composites its tile's sorted list.  Output
 * image [F][3][H][W] = C + T bg, T_final and n_contrib [F][H][W], flags. */
EXPORT void orc_raster_tiles(int F, const orc_camera* cams, const uint32_t* vals, const uint32_t* ranges,
                             const float* mean2d, const float* conic, const float* opacity, const double* color,
                             double* image, double* T_final, uint32_t* n_contrib, uint8_t* flags) {
    int W = cams[0].W, H = cams[0].H;
    int tx_n = (W + 15) / 16, ty_n = (H + 15) / 16;
    orc_splats g = {mean2d, conic, opacity, color};
#pragma omp parallel for collapse(2) schedule(dynamic, 64)
    for (long f = 0; f < F; ++f)
        for (long pix = 0; pix < (long)W * H; ++pix) {
            int px = (int)(pix % W), py = (int)(pix / W);
            long tile = f * (long)tx_n * ty_n + (long)(py / 16) * tx_n + px / 16;
            uint32_t s = ranges[tile * 2], e = ranges[tile * 2 + 1];
            double c[3], T;
            uint32_t nc;
            int fl;
            composite(&g, vals + s, (long)e - (long)s, px, py, c, &T, &nc, &fl);
            for (int k = 0; k < 3; ++k) image[((f * 3 + k) * H + py) * (long)W + px] = c[k] + T * cams[f].bg[k];
            T_final[f * (long)W * H + pix] = T;
            n_contrib[f * (long)W * H + pix] = nc;
            flags[f * (long)W * H + pix] = (uint8_t)fl;
        }
}

typedef struct { uint32_t depth_bits; uint32_t idx; } orc_dorder;

static int cmp_dorder(const void* a, const void* b) {
    const orc_dorder* x = (const orc_dorder*)a;
    const orc_dorder* y = (const orc_dorder*)b;
    if (x->depth_bits != y->depth_bits) return x->depth_bits < y->depth_bits ? -1 : 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

/*
 * Brute-force raster of the listed pixels (or all pixels when n_pix < 0) of
 * one frame: every visible Gaussian of the frame in (depth, index) order; with
 * restrict_tiles only those whose tile rect holds the pixel's tile, which is
 * the tiled renderer's list by construction.  pix is [n_pix][2] (x, y);
 * outputs are per listed pixel: rgb[3], T, n_contrib (counted over the
 * per-pixel list), flag.
 */
EXPORT void orc_raster_brute(const orc_camera* cam, long g0, long g1, const float* mean2d, const float* conic,
                             const float* opacity, const double* color, const float* depth,
                             const int* tile_rect, const uint32_t* tiles, int restrict_tiles, const int* pix,
                             long n_pix, double* rgb, double* T_out, uint32_t* nc_out, uint8_t* flags) {
    long n = 0;
    orc_dorder* ord = (orc_dorder*)malloc(sizeof(orc_dorder) * (size_t)(g1 - g0 > 0 ? g1 - g0 : 1));
    for (long i = g0; i < g1; ++i)
        if (tiles[i]) { ord[n].depth_bits = float_bits(depth[i]); ord[n].idx = (uint32_t)i; ++n; }
    qsort(ord, (size_t)n, sizeof(orc_dorder), cmp_dorder);
    long npx = n_pix < 0 ? (long)cam->W * cam->H : n_pix;
    orc_splats g = {mean2d, conic, opacity, color};
#pragma omp parallel for schedule(dynamic, 16)
    for (long p = 0; p < npx; ++p) {
        int px = n_pix < 0 ? (int)(p % cam->W) : pix[p * 2];
        int py = n_pix < 0 ? (int)(p / cam->W) : pix[p * 2 + 1];
        int tx = px / 16, ty = py / 16;
        uint32_t* list = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(n > 0 ? n : 1));
        long m = 0;
        for (long k = 0; k < n; ++k) {
            uint32_t i = ord[k].idx;
            if (restrict_tiles && !(tile_rect[i * 4] <= tx && tx <= tile_rect[i * 4 + 2] &&
                                    tile_rect[i * 4 + 1] <= ty && ty <= tile_rect[i * 4 + 3]))
                continue;
            list[m++] = i;
        }
        double c[3], T;
        uint32_t nc;
        int fl;
        composite(&g, list, m, px, py, c, &T, &nc, &fl);
        for (int k = 0; k < 3; ++k) rgb[p * 3 + k] = c[k] + T * cam->bg[k];
        T_out[p] = T;
        nc_out[p] = nc;
        flags[p] = (uint8_t)fl;
        free(list);
    }
    free(ord);
}

/* ------------------------------------------------------------------------ */
/* Gradients of an image loss w.r.t. the Gaussians ([SPIN] §3.1 Eq. 1-4 and  */
/* the EWA projection, differentiated by hand), fp64 throughout               */
/* ------------------------------------------------------------------------ */

/*
 * fp64 projection of one Gaussian with the intermediates the backward pass
 * needs.  Same definitions and culling rules as project_one, evaluated in
 * double: p = R mu + t; qn = q / |q|; Rq(qn); M = Rq diag(s); Sigma = M M^T;
 * J = [[fx/z, 0, -fx x/z^2], [0, fy/z, -fy y/z^2]]; T = J R; Sigma2D =
 * T Sigma T^T = [[a, b], [b, c]]; conic (A, B, C) = (c, -b, a) / (a c - b^2);
 * (u, v) = (fx x / z + cx, fy y / z + cy); r = ceil(3 sqrt(lambda_max)).
 */
typedef struct {
    int vis;
    double p[3], qn[4], qlen, Rq[9], M[9], S[9], T[6], a, b, c, det;
    double u, v, A, B, C, depth;
    int tx0, tx1, ty0, ty1;
} orc_g64;

static void project64(const orc_camera* cam, const double* mu, const double* s, const double* q, orc_g64* o) {
    memset(o, 0, sizeof(*o));
    const float* R = cam->R;
    for (int k = 0; k < 3; ++k)
        o->p[k] = (double)R[k * 3] * mu[0] + (double)R[k * 3 + 1] * mu[1] + (double)R[k * 3 + 2] * mu[2] + cam->t[k];
    if (!(o->p[2] > cam->near_z)) return;
    double qq = 0.0;
    for (int k = 0; k < 4; ++k) qq += q[k] * q[k];
    o->qlen = sqrt(qq);
    for (int k = 0; k < 4; ++k) o->qn[k] = q[k] / o->qlen;
    double w = o->qn[0], x = o->qn[1], y = o->qn[2], z = o->qn[3];
    double* Rq = o->Rq;
    Rq[0] = 1 - 2 * (y * y + z * z); Rq[1] = 2 * (x * y - w * z); Rq[2] = 2 * (x * z + w * y);
    Rq[3] = 2 * (x * y + w * z); Rq[4] = 1 - 2 * (x * x + z * z); Rq[5] = 2 * (y * z - w * x);
    Rq[6] = 2 * (x * z - w * y); Rq[7] = 2 * (y * z + w * x); Rq[8] = 1 - 2 * (x * x + y * y);
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) o->M[i * 3 + j] = Rq[i * 3 + j] * s[j];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double acc = 0.0;
            for (int k = 0; k < 3; ++k) acc += o->M[i * 3 + k] * o->M[j * 3 + k];
            o->S[i * 3 + j] = acc;
        }
    double pz = o->p[2];
    double j00 = cam->fx / pz, j02 = -cam->fx * o->p[0] / (pz * pz);
    double j11 = cam->fy / pz, j12 = -cam->fy * o->p[1] / (pz * pz);
    for (int k = 0; k < 3; ++k) {
        o->T[k] = j00 * R[k] + j02 * R[6 + k];
        o->T[3 + k] = j11 * R[3 + k] + j12 * R[6 + k];
    }
    double c2[4];
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) {
            double acc = 0.0;
            for (int k = 0; k < 3; ++k)
                for (int l = 0; l < 3; ++l) acc += o->T[i * 3 + k] * o->S[k * 3 + l] * o->T[j * 3 + l];
            c2[i * 2 + j] = acc;
        }
    o->a = c2[0]; o->b = c2[1]; o->c = c2[3];
    o->det = o->a * o->c - o->b * o->b;
    if (!(o->det > 0.0)) return;
    o->A = o->c / o->det; o->B = -o->b / o->det; o->C = o->a / o->det;
    double mid = 0.5 * (o->a + o->c);
    double disc = mid * mid - o->det;
    double lam = mid + sqrt(disc > 0.0 ? disc : 0.0);
    double r = ceil(3.0 * sqrt(lam));
    o->u = cam->fx * o->p[0] / pz + cam->cx;
    o->v = cam->fy * o->p[1] / pz + cam->cy;
    if (!(isfinite(o->u) && isfinite(o->v) && isfinite(o->A) && isfinite(o->B) && isfinite(o->C) && isfinite(r)))
        return;
    double x0 = ceil((o->u - r) - 0.5), x1 = floor((o->u + r) - 0.5);
    double y0 = ceil((o->v - r) - 0.5), y1 = floor((o->v + r) - 0.5);
    x0 = x0 > 0 ? x0 : 0; y0 = y0 > 0 ? y0 : 0;
    x1 = x1 < cam->W - 1 ? x1 : cam->W - 1; y1 = y1 < cam->H - 1 ? y1 : cam->H - 1;
    if (!(x0 <= x1 && y0 <= y1)) return;
    o->depth = pz;
    o->tx0 = (int)x0 / 16; o->tx1 = (int)x1 / 16; o->ty0 = (int)y0 / 16; o->ty1 = (int)y1 / 16;
    o->vis = 1;
}

/* Chain the gradient of (u, v, A, B, C) back to (mu, s, q) for one projected
 * Gaussian (see project64 for the definitions). */
static void project64_backward(const orc_camera* cam, const double* s, const orc_g64* o, const double g2[5],
                               double gmu[3], double gs[3], double gq[4]) {
    const float* R = cam->R;
    double gu = g2[0], gv = g2[1], gA = g2[2], gB = g2[3], gC = g2[4];
    /* conic = Sigma2D^-1: dL/dSigma2D = -K G K with G the symmetric gradient of K */
    double K[4] = {o->A, o->B, o->B, o->C};
    double G[4] = {gA, 0.5 * gB, 0.5 * gB, gC};
    double KG[4], GS[4];
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) KG[i * 2 + j] = K[i * 2] * G[j] + K[i * 2 + 1] * G[2 + j];
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) GS[i * 2 + j] = -(KG[i * 2] * K[j] + KG[i * 2 + 1] * K[2 + j]);
    /* Sigma2D = T Sigma T^T: dL/dT = 2 GS T Sigma, dL/dSigma = T^T GS T */
    double TS[6];
    for (int i = 0; i < 2; ++i)
        for (int k = 0; k < 3; ++k) {
            double acc = 0.0;
            for (int l = 0; l < 3; ++l) acc += o->T[i * 3 + l] * o->S[l * 3 + k];
            TS[i * 3 + k] = acc;
        }
    double GT[6];
    for (int i = 0; i < 2; ++i)
        for (int k = 0; k < 3; ++k) GT[i * 3 + k] = 2.0 * (GS[i * 2] * TS[k] + GS[i * 2 + 1] * TS[3 + k]);
    double GSig[9];
    for (int k = 0; k < 3; ++k)
        for (int l = 0; l < 3; ++l) {
            double acc = 0.0;
            for (int i = 0; i < 2; ++i)
                for (int j = 0; j < 2; ++j) acc += o->T[i * 3 + k] * GS[i * 2 + j] * o->T[j * 3 + l];
            GSig[k * 3 + l] = acc;
        }
    /* T = J R: dL/dJ = GT R^T (J has entries j00, j02, j11, j12) */
    double gj00 = 0, gj02 = 0, gj11 = 0, gj12 = 0;
    for (int k = 0; k < 3; ++k) {
        gj00 += GT[k] * R[0 * 3 + k];
        gj02 += GT[k] * R[2 * 3 + k];
        gj11 += GT[3 + k] * R[1 * 3 + k];
        gj12 += GT[3 + k] * R[2 * 3 + k];
    }
    double px = o->p[0], py = o->p[1], pz = o->p[2];
    double fx = cam->fx, fy = cam->fy;
    double gp[3];
    gp[0] = gu * fx / pz + gj02 * (-fx / (pz * pz));
    gp[1] = gv * fy / pz + gj12 * (-fy / (pz * pz));
    gp[2] = gu * (-fx * px / (pz * pz)) + gv * (-fy * py / (pz * pz)) + gj00 * (-fx / (pz * pz)) +
            gj02 * (2.0 * fx * px / (pz * pz * pz)) + gj11 * (-fy / (pz * pz)) + gj12 * (2.0 * fy * py / (pz * pz * pz));
    for (int k = 0; k < 3; ++k) gmu[k] = R[0 * 3 + k] * gp[0] + R[1 * 3 + k] * gp[1] + R[2 * 3 + k] * gp[2];
    /* Sigma = M M^T: dL/dM = 2 GSig M;  M = Rq diag(s) */
    double GM[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double acc = 0.0;
            for (int k = 0; k < 3; ++k) acc += GSig[i * 3 + k] * o->M[k * 3 + j];
            GM[i * 3 + j] = 2.0 * acc;
        }
    double GR[9];
    for (int j = 0; j < 3; ++j) {
        double acc = 0.0;
        for (int i = 0; i < 3; ++i) {
            acc += GM[i * 3 + j] * o->Rq[i * 3 + j];
            GR[i * 3 + j] = GM[i * 3 + j] * s[j];
        }
        gs[j] = acc;
    }
    /* Rq(w, x, y, z) of the unit quaternion, then through q / |q| */
    double w = o->qn[0], x = o->qn[1], y = o->qn[2], z = o->qn[3];
    double gn[4];
    gn[0] = 2.0 * (-z * GR[1] + y * GR[2] + z * GR[3] - x * GR[5] - y * GR[6] + x * GR[7]);
    gn[1] = 2.0 * (y * GR[1] + z * GR[2] + y * GR[3] - 2.0 * x * GR[4] - w * GR[5] + z * GR[6] + w * GR[7] -
                   2.0 * x * GR[8]);
    gn[2] = 2.0 * (-2.0 * y * GR[0] + x * GR[1] + w * GR[2] + x * GR[3] + z * GR[5] - w * GR[6] + z * GR[7] -
                   2.0 * y * GR[8]);
    gn[3] = 2.0 * (-2.0 * z * GR[0] - w * GR[1] + x * GR[2] + w * GR[3] - 2.0 * z * GR[4] + y * GR[5] + x * GR[6] +
                   y * GR[7]);
    double dot = gn[0] * w + gn[1] * x + gn[2] * y + gn[3] * z;
    for (int k = 0; k < 4; ++k) gq[k] = (gn[k] - dot * o->qn[k]) / o->qlen;
}

typedef struct { double depth; uint32_t idx; } orc_dsort;

static int cmp_dsort(const void* a, const void* b) {
    const orc_dsort* x = (const orc_dsort*)a;
    const orc_dsort* y = (const orc_dsort*)b;
    if (x->depth != y->depth) return x->depth < y->depth ? -1 : 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

static uint64_t mix64(uint64_t h, uint64_t v) {
    h ^= v + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
    return h * 0xff51afd7ed558ccdull;
}

/*
 * Forward (fp64 projection, fp64 compositing with the rules of composite())
 * and backward of a given image-space gradient gimg = dL/dimage [F][3][H][W].
 * Per pixel, the frame's visible Gaussians whose tile rect holds the pixel's
 * tile are composited in (depth, index) order; the backward pass walks the
 * composited ones from the last to the first with
 *   T_i = T_{i+1} / (1 - alpha_i)  (T after the last = T_final)
 *   dL/dc_i = g alpha_i T_i,   dL/dalpha_i = g . (c_i T_i - S_i / (1 - alpha_i))
 *   S_i = sum_{j > i} c_j alpha_j T_j + T_final bg  (what lies behind i)
 *   alpha = o exp(power) unless clamped at 0.99 (then constant)
 *   power = -0.5 (A dx^2 + C dy^2) - B dx dy,  d = (px + 0.5 - u, py + 0.5 - v)
 * and each Gaussian's (u, v, A, B, C) gradient is chained to (mu, s, q) by
 * project64_backward.  Outputs (all optional but gproj): image [F][3][H][W];
 * gproj [N][9] = d/d(u, v, A, B, C, o, r, g, b); gmeans [N][3], gscales [N][3],
 * gquats [N][4], gopacity [N], gcolors [N][3]; gflag [N] = 1 if the Gaussian
 * took part in a decision within rounding of a threshold (compare only
 * unflagged ones); *signature = a hash of every discrete decision (which
 * Gaussians composite each pixel, clamps, stops): equal signatures mean
 * equal decisions.
 */
EXPORT void orc_render_grad(const orc_camera* cams, int F, const long* frame_offsets, const double* means,
                            const double* scales, const double* quats, const double* opacity, const double* colors,
                            const double* gimg, double* image, double* gproj, double* gmeans, double* gscales,
                            double* gquats, double* gopacity, double* gcolors, uint8_t* gflag, uint64_t* signature) {
    long N = frame_offsets[F];
    int W = cams[0].W, H = cams[0].H;
    orc_g64* P = (orc_g64*)malloc(sizeof(orc_g64) * (size_t)(N > 0 ? N : 1));
    for (long i = 0; i < N; ++i)
        project64(&cams[frame_of(frame_offsets, F, i)], means + i * 3, scales + i * 3, quats + i * 4, &P[i]);
    for (long i = 0; i < N * 9; ++i) gproj[i] = 0.0;
    if (gflag) memset(gflag, 0, (size_t)N);
    uint64_t sig = 0;
    const double u32 = 5.9604644775390625e-08;
    for (int f = 0; f < F; ++f) {
        long g0 = frame_offsets[f], g1 = frame_offsets[f + 1];
        const orc_camera* cam = &cams[f];
        orc_dsort* ord = (orc_dsort*)malloc(sizeof(orc_dsort) * (size_t)(g1 - g0 > 0 ? g1 - g0 : 1));
        long n = 0;
        for (long i = g0; i < g1; ++i)
            if (P[i].vis) { ord[n].depth = P[i].depth; ord[n].idx = (uint32_t)i; ++n; }
        qsort(ord, (size_t)n, sizeof(orc_dsort), cmp_dsort);
        uint32_t* taken = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(n > 0 ? n : 1));
        double* talpha = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double* tG = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        int* tclamp = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
        for (int py = 0; py < H; ++py)
            for (int px = 0; px < W; ++px) {
                int tx = px / 16, ty = py / 16;
                double T = 1.0, Cc[3] = {0, 0, 0}, relT = 0.0;
                long m = 0;
                int fl = 0;
                uint64_t hp = mix64((uint64_t)f, (uint64_t)(py * W + px));
                for (long k = 0; k < n; ++k) {
                    uint32_t i = ord[k].idx;
                    const orc_g64* o = &P[i];
                    if (!(o->tx0 <= tx && tx <= o->tx1 && o->ty0 <= ty && ty <= o->ty1)) continue;
                    double dx = px + 0.5 - o->u, dy = py + 0.5 - o->v;
                    double quad = o->A * dx * dx + o->C * dy * dy, cross = o->B * dx * dy;
                    double power = -0.5 * quad - cross;
                    double mag = 0.5 * fabs(quad) + fabs(cross);
                    double err_p = 2.0 * 6.0 * u32 * mag;
                    int near = fabs(power + 4.5) <= err_p || (fabs(power) <= err_p && mag > 0.0);
                    if (power < -4.5 || power > 0.0) { if (near) { fl = 1; if (gflag) gflag[i] = 1; } continue; }
                    double G = exp(power), ga = opacity[i] * G;
                    double rel_a = 2.0 * (10.0 * u32 + 6.0 * u32 * mag);
                    if (fabs(ga - 0.99) <= rel_a * 0.99) near = 1;
                    int clamp = !(ga < 0.99);
                    double alpha = clamp ? 0.99 : ga;
                    if (fabs(alpha - 1.0 / 255.0) <= rel_a / 255.0) near = 1;
                    if (near) { fl = 1; if (gflag) gflag[i] = 1; }
                    if (alpha < 1.0 / 255.0) continue;
                    for (int ch = 0; ch < 3; ++ch) Cc[ch] += colors[i * 3 + ch] * alpha * T;
                    T = T * (1.0 - alpha);
                    taken[m] = i; talpha[m] = alpha; tG[m] = G; tclamp[m] = clamp; ++m;
                    hp = mix64(hp, (uint64_t)i * 2 + (uint64_t)clamp);
                    relT += 2.0 * (2.0 * u32 + alpha / (1.0 - alpha) * rel_a * 0.5);
                    if (fabs(T - 1e-4) <= relT * 1e-4) { fl = 1; if (gflag) gflag[i] = 1; }
                    if (T < 1e-4) break;
                }
                sig += hp;
                long pix = ((long)f * H + py) * W + px;
                if (image)
                    for (int ch = 0; ch < 3; ++ch) image[((long)f * 3 + ch) * H * W + (long)py * W + px] = Cc[ch] + T * cam->bg[ch];
                if (fl)
                    for (long k = 0; k < m; ++k)
                        if (gflag) gflag[taken[k]] = 1;
                double g[3];
                for (int ch = 0; ch < 3; ++ch) g[ch] = gimg[((long)f * 3 + ch) * H * W + (long)py * W + px];
                double acc[3];
                for (int ch = 0; ch < 3; ++ch) acc[ch] = T * cam->bg[ch];
                double Tn = T;
                for (long k = m - 1; k >= 0; --k) {
                    uint32_t i = taken[k];
                    const orc_g64* o = &P[i];
                    double alpha = talpha[k];
                    double Ti = Tn / (1.0 - alpha);
                    double galpha = 0.0;
                    for (int ch = 0; ch < 3; ++ch) {
                        double ci = colors[i * 3 + ch];
                        gproj[i * 9 + 6 + ch] += g[ch] * alpha * Ti;
                        galpha += g[ch] * (ci * Ti - acc[ch] / (1.0 - alpha));
                        acc[ch] += ci * alpha * Ti;
                    }
                    Tn = Ti;
                    if (tclamp[k]) continue;
                    gproj[i * 9 + 5] += galpha * tG[k];
                    double gpow = galpha * alpha;
                    double dx = px + 0.5 - o->u, dy = py + 0.5 - o->v;
                    gproj[i * 9 + 0] += gpow * (o->A * dx + o->B * dy);
                    gproj[i * 9 + 1] += gpow * (o->C * dy + o->B * dx);
                    gproj[i * 9 + 2] += gpow * (-0.5 * dx * dx);
                    gproj[i * 9 + 3] += gpow * (-dx * dy);
                    gproj[i * 9 + 4] += gpow * (-0.5 * dy * dy);
                }
                (void)pix;
            }
        free(ord); free(taken); free(talpha); free(tG); free(tclamp);
    }
    for (long i = 0; i < N; ++i) {
        double gmu[3] = {0, 0, 0}, gs[3] = {0, 0, 0}, gq[4] = {0, 0, 0, 0};
        if (P[i].vis)
            project64_backward(&cams[frame_of(frame_offsets, F, i)], scales + i * 3, &P[i], gproj + i * 9, gmu, gs, gq);
        for (int k = 0; k < 3; ++k) {
            if (gmeans) gmeans[i * 3 + k] = gmu[k];
            if (gscales) gscales[i * 3 + k] = gs[k];
            if (gcolors) gcolors[i * 3 + k] = gproj[i * 9 + 6 + k];
        }
        for (int k = 0; k < 4; ++k)
            if (gquats) gquats[i * 4 + k] = gq[k];
        if (gopacity) gopacity[i] = gproj[i * 9 + 5];
    }
    if (signature) *signature = sig;
    free(P);
}

/* ------------------------------------------------------------------------ */
/* Decode gradients: backward of [SPIN] §3.3 Eq. 7-11                        */
/* ------------------------------------------------------------------------ */

static double gelu_grad(double x) {
    /* d/dx [0.5 x (1 + erf(x / sqrt 2))] = Phi(x) + x phi(x) */
    return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * exp(-0.5 * x * x) / sqrt(2.0 * acos(-1.0));
}

/*
 * Forward and backward of the decode for one batch, with every parameter in
 * fp64: tables [L][T][F], W[l] row-major [out][in], b[l].  pos [N][3] and
 * tpos [N] (the time of each point).
 *
 * mode bit 0: the MLP input and every hidden activation are rounded to
 *   binary16 in the forward (as the fp16 device path does); the backward
 *   treats that rounding as the identity.
 * mode bit 1: the normalisation and the cell decision are made in fp32 from
 *   (float) pos and (float) t, as orc_normalize and orc_encode do; otherwise
 *   they are fp64.  The Jacobian of the normalisation is fp64 either way.
 *
 * Outputs of the forward: raw [N][11] (head outputs) and the activations of
 * Eq. 11 (scales, quats, colors, opacity); all nullable.  A head of 56
 * outputs is the SH colour decoder ([SPIN] §3.3: s | r | 48 SH coefficients
 * | o): then raw is [N][56], `colors` receives the 48 coefficients per
 * Gaussian (no activation, so dr = dsh) and gc is [N][48].  With the upstream
 * gradients gs [N][3], gq [N][4], gc [N][3], go [N] given (else forward
 * only), the backward accumulates, for L = sum gs.s + gq.q + gc.c + go.o:
 *   g_tables [L][T][F]   += w_c dL/dz           (scatter-add over the corners)
 *   g_W[l], g_b[l]       += outer products / sums over the batch
 *   g_pos [N][3]          = dL/dposition through Eq. 7 and the corner weights
 * through (in order)
 *   Eq. 11: s = exp(min(r, 20)) -> dr = ds s (0 above the clip);
 *           q = r / max(|r|, 1e-12) -> dr = (dq - (dq.q) q) / |r|;
 *           c = sigmoid(r) -> dr = dc c (1 - c); same for o;
 *   Eq. 10: the head is linear; a hidden layer y = act(W x + b) passes
 *           dx = W^T (dy act'(W x + b)) with ReLU' = [a > 0] and
 *           GELU' = Phi(a) + a phi(a);
 *   Eq. 9:  z = sum_c w_c table[c], w_c = prod_axis (bit ? f : 1 - f), so
 *           dz/df_a = sum_c (bit_a ? 1 : -1) prod_{b != a} w_b table[c], and
 *           df_a / dx~_a = res_a - 1 (the time axis carries no gradient);
 *   Eq. 7:  x~ = c(mu) / 4 + 1/2 with c = mu for |mu| <= 1, else
 *           c = g(n) mu, g(n) = 2/n - 1/n^2, whose Jacobian is
 *           g I + (g'(n) / n) mu mu^T, g'(n) = -2/n^2 + 2/n^3.
 * flags [N] (nullable) = 1 where a ReLU pre-activation is exactly 0, a scale
 * output sits at the clip or |r| at its floor (the derivative is one-sided
 * there).  *signature (nullable) hashes every cell index, ReLU sign and clip,
 * so that finite differences can check that +-h keeps the same decisions.
 */
EXPORT void orc_decode_grad(const orc_hash* h, const double* tables, const orc_mlp* m, const double* const* W,
                            const double* const* b, const double* pos, const double* tpos, long N, int mode,
                            const double* gs, const double* gq, const double* gc, const double* go, double* raw_out,
                            double* scales, double* quats, double* colors, double* opacity, double* g_tables,
                            double* const* g_W, double* const* g_b, double* g_pos, uint8_t* flags,
                            uint64_t* signature) {
    int res_s[64], res_t[64], dense[64];
    orc_level_res(h, res_s, res_t, dense);
    const uint32_t mask = (uint32_t)((1UL << h->log2T) - 1);
    const long T = 1L << h->log2T;
    const int L = h->L, F = h->F, LF = L * F, nl = m->n_layers;
    const int backward = gs && gq && gc && go;
    /* head of 56 outputs: the SH colour decoder (s | r | 48 SH | o), whose
       colour slots are the coefficients themselves; else 11 (s | r | c | o) */
    const int sh = m->dims[nl] == 56, head = sh ? 56 : 11, ncol = sh ? 48 : 3;
    /* every branch's layer inputs and pre-activations of the current point */
    double(*xs)[8][512] = (double(*)[8][512])malloc(sizeof(double) * 4 * 8 * 512);
    double(*pre)[8][512] = (double(*)[8][512])malloc(sizeof(double) * 4 * 8 * 512);
    uint64_t sig = 0;
    for (long i = 0; i < N; ++i) {
        uint64_t hs = mix64(0x9e3779b97f4a7c15ull, (uint64_t)i);
        int fl = 0;
        /* Eq. 7-8 */
        double xt[4], J[9];
        const double* mu = pos + i * 3;
        double n = sqrt(mu[0] * mu[0] + mu[1] * mu[1] + mu[2] * mu[2]);
        if (mode & 2) {
            float pf[3] = {(float)mu[0], (float)mu[1], (float)mu[2]}, out[4];
            orc_normalize(h, pf, 3, (float)tpos[i], 1, out);
            for (int a = 0; a < 4; ++a) xt[a] = out[a];
        } else {
            double c[3] = {mu[0], mu[1], mu[2]};
            if (!(n <= 1.0)) {
                double k = (2.0 - 1.0 / n) / n;
                for (int a = 0; a < 3; ++a) c[a] = mu[a] * k;
            }
            double tn = (tpos[i] - h->t_min) / (h->t_max - h->t_min);
            tn = tn < 0.0 ? 0.0 : (tn > 1.0 ? 1.0 : tn);
            for (int a = 0; a < 3; ++a) xt[a] = 0.25 * c[a] + 0.5;
            xt[3] = tn;
        }
        hs = mix64(hs, n <= 1.0);
        for (int r = 0; r < 3; ++r)
            for (int c = 0; c < 3; ++c) {
                if (n <= 1.0) {
                    J[r * 3 + c] = r == c ? 0.25 : 0.0;
                } else {
                    double g = 2.0 / n - 1.0 / (n * n), gp = -2.0 / (n * n) + 2.0 / (n * n * n);
                    J[r * 3 + c] = 0.25 * ((r == c ? g : 0.0) + gp / n * mu[r] * mu[c]);
                }
            }
        /* Eq. 9: per level, the cell, the corner weights and the corner indices */
        double z[512];
        long cidx[64][16];
        double fr[64][4];
        for (int l = 0; l < L; ++l) {
            int res[4] = {res_s[l], res_s[l], res_s[l], res_t[l]};
            int ci[4];
            for (int a = 0; a < 4; ++a) {
                int c;
                double f;
                if (mode & 2) {
                    float p = (float)xt[a] * (float)(res[a] - 1);
                    c = (int)floorf(p);
                    if (c < 0) c = 0;
                    if (c > res[a] - 2) c = res[a] - 2;
                    f = (double)p - (double)c;
                } else {
                    double p = xt[a] * (double)(res[a] - 1);
                    c = (int)floor(p);
                    if (c < 0) c = 0;
                    if (c > res[a] - 2) c = res[a] - 2;
                    f = p - (double)c;
                }
                ci[a] = c;
                fr[l][a] = f;
                hs = mix64(hs, (uint64_t)(uint32_t)c);
            }
            for (int k = 0; k < F; ++k) z[l * F + k] = 0.0;
            for (int corner = 0; corner < 16; ++corner) {
                double w = 1.0;
                uint32_t v[4];
                for (int a = 0; a < 4; ++a) {
                    int bit = (corner >> a) & 1;
                    v[a] = (uint32_t)(ci[a] + bit);
                    w *= bit ? fr[l][a] : 1.0 - fr[l][a];
                }
                long idx = dense[l] ? (long)v[0] + (long)res[0] * ((long)v[1] + (long)res[1] * ((long)v[2] + (long)res[2] * (long)v[3]))
                                    : (long)hash4(v[0], v[1], v[2], v[3], mask);
                cidx[l][corner] = idx;
                for (int k = 0; k < F; ++k) z[l * F + k] += w * tables[((long)l * T + idx) * F + k];
            }
        }
        /* Eq. 10 forward, keeping every layer's input and pre-activation: one
           MLP, or one per attribute whose outputs fill head rows
           [row0[br], row0[br] + width[br]) (scale, rotation, colour, opacity) */
        const int nbr = m->branches ? 4 : 1;
        const int row0[4] = {0, 3, 7, head - 1}, width[4] = {3, 4, ncol, 1};
        double r[512];
        for (int br = 0; br < nbr; ++br) {
            const double* const* Wb = W + br * nl;
            const double* const* bb = b + br * nl;
            for (int k = 0; k < LF; ++k) xs[br][0][k] = (mode & 1) ? round_f16(z[k]) : z[k];
            for (int l = 0; l < nl; ++l) {
                int di = m->dims[l], dout = l + 1 < nl || !m->branches ? m->dims[l + 1] : width[br];
                for (int o = 0; o < dout; ++o) {
                    double s = 0.0;
                    for (int k = 0; k < di; ++k) s += Wb[l][(long)o * di + k] * xs[br][l][k];
                    s += bb[l][o];
                    pre[br][l][o] = s;
                    if (l + 1 < nl) {
                        if (m->act == 0) {
                            if (s == 0.0) fl = 1;
                            hs = mix64(hs, s > 0.0);
                        }
                        double y = act_fn(m->act, s);
                        xs[br][l + 1][o] = (mode & 1) ? round_f16(y) : y;
                    }
                }
            }
            if (m->branches)
                for (int k = 0; k < width[br]; ++k) r[row0[br] + k] = pre[br][nl - 1][k];
            else
                for (int k = 0; k < head; ++k) r[k] = pre[0][nl - 1][k];
        }
        /* Eq. 11 */
        double s3[3], q4[4], c3[3], o1;
        for (int k = 0; k < 3; ++k) {
            s3[k] = exp(r[k] < 20.0 ? r[k] : 20.0);
            if (r[k] == 20.0) fl = 1;
            hs = mix64(hs, r[k] < 20.0);
        }
        double qn = sqrt(r[3] * r[3] + r[4] * r[4] + r[5] * r[5] + r[6] * r[6]);
        if (qn == 1e-12) fl = 1;
        hs = mix64(hs, qn < 1e-12);
        double qd = qn < 1e-12 ? 1e-12 : qn;
        for (int k = 0; k < 4; ++k) q4[k] = r[3 + k] / qd;
        for (int k = 0; k < 3; ++k) c3[k] = sigmoid(r[7 + k]);
        o1 = sigmoid(r[head - 1]);
        if (raw_out)
            for (int k = 0; k < head; ++k) raw_out[i * head + k] = r[k];
        if (scales)
            for (int k = 0; k < 3; ++k) scales[i * 3 + k] = s3[k];
        if (quats)
            for (int k = 0; k < 4; ++k) quats[i * 4 + k] = q4[k];
        if (colors)  /* the RGB colour, or the SH coefficients (no activation) */
            for (int k = 0; k < ncol; ++k) colors[i * ncol + k] = sh ? r[7 + k] : c3[k];
        if (opacity) opacity[i] = o1;
        if (flags) flags[i] = (uint8_t)fl;
        sig += hs;
        if (!backward) continue;
        /* backward of Eq. 11 */
        double gy[512];
        for (int k = 0; k < 3; ++k) gy[k] = r[k] < 20.0 ? gs[i * 3 + k] * s3[k] : 0.0;
        double dot = 0.0;
        for (int k = 0; k < 4; ++k) dot += gq[i * 4 + k] * q4[k];
        for (int k = 0; k < 4; ++k)
            gy[3 + k] = qn < 1e-12 ? gq[i * 4 + k] / 1e-12 : (gq[i * 4 + k] - dot * q4[k]) / qn;
        for (int k = 0; k < ncol; ++k) gy[7 + k] = sh ? gc[i * ncol + k] : gc[i * 3 + k] * c3[k] * (1.0 - c3[k]);
        gy[head - 1] = go[i] * o1 * (1.0 - o1);
        /* backward of Eq. 10, last layer first; with branches each branch
           starts from its head rows and the branches' input gradients add up
           in dz */
        double dz[512];
        for (int k = 0; k < LF; ++k) dz[k] = 0.0;
        for (int br = 0; br < nbr; ++br) {
            const double* const* Wb = W + br * nl;
            double* const* gWb = g_W + br * nl;
            double* const* gbb = g_b + br * nl;
            double g[512];
            const int outw = m->branches ? width[br] : head;
            for (int k = 0; k < outw; ++k) g[k] = gy[(m->branches ? row0[br] : 0) + k];
            for (int l = nl - 1; l >= 0; --l) {
                int di = m->dims[l], dout = l + 1 < nl || !m->branches ? m->dims[l + 1] : width[br];
                if (l + 1 < nl)
                    for (int o = 0; o < dout; ++o)
                        g[o] *= m->act == 0 ? (pre[br][l][o] > 0.0 ? 1.0 : 0.0) : gelu_grad(pre[br][l][o]);
                double gx[512];
                for (int k = 0; k < di; ++k) gx[k] = 0.0;
                for (int o = 0; o < dout; ++o) {
                    gbb[l][o] += g[o];
                    for (int k = 0; k < di; ++k) {
                        gWb[l][(long)o * di + k] += g[o] * xs[br][l][k];
                        gx[k] += Wb[l][(long)o * di + k] * g[o];
                    }
                }
                for (int k = 0; k < di; ++k) g[k] = gx[k];
            }
            for (int k = 0; k < LF; ++k) dz[k] += g[k];
        }
        for (int k = 0; k < LF; ++k) gy[k] = dz[k];
        /* backward of Eq. 9 (tables and cell fractions) and Eq. 7 */
        double gxt[3] = {0.0, 0.0, 0.0};
        for (int l = 0; l < L; ++l) {
            int res[4] = {res_s[l], res_s[l], res_s[l], res_t[l]};
            for (int corner = 0; corner < 16; ++corner) {
                double wa[4];
                for (int a = 0; a < 4; ++a) wa[a] = ((corner >> a) & 1) ? fr[l][a] : 1.0 - fr[l][a];
                double w = ((wa[0] * wa[1]) * wa[2]) * wa[3];
                long idx = cidx[l][corner];
                double tg = 0.0;
                for (int k = 0; k < F; ++k) {
                    g_tables[((long)l * T + idx) * F + k] += w * gy[l * F + k];
                    tg += gy[l * F + k] * tables[((long)l * T + idx) * F + k];
                }
                for (int a = 0; a < 3; ++a) {
                    double d = ((corner >> a) & 1) ? 1.0 : -1.0;
                    for (int e = 0; e < 4; ++e)
                        if (e != a) d *= wa[e];
                    gxt[a] += tg * d * (double)(res[a] - 1);
                }
            }
        }
        for (int c = 0; c < 3; ++c)
            g_pos[i * 3 + c] = J[0 * 3 + c] * gxt[0] + J[1 * 3 + c] * gxt[1] + J[2 * 3 + c] * gxt[2];
    }
    free(xs);
    free(pre);
    if (signature) *signature = sig;
}
