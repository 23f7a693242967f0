/*
 * Oracle: a plain CPU implementation of the dense decoder-only transformer
 * decode step.  TEST INFRASTRUCTURE ONLY (see oracle.h): only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it.
 *
 * What one step computes follows the description of per-token decoding in
 * "How the xAI engineering team cut Grok Bot latency to milliseconds" (§2.1:
 * weights, QKV projection, softmax, weighted sum, FFN, normalisation,
 * logits), made concrete as the standard pre-norm Llama-style block:
 * RMSNorm, fused QKV, half-split RoPE, grouped-query attention with a
 * 1/sqrt(head_dim) softmax scale (the scale the same page's fused-attention
 * listing uses, §3.1), output projection and residual, RMSNorm, SwiGLU FFN
 * and residual, final RMSNorm, untied LM head, greedy argmax.
 *
 * Every step is the plain definition in binary64: dot products are single
 * sequential sums, the softmax is max-subtracted exp / sum, no blocking, no
 * split of the key axis.  OpenMP only spreads independent rows (or heads)
 * over threads and never changes the order of any sum.
 */
#include "oracle.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static __thread char g_err[256];

static void set_err(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

const char* orc_last_error(void) { return g_err; }

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits */

double orc_h2d(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 0x1f, f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* Rounds |x| to a format with `mbits` fraction bits, exponent bias `bias`,
 * largest finite biased exponent `emax_biased`, no saturation.  Returns the
 * magnitude bit pattern (exponent<<mbits | fraction), all-ones exponent with
 * zero fraction for overflow.  Uses rint() in the default rounding mode:
 * round to nearest, ties to even.  Scaling by powers of two is exact in
 * binary64, so the single rint() is the only rounding. */
static uint32_t round_to_small_float(double a, int mbits, int bias, int emax_biased) {
    int emin = 1 - bias;                           /* exponent of the smallest normal */
    if (a < ldexp(1.0, emin)) {                    /* subnormal range: units of 2^(emin-mbits) */
        double r = rint(ldexp(a, mbits - emin));
        return (uint32_t)r;                        /* r == 2^mbits is the smallest normal */
    }
    int E;
    frexp(a, &E);                                  /* a = f*2^E, f in [0.5,1) -> exponent E-1 */
    int e = E - 1;
    double r = rint(ldexp(a, mbits - e));          /* in [2^mbits, 2^(mbits+1)] */
    if (r == ldexp(1.0, mbits + 1)) {
        r = ldexp(1.0, mbits);
        e += 1;
    }
    int be = e + bias;
    if (be > emax_biased) return (uint32_t)(emax_biased + 1) << mbits;   /* infinity */
    return ((uint32_t)be << mbits) | (uint32_t)(r - ldexp(1.0, mbits));
}

uint16_t orc_d2h(double x) {
    if (isnan(x)) return 0x7e00;
    uint16_t s = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a)) return s | 0x7c00;
    return s | (uint16_t)round_to_small_float(a, 10, 15, 30);
}

/* OCP fp8 E5M2: 1 sign, 5 exponent bits (bias 15), 2 fraction bits; inf and
 * NaN like binary16.  Its range is +-57344, the figure the xAI latency page
 * gives for E5M2 (§4.3).  The cache stores the unscaled binary16 value
 * rounded to the nearest E5M2 value (ties to even), overflowing to inf. */
uint8_t orc_e5m2_from_h(uint16_t h) {
    uint8_t s = (h & 0x8000) ? 0x80 : 0;
    if ((h & 0x7c00) == 0x7c00) return (h & 0x3ff) ? (uint8_t)(s | 0x7e) : (uint8_t)(s | 0x7c);
    double a = fabs(orc_h2d(h));
    return s | (uint8_t)round_to_small_float(a, 2, 15, 30);
}

uint16_t orc_h_from_e5m2(uint8_t e) {
    /* E5M2 has the exponent field of binary16 and the top 2 of its 10
     * fraction bits: the value is the binary16 with those bits, zero below. */
    int s = e >> 7, ex = (e >> 2) & 0x1f, f = e & 3;
    double v;
    if (ex == 0)
        v = ldexp((double)f, -16);
    else if (ex == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(4 + f), ex - 17);
    if (isnan(v)) return s ? 0xfe00 : 0x7e00;
    return orc_d2h(s ? -v : v);
}

void orc_h2d_n(const uint16_t* h, size_t n, double* out) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_h2d(h[i]);
}
void orc_d2h_n(const double* x, size_t n, uint16_t* out) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_d2h(x[i]);
}
void orc_e5m2_from_h_n(const uint16_t* h, size_t n, uint8_t* out) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_e5m2_from_h(h[i]);
}
void orc_h_from_e5m2_n(const uint8_t* e, size_t n, uint16_t* out) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_h_from_e5m2(e[i]);
}

/* ------------------------------------------------------------------------ */
/* Segment quantization ("Grok-3 v3.2.4 hot update", §3.2), binary32 only.   */

void orc_seg_quant(const uint16_t* x, int n, uint8_t* codes, float* scale_out, float* zp_out) {
    float mn = INFINITY, mx = -INFINITY;
    for (int i = 0; i < n; ++i) {
        float v = (float)orc_h2d(x[i]);            /* binary16 -> binary32 is exact */
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    float scale = (mx - mn) / 255.0f;
    /* The page's formula gives scale 0 for a segment whose values are all
     * equal.  Then the value itself (its magnitude) is the unit: zp becomes
     * -1, 0 or +1, every code is 0 and (0 - zp) * scale returns the value
     * exactly.  An all-zero segment takes scale 1. */
    if (!(scale > 0.0f)) scale = mn != 0.0f ? fabsf(mn) : 1.0f;
    float zp = rintf(-mn / scale);
    for (int i = 0; i < n; ++i) {
        float v = (float)orc_h2d(x[i]);
        float q = rintf(v / scale) + zp;
        if (q < 0.0f) q = 0.0f;
        if (q > 255.0f) q = 255.0f;
        codes[i] = (uint8_t)q;
    }
    *scale_out = scale;
    *zp_out = zp;
}

float orc_seg_dequant(uint8_t code, float scale, float zp) { return ((float)code - zp) * scale; }

/* ------------------------------------------------------------------------ */
/* Delta quantization ("Grok-3 v3.2.4 hot update deep dive", §3.2: the       */
/* scheme before the adaptive-range one stores the difference between       */
/* adjacent tokens' K/V values instead of the values, then quantizes the     */
/* differences to INT8).  Reading taken where the page is silent: a segment  */
/* of n rows of hd fp16 values keeps its first row as it is (the anchor);    */
/* the differences d[p][j] = x[p][j] - x[p-1][j] (p = 1..n-1) of the exact   */
/* values are taken in binary32 and quantized together as one segment with   */
/* the adaptive-range quantizer of the same section (orc_seg_quant's         */
/* formula, on binary32 inputs); a row is restored by adding the             */
/* dequantized differences in row order, so quantization errors add up      */
/* along the segment.  Binary32 throughout.                                 */

void orc_delta_seal(const uint16_t* x, int n, int hd, uint16_t* anchor, uint8_t* codes, float* scale_out,
                    float* zp_out) {
    for (int j = 0; j < hd; ++j) anchor[j] = x[j];
    const int m = (n - 1) * hd;
    if (m <= 0) {   /* one row: no differences */
        *scale_out = 1.0f;
        *zp_out = 0.0f;
        return;
    }
    float mn = INFINITY, mx = -INFINITY;
    for (int p = 1; p < n; ++p)
        for (int j = 0; j < hd; ++j) {
            float d = (float)orc_h2d(x[p * hd + j]) - (float)orc_h2d(x[(p - 1) * hd + j]);
            if (d < mn) mn = d;
            if (d > mx) mx = d;
        }
    float scale = (mx - mn) / 255.0f;
    if (!(scale > 0.0f)) scale = mn != 0.0f ? fabsf(mn) : 1.0f;   /* as orc_seg_quant */
    float zp = rintf(-mn / scale);
    for (int p = 1; p < n; ++p)
        for (int j = 0; j < hd; ++j) {
            float d = (float)orc_h2d(x[p * hd + j]) - (float)orc_h2d(x[(p - 1) * hd + j]);
            float q = rintf(d / scale) + zp;
            if (q < 0.0f) q = 0.0f;
            if (q > 255.0f) q = 255.0f;
            codes[(p - 1) * hd + j] = (uint8_t)q;
        }
    *scale_out = scale;
    *zp_out = zp;
}

void orc_delta_restore(const uint16_t* anchor, const uint8_t* codes, int n, int hd, float scale, float zp,
                       float* y) {
    for (int j = 0; j < hd; ++j) y[j] = (float)orc_h2d(anchor[j]);
    for (int p = 1; p < n; ++p)
        for (int j = 0; j < hd; ++j) {
            float t = ((float)codes[(p - 1) * hd + j] - zp) * scale;
            y[p * hd + j] = y[(p - 1) * hd + j] + t;
        }
}

void orc_seg_dequant_n(const uint8_t* codes, size_t n, float scale, float zp, float* out) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_seg_dequant(codes[i], scale, zp);
}

/* ------------------------------------------------------------------------ */
/* Weight-only INT4, groups of 128 columns, fp32 scales                      */
/* The rebuild page (section 5.2) dequantizes an INT4 weight as
 * int4_value * scale with the scale in fp32 and rounds the product to fp16
 * (round to nearest) before use; its quantizer is not given.  Here: per
 * (row, group of 128 columns) the symmetric scale amax / 7 in fp32 (1 when
 * the group is all zeros), codes rint(w / scale) clamped to [-8, 7], stored
 * as 4-bit two's complement, column 2j in the low nibble of byte j.         */

void orc_q4_quant(const uint16_t* W, int n, int k, uint8_t* codes, float* scales) {
    const int ng = k / ORC_Q4_GROUP;
    for (int r = 0; r < n; ++r)
        for (int g = 0; g < ng; ++g) {
            const uint16_t* w = W + (size_t)r * k + (size_t)g * ORC_Q4_GROUP;
            float amax = 0.0f;
            for (int i = 0; i < ORC_Q4_GROUP; ++i) {
                const float a = fabsf((float)orc_h2d(w[i]));
                if (a > amax) amax = a;
            }
            float scale = amax / 7.0f;
            if (!(scale > 0.0f)) scale = 1.0f;
            scales[(size_t)r * ng + g] = scale;
            for (int i = 0; i < ORC_Q4_GROUP; i += 2) {
                int q[2];
                for (int h = 0; h < 2; ++h) {
                    float v = rintf((float)orc_h2d(w[i + h]) / scale);
                    if (v < -8.0f) v = -8.0f;
                    if (v > 7.0f) v = 7.0f;
                    q[h] = (int)v;
                }
                codes[((size_t)r * k + (size_t)g * ORC_Q4_GROUP + i) / 2] = (uint8_t)((q[0] & 15) | ((q[1] & 15) << 4));
            }
        }
}

int orc_q4_code(const uint8_t* codes, size_t idx) {
    const int nib = (codes[idx / 2] >> ((idx & 1) * 4)) & 15;
    return nib >= 8 ? nib - 16 : nib;
}

void orc_q4_dequant(const uint8_t* codes, const float* scales, int n, int k, uint16_t* out) {
    const int ng = k / ORC_Q4_GROUP;
    for (int r = 0; r < n; ++r)
        for (int c = 0; c < k; ++c) {
            const float prod = (float)orc_q4_code(codes, (size_t)r * k + c) * scales[(size_t)r * ng + c / ORC_Q4_GROUP];
            out[(size_t)r * k + c] = orc_d2h((double)prod);
        }
}

/* ------------------------------------------------------------------------ */
/* Building blocks                                                           */

static double g_h2d_tab[65536];
static int g_tab_ready = 0;

static void build_tab(void) {
    if (g_tab_ready) return;
    for (int i = 0; i < 65536; ++i) g_h2d_tab[i] = orc_h2d((uint16_t)i);
    g_tab_ready = 1;
}

void orc_rmsnorm(const double* x, const uint16_t* gain, int d, double eps, double* out) {
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / d + eps);
    for (int i = 0; i < d; ++i) out[i] = x[i] * inv * orc_h2d(gain[i]);
}

void orc_rope(double* v, int hd, int pos, double base) {
    int h2 = hd / 2;
    for (int j = 0; j < h2; ++j) {
        double theta = pow(base, -2.0 * j / hd);
        double a = (double)pos * theta;
        double c = cos(a), s = sin(a);
        double x0 = v[j], x1 = v[j + h2];
        v[j] = x0 * c - x1 * s;
        v[j + h2] = x0 * s + x1 * c;
    }
}

void orc_gemv(const uint16_t* W, const double* x, int n, int k, double* y) {
    build_tab();
#pragma omp parallel for schedule(static)
    for (int r = 0; r < n; ++r) {
        const uint16_t* w = W + (size_t)r * k;
        double acc = 0.0;
        for (int c = 0; c < k; ++c) acc += g_h2d_tab[w[c]] * x[c];
        y[r] = acc;
    }
}

void orc_attention(const double* q, const double* K, const double* V, int L, int hd, double* out) {
    double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double scale = 1.0 / sqrt((double)hd);
    double m = -INFINITY;
    for (int i = 0; i < L; ++i) {
        double d = 0.0;
        for (int j = 0; j < hd; ++j) d += q[j] * K[(size_t)i * hd + j];
        s[i] = d * scale;
        if (s[i] > m) m = s[i];
    }
    double l = 0.0;
    for (int i = 0; i < L; ++i) {
        s[i] = exp(s[i] - m);
        l += s[i];
    }
    for (int j = 0; j < hd; ++j) out[j] = 0.0;
    for (int i = 0; i < L; ++i)
        for (int j = 0; j < hd; ++j) out[j] += s[i] * V[(size_t)i * hd + j];
    for (int j = 0; j < hd; ++j) out[j] /= l;
    free(s);
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

int orc_argmax(const double* v, int n) {
    int best = 0;
    for (int i = 1; i < n; ++i)
        if (v[i] > v[best]) best = i;              /* strict: the first maximum wins */
    return best;
}

/* ------------------------------------------------------------------------ */
/* Model                                                                     */

typedef struct {
    const uint16_t *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *wg, *wu, *wd;
} orc_layer;

struct orc_model {
    int L, D, H, Hk, hd, F, V;
    double base, eps;
    uint8_t* blob;
    const uint16_t *embed, *final_norm, *lm_head;
    orc_layer* layer;
    int max_ctx, batch, fmt;
    int store;         /* 0: a step keeps the row already at its position (see orc_set_store) */
    double* computed;  /* optional [lane][max_ctx][hd]: the K/V rows the steps computed (orc_record_rows) */
    int* pos;
    void* kv;          /* [b][layer][which][head][max_ctx][hd] of the format's element */
    uint16_t* stage;   /* INT8: [b][layer][which][head][128][hd] open segment */
    float* meta;       /* INT8: [b][layer][which][head][n_seg][2] (scale, zp) */
    int n_seg;
};

static size_t lane_index(const orc_model* m, int b, int layer, int which, int head) {
    return (((size_t)b * m->L + layer) * 2 + which) * m->Hk + head;
}

static size_t kv_elem_size(int fmt) {
    switch (fmt) {
        case ORC_KV_FP16: return 2;
        case ORC_KV_E5M2: return 1;
        case ORC_KV_INT8_SEG128: return 1;
        default: return 8;
    }
}

static uint32_t rd_u32(const uint8_t* p) { uint32_t v; memcpy(&v, p, 4); return v; }
static int32_t rd_i32(const uint8_t* p) { int32_t v; memcpy(&v, p, 4); return v; }
static float rd_f32(const uint8_t* p) { float v; memcpy(&v, p, 4); return v; }

orc_model* orc_create(const void* blob_v, size_t bytes, int max_ctx, int batch, int kv_format) {
    const uint8_t* blob = (const uint8_t*)blob_v;
    build_tab();
    if (!blob || bytes < 256) { set_err("blob too small"); return NULL; }
    if (memcmp(blob, "RDW1", 4) != 0) { set_err("bad magic"); return NULL; }
    if (rd_u32(blob + 4) != 1 || rd_u32(blob + 8) != 256 || rd_u32(blob + 12) != 1 || rd_u32(blob + 52) != 0) {
        set_err("unsupported version/header/dtype/flags");
        return NULL;
    }
    if (max_ctx <= 0 || batch <= 0 || kv_format < 0 || kv_format > 3) { set_err("bad options"); return NULL; }
    int L = rd_i32(blob + 16), D = rd_i32(blob + 20), H = rd_i32(blob + 24), Hk = rd_i32(blob + 28);
    int hd = rd_i32(blob + 32), F = rd_i32(blob + 36), V = rd_i32(blob + 40);
    if (L <= 0 || D <= 0 || H <= 0 || Hk <= 0 || hd <= 0 || F <= 0 || V <= 0 || H % Hk || hd % 2) {
        set_err("bad dimensions");
        return NULL;
    }
    /* walk the tensor list in blob order */
    size_t off = 256;
    size_t sizes_per_layer[9] = {(size_t)D, (size_t)H * hd * D, (size_t)Hk * hd * D, (size_t)Hk * hd * D,
                                 (size_t)D * H * hd, (size_t)D, (size_t)F * D, (size_t)F * D, (size_t)D * F};
    size_t n_t = 1 + 9 * (size_t)L + 2;
    size_t* offs = (size_t*)malloc(sizeof(size_t) * n_t);
    size_t t = 0;
#define TAKE(nelem)                        \
    do {                                   \
        off = (off + 255) / 256 * 256;     \
        offs[t++] = off;                   \
        off += (size_t)(nelem) * 2;        \
    } while (0)
    TAKE((size_t)V * D);
    for (int l = 0; l < L; ++l)
        for (int i = 0; i < 9; ++i) TAKE(sizes_per_layer[i]);
    TAKE(D);
    TAKE((size_t)V * D);
#undef TAKE
    if (off != bytes) {
        free(offs);
        set_err("blob size %zu, expected %zu", bytes, off);
        return NULL;
    }
    orc_model* m = (orc_model*)calloc(1, sizeof *m);
    m->L = L; m->D = D; m->H = H; m->Hk = Hk; m->hd = hd; m->F = F; m->V = V;
    m->base = rd_f32(blob + 44);
    m->eps = rd_f32(blob + 48);
    m->blob = (uint8_t*)malloc(bytes);
    memcpy(m->blob, blob, bytes);
    const uint16_t* T = (const uint16_t*)m->blob;
#define P(i) (T + offs[i] / 2)
    m->embed = P(0);
    m->layer = (orc_layer*)calloc((size_t)L, sizeof(orc_layer));
    for (int l = 0; l < L; ++l) {
        size_t b0 = 1 + 9 * (size_t)l;
        orc_layer* y = &m->layer[l];
        y->attn_norm = P(b0 + 0); y->wq = P(b0 + 1); y->wk = P(b0 + 2); y->wv = P(b0 + 3);
        y->wo = P(b0 + 4); y->ffn_norm = P(b0 + 5); y->wg = P(b0 + 6); y->wu = P(b0 + 7); y->wd = P(b0 + 8);
    }
    m->final_norm = P(n_t - 2);
    m->lm_head = P(n_t - 1);
#undef P
    free(offs);
    m->max_ctx = max_ctx;
    m->batch = batch;
    m->fmt = kv_format;
    m->store = 1;
    m->pos = (int*)calloc((size_t)batch, sizeof(int));
    size_t lanes = (size_t)batch * L * 2 * Hk;
    m->kv = calloc(lanes * (size_t)max_ctx * hd, kv_elem_size(kv_format));
    if (!m->kv) { set_err("out of host memory for the KV cache"); orc_destroy(m); return NULL; }
    if (kv_format == ORC_KV_INT8_SEG128) {
        m->n_seg = (max_ctx + ORC_SEG - 1) / ORC_SEG;
        m->stage = (uint16_t*)calloc(lanes * ORC_SEG * hd, sizeof(uint16_t));
        m->meta = (float*)calloc(lanes * (size_t)m->n_seg * 2, sizeof(float));
    }
    return m;
}

void orc_destroy(orc_model* m) {
    if (!m) return;
    free(m->blob); free(m->layer); free(m->pos); free(m->kv); free(m->stage); free(m->meta); free(m->computed);
    free(m);
}

void orc_reset(orc_model* m) {
    for (int b = 0; b < m->batch; ++b) m->pos[b] = 0;
}

int orc_pos(const orc_model* m, int b) { return m->pos[b]; }

void orc_dims(const orc_model* m, int* o) {
    o[0] = m->L; o[1] = m->D; o[2] = m->H; o[3] = m->Hk; o[4] = m->hd; o[5] = m->F; o[6] = m->V;
}

void orc_set_store(orc_model* m, int store) { m->store = store != 0; }

int orc_record_rows(orc_model* m, int on) {
    free(m->computed);
    m->computed = NULL;
    if (!on) return 0;
    m->computed = (double*)calloc((size_t)m->batch * m->L * 2 * m->Hk * (size_t)m->max_ctx * m->hd, sizeof(double));
    return m->computed ? 0 : -1;
}

static int rows_region_ok(const orc_model* m, int b, int layer, int which, int head, int pos0, int n);

int orc_get_computed(const orc_model* m, int b, int layer, int which, int head, int pos0, int n, double* dst) {
    if (!m->computed || !rows_region_ok(m, b, layer, which, head, pos0, n)) return -1;
    const size_t lane = lane_index(m, b, layer, which, head);
    memcpy(dst, m->computed + (lane * m->max_ctx + pos0) * m->hd, sizeof(double) * (size_t)n * m->hd);
    return 0;
}

/* The computed (unrounded) K/V rows of one position into the record. */
static void record_rows(orc_model* m, int b, int layer, int pos, const double* k, const double* v) {
    if (!m->computed) return;
    for (int which = 0; which < 2; ++which)
        for (int g = 0; g < m->Hk; ++g)
            memcpy(m->computed + (lane_index(m, b, layer, which, g) * m->max_ctx + pos) * m->hd,
                   (which ? v : k) + (size_t)g * m->hd, sizeof(double) * m->hd);
}

int orc_set_pos(orc_model* m, int b, int pos) {
    if (b < 0 || b >= m->batch || pos < 0 || pos > m->max_ctx) return -1;
    m->pos[b] = pos;
    return 0;
}

/* Start of the segment that is still open (not yet quantized) at `pos`. */
static int open_seg_start(int pos) { return pos / ORC_SEG * ORC_SEG; }

static void store_row(orc_model* m, int b, int layer, int which, int head, int pos, const double* v) {
    size_t lane = lane_index(m, b, layer, which, head);
    size_t base = (lane * m->max_ctx + pos) * m->hd;
    for (int j = 0; j < m->hd; ++j) {
        switch (m->fmt) {
            case ORC_KV_FP16: ((uint16_t*)m->kv)[base + j] = orc_d2h(v[j]); break;
            case ORC_KV_E5M2: ((uint8_t*)m->kv)[base + j] = orc_e5m2_from_h(orc_d2h(v[j])); break;
            case ORC_KV_INT8_SEG128:
                m->stage[(lane * ORC_SEG + pos % ORC_SEG) * m->hd + j] = orc_d2h(v[j]);
                break;
            default: ((double*)m->kv)[base + j] = v[j]; break;
        }
    }
}

int orc_read_row(const orc_model* m, int b, int layer, int which, int head, int pos, double* dst) {
    if (b < 0 || b >= m->batch || layer < 0 || layer >= m->L || which < 0 || which > 1 || head < 0 ||
        head >= m->Hk || pos < 0 || pos >= m->max_ctx)
        return -1;
    size_t lane = lane_index(m, b, layer, which, head);
    size_t base = (lane * m->max_ctx + pos) * m->hd;
    for (int j = 0; j < m->hd; ++j) {
        switch (m->fmt) {
            case ORC_KV_FP16: dst[j] = orc_h2d(((const uint16_t*)m->kv)[base + j]); break;
            case ORC_KV_E5M2: dst[j] = orc_h2d(orc_h_from_e5m2(((const uint8_t*)m->kv)[base + j])); break;
            case ORC_KV_INT8_SEG128:
                if (pos < open_seg_start(m->pos[b])) {
                    const float* mt = m->meta + (lane * m->n_seg + pos / ORC_SEG) * 2;
                    dst[j] = (double)orc_seg_dequant(((const uint8_t*)m->kv)[base + j], mt[0], mt[1]);
                } else {
                    dst[j] = orc_h2d(m->stage[(lane * ORC_SEG + pos % ORC_SEG) * m->hd + j]);
                }
                break;
            default: dst[j] = ((const double*)m->kv)[base + j]; break;
        }
    }
    return 0;
}

static int rows_region_ok(const orc_model* m, int b, int layer, int which, int head, int pos0, int n) {
    return b >= 0 && b < m->batch && layer >= 0 && layer < m->L && which >= 0 && which <= 1 && head >= 0 &&
           head < m->Hk && pos0 >= 0 && n >= 0 && pos0 + n <= m->max_ctx;
}

static int rows_copy(orc_model* m, int b, int layer, int which, int head, int pos0, int n, void* buf, int set) {
    if (!rows_region_ok(m, b, layer, which, head, pos0, n)) return -1;
    size_t lane = lane_index(m, b, layer, which, head);
    size_t hd = (size_t)m->hd;
    if (m->fmt == ORC_KV_INT8_SEG128) {
        int open = open_seg_start(m->pos[b]);
        if (pos0 + n <= open) {                            /* sealed codes */
            uint8_t* p = (uint8_t*)m->kv + (lane * m->max_ctx + pos0) * hd;
            if (set) memcpy(p, buf, n * hd); else memcpy(buf, p, n * hd);
            return 0;
        }
        if (pos0 >= open && pos0 + n <= open + ORC_SEG) {  /* open-segment staging */
            uint16_t* p = m->stage + (lane * ORC_SEG + (pos0 - open)) * hd;
            if (set) memcpy(p, buf, n * hd * 2); else memcpy(buf, p, n * hd * 2);
            return 0;
        }
        return -1;
    }
    size_t es = kv_elem_size(m->fmt);
    uint8_t* p = (uint8_t*)m->kv + (lane * m->max_ctx + pos0) * hd * es;
    if (set) memcpy(p, buf, n * hd * es); else memcpy(buf, p, n * hd * es);
    return 0;
}

int orc_get_rows(const orc_model* m, int b, int layer, int which, int head, int pos0, int n, void* dst) {
    return rows_copy((orc_model*)m, b, layer, which, head, pos0, n, dst, 0);
}

int orc_set_rows(orc_model* m, int b, int layer, int which, int head, int pos0, int n, const void* src) {
    return rows_copy(m, b, layer, which, head, pos0, n, (void*)src, 1);
}

int orc_seg_meta(orc_model* m, int b, int layer, int which, int head, int seg, float* scale, float* zp, int set) {
    if (m->fmt != ORC_KV_INT8_SEG128 || !rows_region_ok(m, b, layer, which, head, 0, 0) || seg < 0 ||
        seg >= m->n_seg)
        return -1;
    float* mt = m->meta + (lane_index(m, b, layer, which, head) * m->n_seg + seg) * 2;
    if (set) { mt[0] = *scale; mt[1] = *zp; } else { *scale = mt[0]; *zp = mt[1]; }
    return 0;
}

void orc_layer0_kv(const orc_model* m, int32_t token, int pos, double* k, double* v) {
    int D = m->D, kvd = m->Hk * m->hd;
    double* x = (double*)malloc(sizeof(double) * D);
    double* r = (double*)malloc(sizeof(double) * D);
    for (int i = 0; i < D; ++i) x[i] = orc_h2d(m->embed[(size_t)token * D + i]);
    orc_rmsnorm(x, m->layer[0].attn_norm, D, m->eps, r);
    orc_gemv(m->layer[0].wk, r, kvd, D, k);
    orc_gemv(m->layer[0].wv, r, kvd, D, v);
    for (int g = 0; g < m->Hk; ++g) orc_rope(k + (size_t)g * m->hd, m->hd, pos, m->base);
    free(x);
    free(r);
}

/* Quantize the open segment of every (layer, K/V, head) of sequence b, once
 * it holds 128 rows ("Grok-3 v3.2.4 hot update", §3.2: one scale and zero
 * point per 128-token segment; here per head, as the cache is per head). */
static void seal_segment(orc_model* m, int b, int seg) {
    size_t hd = (size_t)m->hd;
    for (int l = 0; l < m->L; ++l)
        for (int w = 0; w < 2; ++w)
            for (int g = 0; g < m->Hk; ++g) {
                size_t lane = lane_index(m, b, l, w, g);
                uint8_t* codes = (uint8_t*)m->kv + (lane * m->max_ctx + (size_t)seg * ORC_SEG) * hd;
                float* mt = m->meta + (lane * m->n_seg + seg) * 2;
                orc_seg_quant(m->stage + lane * ORC_SEG * hd, (int)(ORC_SEG * hd), codes, &mt[0], &mt[1]);
            }
}

int orc_step(orc_model* m, const int32_t* tokens, double* logits, int32_t* next) {
    int D = m->D, H = m->H, Hk = m->Hk, hd = m->hd, F = m->F, V = m->V, G = H / Hk;
    for (int b = 0; b < m->batch; ++b) {
        if (m->pos[b] >= m->max_ctx) { set_err("context full"); return -1; }
        if (tokens[b] < 0 || tokens[b] >= V) { set_err("token out of range"); return -1; }
    }
    double* x = (double*)malloc(sizeof(double) * D);
    double* r = (double*)malloc(sizeof(double) * D);
    double* q = (double*)malloc(sizeof(double) * H * hd);
    double* k = (double*)malloc(sizeof(double) * Hk * hd);
    double* v = (double*)malloc(sizeof(double) * Hk * hd);
    double* a = (double*)malloc(sizeof(double) * H * hd);
    double* o = (double*)malloc(sizeof(double) * D);
    double* gt = (double*)malloc(sizeof(double) * F);
    double* up = (double*)malloc(sizeof(double) * F);
    double* lg = (double*)malloc(sizeof(double) * V);

    for (int b = 0; b < m->batch; ++b) {
        int pos = m->pos[b], L = pos + 1;
        for (int i = 0; i < D; ++i) x[i] = orc_h2d(m->embed[(size_t)tokens[b] * D + i]);
        for (int l = 0; l < m->L; ++l) {
            const orc_layer* y = &m->layer[l];
            orc_rmsnorm(x, y->attn_norm, D, m->eps, r);
            orc_gemv(y->wq, r, H * hd, D, q);
            orc_gemv(y->wk, r, Hk * hd, D, k);
            orc_gemv(y->wv, r, Hk * hd, D, v);
            for (int h = 0; h < H; ++h) orc_rope(q + (size_t)h * hd, hd, pos, m->base);
            for (int g = 0; g < Hk; ++g) orc_rope(k + (size_t)g * hd, hd, pos, m->base);
            record_rows(m, b, l, pos, k, v);
            if (m->store)
                for (int g = 0; g < Hk; ++g) {
                    store_row(m, b, l, 0, g, pos, k + (size_t)g * hd);
                    store_row(m, b, l, 1, g, pos, v + (size_t)g * hd);
                }
            /* attention: query head h reads kv head h / G */
#pragma omp parallel for schedule(dynamic, 1)
            for (int g = 0; g < Hk; ++g) {
                double* Kd = (double*)malloc(sizeof(double) * (size_t)L * hd);
                double* Vd = (double*)malloc(sizeof(double) * (size_t)L * hd);
                for (int p = 0; p < L; ++p) {
                    orc_read_row(m, b, l, 0, g, p, Kd + (size_t)p * hd);
                    orc_read_row(m, b, l, 1, g, p, Vd + (size_t)p * hd);
                }
                for (int h = g * G; h < (g + 1) * G; ++h)
                    orc_attention(q + (size_t)h * hd, Kd, Vd, L, hd, a + (size_t)h * hd);
                free(Kd);
                free(Vd);
            }
            orc_gemv(y->wo, a, D, H * hd, o);
            for (int i = 0; i < D; ++i) x[i] += o[i];
            orc_rmsnorm(x, y->ffn_norm, D, m->eps, r);
            orc_gemv(y->wg, r, F, D, gt);
            orc_gemv(y->wu, r, F, D, up);
            for (int i = 0; i < F; ++i) gt[i] = orc_silu(gt[i]) * up[i];
            orc_gemv(y->wd, gt, D, F, o);
            for (int i = 0; i < D; ++i) x[i] += o[i];
        }
        orc_rmsnorm(x, m->final_norm, D, m->eps, r);
        orc_gemv(m->lm_head, r, V, D, lg);
        if (logits) memcpy(logits + (size_t)b * V, lg, sizeof(double) * V);
        if (next) next[b] = orc_argmax(lg, V);
        if (m->store && m->fmt == ORC_KV_INT8_SEG128 && (pos + 1) % ORC_SEG == 0) seal_segment(m, b, pos / ORC_SEG);
        m->pos[b] = pos + 1;
    }
    free(x); free(r); free(q); free(k); free(v); free(a); free(o); free(gt); free(up); free(lg);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Blocked prefill: the decode steps of a prompt, loop-interchanged          */

/* y[t*n + r] = W[r] . x_t for the nt tokens of a block, x held transposed
 * (xt[c*nt + t]).  Each token's sum runs over the columns in order, exactly
 * as orc_gemv's; only the loops are interchanged, so that a weight row is
 * used for every token while it is in cache. */
static void gemv_block(const uint16_t* W, const double* xt, int n, int k, int nt, double* y) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < n; ++r) {
        double acc[ORC_SEG];
        for (int t = 0; t < nt; ++t) acc[t] = 0.0;
        const uint16_t* w = W + (size_t)r * k;
        for (int c = 0; c < k; ++c) {
            const double wc = g_h2d_tab[w[c]];
            const double* xc = xt + (size_t)c * nt;
            for (int t = 0; t < nt; ++t) acc[t] += wc * xc[t];
        }
        for (int t = 0; t < nt; ++t) y[(size_t)t * n + r] = acc[t];
    }
}

static void transpose_block(const double* x, int nt, int k, double* xt) {
    for (int t = 0; t < nt; ++t)
        for (int c = 0; c < k; ++c) xt[(size_t)c * nt + t] = x[(size_t)t * k + c];
}

int orc_prefill(orc_model* m, const int32_t* tokens, int n) {
    if (m->batch != 1) { set_err("prefill: batch-1 models only"); return -1; }
    if (n < 0 || m->pos[0] + n > m->max_ctx) { set_err("prefill: tokens do not fit the context"); return -1; }
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= m->V) { set_err("token out of range"); return -1; }
    const int D = m->D, H = m->H, Hk = m->Hk, hd = m->hd, F = m->F, G = H / Hk;
    const int kmax = F > D ? (F > H * hd ? F : H * hd) : (D > H * hd ? D : H * hd);
    const int nmax = 2 * F > (H + 2 * Hk) * hd ? 2 * F : (H + 2 * Hk) * hd;
    double* x = (double*)malloc(sizeof(double) * ORC_SEG * D);
    double* r = (double*)malloc(sizeof(double) * ORC_SEG * kmax);
    double* xt = (double*)malloc(sizeof(double) * ORC_SEG * kmax);
    double* y = (double*)malloc(sizeof(double) * ORC_SEG * (size_t)nmax);
    double* q = (double*)malloc(sizeof(double) * ORC_SEG * H * hd);
    double* a = (double*)malloc(sizeof(double) * ORC_SEG * H * hd);
    int done = 0;
    while (done < n) {
        /* a block never crosses a 128-position boundary: all of its rows
         * belong to one INT8 segment, which is sealed after the block */
        const int p0 = m->pos[0];
        int nt = ORC_SEG - p0 % ORC_SEG;
        if (nt > n - done) nt = n - done;
        for (int t = 0; t < nt; ++t)
            for (int i = 0; i < D; ++i) x[(size_t)t * D + i] = orc_h2d(m->embed[(size_t)tokens[done + t] * D + i]);
        for (int l = 0; l < m->L; ++l) {
            const orc_layer* w = &m->layer[l];
            for (int t = 0; t < nt; ++t) orc_rmsnorm(x + (size_t)t * D, w->attn_norm, D, m->eps, r + (size_t)t * D);
            transpose_block(r, nt, D, xt);
            const int Nq = H * hd, Nk = Hk * hd;
            gemv_block(w->wq, xt, Nq, D, nt, q);
            gemv_block(w->wk, xt, Nk, D, nt, y);
            gemv_block(w->wv, xt, Nk, D, nt, y + (size_t)nt * Nk);
            for (int t = 0; t < nt; ++t) {
                const int pos = p0 + t;
                double* kt = y + (size_t)t * Nk;
                double* vt = y + (size_t)nt * Nk + (size_t)t * Nk;
                for (int h = 0; h < H; ++h) orc_rope(q + (size_t)t * Nq + (size_t)h * hd, hd, pos, m->base);
                for (int g = 0; g < Hk; ++g) orc_rope(kt + (size_t)g * hd, hd, pos, m->base);
                record_rows(m, 0, l, pos, kt, vt);
                if (m->store)
                    for (int g = 0; g < Hk; ++g) {
                        store_row(m, 0, l, 0, g, pos, kt + (size_t)g * hd);
                        store_row(m, 0, l, 1, g, pos, vt + (size_t)g * hd);
                    }
            }
            /* token t attends to positions 0..p0+t as stored */
#pragma omp parallel for schedule(dynamic, 1)
            for (int tg = 0; tg < nt * Hk; ++tg) {
                const int t = tg / Hk, g = tg % Hk, L = p0 + t + 1;
                double* Kd = (double*)malloc(sizeof(double) * (size_t)L * hd);
                double* Vd = (double*)malloc(sizeof(double) * (size_t)L * hd);
                for (int p = 0; p < L; ++p) {
                    orc_read_row(m, 0, l, 0, g, p, Kd + (size_t)p * hd);
                    orc_read_row(m, 0, l, 1, g, p, Vd + (size_t)p * hd);
                }
                for (int h = g * G; h < (g + 1) * G; ++h)
                    orc_attention(q + (size_t)t * Nq + (size_t)h * hd, Kd, Vd, L, hd, a + (size_t)t * Nq + (size_t)h * hd);
                free(Kd);
                free(Vd);
            }
            transpose_block(a, nt, Nq, xt);
            gemv_block(w->wo, xt, D, Nq, nt, y);
            for (size_t i = 0; i < (size_t)nt * D; ++i) x[i] += y[i];
            for (int t = 0; t < nt; ++t) orc_rmsnorm(x + (size_t)t * D, w->ffn_norm, D, m->eps, r + (size_t)t * D);
            transpose_block(r, nt, D, xt);
            gemv_block(w->wg, xt, F, D, nt, y);
            gemv_block(w->wu, xt, F, D, nt, y + (size_t)nt * F);
            for (int t = 0; t < nt; ++t)
                for (int i = 0; i < F; ++i) {
                    const size_t j = (size_t)t * F + i;
                    r[j] = orc_silu(y[j]) * y[(size_t)nt * F + j];
                }
            transpose_block(r, nt, F, xt);
            gemv_block(w->wd, xt, D, F, nt, y);
            for (size_t i = 0; i < (size_t)nt * D; ++i) x[i] += y[i];
        }
        m->pos[0] = p0 + nt;
        if (m->store && m->fmt == ORC_KV_INT8_SEG128 && (p0 + nt) % ORC_SEG == 0)
            seal_segment(m, 0, (p0 + nt) / ORC_SEG - 1);
        done += nt;
    }
    free(x); free(r); free(xt); free(y); free(q); free(a);
    return 0;
}

