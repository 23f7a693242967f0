/*
 * Oracle for the batch-1 (and batch-B) autoregressive decode step of a dense
 * decoder-only transformer: a plain, slow CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the HIP library.
 *
 * Precision: every floating-point step runs in IEEE binary64, except the
 * rounding points the method itself fixes:
 *   - weights and norm gains are binary16 (the model is an fp16 model);
 *   - K/V rows are rounded to binary16 when stored in the cache (fp16 KV);
 *   - the fp8 E5M2 cache encodes that binary16 value (no scale);
 *   - the per-128-token segment INT8 quantizer computes its scale, zero
 *     point and codes in binary32, the precision the pages prescribe for
 *     quantization scales ("LLM inference architecture rebuild", §5.2: a
 *     binary16 scale lost precision, binary32 fixed it).
 *
 * Parity pins for every function live in the CPU tests; the only parts
 * without an external pin are internal conventions (blob tensor order, which
 * the HIP side reads by the same published layout).
 */
#ifndef RD_ORACLE_H
#define RD_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats ---------------------------------------------------- */
double   orc_h2d(uint16_t h);            /* binary16 -> binary64, exact */
uint16_t orc_d2h(double x);              /* binary64 -> binary16, round-to-nearest-even */
uint8_t  orc_e5m2_from_h(uint16_t h);    /* binary16 -> OCP fp8 E5M2, RNE, overflow -> inf */
uint16_t orc_h_from_e5m2(uint8_t e);     /* E5M2 -> binary16, exact */
/* element-wise array forms of the four conversions above */
void orc_h2d_n(const uint16_t* h, size_t n, double* out);
void orc_d2h_n(const double* x, size_t n, uint16_t* out);
void orc_e5m2_from_h_n(const uint16_t* h, size_t n, uint8_t* out);
void orc_h_from_e5m2_n(const uint8_t* e, size_t n, uint16_t* out);

/* Adaptive-range segment quantization ("Grok-3 v3.2.4 hot update", §3.2):
 * over n binary16 values, min/max -> scale=(max-min)/255,
 * zp=round(-min/scale) (round half to even), code=clamp(round(x/scale)+zp,0,255).
 * All in binary32.  Degenerate max==min uses scale |min| (1 when the
 * segment is all zeros), which reproduces the constant exactly. */
void  orc_seg_quant(const uint16_t* x, int n, uint8_t* codes, float* scale, float* zp);
void  orc_delta_seal(const uint16_t* x, int n, int hd, uint16_t* anchor, uint8_t* codes, float* scale, float* zp);
void  orc_delta_restore(const uint16_t* anchor, const uint8_t* codes, int n, int hd, float scale, float zp, float* y);
float orc_seg_dequant(uint8_t code, float scale, float zp);
void  orc_seg_dequant_n(const uint8_t* codes, size_t n, float scale, float zp, float* out);

/* ---- weight-only INT4 (groups of 128 columns, fp32 scales) ---------------
 * "LLM inference architecture rebuild", §5.2: an INT4 weight is used as
 * fp16(int4_value * scale) with an fp32 scale and round-to-nearest.  The
 * quantizer (not on the pages): per (row, 128-column group) scale =
 * amax / 7 in binary32 (1 for an all-zero group), code = clamp(rint(w /
 * scale), -8, 7), 4-bit two's complement, column 2j in the low nibble of
 * byte j of the row.  k % 128 == 0.  codes: [n][k/2]; scales: [n][k/128]. */
#define ORC_Q4_GROUP 128
void orc_q4_quant(const uint16_t* W, int n, int k, uint8_t* codes, float* scales);
int  orc_q4_code(const uint8_t* codes, size_t idx);     /* signed code of element idx */
/* out (binary16 bits) = fp16(float(code) * scale): binary32 product, then RNE */
void orc_q4_dequant(const uint8_t* codes, const float* scales, int n, int k, uint16_t* out);

/* ---- building blocks (binary64) ----------------------------------------- */
void   orc_rmsnorm(const double* x, const uint16_t* gain, int d, double eps, double* out);
void   orc_rope(double* v, int hd, int pos, double base);      /* in place, pairs (j, j+hd/2) */
void   orc_gemv(const uint16_t* W, const double* x, int n, int k, double* y); /* y = W x */
void   orc_attention(const double* q, const double* K, const double* V, int L, int hd,
                     double* out);                             /* softmax(qK^T/sqrt(hd)) V */
double orc_silu(double z);
int    orc_argmax(const double* v, int n);                    /* lowest index on ties */

/* ---- the model ------------------------------------------------------------ */
enum { ORC_KV_FP16 = 0, ORC_KV_E5M2 = 1, ORC_KV_INT8_SEG128 = 2, ORC_KV_EXACT = 3 };
#define ORC_SEG 128

typedef struct orc_model orc_model;

/* Parses and copies the blob.  Returns NULL on a malformed blob (message in
 * orc_last_error()).  kv_format: ORC_KV_*; ORC_KV_EXACT keeps K/V in binary64
 * (no rounding point at all) and exists only to pin the oracle. */
orc_model*  orc_create(const void* blob, size_t bytes, int max_ctx, int batch, int kv_format);
void        orc_destroy(orc_model* m);
const char* orc_last_error(void);
void        orc_reset(orc_model* m);
int         orc_pos(const orc_model* m, int b);
/* dims: n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ff, vocab */
void        orc_dims(const orc_model* m, int* out7);

/* One decode step for every sequence b in [0,batch): token[b] at the current
 * position, logits [batch*vocab] (may be NULL), next [batch] argmax (may be
 * NULL).  Returns 0, or -1 if a position would pass max_ctx or a token is out
 * of range. */
int orc_step(orc_model* m, const int32_t* tokens, double* logits, int32_t* next);

/* Teacher-forced prompt: tokens[0..n) at positions pos .. pos+n-1 of a
 * batch-1 model, the same decode steps as n calls of orc_step (bit for bit:
 * cache, and every later step) with the loops interchanged: per block of
 * tokens within one 128-position segment, each layer runs for all of the
 * block's tokens (weight rows reused across tokens, each dot product still
 * summed in order), token t attending to positions 0..pos+t as stored; the
 * INT8 seal follows a block that completes a segment.  No logits.  Returns 0,
 * or -1 (batch > 1, context full, token out of range; nothing run). */
int orc_prefill(orc_model* m, const int32_t* tokens, int n);

/* K/V rows of layer 0 for a token at a position, before any cache rounding
 * ([n_kv_heads*head_dim] each, post-RoPE K).  Layer 0 depends on the token
 * alone, so this samples the cache at any position without a prefill. */
void orc_layer0_kv(const orc_model* m, int32_t token, int pos, double* k, double* v);

/* Cache access, for parity checks that feed a cache produced elsewhere.
 * `which` 0 = K, 1 = V.  Rows [pos0, pos0+n) of (b, layer, kv-head):
 *   FP16: uint16 [n*hd]; E5M2: uint8 [n*hd];
 *   INT8_SEG128: rows in sealed segments as uint8 codes, open-segment rows as
 *   uint16 staging (set/get per region; see orc_seg_meta);
 *   EXACT: double [n*hd]. */
int orc_get_rows(const orc_model* m, int b, int layer, int which, int head, int pos0, int n, void* dst);
int orc_set_rows(orc_model* m, int b, int layer, int which, int head, int pos0, int n, const void* src);
int orc_seg_meta(orc_model* m, int b, int layer, int which, int head, int seg, float* scale, float* zp,
                 int set);
/* Dequantized (as-attended) value of one cache row, binary64 [hd]. */
int orc_read_row(const orc_model* m, int b, int layer, int which, int head, int pos, double* dst);
int orc_set_pos(orc_model* m, int b, int pos);
/* store = 0: orc_step and orc_prefill compute the K/V rows of their
 * positions but store nothing in the cache (no row, no INT8 seal);
 * attention reads whatever the cache already holds (set with orc_set_rows
 * and orc_seg_meta).  Tests of the 8-bit formats use it to run steps over
 * the exact stored bytes of another implementation's cache.  Default 1. */
void orc_set_store(orc_model* m, int store);
/* on = 1: from now on every step (orc_step, orc_prefill) also records the
 * K/V rows it computes, before any rounding (binary64, post-RoPE K), for
 * orc_get_computed; on = 0 drops the record.  Returns -1 if out of memory. */
int orc_record_rows(orc_model* m, int on);
int orc_get_computed(const orc_model* m, int b, int layer, int which, int head, int pos0, int n, double* dst);

#ifdef __cplusplus
}
#endif
#endif
