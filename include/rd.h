/*
 * rd.h — C ABI of the MI355X (gfx950) batch-1 decode-step library.
 *
 * The library runs the autoregressive decode step of a dense decoder-only
 * transformer on one GPU: RMSNorm, weight-streaming fp16 GEMVs (fused QKV,
 * output projection, SwiGLU gate/up and down, LM head), RoPE with KV-cache
 * append, single-query attention over the cache split along the key axis
 * with a log-sum-exp merge, and greedy argmax on the device.
 *
 * Sources for what is computed (page titles as printed):
 *  - "Real-time LLM inference on standard GPUs: 3,000 tokens/s per request"
 *    (Kog), section "Memory bandwidth is the main bottleneck ...": at batch 1
 *    every active weight crosses HBM once per token, so
 *    tokens/s <= BW / (beta * weight bytes + KV bytes); section "Where
 *    standard inference stacks lose microseconds": kernel boundaries, CPU
 *    sampling and grid synchronisation are the losses to remove, sampling
 *    stays on the GPU.
 *  - "How the xAI engineering team cut Grok Bot latency to milliseconds",
 *    §2.1 (per-token forward; whole-step graph capture), §2.3 (KV cache in
 *    FP8 E5M2, dequantized to fp16 when read), §3.3 (engine options: model,
 *    device, KV cache dtype, maximum KV length), §4.1 (capture once, replay
 *    with a static input buffer).
 *  - "Grok-3 v3.2.4 hot update deep dive", §3.2: adaptive-range INT8 KV
 *    quantization per 128-token segment, scale=(max-min)/255,
 *    zero_point=round(-min/scale).
 *  - "LLM inference architecture rebuild (state-driven layered design)",
 *    §3.3: kernels called with an explicit softmax scale and returning
 *    errors as values; §5.2: quantization scales kept in fp32.
 *
 * Conventions of every entry point:
 *  - Returns rd_status; RD_OK == 0, errors are negative.  No exception
 *    crosses the ABI and nothing aborts.  rd_last_error() gives a message
 *    for the calling thread's last failure.
 *  - "host" pointers are ordinary CPU memory owned by the caller; "device"
 *    pointers are HIP device memory on the model's (or given) device, owned
 *    by the caller unless said otherwise.
 *  - A model is not thread-safe; distinct models may run on distinct
 *    streams concurrently.
 *  - After an RD_ERR_DEVICE the model is poisoned: every later call on it
 *    returns RD_ERR_DEVICE until rd_model_destroy.
 */
#ifndef RD_H
#define RD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct rd_model rd_model; /* opaque; owns all of its device memory */

typedef enum {
    RD_OK = 0,
    RD_ERR_INVALID_ARG = -1,   /* NULL pointer, size out of range, batch != max_batch, ... */
    RD_ERR_BAD_BLOB = -2,      /* malformed or mis-sized weight blob */
    RD_ERR_OUT_OF_MEMORY = -3, /* device allocation failed */
    RD_ERR_CONTEXT_FULL = -4,  /* position would reach max_context; state unchanged */
    RD_ERR_UNSUPPORTED = -5,   /* valid request the library does not implement */
    RD_ERR_DEVICE = -6,        /* HIP error; the model is poisoned */
    RD_ERR_NUMERIC = -7        /* non-finite logit or out-of-range token seen on the device */
} rd_status;

typedef enum {
    RD_KV_FP16 = 0,        /* K/V rows stored as fp16 */
    RD_KV_FP8_E5M2 = 1,    /* fp16 row rounded to OCP E5M2 (RNE, no scale, overflow -> inf) */
    RD_KV_INT8_SEG128 = 2  /* u8 codes per 128-token segment per (layer, K|V, kv-head) with
                              fp32 scale and zero point; the open segment stays fp16 */
} rd_kv_format;

typedef enum {
    RD_EXEC_AUTO = 0,      /* PERSISTENT where a persistent kernel is built for the model's shape
                              (batch 1; the 2B-class, tiny and small-GQA test shapes with their
                              split counts), otherwise GRAPH */
    RD_EXEC_EAGER = 1,     /* one kernel launch per phase */
    RD_EXEC_GRAPH = 2,     /* the step's launches captured once into a hipGraph, replayed per step */
    RD_EXEC_PERSISTENT = 3 /* one cooperative launch runs a whole run of steps (rd_generate: up to
                              512 per launch); workgroups hand vectors to each other through
                              tagged exchange words instead of grid barriers */
} rd_executor;

typedef struct {
    uint32_t struct_size; /* sizeof(rd_options) */
    int32_t device;       /* HIP device ordinal */
    void* stream;         /* hipStream_t to run on, or NULL for a library-owned stream */
    int32_t max_context;  /* positions per sequence (KV rows allocated), >= 1 */
    int32_t max_batch;    /* independent sequences advancing in lockstep at one position: 1..8.
                           * Batch > 1 runs every GEMV as a thin GEMM on the matrix cores
                           * ("Real-time LLM inference on standard GPUs", section on memory
                           * bandwidth: a weight byte serves every sequence), on the EAGER or
                           * GRAPH executor (PERSISTENT: UNSUPPORTED); needs d_model,
                           * n_heads*head_dim and d_ff multiples of 64, at most 8192. */
    int32_t kv_format;    /* rd_kv_format */
    int32_t executor;     /* rd_executor */
    int32_t attn_splits;  /* maximum key-axis splits per kv-head, 1..256; 0 = default: CUs / kv-heads
                             at batch 1, 2 * CUs / (kv-heads * max_batch) above, within 1..64.
                             Each split covers at least 48 keys.  INT8_SEG128: at least 2 (the
                             open segment is a split of its own; its sealed positions use at most
                             attn_splits - 1).  The persistent kernels merge at most 32
                             (2B-class shape) or 64 (test shapes) splits: with more, AUTO takes
                             GRAPH and PERSISTENT is UNSUPPORTED. */
    int32_t kv_pages;     /* 0: a contiguous cache of max_context rows per sequence.  > 0: a paged
                             cache ("LLM inference architecture rebuild", §3.2: 4 KB pages, a page
                             table per sequence, refcounts, prefix sharing) of this many page
                             groups shared by all sequences.  A page is 4 KiB of one (layer, K/V,
                             kv head): page_rows = 4096 / (head_dim * element bytes) positions; a
                             page group is one page id across all layers, K/V and kv heads.
                             Sequences then sit at their own positions (ragged lengths): a token of
                             -1 in rd_decode_step / rd_prefill sits that sequence out of the step.
                             Needs max_batch 2..8, FP16 or FP8_E5M2, the EAGER or GRAPH executor,
                             and max_context <= 4094 * page_rows. */
} rd_options;

typedef struct {
    int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ff, vocab;
    float rope_base, norm_eps;
    int32_t max_context, max_batch, kv_format, executor, attn_splits;
    uint64_t weight_bytes;      /* device bytes of all weights */
    uint64_t streamed_bytes;    /* weight bytes one step must read (all but the embedding table,
                                   plus one embedding row per sequence) */
    uint64_t kv_bytes;          /* device bytes of the KV cache (all formats' parts) */
    int32_t kv_pages;           /* page groups of a paged cache (0: contiguous) */
    int32_t page_rows;          /* positions per page (0: contiguous) */
} rd_model_info;

/* Initialise an options struct with defaults (device 0, NULL stream,
 * max_context 4096, max_batch 1, fp16 KV, AUTO executor, 0 splits). */
void rd_options_init(rd_options* opt);

/* Create a model from a weight blob ("RDW1"), the engine options of "How
 * the xAI engineering team cut Grok Bot latency to milliseconds", §3.3
 * (model, device, KV cache dtype, maximum KV length): a 256-byte header (magic,
 * version 1, header bytes 256, dtype 1 = fp16, n_layers, d_model, n_heads,
 * n_kv_heads, head_dim, d_ff, vocab as i32, rope_base and norm_eps as f32,
 * flags 0), then fp16 row-major [out,in] tensors on 256-byte boundaries:
 * embed[V,D]; per layer attn_norm[D], wq[H*hd,D], wk[Hk*hd,D], wv[Hk*hd,D],
 * wo[D,H*hd], ffn_norm[D], w_gate[F,D], w_up[F,D], w_down[D,F]; then
 * final_norm[D], lm_head[V,D]; the blob ends there.
 * blob: host, borrowed for the call only (copied and re-tiled).
 * The QKV rows are re-ordered (RoPE pairs adjacent) and the gate/up rows
 * interleaved once, here, into the layout the kernels stream.
 * Errors: INVALID_ARG (NULL, bad options; attn_splits 1 with INT8_SEG128;
 * n_kv_heads * max_context * head_dim * element bytes above 2^31 - 1, the
 * 32-bit offsets of the attention's row loads), BAD_BLOB, UNSUPPORTED (a shape the
 * kernels do not cover: head_dim must be 64 or 128, n_heads / n_kv_heads 1,
 * 2, 4 or 8, d_model and d_ff multiples of 8, d_model <= 4096,
 * n_heads * head_dim <= 4096, d_ff <= 8192; max_batch > 1 with the
 * persistent executor), OUT_OF_MEMORY, DEVICE. */
rd_status rd_model_create(const void* blob, size_t blob_bytes, const rd_options* opt, rd_model** out);

/* Release everything; NULL-safe. */
void rd_model_destroy(rd_model* m);

rd_status rd_model_get_info(const rd_model* m, rd_model_info* out);

/* Position := 0 for every sequence (cache contents become unreachable; a
 * paged cache releases every page). */
rd_status rd_reset(rd_model* m);

/* Position of the next token to be decoded (the same for every sequence;
 * a paged cache: sequence 0's, see rd_seq_position). */
rd_status rd_get_position(const rd_model* m, int32_t* pos);

/* One decode step: the per-token forward of "How the xAI engineering team
 * cut Grok Bot latency to milliseconds", §2.1 (embedding, per layer RMSNorm,
 * QKV, RoPE, attention over the cache, output projection, SwiGLU FFN; final
 * norm, logits), with greedy sampling on the GPU ("Real-time LLM inference
 * on standard GPUs", loss table).  tokens: host [batch] ids at the current position.
 * logits: host [batch*vocab] fp32 or NULL.  next: host [batch] greedy argmax
 * (lowest index on ties) or NULL.  batch must equal max_batch.
 * Paged cache: each sequence decodes at its own position; a token of -1 sits
 * the sequence out (its position and rows unchanged, its next is -1 and its
 * logits meaningless).
 * Errors: INVALID_ARG, CONTEXT_FULL (nothing changed), OUT_OF_MEMORY (paged:
 * the pool is exhausted; nothing changed), NUMERIC (a non-finite logit or an
 * out-of-range token was seen; the step still advanced), DEVICE. */
rd_status rd_decode_step(rd_model* m, const int32_t* tokens, int32_t batch, float* logits, int32_t* next);

/* Teacher-forced steps: tokens (host [n*batch], step-major) are fed at
 * positions pos .. pos+n-1 in order, each through the whole decode step
 * (K/V appended, logits and argmax computed and dropped), the prompt of the
 * decode-with-cache definition.  Runs on the graph path whatever the
 * executor (bit-identical results), enqueues all n steps, then
 * synchronises once.  Errors as rd_decode_step; CONTEXT_FULL (nothing run)
 * if the tokens do not fit; INVALID_ARG (nothing run) for an id out of range. */
rd_status rd_prefill(rd_model* m, const int32_t* tokens, int32_t batch, int32_t n);

/* Batched prefill of sequence 0 (max_batch 1): tokens (host [n]) at
 * positions pos .. pos+n-1, the prompt processed together instead of one
 * decode step per token ("LLM inference architecture rebuild", batch
 * planner: prefill separated from decode; "How the xAI engineering team cut
 * Grok Bot latency to milliseconds", §2.1: block-wise FlashAttention).  It
 * computes what the decode steps would for those positions -- each
 * position's K/V rows, and each position's attention over positions 0..p as
 * stored in the cache format (INT8: segments sealed as they complete) --
 * with the layer products as matrix products on the matrix cores (fp16
 * operands, fp32 sums) in chunks of 2048 tokens, so the cache rows agree
 * with the decode steps' within rounding, not bit for bit.  No logits; the
 * next rd_decode_step continues at pos+n.  Allocates a workspace on the
 * first call (about 100 MB for the 2B-class shape), kept by the model.
 * Synchronises.  Errors: INVALID_ARG (NULL, n < 0, a token out of range;
 * nothing run), CONTEXT_FULL (nothing run), UNSUPPORTED (max_batch > 1, or
 * d_model / d_ff not multiples of 32), OUT_OF_MEMORY, DEVICE. */
rd_status rd_prefill_batched(rd_model* m, const int32_t* tokens, int32_t n);

/* n_steps greedy steps with the token fed back on the device (no host round
 * trip between steps: the whole sequence is decoded without the CPU in the
 * loop, "Real-time LLM inference on standard GPUs", last section).  first: host [batch], the token at the current
 * position.  out_tokens: host [n_steps*batch], step-major: the argmax of
 * every step.  Errors as rd_decode_step; CONTEXT_FULL if the steps do not fit. */
rd_status rd_generate(rd_model* m, const int32_t* first, int32_t batch, int32_t n_steps, int32_t* out_tokens);

/* Same as rd_generate but out_tokens_dev is a device [n_steps*batch] int32
 * buffer and nothing is synchronised: the call only enqueues work on the
 * model's stream (errors found on the device surface at the next
 * synchronising call). */
rd_status rd_generate_async(rd_model* m, const int32_t* first, int32_t batch, int32_t n_steps,
                            int32_t* out_tokens_dev);

/* Wait for the model's stream and report device-side errors. */
rd_status rd_synchronize(rd_model* m);

/* Copy the raw KV storage of (seq < max_batch, layer, which: 0 = K, 1 = V) into host
 * memory dst (capacity cap bytes), in the formats of "How the xAI engineering
 * team cut Grok Bot latency to milliseconds", §2.3 (E5M2) and "Grok-3 v3.2.4
 * hot update deep dive", §3.2 (INT8 per 128-token segment).  Layout per format:
 * A paged cache exports sequence seq's rows gathered through its page table
 * in the FP16 / E5M2 layout below (rows of pages it does not hold: zeros).
 *  FP16:  u16 [n_kv_heads][max_context][head_dim]
 *  E5M2:  u8  [n_kv_heads][max_context][head_dim]
 *  INT8:  u8 codes [n_kv_heads][max_context][head_dim], then
 *         u16 staging [n_kv_heads][128][head_dim] (row = pos % 128), then
 *         f32 meta [n_kv_heads][ceil(max_context/128)][2] (scale, zero point).
 * *written receives the byte count.  Synchronises the stream. */
rd_status rd_debug_export_kv(rd_model* m, int32_t seq, int32_t layer, int32_t which, void* dst, size_t cap,
                             size_t* written);

/* Paged cache (rd_options.kv_pages > 0).  The host keeps each sequence's page
 * table, a refcount per page group and a free list.  Before each step (or run
 * of steps: rd_prefill, rd_generate) every participating sequence gets the
 * pages its new rows need: a missing page from the free list, and a shared
 * page (refcount > 1) that a row is about to be written into is copied first
 * (copy on write).  All or nothing: OUT_OF_MEMORY, with no state changed, when
 * the pool cannot cover the request.  Rows are read through the page table;
 * the results equal the contiguous cache's bit for bit.  The calls below
 * synchronise the model's stream first.  Contiguous models: UNSUPPORTED. */

/* Sequence seq (< max_batch) back to position 0, its pages released. */
rd_status rd_seq_reset(rd_model* m, int32_t seq);

/* Prefix sharing: sequence dst (!= src) takes src's pages of positions
 * 0..pos(src)-1 (refcounts + 1) and src's position; its own pages are
 * released first.  The two then diverge by copy on write. */
rd_status rd_seq_fork(rd_model* m, int32_t src, int32_t dst);

/* Position (rows held) of sequence seq. */
rd_status rd_seq_position(const rd_model* m, int32_t seq, int32_t* pos);

/* Page groups free, in use (refcount > 0) and shared (refcount > 1). */
rd_status rd_kv_page_stats(const rd_model* m, int32_t* free_pages, int32_t* used_pages, int32_t* shared_pages);

/* Overwrite the raw KV storage of (seq, layer, which) from host memory, same
 * layout as rd_debug_export_kv, and set the position of every sequence to
 * pos.  For parity checks that hand the same cache to another
 * implementation. */
rd_status rd_debug_import_kv(rd_model* m, int32_t seq, int32_t layer, int32_t which, const void* src,
                             size_t bytes, int32_t pos);

/* Switch the executor of a live model (the cache and position are kept):
 * EAGER and GRAPH are always available; PERSISTENT only where the model
 * was created with AUTO or PERSISTENT and its shape has a persistent kernel.
 * Errors: INVALID_ARG, UNSUPPORTED. */
rd_status rd_set_executor(rd_model* m, int32_t executor);

/* Rewind every sequence to position pos <= the current position; rows at
 * pos and later become unreachable and are rewritten by the next steps.
 * With the INT8 cache pos must be a multiple of 128 or lie in the segment
 * still open (rows of an older open segment are gone once sealed).
 * Errors: INVALID_ARG. */
rd_status rd_set_position(rd_model* m, int32_t pos);

/* Enqueue `iters` launches of one phase kernel of the step, exactly as the
 * step launches it, for layers (layer + i) % n_layers, at the current
 * position: phase 0 = RMSNorm+QKV+RoPE+append (layers >= 1 variant),
 * 1 = split-K attention + merge, 2 = output projection + residual,
 * 3 = RMSNorm + gate/up + SwiGLU, 4 = down projection + residual.  For
 * timing single kernels on the model's stream; it overwrites activations
 * and the current cache row, so call rd_set_position before decoding again.
 * Errors: INVALID_ARG, DEVICE. */
rd_status rd_debug_run_phase(rd_model* m, int32_t phase, int32_t layer, int32_t iters);

/* One decode step of `token` with the persistent executor, recording an
 * event trace of workgroup 0: ts (host, cap uint64 words) receives
 * [n, code_0, clock_0, code_1, clock_1, ...] with clock the constant 100 MHz
 * wall clock and code = 10 * phase + point (phase 0 QKV, 1 attention split,
 * 2 merge of a query head, 3 output projection, 4 gate/up, 5 down, 6 LM
 * head; point 0 input received, 1 input staged, 2 rows reduced, 3 output
 * published; 99 kernel start, 98 end).  *n receives the event count
 * (at most (cap-1)/2).  Synchronises.  Errors: UNSUPPORTED for other
 * executors, INVALID_ARG, CONTEXT_FULL, DEVICE. */
rd_status rd_debug_trace_step(rd_model* m, int32_t token, uint64_t* ts, int32_t cap, int32_t* n);

/* The same trace for every workgroup of the persistent launch: ts (host)
 * holds n_wg regions of cap uint64 words, region w laid out as above for
 * workgroup w (the clock is one wall clock shared by all CUs, so regions
 * can be compared); *n_wg receives the workgroup count.  ts must hold
 * (workgroups of the launch) * cap words: the count is the device's CU
 * count.  Errors as rd_debug_trace_step. */
rd_status rd_debug_trace_step_all(rd_model* m, int32_t token, uint64_t* ts, int32_t cap, int32_t* n_wg);

const char* rd_last_error(void);

/* ---- kernels of the step, callable alone (device pointers) ------------------
 * Each runs exactly the device code the model's step uses, on the given
 * stream (NULL = the null stream), asynchronously.  Argument errors return
 * INVALID_ARG before anything is enqueued. */

/* y[b][n] = sum_k W[n][k] * x[b][k], fp16 inputs, fp32 accumulate and output:
 * the decode step's weight-streaming matrix-vector product measured alone
 * ("Real-time LLM inference on standard GPUs: 3,000 tokens/s per request",
 * section on memory bandwidth: about 1 FLOP per weight byte at fp16 and
 * batch 1, 8 at batch 8).  W: device fp16 row-major [N][K]; x: device fp16
 * [batch][K]; y: device f32 [batch][N].  batch 1: K a multiple of 8,
 * 8 <= K <= 8192, a streaming kernel with the step's own per-row dot
 * product (same bits as the step's GEMVs).  batch 8: K a multiple of 64,
 * 64 <= K <= 8192, a thin GEMM on the matrix cores (16x16x32 fp16 MFMA
 * tiles, rows 8..15 of the tile unused).  W and x 16-byte aligned.  Nothing
 * is allocated; the launch is asynchronous on `stream`. */
rd_status rd_gemv_f16(const void* W, const void* x, float* y, int32_t N, int32_t K, int32_t batch, void* stream);

/* Single-query attention of n_heads query heads over one sequence's cache
 * with grouped kv heads (query head h reads kv head h / (n_heads/n_kv_heads)):
 * out[h] = softmax(q[h] . K^[g][0..L) * scale) V^[g][0..L), computed as
 * partial softmaxes over at most `splits` key ranges merged by log-sum-exp,
 * where K^, V^ are the rows as stored, dequantized ("How the xAI engineering
 * team cut Grok Bot latency to milliseconds", §3.1: attention with a
 * 1/sqrt(d) scale; "LLM inference architecture rebuild", §3.3: the softmax
 * scale passed explicitly).  The step's own kernels, the cache read-only.
 * q: device f32 [n_heads][hd]; out: device f32 [n_heads][hd].
 * kv_format (rd_kv_format) and K, V (device, [n_kv_heads][ld][hd]):
 *   FP16: fp16 rows;
 *   FP8_E5M2: E5M2 bytes, read as the fp16 with that high byte (§2.3 of the
 *     xAI page);
 *   INT8_SEG128 ("Grok-3 v3.2.4 hot update deep dive", §3.2): u8 codes; the
 *     rows of segment k < (L-1)/128 read as (code - zp) * scale with
 *     (scale, zp) = k_meta/v_meta [n_kv_heads][ceil(ld/128)][2] (f32), the
 *     rows of the open segment (positions (L-1)/128*128 .. L-1) come from
 *     k_stage/v_stage, device u16 [n_kv_heads][128][hd] (fp16, row p % 128).
 *     Other formats: the four pointers are ignored (may be NULL).
 * scale: the softmax scale (1/sqrt(hd) in the model); hd 64 or 128;
 * 1 <= L <= ld; 1 <= splits <= 256 (INT8_SEG128: >= 2, the open segment
 * being a split of its own); n_kv_heads * ld * hd * element bytes below
 * 2 GiB; n_heads <= 128.  q, K, V and the
 * staging rows 16-byte aligned, the tables 8-byte aligned.  Uses a library
 * scratch buffer (split partials), allocated on the device's first call and
 * kept until the process ends: calls that overlap on one device (several
 * streams or threads) race on it. */
rd_status rd_attention(const float* q, const void* K, const void* V, const uint16_t* k_stage,
                       const uint16_t* v_stage, const float* k_meta, const float* v_meta, float* out,
                       int32_t n_heads, int32_t n_kv_heads, int32_t hd, int32_t L, int32_t ld, int32_t kv_format,
                       float scale, int32_t splits, void* stream);

/* rd_attention for callers that cannot allocate device memory (code under
 * hipGraph stream capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the split partials in a
 * fixed 4 MiB device array of the library instead of an allocated scratch.
 * Nothing is allocated, on the first call either (the array's address on the
 * current device is looked up then).  Limit: 256 + n_heads * splits *
 * (hd + 2) * 4 bytes <= 4 MiB, else INVALID_ARG with nothing enqueued.
 * Every call on one GPU uses that GPU's one array: calls that overlap on
 * one GPU (several streams or threads) race; calls in order on one stream
 * are safe (each call rewrites everything it reads). */
rd_status rd_attention_noalloc(const float* q, const void* K, const void* V, const uint16_t* k_stage,
                               const uint16_t* v_stage, const float* k_meta, const float* v_meta, float* out,
                               int32_t n_heads, int32_t n_kv_heads, int32_t hd, int32_t L, int32_t ld,
                               int32_t kv_format, float scale, int32_t splits, void* stream);

/* rd_attention with kv_format FP16 (same kernels, same scratch, same rules). */
rd_status rd_attention_f16(const float* q, const void* K, const void* V, float* out, int32_t n_heads,
                           int32_t n_kv_heads, int32_t hd, int32_t L, int32_t ld, float scale, int32_t splits,
                           void* stream);

/* Weight-only INT4 with fp32 scales ("LLM inference architecture
 * rebuild", §5.2: an INT4 weight is used as fp16(int4_value * scale), the
 * scale in fp32, round-to-nearest; "Real-time LLM inference on standard
 * GPUs", section on memory bandwidth: about 4 FLOP per weight byte at 4
 * bits).  Quantizer (the library's reading; the pages give none): per
 * (row, group of 128 columns) scale = amax / 7 in fp32 (1 for an all-zero
 * group), code = clamp(rint(w / scale), -8, 7), 4-bit two's complement,
 * column 2j in the low nibble of byte j of the row.
 * W: device fp16 [N][K] (16-byte aligned); codes: device u8 [N][K/2];
 * scales: device f32 [N][K/128] (4-byte aligned).  128 <= K <= 8192,
 * K % 128 == 0. */
rd_status rd_q4_quantize(const void* W, int32_t N, int32_t K, uint8_t* codes, float* scales, void* stream);

/* y[n] = sum_k fp16(code[n][k] * scale[n][k/128]) * x[k], fp16 x, fp32
 * accumulation (v_dot2_f32_f16 steps, as the fp16 GEMV), batch 1: the
 * weight-streaming GEMV at 0.53 bytes per weight.  codes, scales as
 * rd_q4_quantize writes them; x: device fp16 [K]; y: device f32 [N].
 * codes and x 16-byte aligned.  Nothing is allocated. */
rd_status rd_gemv_q4(const uint8_t* codes, const float* scales, const void* x, float* y, int32_t N, int32_t K,
                     void* stream);

/* out[i] = E5M2 encoding of the fp16 value in[i] (round to nearest even on
 * the dropped mantissa bits, overflow to inf, NaN to quiet NaN): the KV
 * format of "How the xAI engineering team cut Grok Bot latency to
 * milliseconds", §2.3, whose range §4.3 gives as +-57344.
 * in: device u16 [n]; out: device u8 [n]. */
rd_status rd_e5m2_encode(const uint16_t* in, uint8_t* out, size_t n, void* stream);

/* Segment quantization ("Grok-3 v3.2.4 hot update deep dive", §3.2) of
 * n_seg independent segments of seg_elems fp16 values each: per segment
 * min/max in fp32, scale=(max-min)/255 (when max==min: |min|, or 1 for an
 * all-zero segment, so that the value is kept exactly), zp=rint(-min/scale),
 * code=clamp(rint(x/scale)+zp, 0, 255).
 * in: device u16 [n_seg][seg_elems]; codes: device u8 [n_seg][seg_elems];
 * meta: device f32 [n_seg][2] (scale, zp).  seg_elems <= 65536. */
rd_status rd_seg_quant(const uint16_t* in, int32_t n_seg, int32_t seg_elems, uint8_t* codes, float* meta,
                       void* stream);

/* Delta quantization of n_seg K/V segments ("Grok-3 v3.2.4 hot update deep
 * dive", §3.2: the scheme that stores the differences between adjacent
 * tokens' values and quantizes them to INT8).  A segment is n rows of hd
 * fp16 values.  Its first row is kept as it is (anchor); the differences
 * x[p][j] - x[p-1][j] of rows 1..n-1, in binary32, are quantized together
 * with the formula of rd_seg_quant (their min/max in fp32, scale, zp, codes).
 * in: device u16 [n_seg][n][hd]; anchor: device u16 [n_seg][hd]; codes:
 * device u8 [n_seg][n-1][hd] (may be NULL when n == 1); meta: device f32
 * [n_seg][2] (scale, zp; 1 and 0 when n == 1).  1 <= n <= 4096, hd a
 * multiple of 8 in [8, 1024]; in and anchor 16-byte aligned, codes 8-byte
 * aligned.  Buffers are the caller's; INVALID_ARG on bad sizes, alignment or
 * NULL pointers, nothing launched. */
rd_status rd_delta_seal(const uint16_t* in, int32_t n_seg, int32_t n, int32_t hd, uint16_t* anchor, uint8_t* codes,
                        float* meta, void* stream);

/* The rows of delta-sealed segments restored (same section): out[s][0] =
 * anchor, out[s][p][j] = out[s][p-1][j] + (code - zp) * scale, in binary32
 * rounded after each operation, in row order, so the quantization errors of
 * the differences add up along the segment.  out: device f32 [n_seg][n][hd];
 * the other arguments as rd_delta_seal's outputs (out 16-byte aligned). */
rd_status rd_delta_restore(const uint16_t* anchor, const uint8_t* codes, const float* meta, int32_t n_seg, int32_t n,
                           int32_t hd, float* out, void* stream);

/* *out = index of the largest of v[0..n) (lowest index on ties): the greedy
 * sampling the step keeps on the GPU ("Real-time LLM inference on standard
 * GPUs", loss table).  v: device f32 [n]; out: device i32 [1].  Uses the
 * library scratch of rd_attention (its own part of it): calls that overlap
 * on one device race. */
rd_status rd_argmax_f32(const float* v, int32_t n, int32_t* out, void* stream);

/* Free the scratch buffers of rd_attention, rd_attention_f16 and
 * rd_argmax_f32 on every device that has one (they are allocated again by
 * the next call), after waiting for each such device to go idle; for a
 * process that wants its device memory back before it exits.  No call that
 * uses the scratch may be in flight or start meanwhile.  Errors: DEVICE. */
rd_status rd_release_scratch(void);

#ifdef __cplusplus
}
#endif
#endif
