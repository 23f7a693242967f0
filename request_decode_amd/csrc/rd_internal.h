// Host/device shared structures of the decode-step library (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rd {

constexpr int SEG = 128;       // tokens per INT8 KV segment
constexpr int MAX_SPLITS = 256;
constexpr int WG = 256;        // threads per workgroup of the kernel-per-phase executor (4 waves)

enum KvFmt { KV_FP16 = 0, KV_E5M2 = 1, KV_INT8 = 2 };
enum ErrBits { ERR_TOKEN = 1, ERR_NONFINITE = 2, ERR_STALL = 4 };

// Per-step scalars live on the device so that a captured step is static.
struct StepState {
    int pos;        // position being decoded (0-based)
    int n_gen;      // tokens written to gen_out by this generate call
    int err;        // ErrBits seen on the device
    int pad;
    int token[8];   // token at `pos` for each sequence
    // paged KV cache (sequences at their own positions): sequence b decodes
    // position bpos[b]; a token of -1 sits the step out (act[b] = 0: nothing
    // stored, position kept)
    int bpos[8];
    int act[8];
};

// Weights of one layer in the device layout (see the re-tiling in rd_api.hip).
struct LayerW {
    const _Float16* wqkv;   // [(H+2Hk)*hd][D], rows re-ordered: RoPE pairs adjacent
    const _Float16* wo;     // [D][H*hd]
    const _Float16* wgu;    // [2F][D], rows gate_i, up_i interleaved
    const _Float16* wd;     // [D][F]
    const _Float16* g_attn; // [D]
    const _Float16* g_ffn;  // [D]
};

// Attention of one layer (or of the standalone attention entry point).
struct AttnArgs {
    const float* q;          // [H][hd] post-RoPE queries
    float* out;              // [H][hd] attention output
    const void* kc;          // this layer's K: [Hk][ld][hd] fp16 | e5m2 | u8 codes
    const void* vc;          // this layer's V
    uint16_t* kst;           // INT8: [Hk][128][hd] fp16 open-segment rows of K
    uint16_t* vst;
    float* kmeta;            // INT8: [Hk][nseg][2] (scale, zp)
    float* vmeta;
    void* kcw;               // INT8: writable code rows of K and V (sealed by the merge)
    void* vcw;
    float* part;             // [H][S][hd+2] split partials: o[hd], m, l
    // paged KV cache: kc/vc are this layer's page pool [npages][Hk][R][hd]
    // (R = 1 << pshift positions of one kv head per 4 KiB page), and row p of
    // sequence b lies in page ptab[b*pt_ld + p/R] (-1: not allocated);
    // positions and activity per sequence (pos_ptr + b, act_ptr + b)
    const int* ptab;         // NULL: contiguous cache
    int pt_ld, pshift, npages;
    const int* act_ptr;
    // at least hd*2 bytes that no attention step changes and that decode to
    // finite fp16 and E5M2 values (position 0's RoPE row: cos 1, sin 0; the
    // standalone attention entry point: its queries, whose values are never
    // used there): fetched in place of cache rows whose values are not used
    const void* ro;
    const int* pos_ptr;      // L = *pos_ptr + 1
    int ld, nseg, H, Hk, S;
    float scale;
    int seal;                // INT8: the merge seals a segment the step fills (0: the cache is read-only)
    // B sequences (grid dimension y): sequence b's q, out, part and cache
    // regions lie b strides past sequence 0's (strides in elements of each
    // buffer, the cache ones in bytes)
    int nseq;
    size_t q_bstride, part_bstride, kv_bstride, st_bstride, meta_bstride;
    int pos_bstride;         // 1: a position per sequence (paged), 0: one for all
};
// Sequence b's view of the attention arguments.
__host__ __device__ inline AttnArgs attn_seq(AttnArgs T, int b) {
    T.q += (size_t)b * T.q_bstride;
    T.out += (size_t)b * T.q_bstride;
    T.pos_ptr += b * T.pos_bstride;
    if (T.ptab) {
        T.ptab += (size_t)b * T.pt_ld;
        T.act_ptr += b;
    }
    T.part += (size_t)b * T.part_bstride;
    T.kc = reinterpret_cast<const uint8_t*>(T.kc) + (size_t)b * T.kv_bstride;
    T.vc = reinterpret_cast<const uint8_t*>(T.vc) + (size_t)b * T.kv_bstride;
    T.kcw = reinterpret_cast<uint8_t*>(T.kcw) + (size_t)b * T.kv_bstride;
    T.vcw = reinterpret_cast<uint8_t*>(T.vcw) + (size_t)b * T.kv_bstride;
    if (T.kst) {
        T.kst += (size_t)b * T.st_bstride;
        T.vst += (size_t)b * T.st_bstride;
        T.kmeta += (size_t)b * T.meta_bstride;
        T.vmeta += (size_t)b * T.meta_bstride;
    }
    return T;
}

struct StepArgs {
    int D, H, Hk, hd, F, V, max_ctx, S, kvfmt, n_layers;
    float eps, scale;
    // batch: B sequences in lockstep (B > 1: kernel-per-phase executors only).
    // Activation buffers hold B rows; sequence b's cache regions lie b
    // strides past sequence 0's.
    int B, ncu;
    size_t kv_bstride;       // bytes of one sequence's K (or V) cache
    size_t st_bstride;       // INT8: elements of one sequence's staging rows
    size_t meta_bstride;     // INT8: floats of one sequence's (scale, zp) table
    _Float16* xh;            // B > 1: [B][D] normalised inputs of the QKV and gate/up GEMMs
    // paged KV cache (B > 1): kc/vc are page pools [n_layers][npages][Hk][R][hd],
    // R = 1 << pshift positions per 4 KiB page; sequence b's page table is
    // ptab[b*pt_ld ..] (device, -1: no page); positions per sequence (st->bpos)
    int* ptab;               // NULL: contiguous cache
    int pt_ld, pshift, npages;
    const _Float16* embed;
    const _Float16* g_final;
    const _Float16* lm_head;
    const LayerW* layers;    // host array (used by the host launchers only)
    float* x;                // [D] residual stream
    float* q;                // [H*hd]
    float* a;                // [H*hd]
    float* m;                // [B][F] SwiGLU output (B > 1: fp16 rows, F halves apart)
    float* logits;           // [V]
    float* part;             // [H][S][hd+2]
    float* arg_val;          // [n LM-head workgroups]
    int* arg_idx;
    int* arg_cnt;            // [1 + 16]
    StepState* st;
    int* gen_out;            // [max_ctx]
    const float2* rope;      // [max_ctx][hd/2] (cos, sin)
    void* kc;                // [n_layers][Hk][max_ctx][hd] elements of the KV format
    void* vc;
    uint16_t* stage;         // INT8: [n_layers][2][Hk][128][hd]
    float* meta;             // INT8: [n_layers][2][Hk][nseg][2]
    int nseg;
    // exchange words of the persistent executor: (tag << 32) | payload, the
    // payload fp32 bits or, for "pairs", elements (2w, 2w+1) as two fp16
    uint64_t* xb1;           // [D/2 pairs] residual stream after the down projection
    uint64_t* xb2;           // [D/2 pairs] residual stream after the output projection
    uint64_t* qb;            // [(H+2Hk)*hd] rotated q, then the new K and V rows as stored
    uint64_t* pb;            // [H][S][hd+2] attention split partials
    uint64_t* ab;            // [H*hd/2 pairs] attention output
    uint64_t* mb;            // [F/2 pairs] SwiGLU output
    uint64_t* lb;            // [workgroups] argmax: (value bits << 32) | (index << 12) | tag12
    int* abort_word;         // set when a wait of the persistent kernel gives up
};

// The attention view of layer l of the step's buffers.
__host__ __device__ inline AttnArgs attn_args(const StepArgs& A, int l) {
    AttnArgs T{};
    const size_t es = A.kvfmt == KV_FP16 ? 2 : 1;
    const size_t lay = A.ptab ? (size_t)l * A.npages * A.Hk * ((size_t)1 << A.pshift) * A.hd
                              : (size_t)l * A.Hk * A.max_ctx * A.hd;
    T.q = A.q;
    T.out = A.a;
    T.kc = reinterpret_cast<uint8_t*>(A.kc) + lay * es;
    T.vc = reinterpret_cast<uint8_t*>(A.vc) + lay * es;
    T.kcw = reinterpret_cast<uint8_t*>(A.kc) + lay * es;
    T.vcw = reinterpret_cast<uint8_t*>(A.vc) + lay * es;
    if (A.kvfmt == KV_INT8) {
        T.kst = A.stage + ((size_t)l * 2 + 0) * A.Hk * SEG * A.hd;
        T.vst = A.stage + ((size_t)l * 2 + 1) * A.Hk * SEG * A.hd;
        T.kmeta = A.meta + ((size_t)l * 2 + 0) * A.Hk * A.nseg * 2;
        T.vmeta = A.meta + ((size_t)l * 2 + 1) * A.Hk * A.nseg * 2;
    }
    T.part = A.part;
    T.ro = A.rope;
    T.pos_ptr = &A.st->pos;
    T.ld = A.max_ctx;
    T.nseg = A.nseg;
    T.H = A.H;
    T.Hk = A.Hk;
    T.S = A.S;
    T.scale = A.scale;
    T.nseq = A.B;
    T.seal = 1;
    T.q_bstride = (size_t)A.H * A.hd;
    T.part_bstride = (size_t)A.H * A.S * (A.hd + 2);
    T.kv_bstride = A.kv_bstride;
    T.st_bstride = A.st_bstride;
    T.meta_bstride = A.meta_bstride;
    T.pos_bstride = 0;
    if (A.ptab) {
        T.ptab = A.ptab;
        T.pt_ld = A.pt_ld;
        T.pshift = A.pshift;
        T.npages = A.npages;
        T.pos_ptr = A.st->bpos;
        T.act_ptr = A.st->act;
        T.pos_bstride = 1;
        T.kv_bstride = 0;
    }
    return T;
}

// Persistent executor (rd_persistent.hip).
struct PersistArgs {
    LayerW layer0;            // layer 0's weights; layer l's lie layer_stride bytes further per layer
    long long layer_stride;
    uint32_t tag0;            // exchange tag base: step s, layer l uses tag0 + s*(n_layers+1) + l + 1
    int pos0;                 // position of the first step
    int n_steps;              // steps decoded by this launch
    int out_base;             // gen_out index of the first step's token
    int spin_limit;           // polls before a wait gives up (watchdog)
    unsigned long long* trace;  // optional event trace of workgroup 0 (or of every workgroup,
                                // trace_all): per workgroup [count, then (code, wall clock at
                                // 100 MHz) pairs], 1 + 2*trace_cap words each
    int trace_cap;              // events one workgroup's trace holds
    int trace_all;
};
// Tags one launch of n steps consumes.
inline uint32_t persistent_tags(int n_layers, int n_steps) { return (uint32_t)n_steps * (uint32_t)(n_layers + 1); }
// Trace event codes: 10 * phase + point; phases 0 QKV, 1 attention, 2 merge,
// 3 output projection, 4 gate/up, 5 down, 6 LM head; points 0 input received,
// 1 input staged, 2 rows reduced, 3 output published.
enum { TR_RECV = 0, TR_STAGED = 1, TR_DONE = 2, TR_PUB = 3 };
bool persistent_supported(const StepArgs& A);
hipError_t launch_persistent(const StepArgs& A, const PersistArgs& P, int nwg, hipStream_t s);
hipError_t persistent_max_grid(const StepArgs& A, int device, int* nwg);

// Batched prefill (rd_prefill.hip): workspace of one chunk of up to tc
// prompt tokens.
struct PrefillWs {
    int* tok;       // [tc] token ids of the chunk (device)
    float* x;       // [tc][D] residual rows
    _Float16* xn;   // [tc][D] normalised rows (GEMM operand)
    float* q;       // [tc][H*hd] rotated queries
    _Float16* a;    // [tc][H*hd] attention output (GEMM operand)
    _Float16* m;    // [tc][F] SwiGLU output (GEMM operand)
    _Float16* kt;   // [2][Hk][tc][hd] the chunk's new K and V rows in fp16
    int tc;
};
bool prefill_supported(int D, int H, int hd, int F, int B);
// Positions p0 .. p0+T-1 (T <= ws.tc) of sequence 0, tokens in ws.tok.
hipError_t prefill_chunk(const StepArgs& A, const PrefillWs& ws, int p0, int T, hipStream_t s);

// Weight-only INT4 (rd_q4.hip): codes [N][K/2], scales [N][K/128]; K % 128 == 0, K <= 8192.
hipError_t launch_q4_quant(const void* W, int N, int K, uint8_t* codes, float* scales, hipStream_t s);
hipError_t launch_gemv_q4(const uint8_t* codes, const float* scales, const void* x, float* y, int N, int K, int ncu,
                          hipStream_t s);

// Host launchers (rd_kernels.hip).
int kch_for(int K);
hipError_t launch_step(const StepArgs& A, hipStream_t s);
hipError_t launch_phase(const StepArgs& A, int phase, int layer, hipStream_t s);
hipError_t launch_gemv_f16(const void* W, const void* x, float* y, int N, int K, int batch, int ncu, hipStream_t s);
// Y[b][n] (=|+=) sum_k W[n][k] x[b][k] for b < B <= 8 on the matrix cores; x fp16 or fp32 (row stride ldx),
// y fp32 (row stride ldy); K % 64 == 0, K <= 8192.
hipError_t launch_step_batch(const StepArgs& A, hipStream_t s);
// Paged cache: page group src copied to dst (copy on write).
hipError_t launch_page_copy(const StepArgs& A, int src, int dst, hipStream_t s);
hipError_t launch_attn_any(const AttnArgs& A, int kvfmt, int hd, int G, hipStream_t s);
hipError_t launch_gemm_b8(const _Float16* W, const void* x, bool x_f32, int ldx, float* y, int ldy, bool acc, int N,
                          int K, int B, int ncu, hipStream_t s);
// m[b][i] = fp16(silu(gate_i . x[b]) * (up_i . x[b])) for B <= 8 rows of fp16 x,
// Wgu [2F][K] with gate and up rows interleaved; m row stride ldm.
hipError_t launch_gemm_b8_swiglu(const _Float16* Wgu, const _Float16* x, int ldx, _Float16* m, int ldm, int F, int K,
                                 int B, int ncu, hipStream_t s);
// The batch step's QKV GEMM of layer `layer` over A.xh (B rows), with RoPE
// and the K/V append of each sequence at A.st->pos as its epilogue.
hipError_t launch_gemm_b8_qkv(const StepArgs& A, int layer, const _Float16* Wqkv, hipStream_t s);
hipError_t launch_attention(const AttnArgs& A, int kvfmt, int hd, int G, hipStream_t s);
hipError_t launch_e5m2(const uint16_t* in, uint8_t* out, size_t n, hipStream_t s);
hipError_t launch_seg_quant(const uint16_t* in, int n_seg, int seg_elems, uint8_t* codes, float* meta,
                            hipStream_t s);
hipError_t launch_delta_seal(const uint16_t* in, int n_seg, int n, int hd, uint16_t* anchor, uint8_t* codes,
                             float* meta, hipStream_t s);
hipError_t launch_delta_restore(const uint16_t* anchor, const uint8_t* codes, const float* meta, int n_seg, int n,
                                int hd, float* out, hipStream_t s);
hipError_t launch_argmax(const float* v, int n, int* out, float* part_val, int* part_idx, int* part_cnt,
                         hipStream_t s);
int lm_head_workgroups(int V);
bool step_supported(int D, int H, int Hk, int hd, int F, const char** why);

}  // namespace rd
