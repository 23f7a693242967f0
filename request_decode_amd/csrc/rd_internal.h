// Host/device shared structures of the decode-step library (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rd {

constexpr int SEG = 128;       // tokens per INT8 KV segment
constexpr int MAX_SPLITS = 256;
constexpr int WG = 256;        // threads per workgroup of every kernel (4 waves)

enum KvFmt { KV_FP16 = 0, KV_E5M2 = 1, KV_INT8 = 2 };
enum ErrBits { ERR_TOKEN = 1, ERR_NONFINITE = 2 };

// Per-step scalars live on the device so that a captured step is static.
struct StepState {
    int pos;        // position being decoded (0-based)
    int n_gen;      // tokens written to gen_out by this generate call
    int err;        // ErrBits seen on the device
    int pad;
    int token[8];   // token at `pos` for each sequence
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

struct AttnArgs {
    const float* q;          // [H][hd] post-RoPE queries
    float* out;              // [H][hd] attention output
    void* kc;                // this layer's K: [Hk][ld][hd] fp16 | e5m2 | u8 codes
    void* vc;                // this layer's V
    uint16_t* kst;           // INT8: [Hk][128][hd] fp16 open-segment rows of K
    uint16_t* vst;
    float* kmeta;            // INT8: [Hk][nseg][2] (scale, zp)
    float* vmeta;
    float* part_o;           // [H][MAX_SPLITS][hd]
    float* part_ml;          // [H][MAX_SPLITS][2]
    int* cnt;                // [Hk] arrival counters (zero between uses)
    const int* pos_ptr;      // L = *pos_ptr + 1
    int ld, nseg, H, Hk, S;
    float scale;
};

struct StepArgs {
    int D, H, Hk, hd, F, V, max_ctx, S, kvfmt, n_layers;
    float eps, scale;
    const _Float16* embed;
    const _Float16* g_final;
    const _Float16* lm_head;
    const LayerW* layers;    // host array (used by the host launcher only)
    float* x;                // [D] residual stream
    float* q;                // [H*hd]
    float* a;                // [H*hd]
    float* m;                // [F]
    float* logits;           // [V]
    float* part_o;
    float* part_ml;
    int* cnt;                // [Hk]
    float* arg_val;          // [n LM-head workgroups]
    int* arg_idx;
    int* arg_cnt;            // [1]
    StepState* st;
    int* gen_out;            // [max_ctx]
    const float2* rope;      // [max_ctx][hd/2] (cos, sin)
    void* kc;                // [n_layers][Hk][max_ctx][hd] elements of the KV format
    void* vc;
    uint16_t* stage;         // INT8: [n_layers][2][Hk][128][hd]
    float* meta;             // INT8: [n_layers][2][Hk][nseg][2]
    int nseg;
};

// Persistent executor (rd_persistent.hip).
enum { ERR_BARRIER = 4 };
constexpr int BAR_SUB = 16;                       // barrier sub-counters
constexpr int BAR_STRIDE = 32;                    // ints between barrier words (128-byte lines)
constexpr int BAR_FLAGS = (BAR_SUB + 3) * BAR_STRIDE;       // per-workgroup flag words start here
constexpr int BAR_MAX_WG = 1024;
constexpr int BAR_WORDS = BAR_FLAGS + BAR_MAX_WG * BAR_STRIDE;
struct PersistArgs {
    const LayerW* layers;     // device copy of the per-layer weight pointers
    int* bar;                 // [BAR_WORDS]: sub-counters, top counter, generation, abort flag
    unsigned gen0;            // barrier generation when the launch starts
    int pos0;                 // position of the first step
    int n_steps;              // steps decoded by this launch
    int out_base;             // gen_out index of the first step's token
    int spin_limit;           // polls before a barrier wait gives up (watchdog)
    unsigned long long* trace;  // optional event trace of workgroup 0: [0] = count, then
                                // (code, wall clock at 100 MHz) pairs
    int trace_cap;              // events the trace buffer holds
};
// Trace event codes: 10 * phase + point; phases 0 QKV, 1 attention, 2 output
// projection, 3 gate/up, 4 down, 5 LM head; points 0 barrier wait done,
// 1 input staged, 2 phase work done, 3 arrival counted, 4 next loads issued.
enum { TR_WAIT = 0, TR_STAGED = 1, TR_DONE = 2, TR_ARRIVED = 3, TR_ISSUED = 4 };
// Barriers one launch of n steps passes.
inline unsigned persistent_barriers(int n_layers, int n_steps) {
    return (unsigned)(n_steps * 5 * n_layers + (n_steps - 1));
}
bool persistent_supported(const StepArgs& A);
hipError_t launch_persistent(const StepArgs& A, const PersistArgs& P, int nwg, hipStream_t s);
hipError_t persistent_max_grid(const StepArgs& A, int device, int* nwg);
hipError_t barrier_probe(int nwg, int n, int mode, float* us, int* errbits);

// Host launchers (rd_kernels.hip).
int kch_for(int K);
hipError_t launch_step(const StepArgs& A, hipStream_t s);
hipError_t launch_phase(const StepArgs& A, int phase, int layer, hipStream_t s);
hipError_t launch_gemv_f16(const void* W, const void* x, float* y, int N, int K, hipStream_t s);
hipError_t launch_attention_f16(const AttnArgs& A, int hd, int G, hipStream_t s);
hipError_t launch_e5m2(const uint16_t* in, uint8_t* out, size_t n, hipStream_t s);
hipError_t launch_seg_quant(const uint16_t* in, int n_seg, int seg_elems, uint8_t* codes, float* meta,
                            hipStream_t s);
hipError_t launch_argmax(const float* v, int n, int* out, float* part_val, int* part_idx, int* part_cnt,
                         hipStream_t s);
int lm_head_workgroups(int V);
bool step_supported(int D, int H, int Hk, int hd, int F, const char** why);

}  // namespace rd
