// Host runtime and C ABI of the decode-step library (see include/rd.h).
//
// create: parse the weight blob, re-tile it into the layout the kernels
// stream (once), allocate the KV cache in the requested format, build the
// RoPE table, and set up the executor.  A step is a fixed sequence of
// launches whose per-step scalars (position, token) live in device memory,
// so the whole step can be captured once into a hipGraph and replayed
// ("How the xAI engineering team cut Grok Bot latency to milliseconds",
// §2.1 and §4.1: capture the decode step once, feed it through a static
// buffer, replay it), and generated tokens feed the next step on the device
// without a host round trip (sampling stays on the GPU, "Real-time LLM
// inference on standard GPUs", loss table).
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "rd.h"
#include "rd_internal.h"

using namespace rd;

static thread_local std::string g_err;

static rd_status fail(rd_status st, const std::string& msg) {
    g_err = msg;
    return st;
}

extern "C" const char* rd_last_error(void) { return g_err.c_str(); }

#define HIP_TRY(expr)                                                                         \
    do {                                                                                      \
        hipError_t e_ = (expr);                                                               \
        if (e_ != hipSuccess) return dev_fail(m, #expr, e_);                                  \
    } while (0)

// ---------------------------------------------------------------------------
// blob parsing (host only)
// ---------------------------------------------------------------------------
namespace {

struct BlobDims {
    int L, D, H, Hk, hd, F, V;
    float base, eps;
    size_t embed, final_norm, lm_head;
    std::vector<size_t> layer;  // 9 offsets per layer
};

template <class T>
T rd_le(const uint8_t* p) {
    T v;
    memcpy(&v, p, sizeof v);
    return v;
}

bool parse_blob(const uint8_t* b, size_t n, BlobDims& d, std::string& err) {
    if (!b || n < 256) { err = "blob shorter than its 256-byte header"; return false; }
    if (memcmp(b, "RDW1", 4) != 0) { err = "bad blob magic"; return false; }
    if (rd_le<uint32_t>(b + 4) != 1) { err = "unsupported blob version"; return false; }
    if (rd_le<uint32_t>(b + 8) != 256) { err = "unsupported header size"; return false; }
    if (rd_le<uint32_t>(b + 12) != 1) { err = "unsupported tensor dtype (fp16 = 1 expected)"; return false; }
    if (rd_le<uint32_t>(b + 52) != 0) { err = "unsupported flags"; return false; }
    d.L = rd_le<int32_t>(b + 16); d.D = rd_le<int32_t>(b + 20); d.H = rd_le<int32_t>(b + 24);
    d.Hk = rd_le<int32_t>(b + 28); d.hd = rd_le<int32_t>(b + 32); d.F = rd_le<int32_t>(b + 36);
    d.V = rd_le<int32_t>(b + 40);
    d.base = rd_le<float>(b + 44);
    d.eps = rd_le<float>(b + 48);
    if (d.L <= 0 || d.D <= 0 || d.H <= 0 || d.Hk <= 0 || d.hd <= 0 || d.F <= 0 || d.V <= 0 || d.L > 4096 ||
        d.D > (1 << 20) || d.V > (1 << 24) || d.F > (1 << 22) || d.H > 4096 || d.Hk > 4096 || d.hd > 4096) {
        err = "bad dimensions in blob header";
        return false;
    }
    if (!(d.base > 1.0f) || !(d.eps >= 0.0f) || !isfinite(d.base) || !isfinite(d.eps)) {
        err = "bad rope_base / norm_eps";
        return false;
    }
    size_t off = 256;
    auto take = [&](size_t elems) {
        off = (off + 255) / 256 * 256;
        size_t o = off;
        off += elems * 2;
        return o;
    };
    const size_t D = d.D, H = d.H, Hk = d.Hk, hd = d.hd, F = d.F, V = d.V;
    d.embed = take(V * D);
    d.layer.clear();
    for (int l = 0; l < d.L; ++l) {
        d.layer.push_back(take(D));
        d.layer.push_back(take(H * hd * D));
        d.layer.push_back(take(Hk * hd * D));
        d.layer.push_back(take(Hk * hd * D));
        d.layer.push_back(take(D * H * hd));
        d.layer.push_back(take(D));
        d.layer.push_back(take(F * D));
        d.layer.push_back(take(F * D));
        d.layer.push_back(take(D * F));
    }
    d.final_norm = take(D);
    d.lm_head = take(V * D);
    if (off != n) {
        err = "blob is " + std::to_string(n) + " bytes, its header implies " + std::to_string(off);
        return false;
    }
    return true;
}

}  // namespace

// ---------------------------------------------------------------------------
// model
// ---------------------------------------------------------------------------
struct rd_model {
    int dev = 0;
    hipStream_t stream = nullptr;
    bool own_stream = false;
    hipStream_t cap_stream = nullptr;
    BlobDims d;
    rd_options opt{};
    int S = 64;
    bool poisoned = false;
    int host_pos = 0;

    void* wbuf = nullptr;
    size_t wbytes = 0, streamed = 0;
    std::vector<LayerW> layers;
    const _Float16 *embed = nullptr, *g_final = nullptr, *lm_head = nullptr;

    void* kc = nullptr;
    void* vc = nullptr;
    uint16_t* stage = nullptr;
    float* meta = nullptr;
    size_t kv_bytes = 0;
    int nseg = 0;

    void* act = nullptr;  // activations, partials, counters, state, tables
    StepArgs A{};
    int* gen_host = nullptr;     // pinned [max_ctx]
    float* logits_host = nullptr; // pinned [V]
    StepState* state_host = nullptr;

    hipGraph_t graph = nullptr;
    hipGraphExec_t gexec = nullptr;

    // batched prefill workspace (allocated on the first rd_prefill_batched)
    void* pf_buf = nullptr;
    PrefillWs pf{};

    // paged KV cache (opt.kv_pages > 0): host page tables, refcounts, free list
    bool paged = false;
    int npages = 0, prow = 0, pshift = 0, pt_ld = 0;
    int* ptab_dev = nullptr;        // [max_batch][pt_ld] device copy of ptab
    std::vector<int> ptab;          // [max_batch][pt_ld] page group per page of positions, -1: none
    std::vector<int> refc;          // [npages] sequences holding the group
    std::vector<int> freel;         // free groups (taken from the back)
    std::vector<int> hpos;          // [max_batch] positions (rows held)

    // persistent executor
    long long layer_stride = 0;     // bytes between consecutive layers' weight blocks
    int nwg = 0;                    // workgroups of the cooperative launch (0: not available)
    uint32_t tag = 0;               // exchange tag base of the next launch
};

static rd_status dev_fail(rd_model* m, const char* what, hipError_t e) {
    if (m) m->poisoned = true;
    return fail(RD_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

extern "C" void rd_options_init(rd_options* o) {
    if (!o) return;
    memset(o, 0, sizeof *o);
    o->struct_size = sizeof(rd_options);
    o->max_context = 4096;
    o->max_batch = 1;
    o->kv_format = RD_KV_FP16;
    o->executor = RD_EXEC_AUTO;
}

namespace {

struct Tokens8 {
    int t[8];
};
// clear_err = 0 keeps the error bits of earlier steps, so that a run of
// teacher-forced steps synchronised once reports an error of any of them.
__global__ void k_set_state(StepState* st, int pos, Tokens8 tk, int nb, int reset_gen, int clear_err, Tokens8 bp,
                            int set_bpos) {
    st->pos = pos;
    for (int b = 0; b < nb; ++b) st->token[b] = tk.t[b];
    if (set_bpos)
        for (int b = 0; b < nb; ++b) st->bpos[b] = bp.t[b];
    if (clear_err) st->err = 0;
    if (reset_gen) st->n_gen = 0;
}

__global__ void k_set_int(int* p, int v) { *p = v; }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

void free_model(rd_model* m) {
    if (!m) return;
    (void)hipSetDevice(m->dev);
    // work still queued (rd_generate_async) may be running the graph
    if (m->stream) (void)hipStreamSynchronize(m->stream);
    if (m->gexec) (void)hipGraphExecDestroy(m->gexec);
    if (m->graph) (void)hipGraphDestroy(m->graph);
    (void)hipFree(m->wbuf);
    (void)hipFree(m->kc);
    (void)hipFree(m->vc);
    (void)hipFree(m->stage);
    (void)hipFree(m->meta);
    (void)hipFree(m->act);
    (void)hipFree(m->pf_buf);
    (void)hipFree(m->ptab_dev);
    if (m->gen_host) (void)hipHostFree(m->gen_host);
    if (m->logits_host) (void)hipHostFree(m->logits_host);
    if (m->state_host) (void)hipHostFree(m->state_host);
    if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
    if (m->own_stream && m->stream) (void)hipStreamDestroy(m->stream);
    delete m;
}

// Watchdog of the persistent kernel's waits: polls of about a microsecond.
constexpr int kSpinLimit = 1 << 21;

// One cooperative launch decoding n steps from the current device state.
rd_status persistent_enqueue(rd_model* m, int n, int out_base, unsigned long long* trace = nullptr,
                             int trace_cap = 0, int trace_all = 0) {
    PersistArgs P{};
    P.trace = trace;
    P.trace_cap = trace_cap;
    P.trace_all = trace_all;
    P.layer0 = m->layers[0];
    P.layer_stride = m->layer_stride;
    P.tag0 = m->tag;
    P.pos0 = m->host_pos;
    P.n_steps = n;
    P.out_base = out_base;
    P.spin_limit = kSpinLimit;
    HIP_TRY(launch_persistent(m->A, P, m->nwg, m->stream));
    m->tag += persistent_tags(m->d.L, n);
    return RD_OK;
}

rd_status step_enqueue(rd_model* m) {
    if (m->opt.executor == RD_EXEC_PERSISTENT) return persistent_enqueue(m, 1, 0);
    if (m->opt.executor == RD_EXEC_EAGER) {
        HIP_TRY(launch_step(m->A, m->stream));
        return RD_OK;
    }
    if (!m->gexec) {
        HIP_TRY(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal));
        hipError_t le = launch_step(m->A, m->cap_stream);
        hipGraph_t g = nullptr;
        hipError_t ce = hipStreamEndCapture(m->cap_stream, &g);
        if (le != hipSuccess) return dev_fail(m, "launch_step (capture)", le);
        if (ce != hipSuccess) return dev_fail(m, "hipStreamEndCapture", ce);
        m->graph = g;
        HIP_TRY(hipGraphInstantiate(&m->gexec, m->graph, nullptr, nullptr, 0));
    }
    HIP_TRY(hipGraphLaunch(m->gexec, m->stream));
    return RD_OK;
}

// Tokens of every sequence (host [max_batch], or NULL for zeros) and the
// position into the device step state.
hipError_t set_state(rd_model* m, const int32_t* tokens, bool clear_err = true) {
    Tokens8 tk{}, bp{};
    for (int b = 0; b < m->opt.max_batch; ++b) {
        tk.t[b] = tokens ? tokens[b] : 0;
        bp.t[b] = m->paged ? m->hpos[b] : 0;
    }
    hipLaunchKernelGGL(k_set_state, dim3(1), dim3(1), 0, m->stream, m->A.st, m->host_pos, tk, m->opt.max_batch, 1,
                       clear_err ? 1 : 0, bp, m->paged ? 1 : 0);
    return hipGetLastError();
}
// Token ids in range; a paged cache also takes -1 (the sequence sits the step out).
bool tokens_ok(const rd_model* m, const int32_t* t, int n, bool allow_idle = false) {
    for (int i = 0; i < n; ++i)
        if (!(t[i] >= 0 && t[i] < m->d.V) && !(allow_idle && m->paged && t[i] == -1)) return false;
    return true;
}

// ---- paged KV cache: page groups on the host ----------------------------------
void page_release(rd_model* m, int b) {
    for (int j = 0; j < m->pt_ld; ++j) {
        int& e = m->ptab[(size_t)b * m->pt_ld + j];
        if (e >= 0 && --m->refc[e] == 0) m->freel.push_back(e);
        e = -1;
    }
    m->hpos[b] = 0;
}
// Pages for the next steps[b] positions of each sequence b (from hpos[b]):
// a missing page from the free list, a shared page that a row is about to be
// written into copied first (copy on write; only the page of hpos[b] can be
// shared, since a fork shares pages up to the source's position).  All or
// nothing: OUT_OF_MEMORY with no change when the pool cannot cover it.  Then
// the device page table is brought up to date (enqueued on the stream).
rd_status page_prepare(rd_model* m, const int* steps) {
    const int B = m->opt.max_batch;
    int need = 0;
    for (int b = 0; b < B; ++b) {
        if (steps[b] <= 0) continue;
        const int j0 = m->hpos[b] >> m->pshift, j1 = (m->hpos[b] + steps[b] - 1) >> m->pshift;
        for (int j = j0; j <= j1; ++j) {
            const int e = m->ptab[(size_t)b * m->pt_ld + j];
            need += e < 0 || m->refc[e] > 1;
        }
    }
    if (need > (int)m->freel.size())
        return fail(RD_ERR_OUT_OF_MEMORY, "KV page pool exhausted: " + std::to_string(need) + " page groups needed, " +
                                              std::to_string(m->freel.size()) + " free");
    if (!need) return RD_OK;
    for (int b = 0; b < B; ++b) {
        if (steps[b] <= 0) continue;
        const int j0 = m->hpos[b] >> m->pshift, j1 = (m->hpos[b] + steps[b] - 1) >> m->pshift;
        for (int j = j0; j <= j1; ++j) {
            int& e = m->ptab[(size_t)b * m->pt_ld + j];
            if (e >= 0 && m->refc[e] == 1) continue;
            const int fresh = m->freel.back();
            m->freel.pop_back();
            m->refc[fresh] = 1;
            if (e >= 0) {   // shared: this sequence's copy of the rows so far
                HIP_TRY(launch_page_copy(m->A, e, fresh, m->stream));
                --m->refc[e];
            }
            e = fresh;
        }
    }
    // pageable source: the copy takes the table's current contents
    HIP_TRY(hipMemcpyAsync(m->ptab_dev, m->ptab.data(), m->ptab.size() * 4, hipMemcpyHostToDevice, m->stream));
    return RD_OK;
}

rd_status check_model(const rd_model* m) {
    if (!m) return fail(RD_ERR_INVALID_ARG, "model is NULL");
    if (m->poisoned) return fail(RD_ERR_DEVICE, "model is poisoned by an earlier device error");
    return RD_OK;
}

}  // namespace

extern "C" rd_status rd_model_create(const void* blob, size_t blob_bytes, const rd_options* opt_in, rd_model** out) {
    if (!out) return fail(RD_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!blob) return fail(RD_ERR_INVALID_ARG, "blob is NULL");
    rd_options opt;
    rd_options_init(&opt);
    if (opt_in) {
        if (opt_in->struct_size != sizeof(rd_options)) return fail(RD_ERR_INVALID_ARG, "rd_options.struct_size mismatch");
        opt = *opt_in;
    }
    if (opt.max_context < 1 || opt.max_context > (1 << 22)) return fail(RD_ERR_INVALID_ARG, "max_context out of range");
    if (opt.max_batch < 1 || opt.max_batch > 8) return fail(RD_ERR_UNSUPPORTED, "max_batch must be 1..8");
    if (opt.max_batch > 1 && opt.executor == RD_EXEC_PERSISTENT)
        return fail(RD_ERR_UNSUPPORTED, "the persistent executor runs batch 1 only");
    if (opt.kv_format < RD_KV_FP16 || opt.kv_format > RD_KV_INT8_SEG128)
        return fail(RD_ERR_INVALID_ARG, "bad kv_format");
    if (opt.executor < RD_EXEC_AUTO || opt.executor > RD_EXEC_PERSISTENT) return fail(RD_ERR_INVALID_ARG, "bad executor");
    if (opt.attn_splits < 0 || opt.attn_splits > MAX_SPLITS) return fail(RD_ERR_INVALID_ARG, "attn_splits out of range");
    if (opt.kv_pages < 0) return fail(RD_ERR_INVALID_ARG, "kv_pages < 0");
    if (opt.kv_pages > 0) {
        if (opt.kv_format == RD_KV_INT8_SEG128)
            return fail(RD_ERR_UNSUPPORTED, "a paged cache holds fp16 or E5M2 rows (INT8: contiguous cache)");
        if (opt.max_batch < 2) return fail(RD_ERR_UNSUPPORTED, "a paged cache serves the batch step (max_batch 2..8)");
        if (opt.executor == RD_EXEC_PERSISTENT)
            return fail(RD_ERR_UNSUPPORTED, "a paged cache runs on the EAGER or GRAPH executor");
    }
    if (opt.kv_format == RD_KV_INT8_SEG128 && opt.attn_splits == 1)
        return fail(RD_ERR_INVALID_ARG, "the INT8 cache needs at least 2 attention splits (the open segment has its own)");

    BlobDims d;
    std::string err;
    if (!parse_blob((const uint8_t*)blob, blob_bytes, d, err)) return fail(RD_ERR_BAD_BLOB, err);
    const char* why = nullptr;
    if (!step_supported(d.D, d.H, d.Hk, d.hd, d.F, &why)) return fail(RD_ERR_UNSUPPORTED, why);
    // attention reads a layer's K or V with 32-bit byte offsets
    if (opt.kv_pages == 0 &&
        (uint64_t)d.Hk * opt.max_context * d.hd * (opt.kv_format == RD_KV_FP16 ? 2 : 1) > 0x7fffffffull)
        return fail(RD_ERR_INVALID_ARG, "n_kv_heads * max_context * head_dim * element bytes must stay below 2 GiB");
    if (opt.kv_pages > 0) {
        const int prow = 4096 / (d.hd * (opt.kv_format == RD_KV_FP16 ? 2 : 1));
        if ((opt.max_context + prow - 1) / prow > 4094)
            return fail(RD_ERR_INVALID_ARG, "paged cache: max_context above 4094 pages per sequence");
        if ((uint64_t)opt.kv_pages * d.Hk * 4096 > 0x7fffffffull)
            return fail(RD_ERR_INVALID_ARG, "paged cache: kv_pages * n_kv_heads * 4 KiB must stay below 2 GiB");
    }

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) return fail(RD_ERR_DEVICE, "no HIP device");
    if (opt.device < 0 || opt.device >= ndev) return fail(RD_ERR_INVALID_ARG, "device ordinal out of range");

    rd_model* m = new rd_model();
    m->dev = opt.device;
    m->d = d;
    m->opt = opt;
    // Default key splits per kv-head, at most 64: batch 1, one attention task
    // per CU over all kv-heads (the persistent kernel gives each task a
    // workgroup); B sequences, two tasks per CU over all kv-heads and
    // sequences (fewer, longer tasks: at 8192 keys and B = 8, 8 splits
    // measured 3% faster per step than 32).
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, opt.device) != hipSuccess || cus < 1)
        cus = 1;
    const int s_def = opt.max_batch > 1 ? 2 * cus / ((int)d.Hk * opt.max_batch) : cus / (int)d.Hk;
    m->S = opt.attn_splits ? opt.attn_splits
                           : std::max(opt.kv_format == RD_KV_INT8_SEG128 ? 2 : 1, std::min(64, s_def));
    auto bail = [&](rd_status st) {
        std::string keep = g_err;
        free_model(m);
        g_err = keep;
        return st;
    };
#define CREATE_TRY(expr)                                                                      \
    do {                                                                                      \
        hipError_t e_ = (expr);                                                               \
        if (e_ == hipErrorOutOfMemory) return bail(fail(RD_ERR_OUT_OF_MEMORY, #expr));        \
        if (e_ != hipSuccess) return bail(fail(RD_ERR_DEVICE, std::string(#expr) + ": " + hipGetErrorString(e_))); \
    } while (0)

    CREATE_TRY(hipSetDevice(m->dev));
    if (opt.stream) {
        m->stream = (hipStream_t)opt.stream;
    } else {
        CREATE_TRY(hipStreamCreateWithFlags(&m->stream, hipStreamNonBlocking));
        m->own_stream = true;
    }
    CREATE_TRY(hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking));

    const size_t D = d.D, H = d.H, Hk = d.Hk, hd = d.hd, F = d.F, V = d.V, NL = d.L;
    const size_t NB = opt.max_batch;
    if (NB > 1 && ((D % 64) || ((H * hd) % 64) || (F % 64) || D > 8192 || H * hd > 8192 || F > 8192))
        return bail(fail(RD_ERR_UNSUPPORTED, "batch > 1 needs d_model, n_heads*head_dim, d_ff multiples of 64, <= 8192"));
    const size_t Nqkv = (H + 2 * Hk) * hd;
    // ---- device weight image: embed | per layer {wqkv, wo, wgu, wd, g_attn, g_ffn} | g_final | lm_head
    size_t off = 0;
    auto put = [&](size_t elems) {
        size_t o = off;
        off = align256(off + elems * 2);
        return o;
    };
    const size_t o_embed = put(V * D);
    std::vector<size_t> o_layer;
    for (size_t l = 0; l < NL; ++l) {
        o_layer.push_back(put(Nqkv * D));
        o_layer.push_back(put(D * H * hd));
        o_layer.push_back(put(2 * F * D));
        o_layer.push_back(put(D * F));
        o_layer.push_back(put(D));
        o_layer.push_back(put(D));
    }
    const size_t o_gfinal = put(D);
    const size_t o_lm = put(V * D);
    m->wbytes = off;
    CREATE_TRY(hipMalloc(&m->wbuf, m->wbytes));
    uint8_t* W = (uint8_t*)m->wbuf;
    const uint8_t* B = (const uint8_t*)blob;
    auto up = [&](size_t dst, const void* src, size_t bytes) { return hipMemcpy(W + dst, src, bytes, hipMemcpyHostToDevice); };

    CREATE_TRY(up(o_embed, B + d.embed, V * D * 2));
    std::vector<uint16_t> tmp;
    for (size_t l = 0; l < NL; ++l) {
        const size_t* L9 = &d.layer[l * 9];
        const uint16_t* wq = (const uint16_t*)(B + L9[1]);
        const uint16_t* wk = (const uint16_t*)(B + L9[2]);
        const uint16_t* wv = (const uint16_t*)(B + L9[3]);
        // fused QKV with each RoPE pair (j, j+hd/2) of a q or k head on adjacent rows
        tmp.resize(Nqkv * D);
        for (size_t rho = 0; rho < Nqkv; ++rho) {
            const uint16_t* src;
            if (rho < (H + Hk) * hd) {
                const bool isq = rho < H * hd;
                const size_t r = isq ? rho : rho - H * hd;
                const size_t head = r / hd, w = r % hd, j = w / 2, half = w % 2;
                const size_t srow = head * hd + j + half * (hd / 2);
                src = (isq ? wq : wk) + srow * D;
            } else {
                src = wv + (rho - (H + Hk) * hd) * D;
            }
            memcpy(&tmp[rho * D], src, D * 2);
        }
        CREATE_TRY(up(o_layer[l * 6 + 0], tmp.data(), Nqkv * D * 2));
        CREATE_TRY(up(o_layer[l * 6 + 1], B + L9[4], D * H * hd * 2));
        // gate/up interleaved: row 2i = gate_i, row 2i+1 = up_i
        const uint16_t* wg = (const uint16_t*)(B + L9[6]);
        const uint16_t* wu = (const uint16_t*)(B + L9[7]);
        tmp.resize(2 * F * D);
        for (size_t i = 0; i < F; ++i) {
            memcpy(&tmp[(2 * i) * D], wg + i * D, D * 2);
            memcpy(&tmp[(2 * i + 1) * D], wu + i * D, D * 2);
        }
        CREATE_TRY(up(o_layer[l * 6 + 2], tmp.data(), 2 * F * D * 2));
        CREATE_TRY(up(o_layer[l * 6 + 3], B + L9[8], D * F * 2));
        CREATE_TRY(up(o_layer[l * 6 + 4], B + L9[0], D * 2));
        CREATE_TRY(up(o_layer[l * 6 + 5], B + L9[5], D * 2));
        LayerW Lw;
        Lw.wqkv = (const _Float16*)(W + o_layer[l * 6 + 0]);
        Lw.wo = (const _Float16*)(W + o_layer[l * 6 + 1]);
        Lw.wgu = (const _Float16*)(W + o_layer[l * 6 + 2]);
        Lw.wd = (const _Float16*)(W + o_layer[l * 6 + 3]);
        Lw.g_attn = (const _Float16*)(W + o_layer[l * 6 + 4]);
        Lw.g_ffn = (const _Float16*)(W + o_layer[l * 6 + 5]);
        m->layers.push_back(Lw);
    }
    CREATE_TRY(up(o_gfinal, B + d.final_norm, D * 2));
    CREATE_TRY(up(o_lm, B + d.lm_head, V * D * 2));
    m->embed = (const _Float16*)(W + o_embed);
    m->g_final = (const _Float16*)(W + o_gfinal);
    m->lm_head = (const _Float16*)(W + o_lm);
    m->streamed = (NL * (Nqkv * D + D * H * hd + 2 * F * D + D * F + 2 * D) + D + V * D + D) * 2;

    // ---- KV cache: NB sequences, each [layer][kv-head][ctx][hd]
    const size_t ctx = opt.max_context;
    const size_t kv_seq = NL * Hk * ctx * hd;
    const size_t kv_elems = NB * kv_seq;
    const size_t es = opt.kv_format == RD_KV_FP16 ? 2 : 1;
    m->nseg = (int)((ctx + SEG - 1) / SEG);
    if (opt.kv_pages > 0) {
        // page pools [layer][group][kv head][page_rows][hd], 4 KiB per page
        m->paged = true;
        m->npages = opt.kv_pages;
        m->prow = (int)(4096 / (hd * es));
        while ((1 << m->pshift) < m->prow) ++m->pshift;
        m->pt_ld = (int)((ctx + m->prow - 1) / m->prow);
        const size_t pool = NL * (size_t)m->npages * Hk * 4096;
        CREATE_TRY(hipMalloc(&m->kc, pool));
        CREATE_TRY(hipMalloc(&m->vc, pool));
        CREATE_TRY(hipMemset(m->kc, 0, pool));
        CREATE_TRY(hipMemset(m->vc, 0, pool));
        CREATE_TRY(hipMalloc((void**)&m->ptab_dev, NB * m->pt_ld * 4));
        CREATE_TRY(hipMemset(m->ptab_dev, 0xff, NB * m->pt_ld * 4));   // -1: no page
        m->ptab.assign(NB * m->pt_ld, -1);
        m->refc.assign(m->npages, 0);
        for (int p = m->npages - 1; p >= 0; --p) m->freel.push_back(p);
        m->hpos.assign(NB, 0);
        m->kv_bytes = 2 * pool + NB * m->pt_ld * 4;
    } else {
        CREATE_TRY(hipMalloc(&m->kc, kv_elems * es));
        CREATE_TRY(hipMalloc(&m->vc, kv_elems * es));
        CREATE_TRY(hipMemset(m->kc, 0, kv_elems * es));
        CREATE_TRY(hipMemset(m->vc, 0, kv_elems * es));
        m->kv_bytes = 2 * kv_elems * es;
    }
    if (opt.kv_format == RD_KV_INT8_SEG128) {
        const size_t st_elems = NB * NL * 2 * Hk * SEG * hd, meta_elems = NB * NL * 2 * Hk * m->nseg * 2;
        CREATE_TRY(hipMalloc(&m->stage, st_elems * 2));
        CREATE_TRY(hipMalloc(&m->meta, meta_elems * 4));
        CREATE_TRY(hipMemset(m->stage, 0, st_elems * 2));
        CREATE_TRY(hipMemset(m->meta, 0, meta_elems * 4));
        m->kv_bytes += st_elems * 2 + meta_elems * 4;
    }

    // ---- activations, partials, counters, state, RoPE table
    const int n_lm_wg = lm_head_workgroups(d.V);
    size_t a = 0;
    auto carve = [&](size_t bytes) {
        size_t o = a;
        a = align256(a + bytes);
        return o;
    };
    const size_t o_x = carve(NB * D * 4), o_q = carve(NB * H * hd * 4), o_a = carve(NB * H * hd * 4);
    const size_t o_m = carve(NB * F * 4);
    const size_t o_logits = carve(NB * V * 4);
    const size_t S = m->S;
    const size_t o_part = carve(NB * H * S * (hd + 2) * 4);
    const size_t o_xh = carve(NB > 1 ? NB * D * 2 : 4);
    const int n_arg = n_lm_wg;   // argmax partials of the LM-head kernel
    const size_t o_av = carve(n_arg * 4), o_ai = carve(n_arg * 4), o_ac = carve(64 * 4);
    // exchange words of the persistent executor
    const size_t o_xb1 = carve(D * 8), o_xb2 = carve(D * 8), o_qb = carve(Nqkv * 8), o_pb = carve(H * S * (hd + 2) * 8);
    const size_t o_ab = carve(H * hd * 8), o_mb = carve(F * 8), o_lb = carve(1024 * 8), o_abort = carve(64);
    const size_t o_st = carve(sizeof(StepState)), o_gen = carve(NB * ctx * 4);
    const size_t o_rope = carve(ctx * (hd / 2) * sizeof(float2));
    CREATE_TRY(hipMalloc(&m->act, a));
    CREATE_TRY(hipMemset(m->act, 0, a));
    uint8_t* X = (uint8_t*)m->act;
    {
        std::vector<float2> rope(ctx * (hd / 2));
        for (size_t p = 0; p < ctx; ++p)
            for (size_t j = 0; j < hd / 2; ++j) {
                const double theta = pow((double)d.base, -2.0 * (double)j / (double)hd);
                const double ang = (double)p * theta;
                rope[p * (hd / 2) + j] = make_float2((float)cos(ang), (float)sin(ang));
            }
        CREATE_TRY(hipMemcpy(X + o_rope, rope.data(), rope.size() * sizeof(float2), hipMemcpyHostToDevice));
    }
    CREATE_TRY(hipHostMalloc((void**)&m->gen_host, NB * ctx * 4, hipHostMallocDefault));
    CREATE_TRY(hipHostMalloc((void**)&m->logits_host, NB * V * 4, hipHostMallocDefault));
    CREATE_TRY(hipHostMalloc((void**)&m->state_host, sizeof(StepState), hipHostMallocDefault));

    StepArgs& A = m->A;
    A.D = d.D; A.H = d.H; A.Hk = d.Hk; A.hd = d.hd; A.F = d.F; A.V = d.V;
    A.max_ctx = opt.max_context; A.S = m->S; A.kvfmt = opt.kv_format; A.n_layers = d.L;
    A.eps = d.eps;
    A.scale = (float)(1.0 / sqrt((double)d.hd));
    A.embed = m->embed; A.g_final = m->g_final; A.lm_head = m->lm_head;
    A.layers = m->layers.data();
    A.x = (float*)(X + o_x); A.q = (float*)(X + o_q); A.a = (float*)(X + o_a); A.m = (float*)(X + o_m);
    A.logits = (float*)(X + o_logits);
    A.part = (float*)(X + o_part);
    A.xb1 = (uint64_t*)(X + o_xb1); A.xb2 = (uint64_t*)(X + o_xb2); A.qb = (uint64_t*)(X + o_qb);
    A.pb = (uint64_t*)(X + o_pb); A.ab = (uint64_t*)(X + o_ab); A.mb = (uint64_t*)(X + o_mb);
    A.lb = (uint64_t*)(X + o_lb); A.abort_word = (int*)(X + o_abort);
    A.arg_val = (float*)(X + o_av); A.arg_idx = (int*)(X + o_ai); A.arg_cnt = (int*)(X + o_ac);
    A.st = (StepState*)(X + o_st); A.gen_out = (int*)(X + o_gen);
    A.rope = (const float2*)(X + o_rope);
    A.kc = m->kc; A.vc = m->vc; A.stage = m->stage; A.meta = m->meta; A.nseg = m->nseg;
    A.B = (int)NB;
    A.ncu = cus;
    A.kv_bstride = kv_seq * es;
    A.st_bstride = NL * 2 * Hk * SEG * hd;
    A.meta_bstride = NL * 2 * Hk * (size_t)m->nseg * 2;
    A.xh = (_Float16*)(X + o_xh);
    if (m->paged) {
        A.ptab = m->ptab_dev;
        A.pt_ld = m->pt_ld;
        A.pshift = m->pshift;
        A.npages = m->npages;
        A.kv_bstride = 0;
    }

    // ---- executor: the persistent kernel where its shape is built, else the graph
    if (NB > 1) {
        if (m->opt.executor == RD_EXEC_AUTO) m->opt.executor = RD_EXEC_GRAPH;
    } else if (opt.executor == RD_EXEC_AUTO || opt.executor == RD_EXEC_PERSISTENT) {
        int nwg = 0;
        if (persistent_supported(A) && persistent_max_grid(A, m->dev, &nwg) == hipSuccess && nwg > 0) {
            // the persistent kernel finds layer l's weights layer_stride bytes past layer 0's
            m->layer_stride = NL > 1 ? (long long)(o_layer[6] - o_layer[0]) : 0;
            for (size_t l = 1; l < NL; ++l)
                if (o_layer[6 * l] - o_layer[0] != l * (size_t)m->layer_stride)
                    return bail(fail(RD_ERR_DEVICE, "weight image is not layer-periodic"));
            m->nwg = nwg;
            m->opt.executor = RD_EXEC_PERSISTENT;
        } else if (opt.executor == RD_EXEC_PERSISTENT) {
            return bail(fail(RD_ERR_UNSUPPORTED, "no persistent kernel is built for this model shape"));
        } else {
            m->opt.executor = RD_EXEC_GRAPH;
        }
    }
#undef CREATE_TRY
    *out = m;
    return RD_OK;
}

extern "C" void rd_model_destroy(rd_model* m) { free_model(m); }

extern "C" rd_status rd_model_get_info(const rd_model* m, rd_model_info* o) {
    if (!m || !o) return fail(RD_ERR_INVALID_ARG, "NULL argument");
    o->n_layers = m->d.L; o->d_model = m->d.D; o->n_heads = m->d.H; o->n_kv_heads = m->d.Hk;
    o->head_dim = m->d.hd; o->d_ff = m->d.F; o->vocab = m->d.V;
    o->rope_base = m->d.base; o->norm_eps = m->d.eps;
    o->max_context = m->opt.max_context; o->max_batch = m->opt.max_batch;
    o->kv_format = m->opt.kv_format; o->executor = m->opt.executor; o->attn_splits = m->S;
    o->weight_bytes = m->wbytes;
    o->streamed_bytes = m->streamed;
    o->kv_bytes = m->kv_bytes;
    o->kv_pages = m->npages;
    o->page_rows = m->paged ? m->prow : 0;
    return RD_OK;
}

extern "C" rd_status rd_reset(rd_model* m) {
    rd_status st = check_model(m);
    if (st) return st;
    if (m->paged) {
        HIP_TRY(hipSetDevice(m->dev));
        HIP_TRY(hipStreamSynchronize(m->stream));
        for (int b = 0; b < m->opt.max_batch; ++b) page_release(m, b);
    }
    m->host_pos = 0;
    return RD_OK;
}

extern "C" rd_status rd_get_position(const rd_model* m, int32_t* pos) {
    if (!m || !pos) return fail(RD_ERR_INVALID_ARG, "NULL argument");
    *pos = m->paged ? m->hpos[0] : m->host_pos;
    return RD_OK;
}

extern "C" rd_status rd_seq_reset(rd_model* m, int32_t seq) {
    rd_status st = check_model(m);
    if (st) return st;
    if (!m->paged) return fail(RD_ERR_UNSUPPORTED, "a contiguous cache has no per-sequence pages (rd_reset)");
    if (seq < 0 || seq >= m->opt.max_batch) return fail(RD_ERR_INVALID_ARG, "seq out of range");
    HIP_TRY(hipSetDevice(m->dev));
    HIP_TRY(hipStreamSynchronize(m->stream));
    page_release(m, seq);
    return RD_OK;
}

extern "C" rd_status rd_seq_fork(rd_model* m, int32_t src, int32_t dst) {
    rd_status st = check_model(m);
    if (st) return st;
    if (!m->paged) return fail(RD_ERR_UNSUPPORTED, "prefix sharing needs a paged cache");
    if (src < 0 || src >= m->opt.max_batch || dst < 0 || dst >= m->opt.max_batch || src == dst)
        return fail(RD_ERR_INVALID_ARG, "src and dst must be distinct sequences");
    HIP_TRY(hipSetDevice(m->dev));
    HIP_TRY(hipStreamSynchronize(m->stream));
    page_release(m, dst);
    const int n = (m->hpos[src] + m->prow - 1) >> m->pshift;   // pages holding rows
    for (int j = 0; j < n; ++j) {
        const int e = m->ptab[(size_t)src * m->pt_ld + j];
        m->ptab[(size_t)dst * m->pt_ld + j] = e;
        if (e >= 0) ++m->refc[e];
    }
    m->hpos[dst] = m->hpos[src];
    HIP_TRY(hipMemcpy(m->ptab_dev, m->ptab.data(), m->ptab.size() * 4, hipMemcpyHostToDevice));
    return RD_OK;
}

extern "C" rd_status rd_seq_position(const rd_model* m, int32_t seq, int32_t* pos) {
    if (!m || !pos) return fail(RD_ERR_INVALID_ARG, "NULL argument");
    if (seq < 0 || seq >= m->opt.max_batch) return fail(RD_ERR_INVALID_ARG, "seq out of range");
    *pos = m->paged ? m->hpos[seq] : m->host_pos;
    return RD_OK;
}

extern "C" rd_status rd_kv_page_stats(const rd_model* m, int32_t* free_pages, int32_t* used_pages,
                                      int32_t* shared_pages) {
    if (!m) return fail(RD_ERR_INVALID_ARG, "model is NULL");
    if (!m->paged) return fail(RD_ERR_UNSUPPORTED, "a contiguous cache has no pages");
    int used = 0, shared = 0;
    for (int r : m->refc) {
        used += r > 0;
        shared += r > 1;
    }
    if (free_pages) *free_pages = (int32_t)m->freel.size();
    if (used_pages) *used_pages = used;
    if (shared_pages) *shared_pages = shared;
    return RD_OK;
}

extern "C" rd_status rd_set_executor(rd_model* m, int32_t executor) {
    rd_status st = check_model(m);
    if (st) return st;
    if (executor != RD_EXEC_EAGER && executor != RD_EXEC_GRAPH && executor != RD_EXEC_PERSISTENT)
        return fail(RD_ERR_INVALID_ARG, "executor must be EAGER, GRAPH or PERSISTENT");
    if (executor == RD_EXEC_PERSISTENT && !m->nwg)
        return fail(RD_ERR_UNSUPPORTED, "this model has no persistent kernel (batch > 1, or shape not built)");
    m->opt.executor = executor;
    return RD_OK;
}

extern "C" rd_status rd_set_position(rd_model* m, int32_t pos) {
    rd_status st = check_model(m);
    if (st) return st;
    if (m->paged) return fail(RD_ERR_UNSUPPORTED, "a paged cache keeps a position per sequence (rd_seq_reset)");
    if (pos < 0 || pos > m->host_pos) return fail(RD_ERR_INVALID_ARG, "position must be in [0, current]");
    if (m->opt.kv_format == RD_KV_INT8_SEG128 && pos % SEG != 0 && pos / SEG != m->host_pos / SEG)
        return fail(RD_ERR_INVALID_ARG, "INT8 cache: rewind only to a segment start or inside the open segment");
    m->host_pos = pos;
    return RD_OK;
}

static rd_status finish_sync(rd_model* m);

static rd_status trace_step(rd_model* m, int32_t token, uint64_t* ts, int32_t cap, int all, int32_t* n_out) {
    rd_status st = check_model(m);
    if (st) return st;
    if (!ts || !n_out) return fail(RD_ERR_INVALID_ARG, "NULL argument");
    if (m->opt.executor != RD_EXEC_PERSISTENT) return fail(RD_ERR_UNSUPPORTED, "tracing needs the persistent executor");
    if (m->host_pos >= m->opt.max_context) return fail(RD_ERR_CONTEXT_FULL, "context full");
    if (token < 0 || token >= m->d.V) return fail(RD_ERR_INVALID_ARG, "token id out of range");
    if (cap < 3) return fail(RD_ERR_INVALID_ARG, "trace capacity must be >= 3");
    const int events = (cap - 1) / 2;
    const size_t words = (1 + 2 * (size_t)events) * (all ? (size_t)m->nwg : 1);
    HIP_TRY(hipSetDevice(m->dev));
    unsigned long long* dev = nullptr;
    HIP_TRY(hipMalloc(&dev, words * 8));
    HIP_TRY(hipMemset(dev, 0, words * 8));
    HIP_TRY(set_state(m, &token));
    if ((st = persistent_enqueue(m, 1, 0, dev, events, all))) {
        (void)hipFree(dev);
        return st;
    }
    HIP_TRY(hipMemcpyAsync(m->state_host, m->A.st, sizeof(StepState), hipMemcpyDeviceToHost, m->stream));
    m->host_pos += 1;
    st = finish_sync(m);
    // Each region holds the control wave's events in its lower half and the
    // stream wave's in its upper half (counts packed in word 0); hand them
    // to the caller merged in clock order as [n, code, clock, ...].
    std::vector<uint64_t> h(words);
    HIP_TRY(hipMemcpy(h.data(), dev, words * 8, hipMemcpyDeviceToHost));
    const size_t rw = 1 + 2 * (size_t)events;
    auto merge = [&](const uint64_t* r, uint64_t* out) {
        const size_t nc = std::min<size_t>(r[0] & 0xffffffffu, events / 2);
        const size_t ns = std::min<size_t>(r[0] >> 32, events - events / 2);
        std::vector<std::pair<uint64_t, uint64_t>> ev;
        for (size_t i = 0; i < nc; ++i) ev.push_back({r[2 + 2 * i], r[1 + 2 * i]});
        for (size_t i = 0; i < ns; ++i) ev.push_back({r[2 + 2 * (events / 2 + i)], r[1 + 2 * (events / 2 + i)]});
        std::stable_sort(ev.begin(), ev.end(), [](const auto& a, const auto& b) { return a.first < b.first; });
        out[0] = ev.size();
        for (size_t i = 0; i < ev.size(); ++i) {
            out[1 + 2 * i] = ev[i].second;
            out[2 + 2 * i] = ev[i].first;
        }
        for (size_t i = 1 + 2 * ev.size(); i < rw; ++i) out[i] = 0;
    };
    if (all) {
        for (int w = 0; w < m->nwg; ++w) merge(h.data() + (size_t)w * rw, ts + (size_t)w * cap);
        *n_out = m->nwg;
    } else {
        merge(h.data(), ts);
        *n_out = (int32_t)ts[0];
    }
    (void)hipFree(dev);
    return st;
}

extern "C" rd_status rd_debug_trace_step(rd_model* m, int32_t token, uint64_t* ts, int32_t cap, int32_t* n_out) {
    return trace_step(m, token, ts, cap, 0, n_out);
}

extern "C" rd_status rd_debug_trace_step_all(rd_model* m, int32_t token, uint64_t* ts, int32_t cap, int32_t* n_wg) {
    return trace_step(m, token, ts, cap, 1, n_wg);
}

extern "C" rd_status rd_debug_run_phase(rd_model* m, int32_t phase, int32_t layer, int32_t iters) {
    rd_status st = check_model(m);
    if (st) return st;
    if (phase < 0 || phase > 4 || layer < 0 || layer >= m->d.L || iters < 0)
        return fail(RD_ERR_INVALID_ARG, "bad phase/layer/iters");
    if (m->host_pos >= m->opt.max_context) return fail(RD_ERR_CONTEXT_FULL, "context full");
    HIP_TRY(hipSetDevice(m->dev));
    if (m->opt.max_batch > 1) return fail(RD_ERR_UNSUPPORTED, "phase kernels are the batch-1 step's");
    HIP_TRY(set_state(m, nullptr));
    for (int i = 0; i < iters; ++i) HIP_TRY(launch_phase(m->A, phase, (layer + i) % m->d.L, m->stream));
    return RD_OK;
}

static rd_status finish_sync(rd_model* m) {
    HIP_TRY(hipStreamSynchronize(m->stream));
    if (m->state_host->err & ERR_STALL) {
        m->poisoned = true;
        return fail(RD_ERR_DEVICE, "a wait of the persistent kernel timed out");
    }
    if (m->state_host->err & ERR_TOKEN) return fail(RD_ERR_NUMERIC, "token id out of range seen on the device");
    if (m->state_host->err & ERR_NONFINITE) return fail(RD_ERR_NUMERIC, "non-finite logit");
    return RD_OK;
}

extern "C" rd_status rd_decode_step(rd_model* m, const int32_t* tokens, int32_t batch, float* logits, int32_t* next) {
    rd_status st = check_model(m);
    if (st) return st;
    if (!tokens) return fail(RD_ERR_INVALID_ARG, "tokens is NULL");
    if (batch != m->opt.max_batch) return fail(RD_ERR_INVALID_ARG, "batch must equal max_batch");
    if (!tokens_ok(m, tokens, batch, true)) return fail(RD_ERR_INVALID_ARG, "token id out of range");
    int steps[8] = {};
    for (int b = 0; b < batch; ++b) {
        steps[b] = tokens[b] != -1;
        const int at = m->paged ? m->hpos[b] : m->host_pos;
        if (steps[b] && at >= m->opt.max_context) return fail(RD_ERR_CONTEXT_FULL, "context full");
    }
    HIP_TRY(hipSetDevice(m->dev));
    if (m->paged && (st = page_prepare(m, steps))) return st;
    HIP_TRY(set_state(m, tokens));
    if ((st = step_enqueue(m))) return st;
    if (m->paged)
        for (int b = 0; b < batch; ++b) m->hpos[b] += steps[b];
    const size_t nlog = (size_t)batch * m->d.V;
    if (logits) HIP_TRY(hipMemcpyAsync(m->logits_host, m->A.logits, nlog * 4, hipMemcpyDeviceToHost, m->stream));
    HIP_TRY(hipMemcpyAsync(m->state_host, m->A.st, sizeof(StepState), hipMemcpyDeviceToHost, m->stream));
    m->host_pos += 1;
    st = finish_sync(m);
    if (st == RD_ERR_DEVICE) return st;
    if (logits) memcpy(logits, m->logits_host, nlog * 4);
    if (next)
        for (int b = 0; b < batch; ++b) next[b] = m->state_host->token[b];
    return st;
}

extern "C" rd_status rd_prefill(rd_model* m, const int32_t* tokens, int32_t batch, int32_t n) {
    rd_status st = check_model(m);
    if (st) return st;
    if (!tokens && n > 0) return fail(RD_ERR_INVALID_ARG, "tokens is NULL");
    if (batch != m->opt.max_batch) return fail(RD_ERR_INVALID_ARG, "batch must equal max_batch");
    if (n < 0) return fail(RD_ERR_INVALID_ARG, "n < 0");
    if (!tokens_ok(m, tokens, n * batch, true)) return fail(RD_ERR_INVALID_ARG, "token id out of range");
    int steps[8] = {};
    for (int b = 0; b < batch; ++b) {
        for (int i = 0; i < n; ++i) steps[b] += tokens[(size_t)i * batch + b] != -1;
        if (!m->paged) steps[b] = n;
        const int64_t at = m->paged ? m->hpos[b] : m->host_pos;
        if (at + steps[b] > m->opt.max_context) return fail(RD_ERR_CONTEXT_FULL, "tokens do not fit the context");
    }
    HIP_TRY(hipSetDevice(m->dev));
    if (m->paged && (st = page_prepare(m, steps))) return st;
    // one step per token on the graph path (the persistent kernel reads its
    // token from the device state, which a prompt would overwrite per step)
    const int32_t ex = m->opt.executor;
    if (ex == RD_EXEC_PERSISTENT) m->opt.executor = RD_EXEC_GRAPH;
    for (int i = 0; i < n && !st; ++i) {
        const int32_t* row = tokens + (size_t)i * batch;
        hipError_t e = set_state(m, row, i == 0);
        if (e != hipSuccess) st = dev_fail(m, "k_set_state", e);
        else if (!(st = step_enqueue(m))) {
            m->host_pos += 1;
            if (m->paged)
                for (int b = 0; b < batch; ++b) m->hpos[b] += row[b] != -1;
        }
    }
    m->opt.executor = ex;
    if (st) return st;
    HIP_TRY(hipMemcpyAsync(m->state_host, m->A.st, sizeof(StepState), hipMemcpyDeviceToHost, m->stream));
    return finish_sync(m);
}

// Chunk of the batched prefill: 2048 tokens (the workspace for the 2B-class
// model is about 100 MB).
constexpr int kPrefillChunk = 2048;

extern "C" rd_status rd_prefill_batched(rd_model* m, const int32_t* tokens, int32_t n) {
    rd_status st = check_model(m);
    if (st) return st;
    if (!tokens && n > 0) return fail(RD_ERR_INVALID_ARG, "tokens is NULL");
    if (n < 0) return fail(RD_ERR_INVALID_ARG, "n < 0");
    if (!prefill_supported(m->d.D, m->d.H, m->d.hd, m->d.F, m->opt.max_batch))
        return fail(RD_ERR_UNSUPPORTED, "batched prefill needs batch 1 and d_model, d_ff multiples of 32");
    if ((int64_t)m->host_pos + n > m->opt.max_context) return fail(RD_ERR_CONTEXT_FULL, "tokens do not fit the context");
    if (!tokens_ok(m, tokens, n)) return fail(RD_ERR_INVALID_ARG, "token id out of range");
    if (n == 0) return RD_OK;
    HIP_TRY(hipSetDevice(m->dev));
    if (!m->pf_buf) {
        const size_t tc = kPrefillChunk, D = m->d.D, H = m->d.H, Hk = m->d.Hk, hd = m->d.hd, F = m->d.F;
        size_t a = 0;
        auto carve = [&](size_t bytes) {
            size_t o = a;
            a = align256(a + bytes);
            return o;
        };
        const size_t o_tok = carve((size_t)m->opt.max_context * 4), o_x = carve(tc * D * 4), o_xn = carve(tc * D * 2);
        const size_t o_q = carve(tc * H * hd * 4), o_a = carve(tc * H * hd * 2), o_m = carve(tc * F * 2);
        const size_t o_kt = carve(2 * Hk * tc * hd * 2);
        hipError_t e = hipMalloc(&m->pf_buf, a);
        if (e == hipErrorOutOfMemory) return fail(RD_ERR_OUT_OF_MEMORY, "prefill workspace");
        if (e != hipSuccess) return dev_fail(m, "hipMalloc (prefill workspace)", e);
        uint8_t* b = (uint8_t*)m->pf_buf;
        m->pf = PrefillWs{(int*)(b + o_tok), (float*)(b + o_x), (_Float16*)(b + o_xn), (float*)(b + o_q),
                          (_Float16*)(b + o_a), (_Float16*)(b + o_m), (_Float16*)(b + o_kt), (int)tc};
    }
    HIP_TRY(hipStreamSynchronize(m->stream));
    HIP_TRY(hipMemcpy(m->pf.tok, tokens, (size_t)n * 4, hipMemcpyHostToDevice));
    for (int done = 0; done < n; done += kPrefillChunk) {
        const int T = std::min(kPrefillChunk, n - done);
        PrefillWs ws = m->pf;
        ws.tok = m->pf.tok + done;
        HIP_TRY(prefill_chunk(m->A, ws, m->host_pos + done, T, m->stream));
    }
    HIP_TRY(hipStreamSynchronize(m->stream));
    m->host_pos += n;
    return RD_OK;
}

static rd_status generate_enqueue(rd_model* m, const int32_t* first, int32_t batch, int32_t n) {
    rd_status st = check_model(m);
    if (st) return st;
    if (!first) return fail(RD_ERR_INVALID_ARG, "first is NULL");
    if (batch != m->opt.max_batch) return fail(RD_ERR_INVALID_ARG, "batch must equal max_batch");
    if (n < 0) return fail(RD_ERR_INVALID_ARG, "n_steps < 0");
    // (a paged cache: every sequence takes part in every generated step)
    if (!tokens_ok(m, first, batch)) return fail(RD_ERR_INVALID_ARG, "token id out of range");
    int steps[8] = {};
    for (int b = 0; b < batch; ++b) {
        steps[b] = n;
        const int64_t at = m->paged ? m->hpos[b] : m->host_pos;
        if (at + n > m->opt.max_context) return fail(RD_ERR_CONTEXT_FULL, "steps do not fit the context");
    }
    HIP_TRY(hipSetDevice(m->dev));
    if (m->paged && n > 0 && (st = page_prepare(m, steps))) return st;
    HIP_TRY(set_state(m, first));
    if (m->paged)
        for (int b = 0; b < batch; ++b) m->hpos[b] += n;
    if (m->opt.executor == RD_EXEC_PERSISTENT) {
        // whole runs of steps in one launch, in chunks that keep one kernel short
        constexpr int kChunk = 512;
        for (int done = 0; done < n; done += kChunk) {
            const int c = n - done < kChunk ? n - done : kChunk;
            if ((st = persistent_enqueue(m, c, done))) return st;
            m->host_pos += c;
        }
        return RD_OK;
    }
    for (int i = 0; i < n; ++i)
        if ((st = step_enqueue(m))) return st;
    m->host_pos += n;
    return RD_OK;
}

extern "C" rd_status rd_generate(rd_model* m, const int32_t* first, int32_t batch, int32_t n, int32_t* out) {
    if (!out && n > 0) return fail(RD_ERR_INVALID_ARG, "out_tokens is NULL");
    rd_status st = generate_enqueue(m, first, batch, n);
    if (st) return st;
    if (n == 0) return RD_OK;
    const size_t nt = (size_t)n * batch;
    HIP_TRY(hipMemcpyAsync(m->gen_host, m->A.gen_out, nt * 4, hipMemcpyDeviceToHost, m->stream));
    HIP_TRY(hipMemcpyAsync(m->state_host, m->A.st, sizeof(StepState), hipMemcpyDeviceToHost, m->stream));
    st = finish_sync(m);
    if (st == RD_ERR_DEVICE) return st;
    memcpy(out, m->gen_host, nt * 4);
    return st;
}

extern "C" rd_status rd_generate_async(rd_model* m, const int32_t* first, int32_t batch, int32_t n, int32_t* out_dev) {
    if (!out_dev && n > 0) return fail(RD_ERR_INVALID_ARG, "out_tokens_dev is NULL");
    rd_status st = generate_enqueue(m, first, batch, n);
    if (st) return st;
    if (n > 0)
        HIP_TRY(hipMemcpyAsync(out_dev, m->A.gen_out, (size_t)n * batch * 4, hipMemcpyDeviceToDevice, m->stream));
    HIP_TRY(hipMemcpyAsync(m->state_host, m->A.st, sizeof(StepState), hipMemcpyDeviceToHost, m->stream));
    return RD_OK;
}

extern "C" rd_status rd_synchronize(rd_model* m) {
    rd_status st = check_model(m);
    if (st) return st;
    HIP_TRY(hipSetDevice(m->dev));
    return finish_sync(m);
}

// ---- debug cache access -------------------------------------------------------
namespace {
struct KvRegion {
    uint8_t* dev;
    size_t bytes;
};
// Regions of (layer, which) in export order.
int kv_regions(rd_model* m, int seq, int layer, int which, KvRegion* r) {
    const size_t Hk = m->d.Hk, ctx = m->opt.max_context, hd = m->d.hd;
    const size_t es = m->opt.kv_format == RD_KV_FP16 ? 2 : 1;
    const size_t lay = (size_t)layer * Hk * ctx * hd * es;
    r[0] = {(uint8_t*)(which ? m->vc : m->kc) + seq * m->A.kv_bstride + lay, Hk * ctx * hd * es};
    if (m->opt.kv_format != RD_KV_INT8_SEG128) return 1;
    r[1] = {(uint8_t*)(m->stage + seq * m->A.st_bstride + ((size_t)layer * 2 + which) * Hk * SEG * hd),
            Hk * SEG * hd * 2};
    r[2] = {(uint8_t*)(m->meta + seq * m->A.meta_bstride + ((size_t)layer * 2 + which) * Hk * m->nseg * 2),
            Hk * (size_t)m->nseg * 8};
    return 3;
}
}  // namespace

extern "C" rd_status rd_debug_export_kv(rd_model* m, int32_t seq, int32_t layer, int32_t which, void* dst, size_t cap,
                                        size_t* written) {
    rd_status st = check_model(m);
    if (st) return st;
    if (!dst || seq < 0 || seq >= m->opt.max_batch || layer < 0 || layer >= m->d.L || which < 0 || which > 1)
        return fail(RD_ERR_INVALID_ARG, "bad export arguments");
    if (m->paged) {
        // the sequence's rows gathered through its page table, the contiguous layout
        const size_t Hk = m->d.Hk, ctx = m->opt.max_context, hd = m->d.hd, R = m->prow;
        const size_t es = m->opt.kv_format == RD_KV_FP16 ? 2 : 1, row = hd * es;
        const size_t total = Hk * ctx * row, pool = (size_t)m->npages * Hk * 4096;
        if (cap < total) return fail(RD_ERR_INVALID_ARG, "destination too small: need " + std::to_string(total));
        HIP_TRY(hipSetDevice(m->dev));
        HIP_TRY(hipStreamSynchronize(m->stream));
        std::vector<uint8_t> lay(pool);
        HIP_TRY(hipMemcpy(lay.data(), (const uint8_t*)(which ? m->vc : m->kc) + (size_t)layer * pool, pool,
                          hipMemcpyDeviceToHost));
        uint8_t* out = (uint8_t*)dst;
        memset(out, 0, total);
        for (int j = 0; j < m->pt_ld; ++j) {
            const int e = m->ptab[(size_t)seq * m->pt_ld + j];
            if (e < 0) continue;
            const size_t n = std::min(R, ctx - j * R);
            for (size_t g = 0; g < Hk; ++g)
                memcpy(out + (g * ctx + j * R) * row, lay.data() + ((size_t)e * Hk + g) * 4096, n * row);
        }
        if (written) *written = total;
        return RD_OK;
    }
    KvRegion r[3];
    const int nr = kv_regions(m, seq, layer, which, r);
    size_t total = 0;
    for (int i = 0; i < nr; ++i) total += r[i].bytes;
    if (cap < total) return fail(RD_ERR_INVALID_ARG, "destination too small: need " + std::to_string(total));
    HIP_TRY(hipSetDevice(m->dev));
    HIP_TRY(hipStreamSynchronize(m->stream));
    size_t o = 0;
    for (int i = 0; i < nr; ++i) {
        HIP_TRY(hipMemcpy((uint8_t*)dst + o, r[i].dev, r[i].bytes, hipMemcpyDeviceToHost));
        o += r[i].bytes;
    }
    if (written) *written = total;
    return RD_OK;
}

extern "C" rd_status rd_debug_import_kv(rd_model* m, int32_t seq, int32_t layer, int32_t which, const void* src,
                                        size_t bytes, int32_t pos) {
    rd_status st = check_model(m);
    if (st) return st;
    if (!src || seq < 0 || seq >= m->opt.max_batch || layer < 0 || layer >= m->d.L || which < 0 || which > 1 ||
        pos < 0 || pos > m->opt.max_context)
        return fail(RD_ERR_INVALID_ARG, "bad import arguments");
    if (m->paged) return fail(RD_ERR_UNSUPPORTED, "import into a paged cache");
    KvRegion r[3];
    const int nr = kv_regions(m, seq, layer, which, r);
    size_t total = 0;
    for (int i = 0; i < nr; ++i) total += r[i].bytes;
    if (bytes != total) return fail(RD_ERR_INVALID_ARG, "source must be exactly " + std::to_string(total) + " bytes");
    HIP_TRY(hipSetDevice(m->dev));
    HIP_TRY(hipStreamSynchronize(m->stream));
    size_t o = 0;
    for (int i = 0; i < nr; ++i) {
        HIP_TRY(hipMemcpy(r[i].dev, (const uint8_t*)src + o, r[i].bytes, hipMemcpyHostToDevice));
        o += r[i].bytes;
    }
    m->host_pos = pos;
    return RD_OK;
}

// ---------------------------------------------------------------------------
// standalone kernels
// ---------------------------------------------------------------------------
namespace {
// Scratch of the standalone attention / argmax entry points, one per device,
// allocated on first use and kept until the process ends.  Calls that overlap
// on one device race on it.
struct Scratch {
    float* part = nullptr;  // [heads][MAX_SPLITS][hd+2]
    int* pos = nullptr;
    float* av = nullptr;
    int* ai = nullptr;
    int* acnt = nullptr;
};
constexpr int SCR_HEADS = 128, SCR_HD = 128, SCR_ARG = 1024;
std::mutex g_scr_mu;
Scratch g_scr[64];

hipError_t get_scratch(Scratch** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scr_mu);
    Scratch& s = g_scr[dev];
    if (!s.part) {
        const size_t po = (size_t)SCR_HEADS * MAX_SPLITS * (SCR_HD + 2) * 4;
        const size_t tail = 256 + SCR_ARG * 8 + 256;
        void* p = nullptr;
        if ((e = hipMalloc(&p, po + tail)) != hipSuccess) return e;
        if ((e = hipMemset(p, 0, po + tail)) != hipSuccess) return e;
        uint8_t* b = (uint8_t*)p;
        s.part = (float*)b;
        s.pos = (int*)(b + po);
        s.av = (float*)(s.pos + 64);
        s.ai = (int*)(s.av + SCR_ARG);
        s.acnt = s.ai + SCR_ARG;
    }
    *out = &s;
    return hipSuccess;
}
}  // namespace

extern "C" rd_status rd_release_scratch(void) {
    std::lock_guard<std::mutex> lk(g_scr_mu);
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return fail(RD_ERR_DEVICE, "hipGetDevice failed");
    for (int d = 0; d < 64; ++d) {
        if (!g_scr[d].part) continue;
        if (hipSetDevice(d) != hipSuccess || hipDeviceSynchronize() != hipSuccess || hipFree(g_scr[d].part) != hipSuccess)
            return fail(RD_ERR_DEVICE, "releasing the scratch of device " + std::to_string(d) + " failed");
        g_scr[d] = Scratch{};
    }
    if (hipSetDevice(cur) != hipSuccess) return fail(RD_ERR_DEVICE, "hipSetDevice failed");
    return RD_OK;
}

#define K_TRY(expr)                                                                                  \
    do {                                                                                             \
        hipError_t e_ = (expr);                                                                      \
        if (e_ != hipSuccess) return fail(RD_ERR_DEVICE, std::string(#expr) + ": " + hipGetErrorString(e_)); \
    } while (0)

extern "C" rd_status rd_gemv_f16(const void* W, const void* x, float* y, int32_t N, int32_t K, int32_t batch,
                                 void* stream) {
    if (!W || !x || !y) return fail(RD_ERR_INVALID_ARG, "NULL pointer");
    if (batch != 1 && batch != 8) return fail(RD_ERR_UNSUPPORTED, "batch must be 1 or 8");
    if (batch == 1 && (N < 1 || K < 8 || K % 8 || K > 8192))
        return fail(RD_ERR_INVALID_ARG, "batch 1 needs N >= 1, 8 <= K <= 8192, K % 8 == 0");
    if (batch == 8 && (N < 1 || K < 64 || K % 64 || K > 8192))
        return fail(RD_ERR_INVALID_ARG, "batch 8 needs N >= 1, 64 <= K <= 8192, K % 64 == 0");
    if (((uintptr_t)W | (uintptr_t)x) & 15) return fail(RD_ERR_INVALID_ARG, "W and x must be 16-byte aligned");
    int dev = 0, ncu = 0;
    K_TRY(hipGetDevice(&dev));
    K_TRY(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    K_TRY(launch_gemv_f16(W, x, y, N, K, batch, ncu, (hipStream_t)stream));
    return RD_OK;
}

namespace {
// Checks and launches the step's attention (split partials, then the
// log-sum-exp merge) over a caller's cache, with the partials in `part`
// (H * splits * (hd + 2) floats) and the position word in `posw`.
rd_status attention_call(const float* q, const void* Kc, const void* Vc, const uint16_t* kst, const uint16_t* vst,
                         const float* kmeta, const float* vmeta, float* out, int32_t H, int32_t Hk, int32_t hd,
                         int32_t L, int32_t ld, int32_t kvf, float scale, int32_t splits, hipStream_t st,
                         float* part, int* posw) {
    const int G = H / Hk;
    hipLaunchKernelGGL(k_set_int, dim3(1), dim3(1), 0, st, posw, L - 1);
    K_TRY(hipGetLastError());
    AttnArgs A{};
    A.q = q;
    A.out = out;
    A.kc = Kc;
    A.vc = Vc;
    if (kvf == KV_INT8) {
        A.kst = const_cast<uint16_t*>(kst);
        A.vst = const_cast<uint16_t*>(vst);
        A.kmeta = const_cast<float*>(kmeta);
        A.vmeta = const_cast<float*>(vmeta);
    }
    A.part = part;
    A.ro = q;     // fetched in place of past-the-end rows (values never used)
    A.pos_ptr = posw;
    A.ld = ld;
    A.nseg = (ld + SEG - 1) / SEG;
    A.H = H;
    A.Hk = Hk;
    A.S = splits;
    A.scale = scale;
    A.seal = 0;   // read-only: the caller's cache is never written
    K_TRY(launch_attention(A, kvf, hd, G, st));
    return RD_OK;
}

rd_status attention_args_ok(const float* q, const void* Kc, const void* Vc, const uint16_t* kst, const uint16_t* vst,
                            const float* kmeta, const float* vmeta, const float* out, int32_t H, int32_t Hk,
                            int32_t hd, int32_t L, int32_t ld, int32_t kvf, int32_t splits) {
    if (!q || !Kc || !Vc || !out) return fail(RD_ERR_INVALID_ARG, "NULL pointer");
    if (kvf < RD_KV_FP16 || kvf > RD_KV_INT8_SEG128) return fail(RD_ERR_INVALID_ARG, "bad kv_format");
    if (kvf == RD_KV_INT8_SEG128 && (!kst || !vst || !kmeta || !vmeta))
        return fail(RD_ERR_INVALID_ARG, "the INT8 cache needs staging rows and (scale, zero point) tables");
    if (hd != 64 && hd != 128) return fail(RD_ERR_INVALID_ARG, "hd must be 64 or 128");
    if (H < 1 || Hk < 1 || H % Hk || H > SCR_HEADS) return fail(RD_ERR_INVALID_ARG, "bad head counts");
    const int G = H / Hk;
    if (G != 1 && G != 2 && G != 4 && G != 8) return fail(RD_ERR_INVALID_ARG, "n_heads/n_kv_heads must be 1, 2, 4 or 8");
    if (L < 1 || L > ld) return fail(RD_ERR_INVALID_ARG, "need 1 <= L <= ld");
    if (splits < 1 || splits > MAX_SPLITS) return fail(RD_ERR_INVALID_ARG, "splits out of range");
    if (kvf == RD_KV_INT8_SEG128 && splits < 2)
        return fail(RD_ERR_INVALID_ARG, "the INT8 cache needs at least 2 splits (the open segment has its own)");
    if ((uint64_t)Hk * ld * hd * (kvf == RD_KV_FP16 ? 2 : 1) > 0x7fffffffull)
        return fail(RD_ERR_INVALID_ARG, "n_kv_heads * ld * hd * element bytes must stay below 2 GiB");
    if (((uintptr_t)q | (uintptr_t)Kc | (uintptr_t)Vc | (uintptr_t)kst | (uintptr_t)vst) & 15)
        return fail(RD_ERR_INVALID_ARG, "q, K, V and the staging rows must be 16-byte aligned");
    if (((uintptr_t)kmeta | (uintptr_t)vmeta) & 7) return fail(RD_ERR_INVALID_ARG, "meta tables must be 8-byte aligned");
    return RD_OK;
}
}  // namespace

extern "C" rd_status rd_attention(const float* q, const void* Kc, const void* Vc, const uint16_t* kst,
                                  const uint16_t* vst, const float* kmeta, const float* vmeta, float* out, int32_t H,
                                  int32_t Hk, int32_t hd, int32_t L, int32_t ld, int32_t kv_format, float scale,
                                  int32_t splits, void* stream) {
    rd_status r = attention_args_ok(q, Kc, Vc, kst, vst, kmeta, vmeta, out, H, Hk, hd, L, ld, kv_format, splits);
    if (r) return r;
    Scratch* s = nullptr;
    K_TRY(get_scratch(&s));
    return attention_call(q, Kc, Vc, kst, vst, kmeta, vmeta, out, H, Hk, hd, L, ld, kv_format, scale, splits,
                          (hipStream_t)stream, s->part, s->pos);
}

// ---- rd_attention without any allocation ---------------------------------------
// The split partials and the position word live in a fixed device array (one
// copy per GPU, held until the process ends).  In host code `scratch` names a
// host-side stand-in, not the device copy: its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only
// that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_static_mu;
void* g_static_ptr[64];

hipError_t static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_static_mu);
    if (!g_static_ptr[dev]) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_static_ptr[dev] = p;
    }
    *out = g_static_ptr[dev];
    return hipSuccess;
}
}  // namespace

extern "C" rd_status rd_attention_noalloc(const float* q, const void* Kc, const void* Vc, const uint16_t* kst,
                                          const uint16_t* vst, const float* kmeta, const float* vmeta, float* out,
                                          int32_t H, int32_t Hk, int32_t hd, int32_t L, int32_t ld,
                                          int32_t kv_format, float scale, int32_t splits, void* stream) {
    rd_status r = attention_args_ok(q, Kc, Vc, kst, vst, kmeta, vmeta, out, H, Hk, hd, L, ld, kv_format, splits);
    if (r) return r;
    const size_t need = 256 + (size_t)H * splits * (hd + 2) * sizeof(float);
    if (need > kNoAllocScratchBytes)
        return fail(RD_ERR_INVALID_ARG, "n_heads * splits * (hd + 2) * 4 bytes of split partials exceed the " +
                                            std::to_string(kNoAllocScratchBytes - 256) + "-byte static scratch");
    void* p = nullptr;
    K_TRY(static_scratch(&p));
    uint8_t* b = (uint8_t*)p;
    return attention_call(q, Kc, Vc, kst, vst, kmeta, vmeta, out, H, Hk, hd, L, ld, kv_format, scale, splits,
                          (hipStream_t)stream, (float*)(b + 256), (int*)b);
}

extern "C" rd_status rd_attention_f16(const float* q, const void* Kc, const void* Vc, float* out, int32_t H,
                                      int32_t Hk, int32_t hd, int32_t L, int32_t ld, float scale, int32_t splits,
                                      void* stream) {
    return rd_attention(q, Kc, Vc, nullptr, nullptr, nullptr, nullptr, out, H, Hk, hd, L, ld, RD_KV_FP16, scale,
                        splits, stream);
}

extern "C" rd_status rd_q4_quantize(const void* W, int32_t N, int32_t K, uint8_t* codes, float* scales, void* stream) {
    if (!W || !codes || !scales) return fail(RD_ERR_INVALID_ARG, "NULL pointer");
    if (N < 1 || K < 128 || K % 128 || K > 8192) return fail(RD_ERR_INVALID_ARG, "need N >= 1, K a multiple of 128 in [128, 8192]");
    if (((uintptr_t)W & 15) || ((uintptr_t)codes & 3) || ((uintptr_t)scales & 3))
        return fail(RD_ERR_INVALID_ARG, "W must be 16-byte aligned, codes and scales 4-byte aligned");
    K_TRY(launch_q4_quant(W, N, K, codes, scales, (hipStream_t)stream));
    return RD_OK;
}

extern "C" rd_status rd_gemv_q4(const uint8_t* codes, const float* scales, const void* x, float* y, int32_t N,
                                int32_t K, void* stream) {
    if (!codes || !scales || !x || !y) return fail(RD_ERR_INVALID_ARG, "NULL pointer");
    if (N < 1 || K < 128 || K % 128 || K > 8192) return fail(RD_ERR_INVALID_ARG, "need N >= 1, K a multiple of 128 in [128, 8192]");
    if (((uintptr_t)codes | (uintptr_t)x) & 15) return fail(RD_ERR_INVALID_ARG, "codes and x must be 16-byte aligned");
    if ((uintptr_t)scales & 3) return fail(RD_ERR_INVALID_ARG, "scales must be 4-byte aligned");
    int dev = 0, ncu = 0;
    K_TRY(hipGetDevice(&dev));
    K_TRY(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    K_TRY(launch_gemv_q4(codes, scales, x, y, N, K, ncu, (hipStream_t)stream));
    return RD_OK;
}

extern "C" rd_status rd_e5m2_encode(const uint16_t* in, uint8_t* out, size_t n, void* stream) {
    if ((!in || !out) && n) return fail(RD_ERR_INVALID_ARG, "NULL pointer");
    K_TRY(launch_e5m2(in, out, n, (hipStream_t)stream));
    return RD_OK;
}

extern "C" rd_status rd_seg_quant(const uint16_t* in, int32_t n_seg, int32_t seg_elems, uint8_t* codes, float* meta,
                                  void* stream) {
    if (!in || !codes || !meta) return fail(RD_ERR_INVALID_ARG, "NULL pointer");
    if (n_seg < 0 || seg_elems < 8 || seg_elems % 8 || seg_elems > 65536)
        return fail(RD_ERR_INVALID_ARG, "need n_seg >= 0, seg_elems a multiple of 8 in [8, 65536]");
    if (((uintptr_t)in | (uintptr_t)codes) & 15) return fail(RD_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    K_TRY(launch_seg_quant(in, n_seg, seg_elems, codes, meta, (hipStream_t)stream));
    return RD_OK;
}

extern "C" rd_status rd_delta_seal(const uint16_t* in, int32_t n_seg, int32_t n, int32_t hd, uint16_t* anchor,
                                   uint8_t* codes, float* meta, void* stream) {
    if (!in || !anchor || !meta || (!codes && n > 1)) return fail(RD_ERR_INVALID_ARG, "NULL pointer");
    if (n_seg < 0 || n < 1 || n > 4096 || hd < 8 || hd > 1024 || hd % 8)
        return fail(RD_ERR_INVALID_ARG, "need n_seg >= 0, 1 <= n <= 4096, hd a multiple of 8 in [8, 1024]");
    if ((((uintptr_t)in | (uintptr_t)anchor) & 15) || ((uintptr_t)codes & 7))
        return fail(RD_ERR_INVALID_ARG, "in and anchor must be 16-byte aligned, codes 8-byte aligned");
    K_TRY(launch_delta_seal(in, n_seg, n, hd, anchor, codes, meta, (hipStream_t)stream));
    return RD_OK;
}

extern "C" rd_status rd_delta_restore(const uint16_t* anchor, const uint8_t* codes, const float* meta, int32_t n_seg,
                                      int32_t n, int32_t hd, float* out, void* stream) {
    if (!anchor || !meta || !out || (!codes && n > 1)) return fail(RD_ERR_INVALID_ARG, "NULL pointer");
    if (n_seg < 0 || n < 1 || n > 4096 || hd < 8 || hd > 1024 || hd % 8)
        return fail(RD_ERR_INVALID_ARG, "need n_seg >= 0, 1 <= n <= 4096, hd a multiple of 8 in [8, 1024]");
    if ((((uintptr_t)anchor | (uintptr_t)out) & 15) || ((uintptr_t)codes & 7))
        return fail(RD_ERR_INVALID_ARG, "anchor and out must be 16-byte aligned, codes 8-byte aligned");
    if ((size_t)n_seg * (hd / 8) > 0xffffffffull * 256) return fail(RD_ERR_INVALID_ARG, "too many segments");
    K_TRY(launch_delta_restore(anchor, codes, meta, n_seg, n, hd, out, (hipStream_t)stream));
    return RD_OK;
}

extern "C" rd_status rd_argmax_f32(const float* v, int32_t n, int32_t* out, void* stream) {
    if (!v || !out) return fail(RD_ERR_INVALID_ARG, "NULL pointer");
    if (n < 1) return fail(RD_ERR_INVALID_ARG, "n must be >= 1");
    Scratch* s = nullptr;
    K_TRY(get_scratch(&s));
    K_TRY(launch_argmax(v, n, out, s->av, s->ai, s->acnt, (hipStream_t)stream));
    return RD_OK;
}
