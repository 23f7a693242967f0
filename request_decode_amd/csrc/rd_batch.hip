// The decode step for B (2..8) sequences in lockstep, on the kernel-per-phase
// executors: every GEMV becomes a thin GEMM Y[B][N] = W[N][K] X[B][K] on the
// matrix cores (k_gemm_b8 in rd_gemv.hip: 8 FLOP per weight byte at B = 8,
// still HBM-bound), attention runs per sequence over its own cache (the
// split kernels with a sequence grid dimension), and the argmax is taken per
// sequence ("Real-time LLM inference on standard GPUs: 3,000 tokens/s per
// request", section "Memory bandwidth is the main bottleneck": batching
// shares each weight byte among the sequences).
//
// The GEMM inputs are fp16: the RMSNorm output of the QKV and gate/up GEMMs
// (written by k_b_norm), and the attention output and SwiGLU output, which
// the GEMM converts from fp32 as it loads them.  The residual adds are the
// O and down GEMMs accumulating into x.
#include "rd_phases.h"

namespace rd {

namespace {

constexpr int BW = 256;

// x[b] = E[token[b]] (fp32); an out-of-range token flags ERR_TOKEN and reads row 0.
__global__ __launch_bounds__(BW) void k_b_embed(StepArgs A) {
    const int b = blockIdx.x;
    int tok = A.st->token[b];
    if (tok < 0 || tok >= A.V) {
        if (threadIdx.x == 0) atomicOr(&A.st->err, ERR_TOKEN);
        tok = 0;
    }
    const _Float16* e = A.embed + (size_t)tok * A.D;
    for (int i = threadIdx.x; i < A.D; i += BW) A.x[(size_t)b * A.D + i] = (float)e[i];
}

// xh[b] = fp16(x[b] * (mean(x[b]^2) + eps)^-1/2 * g): thread-strided partial
// sums of squares, wave sums, then the four waves in order.
__global__ __launch_bounds__(BW) void k_b_norm(const float* __restrict__ x, int D, const _Float16* __restrict__ g,
                                               float eps, _Float16* __restrict__ xh) {
    __shared__ float s_w[BW / WAVE];
    const int b = blockIdx.x;
    const float* xb = x + (size_t)b * D;
    float ss = 0.f;
    for (int i = threadIdx.x; i < D; i += BW) ss += xb[i] * xb[i];
    ss = wave_sum(ss);
    if (lane_id() == 0) s_w[wave_id()] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < BW / WAVE; ++w) tot += s_w[w];
    const float inv = 1.0f / sqrtf(tot / (float)D + eps);
    for (int i = threadIdx.x; i < D; i += BW) xh[(size_t)b * D + i] = (_Float16)(xb[i] * inv * (float)g[i]);
}

// RoPE pairs of the QKV GEMM output y[b] (re-ordered rows) and the cache
// append of sequence b (blockIdx.y): one thread per row pair.
template <int KVF>
__global__ __launch_bounds__(BW) void k_b_qkv_epi(StepArgs A, int layer) {
    const int b = blockIdx.y, p = blockIdx.x * BW + threadIdx.x;
    const int N = (A.H + 2 * A.Hk) * A.hd;
    if (2 * p >= N) return;
    const int pos = A.st->pos;
    const float* y = A.y + (size_t)b * N;
    const QkvPair o = qkv_pair(A.hd, A.H, A.Hk, 2 * p, y[2 * p], y[2 * p + 1], A.rope + (size_t)pos * (A.hd / 2));
    if (o.kind == 0) {
        float* q = A.q + (size_t)b * A.H * A.hd;
        q[o.head * A.hd + o.d0] = o.y0;
        q[o.head * A.hd + o.d1] = o.y1;
    } else {
        StepArgs Ab = A;   // sequence b's cache
        Ab.kc = reinterpret_cast<uint8_t*>(A.kc) + (size_t)b * A.kv_bstride;
        Ab.vc = reinterpret_cast<uint8_t*>(A.vc) + (size_t)b * A.kv_bstride;
        if (A.stage) {
            Ab.stage = A.stage + (size_t)b * A.st_bstride;
            Ab.meta = A.meta + (size_t)b * A.meta_bstride;
        }
        const int which = o.kind == 2;
        kv_put<KVF, false>(Ab, layer, which, o.head, pos, o.d0, o.y0);
        kv_put<KVF, false>(Ab, layer, which, o.head, pos, o.d1, o.y1);
    }
}

// m[b][i] = silu(y[b][2i]) * y[b][2i+1] (gate/up rows interleaved).
__global__ __launch_bounds__(BW) void k_b_swiglu(const float* __restrict__ y, float* __restrict__ m, int F) {
    const int b = blockIdx.y, i = blockIdx.x * BW + threadIdx.x;
    if (i >= F) return;
    const float* yb = y + (size_t)b * 2 * F;
    m[(size_t)b * F + i] = silu_mul(yb[2 * i], yb[2 * i + 1]);
}

// Greedy argmax of sequence b's logits (lowest index on ties; a non-finite
// logit flags ERR_NONFINITE): token[b], and gen_out[n_gen*B + b].
__global__ __launch_bounds__(BW) void k_b_argmax(StepArgs A) {
    const int b = blockIdx.x;
    const float* lg = A.logits + (size_t)b * A.V;
    Best best{-INFINITY, INT_MAX};
    bool bad = false;
    for (int i = threadIdx.x; i < A.V; i += BW) {
        const float v = lg[i];
        bad |= !isfinite(v);
        best = better(best, Best{v, i});
    }
    if (bad) atomicOr(&A.st->err, ERR_NONFINITE);
    const Best fin = block_best(best);
    if (threadIdx.x == 0) {
        A.st->token[b] = fin.i;
        const int n = A.st->n_gen;
        if (n < A.max_ctx) A.gen_out[(size_t)n * A.B + b] = fin.i;
    }
}

__global__ void k_b_advance(StepState* st) {
    st->n_gen += 1;
    st->pos += 1;
}

template <int KVF>
hipError_t qkv_epi(const StepArgs& A, int layer, hipStream_t s) {
    const int pairs = (A.H + 2 * A.Hk) * A.hd / 2;
    hipLaunchKernelGGL(k_b_qkv_epi<KVF>, dim3((pairs + BW - 1) / BW, A.B), dim3(BW), 0, s, A, layer);
    return hipGetLastError();
}

}  // namespace

#define B_TRY(expr)                          \
    do {                                     \
        hipError_t e_ = (expr);              \
        if (e_ != hipSuccess) return e_;     \
    } while (0)

hipError_t launch_step_batch(const StepArgs& A, hipStream_t s) {
    const int B = A.B, D = A.D, HD = A.H * A.hd, F = A.F, Nqkv = (A.H + 2 * A.Hk) * A.hd;
    hipLaunchKernelGGL(k_b_embed, dim3(B), dim3(BW), 0, s, A);
    B_TRY(hipGetLastError());
    for (int l = 0; l < A.n_layers; ++l) {
        const LayerW& Lw = A.layers[l];
        hipLaunchKernelGGL(k_b_norm, dim3(B), dim3(BW), 0, s, A.x, D, Lw.g_attn, A.eps, A.xh);
        B_TRY(hipGetLastError());
        B_TRY(launch_gemm_b8(Lw.wqkv, A.xh, false, D, A.y, Nqkv, false, Nqkv, D, B, A.ncu, s));
        switch (A.kvfmt) {
            case KV_FP16: B_TRY(qkv_epi<KV_FP16>(A, l, s)); break;
            case KV_E5M2: B_TRY(qkv_epi<KV_E5M2>(A, l, s)); break;
            default: B_TRY(qkv_epi<KV_INT8>(A, l, s)); break;
        }
        B_TRY(launch_attn_any(attn_args(A, l), A.kvfmt, A.hd, A.H / A.Hk, s));
        B_TRY(launch_gemm_b8(Lw.wo, A.a, true, HD, A.x, D, true, D, HD, B, A.ncu, s));
        hipLaunchKernelGGL(k_b_norm, dim3(B), dim3(BW), 0, s, A.x, D, Lw.g_ffn, A.eps, A.xh);
        B_TRY(hipGetLastError());
        B_TRY(launch_gemm_b8(Lw.wgu, A.xh, false, D, A.y, 2 * F, false, 2 * F, D, B, A.ncu, s));
        hipLaunchKernelGGL(k_b_swiglu, dim3((F + BW - 1) / BW, B), dim3(BW), 0, s, A.y, A.m, F);
        B_TRY(hipGetLastError());
        B_TRY(launch_gemm_b8(Lw.wd, A.m, true, F, A.x, D, true, D, F, B, A.ncu, s));
    }
    hipLaunchKernelGGL(k_b_norm, dim3(B), dim3(BW), 0, s, A.x, D, A.g_final, A.eps, A.xh);
    B_TRY(hipGetLastError());
    B_TRY(launch_gemm_b8(A.lm_head, A.xh, false, D, A.logits, A.V, false, A.V, D, B, A.ncu, s));
    hipLaunchKernelGGL(k_b_argmax, dim3(B), dim3(BW), 0, s, A);
    B_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_b_advance, dim3(1), dim3(1), 0, s, A.st);
    return hipGetLastError();
}

}  // namespace rd
