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
// (written by k_b_norm), the SwiGLU output (written in fp16 by the gate/up
// GEMM's epilogue), and the attention output, which the O GEMM converts
// from fp32 as it loads it.  The QKV GEMM's epilogue applies RoPE and
// appends each sequence's new K/V row; the residual adds are the O and down
// GEMMs accumulating into x.
#include "rd_phases.h"

namespace rd {

namespace {

constexpr int BW = 256;

// x[b] = E[token[b]] (fp32); an out-of-range token flags ERR_TOKEN and reads row 0.
// Paged cache: a token of -1 sits the step out (act[b] = 0, x[b] = 0).
__global__ __launch_bounds__(BW) void k_b_embed(StepArgs A) {
    const int b = blockIdx.x;
    int tok = A.st->token[b];
    if (A.ptab) {
        const bool on = tok != -1;
        if (threadIdx.x == 0) A.st->act[b] = on;
        if (!on) {
            for (int i = threadIdx.x; i < A.D; i += BW) A.x[(size_t)b * A.D + i] = 0.f;
            return;
        }
    }
    if (tok < 0 || tok >= A.V) {
        if (threadIdx.x == 0) atomicOr(&A.st->err, ERR_TOKEN);
        tok = 0;
    }
    const _Float16* e = A.embed + (size_t)tok * A.D;
    for (int i = threadIdx.x; i < A.D; i += BW) A.x[(size_t)b * A.D + i] = (float)e[i];
}

// xh[b] = fp16(x[b] * (mean(x[b]^2) + eps)^-1/2 * g).  D % 64 == 0 and
// D <= 4 * NV * BW: each thread holds NV float4 of the row (and the gains
// for them), all requested before the first is used; per-thread partial
// sums of squares, wave sums, then the four waves in order.
template <int NV>
__global__ __launch_bounds__(BW) void k_b_norm(const float* __restrict__ x, int D, const _Float16* __restrict__ g,
                                               float eps, _Float16* __restrict__ xh) {
    __shared__ float s_w[BW / WAVE];
    const int b = blockIdx.x, n4 = D / 4;
    const float4* xb = reinterpret_cast<const float4*>(x + (size_t)b * D);
    const uint2* gb = reinterpret_cast<const uint2*>(g);
    float4 v[NV];
    uint2 gv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {   // past the row: re-read its last float4 (not used)
        const int i = min((int)threadIdx.x + j * BW, n4 - 1);
        v[j] = xb[i];
        gv[j] = gb[i];
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if ((int)threadIdx.x + j * BW < n4) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    ss = wave_sum(ss);
    if (lane_id() == 0) s_w[wave_id()] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < BW / WAVE; ++w) tot += s_w[w];
    const float inv = 1.0f / sqrtf(tot / (float)D + eps);
    uint2* ob = reinterpret_cast<uint2*>(xh + (size_t)b * D);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = (int)threadIdx.x + j * BW;
        if (i < n4) {
            const h4 gh = __builtin_bit_cast(h4, gv[j]);
            const h4 o = h4{(_Float16)(v[j].x * inv * (float)gh[0]), (_Float16)(v[j].y * inv * (float)gh[1]),
                            (_Float16)(v[j].z * inv * (float)gh[2]), (_Float16)(v[j].w * inv * (float)gh[3])};
            ob[i] = __builtin_bit_cast(uint2, o);
        }
    }
}

hipError_t norm_rows(const float* x, int D, const _Float16* g, float eps, _Float16* xh, int B, hipStream_t s) {
    const int n4 = D / 4;
    if (n4 <= BW) hipLaunchKernelGGL(k_b_norm<1>, dim3(B), dim3(BW), 0, s, x, D, g, eps, xh);
    else if (n4 <= 2 * BW) hipLaunchKernelGGL(k_b_norm<2>, dim3(B), dim3(BW), 0, s, x, D, g, eps, xh);
    else if (n4 <= 4 * BW) hipLaunchKernelGGL(k_b_norm<4>, dim3(B), dim3(BW), 0, s, x, D, g, eps, xh);
    else hipLaunchKernelGGL(k_b_norm<8>, dim3(B), dim3(BW), 0, s, x, D, g, eps, xh);
    return hipGetLastError();
}

// Greedy argmax of sequence b's logits (lowest index on ties; a non-finite
// logit flags ERR_NONFINITE): token[b], and gen_out[n_gen*B + b].  1024
// threads, each with AU logits requested at a time (the ranking is a total
// order, so the split of the row does not change the winner).
constexpr int BWA = 1024, AU = 16;
__global__ __launch_bounds__(BWA) void k_b_argmax(StepArgs A) {
    __shared__ float s_v[BWA / WAVE];
    __shared__ int s_i[BWA / WAVE];
    const int b = blockIdx.x, V = A.V;
    if (A.ptab && !A.st->act[b]) return;   // sat the step out: token stays -1
    const float* lg = A.logits + (size_t)b * V;
    Best best{-INFINITY, INT_MAX};
    bool bad = false;
    for (int base = 0; base < V; base += BWA * AU) {
        float v[AU];
#pragma unroll
        for (int k = 0; k < AU; ++k) v[k] = lg[min(base + k * BWA + (int)threadIdx.x, V - 1)];
#pragma unroll
        for (int k = 0; k < AU; ++k) {
            const int i = base + k * BWA + (int)threadIdx.x;
            if (i < V) {
                bad |= !isfinite(v[k]);
                best = better(best, Best{v[k], i});
            }
        }
    }
    if (bad) atomicOr(&A.st->err, ERR_NONFINITE);
    best = wave_best(best);
    if (lane_id() == 0) {
        s_v[wave_id()] = best.v;
        s_i[wave_id()] = best.i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        Best fin{s_v[0], s_i[0]};
        for (int w = 1; w < BWA / WAVE; ++w) fin = better(fin, Best{s_v[w], s_i[w]});
        A.st->token[b] = fin.i;
        const int n = A.st->n_gen;
        if (n < A.max_ctx) A.gen_out[(size_t)n * A.B + b] = fin.i;
    }
}

__global__ void k_b_advance(StepState* st, int B, int paged) {
    st->n_gen += 1;
    st->pos += 1;
    if (paged)
        for (int b = 0; b < B; ++b) st->bpos[b] += st->act[b];
}

// Paged cache, copy on write: page group src copied to dst.  For every
// (layer, K/V) the Hk pages of a group are contiguous (Hk * 4 KiB).
__global__ __launch_bounds__(BW) void k_page_copy(StepArgs A, int src, int dst) {
    const int l = blockIdx.x >> 1;
    uint8_t* pool = reinterpret_cast<uint8_t*>((blockIdx.x & 1) ? A.vc : A.kc);
    const size_t blk = (size_t)A.Hk * 4096;
    const uint4* sp = reinterpret_cast<const uint4*>(pool + ((size_t)l * A.npages + src) * blk);
    uint4* dp = reinterpret_cast<uint4*>(pool + ((size_t)l * A.npages + dst) * blk);
    for (size_t i = threadIdx.x; i < blk / 16; i += BW) dp[i] = sp[i];
}

}  // namespace

hipError_t launch_page_copy(const StepArgs& A, int src, int dst, hipStream_t s) {
    hipLaunchKernelGGL(k_page_copy, dim3(2 * A.n_layers), dim3(BW), 0, s, A, src, dst);
    return hipGetLastError();
}

#define B_TRY(expr)                          \
    do {                                     \
        hipError_t e_ = (expr);              \
        if (e_ != hipSuccess) return e_;     \
    } while (0)

hipError_t launch_step_batch(const StepArgs& A, hipStream_t s) {
    const int B = A.B, D = A.D, HD = A.H * A.hd, F = A.F;
    hipLaunchKernelGGL(k_b_embed, dim3(B), dim3(BW), 0, s, A);
    B_TRY(hipGetLastError());
    for (int l = 0; l < A.n_layers; ++l) {
        const LayerW& Lw = A.layers[l];
        B_TRY(norm_rows(A.x, D, Lw.g_attn, A.eps, A.xh, B, s));
        B_TRY(launch_gemm_b8_qkv(A, l, Lw.wqkv, s));
        B_TRY(launch_attn_any(attn_args(A, l), A.kvfmt, A.hd, A.H / A.Hk, s));
        B_TRY(launch_gemm_b8(Lw.wo, A.a, true, HD, A.x, D, true, D, HD, B, A.ncu, s));
        B_TRY(norm_rows(A.x, D, Lw.g_ffn, A.eps, A.xh, B, s));
        _Float16* mh = reinterpret_cast<_Float16*>(A.m);   // [B][F] fp16 in the fp32 buffer's space
        B_TRY(launch_gemm_b8_swiglu(Lw.wgu, A.xh, D, mh, F, F, D, B, A.ncu, s));
        B_TRY(launch_gemm_b8(Lw.wd, mh, false, F, A.x, D, true, D, F, B, A.ncu, s));
    }
    B_TRY(norm_rows(A.x, D, A.g_final, A.eps, A.xh, B, s));
    B_TRY(launch_gemm_b8(A.lm_head, A.xh, false, D, A.logits, A.V, false, A.V, D, B, A.ncu, s));
    hipLaunchKernelGGL(k_b_argmax, dim3(B), dim3(BWA), 0, s, A);
    B_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_b_advance, dim3(1), dim3(1), 0, s, A.st, B, A.ptab ? 1 : 0);
    return hipGetLastError();
}

}  // namespace rd
