// Decode-step kernels for gfx950 (CDNA4, wave64).
//
// The step is memory-bound: at batch 1 every weight byte is read once per
// token for about one multiply-add ("Real-time LLM inference on standard
// GPUs: 3,000 tokens/s per request", section "Memory bandwidth is the main
// bottleneck").  Every kernel here is therefore built around streaming its
// weights through HBM with 16-byte coalesced loads, one wavefront per small
// block of rows, the input vector held in registers, and the small
// non-GEMV work (RMSNorm, RoPE, cache append, SwiGLU, residual add, argmax)
// fused into the GEMV that produces or consumes it, so that no extra pass
// over memory and no extra launch is spent on it (the same page's table of
// microsecond losses: non-GEMM work stalling the memory stream; and the
// fusion of attention-side RoPE and normalisation in "How the xAI
// engineering team cut Grok Bot latency to milliseconds", §3.1).
#include <float.h>
#include <limits.h>
#include <math.h>

#include "rd_device.h"
#include "rd_internal.h"

namespace rd {

// ============================================================================
// GEMV building blocks
// ============================================================================
// A length-K input vector is spread over the 64 lanes of a wave in chunks of
// 8 consecutive elements: chunk c of lane l covers columns (c*64+l)*8..+7, the
// same columns the lane reads from every weight row (16 bytes of fp16), so a
// wave-wide load of one chunk of one row is a single fully coalesced 1 KiB
// read.  KCH chunks cover K <= KCH*512; columns past K are zero.

template <int KCH>
__device__ __forceinline__ void load_x_f32(const float* __restrict__ x, int K, float (&xr)[KCH][8]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        if (col < K) {
            const float4 a = *reinterpret_cast<const float4*>(x + col);
            const float4 b = *reinterpret_cast<const float4*>(x + col + 4);
            xr[c][0] = a.x; xr[c][1] = a.y; xr[c][2] = a.z; xr[c][3] = a.w;
            xr[c][4] = b.x; xr[c][5] = b.y; xr[c][6] = b.z; xr[c][7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xr[c][i] = 0.f;
        }
    }
}

template <int KCH>
__device__ __forceinline__ void load_x_f16(const _Float16* __restrict__ x, int K, float (&xr)[KCH][8]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        if (col < K) {
            const h8 v = as_h8(ld16(x + col));
#pragma unroll
            for (int i = 0; i < 8; ++i) xr[c][i] = (float)v[i];
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xr[c][i] = 0.f;
        }
    }
}

// RMSNorm of the register-resident vector: x * (mean(x^2) + eps)^-1/2 * g.
// Every wave holds the whole vector, so each wave normalises on its own and
// no workgroup synchronisation is needed.
template <int KCH>
__device__ __forceinline__ void rmsnorm_regs(float (&xr)[KCH][8], const _Float16* __restrict__ g, int K, float eps) {
    const int lane = threadIdx.x & 63;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < KCH; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += xr[c][i] * xr[c][i];
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)K + eps);
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        if (col < K) {
            const h8 gv = as_h8(ld16(g + col));
#pragma unroll
            for (int i = 0; i < 8; ++i) xr[c][i] = xr[c][i] * inv * (float)gv[i];
        }
    }
}

// acc[r] = W[row0+r, :] . x for R consecutive rows of a row-major [*, K] fp16
// matrix.  All R*KCH loads are issued before the first multiply so that a
// wave keeps R*KCH KiB in flight; rows >= nvalid are skipped.
template <int R, int KCH>
__device__ __forceinline__ void dot_rows(const _Float16* __restrict__ W, int K, int row0, int nvalid,
                                         const float (&xr)[KCH][8], float (&acc)[R]) {
    const int lane = threadIdx.x & 63;
    u4v w[R][KCH];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int col = (c * 64 + lane) * 8;
            if (r < nvalid && col < K)
                w[r][c] = ld_w16(W + (size_t)(row0 + r) * K + col);
            else
                w[r][c] = u4v{0u, 0u, 0u, 0u};
        }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const h8 hw = as_h8(w[r][c]);
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                s0 += (float)hw[i] * xr[c][i];
                s1 += (float)hw[i + 1] * xr[c][i + 1];
            }
        }
        acc[r] = wave_sum(s0 + s1);
    }
}

// ============================================================================
// Phase 1: RMSNorm + fused QKV GEMV + RoPE + KV append
// ============================================================================
// Rows of the fused QKV matrix are re-ordered at load time so that each
// wave's two rows are a RoPE pair (j, j+hd/2) of one q or k head (or two
// consecutive rows of a v head): the rotation and the cache write happen in
// the GEMV epilogue with both halves of the pair in the same wave.

template <int KVF>
__device__ __forceinline__ void store_kv(const StepArgs& A, int layer, int which, int g, int pos, int d, float v) {
    const uint16_t h = f2h_bits(v);
    const size_t idx = (((size_t)layer * A.Hk + g) * A.max_ctx + pos) * A.hd + d;
    void* base = which ? A.vc : A.kc;
    if constexpr (KVF == KV_FP16) {
        reinterpret_cast<uint16_t*>(base)[idx] = h;
    } else if constexpr (KVF == KV_E5M2) {
        reinterpret_cast<uint8_t*>(base)[idx] = e5m2_encode(h);
    } else {
        A.stage[((((size_t)layer * 2 + which) * A.Hk + g) * SEG + pos % SEG) * A.hd + d] = h;
    }
}

template <int KCH, bool EMB, int KVF>
__global__ __launch_bounds__(WG) void k_qkv(StepArgs A, LayerW Lw, int layer) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int D = A.D, hd = A.hd;
    const int pos = A.st->pos;
    float xr[KCH][8];
    if constexpr (EMB) {
        int tok = A.st->token[0];
        if (tok < 0 || tok >= A.V) {
            if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&A.st->err, ERR_TOKEN);
            tok = 0;
        }
        const _Float16* e = A.embed + (size_t)tok * D;
        load_x_f16<KCH>(e, D, xr);
        if (blockIdx.x == 0)
            for (int i = threadIdx.x; i < D; i += WG) A.x[i] = (float)e[i];
    } else {
        load_x_f32<KCH>(A.x, D, xr);
    }
    rmsnorm_regs<KCH>(xr, Lw.g_attn, D, A.eps);

    const int Nq = A.H * hd, Nk = A.Hk * hd, N = Nq + 2 * Nk;
    const int row0 = (blockIdx.x * 4 + wid) * 2;
    if (row0 >= N) return;
    float acc[2];
    dot_rows<2, KCH>(Lw.wqkv, D, row0, 2, xr, acc);
    if (lane != 0) return;
    if (row0 < Nq + Nk) {
        const bool isq = row0 < Nq;
        const int rho = isq ? row0 : row0 - Nq;
        const int head = rho / hd, j = (rho % hd) >> 1;
        const float2 cs = A.rope[(size_t)pos * (hd / 2) + j];
        const float y0 = acc[0] * cs.x - acc[1] * cs.y;
        const float y1 = acc[0] * cs.y + acc[1] * cs.x;
        if (isq) {
            A.q[head * hd + j] = y0;
            A.q[head * hd + j + hd / 2] = y1;
        } else {
            store_kv<KVF>(A, layer, 0, head, pos, j, y0);
            store_kv<KVF>(A, layer, 0, head, pos, j + hd / 2, y1);
        }
    } else {
        const int rho = row0 - Nq - Nk;
        const int head = rho / hd, d = rho % hd;
        store_kv<KVF>(A, layer, 1, head, pos, d, acc[0]);
        store_kv<KVF>(A, layer, 1, head, pos, d + 1, acc[1]);
    }
}

// ============================================================================
// Phase 2: single-query attention, split along the key axis, LSE merge
// ============================================================================
// Workgroup (g, s) handles kv-head g and key range s, for all G query heads
// that share g (the K/V rows are read once for the group).  A K/V row of hd
// fp16 is spread over hd/8 lanes (16 bytes each), so a wave covers
// 64/(hd/8) rows per load and each lane keeps an online softmax state
// (running max m, sum l, 8 output dims) for its rows.  The per-lane states
// are merged through LDS into one partial (m, l, o[hd]) per (head, split);
// the last workgroup of head group g to arrive merges the splits:
//   M = max_s m_s,  out = sum_s e^(m_s-M) o_s / sum_s e^(m_s-M) l_s.
// Splits are at least 64 keys long; splits past the end only arrive.

template <int KVF, int HD>
__device__ __forceinline__ void load_kv_row(const AttnArgs& A, int which, int g, int p, int open0, int sl,
                                            float (&f)[8]) {
    const size_t row = (size_t)g * A.ld + p;
    const void* base = which ? A.vc : A.kc;
    if constexpr (KVF == KV_FP16) {
        const h8 v = as_h8(ld16(reinterpret_cast<const _Float16*>(base) + row * HD + sl * 8));
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
    } else if constexpr (KVF == KV_E5M2) {
        const u2v u = ld8(reinterpret_cast<const uint8_t*>(base) + row * HD + sl * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (float)e5m2_decode((uint8_t)((u[i >> 2] >> ((i & 3) * 8)) & 0xffu));
    } else {
        if (p < open0) {
            const u2v u = ld8(reinterpret_cast<const uint8_t*>(base) + row * HD + sl * 8);
            const float* mt = (which ? A.vmeta : A.kmeta) + ((size_t)g * A.nseg + p / SEG) * 2;
            const float scale = mt[0], zp = mt[1];
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = ((float)((u[i >> 2] >> ((i & 3) * 8)) & 0xffu) - zp) * scale;
        } else {
            const uint16_t* st = which ? A.vst : A.kst;
            const h8 v = as_h8(ld16(st + ((size_t)g * SEG + p % SEG) * HD + sl * 8));
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
        }
    }
}

// Block-wide min and max (256 threads).
__device__ __forceinline__ void block_minmax(float& mn, float& mx, float* sm /* [8] */) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o, WAVE));
        mx = fmaxf(mx, __shfl_xor(mx, o, WAVE));
    }
    const int wid = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        sm[wid] = mn;
        sm[4 + wid] = mx;
    }
    __syncthreads();
    mn = fminf(fminf(sm[0], sm[1]), fminf(sm[2], sm[3]));
    mx = fmaxf(fmaxf(sm[4], sm[5]), fmaxf(sm[6], sm[7]));
}

// Adaptive-range quantization of one segment of n fp16 values ("Grok-3
// v3.2.4 hot update deep dive", §3.2): scale = (max-min)/255,
// zp = round(-min/scale), code = clamp(round(x/scale) + zp, 0, 255), all in
// fp32 with IEEE division and round-half-to-even (v_rndne).  n % 2048 == 0.
__device__ void quantize_segment(const uint16_t* __restrict__ in, int n, uint8_t* __restrict__ codes,
                                 float* __restrict__ meta) {
    __shared__ float sm[8];
    float mn = INFINITY, mx = -INFINITY;
    for (int i = threadIdx.x * 8; i < n; i += WG * 8) {
        const h8 v = as_h8(ld16(in + i));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            mn = fminf(mn, (float)v[j]);
            mx = fmaxf(mx, (float)v[j]);
        }
    }
    block_minmax(mn, mx, sm);
    float scale = (mx - mn) / 255.0f;
    if (!(scale > 0.0f)) scale = 1.0f;
    const float zp = rintf(-mn / scale);
    for (int i = threadIdx.x * 8; i < n; i += WG * 8) {
        const h8 v = as_h8(ld16(in + i));
        unsigned lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float q = fminf(fmaxf(rintf((float)v[j] / scale) + zp, 0.0f), 255.0f);
            const unsigned c = (unsigned)q;
            if (j < 4) lo |= c << (8 * j); else hi |= c << (8 * (j - 4));
        }
        *reinterpret_cast<u2v*>(codes + i) = u2v{lo, hi};
    }
    if (threadIdx.x == 0) {
        meta[0] = scale;
        meta[1] = zp;
    }
}

template <int HD, int G, int KVF>
__global__ __launch_bounds__(WG) void k_attn(AttnArgs A) {
    constexpr int LPR = HD / 8;       // lanes per K/V row
    constexpr int SLOTS = WG / LPR;   // rows per pass of the workgroup
    constexpr int U = 4;              // passes in flight
    __shared__ float sm_m[G][SLOTS], sm_l[G][SLOTS];
    __shared__ float sm_o[G][SLOTS][HD];
    __shared__ int sm_last;
    const int tid = threadIdx.x, sl = tid % LPR, rs = tid / LPR;
    const int g = blockIdx.x / A.S, s = blockIdx.x % A.S;
    const int pos = *A.pos_ptr, L = pos + 1;
    int chunk = (L + A.S - 1) / A.S;
    chunk = (chunk + 63) & ~63;
    const int nact = (L + chunk - 1) / chunk;

    if (s < nact) {
        const int p0 = s * chunk, p1 = min(L, p0 + chunk);
        const int open0 = pos / SEG * SEG;
        float qv[G][8], m[G], l[G], o[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float* qp = A.q + (size_t)(g * G + h) * HD + sl * 8;
            const float4 a = *reinterpret_cast<const float4*>(qp);
            const float4 b = *reinterpret_cast<const float4*>(qp + 4);
            qv[h][0] = a.x * A.scale; qv[h][1] = a.y * A.scale; qv[h][2] = a.z * A.scale; qv[h][3] = a.w * A.scale;
            qv[h][4] = b.x * A.scale; qv[h][5] = b.y * A.scale; qv[h][6] = b.z * A.scale; qv[h][7] = b.w * A.scale;
            m[h] = -INFINITY;
            l[h] = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
        }
        for (int pb = p0; pb < p1; pb += SLOTS * U) {
            float kf[U][8], vf[U][8];
            bool valid[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = pb + u * SLOTS + rs;
                valid[u] = p < p1;
                const int pc = valid[u] ? p : p1 - 1;   // in-range row; its weight is dropped below
                load_kv_row<KVF, HD>(A, 0, g, pc, open0, sl, kf[u]);
                load_kv_row<KVF, HD>(A, 1, g, pc, open0, sl, vf[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float d = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) d += qv[h][i] * kf[u][i];
                    d = group_sum<LPR>(d);
                    if (valid[u]) {
                        const float mn = fmaxf(m[h], d);
                        const float c = expf(m[h] - mn);
                        const float e = expf(d - mn);
                        l[h] = l[h] * c + e;
#pragma unroll
                        for (int i = 0; i < 8; ++i) o[h][i] = o[h][i] * c + e * vf[u][i];
                        m[h] = mn;
                    }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (sl == 0) {
                sm_m[h][rs] = m[h];
                sm_l[h][rs] = l[h];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) sm_o[h][rs][sl * 8 + i] = o[h][i];
        }
        __syncthreads();
        for (int t = tid; t < G * HD; t += WG) {
            const int h = t / HD, d = t % HD;
            float M = -INFINITY;
            for (int r = 0; r < SLOTS; ++r) M = fmaxf(M, sm_m[h][r]);
            float num = 0.f, den = 0.f;
            for (int r = 0; r < SLOTS; ++r) {
                if (sm_m[h][r] == -INFINITY) continue;    // slot saw no key
                const float w = expf(sm_m[h][r] - M);
                num += w * sm_o[h][r][d];
                den += w * sm_l[h][r];
            }
            const size_t ps = (size_t)(g * G + h) * MAX_SPLITS + s;
            A.part_o[ps * HD + d] = num;
            if (d == 0) {
                A.part_ml[ps * 2 + 0] = M;
                A.part_ml[ps * 2 + 1] = den;
            }
        }
    }
    // arrival: the last workgroup of group g merges
    __threadfence();
    __syncthreads();
    if (tid == 0) sm_last = (atomic_add_acqrel(&A.cnt[g], 1) == A.S - 1);
    __syncthreads();
    if (!sm_last) return;
    __threadfence();
    for (int t = tid; t < G * HD; t += WG) {
        const int h = t / HD, d = t % HD;
        const size_t pb = (size_t)(g * G + h) * MAX_SPLITS;
        float M = -INFINITY;
        for (int s2 = 0; s2 < nact; ++s2) M = fmaxf(M, A.part_ml[(pb + s2) * 2]);
        float num = 0.f, den = 0.f;
        for (int s2 = 0; s2 < nact; ++s2) {
            const float w = expf(A.part_ml[(pb + s2) * 2] - M);
            num += w * A.part_o[(pb + s2) * HD + d];
            den += w * A.part_ml[(pb + s2) * 2 + 1];
        }
        A.out[(size_t)(g * G + h) * HD + d] = num / den;
    }
    if (tid == 0) store_relaxed(&A.cnt[g], 0);
    if constexpr (KVF == KV_INT8) {
        if ((pos + 1) % SEG == 0) {
            // the segment that just filled is sealed once, after this step's attention read it
            const int seg = pos / SEG;
            const size_t rows = (size_t)g * A.ld + (size_t)seg * SEG;
            __syncthreads();
            quantize_segment(A.kst + (size_t)g * SEG * HD, SEG * HD, reinterpret_cast<uint8_t*>(A.kc) + rows * HD,
                             A.kmeta + ((size_t)g * A.nseg + seg) * 2);
            __syncthreads();
            quantize_segment(A.vst + (size_t)g * SEG * HD, SEG * HD, reinterpret_cast<uint8_t*>(A.vc) + rows * HD,
                             A.vmeta + ((size_t)g * A.nseg + seg) * 2);
        }
    }
}

// ============================================================================
// Phases 3 and 5: GEMV + residual add  (x[row] += W[row,:] . in)
// ============================================================================
template <int KCH, int R>
__global__ __launch_bounds__(WG) void k_resid(const float* __restrict__ in, int K, const _Float16* __restrict__ W,
                                              float* __restrict__ x, int N) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    float xr[KCH][8];
    load_x_f32<KCH>(in, K, xr);
    const int row0 = (blockIdx.x * 4 + wid) * R;
    if (row0 >= N) return;
    float acc[R];
    dot_rows<R, KCH>(W, K, row0, min(R, N - row0), xr, acc);
    if (lane == 0)
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (row0 + r < N) x[row0 + r] += acc[r];
}

// ============================================================================
// Phase 4: RMSNorm + gate/up GEMV + SwiGLU  (m_i = silu(gate_i) * up_i)
// ============================================================================
template <int KCH>
__global__ __launch_bounds__(WG) void k_gateup(StepArgs A, LayerW Lw) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    float xr[KCH][8];
    load_x_f32<KCH>(A.x, A.D, xr);
    rmsnorm_regs<KCH>(xr, Lw.g_ffn, A.D, A.eps);
    const int row0 = (blockIdx.x * 4 + wid) * 2;
    if (row0 >= 2 * A.F) return;
    float acc[2];
    dot_rows<2, KCH>(Lw.wgu, A.D, row0, 2, xr, acc);
    if (lane == 0) {
        const float gt = acc[0];
        A.m[row0 >> 1] = gt / (1.0f + expf(-gt)) * acc[1];
    }
}

// ============================================================================
// Phase 6: final RMSNorm + LM head + greedy argmax (on the device)
// ============================================================================
struct Best {
    float v;
    int i;
};
__device__ __forceinline__ Best better(Best a, Best b) {
    // larger value wins; equal values: lower index (greedy ties -> lowest id)
    return (a.v > b.v || (a.v == b.v && a.i < b.i)) ? a : b;
}
__device__ __forceinline__ Best wave_best(Best b) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        Best c{__shfl_xor(b.v, o, WAVE), __shfl_xor(b.i, o, WAVE)};
        b = better(b, c);
    }
    return b;
}
// Block-wide best of per-thread candidates; result valid in thread 0.
__device__ __forceinline__ Best block_best(Best b) {
    __shared__ float sv[4];
    __shared__ int si[4];
    b = wave_best(b);
    const int wid = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        sv[wid] = b.v;
        si[wid] = b.i;
    }
    __syncthreads();
    Best r{sv[0], si[0]};
    for (int w = 1; w < 4; ++w) r = better(r, Best{sv[w], si[w]});
    return r;
}

// Reduction of per-workgroup (value, index) partials by the last workgroup
// to arrive; returns true in the workgroup that holds the final answer.
__device__ __forceinline__ bool argmax_finish(Best mine, float* pv, int* pi, int* cnt, Best* out) {
    __shared__ int sm_last;
    if (threadIdx.x == 0) {
        pv[blockIdx.x] = mine.v;
        pi[blockIdx.x] = mine.i;
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) sm_last = (atomic_add_acqrel(cnt, 1) == (int)gridDim.x - 1);
    __syncthreads();
    if (!sm_last) return false;
    __threadfence();
    Best b{-INFINITY, INT_MAX};
    for (int i = threadIdx.x; i < (int)gridDim.x; i += WG) b = better(b, Best{pv[i], pi[i]});
    *out = block_best(b);
    if (threadIdx.x == 0) store_relaxed(cnt, 0);
    return true;
}

template <int KCH>
__global__ __launch_bounds__(WG) void k_lmhead(StepArgs A) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    float xr[KCH][8];
    load_x_f32<KCH>(A.x, A.D, xr);
    rmsnorm_regs<KCH>(xr, A.g_final, A.D, A.eps);
    const int row0 = (blockIdx.x * 4 + wid) * 2;
    Best b{-INFINITY, INT_MAX};
    if (row0 < A.V) {
        float acc[2];
        const int nv = min(2, A.V - row0);
        dot_rows<2, KCH>(A.lm_head, A.D, row0, nv, xr, acc);
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                if (r < nv) {
                    A.logits[row0 + r] = acc[r];
                    if (!isfinite(acc[r])) atomicOr(&A.st->err, ERR_NONFINITE);
                    b = better(b, Best{acc[r], row0 + r});
                }
            }
        }
    }
    b = block_best(b);
    Best fin;
    if (!argmax_finish(b, A.arg_val, A.arg_idx, A.arg_cnt, &fin)) return;
    if (threadIdx.x == 0) {
        StepState* st = A.st;
        st->token[0] = fin.i;
        A.gen_out[st->n_gen] = fin.i;
        st->n_gen += 1;
        st->pos += 1;
    }
}

// ============================================================================
// Standalone kernels (microbench / unit parity)
// ============================================================================
template <int KCH, int R>
__global__ __launch_bounds__(WG) void k_gemv_f16(const _Float16* __restrict__ W, const _Float16* __restrict__ x,
                                                 float* __restrict__ y, int N, int K) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    float xr[KCH][8];
    load_x_f16<KCH>(x, K, xr);
    const int row0 = (blockIdx.x * 4 + wid) * R;
    if (row0 >= N) return;
    float acc[R];
    dot_rows<R, KCH>(W, K, row0, min(R, N - row0), xr, acc);
    if (lane == 0)
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (row0 + r < N) y[row0 + r] = acc[r];
}

__global__ __launch_bounds__(WG) void k_e5m2(const uint16_t* __restrict__ in, uint8_t* __restrict__ out, size_t n) {
    for (size_t i = (size_t)blockIdx.x * WG + threadIdx.x; i < n; i += (size_t)gridDim.x * WG) out[i] = e5m2_encode(in[i]);
}

__global__ __launch_bounds__(WG) void k_seg_quant(const uint16_t* __restrict__ in, int seg_elems,
                                                  uint8_t* __restrict__ codes, float* __restrict__ meta) {
    const size_t off = (size_t)blockIdx.x * seg_elems;
    quantize_segment(in + off, seg_elems, codes + off, meta + (size_t)blockIdx.x * 2);
}

__global__ __launch_bounds__(WG) void k_argmax(const float* __restrict__ v, int n, int* out, float* pv, int* pi,
                                               int* cnt) {
    Best b{-INFINITY, INT_MAX};
    for (int i = blockIdx.x * WG + threadIdx.x; i < n; i += gridDim.x * WG) b = better(b, Best{v[i], i});
    b = block_best(b);
    Best fin;
    if (argmax_finish(b, pv, pi, cnt, &fin) && threadIdx.x == 0) *out = fin.i;
}

// ============================================================================
// Host launchers
// ============================================================================
namespace {

// Supported register-chunk counts: K <= KCH * 512.
int kch_for(int K) {
    const int need = (K + 511) / 512;
    const int opts[] = {1, 2, 4, 8, 11, 16};
    for (int o : opts)
        if (o >= need) return o;
    return -1;
}

#define RD_KCH_SWITCH(kch, ...)                              \
    switch (kch) {                                           \
        case 1: { constexpr int KC = 1; __VA_ARGS__; break; }  \
        case 2: { constexpr int KC = 2; __VA_ARGS__; break; }  \
        case 4: { constexpr int KC = 4; __VA_ARGS__; break; }  \
        case 8: { constexpr int KC = 8; __VA_ARGS__; break; }  \
        case 11: { constexpr int KC = 11; __VA_ARGS__; break; } \
        case 16: { constexpr int KC = 16; __VA_ARGS__; break; } \
        default: return hipErrorInvalidValue;                \
    }

template <int KVF>
hipError_t launch_attn_t(const AttnArgs& A, int hd, int G, hipStream_t s) {
    dim3 grid(A.Hk * A.S), block(WG);
#define RD_ATT(HDv, Gv)                                                  \
    if (hd == HDv && G == Gv) {                                          \
        hipLaunchKernelGGL((k_attn<HDv, Gv, KVF>), grid, block, 0, s, A); \
        return hipGetLastError();                                        \
    }
    RD_ATT(128, 1) RD_ATT(128, 2) RD_ATT(128, 4) RD_ATT(128, 8)
    RD_ATT(64, 1) RD_ATT(64, 2) RD_ATT(64, 4) RD_ATT(64, 8)
#undef RD_ATT
    return hipErrorInvalidValue;
}

hipError_t launch_attn_any(const AttnArgs& A, int kvfmt, int hd, int G, hipStream_t s) {
    switch (kvfmt) {
        case KV_FP16: return launch_attn_t<KV_FP16>(A, hd, G, s);
        case KV_E5M2: return launch_attn_t<KV_E5M2>(A, hd, G, s);
        case KV_INT8: return launch_attn_t<KV_INT8>(A, hd, G, s);
    }
    return hipErrorInvalidValue;
}

template <bool EMB>
hipError_t launch_qkv(const StepArgs& A, const LayerW& Lw, int layer, hipStream_t s) {
    const int N = (A.H + 2 * A.Hk) * A.hd;
    dim3 grid((N + 7) / 8), block(WG);
    RD_KCH_SWITCH(kch_for(A.D),
        switch (A.kvfmt) {
            case KV_FP16: hipLaunchKernelGGL((k_qkv<KC, EMB, KV_FP16>), grid, block, 0, s, A, Lw, layer); break;
            case KV_E5M2: hipLaunchKernelGGL((k_qkv<KC, EMB, KV_E5M2>), grid, block, 0, s, A, Lw, layer); break;
            default: hipLaunchKernelGGL((k_qkv<KC, EMB, KV_INT8>), grid, block, 0, s, A, Lw, layer); break;
        })
    return hipGetLastError();
}

hipError_t launch_resid(const float* in, int K, const _Float16* W, float* x, int N, hipStream_t s) {
    // Few output rows (N = d_model): one row per wave for long K keeps >= 2
    // waves per CU; two rows per wave otherwise.
    const int kch = kch_for(K);
    if (kch >= 8) {
        dim3 grid((N + 3) / 4), block(WG);
        RD_KCH_SWITCH(kch, hipLaunchKernelGGL((k_resid<KC, 1>), grid, block, 0, s, in, K, W, x, N))
    } else {
        dim3 grid((N + 7) / 8), block(WG);
        RD_KCH_SWITCH(kch, hipLaunchKernelGGL((k_resid<KC, 2>), grid, block, 0, s, in, K, W, x, N))
    }
    return hipGetLastError();
}

}  // namespace

int lm_head_workgroups(int V) { return (V + 7) / 8; }

bool step_supported(int D, int H, int Hk, int hd, int F, const char** why) {
    if (hd != 64 && hd != 128) { *why = "head_dim must be 64 or 128"; return false; }
    if (H % Hk != 0) { *why = "n_heads must be a multiple of n_kv_heads"; return false; }
    const int G = H / Hk;
    if (G != 1 && G != 2 && G != 4 && G != 8) { *why = "n_heads/n_kv_heads must be 1, 2, 4 or 8"; return false; }
    if (D % 8 || F % 8) { *why = "d_model and d_ff must be multiples of 8"; return false; }
    if (kch_for(D) < 0 || kch_for(D) > 8) { *why = "d_model must be <= 4096"; return false; }
    if (kch_for(H * hd) < 0 || kch_for(H * hd) > 8) { *why = "n_heads*head_dim must be <= 4096"; return false; }
    if (kch_for(F) < 0) { *why = "d_ff must be <= 8192"; return false; }
    return true;
}

hipError_t launch_step(const StepArgs& A, hipStream_t s) {
    hipError_t e;
    const int G = A.H / A.Hk;
    for (int l = 0; l < A.n_layers; ++l) {
        const LayerW& Lw = A.layers[l];
        e = (l == 0) ? launch_qkv<true>(A, Lw, l, s) : launch_qkv<false>(A, Lw, l, s);
        if (e != hipSuccess) return e;

        AttnArgs T{};
        const size_t lay = (size_t)l * A.Hk * A.max_ctx * A.hd;
        const size_t es = A.kvfmt == KV_FP16 ? 2 : 1;
        T.q = A.q;
        T.out = A.a;
        T.kc = reinterpret_cast<uint8_t*>(A.kc) + lay * es;
        T.vc = reinterpret_cast<uint8_t*>(A.vc) + lay * es;
        if (A.kvfmt == KV_INT8) {
            T.kst = A.stage + ((size_t)l * 2 + 0) * A.Hk * SEG * A.hd;
            T.vst = A.stage + ((size_t)l * 2 + 1) * A.Hk * SEG * A.hd;
            T.kmeta = A.meta + ((size_t)l * 2 + 0) * A.Hk * A.nseg * 2;
            T.vmeta = A.meta + ((size_t)l * 2 + 1) * A.Hk * A.nseg * 2;
        }
        T.part_o = A.part_o;
        T.part_ml = A.part_ml;
        T.cnt = A.cnt;
        T.pos_ptr = &A.st->pos;
        T.ld = A.max_ctx;
        T.nseg = A.nseg;
        T.H = A.H;
        T.Hk = A.Hk;
        T.S = A.S;
        T.scale = A.scale;
        e = launch_attn_any(T, A.kvfmt, A.hd, G, s);
        if (e != hipSuccess) return e;

        e = launch_resid(A.a, A.H * A.hd, Lw.wo, A.x, A.D, s);
        if (e != hipSuccess) return e;
        {
            dim3 grid((2 * A.F + 7) / 8), block(WG);
            RD_KCH_SWITCH(kch_for(A.D), hipLaunchKernelGGL((k_gateup<KC>), grid, block, 0, s, A, Lw))
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        e = launch_resid(A.m, A.F, Lw.wd, A.x, A.D, s);
        if (e != hipSuccess) return e;
    }
    dim3 grid(lm_head_workgroups(A.V)), block(WG);
    RD_KCH_SWITCH(kch_for(A.D), hipLaunchKernelGGL((k_lmhead<KC>), grid, block, 0, s, A))
    return hipGetLastError();
}

hipError_t launch_gemv_f16(const void* W, const void* x, float* y, int N, int K, hipStream_t s) {
    const int kch = kch_for(K);
    if (kch <= 0) return hipErrorInvalidValue;
    if (kch >= 8) {
        dim3 grid((N + 7) / 8), block(WG);
        RD_KCH_SWITCH(kch, hipLaunchKernelGGL((k_gemv_f16<KC, 2>), grid, block, 0, s,
                                              (const _Float16*)W, (const _Float16*)x, y, N, K))
    } else {
        dim3 grid((N + 15) / 16), block(WG);
        RD_KCH_SWITCH(kch, hipLaunchKernelGGL((k_gemv_f16<KC, 4>), grid, block, 0, s,
                                              (const _Float16*)W, (const _Float16*)x, y, N, K))
    }
    return hipGetLastError();
}

hipError_t launch_attention_f16(const AttnArgs& A, int hd, int G, hipStream_t s) {
    return launch_attn_any(A, KV_FP16, hd, G, s);
}

hipError_t launch_e5m2(const uint16_t* in, uint8_t* out, size_t n, hipStream_t s) {
    size_t blocks = (n + WG - 1) / WG;
    if (blocks > 65536) blocks = 65536;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_e5m2, dim3((unsigned)blocks), dim3(WG), 0, s, in, out, n);
    return hipGetLastError();
}

hipError_t launch_seg_quant(const uint16_t* in, int n_seg, int seg_elems, uint8_t* codes, float* meta,
                            hipStream_t s) {
    if (n_seg == 0) return hipSuccess;
    hipLaunchKernelGGL(k_seg_quant, dim3(n_seg), dim3(WG), 0, s, in, seg_elems, codes, meta);
    return hipGetLastError();
}

hipError_t launch_argmax(const float* v, int n, int* out, float* pv, int* pi, int* cnt, hipStream_t s) {
    int blocks = (n + WG * 8 - 1) / (WG * 8);
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_argmax, dim3(blocks), dim3(WG), 0, s, v, n, out, pv, pi, cnt);
    return hipGetLastError();
}

}  // namespace rd
