// Device-side building blocks of the decode step, shared by the one-kernel-
// per-phase executor (rd_kernels.hip) and the persistent executor
// (rd_persistent.hip).  Template flag P selects how data produced inside the
// same launch is exchanged: P = false relies on kernel boundaries (plain
// loads and stores), P = true uses agent-coherent (sc1) stores and loads
// because producer and consumer run in one persistent launch on different
// XCDs whose L2 caches are not coherent with each other.
#pragma once
#include <limits.h>
#include <math.h>

#include "rd_device.h"
#include "rd_internal.h"

namespace rd {

// ---- stores / loads of exchanged data ---------------------------------------------
template <bool P>
__device__ __forceinline__ void xst(float* p, float v) {
    if constexpr (P) st_agent(p, v); else *p = v;
}
template <bool P>
__device__ __forceinline__ float xld(const float* p) {
    if constexpr (P) return ld_agent(p); else return *p;
}
template <bool P>
__device__ __forceinline__ void xst16(uint16_t* p, uint16_t v) {
    if constexpr (P) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); else *p = v;
}
template <bool P>
__device__ __forceinline__ void xst8(uint8_t* p, uint8_t v) {
    if constexpr (P) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); else *p = v;
}
template <bool P>
__device__ __forceinline__ void xst64(uint64_t* p, uint64_t v) {
    if constexpr (P) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); else *p = v;
}
template <bool P>
__device__ __forceinline__ uint64_t xld64(const uint64_t* p) {
    if constexpr (P)
        return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        return *p;
}

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

// Copy n <= NMAX floats (n even, src 8-byte aligned) produced elsewhere in
// this launch into LDS, the workgroup reading each element once.  All of a
// thread's 8-byte loads are issued before the first is used (one memory
// round trip, not one per element); ends with a workgroup barrier.
template <bool P, int NMAX>
__device__ __forceinline__ void stage_vec(float* __restrict__ lds, const float* __restrict__ src, int n) {
    constexpr int IT = (NMAX + 2 * WG - 1) / (2 * WG);
    uint64_t v[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int e = (i * WG + threadIdx.x) * 2;
        v[i] = e < n ? xld64<P>(reinterpret_cast<const uint64_t*>(src + e)) : 0;
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int e = (i * WG + threadIdx.x) * 2;
        if (e < n) *reinterpret_cast<uint64_t*>(lds + e) = v[i];
    }
    __syncthreads();
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

// Issue the loads of R consecutive rows of a row-major [*, K] fp16 matrix
// (R*KCH KiB per wave in flight); rows >= nvalid and columns >= K read as
// zero.  Issued before the input vector is ready, so the weight stream
// starts at once and the prologue hides under its latency.
template <int R, int KCH>
__device__ __forceinline__ void load_rows(const _Float16* __restrict__ W, int K, int row0, int nvalid,
                                          u4v (&w)[R][KCH]) {
    const int lane = threadIdx.x & 63;
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
}

// acc[r] = (loaded row r) . x, reduced over the wave (every lane gets it).
template <int R, int KCH>
__device__ __forceinline__ void dot_loaded(const u4v (&w)[R][KCH], const float (&xr)[KCH][8], float (&acc)[R]) {
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
// QKV epilogue: RoPE on a (j, j+hd/2) pair and the KV-cache append
// ============================================================================
template <int KVF, bool P>
__device__ __forceinline__ void store_kv(const StepArgs& A, int layer, int which, int g, int pos, int d, float v) {
    const uint16_t h = f2h_bits(v);
    const size_t idx = (((size_t)layer * A.Hk + g) * A.max_ctx + pos) * A.hd + d;
    void* base = which ? A.vc : A.kc;
    if constexpr (KVF == KV_FP16) {
        xst16<P>(reinterpret_cast<uint16_t*>(base) + idx, h);
    } else if constexpr (KVF == KV_E5M2) {
        xst8<P>(reinterpret_cast<uint8_t*>(base) + idx, e5m2_encode(h));
    } else {
        xst16<P>(A.stage + ((((size_t)layer * 2 + which) * A.Hk + g) * SEG + pos % SEG) * A.hd + d, h);
    }
}

// Fused row pair (row0, row0+1) of the re-ordered QKV matrix -> q (rotated),
// k (rotated, cached) or v (cached).  Called by one lane.
template <int KVF, bool P>
__device__ __forceinline__ void qkv_epilogue(const StepArgs& A, int layer, int pos, int row0, float a0, float a1) {
    const int hd = A.hd, Nq = A.H * hd, Nk = A.Hk * hd;
    if (row0 < Nq + Nk) {
        const bool isq = row0 < Nq;
        const int rho = isq ? row0 : row0 - Nq;
        const int head = rho / hd, j = (rho % hd) >> 1;
        const float2 cs = A.rope[(size_t)pos * (hd / 2) + j];
        const float y0 = a0 * cs.x - a1 * cs.y;
        const float y1 = a0 * cs.y + a1 * cs.x;
        if (isq) {
            xst<P>(&A.q[head * hd + j], y0);
            xst<P>(&A.q[head * hd + j + hd / 2], y1);
        } else {
            store_kv<KVF, P>(A, layer, 0, head, pos, j, y0);
            store_kv<KVF, P>(A, layer, 0, head, pos, j + hd / 2, y1);
        }
    } else {
        const int rho = row0 - Nq - Nk;
        const int head = rho / hd, d = rho % hd;
        store_kv<KVF, P>(A, layer, 1, head, pos, d, a0);
        store_kv<KVF, P>(A, layer, 1, head, pos, d + 1, a1);
    }
}

// ============================================================================
// Attention: split-K partials, log-sum-exp merge, INT8 segment seal
// ============================================================================
// The attention view of layer l of the step's buffers.
__host__ __device__ inline AttnArgs attn_args(const StepArgs& A, int l) {
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
    return T;
}

// One lane's 8 elements (dims sl*8..+7) of K or V row p, dequantized.
// Under P (one launch may run several steps) a cache line can hold data this
// XCD read before another XCD rewrote it in the same launch: INT8 open-segment
// rows are reused every 128 steps, and a head_dim-64 E5M2 row shares its
// 128-byte line with a neighbour row.  Those reads are agent-coherent; fp16
// rows and sealed INT8 segments are written once and first read afterwards.
template <int KVF, int HD, bool P>
__device__ __forceinline__ void load_kv_row(const AttnArgs& A, int which, int g, int p, int open0, int sl,
                                            float (&f)[8]) {
    const size_t row = (size_t)g * A.ld + p;
    const void* base = which ? A.vc : A.kc;
    if constexpr (KVF == KV_FP16) {
        const h8 v = as_h8(ld16(reinterpret_cast<const _Float16*>(base) + row * HD + sl * 8));
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
    } else if constexpr (KVF == KV_E5M2) {
        const uint64_t u = xld64<P>(reinterpret_cast<const uint64_t*>(reinterpret_cast<const uint8_t*>(base) +
                                                                     row * HD + sl * 8));
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (float)e5m2_decode((uint8_t)(u >> (8 * i)));
    } else {
        if (p < open0) {
            const u2v u = ld8(reinterpret_cast<const uint8_t*>(base) + row * HD + sl * 8);
            const float* mt = (which ? A.vmeta : A.kmeta) + ((size_t)g * A.nseg + p / SEG) * 2;
            const float scale = xld<P>(mt), zp = xld<P>(mt + 1);
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = ((float)((u[i >> 2] >> ((i & 3) * 8)) & 0xffu) - zp) * scale;
        } else {
            const uint16_t* st = which ? A.vst : A.kst;
            const uint64_t* src = reinterpret_cast<const uint64_t*>(st + ((size_t)g * SEG + p % SEG) * HD + sl * 8);
            const uint64_t lo = xld64<P>(src), hi = xld64<P>(src + 1);
            const h8 v = as_h8(u4v{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi, (unsigned)(hi >> 32)});
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
// fp32 with IEEE division and round-half-to-even (v_rndne).  n % 8 == 0.
// Under P the staging rows are read and the codes and (scale, zp) written
// agent-coherently: later steps of the same launch read them on other XCDs.
template <bool P>
__device__ __forceinline__ void quantize_segment(const uint16_t* __restrict__ in, int n, uint8_t* __restrict__ codes,
                                                 float* __restrict__ meta) {
    __shared__ float sm[8];
    auto ld8h = [&](int i) {
        const uint64_t* src = reinterpret_cast<const uint64_t*>(in + i);
        const uint64_t lo = xld64<P>(src), hi = xld64<P>(src + 1);
        return as_h8(u4v{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi, (unsigned)(hi >> 32)});
    };
    float mn = INFINITY, mx = -INFINITY;
    for (int i = threadIdx.x * 8; i < n; i += WG * 8) {
        const h8 v = ld8h(i);
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
        const h8 v = ld8h(i);
        uint64_t packed = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float q = fminf(fmaxf(rintf((float)v[j] / scale) + zp, 0.0f), 255.0f);
            packed |= (uint64_t)(unsigned)q << (8 * j);
        }
        xst64<P>(reinterpret_cast<uint64_t*>(codes + i), packed);
    }
    if (threadIdx.x == 0) {
        xst<P>(meta, scale);
        xst<P>(meta + 1, zp);
    }
}

// Log-sum-exp merge of the nact split partials of the G heads of group g:
// the (m_s, l_s) pairs go through LDS once, then every output element reads
// its nact partial values with independent (batched) loads:
//   M = max_s m_s,  out = sum_s e^(m_s-M) o_s / sum_s e^(m_s-M) l_s.
template <int HD, int G, bool P>
__device__ __forceinline__ void merge_splits(const AttnArgs& A, int g, int nact) {
    __shared__ float s_w[G][MAX_SPLITS];
    __shared__ float s_inv[G];
    const int tid = threadIdx.x;
    for (int t = tid; t < G * nact; t += WG) {
        const int h = t / nact, s2 = t % nact;
        s_w[h][s2] = ld_agent(&A.part_ml[((size_t)(g * G + h) * MAX_SPLITS + s2) * 2]);
    }
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
        for (int s2 = 0; s2 < nact; ++s2) M = fmaxf(M, s_w[tid][s2]);
        float den = 0.f;
        for (int s2 = 0; s2 < nact; ++s2) {
            const float w = expf(s_w[tid][s2] - M);
            den += w * ld_agent(&A.part_ml[((size_t)(g * G + tid) * MAX_SPLITS + s2) * 2 + 1]);
            s_w[tid][s2] = w;
        }
        s_inv[tid] = 1.0f / den;
    }
    __syncthreads();
    for (int t = tid; t < G * HD; t += WG) {
        const int h = t / HD, d = t % HD;
        const float* po = A.part_o + (size_t)(g * G + h) * MAX_SPLITS * HD + d;
        float num = 0.f;
        int s2 = 0;
        for (; s2 + 8 <= nact; s2 += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = ld_agent(po + (size_t)(s2 + u) * HD);
#pragma unroll
            for (int u = 0; u < 8; ++u) num += s_w[h][s2 + u] * v[u];
        }
        for (; s2 < nact; ++s2) num += s_w[h][s2] * ld_agent(po + (size_t)s2 * HD);
        xst<P>(&A.out[(size_t)(g * G + h) * HD + d], num * s_inv[h]);
    }
}

// Number of key splits in use and their length for L attended positions:
// splits of at least 64 keys, at most S of them.
__device__ __forceinline__ void split_plan(int L, int S, int& chunk, int& nact) {
    chunk = (L + S - 1) / S;
    chunk = (chunk + 63) & ~63;
    nact = (L + chunk - 1) / chunk;
}

// Partial softmax attention of the G query heads of kv-head g over keys
// [s*chunk, min(L, (s+1)*chunk)).  A K/V row of HD fp16 spreads over HD/8
// lanes (16 bytes each), so the workgroup covers 256/(HD/8) rows per pass;
// each lane keeps an online-softmax state (running max, sum, 8 output dims)
// for its rows; the states are combined through LDS into one partial
// (m, l, o[HD]) per head, stored agent-coherently for the merge.
template <int HD, int G, int KVF, bool P>
__device__ __forceinline__ void attn_split(const AttnArgs& A, int g, int s, int chunk, int pos) {
    constexpr int LPR = HD / 8;       // lanes per K/V row
    constexpr int SLOTS = WG / LPR;   // rows per pass of the workgroup
    constexpr int U = 4;              // passes in flight
    __shared__ float sm_m[G][SLOTS], sm_l[G][SLOTS];
    __shared__ float sm_o[G][SLOTS][HD];
    const int tid = threadIdx.x, sl = tid % LPR, rs = tid / LPR;
    const int L = pos + 1;
    const int p0 = s * chunk, p1 = min(L, p0 + chunk);
    const int open0 = pos / SEG * SEG;
    float qv[G][8], m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float* qp = A.q + (size_t)(g * G + h) * HD + sl * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[h][i] = xld<P>(qp + i) * A.scale;
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
            load_kv_row<KVF, HD, P>(A, 0, g, pc, open0, sl, kf[u]);
            load_kv_row<KVF, HD, P>(A, 1, g, pc, open0, sl, vf[u]);
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
        st_agent(&A.part_o[ps * HD + d], num);
        if (d == 0) {
            st_agent(&A.part_ml[ps * 2 + 0], M);
            st_agent(&A.part_ml[ps * 2 + 1], den);
        }
    }
    __syncthreads();   // sm_* reused by the next task of this workgroup
}

// After a split's partial is stored: the last of the nact splits of group g
// merges them, and on the step that fills an INT8 segment seals it (once,
// after this step's attention has read it).
template <int HD, int G, int KVF, bool P>
__device__ __forceinline__ void attn_arrive(const AttnArgs& A, int g, int nact, int pos) {
    if (!arrive_last(&A.cnt[g], nact)) return;
    merge_splits<HD, G, P>(A, g, nact);
    if constexpr (KVF == KV_INT8) {
        if ((pos + 1) % SEG == 0) {
            const int seg = pos / SEG;
            const size_t rows = (size_t)g * A.ld + (size_t)seg * SEG;
            __syncthreads();
            quantize_segment<P>(A.kst + (size_t)g * SEG * HD, SEG * HD, reinterpret_cast<uint8_t*>(A.kc) + rows * HD,
                             A.kmeta + ((size_t)g * A.nseg + seg) * 2);
            __syncthreads();
            quantize_segment<P>(A.vst + (size_t)g * SEG * HD, SEG * HD, reinterpret_cast<uint8_t*>(A.vc) + rows * HD,
                             A.vmeta + ((size_t)g * A.nseg + seg) * 2);
        }
    }
    __syncthreads();
}

// ============================================================================
// Greedy argmax on the device
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
// Block-wide best of per-thread candidates; the same result in every thread.
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

// Two-level arrival: workgroup `id` of n counts on sub-counter id % ARG_SUB,
// the last of each sub-group on the top counter, so no counter sees more
// than ~n/ARG_SUB atomics; true in every thread of the last workgroup.
// cnt: [1 + ARG_SUB] ints, zero between uses.
constexpr int ARG_SUB = 16;
__device__ __forceinline__ bool arrive_last_tree(int* cnt, int id, int n) {
    __shared__ int s_last;
    drain_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
        const int sub = id % ARG_SUB;
        const int members = (n - 1 - sub) / ARG_SUB + 1;
        int last = 0;
        if (__hip_atomic_fetch_add(&cnt[1 + sub], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
            st_agent(&cnt[1 + sub], 0);
            const int groups = min(n, ARG_SUB);
            if (__hip_atomic_fetch_add(&cnt[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == groups - 1) {
                st_agent(&cnt[0], 0);
                last = 1;
            }
        }
        s_last = last;
    }
    __syncthreads();
    return s_last != 0;
}

// Per-workgroup partial (value, index) -> the last of n workgroups reduces
// all partials; true (with *out) in that workgroup.
__device__ __forceinline__ bool argmax_finish(Best mine, int id, int n, float* pv, int* pi, int* cnt, Best* out) {
    if (threadIdx.x == 0) {
        st_agent(&pv[id], mine.v);
        st_agent(&pi[id], mine.i);
    }
    if (!arrive_last_tree(cnt, id, n)) return false;
    Best b{-INFINITY, INT_MAX};
    for (int i = threadIdx.x; i < n; i += WG) b = better(b, Best{ld_agent(&pv[i]), ld_agent(&pi[i])});
    *out = block_best(b);
    return true;
}

}  // namespace rd
