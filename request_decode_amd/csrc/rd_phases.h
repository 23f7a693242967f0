// Device-side arithmetic of the decode step, shared by the kernel-per-phase
// executor (rd_kernels.hip) and the persistent executor (rd_persistent.hip).
// Every reduction here has one fixed association order, and both executors
// call these same functions, so they produce identical bits; only where the
// data comes from differs.  Template flag P selects how data written inside
// the same launch is read: P = false relies on kernel boundaries (plain
// loads and stores), P = true uses agent-coherent (sc1) accesses because a
// persistent launch spans several steps on XCDs whose L2 caches are not
// coherent with each other.
#pragma once
#include <limits.h>
#include <math.h>

#include "rd_device.h"
#include "rd_internal.h"

namespace rd {

// ============================================================================
// GEMV building blocks
// ============================================================================
// A length-K input vector is spread over the 64 lanes of a wave in chunks of
// 8 consecutive elements: chunk c of lane l covers columns (c*64+l)*8..+7,
// the same columns the lane reads from every weight row (16 bytes of fp16),
// so a wave-wide load of one chunk of one row is a single coalesced 1 KiB
// read.  KCH chunks cover K <= KCH*512; columns past K are zero.

template <int KCH>
__device__ __forceinline__ void load_x_f32(const float* __restrict__ x, int K, float (&xr)[KCH][8]) {
    const int lane = lane_id();
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

// The same, each element rounded to fp16 (nearest even): the precision in
// which the GEMV inputs of the step travel between workgroups (the residual
// stream itself stays fp32 where it is accumulated).
template <int KCH>
__device__ __forceinline__ void load_x_f32_h(const float* __restrict__ x, int K, float (&xr)[KCH][8]) {
    load_x_f32<KCH>(x, K, xr);
#pragma unroll
    for (int c = 0; c < KCH; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) xr[c][i] = (float)(_Float16)xr[c][i];
}

template <int KCH>
__device__ __forceinline__ void load_x_f16(const _Float16* __restrict__ x, int K, float (&xr)[KCH][8]) {
    const int lane = lane_id();
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

// The gains of an RMSNorm in the lane's chunk layout (loaded ahead of use).
template <int KCH>
__device__ __forceinline__ void load_gain(const _Float16* __restrict__ g, int K, u4v (&gv)[KCH]) {
    const int lane = lane_id();
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        gv[c] = col < K ? ld16(g + col) : u4v{0u, 0u, 0u, 0u};
    }
}
// RMSNorm of the register-resident vector: x * (mean(x^2) + eps)^-1/2 * g.
template <int KCH>
__device__ __forceinline__ void rmsnorm_gain(float (&xr)[KCH][8], const u4v (&gv)[KCH], int K, float eps) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < KCH; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += xr[c][i] * xr[c][i];
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)K + eps);
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const h8 g8 = as_h8(gv[c]);
#pragma unroll
        for (int i = 0; i < 8; ++i) xr[c][i] = xr[c][i] * inv * (float)g8[i];
    }
}
template <int KCH>
__device__ __forceinline__ void rmsnorm_regs(float (&xr)[KCH][8], const _Float16* __restrict__ g, int K, float eps) {
    u4v gv[KCH];
    load_gain<KCH>(g, K, gv);
    rmsnorm_gain<KCH>(xr, gv, K, eps);
}

// Issue the loads of R consecutive rows of a row-major [*, K] fp16 matrix;
// rows >= nvalid and columns >= K read as zero.
template <int R, int KCH>
__device__ __forceinline__ void load_rows(const _Float16* __restrict__ W, int K, int row0, int nvalid,
                                          u4v (&w)[R][KCH]) {
    const int lane = lane_id();
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

// The GEMV operand: the fp16 rounding (nearest even) of the register-resident
// vector, 8 halves per chunk in one u4v (column order kept).
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    return (uint32_t)f2h_bits(lo) | ((uint32_t)f2h_bits(hi) << 16);
}
template <int KCH>
__device__ __forceinline__ void pack_x(const float (&xr)[KCH][8], u4v (&xh)[KCH]) {
#pragma unroll
    for (int c = 0; c < KCH; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) xh[c][i] = pack_h2(xr[c][2 * i], xr[c][2 * i + 1]);
}

// out[r] = row r . x for NR loaded rows (columns past K already zero) and
// the fp16 operand x, the same value in every lane.  Per lane: two running
// fp32 sums over the chunks in order, each step a two-term fp16 dot product
// (v_dot2_f32_f16: words 0, 2 of a chunk into the first sum, words 1, 3 into
// the second); then the 16-lane DPP row sums and the four rows in a fixed
// order.
template <int NR, int KCH>
__device__ __forceinline__ void dot_rows(const u4v (&w)[NR][KCH], const u4v (&xh)[KCH], float (&out)[NR]) {
    float s0[NR], s1[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) s0[r] = s1[r] = 0.f;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            // (vector elements go through plain locals before the bit casts)
            const u4v wv = w[r][c], xv = xh[c];
            const unsigned w0 = wv.x, w1 = wv.y, w2 = wv.z, w3 = wv.w;
            const unsigned x0 = xv.x, x1 = xv.y, x2 = xv.z, x3 = xv.w;
            s0[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w0), __builtin_bit_cast(h2, x0), s0[r], false);
            s1[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w1), __builtin_bit_cast(h2, x1), s1[r], false);
            s0[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w2), __builtin_bit_cast(h2, x2), s0[r], false);
            s1[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w3), __builtin_bit_cast(h2, x3), s1[r], false);
        }
    }
    float v[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) v[r] = row16_sum(s0[r] + s1[r]);
#pragma unroll
    for (int r = 0; r < NR; ++r)
        out[r] = ((readlane_f(v[r], 0) + readlane_f(v[r], 16)) + readlane_f(v[r], 32)) + readlane_f(v[r], 48);
}

// SwiGLU output m = silu(gate) * up, rounded to fp16 (nearest even): the
// precision the down projection takes it in, in every executor (the
// persistent one exchanges it as fp16 pairs).
__device__ __forceinline__ float silu_mul(float gt, float up) {
    return (float)(_Float16)(gt / (1.0f + expf(-gt)) * up);
}

// ============================================================================
// QKV epilogue: RoPE on a (j, j+hd/2) pair and the KV-cache append
// ============================================================================
// Row pair (row0, row0+1) of the re-ordered QKV matrix: kind 0 = q head,
// 1 = k head (both rotated: rows 2j, 2j+1 of a head are dims j and j+hd/2),
// 2 = v (rows are consecutive dims).  rope: the (cos, sin) row of the
// position, or (own) the pair's own (cos, sin).
struct QkvPair {
    int kind, head, d0, d1;
    float y0, y1;
};
__device__ __forceinline__ QkvPair qkv_pair(int hd, int H, int Hk, int row0, float a0, float a1, const float2* rope,
                                            bool own = false) {
    QkvPair o;
    const int Nq = H * hd, Nk = Hk * hd;
    if (row0 < Nq + Nk) {
        const bool isq = row0 < Nq;
        const int rho = isq ? row0 : row0 - Nq;
        const int j = (rho % hd) >> 1;
        const float2 cs = own ? rope[0] : rope[j];
        o.kind = isq ? 0 : 1;
        o.head = rho / hd;
        o.d0 = j;
        o.d1 = j + hd / 2;
        // explicit fused forms: one rounding order wherever this is inlined
        o.y0 = fmaf(a0, cs.x, -(a1 * cs.y));
        o.y1 = fmaf(a0, cs.y, a1 * cs.x);
    } else {
        const int rho = row0 - Nq - Nk;
        o.kind = 2;
        o.head = rho / hd;
        o.d0 = rho % hd;
        o.d1 = o.d0 + 1;
        o.y0 = a0;
        o.y1 = a1;
    }
    return o;
}

// Store one element of the new K (which = 0) or V row in the cache format
// and return the value attention will read back for it.
template <int KVF, bool P>
__device__ __forceinline__ float kv_put(const StepArgs& A, int layer, int which, int g, int pos, int d, float v) {
    const uint16_t h = f2h_bits(v);
    const size_t idx = (((size_t)layer * A.Hk + g) * A.max_ctx + pos) * A.hd + d;
    void* base = which ? A.vc : A.kc;
    if constexpr (KVF == KV_FP16) {
        uint16_t* p = reinterpret_cast<uint16_t*>(base) + idx;
        if constexpr (P) __hip_atomic_store(p, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); else *p = h;
        return h_bits2f(h);
    } else if constexpr (KVF == KV_E5M2) {
        const uint8_t e = e5m2_encode(h);
        uint8_t* p = reinterpret_cast<uint8_t*>(base) + idx;
        if constexpr (P) __hip_atomic_store(p, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); else *p = e;
        return (float)e5m2_decode(e);
    } else {
        uint16_t* p = A.stage + ((((size_t)layer * 2 + which) * A.Hk + g) * SEG + pos % SEG) * A.hd + d;
        if constexpr (P) __hip_atomic_store(p, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); else *p = h;
        return h_bits2f(h);
    }
}

// ============================================================================
// Attention: one wave per (kv-head, key split) task
// ============================================================================
// A K/V row of HD elements spreads over LPR = HD/8 lanes (8 elements each);
// a wave covers RPW = 64/LPR rows per load.  Lane (slot r, part j) keeps an
// online-softmax state for its rows: running max m, sum l, and output dims
// j*8..j*8+7, for each of the G query heads of the group.
template <int HD>
struct AttnGeo {
    static constexpr int LPR = HD / 8;
    static constexpr int RPW = WAVE / LPR;
    static constexpr int U = 4;                 // rows per lane per batch
    static constexpr int BATCH = RPW * U;       // rows per batch
    static constexpr int NPART = HD / 64;       // merge tasks per query head (64 dims each)
};

// Splits of L attended positions: at most S of them, each a multiple of 4
// keys and at least 48 (one 16-row batch for each of the three waves that
// reduce a split): below that, a split's latency no longer shrinks, and every
// extra split is one more partial for the merge to wait for.
__device__ __forceinline__ void split_plan(int L, int S, int& chunk, int& nact) {
    chunk = (L + S - 1) / S;
    chunk = (chunk + 3) & ~3;
    chunk = chunk < 48 ? 48 : chunk;
    nact = (L + chunk - 1) / chunk;
}

// One lane's 8 elements (dims j*8..+7) of K or V row p as stored, and their
// dequantization.  Under P the reads that can meet a stale line are
// agent-coherent: INT8 open-segment rows (the staging buffer is reused every
// 128 steps), INT8 scales (several segments share a line), head_dim-64 E5M2
// rows (two rows share a 128-byte line, so fetching an older row can bring in
// the line of the row being written).  The other rows (fp16 rows, head_dim-128
// E5M2 rows, sealed codes: whole lines of one row, or of one sealed segment)
// are first fetched in a step after the one that wrote them: the row of the
// current step is never fetched from the cache under P (kv_batch_raw).
struct KvRaw {
    u4v d;         // fp16: 8 halves; E5M2: 8 bytes in d.x, d.y; INT8: codes in d.x, d.y or 8 fp16
    float scale;   // INT8 sealed row: its segment's scale and zero point; < 0: an fp16 open-segment row
    float zp;
};
template <int HD, int KVF, bool P>
__device__ __forceinline__ KvRaw kv_raw(const AttnArgs& A, int which, int g, int p, int open0, int j) {
    const size_t row = (size_t)g * A.ld + p;
    const void* base = which ? A.vc : A.kc;
    KvRaw r;
    r.scale = -1.f;
    r.zp = 0.f;
    if constexpr (KVF == KV_FP16) {
        r.d = __builtin_nontemporal_load(
            reinterpret_cast<const u4v*>(reinterpret_cast<const _Float16*>(base) + row * HD + j * 8));
    } else if constexpr (KVF == KV_E5M2) {
        const uint64_t* src = reinterpret_cast<const uint64_t*>(reinterpret_cast<const uint8_t*>(base) + row * HD + j * 8);
        const uint64_t u = (P && HD == 64) ? ld_agent(src) : __builtin_nontemporal_load(src);
        r.d = u4v{(unsigned)u, (unsigned)(u >> 32), 0u, 0u};
    } else {
        if (p < open0) {
            const u2v u = ld8(reinterpret_cast<const uint8_t*>(base) + row * HD + j * 8);
            const float* mt = (which ? A.vmeta : A.kmeta) + ((size_t)g * A.nseg + p / SEG) * 2;
            r.scale = P ? ld_agent(mt) : mt[0];
            r.zp = P ? ld_agent(mt + 1) : mt[1];
            r.d = u4v{u.x, u.y, 0u, 0u};
        } else {
            const uint16_t* st = which ? A.vst : A.kst;
            const uint64_t* src = reinterpret_cast<const uint64_t*>(st + ((size_t)g * SEG + p % SEG) * HD + j * 8);
            const uint64_t lo = P ? ld_agent(src) : src[0], hi = P ? ld_agent(src + 1) : src[1];
            r.d = u4v{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi, (unsigned)(hi >> 32)};
        }
    }
    return r;
}
template <int KVF>
__device__ __forceinline__ void kv_cvt(const KvRaw& r, float (&f)[8]) {
    if constexpr (KVF == KV_E5M2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (float)e5m2_decode((uint8_t)(r.d[i >> 2] >> ((i & 3) * 8)));
    } else if constexpr (KVF == KV_INT8) {
        if (r.scale >= 0.f) {
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = ((float)((r.d[i >> 2] >> ((i & 3) * 8)) & 0xffu) - r.zp) * r.scale;
            return;
        }
        const h8 v = as_h8(r.d);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
    } else {
        const h8 v = as_h8(r.d);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
    }
}

// Row of slot `slot`, batch position u, of the batch starting at pb.
template <int HD>
__device__ __forceinline__ int batch_row(int pb, int u, int slot) { return pb + u * AttnGeo<HD>::RPW + slot; }

// The raw K and V elements of this lane's U rows of the batch starting at pb
// (rows at or past p1 read row p0 instead; they are masked when reduced).
// Under P (one launch, several steps), row pos, the one this step writes, is
// not fetched from the fp16 or E5M2 cache either: its value comes from the
// exchange (the caller's fix), and a fetch racing its store could leave a copy
// of the line from before the store in this XCD's L2, which a later step of
// the same launch would then read.  Such rows fetch an older row instead (p0,
// or pos - 1 when the split starts at pos); at pos 0 nothing is fetched.
template <int HD, int KVF, bool P>
__device__ __forceinline__ void kv_batch_raw(const AttnArgs& A, int g, int pb, int p0, int p1, int open0, int pos,
                                             KvRaw (&kr)[AttnGeo<HD>::U], KvRaw (&vr)[AttnGeo<HD>::U]) {
    using Geo = AttnGeo<HD>;
    const int lane = lane_id(), slot = lane / Geo::LPR, j = lane % Geo::LPR;
    if constexpr (KVF == KV_INT8) {
        // the (scale, zp) pairs of the at most two segments the batch's rows
        // fall in, one 8-byte load each for K and V (the same address in
        // every lane), instead of two loads per row
        const int last = min(pb + Geo::BATCH, p1) - 1;
        const int s0 = pb / SEG, s1 = last / SEG;
        const bool sealed0 = s0 * SEG < open0, sealed1 = s1 != s0 && s1 * SEG < open0;
        auto meta = [&](const float* m, int sg) {
            const uint64_t* q = reinterpret_cast<const uint64_t*>(m + ((size_t)g * A.nseg + sg) * 2);
            return P ? ld_agent(q) : *q;
        };
        const uint64_t mk0 = sealed0 ? meta(A.kmeta, s0) : 0ull, mv0 = sealed0 ? meta(A.vmeta, s0) : 0ull;
        const uint64_t mk1 = sealed1 ? meta(A.kmeta, s1) : mk0, mv1 = sealed1 ? meta(A.vmeta, s1) : mv0;
        // every row of the batch sealed (the common case, decided for the
        // whole wave): no branch between a row's load and its registers, so
        // that all of the batch's loads stay in flight together
        if (last < open0 && p0 < open0) {
#pragma unroll
            for (int u = 0; u < Geo::U; ++u) {
                const int p = batch_row<HD>(pb, u, slot);
                const int pc = p < p1 ? p : p0;
                const size_t row = (size_t)g * A.ld + pc;
                const u2v ck = ld8(reinterpret_cast<const uint8_t*>(A.kc) + row * HD + j * 8);
                const u2v cv = ld8(reinterpret_cast<const uint8_t*>(A.vc) + row * HD + j * 8);
                const bool hi = pc / SEG != s0;
                const uint64_t mk = hi ? mk1 : mk0, mv = hi ? mv1 : mv0;
                kr[u] = KvRaw{u4v{ck.x, ck.y, 0u, 0u}, __uint_as_float((uint32_t)mk), __uint_as_float((uint32_t)(mk >> 32))};
                vr[u] = KvRaw{u4v{cv.x, cv.y, 0u, 0u}, __uint_as_float((uint32_t)mv), __uint_as_float((uint32_t)(mv >> 32))};
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < Geo::U; ++u) {
            const int p = batch_row<HD>(pb, u, slot);
            const int pc = p < p1 ? p : p0;
            const size_t row = (size_t)g * A.ld + pc;
            if (pc < open0) {
                const u2v ck = ld8(reinterpret_cast<const uint8_t*>(A.kc) + row * HD + j * 8);
                const u2v cv = ld8(reinterpret_cast<const uint8_t*>(A.vc) + row * HD + j * 8);
                const bool hi = pc / SEG != s0;
                const uint64_t mk = hi ? mk1 : mk0, mv = hi ? mv1 : mv0;
                kr[u] = KvRaw{u4v{ck.x, ck.y, 0u, 0u}, __uint_as_float((uint32_t)mk), __uint_as_float((uint32_t)(mk >> 32))};
                vr[u] = KvRaw{u4v{cv.x, cv.y, 0u, 0u}, __uint_as_float((uint32_t)mv), __uint_as_float((uint32_t)(mv >> 32))};
            } else {
                kr[u] = kv_raw<HD, KVF, P>(A, 0, g, pc, open0, j);
                vr[u] = kv_raw<HD, KVF, P>(A, 1, g, pc, open0, j);
            }
        }
    } else {
        if constexpr (P) {
            if (pos == 0) {   // the only row is the new one (wave-uniform)
#pragma unroll
                for (int u = 0; u < Geo::U; ++u) kr[u] = vr[u] = KvRaw{u4v{0u, 0u, 0u, 0u}, -1.f, 0.f};
                return;
            }
        }
        const int alt = P && p0 == pos ? pos - 1 : p0;
#pragma unroll
        for (int u = 0; u < Geo::U; ++u) {
            const int p = batch_row<HD>(pb, u, slot);
            const int pc = p < p1 && !(P && p == pos) ? p : alt;
            kr[u] = kv_raw<HD, KVF, P>(A, 0, g, pc, open0, j);
            vr[u] = kv_raw<HD, KVF, P>(A, 1, g, pc, open0, j);
        }
    }
}
template <int HD, int KVF>
__device__ __forceinline__ void kv_batch_cvt(int pb, int p1, const KvRaw (&kr)[AttnGeo<HD>::U],
                                             const KvRaw (&vr)[AttnGeo<HD>::U], float (&kf)[AttnGeo<HD>::U][8],
                                             float (&vf)[AttnGeo<HD>::U][8], bool (&valid)[AttnGeo<HD>::U]) {
    const int slot = lane_id() / AttnGeo<HD>::LPR;
#pragma unroll
    for (int u = 0; u < AttnGeo<HD>::U; ++u) {
        valid[u] = batch_row<HD>(pb, u, slot) < p1;
        kv_cvt<KVF>(kr[u], kf[u]);
        kv_cvt<KVF>(vr[u], vf[u]);
    }
}

// Scores are kept in log2 units: the query is pre-multiplied by
// scale * log2(e), so every exponential is one hardware exp2 (v_exp_f32).
constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int HD, int G>
struct AttnAcc {
    float m[G], l[G], o[G][8];
    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m[h] = -INFINITY;
            l[h] = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
        }
    }
    // Scores of the batch's rows against the pre-scaled queries; then per
    // slot one online-softmax update for the whole batch: the new maximum,
    // one rescale of the running sum and output, and the batch's rows added
    // in order.
    __device__ __forceinline__ void batch(const float (&qv)[G][8], const float (&kf)[AttnGeo<HD>::U][8],
                                          const float (&vf)[AttnGeo<HD>::U][8], const bool (&valid)[AttnGeo<HD>::U]) {
        constexpr int U = AttnGeo<HD>::U;
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) d += qv[h][i] * kf[u][i];
                d = group_sum<AttnGeo<HD>::LPR>(d);
                sc[u][h] = valid[u] ? d : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mb = m[h];
#pragma unroll
            for (int u = 0; u < U; ++u) mb = fmaxf(mb, sc[u][h]);
            if (mb == -INFINITY) continue;   // this slot has seen no key yet
            const float c = exp2_fast(m[h] - mb);
            l[h] *= c;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[h][i] *= c;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float e = exp2_fast(sc[u][h] - mb);
                l[h] += e;
#pragma unroll
                for (int i = 0; i < 8; ++i) o[h][i] += e * vf[u][i];
            }
            m[h] = mb;
        }
    }
    // Combine the RPW slots: M = max of the slot maxima, each slot weighted
    // by 2^(m_slot - M) (0 for a slot that saw no key); afterwards every lane
    // of part j holds the task's partial (M, l, o[j*8..+7]).
    __device__ __forceinline__ void finish() {
        constexpr int LPR = AttnGeo<HD>::LPR, RPW = AttnGeo<HD>::RPW;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float M = -INFINITY;
#pragma unroll
            for (int r = 0; r < RPW; ++r) M = fmaxf(M, readlane_f(m[h], r * LPR));
            const float w = m[h] == -INFINITY ? 0.f : exp2_fast(m[h] - M);
            const float wl = w * l[h];
            float L = 0.f;
#pragma unroll
            for (int r = 0; r < RPW; ++r) L += readlane_f(wl, r * LPR);
            // v + v[l ^ s] for s = LPR, ..., 32 (row rotation by 8 is l ^ 8 in a
            // row of 16; the swaps add the same two values in either order)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float v = w * o[h][i];
                if constexpr (LPR == 8) v += dpp_f<0x128>(v);
                v = swap16_sum(v);
                o[h][i] = swap32_sum(v);
            }
            m[h] = M;
            l[h] = L;
        }
    }
};

// ============================================================================
// One attention split on the NW waves of a workgroup
// ============================================================================
// Both executors reduce a split on ATT_WAVES waves (in the persistent kernel
// its stream waves), so that they produce the same bits.
constexpr int ATT_WAVES = 3;
// Wave w takes the batches p0 + (w + NW*i)*BATCH of the split [p0, p1), with
// the raw rows of the next two of its batches in flight while one is reduced
// (three buffers).  The caller loads buffer 0 (attn_wave_first) before
// attn_wave_run; fix(pb, kf, vf) may replace converted rows (the row being
// written this step, taken from the exchange instead of the cache).
template <int HD>
using KvBuf = KvRaw[3][AttnGeo<HD>::U];

template <int HD, int KVF, bool P, int NW>
__device__ __forceinline__ void attn_wave_first(const AttnArgs& T, int g, int p0, int p1, int open0, int pos, int w,
                                                KvBuf<HD>& kb, KvBuf<HD>& vb) {
    const int pb = p0 + w * AttnGeo<HD>::BATCH;
    if (pb < p1) kv_batch_raw<HD, KVF, P>(T, g, pb, p0, p1, open0, pos, kb[0], vb[0]);
}
template <int HD, int G, int KVF, bool P, int NW, class Fix>
__device__ __forceinline__ void attn_wave_run(const AttnArgs& T, int g, int p0, int p1, int open0, int pos, int w,
                                              const float (&qv)[G][8], AttnAcc<HD, G>& acc, KvBuf<HD>& kb,
                                              KvBuf<HD>& vb, Fix fix) {
    using Geo = AttnGeo<HD>;
    constexpr int STEP = NW * Geo::BATCH;
    const int pf = p0 + w * Geo::BATCH;
    if (pf >= p1) return;
    if (pf + STEP < p1) kv_batch_raw<HD, KVF, P>(T, g, pf + STEP, p0, p1, open0, pos, kb[1], vb[1]);
    for (int i = 0;; i += 3) {
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int pb = pf + (i + r) * STEP;
            if (pb >= p1) return;
            const int pn = pb + 2 * STEP;
            if (pn < p1) kv_batch_raw<HD, KVF, P>(T, g, pn, p0, p1, open0, pos, kb[(r + 2) % 3], vb[(r + 2) % 3]);
            float kf[Geo::U][8], vf[Geo::U][8];
            bool valid[Geo::U];
            kv_batch_cvt<HD, KVF>(pb, p1, kb[r], vb[r], kf, vf, valid);
            fix(pb, kf, vf);
            acc.batch(qv, kf, vf, valid);
        }
    }
}
// The NW wave partials of a split, combined in wave order with the same
// log-sum-exp rule as the split merge: M = max_w m_w, f_w = 2^(m_w - M)
// (0 for a wave that saw no key), l = sum_w f_w l_w, o = sum_w f_w o_w.
// s_att: LDS [NW][G][HD+2].  Every wave stores (attn_part_store), the
// workgroup synchronises, then any one wave combines.
template <int HD, int G>
__device__ __forceinline__ void attn_part_store(float* s_att, int w, const AttnAcc<HD, G>& acc) {
    const int lane = lane_id(), j = lane % AttnGeo<HD>::LPR;
    if (lane < AttnGeo<HD>::LPR) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float* d = s_att + (w * G + h) * (HD + 2);
#pragma unroll
            for (int i = 0; i < 8; ++i) d[j * 8 + i] = acc.o[h][i];
            if (lane == 0) {
                d[HD] = acc.m[h];
                d[HD + 1] = acc.l[h];
            }
        }
    }
}
template <int HD, int G, int NW>
__device__ __forceinline__ void attn_combine(const float* s_att, AttnAcc<HD, G>& out) {
    const int j = lane_id() % AttnGeo<HD>::LPR;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float mw[NW];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            mw[w] = s_att[(w * G + h) * (HD + 2) + HD];
            M = fmaxf(M, mw[w]);
        }
        float L = 0.f, o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float* d = s_att + (w * G + h) * (HD + 2);
            const float f = mw[w] == -INFINITY ? 0.f : exp2_fast(mw[w] - M);
            L += f * d[HD + 1];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] += f * d[j * 8 + i];
        }
        out.m[h] = M;
        out.l[h] = L;
#pragma unroll
        for (int i = 0; i < 8; ++i) out.o[h][i] = o[i];
    }
}

// ============================================================================
// Log-sum-exp merge of the split partials of one query head
// ============================================================================
// Partial s of query head h lives at part[(h*S + s)*(HD+2)]: o[HD], m, l.
// Lane t of the wave holds (m, l) of splits t, t+64, ... (NC chunks), with
// m in log2 units:
//   M = max_s m_s, w_s = 2^(m_s - M), den = sum_s w_s l_s (per lane over its
//   chunks in order, then the wave sum), out[d] = sum_s w_s o_s[d] / den
//   with s ascending.
constexpr int MERGE_NC = MAX_SPLITS / 64;
struct MergeW {
    float w[MERGE_NC];
    float den;
};
__device__ __forceinline__ MergeW merge_weights(int nact, const float (&ms)[MERGE_NC], const float (&ls)[MERGE_NC]) {
    const int lane = lane_id();
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < MERGE_NC; ++c)
        if (c * 64 + lane < nact) M = fmaxf(M, ms[c]);
    M = wave_max(M);
    MergeW r;
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < MERGE_NC; ++c) {
        const bool live = c * 64 + lane < nact && ms[c] != -INFINITY;
        r.w[c] = live ? exp2_fast(ms[c] - M) : 0.f;
        if (live) d += r.w[c] * ls[c];
    }
    r.den = wave_sum(d);
    return r;
}
// num += sum over the NS splits s of chunk c of w_s * ov[s - 64c], s
// ascending; splits past nact carry weight 0 and a finite ov (0), so they
// add +0 and need no test.
template <int NS>
__device__ __forceinline__ void merge_acc(float& num, int c, const MergeW& mw, const float (&ov)[64]) {
    float w = mw.w[0];
#pragma unroll
    for (int cc = 1; cc < MERGE_NC; ++cc)
        if (cc == c) w = mw.w[cc];
#pragma unroll
    for (int k = 0; k < NS; ++k) num += readlane_f(w, k) * ov[k];
}

// ============================================================================
// INT8 segment seal (one wave)
// ============================================================================
// Adaptive-range quantization of one segment of n fp16 values ("Grok-3
// v3.2.4 hot update deep dive", §3.2): scale = (max-min)/255,
// zp = round(-min/scale), code = clamp(round(x/scale) + zp, 0, 255), all in
// fp32 with IEEE division and round-half-to-even (rint); when max == min,
// scale |min| (1 for zeros), so the value is reproduced exactly.  n % 8 == 0.  Under P the inputs are read and the codes and
// (scale, zp) written agent-coherently.
template <bool P>
__device__ __forceinline__ void seal_segment(const uint16_t* __restrict__ in, int n, uint8_t* __restrict__ codes,
                                             float* __restrict__ meta) {
    const int lane = lane_id();
    auto ld8h = [&](int i) {
        const uint64_t* src = reinterpret_cast<const uint64_t*>(in + i);
        const uint64_t lo = P ? ld_agent(src) : src[0], hi = P ? ld_agent(src + 1) : src[1];
        return as_h8(u4v{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi, (unsigned)(hi >> 32)});
    };
    float mn = INFINITY, mx = -INFINITY;
    for (int i = lane * 8; i < n; i += 512) {
        const h8 v = ld8h(i);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            mn = fminf(mn, (float)v[k]);
            mx = fmaxf(mx, (float)v[k]);
        }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    float scale = (mx - mn) / 255.0f;
    // one repeated value: its magnitude is the unit (every code 0, exact);
    // an all-zero segment takes scale 1
    if (!(scale > 0.0f)) scale = mn != 0.0f ? fabsf(mn) : 1.0f;
    const float zp = rintf(-mn / scale);
    for (int i = lane * 8; i < n; i += 512) {
        const h8 v = ld8h(i);
        uint64_t packed = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float q = fminf(fmaxf(rintf((float)v[k] / scale) + zp, 0.0f), 255.0f);
            packed |= (uint64_t)(unsigned)q << (8 * k);
        }
        uint64_t* dst = reinterpret_cast<uint64_t*>(codes + i);
        if constexpr (P) st_agent(dst, packed); else *dst = packed;
    }
    if (lane == 0) {
        if constexpr (P) {
            st_agent(meta, scale);
            st_agent(meta + 1, zp);
        } else {
            meta[0] = scale;
            meta[1] = zp;
        }
    }
}

// Seal kv-head g's K and V segments of the layer viewed by T, which hold
// positions up to pos ((pos+1) % 128 == 0).
template <int HD, bool P>
__device__ __forceinline__ void seal_head(const AttnArgs& T, int g, int pos) {
    const int seg = pos / SEG;
    const size_t rows = (size_t)g * T.ld + (size_t)seg * SEG;
    seal_segment<P>(T.kst + (size_t)g * SEG * HD, SEG * HD, reinterpret_cast<uint8_t*>(T.kcw) + rows * HD,
                    T.kmeta + ((size_t)g * T.nseg + seg) * 2);
    seal_segment<P>(T.vst + (size_t)g * SEG * HD, SEG * HD, reinterpret_cast<uint8_t*>(T.vcw) + rows * HD,
                    T.vmeta + ((size_t)g * T.nseg + seg) * 2);
}

// ============================================================================
// Greedy argmax
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
// Block-wide best of per-thread candidates (256 threads); the same result in
// every thread.
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
