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

// One chunk of dot_rows: the chunk's two-term products into the two running
// sums of each row.
template <int NR>
__device__ __forceinline__ void dot_chunk(const u4v (&w)[NR], const u4v xv, float (&s0)[NR], float (&s1)[NR]) {
    const unsigned x0 = xv.x, x1 = xv.y, x2 = xv.z, x3 = xv.w;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        // (vector elements go through plain locals before the bit casts)
        const u4v wv = w[r];
        const unsigned w0 = wv.x, w1 = wv.y, w2 = wv.z, w3 = wv.w;
        s0[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w0), __builtin_bit_cast(h2, x0), s0[r], false);
        s1[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w1), __builtin_bit_cast(h2, x1), s1[r], false);
        s0[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w2), __builtin_bit_cast(h2, x2), s0[r], false);
        s1[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w3), __builtin_bit_cast(h2, x3), s1[r], false);
    }
}
// The row sums of dot_rows from the running sums.
template <int NR>
__device__ __forceinline__ void dot_finish(const float (&s0)[NR], const float (&s1)[NR], float (&out)[NR]) {
    float v[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) v[r] = row16_sum(s0[r] + s1[r]);
#pragma unroll
    for (int r = 0; r < NR; ++r)
        out[r] = ((readlane_f(v[r], 0) + readlane_f(v[r], 16)) + readlane_f(v[r], 32)) + readlane_f(v[r], 48);
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
        u4v wc[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) wc[r] = w[r][c];
        dot_chunk<NR>(wc, xh[c], s0, s1);
    }
    dot_finish<NR>(s0, s1, out);
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
// 2 = v (rows are consecutive dims).  cs: the pair's (cos, sin) (rope_col
// gives its column in the position's RoPE row; unused for v).
struct QkvPair {
    int kind, head, d0, d1;
    float y0, y1;
};
__device__ __forceinline__ int rope_col(int hd, int H, int row0) {
    const int Nq = H * hd;
    return ((row0 < Nq ? row0 : row0 - Nq) % hd) >> 1;
}
__device__ __forceinline__ QkvPair qkv_pair_cs(int hd, int H, int Hk, int row0, float a0, float a1, float2 cs) {
    QkvPair o;
    const int Nq = H * hd, Nk = Hk * hd;
    if (row0 < Nq + Nk) {
        const bool isq = row0 < Nq;
        const int rho = isq ? row0 : row0 - Nq;
        const int j = (rho % hd) >> 1;
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
// The same with the position's RoPE row (cos, sin) pairs.
__device__ __forceinline__ QkvPair qkv_pair(int hd, int H, int Hk, int row0, float a0, float a1, const float2* rope) {
    const float2 cs = row0 < (H + Hk) * hd ? rope[rope_col(hd, H, row0)] : make_float2(1.f, 0.f);
    return qkv_pair_cs(hd, H, Hk, row0, a0, a1, cs);
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

// Element d of this step's K (which = 0) or V row of kv head g at position
// pos of sequence b, into its page of a paged cache (fp16 or E5M2); the
// host allocates the page before the step.
template <int KVF>
__device__ __forceinline__ void kv_put_paged(const StepArgs& A, int b, int layer, int which, int g, int pos, int d,
                                             float v) {
    static_assert(KVF != KV_INT8, "paged caches hold fp16 or E5M2 rows");
    const int page = A.ptab[(size_t)b * A.pt_ld + (pos >> A.pshift)];
    if (page < 0) return;
    const size_t R = (size_t)1 << A.pshift;
    const size_t idx = ((((size_t)layer * A.npages + page) * A.Hk + g) * R + (pos & (R - 1))) * A.hd + d;
    const uint16_t h = f2h_bits(v);
    if constexpr (KVF == KV_FP16) reinterpret_cast<uint16_t*>(which ? A.vc : A.kc)[idx] = h;
    else reinterpret_cast<uint8_t*>(which ? A.vc : A.kc)[idx] = e5m2_encode(h);
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
    static constexpr int NPART = HD / 64;       // merge tasks per query head (64 dims each)
};

// ---- splits ---------------------------------------------------------------
// The L attended positions of a step are cut into splits, one workgroup
// each.  fp16 and E5M2: at most S splits of `chunk` positions, a multiple of
// 4 and at least 48 (one 16-row batch for each of the three waves that reduce
// a split: below that a split's latency no longer shrinks, and every extra
// split is one more partial for the merge to wait for).  INT8: the sealed
// positions [0, open0) in at most S - 1 such splits, then one split over the
// open segment [open0, L), whose rows are fp16 staging rows, so that every
// split reads one kind of row (S >= 2).
struct SplitPlan {
    int chunk;   // positions per split of the cut range
    int ncut;    // splits of the cut range [0, end)
    int end;     // L (fp16, E5M2) or open0 (INT8)
    int nact;    // splits in use: ncut, plus the open-segment split for INT8
};
__device__ __forceinline__ SplitPlan split_plan(int L, int S, int kvf) {
    SplitPlan sp;
    const bool i8 = kvf == KV_INT8;
    sp.end = i8 ? (L - 1) / SEG * SEG : L;
    const int n = i8 ? S - 1 : S;
    int chunk = (sp.end + n - 1) / n;
    chunk = (chunk + 3) & ~3;
    sp.chunk = chunk < 48 ? 48 : chunk;
    sp.ncut = (sp.end + sp.chunk - 1) / sp.chunk;
    sp.nact = sp.ncut + (i8 ? 1 : 0);
    return sp;
}
// Positions [p0, p1) of split s < nact.
__device__ __forceinline__ void split_range(const SplitPlan& sp, int L, int s, int& p0, int& p1) {
    if (s < sp.ncut) {
        p0 = s * sp.chunk;
        p1 = min(sp.end, p0 + sp.chunk);
    } else {
        p0 = sp.end;
        p1 = L;
    }
}

// ---- K/V rows of a split ----------------------------------------------------
// A source reads the rows of one kind of split with buffer loads.  A row that
// must not be fetched (past the split, in a batch past the wave's last one,
// or, in the persistent kernel (P), the row this step writes, whose value
// comes from the exchange) gets an offset past the end of its buffer, and its
// load returns zeros without touching memory.  So every batch of a source
// issues the same loads, with no branch between a load and its registers: the
// compiler's count of outstanding loads stays exact, and a batch waits only
// for its own rows while the two batches after it stay in flight.
//
// Under P the reads that can meet a stale line are agent-coherent: INT8
// open-segment rows (the staging buffer is reused every 128 steps), INT8
// (scale, zp) pairs (several segments share a line), head_dim-64 E5M2 rows
// (two rows share a 128-byte line, so fetching an older row can bring in the
// line of the row being written).  The other rows (fp16 rows, head_dim-128
// E5M2 rows, sealed codes: whole lines of one row, or of one sealed segment)
// are first fetched in a step after the one that wrote them.
enum { SRC_F16 = 0, SRC_E5M2 = 1, SRC_I8 = 2, SRC_STAGE = 3 };
constexpr uint32_t ROW_NONE = 0x80000000u;   // past every attention buffer (each below 2 GiB)
constexpr int AUX_PLAIN = 0, AUX_NT = 2, AUX_AGENT = 16;   // cache bits: none, nt, sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const void* base, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)(bytes < 0x7fffffffu ? bytes : 0x7fffffffu),
                                             0x00020000);
}
// Registers of one batch's raw rows, shared by the sources of a cache format
// (the INT8 sealed and open-segment sources use the same words).
template <int KVF>
struct KvBuf {
    uint32_t w[KVF == KV_INT8 ? 40 : 32];
};

// PG: a paged cache (batch step only): row p's page comes from the split's
// page-table entries staged in LDS (pt, first entry pt0); a row in a page
// that is not allocated reads as zeros like a row not fetched.
template <int HD, int SRC, bool P, bool PG = false>
struct KvSrc {
    using Geo = AttnGeo<HD>;
    // rows per lane per batch: 16 bytes per lane and row for fp16 rows, 8 for
    // the 8-bit codes, whose batches hold twice the rows (the same bytes)
    static constexpr int U = (SRC == SRC_E5M2 || SRC == SRC_I8) ? 8 : 4;
    static constexpr int BATCH = Geo::RPW * U;
    static constexpr bool WIDE = SRC == SRC_F16 || SRC == SRC_STAGE;
    static constexpr int RW = WIDE ? 4 : 2;   // words per row
    static constexpr int LOADS = 2 * U + (SRC == SRC_I8 ? 4 : 0);
    static constexpr int ES = WIDE ? 2 : 1;   // bytes per element
    static constexpr int AUX = SRC == SRC_F16    ? AUX_NT
                               : SRC == SRC_E5M2 ? ((P && HD == 64) ? AUX_AGENT : AUX_NT)
                               : SRC == SRC_I8   ? AUX_NT
                                                 : (P ? AUX_AGENT : AUX_PLAIN);
    static constexpr int AUX_META = P ? AUX_AGENT : AUX_PLAIN;
    static constexpr int KVF = SRC == SRC_I8 || SRC == SRC_STAGE ? KV_INT8 : SRC;
    using Buf = KvBuf<KVF>;
    static_assert(2 * U * RW + (SRC == SRC_I8 ? 8 : 0) <= (int)(sizeof(Buf) / 4), "KvBuf");

    static_assert(!PG || SRC == SRC_F16 || SRC == SRC_E5M2, "paged caches hold fp16 or E5M2 rows");
    __amdgpu_buffer_rsrc_t rk, rv, rmk, rmv;
    int g, ld, nseg, pos;
    int pshift, Hk, pt0, pt_n;
    const int* pt;

    __device__ __forceinline__ KvSrc(const AttnArgs& A, int g_, int pos_, const int* pt_ = nullptr, int pt0_ = 0,
                                     int pt_n_ = 0)
        : g(g_), pos(pos_), pt(pt_), pt0(pt0_), pt_n(pt_n_) {
        nseg = A.nseg;
        pshift = A.pshift;
        Hk = A.Hk;
        if constexpr (PG) {
            ld = 0;
            const size_t bytes = (size_t)A.npages * A.Hk * ((size_t)1 << A.pshift) * HD * ES;
            rk = attn_rsrc(A.kc, bytes);
            rv = attn_rsrc(A.vc, bytes);
        } else if constexpr (SRC == SRC_STAGE) {
            ld = SEG;
            rk = attn_rsrc(A.kst, (size_t)A.Hk * SEG * HD * 2);
            rv = attn_rsrc(A.vst, (size_t)A.Hk * SEG * HD * 2);
        } else {
            ld = A.ld;
            rk = attn_rsrc(A.kc, (size_t)A.Hk * A.ld * HD * ES);
            rv = attn_rsrc(A.vc, (size_t)A.Hk * A.ld * HD * ES);
        }
        if constexpr (SRC == SRC_I8) {
            rmk = attn_rsrc(A.kmeta, (size_t)A.Hk * A.nseg * 8);
            rmv = attn_rsrc(A.vmeta, (size_t)A.Hk * A.nseg * 8);
        }
    }
    __device__ __forceinline__ uint32_t row_off(int p, int j) const {
        if constexpr (PG) {
            // rows past the split (never fetched) may lie past the staged
            // entries: their index is clamped to an entry that exists
            const int e = (p >> pshift) - pt0;
            const int page = pt[e < pt_n ? e : 0];
            const int r = p & ((1 << pshift) - 1);
            return page < 0 ? ROW_NONE : ((((uint32_t)page * Hk + g) << pshift) + r) * (uint32_t)(HD * ES) + j * 8 * ES;
        }
        const int r = SRC == SRC_STAGE ? p % SEG : p;
        return ((uint32_t)(g * ld + r) * HD + j * 8) * ES;
    }
    // The raw rows of the batch starting at pb (pb <= p1; pb == p1: a batch
    // past the split's end, nothing fetched).
    __device__ __forceinline__ void load(int pb, int p1, Buf& b) const {
        const int lane = lane_id(), slot = lane / Geo::LPR, j = lane % Geo::LPR;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = pb + u * Geo::RPW + slot;
            const bool fetch = p < p1 && !(P && p == pos);
            const uint32_t off = fetch ? row_off(p, j) : ROW_NONE;
            if constexpr (WIDE) {
                const u4v k = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, AUX);
                const u4v v = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, AUX);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    b.w[(2 * u) * 4 + i] = k[i];
                    b.w[(2 * u + 1) * 4 + i] = v[i];
                }
            } else {
                const u2v k = __builtin_amdgcn_raw_buffer_load_b64(rk, off, 0, AUX);
                const u2v v = __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, AUX);
                b.w[(2 * u) * 2] = k.x;
                b.w[(2 * u) * 2 + 1] = k.y;
                b.w[(2 * u + 1) * 2] = v.x;
                b.w[(2 * u + 1) * 2 + 1] = v.y;
            }
        }
        if constexpr (SRC == SRC_I8) {
            // the (scale, zp) pairs of the at most two segments the batch's
            // rows fall in, one 8-byte load each for K and V (the same
            // address in every lane)
            const bool any = pb < p1;
            const int s0 = pb / SEG, s1 = (min(pb + BATCH, p1) - 1) / SEG;
            const uint32_t m0 = any ? (uint32_t)(g * nseg + s0) * 8 : ROW_NONE;
            const uint32_t m1 = any ? (uint32_t)(g * nseg + s1) * 8 : ROW_NONE;
            const u2v mk0 = __builtin_amdgcn_raw_buffer_load_b64(rmk, m0, 0, AUX_META);
            const u2v mv0 = __builtin_amdgcn_raw_buffer_load_b64(rmv, m0, 0, AUX_META);
            const u2v mk1 = __builtin_amdgcn_raw_buffer_load_b64(rmk, m1, 0, AUX_META);
            const u2v mv1 = __builtin_amdgcn_raw_buffer_load_b64(rmv, m1, 0, AUX_META);
            b.w[32] = mk0.x; b.w[33] = mk0.y; b.w[34] = mv0.x; b.w[35] = mv0.y;
            b.w[36] = mk1.x; b.w[37] = mk1.y; b.w[38] = mv1.x; b.w[39] = mv1.y;
        }
    }
    // Row u (position p) of the batch at pb as floats: which = 0 K, 1 V.
    // INT8 codes give code - zp; the row's scale is then applied once
    // (mul), to the row's score for K and to its softmax weight for V.
    static constexpr bool SCALED = SRC == SRC_I8;
    // Word k of the (scale, zp) pair for K (which = 0) or V of row p's
    // segment.  A select between two fixed words: an index that depends on
    // p would keep the buffer's metadata words in scratch memory.
    __device__ __forceinline__ uint32_t meta(const Buf& b, int pb, int p, int which, int k) const {
        const bool second = p >= (pb / SEG + 1) * SEG;
        const uint32_t w0 = which ? b.w[34 + k] : b.w[32 + k];
        const uint32_t w1 = which ? b.w[38 + k] : b.w[36 + k];
        return second ? w1 : w0;
    }
    __device__ __forceinline__ float mul(const Buf& b, int pb, int p, int which) const {
        return __uint_as_float(meta(b, pb, p, which, 0));
    }
    __device__ __forceinline__ void cvt(const Buf& b, int pb, int u, int p, int which, float (&f)[8]) const {
        const int base = (2 * u + which) * RW;
        if constexpr (WIDE) {
            const h8 v = as_h8(u4v{b.w[base], b.w[base + 1], b.w[base + 2], b.w[base + 3]});
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
        } else if constexpr (SRC == SRC_E5M2) {
            // an E5M2 byte is the high byte of the binary16 it encodes: two
            // bytes become a pair of halves in one byte permute
            typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const uint32_t x = b.w[base + d];
                const h2 lo = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0u, x, 0x010c000cu));
                const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0u, x, 0x030c020cu));
                f[4 * d] = (float)lo[0];
                f[4 * d + 1] = (float)lo[1];
                f[4 * d + 2] = (float)hi[0];
                f[4 * d + 3] = (float)hi[1];
            }
        } else {
            // INT8: code - zp with the zero point of the row's segment (the
            // batch's rows fall in the segment of pb or the next one)
            const float zp = __uint_as_float(meta(b, pb, p, which, 1));
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = (float)((b.w[base + (i >> 2)] >> ((i & 3) * 8)) & 0xffu) - zp;
        }
    }
};
// Scores are kept in log2 units: the query is pre-multiplied by
// scale * log2(e), so every exponential is one hardware exp2 (v_exp_f32).
constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A row replaced after conversion (the persistent kernel's row of the current
// step, whose K and V come from the exchange): active(pb, n) says whether
// rows [pb, pb + n) can hold it (the same in every lane), apply(p, which, f)
// replaces row p's converted K (which = 0) or V.
struct NoFix {
    __device__ __forceinline__ bool active(int, int) const { return false; }
    __device__ __forceinline__ void apply(int, int, float (&)[8]) const {}
};

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
    // One batch of U rows per lane: their scores against the pre-scaled
    // queries; then per slot one online-softmax update for the whole batch:
    // the new maximum, one rescale of the running sum and output, and the
    // batch's rows added in order.  A row's K is converted for its scores and
    // its V for the output, each once for all G heads; fix may replace a
    // converted row.  A slot that has seen no key yet (maximum -inf) keeps
    // its state.
    // Every product-sum is an explicit fma and nothing else is contracted:
    // the executors place this code in different blocks (the persistent
    // kernel's row fix branches inside it), and contraction decided per
    // block would round differently in each.
    template <class Src, class Buf, class Fix>
    __device__ __forceinline__ void batch(const float (&qv)[G][8], const Src& src, const Buf& b, int pb, int p1,
                                          const Fix& fix) {
#pragma clang fp contract(off)
        constexpr int U = Src::U;
        const int slot = lane_id() / AttnGeo<HD>::LPR;
        const bool fx = fix.active(pb, Src::BATCH);
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = pb + u * AttnGeo<HD>::RPW + slot;
            float kf[8];
            src.cvt(b, pb, u, p, 0, kf);
            if (fx) fix.apply(p, 0, kf);
            const float km = Src::SCALED ? src.mul(b, pb, p, 0) : 1.f;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) d = __builtin_fmaf(qv[h][i], kf[i], d);
                d = group_sum<AttnGeo<HD>::LPR>(d);
                if constexpr (Src::SCALED) d *= km;
                sc[u][h] = p < p1 ? d : -INFINITY;
            }
        }
        float e[U][G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mb = m[h];
#pragma unroll
            for (int u = 0; u < U; ++u) mb = fmaxf(mb, sc[u][h]);
            const bool none = mb == -INFINITY;
            const float c = none ? 1.f : exp2_fast(m[h] - mb);
            l[h] *= c;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[h][i] *= c;
#pragma unroll
            for (int u = 0; u < U; ++u) e[u][h] = none ? 0.f : exp2_fast(sc[u][h] - mb);
            m[h] = mb;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = pb + u * AttnGeo<HD>::RPW + slot;
            float vf[8];
            src.cvt(b, pb, u, p, 1, vf);
            if (fx) fix.apply(p, 1, vf);
            const float vm = Src::SCALED ? src.mul(b, pb, p, 1) : 1.f;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                l[h] += e[u][h];
                const float ew = Src::SCALED ? e[u][h] * vm : e[u][h];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[h][i] = __builtin_fmaf(ew, vf[i], o[h][i]);
            }
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
// attn_wave_run.  With three or more batches, every slot of a three-batch
// group loads, also past the wave's last batch (nothing is fetched there),
// and the loop exits only at the end of a group: an exit inside the group
// would give the loop header a path on which a group's loads are still
// pending, and the compiler would then wait for all of them there.
template <class Src, int NW>
__device__ __forceinline__ void attn_wave_first(const Src& src, int p0, int p1, int w, typename Src::Buf (&kb)[3]) {
    src.load(min(p0 + w * Src::BATCH, p1), p1, kb[0]);
}
template <class Src, int NW, int HD, int G, class Fix>
__device__ __forceinline__ void attn_wave_run(const Src& src, int p0, int p1, int w, const float (&qv)[G][8],
                                              AttnAcc<HD, G>& acc, typename Src::Buf (&kb)[3], const Fix& fix) {
    constexpr int STEP = NW * Src::BATCH;
    const int pf = p0 + w * Src::BATCH;
    if (pf >= p1) return;
    // one or two batches (short contexts): straight-line, nothing loaded past
    // the wave's last batch
    if (pf + 2 * STEP >= p1) {
        if (pf + STEP >= p1) {
            wait_vm<0>();
            __builtin_amdgcn_sched_barrier(0);
            acc.batch(qv, src, kb[0], pf, p1, fix);
        } else {
            src.load(pf + STEP, p1, kb[1]);
            __builtin_amdgcn_sched_barrier(0);
            wait_vm<Src::LOADS>();
            __builtin_amdgcn_sched_barrier(0);
            acc.batch(qv, src, kb[0], pf, p1, fix);
            wait_vm<0>();
            __builtin_amdgcn_sched_barrier(0);
            acc.batch(qv, src, kb[1], pf + STEP, p1, fix);
        }
        return;
    }
    src.load(pf + STEP, p1, kb[1]);
    for (int pg = pf; pg < p1; pg += 3 * STEP) {
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int pb = pg + r * STEP;
            src.load(min(pb + 2 * STEP, p1), p1, kb[(r + 2) % 3]);
            // all of them issued before the wait for batch pb's rows: the
            // two batches loaded after it may stay in flight (the wait also
            // settles a skipped slot's buffer, so that no path reaches the
            // loop header with it pending)
            __builtin_amdgcn_sched_barrier(0);
            wait_vm<2 * Src::LOADS>();
            __builtin_amdgcn_sched_barrier(0);
            if (pb < p1) acc.batch(qv, src, kb[r], pb, p1, fix);
        }
    }
}
// Calls f with the row source of a split: the cache format's rows, or for
// INT8 the sealed codes or (open: the open-segment split) the fp16 staging.
template <int HD, int KVF, class F>
__device__ __forceinline__ void with_src_paged(const AttnArgs& T, int g, int pos, const int* pt, int pt0, int pt_n,
                                               F f) {
    static_assert(KVF != KV_INT8, "paged caches hold fp16 or E5M2 rows");
    f(KvSrc<HD, KVF == KV_FP16 ? SRC_F16 : SRC_E5M2, false, true>(T, g, pos, pt, pt0, pt_n));
}
template <int HD, int KVF, bool P, class F>
__device__ __forceinline__ void with_src(const AttnArgs& T, int g, int pos, bool open, F f) {
    if constexpr (KVF == KV_INT8) {
        if (open)
            f(KvSrc<HD, SRC_STAGE, P>(T, g, pos));
        else
            f(KvSrc<HD, SRC_I8, P>(T, g, pos));
    } else {
        f(KvSrc<HD, KVF == KV_FP16 ? SRC_F16 : SRC_E5M2, P>(T, g, pos));
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
// Head h's wave weights f_w, its M and its L, and one output dim d: the
// products are explicit FMAs in wave order from zero, so whichever lane
// computes a value, and however many it computes, the bits are the same.
template <int HD, int G, int NW>
struct AttnWaves {
    float f[NW], M, L;
    __device__ __forceinline__ AttnWaves(const float* s_att, int h) {
#pragma clang fp contract(off)
        float mw[NW];
        M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            mw[w] = s_att[(w * G + h) * (HD + 2) + HD];
            M = fmaxf(M, mw[w]);
        }
        L = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            f[w] = mw[w] == -INFINITY ? 0.f : exp2_fast(mw[w] - M);
            L = __builtin_fmaf(f[w], s_att[(w * G + h) * (HD + 2) + HD + 1], L);
        }
    }
    __device__ __forceinline__ float o(const float* s_att, int h, int d) const {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v = __builtin_fmaf(f[w], s_att[(w * G + h) * (HD + 2) + d], v);
        return v;
    }
};
template <int HD, int G, int NW>
__device__ __forceinline__ void attn_combine(const float* s_att, AttnAcc<HD, G>& out) {
    const int j = lane_id() % AttnGeo<HD>::LPR;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const AttnWaves<HD, G, NW> aw(s_att, h);
        out.m[h] = aw.M;
        out.l[h] = aw.L;
#pragma unroll
        for (int i = 0; i < 8; ++i) out.o[h][i] = aw.o(s_att, h, j * 8 + i);
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
