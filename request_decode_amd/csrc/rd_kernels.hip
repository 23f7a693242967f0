// Decode-step kernels for gfx950 (CDNA4, wave64): the one-kernel-per-phase
// executor (eager launches, or the whole step captured into a hipGraph) and
// the standalone kernels of the C ABI.
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
#include "rd_phases.h"

namespace rd {

// ---- phase 1: RMSNorm + fused QKV GEMV + RoPE + KV append ------------------------
// Rows of the fused QKV matrix are re-ordered at load time so that each
// wave's two rows are a RoPE pair (j, j+hd/2) of one q or k head (or two
// consecutive rows of a v head): the rotation and the cache write happen in
// the GEMV epilogue with both halves of the pair in the same wave.
template <int KCH, bool EMB, int KVF>
__global__ __launch_bounds__(WG) void k_qkv(StepArgs A, LayerW Lw, int layer) {
    const int lane = lane_id(), wid = wave_id();
    const int D = A.D;
    const int N = (A.H + 2 * A.Hk) * A.hd;
    const int row0 = (blockIdx.x * 4 + wid) * 2;
    u4v w[2][KCH];
    load_rows<2, KCH>(Lw.wqkv, D, row0, row0 < N ? 2 : 0, w);
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
        load_x_f32_h<KCH>(A.x, D, xr);
    }
    rmsnorm_regs<KCH>(xr, Lw.g_attn, D, A.eps);
    if (row0 >= N) return;
    u4v xh[KCH];
    pack_x<KCH>(xr, xh);
    float acc[2];
    dot_rows<2, KCH>(w, xh, acc);
    if (lane == 0) {
        const QkvPair o = qkv_pair(A.hd, A.H, A.Hk, row0, acc[0], acc[1], A.rope + (size_t)pos * (A.hd / 2));
        if (o.kind == 0) {
            A.q[o.head * A.hd + o.d0] = o.y0;
            A.q[o.head * A.hd + o.d1] = o.y1;
        } else {
            const int which = o.kind == 2;
            kv_put<KVF, false>(A, layer, which, o.head, pos, o.d0, o.y0);
            kv_put<KVF, false>(A, layer, which, o.head, pos, o.d1, o.y1);
        }
    }
}

// ---- phase 2a: split-K attention partials, one wave per (kv-head, split) ---------
// The wave reads each K/V row of its key range once for all G query heads of
// the group.  Tasks past the splits in use at this position exit at once.
// PG: a paged cache (the batch step): the split's page-table entries are
// staged in LDS first; a sequence that sits the step out is skipped.
constexpr int PAGE_ENTRIES = 4096;   // page-table entries one split can span
template <int HD, int G, int KVF, bool PG = false>
__global__ __launch_bounds__(ATT_WAVES * WAVE) void k_attn(AttnArgs T0) {
    using Geo = AttnGeo<HD>;
    const AttnArgs T = attn_seq(T0, blockIdx.y);   // sequence blockIdx.y
    constexpr int NW = ATT_WAVES;
    __shared__ float s_att[NW * G * (HD + 2)];
    __shared__ int s_pt[PG ? PAGE_ENTRIES : 1];
    if constexpr (PG) {
        if (!*T.act_ptr) return;
    }
    const int pos = *T.pos_ptr, L = pos + 1;
    const SplitPlan pl = split_plan(L, T.S, KVF);
    const int t = blockIdx.x;   // one split of one kv-head per workgroup
    if (t >= T.Hk * pl.nact) return;
    const int g = t / pl.nact, s = t % pl.nact, w = wave_id();
    const int lane = lane_id(), j = lane % Geo::LPR;
    int p0, p1;
    split_range(pl, L, s, p0, p1);
    AttnAcc<HD, G> acc;
    acc.clear();
    auto run = [&](auto src) {
        using Src = decltype(src);
        typename Src::Buf kb[3];
        attn_wave_first<Src, NW>(src, p0, p1, w, kb);
        const float qs = T.scale * LOG2E;
        float qv[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i) qv[h][i] = T.q[(g * G + h) * HD + j * 8 + i] * qs;
        attn_wave_run<Src, NW>(src, p0, p1, w, qv, acc, kb, NoFix{});
    };
    if constexpr (PG) {
        const int pt0 = p0 >> T.pshift, npt = ((p1 - 1) >> T.pshift) - pt0 + 1;   // npt <= PAGE_ENTRIES (host check)
        for (int i = threadIdx.x; i < npt; i += ATT_WAVES * WAVE) s_pt[i] = T.ptab[pt0 + i];
        __syncthreads();
        with_src_paged<HD, KVF>(T, g, pos, s_pt, pt0, npt, run);
    } else {
        with_src<HD, KVF, false>(T, g, pos, s == pl.ncut, run);
    }
    acc.finish();
    attn_part_store<HD, G>(s_att, w, acc);
    __syncthreads();
    if (w != 0) return;
    attn_combine<HD, G, NW>(s_att, acc);
    if (lane < Geo::LPR) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float* dst = T.part + ((size_t)(g * G + h) * T.S + s) * (HD + 2);
#pragma unroll
            for (int i = 0; i < 8; ++i) dst[j * 8 + i] = acc.o[h][i];
            if (lane == 0) {
                dst[HD] = acc.m[h];
                dst[HD + 1] = acc.l[h];
            }
        }
    }
}

// ---- phase 2b: log-sum-exp merge, one wave per (query head, 64 dims); on the
// step that fills an INT8 segment the first merge wave of each kv-head seals
// it (after every split of this step has read the open segment).
template <int HD, int G, int KVF>
__global__ __launch_bounds__(WG) void k_merge(AttnArgs T0) {
    using Geo = AttnGeo<HD>;
    const AttnArgs T = attn_seq(T0, blockIdx.y);   // sequence blockIdx.y
    if (T.ptab && !*T.act_ptr) return;             // paged: the sequence sits this step out
    const int pos = *T.pos_ptr;
    const int nact = split_plan(pos + 1, T.S, KVF).nact;
    const int t = blockIdx.x * (WG / WAVE) + wave_id();
    if (t >= T.H * Geo::NPART) return;
    const int h = t / Geo::NPART, part = t % Geo::NPART, lane = lane_id();
    const float* base = T.part + (size_t)h * T.S * (HD + 2);
    float ms[MERGE_NC], ls[MERGE_NC];
#pragma unroll
    for (int c = 0; c < MERGE_NC; ++c) {
        const int s = c * 64 + lane;
        ms[c] = s < nact ? base[(size_t)s * (HD + 2) + HD] : -INFINITY;
        ls[c] = s < nact ? base[(size_t)s * (HD + 2) + HD + 1] : 0.f;
    }
    const MergeW mw = merge_weights(nact, ms, ls);
    const int d = part * 64 + lane;
    float num = 0.f;
#pragma unroll
    for (int c = 0; c < MERGE_NC; ++c) {
        if (c * 64 >= nact) break;
        float ov[64];
#pragma unroll
        for (int k = 0; k < 64; ++k) ov[k] = c * 64 + k < nact ? base[(size_t)(c * 64 + k) * (HD + 2) + d] : 0.f;
        merge_acc<64>(num, c, mw, ov);
    }
    T.out[h * HD + d] = num / mw.den;
    if constexpr (KVF == KV_INT8) {
        if (T.seal && (pos + 1) % SEG == 0 && part == 0 && h % G == 0) seal_head<HD, false>(T, h / G, pos);
    }
}

// ---- phases 3 and 5: GEMV + residual add (x[row] += W[row,:] . in) -------------
template <int KCH, int R>
__global__ __launch_bounds__(WG) void k_resid(const float* __restrict__ in, int K, const _Float16* __restrict__ W,
                                              float* __restrict__ x, int N) {
    const int lane = lane_id(), wid = wave_id();
    const int row0 = (blockIdx.x * 4 + wid) * R;
    u4v w[R][KCH];
    load_rows<R, KCH>(W, K, row0, max(0, min(R, N - row0)), w);
    float xr[KCH][8];
    load_x_f32<KCH>(in, K, xr);
    if (row0 >= N) return;
    u4v xh[KCH];
    pack_x<KCH>(xr, xh);
    float acc[R];
    dot_rows<R, KCH>(w, xh, acc);
    if (lane == 0)
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (row0 + r < N) x[row0 + r] += acc[r];
}

// ---- phase 4: RMSNorm + gate/up GEMV + SwiGLU (m_i = silu(gate_i) * up_i) -------
template <int KCH>
__global__ __launch_bounds__(WG) void k_gateup(StepArgs A, LayerW Lw) {
    const int lane = lane_id(), wid = wave_id();
    const int row0 = (blockIdx.x * 4 + wid) * 2;
    u4v w[2][KCH];
    load_rows<2, KCH>(Lw.wgu, A.D, row0, row0 < 2 * A.F ? 2 : 0, w);
    float xr[KCH][8];
    load_x_f32_h<KCH>(A.x, A.D, xr);
    rmsnorm_regs<KCH>(xr, Lw.g_ffn, A.D, A.eps);
    if (row0 >= 2 * A.F) return;
    u4v xh[KCH];
    pack_x<KCH>(xr, xh);
    float acc[2];
    dot_rows<2, KCH>(w, xh, acc);
    if (lane == 0) A.m[row0 >> 1] = silu_mul(acc[0], acc[1]);
}

// ---- phase 6: final RMSNorm + LM head + greedy argmax on the device ---------------
// Each wave streams a contiguous run of LM_ROWS rows in blocks of 4, with the
// next block's loads in flight while the current one is reduced.
constexpr int LM_ROWS = 16;
template <int KCH>
__global__ __launch_bounds__(WG) void k_lmhead(StepArgs A) {
    const int lane = lane_id(), wid = wave_id();
    const int rbeg = (blockIdx.x * 4 + wid) * LM_ROWS;
    const int rend = min(A.V, rbeg + LM_ROWS);
    u4v wa[4][KCH], wb[4][KCH];
    load_rows<4, KCH>(A.lm_head, A.D, rbeg, max(0, min(4, rend - rbeg)), wa);
    float xr[KCH][8];
    load_x_f32_h<KCH>(A.x, A.D, xr);
    rmsnorm_regs<KCH>(xr, A.g_final, A.D, A.eps);
    u4v xh[KCH];
    pack_x<KCH>(xr, xh);
    Best b{-INFINITY, INT_MAX};
    auto consume = [&](const u4v (&w)[4][KCH], int r0) {
        float acc[4];
        dot_rows<4, KCH>(w, xh, acc);
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (r0 + r < rend) {
                    A.logits[r0 + r] = acc[r];
                    if (!isfinite(acc[r])) atomicOr(&A.st->err, ERR_NONFINITE);
                    b = better(b, Best{acc[r], r0 + r});
                }
            }
        }
    };
    for (int r = rbeg; r < rend; r += 8) {
        load_rows<4, KCH>(A.lm_head, A.D, r + 4, max(0, min(4, rend - r - 4)), wb);
        consume(wa, r);
        if (r + 4 >= rend) break;
        load_rows<4, KCH>(A.lm_head, A.D, r + 8, max(0, min(4, rend - r - 8)), wa);
        consume(wb, r + 4);
    }
    b = block_best(b);
    Best fin;
    if (!argmax_finish(b, blockIdx.x, gridDim.x, A.arg_val, A.arg_idx, A.arg_cnt, &fin)) return;
    if (threadIdx.x == 0) {
        StepState* st = A.st;
        st->token[0] = fin.i;
        if (st->n_gen < A.max_ctx) A.gen_out[st->n_gen] = fin.i;
        st->n_gen += 1;
        st->pos += 1;
    }
}

// ---- standalone kernels (unit parity) --------------------------------------------
__global__ __launch_bounds__(WG) void k_e5m2(const uint16_t* __restrict__ in, uint8_t* __restrict__ out, size_t n) {
    for (size_t i = (size_t)blockIdx.x * WG + threadIdx.x; i < n; i += (size_t)gridDim.x * WG) out[i] = e5m2_encode(in[i]);
}

// One wave per segment (the seal of the decode step, called alone).
__global__ __launch_bounds__(WAVE) void k_seg_quant(const uint16_t* __restrict__ in, int seg_elems,
                                                   uint8_t* __restrict__ codes, float* __restrict__ meta) {
    const size_t off = (size_t)blockIdx.x * seg_elems;
    seal_segment<false>(in + off, seg_elems, codes + off, meta + (size_t)blockIdx.x * 2);
}

// ---- delta quantization of K/V segments ("Grok-3 v3.2.4 hot update deep
// dive", §3.2: the adjacent-token differences of the values, quantized to
// INT8).  A segment is n rows of hd fp16 values (hd % 8 == 0): its first row
// is kept as the anchor, and the differences x[p] - x[p-1] (binary32) of rows
// 1..n-1 are quantized together with the adaptive-range formula of
// seal_segment.  One workgroup per segment; a thread takes 8 consecutive
// differences at a time (16-byte loads of both rows, 8-byte code stores).
__device__ __forceinline__ void delta8(const uint16_t* x, int hd, int i, float (&d)[8]) {
    const h8 a = as_h8(ld16(x + hd + i)), b = as_h8(ld16(x + i));
#pragma unroll
    for (int k = 0; k < 8; ++k) d[k] = (float)a[k] - (float)b[k];
}
__global__ __launch_bounds__(WG) void k_delta_seal(const uint16_t* __restrict__ in, int n, int hd,
                                                   uint16_t* __restrict__ anchor, uint8_t* __restrict__ codes,
                                                   float* __restrict__ meta) {
    __shared__ float s_mn[WG / WAVE], s_mx[WG / WAVE];
    const size_t seg = blockIdx.x;
    const uint16_t* x = in + seg * (size_t)n * hd;
    const int m = (n - 1) * hd;   // differences: element i is x[hd + i] - x[i]
    for (int j = threadIdx.x * 8; j < hd; j += WG * 8)
        *reinterpret_cast<u4v*>(anchor + seg * hd + j) = ld16(x + j);
    if (m == 0) {   // one row: no differences
        if (threadIdx.x == 0) {
            meta[seg * 2] = 1.0f;
            meta[seg * 2 + 1] = 0.0f;
        }
        return;
    }
    // segments of up to DELTA_REG groups of 8 per thread (128 x 128: 8) keep
    // their differences in registers for the second pass; larger ones read
    // the segment again
    constexpr int DELTA_REG = 8;
    const bool in_regs = m <= DELTA_REG * WG * 8;
    float dr[DELTA_REG][8];
    float mn = INFINITY, mx = -INFINITY;
    if (in_regs) {
#pragma unroll
        for (int r = 0; r < DELTA_REG; ++r) {
            const int i = (threadIdx.x + r * WG) * 8;
            if (i < m) {
                delta8(x, hd, i, dr[r]);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    mn = fminf(mn, dr[r][k]);
                    mx = fmaxf(mx, dr[r][k]);
                }
            }
        }
    } else {
        for (int i = threadIdx.x * 8; i < m; i += WG * 8) {
            float d[8];
            delta8(x, hd, i, d);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                mn = fminf(mn, d[k]);
                mx = fmaxf(mx, d[k]);
            }
        }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane_id() == 0) {
        s_mn[wave_id()] = mn;
        s_mx[wave_id()] = mx;
    }
    __syncthreads();
    mn = s_mn[0];
    mx = s_mx[0];
#pragma unroll
    for (int w = 1; w < WG / WAVE; ++w) {
        mn = fminf(mn, s_mn[w]);
        mx = fmaxf(mx, s_mx[w]);
    }
    float scale = (mx - mn) / 255.0f;
    if (!(scale > 0.0f)) scale = mn != 0.0f ? fabsf(mn) : 1.0f;   // one repeated difference (seal_segment)
    const float zp = rintf(-mn / scale);
    uint8_t* c = codes + seg * (size_t)m;
    auto code8 = [&](const float (&d)[8]) {
        uint64_t packed = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            packed |= (uint64_t)(unsigned)fminf(fmaxf(rintf(d[k] / scale) + zp, 0.0f), 255.0f) << (8 * k);
        return packed;
    };
    if (in_regs) {
#pragma unroll
        for (int r = 0; r < DELTA_REG; ++r) {
            const int i = (threadIdx.x + r * WG) * 8;
            if (i < m) *reinterpret_cast<uint64_t*>(c + i) = code8(dr[r]);
        }
    } else {
        for (int i = threadIdx.x * 8; i < m; i += WG * 8) {   // the segment again (it is in the cache by now)
            float d[8];
            delta8(x, hd, i, d);
            *reinterpret_cast<uint64_t*>(c + i) = code8(d);
        }
    }
    if (threadIdx.x == 0) {
        meta[seg * 2] = scale;
        meta[seg * 2 + 1] = zp;
    }
}

// The rows of delta-sealed segments restored: one thread per (segment, 8
// consecutive elements of a row), adding the dequantized differences in row
// order: y[0] = anchor, y[p] = y[p-1] + (code - zp) * scale (binary32,
// rounded after each operation; 8 independent sums per thread).
__global__ __launch_bounds__(WG) void k_delta_restore(const uint16_t* __restrict__ anchor,
                                                      const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ meta, int n_seg, int n, int hd,
                                                      float* __restrict__ out) {
#pragma clang fp contract(off)   // a product and a sum, each rounded (no fused multiply-add)
    const int g8 = hd / 8;
    const size_t t = (size_t)blockIdx.x * WG + threadIdx.x;
    if (t >= (size_t)n_seg * g8) return;
    const size_t seg = t / g8;
    const int j = (int)(t % g8) * 8;
    const float scale = meta[seg * 2], zp = meta[seg * 2 + 1];
    const h8 a = as_h8(ld16(anchor + seg * hd + j));
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = (float)a[k];
    float* o = out + seg * (size_t)n * hd + j;
    const uint8_t* c = codes + seg * (size_t)(n - 1) * hd + j;
    reinterpret_cast<float4*>(o)[0] = float4{y[0], y[1], y[2], y[3]};
    reinterpret_cast<float4*>(o)[1] = float4{y[4], y[5], y[6], y[7]};
    for (int p = 1; p < n; ++p) {
        const uint64_t cw = *reinterpret_cast<const uint64_t*>(c + (size_t)(p - 1) * hd);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float d = ((float)(unsigned)((cw >> (8 * k)) & 0xffu) - zp) * scale;
            y[k] = y[k] + d;
        }
        float* op = o + (size_t)p * hd;
        reinterpret_cast<float4*>(op)[0] = float4{y[0], y[1], y[2], y[3]};
        reinterpret_cast<float4*>(op)[1] = float4{y[4], y[5], y[6], y[7]};
    }
}

__global__ __launch_bounds__(WG) void k_argmax(const float* __restrict__ v, int n, int* out, float* pv, int* pi,
                                               int* cnt) {
    Best b{-INFINITY, INT_MAX};
    for (int i = blockIdx.x * WG + threadIdx.x; i < n; i += gridDim.x * WG) b = better(b, Best{v[i], i});
    b = block_best(b);
    Best fin;
    if (argmax_finish(b, blockIdx.x, gridDim.x, pv, pi, cnt, &fin) && threadIdx.x == 0) *out = fin.i;
}

// ============================================================================
// Host launchers
// ============================================================================
int kch_for(int K) {
    const int need = (K + 511) / 512;
    const int opts[] = {1, 2, 4, 8, 11, 16};
    for (int o : opts)
        if (o >= need) return o;
    return -1;
}

namespace {

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
    const int wpb = WG / WAVE;
    const int nseq = A.nseq > 1 ? A.nseq : 1;
    dim3 grid(A.Hk * A.S, nseq), ablock(ATT_WAVES * WAVE), block(WG);   // k_attn: one split per workgroup
    dim3 mgrid((A.H * (hd / 64) + wpb - 1) / wpb, nseq);
#define RD_ATT(HDv, Gv)                                                                      \
    if (hd == HDv && G == Gv) {                                                              \
        if constexpr (KVF != KV_INT8) {                                                      \
            if (A.ptab) hipLaunchKernelGGL((k_attn<HDv, Gv, KVF, true>), grid, ablock, 0, s, A); \
            else hipLaunchKernelGGL((k_attn<HDv, Gv, KVF>), grid, ablock, 0, s, A);              \
        } else {                                                                             \
            if (A.ptab) return hipErrorInvalidValue;                                         \
            hipLaunchKernelGGL((k_attn<HDv, Gv, KVF>), grid, ablock, 0, s, A);                   \
        }                                                                                    \
        hipLaunchKernelGGL((k_merge<HDv, Gv, KVF>), mgrid, block, 0, s, A);                  \
        return hipGetLastError();                                                            \
    }
    RD_ATT(128, 1) RD_ATT(128, 2) RD_ATT(128, 4) RD_ATT(128, 8)
    RD_ATT(64, 1) RD_ATT(64, 2) RD_ATT(64, 4) RD_ATT(64, 8)
#undef RD_ATT
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

hipError_t launch_attn_any(const AttnArgs& A, int kvfmt, int hd, int G, hipStream_t s) {
    switch (kvfmt) {
        case KV_FP16: return launch_attn_t<KV_FP16>(A, hd, G, s);
        case KV_E5M2: return launch_attn_t<KV_E5M2>(A, hd, G, s);
        case KV_INT8: return launch_attn_t<KV_INT8>(A, hd, G, s);
    }
    return hipErrorInvalidValue;
}

int lm_head_workgroups(int V) { return (V + 4 * LM_ROWS - 1) / (4 * LM_ROWS); }

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

// One phase of one layer: 0 QKV (first=true: the layer-0 variant that reads
// the embedding), 1 attention, 2 output projection, 3 gate/up, 4 down.
static hipError_t launch_layer_phase(const StepArgs& A, int phase, int l, bool first, hipStream_t s) {
    const LayerW& Lw = A.layers[l];
    switch (phase) {
        case 0: return first ? launch_qkv<true>(A, Lw, l, s) : launch_qkv<false>(A, Lw, l, s);
        case 1: return launch_attn_any(attn_args(A, l), A.kvfmt, A.hd, A.H / A.Hk, s);
        case 2: return launch_resid(A.a, A.H * A.hd, Lw.wo, A.x, A.D, s);
        case 3: {
            dim3 grid((2 * A.F + 7) / 8), block(WG);
            RD_KCH_SWITCH(kch_for(A.D), hipLaunchKernelGGL((k_gateup<KC>), grid, block, 0, s, A, Lw))
            return hipGetLastError();
        }
        case 4: return launch_resid(A.m, A.F, Lw.wd, A.x, A.D, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_phase(const StepArgs& A, int phase, int layer, hipStream_t s) {
    return launch_layer_phase(A, phase, layer, false, s);
}

hipError_t launch_step(const StepArgs& A, hipStream_t s) {
    if (A.B > 1) return launch_step_batch(A, s);
    for (int l = 0; l < A.n_layers; ++l)
        for (int ph = 0; ph < 5; ++ph) {
            hipError_t e = launch_layer_phase(A, ph, l, l == 0, s);
            if (e != hipSuccess) return e;
        }
    dim3 grid(lm_head_workgroups(A.V)), block(WG);
    RD_KCH_SWITCH(kch_for(A.D), hipLaunchKernelGGL((k_lmhead<KC>), grid, block, 0, s, A))
    return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& A, int kvfmt, int hd, int G, hipStream_t s) {
    return launch_attn_any(A, kvfmt, hd, G, s);
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
    hipLaunchKernelGGL(k_seg_quant, dim3(n_seg), dim3(WAVE), 0, s, in, seg_elems, codes, meta);
    return hipGetLastError();
}

hipError_t launch_delta_seal(const uint16_t* in, int n_seg, int n, int hd, uint16_t* anchor, uint8_t* codes,
                             float* meta, hipStream_t s) {
    if (n_seg == 0) return hipSuccess;
    hipLaunchKernelGGL(k_delta_seal, dim3(n_seg), dim3(WG), 0, s, in, n, hd, anchor, codes, meta);
    return hipGetLastError();
}

hipError_t launch_delta_restore(const uint16_t* anchor, const uint8_t* codes, const float* meta, int n_seg, int n,
                                int hd, float* out, hipStream_t s) {
    const size_t threads = (size_t)n_seg * (hd / 8);
    if (threads == 0) return hipSuccess;
    hipLaunchKernelGGL(k_delta_restore, dim3((unsigned)((threads + WG - 1) / WG)), dim3(WG), 0, s, anchor, codes,
                       meta, n_seg, n, hd, out);
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
