// Batched prefill for gfx950: the prompt's tokens go through each layer
// together, as matrix products on the matrix cores, instead of one decode
// step per token.  The pages describe the prompt and the decode steps as
// separate phases ("LLM inference architecture rebuild", the batch planner
// layer's prefill/decode separation) and the prompt's attention as a
// block-wise FlashAttention schedule ("How the xAI engineering team cut Grok
// Bot latency to milliseconds", §2.1).  What it computes is the decode
// step's definition for every prompt position: position p's K/V rows, from
// the same layer math, and position p's attention over positions 0..p as
// stored in the cache format; the rows it leaves in the cache are what the
// decode steps read next.
//
// A chunk of up to TC tokens at positions p0 .. p0+T-1 runs, per layer:
//   RMSNorm (fp16 operand rows) -> QKV GEMM with RoPE and the K/V store as
//   its epilogue -> (INT8) seal of the segments the chunk completes ->
//   causal attention -> O GEMM added into the residual rows -> RMSNorm ->
//   gate/up GEMM with SwiGLU as its epilogue -> down GEMM added into the
//   residual rows.
// Every operand of a GEMM is fp16 and every product sums in fp32, as in the
// decode step; the summation order is the matrix cores' (the decode step's
// dot products are v_dot2 chains), so the rows agree with the decode step's
// within rounding, not bit for bit.
#include "rd_phases.h"

namespace rd {

namespace {

typedef _Float16 hv8 __attribute__((ext_vector_type(8)));
typedef float fv4 __attribute__((ext_vector_type(4)));

constexpr int PT = 256;   // threads per workgroup (4 waves)

// ---- embedding and RMSNorm ---------------------------------------------------------
__global__ __launch_bounds__(PT) void k_pf_embed(const int* __restrict__ tok, int T, const _Float16* __restrict__ E,
                                                 int D, float* __restrict__ X) {
    const int t = blockIdx.x;
    if (t >= T) return;
    const _Float16* e = E + (size_t)tok[t] * D;
    for (int i = threadIdx.x; i < D; i += PT) X[(size_t)t * D + i] = (float)e[i];
}

// Xn[t] = fp16(h * (mean(h^2) + eps)^-1/2 * g) with h = fp16(X[t]): one wave
// per row (the residual enters a norm as an fp16 GEMV operand, as in the
// decode step).  D % 8 == 0.
__global__ __launch_bounds__(PT) void k_pf_norm(const float* __restrict__ X, int T, int D,
                                                const _Float16* __restrict__ g, float eps, _Float16* __restrict__ Xn) {
    const int t = blockIdx.x * (PT / WAVE) + wave_id();
    if (t >= T) return;
    const int lane = lane_id();
    const float* x = X + (size_t)t * D;
    float ss = 0.f;
    for (int i = lane * 8; i < D; i += WAVE * 8)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float h = (float)(_Float16)x[i + k];
            ss += h * h;
        }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + eps);
    for (int i = lane * 8; i < D; i += WAVE * 8) {
        const h8 gv = as_h8(ld16(g + i));
        h8 o;
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = (_Float16)((float)(_Float16)x[i + k] * inv * (float)gv[k]);
        *reinterpret_cast<h8*>(Xn + (size_t)t * D + i) = o;
    }
}

// ---- GEMM on the matrix cores ------------------------------------------------------
// C[t][n] = sum_k A[t][k] * W[n][k] for t < T, n < N; A fp16 [T][K] (row
// stride K), W fp16 [N][K]; K % 32 == 0.  A workgroup computes a 128 x 128
// tile in steps of 32 columns of K, staged through LDS (double-buffered,
// rows padded to 40 halves against bank conflicts); wave w owns the 64 x 64
// quarter (w / 2, w % 2) as 4 x 4 tiles of v_mfma_f32_16x16x32_f16.  With
// the tile's operands A (rows: tokens) and B (rows: weight rows), lane l
// supplies row l % 16 and columns 8 (l / 16) .. +7 of the 32-column step,
// and the result lane l holds C[4 (l / 16) + j][l % 16], j = 0..3.
constexpr int GB = 128, GK = 32, GLD = 40;
enum { PE_STORE = 0, PE_RESID = 1, PE_SWIGLU = 2, PE_QKV = 3 };

struct PfArgs {
    int T, p0, layer, Tc;      // chunk rows, their first position, layer, row stride of the chunk buffers
    float* q;                  // QKV: [T][H*hd] rotated queries (fp32)
    _Float16* kt;              // QKV: [Hk][Tc][hd] new K rows (fp16), and V after Hk*Tc*hd
};

template <int EPI, int KVF>
__global__ __launch_bounds__(PT) void k_pf_gemm(const _Float16* __restrict__ Am, const _Float16* __restrict__ W,
                                                void* __restrict__ out, int T, int N, int K, StepArgs SA, PfArgs PA) {
    __shared__ __attribute__((aligned(16))) _Float16 As[2][GB * GLD];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[2][GB * GLD];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int t0 = blockIdx.y * GB, n0 = blockIdx.x * GB;
    // global -> LDS: thread tid moves rows tid / 4 and tid / 4 + 64, chunk tid % 4
    const int lr = tid >> 2, lc = (tid & 3) * 8;
    auto gload = [&](int k0, u4v (&a)[2], u4v (&b)[2]) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int ta = t0 + lr + 64 * r, nb = n0 + lr + 64 * r;
            a[r] = ta < T ? ld16(Am + (size_t)ta * K + k0 + lc) : u4v{0u, 0u, 0u, 0u};
            b[r] = nb < N ? ld16(W + (size_t)nb * K + k0 + lc) : u4v{0u, 0u, 0u, 0u};
        }
    };
    auto sstore = [&](int buf, const u4v (&a)[2], const u4v (&b)[2]) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            *reinterpret_cast<u4v*>(&As[buf][(lr + 64 * r) * GLD + lc]) = a[r];
            *reinterpret_cast<u4v*>(&Bs[buf][(lr + 64 * r) * GLD + lc]) = b[r];
        }
    };
    fv4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fv4{0.f, 0.f, 0.f, 0.f};
    u4v ra[2], rb[2];
    gload(0, ra, rb);
    sstore(0, ra, rb);
    __syncthreads();
    const int nk = K / GK;
    const int fr = lane & 15, fc = (lane >> 4) * 8;
    for (int kb = 0; kb < nk; ++kb) {
        const int cur = kb & 1;
        if (kb + 1 < nk) gload((kb + 1) * GK, ra, rb);
        u4v af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            af[i] = *reinterpret_cast<const u4v*>(&As[cur][(wm * 64 + i * 16 + fr) * GLD + fc]);
            bf[i] = *reinterpret_cast<const u4v*>(&Bs[cur][(wn * 64 + i * 16 + fr) * GLD + fc]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(hv8, af[i]),
                                                                   __builtin_bit_cast(hv8, bf[j]), acc[i][j], 0, 0, 0);
        if (kb + 1 < nk) sstore(cur ^ 1, ra, rb);
        __syncthreads();
    }
    // epilogue: lane holds rows t0 + 64 wm + 16 i + 4 (lane / 16) + e, columns n0 + 64 wn + 16 j + lane % 16
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 64 + j * 16 + (lane & 15);
            float part[4];
            if constexpr (EPI == PE_SWIGLU || EPI == PE_QKV) {
#pragma unroll
                for (int e = 0; e < 4; ++e) part[e] = __shfl_xor(acc[i][j][e], 1);   // the pair's other column
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = t0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
                if (t >= T || n >= N) continue;
                const float v = acc[i][j][e];
                if constexpr (EPI == PE_STORE) {
                    reinterpret_cast<float*>(out)[(size_t)t * N + n] = v;
                } else if constexpr (EPI == PE_RESID) {
                    reinterpret_cast<float*>(out)[(size_t)t * N + n] += v;
                } else if constexpr (EPI == PE_SWIGLU) {
                    // rows 2i (gate) and 2i + 1 (up) -> m_i, fp16 (the decode step's silu_mul)
                    if ((n & 1) == 0) reinterpret_cast<_Float16*>(out)[(size_t)t * (N / 2) + n / 2] =
                        (_Float16)silu_mul(v, part[e]);
                } else {
                    if ((n & 1) != 0) continue;
                    const int pos = PA.p0 + t;
                    const QkvPair o = qkv_pair(SA.hd, SA.H, SA.Hk, n, v, part[e], SA.rope + (size_t)pos * (SA.hd / 2));
                    if (o.kind == 0) {
                        float* qd = PA.q + (size_t)t * SA.H * SA.hd + o.head * SA.hd;
                        qd[o.d0] = o.y0;
                        qd[o.d1] = o.y1;
                    } else {
                        const int which = o.kind == 2;
                        _Float16* kt = PA.kt + (size_t)which * SA.Hk * PA.Tc * SA.hd +
                                       ((size_t)o.head * PA.Tc + t) * SA.hd;
                        kt[o.d0] = (_Float16)o.y0;
                        kt[o.d1] = (_Float16)o.y1;
                        if constexpr (KVF != KV_INT8) {   // fp16 / E5M2 rows straight into the cache
                            kv_put<KVF, false>(SA, PA.layer, which, o.head, pos, o.d0, o.y0);
                            kv_put<KVF, false>(SA, PA.layer, which, o.head, pos, o.d1, o.y1);
                        }
                    }
                }
            }
        }
}

// ---- INT8: segments the chunk completes, and the open segment's staging rows -----------
// One workgroup per (K/V, kv head, segment touched by the chunk).  STAGE =
// false (before the attention): the segment's 128 rows are gathered into
// LDS in fp16 (rows before p0 from the staging rows the cache holds, the
// chunk's rows from kt) and a complete segment is quantized by the decode
// step's seal (one wave).  STAGE = true (after the attention, which still
// reads the staging rows of the segment open at p0): the new rows of a
// segment the chunk leaves open go to the staging rows.
template <int HD, bool STAGE>
__global__ __launch_bounds__(PT) void k_pf_seal(StepArgs SA, PfArgs PA) {
    __shared__ __attribute__((aligned(16))) uint16_t seg[SEG * HD];
    const int s0 = PA.p0 / SEG, s_end = (PA.p0 + PA.T - 1) / SEG;
    const int nsg = s_end - s0 + 1;
    const int which = blockIdx.x / (SA.Hk * nsg), rem = blockIdx.x % (SA.Hk * nsg);
    const int g = rem / nsg, s = s0 + rem % nsg;
    const AttnArgs T = attn_args(SA, PA.layer);
    uint16_t* stage = (which ? T.vst : T.kst) + (size_t)g * SEG * HD;
    const _Float16* kt = PA.kt + (size_t)which * SA.Hk * PA.Tc * HD + (size_t)g * PA.Tc * HD;
    const int first = s * SEG, last = min(first + SEG, PA.p0 + PA.T);   // rows [first, last) exist
    if constexpr (STAGE) {
        if (last - first == SEG) return;
        for (int i = threadIdx.x; i < (last - first) * HD / 8; i += PT) {
            const int r = i / (HD / 8), c = (i % (HD / 8)) * 8, p = first + r;
            if (p >= PA.p0) *reinterpret_cast<u4v*>(stage + (size_t)r * HD + c) = ld16(kt + (size_t)(p - PA.p0) * HD + c);
        }
        return;
    }
    for (int i = threadIdx.x; i < SEG * HD / 8; i += PT) {
        const int r = i / (HD / 8), c = (i % (HD / 8)) * 8, p = first + r;
        u4v v = u4v{0u, 0u, 0u, 0u};
        if (p < PA.p0) v = ld16(stage + (size_t)r * HD + c);
        else if (p < last) v = ld16(kt + (size_t)(p - PA.p0) * HD + c);
        *reinterpret_cast<u4v*>(&seg[r * HD + c]) = v;
    }
    __syncthreads();
    if (last - first == SEG && threadIdx.x < WAVE) {
        uint8_t* codes = reinterpret_cast<uint8_t*>(which ? T.vcw : T.kcw) + ((size_t)g * T.ld + first) * HD;
        float* meta = (which ? T.vmeta : T.kmeta) + ((size_t)g * T.nseg + s) * 2;
        seal_segment<false>(seg, SEG * HD, codes, meta);
    }
}

// ---- causal attention of the chunk's queries on the matrix cores ----------------------
// Workgroup = (block of 64 positions aligned to 64, query head h); wave w
// owns 16 query rows.  Keys run in blocks of 64 up to the block's last
// position.  Per key block: K and V rows in fp16 into LDS (V transposed:
// [dim][key]), S = Q K^T (scores in log2 units: q pre-scaled by
// scale * log2 e and rounded to fp16), causal mask, online softmax per row
// (running max m, sum l), P = 2^(S - m) rounded to fp16 through LDS into
// the operand layout, O += P V.  Rows as stored: fp16, or E5M2 read as the
// fp16 with that high byte, or INT8 (a row of an earlier segment than the
// query block's: (code - zp) * scale rounded to fp16; of the same segment:
// its fp16 value, from the staging rows or the chunk's kt).
template <int HD, int KVF>
__global__ __launch_bounds__(PT) void k_pf_attn(StepArgs SA, PfArgs PA, _Float16* __restrict__ out) {
    constexpr int KB = 64, KLD = HD + 8, VLD = KB + 8, PLD = KB + 8;
    __shared__ __attribute__((aligned(16))) _Float16 Ks[KB * KLD];
    __shared__ __attribute__((aligned(16))) _Float16 Vt[HD * VLD];
    __shared__ __attribute__((aligned(16))) _Float16 Ps[4][16 * PLD];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h = blockIdx.y, G = SA.H / SA.Hk, g = h / G;
    const int qa = (PA.p0 / 64 + blockIdx.x) * 64;         // first position of the block
    const int q_lo = max(qa, PA.p0), q_hi = min(qa + 64, PA.p0 + PA.T);   // its positions in the chunk
    if (q_lo >= q_hi) return;
    const AttnArgs T = attn_args(SA, PA.layer);
    const int sq = qa / SEG;                               // the block's segment (INT8)
    const int fr = lane & 15, fq = lane >> 4;
    // queries of this wave: positions qa + 16 w + fr (A operand rows)
    const float qs = SA.scale * LOG2E;
    u4v qf[HD / 32];
    {
        const int p = qa + 16 * w + fr;
        const bool ok = p >= q_lo && p < q_hi;
        const float* qr = PA.q + (size_t)(ok ? p - PA.p0 : 0) * SA.H * HD + h * HD;
#pragma unroll
        for (int ks = 0; ks < HD / 32; ++ks) {
            h8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = ok ? (_Float16)(qr[ks * 32 + fq * 8 + i] * qs) : (_Float16)0.f;
            qf[ks] = __builtin_bit_cast(u4v, v);
        }
    }
    fv4 o[HD / 16];
#pragma unroll
    for (int d = 0; d < HD / 16; ++d) o[d] = fv4{0.f, 0.f, 0.f, 0.f};
    float m[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        m[e] = -INFINITY;
        l[e] = 0.f;
    }
    const _Float16* ktb = PA.kt + (size_t)g * PA.Tc * HD;
    const _Float16* vtb = PA.kt + (size_t)SA.Hk * PA.Tc * HD + (size_t)g * PA.Tc * HD;
    const int kend = q_hi;                                 // keys 0 .. q_hi - 1
    for (int k0 = 0; k0 < kend; k0 += KB) {
        __syncthreads();   // the previous block's K, V and P are no longer read
        // K and V rows k0 .. k0 + 63 as fp16: thread tid loads 8 elements of
        // row tid / (HD / 8) (+ 256 / (HD / 8) per pass)
        constexpr int CPR = HD / 8, RPP = PT / CPR;
        for (int r = tid / CPR; r < KB; r += RPP) {
            const int c = (tid % CPR) * 8, p = k0 + r;
            h8 kv[2];
#pragma unroll
            for (int which = 0; which < 2; ++which) {
                h8 v;
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = (_Float16)0.f;
                if (p < kend) {
                    const size_t row = (size_t)g * T.ld + p;
                    const void* base = which ? T.vc : T.kc;
                    if constexpr (KVF == KV_FP16) {
                        v = as_h8(ld16(reinterpret_cast<const _Float16*>(base) + row * HD + c));
                    } else if constexpr (KVF == KV_E5M2) {
                        const u2v b = ld8(reinterpret_cast<const uint8_t*>(base) + row * HD + c);
#pragma unroll
                        for (int i = 0; i < 8; ++i) v[i] = e5m2_decode((uint8_t)(b[i >> 2] >> ((i & 3) * 8)));
                    } else {
                        if (p / SEG < sq) {
                            const u2v b = ld8(reinterpret_cast<const uint8_t*>(base) + row * HD + c);
                            const float* mt = (which ? T.vmeta : T.kmeta) + ((size_t)g * T.nseg + p / SEG) * 2;
                            const float sc = mt[0], zp = mt[1];
#pragma unroll
                            for (int i = 0; i < 8; ++i)
                                v[i] = (_Float16)(((float)((b[i >> 2] >> ((i & 3) * 8)) & 0xffu) - zp) * sc);
                        } else if (p >= PA.p0) {
                            v = as_h8(ld16((which ? vtb : ktb) + (size_t)(p - PA.p0) * HD + c));
                        } else {
                            const uint16_t* st = (which ? T.vst : T.kst) + ((size_t)g * SEG + p % SEG) * HD + c;
                            v = as_h8(ld16(st));
                        }
                    }
                }
                kv[which] = v;
            }
            *reinterpret_cast<h8*>(&Ks[r * KLD + c]) = kv[0];
#pragma unroll
            for (int i = 0; i < 8; ++i) Vt[(c + i) * VLD + r] = kv[1][i];
        }
        __syncthreads();
        // S = Q K^T: 4 tiles of 16 keys
        fv4 sc[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            sc[kt] = fv4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < HD / 32; ++ks) {
                const u4v kf = *reinterpret_cast<const u4v*>(&Ks[(kt * 16 + fr) * KLD + ks * 32 + fq * 8]);
                sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(hv8, qf[ks]),
                                                                __builtin_bit_cast(hv8, kf), sc[kt], 0, 0, 0);
            }
        }
        // mask and online softmax: lane holds rows 4 fq + e, keys k0 + 16 kt + fr
        float mb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int qp = qa + 16 * w + 4 * fq + e;
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const int kp = k0 + kt * 16 + fr;
                if (kp > qp || kp >= kend) sc[kt][e] = -INFINITY;
                mx = fmaxf(mx, sc[kt][e]);
            }
            // max over the 16 lanes of this row group (quad swaps, then row
            // rotations by 4 and 8: every lane ends with the row's maximum)
            mx = fmaxf(mx, dpp_f<0xB1>(mx));
            mx = fmaxf(mx, dpp_f<0x4E>(mx));
            mx = fmaxf(mx, dpp_f<0x124>(mx));
            mx = fmaxf(mx, dpp_f<0x128>(mx));
            mb[e] = fmaxf(m[e], mx);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float mrow = mb[e];
            const float mn = mrow == -INFINITY ? 0.f : mrow;
            const float c = m[e] == -INFINITY ? 0.f : exp2_fast(m[e] - mn);
            float ps = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const float pv = sc[kt][e] == -INFINITY ? 0.f : exp2_fast(sc[kt][e] - mn);
                const _Float16 ph = (_Float16)pv;
                ps += (float)ph;
                Ps[w][(4 * fq + e) * PLD + kt * 16 + fr] = ph;
            }
            // row sum over the 16 lanes
            ps += dpp_f<0xB1>(ps);
            ps += dpp_f<0x4E>(ps);
            ps += dpp_f<0x124>(ps);
            ps += dpp_f<0x128>(ps);
            ps = __shfl(ps, lane & ~15, WAVE);
            l[e] = l[e] * c + ps;
            m[e] = mrow;
#pragma unroll
            for (int d = 0; d < HD / 16; ++d) o[d][e] *= c;
        }
        __syncthreads();   // P written (each wave reads only its own P, but keep LDS ordered)
        // O += P V: A = P rows (16 queries) x 32 keys, B = V^T rows (16 dims) x 32 keys
#pragma unroll
        for (int ks = 0; ks < KB / 32; ++ks) {
            const u4v pf = *reinterpret_cast<const u4v*>(&Ps[w][fr * PLD + ks * 32 + fq * 8]);
#pragma unroll
            for (int d = 0; d < HD / 16; ++d) {
                const u4v vf = *reinterpret_cast<const u4v*>(&Vt[(d * 16 + fr) * VLD + ks * 32 + fq * 8]);
                o[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(hv8, pf), __builtin_bit_cast(hv8, vf),
                                                              o[d], 0, 0, 0);
            }
        }
    }
    // out[p][h*HD + d] = fp16(O / l): lane holds rows 4 fq + e, dims 16 d + fr
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int p = qa + 16 * w + 4 * fq + e;
        if (p < q_lo || p >= q_hi) continue;
        const float inv = 1.0f / l[e];
        _Float16* orow = out + (size_t)(p - PA.p0) * SA.H * HD + h * HD;
#pragma unroll
        for (int d = 0; d < HD / 16; ++d) orow[d * 16 + fr] = (_Float16)(o[d][e] * inv);
    }
}

template <int EPI, int KVF>
hipError_t gemm(const _Float16* Am, const _Float16* W, void* out, int T, int N, int K, const StepArgs& SA,
                const PfArgs& PA, hipStream_t s) {
    dim3 grid((N + GB - 1) / GB, (T + GB - 1) / GB);
    hipLaunchKernelGGL((k_pf_gemm<EPI, KVF>), grid, dim3(PT), 0, s, Am, W, out, T, N, K, SA, PA);
    return hipGetLastError();
}

template <int KVF>
hipError_t prefill_chunk_t(const StepArgs& A, const PrefillWs& ws, int p0, int T, hipStream_t s) {
    const int D = A.D, H = A.H, Hk = A.Hk, hd = A.hd, F = A.F;
    const int Nqkv = (H + 2 * Hk) * hd;
    hipLaunchKernelGGL(k_pf_embed, dim3(T), dim3(PT), 0, s, ws.tok, T, A.embed, D, ws.x);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    PfArgs PA{T, p0, 0, ws.tc, ws.q, ws.kt};
    const dim3 ngrid((T + 3) / 4);
    const int nqb = (p0 + T - 1) / 64 - p0 / 64 + 1;
    for (int l = 0; l < A.n_layers; ++l) {
        const LayerW& Lw = A.layers[l];
        PA.layer = l;
        hipLaunchKernelGGL(k_pf_norm, ngrid, dim3(PT), 0, s, ws.x, T, D, Lw.g_attn, A.eps, ws.xn);
        if ((e = gemm<PE_QKV, KVF>(ws.xn, Lw.wqkv, nullptr, T, Nqkv, D, A, PA, s)) != hipSuccess) return e;
        const int nsg = (p0 + T - 1) / SEG - p0 / SEG + 1;
        if constexpr (KVF == KV_INT8) {
            if (hd == 128) hipLaunchKernelGGL((k_pf_seal<128, false>), dim3(2 * Hk * nsg), dim3(PT), 0, s, A, PA);
            else hipLaunchKernelGGL((k_pf_seal<64, false>), dim3(2 * Hk * nsg), dim3(PT), 0, s, A, PA);
        }
        if (hd == 128) hipLaunchKernelGGL((k_pf_attn<128, KVF>), dim3(nqb, H), dim3(PT), 0, s, A, PA, ws.a);
        else hipLaunchKernelGGL((k_pf_attn<64, KVF>), dim3(nqb, H), dim3(PT), 0, s, A, PA, ws.a);
        if constexpr (KVF == KV_INT8) {
            if (hd == 128) hipLaunchKernelGGL((k_pf_seal<128, true>), dim3(2 * Hk * nsg), dim3(PT), 0, s, A, PA);
            else hipLaunchKernelGGL((k_pf_seal<64, true>), dim3(2 * Hk * nsg), dim3(PT), 0, s, A, PA);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = gemm<PE_RESID, KVF>(ws.a, Lw.wo, ws.x, T, D, H * hd, A, PA, s)) != hipSuccess) return e;
        hipLaunchKernelGGL(k_pf_norm, ngrid, dim3(PT), 0, s, ws.x, T, D, Lw.g_ffn, A.eps, ws.xn);
        if ((e = gemm<PE_SWIGLU, KVF>(ws.xn, Lw.wgu, ws.m, T, 2 * F, D, A, PA, s)) != hipSuccess) return e;
        if ((e = gemm<PE_RESID, KVF>(ws.m, Lw.wd, ws.x, T, D, F, A, PA, s)) != hipSuccess) return e;
    }
    return hipGetLastError();
}

}  // namespace

bool prefill_supported(int D, int H, int hd, int F, int B) {
    return B == 1 && (hd == 64 || hd == 128) && D % GK == 0 && F % GK == 0 && (H * hd) % GK == 0;
}

hipError_t prefill_chunk(const StepArgs& A, const PrefillWs& ws, int p0, int T, hipStream_t s) {
    if (T < 1 || T > ws.tc) return hipErrorInvalidValue;
    switch (A.kvfmt) {
        case KV_FP16: return prefill_chunk_t<KV_FP16>(A, ws, p0, T, s);
        case KV_E5M2: return prefill_chunk_t<KV_E5M2>(A, ws, p0, T, s);
        case KV_INT8: return prefill_chunk_t<KV_INT8>(A, ws, p0, T, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace rd
