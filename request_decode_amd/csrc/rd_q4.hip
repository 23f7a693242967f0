// Weight-only INT4 GEMV for gfx950: y = W^ x at batch 1, W^ stored as 4-bit
// codes in groups of 128 columns with one fp32 scale per (row, group).
//
// The pages give the bound this attacks and the dequantization it must use:
// at batch 1 each weight byte carries one multiply-add, so a 4-bit weight
// moves four times the work per byte of an fp16 one ("Real-time LLM
// inference on standard GPUs: 3,000 tokens/s per request", section on
// memory bandwidth: FP8 about 2 FLOP/B, FP4 about 4); an INT4 weight is used
// as fp16(int4_value * scale) with the scale in fp32 and round-to-nearest
// ("LLM inference architecture rebuild", section 5.2, where an fp16 scale
// had lost precision).  The quantizer (symmetric, scale = amax / 7 per
// group) is this library's reading; both are bit-exact against the oracle.
#include "rd_phases.h"

namespace rd {

namespace {

constexpr int QG = 128;   // columns per scale group
constexpr int QT = 256;   // threads per workgroup

// One thread per (row, group): scale = amax / 7 in fp32 (1 for an all-zero
// group), code = clamp(rint(w / scale), -8, 7), column 2j in the low nibble
// of byte j.
__global__ __launch_bounds__(QT) void k_q4_quant(const _Float16* __restrict__ W, int N, int K,
                                                 uint8_t* __restrict__ codes, float* __restrict__ scales) {
    const int ng = K / QG;
    const long long id = (long long)blockIdx.x * QT + threadIdx.x;
    if (id >= (long long)N * ng) return;
    const int r = (int)(id / ng), g = (int)(id % ng);
    const _Float16* w = W + (size_t)r * K + (size_t)g * QG;
    float amax = 0.f;
    for (int i = 0; i < QG; i += 8) {
        const h8 v = as_h8(ld16(w + i));
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf((float)v[k]));
    }
    float scale = amax / 7.0f;
    if (!(scale > 0.0f)) scale = 1.0f;
    scales[(size_t)r * ng + g] = scale;
    uint8_t* dst = codes + ((size_t)r * K + (size_t)g * QG) / 2;
    for (int i = 0; i < QG; i += 8) {
        const h8 v = as_h8(ld16(w + i));
        unsigned word = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float q = fminf(fmaxf(rintf((float)v[k] / scale), -8.0f), 7.0f);
            word |= ((unsigned)(int)q & 15u) << (4 * k);
        }
        *reinterpret_cast<unsigned*>(dst + i / 2) = word;
    }
}

// fp16(code * scale) for the two codes of byte p of a word: the binary32
// product rounded to nearest, packed as an fp16 pair.
__device__ __forceinline__ h2 dq_pair(unsigned word, int p, float s) {
    const int q0 = __builtin_amdgcn_sbfe((int)word, 8 * p, 4);
    const int q1 = __builtin_amdgcn_sbfe((int)word, 8 * p + 4, 4);
    return h2{(_Float16)((float)q0 * s), (_Float16)((float)q1 * s)};
}

// One row per wave; NB rows' loads in flight per wave; lane l covers
// columns (c*64 + l)*32 .. +31 of chunk c (16 bytes of codes, one scale),
// the fp16 x of those columns in registers.  Per lane, two fp32 chains of
// v_dot2_f32_f16 steps over the chunks in order, then the wave sum.
template <int KC, int NB>
__global__ __launch_bounds__(QT) void k_gemv_q4(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                                                const _Float16* __restrict__ x, float* __restrict__ y, int N, int K) {
    const int wid = wave_id(), nw = QT / WAVE, lane = lane_id();
    const int ng = K / QG;
    const int per = (N + gridDim.x - 1) / gridDim.x;
    const int r0 = min(N, (int)blockIdx.x * per), r1 = min(N, r0 + per);
    u4v xh[KC][4];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        const int col = (c * 64 + lane) * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) xh[c][i] = col < K ? ld16(x + col + 8 * i) : u4v{0u, 0u, 0u, 0u};
    }
    u4v wq[NB][KC];
    float sc[NB][KC];
    auto load = [&](int b, int r) {
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const int col = (c * 64 + lane) * 32;
            const bool ok = r < r1 && col < K;
            wq[b][c] = ok ? ld_w16(codes + ((size_t)r * K + col) / 2) : u4v{0u, 0u, 0u, 0u};
            sc[b][c] = ok ? scales[(size_t)r * ng + col / QG] : 0.f;
        }
    };
#pragma unroll
    for (int b = 0; b < NB; ++b) load(b, r0 + b * nw + wid);
    for (int j = 0;; j += NB) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int r = r0 + (j + b) * nw + wid;
            if (r >= r1) return;
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int c = 0; c < KC; ++c) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const unsigned word = wq[b][c][i];
                    const u4v xv = xh[c][i];
                    s0 = __builtin_amdgcn_fdot2(dq_pair(word, 0, sc[b][c]), __builtin_bit_cast(h2, (unsigned)xv.x), s0, false);
                    s1 = __builtin_amdgcn_fdot2(dq_pair(word, 1, sc[b][c]), __builtin_bit_cast(h2, (unsigned)xv.y), s1, false);
                    s0 = __builtin_amdgcn_fdot2(dq_pair(word, 2, sc[b][c]), __builtin_bit_cast(h2, (unsigned)xv.z), s0, false);
                    s1 = __builtin_amdgcn_fdot2(dq_pair(word, 3, sc[b][c]), __builtin_bit_cast(h2, (unsigned)xv.w), s1, false);
                }
            }
            load(b, r0 + (j + b + NB) * nw + wid);
            const float v = wave_sum(s0 + s1);
            if (lane == 0) y[r] = v;
        }
    }
}

}  // namespace

hipError_t launch_q4_quant(const void* W, int N, int K, uint8_t* codes, float* scales, hipStream_t s) {
    const long long n = (long long)N * (K / QG);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_q4_quant, dim3((unsigned)((n + QT - 1) / QT)), dim3(QT), 0, s, (const _Float16*)W, N, K,
                       codes, scales);
    return hipGetLastError();
}

hipError_t launch_gemv_q4(const uint8_t* codes, const float* scales, const void* x, float* y, int N, int K, int ncu,
                          hipStream_t s) {
    const int kc = (K + 2047) / 2048;
    const _Float16* xh = (const _Float16*)x;
#define RD_Q4(KCv)                                                                                          \
    case KCv:                                                                                               \
        hipLaunchKernelGGL((k_gemv_q4<KCv, 2>), dim3(4 * ncu), dim3(QT), 0, s, codes, scales, xh, y, N, K); \
        break;
    switch (kc) {
        RD_Q4(1) RD_Q4(2) RD_Q4(3) RD_Q4(4)
        default: return hipErrorInvalidValue;
    }
#undef RD_Q4
    return hipGetLastError();
}

}  // namespace rd
