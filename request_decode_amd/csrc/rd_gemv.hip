// Weight-streaming GEMV kernels for the standalone GEMV entry point (the
// decode step's matrix shapes, measured alone): y[b][n] = sum_k W[n][k] x[b][k]
// with fp16 W and x, fp32 accumulation.
//
// At batch 1 every weight byte is used for one multiply-add, so the kernel is
// an HBM stream ("Real-time LLM inference on standard GPUs: 3,000 tokens/s
// per request", section "Memory bandwidth is the main bottleneck": about
// 1 FLOP per weight byte at fp16).  At batch 8 a weight byte serves 8
// multiply-adds, still far below the matrix cores' balance point, so the
// batch-8 kernel is the same stream feeding MFMA thin-GEMM tiles.
#include "rd_phases.h"

namespace rd {

namespace {

constexpr int GW = 256;   // threads per workgroup (4 waves)

// ---- batch 1 ---------------------------------------------------------------------
// One workgroup per CU walks a contiguous block of rows; each wave takes NR
// rows at a time (rows r0 + NR*wid + NR*nw*j), and the next group's loads
// (NR * KCH KiB per wave) are in flight while the current group is reduced.
// The x vector is in registers in the chunk layout of dot_rows.
template <int KCH, int NR>
__global__ __launch_bounds__(GW) void k_gemv_b1(const _Float16* __restrict__ W, const _Float16* __restrict__ x,
                                                 float* __restrict__ y, int N, int K) {
    const int wid = wave_id(), nw = GW / WAVE, lane = lane_id();
    const int per = (N + gridDim.x - 1) / gridDim.x;
    const int r0 = min(N, (int)blockIdx.x * per), r1 = min(N, r0 + per);
    int r = r0 + wid * NR;
    u4v wa[NR][KCH], wb[NR][KCH];
    load_rows<NR, KCH>(W, K, r, max(0, min(NR, r1 - r)), wa);
    float xr[KCH][8];
    load_x_f16<KCH>(x, K, xr);
    auto finish = [&](const u4v (&w)[NR][KCH], int row) {
        float acc[NR];
        dot_rows<NR, KCH>(w, xr, acc);
        if (lane == 0)
#pragma unroll
            for (int i = 0; i < NR; ++i)
                if (row + i < r1) y[row + i] = acc[i];
    };
    while (r < r1) {
        const int rn = r + NR * nw;
        load_rows<NR, KCH>(W, K, rn, max(0, min(NR, r1 - rn)), wb);
        finish(wa, r);
        r = rn;
        if (r >= r1) break;
        const int rn2 = r + NR * nw;
        load_rows<NR, KCH>(W, K, rn2, max(0, min(NR, r1 - rn2)), wa);
        finish(wb, r);
        r = rn2;
    }
}

// ---- batch 8 (MFMA) ------------------------------------------------------------------
// v_mfma_f32_16x16x32_f16 with M = batch (rows 8..15 zero), N = 16 weight
// rows, K = 32.  Lane l (n = l % 16, q = l / 16) loads 32 contiguous bytes
// of weight row n at columns k0 + 16q .. +15 (four lanes cover a 128-byte
// line of the row), which feed two MFMAs: its first 8 halves in the first,
// the last 8 in the second.  A dot product may take its terms in any order
// as long as both operands use the same order, so the batch operand is
// loaded with the same permutation of k: lane (m, q) holds x[m][k0 + 16q ..
// +15].  Output layout of the 16x16 accumulator: lane l holds rows
// m = 4*(l/16) + j, column n = l % 16.
//
// Work unit = (block of 16 weight rows, one of KS parts of K).  Each
// workgroup is resident for the whole launch (grid <= CU count), stages x
// ([8][K] fp16) in LDS once, and walks groups of 4 units (4/KS blocks, all
// KS parts of each, one unit per wave); with KS > 1 the parts are summed
// through LDS in part order, so the result does not depend on timing.
typedef _Float16 hv8 __attribute__((ext_vector_type(8)));
typedef float fv4 __attribute__((ext_vector_type(4)));
constexpr int B8_KMAX = 8192;   // x [8][K+8] fp16 in LDS: 128 KiB + 128 B
constexpr int B8_U = 8;         // 64-column steps in flight per wave (16 KiB)

template <int KS>
__global__ __launch_bounds__(GW) void k_gemv_b8(const _Float16* __restrict__ W, const _Float16* __restrict__ x,
                                                float* __restrict__ y, int N, int K) {
    // x rows at a stride of K + 8 halves: the 8 rows a ds_read_b128 touches
    // at one column fall on different banks.  Then [4][64] fv4 partials.
    extern __shared__ __attribute__((aligned(16))) _Float16 s_x[];
    const int xs = K + 8;
    fv4* s_red = reinterpret_cast<fv4*>(s_x + 8 * xs);
    const int wid = wave_id(), lane = lane_id();
    for (int i = threadIdx.x * 8; i < 8 * K; i += GW * 8)
        *reinterpret_cast<u4v*>(s_x + (i / K) * xs + i % K) = ld16(x + i);
    __syncthreads();
    constexpr int BPG = 4 / KS;   // blocks per group of 4 units
    const int nblk = (N + 15) / 16, ngrp = (nblk + BPG - 1) / BPG;
    const int n = lane % 16, q = lane / 16;
    const int nsteps = K / 64, part = wid % KS;
    const int s_beg = part * nsteps / KS, s_end = (part + 1) * nsteps / KS;
    for (int g = blockIdx.x; g < ngrp; g += gridDim.x) {
        const int blk = g * BPG + wid / KS;
        fv4 acc = {0.f, 0.f, 0.f, 0.f};
        if (blk < nblk) {
            const int row = min(blk * 16 + n, N - 1);   // rows past N read row N-1; never stored
            const _Float16* wp = W + (size_t)row * K + 16 * q;
            const _Float16* xp = s_x + (n & 7) * xs + 16 * q;
            u4v wv[B8_U][2];
#pragma unroll
            for (int u = 0; u < B8_U; ++u)
                if (s_beg + u < s_end) {
                    wv[u][0] = ld_w16(wp + (s_beg + u) * 64);
                    wv[u][1] = ld_w16(wp + (s_beg + u) * 64 + 8);
                }
            for (int s0 = s_beg; s0 < s_end; s0 += B8_U) {
#pragma unroll
                for (int u = 0; u < B8_U; ++u) {
                    const int s = s0 + u;
                    if (s >= s_end) break;
                    const u4v w0 = wv[u][0], w1 = wv[u][1];
                    if (s + B8_U < s_end) {
                        wv[u][0] = ld_w16(wp + (s + B8_U) * 64);
                        wv[u][1] = ld_w16(wp + (s + B8_U) * 64 + 8);
                    }
                    u4v a0 = *reinterpret_cast<const u4v*>(xp + s * 64);
                    u4v a1 = *reinterpret_cast<const u4v*>(xp + s * 64 + 8);
                    if (n >= 8) a0 = a1 = u4v{0u, 0u, 0u, 0u};
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(hv8, a0),
                                                                 __builtin_bit_cast(hv8, w0), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(hv8, a1),
                                                                 __builtin_bit_cast(hv8, w1), acc, 0, 0, 0);
                }
            }
        }
        if constexpr (KS > 1) {
            s_red[wid * 64 + lane] = acc;
            __syncthreads();
            if (part == 0) {
#pragma unroll
                for (int p = 1; p < KS; ++p) acc += s_red[(wid + p) * 64 + lane];
            }
            __syncthreads();
        }
        if (part == 0 && blk < nblk) {
            const int on = blk * 16 + n;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ob = 4 * q + j;
                if (ob < 8 && on < N) y[(size_t)ob * N + on] = acc[j];
            }
        }
    }
}

}  // namespace

hipError_t launch_gemv_f16(const void* W, const void* x, float* y, int N, int K, int batch, int ncu, hipStream_t s) {
    if (batch == 8) {
        if (K % 64 || K > B8_KMAX) return hipErrorInvalidValue;
        const int nblk = (N + 15) / 16;
        const int ks = nblk >= 4 * ncu ? 1 : nblk >= 2 * ncu ? 2 : 4;
        const int ngrp = (nblk * ks + 3) / 4;
        const int grid = std::min(ngrp, ncu);
        const size_t lds = (size_t)8 * (K + 8) * 2 + 4 * 64 * 16;
        const void* fn = ks == 1 ? (const void*)&k_gemv_b8<1> : ks == 2 ? (const void*)&k_gemv_b8<2>
                                                                        : (const void*)&k_gemv_b8<4>;
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        const auto* Wh = (const _Float16*)W;
        const auto* xh = (const _Float16*)x;
        if (ks == 1) hipLaunchKernelGGL(k_gemv_b8<1>, dim3(grid), dim3(GW), lds, s, Wh, xh, y, N, K);
        else if (ks == 2) hipLaunchKernelGGL(k_gemv_b8<2>, dim3(grid), dim3(GW), lds, s, Wh, xh, y, N, K);
        else hipLaunchKernelGGL(k_gemv_b8<4>, dim3(grid), dim3(GW), lds, s, Wh, xh, y, N, K);
        return hipGetLastError();
    }
    if (batch != 1) return hipErrorInvalidValue;
    const int kch = kch_for(K);
    const int grid = std::min(ncu, (N + 7) / 8);
#define RD_B1(KC)                                                                                    \
    case KC:                                                                                         \
        hipLaunchKernelGGL((k_gemv_b1<KC, (KC >= 11 ? 1 : 2)>), dim3(grid), dim3(GW), 0, s, (const _Float16*)W, \
                           (const _Float16*)x, y, N, K);                                             \
        break;
    switch (kch) {
        RD_B1(1) RD_B1(2) RD_B1(4) RD_B1(8) RD_B1(11) RD_B1(16)
        default: return hipErrorInvalidValue;
    }
#undef RD_B1
    return hipGetLastError();
}

}  // namespace rd
