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

constexpr int GW = 256;   // threads per batch-1 workgroup (4 waves)

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// ---- batch 1 ---------------------------------------------------------------------
// Each workgroup owns a contiguous block of rows; its waves take NR rows at
// a time, round robin, and keep NB groups of loads in registers: while one
// group is reduced the next NB - 1 are in flight.  Launched with several
// workgroups per CU so that about 128 KiB per CU are in flight, which the
// HBM needs to stream at full rate.
template <int KCH, int NR, int NB>
__global__ __launch_bounds__(GW) void k_gemv_b1(const _Float16* __restrict__ W, const _Float16* __restrict__ x,
                                                 float* __restrict__ y, int N, int K) {
    const int wid = wave_id(), nw = GW / WAVE, lane = lane_id();
    const int per = (N + gridDim.x - 1) / gridDim.x;
    const int r0 = min(N, (int)blockIdx.x * per), r1 = min(N, r0 + per);
    u4v w[NB][NR][KCH];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int r = r0 + (b * nw + wid) * NR;
        load_rows<NR, KCH>(W, K, r, max(0, min(NR, r1 - r)), w[b]);
    }
    u4v xh[KCH];
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const int col = (c * 64 + lane) * 8;
        xh[c] = col < K ? ld16(x + col) : u4v{0u, 0u, 0u, 0u};
    }
    for (int j = 0;; j += NB) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int r = r0 + ((j + b) * nw + wid) * NR;
            if (r >= r1) return;
            float acc[NR];
            dot_rows<NR, KCH>(w[b], xh, acc);
            if (lane == 0)
#pragma unroll
                for (int i = 0; i < NR; ++i)
                    if (r + i < r1) y[r + i] = acc[i];
            const int rn = r0 + ((j + b + NB) * nw + wid) * NR;
            load_rows<NR, KCH>(W, K, rn, max(0, min(NR, r1 - rn)), w[b]);
        }
    }
}

// ---- batch 8 (MFMA) ------------------------------------------------------------------
// v_mfma_f32_16x16x32_f16 with M = batch (rows 8..15 zero), N = 16 weight
// rows, K = 32: lane l of the weight operand holds 8 k-values of row l % 16,
// lane l of the batch operand 8 k-values of batch row l % 16, and the result
// lane l holds rows m = 4*(l/16) + j of column n = l % 16.  A dot product
// may take its terms in any order if both operands use the same order, so
// which k-values a lane holds is free as long as x and W agree.
//
// HBM streams best when each load instruction reads whole 128-byte lines,
// but the operand layout wants 16 rows per instruction.  So W goes through
// a per-wave LDS ring: LDS-DMA loads (lane l: row l/8, then row 8 + l/8,
// 16-byte chunk l%8 of the row's 128-byte line of the 64-column step) land
// each row line contiguously in LDS, with chunk c stored at position
// c ^ (row % 8) so that the operand reads (row l % 16, chunk 4j + l/16 for
// MFMA j) hit distinct banks.  The batch operand for a wave's K range is
// loaded into registers once (chunk 4j + l/16 of each step).
//
// Work unit = (16-row block, one of KS parts of K).  Workgroups walk groups
// of units, one unit per wave; with KS > 1 the parts of a block are summed
// through LDS in part order, so the result does not depend on timing.
typedef _Float16 hv8 __attribute__((ext_vector_type(8)));
typedef float fv4 __attribute__((ext_vector_type(4)));
constexpr int B8_SMAX = 16;   // 64-column steps per unit (x operand registers)

// x: B rows of K, row stride ldx, fp16 or (XF32) fp32 converted to fp16 as it
// is loaded; y: B rows of N, row stride ldy, written or (ACC) added to.
// Rows B..15 of the MFMA tile are zero.
template <int KS, int T, int U, bool XF32, bool ACC>
__global__ __launch_bounds__(T) void k_gemm_b8(const _Float16* __restrict__ W, const void* __restrict__ xv, int ldx,
                                               float* __restrict__ y, int ldy, int N, int K, int B) {
    extern __shared__ __attribute__((aligned(16))) char s_lds[];   // [T/64][U][2 KiB] ring, [T/64][64] fv4
    constexpr int NWV = T / WAVE, BPG = NWV / KS;
    const int wid = wave_id(), lane = lane_id();
    char* ring = s_lds + wid * U * 2048;
    fv4* s_red = reinterpret_cast<fv4*>(s_lds + NWV * U * 2048);
    const int nblk = (N + 15) / 16, ngrp = (nblk + BPG - 1) / BPG;
    const int n = lane % 16, q = lane / 16;
    const int nsteps = K / 64, part = wid % KS;
    const int s_beg = part * nsteps / KS, ns = (part + 1) * nsteps / KS - s_beg;   // ns <= B8_SMAX
    u4v xa[B8_SMAX][2];
    const int xr = n < B ? n : 0;
#pragma unroll
    for (int t = 0; t < B8_SMAX; ++t) {
        const bool ok = t < ns && n < B;
        const size_t c0 = (size_t)xr * ldx + (s_beg + t) * 64 + 8 * q;
        if constexpr (XF32) {
            const float* xp = reinterpret_cast<const float*>(xv) + c0;
#pragma unroll
            for (int hlf = 0; hlf < 2; ++hlf) {
                h8 v;
                if (ok) {
                    const float4 a = *reinterpret_cast<const float4*>(xp + 32 * hlf);
                    const float4 b = *reinterpret_cast<const float4*>(xp + 32 * hlf + 4);
                    v = h8{(_Float16)a.x, (_Float16)a.y, (_Float16)a.z, (_Float16)a.w,
                           (_Float16)b.x, (_Float16)b.y, (_Float16)b.z, (_Float16)b.w};
                } else {
                    v = h8{0, 0, 0, 0, 0, 0, 0, 0};
                }
                xa[t][hlf] = __builtin_bit_cast(u4v, v);
            }
        } else {
            const _Float16* xp = reinterpret_cast<const _Float16*>(xv) + c0;
            xa[t][0] = ok ? ld16(xp) : u4v{0u, 0u, 0u, 0u};
            xa[t][1] = ok ? ld16(xp + 32) : u4v{0u, 0u, 0u, 0u};
        }
    }
    const int lr = lane / 8, lc = (lane % 8) ^ lr;
    const int rd0 = (n / 8) * 1024 + (n % 8) * 128 + (q ^ (n % 8)) * 16;
    const int rd1 = (n / 8) * 1024 + (n % 8) * 128 + ((4 + q) ^ (n % 8)) * 16;
    for (int g = blockIdx.x; g < ngrp; g += gridDim.x) {
        const int blk = g * BPG + wid / KS;
        fv4 acc = {0.f, 0.f, 0.f, 0.f};
        if (blk < nblk && ns > 0) {
            // rows past N read row N - 1 (never stored)
            const char* g0 = (const char*)(W + (size_t)min(blk * 16 + lr, N - 1) * K + s_beg * 64) + lc * 16;
            const char* g1 = (const char*)(W + (size_t)min(blk * 16 + 8 + lr, N - 1) * K + s_beg * 64) + lc * 16;
            auto issue = [&](int t, int slot) {   // t in [0, ns)
                __builtin_amdgcn_global_load_lds((glb_void*)(g0 + t * 128), (lds_void*)(ring + slot * 2048), 16, 0, 2);
                __builtin_amdgcn_global_load_lds((glb_void*)(g1 + t * 128), (lds_void*)(ring + slot * 2048 + 1024), 16,
                                                 0, 2);
            };
#pragma unroll
            for (int u = 0; u < U; ++u) issue(min(u, ns - 1), u);
#pragma unroll
            for (int t = 0; t < B8_SMAX; ++t) {
                if (t < ns) {
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (U - 1)) : "memory");
                    const int slot = t % U;
                    const u4v w0 = *reinterpret_cast<const u4v*>(ring + slot * 2048 + rd0);
                    const u4v w1 = *reinterpret_cast<const u4v*>(ring + slot * 2048 + rd1);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    issue(min(t + U, ns - 1), slot);   // past the end: a harmless re-read of the last step
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(hv8, xa[t][0]),
                                                                 __builtin_bit_cast(hv8, w0), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(hv8, xa[t][1]),
                                                                 __builtin_bit_cast(hv8, w1), acc, 0, 0, 0);
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
                if (ob < B && on < N) {
                    if constexpr (ACC) y[(size_t)ob * ldy + on] += acc[j];
                    else y[(size_t)ob * ldy + on] = acc[j];
                }
            }
        }
    }
}

template <int KS, int T, int U, bool XF32, bool ACC>
hipError_t launch_b8(const _Float16* W, const void* x, int ldx, float* y, int ldy, int N, int K, int B, int gmul,
                     int ncu, hipStream_t s) {
    const size_t lds = (size_t)(T / WAVE) * U * 2048 + (T / WAVE) * 1024;
    static bool attr_set = false;   // the attribute is per function, the same value every time
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)&k_gemm_b8<KS, T, U, XF32, ACC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int nblk = (N + 15) / 16, ngrp = (nblk * KS + T / WAVE - 1) / (T / WAVE);
    hipLaunchKernelGGL((k_gemm_b8<KS, T, U, XF32, ACC>), dim3(std::min(ngrp, gmul * ncu)), dim3(T), lds, s, W, x,
                       ldx, y, ldy, N, K, B);
    return hipGetLastError();
}
template <bool XF32, bool ACC>
hipError_t launch_b8_k(const _Float16* W, const void* x, int ldx, float* y, int ldy, int N, int K, int B, int ncu,
                       hipStream_t s) {
    // K <= 4096: 4 parts of <= 16 steps, 4-wave workgroups, 4 per CU;
    // K <= 8192: 8 parts, 8-wave workgroups, one per CU.
    if (K <= 4096) return launch_b8<4, 256, 4, XF32, ACC>(W, x, ldx, y, ldy, N, K, B, 4, ncu, s);
    return launch_b8<8, 512, 6, XF32, ACC>(W, x, ldx, y, ldy, N, K, B, 1, ncu, s);
}

}  // namespace

hipError_t launch_gemv_f16(const void* W, const void* x, float* y, int N, int K, int batch, int ncu, hipStream_t s) {
    const auto* Wh = (const _Float16*)W;
    const auto* xh = (const _Float16*)x;
    if (batch == 8) {
        if (K % 64 || K > 8192) return hipErrorInvalidValue;
        return launch_b8_k<false, false>(Wh, x, K, y, N, N, K, 8, ncu, s);
    }
    if (batch != 1) return hipErrorInvalidValue;
    const int kch = kch_for(K);
    // one row per wave; two groups in flight and 4 workgroups per CU up to
    // K = 4096, three groups and 2 per CU above
#define RD_B1(KC, NB, G)                                                                                     \
    case KC:                                                                                                 \
        hipLaunchKernelGGL((k_gemv_b1<KC, 1, NB>), dim3(G * ncu), dim3(GW), 0, s, Wh, xh, y, N, K);          \
        break;
    switch (kch) {
        RD_B1(1, 2, 4) RD_B1(2, 2, 4) RD_B1(4, 2, 4) RD_B1(8, 2, 4) RD_B1(11, 3, 2) RD_B1(16, 3, 2)
        default: return hipErrorInvalidValue;
    }
#undef RD_B1
    return hipGetLastError();
}

hipError_t launch_gemm_b8(const _Float16* W, const void* x, bool x_f32, int ldx, float* y, int ldy, bool acc, int N,
                          int K, int B, int ncu, hipStream_t s) {
    if (K % 64 || K > 8192 || B < 1 || B > 8) return hipErrorInvalidValue;
    if (x_f32) return acc ? launch_b8_k<true, true>(W, x, ldx, y, ldy, N, K, B, ncu, s)
                          : launch_b8_k<true, false>(W, x, ldx, y, ldy, N, K, B, ncu, s);
    return acc ? launch_b8_k<false, true>(W, x, ldx, y, ldy, N, K, B, ncu, s)
               : launch_b8_k<false, false>(W, x, ldx, y, ldy, N, K, B, ncu, s);
}

}  // namespace rd
