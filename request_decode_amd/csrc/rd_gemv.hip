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

// Wait until at most n (0..31, wave-uniform) vector-memory operations of
// this wave are outstanding: s_waitcnt takes only an immediate.
__device__ __forceinline__ void wait_vm_upto(int n) {
#define RD_VMW(k) \
    case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
    switch (n) {
        RD_VMW(1) RD_VMW(2) RD_VMW(3) RD_VMW(4) RD_VMW(5) RD_VMW(6) RD_VMW(7) RD_VMW(8) RD_VMW(9) RD_VMW(10)
        RD_VMW(11) RD_VMW(12) RD_VMW(13) RD_VMW(14) RD_VMW(15) RD_VMW(16) RD_VMW(17) RD_VMW(18) RD_VMW(19)
        RD_VMW(20) RD_VMW(21) RD_VMW(22) RD_VMW(23) RD_VMW(24) RD_VMW(25) RD_VMW(26) RD_VMW(27) RD_VMW(28)
        RD_VMW(29) RD_VMW(30) RD_VMW(31)
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
#undef RD_VMW
}

// ---- batch 8 (MFMA) ------------------------------------------------------------------
// v_mfma_f32_16x16x32_f16 with M = batch (rows past B not stored), N = 16 weight
// rows, K = 32: lane l of the weight operand holds 8 k-values of row l % 16,
// lane l of the batch operand 8 k-values of batch row l % 16, and the result
// lane l holds rows m = 4*(l/16) + j of column n = l % 16.  A dot product
// may take its terms in any order if both operands use the same order, so
// which k-values a lane holds is free as long as x and W agree.
//
// HBM streams best when each load instruction reads whole 128-byte lines,
// but the operand layout wants 16 rows per instruction.  So W goes through
// a per-wave LDS ring: LDS-DMA loads (lane l: row l/8, 16-byte chunk l%8 of
// the row's 128-byte line of the 64-column step) land each row line
// contiguously in LDS, with chunk c stored at position c ^ (row % 8) so
// that the operand reads (row n, chunk 4j + l/16 for MFMA j) hit distinct
// banks.  The batch operand for a wave's K range is loaded into registers
// once (chunk 4j + l/16 of each step).
//
// A block is R weight rows: 16, one tile column per row, or 8 when the
// matrix has too few rows to give every CU a block of 16 (the tile's
// columns 8..15 repeat rows 0..7 and are not stored: the matrix cores have
// time to spare, the HBM stream is what counts).  Work unit = (block, one
// of KS parts of K).  Workgroups walk groups of units, one unit per wave;
// with KS > 1 the parts of a block are summed through LDS in part order, so
// the result does not depend on timing.
typedef _Float16 hv8 __attribute__((ext_vector_type(8)));
typedef float fv4 __attribute__((ext_vector_type(4)));
constexpr int B8_SMAX = 16;   // 64-column steps per unit (x operand registers)


// x: B rows of K, row stride ldx, fp16 or (XF32) fp32 converted to fp16 as it
// is loaded.  Output (row stride ldy): EPI_STORE: y[b][n] (fp32) written or
// (ACC) added to; EPI_SWIGLU: W holds gate and up rows interleaved (row 2i
// gate i, row 2i + 1 up i) and the output is fp16 silu(gate) * up at
// column i (SwiGLU, "Real-time LLM inference on standard GPUs: 3,000
// tokens/s per request", fused FFN); EPI_QKV + KV format: W is the fused
// QKV weight with RoPE pairs in adjacent rows, and the epilogue rotates each
// pair and writes q, or appends the K/V elements to sequence b's cache at
// the step's position (EA, layer; qkv_pair and kv_put, the per-pair
// arithmetic of the batch-1 QKV kernel).  Tile rows B..15 repeat batch row
// 0 and are not stored (a tile row of the result depends only on the same
// row of the batch operand).
// U ring slots of R * 128 bytes per wave; a wave requests each step of its
// unit once (U - 1 steps ahead of the one it reduces).
constexpr int EPI_STORE = 0, EPI_SWIGLU = 1, EPI_QKV = 2;   // EPI_QKV + KvFmt
template <int R, int KS, int T, int U, bool XF32, bool ACC, int EPI>
__global__ __launch_bounds__(T) void k_gemm_b8(const _Float16* __restrict__ W, const void* __restrict__ xv, int ldx,
                                               void* __restrict__ yv, int ldy, int N, int K, int B, StepArgs EA,
                                               int layer) {
    static_assert(R == 8 || R == 16, "row block");
    constexpr int NWV = T / WAVE, BPG = NWV / KS, SB = R * 128, LPS = R / 8;   // LPS: loads per step
    static_assert(LPS * (U - 1) <= 31, "wait count");
    extern __shared__ __attribute__((aligned(16))) char s_lds[];   // [T/64][U][SB] ring, [T/64][64] fv4
    const int wid = wave_id(), lane = lane_id();
    char* ring = s_lds + wid * U * SB;
    fv4* s_red = reinterpret_cast<fv4*>(s_lds + NWV * U * SB);
    const int nblk = (N + R - 1) / R, ngrp = (nblk + BPG - 1) / BPG;
    const int n = lane % 16, q = lane / 16, nr = n % R;
    const int nsteps = K / 64, part = wid % KS;
    const int s_beg = part * nsteps / KS, ns = (part + 1) * nsteps / KS - s_beg;   // ns <= B8_SMAX
    const int lr = lane / 8, lc = (lane % 8) ^ lr;
    const int rd0 = (nr / 8) * 1024 + (nr % 8) * 128 + (q ^ (nr % 8)) * 16;
    const int rd1 = (nr / 8) * 1024 + (nr % 8) * 128 + ((4 + q) ^ (nr % 8)) * 16;
    // rows past N read row N - 1 (never stored)
    const char* g0 = nullptr;
    const char* g1 = nullptr;
    auto unit = [&](int g) {   // point g0/g1 at group g's unit; false: no unit for this wave
        const int blk = g * BPG + wid / KS;
        if (blk >= nblk || ns <= 0) return false;
        g0 = (const char*)(W + (size_t)min(blk * R + lr, N - 1) * K + s_beg * 64) + lc * 16;
        g1 = (const char*)(W + (size_t)min(blk * R + 8 + lr, N - 1) * K + s_beg * 64) + lc * 16;
        return true;
    };
    auto issue = [&](int t, int slot) {   // t in [0, ns)
        __builtin_amdgcn_global_load_lds((glb_void*)(g0 + t * 128), (lds_void*)(ring + slot * SB), 16, 0, 2);
        if constexpr (R == 16)
            __builtin_amdgcn_global_load_lds((glb_void*)(g1 + t * 128), (lds_void*)(ring + slot * SB + 1024), 16, 0,
                                             2);
    };
    auto prime = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < ns) issue(u, u);
    };
    // Batch operand, in chunks of 4 steps (only whole chunks past ns are
    // skipped: steps past ns re-read step ns - 1, never used; rows past B read
    // row 0 and only reach tile rows that are not stored).  The loads of the
    // first 8 steps go out before the first group's weight requests and the
    // rest after them, so a wait for the operand never waits for the
    // weights: fp16 operands are used as loaded, fp32 ones are converted
    // once the weight requests are out.
    u4v xa[B8_SMAX][2];
    const int xr = n < B ? n : 0;
    const size_t cb = (size_t)xr * ldx + s_beg * 64 + 8 * q;
    typedef fv4 xf32_chunk[4][4];
    auto load_f32 = [&](int t0, xf32_chunk& f) {
        const float* xb = reinterpret_cast<const float*>(xv) + cb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float* xp = xb + min(t0 + i, ns - 1) * 64;
            f[i][0] = *reinterpret_cast<const fv4*>(xp);
            f[i][1] = *reinterpret_cast<const fv4*>(xp + 4);
            f[i][2] = *reinterpret_cast<const fv4*>(xp + 32);
            f[i][3] = *reinterpret_cast<const fv4*>(xp + 36);
        }
    };
    auto cvt_f32 = [&](int t0, xf32_chunk& f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int hlf = 0; hlf < 2; ++hlf) {
                // the values are taken here, not earlier (the compiler would
                // otherwise convert them, and wait for them, before the
                // weight requests)
                fv4 a = f[i][2 * hlf], b = f[i][2 * hlf + 1];
                asm volatile("" : "+v"(a), "+v"(b));
                const h8 v = h8{(_Float16)a.x, (_Float16)a.y, (_Float16)a.z, (_Float16)a.w,
                                (_Float16)b.x, (_Float16)b.y, (_Float16)b.z, (_Float16)b.w};
                xa[t0 + i][hlf] = __builtin_bit_cast(u4v, v);
            }
        }
    };
    auto load_f16 = [&](int t0) {
        const _Float16* xb = reinterpret_cast<const _Float16*>(xv) + cb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const _Float16* xp = xb + min(t0 + i, ns - 1) * 64;
            xa[t0 + i][0] = ld16(xp);
            xa[t0 + i][1] = ld16(xp + 32);
        }
    };
    xf32_chunk f0, f1;
    if constexpr (XF32) {
        if (ns > 0) load_f32(0, f0);
        if (ns > 4) load_f32(4, f1);
    } else {
#pragma unroll
        for (int t0 = 0; t0 < B8_SMAX; t0 += 4)
            if (t0 < ns) load_f16(t0);
    }
    bool live = unit(blockIdx.x);
    if (live) prime();
    if constexpr (XF32) {
        if (ns > 0) cvt_f32(0, f0);
        if (ns > 4) cvt_f32(4, f1);
#pragma unroll
        for (int t0 = 8; t0 < B8_SMAX; t0 += 4) {
            if (t0 < ns) {
                xf32_chunk f;
                load_f32(t0, f);
                cvt_f32(t0, f);
            }
        }
    }
    for (int g = blockIdx.x; g < ngrp; g += gridDim.x) {
        const int blk = g * BPG + wid / KS;
        if (g != (int)blockIdx.x) {
            live = unit(g);
            if (live) prime();
        }
        fv4 acc = {0.f, 0.f, 0.f, 0.f};
        if (live) {
#pragma unroll
            for (int t = 0; t < B8_SMAX; ++t) {
                if (t < ns) {
                    // steps t+1 .. min(t + U - 1, ns - 1) may still be in flight
                    // (and, in the first group, the operand loads issued after them)
                    wait_vm_upto(LPS * min(U - 1, ns - 1 - t));
                    const int slot = t % U;
                    const u4v w0 = *reinterpret_cast<const u4v*>(ring + slot * SB + rd0);
                    const u4v w1 = *reinterpret_cast<const u4v*>(ring + slot * SB + rd1);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    if (t + U < ns) issue(t + U, slot);
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
        if constexpr (EPI == EPI_SWIGLU) {
            if (part == 0 && blk < nblk) {   // the partner row's sums: lane n ^ 1, same batch rows
                float up[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) up[j] = __shfl_xor(acc[j], 1);
                const int on = blk * R + n;
                if (n < R && (n & 1) == 0 && on < N) {
                    _Float16* m = reinterpret_cast<_Float16*>(yv);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int ob = 4 * q + j;
                        if (ob < B) m[(size_t)ob * ldy + on / 2] = (_Float16)silu_mul(acc[j], up[j]);
                    }
                }
            }
        } else if constexpr (EPI >= EPI_QKV) {
            if (part == 0 && blk < nblk) {   // the pair's second row: lane n ^ 1, same batch rows
                float a1[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) a1[j] = __shfl_xor(acc[j], 1);
                const int on = blk * R + n;
                if (n < R && (n & 1) == 0 && on < N) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int ob = 4 * q + j;
                        if (ob >= B) continue;
                        // paged cache: each sequence at its own position, and
                        // one that sits the step out stores nothing
                        if (EA.ptab && !EA.st->act[ob]) continue;
                        const int pos = EA.ptab ? EA.st->bpos[ob] : EA.st->pos;
                        const float2* rope = EA.rope + (size_t)pos * (EA.hd / 2);
                        const QkvPair o = qkv_pair(EA.hd, EA.H, EA.Hk, on, acc[j], a1[j], rope);
                        if (o.kind == 0) {
                            float* qv = EA.q + (size_t)ob * EA.H * EA.hd + o.head * EA.hd;
                            qv[o.d0] = o.y0;
                            qv[o.d1] = o.y1;
                        } else if (EA.ptab) {
                            if constexpr (EPI - EPI_QKV != KV_INT8) {
                                const int which = o.kind == 2;
                                kv_put_paged<EPI - EPI_QKV>(EA, ob, layer, which, o.head, pos, o.d0, o.y0);
                                kv_put_paged<EPI - EPI_QKV>(EA, ob, layer, which, o.head, pos, o.d1, o.y1);
                            }
                        } else {
                            StepArgs Ab = EA;   // sequence ob's cache
                            Ab.kc = reinterpret_cast<uint8_t*>(EA.kc) + (size_t)ob * EA.kv_bstride;
                            Ab.vc = reinterpret_cast<uint8_t*>(EA.vc) + (size_t)ob * EA.kv_bstride;
                            if (EA.stage) {
                                Ab.stage = EA.stage + (size_t)ob * EA.st_bstride;
                                Ab.meta = EA.meta + (size_t)ob * EA.meta_bstride;
                            }
                            const int which = o.kind == 2;
                            kv_put<EPI - EPI_QKV, false>(Ab, layer, which, o.head, pos, o.d0, o.y0);
                            kv_put<EPI - EPI_QKV, false>(Ab, layer, which, o.head, pos, o.d1, o.y1);
                        }
                    }
                }
            }
        } else if (part == 0 && blk < nblk && n < R) {
            float* y = reinterpret_cast<float*>(yv);
            const int on = blk * R + n;
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

template <int R, int KS, int T, int U, bool XF32, bool ACC, int EPI>
hipError_t launch_b8(const _Float16* W, const void* x, int ldx, void* y, int ldy, int N, int K, int B, int gmul,
                     int ncu, hipStream_t s, const StepArgs& EA, int layer) {
    const size_t lds = (size_t)(T / WAVE) * U * R * 128 + (T / WAVE) * 1024;
    static bool attr_set = false;   // the attribute is per function, the same value every time
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)&k_gemm_b8<R, KS, T, U, XF32, ACC, EPI>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int nblk = (N + R - 1) / R, ngrp = (nblk * KS + T / WAVE - 1) / (T / WAVE);
    hipLaunchKernelGGL((k_gemm_b8<R, KS, T, U, XF32, ACC, EPI>), dim3(std::min(ngrp, gmul * ncu)), dim3(T), lds, s, W,
                       x, ldx, y, ldy, N, K, B, EA, layer);
    return hipGetLastError();
}
template <bool XF32, bool ACC, int EPI>
hipError_t launch_b8_k(const _Float16* W, const void* x, int ldx, void* y, int ldy, int N, int K, int B, int ncu,
                       hipStream_t s, const StepArgs& EA = StepArgs{}, int layer = 0) {
    // K <= 4096: 4 parts of <= 16 steps, 4-wave workgroups, up to 4 per CU;
    // K <= 8192: 8 parts, 8-wave workgroups, one per CU.  Blocks of 8 rows
    // when blocks of 16 would leave CUs without a workgroup.
    const bool r8 = (N + 15) / 16 < ncu;
    if (K <= 4096) {
        if (r8) return launch_b8<8, 4, 256, 8, XF32, ACC, EPI>(W, x, ldx, y, ldy, N, K, B, 4, ncu, s, EA, layer);
        return launch_b8<16, 4, 256, 4, XF32, ACC, EPI>(W, x, ldx, y, ldy, N, K, B, 4, ncu, s, EA, layer);
    }
    if (r8) return launch_b8<8, 8, 512, 12, XF32, ACC, EPI>(W, x, ldx, y, ldy, N, K, B, 1, ncu, s, EA, layer);
    return launch_b8<16, 8, 512, 6, XF32, ACC, EPI>(W, x, ldx, y, ldy, N, K, B, 1, ncu, s, EA, layer);
}

}  // namespace

hipError_t launch_gemv_f16(const void* W, const void* x, float* y, int N, int K, int batch, int ncu, hipStream_t s) {
    const auto* Wh = (const _Float16*)W;
    const auto* xh = (const _Float16*)x;
    if (batch == 8) {
        if (K % 64 || K > 8192) return hipErrorInvalidValue;
        return launch_b8_k<false, false, EPI_STORE>(Wh, x, K, y, N, N, K, 8, ncu, s);
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
    if (x_f32) return acc ? launch_b8_k<true, true, EPI_STORE>(W, x, ldx, y, ldy, N, K, B, ncu, s)
                          : launch_b8_k<true, false, EPI_STORE>(W, x, ldx, y, ldy, N, K, B, ncu, s);
    return acc ? launch_b8_k<false, true, EPI_STORE>(W, x, ldx, y, ldy, N, K, B, ncu, s)
               : launch_b8_k<false, false, EPI_STORE>(W, x, ldx, y, ldy, N, K, B, ncu, s);
}

hipError_t launch_gemm_b8_swiglu(const _Float16* Wgu, const _Float16* x, int ldx, _Float16* m, int ldm, int F, int K,
                                 int B, int ncu, hipStream_t s) {
    if (K % 64 || K > 8192 || B < 1 || B > 8) return hipErrorInvalidValue;
    return launch_b8_k<false, false, EPI_SWIGLU>(Wgu, x, ldx, m, ldm, 2 * F, K, B, ncu, s);
}

hipError_t launch_gemm_b8_qkv(const StepArgs& A, int layer, const _Float16* Wqkv, hipStream_t s) {
    const int N = (A.H + 2 * A.Hk) * A.hd, K = A.D;
    if (K % 64 || K > 8192 || A.B < 1 || A.B > 8) return hipErrorInvalidValue;
    switch (A.kvfmt) {
        case KV_FP16:
            return launch_b8_k<false, false, EPI_QKV + KV_FP16>(Wqkv, A.xh, K, nullptr, 0, N, K, A.B, A.ncu, s, A, layer);
        case KV_E5M2:
            return launch_b8_k<false, false, EPI_QKV + KV_E5M2>(Wqkv, A.xh, K, nullptr, 0, N, K, A.B, A.ncu, s, A, layer);
        default:
            return launch_b8_k<false, false, EPI_QKV + KV_INT8>(Wqkv, A.xh, K, nullptr, 0, N, K, A.B, A.ncu, s, A, layer);
    }
}

}  // namespace rd
