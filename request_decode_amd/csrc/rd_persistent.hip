// Persistent decode-step executor for gfx950: one cooperative launch runs
// whole decode steps, one workgroup per CU, with device-side grid barriers
// between the phases instead of kernel boundaries.
//
// Why: at batch 1 a phase streams only 8-46 MB, so a kernel per phase pays
// its launch, ramp-up, first-byte latency and drain every time, and the
// memory stream stops at each boundary ("Real-time LLM inference on
// standard GPUs: 3,000 tokens/s per request", table of microsecond losses:
// kernel boundaries and grid synchronisation; the fix it names is a single
// resident program with the next phase's loads issued across the sync).
//
// Memory-level parallelism: with one 4-wave workgroup per CU, HBM stays busy
// only if every wave keeps tens of KiB of loads outstanding.  Each GEMV
// phase is therefore a RowStream: a ring of DEPTH register buffers, each a
// task of R rows; reducing task t is followed at once by issuing task
// t + 4*DEPTH into the freed buffer.  The weights never depend on
// activations, so each barrier is split into arrive and wait and the next
// phase's whole ring is issued in between; the gate/up ring is issued even
// earlier, before the attention -> output-projection barrier, so that its
// 32 MB stream runs under the latency-bound attention and projection.
//
// Data produced and consumed inside the launch (residual stream, q, the
// attention output, SwiGLU output, partials, the new K/V row) is written
// with agent-coherent stores and read with agent-coherent loads, staged once
// per workgroup in LDS; see rd_device.h.
#include "rd_phases.h"

namespace rd {

namespace {

// ---- grid barrier -------------------------------------------------------------
// Arrival: every workgroup's stores are drained, then thread 0 counts on
// sub-counter blockIdx % BAR_SUB; the last of a sub-group counts on the top
// counter; the last overall resets the counters and publishes the next
// generation.  Waiting: thread 0 polls the generation word.  A spin limit
// turns a barrier that never completes into an error flag and an abort that
// lets every wave run to the end of the kernel.
__device__ __forceinline__ void grid_arrive(const PersistArgs& P, unsigned gen) {
    drain_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
        int* bar = P.bar;
        const int nwg = gridDim.x, id = blockIdx.x;
        const int sub = id % BAR_SUB;
        const int members = (nwg - 1 - sub) / BAR_SUB + 1, groups = min(nwg, BAR_SUB);
        if (__hip_atomic_fetch_add(&bar[sub * BAR_STRIDE], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            members - 1) {
            st_agent(&bar[sub * BAR_STRIDE], 0);
            drain_vmem();
            if (__hip_atomic_fetch_add(&bar[BAR_SUB * BAR_STRIDE], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                groups - 1) {
                st_agent(&bar[BAR_SUB * BAR_STRIDE], 0);
                drain_vmem();
                st_agent(&bar[(BAR_SUB + 1) * BAR_STRIDE], (int)(gen + 1));
            }
        }
    }
}

__device__ __forceinline__ void grid_wait(const PersistArgs& P, unsigned& gen, int* err) {
    if (threadIdx.x == 0) {
        const int* genw = &P.bar[(BAR_SUB + 1) * BAR_STRIDE];
        int* abort = &P.bar[(BAR_SUB + 2) * BAR_STRIDE];
        const unsigned target = gen + 1;
        int n = 0;
        while ((int)((unsigned)ld_agent(genw) - target) < 0) {
            __builtin_amdgcn_s_sleep(1);
            if ((++n & 255) == 0) {
                if (ld_agent(abort)) break;
                if (n > P.spin_limit) {
                    st_agent(abort, 1);
                    atomicOr(err, ERR_BARRIER);
                    break;
                }
            }
        }
    }
    __syncthreads();
    gen += 1;
}

// ---- alternative barrier schemes (measured by the barrier probe) ------------------
// Epoch e = the barrier's 1-based index since the words were zeroed; all
// counters and flags only grow, so nothing is reset on the critical path.
//   1: one counter, every workgroup adds 1 and polls it until e * nwg;
//   2: BAR_SUB sub-counters (id % BAR_SUB); a sub-group's last arrival adds 1
//      to the top counter; every workgroup polls the top until e * groups;
//   3: flags: workgroup b stores e into word b of a packed array; every
//      workgroup's threads poll all flags (one each) until all reach e;
//   4: as 3 with each flag on its own 128-byte line.
template <int MODE>
__device__ __forceinline__ void bar_arrive(const PersistArgs& P, unsigned gen) {
    if constexpr (MODE == 0) {
        grid_arrive(P, gen);
        return;
    }
    drain_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
        int* bar = P.bar;
        const unsigned e = gen + 1;
        const int nwg = gridDim.x, id = blockIdx.x;
        if constexpr (MODE == 1) {
            __hip_atomic_fetch_add(&bar[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if constexpr (MODE == 2) {
            const int sub = id % BAR_SUB;
            const unsigned members = (unsigned)((nwg - 1 - sub) / BAR_SUB + 1);
            const unsigned old =
                (unsigned)__hip_atomic_fetch_add(&bar[sub * BAR_STRIDE], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1u == e * members)
                __hip_atomic_fetch_add(&bar[BAR_SUB * BAR_STRIDE], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if constexpr (MODE == 3 || MODE == 5 || MODE == 6) {
            st_agent(&bar[BAR_FLAGS + id], (int)e);
        } else {
            st_agent(&bar[BAR_FLAGS + id * BAR_STRIDE], (int)e);
        }
    }
}

template <int MODE>
__device__ __forceinline__ void bar_wait(const PersistArgs& P, unsigned& gen, int* err) {
    if constexpr (MODE == 0) {
        grid_wait(P, gen, err);
        return;
    }
    const unsigned e = gen + 1;
    const int nwg = gridDim.x;
    int* abort = &P.bar[(BAR_SUB + 2) * BAR_STRIDE];
    if constexpr (MODE == 1 || MODE == 2) {
        if (threadIdx.x == 0) {
            const int* w = MODE == 1 ? &P.bar[0] : &P.bar[BAR_SUB * BAR_STRIDE];
            const unsigned target = MODE == 1 ? e * (unsigned)nwg : e * (unsigned)min(nwg, BAR_SUB);
            int n = 0;
            while ((int)((unsigned)ld_agent(w) - target) < 0) {
                __builtin_amdgcn_s_sleep(1);
                if ((++n & 255) == 0) {
                    if (ld_agent(abort)) break;
                    if (n > P.spin_limit) {
                        st_agent(abort, 1);
                        atomicOr(err, ERR_BARRIER);
                        break;
                    }
                }
            }
        }
        __syncthreads();
    } else if constexpr (MODE == 5 || MODE == 6) {
        // wave 0 alone polls the packed flags, two per 8-byte load, and votes
        if (threadIdx.x < WAVE) {
            int n = 0;
            while (true) {
                int ok = 1;
                for (int i = threadIdx.x * 2; i < nwg; i += 2 * WAVE) {
                    const uint64_t v = xld64<true>(reinterpret_cast<const uint64_t*>(&P.bar[BAR_FLAGS + i]));
                    ok &= (int)((unsigned)v - e) >= 0;
                    if (i + 1 < nwg) ok &= (int)((unsigned)(v >> 32) - e) >= 0;
                }
                if (__ballot(ok) == ~0ull) break;
                if constexpr (MODE == 5) __builtin_amdgcn_s_sleep(1);
                if ((++n & 255) == 0) {
                    if (ld_agent(abort)) break;
                    if (n > P.spin_limit) {
                        if (threadIdx.x == 0) {
                            st_agent(abort, 1);
                            atomicOr(err, ERR_BARRIER);
                        }
                        break;
                    }
                }
            }
        }
        __syncthreads();
    } else {
        const int stride = MODE == 3 ? 1 : BAR_STRIDE;
        int n = 0;
        while (true) {
            int ok = 1;
            for (int i = threadIdx.x; i < nwg; i += WG)
                ok &= (int)((unsigned)ld_agent(&P.bar[BAR_FLAGS + i * stride]) - e) >= 0;
            if (__syncthreads_and(ok)) break;
            __builtin_amdgcn_s_sleep(1);
            if ((++n & 255) == 0) {
                if (__syncthreads_or(threadIdx.x == 0 ? ld_agent(abort) : 0)) break;
                if (n > P.spin_limit) {
                    if (threadIdx.x == 0) {
                        st_agent(abort, 1);
                        atomicOr(err, ERR_BARRIER);
                    }
                    break;
                }
            }
        }
    }
    gen += 1;
}

// The scheme the decode kernel uses: measured on MI355X with one workgroup
// per CU, packed epoch flags polled by every thread took 1.4 us per barrier,
// the two-level counter tree 2.3-2.6 us, a single counter 3.8 us.
constexpr int BAR_MODE = 3;

// Task range of this workgroup when T tasks are spread evenly over gridDim.x.
__device__ __forceinline__ void wg_range(int T, int& beg, int& end) {
    beg = (int)((long long)T * blockIdx.x / gridDim.x);
    end = (int)((long long)T * (blockIdx.x + 1) / gridDim.x);
}

// A wave's share of one GEMV phase: task t = rows [t*R, t*R+R) of the
// row-major [N, K] matrix W; this workgroup's tasks are a contiguous range
// and its waves take every 4th; DEPTH tasks are in flight per wave.
template <int R, int KCH, int DEPTH>
struct RowStream {
    u4v buf[DEPTH][R][KCH];
    const _Float16* W;
    int K, N, t0, tend;

    __device__ __forceinline__ void issue(int d, int t) {
        load_rows<R, KCH>(W, K, t * R, t < tend ? min(R, N - t * R) : 0, buf[d]);
    }
    // Issue this wave's first DEPTH tasks of a phase of T tasks.
    __device__ __forceinline__ void start(const _Float16* W_, int K_, int N_, int T) {
        W = W_;
        K = K_;
        N = N_;
        int beg;
        wg_range(T, beg, tend);
        t0 = beg + (int)(threadIdx.x >> 6);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) issue(d, t0 + 4 * d);
    }
    // Reduce every task against the register-resident input xr, in order,
    // refilling each buffer as soon as it is consumed.
    template <class Epi>
    __device__ __forceinline__ void run(const float (&xr)[KCH][8], Epi&& epi) {
        for (int base = t0; base < tend; base += 4 * DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int t = base + 4 * d;
                if (t < tend) {
                    float acc[R];
                    dot_loaded<R, KCH>(buf[d], xr, acc);
                    epi(t, acc);
                    issue(d, t + 4 * DEPTH);
                }
            }
        }
    }
};

}  // namespace

// Ring depths, sized to the work per wave at the 2B-class shapes with one
// workgroup per CU (1024 waves): QKV 2 tasks, output projection 1, gate/up
// 5-6, down 2, LM head ~8; every wave's whole QKV, O and down share is in
// flight at once, gate/up and LM head keep 32 KiB in flight per wave.
template <int KD, int KA, int KF, int HD, int G, int KVF>
__global__ __launch_bounds__(WG) void k_persist(StepArgs A, PersistArgs P) {
    constexpr int KMAX = KF > KD ? (KF > KA ? KF : KA) : (KD > KA ? KD : KA);
    constexpr int DQ = 2, DO = 2, DG = 4, DD = 2, DL = 2;
    __shared__ __attribute__((aligned(16))) float s_vec[KMAX * 512];
    const int lane = threadIdx.x & 63;
    const int D = A.D, F = A.F, V = A.V;
    const int Nqkv = (A.H + 2 * A.Hk) * A.hd, Na = A.H * A.hd;
    unsigned gen = P.gen0;
    int* err = &A.st->err;
    int n_ev = 0;
    auto TR = [&](int code) {
        if (P.trace && blockIdx.x == 0 && threadIdx.x == 0 && n_ev < P.trace_cap) {
            P.trace[1 + 2 * n_ev] = (unsigned long long)code;
            P.trace[2 + 2 * n_ev] = wall_clock64();
            P.trace[0] = (unsigned long long)++n_ev;
        }
    };
    TR(99);

    int tok = A.st->token[0];
    if (tok < 0 || tok >= V) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err, ERR_TOKEN);
        tok = 0;
    }

    RowStream<2, KD, DQ> sq;
    sq.start(P.layers[0].wqkv, D, Nqkv, Nqkv / 2);

    for (int step = 0; step < P.n_steps; ++step) {
        const int pos = P.pos0 + step;
        for (int l = 0; l < A.n_layers; ++l) {
            const LayerW Lw = P.layers[l];
            // ---------------- RMSNorm + QKV + RoPE + KV append ----------------
            {
                float xr[KD][8];
                if (l == 0) {
                    load_x_f16<KD>(A.embed + (size_t)tok * D, D, xr);
                } else {
                    stage_vec<true, KD * 512>(s_vec, A.x, D);
                    load_x_f32<KD>(s_vec, D, xr);
                }
                rmsnorm_regs<KD>(xr, Lw.g_attn, D, A.eps);
                TR(0 + TR_STAGED);
                sq.run(xr, [&](int t, const float (&acc)[2]) {
                    if (lane == 0) qkv_epilogue<KVF, true>(A, l, pos, 2 * t, acc[0], acc[1]);
                });
            }
            TR(0 + TR_DONE);
            RowStream<2, KA, DO> so;
            bar_arrive<BAR_MODE>(P, gen);
            TR(0 + TR_ARRIVED);
            so.start(Lw.wo, Na, D, D / 2);
            TR(0 + TR_ISSUED);
            bar_wait<BAR_MODE>(P, gen, err);
            TR(10 + TR_WAIT);
            // ---------------- attention (split-K, LSE merge, INT8 seal) ----------------
            {
                const AttnArgs T = attn_args(A, l);
                int chunk, nact;
                split_plan(pos + 1, A.S, chunk, nact);
                for (int t = blockIdx.x; t < A.Hk * nact; t += gridDim.x) {
                    const int g = t / nact, s = t % nact;
                    attn_split<HD, G, KVF, true>(T, g, s, chunk, pos);
                    attn_arrive<HD, G, KVF, true>(T, g, nact, pos);
                }
            }
            TR(10 + TR_DONE);
            RowStream<2, KD, DG> sg;
            bar_arrive<BAR_MODE>(P, gen);
            TR(10 + TR_ARRIVED);
            sg.start(Lw.wgu, D, 2 * F, F);
            TR(10 + TR_ISSUED);
            bar_wait<BAR_MODE>(P, gen, err);
            TR(20 + TR_WAIT);
            // ---------------- output projection + residual ----------------
            {
                float xr[KA][8];
                stage_vec<true, KA * 512>(s_vec, A.a, Na);
                load_x_f32<KA>(s_vec, Na, xr);
                TR(20 + TR_STAGED);
                so.run(xr, [&](int t, const float (&acc)[2]) {
                    if (lane == 0) {
#pragma unroll
                        for (int r = 0; r < 2; ++r) {
                            const int row = 2 * t + r;
                            const float base = (l == 0) ? (float)A.embed[(size_t)tok * D + row] : ld_agent(&A.x[row]);
                            st_agent(&A.x[row], base + acc[r]);
                        }
                    }
                });
            }
            TR(20 + TR_DONE);
            bar_arrive<BAR_MODE>(P, gen);
            TR(20 + TR_ARRIVED);
            bar_wait<BAR_MODE>(P, gen, err);
            TR(30 + TR_WAIT);
            // ---------------- RMSNorm + gate/up + SwiGLU ----------------
            {
                float xr[KD][8];
                stage_vec<true, KD * 512>(s_vec, A.x, D);
                load_x_f32<KD>(s_vec, D, xr);
                rmsnorm_regs<KD>(xr, Lw.g_ffn, D, A.eps);
                TR(30 + TR_STAGED);
                sg.run(xr, [&](int t, const float (&acc)[2]) {
                    if (lane == 0) st_agent(&A.m[t], acc[0] / (1.0f + expf(-acc[0])) * acc[1]);
                });
            }
            TR(30 + TR_DONE);
            RowStream<1, KF, DD> sd;
            bar_arrive<BAR_MODE>(P, gen);
            TR(30 + TR_ARRIVED);
            sd.start(Lw.wd, F, D, D);
            TR(30 + TR_ISSUED);
            bar_wait<BAR_MODE>(P, gen, err);
            TR(40 + TR_WAIT);
            // ---------------- down projection + residual ----------------
            {
                float xr[KF][8];
                stage_vec<true, KF * 512>(s_vec, A.m, F);
                load_x_f32<KF>(s_vec, F, xr);
                TR(40 + TR_STAGED);
                sd.run(xr, [&](int t, const float (&acc)[1]) {
                    if (lane == 0) st_agent(&A.x[t], ld_agent(&A.x[t]) + acc[0]);
                });
            }
            TR(40 + TR_DONE);
            bar_arrive<BAR_MODE>(P, gen);
            TR(40 + TR_ARRIVED);
            if (l + 1 < A.n_layers) {
                sq.start(P.layers[l + 1].wqkv, D, Nqkv, Nqkv / 2);
                TR(40 + TR_ISSUED);
                bar_wait<BAR_MODE>(P, gen, err);
                TR(0 + TR_WAIT);
            }
        }
        // ---------------- final RMSNorm + LM head + argmax ----------------
        {
            RowStream<4, KD, DL> sl;
            sl.start(A.lm_head, D, V, (V + 3) / 4);
            TR(40 + TR_ISSUED);
            bar_wait<BAR_MODE>(P, gen, err);
            TR(50 + TR_WAIT);
            float xr[KD][8];
            stage_vec<true, KD * 512>(s_vec, A.x, D);
            load_x_f32<KD>(s_vec, D, xr);
            rmsnorm_regs<KD>(xr, A.g_final, D, A.eps);
            TR(50 + TR_STAGED);
            Best b{-INFINITY, INT_MAX};
            sl.run(xr, [&](int t, const float (&acc)[4]) {
                if (lane == 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 4 * t + r;
                        if (row < V) {
                            A.logits[row] = acc[r];
                            if (!isfinite(acc[r])) atomicOr(err, ERR_NONFINITE);
                            b = better(b, Best{acc[r], row});
                        }
                    }
                }
            });
            TR(50 + TR_DONE);
            b = block_best(b);
            Best fin;
            if (argmax_finish(b, blockIdx.x, gridDim.x, A.arg_val, A.arg_idx, A.arg_cnt, &fin) &&
                threadIdx.x == 0) {
                st_agent(&A.st->token[0], fin.i);
                A.gen_out[P.out_base + step] = fin.i;
                if (step + 1 == P.n_steps) {
                    A.st->pos = P.pos0 + P.n_steps;
                    A.st->n_gen = P.out_base + P.n_steps;
                }
            }
        }
        if (step + 1 < P.n_steps) {
            bar_arrive<BAR_MODE>(P, gen);
            sq.start(P.layers[0].wqkv, D, Nqkv, Nqkv / 2);
            bar_wait<BAR_MODE>(P, gen, err);
            tok = ld_agent(&A.st->token[0]);
        }
    }
    TR(98);
}

// n back-to-back grid barriers and nothing else (barrier latency probe).
template <int MODE>
__global__ __launch_bounds__(WG) void k_barrier_probe(PersistArgs P, int n, int* err) {
    unsigned gen = P.gen0;
    for (int i = 0; i < n; ++i) {
        bar_arrive<MODE>(P, gen);
        bar_wait<MODE>(P, gen, err);
    }
}

// ---- host side ------------------------------------------------------------------------
namespace {
struct Shape {
    int KD, KA, KF, HD, G;
};
// Instantiated shapes: the 2B-class model, the 1-layer tiny model, and a
// small GQA model used by the tests.
constexpr Shape kShapes[] = {{4, 4, 11, 128, 2}, {1, 1, 2, 64, 1}, {1, 1, 4, 64, 4}};

Shape shape_of(const StepArgs& A) {
    return Shape{kch_for(A.D), kch_for(A.H * A.hd), kch_for(A.F), A.hd, A.H / A.Hk};
}
bool same(const Shape& a, const Shape& b) {
    return a.KD == b.KD && a.KA == b.KA && a.KF == b.KF && a.HD == b.HD && a.G == b.G;
}

template <int KD, int KA, int KF, int HD, int G>
const void* kernel_for_fmt(int kvfmt) {
    switch (kvfmt) {
        case KV_FP16: return (const void*)&k_persist<KD, KA, KF, HD, G, KV_FP16>;
        case KV_E5M2: return (const void*)&k_persist<KD, KA, KF, HD, G, KV_E5M2>;
        case KV_INT8: return (const void*)&k_persist<KD, KA, KF, HD, G, KV_INT8>;
    }
    return nullptr;
}

const void* kernel_for(const StepArgs& A) {
    const Shape s = shape_of(A);
    if (same(s, kShapes[0])) return kernel_for_fmt<4, 4, 11, 128, 2>(A.kvfmt);
    if (same(s, kShapes[1])) return kernel_for_fmt<1, 1, 2, 64, 1>(A.kvfmt);
    if (same(s, kShapes[2])) return kernel_for_fmt<1, 1, 4, 64, 4>(A.kvfmt);
    return nullptr;
}
}  // namespace

bool persistent_supported(const StepArgs& A) { return kernel_for(A) != nullptr; }

hipError_t persistent_max_grid(const StepArgs& A, int device, int* nwg) {
    const void* k = kernel_for(A);
    if (!k) return hipErrorInvalidValue;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) return e;
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, WG, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    *nwg = prop.multiProcessorCount;   // one workgroup per CU
    return hipSuccess;
}

hipError_t launch_persistent(const StepArgs& A, const PersistArgs& P, int nwg, hipStream_t s) {
    const void* k = kernel_for(A);
    if (!k) return hipErrorInvalidValue;
    StepArgs a = A;
    PersistArgs p = P;
    void* args[] = {&a, &p};
    return hipLaunchCooperativeKernel(k, dim3(nwg), dim3(WG), args, 0, s);
}

hipError_t barrier_probe(int nwg, int n, int mode, float* us, int* errbits) {
    int* bar = nullptr;
    int* err = nullptr;
    hipEvent_t e0, e1;
    hipError_t e;
    const void* kern = nullptr;
    switch (mode) {
        case 0: kern = (const void*)&k_barrier_probe<0>; break;
        case 1: kern = (const void*)&k_barrier_probe<1>; break;
        case 2: kern = (const void*)&k_barrier_probe<2>; break;
        case 3: kern = (const void*)&k_barrier_probe<3>; break;
        case 4: kern = (const void*)&k_barrier_probe<4>; break;
        case 5: kern = (const void*)&k_barrier_probe<5>; break;
        case 6: kern = (const void*)&k_barrier_probe<6>; break;
        default: return hipErrorInvalidValue;
    }
    if (nwg < 1 || nwg > BAR_MAX_WG) return hipErrorInvalidValue;
    if ((e = hipMalloc(&bar, BAR_WORDS * sizeof(int) + 256)) != hipSuccess) return e;
    err = bar + BAR_WORDS;
    if ((e = hipMemset(bar, 0, BAR_WORDS * sizeof(int) + 256)) != hipSuccess) goto out;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    {
        PersistArgs P{};
        P.bar = bar;
        P.spin_limit = 1 << 24;
        int nn = n;
        void* args[] = {&P, &nn, &err};
        (void)hipEventRecord(e0, nullptr);
        e = hipLaunchCooperativeKernel(kern, dim3(nwg), dim3(WG), args, 0, nullptr);
        (void)hipEventRecord(e1, nullptr);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.f;
        (void)hipEventElapsedTime(&ms, e0, e1);
        *us = ms * 1000.0f / (float)n;
        (void)hipMemcpy(errbits, err, sizeof(int), hipMemcpyDeviceToHost);
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
out:
    (void)hipFree(bar);
    return e;
}

}  // namespace rd
