// Persistent decode-step executor for gfx950: one cooperative launch runs
// whole decode steps, one workgroup per CU, with no grid barrier at all.
//
// Why: at batch 1 a phase streams only 8-46 MB, so a kernel per phase pays
// its launch, ramp-up, first-byte latency and drain every time, and the
// memory stream stops at each boundary ("Real-time LLM inference on
// standard GPUs: 3,000 tokens/s per request", table of microsecond losses:
// kernel boundaries and grid synchronisation; the fix it names is a single
// resident program whose weight prefetch overlaps the compute sections).
//
// Dataflow instead of barriers.  Every vector one phase hands to the next
// (the residual stream after each projection, the rotated q with the new
// K/V row, the attention partials and output, the SwiGLU output, the argmax
// candidates) is published as 64-bit words that carry the payload in the low
// half (an fp32 value, or two fp16 elements of a GEMV operand) and a tag
// naming the (step, layer) in the high half, written with one
// agent-coherent store each.  A consumer polls exactly the words it needs
// until every tag matches; a word is never torn, so seeing the tag means
// seeing the value, and the data arrives in the same round trip that
// signals it.  Only words still missing are fetched again.  Each object has
// one buffer: the next write of any object causally follows every read of
// its previous contents (every phase needs the whole output of the one
// before it), so no reader can meet a newer tag than the one it waits for.
//
// Roles inside a workgroup (4 waves, one per SIMD: the control wave has a
// SIMD and its whole register file to itself).  A wave's vector-memory
// counter completes in order, so a load the critical path waits on would sit
// behind every weight load the same wave has in flight; the roles are split:
//   - waves 1..3 (stream) only move and reduce weights.  Each owns a ring of
//     RING 1 KiB slots in LDS and a cursor over the weight rows it reduces,
//     in the order it reduces them, across phases, layers and steps.  Loads
//     go straight from HBM into the ring (global_load_lds_dwordx4,
//     non-temporal: no VGPRs held, nothing kept in L2), RING slots ahead of
//     the row being reduced, so the ring keeps filling with the next
//     phases' rows while the control wave waits for inputs or attends.
//   - wave 0 (control) polls each phase's input, stages it into LDS (with
//     the RMSNorm where the phase has one), runs every epilogue from the row
//     sums (RoPE and the KV append, residual adds, SwiGLU, logits, argmax),
//     polls the query and the new K/V row of the workgroup's attention split
//     and combines the stream waves' partials of it, and in some workgroups
//     merges one query head.  The stream waves reduce the split's key rows
//     (the first batch fetched at the end of their QKV rows).
//
// Every arithmetic step is the one the kernel-per-phase executor performs
// (rd_phases.h), in the same order, so both executors give identical bits.
#include <algorithm>

#include "rd_phases.h"

namespace rd {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int NSW = 3;                  // stream waves per workgroup (waves 1..3)
constexpr int PWG = (NSW + 1) * WAVE;   // threads per workgroup
constexpr int UNIT = 1024;              // bytes per ring slot: 16 per lane, one chunk of one row
constexpr int RING = 47;                // ring slots per stream wave
constexpr int PART_MAX = 512;           // row sums a workgroup holds per phase
constexpr int OWN_MAX = 64;             // residual-stream rows a workgroup owns
constexpr int LB_MAX = 1024;            // workgroups (argmax candidates)

// buf[i] with a 32-bit byte offset on a scalar base (one VGPR per address).
__device__ __forceinline__ const uint64_t* word_at(const uint64_t* buf, int i) {
    return reinterpret_cast<const uint64_t*>(reinterpret_cast<const char*>(buf) + (uint32_t)i * 8u);
}

// Workgroup barrier that orders LDS only.  The waves of a workgroup share
// nothing but LDS (the staged input, the row sums, the trace counter; each
// ring is read only by the wave that fills it), so a barrier waits for this
// wave's LDS operations and nothing else.  __syncthreads() would also wait
// for every outstanding global load: a stream wave would drain its whole
// ring at each phase boundary and lose the prefetch.  The memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS accesses of the stream waves are inline asm.  Their LDS-DMA ring loads
// are outstanding at all times, and the compiler cannot tell that an LDS
// read or write does not touch a slot still being filled, so before every
// LDS instruction it emits it would wait for all outstanding loads
// (vmcnt(0)): the ring would drain at each row group.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)reinterpret_cast<uintptr_t>((lds_void*)p);
}
// n (1..8) 16-byte LDS reads and the wait for them, as one asm statement:
// the results exist only once the statement ends (as separate statements,
// the compiler could copy a destination before its load landed).  Outputs
// are early-clobber: no destination may share a register with an address
// that a later read of the same statement still uses.
__device__ __forceinline__ void lds_read_wait1(u4v* d, const unsigned* a) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(d[0]) : "v"(a[0]) : "memory");
}
__device__ __forceinline__ void lds_read_wait2(u4v* d, const unsigned* a) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)" : "=&v"(d[0]), "=&v"(d[1]) : "v"(a[0]), "v"(a[1]) : "memory");
}
__device__ __forceinline__ void lds_read_wait3(u4v* d, const unsigned* a) {
    asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\ts_waitcnt lgkmcnt(0)" : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]) : "v"(a[0]), "v"(a[1]), "v"(a[2]) : "memory");
}
__device__ __forceinline__ void lds_read_wait4(u4v* d, const unsigned* a) {
    asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)" : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]) : "memory");
}
__device__ __forceinline__ void lds_read_wait5(u4v* d, const unsigned* a) {
    asm volatile("ds_read_b128 %0, %5\n\tds_read_b128 %1, %6\n\tds_read_b128 %2, %7\n\tds_read_b128 %3, %8\n\tds_read_b128 %4, %9\n\ts_waitcnt lgkmcnt(0)" : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]) : "memory");
}
__device__ __forceinline__ void lds_read_wait6(u4v* d, const unsigned* a) {
    asm volatile("ds_read_b128 %0, %6\n\tds_read_b128 %1, %7\n\tds_read_b128 %2, %8\n\tds_read_b128 %3, %9\n\tds_read_b128 %4, %10\n\tds_read_b128 %5, %11\n\ts_waitcnt lgkmcnt(0)" : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]) : "memory");
}
__device__ __forceinline__ void lds_read_wait7(u4v* d, const unsigned* a) {
    asm volatile("ds_read_b128 %0, %7\n\tds_read_b128 %1, %8\n\tds_read_b128 %2, %9\n\tds_read_b128 %3, %10\n\tds_read_b128 %4, %11\n\tds_read_b128 %5, %12\n\tds_read_b128 %6, %13\n\ts_waitcnt lgkmcnt(0)" : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]), "=&v"(d[6]) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]) : "memory");
}
__device__ __forceinline__ void lds_read_wait8(u4v* d, const unsigned* a) {
    asm volatile("ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\tds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\ts_waitcnt lgkmcnt(0)" : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]), "=&v"(d[6]), "=&v"(d[7]) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]) : "memory");
}
template <int N>
__device__ __forceinline__ void lds_read_wait(u4v (&d)[N], const unsigned (&a)[N]) {
#pragma unroll
    for (int i = 0; i < N; i += 8) {
        constexpr int dummy = 0;
        (void)dummy;
        const int m = N - i < 8 ? N - i : 8;
        switch (m) {
            case 1: lds_read_wait1(d + i, a + i); break;
            case 2: lds_read_wait2(d + i, a + i); break;
            case 3: lds_read_wait3(d + i, a + i); break;
            case 4: lds_read_wait4(d + i, a + i); break;
            case 5: lds_read_wait5(d + i, a + i); break;
            case 6: lds_read_wait6(d + i, a + i); break;
            case 7: lds_read_wait7(d + i, a + i); break;
            default: lds_read_wait8(d + i, a + i); break;
        }
    }
}
__device__ __forceinline__ void lds_write4(unsigned addr, float v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
// The O and down phases' inputs arrive chunk by chunk (stage_stream): the control
// wave writes a chunk to LDS, waits for the write, then publishes the count
// of staged chunks in s_flag; stream waves read the count before the chunk.
__device__ __forceinline__ void post_count(int* s_flag, int n) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\tds_write_b32 %0, %1" ::"v"(lds_addr(s_flag)), "v"(n) : "memory");
}
__device__ __forceinline__ int read_count(const int* s_flag) {
    int v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(s_flag)) : "memory");
    return __builtin_amdgcn_readfirstlane(v);
}
constexpr int COUNT_SPIN = 1 << 24;   // reads of the count before a stream wave goes on regardless

__device__ __forceinline__ uint64_t tagged(float v, uint32_t tag) {
    return ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
}
__device__ __forceinline__ void publish(uint64_t* p, float v, uint32_t tag) { st_agent(p, tagged(v, tag)); }
__device__ __forceinline__ void publish_bits(uint64_t* p, uint32_t v, uint32_t tag) {
    st_agent(p, ((uint64_t)tag << 32) | (uint64_t)v);
}
__device__ __forceinline__ uint32_t tag_of(const StepArgs& A, const PersistArgs& P, int step, int layer) {
    return P.tag0 + (uint32_t)step * (uint32_t)(A.n_layers + 1) + (uint32_t)layer + 1u;
}
// 12-bit tag of the argmax words: never 0, so zero-filled words never match.
__device__ __forceinline__ uint32_t tag12(uint32_t tag) { return tag % 4095u + 1u; }

// ---- waiting ------------------------------------------------------------------
// Every wait counts its polls; past the spin limit it raises the abort word
// and an error bit, and every wait that sees the abort word gives up too, so
// a launch always runs to its end.
struct Waiter {
    int* abort_word;
    int* err;
    int limit, n;
    __device__ __forceinline__ bool again() {   // false: give up
        if ((++n & 63) == 0) {
            if (ld_agent(abort_word)) return false;
            if (n > limit) {
                if (lane_id() == 0) {
                    st_agent(abort_word, 1);
                    atomicOr(err, ERR_STALL);
                }
                return false;
            }
        }
        return true;
    }
};

// Poll NW words per lane (word idx(k) where act(k)) until each carries tag;
// val[k] receives the values (0 where !act(k)).  A word is fetched again
// only while the copy in hand still has an old tag; inactive words start as
// received.
template <int NW, class IDX, class ACT>
__device__ __forceinline__ void poll_words(Waiter& wt, const uint64_t* buf, IDX&& idx, ACT&& act, uint32_t tag,
                                           float (&val)[NW]) {
    const uint64_t done = (uint64_t)tag << 32;
    uint64_t v[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) v[k] = act(k) ? 0ull : done;
    wt.n = 0;
    while (true) {
#pragma unroll
        for (int k = 0; k < NW; ++k)
            if ((uint32_t)(v[k] >> 32) != tag) v[k] = ld_agent(word_at(buf, idx(k)));
        bool all = true;
#pragma unroll
        for (int k = 0; k < NW; ++k) all &= (uint32_t)(v[k] >> 32) == tag;
        if (__all(all)) break;
        if (!wt.again()) break;
    }
#pragma unroll
    for (int k = 0; k < NW; ++k) val[k] = __uint_as_float((uint32_t)v[k]);
}

// Poll a K-element vector published as fp16 pairs (word w: elements 2w,
// 2w+1) into the GEMV input layout in registers (lane l, chunk c: elements
// (c*64+l)*8..+7), which the RMSNorm sums in.  The poll loads read 16
// bytes per lane and whole lines (as stage_stream16: load i of chunk c reads
// the chunk's words i*128 + 2*lane, +1, each word checked for its own tag),
// and the words reach the lane layout through LDS (s, whose chunks the
// caller has not posted yet).
template <int KCH>
__device__ __forceinline__ void poll_vec_h2(Waiter& wt, const uint64_t* buf, int K, uint32_t tag, float* s,
                                               float (&xr)[KCH][8]) {
    const int lane = lane_id();
    const __amdgpu_buffer_rsrc_t rs = attn_rsrc(buf, (size_t)K * 4);
    auto pair = [&](int k) { return (k / 2) * 256 + (k % 2) * 128 + 2 * lane; };
    u4v v[KCH * 2];
#pragma unroll
    for (int k = 0; k < KCH * 2; ++k) v[k] = 2 * pair(k) < K ? u4v{0u, 0u, 0u, 0u} : u4v{0u, tag, 0u, tag};
    wt.n = 0;
    while (true) {
#pragma unroll
        for (int k = 0; k < KCH * 2; ++k)
            if (v[k].y != tag || v[k].w != tag)
                v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)pair(k) * 8u, 0, AUX_AGENT);
        bool all = true;
#pragma unroll
        for (int k = 0; k < KCH * 2; ++k) all &= v[k].y == tag && v[k].w == tag;
        if (__all(all)) break;
        if (!wt.again()) break;
    }
#pragma unroll
    for (int k = 0; k < KCH * 2; ++k) reinterpret_cast<u2v*>(s)[pair(k) / 2] = u2v{v[k].x, v[k].z};
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const u4v w = reinterpret_cast<const u4v*>(s)[c * 64 + lane];
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xr[c][2 * i] = h_bits2f((uint16_t)(u[i] & 0xffffu));
            xr[c][2 * i + 1] = h_bits2f((uint16_t)(u[i] >> 16));
        }
    }
}

// The O and down phases' input (fp16 pairs, word w: elements 2w, 2w+1),
// polled and staged as it goes: after each round of polls, the chunks
// complete in every lane are written to LDS in chunk order (the layout of
// regs_to_lds: LDS word j of a chunk holds its pair j) and their count posted
// (fl + chunks staged), so the stream waves start on the first chunks while
// later ones are still on their way.  No norm needs the elements in a lane's
// registers here, so load i of chunk c reads the chunk's pairs i*64 + lane:
// 512 contiguous bytes per load instruction, each line requested once per
// round (four loads of one lane's four consecutive pairs would span 2 KB
// each and request every line four times).  A wait that gives up stages the
// rest as they stand.
template <int KCH>
__device__ __forceinline__ void stage_stream(Waiter& wt, const uint64_t* buf, int K, uint32_t tag, float* s,
                                             int* s_flag, int fl) {
    const int lane = lane_id();
    const uint64_t done = (uint64_t)tag << 32;
    auto pair = [&](int k) { return (k / 4) * 256 + (k % 4) * 64 + lane; };
    uint64_t v[KCH * 4];
#pragma unroll
    for (int k = 0; k < KCH * 4; ++k) v[k] = 2 * pair(k) < K ? 0ull : done;
    int staged = 0;
    bool live = true;
    wt.n = 0;
    while (true) {
#pragma unroll
        for (int k = 0; k < KCH * 4; ++k)
            if ((uint32_t)(v[k] >> 32) != tag) v[k] = ld_agent(word_at(buf, pair(k)));
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            if (c == staged) {
                bool ok = true;
#pragma unroll
                for (int i = 0; i < 4; ++i) ok &= (uint32_t)(v[c * 4 + i] >> 32) == tag;
                if (__all(ok) || !live) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) reinterpret_cast<uint32_t*>(s)[pair(c * 4 + i)] = (uint32_t)v[c * 4 + i];
                    ++staged;
                    post_count(s_flag, fl + staged);
                }
            }
        }
        if (staged == KCH || !live) break;
        live = wt.again();
    }
}

// stage_stream with 16-byte poll loads: lane l's load i of chunk c reads the
// chunk's words i*128 + 2l, +1 (1 KiB contiguous per load instruction, half
// the instructions per round).  Each 8-byte word was written by one 64-bit
// store and carries its own tag, so each is checked on its own.  A poll
// round waits for all of its loads, and each load instruction queues in the
// CU's memory path behind the weight refills: for the down input (d_ff
// elements, 44 eight-byte loads per lane) fewer instructions shorten the
// round.  (agent-coherent buffer loads, as the attention's.)
template <int KCH>
__device__ __forceinline__ void stage_stream16(Waiter& wt, const uint64_t* buf, int K, uint32_t tag, float* s,
                                               int* s_flag, int fl) {
    const int lane = lane_id();
    const __amdgpu_buffer_rsrc_t rs = attn_rsrc(buf, (size_t)K * 4);
    auto pair = [&](int k) { return (k / 2) * 256 + (k % 2) * 128 + 2 * lane; };
    u4v v[KCH * 2];
#pragma unroll
    for (int k = 0; k < KCH * 2; ++k) v[k] = 2 * pair(k) < K ? u4v{0u, 0u, 0u, 0u} : u4v{0u, tag, 0u, tag};
    int staged = 0;
    bool live = true;
    wt.n = 0;
    while (true) {
#pragma unroll
        for (int k = 0; k < KCH * 2; ++k)
            if (v[k].y != tag || v[k].w != tag)
                v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)pair(k) * 8u, 0, AUX_AGENT);
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            if (c == staged) {
                bool ok = true;
#pragma unroll
                for (int i = 0; i < 2; ++i) ok &= v[c * 2 + i].y == tag && v[c * 2 + i].w == tag;
                if (__all(ok) || !live) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        reinterpret_cast<u2v*>(s)[pair(c * 2 + i) / 2] = u2v{v[c * 2 + i].x, v[c * 2 + i].z};
                    ++staged;
                    post_count(s_flag, fl + staged);
                }
            }
        }
        if (staged == KCH || !live) break;
        live = wt.again();
    }
}

// A normalised operand (xr) into LDS chunk by chunk, each chunk's count
// posted as soon as it is written (the RMSNorm phases: the norm needs the
// whole vector, then the stream waves start on chunk 0 while the control
// wave writes the rest).  The layout and values of regs_to_lds.
template <int KCH>
__device__ __forceinline__ void stage_chunks(float* s, const float (&xr)[KCH][8], int* s_flag, int fl) {
    const int lane = lane_id();
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        float x1[1][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x1[0][i] = xr[c][i];
        u4v xh[1];
        pack_x<1>(x1, xh);
        reinterpret_cast<u4v*>(s)[c * 64 + lane] = xh[0];
        post_count(s_flag, fl + c + 1);
    }
}

// The GEMV operand of a phase into LDS for the stream waves: the fp16
// rounding of the vector (pack_x), 16 bytes per lane and chunk at byte
// (c*64 + lane)*16, zero past K.
template <int KCH>
__device__ __forceinline__ void regs_to_lds(float* s, const float (&xr)[KCH][8]) {
    const int lane = lane_id();
    u4v xh[KCH];
    pack_x<KCH>(xr, xh);
#pragma unroll
    for (int c = 0; c < KCH; ++c) reinterpret_cast<u4v*>(s)[c * 64 + lane] = xh[c];
}

// ---- event trace -----------------------------------------------------------------
// Lane 0 of the control wave appends (code, wall clock) events to the lower
// half of the workgroup's region, counted in LDS; stream wave 0 fills the
// upper half (StreamTracer).  The control wave writes both counts out at the
// end of the launch.  Inline: a call would make the wave wait for all its
// outstanding memory operations at the callee's entry and skew the times.
__device__ __forceinline__ void trace_event(unsigned long long* tb, int cap, int* s_nev, int code) {
    if (lane_id() == 0) {
        const int i = atomicAdd(s_nev, 1);
        if (i < cap / 2) {
            tb[1 + 2 * i] = (unsigned long long)code;
            tb[2 + 2 * i] = wall_clock64();
        }
    }
}
struct Tracer {
    unsigned long long* tb;   // this workgroup's region, or null
    int cap;
    int* s_nev;
    __device__ __forceinline__ void operator()(int code) const {
        if (tb) trace_event(tb, cap, s_nev, code);
    }
};
// The stream waves' tracer: wave 0 of them records into the upper half of
// the workgroup's region with a register count, inline and without LDS
// access (an LDS atomic or a call would drain the wave's load ring, see
// lds_read_wait).
struct StreamTracer {
    unsigned long long* tb;
    int cap, n;
    __device__ __forceinline__ void operator()(int code) {
        if (tb) {
            if (lane_id() == 0 && n < cap - cap / 2) {
                const int i = cap / 2 + n;
                tb[1 + 2 * i] = (unsigned long long)code;
                tb[2 + 2 * i] = wall_clock64();
            }
            ++n;
        }
    }
};
__device__ __forceinline__ Tracer make_tracer(const PersistArgs& P, int* s_nev) {
    Tracer t{nullptr, 0, s_nev};
    if (P.trace && (P.trace_all || blockIdx.x == 0)) {
        t.tb = P.trace + (P.trace_all ? (size_t)blockIdx.x * (1 + 2 * (size_t)P.trace_cap) : 0);
        t.cap = P.trace_cap;
    }
    return t;
}

// ---- weight schedule ------------------------------------------------------------
// Rows [r0, r1) of this workgroup when N rows are dealt to the grid in tasks
// of rpt consecutive rows (T * blockIdx < 2^32 for every shape built).
__device__ __forceinline__ void wg_rows(int N, int rpt, int& r0, int& r1) {
    const unsigned T = (unsigned)(N / rpt), b = blockIdx.x, n = gridDim.x;
    r0 = (int)(T * b / n) * rpt;
    r1 = (int)(T * (b + 1) / n) * rpt;
}

// Phase ph of a step: 4 per layer (QKV, output projection, gate/up, down),
// then the LM head.  RoPE pairs and gate/up pairs stay in one workgroup.
struct PhaseGeo {
    const _Float16* W;
    int K, kch;
    int r0, r1;   // this workgroup's rows
};
// Layer l's copy of a weight whose layer-0 copy is at p0: the weight image
// repeats one layer block at a fixed stride, so every weight address is
// scalar arithmetic on kernel arguments.
__device__ __forceinline__ const _Float16* layer_w(const PersistArgs& P, const _Float16* p0, int l) {
    return reinterpret_cast<const _Float16*>(reinterpret_cast<const char*>(p0) + (long long)l * P.layer_stride);
}

template <int KD, int KA, int KF>
__device__ __forceinline__ PhaseGeo phase_geo(const StepArgs& A, const PersistArgs& P, int ph) {
    PhaseGeo g;
    if (ph == 4 * A.n_layers) {
        g.W = A.lm_head; g.K = A.D; g.kch = KD;
        wg_rows(A.V, 1, g.r0, g.r1);
    } else {
        const int l = ph >> 2;
        switch (ph & 3) {
            case 0:
                g.W = layer_w(P, P.layer0.wqkv, l); g.K = A.D; g.kch = KD;
                wg_rows((A.H + 2 * A.Hk) * A.hd, 2, g.r0, g.r1);
                break;
            // O and down: owned residual rows in pairs (published as fp16 pairs)
            case 1: g.W = layer_w(P, P.layer0.wo, l); g.K = A.H * A.hd; g.kch = KA; wg_rows(A.D, 2, g.r0, g.r1); break;
            // gate/up in tasks of 4 rows: each workgroup's SwiGLU outputs are
            // whole fp16 pairs of the exchange
            case 2: g.W = layer_w(P, P.layer0.wgu, l); g.K = A.D; g.kch = KD; wg_rows(2 * A.F, 4, g.r0, g.r1); break;
            default: g.W = layer_w(P, P.layer0.wd, l); g.K = A.F; g.kch = KF; wg_rows(A.D, 2, g.r0, g.r1); break;
        }
    }
    return g;
}
__device__ __forceinline__ void wave_rows(const PhaseGeo& g, int sw, int& ra, int& rb) {
    const int n = g.r1 - g.r0;
    ra = g.r0 + n * sw / NSW;
    rb = g.r0 + n * (sw + 1) / NSW;
}

// A stream wave's load cursor: the next 1 KiB chunk to request and the ring
// slot it goes to.  Past the last row of the launch it keeps requesting the
// first rows of the LM head (never reduced), so that exactly RING requests
// are always outstanding or landed beyond the slot being read and every wait
// is the same constant.
// The wave's rows of each of the five phase kinds (QKV, output projection,
// gate/up, down, LM head) are the same in every layer and step; they are
// computed once, so moving to the next phase is a table lookup.
// FK (every K a multiple of 512): a wave's rows of one phase are one
// contiguous byte range of whole 1 KiB chunks, so the cursor is a pointer
// and a count of chunks left in the range.  Otherwise rows end inside a
// chunk: the cursor walks (row, chunk) and lanes past K read the chunk's
// first 16 bytes (in bounds), masked when reduced.
// a[k] for a wave-uniform k through selects: a private array indexed at run
// time would live in scratch memory.
__device__ __forceinline__ int pick5(const int (&a)[5], int k) {
    return k == 0 ? a[0] : k == 1 ? a[1] : k == 2 ? a[2] : k == 3 ? a[3] : a[4];
}

template <int KD, int KA, int KF, bool FK>
struct Feeder {
    const char* p;   // FK: next chunk; else: start of the current row
    int left;        // FK: chunks left in the current range
    int K, kch, c, row, rend;   // !FK
    int ph, step, slot;
    unsigned char* ring;
    int ra[5], nr[5], r0[5];    // per phase kind: this wave's first row and row count, the workgroup's first row

    __device__ __forceinline__ void init(const StepArgs& A, const PersistArgs& P, int sw) {
        for (int k = 0; k < 5; ++k) {
            const PhaseGeo g = phase_geo<KD, KA, KF>(A, P, k == 4 ? 4 * A.n_layers : k);
            int a, b;
            wave_rows(g, sw, a, b);
            ra[k] = a;
            nr[k] = b - a;
            r0[k] = g.r0;
        }
    }
    __device__ __forceinline__ void seek(const StepArgs& A, const PersistArgs& P) {
        const int NP = 4 * A.n_layers + 1;
        while (true) {
            if (ph == NP) {
                ph = 0;
                if (++step >= P.n_steps) {
                    p = reinterpret_cast<const char*>(A.lm_head);
                    left = INT_MAX;
                    K = A.D;
                    kch = KD;
                    c = 0;
                    row = 0;
                    rend = INT_MAX;
                    return;
                }
            }
            const int k = ph == NP - 1 ? 4 : (ph & 3), l = ph >> 2;
            const int nrk = pick5(nr, k), rak = pick5(ra, k);
            if (nrk > 0) {
                const _Float16* W;
                switch (k) {
                    case 0: W = layer_w(P, P.layer0.wqkv, l); K = A.D; kch = KD; break;
                    case 1: W = layer_w(P, P.layer0.wo, l); K = A.H * A.hd; kch = KA; break;
                    case 2: W = layer_w(P, P.layer0.wgu, l); K = A.D; kch = KD; break;
                    case 3: W = layer_w(P, P.layer0.wd, l); K = A.F; kch = KF; break;
                    default: W = A.lm_head; K = A.D; kch = KD; break;
                }
                p = reinterpret_cast<const char*>(W + (size_t)rak * K);
                left = nrk * kch;
                c = 0;
                row = rak;
                rend = rak + nrk;
                return;
            }
            ++ph;
        }
    }
    __device__ __forceinline__ void issue(const StepArgs& A, const PersistArgs& P) {
        // cache policy 2: non-temporal (every weight byte is read once per step)
        if constexpr (FK) {
            __builtin_amdgcn_global_load_lds((glb_void*)(p + (uint32_t)lane_id() * 16u),
                                             (lds_void*)(ring + slot * UNIT), 16, 0, 2);
            p += UNIT;
            slot = slot + 1 == RING ? 0 : slot + 1;
            if (--left == 0) {
                ++ph;
                seek(A, P);
            }
        } else {
            unsigned off = (unsigned)lane_id() * 16u;
            if (c * 1024 + (int)off >= 2 * K) off = 0;
            __builtin_amdgcn_global_load_lds((glb_void*)(p + c * 1024 + off), (lds_void*)(ring + slot * UNIT), 16, 0,
                                             2);
            slot = slot + 1 == RING ? 0 : slot + 1;
            if (++c == kch) {
                c = 0;
                p += 2 * K;
                if (++row == rend) {
                    ++ph;
                    seek(A, P);
                }
            }
        }
    }
    // n refills; while the current range has more than n chunks left (FK),
    // unrolled without the per-chunk range test.
    template <int N>
    __device__ __forceinline__ void issue_n(const StepArgs& A, const PersistArgs& P) {
        if constexpr (FK) {
            if (left > N) {
                const unsigned off = (unsigned)lane_id() * 16u;
                int sl = slot;
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    __builtin_amdgcn_global_load_lds((glb_void*)(p + i * UNIT + off), (lds_void*)(ring + sl * UNIT),
                                                     16, 0, 2);
                    sl = sl + 1 == RING ? 0 : sl + 1;
                }
                p += N * UNIT;
                left -= N;
                slot = sl;
                return;
            }
        }
        for (int i = 0; i < N; ++i) issue(A, P);
    }
    __device__ __forceinline__ void start(const StepArgs& A, const PersistArgs& P, int sw, unsigned char* r) {
        ring = r;
        init(A, P, sw);
        ph = 0;
        step = 0;
        slot = 0;
        seek(A, P);
        for (int i = 0; i < RING; ++i) issue(A, P);
    }
};

// Reduce the next NR rows (KCH chunks each) of the wave's stream against the
// register-resident input xr: wait for their slots, read them, refill them,
// then the dot products of dot_rows.
template <int NR, int KCH, bool FK, class F>
__device__ __forceinline__ void consume_rows(F& f, const StepArgs& A, const PersistArgs& P, int sw,
                                             unsigned char* ring, const u4v (&xh)[KCH], int K,
                                             float (&out)[NR]) {
    static_assert(NR * KCH <= RING, "ring shorter than the rows reduced together");
    const int lane = lane_id();
    const unsigned base = lds_addr(ring) + (unsigned)lane * 16u;
    unsigned ad[NR * KCH];
    int s = f.slot;
#pragma unroll
    for (int i = 0; i < NR * KCH; ++i) {
        ad[i] = base + (unsigned)s * UNIT;
        s = s + 1 == RING ? 0 : s + 1;
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(RING - NR * KCH) : "memory");
    u4v wl[NR * KCH];
    lds_read_wait<NR * KCH>(wl, ad);   // slots read before they are refilled
    u4v w[NR][KCH];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int c = 0; c < KCH; ++c) w[r][c] = wl[r * KCH + c];
    f.template issue_n<NR * KCH>(A, P);
    if constexpr (!FK) {
#pragma unroll
        for (int c = 0; c < KCH; ++c)
            if ((c * 64 + lane) * 8 >= K)
#pragma unroll
                for (int r = 0; r < NR; ++r) w[r][c] = u4v{0u, 0u, 0u, 0u};
    }
    dot_rows<NR, KCH>(w, xh, out);
}

// consume_rows for the first rows of a phase whose input is staged chunk by
// chunk (stage_stream): the rows' chunks are taken from the ring as in
// consume_rows, then each chunk of the input is read once its count is
// posted (fl: the count before this phase), into xh for the later rows, and
// reduced at once.  The slots are refilled at once, (late) once chunk 0 is
// posted, or (gate > 0) once the control wave's count of attention publishes
// reaches gate.  The sums are dot_rows' in the same order.
template <int NR, int KCH, bool FK, class F>
__device__ __forceinline__ void consume_rows_strm(F& f, const StepArgs& A, const PersistArgs& P,
                                                  unsigned char* ring, const float* s_r, const int* s_flag, int fl,
                                                  u4v (&xh)[KCH], int K, float (&out)[NR], bool late,
                                                  int gate = 0) {
    static_assert(NR * KCH <= RING, "ring shorter than the rows reduced together");
    const int lane = lane_id();
    const unsigned base = lds_addr(ring) + (unsigned)lane * 16u;
    unsigned ad[NR * KCH];
    int s = f.slot;
#pragma unroll
    for (int i = 0; i < NR * KCH; ++i) {
        ad[i] = base + (unsigned)s * UNIT;
        s = s + 1 == RING ? 0 : s + 1;
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(RING - NR * KCH) : "memory");
    u4v wl[NR * KCH];
    lds_read_wait<NR * KCH>(wl, ad);   // slots read before they are refilled
    if (!late) {
        // gate > 0 (O, down): once the control wave has issued the stores of
        // the attention split or the SwiGLU output (it posts their count in
        // s_flag[1]), so that they do not queue behind these refills in the
        // CU's memory path
        if (gate > 0)
            for (int it = 0; it < COUNT_SPIN && read_count(s_flag + 1) < gate; ++it) {
            }
        f.template issue_n<NR * KCH>(A, P);
    }
    if constexpr (!FK) {
#pragma unroll
        for (int c = 0; c < KCH; ++c)
            if ((c * 64 + lane) * 8 >= K)
#pragma unroll
                for (int r = 0; r < NR; ++r) wl[r * KCH + c] = u4v{0u, 0u, 0u, 0u};
    }
    const unsigned xb = lds_addr(s_r) + (unsigned)lane * 16u;
    float s0[NR], s1[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) s0[r] = s1[r] = 0.f;
    int have = 0;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        for (int it = 0; have <= c && it < COUNT_SPIN; ++it) have = read_count(s_flag) - fl;
        if (c == 0 && late) f.template issue_n<NR * KCH>(A, P);
        {
            const unsigned a1[1] = {xb + (unsigned)c * 1024u};
            u4v x1[1];
            lds_read_wait<1>(x1, a1);
            xh[c] = x1[0];
        }
        u4v wc[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) wc[r] = wl[r * KCH + c];
        dot_chunk<NR>(wc, xh[c], s0, s1);
    }
    dot_finish<NR>(s0, s1, out);
}

// A stream wave's share of GEMV phase ph, between the workgroup barriers
// that bracket it: its rows' sums into s_part.  STRM: the input is staged
// chunk by chunk (no barrier before the phase; s_flag, fl as in
// consume_rows_strm).
template <int KCH, int KD, int KA, int KF, bool FK, bool STRM = false, class F, class Tail>
__device__ __forceinline__ void stream_phase(F& f, const StepArgs& A, const PersistArgs& P, int sw,
                                             unsigned char* ring, const float* s_r, float* s_part, int ph,
                                             StreamTracer& tr, Tail tail, const int* s_flag = nullptr,
                                             int fl = 0, int gate = 0) {
    constexpr int NR = KCH <= 4 ? 2 : 1;
    if constexpr (!STRM) lds_barrier();   // input staged
    const int kind = ph == 4 * A.n_layers ? 4 : (ph & 3);
    if (sw == 0) tr(100 + 10 * kind);
    const int K = kind == 1 ? A.H * A.hd : kind == 3 ? A.F : A.D;
    const int ra = pick5(f.ra, kind), rb = ra + pick5(f.nr, kind), r0 = pick5(f.r0, kind);
    // QKV and gate/up (inputs normalised by the control wave): the first
    // rows' slots are refilled once chunk 0 is posted.  At phase entry the
    // control wave is publishing the previous phase's output, and those
    // stores would queue behind the refills in the CU's memory path; by
    // chunk 0 its poll is over.  O and down refill at entry: their chunk 0
    // arrives while the control wave still polls the rest.
    const bool late = kind == 0 || kind == 2;
    if (ra < rb) {
        u4v xh[KCH];
        const unsigned sp = lds_addr(s_part);
        int r = ra;
        if constexpr (STRM) {   // the first rows as the input's chunks arrive
            if (r + NR <= rb) {
                float v[NR];
                consume_rows_strm<NR, KCH, FK>(f, A, P, ring, s_r, s_flag, fl, xh, K, v, late, gate);
                if (sw == 0) tr(101 + 10 * kind);
                if (lane_id() == 0)
#pragma unroll
                    for (int k = 0; k < NR; ++k) lds_write4(sp + 4u * (unsigned)(r + k - r0), v[k]);
                r += NR;
            } else {
                float v[1];
                consume_rows_strm<1, KCH, FK>(f, A, P, ring, s_r, s_flag, fl, xh, K, v, late, gate);
                if (lane_id() == 0) lds_write4(sp + 4u * (unsigned)(r - r0), v[0]);
                r += 1;
            }
        } else {   // the fp16 operand from LDS (regs_to_lds), as asm (see lds_read_wait)
            const unsigned base = lds_addr(s_r) + (unsigned)lane_id() * 16u;
            unsigned ad[KCH];
#pragma unroll
            for (int c = 0; c < KCH; ++c) ad[c] = base + (unsigned)c * 1024u;
            lds_read_wait<KCH>(xh, ad);
        }
        for (; r + NR <= rb; r += NR) {
            float v[NR];
            consume_rows<NR, KCH, FK>(f, A, P, sw, ring, xh, K, v);
            if (sw == 0 && r == ra) tr(101 + 10 * kind);
            if (lane_id() == 0)
#pragma unroll
                for (int k = 0; k < NR; ++k) lds_write4(sp + 4u * (unsigned)(r + k - r0), v[k]);
        }
        if (r < rb) {
            float v[1];
            consume_rows<1, KCH, FK>(f, A, P, sw, ring, xh, K, v);
            if (lane_id() == 0) lds_write4(sp + 4u * (unsigned)(r - r0), v[0]);
        }
    }
    if (sw == 0) tr(102 + 10 * kind);
    tail();
    lds_barrier();   // row sums complete
}

// ---- attention split on all waves of the workgroup --------------------------------------
// Workgroup b < Hk * nact owns split s of kv-head g (t = b); stream wave sw
// is attention wave sw.  Between the QKV and O phases: the control wave polls
// q and the new K/V row, writes them to LDS (s_r: [NQ][64] floats, the lane
// layout of the poll) and meets the stream waves at a barrier; each stream
// wave reduces its batches and stores its partial (s_r + NQ*64:
// [NWA][G][HD+2]); after a second barrier the control wave combines them and
// publishes the split's partial.  The stream waves fetch their first batch
// at the end of their QKV rows.
constexpr int NWA = NSW;
static_assert(NWA == ATT_WAVES, "the graph executor's attention uses the same number of waves");
struct AttnSplit {
    int pos, L, t, g, s, p0, p1, nact;
    bool open;   // INT8: the split over the open segment (fp16 staging rows)
};
template <int KVF>
__device__ __forceinline__ AttnSplit attn_split(const StepArgs& A, const PersistArgs& P, int step) {
    AttnSplit r;
    r.pos = P.pos0 + step;
    r.L = r.pos + 1;
    const SplitPlan pl = split_plan(r.L, A.S, KVF);
    r.nact = pl.nact;
    r.t = (int)blockIdx.x < A.Hk * pl.nact ? (int)blockIdx.x : -1;
    r.g = r.t / pl.nact;
    r.s = r.t % pl.nact;
    split_range(pl, r.L, r.s, r.p0, r.p1);
    r.open = KVF == KV_INT8 && r.s == pl.ncut;
    return r;
}
template <int HD, int G>
constexpr int attn_nq() { return G * 8 + 16; }
// Row pos: this step's K/V row, from the exchange (it may not be visible in
// the cache yet; the sources never fetch it under P).
// (The lane's K and V values are held by value and picked as values: a
// conditional on two array elements selects their addresses and keeps the
// arrays in scratch memory.)
struct FixNewRow {
    int pos;
    float kn[8], vn[8];
    __device__ __forceinline__ bool active(int pb, int n) const { return pb <= pos && pos < pb + n; }
    __device__ __forceinline__ void apply(int p, int which, float (&f)[8]) const {
        if (p == pos)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float k = kn[i], v = vn[i];
                f[i] = which ? v : k;
            }
    }
};
template <int HD, int G, int KVF>
__device__ __forceinline__ void attn_stream(const AttnArgs& T, const StepArgs& A, const AttnSplit& sp, int w,
                                            float* s_r, KvBuf<KVF> (&kb)[3], StreamTracer& tr) {
    constexpr int NQ = attn_nq<HD, G>();
    lds_barrier();   // q and the new row staged
    if (w == 0) tr(140);
    if (sp.t >= 0) {
        // (value k of the lane's 8 dims at s_r[k * LPR + j]: the lanes of
        // every slot read the same words, an LDS broadcast)
        constexpr int LPR = AttnGeo<HD>::LPR;
        const int j = lane_id() % LPR;
        float qv[G][8], kn[8], vn[8];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i) qv[h][i] = s_r[(h * 8 + i) * LPR + j] * (A.scale * LOG2E);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kn[i] = s_r[(G * 8 + i) * LPR + j];
            vn[i] = s_r[(G * 8 + 8 + i) * LPR + j];
        }
        AttnAcc<HD, G> acc;
        acc.clear();
        with_src<HD, KVF, true>(T, sp.g, sp.pos, sp.open, [&](auto src) {
            using Src = decltype(src);
            FixNewRow fx;
            fx.pos = sp.pos;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                fx.kn[i] = kn[i];
                fx.vn[i] = vn[i];
            }
            attn_wave_run<Src, NWA>(src, sp.p0, sp.p1, w, qv, acc, kb, fx);
        });
        if (w == 0) tr(141);
        acc.finish();
        attn_part_store<HD, G>(s_r + NQ * 64, w, acc);
    }
    lds_barrier();   // partials stored
}

template <int KD, int KA, int KF, int HD, int G, int KVF, bool FK>
__device__ __forceinline__ void stream_role(const StepArgs& A, const PersistArgs& P, int sw, unsigned char* ring,
                                            float* s_r, float* s_part, const int* s_flag, int* s_nev) {
    const Tracer ct = make_tracer(P, s_nev);
    StreamTracer tr{sw == 0 ? ct.tb : nullptr, ct.cap, 0};
    Feeder<KD, KA, KF, FK> f;
    f.start(A, P, sw, ring);
    const int NL = A.n_layers;
    auto none = [] {};
    int fl = 0;     // input chunks of the layers' GEMV phases posted so far
    int pubs = 0;   // the control wave's posted publishes (attention split, SwiGLU) so far
    for (int step = 0; step < P.n_steps; ++step) {
        const AttnSplit sp = attn_split<KVF>(A, P, step);
        for (int l = 0; l < NL; ++l) {
            const AttnArgs T = attn_args(A, l);
            KvBuf<KVF> kb[3];
            // after its QKV rows: the raw K/V rows of its first attention batch
            stream_phase<KD, KD, KA, KF, FK, true>(f, A, P, sw, ring, s_r, s_part, 4 * l, tr, [&] {
                if (sp.t >= 0)
                    with_src<HD, KVF, true>(T, sp.g, sp.pos, sp.open, [&](auto src) {
                        attn_wave_first<decltype(src), NWA>(src, sp.p0, sp.p1, sw, kb);
                    });
            }, s_flag, fl);
            fl += KD;
            attn_stream<HD, G, KVF>(T, A, sp, sw, s_r, kb, tr);
            ++pubs;
            stream_phase<KA, KD, KA, KF, FK, true>(f, A, P, sw, ring, s_r, s_part, 4 * l + 1, tr, none, s_flag, fl,
                                                   pubs);
            fl += KA;
            stream_phase<KD, KD, KA, KF, FK, true>(f, A, P, sw, ring, s_r, s_part, 4 * l + 2, tr, none, s_flag, fl);
            fl += KD;
            ++pubs;
            stream_phase<KF, KD, KA, KF, FK, true>(f, A, P, sw, ring, s_r, s_part, 4 * l + 3, tr, none, s_flag, fl,
                                                   pubs);
            fl += KF;
        }
        stream_phase<KD, KD, KA, KF, FK>(f, A, P, sw, ring, s_r, s_part, 4 * NL, tr, none);
    }
    drain_vmem();   // the trailing ring requests land before the wave ends
    if (sw == 0 && lane_id() == 0) s_nev[1] = min(tr.n, tr.cap - tr.cap / 2);
    lds_barrier();   // matches the control wave's last barrier (trace count)
}

// ---- control wave ---------------------------------------------------------------------
template <int KD, int KA, int KF, int HD, int G, int KVF, int SMAX>
__device__ __forceinline__ void control_role(const StepArgs& A, const PersistArgs& P, float* s_r,
                                             const float* s_part, float* s_own, int* s_flag, int* s_nev) {
    using Geo = AttnGeo<HD>;
    constexpr int LPR = Geo::LPR;
    const int lane = lane_id(), NL = A.n_layers, b = blockIdx.x, nwg = gridDim.x;
    Waiter wt{A.abort_word, &A.st->err, P.spin_limit, 0};
    const Tracer TR = make_tracer(P, s_nev);
    int fl = 0;   // input chunks of the layers' GEMV phases posted so far
    int pubs = 0;   // publishes posted for the stream waves (attention split, SwiGLU)
    TR(99);
    auto check_token = [&](int t) {
        if (t < 0 || t >= A.V) {
            if (b == 0 && lane == 0) atomicOr(&A.st->err, ERR_TOKEN);
            t = 0;
        }
        return t;
    };
    int tok = check_token(A.st->token[0]);
    const int Nq = A.H * HD, Nk = A.Hk * HD;
    // merge task of this workgroup: query head hm, 64 dims from part*64
    const int nmt = A.H * Geo::NPART, mstride = nwg / nmt;
    const int mt = (b % mstride == 0 && b / mstride < nmt) ? b / mstride : -1;
    const int hm = mt / Geo::NPART, mpart = mt % Geo::NPART;
    int qr0, qr1, dr0, dr1, gr0, gr1, lr0, lr1;
    {
        const PhaseGeo gq = phase_geo<KD, KA, KF>(A, P, 0), gd = phase_geo<KD, KA, KF>(A, P, 1),
                       gg = phase_geo<KD, KA, KF>(A, P, 2), gl = phase_geo<KD, KA, KF>(A, P, 4 * NL);
        qr0 = gq.r0; qr1 = gq.r1; dr0 = gd.r0; dr1 = gd.r1; gr0 = gg.r0; gr1 = gg.r1; lr0 = gl.r0; lr1 = gl.r1;
    }

    for (int step = 0; step < P.n_steps; ++step) {
        const AttnSplit sp = attn_split<KVF>(A, P, step);
        const int pos = sp.pos, L = sp.L, t = sp.t, g = sp.g, s = sp.s, p1 = sp.p1, nact = sp.nact;
        const float2* rope = A.rope + (size_t)pos * (HD / 2);
        // gains of the first RMSNorm (later ones are loaded while the wait before
        // them is pending, so that their latency hides in the wait)
        u4v gain[KD];
        load_gain<KD>(P.layer0.g_attn, A.D, gain);
        for (int l = 0; l < NL; ++l) {
            const uint32_t tag = tag_of(A, P, step, l);
            const AttnArgs T = attn_args(A, l);
            // ---------------- RMSNorm + QKV + RoPE + KV append ----------------
            {
                float xr[KD][8];
                if (l == 0) {
                    const _Float16* e = A.embed + (size_t)tok * A.D;
                    load_x_f16<KD>(e, A.D, xr);
                    for (int i = lane; i < dr1 - dr0; i += WAVE) s_own[i] = (float)e[dr0 + i];
                } else {
                    poll_vec_h2<KD>(wt, A.xb1, A.D, tag_of(A, P, step, l - 1), s_r, xr);
                }
                TR(0 + TR_RECV);
                rmsnorm_gain<KD>(xr, gain, A.D, A.eps);
                stage_chunks<KD>(s_r, xr, s_flag, fl);
                fl += KD;
            }
            TR(0 + TR_STAGED);
            // (cos, sin) of the RoPE pair each lane rotates in the epilogue,
            // loaded while the rows stream (kept for the whole step it would
            // be spilled)
            // (every lane loads one: the column is in the row for any lane)
            const float2 cs_lane = rope[rope_col(HD, A.H, qr0 + 2 * lane)];
            lds_barrier();   // row sums complete
            TR(0 + TR_DONE);
            // On the step that seals an INT8 segment the merge reads the open
            // segment, this step's row included: that row is stored before the
            // q/k/v words that lead to the merge are published.
            const bool seal_step = KVF == KV_INT8 && (pos + 1) % SEG == 0;
            for (int q = lane; 2 * q < qr1 - qr0; q += WAVE) {
                // (not `q == lane ? cs_lane : rope[..]`: a conditional on two
                // float2 lvalues selects their addresses, which puts cs_lane
                // in scratch memory)
                float2 cs = cs_lane;
                if (q != lane) cs = rope[rope_col(HD, A.H, qr0 + 2 * q)];
                const QkvPair o = qkv_pair_cs(HD, A.H, A.Hk, qr0 + 2 * q, s_part[2 * q], s_part[2 * q + 1], cs);
                if (o.kind == 0) {
                    publish(&A.qb[o.head * HD + o.d0], o.y0, tag);
                    publish(&A.qb[o.head * HD + o.d1], o.y1, tag);
                } else {
                    const int which = o.kind == 2;
                    uint64_t* dst = A.qb + Nq + which * Nk + o.head * HD;
                    const float s0 = kv_put<KVF, true>(A, l, which, o.head, pos, o.d0, o.y0);
                    const float s1 = kv_put<KVF, true>(A, l, which, o.head, pos, o.d1, o.y1);
                    if (seal_step) drain_vmem();
                    publish(&dst[o.d0], s0, tag);
                    publish(&dst[o.d1], s1, tag);
                }
            }
            TR(0 + TR_PUB);
            // ---------------- attention split (all waves) ----------------
            constexpr int NQ = attn_nq<HD, G>();
            if (t >= 0) {
                const int lane = lane_id();
                const bool has_new = p1 == L;
                // q of the group's heads, then the new K and V rows of kv-head
                // g: (G + 2) * HD words (word w: q head w / HD, or K, V), polled
                // by all 64 lanes with contiguous loads: 16 bytes per lane (load
                // i: words i*128 + 2*lane, +1, each with its own tag) where the
                // words fill whole loads, else 8 (load i: word i*64 + lane)
                constexpr int NWL = (G + 2) * HD / 64;
                static_assert((G + 2) * HD % 64 == 0, "q, K and V words in whole loads");
                auto waddr = [&](int w) {
                    return w < G * HD ? g * G * HD + w : Nq + (w / HD - G) * Nk + g * HD + w % HD;
                };
                auto widx = [&](int i) { return waddr(i * 64 + lane); };
                auto widx2 = [&](int i) { return waddr(i * 128 + 2 * lane); };
                // to the stream waves' layout: value k of lane j of a slot at
                // s_r[k * LPR + j] is dim j * 8 + k % 8 of vector k / 8 (the G
                // q heads, then K, V); every slot reads the same words
                if constexpr ((G + 2) * HD % 128 == 0) {
                    constexpr int NL2 = NWL / 2;
                    const __amdgpu_buffer_rsrc_t rs = attn_rsrc(A.qb, (size_t)(Nq + 2 * Nk) * 8);
                    u4v v2[NL2];
#pragma unroll
                    for (int i = 0; i < NL2; ++i)
                        v2[i] = i * 128 + 2 * lane < G * HD || has_new ? u4v{0u, 0u, 0u, 0u} : u4v{0u, tag, 0u, tag};
                    wt.n = 0;
                    while (true) {
#pragma unroll
                        for (int i = 0; i < NL2; ++i)
                            if (v2[i].y != tag || v2[i].w != tag)
                                v2[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)widx2(i) * 8u, 0, AUX_AGENT);
                        bool all = true;
#pragma unroll
                        for (int i = 0; i < NL2; ++i) all &= v2[i].y == tag && v2[i].w == tag;
                        if (__all(all)) break;
                        if (!wt.again()) break;
                    }
                    TR(10 + TR_RECV);
#pragma unroll
                    for (int i = 0; i < NL2; ++i)
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int w = i * 128 + 2 * lane + e, d = w % HD;
                            s_r[((w / HD) * 8 + d % 8) * LPR + d / 8] = __uint_as_float(e ? v2[i].z : v2[i].x);
                        }
                } else {
                    float wv[NWL];
                    poll_words<NWL>(wt, A.qb, widx, [&](int i) { return i * 64 + lane < G * HD || has_new; }, tag,
                                    wv);
                    TR(10 + TR_RECV);
#pragma unroll
                    for (int i = 0; i < NWL; ++i) {
                        const int w = i * 64 + lane, d = w % HD;
                        s_r[((w / HD) * 8 + d % 8) * LPR + d / 8] = wv[i];
                    }
                }
            }
            lds_barrier();   // q and the new row staged for the stream waves
            lds_barrier();   // every wave's partial stored
            if (t >= 0) {
                // the waves' partials combined and published by all 64 lanes
                // (HD / 64 dims each per head; the arithmetic of attn_combine)
                const float* sa = s_r + NQ * 64;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const AttnWaves<HD, G, NWA> aw(sa, h);
                    uint64_t* dst = A.pb + ((size_t)(g * G + h) * A.S + s) * (HD + 2);
#pragma unroll
                    for (int k = 0; k < HD / 64; ++k) publish(&dst[k * 64 + lane], aw.o(sa, h, k * 64 + lane), tag);
                    if (lane == 0) {
                        publish(&dst[HD], aw.M, tag);
                        publish(&dst[HD + 1], aw.L, tag);
                    }
                }
                TR(10 + TR_PUB);
            }
            post_count(s_flag + 1, ++pubs);   // the split's stores are issued: the O refills may follow
            // ---------------- merge of one query head ----------------
            if (mt >= 0) {
                const int lane = lane_id();
                const uint64_t* base = A.pb + (size_t)hm * A.S * (HD + 2);
                // o of splits 0..SMAX-1 at this lane's dim, then (m, l) of split `lane`
                constexpr int NM = SMAX + 2;
                float val[NM];
#pragma unroll
                for (int k = 0; k < NM; ++k) val[k] = k == SMAX ? -INFINITY : 0.f;
                auto midx = [&](int k) {
                    return k < SMAX ? k * (HD + 2) + mpart * 64 + lane : lane * (HD + 2) + HD + (k - SMAX);
                };
                poll_words<NM>(wt, base, midx, [&](int k) { return k < SMAX ? k < nact : lane < nact; }, tag, val);
                TR(20 + TR_RECV);
                float ms[MERGE_NC], ls[MERGE_NC];
#pragma unroll
                for (int c = 0; c < MERGE_NC; ++c) {
                    ms[c] = c == 0 ? val[SMAX] : -INFINITY;
                    ls[c] = c == 0 ? val[SMAX + 1] : 0.f;
                }
                const MergeW mw = merge_weights(nact, ms, ls);
                float ov[64];
#pragma unroll
                for (int k = 0; k < 64; ++k) ov[k] = k < SMAX ? val[k] : 0.f;
                float num = 0.f;
                merge_acc<SMAX>(num, 0, mw, ov);
                // dims (d, d+1) as one fp16 pair per word
                const float av = num / mw.den, av1 = __shfl_down(av, 1, WAVE);
                if ((lane & 1) == 0) publish_bits(&A.ab[(hm * HD + mpart * 64 + lane) / 2], pack_h2(av, av1), tag);
                if constexpr (KVF == KV_INT8) {
                    if ((pos + 1) % SEG == 0 && mpart == 0 && hm % G == 0) {
                        seal_head<HD, true>(T, hm / G, pos);
                        drain_vmem();
                    }
                }
                TR(20 + TR_PUB);
            }
            // ---------------- output projection + residual ----------------
            // (the input staged chunk by chunk, as for down)
            stage_stream<KA>(wt, A.ab, A.H * HD, tag, s_r, s_flag, fl);
            fl += KA;
            TR(30 + TR_RECV);
            lds_barrier();
            TR(30 + TR_DONE);
            for (int q = lane; 2 * q < dr1 - dr0; q += WAVE) {   // (dr1 - dr0) even
                const float x0 = s_own[2 * q] + s_part[2 * q], x1 = s_own[2 * q + 1] + s_part[2 * q + 1];
                s_own[2 * q] = x0;
                s_own[2 * q + 1] = x1;
                publish_bits(&A.xb2[dr0 / 2 + q], pack_h2(x0, x1), tag);
            }
            TR(30 + TR_PUB);
            load_gain<KD>(layer_w(P, P.layer0.g_ffn, l), A.D, gain);
            // ---------------- RMSNorm + gate/up + SwiGLU ----------------
            {
                float xr[KD][8];
                poll_vec_h2<KD>(wt, A.xb2, A.D, tag, s_r, xr);
                TR(40 + TR_RECV);
                rmsnorm_gain<KD>(xr, gain, A.D, A.eps);
                stage_chunks<KD>(s_r, xr, s_flag, fl);
                fl += KD;
            }
            lds_barrier();   // row sums complete
            TR(40 + TR_DONE);
            // m[i], m[i+1] as one fp16 pair per word (gr0 % 4 == 0)
            for (int q = lane; 4 * q < gr1 - gr0; q += WAVE)
                publish_bits(&A.mb[gr0 / 4 + q],
                             pack_h2(silu_mul(s_part[4 * q], s_part[4 * q + 1]),
                                     silu_mul(s_part[4 * q + 2], s_part[4 * q + 3])), tag);
            TR(40 + TR_PUB);
            post_count(s_flag + 1, ++pubs);   // the SwiGLU stores are issued: the down refills may follow
            // ---------------- down projection + residual ----------------
            // (the input staged chunk by chunk: the stream waves start on the
            // chunks that have arrived, no barrier before the rows)
            stage_stream16<KF>(wt, A.mb, A.F, tag, s_r, s_flag, fl);
            fl += KF;
            TR(50 + TR_RECV);
            lds_barrier();
            TR(50 + TR_DONE);
            // This layer's cache rows are stored (acknowledged) before the
            // residual stream that every later reader depends on is published.
            drain_vmem();
            for (int q = lane; 2 * q < dr1 - dr0; q += WAVE) {
                const float x0 = s_own[2 * q] + s_part[2 * q], x1 = s_own[2 * q + 1] + s_part[2 * q + 1];
                s_own[2 * q] = x0;
                s_own[2 * q + 1] = x1;
                publish_bits(&A.xb1[dr0 / 2 + q], pack_h2(x0, x1), tag);
            }
            TR(50 + TR_PUB);
            load_gain<KD>(l + 1 < NL ? layer_w(P, P.layer0.g_attn, l + 1) : A.g_final, A.D, gain);
        }
        // ---------------- final RMSNorm + LM head + argmax ----------------
        {
            float xr[KD][8];
            poll_vec_h2<KD>(wt, A.xb1, A.D, tag_of(A, P, step, NL - 1), s_r, xr);
            TR(60 + TR_RECV);
            rmsnorm_gain<KD>(xr, gain, A.D, A.eps);
            regs_to_lds<KD>(s_r, xr);
        }
        lds_barrier();
        lds_barrier();
        TR(60 + TR_DONE);
        const uint32_t ltag = tag12(tag_of(A, P, step, NL));
        {
            Best bst{-INFINITY, INT_MAX};
            for (int i = lane; i < lr1 - lr0; i += WAVE) {
                const float v = s_part[i];
                A.logits[lr0 + i] = v;
                if (!isfinite(v)) atomicOr(&A.st->err, ERR_NONFINITE);
                bst = better(bst, Best{v, lr0 + i});
            }
            bst = wave_best(bst);
            if (lane == 0) {
                const uint32_t ix = bst.i == INT_MAX ? 0xFFFFFu : (uint32_t)bst.i;
                st_agent(&A.lb[b], ((uint64_t)__float_as_uint(bst.v) << 32) | ((uint64_t)ix << 12) | ltag);
            }
        }
        // every workgroup reads all candidates: the next step's token
        {
            constexpr int NW = LB_MAX / WAVE;
            const int lane = lane_id();
            Best bst{-INFINITY, INT_MAX};
            bool need[NW];
#pragma unroll
            for (int k = 0; k < NW; ++k) need[k] = k * WAVE + lane < nwg;
            wt.n = 0;
            while (true) {
                uint64_t v[NW];
#pragma unroll
                for (int k = 0; k < NW; ++k)
                    if (need[k]) v[k] = ld_agent(word_at(A.lb, k * WAVE + lane));
                bool all = true;
#pragma unroll
                for (int k = 0; k < NW; ++k)
                    if (need[k]) {
                        if ((uint32_t)(v[k] & 0xFFFu) == ltag) {
                            const uint32_t ix = (uint32_t)(v[k] >> 12) & 0xFFFFFu;
                            bst = better(bst, Best{__uint_as_float((uint32_t)(v[k] >> 32)),
                                                   ix == 0xFFFFFu ? INT_MAX : (int)ix});
                            need[k] = false;
                        } else {
                            all = false;
                        }
                    }
                if (__all(all)) break;
                if (!wt.again()) break;
            }
            bst = wave_best(bst);
            tok = check_token(bst.i);
        }
        TR(60 + TR_PUB);
        if (b == 0 && lane == 0) {
            A.gen_out[P.out_base + step] = tok;
            if (step + 1 == P.n_steps) {
                A.st->token[0] = tok;
                A.st->pos = P.pos0 + P.n_steps;
                A.st->n_gen = P.out_base + P.n_steps;
            }
        }
    }
    TR(98);
    lds_barrier();   // every wave's events are recorded
    // count word: control events (lower half of the region) | stream events << 32
    if (TR.tb && lane == 0)
        TR.tb[0] = (unsigned long long)min(s_nev[0], TR.cap / 2) | ((unsigned long long)s_nev[1] << 32);
}

}  // namespace

// FK: every K (d_model, n_heads*head_dim, d_ff) is exactly its chunk count x 512.
// Both roles pass the same sequence of workgroup barriers: two per GEMV phase
// (input staged; row sums complete).
template <int KD, int KA, int KF, int HD, int G, int KVF, bool FK, int SMAX>
__global__ __launch_bounds__(PWG) void k_persist(StepArgs A, PersistArgs P) {
    constexpr int KIN = KF > KA ? (KF > KD ? KF : KD) : (KA > KD ? KA : KD);
    constexpr int NATT = attn_nq<HD, G>() * 64 + NWA * G * (HD + 2);
    constexpr int NSR = KIN * 256 > NATT ? KIN * 256 : NATT;   // fp16 GEMV operand: KIN KiB
    __shared__ __attribute__((aligned(16))) unsigned char s_ring[NSW * RING * UNIT];
    // the phase's GEMV input; between the QKV and O phases the attention exchange
    __shared__ __attribute__((aligned(16))) float s_r[NSR];
    __shared__ float s_part[PART_MAX];                             // row sums of the phase
    __shared__ float s_own[OWN_MAX];                               // owned rows of the residual stream
    __shared__ int s_nev[2];                                       // trace events: control, stream
    __shared__ int s_flag[2];   // GEMV input chunks posted; the control wave's publishes (attention, SwiGLU)
    const int wid = wave_id();
    if (threadIdx.x < 2) s_nev[threadIdx.x] = 0;
    if (threadIdx.x < 2) s_flag[threadIdx.x] = 0;
    lds_barrier();
    if (wid == 0)
        control_role<KD, KA, KF, HD, G, KVF, SMAX>(A, P, s_r, s_part, s_own, s_flag, s_nev);
    else
        stream_role<KD, KA, KF, HD, G, KVF, FK>(A, P, wid - 1, s_ring + (wid - 1) * RING * UNIT, s_r, s_part,
                                                s_flag, s_nev);
}

// ---- host side ------------------------------------------------------------------------
namespace {
struct Shape {
    int KD, KA, KF, HD, G;
};
// Most key splits per kv-head each instantiation merges (the default split
// count is CUs / n_kv_heads, at most 64).
// Instantiated shapes: the 2B-class model, the 1-layer tiny model, and a
// small GQA model used by the tests.
constexpr Shape kShapes[] = {{4, 4, 11, 128, 2}, {1, 1, 2, 64, 1}, {1, 1, 4, 64, 4}};

Shape shape_of(const StepArgs& A) {
    return Shape{kch_for(A.D), kch_for(A.H * A.hd), kch_for(A.F), A.hd, A.H / A.Hk};
}
bool same(const Shape& a, const Shape& b) {
    return a.KD == b.KD && a.KA == b.KA && a.KF == b.KF && a.HD == b.HD && a.G == b.G;
}

template <int KD, int KA, int KF, int HD, int G, bool FK, int SMAX>
const void* kernel_for_fmt(int kvfmt) {
    switch (kvfmt) {
        case KV_FP16: return (const void*)&k_persist<KD, KA, KF, HD, G, KV_FP16, FK, SMAX>;
        case KV_E5M2: return (const void*)&k_persist<KD, KA, KF, HD, G, KV_E5M2, FK, SMAX>;
        case KV_INT8: return (const void*)&k_persist<KD, KA, KF, HD, G, KV_INT8, FK, SMAX>;
    }
    return nullptr;
}

const void* kernel_for(const StepArgs& A, int* smax) {
    const Shape s = shape_of(A);
    const bool full = A.D == s.KD * 512 && A.H * A.hd == s.KA * 512 && A.F == s.KF * 512;
    if (same(s, kShapes[0]) && full) { *smax = 32; return kernel_for_fmt<4, 4, 11, 128, 2, true, 32>(A.kvfmt); }
    if (same(s, kShapes[1])) { *smax = 64; return kernel_for_fmt<1, 1, 2, 64, 1, false, 64>(A.kvfmt); }
    if (same(s, kShapes[2])) { *smax = 64; return kernel_for_fmt<1, 1, 4, 64, 4, false, 64>(A.kvfmt); }
    return nullptr;
}

// Most rows one workgroup reduces in a phase when the rows are dealt to nwg
// workgroups in tasks of rpt.
int rows_per_wg(int N, int rpt, int nwg) { return ((N / rpt + nwg - 1) / nwg) * rpt; }
}  // namespace

bool persistent_supported(const StepArgs& A) {
    int smax = 0;
    return kernel_for(A, &smax) != nullptr && A.S <= smax;
}

hipError_t persistent_max_grid(const StepArgs& A, int device, int* nwg) {
    int smax = 0;
    const void* k = kernel_for(A, &smax);
    if (!k || A.S > smax) return hipErrorInvalidValue;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) return e;
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, PWG, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    const int n = prop.multiProcessorCount;   // one workgroup per CU
    const int most = std::max(std::max(rows_per_wg((A.H + 2 * A.Hk) * A.hd, 2, n), rows_per_wg(2 * A.F, 2, n)),
                              std::max(rows_per_wg(A.D, 1, n), rows_per_wg(A.V, 1, n)));
    // every attention task and merge task needs a workgroup of its own
    const int ntask = A.Hk * A.S, nmerge = A.H * (A.hd / 64);
    // past its last row each stream wave keeps requesting the LM head from
    // its first byte (up to RING chunks, plus a partial row): it must be that long
    const bool lm_short = (size_t)A.V * A.D * 2 < (size_t)RING * UNIT + (size_t)A.D * 2;
    if (most > PART_MAX || rows_per_wg(A.D, 1, n) > OWN_MAX || n > LB_MAX || ntask > n || nmerge > n ||
        A.V >= (1 << 20) || lm_short)
        return hipErrorInvalidConfiguration;
    *nwg = n;
    return hipSuccess;
}

hipError_t launch_persistent(const StepArgs& A, const PersistArgs& P, int nwg, hipStream_t s) {
    int smax = 0;
    const void* k = kernel_for(A, &smax);
    if (!k || A.S > smax) return hipErrorInvalidValue;
    if (P.n_steps < 1) return hipErrorInvalidValue;
    StepArgs a = A;
    PersistArgs p = P;
    void* args[] = {&a, &p};
    return hipLaunchCooperativeKernel(k, dim3(nwg), dim3(PWG), args, 0, s);
}

}  // namespace rd
