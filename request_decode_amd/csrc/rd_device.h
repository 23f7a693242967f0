// Device helpers shared by the decode-step kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rd {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// The wave's index in its workgroup as a wave-uniform (scalar) value, so that
// addresses derived from it stay in scalar registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
// The lane index, passed through an empty asm so that values derived from it
// are computed where they are used: in a long persistent loop the compiler
// would otherwise hoist every lane-dependent address out of the loop and keep
// it live across the whole body, spilling registers.
__device__ __forceinline__ int lane_id() {
    int l = (int)(threadIdx.x & 63);
    asm volatile("" : "+v"(l));
    return l;
}

// ---- loads ----------------------------------------------------------------
// Weights are read exactly once per step and never reused inside it, so they
// are fetched with the non-temporal hint (no point keeping them in L2/MALL).
__device__ __forceinline__ u4v ld_w16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
}
__device__ __forceinline__ u4v ld16(const void* p) { return *reinterpret_cast<const u4v*>(p); }
__device__ __forceinline__ u2v ld8(const void* p) { return *reinterpret_cast<const u2v*>(p); }

__device__ __forceinline__ h8 as_h8(u4v u) { return __builtin_bit_cast(h8, u); }

// ---- wave reductions ----------------------------------------------------------
// DPP lane exchange (no LDS round trip, unlike a ds_bpermute shuffle):
// 0xB1 / 0x4E swap neighbours / pairs inside each quad, 0x124 / 0x128 rotate
// a row of 16 lanes by 4 / 8, 0x141 mirrors each half-row of 8 lanes, 0x150
// broadcasts lane 0 of each row to the whole row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// Sum of each row of 16 lanes, valid in lane 0 of the row (the other lanes
// hold the same terms associated differently).
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x124>(v);
    v += dpp_f<0x128>(v);
    return v;
}
// Sum over the 64 lanes: one association order, the same value in every lane.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    return ((readlane_f(v, 0) + readlane_f(v, 16)) + readlane_f(v, 32)) + readlane_f(v, 48);
}
// Sum over aligned groups of N lanes (N = 8 or 16), the same bits in every
// lane of a group.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
    if constexpr (N == 16) {
        return dpp_f<0x150>(row16_sum(v));
    } else {
        v += dpp_f<0xB1>(v);
        v += dpp_f<0x4E>(v);
        return v + dpp_f<0x141>(v);
    }
}
// gfx950 lane swaps between rows: swap16 pairs row 2k with row 2k+1 (lanes
// l and l ^ 16), swap32 the two halves (lanes l and l ^ 32); each returns
// the pair (first: the even row's / lower half's value, second: the other)
// in every lane of the pair, a VALU operation with no LDS round trip.
__device__ __forceinline__ float swap16_sum(float v) {
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float swap32_sum(float v) {
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
// Row 0's value (lanes 0..15) in the same lane of every row.
__device__ __forceinline__ float row0_bcast(float v) {
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const auto r = __builtin_amdgcn_permlane32_swap(q[0], q[0], false, false);
    return __uint_as_float(r[0]);
}
// Maximum over the 64 lanes, in every lane: row maxima by DPP, then the
// row pairs and halves by lane swaps.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x128>(v));
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, WAVE));
    return v;
}

// ---- number formats -----------------------------------------------------------
// fp16 -> E5M2: E5M2 is the upper byte of an fp16 with the low 8 fraction bits
// dropped.  Round to nearest even on those 8 bits by adding 0x7F plus the bit
// that becomes the new LSB, then shifting; a carry out of the fraction moves
// into the exponent, and past the largest finite value it lands on the
// infinity pattern (no saturation).  Every NaN becomes the quiet NaN 0x7E
// with its sign.
__device__ __forceinline__ uint8_t e5m2_encode(uint16_t h) {
    if ((h & 0x7c00u) == 0x7c00u && (h & 0x03ffu)) return (uint8_t)(((h >> 8) & 0x80u) | 0x7eu);
    unsigned r = (unsigned)h + 0x7fu + ((h >> 8) & 1u);
    return (uint8_t)(r >> 8);
}
// E5M2 -> fp16 is exact: the byte becomes the high byte of the fp16 pattern.
__device__ __forceinline__ _Float16 e5m2_decode(uint8_t e) {
    return __builtin_bit_cast(_Float16, (uint16_t)((uint16_t)e << 8));
}
__device__ __forceinline__ uint16_t f2h_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float h_bits2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// ---- cross-workgroup exchange inside one kernel --------------------------------
// The L2 is per XCD, so data one workgroup hands to another must not sit in
// a non-coherent L2 line.  An agent-scope release/acquire fence would write
// back and invalidate the whole L2 of the XCD, far too costly per exchange.
// Instead the exchanged words are written and read with agent-scope (sc1)
// relaxed atomic stores and loads, which are coherent across XCDs on their
// own.
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_agent(const int* p) {
    return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's outstanding vector-memory operations completed
// (loads returned, stores acknowledged at the coherence point).
__device__ __forceinline__ void drain_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order, so every older one is done).
// A real s_waitcnt the compiler sees and accounts for: where its own count
// is lost (loads behind a loop of unknown trip count) it would otherwise
// wait for all of them.  vmcnt is 6 bits on gfx9: bits 3:0 and 15:14;
// expcnt (6:4) and lgkmcnt (11:8) at their maxima do not wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Count this workgroup's arrival on *cnt after all of its threads' stores
// completed; true in every thread of the workgroup that arrives last of
// `expected`.  The last one resets the counter for the next use (which must
// come after a kernel boundary).
__device__ __forceinline__ bool arrive_last(int* cnt, int expected) {
    __shared__ int s_last;
    drain_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == expected - 1);
        if (s_last) st_agent(cnt, 0);
    }
    __syncthreads();
    return s_last != 0;
}

}  // namespace rd
