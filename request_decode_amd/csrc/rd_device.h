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
// Butterfly over the 64 lanes: every lane ends with the full result.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}
// Sum over aligned groups of `n` lanes (n a power of two <= 64).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = N / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
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

// ---- cross-workgroup exchange inside one kernel --------------------------------
// The L2 is per XCD, so data one workgroup hands to another must not sit in
// a non-coherent L2 line.  An agent-scope release/acquire fence would write
// back and invalidate the whole L2 of the XCD (buffer_wbl2 / buffer_inv),
// far too costly once per workgroup.  Instead the exchanged words are
// written and read with agent-scope (sc1) relaxed atomic stores and loads,
// which are coherent across XCDs on their own; the only ordering needed is
// that a workgroup's stores have completed (vmcnt drained) before its
// arrival is counted, and that the reader's loads are issued after it saw
// the final count.
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_agent(const int* p) {
    return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's outstanding vector-memory operations completed.
__device__ __forceinline__ void drain_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Count this workgroup's arrival on *cnt after all of its threads' st_agent
// stores completed; true in every thread of the workgroup that arrives
// last of `expected`.  The last one resets the counter for the next use
// (which must come after a kernel boundary).
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
