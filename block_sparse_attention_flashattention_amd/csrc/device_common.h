// Device-side helpers shared by the forward kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vsa_internal.h"

namespace vsa {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLn2 = 0.6931471805599453f;
// A stale row max is kept while a tile's max exceeds it by at most this many
// powers of two, so un-normalised probabilities stay <= 2^8 (exact in math;
// the final division by the row sum uses the same stale max).
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats -> two bf16 (round to nearest even) in one 32-bit word.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Value of x held by lane (l ^ 32), combined with x: returns op(x, other).
__device__ __forceinline__ float halfwave_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS barrier across the workgroup: waits for this wave's LDS operations and
// keeps the compiler from moving memory accesses across it. Outstanding
// global loads (including loads into LDS) are NOT waited for.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// 16-byte direct-to-LDS load: lane l reads 16 bytes at base + voff and writes
// them to LDS byte address lds + 16*l (lds and base wave-uniform). Issued
// through inline asm so that the compiler's conservative wait on later LDS
// reads of other buffers is not inserted; completion is awaited explicitly
// with wait_global_loads() before the barrier that publishes the data.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds) {
    // both operands are uniform; pin them to scalar registers
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    base = (const void*)(uintptr_t)(((uint64_t)bhi << 32) | blo);
    lds = __builtin_amdgcn_readfirstlane(lds);
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(base), "s"(lds)
        : "memory", "m0");
}
// A wave-uniform pointer pinned to scalar registers, so that address
// arithmetic on it stays on the scalar unit.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
    const uint64_t b = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// A CSR entry as staged in LDS: -1 for an index outside [0, nkv), else the
// tile index with the number of invalid keys of the tile (block_kv minus its
// clamped valid count; 0 without valid counts) in the bits above kTileBits.
// Kernels built without partial tiles (PARTIAL = false) stage the raw index
// and treat every in-range tile as full.
template <bool PARTIAL>
__device__ __forceinline__ int stage_entry(int t, int nkv, int block_kv, const int32_t* kv_valid) {
    if (t < 0 || t >= nkv) return -1;
    if constexpr (!PARTIAL) return t;
    const int nv = kv_valid[t];
    const int invalid = nv < 0 ? block_kv : (nv > block_kv ? 0 : block_kv - nv);
    return t | (invalid << kTileBits);
}
template <bool PARTIAL>
__device__ __forceinline__ int entry_tile(int e) {
    if constexpr (!PARTIAL) return e;
    return e < 0 ? -1 : (e & (kMaxTilesPartial - 1));
}
// valid keys of a staged entry's tile (0 for an out-of-range entry)
template <bool PARTIAL>
__device__ __forceinline__ int entry_keys(int e, int block_kv) {
    if constexpr (!PARTIAL) return e < 0 ? 0 : block_kv;
    return e < 0 ? 0 : block_kv - (e >> kTileBits);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

// Wait for every outstanding global load of this wave (data landed in LDS).
__device__ __forceinline__ void wait_global_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs. Map
// them so each XCD takes a contiguous run of [0, gridDim.x) instead: the
// work-list entries it processes concurrently then share K/V tiles in its own
// L2. A bijection for any grid size.
__device__ __forceinline__ int xcd_contiguous_block() {
    const int nwg = gridDim.x, xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int per = nwg / 8, rem = nwg % 8;
    return (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

}  // namespace dev
}  // namespace vsa
