// Device-side helpers for the gfx950 kernels: 16-byte non-temporal vector
// access, element unpack/pack for the three supported types, and the
// averaging epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gc_internal.h"

namespace gcdev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#ifndef GC_THREADS
#define GC_THREADS 256
#endif
constexpr int kThreads = GC_THREADS;  // 64-wide wavefronts per workgroup: kThreads / 64

// Build-time tuning knobs (defaults are the measured best on MI355X).
#ifndef GC_NT_LOAD
#define GC_NT_LOAD 1
#endif
#ifndef GC_NT_STORE
#define GC_NT_STORE 1
#endif

// Streaming data is touched exactly once per launch, so loads and stores carry
// the non-temporal hint: they should not displace other data in L2 / MALL.
__device__ __forceinline__ u32x4 ld16(const void* p) {
#if GC_NT_LOAD
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
#if GC_NT_STORE
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
#else
  *reinterpret_cast<u32x4*>(p) = v;
#endif
}
__device__ __forceinline__ void st8(void* p, u32x2 v) {
#if GC_NT_STORE
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
#else
  *reinterpret_cast<u32x2*>(p) = v;
#endif
}

// 16-byte store with a cache policy (gci::StorePolicy).  Device scope has no
// builtin for a 16-byte store, so those two are inline assembly.  A VALU write
// to the data registers of a store wider than 8 bytes needs two wait states
// after the store on this architecture; the compiler inserts them after its own
// stores but cannot after an asm statement, hence the s_nop (two wait states).
template <int POL>
__device__ __forceinline__ void st16p(void* p, u32x4 v) {
  if constexpr (POL == gci::kStoreDevNT) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
  } else if constexpr (POL == gci::kStoreDev) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
  } else {
    st16(p, v);
  }
}

// Vector u (0..U-1) of this thread within a tile of kThreads * U vectors that
// starts at vector tv0.  WAVE = true: each wavefront covers its U * 64 vectors
// contiguously (a wavefront's U load instructions per rank read one run of
// U KiB); false: the workgroup covers kThreads consecutive vectors per u (each
// instruction reads 1 KiB, the U of them kThreads * 16 bytes apart).
template <int U, bool WAVE>
__device__ __forceinline__ uint64_t tile_vec(uint64_t tv0, int u) {
  if constexpr (WAVE) return tv0 + (threadIdx.x >> 6) * (64 * U) + u * 64 + (threadIdx.x & 63);
  else return tv0 + u * kThreads + threadIdx.x;
}

// ---------------------------------------------------------------- inputs
// In::VE elements fill one 16-byte vector; In::Acc is the reduction type
// (fp32 for bf16 / fp32 data, uint32 with wrap-around for int32 data).

struct InBf16 {
  static constexpr int VE = 8;
  static constexpr int ES = 2;
  typedef float Acc;
  __device__ static __forceinline__ float one(const void* base, uint64_t e) {
    const uint16_t b = reinterpret_cast<const uint16_t*>(base)[e];
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
};

struct InF32 {
  static constexpr int VE = 4;
  static constexpr int ES = 4;
  typedef float Acc;
  __device__ static __forceinline__ float one(const void* base, uint64_t e) {
    return reinterpret_cast<const float*>(base)[e];
  }
};

struct InI32 {
  static constexpr int VE = 4;
  static constexpr int ES = 4;
  typedef uint32_t Acc;
  __device__ static __forceinline__ uint32_t one(const void* base, uint64_t e) {
    return reinterpret_cast<const uint32_t*>(base)[e];
  }
};

// ---------------------------------------------------------------- epilogue
// Average: one correctly rounded fp32 division by N.  Integers never average.
__device__ __forceinline__ float finish(float x, bool avg, float n) { return avg ? __fdiv_rn(x, n) : x; }
__device__ __forceinline__ uint32_t finish(uint32_t x, bool, float) { return x; }

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x)));
}

// ---------------------------------------------------------------- outputs
// Element size of each output type, and the bytes one vector of VE results
// occupies (the store width the output alignment is checked against).

struct OutBf16 {
  static constexpr int ES = 2;
  static constexpr int vec_bytes(int VE) { return 2 * VE; }
};

struct OutF32 {
  static constexpr int ES = 4;
  static constexpr int vec_bytes(int VE) { return 4 * VE; }
};

struct OutI32 {
  static constexpr int ES = 4;
  static constexpr int vec_bytes(int VE) { return 4 * VE; }
};

}  // namespace gcdev
