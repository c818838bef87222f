// Device helpers shared by the reduction kernels: unpack a 16-byte vector
// into reduction-type values, fold N ranks' vectors in a given rank order
// (all loads of a batch issued before the first add), and pack / store the
// results in the output type.
#pragma once

#include "device_common.h"

namespace gcdev {

template <class In>
__device__ __forceinline__ void unpack(const u32x4& v, typename In::Acc (&x)[In::VE]);

template <>
__device__ __forceinline__ void unpack<InBf16>(const u32x4& v, float (&x)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(v[k] << 16);
    x[2 * k + 1] = __uint_as_float(v[k] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void unpack<InF32>(const u32x4& v, float (&x)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(v[k]);
}
template <>
__device__ __forceinline__ void unpack<InI32>(const u32x4& v, uint32_t (&x)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) x[k] = v[k];
}

// Packed result words of VE elements of the output type.
template <class Out, int VE>
struct Words {
  static constexpr int NW = VE * Out::ES / 4;
  uint32_t w[NW];
};

template <class Out, int VE, class Acc>
__device__ __forceinline__ Words<Out, VE> pack(const Acc (&x)[VE]) {
  Words<Out, VE> r;
  if constexpr (Out::ES == 2) {
#pragma unroll
    for (int k = 0; k < VE / 2; ++k) r.w[k] = bf16_bits(x[2 * k]) | (bf16_bits(x[2 * k + 1]) << 16);
  } else if constexpr (sizeof(Acc) == 4 && __is_same(Acc, float)) {
#pragma unroll
    for (int k = 0; k < VE; ++k) r.w[k] = __float_as_uint(x[k]);
  } else {
#pragma unroll
    for (int k = 0; k < VE; ++k) r.w[k] = x[k];
  }
  return r;
}

template <class Out, int VE, int POL = gci::kStoreNT>
__device__ __forceinline__ void put(char* p, const Words<Out, VE>& r) {
  constexpr int NW = Words<Out, VE>::NW;
  if constexpr (NW == 2) {
    st8(p, u32x2{r.w[0], r.w[1]});
  } else {
#pragma unroll
    for (int h = 0; h < NW / 4; ++h)
      st16p<POL>(p + 16 * h, u32x4{r.w[4 * h], r.w[4 * h + 1], r.w[4 * h + 2], r.w[4 * h + 3]});
  }
}

// Results of 32 bytes per lane (eight fp32 from eight bf16 inputs) regrouped
// so that each of a wavefront's two store instructions writes 1 KiB
// contiguously.  Lane l holds vector vw + l of the wavefront (vw its first);
// half h of the result, for lane l, is half (l & 1) of vector vw + 32 h + l/2,
// fetched from that lane with ds_bpermute, and goes to byte 1024 h + 16 l of
// the wavefront's 2 KiB.  Stored per lane as two 16-byte halves of its own
// 32 bytes, each instruction wrote every other 16 bytes: lines then left L2
// half written and were written back twice (14 % more write traffic).  Every
// lane of the wavefront must execute this (cross-lane reads).
template <class Out, int VE>
__device__ __forceinline__ void wave_halves32(const Words<Out, VE>& w, u32x4& h0, u32x4& h1) {
  static_assert(Words<Out, VE>::NW == 8, "32-byte results per lane");
  const uint32_t lane = threadIdx.x & 63;
  u32x4 h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int src = static_cast<int>((32 * half + (lane >> 1)) << 2);
    uint32_t x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      x[k] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src, static_cast<int>(w.w[k])));
    h[half] = (lane & 1) ? u32x4{x[4], x[5], x[6], x[7]} : u32x4{x[0], x[1], x[2], x[3]};
  }
  h0 = h[0];
  h1 = h[1];
}

__device__ __forceinline__ uint32_t next_rank(uint32_t r, uint32_t N) { return r + 1 == N ? 0 : r + 1; }

// A partial as the ring forwards it when WIRE is set: rounded to the input's
// storage type (bf16, round to nearest even) before the next rank adds its
// term (DTLM §11: low-precision communication, fp32 arithmetic).  Identity for
// fp32 and int32 data and when WIRE is clear.
template <class In, bool WIRE>
__device__ __forceinline__ typename In::Acc on_wire(typename In::Acc x) {
  if constexpr (WIRE && In::ES == 2) return __uint_as_float(bf16_bits(x) << 16);
  else return x;
}

// `in` points at the N rank pointers (kernel arguments; wavefront-uniform).
// base: index of rank 0 of the folded set in `in` (a group of a larger mesh).
template <class In, bool WIRE = false>
__device__ __forceinline__ typename In::Acc fold_one(const char* const* in, uint32_t first, uint32_t N, uint64_t E,
                                                     uint32_t base = 0) {
  typename In::Acc acc = In::one(in[base + first], E);
  uint32_t r = first;
  for (uint32_t k = 1; k < N; ++k) {
    r = next_rank(r, N);
    acc = on_wire<In, WIRE>(acc) + In::one(in[base + r], E);
  }
  return acc;
}

template <class Out, class Acc>
__device__ __forceinline__ void put_one(char* base, uint64_t e, Acc x) {
  if constexpr (Out::ES == 2) {
    reinterpret_cast<uint16_t*>(base)[e] = static_cast<uint16_t>(bf16_bits(x));
  } else {
    reinterpret_cast<Acc*>(base)[e] = x;
  }
}

// Loads KB ranks' vectors (ranks r, r+1, ... mod N) for the U byte offsets,
// all issued before the first add, then folds them into acc in that order.
// FIRST: the batch starts the fold (acc takes the first rank's values).
template <class In, int KB, int U, bool FIRST, bool WIRE = false>
__device__ __forceinline__ void fold_batch(const char* const* in, uint32_t& r, uint32_t N, const uint64_t (&off)[U],
                                           typename In::Acc (&acc)[U][In::VE], uint32_t rank0 = 0) {
  constexpr int VE = In::VE;
  typedef typename In::Acc Acc;
  u32x4 raw[KB][U];
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    const char* base = in[rank0 + r];
#pragma unroll
    for (int u = 0; u < U; ++u) raw[k][u] = ld16(base + off[u]);
    r = next_rank(r, N);
  }
#pragma unroll
  for (int k = 0; k < KB; ++k) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Acc x[VE];
      unpack<In>(raw[k][u], x);
      if (FIRST && k == 0) {
#pragma unroll
        for (int l = 0; l < VE; ++l) acc[u][l] = x[l];
      } else {
#pragma unroll
        for (int l = 0; l < VE; ++l) acc[u][l] = on_wire<In, WIRE>(acc[u][l]) + x[l];
      }
    }
  }
}

// The remaining n (1..7) ranks of a runtime-N fold, as one batch.
template <class In, int U, bool FIRST, bool WIRE = false>
__device__ __forceinline__ void fold_rest(const char* const* in, uint32_t& r, uint32_t N, uint32_t n,
                                          const uint64_t (&off)[U], typename In::Acc (&acc)[U][In::VE],
                                          uint32_t rank0 = 0) {
  switch (n) {
    case 1: fold_batch<In, 1, U, FIRST, WIRE>(in, r, N, off, acc, rank0); break;
    case 2: fold_batch<In, 2, U, FIRST, WIRE>(in, r, N, off, acc, rank0); break;
    case 3: fold_batch<In, 3, U, FIRST, WIRE>(in, r, N, off, acc, rank0); break;
    case 4: fold_batch<In, 4, U, FIRST, WIRE>(in, r, N, off, acc, rank0); break;
    case 5: fold_batch<In, 5, U, FIRST, WIRE>(in, r, N, off, acc, rank0); break;
    case 6: fold_batch<In, 6, U, FIRST, WIRE>(in, r, N, off, acc, rank0); break;
    case 7: fold_batch<In, 7, U, FIRST, WIRE>(in, r, N, off, acc, rank0); break;
    default: break;
  }
}

// Full fold of U vectors at byte offsets `off` over the N ranks in order
// first, first+1, ... (mod N).  NF > 0: N fixed at compile time.  WIRE: every
// partial is rounded as the ring forwards it before the next term is added.
// rank0: index in `in` of the folded set's rank 0 (a group of a larger mesh).
template <class In, int NF, int U, bool WIRE = false>
__device__ __forceinline__ void fold_vec(const char* const* in, uint32_t first, uint32_t N, const uint64_t (&off)[U],
                                         typename In::Acc (&acc)[U][In::VE], uint32_t rank0 = 0) {
  uint32_t r = first;
  if constexpr (NF > 0) {
    fold_batch<In, NF, U, true, WIRE>(in, r, NF, off, acc, rank0);
  } else if (N >= 8) {
    fold_batch<In, 8, U, true, WIRE>(in, r, N, off, acc, rank0);
    uint32_t k0 = 8;
    for (; k0 + 8 <= N; k0 += 8) fold_batch<In, 8, U, false, WIRE>(in, r, N, off, acc, rank0);
    fold_rest<In, U, false, WIRE>(in, r, N, N - k0, off, acc, rank0);
  } else {
    fold_rest<In, U, true, WIRE>(in, r, N, N, off, acc, rank0);
  }
}

}  // namespace gcdev
