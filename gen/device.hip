// Device twin of the counter-based input generator (gen/host.py): fills HBM
// buffers with the same bits the host computes for the same (key, index).
// Input generation only; nothing here belongs to the collectives.
//
//   mix64     SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014)
//   U64(i,m)  mix64(key + (4*i + m) * 0x9E3779B97F4A7C15)
//   uniform   ((U64(i,0) >> 40) - 2^23) * 2^-23
//   normal    (sum_{m<4} (U64(i,m) >> 32) * 2^-32 - 2) * scale, scale = sqrt(3)*sigma
//             computed on the host; double -> fp32 conversion; bf16 = top 16 bits
//   int32     top 32 bits of U64(i,0)

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t u64(uint64_t key, uint64_t i, uint64_t m) {
  return mix64(key + (4 * i + m) * kGolden);
}

__device__ __forceinline__ float normal_f32(uint64_t key, uint64_t i, double scale) {
  uint64_t s = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) s += u64(key, i, m) >> 32;
  const double z = static_cast<double>(s) * 0x1p-32 - 2.0;
  return static_cast<float>(z * scale);
}

__global__ void uniform_f32_kernel(float* out, uint64_t n, uint64_t key, uint64_t base) {
  for (uint64_t k = blockIdx.x * static_cast<uint64_t>(blockDim.x) + threadIdx.x; k < n;
       k += static_cast<uint64_t>(gridDim.x) * blockDim.x) {
    const int64_t top = static_cast<int64_t>(u64(key, base + k, 0) >> 40);
    out[k] = static_cast<float>(static_cast<double>(top - (int64_t(1) << 23)) * 0x1p-23);
  }
}

__global__ void normal_bf16_kernel(uint16_t* out, uint64_t n, uint64_t key, uint64_t base, double scale) {
  for (uint64_t k = blockIdx.x * static_cast<uint64_t>(blockDim.x) + threadIdx.x; k < n;
       k += static_cast<uint64_t>(gridDim.x) * blockDim.x) {
    out[k] = static_cast<uint16_t>(__float_as_uint(normal_f32(key, base + k, scale)) >> 16);
  }
}

__global__ void normal_f32_kernel(float* out, uint64_t n, uint64_t key, uint64_t base, double scale) {
  for (uint64_t k = blockIdx.x * static_cast<uint64_t>(blockDim.x) + threadIdx.x; k < n;
       k += static_cast<uint64_t>(gridDim.x) * blockDim.x) {
    out[k] = normal_f32(key, base + k, scale);
  }
}

__global__ void int32_kernel(int32_t* out, uint64_t n, uint64_t key, uint64_t base) {
  for (uint64_t k = blockIdx.x * static_cast<uint64_t>(blockDim.x) + threadIdx.x; k < n;
       k += static_cast<uint64_t>(gridDim.x) * blockDim.x) {
    out[k] = static_cast<int32_t>(static_cast<uint32_t>(u64(key, base + k, 0) >> 32));
  }
}

// Row r of the output holds token tokens[r]'s hidden vector:
// element (r, h) = normal(key, tokens[r] * hidden + h).
__global__ void normal_bf16_rows_kernel(uint16_t* out, const int32_t* tokens, uint64_t nrows, uint64_t hidden,
                                        uint64_t key, double scale) {
  const uint64_t n = nrows * hidden;
  for (uint64_t k = blockIdx.x * static_cast<uint64_t>(blockDim.x) + threadIdx.x; k < n;
       k += static_cast<uint64_t>(gridDim.x) * blockDim.x) {
    const uint64_t r = k / hidden;
    const uint64_t h = k - r * hidden;
    const uint64_t idx = static_cast<uint64_t>(tokens[r]) * hidden + h;
    out[k] = static_cast<uint16_t>(__float_as_uint(normal_f32(key, idx, scale)) >> 16);
  }
}

unsigned grid_for(uint64_t n) {
  const uint64_t blocks = (n + 255) / 256;
  return static_cast<unsigned>(blocks < 16384 ? (blocks ? blocks : 1) : 16384);
}

int done(hipError_t e) { return e == hipSuccess ? 0 : static_cast<int>(e); }

}  // namespace

extern "C" {

int gcgen_uniform_f32(float* out, uint64_t n, uint64_t key, uint64_t base, hipStream_t s) {
  if (!n) return 0;
  hipLaunchKernelGGL(uniform_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, out, n, key, base);
  return done(hipGetLastError());
}

int gcgen_normal_bf16(uint16_t* out, uint64_t n, uint64_t key, uint64_t base, double scale, hipStream_t s) {
  if (!n) return 0;
  hipLaunchKernelGGL(normal_bf16_kernel, dim3(grid_for(n)), dim3(256), 0, s, out, n, key, base, scale);
  return done(hipGetLastError());
}

int gcgen_normal_f32(float* out, uint64_t n, uint64_t key, uint64_t base, double scale, hipStream_t s) {
  if (!n) return 0;
  hipLaunchKernelGGL(normal_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, out, n, key, base, scale);
  return done(hipGetLastError());
}

int gcgen_int32(int32_t* out, uint64_t n, uint64_t key, uint64_t base, hipStream_t s) {
  if (!n) return 0;
  hipLaunchKernelGGL(int32_kernel, dim3(grid_for(n)), dim3(256), 0, s, out, n, key, base);
  return done(hipGetLastError());
}

int gcgen_normal_bf16_rows(uint16_t* out, const int32_t* tokens, uint64_t nrows, uint64_t hidden, uint64_t key,
                           double scale, hipStream_t s) {
  if (!nrows || !hidden) return 0;
  hipLaunchKernelGGL(normal_bf16_rows_kernel, dim3(grid_for(nrows * hidden)), dim3(256), 0, s, out, tokens, nrows,
                     hidden, key, scale);
  return done(hipGetLastError());
}

}  // extern "C"
