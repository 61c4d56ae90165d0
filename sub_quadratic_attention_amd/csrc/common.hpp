// Shared device helpers of the thin-attention HIP library (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace thin {

// A kernel launch that, given an event, has its own dispatch signal that
// event on completion (hipExtLaunchKernelGGL's stop event) instead of a
// separate marker in the stream's queue.
template <typename F, typename... Args>
inline void launch_signal(F kernel, const dim3& grid, const dim3& block, uint32_t lds, hipStream_t s,
                          hipEvent_t done, Args... args) {
  if (done)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, nullptr, done, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}


typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(double)))) double f64x4_t;

// ---------------------------------------------------------------------------
// Input element access.  Inputs are float32, bfloat16 (raw 16-bit patterns) or
// OCP FP8 E4M3 (E4M3FN: 1 sign, 4 exponent bits of bias 7, 3 mantissa bits,
// no infinities; raw bytes).
// ---------------------------------------------------------------------------
enum : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };   // element types, as the C ABI numbers them

template <int ET>
constexpr int elt_size() { return ET == kF32 ? 4 : (ET == kBF16 ? 2 : 1); }

// The low byte of `word` as an E4M3 value, widened exactly (gfx950 converts
// the OCP format).
__device__ __forceinline__ float fp8_low_to_float(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 0);
}

// Byte b (0..3) of `word` as an E4M3 value.
__device__ __forceinline__ float fp8_byte_to_float(uint32_t word, int b) { return fp8_low_to_float(word >> (8 * b)); }

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (NaN kept quiet).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11).  Counter words
// (c0, c1, c2, c3), key (seed, 0).  One round maps (x0, x1, x2, x3) to
// (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)); the key
// is then bumped by the Weyl increments.
// ---------------------------------------------------------------------------
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

__device__ __forceinline__ void philox4x64_10(uint64_t x[4], uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t lo0 = kPhiloxM0 * x[0];
    const uint64_t hi0 = __umul64hi(kPhiloxM0, x[0]);
    const uint64_t lo1 = kPhiloxM1 * x[2];
    const uint64_t hi1 = __umul64hi(kPhiloxM1, x[2]);
    const uint64_t y0 = hi1 ^ x[1] ^ k0;
    const uint64_t y2 = hi0 ^ x[3] ^ k1;
    x[0] = y0;
    x[1] = lo1;
    x[2] = y2;
    x[3] = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
}

// First output word for counter (c0, c1, c2, c3) under key (seed, 0).
__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                                 uint64_t seed) {
  uint64_t x[4] = {c0, c1, c2, c3};
  philox4x64_10(x, seed, 0);
  return x[0];
}

// Uniform in [0, 1): the top 53 bits of word 0 times 2^-53 (exact in double).
__device__ __forceinline__ double philox_uniform(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                                 uint64_t seed) {
  return static_cast<double>(philox_word0(c0, c1, c2, c3, seed) >> 11) * 0x1.0p-53;
}

// The dispatcher hands workgroups to the chip's 8 XCDs round-robin by linear
// id, and each XCD has its own L2.  Remap the linear id so that every XCD
// receives one contiguous range of logical ids: neighbouring tiles, which read
// the same rows, then share one L2 instead of fetching them eight times.
__device__ __forceinline__ int64_t xcd_remap(int64_t pid, int64_t total) {
  constexpr int64_t kXcd = 8;
  const int64_t q = total / kXcd, r = total % kXcd;
  const int64_t x = pid % kXcd, local = pid / kXcd;
  return x * q + (x < r ? x : r) + local;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace thin
