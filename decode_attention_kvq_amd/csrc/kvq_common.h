// Device helpers shared by the libkvq kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Exact fp64 image of a bf16 / fp32 input element.
template <bool BF16>
__device__ __forceinline__ double load_input(const void* p, size_t idx) {
  if constexpr (BF16) {
    const uint32_t bits = static_cast<uint32_t>(static_cast<const uint16_t*>(p)[idx]) << 16;
    return static_cast<double>(__uint_as_float(bits));
  } else {
    return static_cast<double>(static_cast<const float*>(p)[idx]);
  }
}

// fp64 -> fp16 bits, round to nearest, ties to even, in one step from the
// fp64 value (no intermediate fp32 rounding).  Overflow goes to infinity,
// values below half the smallest subnormal go to signed zero.
__device__ __forceinline__ uint16_t f64_to_f16_rne(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(u >> 48) & 0x8000u;
  const int bexp = static_cast<int>((u >> 52) & 0x7FF);
  const uint64_t mant = u & 0xFFFFFFFFFFFFFull;
  if (bexp == 0x7FF) return static_cast<uint16_t>(sign | 0x7C00u | (mant ? 0x200u : 0u));
  if (bexp == 0) return static_cast<uint16_t>(sign);  // fp64 zero / subnormal: far below fp16 range
  const int e = bexp - 1023;
  if (e > 15) return static_cast<uint16_t>(sign | 0x7C00u);
  const uint64_t sig = mant | (1ull << 52);
  uint32_t hexp;
  int shift;
  if (e >= -14) {
    hexp = static_cast<uint32_t>(e + 15);
    shift = 42;
  } else {
    hexp = 0;
    shift = 28 - e;  // subnormal: unit 2^-24
  }
  if (shift >= 64) return static_cast<uint16_t>(sign);
  uint64_t m = sig >> shift;
  const uint64_t rest = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rest > half || (rest == half && (m & 1ull))) ++m;
  uint32_t r;
  if (hexp) {
    if (m == 2048) {
      m = 1024;
      ++hexp;
    }
    if (hexp >= 31) return static_cast<uint16_t>(sign | 0x7C00u);
    r = (hexp << 10) | static_cast<uint32_t>(m & 0x3FF);
  } else {
    r = static_cast<uint32_t>(m);  // 1024 becomes the smallest normal
  }
  return static_cast<uint16_t>(sign | r);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// Orders LDS traffic between the lanes of one wavefront.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Byte offsets inside one lane-major 8d-byte group block (see kvq.h).
template <int D>
__device__ __forceinline__ int key_code_byte(int t, int c) {
  constexpr int W = D / 8;
  const int lane = ((c & 31) >> 3) * 16 + (t & 15);
  return lane * W + (t >> 4) * (D / 16) + (c >> 5) * 2 + ((c & 7) >> 2);
}

template <int D>
__device__ __forceinline__ int value_code_byte(int t, int c) {
  constexpr int W = D / 8;
  const int lane = ((t & 15) >> 2) * 16 + (c & 15);
  return lane * W + (c >> 4) * 2 + (t >> 4);
}

}  // namespace kvq
