// Query rotation body, shared by the standalone rotation kernel and the
// fused append-and-rotate launch: q_rot = H_d (s * q) / sqrt(d) for one query
// head per 16 lanes (OmniKVQuant page, Sec. 1 Introduction, Implementation
// bullet: one query rotated per head).
//
// d / 16 channels per lane; the transform runs in fp64 (exact for bf16 /
// fp32 inputs) inside the lane and then across the head's 16 lanes (DPP quad
// permutes and swizzles, no LDS memory), and is rounded once to fp32 after
// the 1 / sqrt(d) scaling.  Every function here turns floating-point
// contraction off for its own body (the including file's setting does not
// matter); the lane butterflies' fma has a +-1 factor, so it rounds exactly
// like the addition it stands for.
#pragma once

#include "kvq_common.h"
#include "kvq_internal.h"

namespace kvq {
namespace rotq {

constexpr int kLanes = 16;                         // lanes per query head

template <int M>
__device__ __forceinline__ int xor_lane(int v) {
  if constexpr (M == 1) return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  if constexpr (M == 2) return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  return __builtin_amdgcn_ds_swizzle(v, (M << 10) | 0x1F);                                  // bit mode: xor M
}

template <int M>
__device__ __forceinline__ double xor_lane(double v) {
  const long long u = __double_as_longlong(v);
  const int lo = xor_lane<M>(static_cast<int>(u & 0xFFFFFFFF));
  const int hi = xor_lane<M>(static_cast<int>(u >> 32));
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

// x + x[lane ^ M] where the lane bit is clear, x[lane ^ M] - x where it is set
// (sgn = +1 / -1; the product is exact, so the fma rounds once, like the sum).
template <int M>
__device__ __forceinline__ double butterfly(double x, double sgn) {
  return __builtin_fma(sgn, x, xor_lane<M>(x));
}

// Channels sub * CH .. sub * CH + CH - 1 of the rotated head bi (= b * Hq +
// i), computed by the 16 lanes whose lane-in-head index is `sub`; all 16
// lanes of a head must call it together.
template <int D, bool BF16>
__device__ __forceinline__ void rotate_values(const RotateArgs& a, int bi, int sub, float (&o)[D / kLanes]) {
#pragma clang fp contract(off)
  constexpr int CH = D / kLanes;                   // channels per lane: 8 (d = 128) or 4 (d = 64)
  constexpr int ESZ = BF16 ? 2 : 4;
  const int h = (bi % a.hq) / a.group;
  const int c0 = sub * CH;

  uint32_t qw[CH * ESZ / 4];
  {
    const char* src = static_cast<const char*>(a.q) + (static_cast<size_t>(bi) * D + c0) * ESZ;
    if constexpr (CH * ESZ == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(src);
      qw[0] = v.x; qw[1] = v.y;
    } else {
#pragma unroll
      for (int k = 0; k < CH * ESZ / 16; ++k) {
        const uint4 v = reinterpret_cast<const uint4*>(src)[k];
        qw[4 * k] = v.x; qw[4 * k + 1] = v.y; qw[4 * k + 2] = v.z; qw[4 * k + 3] = v.w;
      }
    }
  }
  uint32_t sw[CH / 4];
#pragma unroll
  for (int k = 0; k < CH / 4; ++k) sw[k] = reinterpret_cast<const uint32_t*>(a.signs + h * D + c0)[k];

  double x[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    uint32_t bits;
    if constexpr (BF16) bits = (i & 1) ? (qw[i >> 1] & 0xFFFF0000u) : (qw[i >> 1] << 16);
    else bits = qw[i];
    // the sign is +-1: flip the fp32 sign bit where it is negative
    bits ^= ((sw[i >> 2] >> (8 * (i & 3))) & 0x80u) << 24;
    x[i] = static_cast<double>(__uint_as_float(bits));
  }
  // channel c = sub * CH + i: the transform over i inside the lane, over sub
  // across the head's 16 lanes (the two commute)
#pragma unroll
  for (int hh = 1; hh < CH; hh <<= 1) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (!(i & hh)) {
        const double u = x[i], v = x[i + hh];
        x[i] = u + v;
        x[i + hh] = u - v;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) x[i] = butterfly<1>(x[i], (sub & 1) ? -1.0 : 1.0);
#pragma unroll
  for (int i = 0; i < CH; ++i) x[i] = butterfly<2>(x[i], (sub & 2) ? -1.0 : 1.0);
#pragma unroll
  for (int i = 0; i < CH; ++i) x[i] = butterfly<4>(x[i], (sub & 4) ? -1.0 : 1.0);
#pragma unroll
  for (int i = 0; i < CH; ++i) x[i] = butterfly<8>(x[i], (sub & 8) ? -1.0 : 1.0);

#pragma unroll
  for (int i = 0; i < CH; ++i) o[i] = static_cast<float>(x[i] * a.inv_sqrt_d);
}

// Rotates head bi_raw (= b * Hq + i) into q_rot with the 16 lanes whose
// lane-in-head index is `sub`.  All 16 lanes of a head must call it
// together; a head index past n_heads works on the last head and stores
// nothing.
template <int D, bool BF16>
__device__ __forceinline__ void rotate_head(const RotateArgs& a, int n_heads, int bi_raw, int sub) {
  constexpr int CH = D / kLanes;
  const bool live = bi_raw < n_heads;
  const int bi = live ? bi_raw : n_heads - 1;
  float o[CH];
  rotate_values<D, BF16>(a, bi, sub, o);
  if (live) {
    float4* dst = reinterpret_cast<float4*>(a.q_rot + static_cast<size_t>(bi) * D + sub * CH);
#pragma unroll
    for (int k = 0; k < CH / 4; ++k) dst[k] = float4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
  }
}

}  // namespace rotq
}  // namespace kvq
