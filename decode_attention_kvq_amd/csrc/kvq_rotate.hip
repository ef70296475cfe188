// Query rotation: each query head is rotated once with the Hadamard signs of
// its KV head, q_rot = H_d (s * q) / sqrt(d), so that scores against the
// rotated keys equal scores against the original keys (OmniKVQuant page,
// Sec. 1 Introduction, Implementation bullet: one query rotated per head).
//
// One wavefront per (session, query head); the transform runs in fp64 across
// the wavefront's lanes (exact for bf16 inputs) and is rounded once to fp32.
#include "kvq_common.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

template <int D, bool BF16>
__global__ __launch_bounds__(64) void rotate_query_kernel(RotateArgs a) {
  constexpr int CH = D / 64;   // channels per lane
  const int bi = blockIdx.x;   // b * Hq + i
  const int h = (bi % a.hq) / a.group;
  const int lane = threadIdx.x;
  double x[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int c = lane * CH + k;
    x[k] = load_input<BF16>(a.q, static_cast<size_t>(bi) * D + c) * static_cast<double>(a.signs[h * D + c]);
  }
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
  for (int hh = CH; hh < D; hh <<= 1) {
    const int m = hh / CH;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const double p = __shfl_xor(x[i], m);
      x[i] = (lane & m) ? (p - x[i]) : (x[i] + p);
    }
  }
#pragma unroll
  for (int k = 0; k < CH; ++k)
    a.q_rot[static_cast<size_t>(bi) * D + lane * CH + k] = static_cast<float>(x[k] * a.inv_sqrt_d);
}

}  // namespace

hipError_t launch_rotate_query(int d, bool bf16, int batch, const RotateArgs& a, hipStream_t s) {
  const dim3 grid(batch * a.hq);
  if (d == 64) {
    if (bf16) hipLaunchKernelGGL((rotate_query_kernel<64, true>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((rotate_query_kernel<64, false>), grid, dim3(64), 0, s, a);
  } else {
    if (bf16) hipLaunchKernelGGL((rotate_query_kernel<128, true>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((rotate_query_kernel<128, false>), grid, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kvq
