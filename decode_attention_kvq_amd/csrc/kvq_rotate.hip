// Query rotation kernel (kvq_rotate_query): 16 query heads per 256-thread
// workgroup, 16 lanes per head; the body is in kvq_rotate.h.
#include "kvq_rotate.h"

namespace kvq {

namespace {

constexpr int kRotThreads = 256;

template <int D, bool BF16>
__global__ __launch_bounds__(kRotThreads) void rotate_query_kernel(RotateArgs a, int n_heads) {
  const int tid = threadIdx.x;
  rotq::rotate_head<D, BF16>(a, n_heads, blockIdx.x * (kRotThreads / rotq::kLanes) + tid / rotq::kLanes,
                             tid % rotq::kLanes);
}

template <int D, bool BF16>
void launch_rotate_t(int n_heads, const RotateArgs& a, hipStream_t s) {
  constexpr int per_block = kRotThreads / rotq::kLanes;
  const dim3 grid((n_heads + per_block - 1) / per_block);
  hipLaunchKernelGGL((rotate_query_kernel<D, BF16>), grid, dim3(kRotThreads), 0, s, a, n_heads);
}

}  // namespace

hipError_t launch_rotate_query(int d, bool bf16, int batch, const RotateArgs& a, hipStream_t s) {
  const int n_heads = batch * a.hq;
  if (d == 64) {
    if (bf16) launch_rotate_t<64, true>(n_heads, a, s);
    else launch_rotate_t<64, false>(n_heads, a, s);
  } else {
    if (bf16) launch_rotate_t<128, true>(n_heads, a, s);
    else launch_rotate_t<128, false>(n_heads, a, s);
  }
  return hipGetLastError();
}

}  // namespace kvq
