// Measurement aid: a plain streaming read of a device buffer, the floor for
// one read-only kernel of a given size on this GPU (the decode reads its
// packed cache once, so its time cannot go below this read of the same
// bytes).  Every thread issues 16-byte loads, four in flight, over a
// grid-stride range and folds the words with XOR; one word per workgroup is
// written to `sink` so that the loads cannot be dropped.
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                                    uint32_t* __restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kProbeThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // fold the workgroup's words: one atomic per wavefront into its slot
  for (int o = 32; o > 0; o >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o));
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kProbeThreads), 0, s,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace kvq
