// Quantize-append kernel (kvq_quantize_append, kvq_append_and_rotate): the
// append workgroups run the body of kvq_append.h; with a fused query
// rotation, extra grid columns rotate the step's query heads (kvq_rotate.h)
// while the append runs.  Method: OmniKVQuant page, Sec. 2 Method.
#include "kvq_append.h"

namespace kvq {

namespace {

using app::kAppendThreads;
constexpr int kComputeUnits = 256;

// WIDE: a chunk with more workgroups than compute units; the register
// budget then allows two workgroups per CU (a few registers spill, which a
// one-position append, bound by its latency, would pay for).
template <int D, bool BF16, int BITS, bool WIDE>
__global__ __launch_bounds__(kAppendThreads, WIDE ? 4 : 1) void append_kernel(AppendArgs a) {
  __shared__ app::AppendSmem<D> sm;
  __shared__ int s_last;
  const int tid = threadIdx.x;
  if (static_cast<int>(blockIdx.x) >= a.append_x) {
    // ================= fused query rotation: 32 heads per workgroup
    const int r = (static_cast<int>(blockIdx.x) - a.append_x) * static_cast<int>(gridDim.z * gridDim.y) +
                  static_cast<int>(blockIdx.z * gridDim.y + blockIdx.y);
    const int first = r * (kAppendThreads / rotq::kLanes);
    if (first < a.rot_heads) {
      const int bi = first + tid / rotq::kLanes, sub = tid % rotq::kLanes;
      if (a.rot_bf16) rotq::rotate_head<D, true>(a.rq, a.rot_heads, bi, sub);
      else rotq::rotate_head<D, false>(a.rq, a.rot_heads, bi, sub);
    }
    return;   // no ticket: only the append's workgroups count
  }
  // Dispatch order (workgroups start in the order of their linear index):
  // the value workgroups (the longer ones: a group's rotation R_m^T v) of
  // every group but the last, over all (KV head, session) pairs, then their
  // key workgroups, then both workgroups of the last group, which is empty
  // when the chunk starts on a group boundary (the grid covers any start).
  // A chunk with more workgroups than slots then leaves only those empty
  // ones for a second round.
  const int P = static_cast<int>(gridDim.y * gridDim.z);   // (KV head, session) pairs
  const int G = a.append_x / 2;                              // groups the append may touch
  const int i = static_cast<int>(blockIdx.x) + a.append_x * static_cast<int>(blockIdx.z * gridDim.y + blockIdx.y);
  const int nmain = (G - 1) * P;
  int grp, pair;
  bool val;
  if (i < nmain) {
    val = true;
    grp = i / P;
    pair = i % P;
  } else if (i < 2 * nmain) {
    val = false;
    grp = (i - nmain) / P;
    pair = (i - nmain) % P;
  } else {
    const int j = i - 2 * nmain;
    val = j < P;
    grp = G - 1;
    pair = j % P;
  }
  const int bx = 2 * grp + (val ? 1 : 0);
  app::append_group<D, BF16, BITS>(a, sm, s_last, bx, pair % static_cast<int>(gridDim.y),
                                   pair / static_cast<int>(gridDim.y), a.append_x * static_cast<int>(gridDim.y));
}

template <int D, bool BF16>
hipError_t launch_append_t(int nb, AppendArgs a, hipStream_t s) {
  // two workgroups (keys, values) per touched group, then the columns of
  // the fused query rotation (32 heads per workgroup)
  a.append_x = 2 * ((a.n_new + 30) / kGroupTokens + 1);
  const int rot_wgs = (a.rot_heads + kAppendThreads / rotq::kLanes - 1) / (kAppendThreads / rotq::kLanes);
  const int rot_x = (rot_wgs + a.hkv * nb - 1) / (a.hkv * nb);
  const dim3 grid(a.append_x + rot_x, a.hkv, nb);
  const bool wide = static_cast<long long>(a.append_x) * a.hkv * nb > kComputeUnits;
#define KVQ_APPEND(B)                                                                                   \
  do {                                                                                                  \
    if (wide) hipLaunchKernelGGL((append_kernel<D, BF16, B, true>), grid, dim3(kAppendThreads), 0, s, a);  \
    else hipLaunchKernelGGL((append_kernel<D, BF16, B, false>), grid, dim3(kAppendThreads), 0, s, a);      \
  } while (0)
  if (a.bits == 4) KVQ_APPEND(4);
  else if (a.bits == 3) KVQ_APPEND(3);
  else KVQ_APPEND(2);
#undef KVQ_APPEND
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int d, bool bf16, int nb, const AppendArgs& a, hipStream_t s) {
  if (d == 64) return bf16 ? launch_append_t<64, true>(nb, a, s) : launch_append_t<64, false>(nb, a, s);
  return bf16 ? launch_append_t<128, true>(nb, a, s) : launch_append_t<128, false>(nb, a, s);
}

}  // namespace kvq
