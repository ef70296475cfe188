// Quantize-append kernels: keys (randomized Hadamard rotation + per-group
// min-max scaling onto the fixed codebook) and values (per-modality rotation
// + norm scaling onto the fixed codebook), written into the lane-major
// 2-bit group blocks of the paged cache.
//
// Method: OmniKVQuant page, Sec. 2 Method (TurboQuant bullet, and the two
// OmniKVQuant bullets for keys and values).
//
// Every decision (statistics, codes) is taken in fp64, with the same
// operation order as the definition, so that the stored codes and fp16
// statistics are exactly those of an fp64 reference.  This file is compiled
// with -ffp-contract=off for that reason.
#include "kvq_common.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

// Physical group-block index of absolute position t0 (a multiple of 32) of
// session sb, KV head h; -1 if the page table entry is out of range.
__device__ __forceinline__ long long group_block(const AppendArgs& a, int sb, int h, int t0) {
  const int page = t0 / a.page_tokens;
  if (page >= a.max_pages) return -1;
  const int phys = a.page_table[static_cast<size_t>(sb) * a.max_pages + page];
  if (phys < 0 || phys >= a.num_pages) return -1;
  const int gp = a.page_tokens / kGroupTokens;
  return (static_cast<long long>(phys) * a.hkv + h) * gp + (t0 % a.page_tokens) / kGroupTokens;
}

// One workgroup re-quantizes one 32-token key group touched by the append:
// the group's earlier positions come from the raw key tail, the rest from
// k_new.  256 threads: 8 threads per position, D/8 channels each.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void key_append_kernel(AppendArgs a) {
  constexpr int CH = D / 8;
  __shared__ double s_red[4][2][D];
  __shared__ double s_lohi[2][D];
  __shared__ __align__(16) uint8_t s_blk[8 * D];

  const int b = blockIdx.z, h = blockIdx.y;
  const int sb = a.b0 + b;
  const int L_old = a.seq_len[sb];
  const int L_new = L_old + a.n_new;
  const int t0 = (L_old / kGroupTokens + static_cast<int>(blockIdx.x)) * kGroupTokens;
  if (t0 >= L_new) return;
  const long long blk = group_block(a, sb, h, t0);
  if (blk < 0) return;
  const int n_tok = min(kGroupTokens, L_new - t0);

  const int tid = threadIdx.x, tok = tid >> 3, part = tid & 7;
  const int lane = tid & 63, wave = tid >> 6;
  const int cb = part * CH;
  const int t = t0 + tok;
  const bool present = tok < n_tok;

  double x[CH];
  if (present) {
    const void* src;
    size_t row;
    if (t < L_old) {
      src = a.k_tail;
      row = ((static_cast<size_t>(sb) * a.hkv + h) * kGroupTokens + (t & 31)) * D;
    } else {
      src = a.k_new;
      row = ((static_cast<size_t>(b) * a.n_new + (t - L_old)) * a.hkv + h) * D;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i)
      x[i] = load_input<BF16>(src, row + cb + i) * static_cast<double>(a.signs[h * D + cb + i]);
  } else {
#pragma unroll
    for (int i = 0; i < CH; ++i) x[i] = 0.0;
  }

  // Unnormalised Walsh-Hadamard transform of the position's D channels:
  // strides below CH inside the thread, larger strides across the 8 threads
  // of the position (lanes tid ^ 1, 2, 4).
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
      x[i] = (part & m) ? (p - x[i]) : (x[i] + p);
    }
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) x[i] = x[i] * a.inv_sqrt_d;

  // Per-channel min / max over the group's present positions.
  double mn[CH], mx[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    mn[i] = present ? x[i] : __builtin_inf();
    mx[i] = present ? x[i] : -__builtin_inf();
  }
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      mn[i] = fmin(mn[i], __shfl_xor(mn[i], off));
      mx[i] = fmax(mx[i], __shfl_xor(mx[i], off));
    }
  }
  if (lane < 8) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      s_red[wave][0][cb + i] = mn[i];
      s_red[wave][1][cb + i] = mx[i];
    }
  }
  __syncthreads();
  if (tid < D) {
    double lo = s_red[0][0][tid], hi = s_red[0][1][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      lo = fmin(lo, s_red[w][0][tid]);
      hi = fmax(hi, s_red[w][1][tid]);
    }
    const uint16_t lo16 = f64_to_f16_rne(lo), hi16 = f64_to_f16_rne(hi);
    uint16_t* st = a.k_stats + static_cast<size_t>(blk) * 2 * D;
    st[tid] = lo16;
    st[D + tid] = hi16;
    s_lohi[0][tid] = static_cast<double>(f16_bits_to_f32(lo16));
    s_lohi[1][tid] = static_cast<double>(f16_bits_to_f32(hi16));
  }
  __syncthreads();

  // Codes: z = c0 + ((y - LO) * (c3 - c0)) / (HI - LO); code = thresholds reached.
  const double span_c = a.c3 - a.c0;
#pragma unroll
  for (int q4 = 0; q4 < CH / 4; ++q4) {
    uint32_t byte = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = cb + 4 * q4 + i;
      uint32_t code = 0;
      if (present) {
        const double LO = s_lohi[0][c], HI = s_lohi[1][c];
        if (HI > LO) {
          const double z = a.c0 + ((x[4 * q4 + i] - LO) * span_c) / (HI - LO);
          code = (z >= a.thr0 ? 1u : 0u) + (z >= a.thr1 ? 1u : 0u) + (z >= a.thr2 ? 1u : 0u);
        }
      }
      byte |= code << (2 * i);
    }
    s_blk[key_code_byte<D>(tok, cb + 4 * q4)] = static_cast<uint8_t>(byte);
  }
  __syncthreads();
  if (tid < D / 2) {
    uint4* dst = reinterpret_cast<uint4*>(a.k_codes + static_cast<size_t>(blk) * 8 * D);
    dst[tid] = reinterpret_cast<const uint4*>(s_blk)[tid];
  }
}

// One workgroup quantizes the new positions of one 32-token group of values
// (merging with the codes already stored for the group's earlier positions).
// 256 threads = TQ parts x D output channels: part p accumulates
// r_j = sum_i R_{h,m}[i][j] v_i over its slice of i for every new position,
// so each element of R is read once per workgroup and the loads of a slice
// are independent; the parts are then summed in a fixed order.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void value_append_kernel(AppendArgs a) {
  constexpr int TQ = 256 / D;       // parts of the i range
  constexpr int IQ = D / TQ;        // rows of R per part
  constexpr int W = D / 8;
  __shared__ double s_v[kGroupTokens][D];
  __shared__ double s_r[TQ - 1][kGroupTokens][D];
  __shared__ double s_n[kGroupTokens];
  __shared__ uint8_t s_mod[kGroupTokens];
  __shared__ uint8_t s_code[kGroupTokens][D];

  const int b = blockIdx.z, h = blockIdx.y;
  const int sb = a.b0 + b;
  const int L_old = a.seq_len[sb];
  const int L_new = L_old + a.n_new;
  const int t0 = (L_old / kGroupTokens + static_cast<int>(blockIdx.x)) * kGroupTokens;
  if (t0 >= L_new) return;
  const long long blk = group_block(a, sb, h, t0);
  if (blk < 0) return;
  const int s_first = max(L_old - t0, 0);
  const int s_end = min(kGroupTokens, L_new - t0);
  const int tid = threadIdx.x;

  for (int idx = tid; idx < kGroupTokens * D; idx += 256) {
    const int s = idx / D, c = idx % D;
    if (s >= s_first && s < s_end) {
      const size_t src = ((static_cast<size_t>(b) * a.n_new + (t0 + s - L_old)) * a.hkv + h) * D + c;
      s_v[s][c] = load_input<BF16>(a.v_new, src);
    }
  }
  if (tid < kGroupTokens) {
    const int s = tid;
    if (s >= s_first && s < s_end) s_mod[s] = a.modality_new[static_cast<size_t>(b) * a.n_new + (t0 + s - L_old)];
  }
  __syncthreads();
  // Which modalities occur among the new positions (uniform across the block).
  uint32_t present = 0;
  for (int s = s_first; s < s_end; ++s) present |= (s_mod[s] < kModalities) ? (1u << s_mod[s]) : 0u;
  if (tid < kGroupTokens) {
    const int s = tid;
    if (s >= s_first && s < s_end) {
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc = acc + s_v[s][c] * s_v[s][c];
      s_n[s] = sqrt(acc);
    }
  }

  const int jc = tid % D, part = tid / D;
  const int i0 = part * IQ;
  double acc[kGroupTokens];
#pragma unroll
  for (int s = 0; s < kGroupTokens; ++s) acc[s] = 0.0;
  for (int m = 0; m < kModalities; ++m) {
    if (!(present & (1u << m))) continue;
    const float* Rm = a.rot + ((static_cast<size_t>(h) * kModalities + m) * D + i0) * D + jc;
    for (int i = 0; i < IQ; i += 16) {
      double r[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) r[u] = static_cast<double>(Rm[(i + u) * D]);
#pragma unroll
      for (int s = 0; s < kGroupTokens; ++s) {
        if (s >= s_first && s < s_end && s_mod[s] == m) {
#pragma unroll
          for (int u = 0; u < 16; ++u) acc[s] = fma(r[u], s_v[s][i0 + i + u], acc[s]);
        }
      }
    }
  }
  if (part > 0) {
#pragma unroll
    for (int s = 0; s < kGroupTokens; ++s)
      if (s >= s_first && s < s_end) s_r[part - 1][s][jc] = acc[s];
  }
  __syncthreads();
  if (part == 0) {
#pragma unroll
    for (int s = 0; s < kGroupTokens; ++s) {
      if (s >= s_first && s < s_end) {
        double r = acc[s];
        for (int p = 1; p < TQ; ++p) r = r + s_r[p - 1][s][jc];
        const double n = s_n[s];
        uint32_t code = 0;
        if (n > 0.0) {
          const double z = (a.sqrt_d * r) / n;
          code = (z >= a.thr0 ? 1u : 0u) + (z >= a.thr1 ? 1u : 0u) + (z >= a.thr2 ? 1u : 0u);
        }
        s_code[s][jc] = static_cast<uint8_t>(code);
      }
    }
  }
  __syncthreads();

  // Rewrite the group block: earlier positions keep their stored codes.
  uint8_t* vb = a.v_codes + static_cast<size_t>(blk) * 8 * D;
  for (int byte = tid; byte < 8 * D; byte += 256) {
    const int L = byte / W, wi = byte % W;
    const int nt = wi >> 1, hf = wi & 1, kg = L >> 4, col = L & 15;
    const int c = nt * 16 + col;
    const uint32_t old = s_first > 0 ? vb[byte] : 0u;
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = hf * 16 + kg * 4 + i;
      uint32_t code;
      if (s < s_first) code = (old >> (2 * i)) & 3u;
      else if (s < s_end) code = s_code[s][c];
      else code = 0u;
      out |= code << (2 * i);
    }
    vb[byte] = static_cast<uint8_t>(out);
  }
  if (tid < kGroupTokens) {
    const int s = tid;
    if (s >= s_first && s < s_end) {
      const int phys = static_cast<int>(blk / (static_cast<long long>(a.hkv) * (a.page_tokens / kGroupTokens)));
      const int pos = (t0 + s) % a.page_tokens;
      a.v_norms[(static_cast<size_t>(phys) * a.hkv + h) * a.page_tokens + pos] = f64_to_f16_rne(s_n[s]);
      if (h == 0) a.modality[static_cast<size_t>(phys) * a.page_tokens + pos] = s_mod[s];
    }
  }
}

// After both quantize kernels: save the raw keys of the (new) open group into
// the tail and advance seq_len.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void finalize_append_kernel(AppendArgs a) {
  const int b = blockIdx.x, sb = a.b0 + b;
  const int L_old = a.seq_len[sb];
  const int L_new = L_old + a.n_new;
  const int start = max((L_new / kGroupTokens) * kGroupTokens, L_old);
  const int count = L_new - start;
  const size_t elems = static_cast<size_t>(count) * a.hkv * D;
  for (size_t idx = threadIdx.x; idx < elems; idx += blockDim.x) {
    const int c = static_cast<int>(idx % D);
    const int h = static_cast<int>((idx / D) % a.hkv);
    const int tt = static_cast<int>(idx / (static_cast<size_t>(D) * a.hkv));
    const int t = start + tt;
    const size_t src = ((static_cast<size_t>(b) * a.n_new + (t - L_old)) * a.hkv + h) * D + c;
    const size_t dst = ((static_cast<size_t>(sb) * a.hkv + h) * kGroupTokens + (t & 31)) * D + c;
    if constexpr (BF16) {
      static_cast<uint16_t*>(a.k_tail)[dst] = static_cast<const uint16_t*>(a.k_new)[src];
    } else {
      static_cast<float*>(a.k_tail)[dst] = static_cast<const float*>(a.k_new)[src];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.seq_len[sb] = L_new;
}

template <int D, bool BF16>
hipError_t launch_append_t(int nb, const AppendArgs& a, hipStream_t s) {
  const dim3 grid((a.n_new + 30) / kGroupTokens + 1, a.hkv, nb);
  hipLaunchKernelGGL((key_append_kernel<D, BF16>), grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL((value_append_kernel<D, BF16>), grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL((finalize_append_kernel<D, BF16>), dim3(nb), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int d, bool bf16, int nb, const AppendArgs& a, hipStream_t s) {
  if (d == 64) return bf16 ? launch_append_t<64, true>(nb, a, s) : launch_append_t<64, false>(nb, a, s);
  return bf16 ? launch_append_t<128, true>(nb, a, s) : launch_append_t<128, false>(nb, a, s);
}

}  // namespace kvq
