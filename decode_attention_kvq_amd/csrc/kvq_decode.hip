// Fused decode attention over the 2-bit packed cache (OmniKVQuant page,
// Sec. 1 Introduction, Implementation bullet; Abstract): the codes are
// unpacked inside attention, scores use the already-rotated query, values are
// aggregated per modality in their rotated frames, and the inverse value
// rotations are applied once per modality after aggregation.
//
// Partition kernel: one wavefront per (session, KV head, context partition)
// serves all G query heads of the KV head, streaming 32-position groups:
//   score   s_t = scale * (sum_c q_c LO_c + sum_c (q_c (HI_c - LO_c)) l[code])
//           with l[code] = (c[code] - c0) / (c3 - c0)
//   softmax online (running max / sum per head, base-2 exponent)
//   values  A_m += p_t (N_t / sqrt(d)) c[vcode]   (three accumulators per head)
// Merge kernel: one workgroup per (session, query head) rescales and sums the
// partitions, applies out = sum_m R_m A_m / l.
#include "kvq_common.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxSplits = 4096;

template <int D>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeArgs a) {
  constexpr int W = D / 8;
  constexpr int CPL = D / 64;   // value channels per lane: c = lane + 64 k
  constexpr int GM = kMaxGroupHeads;
  __shared__ float s_q[GM][D];
  __shared__ float s_qt[kWaves][GM][D];
  __shared__ float s_w[kWaves][GM][kGroupTokens];
  __shared__ __align__(16) uint8_t s_k[kWaves][8 * D];
  __shared__ __align__(16) uint8_t s_v[kWaves][8 * D];
  __shared__ float s_nrm[kWaves][kGroupTokens];
  __shared__ uint8_t s_mod[kWaves][kGroupTokens];

  const int b = blockIdx.z, h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int split = blockIdx.x * kWaves + wave;
  const int G = a.group;
  const int L = a.seq_len[b];
  const int gp = a.page_tokens / kGroupTokens;

  for (int idx = threadIdx.x; idx < G * D; idx += 256)
    s_q[idx / D][idx % D] = a.q_rot[(static_cast<size_t>(b) * a.hq + h * G + idx / D) * D + idx % D];
  __syncthreads();

  float m_run[GM], l_run[GM], acc[GM][kModalities][CPL];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    m_run[hh] = -__builtin_inff();
    l_run[hh] = 0.f;
#pragma unroll
    for (int m = 0; m < kModalities; ++m)
#pragma unroll
      for (int k = 0; k < CPL; ++k) acc[hh][m][k] = 0.f;
  }

  // The last partition runs to the session's current length, so a launch
  // planned for a shorter context (e.g. replayed from a captured graph while
  // the cache grows) still covers every cached position.
  const int tb = split * a.split_tokens;
  const int te = (split == a.splits - 1) ? L : min(tb + a.split_tokens, L);
  const int tok = lane & 31, half = lane >> 5;

  for (int t0 = tb; t0 < te; t0 += kGroupTokens) {
    const int page = t0 / a.page_tokens;
    const int phys = page < a.max_pages ? a.page_table[static_cast<size_t>(b) * a.max_pages + page] : -1;
    if (phys < 0 || phys >= a.num_pages) continue;   // unmapped page: nothing to read
    const size_t blk = (static_cast<size_t>(phys) * a.hkv + h) * gp + (t0 % a.page_tokens) / kGroupTokens;
    const size_t prow = (static_cast<size_t>(phys) * a.hkv + h) * a.page_tokens + (t0 % a.page_tokens);

    // Stage the group's key / value code blocks, norms and modalities.
    if (lane * 16 < 8 * D) {
      reinterpret_cast<uint4*>(s_k[wave])[lane] = reinterpret_cast<const uint4*>(a.k_codes + blk * 8 * D)[lane];
      reinterpret_cast<uint4*>(s_v[wave])[lane] = reinterpret_cast<const uint4*>(a.v_codes + blk * 8 * D)[lane];
    }
    if (lane < kGroupTokens) {
      const bool ok = t0 + lane < te;
      s_nrm[wave][lane] = ok ? f16_bits_to_f32(a.v_norms[prow + lane]) * a.value_scale : 0.f;
      s_mod[wave][lane] = ok ? a.modality[static_cast<size_t>(phys) * a.page_tokens + (t0 % a.page_tokens) + lane] : 0;
    }

    // Fold the group statistics into the query: q~ = q (HI - LO), bias = q . LO.
    float lo[CPL], dl[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = lane + 64 * k;
      const float LO = f16_bits_to_f32(a.k_stats[blk * 2 * D + c]);
      const float HI = f16_bits_to_f32(a.k_stats[blk * 2 * D + D + c]);
      lo[k] = LO;
      dl[k] = HI - LO;
    }
    float bias[GM];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      bias[hh] = 0.f;
      if (hh < G) {
        float p = 0.f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          const int c = lane + 64 * k;
          p += s_q[hh][c] * lo[k];
          s_qt[wave][hh][c] = s_q[hh][c] * dl[k];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
        bias[hh] = p;
      }
    }
    wave_sync();

    // Scores: lane = (position tok, channel half).
    float sc[GM];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) sc[hh] = 0.f;
    for (int cc = 0; cc < D / 2; ++cc) {
      const int c = half * (D / 2) + cc;
      const uint32_t code = (s_k[wave][key_code_byte<D>(tok, c)] >> (2 * (c & 3))) & 3u;
      const float lv = a.lv[code];
#pragma unroll
      for (int hh = 0; hh < GM; ++hh)
        if (hh < G) sc[hh] += s_qt[wave][hh][c] * lv;
    }
    const bool valid = t0 + tok < te;
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      if (hh < G) {
        const float s = (sc[hh] + __shfl_xor(sc[hh], 32) + bias[hh]) * a.scale_log2e;
        float mx = valid ? s : -__builtin_inff();
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        const float m_new = fmaxf(m_run[hh], mx);
        const float alpha = exp2f(m_run[hh] - m_new);   // 0 when m_run is -inf
        const float p = valid ? exp2f(s - m_new) : 0.f;
        float ps = p;
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
        l_run[hh] = l_run[hh] * alpha + ps;
        m_run[hh] = m_new;
#pragma unroll
        for (int m = 0; m < kModalities; ++m)
#pragma unroll
          for (int k = 0; k < CPL; ++k) acc[hh][m][k] *= alpha;
        if (lane < kGroupTokens) s_w[wave][hh][tok] = p * s_nrm[wave][tok];
      }
    }
    wave_sync();

    // Values: lane = channels lane + 64 k; loop over the group's positions.
    const int nt = min(kGroupTokens, te - t0);
    for (int tt = 0; tt < nt; ++tt) {
      const int m = s_mod[wave][tt];
      float cv[CPL];
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int c = lane + 64 * k;
        const uint32_t code = (s_v[wave][value_code_byte<D>(tt, c)] >> (2 * (tt & 3))) & 3u;
        cv[k] = a.cv[code];
      }
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        if (hh < G) {
          const float w = s_w[wave][hh][tt];
#pragma unroll
          for (int k = 0; k < CPL; ++k) {
            if (m == 0) acc[hh][0][k] += w * cv[k];
            else if (m == 1) acc[hh][1][k] += w * cv[k];
            else acc[hh][2][k] += w * cv[k];
          }
        }
      }
    }
    wave_sync();
  }

  // Partial result of this partition for each query head of the group.
  constexpr int PS = 2 + kModalities * D;
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    if (hh < G) {
      float* part = a.partials + ((static_cast<size_t>(b) * a.hq + h * G + hh) * a.splits + split) * PS;
      if (lane == 0) {
        part[0] = m_run[hh];
        part[1] = l_run[hh];
      }
#pragma unroll
      for (int m = 0; m < kModalities; ++m)
#pragma unroll
        for (int k = 0; k < CPL; ++k) part[2 + m * D + lane + 64 * k] = acc[hh][m][k];
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PS = 2 + kModalities * D;
  __shared__ float s_e[kMaxSplits];
  __shared__ float s_A[kModalities][D];
  __shared__ float s_red[256];
  const int i = blockIdx.x, b = blockIdx.y;
  const int h = i / a.group;
  const int tid = threadIdx.x;
  const float* P = a.partials + (static_cast<size_t>(b) * a.hq + i) * a.splits * PS;

  float mx = -__builtin_inff();
  for (int s = tid; s < a.splits; s += 256) mx = fmaxf(mx, P[static_cast<size_t>(s) * PS]);
  s_red[tid] = mx;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) s_red[tid] = fmaxf(s_red[tid], s_red[tid + off]);
    __syncthreads();
  }
  const float M = s_red[0];
  __syncthreads();
  float ls = 0.f;
  for (int s = tid; s < a.splits; s += 256) {
    const float ms = P[static_cast<size_t>(s) * PS];
    const float e = (ms == -__builtin_inff()) ? 0.f : exp2f(ms - M);
    s_e[s] = e;
    ls += e * P[static_cast<size_t>(s) * PS + 1];
  }
  s_red[tid] = ls;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) s_red[tid] += s_red[tid + off];
    __syncthreads();
  }
  const float l = s_red[0];
  for (int idx = tid; idx < kModalities * D; idx += 256) {
    float A = 0.f;
    for (int s = 0; s < a.splits; ++s) A += s_e[s] * P[static_cast<size_t>(s) * PS + 2 + idx];
    s_A[idx / D][idx % D] = A;
  }
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
    for (int m = 0; m < kModalities; ++m) {
      const float* R = a.rot + ((static_cast<size_t>(h) * kModalities + m) * D + tid) * D;
      for (int j = 0; j < D; ++j) o += R[j] * s_A[m][j];
    }
    a.out[(static_cast<size_t>(b) * a.hq + i) * D + tid] = (l > 0.f) ? o / l : 0.f;
  }
}

template <int D>
hipError_t launch_decode_t(int batch, const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_partition_kernel<D>), dim3(a.splits / kWaves, a.hkv, batch), dim3(256), 0, s, a);
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.hq, batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int d, int batch, const DecodeArgs& a, hipStream_t s) {
  return d == 64 ? launch_decode_t<64>(batch, a, s) : launch_decode_t<128>(batch, a, s);
}

}  // namespace kvq
