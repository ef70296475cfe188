// Quantize-append: keys (randomized Hadamard rotation + per-group min-max
// scaling onto the fixed codebook) and values (per-modality rotation + norm
// scaling onto the fixed codebook), written into the lane-major 2-bit group
// blocks of the paged cache.
//
// Method: OmniKVQuant page, Sec. 2 Method (TurboQuant bullet, and the two
// OmniKVQuant bullets for keys and values).
//
// Every decision is taken in fp64.  The statistics follow the definition's
// operation order, so the stored fp16 LO / HI are exactly those of an fp64
// reference; the key codes take the division once per channel and the value
// rotation sums in a fixed order, which can only change a code whose
// normalised value lies within a few ulps of a decision threshold.  This
// file is compiled with -ffp-contract=off so that no operation is fused
// behind the code's back.
//
// One launch.  Workgroup (j, h, b) re-quantizes the j-th 32-position group
// touched by the append of session b, KV head h: all the group's keys (the
// earlier ones from the raw key tail) and the group's new values.  Workgroup
// j = 0 is the only reader of the key tail, so it is also the one that
// stores the raw keys of the new open group (after its own reads).  Every
// workgroup takes a ticket when done; the last one of a session advances its
// length, so no workgroup can see the new length before it read the old one.
//
// Latency matters more than throughput for the common one-position append:
// every global load a workgroup needs is issued in two waves (inputs, then
// the rotation rows of the modality found in them), and the key transform
// runs while the rotation rows are in flight.
#include "kvq_common.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int kAppendThreads = 256;

// Value of lane ^ M (M = 1, 2, 4) for a double: quad permutations through DPP
// for M = 1, 2, a swizzle for M = 4 (no LDS memory traffic).
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

// Channel-major staging with rows padded to 33 positions: the writes of the
// 8-threads-per-position layout and the per-channel reads both spread over
// the LDS banks.
constexpr int kPadTok = kGroupTokens + 1;

template <int D>
struct AppendSmem {
  static constexpr int TQ = kAppendThreads / D;   // parts of the value rotation's i range
  union {
    double y[D][kPadTok];                         // rotated keys (statistics pass)
    double r[TQ][kGroupTokens][D];                // value rotation partial sums
  } u;
  double v[D][kPadTok];                           // new values
  double lohi[2][D];                              // fp16 statistics as fp64
  double n[kGroupTokens];                         // value norms
  __align__(16) uint8_t kblk[8 * D];              // key codes of the group (lane-major)
  uint8_t code[kGroupTokens][D];                  // value codes of the new positions
  uint8_t mod[kGroupTokens];
  int last;
};

template <int D, bool BF16>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  constexpr int CH = D / 8;                       // channels per thread (keys, inputs)
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int NV = CH * ESZ / 16;               // uint4 per thread per input row slice
  constexpr int TQ = AppendSmem<D>::TQ;
  constexpr int IQ = D / TQ;                      // rows of R per part
  constexpr int W = D / 8;
  __shared__ AppendSmem<D> sm;

  const int b = blockIdx.z, h = blockIdx.y, j = blockIdx.x;
  const int sb = a.b0 + b;
  const int tid = threadIdx.x, lane = tid & 63;
  const int jc = tid % D, pq = tid / D, i0 = pq * IQ;

  // Round trip 1: the session length, and the modalities of every new
  // position this group could hold (rows [32 j - 32, 32 j + 32) of the
  // append, whatever the old length), which pick the rotation rows to fetch.
  const int L_old = a.seq_len[sb];
  const int widx = 32 * j - 32 + lane;
  const bool wok = widx >= 0 && widx < a.n_new;
  const uint32_t wmod = a.modality_new[static_cast<size_t>(b) * a.n_new + min(max(widx, 0), a.n_new - 1)];
  uint32_t wmods = 0;
#pragma unroll
  for (int m = 0; m < kModalities; ++m)
    if (__any(wok && wmod == static_cast<uint32_t>(m))) wmods |= 1u << m;
  const int mpre = wmods ? __builtin_ctz(wmods) : 0;

  // Round trip 2: page table, key / value inputs, signs, the exact
  // modalities, and the prefetched rotation rows.
  const int L_new = L_old + a.n_new;
  const int t0 = (L_old / kGroupTokens + j) * kGroupTokens;
  const bool active = t0 < L_new;
  int phys = -1;
  if (active) {
    const int page = t0 / a.page_tokens;
    phys = page < a.max_pages ? a.page_table[static_cast<size_t>(sb) * a.max_pages + page] : -1;
  }
  const int s_first = max(L_old - t0, 0);        // first new position of the group
  const int s_end = min(kGroupTokens, L_new - t0);
  const int tok = tid >> 3, part = tid & 7, cb = part * CH;
  const bool present = tok < s_end;
  const int inew = min(max(t0 + tok - L_old, 0), a.n_new - 1);   // clamped row of k_new / v_new
  const char* krow = (t0 + tok < L_old)
      ? static_cast<const char*>(a.k_tail) + (((static_cast<size_t>(sb) * a.hkv + h) * kGroupTokens + tok) * D + cb) * ESZ
      : static_cast<const char*>(a.k_new) + (((static_cast<size_t>(b) * a.n_new + inew) * a.hkv + h) * D + cb) * ESZ;
  const char* vrow = static_cast<const char*>(a.v_new) + (((static_cast<size_t>(b) * a.n_new + inew) * a.hkv + h) * D + cb) * ESZ;
  uint4 kin[NV], vin[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    kin[u] = reinterpret_cast<const uint4*>(krow)[u];
    vin[u] = reinterpret_cast<const uint4*>(vrow)[u];
  }
  int8_t sg[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) sg[i] = a.signs[h * D + cb + i];
  const int ms = lane & 31;                      // this lane's modality slot
  const bool ms_fresh = ms >= s_first && ms < s_end;
  const uint32_t mod_l = a.modality_new[static_cast<size_t>(b) * a.n_new + min(max(t0 + ms - L_old, 0), a.n_new - 1)];
  float rr[IQ];
  {
    const float* Rm = a.rot + ((static_cast<size_t>(h) * kModalities + mpre) * D + i0) * D + jc;
#pragma unroll
    for (int i = 0; i < IQ; ++i) rr[i] = Rm[static_cast<size_t>(i) * D];
  }

  const long long blk = (active && phys >= 0 && phys < a.num_pages)
      ? (static_cast<long long>(phys) * a.hkv + h) * (a.page_tokens / kGroupTokens) + (t0 % a.page_tokens) / kGroupTokens
      : -1;
  if (blk >= 0) {
    // Round trip 3 (needed only at the end): the group's stored value codes,
    // for positions before s_first.  The 8D-byte block is 2D words: thread
    // tid < 2D owns word tid.
    uint8_t* vb = a.v_codes + static_cast<size_t>(blk) * 8 * D;
    const bool vword = tid < 2 * D;
    const uint32_t old_v = (s_first > 0 && vword) ? reinterpret_cast<const uint32_t*>(vb)[tid] : 0u;

    // Modalities among the new positions (every wave computes the same mask).
    uint32_t mods = 0;
#pragma unroll
    for (int m = 0; m < kModalities; ++m)
      if (__any(ms_fresh && mod_l == static_cast<uint32_t>(m))) mods |= 1u << m;
    if (tid < kGroupTokens) sm.mod[tid] = static_cast<uint8_t>(mod_l);

    // ---- keys: y = H (s * k) / sqrt(d) in fp64 (exact up to the one scaling)
    double x[CH], vv[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if constexpr (BF16) {
        const uint32_t kw = reinterpret_cast<const uint32_t*>(kin)[i >> 1];
        const uint32_t vw = reinterpret_cast<const uint32_t*>(vin)[i >> 1];
        x[i] = static_cast<double>(__uint_as_float((i & 1) ? (kw & 0xFFFF0000u) : (kw << 16))) * static_cast<double>(sg[i]);
        vv[i] = static_cast<double>(__uint_as_float((i & 1) ? (vw & 0xFFFF0000u) : (vw << 16)));
      } else {
        x[i] = static_cast<double>(reinterpret_cast<const float*>(kin)[i]) * static_cast<double>(sg[i]);
        vv[i] = static_cast<double>(reinterpret_cast<const float*>(vin)[i]);
      }
    }
    // Unnormalised Walsh-Hadamard transform of the position's D channels:
    // strides below CH inside the thread, larger strides across the 8
    // threads of the position (lanes tid ^ 1, 2, 4).
#pragma unroll
    for (int hh = 1; hh < CH; hh <<= 1) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        if (!(i & hh)) {
          const double p = x[i], q = x[i + hh];
          x[i] = p + q;
          x[i + hh] = p - q;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const double p = xor_lane<1>(x[i]);
      x[i] = (part & 1) ? (p - x[i]) : (x[i] + p);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const double p = xor_lane<2>(x[i]);
      x[i] = (part & 2) ? (p - x[i]) : (x[i] + p);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const double p = xor_lane<4>(x[i]);
      x[i] = (part & 4) ? (p - x[i]) : (x[i] + p);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      x[i] = x[i] * a.inv_sqrt_d;
      sm.u.y[cb + i][tok] = x[i];
      sm.v[cb + i][tok] = vv[i];
    }
    // Value norms: sum of squares over the thread's channels, then over the
    // 8 threads of the position.
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < CH; ++i) ss = ss + vv[i] * vv[i];
    ss = ss + xor_lane<1>(ss);
    ss = ss + xor_lane<2>(ss);
    ss = ss + xor_lane<4>(ss);
    if (part == 0) sm.n[tok] = sqrt(ss);
    __syncthreads();

    // ---- key statistics: per channel min / max over the present positions
    if (tid < D) {
      double lo = sm.u.y[tid][0], hi = lo;
#pragma unroll
      for (int t = 1; t < kGroupTokens; ++t) {
        const double yv = sm.u.y[tid][t];
        lo = t < s_end ? fmin(lo, yv) : lo;
        hi = t < s_end ? fmax(hi, yv) : hi;
      }
      const uint16_t lo16 = f64_to_f16_rne(lo), hi16 = f64_to_f16_rne(hi);
      uint16_t* st = a.k_stats + static_cast<size_t>(blk) * 2 * D;
      st[tid] = lo16;
      st[D + tid] = hi16;
      // LO and the per-channel factor (c3 - c0) / (HI - LO) (HI - LO is exact
      // in fp64); 0 marks HI == LO (every code 0).
      const double LO = static_cast<double>(f16_bits_to_f32(lo16)), HI = static_cast<double>(f16_bits_to_f32(hi16));
      sm.lohi[0][tid] = LO;
      sm.lohi[1][tid] = HI > LO ? (a.c3 - a.c0) / (HI - LO) : 0.0;
    }
    __syncthreads();

    // ---- key codes: z = c0 + (y - LO) (c3 - c0) / (HI - LO); code = thresholds
    // reached.  The division is taken once per channel; z may differ from the
    // definition's rounding order in its last bits, which can only move a
    // value lying within a few ulps of a threshold.
#pragma unroll
    for (int q4 = 0; q4 < CH / 4; ++q4) {
      uint32_t byte = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = cb + 4 * q4 + i;
        uint32_t code = 0;
        const double LO = sm.lohi[0][c], f = sm.lohi[1][c];
        if (present && f > 0.0) {
          const double z = a.c0 + (x[4 * q4 + i] - LO) * f;
          code = (z >= a.thr0 ? 1u : 0u) + (z >= a.thr1 ? 1u : 0u) + (z >= a.thr2 ? 1u : 0u);
        }
        byte |= code << (2 * i);
      }
      sm.kblk[key_code_byte<D>(tok, cb + 4 * q4)] = static_cast<uint8_t>(byte);
    }

    // ---- values: r = R_m^T v over this thread's rows [i0, i0 + IQ) of R
    // (fixed order), one modality at a time; the rows of modality mpre were
    // loaded above.
    for (int m = 0; m < kModalities; ++m) {
      if (!(mods & (1u << m))) continue;
      if (m != mpre) {
        const float* Rm = a.rot + ((static_cast<size_t>(h) * kModalities + m) * D + i0) * D + jc;
#pragma unroll
        for (int i = 0; i < IQ; ++i) rr[i] = Rm[static_cast<size_t>(i) * D];
      }
      for (int s = s_first; s < s_end; ++s) {
        if (sm.mod[s] != m) continue;
        // four interleaved partial sums, added in a fixed order
        double acc4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int i = 0; i < IQ; ++i) acc4[i & 3] = fma(static_cast<double>(rr[i]), sm.v[i0 + i][s], acc4[i & 3]);
        sm.u.r[pq][s][jc] = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
      }
    }
    __syncthreads();
    if (pq == 0) {
      for (int s = s_first; s < s_end; ++s) {
        double r = sm.u.r[0][s][jc];
#pragma unroll
        for (int p = 1; p < TQ; ++p) r = r + sm.u.r[p][s][jc];
        const double n = sm.n[s];
        uint32_t code = 0;
        if (n > 0.0 && sm.mod[s] < kModalities) {
          const double z = (a.sqrt_d * r) / n;
          code = (z >= a.thr0 ? 1u : 0u) + (z >= a.thr1 ? 1u : 0u) + (z >= a.thr2 ? 1u : 0u);
        }
        sm.code[s][jc] = static_cast<uint8_t>(code);
      }
    }
    __syncthreads();

    // ---- stores: key block, value block (earlier positions keep their
    // stored codes), norms, modality
    if (tid < D / 2) {
      uint4* dst = reinterpret_cast<uint4*>(a.k_codes + static_cast<size_t>(blk) * 8 * D);
      dst[tid] = reinterpret_cast<const uint4*>(sm.kblk)[tid];
    }
    if (vword) {
      uint32_t outw = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int byte = 4 * tid + k;
        const int L = byte / W, wi = byte % W;
        const int nt = wi >> 1, hf = wi & 1, kg = L >> 4, col = L & 15;
        const int c = nt * 16 + col;
        uint32_t out = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = hf * 16 + kg * 4 + i;
          uint32_t code;
          if (s < s_first) code = (old_v >> (8 * k + 2 * i)) & 3u;
          else if (s < s_end) code = sm.code[s][c];
          else code = 0u;
          out |= code << (2 * i);
        }
        outw |= out << (8 * k);
      }
      reinterpret_cast<uint32_t*>(vb)[tid] = outw;
    }
    if (tid < kGroupTokens && tid >= s_first && tid < s_end) {
      const int phys = static_cast<int>(blk / (static_cast<long long>(a.hkv) * (a.page_tokens / kGroupTokens)));
      const int pos = (t0 + tid) % a.page_tokens;
      a.v_norms[(static_cast<size_t>(phys) * a.hkv + h) * a.page_tokens + pos] = f64_to_f16_rne(sm.n[tid]);
      if (h == 0) a.modality[static_cast<size_t>(phys) * a.page_tokens + pos] = sm.mod[tid];
    }
  }

  // Raw keys of the new open group go to the tail; workgroup 0 is the only
  // reader of the tail and its reads are done (the barriers above).
  const int open0 = (L_new / kGroupTokens) * kGroupTokens;
  if (j == 0 && open0 < L_new) {
    const int start = max(open0, L_old);
    const int count = L_new - start;
    for (int idx = tid; idx < count * D; idx += kAppendThreads) {
      const int c = idx % D, t = start + idx / D;
      const size_t src = ((static_cast<size_t>(b) * a.n_new + (t - L_old)) * a.hkv + h) * D + c;
      const size_t dst = ((static_cast<size_t>(sb) * a.hkv + h) * kGroupTokens + (t & 31)) * D + c;
      if constexpr (BF16) {
        static_cast<uint16_t*>(a.k_tail)[dst] = static_cast<const uint16_t*>(a.k_new)[src];
      } else {
        static_cast<float*>(a.k_tail)[dst] = static_cast<const float*>(a.k_new)[src];
      }
    }
  }
  // Completion ticket of the session: the last workgroup advances seq_len
  // and rearms the ticket for the next append.
  __syncthreads();
  if (tid == 0) {
    const int total = static_cast<int>(gridDim.x * gridDim.y);
    const int t = __hip_atomic_fetch_add(&a.tickets[sb], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = (t == total - 1);
  }
  __syncthreads();
  if (sm.last && tid == 0) {
    __hip_atomic_store(&a.tickets[sb], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.seq_len[sb], L_new, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int D, bool BF16>
hipError_t launch_append_t(int nb, const AppendArgs& a, hipStream_t s) {
  const dim3 grid((a.n_new + 30) / kGroupTokens + 1, a.hkv, nb);
  hipLaunchKernelGGL((append_kernel<D, BF16>), grid, dim3(kAppendThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int d, bool bf16, int nb, const AppendArgs& a, hipStream_t s) {
  if (d == 64) return bf16 ? launch_append_t<64, true>(nb, a, s) : launch_append_t<64, false>(nb, a, s);
  return bf16 ? launch_append_t<128, true>(nb, a, s) : launch_append_t<128, false>(nb, a, s);
}

}  // namespace kvq
