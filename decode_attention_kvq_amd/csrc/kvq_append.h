// Quantize-append: keys (randomized Hadamard rotation + per-group min-max
// scaling onto the fixed codebook; or, for the TurboQuant baseline, per-token
// norm scaling) and values (per-modality rotation + norm scaling onto the
// fixed codebook), written into the lane-major 2-bit group blocks of the
// paged cache.
//
// Method: OmniKVQuant page, Sec. 2 Method (TurboQuant bullet, and the two
// OmniKVQuant bullets for keys and values).
//
// Every decision is taken in fp64.  The statistics follow the definition's
// operation order, so the stored fp16 LO / HI are exactly those of an fp64
// reference; the key codes take the division once per channel and the value
// rotation sums in a fixed order (the matrix cores' own), which can only change a code whose
// normalised value lies within a few ulps of a decision threshold.  The
// body turns floating-point contraction off, so that no operation is fused
// behind the code's back whatever the including file's setting (the
// transform's explicit fma has a +-1 factor, so it rounds exactly like the
// addition it stands for).
//
// The body (append_group) serves two kernels: the append kernel of
// kvq_append.hip and the fused decode step, where the append's workgroups
// run beside the decode partitions.  For the j-th 32-position group touched by the append of
// session b, KV head h, two workgroups run side by side: (2 j, h, b)
// re-quantizes all the group's keys (the earlier ones from the raw key tail)
// and (2 j + 1, h, b) quantizes the group's new values.  The key workgroup of
// group 0 is the only reader of the key tail, so it is also the one that
// stores the raw keys of the new open group (after its own reads).  Every
// workgroup takes a ticket when done; the last one of a session advances its
// length, so no workgroup can see the new length before it read the old one
// (the fused step defers this to its merge, and also copies the open group's
// blocks, statistics, norms and modality bytes to a record in shared memory;
// with a record, the cache writes are left to the caller, which makes them
// from the record after its last load: on this GPU one counter tracks
// loads and stores alike, so a load issued after a store is waited for
// together with it).
//
// Latency matters for the common one-position append, throughput for a
// chunk: each role issues its global loads in at most two dependent rounds,
// 16 threads share one position's channels (a short fp64 transform), the
// statistics are reduced across lanes, and the value rotation R_m^T v of all
// the group's new positions runs on the fp64 matrix cores (16 x 16 tiles of
// positions x output channels) instead of one position after another.
#pragma once

#include "kvq_common.h"
#include "kvq_internal.h"
#include "kvq_rotate.h"

namespace kvq {
namespace app {

typedef double doublex4 __attribute__((ext_vector_type(4)));

constexpr int kAppendThreads = 512;
constexpr int kPosThreads = 16;                   // threads sharing one position's channels

using rotq::butterfly;
using rotq::xor_lane;

template <int M>
__device__ __forceinline__ double lanes_sum(double x) {
  x = x + xor_lane<1>(x);
  x = x + xor_lane<2>(x);
  if constexpr (M > 4) x = x + xor_lane<4>(x);
  if constexpr (M > 8) x = x + xor_lane<8>(x);
  return x;
}

// Loads of a thread's slice of one input row (CH elements of ESZ bytes).
template <int NWORDS>
__device__ __forceinline__ void load_words(const void* p, uint32_t (&w)[NWORDS]) {
  if constexpr (NWORDS == 2) {
    const uint2 v = *static_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int k = 0; k < NWORDS / 4; ++k) {
      const uint4 v = static_cast<const uint4*>(p)[k];
      w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }
  }
}

// Element i of the slice as fp32 (exact for bf16 and fp32 inputs).
template <bool BF16, int NWORDS>
__device__ __forceinline__ uint32_t element_bits(const uint32_t (&w)[NWORDS], int i) {
  if constexpr (BF16) return (i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16);
  return w[i];
}

template <int D>
struct KeySmem {
  double y[kGroupTokens][D + 1];                  // rotated keys, one row per position (padded: the statistics
                                                  // read one channel of 8 positions per 4 lanes)
  double lohi[2][D];                              // LO and the per-channel factor
  __align__(16) uint8_t kblk[8 * D];              // the group's 2-bit key codes (lane-major)
  uint8_t code[kGroupTokens][D];                  // 3- / 4-bit key codes, one byte each
};

template <int D>
struct ValSmem {
  float v[kGroupTokens][D + 1];                   // new values (the inputs are exact in fp32); rows padded so a
                                                  // column of 16 positions spans 16 LDS banks
  double n[kGroupTokens];                         // value norms
  uint8_t code[kGroupTokens][D];                  // value codes (3- / 4-bit: also the earlier positions)
  uint8_t mod[kGroupTokens];
  uint32_t oldw[4 * D];                           // 3- / 4-bit: the group's stored value block
};

// Level index of a normalised value: the number of decision thresholds it
// reaches (the thresholds ascend; ties go up).
template <int BITS>
__device__ __forceinline__ uint32_t level_index(const AppendArgs& a, double z) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < (1 << BITS) - 1; ++i) c += z >= a.thr[i] ? 1u : 0u;
  return c;
}

// b-bit lane-major blocks (include/kvq.h): lane L owns b D / 64 words, a bit
// stream of operand units of 8 codes, code k of unit u at bit 8 b u + b k.
// Position and channel of code g (unit g / 8, k = g % 8) of lane L:
//   keys   t = 16 (u / (D/32)) + L % 16,  c = 32 (u % (D/32)) + 8 (L / 16) + k
//   values t = 16 (k / 4) + 4 (L / 16) + k % 4,  c = 16 u + L % 16
template <int D, bool VALUE>
__device__ __forceinline__ void code_slot(int lane, int g, int& t, int& c) {
  const int u = g >> 3, k = g & 7;
  if constexpr (VALUE) {
    t = 16 * (k >> 2) + 4 * (lane >> 4) + (k & 3);
    c = 16 * u + (lane & 15);
  } else {
    t = 16 * (u / (D / 32)) + (lane & 15);
    c = 32 * (u % (D / 32)) + 8 * (lane >> 4) + k;
  }
}

// Word w (of the block's b D words) of a b-bit block, from one code byte per
// (position, channel); code(t, c) gives the code of a slot.
template <int D, bool VALUE, typename F>
__device__ __forceinline__ uint32_t pack_word(int bits, int w, F code) {
  const int wpl = bits * D / 64;                 // words per lane
  const int lane = w / wpl, b0 = 32 * (w % wpl);
  uint32_t out = 0;
  for (int g = b0 / bits; g * bits < b0 + 32; ++g) {
    int t, c;
    code_slot<D, VALUE>(lane, g, t, c);
    const int sh = g * bits - b0;
    const uint32_t v = code(t, c);
    out |= sh >= 0 ? (v << sh) : (v >> -sh);
  }
  return out;
}

// Code of value slot (t, c) in a stored b-bit block (words in LDS).
template <int D>
__device__ __forceinline__ uint32_t unpack_value_code(int bits, const uint32_t* words, int t, int c) {
  const int L = 16 * ((t & 15) >> 2) + (c & 15), u = c >> 4, k = 4 * (t >> 4) + (t & 3);
  const int p = 8 * bits * u + bits * k;          // bit in the lane's stream
  const int wpl = bits * D / 64;
  const int wi = L * wpl + (p >> 5), sh = p & 31;
  uint32_t v = words[wi] >> sh;
  if (sh + bits > 32) v |= words[wi + 1] << (32 - sh);
  return v & ((1u << bits) - 1u);
}

template <int D>
union AppendSmem {
  KeySmem<D> k;
  ValSmem<D> v;
};

// The append work of one workgroup: group bx >> 1 of the append (counted
// from the session's open group) of session a.b0 + b, KV head h; keys when
// bx is even, values when odd.  All kAppendThreads threads call it together.
// sm and s_last live in the caller's shared memory; ticket_total is the
// number of workgroups of one session that take a completion ticket.
// stage: null, or (the fused decode step: one-position appends to a 2-bit
// cache with group statistics) a record in the caller's shared memory that
// receives a copy of the open group (kStage* layout).
template <int D, bool BF16, int BITS>
__device__ __forceinline__ void append_group(const AppendArgs& a, AppendSmem<D>& sm, int& s_last, int bx, int h,
                                             int b, int ticket_total, uint8_t* stage = nullptr) {
#pragma clang fp contract(off)
  constexpr int CH = D / kPosThreads;             // channels per thread (inputs, transform, key codes)
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int NWORDS = CH * ESZ / 4;
  constexpr int QR = kAppendThreads / D;          // threads per channel (statistics), parts of R's rows (values)
  constexpr int TPQ = kGroupTokens / QR;          // positions per statistics thread
  constexpr int W = D / 8;
  static_assert(kPosThreads * kGroupTokens == kAppendThreads, "one thread per (position, slice)");
  const int tid = threadIdx.x;
  const int j = bx >> 1;
  const bool vrole = bx & 1;
  const int sb = a.b0 + b;
  const int lane = tid & 63;
  const int tok = tid / kPosThreads, part = tid % kPosThreads, cb = part * CH;

  // Round trip 1: every load that needs only the kernel arguments, issued
  // together and without branching on the role (a branch would make the
  // compiler wait for one role's loads before the next ones): the signs of
  // channels cb.. (the key transform), the modalities of every new position
  // the group could hold (rows [32 j - 32, 32 j + 32) of the append,
  // whatever the old length: they pick the rotation rows the value
  // workgroup prefetches), and the session length.  A one-position append
  // (the decode step) also reads its input rows here: row tok of the raw
  // tail and the new row (key workgroup: position tok of the open group is
  // one of the two), or the new row (value workgroup).  Longer appends read
  // theirs once the length has placed the group.
  const bool one = a.n_new == 1;
  uint32_t sgw[CH / 4];
#pragma unroll
  for (int k = 0; k < CH / 4; ++k) sgw[k] = reinterpret_cast<const uint32_t*>(a.signs + h * D + cb)[k];
  const int widx = 32 * j - 32 + lane;
  const bool wok = widx >= 0 && widx < a.n_new;
  const uint32_t wmod = a.modality_new[static_cast<size_t>(b) * a.n_new + min(max(widx, 0), a.n_new - 1)];
  uint32_t w_tail[NWORDS], w_one[NWORDS];
  if (one) {
    const char* tail_row = static_cast<const char*>(a.k_tail) +
                           (((static_cast<size_t>(sb) * a.hkv + h) * kGroupTokens + tok) * D + cb) * ESZ;
    const char* new_row = static_cast<const char*>(vrole ? a.v_new : a.k_new) +
                          ((static_cast<size_t>(b) * a.hkv + h) * D + cb) * ESZ;
    load_words(tail_row, w_tail);
    load_words(new_row, w_one);
  }
  const int L_old = a.seq_len[sb];
  int mpre = 0;
  if (vrole) {
    uint32_t wmods = 0;
#pragma unroll
    for (int m = 0; m < kModalities; ++m)
      if (__any(wok && wmod == static_cast<uint32_t>(m))) wmods |= 1u << m;
    mpre = wmods ? __builtin_ctz(wmods) : 0;
  }

  // Round trip 2: the page table, the inputs of a longer append, and (values)
  // the prefetched rotation rows.  The arithmetic does not wait for the
  // page: only the stores (and the read of the group's earlier value codes)
  // need it, so a group on an unmapped page is computed and dropped.
  const int L_new = L_old + a.n_new;
  const int t0 = (L_old / kGroupTokens + j) * kGroupTokens;
  const bool active = t0 < L_new;
  const int s_first = max(L_old - t0, 0);        // first new position of the group
  const int s_end = min(kGroupTokens, L_new - t0);
  const bool present = tok < s_end;
  const int inew = min(max(t0 + tok - L_old, 0), a.n_new - 1);   // clamped row of k_new / v_new
  // A longer append's input row (position tok of the group: the raw tail's
  // row or row inew of the new keys; row inew of the new values), issued
  // before the page entry so that waiting for it never waits for the page.
  uint32_t w_in[NWORDS];
  if (!one) {
    const char* row = vrole
        ? static_cast<const char*>(a.v_new) + (((static_cast<size_t>(b) * a.n_new + inew) * a.hkv + h) * D + cb) * ESZ
        : (t0 + tok < L_old)
            ? static_cast<const char*>(a.k_tail) + (((static_cast<size_t>(sb) * a.hkv + h) * kGroupTokens + tok) * D + cb) * ESZ
            : static_cast<const char*>(a.k_new) + (((static_cast<size_t>(b) * a.n_new + inew) * a.hkv + h) * D + cb) * ESZ;
    load_words<NWORDS>(row, w_in);
  }
  const int page = t0 / a.page_tokens;
  const int pt_raw = a.page_table[static_cast<size_t>(sb) * a.max_pages + min(page, a.max_pages - 1)];
  // The group's block (-1: not stored), formed where it is first needed so
  // that the wait for the page entry comes as late as possible.
  auto phys_of = [&]() { return (active && page < a.max_pages) ? __builtin_amdgcn_readfirstlane(pt_raw) : -1; };
  auto block_of = [&](int phys) -> long long {
    return (active && phys >= 0 && phys < a.num_pages)
        ? (static_cast<long long>(phys) * a.hkv + h) * (a.page_tokens / kGroupTokens) + (t0 % a.page_tokens) / kGroupTokens
        : -1;
  };

  // The key block of the group: 2 bits as built in LDS, wider codes packed
  // from one byte per code.
  auto store_key_block = [&](long long blk_) {
    if (BITS == 2) {
      if (tid < D / 2) {
        const uint4 v = reinterpret_cast<const uint4*>(sm.k.kblk)[tid];
        if (stage) reinterpret_cast<uint4*>(stage + kStageCodes)[tid] = v;
        else reinterpret_cast<uint4*>(a.k_codes + static_cast<size_t>(blk_) * 8 * D)[tid] = v;
      }
    } else {
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.k_codes + static_cast<size_t>(blk_) * 4 * BITS * D);
      for (int w = tid; w < BITS * D; w += kAppendThreads)
        dst[w] = pack_word<D, false>(BITS, w, [&](int t, int c) { return static_cast<uint32_t>(sm.k.code[t][c]); });
    }
  };

  if (!vrole) {
    // ================= keys =================
    uint32_t kw[NWORDS];
    const bool from_tail = t0 + tok < L_old;
#pragma unroll
    for (int i = 0; i < NWORDS; ++i) kw[i] = !one ? w_in[i] : from_tail ? w_tail[i] : w_one[i];

    {
      // ---- y = H (s * k) / sqrt(d) in fp64 (exact up to the one scaling).
      // Channel c = part * CH + i: the transform over i runs inside the
      // thread, the one over part across the 16 lanes of the position.
      double x[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        // the sign is +-1: flip the fp32 sign bit where it is negative
        const uint32_t sbit = ((sgw[i >> 2] >> (8 * (i & 3))) & 0x80u) << 24;
        x[i] = static_cast<double>(__uint_as_float(element_bits<BF16>(kw, i) ^ sbit));
      }
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
      for (int i = 0; i < CH; ++i) x[i] = butterfly<1>(x[i], (part & 1) ? -1.0 : 1.0);
#pragma unroll
      for (int i = 0; i < CH; ++i) x[i] = butterfly<2>(x[i], (part & 2) ? -1.0 : 1.0);
#pragma unroll
      for (int i = 0; i < CH; ++i) x[i] = butterfly<4>(x[i], (part & 4) ? -1.0 : 1.0);
#pragma unroll
      for (int i = 0; i < CH; ++i) x[i] = butterfly<8>(x[i], (part & 8) ? -1.0 : 1.0);
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        x[i] = x[i] * a.inv_sqrt_d;
        sm.k.y[tok][cb + i] = x[i];
      }
      __syncthreads();
      const long long blk = block_of(phys_of());
      if (stage && tid == 0) {
        int* meta = reinterpret_cast<int*>(stage + kStageMeta);
        meta[0] = blk >= 0 ? 1 : 0;   // blocks stored (the page is mapped)
        meta[1] = s_end;              // positions of the group
        meta[2] = t0;                 // its first position
        meta[3] = s_first;            // its first new position
        meta[4] = phys_of();
        *reinterpret_cast<long long*>(stage + kStageBlock) = blk;
      }

      if (a.key_mode == KVQ_KEYS_PER_TOKEN) {
        // ---- per-token keys (TurboQuant): n = ||k|| (squares over the
        // thread's channels, then across the 16 lanes of the position, as for
        // the values), z = sqrt(d) y / n, nearest level; the norms go to the
        // first 32 entries of the group's statistics block.
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const double f = static_cast<double>(__uint_as_float(element_bits<BF16>(kw, i)));
          ss = ss + f * f;
        }
        ss = lanes_sum<kPosThreads>(ss);
        const double n = sqrt(ss);
#pragma unroll
        for (int q4 = 0; q4 < CH / 4; ++q4) {
          uint32_t byte = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t code = 0;
            if (present && n > 0.0) {
              const double z = (a.sqrt_d * x[4 * q4 + i]) / n;
              code = level_index<BITS>(a, z);
            }
            byte |= code << (2 * i);
            if (BITS != 2) sm.k.code[tok][cb + 4 * q4 + i] = static_cast<uint8_t>(code);
          }
          if (BITS == 2) sm.k.kblk[key_code_byte<D>(tok, cb + 4 * q4)] = static_cast<uint8_t>(byte);
        }
        if (part == 0 && blk >= 0) a.k_stats[static_cast<size_t>(blk) * 2 * D + tok] = present ? f64_to_f16_rne(n) : uint16_t(0);
        __syncthreads();
        if (blk >= 0) store_key_block(blk);
      } else {

      // ---- statistics: per channel min / max over the present positions;
      // QR threads per channel each take TPQ positions, then combine across
      // lanes (min / max are exact in any order).
      {
        const int c = tid / QR, q = tid % QR;
        double lo = __builtin_inf(), hi = -__builtin_inf();
#pragma unroll
        for (int k = 0; k < TPQ; ++k) {
          const int t = q * TPQ + k;
          const double yv = sm.k.y[t][c];
          lo = t < s_end ? fmin(lo, yv) : lo;
          hi = t < s_end ? fmax(hi, yv) : hi;
        }
        lo = fmin(lo, xor_lane<1>(lo));
        hi = fmax(hi, xor_lane<1>(hi));
        lo = fmin(lo, xor_lane<2>(lo));
        hi = fmax(hi, xor_lane<2>(hi));
        if constexpr (QR > 4) {
          lo = fmin(lo, xor_lane<4>(lo));
          hi = fmax(hi, xor_lane<4>(hi));
        }
        if (q == 0) {
          const uint16_t lo16 = f64_to_f16_rne(lo), hi16 = f64_to_f16_rne(hi);
          if (blk >= 0) {
            uint16_t* st = stage ? reinterpret_cast<uint16_t*>(stage + kStageCodes + 16 * D)
                                 : a.k_stats + static_cast<size_t>(blk) * 2 * D;
            st[c] = lo16;
            st[D + c] = hi16;
          }
          // LO and the per-channel factor (c3 - c0) / (HI - LO) (HI - LO is
          // exact in fp64); 0 marks HI == LO (every code 0).
          const double LO = static_cast<double>(f16_bits_to_f32(lo16)), HI = static_cast<double>(f16_bits_to_f32(hi16));
          sm.k.lohi[0][c] = LO;
          sm.k.lohi[1][c] = HI > LO ? (a.cmax - a.c0) / (HI - LO) : 0.0;
        }
      }
      __syncthreads();

      // ---- key codes: z = c0 + (y - LO) (c3 - c0) / (HI - LO); code =
      // thresholds reached.  The division is taken once per channel; z may
      // differ from the definition's rounding order in its last bits, which
      // can only move a value lying within a few ulps of a threshold.
#pragma unroll
      for (int q4 = 0; q4 < CH / 4; ++q4) {
        uint32_t byte = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = cb + 4 * q4 + i;
          uint32_t code = 0;
          const double LO = sm.k.lohi[0][c], f = sm.k.lohi[1][c];
          if (present && f > 0.0) {
            const double z = a.c0 + (x[4 * q4 + i] - LO) * f;
            code = level_index<BITS>(a, z);
          }
          byte |= code << (2 * i);
          if (BITS != 2) sm.k.code[tok][c] = static_cast<uint8_t>(code);
        }
        if (BITS == 2) sm.k.kblk[key_code_byte<D>(tok, cb + 4 * q4)] = static_cast<uint8_t>(byte);
      }
      __syncthreads();
      if (blk >= 0) store_key_block(blk);
      }   // group min-max keys
    }

    // Raw keys of the new open group go to the tail; the key workgroup of
    // group 0 is the only reader of the tail and its reads are done (their
    // values were used above).
    const int open0 = (L_new / kGroupTokens) * kGroupTokens;
    if (!stage && j == 0 && open0 < L_new) {
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
  } else {
    // ================= values =================
    uint32_t vw[NWORDS];
#pragma unroll
    for (int i = 0; i < NWORDS; ++i) vw[i] = one ? w_one[i] : w_in[i];
    const int ms = lane & 31;                      // this lane's modality slot
    const bool ms_fresh = ms >= s_first && ms < s_end;
    const uint32_t mod_l = a.modality_new[static_cast<size_t>(b) * a.n_new + min(max(t0 + ms - L_old, 0), a.n_new - 1)];
    // Rotation on the fp64 matrix cores (v_mfma_f64_16x16x4f64): a tile of 16
    // positions x 16 output channels, D[s][c] = sum_i v[s][i] R[i][c], sums
    // over D / 4 steps of 4 rows.  Wavefront w takes channel tile w % NTC
    // (and, with fewer channel tiles than wavefronts, position tile w / NTC);
    // at step k lane l holds B = R[4k + l/16][16 nt + l%16] and
    // A = v[16 mt + l%16][4k + l/16], and the tile's results
    // D[16 mt + 4r + l/16][16 nt + l%16], r < 4.  The rows of modality mpre
    // are loaded here, with the other round-trip-2 loads.
    constexpr int NTC = D / 16;                    // channel tiles
    constexpr int KS = D / 4;                      // steps of 4 rows
    const int wv = tid >> 6;
    const int c_out = 16 * (wv % NTC) + (lane & 15);
    float rb[KS];
    auto load_rot = [&](int m) {
      const float* Rm = a.rot + (static_cast<size_t>(h) * kModalities + m) * D * D + c_out;
#pragma unroll
      for (int k = 0; k < KS; ++k) rb[k] = Rm[static_cast<size_t>(4 * k + (lane >> 4)) * D];
    };
    load_rot(mpre);
    const int phys = phys_of();
    const long long blk = block_of(phys);
    // Round trip 3 (needed only at the end): the group's stored value codes,
    // for positions before s_first.  The 8D-byte block is 2D words: thread
    // tid < 2D owns word tid.
    const bool stored = blk >= 0;
    uint8_t* vb = a.v_codes + static_cast<size_t>(stored ? blk : 0) * 4 * BITS * D;
    const bool vword = BITS == 2 && tid < 2 * D;
    const uint32_t old_v = (stored && s_first > 0 && vword) ? reinterpret_cast<const uint32_t*>(vb)[tid] : 0u;
    if (BITS != 2 && stored && s_first > 0)
      for (int w = tid; w < BITS * D; w += kAppendThreads) sm.v.oldw[w] = reinterpret_cast<const uint32_t*>(vb)[w];
    // The staging record takes every position's norm and modality byte: the
    // earlier positions' from the cache.
    uint16_t old_n = 0;
    uint8_t old_m = 0;
    if (stage && stored && tid < s_first) {
      const int pos = (t0 + tid) % a.page_tokens;
      old_n = a.v_norms[(static_cast<size_t>(phys) * a.hkv + h) * a.page_tokens + pos];
      old_m = a.modality[static_cast<size_t>(phys) * a.page_tokens + pos];
    }

    // Modalities among the new positions (every wave computes the same mask).
    uint32_t mods = 0;
#pragma unroll
    for (int m = 0; m < kModalities; ++m)
      if (__any(ms_fresh && mod_l == static_cast<uint32_t>(m))) mods |= 1u << m;
    if (tid < kGroupTokens) sm.v.mod[tid] = static_cast<uint8_t>(mod_l);

    // Inputs to LDS, and the norms: sum of squares over the thread's
    // channels, then over the 16 threads of the position.
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const float f = __uint_as_float(element_bits<BF16>(vw, i));
      sm.v.v[tok][cb + i] = f;
      ss = ss + static_cast<double>(f) * static_cast<double>(f);
    }
    ss = lanes_sum<kPosThreads>(ss);
    if (part == 0) sm.v.n[tok] = sqrt(ss);
    __syncthreads();
    // 3- / 4-bit: the earlier positions' codes, out of the stored block
    if (BITS != 2)
      for (int e = tid; e < s_first * D; e += kAppendThreads)
        sm.v.code[e / D][e % D] = static_cast<uint8_t>(unpack_value_code<D>(BITS, sm.v.oldw, e / D, e % D));

    // ---- r = R_m^T v on the matrix cores, one modality at a time, over the
    // position tiles that hold new positions.  Each output sums its D exact
    // products (bf16 or fp32 times fp32) in fp64 in one fixed order whatever
    // the tile's other rows hold (rows of positions that are not new are
    // computed from stale data and dropped), so a position's code does not
    // depend on how the stream was chunked.
    const int mt_lo = s_first >> 4, mt_hi = (s_end - 1) >> 4;
    constexpr int MT0 = NTC < 8 ? 8 / NTC : 1;     // wavefronts per channel tile
    for (int m = 0; m < kModalities; ++m) {
      if (!(mods & (1u << m))) continue;
      if (m != mpre) load_rot(m);
      for (int mt = mt_lo + wv / NTC; mt <= mt_hi; mt += MT0) {
        doublex4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          const double av = static_cast<double>(sm.v.v[16 * mt + (lane & 15)][4 * k + (lane >> 4)]);
          // (opaque, so that the 32 conversions are not hoisted out of the
          // tile loop as 64 more live registers)
          float rk = rb[k];
          asm volatile("" : "+v"(rk));
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, static_cast<double>(rk), acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 16 * mt + 4 * r + (lane >> 4);
          if (s >= s_first && s < s_end && sm.v.mod[s] == m) {
            const double n = sm.v.n[s];
            uint32_t code = 0;
            if (n > 0.0) {
              const double z = (a.sqrt_d * acc[r]) / n;
              code = level_index<BITS>(a, z);
            }
            sm.v.code[s][c_out] = static_cast<uint8_t>(code);
          }
        }
      }
    }
    __syncthreads();

    // ---- stores: value block (earlier positions keep their stored codes;
    // a position with a modality outside the known ones gets code 0), norms,
    // modality
    if (stored && vword) {
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
          else if (s < s_end) code = sm.v.mod[s] < kModalities ? sm.v.code[s][c] : 0u;
          else code = 0u;
          out |= code << (2 * i);
        }
        outw |= out << (8 * k);
      }
      if (stage) reinterpret_cast<uint32_t*>(stage + kStageCodes + 8 * D)[tid] = outw;
      else reinterpret_cast<uint32_t*>(vb)[tid] = outw;
    }
    if (BITS != 2 && stored && !stage) {
      auto vcode = [&](int t, int c) -> uint32_t {
        if (t < s_first) return sm.v.code[t][c];
        if (t < s_end) return sm.v.mod[t] < kModalities ? sm.v.code[t][c] : 0u;
        return 0u;
      };
      for (int w = tid; w < BITS * D; w += kAppendThreads)
        reinterpret_cast<uint32_t*>(vb)[w] = pack_word<D, true>(BITS, w, vcode);
    }
    if (!stage && stored && tid < kGroupTokens && tid >= s_first && tid < s_end) {
      const int pos = (t0 + tid) % a.page_tokens;
      a.v_norms[(static_cast<size_t>(phys) * a.hkv + h) * a.page_tokens + pos] = f64_to_f16_rne(sm.v.n[tid]);
      if (h == 0) a.modality[static_cast<size_t>(phys) * a.page_tokens + pos] = sm.v.mod[tid];
    }
    if (stage && stored && tid < kGroupTokens) {
      const bool fresh = tid >= s_first && tid < s_end;
      reinterpret_cast<uint16_t*>(stage + kStageNorms)[tid] =
          tid < s_first ? old_n : fresh ? f64_to_f16_rne(sm.v.n[tid]) : uint16_t(0);
      stage[kStageMods + tid] = tid < s_first ? old_m : fresh ? sm.v.mod[tid] : uint8_t(0);
    }
  }

  // Completion ticket of the session: the last workgroup advances seq_len
  // and rearms the ticket for the next append.  The only order needed is
  // that every workgroup's read of seq_len precedes the last workgroup's
  // store: each workgroup used that value (waited for it) before this
  // barrier and its ticket, so relaxed atomics suffice.  The cache writes
  // need no release here: the next kernel starts after this one completes.
  if (a.defer_len) return;   // the caller advances the length
  __syncthreads();
  if (tid == 0) {
    const int t = __hip_atomic_fetch_add(&a.tickets[sb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (t == ticket_total - 1);
  }
  __syncthreads();
  if (s_last && tid == 0) {
    __hip_atomic_store(&a.tickets[sb], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.seq_len[sb], L_new, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace app
}  // namespace kvq
