// Fused decode attention over the 2-bit packed cache (OmniKVQuant page,
// Sec. 1 Introduction, Implementation bullet; Abstract): the codes are
// unpacked inside attention, scores use the already-rotated query, values are
// aggregated per modality in their rotated frames, and the inverse value
// rotations are applied once per modality after aggregation.  No dense key or
// value is ever written.
//
// Partition kernel (one workgroup = NW wavefronts = one context partition of
// one (session, KV head)).  Each wavefront takes one 32-position group at a
// time and serves all G <= 16 query heads of the KV head on the matrix cores
// (v_mfma_f32_16x16x32_f16):
//
//   codes -> fp16 operands through a 256-entry byte table in LDS (a copy per
//            lane pair of banks, so lookups never conflict): one byte of four
//            2-bit codes becomes four centred levels
//            l = (2 c - c0 - c3) / (c3 - c0) in [-1, 1];
//   keys    k_hat = mid + half * l with mid/half = (HI +- LO) / 2 per channel;
//   scores  S^T[t][i] = sum_c mid_c q_ic + sum_c l_tc (q_ic half_c): rows = 16
//           positions, columns = 16 query heads; the first sum from the stored
//           fp16 LO/HI rows, the second with q~ = q * half split in two fp16
//           halves, so the scores keep fp32-level accuracy;
//   softmax online, base 2, per query head;
//   values  A_m^T[c][.] += sum_t l_tc w_t (w = p * N_t): rows = 16 channels,
//           columns = (modality slot, query head) pairs.  With G <= 5 the
//           three modalities share one accumulator set, with G <= 8 two sets,
//           else three: the score result already sits in the operand layout,
//           and slot columns take their head's weights by a DPP row shift.
// Value levels are c = cmid + chalf * l; sum_t w_t per modality is also kept
// when the codebook is not symmetric (cmid != 0).
//
// Merge kernel: workgroups of (session, query head, block of output rows)
// rescale and sum the partitions and apply the three R_m in a fixed order
// (bitwise reproducible).
#include <type_traits>

#include "kvq_append.h"
#include "kvq_common.h"
#include "kvq_internal.h"
#include "kvq_rotate.h"

namespace kvq {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTabCopies = 32;     // byte-table copies: lane l reads copy l % 32
constexpr float kLazyMax = 8.f;    // headroom (base-2 units) of the softmax reference max
// Value weights p * N are fp16 matrix-core operands.  They are formed as
// 2^(s - m_run + wshift) * N with wshift = kWeightExp + 14 - nE, where every
// norm N seen so far is below 2^(nE - 14): the weights stay below
// 2^kWeightExp (fp16 overflows at 2^16) and the largest ones far above the
// fp16 subnormal range, whatever the scale of the values.  The factor is a
// shift of the softmax reference (the partial stores m_run - wshift), so it
// cancels in the output.
constexpr int kWeightExp = 15;
constexpr int kPageRun = kPartitionPages;   // page-table entries of one partition kept in LDS
constexpr int kMaxSplits = 4096;

__device__ __forceinline__ floatx4 mfma(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Four fp16 levels of the four 2-bit codes of one byte of `word`.
__device__ __forceinline__ uint2 lookup(const uint2* tab, uint32_t word, uint32_t sel, uint32_t lane_off) {
  // v_perm_b32: result byte 0 = lane offset, byte 1 = the code byte, bytes 2..3 = 0
  const uint32_t off = __builtin_amdgcn_perm(word, lane_off, sel);
  return *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(tab) + off);
}

__device__ __forceinline__ half8 as_half8(uint2 lo, uint2 hi) {
  uint4 v;
  v.x = lo.x;
  v.y = lo.y;
  v.z = hi.x;
  v.w = hi.y;
  return __builtin_bit_cast(half8, v);
}

// Selector placing byte j (0..3) of the first operand at result byte 1.
__device__ __forceinline__ constexpr uint32_t byte_sel(int j) { return 0x0C0C0000u | ((4u + j) << 8); }

// Within each row of 16 lanes, lanes >= S take the value of lane - S.
template <int S>
__device__ __forceinline__ uint32_t row_shr(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v),
                                                           0x110 + S, 0xF, 0xF, false));
}

// Modality slots: the 16 value-accumulator columns are split into SLOTS slots
// of GP columns; column c of set k holds head c % GP of modality k*SLOTS + c/GP.
template <int SLOTS>
struct Slots {
  static constexpr int GP = SLOTS == 1 ? 16 : (SLOTS == 2 ? 8 : 5);
  static constexpr int NSETS = (kModalities + SLOTS - 1) / SLOTS;
};

// Moves a value of score column (col % GP) to value column col.
template <int SLOTS>
__device__ __forceinline__ uint32_t to_value_column(uint32_t v) {
  constexpr int GP = Slots<SLOTS>::GP;
  if constexpr (SLOTS == 2) return row_shr<GP>(v, v);
  if constexpr (SLOTS == 3) return row_shr<2 * GP>(row_shr<GP>(v, v), v);
  return v;
}

template <int D>
struct GroupLoad {
  uint32_t kc[D / 32];   // lane-major key codes (D/8 bytes)
  uint32_t vc[D / 32];   // lane-major value codes
  uint32_t st[D / 64];   // this lane's share of the LO/HI rows (4D bytes per group)
  uint2 nrm0, nrm1;      // fp16 norms of positions 4kg..4kg+3 and 16+4kg..16+4kg+3
  uint32_t md0, md1;     // modality bytes of the same positions
};

// Page of position t >= 0 and its index inside the page: a shift and a mask
// when page_tokens is a power of two (the common case), else a division.
__device__ __forceinline__ int page_of(const DecodeArgs& a, int t) {
  if (a.page_shift >= 0) return t >> a.page_shift;
  return static_cast<int>(static_cast<unsigned>(t) / static_cast<unsigned>(a.page_tokens));
}
__device__ __forceinline__ int in_page(const DecodeArgs& a, int t) {
  if (a.page_shift >= 0) return t & (a.page_tokens - 1);
  return static_cast<int>(static_cast<unsigned>(t) % static_cast<unsigned>(a.page_tokens));
}

// Physical page of logical page pg (>= page0) of session b: from the
// partition's page run in LDS (its first `run` entries were loaded) when it
// lies inside it, else from the page
// table in global memory through scalar loads.  The second case only arises
// for the last partition of a session that grew on the device after the plan
// was made (a captured decode replayed while appends advance the length); it
// is slower, never wrong.  -1 past the end of the table.
__device__ __forceinline__ int phys_page(const DecodeArgs& a, const int* s_pt, int run, int b, int page0, int pg) {
  const int i = pg - page0;
  if (i < run) return __builtin_amdgcn_readfirstlane(s_pt[i]);
  if (pg >= a.max_pages) return -1;
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)(a.page_table);
  return ptab[static_cast<size_t>(b) * a.max_pages + pg];
}

// Where this workgroup's partition sits in the plan (DecodeArgs): its
// session b, its index `split` in the session, the session's partition count
// n and first partial slot slot0, and the partition's planned positions
// [tb, tend) (the last partition of a session takes every position past it).
struct Place {
  int b, split, n, slot0, tb, tend;
};
__device__ __forceinline__ Place place_of(const DecodeArgs& a) {
  Place p;
  int tokens, extra;
  if (a.ntab > 0) {
    const int x = blockIdx.x;
    int lo = 0, hi = a.ntab - 1;   // the last session whose slots start at or before x
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tab_start[mid] <= x) lo = mid;
      else hi = mid - 1;
    }
    p.b = lo;
    p.slot0 = a.tab_start[lo];
    p.n = a.tab_start[lo + 1] - p.slot0 - a.step;
    p.split = x - p.slot0;
    tokens = a.tab_tokens[lo];
    extra = a.tab_extra[lo];
  } else {
    p.b = blockIdx.z;
    p.slot0 = p.b * (a.splits + a.step);
    p.n = a.splits;
    p.split = blockIdx.x;
    tokens = a.split_tokens;
    extra = a.split_extra;
  }
  p.tb = p.split * tokens + kGroupTokens * min(p.split, extra);
  p.tend = p.tb + tokens + (p.split < extra ? kGroupTokens : 0);
  return p;
}

// Positions of session b the decode may attend: its device length, bounded
// by the capacity of its page-table row.
__device__ __forceinline__ int session_length(const DecodeArgs& a, int b) {
  return min(a.seq_len[b], a.max_pages * a.page_tokens);
}

// Issues the loads of the group at position t0 (on physical page phys0)
// without branching, so the compiler can count outstanding loads exactly: a
// group outside [0, te) or on an unmapped page reads page 0 instead and is
// flagged invalid.
template <int D>
__device__ __forceinline__ void load_group(const DecodeArgs& a, int h, int t0, int te, int lane, int kg,
                                           int phys0, GroupLoad<D>& g, bool& ok) {
  const int page = page_of(a, t0);
  ok = t0 < te && page < a.max_pages && phys0 >= 0 && phys0 < a.num_pages;
  const int phys = ok ? phys0 : 0;
  const int gp = a.page_tokens / kGroupTokens;
  const int tin = ok ? in_page(a, t0) : 0;
  const size_t blk = (static_cast<size_t>(phys) * a.hkv + h) * gp + tin / kGroupTokens;
  const uint32_t* kp = reinterpret_cast<const uint32_t*>(a.k_codes + blk * 8 * D) + lane * (D / 32);
  const uint32_t* vp = reinterpret_cast<const uint32_t*>(a.v_codes + blk * 8 * D) + lane * (D / 32);
  if constexpr (D == 128) {
    const uint4 k4 = *reinterpret_cast<const uint4*>(kp);
    const uint4 v4 = *reinterpret_cast<const uint4*>(vp);
    g.kc[0] = k4.x; g.kc[1] = k4.y; g.kc[2] = k4.z; g.kc[3] = k4.w;
    g.vc[0] = v4.x; g.vc[1] = v4.y; g.vc[2] = v4.z; g.vc[3] = v4.w;
    const uint2 s2 = reinterpret_cast<const uint2*>(a.k_stats + blk * 2 * D)[lane];
    g.st[0] = s2.x; g.st[1] = s2.y;
  } else {
    const uint2 k2 = *reinterpret_cast<const uint2*>(kp);
    const uint2 v2 = *reinterpret_cast<const uint2*>(vp);
    g.kc[0] = k2.x; g.kc[1] = k2.y;
    g.vc[0] = v2.x; g.vc[1] = v2.y;
    g.st[0] = reinterpret_cast<const uint32_t*>(a.k_stats + blk * 2 * D)[lane];
  }
  const uint16_t* np = a.v_norms + (static_cast<size_t>(phys) * a.hkv + h) * a.page_tokens + tin;
  g.nrm0 = *reinterpret_cast<const uint2*>(np + 4 * kg);
  g.nrm1 = *reinterpret_cast<const uint2*>(np + 16 + 4 * kg);
  const uint8_t* mp = a.modality + static_cast<size_t>(phys) * a.page_tokens + tin;
  g.md0 = *reinterpret_cast<const uint32_t*>(mp + 4 * kg);
  g.md1 = *reinterpret_cast<const uint32_t*>(mp + 16 + 4 * kg);
}

// Per-wavefront running state of one partition.
template <int D, int SLOTS, bool ASYM>
struct WaveState {
  static constexpr int NSETS = Slots<SLOTS>::NSETS;
  float m_run;                      // running max (base 2) of this lane's score head
  float l_run;                      // this lane's share of the softmax denominator (scaled like the weights)
  int nE;                           // norm reference: every value norm seen is below 2^(nE - 14) (wave-uniform)
  float wshift;                     // kWeightExp + 14 - nE: the weights carry the factor 2^wshift
  floatx4 acc[NSETS][D / 16];       // value accumulators (columns = slot/head pairs)
  floatx4 accs[ASYM ? NSETS : 1];   // sum of weights per column (non-symmetric codebook)
  int mask;                         // modalities that received weight
};

__device__ __forceinline__ int group_pos(int kg, int i) { return (i < 4) ? (4 * kg + i) : (16 + 4 * kg + i - 4); }

// Byte-table entry e: the fp16 levels of the four 2-bit codes in e (code i
// in bits 2i..2i+1), level k read from bytes 2k, 2k + 1 of {t1 : t0} by
// byte permutes.
__device__ __forceinline__ uint2 tab_entry(uint32_t e, uint32_t t0, uint32_t t1) {
  const uint32_t s0 = (e & 3u) * 0x0202u + ((e >> 2) & 3u) * 0x02020000u + 0x01000100u;
  const uint32_t s1 = ((e >> 4) & 3u) * 0x0202u + (e >> 6) * 0x02020000u + 0x01000100u;
  return uint2{__builtin_amdgcn_perm(t1, t0, s0), __builtin_amdgcn_perm(t1, t0, s1)};
}

// max(E, 1) over the fp16 exponent fields E of a group's 32 value norms
// (norms are >= 0, so their bit patterns order like their values); lanes of
// a row hold the same 8 norms, the four rows hold the group's 32.  keep = the
// number of leading positions of the group that hold data (later slots may
// hold anything and are left out).  Wave-uniform result.
__device__ __forceinline__ int group_norm_exponent(uint2 n0, uint2 n1, int kg, int keep) {
  const uint32_t w[4] = {n0.x, n0.y, n1.x, n1.y};
  uint32_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p0 = (r < 2 ? 4 * kg : 16 + 4 * kg) + 2 * (r & 1);   // positions of the two halves
    const uint32_t lo = p0 < keep ? (w[r] & 0x7FFFu) : 0u;
    const uint32_t hi = p0 + 1 < keep ? ((w[r] >> 16) & 0x7FFFu) : 0u;
    m = max(m, max(lo, hi));
  }
  const int e = static_cast<int>(m >> 10);
  const int e01 = max(__builtin_amdgcn_readlane(e, 0), __builtin_amdgcn_readlane(e, 16));
  const int e23 = max(__builtin_amdgcn_readlane(e, 32), __builtin_amdgcn_readlane(e, 48));
  return max(max(e01, e23), 1);
}

// Modality bits of accumulator set k (modalities k SLOTS .. k SLOTS + SLOTS - 1).
template <int SLOTS>
__device__ __forceinline__ int set_bits(int k) {
  return (((1 << SLOTS) - 1) << (k * SLOTS)) & ((1 << kModalities) - 1);
}

// OR of a small per-lane bit set over the wavefront, one ballot per bit
// (an LDS atomic with a per-lane operand would be serialised lane by lane).
__device__ __forceinline__ int wave_or_bits(int bits) {
  int r = 0;
#pragma unroll
  for (int m = 0; m < kModalities; ++m) r |= (__ballot((bits >> m) & 1) != 0ull) ? (1 << m) : 0;
  return r;
}

// Exact fp32 difference of fp16 fields (low or high half) of two registers.
__device__ __forceinline__ float f16_diff_lo(uint32_t a2, uint32_t b2) {
  float d;
  asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,1]" : "=v"(d) : "v"(a2), "v"(b2));
  return d;
}
__device__ __forceinline__ float f16_diff_hi(uint32_t a2, uint32_t b2) {
  float d;
  asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(a2), "v"(b2));
  return d;
}

// q * d (fp32 operands) split into fp16 hi + lo for two channels at once:
// hi = fp16(q d), lo = fp16(q d - hi), so that hi + lo equals q d to about
// 2^-22 relative.  Returns {hi pair, lo pair}.
__device__ __forceinline__ uint2 split_product(float q0, float d0, float q1, float d1) {
  uint32_t hi, lo;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0\n\t"
      "v_fma_mixhi_f16 %0, %3, %4, 0"
      : "=&v"(hi) : "v"(q0), "v"(d0), "v"(q1), "v"(d1));
  asm("v_fma_mixlo_f16 %0, %1, %2, -%5 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %3, %4, -%5 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(lo) : "v"(q0), "v"(d0), "v"(q1), "v"(d1), "v"(hi));
  return uint2{hi, lo};
}

// fp16 pair {p0 * n.lo, p1 * n.hi} from fp32 p and a register holding two fp16 norms.
__device__ __forceinline__ uint32_t weight_pair(float p0, float p1, uint32_t n2) {
  uint32_t w;
  asm("v_fma_mixlo_f16 %0, %1, %3, 0 op_sel_hi:[0,1,0]\n\t"
      "v_fma_mixhi_f16 %0, %2, %3, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
      : "=&v"(w) : "v"(p0), "v"(p1), "v"(n2));
  return w;
}

// Max / sum over the four rows (kg) of a wavefront for each of the 16
// columns, with the permlane swaps (no LDS).  Every lane gets the result.
__device__ __forceinline__ float rows_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Query operands of a lane (score column col, row group kg), constant over
// the partition: q * scale * log2(e) / 2 on the lane's channels
// 32 kt + 8 kg + i in fp32, and the operand of the group-bias product.  With
// G <= 8 (BHL) the bias operand holds q's fp16 hi part in columns 0..7 and its
// lo part in columns 8..15, so one product per statistics row covers both;
// otherwise hi and lo are separate operands.
template <int D, bool BHL>
struct QueryOps {
  float hq[D / 32][8];
  half8 bq[D / 32];                 // BHL: hi (col < 8) or lo (col >= 8); else hi
  half8 bq_lo[BHL ? 1 : D / 32];    // !BHL: lo
};

// FULL: all 32 positions of the group are inside the partition.
template <int D, int SLOTS, bool ASYM, bool BHL, bool FULL>
__device__ __forceinline__ void process_group(const GroupLoad<D>& cur, int t0, int te, int kg, int col,
                                              const uint2* tab, uint16_t* st_lds, uint32_t lane_off,
                                              const QueryOps<D, BHL>& qo, WaveState<D, SLOTS, ASYM>& ws,
                                              int lane) {
  constexpr int KT = D / 32;
  constexpr int CT = D / 16;
  constexpr int GP = Slots<SLOTS>::GP;
  constexpr int NSETS = Slots<SLOTS>::NSETS;

  // Stage the group's LO / HI rows; each lane then reads the 8-channel runs
  // of its row group.
  if constexpr (D == 128) {
    reinterpret_cast<uint2*>(st_lds)[lane] = uint2{cur.st[0], cur.st[1]};
  } else {
    reinterpret_cast<uint32_t*>(st_lds)[lane] = cur.st[0];
  }
  wave_sync();

  floatx4 bias4 = {0.f, 0.f, 0.f, 0.f}, bias4_lo = {0.f, 0.f, 0.f, 0.f};
  floatx4 sc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const uint4 lo4 = *reinterpret_cast<const uint4*>(st_lds + 32 * kt + 8 * kg);
    const uint4 hi4 = *reinterpret_cast<const uint4*>(st_lds + D + 32 * kt + 8 * kg);
    // Group bias sum_c q_c (LO_c + HI_c) (q carries the 1/2): every row of
    // the product holds it.
    bias4 = mfma(__builtin_bit_cast(half8, lo4), qo.bq[kt], bias4);
    bias4 = mfma(__builtin_bit_cast(half8, hi4), qo.bq[kt], bias4);
    if constexpr (!BHL) {
      bias4_lo = mfma(__builtin_bit_cast(half8, lo4), qo.bq_lo[kt], bias4_lo);
      bias4_lo = mfma(__builtin_bit_cast(half8, hi4), qo.bq_lo[kt], bias4_lo);
    }
    // q~ = q (HI - LO) / 2 as fp16 hi + lo on this K-tile's 8 channels.
    const uint32_t lw[4] = {lo4.x, lo4.y, lo4.z, lo4.w};
    const uint32_t hw[4] = {hi4.x, hi4.y, hi4.z, hi4.w};
    uint32_t th[4], tl[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float d0 = f16_diff_lo(hw[p], lw[p]);
      const float d1 = f16_diff_hi(hw[p], lw[p]);
      const uint2 s = split_product(qo.hq[kt][2 * p], d0, qo.hq[kt][2 * p + 1], d1);
      th[p] = s.x;
      tl[p] = s.y;
    }
    const half8 qt_hi = __builtin_bit_cast(half8, uint4{th[0], th[1], th[2], th[3]});
    const half8 qt_lo = __builtin_bit_cast(half8, uint4{tl[0], tl[1], tl[2], tl[3]});
    // Scores for positions 16 mt + 4 kg + j of head `col`, this K-tile.
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int j0 = mt * (D / 16) + kt * 2;   // code bytes j0, j0 + 1 of this (mt, kt)
      const uint2 x0 = lookup(tab, cur.kc[j0 >> 2], byte_sel(j0 & 3), lane_off);
      const uint2 x1 = lookup(tab, cur.kc[(j0 + 1) >> 2], byte_sel((j0 + 1) & 3), lane_off);
      const half8 ak = as_half8(x0, x1);
      sc[mt] = mfma(ak, qt_hi, sc[mt]);
      sc[mt] = mfma(ak, qt_lo, sc[mt]);
    }
  }
  wave_sync();   // the LDS staging may be overwritten by the next group

  // Column bias: hi + lo parts (columns col and col +- 8 when BHL).
  float bias = bias4[0];
  if constexpr (BHL) {
    bias += __uint_as_float(static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(__float_as_uint(bias)), 0x128, 0xF, 0xF, false)));
  } else {
    bias += bias4_lo[0];
  }

  // Online softmax (base 2) for head `col` over this group's positions.
  bool valid[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) valid[i] = FULL || t0 + group_pos(kg, i) < te;
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 8; ++i) mx = valid[i] ? fmaxf(mx, sc[i >> 2][i & 3]) : mx;
  mx = rows_max(mx) + bias;
  // The reference max m_run only moves when a score passes it, and then to
  // kLazyMax above the new max: weights 2^(s - m_run) stay <= 1, and the
  // rescale of the accumulators (exact either way) is rarely needed.  The
  // norm reference moves when a norm reaches it (see kWeightExp).
  const int gE = group_norm_exponent(cur.nrm0, cur.nrm1, kg, FULL ? kGroupTokens : te - t0);
  if (__any(mx > ws.m_run) || gE > ws.nE) {
    const float m_new = fmaxf(ws.m_run, mx + kLazyMax);
    const int nE_new = max(ws.nE, gE);
    const float alpha = exp2f((ws.m_run - m_new) - static_cast<float>(nE_new - ws.nE));   // 0 on the first group
    ws.l_run *= alpha;
    const float alpha_v = __uint_as_float(to_value_column<SLOTS>(__float_as_uint(alpha)));
#pragma unroll
    for (int k = 0; k < NSETS; ++k) {
      if constexpr (ASYM) ws.accs[k] *= alpha_v;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) ws.acc[k][ct] *= alpha_v;
    }
    ws.m_run = m_new;
    ws.nE = nE_new;
    ws.wshift = static_cast<float>(kWeightExp + 14 - nE_new);
  }
  const float off = ws.m_run - bias - ws.wshift;
  const uint32_t n4[4] = {cur.nrm0.x, cur.nrm0.y, cur.nrm1.x, cur.nrm1.y};
  uint32_t wp[4];   // fp16 weights p * N of the lane's 8 positions, two per register
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i0 = 2 * r, i1 = 2 * r + 1;
    // arguments are <= wshift <= 28: the raw base-2 exponential flushes only results below 2^-126
    float p0 = __builtin_amdgcn_exp2f(sc[i0 >> 2][i0 & 3] - off);
    float p1 = __builtin_amdgcn_exp2f(sc[i1 >> 2][i1 & 3] - off);
    if constexpr (!FULL) {
      p0 = valid[i0] ? p0 : 0.f;
      p1 = valid[i1] ? p1 : 0.f;
    }
    ws.l_run += p0 + p1;
    wp[r] = to_value_column<SLOTS>(weight_pair(p0, p1, n4[r]));
  }

  // Value operands: rows = channels 16 ct + col, k = the positions of the scores.
  half8 av[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int j0 = 2 * ct;
    const uint2 x0 = lookup(tab, cur.vc[j0 >> 2], byte_sel(j0 & 3), lane_off);
    const uint2 x1 = lookup(tab, cur.vc[(j0 + 1) >> 2], byte_sel((j0 + 1) & 3), lane_off);
    av[ct] = as_half8(x0, x1);
  }

  // Accumulate each modality set whose modalities occur in the group.
  const int slot = col / GP;
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(cur.md0 & 0xFFu);
  const bool uniform = FULL && __all(cur.md0 == m0 * 0x01010101u && cur.md1 == m0 * 0x01010101u);
  const uint32_t md[2] = {cur.md0, cur.md1};
#pragma unroll
  for (int k = 0; k < NSETS; ++k) {
    const uint32_t lo_mod = static_cast<uint32_t>(k * SLOTS);
    const uint32_t my_mod = lo_mod + static_cast<uint32_t>(slot);   // this column's modality
    const bool col_ok = slot < SLOTS && my_mod < kModalities;
    bool present;
    uint32_t bm[4];
    int got = 0;   // modalities of this set that receive weight
    if (uniform) {
      present = m0 >= lo_mod && m0 < lo_mod + SLOTS && m0 < kModalities;
      got = present ? (1 << m0) : 0;
      const bool take = col_ok && my_mod == m0;
#pragma unroll
      for (int r = 0; r < 4; ++r) bm[r] = take ? wp[r] : 0u;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t keep = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = 2 * r + u;
          const uint32_t tm = (md[i >> 2] >> (8 * (i & 3))) & 0xFFu;
          if (valid[i] && tm >= lo_mod && tm < lo_mod + SLOTS && tm < kModalities) got |= 1 << tm;
          keep |= (col_ok && tm == my_mod) ? (0xFFFFu << (16 * u)) : 0u;
        }
        bm[r] = wp[r] & keep;
      }
      present = __any(got != 0);
    }
    if (present) {
      const half8 bw = __builtin_bit_cast(half8, uint4{bm[0], bm[1], bm[2], bm[3]});
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) ws.acc[k][ct] = mfma(av[ct], bw, ws.acc[k][ct]);
      if constexpr (ASYM) {
        const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
        ws.accs[k] = mfma(ones, bw, ws.accs[k]);
      }
      ws.mask |= got;
    }
  }
}

template <int D, int SLOTS, int NW, bool ASYM, bool BHL>
__global__ __launch_bounds__(NW * 64, 1) void decode_partition_kernel(DecodeArgs a) {
  constexpr int KT = D / 32;
  constexpr int CT = D / 16;
  constexpr int GP = Slots<SLOTS>::GP;
  constexpr int NSETS = Slots<SLOTS>::NSETS;
  constexpr int PS = kPartialHeader + kModalities * D;
  constexpr int kPrefetch = 2;     // groups in flight per wavefront
  constexpr int NPOS = NSETS * CT * 64;   // float4 accumulator slots of one wavefront
  union Smem {
    struct {
      uint2 tab[256 * kTabCopies];       // 64 KB: entry e, copy c at byte e*256 + c*8
      uint16_t stats[NW][2][D];          // per-wave staging of one group's LO / HI rows
    } s;
    float4 red[NW][NPOS];                // the wavefronts' rescaled accumulators
  };
  __shared__ Smem sm;
  __shared__ float s_m[NW][kMaxGroupHeads];
  __shared__ float s_l[NW][kMaxGroupHeads];
  __shared__ float s_s[NW][kModalities][kMaxGroupHeads];
  __shared__ int s_mask;
  __shared__ int s_pt[kPageRun];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) index
  const int kg = lane >> 4, col = lane & 15;
  const Place pl = place_of(a);
  const int split = pl.split, h = blockIdx.y, b = pl.b;
  const int G = a.group;
  const int L = session_length(a, b);
  const int tb = pl.tb;
  const int te = (split == pl.n - 1) ? L : min(pl.tend, L);
  const int te_full = te & ~(kGroupTokens - 1);   // tb is a multiple of 32
  const int stride = NW * kGroupTokens;
  const int first = tb + wave * kGroupTokens;

  // Loads first (the query, the page-table run of the partition, the first
  // groups), so that their latency overlaps the table set-up.  This lane's
  // score head (padding columns reuse the last head; ignored): q on channels
  // 32 kt + 8 kg + i, two float4 per K-tile.
  const int qcol = BHL ? (col & 7) : col;
  const int qh = h * G + min(qcol, G - 1);
  const float4* qp = reinterpret_cast<const float4*>(a.q_rot + (static_cast<size_t>(b) * a.hq + qh) * D);
  float4 qraw[KT][2];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    qraw[kt][0] = qp[(32 * kt + 8 * kg) / 4];
    qraw[kt][1] = qp[(32 * kt + 8 * kg) / 4 + 1];
  }
  // Page-table entries of the partition's pages (the plan keeps a partition
  // within kPageRun pages), read by the main loop from LDS.
  const int page0 = page_of(a, tb);
  for (int i = tid; i < kPageRun; i += NW * 64) {
    const int pg = page0 + i;
    s_pt[i] = pg < a.max_pages ? a.page_table[static_cast<size_t>(b) * a.max_pages + pg] : -1;
  }
  // The first groups take their pages through the constant address space
  // (scalar loads).
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)(a.page_table + static_cast<size_t>(b) * a.max_pages);
  GroupLoad<D> buf[kPrefetch];
  bool ok[kPrefetch];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) {
    const int t = first + k * stride;
    const int phys = ptab[min(page_of(a, t), a.max_pages - 1)];
    load_group<D>(a, h, t, te_full, lane, kg, phys, buf[k], ok[k]);
  }

  // Byte table: entry e = four fp16 levels of the codes in bits 2i..2i+1 of
  // e; thread tid fills 16 of entry (tid / 2)'s 32 copies.
  {
    const int e = tid >> 1;
    const uint32_t t0 = a.level_f16[0], t1 = a.level_f16[1];
    const uint2 v = tab_entry(e, t0, t1);
    for (int c = (tid & 1) * 16; c < (tid & 1) * 16 + 16; ++c) sm.s.tab[e * kTabCopies + c] = v;
    if constexpr (NW * 64 < 512) {
      // fewer threads than 2 per entry: the first pass covered entries < NW * 32
      for (int e2 = e + NW * 32; e2 < 256; e2 += NW * 32) {
        const uint2 v2 = tab_entry(e2, t0, t1);
        for (int c = (tid & 1) * 16; c < (tid & 1) * 16 + 16; ++c) sm.s.tab[e2 * kTabCopies + c] = v2;
      }
    }
  }

  QueryOps<D, BHL> qo;
  {
    const float sc = a.scale_log2e * 0.5f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const float qv[8] = {qraw[kt][0].x, qraw[kt][0].y, qraw[kt][0].z, qraw[kt][0].w,
                           qraw[kt][1].x, qraw[kt][1].y, qraw[kt][1].z, qraw[kt][1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = qv[i] * sc;
        qo.hq[kt][i] = v;
        const _Float16 hi = static_cast<_Float16>(v);
        const _Float16 lo = static_cast<_Float16>(v - static_cast<float>(hi));
        if constexpr (BHL) {
          qo.bq[kt][i] = col < 8 ? hi : lo;
        } else {
          qo.bq[kt][i] = hi;
          qo.bq_lo[kt][i] = lo;
        }
      }
    }
  }
  const uint32_t lane_off = static_cast<uint32_t>(lane & (kTabCopies - 1)) << 3;

  WaveState<D, SLOTS, ASYM> ws;
  ws.m_run = -__builtin_inff();
  ws.l_run = 0.f;
  ws.nE = 1;
  ws.wshift = static_cast<float>(kWeightExp + 13);
  ws.mask = 0;
#pragma unroll
  for (int k = 0; k < NSETS; ++k) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) ws.acc[k][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int k = 0; k < (ASYM ? NSETS : 1); ++k) ws.accs[k] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (tid == 0) s_mask = 0;
  __syncthreads();

  const uint2* tab = sm.s.tab;
  uint16_t* st_lds = &sm.s.stats[wave][0][0];

  // Prefetch ring over the partition's full groups: each wavefront keeps
  // kPrefetch groups in flight.  The one partial group a partition can end
  // with (the session's last) is handled after the loop.
  for (int base = first; base < te_full; base += kPrefetch * stride) {
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
      const int nxt = base + (k + kPrefetch) * stride;
      const int pn = nxt < te_full ? phys_page(a, s_pt, kPageRun, b, page0, page_of(a, nxt)) : -1;
      if (ok[k])
        process_group<D, SLOTS, ASYM, BHL, true>(buf[k], base + k * stride, te, kg, col, tab, st_lds, lane_off, qo,
                                                 ws, lane);
      load_group<D>(a, h, nxt, te_full, lane, kg, pn, buf[k], ok[k]);
    }
  }
  if (te_full >= tb && te_full < te && ((te_full - tb) / kGroupTokens) % NW == wave) {
    load_group<D>(a, h, te_full, te, lane, kg, phys_page(a, s_pt, kPageRun, b, page0, page_of(a, te_full)), buf[0], ok[0]);
    if (ok[0])
      process_group<D, SLOTS, ASYM, BHL, false>(buf[0], te_full, te, kg, col, tab, st_lds, lane_off, qo, ws, lane);
  }

  // ---- merge the wavefronts of the workgroup, write one partial per query head
  const float l_col = rows_sum(ws.l_run);
  const int slot = col / GP, hp = col % GP;
  if (kg == 0) {
    s_m[wave][col] = ws.m_run - ws.wshift;   // the reference of the scaled sums
    s_l[wave][col] = l_col;
    if (slot < SLOTS) {
#pragma unroll
      for (int k = 0; k < NSETS; ++k) {
        const int m = k * SLOTS + slot;
        if (m < kModalities) s_s[wave][m][hp] = ASYM ? ws.accs[ASYM ? k : 0][0] : 0.f;
      }
    }
  }
  {
    const int wm = wave_or_bits(ws.mask);
    if (lane == 0 && wm) atomicOr(&s_mask, wm);
  }
  __syncthreads();   // every wavefront is past its main loop: the byte table is dead
  // Bring the value columns (head hp) to the workgroup max of that head and
  // hand them to LDS; then every thread sums a share over the wavefronts in
  // a fixed order (bitwise reproducible) and writes it out.
  {
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][hp]);
    const float mw = s_m[wave][hp];
    // (arguments <= 0: the raw base-2 exponential only flushes results below 2^-126)
    const float e = (mw == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
#pragma unroll
    for (int k = 0; k < NSETS; ++k)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const floatx4 v = ws.acc[k][ct] * e;
        sm.red[wave][(k * CT + ct) * 64 + lane] = float4{v[0], v[1], v[2], v[3]};
      }
  }
  __syncthreads();
  const int wmask = s_mask;
  for (int pos = tid; pos < NPOS; pos += NW * 64) {
    const int ln = pos & 63, kct = pos >> 6;
    const int k = kct / CT, ct = kct % CT;
    const int c2 = ln & 15, kg2 = ln >> 4;
    const int sl2 = c2 / GP, hp2 = c2 % GP;
    const int m = k * SLOTS + sl2;
    if (sl2 < SLOTS && m < kModalities && hp2 < G && (wmask & (1 << m))) {
      float4 s = sm.red[0][pos];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float4 v = sm.red[w][pos];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
      }
      float* part = a.partials + (static_cast<size_t>(h * G + hp2) * a.pstride + pl.slot0 + split) * PS;
      *reinterpret_cast<float4*>(part + kPartialHeader + m * D + 16 * ct + 4 * kg2) = s;
    }
  }
  if (tid < G * kPartialHeader) {
    const int hh = tid / kPartialHeader, f = tid % kPartialHeader;
    float* part = a.partials + (static_cast<size_t>(h * G + hh) * a.pstride + pl.slot0 + split) * PS;
    float Mh = -__builtin_inff();
    for (int w = 0; w < NW; ++w) Mh = fmaxf(Mh, s_m[w][hh]);
    float v = 0.f;
    if (f == 0) {
      v = Mh;
    } else if (f == 1 || (f >= 4 && f < 4 + kModalities)) {
      for (int w = 0; w < NW; ++w) {
        const float mww = s_m[w][hh];
        if (mww != -__builtin_inff()) v += __builtin_amdgcn_exp2f(mww - Mh) * (f == 1 ? s_l[w][hh] : s_s[w][f - 4][hh]);
      }
    } else if (f == 2) {
      v = __int_as_float(wmask);
    }
    part[f] = v;
  }
}

// fp32 -> bf16 bits, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Reductions over lanes without LDS round trips: DPP inside rows of 16
// lanes (quad swaps, half-row and row mirrors), then the permlane swaps
// across rows.  Every lane of the group gets the same result (each step adds
// or maxes a pair in both orders, which are equal).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __uint_as_float(static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(__float_as_uint(v)), CTRL, 0xF, 0xF, false)));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);   // row_half_mirror
  v += dpp_f<0x140>(v);   // row_mirror
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

// ---------------------------------------------------------------------------
// Operand registers of one group for the streaming kernel below.
template <int D, int BITS = 2>
struct ConsumerLoad {
  uint32_t kc[BITS * D / 64];   // the lane's key code words (b d / 16 bytes of the group block)
  uint32_t vc[BITS * D / 64];
  uint2 nrm0, nrm1;
  uint2 knrm0, knrm1;     // per-token key norms (per-token key mode only)
  uint32_t md0, md1;
};

// Buffer resource over `bytes` bytes at `base` (raw, untyped).  A load whose
// offset is outside [0, bytes) returns zero without a memory access, so a
// wavefront can issue the loads of a group it will not use (bytes = 0) and
// keep the count of its loads in flight fixed.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// NW consecutive 32-bit words at byte offset voff (per lane) + soff, in as
// few buffer loads as the width allows.
template <int NW>
__device__ __forceinline__ void load_lane_words(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint32_t (&w)[NW]) {
#pragma unroll
  for (int i = 0; i + 4 <= NW; i += 4) {
    const uint4 x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 4 * i, soff, 0));
    w[i] = x.x; w[i + 1] = x.y; w[i + 2] = x.z; w[i + 3] = x.w;
  }
  constexpr int R = NW & 3;
  if constexpr (R >= 2) {
    const uint2 x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff + 4 * (NW - R), soff, 0));
    w[NW - R] = x.x; w[NW - R + 1] = x.y;
  }
  if constexpr (R & 1) w[NW - 1] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4 * (NW - 1), soff, 0);
}

// The pair-table entries behind operand unit u (8 codes, 8 BITS bits from bit
// 8 BITS u of the lane's code words) for BITS = 3, 4: four lookups, each
// giving two codes' levels.  4 bits: a byte holds 2 codes; 3 bits: a 6-bit
// field does.  An entry is {hi: the two levels in fp16, lo: 2^12 times what
// fp16 missed of them}, one 8-byte copy per lane pair of banks (32 copies,
// 256 bytes per entry), so lane_off = 8 (lane % 32) as for the byte table.
template <int BITS, int NW>
__device__ __forceinline__ void unit_pairs(const uint32_t (&w)[NW], int u, const uint2* tab, uint32_t lane_off,
                                           uint2 (&e)[4]) {
  const char* base = reinterpret_cast<const char*>(tab);
  if constexpr (BITS == 4) {
    const uint32_t x = w[u];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      e[i] = *reinterpret_cast<const uint2*>(base + __builtin_amdgcn_perm(x, lane_off, byte_sel(i)));
  } else {
    const int b0 = 24 * u, wi = b0 >> 5, sh = b0 & 31;
    uint32_t x = w[wi] >> sh;
    if (sh > 8) x |= w[wi + 1] << (32 - sh);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      e[i] = *reinterpret_cast<const uint2*>(base + ((((x >> (6 * i)) & 63u) << 8) | lane_off));
  }
}

// The 8 fp16 levels of operand unit u in code order.  2 bits: two lookups in
// the byte table (a byte holds 4 codes); 3 and 4 bits: the hi parts of the
// unit's pair entries.
template <int BITS, int NW>
__device__ __forceinline__ half8 unit_operand(const uint32_t (&w)[NW], int u, const uint2* tab, uint32_t lane_off) {
  if constexpr (BITS == 2) {
    const int j0 = 2 * u;
    return as_half8(lookup(tab, w[j0 >> 2], byte_sel(j0 & 3), lane_off),
                    lookup(tab, w[(j0 + 1) >> 2], byte_sel((j0 + 1) & 3), lane_off));
  } else {
    uint2 e[4];
    unit_pairs<BITS>(w, u, tab, lane_off, e);
    return __builtin_bit_cast(half8, uint4{e[0].x, e[1].x, e[2].x, e[3].x});
  }
}

// 3 / 4 bits: the hi and the (2^12-scaled) lo levels of operand unit u.
template <int BITS, int NW>
__device__ __forceinline__ void unit_operand_hilo(const uint32_t (&w)[NW], int u, const uint2* tab,
                                                  uint32_t lane_off, half8& hi, half8& lo) {
  uint2 e[4];
  unit_pairs<BITS>(w, u, tab, lane_off, e);
  hi = __builtin_bit_cast(half8, uint4{e[0].x, e[1].x, e[2].x, e[3].x});
  lo = __builtin_bit_cast(half8, uint4{e[0].y, e[1].y, e[2].y, e[3].y});
}

// Pair-table entry e: codes e % 2^BITS (low half) and e / 2^BITS (high half);
// x from the fp16 levels, y from their 2^12-scaled remainders.
template <int BITS>
__device__ __forceinline__ uint2 pair_entry(uint32_t e, const uint32_t (&lv)[8], const uint32_t (&lr)[8]) {
  const uint32_t k0 = e & ((1u << BITS) - 1u), k1 = e >> BITS;
  auto half_of = [](const uint32_t (&t)[8], uint32_t k) { return (t[k >> 1] >> (16 * (k & 1))) & 0xFFFFu; };
  return uint2{half_of(lv, k0) | (half_of(lv, k1) << 16), half_of(lr, k0) | (half_of(lr, k1) << 16)};
}

// ---------------------------------------------------------------------------
// Streaming partition kernel (G <= 8).
//
// Every wavefront of the workgroup streams its own contiguous run of the
// partition's 32-position groups and never waits for another wavefront until
// the epilogue: a group's statistics are fetched two groups ahead and its
// codes, norms and modality bytes one group ahead (buffer loads from
// resources built once per kernel), and while a group's scores run the
// wavefront prepares the next group's statistics-dependent operands itself:
//   - the group bias sum_c q_c (LO_c + HI_c) / 2 on the matrix cores, with
//     the staged LO / HI rows as the A operand (rows 4kg, 4kg+2: LO; rows
//     4kg+1, 4kg+3: HI) and q's fp16 hi / lo parts as the columns, so every
//     lane of column col ends up with the bias of head col & 7;
//   - q~ = q (HI - LO) / 2 as fp16 hi + lo, computed channel-major (a lane
//     takes 8 channels of 1 or 2 heads, so every product is formed once) and
//     handed to the score operand layout through a wavefront-private LDS slot
//     of 16-byte cells.
// The scores, online softmax and value sums follow the partition kernel
// above; the epilogue merges the wavefronts in LDS in a fixed order and
// writes one partial per query head.
constexpr int kSwWaves = 8;       // wavefronts per workgroup (the plan's unit is 32 * 8 positions)
constexpr int kQtStride = 17;     // cells per channel block in a q~ slot (16 columns + 1, spreads the banks)

template <int D>
struct SwSlot {
  uint4 qt[D / 8][kQtStride];     // [channel block cb][column]: channels 8cb..8cb+7 (hi: cols 0..7, lo: 8..15)
};

// Buffer resources over the cache arrays, built once per kernel (every array
// is below 2^31 bytes, checked on the host), plus a null resource whose loads
// return zero without touching memory.  A group's loads take its block
// offset as the scalar offset and a fixed per-lane vector offset.
struct SwRsrc {
  __amdgpu_buffer_rsrc_t k, v, st, nrm, md, null;
};

__device__ __forceinline__ SwRsrc sw_rsrc(const DecodeArgs& a) {
  SwRsrc r;
  r.k = span_rsrc(a.k_codes, 0x7FFFFFFF);
  r.v = span_rsrc(a.v_codes, 0x7FFFFFFF);
  r.st = span_rsrc(a.k_stats, 0x7FFFFFFF);
  r.nrm = span_rsrc(a.v_norms, 0x7FFFFFFF);
  r.md = span_rsrc(a.modality, 0x7FFFFFFF);
  r.null = span_rsrc(a.k_codes, 0);
  return r;
}

// Heads per producer lane: D / 8 channel blocks x 8 heads over 64 lanes.
template <int D>
struct SwShape {
  static constexpr int CB = D / 8;
  static constexpr int HPL = 8 * CB / 64;
};

// Bias and q~ of one group from its statistics registers; `stage` is the
// wavefront's 4D-byte staging of the LO / HI rows.
//
// Per-token key mode: the keys carry no group statistics; the rows staged
// for the bias hold c0 + c3 as an fp16 hi + lo pair (so the bias is
// sum_c q_c (c0 + c3) / 2), and the channel range HI - LO is the constant
// c3 - c0 (`range`): q~ is the same for every group.
template <int D, bool TQ = false>
__device__ __forceinline__ float sw_produce(const uint32_t (&st)[D / 64], uint16_t* stage, SwSlot<D>* slot,
                                            const float (&qs)[SwShape<D>::HPL][8], const uint4 (&bq)[D / 32],
                                            int lane, int kg, float range = 0.f) {
  constexpr int KT = D / 32;
  constexpr int CB = SwShape<D>::CB;
  constexpr int HPL = SwShape<D>::HPL;
  if constexpr (D == 128) {
    reinterpret_cast<uint2*>(stage)[lane] = uint2{st[0], st[1]};
  } else {
    reinterpret_cast<uint32_t*>(stage)[lane] = st[0];
  }
  wave_sync();
  const uint16_t* arow = stage + ((lane & 1) ? D : 0);   // A-operand row = lane & 15
  floatx4 bacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
    bacc = mfma(__builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(arow + 32 * kt + 8 * kg)),
                __builtin_bit_cast(half8, bq[kt]), bacc);
  const int cb = lane % CB, hs = lane / CB;
  const uint4 lo4 = *reinterpret_cast<const uint4*>(stage + 8 * cb);
  const uint4 hi4 = *reinterpret_cast<const uint4*>(stage + D + 8 * cb);
  const uint32_t lw[4] = {lo4.x, lo4.y, lo4.z, lo4.w};
  const uint32_t hw[4] = {hi4.x, hi4.y, hi4.z, hi4.w};
  // The products below are hand-written instructions: make the LDS operands
  // (query, statistics) complete first rather than rely on the compiler's
  // wait insertion for inline assembly.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  float d[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if constexpr (TQ) {
      d[2 * p] = range;
      d[2 * p + 1] = range;
    } else {
      d[2 * p] = f16_diff_lo(hw[p], lw[p]);
      d[2 * p + 1] = f16_diff_hi(hw[p], lw[p]);
    }
  }
#pragma unroll
  for (int u = 0; u < HPL; ++u) {
    const int head = hs * HPL + u;
    uint32_t th[4], tl[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint2 sp = split_product(qs[u][2 * p], d[2 * p], qs[u][2 * p + 1], d[2 * p + 1]);
      th[p] = sp.x;
      tl[p] = sp.y;
    }
    slot->qt[cb][head] = uint4{th[0], th[1], th[2], th[3]};
    slot->qt[cb][8 + head] = uint4{tl[0], tl[1], tl[2], tl[3]};
  }
  // rows 4kg (LO) and 4kg + 1 (HI); the partner column (col ^ 8) holds the
  // other part of q
  float bias = bacc[0] + bacc[1];
  bias += dpp_f<0x128>(bias);
  wave_sync();
  return bias;
}

// Consumer step of the streaming kernel, in two parts so that the caller can
// place independent work (the next group's operands) between the loads of
// the codes and the softmax: sw_front looks up the key and value operands
// and forms the scores (q~ from the wavefront's slot); sw_back runs the
// online softmax and the value sums.
template <int D>
struct SwFront {
  floatx4 sc[2];
  floatx4 sl[2];   // 3 / 4 bits: the scores' lo-level part (times 2^12)
};

template <int D, int BITS>
__device__ __forceinline__ void sw_front(const ConsumerLoad<D, BITS>& cur, const SwSlot<D>* slot, int kg, int col,
                                         const uint2* tab, uint32_t lane_off, SwFront<D>& f) {
  constexpr int KT = D / 32;
  f.sc[0] = floatx4{0.f, 0.f, 0.f, 0.f};
  f.sc[1] = floatx4{0.f, 0.f, 0.f, 0.f};
  if constexpr (BITS != 2) {
    f.sl[0] = floatx4{0.f, 0.f, 0.f, 0.f};
    f.sl[1] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const half8 qt = __builtin_bit_cast(half8, slot->qt[4 * kt + kg][col]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {   // operand unit (positions 16 mt.., channels 32 kt..)
      if constexpr (BITS == 2) {
        f.sc[mt] = mfma(unit_operand<BITS>(cur.kc, mt * (D / 32) + kt, tab, lane_off), qt, f.sc[mt]);
      } else {
        half8 hi, lo;
        unit_operand_hilo<BITS>(cur.kc, mt * (D / 32) + kt, tab, lane_off, hi, lo);
        f.sc[mt] = mfma(hi, qt, f.sc[mt]);
        f.sl[mt] = mfma(lo, qt, f.sl[mt]);
      }
    }
  }
}

// Softmax and value sums of one group with rem valid positions (1..32: 32
// for a full group, fewer for the session's last group).  Positions past rem
// get the score -inf, hence the weight 0.  The weights are formed against the
// current reference max right away; the group's own max only decides (off the
// critical path) whether the reference must move first, which is rare: the
// reference sits kLazyMax above every score seen so far.  Groups of one single
// modality (the common case inside a video, audio or text run) form their
// weight operands with one select per set; others go through per-position
// modality masks.
//
// Per-token key mode (TQ): score i is (bias + dot_i) N_i / sqrt(d), with the
// key norm N_i of the lane's position i (fp16 pairs in knrm0 / knrm1, in the
// value norms' order); the bias is then folded in and not added again.
template <int D, int SLOTS, bool ASYM, bool TQ = false, int BITS = 2>
__device__ __forceinline__ void sw_back1(const ConsumerLoad<D, BITS>& ca, const SwFront<D>& fa, float bias_in, int rem_a,
                                         int kg, int col, const uint2* tab, uint32_t lane_off,
                                         WaveState<D, SLOTS, ASYM>& ws, float key_scale = 0.f) {
  constexpr int CT = D / 16;
  constexpr int GP = Slots<SLOTS>::GP;
  constexpr int NSETS = Slots<SLOTS>::NSETS;
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = fa.sc[i >> 2][i & 3] + dpp_f<0x128>(fa.sc[i >> 2][i & 3]);
  if constexpr (BITS != 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] += 0x1p-12f * (fa.sl[i >> 2][i & 3] + dpp_f<0x128>(fa.sl[i >> 2][i & 3]));
  }
  float bias_a = bias_in;
  if constexpr (TQ) {
    const uint32_t kn[4] = {ca.knrm0.x, ca.knrm0.y, ca.knrm1.x, ca.knrm1.y};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float n0 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(kn[r] & 0xFFFFu)));
      const float n1 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(kn[r] >> 16)));
      s[2 * r] = (s[2 * r] + bias_in) * (n0 * key_scale);
      s[2 * r + 1] = (s[2 * r + 1] + bias_in) * (n1 * key_scale);
    }
    bias_a = 0.f;
  }
  if (rem_a < kGroupTokens) {
    int ra = rem_a;
    asm volatile("" : "+s"(ra));
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = group_pos(kg, i) < ra ? s[i] : -__builtin_inff();
  }
  const uint32_t na[4] = {ca.nrm0.x, ca.nrm0.y, ca.nrm1.x, ca.nrm1.y};
  float pe[8];
  uint32_t wa[4];
  auto weights = [&](float m_ref) {
    const float oa = m_ref - bias_a - ws.wshift;
#pragma unroll
    for (int i = 0; i < 8; ++i) pe[i] = __builtin_amdgcn_exp2f(s[i] - oa);
#pragma unroll
    for (int r = 0; r < 4; ++r) wa[r] = to_value_column<SLOTS>(weight_pair(pe[2 * r], pe[2 * r + 1], na[r]));
  };
  weights(ws.m_run);
  float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  mx = rows_max(mx) + bias_a;
  const int gE = group_norm_exponent(ca.nrm0, ca.nrm1, kg, rem_a);
  if (__any(mx > ws.m_run) || gE > ws.nE) {
    const float m_new = fmaxf(ws.m_run, mx + kLazyMax);
    const int nE_new = max(ws.nE, gE);
    const float alpha = exp2f((ws.m_run - m_new) - static_cast<float>(nE_new - ws.nE));   // 0 on the first group
    ws.l_run *= alpha;
    const float alpha_v = __uint_as_float(to_value_column<SLOTS>(__float_as_uint(alpha)));
#pragma unroll
    for (int k = 0; k < NSETS; ++k) {
      if constexpr (ASYM) ws.accs[k] *= alpha_v;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) ws.acc[k][ct] *= alpha_v;
    }
    ws.m_run = m_new;
    ws.nE = nE_new;
    ws.wshift = static_cast<float>(kWeightExp + 14 - nE_new);
    // arguments are now <= wshift (or -inf): the raw base-2 exponential flushes only results below 2^-126
    weights(ws.m_run);
  }
  ws.l_run += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
  // Weight operands of the accumulator sets: set k's column (slot_c, hp)
  // keeps the positions whose modality is k SLOTS + slot_c.  Only these
  // operands depend on the branch; every set then takes its matrix-core
  // products unconditionally (a set without its modalities adds exact
  // zeros), so the accumulators are updated in place, never copied.  The
  // lane's modality bits go into ws.mask, OR-ed over the wavefront at the end.
  const int slot_c = col / GP;
  uint32_t bs[NSETS][4];
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(ca.md0 & 0xFFu);
  const uint32_t mm = m0 * 0x01010101u;
  const bool uniform = rem_a == kGroupTokens && m0 < kModalities && __all(ca.md0 == mm && ca.md1 == mm);
  if (uniform) {
    const int k0 = static_cast<int>(m0) / SLOTS;
    const bool take = slot_c == static_cast<int>(m0) - k0 * SLOTS;
#pragma unroll
    for (int k = 0; k < NSETS; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) bs[k][r] = (take && k == k0) ? wa[r] : 0u;
    ws.mask |= 1 << m0;
  } else {
    int ra = rem_a;
    uint32_t mda[2] = {ca.md0, ca.md1};
    asm volatile("" : "+s"(ra), "+v"(mda[0]), "+v"(mda[1]));
    int got = 0;
#pragma unroll
    for (int k = 0; k < NSETS; ++k) {
      const uint32_t lo_mod = static_cast<uint32_t>(k * SLOTS);
      const uint32_t my_mod = lo_mod + static_cast<uint32_t>(slot_c);
      const bool col_ok = slot_c < SLOTS && my_mod < kModalities;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t keep_a = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = 2 * r + u;
          const uint32_t ta = (mda[i >> 2] >> (8 * (i & 3))) & 0xFFu;
          if (group_pos(kg, i) < ra && ta >= lo_mod && ta < lo_mod + SLOTS && ta < kModalities) got |= 1 << ta;
          keep_a |= (col_ok && ta == my_mod) ? (0xFFFFu << (16 * u)) : 0u;
        }
        bs[k][r] = wa[r] & keep_a;
      }
    }
    ws.mask |= got;
  }
  half8 bw[NSETS];
#pragma unroll
  for (int k = 0; k < NSETS; ++k) bw[k] = __builtin_bit_cast(half8, uint4{bs[k][0], bs[k][1], bs[k][2], bs[k][3]});
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const half8 va = unit_operand<BITS>(ca.vc, ct, tab, lane_off);   // channels 16 ct + lane % 16
#pragma unroll
    for (int k = 0; k < NSETS; ++k) ws.acc[k][ct] = mfma(va, bw[k], ws.acc[k][ct]);
  }
  if constexpr (ASYM) {
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
    for (int k = 0; k < NSETS; ++k) ws.accs[k] = mfma(ones, bw[k], ws.accs[k]);
  }
}

// Shared memory of the fused step's append workgroup.
template <int D>
struct StepSmem {
  app::AppendSmem<D> app;
  float q[8][D];                        // the KV head's query heads, rotated
  float sc[8][kGroupTokens];            // open group: scores (base 2), -inf where nothing is attended
  float w[8][kModalities][kGroupTokens];   // weights 2^(s - M) N of the positions of each modality (else 0)
  float nrm[kGroupTokens];
  int mod[kGroupTokens];
  int last;                             // the append's ticket flag (unused: the merge advances the lengths)
  float lv[4];                          // the normalized levels
  __align__(16) uint8_t rec[stage_record_bytes(D)];   // the open group (kStage* layout)
};

// The fused step's work for (session b, KV head h) beside the partitions:
// the append of the step's position (the key role, then the value role of
// kvq_append.h, which also copy the open group to a record in this
// workgroup's shared memory), then
// the open group's partial for every query head i of the KV head, as the
// session's last partial slot (`slot`) in the partitions' form: scores
// s_t = scale log2(e) <q_rot_i, k_hat_t> with k_hat = (HI + LO) / 2 +
// level (HI - LO) / 2, reference max M = max_t s_t, denominator
// sum_t 2^(s_t - M), per modality m the sums of the weights 2^(s_t - M) N_t
// times the normalized value levels (a position whose modality is not a
// known one counts in the denominator only).  Runs in fp32.  All 512
// threads call it.
template <int D, bool BF16>
__device__ __forceinline__ void step_append_open_group(const DecodeArgs& a, const AppendArgs& ap, StepSmem<D>& sm,
                                                       int h, int b, int slot) {
  constexpr int NT = kSwWaves * 64;
  constexpr int OQ = D / 16;                      // scores: channels per thread, 16 threads per position
  constexpr int VG = NT / D;                      // values: threads per channel (query heads dealt round robin)
  constexpr int PS = kPartialHeader + kModalities * D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group;
  // the four levels in shared memory: indexing the argument array by a
  // code would be a memory load per use
  if (tid < 4) sm.lv[tid] = a.level_f32[tid];
  auto level = [&](uint32_t c) { return sm.lv[c]; };
  // the new key row, for the raw tail (stored at the end with the cache
  // writes): one 32-bit word per thread
  constexpr int KW = D * (BF16 ? 2 : 4) / 4;
  const uint32_t kraw = tid < KW
      ? reinterpret_cast<const uint32_t*>(ap.k_new)[static_cast<size_t>(b * a.hkv + h) * KW + tid] : 0u;
  if (wave < 2) {
    // the KV head's query heads (16 lanes per head, head 4 w .. 4 w + 3 on wavefront w)
    constexpr int RCH = D / rotq::kLanes;
    const int hl = 4 * wave + lane / rotq::kLanes, sub = lane % rotq::kLanes;
    float o[RCH];
    rotq::rotate_values<D, BF16>(ap.rq, b * a.hq + h * G + min(hl, G - 1), sub, o);
#pragma unroll
    for (int i = 0; i < RCH; ++i) sm.q[hl][sub * RCH + i] = o[i];
  }
  app::append_group<D, BF16, 2>(ap, sm.app, sm.last, 0, h, b, 0, sm.rec);
  __syncthreads();
  app::append_group<D, BF16, 2>(ap, sm.app, sm.last, 1, h, b, 0, sm.rec);
  __syncthreads();   // the open group's record is complete

  const uint8_t* rec = sm.rec;
  {
    // scores: thread (t, part) takes channels part OQ .. of position t
    const int t = tid / 16, part = tid % 16, c0 = part * OQ;
    const int2 meta = *reinterpret_cast<const int2*>(rec + kStageMeta);
    const uint16_t* lohi = reinterpret_cast<const uint16_t*>(rec + kStageCodes + 16 * D);
    float kh[OQ];
#pragma unroll
    for (int i = 0; i < OQ; ++i) {
      const float lo = f16_bits_to_f32(lohi[c0 + i]), hi = f16_bits_to_f32(lohi[D + c0 + i]);
      const uint32_t byte = rec[kStageCodes + key_code_byte<D>(t, c0 + (i & ~3))];
      const float lvl = level((byte >> (2 * (i & 3))) & 3u);
      kh[i] = (hi + lo) * 0.5f + (hi - lo) * 0.5f * lvl;
    }
    const bool live = meta.x != 0 && t < meta.y;
    for (int i = 0; i < G; ++i) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < OQ; ++c) dot += sm.q[i][c0 + c] * kh[c];
      dot = row16_sum(dot);
      if (part == 0) sm.sc[i][t] = live ? dot * a.scale_log2e : -__builtin_inff();
    }
    if (part == 0) {
      sm.nrm[t] = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(rec + kStageNorms)[t]);
      sm.mod[t] = rec[kStageMods + t];
    }
  }
  __syncthreads();
  if (wave < G) {
    // softmax of query head `wave`: lane t < 32 takes position t
    const int t = lane & (kGroupTokens - 1);
    const float sc = lane < kGroupTokens ? sm.sc[wave][t] : -__builtin_inff();
    const float mo = wave_max(sc);
    const float e = (mo == -__builtin_inff() || sc == -__builtin_inff()) ? 0.f : exp2f(sc - mo);
    const float lsum = wave_sum(e);
    const int md = sm.mod[t];
    int mk = 0;
#pragma unroll
    for (int m = 0; m < kModalities; ++m)
      if (__any(e > 0.f && md == m)) mk |= 1 << m;
    if (lane < kGroupTokens) {
      const float x = e * sm.nrm[t];
#pragma unroll
      for (int m = 0; m < kModalities; ++m) sm.w[wave][m][t] = md == m ? x : 0.f;
    }
    float* part = a.partials + (static_cast<size_t>(h * G + wave) * a.pstride + slot) * PS;
    if (lane < kPartialHeader)
      part[lane] = lane == 0 ? mo : lane == 1 ? lsum : lane == 2 ? __int_as_float(mk) : 0.f;
  }
  __syncthreads();
  {
    // value sums: channel c, query heads i = tid / D, + VG, ...
    // (the channel's levels are decoded once; the modality split is in the
    // weights, so the sums take no per-position branch or select)
    const int c = tid % D;
    float lvl[kGroupTokens];
#pragma unroll
    for (int k = 0; k < kGroupTokens / 4; ++k) {
      const uint32_t vb = rec[kStageCodes + 8 * D + value_code_byte<D>(4 * k, c)];
#pragma unroll
      for (int u = 0; u < 4; ++u) lvl[4 * k + u] = level((vb >> (2 * u)) & 3u);
    }
    for (int i = tid / D; i < G; i += VG) {
      float av[kModalities] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < kGroupTokens; ++t)
#pragma unroll
        for (int m = 0; m < kModalities; ++m) av[m] += sm.w[i][m][t] * lvl[t];
      float* part = a.partials + (static_cast<size_t>(h * G + i) * a.pstride + slot) * PS;
#pragma unroll
      for (int m = 0; m < kModalities; ++m) part[kPartialHeader + m * D + c] = av[m];
    }
  }

  // The append's cache writes, from the record, after the workgroup's last
  // load: the group's key and value blocks and statistics, the new
  // position's norm and modality byte, and its raw key in the tail when the
  // group stays open.
  {
    const int* meta = reinterpret_cast<const int*>(rec + kStageMeta);
    const int t0 = meta[2], s_first = meta[3], s_end = meta[1], phys = meta[4];
    if (meta[0]) {
      const long long blk = *reinterpret_cast<const long long*>(rec + kStageBlock);
      const uint4* src = reinterpret_cast<const uint4*>(rec + kStageCodes);
      if (tid < D / 2) {
        reinterpret_cast<uint4*>(ap.k_codes + static_cast<size_t>(blk) * 8 * D)[tid] = src[tid];
      } else if (tid < D) {
        reinterpret_cast<uint4*>(ap.v_codes + static_cast<size_t>(blk) * 8 * D)[tid - D / 2] = src[tid];
      } else if (tid < D + D / 4) {
        reinterpret_cast<uint4*>(ap.k_stats + static_cast<size_t>(blk) * 2 * D)[tid - D] = src[tid];
      }
      if (tid >= s_first && tid < s_end) {
        const int pos = (t0 + tid) % ap.page_tokens;
        ap.v_norms[(static_cast<size_t>(phys) * ap.hkv + h) * ap.page_tokens + pos] =
            reinterpret_cast<const uint16_t*>(rec + kStageNorms)[tid];
        if (h == 0) ap.modality[static_cast<size_t>(phys) * ap.page_tokens + pos] = rec[kStageMods + tid];
      }
    }
    const int L_old = t0 + s_first;
    if (((L_old + 1) & (kGroupTokens - 1)) != 0 && tid < KW) {
      const int sb = ap.b0 + b;
      reinterpret_cast<uint32_t*>(ap.k_tail)[(static_cast<size_t>(sb * ap.hkv + h) * kGroupTokens + (L_old & 31)) * KW + tid] = kraw;
    }
  }
}

// STEP: the fused decode step's launch.  The column after each session's
// partitions runs the step's append and the open group's partial for each
// (session, KV head)
// (step_append_open_group) in this kernel's shared memory; the partitions
// rotate their own query heads (ap.rq, inputs in bf16 when BF16) and attend
// the closed groups only, positions below 32 floor(L / 32) of the session's
// length L before the append.  Neither side reads what the other writes.
template <int D, int SLOTS, bool ASYM, bool TQ, int BITS, bool STEP = false, bool BF16 = false>
__global__ __launch_bounds__(kSwWaves * 64, 1) void decode_partition_sw_kernel(DecodeArgs a, AppendArgs ap) {
  constexpr int KT = D / 32;
  constexpr int CT = D / 16;
  constexpr int GP = Slots<SLOTS>::GP;
  constexpr int NSETS = Slots<SLOTS>::NSETS;
  constexpr int PS = kPartialHeader + kModalities * D;
  constexpr int NW = kSwWaves;
  constexpr int NT = NW * 64;
  constexpr int NPOS = NSETS * CT * 64;
  constexpr int CB = SwShape<D>::CB;
  constexpr int HPL = SwShape<D>::HPL;
  union Smem {
    struct {
      uint2 tab[256 * kTabCopies];          // 64 KB byte table
      SwSlot<D> slots[NW][2];               // q~ of the wavefront's current pair of groups
      uint16_t stage[NW][2][2 * D];         // LO / HI rows of the pair being prepared
    } s;
    float4 red[NW][NPOS];                   // the wavefronts' rescaled accumulators
    StepSmem<D> step;                       // STEP: the append's workgroups
  };
  __shared__ Smem sm;
  __shared__ float s_m[NW][kMaxGroupHeads];
  __shared__ float s_l[NW][kMaxGroupHeads];
  __shared__ float s_s[NW][kModalities][kMaxGroupHeads];
  __shared__ int s_mask;
  __shared__ int s_cmask[NW];
  __shared__ float4 s_qs[2 * HPL * 64];   // producer lanes' q (scaled), [2u + half][lane]
  __shared__ uint4 s_bq[KT * 64];         // bias operand of every lane, [kt][lane]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4, col = lane & 15;
  const Place pl = place_of(a);
  const int split = pl.split, h = blockIdx.y, b = pl.b;
  if constexpr (STEP) {
    if (split >= pl.n) {
      static_assert(NT == app::kAppendThreads, "the append's workgroup size");
      step_append_open_group<D, BF16>(a, ap, sm.step, h, b, pl.slot0 + pl.n);
      return;
    }
  }
  const int G = a.group;
  // STEP: the closed groups only (the append rewrites the open one)
  const int L = STEP ? (session_length(a, b) & ~(kGroupTokens - 1)) : session_length(a, b);
  const int tb = pl.tb;
  const int te = (split == pl.n - 1) ? L : min(pl.tend, L);
  const int ng = te > tb ? (te - tb + kGroupTokens - 1) / kGroupTokens : 0;   // groups of the partition
  // The groups are dealt to the wavefronts round robin: step j of wavefront
  // w is group w + NW j, so the NW wavefronts read NW adjacent blocks at a
  // time, and the mapped pages of a sparse page set (a 256-position page
  // holds 8 groups) fall to every wavefront alike.
  const int steps = (ng + NW - 1) / NW;
  const int ps = a.page_shift;                     // page_tokens is a power of two here
  const int pmask = a.page_tokens - 1;
  // Page-table entries of the wavefront's own groups, one per lane: lane j
  // holds the physical page of the group of step j (-1 past the table).  A
  // step reads its entry with v_readlane, so finding a group's block needs
  // no LDS access (an LDS or scalar-memory read would make the wavefront
  // wait for every LDS operation it has in flight).  The load does not wait
  // for the session length.
  int v_page = -1;
  {
    const int pgl = (tb + (wave + NW * lane) * kGroupTokens) >> ps;
    if (pgl < a.max_pages) v_page = a.page_table[static_cast<size_t>(b) * a.max_pages + pgl];
  }
  // The session's page-table row for steps from 64 on (a partition that grew
  // past its plan): read with vector loads, which leave the LDS and
  // scalar-memory counter alone.
  const __amdgpu_buffer_rsrc_t rpt = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(a.page_table + static_cast<size_t>(b) * a.max_pages), 0, a.max_pages * 4, 0x00020000);
  const SwRsrc rs = sw_rsrc(a);
  const int hoff = h * (a.page_tokens / kGroupTokens);

  // Query constants: the producer lanes' q on channels 8cb..8cb+7 of their
  // heads, and the bias operand (q's fp16 hi part in columns 0..7, lo part
  // in columns 8..15, channels 32kt + 8kg + i).  Both carry scale * log2(e) / 2.
  const float qsc = a.scale_log2e * 0.5f;
  if constexpr (STEP) {
    // The group's query heads rotated here, 16 lanes per head (head hl =
    // 4 w .. 4 w + 3 on wavefront w < 2, channels RCH sub ..), and written
    // straight into both layouts (the split-0 partition also stores q_rot).
    if (wave < 2) {
      constexpr int RCH = D / rotq::kLanes;
      const int hl = 4 * wave + lane / rotq::kLanes, sub = lane % rotq::kLanes;
      const int bi = b * a.hq + h * G + min(hl, G - 1);
      float o[RCH];
      rotq::rotate_values<D, BF16>(ap.rq, bi, sub, o);
      if (split == 0 && hl < G) {
        float4* dst = reinterpret_cast<float4*>(ap.rq.q_rot + static_cast<size_t>(bi) * D + sub * RCH);
#pragma unroll
        for (int k = 0; k < RCH / 4; ++k) dst[k] = float4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
      }
      const int hs = hl / HPL, u = hl % HPL;
#pragma unroll
      for (int k = 0; k < RCH / 4; ++k) {
        const int c4 = sub * RCH + 4 * k;            // channels c4 .. c4 + 3
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = o[4 * k + i] * qsc;
        s_qs[(2 * u + ((c4 >> 2) & 1)) * 64 + hs * CB + (c4 >> 3)] = float4{v[0], v[1], v[2], v[3]};
        _Float16 hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = static_cast<_Float16>(v[i]);
          lo[i] = static_cast<_Float16>(v[i] - static_cast<float>(hi[i]));
        }
        uint2* bq2 = reinterpret_cast<uint2*>(s_bq);
        const int l0 = (c4 >> 5) * 64 + ((c4 & 31) >> 3) * 16 + hl;   // [kt][kg * 16 + column]
        bq2[2 * l0 + ((c4 & 7) >> 2)] = __builtin_bit_cast(uint2, hi);
        bq2[2 * (l0 + 8) + ((c4 & 7) >> 2)] = __builtin_bit_cast(uint2, lo);
      }
    }
  } else {
    if (wave == 0) {
      const int cb = lane % CB, hs = lane / CB;
#pragma unroll
      for (int u = 0; u < HPL; ++u) {
        const int qh = h * G + min(hs * HPL + u, G - 1);
        const float4* qp = reinterpret_cast<const float4*>(a.q_rot + (static_cast<size_t>(b) * a.hq + qh) * D + 8 * cb);
        const float4 q0 = qp[0], q1 = qp[1];
        s_qs[(2 * u) * 64 + lane] = float4{q0.x * qsc, q0.y * qsc, q0.z * qsc, q0.w * qsc};
        s_qs[(2 * u + 1) * 64 + lane] = float4{q1.x * qsc, q1.y * qsc, q1.z * qsc, q1.w * qsc};
      }
    }
    if (wave == 1) {
      const int qh = h * G + min(col & 7, G - 1);
      const float4* qp = reinterpret_cast<const float4*>(a.q_rot + (static_cast<size_t>(b) * a.hq + qh) * D);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const float4 q0 = qp[(32 * kt + 8 * kg) / 4], q1 = qp[(32 * kt + 8 * kg) / 4 + 1];
        const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        half8 bq;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float v = qv[i] * qsc;
          const _Float16 hi = static_cast<_Float16>(v);
          bq[i] = col < 8 ? hi : static_cast<_Float16>(v - static_cast<float>(hi));
        }
        s_bq[kt * 64 + lane] = __builtin_bit_cast(uint4, bq);
      }
    }
  }

  if constexpr (BITS == 2) {
    // Byte table (two copies of an entry per 16-byte store).
    for (int i = tid; i < 256 * kTabCopies / 2; i += NT) {
      const uint2 v = tab_entry(static_cast<uint32_t>(i) / (kTabCopies / 2), a.level_f16[0], a.level_f16[1]);
      reinterpret_cast<uint4*>(sm.s.tab)[i] = uint4{v.x, v.y, v.x, v.y};
    }
  } else {
    // Pair table: 2^(2 BITS) entries of 32 8-byte copies (two per 16-byte store).
    for (int i = tid; i < (1 << (2 * BITS)) * 16; i += NT) {
      const uint2 v = pair_entry<BITS>(static_cast<uint32_t>(i) >> 4, a.level_f16, a.level_lo_f16);
      reinterpret_cast<uint4*>(sm.s.tab)[i] = uint4{v.x, v.y, v.x, v.y};
    }
  }
  if (tid == 0) s_mask = 0;
  const uint32_t lane_off = static_cast<uint32_t>(lane & (kTabCopies - 1)) << 3;
  WaveState<D, SLOTS, ASYM> ws;
  ws.m_run = -__builtin_inff();
  ws.l_run = 0.f;
  ws.nE = 1;
  ws.wshift = static_cast<float>(kWeightExp + 13);
  ws.mask = 0;
#pragma unroll
  for (int k = 0; k < NSETS; ++k)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) ws.acc[k][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < (ASYM ? NSETS : 1); ++k) ws.accs[k] = floatx4{0.f, 0.f, 0.f, 0.f};
  uint16_t* stage_a = &sm.s.stage[wave][0][0];
  uint16_t* stage_b = &sm.s.stage[wave][1][0];
  SwSlot<D>* slot_a = &sm.s.slots[wave][0];
  SwSlot<D>* slot_b = &sm.s.slots[wave][1];
  __syncthreads();   // the byte table is complete
  const uint2* tab = sm.s.tab;

  // Group j of the wavefront's run: block and modality offsets (block 0 for
  // an invalid group, see sw_load); returns whether the group is valid.
  auto locate = [&](int j, int& blk, int& moff) {
    const int gi = wave + NW * j;
    const int t0 = tb + gi * kGroupTokens;
    const bool inside = j < steps && gi < ng;
    int phys = -1;
    if (inside) {
      if (j < 64) {
        phys = __builtin_amdgcn_readlane(v_page, j);
      } else {
        const int pg = t0 >> ps;
        phys = pg < a.max_pages ? __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(rpt, 0, 4 * pg, 0))
                                : -1;
      }
    }
    const bool ok = inside && phys >= 0 && phys < a.num_pages;
    const int tin = t0 & pmask;
    blk = ok ? phys * a.blocks_per_page + hoff + (tin >> 5) : 0;
    moff = ok ? phys * a.page_tokens + tin : 0;
    return ok;
  };
  auto load_stats = [&](int j, uint32_t (&st)[D / 64]) {
    int blk, moff;
    locate(j, blk, moff);
    if constexpr (D == 128) {
      const uint2 s2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs.st, lane * 8, blk * (4 * D), 0));
      st[0] = s2.x;
      st[1] = s2.y;
    } else {
      st[0] = __builtin_amdgcn_raw_buffer_load_b32(rs.st, lane * 4, blk * (4 * D), 0);
    }
  };
  auto load_codes = [&](int j, ConsumerLoad<D, BITS>& c) {
    int blk, moff;
    const bool ok = locate(j, blk, moff);
    constexpr int LW = BITS * D / 64;   // code words per lane
    load_lane_words<LW>(rs.k, lane * 4 * LW, blk * (4 * BITS * D), c.kc);
    load_lane_words<LW>(rs.v, lane * 4 * LW, blk * (4 * BITS * D), c.vc);
    c.nrm0 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs.nrm, 8 * kg, blk * 64, 0));
    c.nrm1 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs.nrm, 32 + 8 * kg, blk * 64, 0));
    c.md0 = __builtin_amdgcn_raw_buffer_load_b32(rs.md, 4 * kg, moff, 0);
    c.md1 = __builtin_amdgcn_raw_buffer_load_b32(rs.md, 16 + 4 * kg, moff, 0);
    if constexpr (TQ) {
      // per-token key norms: the first 64 bytes of the group's statistics block
      c.knrm0 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs.st, 8 * kg, blk * (4 * D), 0));
      c.knrm1 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs.st, 32 + 8 * kg, blk * (4 * D), 0));
    }
    return ok;
  };

  // The producer lanes' q, read from LDS.
  auto read_qs = [&](float (&q)[HPL][8]) {
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      const float4 q0 = s_qs[(2 * u) * 64 + lane], q1 = s_qs[(2 * u + 1) * 64 + lane];
      q[u][0] = q0.x; q[u][1] = q0.y; q[u][2] = q0.z; q[u][3] = q0.w;
      q[u][4] = q1.x; q[u][5] = q1.y; q[u][6] = q1.z; q[u][7] = q1.w;
    }
  };
  // Rings with fixed registers (group j uses ring j & 1): a group's
  // statistics are fetched two groups ahead, its codes one group ahead, and
  // its operands (q~, bias) are prepared during the previous group.
  ConsumerLoad<D, BITS> cr[2];
  bool okr[2];
  uint32_t sr[2][D / 64];
  if constexpr (!TQ) {
    load_stats(0, sr[0]);
    load_stats(1, sr[1]);
  } else {
    // constant rows: c0 + c3 (= 2 cmid) as an fp16 hi part (the LO row,
    // staged by lanes 0..31) and lo part (the HI row, lanes 32..63)
    const float csum = 2.f * a.cmid;
    const _Float16 shi = static_cast<_Float16>(csum);
    const _Float16 slo = static_cast<_Float16>(csum - static_cast<float>(shi));
    const uint32_t h2 = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, shi)) * 0x10001u;
    const uint32_t l2 = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, slo)) * 0x10001u;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) sr[0][i] = lane < 32 ? h2 : l2;
  }
  okr[0] = load_codes(0, cr[0]);

  uint4 bqr[KT];   // the bias operand, the same for every group: kept in registers
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) bqr[kt] = s_bq[kt * 64 + lane];
  float qs[HPL][8];
  float bias = 0.f;
  if (steps > 0) {
    read_qs(qs);
    if constexpr (TQ) bias = sw_produce<D, true>(sr[0], stage_a, slot_a, qs, bqr, lane, kg, 2.f * a.chalf);
    else bias = sw_produce<D>(sr[0], stage_a, slot_a, qs, bqr, lane, kg);
  }
  auto step = [&](int j, auto ring) {
    constexpr int r = decltype(ring)::value;
    constexpr int r2 = r ^ 1;
    SwSlot<D>* slot_cur = (r && !TQ) ? slot_b : slot_a;
    SwSlot<D>* slot_nxt = r ? slot_a : slot_b;
    uint16_t* stage_nxt = r ? stage_a : stage_b;
    okr[r2] = load_codes(j + 1, cr[r2]);
    // A group on an unmapped page (or past the run) costs only its loop
    // step: no scores, no operands for it, no softmax (the branches are
    // uniform; a skipped group leaves its q~ slot untouched).
    SwFront<D> f;
    if (okr[r]) sw_front<D, BITS>(cr[r], slot_cur, kg, col, tab, lane_off, f);
    float bias_next = bias;
    if constexpr (!TQ) {
      if (j + 1 < steps && okr[r2]) bias_next = sw_produce<D>(sr[r2], stage_nxt, slot_nxt, qs, bqr, lane, kg);
      load_stats(j + 2, sr[r]);
    }
    const int t0 = tb + (wave + NW * j) * kGroupTokens;
    if (okr[r])
      sw_back1<D, SLOTS, ASYM, TQ, BITS>(cr[r], f, bias, min(te - t0, kGroupTokens), kg, col, tab, lane_off, ws,
                                         a.value_scale);
    bias = bias_next;
  };
  for (int j = 0; j < steps; j += 2) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 < steps) step(j + 1, std::integral_constant<int, 1>{});
  }

  // ---- merge the wavefronts of the workgroup
  const int c = wave;
  const int slot_c = col / GP, hp = col % GP;
  const float l_col = rows_sum(ws.l_run);
  if (kg == 0) {
    s_m[c][col] = ws.m_run - ws.wshift;   // the reference of the scaled sums
    s_l[c][col] = l_col;
    if (slot_c < SLOTS) {
#pragma unroll
      for (int k = 0; k < NSETS; ++k) {
        const int m = k * SLOTS + slot_c;
        if (m < kModalities) s_s[c][m][hp] = ASYM ? ws.accs[ASYM ? k : 0][0] : 0.f;
      }
    }
  }
  const int wm = wave_or_bits(ws.mask);
  if (lane == 0) {
    s_cmask[c] = wm;
    if (wm) atomicOr(&s_mask, wm);
  }
  __syncthreads();   // the table and slots are dead from here on
  {
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][hp]);
    const float mw = s_m[c][hp];
    const float e = (mw == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    // only columns of a real head whose modality received weight are handed over
#pragma unroll
    for (int k = 0; k < NSETS; ++k) {
      if (!(wm & set_bits<SLOTS>(k))) continue;
      const int m = k * SLOTS + slot_c;
      if (slot_c < SLOTS && m < kModalities && hp < G && ((wm >> m) & 1)) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const floatx4 v = ws.acc[k][ct] * e;
          sm.red[c][(k * CT + ct) * 64 + lane] = float4{v[0], v[1], v[2], v[3]};
        }
      }
    }
  }
  __syncthreads();
  const int wmask = s_mask;
  for (int pos = tid; pos < NPOS; pos += NT) {
    const int ln = pos & 63, kct = pos >> 6;
    const int k = kct / CT, ct = kct % CT;
    const int c2 = ln & 15, kg2 = ln >> 4;
    const int sl2 = c2 / GP, hp2 = c2 % GP;
    const int m = k * SLOTS + sl2;
    if (sl2 < SLOTS && m < kModalities && hp2 < G && (wmask & (1 << m))) {
      // all reads first (a wavefront that did not touch modality m left its
      // slot unwritten: selected away, in a fixed order)
      float4 v[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) v[w] = sm.red[w][pos];
      float4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const bool t = (s_cmask[w] >> m) & 1;
        sum.x += t ? v[w].x : 0.f;
        sum.y += t ? v[w].y : 0.f;
        sum.z += t ? v[w].z : 0.f;
        sum.w += t ? v[w].w : 0.f;
      }
      float* part = a.partials + (static_cast<size_t>(h * G + hp2) * a.pstride + pl.slot0 + split) * PS;
      *reinterpret_cast<float4*>(part + kPartialHeader + m * D + 16 * ct + 4 * kg2) = sum;
    }
  }
  if (tid < G * kPartialHeader) {
    const int hh = tid / kPartialHeader, f = tid % kPartialHeader;
    float* part = a.partials + (static_cast<size_t>(h * G + hh) * a.pstride + pl.slot0 + split) * PS;
    float Mh = -__builtin_inff();
    for (int w = 0; w < NW; ++w) Mh = fmaxf(Mh, s_m[w][hh]);
    float v = 0.f;
    if (f == 0) {
      v = Mh;
    } else if (f == 1 || (f >= 4 && f < 4 + kModalities)) {
      for (int w = 0; w < NW; ++w) {
        const float mww = s_m[w][hh];
        if (mww != -__builtin_inff())
          v += __builtin_amdgcn_exp2f(mww - Mh) * (f == 1 ? s_l[w][hh] : s_s[w][f - 4][hh]);
      }
    } else if (f == 2) {
      v = __int_as_float(wmask);
    }
    part[f] = v;
  }
}

// Merge: workgroup (session, query head, row block) rescales every
// partition's partial to the global max, sums them per modality, and applies
// the rows [rb D/RB, (rb+1) D/RB) of the inverse value rotations,
// out = sum_m R_m A_m / l.  Every global load (headers, accumulator blocks,
// rotation rows) is issued before the first reduction, so the kernel costs
// one memory round trip; all sums run in a fixed order (bitwise
// reproducible).  All workgroups of one KV head are numbered so that they
// land on the same XCD (workgroups are dealt to the 8 XCDs round robin) and
// share the head's rotations and partials through that XCD's L2.
constexpr int kMergeThreads = 512;
constexpr int kMergeChunk = 16;    // partial blocks in flight per thread
constexpr int kXcds = 8;

template <int D>
struct MergeShape {
  static constexpr int RB = D / 32;                 // row blocks per head
  static constexpr int RR = D / RB;                 // rows per block
};

// STEP (the fused decode step's merge): the partials include the open
// group's (the last one of each head), and one workgroup per session
// advances its length.
template <int D, bool ASYM, bool STEP = false>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PS = kPartialHeader + kModalities * D;
  constexpr int F4 = D / 4;                        // float4 per accumulator block
  constexpr int NCOL = kModalities * F4;           // (modality, float4) columns
  constexpr int SG = kMergeThreads / NCOL;         // split subsets
  constexpr int RB = MergeShape<D>::RB;
  constexpr int RR = MergeShape<D>::RR;
  constexpr int QT = kMergeThreads / RR;           // threads per output row
  constexpr int JQ = D / QT;                       // columns of R per thread
  constexpr int NW = kMergeThreads / 64;
  static_assert(JQ % 4 == 0, "rotation columns per thread");
  __shared__ float s_e[kMaxSplits];
  __shared__ uint8_t s_mk[kMaxSplits];
  __shared__ float4 s_part[SG][NCOL];
  __shared__ float s_A[kModalities][D];
  __shared__ float s_red[NW][2 + kModalities];
  __shared__ float s_M;
  static_assert(!(STEP && ASYM), "the fused step takes a symmetric codebook");

  // Workgroup -> (session b, KV head h, query head of the group gq, row
  // block rb): every workgroup of one (session, KV head) key sits on the XCD
  // key mod 8 (workgroups are dealt to the XCDs round robin), so the key's
  // rotations and partials are fetched from HBM once and shared through that
  // XCD's L2; with fewer than 8 keys the other XCDs stay idle.
  const int x = blockIdx.x % kXcds, y = blockIdx.x / kXcds;
  const int per_key = a.group * RB;
  const int keys = a.batch * a.hkv;
  const int key = (y / per_key) * kXcds + x;       // b * Hkv + h
  const int item = y % per_key;
  if (key >= keys) return;
  const int gq = item / RB, rb = item % RB;
  const int h = key % a.hkv;
  const int i = h * a.group + gq;
  const int hi = (key / a.hkv) * a.hq + i;         // b * Hq + i
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = key / a.hkv;
  int slot0, S;
  if (a.ntab > 0) {
    slot0 = a.tab_start[b];
    S = a.tab_start[b + 1] - slot0;
  } else {
    slot0 = b * (a.splits + a.step);
    S = a.splits + a.step;
  }
  const size_t head = static_cast<size_t>(hi);
  const float* P = a.partials + (static_cast<size_t>(i) * a.pstride + slot0) * PS;

  // Rotation rows: row rb RR + tid / QT, columns [q JQ, (q+1) JQ) of all three R_m.
  const int rloc = tid / QT, q = tid % QT;
  const int row = rb * RR + rloc;
  float4 R[kModalities][JQ / 4];
#pragma unroll
  for (int m = 0; m < kModalities; ++m) {
    const float4* Rp = reinterpret_cast<const float4*>(
        a.rot + ((static_cast<size_t>(h) * kModalities + m) * D + row) * D + q * JQ);
#pragma unroll
    for (int j4 = 0; j4 < JQ / 4; ++j4) R[m][j4] = Rp[j4];
  }
  // First chunk of this thread's accumulator blocks: column (m, f4), splits
  // g, g + SG, ... (indices past the last split re-read it: the loads stay
  // branch-free, so they are all in flight at once; the extra values are
  // never used).
  const int col = tid % NCOL, g = tid / NCOL;
  const bool loader = g < SG;
  const int cm = col / F4, cf = col % F4;
  // (every thread loads, the clamped indices stay inside the head's partials;
  // only the loaders' values are used)
  float4 blk[kMergeChunk];
#pragma unroll
  for (int k = 0; k < kMergeChunk; ++k) {
    const int s = min(g + k * SG, S - 1);
    blk[k] = reinterpret_cast<const float4*>(P + static_cast<size_t>(s) * PS + kPartialHeader + cm * D)[cf];
  }
  // Headers: [m, l, mask, -, S0, S1, S2, -] of splits tid, tid + 512, ...
  // (the first one stays in registers).
  const float4 ninf4 = {-__builtin_inff(), 0.f, 0.f, 0.f};
  const float4 hd0r = reinterpret_cast<const float4*>(P + static_cast<size_t>(min(tid, S - 1)) * PS)[0];
  const float4 hd0 = tid < S ? hd0r : ninf4;
  float4 hd1 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (ASYM) {
    if (tid < S) hd1 = reinterpret_cast<const float4*>(P + static_cast<size_t>(tid) * PS)[1];
  }
  float mx = hd0.x;
  for (int s = tid + kMergeThreads; s < S; s += kMergeThreads) mx = fmaxf(mx, P[static_cast<size_t>(s) * PS]);
  mx = wave_max(mx);
  if (lane == 0) s_red[wave][0] = mx;
  __syncthreads();
  if (tid == 0) {
    float M = s_red[0][0];
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_red[w][0]);
    s_M = M;
  }
  __syncthreads();
  const float M = s_M;
  float ls = 0.f, ss[kModalities] = {0.f, 0.f, 0.f};
  for (int s = tid; s < S; s += kMergeThreads) {
    const float4 h0 = s == tid ? hd0 : reinterpret_cast<const float4*>(P + static_cast<size_t>(s) * PS)[0];
    const float e = (h0.x == -__builtin_inff()) ? 0.f : exp2f(h0.x - M);
    const int pm = e > 0.f ? __float_as_int(h0.z) : 0;
    s_e[s] = e;
    s_mk[s] = static_cast<uint8_t>(pm);
    ls += e * h0.y;
    if constexpr (ASYM) {
      const float4 h1 = s == tid ? hd1 : reinterpret_cast<const float4*>(P + static_cast<size_t>(s) * PS)[1];
      ss[0] += (pm & 1) ? e * h1.x : 0.f;
      ss[1] += (pm & 2) ? e * h1.y : 0.f;
      ss[2] += (pm & 4) ? e * h1.z : 0.f;
    }
  }
  ls = wave_sum(ls);
  if constexpr (ASYM)
#pragma unroll
    for (int m = 0; m < kModalities; ++m) ss[m] = wave_sum(ss[m]);
  if (lane == 0) {
    s_red[wave][1] = ls;
#pragma unroll
    for (int m = 0; m < kModalities; ++m) s_red[wave][2 + m] = ss[m];
  }
  __syncthreads();

  // Weighted sums of the accumulator blocks (absent modalities are selected
  // away, never multiplied: their blocks hold stale data).
  if (loader) {
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint8_t bit = static_cast<uint8_t>(1u << cm);
    for (int base = 0; base < S; base += kMergeChunk * SG) {
      if (base > 0) {
#pragma unroll
        for (int k = 0; k < kMergeChunk; ++k) {
          const int s = min(base + g + k * SG, S - 1);
          blk[k] = reinterpret_cast<const float4*>(P + static_cast<size_t>(s) * PS + kPartialHeader + cm * D)[cf];
        }
      }
      // weights and masks of the chunk first (no branch between the LDS
      // reads), then the sums in split order
      float ek[kMergeChunk];
      bool pk[kMergeChunk];
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) {
        const int s = base + g + k * SG;
        const int sc = min(s, S - 1);
        ek[k] = s_e[sc];
        pk[k] = (s < S) & ((s_mk[sc] & bit) != 0);   // both sides read: no branch
      }
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) {
        acc.x += pk[k] ? ek[k] * blk[k].x : 0.f;
        acc.y += pk[k] ? ek[k] * blk[k].y : 0.f;
        acc.z += pk[k] ? ek[k] * blk[k].z : 0.f;
        acc.w += pk[k] ? ek[k] * blk[k].w : 0.f;
      }
    }
    s_part[g][col] = acc;
  }
  __syncthreads();
  if (tid < NCOL) {
    float4 v = s_part[0][tid];
#pragma unroll
    for (int gg = 1; gg < SG; ++gg) {
      v.x += s_part[gg][tid].x;
      v.y += s_part[gg][tid].y;
      v.z += s_part[gg][tid].z;
      v.w += s_part[gg][tid].w;
    }
    const int m = tid / F4, f = tid % F4;
    s_A[m][4 * f + 0] = v.x;
    s_A[m][4 * f + 1] = v.y;
    s_A[m][4 * f + 2] = v.z;
    s_A[m][4 * f + 3] = v.w;
  }
  __syncthreads();

  // out[row] = (chalf sum_m R_m A_m + cmid sum_m S_m rowsum(R_m)) / (sqrt(d) l)
  float l = 0.f, Sm[kModalities] = {0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    l += s_red[w][1];
#pragma unroll
    for (int m = 0; m < kModalities; ++m) Sm[m] += s_red[w][2 + m];
  }
  float acc = 0.f, rs = 0.f;
#pragma unroll
  for (int m = 0; m < kModalities; ++m) {
    float am = 0.f, rm = 0.f;
#pragma unroll
    for (int j4 = 0; j4 < JQ / 4; ++j4) {
      const float* A = &s_A[m][q * JQ + 4 * j4];
      const float4 r = R[m][j4];
      am += r.x * A[0] + r.y * A[1] + r.z * A[2] + r.w * A[3];
      if constexpr (ASYM) rm += r.x + r.y + r.z + r.w;
    }
    acc += am;
    if constexpr (ASYM) rs += Sm[m] * rm;
  }
  static_assert(QT == 16, "one output row per 16-lane row");
  acc = row16_sum(acc);
  if constexpr (ASYM) rs = row16_sum(rs);
  if constexpr (STEP) {
    // one workgroup per session advances its length (nothing else in this
    // launch reads it)
    if (tid == 0 && item == 0 && h == 0) a.step_len[b] += 1;
  }
  if (q == 0) {
    const float o = (l > 0.f) ? (a.chalf * acc + a.cmid * rs) * (a.value_scale / l) : 0.f;
    if (a.out_bf16)
      static_cast<uint16_t*>(a.out)[head * D + row] = f32_to_bf16_rne(o);
    else
      static_cast<float*>(a.out)[head * D + row] = o;
  }
}

// Merge for few partials per query head (every session's partitions plus
// the step's slot at most kMergeHeadsSplits): workgroup (session, KV head,
// row block) takes every query head of the group, so the rows of the three
// inverse value rotations are loaded once for the G heads (the per-head
// merge loads them once per head, which dominates when each head has only a
// few partials to reduce).  Every load (rotation rows, headers, accumulator
// blocks) is issued before the first reduction; per head the partials are
// rescaled to the head's max and summed per modality in partition order,
// then out = sum_m R_m A_m / l for the block's rows.  The workgroups of one
// key sit on the XCD key mod 8, as in the per-head merge.
constexpr int kMergeHeadsSplits = 8;

template <int D, bool ASYM, bool STEP = false>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_heads_kernel(DecodeArgs a) {
  constexpr int PS = kPartialHeader + kModalities * D;
  constexpr int F4 = D / 4;                        // float4 per accumulator block
  constexpr int RB = MergeShape<D>::RB;
  constexpr int RR = MergeShape<D>::RR;
  constexpr int QT = kMergeThreads / RR;           // threads per output row
  constexpr int JQ = D / QT;                       // columns of R per thread
  constexpr int SM = kMergeHeadsSplits;
  constexpr int NIT = kMaxGroupHeads * kModalities * F4;   // (head, modality, float4) items at most
  constexpr int NI = (NIT + kMergeThreads - 1) / kMergeThreads;
  static_assert(JQ % 4 == 0 && QT == 16, "one output row per 16-lane row");
  static_assert(!(STEP && ASYM), "the fused step takes a symmetric codebook");
  __shared__ float s_hm[kMaxGroupHeads][SM];
  __shared__ float s_hl[kMaxGroupHeads][SM];
  __shared__ float s_hs[kMaxGroupHeads][SM][kModalities];
  __shared__ uint8_t s_mk[kMaxGroupHeads][SM];
  __shared__ float s_e[kMaxGroupHeads][SM];
  __shared__ float s_l[kMaxGroupHeads];
  __shared__ float s_sm[kMaxGroupHeads][kModalities];
  __shared__ float s_A[kMaxGroupHeads][kModalities][D];

  const int x = blockIdx.x % kXcds, y = blockIdx.x / kXcds;
  const int keys = a.batch * a.hkv;
  const int key = (y / RB) * kXcds + x;            // b * Hkv + h
  const int rb = y % RB;
  if (key >= keys) return;
  const int h = key % a.hkv, b = key / a.hkv, G = a.group;
  const int tid = threadIdx.x;
  int slot0, S;
  if (a.ntab > 0) {
    slot0 = a.tab_start[b];
    S = a.tab_start[b + 1] - slot0;
  } else {
    slot0 = b * (a.splits + a.step);
    S = a.splits + a.step;
  }
  auto head_partials = [&](int gq) {
    return a.partials + (static_cast<size_t>(h * G + gq) * a.pstride + slot0) * PS;
  };

  // Rotation rows: row rb RR + tid / QT, columns [q JQ, (q+1) JQ) of all three R_m.
  const int rloc = tid / QT, q = tid % QT;
  const int row = rb * RR + rloc;
  float4 R[kModalities][JQ / 4];
#pragma unroll
  for (int m = 0; m < kModalities; ++m) {
    const float4* Rp = reinterpret_cast<const float4*>(
        a.rot + ((static_cast<size_t>(h) * kModalities + m) * D + row) * D + q * JQ);
#pragma unroll
    for (int j4 = 0; j4 < JQ / 4; ++j4) R[m][j4] = Rp[j4];
  }
  // Accumulator blocks: item it = (head, modality, float4) of every split
  // (indices past the last split re-read it: branch-free, all in flight).
  const int nit = G * kModalities * F4;
  float4 blk[NI][SM];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    if (u * kMergeThreads >= nit) break;           // (uniform) no item of this round
    const int it = min(tid + u * kMergeThreads, nit - 1);
    const int gq = it / (kModalities * F4), m = (it / F4) % kModalities, f = it % F4;
    const float* P = head_partials(gq);
#pragma unroll
    for (int sp = 0; sp < SM; ++sp)
      blk[u][sp] = reinterpret_cast<const float4*>(P + static_cast<size_t>(min(sp, S - 1)) * PS + kPartialHeader +
                                                   m * D)[f];
  }
  // Headers of (head, split) = (t / SM, t % SM).
  for (int t = tid; t < G * SM; t += kMergeThreads) {
    const int gq = t / SM, sp = t % SM;
    float4 h0 = {-__builtin_inff(), 0.f, 0.f, 0.f}, h1 = {0.f, 0.f, 0.f, 0.f};
    if (sp < S) {
      const float4* hp = reinterpret_cast<const float4*>(head_partials(gq) + static_cast<size_t>(sp) * PS);
      h0 = hp[0];
      if constexpr (ASYM) h1 = hp[1];
    }
    s_hm[gq][sp] = h0.x;
    s_hl[gq][sp] = h0.y;
    s_mk[gq][sp] = static_cast<uint8_t>(h0.x == -__builtin_inff() ? 0 : __float_as_int(h0.z));
    s_hs[gq][sp][0] = h1.x;
    s_hs[gq][sp][1] = h1.y;
    s_hs[gq][sp][2] = h1.z;
  }
  __syncthreads();
  // Per head: its max, the splits' weights, l and (asymmetric codebook) the
  // per-modality weight sums, in split order.
  if (tid < G) {
    const int gq = tid;
    float M = -__builtin_inff();
    for (int sp = 0; sp < S; ++sp) M = fmaxf(M, s_hm[gq][sp]);
    float l = 0.f, sm[kModalities] = {0.f, 0.f, 0.f};
    for (int sp = 0; sp < SM; ++sp) {
      const float mv = s_hm[gq][sp];
      const float e = (sp >= S || mv == -__builtin_inff()) ? 0.f : exp2f(mv - M);
      s_e[gq][sp] = e;
      l += e * s_hl[gq][sp];
      if constexpr (ASYM) {
        const int pm = s_mk[gq][sp];
#pragma unroll
        for (int m = 0; m < kModalities; ++m) sm[m] += (pm >> m) & 1 ? e * s_hs[gq][sp][m] : 0.f;
      }
    }
    s_l[gq] = l;
#pragma unroll
    for (int m = 0; m < kModalities; ++m) s_sm[gq][m] = sm[m];
  }
  __syncthreads();
  // Weighted sums of the accumulator blocks, in split order (absent
  // modalities are selected away, never multiplied: their blocks hold stale
  // data).
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int it = tid + u * kMergeThreads;
    if (it < nit) {
      const int gq = it / (kModalities * F4), m = (it / F4) % kModalities, f = it % F4;
      float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sp = 0; sp < SM; ++sp) {
        const bool p = sp < S && ((s_mk[gq][sp] >> m) & 1);
        const float e = s_e[gq][sp];
        acc.x += p ? e * blk[u][sp].x : 0.f;
        acc.y += p ? e * blk[u][sp].y : 0.f;
        acc.z += p ? e * blk[u][sp].z : 0.f;
        acc.w += p ? e * blk[u][sp].w : 0.f;
      }
      *reinterpret_cast<float4*>(&s_A[gq][m][4 * f]) = acc;
    }
  }
  __syncthreads();
  if constexpr (STEP) {
    // one workgroup per session advances its length (nothing else in this
    // launch reads it)
    if (tid == 0 && rb == 0 && h == 0) a.step_len[b] += 1;
  }
  // out[row] = (chalf sum_m R_m A_m + cmid sum_m S_m rowsum(R_m)) / (sqrt(d) l), per head
  float rsum[kModalities] = {0.f, 0.f, 0.f};
  if constexpr (ASYM) {
#pragma unroll
    for (int m = 0; m < kModalities; ++m) {
      float rm = 0.f;
#pragma unroll
      for (int j4 = 0; j4 < JQ / 4; ++j4) rm += R[m][j4].x + R[m][j4].y + R[m][j4].z + R[m][j4].w;
      rsum[m] = row16_sum(rm);
    }
  }
  for (int gq = 0; gq < G; ++gq) {
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < kModalities; ++m) {
      float am = 0.f;
#pragma unroll
      for (int j4 = 0; j4 < JQ / 4; ++j4) {
        const float* A = &s_A[gq][m][q * JQ + 4 * j4];
        const float4 r = R[m][j4];
        am += r.x * A[0] + r.y * A[1] + r.z * A[2] + r.w * A[3];
      }
      acc += am;
    }
    acc = row16_sum(acc);
    if (q == 0) {
      float rs = 0.f;
      if constexpr (ASYM)
#pragma unroll
        for (int m = 0; m < kModalities; ++m) rs += s_sm[gq][m] * rsum[m];
      const float l = s_l[gq];
      const float o = (l > 0.f) ? (a.chalf * acc + a.cmid * rs) * (a.value_scale / l) : 0.f;
      const size_t head = static_cast<size_t>(b) * a.hq + h * G + gq;
      if (a.out_bf16)
        static_cast<uint16_t*>(a.out)[head * D + row] = f32_to_bf16_rne(o);
      else
        static_cast<float*>(a.out)[head * D + row] = o;
    }
  }
}

// Grid of a partition launch (see the plan in DecodeArgs).
dim3 partition_grid(int batch, const DecodeArgs& a) {
  return a.ntab > 0 ? dim3(a.pstride, a.hkv, 1) : dim3(a.splits + a.step, a.hkv, batch);
}

template <int D, int SLOTS, int NW>
void launch_partition(int batch, const DecodeArgs& a, hipStream_t s) {
  constexpr bool BHL = SLOTS >= 2;   // G <= 8
  const dim3 grid = partition_grid(batch, a);
  if (a.cmid != 0.f)
    hipLaunchKernelGGL((decode_partition_kernel<D, SLOTS, NW, true, BHL>), grid, dim3(NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((decode_partition_kernel<D, SLOTS, NW, false, BHL>), grid, dim3(NW * 64), 0, s, a);
}

template <int D, int SLOTS, int BITS>
void launch_partition_sw_bits(int batch, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid = partition_grid(batch, a);
  const dim3 block(kSwWaves * 64);
  if (a.key_mode == KVQ_KEYS_PER_TOKEN) {
    if (a.cmid != 0.f)
      hipLaunchKernelGGL((decode_partition_sw_kernel<D, SLOTS, true, true, BITS>), grid, block, 0, s, a,
                         AppendArgs{});
    else
      hipLaunchKernelGGL((decode_partition_sw_kernel<D, SLOTS, false, true, BITS>), grid, block, 0, s, a,
                         AppendArgs{});
  } else {
    if (a.cmid != 0.f)
      hipLaunchKernelGGL((decode_partition_sw_kernel<D, SLOTS, true, false, BITS>), grid, block, 0, s, a,
                         AppendArgs{});
    else
      hipLaunchKernelGGL((decode_partition_sw_kernel<D, SLOTS, false, false, BITS>), grid, block, 0, s, a,
                         AppendArgs{});
  }
}

template <int D, int SLOTS>
void launch_partition_sw(int batch, const DecodeArgs& a, hipStream_t s) {
  if (a.bits == 4) launch_partition_sw_bits<D, SLOTS, 4>(batch, a, s);
  else if (a.bits == 3) launch_partition_sw_bits<D, SLOTS, 3>(batch, a, s);
  else launch_partition_sw_bits<D, SLOTS, 2>(batch, a, s);
}

// Merge grid: per (session, KV head) key, group * RB workgroups (RB with few
// partials per head, decode_merge_heads_kernel), all on the XCD key mod 8
// (see decode_merge_kernel).
template <int D, bool ASYM, bool STEP>
void launch_merge(int batch, const DecodeArgs& a, hipStream_t s) {
  const int keys = a.hkv * batch;
  if (a.splits + a.step <= kMergeHeadsSplits) {
    // few partials per head: one workgroup per (key, row block) for all heads
    const int rows = ((keys + kXcds - 1) / kXcds) * MergeShape<D>::RB;
    hipLaunchKernelGGL((decode_merge_heads_kernel<D, ASYM, STEP>), dim3(kXcds * rows), dim3(kMergeThreads), 0, s,
                       a);
    return;
  }
  const int per_key = a.group * MergeShape<D>::RB;
  const int rows = ((keys + kXcds - 1) / kXcds) * per_key;
  hipLaunchKernelGGL((decode_merge_kernel<D, ASYM, STEP>), dim3(kXcds * rows), dim3(kMergeThreads), 0, s, a);
}

template <int D>
hipError_t launch_decode_t(int batch, const DecodeArgs& a, hipStream_t s) {
  if (!a.offsets31 || a.page_shift < 0) launch_partition<D, 1, kDecodeWaves / 2>(batch, a, s);
  else if (a.group <= 5) launch_partition_sw<D, 3>(batch, a, s);
  else if (a.group <= 8) launch_partition_sw<D, 2>(batch, a, s);
  else launch_partition<D, 1, kDecodeWaves / 2>(batch, a, s);
  if (a.cmid != 0.f) launch_merge<D, true, false>(batch, a, s);
  else launch_merge<D, false, false>(batch, a, s);
  return hipGetLastError();
}

// Fused decode step: partitions + the append's two workgroups per (session,
// KV head) in one grid (2-bit codes, group statistics, symmetric codebook,
// G <= 8, power-of-two pages, 31-bit offsets: the caller checks), then the
// merge with the open group.
template <int D, int SLOTS, bool BF16>
void launch_step_partition(int batch, const DecodeArgs& a, const AppendArgs& ap, hipStream_t s) {
  const dim3 grid = partition_grid(batch, a);
  hipLaunchKernelGGL((decode_partition_sw_kernel<D, SLOTS, false, false, 2, true, BF16>), grid,
                     dim3(kSwWaves * 64), 0, s, a, ap);
}

template <int D>
hipError_t launch_decode_step_t(bool bf16, int batch, const DecodeArgs& a, const AppendArgs& ap, hipStream_t s) {
  if (a.group <= 5) {
    if (bf16) launch_step_partition<D, 3, true>(batch, a, ap, s);
    else launch_step_partition<D, 3, false>(batch, a, ap, s);
  } else {
    if (bf16) launch_step_partition<D, 2, true>(batch, a, ap, s);
    else launch_step_partition<D, 2, false>(batch, a, ap, s);
  }
  launch_merge<D, false, true>(batch, a, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int d, int batch, const DecodeArgs& a, hipStream_t s) {
  return d == 64 ? launch_decode_t<64>(batch, a, s) : launch_decode_t<128>(batch, a, s);
}

hipError_t launch_decode_step(int d, bool bf16, int batch, const DecodeArgs& a, const AppendArgs& ap,
                              hipStream_t s) {
  return d == 64 ? launch_decode_step_t<64>(bf16, batch, a, ap, s) : launch_decode_step_t<128>(bf16, batch, a, ap, s);
}

}  // namespace kvq
