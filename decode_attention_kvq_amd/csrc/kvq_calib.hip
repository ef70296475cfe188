// Value-basis calibration (kvq_calib.h): attention-contribution weights,
// weighted per-modality covariances and their eigenbases, all in fp64.
//
// OmniKVQuant page, Sec. 2 Method, second "OmniKVQuant" bullet: value
// directions are weighted by their contribution to attention outputs, a
// covariance is formed per modality, and its eigenbasis is the modality's
// rotation.  Calibration runs once, off the decode path; every sum below has
// a fixed order, so results do not depend on timing.
//
// fp64 matrix and vector peaks are the same on this chip: the scores run on
// the vector ALUs with fp64 FMAs, the covariance (a product of staged tiles)
// on the fp64 matrix cores, where one instruction takes 1,024 multiply-adds
// from two operand registers per lane instead of reading them from LDS.
#include <math.h>

#include <algorithm>

#include "kvq_calib.h"
#include "kvq_common.h"

namespace kvq {
namespace {

constexpr int kCalibModalities = 3;
constexpr int kRowChunk = 16;        // query rows whose scores a thread forms together
constexpr int kTokBlock = 256;       // tokens per workgroup in the score kernels
constexpr int kJacobiSweeps = 50;    // hard cap on Jacobi sweeps

// ------------------------------------------------------------ contribution

struct ContribArgs {
  const void* k;          // [n][hkv][D]
  const void* q;          // [nq][hq][D]
  double* weights;        // [hkv][n]
  double* part;           // [hkv][nblk][rows][2] per-block (max, sum)
  double* stats;          // [hkv][rows][2] final (max, sum)
  int32_t n, hkv, hq, group, rows, nblk;
  double scale;
};

// Scores of token t against kRowChunk staged query rows, each an fp64 dot
// product accumulated with FMAs in channel order 0 .. D-1.  Both score
// kernels use this one routine, so they see bitwise identical scores.
template <int D, bool KB>
__device__ __forceinline__ void chunk_dots(const void* k, size_t row_off, const double (*sq)[D],
                                           double (&dot)[kRowChunk]) {
#pragma unroll
  for (int r = 0; r < kRowChunk; ++r) dot[r] = 0.0;
  for (int c = 0; c < D; c += 8) {
    double kv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) kv[u] = load_input<KB>(k, row_off + c + u);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int r = 0; r < kRowChunk; ++r) dot[r] = __builtin_fma(kv[u], sq[r][c + u], dot[r]);
  }
}

// Stage query rows r0 .. r0 + kRowChunk - 1 of KV head h (row r = query
// i * G + head g) as fp64; rows past `rows` are zero.
template <int D, bool QB>
__device__ __forceinline__ void stage_rows(const ContribArgs& a, int h, int r0, double (*sq)[D]) {
  for (int e = threadIdx.x; e < kRowChunk * D; e += blockDim.x) {
    const int rr = e / D, c = e % D;
    const int r = r0 + rr;
    double v = 0.0;
    if (r < a.rows) {
      const int i = r / a.group, g = r % a.group;
      v = load_input<QB>(a.q, (static_cast<size_t>(i) * a.hq + h * a.group + g) * D + c);
    }
    sq[rr][c] = v;
  }
}

// (max, sum of exp(s - max)) merge; an empty side has max -inf and sum 0.
__device__ __forceinline__ void merge_ms(double& m, double& l, double m2, double l2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    l = l2;
    return;
  }
  const double M = fmax(m, m2);
  l = l * exp(m - M) + l2 * exp(m2 - M);
  m = M;
}

// Per (KV head, block of kTokBlock tokens, query row): max and sum of
// exp(score - max) over the block's tokens.  Thread = token.  The block max
// comes first (a max is exact in any order), then one exponential per
// (token, row), summed by a fixed butterfly in each wavefront and over the
// wavefronts in order.
template <int D, bool KB, bool QB>
__global__ __launch_bounds__(kTokBlock) void calib_block_stats_kernel(ContribArgs a) {
  constexpr int NWB = kTokBlock / 64;
  __shared__ double sq[kRowChunk][D];
  __shared__ double red[NWB][kRowChunk];
  __shared__ double s_bm[kRowChunk];
  const int h = blockIdx.y, blk = blockIdx.x;
  const int t = blk * kTokBlock + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool ok = t < a.n;
  const size_t row_off = (static_cast<size_t>(ok ? t : 0) * a.hkv + h) * D;
  for (int r0 = 0; r0 < a.rows; r0 += kRowChunk) {
    __syncthreads();
    stage_rows<D, QB>(a, h, r0, sq);
    __syncthreads();
    double dot[kRowChunk];
    chunk_dots<D, KB>(a.k, row_off, sq, dot);
    double sc[kRowChunk];
#pragma unroll
    for (int r = 0; r < kRowChunk; ++r) {
      sc[r] = ok ? a.scale * dot[r] : -INFINITY;
      double m = sc[r];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
      if (lane == 0) red[wave][r] = m;
    }
    __syncthreads();
    if (threadIdx.x < kRowChunk) {
      double m = red[0][threadIdx.x];
      for (int w = 1; w < NWB; ++w) m = fmax(m, red[w][threadIdx.x]);
      s_bm[threadIdx.x] = m;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRowChunk; ++r) {
      // a block has at least one token, so its max is finite
      double l = ok ? exp(sc[r] - s_bm[r]) : 0.0;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off, 64);
      if (lane == 0) red[wave][r] = l;
    }
    __syncthreads();
    if (threadIdx.x < kRowChunk && r0 + static_cast<int>(threadIdx.x) < a.rows) {
      const int r = threadIdx.x;
      double l = red[0][r];
      for (int w = 1; w < NWB; ++w) l += red[w][r];
      double* out = a.part + ((static_cast<size_t>(h) * a.nblk + blk) * a.rows + r0 + r) * 2;
      out[0] = s_bm[r];
      out[1] = l;
    }
  }
}

// Final (max, sum) per (KV head, row).  One wavefront per row: lane l merges
// blocks l, l + 64, ... in order, then a fixed butterfly merges the lanes.
__global__ __launch_bounds__(64) void calib_stats_merge_kernel(ContribArgs a) {
  const int r = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  double m = -INFINITY, l = 0.0;
  for (int b = lane; b < a.nblk; b += 64) {
    const double* p = a.part + ((static_cast<size_t>(h) * a.nblk + b) * a.rows + r) * 2;
    merge_ms(m, l, p[0], p[1]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double m2 = __shfl_xor(m, off, 64);
    const double l2 = __shfl_xor(l, off, 64);
    merge_ms(m, l, m2, l2);
  }
  if (lane == 0) {
    a.stats[(static_cast<size_t>(h) * a.rows + r) * 2] = m;
    a.stats[(static_cast<size_t>(h) * a.rows + r) * 2 + 1] = l;
  }
}

// w[h][t] = (1 / rows) sum_r exp(s_rt - m_r) / l_r, rows in order.
template <int D, bool KB, bool QB>
__global__ __launch_bounds__(kTokBlock) void calib_weights_kernel(ContribArgs a) {
  __shared__ double sq[kRowChunk][D];
  __shared__ double s_m[kRowChunk], s_l[kRowChunk];
  const int h = blockIdx.y;
  const int t = blockIdx.x * kTokBlock + threadIdx.x;
  const bool ok = t < a.n;
  const size_t row_off = (static_cast<size_t>(ok ? t : 0) * a.hkv + h) * D;
  double acc = 0.0;
  for (int r0 = 0; r0 < a.rows; r0 += kRowChunk) {
    __syncthreads();
    stage_rows<D, QB>(a, h, r0, sq);
    if (threadIdx.x < kRowChunk) {
      const int r = r0 + threadIdx.x;
      const bool in = r < a.rows;
      s_m[threadIdx.x] = in ? a.stats[(static_cast<size_t>(h) * a.rows + r) * 2] : 0.0;
      s_l[threadIdx.x] = in ? a.stats[(static_cast<size_t>(h) * a.rows + r) * 2 + 1] : 1.0;
    }
    __syncthreads();
    double dot[kRowChunk];
    chunk_dots<D, KB>(a.k, row_off, sq, dot);
    const int nr = min(kRowChunk, a.rows - r0);
#pragma unroll
    for (int r = 0; r < kRowChunk; ++r)
      if (r < nr) acc += exp(a.scale * dot[r] - s_m[r]) / s_l[r];
  }
  if (ok) a.weights[static_cast<size_t>(h) * a.n + t] = acc / static_cast<double>(a.rows);
}

// -------------------------------------------------------------- covariance

struct CovArgs {
  const void* v;            // [n][hkv][D]
  const uint8_t* modality;  // [n]
  const double* weights;    // [hkv][n]
  double* cov;              // [hkv][3][D][D]
  double* wsum;             // [hkv][3]
  double* part_mean;        // [mean_splits][hkv][3][D + 1]: sum w v (D entries), then sum w
  double* mean;             // [hkv][3][D]
  int32_t* order;           // [n]: the tokens grouped by modality (calib_group_*_kernel)
  int32_t* counts;          // [3]: tokens per modality
  int32_t* group_blk;       // [ceil(n / 1024)][3]: per-block counts, then starting positions
  double* part_cov;         // [S][hkv][3][D][D], entries i <= j
  int32_t n, hkv, splits;   // covariance: each modality's tokens in `splits` ranges
  int32_t mean_splits, mean_split_tokens;  // weighted-mean pass's token splits
};

// Eight consecutive inputs from element idx (a multiple of 8), exactly.
template <bool VB>
__device__ __forceinline__ void load8(const void* p, size_t idx, float (&x)[8]) {
  if constexpr (VB) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + idx);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + idx);
    const float4 a = q[0], b = q[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Partial weighted sums of one (split, KV head): thread = (token phase, 8
// channels); each phase takes the split's tokens ph, ph + P, ... in
// increasing order, and the phases are combined in phase order.
template <int D, bool VB>
__global__ __launch_bounds__(256) void calib_mean_part_kernel(CovArgs a) {
  constexpr int TPR = D / 8;        // threads per token row
  constexpr int P = 256 / TPR;      // token phases
  constexpr int U = 4;              // tokens whose loads are issued together
  __shared__ double s_wv[P][kCalibModalities][D];
  __shared__ double s_w[P][kCalibModalities];
  const int s = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int ph = tid / TPR, c0 = (tid % TPR) * 8;
  const int t0 = s * a.mean_split_tokens, t1 = min(a.n, t0 + a.mean_split_tokens);
  double wv[kCalibModalities][8], ws[kCalibModalities];
#pragma unroll
  for (int m = 0; m < kCalibModalities; ++m) {
    ws[m] = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) wv[m][i] = 0.0;
  }
  for (int tb = t0 + ph; tb < t1; tb += U * P) {
    int md[U];
    double wt[U];
    float x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + u * P;
      const bool in = t < t1;
      const int tt = in ? t : t0;
      md[u] = in ? a.modality[tt] : 3;
      wt[u] = a.weights[static_cast<size_t>(h) * a.n + tt];
      load8<VB>(a.v, (static_cast<size_t>(tt) * a.hkv + h) * D + c0, x[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)   // tokens in increasing order
#pragma unroll
      for (int m = 0; m < kCalibModalities; ++m) {
        const bool take = md[u] == m;
        ws[m] = take ? ws[m] + wt[u] : ws[m];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          wv[m][i] = take ? __builtin_fma(wt[u], static_cast<double>(x[u][i]), wv[m][i]) : wv[m][i];
      }
  }
#pragma unroll
  for (int m = 0; m < kCalibModalities; ++m)
#pragma unroll
    for (int i = 0; i < 8; ++i) s_wv[ph][m][c0 + i] = wv[m][i];
  if (c0 == 0)
#pragma unroll
    for (int m = 0; m < kCalibModalities; ++m) s_w[ph][m] = ws[m];
  __syncthreads();
  double* out = a.part_mean + (static_cast<size_t>(s) * a.hkv + h) * kCalibModalities * (D + 1);
  for (int e = tid; e < kCalibModalities * D; e += 256) {
    const int m = e / D, c = e % D;
    double x = s_wv[0][m][c];
    for (int p = 1; p < P; ++p) x += s_wv[p][m][c];
    out[m * (D + 1) + c] = x;
  }
  if (tid < kCalibModalities) {
    double w = s_w[0][tid];
    for (int p = 1; p < P; ++p) w += s_w[p][tid];
    out[tid * (D + 1) + D] = w;
  }
}

// Means and weight sums: the splits merged in split order.  Thread = (h, m, c).
template <int D>
__global__ __launch_bounds__(256) void calib_mean_merge_kernel(CovArgs a) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= a.hkv * kCalibModalities * D) return;
  const int c = e % D, hm = e / D;
  const int h = hm / kCalibModalities, m = hm % kCalibModalities;
  constexpr int U = 8;   // splits whose partial sums are loaded together
  const size_t stride = static_cast<size_t>(a.hkv) * kCalibModalities * (D + 1);
  const double* p0 = a.part_mean + (static_cast<size_t>(h) * kCalibModalities + m) * (D + 1);
  double sx = 0.0, sw = 0.0;
  for (int s0 = 0; s0 < a.mean_splits; s0 += U) {
    double x[U], w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = s0 + u < a.mean_splits;
      x[u] = in ? p0[(s0 + u) * stride + c] : 0.0;
      w[u] = in ? p0[(s0 + u) * stride + D] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {   // splits in increasing order
      sx += x[u];
      sw += w[u];
    }
  }
  a.mean[static_cast<size_t>(hm) * D + c] = sw > 0.0 ? sx / sw : 0.0;
  if (c == 0) a.wsum[hm] = sw;
}

// The calibration tokens grouped by modality, for the covariance: `order`
// lists the tokens of modality 0 in increasing order, then those of 1, then
// those of 2 (tokens with another modality byte are left out), and counts[m]
// is the number of tokens of modality m.  Three launches over blocks of
// 1,024 tokens: each block counts its tokens per modality; one workgroup
// turns the counts into each block's starting position per modality; each
// block writes its tokens there, ranked within the block by wavefront
// ballots (lanes in token order, wavefronts in order).
constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;

__device__ __forceinline__ int group_modality(const CovArgs& a, int t) {
  return t < a.n ? a.modality[t] : kCalibModalities;
}

__global__ __launch_bounds__(kGroupThreads) void calib_group_count_kernel(CovArgs a) {
  __shared__ int s_c[kGroupWaves][kCalibModalities];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = group_modality(a, b * kGroupThreads + tid);
#pragma unroll
  for (int k = 0; k < kCalibModalities; ++k) {
    const int c = __popcll(__ballot(m == k));
    if (lane == 0) s_c[wave][k] = c;
  }
  __syncthreads();
  if (tid < kCalibModalities) {
    int c = 0;
    for (int w = 0; w < kGroupWaves; ++w) c += s_c[w][tid];
    a.group_blk[static_cast<size_t>(b) * kCalibModalities + tid] = c;
  }
}

// Block counts -> starting positions (in place), and counts[m].
__global__ __launch_bounds__(kGroupThreads) void calib_group_scan_kernel(CovArgs a, int nblk) {
  __shared__ int s_sc[kCalibModalities][kGroupThreads];
  __shared__ int s_base[kCalibModalities];
  const int tid = threadIdx.x;
  int tot[kCalibModalities] = {0, 0, 0};
  for (int b = tid; b < nblk; b += kGroupThreads)
#pragma unroll
    for (int k = 0; k < kCalibModalities; ++k) tot[k] += a.group_blk[static_cast<size_t>(b) * kCalibModalities + k];
  // inclusive scans of s_sc[k][0 ..) over the threads (Hillis-Steele)
  auto scan = [&](const int (&c)[kCalibModalities]) {
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kCalibModalities; ++k) s_sc[k][tid] = c[k];
    __syncthreads();
    for (int off = 1; off < kGroupThreads; off <<= 1) {
      int v[kCalibModalities];
#pragma unroll
      for (int k = 0; k < kCalibModalities; ++k) v[k] = tid >= off ? s_sc[k][tid - off] : 0;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kCalibModalities; ++k) s_sc[k][tid] += v[k];
      __syncthreads();
    }
  };
  scan(tot);
  if (tid < kCalibModalities) a.counts[tid] = s_sc[tid][kGroupThreads - 1];
  if (tid == 0) {
    s_base[0] = 0;
    s_base[1] = s_sc[0][kGroupThreads - 1];
    s_base[2] = s_sc[0][kGroupThreads - 1] + s_sc[1][kGroupThreads - 1];
  }
  __syncthreads();
  int carry[kCalibModalities] = {s_base[0], s_base[1], s_base[2]};
  for (int b0 = 0; b0 < nblk; b0 += kGroupThreads) {
    const int b = b0 + tid;
    int c[kCalibModalities];
#pragma unroll
    for (int k = 0; k < kCalibModalities; ++k) c[k] = b < nblk ? a.group_blk[static_cast<size_t>(b) * kCalibModalities + k] : 0;
    scan(c);
    if (b < nblk)
#pragma unroll
      for (int k = 0; k < kCalibModalities; ++k)
        a.group_blk[static_cast<size_t>(b) * kCalibModalities + k] = carry[k] + s_sc[k][tid] - c[k];
#pragma unroll
    for (int k = 0; k < kCalibModalities; ++k) carry[k] += s_sc[k][kGroupThreads - 1];
  }
}

__global__ __launch_bounds__(kGroupThreads) void calib_group_scatter_kernel(CovArgs a) {
  __shared__ int s_c[kGroupWaves][kCalibModalities];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = b * kGroupThreads + tid;
  const int m = group_modality(a, t);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = 0;
#pragma unroll
  for (int k = 0; k < kCalibModalities; ++k) {
    const uint64_t mk = __ballot(m == k);
    if (m == k) rank = __popcll(mk & below);
    if (lane == 0) s_c[wave][k] = __popcll(mk);
  }
  __syncthreads();
  if (m < kCalibModalities) {
    int at = a.group_blk[static_cast<size_t>(b) * kCalibModalities + m] + rank;
    for (int w = 0; w < wave; ++w) at += s_c[w][m];
    a.order[at] = t;
  }
}

// Partial covariances of one (split s, KV head h) on the fp64 matrix cores,
// modality by modality: range s of modality m's tokens (`order`, each
// modality's list cut into `splits` ranges of a multiple of 4 tokens, so
// every workgroup gets the same share of every modality) goes through LDS
// 64 tokens at a time, and every 4 tokens are one k-step of
// v_mfma_f64_16x16x4f64 per 16 x 16 tile of the upper triangle:
// C[i][j] += sum_t (w_t x_ti) x_tj with x = v - mu_m (A: lane l holds
// token l / 16, channel i = l % 16 of the tile's rows; B the same token and
// column channel; x staged in LDS as fp64, centred once; D element r of lane l is entry (4 r + l / 16, l % 16)).
// The 36 (d = 128) or 10 (d = 64) tiles are dealt to 12 or 10 wavefronts,
// three or one each.
// Entries i <= j are stored; the merge mirrors them, so the result is
// exactly symmetric.  Each k-step adds its products in the matrix core's
// fixed order, k-steps in token order: the result depends only on the
// inputs and the plan.
typedef double calib_dx4 __attribute__((ext_vector_type(4)));
constexpr int kCovChunk = 64;   // tokens staged per step

template <int D>
struct CovShape {
  static constexpr int NB = D / 16;                 // 16-channel blocks
  static constexpr int NTL = NB * (NB + 1) / 2;     // tiles (bi <= bj): 36 or 10
  static constexpr int TPW = D == 128 ? 3 : 1;      // tiles per wavefront, the same for all
  static constexpr int NWV = NTL / TPW;             // wavefronts: 12 or 10
  static constexpr int NT = NWV * 64;
  static constexpr int LDX = D + 16;                // staged row stride in doubles: rows 4k, 4k + 1
                                                    // of a k-step (one half-wavefront) use disjoint banks
  static constexpr int PPR = D / 8;                 // staging pieces (8 channels) per token row
  static constexpr int NPC = (kCovChunk * PPR + NT - 1) / NT;   // pieces per thread at most
};

// Tile e of the NB (NB + 1) / 2 upper-triangle 16 x 16 tiles, row-major.
template <int NB>
__device__ __forceinline__ void cov_tile(int e, int& bi, int& bj) {
  bi = 0;
  while (e >= NB - bi) {
    e -= NB - bi;
    ++bi;
  }
  bj = bi + e;
}

template <int D, bool VB>
__global__ __launch_bounds__(CovShape<D>::NT) void calib_cov_part_kernel(CovArgs a) {
  using S = CovShape<D>;
  constexpr int TPW = S::TPW;
  constexpr int NT = S::NT;
  static_assert(S::NWV * TPW == S::NTL, "every wavefront takes TPW tiles");
  __shared__ double xs[kCovChunk][S::LDX];   // centred values x = v - mu_m of the chunk's tokens
  __shared__ double s_w[kCovChunk];
  __shared__ double s_mu[D];
  const int s = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // the wavefront's tiles TPW wave .. TPW wave + TPW - 1: LDS offsets of this
  // lane's channel in the tile's row and column blocks (a diagonal tile reads
  // the same channel twice: no branch in the loop)
  int ci[TPW], cj[TPW], bi[TPW], bj[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    cov_tile<S::NB>(TPW * wave + u, bi[u], bj[u]);
    ci[u] = 16 * bi[u] + (lane & 15);
    cj[u] = 16 * bj[u] + (lane & 15);
  }
  // staging: piece p = (token row p / PPR, channels 8 (p % PPR) ..) for
  // p = tid, tid + NT, ...; the raw 16-byte words of the next chunk are
  // loaded while this one is used (and waited for only when staged), its
  // token indices one chunk earlier still
  constexpr int EB = VB ? 2 : 4;                 // bytes per input element
  constexpr int WPP = 8 * EB / 16;               // 16-byte words per piece
  uint4 xr[S::NPC][WPP];
  double wr[S::NPC];
  bool vr[S::NPC];
  int tn[S::NPC];
  auto piece_ok = [&](int k) { return tid + k * NT < kCovChunk * S::PPR; };
  auto fetch = [&]() {
#pragma unroll
    for (int k = 0; k < S::NPC; ++k) {
      const int p = tid + k * NT;
      const int t = piece_ok(k) ? tn[k] : -1;
      const int tt = t >= 0 ? t : 0;
      const uint4* src = reinterpret_cast<const uint4*>(
          static_cast<const char*>(a.v) + ((static_cast<size_t>(tt) * a.hkv + h) * D + 8 * (p % S::PPR)) * EB);
#pragma unroll
      for (int q = 0; q < WPP; ++q) xr[k][q] = src[q];
      wr[k] = a.weights[static_cast<size_t>(h) * a.n + tt];
      vr[k] = t >= 0;
    }
  };

  int off = 0;
  for (int m = 0; m < kCalibModalities; ++m) {
    const int cnt = a.counts[m];
    const int64_t per = ((static_cast<int64_t>(cnt) + a.splits - 1) / a.splits + 3) & ~static_cast<int64_t>(3);
    const int r0 = static_cast<int>(min(static_cast<int64_t>(cnt), s * per));
    const int r1 = static_cast<int>(min(static_cast<int64_t>(cnt), r0 + per));
    auto tokens = [&](int base) {   // token of each of the thread's pieces in the chunk at base
#pragma unroll
      for (int k = 0; k < S::NPC; ++k) {
        const int r = base + (tid + k * NT) / S::PPR;
        tn[k] = r < r1 ? a.order[static_cast<size_t>(off) + r] : -1;
      }
    };
    calib_dx4 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = calib_dx4{0.0, 0.0, 0.0, 0.0};
    __syncthreads();   // the previous modality's staging has read s_mu
    if (tid < D) s_mu[tid] = a.mean[(static_cast<size_t>(h) * kCalibModalities + m) * D + tid];
    if (r0 < r1) {
      tokens(r0);
      fetch();
      tokens(r0 + kCovChunk);
    }
    for (int base = r0; base < r1; base += kCovChunk) {
      __syncthreads();   // s_mu is set; the previous chunk's reads are done
#pragma unroll
      for (int k = 0; k < S::NPC; ++k) {
        if (!piece_ok(k)) continue;
        const int p = tid + k * NT, row = p / S::PPR, c0 = 8 * (p % S::PPR);
        const uint32_t* wd = reinterpret_cast<const uint32_t*>(xr[k]);
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          float f0, f1;
          if constexpr (VB) {
            f0 = __uint_as_float(wd[i / 2] << 16);
            f1 = __uint_as_float(wd[i / 2] & 0xFFFF0000u);
          } else {
            f0 = __uint_as_float(wd[i]);
            f1 = __uint_as_float(wd[i + 1]);
          }
          const double x0 = vr[k] ? static_cast<double>(f0) - s_mu[c0 + i] : 0.0;
          const double x1 = vr[k] ? static_cast<double>(f1) - s_mu[c0 + i + 1] : 0.0;
          *reinterpret_cast<double2*>(&xs[row][c0 + i]) = double2{x0, x1};
        }
        if (p % S::PPR == 0) s_w[row] = vr[k] ? wr[k] : 0.0;
      }
      __syncthreads();
      if (base + kCovChunk < r1) {
        fetch();
        tokens(base + 2 * kCovChunk);
      }
      const int nks = (min(kCovChunk, r1 - base) + 3) / 4;
      for (int ks = 0; ks < nks; ++ks) {
        const int tok = 4 * ks + (lane >> 4);
        const double w = s_w[tok];
        const double* row = xs[tok];
        double xa[TPW], xb[TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          xa[u] = row[ci[u]];
          xb[u] = row[cj[u]];
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u) acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(w * xa[u], xb[u], acc[u], 0, 0, 0);
      }
    }
    double* out = a.part_cov + ((static_cast<size_t>(s) * a.hkv + h) * kCalibModalities + m) * D * D;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = 4 * r + (lane >> 4), jj = lane & 15;
        if (bi[u] != bj[u] || ii <= jj) out[static_cast<size_t>(16 * bi[u] + ii) * D + 16 * bj[u] + jj] = acc[u][r];
      }
    }
    off += cnt;
  }
}

// Covariances: the splits' partial sums in split order, divided by W.
// Thread (i, j), i <= j, reads the stored entry (its row, so the reads of a
// wavefront are contiguous) and writes entries (i, j) and (j, i).
template <int D>
__global__ __launch_bounds__(256) void calib_cov_merge_kernel(CovArgs a) {
  const size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t per = static_cast<size_t>(D) * D;
  if (e >= static_cast<size_t>(a.hkv) * kCalibModalities * per) return;
  const size_t hm = e / per;
  const int i = static_cast<int>(e % per) / D, j = static_cast<int>(e % per) % D;
  if (i > j) return;
  const double* p = a.part_cov + e;
  const size_t stride = static_cast<size_t>(a.hkv) * kCalibModalities * per;
  constexpr int U = 8;   // splits whose partial sums are loaded together
  double x = 0.0;
  for (int s0 = 0; s0 < a.splits; s0 += U) {
    double v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = s0 + u < a.splits ? p[(s0 + u) * stride] : 0.0;
#pragma unroll
    for (int u = 0; u < U; ++u) x += v[u];   // splits in increasing order
  }
  const double w = a.wsum[hm];
  const double c = w > 0.0 ? x / w : 0.0;
  a.cov[e] = c;
  a.cov[hm * per + static_cast<size_t>(j) * D + i] = c;
}

// -------------------------------------------------------------- eigenbasis

// Cyclic Jacobi on one symmetric matrix per workgroup (Golub & Van Loan,
// "Matrix Computations", Sec. 8.5: the symmetric Schur 2 x 2 rotation and
// the parallel ordering).  Each sweep visits every pair (p, q) once through
// D - 1 rounds of D / 2 disjoint pairs (round-robin ordering: player 0
// fixed, the others rotated).
//
// Phase 1 rotates A alone, in LDS, keeping its upper triangle only: a
// round forms its rotations from the current matrix, then applies J^T A J
// one 2 x 2 block (ki, kj), ki <= kj, at a time.  A pair
// whose off-diagonal entry is negligible (against its diagonal, or below
// the rounding noise of the whole matrix) is set to zero without a rotation;
// the sweeps end when one rotates nothing (at most kJacobiSweeps).  Each
// round's rotations (c, s) go to a log in the workspace; a round that
// rotates no pair skips the update.
// Phase 2 replays the log on V = I: V <- V J round by round with phase 1's
// own (c, s).  The columns of V^T are independent under the rotations, so
// the replay runs as many workgroups per matrix, each on a block of
// kReplayCols columns of V^T (one lane per pair).  A last pass orders the
// eigenvectors by eigenvalue and fixes their signs.
template <int D>
constexpr int jacobi_threads() { return D == 128 ? 1024 : 256; }
constexpr int kReplayCols = 8;     // columns of V^T per replay workgroup
constexpr int kReplayChunk = 16;   // rounds of the log staged in LDS at a time

// The eigenbasis workspace: the rotation log, then per matrix its round
// count, its eigenvalues (unsorted) and V^T.
struct EigLayout {
  size_t log, rounds, lam, vt, total;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

EigLayout eig_layout(int count, int d) {
  EigLayout L;
  size_t o = 0;
  L.log = o;
  o += align256(static_cast<size_t>(count) * kJacobiSweeps * (d - 1) * (d / 2) * 2 * sizeof(double));
  L.rounds = o;
  o += align256(static_cast<size_t>(count) * sizeof(int));
  L.lam = o;
  o += align256(static_cast<size_t>(count) * d * sizeof(double));
  L.vt = o;
  o += static_cast<size_t>(count) * d * d * sizeof(double);
  L.total = o;
  return L;
}

// Pair k of round r of the round-robin ordering, as (p, q) with p < q.
template <int D>
__device__ __forceinline__ void jacobi_pair(int r, int k, int& p, int& q) {
  const int x = k == 0 ? 0 : 1 + (k - 1 + r) % (D - 1);
  const int y = 1 + (D - 2 - k + r) % (D - 1);
  p = min(x, y);
  q = max(x, y);
}

// Block task e of the NP (NP + 1) / 2 pairs (ki, kj) with ki <= kj: rows
// r and NP - 1 - r of that triangle (NP - r and r + 1 entries) share row r
// of an (NP / 2) x (NP + 1) rectangle, e = (NP + 1) r + c.
template <int NP>
__device__ __forceinline__ void block_task(int e, int& ki, int& kj) {
  const int r = e / (NP + 1), c = e % (NP + 1);
  if (c < NP - r) {
    ki = r;
    kj = r + c;
  } else {
    ki = NP - 1 - r;
    kj = ki + c - (NP - r);
  }
}

// Phase 1 keeps entry (x, y) of the symmetric A at (min, max) only.
template <int LD>
__device__ __forceinline__ int upper(int x, int y) { return min(x, y) * LD + max(x, y); }

// Barrier for LDS traffic only: the log's global stores stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D>
__global__ __launch_bounds__(jacobi_threads<D>()) void calib_jacobi_kernel(const double* cov, double2* logs,
                                                                           int* rounds_out, double* lam_out) {
  constexpr int NP = D / 2;
  constexpr int LD = D + 1;
  constexpr int NT = jacobi_threads<D>();
  // 2 x 2 block tasks (ki, kj), ki <= kj: NP (NP + 1) / 2 of them, numbered
  // densely (block_task) and dealt round robin, NAT per thread at most
  constexpr int NTASK = NP * (NP + 1) / 2;
  constexpr int NAT = (NTASK + NT - 1) / NT;
  static_assert(NT >= D, "one thread per eigenvalue at the end");
  constexpr double kNegligible = 0x1p-53;   // |a_pq| <= 2^-53 sqrt(|a_pp a_qq|): already diagonal to rounding
  __shared__ double A[D * LD];
  __shared__ double2 s_cs[NP];             // (c, s) of each pair
  __shared__ double s_t[NP];
  __shared__ int s_pq[NP];                 // p | q << 16 of each pair
  __shared__ int s_changed;
  __shared__ int s_rot[2];                 // the round rotates some pair
  __shared__ double s_sq[NT];
  const int mat = blockIdx.x, tid = threadIdx.x;
  const double* C = cov + static_cast<size_t>(mat) * D * D;
  double2* log = logs + static_cast<size_t>(mat) * kJacobiSweeps * (D - 1) * NP;
  double sq = 0.0;
  for (int e = tid; e < D * D; e += NT) {
    const int i = e / D, j = e % D;
    const double x = i <= j ? C[static_cast<size_t>(i) * D + j] : C[static_cast<size_t>(j) * D + i];
    A[i * LD + j] = x;
    sq = __builtin_fma(x, x, sq);
  }
  // |A|_F^2 by a fixed tree: a rotation leaves rounding noise of order
  // 2^-53 |A|_F off the diagonal, so entries below 2^-51 |A|_F are left alone
  s_sq[tid] = sq;
  __syncthreads();
  for (int st = NT / 2; st > 0; st >>= 1) {
    if (tid < st) s_sq[tid] += s_sq[tid + st];
    __syncthreads();
  }
  const double floor_abs = 0x1p-51 * sqrt(s_sq[0]);

  // ---- phase 1: A <- J^T A J until a sweep rotates nothing
  int sweeps = 0;
  int rc = 0;   // rounds so far (the per-round flag alternates between two slots)
  for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
    __syncthreads();
    if (tid == 0) s_changed = 0;
    __syncthreads();
    for (int r = 0; r < D - 1; ++r) {
      if (tid < NP) {
        const int k = tid;
        int p, q;
        jacobi_pair<D>(r, k, p, q);
        const double app = A[p * LD + p], aqq = A[q * LD + q], apq = A[p * LD + q];
        double t = 0.0;
        if (fabs(apq) > kNegligible * sqrt(fabs(app) * fabs(aqq)) && fabs(apq) > floor_abs) {
          const double theta = (aqq - app) / (2.0 * apq);
          if (fabs(theta) > 1e100) {
            t = 0.5 / theta;
          } else {
            t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(1.0 + theta * theta));
          }
          s_changed = 1;
        }
        const double c = 1.0 / sqrt(1.0 + t * t);
        s_pq[k] = p | (q << 16);
        s_cs[k] = double2{c, t * c};
        s_t[k] = t;
        log[(static_cast<size_t>(sweep) * (D - 1) + r) * NP + k] = double2{c, t * c};
        // a pair left alone gets the exact zero its own task would write
        // (the other tasks never touch entry (p, q))
        if (t == 0.0) A[p * LD + q] = 0.0;
        const bool any = __any(t != 0.0);   // (the pairs are all in wavefront 0)
        if (k == 0) s_rot[rc & 1] = any;
      }
      lds_barrier();
      // a round that rotates nothing leaves every other entry as it is
      if (!s_rot[rc++ & 1]) continue;
      // this round's tasks touch disjoint entries: all loads (their
      // addresses kept), then all stores
      double blk[NAT][4];
      int adr[NAT][4];
#pragma unroll
      for (int u = 0; u < NAT; ++u) {
        const int e = tid + u * NT;
        if (e < NTASK) {
          int ki, kj;
          block_task<NP>(e, ki, kj);
          const int pqi = s_pq[ki], pqj = s_pq[kj];
          const int pi = pqi & 0xFFFF, qi = pqi >> 16, pj = pqj & 0xFFFF, qj = pqj >> 16;
          adr[u][0] = upper<LD>(pi, pj);
          adr[u][1] = upper<LD>(pi, qj);
          adr[u][2] = upper<LD>(qi, pj);
          adr[u][3] = upper<LD>(qi, qj);
#pragma unroll
          for (int x = 0; x < 4; ++x) blk[u][x] = A[adr[u][x]];
        }
      }
#pragma unroll
      for (int u = 0; u < NAT; ++u) {
        const int e = tid + u * NT;
        if (e >= NTASK) continue;
        int ki, kj;
        block_task<NP>(e, ki, kj);
        const double a_pp = blk[u][0], a_pq = blk[u][1], a_qp = blk[u][2], a_qq = blk[u][3];
        if (ki == kj) {
          // the rotated pair itself (entries (p, p), (p, q), (q, q)): exact
          // zero off the diagonal
          const double t = s_t[ki];
          A[adr[u][0]] = a_pp - t * a_pq;
          A[adr[u][3]] = a_qq + t * a_pq;
          A[adr[u][1]] = 0.0;
          continue;
        }
        const double2 csi = s_cs[ki], csj = s_cs[kj];
        const double ci = csi.x, si = csi.y, cj = csj.x, sj = csj.y;
        // rows (J_i^T from the left), then columns (J_j from the right)
        const double r_pp = ci * a_pp - si * a_qp, r_pq = ci * a_pq - si * a_qq;
        const double r_qp = si * a_pp + ci * a_qp, r_qq = si * a_pq + ci * a_qq;
        const double n_pp = cj * r_pp - sj * r_pq, n_pq = sj * r_pp + cj * r_pq;
        const double n_qp = cj * r_qp - sj * r_qq, n_qq = sj * r_qp + cj * r_qq;
        A[adr[u][0]] = n_pp;
        A[adr[u][1]] = n_pq;
        A[adr[u][2]] = n_qp;
        A[adr[u][3]] = n_qq;
      }
      lds_barrier();
    }
    sweeps = sweep + 1;
    if (!s_changed) break;
  }
  if (tid < D) lam_out[static_cast<size_t>(mat) * D + tid] = A[tid * LD + tid];
  if (tid == 0) rounds_out[mat] = sweeps * (D - 1);
}

// Phase 2: V^T <- J^T V^T from the identity, on columns [cb W, (cb + 1) W)
// of V^T (W = kReplayCols) per workgroup.  The columns do not interact, so
// each of the replay_waves wavefronts takes W / replay_waves of them alone:
// lane k applies pair k of every round (two lanes per pair at d = 64, each
// on half the wavefront's columns), with no barrier between rounds; a pair
// that was left alone (s = 0, c = 1) leaves its rows as they are.  The log
// is staged kReplayChunk rounds at a time through LDS by the whole
// workgroup, the next chunk's loads in flight while the current one is
// applied.
template <int D>
constexpr int replay_waves() { return D == 128 ? 8 : 4; }   // one column per lane

template <int D>
__global__ __launch_bounds__(64 * replay_waves<D>()) void calib_jacobi_replay_kernel(const double2* logs,
                                                                                     const int* rounds_in, double* vt) {
  constexpr int NP = D / 2;
  constexpr int W = kReplayCols;
  constexpr int NT = 64 * replay_waves<D>();
  constexpr int CB = D / W;              // column blocks per matrix
  constexpr int WW = W / replay_waves<D>();   // columns per wavefront
  constexpr int LPP = 64 / NP;           // lanes per pair
  constexpr int CPL = WW / LPP;          // columns per lane
  constexpr int LDB = W + 1;             // row stride in doubles
  constexpr int CH = kReplayChunk;
  constexpr int PRE = CH * NP / NT;      // log entries per thread per chunk
  static_assert(LPP * NP == 64 && CPL * LPP == WW && WW * replay_waves<D>() == W && PRE * NT == CH * NP,
                "replay shape");
  __shared__ double V[D * LDB];
  __shared__ double2 s_cs[2][CH * NP];
  const int mat = blockIdx.x / CB, cb = blockIdx.x % CB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = lane % NP, c0 = wave * WW + (lane / NP) * CPL;
  const double2* log = logs + static_cast<size_t>(mat) * kJacobiSweeps * (D - 1) * NP;
  const int rounds = rounds_in[mat];
  for (int e = tid; e < D * W; e += NT) {
    const int i = e / W, j = e % W;
    V[i * LDB + j] = (i == cb * W + j) ? 1.0 : 0.0;
  }
  const int nch = (rounds + CH - 1) / CH;
  double2 pre[PRE];
  auto fetch = [&](int ch) {
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
      const int idx = u * NT + tid;                    // (round in chunk) * NP + pair
      const bool in = ch * CH + idx / NP < rounds;
      pre[u] = in ? log[static_cast<size_t>(ch) * CH * NP + idx] : double2{1.0, 0.0};
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PRE; ++u) s_cs[buf][u * NT + tid] = pre[u];
  };
  if (nch > 0) {
    fetch(0);
    stash(0);
  }
  if (nch > 1) fetch(1);
  lds_barrier();
  // pair k of round r is (x, y) = (k == 0 ? 0 : 1 + (k - 1 + r) mod (D - 1),
  // 1 + (D - 2 - k + r) mod (D - 1)) (jacobi_pair), kept as two counters
  int xm = (k + D - 2) % (D - 1), ym = (D - 2 - k) % (D - 1);
  for (int ch = 0; ch < nch; ++ch) {
    const int buf = ch & 1;
    const int nr = min(CH, rounds - ch * CH);
    double2 cs = s_cs[buf][k];
    for (int i = 0; i < nr; ++i) {
      // the next round's (c, s), read ahead (the last one re-reads itself)
      const double2 cs_next = s_cs[buf][min(i + 1, CH - 1) * NP + k];
      const int x = k == 0 ? 0 : 1 + xm, y = 1 + ym;
      const int p = min(x, y), q = max(x, y);
      if (cs.y != 0.0) {
        double wx[CPL], wy[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          wx[j] = V[p * LDB + c0 + j];
          wy[j] = V[q * LDB + c0 + j];
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          V[p * LDB + c0 + j] = cs.x * wx[j] - cs.y * wy[j];
          V[q * LDB + c0 + j] = cs.y * wx[j] + cs.x * wy[j];
        }
      }
      xm = xm == D - 2 ? 0 : xm + 1;
      ym = ym == D - 2 ? 0 : ym + 1;
      // the round's rows are written before the wavefront's next reads
      // (only this wavefront touches its columns)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      cs = cs_next;
    }
    // chunk ch + 1 into the buffer of chunk ch - 1, which every wavefront
    // finished before the previous barrier
    if (ch + 1 < nch) stash(buf ^ 1);
    if (ch + 2 < nch) fetch(ch + 2);
    lds_barrier();
  }
  double* out = vt + static_cast<size_t>(mat) * D * D + cb * W;
  for (int e = tid; e < D * W; e += NT) {
    const int i = e / W, j = e % W;
    out[static_cast<size_t>(i) * D + j] = V[i * LDB + j];
  }
}

// The eigenvectors (rows of V^T) in decreasing eigenvalue order (ties by
// index), each signed so that its largest-magnitude component (the first
// of equal ones) is positive; rot[i][rank] = component i, as fp32.
template <int D>
__global__ __launch_bounds__(256) void calib_jacobi_finalize_kernel(const double* vt, const double* lam_in,
                                                                    float* rot, double* evals) {
  constexpr int LD = D + 1;
  __shared__ double A[D * LD];
  __shared__ double s_lam[D];
  const int mat = blockIdx.x, tid = threadIdx.x;
  const double* src = vt + static_cast<size_t>(mat) * D * D;
  for (int e = tid; e < D * D; e += 256) A[(e / D) * LD + e % D] = src[e];
  if (tid < D) s_lam[tid] = lam_in[static_cast<size_t>(mat) * D + tid];
  __syncthreads();
  if (tid < D) {
    const double lam = s_lam[tid];
    int rank = 0;
    for (int k = 0; k < D; ++k) {
      const double lk = s_lam[k];
      rank += (lk > lam || (lk == lam && k < tid)) ? 1 : 0;
    }
    const double* wr = &A[tid * LD];
    int best = 0;
    double bv = fabs(wr[0]);
    for (int i = 1; i < D; ++i) {
      const double x = fabs(wr[i]);
      if (x > bv) {
        bv = x;
        best = i;
      }
    }
    const double sg = wr[best] < 0.0 ? -1.0 : 1.0;
    float* R = rot + static_cast<size_t>(mat) * D * D;
    for (int i = 0; i < D; ++i) R[static_cast<size_t>(i) * D + rank] = static_cast<float>(sg * wr[i]);
    evals[static_cast<size_t>(mat) * D + rank] = lam;
  }
}

// ------------------------------------------------------------------- host

struct CalibPlan {
  int rows, nblk;          // contribution
  int splits;               // covariance: token ranges per modality
  int mean_splits, mean_split_tokens;  // weighted means: 1024 tokens per split
  size_t contrib_bytes, cov_bytes, eig_bytes;
};

kvq_status check_shape(const kvq_calib_shape* s) {
  if (!s) return KVQ_ERR_INVALID;
  if (s->head_dim != 64 && s->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  if (s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->n_q_heads % s->n_kv_heads != 0) return KVQ_ERR_INVALID;
  if (s->n_tokens < 0 || s->n_queries <= 0) return KVQ_ERR_INVALID;
  if (static_cast<int64_t>(s->n_queries) * s->n_q_heads > (1 << 24)) return KVQ_ERR_INVALID;
  return KVQ_OK;
}

bool dtype_ok(int32_t t) { return t == KVQ_F32 || t == KVQ_BF16; }

CalibPlan plan_calib(const kvq_calib_shape* s) {
  CalibPlan p;
  const int d = s->head_dim, hkv = s->n_kv_heads, n = s->n_tokens;
  p.rows = s->n_queries * (s->n_q_heads / hkv);
  p.nblk = std::max(1, (n + kTokBlock - 1) / kTokBlock);
  p.contrib_bytes = align256(static_cast<size_t>(hkv) * p.nblk * p.rows * 2 * sizeof(double)) +
                    align256(static_cast<size_t>(hkv) * p.rows * 2 * sizeof(double));
  // covariance: each modality's tokens in `splits` ranges, one workgroup per
  // (range, KV head) for all three modalities: at most 256 workgroups (one
  // per CU), about 256 tokens per workgroup at least
  int splits = std::max(1, 256 / hkv);
  splits = std::min(splits, std::max(1, (n + 255) / 256));
  p.splits = splits;
  p.mean_split_tokens = 1024;
  p.mean_splits = std::max(1, (n + 1023) / 1024);
  p.cov_bytes = align256(static_cast<size_t>(p.mean_splits) * hkv * kCalibModalities * (d + 1) * sizeof(double)) +
                align256(static_cast<size_t>(hkv) * kCalibModalities * d * sizeof(double)) +
                align256((static_cast<size_t>(n) + 4 + 3 * (static_cast<size_t>(n) / 1024 + 1)) * sizeof(int32_t)) +
                align256(static_cast<size_t>(splits) * hkv * kCalibModalities * d * d * sizeof(double));
  p.eig_bytes = eig_layout(3 * hkv, d).total;
  return p;
}

template <int D>
void launch_eigenbasis(int count, const double* cov, double2* log, int* rounds, double* lam, double* vt, float* rot,
                       double* evals, hipStream_t st) {
  hipLaunchKernelGGL(calib_jacobi_kernel<D>, dim3(count), dim3(jacobi_threads<D>()), 0, st, cov, log, rounds, lam);
  hipLaunchKernelGGL(calib_jacobi_replay_kernel<D>, dim3(count * (D / kReplayCols)), dim3(64 * replay_waves<D>()), 0, st,
                     log, rounds, vt);
  hipLaunchKernelGGL(calib_jacobi_finalize_kernel<D>, dim3(count), dim3(256), 0, st, vt, lam, rot, evals);
}

template <int D>
void launch_contribution(const ContribArgs& a, bool kb, bool qb, hipStream_t st) {
  const dim3 gb(a.nblk, a.hkv), gm(a.rows, a.hkv);
#define KVQ_CONTRIB(KB, QB)                                                                    \
  do {                                                                                         \
    hipLaunchKernelGGL((calib_block_stats_kernel<D, KB, QB>), gb, dim3(kTokBlock), 0, st, a); \
    hipLaunchKernelGGL(calib_stats_merge_kernel, gm, dim3(64), 0, st, a);                      \
    hipLaunchKernelGGL((calib_weights_kernel<D, KB, QB>), gb, dim3(kTokBlock), 0, st, a);     \
  } while (0)
  if (kb && qb) KVQ_CONTRIB(true, true);
  else if (kb) KVQ_CONTRIB(true, false);
  else if (qb) KVQ_CONTRIB(false, true);
  else KVQ_CONTRIB(false, false);
#undef KVQ_CONTRIB
}

template <int D>
void launch_covariance(const CovArgs& a, bool vb, hipStream_t st) {
  const dim3 gpart(a.mean_splits, a.hkv);
  const dim3 gmm((a.hkv * kCalibModalities * D + 255) / 256);
  const dim3 gcov(a.splits, a.hkv);
  constexpr int cov_threads = CovShape<D>::NT;
  const size_t ncov = static_cast<size_t>(a.hkv) * kCalibModalities * D * D;
  const dim3 gcm(static_cast<unsigned>((ncov + 255) / 256));
  const int nblk = std::max(1, (a.n + kGroupThreads - 1) / kGroupThreads);
  hipLaunchKernelGGL(calib_group_count_kernel, dim3(nblk), dim3(kGroupThreads), 0, st, a);
  hipLaunchKernelGGL(calib_group_scan_kernel, dim3(1), dim3(kGroupThreads), 0, st, a, nblk);
  hipLaunchKernelGGL(calib_group_scatter_kernel, dim3(nblk), dim3(kGroupThreads), 0, st, a);
  if (vb) {
    hipLaunchKernelGGL((calib_mean_part_kernel<D, true>), gpart, dim3(256), 0, st, a);
    hipLaunchKernelGGL((calib_mean_merge_kernel<D>), gmm, dim3(256), 0, st, a);
    hipLaunchKernelGGL((calib_cov_part_kernel<D, true>), gcov, dim3(cov_threads), 0, st, a);
  } else {
    hipLaunchKernelGGL((calib_mean_part_kernel<D, false>), gpart, dim3(256), 0, st, a);
    hipLaunchKernelGGL((calib_mean_merge_kernel<D>), gmm, dim3(256), 0, st, a);
    hipLaunchKernelGGL((calib_cov_part_kernel<D, false>), gcov, dim3(cov_threads), 0, st, a);
  }
  hipLaunchKernelGGL((calib_cov_merge_kernel<D>), gcm, dim3(256), 0, st, a);
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" {

size_t kvq_calib_workspace_bytes(const kvq_calib_shape* shape) {
  if (check_shape(shape) != KVQ_OK) return 0;
  const CalibPlan p = plan_calib(shape);
  return std::max(p.contrib_bytes, std::max(p.cov_bytes, p.eig_bytes));
}

size_t kvq_calib_eigenbasis_workspace_bytes(int32_t count, int32_t head_dim) {
  if (count < 0 || (head_dim != 64 && head_dim != 128)) return 0;
  // the rotation log, (c, s) per (sweep, round, pair), and V^T per matrix
  return eig_layout(count, head_dim).total;
}

kvq_status kvq_calib_contribution(const kvq_calib_shape* shape, const void* k, int32_t k_dtype, const void* q,
                                  int32_t q_dtype, double scale, double* weights, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  kvq_status st = check_shape(shape);
  if (st != KVQ_OK) return st;
  if (!dtype_ok(k_dtype) || !dtype_ok(q_dtype)) return KVQ_ERR_UNSUPPORTED;
  if (!(scale > 0.0) || !isfinite(scale)) return KVQ_ERR_INVALID;
  if (shape->n_tokens == 0) return KVQ_OK;
  if (!k || !q || !weights) return KVQ_ERR_INVALID;
  const CalibPlan p = plan_calib(shape);
  if (!workspace || workspace_bytes < p.contrib_bytes) return KVQ_ERR_WORKSPACE;
  ContribArgs a;
  a.k = k;
  a.q = q;
  a.weights = weights;
  a.part = static_cast<double*>(workspace);
  a.stats = reinterpret_cast<double*>(static_cast<char*>(workspace) +
                                      align256(static_cast<size_t>(shape->n_kv_heads) * p.nblk * p.rows * 2 *
                                               sizeof(double)));
  a.n = shape->n_tokens;
  a.hkv = shape->n_kv_heads;
  a.hq = shape->n_q_heads;
  a.group = shape->n_q_heads / shape->n_kv_heads;
  a.rows = p.rows;
  a.nblk = p.nblk;
  a.scale = scale;
  (void)hipGetLastError();
  if (shape->head_dim == 128) launch_contribution<128>(a, k_dtype == KVQ_BF16, q_dtype == KVQ_BF16, stream);
  else launch_contribution<64>(a, k_dtype == KVQ_BF16, q_dtype == KVQ_BF16, stream);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

kvq_status kvq_calib_covariance(const kvq_calib_shape* shape, const void* v, int32_t v_dtype,
                                const uint8_t* modality, const double* weights, double* cov, double* weight_sum,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  kvq_status st = check_shape(shape);
  if (st != KVQ_OK) return st;
  if (!dtype_ok(v_dtype)) return KVQ_ERR_UNSUPPORTED;
  if (!cov || !weight_sum) return KVQ_ERR_INVALID;
  if (shape->n_tokens > 0 && (!v || !modality || !weights)) return KVQ_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(v) % 16 != 0) return KVQ_ERR_INVALID;   // read in 16-byte pieces
  const CalibPlan p = plan_calib(shape);
  if (!workspace || workspace_bytes < p.cov_bytes) return KVQ_ERR_WORKSPACE;
  const int d = shape->head_dim, hkv = shape->n_kv_heads;
  CovArgs a;
  a.v = v;
  a.modality = modality;
  a.weights = weights;
  a.cov = cov;
  a.wsum = weight_sum;
  char* w = static_cast<char*>(workspace);
  a.part_mean = reinterpret_cast<double*>(w);
  w += align256(static_cast<size_t>(p.mean_splits) * hkv * kCalibModalities * (d + 1) * sizeof(double));
  a.mean = reinterpret_cast<double*>(w);
  w += align256(static_cast<size_t>(hkv) * kCalibModalities * d * sizeof(double));
  a.counts = reinterpret_cast<int32_t*>(w);
  a.order = a.counts + 4;
  a.group_blk = a.order + shape->n_tokens;
  w += align256((static_cast<size_t>(shape->n_tokens) + 4 + 3 * (static_cast<size_t>(shape->n_tokens) / 1024 + 1)) *
                sizeof(int32_t));
  a.part_cov = reinterpret_cast<double*>(w);
  a.n = shape->n_tokens;
  a.hkv = hkv;
  a.splits = p.splits;
  a.mean_splits = p.mean_splits;
  a.mean_split_tokens = p.mean_split_tokens;
  (void)hipGetLastError();
  if (d == 128) launch_covariance<128>(a, v_dtype == KVQ_BF16, stream);
  else launch_covariance<64>(a, v_dtype == KVQ_BF16, stream);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

kvq_status kvq_calib_eigenbasis(int32_t count, int32_t head_dim, const double* cov, float* rot, double* eigenvalues,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (count < 0) return KVQ_ERR_INVALID;
  if (head_dim != 64 && head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  if (count == 0) return KVQ_OK;
  if (!cov || !rot || !eigenvalues) return KVQ_ERR_INVALID;
  if (!workspace || workspace_bytes < kvq_calib_eigenbasis_workspace_bytes(count, head_dim)) return KVQ_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return KVQ_ERR_INVALID;   // (c, s) pairs: 16-byte loads
  (void)hipGetLastError();
  const EigLayout L = eig_layout(count, head_dim);
  char* w = static_cast<char*>(workspace);
  double2* log = reinterpret_cast<double2*>(w + L.log);
  int* rounds = reinterpret_cast<int*>(w + L.rounds);
  double* lam = reinterpret_cast<double*>(w + L.lam);
  double* vt = reinterpret_cast<double*>(w + L.vt);
  if (head_dim == 128) launch_eigenbasis<128>(count, cov, log, rounds, lam, vt, rot, eigenvalues, stream);
  else launch_eigenbasis<64>(count, cov, log, rounds, lam, vt, rot, eigenvalues, stream);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

}  // extern "C"
