// Value-basis calibration (kvq_calib.h): attention-contribution weights,
// weighted per-modality covariances and their eigenbases, all in fp64.
//
// OmniKVQuant page, Sec. 2 Method, second "OmniKVQuant" bullet: value
// directions are weighted by their contribution to attention outputs, a
// covariance is formed per modality, and its eigenbasis is the modality's
// rotation.  Calibration runs once, off the decode path; every sum below has
// a fixed order, so results do not depend on timing.
//
// fp64 matrix and vector throughput are the same on this chip, so the
// contractions (scores, covariance) run on the vector ALUs with fp64 FMAs.
#include <math.h>

#include <algorithm>

#include "kvq_calib.h"
#include "kvq_common.h"

namespace kvq {
namespace {

constexpr int kCalibModalities = 3;
constexpr int kRowChunk = 16;        // query rows whose scores a thread forms together
constexpr int kTokBlock = 256;       // tokens per workgroup in the score kernels
constexpr int kTile = 32;            // covariance tile (kTile x kTile entries)
constexpr int kTileTokens = 64;      // tokens staged in LDS per covariance step
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
// exp(score - max) over the block's tokens.  Thread = token.
template <int D, bool KB, bool QB>
__global__ __launch_bounds__(kTokBlock) void calib_block_stats_kernel(ContribArgs a) {
  __shared__ double sq[kRowChunk][D];
  __shared__ double red_m[kTokBlock / 64][kRowChunk], red_l[kTokBlock / 64][kRowChunk];
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
#pragma unroll
    for (int r = 0; r < kRowChunk; ++r) {
      double m = ok ? a.scale * dot[r] : -INFINITY;
      double l = ok ? 1.0 : 0.0;
      // butterfly over the wavefront (fixed pattern; lane 0 keeps the result)
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const double m2 = __shfl_xor(m, off, 64);
        const double l2 = __shfl_xor(l, off, 64);
        merge_ms(m, l, m2, l2);
      }
      if (lane == 0) {
        red_m[wave][r] = m;
        red_l[wave][r] = l;
      }
    }
    __syncthreads();
    if (threadIdx.x < kRowChunk && r0 + static_cast<int>(threadIdx.x) < a.rows) {
      const int r = threadIdx.x;
      double m = red_m[0][r], l = red_l[0][r];
      for (int w = 1; w < kTokBlock / 64; ++w) merge_ms(m, l, red_m[w][r], red_l[w][r]);
      double* out = a.part + ((static_cast<size_t>(h) * a.nblk + blk) * a.rows + r0 + r) * 2;
      out[0] = m;
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
  double* part_cov;         // [S][hkv][3][D][D]
  int32_t n, hkv, splits, split_tokens;   // covariance tiles' token splits
  int32_t mean_splits, mean_split_tokens;  // weighted-mean pass's token splits
};

// Partial weighted sums of one (split, KV head): thread = (phase, channel);
// phases stride the split's tokens and are combined in phase order.
template <int D, bool VB>
__global__ __launch_bounds__(256) void calib_mean_part_kernel(CovArgs a) {
  constexpr int P = 256 / D;
  __shared__ double s_wv[P][kCalibModalities][D];
  __shared__ double s_w[P][kCalibModalities];
  constexpr int U = 4;   // tokens whose loads are issued together
  const int s = blockIdx.x, h = blockIdx.y;
  const int ph = threadIdx.x / D, c = threadIdx.x % D;
  const int t0 = s * a.mean_split_tokens, t1 = min(a.n, t0 + a.mean_split_tokens);
  double wv[kCalibModalities] = {0.0, 0.0, 0.0}, ws[kCalibModalities] = {0.0, 0.0, 0.0};
  for (int tb = t0 + ph; tb < t1; tb += U * P) {
    int md[U];
    double wt[U], x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + u * P;
      const bool in = t < t1;
      md[u] = in ? a.modality[t] : 3;
      wt[u] = in ? a.weights[static_cast<size_t>(h) * a.n + t] : 0.0;
      x[u] = in ? load_input<VB>(a.v, (static_cast<size_t>(t) * a.hkv + h) * D + c) : 0.0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {   // tokens in increasing order
      if (md[u] == 0) { wv[0] = __builtin_fma(wt[u], x[u], wv[0]); ws[0] += wt[u]; }
      else if (md[u] == 1) { wv[1] = __builtin_fma(wt[u], x[u], wv[1]); ws[1] += wt[u]; }
      else if (md[u] == 2) { wv[2] = __builtin_fma(wt[u], x[u], wv[2]); ws[2] += wt[u]; }
    }
  }
#pragma unroll
  for (int m = 0; m < kCalibModalities; ++m) s_wv[ph][m][c] = wv[m];
  if (c == 0)
#pragma unroll
    for (int m = 0; m < kCalibModalities; ++m) s_w[ph][m] = ws[m];
  __syncthreads();
  if (ph == 0) {
    double* out = a.part_mean + (static_cast<size_t>(s) * a.hkv + h) * kCalibModalities * (D + 1);
#pragma unroll
    for (int m = 0; m < kCalibModalities; ++m) {
      double x = s_wv[0][m][c];
      for (int p = 1; p < P; ++p) x += s_wv[p][m][c];
      out[m * (D + 1) + c] = x;
      if (c == 0) {
        double w = s_w[0][m];
        for (int p = 1; p < P; ++p) w += s_w[p][m];
        out[m * (D + 1) + D] = w;
      }
    }
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

// Partial covariance tile of one (split, KV head): entries (i, j) of tile
// (bi, bj), bi <= bj, for the three modalities.  Each term is w * (x_i x_j)
// with the product of the centred values formed first, so entry (j, i) of a
// diagonal tile, formed by another thread, is the same number; off-diagonal
// tiles are written to both halves.  Thread = 2 x 2 entries.
template <int D, bool VB>
__global__ __launch_bounds__(256) void calib_cov_part_kernel(CovArgs a) {
  constexpr int NB = D / kTile;
  __shared__ double xi[kTileTokens][kTile + 1];
  __shared__ double xj[kTileTokens][kTile + 1];
  __shared__ double s_w[kTileTokens];
  __shared__ int s_md[kTileTokens];
  __shared__ double s_mean[kCalibModalities][2][kTile];
  // tile index -> (bi, bj) with bi <= bj
  int tile = blockIdx.x, bi = 0;
  while (tile >= NB - bi) {
    tile -= NB - bi;
    ++bi;
  }
  const int bj = bi + tile;
  const int s = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x;
  const int ti = tid / 16, tj = tid % 16;
  const int t0 = s * a.split_tokens, t1 = min(a.n, t0 + a.split_tokens);
  if (tid < kCalibModalities * 2 * kTile) {
    const int m = tid / (2 * kTile), side = (tid / kTile) & 1, cc = tid % kTile;
    const int ch = (side ? bj : bi) * kTile + cc;
    s_mean[m][side][cc] = a.mean[(static_cast<size_t>(h) * kCalibModalities + m) * D + ch];
  }
  double acc0[4] = {0.0, 0.0, 0.0, 0.0}, acc1[4] = {0.0, 0.0, 0.0, 0.0}, acc2[4] = {0.0, 0.0, 0.0, 0.0};
  for (int base = t0; base < t1; base += kTileTokens) {
    __syncthreads();
    if (tid < kTileTokens) {
      const int t = base + tid;
      int m = 3;
      double w = 0.0;
      if (t < t1) {
        m = a.modality[t];
        w = a.weights[static_cast<size_t>(h) * a.n + t];
      }
      s_md[tid] = m < kCalibModalities ? m : 3;
      s_w[tid] = w;
    }
    __syncthreads();
    for (int e = tid; e < kTileTokens * kTile; e += 256) {
      const int tt = e / kTile, cc = e % kTile;
      const int t = base + tt;
      const int m = s_md[tt];
      double vi = 0.0, vj = 0.0;
      if (m < kCalibModalities) {
        const size_t row = (static_cast<size_t>(t) * a.hkv + h) * D;
        vi = load_input<VB>(a.v, row + bi * kTile + cc) - s_mean[m][0][cc];
        vj = load_input<VB>(a.v, row + bj * kTile + cc) - s_mean[m][1][cc];
      }
      xi[tt][cc] = vi;
      xj[tt][cc] = vj;
    }
    __syncthreads();
    const int nt = min(kTileTokens, t1 - base);
    for (int tt = 0; tt < nt; ++tt) {
      const int m = s_md[tt];
      if (m >= kCalibModalities) continue;
      const double w = s_w[tt];
      const double a0 = xi[tt][2 * ti], a1 = xi[tt][2 * ti + 1];
      const double b0 = xj[tt][2 * tj], b1 = xj[tt][2 * tj + 1];
      const double p00 = a0 * b0, p01 = a0 * b1, p10 = a1 * b0, p11 = a1 * b1;
      if (m == 0) {
        acc0[0] = __builtin_fma(w, p00, acc0[0]); acc0[1] = __builtin_fma(w, p01, acc0[1]);
        acc0[2] = __builtin_fma(w, p10, acc0[2]); acc0[3] = __builtin_fma(w, p11, acc0[3]);
      } else if (m == 1) {
        acc1[0] = __builtin_fma(w, p00, acc1[0]); acc1[1] = __builtin_fma(w, p01, acc1[1]);
        acc1[2] = __builtin_fma(w, p10, acc1[2]); acc1[3] = __builtin_fma(w, p11, acc1[3]);
      } else {
        acc2[0] = __builtin_fma(w, p00, acc2[0]); acc2[1] = __builtin_fma(w, p01, acc2[1]);
        acc2[2] = __builtin_fma(w, p10, acc2[2]); acc2[3] = __builtin_fma(w, p11, acc2[3]);
      }
    }
  }
  const int i0 = bi * kTile + 2 * ti, j0 = bj * kTile + 2 * tj;
  auto store = [&](int m, double x00, double x01, double x10, double x11) {
    double* out = a.part_cov + ((static_cast<size_t>(s) * a.hkv + h) * kCalibModalities + m) * D * D;
    const double x[4] = {x00, x01, x10, x11};
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        out[static_cast<size_t>(i0 + u) * D + j0 + v] = x[2 * u + v];
        if (bi != bj) out[static_cast<size_t>(j0 + v) * D + i0 + u] = x[2 * u + v];
      }
  };
  store(0, acc0[0], acc0[1], acc0[2], acc0[3]);
  store(1, acc1[0], acc1[1], acc1[2], acc1[3]);
  store(2, acc2[0], acc2[1], acc2[2], acc2[3]);
}

// Covariances: the splits' partial sums in split order, divided by W.
template <int D>
__global__ __launch_bounds__(256) void calib_cov_merge_kernel(CovArgs a) {
  const size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t per = static_cast<size_t>(D) * D;
  if (e >= static_cast<size_t>(a.hkv) * kCalibModalities * per) return;
  const size_t hm = e / per;
  double x = 0.0;
  for (int s = 0; s < a.splits; ++s) x += a.part_cov[static_cast<size_t>(s) * a.hkv * kCalibModalities * per + e];
  const double w = a.wsum[hm];
  a.cov[e] = w > 0.0 ? x / w : 0.0;
}

// -------------------------------------------------------------- eigenbasis

// Cyclic Jacobi on one symmetric matrix per workgroup (Golub & Van Loan,
// "Matrix Computations", Sec. 8.5: the symmetric Schur 2 x 2 rotation and
// the parallel ordering).  Each sweep visits every pair (p, q) once through
// D - 1 rounds of D / 2 disjoint pairs (round-robin ordering: player 0
// fixed, the others rotated).
//
// Phase 1 rotates A alone, in LDS: a round forms its rotations from the
// current matrix, then applies J^T A J one 2 x 2 block at a time (blocks
// (ki, kj) and (kj, ki) from one task, so A stays exactly symmetric).  A pair
// whose off-diagonal entry is negligible (against its diagonal, or below
// the rounding noise of the whole matrix) is set to zero without a rotation;
// the sweeps end when one rotates nothing (at most kJacobiSweeps).  Each
// round's tangents t go to a log in the workspace.
// Phase 2 replays the log on V = I (V^T kept in LDS where A was):
// V <- V J round by round, c and s recomputed from t with the same
// operations as in phase 1, so they are the same numbers.
template <int D>
constexpr int jacobi_threads() { return D == 128 ? 512 : 256; }

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

// Barrier for LDS traffic only: the log's global stores stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D>
__global__ __launch_bounds__(jacobi_threads<D>()) void calib_jacobi_kernel(const double* cov, float* rot,
                                                                           double* evals, double* work) {
  constexpr int NP = D / 2;
  constexpr int LD = D + 1;
  constexpr int NT = jacobi_threads<D>();
  // 2 x 2 block tasks (ki, kj), ki <= kj: NP (NP + 1) / 2 of them, numbered
  // densely (block_task) and dealt round robin, NAT per thread at most
  constexpr int NTASK = NP * (NP + 1) / 2;
  constexpr int NAT = (NTASK + NT - 1) / NT;
  constexpr int NWT = NP * D / NT;    // (pair, column) tasks of V^T per thread
  static_assert(NWT * NT == NP * D && NT >= D && D % NWT == 0, "tasks divide evenly");
  constexpr double kNegligible = 0x1p-53;   // |a_pq| <= 2^-53 sqrt(|a_pp a_qq|): already diagonal to rounding
  __shared__ double A[D * LD];             // phase 1: A; phase 2: V^T (row j = column j of V)
  __shared__ double s_c[2][NP], s_s[2][NP], s_t[NP];
  __shared__ int s_p[2][NP], s_q[2][NP];
  __shared__ int s_changed;
  __shared__ double s_lam[D];
  __shared__ double s_sq[NT];
  const int mat = blockIdx.x, tid = threadIdx.x;
  const double* C = cov + static_cast<size_t>(mat) * D * D;
  double* log = work + static_cast<size_t>(mat) * kJacobiSweeps * (D - 1) * NP;
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
        s_p[0][k] = p;
        s_q[0][k] = q;
        s_c[0][k] = c;
        s_s[0][k] = t * c;
        s_t[k] = t;
        log[(static_cast<size_t>(sweep) * (D - 1) + r) * NP + k] = t;
      }
      lds_barrier();
      // this round's tasks touch disjoint entries: all loads, then all stores
      double blk[NAT][4];
#pragma unroll
      for (int u = 0; u < NAT; ++u) {
        const int e = tid + u * NT;
        if (e < NTASK) {
          int ki, kj;
          block_task<NP>(e, ki, kj);
          const int pi = s_p[0][ki], qi = s_q[0][ki], pj = s_p[0][kj], qj = s_q[0][kj];
          blk[u][0] = A[pi * LD + pj];
          blk[u][1] = A[pi * LD + qj];
          blk[u][2] = A[qi * LD + pj];
          blk[u][3] = A[qi * LD + qj];
        }
      }
#pragma unroll
      for (int u = 0; u < NAT; ++u) {
        const int e = tid + u * NT;
        if (e >= NTASK) continue;
        int ki, kj;
        block_task<NP>(e, ki, kj);
        const int pi = s_p[0][ki], qi = s_q[0][ki], pj = s_p[0][kj], qj = s_q[0][kj];
        const double a_pp = blk[u][0], a_pq = blk[u][1], a_qp = blk[u][2], a_qq = blk[u][3];
        if (ki == kj) {
          // the rotated pair itself: exact zero off the diagonal
          const double t = s_t[ki];
          A[pi * LD + pi] = a_pp - t * a_pq;
          A[qi * LD + qi] = a_qq + t * a_pq;
          A[pi * LD + qi] = 0.0;
          A[qi * LD + pi] = 0.0;
          continue;
        }
        const double ci = s_c[0][ki], si = s_s[0][ki], cj = s_c[0][kj], sj = s_s[0][kj];
        // rows (J_i^T from the left), then columns (J_j from the right)
        const double r_pp = ci * a_pp - si * a_qp, r_pq = ci * a_pq - si * a_qq;
        const double r_qp = si * a_pp + ci * a_qp, r_qq = si * a_pq + ci * a_qq;
        const double n_pp = cj * r_pp - sj * r_pq, n_pq = sj * r_pp + cj * r_pq;
        const double n_qp = cj * r_qp - sj * r_qq, n_qq = sj * r_qp + cj * r_qq;
        A[pi * LD + pj] = n_pp;
        A[pj * LD + pi] = n_pp;
        A[pi * LD + qj] = n_pq;
        A[qj * LD + pi] = n_pq;
        A[qi * LD + pj] = n_qp;
        A[pj * LD + qi] = n_qp;
        A[qi * LD + qj] = n_qq;
        A[qj * LD + qi] = n_qq;
      }
      lds_barrier();
    }
    sweeps = sweep + 1;
    if (!s_changed) break;
  }
  __syncthreads();   // the log is complete and visible to the workgroup
  if (tid < D) s_lam[tid] = A[tid * LD + tid];
  __syncthreads();

  // ---- phase 2: V^T <- J^T V^T, replayed from the log, starting from I
  for (int e = tid; e < D * D; e += NT) A[(e / D) * LD + e % D] = (e / D == e % D) ? 1.0 : 0.0;
  // the log is read one round ahead, so its load waits behind a round's work
  const int rounds = sweeps * (D - 1);
  double t_next = (tid < NP && rounds > 0) ? log[tid] : 0.0;
  for (int sweep = 0; sweep < sweeps; ++sweep) {
    for (int r = 0; r < D - 1; ++r) {
      // parameter buffers alternate with the round count (D - 1 rounds per
      // sweep is odd, so not with r): one barrier per round suffices
      const int round = sweep * (D - 1) + r;
      const int b = round & 1;
      if (tid < NP) {
        const int k = tid;
        int p, q;
        jacobi_pair<D>(r, k, p, q);
        const double t = t_next;
        if (round + 1 < rounds) t_next = log[static_cast<size_t>(round + 1) * NP + k];
        const double c = 1.0 / sqrt(1.0 + t * t);
        s_p[b][k] = p;
        s_q[b][k] = q;
        s_c[b][k] = c;
        s_s[b][k] = t * c;
      }
      lds_barrier();   // (the prefetched log load stays in flight)
      // thread = one pair, columns i0, i0 + D / NWT, ...: the pair's
      // parameters are read once per round
      constexpr int CS = D / NWT;                 // column stride
      const int k = tid / CS, i0 = tid % CS;
      const int rp = s_p[b][k] * LD, rq = s_q[b][k] * LD;
      const double c = s_c[b][k], sn = s_s[b][k];
      double wx[NWT], wy[NWT];
#pragma unroll
      for (int u = 0; u < NWT; ++u) {
        wx[u] = A[rp + i0 + u * CS];
        wy[u] = A[rq + i0 + u * CS];
      }
#pragma unroll
      for (int u = 0; u < NWT; ++u) {
        A[rp + i0 + u * CS] = c * wx[u] - sn * wy[u];
        A[rq + i0 + u * CS] = sn * wx[u] + c * wy[u];
      }
    }
  }
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
  int splits, split_tokens;  // covariance tiles
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

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

CalibPlan plan_calib(const kvq_calib_shape* s) {
  CalibPlan p;
  const int d = s->head_dim, hkv = s->n_kv_heads, n = s->n_tokens;
  p.rows = s->n_queries * (s->n_q_heads / hkv);
  p.nblk = std::max(1, (n + kTokBlock - 1) / kTokBlock);
  p.contrib_bytes = align256(static_cast<size_t>(hkv) * p.nblk * p.rows * 2 * sizeof(double)) +
                    align256(static_cast<size_t>(hkv) * p.rows * 2 * sizeof(double));
  // covariance: about 512 workgroups, at least 256 tokens per split, at most 64 splits
  const int nb = d / kTile;
  const int tiles = nb * (nb + 1) / 2;
  int splits = std::max(1, (512 + tiles * hkv - 1) / (tiles * hkv));
  splits = std::min(splits, std::max(1, (n + 255) / 256));
  splits = std::min(splits, 64);
  int per = (std::max(n, 1) + splits - 1) / splits;
  per = ((per + kTileTokens - 1) / kTileTokens) * kTileTokens;
  splits = std::max(1, (n + per - 1) / per);
  p.splits = splits;
  p.split_tokens = per;
  p.mean_split_tokens = 1024;
  p.mean_splits = std::max(1, (n + 1023) / 1024);
  p.cov_bytes = align256(static_cast<size_t>(p.mean_splits) * hkv * kCalibModalities * (d + 1) * sizeof(double)) +
                align256(static_cast<size_t>(hkv) * kCalibModalities * d * sizeof(double)) +
                align256(static_cast<size_t>(splits) * hkv * kCalibModalities * d * d * sizeof(double));
  p.eig_bytes = static_cast<size_t>(3) * hkv * kJacobiSweeps * (d - 1) * (d / 2) * sizeof(double);
  return p;
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
  constexpr int NB = D / kTile;
  const dim3 gpart(a.mean_splits, a.hkv);
  const dim3 gmm((a.hkv * kCalibModalities * D + 255) / 256);
  const dim3 gtile(NB * (NB + 1) / 2, a.splits, a.hkv);
  const size_t ncov = static_cast<size_t>(a.hkv) * kCalibModalities * D * D;
  const dim3 gcm(static_cast<unsigned>((ncov + 255) / 256));
  if (vb) {
    hipLaunchKernelGGL((calib_mean_part_kernel<D, true>), gpart, dim3(256), 0, st, a);
    hipLaunchKernelGGL((calib_mean_merge_kernel<D>), gmm, dim3(256), 0, st, a);
    hipLaunchKernelGGL((calib_cov_part_kernel<D, true>), gtile, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((calib_mean_part_kernel<D, false>), gpart, dim3(256), 0, st, a);
    hipLaunchKernelGGL((calib_mean_merge_kernel<D>), gmm, dim3(256), 0, st, a);
    hipLaunchKernelGGL((calib_cov_part_kernel<D, false>), gtile, dim3(256), 0, st, a);
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
  // the rotation log: one tangent per (sweep, round, pair)
  return static_cast<size_t>(count) * kJacobiSweeps * (head_dim - 1) * (head_dim / 2) * sizeof(double);
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
  a.part_cov = reinterpret_cast<double*>(w);
  a.n = shape->n_tokens;
  a.hkv = hkv;
  a.splits = p.splits;
  a.split_tokens = p.split_tokens;
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
  (void)hipGetLastError();
  double* work = static_cast<double*>(workspace);
  if (head_dim == 128)
    hipLaunchKernelGGL(calib_jacobi_kernel<128>, dim3(count), dim3(jacobi_threads<128>()), 0, stream, cov, rot,
                       eigenvalues, work);
  else
    hipLaunchKernelGGL(calib_jacobi_kernel<64>, dim3(count), dim3(jacobi_threads<64>()), 0, stream, cov, rot,
                       eigenvalues, work);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

}  // extern "C"
