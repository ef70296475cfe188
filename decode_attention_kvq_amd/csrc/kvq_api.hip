// Host side of the C ABI: argument validation, partition planning and kernel
// dispatch.  Nothing here allocates device memory or synchronises.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <queue>
#include <utility>

#include "kvq_internal.h"

namespace {

using kvq::kGroupTokens;
using kvq::kMaxGroupHeads;

bool codebook_ok(const float* c, int n) {
  for (int k = 0; k < n; ++k)
    if (!isfinite(c[k]) || (k > 0 && !(c[k - 1] < c[k]))) return false;
  return true;
}

kvq_status check_config(const kvq_config* cfg) {
  if (!cfg) return KVQ_ERR_INVALID;
  if (cfg->head_dim != 64 && cfg->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  if (cfg->n_q_heads <= 0 || cfg->n_kv_heads <= 0 || cfg->batch <= 0) return KVQ_ERR_INVALID;
  if (cfg->n_q_heads % cfg->n_kv_heads != 0) return KVQ_ERR_INVALID;
  if (cfg->n_q_heads / cfg->n_kv_heads > kMaxGroupHeads) return KVQ_ERR_UNSUPPORTED;
  if (cfg->page_tokens <= 0 || cfg->page_tokens % kGroupTokens != 0) return KVQ_ERR_INVALID;
  if (cfg->max_pages <= 0 || cfg->num_pages <= 0) return KVQ_ERR_INVALID;
  if ((int64_t)cfg->max_pages * cfg->page_tokens > INT32_MAX) return KVQ_ERR_INVALID;
  if (cfg->kv_dtype != KVQ_F32 && cfg->kv_dtype != KVQ_BF16) return KVQ_ERR_UNSUPPORTED;
  if (cfg->key_mode != KVQ_KEYS_GROUP_MINMAX && cfg->key_mode != KVQ_KEYS_PER_TOKEN) return KVQ_ERR_INVALID;
  if (cfg->bits < 2 || cfg->bits > 4) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

kvq_status check_params(const kvq_config* cfg, const kvq_params* p) {
  if (!p || !p->signs || !p->rot) return KVQ_ERR_INVALID;
  if (!codebook_ok(p->codebook, 1 << cfg->bits)) return KVQ_ERR_INVALID;
  return KVQ_OK;
}

kvq_status check_cache(const kvq_cache* c) {
  if (!c || !c->k_codes || !c->k_stats || !c->v_codes || !c->v_norms || !c->modality ||
      !c->page_table || !c->seq_len || !c->k_tail || !c->append_tickets || !c->seq_len_host)
    return KVQ_ERR_INVALID;
  return KVQ_OK;
}

// Context partitions of a decode: each (session, KV head) context is split
// into partitions of near-equal whole 32-position groups (the first `extra`
// of a session's partitions one group longer), one workgroup each.  The
// partitions of all sessions fill the compute units once (256 CUs; long
// partitions beat rounds of short ones, which each pay the set-up and the
// epilogue again).  Up to kPlanSessions sessions get partition counts of
// their own: every session starts with its minimum (one partition, or more
// when a partition would span more than kPartitionPages - 2 pages, which the
// older partition kernel keeps in LDS) and the remaining grid columns go
// one at a time to the session whose partitions are longest, so a ragged
// batch ends together; no partition gets fewer than 8 groups' worth of
// columns (one group per wavefront).  Larger batches share one uniform
// count.  step = 1 (the fused decode step) adds one slot and one grid column
// per session for the open group.  The plan depends only on (cfg, the
// host-side lengths, step).
using Plan = kvq::DecodeArgs;   // the plan's fields of the kernel arguments

constexpr int64_t kUnit = kGroupTokens * kvq::kDecodeWaves;
constexpr int64_t kMaxPlanSplits = 4096;

int64_t max_split_tokens(const kvq_config* cfg) {
  return ((int64_t)(kvq::kPartitionPages - 2) * cfg->page_tokens / kUnit) * kUnit;
}

int64_t cap_groups(const kvq_config* cfg) { return max_split_tokens(cfg) / kGroupTokens; }
int64_t groups_of(int64_t len) { return (std::max<int64_t>(len, 0) + kGroupTokens - 1) / kGroupTokens; }
int64_t min_parts(const kvq_config* cfg, int64_t groups) {
  return std::max<int64_t>(1, (groups + cap_groups(cfg) - 1) / cap_groups(cfg));
}
int64_t max_parts(const kvq_config* cfg, int64_t groups) {
  return std::max(min_parts(cfg, groups), (groups + kvq::kDecodeWaves - 1) / kvq::kDecodeWaves);
}
// grid columns that give one workgroup per compute unit
int64_t plan_columns(const kvq_config* cfg) { return std::max<int64_t>(1, 256 / cfg->n_kv_heads); }

// lens: host-side session lengths; every session is planned for lens[b] + extra positions.
Plan plan_decode(const kvq_config* cfg, const int32_t* lens, int32_t extra, int step) {
  Plan p{};
  const int B = cfg->batch;
  const int64_t cols = plan_columns(cfg);
  p.step = step;
  if (B <= kvq::kPlanSessions) {
    int64_t g[kvq::kPlanSessions], n[kvq::kPlanSessions];
    int64_t used = 0;
    for (int b = 0; b < B; ++b) {
      g[b] = groups_of((int64_t)lens[b] + extra);
      n[b] = min_parts(cfg, g[b]);
      used += n[b] + step;
    }
    // (partition length in groups, -session): the longest partitions first, then the lowest session
    std::priority_queue<std::pair<int64_t, int>> q;
    for (int b = 0; b < B; ++b)
      if (n[b] < max_parts(cfg, g[b])) q.push({(g[b] + n[b] - 1) / n[b], -b});
    while (used < cols && !q.empty()) {
      const int b = -q.top().second;
      q.pop();
      ++n[b];
      ++used;
      if (n[b] < max_parts(cfg, g[b])) q.push({(g[b] + n[b] - 1) / n[b], -b});
    }
    p.ntab = B;
    p.tab_start[0] = 0;
    for (int b = 0; b < B; ++b) {
      p.tab_start[b + 1] = p.tab_start[b] + (int)(n[b] + step);
      p.tab_tokens[b] = (int)(g[b] / n[b] * kGroupTokens);
      p.tab_extra[b] = (int)(g[b] % n[b]);
    }
    p.pstride = p.tab_start[B];
    p.splits = (int)*std::max_element(n, n + B);
  } else {
    int32_t max_len = 0;
    for (int b = 0; b < B; ++b) max_len = std::max(max_len, lens[b]);
    const int64_t g = groups_of((int64_t)max_len + extra);
    int64_t n = std::max<int64_t>(1, cols / B - step);
    n = std::max(min_parts(cfg, g), std::min(n, max_parts(cfg, g)));
    p.ntab = 0;
    p.splits = (int)n;
    p.split_tokens = (int)(g / n * kGroupTokens);
    p.split_extra = (int)(g % n);
    p.pstride = (int)(B * (n + step));
  }
  return p;
}

// Longest context the plan supports (a session's partitions and the step's
// slot stay within kMaxPlanSplits).
bool plan_supported(const kvq_config* cfg, int32_t max_len) {
  return (int64_t)max_len <= (kMaxPlanSplits - 1) * max_split_tokens(cfg);
}

// Upper bound of plan_decode(cfg, lens, extra, step).pstride over every
// length <= max_len (extra included), so a workspace sized for max_len
// serves every shorter context too.
int64_t slots_bound(const kvq_config* cfg, int32_t max_len, int step) {
  const int64_t B = cfg->batch;
  return std::max(plan_columns(cfg), B * (min_parts(cfg, groups_of(max_len)) + step)) + B * step;
}

// Workspace: one partial result per (query head, slot).
size_t workspace_floats(const kvq_config* cfg, int64_t slots) {
  return (size_t)cfg->n_q_heads * slots * (kvq::kPartialHeader + 3 * cfg->head_dim);
}

}  // namespace

extern "C" {

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_CAPACITY: return "cache capacity exceeded";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_LAUNCH: return "kernel launch failed";
    case KVQ_ERR_SCRATCH: return "decode partials exceed the no-allocation scratch (KVQ_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

kvq_status kvq_cache_buffer_bytes(const kvq_config* cfg, size_t out[6]) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!out) return KVQ_ERR_INVALID;
  const size_t d = cfg->head_dim, hkv = cfg->n_kv_heads, pt = cfg->page_tokens, np = cfg->num_pages;
  const size_t groups = np * hkv * (pt / kGroupTokens);
  out[0] = groups * 4 * cfg->bits * d;     // k_codes
  out[1] = groups * 2 * d * 2;             // k_stats (fp16)
  out[2] = groups * 4 * cfg->bits * d;     // v_codes
  out[3] = np * hkv * pt * 2;              // v_norms (fp16)
  out[4] = np * pt;                        // modality
  out[5] = (size_t)cfg->batch * hkv * kGroupTokens * d * (cfg->kv_dtype == KVQ_BF16 ? 2 : 4);
  return KVQ_OK;
}

// Validation and kernel arguments of an append (nothing is launched).
static kvq_status prepare_append(const kvq_config* cfg, const kvq_cache* cache, const kvq_params* params,
                                 int32_t b0, int32_t nb, int32_t n_new, const void* k_new, const void* v_new,
                                 const uint8_t* modality_new, kvq::AppendArgs& a) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if ((st = check_params(cfg, params)) != KVQ_OK) return st;
  if ((st = check_cache(cache)) != KVQ_OK) return st;
  if (b0 < 0 || nb <= 0 || b0 + nb > cfg->batch || n_new < 0) return KVQ_ERR_INVALID;
  if (n_new == 0) return KVQ_OK;
  if (!k_new || !v_new || !modality_new) return KVQ_ERR_INVALID;
  const int64_t cap = (int64_t)cfg->max_pages * cfg->page_tokens;
  for (int b = b0; b < b0 + nb; ++b) {
    if (cache->seq_len_host[b] < 0) return KVQ_ERR_INVALID;
    if ((int64_t)cache->seq_len_host[b] + n_new > cap) return KVQ_ERR_CAPACITY;
  }
  const double sd = sqrt((double)cfg->head_dim);
  a = kvq::AppendArgs{};
  a.k_codes = cache->k_codes;
  a.k_stats = cache->k_stats;
  a.v_codes = cache->v_codes;
  a.v_norms = cache->v_norms;
  a.modality = cache->modality;
  a.page_table = cache->page_table;
  a.seq_len = cache->seq_len;
  a.k_tail = cache->k_tail;
  a.tickets = cache->append_tickets;
  a.k_new = k_new;
  a.v_new = v_new;
  a.modality_new = modality_new;
  a.signs = params->signs;
  a.rot = params->rot;
  a.b0 = b0;
  a.n_new = n_new;
  a.hkv = cfg->n_kv_heads;
  a.page_tokens = cfg->page_tokens;
  a.max_pages = cfg->max_pages;
  a.num_pages = cfg->num_pages;
  a.inv_sqrt_d = 1.0 / sd;
  a.sqrt_d = sd;
  const int n = 1 << cfg->bits;
  a.c0 = params->codebook[0];
  a.cmax = params->codebook[n - 1];
  a.nthr = n - 1;
  for (int k = 0; k < 15; ++k)
    a.thr[k] = k < n - 1 ? ((double)params->codebook[k] + (double)params->codebook[k + 1]) / 2.0 : INFINITY;
  a.bits = cfg->bits;
  a.key_mode = cfg->key_mode;
  a.rot_heads = 0;
  return KVQ_OK;
}

// Validation and kernel arguments of a query rotation.
static kvq_status prepare_rotate(const kvq_config* cfg, const kvq_params* params, int32_t batch, const void* q,
                                 int32_t q_dtype, float* q_rot, kvq::RotateArgs& a) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!params || !params->signs) return KVQ_ERR_INVALID;
  if (batch <= 0 || !q || !q_rot) return KVQ_ERR_INVALID;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return KVQ_ERR_UNSUPPORTED;
  a.q = q;
  a.q_rot = q_rot;
  a.signs = params->signs;
  a.hq = cfg->n_q_heads;
  a.group = cfg->n_q_heads / cfg->n_kv_heads;
  a.inv_sqrt_d = 1.0 / sqrt((double)cfg->head_dim);
  return KVQ_OK;
}

kvq_status kvq_quantize_append(const kvq_config* cfg, kvq_cache* cache, const kvq_params* params,
                               int32_t b0, int32_t nb, int32_t n_new, const void* k_new,
                               const void* v_new, const uint8_t* modality_new, hipStream_t stream) {
  kvq::AppendArgs a;
  const kvq_status st = prepare_append(cfg, cache, params, b0, nb, n_new, k_new, v_new, modality_new, a);
  if (st != KVQ_OK || n_new == 0) return st;
  hipError_t e = kvq::launch_append(cfg->head_dim, cfg->kv_dtype == KVQ_BF16, nb, a, stream);
  if (e != hipSuccess) return KVQ_ERR_LAUNCH;
  for (int b = b0; b < b0 + nb; ++b) cache->seq_len_host[b] += n_new;
  return KVQ_OK;
}

kvq_status kvq_append_and_rotate(const kvq_config* cfg, kvq_cache* cache, const kvq_params* params,
                                 int32_t b0, int32_t nb, int32_t n_new, const void* k_new,
                                 const void* v_new, const uint8_t* modality_new, int32_t batch,
                                 const void* q, int32_t q_dtype, float* q_rot, hipStream_t stream) {
  kvq::AppendArgs a;
  kvq::RotateArgs r;
  kvq_status st = prepare_append(cfg, cache, params, b0, nb, n_new, k_new, v_new, modality_new, a);
  if (st != KVQ_OK) return st;
  if ((st = prepare_rotate(cfg, params, batch, q, q_dtype, q_rot, r)) != KVQ_OK) return st;
  hipError_t e;
  if (n_new == 0) {
    e = kvq::launch_rotate_query(cfg->head_dim, q_dtype == KVQ_BF16, batch, r, stream);
  } else {
    a.rq = r;
    a.rot_heads = batch * cfg->n_q_heads;
    a.rot_bf16 = q_dtype == KVQ_BF16;
    e = kvq::launch_append(cfg->head_dim, cfg->kv_dtype == KVQ_BF16, nb, a, stream);
  }
  if (e != hipSuccess) return KVQ_ERR_LAUNCH;
  for (int b = b0; b < b0 + nb; ++b) cache->seq_len_host[b] += n_new;
  return KVQ_OK;
}

kvq_status kvq_rotate_query(const kvq_config* cfg, const kvq_params* params, int32_t batch,
                            const void* q, int32_t q_dtype, float* q_rot, hipStream_t stream) {
  kvq::RotateArgs a;
  const kvq_status st = prepare_rotate(cfg, params, batch, q, q_dtype, q_rot, a);
  if (st != KVQ_OK) return st;
  hipError_t e = kvq::launch_rotate_query(cfg->head_dim, q_dtype == KVQ_BF16, batch, a, stream);
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t max_len) {
  if (check_config(cfg) != KVQ_OK || max_len < 0) return 0;
  return workspace_floats(cfg, slots_bound(cfg, max_len, 0)) * sizeof(float);
}

size_t kvq_decode_step_workspace_bytes(const kvq_config* cfg, int32_t max_len) {
  if (check_config(cfg) != KVQ_OK || max_len < 0) return 0;
  return workspace_floats(cfg, slots_bound(cfg, max_len, 1)) * sizeof(float);
}

}  // extern "C"

// ------------------------------------------------ decode without allocation
//
// The partial results of kvq_decode_attention_noalloc live in `scratch`, a
// device array of this file that each GPU the library runs on holds until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): its device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// kept in g_scratch_ptr.
static __device__ __align__(256) float scratch[KVQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, or null on error.
static void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Checks of a decode's own arguments (those of the cache, parameters and
// configuration included) and its plan for the host-side lengths (+ extra
// positions, the fused step's append), with the longest length.
static kvq_status check_decode(const kvq_config* cfg, const kvq_cache* cache, const kvq_params* params,
                               const void* q, float scale, const void* out, int32_t out_dtype, int32_t extra,
                               int32_t& max_len) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if ((st = check_params(cfg, params)) != KVQ_OK) return st;
  if ((st = check_cache(cache)) != KVQ_OK) return st;
  if (!q || !out || !isfinite(scale)) return KVQ_ERR_INVALID;
  if (out_dtype != KVQ_F32 && out_dtype != KVQ_BF16) return KVQ_ERR_UNSUPPORTED;
  max_len = 0;
  const int64_t cap = (int64_t)cfg->max_pages * cfg->page_tokens;
  for (int b = 0; b < cfg->batch; ++b) {
    if (cache->seq_len_host[b] < 0 || cache->seq_len_host[b] > cap) return KVQ_ERR_INVALID;
    if ((int64_t)cache->seq_len_host[b] + extra > cap) return KVQ_ERR_CAPACITY;
    max_len = std::max(max_len, cache->seq_len_host[b] + extra);
  }
  if (!plan_supported(cfg, max_len)) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

// Kernel arguments of a decode with the given plan and partials buffer.
static kvq::DecodeArgs decode_args(const kvq_config* cfg, const kvq_cache* cache, const kvq_params* params,
                                   const float* q_rot, float scale, void* out, int32_t out_dtype, const Plan& plan,
                                   void* partials) {
  const int nlev = 1 << cfg->bits;
  const double c0 = params->codebook[0], c3 = params->codebook[nlev - 1];   // outer levels
  kvq::DecodeArgs a = plan;   // the plan's fields
  a.k_codes = cache->k_codes;
  a.k_stats = cache->k_stats;
  a.v_codes = cache->v_codes;
  a.v_norms = cache->v_norms;
  a.modality = cache->modality;
  a.page_table = cache->page_table;
  a.seq_len = cache->seq_len;
  a.q_rot = q_rot;
  a.rot = params->rot;
  a.out = out;
  a.out_bf16 = out_dtype == KVQ_BF16;
  a.partials = static_cast<float*>(partials);
  a.batch = cfg->batch;
  a.hq = cfg->n_q_heads;
  a.hkv = cfg->n_kv_heads;
  a.group = cfg->n_q_heads / cfg->n_kv_heads;
  a.page_tokens = cfg->page_tokens;
  a.max_pages = cfg->max_pages;
  a.num_pages = cfg->num_pages;
  a.page_shift = -1;
  if ((cfg->page_tokens & (cfg->page_tokens - 1)) == 0) {
    a.page_shift = 0;
    while ((1 << a.page_shift) < cfg->page_tokens) ++a.page_shift;
  }
  a.blocks_per_page = cfg->n_kv_heads * (cfg->page_tokens / kGroupTokens);
  // The streaming partition kernel addresses every cache array with 31-bit
  // byte offsets; larger pools take the pointer-addressed kernel.
  a.offsets31 = (size_t)cfg->num_pages * cfg->n_kv_heads * cfg->page_tokens * cfg->head_dim * cfg->bits / 8 <
                ((size_t)1 << 31);
  a.scale_log2e = (float)((double)scale * 1.4426950408889634);
  a.value_scale = (float)(1.0 / sqrt((double)cfg->head_dim));
  // normalized levels l_k = (2 c_k - c0 - c_{n-1}) / (c_{n-1} - c0) as fp16
  // and, for the scores at 3 / 4 bits, 2^12 times the part fp16 missed
  uint16_t lv[16] = {0}, lr[16] = {0};
  for (int k = 0; k < nlev; ++k) {
    const double l = (2.0 * params->codebook[k] - c0 - c3) / (c3 - c0);
    const _Float16 v = (_Float16)l;
    lv[k] = __builtin_bit_cast(uint16_t, v);
    lr[k] = __builtin_bit_cast(uint16_t, (_Float16)((l - (double)v) * 4096.0));
    if (k < 4) a.level_f32[k] = (float)l;
  }
  for (int w = 0; w < 8; ++w) {
    a.level_f16[w] = lv[2 * w] | ((uint32_t)lv[2 * w + 1] << 16);
    a.level_lo_f16[w] = lr[2 * w] | ((uint32_t)lr[2 * w + 1] << 16);
  }
  a.cmid = (float)((c0 + c3) / 2.0);
  a.chalf = (float)((c3 - c0) / 2.0);
  a.key_mode = cfg->key_mode;
  a.bits = cfg->bits;
  return a;
}

// Per-token keys and 3- / 4-bit codes run on the streaming partition kernel
// only.
static bool decode_supported(const kvq::DecodeArgs& a) {
  return !((a.key_mode == KVQ_KEYS_PER_TOKEN || a.bits != 2) && (a.group > 8 || !a.offsets31 || a.page_shift < 0));
}

// The decode behind both entry points: the partial results go to the
// caller's `workspace` (workspace_bytes long) or, with scratch = true, to the
// current device's scratch array; every argument is checked before either is
// touched.
static kvq_status decode_impl(const kvq_config* cfg, const kvq_cache* cache, const kvq_params* params,
                              const float* q_rot, float scale, void* out, int32_t out_dtype, void* workspace,
                              size_t workspace_bytes, bool scratch, hipStream_t stream) {
  int32_t max_len = 0;
  kvq_status st = check_decode(cfg, cache, params, q_rot, scale, out, out_dtype, 0, max_len);
  if (st != KVQ_OK) return st;
  const Plan plan = plan_decode(cfg, cache->seq_len_host, 0, 0);
  const size_t need = workspace_floats(cfg, plan.pstride) * sizeof(float);
  if (scratch) {
    if (need > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_SCRATCH;
  } else if (!workspace || workspace_bytes < need) {
    return KVQ_ERR_WORKSPACE;
  }
  kvq::DecodeArgs a = decode_args(cfg, cache, params, q_rot, scale, out, out_dtype, plan, workspace);
  if (!decode_supported(a)) return KVQ_ERR_UNSUPPORTED;
  if (scratch) {
    a.partials = static_cast<float*>(scratch_address());
    if (!a.partials) return KVQ_ERR_LAUNCH;
  }
  hipError_t e = kvq::launch_decode(cfg->head_dim, cfg->batch, a, stream);
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}


extern "C" {

kvq_status kvq_decode_attention(const kvq_config* cfg, const kvq_cache* cache,
                                const kvq_params* params, const float* q_rot, float scale,
                                void* out, int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return decode_impl(cfg, cache, params, q_rot, scale, out, out_dtype, workspace, workspace_bytes, false, stream);
}

kvq_status kvq_decode_attention_noalloc(const kvq_config* cfg, const kvq_cache* cache,
                                        const kvq_params* params, const float* q_rot, float scale,
                                        void* out, int32_t out_dtype, hipStream_t stream) {
  return decode_impl(cfg, cache, params, q_rot, scale, out, out_dtype, nullptr, KVQ_NOALLOC_SCRATCH_BYTES, true,
                     stream);
}

kvq_status kvq_decode_step(const kvq_config* cfg, kvq_cache* cache, const kvq_params* params,
                           const void* k_new, const void* v_new, const uint8_t* modality_new, const void* q,
                           int32_t q_dtype, float* q_rot, float scale, void* out, int32_t out_dtype,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // every check first: nothing is launched unless the whole step can run
  kvq::AppendArgs ap;
  kvq::RotateArgs r;
  kvq_status st = prepare_append(cfg, cache, params, 0, cfg ? cfg->batch : 0, 1, k_new, v_new, modality_new, ap);
  if (st != KVQ_OK) return st;
  if ((st = prepare_rotate(cfg, params, cfg->batch, q, q_dtype, q_rot, r)) != KVQ_OK) return st;
  int32_t max_len = 0;
  if ((st = check_decode(cfg, cache, params, q_rot, scale, out, out_dtype, 1, max_len)) != KVQ_OK) return st;
  const int group = cfg->n_q_heads / cfg->n_kv_heads;
  const bool pow2 = (cfg->page_tokens & (cfg->page_tokens - 1)) == 0;
  const bool offsets31 = (size_t)cfg->num_pages * cfg->n_kv_heads * cfg->page_tokens * cfg->head_dim * cfg->bits / 8 <
                         ((size_t)1 << 31);
  const bool fused = cfg->bits == 2 && cfg->key_mode == KVQ_KEYS_GROUP_MINMAX &&
                     params->codebook[0] == -params->codebook[3] && group <= 8 && pow2 && offsets31 &&
                     q_dtype == cfg->kv_dtype;
  // the fused step plans one more slot (and grid column) per session for the open group
  const Plan plan = plan_decode(cfg, cache->seq_len_host, 1, fused ? 1 : 0);
  const size_t need = workspace_floats(cfg, plan.pstride) * sizeof(float);
  if (!workspace || workspace_bytes < need) return KVQ_ERR_WORKSPACE;
  kvq::DecodeArgs a = decode_args(cfg, cache, params, q_rot, scale, out, out_dtype, plan, workspace);
  if (!decode_supported(a)) return KVQ_ERR_UNSUPPORTED;
  hipError_t e;
  if (!fused) {
    // the same work as kvq_append_and_rotate followed by kvq_decode_attention
    ap.rq = r;
    ap.rot_heads = cfg->batch * cfg->n_q_heads;
    ap.rot_bf16 = q_dtype == KVQ_BF16;
    e = kvq::launch_append(cfg->head_dim, cfg->kv_dtype == KVQ_BF16, cfg->batch, ap, stream);
    if (e == hipSuccess) e = kvq::launch_decode(cfg->head_dim, cfg->batch, a, stream);
  } else {
    ap.rq = r;
    ap.rot_heads = 0;
    ap.append_x = 2;
    ap.defer_len = 1;
    a.step_len = cache->seq_len;
    e = kvq::launch_decode_step(cfg->head_dim, cfg->kv_dtype == KVQ_BF16, cfg->batch, a, ap, stream);
  }
  if (e != hipSuccess) return KVQ_ERR_LAUNCH;
  for (int b = 0; b < cfg->batch; ++b) cache->seq_len_host[b] += 1;
  return KVQ_OK;
}

kvq_status kvq_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups,
                                 hipStream_t stream) {
  if (!buf || !sink || workgroups <= 0 || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15))
    return KVQ_ERR_INVALID;
  return kvq::launch_stream_read(buf, bytes, sink, workgroups, stream) == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

}  // extern "C"
