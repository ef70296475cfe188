// Internal declarations shared by the HIP translation units of libkvq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kGroupTokens = 32;   // key-statistics group length (positions 32g .. 32g+31)
constexpr int kModalities = 3;     // video, audio, text
constexpr int kMaxGroupHeads = 16; // query heads per KV head supported by the kernels

// Arguments of the append kernel (passed by value).
struct RotateArgs {
  const void* q;
  float* q_rot;
  const int8_t* signs;
  int32_t hq, group;   // group = Hq / Hkv
  double inv_sqrt_d;
};

struct AppendArgs {
  uint8_t* k_codes;
  uint16_t* k_stats;
  uint8_t* v_codes;
  uint16_t* v_norms;
  uint8_t* modality;
  const int32_t* page_table;
  int32_t* seq_len;
  void* k_tail;
  int32_t* tickets;    // [batch] completion tickets, zero between appends
  const void* k_new;
  const void* v_new;
  const uint8_t* modality_new;
  const int8_t* signs;
  const float* rot;
  int32_t b0, n_new, hkv, page_tokens, max_pages, num_pages;
  double inv_sqrt_d;   // fl(1 / fl(sqrt(d))), computed on the host
  double sqrt_d;       // fl(sqrt(d))
  double c0, cmax;     // outer levels c0, c_{n-1} (exact fp64 images of the fp32 levels)
  double thr[15];      // decision thresholds (c_k + c_{k+1}) / 2, k < n - 1 (then +inf)
  int32_t nthr;        // n - 1 thresholds, n = 2^bits levels
  int32_t bits;        // code width (2, 3, 4)
  int32_t key_mode;         // KVQ_KEYS_GROUP_MINMAX or KVQ_KEYS_PER_TOKEN
  // Query rotation fused into the same launch (kvq_append_and_rotate):
  // rot_heads query heads (0: none), q in bf16 if rot_bf16.  The launcher
  // sets append_x, the grid columns of the append's own workgroups.
  RotateArgs rq;
  int32_t rot_heads, rot_bf16, append_x;
  // Fused decode step: the append leaves the session lengths to the step's
  // merge.
  int32_t defer_len;
};

// Open-group record of the fused decode step, in the shared memory of the
// workgroup that runs the step's append for one (session, KV head): written
// by the append's key and value roles, then read for the open group's
// partial.  Byte offsets:
constexpr int kStageMeta = 0;      // int32 [0]: 1 if the group's page is mapped, [1]: positions in the group,
                                   // [2]: its first position, [3]: its first new position, [4]: its page
constexpr int kStageBlock = 24;    // int64: its 32-position block (-1: not stored)
constexpr int kStageNorms = 64;    // 32 fp16 value norms
constexpr int kStageMods = 128;    // 32 modality bytes
constexpr int kStageCodes = 256;   // key block (8d bytes), value block (8d bytes), LO and HI rows (2d fp16 each)
__host__ __device__ constexpr int stage_record_bytes(int d) { return kStageCodes + 20 * d; }

// Decode partitions: a workgroup of kDecodeWaves wavefronts streams one
// contiguous range of 32-position groups of one (session, KV head) and writes
// one partial result per query head of the group:
//   [0] running max (base-2 units)  [1] softmax denominator
//   [2] bit mask of modalities with value mass  [3] unused
//   [4..6] per-modality weight sums (only needed for a non-symmetric codebook)
//   [7] unused, then [3][d] per-modality value accumulators.
constexpr int kDecodeWaves = 8;
constexpr int kPartialHeader = 8;
constexpr int kPartitionPages = 512;   // pages one partition may span (the kernel keeps their entries in LDS)
constexpr int kPlanSessions = 128;     // sessions a per-session partition plan can describe

struct DecodeArgs {
  const uint8_t* k_codes;
  const uint16_t* k_stats;
  const uint8_t* v_codes;
  const uint16_t* v_norms;
  const uint8_t* modality;
  const int32_t* page_table;
  const int32_t* seq_len;
  const float* q_rot;
  const float* rot;
  void* out;              // [B][Hq][d] fp32, or bf16 when out_bf16
  float* partials;        // workspace: [Hq][pstride][kPartialHeader + 3d] partials (query head i of every session)
  int32_t batch;
  int32_t hq, hkv, group, page_tokens, max_pages, num_pages;
  // Partition plan.  Session b owns partial slots (and grid columns)
  // [start_b, start_b + n_b + step) of every query head's row of pstride
  // slots: n_b partitions of `tokens` positions (a multiple of 32), the
  // first `extra` of them one 32-position group longer, then (step = 1,
  // the fused decode step) the open group's slot.  Uniform plan (ntab = 0):
  // n_b = splits, tokens = split_tokens, extra = split_extra,
  // start_b = b (splits + step), grid (splits + step, hkv, batch).  Per
  // session (ntab = batch <= kPlanSessions): start_b = tab_start[b],
  // n_b = tab_start[b + 1] - start_b - step, tokens = tab_tokens[b],
  // extra = tab_extra[b], grid (pstride, hkv, 1).
  int32_t splits;
  int32_t split_tokens;
  int32_t split_extra;
  int32_t step;
  int32_t pstride;
  int32_t ntab;
  int32_t tab_start[kPlanSessions + 1];
  int32_t tab_tokens[kPlanSessions];
  int32_t tab_extra[kPlanSessions];
  int32_t page_shift;     // log2(page_tokens) when it is a power of two, else -1
  int32_t blocks_per_page; // hkv * page_tokens / 32: 32-position blocks of one physical page
  int32_t offsets31;       // every cache array is below 2^31 bytes
  float scale_log2e;      // softmax scale * log2(e)
  float value_scale;      // 1 / sqrt(d)
  float cmid, chalf;      // codebook centre (c0 + c3) / 2 and half range (c3 - c0) / 2
  int32_t key_mode;       // KVQ_KEYS_GROUP_MINMAX or KVQ_KEYS_PER_TOKEN
  int32_t bits;           // code width (2, 3, 4)
  int32_t out_bf16;       // write the output as bf16 (round to nearest even) instead of fp32
  uint32_t level_f16[8];  // normalized levels (2 c_k - c0 - c_{n-1}) / (c_{n-1} - c0) as fp16 bits, k < n
  uint32_t level_lo_f16[8]; // 2^12 (level - fp16 level) as fp16 bits (3 / 4 bits: the scores' lo part)
  // Fused decode step (null / unused otherwise): the lengths the merge
  // advances, and the 2-bit normalized levels in fp32.
  int32_t* step_len;
  float level_f32[4];
};

hipError_t launch_append(int d, bool bf16, int nb, const AppendArgs& a, hipStream_t s);
hipError_t launch_rotate_query(int d, bool bf16, int batch, const RotateArgs& a, hipStream_t s);
hipError_t launch_decode(int d, int batch, const DecodeArgs& a, hipStream_t s);
// Fused decode step: the partitions over the closed groups and, per
// (session, KV head), one workgroup for the append (ap: one position per
// session, every session) and the open group's partial, in one launch; then
// the merge.  bf16: query and cache inputs in bf16.
hipError_t launch_decode_step(int d, bool bf16, int batch, const DecodeArgs& a, const AppendArgs& ap,
                              hipStream_t s);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, hipStream_t s);

}  // namespace kvq
