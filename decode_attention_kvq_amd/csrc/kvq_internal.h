// Internal declarations shared by the HIP translation units of libkvq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kGroupTokens = 32;   // key-statistics group length (positions 32g .. 32g+31)
constexpr int kModalities = 3;     // video, audio, text
constexpr int kMaxGroupHeads = 16; // query heads per KV head supported by the kernels

// Arguments of the three append kernels (passed by value).
struct AppendArgs {
  uint8_t* k_codes;
  uint16_t* k_stats;
  uint8_t* v_codes;
  uint16_t* v_norms;
  uint8_t* modality;
  const int32_t* page_table;
  int32_t* seq_len;
  void* k_tail;
  const void* k_new;
  const void* v_new;
  const uint8_t* modality_new;
  const int8_t* signs;
  const float* rot;
  int32_t b0, n_new, hkv, page_tokens, max_pages, num_pages;
  double inv_sqrt_d;   // fl(1 / fl(sqrt(d))), computed on the host
  double sqrt_d;       // fl(sqrt(d))
  double c0, c3;       // outer levels (exact fp64 images of the fp32 levels)
  double thr0, thr1, thr2;  // decision thresholds (c_k + c_{k+1}) / 2
};

struct RotateArgs {
  const void* q;
  float* q_rot;
  const int8_t* signs;
  int32_t hq, group;   // group = Hq / Hkv
  double inv_sqrt_d;
};

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
  float* out;
  float* partials;        // [B][Hq][splits][2 + 3d]
  int32_t hq, hkv, group, page_tokens, max_pages, num_pages;
  int32_t splits;         // partitions per (session, KV head)
  int32_t split_tokens;   // positions per partition (multiple of 32)
  float scale_log2e;      // softmax scale * log2(e)
  float value_scale;      // 1 / sqrt(d)
  float lv[4];            // key levels mapped to [0, 1]: (c_k - c0) / (c3 - c0)
  float cv[4];            // value levels c_k
};

hipError_t launch_append(int d, bool bf16, int nb, const AppendArgs& a, hipStream_t s);
hipError_t launch_rotate_query(int d, bool bf16, int batch, const RotateArgs& a, hipStream_t s);
hipError_t launch_decode(int d, int batch, const DecodeArgs& a, hipStream_t s);

}  // namespace kvq
