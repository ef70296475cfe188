/*
 * kvq.h - C ABI of the MI355X (gfx950) library for rotation-based 2-bit
 * KV-cache quantization with fused decode attention over the packed cache.
 *
 * Method (OmniKVQuant page, paperlayer.ai summary of arXiv 2609.11582):
 *   - keys: randomized Hadamard rotation, min-max scaling inside short
 *     consecutive-token groups with the group statistics stored, and the
 *     shared fixed codebook on the scaled values (Sec. 2 Method, key bullet);
 *   - values: a separate rotation per modality, then the fixed codebook on
 *     the magnitude-normalised rotated coordinates (Sec. 2 Method, TurboQuant
 *     and value bullets);
 *   - decode: one query rotation per head, attention computed directly on
 *     the 2-bit codes, inverse value rotations applied once after the
 *     aggregation; no dense FP16 cache is ever formed (Sec. 1, Implementation
 *     bullet; Abstract).
 *
 * Conventions shared by every entry point
 *   - All pointers named "device" are HIP device memory owned by the caller;
 *     the library allocates nothing and keeps no global state, apart from
 *     the static device array of kvq_decode_attention_noalloc (see there).
 *   - Keys, values, queries and the value bases must be finite: a NaN or an
 *     infinity gives unspecified codes and outputs (nothing on the device
 *     checks for them).
 *   - Every call is asynchronous on the given stream (0 = null stream).  No
 *     call synchronises.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed validation returns an error code and changes no state.
 *   - Launch failures are reported as KVQ_ERR_LAUNCH.
 *   - d (head_dim) is 64 or 128; G = n_q_heads / n_kv_heads is an integer in
 *     [1, 16]; query head i reads KV head floor(i / G).
 *   - Modalities: 0 video, 1 audio, 2 text.  Keys are grouped in 32-token
 *     groups aligned to absolute positions 32g.
 *
 * Packed cache (paged; a contiguous cache is an identity page table).
 * page_tokens is a multiple of 32; GP = page_tokens / 32 groups per page;
 * b = kvq_config.bits.  Physical page p, KV head h, group-in-page j,
 * position-in-page s:
 *   k_codes  [num_pages][Hkv][GP][4bd] bytes  b-bit key codes of one group
 *   v_codes  [num_pages][Hkv][GP][4bd] bytes  b-bit value codes of one group
 *   k_stats  [num_pages][Hkv][GP][2][d] fp16  rotated-key group min (row 0) and max (row 1)
 *   v_norms  [num_pages][Hkv][page_tokens] fp16  value norms
 *   modality [num_pages][page_tokens] uint8
 * Inside one 4bd-byte group block the codes are laid out for the decode
 * kernel's matrix-core operands ("lane-major"): lane L in [0, 64) owns the
 * W = bd/16 bytes at L*W, read as a little-endian bit stream of operand
 * units of 8 codes (8b bits); code k of unit u starts at bit 8b*u + b*k:
 *   key   (token t in 0..31, channel c): L = ((c % 32) / 8) * 16 + t % 16,
 *         u = (t / 16)*(d/32) + c / 32, k = c % 8
 *   value (token t, channel c):          L = ((t % 16) / 4) * 16 + c % 16,
 *         u = c / 16, k = (t / 16)*4 + t % 4
 * With b = 2 this is byte L*W + (t/16)*(d/16) + (c/32)*2 + (c%8)/4, bits
 * 2*(c%4) for keys and byte L*W + (c/16)*2 + t/16, bits 2*(t%4) for values.
 * 3- and 4-bit codes (Sec. 3 Experiments, ablation over 2 to 4 bits) are
 * decoded by the streaming partition kernel only: G <= 8, page_tokens a
 * power of two and every cache array below 2^31 bytes (KVQ_ERR_UNSUPPORTED
 * otherwise).
 * Slots past the session length hold unspecified codes and are never read
 * as data.  The raw key tail keeps the keys of the open (partial) group:
 *   k_tail   [batch][Hkv][32][d] in kv_dtype, slot = position % 32
 *
 * Sparse page sets (OmniTide page, Sec. 6 OmniPage and Sec. 6.1: pages sized
 * to the attention tile, so that a page emptied by eviction can be skipped
 * whole).  A page-table entry outside
 * [0, num_pages), -1 by convention, marks a logical page that is not
 * retained: the decode reads nothing from it and its positions take no part
 * in the softmax, and an append writes no codes, statistics, norms or
 * modality bytes for positions on it (they are dropped; the session length
 * still advances and the raw key tail is still kept).  Mapping a page again
 * later exposes whatever its physical page holds.  A session with no
 * retained position decodes to zeros.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = 1,      /* null pointer, bad shape, bad codebook, bad index range */
  KVQ_ERR_UNSUPPORTED = 2,  /* d not in {64,128}, G > 16, dtype not supported */
  KVQ_ERR_CAPACITY = 3,     /* append would exceed max_pages * page_tokens */
  KVQ_ERR_WORKSPACE = 4,    /* decode workspace null or too small */
  KVQ_ERR_LAUNCH = 5,       /* a HIP launch failed */
  KVQ_ERR_SCRATCH = 6       /* kvq_decode_attention_noalloc: partials beyond the static scratch */
} kvq_status;

typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1 } kvq_dtype;

/* Key codec of a cache (kvq_config.key_mode).
 *   KVQ_KEYS_GROUP_MINMAX (0): OmniKVQuant's keys (Sec. 2 Method, key
 *     bullet): min-max statistics per 32-token group and channel.
 *   KVQ_KEYS_PER_TOKEN (1): the TurboQuant baseline (Sec. 2 Method,
 *     TurboQuant bullet: magnitude apart, randomized Hadamard, fixed codebook
 *     on the rotated direction): n = ||k||, y = H_d (s_h * k) / sqrt(d),
 *     code = nearest level of sqrt(d) y / n, norm stored as fp16.  The norms
 *     of a group's 32 positions occupy the first 32 fp16 entries of the
 *     group's k_stats block (row 0); the rest of the block is unused.  The
 *     decode reconstructs k_hat = (N / sqrt(d)) c[code].  Supported by the
 *     decode for G <= 8, page_tokens a power of two and a pool whose arrays
 *     stay below 2^31 bytes (KVQ_ERR_UNSUPPORTED otherwise).  With
 *     kvq_params.rot set to the randomized Hadamard for every modality
 *     (R_{h,m} = diag(s_h) H_d / sqrt(d)), the cache is the TurboQuant
 *     baseline run through the same kernels. */
typedef enum { KVQ_KEYS_GROUP_MINMAX = 0, KVQ_KEYS_PER_TOKEN = 1 } kvq_key_mode;

typedef struct kvq_config {
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t n_q_heads;    /* Hq */
  int32_t n_kv_heads;   /* Hkv; Hq % Hkv == 0 and Hq / Hkv <= 16 */
  int32_t batch;        /* sessions B */
  int32_t page_tokens;  /* tokens per page, multiple of 32 */
  int32_t max_pages;    /* page-table row length: capacity = max_pages * page_tokens */
  int32_t num_pages;    /* physical pages in the pool */
  int32_t kv_dtype;     /* kvq_dtype of appended K/V (and of the raw key tail) */
  int32_t key_mode;     /* kvq_key_mode: the key codec of the whole cache */
  int32_t bits;         /* code width b: 2, 3 or 4 bits per element, 2^b codebook levels */
} kvq_config;

typedef struct kvq_cache {
  uint8_t*       k_codes;     /* device */
  uint16_t*      k_stats;     /* device, fp16 bits */
  uint8_t*       v_codes;     /* device */
  uint16_t*      v_norms;     /* device, fp16 bits */
  uint8_t*       modality;    /* device */
  const int32_t* page_table;  /* device [batch][max_pages]: physical page of each logical page,
                                  -1 for a page that is not retained */
  int32_t*       seq_len;     /* device [batch]: cached positions per session */
  void*          k_tail;      /* device [batch][Hkv][32][d] kv_dtype */
  int32_t*       append_tickets; /* device [batch], zero when the cache is created; the
                                    append kernel's completion tickets (back to zero after
                                    every append) */
  int32_t*       seq_len_host;/* host [batch]: mirror of seq_len kept by the library */
} kvq_cache;

typedef struct kvq_params {
  const int8_t* signs;        /* device [Hkv][d], each +1 or -1: Hadamard signs per KV head */
  const float*  rot;          /* device [Hkv][3][d][d] row-major R_{h,m}; columns are the basis */
  float         codebook[16]; /* the first n = 2^bits entries: strictly increasing reconstruction
                                 levels c0 < ... < c_{n-1}; the rest is ignored */
} kvq_params;

/* Bytes of each cache buffer for a configuration, in the order k_codes,
 * k_stats, v_codes, v_norms, modality, k_tail.  Returns KVQ_ERR_INVALID /
 * KVQ_ERR_UNSUPPORTED for a bad configuration. */
kvq_status kvq_cache_buffer_bytes(const kvq_config* cfg, size_t bytes_out[6]);

/*
 * kvq_quantize_append - quantize n_new tokens per session and append them
 * to sessions [b0, b0 + nb) of the packed cache (Sec. 2 Method: key and
 * value bullets).
 *
 * k_new, v_new: device [nb][n_new][Hkv][d] in cfg->kv_dtype.
 * modality_new: device [nb][n_new] uint8 in {0,1,2}.
 * Keys: y = H_d (s_h * k) / sqrt(d) in fp64; the group touched by the append
 * (including the open group, whose earlier keys come from k_tail) is
 * re-quantized with lo/hi = min/max of y over its present tokens, stored as
 * fp16 (round to nearest even); codes map [LO, HI] onto [c0, c3] and take
 * the nearest level.  Values: n = ||v||, z = sqrt(d) (R_{h,m}^T v) / n in
 * fp64, nearest level, norm stored as fp16.  seq_len and seq_len_host
 * advance by n_new (seq_len by the last workgroup to finish, through
 * append_tickets).  One kernel is launched on `stream`; appends to the same
 * cache must not overlap in time.
 * Errors: KVQ_ERR_INVALID (null pointers, b0/nb out of range, n_new < 0,
 * codebook not increasing), KVQ_ERR_CAPACITY (some session would exceed
 * max_pages * page_tokens, judged on seq_len_host), KVQ_ERR_UNSUPPORTED.
 */
kvq_status kvq_quantize_append(const kvq_config* cfg, kvq_cache* cache, const kvq_params* params,
                               int32_t b0, int32_t nb, int32_t n_new,
                               const void* k_new, const void* v_new,
                               const uint8_t* modality_new, hipStream_t stream);

/*
 * kvq_rotate_query - rotate every query head once with its KV head's
 * Hadamard signs (Sec. 1, Implementation bullet):
 * q_rot[b][i] = H_d (s_{floor(i/G)} * q[b][i]) / sqrt(d), computed in fp64
 * and rounded once to fp32.
 * q: device [batch][Hq][d] in q_dtype (KVQ_F32 or KVQ_BF16); q_rot: device
 * [batch][Hq][d] fp32.  Errors: KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED.
 */
kvq_status kvq_rotate_query(const kvq_config* cfg, const kvq_params* params, int32_t batch,
                            const void* q, int32_t q_dtype, float* q_rot, hipStream_t stream);

/*
 * kvq_append_and_rotate - the two independent first steps of a decode step
 * (Sec. 2 Method, key and value bullets; Sec. 1, Implementation bullet) in
 * one launch: exactly kvq_quantize_append(cfg, cache, params, b0, nb, n_new,
 * k_new, v_new, modality_new, stream) followed by kvq_rotate_query(cfg,
 * params, batch, q, q_dtype, q_rot, stream), with identical results.  Extra
 * workgroups of the append's launch rotate the query heads while the append
 * runs, which saves one kernel launch per step.  With n_new == 0 only the
 * rotation is launched.  Arguments, layouts and ownership are those of the
 * two calls; q and q_rot must not overlap the append's inputs or the cache.
 * Errors: those of either call, all checked before anything is launched.
 */
kvq_status kvq_append_and_rotate(const kvq_config* cfg, kvq_cache* cache, const kvq_params* params,
                                 int32_t b0, int32_t nb, int32_t n_new,
                                 const void* k_new, const void* v_new,
                                 const uint8_t* modality_new, int32_t batch,
                                 const void* q, int32_t q_dtype, float* q_rot, hipStream_t stream);

/* Workspace bytes kvq_decode_attention needs when the longest session holds
 * max_len positions (split-K partial results). */
size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t max_len);

/*
 * kvq_decode_attention - one decode step of every query head against the
 * packed cache (Sec. 1, Implementation bullet; Abstract: no dense FP16 cache).
 * For query head i of session b, over positions t < seq_len[b] whose
 * logical page is mapped (see sparse page sets above):
 *   s_t = scale * <q_rot[b][i], k_hat_t>,  k_hat_t = LO + (c[code]-c0)(HI-LO)/(c3-c0)
 *   p = softmax(s);  A_m = sum_{t: modality m} p_t (N_t / sqrt(d)) c[vcode_t]
 *   out[b][i] = sum_m R_{h,m} A_m
 * The context is split into partitions processed in parallel (online
 * softmax per partition); a second kernel merges them and applies R_{h,m}.
 * q_rot: device [batch][Hq][d] fp32 (from kvq_rotate_query).
 * out: device [batch][Hq][d] in out_dtype: KVQ_F32, or KVQ_BF16 (the fp32
 * result rounded to nearest even); a session with no attended position
 * gives zeros.  Pages that are not retained still count towards the plan
 * (their steps are skipped, not compacted away).
 * Plan and replay: the partition plan comes from seq_len_host at the call
 * (up to 128 sessions get partition counts of their own, so a ragged batch
 * ends together; larger batches share one).  The kernels read the lengths
 * from the device seq_len, so a decode
 * captured in a HIP graph and replayed after appends have advanced seq_len
 * on the device stays correct: the last partition of each session takes
 * every position past the plan, up to max_pages * page_tokens (the kernels
 * bound the length there), reading its page-table entries beyond the
 * planned span from global memory.  It only gets slower as the sessions
 * outgrow the captured plan.
 * workspace: device, at least kvq_decode_workspace_bytes(cfg,
 * max(seq_len_host)) bytes, owned by the caller; calls that share a
 * workspace must not overlap in time.
 * Errors: KVQ_ERR_INVALID (null pointers, lengths outside [0, capacity],
 * non-finite scale), KVQ_ERR_WORKSPACE, KVQ_ERR_LAUNCH, KVQ_ERR_UNSUPPORTED
 * (out_dtype not KVQ_F32 / KVQ_BF16; a session longer than 4095 partitions
 * of at most 510 pages each, i.e. 4095 * floor(510 * page_tokens / 256) *
 * 256 positions).
 */
kvq_status kvq_decode_attention(const kvq_config* cfg, const kvq_cache* cache,
                                const kvq_params* params, const float* q_rot, float scale,
                                void* out, int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Workspace bytes kvq_decode_step needs when the longest session holds
 * max_len positions after the step (split-K partial results, one more per
 * query head for the open group). */
size_t kvq_decode_step_workspace_bytes(const kvq_config* cfg, int32_t max_len);

/*
 * kvq_decode_step - one whole decode step of every session (Sec. 2 Method,
 * key and value bullets; Sec. 1, Implementation bullet): append one position
 * to each session of the batch, rotate the queries, and attend every
 * position including the new one.  The result is that of
 *   kvq_append_and_rotate(cfg, cache, params, 0, cfg->batch, 1, k_new, v_new,
 *                         modality_new, cfg->batch, q, q_dtype, q_rot, stream)
 *   kvq_decode_attention(cfg, cache, params, q_rot, scale, out, out_dtype,
 *                        workspace, workspace_bytes, stream)
 * with the same cache bytes, lengths and q_rot, bit for bit, and out equal up
 * to fp32 rounding (the open group is summed in another order).
 * With 2-bit codes, group-statistics keys, a symmetric codebook (c0 = -c3),
 * G <= 8, a power-of-two page_tokens, cache arrays below 2^31 bytes and
 * q_dtype == kv_dtype, the step runs in two launches instead of three: the
 * first runs the decode partitions over each session's closed groups
 * (positions below 32 floor(L / 32), L = the length before the step; the
 * partitions rotate their own query heads) side by side with one workgroup
 * per session and KV head that runs the append and then attends the open
 * group [32 floor(L / 32), L + 1) as one more partial; the second merges
 * the partials and advances the lengths.  Other configurations launch the
 * two calls above.
 * k_new, v_new: device [batch][1][Hkv][d] in cfg->kv_dtype; modality_new:
 * device [batch][1] uint8; q: device [batch][Hq][d] in q_dtype; q_rot:
 * device [batch][Hq][d] fp32 (written); out: device [batch][Hq][d] in
 * out_dtype.  workspace: device, at least
 * kvq_decode_step_workspace_bytes(cfg, max(seq_len_host) + 1), owned by the
 * caller; steps that share a workspace or a cache must not overlap in time.
 * Plan and replay: as for kvq_decode_attention, from max(seq_len_host) + 1;
 * a captured step replayed later appends at, and attends up to, the device
 * lengths of the replay.
 * Errors: those of the two calls (KVQ_ERR_CAPACITY when a session is full),
 * all checked before anything is launched.
 */
kvq_status kvq_decode_step(const kvq_config* cfg, kvq_cache* cache, const kvq_params* params,
                           const void* k_new, const void* v_new, const uint8_t* modality_new,
                           const void* q, int32_t q_dtype, float* q_rot, float scale,
                           void* out, int32_t out_dtype, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * kvq_decode_attention_noalloc - kvq_decode_attention for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus the workspace),
 * same kernels and plan, bitwise the same output.  The split-K partial
 * results go to a device array inside the library,
 * KVQ_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held by each GPU the library
 * runs on until the process ends; the call itself allocates and frees
 * nothing.  Nothing in the array needs to start at zero (every partial a
 * decode reads, it writes first).  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (two streams, two host
 * threads) race and give wrong results; serialise them.  The partials of a
 * decode take Hq * P * (8 + 3 d) * 4 bytes, P the partitions of all
 * sessions together in the plan of seq_len_host (about 256 / Hkv: one
 * workgroup per compute unit); larger requests return
 * KVQ_ERR_SCRATCH before anything is launched.  Errors: those of
 * kvq_decode_attention except KVQ_ERR_WORKSPACE, plus KVQ_ERR_SCRATCH;
 * KVQ_ERR_LAUNCH also when the scratch address cannot be obtained.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_config* cfg, const kvq_cache* cache,
                                        const kvq_params* params, const float* q_rot, float scale,
                                        void* out, int32_t out_dtype, hipStream_t stream);

/*
 * kvq_probe_stream_read - measurement aid, not part of the method: one
 * launch that reads `bytes` of device memory at `buf` once (16-byte loads,
 * `workgroups` workgroups of 256 threads, grid-stride) and XORs one word per
 * workgroup into sink[0 .. workgroups).  Timing it over buffers the size of
 * a decode's algorithmic bytes gives the floor for one read-only kernel of
 * that size on this GPU.  buf: device, 16-byte aligned, bytes a positive
 * multiple of 16; sink: device, workgroups words.  Errors: KVQ_ERR_INVALID,
 * KVQ_ERR_LAUNCH.
 */
kvq_status kvq_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups,
                                 hipStream_t stream);

/* Static description of a status code. */
const char* kvq_status_string(kvq_status status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
