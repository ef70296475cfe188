/*
 * kvq_calib.h - C ABI of the value-basis calibration in libkvq (MI355X,
 * gfx950): the per-modality value rotations R_{h,m} that kvq_params.rot
 * holds, derived from calibration data.
 *
 * Method (OmniKVQuant page, paperlayer.ai summary of arXiv 2609.11582,
 * Sec. 2 Method, second "OmniKVQuant" bullet): value directions are weighted
 * by their contribution to attention outputs, a covariance matrix is formed
 * separately for each modality, and its eigenbasis becomes that modality's
 * rotation.  The page fixes no formula; this library reads it as:
 *   - contribution of calibration token t of KV head h:
 *       w[h][t] = (1 / (nq G)) sum_{query i, head g of the group}
 *                 softmax_t(scale * <q[i][hG + g], k[t][h]>)
 *     (softmax over the n calibration tokens, full-precision keys);
 *   - covariance of modality m: C = sum_t w_t (v_t - mu)(v_t - mu)^T / W over
 *     the tokens of modality m, W = sum_t w_t, mu = sum_t w_t v_t / W; C = 0
 *     and mu = 0 when W == 0; tokens whose modality byte is not 0, 1 or 2
 *     take no part;
 *   - eigenbasis: the columns of R are unit eigenvectors of C in decreasing
 *     eigenvalue order, each with its largest-magnitude component (the
 *     first one on a tie) positive.
 *
 * All arithmetic is fp64; inputs are read exactly (bf16 / fp32 -> fp64).
 * The three steps are separate calls so that each can be checked on its
 * own; run in order on one stream they give the whole calibration.
 * Conventions are those of kvq.h: caller-owned device buffers, asynchronous
 * calls on the given stream, host-side validation before any launch, a
 * status code per call, nothing allocated by the library.  The results do
 * not depend on the launch configuration (fixed summation orders).
 */
#ifndef KVQ_CALIB_H
#define KVQ_CALIB_H

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvq_calib_shape {
  int32_t head_dim;    /* d: 64 or 128 */
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv; Hq % Hkv == 0 */
  int32_t n_tokens;    /* n >= 0 calibration tokens */
  int32_t n_queries;   /* nq >= 1 calibration queries per query head */
} kvq_calib_shape;

/* Workspace bytes that cover kvq_calib_contribution, kvq_calib_covariance
 * and kvq_calib_eigenbasis with count = 3 * Hkv for this shape (0 for an
 * invalid shape). */
size_t kvq_calib_workspace_bytes(const kvq_calib_shape* shape);

/* Workspace bytes of kvq_calib_eigenbasis for `count` matrices of size d. */
size_t kvq_calib_eigenbasis_workspace_bytes(int32_t count, int32_t head_dim);

/*
 * kvq_calib_contribution - attention-contribution weight of every
 * calibration token (Sec. 2 Method, value bullet: directions weighted by
 * their contribution to attention outputs).
 * k: device [n][Hkv][d] in k_dtype; q: device [nq][Hq][d] in q_dtype;
 * scale > 0 (e.g. 1 / sqrt(d)); weights: device [Hkv][n] fp64 output, each
 * KV head's weights summing to one (n > 0).  Query head i belongs to KV head
 * floor(i / G).
 * Errors: KVQ_ERR_INVALID (null pointer, bad shape, scale not positive and
 * finite), KVQ_ERR_UNSUPPORTED (d, dtype), KVQ_ERR_WORKSPACE, KVQ_ERR_LAUNCH.
 */
kvq_status kvq_calib_contribution(const kvq_calib_shape* shape, const void* k, int32_t k_dtype,
                                  const void* q, int32_t q_dtype, double scale, double* weights,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kvq_calib_covariance - the weighted covariance of each (KV head,
 * modality) (Sec. 2 Method, value bullet: a covariance computed separately
 * per modality).
 * v: device [n][Hkv][d] in v_dtype, 16-byte aligned; modality: device [n] uint8; weights:
 * device [Hkv][n] fp64 (e.g. from kvq_calib_contribution); cov: device
 * [Hkv][3][d][d] fp64 output, exactly symmetric; weight_sum: device [Hkv][3]
 * fp64 output (W per modality).
 * Errors: KVQ_ERR_INVALID (null pointer, bad shape, v not 16-byte aligned),
 * KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_LAUNCH.
 */
kvq_status kvq_calib_covariance(const kvq_calib_shape* shape, const void* v, int32_t v_dtype,
                                const uint8_t* modality, const double* weights, double* cov,
                                double* weight_sum, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * kvq_calib_eigenbasis - eigenbasis of `count` symmetric d x d matrices
 * (Sec. 2 Method, value bullet: a modality-specific eigenbasis), by cyclic
 * Jacobi rotations in fp64 (one workgroup per matrix rotates it, at most 50
 * sweeps, logging each round's rotations in the workspace; then d / 8
 * workgroups per matrix accumulate the eigenvectors from the log, one block
 * of columns each; three launches on `stream`).
 * cov: device [count][d][d] fp64, symmetric (only entries i <= j are read);
 * rot: device [count][d][d] fp32 output, rot[i][j] = component i of
 * eigenvector j (the kvq_params.rot layout when count = 3 * Hkv and cov
 * comes from kvq_calib_covariance); eigenvalues: device [count][d] fp64
 * output, decreasing.  A zero matrix gives the identity.  workspace: device,
 * 16-byte aligned, kvq_calib_eigenbasis_workspace_bytes(count, d) bytes.
 * Errors: KVQ_ERR_INVALID (count < 0, null pointer, workspace not 16-byte
 * aligned), KVQ_ERR_UNSUPPORTED (d), KVQ_ERR_WORKSPACE, KVQ_ERR_LAUNCH.
 */
kvq_status kvq_calib_eigenbasis(int32_t count, int32_t head_dim, const double* cov, float* rot,
                                double* eigenvalues, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_CALIB_H */
