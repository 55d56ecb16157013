/*
 * tlglayer — the two operations that complete a GPT-2 block around its
 * linear layers, on one MI355X (gfx950).  They live in libtlgemm.so beside
 * the GEMM entry points of tlgemm.h and share its conventions: raw device
 * pointers owned by the caller, a hipStream_t passed as void* (NULL: the
 * default stream), enqueue-and-return, TLG_ERR_* status codes with the
 * message from gemm_last_error(), no allocation, no exception.
 *
 * Element types are tlg_dtype (tlgemm.h): inputs and outputs of one call
 * share the type; arithmetic and the saved statistics are fp32.
 */
#ifndef TLGLAYER_H
#define TLGLAYER_H

#include <stddef.h>
#include <stdint.h>

#include "tlgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * tlg_layernorm — Y[r][c] = (X[r][c] - mean_r) * rstd_r * gamma[c] + beta[c]
 * over each row r of X [rows][C], with mean_r the row mean, var_r the biased
 * row variance and rstd_r = 1/sqrt(var_r + eps).
 *
 * The layer normalisation of "mage-003: What the kernels were short of"
 * (layer-normalisation section), whose statistics come from a single read of
 * the row held in registers; here a wave holds two whole rows, so that
 * each lane has all of their loads in flight at once.
 *
 * X, Y: [rows][C] row-major; gamma, beta: [C]; all of type dt.  mean and
 * rstd: [rows] fp32, each may be NULL (not written).  Y, mean and rstd must
 * not overlap each other, X, gamma or beta.  Requires rows >= 1, 1 <= C <= 4096, eps >= 0, every pointer
 * aligned to its element size (TLG_ERR_MISALIGNED otherwise); C > 4096 is
 * TLG_ERR_UNSUPPORTED.
 */
int tlg_layernorm(const void* X, const void* gamma, const void* beta, void* Y, float* mean, float* rstd,
                  int64_t rows, int64_t C, float eps, tlg_dtype dt, void* stream);

/*
 * tlg_attention — scaled dot-product attention of each head over the output
 * of a GPT-2 qkv projection, fused: the score matrix is never written.
 *
 * "Writing a CUDA matmul that catches cuBLAS", section "Fusing attention:
 * the score matrix never exists": an online softmax (running maximum and sum,
 * earlier partial results rescaled when the maximum rises), causality as a
 * loop bound, and q, k, v read in place from the (B, T, 3C) projection.
 *
 * qkv: [B][T][3C] with C = n_head * head_size; the query of head h at
 * position t is qkv[b][t][h*head_size .. +head_size), its key C further on
 * and its value 2C further on.  out: [B][T][C], out[b][i][h*head_size + d] =
 * sum_j p_ij v_j[d] with p_ij = softmax_j(q_i . k_j / sqrt(head_size)) over
 * j <= i (causal != 0) or all j.  lse: [B][n_head][T] fp32, the log-sum-exp
 * of each row of scores (what a backward pass rebuilds the probabilities
 * from), or NULL.  out and lse must not overlap qkv or each other.
 *
 * Requires B, T, n_head >= 1, head_size == 64, T <= 256 (keys and values of
 * one head stay in LDS), B * n_head < 2^31, qkv and out 16-byte aligned
 * (TLG_ERR_MISALIGNED otherwise); other sizes are TLG_ERR_UNSUPPORTED.
 */
int tlg_attention(const void* qkv, void* out, float* lse, int64_t B, int64_t T, int64_t n_head, int64_t head_size,
                  tlg_dtype dt, int causal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TLGLAYER_H */
