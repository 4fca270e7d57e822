/*
 * h3oracle.h -- plain CPU oracle for the fused per-token DiT operators.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may call anything declared here.  The
 * GPU library never includes, links or calls this code, and this code never
 * includes or calls the GPU library: the two share nothing but the seeded
 * input generator, which lives in its own module and holds none of the
 * operators' arithmetic.
 *
 * What is computed, and where it comes from:
 *   The pages that describe the path (the LMSYS MiniMax-H3 performance report
 *   as summarised on news.cocoloop.cn, section "Só com três camadas…", and
 *   the ceviu.com.br newsletter "SGLang acelera MiniMax-H3 em GPUs H200…")
 *   name the fused operators -- AdaLN modulate, gated residual, SwiGLU and
 *   QK RMSNorm with 3D RoPE -- and state that fusing them changes no result.
 *   They print no formula.  Each function below therefore evaluates the
 *   standard published definition of its operator, cited at the function:
 *     LayerNorm        Ba, Kiros & Hinton (2016), "Layer Normalization", eq. 4
 *     AdaLN modulate   Peebles & Xie (2023), "Scalable Diffusion Models with
 *                      Transformers", adaLN(-Zero) block: LN(x)(1+scale)+shift,
 *                      and the gate alpha applied before the residual add
 *     SwiGLU           Shazeer (2020), "GLU Variants Improve Transformer":
 *                      Swish_1(xW) * (xV), Swish_1(z) = z * sigmoid(z)
 *     RMSNorm          Zhang & Sennrich (2019), "Root Mean Square Layer
 *                      Normalization", eq. 4 (no bias)
 *     RoPE             Su et al. (2021), "RoFormer", eq. 34 (the sparse form
 *                      of the rotation: interleaved pairs, theta_i =
 *                      base^(-2(i-1)/d))
 *   applied per axis of a (t, h, w) grid split of the head dimension.
 *
 * Arithmetic: every input element is read exactly (bf16 -> fp32 by a 16-bit
 * shift -> double), every operation is carried out in double, and each
 * output element is rounded once to its storage type (double -> fp32 with the
 * C cast, round-to-nearest-even; fp32 -> bf16 round-to-nearest-even).
 *
 * Layout: all arrays are dense row-major.  "rows" is the token count of the
 * slice handed over; group / position arrays make sampled (non-contiguous)
 * rows of a larger workload expressible without strides.
 */
#ifndef H3ORACLE_H
#define H3ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage types understood by the oracle */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* RoPE pair layouts inside one axis chunk */
enum { ORACLE_PAIR_INTERLEAVED = 0, ORACLE_PAIR_HALF_SPLIT = 1 };

int oracle_abi_version(void);

/* Number of OpenMP threads the row loops use (for the CPU baseline report). */
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

/* --- scalar conversions, exposed so the tests can pin them ------------- */
float    oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f32_to_bf16(float f);

/* --- token positions ---------------------------------------------------
 * Row r of the slice is global token p = (token_offset + r) mod L with
 * L = T*H*W + n_audio.  Video tokens come first in raster order (t slowest,
 * w fastest); audio token k = p - T*H*W follows and sits at (t=k, h=0, w=0).
 * pos is [rows, 3] int32 (t, h, w).
 */
void oracle_positions(int32_t* pos, int64_t rows, int64_t token_offset,
                      int32_t T, int32_t H, int32_t W, int32_t n_audio);

/* --- AdaLN modulate -------------------------------------------------------
 * y[r,:] = (x[r,:] - mean) / sqrt(var + eps) * (1 + scale[g,:]) + shift[g,:]
 * mean, var over the hidden dimension (biased variance, two-pass).
 * g = group[r] if group != NULL, else r / rows_per_group.
 * shift/scale are [groups, hidden] of type mod_dtype.
 */
void oracle_adaln_modulate(void* y, int y_dtype, const void* x, int x_dtype,
                           const void* shift, const void* scale, int mod_dtype,
                           const int64_t* group, int64_t rows_per_group,
                           int64_t rows, int64_t hidden, float eps);

/* --- AdaLN modulate over a LayerNorm with affine parameters ------------------
 * y[r,:] = (gamma * (x[r,:] - mean) / sqrt(var + eps) + beta) * (1 + scale[g,:])
 *          + shift[g,:]
 * gamma, beta: [hidden] of mod_dtype, shared by all rows; the rest as above. */
void oracle_adaln_affine_modulate(void* y, int y_dtype, const void* x, int x_dtype,
                                  const void* gamma, const void* beta,
                                  const void* shift, const void* scale, int mod_dtype,
                                  const int64_t* group, int64_t rows_per_group,
                                  int64_t rows, int64_t hidden, float eps);

/* --- gated residual ---------------------------------------------------------
 * x[r,:] = x[r,:] + gate[g,:] * h[r,:]   (in place; gate has x's type) */
void oracle_gated_residual(void* x, int x_dtype, const void* h, int h_dtype,
                           const void* gate, const int64_t* group,
                           int64_t rows_per_group, int64_t rows, int64_t hidden);

/* --- SwiGLU -------------------------------------------------------------------
 * out[r,j] = a[r,j] * sigmoid(a[r,j]) * b[r,j]
 * gate_up is [rows, 2*inner]: a = columns [0, inner), b = [inner, 2*inner). */
void oracle_swiglu(void* out, const void* gate_up, int dtype,
                   int64_t rows, int64_t inner);

/* --- RoPE frequency table ---------------------------------------------------
 * inv_freq[p] for the head_dim/2 rotation pairs, in head-dimension order of
 * the chunks [t | h | w]; pair j of chunk c (size d_c) gets
 * theta^(-2j/d_c), evaluated in double and rounded once to fp32. */
void oracle_rope_inv_freq(float* inv_freq, int32_t d_t, int32_t d_h,
                          int32_t d_w, double theta);

/* --- per-head QK RMSNorm + 3D RoPE ------------------------------------------
 * For each row r, tensor (q then k) and head i, with v = the head's head_dim
 * values:  u = v / sqrt(mean(v^2) + eps) * w   (w = q_weight or k_weight),
 * then every rotation pair (e0, e1) of axis chunk c is rotated by
 *   phi = pos[r, c] * inv_freq[pair]:
 *   (u0, u1) -> (u0 cos phi - u1 sin phi, u0 sin phi + u1 cos phi).
 * angle_mode 0: phi = fl32(fl32(pos) * inv_freq_f32) then cos/sin in double.
 * angle_mode 1: phi in double from the exact frequency (for comparison).
 * pairing: ORACLE_PAIR_INTERLEAVED -> pairs (2j, 2j+1) of the chunk;
 *          ORACLE_PAIR_HALF_SPLIT  -> pairs (j, j + d_c/2) of the chunk.
 * q, k, q_out, k_out are [rows, heads, head_dim]; weights [head_dim];
 * pos is [rows, 3]. */
void oracle_qk_rmsnorm_rope3d(void* q_out, void* k_out, const void* q,
                              const void* k, const void* q_weight,
                              const void* k_weight, int dtype, int64_t rows,
                              int32_t heads, int32_t head_dim, float eps,
                              const int32_t* pos, int32_t d_t, int32_t d_h,
                              int32_t d_w, double theta, int angle_mode,
                              int pairing);

/* --- fused gated residual + AdaLN modulate ------------------------------------
 * The composition of the two operators as a block runs them back to back:
 * x <- x + gate*h (rounded to x's type), then y = AdaLN(x; shift, scale). */
void oracle_gated_residual_adaln(void* x, int x_dtype, const void* h,
                                 int h_dtype, const void* gate, void* y,
                                 int y_dtype, const void* shift,
                                 const void* scale, const int64_t* group,
                                 int64_t rows_per_group, int64_t rows,
                                 int64_t hidden, float eps);

/* --- residual-difference statistics for step reuse -----------------------------
 * Returns, in out[0..1], sum |cur - prev| and sum |prev| over the whole
 * [rows, hidden] tensor, both in double; the relative L1 difference is
 * out[0] / out[1]. */
void oracle_residual_l1(double* out, const void* cur, const void* prev,
                        int dtype, int64_t rows, int64_t hidden);

/* --- block-sparse attention router (SubBlock) ----------------------------------
 * Token block b holds rows [b*block, min(rows, (b+1)*block)); the last block
 * may be short.  x is [rows, heads, head_dim].
 * pooled[h, b, d] = mean over the rows of block b of x[r, h, d] (double). */
void oracle_subblock_pool(double* pooled, const void* x, int dtype,
                          int64_t rows, int32_t heads, int32_t head_dim,
                          int32_t block);

/* scores[h, i, j] = sum_d pq[h, i, d] * pk[h, j, d]: the mean of q_a . k_b over
 * every token pair (a in query block i, b in key block j).
 * pq is [heads, nbq, head_dim], pk [heads, nbk, head_dim]. */
void oracle_subblock_scores(double* scores, const double* pq, const double* pk,
                            int32_t heads, int64_t nbq, int64_t nbk,
                            int32_t head_dim);

/* Key blocks kept per query block at denoising step `step` (1-based): all of
 * them before step first_step, else nb - floor(sparsity * nb) (sparsity is the
 * skipped fraction; the product is one double multiply). */
int64_t oracle_subblock_keep(int64_t nb, double sparsity, int32_t step,
                             int32_t first_step);

/* kv[h, i, 0:keep] = the keep key blocks with the largest scores[h, i, :]
 * (equal scores: lower block index first), listed in ascending block order. */
void oracle_subblock_select(int32_t* kv, const double* scores, int32_t heads,
                            int64_t nbq, int64_t nbk, int64_t keep);

#ifdef __cplusplus
}
#endif
#endif
