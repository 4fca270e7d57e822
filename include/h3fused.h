/*
 * h3fused.h -- C ABI of libh3fused: fused, memory-bound per-token operators of
 * a single-stream audio+video diffusion transformer (MiniMax-H3 style DiT), and
 * the block router of its block-sparse attention, implemented as hand-written
 * HIP kernels for gfx950 (MI355X, CDNA4).
 *
 * Sources.  The operators are the ones the LMSYS performance report on
 * MiniMax-H3 with SGLang Diffusion names as fused kernels (summary page on
 * news.cocoloop.cn, "minimax-h3-sglang-h200", section "Só com três
 * camadas…": AdaLN update, gated residual, SwiGLU, QK RMSNorm with 3D RoPE,
 * fused to cut round trips through GPU memory without changing any result),
 * also listed by the ceviu.com.br newsletter "SGLang acelera MiniMax-H3 em
 * GPUs H200…".  The model facts (one dense single-stream transformer over a
 * joint video+audio token sequence; a VisualVAE with 16x spatial / 4x temporal
 * compression; an AdaLN branch whose outputs are token independent and can be
 * precomputed) come from the studioglobal.ai explainer "MiniMax H3 mở trọng
 * số…", section "Kiến trúc…", and the arex-research.com article on H3 and
 * TPUs, section "H3 的开源底子".  The pages print no formula; each entry point
 * states the standard definition it computes.
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers (hipMalloc / torch CUDA tensors) unless a
 *     parameter says otherwise.  The caller owns all memory; the library
 *     keeps no pointer after a call returns and allocates nothing.
 *   - Tensors are row-major with unit inner stride; every *_row_stride /
 *     *_head_stride / *_group_stride is in ELEMENTS of that tensor's type.
 *   - Vector width: 4 elements when any tensor of the call is fp32, 8 elements
 *     when all are bf16.  hidden / inner / head_dim and every stride must be
 *     multiples of it, and every pointer must be 16-byte aligned.
 *   - Arithmetic is fp32 whatever the storage type; each output element is
 *     rounded once (round to nearest even) to its storage type.
 *   - Modulation vectors (shift, scale, gate) are [groups, hidden] rows: token
 *     row r uses group g = r / rows_per_group (rows_per_group = rows gives one
 *     vector for the whole call; 1 gives per-token modulation).
 *   - For the per-token operators rows == 0 is a no-op that returns H3F_OK
 *     before any other check.  The residual difference and the router reject
 *     it (they have no result for an empty tensor; see there).
 *   - Validation is synchronous and happens before any launch; a bad argument
 *     returns an error code and launches nothing.  No call aborts or throws.
 *   - Aliasing: an output may be exactly the same tensor as an input (same
 *     pointer, same strides, same type); any other overlap between an output
 *     and another tensor of the call is H3F_ERR_ALIASING.  Tensors that are
 *     interleaved with the same row stride (q, k, v of one packed qkv buffer)
 *     do not overlap and are accepted.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream).  A fault inside a kernel surfaces at the caller's next
 *     synchronisation.  Launch failures return H3F_ERR_LAUNCH.
 *   - Every entry point is reentrant and keeps no state between calls, except
 *     h3f_residual_l1_noalloc, whose partial sums live in a device array the
 *     library owns (see there: calls that overlap on one GPU race).
 */
#ifndef H3FUSED_H
#define H3FUSED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3F_ABI_VERSION 1

typedef enum { H3F_F32 = 0, H3F_BF16 = 1 } h3f_dtype_t;

typedef enum {
    H3F_OK = 0,
    H3F_ERR_NULL_POINTER = 1,
    H3F_ERR_BAD_SHAPE = 2,
    H3F_ERR_BAD_STRIDE = 3,
    H3F_ERR_MISALIGNED = 4,
    H3F_ERR_BAD_DTYPE = 5,
    H3F_ERR_ALIASING = 6,
    H3F_ERR_LAUNCH = 7,
    H3F_ERR_UNSUPPORTED = 8,
    H3F_ERR_WORKSPACE = 9,
    H3F_ERR_BAD_VALUE = 10
} h3f_status_t;

/* RoPE pair layouts inside one axis chunk of size d_c */
typedef enum {
    H3F_ROPE_INTERLEAVED = 0, /* pairs (2j, 2j+1)      (RoFormer, eq. 34)          */
    H3F_ROPE_HALF_SPLIT = 1   /* pairs (j, j + d_c/2)  (rotate-half layout)        */
} h3f_rope_pairing_t;

/*
 * Token grid and RoPE parameters of one joint video+audio sequence.
 *   The sequence holds T*H*W video tokens in raster order (t slowest, w
 *   fastest) followed by n_audio audio tokens; audio token k sits at
 *   (t = k, h = 0, w = 0).  Row r of a call is global token
 *   p = (token_offset + r) mod (T*H*W + n_audio), so a batch of B sequences
 *   stacked along rows, or a shard of a sequence, is described by the same
 *   struct.  (The pages fix the VAE factors that set T, H, W -- studioglobal.ai
 *   explainer, section "Kiến trúc…" -- but neither the token order nor the
 *   audio positions; these are readings.)
 *   The head dimension is split into axis chunks [t | h | w] of sizes d_t, d_h,
 *   d_w (d_t + d_h + d_w == head_dim, each a positive multiple of the vector
 *   width, each a multiple of 16 for H3F_ROPE_HALF_SPLIT).  Pair j of chunk c
 *   rotates by phi = fl32(fl32(pos_c) * fl32(theta^(-2j/d_c))).
 *   positions: optional device int32 [rows, 3] array of (t, h, w) that, when
 *   not NULL, replaces the grid derivation (T, H, W, n_audio, token_offset are
 *   then ignored).
 */
typedef struct {
    int32_t T, H, W, n_audio;
    int32_t d_t, d_h, d_w;
    int32_t pairing; /* h3f_rope_pairing_t */
    double theta;    /* RoPE base, 10000 in RoFormer */
    int64_t token_offset;
    const int32_t* positions;
} h3f_rope3d_t;

/* Library ABI version (H3F_ABI_VERSION of the build). */
int h3f_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* h3f_status_string(h3f_status_t status);

/*
 * Token positions: writes pos[r] = (t, h, w) of row r as described for
 * h3f_rope3d_t (positions member ignored).  pos: device int32 [rows, 3],
 * 4-byte aligned.  Integer work, bit-exact.
 * Errors: NULL pos or grid; T, H, W < 1 or n_audio < 0 (BAD_SHAPE).
 */
h3f_status_t h3f_rope3d_positions(int32_t* pos, int64_t rows, const h3f_rope3d_t* grid,
                                  void* stream);

/*
 * AdaLN modulate (fused LayerNorm + modulation; the report's "AdaLN update").
 *   y[r,:] = (x[r,:] - mean_r) / sqrt(var_r + eps) * (1 + scale[g,:]) + shift[g,:]
 * mean and (biased) var over the hidden dimension; LayerNorm has no affine of
 * its own (DiT adaLN: Peebles & Xie 2023).
 *   y: [rows, hidden] of y_dtype, row stride y_row_stride.
 *   x: [rows, hidden] of x_dtype, row stride x_row_stride.
 *   shift, scale: [groups, hidden] of x_dtype, group stride mod_group_stride.
 * Supported (x, y) types: (f32, f32), (bf16, bf16), (f32, bf16).
 * hidden <= 16384 (bf16 x) or 8192 (f32 x); else H3F_ERR_UNSUPPORTED.
 * y may be x itself (same pointer, stride and type).
 */
h3f_status_t h3f_adaln_modulate(void* y, h3f_dtype_t y_dtype, int64_t y_row_stride,
                                const void* x, h3f_dtype_t x_dtype, int64_t x_row_stride,
                                const void* shift, const void* scale, int64_t mod_group_stride,
                                int64_t rows_per_group, int64_t rows, int64_t hidden, float eps,
                                void* stream);

/*
 * AdaLN modulate over a LayerNorm that keeps its own affine gain and bias
 * (Ba, Kiros & Hinton 2016, eq. 4), for models whose LayerNorm is not
 * affine-free:
 *   y[r,:] = (gamma * (x[r,:] - mean_r) / sqrt(var_r + eps) + beta)
 *            * (1 + scale[g,:]) + shift[g,:]
 * gamma, beta: [hidden] of x_dtype, 16-byte aligned, shared by every row and
 * group; they must not overlap y.  Everything else as h3f_adaln_modulate.
 */
h3f_status_t h3f_adaln_affine_modulate(void* y, h3f_dtype_t y_dtype, int64_t y_row_stride,
                                       const void* x, h3f_dtype_t x_dtype, int64_t x_row_stride,
                                       const void* gamma, const void* beta, const void* shift,
                                       const void* scale, int64_t mod_group_stride,
                                       int64_t rows_per_group, int64_t rows, int64_t hidden,
                                       float eps, void* stream);

/*
 * Gated residual (the report's "residual com gate"), in place:
 *   x[r,:] = x[r,:] + gate[g,:] * h[r,:]
 *   x: [rows, hidden] of x_dtype (read and written); h: [rows, hidden] of
 *   h_dtype; gate: [groups, hidden] of x_dtype.
 * Supported (x, h) types: (f32, f32), (bf16, bf16), (f32, bf16).
 * h must not overlap x.
 */
h3f_status_t h3f_gated_residual(void* x, h3f_dtype_t x_dtype, int64_t x_row_stride,
                                const void* h, h3f_dtype_t h_dtype, int64_t h_row_stride,
                                const void* gate, int64_t gate_group_stride,
                                int64_t rows_per_group, int64_t rows, int64_t hidden,
                                void* stream);

/*
 * SwiGLU (Shazeer 2020): out[r,j] = a[r,j] * sigmoid(a[r,j]) * b[r,j].
 *   out, a, b: [rows, inner] of dtype, each with its own row stride.  For the
 *   usual packed gate/up projection output gu [rows, 2*inner] pass
 *   a = gu, b = gu + inner, a_row_stride = b_row_stride = 2*inner.
 * out may be a or b itself (same pointer and stride).
 */
h3f_status_t h3f_swiglu(void* out, int64_t out_row_stride, const void* a, int64_t a_row_stride,
                        const void* b, int64_t b_row_stride, h3f_dtype_t dtype, int64_t rows,
                        int64_t inner, void* stream);

/*
 * Per-head QK RMSNorm + 3D RoPE (the report's "QK RMSNorm com 3D RoPE").
 * For every row r, head i and tensor (q, k), with v the head's head_dim values:
 *   u = v / sqrt(mean(v^2) + eps) * w        (RMSNorm, Zhang & Sennrich 2019;
 *                                             w = q_weight or k_weight [head_dim])
 *   each rotation pair (u0, u1) of axis chunk c at position pos_c(r):
 *   (u0, u1) <- (u0 cos phi - u1 sin phi, u0 sin phi + u1 cos phi)
 * Element (r, i, d) of q is at q + r*q_row_stride + i*q_head_stride + d, and
 * likewise for k, q_out, k_out (a packed qkv [rows, 3, heads, head_dim]
 * buffer gives q_row_stride = 3*heads*head_dim, k = q + heads*head_dim).
 * q_out / k_out may be q / k themselves (same pointer and strides).
 * head_dim / vector width must be a power of two <= 64 (head_dim <= 512 for
 * bf16, <= 256 for f32); head strides >= head_dim.
 */
h3f_status_t h3f_qk_rmsnorm_rope3d(void* q_out, int64_t q_out_row_stride,
                                   int64_t q_out_head_stride, void* k_out,
                                   int64_t k_out_row_stride, int64_t k_out_head_stride,
                                   const void* q, int64_t q_row_stride, int64_t q_head_stride,
                                   const void* k, int64_t k_row_stride, int64_t k_head_stride,
                                   const void* q_weight, const void* k_weight,
                                   h3f_dtype_t dtype, int64_t rows, int32_t heads,
                                   int32_t head_dim, float eps, const h3f_rope3d_t* rope,
                                   void* stream);

/*
 * Gated residual followed by AdaLN modulate on the updated stream, in one
 * pass over x (the two operators the report lists together, composed in the
 * order a DiT block runs them):
 *   x[r,:] = x[r,:] + gate[g,:] * h[r,:]            (stored rounded to x_dtype)
 *   y[r,:] = AdaLN(x[r,:]; shift[g,:], scale[g,:])  (computed from the stored x)
 * Same types, limits and rules as h3f_gated_residual and h3f_adaln_modulate;
 * gate, shift and scale share mod_group_stride; y must not overlap x or h.
 */
h3f_status_t h3f_gated_residual_adaln(void* x, h3f_dtype_t x_dtype, int64_t x_row_stride,
                                      const void* h, h3f_dtype_t h_dtype, int64_t h_row_stride,
                                      const void* gate, const void* shift, const void* scale,
                                      int64_t mod_group_stride, int64_t rows_per_group,
                                      void* y, h3f_dtype_t y_dtype, int64_t y_row_stride,
                                      int64_t rows, int64_t hidden, float eps, void* stream);

/*
 * Residual difference between neighbouring denoising steps, the reuse test of
 * step caching (the report page's Cache-DiT paragraph, section "Só com três
 * camadas…": reuse when a residual difference is under a threshold such as
 * 0.04 or 0.08; the page gives no formula -- the relative L1 distance is the
 * reading used here):
 *   out[0] = sum |cur - prev|,  out[1] = sum |prev|,  out[2] = out[0] / out[1]
 * over all [rows, hidden] elements.  out: device double[3].  cur, prev:
 * [rows, hidden] of dtype with their own row strides.  Deterministic: fixed
 * partition, fp32 sums inside a workgroup, fp64 across workgroups in index
 * order (bit-identical run to run).  workspace: device scratch of at least
 * h3f_residual_l1_workspace_bytes(rows, hidden, dtype) bytes, 16-byte aligned,
 * owned by the caller, contents need no initialisation; calls that share a
 * workspace must be ordered on one stream.  Unlike the operators, rows == 0
 * is rejected (H3F_ERR_BAD_SHAPE): an empty tensor has no relative
 * difference.  If sum |prev| is 0, out[2] is inf or NaN (IEEE division).
 * Returns 0 from the size query for an invalid or unsupported shape or type.
 */
size_t h3f_residual_l1_workspace_bytes(int64_t rows, int64_t hidden, h3f_dtype_t dtype);
h3f_status_t h3f_residual_l1(double* out, const void* cur, int64_t cur_row_stride,
                             const void* prev, int64_t prev_row_stride, h3f_dtype_t dtype,
                             int64_t rows, int64_t hidden, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * h3f_residual_l1 for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and result, bit for bit, with the per-workgroup partial sums kept in
 * a device array the library owns instead of a caller workspace.  The call
 * itself allocates nothing and frees nothing.
 *   Limit: the array holds h3f_residual_l1_noalloc_max_bytes() bytes (4 MiB);
 *   a call whose h3f_residual_l1_workspace_bytes(rows, hidden, dtype) is larger
 *   is rejected with H3F_ERR_WORKSPACE (bf16 at hidden 5120: up to 838,860
 *   rows).  Each GPU the library runs on holds its own copy of the array until
 *   the process ends; its address is looked up once per device, on the first
 *   call with that device current (H3F_ERR_LAUNCH if the lookup fails) -- a
 *   caller that captures the call in a graph makes one call before capturing.
 *   Sharing: every call on one GPU uses that GPU's array, which keeps the last
 *   call's partial sums (each call writes all the sums it reads, so no clearing
 *   is needed).  Calls that may run concurrently on one GPU (other streams,
 *   other host threads without ordering) race on the array and must not
 *   overlap; calls ordered on one stream are safe.
 * Arguments, result and other errors as h3f_residual_l1.
 */
size_t h3f_residual_l1_noalloc_max_bytes(void);
h3f_status_t h3f_residual_l1_noalloc(double* out, const void* cur, int64_t cur_row_stride,
                                     const void* prev, int64_t prev_row_stride,
                                     h3f_dtype_t dtype, int64_t rows, int64_t hidden,
                                     void* stream);

/*
 * Block-sparse attention router (SubBlock).  The report page (section "Só com
 * três camadas…", SubBlock paragraph) describes a block router that, from the
 * tenth denoising step on, cuts the key/value blocks each attention
 * computation uses, at sparsity 0.75 or 0.80; the newsletter page says the
 * blocks skipped are the least important ones; the report page's section
 * "Alguns limites…" restricts it to long non-causal attention in BF16 with
 * head dimension 128 and at least 4096 tokens.  Block size, pooling and score
 * are not given.  Reading implemented here, per head h:
 *   - token block b = rows [b*block, min(rows, (b+1)*block)), the last one
 *     possibly short; n_blocks = ceil(rows / block) for queries and keys;
 *   - qm[h,b,:], km[h,b,:] = mean over the block's tokens (fp32);
 *   - scores[h,i,j] = qm[h,i,:] . km[h,j,:], the mean attention logit q.k of
 *     all token pairs of query block i and key block j (the softmax scale
 *     1/sqrt(head_dim) is a positive constant and does not change the order);
 *   - kv_blocks[h,i,0:keep] = the keep key blocks with the largest scores
 *     (equal scores: lower block index first), in ascending block order;
 *   - keep = n_blocks - floor(sparsity * n_blocks) (one double multiply; the
 *     skipped fraction is sparsity) at step >= H3F_SUBBLOCK_FIRST_STEP, and
 *     keep = n_blocks (every block, dense attention) before it.  Steps count
 *     from 1.
 *
 * h3f_subblock_plan: host-only sizes of one call.  *n_blocks, *keep and
 * *workspace_bytes (any may be NULL) receive the block count, the key blocks
 * kept per query block, and the device scratch the route call needs.
 *
 * h3f_subblock_route: q, k are bf16 [rows, heads, head_dim] with their own
 * row / head strides in elements (e.g. the q, k outputs of
 * h3f_qk_rmsnorm_rope3d; strides multiples of 8, pointers 16-byte aligned).
 * kv_blocks: device int32 [heads, n_blocks, keep], dense, 4-byte aligned.
 * scores: device fp32 [heads, n_blocks, n_blocks], 16-byte aligned, row
 * (h, i) starting (h * n_blocks + i) * scores_row_stride floats in;
 * scores_row_stride >= n_blocks (n_blocks for dense rows).  Only the first
 * n_blocks floats of a row are written, on routed steps only (the pointer is
 * required on every step).  A stride that is a multiple of 32 (128-byte rows)
 * lets every cache line of scores be written whole by one wavefront, which
 * dense rows of most block counts do not allow.  workspace: device scratch of
 * at least workspace_bytes (16-byte aligned, no initialisation needed; calls
 * sharing one must be ordered on one stream).  Outputs and workspace must not
 * overlap each other or q, k.  On a dense step (step <
 * H3F_SUBBLOCK_FIRST_STEP) the call only writes kv_blocks[h,i,:] =
 * 0..n_blocks-1 and reads neither q nor k.
 * Errors: H3F_ERR_UNSUPPORTED for a dtype other than bf16, head_dim != 128,
 * rows < 4096 (unlike the per-token operators, rows == 0 is not a no-op),
 * n_blocks > 8192, heads > 4096, a q / k stride above 2^31 elements or one
 * head's scores above 2^32 - 16 bytes (n_blocks * scores_row_stride * 4);
 * H3F_ERR_BAD_VALUE for sparsity outside [0, 1) or step < 1;
 * H3F_ERR_BAD_SHAPE for block < 1 or heads < 1; H3F_ERR_BAD_STRIDE for
 * scores_row_stride < n_blocks.
 * Deterministic: fixed summation order; bit-identical run to run.  -0 and +0
 * scores rank equal; with non-finite q / k values the kept lists are still
 * exactly keep valid, ascending block indices, but which ones is unspecified.
 */
#define H3F_SUBBLOCK_FIRST_STEP 10
h3f_status_t h3f_subblock_plan(int64_t rows, int32_t heads, int32_t head_dim, int32_t block,
                               double sparsity, int32_t step, int32_t* n_blocks, int32_t* keep,
                               size_t* workspace_bytes);
h3f_status_t h3f_subblock_route(int32_t* kv_blocks, float* scores, int64_t scores_row_stride,
                                const void* q, int64_t q_row_stride, int64_t q_head_stride,
                                const void* k, int64_t k_row_stride, int64_t k_head_stride,
                                h3f_dtype_t dtype, int64_t rows, int32_t heads,
                                int32_t head_dim, int32_t block, double sparsity,
                                int32_t step, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * QK RMSNorm + 3D RoPE with the router's block pooling fused in.  Writes
 * q_out and k_out exactly as h3f_qk_rmsnorm_rope3d does (bit-identical), and
 * in the same pass the router's block means of the values as stored --
 * qm[h,b,:], km[h,b,:] over token blocks of `block` rows, as described for
 * h3f_subblock_route -- into `workspace`, so that a routed step needs no
 * second read of q_out and k_out (h3f_subblock_route_pooled then finishes the
 * route from the workspace).  This keeps the tensors resident in the producing
 * kernel instead of re-reading them, the fusion the report page credits with
 * its gains (section "Só com três camadas…").
 * Arguments as h3f_qk_rmsnorm_rope3d, plus block and the workspace of
 * h3f_subblock_plan (same rows, heads, head_dim, block); the router's
 * preconditions apply (bf16, head_dim 128, rows >= 4096, n_blocks <= 8192,
 * heads <= 4096; H3F_ERR_UNSUPPORTED otherwise, and rows == 0 is rejected).
 * Errors: as h3f_qk_rmsnorm_rope3d; H3F_ERR_WORKSPACE for a missing,
 * misaligned or short workspace; H3F_ERR_ALIASING if it overlaps a tensor.
 * Each block sum is formed in fp32 in a fixed order: 16 wavefronts each add
 * the block's 2-token chunks w, w + 16, w + 32, ... (w = 0..15) in order, and
 * the 16 partial sums are then added in wavefront order.  The order depends
 * only on the shape, so the means are the same run to run, but they can
 * differ from the separate route's (which sums differently) in the last bits.
 */
h3f_status_t h3f_qk_rmsnorm_rope3d_pool(void* q_out, int64_t q_out_row_stride,
                                        int64_t q_out_head_stride, void* k_out,
                                        int64_t k_out_row_stride, int64_t k_out_head_stride,
                                        const void* q, int64_t q_row_stride,
                                        int64_t q_head_stride, const void* k,
                                        int64_t k_row_stride, int64_t k_head_stride,
                                        const void* q_weight, const void* k_weight,
                                        h3f_dtype_t dtype, int64_t rows, int32_t heads,
                                        int32_t head_dim, float eps, const h3f_rope3d_t* rope,
                                        int32_t block, void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * The router's score and selection from block means already in `workspace`
 * (written by h3f_qk_rmsnorm_rope3d_pool with the same rows, heads, head_dim
 * and block, earlier on the same stream).  Outputs, sizes, step rule, errors
 * and determinism as h3f_subblock_route; on a dense step the workspace is
 * neither needed nor read.
 */
h3f_status_t h3f_subblock_route_pooled(int32_t* kv_blocks, float* scores,
                                       int64_t scores_row_stride, int64_t rows, int32_t heads,
                                       int32_t head_dim, int32_t block, double sparsity,
                                       int32_t step, const void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Streaming copy (measurement helper, not an operator): dst[0:bytes) =
 * src[0:bytes) with 16-byte vector loads and stores.  Used to measure the
 * achievable HBM bandwidth and to calibrate hardware byte counters.  bytes
 * must be a multiple of 16; dst and src must not overlap.
 */
h3f_status_t h3f_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);

/*
 * The two directions of the copy alone (measurement helpers, not operators):
 * h3f_stream_read reads src[0:bytes) with 16-byte vector loads -- streaming
 * (non-temporal) loads, or ordinary cached loads when `cached` is non-zero --
 * and folds the words it loaded; it writes 4 bytes to `sink` (device, 16 bytes,
 * 16-byte aligned) only if the fold hits a fixed 32-bit value, so in practice
 * it stores nothing.  h3f_stream_fill writes the 32-bit `value` repeatedly over
 * dst[0:bytes) with 16-byte streaming stores.  bytes must be a multiple of 16.
 * Errors: NULL_POINTER, BAD_SHAPE, MISALIGNED; ALIASING if sink overlaps src.
 */
h3f_status_t h3f_stream_read(const void* src, int64_t bytes, int32_t cached, void* sink,
                             void* stream);
h3f_status_t h3f_stream_fill(void* dst, int64_t bytes, uint32_t value, void* stream);

/*
 * The write-only stream in store bursts (measurement helper): as
 * h3f_stream_fill, but each 64-wide wavefront writes its own contiguous
 * kib_per_wavefront KiB (1, 2, 5 or 10) with 16-byte streaming stores before it
 * ends, wavefronts in address order.  It measures what a wavefront that stores
 * several KiB can write, the pattern of kernels that hold a whole row (a 10 KiB
 * row at hidden 5120 in bf16) between their loads and stores.  Errors as
 * h3f_stream_fill; H3F_ERR_UNSUPPORTED for another kib_per_wavefront.
 */
h3f_status_t h3f_stream_fill_bursts(void* dst, int64_t bytes, uint32_t value,
                                    int32_t kib_per_wavefront, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* H3FUSED_H */
