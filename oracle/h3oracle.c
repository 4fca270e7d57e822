/*
 * h3oracle.c -- plain CPU oracle for the fused per-token DiT operators.
 *
 * TEST INFRASTRUCTURE ONLY (see h3oracle.h).  Slow and obvious on purpose:
 * one row at a time, double arithmetic, one rounding per stored element.
 * The only parallelism is an OpenMP split over independent rows, which does
 * not change any arithmetic.
 *
 * Built with gcc -O2 -ffp-contract=off (no fused multiply-add, so every
 * float expression rounds exactly as written).
 */
#include "h3oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_abi_version(void) { return 1; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------------------
 * bf16 <-> fp32.  bf16 is the upper 16 bits of an IEEE binary32 value, so the
 * widening is exact; the narrowing rounds to nearest, ties to even, and keeps
 * NaN a (quiet) NaN.
 * ------------------------------------------------------------------------- */
float oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

static double ld(const void* p, int dtype, int64_t i) {
    if (dtype == ORACLE_F32) return (double)((const float*)p)[i];
    return (double)oracle_bf16_to_f32(((const uint16_t*)p)[i]);
}

static void st(void* p, int dtype, int64_t i, double v) {
    float f = (float)v; /* double -> fp32, round to nearest even */
    if (dtype == ORACLE_F32)
        ((float*)p)[i] = f;
    else
        ((uint16_t*)p)[i] = oracle_f32_to_bf16(f);
}

static int64_t group_of(const int64_t* group, int64_t rows_per_group, int64_t r) {
    if (group) return group[r];
    return rows_per_group > 0 ? r / rows_per_group : 0;
}

/* ---------------------------------------------------------------------------
 * Token positions.  The report page (news.cocoloop.cn, MiniMax-H3 on
 * SGLang/H200) and the ceviu.com.br newsletter describe one joint sequence of
 * video and audio tokens; the studioglobal.ai explainer ("MiniMax H3 mở trọng
 * số…", section "Kiến trúc…") gives the VisualVAE factors that set the
 * (t, h, w) latent grid.  Token order (video raster first, then audio) and
 * audio positions (t = k, h = w = 0) are readings the pages leave open.
 * ------------------------------------------------------------------------- */
void oracle_positions(int32_t* pos, int64_t rows, int64_t token_offset,
                      int32_t T, int32_t H, int32_t W, int32_t n_audio) {
    const int64_t n_video = (int64_t)T * H * W;
    const int64_t L = n_video + n_audio;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t p = (token_offset + r) % L;
        int32_t t, h, w;
        if (p < n_video) {
            t = (int32_t)(p / ((int64_t)H * W));
            h = (int32_t)((p / W) % H);
            w = (int32_t)(p % W);
        } else {
            t = (int32_t)(p - n_video);
            h = 0;
            w = 0;
        }
        pos[3 * r + 0] = t;
        pos[3 * r + 1] = h;
        pos[3 * r + 2] = w;
    }
}

/* ---------------------------------------------------------------------------
 * AdaLN modulate.  Operator named in the report page's section "Só com três
 * camadas…" (fused AdaLN update) and in the ceviu.com.br newsletter; its
 * modulation vectors are token independent per the studioglobal.ai explainer
 * (section "Kiến trúc…": the AdaLN branch outputs can be precomputed and
 * cached).  Definition: LayerNorm without affine (Ba et al. 2016, eq. 4, with
 * the biased variance), then the DiT modulation (1 + scale), + shift.
 * ------------------------------------------------------------------------- */
static void adaln_row(void* y, int y_dtype, const void* x, int x_dtype,
                      const void* shift, const void* scale, int mod_dtype,
                      int64_t r, int64_t g, int64_t D, double eps) {
    double sum = 0.0;
    for (int64_t c = 0; c < D; ++c) sum += ld(x, x_dtype, r * D + c);
    const double mean = sum / (double)D;
    double ss = 0.0;
    for (int64_t c = 0; c < D; ++c) {
        const double d = ld(x, x_dtype, r * D + c) - mean;
        ss += d * d;
    }
    const double var = ss / (double)D;
    const double denom = sqrt(var + eps);
    for (int64_t c = 0; c < D; ++c) {
        const double xhat = (ld(x, x_dtype, r * D + c) - mean) / denom;
        const double sc = ld(scale, mod_dtype, g * D + c);
        const double sh = ld(shift, mod_dtype, g * D + c);
        st(y, y_dtype, r * D + c, xhat * (1.0 + sc) + sh);
    }
}

void oracle_adaln_modulate(void* y, int y_dtype, const void* x, int x_dtype,
                           const void* shift, const void* scale, int mod_dtype,
                           const int64_t* group, int64_t rows_per_group,
                           int64_t rows, int64_t hidden, float eps) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        adaln_row(y, y_dtype, x, x_dtype, shift, scale, mod_dtype, r,
                  group_of(group, rows_per_group, r), hidden, (double)eps);
}

/* ---------------------------------------------------------------------------
 * LayerNorm with its own affine gain and bias (Ba, Kiros & Hinton 2016, eq. 4:
 * g * (a - mean) / sigma + b), then the AdaLN modulation of that output.  A
 * variant of the reading above for models whose LayerNorm keeps its affine
 * parameters; gamma and beta are [hidden], shared by every row and group.
 * ------------------------------------------------------------------------- */
static void adaln_affine_row(void* y, int y_dtype, const void* x, int x_dtype,
                             const void* gamma, const void* beta,
                             const void* shift, const void* scale, int mod_dtype,
                             int64_t r, int64_t g, int64_t D, double eps) {
    double sum = 0.0;
    for (int64_t c = 0; c < D; ++c) sum += ld(x, x_dtype, r * D + c);
    const double mean = sum / (double)D;
    double ss = 0.0;
    for (int64_t c = 0; c < D; ++c) {
        const double d = ld(x, x_dtype, r * D + c) - mean;
        ss += d * d;
    }
    const double sigma = sqrt(ss / (double)D + eps);
    for (int64_t c = 0; c < D; ++c) {
        const double ln = ld(gamma, mod_dtype, c) * (ld(x, x_dtype, r * D + c) - mean) / sigma +
                          ld(beta, mod_dtype, c);
        const double sc = ld(scale, mod_dtype, g * D + c);
        const double sh = ld(shift, mod_dtype, g * D + c);
        st(y, y_dtype, r * D + c, ln * (1.0 + sc) + sh);
    }
}

void oracle_adaln_affine_modulate(void* y, int y_dtype, const void* x, int x_dtype,
                                  const void* gamma, const void* beta,
                                  const void* shift, const void* scale, int mod_dtype,
                                  const int64_t* group, int64_t rows_per_group,
                                  int64_t rows, int64_t hidden, float eps) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        adaln_affine_row(y, y_dtype, x, x_dtype, gamma, beta, shift, scale, mod_dtype, r,
                         group_of(group, rows_per_group, r), hidden, (double)eps);
}

/* ---------------------------------------------------------------------------
 * Gated residual.  Named in the report page's section "Só com três
 * camadas…" (residual with gate).  Definition: the DiT block's gated
 * residual, x <- x + alpha * h, alpha broadcast over tokens like the AdaLN
 * modulation.
 * ------------------------------------------------------------------------- */
static void gated_row(void* x, int x_dtype, const void* h, int h_dtype,
                      const void* gate, int64_t r, int64_t g, int64_t D) {
    for (int64_t c = 0; c < D; ++c) {
        const double xv = ld(x, x_dtype, r * D + c);
        const double gv = ld(gate, x_dtype, g * D + c);
        const double hv = ld(h, h_dtype, r * D + c);
        st(x, x_dtype, r * D + c, xv + gv * hv);
    }
}

void oracle_gated_residual(void* x, int x_dtype, const void* h, int h_dtype,
                           const void* gate, const int64_t* group,
                           int64_t rows_per_group, int64_t rows, int64_t hidden) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        gated_row(x, x_dtype, h, h_dtype, gate, r,
                  group_of(group, rows_per_group, r), hidden);
}

/* ---------------------------------------------------------------------------
 * SwiGLU.  Named in the report page's section "Só com três camadas…" and in
 * the ceviu.com.br newsletter.  Definition (Shazeer 2020): Swish_1(a) * b with
 * Swish_1(z) = z * sigmoid(z) = z / (1 + exp(-z)); a and b are the two halves
 * of the fused gate/up projection output.
 * ------------------------------------------------------------------------- */
void oracle_swiglu(void* out, const void* gate_up, int dtype, int64_t rows,
                   int64_t inner) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < inner; ++j) {
            const double a = ld(gate_up, dtype, r * 2 * inner + j);
            const double b = ld(gate_up, dtype, r * 2 * inner + inner + j);
            const double silu = a / (1.0 + exp(-a));
            st(out, dtype, r * inner + j, silu * b);
        }
    }
}

/* ---------------------------------------------------------------------------
 * RoPE frequencies.  RoFormer (Su et al. 2021, eq. 15): theta_i =
 * base^(-2(i-1)/d) for pair i = 1..d/2 of a d-dimensional rotation; here each
 * axis chunk [t | h | w] of the head dimension is its own rotation of size
 * d_c, so pair j of chunk c uses base^(-2j/d_c).
 * ------------------------------------------------------------------------- */
void oracle_rope_inv_freq(float* inv_freq, int32_t d_t, int32_t d_h,
                          int32_t d_w, double theta) {
    const int32_t dims[3] = {d_t, d_h, d_w};
    int32_t p = 0;
    for (int c = 0; c < 3; ++c)
        for (int32_t j = 0; j < dims[c] / 2; ++j)
            inv_freq[p++] = (float)pow(theta, -2.0 * (double)j / (double)dims[c]);
}

/* ---------------------------------------------------------------------------
 * QK RMSNorm + 3D RoPE.  Named as one fused operator in the report page's
 * section "Só com três camadas…" and in the ceviu.com.br newsletter.
 * RMSNorm per head (Zhang & Sennrich 2019, eq. 4, gain w, no bias), applied
 * before the rotation; RoPE per axis chunk (Su et al. 2021, eq. 34).
 * ------------------------------------------------------------------------- */
static void qk_head(void* out, const void* in, const void* weight, int dtype,
                    int64_t base, int32_t Dh, double eps, const int32_t* p3,
                    const int32_t dims[3], const float* inv_freq_f32,
                    double theta, int angle_mode, int pairing) {
    double u[1024];
    double ss = 0.0;
    for (int32_t d = 0; d < Dh; ++d) {
        const double v = ld(in, dtype, base + d);
        ss += v * v;
    }
    const double rms = sqrt(ss / (double)Dh + eps);
    for (int32_t d = 0; d < Dh; ++d)
        u[d] = ld(in, dtype, base + d) / rms * ld(weight, dtype, d);

    int32_t start = 0, pair = 0;
    for (int c = 0; c < 3; ++c) {
        const int32_t dc = dims[c];
        for (int32_t j = 0; j < dc / 2; ++j, ++pair) {
            double phi;
            if (angle_mode == 0) {
                const float pf = (float)p3[c];
                const float ang = pf * inv_freq_f32[pair]; /* one fp32 rounding */
                phi = (double)ang;
            } else {
                phi = (double)p3[c] * pow(theta, -2.0 * (double)j / (double)dc);
            }
            int32_t e0, e1;
            if (pairing == ORACLE_PAIR_INTERLEAVED) {
                e0 = start + 2 * j;
                e1 = start + 2 * j + 1;
            } else {
                e0 = start + j;
                e1 = start + j + dc / 2;
            }
            const double cs = cos(phi), sn = sin(phi);
            const double a = u[e0], b = u[e1];
            u[e0] = a * cs - b * sn;
            u[e1] = a * sn + b * cs;
        }
        start += dc;
    }
    for (int32_t d = 0; d < Dh; ++d) st(out, dtype, base + d, u[d]);
}

void oracle_qk_rmsnorm_rope3d(void* q_out, void* k_out, const void* q,
                              const void* k, const void* q_weight,
                              const void* k_weight, int dtype, int64_t rows,
                              int32_t heads, int32_t head_dim, float eps,
                              const int32_t* pos, int32_t d_t, int32_t d_h,
                              int32_t d_w, double theta, int angle_mode,
                              int pairing) {
    const int32_t dims[3] = {d_t, d_h, d_w};
    float inv_freq[512];
    if (head_dim > 1024 || d_t + d_h + d_w != head_dim) return;
    oracle_rope_inv_freq(inv_freq, d_t, d_h, d_w, theta);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int32_t i = 0; i < heads; ++i) {
            const int64_t base = (r * heads + i) * (int64_t)head_dim;
            qk_head(q_out, q, q_weight, dtype, base, head_dim, (double)eps,
                    pos + 3 * r, dims, inv_freq, theta, angle_mode, pairing);
            qk_head(k_out, k, k_weight, dtype, base, head_dim, (double)eps,
                    pos + 3 * r, dims, inv_freq, theta, angle_mode, pairing);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Gated residual followed by AdaLN on the updated stream: the two operators
 * the report page lists side by side (section "Só com três camadas…"),
 * composed in the order a DiT block runs them.
 * ------------------------------------------------------------------------- */
void oracle_gated_residual_adaln(void* x, int x_dtype, const void* h,
                                 int h_dtype, const void* gate, void* y,
                                 int y_dtype, const void* shift,
                                 const void* scale, const int64_t* group,
                                 int64_t rows_per_group, int64_t rows,
                                 int64_t hidden, float eps) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t g = group_of(group, rows_per_group, r);
        gated_row(x, x_dtype, h, h_dtype, gate, r, g, hidden);
        adaln_row(y, y_dtype, x, x_dtype, shift, scale, x_dtype, r, g, hidden,
                  (double)eps);
    }
}

/* ---------------------------------------------------------------------------
 * Residual difference between neighbouring denoising steps.  The report
 * page (section "Só com três camadas…", Cache-DiT paragraph) decides reuse by
 * comparing a residual difference with a threshold (0.04 / 0.08) but gives no
 * formula; the reading here is the relative L1 distance
 * sum|cur - prev| / sum|prev|.
 * ------------------------------------------------------------------------- */
void oracle_residual_l1(double* out, const void* cur, const void* prev,
                        int dtype, int64_t rows, int64_t hidden) {
    double num = 0.0, den = 0.0;
    for (int64_t i = 0; i < rows * hidden; ++i) {
        const double c = ld(cur, dtype, i);
        const double p = ld(prev, dtype, i);
        num += fabs(c - p);
        den += fabs(p);
    }
    out[0] = num;
    out[1] = den;
}

/* ---------------------------------------------------------------------------
 * Block-sparse attention router.  The report page (section "Só com três
 * camadas…", SubBlock paragraph) describes a block router that, from the
 * tenth denoising step on, keeps only part of the key/value blocks (sparsity
 * 0.75 or 0.80); the newsletter page says the skipped blocks are the ones
 * that matter least.  Block size, pooling and score are not given.  Reading:
 * mean-pool each block of tokens per head, score a (query block, key block)
 * pair by the dot product of the two means -- which equals the average
 * attention logit q.k over all token pairs of the two blocks -- and keep the
 * highest-scoring key blocks.
 * ------------------------------------------------------------------------- */
void oracle_subblock_pool(double* pooled, const void* x, int dtype,
                          int64_t rows, int32_t heads, int32_t head_dim,
                          int32_t block) {
    const int64_t nb = (rows + block - 1) / block;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t r0 = b * block;
        const int64_t r1 = r0 + block < rows ? r0 + block : rows;
        for (int32_t h = 0; h < heads; ++h) {
            for (int32_t d = 0; d < head_dim; ++d) {
                double s = 0.0;
                for (int64_t r = r0; r < r1; ++r)
                    s += ld(x, dtype, (r * heads + h) * head_dim + d);
                pooled[((int64_t)h * nb + b) * head_dim + d] = s / (double)(r1 - r0);
            }
        }
    }
}

void oracle_subblock_scores(double* scores, const double* pq, const double* pk,
                            int32_t heads, int64_t nbq, int64_t nbk,
                            int32_t head_dim) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nbq; ++i) {
        for (int32_t h = 0; h < heads; ++h) {
            const double* a = pq + ((int64_t)h * nbq + i) * head_dim;
            for (int64_t j = 0; j < nbk; ++j) {
                const double* c = pk + ((int64_t)h * nbk + j) * head_dim;
                double s = 0.0;
                for (int32_t d = 0; d < head_dim; ++d) s += a[d] * c[d];
                scores[((int64_t)h * nbq + i) * nbk + j] = s;
            }
        }
    }
}

int64_t oracle_subblock_keep(int64_t nb, double sparsity, int32_t step,
                             int32_t first_step) {
    if (step < first_step) return nb;
    const double skipped = sparsity * (double)nb;
    return nb - (int64_t)floor(skipped);
}

typedef struct {
    double score;
    int32_t block;
} scored_block;

/* larger score first; equal scores: lower block index first */
static int by_score_desc(const void* pa, const void* pb) {
    const scored_block* a = (const scored_block*)pa;
    const scored_block* b = (const scored_block*)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->block > b->block) - (a->block < b->block);
}

static int by_index_asc(const void* pa, const void* pb) {
    const int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

void oracle_subblock_select(int32_t* kv, const double* scores, int32_t heads,
                            int64_t nbq, int64_t nbk, int64_t keep) {
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < (int64_t)heads * nbq; ++row) {
        scored_block* tmp = (scored_block*)malloc((size_t)nbk * sizeof *tmp);
        for (int64_t j = 0; j < nbk; ++j) {
            tmp[j].score = scores[row * nbk + j];
            tmp[j].block = (int32_t)j;
        }
        qsort(tmp, (size_t)nbk, sizeof *tmp, by_score_desc);
        int32_t* out = kv + row * keep;
        for (int64_t t = 0; t < keep; ++t) out[t] = tmp[t].block;
        qsort(out, (size_t)keep, sizeof *out, by_index_asc);
        free(tmp);
    }
}
