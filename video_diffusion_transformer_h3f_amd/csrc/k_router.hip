// k_router.hip -- block-sparse attention router (SubBlock): mean-pool token
// blocks of q and k per head, score every (query block, key block) pair by
// the dot product of the means, keep the highest-scoring key blocks.
//
// Three kernels, all deterministic (fixed summation order, no float atomics):
//   pool    reads q and k once (the HBM-bound part: 2 * rows * heads * 256 B at
//           head_dim 128) and writes fp32 block means to the workspace,
//           [2][heads][n_blocks][128].  A workgroup owns one (tensor, block,
//           group of 4 heads); lane (head hh, 8-element chunk c) walks the
//           block's rows -- each wave load is one contiguous 1 KB row segment
//           when heads are packed -- and sums in fp32 in row order; the waves
//           of a workgroup split the rows round-robin and are added in wave
//           order through LDS.
//   score   scores[h] = Qm[h] Km[h]^T on the matrix cores: fp32 MFMA
//           16x16x4, a 64x64 output tile per workgroup, 32x32 per wave.  The
//           contraction index is split as d = 32 g + kk (g = lane / 16 picks
//           the MFMA k slot, kk the instruction), so each lane reads 32
//           consecutive floats of its row of Qm and of Km.
//   select  one workgroup per (head, query block): the row of scores becomes
//           order-preserving uint32 keys in LDS, a 4-pass 8-bit radix select
//           finds the keep-th largest key T, and two ordered prefix sums emit
//           every block with key > T plus the lowest-index blocks with key ==
//           T, in ascending block order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "h3f_device.hpp"
#include "h3f_validate.hpp"

namespace h3f {
namespace {

constexpr int kHeadDim = 128;
constexpr int64_t kMinRows = 4096;
constexpr int kMaxBlocks = 8192;

// ---------------------------------------------------------------------------
// pool
// ---------------------------------------------------------------------------
#ifndef H3F_POOL_WAVES
#define H3F_POOL_WAVES 4
#endif
#ifndef H3F_POOL_UNROLL
#define H3F_POOL_UNROLL 8
#endif
constexpr int kPoolWaves = H3F_POOL_WAVES;
constexpr int kPoolUnroll = H3F_POOL_UNROLL;
constexpr int kHeadsPerGroup = 4;  // 4 heads x 16 lanes x 8 bf16 = one wave

struct PoolArgs {
    const char* base[2];      // q, k
    int64_t row_stride[2];    // bytes
    int64_t head_stride[2];   // bytes
    int64_t rows;
    int32_t heads;
    int32_t block;
    uint32_t n_blocks;
    uint32_t n_groups;        // ceil(heads / 4)
    float* pooled;            // [2][heads][n_blocks][128]
};

template <int WAVES, int U>
__global__ void __launch_bounds__(64 * WAVES) subblock_pool_kernel(PoolArgs a) {
    __shared__ float part[WAVES > 1 ? WAVES - 1 : 1][64][8];
    const uint32_t per_tensor = a.n_blocks * a.n_groups;
    const uint32_t t = blockIdx.x >= per_tensor ? 1u : 0u;
    const uint32_t rem = blockIdx.x - t * per_tensor;
    const uint32_t b = rem / a.n_groups;
    const uint32_t grp = rem - b * a.n_groups;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int hh = lane >> 4;
    const int c = lane & 15;
    const int head = (int)grp * kHeadsPerGroup + hh;

    const int64_t r0 = (int64_t)b * a.block;
    const int64_t nrows = std::min<int64_t>(a.block, a.rows - r0);
    const int64_t rs = a.row_stride[t];
    const int64_t hs = a.head_stride[t];
    const int64_t row_span = (int64_t)(a.heads - 1) * hs + kHeadDim * 2;
    const rsrc_t rsrc = make_rsrc(a.base[t] + r0 * rs, span_bytes(nrows, rs, row_span));
    // Lanes of heads past the last one read inside the resource and are never stored.
    const uint32_t col = (uint32_t)(std::min(head, a.heads - 1) * hs) + (uint32_t)c * 16u;

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // Rows past the block's end fall outside the resource and load as zeros.
    const int iters = (int)((nrows + WAVES - 1) / WAVES);
    for (int it = 0; it < iters; it += U) {
        Vec<__bf16, 8> v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t r = (uint32_t)((it + u) * WAVES + wave);
            v[u].template load_buf<kLoadStream>(rsrc, r * (uint32_t)rs + col);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (it + u < iters) {
                float f[8];
                v[u].to_float(f);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += f[i];
            }
        }
    }
    if constexpr (WAVES > 1) {
        if (wave > 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) part[wave - 1][lane][i] = acc[i];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 0; w < WAVES - 1; ++w) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += part[w][lane][i];
        }
    }
    if (head >= a.heads) return;
    const float n = (float)nrows;
    float4 m0, m1;
    m0.x = acc[0] / n; m0.y = acc[1] / n; m0.z = acc[2] / n; m0.w = acc[3] / n;
    m1.x = acc[4] / n; m1.y = acc[5] / n; m1.z = acc[6] / n; m1.w = acc[7] / n;
    float* dst = a.pooled + (((size_t)t * a.heads + head) * a.n_blocks + b) * kHeadDim + c * 8;
    reinterpret_cast<float4*>(dst)[0] = m0;
    reinterpret_cast<float4*>(dst)[1] = m1;
}

// ---------------------------------------------------------------------------
// score (fp32 MFMA)
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;       // output tile per workgroup (rows and columns)
constexpr int kWaveTile = 32;   // per wave: 2 x 2 MFMA tiles of 16 x 16

struct ScoreArgs {
    const float* pooled;  // [2][heads][nb][128]
    float* scores;        // [heads][nb][nb]
    int32_t heads;
    uint32_t nb;
    uint32_t tiles;       // ceil(nb / 64)
};

// 32 consecutive floats of row `row` starting at column 32 * g, zero past nb.
__device__ __forceinline__ void load_row32(float (&dst)[32], rsrc_t r, uint32_t row, int g) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const u32x4 x = buf_ld<kLoadReuse>(r, row * (kHeadDim * 4u) + (uint32_t)g * 128u + 16u * v);
        dst[4 * v + 0] = __uint_as_float(x[0]);
        dst[4 * v + 1] = __uint_as_float(x[1]);
        dst[4 * v + 2] = __uint_as_float(x[2]);
        dst[4 * v + 3] = __uint_as_float(x[3]);
    }
}

__global__ void __launch_bounds__(256) subblock_score_kernel(ScoreArgs a) {
    const uint32_t per_head = a.tiles * a.tiles;
    const uint32_t h = blockIdx.x / per_head;
    const uint32_t rem = blockIdx.x - h * per_head;
    const uint32_t ti = rem / a.tiles;
    const uint32_t tj = rem - ti * a.tiles;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ri = lane & 15;  // row of a 16-row operand tile this lane supplies
    const int g = lane >> 4;   // MFMA k slot
    const uint32_t i0 = ti * kTile + (wave >> 1) * kWaveTile;
    const uint32_t j0 = tj * kTile + (wave & 1) * kWaveTile;

    const uint32_t mat_bytes = a.nb * kHeadDim * 4u;
    const float* qm = a.pooled + (size_t)h * a.nb * kHeadDim;
    const float* km = a.pooled + ((size_t)a.heads + h) * a.nb * kHeadDim;
    const rsrc_t rq = make_rsrc(qm, mat_bytes);
    const rsrc_t rk = make_rsrc(km, mat_bytes);

    float A[2][32], B[2][32];
#pragma unroll
    for (int m = 0; m < 2; ++m) load_row32(A[m], rq, i0 + 16 * m + ri, g);
#pragma unroll
    for (int n = 0; n < 2; ++n) load_row32(B[n], rk, j0 + 16 * n + ri, g);

    f32x4 acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n)
                acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[m][kk], B[n][kk], acc[m][n], 0, 0, 0);
    }
    // Result element (row 4 * g + e, column ri) of each 16 x 16 tile sits in
    // lane (ri, g), register e.
    float* out = a.scores + (size_t)h * a.nb * a.nb;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const uint32_t j = j0 + 16 * n + ri;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t i = i0 + 16 * m + 4 * g + e;
                if (i < a.nb && j < a.nb) out[(size_t)i * a.nb + j] = acc[m][n][e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// select
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 256;

struct SelectArgs {
    const float* scores;  // [heads][nb][nb]
    int32_t* kv;          // [heads][nb][keep]
    uint32_t nb;
    uint32_t keep;
};

// Order-preserving map of a finite float to uint32 (-0 is taken as +0).
__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the workgroup in thread order; *total gets
// the sum.  Uses red[0..4].
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* red, uint32_t* total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) red[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) {
        const uint32_t s = red[w];
        if (w < wave) before += s;
        all += s;
    }
    __syncthreads();  // red may be reused by the next scan
    *total = all;
    return before + x - v;
}

__global__ void __launch_bounds__(kSelThreads) subblock_select_kernel(SelectArgs a) {
    extern __shared__ uint32_t keys[];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t red[4];
    __shared__ uint32_t found_digit, found_above;
    const uint32_t row = blockIdx.x;  // h * nb + i
    const float* s = a.scores + (size_t)row * a.nb;
    for (uint32_t j = threadIdx.x; j < a.nb; j += kSelThreads) keys[j] = order_key(s[j]);

    // Radix select of the keep-th largest key, 8 bits at a time from the top.
    uint32_t prefix = 0, mask = 0, need = a.keep;
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[threadIdx.x] = 0;
        __syncthreads();
        for (uint32_t j = threadIdx.x; j < a.nb; j += kSelThreads) {
            const uint32_t key = keys[j];
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            const int L = threadIdx.x;
            const uint32_t c0 = hist[4 * L], c1 = hist[4 * L + 1], c2 = hist[4 * L + 2],
                           c3 = hist[4 * L + 3];
            const uint32_t own = c0 + c1 + c2 + c3;
            uint32_t x = own;  // inclusive sum over lanes >= L
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_down(x, off, 64);
                if (L + off < 64) x += y;
            }
            // ge[d]: keys (matching the prefix) whose digit is >= d
            const uint32_t ge3 = x - own + c3, ge2 = ge3 + c2, ge1 = ge2 + c1, ge0 = ge1 + c0;
            const uint32_t above = x - own;  // digits > 4L + 3
            // the digit is the largest d with ge[d] >= need; exactly one lane owns it
            if (ge3 >= need && above < need) { found_digit = 4 * L + 3; found_above = above; }
            else if (ge2 >= need && ge3 < need) { found_digit = 4 * L + 2; found_above = ge3; }
            else if (ge1 >= need && ge2 < need) { found_digit = 4 * L + 1; found_above = ge2; }
            else if (ge0 >= need && ge1 < need) { found_digit = 4 * L; found_above = ge1; }
        }
        __syncthreads();
        prefix |= found_digit << shift;
        mask |= 255u << shift;
        need -= found_above;
        __syncthreads();  // found_* are rewritten by the next pass
    }
    const uint32_t T = prefix;  // the keep-th largest key; `need` keys equal to it are kept

    // Each thread owns a contiguous run of block indices, so thread-order
    // prefix sums are block-order prefix sums.
    const uint32_t per = (a.nb + kSelThreads - 1) / kSelThreads;
    const uint32_t j0 = std::min(a.nb, threadIdx.x * per);
    const uint32_t j1 = std::min(a.nb, j0 + per);
    uint32_t n_eq = 0;
    for (uint32_t j = j0; j < j1; ++j) n_eq += keys[j] == T ? 1u : 0u;
    uint32_t total;
    const uint32_t eq_before = block_exclusive_scan(n_eq, red, &total);
    uint32_t n_sel = 0;
    for (uint32_t j = j0, e = eq_before; j < j1; ++j) {
        const uint32_t key = keys[j];
        if (key > T) ++n_sel;
        else if (key == T) { n_sel += e < need ? 1u : 0u; ++e; }
    }
    const uint32_t sel_before = block_exclusive_scan(n_sel, red, &total);
    int32_t* out = a.kv + (size_t)row * a.keep;
    uint32_t pos = sel_before;
    for (uint32_t j = j0, e = eq_before; j < j1; ++j) {
        const uint32_t key = keys[j];
        bool take = key > T;
        if (key == T) { take = e < need; ++e; }
        if (take && pos < a.keep) out[pos++] = (int32_t)j;  // exactly keep are taken
    }
}

// Dense step: every query block keeps every key block, in order.
__global__ void __launch_bounds__(256) subblock_dense_kernel(int32_t* kv, uint32_t nb, uint64_t total) {
    for (uint64_t x = (uint64_t)blockIdx.x * 256 + threadIdx.x; x < total;
         x += (uint64_t)gridDim.x * 256)
        kv[x] = (int32_t)(x % nb);
}

inline int64_t keep_for(int64_t nb, double sparsity, int32_t step) {
    if (step < H3F_SUBBLOCK_FIRST_STEP) return nb;
    const double skipped = sparsity * (double)nb;
    return nb - (int64_t)std::floor(skipped);
}

inline size_t workspace_for(int64_t nb, int32_t heads) {
    return (size_t)2 * heads * nb * kHeadDim * sizeof(float);
}

h3f_status_t check_plan(int64_t rows, int32_t heads, int32_t head_dim, int32_t block,
                        double sparsity, int32_t step) {
    if (rows < 0 || heads < 1 || block < 1 || head_dim < 1) return H3F_ERR_BAD_SHAPE;
    if (!(sparsity >= 0.0 && sparsity < 1.0) || step < 1) return H3F_ERR_BAD_VALUE;
    if (head_dim != kHeadDim || rows < kMinRows) return H3F_ERR_UNSUPPORTED;
    if ((rows + block - 1) / block > kMaxBlocks || heads > 4096) return H3F_ERR_UNSUPPORTED;
    // a sparsity within rounding of 1 could leave no block at all
    if (keep_for((rows + block - 1) / block, sparsity, step) < 1) return H3F_ERR_BAD_VALUE;
    return H3F_OK;
}

}  // namespace
}  // namespace h3f

using namespace h3f;

extern "C" h3f_status_t h3f_subblock_plan(int64_t rows, int32_t heads, int32_t head_dim,
                                          int32_t block, double sparsity, int32_t step,
                                          int32_t* n_blocks, int32_t* keep,
                                          size_t* workspace_bytes) {
    const h3f_status_t st = check_plan(rows, heads, head_dim, block, sparsity, step);
    if (st != H3F_OK) return st;
    const int64_t nb = (rows + block - 1) / block;
    if (n_blocks) *n_blocks = (int32_t)nb;
    if (keep) *keep = (int32_t)keep_for(nb, sparsity, step);
    if (workspace_bytes) *workspace_bytes = workspace_for(nb, heads);
    return H3F_OK;
}

extern "C" h3f_status_t h3f_subblock_route(int32_t* kv_blocks, float* scores, const void* q,
                                           int64_t q_row_stride, int64_t q_head_stride,
                                           const void* k, int64_t k_row_stride,
                                           int64_t k_head_stride, h3f_dtype_t dtype, int64_t rows,
                                           int32_t heads, int32_t head_dim, int32_t block,
                                           double sparsity, int32_t step, void* workspace,
                                           size_t workspace_bytes, void* stream) {
    if (!kv_blocks || !scores || !q || !k) return H3F_ERR_NULL_POINTER;
    if (!dtype_ok(dtype)) return H3F_ERR_BAD_DTYPE;
    const h3f_status_t st = check_plan(rows, heads, head_dim, block, sparsity, step);
    if (st != H3F_OK) return st;
    if (dtype != H3F_BF16) return H3F_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k)) return H3F_ERR_MISALIGNED;
    if ((reinterpret_cast<uintptr_t>(kv_blocks) & 3u) || (reinterpret_cast<uintptr_t>(scores) & 3u))
        return H3F_ERR_MISALIGNED;
    constexpr int V = 8;
    if (q_row_stride % V || k_row_stride % V) return H3F_ERR_BAD_STRIDE;
    if (heads > 1 && (q_head_stride % V || k_head_stride % V || q_head_stride < head_dim ||
                      k_head_stride < head_dim))
        return H3F_ERR_BAD_STRIDE;
    const int64_t qhs = heads > 1 ? q_head_stride : head_dim;
    const int64_t khs = heads > 1 ? k_head_stride : head_dim;
    const int64_t q_span = (int64_t)(heads - 1) * qhs + head_dim;
    const int64_t k_span = (int64_t)(heads - 1) * khs + head_dim;
    const Region rq = region2d(q, rows, q_row_stride, q_span, 2);
    const Region rk = region2d(k, rows, k_row_stride, k_span, 2);
    if (!rows_separate(rq) || !rows_separate(rk)) return H3F_ERR_BAD_STRIDE;
    // one block of rows (plus the rows an unrolled batch reads past its end,
    // which must stay outside the resource) is addressed with 32-bit offsets
    if ((int64_t)(block + kPoolUnroll * kPoolWaves) * std::max(q_row_stride, k_row_stride) * 2 +
            2 * std::max(q_span, k_span) > 0xFFFFFFF0ll)
        return H3F_ERR_UNSUPPORTED;

    const int64_t nb = (rows + block - 1) / block;
    const int64_t keep = keep_for(nb, sparsity, step);
    const size_t need = workspace_for(nb, heads);
    const bool routed = step >= H3F_SUBBLOCK_FIRST_STEP;
    if (routed && (!workspace || !aligned16(workspace) || workspace_bytes < need))
        return H3F_ERR_WORKSPACE;
    const Region rkv = region2d(kv_blocks, 1, 0, (int64_t)heads * nb * keep * 4, 1);
    const Region rsc = region2d(scores, 1, 0, (int64_t)heads * nb * nb * 4, 1);
    const Region rws = region2d(workspace, 1, 0, routed ? (int64_t)need : 0, 1);
    if (!disjoint(rkv, rq) || !disjoint(rkv, rk) || !disjoint(rkv, rws) ||
        (routed && (!disjoint(rkv, rsc) || !disjoint(rsc, rq) || !disjoint(rsc, rk) ||
                    !disjoint(rsc, rws) || !disjoint(rws, rq) || !disjoint(rws, rk))))
        return H3F_ERR_ALIASING;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint64_t total = (uint64_t)heads * nb * keep;
    if (!routed) {
        const unsigned blocks = (unsigned)std::min<uint64_t>((total + 255) / 256, 65536);
        hipLaunchKernelGGL(subblock_dense_kernel, dim3(blocks), dim3(256), 0, s, kv_blocks,
                           (uint32_t)nb, total);
        return hipGetLastError() == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
    }

    PoolArgs pa;
    pa.base[0] = static_cast<const char*>(q);
    pa.base[1] = static_cast<const char*>(k);
    pa.row_stride[0] = q_row_stride * 2;
    pa.row_stride[1] = k_row_stride * 2;
    pa.head_stride[0] = qhs * 2;
    pa.head_stride[1] = khs * 2;
    pa.rows = rows;
    pa.heads = heads;
    pa.block = block;
    pa.n_blocks = (uint32_t)nb;
    pa.n_groups = (uint32_t)((heads + kHeadsPerGroup - 1) / kHeadsPerGroup);
    pa.pooled = static_cast<float*>(workspace);
    hipLaunchKernelGGL((subblock_pool_kernel<kPoolWaves, kPoolUnroll>),
                       dim3(2 * pa.n_blocks * pa.n_groups), dim3(64 * kPoolWaves), 0, s, pa);

    ScoreArgs sa;
    sa.pooled = pa.pooled;
    sa.scores = scores;
    sa.heads = heads;
    sa.nb = (uint32_t)nb;
    sa.tiles = (uint32_t)((nb + kTile - 1) / kTile);
    hipLaunchKernelGGL(subblock_score_kernel, dim3((unsigned)(heads * sa.tiles * sa.tiles)),
                       dim3(256), 0, s, sa);

    SelectArgs se;
    se.scores = scores;
    se.kv = kv_blocks;
    se.nb = (uint32_t)nb;
    se.keep = (uint32_t)keep;
    hipLaunchKernelGGL(subblock_select_kernel, dim3((unsigned)(heads * nb)), dim3(kSelThreads),
                       (size_t)nb * sizeof(uint32_t), s, se);
    return hipGetLastError() == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}
