// k_router.hip -- block-sparse attention router (SubBlock): mean-pool token
// blocks of q and k per head, score every (query block, key block) pair by
// the dot product of the means, keep the highest-scoring key blocks.
//
// Three kernels, all deterministic (fixed summation order, no float atomics):
//   pool    reads q and k once (the HBM-bound part: 2 * rows * heads * 256 B at
//           head_dim 128) and writes fp32 block means to the workspace,
//           [2][heads][n_blocks][128].  Dense q / k: one 128-thread workgroup
//           per (tensor, block) streams the block's contiguous bytes front to
//           back (flat form).  Other layouts: a workgroup owns one (tensor,
//           block, group of 4 heads); lane (head hh, 8-element chunk c) walks
//           the block's rows and the waves split the rows round-robin.  Sums
//           are fp32 in a fixed order.
//   score   scores[h] = Qm[h] Km[h]^T on the matrix cores (fp32 MFMA 16x16x4).
//           A workgroup holds a 64-row tile of Qm in registers (32 x 32 per
//           wave) and walks a run of 64-column tiles of Km with the next
//           tile's loads in flight; the contraction index is split as
//           d = 16 v + 4 g + e (g = lane / 16 picks the MFMA k slot,
//           instruction 4 v + e), the same split for both operands, so the 4
//           lanes of a row read 64 contiguous bytes.
//   select  one wavefront per (head, query block): the row of scores becomes
//           order-preserving uint32 keys in registers; an interpolation /
//           bisection search with ballot counts brackets the keep-th largest
//           key, a 64-lane sort of the last few candidates pins it down, and
//           ballot compaction writes the kept blocks in ascending order.
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
#ifndef H3F_POOL_FLAT
#define H3F_POOL_FLAT 1
#endif
constexpr int kPoolWaves = H3F_POOL_WAVES;
constexpr int kPoolUnroll = H3F_POOL_UNROLL;
constexpr int kHeadsPerGroup = 4;  // 4 heads x 16 lanes x 8 bf16 = one wave

template <int P>
constexpr int mult_max_slots();  // accumulator slots of a flat-pool workgroup (defined below)

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

// Flat form, for q / k whose rows and heads are packed ([rows, heads, 128]
// dense): block b of a tensor is one contiguous range of nrows * cpr 16-byte
// chunks (cpr = 16 * heads per row).  A workgroup of T = kFlatThreads threads
// streams it front to back, T * 16 bytes per step; thread t takes chunks
// t + T k.  Its column (t + T k) mod cpr repeats with period P = cpr /
// gcd(T, cpr), so it keeps P accumulators and slot k mod P always meets the
// same column.  The slots of all threads, L = t + T s (s < P), cover
// [0, mult * cpr) exactly, with mult = T / gcd(T, cpr) copies of each column;
// when mult > 1 the copies are added in copy order through LDS.  Fixed order
// throughout.  Measured at the 5 s shape: 128 threads with 8 loads in flight
// per thread beat 64-512 threads and 4-16 loads.
#ifndef H3F_FLAT_THREADS
#define H3F_FLAT_THREADS 128
#endif
#ifndef H3F_FLAT_DEPTH
#define H3F_FLAT_DEPTH 8
#endif
constexpr int kFlatThreads = H3F_FLAT_THREADS;
constexpr int kFlatDepth = H3F_FLAT_DEPTH;

template <int P>
constexpr int mult_max_slots() { return P * kFlatThreads; }

template <int P>
__global__ void __launch_bounds__(kFlatThreads) subblock_pool_flat_kernel(PoolArgs a, uint32_t cpr,
                                                                          uint32_t mult) {
    constexpr int U = P * ((kFlatDepth + P - 1) / P);  // loads in flight per thread, a multiple of P
    __shared__ float part[mult_max_slots<P>()][8];
    const uint32_t t = blockIdx.x >= a.n_blocks ? 1u : 0u;
    const uint32_t b = blockIdx.x - t * a.n_blocks;
    const uint32_t tid = threadIdx.x;
    const int64_t r0 = (int64_t)b * a.block;
    const int64_t nrows = std::min<int64_t>(a.block, a.rows - r0);
    const uint32_t n_chunks = (uint32_t)nrows * cpr;
    const rsrc_t rsrc = make_rsrc(a.base[t] + r0 * a.row_stride[t], n_chunks * 16u);
    const uint32_t steps = (n_chunks + kFlatThreads - 1) / kFlatThreads;

    float acc[P][8];
#pragma unroll
    for (int s = 0; s < P; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[s][i] = 0.f;
    for (uint32_t k0 = 0; k0 < steps; k0 += U) {
        Vec<__bf16, 8> v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)  // chunks past the block's end read as zeros
            v[u].template load_buf<kLoadStream>(rsrc, (tid + kFlatThreads * (k0 + u)) * 16u);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float f[8];
            v[u].to_float(f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u % P][i] += f[i];
        }
    }
    const float n = (float)nrows;
    float* out_t = a.pooled + (size_t)t * a.heads * a.n_blocks * kHeadDim;
    auto store_mean = [&](uint32_t col, const float (&sum)[8]) {
        const uint32_t head = col >> 4, d8 = col & 15u;
        float* dst = out_t + ((size_t)head * a.n_blocks + b) * kHeadDim + d8 * 8;
        float4 m0, m1;
        m0.x = sum[0] / n; m0.y = sum[1] / n; m0.z = sum[2] / n; m0.w = sum[3] / n;
        m1.x = sum[4] / n; m1.y = sum[5] / n; m1.z = sum[6] / n; m1.w = sum[7] / n;
        reinterpret_cast<float4*>(dst)[0] = m0;
        reinterpret_cast<float4*>(dst)[1] = m1;
    };
    if (mult == 1) {  // slot s of thread t is column t + kFlatThreads * s
#pragma unroll
        for (int s = 0; s < P; ++s) store_mean(tid + kFlatThreads * s, acc[s]);
        return;
    }
#pragma unroll
    for (int s = 0; s < P; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) part[tid + kFlatThreads * s][i] = acc[s][i];
    __syncthreads();
    for (uint32_t col = tid; col < cpr; col += kFlatThreads) {
        float sum[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) sum[i] = 0.f;
        for (uint32_t c = 0; c < mult; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) sum[i] += part[c * cpr + col][i];
        store_mean(col, sum);
    }
}

// ---------------------------------------------------------------------------
// score (fp32 MFMA)
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;       // output tile per workgroup (rows and columns)
constexpr int kWaveTile = 32;   // per wave: 2 x 2 MFMA tiles of 16 x 16

struct ScoreArgs {
    const float* pooled;  // [2][heads][nb][128]
    float* scores;        // [heads][nb][ss], the first nb columns of each row
    int32_t heads;
    uint32_t nb;
    uint32_t ss;          // row stride of scores in floats (>= nb)
    uint32_t tiles;       // ceil(nb / 64)
};

// The 32 floats of row `row` this lane feeds to the MFMAs: columns
// 16 v + 4 g + e (v < 8, e < 4) in register 4 v + e, zero past nb.  Per load
// instruction the 4 lanes of a row read one contiguous 64-byte piece of it.
__device__ __forceinline__ void load_row32(float (&dst)[32], rsrc_t r, uint32_t row, int g) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const u32x4 x = buf_ld<kLoadReuse>(r, row * (kHeadDim * 4u) + 64u * v + (uint32_t)g * 16u);
        dst[4 * v + 0] = __uint_as_float(x[0]);
        dst[4 * v + 1] = __uint_as_float(x[1]);
        dst[4 * v + 2] = __uint_as_float(x[2]);
        dst[4 * v + 3] = __uint_as_float(x[3]);
    }
}

// Score tiles are numbered XCD by XCD (xcd_linear), so the few heads in
// flight on an XCD share its L2.

// Strip form: a workgroup keeps one 64-row tile of Qm in registers and walks
// a run of kScoreRun 64-column tiles of Km, each in two halves of the
// contraction (head_dim columns 0..63, then 64..127).  Each half tile (64
// rows x 64 floats) is gathered into LDS once per workgroup with 16-byte
// buffer-to-LDS loads, already in the order the matrix instructions take it:
// 1 KiB fragments (rows 16 R .. 16 R + 15, columns 16 v .. 16 v + 15) in which
// lane ri + 16 g holds row 16 R + ri, columns 16 v + 4 g .. + 3.  Every
// wavefront then reads its operands with linear, conflict-free 16-byte LDS
// reads, and the two wavefronts that share key columns do not load them
// twice.  Two 16 KiB buffers alternate, the next half tile's gather in flight
// during the current half's matrix instructions (one barrier per half).  The
// MFMA is fed Km as its first operand and Qm as its second, so it produces
// the transposed tile: lane (ri, g) holds scores[i0 + ri][j0 + 4 g .. 4 g +
// 3], one 16-byte store per 16 x 16 tile after the second half.  Rows and
// column tiles past the last block read zeros and store nothing.  Measured at
// the 5 s shape: 125 us with the operands pipelined through registers, 115 us
// with whole key tiles in two 32 KiB buffers (two workgroups per CU), 103-108
// us with half tiles (32 KiB of LDS and 126 registers: four workgroups per
// CU); runs of 4 and 16 tiles were slower than 8 in both LDS forms.
#ifndef H3F_SCORE_RUN
#define H3F_SCORE_RUN 8
#endif
constexpr uint32_t kScoreRun = H3F_SCORE_RUN;  // column tiles per workgroup

// acc[m][n][e] = scores[i0 + 16 m + ri][j0 + 16 n + 4 g + e].  Stores go
// through a buffer resource over the head's score matrix; an element outside
// the matrix gets an offset past the resource's end and is dropped, so there
// is no branch.  A lane's 4 columns go out as one 16-byte store when all 4 lie
// inside the row (a multi-dword buffer store needs only dword alignment, so
// rows that start 4- or 8-byte aligned take it too).  When nb is not a
// multiple of 4, the one group per row that straddles the row's end is
// written by extra stores that every group issues and only that one keeps:
// SB = 8 (nb = 2 mod 4, 2 columns left) adds an 8-byte store, SB = 4 (nb odd,
// 1 or 3 left) an 8-byte and a 4-byte one.  Every tile thus issues a fixed
// number of stores in straight-line code, and the wait for the next tile's
// operand loads never includes them.  The stores keep the default write-back
// policy: L2 merges the 64-byte row pieces into whole lines (the streaming
// policies ran 145 and 171 us instead of 111).  Measured at the 5 s shape
// (978 blocks): two 8-byte stores for every group (each instruction writing
// every other 8 bytes of the rows it touches) 115 us, this form 108 us.
// Choosing the store width per tile with a branch was no better than 113 us:
// where the two store counts meet, the compiler waits for every store before
// the barrier.
constexpr uint32_t kDropped = 0xFFFFFFF0u;

template <int SB>
__device__ __forceinline__ void store_tile32_t(rsrc_t r, uint32_t nb, uint32_t ss, uint32_t i0,
                                               uint32_t j0, int ri, int g, const f32x4 (&acc)[2][2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const uint32_t i = i0 + 16 * m + ri;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const uint32_t j = j0 + 16 * n + 4 * g;
            const uint32_t off = (i * ss + j) * 4u;
            const f32x4 v = acc[m][n];
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r,
                                                   i < nb && j + 3 < nb ? off : kDropped, 0, 0);
            if constexpr (SB != 16) {
                const bool straddle = i < nb && j < nb && j + 3 >= nb;
                const uint32_t left = nb - j;  // columns left in the row (straddle: 1 .. 3)
                const u32x2 w = {__float_as_uint(v[0]), __float_as_uint(v[1])};
                __builtin_amdgcn_raw_buffer_store_b64(w, r, straddle && left >= 2 ? off : kDropped,
                                                      0, 0);
                if constexpr (SB == 4) {
                    // the last column of an odd remainder: j (1 left) or j + 2 (3 left)
                    const float last = left == 3 ? v[2] : v[0];
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __float_as_uint(last), r,
                        straddle && (left & 1) ? off + 4u * (left - 1) : kDropped, 0, 0);
                }
            }
        }
    }
}

constexpr int kTileFrags = (kTile / 16) * 8;  // 1 KiB fragments per 64-row key tile

// vmcnt(n stores per tile): this wavefront's gather of the next tile is
// complete while the current tile's stores, issued after it, may still be in
// flight.
template <int SB>
__device__ __forceinline__ void wait_own_gather() {
    constexpr int n = SB == 16 ? 4 : (SB == 8 ? 8 : 12);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

template <int SB>
__global__ void __launch_bounds__(256) subblock_score_kernel(ScoreArgs a) {
    constexpr int HF = kTileFrags / 2;  // 1 KiB fragments per half key tile (64 columns)
    __shared__ u32x4 kbuf[2][HF * 64];
    const uint32_t runs = (a.tiles + kScoreRun - 1) / kScoreRun;
    const uint32_t per_head = a.tiles * runs;
    const uint32_t w = xcd_linear(blockIdx.x, (uint32_t)a.heads * per_head);
    const uint32_t h = w / per_head;
    const uint32_t rem = w - h * per_head;
    const uint32_t ti = rem / runs;
    const uint32_t run = rem - ti * runs;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ri = lane & 15;
    const int g = lane >> 4;
    const uint32_t i0 = ti * kTile + (wave >> 1) * kWaveTile;
    const uint32_t jrun = run * kScoreRun * kTile;
    const int rj = (wave & 1) * 2;  // first 16-row group of this wavefront's key rows

    const uint32_t mat_bytes = a.nb * kHeadDim * 4u;
    const rsrc_t rq = make_rsrc(a.pooled + (size_t)h * a.nb * kHeadDim, mat_bytes);
    const rsrc_t rk = make_rsrc(a.pooled + ((size_t)a.heads + h) * a.nb * kHeadDim, mat_bytes);
    const rsrc_t ro = make_rsrc(a.scores + (size_t)h * a.nb * a.ss, a.nb * a.ss * 4u);

    // step s = 2 t + hk: half hk of key tile t.  Wavefront w gathers fragments
    // 4 w .. 4 w + 3 of it into buffer b; fragment f = 4 R + v' holds rows
    // 16 R .. + 15 (rows past nb read 0), columns 64 hk + 16 v' .. + 15
    auto gather = [&](int s, int b) {
        const uint32_t t = (uint32_t)(s >> 1);
        const uint32_t hk = (uint32_t)(s & 1);
#pragma unroll
        for (int f4 = 0; f4 < HF / 4; ++f4) {
            const int f = wave * (HF / 4) + f4;
            const uint32_t row = jrun + t * kTile + 16u * (uint32_t)(f >> 2) + (uint32_t)ri;
            const uint32_t off =
                row * (kHeadDim * 4u) + 256u * hk + 64u * (uint32_t)(f & 3) + 16u * (uint32_t)g;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (__attribute__((address_space(3))) void*)&kbuf[b][f * 64], 16, off, 0, 0,
                kLoadReuse);
        }
    };

    float A[2][32], B[2][16];
#pragma unroll
    for (int m = 0; m < 2; ++m) load_row32(A[m], rq, i0 + 16 * m + ri, g);
    gather(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    f32x4 acc[2][2];
    constexpr int NS = 2 * (int)kScoreRun;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int hk = s & 1;
        if (s > 0) {
            // this wavefront's gather of step s is complete; after a second half
            // the tile's stores, issued after it, may still be in flight
            if (hk == 0)
                wait_own_gather<SB>();
            else
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing was stored
        }
        __syncthreads();  // every gather of step s is complete; the other buffer is free
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const u32x4 x = kbuf[s & 1][((rj + n) * 4 + v) * 64 + lane];
                B[n][4 * v + 0] = __uint_as_float(x[0]);
                B[n][4 * v + 1] = __uint_as_float(x[1]);
                B[n][4 * v + 2] = __uint_as_float(x[2]);
                B[n][4 * v + 3] = __uint_as_float(x[3]);
            }
        if (s + 1 < NS) gather(s + 1, (s + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (hk == 0) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 2; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(B[n][kk], A[m][16 * hk + kk],
                                                                     acc[m][n], 0, 0, 0);
        if (hk == 1)
            store_tile32_t<SB>(ro, a.nb, a.ss, i0,
                               jrun + (uint32_t)(s >> 1) * kTile + (wave & 1) * kWaveTile, ri, g,
                               acc);
    }
}

// ---------------------------------------------------------------------------
// select
// ---------------------------------------------------------------------------
constexpr int kSelWaves = 4;  // rows per workgroup, one wavefront each

struct SelectArgs {
    const float* scores;  // [heads][nb][ss]
    int32_t* kv;          // [heads][nb][keep]
    uint32_t rows;        // heads * nb
    uint32_t nb;
    uint32_t ss;          // row stride of scores in floats
    uint32_t keep;
    float z;  // first probe at mean + z * std of the row (z: normal quantile of the kept share)
};

// z with P(Z > z) = p for a standard normal Z (Abramowitz & Stegun 26.2.23,
// |error| < 4.5e-4; p clamped into (0, 1)).  Only the select kernel's first
// guess depends on it.
inline float normal_upper_quantile(double p) {
    p = std::min(std::max(p, 1e-6), 1.0 - 1e-6);
    const double q = p < 0.5 ? p : 1.0 - p;
    const double t = std::sqrt(-2.0 * std::log(q));
    const double x = t - (2.515517 + 0.802853 * t + 0.010328 * t * t) /
                             (1.0 + 1.432788 * t + 0.189269 * t * t + 0.001308 * t * t * t);
    return (float)(p < 0.5 ? x : -x);
}

// Order-preserving map of a float to uint32 (-0 is taken as +0).
__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The float an order key stands for.
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

// Number of lanes below this one whose bit is set in mask.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// One wavefront per row of scores; lane L holds keys of blocks L + 64 m,
// m < KPL (nb <= 64 KPL).  The keep-th largest key T is bracketed by a search
// over [min key, max key] with the invariant count(key >= lo) >= keep >
// count(key > hi); each count is a ballot per register and a scalar popcount.
// The first probe sits at mean + z * std of the row, where a normally
// distributed row would have keep scores above it; later probes interpolate
// linearly between the bracket's float values and counts, falling back to the
// value midpoint when a step does not halve the keys in the bracket, and to
// the integer midpoint when neither splits it.  Every probe only narrows the
// bracket by an exact count, so the guess decides the number of probes, never
// the result (measured on rows like the 5 s shape's, 978 blocks keeping 196: 7.2
// probes on average from [min, max], 3.8 from the guess).  The search
// stops at a probe with exactly keep keys at or above it, or once at most 64
// keys remain in the bracket; those are sorted across the lanes and T is read
// at its rank.  The kept blocks -- every key > T, then keys == T in block
// order until keep are taken -- are written in block order by ballot
// compaction.  LDS holds only each wave's own 64 candidates; no barrier.
template <int KPL>
__global__ void __launch_bounds__(64 * kSelWaves) subblock_select_kernel(SelectArgs a) {
    // wave-uniform (readfirstlane), so the row's buffer resource lives in SGPRs
    const uint32_t row = __builtin_amdgcn_readfirstlane(blockIdx.x * kSelWaves + (threadIdx.x >> 6));
    if (row >= a.rows) return;  // whole wavefront
    const uint32_t lane = threadIdx.x & 63;
    // All KPL loads are issued before any is used: a buffer resource over the
    // row returns 0 past its end, so no load sits behind a branch.
    const rsrc_t rs = make_rsrc(a.scores + (size_t)row * a.ss, a.nb * 4u);
    uint32_t sv[KPL];  // raw fp32 bits
#pragma unroll
    for (int m = 0; m < KPL; ++m)
        sv[m] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(
                                                 rs, (lane + 64u * m) * 4u, 0, kLoadStream));
    uint32_t key[KPL];
    // Padding slots hold key 0 and real keys are >= 1, so every probe (> lo >=
    // 1) and the final threshold leave the padding out without a separate test.
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const bool valid = lane + 64u * m < a.nb;
        const uint32_t k = max(order_key(__uint_as_float(sv[m])), 1u);
        key[m] = valid ? k : 0u;
        kmin = min(kmin, valid ? k : 0xFFFFFFFFu);
        kmax = max(kmax, key[m]);
    }
    auto count_ge = [&](uint32_t t) {
        uint32_t n = 0;
#pragma unroll
        for (int m = 0; m < KPL; ++m) n += (uint32_t)__popcll(__ballot(key[m] >= t));
        return n;
    };
    // Invariant: count(key >= lo) = c_lo >= keep > c_hi = count(key > hi).
    uint32_t lo = __builtin_amdgcn_readfirstlane(wave_min_u32(kmin));
    uint32_t hi = __builtin_amdgcn_readfirstlane(wave_max_u32(kmax));
    uint32_t c_lo = a.nb, c_hi = 0;
    // the first guess: padding slots read 0.0 and add nothing to the sums
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const float v = __uint_as_float(sv[m]);
        s1 += v;
        s2 = __builtin_fmaf(v, v, s2);
    }
    const float inv_nb = 1.0f / (float)a.nb;
    const float mean = wave_sum(s1) * inv_nb;
    const float var = wave_sum(s2) * inv_nb - mean * mean;
    const uint32_t guess = __builtin_amdgcn_readfirstlane(
        order_key(mean + a.z * __builtin_sqrtf(var > 0.f ? var : 0.f)));
    bool interpolate = true, exact = false;
    for (int probe = 0; lo < hi && c_lo - c_hi > 64u; ++probe) {
        const float vlo = key_value(lo), vhi = key_value(hi);
        // interpolation: where a straight line through (vlo, c_lo), (vhi, c_hi)
        // crosses keep; bisection of the value interval when the last
        // interpolation step did not halve the candidates
        const float f = interpolate ? ((float)(c_lo - a.keep) + 0.5f) *
                                          __builtin_amdgcn_rcpf((float)(c_lo - c_hi))
                                    : 0.5f;
        uint32_t mid = probe == 0 ? guess : order_key(vlo + f * (vhi - vlo));
        if (probe >= 24 || !(mid > lo && mid <= hi)) mid = lo + ((hi - lo) >> 1) + 1u;
        const uint32_t c = count_ge(mid);
        const uint32_t before = c_lo - c_hi;
        if (c >= a.keep) {
            lo = mid;
            c_lo = c;
            if (c == a.keep) {
                exact = true;
                break;
            }
        } else {
            hi = mid - 1u;
            c_hi = c;
        }
        interpolate = !interpolate || 2u * (c_lo - c_hi) <= before;
    }
    uint32_t T, n_gt, n_ge;
    if (!exact && lo < hi) {
        // At most 64 keys lie in [lo, hi]: gather them into one register per
        // lane (wave-private LDS, in block order), sort them descending with a
        // 64-lane bitonic network, and read T at rank keep - c_hi.
        __shared__ uint32_t cand[kSelWaves][64];
        uint32_t* my = cand[threadIdx.x >> 6];
        uint32_t n = 0;
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const bool in = key[m] >= lo && key[m] <= hi;
            const uint64_t mask = __ballot(in);
            const uint32_t at = n + lanes_below(mask);
            if (in && at < 64u) my[at] = key[m];
            n += (uint32_t)__popcll(mask);
        }
        __builtin_amdgcn_wave_barrier();
        uint32_t v = lane < n ? my[lane] : 0u;  // 0 sorts below every key
#pragma unroll
        for (uint32_t k = 2; k <= 64; k <<= 1) {
#pragma unroll
            for (uint32_t j = k >> 1; j > 0; j >>= 1) {
                const uint32_t other = (uint32_t)__shfl_xor((int)v, (int)j, 64);
                const bool keep_max = ((lane & k) == 0) == ((lane & j) == 0);
                v = keep_max ? max(v, other) : min(v, other);
            }
        }
        T = __builtin_amdgcn_readlane(v, (int)(a.keep - c_hi - 1u));
        n_gt = c_hi + (uint32_t)__popcll(__ballot(v > T));
        n_ge = n_gt + (uint32_t)__popcll(__ballot(v == T));
    } else {
        T = lo;  // c_lo = count(key >= T)
        n_gt = T == 0xFFFFFFFFu ? 0u : count_ge(T + 1u);
        n_ge = c_lo;
    }
    const uint32_t need = a.keep - n_gt;  // keys equal to T to take, lowest blocks first

    int32_t* out = a.kv + (size_t)row * a.keep;
    uint32_t pos = 0, eq_seen = 0;
    if (n_ge == a.keep) {
        // every key equal to T is kept: the kept blocks are exactly key >= T
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const bool take = key[m] >= T;  // T >= 1: padding never matches
            const uint64_t take_mask = __ballot(take);
            const uint32_t at = pos + lanes_below(take_mask);
            if (take && at < a.keep) out[at] = (int32_t)(lane + 64u * m);
            pos += (uint32_t)__popcll(take_mask);
        }
        return;
    }
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const uint32_t j = lane + 64u * m;
        const bool gt = key[m] > T;
        const bool eq = key[m] == T;  // T >= 1: padding never matches
        const uint64_t eq_mask = __ballot(eq);
        const bool take = gt || (eq && eq_seen + lanes_below(eq_mask) < need);
        const uint64_t take_mask = __ballot(take);
        const uint32_t at = pos + lanes_below(take_mask);
        if (take && at < a.keep) out[at] = (int32_t)j;  // exactly keep are taken
        pos += (uint32_t)__popcll(take_mask);
        eq_seen += (uint32_t)__popcll(eq_mask);
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
    if (ceil_div(rows, block) > kMaxBlocks || heads > 4096) return H3F_ERR_UNSUPPORTED;
    // a sparsity within rounding of 1 could leave no block at all
    if (keep_for(ceil_div(rows, block), sparsity, step) < 1) return H3F_ERR_BAD_VALUE;
    return H3F_OK;
}

// Rows of scores lie scores_row_stride >= n_blocks floats apart, and one
// head's matrix is addressed with 32-bit byte offsets that must stay below
// the offset that marks a dropped store.
h3f_status_t check_scores_stride(int64_t nb, int64_t scores_row_stride) {
    if (scores_row_stride < nb) return H3F_ERR_BAD_STRIDE;
    if (scores_row_stride > (int64_t)kDropped / (4 * nb)) return H3F_ERR_UNSUPPORTED;
    return H3F_OK;
}

// Block scores from the pooled means, then the kept lists (routed steps).
void launch_score_select(const float* pooled, float* scores, int64_t scores_row_stride,
                         int32_t* kv_blocks, int32_t heads, int64_t nb, int64_t keep,
                         hipStream_t s) {
    ScoreArgs sa;
    sa.pooled = pooled;
    sa.scores = scores;
    sa.heads = heads;
    sa.nb = (uint32_t)nb;
    sa.ss = (uint32_t)scores_row_stride;
    sa.tiles = (uint32_t)((nb + kTile - 1) / kTile);
    const dim3 scg((unsigned)(heads * sa.tiles * ((sa.tiles + kScoreRun - 1) / kScoreRun)));
    if (nb % 4 == 0)
        hipLaunchKernelGGL(subblock_score_kernel<16>, scg, dim3(256), 0, s, sa);
    else if (nb % 2 == 0)
        hipLaunchKernelGGL(subblock_score_kernel<8>, scg, dim3(256), 0, s, sa);
    else
        hipLaunchKernelGGL(subblock_score_kernel<4>, scg, dim3(256), 0, s, sa);

    SelectArgs se;
    se.scores = scores;
    se.kv = kv_blocks;
    se.rows = (uint32_t)(heads * nb);
    se.nb = (uint32_t)nb;
    se.ss = (uint32_t)scores_row_stride;
    se.keep = (uint32_t)keep;
    se.z = normal_upper_quantile((double)keep / (double)nb);
    const dim3 sg((se.rows + kSelWaves - 1) / kSelWaves), sb(64 * kSelWaves);
    if (nb <= 64 * 4)
        hipLaunchKernelGGL(subblock_select_kernel<4>, sg, sb, 0, s, se);
    else if (nb <= 64 * 16)
        hipLaunchKernelGGL(subblock_select_kernel<16>, sg, sb, 0, s, se);
    else if (nb <= 64 * 32)
        hipLaunchKernelGGL(subblock_select_kernel<32>, sg, sb, 0, s, se);
    else
        hipLaunchKernelGGL(subblock_select_kernel<128>, sg, sb, 0, s, se);
}

// Every block kept (dense steps): kv[h, i, :] = 0 .. nb - 1.
h3f_status_t launch_dense(int32_t* kv_blocks, int32_t heads, int64_t nb, int64_t keep,
                          hipStream_t s) {
    const uint64_t total = (uint64_t)heads * nb * keep;
    const unsigned blocks = (unsigned)std::min<uint64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL(subblock_dense_kernel, dim3(blocks), dim3(256), 0, s, kv_blocks,
                       (uint32_t)nb, total);
    return hipGetLastError() == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
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
    const int64_t nb = ceil_div(rows, block);
    if (n_blocks) *n_blocks = (int32_t)nb;
    if (keep) *keep = (int32_t)keep_for(nb, sparsity, step);
    if (workspace_bytes) *workspace_bytes = workspace_for(nb, heads);
    return H3F_OK;
}

extern "C" h3f_status_t h3f_subblock_route(int32_t* kv_blocks, float* scores,
                                           int64_t scores_row_stride, const void* q,
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
    if (!aligned16(q) || !aligned16(k) || !aligned16(scores)) return H3F_ERR_MISALIGNED;
    if (reinterpret_cast<uintptr_t>(kv_blocks) & 3u) return H3F_ERR_MISALIGNED;
    constexpr int V = 8;
    constexpr int64_t kMaxStride = int64_t(1) << 31;  // keeps every span product in range
    if (std::max(q_row_stride, k_row_stride) > kMaxStride ||
        (heads > 1 && std::max(q_head_stride, k_head_stride) > kMaxStride))
        return H3F_ERR_UNSUPPORTED;
    if (q_row_stride % V || k_row_stride % V) return H3F_ERR_BAD_STRIDE;
    if (heads > 1 && (q_head_stride % V || k_head_stride % V || q_head_stride < head_dim ||
                      k_head_stride < head_dim))
        return H3F_ERR_BAD_STRIDE;
    const int64_t qhs = heads > 1 ? q_head_stride : head_dim;
    const int64_t khs = heads > 1 ? k_head_stride : head_dim;
    if (!extent_ok(heads, qhs, head_dim, 2) || !extent_ok(heads, khs, head_dim, 2))
        return H3F_ERR_UNSUPPORTED;
    const int64_t q_span = (int64_t)(heads - 1) * qhs + head_dim;
    const int64_t k_span = (int64_t)(heads - 1) * khs + head_dim;
    if (!extent_ok(rows, q_row_stride, q_span, 2) || !extent_ok(rows, k_row_stride, k_span, 2))
        return H3F_ERR_UNSUPPORTED;
    const Region rq = region2d(q, rows, q_row_stride, q_span, 2);
    const Region rk = region2d(k, rows, k_row_stride, k_span, 2);
    if (!rows_separate(rq) || !rows_separate(rk)) return H3F_ERR_BAD_STRIDE;
    // one block of rows (plus the rows an unrolled batch reads past its end,
    // which must stay outside the resource) is addressed with 32-bit offsets
    {
        const int64_t span_bytes = 2 * std::max(q_span, k_span);
        const int64_t block_rows = (int64_t)block + (kPoolUnroll + 1) * kPoolWaves;
        if (span_bytes >= 0xFFFFFFF0ll ||
            2 * std::max(q_row_stride, k_row_stride) > (0xFFFFFFF0ll - span_bytes - 1) / block_rows)
            return H3F_ERR_UNSUPPORTED;
    }

    const int64_t nb = ceil_div(rows, block);
    const int64_t keep = keep_for(nb, sparsity, step);
    const h3f_status_t sst = check_scores_stride(nb, scores_row_stride);
    if (sst != H3F_OK) return sst;
    const size_t need = workspace_for(nb, heads);
    const bool routed = step >= H3F_SUBBLOCK_FIRST_STEP;
    if (routed && (!workspace || !aligned16(workspace) || workspace_bytes < need))
        return H3F_ERR_WORKSPACE;
    const Region rkv = region2d(kv_blocks, 1, 0, (int64_t)heads * nb * keep * 4, 1);
    const Region rsc = region2d(scores, (int64_t)heads * nb, scores_row_stride, nb, 4);
    const Region rws = region2d(workspace, 1, 0, routed ? (int64_t)need : 0, 1);
    if (!disjoint(rkv, rq) || !disjoint(rkv, rk) || !disjoint(rkv, rws) ||
        (routed && (!disjoint(rkv, rsc) || !disjoint(rsc, rq) || !disjoint(rsc, rk) ||
                    !disjoint(rsc, rws) || !disjoint(rws, rq) || !disjoint(rws, rk))))
        return H3F_ERR_ALIASING;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!routed) return launch_dense(kv_blocks, heads, nb, keep, s);

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
    // flat streaming when both tensors are [rows, heads, 128] dense and a thread
    // needs at most 8 accumulator slots
    const uint32_t cpr = (uint32_t)heads * 16u;
    uint32_t gcd = kFlatThreads, c2 = cpr;
    while (c2) { const uint32_t r = gcd % c2; gcd = c2; c2 = r; }
    const uint32_t P = cpr / gcd, mult = (uint32_t)kFlatThreads / gcd;
    const bool dense = q_row_stride == (int64_t)heads * head_dim && k_row_stride == q_row_stride &&
                       qhs == head_dim && khs == head_dim;
    // the unrolled tail (at most 16 steps of 2 KiB) must stay within 32-bit offsets
    const bool fits = (int64_t)block * cpr * 16 + (2 * kFlatDepth + 1) * kFlatThreads * 16 < 0xFFFFFFF0ll;
    if (H3F_POOL_FLAT && dense && P <= 8 && fits) {
        const dim3 fg(2 * pa.n_blocks), fb(kFlatThreads);
        switch (P) {
            case 1: hipLaunchKernelGGL(subblock_pool_flat_kernel<1>, fg, fb, 0, s, pa, cpr, mult); break;
            case 2: hipLaunchKernelGGL(subblock_pool_flat_kernel<2>, fg, fb, 0, s, pa, cpr, mult); break;
            case 3: hipLaunchKernelGGL(subblock_pool_flat_kernel<3>, fg, fb, 0, s, pa, cpr, mult); break;
            case 4: hipLaunchKernelGGL(subblock_pool_flat_kernel<4>, fg, fb, 0, s, pa, cpr, mult); break;
            case 5: hipLaunchKernelGGL(subblock_pool_flat_kernel<5>, fg, fb, 0, s, pa, cpr, mult); break;
            case 6: hipLaunchKernelGGL(subblock_pool_flat_kernel<6>, fg, fb, 0, s, pa, cpr, mult); break;
            case 7: hipLaunchKernelGGL(subblock_pool_flat_kernel<7>, fg, fb, 0, s, pa, cpr, mult); break;
            default: hipLaunchKernelGGL(subblock_pool_flat_kernel<8>, fg, fb, 0, s, pa, cpr, mult); break;
        }
    } else {
        hipLaunchKernelGGL((subblock_pool_kernel<kPoolWaves, kPoolUnroll>),
                           dim3(2 * pa.n_blocks * pa.n_groups), dim3(64 * kPoolWaves), 0, s, pa);
    }

    launch_score_select(pa.pooled, scores, scores_row_stride, kv_blocks, heads, nb, keep, s);
    return hipGetLastError() == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}

extern "C" h3f_status_t h3f_subblock_route_pooled(int32_t* kv_blocks, float* scores,
                                                  int64_t scores_row_stride, int64_t rows,
                                                  int32_t heads, int32_t head_dim, int32_t block,
                                                  double sparsity, int32_t step,
                                                  const void* workspace, size_t workspace_bytes,
                                                  void* stream) {
    if (!kv_blocks || !scores) return H3F_ERR_NULL_POINTER;
    const h3f_status_t st = check_plan(rows, heads, head_dim, block, sparsity, step);
    if (st != H3F_OK) return st;
    if (!aligned16(scores)) return H3F_ERR_MISALIGNED;
    if (reinterpret_cast<uintptr_t>(kv_blocks) & 3u) return H3F_ERR_MISALIGNED;
    const int64_t nb = ceil_div(rows, block);
    const int64_t keep = keep_for(nb, sparsity, step);
    const h3f_status_t sst = check_scores_stride(nb, scores_row_stride);
    if (sst != H3F_OK) return sst;
    const size_t need = workspace_for(nb, heads);
    const bool routed = step >= H3F_SUBBLOCK_FIRST_STEP;
    if (routed && (!workspace || !aligned16(workspace) || workspace_bytes < need))
        return H3F_ERR_WORKSPACE;
    const Region rkv = region2d(kv_blocks, 1, 0, (int64_t)heads * nb * keep * 4, 1);
    const Region rsc = region2d(scores, (int64_t)heads * nb, scores_row_stride, nb, 4);
    const Region rws = region2d(workspace, 1, 0, routed ? (int64_t)need : 0, 1);
    if (!disjoint(rkv, rws) || (routed && (!disjoint(rkv, rsc) || !disjoint(rsc, rws))))
        return H3F_ERR_ALIASING;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!routed) return launch_dense(kv_blocks, heads, nb, keep, s);
    launch_score_select(static_cast<const float*>(workspace), scores, scores_row_stride, kv_blocks,
                        heads, nb, keep, s);
    return hipGetLastError() == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}
