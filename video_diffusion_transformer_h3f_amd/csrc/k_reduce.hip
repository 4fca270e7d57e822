// k_reduce.hip -- relative L1 residual difference (step-reuse test).
//
// Design (gfx950): a pure two-stream read.  Stage 1: the [rows, cols] problem
// is flattened into 16-byte chunks; a 256-thread workgroup owns 256 * U
// consecutive chunks (U = 8: 16 loads in flight per lane; reads stream well at
// this depth, unlike read-write kernels), accumulates |cur - prev| and |prev|
// in fp32 per lane, reduces them inside each wavefront with DPP, across its
// four wavefronts through LDS in fixed order, and writes one fp64 pair to the
// workspace.  Stage 2: one workgroup adds the pairs in index order in fp64.
// The partition depends only on the shape, so the result is bit-identical run
// to run; no atomics.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "h3f_device.hpp"
#include "h3f_validate.hpp"

namespace h3f {
namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 8;
constexpr int kTile = kBlock * kUnroll;
constexpr int64_t kMaxChunks = (int64_t(1) << 31) - kTile;

struct Stream2 {
    const char* base;
    int64_t stride;  // bytes
    int64_t rows;
    int32_t row_bytes;
};

__device__ __forceinline__ rsrc_t tile_rsrc2(const Stream2& s, uint32_t r0) {
    return make_rsrc(s.base + (int64_t)r0 * s.stride,
                     span_bytes(s.rows - (int64_t)r0, s.stride, s.row_bytes));
}

template <typename T, int VEC>
__global__ void __launch_bounds__(kBlock)
residual_l1_partial(Stream2 cs, Stream2 ps, FastDiv div_cols, uint32_t n_chunks,
                    double* __restrict__ partial) {
    __shared__ float red[2][kBlock / 64];
    const uint32_t tile0 = blockIdx.x * (uint32_t)kTile;
    const uint32_t row0 = fdiv(tile0, div_cols);
    const rsrc_t rc = tile_rsrc2(cs, row0);
    const rsrc_t rp = tile_rsrc2(ps, row0);
    Vec<T, VEC> cv[kUnroll], pv[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t idx = tile0 + u * kBlock + threadIdx.x;
        ok[u] = idx < n_chunks;
        const uint32_t row = fdiv(idx, div_cols);
        const uint32_t cb = (idx - row * div_cols.d) * (uint32_t)(VEC * sizeof(T));
        if (ok[u]) {
            cv[u].template load_buf<kLoadStream>(rc, (row - row0) * (uint32_t)cs.stride + cb);
            pv[u].template load_buf<kLoadStream>(rp, (row - row0) * (uint32_t)ps.stride + cb);
        } else {
            cv[u].zero();
            pv[u].zero();
        }
    }
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        float c[VEC], p[VEC];
        cv[u].to_float(c);
        pv[u].to_float(p);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            num += fabsf(c[i] - p[i]);
            den += fabsf(p[i]);
        }
    }
    num = wave_sum(num);
    den = wave_sum(den);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][w] = num;
        red[1][w] = den;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double n = 0.0, d = 0.0;
#pragma unroll
        for (int k = 0; k < kBlock / 64; ++k) {
            n += (double)red[0][k];
            d += (double)red[1][k];
        }
        partial[2 * (size_t)blockIdx.x] = n;
        partial[2 * (size_t)blockIdx.x + 1] = d;
    }
}

// One workgroup of kFinal threads: thread t adds pairs t, t + kFinal, ... in
// order (4 independent accumulators, combined in fixed order, so the loads
// overlap); then a fixed tree over the kFinal partial sums in LDS.
constexpr int kFinal = 1024;
__global__ void __launch_bounds__(kFinal)
residual_l1_final(const double* __restrict__ partial, int64_t n_pairs, double* __restrict__ out) {
    __shared__ double sn[kFinal], sd[kFinal];
    double n[4] = {0.0, 0.0, 0.0, 0.0}, d[4] = {0.0, 0.0, 0.0, 0.0};
    int64_t i = threadIdx.x;
    for (; i + 3 * kFinal < n_pairs; i += 4 * kFinal) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            n[k] += partial[2 * (i + k * kFinal)];
            d[k] += partial[2 * (i + k * kFinal) + 1];
        }
    }
    for (int k = 0; i < n_pairs; i += kFinal, ++k) {
        n[k] += partial[2 * i];
        d[k] += partial[2 * i + 1];
    }
    sn[threadIdx.x] = (n[0] + n[1]) + (n[2] + n[3]);
    sd[threadIdx.x] = (d[0] + d[1]) + (d[2] + d[3]);
    __syncthreads();
    for (int s = kFinal / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            sn[threadIdx.x] += sn[threadIdx.x + s];
            sd[threadIdx.x] += sd[threadIdx.x + s];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        out[0] = sn[0];
        out[1] = sd[0];
        out[2] = sn[0] / sd[0];
    }
}

inline int64_t n_partials(int64_t rows, int64_t cpr) {
    // launches of at most kMaxChunks chunks, each split into kTile tiles
    const int64_t rows_per_launch = std::max<int64_t>(1, kMaxChunks / cpr);
    int64_t total = 0;
    for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
        const int64_t nr = std::min(rows - r0, rows_per_launch);
        total += (nr * cpr + kTile - 1) / kTile;
    }
    return total;
}

inline bool tile_fits2(int64_t cpr, int64_t stride_bytes, int64_t row_bytes) {
    // (kTile / cpr + 2) * stride_bytes + row_bytes < 0xFFFFFFF0, without overflow
    if (row_bytes >= 0xFFFFFFF0ll) return false;
    return stride_bytes <= (0xFFFFFFF0ll - row_bytes - 1) / (kTile / cpr + 2);
}

template <typename T, int VEC>
hipError_t launch_l1(double* out, const void* cur, int64_t c_rs, const void* prev, int64_t p_rs,
                     int64_t rows, int64_t hidden, double* partial, hipStream_t st) {
    const int64_t cpr = hidden / VEC;
    const int64_t rows_per_launch = std::max<int64_t>(1, kMaxChunks / cpr);
    int64_t done = 0;
    for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
        const int64_t nr = std::min(rows - r0, rows_per_launch);
        const uint32_t n = (uint32_t)(nr * cpr);
        const unsigned blocks = (unsigned)((n + kTile - 1) / kTile);
        Stream2 cs{static_cast<const char*>(cur) + r0 * c_rs * (int64_t)sizeof(T),
                   c_rs * (int64_t)sizeof(T), nr, (int32_t)(hidden * sizeof(T))};
        Stream2 ps{static_cast<const char*>(prev) + r0 * p_rs * (int64_t)sizeof(T),
                   p_rs * (int64_t)sizeof(T), nr, (int32_t)(hidden * sizeof(T))};
        hipLaunchKernelGGL((residual_l1_partial<T, VEC>), dim3(blocks), dim3(kBlock), 0, st, cs,
                           ps, make_fastdiv((uint32_t)cpr), n, partial + 2 * done);
        done += blocks;
    }
    hipLaunchKernelGGL(residual_l1_final, dim3(1), dim3(kFinal), 0, st, partial, done, out);
    return hipGetLastError();
}

}  // namespace
}  // namespace h3f

using namespace h3f;

extern "C" size_t h3f_residual_l1_workspace_bytes(int64_t rows, int64_t hidden,
                                                  h3f_dtype_t dtype) {
    if (rows <= 0 || hidden <= 0 || !dtype_ok(dtype)) return 0;
    const int V = vec_width(dtype == H3F_F32);
    if (hidden % V) return 0;
    if (rows > 0x7fffffff || hidden / V > 0x7fffffff) return 0;  // sizes the call rejects
    return (size_t)n_partials(rows, hidden / V) * 2 * sizeof(double);
}

namespace {

// Checks shared by the workspace and the no-allocation entry points; on success
// *cs / *ps hold the row strides the kernels use.
h3f_status_t l1_validate(const double* out, const void* cur, int64_t cur_row_stride,
                         const void* prev, int64_t prev_row_stride, h3f_dtype_t dtype,
                         int64_t rows, int64_t hidden, int64_t* cs_out, int64_t* ps_out) {
    if (!out) return H3F_ERR_NULL_POINTER;
    if (rows < 0 || hidden <= 0) return H3F_ERR_BAD_SHAPE;
    if (rows == 0) return H3F_ERR_BAD_SHAPE;  // the relative difference needs at least one element
    if (!cur || !prev) return H3F_ERR_NULL_POINTER;
    if (!dtype_ok(dtype)) return H3F_ERR_BAD_DTYPE;
    const int V = vec_width(dtype == H3F_F32);
    if (hidden % V) return H3F_ERR_BAD_SHAPE;
    if (rows > 0x7fffffff || hidden / V > 0x7fffffff) return H3F_ERR_UNSUPPORTED;
    if (!aligned16(cur) || !aligned16(prev)) return H3F_ERR_MISALIGNED;
    if ((reinterpret_cast<uintptr_t>(out) & 7u) != 0) return H3F_ERR_MISALIGNED;
    if (rows > 1 && (cur_row_stride % V || prev_row_stride % V)) return H3F_ERR_BAD_STRIDE;
    const int e = dtype_bytes(dtype);
    const int64_t cs = rows > 1 ? cur_row_stride : hidden;
    const int64_t ps = rows > 1 ? prev_row_stride : hidden;
    if (!extent_ok(rows, cs, hidden, e) || !extent_ok(rows, ps, hidden, e)) return H3F_ERR_UNSUPPORTED;
    const Region rc = region2d(cur, rows, cs, hidden, e);
    const Region rp = region2d(prev, rows, ps, hidden, e);
    if (!rows_separate(rc) || !rows_separate(rp)) return H3F_ERR_BAD_STRIDE;
    if (!tile_fits2(hidden / V, cs * e, hidden * e) || !tile_fits2(hidden / V, ps * e, hidden * e))
        return H3F_ERR_UNSUPPORTED;
    const Region ro = region2d(out, 1, 0, 3 * sizeof(double), 1);
    if (!disjoint(ro, rc) || !disjoint(ro, rp)) return H3F_ERR_ALIASING;
    *cs_out = cs;
    *ps_out = ps;
    return H3F_OK;
}

h3f_status_t l1_launch(double* out, const void* cur, int64_t cs, const void* prev, int64_t ps,
                       h3f_dtype_t dtype, int64_t rows, int64_t hidden, double* partial,
                       void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t err =
        dtype == H3F_BF16
            ? launch_l1<__bf16, 8>(out, cur, cs, prev, ps, rows, hidden, partial, st)
            : launch_l1<float, 4>(out, cur, cs, prev, ps, rows, hidden, partial, st);
    return err == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// Library-owned scratch for h3f_residual_l1_noalloc: the per-workgroup partial
// sums live in this file-scope device array instead of a caller workspace.
// Each GPU the library runs on holds its own copy until the process ends.  Host
// code never passes the array's name to a kernel or a copy (on the host it is
// only a stand-in symbol): the device address is taken once per device with
// hipGetSymbolAddress, with that device current, and that address is used.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(4) << 20;  // 262,144 (sum, sum) pairs
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, or nullptr on failure.
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" h3f_status_t h3f_residual_l1(double* out, const void* cur, int64_t cur_row_stride,
                                        const void* prev, int64_t prev_row_stride,
                                        h3f_dtype_t dtype, int64_t rows, int64_t hidden,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    int64_t cs = 0, ps = 0;
    const h3f_status_t s = l1_validate(out, cur, cur_row_stride, prev, prev_row_stride, dtype,
                                       rows, hidden, &cs, &ps);
    if (s != H3F_OK) return s;
    const int e = dtype_bytes(dtype);
    const size_t need = h3f_residual_l1_workspace_bytes(rows, hidden, dtype);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return H3F_ERR_WORKSPACE;
    const Region rw = region2d(workspace, 1, 0, (int64_t)need, 1);
    const Region ro = region2d(out, 1, 0, 3 * sizeof(double), 1);
    if (!disjoint(rw, region2d(cur, rows, cs, hidden, e)) ||
        !disjoint(rw, region2d(prev, rows, ps, hidden, e)) || !disjoint(ro, rw))
        return H3F_ERR_ALIASING;
    return l1_launch(out, cur, cs, prev, ps, dtype, rows, hidden, static_cast<double*>(workspace),
                     stream);
}

extern "C" size_t h3f_residual_l1_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" h3f_status_t h3f_residual_l1_noalloc(double* out, const void* cur,
                                                int64_t cur_row_stride, const void* prev,
                                                int64_t prev_row_stride, h3f_dtype_t dtype,
                                                int64_t rows, int64_t hidden, void* stream) {
    int64_t cs = 0, ps = 0;
    const h3f_status_t s = l1_validate(out, cur, cur_row_stride, prev, prev_row_stride, dtype,
                                       rows, hidden, &cs, &ps);
    if (s != H3F_OK) return s;
    if (h3f_residual_l1_workspace_bytes(rows, hidden, dtype) > kScratchBytes)
        return H3F_ERR_WORKSPACE;  // more partial sums than the library's scratch holds
    void* partial = scratch_for_current_device();
    if (!partial) return H3F_ERR_LAUNCH;
    // every partial pair is written by the first kernel before the second reads it,
    // so the scratch needs no clearing between calls
    return l1_launch(out, cur, cs, prev, ps, dtype, rows, hidden, static_cast<double*>(partial),
                     stream);
}
