// k_elementwise.hip -- streaming operators of libh3fused: gated residual,
// SwiGLU, and the streaming-copy measurement helper.
//
// Design (gfx950): the [rows, cols] problem is flattened into row-major
// vector chunks of VEC elements (one 16-byte quad for bf16, one or two for
// fp32).  A 256-thread workgroup owns 256 * UNROLL consecutive chunks; thread
// t takes chunks base + t + 256 * u, so each wavefront instruction touches 64
// consecutive chunks (1 KiB of bf16) and every thread keeps UNROLL
// independent loads per stream in flight before it computes.  Row / column of
// a chunk come from one multiply-high division by the row length; the
// broadcast modulation row comes from a second division by rows_per_group.
// Streams touched once use non-temporal loads and stores.
#include <hip/hip_runtime.h>

#include "h3f_device.hpp"
#include "h3f_validate.hpp"

namespace h3f {
namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 4;
// Largest number of chunks one launch indexes with 32-bit arithmetic.
constexpr int64_t kMaxChunksPerLaunch = (int64_t(1) << 31) - kBlock * kUnroll;

// ---------------------------------------------------------------------------
// Gated residual: x[r, :] += gate[g(r), :] * h[r, :]   (fp32 arithmetic)
// ---------------------------------------------------------------------------
template <typename TX, typename TH, int VEC>
__global__ void __launch_bounds__(kBlock)
gated_residual_kernel(TX* __restrict__ x, int64_t x_rs, const TH* __restrict__ h, int64_t h_rs,
                      const TX* __restrict__ gate, int64_t gate_gs, FastDiv div_cols,
                      FastDiv div_group, uint32_t row_base, uint32_t n_chunks) {
    const uint32_t base = blockIdx.x * (uint32_t)(kBlock * kUnroll) + threadIdx.x;
    Vec<TX, VEC> xv[kUnroll];
    Vec<TH, VEC> hv[kUnroll];
    Vec<TX, VEC> gv[kUnroll];
    int64_t xoff[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t idx = base + u * kBlock;
        ok[u] = idx < n_chunks;
        const uint32_t row = fdiv(idx, div_cols);
        const uint32_t col = (idx - row * div_cols.d) * VEC;
        const uint32_t grp = fdiv(row_base + row, div_group);
        xoff[u] = (int64_t)row * x_rs + col;
        if (ok[u]) {
            xv[u].template load<true>(x + xoff[u]);
            hv[u].template load<true>(h + (int64_t)row * h_rs + col);
            gv[u].template load<false>(gate + (int64_t)grp * gate_gs + col);
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (!ok[u]) continue;
        float xf[VEC], hf[VEC], gf[VEC];
        xv[u].to_float(xf);
        hv[u].to_float(hf);
        gv[u].to_float(gf);
#pragma unroll
        for (int i = 0; i < VEC; ++i) xf[i] = __builtin_fmaf(gf[i], hf[i], xf[i]);
        xv[u].from_float(xf);
        xv[u].template store<true>(x + xoff[u]);
    }
}

// ---------------------------------------------------------------------------
// SwiGLU: out = a * sigmoid(a) * b.  sigmoid via the hardware exp2 (v_exp_f32)
// and reciprocal (v_rcp_f32): a / (1 + 2^(-a log2 e)).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float silu_f(float a) {
    const float e = __builtin_amdgcn_exp2f(-a * 1.4426950408889634f);
    return a * __builtin_amdgcn_rcpf(1.0f + e);
}

template <typename T, int VEC>
__global__ void __launch_bounds__(kBlock)
swiglu_kernel(T* __restrict__ out, int64_t o_rs, const T* __restrict__ a, int64_t a_rs,
              const T* __restrict__ b, int64_t b_rs, FastDiv div_cols, uint32_t n_chunks) {
    const uint32_t base = blockIdx.x * (uint32_t)(kBlock * kUnroll) + threadIdx.x;
    Vec<T, VEC> av[kUnroll], bv[kUnroll];
    int64_t ooff[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t idx = base + u * kBlock;
        ok[u] = idx < n_chunks;
        const uint32_t row = fdiv(idx, div_cols);
        const uint32_t col = (idx - row * div_cols.d) * VEC;
        ooff[u] = (int64_t)row * o_rs + col;
        if (ok[u]) {
            av[u].template load<true>(a + (int64_t)row * a_rs + col);
            bv[u].template load<true>(b + (int64_t)row * b_rs + col);
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (!ok[u]) continue;
        float af[VEC], bf[VEC], of[VEC];
        av[u].to_float(af);
        bv[u].to_float(bf);
#pragma unroll
        for (int i = 0; i < VEC; ++i) of[i] = silu_f(af[i]) * bf[i];
        Vec<T, VEC> ov;
        ov.from_float(of);
        ov.template store<true>(out + ooff[u]);
    }
}

// ---------------------------------------------------------------------------
// Streaming copy (measurement helper).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBlock)
stream_copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, uint64_t n_quads) {
    const uint64_t base = (uint64_t)blockIdx.x * (kBlock * kUnroll) + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint64_t i = base + (uint64_t)u * kBlock;
        if (i < n_quads) v[u] = ld16_nt(src + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint64_t i = base + (uint64_t)u * kBlock;
        if (i < n_quads) st16_nt(dst + i, v[u]);
    }
}

inline unsigned blocks_for(int64_t chunks) {
    return (unsigned)((chunks + kBlock * kUnroll - 1) / (kBlock * kUnroll));
}

// Rows per launch so that rows * chunks_per_row stays inside 32-bit indexing.
inline int64_t rows_per_launch(int64_t chunks_per_row) {
    int64_t r = kMaxChunksPerLaunch / chunks_per_row;
    return r < 1 ? 1 : r;
}

template <typename TX, typename TH, int VEC>
h3f_status_t launch_gated(void* x, int64_t x_rs, const void* h, int64_t h_rs, const void* gate,
                          int64_t gate_gs, int64_t rows_per_group, int64_t rows, int64_t hidden,
                          hipStream_t st) {
    const int64_t cpr = hidden / VEC;
    const int64_t step = rows_per_launch(cpr);
    const int64_t rpg = rows_per_group > rows ? rows : rows_per_group;
    for (int64_t r0 = 0; r0 < rows; r0 += step) {
        const int64_t nr = rows - r0 < step ? rows - r0 : step;
        const uint32_t n = (uint32_t)(nr * cpr);
        hipLaunchKernelGGL((gated_residual_kernel<TX, TH, VEC>), dim3(blocks_for(n)), dim3(kBlock),
                           0, st, static_cast<TX*>(x) + r0 * x_rs, x_rs,
                           static_cast<const TH*>(h) + r0 * h_rs, h_rs,
                           static_cast<const TX*>(gate), gate_gs, make_fastdiv((uint32_t)cpr),
                           make_fastdiv((uint32_t)rpg), (uint32_t)r0, n);
    }
    return hipGetLastError() == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}

template <typename T, int VEC>
h3f_status_t launch_swiglu(void* out, int64_t o_rs, const void* a, int64_t a_rs, const void* b,
                           int64_t b_rs, int64_t rows, int64_t inner, hipStream_t st) {
    const int64_t cpr = inner / VEC;
    const int64_t step = rows_per_launch(cpr);
    for (int64_t r0 = 0; r0 < rows; r0 += step) {
        const int64_t nr = rows - r0 < step ? rows - r0 : step;
        const uint32_t n = (uint32_t)(nr * cpr);
        hipLaunchKernelGGL((swiglu_kernel<T, VEC>), dim3(blocks_for(n)), dim3(kBlock), 0, st,
                           static_cast<T*>(out) + r0 * o_rs, o_rs,
                           static_cast<const T*>(a) + r0 * a_rs, a_rs,
                           static_cast<const T*>(b) + r0 * b_rs, b_rs,
                           make_fastdiv((uint32_t)cpr), n);
    }
    return hipGetLastError() == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}

}  // namespace
}  // namespace h3f

using namespace h3f;

extern "C" h3f_status_t h3f_gated_residual(void* x, h3f_dtype_t x_dtype, int64_t x_row_stride,
                                           const void* h, h3f_dtype_t h_dtype,
                                           int64_t h_row_stride, const void* gate,
                                           int64_t gate_group_stride, int64_t rows_per_group,
                                           int64_t rows, int64_t hidden, void* stream) {
    if (rows == 0) return H3F_OK;
    if (!x || !h || !gate) return H3F_ERR_NULL_POINTER;
    if (!dtype_ok(x_dtype) || !dtype_ok(h_dtype)) return H3F_ERR_BAD_DTYPE;
    if (x_dtype == H3F_BF16 && h_dtype == H3F_F32) return H3F_ERR_BAD_DTYPE;
    if (rows < 0 || hidden <= 0 || rows_per_group < 1) return H3F_ERR_BAD_SHAPE;
    if (rows > 0x7fffffff) return H3F_ERR_UNSUPPORTED;
    const int V = vec_width(x_dtype == H3F_BF16 || h_dtype == H3F_BF16);
    if (hidden % V) return H3F_ERR_BAD_SHAPE;
    if (hidden / V > 0x7fffffff) return H3F_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(h) || !aligned16(gate)) return H3F_ERR_MISALIGNED;
    const int64_t groups = groups_for(rows, rows_per_group);
    if ((rows > 1 && (x_row_stride % V || h_row_stride % V)) ||
        (groups > 1 && gate_group_stride % V))
        return H3F_ERR_BAD_STRIDE;
    const int ex = dtype_bytes(x_dtype), eh = dtype_bytes(h_dtype);
    const Region rx = region2d(x, rows, x_row_stride, hidden, ex);
    const Region rh = region2d(h, rows, h_row_stride, hidden, eh);
    const Region rg = region2d(gate, groups, gate_group_stride, hidden, ex);
    if (!rows_separate(rx) || !rows_separate(rh) || !rows_separate(rg)) return H3F_ERR_BAD_STRIDE;
    if (!disjoint(rx, rh) || !disjoint(rx, rg)) return H3F_ERR_ALIASING;
    const int64_t xs = rows > 1 ? x_row_stride : hidden;
    const int64_t hs = rows > 1 ? h_row_stride : hidden;
    const int64_t gs = groups > 1 ? gate_group_stride : 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (x_dtype == H3F_F32 && h_dtype == H3F_F32)
        return launch_gated<float, float, 4>(x, xs, h, hs, gate, gs, rows_per_group, rows, hidden,
                                             st);
    if (x_dtype == H3F_BF16)
        return launch_gated<__bf16, __bf16, 8>(x, xs, h, hs, gate, gs, rows_per_group, rows,
                                               hidden, st);
    return launch_gated<float, __bf16, 8>(x, xs, h, hs, gate, gs, rows_per_group, rows, hidden,
                                          st);
}

extern "C" h3f_status_t h3f_swiglu(void* out, int64_t out_row_stride, const void* a,
                                   int64_t a_row_stride, const void* b, int64_t b_row_stride,
                                   h3f_dtype_t dtype, int64_t rows, int64_t inner, void* stream) {
    if (rows == 0) return H3F_OK;
    if (!out || !a || !b) return H3F_ERR_NULL_POINTER;
    if (!dtype_ok(dtype)) return H3F_ERR_BAD_DTYPE;
    if (rows < 0 || inner <= 0) return H3F_ERR_BAD_SHAPE;
    const int V = vec_width(dtype == H3F_BF16);
    if (inner % V) return H3F_ERR_BAD_SHAPE;
    if (inner / V > 0x7fffffff) return H3F_ERR_UNSUPPORTED;
    if (!aligned16(out) || !aligned16(a) || !aligned16(b)) return H3F_ERR_MISALIGNED;
    if (rows > 1 && (out_row_stride % V || a_row_stride % V || b_row_stride % V))
        return H3F_ERR_BAD_STRIDE;
    const int e = dtype_bytes(dtype);
    const Region ro = region2d(out, rows, out_row_stride, inner, e);
    const Region ra = region2d(a, rows, a_row_stride, inner, e);
    const Region rb = region2d(b, rows, b_row_stride, inner, e);
    if (!rows_separate(ro) || !rows_separate(ra) || !rows_separate(rb)) return H3F_ERR_BAD_STRIDE;
    if (!alias_ok(ro, ra, true) || !alias_ok(ro, rb, true)) return H3F_ERR_ALIASING;
    const int64_t os = rows > 1 ? out_row_stride : inner;
    const int64_t as = rows > 1 ? a_row_stride : inner;
    const int64_t bs = rows > 1 ? b_row_stride : inner;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == H3F_BF16)
        return launch_swiglu<__bf16, 8>(out, os, a, as, b, bs, rows, inner, st);
    return launch_swiglu<float, 4>(out, os, a, as, b, bs, rows, inner, st);
}

extern "C" h3f_status_t h3f_stream_copy(void* dst, const void* src, int64_t bytes, void* stream) {
    if (bytes == 0) return H3F_OK;
    if (!dst || !src) return H3F_ERR_NULL_POINTER;
    if (bytes < 0 || bytes % 16) return H3F_ERR_BAD_SHAPE;
    if (!aligned16(dst) || !aligned16(src)) return H3F_ERR_MISALIGNED;
    const Region rd = region2d(dst, 1, 0, bytes, 1);
    const Region rs = region2d(src, 1, 0, bytes, 1);
    if (!disjoint(rd, rs)) return H3F_ERR_ALIASING;
    const uint64_t n = (uint64_t)bytes / 16;
    const uint64_t blocks = (n + kBlock * kUnroll - 1) / (kBlock * kUnroll);
    if (blocks > 0xffffffffull) return H3F_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), static_cast<u32x4*>(dst),
                       static_cast<const u32x4*>(src), n);
    return hipGetLastError() == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}
