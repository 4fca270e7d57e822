// k_adaln.hip -- AdaLN modulate and the fused gated residual + AdaLN.
//
// Design (gfx950): one 64-wide wavefront owns one token row and keeps the
// whole row in VGPRs (NV chunks of VEC elements per lane; hidden 5120 bf16 is
// 10 x 16-byte quads per lane).  x is read from HBM exactly once: the mean and
// then the centred second moment are reduced from registers (DPP / swizzle
// inside the wave, no LDS, no barrier), and the normalised, modulated row is
// written once.  The fused variant first applies the gated residual to the
// registers, rounds to x's storage type, writes x back, and normalises that
// stored value -- so it reads x once instead of twice.
// Modulation vectors: when the whole call uses one group (the usual case: one
// precomputed AdaLN vector set per sample), each workgroup stages them once
// in LDS and its wavefronts read them from there; otherwise every row reads
// its group's vectors through the cache hierarchy (L1/L2, not HBM).
// Measured on MI355X: one row per wavefront, no grid-stride reuse, is the
// fastest organisation (multi-wavefront rows pay more in barriers or in
// modulation staging than they gain in finer-grained streaming).  What sets
// its time is the 10 KiB (hidden 5120, bf16) each wavefront stores: a
// wavefront that stores 10 KiB writes at about 5.5 TB/s against 7.1 TB/s at
// 1 KiB, and reading the row bytes at the read-only rate then writing them at
// that rate gives the time the kernel takes.  The order in which a wavefront issues its
// row loads matters by ~3%: they go out strictly in address order (scheduling
// barriers keep the compiler from interleaving them).  The plain kernel stages
// the modulation first and then issues a bf16 row at raised wave priority, so
// a wavefront's loads leave back to back; the fused kernel, which has twice the
// loads per row, instead issues x before the staging so that the row's latency
// overlaps the staging and the barrier.  Each choice was the faster of the two
// for its kernel (about 5% each at hidden 5120).
#include <hip/hip_runtime.h>

#include "h3f_device.hpp"
#include "h3f_validate.hpp"

namespace h3f {
namespace {

#ifndef H3F_ADALN_WAVES
#define H3F_ADALN_WAVES 4
#endif
constexpr int kWaves = H3F_ADALN_WAVES;  // wavefronts (= rows) per workgroup

struct AdalnArgs {
    void* y;
    int64_t y_rs;  // bytes
    void* x;
    int64_t x_rs;  // bytes
    const void* h;
    int64_t h_rs;  // bytes
    const void* gate;
    const void* shift;
    const void* scale;
    const void* gamma;  // LayerNorm affine gain and bias, [hidden], shared by all rows
    const void* beta;
    int64_t mod_gs;  // bytes
    FastDiv div_group;
    int64_t rows;
    int32_t nvec;  // hidden / VEC
    int32_t hidden;
    float inv_hidden;
    float eps;
};

// Modulation vector chunk c of group grp: from LDS (staged, single group) or memory.
template <typename TX, int VEC, bool LDSMOD>
struct ModSource {
    static constexpr int Q = Vec<TX, VEC>::kQuads;
    const u32x4* lds;  // [n_vectors][nvec * Q]
    int32_t nvec;
    rsrc_t r[4];
    __device__ __forceinline__ void get(int which, uint32_t c, Vec<TX, VEC>& v) const {
        if constexpr (LDSMOD) {
#pragma unroll
            for (int k = 0; k < Q; ++k) v.q[k] = lds[(which * nvec + c) * Q + k];
        } else {
            v.template load_buf<kLoadReuse>(r[which], c * (VEC * sizeof(TX)));
        }
    }
};

extern __shared__ u32x4 adaln_lds[];

// Copies group 0's NMOD modulation vectors (nvec chunks of Q quads each) into
// LDS; every thread of the workgroup must call it (it ends with a barrier).
template <int NMOD, int Q, int NTHREADS>
__device__ __forceinline__ void stage_mods(const void* const* mods, int32_t nvec) {
    const int per = nvec * Q;
    for (int i = threadIdx.x; i < NMOD * per; i += NTHREADS) {
        const int which = i / per;
        adaln_lds[i] = ld16(static_cast<const char*>(mods[which]) + (size_t)(i - which * per) * 16);
    }
    __syncthreads();
}

// Vectors read per row: shift, scale, then gate (FUSED) or gamma, beta (AFFINE).
template <typename TX, typename TY, typename TH, int VEC, int NV, bool FUSED, bool LDSMOD,
          bool AFFINE>
__global__ void __launch_bounds__(kWaves * 64) adaln_kernel(AdalnArgs a) {
    static_assert(!(FUSED && AFFINE), "the fused form has no LayerNorm affine");
    constexpr int Q = Vec<TX, VEC>::kQuads;
    constexpr int NMOD = FUSED ? 3 : (AFFINE ? 4 : 2);
    const int lane = threadIdx.x & 63;
    const uint32_t xrow_bytes = (uint32_t)a.hidden * sizeof(TX);
    const void* mods[4] = {a.shift, a.scale, FUSED ? a.gate : a.gamma, a.beta};

    ModSource<TX, VEC, LDSMOD> ms;
    ms.nvec = a.nvec;
    ms.lds = adaln_lds;
    // the fused kernel stages after issuing its x loads (see the file comment)
    constexpr bool kStageLate = LDSMOD && FUSED;
    if constexpr (LDSMOD && !kStageLate) stage_mods<NMOD, Q, kWaves * 64>(mods, a.nvec);

    const int64_t row_raw = uniform64((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6));
    if constexpr (!kStageLate)
        if (row_raw >= a.rows) return;
    // with late staging a spare wavefront of the last workgroup must still reach
    // the barrier: it loads the last row again and returns before any store
    const int64_t row = row_raw < a.rows ? row_raw : a.rows - 1;
    const uint32_t grp = fdiv((uint32_t)row, a.div_group);
    if constexpr (!LDSMOD) {
#pragma unroll
        for (int m = 0; m < NMOD; ++m) {
            const bool shared = AFFINE && m >= 2;  // gamma, beta: one row for every group
            ms.r[m] = make_rsrc(static_cast<const char*>(mods[m]) + (shared ? 0 : grp * a.mod_gs),
                                xrow_bytes);
        }
    }
    char* xr = static_cast<char*>(a.x) + row * a.x_rs;
    const rsrc_t rx = make_rsrc(xr, xrow_bytes);
    float v[NV][VEC];
    bool valid[NV];
    {
        Vec<TX, VEC> xv[NV];
        // raised priority pays for bf16 rows (10 loads at hidden 5120) and costs ~2%
        // for fp32 rows (20 loads), which keep the default
        constexpr bool kPrio = !FUSED && sizeof(TX) == 2;
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(3);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = i * 64 + lane;
            valid[i] = c < a.nvec;
            xv[i].template load_buf<kLoadStream>(rx, (uint32_t)c * (VEC * sizeof(TX)));
            __builtin_amdgcn_sched_barrier(0);  // keep the loads in address order
        }
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
        if constexpr (kStageLate) {
            stage_mods<NMOD, Q, kWaves * 64>(mods, a.nvec);
            if (row_raw >= a.rows) return;
        }
        if constexpr (FUSED) {
            const rsrc_t rh = make_rsrc(static_cast<const char*>(a.h) + row * a.h_rs,
                                        (uint32_t)a.hidden * sizeof(TH));
            Vec<TH, VEC> hv[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i)
                hv[i].template load_buf<kLoadStream>(rh, (uint32_t)(i * 64 + lane) * (VEC * sizeof(TH)));
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const uint32_t c = i * 64 + lane;
                Vec<TX, VEC> gv;
                if (valid[i]) ms.get(2, c, gv); else gv.zero();
                float xf[VEC], hf[VEC], gf[VEC];
                xv[i].to_float(xf);
                hv[i].to_float(hf);
                gv.to_float(gf);
#pragma unroll
                for (int j = 0; j < VEC; ++j) xf[j] = __builtin_fmaf(gf[j], hf[j], xf[j]);
                xv[i].from_float(xf);  // round to x's storage type
                xv[i].template store_buf<kStoreStream>(rx, c * (VEC * sizeof(TX)));
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) xv[i].to_float(v[i]);
    }

    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < VEC; ++j) s += v[i][j];
    const float mean = wave_sum(s) * a.inv_hidden;

    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (!valid[i]) continue;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const float d = v[i][j] - mean;
            ss = __builtin_fmaf(d, d, ss);
        }
    }
    const float var = wave_sum(ss) * a.inv_hidden;
    const float rstd = __builtin_amdgcn_rsqf(var + a.eps);

    const rsrc_t ry = make_rsrc(static_cast<char*>(a.y) + row * a.y_rs,
                                (uint32_t)a.hidden * sizeof(TY));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (!valid[i]) continue;
        const uint32_t c = i * 64 + lane;
        Vec<TX, VEC> shv, scv;
        ms.get(0, c, shv);
        ms.get(1, c, scv);
        float sh[VEC], sc[VEC], o[VEC];
        shv.to_float(sh);
        scv.to_float(sc);
#pragma unroll
        for (int j = 0; j < VEC; ++j) o[j] = (v[i][j] - mean) * rstd;
        if constexpr (AFFINE) {
            Vec<TX, VEC> gmv, btv;
            ms.get(2, c, gmv);
            ms.get(3, c, btv);
            float gm[VEC], bt[VEC];
            gmv.to_float(gm);
            btv.to_float(bt);
#pragma unroll
            for (int j = 0; j < VEC; ++j) o[j] = __builtin_fmaf(o[j], gm[j], bt[j]);
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j) o[j] = __builtin_fmaf(o[j], 1.0f + sc[j], sh[j]);
        Vec<TY, VEC> ov;
        ov.from_float(o);
        ov.template store_buf<kStoreStream>(ry, c * (VEC * sizeof(TY)));
    }
}

template <typename TX, typename TY, typename TH, int VEC, bool FUSED, bool AFFINE, int NV>
hipError_t launch_nv(const AdalnArgs& a, bool single_group, hipStream_t st) {
    const int64_t blocks = (a.rows + kWaves - 1) / kWaves;
    const size_t lds = (size_t)(FUSED ? 3 : (AFFINE ? 4 : 2)) * a.nvec * Vec<TX, VEC>::kQuads * 16;
    // stage in LDS when there is one group and the staged vectors leave room for
    // several workgroups per CU
    if (single_group && lds <= 48 * 1024)
        hipLaunchKernelGGL((adaln_kernel<TX, TY, TH, VEC, NV, FUSED, true, AFFINE>),
                           dim3((unsigned)blocks), dim3(kWaves * 64), lds, st, a);
    else
        hipLaunchKernelGGL((adaln_kernel<TX, TY, TH, VEC, NV, FUSED, false, AFFINE>),
                           dim3((unsigned)blocks), dim3(kWaves * 64), 0, st, a);
    return hipGetLastError();
}

template <typename TX, typename TY, typename TH, int VEC, bool FUSED, bool AFFINE = false>
h3f_status_t dispatch(const AdalnArgs& a, int max_nv, bool single_group, hipStream_t st) {
    const int need = (a.nvec + 63) / 64;
    hipError_t e = hipErrorInvalidValue;
#define H3F_NV_CASE(N)                                                   \
    else if (need <= N && N <= max_nv)                                   \
        e = launch_nv<TX, TY, TH, VEC, FUSED, AFFINE, N>(a, single_group, st);
    if (false) {
    }
    H3F_NV_CASE(1) H3F_NV_CASE(2) H3F_NV_CASE(3) H3F_NV_CASE(4) H3F_NV_CASE(5) H3F_NV_CASE(6)
    H3F_NV_CASE(8) H3F_NV_CASE(10) H3F_NV_CASE(12) H3F_NV_CASE(16)
    H3F_NV_CASE(20) H3F_NV_CASE(24) H3F_NV_CASE(32)
    else return H3F_ERR_UNSUPPORTED;
#undef H3F_NV_CASE
    return e == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}

// Largest hidden size held in registers: 32 chunks per lane of 8 bf16 or of 4
// fp32 (x fp32 always uses 4-element chunks).
inline int64_t max_hidden(h3f_dtype_t x_dtype) { return x_dtype == H3F_BF16 ? 16384 : 8192; }
inline int max_nv_for(h3f_dtype_t, int) { return 32; }

h3f_status_t check_mod(const void* p, int64_t groups, int64_t gs, int64_t hidden, int V) {
    if (!aligned16(p)) return H3F_ERR_MISALIGNED;
    if (groups > 1 && gs % V) return H3F_ERR_BAD_STRIDE;
    (void)hidden;
    return H3F_OK;
}

}  // namespace
}  // namespace h3f

using namespace h3f;

namespace {

// Shared by the plain and the LayerNorm-affine entry points (gamma, beta NULL
// for the plain one).
h3f_status_t adaln_entry(void* y, h3f_dtype_t y_dtype, int64_t y_row_stride, const void* x,
                         h3f_dtype_t x_dtype, int64_t x_row_stride, const void* gamma,
                         const void* beta, const void* shift, const void* scale,
                         int64_t mod_group_stride, int64_t rows_per_group, int64_t rows,
                         int64_t hidden, float eps, void* stream) {
    const bool affine = gamma != nullptr;
    if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return H3F_ERR_BAD_DTYPE;
    if (x_dtype == H3F_BF16 && y_dtype == H3F_F32) return H3F_ERR_BAD_DTYPE;
    if (rows < 0 || hidden <= 0 || rows_per_group < 1) return H3F_ERR_BAD_SHAPE;
    const int V = vec_width(x_dtype == H3F_F32 || y_dtype == H3F_F32);
    if (hidden % V) return H3F_ERR_BAD_SHAPE;
    if (hidden > max_hidden(x_dtype) || rows > 0x7fffffff) return H3F_ERR_UNSUPPORTED;
    if (!aligned16(y) || !aligned16(x)) return H3F_ERR_MISALIGNED;
    if (affine && (!aligned16(gamma) || !aligned16(beta))) return H3F_ERR_MISALIGNED;
    const int64_t groups = groups_for(rows, rows_per_group);
    h3f_status_t s;
    if ((s = check_mod(shift, groups, mod_group_stride, hidden, V)) != H3F_OK) return s;
    if ((s = check_mod(scale, groups, mod_group_stride, hidden, V)) != H3F_OK) return s;
    if (rows > 1 && (x_row_stride % V || y_row_stride % V)) return H3F_ERR_BAD_STRIDE;
    const int ex = dtype_bytes(x_dtype), ey = dtype_bytes(y_dtype);
    if (!extent_ok(rows, x_row_stride, hidden, ex) || !extent_ok(rows, y_row_stride, hidden, ey) ||
        !extent_ok(groups, mod_group_stride, hidden, ex))
        return H3F_ERR_UNSUPPORTED;
    const Region rx = region2d(x, rows, x_row_stride, hidden, ex);
    const Region ry = region2d(y, rows, y_row_stride, hidden, ey);
    const Region rsh = region2d(shift, groups, mod_group_stride, hidden, ex);
    const Region rsc = region2d(scale, groups, mod_group_stride, hidden, ex);
    if (!rows_separate(rx) || !rows_separate(ry) || !rows_separate(rsh) || !rows_separate(rsc))
        return H3F_ERR_BAD_STRIDE;
    if (!alias_ok(ry, rx, x_dtype == y_dtype) || !disjoint(ry, rsh) || !disjoint(ry, rsc))
        return H3F_ERR_ALIASING;
    if (affine && (!disjoint(ry, region2d(gamma, 1, 0, hidden, ex)) ||
                   !disjoint(ry, region2d(beta, 1, 0, hidden, ex))))
        return H3F_ERR_ALIASING;

    AdalnArgs a{};
    a.y = y;
    a.y_rs = (rows > 1 ? y_row_stride : hidden) * ey;
    a.x = const_cast<void*>(x);
    a.x_rs = (rows > 1 ? x_row_stride : hidden) * ex;
    a.shift = shift;
    a.scale = scale;
    a.gamma = gamma;
    a.beta = beta;
    a.mod_gs = (groups > 1 ? mod_group_stride : 0) * ex;
    a.div_group = make_fastdiv((uint32_t)(rows_per_group > rows ? rows : rows_per_group));
    a.rows = rows;
    a.nvec = (int32_t)(hidden / V);
    a.hidden = (int32_t)hidden;
    a.inv_hidden = 1.0f / (float)hidden;
    a.eps = eps;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int mnv = max_nv_for(x_dtype, V);
    const bool one = groups == 1;
    if (affine) {
        if (x_dtype == H3F_F32 && y_dtype == H3F_F32)
            return dispatch<float, float, float, 4, false, true>(a, mnv, one, st);
        if (x_dtype == H3F_BF16)
            return dispatch<__bf16, __bf16, __bf16, 8, false, true>(a, mnv, one, st);
        return dispatch<float, __bf16, float, 4, false, true>(a, mnv, one, st);
    }
    if (x_dtype == H3F_F32 && y_dtype == H3F_F32)
        return dispatch<float, float, float, 4, false>(a, mnv, one, st);
    if (x_dtype == H3F_BF16)
        return dispatch<__bf16, __bf16, __bf16, 8, false>(a, mnv, one, st);
    return dispatch<float, __bf16, float, 4, false>(a, mnv, one, st);
}

}  // namespace

extern "C" h3f_status_t h3f_adaln_modulate(void* y, h3f_dtype_t y_dtype, int64_t y_row_stride,
                                           const void* x, h3f_dtype_t x_dtype,
                                           int64_t x_row_stride, const void* shift,
                                           const void* scale, int64_t mod_group_stride,
                                           int64_t rows_per_group, int64_t rows, int64_t hidden,
                                           float eps, void* stream) {
    if (rows == 0) return H3F_OK;
    if (!y || !x || !shift || !scale) return H3F_ERR_NULL_POINTER;
    return adaln_entry(y, y_dtype, y_row_stride, x, x_dtype, x_row_stride, nullptr, nullptr,
                       shift, scale, mod_group_stride, rows_per_group, rows, hidden, eps, stream);
}

extern "C" h3f_status_t h3f_adaln_affine_modulate(
    void* y, h3f_dtype_t y_dtype, int64_t y_row_stride, const void* x, h3f_dtype_t x_dtype,
    int64_t x_row_stride, const void* gamma, const void* beta, const void* shift,
    const void* scale, int64_t mod_group_stride, int64_t rows_per_group, int64_t rows,
    int64_t hidden, float eps, void* stream) {
    if (rows == 0) return H3F_OK;
    if (!y || !x || !gamma || !beta || !shift || !scale) return H3F_ERR_NULL_POINTER;
    return adaln_entry(y, y_dtype, y_row_stride, x, x_dtype, x_row_stride, gamma, beta, shift,
                       scale, mod_group_stride, rows_per_group, rows, hidden, eps, stream);
}

extern "C" h3f_status_t h3f_gated_residual_adaln(
    void* x, h3f_dtype_t x_dtype, int64_t x_row_stride, const void* h, h3f_dtype_t h_dtype,
    int64_t h_row_stride, const void* gate, const void* shift, const void* scale,
    int64_t mod_group_stride, int64_t rows_per_group, void* y, h3f_dtype_t y_dtype,
    int64_t y_row_stride, int64_t rows, int64_t hidden, float eps, void* stream) {
    if (rows == 0) return H3F_OK;
    if (!x || !h || !gate || !shift || !scale || !y) return H3F_ERR_NULL_POINTER;
    if (!dtype_ok(x_dtype) || !dtype_ok(h_dtype) || !dtype_ok(y_dtype)) return H3F_ERR_BAD_DTYPE;
    if (x_dtype == H3F_BF16 && (h_dtype == H3F_F32 || y_dtype == H3F_F32))
        return H3F_ERR_BAD_DTYPE;
    if (rows < 0 || hidden <= 0 || rows_per_group < 1) return H3F_ERR_BAD_SHAPE;
    const int V = vec_width(x_dtype == H3F_F32 || h_dtype == H3F_F32 || y_dtype == H3F_F32);
    if (hidden % V) return H3F_ERR_BAD_SHAPE;
    if (hidden > max_hidden(x_dtype) || rows > 0x7fffffff) return H3F_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(h) || !aligned16(y)) return H3F_ERR_MISALIGNED;
    const int64_t groups = groups_for(rows, rows_per_group);
    h3f_status_t s;
    if ((s = check_mod(gate, groups, mod_group_stride, hidden, V)) != H3F_OK) return s;
    if ((s = check_mod(shift, groups, mod_group_stride, hidden, V)) != H3F_OK) return s;
    if ((s = check_mod(scale, groups, mod_group_stride, hidden, V)) != H3F_OK) return s;
    if (rows > 1 && (x_row_stride % V || h_row_stride % V || y_row_stride % V))
        return H3F_ERR_BAD_STRIDE;
    const int ex = dtype_bytes(x_dtype), eh = dtype_bytes(h_dtype), ey = dtype_bytes(y_dtype);
    if (!extent_ok(rows, x_row_stride, hidden, ex) || !extent_ok(rows, h_row_stride, hidden, eh) ||
        !extent_ok(rows, y_row_stride, hidden, ey) || !extent_ok(groups, mod_group_stride, hidden, ex))
        return H3F_ERR_UNSUPPORTED;
    const Region rx = region2d(x, rows, x_row_stride, hidden, ex);
    const Region rh = region2d(h, rows, h_row_stride, hidden, eh);
    const Region ry = region2d(y, rows, y_row_stride, hidden, ey);
    const Region rg = region2d(gate, groups, mod_group_stride, hidden, ex);
    const Region rsh = region2d(shift, groups, mod_group_stride, hidden, ex);
    const Region rsc = region2d(scale, groups, mod_group_stride, hidden, ex);
    if (!rows_separate(rx) || !rows_separate(rh) || !rows_separate(ry) || !rows_separate(rg) ||
        !rows_separate(rsh) || !rows_separate(rsc))
        return H3F_ERR_BAD_STRIDE;
    const Region* others_x[] = {&rh, &rg, &rsh, &rsc, &ry};
    for (const Region* o : others_x)
        if (!disjoint(rx, *o)) return H3F_ERR_ALIASING;
    const Region* others_y[] = {&rh, &rg, &rsh, &rsc};
    for (const Region* o : others_y)
        if (!disjoint(ry, *o)) return H3F_ERR_ALIASING;

    AdalnArgs a{};
    a.y = y;
    a.y_rs = (rows > 1 ? y_row_stride : hidden) * ey;
    a.x = x;
    a.x_rs = (rows > 1 ? x_row_stride : hidden) * ex;
    a.h = h;
    a.h_rs = (rows > 1 ? h_row_stride : hidden) * eh;
    a.gate = gate;
    a.shift = shift;
    a.scale = scale;
    a.mod_gs = (groups > 1 ? mod_group_stride : 0) * ex;
    a.div_group = make_fastdiv((uint32_t)(rows_per_group > rows ? rows : rows_per_group));
    a.rows = rows;
    a.nvec = (int32_t)(hidden / V);
    a.hidden = (int32_t)hidden;
    a.inv_hidden = 1.0f / (float)hidden;
    a.eps = eps;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int mnv = max_nv_for(x_dtype, V);
    const bool one = groups == 1;
    if (x_dtype == H3F_BF16) return dispatch<__bf16, __bf16, __bf16, 8, true>(a, mnv, one, st);
    if (h_dtype == H3F_F32 && y_dtype == H3F_F32)
        return dispatch<float, float, float, 4, true>(a, mnv, one, st);
    if (h_dtype == H3F_F32) return dispatch<float, __bf16, float, 4, true>(a, mnv, one, st);
    if (y_dtype == H3F_F32) return dispatch<float, float, __bf16, 4, true>(a, mnv, one, st);
    return dispatch<float, __bf16, __bf16, 4, true>(a, mnv, one, st);
}
