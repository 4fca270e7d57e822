// k_qk_rope.hip -- per-head QK RMSNorm fused with 3D RoPE, and the token
// position helper.
//
// Design (gfx950): one 64-wide wavefront owns one token row at a time.  A head
// of head_dim elements is LPH = head_dim / VEC lanes of one 16-byte chunk each
// (bf16 head_dim 128: 16 lanes, i.e. one DPP row), so a wavefront instruction
// covers 64 / LPH head-rows and the token's 2 * heads head-rows of q and k take
// ceil(2 * heads * LPH / 64) loads, issued CH at a time before any is consumed.
// The RMS of a head is a DPP reduction inside its LPH lanes (no LDS, no
// barrier).  The lane owns whole rotation pairs (interleaved layout) or fetches
// its partner chunk with a lane shuffle (half-split layout).  The token's
// position is wave-uniform; cos / sin of the lane's pairs are generated in
// registers once per token and reused for all 2 * heads head-rows.
#include <hip/hip_runtime.h>
#include <math.h>

#include "h3f_device.hpp"
#include "h3f_validate.hpp"

namespace h3f {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 2;
constexpr int kMaxPairs = 256;

struct GridArgs {
    int32_t T, H, W, n_audio;
    int64_t n_video;  // T * H * W
    int64_t period;   // n_video + n_audio
    int64_t token_offset;
    const int32_t* positions;
};

struct QKArgs {
    void* q_out;
    int64_t qo_rs, qo_hs;
    void* k_out;
    int64_t ko_rs, ko_hs;
    const void* q;
    int64_t q_rs, q_hs;
    const void* k;
    int64_t k_rs, k_hs;
    const void* qw;
    const void* kw;
    int64_t rows;
    int32_t heads;
    int32_t head_dim;
    float inv_head_dim;
    float eps;
    int32_t c1, c2;  // axis chunk bounds inside a head: [0,c1) t, [c1,c2) h, [c2,head_dim) w
    GridArgs grid;
    float inv_freq[kMaxPairs];  // per rotation pair, chunk order [t | h | w]
};

// (t, h, w) of row `row`: video raster order (t slowest), then audio (k, 0, 0).
__device__ __forceinline__ void token_position(const GridArgs& g, int64_t row, int32_t& t,
                                               int32_t& h, int32_t& w) {
    if (g.positions) {
        t = g.positions[3 * row + 0];
        h = g.positions[3 * row + 1];
        w = g.positions[3 * row + 2];
        return;
    }
    const int64_t p = (g.token_offset + row) % g.period;
    if (p < g.n_video) {
        const int64_t hw = (int64_t)g.H * g.W;
        t = (int32_t)(p / hw);
        const int64_t rem = p - (int64_t)t * hw;
        h = (int32_t)(rem / g.W);
        w = (int32_t)(rem - (int64_t)h * g.W);
    } else {
        t = (int32_t)(p - g.n_video);
        h = 0;
        w = 0;
    }
}

template <typename T, int VEC, int LPH, int CH, bool HALF>
__global__ void __launch_bounds__(kWaves * 64) qk_rmsnorm_rope3d_kernel(QKArgs a) {
    constexpr int GPW = 64 / LPH;                 // head-rows per wavefront load
    constexpr int NA = HALF ? VEC : VEC / 2;      // angles per lane
    const int lane = threadIdx.x & 63;
    const int gsub = lane / LPH;                  // head-row slot of this lane
    const int e0 = (lane % LPH) * VEC;            // first element of the lane in its head
    const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;

    // Axis of the lane's elements, rotation pair ids and partner lane.
    const int axis = e0 < a.c1 ? 0 : (e0 < a.c2 ? 1 : 2);
    const int cstart = axis == 0 ? 0 : (axis == 1 ? a.c1 : a.c2);
    const int cend = axis == 0 ? a.c1 : (axis == 1 ? a.c2 : a.head_dim);
    const int chalf = (cend - cstart) / 2;
    const bool first_half = (e0 - cstart) < chalf;
    float freq[NA];
#pragma unroll
    for (int m = 0; m < NA; ++m) {
        int pair;
        if (HALF)
            pair = cstart / 2 + ((e0 - cstart + m) % chalf);
        else
            pair = e0 / 2 + m;
        freq[m] = a.inv_freq[pair];
    }
    const int partner = HALF ? (first_half ? lane + chalf / VEC : lane - chalf / VEC) : lane;

    // Norm weights of the lane's elements, for q and for k.
    float wq[VEC], wk[VEC];
    {
        Vec<T, VEC> t;
        t.template load<false>(static_cast<const T*>(a.qw) + e0);
        t.to_float(wq);
        t.template load<false>(static_cast<const T*>(a.kw) + e0);
        t.to_float(wk);
    }

    const int head_rows = 2 * a.heads;
    const int n_loads = (head_rows + GPW - 1) / GPW;

    for (int64_t row = wave; row < a.rows; row += nwaves) {
        int32_t pt, ph, pw;
        token_position(a.grid, row, pt, ph, pw);
        const float pf = (float)(axis == 0 ? pt : (axis == 1 ? ph : pw));
        float cs[NA], sn[NA];
#pragma unroll
        for (int m = 0; m < NA; ++m) {
            const float phi = pf * freq[m];
            sincosf(phi, &sn[m], &cs[m]);
        }

        for (int l0 = 0; l0 < n_loads; l0 += CH) {
            Vec<T, VEC> buf[CH];
            const T* src[CH];
            T* dst[CH];
            bool ok[CH], isk[CH];
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int hr = (l0 + j) * GPW + gsub;
                ok[j] = hr < head_rows;
                isk[j] = hr >= a.heads;
                const int hd = isk[j] ? hr - a.heads : hr;
                if (isk[j]) {
                    src[j] = static_cast<const T*>(a.k) + row * a.k_rs + (int64_t)hd * a.k_hs + e0;
                    dst[j] = static_cast<T*>(a.k_out) + row * a.ko_rs + (int64_t)hd * a.ko_hs + e0;
                } else {
                    src[j] = static_cast<const T*>(a.q) + row * a.q_rs + (int64_t)hd * a.q_hs + e0;
                    dst[j] = static_cast<T*>(a.q_out) + row * a.qo_rs + (int64_t)hd * a.qo_hs + e0;
                }
                if (ok[j])
                    buf[j].template load<true>(src[j]);
                else
                    buf[j].zero();
            }
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                float v[VEC];
                buf[j].to_float(v);
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < VEC; ++i) ss = __builtin_fmaf(v[i], v[i], ss);
                ss = group_sum<LPH>(ss);
                const float rstd = __builtin_amdgcn_rsqf(ss * a.inv_head_dim + a.eps);
                float u[VEC];
#pragma unroll
                for (int i = 0; i < VEC; ++i) u[i] = v[i] * rstd * (isk[j] ? wk[i] : wq[i]);
                float o[VEC];
                if constexpr (!HALF) {
#pragma unroll
                    for (int m = 0; m < VEC / 2; ++m) {
                        const float u0 = u[2 * m], u1 = u[2 * m + 1];
                        o[2 * m] = u0 * cs[m] - u1 * sn[m];
                        o[2 * m + 1] = u0 * sn[m] + u1 * cs[m];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) {
                        const float pv = __shfl(u[i], partner, 64);
                        o[i] = first_half ? u[i] * cs[i] - pv * sn[i] : pv * sn[i] + u[i] * cs[i];
                    }
                }
                if (ok[j]) {
                    Vec<T, VEC> ov;
                    ov.from_float(o);
                    ov.template store<true>(dst[j]);
                }
            }
        }
    }
}

__global__ void __launch_bounds__(256) positions_kernel(int32_t* __restrict__ pos, int64_t rows,
                                                        GridArgs g) {
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (r >= rows) return;
    int32_t t, h, w;
    token_position(g, r, t, h, w);
    pos[3 * r + 0] = t;
    pos[3 * r + 1] = h;
    pos[3 * r + 2] = w;
}

constexpr int kCH = 10;

template <typename T, int VEC, int LPH, bool HALF>
hipError_t launch_lph(const QKArgs& a, hipStream_t st) {
    int64_t blocks = (a.rows + kWaves * kRowsPerWave - 1) / (kWaves * kRowsPerWave);
    if (blocks > 0x7fffffff) blocks = 0x7fffffff;
    hipLaunchKernelGGL((qk_rmsnorm_rope3d_kernel<T, VEC, LPH, kCH, HALF>), dim3((unsigned)blocks),
                       dim3(kWaves * 64), 0, st, a);
    return hipGetLastError();
}

template <typename T, int VEC, bool HALF>
hipError_t dispatch_lph(const QKArgs& a, int lph, hipStream_t st) {
    switch (lph) {
        case 2: return launch_lph<T, VEC, 2, HALF>(a, st);
        case 4: return launch_lph<T, VEC, 4, HALF>(a, st);
        case 8: return launch_lph<T, VEC, 8, HALF>(a, st);
        case 16: return launch_lph<T, VEC, 16, HALF>(a, st);
        case 32: return launch_lph<T, VEC, 32, HALF>(a, st);
        case 64: return launch_lph<T, VEC, 64, HALF>(a, st);
        default: return hipErrorInvalidValue;
    }
}

h3f_status_t grid_args(const h3f_rope3d_t* r, GridArgs& g) {
    g.positions = r->positions;
    g.T = r->T;
    g.H = r->H;
    g.W = r->W;
    g.n_audio = r->n_audio;
    g.token_offset = r->token_offset;
    if (!r->positions) {
        if (r->T < 1 || r->H < 1 || r->W < 1 || r->n_audio < 0) return H3F_ERR_BAD_SHAPE;
        if (r->token_offset < 0) return H3F_ERR_BAD_SHAPE;
    }
    g.n_video = (int64_t)(r->T > 0 ? r->T : 0) * (r->H > 0 ? r->H : 0) * (r->W > 0 ? r->W : 0);
    g.period = g.n_video + (r->n_audio > 0 ? r->n_audio : 0);
    if (g.period < 1) g.period = 1;
    return H3F_OK;
}

}  // namespace
}  // namespace h3f

using namespace h3f;

extern "C" h3f_status_t h3f_rope3d_positions(int32_t* pos, int64_t rows, const h3f_rope3d_t* grid,
                                             void* stream) {
    if (rows == 0) return H3F_OK;
    if (!pos || !grid) return H3F_ERR_NULL_POINTER;
    if (rows < 0) return H3F_ERR_BAD_SHAPE;
    if ((reinterpret_cast<uintptr_t>(pos) & 3u) != 0) return H3F_ERR_MISALIGNED;
    h3f_rope3d_t g = *grid;
    g.positions = nullptr;
    GridArgs ga;
    h3f_status_t s = grid_args(&g, ga);
    if (s != H3F_OK) return s;
    const int64_t blocks = (rows + 255) / 256;
    if (blocks > 0x7fffffff) return H3F_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(positions_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), pos, rows, ga);
    return hipGetLastError() == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}

extern "C" h3f_status_t h3f_qk_rmsnorm_rope3d(
    void* q_out, int64_t q_out_row_stride, int64_t q_out_head_stride, void* k_out,
    int64_t k_out_row_stride, int64_t k_out_head_stride, const void* q, int64_t q_row_stride,
    int64_t q_head_stride, const void* k, int64_t k_row_stride, int64_t k_head_stride,
    const void* q_weight, const void* k_weight, h3f_dtype_t dtype, int64_t rows, int32_t heads,
    int32_t head_dim, float eps, const h3f_rope3d_t* rope, void* stream) {
    if (rows == 0) return H3F_OK;
    if (!q_out || !k_out || !q || !k || !q_weight || !k_weight || !rope)
        return H3F_ERR_NULL_POINTER;
    if (!dtype_ok(dtype)) return H3F_ERR_BAD_DTYPE;
    if (rows < 0 || heads < 1 || head_dim < 1) return H3F_ERR_BAD_SHAPE;
    const int V = vec_width(dtype == H3F_BF16);
    if (head_dim % V) return H3F_ERR_BAD_SHAPE;
    const int lph = head_dim / V;
    if (lph < 2 || lph > 64 || (lph & (lph - 1))) return H3F_ERR_UNSUPPORTED;
    if (rope->d_t < V || rope->d_h < V || rope->d_w < V || rope->d_t % V || rope->d_h % V ||
        rope->d_w % V || rope->d_t + rope->d_h + rope->d_w != head_dim)
        return H3F_ERR_BAD_SHAPE;
    if (rope->pairing != H3F_ROPE_INTERLEAVED && rope->pairing != H3F_ROPE_HALF_SPLIT)
        return H3F_ERR_UNSUPPORTED;
    if (rope->pairing == H3F_ROPE_HALF_SPLIT &&
        (rope->d_t % (2 * V) || rope->d_h % (2 * V) || rope->d_w % (2 * V)))
        return H3F_ERR_UNSUPPORTED;
    if (!(rope->theta > 0.0)) return H3F_ERR_BAD_SHAPE;
    if (rows > 0x7fffffff || (int64_t)heads * 2 > 0x7fffffff) return H3F_ERR_UNSUPPORTED;
    if (!aligned16(q_out) || !aligned16(k_out) || !aligned16(q) || !aligned16(k) ||
        !aligned16(q_weight) || !aligned16(k_weight))
        return H3F_ERR_MISALIGNED;
    if (rope->positions && (reinterpret_cast<uintptr_t>(rope->positions) & 3u))
        return H3F_ERR_MISALIGNED;
    const int64_t strides[] = {q_out_row_stride, q_out_head_stride, k_out_row_stride,
                               k_out_head_stride, q_row_stride, q_head_stride,
                               k_row_stride, k_head_stride};
    for (int i = 0; i < 8; ++i) {
        const bool is_head = (i & 1) == 1;
        if (is_head && heads <= 1) continue;
        if (!is_head && rows <= 1) continue;
        if (strides[i] % V) return H3F_ERR_BAD_STRIDE;
    }
    if (heads > 1 && (q_out_head_stride < head_dim || k_out_head_stride < head_dim ||
                      q_head_stride < head_dim || k_head_stride < head_dim))
        return H3F_ERR_BAD_STRIDE;
    const int e = dtype_bytes(dtype);
    auto region = [&](const void* p, int64_t rs, int64_t hs) {
        const int64_t span = ((heads > 1 ? (int64_t)(heads - 1) * hs : 0) + head_dim);
        return region2d(p, rows, rows > 1 ? rs : span, span, e);
    };
    const Region rqo = region(q_out, q_out_row_stride, q_out_head_stride);
    const Region rko = region(k_out, k_out_row_stride, k_out_head_stride);
    const Region rq = region(q, q_row_stride, q_head_stride);
    const Region rk = region(k, k_row_stride, k_head_stride);
    if (!rows_separate(rqo) || !rows_separate(rko) || !rows_separate(rq) || !rows_separate(rk))
        return H3F_ERR_BAD_STRIDE;
    const Region rw1 = region2d(q_weight, 1, head_dim, head_dim, e);
    const Region rw2 = region2d(k_weight, 1, head_dim, head_dim, e);
    // q_out: may be q exactly; must not touch k, k_out or the weights.
    if (!alias_ok(rqo, rq, true) || !disjoint(rqo, rk) || !disjoint(rqo, rko) ||
        !disjoint(rqo, rw1) || !disjoint(rqo, rw2))
        return H3F_ERR_ALIASING;
    if (!alias_ok(rko, rk, true) || !disjoint(rko, rq) || !disjoint(rko, rw1) ||
        !disjoint(rko, rw2))
        return H3F_ERR_ALIASING;
    // exact aliasing also needs identical head strides
    if (same_region(rqo, rq) && heads > 1 && q_out_head_stride != q_head_stride)
        return H3F_ERR_ALIASING;
    if (same_region(rko, rk) && heads > 1 && k_out_head_stride != k_head_stride)
        return H3F_ERR_ALIASING;

    QKArgs a{};
    a.q_out = q_out;
    a.qo_rs = q_out_row_stride;
    a.qo_hs = q_out_head_stride;
    a.k_out = k_out;
    a.ko_rs = k_out_row_stride;
    a.ko_hs = k_out_head_stride;
    a.q = q;
    a.q_rs = q_row_stride;
    a.q_hs = q_head_stride;
    a.k = k;
    a.k_rs = k_row_stride;
    a.k_hs = k_head_stride;
    a.qw = q_weight;
    a.kw = k_weight;
    a.rows = rows;
    a.heads = heads;
    a.head_dim = head_dim;
    a.inv_head_dim = 1.0f / (float)head_dim;
    a.eps = eps;
    a.c1 = rope->d_t;
    a.c2 = rope->d_t + rope->d_h;
    h3f_status_t s = grid_args(rope, a.grid);
    if (s != H3F_OK) return s;
    // Frequencies theta^(-2j/d_c), evaluated in double and rounded once to fp32.
    const int32_t dims[3] = {rope->d_t, rope->d_h, rope->d_w};
    int p = 0;
    for (int c = 0; c < 3; ++c)
        for (int32_t j = 0; j < dims[c] / 2; ++j)
            a.inv_freq[p++] = (float)pow(rope->theta, -2.0 * (double)j / (double)dims[c]);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool half = rope->pairing == H3F_ROPE_HALF_SPLIT;
    hipError_t err;
    if (dtype == H3F_BF16)
        err = half ? dispatch_lph<__bf16, 8, true>(a, lph, st)
                   : dispatch_lph<__bf16, 8, false>(a, lph, st);
    else
        err = half ? dispatch_lph<float, 4, true>(a, lph, st)
                   : dispatch_lph<float, 4, false>(a, lph, st);
    return err == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}
