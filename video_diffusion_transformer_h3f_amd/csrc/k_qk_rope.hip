// k_qk_rope.hip -- per-head QK RMSNorm fused with 3D RoPE, and the token
// position helper.
//
// Design (gfx950): a head of head_dim elements is LPH = head_dim / VEC lanes of
// one 16-byte chunk each (bf16 head_dim 128: 16 lanes, one DPP row), so one
// wavefront load covers GPW = 64 / LPH head-rows.  The token's q heads take
// nl = ceil(heads / GPW) such loads and its k heads another nl; each of these
// 2 * nl "slots" of each token is one independent 64-thread workgroup that does
// exactly one 16-byte load and one 16-byte store per lane.  Measured on MI355X,
// this finest work granularity streams best (many short wavefronts, about one
// KiB in flight each); a wavefront that holds a whole token row is ~10% slower.
// The RMS of a head is a DPP reduction inside its LPH lanes (no LDS, no
// barrier).  The token's position is wave-uniform scalar arithmetic.  cos / sin
// are generated in registers: with the interleaved layout and at most 64
// rotation pairs, lane L computes pair L once and the lanes of each head fetch
// their pairs with lane shuffles; otherwise each lane computes its own pairs.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include "h3f_device.hpp"
#include "h3f_validate.hpp"

namespace h3f {
namespace {

constexpr int kMaxPairs = 256;

typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// A buffer offset past any resource: the store is dropped.
constexpr uint32_t kDroppedOffset = 0xFFFFFFF0u;

// Token grid: row r (of the whole call) is token p = (offset + r) mod period;
// offset is reduced modulo period on the host and offset + rows < 2^31.
struct GridArgs {
    uint32_t n_video, period, offset, W, HW;
    FastDiv div_period, div_hw, div_w;
    const int32_t* positions;  // optional [rows, 3]
};

// Row / head strides in bytes.
struct QKArgs {
    char* q_out;
    int64_t qo_rs, qo_hs;
    char* k_out;
    int64_t ko_rs, ko_hs;
    const char* q;
    int64_t q_rs, q_hs;
    const char* k;
    int64_t k_rs, k_hs;
    uint32_t qo_span, ko_span, q_span, k_span;  // bytes of one row's heads
    const char* qw;
    const char* kw;
    int64_t row0;         // first row of this launch
    uint32_t n_q_blocks;  // rows of this launch * nl: blocks [0, n) are q, [n, 2n) are k
    FastDiv div_nl;       // nl slots per tensor per token
    int32_t nl;           // loads per tensor per token
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
    uint32_t p = g.offset + (uint32_t)row;
    p -= fdiv(p, g.div_period) * g.period;
    if (p < g.n_video) {
        const uint32_t tt = fdiv(p, g.div_hw);
        const uint32_t rem = p - tt * g.HW;
        const uint32_t hh = fdiv(rem, g.div_w);
        t = (int32_t)tt;
        h = (int32_t)hh;
        w = (int32_t)(rem - hh * g.W);
    } else {
        t = (int32_t)(p - g.n_video);
        h = 0;
        w = 0;
    }
}

// What a lane needs of the frequency table, read once per workgroup (the table
// lives in the kernel arguments; indexing it by lane is a memory load, which
// inside a token loop would also wait for every load in flight).
template <int VEC, int LPH, bool HALF>
struct LaneFreq {
    static constexpr int NA = HALF ? VEC : VEC / 2;  // rotation pairs touched by a lane
    static constexpr bool kShared = !HALF && LPH * VEC / 2 <= 64;
    float f[kShared ? 1 : NA];  // shared: pair `lane`; otherwise the lane's own pairs
    int ax;                     // axis (0 t, 1 h, 2 w) of those pairs
};

template <int VEC, int LPH, bool HALF>
__device__ __forceinline__ LaneFreq<VEC, LPH, HALF> lane_freq(const QKArgs& a, int lane, int e0) {
    using LF = LaneFreq<VEC, LPH, HALF>;
    LF lf;
    if constexpr (LF::kShared) {
        // lane L holds pair L (pair p covers elements 2p, 2p + 1)
        const int e = 2 * lane;
        lf.ax = e < a.c1 ? 0 : (e < a.c2 ? 1 : 2);
        lf.f[0] = lane < LPH * VEC / 2 ? a.inv_freq[lane] : 0.f;
    } else {
        lf.ax = e0 < a.c1 ? 0 : (e0 < a.c2 ? 1 : 2);
        const int cstart = lf.ax == 0 ? 0 : (lf.ax == 1 ? a.c1 : a.c2);
        const int cend = lf.ax == 0 ? a.c1 : (lf.ax == 1 ? a.c2 : a.head_dim);
        const int chalf = (cend - cstart) / 2;
#pragma unroll
        for (int m = 0; m < LF::NA; ++m) {
            const int pair = HALF ? cstart / 2 + ((e0 - cstart + m) % chalf) : e0 / 2 + m;
            lf.f[m] = a.inv_freq[pair];
        }
    }
    return lf;
}

// One lane's share of one head-row of a token at position (pt, ph, pw): RMSNorm
// of the head (a DPP reduction over its LPH lanes) times the weight, then the
// 3D rotation of the lane's pairs.  o receives the rotated values in fp32
// (rounded by the caller).
template <typename T, int VEC, int LPH, bool HALF>
__device__ __forceinline__ void qk_token(const QKArgs& a, int32_t pt, int32_t ph, int32_t pw,
                                         int lane, int e0, const LaneFreq<VEC, LPH, HALF>& lf,
                                         const float (&w)[VEC], const Vec<T, VEC>& buf,
                                         float (&o)[VEC]) {
    using LF = LaneFreq<VEC, LPH, HALF>;
    constexpr int NA = LF::NA;
    const float pf = (float)(lf.ax == 0 ? pt : (lf.ax == 1 ? ph : pw));
    float cs[NA], sn[NA];
    if constexpr (LF::kShared) {
        float s1 = 0.f, c1 = 1.f;
        if (lane < LPH * VEC / 2) sincosf(pf * lf.f[0], &s1, &c1);
#pragma unroll
        for (int m = 0; m < NA; ++m) {
            cs[m] = __shfl(c1, e0 / 2 + m, 64);
            sn[m] = __shfl(s1, e0 / 2 + m, 64);
        }
    } else {
#pragma unroll
        for (int m = 0; m < NA; ++m) sincosf(pf * lf.f[m], &sn[m], &cs[m]);
    }

    float v[VEC];
    buf.to_float(v);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) ss = __builtin_fmaf(v[i], v[i], ss);
    ss = group_sum<LPH>(ss);
    const float rstd = __builtin_amdgcn_rsqf(ss * a.inv_head_dim + a.eps);
    float u[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) u[i] = v[i] * rstd * w[i];
    if constexpr (!HALF) {
#pragma unroll
        for (int m = 0; m < VEC / 2; ++m) {
            const float u0 = u[2 * m], u1 = u[2 * m + 1];
            o[2 * m] = u0 * cs[m] - u1 * sn[m];
            o[2 * m + 1] = u0 * sn[m] + u1 * cs[m];
        }
    } else {
        // pairs (j, j + d_c/2): the partner chunk sits chalf / VEC lanes away
        const int cstart = lf.ax == 0 ? 0 : (lf.ax == 1 ? a.c1 : a.c2);
        const int cend = lf.ax == 0 ? a.c1 : (lf.ax == 1 ? a.c2 : a.head_dim);
        const int chalf = (cend - cstart) / 2;
        const bool first = (e0 - cstart) < chalf;
        const int partner = first ? lane + chalf / VEC : lane - chalf / VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const float pv = __shfl(u[i], partner, 64);
            o[i] = first ? u[i] * cs[i] - pv * sn[i] : pv * sn[i] + u[i] * cs[i];
        }
    }
}

template <typename T, int VEC>
__device__ __forceinline__ void load_weights(const char* wp, int e0, float (&w)[VEC]) {
    Vec<T, VEC> t;
    t.template load<false>(reinterpret_cast<const T*>(wp) + e0);
    t.to_float(w);
}

template <typename T, int VEC, int LPH, bool HALF>
__global__ void __launch_bounds__(64) qk_rmsnorm_rope3d_kernel(QKArgs a) {
    constexpr int GPW = 64 / LPH;             // head-rows per wavefront load
    const int lane = threadIdx.x;
    const int gsub = lane / LPH;        // head-row slot of this lane
    const int e0 = (lane % LPH) * VEC;  // first element of the lane in its head

    // Which tensor, token and slot: wave-uniform.  Tensor-major order (every q
    // slot of the launch, then every k slot) keeps one input and one output
    // stream live at a time; interleaving q and k per token measured ~5% slower.
    const uint32_t bid = blockIdx.x;
    const bool isk = bid >= a.n_q_blocks;
    const uint32_t bb = isk ? bid - a.n_q_blocks : bid;
    const uint32_t rr = fdiv(bb, a.div_nl);
    const uint32_t slot = bb - rr * (uint32_t)a.nl;
    const int64_t row = a.row0 + rr;
    const uint32_t hd = slot * GPW + gsub;

    // One 16-byte chunk per lane; a head slot past the last head lies outside the
    // row's resource (offset >= heads * head_stride >= span): reads 0, not stored.
    const rsrc_t rin = isk ? make_rsrc(a.k + row * a.k_rs, a.k_span)
                           : make_rsrc(a.q + row * a.q_rs, a.q_span);
    const uint32_t e0b = (uint32_t)e0 * sizeof(T);
    Vec<T, VEC> buf;
    buf.template load_buf<kLoadStream>(rin, hd * (uint32_t)(isk ? a.k_hs : a.q_hs) + e0b);

    float w[VEC];
    load_weights<T, VEC>(isk ? a.kw : a.qw, e0, w);
    const LaneFreq<VEC, LPH, HALF> lf = lane_freq<VEC, LPH, HALF>(a, lane, e0);
    int32_t pt, ph, pw;
    token_position(a.grid, row, pt, ph, pw);
    float o[VEC];
    qk_token<T, VEC, LPH, HALF>(a, pt, ph, pw, lane, e0, lf, w, buf, o);
    Vec<T, VEC> ov;
    ov.from_float(o);
    const rsrc_t rout = isk ? make_rsrc(a.k_out + row * a.ko_rs, a.ko_span)
                            : make_rsrc(a.q_out + row * a.qo_rs, a.qo_span);
    ov.template store_buf<kStoreStream>(rout, hd * (uint32_t)(isk ? a.ko_hs : a.qo_hs) + e0b);
}

// Router pooling fused into the operator.  The block-sparse router ranks key
// blocks by the means of the post-RoPE q and k over blocks of `block` tokens;
// computed here, from the values as stored, they cost no second pass over q
// and k.  One workgroup of kPoolWaves wavefronts per (tensor, token block,
// head-row slot): wavefront v takes the block's chunks of kPoolTokens tokens
// v, v + kPoolWaves, ... (a chunk's loads in flight together), does for each
// token exactly what qk_rmsnorm_rope3d_kernel does (same code, so the stored
// outputs are bit-identical) and adds the stored, rounded values into fp32
// sums; the wavefronts' sums are added in wavefront order through LDS and
// their means go to pooled[tensor][head][block][head_dim], the router's
// workspace layout.  Many wavefronts per block are needed: a token's work is a
// chain of dependent steps (sincos, lane shuffles, the RMS reduction), and one
// wavefront walking a whole block alone left the chip mostly waiting on them.
// Measured side by side at the 5 s shape (tokens per chunk x wavefronts),
// before the per-token code was tuned further: 8 x 1 1.03 ms, 8 x 4 0.99,
// 4 x 8 0.95, 2 x 8 0.92, 1 x 16 0.93, 2 x 16 0.91.  The tuned 2 x 16 form runs
// 0.86-0.87 ms, against 0.76 ms for the plain operator plus 0.41 ms for the
// router's separate pooling.  Each wavefront stores 8 KiB (its 8 tokens),
// and wavefronts that store several KiB write more slowly than ones that
// store one (about 5.5 against 7.1 TB/s at 10 KiB and 1 KiB per wavefront).
constexpr int kPoolTokens = 2;
constexpr int kPoolWaves = 16;

struct PoolOut {
    float* pooled;        // [2][heads][n_blocks][head_dim] fp32
    int64_t rows;
    int32_t block;
    int32_t heads;
    uint32_t n_blocks;
    uint32_t n_q_blocks;  // n_blocks * nl: workgroups [0, n) are q, [n, 2n) are k
};

template <typename T, int VEC, int LPH, bool HALF>
__global__ void __launch_bounds__(64 * kPoolWaves) qk_pool_kernel(QKArgs a, PoolOut p) {
    constexpr int GPW = 64 / LPH;
    constexpr int U = kPoolTokens;
    constexpr int NW = kPoolWaves;
    __shared__ float part[NW - 1][64][VEC];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gsub = lane / LPH;
    const int e0 = (lane % LPH) * VEC;
    const uint32_t bid = blockIdx.x;
    const bool isk = bid >= p.n_q_blocks;
    const uint32_t bb = isk ? bid - p.n_q_blocks : bid;
    const uint32_t b = fdiv(bb, a.div_nl);
    const uint32_t slot = bb - b * (uint32_t)a.nl;
    const uint32_t hd = slot * GPW + gsub;
    // A resource here spans several token rows, so a head slot past the last
    // head is not out of range: such lanes read head 0 and store nothing.
    const bool live = hd < (uint32_t)p.heads;
    const uint32_t e0b = (uint32_t)e0 * sizeof(T);
    const char* in = isk ? a.k : a.q;
    const int64_t in_rs = isk ? a.k_rs : a.q_rs;
    const uint32_t in_span = isk ? a.k_span : a.q_span;
    const uint32_t in_off = (live ? hd : 0u) * (uint32_t)(isk ? a.k_hs : a.q_hs) + e0b;
    char* out = isk ? a.k_out : a.q_out;
    const int64_t out_rs = isk ? a.ko_rs : a.qo_rs;
    const uint32_t out_span = isk ? a.ko_span : a.qo_span;
    const uint32_t out_off = (live ? hd : 0u) * (uint32_t)(isk ? a.ko_hs : a.qo_hs) + e0b;

    float w[VEC];
    load_weights<T, VEC>(isk ? a.kw : a.qw, e0, w);
    const LaneFreq<VEC, LPH, HALF> lf = lane_freq<VEC, LPH, HALF>(a, lane, e0);
    const int64_t r_begin = (int64_t)b * p.block;
    const int64_t r_end = r_begin + p.block < p.rows ? r_begin + p.block : p.rows;
    float sum[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) sum[i] = 0.f;
    // Chunks of U tokens, double-buffered: a wavefront loads its next chunk
    // before it computes and stores the current one, so waiting for a chunk's
    // loads never includes the previous chunk's stores (the vector memory
    // counter counts both, in order).  Every chunk issues the same memory
    // operations -- U loads, one positions load and U stores -- so those waits
    // stay exact: stores past the block's last token or for a head past the
    // last are dropped (offset outside the resource), derived positions and the
    // prefetch after a wavefront's last chunk use zero-length resources (issued,
    // moving no bytes).  Explicit positions are read with their chunk's data: 3
    // int32 per token, one 12-byte load by lanes 0 .. U-1, handed to the other
    // lanes by shuffles.
    const int nchunks = (int)((r_end - r_begin + U - 1) / U);
    const int32_t* posp = a.grid.positions;
    auto load_chunk = [&](int c, bool real, Vec<T, VEC> (&bf)[U], u32x3& pos) {
        const int64_t r0 = r_begin + (int64_t)c * U;
        const int n = (int)(r_end - r0 < U ? r_end - r0 : U);
        // rows past the block's last read as zeros (outside the resource)
        const rsrc_t rin = make_rsrc(in + r0 * in_rs,
                                     real ? (uint32_t)((n - 1) * in_rs) + in_span : 0u);
#pragma unroll
        for (int u = 0; u < U; ++u)
            bf[u].template load_buf<kLoadStream>(rin, (uint32_t)(u * in_rs) + in_off);
        const rsrc_t rp = make_rsrc(posp ? posp + 3 * r0 : posp, posp && real ? (uint32_t)n * 12u : 0u);
        pos = __builtin_bit_cast(
            u32x3, __builtin_amdgcn_raw_buffer_load_b96(rp, (uint32_t)(lane & (U - 1)) * 12u, 0, 0));
    };
    auto process = [&](int c, const Vec<T, VEC> (&bf)[U], const u32x3& pos) {
        const int64_t r0 = r_begin + (int64_t)c * U;
        const int n = (int)(r_end - r0 < U ? r_end - r0 : U);
        const rsrc_t rout = make_rsrc(out + r0 * out_rs, (uint32_t)((n - 1) * out_rs) + out_span);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int32_t pt, ph, pw;
            if (posp) {
                pt = __shfl((int)pos[0], u, 64);
                ph = __shfl((int)pos[1], u, 64);
                pw = __shfl((int)pos[2], u, 64);
            } else {
                token_position(a.grid, r0 + u, pt, ph, pw);
            }
            float o[VEC];
            qk_token<T, VEC, LPH, HALF>(a, pt, ph, pw, lane, e0, lf, w, bf[u], o);
            Vec<T, VEC> ov;
            ov.from_float(o);
            ov.template store_buf<kStoreStream>(
                rout, u < n && live ? (uint32_t)(u * out_rs) + out_off : kDroppedOffset);
            if (u < n) {
                float st[VEC];
                ov.to_float(st);  // the mean is of the stored values
#pragma unroll
                for (int i = 0; i < VEC; ++i) sum[i] += st[i];
            }
        }
    };
    Vec<T, VEC> buf0[U], buf1[U];
    u32x3 pos0, pos1;
    // this wavefront's chunks: wv, wv + NW, ... (a wavefront with none loads
    // chunk 0 and computes nothing)
    load_chunk(wv < nchunks ? wv : 0, wv < nchunks, buf0, pos0);
    for (int c = wv; c < nchunks; c += 2 * NW) {
        load_chunk(c + NW < nchunks ? c + NW : c, c + NW < nchunks, buf1, pos1);
        process(c, buf0, pos0);
        if (c + NW >= nchunks) break;
        load_chunk(c + 2 * NW < nchunks ? c + 2 * NW : c + NW, c + 2 * NW < nchunks, buf0, pos0);
        process(c + NW, buf1, pos1);
    }
    // add the wavefronts' sums in wavefront order
    if (wv > 0) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) part[wv - 1][lane][i] = sum[i];
    }
    __syncthreads();
    if (wv > 0) return;
#pragma unroll
    for (int v = 0; v < NW - 1; ++v)
#pragma unroll
        for (int i = 0; i < VEC; ++i) sum[i] += part[v][lane][i];
    if (!live) return;
    const float nt = (float)(r_end - r_begin);
    float* dst = p.pooled +
                 (((size_t)(isk ? 1 : 0) * p.heads + hd) * p.n_blocks + b) * (size_t)a.head_dim + e0;
#pragma unroll
    for (int i = 0; i < VEC; i += 4)
        *reinterpret_cast<float4*>(dst + i) =
            make_float4(sum[i] / nt, sum[i + 1] / nt, sum[i + 2] / nt, sum[i + 3] / nt);
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

template <typename T, int VEC, int LPH, bool HALF>
hipError_t launch_lph(QKArgs a, int64_t rows, hipStream_t st) {
    const int64_t slots = 2 * (int64_t)a.nl;
    const int64_t step = 0x7fffffffll / slots;
    for (int64_t r0 = 0; r0 < rows; r0 += step) {
        const int64_t nr = rows - r0 < step ? rows - r0 : step;
        a.row0 = r0;
        a.n_q_blocks = (uint32_t)(nr * a.nl);
        hipLaunchKernelGGL((qk_rmsnorm_rope3d_kernel<T, VEC, LPH, HALF>),
                           dim3((unsigned)(nr * slots)), dim3(64), 0, st, a);
    }
    return hipGetLastError();
}

template <typename T, int VEC, bool HALF>
hipError_t dispatch_lph(const QKArgs& a, int lph, int64_t rows, hipStream_t st) {
    switch (lph) {
        case 2: return launch_lph<T, VEC, 2, HALF>(a, rows, st);
        case 4: return launch_lph<T, VEC, 4, HALF>(a, rows, st);
        case 8: return launch_lph<T, VEC, 8, HALF>(a, rows, st);
        case 16: return launch_lph<T, VEC, 16, HALF>(a, rows, st);
        case 32: return launch_lph<T, VEC, 32, HALF>(a, rows, st);
        case 64: return launch_lph<T, VEC, 64, HALF>(a, rows, st);
        default: return hipErrorInvalidValue;
    }
}

// Grid description for the kernels; rows + reduced offset must stay below 2^31.
h3f_status_t grid_args(const h3f_rope3d_t* r, int64_t rows, GridArgs& g) {
    g.positions = r->positions;
    if (r->positions) {
        g.n_video = g.period = g.offset = g.W = g.HW = 1;
        g.div_period = g.div_hw = g.div_w = make_fastdiv(1);
        return H3F_OK;
    }
    if (r->T < 1 || r->H < 1 || r->W < 1 || r->n_audio < 0) return H3F_ERR_BAD_SHAPE;
    if (r->token_offset < 0) return H3F_ERR_BAD_SHAPE;
    const int64_t hw = (int64_t)r->H * r->W;  // < 2^62: no overflow
    if (hw > 0x7fffffffll) return H3F_ERR_UNSUPPORTED;
    const int64_t nv = hw * r->T;              // < 2^62 once hw < 2^31
    const int64_t period = nv + r->n_audio;
    if (period > 0x7fffffffll) return H3F_ERR_UNSUPPORTED;
    const int64_t off = r->token_offset % period;
    if (off + rows > 0x7fffffffll) return H3F_ERR_UNSUPPORTED;
    g.n_video = (uint32_t)nv;
    g.period = (uint32_t)period;
    g.offset = (uint32_t)off;
    g.W = (uint32_t)r->W;
    g.HW = (uint32_t)hw;
    g.div_period = make_fastdiv(g.period);
    g.div_hw = make_fastdiv(g.HW);
    g.div_w = make_fastdiv(g.W);
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
    h3f_status_t s = grid_args(&g, rows, ga);
    if (s != H3F_OK) return s;
    const int64_t blocks = (rows + 255) / 256;
    hipLaunchKernelGGL(positions_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), pos, rows, ga);
    return hipGetLastError() == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}

namespace {

// Regions of the tensors of one call, for the fused form's extra checks.
struct QKRegions {
    Region qo, ko, q, k, qw, kw;
};

// Validation of a QK RMSNorm + RoPE call and its kernel arguments (shared by
// the plain and the pooled entry points); rows >= 1.
h3f_status_t qk_prepare(QKArgs& a, int& lph, QKRegions& reg, void* q_out, int64_t q_out_row_stride,
                        int64_t q_out_head_stride, void* k_out, int64_t k_out_row_stride,
                        int64_t k_out_head_stride, const void* q, int64_t q_row_stride,
                        int64_t q_head_stride, const void* k, int64_t k_row_stride,
                        int64_t k_head_stride, const void* q_weight, const void* k_weight,
                        h3f_dtype_t dtype, int64_t rows, int32_t heads, int32_t head_dim,
                        float eps, const h3f_rope3d_t* rope) {
    if (!q_out || !k_out || !q || !k || !q_weight || !k_weight || !rope)
        return H3F_ERR_NULL_POINTER;
    if (!dtype_ok(dtype)) return H3F_ERR_BAD_DTYPE;
    if (rows < 0 || heads < 1 || head_dim < 1) return H3F_ERR_BAD_SHAPE;
    const int V = vec_width(dtype == H3F_F32);
    if (head_dim % V) return H3F_ERR_BAD_SHAPE;
    lph = head_dim / V;
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
    if (rows > 0x7fffffff || heads > 0x3fffffff) return H3F_ERR_UNSUPPORTED;
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
    {
        const int64_t rs_[] = {q_out_row_stride, k_out_row_stride, q_row_stride, k_row_stride};
        const int64_t hs_[] = {q_out_head_stride, k_out_head_stride, q_head_stride, k_head_stride};
        for (int i = 0; i < 4; ++i) {
            if (!extent_ok(heads, hs_[i], head_dim, e)) return H3F_ERR_UNSUPPORTED;
            const int64_t span = (heads > 1 ? (int64_t)(heads - 1) * hs_[i] : 0) + head_dim;
            if (!extent_ok(rows, rs_[i], span, e)) return H3F_ERR_UNSUPPORTED;
        }
    }
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
    // One row's heads are addressed through a 32-bit buffer resource; slots past the
    // last head reach at most 64 head strides beyond the row span.
    {
        const int64_t hs_max = (int64_t)head_dim * e +
            (heads > 1 ? e * std::max(std::max(q_out_head_stride, k_out_head_stride),
                                      std::max(q_head_stride, k_head_stride)) : 0);
        const int64_t span_max = std::max(std::max(rqo.span, rko.span), std::max(rq.span, rk.span));
        if (span_max > 0xFFFFFFF0ll || hs_max > (0xFFFFFFF0ll - span_max) / 64)
            return H3F_ERR_UNSUPPORTED;
    }
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

    a.q_out = static_cast<char*>(q_out);
    a.qo_rs = q_out_row_stride * e;
    a.qo_hs = (heads > 1 ? q_out_head_stride : head_dim) * e;
    a.k_out = static_cast<char*>(k_out);
    a.ko_rs = k_out_row_stride * e;
    a.ko_hs = (heads > 1 ? k_out_head_stride : head_dim) * e;
    a.q = static_cast<const char*>(q);
    a.q_rs = q_row_stride * e;
    a.q_hs = (heads > 1 ? q_head_stride : head_dim) * e;
    a.k = static_cast<const char*>(k);
    a.k_rs = k_row_stride * e;
    a.k_hs = (heads > 1 ? k_head_stride : head_dim) * e;
    a.qo_span = (uint32_t)rqo.span;
    a.ko_span = (uint32_t)rko.span;
    a.q_span = (uint32_t)rq.span;
    a.k_span = (uint32_t)rk.span;
    a.qw = static_cast<const char*>(q_weight);
    a.kw = static_cast<const char*>(k_weight);
    const int gpw = 64 / lph;
    a.nl = (heads + gpw - 1) / gpw;
    a.div_nl = make_fastdiv((uint32_t)a.nl);
    a.head_dim = head_dim;
    a.inv_head_dim = 1.0f / (float)head_dim;
    a.eps = eps;
    a.c1 = rope->d_t;
    a.c2 = rope->d_t + rope->d_h;
    h3f_status_t s = grid_args(rope, rows, a.grid);
    if (s != H3F_OK) return s;
    // Frequencies theta^(-2j/d_c), evaluated in double and rounded once to fp32.
    const int32_t dims[3] = {rope->d_t, rope->d_h, rope->d_w};
    int p = 0;
    for (int c = 0; c < 3; ++c)
        for (int32_t j = 0; j < dims[c] / 2; ++j)
            a.inv_freq[p++] = (float)pow(rope->theta, -2.0 * (double)j / (double)dims[c]);
    reg = QKRegions{rqo, rko, rq, rk, rw1, rw2};
    return H3F_OK;
}

template <bool HALF>
hipError_t launch_pool(const QKArgs& a, const PoolOut& p, hipStream_t st) {
    hipLaunchKernelGGL((qk_pool_kernel<__bf16, 8, 16, HALF>), dim3(2 * p.n_q_blocks),
                       dim3(64 * kPoolWaves), 0, st, a, p);
    return hipGetLastError();
}

}  // namespace

extern "C" h3f_status_t h3f_qk_rmsnorm_rope3d(
    void* q_out, int64_t q_out_row_stride, int64_t q_out_head_stride, void* k_out,
    int64_t k_out_row_stride, int64_t k_out_head_stride, const void* q, int64_t q_row_stride,
    int64_t q_head_stride, const void* k, int64_t k_row_stride, int64_t k_head_stride,
    const void* q_weight, const void* k_weight, h3f_dtype_t dtype, int64_t rows, int32_t heads,
    int32_t head_dim, float eps, const h3f_rope3d_t* rope, void* stream) {
    if (rows == 0) return H3F_OK;
    QKArgs a{};
    int lph = 0;
    QKRegions reg;
    const h3f_status_t s = qk_prepare(a, lph, reg, q_out, q_out_row_stride, q_out_head_stride,
                                      k_out, k_out_row_stride, k_out_head_stride, q,
                                      q_row_stride, q_head_stride, k, k_row_stride,
                                      k_head_stride, q_weight, k_weight, dtype, rows, heads,
                                      head_dim, eps, rope);
    if (s != H3F_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool half = rope->pairing == H3F_ROPE_HALF_SPLIT;
    hipError_t err;
    if (dtype == H3F_BF16)
        err = half ? dispatch_lph<__bf16, 8, true>(a, lph, rows, st)
                   : dispatch_lph<__bf16, 8, false>(a, lph, rows, st);
    else
        err = half ? dispatch_lph<float, 4, true>(a, lph, rows, st)
                   : dispatch_lph<float, 4, false>(a, lph, rows, st);
    return err == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}

extern "C" h3f_status_t h3f_qk_rmsnorm_rope3d_pool(
    void* q_out, int64_t q_out_row_stride, int64_t q_out_head_stride, void* k_out,
    int64_t k_out_row_stride, int64_t k_out_head_stride, const void* q, int64_t q_row_stride,
    int64_t q_head_stride, const void* k, int64_t k_row_stride, int64_t k_head_stride,
    const void* q_weight, const void* k_weight, h3f_dtype_t dtype, int64_t rows, int32_t heads,
    int32_t head_dim, float eps, const h3f_rope3d_t* rope, int32_t block, void* workspace,
    size_t workspace_bytes, void* stream) {
    if (!q_out || !k_out || !q || !k || !q_weight || !k_weight || !rope)
        return H3F_ERR_NULL_POINTER;
    // the router's preconditions (bf16, head_dim 128, rows >= 4096, block and
    // head counts) and its workspace size
    int32_t nb = 0;
    size_t need = 0;
    h3f_status_t s = h3f_subblock_plan(rows, heads, head_dim, block, 0.0,
                                       H3F_SUBBLOCK_FIRST_STEP, &nb, nullptr, &need);
    if (s != H3F_OK) return s;
    if (!dtype_ok(dtype)) return H3F_ERR_BAD_DTYPE;
    if (dtype != H3F_BF16) return H3F_ERR_UNSUPPORTED;
    QKArgs a{};
    int lph = 0;
    QKRegions reg;
    s = qk_prepare(a, lph, reg, q_out, q_out_row_stride, q_out_head_stride, k_out,
                   k_out_row_stride, k_out_head_stride, q, q_row_stride, q_head_stride, k,
                   k_row_stride, k_head_stride, q_weight, k_weight, dtype, rows, heads, head_dim,
                   eps, rope);
    if (s != H3F_OK) return s;
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return H3F_ERR_WORKSPACE;
    const Region rws = region2d(workspace, 1, 0, (int64_t)need, 1);
    const Region* others[] = {&reg.qo, &reg.ko, &reg.q, &reg.k, &reg.qw, &reg.kw};
    for (const Region* o : others)
        if (!disjoint(rws, *o)) return H3F_ERR_ALIASING;
    // kPoolTokens rows of a tensor are addressed through one 32-bit resource
    const int64_t rs_max = std::max(std::max(a.q_rs, a.k_rs), std::max(a.qo_rs, a.ko_rs));
    const int64_t span_max = std::max(std::max(reg.q.span, reg.k.span),
                                      std::max(reg.qo.span, reg.ko.span));
    if (rs_max > (0xFFFFFFF0ll - span_max) / kPoolTokens) return H3F_ERR_UNSUPPORTED;

    PoolOut p;
    p.pooled = static_cast<float*>(workspace);
    p.rows = rows;
    p.block = block;
    p.heads = heads;
    p.n_blocks = (uint32_t)nb;
    p.n_q_blocks = (uint32_t)nb * (uint32_t)a.nl;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t err = rope->pairing == H3F_ROPE_HALF_SPLIT ? launch_pool<true>(a, p, st)
                                                                 : launch_pool<false>(a, p, st);
    return err == hipSuccess ? H3F_OK : H3F_ERR_LAUNCH;
}
