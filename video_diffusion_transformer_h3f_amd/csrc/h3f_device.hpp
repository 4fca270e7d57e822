// h3f_device.hpp -- device-side building blocks shared by the libh3fused kernels:
// 16-byte vector memory access, bf16 <-> fp32 conversion, and DPP / swizzle
// reductions inside groups of lanes of a 64-wide wavefront (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3f {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// 16-byte loads / stores.  The non-temporal forms mark streams that are
// touched once, so they do not displace reused data (modulation vectors,
// norm weights) from the caches.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ---------------------------------------------------------------------------
// Buffer (MUBUF) access through a wave-uniform resource over [base, base +
// bytes).  Loads outside the range return 0 and stores outside it are
// dropped, so a row's ragged tail needs no branch.  The cache-policy bits of
// gfx950 (sc0 = 1, nt = 2, sc1 = 16) are chosen per stream:
//   kLoadStream  = nt             streaming read, not kept in L2
//   kStoreStream = sc0 | sc1 | nt streaming write-through: measured on MI355X
//                                 as the fastest store form for data that is
//                                 not re-read (about 3% over nt alone)
//   kLoadReuse   = 0              cached read (modulation vectors, weights)
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

#ifndef H3F_LOAD_AUX
#define H3F_LOAD_AUX 2
#endif
#ifndef H3F_STORE_AUX
#define H3F_STORE_AUX 19
#endif
constexpr int kLoadStream = H3F_LOAD_AUX;
constexpr int kStoreStream = H3F_STORE_AUX;
constexpr int kLoadReuse = 0;

// Data-format word of a raw 32-bit buffer resource on gfx9.
constexpr int kRsrcFlags = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRsrcFlags);
}

template <int AUX>
__device__ __forceinline__ u32x4 buf_ld(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}

template <int AUX>
__device__ __forceinline__ void buf_st(rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, AUX);
}

// Byte count of a resource covering `rows` rows of `row_bytes` bytes spaced
// `stride_bytes` apart, clamped to what a resource can address.
__host__ __device__ __forceinline__ uint32_t span_bytes(int64_t rows, int64_t stride_bytes,
                                                        int64_t row_bytes) {
    if (rows <= 0) return 0;
    const int64_t b = (rows - 1) * stride_bytes + row_bytes;
    return b > 0xFFFFFFF0ll ? 0xFFFFFFF0u : (uint32_t)b;
}

// Make a wave-uniform value provably uniform (lives in an SGPR).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// Vec<T, N>: N consecutive elements of storage type T (float or __bf16) held
// raw (whole 16-byte quads, or one 8-byte pair for 4 bf16 next to fp32
// streams); widened to fp32 on use, narrowed with one round-to-nearest-even
// (v_cvt_pk_bf16_f32 on gfx950) on store.
// ---------------------------------------------------------------------------
template <typename T, int N>
struct Vec {
    static constexpr int kBytes = N * (int)sizeof(T);
    static_assert(kBytes == 8 || (kBytes >= 16 && kBytes % 16 == 0),
                  "vector must be 8 bytes or whole 16-byte quads");
    static constexpr int kQuads = kBytes / 16;  // 0 for an 8-byte vector
    static constexpr int kWords = kBytes / 4;
    u32x4 q[kQuads > 0 ? kQuads : 1];  // an 8-byte vector uses q[0].xy

    __device__ __forceinline__ unsigned word(int i) const { return q[i / 4][i % 4]; }
    __device__ __forceinline__ void set_word(int i, unsigned v) { q[i / 4][i % 4] = v; }

    template <bool NT>
    __device__ __forceinline__ void load(const T* p) {
        if constexpr (kBytes == 8) {
            const u32x2 v = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p))
                               : *reinterpret_cast<const u32x2*>(p);
            q[0][0] = v[0];
            q[0][1] = v[1];
        } else {
#pragma unroll
            for (int i = 0; i < kQuads; ++i)
                q[i] = NT ? ld16_nt(p + i * (16 / (int)sizeof(T))) : ld16(p + i * (16 / (int)sizeof(T)));
        }
    }
    // Buffer forms: byte offset of the first element inside the resource.
    template <int AUX>
    __device__ __forceinline__ void load_buf(rsrc_t r, uint32_t off) {
        if constexpr (kBytes == 8) {
            const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
            q[0][0] = v[0];
            q[0][1] = v[1];
        } else {
#pragma unroll
            for (int i = 0; i < kQuads; ++i) q[i] = buf_ld<AUX>(r, off + 16u * i);
        }
    }
    template <int AUX>
    __device__ __forceinline__ void store_buf(rsrc_t r, uint32_t off) const {
        if constexpr (kBytes == 8) {
            const u32x2 v = {q[0][0], q[0][1]};
            __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, AUX);
        } else {
#pragma unroll
            for (int i = 0; i < kQuads; ++i) buf_st<AUX>(r, off + 16u * i, q[i]);
        }
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < (kQuads > 0 ? kQuads : 1); ++i) q[i] = u32x4{0u, 0u, 0u, 0u};
    }
    __device__ __forceinline__ void to_float(float (&f)[N]) const {
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < kWords; ++i) f[i] = __uint_as_float(word(i));
        } else {
#pragma unroll
            for (int i = 0; i < kWords; ++i) {
                f[2 * i] = __uint_as_float(word(i) << 16);
                f[2 * i + 1] = __uint_as_float(word(i) & 0xffff0000u);
            }
        }
    }
    __device__ __forceinline__ void from_float(const float (&f)[N]) {
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < kWords; ++i) set_word(i, __float_as_uint(f[i]));
        } else {
#pragma unroll
            for (int i = 0; i < kWords; ++i) {
                const f32x2 v = {f[2 * i], f[2 * i + 1]};
                set_word(i, __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2)));
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Reductions over aligned groups of L lanes (L = 1, 2, ..., 64).  Every lane of
// a group ends with the same, bit-identical sum (each step adds a value and its
// mirror, and fp32 addition is commutative).  Steps:
//   xor 1, xor 2  : DPP quad_perm
//   8-lane       : DPP row_half_mirror (lane i <- 7 - i within 8)
//   16-lane      : DPP row_mirror      (lane i <- 15 - i within 16)
//   32-lane      : ds_swizzle, xor 16 within 32
//   64-lane      : ds_bpermute, xor 32
// The caller keeps all 64 lanes active at the call.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int L>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16 || L == 32 || L == 64, "L");
    if constexpr (L >= 2) v += dpp_mov<0xB1>(v);   // quad_perm(1,0,3,2)
    if constexpr (L >= 4) v += dpp_mov<0x4E>(v);   // quad_perm(2,3,0,1)
    if constexpr (L >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror
    if constexpr (L >= 16) v += dpp_mov<0x140>(v); // row_mirror
    if constexpr (L >= 32)
        v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // xor 16
    if constexpr (L >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Sum over the whole wavefront, returned as a wave-uniform value.
__device__ __forceinline__ float wave_sum(float v) {
    v = group_sum<32>(v);
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    return lo + hi;
}

// ---------------------------------------------------------------------------
// Workgroup order across the XCDs.  Workgroups of a launch are dealt to the 8
// XCDs round robin (workgroup w runs on XCD w mod 8), each with its own L2.
// xcd_linear(w, n) renumbers them so that each XCD takes one contiguous run of
// the n work items instead of every eighth one.
// ---------------------------------------------------------------------------
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint32_t xcd_linear(uint32_t w, uint32_t n) {
    const uint32_t per = n / kXcds, extra = n % kXcds;
    const uint32_t x = w % kXcds, slot = w / kXcds;
    return x < extra ? x * (per + 1) + slot : extra * (per + 1) + (x - extra) * per + slot;
}

// ---------------------------------------------------------------------------
// Unsigned 32-bit division by a run-time invariant divisor d >= 1 for
// dividends n < 2^31: q = (mulhi(n, m) + n) >> s with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1 (Granlund & Montgomery, PLDI 1994, sec. 4).
// ---------------------------------------------------------------------------
struct FastDiv {
    uint32_t d, m, s;
};

__host__ inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((uint64_t(1) << s) < d) ++s;
    f.s = s;
    f.m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return (__umulhi(n, f.m) + n) >> f.s;
}

}  // namespace h3f
