// h3f_validate.hpp -- host-side argument validation for the libh3fused entry
// points.  Pure integer logic: no HIP call, so every error path can be driven
// on a machine without a GPU.
#pragma once

#include <stdint.h>

#include "../../include/h3fused.h"

namespace h3f {

inline int dtype_bytes(h3f_dtype_t t) { return t == H3F_BF16 ? 2 : 4; }
inline bool dtype_ok(int t) { return t == H3F_F32 || t == H3F_BF16; }

// Elements per lane chunk: 4 when any tensor of the call is fp32 (one 16-byte
// quad of fp32; bf16 streams then move 8 bytes per lane), 8 when all are bf16.
// Every load / store instruction of a wavefront is then contiguous.
inline int vec_width(bool any_f32) { return any_f32 ? 4 : 8; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Footprint of a strided tensor: rows x [0, span) bytes, rows `stride` bytes apart.
struct Region {
    uintptr_t base;
    int64_t rows;
    int64_t stride;  // bytes between rows (ignored when rows == 1)
    int64_t span;    // bytes touched inside one row

    uintptr_t lo() const { return base; }
    uintptr_t hi() const { return base + (uintptr_t)((rows > 1 ? (rows - 1) * stride : 0) + span); }
};

// The byte extent of rows x cols elements, rows `stride` elements apart, is
// below 2^62, so every footprint computed from these values (region2d, spans,
// offsets) stays inside int64.  Evaluated in 128-bit arithmetic.
inline bool extent_ok(int64_t rows, int64_t stride_elems, int64_t cols, int esize) {
    if (rows <= 0 || cols <= 0) return true;
    const __int128 s = stride_elems < 0 ? -(__int128)stride_elems : (__int128)stride_elems;
    const __int128 ext = ((__int128)(rows - 1) * s + cols) * esize;
    return ext < ((__int128)1 << 62);
}

inline Region region2d(const void* p, int64_t rows, int64_t row_stride_elems, int64_t cols,
                       int esize) {
    Region r;
    r.base = reinterpret_cast<uintptr_t>(p);
    r.rows = rows;
    r.stride = row_stride_elems * esize;
    r.span = cols * esize;
    return r;
}

inline bool same_region(const Region& a, const Region& b) {
    return a.base == b.base && a.rows == b.rows && a.span == b.span &&
           (a.rows <= 1 || a.stride == b.stride);
}

// True when the two footprints provably share no byte.  Exact for plain
// ranges and for two tensors interleaved with one common row stride (q, k, v
// of one packed buffer); conservative (reports overlap) otherwise.
inline bool disjoint(const Region& a, const Region& b) {
    if (a.rows <= 0 || b.rows <= 0 || a.span <= 0 || b.span <= 0) return true;
    if (a.hi() <= b.lo() || b.hi() <= a.lo()) return true;
    if (a.rows > 1 && b.rows > 1 && a.stride == b.stride && a.span <= a.stride &&
        b.span <= b.stride) {
        const int64_t S = a.stride;
        const int64_t diff = (int64_t)(b.base - a.base);
        int64_t d = diff % S;
        if (d < 0) d += S;
        // b's row starts d bytes into a's row period; its interval [d, d + span_b)
        // must sit between the end of a's interval and the start of a's next row.
        if (a.span <= d && d + b.span <= S) {
            // rows must also overlap in the period sense only; a different row
            // count cannot create a new overlap inside one period.
            return true;
        }
    }
    return false;
}

// An output may be exactly one of the inputs, or share no byte with it.
inline bool alias_ok(const Region& out, const Region& other, bool same_type) {
    if (same_region(out, other)) return same_type;
    return disjoint(out, other);
}

// Row footprint must not fold onto itself.
inline bool rows_separate(const Region& r) { return r.rows <= 1 || r.stride >= r.span; }

// ceil(n / d) for n >= 0, d >= 1, without the overflow of (n + d - 1) / d.
inline int64_t ceil_div(int64_t n, int64_t d) { return n / d + (n % d != 0); }

inline int64_t groups_for(int64_t rows, int64_t rows_per_group) {
    return ceil_div(rows, rows_per_group);
}

}  // namespace h3f
