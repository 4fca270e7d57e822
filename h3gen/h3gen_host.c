/*
 * h3gen_host.c -- host side of the seeded input generator (see h3gen_core.h).
 * Built with gcc -ffp-contract=off so z * sigma and + mu round separately,
 * exactly as the device side does.
 */
#include "h3gen_core.h"

#ifdef _OPENMP
#include <omp.h>
#endif

int h3gen_abi_version(void) { return 1; }

/*
 * Fill rows [row0, row0 + rows) of a logical [*, cols] tensor into dst, whose
 * rows are row_stride elements apart.  dtype: H3GEN_F32 or H3GEN_BF16.
 */
void h3gen_fill_host(void* dst, int dtype, int64_t row0, int64_t rows,
                     int64_t cols, int64_t row_stride, uint64_t seed,
                     uint64_t tensor_id, float mu, float sigma) {
    const uint64_t s = h3gen_stream(seed, tensor_id);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            const uint64_t i = (uint64_t)(row0 + r) * (uint64_t)cols + (uint64_t)c;
            float v = h3gen_unit(s, i) * sigma;
            v = v + mu;
            if (dtype == H3GEN_F32)
                ((float*)dst)[r * row_stride + c] = v;
            else
                ((uint16_t*)dst)[r * row_stride + c] = h3gen_bf16_rne(v);
        }
    }
}

/* Fill rows listed in row_ids (global logical rows) into a dense [n, cols] dst. */
void h3gen_fill_rows_host(void* dst, int dtype, const int64_t* row_ids,
                          int64_t n, int64_t cols, uint64_t seed,
                          uint64_t tensor_id, float mu, float sigma) {
    const uint64_t s = h3gen_stream(seed, tensor_id);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            const uint64_t i = (uint64_t)row_ids[r] * (uint64_t)cols + (uint64_t)c;
            float v = h3gen_unit(s, i) * sigma;
            v = v + mu;
            if (dtype == H3GEN_F32)
                ((float*)dst)[r * cols + c] = v;
            else
                ((uint16_t*)dst)[r * cols + c] = h3gen_bf16_rne(v);
        }
    }
}

/* Fill columns [col0, col0 + ncols) of rows [row0, row0 + rows) of a logical
 * [*, cols] tensor into a dense [rows, ncols] dst. */
void h3gen_fill_cols_host(void* dst, int dtype, int64_t row0, int64_t rows,
                          int64_t cols, int64_t col0, int64_t ncols,
                          uint64_t seed, uint64_t tensor_id, float mu,
                          float sigma) {
    const uint64_t s = h3gen_stream(seed, tensor_id);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < ncols; ++c) {
            const uint64_t i = (uint64_t)(row0 + r) * (uint64_t)cols + (uint64_t)(col0 + c);
            float v = h3gen_unit(s, i) * sigma;
            v = v + mu;
            if (dtype == H3GEN_F32)
                ((float*)dst)[r * ncols + c] = v;
            else
                ((uint16_t*)dst)[r * ncols + c] = h3gen_bf16_rne(v);
        }
    }
}
