// h3gen_device.hip -- device side of the seeded input generator (see h3gen_core.h).
//
// One thread per element of a logical [rows, cols] tensor stored with a row
// stride.  __fmul_rn / __fadd_rn keep the two fp32 roundings separate (no
// contraction into a fused multiply-add), which makes the values
// bit-identical to the host side.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3gen_core.h"

namespace {

template <int DTYPE>
__global__ void __launch_bounds__(256) fill_kernel(void* __restrict__ dst, int64_t row0, int64_t rows,
                                                   int64_t cols, int64_t row_stride, uint64_t stream,
                                                   float mu, float sigma) {
    const int64_t total = rows * cols;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += step) {
        const int64_t r = e / cols;
        const int64_t c = e - r * cols;
        const uint64_t i = (uint64_t)(row0 + r) * (uint64_t)cols + (uint64_t)c;
        const float v = __fadd_rn(__fmul_rn(h3gen_unit(stream, i), sigma), mu);
        if (DTYPE == H3GEN_F32)
            static_cast<float*>(dst)[r * row_stride + c] = v;
        else
            static_cast<uint16_t*>(dst)[r * row_stride + c] = h3gen_bf16_rne(v);
    }
}

}  // namespace

extern "C" int h3gen_dev_abi_version(void) { return 1; }

// Returns 0 on success, a hipError_t value otherwise.  Asynchronous on stream.
extern "C" int h3gen_fill_device(void* dst, int dtype, int64_t row0, int64_t rows, int64_t cols,
                                 int64_t row_stride, uint64_t seed, uint64_t tensor_id, float mu,
                                 float sigma, void* stream) {
    if (rows <= 0 || cols <= 0) return 0;
    if (!dst || row_stride < cols || (dtype != H3GEN_F32 && dtype != H3GEN_BF16))
        return (int)hipErrorInvalidValue;
    const uint64_t s = h3gen_stream(seed, tensor_id);
    const int64_t total = rows * cols;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == H3GEN_F32)
        hipLaunchKernelGGL(fill_kernel<H3GEN_F32>, dim3((unsigned)blocks), dim3(256), 0, st, dst,
                           row0, rows, cols, row_stride, s, mu, sigma);
    else
        hipLaunchKernelGGL(fill_kernel<H3GEN_BF16>, dim3((unsigned)blocks), dim3(256), 0, st, dst,
                           row0, rows, cols, row_stride, s, mu, sigma);
    return (int)hipGetLastError();
}
