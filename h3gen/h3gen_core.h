/*
 * h3gen_core.h -- seeded, counter-based input generator (host C and HIP device).
 *
 * This module produces the synthetic inputs that both the GPU library's tests
 * and the CPU oracle consume.  It holds none of the operators' arithmetic.
 *
 * Element value = f(seed, tensor_id, logical index), independent of memory
 * layout, so a strided tensor and a dense one with the same logical shape hold
 * the same values, and the host can regenerate any row that the device filled.
 *
 * Construction:
 *   - SplitMix64 (Steele, Lea & Flood, "Fast Splittable Pseudorandom Number
 *     Generators", OOPSLA 2014): state_n = s + n * GAMMA, output = mix(state_n).
 *     The stream start s is mix(mix(seed) + tensor_id * GAMMA).
 *   - Element i consumes outputs n = 3i, 3i+1, 3i+2 (192 bits) as twelve
 *     16-bit uniforms k_0..k_11 in [0, 65535].
 *   - Irwin-Hall sum of twelve U(0,1) variates (k + 1/2) / 65536: the sum
 *     minus 6 has mean 0, variance 1 - 2^-32 and lies in [-6, 6]; it stands in
 *     for N(0, 1).  In integers: z = (sum k - 393210) / 65536, exact in fp32.
 *   - value = fl32(fl32(z * sigma) + mu) with no fused multiply-add, then for
 *     bf16 storage one round-to-nearest-even of that fp32 value.
 * Every step is integer or a single correctly rounded fp32 operation, so host
 * and device results are bit-identical.
 */
#ifndef H3GEN_CORE_H
#define H3GEN_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define H3GEN_FN __host__ __device__ static inline
#else
#define H3GEN_FN static inline
#endif

#define H3GEN_GAMMA 0x9E3779B97F4A7C15ULL

enum { H3GEN_F32 = 0, H3GEN_BF16 = 1 };

H3GEN_FN uint64_t h3gen_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

H3GEN_FN uint64_t h3gen_stream(uint64_t seed, uint64_t tensor_id) {
    return h3gen_mix64(h3gen_mix64(seed) + tensor_id * H3GEN_GAMMA);
}

/* Irwin-Hall(12) - 6 for logical element i of the stream, as an exact fp32. */
H3GEN_FN float h3gen_unit(uint64_t stream, uint64_t i) {
    int32_t sum = 0;
    for (int j = 0; j < 3; ++j) {
        uint64_t w = h3gen_mix64(stream + (3 * i + (uint64_t)j + 1) * H3GEN_GAMMA);
        sum += (int32_t)(w & 0xffffu) + (int32_t)((w >> 16) & 0xffffu) +
               (int32_t)((w >> 32) & 0xffffu) + (int32_t)(w >> 48);
    }
    return (float)(sum - 393210) * (1.0f / 65536.0f);
}

H3GEN_FN uint32_t h3gen_f32_bits(float f) {
    union { float f; uint32_t u; } c;
    c.f = f;
    return c.u;
}

H3GEN_FN uint16_t h3gen_bf16_rne(float f) {
    uint32_t u = h3gen_f32_bits(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

#endif
