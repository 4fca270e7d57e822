// Calls every libh3fused entry point with invalid and extreme arguments --
// null, misaligned, bad shapes, overlapping, and strides whose footprints
// overflow 64-bit byte counts -- so that an address/undefined-behaviour
// sanitizer build of the library's host code can check the validation layer.
// Every call here must be rejected before any launch (fake device addresses
// are never dereferenced).  Exit status 0 when every status matches.
#include <cstdint>
#include <cstdio>

#include "h3fused.h"

static int failures = 0;
#define EXPECT(call, want)                                                               \
    do {                                                                                 \
        const int got = (int)(call);                                                     \
        if (got != (int)(want)) {                                                        \
            std::printf("line %d: got %d want %d\n", __LINE__, got, (int)(want));        \
            ++failures;                                                                  \
        }                                                                                \
    } while (0)

static void* A(int n) { return reinterpret_cast<void*>(uintptr_t(0x10000000) * (n + 1)); }

int main() {
    const int64_t big = int64_t(1) << 61, huge = INT64_MAX - 7;
    const h3f_dtype_t B = H3F_BF16, F = H3F_F32;

    // gated residual
    EXPECT(h3f_gated_residual(nullptr, B, 256, A(1), B, 256, A(2), 0, 10, 10, 256, nullptr),
           H3F_ERR_NULL_POINTER);
    EXPECT(h3f_gated_residual(A(0), B, big, A(1), B, 256, A(2), 0, 10, 10, 256, nullptr),
           H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_gated_residual(A(0), B, huge & ~int64_t(7), A(1), B, 256, A(2), 0, 10, 10, 256,
                              nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_gated_residual(A(0), B, -256, A(1), B, 256, A(2), 0, 10, 10, 256, nullptr),
           H3F_ERR_BAD_STRIDE);
    EXPECT(h3f_gated_residual(A(0), B, 256, A(1), B, 256, A(2), 0, 10, int64_t(1) << 40, 256,
                              nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_gated_residual(A(0), B, 260, A(1), B, 256, A(2), 0, INT64_MAX, 10, 256, nullptr),
           H3F_ERR_BAD_STRIDE);  // group count of a huge rows_per_group
    // SwiGLU
    EXPECT(h3f_swiglu(A(0), 64, A(1), big, A(2), 128, B, 10, 64, nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_swiglu(A(0), 64, A(1), 128, A(2), 128, B, 10, huge & ~int64_t(7), nullptr),
           H3F_ERR_UNSUPPORTED);
    // AdaLN and the fused form
    EXPECT(h3f_adaln_modulate(A(0), B, 512, A(1), B, big, A(2), A(3), 0, 4, 10, 512, 1e-6f,
                              nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_adaln_modulate(A(0), B, 512, A(1), B, 512, A(2), A(3), huge & ~int64_t(7), 1, 10,
                              512, 1e-6f, nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_adaln_affine_modulate(A(0), B, 512, A(1), B, big, A(6), A(7), A(2), A(3), 0, 4,
                                     10, 512, 1e-6f, nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_adaln_affine_modulate(A(0), B, 512, A(1), B, 512, nullptr, A(7), A(2), A(3), 0, 4,
                                     10, 512, 1e-6f, nullptr), H3F_ERR_NULL_POINTER);
    EXPECT(h3f_adaln_affine_modulate(A(0), B, 512, A(1), B, 512, A(6), A(7), A(2), A(3),
                                     huge & ~int64_t(7), 1, 10, 512, 1e-6f, nullptr),
           H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_gated_residual_adaln(A(0), F, 512, A(1), B, big, A(2), A(3), A(4), 0, 4, A(5), B,
                                    512, 10, 512, 1e-6f, nullptr), H3F_ERR_UNSUPPORTED);
    // QK RMSNorm + RoPE
    h3f_rope3d_t r{};
    r.T = 2; r.H = 6; r.W = 8; r.n_audio = 16; r.d_t = 32; r.d_h = 48; r.d_w = 48;
    r.pairing = H3F_ROPE_INTERLEAVED; r.theta = 10000.0;
    EXPECT(h3f_qk_rmsnorm_rope3d(A(0), 5120, big, A(1), 5120, 128, A(2), 5120, 128, A(3), 5120,
                                 128, A(4), A(5), B, 10, 40, 128, 1e-6f, &r, nullptr),
           H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_qk_rmsnorm_rope3d(A(0), huge & ~int64_t(7), 128, A(1), 5120, 128, A(2), 5120, 128,
                                 A(3), 5120, 128, A(4), A(5), B, 10, 40, 128, 1e-6f, &r, nullptr),
           H3F_ERR_UNSUPPORTED);
    r.token_offset = INT64_MIN;
    EXPECT(h3f_qk_rmsnorm_rope3d(A(0), 5120, 128, A(1), 5120, 128, A(2), 5120, 128, A(3), 5120,
                                 128, A(4), A(5), B, 10, 40, 128, 1e-6f, &r, nullptr),
           H3F_ERR_BAD_SHAPE);
    r.token_offset = 0;
    r.T = INT32_MAX; r.H = INT32_MAX; r.W = INT32_MAX;
    EXPECT(h3f_rope3d_positions(static_cast<int32_t*>(A(0)), 10, &r, nullptr),
           H3F_ERR_UNSUPPORTED);
    // residual difference
    EXPECT(h3f_residual_l1(static_cast<double*>(A(0)), A(1), big, A(2), 512, B, 4, 512, A(3),
                           1 << 20, nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT((int)h3f_residual_l1_workspace_bytes(INT64_MAX, 8, B), 0);  // unsupported size
    EXPECT((int)(h3f_residual_l1_workspace_bytes(125120, 5120, B) > 0), 1);
    // router
    int32_t nb = 0, keep = 0;
    size_t ws = 0;
    EXPECT(h3f_subblock_plan(INT64_MAX, 1, 128, 1, 0.8, 10, &nb, &keep, &ws), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_subblock_plan(125120, 40, 128, 128, 0.8, 10, &nb, &keep, &ws), H3F_OK);
    EXPECT(nb, 978);
    EXPECT(keep, 196);
    EXPECT(h3f_subblock_route(static_cast<int32_t*>(A(0)), static_cast<float*>(A(1)), 32, A(2),
                              huge & ~int64_t(7), 128, A(3), 1024, 128, B, 4096, 8, 128, 128,
                              0.8, 10, A(4), 1 << 20, nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_subblock_route(static_cast<int32_t*>(A(0)), static_cast<float*>(A(1)), 32, A(2),
                              1024, big, A(3), 1024, 128, B, 4096, 8, 128, 128, 0.8, 10, A(4),
                              1 << 20, nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_subblock_route(static_cast<int32_t*>(A(0)), static_cast<float*>(A(1)), 32, A(2),
                              1024, 128, A(3), 1024, 128, B, int64_t(1) << 44, 8, 128,
                              INT32_MAX, 0.8, 10, A(4), 1 << 20, nullptr), H3F_ERR_UNSUPPORTED);
    // QK with the router pooling fused in, and the route from pooled means
    EXPECT(h3f_qk_rmsnorm_rope3d_pool(A(0), 5120, 128, A(1), 5120, 128, A(2), big, 128, A(3), 5120,
                                      128, A(4), A(5), B, 4096, 40, 128, 1e-6f, &r, 128, A(6),
                                      1 << 24, nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_qk_rmsnorm_rope3d_pool(A(0), 5120, 128, A(1), 5120, 128, A(2), 5120, 128, A(3),
                                      5120, 128, A(4), A(5), B, INT64_MAX, 40, 128, 1e-6f, &r, 128,
                                      A(6), 1 << 24, nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_subblock_route(static_cast<int32_t*>(A(0)), static_cast<float*>(A(1)), INT64_MAX,
                              A(2), 1024, 128, A(3), 1024, 128, B, 4096, 8, 128, 128, 0.8, 10,
                              A(4), 1 << 20, nullptr), H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_subblock_route_pooled(static_cast<int32_t*>(A(0)), static_cast<float*>(A(1)),
                                     32, INT64_MAX, 8, 128, 1, 0.8, 10, A(2), 1 << 20, nullptr),
           H3F_ERR_UNSUPPORTED);
    EXPECT(h3f_subblock_route_pooled(static_cast<int32_t*>(A(0)), static_cast<float*>(A(1)),
                                     32, int64_t(1) << 44, 8, 128, INT32_MAX, 0.8, 10, A(2),
                                     1 << 20, nullptr), H3F_ERR_UNSUPPORTED);
    // copy helper
    EXPECT(h3f_stream_copy(A(0), A(1), -16, nullptr), H3F_ERR_BAD_SHAPE);
    EXPECT(h3f_stream_copy(A(0), A(0), 1 << 20, nullptr), H3F_ERR_ALIASING);
    for (int s = 0; s <= 10; ++s)
        if (!h3f_status_string(static_cast<h3f_status_t>(s))) ++failures;
    std::printf("abi sanitizer run: %s (%d mismatches)\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
