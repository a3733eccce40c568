// Drives every argument check of the C ABI (include/fa2.h) that returns before
// a HIP call, for a build of fa2_api.hip's host code under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Fake, never dereferenced device addresses.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "fa2.h"

static int failures = 0;
#define EXPECT(call, want)                                                                       \
    do {                                                                                         \
        const fa2_status got_ = (call);                                                          \
        if (got_ != (want)) {                                                                    \
            std::fprintf(stderr, "line %d: %s -> %d, expected %d (%s)\n", __LINE__, #call,      \
                         (int)got_, (int)(want), fa2_last_error());                              \
            ++failures;                                                                          \
        }                                                                                        \
    } while (0)

static void* A(int i) { return reinterpret_cast<void*>((uintptr_t)1 << 40 | (uintptr_t)i << 36); }

int main() {
    void* p[10];
    for (int i = 0; i < 10; ++i) p[i] = A(i);
    const float* L = static_cast<const float*>(p[4]);
    const int B = 2, Hq = 4, Hkv = 2, N = 100, d = 128;
    const size_t ws = fa2_bwd_workspace_bytes(B, Hq, Hkv, N, d);
    const size_t ws_atomic = fa2_bwd_stages_workspace_bytes(FA2_BWD_ALL | FA2_BWD_DQ_ATOMIC, B, Hq, Hkv, N, d);
    if (ws == 0 || ws_atomic <= ws) ++failures;
    // Valid requests pass the validators.
    EXPECT(fa2_validate_fwd(p[0], p[1], p[2], p[3], L, B, Hq, Hkv, N, d, 1, 0.125f), FA2_OK);
    EXPECT(fa2_validate_bwd(p[0], p[1], p[2], p[3], L, p[5], p[6], p[7], p[8], p[9], ws, B, Hq, Hkv, N, d, 1,
                            0.125f), FA2_OK);
    // Sizes, head dims, scales, grouping, overflow.
    const int bad_sizes[][5] = {{-1, 4, 2, 100, 128}, {2, -4, 2, 100, 128}, {2, 4, -2, 100, 128},
                                {2, 4, 2, -100, 128}, {2, 6, 4, 100, 128}, {2, 4, 0, 100, 128}};
    for (const auto& s : bad_sizes)
        EXPECT(fa2_validate_fwd(p[0], p[1], p[2], p[3], L, s[0], s[1], s[2], s[3], s[4], 1, 0.125f),
               FA2_ERR_INVALID_ARGUMENT);
    for (int dd : {0, 1, 32, 96, 192, 512})
        EXPECT(fa2_validate_fwd(p[0], p[1], p[2], p[3], L, B, Hq, Hkv, N, dd, 1, 0.125f), FA2_ERR_UNSUPPORTED);
    for (float sc : {0.f, -1.f, __builtin_inff(), __builtin_nanf("")})
        EXPECT(fa2_validate_fwd(p[0], p[1], p[2], p[3], L, B, Hq, Hkv, N, d, 1, sc), FA2_ERR_INVALID_ARGUMENT);
    const int big = 0x7fffffff;
    if (fa2_validate_fwd(p[0], p[1], p[2], p[3], L, big, big, 1, big, 256, 1, 0.1f) == FA2_OK) ++failures;
    if (fa2_bwd_workspace_bytes(big, big, 1, big, 256) != 0) ++failures;
    // Empty problems with NULL pointers.
    EXPECT(fa2_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, Hq, Hkv, N, d, 1, 0.1f, nullptr), FA2_OK);
    EXPECT(fa2_bwd_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, B, Hq,
                           Hkv, 0, d, 1, 0.1f, nullptr), FA2_OK);
    // NULL, misaligned and aliased pointers; workspace size and alignment.
    for (int i = 0; i < 9; ++i) {
        void* q[10];
        std::memcpy(q, p, sizeof p);
        q[i] = nullptr;
        EXPECT(fa2_validate_bwd(q[0], q[1], q[2], q[3], static_cast<const float*>(q[4]), q[5], q[6], q[7], q[8],
                                q[9], ws, B, Hq, Hkv, N, d, 1, 0.125f), FA2_ERR_INVALID_ARGUMENT);
        q[i] = static_cast<char*>(p[i]) + 2;
        EXPECT(fa2_validate_bwd(q[0], q[1], q[2], q[3], static_cast<const float*>(q[4]), q[5], q[6], q[7], q[8],
                                q[9], ws, B, Hq, Hkv, N, d, 1, 0.125f), FA2_ERR_INVALID_ARGUMENT);
        q[i] = p[(i + 3) % 6];   // an output or input made to alias another buffer
        if (i >= 6)
            EXPECT(fa2_bwd(q[0], q[1], q[2], q[3], static_cast<const float*>(q[4]), q[5], q[6], q[7], q[8], q[9],
                           ws, B, Hq, Hkv, N, d, 1, 0.125f, nullptr), FA2_ERR_INVALID_ARGUMENT);
    }
    EXPECT(fa2_bwd(p[0], p[1], p[2], p[3], L, p[5], p[6], p[7], p[8], p[9], ws - 1, B, Hq, Hkv, N, d, 1, 0.125f,
                   nullptr), FA2_ERR_INVALID_ARGUMENT);
    EXPECT(fa2_bwd_stages(FA2_BWD_ALL | FA2_BWD_DQ_ATOMIC, p[0], p[1], p[2], p[3], L, p[5], p[6], p[7], p[8], p[9],
                          ws, B, Hq, Hkv, N, d, 1, 0.125f, nullptr), FA2_ERR_INVALID_ARGUMENT);
    EXPECT(fa2_bwd(p[0], p[1], p[2], p[3], L, p[5], p[6], p[7], p[8], static_cast<char*>(p[9]) + 16, ws, B, Hq,
                   Hkv, N, d, 1, 0.125f, nullptr), FA2_ERR_INVALID_ARGUMENT);
    for (unsigned m : {0u, 8u, 16u, 0xffffffffu})
        EXPECT(fa2_bwd_stages(m, p[0], p[1], p[2], p[3], L, p[5], p[6], p[7], p[8], p[9], ws, B, Hq, Hkv, N, d, 1,
                              0.125f, nullptr), FA2_ERR_INVALID_ARGUMENT);
    // f16 entry points share the checks.
    EXPECT(fa2_fwd_f16(p[0], p[1], p[2], p[3], static_cast<float*>(p[4]), B, 6, 4, N, d, 1, 0.1f, nullptr),
           FA2_ERR_INVALID_ARGUMENT);
    EXPECT(fa2_bwd_f16(p[0], p[1], p[2], p[3], L, p[5], p[6], p[7], p[8], p[9], ws, B, Hq, Hkv, N, 96, 1, 0.1f,
                       nullptr), FA2_ERR_UNSUPPORTED);
    // Block-sparse: mask NULL, unsupported head dim / N, output overlapping the mask.
    const unsigned char* mask = static_cast<const unsigned char*>(A(12));
    EXPECT(fa2_fwd_block_sparse(p[0], p[1], p[2], p[3], static_cast<float*>(p[4]), nullptr, B, Hq, Hkv, 300, d, 1,
                                0.1f, nullptr), FA2_ERR_INVALID_ARGUMENT);
    EXPECT(fa2_fwd_block_sparse(p[0], p[1], p[2], p[3], static_cast<float*>(p[4]), mask, 1, 1, 1, 262145, 64, 1,
                                0.1f, nullptr), FA2_ERR_UNSUPPORTED);
    EXPECT(fa2_fwd_block_sparse(p[0], p[1], p[2], p[3], static_cast<float*>(p[4]),
                                static_cast<const unsigned char*>(p[3]) + 64, B, Hq, Hkv, 300, d, 1, 0.1f, nullptr),
           FA2_ERR_INVALID_ARGUMENT);
    const size_t ws300 = fa2_bwd_workspace_bytes(B, Hq, Hkv, 300, d);
    EXPECT(fa2_bwd_block_sparse(p[0], p[1], p[2], p[3], L, p[5], p[6], p[7], p[8], nullptr, p[9], ws300, B, Hq, Hkv,
                                300, d, 1, 0.1f, nullptr), FA2_ERR_INVALID_ARGUMENT);
    // The allocation-free backward: checks, and problems above its static scratch.
    EXPECT(fa2_bwd_noalloc(p[0], p[1], p[2], p[3], L, p[5], p[6], p[7], p[8], B, 6, 4, N, d, 1, 0.1f, nullptr),
           FA2_ERR_INVALID_ARGUMENT);
    EXPECT(fa2_bwd_noalloc(p[0], p[1], p[2], p[3], L, p[5], p[6], p[7], p[8], 1, 33, 1, 65536, 64, 1, 0.1f,
                           nullptr), FA2_ERR_UNSUPPORTED);
    // Status strings and the last error.
    for (int s = -1; s < 6; ++s)
        if (!fa2_status_string(s)) ++failures;
    if (std::strlen(fa2_last_error()) == 0) ++failures;
    if (failures) std::fprintf(stderr, "%d failure(s)\n", failures);
    else std::printf("validators ok\n");
    return failures ? 1 : 0;
}
