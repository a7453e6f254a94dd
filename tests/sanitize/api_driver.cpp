// Drives the host side of libgdn2's C ABI on the paths that need no GPU -- workspace and buffer
// sizes, every argument check that refuses a call before any launch, the status strings -- so
// that a build with AddressSanitizer and UndefinedBehaviorSanitizer on the host code can check
// them.  Fake device pointers are never dereferenced: each call must fail its checks first.
// Exit 0 on success.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn2.h"

static int fails = 0;
#define EXPECT(cond)                                             \
    do {                                                         \
        if (!(cond)) {                                           \
            printf("FAILED line %d: %s\n", __LINE__, #cond);     \
            ++fails;                                             \
        }                                                        \
    } while (0)

int main() {
    void *f = reinterpret_cast<void *>(uintptr_t(0x10000)), *odd = reinterpret_cast<void *>(uintptr_t(0x10008));
    float *ff = static_cast<float *>(f);
    const size_t bad = (size_t)-1;
    for (int dk : {32, 64, 128, 96})
        for (int dv : {32, 64, 128, 256})
            for (int dt : {0, 1}) {
                gdn2_shape s = {3, 257, 5, dk, dv, 64, dt, 0, 0};
                const bool ok = dk != 96 && dv != 256;
                EXPECT((gdn2_chunk_fwd_workspace_size(&s) == bad) == !ok);
                EXPECT((gdn2_chunk_bwd_workspace_size(&s) == bad) == !ok);
                EXPECT((gdn2_chunk_factors_bytes(&s) == bad) == !ok);
                EXPECT((gdn2_chunk_states_bytes(&s) == bad) == !ok);
                EXPECT((gdn2_output_bwd_workspace_size(&s) == bad) == !ok);
                EXPECT(gdn2_chunk_sweeps_fused(&s) == (ok ? gdn2_chunk_sweeps_fused(&s) : -1));
            }
    gdn2_shape s = {2, 100, 3, 128, 64, 64, 1, 0, 0};
    EXPECT(gdn2_chunk_fwd(nullptr, f, f, f, f, f, f, nullptr, ff, nullptr, f, 1, nullptr) == GDN2_ERR_INVALID_ARG);
    EXPECT(gdn2_chunk_fwd(&s, f, f, f, f, f, f, nullptr, nullptr, nullptr, f, 1, nullptr) == GDN2_ERR_INVALID_ARG);
    EXPECT(gdn2_chunk_fwd(&s, odd, f, f, f, f, f, nullptr, ff, nullptr, f, 1 << 30, nullptr) == GDN2_ERR_INVALID_ARG);
    EXPECT(gdn2_chunk_fwd(&s, f, f, f, f, f, f, nullptr, ff, nullptr, nullptr, 0, nullptr) == GDN2_ERR_WORKSPACE);
    EXPECT(gdn2_chunk_fwd(&s, f, f, f, f, f, f, nullptr, ff, nullptr, f, 16, nullptr) == GDN2_ERR_WORKSPACE);
    EXPECT(gdn2_chunk_bwd(&s, f, f, f, f, f, f, nullptr, ff, nullptr, ff, ff, ff, ff, ff, ff, nullptr, nullptr, 0,
                          nullptr) == GDN2_ERR_WORKSPACE);
    EXPECT(gdn2_chunk_bwd(&s, f, f, f, f, f, f, nullptr, nullptr, nullptr, ff, ff, ff, ff, ff, ff, nullptr, f, 1 << 30,
                          nullptr) == GDN2_ERR_INVALID_ARG);
    EXPECT(gdn2_chunk_bwd_factors(&s, f, f, f, f, nullptr, nullptr) == GDN2_ERR_INVALID_ARG);
    EXPECT(gdn2_chunk_fwd_factored(&s, f, f, f, nullptr, nullptr, nullptr, nullptr, nullptr) == GDN2_ERR_INVALID_ARG);
    EXPECT(gdn2_chunk_bwd_reverse(&s, f, ff, nullptr, nullptr, nullptr, nullptr) == GDN2_ERR_INVALID_ARG);
    EXPECT(gdn2_chunk_sweeps(&s, f, f, f, nullptr, ff, nullptr, nullptr, nullptr, ff, ff, nullptr, nullptr) ==
           GDN2_ERR_INVALID_ARG);
    EXPECT(gdn2_chunk_bwd_grads(&s, f, f, f, f, f, f, ff, ff, ff, nullptr, ff, ff, ff, ff, ff, ff, nullptr) ==
           GDN2_ERR_INVALID_ARG);
    gdn2_shape one = s;
    one.T = 2;
    EXPECT(gdn2_step(&one, f, f, f, f, f, f, nullptr, ff, ff, nullptr) == GDN2_ERR_INVALID_ARG);
    EXPECT(gdn2_output_fwd(&s, ff, f, 0, nullptr, -1.f, f, 0, nullptr) == GDN2_ERR_INVALID_ARG);
    EXPECT(gdn2_output_bwd(&s, ff, f, 0, nullptr, 1e-6f, ff, ff, ff, ff, nullptr, 0, nullptr) == GDN2_ERR_WORKSPACE);
    gdn2_shape big = {1, 16384, 16, 128, 128, 64, 1, 0, 0};
    EXPECT(gdn2_chunk_fwd_noalloc(&big, f, f, f, f, f, f, nullptr, ff, nullptr, nullptr) == GDN2_ERR_SCRATCH);
    gdn2_shape badchunk = s;
    badchunk.chunk = 32;
    EXPECT(gdn2_chunk_fwd_noalloc(&badchunk, f, f, f, f, f, f, nullptr, ff, nullptr, nullptr) == GDN2_ERR_UNSUPPORTED);
    gdn2_shape huge = {1 << 14, 1 << 14, 16, 128, 128, 64, 1, 0, 0};
    EXPECT(gdn2_chunk_fwd_workspace_size(&huge) == bad);
    for (int c = -1; c < 8; ++c) EXPECT(gdn2_strerror(c) != nullptr && strlen(gdn2_strerror(c)) > 0);
    printf("%s (%d failed)\n", fails ? "FAILED" : "ok", fails);
    return fails != 0;
}
