// Drives libkda's host side (argument validation, planning, size queries,
// plan descriptions) for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code.  Every call here either
// returns a status before anything is enqueued or is host-only, so no device
// is needed.  Addresses passed as tensors are never dereferenced: validation
// rejects the call first.  Exit status 0 when every call returned what the
// header promises.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "kda.h"

static int failures = 0;
#define EXPECT(cond)                                                                              \
    do {                                                                                          \
        if (!(cond)) {                                                                            \
            std::printf("FAILED line %d: %s (last error: %s)\n", __LINE__, #cond, kda_last_error()); \
            ++failures;                                                                           \
        }                                                                                         \
    } while (0)

static void* at(uintptr_t mib) { return reinterpret_cast<void*>(uintptr_t(0x10000) + (mib << 20)); }

int main()
{
    const kda_dtype_t BF = KDA_BF16, F = KDA_F32;
    EXPECT(kda_version() > 0);
    for (int s = 0; s <= 5; ++s) EXPECT(std::strlen(kda_status_string(kda_status_t(s))) > 0);
    EXPECT(std::strlen(kda_status_string(kda_status_t(99))) > 0);
    EXPECT(kda_last_error() != nullptr);

    // gate
    EXPECT(kda_gate(at(0), (const float*)at(1), at(2), -1, 2, 32, BF, -5.f, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_gate(at(0), (const float*)at(1), at(2), 4, 2, 32, kda_dtype_t(7), -5.f, nullptr) == KDA_ERR_UNSUPPORTED);
    EXPECT(kda_gate(at(0), (const float*)at(1), at(2), 4, 2, 32, BF, -5.5f, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_gate(at(0), (const float*)at(1), at(2), 4, 2, 32, BF, NAN, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_gate(nullptr, (const float*)at(1), at(2), 4, 2, 32, BF, -5.f, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_gate(nullptr, nullptr, nullptr, 0, 2, 32, BF, -5.f, nullptr) == KDA_OK);

    // workspace sizes and plans over a grid of shapes, valid and not
    const int dims[] = {16, 32, 64, 96, 128};
    const int64_t lens[] = {-1, 0, 1, 63, 64, 65, 8192, int64_t(1) << 20, int64_t(0x7fffffff), int64_t(1) << 31};
    for (int dk : dims)
        for (int dv : dims)
            for (int64_t T : lens)
                for (int N : {0, 1, 3})
                    for (kda_dtype_t dt : {BF, F}) {
                        const size_t w = kda_prefill_workspace_size(T, N, 8, dk, dv, 64, dt);
                        const int64_t n = kda_describe_prefill_plan(T, N, 8, dk, dv, dt, N > 1, nullptr, 0);
                        EXPECT((w == 0) == (n < 0) || T == 0);
                        if (n >= 0) {
                            std::string buf(size_t(n) + 1, 'x');
                            EXPECT(kda_describe_prefill_plan(T, N, 8, dk, dv, dt, N > 1, &buf[0], buf.size()) == n);
                            EXPECT(buf[size_t(n)] == '\0' && std::strlen(buf.c_str()) == size_t(n));
                            char small[7];
                            EXPECT(kda_describe_prefill_plan(T, N, 8, dk, dv, dt, N > 1, small, sizeof(small)) == n);
                            EXPECT(std::strlen(small) == sizeof(small) - 1);
                        }
                        const size_t wb = kda_backward_workspace_size(T, N, 8, dk, dv);
                        const int64_t nb = kda_describe_backward_plan(T, N, 8, dk, dv, dt, nullptr, 0);
                        EXPECT((wb == 0) == (nb < 0));
                        (void)kda_test_prefill_workspace_size(T, N, 8, dk, dv, dt, 3, 64);
                        (void)kda_test_backward_workspace_size(T, N, 8, dk, dv, 192);
                        size_t off = 0;
                        (void)kda_test_prefill_flags(T, N, 8, dk, dv, dt, 0, -1, &off);
                    }
    EXPECT(kda_describe_prefill_plan(64, 1, 2, 32, 32, BF, 0, nullptr, 8) == -1);

    // checkpoint counts from a host cu_seqlens
    const int32_t cu[5] = {0, 700, 700, 1800, 1800};
    EXPECT(kda_checkpoint_count(cu, 4, 1800, 512) == 1 + 2);
    EXPECT(kda_checkpoint_count(nullptr, 1, 1800, 64) == 1800 / 64);
    EXPECT(kda_checkpoint_count(cu, 4, 1800, 0) < 0);
    EXPECT(kda_checkpoint_count(cu, 0, 1800, 64) < 0);

    // prefill rejections
    const size_t need = kda_prefill_workspace_size(256, 1, 2, 64, 64, 64, BF);
    auto prefill = [&](int N, int64_t T, int dk, kda_dtype_t dt, void* o, size_t wsb) {
        return kda_prefill(at(0), at(1), at(2), at(3), at(4), nullptr, N, T, 2, dk, 64, 64, nullptr,
                           (float*)at(8), o, dt, at(32), wsb, nullptr);
    };
    EXPECT(prefill(0, 256, 64, BF, at(16), need) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(prefill(3, 256, 64, BF, at(16), need) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(prefill(1, 256, 96, BF, at(16), need) == KDA_ERR_UNSUPPORTED);
    EXPECT(prefill(1, 256, 64, F, at(16), 0) == KDA_ERR_WORKSPACE_TOO_SMALL);  // the fp32 token-serial path
    EXPECT(prefill(1, int64_t(1) << 31, 64, BF, at(16), need) == KDA_ERR_UNSUPPORTED);
    EXPECT(prefill(1, 256, 64, BF, nullptr, need) == KDA_ERR_INVALID_ARGUMENT);
    if (need > 0) EXPECT(prefill(1, 256, 64, BF, at(16), need - 1) == KDA_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(prefill(1, 256, 64, BF, (char*)at(0) + 8, need) == KDA_ERR_INVALID_ARGUMENT);  // o aliases q

    // the no-allocation form refuses what its static scratch cannot hold (64
    // packed sequences over 2^30 tokens: hundreds of MB of workspace)
    EXPECT(kda_prefill_gated_noalloc(at(0), at(1), at(2), at(3), (const float*)at(4), -5.f, at(5),
                                     (const int32_t*)at(6), 64, int64_t(1) << 30, 64, 128, 128, 64, nullptr,
                                     (float*)at(8), at(16), BF, 0, nullptr, 0, nullptr) == KDA_ERR_UNSUPPORTED);

    // backward rejections
    const size_t bneed = kda_backward_workspace_size(256, 1, 2, 64, 64);
    auto backward = [&](int N, int64_t T, int dk, const float* ck, int64_t cap, int iv, size_t wsb) {
        return kda_backward(at(0), at(1), at(2), at(3), at(4), nullptr, N, T, 2, dk, 64, nullptr, ck, cap, iv, at(5),
                            nullptr, (float*)at(8), (float*)at(9), (float*)at(10), (float*)at(11), (float*)at(12),
                            (float*)at(13), BF, at(64), wsb, nullptr);
    };
    EXPECT(backward(0, 256, 64, nullptr, 0, 64, bneed) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(backward(1, 256, 96, nullptr, 0, 64, bneed) == KDA_ERR_UNSUPPORTED);
    EXPECT(backward(1, 256, 64, (const float*)at(20), 4, 96, bneed) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(backward(1, 8192, 64, nullptr, 0, 64, bneed) == KDA_ERR_UNSUPPORTED);  // long input, no checkpoints
    EXPECT(backward(1, 256, 64, nullptr, 0, 64, bneed - 1) == KDA_ERR_WORKSPACE_TOO_SMALL);

    // decode, verify, commit rejections
    EXPECT(kda_decode_step(at(0), at(1), at(2), at(3), at(4), (float*)at(8), at(64), 4, 2, 96, 64, BF, nullptr) ==
           KDA_ERR_UNSUPPORTED);
    EXPECT(kda_decode_step(at(0), at(1), at(2), at(3), at(4), (float*)((char*)at(8) + 4), at(64), 4, 2, 64, 64, BF,
                           nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_decode_step(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 2, 64, 64, BF,
                           nullptr) == KDA_OK);
    EXPECT(kda_decode_step_gated(at(0), at(1), at(2), at(3), (const float*)at(5), 0.5f, at(4), (float*)at(8), at(64),
                                 4, 2, 64, 64, BF, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_verify(at(0), at(1), at(2), at(3), at(4), (const float*)at(8), at(64), 4, KDA_MAX_DRAFT + 1, 2, 64,
                      64, BF, nullptr) != KDA_OK);
    EXPECT(kda_commit(at(1), at(2), at(3), at(4), (const int32_t*)at(96), (float*)at(8), 4, 0, 2, 64, 64, BF,
                      nullptr) != KDA_OK);

    std::printf("libkda host driver: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
