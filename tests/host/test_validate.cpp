// Host-only unit test of the C ABI's argument checks (fa_validate.h).
// Built with g++ (no HIP) and run on the CPU; exits non-zero on the first failure.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <string_view>

#include "fa_validate.h"

static int failures = 0;
#define EXPECT_EQ(a, b)                                                                \
    do {                                                                               \
        const long long _a = (long long)(a), _b = (long long)(b);                     \
        if (_a != _b) {                                                                \
            std::fprintf(stderr, "%s:%d: %s = %lld, expected %lld\n", __FILE__,        \
                         __LINE__, #a, _a, _b);                                        \
            ++failures;                                                                \
        }                                                                              \
    } while (0)

int main() {
    using namespace fa_host;
    int dummy = 0;
    const void* p = &dummy;
    const float inf = std::numeric_limits<float>::infinity();
    const float nan = std::numeric_limits<float>::quiet_NaN();

    // forward: valid
    EXPECT_EQ(check_fwd(p, p, p, p, 8, 16, 2048, 128, 0, 0.088f, FA_BF16), FA_OK);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 2, 256, 64, 1, 0.125f, FA_F32), FA_OK);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, 1, 64, 1, 0.f, FA_BF16), FA_OK);
    // forward: invalid
    EXPECT_EQ(check_fwd(nullptr, p, p, p, 1, 1, 1, 64, 0, 1.f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, nullptr, p, p, 1, 1, 1, 64, 0, 1.f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, nullptr, p, 1, 1, 1, 64, 0, 1.f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, p, nullptr, 1, 1, 1, 64, 0, 1.f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, p, p, 0, 1, 1, 64, 0, 1.f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 0, 1, 64, 0, 1.f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, 0, 64, 0, 1.f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, -5, 64, 0, 1.f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, 1, 64, 2, 1.f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, 1, 64, 0, inf, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, 1, 64, 0, nan, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, p, p, 65535, 65535, 2147483647, 128, 0, 1.f, FA_BF16),
              FA_ERR_INVALID);
    // forward: unsupported
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, 1 << 23, 128, 0, 1.f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, (1 << 23) - 64, 128, 0, 1.f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, (1 << 23) - 65, 128, 0, 1.f, FA_BF16), FA_OK);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, 1, 96, 0, 1.f, FA_BF16), FA_ERR_UNSUPPORTED);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, 1, 256, 0, 1.f, FA_BF16), FA_ERR_UNSUPPORTED);
    EXPECT_EQ(check_fwd(p, p, p, p, 1, 1, 1, 64, 0, 1.f, 7), FA_ERR_UNSUPPORTED);

    // decode workspace sizing: S * H * ceil(max_blocks / 32) * (d + 2) floats
    EXPECT_EQ(decode_workspace_bytes(64, 32, 128, 16, 512), 64ull * 32 * 16 * 130 * 4);
    EXPECT_EQ(decode_workspace_bytes(1, 1, 64, 16, 1), 1ull * 1 * 1 * 66 * 4);
    EXPECT_EQ(decode_workspace_bytes(1, 1, 64, 16, 33), 2ull * 66 * 4);
    EXPECT_EQ(decode_workspace_bytes(0, 1, 64, 16, 1), 0);
    EXPECT_EQ(decode_workspace_bytes(1, 1, 64, 16, 0), 0);

    const size_t ws = decode_workspace_bytes(64, 32, 128, 16, 512);
    // decode: valid
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 64, 32, 128, 16, 512, 17874, 0.088f, FA_BF16, p, ws),
              FA_OK);
    // decode: invalid
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 64, 32, 128, 16, 512, 17874, 0.088f, FA_BF16, p,
                           ws - 1), FA_ERR_INVALID);
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 64, 32, 128, 16, 512, 17874, 0.088f, FA_BF16,
                           nullptr, ws), FA_ERR_INVALID);
    EXPECT_EQ(check_decode(p, p, p, nullptr, p, p, 64, 32, 128, 16, 512, 17874, 0.1f, FA_BF16,
                           p, ws), FA_ERR_INVALID);
    EXPECT_EQ(check_decode(p, p, p, p, nullptr, p, 64, 32, 128, 16, 512, 17874, 0.1f, FA_BF16,
                           p, ws), FA_ERR_INVALID);
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 64, 32, 128, 16, 512, 0, 0.1f, FA_BF16, p, ws),
              FA_ERR_INVALID);
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 64, 32, 128, 16, 512, 17874, inf, FA_BF16, p, ws),
              FA_ERR_INVALID);
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 0, 32, 128, 16, 512, 17874, 0.1f, FA_BF16, p, ws),
              FA_ERR_INVALID);
    // decode grid: x = S * H (sequence, head) pairs, y = ceil(max_blocks / 32) chunks
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 1, 65535, 64, 16, 65535 * 32, 17874, 0.1f, FA_BF16,
                           p, SIZE_MAX), FA_OK);                       // 65535 chunks
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 1, 65535, 64, 16, 65535 * 32 + 1, 17874, 0.1f,
                           FA_BF16, p, SIZE_MAX), FA_ERR_INVALID);     // 65536 chunks
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 65535, 32768, 64, 16, 1, 17874, 0.1f, FA_BF16, p,
                           SIZE_MAX), FA_OK);                          // 2147450880 pairs
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 65535, 32769, 64, 16, 1, 17874, 0.1f, FA_BF16, p,
                           SIZE_MAX), FA_ERR_INVALID);                 // 2147516415 pairs
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 1, 65536, 64, 16, 512, 17874, 0.1f, FA_BF16, p,
                           SIZE_MAX), FA_ERR_INVALID);
    // decode: unsupported
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 64, 32, 128, 8, 512, 17874, 0.1f, FA_BF16, p, ws),
              FA_ERR_UNSUPPORTED);
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 64, 32, 96, 16, 512, 17874, 0.1f, FA_BF16, p, ws),
              FA_ERR_UNSUPPORTED);
    EXPECT_EQ(check_decode(p, p, p, p, p, p, 64, 32, 128, 16, 512, 17874, 0.1f, FA_F32, p, ws),
              FA_ERR_UNSUPPORTED);

    // backward workspace: 256 bytes per 32 rows of every head
    EXPECT_EQ(bwd_workspace_bytes(8, 16, 2048, 128), 8ull * 16 * 64 * 256);
    EXPECT_EQ(bwd_workspace_bytes(1, 1, 65, 64), 3ull * 256);
    EXPECT_EQ(bwd_workspace_bytes(1, 1, 0, 64), 0);
    const size_t bws = bwd_workspace_bytes(8, 16, 2048, 128);
    // backward: valid
    EXPECT_EQ(check_bwd(p, p, p, p, p, p, p, p, p, 8, 16, 2048, 128, 1, 0.088f, FA_BF16, p, bws),
              FA_OK);
    EXPECT_EQ(check_bwd(p, p, p, p, p, p, p, p, p, 1, 1, 1, 64, 0, -0.5f, FA_BF16, p, 1024),
              FA_OK);
    // backward: invalid
    EXPECT_EQ(check_bwd(p, p, p, p, nullptr, p, p, p, p, 1, 1, 1, 64, 0, 1.f, FA_BF16, p, 1024),
              FA_ERR_INVALID);
    EXPECT_EQ(check_bwd(p, p, p, p, p, nullptr, p, p, p, 1, 1, 1, 64, 0, 1.f, FA_BF16, p, 1024),
              FA_ERR_INVALID);
    EXPECT_EQ(check_bwd(p, p, p, p, p, p, p, p, nullptr, 1, 1, 1, 64, 0, 1.f, FA_BF16, p, 1024),
              FA_ERR_INVALID);
    EXPECT_EQ(check_bwd(nullptr, p, p, p, p, p, p, p, p, 1, 1, 1, 64, 0, 1.f, FA_BF16, p, 1024),
              FA_ERR_INVALID);
    EXPECT_EQ(check_bwd(p, p, p, p, p, p, p, p, p, 8, 16, 2048, 128, 1, 0.088f, FA_BF16, p,
                        bws - 1), FA_ERR_INVALID);
    EXPECT_EQ(check_bwd(p, p, p, p, p, p, p, p, p, 1, 1, 1, 64, 0, 1.f, FA_BF16, nullptr, 1024),
              FA_ERR_INVALID);
    EXPECT_EQ(check_bwd(p, p, p, p, p, p, p, p, p, 1, 1, 1, 64, 0, nan, FA_BF16, p, 1024),
              FA_ERR_INVALID);
    // backward: unsupported
    EXPECT_EQ(check_bwd(p, p, p, p, p, p, p, p, p, 1, 1, 1, 64, 0, 1.f, FA_F32, p, 1024),
              FA_ERR_UNSUPPORTED);
    EXPECT_EQ(check_bwd(p, p, p, p, p, p, p, p, p, 1, 1, 1, 96, 0, 1.f, FA_BF16, p, 1024),
              FA_ERR_UNSUPPORTED);

    // prefill: valid
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 16, 32, 128, 16, 319, 3262, 15516, 1651, 1,
                            0.088f, FA_BF16), FA_OK);
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 1, 1, 64, 16, 1, 1, 1, 1, 0, -1.f, FA_BF16),
              FA_OK);
    // prefill: invalid
    EXPECT_EQ(check_prefill(p, p, p, p, p, nullptr, p, 1, 1, 64, 16, 1, 1, 1, 1, 0, 1.f, FA_BF16),
              FA_ERR_INVALID);
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 1, 1, 64, 16, 1, 1, 0, 1, 0, 1.f, FA_BF16),
              FA_ERR_INVALID);
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 1, 1, 64, 16, 1, 1, 1, 0, 0, 1.f, FA_BF16),
              FA_ERR_INVALID);
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 1, 1, 64, 16, 1, 1, 1, 1, 3, 1.f, FA_BF16),
              FA_ERR_INVALID);
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 65535, 65535, 64, 16, 1, 1, 1, 129, 0, 1.f,
                            FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 1, 1, 64, 16, 1, 1, 1, 1, 0, nan, FA_BF16),
              FA_ERR_INVALID);
    // prefill: the grid counts the (sequence, head) pairs padded to a multiple of 8
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 2147483640, 1, 64, 16, 1, 1, 1, 1, 0, 1.f,
                            FA_BF16), FA_OK);
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 2147483641, 1, 64, 16, 1, 1, 1, 1, 0, 1.f,
                            FA_BF16), FA_ERR_INVALID);
    // prefill: unsupported
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 1, 1, 96, 16, 1, 1, 1, 1, 0, 1.f, FA_BF16),
              FA_ERR_UNSUPPORTED);
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 1, 1, 64, 32, 1, 1, 1, 1, 0, 1.f, FA_BF16),
              FA_ERR_UNSUPPORTED);
    EXPECT_EQ(check_prefill(p, p, p, p, p, p, p, 1, 1, 64, 16, 1, 1, 1, 1, 0, 1.f, FA_F32),
              FA_ERR_UNSUPPORTED);

    // tree: valid, then a missing parent array, then a tree too large
    EXPECT_EQ(check_tree(p, p, p, p, p, p, p, p, 64, 32, 128, 16, 520, 14707, 4096, 64, 0.088f,
                         FA_BF16), FA_OK);
    EXPECT_EQ(check_tree(p, p, p, p, p, p, nullptr, p, 64, 32, 128, 16, 520, 14707, 4096, 64,
                         0.088f, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_tree(p, p, p, p, p, p, p, p, 64, 32, 128, 16, 520, 14707, 4096, 65, 0.088f,
                         FA_BF16), FA_ERR_UNSUPPORTED);

    // rope
    EXPECT_EQ(check_rope(p, p, p, p, 8, 16, 2048, 128, FA_BF16), FA_OK);
    EXPECT_EQ(check_rope(p, p, nullptr, p, 8, 16, 2048, 128, FA_BF16), FA_ERR_INVALID);
    EXPECT_EQ(check_rope(p, p, p, p, 8, 16, 2048, 96, FA_BF16), FA_ERR_UNSUPPORTED);
    EXPECT_EQ(fwd_rope_workspace_bytes(8, 16, 2048, 128), 8ull * 16 * 2048 * 128 * 2);
    EXPECT_EQ(check_fwd_rope(p, p, p, p, p, p, 8, 16, 2048, 128, 1, 0.088f, FA_BF16, p,
                             fwd_rope_workspace_bytes(8, 16, 2048, 128)), FA_OK);
    EXPECT_EQ(check_fwd_rope(p, p, p, p, p, p, 8, 16, 2048, 128, 1, 0.088f, FA_BF16, p, 100),
              FA_ERR_INVALID);
    EXPECT_EQ(check_fwd_rope(p, p, p, p, nullptr, p, 8, 16, 2048, 128, 1, 0.088f, FA_BF16, p,
                             fwd_rope_workspace_bytes(8, 16, 2048, 128)), FA_ERR_INVALID);

    EXPECT_EQ(std::string_view(status_string(FA_OK)).size() > 0, 1);
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("all host validation checks passed\n");
    return 0;
}
