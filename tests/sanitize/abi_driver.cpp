// Drives every entry point of the C ABI (include/attn.h) through its host
// code with valid, invalid and extreme arguments, under ASan and UBSan. The
// tensor pointers are device-address stand-ins that the host code only
// compares and aligns, never dereferences (the launchers are host stand-ins).
// Exit status 0 when every call returned the expected status.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attn.h"

namespace attn {
extern int g_launches;
}

static int fails = 0;
#define EXPECT(call, want)                                                                                 \
    do {                                                                                                   \
        const int got_ = (call);                                                                           \
        if (got_ != (want)) {                                                                              \
            std::fprintf(stderr, "line %d: %s -> %d (%s), expected %d\n", __LINE__, #call, got_,         \
                         attn_last_error(), (int)(want));                                                  \
            ++fails;                                                                                       \
        }                                                                                                  \
    } while (0)

static void* P(unsigned long long off) { return reinterpret_cast<void*>(0x7f0000000000ull + off); }
static const int32_t* I(unsigned long long off) { return static_cast<const int32_t*>(P(off)); }
static const uint8_t* U(unsigned long long off) { return static_cast<const uint8_t*>(P(off)); }
static float* F(unsigned long long off) { return static_cast<float*>(P(off)); }

int main() {
    const unsigned long long G = 1ull << 36;   // spacing between stand-in tensors
    // attn_fwd
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(3 * G), 1, 2, 64, 64, 128, 1, ATTN_BF16), ATTN_OK);
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(3 * G), 2, 3, 65, 200, 64, 1, ATTN_F16), ATTN_OK);
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(3 * G), 1, 2, 64, 64, 32, 0, ATTN_F32), ATTN_OK);
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(3 * G), 1, 2, 64, 64, 96, 1, ATTN_BF16), ATTN_ERR_UNSUPPORTED);
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(3 * G), 1, 2, 64, 64, 128, 2, ATTN_BF16), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(3 * G), 1, 2, 65, 64, 128, 1, ATTN_BF16), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(8), 1, 2, 64, 64, 128, 1, ATTN_BF16), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(0), 1, 2, 64, 64, 128, 1, ATTN_BF16), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(3 * G), -1, 2, 64, 64, 128, 1, ATTN_BF16), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(3 * G), 1, 2, 64, 64, 128, 1, 7), ATTN_ERR_UNSUPPORTED);
    EXPECT(attn_fwd(nullptr, P(G), P(2 * G), P(3 * G), 1, 2, 64, 64, 128, 1, ATTN_BF16), ATTN_ERR_INVALID_ARG);
    // extreme sizes: every product must be checked before it is formed
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(3 * G), INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128, 1, ATTN_BF16),
           ATTN_ERR_INVALID_ARG);
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(3 * G), 1, INT_MAX, 1 << 20, 1 << 20, 128, 0, ATTN_BF16),
           attn_fwd(P(0), P(G), P(2 * G), P(3 * G), 1, INT_MAX, 1 << 20, 1 << 20, 128, 0, ATTN_BF16));
    EXPECT(attn_fwd(P(0), P(G), P(2 * G), P(3 * G), 0, 2, 64, 64, 128, 1, ATTN_BF16), ATTN_OK);   // empty call
    // attn_fwd_kvcache and attn_fwd_mask
    EXPECT(attn_fwd_kvcache(P(0), P(G), P(2 * G), I(3 * G), P(4 * G), F(5 * G), 8, 32, 512, 4096, 128, 1,
                            ATTN_BF16), ATTN_OK);
    EXPECT(attn_fwd_kvcache(P(0), P(G), P(2 * G), nullptr, P(4 * G), nullptr, 1, 2, 64, 64, 128, 1, ATTN_BF16),
           ATTN_OK);
    EXPECT(attn_fwd_kvcache(P(0), P(G), P(2 * G), I(3 * G + 2), P(4 * G), nullptr, 1, 2, 64, 64, 128, 1,
                            ATTN_BF16), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_fwd_kvcache(P(0), P(G), P(2 * G), I(3 * G), P(4 * G), F(4 * G), 1, 2, 64, 64, 128, 1, ATTN_BF16),
           ATTN_ERR_INVALID_ARG);
    EXPECT(attn_fwd_mask(P(0), P(G), P(2 * G), U(3 * G), P(4 * G), F(5 * G), 2, 4, 100, 300, 64, 0, ATTN_F16),
           ATTN_OK);
    EXPECT(attn_fwd_mask(P(0), P(G), P(2 * G), U(3 * G), P(4 * G), nullptr, INT_MAX, 4, 100, 300, 64, 0,
                         ATTN_F16), ATTN_ERR_INVALID_ARG);
    // decode
    const size_t wsb = attn_decode_workspace_bytes(16, 32, 4096, 128);
    if (wsb != (size_t)(256 + 15) * 32 * (132 * 4 + 8)) {
        std::fprintf(stderr, "workspace bytes %zu\n", wsb);
        ++fails;
    }
    EXPECT(attn_decode_workspace_bytes(INT_MAX, INT_MAX, 1, 128) == 0, 1);   // beyond the planner's limits
    EXPECT(attn_decode_workspace_bytes(16, 32, 4096, 7) == 0, 1);            // no such head dim
    EXPECT(attn_decode(P(0), P(G), P(2 * G), I(3 * G), P(4 * G), 16, 32, 4096, 128, ATTN_BF16, P(5 * G), wsb),
           ATTN_OK);
    EXPECT(attn_decode(P(0), P(G), P(2 * G), I(3 * G), P(4 * G), 16, 32, 4096, 128, ATTN_BF16, P(5 * G), wsb - 1),
           ATTN_ERR_WORKSPACE);
    EXPECT(attn_decode(P(0), P(G), P(2 * G), I(3 * G), P(4 * G), 16, 32, 4096, 128, ATTN_BF16, nullptr, wsb),
           ATTN_ERR_WORKSPACE);
    EXPECT(attn_decode(P(0), P(G), P(2 * G), I(3 * G), P(4 * G), INT_MAX, 32, INT_MAX, 128, ATTN_BF16, P(5 * G),
                       wsb), ATTN_ERR_UNSUPPORTED);
    EXPECT(attn_decode(P(0), P(G), P(2 * G), I(3 * G), P(4 * G), 1 << 16, 1 << 16, 16, 128, ATTN_BF16, P(5 * G),
                       wsb), attn_decode(P(0), P(G), P(2 * G), I(3 * G), P(4 * G), 1 << 16, 1 << 16, 16, 128,
                                         ATTN_BF16, P(5 * G), wsb));
    EXPECT(attn_decode(P(0), P(G), P(2 * G), I(3 * G), P(0), 16, 32, 4096, 128, ATTN_BF16, P(5 * G), wsb),
           ATTN_ERR_INVALID_ARG);
    EXPECT(attn_decode(P(0), P(G), P(2 * G), I(3 * G), P(4 * G), 0, 32, 4096, 128, ATTN_BF16, nullptr, 0), ATTN_OK);
    EXPECT(attn_decode_noalloc(P(0), P(G), P(2 * G), I(3 * G), P(4 * G), 16, 32, 4096, 128, ATTN_BF16), ATTN_OK);
    EXPECT(attn_decode_noalloc(P(0), P(G), P(2 * G), I(3 * G), P(4 * G), 1000, 64, 16, 128, ATTN_BF16),
           ATTN_ERR_WORKSPACE);
    // Q/K/V projection, position table, masked softmax
    EXPECT(attn_qkv_proj(P(0), P(G), P(2 * G), P(3 * G), P(4 * G), 2048, 4096, 32, 128, ATTN_BF16), ATTN_OK);
    EXPECT(attn_qkv_proj(P(0), P(G), P(2 * G), P(3 * G), P(4 * G), 100, 3 << 20, 2, 64, ATTN_BF16),
           ATTN_ERR_UNSUPPORTED);
    EXPECT(attn_qkv_proj(P(0), P(G), P(2 * G), P(3 * G), P(4 * G), INT_MAX, INT_MAX - 31, INT_MAX, 128, ATTN_BF16),
           attn_qkv_proj(P(0), P(G), P(2 * G), P(3 * G), P(4 * G), INT_MAX, INT_MAX - 31, INT_MAX, 128, ATTN_BF16));
    EXPECT(attn_sinusoidal_pe(F(0), 4096, 4096, 0), ATTN_OK);
    EXPECT(attn_sinusoidal_pe(F(0), 4096, 4095, 0), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_sinusoidal_pe(F(0), INT_MAX, INT_MAX - 1, INT_MAX), attn_sinusoidal_pe(F(0), INT_MAX, INT_MAX - 1,
                                                                                           INT_MAX));
    EXPECT(attn_masked_softmax(P(0), P(G), 1, 32, 2048, 2048, 0.088f, 1, ATTN_BF16), ATTN_OK);
    EXPECT(attn_masked_softmax(P(0), P(0), 1, 32, 2048, 2048, 0.088f, 1, ATTN_BF16), ATTN_OK);   // in place
    EXPECT(attn_masked_softmax(P(0), P(G), INT_MAX, INT_MAX, INT_MAX, INT_MAX, 1.f, 0, ATTN_F32),
           attn_masked_softmax(P(0), P(G), INT_MAX, INT_MAX, INT_MAX, INT_MAX, 1.f, 0, ATTN_F32));
    // plans and plumbing
    attn_fwd_plan_t fp;
    EXPECT(attn_fwd_plan(1, 32, 2048, 2048, 128, 1, ATTN_BF16, &fp), ATTN_OK);
    EXPECT(attn_fwd_plan(INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128, 1, ATTN_BF16, &fp), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_fwd_plan(1, 32, 2048, 2048, 128, 1, ATTN_BF16, nullptr), ATTN_ERR_INVALID_ARG);
    attn_decode_plan_t dp;
    EXPECT(attn_decode_plan(16, 32, 4096, 128, ATTN_BF16, &dp), ATTN_OK);
    EXPECT(attn_decode_plan(INT_MAX, INT_MAX, INT_MAX, 128, ATTN_BF16, &dp), attn_decode_plan(INT_MAX, INT_MAX,
                                                                                              INT_MAX, 128,
                                                                                              ATTN_BF16, &dp));
    EXPECT(attn_set_stream(nullptr), ATTN_OK);
    EXPECT(attn_set_timing_events(nullptr, nullptr), ATTN_OK);
    EXPECT(attn_set_clock_probe(P(4)), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_set_clock_probe(nullptr), ATTN_OK);
    for (int s = -3; s < 10; ++s)
        if (!attn_status_string(s) || std::strlen(attn_status_string(s)) == 0) ++fails;
    for (int x = 0; x < 4096; x += 37) {
        const int y = attn_xcd_remap(x, 4096);
        if (y < 0 || y >= 4096) ++fails;
    }
    if (attn::g_launches == 0) ++fails;   // the valid calls reached their launchers
    std::printf("abi driver: %d launches, %d failures\n", attn::g_launches, fails);
    return fails != 0;
}
