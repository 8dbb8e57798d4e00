// Calls every entry point of include/fluxattn.h with valid arguments and with each
// class of invalid argument, against the host-only launcher stubs, so that a build
// with AddressSanitizer and UndefinedBehaviorSanitizer runs the ABI's validation,
// workspace sizing and dispatch code.  Device pointers are stand-in host
// addresses that the stubs never dereference; host route copies are real.  Exit
// status 0 means every call returned the documented status.  Test infrastructure.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fluxattn.h"

extern int g_launches;

static int failures = 0;

static void expect(int line, fa_status got, fa_status want)
{
    const char *msg = fa_last_error();
    const bool msg_ok = (got == FA_OK) ? msg[0] == '\0' : msg[0] != '\0';
    if (got != want || !msg_ok) {
        std::fprintf(stderr, "line %d: status %d, expected %d (message '%s')\n", line, (int)got,
                     (int)want, msg);
        ++failures;
    }
}
#define EXPECT(call, want) expect(__LINE__, (call), (want))

int main()
{
    static char dev[1 << 16];  // stand-in device memory: never dereferenced
    void *P = dev;
    const int32_t *CU = reinterpret_cast<const int32_t *>(dev);
    const uint8_t *RT = reinterpret_cast<const uint8_t *>(dev);
    std::vector<char> ws(1 << 20);
    const float sc = 0.088f;

    // ---- helpers
    if (fa_abi_version() <= 0) ++failures;
    const size_t rws = fa_router_workspace_size(2, 4096, 256);
    if (rws == 0 || fa_router_workspace_size(0, 4096, 256) != 0) ++failures;
    if (fa_decode_workspace_size(2, 32, 128, 1000) == 0 ||
        fa_decode_workspace_size(2, 32, 128, -1) != 0) ++failures;
    if (fa_xattn_workspace_size(1, 32, 16) == 0 || fa_xattn_workspace_size(1, 32, 4097) != 0)
        ++failures;

    // ---- router
    std::vector<char> rbuf(rws);
    EXPECT(fa_router_decide(P, FA_BF16, CU, 2, 4096, 64, (float *)P, (float *)P, 256, (float *)P,
                            (float *)P, 32, (uint8_t *)P, nullptr, rbuf.data(), rws, nullptr),
           FA_OK);
    EXPECT(fa_router_decide(nullptr, FA_BF16, CU, 2, 4096, 64, (float *)P, (float *)P, 256,
                            (float *)P, (float *)P, 32, (uint8_t *)P, nullptr, rbuf.data(), rws,
                            nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_router_decide(P, 7, CU, 2, 4096, 64, (float *)P, (float *)P, 256, (float *)P,
                            (float *)P, 32, (uint8_t *)P, nullptr, rbuf.data(), rws, nullptr),
           FA_ERR_UNSUPPORTED);
    EXPECT(fa_router_decide(P, FA_BF16, CU, 2, 4096, 64, (float *)P, (float *)P, 256, (float *)P,
                            (float *)P, 32, (uint8_t *)P, nullptr, rbuf.data(), rws - 1, nullptr),
           FA_ERR_WORKSPACE);
    EXPECT(fa_router_decide(P, FA_BF16, CU, 2, 4096, 0, (float *)P, (float *)P, 256, (float *)P,
                            (float *)P, 32, (uint8_t *)P, nullptr, rbuf.data(), rws, nullptr),
           FA_ERR_INVALID_ARG);

    // ---- block plan
    EXPECT(fa_block_plan(CU, 2, 16, RT, 4, 1, 128, 2048, 64, (int32_t *)P, nullptr), FA_OK);
    EXPECT(fa_block_plan(CU, 2, 16, RT, 4, 4, 128, 2048, 64, (int32_t *)P, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_block_plan(CU, 2, 16, RT, 4, 1, 100, 2048, 64, (int32_t *)P, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_block_plan(CU, 2, 16, RT, 4, 1, 128, 2048, 48, (int32_t *)P, nullptr),
           FA_ERR_INVALID_ARG);

    // ---- prefill (all kinds of host route copy)
    const uint8_t r_fa[2] = {1, 1}, r_sa[2] = {0, 0}, r_mix[2] = {1, 0};
    for (const uint8_t *rh : {(const uint8_t *)nullptr, r_fa, r_sa, r_mix})
        for (int dt : {FA_BF16, FA_F32})
            for (int d : {64, 128})
                EXPECT(fa_attn_prefill(P, P, P, P, (float *)P, dt, CU, 2, 1000, 32, 8, d, RT, rh,
                                       1, 0, 128, 2048, 64, sc, nullptr), FA_OK);
    EXPECT(fa_attn_prefill(P, P, P, P, nullptr, FA_BF16, CU, 2, 1000, 32, 6, 128, RT, nullptr, 1,
                           0, 128, 2048, 64, sc, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_attn_prefill(P, P, P, P, nullptr, FA_BF16, CU, 2, 1000, 32, 8, 96, RT, nullptr, 1,
                           0, 128, 2048, 64, sc, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_attn_prefill(P, P, P, P, nullptr, FA_BF16, CU, 2, 1000, 32, 8, 128, RT, nullptr, 1,
                           0, 128, 2048, 64, NAN, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_attn_prefill(P, P, P, P, nullptr, FA_BF16, CU, 0, 1000, 32, 8, 128, RT, nullptr, 1,
                           0, 128, 2048, 64, sc, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_attn_prefill(P, P, P, nullptr, nullptr, FA_BF16, CU, 2, 1000, 32, 8, 128, RT,
                           nullptr, 1, 0, 128, 2048, 64, sc, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_attn_prefill_kv(P, P, P, P, nullptr, FA_BF16, CU, CU, 2, 100, 32, 8, 128, RT, r_mix,
                              1, 0, 128, 2048, 64, sc, nullptr), FA_OK);
    EXPECT(fa_attn_prefill_kv(P, P, P, P, nullptr, FA_BF16, CU, nullptr, 2, 100, 32, 8, 128, RT,
                              r_mix, 1, 0, 128, 2048, 64, sc, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_attn_prefill_triangle(P, P, P, P, nullptr, FA_BF16, CU, 2, 1000, 32, 8, 128, RT,
                                    r_sa, 1, 0, 128, 2048, 64, 1024, sc, nullptr), FA_OK);
    EXPECT(fa_attn_prefill_triangle(P, P, P, P, nullptr, FA_BF16, CU, 2, 1000, 32, 8, 128, RT,
                                    r_sa, 1, 0, 128, 2048, 64, 100, sc, nullptr),
           FA_ERR_INVALID_ARG);

    // ---- XAttention
    const size_t xws = fa_xattn_workspace_size(2, 32, 9);
    EXPECT(fa_xattn_scores(P, P, FA_BF16, CU, 2, 1100, 32, 8, 128, 128, 8, sc, (float *)P, 9, P,
                           xws, nullptr), FA_OK);
    EXPECT(fa_xattn_scores(P, P, FA_BF16, CU, 2, 1200, 32, 8, 128, 128, 8, sc, (float *)P, 9, P,
                           xws, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_xattn_scores(P, P, FA_BF16, CU, 2, 1100, 32, 8, 128, 128, 8, sc, (float *)P, 9, P,
                           xws - 1, nullptr), FA_ERR_WORKSPACE);
    EXPECT(fa_xattn_scores(P, P, FA_BF16, CU, 2, 1100, 32, 8, 128, 64, 8, sc, (float *)P, 9, P,
                           xws, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_xattn_scores(P, P, FA_BF16, CU, 2, 1100, 24, 8, 128, 128, 8, sc, (float *)P, 9, P,
                           xws, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_xattn_select((float *)P, CU, 2, 32, 9, 128, 0.9f, (uint32_t *)P, nullptr), FA_OK);
    EXPECT(fa_xattn_select((float *)P, CU, 2, 32, 9, 128, -1.0f, (uint32_t *)P, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_attn_prefill_xattn(P, P, P, P, nullptr, FA_BF16, CU, 2, 1100, 32, 8, 128, 128,
                                 (const uint32_t *)P, 9, sc, nullptr), FA_OK);
    EXPECT(fa_attn_prefill_xattn(P, P, P, P, nullptr, FA_BF16, CU, 2, 1100, 32, 8, 128, 32,
                                 (const uint32_t *)P, 9, sc, nullptr), FA_ERR_INVALID_ARG);

    // ---- decode, ring decode and KV compaction
    const size_t dws = fa_decode_workspace_size(2, 32, 128, 5000);
    for (const uint8_t *rh : {(const uint8_t *)nullptr, r_fa, r_sa, r_mix})
        EXPECT(fa_attn_decode(P, P, (float *)P, P, P, P, P, 5000, CU, FA_BF16, 2, 32, 8, 128, RT,
                              rh, 1, 0, 128, 2048, 64, sc, ws.data(), dws, nullptr), FA_OK);
    EXPECT(fa_attn_decode(P, P, nullptr, P, nullptr, P, P, 5000, CU, FA_BF16, 2, 32, 8, 128, RT,
                          nullptr, 1, 0, 128, 2048, 64, sc, ws.data(), dws, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_attn_decode(P, P, nullptr, nullptr, nullptr, P, P, 5000, CU, FA_BF16, 2, 32, 8,
                          128, RT, nullptr, 1, 0, 128, 2048, 64, sc, ws.data(), 16, nullptr),
           FA_ERR_WORKSPACE);
    EXPECT(fa_attn_decode(P, P, nullptr, nullptr, nullptr, P, P, 5000, CU, FA_BF16, 2, 96, 8,
                          128, RT, nullptr, 1, 0, 128, 2048, 64, sc, ws.data(), dws, nullptr),
           FA_ERR_UNSUPPORTED);
    EXPECT(fa_attn_decode_noalloc(P, P, nullptr, P, P, P, P, 5000, CU, FA_BF16, 2, 32, 8, 128,
                                  RT, r_mix, 1, 0, 128, 2048, 64, sc, nullptr), FA_OK);
    EXPECT(fa_attn_decode_noalloc(P, P, nullptr, nullptr, nullptr, P, P, 1 << 20, CU, FA_BF16,
                                  512, 32, 8, 128, RT, nullptr, 1, 0, 128, 2048, 64, sc, nullptr),
           FA_ERR_WORKSPACE);
    EXPECT(fa_attn_decode_noalloc(P, P, nullptr, P, nullptr, P, P, 5000, CU, FA_BF16, 2, 32, 8,
                                  128, RT, nullptr, 1, 0, 128, 2048, 64, sc, nullptr),
           FA_ERR_INVALID_ARG);
    const size_t rws2 = fa_decode_workspace_size(2, 32, 128, 2176);
    EXPECT(fa_attn_decode_ring(P, P, nullptr, P, P, P, P, 2176, CU, FA_BF16, 2, 32, 8, 128, 128,
                               2048, 64, sc, ws.data(), rws2, nullptr), FA_OK);
    EXPECT(fa_attn_decode_ring(P, P, nullptr, P, P, P, P, 2000, CU, FA_BF16, 2, 32, 8, 128, 128,
                               2048, 64, sc, ws.data(), rws2, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_kv_compact(P, P, FA_BF16, CU, 2, 8, 128, 128, 2048, 64, P, P, 2176, nullptr), FA_OK);
    EXPECT(fa_kv_compact(P, P, FA_BF16, CU, 2, 8, 128, 128, 2048, 64, P, P, 2175, nullptr),
           FA_ERR_INVALID_ARG);

    if (g_launches == 0) ++failures;  // the valid calls reached the launchers
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("abi driver ok (%d launches)\n", g_launches);
    return 0;
}
