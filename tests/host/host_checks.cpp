// Every argument check of the C ABI and the propagation of HIP runtime
// errors, driven against a faked runtime (no GPU). Built with the address
// and undefined-behaviour sanitizers by tests/test_host_hardening.py; prints
// one line per failed check and "host checks passed" when all hold.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include <hip/hip_runtime_api.h>

#include "sparse_ffn.h"

extern hipError_t g_fake_runtime_status;
extern hipError_t g_fake_launch_status;
extern int g_fake_launches;

static int g_failed = 0;

static void expect(bool ok, const char* what, int line) {
    if (!ok) {
        std::printf("FAILED line %d: %s (last error: \"%s\")\n", line, what, sparse_ffn_last_error());
        ++g_failed;
    }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)
#define EXPECT_STATUS(call, st) expect((call) == (st), #call " == " #st, __LINE__)

// distinct, suitably aligned fake device addresses (never dereferenced)
static void* dev(uintptr_t k) { return reinterpret_cast<void*>((uintptr_t)0x10000000u + k * 0x100000u); }

static sffn_config_t full_cfg() {
    sffn_config_t c{};
    c.d = 4096; c.d_i = 14336; c.rank = 448; c.bank = 64; c.keep = 16;
    c.dtype = SFFN_BF16; c.gate = SFFN_GATE_PREDICTOR; c.flags = 0;
    return c;
}

static bool has_text(const char* s) { return s && std::strlen(s) > 0; }

int main() {
    // ---- configs ---------------------------------------------------------
    sffn_config_t c = full_cfg();
    EXPECT(sparse_ffn_packed_size(&c) > 0);
    EXPECT(sparse_ffn_packed_size(nullptr) == 0);
    const struct { const char* name; void (*bad)(sffn_config_t&); } bad_cfgs[] = {
        {"d <= 0", [](sffn_config_t& x) { x.d = 0; }},
        {"d_i <= 0", [](sffn_config_t& x) { x.d_i = -64; }},
        {"rank <= 0", [](sffn_config_t& x) { x.rank = 0; }},
        {"bank != 64", [](sffn_config_t& x) { x.bank = 32; }},
        {"keep 0", [](sffn_config_t& x) { x.keep = 0; }},
        {"keep 65", [](sffn_config_t& x) { x.keep = 65; }},
        {"d_i % 64", [](sffn_config_t& x) { x.d_i = 1000; }},
        {"d_i too large", [](sffn_config_t& x) { x.d_i = 65536 + 64; }},
        {"d % 64", [](sffn_config_t& x) { x.d = 100; }},
        {"rank % 32", [](sffn_config_t& x) { x.rank = 40; }},
        {"dtype", [](sffn_config_t& x) { x.dtype = (sffn_dtype_t)7; }},
        {"gate", [](sffn_config_t& x) { x.gate = (sffn_gate_t)9; }},
        {"flags", [](sffn_config_t& x) { x.flags = 6; }},
        {"INT_MIN d", [](sffn_config_t& x) { x.d = INT32_MIN; }},
        {"INT_MAX d_i", [](sffn_config_t& x) { x.d_i = INT32_MAX; }},
    };
    for (const auto& b : bad_cfgs) {
        sffn_config_t x = full_cfg();
        b.bad(x);
        if (sparse_ffn_packed_size(&x) != 0) {
            std::printf("FAILED: packed size accepted bad config (%s)\n", b.name);
            ++g_failed;
        }
        sffn_handle_t h = nullptr;
        const sffn_status_t st = sparse_ffn_create(&x, dev(1), dev(2), dev(3), dev(4), dev(5), nullptr, dev(6),
                                                   (size_t)1 << 40, nullptr, &h);
        if (st == SFFN_OK || h != nullptr || !has_text(sparse_ffn_last_error())) {
            std::printf("FAILED: create accepted bad config (%s)\n", b.name);
            ++g_failed;
        }
    }

    // ---- create ------------------------------------------------------------
    const size_t need = sparse_ffn_packed_size(&c);
    sffn_handle_t h = nullptr;
    EXPECT_STATUS(sparse_ffn_create(&c, nullptr, dev(2), dev(3), dev(4), dev(5), nullptr, dev(6), need, nullptr, &h),
                  SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_create(&c, dev(1), dev(2), dev(3), dev(4), dev(5), nullptr, dev(6), need, nullptr, nullptr),
                  SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_create(&c, (char*)dev(1) + 8, dev(2), dev(3), dev(4), dev(5), nullptr, dev(6), need,
                                    nullptr, &h),
                  SFFN_ERR_INVALID_ARG);
    EXPECT(std::strstr(sparse_ffn_last_error(), "aligned") != nullptr);
    EXPECT_STATUS(sparse_ffn_create(&c, dev(1), dev(2), dev(3), dev(4), dev(5), (const float*)((char*)dev(7) + 4),
                                    dev(6), need, nullptr, &h),
                  SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_create(&c, dev(1), dev(2), dev(3), dev(4), dev(5), nullptr, dev(6), need - 1, nullptr, &h),
                  SFFN_ERR_WORKSPACE);
    EXPECT(h == nullptr);
    // the runtime fails while packing: SFFN_ERR_HIP, no handle
    g_fake_runtime_status = hipErrorOutOfMemory;
    EXPECT_STATUS(sparse_ffn_create(&c, dev(1), dev(2), dev(3), dev(4), dev(5), nullptr, dev(6), need, nullptr, &h),
                  SFFN_ERR_HIP);
    EXPECT(h == nullptr);
    EXPECT(std::strstr(sparse_ffn_last_error(), "sparse_ffn_create") != nullptr);
    EXPECT(std::strstr(sparse_ffn_last_error(), "injected") != nullptr);
    g_fake_runtime_status = hipSuccess;
    g_fake_launch_status = hipErrorLaunchFailure;      // the transpose kernel fails to launch
    EXPECT_STATUS(sparse_ffn_create(&c, dev(1), dev(2), dev(3), dev(4), dev(5), nullptr, dev(6), need, nullptr, &h),
                  SFFN_ERR_HIP);
    EXPECT(h == nullptr);
    g_fake_launch_status = hipSuccess;
    EXPECT_STATUS(sparse_ffn_create(&c, dev(1), dev(2), dev(3), dev(4), dev(5), nullptr, dev(6), need, nullptr, &h),
                  SFFN_OK);
    EXPECT(h != nullptr);
    EXPECT(std::strlen(sparse_ffn_last_error()) == 0);

    // ---- forward -----------------------------------------------------------
    const size_t ws1 = sparse_ffn_workspace_size(h, 1);
    EXPECT(ws1 > 0);
    EXPECT(sparse_ffn_workspace_size(h, 0) == 0);
    EXPECT(sparse_ffn_workspace_size(h, -3) == 0);
    EXPECT(sparse_ffn_workspace_size(nullptr, 4) == 0);
    void* x = dev(10); void* y = dev(11); void* ws = dev(12);
    uint64_t* mask = (uint64_t*)dev(13); float* logits = (float*)dev(14);
    EXPECT_STATUS(sparse_ffn_forward(nullptr, x, 1, y, nullptr, nullptr, ws, ws1, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_forward(h, x, -1, y, nullptr, nullptr, ws, ws1, nullptr), SFFN_ERR_INVALID_ARG);
    const int before = g_fake_launches;
    EXPECT_STATUS(sparse_ffn_forward(h, nullptr, 0, nullptr, nullptr, nullptr, nullptr, 0, nullptr), SFFN_OK);
    EXPECT(g_fake_launches == before);                 // T = 0 enqueues nothing
    EXPECT_STATUS(sparse_ffn_forward(h, nullptr, 1, y, nullptr, nullptr, ws, ws1, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_forward(h, x, 1, nullptr, nullptr, nullptr, ws, ws1, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_forward(h, (char*)x + 2, 1, y, nullptr, nullptr, ws, ws1, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_forward(h, x, 1, (char*)y + 4, nullptr, nullptr, ws, ws1, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_forward(h, x, 1, y, (uint64_t*)((char*)mask + 8), nullptr, ws, ws1, nullptr),
                  SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_forward(h, x, 1, y, nullptr, (float*)((char*)logits + 4), ws, ws1, nullptr),
                  SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_forward(h, x, 1, y, nullptr, nullptr, nullptr, ws1, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_forward(h, x, 1, y, nullptr, nullptr, (char*)ws + 16, ws1, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_forward(h, x, 1, y, nullptr, nullptr, ws, ws1 - 1, nullptr), SFFN_ERR_WORKSPACE);
    // token counts whose sizes would overflow are refused before any arithmetic on them
    for (int64_t T : {(int64_t)1 << 31, (int64_t)1 << 40, (int64_t)1 << 62, INT64_MAX}) {
        EXPECT_STATUS(sparse_ffn_forward(h, x, T, y, nullptr, nullptr, ws, (size_t)-1, nullptr), SFFN_ERR_UNSUPPORTED);
        EXPECT_STATUS(sparse_ffn_forward_noalloc(h, x, T, y, nullptr, nullptr, nullptr), SFFN_ERR_UNSUPPORTED);
        EXPECT(sparse_ffn_workspace_size(h, T) == 0);
    }
    for (int64_t T : {1, 3, 4, 5, 32, 64, 65, 256, 300, 4096}) {
        const size_t need_T = sparse_ffn_workspace_size(h, T);
        EXPECT(need_T > 0);
        EXPECT_STATUS(sparse_ffn_forward(h, x, T, y, mask, logits, ws, need_T, nullptr), SFFN_OK);
    }
    // a kernel launch that fails surfaces as SFFN_ERR_HIP with the detail
    g_fake_launch_status = hipErrorLaunchFailure;
    for (int64_t T : {1, 32, 300}) {
        EXPECT_STATUS(sparse_ffn_forward(h, x, T, y, nullptr, nullptr, ws, sparse_ffn_workspace_size(h, T), nullptr),
                      SFFN_ERR_HIP);
        EXPECT(std::strstr(sparse_ffn_last_error(), "sparse_ffn_forward") != nullptr);
        EXPECT(std::strstr(sparse_ffn_last_error(), "injected HIP error") != nullptr);
    }
    g_fake_launch_status = hipSuccess;

    // ---- forward without allocation ------------------------------------------
    EXPECT_STATUS(sparse_ffn_forward_noalloc(nullptr, x, 1, y, nullptr, nullptr, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_forward_noalloc(h, x, -2, y, nullptr, nullptr, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_forward_noalloc(h, x, 0, y, nullptr, nullptr, nullptr), SFFN_OK);
    EXPECT_STATUS(sparse_ffn_forward_noalloc(h, x, 4096, y, nullptr, nullptr, nullptr), SFFN_ERR_WORKSPACE);
    EXPECT(std::strstr(sparse_ffn_last_error(), "scratch") != nullptr);
    g_fake_runtime_status = hipErrorInvalidSymbol;     // the scratch address cannot be looked up
    EXPECT_STATUS(sparse_ffn_forward_noalloc(h, x, 1, y, nullptr, nullptr, nullptr), SFFN_ERR_HIP);
    EXPECT(std::strstr(sparse_ffn_last_error(), "hip") != nullptr);
    g_fake_runtime_status = hipSuccess;
    EXPECT_STATUS(sparse_ffn_forward_noalloc(h, x, 1, y, mask, nullptr, nullptr), SFFN_OK);
    EXPECT_STATUS(sparse_ffn_forward_noalloc(h, x, 64, y, mask, logits, nullptr), SFFN_OK);
    EXPECT_STATUS(sparse_ffn_forward_noalloc(h, (char*)x + 2, 1, y, nullptr, nullptr, nullptr), SFFN_ERR_INVALID_ARG);

    // ---- bank_topk -------------------------------------------------------------
    const float* lg = (const float*)dev(20);
    EXPECT_STATUS(bank_topk(lg, -1, 1024, 16, mask, nullptr, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(bank_topk(lg, 4, 0, 16, mask, nullptr, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(bank_topk(lg, 4, 1000, 16, mask, nullptr, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(bank_topk(lg, 4, 65600, 16, mask, nullptr, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(bank_topk(lg, 4, 1024, 0, mask, nullptr, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(bank_topk(lg, 4, 1024, 65, mask, nullptr, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(bank_topk(nullptr, 4, 1024, 16, mask, nullptr, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(bank_topk(lg, 4, 1024, 16, nullptr, nullptr, nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(bank_topk(lg, 4, 1024, 16, mask, (uint16_t*)((char*)dev(21) + 2), nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(bank_topk(nullptr, 0, 1024, 16, nullptr, nullptr, nullptr), SFFN_OK);
    for (int64_t T : {(int64_t)1 << 40, (int64_t)1 << 62, INT64_MAX})
        EXPECT_STATUS(bank_topk(lg, T, 1024, 16, mask, nullptr, nullptr), SFFN_ERR_UNSUPPORTED);
    EXPECT_STATUS(bank_topk(lg, 4, 1024, 16, mask, nullptr, nullptr), SFFN_OK);
    g_fake_launch_status = hipErrorLaunchFailure;
    EXPECT_STATUS(bank_topk(lg, 4, 1024, 16, mask, nullptr, nullptr), SFFN_ERR_HIP);
    EXPECT(std::strstr(sparse_ffn_last_error(), "bank_topk") != nullptr);
    g_fake_launch_status = hipSuccess;

    // ---- backward ----------------------------------------------------------------
    float* g[7];
    for (int i = 0; i < 7; ++i) g[i] = (float*)dev(30 + i);
    const size_t bws = sparse_ffn_backward_workspace_size(h, 64);
    EXPECT(bws > 0);
    EXPECT(sparse_ffn_backward_workspace_size(h, 0) == 0);
    EXPECT_STATUS(sparse_ffn_backward(nullptr, x, x, mask, 64, 1.f, g[0], g[1], g[2], g[3], g[4], g[5], g[6], ws, bws,
                                      nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_backward(h, x, x, mask, -1, 1.f, g[0], g[1], g[2], g[3], g[4], g[5], g[6], ws, bws, nullptr),
                  SFFN_ERR_INVALID_ARG);
    for (float tau : {0.f, -1.f, NAN})
        EXPECT_STATUS(sparse_ffn_backward(h, x, x, mask, 64, tau, g[0], g[1], g[2], g[3], g[4], g[5], g[6], ws, bws,
                                          nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_backward(h, x, x, mask, 64, 1.f, g[0], nullptr, g[2], g[3], g[4], g[5], g[6], ws, bws,
                                      nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_backward(h, x, x, nullptr, 64, 1.f, g[0], g[1], g[2], g[3], g[4], g[5], g[6], ws, bws,
                                      nullptr), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_backward(h, x, x, mask, 64, 1.f, g[0], g[1], g[2], g[3], g[4], g[5], g[6], ws, bws - 1,
                                      nullptr), SFFN_ERR_WORKSPACE);
    for (int64_t T : {(int64_t)1 << 40, (int64_t)1 << 62, INT64_MAX})
        EXPECT_STATUS(sparse_ffn_backward(h, x, x, mask, T, 1.f, g[0], g[1], g[2], g[3], g[4], g[5], g[6], ws,
                                          (size_t)-1, nullptr), SFFN_ERR_UNSUPPORTED);
    EXPECT_STATUS(sparse_ffn_backward(h, x, x, mask, 64, INFINITY, g[0], g[1], g[2], g[3], g[4], g[5], g[6], ws, bws,
                                      nullptr), SFFN_OK);
    EXPECT_STATUS(sparse_ffn_backward(h, nullptr, nullptr, nullptr, 0, 1.f, nullptr, g[1], g[2], g[3], g[4], g[5], g[6],
                                      nullptr, 0, nullptr), SFFN_OK);
    g_fake_launch_status = hipErrorLaunchFailure;
    EXPECT_STATUS(sparse_ffn_backward(h, x, x, mask, 64, 1.f, g[0], g[1], g[2], g[3], g[4], g[5], g[6], ws, bws,
                                      nullptr), SFFN_ERR_HIP);
    EXPECT(std::strstr(sparse_ffn_last_error(), "sparse_ffn_backward") != nullptr);
    g_fake_launch_status = hipSuccess;

    // ---- profiling helpers, status strings ------------------------------------------
    void* evs[2 * SFFN_STAGES];
    for (int i = 0; i < 2 * SFFN_STAGES; ++i) evs[i] = dev(40 + i);
    EXPECT_STATUS(sparse_ffn_set_stage_events(nullptr, evs, 2 * SFFN_STAGES), SFFN_ERR_INVALID_ARG);
    EXPECT_STATUS(sparse_ffn_set_stage_events(h, evs, 2 * SFFN_STAGES - 1), SFFN_ERR_INVALID_ARG);
    evs[3] = nullptr;
    EXPECT_STATUS(sparse_ffn_set_stage_events(h, evs, 2 * SFFN_STAGES), SFFN_ERR_INVALID_ARG);
    evs[3] = dev(43);
    EXPECT_STATUS(sparse_ffn_set_stage_events(h, evs, 2 * SFFN_STAGES), SFFN_OK);
    EXPECT_STATUS(sparse_ffn_set_stage_events(h, nullptr, 0), SFFN_OK);
    for (int64_t T : {1, 32, 4096})
        for (int i = 0; i < SFFN_STAGES; ++i) EXPECT(has_text(sparse_ffn_stage_name(h, T, i)));
    EXPECT(sparse_ffn_stage_name(h, 1, -1) == nullptr);
    EXPECT(sparse_ffn_stage_name(h, 1, SFFN_STAGES) == nullptr);
    EXPECT(sparse_ffn_stage_name(nullptr, 1, 0) == nullptr);
    for (int s = 0; s <= 5; ++s) EXPECT(has_text(sparse_ffn_status_string((sffn_status_t)s)));
    EXPECT(has_text(sparse_ffn_status_string((sffn_status_t)-7)));
    sparse_ffn_destroy(h);
    sparse_ffn_destroy(nullptr);

    if (g_failed) {
        std::printf("%d host checks failed\n", g_failed);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
