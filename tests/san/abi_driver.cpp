// Host-side checks of the C ABI's argument validation, built with
// AddressSanitizer and UndefinedBehaviorSanitizer against the real C-ABI
// layer (dqg_api.cpp) and stand-in launchers.  Every call below must be
// rejected with its documented code before any launch; pointers that are
// never dereferenced stand for device buffers.  Exit status 0 when every
// check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "../../include/dqg.h"

namespace dqg {
extern int g_stub_launches;
}

namespace {

int g_failed = 0, g_checks = 0;

void expect(bool ok, const char *what, int line) {
    ++g_checks;
    if (!ok) {
        ++g_failed;
        std::fprintf(stderr, "FAIL line %d: %s (last error: %s)\n", line, what, dqg_last_error());
    }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

void *fake(uintptr_t a) { return reinterpret_cast<void *>(a); }

dqg_matrix mat(int fmt = 4, int O = 64, int K = 256, int gs = 32, uintptr_t q = 0x10000, uintptr_t q2 = 0,
               uintptr_t s = 0x20000) {
    return dqg_matrix{fmt, O, K, gs, fake(q), fake(q2), static_cast<const float *>(fake(s))};
}

const float *const X = static_cast<const float *>(fake(0x30000));
float *const Y = static_cast<float *>(fake(0x40000));

void matrices() {
    struct Case {
        dqg_matrix m;
        int code;
    } cases[] = {
        {mat(3), -2},
        {mat(4, 64, 256, 48), -2},
        {mat(4, 64, 256, 16), -2},
        {mat(4, 64, 96, 64), -3},
        {mat(4, 64, 100), -3},
        {mat(1, 64, 512, 32), -2},
        {mat(1, 64, 520, 520), -3},
        {mat(5, 64, 256, 32), -2},
        {mat(5, 64, 96, 64), -3},
        {mat(7, 64, 256, 64), -2},
        {mat(4, 0), -3},
        {mat(4, 64, 256, 32, 0x10008), -1},
        {mat(4, 64, 256, 32, 0x10000, 0, 0x20002), -1},
        {mat(5, 64, 256, 64, 0x10000, 0), -1},
        {mat(10, 64, 256, 32, 0x10000, 0, 0), -2},
        {mat(11, 64, 256, 256), -1},
        {mat(14, 64, 100, 0, 0x10000, 0, 0), -3},
        {mat(10, 64, 6, 0, 0x10000, 0, 0), -3},
        {mat(12, 64, 256, 64), -2},
        {mat(12, 64, 192, 128), -3},
        {mat(12, 64, 256, 128, 0x10000, 0, 0), -1},
        {mat(13, 64, 256, 16), -2},
        {mat(13, 64, 256, 48), -2},
        {mat(13, 64, 96, 64), -3},
        {mat(13, 64, 256, 64, 0x10000, 0, 0), -1},
        {mat(9), -2},
        {mat(15), -2},
        {mat(4, -5), -3},
        {mat(4, 64, -256), -3},
    };
    for (const Case &c : cases) {
        const int rc = dqg_matmul(&c.m, X, 1, Y, nullptr);
        EXPECT(rc == c.code);
        EXPECT(std::strlen(dqg_last_error()) > 0);
        EXPECT(dqg_dequant(&c.m, Y, nullptr) == c.code);
    }
    EXPECT(dqg_matmul(nullptr, X, 1, Y, nullptr) == -1);
}

void vectors() {
    const dqg_matrix m = mat();
    EXPECT(dqg_matmul(&m, nullptr, 1, Y, nullptr) == -1);
    EXPECT(dqg_matmul(&m, X + 1, 1, Y, nullptr) == -1);
    EXPECT(dqg_matmul(&m, X, 0, Y, nullptr) == -1);
    EXPECT(dqg_matmul(&m, X, -3, Y, nullptr) == -1);
    EXPECT(dqg_matmul(&m, X, 1, nullptr, nullptr) == -1);
    EXPECT(dqg_dequant(&m, nullptr, nullptr) == -1);
    const dqg_matrix g = mat(), u = mat(4, 64, 512);
    EXPECT(dqg_gate_up(&g, &u, X, 1, Y, nullptr) == -3);
    const float bad_limits[] = {0.f, -1.f, std::numeric_limits<float>::quiet_NaN(),
                                -std::numeric_limits<float>::infinity()};
    for (float L : bad_limits) EXPECT(dqg_gate_up_clamped(&g, &g, X, 1, L, Y, nullptr) == -1);
}

void groups() {
    EXPECT(dqg_expert_group(nullptr, 1, 8, static_cast<const int32_t *>(fake(0x1000)),
                            static_cast<const float *>(fake(0x2000)), -1, X, Y, fake(0x50000), 1 << 20,
                            nullptr) == -1);
    EXPECT(dqg_expert_group_noalloc(nullptr, 1, 8, static_cast<const int32_t *>(fake(0x1000)),
                                    static_cast<const float *>(fake(0x2000)), -1, X, Y, nullptr) == -1);
    EXPECT(dqg_expert_group_scratch_bytes(nullptr, 1, 8) == 0);
    dqg_ticket t{};
    EXPECT(dqg_expert_group_take(&t) == -1);
    EXPECT(dqg_expert_group_take(nullptr) == -1);
    EXPECT(dqg_expert_table_set_swiglu_limit(nullptr, 1.f) == -1);
    EXPECT(dqg_expert_table_set_activation(nullptr, DQG_ACT_SWIGLU_V4) == -1);
    // tables whose shapes or formats disagree, or that hold no expert
    dqg_expert_table *out = nullptr;
    dqg_expert e{mat(4, 32, 64), mat(4, 32, 64), mat(4, 64, 64)};   // down must be [64 x 32]
    EXPECT(dqg_expert_table_create(&e, 1, &out) == -3 && out == nullptr);
    dqg_expert e2{mat(4, 32, 64), mat(7, 32, 64), mat(4, 64, 32)};
    EXPECT(dqg_expert_table_create(&e2, 1, &out) == -3 && out == nullptr);
    EXPECT(dqg_expert_table_create(&e2, 0, &out) == -1);
    EXPECT(dqg_expert_table_create(nullptr, 1, &out) == -1);
    dqg_expert_table_destroy(nullptr);
}

void routes() {
    const float *L = static_cast<const float *>(fake(0x60000));
    int32_t *ids = static_cast<int32_t *>(fake(0x70000));
    float *w = static_cast<float *>(fake(0x80000));
    const float inf = std::numeric_limits<float>::infinity(), nan = std::numeric_limits<float>::quiet_NaN();
    struct Case {
        int S, E, k, mode, renorm;
        uintptr_t bias;
        float scale;
        const float *logits;
        int32_t *ids;
        float *w;
    } cases[] = {
        {0, 64, 8, 0, 0, 0, 1.f, L, ids, w},    {1, 0, 1, 0, 0, 0, 1.f, L, ids, w},
        {1, 1025, 8, 0, 0, 0, 1.f, L, ids, w},  {1, 64, 0, 0, 0, 0, 1.f, L, ids, w},
        {1, 6, 7, 0, 0, 0, 1.f, L, ids, w},     {1, 256, 65, 0, 0, 0, 1.f, L, ids, w},
        {1, 64, 8, 2, 0, 0, 1.f, L, ids, w},    {1, 64, 8, 0, 2, 0, 1.f, L, ids, w},
        {1, 64, 8, 0, 0, 0, inf, L, ids, w},    {1, 64, 8, 0, 0, 0, nan, L, ids, w},
        {1, 64, 8, 0, 0, 0, 1.f, nullptr, ids, w},
        {1, 64, 8, 0, 0, 0, 1.f, L + 0, ids + 0, w + 0},   // valid but for the misaligned ones below
    };
    for (int i = 0; i < 11; ++i) {
        const Case &c = cases[i];
        EXPECT(dqg_route(c.logits, c.S, c.E, c.k, c.mode, c.renorm, static_cast<const float *>(fake(c.bias)),
                         c.scale, c.ids, c.w, nullptr) == -1);
    }
    const char *Lc = reinterpret_cast<const char *>(L);
    EXPECT(dqg_route(reinterpret_cast<const float *>(Lc + 2), 1, 64, 8, 0, 0, nullptr, 1.f, ids, w, nullptr) == -1);
    EXPECT(dqg_route(L, 1, 64, 8, 0, 0, static_cast<const float *>(fake(0x90002)), 1.f, ids, w, nullptr) == -1);
    EXPECT(dqg_route(L, 1, 64, 8, 0, 0, nullptr, 1.f, nullptr, w, nullptr) == -1);
    EXPECT(dqg_route(L, 1, 64, 8, 0, 0, nullptr, 1.f, ids,
                     reinterpret_cast<float *>(reinterpret_cast<char *>(w) + 1), nullptr) == -1);
}

void reads_and_counters() {
    uint32_t *sink = static_cast<uint32_t *>(fake(0x40000));
    EXPECT(dqg_read_bytes(nullptr, 1024, sink, nullptr) == -1);
    EXPECT(dqg_read_bytes(fake(0x30008), 1024, sink, nullptr) == -1);
    EXPECT(dqg_read_bytes(fake(0x30000), 0, sink, nullptr) == -1);
    EXPECT(dqg_read_bytes(fake(0x30000), 1000, sink, nullptr) == -1);
    EXPECT(dqg_read_bytes(fake(0x30000), 1024, nullptr, nullptr) == -1);
    dqg_stats_reset();
    const dqg_matrix m = mat(3);
    dqg_matmul(&m, X, 1, Y, nullptr);
    dqg_counters c{};
    dqg_stats(&c);
    EXPECT(c.calls_matmul == 1 && c.launches == 0);
    EXPECT(dqg_prof_begin(-1) == -1);
    int32_t n = -1;
    dqg_prof_launch rec[4];
    EXPECT(dqg_prof_end_launches(rec, 4, &n) != 0 || n == 0);
}

}  // namespace

int main() {
    matrices();
    vectors();
    groups();
    routes();
    reads_and_counters();
    EXPECT(dqg::g_stub_launches == 0);
    std::printf("%d checks, %d failed\n", g_checks, g_failed);
    return g_failed ? 1 : 0;
}
