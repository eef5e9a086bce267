// Host-only driver of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitizers.py).
// It calls only paths that return before any launch: dims validation,
// workspace sizing, status strings, the argument checks of every entry point
// and the host-only slot planner, over ordinary, limit and invalid inputs. A
// sanitizer report or a failed expectation exits non-zero.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "hsakv.h"

static int failures = 0;

#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static hsakv_dims dims(int H, int d, int Lq, int tpf, int Psize, int P, int Kp, int Binter, int Bintra, int Bq,
                       int r, int dtype) {
    hsakv_dims x;
    x.H = H; x.d = d; x.Lq = Lq; x.tokens_per_frame = tpf; x.Psize = Psize; x.P = P; x.Kp = Kp;
    x.Binter = Binter; x.Bintra = Bintra; x.Bq = Bq; x.r = r; x.dtype = dtype;
    return x;
}

// a 256-byte aligned stand-in device address that no call here dereferences
static void* const FAKE = reinterpret_cast<void*>(uintptr_t(1) << 20);

static void check_validation() {
    const hsakv_dims ok[] = {
        dims(2, 64, 256, 16, 8, 6, 2, 128, 64, 64, 32, HSAKV_F32),
        dims(12, 128, 4680, 1560, 8, 32, 4, 128, 64, 64, 256, HSAKV_BF16),
        dims(12, 128, 4680, 1560, 8, 96, 4, 128, 64, 64, 256, HSAKV_BF16),
        dims(40, 128, 4680, 1560, 8, 32, 4, 128, 64, 64, 256, HSAKV_BF16),
        dims(40, 128, 10800, 3600, 8, 24, 4, 128, 64, 64, 512, HSAKV_BF16),
        dims(1, 64, 1, 1, 1, 1, 1, 64, 64, 64, 32, HSAKV_BF16),
    };
    for (const hsakv_dims& d : ok) {
        EXPECT(hsakv_validate(&d) == HSAKV_OK);
        for (int e = 0; e <= 9; ++e) {
            const size_t n = hsakv_workspace_bytes(&d, e);
            EXPECT(n < (size_t(1) << 40));
        }
        EXPECT(hsakv_workspace_bytes(&d, 99) == 0);
    }
    const hsakv_dims base = ok[1];
    struct Bad {
        hsakv_dims d;
        int code;
    };
    std::vector<Bad> bad;
    auto with = [&](auto f, int code) {
        hsakv_dims d = base;
        f(d);
        bad.push_back({d, code});
    };
    with([](hsakv_dims& d) { d.H = 0; }, HSAKV_ERR_BAD_DIMS);
    with([](hsakv_dims& d) { d.Lq = -5; }, HSAKV_ERR_BAD_DIMS);
    with([](hsakv_dims& d) { d.r = 0; }, HSAKV_ERR_BAD_DIMS);
    with([](hsakv_dims& d) { d.d = 96; }, HSAKV_ERR_UNSUPPORTED);
    with([](hsakv_dims& d) { d.Bq = 32; }, HSAKV_ERR_UNSUPPORTED);
    with([](hsakv_dims& d) { d.Binter = 100; }, HSAKV_ERR_UNSUPPORTED);
    with([](hsakv_dims& d) { d.Bintra = 1024; }, HSAKV_ERR_UNSUPPORTED);
    with([](hsakv_dims& d) { d.r = 33; }, HSAKV_ERR_UNSUPPORTED);
    with([](hsakv_dims& d) { d.r = 2048; }, HSAKV_ERR_UNSUPPORTED);
    with([](hsakv_dims& d) { d.Kp = 65; }, HSAKV_ERR_UNSUPPORTED);
    with([](hsakv_dims& d) { d.H = 257; }, HSAKV_ERR_UNSUPPORTED);
    with([](hsakv_dims& d) { d.H = 200; }, HSAKV_ERR_UNSUPPORTED);              // H d > 16384
    with([](hsakv_dims& d) { d.tokens_per_frame = 1 << 28; }, HSAKV_ERR_BAD_DIMS);  // Tp > 2^30
    with([](hsakv_dims& d) { d.tokens_per_frame = 1 << 26; d.Kp = 64; }, HSAKV_ERR_BAD_DIMS);  // L >= 2^31
    with([](hsakv_dims& d) { d.P = 65537; }, HSAKV_ERR_UNSUPPORTED);
    with([](hsakv_dims& d) { d.tokens_per_frame = 100000; }, HSAKV_ERR_UNSUPPORTED);  // NB > 4096
    with([](hsakv_dims& d) { d.dtype = 7; }, HSAKV_ERR_BAD_DTYPE);
    for (const Bad& b : bad) {
        EXPECT(hsakv_validate(&b.d) == b.code);
        for (int e = 0; e <= 9; ++e) EXPECT(hsakv_workspace_bytes(&b.d, e) == 0);
    }
    EXPECT(hsakv_validate(nullptr) == HSAKV_ERR_NULL_ARG);
    EXPECT(hsakv_workspace_bytes(nullptr, 0) == 0);
    for (int s = -12; s <= 2; ++s) EXPECT(hsakv_status_str(s) != nullptr && std::strlen(hsakv_status_str(s)) > 0);
    EXPECT(hsakv_version() > 0);
}

static void check_entry_points() {
    const hsakv_dims d = dims(12, 128, 4680, 1560, 8, 32, 4, 128, 64, 64, 256, HSAKV_BF16);
    hsakv_dims bad = d;
    bad.d = 96;
    void* F = FAKE;
    char* mis = static_cast<char*>(FAKE) + 4;
    float tau[12];
    for (float& t : tau) t = 0.5f;
    float bad_tau[12];
    for (float& t : bad_tau) t = 0.f;

    EXPECT(hkv_page_summary(nullptr, F, (float*)F, F, 1 << 30, nullptr) == HSAKV_ERR_NULL_ARG);
    EXPECT(hkv_page_summary(&bad, F, (float*)F, F, 1 << 30, nullptr) == HSAKV_ERR_UNSUPPORTED);
    EXPECT(hkv_page_summary(&d, mis, (float*)F, F, 1 << 30, nullptr) == HSAKV_ERR_MISALIGNED);
    EXPECT(hkv_page_summary(&d, F, (float*)F, F, 16, nullptr) == HSAKV_ERR_WORKSPACE);

    EXPECT(hkv_gather(&d, F, F, (const float*)F, (const int32_t*)F, 0, nullptr, nullptr, F, (int32_t*)F,
                      (int32_t*)F, F, F, F, 0, nullptr) == HSAKV_ERR_WORKSPACE);
    EXPECT(hkv_gather(&d, nullptr, F, (const float*)F, (const int32_t*)F, 0, nullptr, nullptr, F, (int32_t*)F,
                      (int32_t*)F, F, F, F, size_t(1) << 30, nullptr) == HSAKV_ERR_NULL_ARG);
    hsakv_retrieval badpol{17, 0, 0};
    EXPECT(hkv_gather(&d, F, F, (const float*)F, (const int32_t*)F, 0, &badpol, nullptr, F, (int32_t*)F,
                      (int32_t*)F, F, F, F, size_t(1) << 30, nullptr) != HSAKV_OK);
    hsakv_tiers half_tiers{(int32_t*)F, nullptr, F};
    EXPECT(hkv_gather(&d, F, F, (const float*)F, (const int32_t*)F, 0, nullptr, &half_tiers, F, (int32_t*)F,
                      (int32_t*)F, F, F, F, size_t(1) << 30, nullptr) == HSAKV_ERR_NULL_ARG);

    EXPECT(hsa_select(&d, F, F, F, (const int32_t*)F, bad_tau, (int32_t*)F, (int32_t*)F, nullptr, nullptr, F,
                      size_t(1) << 30, nullptr) == HSAKV_ERR_BAD_TAU);
    EXPECT(hsa_select(&d, F, F, F, (const int32_t*)F, nullptr, (int32_t*)F, (int32_t*)F, nullptr, nullptr, F,
                      size_t(1) << 30, nullptr) == HSAKV_ERR_NULL_ARG);
    EXPECT(hsa_select(&d, F, F, F, (const int32_t*)F, tau, (int32_t*)F, (int32_t*)F, nullptr, nullptr, F, 8,
                      nullptr) == HSAKV_ERR_WORKSPACE);

    EXPECT(hsa_sparse_attn(&d, F, F, F, F, F, (const int32_t*)F, (const int32_t*)F, (const int32_t*)F,
                           (float*)F, F, 8, nullptr) == HSAKV_ERR_WORKSPACE);
    EXPECT(hsa_sparse_attn(&d, mis, F, F, F, F, (const int32_t*)F, (const int32_t*)F, (const int32_t*)F,
                           (float*)F, F, size_t(1) << 30, nullptr) == HSAKV_ERR_MISALIGNED);
    EXPECT(hsa_linear_branch(&d, F, F, F, F, F, (const int32_t*)F, F, F, (float*)F, nullptr, nullptr, F, 8,
                             nullptr) == HSAKV_ERR_WORKSPACE);
    EXPECT(hsa_fuse(&d, F, (const float*)F, (const float*)F, (const float*)F, (const float*)F, nullptr, nullptr,
                    nullptr) == HSAKV_ERR_NULL_ARG);

    hsakv_inputs in;
    std::memset(&in, 0, sizeof(in));
    hsakv_outputs out;
    std::memset(&out, 0, sizeof(out));
    EXPECT(hsa_forward(&d, tau, 0, nullptr, nullptr, &in, &out, F, size_t(1) << 30, nullptr, nullptr) ==
           HSAKV_ERR_NULL_ARG);
    EXPECT(hsa_forward(&d, bad_tau, 0, nullptr, nullptr, &in, &out, F, size_t(1) << 30, nullptr, nullptr) ==
           HSAKV_ERR_BAD_TAU);

    EXPECT(hsa_backward_params(&d, F, F, F, F, F, (const int32_t*)F, (const float*)F, (const float*)F,
                               (const float*)F, (const float*)F, (const float*)F, (const float*)F, F, (float*)F,
                               (float*)F, (float*)F, (float*)F, F, 8, nullptr, nullptr) == HSAKV_ERR_WORKSPACE);
    EXPECT(hkv_page_commit(&d, F, F, (float*)F, (int32_t*)F, F, F, -1, 0, 0, nullptr, 0, nullptr) ==
           HSAKV_ERR_BAD_DIMS);
    EXPECT(hsa_sparse_attn_static(&bad, F, F, F, F, F, (const int32_t*)F, (const int32_t*)F, (const int32_t*)F,
                                  (float*)F, nullptr) == HSAKV_ERR_UNSUPPORTED);
    EXPECT(hsakv_last_hip_error() == 0);
}

// The slot planner against its rule: after a plan every wanted page has a
// slot, the two maps agree, and promotions fit the slots.
static void check_planner() {
    std::mt19937 rng(1234);
    for (int trial = 0; trial < 300; ++trial) {
        const int P = 1 + int(rng() % 40), slots = int(rng() % 10);
        std::vector<int32_t> sop(P, -1), pos(slots, -1);
        std::vector<int64_t> last(P, 0);
        for (int step = 1; step <= 20; ++step) {
            const int nw = int(rng() % 6);
            std::vector<int32_t> want(nw);
            for (int32_t& w : want) w = int32_t(rng() % P);
            const int cap = nw > 0 ? nw : 1;
            std::vector<int32_t> pp(cap), ps(cap), up(2 * cap), uv(2 * cap);
            int32_t np = -1, nu = -1;
            const int st = hkv_tier_plan(P, slots, sop.data(), pos.data(), last.data(), step, want.data(), nw,
                                         pp.data(), ps.data(), &np, up.data(), uv.data(), &nu);
            EXPECT(st == HSAKV_OK);
            EXPECT(np >= 0 && np <= cap && np <= slots);
            EXPECT(nu >= 0 && nu <= 2 * np);
            for (int s = 0; s < slots; ++s)
                if (pos[s] >= 0) EXPECT(sop[pos[s]] == s);
            for (int p = 0; p < P; ++p)
                if (sop[p] >= 0) EXPECT(sop[p] < slots && pos[sop[p]] == p);
            if (nw <= slots)
                for (int32_t w : want) EXPECT(sop[w] >= 0);
        }
    }
    int32_t sop[4] = {-1, -1, -1, -1}, pos[2] = {-1, -1}, np = 0, nu = 0, pp[2], ps[2], up[4], uv[4];
    int64_t last[4] = {0, 0, 0, 0};
    int32_t bad_want[1] = {4};
    EXPECT(hkv_tier_plan(4, 2, sop, pos, last, 1, bad_want, 1, pp, ps, &np, up, uv, &nu) == HSAKV_ERR_BAD_DIMS);
    EXPECT(hkv_tier_plan(4, 2, nullptr, pos, last, 1, bad_want, 1, pp, ps, &np, up, uv, &nu) == HSAKV_ERR_NULL_ARG);
}

int main() {
    check_validation();
    check_entry_points();
    check_planner();
    if (failures) {
        std::fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    std::printf("host ABI driver: all checks passed\n");
    return 0;
}
