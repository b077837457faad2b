// Host-side argument handling of libawq under AddressSanitizer and UndefinedBehaviorSanitizer
// (built by tests/test_host_sanitizers.py; needs no GPU).  Every call below is rejected on the
// host before anything is enqueued, so no device is touched: the "device" pointers are host
// canary buffers that must come back unchanged, and the host arrays of awq_search_multi are
// exactly n_w long, so a read past them is reported.  The workspace-size queries are also driven
// with extreme sizes, where an overflow in the size arithmetic would be undefined behaviour.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "../include/awq.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

namespace {
constexpr size_t kCanary = 1 << 16;
struct Canary {
    std::vector<unsigned char> b;
    Canary() : b(kCanary + 256, 0xA5) {}
    void* p() { return (void*)(((uintptr_t)b.data() + 255) & ~(uintptr_t)255); }   // 256-byte aligned
    bool intact() const {
        for (unsigned char c : b)
            if (c != 0xA5) return false;
        return true;
    }
};
awq_qconfig cfg(int g = 128, int zp = 1, int ng = 21, float clip = 0.f, int bits = 4) {
    awq_qconfig c;
    c.w_bit = bits;
    c.group_size = g;
    c.zero_point = zp;
    c.n_grid = ng;
    c.clip_ratio = clip;
    return c;
}
}  // namespace

int main() {
    Canary a, b, c, d, e, w;
    void* odd = (char*)a.p() + 2;
    const size_t big = (size_t)1 << 40;
    const int64_t huge = std::numeric_limits<int64_t>::max();
    const awq_qconfig ok = cfg();
    const awq_qconfig bad_cfgs[] = {cfg(128, 1, 21, 0.f, 3), cfg(96), cfg(128, 1, 1), cfg(128, 1, 65),
                                    cfg(128, 2), cfg(128, 1, 21, 1.5f), cfg(128, 1, 21, NAN)};

    // ---- statistic and its variants
    EXPECT(awq_act_stats(nullptr, 8, 16, (double*)b.p(), 0, 8, (float*)c.p(), w.p(), big, nullptr) < 0);
    EXPECT(awq_act_stats(a.p(), 0, 16, (double*)b.p(), 0, 8, (float*)c.p(), w.p(), big, nullptr) < 0);
    EXPECT(awq_act_stats(a.p(), 8, 16, (double*)b.p(), 2, 8, (float*)c.p(), w.p(), big, nullptr) < 0);
    EXPECT(awq_act_stats(a.p(), 8, 16, (double*)b.p(), 0, 7, (float*)c.p(), w.p(), big, nullptr) < 0);
    EXPECT(awq_act_stats(odd, 8, 16, (double*)b.p(), 0, 8, (float*)c.p(), w.p(), big, nullptr) < 0);
    EXPECT(awq_act_stats(a.p(), 4096, 4096, (double*)b.p(), 0, 4096, (float*)c.p(), w.p(), 8, nullptr) ==
           AWQ_ERR_WORKSPACE);
    EXPECT(awq_act_max(a.p(), 8, 16, (float*)b.p(), 3, w.p(), big, nullptr) < 0);
    EXPECT(awq_act_max(a.p(), -1, 16, (float*)b.p(), 0, w.p(), big, nullptr) < 0);
    EXPECT(awq_weight_mean_abs(a.p(), 0, 16, (float*)b.p(), nullptr) < 0);
    EXPECT(awq_weight_mean_abs(a.p(), (int64_t)1 << 40, 16, (float*)b.p(), nullptr) < 0);
    EXPECT(awq_scale_table(nullptr, 16, 21, (float*)b.p(), nullptr) < 0);
    EXPECT(awq_scale_table((float*)a.p(), 16, 65, (float*)b.p(), nullptr) == AWQ_ERR_UNSUPPORTED);
    EXPECT(awq_scale_table_ex((float*)a.p(), nullptr, 16, 21, 2, (float*)b.p(), nullptr) < 0);
    EXPECT(awq_scale_table_ex((float*)a.p(), (float*)odd, 16, 21, 0, (float*)b.p(), nullptr) < 0);

    // ---- searches
    for (const awq_qconfig& bc : bad_cfgs) {
        EXPECT(awq_search(a.p(), 8, a.p(), 128, 16, (float*)a.p(), &bc, w.p(), big, (double*)b.p(), (int32_t*)c.p(),
                          (float*)d.p(), nullptr) < 0);
        EXPECT(awq_search_table(a.p(), 8, a.p(), 128, 16, (float*)a.p(), &bc, w.p(), big, (double*)b.p(),
                                (int32_t*)c.p(), (float*)d.p(), nullptr) < 0);
        EXPECT(awq_pack(a.p(), 128, 16, (float*)a.p(), &bc, (uint32_t*)b.p(), (float*)c.p(), (uint8_t*)d.p(),
                        nullptr) < 0);
        EXPECT(awq_search_workspace_size(8, 128, 16, &bc) == 0);
    }
    EXPECT(awq_search(a.p(), 8, a.p(), 128, 16, (float*)a.p(), nullptr, w.p(), big, (double*)b.p(), (int32_t*)c.p(),
                      (float*)d.p(), nullptr) < 0);
    EXPECT(awq_search(a.p(), 8, a.p(), 100, 16, (float*)a.p(), &ok, w.p(), big, (double*)b.p(), (int32_t*)c.p(),
                      (float*)d.p(), nullptr) < 0);
    EXPECT(awq_search(a.p(), (int64_t)1 << 24, a.p(), 1 << 14, 16, (float*)a.p(), &ok, w.p(), big, (double*)b.p(),
                      (int32_t*)c.p(), (float*)d.p(), nullptr) < 0);   // T K >= 2^31
    const size_t need = awq_search_workspace_size(8, 128, 16, &ok);
    EXPECT(need > 0);
    EXPECT(awq_search(a.p(), 8, a.p(), 128, 16, (float*)a.p(), &ok, w.p(), need - 1, (double*)b.p(), (int32_t*)c.p(),
                      (float*)d.p(), nullptr) == AWQ_ERR_WORKSPACE);
    EXPECT(awq_search(a.p(), 8, a.p(), 128, 16, (float*)a.p(), &ok, (char*)w.p() + 16, big, (double*)b.p(),
                      (int32_t*)c.p(), (float*)d.p(), nullptr) == AWQ_ERR_INVALID_ARG);   // workspace alignment
    EXPECT(awq_clip_search(a.p(), 8, a.p(), 128, 16, (float*)a.p(), &ok, 0.f, w.p(), big, (double*)b.p(),
                           (int32_t*)c.p(), (float*)d.p(), nullptr) < 0);
    EXPECT(awq_clip_search(a.p(), 8, a.p(), 128, 16, (float*)a.p(), &ok, NAN, w.p(), big, (double*)b.p(),
                           (int32_t*)c.p(), (float*)d.p(), nullptr) < 0);
    {
        const int64_t Ns[3] = {24, 8, 40};
        const void* Ws[3] = {a.p(), b.p(), c.p()};
        const int64_t Nbad[3] = {24, 0, 40};
        const void* Wnull[3] = {a.p(), nullptr, c.p()};
        const void* Wodd[3] = {a.p(), odd, c.p()};
        EXPECT(awq_search_multi_workspace_size(8, 128, 3, Ns, &ok) == awq_search_workspace_size(8, 128, 96, &ok));
        EXPECT(awq_search_multi_workspace_size(8, 128, 3, Nbad, &ok) == 0);
        EXPECT(awq_search_multi_workspace_size(8, 128, 0, Ns, &ok) == 0);
        EXPECT(awq_search_multi_workspace_size(8, 128, AWQ_MAX_PROJECTIONS + 1, Ns, &ok) == 0);
        EXPECT(awq_search_multi(a.p(), 8, 3, Wnull, Ns, 128, (float*)a.p(), &ok, w.p(), big, (double*)b.p(), nullptr,
                                (int32_t*)c.p(), (float*)d.p(), nullptr) < 0);
        EXPECT(awq_search_multi(a.p(), 8, 3, Wodd, Ns, 128, (float*)a.p(), &ok, w.p(), big, (double*)b.p(), nullptr,
                                (int32_t*)c.p(), (float*)d.p(), nullptr) < 0);
        EXPECT(awq_search_multi(a.p(), 8, 3, Ws, Nbad, 128, (float*)a.p(), &ok, w.p(), big, (double*)b.p(), nullptr,
                                (int32_t*)c.p(), (float*)d.p(), nullptr) < 0);
        EXPECT(awq_search_multi(a.p(), 8, 3, Ws, Ns, 128, (float*)a.p(), &ok, w.p(), 16, (double*)b.p(), nullptr,
                                (int32_t*)c.p(), (float*)d.p(), nullptr) == AWQ_ERR_WORKSPACE);
        EXPECT(awq_search_multi(a.p(), 8, 3, Ws, Ns, 128, (float*)a.p(), &ok, w.p(), big, (double*)b.p(),
                                (double*)odd, (int32_t*)c.p(), (float*)d.p(), nullptr) < 0);
    }
    // ---- greedy
    EXPECT(awq_greedy_workspace_size(256, 40, &ok, 1) == 0);
    EXPECT(awq_greedy_search(a.p(), 256, 40, (float*)a.p(), &ok, 20, 0, w.p(), big, (float*)b.p(), nullptr, nullptr,
                             nullptr) < 0);
    EXPECT(awq_greedy_search(a.p(), 256, 40, (float*)a.p(), &ok, 33, 3, w.p(), big, (float*)b.p(), nullptr, nullptr,
                             nullptr) < 0);
    {
        const awq_qconfig clipped = cfg(128, 1, 21, 0.9f);
        EXPECT(awq_greedy_search(a.p(), 256, 40, (float*)a.p(), &clipped, 20, 3, w.p(), big, (float*)b.p(), nullptr,
                                 nullptr, nullptr) == AWQ_ERR_UNSUPPORTED);
    }
    EXPECT(awq_greedy_search(a.p(), (int64_t)128 * 70000, 40, (float*)a.p(), &ok, 20, 3, w.p(), big, (float*)b.p(),
                             nullptr, nullptr, nullptr) < 0);   // more than 65535 groups
    // ---- pack
    EXPECT(awq_pack(a.p(), (int64_t)128 * 70000, 16, (float*)a.p(), &ok, (uint32_t*)b.p(), (float*)c.p(),
                    (uint8_t*)d.p(), nullptr) < 0);
    EXPECT(awq_pack(odd, 128, 16, (float*)a.p(), &ok, (uint32_t*)b.p(), (float*)c.p(), (uint8_t*)d.p(), nullptr) < 0);
    // ---- W4A16 product, with and without a workspace
    EXPECT(awq_w4a16_gemm(a.p(), 1, (float*)a.p(), (uint32_t*)a.p(), (float*)a.p(), (uint8_t*)a.p(), 128, 12, 128,
                          b.p(), w.p(), big, nullptr) == AWQ_ERR_INVALID_ARG);
    EXPECT(awq_w4a16_gemm(a.p(), 1, (float*)a.p(), (uint32_t*)a.p(), (float*)a.p(), (uint8_t*)a.p(), 128, 16, 96,
                          b.p(), w.p(), big, nullptr) == AWQ_ERR_UNSUPPORTED);
    EXPECT(awq_w4a16_gemm(a.p(), 1, (float*)a.p(), (uint32_t*)a.p(), (float*)a.p(), (uint8_t*)a.p(), 8192, 8192, 128,
                          b.p(), (char*)w.p() + 16, big, nullptr) == AWQ_ERR_INVALID_ARG);
    EXPECT(awq_w4a16_gemm(a.p(), 1, (float*)a.p(), (uint32_t*)a.p(), (float*)a.p(), (uint8_t*)a.p(), 8192, 8192, 128,
                          b.p(), w.p(), 16, nullptr) == AWQ_ERR_WORKSPACE);
    EXPECT(awq_w4a16_gemm(a.p(), 1, (float*)a.p(), (uint32_t*)a.p(), (float*)a.p(), (uint8_t*)a.p(), 128,
                          (int64_t)1 << 40, 128, b.p(), w.p(), big, nullptr) == AWQ_ERR_INVALID_ARG);
    EXPECT(awq_w4a16_gemm(a.p(), (int64_t)1 << 40, (float*)a.p(), (uint32_t*)a.p(), (float*)a.p(), (uint8_t*)a.p(),
                          128, 16, 128, b.p(), w.p(), big, nullptr) < 0);
    EXPECT(awq_w4a16_gemm(a.p(), 1, (float*)odd, (uint32_t*)a.p(), (float*)a.p(), (uint8_t*)a.p(), 128, 16, 128,
                          b.p(), w.p(), big, nullptr) == AWQ_ERR_INVALID_ARG);
    EXPECT(awq_w4a16_gemm_noalloc(a.p(), 1, (float*)a.p(), (uint32_t*)a.p(), (float*)a.p(), (uint8_t*)a.p(), 8192,
                                  4194304 - 256, 128, b.p(), nullptr) == AWQ_ERR_SCRATCH);
    EXPECT(awq_w4a16_gemm_noalloc(a.p(), 1, (float*)a.p(), (uint32_t*)a.p(), (float*)a.p(), (uint8_t*)a.p(), 128,
                                  12, 128, b.p(), nullptr) == AWQ_ERR_INVALID_ARG);

    // ---- size queries at the edges: no overflow, no crash
    const int64_t edge[] = {0, 1, 7, 8, 128, 4096, (int64_t)1 << 31, (int64_t)1 << 40, huge, -1};
    size_t sink = 0;
    for (int64_t x : edge)
        for (int64_t y : edge) {
            sink += awq_act_stats_workspace_size(x, y);
            sink += awq_search_workspace_size(x, y, 16, &ok);
            sink += awq_search_workspace_size(8, 128, y, &ok);
            sink += awq_greedy_workspace_size(x, y, &ok, 20);
            sink += awq_w4a16_gemm_workspace_size(x, y, 16, 128);
            sink += awq_w4a16_gemm_workspace_size(1, 8192, y, 128);
        }
    EXPECT(awq_w4a16_gemm_static_scratch_bytes() >= ((size_t)16 << 20));
    for (int st = -6; st <= 1; ++st) EXPECT(awq_status_string(st) != nullptr);

    EXPECT(a.intact() && b.intact() && c.intact() && d.intact() && e.intact() && w.intact());
    std::printf("host checks: %d failures (size sink %zu)\n", failures, sink);
    return failures ? 1 : 0;
}
