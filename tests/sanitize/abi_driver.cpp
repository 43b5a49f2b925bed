// Host-side driver of the C ABI for the sanitizer build: every entry point of
// include/lix.h called with argument sets that must fail validation (checked
// against the documented status), plus a seeded sweep over extreme sizes and
// pointer values (each result must be a documented status).  Pointers are
// fake addresses that are never dereferenced: a call that passes validation
// stops at the device check (LIX_ERR_DEVICE), before any launch.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "lix.h"

namespace {

int g_failures = 0;
long g_calls = 0;

void expect(int got, int want, const char* what, int line) {
    ++g_calls;
    if (got != want) {
        std::fprintf(stderr, "line %d: %s: got %d (%s), want %d\n", line, what, got, lix_status_string(got), want);
        ++g_failures;
    }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

void* fake(uintptr_t off) { return reinterpret_cast<void*>((uintptr_t)1 << 20 | off); }

bool documented(int st) {
    return st == LIX_OK || st == LIX_ERR_NULL || st == LIX_ERR_SHAPE || st == LIX_ERR_UNSUPPORTED ||
           st == LIX_ERR_DEVICE || st == LIX_ERR_LAUNCH;
}

// Deterministic generator (splitmix64).
uint64_t g_state = 0x243F6A8885A308D3ull;
uint64_t next_u64() {
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int pick_int() {
    static const int vals[] = {INT_MIN, -65536, -2, -1, 0, 1, 2, 3, 4, 7, 8, 15, 16, 17, 31, 32, 48, 63, 64, 65,
                               96, 127, 128, 129, 255, 256, 2047, 2048, 2049, 4096, 8192, 32768, 32769, 65536,
                               65537, 131071, 131072, 1 << 20, 1 << 24, 1 << 30, INT_MAX};
    return vals[next_u64() % (sizeof(vals) / sizeof(vals[0]))];
}

void* pick_ptr() {
    switch (next_u64() % 5) {
        case 0: return nullptr;
        case 1: return fake(1);
        case 2: return fake(2);
        case 3: return fake(4);
        default: return fake(0);
    }
}

template <class T>
T* P(uintptr_t off = 0) { return static_cast<T*>(fake(off)); }

}  // namespace

int main() {
    const int NUL = LIX_ERR_NULL, SHP = LIX_ERR_SHAPE, UNS = LIX_ERR_UNSUPPORTED, DEV = LIX_ERR_DEVICE;
    void* p = fake(0);
    const int32_t* ip = P<const int32_t>();

    // ---- status strings
    for (int st = -8; st <= 2; ++st) {
        const char* s = lix_status_string(st);
        if (s == nullptr || std::strlen(s) == 0) { std::fprintf(stderr, "empty status string %d\n", st); ++g_failures; }
    }
    if (lix_version() < 100) ++g_failures;

    // ---- lix_indexer_logits
    auto logits = [&](const void* q, const void* k, const float* w, int B, int S, int Skv, int H, int D, int c,
                      const int32_t* ks, const int32_t* ke, float* out) {
        return lix_indexer_logits(q, k, w, B, S, Skv, H, D, c, ks, ke, out, nullptr);
    };
    float* fp = P<float>();
    EXPECT(logits(nullptr, p, fp, 1, 8, 2, 64, 128, 4, nullptr, nullptr, fp), NUL);
    EXPECT(logits(p, p, fp, 0, 8, 2, 64, 128, 4, nullptr, nullptr, fp), SHP);
    EXPECT(logits(p, p, fp, 1, 8, 2, 64, 128, 0, nullptr, nullptr, fp), SHP);
    EXPECT(logits(p, p, fp, 1, 8, 2, 64, 128, 4, ip, nullptr, fp), SHP);
    EXPECT(logits(p, p, fp, 1, 8, 2, 48, 128, 4, nullptr, nullptr, fp), UNS);
    EXPECT(logits(p, p, fp, 1, 8, 2, 64, 24, 4, nullptr, nullptr, fp), UNS);
    EXPECT(logits(fake(8), p, fp, 1, 8, 2, 64, 128, 4, nullptr, nullptr, fp), UNS);
    EXPECT(logits(p, p, fp, INT_MAX, INT_MAX, INT_MAX, 128, 256, 4, nullptr, nullptr, fp), UNS);
    EXPECT(logits(p, p, fp, 131072, 8, 2, 64, 128, 4, nullptr, nullptr, fp), UNS);
    EXPECT(logits(p, p, fp, 1, 8, 2, 64, 128, 4, nullptr, nullptr, fp), DEV);
    EXPECT(lix_indexer_logits_visible(nullptr, p, fp, 1, 8, 2, 64, 128, 4, nullptr, nullptr, fp, nullptr), NUL);
    EXPECT(lix_indexer_logits_visible(p, p, fp, 1, 8, 2, 48, 128, 4, nullptr, nullptr, fp, nullptr), UNS);
    EXPECT(lix_indexer_logits_visible(p, p, fp, 1, 8, 2, 64, 128, 4, nullptr, nullptr, fp, nullptr), DEV);

    // ---- lix_topk (fused and materialized)
    int32_t* op = P<int32_t>();
    auto topk = [&](const void* q, const float* lg, int B, int S, int Skv, int H, int D, int c, int tk) {
        return lix_topk(q, q, q ? fp : nullptr, lg, B, S, Skv, H, D, c, nullptr, nullptr, tk, fp, op, nullptr);
    };
    EXPECT(topk(nullptr, nullptr, 1, 8, 4, 64, 128, 4, 2), NUL);
    EXPECT(topk(p, nullptr, 1, 8, 4, 64, 128, 4, 5), SHP);
    EXPECT(topk(p, nullptr, 1, 8, 4, 4, 128, 4, 2), UNS);
    EXPECT(topk(p, nullptr, 1, 8, 4096, 8, 128, 4, 1024), UNS);
    EXPECT(topk(p, nullptr, 1, 8, 70000, 64, 128, 4, 16), UNS);
    EXPECT(topk(p, nullptr, 1, 8, 4096, 64, 128, 4, 2048), DEV);
    EXPECT(topk(nullptr, fp, 1, 8, 4096, 0, 0, 4, 2048), DEV);
    EXPECT(topk(nullptr, fp, INT_MAX, INT_MAX, 4096, 0, 0, 4, 2048), UNS);

    // ---- fused support query agrees with lix_topk
    for (int H : {1, 2, 4, 8, 16, 32, 64, 128, 3, 0, -8, 256})
        for (int D : {16, 32, 64, 128, 256, 0, 24, 272})
            for (int tk : {1, 383, 384, 576, 577, 1216, 2048, 2049, -1})
                for (int Skv : {4096, 65536, 65537}) {
                    const int sup = lix_topk_fused_supported(Skv, H, D, tk);
                    const int st = topk(p, nullptr, 1, 8, Skv, H, D, 4, tk);
                    if ((sup == 1) != (st == DEV)) {
                        std::fprintf(stderr, "fused support %d vs status %d at H=%d D=%d topk=%d Skv=%d\n", sup, st,
                                     H, D, tk, Skv);
                        ++g_failures;
                    }
                    ++g_calls;
                }

    // ---- lix_topk_scores, lix_indexer_scores_at, lix_indexer_backward, V4.1, lix_topk_bf16
    EXPECT(lix_topk_scores(nullptr, ip, 1, 4, 8, 2, fp, nullptr), NUL);
    EXPECT(lix_topk_scores(fp, ip, 1, 4, 8, 0, fp, nullptr), SHP);
    EXPECT(lix_topk_scores(fp, ip, 1 << 16, 1 << 16, 8, 1 << 16, fp, nullptr), UNS);
    EXPECT(lix_topk_scores(fp, ip, 1, 4, 8, 2, fp, nullptr), DEV);
    EXPECT(lix_indexer_scores_at(p, p, fp, ip, 1, 8, 4, 64, 128, 4, nullptr, nullptr, 0, fp, nullptr), SHP);
    EXPECT(lix_indexer_scores_at(p, p, fp, ip, 1, 8, 4, 64, 128, 4, nullptr, nullptr, 2, fp, nullptr), DEV);
    const long long ws = lix_indexer_backward_workspace_bytes(1, 8, 4, 64, 128, 2);
    if (ws <= 0) ++g_failures;
    if (lix_indexer_backward_workspace_bytes(1, 8, 40000, 64, 128, 2) != -1) ++g_failures;
    if (lix_indexer_backward_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 64, 128, 2) != -1) ++g_failures;
    EXPECT(lix_indexer_backward(p, p, fp, ip, fp, 1, 8, 4, 64, 128, 4, nullptr, nullptr, 2, fp, fp, fp, p, ws - 1,
                                nullptr), SHP);
    EXPECT(lix_indexer_backward(p, p, fp, ip, fp, 1, 8, 4, 128, 128, 4, nullptr, nullptr, 2, fp, fp, fp, p, ws,
                                nullptr), UNS);
    EXPECT(lix_indexer_backward(p, p, fp, ip, fp, 1, 8, 4, 64, 128, 4, nullptr, nullptr, 2, fp, fp, fp, p, ws,
                                nullptr), DEV);
    const uint8_t* al = P<const uint8_t>();
    EXPECT(lix_indexer_scores_v41(p, p, p, al, 1, 4, 2, 6, 128, p, nullptr), UNS);
    EXPECT(lix_indexer_scores_v41(p, p, p, al, 1, 4, 2, 64, 128, p, nullptr), DEV);
    auto streaming = [&](int B, int S, int Skv, int H, int D, int tk, void* w, long long wb) {
        return lix_topk_streaming(p, p, fp, B, S, Skv, H, D, 4, nullptr, nullptr, tk, fp, op, w, wb, nullptr);
    };
    EXPECT(streaming(1, 8, 4, 64, 128, 2, nullptr, 1 << 20), NUL);
    EXPECT(streaming(1, 8, 4, 64, 128, 5, p, 1 << 20), SHP);
    EXPECT(streaming(1, 8, 8193, 64, 128, 5, p, 1 << 20), UNS);
    EXPECT(streaming(1, 8, 8192, 64, 128, 5, p, 4 * 8192 * 4 - 1), SHP);
    EXPECT(streaming(1, 8, 8192, 64, 128, 5, fake(128), 4 * 8192 * 4), UNS);
    EXPECT(streaming(1, 8, 8192, 64, 128, 5, p, 4 * 8192 * 4), DEV);
    EXPECT(streaming(INT_MAX, INT_MAX, 8192, 128, 256, 5, p, 1LL << 40), UNS);
    if (lix_topk_streaming_workspace_bytes(1, 8, 8193, 64, 128) != -1) ++g_failures;
    if (lix_topk_streaming_workspace_bytes(INT_MAX, INT_MAX, 8192, 64, 128) != -1) ++g_failures;
    EXPECT(lix_topk_bf16(p, 1, 8, 8193, 4, p, op, nullptr), UNS);
    EXPECT(lix_topk_bf16(p, 1, 8, 16, 4, p, op, nullptr), DEV);

    // ---- seeded sweep over extreme sizes and pointers: only documented statuses, no sanitizer report
    for (int it = 0; it < 20000; ++it) {
        int st;
        switch (it % 8) {
            case 0:
                st = lix_indexer_logits(pick_ptr(), pick_ptr(), (float*)pick_ptr(), pick_int(), pick_int(), pick_int(),
                                        pick_int(), pick_int(), pick_int(), nullptr, nullptr, (float*)pick_ptr(),
                                        nullptr);
                break;
            case 1:
                st = lix_topk(pick_ptr(), pick_ptr(), (float*)pick_ptr(), (float*)pick_ptr(), pick_int(), pick_int(),
                              pick_int(), pick_int(), pick_int(), pick_int(), nullptr, nullptr, pick_int(),
                              (float*)pick_ptr(), (int32_t*)pick_ptr(), nullptr);
                break;
            case 2:
                st = lix_topk_scores((float*)pick_ptr(), (int32_t*)pick_ptr(), pick_int(), pick_int(), pick_int(),
                                     pick_int(), (float*)pick_ptr(), nullptr);
                break;
            case 3:
                st = lix_indexer_scores_at(pick_ptr(), pick_ptr(), (float*)pick_ptr(), (int32_t*)pick_ptr(),
                                           pick_int(), pick_int(), pick_int(), pick_int(), pick_int(), pick_int(),
                                           (int32_t*)pick_ptr(), (int32_t*)pick_ptr(), pick_int(),
                                           (float*)pick_ptr(), nullptr);
                break;
            case 4: {
                const int B = pick_int(), S = pick_int(), Skv = pick_int(), H = pick_int(), D = pick_int();
                (void)lix_indexer_backward_workspace_bytes(B, S, Skv, H, D, pick_int());
                st = lix_indexer_backward(pick_ptr(), pick_ptr(), (float*)pick_ptr(), (int32_t*)pick_ptr(),
                                          (float*)pick_ptr(), B, S, Skv, H, D, pick_int(), nullptr, nullptr,
                                          pick_int(), (float*)pick_ptr(), (float*)pick_ptr(), (float*)pick_ptr(),
                                          pick_ptr(), (long long)pick_int() * 4096, nullptr);
                break;
            }
            case 5:
                st = lix_indexer_scores_v41(pick_ptr(), pick_ptr(), pick_ptr(), (uint8_t*)pick_ptr(), pick_int(),
                                            pick_int(), pick_int(), pick_int(), pick_int(), pick_ptr(), nullptr);
                break;
            case 6:
                st = lix_topk_streaming(pick_ptr(), pick_ptr(), (float*)pick_ptr(), pick_int(), pick_int(), pick_int(),
                                        pick_int(), pick_int(), pick_int(), nullptr, nullptr, pick_int(),
                                        (float*)pick_ptr(), (int32_t*)pick_ptr(), pick_ptr(),
                                        (long long)pick_int() * 64, nullptr);
                break;
            default:
                st = lix_topk_bf16(pick_ptr(), pick_int(), pick_int(), pick_int(), pick_int(), pick_ptr(),
                                   (int32_t*)pick_ptr(), nullptr);
                (void)lix_topk_fused_supported(pick_int(), pick_int(), pick_int(), pick_int());
                break;
        }
        ++g_calls;
        if (!documented(st) || st == LIX_OK || st == LIX_ERR_LAUNCH) {
            std::fprintf(stderr, "sweep call %d returned %d\n", it, st);
            ++g_failures;
        }
    }
    std::printf("abi_driver: %ld calls, %d failures\n", g_calls, g_failures);
    return g_failures == 0 ? 0 : 1;
}
