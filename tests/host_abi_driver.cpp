// Host driver for the AddressSanitizer run of the C ABI (tests/test_host_asan.py).
//
// Linked against an ASan-instrumented host build of every csrc/*.hip, it calls
// each entry point of include/fa.h with arguments the library must reject
// before any HIP call (null and misaligned pointers, bad shapes, short
// workspaces, bad group or window sizes, out-of-range calibration and probe
// arguments), checks the returned code, and reads every error string.  No
// GPU is touched.  ASan aborts the run on any invalid host memory access in
// the validation, size arithmetic or error-string code.
//
// "--selftest-overflow" reads one element past a heap array instead, so the
// test can show that the sanitizer is live in this build.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fa.h"

namespace {

int failures = 0;

void expect(const char* what, int got, int want) {
    if (got != want) {
        std::printf("FAIL %s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(uintptr_t{0x10000} + off); }

}  // namespace

int main(int argc, char** argv) {
    if (argc > 1 && std::strcmp(argv[1], "--selftest-overflow") == 0) {
        std::vector<int> v(8, 1);
        volatile int* p = v.data();
        return p[8];                                        // one past the end
    }
    void* F = fake();
    const float nan = std::nanf(""), inf = INFINITY;

    // forward (bf16 and fp32): each null pointer, shapes, scale, d, size limit, alignment
    for (int fp32 = 0; fp32 < 2; ++fp32) {
        auto fwd = [&](void* q, void* k, void* v, void* o, void* l, int B, int H, int N, int d, float sc) {
            return fp32 ? fa_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)o, (float*)l,
                                     B, H, N, d, sc, 0, nullptr)
                        : fa_fwd(q, k, v, o, (float*)l, B, H, N, d, sc, 0, nullptr);
        };
        for (int i = 0; i < 5; ++i) {
            void* p[5] = {F, F, F, F, F};
            p[i] = nullptr;
            expect("fwd null", fwd(p[0], p[1], p[2], p[3], p[4], 1, 1, 8, 64, 0.1f), FA_ERR_INVALID_ARG);
            p[i] = fake(8);
            expect("fwd misaligned", fwd(p[0], p[1], p[2], p[3], p[4], 1, 1, 8, 64, 0.1f), FA_ERR_MISALIGNED);
        }
        expect("fwd B", fwd(F, F, F, F, F, 0, 1, 8, 64, 0.1f), FA_ERR_INVALID_ARG);
        expect("fwd H", fwd(F, F, F, F, F, 1, -1, 8, 64, 0.1f), FA_ERR_INVALID_ARG);
        expect("fwd N", fwd(F, F, F, F, F, 1, 1, 0, 64, 0.1f), FA_ERR_INVALID_ARG);
        expect("fwd nan", fwd(F, F, F, F, F, 1, 1, 8, 64, nan), FA_ERR_INVALID_ARG);
        expect("fwd inf", fwd(F, F, F, F, F, 1, 1, 8, 64, inf), FA_ERR_INVALID_ARG);
        for (int d : {0, 32, 96, 256}) expect("fwd d", fwd(F, F, F, F, F, 1, 1, 8, d, 0.1f), FA_ERR_UNSUPPORTED);
        expect("fwd size", fwd(F, F, F, F, F, 1, 8, 1 << 20, 128, 0.1f), FA_ERR_UNSUPPORTED);
        expect("fwd size INT_MAX", fwd(F, F, F, F, F, 1 << 30, 1 << 30, 1 << 30, 128, 0.1f), FA_ERR_UNSUPPORTED);
    }

    // backward and its workspace
    const size_t need = fa_bwd_workspace_size(1, 1, 8, 64);
    expect("workspace size", (int)(need == 512), 1);
    expect("workspace size bad", (int)fa_bwd_workspace_size(0, 1, 8, 64), 0);
    expect("workspace size huge", (int)(fa_bwd_workspace_size(1 << 30, 1 << 30, 1 << 30, 64) == 0), 1);
    auto bwd = [&](void* const* p, int B, int d, float sc, void* ws, size_t wsb) {
        return fa_bwd(p[0], p[1], p[2], p[3], p[4], (const float*)p[5], p[6], p[7], p[8], B, 1, 8, d, sc, 1, ws,
                      wsb, nullptr);
    };
    for (int i = 0; i < 9; ++i) {
        void* p[9] = {F, F, F, F, F, F, F, F, F};
        p[i] = nullptr;
        expect("bwd null", bwd(p, 1, 64, 0.1f, F, 1 << 20), FA_ERR_INVALID_ARG);
        p[i] = fake(4);
        expect("bwd misaligned", bwd(p, 1, 64, 0.1f, F, 1 << 20), FA_ERR_MISALIGNED);
    }
    void* ok9[9] = {F, F, F, F, F, F, F, F, F};
    expect("bwd B", bwd(ok9, 0, 64, 0.1f, F, 1 << 20), FA_ERR_INVALID_ARG);
    expect("bwd nan", bwd(ok9, 1, 64, nan, F, 1 << 20), FA_ERR_INVALID_ARG);
    expect("bwd d", bwd(ok9, 1, 100, 0.1f, F, 1 << 20), FA_ERR_UNSUPPORTED);
    expect("bwd ws null", bwd(ok9, 1, 64, 0.1f, nullptr, 1 << 20), FA_ERR_WORKSPACE);
    expect("bwd ws misaligned", bwd(ok9, 1, 64, 0.1f, fake(16), 1 << 20), FA_ERR_WORKSPACE);
    expect("bwd ws short", bwd(ok9, 1, 64, 0.1f, F, need - 1), FA_ERR_WORKSPACE);

    // the backward's separate steps
    expect("pre null", fa_bwd_preprocess(nullptr, F, (const float*)F, 1, 1, 8, 64, F, 1 << 20, nullptr),
           FA_ERR_INVALID_ARG);
    expect("pre ws", fa_bwd_preprocess(F, F, (const float*)F, 1, 1, 8, 64, F, 16, nullptr), FA_ERR_WORKSPACE);
    expect("pre size", fa_bwd_preprocess(F, F, (const float*)F, 1 << 12, 1 << 8, 1 << 9, 64, F, 1 << 20, nullptr),
           FA_ERR_UNSUPPORTED);
    expect("dkdv scale", fa_bwd_dkdv(F, F, F, F, F, F, 1, 1, 8, 64, inf, 0, F, 1 << 20, nullptr),
           FA_ERR_INVALID_ARG);
    expect("dkdv rows", fa_bwd_dkdv(F, F, F, F, F, F, 1, 1 << 16, 1, 128, 0.1f, 0, F, 1 << 30, nullptr),
           FA_ERR_UNSUPPORTED);
    expect("dq ws", fa_bwd_dq(F, F, F, F, F, 1, 1, 8, 64, 0.1f, 0, fake(128), 1 << 20, nullptr), FA_ERR_WORKSPACE);
    expect("dq d", fa_bwd_dq(F, F, F, F, F, 1, 1, 8, 32, 0.1f, 0, F, 1 << 20, nullptr), FA_ERR_UNSUPPORTED);
    for (int i = 0; i < 7; ++i) {
        void* p[7] = {F, F, F, F, F, F, F};
        p[i] = nullptr;
        expect("dq_stats null",
               fa_bwd_dq_stats(p[0], p[1], p[2], p[3], p[4], (const float*)p[5], p[6], 1, 1, 8, 64, 0.1f, 0, F,
                               1 << 20, nullptr),
               FA_ERR_INVALID_ARG);
    }

    // grouped-query attention and sliding windows
    for (int hkv : {0, -1, 4, 7})
        expect("gqa hkv", fa_fwd_gqa(F, F, F, F, (float*)F, 1, 6, hkv, 8, 64, 0.1f, 0, nullptr),
               FA_ERR_INVALID_ARG);
    expect("gqa ws", fa_bwd_gqa(F, F, F, F, F, (const float*)F, F, F, F, 1, 6, 2, 8, 64, 0.1f, 0, F,
                                fa_bwd_workspace_size(1, 6, 8, 64) - 1, nullptr),
           FA_ERR_WORKSPACE);
    for (int w : {0, -3})
        expect("window", fa_fwd_window(F, F, F, F, (float*)F, 1, 4, 2, 8, 64, 0.1f, w, nullptr), FA_ERR_INVALID_ARG);
    expect("window bwd ws", fa_bwd_window(F, F, F, F, F, (const float*)F, F, F, F, 1, 4, 2, 8, 64, 0.1f, 3, F,
                                          fa_bwd_workspace_size(1, 4, 8, 64) - 1, nullptr),
           FA_ERR_WORKSPACE);

    // FP8 forward: descales need 4-byte alignment, the rest 16
    for (int i = 0; i < 8; ++i) {
        void* p[8] = {F, F, F, F, F, F, F, F};
        p[i] = nullptr;
        auto call = [&]() {
            return fa_fwd_fp8(p[0], p[1], p[2], (const float*)p[3], (const float*)p[4], (const float*)p[5], p[6],
                              (float*)p[7], 1, 4, 2, 8, 64, 0.1f, 0, 0, nullptr);
        };
        expect("fp8 null", call(), FA_ERR_INVALID_ARG);
        p[i] = fake(i >= 3 && i <= 5 ? 2 : 8);
        expect("fp8 misaligned", call(), FA_ERR_MISALIGNED);
    }
    expect("fp8 window", fa_fwd_fp8(F, F, F, (const float*)F, (const float*)F, (const float*)F, F, (float*)F, 1, 4,
                                    2, 8, 64, 0.1f, 0, 4, nullptr),
           FA_ERR_INVALID_ARG);

    // the entry point that allocates nothing: shapes past its static scratch
    expect("noalloc scratch",
           fa_bwd_noalloc(F, F, F, F, F, (const float*)F, F, F, F, 64, 64, 1 << 14, 64, 0.1f, 0, nullptr),
           FA_ERR_SCRATCH);
    expect("noalloc max", (int)(fa_bwd_noalloc_max_workspace() == (size_t{16} << 20)), 1);

    // merge of two results over disjoint key ranges
    for (int i = 0; i < 6; ++i) {
        void* p[6] = {F, F, F, F, F, F};
        p[i] = nullptr;
        auto call = [&](int B, int N, int d) {
            return fa_merge(p[0], (const float*)p[1], p[2], (const float*)p[3], p[4], (float*)p[5], B, 2, N, d,
                            nullptr);
        };
        expect("merge null", call(1, 8, 64), FA_ERR_INVALID_ARG);
        p[i] = fake(4);
        expect("merge misaligned", call(1, 8, 64), FA_ERR_MISALIGNED);
        p[i] = F;
        expect("merge d", call(1, 8, 96), FA_ERR_UNSUPPORTED);
        expect("merge size INT_MAX", call(1 << 30, 1 << 30, 128), FA_ERR_UNSUPPORTED);
    }

    // calibration and probe
    expect("calib null", fa_calibrate_mfma(nullptr, 4, 4, 10, 0, nullptr), FA_ERR_INVALID_ARG);
    expect("calib mode", fa_calibrate_mfma((float*)F, 4, 4, 10, 8, nullptr), FA_ERR_INVALID_ARG);
    expect("calib misaligned", fa_calibrate_mfma((float*)fake(2), 4, 4, 10, 0, nullptr), FA_ERR_MISALIGNED);
    expect("probe k", fa_probe_mfma(0, F, F, (float*)F, 1, 24, nullptr), FA_ERR_INVALID_ARG);
    expect("probe size", fa_probe_mfma(1, F, F, (float*)F, 1 << 16, 1 << 16, nullptr), FA_ERR_UNSUPPORTED);
    expect("probe size wrap", fa_probe_mfma(1, F, F, (float*)F, 1 << 30, 1 << 30, nullptr), FA_ERR_UNSUPPORTED);
    expect("calib grid", fa_calibrate_mfma((float*)F, (1 << 22) + 1, 4, 10, 0, nullptr), FA_ERR_UNSUPPORTED);

    // every error string, and an unknown code
    size_t total = 0;
    for (int code = -7; code <= 1; ++code) total += std::strlen(fa_strerror(code));
    expect("strerror", (int)(total > 0), 1);

    if (failures) return 1;
    std::printf("OK\n");
    return 0;
}
