// C ABI of the attention library (declared in include/fa.h).
//
// Every entry point validates its arguments on the host before any HIP call,
// so invalid calls return an error code without touching device state.  The
// library never allocates, frees or synchronises; launches go to the caller's
// stream.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int check_shape(int B, int H, int N, int d, float scale) {
    if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    // per-lane byte offsets within one batch's [N, H, d] rows stay below 2^31:
    // N * H * d < 2^30, tested as N * H < 2^30 / d (d divides 2^30), so no
    // product can overflow (N, H < 2^31, so N * H < 2^62)
    if ((long long)N * H >= (1LL << 30) / d) return FA_ERR_UNSUPPORTED;
    // grid size: B * H * ceil(N / 64) workgroups must fit a 32-bit grid
    // (H * ceil(N / 64) < 2^24 after the test above, so this fits 64 bits)
    if ((long long)B * H * ((N + 63) / 64) >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

// grouped-query attention: H_kv K/V heads, each shared by H / H_kv query heads
int check_groups(int H, int H_kv) {
    if (H_kv < 1 || H_kv > H || H % H_kv != 0) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

int fwd_common(const void* q, const void* k, const void* v, const void* o, const void* lse, int B,
               int H, int N, int d, float scale) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    const int rc = check_shape(B, H, N, d, scale);
    if (rc != FA_OK) return rc;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_MISALIGNED;
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, hipStream_t stream) {
    return fa_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, scale, causal, stream);
}

namespace {
// window > 0: causal sliding window; 0: none
int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
             int N, int d, float scale, int causal, int window, hipStream_t stream) {
    int rc = fwd_common(q, k, v, o, lse, B, H, N, d, scale);
    if (rc != FA_OK) return rc;
    if ((rc = check_groups(H, H_kv)) != FA_OK) return rc;
    if (fa::launch_fwd_bf16(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal != 0, window, stream) !=
        hipSuccess)
        return FA_ERR_LAUNCH;
    return FA_OK;
}
}  // namespace

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
               int N, int d, float scale, int causal, hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, 0, stream);
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int H_kv, int N, int d, float scale, int window, hipStream_t stream) {
    if (window < 1) return FA_ERR_INVALID_ARG;
    return fwd_impl(q, k, v, o, lse, B, H, H_kv, N, d, scale, 1, window, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
               const float* k_descale, const float* v_descale, void* o, float* lse, int B, int H,
               int H_kv, int N, int d, float scale, int causal, int window, hipStream_t stream) {
    int rc = fwd_common(q, k, v, o, lse, B, H, N, d, scale);
    if (rc != FA_OK) return rc;
    if ((rc = check_groups(H, H_kv)) != FA_OK) return rc;
    if (!q_descale || !k_descale || !v_descale) return FA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(q_descale) | reinterpret_cast<uintptr_t>(k_descale) |
         reinterpret_cast<uintptr_t>(v_descale)) & 3u)
        return FA_ERR_MISALIGNED;
    if (window < 0 || (window > 0 && !causal)) return FA_ERR_INVALID_ARG;
    if (fa::launch_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse, B, H, H_kv, N, d, scale,
                           causal != 0, window, stream) != hipSuccess)
        return FA_ERR_LAUNCH;
    return FA_OK;
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, hipStream_t stream) {
    const int rc = fwd_common(q, k, v, o, lse, B, H, N, d, scale);
    if (rc != FA_OK) return rc;
    if (fa::launch_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal != 0, stream) != hipSuccess)
        return FA_ERR_LAUNCH;
    return FA_OK;
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
    if (check_shape(B, H, N, d, 1.0f) != FA_OK) return 0;
    const size_t stat_rows = (size_t)B * H * fa::bwd_rows_padded(N);
    return 2 * align256(stat_rows * sizeof(float));
}

namespace {
struct Workspace {
    float* lse2;     // LSE * log2(e), [B, H, Npad] (padding +inf)
    float* delta;    // -D, D = rowsum(dO * O), [B, H, Npad] (padding 0)
};

int check_workspace(void* workspace, size_t workspace_bytes, int B, int H, int N, int d, Workspace* ws) {
    const size_t need = fa_bwd_workspace_size(B, H, N, d);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < need)
        return FA_ERR_WORKSPACE;
    const size_t stat = align256((size_t)B * H * fa::bwd_rows_padded(N) * sizeof(float));
    char* w = static_cast<char*>(workspace);
    ws->lse2 = reinterpret_cast<float*>(w);
    ws->delta = reinterpret_cast<float*>(w + stat);
    return FA_OK;
}

int all_aligned(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (!p) return FA_ERR_INVALID_ARG;
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_MISALIGNED;
    return FA_OK;
}

// the key-block kernel addresses the row statistics with 32-bit byte offsets
int check_bwd_shape(int B, int H, int N, int d, float scale) {
    const int rc = check_shape(B, H, N, d, scale);
    if (rc != FA_OK) return rc;
    if ((long long)B * H * fa::bwd_rows_padded(N) >= (1LL << 28)) return FA_ERR_UNSUPPORTED;
    // byte offsets of rows up to N + 255 (tiles overhanging the last row,
    // which read zeros through a range-checked load) must not wrap 32 bits
    if ((long long)(N + 256) * H * d * 2 >= (1LL << 32)) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}
}  // namespace

int fa_bwd_preprocess(const void* o, const void* dout, const float* lse, int B, int H, int N, int d,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = all_aligned({o, dout, lse});
    if (rc != FA_OK) return rc;
    if ((rc = check_bwd_shape(B, H, N, d, 1.0f)) != FA_OK) return rc;
    Workspace ws;
    if ((rc = check_workspace(workspace, workspace_bytes, B, H, N, d, &ws)) != FA_OK) return rc;
    if (fa::launch_bwd_preprocess(o, dout, lse, B, H, N, d, ws.lse2, ws.delta, stream) != hipSuccess)
        return FA_ERR_LAUNCH;
    return FA_OK;
}

namespace {
int bwd_dkdv_impl(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                  int B, int H, int H_kv, int N, int d, float scale, int causal, int window,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = all_aligned({q, k, v, dout, dk, dv});
    if (rc != FA_OK) return rc;
    if ((rc = check_bwd_shape(B, H, N, d, scale)) != FA_OK) return rc;
    if ((rc = check_groups(H, H_kv)) != FA_OK) return rc;
    Workspace ws;
    if ((rc = check_workspace(workspace, workspace_bytes, B, H, N, d, &ws)) != FA_OK) return rc;
    if (fa::launch_bwd_dkdv(q, k, v, dout, dk, dv, B, H, H_kv, N, d, scale, causal != 0, window, ws.lse2,
                            ws.delta, stream) != hipSuccess)
        return FA_ERR_LAUNCH;
    return FA_OK;
}

// o and lse null: the statistics come from the workspace (fa_bwd_preprocess);
// otherwise the kernel forms them and writes them there
int bwd_dq_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, int B, int H, int H_kv, int N, int d, float scale, int causal,
                int window, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = all_aligned({q, k, v, dout, dq});
    if (rc != FA_OK) return rc;
    if (o && (rc = all_aligned({o, lse})) != FA_OK) return rc;
    if ((rc = check_bwd_shape(B, H, N, d, scale)) != FA_OK) return rc;
    if ((rc = check_groups(H, H_kv)) != FA_OK) return rc;
    Workspace ws;
    if ((rc = check_workspace(workspace, workspace_bytes, B, H, N, d, &ws)) != FA_OK) return rc;
    if (fa::launch_bwd_dq(q, k, v, dout, dq, B, H, H_kv, N, d, scale, causal != 0, window, o, lse, ws.lse2,
                          ws.delta, stream) != hipSuccess)
        return FA_ERR_LAUNCH;
    return FA_OK;
}
}  // namespace

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv, int B,
                int H, int N, int d, float scale, int causal, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
    return bwd_dkdv_impl(q, k, v, dout, dk, dv, B, H, H, N, d, scale, causal, 0, workspace,
                         workspace_bytes, stream);
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq, int B, int H,
              int N, int d, float scale, int causal, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
    return bwd_dq_impl(q, k, v, nullptr, dout, nullptr, dq, B, H, H, N, d, scale, causal, 0, workspace,
                       workspace_bytes, stream);
}

int fa_bwd_dq_stats(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, int B, int H, int N, int d, float scale, int causal,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!o || !lse) return FA_ERR_INVALID_ARG;
    return bwd_dq_impl(q, k, v, o, dout, lse, dq, B, H, H, N, d, scale, causal, 0, workspace,
                       workspace_bytes, stream);
}

namespace {
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d,
             float scale, int causal, int window, void* workspace, size_t workspace_bytes,
             hipStream_t stream) {
    // validate everything before the first launch
    int rc = all_aligned({q, k, v, o, dout, lse, dq, dk, dv});
    if (rc != FA_OK) return rc;
    if ((rc = check_bwd_shape(B, H, N, d, scale)) != FA_OK) return rc;
    if ((rc = check_groups(H, H_kv)) != FA_OK) return rc;
    Workspace ws;
    if ((rc = check_workspace(workspace, workspace_bytes, B, H, N, d, &ws)) != FA_OK) return rc;
    // dQ first: it forms the row statistics and leaves them in the workspace
    // for the key-block kernel
    if ((rc = bwd_dq_impl(q, k, v, o, dout, lse, dq, B, H, H_kv, N, d, scale, causal, window, workspace,
                          workspace_bytes, stream)) != FA_OK)
        return rc;
    return bwd_dkdv_impl(q, k, v, dout, dk, dv, B, H, H_kv, N, d, scale, causal, window, workspace,
                         workspace_bytes, stream);
}
}  // namespace

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d,
               float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale, causal, 0, workspace,
                    workspace_bytes, stream);
}

int fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d,
                  float scale, int window, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (window < 1) return FA_ERR_INVALID_ARG;
    return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale, 1, window, workspace,
                    workspace_bytes, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
           int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, scale, causal, workspace,
                      workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free backward: the workspace is a static device array.
//
// Each GPU that runs this library holds its own copy of `scratch` from the
// moment the code object is loaded until the process ends.  In host code the
// array's name is only a host-side stand-in, so its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and only
// that address is handed to kernels.  Every call on one GPU shares the array:
// calls that overlap on one GPU (different streams, or threads) race.
// Nothing in it needs clearing: the first backward step writes every row
// statistic (padding included) before the second reads them.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on device `dev` (which must be current).
int scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_LAUNCH;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return FA_OK;
}
}  // namespace

extern "C" {

size_t fa_bwd_noalloc_max_workspace(void) { return kScratchBytes; }

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                   int causal, hipStream_t stream) {
    // the same checks as fa_bwd, before any HIP call
    int rc = all_aligned({q, k, v, o, dout, lse, dq, dk, dv});
    if (rc != FA_OK) return rc;
    if ((rc = check_bwd_shape(B, H, N, d, scale)) != FA_OK) return rc;
    if (fa_bwd_workspace_size(B, H, N, d) > kScratchBytes) return FA_ERR_SCRATCH;
    // the stream's device must be the current one: the scratch address is
    // looked up for the current device
    int cur = 0, sdev = 0;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess)
        return FA_ERR_LAUNCH;
    if (sdev != cur) return FA_ERR_INVALID_ARG;
    void* ws = nullptr;
    if ((rc = scratch_address(cur, &ws)) != FA_OK) return rc;
    return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, scale, causal, 0, ws, kScratchBytes,
                    stream);
}

int fa_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o, float* lse,
             int B, int H, int N, int d, hipStream_t stream) {
    if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse) return FA_ERR_INVALID_ARG;
    const int rc = check_shape(B, H, N, d, 1.0f);
    if (rc != FA_OK) return rc;
    // one thread per 8 features: the grid must fit 32 bits
    if ((long long)B * H * N * (d / 8) / 256 >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
    for (const void* p : {o_a, (const void*)lse_a, o_b, (const void*)lse_b, (const void*)o, (const void*)lse})
        if (!aligned16(p)) return FA_ERR_MISALIGNED;
    if (fa::launch_merge(o_a, lse_a, o_b, lse_b, o, lse, B, H, N, d, stream) != hipSuccess) return FA_ERR_LAUNCH;
    return FA_OK;
}

int fa_calibrate_mfma(float* out, int n_workgroups, int waves_per_workgroup, int iters, int mode,
                      hipStream_t stream) {
    if (!out || n_workgroups < 1 || waves_per_workgroup < 1 || waves_per_workgroup > 4 || iters < 1)
        return FA_ERR_INVALID_ARG;
    // one checksum per thread at a 32-bit index
    if (n_workgroups > (1 << 22)) return FA_ERR_UNSUPPORTED;
    if (mode < 0 || mode > 7) return FA_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(out) & 3u) return FA_ERR_MISALIGNED;
    if (fa::launch_calib_mfma(out, n_workgroups, waves_per_workgroup, iters, mode, stream) !=
        hipSuccess)
        return FA_ERR_LAUNCH;
    return FA_OK;
}

int fa_probe_mfma(int fp8, const void* a, const void* b, float* c, int n_tiles, int k, hipStream_t stream) {
    if (!a || !b || !c || n_tiles < 1 || k < 1 || (fp8 != 0 && fp8 != 1)) return FA_ERR_INVALID_ARG;
    if (k % (fp8 ? 64 : 16) != 0) return FA_ERR_INVALID_ARG;
    // A and B hold n_tiles * 32 * k elements at 32-bit offsets; the row
    // bytes are bounded first, so the total cannot overflow 64 bits
    const long long row = 32LL * k * (fp8 ? 1 : 2);
    if (row >= (1LL << 31) || n_tiles * row >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
    if (!aligned16(a) || !aligned16(b) || (reinterpret_cast<uintptr_t>(c) & 3u)) return FA_ERR_MISALIGNED;
    if (fa::launch_probe_mfma(fp8, a, b, c, n_tiles, k, stream) != hipSuccess) return FA_ERR_LAUNCH;
    return FA_OK;
}

const char* fa_strerror(int code) {
    switch (code) {
        case FA_OK: return "success";
        case FA_ERR_INVALID_ARG: return "invalid argument (null pointer, B/H/N < 1, non-finite scale, or H_kv not dividing H)";
        case FA_ERR_UNSUPPORTED: return "unsupported shape (d must be 64 or 128, N*H*d < 2^30)";
        case FA_ERR_MISALIGNED: return "pointer not 16-byte aligned";
        case FA_ERR_WORKSPACE: return "workspace null, not 256-byte aligned or smaller than fa_bwd_workspace_size()";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_SCRATCH: return "shape needs more workspace than fa_bwd_noalloc's static scratch holds";
        default: return "unknown error code";
    }
}

}  // extern "C"
