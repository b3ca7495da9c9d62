// Host-side launchers of the attention kernels (called by the C ABI layer
// after argument validation).  Each enqueues on `stream` and returns the
// launch status.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Hkv: K/V heads (H for multi-head attention; H a multiple of Hkv).  Query
// head h uses K/V head h / (H / Hkv).  window (causal only): query i sees keys
// j with i - window < j <= i; window <= 0 means no window.
constexpr int kNoWindow = 1 << 30;
// The window the kernels see.  A window of N or more hides no key, so it is
// plain causal attention; it becomes kNoWindow, which keeps the kernels'
// 32-bit window arithmetic (row + window, row - window) far from overflow
// for any caller value up to INT_MAX.
inline int effective_window(int window, int N) { return window > 0 && window < N ? window : kNoWindow; }
// Launch order of a causal grid (order_blocks, odd_generation): `gen` is the
// number of workgroups one XCD runs at once, from the kernel's occupancy and
// the device's CU count, or 0 for no alternating sweeps (sliding windows,
// whose blocks all have about the same range, and heads whose streamed
// operands fit in one XCD's L2); `group` the number of heads an XCD takes
// at a time.  kernel: the kernel's address; threads: its workgroup size; nb:
// its blocks per head; d: head dimension; N: sequence length; window: a
// sliding window narrower than N.  Host only; the occupancy is cached per
// device and kernel.
// Workgroups of `kernel` (with `threads` threads each) one XCD runs at once,
// from its occupancy and the device's CU count (cached per device and
// kernel); 0 if the runtime cannot say.
int xcd_slots(const void* kernel, int threads, hipStream_t stream);
struct Schedule {
    int gen;
    int group;
};
Schedule causal_schedule(const void* kernel, int threads, int nb, int d, int N, bool window,
                         hipStream_t stream);

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int Hkv, int N, int d, float scale, bool causal, int window,
                           hipStream_t stream);

// FP8 forward: Q, K, V are OCP E4M3 codes; q_descale [B*H], k_descale and
// v_descale [B*Hkv] are device fp32 arrays (value = code * descale).
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                          const float* k_descale, const float* v_descale, void* o, float* lse, int B,
                          int H, int Hkv, int N, int d, float scale, bool causal, int window,
                          hipStream_t stream);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                          int H, int N, int d, float scale, bool causal, hipStream_t stream);

// Backward steps: row statistics (padded D and LSE * log2 e); the
// key-block kernel (dK, dV); the query-block kernel (dQ).  Row statistics are
// padded per head to bwd_rows_padded(N) rows.  launch_bwd_dq with o and lse
// (not null) forms the statistics itself and writes them to lse2 / delta;
// with o == nullptr it reads them there.
int bwd_rows_padded(int N);
hipError_t launch_bwd_preprocess(const void* o, const void* dout, const float* lse, int B, int H,
                                 int N, int d, float* lse2, float* delta, hipStream_t stream);
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk,
                           void* dv, int B, int H, int Hkv, int N, int d, float scale, bool causal,
                           int window, const float* lse2, const float* delta, hipStream_t stream);
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
                         int B, int H, int Hkv, int N, int d, float scale, bool causal, int window,
                         const void* o, const float* lse, float* lse2, float* delta, hipStream_t stream);

// Matrix-core calibration: n_workgroups x `waves` waves, each `iters` rounds
// of 16 32x32x16 bf16 MFMAs on 8 independent chains; `mode` 0 - 4 as in
// fa_calibrate_mfma; one checksum per thread into out.
hipError_t launch_calib_mfma(float* out, int n_workgroups, int waves, int iters, int mode,
                             hipStream_t stream);

// Matrix-core probe: C[t] = A[t] B[t]^T for n_tiles 32 x 32 tiles with
// contraction length k, on the bf16 (fp8 = 0) or E4M3 (fp8 = 1) MFMA.
hipError_t launch_probe_mfma(int fp8, const void* a, const void* b, float* c, int n_tiles, int k,
                             hipStream_t stream);

// Merge of two (O, LSE) results over disjoint key ranges (fa_merge).
hipError_t launch_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o,
                        float* lse, int B, int H, int N, int d, hipStream_t stream);

}  // namespace fa
