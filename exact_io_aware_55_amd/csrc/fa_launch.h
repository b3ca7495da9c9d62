// Host-side launchers of the attention kernels (called by the C ABI layer
// after argument validation).  Each enqueues on `stream` and returns the
// launch status.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int N, int d, float scale, bool causal, hipStream_t stream);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                          int H, int N, int d, float scale, bool causal, hipStream_t stream);

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                           int H, int N, int d, float scale, bool causal, float* delta,
                           float* dq_acc, hipStream_t stream);

}  // namespace fa
