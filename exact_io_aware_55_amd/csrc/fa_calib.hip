// Matrix-core calibration kernel for the roofline harness.
//
// Every wave runs `iters` rounds of eight independent chains of
// v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic inside the
// loop), so the matrix cores are busy for as long as the dependency rules
// allow.  Its measured rate is the sustainable dense bf16 rate of the chip
// under this clock and power; its MFMA-busy counter reading checks the
// normalisation used for the attention kernels (busy cycles over
// GRBM_GUI_ACTIVE x SIMDs).  Optionally each MFMA is accompanied by
// `valu` vector instructions of the kind the online softmax issues (an FMA
// and an exp2, alternately), to measure what such work costs beside the
// products.  The result checksum is written so the compiler keeps the work.
#include "fa_common.h"

namespace fa {

template <int VALU>
__global__ __launch_bounds__(256) void calib_mfma_kernel(float* __restrict__ out, int iters) {
    constexpr int CH = 8;                      // independent accumulator chains
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
        b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
    }
    f32x16 acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = f32x16{};
    // VALU work: independent registers, so the vector instructions need not
    // wait for one another (as the softmax's per-score instructions do not)
    float xv[VALU > 0 ? VALU : 1];
#pragma unroll
    for (int v = 0; v < (VALU > 0 ? VALU : 1); ++v) xv[v] = 0.25f * (float)(lane + v);
#pragma clang loop unroll(disable)
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            acc[c] = mfma32x32x16(a, b, acc[c]);
#pragma unroll
            for (int v = 0; v < VALU; ++v)
                xv[v] = (v & 1) ? fast_exp2(-xv[v]) : __builtin_fmaf(xv[v], 0.999f, 0.001f);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < (VALU > 0 ? VALU : 1); ++v) s += xv[v];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

hipError_t launch_calib_mfma(float* out, int n_workgroups, int waves, int iters, int valu,
                             hipStream_t stream) {
    const dim3 grid((unsigned)n_workgroups), block((unsigned)(64 * waves));
    switch (valu) {
        case 0: hipLaunchKernelGGL(calib_mfma_kernel<0>, grid, block, 0, stream, out, iters); break;
        case 2: hipLaunchKernelGGL(calib_mfma_kernel<2>, grid, block, 0, stream, out, iters); break;
        case 4: hipLaunchKernelGGL(calib_mfma_kernel<4>, grid, block, 0, stream, out, iters); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fa
