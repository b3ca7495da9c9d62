// Matrix-core calibration kernel for the roofline harness.
//
// Every wave runs `iters` rounds of eight independent chains of
// v_mfma_f32_32x32x16_bf16 (no global memory traffic inside the loop), so
// the matrix cores are busy for as long as the dependency rules allow.  Its
// rate and MFMA-busy counter give the sustainable dense bf16 rate of the chip
// and check the normalisation used for the attention kernels (busy cycles
// over GRBM_GUI_ACTIVE x SIMDs).  Modes:
//   0  register operands that never change (the multipliers barely toggle);
//   1  random register operands: eight different A and eight different B
//      tiles per wave, paired differently by consecutive MFMAs, as in real data;
//   2  mode 1 plus one FMA and one exp2 per MFMA (independent registers, as
//      the online softmax issues them);
//   3  mode 1 plus two FMAs and two exp2 per MFMA;
//   4  mode 1 with the A operand read from LDS by one ds_read_b128 per MFMA
//      (1 KB per wave), eight reads in flight, as the attention kernels read
//      their K/V or Q/dO operands.
// A checksum per thread is written so the compiler keeps the work.
#include "fa_common.h"

namespace fa {

namespace {
constexpr int CH = 8;                          // independent accumulator chains

__device__ __forceinline__ void random_tiles(bf16x8* a, bf16x8* b) {
    unsigned h = 2166136261u ^ (unsigned)(blockIdx.x * 977u + threadIdx.x * 131u);
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            h = h * 16777619u + 0x9e3779b9u;
            h ^= h >> 13;
            a[c][e] = (__bf16)(((float)(h & 0xffffu) - 32768.f) * (1.f / 16384.f));
            h = h * 16777619u + 0x7f4a7c15u;
            h ^= h >> 11;
            b[c][e] = (__bf16)(((float)(h & 0xffffu) - 32768.f) * (1.f / 16384.f));
        }
}

__device__ __forceinline__ float checksum(const f32x16* acc, float s) {
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    return s;
}
}  // namespace

// modes 0 - 3: register operands, VALU vector instructions per MFMA
template <bool RANDOM, int VALU>
__global__ __launch_bounds__(256) void calib_mfma_kernel(float* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a[CH], b[CH];
    if constexpr (RANDOM) {
        random_tiles(a, b);
    } else {
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                a[c][e] = (__bf16)(0.001f * (float)((lane + e) & 7));
                b[c][e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
            }
    }
    f32x16 acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = f32x16{};
    // vector work on independent registers, so the instructions need not
    // wait for one another (as the softmax's per-score instructions do not)
    float xv[VALU > 0 ? VALU : 1];
#pragma unroll
    for (int v = 0; v < (VALU > 0 ? VALU : 1); ++v) xv[v] = 0.25f * (float)(lane + v);
#pragma clang loop unroll(disable)
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                // constant mode: the same tiles every time; random mode: a
                // different pairing of the eight tiles in consecutive MFMAs
                acc[c] = RANDOM ? mfma32x32x16(a[c], b[(c + 3 + 2 * half) & (CH - 1)], acc[c])
                                : mfma32x32x16(a[0], b[0], acc[c]);
#pragma unroll
                for (int v = 0; v < VALU; ++v)
                    xv[v] = (v & 1) ? fast_exp2(-xv[v]) : __builtin_fmaf(xv[v], 0.999f, 0.001f);
            }
    }
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < (VALU > 0 ? VALU : 1); ++v) s += xv[v];
    out[blockIdx.x * blockDim.x + threadIdx.x] = checksum(acc, s);
}

// mode 4: random B operands in registers, A operands read from LDS
__global__ __launch_bounds__(256) void calib_mfma_lds_kernel(float* __restrict__ out, int iters) {
    __shared__ __attribute__((aligned(16))) char lds[4 * CH * 1024];   // 8 KB per wave
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    bf16x8 a[CH], b[CH];
    random_tiles(a, b);
    // each wave's LDS holds its eight random A tiles (1 KB each)
#pragma unroll
    for (int c = 0; c < CH; ++c)
        *reinterpret_cast<bf16x8*>(lds + wave * CH * 1024 + c * 1024 + lane * 16) = a[c];
    __syncthreads();
    const lds_char* base = as_lds(lds) + wave * CH * 1024 + lane * 16;
    f32x16 acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = f32x16{};
    bf16x8 op[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) op[c] = lds_read_b128(base + c * 1024);
#pragma clang loop unroll(disable)
    for (int it = 0; it < 2 * iters; ++it) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bf16x8 cur = op[c];
            op[c] = lds_read_b128(base + ((c + it + 1) & (CH - 1)) * 1024);
            acc[c] = mfma32x32x16(cur, b[(c + 3) & (CH - 1)], acc[c]);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) s += (float)op[c][c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = checksum(acc, s);
}

hipError_t launch_calib_mfma(float* out, int n_workgroups, int waves, int iters, int mode,
                             hipStream_t stream) {
    const dim3 grid((unsigned)n_workgroups), block((unsigned)(64 * waves));
    switch (mode) {
        case 0: hipLaunchKernelGGL((calib_mfma_kernel<false, 0>), grid, block, 0, stream, out, iters); break;
        case 1: hipLaunchKernelGGL((calib_mfma_kernel<true, 0>), grid, block, 0, stream, out, iters); break;
        case 2: hipLaunchKernelGGL((calib_mfma_kernel<true, 2>), grid, block, 0, stream, out, iters); break;
        case 3: hipLaunchKernelGGL((calib_mfma_kernel<true, 4>), grid, block, 0, stream, out, iters); break;
        case 4: hipLaunchKernelGGL(calib_mfma_lds_kernel, grid, block, 0, stream, out, iters); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fa
