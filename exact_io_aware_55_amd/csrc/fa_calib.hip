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
//      their K/V or Q/dO operands;
//   5  mode 4 plus three FMAs and one exp2 per MFMA: the forward's mix per
//      MFMA (one score per lane: exponent FMA, exp2, row sum, half a
//      conversion, loop and mask work);
//   6  mode 5 with each LDS read feeding two MFMAs (0.5 KB per MFMA), the
//      mix of a forward whose waves hold 64 queries instead of 32;
//   7  mode 4 plus four FMAs and one exp2 per two MFMAs: the dK/dV kernel's
//      mix per MFMA (2.5 vector instructions, half of one an exp2).
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

// modes 4 - 7: random B operands in registers, A operands read from LDS, one
// read per REUSE MFMAs; NFMA FMAs and NEXP exp2 beside every EVERY-th MFMA
// on independent registers
template <int REUSE, int NFMA, int NEXP, int EVERY = 1>
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
    constexpr int NOP = CH / REUSE;            // reads in flight
    bf16x8 op[NOP];
#pragma unroll
    for (int c = 0; c < NOP; ++c) op[c] = lds_read_b128(base + c * 1024);
    constexpr int NV = NFMA + NEXP > 0 ? NFMA + NEXP : 1;
    float xv[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) xv[v] = 0.25f * (float)(lane + v);
#pragma clang loop unroll(disable)
    for (int it = 0; it < 2 * iters; ++it) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int o = c / REUSE;
            const bf16x8 cur = op[o];
            if (c % REUSE == REUSE - 1) op[o] = lds_read_b128(base + ((o + it + 1) & (CH - 1)) * 1024);
            acc[c] = mfma32x32x16(cur, b[(c + 3) & (CH - 1)], acc[c]);
            if (c % EVERY == 0) {
#pragma unroll
                for (int v = 0; v < NFMA; ++v) xv[v] = __builtin_fmaf(xv[v], 0.999f, 0.001f);
#pragma unroll
                for (int v = 0; v < NEXP; ++v) xv[NFMA + v] = fast_exp2(-xv[NFMA + v]);
            }
        }
    }
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < NFMA + NEXP; ++v) s += xv[v];
#pragma unroll
    for (int c = 0; c < NOP; ++c) s += (float)op[c][c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = checksum(acc, s);
}

// ---------------------------------------------------------------------------
// Matrix-core probe: C = A B^T for independent 32 x 32 tiles on the matrix
// core the attention kernels use, so tests can measure its accumulation
// error against exact products.  One wave per tile: A [tile][32][k] and
// B [tile][32][k] row-major (the contraction index fastest), C [tile][32][32]
// fp32 with C[i][c] = sum_j A[i][j] B[c][j].  FP8 = false: bf16 operands on
// v_mfma_f32_32x32x16_bf16 (k a multiple of 16); true: OCP E4M3 codes on
// v_mfma_f32_32x32x64_f8f6f4 (k a multiple of 64).  Lane l supplies row
// l & 31 of A (column l & 31 of B) and the contraction slots
// KC/2 * (l >> 5) .. + KC/2 - 1 of each KC-long chunk; consecutive chunks
// accumulate in the same fp32 accumulator, as the kernels chain them.
// ---------------------------------------------------------------------------
typedef int i32x8p __attribute__((ext_vector_type(8)));
template <bool FP8>
__global__ __launch_bounds__(256) void probe_mfma_kernel(const char* __restrict__ A, const char* __restrict__ B,
                                                         float* __restrict__ C, int n_tiles, int k) {
    const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tile >= n_tiles) return;
    const int lane = threadIdx.x & 63, l32 = lane & 31, hl = lane >> 5;
    constexpr int EB = FP8 ? 1 : 2;            // bytes per element
    constexpr int KC = FP8 ? 64 : 16;          // contraction per MFMA
    const long row_bytes = (long)k * EB;
    const char* a = A + ((long)tile * 32 + l32) * row_bytes + (KC / 2) * hl * EB;
    const char* b = B + ((long)tile * 32 + l32) * row_bytes + (KC / 2) * hl * EB;
    f32x16 acc = f32x16{};
    for (int c0 = 0; c0 < k; c0 += KC) {
        if constexpr (FP8) {
            const u32x4* pa = reinterpret_cast<const u32x4*>(a + c0);
            const u32x4* pb = reinterpret_cast<const u32x4*>(b + c0);
            const i32x8p va = __builtin_bit_cast(i32x8p, __builtin_shufflevector(pa[0], pa[1], 0, 1, 2, 3, 4, 5, 6, 7));
            const i32x8p vb = __builtin_bit_cast(i32x8p, __builtin_shufflevector(pb[0], pb[1], 0, 1, 2, 3, 4, 5, 6, 7));
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 0, 0, 0, 0, 0, 0);
        } else {
            const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4*>(a + c0 * EB));
            const bf16x8 vb = as_bf16x8(*reinterpret_cast<const u32x4*>(b + c0 * EB));
            acc = mfma32x32x16(va, vb, acc);
        }
    }
    float* dst = C + (long)tile * 32 * 32 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[(8 * (r >> 2) + 4 * hl + (r & 3)) * 32] = acc[r];
}

hipError_t launch_probe_mfma(int fp8, const void* a, const void* b, float* c, int n_tiles, int k,
                             hipStream_t stream) {
    const dim3 grid((unsigned)((n_tiles + 3) / 4)), block(256);
    auto A = static_cast<const char*>(a);
    auto B = static_cast<const char*>(b);
    if (fp8) hipLaunchKernelGGL(probe_mfma_kernel<true>, grid, block, 0, stream, A, B, c, n_tiles, k);
    else hipLaunchKernelGGL(probe_mfma_kernel<false>, grid, block, 0, stream, A, B, c, n_tiles, k);
    return hipGetLastError();
}

hipError_t launch_calib_mfma(float* out, int n_workgroups, int waves, int iters, int mode,
                             hipStream_t stream) {
    const dim3 grid((unsigned)n_workgroups), block((unsigned)(64 * waves));
    switch (mode) {
        case 0: hipLaunchKernelGGL((calib_mfma_kernel<false, 0>), grid, block, 0, stream, out, iters); break;
        case 1: hipLaunchKernelGGL((calib_mfma_kernel<true, 0>), grid, block, 0, stream, out, iters); break;
        case 2: hipLaunchKernelGGL((calib_mfma_kernel<true, 2>), grid, block, 0, stream, out, iters); break;
        case 3: hipLaunchKernelGGL((calib_mfma_kernel<true, 4>), grid, block, 0, stream, out, iters); break;
        case 4: hipLaunchKernelGGL((calib_mfma_lds_kernel<1, 0, 0>), grid, block, 0, stream, out, iters); break;
        case 5: hipLaunchKernelGGL((calib_mfma_lds_kernel<1, 3, 1>), grid, block, 0, stream, out, iters); break;
        case 6: hipLaunchKernelGGL((calib_mfma_lds_kernel<2, 3, 1>), grid, block, 0, stream, out, iters); break;
        case 7: hipLaunchKernelGGL((calib_mfma_lds_kernel<1, 4, 1, 2>), grid, block, 0, stream, out, iters); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fa
