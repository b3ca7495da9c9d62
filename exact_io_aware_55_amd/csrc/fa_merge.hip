// Merge of two attention results over disjoint key ranges of the same
// queries into the result over their union.
//
// The online softmax (explainer page "Flash Attention", section "Tiling";
// glossary page "Flash Attention", section "How it works") rescales a
// partial output by exp(m_old - m_new) when the running maximum grows.  The
// same rescaling, applied once to two finished results (O_a, LSE_a) and
// (O_b, LSE_b), gives with L = log(exp(LSE_a) + exp(LSE_b))
//     O = exp(LSE_a - L) O_a + exp(LSE_b - L) O_b,   LSE = L.
// This is what combines the per-device results when a sequence's keys are
// split across devices, and it lets a caller accumulate in place.
//
// HBM-bound: one thread per 8 features of one query row (16-byte loads of
// both O rows and a 16-byte store), the two row LSEs read by every thread of
// the row.  The rows of one wave are whole (64 is a multiple of d / 8), so an
// in-place LSE store cannot overtake another lane's read of it.
#include <math.h>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {
constexpr int kMergeThreads = 256;
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const __bf16* oa, const float* la, const __bf16* ob,
                                                              const float* lb, __bf16* o, float* lse, int H, int N,
                                                              long rows) {
    constexpr int TPR = D / 8;                 // threads per row
    const long t = (long)blockIdx.x * kMergeThreads + threadIdx.x;
    const long row = t / TPR;                  // [B, N, H] order
    if (row >= rows) return;
    const int part = (int)(t - row * TPR);
    const long bn = row / H;
    const int h = (int)(row - bn * H);
    const long b = bn / N;
    const int n = (int)(bn - b * N);
    const long li = (b * H + h) * N + n;       // [B, H, N]
    const float a = la[li], c = lb[li];
    float wa, wb, l;
    if (isnan(a) || isnan(c)) {
        wa = wb = l = NAN;
    } else {
        const float m = fmaxf(a, c);
        if (m == -INFINITY) {                  // neither range sees a key
            wa = wb = 0.f;
            l = -INFINITY;
        } else {
            const float ea = expf(a - m), eb = expf(c - m);
            const float s = ea + eb;
            wa = ea / s;
            wb = eb / s;
            l = m + logf(s);
        }
    }
    const long e = row * D + part * 8;
    const u32x4 va = ld_global16(oa + e), vb = ld_global16(ob + e);
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float x[2];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
            const float xa = __builtin_bit_cast(float, hlf ? va[w] & 0xffff0000u : va[w] << 16);
            const float xb = __builtin_bit_cast(float, hlf ? vb[w] & 0xffff0000u : vb[w] << 16);
            // a range of weight 0 contributes nothing, whatever its O holds
            x[hlf] = (wa == 0.f ? 0.f : wa * xa) + (wb == 0.f ? 0.f : wb * xb);
        }
        out[w] = pack_bf16x2(x[0], x[1]);
    }
    *reinterpret_cast<u32x4*>(o + e) = out;
    if (part == 0) lse[li] = l;
}

hipError_t launch_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o,
                        float* lse, int B, int H, int N, int d, hipStream_t stream) {
    const long rows = (long)B * N * H;
    const long threads = rows * (d / 8);
    const dim3 grid((unsigned)((threads + kMergeThreads - 1) / kMergeThreads)), block(kMergeThreads);
    auto oa = static_cast<const __bf16*>(o_a);
    auto ob = static_cast<const __bf16*>(o_b);
    auto op = static_cast<__bf16*>(o);
    if (d == 128)
        hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, stream, oa, lse_a, ob, lse_b, op, lse, H, N, rows);
    else
        hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, stream, oa, lse_a, ob, lse_b, op, lse, H, N, rows);
    return hipGetLastError();
}

}  // namespace fa
