// Forward pass of exact attention on gfx950 (bf16 MFMA path and fp32 path).
//
// Method (explainer page "Flash Attention", section "Tiling"; glossary page
// "Flash Attention", section "How it works"): a workgroup owns one block of
// queries, streams the key/value blocks of its head through LDS, keeps a
// running row maximum m and sum l, rescales the partial output by
// exp(m_old - m_new) whenever the maximum grows, divides by l once at the end
// and writes only O and one statistic per row (LSE = m + ln l).
//
// bf16 kernel layout (per workgroup: 4 waves, 128 queries, K/V blocks of 64):
//  * each wave owns 32 queries and keeps them in registers as the B operand of
//    S^T = K Q^T, so a lane holds the scores of ONE query against 16 keys of
//    each 32-key MFMA tile.  The row max/sum are in-lane reductions plus one
//    exchange between the two lane halves.
//  * P^T stays in registers: after exp and the bf16 conversion, registers of
//    the S^T accumulator are directly the B operand of O^T += V^T P^T.
//  * K is staged row-major in LDS (rows padded by 16 B); V is staged
//    transposed (V^T, one row per feature) with keys placed in the k-slot
//    order of the P^T registers and 16-byte chunks XOR-swizzled per row.
//  * K/V blocks are double-buffered in LDS and the next block is prefetched
//    into registers while the current one is multiplied: one barrier per block.
//  * exponentials are v_exp_f32 (base 2) with scale * log2(e) folded into one
//    FMA per score.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace fwd {
constexpr int BR = 128;     // queries per workgroup
constexpr int BC = 64;      // keys per K/V block
constexpr int NT = 256;     // threads per workgroup (4 waves)
}  // namespace fwd

// Maps a linear workgroup id to (head, query block) so that the workgroups the
// hardware places on one XCD (ids congruent mod 8) take a contiguous range of
// query blocks: those share K/V of the same heads and hit the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    const int per = nblocks >> 3, rem = nblocks & 7;
    const int x = bid & 7, i = bid >> 3;
    return x * per + (x < rem ? x : rem) + i;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(fwd::NT) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int H, int N, float scale_log2, int nqb) {
    using namespace fwd;
    constexpr int KP = D * 2 + 16;             // K row pitch (bytes)
    constexpr int K_BYTES = BC * KP;
    constexpr int VT_BYTES = D * BC * 2;       // V^T rows of 64 keys = 128 B
    constexpr int STAGE = K_BYTES + VT_BYTES;
    constexpr int DC = D / 16;                 // k-chunks over the feature dim
    constexpr int DT = D / 32;                 // 32-row tiles of O^T
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int KLD = BC * CPR / NT;         // K chunks loaded per thread
    constexpr int KPT = D / 32;                // keys per thread in the V transpose

    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;

    const int nblocks = gridDim.x;
    const int logical = xcd_remap(blockIdx.x, nblocks);
    const int bh = logical / nqb;
    int qb = logical - bh * nqb;
    if (CAUSAL) qb = nqb - 1 - qb;             // longest rows first
    const int b = bh / H, h = bh - b * H;
    const long row_stride = (long)H * D;       // elements between sequence rows
    const long head_off = ((long)b * N * H + h) * D;
    const __bf16* Qh = Q + head_off;
    const __bf16* Kh = K + head_off;
    const __bf16* Vh = V + head_off;

    const int q0 = qb * BR;
    const int qw = q0 + wave * 32;             // first query of this wave
    const int my_q = qw + l32;

    // Queries of this lane, as B-operand chunks of S^T = K Q^T.
    bf16x8 qreg[DC];
    {
        const bool ok = my_q < N;
        const __bf16* src = Qh + (long)(ok ? my_q : 0) * row_stride + 8 * hl;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            u32x4 v = ok ? ld_global16(src + 16 * c) : u32x4{0, 0, 0, 0};
            qreg[c] = as_bf16x8(v);
        }
    }

    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kv_end + BC - 1) / BC;

    // ---- register staging of one K/V block ----
    u32x4 kst[KLD];
    u32x4 vst[KPT];
    auto load_tile = [&](int t) {
        const int j0 = t * BC;
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int c = tid + NT * i;
            const int r = c / CPR, cc = c % CPR;
            const int key = j0 + r;
            kst[i] = key < N ? ld_global16(Kh + (long)key * row_stride + cc * 8) : u32x4{0, 0, 0, 0};
        }
        const int dblk = tid % CPR, kg = tid / CPR;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int key = j0 + kg * KPT + i;
            vst[i] = key < N ? ld_global16(Vh + (long)key * row_stride + dblk * 8) : u32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&](int buf) {
        char* kb = smem + buf * STAGE;
        char* vb = kb + K_BYTES;
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int c = tid + NT * i;
            const int r = c / CPR, cc = c % CPR;
            st_lds16(kb + r * KP + cc * 16, kst[i]);
        }
        // transpose KPT keys x 8 features into 8 rows of V^T
        const int dblk = tid % CPR, kg = tid / CPR;
        const int pos = kslot_pos(kg * KPT);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = dblk * 8 + e;
            const int w = e >> 1, sh = (e & 1) * 16;
            char* dst = vb + d * 128 + (((pos >> 3) ^ swz8(d)) << 4) + (pos & 7) * 2;
            if constexpr (KPT == 4) {
                const uint32_t a0 = (vst[0][w] >> sh) & 0xffffu, a1 = (vst[1][w] >> sh) & 0xffffu;
                const uint32_t a2 = (vst[2][w] >> sh) & 0xffffu, a3 = (vst[3][w] >> sh) & 0xffffu;
                st_lds8(dst, u32x2{a0 | (a1 << 16), a2 | (a3 << 16)});
            } else {
                const uint32_t a0 = (vst[0][w] >> sh) & 0xffffu, a1 = (vst[1][w] >> sh) & 0xffffu;
                st_lds4(dst, a0 | (a1 << 16));
            }
        }
    };

    f32x16 oacc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;   // running max of scale*log2(e)*s for this lane's query
    float l_run = 0.f;         // running sum over this lane's half of the keys
    const bool pos_scale = scale_log2 >= 0.f;
    const float masked = pos_scale ? -INFINITY : INFINITY;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const bool has_next = t + 1 < ntiles;
        if (has_next) load_tile(t + 1);

        const int j0 = t * BC;
        const bool wave_active = !CAUSAL || j0 <= qw + 31;
        if (wave_active) {
            const char* kb = smem + buf * STAGE;
            const char* vb = kb + K_BYTES;
            // S^T = K Q^T for two 32-key tiles
            f32x16 s[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                s[kt] = f32x16{};
                const char* krow = kb + (kt * 32 + l32) * KP + hl * 16;
#pragma unroll
                for (int c = 0; c < DC; ++c) s[kt] = mfma32x32x16(ld_lds_bf16x8(krow + c * 32), qreg[c], s[kt]);
            }
            // masks: keys past N (ragged tail) and, for causal, keys after the query
            const bool need_mask = (j0 + BC > N) || (CAUSAL && j0 + BC - 1 > qw);
            if (need_mask) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = j0 + kt * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
                        const bool vis = key < N && (!CAUSAL || key <= my_q);
                        s[kt][r] = vis ? s[kt][r] : masked;
                    }
            }
            // block maximum of the scaled scores for this query (both lane halves)
            float mx = s[0][0];
            if (pos_scale) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
            } else {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fminf(mx, s[kt][r]);
            }
            mx = pos_scale ? fmaxf(mx, __shfl_xor(mx, 32)) : fminf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx * scale_log2);
            const float m_sub = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_sub);
            m_run = m_new;
            // P = exp2(s * scale*log2e - m); row sum; pack to bf16 k-chunks
            bf16x8 pb[4];
            float lsum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = fast_exp2(__builtin_fmaf(s[kt][r], scale_log2, -m_sub));
                    // a masked score must give exactly 0, also when scale == 0
                    if (need_mask) p = s[kt][r] == masked ? 0.f : p;
                    lsum += p;
                    pb[kt * 2 + (r >> 3)][r & 7] = (__bf16)p;
                }
            l_run = l_run * alpha + lsum;
#pragma unroll
            for (int i = 0; i < DT; ++i) oacc[i] *= alpha;
            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = dt * 32 + l32;
                const char* vrow = vb + d * 128;
                const int sw = swz8(d);
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
                    oacc[dt] = mfma32x32x16(ld_lds_bf16x8(vrow + (((2 * cc + hl) ^ sw) << 4)), pb[cc], oacc[dt]);
            }
        }
        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O / l, LSE = m ln2 + ln l ----
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    if (my_q < N) {
        __bf16* dst = O + head_off + (long)my_q * row_stride;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = dt * 32 + g * 8 + hl * 4;
                const uint32_t w0 = pack_bf16x2(oacc[dt][g * 4 + 0] * inv, oacc[dt][g * 4 + 1] * inv);
                const uint32_t w1 = pack_bf16x2(oacc[dt][g * 4 + 2] * inv, oacc[dt][g * 4 + 3] * inv);
                *reinterpret_cast<u32x2*>(dst + d) = u32x2{w0, w1};
            }
        if (hl == 0) LSE[(long)bh * N + my_q] = m_run * kLn2 + __logf(l_tot);
    }
}

// ---------------------------------------------------------------------------
// fp32 path: fp32 inputs, outputs and arithmetic (VALU FMA, no MFMA).  One
// thread per query; K/V blocks of BC rows staged in LDS and read as
// broadcasts; the online softmax is updated once per group of 8 keys.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int H, int N, float scale, int causal, int nqb) {
    constexpr int NT = 128;
    constexpr int BC = D == 64 ? 256 : 128;
    constexpr int G = 8;
    __shared__ __attribute__((aligned(16))) float ks[BC * D];
    __shared__ __attribute__((aligned(16))) float vs[BC * D];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
    const int b = bh / H, h = bh - b * H;
    const long row_stride = (long)H * D;
    const long head_off = ((long)b * N * H + h) * D;
    const int my_q = qb * NT + tid;
    const bool valid = my_q < N;

    float q[D], o[D];
    {
        const float* src = Q + head_off + (long)(valid ? my_q : 0) * row_stride;
#pragma unroll
        for (int i = 0; i < D; ++i) {
            q[i] = valid ? src[i] : 0.f;
            o[i] = 0.f;
        }
    }
    float m = -INFINITY, l = 0.f;
    const int q_last = min(N, qb * NT + NT) - 1;
    const int kv_end = causal ? q_last + 1 : N;

    for (int j0 = 0; j0 < kv_end; j0 += BC) {
        __syncthreads();
        for (int c = tid; c < BC * D / 4; c += NT) {
            const int r = c / (D / 4), cc = c % (D / 4);
            const int key = j0 + r;
            f32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
            if (key < N) {
                kv = *reinterpret_cast<const f32x4*>(K + head_off + (long)key * row_stride + cc * 4);
                vv = *reinterpret_cast<const f32x4*>(V + head_off + (long)key * row_stride + cc * 4);
            }
            *reinterpret_cast<f32x4*>(ks + r * D + cc * 4) = kv;
            *reinterpret_cast<f32x4*>(vs + r * D + cc * 4) = vv;
        }
        __syncthreads();
        const int kmax = min(BC, kv_end - j0);
        for (int j = 0; j < kmax; j += G) {
            float s[G];
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const float* kr = ks + (j + u) * D;
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < D; ++i) acc = __builtin_fmaf(q[i], kr[i], acc);
                const int key = j0 + j + u;
                const bool vis = j + u < kmax && key < N && (!causal || key <= my_q);
                s[u] = vis ? acc * scale : -INFINITY;
                mx = fmaxf(mx, s[u]);
            }
            const float m_new = fmaxf(m, mx);
            const float m_sub = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = exp2f((m - m_sub) * kLog2e);
            float p[G];
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < G; ++u) {
                p[u] = exp2f((s[u] - m_sub) * kLog2e);
                ps += p[u];
            }
            l = l * alpha + ps;
#pragma unroll
            for (int i = 0; i < D; ++i) {
                float acc = o[i] * alpha;
#pragma unroll
                for (int u = 0; u < G; ++u) acc = __builtin_fmaf(p[u], vs[(j + u) * D + i], acc);
                o[i] = acc;
            }
            m = m_new;
        }
    }
    if (valid) {
        float* dst = O + head_off + (long)my_q * row_stride;
        const float inv = 1.f / l;
#pragma unroll
        for (int i = 0; i < D; ++i) dst[i] = o[i] * inv;
        LSE[(long)bh * N + my_q] = m + logf(l);
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int N, int d, float scale, bool causal, hipStream_t stream) {
    const int nqb = (N + fwd::BR - 1) / fwd::BR;
    const dim3 grid((unsigned)(B * H * nqb)), block(fwd::NT);
    const float sl2 = scale * kLog2e;
    auto Qp = static_cast<const __bf16*>(q);
    auto Kp = static_cast<const __bf16*>(k);
    auto Vp = static_cast<const __bf16*>(v);
    auto Op = static_cast<__bf16*>(o);
    if (d == 128) {
        if (causal)
            hipLaunchKernelGGL((fwd_bf16_kernel<128, true>), grid, block, 0, stream, Qp, Kp, Vp, Op, lse, H, N, sl2, nqb);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<128, false>), grid, block, 0, stream, Qp, Kp, Vp, Op, lse, H, N, sl2, nqb);
    } else {
        if (causal)
            hipLaunchKernelGGL((fwd_bf16_kernel<64, true>), grid, block, 0, stream, Qp, Kp, Vp, Op, lse, H, N, sl2, nqb);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<64, false>), grid, block, 0, stream, Qp, Kp, Vp, Op, lse, H, N, sl2, nqb);
    }
    return hipGetLastError();
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                          int H, int N, int d, float scale, bool causal, hipStream_t stream) {
    const int nqb = (N + 127) / 128;
    const dim3 grid((unsigned)(B * H * nqb)), block(128);
    if (d == 128)
        hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, block, 0, stream, q, k, v, o, lse, H, N, scale, (int)causal, nqb);
    else
        hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, block, 0, stream, q, k, v, o, lse, H, N, scale, (int)causal, nqb);
    return hipGetLastError();
}

}  // namespace fa
