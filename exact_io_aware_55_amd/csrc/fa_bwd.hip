// Backward pass of exact attention on gfx950 by recomputation.
//
// The forward keeps only O and LSE per row; the backward recomputes
// P = exp(scale * Q K^T - LSE) tile by tile instead of reading a stored N x N
// matrix (explainer page "Flash Attention", section "Recomputation beim
// Rueckwaertsdurchlauf"; glossary page "Flash Attention", section "How it
// works").  The gradient formulas are the standard softmax Jacobian:
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels run on the caller's stream:
//   1. bwd_pre:  D_i = rowsum(dO * O) in fp32, and zero the fp32 dQ accumulator.
//   2. bwd_main: one workgroup per block of 128 keys of one head (4 waves,
//      32 keys each).  K and V of a wave's keys stay in registers; the
//      workgroup walks the query blocks (causal: only those that can see its
//      keys), recomputes S = Q K^T and P, and accumulates dV^T and dK^T in
//      registers.  dS goes through LDS so the workgroup can form its
//      contribution dS K to dQ, added into the fp32 accumulator with
//      hardware float atomics.
//   3. bwd_dq_convert: dQ accumulator (fp32) -> bf16.
//
// MFMA orientation: S = Q K_w^T puts one key per lane (lane & 31) and the
// queries in registers, so P and dS in registers are directly the B operand
// of dV^T += dO^T P and dK^T += Q^T dS (contraction over queries).  dO^T and
// Q^T are staged transposed in LDS with queries in the k-slot order of those
// registers.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace bwd {
constexpr int NT = 256;      // threads per workgroup (4 waves)
constexpr int KB = 128;      // keys per workgroup (32 per wave)
}  // namespace bwd

// XOR swizzles of 16-byte chunks per LDS row, chosen so that 16 consecutive
// rows read at the same logical chunk fall on distinct banks.
__device__ __forceinline__ int swz4(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
__device__ __forceinline__ int swz16(int row) { return row & 15; }

__device__ __forceinline__ int xcd_remap_b(int bid, int nblocks) {
    const int per = nblocks >> 3, rem = nblocks & 7;
    const int x = bid & 7, i = bid >> 3;
    return x * per + (x < rem ? x : rem) + i;
}

// ---------------------------------------------------------------------------
// 1. D_i = sum_k dO_ik O_ik (fp32) and dQ accumulator := 0.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ O,
                                                      const __bf16* __restrict__ dO,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ dq_acc, int H, int N,
                                                      long rows) {
    constexpr int TPR = D / 8;                 // threads per row (8 elements each)
    constexpr int RPB = 256 / TPR;             // rows per block
    const int tid = threadIdx.x;
    const long row = (long)blockIdx.x * RPB + tid / TPR;
    const int part = tid % TPR;
    float acc = 0.f;
    if (row < rows) {
        const long off = row * D + part * 8;
        const u32x4 a = ld_global16(O + off), g = ld_global16(dO + off);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a0 = __builtin_bit_cast(float, a[w] << 16), a1 = __builtin_bit_cast(float, a[w] & 0xffff0000u);
            const float g0 = __builtin_bit_cast(float, g[w] << 16), g1 = __builtin_bit_cast(float, g[w] & 0xffff0000u);
            acc = __builtin_fmaf(a0, g0, acc);
            acc = __builtin_fmaf(a1, g1, acc);
        }
        f32x4 z = {0, 0, 0, 0};
        *reinterpret_cast<f32x4*>(dq_acc + off) = z;
        *reinterpret_cast<f32x4*>(dq_acc + off + 4) = z;
    }
#pragma unroll
    for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
    if (row < rows && part == 0) {
        // row = (b * N + i) * H + h  ->  delta[(b * H + h) * N + i]
        const long bi = row / H;
        const int h = (int)(row - bi * H);
        const long b = bi / N;
        const int i = (int)(bi - b * N);
        delta[(b * H + h) * N + i] = acc;
    }
}

// ---------------------------------------------------------------------------
// 2. main backward kernel
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(bwd::NT) void bwd_main_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dlt,
    float* __restrict__ dq_acc, __bf16* __restrict__ dK, __bf16* __restrict__ dV, int H, int N,
    float scale, float scale_log2, int nkb) {
    using namespace bwd;
    constexpr int BR = 4096 / D;               // queries per step: 32 (d=128) or 64 (d=64)
    constexpr int MQ = BR / 32;                // 32-query tiles per step
    constexpr int DC = D / 16;                 // k-chunks over features
    constexpr int DT = D / 32;                 // 32-row feature tiles
    constexpr int QC = BR / 16;                // k-chunks over the step's queries
    constexpr int RP = D * 2 + 16;             // row-major Q/dO pitch (bytes)
    constexpr int TRP = BR * 2;                // transposed Q^T/dO^T row (bytes)
    constexpr int SP = KB * 2 + 16;            // dS row pitch (bytes)
    constexpr int KTP = KB * 2;                // K^T row (bytes), 16 chunks
    constexpr int CPR = D / 8;                 // 16-byte chunks per feature row
    constexpr int QPT = 2;                     // queries per thread in the staging
    static_assert(BR * CPR == NT * QPT, "staging layout");

    constexpr int OFF_Q = 0;
    constexpr int OFF_DO = OFF_Q + BR * RP;
    constexpr int OFF_QT = OFF_DO + BR * RP;
    constexpr int OFF_DOT = OFF_QT + D * TRP;
    constexpr int OFF_DS = OFF_DOT + D * TRP;
    constexpr int OFF_KT = OFF_DS + BR * SP;
    constexpr int OFF_L = OFF_KT + D * KTP;
    constexpr int OFF_DL = OFF_L + BR * 4;
    constexpr int LDS_BYTES = OFF_DL + BR * 4;
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;

    const int logical = xcd_remap_b(blockIdx.x, gridDim.x);
    const int bh = logical / nkb;
    const int kb = logical - bh * nkb;
    const int b = bh / H, h = bh - b * H;
    const long row_stride = (long)H * D;
    const long head_off = ((long)b * N * H + h) * D;
    const __bf16* Qh = Q + head_off;
    const __bf16* Kh = K + head_off;
    const __bf16* Vh = V + head_off;
    const __bf16* dOh = dO + head_off;
    float* dQh = dq_acc + head_off;
    const float* LSEh = LSE + (long)bh * N;
    const float* Dh = Dlt + (long)bh * N;

    const int k0 = kb * KB;
    const int my_key = k0 + wave * 32 + l32;   // key of this lane in S / P / dS
    const bool key_ok = my_key < N;

    // K and V rows of this lane's key, as B-operand chunks (features 16c + 8h..).
    bf16x8 kreg[DC], vreg[DC];
    {
        const long off = (long)(key_ok ? my_key : 0) * row_stride + 8 * hl;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            kreg[c] = as_bf16x8(key_ok ? ld_global16(Kh + off + 16 * c) : u32x4{0, 0, 0, 0});
            vreg[c] = as_bf16x8(key_ok ? ld_global16(Vh + off + 16 * c) : u32x4{0, 0, 0, 0});
        }
    }
    // K^T of the whole key block in LDS (rows = features, keys contiguous).
    {
        char* kt = smem + OFF_KT;
        for (int c = tid; c < KB * CPR; c += NT) {
            const int r = c / CPR, cc = c % CPR;
            const int key = k0 + r;
            const u32x4 v = key < N ? ld_global16(Kh + (long)key * row_stride + cc * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = cc * 8 + e;
                const uint16_t val = (uint16_t)(v[e >> 1] >> ((e & 1) * 16));
                *reinterpret_cast<uint16_t*>(kt + d * KTP + ((((r >> 3) ^ swz16(d)) << 4) | ((r & 7) * 2))) = val;
            }
        }
    }

    f32x16 dvacc[DT], dkacc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) {
        dvacc[i] = f32x16{};
        dkacc[i] = f32x16{};
    }

    // query steps this key block takes part in
    const int nsteps = (N + BR - 1) / BR;
    const int first = CAUSAL ? k0 / BR : 0;

    // register staging of one step (Q, dO rows 2*qg, 2*qg+1, features dblk*8..)
    const int dblk = tid % CPR, qg = tid / CPR;
    u32x4 qst[QPT], ost[QPT];
    float lst = 0.f, dst_ = 0.f;
    auto load_step = [&](int s) {
        const int i0 = s * BR;
#pragma unroll
        for (int j = 0; j < QPT; ++j) {
            const int q = i0 + qg * QPT + j;
            const bool ok = q < N;
            const long off = (long)(ok ? q : 0) * row_stride + dblk * 8;
            qst[j] = ok ? ld_global16(Qh + off) : u32x4{0, 0, 0, 0};
            ost[j] = ok ? ld_global16(dOh + off) : u32x4{0, 0, 0, 0};
        }
        if (tid < BR) {
            const int q = i0 + tid;
            lst = q < N ? LSEh[q] * kLog2e : INFINITY;
            dst_ = q < N ? Dh[q] : 0.f;
        }
    };
    auto store_step = [&]() {
        const int tq = kslot_pos(qg * QPT);    // position of the query pair in k-slot order
#pragma unroll
        for (int j = 0; j < QPT; ++j) {
            const int r = qg * QPT + j;
            st_lds16(smem + OFF_Q + r * RP + dblk * 16, qst[j]);
            st_lds16(smem + OFF_DO + r * RP + dblk * 16, ost[j]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = dblk * 8 + e;
            const int w = e >> 1, sh = (e & 1) * 16;
            const int sw = (TRP == 64) ? swz4(d) : swz8(d);
            const int boff = d * TRP + ((((tq >> 3) ^ sw) << 4) | ((tq & 7) * 2));
            st_lds4(smem + OFF_QT + boff, ((qst[0][w] >> sh) & 0xffffu) | (((qst[1][w] >> sh) & 0xffffu) << 16));
            st_lds4(smem + OFF_DOT + boff, ((ost[0][w] >> sh) & 0xffffu) | (((ost[1][w] >> sh) & 0xffffu) << 16));
        }
        if (tid < BR) {
            reinterpret_cast<float*>(smem + OFF_L)[tid] = lst;
            reinterpret_cast<float*>(smem + OFF_DL)[tid] = dst_;
        }
    };

    // dQ tile owned by this wave in the dQ product: 32 queries x 32 features
    constexpr int DQT = D / 32;                // feature tiles across dQ
    const int dq_qt = wave / DQT, dq_dt = wave % DQT;

    if (first < nsteps) load_step(first);
    for (int s = first; s < nsteps; ++s) {
        __syncthreads();                       // previous step done with LDS
        store_step();
        __syncthreads();
        if (s + 1 < nsteps) load_step(s + 1);
        const int i0 = s * BR;

        const float* Ls = reinterpret_cast<const float*>(smem + OFF_L);
        const float* Ds = reinterpret_cast<const float*>(smem + OFF_DL);
        bf16x8 pb[QC], dsb[QC];
#pragma unroll
        for (int m = 0; m < MQ; ++m) {
            // S = Q K_w^T and dP = dO V_w^T for 32 queries (rows) x 32 keys (lanes)
            f32x16 sacc = f32x16{}, pacc = f32x16{};
            const char* qrow = smem + OFF_Q + (m * 32 + l32) * RP + hl * 16;
            const char* orow = smem + OFF_DO + (m * 32 + l32) * RP + hl * 16;
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                sacc = mfma32x32x16(ld_lds_bf16x8(qrow + c * 32), kreg[c], sacc);
                pacc = mfma32x32x16(ld_lds_bf16x8(orow + c * 32), vreg[c], pacc);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ql = m * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
                const int q = i0 + ql;
                const bool vis = key_ok && (!CAUSAL || my_key <= q);
                const float p = vis ? fast_exp2(__builtin_fmaf(sacc[r], scale_log2, -Ls[ql])) : 0.f;
                const float ds = p * (pacc[r] - Ds[ql]);
                pb[m * 2 + (r >> 3)][r & 7] = (__bf16)p;
                dsb[m * 2 + (r >> 3)][r & 7] = (__bf16)ds;
                // dS to LDS in natural [query][key] order for the dQ product
                *reinterpret_cast<__bf16*>(smem + OFF_DS + ql * SP + (wave * 32 + l32) * 2) = (__bf16)ds;
            }
        }
        // dV^T += dO^T P,  dK^T += Q^T dS  (contraction over the step's queries)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int d = dt * 32 + l32;
            const int sw = (TRP == 64) ? swz4(d) : swz8(d);
            const char* ort = smem + OFF_DOT + d * TRP;
            const char* qrt = smem + OFF_QT + d * TRP;
#pragma unroll
            for (int cq = 0; cq < QC; ++cq) {
                const int off = ((2 * cq + hl) ^ sw) << 4;
                dvacc[dt] = mfma32x32x16(ld_lds_bf16x8(ort + off), pb[cq], dvacc[dt]);
                dkacc[dt] = mfma32x32x16(ld_lds_bf16x8(qrt + off), dsb[cq], dkacc[dt]);
            }
        }
        __syncthreads();                       // dS of all four waves in LDS
        // dQ[32 queries x 32 features] += dS[32 x 128 keys] K[128 keys x 32 features]
        {
            f32x16 acc = f32x16{};
            const char* srow = smem + OFF_DS + (dq_qt * 32 + l32) * SP + hl * 16;
            const int d = dq_dt * 32 + l32;
            const char* krow = smem + OFF_KT + d * KTP;
            const int sw = swz16(d);
#pragma unroll
            for (int c = 0; c < KB / 16; ++c)
                acc = mfma32x32x16(ld_lds_bf16x8(srow + c * 32), ld_lds_bf16x8(krow + (((2 * c + hl) ^ sw) << 4)), acc);
            // C layout: lane = feature column, registers = query rows
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = i0 + dq_qt * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
                if (q < N) unsafeAtomicAdd(dQh + (long)q * row_stride + d, acc[r] * scale);
            }
        }
    }

    // epilogue: dK = scale * dK^T^T, dV -> bf16.  C layout of dV^T / dK^T:
    // lane = key column, registers = feature rows 8g + 4h + t.
    if (key_ok) {
        __bf16* dkr = dK + head_off + (long)my_key * row_stride;
        __bf16* dvr = dV + head_off + (long)my_key * row_stride;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = dt * 32 + g * 8 + hl * 4;
                const f32x16& kk = dkacc[dt];
                const f32x16& vv = dvacc[dt];
                *reinterpret_cast<u32x2*>(dkr + d) =
                    u32x2{pack_bf16x2(kk[g * 4] * scale, kk[g * 4 + 1] * scale),
                          pack_bf16x2(kk[g * 4 + 2] * scale, kk[g * 4 + 3] * scale)};
                *reinterpret_cast<u32x2*>(dvr + d) =
                    u32x2{pack_bf16x2(vv[g * 4], vv[g * 4 + 1]), pack_bf16x2(vv[g * 4 + 2], vv[g * 4 + 3])};
            }
    }
}

// ---------------------------------------------------------------------------
// 3. dQ accumulator (fp32) -> bf16
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ acc,
                                                             __bf16* __restrict__ dq, long n8) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const f32x4 a = *reinterpret_cast<const f32x4*>(acc + i * 8);
    const f32x4 c = *reinterpret_cast<const f32x4*>(acc + i * 8 + 4);
    *reinterpret_cast<u32x4*>(dq + i * 8) =
        u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
}

hipError_t launch_bwd_preprocess(const void* o, const void* dout, int B, int H, int N, int d,
                                 float* delta, float* dq_acc, hipStream_t stream) {
    auto Op = static_cast<const __bf16*>(o);
    auto dOp = static_cast<const __bf16*>(dout);
    const long rows = (long)B * N * H;
    const int rpb = 256 / (d / 8);
    const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
    if (d == 128)
        hipLaunchKernelGGL((bwd_pre_kernel<128>), grid, dim3(256), 0, stream, Op, dOp, delta, dq_acc, H, N, rows);
    else
        hipLaunchKernelGGL((bwd_pre_kernel<64>), grid, dim3(256), 0, stream, Op, dOp, delta, dq_acc, H, N, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_kv_blocks(const void* q, const void* k, const void* v, const void* dout,
                                const float* lse, void* dk, void* dv, int B, int H, int N, int d,
                                float scale, bool causal, const float* delta, float* dq_acc,
                                hipStream_t stream) {
    auto Qp = static_cast<const __bf16*>(q);
    auto Kp = static_cast<const __bf16*>(k);
    auto Vp = static_cast<const __bf16*>(v);
    auto dOp = static_cast<const __bf16*>(dout);
    auto dKp = static_cast<__bf16*>(dk);
    auto dVp = static_cast<__bf16*>(dv);
    const int nkb = (N + bwd::KB - 1) / bwd::KB;
    const dim3 grid((unsigned)(B * H * nkb)), block(bwd::NT);
    const float sl2 = scale * kLog2e;
#define FA_BWD_LAUNCH(DD, CC)                                                                    \
    hipLaunchKernelGGL((bwd_main_kernel<DD, CC>), grid, block, 0, stream, Qp, Kp, Vp, dOp, lse, \
                       delta, dq_acc, dKp, dVp, H, N, scale, sl2, nkb)
    if (d == 128) {
        if (causal) FA_BWD_LAUNCH(128, true);
        else FA_BWD_LAUNCH(128, false);
    } else {
        if (causal) FA_BWD_LAUNCH(64, true);
        else FA_BWD_LAUNCH(64, false);
    }
#undef FA_BWD_LAUNCH
    return hipGetLastError();
}

hipError_t launch_bwd_dq_convert(void* dq, int B, int H, int N, int d, const float* dq_acc,
                                 hipStream_t stream) {
    const long n8 = (long)B * N * H * d / 8;
    hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                       dq_acc, static_cast<__bf16*>(dq), n8);
    return hipGetLastError();
}

}  // namespace fa
