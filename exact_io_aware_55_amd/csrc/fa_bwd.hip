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
//   1. bwd_pre:  D_i = rowsum(dO * O) and LSE_i * log2(e) into per-head rows
//      padded to a multiple of 64 (padding: D = 0, LSE = +inf, so padded
//      queries get P = 0), and zero the fp32 dQ accumulator.
//   2. bwd_kv:   one workgroup per block of 128 keys of one head (4 waves, one
//      per SIMD, 32 keys each).  K and V of a wave's keys, and the K^T slice
//      the wave needs for dQ, stay in registers.  The workgroup walks the
//      query blocks of 64 rows that can see its keys; Q, dO and the row
//      statistics stream into a 3-stage LDS ring by direct global -> LDS
//      loads.  Per block it recomputes S = Q K^T and P, forms dP = dO V^T and
//      dS, accumulates dV^T += dO^T P and dK^T += Q^T dS in registers, and
//      adds its share of dQ = dS K into the fp32 accumulator with hardware
//      float atomics.  Workgroups of one head start at different query
//      blocks so their atomics and loads spread over the dQ rows.
//   3. bwd_dq_convert: dQ accumulator (fp32) -> bf16.
//
// MFMA orientation: S = Q K_w^T puts one key per lane (lane & 31) and the
// queries in registers, so P and dS in registers are directly the B operand
// of dV^T += dO^T P and dK^T += Q^T dS (contraction over queries).  dO^T and
// Q^T come from the row-major tiles by transposing LDS reads
// (ds_read_b64_tr_b16).  dS crosses lanes once: each lane writes its key's
// column of dS^T to LDS and the dQ product reads it back transposed.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace bwd {
constexpr int NT = 256;      // threads per workgroup (4 waves, one per SIMD)
constexpr int NW = 4;
constexpr int KB = 128;      // keys per workgroup (32 per wave)
constexpr int BR = 64;       // queries per step
constexpr int NSTAGE = 3;    // query blocks resident in the LDS ring
constexpr int ROWPAD = 64;   // row-statistic padding (= BR)
}  // namespace bwd

__device__ __forceinline__ int xcd_remap_b(int bid, int nblocks) {
    const int per = nblocks >> 3, rem = nblocks & 7;
    const int x = bid & 7, i = bid >> 3;
    return x * per + (x < rem ? x : rem) + i;
}

// ---------------------------------------------------------------------------
// 1. D_i = sum_k dO_ik O_ik, LSE_i * log2(e) (padded rows), dQ accumulator := 0.
// Rows are enumerated in [B, H, Npad] order.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ O,
                                                      const __bf16* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      float* __restrict__ lse2,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ dq_acc, int H, int N,
                                                      int Npad, long rows) {
    constexpr int TPR = D / 8;                 // threads per row (8 elements each)
    constexpr int RPB = 256 / TPR;             // rows per block
    const int tid = threadIdx.x;
    const long row = (long)blockIdx.x * RPB + tid / TPR;
    const int part = tid % TPR;
    const long bh = row / Npad;
    const int i = (int)(row - bh * Npad);
    const bool live = row < rows && i < N;
    float acc = 0.f;
    if (live) {
        const long b = bh / H, h = bh - b * H;
        const long off = ((b * N + i) * H + h) * D + part * 8;
        const u32x4 a = ld_global16(O + off), g = ld_global16(dO + off);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a0 = __builtin_bit_cast(float, a[w] << 16), a1 = __builtin_bit_cast(float, a[w] & 0xffff0000u);
            const float g0 = __builtin_bit_cast(float, g[w] << 16), g1 = __builtin_bit_cast(float, g[w] & 0xffff0000u);
            acc = __builtin_fmaf(a0, g0, acc);
            acc = __builtin_fmaf(a1, g1, acc);
        }
        const f32x4 z = {0, 0, 0, 0};
        *reinterpret_cast<f32x4*>(dq_acc + off) = z;
        *reinterpret_cast<f32x4*>(dq_acc + off + 4) = z;
    }
#pragma unroll
    for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
    if (row < rows && part == 0) {
        delta[row] = live ? acc : 0.f;
        lse2[row] = live ? LSE[bh * N + i] * kLog2e : INFINITY;
    }
}

// ---------------------------------------------------------------------------
// 2. key-block kernel
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(bwd::NT, 1) void bwd_kv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ stats, int delta_off,
    float* __restrict__ dq_acc, __bf16* __restrict__ dK, __bf16* __restrict__ dV, int H, int N,
    int Npad, float scale, float scale_log2, int nkb) {
    using namespace bwd;
    constexpr int DC = D / 16;                 // k-chunks over features
    constexpr int DT = D / 32;                 // 32-feature sub-tiles
    constexpr int QT = BR * D * 2;             // bytes of a Q or dO tile
    constexpr int SUBQ = BR * 64;              // Q/dO sub-tile: BR rows x 32 features
    constexpr int STAGE = 2 * QT + NW * 1024;  // Q, dO, one stats copy per wave
    constexpr int KVB = KB * D * 2;            // bytes of a K or V block
    constexpr int SUBK = KB * 64;              // K/V/dS^T sub-tile: KB rows x 32 columns
    constexpr int RING = NSTAGE * STAGE;
    constexpr int DST = KB * BR * 2;           // dS^T tile
    constexpr int SEG_QO = 2 * QT / 1024 / NW; // Q + dO segments per wave per step
    constexpr int DMA_W = SEG_QO + 1;          // direct loads per wave per step
    constexpr int SEG_KV = KVB / 1024 / NW;    // K (and V) segments per wave at start
    static_assert(2 * KVB <= RING, "K/V staging fits in the ring");
    static_assert(DMA_W <= 15, "vmcnt immediate");
    __shared__ __attribute__((aligned(1024))) char smem[RING + DST];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;
    const int tg = lane >> 4, tj = lane & 15;  // transposing-read group and lane

    const int logical = xcd_remap_b(blockIdx.x, gridDim.x);
    const int bh = logical / nkb;
    const int kb = logical - bh * nkb;
    const int b = bh / H, h = bh - b * H;
    const int row_stride = H * D;
    const unsigned row_bytes = (unsigned)row_stride * 2u;
    const long head_off = ((long)b * N * H + h) * D;
    const char* Qh = reinterpret_cast<const char*>(Q + head_off);
    const char* Kh = reinterpret_cast<const char*>(K + head_off);
    const char* Vh = reinterpret_cast<const char*>(V + head_off);
    const char* dOh = reinterpret_cast<const char*>(dO + head_off);
    float* dQh = dq_acc + head_off;
    const unsigned lds0 = lds_offset(smem);
    const lds_char* L = as_lds(smem);

    const int k0 = kb * KB;
    const int key_local = wave * 32 + l32;
    const int my_key = k0 + key_local;         // key of this lane in S / P / dS
    const bool key_ok = my_key < N;

    // transposing-read lane pattern: rows R_w = 4 (tg >> 1) + (tj >> 2) (+8 for
    // the second read), 8 bytes at column 16 (tg & 1) + 4 (tj & 3) of a 32-wide
    // sub-tile; the swizzle only depends on bits 1..3 of the row
    const int tr_r0 = 4 * (tg >> 1) + (tj >> 2), tr_r1 = tr_r0 + 8;
    const int tr_cl = 2 * (tg & 1) + ((tj & 3) >> 1);
    const int tr0 = tr_r0 * 64 + ((tr_cl ^ dual_swz(tr_r0)) << 4) + ((tj & 1) << 3);
    const int tr1 = tr_r1 * 64 + ((tr_cl ^ dual_swz(tr_r1)) << 4) + ((tj & 1) << 3);

    // ---- K and V blocks -> LDS (sub-tiled [DT][KB][32], swizzled) -> registers ----
#pragma unroll
    for (int i = 0; i < SEG_KV; ++i) {
        const int seg = wave * SEG_KV + i;
        const int sub = seg / (SUBK / 1024), r = (seg % (SUBK / 1024)) * 16 + (lane >> 2);
        const unsigned go = (unsigned)min(k0 + r, N - 1) * row_bytes + sub * 64 + (((lane & 3) ^ dual_swz(r)) << 4);
        dma16(Kh, go, __builtin_amdgcn_readfirstlane(lds0 + seg * 1024));
        dma16(Vh, go, __builtin_amdgcn_readfirstlane(lds0 + KVB + seg * 1024));
    }
    FA_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    // B operands of S = Q K_w^T and dP = dO V_w^T: key row key_local, features 16c + 8hl..
    bf16x8 kreg[DC], vreg[DC];
    {
        const int a0 = key_local * 64 + ((hl ^ dual_swz(key_local)) << 4);
        const int a1 = key_local * 64 + (((2 + hl) ^ dual_swz(key_local)) << 4);
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const int off = ((c & 1) ? a1 : a0) + (c >> 1) * SUBK;
            kreg[c] = lds_read_b128(L + off);
            vreg[c] = lds_read_b128(L + KVB + off);
        }
    }
    // B operand of dQ[:, 32 dq_dt + ..] = dS K: feature column 32 dq_dt + l32,
    // k-slots = keys in the transposing-read order (same as the dS A operand)
    constexpr int DQT = D / 32;                // feature tiles of dQ
    const int dq_dt = wave % DQT, dq_qt0 = wave / DQT;   // D=128: qt 0,1 ; D=64: qt = wave/2
    constexpr int DQ_NQ = (BR / 32) * DQT / NW;          // query tiles per wave (2 or 1)
    bf16x8 ktreg[KB / 16];
#pragma unroll
    for (int c = 0; c < KB / 16; ++c) {
        const lds_char* p = L + dq_dt * SUBK + c * 16 * 64;
        const bf16x4 lo = lds_read_tr16(p + tr0), hi = lds_read_tr16(p + tr1);
        ktreg[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // the ring overwrites the K/V staging: everyone must have read it
    __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();

    // ---- query steps: first..nsteps-1, rotated per key block ----
    const int nsteps = (N + BR - 1) / BR;
    const int first = CAUSAL ? k0 / BR : 0;
    const int nst = nsteps - first;
    const int stagger = nst > 0 ? kb % nst : 0;
    auto step_of = [&](int it) {
        int s = it + stagger;
        s = s >= nst ? s - nst : s;
        return first + s;
    };

    // direct loads of one step: SEG_QO segments of Q/dO per wave + the stats
    int ld_r[SEG_QO], ld_c[SEG_QO];
#pragma unroll
    for (int i = 0; i < SEG_QO; ++i) {
        const int seg = wave * SEG_QO + i;
        const int sseg = seg % (QT / 1024);
        const int sub = sseg / (SUBQ / 1024), r = (sseg % (SUBQ / 1024)) * 16 + (lane >> 2);
        ld_r[i] = r;
        ld_c[i] = sub * 64 + (((lane & 3) ^ dual_swz(r)) << 4);
    }
    const unsigned st_lane = (unsigned)((bh * Npad + 4 * (lane & 15)) * 4 + ((lane & 16) ? delta_off : 0));
    auto issue_step = [&](int it) {
        const int i0 = step_of(it) * BR;
        const unsigned base = lds0 + (it % NSTAGE) * STAGE;
#pragma unroll
        for (int i = 0; i < SEG_QO; ++i) {
            const int seg = wave * SEG_QO + i;
            const unsigned go = (unsigned)min(i0 + ld_r[i], N - 1) * row_bytes + ld_c[i];
            dma16(seg < QT / 1024 ? Qh : dOh, go, __builtin_amdgcn_readfirstlane(base + seg * 1024));
        }
        dma16(stats, st_lane + i0 * 4, __builtin_amdgcn_readfirstlane(base + 2 * QT + wave * 1024));
    };
    if (nst > 0) issue_step(0);
    if (nst > 1) issue_step(1);

    f32x16 dvacc[DT], dkacc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) {
        dvacc[i] = f32x16{};
        dkacc[i] = f32x16{};
    }

    // per-lane LDS offsets (within a stage) of the operand reads
    const int a_rd0 = l32 * 64 + ((hl ^ dual_swz(l32)) << 4);        // Q/dO rows, even c
    const int a_rd1 = l32 * 64 + (((2 + hl) ^ dual_swz(l32)) << 4);  // odd c
    const int ds_wr = RING + key_local * 64 + (hl << 3);              // dS^T row of this key
    const int ds_sw = dual_swz(key_local);

#pragma clang loop unroll(disable)
    for (int it = 0; it < nst; ++it) {
        if (it + 1 < nst) FA_WAIT_VMCNT(DMA_W);
        else FA_WAIT_VMCNT(0);
        __builtin_amdgcn_s_barrier();
        if (it + 2 < nst) issue_step(it + 2);

        const int i0 = step_of(it) * BR;
        const lds_char* stage = L + (it % NSTAGE) * STAGE;
        const lds_char* qa0 = stage + a_rd0;
        const lds_char* qa1 = stage + a_rd1;
        const lds_char* t0 = stage + tr0;
        const lds_char* t1 = stage + tr1;
        const lds_char* sw = stage + 2 * QT + wave * 1024 + hl * 16;
        asm volatile("" : "+v"(qa0), "+v"(qa1), "+v"(t0), "+v"(t1), "+v"(sw));

        const bool wave_on = !CAUSAL || (k0 + wave * 32 <= i0 + BR - 1);
        if (wave_on) {
            u32x4 pb[BR / 16], dsb[BR / 16];
            const bool need_mask = (i0 + BR > N) || (k0 + KB > N) || (CAUSAL && k0 + KB - 1 > i0);
#pragma unroll
            for (int m = 0; m < BR / 32; ++m) {
                // S = Q K_w^T, dP = dO V_w^T: 32 queries (registers) x 32 keys (lanes)
                f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
                for (int c = 0; c < DC; ++c) {
                    const lds_char* a = ((c & 1) ? qa1 : qa0) + (c >> 1) * SUBQ + m * 32 * 64;
                    sacc = mfma32x32x16(lds_read_b128(a), kreg[c], sacc);
                    pacc = mfma32x32x16(lds_read_b128(a + QT), vreg[c], pacc);
                }
                // statistics of the lane's queries 32m + 8g + 4hl + (0..3)
                f32x4 lse4[4], dl4[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    lse4[g] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(sw + (32 * m + 8 * g) * 4);
                    dl4[g] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(sw + 256 + (32 * m + 8 * g) * 4);
                }
                float pv[16], dsv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(__builtin_fmaf(sacc[r], scale_log2, -lse4[r >> 2][r & 3]));
                    pv[r] = p;
                    dsv[r] = p * (pacc[r] - dl4[r >> 2][r & 3]);
                }
                if (need_mask) {
                    // query of register r = i0 + 4 hl + off, off = 32m + 8(r>>2) + (r&3)
                    const int lim_n = N - i0 - 4 * hl;            // q < N      <=> off < lim_n
                    const int lim_c = my_key - i0 - 4 * hl;       // key <= q   <=> off >= lim_c
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = 32 * m + 8 * (r >> 2) + (r & 3);
                        const bool vis = key_ok && off < lim_n && (!CAUSAL || off >= lim_c);
                        pv[r] = vis ? pv[r] : 0.f;
                        dsv[r] = vis ? dsv[r] : 0.f;
                    }
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t p01 = pack_bf16x2(pv[4 * g], pv[4 * g + 1]);
                    const uint32_t p23 = pack_bf16x2(pv[4 * g + 2], pv[4 * g + 3]);
                    const uint32_t d01 = pack_bf16x2(dsv[4 * g], dsv[4 * g + 1]);
                    const uint32_t d23 = pack_bf16x2(dsv[4 * g + 2], dsv[4 * g + 3]);
                    pb[2 * m + (g >> 1)][2 * (g & 1)] = p01;
                    pb[2 * m + (g >> 1)][2 * (g & 1) + 1] = p23;
                    dsb[2 * m + (g >> 1)][2 * (g & 1)] = d01;
                    dsb[2 * m + (g >> 1)][2 * (g & 1) + 1] = d23;
                    // dS^T[key][queries 32m + 8g + 4hl .. +3]
                    st_lds8(smem + ds_wr + m * SUBK + ((g ^ ds_sw) << 4), u32x2{d01, d23});
                }
            }
            // dV^T += dO^T P and dK^T += Q^T dS over the step's queries
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int cq = 0; cq < BR / 16; ++cq) {
                    const int off = dt * SUBQ + cq * 16 * 64;
                    const bf16x8 ot = __builtin_shufflevector(lds_read_tr16(t0 + QT + off), lds_read_tr16(t1 + QT + off),
                                                              0, 1, 2, 3, 4, 5, 6, 7);
                    dvacc[dt] = mfma32x32x16(ot, __builtin_bit_cast(bf16x8, pb[cq]), dvacc[dt]);
                    const bf16x8 qt = __builtin_shufflevector(lds_read_tr16(t0 + off), lds_read_tr16(t1 + off),
                                                              0, 1, 2, 3, 4, 5, 6, 7);
                    dkacc[dt] = mfma32x32x16(qt, __builtin_bit_cast(bf16x8, dsb[cq]), dkacc[dt]);
                }
        } else {
            // keys all after the step's queries: contribute dS = 0 to dQ
#pragma unroll
            for (int m = 0; m < BR / 32; ++m)
#pragma unroll
                for (int g = 0; g < 4; ++g) st_lds8(smem + ds_wr + m * SUBK + ((g ^ ds_sw) << 4), u32x2{0u, 0u});
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);    // this wave's dS^T writes done
        __builtin_amdgcn_s_barrier();          // everyone's dS^T visible

        // dQ[queries 32 qt.., features 32 dq_dt..] += dS K over the block's keys
        const lds_char* d0 = L + RING + tr0;
        const lds_char* d1 = L + RING + tr1;
        asm volatile("" : "+v"(d0), "+v"(d1));
#pragma unroll
        for (int qi = 0; qi < DQ_NQ; ++qi) {
            const int qt = dq_qt0 + qi * (NW / DQT);
            f32x16 acc = f32x16{};
#pragma unroll
            for (int c = 0; c < KB / 16; ++c) {
                const int off = qt * SUBK + c * 16 * 64;
                const bf16x8 dsa = __builtin_shufflevector(lds_read_tr16(d0 + off), lds_read_tr16(d1 + off),
                                                           0, 1, 2, 3, 4, 5, 6, 7);
                acc = mfma32x32x16(dsa, ktreg[c], acc);
            }
            // C layout: lane = feature column, registers = queries 32qt + 8(r>>2) + 4hl + (r&3)
            const int lim_n = N - i0 - 32 * qt - 4 * hl;
            float* dst = dQh + (long)(i0 + 32 * qt + 4 * hl) * row_stride + dq_dt * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int off = 8 * (r >> 2) + (r & 3);
                if (off < lim_n) unsafeAtomicAdd(dst + (long)off * row_stride, acc[r] * scale);
            }
        }
    }

    // epilogue: dK = scale * (dK^T)^T, dV; C layout of dV^T / dK^T: lane = key
    // column, registers = feature rows 8g + 4h + t
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

int bwd_rows_padded(int N) { return (N + bwd::ROWPAD - 1) / bwd::ROWPAD * bwd::ROWPAD; }

hipError_t launch_bwd_preprocess(const void* o, const void* dout, const float* lse, int B, int H,
                                 int N, int d, float* lse2, float* delta, float* dq_acc,
                                 hipStream_t stream) {
    auto Op = static_cast<const __bf16*>(o);
    auto dOp = static_cast<const __bf16*>(dout);
    const int Npad = bwd_rows_padded(N);
    const long rows = (long)B * H * Npad;
    const int rpb = 256 / (d / 8);
    const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
    if (d == 128)
        hipLaunchKernelGGL((bwd_pre_kernel<128>), grid, dim3(256), 0, stream, Op, dOp, lse, lse2, delta, dq_acc, H, N, Npad, rows);
    else
        hipLaunchKernelGGL((bwd_pre_kernel<64>), grid, dim3(256), 0, stream, Op, dOp, lse, lse2, delta, dq_acc, H, N, Npad, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_kv_blocks(const void* q, const void* k, const void* v, const void* dout,
                                void* dk, void* dv, int B, int H, int N, int d, float scale,
                                bool causal, const float* lse2, const float* delta, float* dq_acc,
                                hipStream_t stream) {
    auto Qp = static_cast<const __bf16*>(q);
    auto Kp = static_cast<const __bf16*>(k);
    auto Vp = static_cast<const __bf16*>(v);
    auto dOp = static_cast<const __bf16*>(dout);
    auto dKp = static_cast<__bf16*>(dk);
    auto dVp = static_cast<__bf16*>(dv);
    const int Npad = bwd_rows_padded(N);
    const int nkb = (N + bwd::KB - 1) / bwd::KB;
    const dim3 grid((unsigned)(B * H * nkb)), block(bwd::NT);
    const float sl2 = scale * kLog2e;
    const int delta_off = (int)((const char*)delta - (const char*)lse2);
#define FA_BWD_LAUNCH(DD, CC)                                                                      \
    hipLaunchKernelGGL((bwd_kv_kernel<DD, CC>), grid, block, 0, stream, Qp, Kp, Vp, dOp, lse2,    \
                       delta_off, dq_acc, dKp, dVp, H, N, Npad, scale, sl2, nkb)
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
