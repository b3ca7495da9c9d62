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
//   1. bwd_pre:  -D_i = -rowsum(dO * O) and LSE_i * log2(e) into per-head rows
//      padded to a multiple of 64 (padding: D = 0, LSE = +inf, so padded
//      queries get P = 0).
//   2. bwd_dkdv: one workgroup per block of 128 keys of one head (4 waves, one
//      per SIMD, 32 keys each).  K and V of a wave's keys stay in registers.
//      The workgroup walks the query blocks of 64 rows that can see its keys;
//      Q, dO and the row statistics stream into an LDS ring (4 stages and one
//      barrier per two steps at d = 128, 3 stages at d = 64) by direct
//      global -> LDS loads.  Per block it recomputes S = Q K^T and P, forms
//      dP = dO V^T and dS, and accumulates dV^T += dO^T P and dK^T += Q^T dS
//      in registers.
//   3. bwd_dq:   one workgroup per block of 256 queries (8 waves, 32 queries
//      each, two waves per SIMD), laid out like the forward: Q and dO of a
//      wave's queries stay in registers, K/V blocks of 64 keys stream through
//      an LDS ring (4 stages at d = 128, 3 at d = 64).  Per block it
//      recomputes S^T = K Q^T, P^T and dP^T = V dO^T (one query per lane, so
//      LSE and D are per-lane scalars),
//      forms dS^T and accumulates dQ^T += K^T dS^T with dS^T straight from
//      registers.  Splitting dQ out costs two extra matrix products (S and dP
//      are formed twice) but needs no atomics and no LDS round trip for dS,
//      and every gradient is bitwise repeatable.
//
// MFMA orientation in bwd_dkdv: S = Q K_w^T puts one key per lane (lane & 31)
// and the queries in registers, so P and dS in registers are directly the B
// operand of dV^T += dO^T P and dK^T += Q^T dS (contraction over queries).
// dO^T and Q^T come from the row-major tiles by transposing LDS reads
// (ds_read_b64_tr_b16).  In bwd_dq the transposing read gives K^T.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace bwd {
constexpr int NT = 256;      // threads per workgroup (4 waves, one per SIMD)
constexpr int NW = 4;
constexpr int KB = 128;      // keys per workgroup (32 per wave)
constexpr int BR = 64;       // queries per step
constexpr int ROWPAD = 64;   // row-statistic padding (= BR)
constexpr int PRE_RPT = 2;   // preprocess rows per thread (2 measured best; 4 and 8 slower)
}  // namespace bwd


// ---------------------------------------------------------------------------
// 1. -D_i = -sum_k dO_ik O_ik and LSE_i * log2(e) (padded rows).
// Rows are enumerated in [B, H, Npad] order.
// ---------------------------------------------------------------------------
// Each thread keeps RPT rows' loads in flight (2 RPT 16-byte loads): the
// kernel is bound by HBM latency and bandwidth, not arithmetic.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ O,
                                                      const __bf16* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      float* __restrict__ lse2,
                                                      float* __restrict__ delta, int H, int N,
                                                      int Npad, long rows) {
    constexpr int TPR = D / 8;                 // threads per row (8 elements each)
    constexpr int RG = 256 / TPR;              // row groups per block
    constexpr int RPT = bwd::PRE_RPT;          // rows per thread
    const int tid = threadIdx.x;
    const int part = tid % TPR, rg = tid / TPR;
    u32x4 a[RPT], g[RPT];
    long row[RPT];
    bool live[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        // rows of one block: RPT passes of RG consecutive rows
        row[j] = ((long)blockIdx.x * RPT + j) * RG + rg;
        const long bh = row[j] / Npad;
        const int i = (int)(row[j] - bh * Npad);
        live[j] = row[j] < rows && i < N;
        if (live[j]) {
            const long b = bh / H, h = bh - b * H;
            const long off = ((b * N + i) * H + h) * D + part * 8;
            a[j] = ld_global16(O + off);
            g[j] = ld_global16(dO + off);
        }
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        float acc = 0.f;
        if (live[j]) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float a0 = __builtin_bit_cast(float, a[j][w] << 16), a1 = __builtin_bit_cast(float, a[j][w] & 0xffff0000u);
                const float g0 = __builtin_bit_cast(float, g[j][w] << 16), g1 = __builtin_bit_cast(float, g[j][w] & 0xffff0000u);
                acc = __builtin_fmaf(a0, g0, acc);
                acc = __builtin_fmaf(a1, g1, acc);
            }
        }
#pragma unroll
        for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
        if (row[j] < rows && part == 0) {
            const long bh = row[j] / Npad;
            const int i = (int)(row[j] - bh * Npad);
            delta[row[j]] = live[j] ? -acc : 0.f;   // stored negated: it seeds dP
            lse2[row[j]] = live[j] ? LSE[bh * N + i] * kLog2e : INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// 2. dK, dV: key-block kernel
// ---------------------------------------------------------------------------
// WIN: a sliding window narrower than N (causal only); without it the mask
// is the causal compare alone
template <int D, bool CAUSAL, bool WIN>
__global__ __launch_bounds__(bwd::NT, D == 64 ? 2 : 1) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ stats, int delta_off,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int H, int G, int N, int window, int Npad,
    float scale, float scale_log2, int nkb, int gen, int group) {
    using namespace bwd;
    constexpr int DC = D / 16;                 // k-chunks over features
    constexpr int DT = D / 32;                 // 32-feature sub-tiles
    constexpr int QT = BR * D * 2;             // bytes of a Q or dO tile
    constexpr int SUBQ = BR * 64;              // Q/dO sub-tile: BR rows x 32 features
    constexpr int STAGE = 2 * QT + NW * 1024;  // Q, dO, one stats copy per wave
    constexpr int KVB = KB * D * 2;            // bytes of a K or V block
    constexpr int SUBK = KB * 64;              // K/V sub-tile: KB rows x 32 features
    // query blocks resident in the LDS ring: 4 at d = 128, where one
    // barrier serves two steps (145 KB of LDS), 3 at d = 64, where two
    // workgroups share a CU and each step has its barrier
    constexpr int NSTAGE = D == 128 ? 4 : 3;
    constexpr bool PAIRED = NSTAGE == 4;
    constexpr int RING = NSTAGE * STAGE;
    constexpr int SEG_QO = 2 * QT / 1024 / NW; // Q + dO segments per wave per step
    constexpr int DMA_W = SEG_QO + 1;          // direct loads per wave per step
    constexpr int SEG_KV = KVB / 1024 / NW;    // K (and V) segments per wave at start
    static_assert(2 * KVB <= RING, "K/V staging fits in the ring");
    static_assert(DMA_W <= 15, "vmcnt immediate");
    // the ring, then 1 KB that absorbs the direct loads of the steps past the
    // last one (every step issues the same loads, so no branch is needed)
    __shared__ __attribute__((aligned(1024))) char smem[RING + 1024];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hl = lane >> 5;
    const int tg = lane >> 4, tj = lane & 15;  // transposing-read group and lane

    // one workgroup per (batch, K/V head, key block); with grouped-query
    // attention the G query heads hk G .. hk G + G - 1 share K/V head hk, and
    // the workgroup walks the query blocks of all of them (G = 1: one head)
    const int Hkv = H / G;
    int bhk, kb;                               // causal: key block 0 (the longest) first
    order_blocks(blockIdx.x, gridDim.x, nkb, CAUSAL, false, bhk, kb, group);
    const int b = bhk / Hkv, hk = bhk - b * Hkv;
    const int row_stride = H * D;
    const unsigned row_bytes = (unsigned)row_stride * 2u;
    const int kv_stride = Hkv * D;
    const unsigned kv_row_bytes = (unsigned)kv_stride * 2u;
    const long q_off = ((long)b * N * H + hk * G) * D;   // first query head of the group
    const long kv_off = ((long)b * N * Hkv + hk) * D;
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
    const lds_char* L = as_lds(smem);
    // byte ranges: the group's query heads (adjacent within a row) and the K/V
    // head; loads of rows past N read zeros
    const unsigned q_bytes = (unsigned)(N - 1) * row_bytes + 2 * D * G;
    const unsigned kv_bytes = (unsigned)(N - 1) * kv_row_bytes + 2 * D;
    const __amdgpu_buffer_rsrc_t rQ = byte_rsrc(Q + q_off, q_bytes), rdO = byte_rsrc(dO + q_off, q_bytes);
    const __amdgpu_buffer_rsrc_t rK = byte_rsrc(K + kv_off, kv_bytes), rV = byte_rsrc(V + kv_off, kv_bytes);

    const int k0 = kb * KB;
    const int key_local = wave * 32 + l32;
    const int my_key = k0 + key_local;         // key of this lane in S / P / dS

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
        // keys past N load as zeros; their columns of dK and dV are never stored
        const unsigned go = (unsigned)(k0 + r) * kv_row_bytes + sub * 64 + (((lane & 3) ^ dual_swz(r)) << 4);
        dma16_buf(rK, go, lds0 + seg * 1024);
        dma16_buf(rV, go, lds0 + KVB + seg * 1024);
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
    // the ring overwrites the K/V staging: everyone must have read it
    __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();

    // ---- query steps: for each query head g of the group, blocks
    // first..last in order (or the whole sequence reversed, see rev), so the
    // key blocks of one head that run at once read the same query blocks at
    // about the same time (L2 hits) ----
    // causal: queries k0 .. k0 + KB - 1 + window - 1 can see these keys
    // (query i sees keys j with i - window < j <= i; window >= N: plain causal)
    const int nsteps = (N + BR - 1) / BR;
    const int first = CAUSAL ? k0 / BR : 0;
    const int last = CAUSAL ? min(nsteps - 1, (k0 + KB - 2 + window) / BR) : nsteps - 1;
    const int nst = last - first + 1;          // per query head
    const int nst_all = G * nst;
    // causal workgroups of an even generation (those that start together)
    // walk their steps from the last query block down to the diagonal
    const bool rev = CAUSAL && !WIN && gen > 0 && !odd_generation(blockIdx.x, gen);
    auto step_of = [&](int it, int& g) {       // query block of step it, and its head
        if (rev) it = nst_all - 1 - it;
        g = it / nst;
        return first + (it - g * nst);
    };

    // direct loads of one step: SEG_QO segments of Q/dO per wave + the stats;
    // ld_off: byte offset of the lane's 16 bytes relative to the step's first row
    unsigned ld_off[SEG_QO];
#pragma unroll
    for (int i = 0; i < SEG_QO; ++i) {
        const int seg = wave * SEG_QO + i;
        const int sseg = seg % (QT / 1024);
        const int sub = sseg / (SUBQ / 1024), r = (sseg % (SUBQ / 1024)) * 16 + (lane >> 2);
        ld_off[i] = (unsigned)r * row_bytes + sub * 64 + (((lane & 3) ^ dual_swz(r)) << 4);
    }
    const unsigned st_lane = (unsigned)(((b * H + hk * G) * Npad + 4 * (lane & 15)) * 4 + ((lane & 16) ? delta_off : 0));
    // Direct loads of step `it`: where they go (uniform) and load i of them.  A
    // step past the last one reloads step 0 into the spare kilobyte instead.
    struct StepLoads {
        unsigned lds;                          // LDS byte offset of segment 0
        unsigned seg;                          // LDS stride per segment (0: spare)
        unsigned row0;                         // byte offset of its first Q/dO row
        unsigned st0;                          // byte offset of its statistics
    };
    auto step_loads = [&](int it) {
        const bool real = it < nst_all;
        int g;
        const int i0 = step_of(real ? it : 0, g) * BR;
        StepLoads sl;
        sl.lds = (unsigned)__builtin_amdgcn_readfirstlane(real ? lds0 + (it % NSTAGE) * STAGE : lds0 + RING);
        sl.seg = real ? 1024u : 0u;
        sl.row0 = (unsigned)__builtin_amdgcn_readfirstlane((int)((unsigned)i0 * row_bytes + (unsigned)g * 2 * D));
        sl.st0 = (unsigned)__builtin_amdgcn_readfirstlane((g * Npad + i0) * 4);
        return sl;
    };
    auto issue_load = [&](const StepLoads& sl, int i) {
        if (i < SEG_QO) {
            const int seg = wave * SEG_QO + i;
            dma16_buf(seg < QT / 1024 ? rQ : rdO, sl.row0 + ld_off[i], sl.lds + seg * sl.seg);
        } else {
            dma16(stats, st_lane + sl.st0, sl.lds + (2 * QT / 1024 + wave) * sl.seg);
        }
    };
    {
        const StepLoads s0 = step_loads(0), s1 = step_loads(1);
#pragma unroll
        for (int i = 0; i < DMA_W; ++i) issue_load(s0, i);
#pragma unroll
        for (int i = 0; i < DMA_W; ++i) issue_load(s1, i);
    }

    f32x16 dvacc[DT], dkacc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) {
        dvacc[i] = f32x16{};
        dkacc[i] = f32x16{};
    }

    // per-lane LDS offsets (within a stage) of the operand reads
    const int a_rd0 = l32 * 64 + ((hl ^ dual_swz(l32)) << 4);        // Q/dO rows, even c
    const int a_rd1 = l32 * 64 + (((2 + hl) ^ dual_swz(l32)) << 4);  // odd c

    // One query step (its position it in the sweep), masked or not.
    auto step = [&](int it, auto masked) {
        // 3 stages: this step's loads are done once at most one step's loads
        // are in flight; after the barrier nobody reads the stage of step
        // it - 1, which the loads of step it + 2 (spread over the units below)
        // refill.  4 stages (paired): even steps wait for every load in flight
        // (those of this step and the next), and their barrier retires all
        // reads of steps it - 2 and it - 1, whose stages the loads of steps
        // it + 2 and it + 3 refill; odd steps need neither.
        if constexpr (PAIRED) {
            if ((it & 1) == 0) {
                FA_WAIT_VMCNT(0);
                __builtin_amdgcn_s_barrier();
            }
        } else {
            FA_WAIT_VMCNT(DMA_W);
            __builtin_amdgcn_s_barrier();
        }
        FA_SYNC_POINT();

        int g_unused;
        const int i0 = step_of(it, g_unused) * BR;
        const StepLoads next = step_loads(it + 2);

        const lds_char* stage = L + (it % NSTAGE) * STAGE;
        const lds_char* qa0 = stage + a_rd0;
        const lds_char* qa1 = stage + a_rd1;
        const lds_char* t0 = stage + tr0;
        const lds_char* t1 = stage + tr1;
        const lds_char* sw = stage + 2 * QT + wave * 1024 + hl * 16;
        asm volatile("" : "+v"(qa0), "+v"(qa1), "+v"(t0), "+v"(t1), "+v"(sw));

        // Masking.  Queries past N need none: their padded statistics
        // (LSE = +inf, D = 0) give P = 0 and dS = 0.  Keys past N need none
        // either: column j of dV^T and dK^T only depends on column j of P and
        // dS, and those columns are never stored.  So only the causal mask
        // remains: the query of register r of half m, i0 + 4 hl + 32m +
        // 8(r>>2) + (r&3), must not precede the lane's key (nor, with a
        // sliding window, reach window rows past it).  It is applied on every
        // step, as a second copy of the step for the diagonal blocks would
        // cost more in register moves than the compares.
        const int lim_c = my_key - i0 - 4 * hl;
        const int lim_w = lim_c + window - 1;      // window: query < key + window
        // One step, software-pipelined by hand.  With one wave per SIMD
        // nothing else hides LDS latency, so the step is cut into NU units of
        // two MFMAs each; the operand reads of unit u + PF and the statistics
        // of a later softmax chunk are issued in unit u, and the softmax of one
        // 32-query half runs in pieces beside the products of the next units.
        // Scheduling fences between units keep the compiler from sinking the
        // reads back next to their MFMAs.
        //   units 0 .. DC-1:        S/dP of queries 0..31   (one chunk c each)
        //   units DC .. 2DC-1:      S/dP of queries 32..63
        //   units 2DC .. NU-1:      dV^T/dK^T, query chunk cq major, feature tile dt
        //   softmax of half 0 in units DC+1 .. 2DC, of half 1 in 2DC+1 .. 3DC,
        //   DC chunks of RC = 16/DC registers each
        auto body = [&](auto masked) {
            constexpr bool MASK = decltype(masked)::value;
            constexpr int NS = 2 * DC;                 // S/dP units
            constexpr int NU = NS + 4 * DT;            // all units
            constexpr int PF = D == 64 ? 1 : 3;        // prefetch distance in units
            constexpr int RC = 16 / DC;                // softmax registers per chunk
            static_assert(3 * DC <= NU, "softmax chunks fit in the step");
            bf16x8 opa[NU], opb[NU];                   // operands of each unit
            f32x4 lse4[2][4], dl4[2][4];
            f32x16 sacc[2], pacc[2];
            u32x4 pb[BR / 16], dsb[BR / 16];
            auto issue_reads = [&](auto ucon) {
                constexpr int u = decltype(ucon)::value;
                if constexpr (u < NS && u % DC == 0) {
                    // -D of half u / DC, in the C layout: it seeds dP's accumulator
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        dl4[u / DC][g] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
                            sw + 256 + (32 * (u / DC) + 8 * g) * 4);
                }
                if constexpr (u < NS) {
                    constexpr int m = u / DC, c = u % DC;
                    const lds_char* a = ((c & 1) ? qa1 : qa0) + (c >> 1) * SUBQ + m * 32 * 64;
                    opa[u] = lds_read_b128(a);
                    opb[u] = lds_read_b128(a + QT);
                } else if constexpr (u < NU) {
                    constexpr int cq = (u - NS) / DT, dt = (u - NS) % DT;
                    constexpr int off = dt * SUBQ + cq * 16 * 64;
                    opa[u] = __builtin_shufflevector(lds_read_tr16(t0 + QT + off), lds_read_tr16(t1 + QT + off),
                                                     0, 1, 2, 3, 4, 5, 6, 7);
                    opb[u] = __builtin_shufflevector(lds_read_tr16(t0 + off), lds_read_tr16(t1 + off),
                                                     0, 1, 2, 3, 4, 5, 6, 7);
                }
                // LSE of the softmax chunk that runs in unit u
                constexpr int m = u <= 2 * DC ? 0 : 1;
                constexpr int ch = u - (m == 0 ? DC + 1 : 2 * DC + 1);
                if constexpr (ch >= 0 && ch < DC && (ch * RC) % 4 == 0) {
                    constexpr int g = ch * RC / 4;
                    lse4[m][g] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(sw + (32 * m + 8 * g) * 4);
                }
            };
            auto softmax_chunk = [&](auto ucon) {
                constexpr int u = decltype(ucon)::value;
                constexpr int m = u <= 2 * DC ? 0 : 1;
                constexpr int ch = u - (m == 0 ? DC + 1 : 2 * DC + 1);
                if constexpr (ch >= 0 && ch < DC) {
#pragma unroll
                    for (int j = 0; j < RC; j += 2) {
                        const int r = ch * RC + j;     // registers r, r + 1
                        float pv[2], dsv[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int rr = r + e;
                            float x = __builtin_fmaf(sacc[m][rr], scale_log2, -lse4[m][rr >> 2][rr & 3]);
                            if constexpr (MASK) {
                                // hidden pairs get exp2(-inf) = 0, and so dS = 0 as dP is finite
                                const int off = 32 * m + 8 * (rr >> 2) + (rr & 3);
                                const bool vis = WIN ? (off >= lim_c) & (off <= lim_w) : off >= lim_c;
                                x = vis ? x : -INFINITY;
                            }
                            const float p = fast_exp2(x);
                            pv[e] = p;
                            dsv[e] = p * pacc[m][rr];      // pacc = dP - D
                        }
                        const int g = r >> 2;
                        pb[2 * m + (g >> 1)][2 * (g & 1) + ((r >> 1) & 1)] = pack_bf16x2(pv[0], pv[1]);
                        dsb[2 * m + (g >> 1)][2 * (g & 1) + ((r >> 1) & 1)] = pack_bf16x2(dsv[0], dsv[1]);
                    }
                }
            };
            auto products = [&](auto ucon) {
                constexpr int u = decltype(ucon)::value;
                if constexpr (u < NS) {
                    constexpr int m = u / DC, c = u % DC;
                    if constexpr (c == 0) {
                        sacc[m] = f32x16{};
                        pacc[m] = __builtin_shufflevector(
                            __builtin_shufflevector(dl4[m][0], dl4[m][1], 0, 1, 2, 3, 4, 5, 6, 7),
                            __builtin_shufflevector(dl4[m][2], dl4[m][3], 0, 1, 2, 3, 4, 5, 6, 7),
                            0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
                    }
                    sacc[m] = mfma32x32x16(opa[u], kreg[c], sacc[m]);
                    pacc[m] = mfma32x32x16(opb[u], vreg[c], pacc[m]);
                } else {
                    constexpr int cq = (u - NS) / DT, dt = (u - NS) % DT;
                    if constexpr (D == 128) {
                        mfma_acc(dvacc[dt], opa[u], pb[cq]);
                        mfma_acc(dkacc[dt], opb[u], dsb[cq]);
                    } else {
                        dvacc[dt] = mfma32x32x16(opa[u], __builtin_bit_cast(bf16x8, pb[cq]), dvacc[dt]);
                        dkacc[dt] = mfma32x32x16(opb[u], __builtin_bit_cast(bf16x8, dsb[cq]), dkacc[dt]);
                    }
                }
            };
            static_for<PF>([&](auto u) { issue_reads(u); });
            __builtin_amdgcn_sched_barrier(0);
            static_for<NU>([&](auto u) {
                constexpr int uu = decltype(u)::value;
                issue_reads(flag_int<uu + PF>{});
                // the direct loads of step it + 2, one every other unit
                if constexpr (uu == 1) FA_SYNC_POINT();
                if constexpr (uu % 2 == 1 && uu / 2 < DMA_W) issue_load(next, uu / 2);
                softmax_chunk(u);
                products(u);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        body(masked);
    };
    if constexpr (CAUSAL) {
        // Only two kinds of step need the mask's compares and select: those
        // whose queries start before the block's last key (one of them can
        // precede a key; the first nm steps of each query head's range), and
        // with a window those whose last query lies window rows or more past
        // the block's first key (from step sw on).  The others run in loops
        // of their own without it (one body per loop: no register copies).
        // When the sweep runs from the last query block down (never with a
        // window) the nm diagonal steps come last.
        const int nm = min(nst, (k0 + KB - 2) / BR - first + 1);
        const int sw = WIN ? min(nst, max(nm, (k0 + window) / BR - first)) : nst;
        for (int gi = 0; gi < G; ++gi) {
            const int base = gi * nst;
            const int u_lo = base + (rev ? 0 : nm);           // unmasked steps [u_lo, u_hi)
            const int u_hi = base + (rev ? nst - nm : sw);
#pragma clang loop unroll(disable)
            for (int it = base; it < u_lo; ++it) step(it, flag_t<true>{});
#pragma clang loop unroll(disable)
            for (int it = u_lo; it < u_hi; ++it) step(it, flag_t<false>{});
#pragma clang loop unroll(disable)
            for (int it = u_hi; it < base + nst; ++it) step(it, flag_t<true>{});
        }
    } else {
#pragma clang loop unroll(disable)
        for (int it = 0; it < nst_all; ++it) step(it, flag_t<false>{});
    }
    FA_WAIT_VMCNT(0);                          // the loads past the last step
    // the accumulators are read below by VALU after MFMAs the compiler does
    // not see (inline assembly): wait out the MFMA result latency
    FA_MFMA_DRAIN();

    // epilogue: dK = scale * (dK^T)^T, dV; C layout of dV^T / dK^T: lane = key
    // column, registers = feature rows 8g + 4h + t.  Both go out through the
    // wave's part of the ring, whole rows per store.
    static_assert(NW * 2 * RowStage<D>::BYTES <= RING, "row staging fits in the ring");
    __syncthreads();                           // every wave is done with the ring
    char* rk = smem + wave * 2 * RowStage<D>::BYTES;
    char* rv = rk + RowStage<D>::BYTES;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x16& kk = dkacc[dt];
            const f32x16& vv = dvacc[dt];
            RowStage<D>::put(rk, dt * 4 + g,
                             u32x2{pack_bf16x2(kk[g * 4] * scale, kk[g * 4 + 1] * scale),
                                   pack_bf16x2(kk[g * 4 + 2] * scale, kk[g * 4 + 3] * scale)});
            RowStage<D>::put(rv, dt * 4 + g,
                             u32x2{pack_bf16x2(vv[g * 4], vv[g * 4 + 1]), pack_bf16x2(vv[g * 4 + 2], vv[g * 4 + 3])});
        }
    const int kw = k0 + wave * 32;             // first key of this wave
    RowStage<D>::store(rk, dK + kv_off + (long)kw * kv_stride, kv_stride, N - kw);
    RowStage<D>::store(rv, dV + kv_off + (long)kw * kv_stride, kv_stride, N - kw);
}

// ---------------------------------------------------------------------------
// 3. dQ: query-block kernel
// ---------------------------------------------------------------------------
namespace bwdq {
constexpr int BR = 256;      // queries per workgroup (8 waves x 32)
constexpr int BC = 64;       // keys per K/V block
constexpr int NT = 512;
constexpr int NW = 8;
}  // namespace bwdq

// WIN: a sliding window narrower than N (causal only).  STATS: the kernel
// forms the row statistics itself from O, dO and the forward's LSE (D_i =
// dO_i . O_i, LSE_i log2 e), uses them, and writes both padded rows into
// lse2 / delta for the key-block kernel, which then runs after it; without
// STATS it reads them there, written by the preprocess kernel.
template <int D, bool CAUSAL, bool WIN, bool STATS>
__global__ __launch_bounds__(bwdq::NT, 1) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const __bf16* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ lse2, float* __restrict__ delta,
    __bf16* __restrict__ dQ, int H, int G, int N, int window, int Npad, float scale, float scale_log2,
    int nqb, int gen, int group) {
    using namespace bwdq;
    // K/V blocks resident in the LDS ring: 4 at d = 128, where one barrier
    // serves two blocks (129 KB of LDS), 3 at d = 64
    constexpr int NSTAGE = D == 128 ? 4 : 3;
    constexpr bool PAIRED = NSTAGE == 4;
    constexpr int DC = D / 16;
    constexpr int DT = D / 32;
    constexpr int TILE = BC * D * 2;           // one K or V block
    constexpr int STAGE = 2 * TILE;
    constexpr int SUB = BC * 64;               // sub-tile: BC rows x 32 features
    constexpr int SEGS = TILE / 1024;
    constexpr int SEG_W = SEGS / NW;           // segments per wave per tensor
    constexpr int SEG_SUB = SUB / 1024;
    static_assert(SEGS % NW == 0, "segments per wave");
    static_assert(2 * SEG_W <= 15, "vmcnt immediate");
    // the ring, then 1 KB that absorbs the direct loads of tiles past the last
    // one (every tile issues the same loads, so no branch is needed)
    __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE + 1024];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hl = lane >> 5;
    const int tg = lane >> 4, tj = lane & 15;

    int bh, qb;                                // causal: longest query blocks first
    order_blocks(blockIdx.x, gridDim.x, nqb, CAUSAL, true, bh, qb, group);
    const int b = bh / H, h = bh - b * H;
    const int row_stride = H * D;
    const long head_off = ((long)b * N * H + h) * D;
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
    const lds_char* L = as_lds(smem);
    // grouped-query attention: G query heads share one K/V head (G = 1: one each)
    const int Hkv = H / G;
    const unsigned kv_row_bytes = (unsigned)(Hkv * D) * 2u;
    const long kv_off = ((long)b * N * Hkv + h / G) * D;
    // K and V rows past N load as zeros: such a key then adds dS * 0 to dQ,
    // so ragged tails need no mask
    const unsigned kv_bytes = (unsigned)(N - 1) * kv_row_bytes + 2 * D;
    const __amdgpu_buffer_rsrc_t rK = byte_rsrc(K + kv_off, kv_bytes);
    const __amdgpu_buffer_rsrc_t rV = byte_rsrc(V + kv_off, kv_bytes);

    const int q0 = qb * BR;
    const int qw = q0 + wave * 32;
    const int my_q = qw + l32;
    const int q_rd = min(my_q, N - 1);         // rows past N: finite data, never stored

    // Key tiles t_lo .. ntiles-1 (causal: query i sees keys j with
    // i - window < j <= i; window >= N is plain causal).  Tiles every query of
    // the workgroup sees whole, [t_ulo, t_uhi), run unmasked; those on the
    // window edge or the diagonal are masked.  Keys past N need no mask.
    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kv_end + BC - 1) / BC;
    const int t_lo = CAUSAL ? max(0, q0 - window + 1) / BC : 0;
    const int t_uhi = CAUSAL ? max(t_lo, min(ntiles, (q0 + 1) / BC)) : ntiles;
    const int t_ulo = CAUSAL ? min(t_uhi, max(t_lo, (max(0, q0 + BR - window) + BC - 1) / BC)) : 0;
    // causal workgroups of an odd generation run their unmasked tiles from
    // the diagonal down (position t visits tile sweep_block(t))
    const bool rev = CAUSAL && !WIN && odd_generation(blockIdx.x, gen);

    unsigned ld_off[SEG_W];                    // lane's bytes relative to the tile's first row
#pragma unroll
    for (int i = 0; i < SEG_W; ++i) {
        const int seg = wave * SEG_W + i;
        const int sub = seg / SEG_SUB, r = (seg % SEG_SUB) * 16 + (lane >> 2);
        ld_off[i] = (unsigned)r * kv_row_bytes + sub * 64 + (((lane & 3) ^ dual_swz(r)) << 4);
    }
    // direct loads of tile t (a tile past the last one goes to the spare KB)
    auto issue_tile = [&](int t) {
        const bool real = t < ntiles;
        const unsigned kb = __builtin_amdgcn_readfirstlane(real ? lds0 + ((t - t_lo) % NSTAGE) * STAGE
                                                                : lds0 + NSTAGE * STAGE);
        const unsigned segb = real ? 1024u : 0u;
        const unsigned row0 = (unsigned)(real ? sweep_block(t, t_ulo, t_uhi, rev) * BC : 0) * kv_row_bytes;
#pragma unroll
        for (int i = 0; i < SEG_W; ++i) {
            const int seg = wave * SEG_W + i;
            dma16_buf(rK, row0 + ld_off[i], kb + seg * segb);
            dma16_buf(rV, row0 + ld_off[i], kb + (TILE / 1024 + seg) * segb);
        }
    };
    issue_tile(t_lo);
    issue_tile(t_lo + 1);

    // this lane's query: Q and dO as B operands (features 16c + 8hl ..), LSE, D
    bf16x8 qreg[DC], oreg[DC];
    {
        const __bf16* qs = Q + head_off + (long)q_rd * row_stride + 8 * hl;
        const __bf16* os = dO + head_off + (long)q_rd * row_stride + 8 * hl;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            qreg[c] = as_bf16x8(ld_global16(qs + 16 * c));
            oreg[c] = as_bf16x8(ld_global16(os + 16 * c));
        }
    }
    float lq, dq_row;                          // LSE log2 e and -D of this lane's query
    if constexpr (STATS) {
        // D = dO . O over the lane's half of the features (those of its Q and
        // dO registers), then the other half from the partner lane
        const __bf16* os_ = O + head_off + (long)q_rd * row_stride + 8 * hl;
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const u32x4 ov = ld_global16(os_ + 16 * c);
            const u32x4 gv = __builtin_bit_cast(u32x4, oreg[c]);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                part = __builtin_fmaf(__builtin_bit_cast(float, ov[w] << 16),
                                      __builtin_bit_cast(float, gv[w] << 16), part);
                part = __builtin_fmaf(__builtin_bit_cast(float, ov[w] & 0xffff0000u),
                                      __builtin_bit_cast(float, gv[w] & 0xffff0000u), part);
            }
        }
        const float dsum = halves_sum(part);
        // rows past N (padding): LSE = +inf and D = 0, so P = 0 and dS = 0
        const bool live = my_q < N;
        const float lrow = LSE[(long)bh * N + q_rd];
        lq = live ? lrow * kLog2e : INFINITY;
        dq_row = live ? -dsum : 0.f;
        if (hl == 0 && my_q < Npad) {
            lse2[(long)bh * Npad + my_q] = lq;
            delta[(long)bh * Npad + my_q] = dq_row;
        }
    } else {
        lq = lse2[(long)bh * Npad + q_rd];
        dq_row = delta[(long)bh * Npad + q_rd];
    }
    // consume the loads here so no wait for them lands inside the loop
#pragma unroll
    for (int c = 0; c < DC; ++c) asm volatile("" : "+v"(qreg[c]), "+v"(oreg[c]));
    asm volatile("" : "+v"(lq), "+v"(dq_row));

    f32x16 dqacc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) dqacc[i] = f32x16{};

    const int a_rd0 = l32 * 64 + ((hl ^ dual_swz(l32)) << 4);        // K/V rows, even c
    const int a_rd1 = l32 * 64 + (((2 + hl) ^ dual_swz(l32)) << 4);  // odd c
    const int tr_r0 = 4 * (tg >> 1) + (tj >> 2), tr_r1 = tr_r0 + 8;
    const int tr_cl = 2 * (tg & 1) + ((tj & 3) >> 1);
    const int tr0 = tr_r0 * 64 + ((tr_cl ^ dual_swz(tr_r0)) << 4) + ((tj & 1) << 3);
    const int tr1 = tr_r1 * 64 + ((tr_cl ^ dual_swz(tr_r1)) << 4) + ((tj & 1) << 3);

    // one K/V tile (sweep position t; masked positions are their own tile):
    // wait for its loads, start those of position t + 2, then
    // S^T = K Q^T, dP^T = V dO^T (lane = query), dS^T, dQ^T += K^T dS^T
    auto tile = [&](int t, auto masked) {
        constexpr bool MASK = decltype(masked)::value;
        // 3 stages: wait for this block (the next may be in flight); the
        // barrier retires the reads of block t - 1, whose stage the loads of
        // block t + 2 refill.  4 stages (paired): even blocks (counted from
        // t_lo) wait for both blocks in flight, and their barrier retires the
        // reads of blocks t - 2 and t - 1, whose stages blocks t + 2 and t + 3
        // refill; odd blocks need neither.
        if constexpr (PAIRED) {
            if (((t - t_lo) & 1) == 0) {
                FA_WAIT_VMCNT(0);
                __builtin_amdgcn_s_barrier();
            }
        } else {
            FA_WAIT_VMCNT(2 * SEG_W);
            __builtin_amdgcn_s_barrier();
        }
        FA_SYNC_POINT();
        if constexpr (MASK) issue_tile(t + 2);

        const int j0 = t * BC;
        // every key after this wave's queries, or before all of their windows
        if (MASK && (j0 > qw + 31 || j0 + BC - 1 < qw - window + 1)) return;
        const lds_char* stage = L + ((t - t_lo) % NSTAGE) * STAGE;
        const lds_char* ka0 = stage + a_rd0;
        const lds_char* ka1 = stage + a_rd1;
        const lds_char* kt0 = stage + tr0;
        const lds_char* kt1 = stage + tr1;
        asm volatile("" : "+v"(ka0), "+v"(ka1), "+v"(kt0), "+v"(kt1));
        // dP^T's accumulator starts at -D (one per lane: the lane's query),
        // so it ends as dP^T - D
        // feature-chunk major: four independent accumulator chains (S^T and
        // dP^T of both 32-key tiles), with the K and V operands of chunk
        // c + 1 read while the products of chunk c run
        f32x16 s[2], dp[2];
        bf16x8 kop[2][2], vop[2][2];
        auto read_kv = [&](int c, int buf) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const lds_char* a = ((c & 1) ? ka1 : ka0) + (c >> 1) * SUB + kt * 32 * 64;
                kop[buf][kt] = lds_read_b128(a);
                vop[buf][kt] = lds_read_b128(a + TILE);
            }
        };
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s[kt] = f32x16{};
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[kt][r] = dq_row;
        }
        read_kv(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            if (c + 1 < DC) read_kv(c + 1, (c + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                s[kt] = mfma32x32x16(kop[c & 1][kt], qreg[c], s[kt]);
                dp[kt] = mfma32x32x16(vop[c & 1][kt], oreg[c], dp[kt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // unmasked tiles start the loads of tile t + 2 here, behind the S^T and
        // dP^T reads, rather than as a burst at the top (masked tiles may
        // return early, so they issue first)
        if constexpr (!MASK) {
            FA_SYNC_POINT();
            issue_tile(t + 2);
        }
        // dS^T = P^T (dP^T - D), P^T = exp2(S^T scale log2e - LSE log2e); on
        // diagonal tiles keys after the lane's query get exp2(-inf) = 0
        u32x4 dsb[4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt][r] = __builtin_fmaf(s[kt][r], scale_log2, -lq);
        // a masked tile masks only the waves that do not see all of it
        if constexpr (MASK) {
            const bool whole = j0 + BC - 1 <= qw && (!WIN || j0 >= qw + 32 - window);
            if (__builtin_expect(!whole, 1)) {
                const int lim_c = my_q - j0 - 4 * hl;  // key = j0 + 4hl + off: key <= q <=> off <= lim_c
                const int lim_w = lim_c - window + 1;  // window: key > q - window <=> off >= lim_w
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = kt * 32 + (r >> 2) * 8 + (r & 3);
                        s[kt][r] = (off <= lim_c && (!WIN || off >= lim_w)) ? s[kt][r] : -INFINITY;
                    }
            }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float d0 = fast_exp2(s[kt][r]) * dp[kt][r];
                const float d1 = fast_exp2(s[kt][r + 1]) * dp[kt][r + 1];
                dsb[kt * 2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(d0, d1);
            }
        // dQ^T += K^T dS^T; A operand = K^T from the row-major K block.  Key
        // chunk major: DT independent chains, the K^T operands of chunk cc + 1
        // read while the products of chunk cc run
        bf16x8 kto[2][DT];
        auto read_kt = [&](int cc, int buf) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int off = dt * SUB + cc * 16 * 64;
                kto[buf][dt] = __builtin_shufflevector(lds_read_tr16(kt0 + off), lds_read_tr16(kt1 + off), 0, 1,
                                                       2, 3, 4, 5, 6, 7);
            }
        };
        read_kt(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            if (cc + 1 < 4) read_kt(cc + 1, (cc + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                dqacc[dt] = mfma32x32x16(kto[cc & 1][dt], __builtin_bit_cast(bf16x8, dsb[cc]), dqacc[dt]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
#pragma clang loop unroll(disable)
    for (int t = t_lo; t < t_ulo; ++t) tile(t, flag_t<CAUSAL>{});
#pragma clang loop unroll(disable)
    for (int t = t_ulo; t < t_uhi; ++t) tile(t, flag_t<false>{});
    if constexpr (CAUSAL) {
#pragma clang loop unroll(disable)
        for (int t = t_uhi; t < ntiles; ++t) tile(t, flag_t<true>{});
    }
    FA_WAIT_VMCNT(0);                          // the loads past the last tile

    // epilogue: dQ = scale * dQ^T^T -> bf16; lane = query, registers = features;
    // out through the wave's part of the ring, whole rows per store
    static_assert(NW * RowStage<D>::BYTES <= NSTAGE * STAGE, "row staging fits in the ring");
    __syncthreads();                           // every wave is done with the ring
    char* rs = smem + wave * RowStage<D>::BYTES;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            RowStage<D>::put(rs, dt * 4 + g,
                             u32x2{pack_bf16x2(dqacc[dt][g * 4] * scale, dqacc[dt][g * 4 + 1] * scale),
                                   pack_bf16x2(dqacc[dt][g * 4 + 2] * scale, dqacc[dt][g * 4 + 3] * scale)});
    RowStage<D>::store(rs, dQ + head_off + (long)qw * row_stride, row_stride, N - qw);
}

int bwd_rows_padded(int N) { return (N + bwd::ROWPAD - 1) / bwd::ROWPAD * bwd::ROWPAD; }

hipError_t launch_bwd_preprocess(const void* o, const void* dout, const float* lse, int B, int H,
                                 int N, int d, float* lse2, float* delta, hipStream_t stream) {
    auto Op = static_cast<const __bf16*>(o);
    auto dOp = static_cast<const __bf16*>(dout);
    const int Npad = bwd_rows_padded(N);
    const long rows = (long)B * H * Npad;
    const int rpb = 256 / (d / 8) * bwd::PRE_RPT;
    const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
    if (d == 128)
        hipLaunchKernelGGL((bwd_pre_kernel<128>), grid, dim3(256), 0, stream, Op, dOp, lse, lse2, delta, H, N, Npad, rows);
    else
        hipLaunchKernelGGL((bwd_pre_kernel<64>), grid, dim3(256), 0, stream, Op, dOp, lse, lse2, delta, H, N, Npad, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk,
                           void* dv, int B, int H, int Hkv, int N, int d, float scale, bool causal,
                           int window, const float* lse2, const float* delta, hipStream_t stream) {
    const int G = H / Hkv;
    const int win = effective_window(window, N);
    auto Qp = static_cast<const __bf16*>(q);
    auto Kp = static_cast<const __bf16*>(k);
    auto Vp = static_cast<const __bf16*>(v);
    auto dOp = static_cast<const __bf16*>(dout);
    auto dKp = static_cast<__bf16*>(dk);
    auto dVp = static_cast<__bf16*>(dv);
    const int Npad = bwd_rows_padded(N);
    const int nkb = (N + bwd::KB - 1) / bwd::KB;
    const dim3 grid((unsigned)(B * Hkv * nkb)), block(bwd::NT);
    const float sl2 = scale * kLog2e;
    const int delta_off = (int)((const char*)delta - (const char*)lse2);
    const bool narrow = causal && win < N;     // a window that hides keys
#define FA_BWD_LAUNCH(DD, CC, WW)                                                                      \
    do {                                                                                               \
        const void* kf = (const void*)bwd_dkdv_kernel<DD, CC, WW>;                                     \
        const Schedule sc = causal ? causal_schedule(kf, bwd::NT, nkb, d, N, narrow, stream) : Schedule{0, 1}; \
        hipLaunchKernelGGL((bwd_dkdv_kernel<DD, CC, WW>), grid, block, 0, stream, Qp, Kp, Vp, dOp, lse2, \
                           delta_off, dKp, dVp, H, G, N, win, Npad, scale, sl2, nkb, sc.gen, sc.group); \
    } while (0)
    if (d == 128) {
        if (narrow) FA_BWD_LAUNCH(128, true, true);
        else if (causal) FA_BWD_LAUNCH(128, true, false);
        else FA_BWD_LAUNCH(128, false, false);
    } else {
        if (narrow) FA_BWD_LAUNCH(64, true, true);
        else if (causal) FA_BWD_LAUNCH(64, true, false);
        else FA_BWD_LAUNCH(64, false, false);
    }
#undef FA_BWD_LAUNCH
    return hipGetLastError();
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
                         int B, int H, int Hkv, int N, int d, float scale, bool causal, int window,
                         const void* o, const float* lse, float* lse2, float* delta, hipStream_t stream) {
    const int G = H / Hkv;
    const int win = effective_window(window, N);
    auto Qp = static_cast<const __bf16*>(q);
    auto Kp = static_cast<const __bf16*>(k);
    auto Vp = static_cast<const __bf16*>(v);
    auto dOp = static_cast<const __bf16*>(dout);
    auto Op = static_cast<const __bf16*>(o);
    auto dQp = static_cast<__bf16*>(dq);
    const int Npad = bwd_rows_padded(N);
    const int nqb = (N + bwdq::BR - 1) / bwdq::BR;
    const dim3 grid((unsigned)(B * H * nqb)), block(bwdq::NT);
    const float sl2 = scale * kLog2e;
    const bool narrow = causal && win < N;
    const bool stats = o != nullptr;
#define FA_BWDQ_LAUNCH(DD, CC, WW)                                                                  \
    do {                                                                                            \
        const void* kf = stats ? (const void*)bwd_dq_kernel<DD, CC, WW, true>                      \
                               : (const void*)bwd_dq_kernel<DD, CC, WW, false>;                    \
        const Schedule sc = causal ? causal_schedule(kf, bwdq::NT, nqb, d, N, narrow, stream) : Schedule{0, 1}; \
        if (stats)                                                                                  \
            hipLaunchKernelGGL((bwd_dq_kernel<DD, CC, WW, true>), grid, block, 0, stream, Qp, Kp,  \
                               Vp, dOp, Op, lse, lse2, delta, dQp, H, G, N, win, Npad, scale, sl2,  \
                               nqb, sc.gen, sc.group);                                              \
        else                                                                                        \
            hipLaunchKernelGGL((bwd_dq_kernel<DD, CC, WW, false>), grid, block, 0, stream, Qp, Kp, \
                               Vp, dOp, Op, lse, lse2, delta, dQp, H, G, N, win, Npad, scale, sl2,  \
                               nqb, sc.gen, sc.group);                                              \
    } while (0)
    if (d == 128) {
        if (narrow) FA_BWDQ_LAUNCH(128, true, true);
        else if (causal) FA_BWDQ_LAUNCH(128, true, false);
        else FA_BWDQ_LAUNCH(128, false, false);
    } else {
        if (narrow) FA_BWDQ_LAUNCH(64, true, true);
        else if (causal) FA_BWDQ_LAUNCH(64, true, false);
        else FA_BWDQ_LAUNCH(64, false, false);
    }
#undef FA_BWDQ_LAUNCH
    return hipGetLastError();
}

}  // namespace fa
