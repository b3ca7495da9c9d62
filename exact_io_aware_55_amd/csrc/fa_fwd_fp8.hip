// Forward pass of exact attention with FP8 inputs on gfx950.
//
// Method as in the bf16 forward (explainer page "Flash Attention", section
// "Tiling"; glossary page "Flash Attention", section "How it works"): one
// workgroup per block of queries, K/V blocks streamed through LDS, a running
// row maximum and sum, O rescaled when the maximum grows, O and
// LSE = m + ln l written once.  FP8 is the precision that the pages name for
// FlashAttention-3 (explainer, "Versionen: Flash Attention 2 und Flash
// Attention 3"; glossary, "FlashAttention-2, -3 and -4").
//
// Inputs are OCP E4M3 codes with one fp32 descale factor per (batch, head)
// for each of Q, K and V: the real value is code * descale.  Both products
// run on the fp8 matrix core (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulate):
//  * S^T = K Q^T from the codes; scale * descale_q * descale_k * log2(e) is
//    folded into the one FMA before each exponential;
//  * O^T += V^T P^T with P rounded to E4M3 (P <= 2^8 < 448: the running
//    maximum is raised whenever a block's probabilities would exceed that); the row sum l adds the unrounded fp32 P, and
//    descale_v / l is applied once at the end.  O is written in bf16.
//
// Layout (per workgroup: 8 waves x 32 queries, K/V blocks of 128 keys at
// d = 128, 64 at d = 64):
//  * a lane keeps its query's codes as the B operand of S^T = K Q^T: 32 bytes
//    (features 64 m + 32 h .. +31, h the lane half) per 64-feature MFMA; K is
//    read with the same byte order, two 16-byte LDS reads per MFMA;
//  * K and V blocks sit in LDS as [D/64 sub-tiles][BC rows][64 bytes] with
//    16-byte chunks XOR-swizzled per row.  V is read with ds_read_b64_tr_b8:
//    a 16-lane group reads 8 consecutive rows x 16 bytes and lane j receives
//    byte column j of those rows.  A lane's P bytes hold keys
//    16 c + 8 a + 4 h + t (c chunk, a = e >> 2, t = e & 3); the direct loads
//    place key k at LDS row k with bits 2 and 3 swapped, so rows
//    16 c + 8 h + e are exactly those keys and the V^T operand needs no
//    register shuffling;
//  * blocks stream through a 3-stage ring of direct global -> LDS loads
//    issued two blocks ahead, one barrier per block, as in the bf16 kernel.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace fwd8 {
constexpr int BR = 256;     // queries per workgroup (8 waves x 32)
constexpr int NT = 512;     // threads per workgroup
constexpr int NW = NT / 64; // waves
constexpr int NSTAGE = 3;   // K/V blocks resident in the LDS ring
}  // namespace fwd8

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// 32x32x64 E4M3 x E4M3 -> fp32.  Format selectors 0 (E4M3 for both
// operands); zero block-scale operands select the unscaled instruction.
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ u32x4 lds_read_u128(const lds_char* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}
__device__ __forceinline__ i32x2 lds_read_tr8(const lds_char* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}
__device__ __forceinline__ i32x8 join16(const u32x4& lo, const u32x4& hi) {
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// K rows are read 16 bytes per lane down 32 consecutive rows; the swizzle
// puts rows R, R+4, R+8, R+12 of one logical chunk on different banks.
__device__ __forceinline__ int k8_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }
// V is read by 32 lanes as 8 rows x 2 adjacent chunks: flipping chunk bit 1
// with row bit 2 makes those 16 (row, chunk) pairs cover all 64 banks.
__device__ __forceinline__ int v8_swz(int row) { return ((row >> 2) & 1) << 1; }

template <int D, bool CAUSAL, bool POS>
__global__ __launch_bounds__(fwd8::NT, 1) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ q_descale, const float* __restrict__ k_descale,
    const float* __restrict__ v_descale, __bf16* __restrict__ O, float* __restrict__ LSE, int H, int G,
    int N, int window, float scale_log2, int nqb) {
    using namespace fwd8;
    // keys per K/V block: 128 at d = 128 (halves the per-block barrier, load
    // and loop work against the short fp8 products; measured 10% faster),
    // 64 at d = 64
    constexpr int BC = D == 128 ? 128 : 64;
    constexpr int TILE = BC * D;               // bytes of one K or V block
    constexpr int STAGE = 2 * TILE;            // K then V
    constexpr int SUB = BC * 64;               // one 64-feature sub-tile
    constexpr int DK = D / 64;                 // MFMAs over the feature dim (k = 64)
    constexpr int DT = D / 32;                 // 32-row tiles of O^T
    constexpr int SEGS = TILE / 1024;          // 1 KB segments per tensor and block
    constexpr int SEG_SUB = SUB / 1024;        // segments per sub-tile
    constexpr int NL = 2 * SEGS / NW;          // direct loads per wave and block
    constexpr int KT = BC / 32;                // 32-key score tiles per block
    constexpr int KP = BC / 64;                // 64-key P V products per feature tile
    static_assert((2 * SEGS) % NW == 0 && NL >= 1, "segments per wave");
    static_assert(NL <= 15, "vmcnt immediate");
    // the ring, then 1 KB for the direct loads past the last block; at least
    // the epilogue's row staging (32 KB at d = 64, more than that ring)
    constexpr int SMEM = NSTAGE * STAGE + 1024 > NW * RowStage<D>::BYTES ? NSTAGE * STAGE + 1024
                                                                         : NW * RowStage<D>::BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hl = lane >> 5;

    int bh, qb;                                // causal: longest query blocks first
    order_blocks(blockIdx.x, gridDim.x, nqb, CAUSAL, true, bh, qb, causal_group<D>());
    const int b = bh / H, h = bh - b * H;
    const int Hkv = H / G, hk = h / G;
    const int row_stride = H * D;              // elements between rows (Q bytes, O bf16)
    const long head_off = ((long)b * N * H + h) * D;
    const int q0 = qb * BR;
    const int qw = q0 + wave * 32;
    const int my_q = qw + l32;

    const float dq = q_descale[bh], dk = k_descale[b * Hkv + hk], dv = v_descale[b * Hkv + hk];
    if (!(dq > 0.f && dk > 0.f && dv > 0.f && __builtin_isfinite(dq) && __builtin_isfinite(dk) &&
          __builtin_isfinite(dv))) {
        // a descale factor that is not positive and finite: NaN rows
        if (my_q < N) {
            __bf16* dst = O + head_off + (long)my_q * row_stride;
            for (int d = hl * (D / 2); d < (hl + 1) * (D / 2); ++d) dst[d] = (__bf16)NAN;
            if (hl == 0) LSE[(long)bh * N + my_q] = NAN;
        }
        return;
    }
    const float sl2 = scale_log2 * dq * dk;

    const unsigned kv_row_bytes = (unsigned)(Hkv * D);
    const long kv_off = ((long)b * N * Hkv + hk) * D;
    // rows past N read zeros (range-checked loads); their scores are masked
    const unsigned kv_bytes = (unsigned)(N - 1) * kv_row_bytes + D;
    const __amdgpu_buffer_rsrc_t rK = byte_rsrc(K + kv_off, kv_bytes);
    const __amdgpu_buffer_rsrc_t rV = byte_rsrc(V + kv_off, kv_bytes);

    // Key blocks as in the bf16 kernel: [t_lo, t_ulo) and [t_uhi, ntiles)
    // masked (window edge; diagonal or ragged last block), [t_ulo, t_uhi) not.
    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kv_end + BC - 1) / BC;
    const int t_lo = CAUSAL ? max(0, q0 - window + 1) / BC : 0;
    const int t_uhi = max(t_lo, min(N / BC, CAUSAL ? (q0 + 1) / BC : ntiles));
    const int t_ulo = CAUSAL ? min(t_uhi, max(t_lo, (max(0, q0 + BR - window) + BC - 1) / BC)) : 0;

    // Direct loads: wave w fills 1 KB segments w NL .. w NL + NL - 1 of the
    // stage (K's SEGS segments, then V's).  Lane i writes bytes
    // [16 i, 16 i + 16) of its segment: LDS row 16 (seg % SEG_SUB) + i / 4 of
    // sub-tile seg / SEG_SUB, physical chunk i % 4.
    unsigned ld_off[NL], ld_dst[NL];
    bool ld_v[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int s = wave * NL + i;
        const bool is_v = s >= SEGS;
        const int seg = is_v ? s - SEGS : s;
        const int sub = seg / SEG_SUB, r = (seg % SEG_SUB) * 16 + lane / 4;
        const int key = is_v ? kslot_pos(r) : r;
        const int chunk = (lane & 3) ^ (is_v ? v8_swz(r) : k8_swz(r));
        ld_off[i] = (unsigned)key * kv_row_bytes + sub * 64 + (chunk << 4);
        ld_dst[i] = (unsigned)s * 1024u;
        ld_v[i] = is_v;
    }
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
    auto issue_tile = [&](int t) {
        const bool real = t < ntiles;
        const unsigned kb = __builtin_amdgcn_readfirstlane(real ? lds0 + ((t - t_lo) % NSTAGE) * STAGE
                                                                : lds0 + NSTAGE * STAGE);
        const unsigned row0 = (unsigned)(real ? t * BC : 0) * kv_row_bytes;
#pragma unroll
        for (int i = 0; i < NL; ++i)
            dma16_buf(ld_v[i] ? rV : rK, row0 + ld_off[i], kb + (real ? ld_dst[i] : 0u));
    };

    issue_tile(t_lo);
    issue_tile(t_lo + 1);

    // this lane's query codes (rows past N read row N-1; never stored)
    i32x8 qreg[DK];
    {
        const uint8_t* src = Q + head_off + (long)min(my_q, N - 1) * row_stride + 32 * hl;
#pragma unroll
        for (int m = 0; m < DK; ++m) qreg[m] = join16(ld_global16(src + 64 * m), ld_global16(src + 64 * m + 16));
    }
#pragma unroll
    for (int m = 0; m < DK; ++m) asm volatile("" : "+v"(qreg[m]));

    f32x16 oacc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
    // packed E4M3 P of a block (the B operands of O^T += V^T P^T), carried
    // from block to block so that each packing starts from a live register
    i32x8 pw[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) pw[j] = i32x8{};
    // running maximum (log2 units): raised only when a block's probabilities
    // grow too large (see below), so P = exp2(x - m) stays <= 256 < 448
    float m_run = -INFINITY;
    float l_run = 0.f;
    constexpr float masked = POS ? -INFINITY : INFINITY;

    // per-lane LDS offsets within a stage
    const int k_rd0 = l32 * 64 + (((2 * hl) ^ k8_swz(l32)) << 4);
    const int k_rd1 = l32 * 64 + (((2 * hl + 1) ^ k8_swz(l32)) << 4);
    const int tr_j = lane & 15, tr_g = (lane >> 4) & 1;
    const int tr_row = 8 * hl + (tr_j >> 1);
    const int v_rd0 = TILE + tr_row * 64 + (((0 + tr_g) ^ v8_swz(tr_row)) << 4) + 8 * (tr_j & 1);
    const int v_rd1 = TILE + tr_row * 64 + (((2 + tr_g) ^ v8_swz(tr_row)) << 4) + 8 * (tr_j & 1);

    auto block = [&](int t, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        FA_WAIT_VMCNT(NL);
        __builtin_amdgcn_s_barrier();
        FA_SYNC_POINT();
        if constexpr (MASK) issue_tile(t + 2);

        const int j0 = t * BC;
        if (MASK && CAUSAL && (j0 > qw + 31 || j0 + BC - 1 < qw - window + 1)) return;
        const lds_char* stage = as_lds(smem) + ((t - t_lo) % NSTAGE) * STAGE;
        const lds_char* kb0 = stage + k_rd0;
        const lds_char* kb1 = stage + k_rd1;
        const lds_char* vb0 = stage + v_rd0;
        const lds_char* vb1 = stage + v_rd1;
        asm volatile("" : "+v"(kb0), "+v"(kb1), "+v"(vb0), "+v"(vb1));
        // S^T = K Q^T for the block's 32-key tiles
        f32x16 s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            s[kt] = f32x16{};
#pragma unroll
            for (int m = 0; m < DK; ++m) {
                const int o = m * SUB + kt * 32 * 64;
                s[kt] = mfma_fp8(join16(lds_read_u128(kb0 + o), lds_read_u128(kb1 + o)), qreg[m], s[kt]);
            }
        }
        if constexpr (!MASK) {
            FA_SYNC_POINT();
            issue_tile(t + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MASK) {
            const int lim_n = N - j0 - 4 * hl;
            const int lim_c = my_q - j0 - 4 * hl;
            const int lim_w = lim_c - window + 1;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kt * 32 + (r >> 2) * 8 + (r & 3);
                    const bool vis = off < lim_n && (!CAUSAL || (off <= lim_c && off >= lim_w));
                    s[kt][r] = vis ? s[kt][r] : masked;
                }
        }
        // P = exp2(x - m) against the running maximum as it stands; l sums the
        // fp32 values, the product uses E4M3.  Byte 16 kt + r of the packed
        // operand holds register r of tile kt.  A lane whose block sum exceeds
        // kSumMax (so some P might exceed 2^8), or whose row has no maximum
        // yet, sends the wave through the slow path: block maximum, rescale of
        // O and l, exponentials again.  Every P that reaches the E4M3 product
        // is then at most 2^8 < 448, and O, l and LSE all use the same m.
        constexpr float kSumMax = 256.f;
        float ls0, ls1;
        auto exps = [&](float m_sub) {
            ls0 = 0.f;
            ls1 = 0.f;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    float p[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        p[e] = fast_exp2(__builtin_fmaf(s[kt][r + e], sl2, -m_sub));
                        if constexpr (MASK) p[e] = s[kt][r + e] == masked ? 0.f : p[e];
                    }
                    ls0 += p[0] + p[2];
                    ls1 += p[1] + p[3];
                    // the two converts overwrite both halves of the word, so
                    // its previous contents (last block's) are never seen
                    const int e8 = (kt & 1) * 4 + (r >> 2);
                    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pw[kt >> 1][e8], false);
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
                    pw[kt >> 1][e8] = w;
                }
        };
        exps(m_run == -INFINITY ? 0.f : m_run);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(ls0 + ls1 <= kSumMax) || m_run == -INFINITY) != 0, 0)) {
            float mx = s[0][0];
            if constexpr (POS) {
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
                mx = halves_max(mx);
            } else {
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fminf(mx, s[kt][r]);
                mx = halves_min(mx);
            }
            const float m_new = fmaxf(m_run, mx * sl2);
            // a row that has seen no visible key yet has l = 0 and O = 0: any
            // finite alpha will do, and -inf - -inf is NaN
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < DT; ++i) oacc[i] *= alpha;
            exps(m_run == -INFINITY ? 0.f : m_run);
        }
        l_run += ls0 + ls1;
        __builtin_amdgcn_sched_barrier(0);
        // O^T += V^T P^T: four transposing reads give the 32 key bytes of one
        // feature row, in the order of the P bytes
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < KP; ++j) {
                const lds_char* vb = ((dt & 1) ? vb1 : vb0) + (dt >> 1) * SUB + j * 64 * 64;
                const i32x2 a0 = lds_read_tr8(vb);
                const i32x2 a1 = lds_read_tr8(vb + 16 * 64);
                const i32x2 a2 = lds_read_tr8(vb + 32 * 64);
                const i32x2 a3 = lds_read_tr8(vb + 48 * 64);
                const i32x8 va = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
                oacc[dt] = mfma_fp8(va, pw[j], oacc[dt]);
            }
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma clang loop unroll(disable)
    for (int t = t_lo; t < t_ulo; ++t) block(t, std::true_type{});
#pragma clang loop unroll(disable)
    for (int t = t_ulo; t < t_uhi; ++t) block(t, std::false_type{});
#pragma clang loop unroll(disable)
    for (int t = t_uhi; t < ntiles; ++t) block(t, std::true_type{});
    FA_WAIT_VMCNT(0);

    // ---- epilogue: O = descale_v * O / l, LSE = m ln2 + ln l ----
    const float l_tot = halves_sum(l_run);
    const float f = dv / l_tot;
    // O rows through the wave's part of the LDS, whole rows per store
    __syncthreads();                           // every wave is done with the ring
    char* rs = smem + wave * RowStage<D>::BYTES;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t w0 = pack_bf16x2(oacc[dt][g * 4 + 0] * f, oacc[dt][g * 4 + 1] * f);
            const uint32_t w1 = pack_bf16x2(oacc[dt][g * 4 + 2] * f, oacc[dt][g * 4 + 3] * f);
            RowStage<D>::put(rs, dt * 4 + g, u32x2{w0, w1});
        }
    RowStage<D>::store(rs, O + head_off + (long)qw * row_stride, row_stride, N - qw);
    if (my_q < N && hl == 0) LSE[(long)bh * N + my_q] = m_run * kLn2 + __logf(l_tot);
}

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                          const float* k_descale, const float* v_descale, void* o, float* lse, int B,
                          int H, int Hkv, int N, int d, float scale, bool causal, int window,
                          hipStream_t stream) {
    const int G = H / Hkv;
    const int nqb = (N + fwd8::BR - 1) / fwd8::BR;
    const dim3 grid((unsigned)(B * H * nqb)), block(fwd8::NT);
    const float sl2 = scale * kLog2e;
    auto Qp = static_cast<const uint8_t*>(q);
    auto Kp = static_cast<const uint8_t*>(k);
    auto Vp = static_cast<const uint8_t*>(v);
    auto Op = static_cast<__bf16*>(o);
    const int win = effective_window(window, N);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, stream, Qp, Kp, Vp, q_descale, k_descale, v_descale, Op,
                           lse, H, G, N, win, sl2, nqb);
    };
    const bool pos = sl2 >= 0.f;
    if (d == 128) {
        if (causal) pos ? go(fwd_fp8_kernel<128, true, true>) : go(fwd_fp8_kernel<128, true, false>);
        else pos ? go(fwd_fp8_kernel<128, false, true>) : go(fwd_fp8_kernel<128, false, false>);
    } else {
        if (causal) pos ? go(fwd_fp8_kernel<64, true, true>) : go(fwd_fp8_kernel<64, true, false>);
        else pos ? go(fwd_fp8_kernel<64, false, true>) : go(fwd_fp8_kernel<64, false, false>);
    }
    return hipGetLastError();
}

}  // namespace fa
