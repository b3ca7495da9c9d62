// Forward pass of exact attention on gfx950 (bf16 MFMA path and fp32 path).
//
// Method (explainer page "Flash Attention", section "Tiling"; glossary page
// "Flash Attention", section "How it works"): a workgroup owns one block of
// queries, streams the key/value blocks of its head through LDS, keeps a
// running row maximum m and sum l, rescales the partial output by
// exp(m_old - m_new) whenever the maximum grows, divides by l once at the end
// and writes only O and one statistic per row (LSE = m + ln l).
//
// bf16 kernel layout (per workgroup: 8 waves, 256 queries):
//  * each wave owns 32 queries and keeps them in registers as the B operand of
//    S^T = K Q^T, so a lane holds the scores of ONE query against 16 keys of
//    each 32-key MFMA tile.  The row max/sum are in-lane reductions plus one
//    exchange between the two lane halves.
//  * P^T stays in registers: after exp and the bf16 conversion, registers of
//    the S^T accumulator are directly the B operand of O^T += V^T P^T.
//  * K and V are staged row-major in LDS (64-byte rows of 32 features, 16-byte
//    chunks XOR-swizzled per row); V^T comes from transposing LDS reads
//    (ds_read_b64_tr_b16) with keys in the k-slot order of the P^T registers.
//  * K/V blocks (128 keys at d = 128, 64 at d = 64) stream through an LDS
//    ring (2 and 3 stages) by direct global -> LDS loads issued one or two
//    blocks ahead: one barrier per block.
//  * exponentials are v_exp_f32 (base 2) with scale * log2(e) folded into one
//    FMA per score, which turns S^T in place into the exponents
//    x = scale log2(e) s - m (masked keys: -inf).
//  * the running maximum is raised lazily: the exponentials run against it
//    with no block maximum, and a block sum that grows too large sends the
//    wave through a rescaling slow path.  At d = 64 the kernel is held to 128
//    registers per wave, so four waves share each SIMD (two workgroups per
//    CU); the few values that do not fit are spilled outside the block loop.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace fwd {
constexpr int BR = 256;     // queries per workgroup (8 waves x 32)
constexpr int NT = 512;     // threads per workgroup
constexpr int NW = NT / 64; // waves
}  // namespace fwd

// LDS layout of one K or V block (BC keys): D/32 sub-tiles [BC keys][32
// features] with 64-byte rows (4 chunks of 16 bytes), chunk c of row R stored
// at chunk c ^ swizzle(R).
//  * K is read 16 bytes per lane down 32 consecutive rows (A operand of
//    S^T = K Q^T); its swizzle ((R >> 1) ^ (R >> 2)) & 3 keeps the rows read
//    together on distinct banks.
//  * V is read with ds_read_tr16_b64 (A operand of O^T = V^T P^T): each
//    16-lane group reads 4 consecutive rows x 32 bytes; swizzle 2((R >> 1) & 1).
// Both swizzles depend only on the lane for every read of a block, so each
// read is a per-lane base plus an immediate offset.
__device__ __forceinline__ int k_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }
__device__ __forceinline__ int v_swz(int row) { return ((row >> 1) & 1) << 1; }

// WIN: a sliding window narrower than N (causal only); without it the
// causal mask is one compare per score
template <int D, bool CAUSAL, bool WIN>
__global__ __launch_bounds__(fwd::NT, D == 64 ? 4 : 1) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int H, int G, int N, int window, float scale_log2,
    int nqb, int gen, int group) {
    using namespace fwd;
    // keys per K/V block and blocks resident in the LDS ring: 128 keys in a
    // 2-stage ring at d = 128 (half the per-block barrier, load and loop work;
    // 129 KB of LDS), 64 keys in a 3-stage ring at d = 64.  Loads run
    // NSTAGE - 1 blocks ahead.
    constexpr int BC = D == 128 ? 128 : 64;
    constexpr int NSTAGE = D == 128 ? 2 : 3;
    constexpr int KT = BC / 32;                // 32-key score tiles per block
    constexpr int TILE = BC * D * 2;           // one K or V block
    constexpr int STAGE = 2 * TILE;            // K then V
    constexpr int SUB = BC * 64;               // one sub-tile (32 features)
    constexpr int DC = D / 16;                 // k-chunks over the feature dim
    constexpr int DT = D / 32;                 // 32-row tiles of O^T (= sub-tiles)
    constexpr int SEGS = TILE / 1024;          // 1 KB segments per block (one wave load each)
    constexpr int SEG_W = SEGS / NW;           // segments per wave per tensor
    constexpr int SEG_SUB = SUB / 1024;        // segments per sub-tile
    static_assert(SEGS % NW == 0, "segments per wave");

    static_assert((NSTAGE - 1) * 2 * SEG_W <= 15, "vmcnt immediate");
    // the ring, then 1 KB that absorbs the direct loads of blocks past the
    // last one (every block issues the same loads, so no branch is needed)
    __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE + 1024];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hl = lane >> 5;

    const int nblocks = gridDim.x;
    int bh, qb;                                // causal: longest query blocks first
    order_blocks(blockIdx.x, nblocks, nqb, CAUSAL, true, bh, qb, group);
    const int b = bh / H, h = bh - b * H;
    const int row_stride = H * D;              // elements between sequence rows (N*H*D < 2^31)
    const long head_off = ((long)b * N * H + h) * D;
    // grouped-query attention: G query heads share one K/V head (G = 1: one each)
    const int Hkv = H / G;
    const unsigned kv_row_bytes = (unsigned)(Hkv * D) * 2u;
    const long kv_off = ((long)b * N * Hkv + h / G) * D;
    // K and V rows past N read zeros (range-checked loads); their scores are
    // masked, so they get weight exactly 0
    const unsigned kv_bytes = (unsigned)(N - 1) * kv_row_bytes + 2 * D;
    const __amdgpu_buffer_rsrc_t rK = byte_rsrc(K + kv_off, kv_bytes);
    const __amdgpu_buffer_rsrc_t rV = byte_rsrc(V + kv_off, kv_bytes);

    const int q0 = qb * BR;
    const int qw = q0 + wave * 32;             // first query of this wave
    const int my_q = qw + l32;

    // Key blocks t_lo .. ntiles-1.  Causal: query i sees keys j with
    // i - window < j <= i (window >= N: plain causal), so blocks wholly before
    // the block's first window are skipped.  Blocks every query of the
    // workgroup sees whole, [t_ulo, t_uhi), run unmasked; the others (window
    // edge, causal diagonal, a ragged last block) are masked.
    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kv_end + BC - 1) / BC;
    const int t_lo = CAUSAL ? max(0, q0 - window + 1) / BC : 0;
    const int t_uhi = max(t_lo, min(N / BC, CAUSAL ? (q0 + 1) / BC : ntiles));
    const int t_ulo = CAUSAL ? min(t_uhi, max(t_lo, (max(0, q0 + BR - window) + BC - 1) / BC)) : 0;
    // causal workgroups of an odd generation run their unmasked blocks from
    // the diagonal down (position t visits block sweep_block(t)); the masked
    // blocks and every other workgroup go in ascending order
    const bool rev = CAUSAL && !WIN && odd_generation(blockIdx.x, gen);

    // Direct global -> LDS loads of one K/V block: each wave fills SEG_W 1 KB
    // segments of K and of V; lane i writes bytes [16 i, 16 i + 16) of its
    // segment (row 16 (seg % SEG_SUB) + i / 4 of sub-tile seg / SEG_SUB,
    // physical chunk i % 4), so it loads the global chunk that belongs there.
    unsigned k_off[SEG_W], v_off[SEG_W];       // relative to the block's first row
#pragma unroll
    for (int i = 0; i < SEG_W; ++i) {
        const int seg = wave * SEG_W + i;
        const int sub = seg / SEG_SUB, r = (seg % SEG_SUB) * 16 + lane / 4;
        k_off[i] = (unsigned)r * kv_row_bytes + sub * 64 + (((lane & 3) ^ k_swz(r)) << 4);
        v_off[i] = (unsigned)r * kv_row_bytes + sub * 64 + (((lane & 3) ^ v_swz(r)) << 4);
    }
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
    auto issue_tile = [&](int t) {
        const bool real = t < ntiles;
        const unsigned kb = __builtin_amdgcn_readfirstlane(real ? lds0 + ((t - t_lo) % NSTAGE) * STAGE
                                                                : lds0 + NSTAGE * STAGE);
        const unsigned segb = real ? 1024u : 0u;
        const unsigned row0 = (unsigned)(real ? sweep_block(t, t_ulo, t_uhi, rev) * BC : 0) * kv_row_bytes;
#pragma unroll
        for (int i = 0; i < SEG_W; ++i) {
            const int seg = wave * SEG_W + i;
            dma16_buf(rK, row0 + k_off[i], kb + seg * segb);
            dma16_buf(rV, row0 + v_off[i], kb + (TILE / 1024 + seg) * segb);
        }
    };

#pragma unroll
    for (int i = 0; i < NSTAGE - 1; ++i) issue_tile(t_lo + i);

    // Queries of this lane, as B-operand chunks of S^T = K Q^T.  Rows past N
    // read row N-1 (finite data whose results are never stored).
    bf16x8 qreg[DC];
    {
        const __bf16* src = Q + head_off + (long)min(my_q, N - 1) * row_stride + 8 * hl;
#pragma unroll
        for (int c = 0; c < DC; ++c) qreg[c] = as_bf16x8(ld_global16(src + 16 * c));
    }
    // Consume the Q registers here (the empty asm reads them), so the compiler
    // waits for the Q loads before the loop rather than inside it, where the
    // wait would also stall on the block prefetch.
#pragma unroll
    for (int c = 0; c < DC; ++c) asm volatile("" : "+v"(qreg[c]));

    f32x16 oacc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
    // Running max of scale*log2(e)*s for this lane's query (log2 units),
    // raised only when a block's probabilities grow too large (see below).
    float m_run = -INFINITY;
    float l_run = 0.f;         // running sum over this lane's half of the keys

    // per-lane LDS byte offsets of the operand reads (within a stage)
    const int k_rd0 = l32 * 64 + ((hl ^ k_swz(l32)) << 4);          // even k-chunks c
    const int k_rd1 = l32 * 64 + (((2 + hl) ^ k_swz(l32)) << 4);    // odd k-chunks c
    const int tr_g = lane >> 4, tr_j = lane & 15;
    const int tr_row = 4 * (tr_g >> 1) + (tr_j >> 2);                // + 16 cc + 8 w
    const int v_rd = TILE + tr_row * 64 + (((2 * (tr_g & 1) + ((tr_j & 3) >> 1)) ^ v_swz(tr_row)) << 4) +
                     ((tr_j & 1) << 3);

    // One K/V block (sweep position t; masked positions are their own
    // block): wait for its loads (the next block may still be in
    // flight), make every wave's part visible (the barrier also retires all
    // reads of block t - 1, whose stage the loads of block t + 2 refill), then
    // S^T = K Q^T, the online softmax and O^T += V^T P^T.
    // NL: the block's first NL 32-key tiles are computed; on a masked causal
    // block the tiles whose keys all follow the wave's last query are
    // invisible to every query of the wave and are skipped (their P is 0)
    auto block = [&](int t, auto mask_tag, auto nl_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr int NL = decltype(nl_tag)::value;
        const int j0 = t * BC;
        // per-iteration bases; the empty asm keeps the compiler from
        // hoisting base + offset sums into separate registers, so the
        // offsets fold into the LDS instructions
        const lds_char* stage = as_lds(smem) + ((t - t_lo) % NSTAGE) * STAGE;
        const lds_char* kb0 = stage + k_rd0;
        const lds_char* kb1 = stage + k_rd1;
        const lds_char* vb = stage + v_rd;
        asm volatile("" : "+v"(kb0), "+v"(kb1), "+v"(vb));
        // S^T = K Q^T for the block's 32-key tiles
        // feature-chunk major: NL independent accumulator chains, and the K
        // operands of chunk c + 1 read while the products of chunk c run
        f32x16 s[NL];
        bf16x8 kop[2][NL];
        auto read_k = [&](int c, bf16x8* dst) {
#pragma unroll
            for (int kt = 0; kt < NL; ++kt)
                dst[kt] = lds_read_b128(((c & 1) ? kb1 : kb0) + (c >> 1) * SUB + kt * 32 * 64);
        };
#pragma unroll
        for (int kt = 0; kt < NL; ++kt) s[kt] = f32x16{};
        read_k(0, kop[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            if (c + 1 < DC) read_k(c + 1, kop[(c + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kt = 0; kt < NL; ++kt) s[kt] = mfma32x32x16(kop[c & 1][kt], qreg[c], s[kt]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // unmasked blocks start the loads of block t + NSTAGE - 1 here,
        // behind the K reads, rather than as a burst at the top
        if constexpr (!MASK) {
            FA_SYNC_POINT();
            issue_tile(t + NSTAGE - 1);
        }
        // keep the V reads below the softmax (register pressure)
        __builtin_amdgcn_sched_barrier(0);
        // x = scale log2(e) s - m_sub in place, the exponent of P against the
        // running maximum as it stands; a masked key gets x = -inf, so its P
        // is exactly 0 (also when scale == 0)
        const float m_sub = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
        for (int kt = 0; kt < NL; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt][r] = __builtin_fmaf(s[kt][r], scale_log2, -m_sub);
        // A masked block masks only the waves that do not see all of it:
        // causal, keys after the query or before its window (a query never
        // sees a key past N, so that needs no test of its own); otherwise
        // keys past N.  Key of register r = j0 + 4 hl + off(kt, r), off a
        // constant: compare the constant with one per-lane limit.
        if constexpr (MASK) {
            const bool whole = CAUSAL ? (j0 + BC - 1 <= qw && (!WIN || j0 >= qw + 32 - window))
                                      : j0 + BC <= N;
            if (__builtin_expect(!whole, 1)) {
                const int lim_n = N - j0 - 4 * hl;        // visible iff off < lim_n
                const int lim_c = my_q - j0 - 4 * hl;     // causal: off <= lim_c
                const int lim_w = lim_c - window + 1;     // window: off >= lim_w
#pragma unroll
                for (int kt = 0; kt < NL; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = kt * 32 + (r >> 2) * 8 + (r & 3);
                        const bool vis = CAUSAL ? off <= lim_c && (!WIN || off >= lim_w) : off < lim_n;
                        s[kt][r] = vis ? s[kt][r] : -INFINITY;
                    }
            }
        }
        // P = exp2(x): the row sum accumulates the fp32 values (so LSE keeps
        // fp32 accuracy), the PV product uses P rounded to bf16
        u32x4 pw[2 * NL];
        float ls0, ls1;
        auto exps = [&]() {
            float la[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < NL; ++kt)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = fast_exp2(s[kt][r]);
                    const float p1 = fast_exp2(s[kt][r + 1]);
                    la[(r >> 1) & 1] += p0;
                    la[2 + ((r >> 1) & 1)] += p1;
                    pw[kt * 2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(p0, p1);
                }
            ls0 = la[0] + la[1];
            ls1 = la[2] + la[3];
        };
        // Raise the running maximum to the block's (rows with no visible key
        // yet keep -inf), rescale O and l, and shift x to the new maximum.
        // O, l and LSE all use the same m, so the result is exact whichever m
        // was used.
        auto raise = [&](float mx) {
            const float m_new = fmaxf(m_run, m_sub + mx);
            // a row that has seen no visible key yet (possible at a sliding
            // window's edge while other rows of the wave rescale) has l = 0
            // and O = 0: any finite alpha will do, and -inf - -inf is NaN
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < DT; ++i) oacc[i] *= alpha;
            const float delta = m_new == -INFINITY ? 0.f : m_new - m_sub;
#pragma unroll
            for (int kt = 0; kt < NL; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kt][r] -= delta;
        };
        auto block_max = [&]() {
            float mx = s[0][0];
#pragma unroll
            for (int kt = 0; kt < NL; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
            return halves_max(mx);
        };
        // Exponentials first, against the running maximum.  A lane whose
        // block sum exceeds 2^16, or whose row has no maximum yet, sends the
        // wave through the slow path (block maximum, rescale, exponentials
        // again).  A lane sums BC / 2 <= 64 values of its query, so its sum
        // passes 2^16 only through an x above 8: the slow path always raises
        // the maximum, and on the fast path P < 2^16 keeps P, l and O far
        // from the fp32 range.
        exps();
        if (__builtin_expect(
                __builtin_amdgcn_ballot_w64(!(ls0 + ls1 <= 65536.f) || m_run == -INFINITY) != 0, 0)) {
            raise(block_max());
            exps();
        }
        l_run += ls0 + ls1;
        __builtin_amdgcn_sched_barrier(0);
        // O^T += V^T P^T; the A operand (8 keys of one feature row) comes
        // from two transposing reads: keys 16cc + 4h + 0..3 and +8.
        // key-chunk major: DT independent accumulator chains, and the V^T
        // operands of chunk cc + 1 read while the products of chunk cc run
        bf16x8 vop[2][DT];
        auto read_v = [&](int cc, bf16x8* dst) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const lds_char* a0 = vb + dt * SUB + cc * 16 * 64;
                dst[dt] = __builtin_shufflevector(lds_read_tr16(a0), lds_read_tr16(a0 + 8 * 64), 0, 1, 2, 3,
                                                  4, 5, 6, 7);
            }
        };
        read_v(0, vop[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cc = 0; cc < 2 * NL; ++cc) {
            if (cc + 1 < 2 * NL) read_v(cc + 1, vop[(cc + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                oacc[dt] = mfma32x32x16(vop[cc & 1][dt], __builtin_bit_cast(bf16x8, pw[cc]), oacc[dt]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto step = [&](int t, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        FA_WAIT_VMCNT((NSTAGE - 2) * 2 * SEG_W);
        __builtin_amdgcn_s_barrier();
        FA_SYNC_POINT();
        if constexpr (MASK) issue_tile(t + NSTAGE - 1);  // masked blocks may return early

        const int j0 = t * BC;
        // every key after this wave's queries, or before all of their windows
        if (MASK && CAUSAL && (j0 > qw + 31 || j0 + BC - 1 < qw - window + 1)) return;
        if constexpr (MASK && CAUSAL) {
            const int nl = min(KT, (qw + 31 - j0) / 32 + 1);   // >= 1 after the test above
            if (nl >= KT) block(t, mask_tag, flag_int<KT>{});
            else if constexpr (KT == 4) {
                if (nl == 3) block(t, mask_tag, flag_int<3>{});
                else if (nl == 2) block(t, mask_tag, flag_int<2>{});
                else block(t, mask_tag, flag_int<1>{});
            } else {
                block(t, mask_tag, flag_int<1>{});
            }
        } else {
            block(t, mask_tag, flag_int<KT>{});
        }
    };
#pragma clang loop unroll(disable)
    for (int t = t_lo; t < t_ulo; ++t) step(t, std::true_type{});
#pragma clang loop unroll(disable)
    for (int t = t_ulo; t < t_uhi; ++t) step(t, std::false_type{});
#pragma clang loop unroll(disable)
    for (int t = t_uhi; t < ntiles; ++t) step(t, std::true_type{});
    FA_WAIT_VMCNT(0);                          // the loads past the last block

    // ---- epilogue: O = O / l, LSE = m ln2 + ln l ----
    const float l_tot = halves_sum(l_run);
    const float inv = 1.f / l_tot;
    // O rows through the wave's part of the ring, whole rows per store
    // (rows past N hold finite or non-finite values and are not stored)
    static_assert(NW * RowStage<D>::BYTES <= NSTAGE * STAGE, "row staging fits in the ring");
    __syncthreads();                           // every wave is done with the ring
    char* rs = smem + wave * RowStage<D>::BYTES;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t w0 = pack_bf16x2(oacc[dt][g * 4 + 0] * inv, oacc[dt][g * 4 + 1] * inv);
            const uint32_t w1 = pack_bf16x2(oacc[dt][g * 4 + 2] * inv, oacc[dt][g * 4 + 3] * inv);
            RowStage<D>::put(rs, dt * 4 + g, u32x2{w0, w1});
        }
    RowStage<D>::store(rs, O + head_off + (long)qw * row_stride, row_stride, N - qw);
    if (my_q < N && hl == 0) LSE[(long)bh * N + my_q] = m_run * kLn2 + __logf(l_tot);
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
                           int H, int Hkv, int N, int d, float scale, bool causal, int window,
                           hipStream_t stream) {
    const int G = H / Hkv;
    const int nqb = (N + fwd::BR - 1) / fwd::BR;
    const dim3 grid((unsigned)(B * H * nqb)), block(fwd::NT);
    const float sl2 = scale * kLog2e;
    auto Qp = static_cast<const __bf16*>(q);
    auto Kp = static_cast<const __bf16*>(k);
    auto Vp = static_cast<const __bf16*>(v);
    auto Op = static_cast<__bf16*>(o);
    const int win = effective_window(window, N);
    const bool narrow = causal && win < N;
    auto go = [&](auto kern) {
        const Schedule sc = causal ? causal_schedule((const void*)kern, fwd::NT, nqb, d, N, narrow, stream)
                                   : Schedule{0, 1};
        hipLaunchKernelGGL(kern, grid, block, 0, stream, Qp, Kp, Vp, Op, lse, H, G, N, win, sl2, nqb, sc.gen,
                           sc.group);
    };
    if (d == 128) {
        if (!causal) go(fwd_bf16_kernel<128, false, false>);
        else narrow ? go(fwd_bf16_kernel<128, true, true>) : go(fwd_bf16_kernel<128, true, false>);
    } else {
        if (!causal) go(fwd_bf16_kernel<64, false, false>);
        else narrow ? go(fwd_bf16_kernel<64, true, true>) : go(fwd_bf16_kernel<64, true, false>);
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
