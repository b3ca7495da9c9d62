// Shared device helpers for the gfx950 attention kernels: vector types, the
// bf16 MFMA wrapper, global/LDS vector access and the LDS layout functions.
//
// MFMA lane layout used throughout (v_mfma_f32_32x32x16_bf16, 64 lanes):
//   A (32 x 16):  lane l holds row (l & 31), eight k-slots 8*(l >> 5) + e
//   B (16 x 32):  lane l holds column (l & 31), eight k-slots 8*(l >> 5) + e
//   C (32 x 32):  lane l holds column (l & 31); register r holds row
//                 8*(r >> 2) + 4*(l >> 5) + (r & 3)
// A contraction only needs A and B to agree on which data sits in which
// k-slot, so the kernels are free to place keys (or queries) in k-slots in
// any order, as long as both operands use the same order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// acc += a * b on a 32x32x16 bf16 MFMA with the accumulator held in AGPRs.
// The d = 128 backward keeps dV^T and dK^T (128 registers) there so that the
// VGPRs stay free for the score tiles (and vector instructions issued beside
// an MFMA cost less with its accumulator in AGPRs).  Written as inline assembly because the compiler picks one register
// form for all MFMAs of a kernel.  The compiler cannot see the hazards of an
// MFMA inside assembly, so callers must (a) leave the MFMA result latency
// before any vector instruction reads the accumulator (explicit s_nop), and
// (b) not feed it VGPRs written by the two preceding vector instructions.
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const u32x4& b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// wait states after inline-assembly MFMAs before their accumulators are read
#define FA_MFMA_DRAIN() asm volatile("s_nop 15\n\ts_nop 15" ::: "memory")

// 16-byte direct load through a buffer resource (buffer_load_dwordx4 ... lds):
// as dma16, but the offset is checked against the resource's byte range and
// lanes outside it read zeros, so tiles past the last row need no clamping.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc(const void* base, unsigned bytes) {
    // raw buffer: stride 0, range in bytes, 32-bit data format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rsrc, unsigned offset, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(offset), "s"(rsrc), "s"(lds_base)
                 : "memory", "m0");
}

// compile-time constants for generic lambdas
template <bool B>
struct flag_t {
    static constexpr bool value = B;
};
template <int I>
struct flag_int {
    static constexpr int value = I;
};
// f(flag_int<0>{}), ..., f(flag_int<N-1>{}) in order, fully unrolled
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_from(F&& f) {
    if constexpr (I < N) {
        f(flag_int<I>{});
        static_for_from<I + 1, N>(f);
    }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_from<0, N>(f);
}

// Maps a linear workgroup id to (head, query block) so that the workgroups the
// hardware places on one XCD (ids congruent mod 8) take a contiguous range of
// query blocks: those share K/V of the same heads and hit the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    const int per = nblocks >> 3, rem = nblocks & 7;
    const int x = bid & 7, i = bid >> 3;
    return x * per + (x < rem ? x : rem) + i;
}

// (head, block) of a workgroup.  Ids the hardware sends to one XCD (ids
// congruent mod 8) cover whole heads, so their K/V (or Q/dO) stay in that
// XCD's L2.  With a causal mask the work of a block depends on its index:
// `desc` says the longest block has the highest index (query blocks) rather
// than index 0 (key blocks).  When every XCD's share is a whole number of
// heads, the XCD takes its heads `group` at a time: the longest block of each
// head of the group, then the next longest, and so on, so no long block
// starts near the end of the grid.  Otherwise heads are taken one at a time,
// each longest block first.  The launcher picks `group` (causal_schedule):
// one head at a time where a head's streamed operands exceed the L2, so
// that a generation of workgroups (odd_generation) covers as much of one
// head as it can; pairs of heads at d = 128 and all heads at d = 64 below
// that, which measured fastest there (pairs made the d = 128 causal backward
// 4.7% faster than all heads at once; at d = 64 pairs made the causal
// forward up to 12% slower).  The FP8 forward uses causal_group.
template <int D>
constexpr int causal_group() { return D == 128 ? 2 : 1 << 20; }

// Sweep direction of a causal workgroup.  A causal block's range of key (or
// query) blocks depends on its index, so the workgroups an XCD runs at once
// end at different times and their successors start one by one.  Ids on one
// XCD (bid >> 3 = position in its sequence) start in generations of `gen`
// workgroups, as many as the XCD holds at once: the first generation starts
// together, the next one by one as the first ends, the third together again
// when the second ends, and so on.  Workgroups that start together stay in
// step if they sweep from the far end of their ranges toward the diagonal
// (all read block 0, then 1, ...); workgroups that start one by one stay in
// step if they sweep from the diagonal outward, because each starts as far
// along the shared sweep as its range is shorter than its predecessor's.
// Either way the workgroups of a head running at once read the same block at
// about the same time, and the XCD's L2 serves the re-reads.  Result: odd
// generation, i.e. started one by one (gen = 0: no alternation).
__device__ __forceinline__ bool odd_generation(int bid, int gen) {
    return gen > 0 && (((bid >> 3) / gen) & 1) != 0;
}
// Block visited at sweep position t: blocks [ulo, uhi) in reverse order when
// rev is set, any other t as it is
__device__ __forceinline__ int sweep_block(int t, int ulo, int uhi, bool rev) {
    return rev && t >= ulo && t < uhi ? ulo + uhi - 1 - t : t;
}
__device__ __forceinline__ void order_blocks(int bid, int nblocks, int nb, bool causal, bool desc, int& bh,
                                             int& blk, int group) {
    int rank;
    if (causal && nblocks % (8 * nb) == 0) {
        const int nh = nblocks / (8 * nb);     // heads per XCD
        const int x = bid & 7, i = bid >> 3;
        const int grp = nh < group ? nh : group;
        const int gi = i / (grp * nb), j = i - gi * (grp * nb);
        const int gsz = min(grp, nh - gi * grp);   // the last group may be smaller
        rank = j / gsz;
        bh = x * nh + gi * grp + (j - rank * gsz);
    } else {
        const int logical = xcd_remap(bid, nblocks);
        bh = logical / nb;
        rank = logical - bh * nb;
    }
    blk = causal && desc ? nb - 1 - rank : rank;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
// LDS (address space 3) byte pointers, for reads whose offsets should fold
// into the instruction's immediate field
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ bf16x8 lds_read_b128(const lds_char* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p));
}
__device__ __forceinline__ bf16x4 lds_read_tr16(const lds_char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}
__device__ __forceinline__ const lds_char* as_lds(const void* p) {
    return (const lds_char*)(p);
}
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Row-major bf16 output through LDS.  A wave holds 32 rows x D features with
// one row per lane (lane & 31) and, of 16-byte chunk c (features 8c .. 8c + 7),
// the four features 8c + 4 (lane >> 5) .. + 3 in registers: the layout of a
// transposed 32x32 MFMA result.  Stored from there, each store instruction
// would put 16 bytes into each of 32 rows, and the L2 may write a 128-byte
// line back before its other pieces arrive (partial writes that add bytes,
// depending on timing).  So the rows go to the wave's LDS region and come
// back with D / 8 lanes per row: every store instruction then writes whole
// rows.  Chunk c of row r sits at chunk c ^ (r mod D / 8), and the 8-byte half
// a lane writes is flipped when bit 3 of its row is set, so that each group
// of 16 lanes of an 8-byte write (rows r .. r + 15, one chunk) covers 128
// distinct bytes of the 32 banks; the reads swap those rows' halves back.
// The region must not be in use by other waves.
template <int D>
struct RowStage {
    static constexpr int BYTES = 32 * D * 2;   // LDS bytes per wave
    static constexpr int NCH = D / 8;          // 16-byte chunks per row
    static constexpr int RPI = 64 / NCH;       // rows per store instruction
    __device__ __forceinline__ static int at(int r, int c) { return r * (2 * D) + ((c ^ (r & (NCH - 1))) << 4); }
    // The lane index is formed afresh (mbcnt) in put and store, so that no
    // value derived from it has to stay live, or spill, through the main loop.
    __device__ __forceinline__ static int lane_id() {
        return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    }
    // the lane's 8 bytes of chunk c of its row
    __device__ __forceinline__ static void put(void* region, int c, u32x2 v) {
        const int lane = lane_id();
        const int half = (lane >> 5) ^ ((lane >> 3) & 1);
        auto p = (__attribute__((address_space(3))) char*)(region) + at(lane & 31, c) + (half << 3);
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(p) = v;
    }
    // rows 0 .. nrows - 1 to dst + r * stride elements; nrows is the same
    // for the whole wave (all LDS reads are issued before the first store)
    __device__ __forceinline__ static void store(const void* region, __bf16* dst, long stride, int nrows) {
        constexpr int NI = 32 / RPI;
        const int lane = lane_id();
        const int rr = lane / NCH, c = lane % NCH;
        u32x4 v[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const u32x4 w = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                as_lds(region) + at(i * RPI + rr, c));
            // the RPI rows of one read share bit 3 (RPI is 4 or 8)
            v[i] = ((i * RPI) & 8) ? __builtin_shufflevector(w, w, 2, 3, 0, 1) : w;
        }
        __bf16* p = dst + (long)rr * stride + 8 * c;
        if (nrows >= 32) {
#pragma unroll
            for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(p + (long)i * RPI * stride) = v[i];
        } else {
#pragma unroll
            for (int i = 0; i < NI; ++i)
                if (i * RPI + rr < nrows) *reinterpret_cast<u32x4*>(p + (long)i * RPI * stride) = v[i];
        }
    }
};

// 16-byte direct global -> LDS load (global_load_lds_dwordx4): every lane
// reads 16 bytes at base + offset and the wave writes them to LDS at
// lds_base + 16 * lane.  Issued through asm so the compiler does not order
// later LDS reads behind it (it cannot tell which LDS bytes a DMA writes);
// callers wait on vmcnt themselves.  M0 carries the LDS base; nothing else
// in these kernels uses M0.
__device__ __forceinline__ unsigned lds_offset(const void* p) {
    return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void dma16(const void* base, unsigned offset, unsigned lds_base) {
    // the base must be wave-uniform; readfirstlane puts it in SGPRs.  The
    // builtin returns a signed int: widen through unsigned, or a low half
    // with bit 31 set would sign-extend over the high half.
    const unsigned long long b = reinterpret_cast<unsigned long long>(base);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
    const unsigned long long sb = ((unsigned long long)hi << 32) | (unsigned long long)lo;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(offset), "s"(sb), "s"(lds_base)
                 : "memory", "m0");
}
// s_waitcnt vmcnt(n) only (expcnt and lgkmcnt left alone), n <= 15
#define FA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))

// Synchronisation check build (compiled with -DFA_DEBUG_SYNC, the library
// libfa_sync.so): at the start of every K/V block or query step and before
// every refill of an LDS ring stage, each wave waits for all of its memory
// operations and meets the other waves at a barrier.  The pipelines then run
// without any overlap of loads and reads; outputs must equal the normal
// build's bit for bit, so a difference shows a missing wait or barrier.
#ifdef FA_DEBUG_SYNC
#define FA_SYNC_POINT()                    \
    do {                                   \
        __builtin_amdgcn_s_waitcnt(0);     \
        __builtin_amdgcn_s_barrier();      \
    } while (0)
#else
#define FA_SYNC_POINT() \
    do {                \
    } while (0)
#endif

// Packs two floats into one dword of two bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// Key (or query) order inside one 16-wide k-chunk.  The C layout gives a lane
// the rows 8g + 4h + t (g, t in 0..3, h = lane half); taking registers
// 8c..8c+7 of a C tile as the B operand of the next product places row
// 16c' + 8a + 4h + t (a = e >> 2, t = e & 3) in k-slot 8h + 4a + t.  The
// matching A operand must therefore store index 8a + 4b + t of a chunk at
// position 8b + 4a + t: bits 2 and 3 of the index swap places.
__device__ __forceinline__ int kslot_pos(int idx) {
    return (idx & ~15) | (((idx >> 2) & 1) << 3) | (((idx >> 3) & 1) << 2) | (idx & 3);
}

// Combines a per-lane value with the lane 32 apart (the other half of the
// same MFMA column) using v_permlane32_swap: r[0] is the value of lane l & 31,
// r[1] that of lane 32 + (l & 31).
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float halves_min(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
    return fminf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Swizzle of 16-byte chunks in 64-byte LDS rows for tiles read both ways:
// 16 bytes per lane down 32 consecutive rows (ds_read_b128) and transposed
// (ds_read_tr16_b64, 4 consecutive rows x 32 bytes per 16-lane group).
// chunk' = chunk ^ (R2 | (R1 ^ R3) << 1) keeps both patterns at the minimum
// number of LDS cycles for 128-byte/clock banking.
__device__ __forceinline__ int dual_swz(int row) {
    return ((row >> 2) & 1) | ((((row >> 1) ^ (row >> 3)) & 1) << 1);
}

}  // namespace fa
