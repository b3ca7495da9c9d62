/*
 * fa.h -- exact attention (FlashAttention) forward and backward on AMD gfx950.
 *
 * What is computed.  For every batch b and head h, with X_bh the N x d matrix
 * X[b, :, h, :]:
 *
 *     S = scale * Q K^T                       (optionally causal: key j is
 *                                              visible to query i iff j <= i)
 *     P = softmax over each row of S          (online, block by block)
 *     O = P V,   LSE_i = log(sum_j exp(S_ij))  (natural log)
 *
 * The forward streams K/V blocks through on-chip memory and keeps a running
 * row maximum and sum, rescaling the partial output when the maximum grows;
 * only O and one statistic per row go back to memory.  (Explainer page
 * "Flash Attention", sections "Tiling" and "Speicherbedarf und
 * Laufzeitverhalten"; glossary page "Flash Attention", section "How it
 * works".)  The per-row statistic is exported as LSE = m + ln(l), which
 * carries the row maximum and row sum that the pages keep.
 *
 * The backward recomputes P = exp(S - LSE) tile by tile instead of storing
 * the N x N matrix (explainer page, "Recomputation beim Rueckwaertsdurchlauf";
 * glossary page, "How it works") and returns the gradients of
 * L = sum(O * dO):
 *
 *     dV = P^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,
 *     dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *
 * Layouts.  q, k, v, o, dout, dq, dk, dv: [B, N, H, d] contiguous, row-major
 * (d fastest).  lse: [B, H, N] contiguous fp32.  bf16 entry points take
 * bfloat16 tensors; arithmetic is fp32 (P and dS are rounded to bf16 before
 * their matrix products, outputs are rounded to bf16 once).  The fp32 entry
 * point takes and returns fp32 and computes in fp32 throughout.
 *
 * Supported: d in {64, 128}; B, H, N >= 1; N * H * d < 2^30 (per-lane
 * 32-bit byte offsets within one batch's rows); any finite scale.  Pointers must be device pointers aligned to 16 bytes.
 *
 * Ownership and streams.  The caller owns every buffer (including the
 * backward workspace).  The library never allocates, frees or synchronises:
 * each call validates its arguments on the host, enqueues kernels on
 * `stream` and returns.  Outputs are valid once the stream reaches that point.
 * O and LSE of fa_fwd are the inputs fa_bwd expects.  The forward never reads
 * `o` or `lse`.  Calls are thread-safe.
 *
 * Errors.  0 on success, otherwise a negative FA_ERR_* code.  All argument
 * checks happen before any HIP call, so an invalid call touches no device
 * state.  FA_ERR_LAUNCH reports a failed kernel launch; faults during
 * execution surface on the stream as usual.  NaN or Inf inputs propagate.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1, /* null pointer, B/H/N < 1, non-finite scale,
                                H_kv < 1 or not dividing H (GQA calls),
                                window < 1 (sliding-window calls) */
    FA_ERR_UNSUPPORTED = -2, /* d not in {64, 128}, or N*H*d >= 2^30     */
    FA_ERR_MISALIGNED = -3,  /* a pointer not 16-byte aligned             */
    FA_ERR_WORKSPACE = -4,   /* workspace null, misaligned or too small   */
    FA_ERR_LAUNCH = -5,      /* the HIP runtime rejected a kernel launch  */
    FA_ERR_SCRATCH = -6      /* fa_bwd_noalloc: the shape needs more
                                workspace than its static scratch holds  */
};

/* bf16 forward.  q, k, v: bf16 [B,N,H,d] inputs; o: bf16 [B,N,H,d] output;
 * lse: fp32 [B,H,N] output.  Tiled online softmax over K/V blocks. */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* fp32 forward: same contract with fp32 tensors and fp32 arithmetic
 * (K/V blocks of 256 rows for d = 64, 128 rows for d = 128). */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Bytes of device workspace fa_bwd needs for this shape (0 if the shape is
 * invalid).  It holds two fp32 row statistics per head, padded to a multiple
 * of 64 rows ([B,H,Npad]: LSE * log2(e) and -D with D = rowsum(dO * O)),
 * each 256-byte aligned. */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/* bf16 backward with recomputation.  q, k, v, o, dout: bf16 [B,N,H,d]
 * inputs (o and lse as produced by fa_fwd with the same scale and causal);
 * dq, dk, dv: bf16 [B,N,H,d] outputs.  workspace: device memory of at least
 * fa_bwd_workspace_size(B,H,N,d) bytes, 256-byte aligned, owned by the
 * caller; its contents on entry are ignored and on exit are scratch. */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal,
           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Three backward steps, exported separately so a caller can schedule or
 * time them individually (fa_bwd itself runs the two-step order below:
 * fa_bwd_dq_stats, then fa_bwd_dkdv).  They share fa_bwd's workspace; the
 * first must complete (same stream) before either of the others:
 *   fa_bwd_preprocess: -D_i = -sum_k dO_ik O_ik and LSE_i * log2(e) into the
 *                      workspace.  D is the softmax-Jacobian term of the
 *                      backward (not on the pages, which only require
 *                      recomputation).
 *   fa_bwd_dkdv:       for each block of 128 keys, walk the query blocks that
 *                      can see them, recompute P = exp(scale QK^T - LSE) and
 *                      dS, and write dK and dV (bf16).
 *   fa_bwd_dq:         for each block of 256 queries, walk the key blocks it
 *                      can see, recompute P and dS, and write dQ (bf16).
 * Every output is written once by one workgroup (no atomics), so all three
 * gradients are bitwise repeatable.  Arguments have the meaning and layout
 * given for fa_bwd.  Backward calls also require B * H * Npad < 2^28
 * (Npad = N rounded up to a multiple of 64) and (N + 256) * H * d * 2 < 2^32,
 * else FA_ERR_UNSUPPORTED. */
int fa_bwd_preprocess(const void* o, const void* dout, const float* lse, int B, int H, int N,
                      int d, void* workspace, size_t workspace_bytes, hipStream_t stream);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                void* workspace, size_t workspace_bytes, hipStream_t stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
              int B, int H, int N, int d, float scale, int causal,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* dQ step that forms the row statistics itself, so no preprocess step runs
 * (the backward by recomputation of the explainer page "Flash Attention",
 * section "Recomputation beim Rueckwaertsdurchlauf"; D is the softmax-Jacobian
 * term of that backward, not on the pages):
 * per query it reads O and dO (bf16 [B,N,H,d], O as produced by fa_fwd) and
 * the forward's lse (fp32 [B,H,N]), forms D_i = sum_k dO_ik O_ik and
 * LSE_i * log2(e), uses them for dQ, and writes both into the workspace
 * (same layout and padding as fa_bwd_preprocess).  fa_bwd_dkdv may run after
 * it on the same stream.  fa_bwd runs exactly this pair: fa_bwd_dq_stats,
 * then fa_bwd_dkdv.  Arguments, errors and limits as for fa_bwd. */
int fa_bwd_dq_stats(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, int B, int H, int N, int d, float scale, int causal,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Grouped-query attention (explainer page "Flash Attention", section
 * "Varianten und Erweiterungen", subsection "Grouped Query Attention": several
 * query heads share one K/V head).  q, o, dout, dq: [B,N,H,d]; k, v, dk, dv:
 * [B,N,H_kv,d]; lse: [B,H,N]; H must be a multiple of H_kv, and query head h
 * uses K/V head h / (H / H_kv) (contiguous groups).  H_kv = H is multi-head
 * attention (fa_fwd / fa_bwd are exactly that call); H_kv = 1 is multi-query
 * attention.  dk and dv sum over the query heads of a group; every gradient
 * is still written once by one workgroup.  Workspace: fa_bwd_workspace_size(
 * B, H, N, d) bytes (statistics are per query head).  Same errors, limits
 * and stream semantics as fa_fwd / fa_bwd, plus FA_ERR_INVALID_ARG for an
 * H_kv that does not divide H.  The dK/dV kernel runs one workgroup per
 * (batch, K/V head, 128 keys), so small B * H_kv * N fill few compute units. */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int N, int d, float scale, int causal, hipStream_t stream);
int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv,
               int B, int H, int H_kv, int N, int d, float scale, int causal,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Causal sliding-window attention (explainer page "Flash Attention", section
 * "Varianten und Erweiterungen", subsection "Sliding Window Attention": each
 * position attends to a fixed neighbourhood, and key blocks wholly outside
 * it are neither loaded nor computed).  Query i sees keys j with
 * i - window < j <= i (the window counts the query's own key); window >= N
 * is plain causal attention.  Grouped K/V heads as in fa_fwd_gqa (H_kv = H
 * for multi-head attention).  lse holds the log-sum-exp over the window;
 * fa_bwd_window takes the O and LSE of fa_fwd_window with the same window.
 * window < 1 returns FA_ERR_INVALID_ARG; otherwise as fa_fwd_gqa /
 * fa_bwd_gqa. */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int H_kv, int N, int d, float scale, int window, hipStream_t stream);
int fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv,
                  int B, int H, int H_kv, int N, int d, float scale, int window,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* FP8 forward (explainer page "Flash Attention", section "Versionen: Flash
 * Attention 2 und Flash Attention 3", and glossary page "Flash Attention",
 * section "FlashAttention-2, -3 and -4": FlashAttention-3 runs attention in
 * FP8).  The pages fix no format; here:
 *   q        device, OCP E4M3 byte codes [B, N, H, d], 16-byte aligned
 *   k, v     device, E4M3 codes [B, N, H_kv, d] (H a multiple of H_kv, query
 *            head h reads K/V head h / (H / H_kv); H_kv = H: multi-head)
 *   q_descale  device fp32 [B, H]; k_descale, v_descale: device fp32
 *            [B, H_kv]; 4-byte aligned.  The real value of a code c is
 *            decode(c) * descale of its (batch, head).
 *   o        device bf16 [B, N, H, d]: attention of the decoded values
 *   lse      device fp32 [B, H, N], natural-log log-sum-exp of the scaled
 *            scores of the decoded values
 *   causal   0 / 1; window: 0 = none, >= 1 = causal sliding window as in
 *            fa_fwd_window (window > 0 with causal = 0 is INVALID_ARG)
 * Both products run on the fp8 matrix cores; the probabilities are rounded
 * to E4M3 before the product with V, so O carries a relative error of up to
 * about 2^-4 per probability (the row sum and LSE use the unrounded values).
 * A descale factor that is not positive and finite makes the rows of its
 * heads NaN (checked on the device).  Errors as fa_fwd_gqa; null or
 * misaligned descale pointers return INVALID_ARG / MISALIGNED. */
int fa_fwd_fp8(const void* q, const void* k, const void* v,
               const float* q_descale, const float* k_descale, const float* v_descale,
               void* o, float* lse, int B, int H, int H_kv, int N, int d, float scale,
               int causal, int window, hipStream_t stream);

/* Backward that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  It is fa_bwd (same kernels, arguments, layouts and
 * results, bit for bit) without the workspace arguments: the workspace is a
 * static device array of fa_bwd_noalloc_max_workspace() bytes (16 MiB) in
 * the library, which every GPU that runs the library holds until the process
 * ends.  Shapes with fa_bwd_workspace_size(B, H, N, d) above that (B * H *
 * Npad above 2^21 rows, Npad = N rounded up to 64) return FA_ERR_SCRATCH
 * before any HIP call.  `stream` must belong to the current device
 * (FA_ERR_INVALID_ARG otherwise).  The first call on a device looks up the
 * array's device address (hipGetSymbolAddress; FA_ERR_LAUNCH if that fails);
 * no call allocates or frees memory.  All calls on one GPU share the array,
 * so calls that overlap on one GPU (other streams or threads) race; calls
 * on one stream are ordered and safe.  Nothing in the array needs clearing
 * between calls. */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal, hipStream_t stream);
size_t fa_bwd_noalloc_max_workspace(void);

/* Merge of two attention results over disjoint key ranges of the same
 * queries into the result over their union (explainer page "Flash
 * Attention", section "Tiling": the rescaling of a partial output by
 * exp(m_old - m_new) when the running maximum grows, applied once to two
 * finished results).  Per row, with L = log(exp(lse_a) + exp(lse_b)):
 *     o = exp(lse_a - L) o_a + exp(lse_b - L) o_b,   lse = L,
 * in fp32, o rounded to bf16 once.  This combines the results of devices
 * that each hold a range of the keys.  o_a, o_b, o: device bf16 [B,N,H,d];
 * lse_a, lse_b, lse: device fp32 [B,H,N]; all 16-byte aligned.  A range of
 * weight 0 (its LSE -inf, or so far below the other's that its weight
 * underflows) contributes nothing, whatever its o holds; a row with both
 * LSEs -inf gets o = 0 and lse = -inf; NaN in either LSE gives a NaN row;
 * NaN or Inf in an o of nonzero weight propagates.  o may be o_a or o_b and
 * lse may be lse_a or lse_b (accumulation in place); no other overlap is
 * allowed.  Shapes as fa_fwd.  INVALID_ARG for null pointers or B/H/N < 1;
 * UNSUPPORTED for d or sizes as fa_fwd; MISALIGNED; LAUNCH. */
int fa_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o, float* lse,
             int B, int H, int N, int d, hipStream_t stream);

/* Measurement aid (not part of attention): the matrix-core calibration
 * kernel of the roofline harness.  Launches n_workgroups workgroups of
 * waves_per_workgroup (1..4) waves; each wave runs `iters` rounds of 16
 * v_mfma_f32_32x32x16_bf16 on eight independent accumulator chains (32768
 * flops each, so n_workgroups * waves * iters * 16 * 32768 flops per launch).
 * mode: 0 register operands that never change; 1 random register operands
 * (eight A and eight B tiles per wave, paired differently by consecutive
 * MFMAs); 2 mode 1 plus an FMA and an exp2 per MFMA; 3 mode 1 plus two FMAs
 * and two exp2 per MFMA; 4 mode 1 with the A operand read from LDS (one
 * ds_read_b128 per MFMA); 5 mode 4 plus three FMAs and one exp2 per MFMA
 * (the forward's mix per MFMA); 6 mode 5 with each LDS read feeding two
 * MFMAs (0.5 KB per MFMA, the mix of 64 queries per wave); 7 mode 4 plus
 * four FMAs and one exp2 per two MFMAs (the dK/dV kernel's mix).  out: device fp32 with n_workgroups * 64 *
 * waves_per_workgroup elements (checksums, 4-byte aligned).  The rates of
 * modes 0 and 1 are the chip's dense bf16 rate with and without operand
 * switching (the second is what real data sees); the MFMA-busy counter of
 * mode 0 checks the busy-cycle normalisation.  INVALID_ARG for out null or
 * counts or mode out of range; UNSUPPORTED for more than 2^22 workgroups;
 * MISALIGNED; LAUNCH. */
int fa_calibrate_mfma(float* out, int n_workgroups, int waves_per_workgroup, int iters, int mode,
                      hipStream_t stream);

/* Measurement aid (not part of attention): the matrix-core probe used to
 * measure the accumulation error of the MFMA instructions the kernels use.
 * For n_tiles independent 32 x 32 tiles it computes, in fp32 on the matrix
 * core, C[t][i][c] = sum_j A[t][i][j] * B[t][c][j] with contraction length
 * k, chaining k / 16 (bf16, fp8 = 0: v_mfma_f32_32x32x16_bf16) or k / 64
 * (fp8 = 1: OCP E4M3 codes, v_mfma_f32_32x32x64_f8f6f4) MFMAs in one fp32
 * accumulator.  a, b: device [n_tiles][32][k] row-major (bf16 or byte
 * codes), 16-byte aligned; c: device fp32 [n_tiles][32][32], 4-byte aligned.
 * INVALID_ARG for null pointers, counts below 1, fp8 not 0 or 1, or k not a
 * multiple of 16 (bf16) / 64 (fp8); UNSUPPORTED when an operand reaches
 * 2^31 bytes; MISALIGNED; LAUNCH. */
int fa_probe_mfma(int fp8, const void* a, const void* b, float* c, int n_tiles, int k, hipStream_t stream);

/* Human-readable text for a return code (static storage). */
const char* fa_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
