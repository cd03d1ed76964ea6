/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) speculative-decoding
 * verification library (libspecverify.so).
 *
 * The library implements the target model's verification step of
 * speculative decoding as two stages:
 *   spec_verify_linear  the verify linear layer, Y = X W, whose row count
 *                       grows from B to B(1+D) when D drafts are verified;
 *   spec_accept         the batched accept/reject pass over the target's
 *                       vocabulary distributions.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers, allocated and owned by the caller.
 *    The library allocates nothing and keeps no state between calls, so
 *    calls on different streams may run concurrently provided their
 *    workspaces do not overlap.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls enqueue work on it and return; outputs are valid once the stream
 *    has synchronised.
 *  - Host-side argument validation happens before any HIP call; a rejected
 *    call returns a negative code and enqueues nothing.  A failed kernel
 *    launch returns SPEC_ERR_HIP.  Bad DATA (non-finite logits, an
 *    out-of-range token, ...) does not fail the call: it is reported per row
 *    through out_status.
 *  - All tensors are dense and row-major (last index fastest).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of the logits / activations. */
typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* Return codes. */
#define SPEC_OK 0
#define SPEC_ERR_INVALID_ARG (-1) /* null pointer, bad size, bad dtype, bad temperature */
#define SPEC_ERR_WORKSPACE (-2)   /* workspace missing or smaller than required */
#define SPEC_ERR_HIP (-3)         /* a HIP launch or runtime call failed */

/* Per-row status bits written to out_status[b]; 0 = row processed normally.
 * A row with any of the first four bits set is invalid: out_accepted[b] = -1
 * and its out_tokens row is all -1. */
#define SPEC_ROW_NONFINITE 1   /* a NaN or +Inf logit, or an all -Inf position, at a position <= L_b */
#define SPEC_ROW_BAD_TOKEN 2   /* a draft token outside [0, V) at a position < L_b */
#define SPEC_ROW_BAD_LEN 4     /* L_b outside [0, K] */
#define SPEC_ROW_ZERO_Q 8      /* q_i(x_i) not > 0 at a position < L_b (stochastic mode) */
#define SPEC_ROW_RESID_ZERO 16 /* informational: the residual max(p - q, 0) summed to 0,
                                  the token was drawn from p instead */
#define SPEC_ROW_STALLED 32    /* the row's workgroups did not all make progress within the
                                  wait bound (about 0.1 s); out_accepted[b] = -1, the rest
                                  of the row's outputs are unspecified, and the workspace
                                  must be zero-filled again before its next use */

/* Limits. */
#define SPEC_MAX_DRAFT 255 /* K <= 255 */

/* ------------------------------------------------------------------------
 * spec_accept -- batched accept/reject of K drafted tokens per row.
 *
 * Defined by: page "Speculative decoding and early exit: accelerated
 * autoregressive decoding" (reactapp.top), section "Speculative decoding:
 * draft first, then verify", listing `speculative_decode` (accept/reject
 * block); page "Decode is memory-bound: ~59 tok/s ceiling on an RTX 4090,
 * and how speculative decoding beats it" (trefon.com), section
 * "Speculative decoding" (acceptance with probability min(1, p(x)/q(x)),
 * exactness of the output distribution, greedy longest-prefix rule).
 *
 * For each row b (independently) with draft length L_b:
 *   p_i = softmax(target_logits[b, i, :] / T)                 for i <= L_b
 *   for i = 0 .. L_b-1: accept x_i iff u_acc(b, i) < min(1, p_i(x_i) / q_i(x_i));
 *     stop at the first rejection a_b (a_b = L_b if none);
 *   if a_b < L_b: token = draw from max(p_{a_b} - q_{a_b}, 0) (normalised)
 *   else        : token = draw from p_{L_b} (the bonus token)
 *   out_tokens[b, :] = x_0 .. x_{a_b-1}, token, -1 ...;  out_accepted[b] = a_b.
 * Draws use the inverse CDF: with weights w and t = u_smp(b, a_b) * sum(w),
 * the token is the smallest j whose inclusive prefix sum exceeds t.
 * Uniforms: one Philox4x32-10 block per (row, position) with
 *   counter = (i, row_base + b, offset_lo, offset_hi), key = (seed_lo, seed_hi);
 *   u_acc = (word0 >> 8) * 2^-24, u_smp = (word1 >> 8) * 2^-24.
 * temperature == 0 selects the greedy limit: g_i = argmax_j logits[b, i, j]
 * (lowest index on ties), accept while x_i == g_i, emit g_{a_b}; no uniforms
 * are consumed and draft_probs is not read.
 *
 * Arguments:
 *   target_logits  [B, K+1, V] of logits_dtype (fp32 or bf16)
 *   draft_probs    [B, K, V] fp32 draft distributions q (already tempered by
 *                  the drafter); may be NULL iff temperature == 0.  Only
 *                  q_i(x_i) is validated; q rows must hold probabilities.
 *   draft_tokens   [B, K] int32 (may be NULL iff K == 0)
 *   draft_lens     [B] int32 L_b in [0, K], or NULL meaning every L_b = K
 *   B, K, V        rows (>= 0), max draft length (0..SPEC_MAX_DRAFT), vocab
 *                  (1 .. 4194304 for fp32 logits, .. 8388608 for bf16)
 *   row_base       global index of row 0 (>= 0, row_base + B <= 2^32): the
 *                  Philox stream of row b is that of global row row_base + b,
 *                  so a batch split into row shards reproduces the unsplit call
 *   temperature    finite, >= 0 (applies to the target logits only)
 *   philox_seed, philox_offset   the Philox key and counter high words
 *   out_tokens     [B, K+1] int32
 *   out_accepted   [B] int32: a_b, or -1 for an invalid row
 *   out_p_draft    [B, K] fp32 or NULL: p_i(x_i) for i < L_b (1/0 in greedy
 *                  mode: whether x_i is the argmax); -1 elsewhere and for
 *                  invalid rows
 *   out_status     [B] int32 or NULL: SPEC_ROW_* bits
 *   workspace      device scratch of at least spec_accept_workspace_bytes(B, K, V)
 *                  bytes, 16-byte aligned.  Its first 256 * B bytes hold
 *                  per-row counters through which the workgroups of a row
 *                  hand work to one another: they must be ZERO when the call
 *                  starts, and every call leaves them zero again.  So a
 *                  workspace zero-filled once serves every later call with
 *                  the same or fewer rows (any K, V).  Calls that may run
 *                  concurrently need separate workspaces.
 * Errors: SPEC_ERR_INVALID_ARG, SPEC_ERR_WORKSPACE, SPEC_ERR_HIP.
 * B == 0 returns SPEC_OK without launching.
 * ---------------------------------------------------------------------- */
size_t spec_accept_workspace_bytes(int64_t B, int K, int64_t V);

int spec_accept(const void* target_logits, int logits_dtype,
                const float* draft_probs, const int32_t* draft_tokens,
                const int32_t* draft_lens, int64_t B, int K, int64_t V,
                int64_t row_base, float temperature, uint64_t philox_seed,
                uint64_t philox_offset, int32_t* out_tokens, int32_t* out_accepted,
                float* out_p_draft, int32_t* out_status, void* workspace,
                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spec_verify_linear -- Y[M, N] = X[M, Kd] W[Kd, N], bf16 operands, fp32
 * accumulation, Y stored as fp32 or bf16 (round to nearest even).
 *
 * Defined by: page "New technical post reveals how speculative decoding
 * accelerates LLM inference without hurting accuracy" (agentnet.co.il),
 * sections "The formula behind the speedup" and "GEMM-M grows, a small
 * batch suffices": verifying D drafts multiplies the row count of every
 * linear layer of the target by (1+D), which is memory-bound at small
 * M = B(1+D) and turns compute-bound as D grows.
 *
 * Arguments:
 *   X   [M, Kd] bf16, row-major (Kd contiguous)
 *   W   [Kd, N] bf16, row-major (N contiguous), i.e. stored input-major
 *   Y   [M, N] of y_dtype
 *   M >= 0, N >= 1, Kd >= 1; N and Kd must be multiples of 8 and X, W, Y
 *   16-byte aligned (SPEC_ERR_INVALID_ARG otherwise).  M == 0 returns
 *   SPEC_OK without launching.
 *   workspace   device scratch of at least
 *               spec_verify_linear_workspace_bytes(M, N, Kd) bytes (may be
 *               NULL when that is 0); its contents need not be initialised.
 * ---------------------------------------------------------------------- */
size_t spec_verify_linear_workspace_bytes(int64_t M, int64_t N, int64_t Kd);

int spec_verify_linear(const void* X, const void* W, void* Y, int y_dtype,
                       int64_t M, int64_t N, int64_t Kd, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Human-readable text of a return code (static storage). */
const char* spec_status_string(int code);

/* ABI version of this header (incremented on incompatible changes). */
#define SPEC_VERIFY_ABI_VERSION 1
int spec_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
