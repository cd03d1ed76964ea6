/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) speculative-decoding
 * verification library (libspecverify.so).
 *
 * The library implements the target model's verification step of
 * speculative decoding as two stages:
 *   spec_verify_linear  the verify linear layer, Y = X W, whose row count
 *                       grows from B to B(1+D) when D drafts are verified
 *                       (spec_verify_linear_packed: the same with W stored
 *                       once in the MFMA operand order by spec_pack_weight);
 *   spec_accept         the batched accept/reject pass over the target's
 *                       vocabulary distributions (spec_accept_sampled: the
 *                       same with the draft as logits and the sampler's
 *                       top-p / min-p filters on both distributions);
 * and the control around it:
 *   spec_verify_attention  the verify pass's attention: K+1 causal
 *                       queries per sequence against its KV cache;
 *   spec_adapt          acceptance telemetry and the next draft depth per
 *                       row, on the GPU, from spec_accept's output;
 *   spec_plan_depth     (host) the draft depth per batch size from a
 *                       measured verify-cost curve.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers, allocated and owned by the caller
 *    (spec_plan_depth alone takes host arrays).
 *    The library allocates nothing and keeps no state between calls, so
 *    calls on different streams may run concurrently provided their
 *    workspaces do not overlap (spec_accept_noalloc alone uses a static
 *    device array of its own; see there).
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
#define SPEC_ROW_NONFINITE 1   /* a NaN or +Inf logit, or an all -Inf position, at a target
                                  position the pass reads: positions 0, 1, ... in order up to
                                  the first rejection (or L_b), as the listing's loop stops
                                  there; positions after it are not read.  With
                                  spec_accept_sampled also any draft position i < L_b */
#define SPEC_ROW_BAD_TOKEN 2   /* a draft token outside [0, V) at a position < L_b */
#define SPEC_ROW_BAD_LEN 4     /* L_b outside [0, K] */
#define SPEC_ROW_ZERO_Q 8      /* q_i(x_i) not > 0 at a position < L_b (stochastic mode) */
#define SPEC_ROW_RESID_ZERO 16 /* informational: the residual max(p - q, 0) summed to 0,
                                  the token was drawn from p instead */
#define SPEC_ROW_STALLED 32    /* a workgroup of the row waited for the row's decision past
                                  the wait bound (about 0.1 s) and gave up; out_accepted[b]
                                  = -1 and out_tokens[b] is all -1 (out_p_draft[b] is
                                  unspecified).  The workspace stays valid for later calls */

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
 *   out_p_draft    [B, K] fp32 or NULL: p_i(x_i) at the tested positions,
 *                  i <= a_b and i < L_b (1/0 in greedy mode: whether x_i is
 *                  the argmax); -1 elsewhere and for invalid rows
 *   out_status     [B] int32 or NULL: SPEC_ROW_* bits
 *   workspace      device scratch of at least spec_accept_workspace_bytes(B, K, V)
 *                  bytes, 16-byte aligned.  Its first 256 * B bytes hold
 *                  per-row counters through which the workgroups of a row
 *                  hand work to one another: they must be ZERO when the call
 *                  starts, and every call leaves them zero again (also one
 *                  in which a row stalled).  So a workspace zero-filled once
 *                  serves every later call with the same or fewer rows (any
 *                  K, V).  Calls that may run concurrently need separate
 *                  workspaces.
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
 * spec_accept_noalloc -- spec_accept for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, arguments and outputs, with no
 * workspace argument.
 *
 * The workspace is a static device array of 16 MiB inside the library, one
 * per GPU, held until the process ends.  On the first call on a device the
 * library takes the array's device address (hipGetSymbolAddress) and clears
 * it with a kernel on `stream`; no call allocates or frees memory.  A call
 * whose workspace, spec_accept_workspace_bytes(B, K, V), exceeds 16 MiB
 * returns SPEC_ERR_WORKSPACE before any launch (the fused step's B = 32,
 * K = 5, V = 151936 needs 2.5 MiB; B = 64, K = 7, V = 128256 needs 4.3 MiB).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or host threads) race and give wrong results;
 * order them on one stream.  Each call leaves the array's row records zero,
 * as the next call needs them.
 * Errors: as spec_accept, plus SPEC_ERR_HIP if the array's address cannot
 * be obtained.
 * ---------------------------------------------------------------------- */
int spec_accept_noalloc(const void* target_logits, int logits_dtype,
                        const float* draft_probs, const int32_t* draft_tokens,
                        const int32_t* draft_lens, int64_t B, int K, int64_t V,
                        int64_t row_base, float temperature, uint64_t philox_seed,
                        uint64_t philox_offset, int32_t* out_tokens, int32_t* out_accepted,
                        float* out_p_draft, int32_t* out_status, void* stream);

/* ------------------------------------------------------------------------
 * spec_accept_sampled -- accept/reject with the production sampler's
 * filters; the draft is given as logits.
 *
 * Defined by: page "Decode is memory-bound: ~59 tok/s ceiling on an RTX
 * 4090, and how speculative decoding beats it" (trefon.com), section "Two
 * things that follow from the math" (production sampler: temperature 0.6,
 * top-p 0.95, min-p 0.05; the draft sampler matched to the target's) and
 * section "Speculative decoding" (acceptance rule, exactness); page
 * "Speculative decoding and early exit ..." (reactapp.top), listing
 * speculative_decode (q is the tempered softmax of the draft's logits).
 *
 * For each row, as spec_accept, with p and q replaced by the filtered
 * distributions p' = F(softmax(target_logits[b,i,:] / temperature)) and
 * q' = F(softmax(draft_logits[b,i,:] / draft_temperature)), where F keeps
 * token j iff (a) the probability of the tokens with a strictly larger logit
 * sums to less than top_p and (b) p_j >= min_p * max_k p_k, and renormalises
 * the kept mass.  top_p == 1 and min_p == 0 turn (a) and (b) off.  A draft
 * token outside q''s kept set makes the row invalid (SPEC_ROW_ZERO_Q).
 * out_p_draft holds p'_i(x_i) at the tested positions.  The drafted tokens
 * are validated for all L_b drafts (range, finite draft logits, token in q''s
 * kept set).  Same uniforms, inverse-CDF rule, residual
 * fall-back and per-row status bits as spec_accept.  The filters are
 * resolved exactly: the top-p cut is the exact logit at which the mass,
 * counted from the top in 2^-40 fixed point of fp32 weights, reaches top_p
 * of the total.
 *
 * Arguments: as spec_accept, except
 *   draft_logits   [B, K, V] of logits_dtype (the same dtype as the target)
 *   temperature, draft_temperature   finite, > 0 (no greedy mode here)
 *   top_p in (0, 1]; min_p in [0, 1)
 *   workspace      spec_accept_sampled_workspace_bytes(B, K, V) bytes,
 *                  16-byte aligned; its first 256 * B bytes must be ZERO when
 *                  the call starts (every call leaves them zero)
 * Two launches on `stream`: per-distribution statistics (max, top-p cut,
 * kept mass), then the decisions and draws.
 * ---------------------------------------------------------------------- */
size_t spec_accept_sampled_workspace_bytes(int64_t B, int K, int64_t V);

int spec_accept_sampled(const void* target_logits, const void* draft_logits, int logits_dtype,
                        const int32_t* draft_tokens, const int32_t* draft_lens, int64_t B, int K,
                        int64_t V, int64_t row_base, float temperature, float draft_temperature,
                        float top_p, float min_p, uint64_t philox_seed, uint64_t philox_offset,
                        int32_t* out_tokens, int32_t* out_accepted, float* out_p_draft,
                        int32_t* out_status, void* workspace, size_t workspace_bytes,
                        void* stream);

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
 *               The size is that of the current device's plan (it depends
 *               on the device's compute-unit count): query it with the
 *               device the call will run on current.
 * ---------------------------------------------------------------------- */
size_t spec_verify_linear_workspace_bytes(int64_t M, int64_t N, int64_t Kd);

int spec_verify_linear(const void* X, const void* W, void* Y, int y_dtype,
                       int64_t M, int64_t N, int64_t Kd, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spec_pack_weight / spec_verify_linear_packed -- the same product,
 * Y[M, N] = X[M, K] W[K, N] (bf16 operands, fp32 accumulation, Y fp32 or
 * bf16), with W rewritten once into the operand order of the gfx950 MFMA
 * (v_mfma_f32_16x16x32_bf16), for a weight that every verify pass reads
 * whole, such as the lm-head.  The packed product streams W straight into
 * registers instead of through LDS.
 *
 * Defined by: page "New technical post reveals how speculative decoding
 * accelerates LLM inference without hurting accuracy" (agentnet.co.il),
 * sections "The formula behind the speedup" and "GEMM-M grows, a small
 * batch suffices" (as spec_verify_linear).
 *
 * Packed layout: 2 KB blocks, block (s, c) for k rows 32 s .. 32 s + 31 and
 * columns 32 c .. 32 c + 31 at byte (s C + c) 2048, C = ceil(N / 32).  In a
 * block, the 16 bytes at 16 (64 h + l), h in {0, 1}, l < 64, hold
 * W[32 s + 8 (l / 16) + j][32 c + 16 h + l % 16] for j = 0..7.  Columns at
 * or past N are zero.
 *
 * spec_packed_weight_bytes(K, N): size of the packed W; 0 for an
 *   unsupported shape (K must be a positive multiple of 64, at most 2^30;
 *   1 <= N <= 2^36).
 * spec_pack_weight(W, Wp, K, N, stream): W [K, N] bf16 row-major (2-byte
 *   aligned) into Wp (caller-owned device memory of
 *   spec_packed_weight_bytes(K, N) bytes, 16-byte aligned); enqueued on
 *   stream.  SPEC_ERR_INVALID_ARG for a bad shape or pointer.
 * spec_verify_linear_packed(X, Wp, Y, y_dtype, M, N, K, workspace,
 *   workspace_bytes, stream):
 *   X   [M, K] bf16, row-major (K contiguous), 16-byte aligned
 *   Wp  the packed W of the same K and N, 16-byte aligned
 *   Y   [M, N] of y_dtype (SPEC_F32 or SPEC_BF16), 16-byte aligned
 *   M >= 0 (M == 0 returns SPEC_OK without launching); K and N as above
 *   (SPEC_ERR_INVALID_ARG otherwise).
 *   workspace   device scratch of at least
 *               spec_verify_linear_packed_workspace_bytes(M, N, K) bytes
 *               (may be NULL when that is 0; contents need not be
 *               initialised), 16-byte aligned, else SPEC_ERR_WORKSPACE.
 *               The size depends on the current device's compute-unit
 *               count: query it with that device current.
 *   Results equal spec_verify_linear's up to the order of the fp32 sums.
 * ---------------------------------------------------------------------- */
size_t spec_packed_weight_bytes(int64_t K, int64_t N);

int spec_pack_weight(const void* W, void* Wp, int64_t K, int64_t N, void* stream);

size_t spec_verify_linear_packed_workspace_bytes(int64_t M, int64_t N, int64_t K);

int spec_verify_linear_packed(const void* X, const void* Wp, void* Y, int y_dtype,
                              int64_t M, int64_t N, int64_t K, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spec_adapt -- acceptance telemetry and the adaptive draft depth, run on
 * the GPU after a verify pass, from that pass's out_accepted.
 *
 * Defined by: page "Decode is memory-bound: ~59 tok/s ceiling on an RTX
 * 4090, and how speculative decoding beats it" (trefon.com), section "Two
 * things that follow from the math" (the adaptive mode caps the draft depth
 * once the measured acceptance falls under 35%) and the closing rules (pick
 * the depth from the measured acceptance, keep measuring); section
 * "Speculative decoding" (E(a, k) = 1 + a + ... + a^k, speedup
 * E / (k c + 1)).  Page "Speculative decoding and early exit ..."
 * (reactapp.top), section "Production perspective" and the operational
 * checklist (acceptance rate, mean accepted length, acceptance histograms).
 *
 * For each row b with a = accepted[b] and L = draft_lens[b] (K if NULL):
 *   - a valid row (0 <= L <= K, 0 <= a <= L) ran a + 1 acceptance tests if
 *     a < L, else a; if it ran any, (a, tests) enters the row's record, a
 *     ring of its last 16 such passes.  Any other row (a = -1 from an
 *     invalid accept row, or inconsistent values) is counted as invalid and
 *     leaves its record unchanged.
 *   - S, N = accepted drafts and tests over the record's last
 *     min(window, recorded) passes; the measured acceptance is S / N.
 *   - next_lens[b] = k_max if N == 0; otherwise
 *       SPEC_ADAPT_THRESHOLD: k_min if S < accept_floor * N (fp64), else k_max;
 *       SPEC_ADAPT_SPEEDUP:   the k in [k_min, k_max] maximising
 *                             E(S/N, k) / (k * draft_cost + 1), lowest on ties
 *                             (fp64, E summed term by term).
 * Telemetry: the block of SPEC_ADAPT_TELEMETRY_WORDS uint64 counters is
 * ADDED to (zero it once to start counting).  Word layout:
 *   [0] valid rows  [1] invalid rows  [2] drafted (sum L)  [3] tests run
 *   [4] accepted drafts (sum a)  [5] emitted tokens (sum a + 1)  [6] calls
 *   [8 + i]   tests run at draft position i        (i < SPEC_ADAPT_MAX_K)
 *   [40 + i]  drafts accepted at position i        (i < SPEC_ADAPT_MAX_K)
 *   [72 + d]  rows given next depth d               (d <= SPEC_ADAPT_MAX_K)
 *   [105 + L * 33 + a]  valid rows with draft length L and a accepted drafts
 *   the rest reserved (left as they are).
 *
 * Arguments (device pointers, caller-owned):
 *   accepted     [B] int32 (spec_accept's out_accepted)
 *   draft_lens   [B] int32 or NULL (every row verified K drafts)
 *   B            rows, 0 .. 2^31; K: the max draft length of that pass, 0..32
 *   state        [B] records of SPEC_ADAPT_STATE_BYTES, 16-byte aligned;
 *                zero = no history.  Bytes 0-15 the accepted counts of the
 *                ring, 16-31 the test counts, 32-35 the passes recorded
 *                (uint32; the ring slot of pass n is n mod 16), 36-39 the
 *                last depth chosen (int32), 40-63 reserved.
 *   telemetry    SPEC_ADAPT_TELEMETRY_WORDS uint64, 8-byte aligned
 *   next_lens    [B] int32: the next pass's draft length per row
 *   1 <= k_min <= k_max <= SPEC_ADAPT_MAX_K; 1 <= window <= 16
 *   policy       SPEC_ADAPT_THRESHOLD or SPEC_ADAPT_SPEEDUP
 *   accept_floor in [0, 1] (0.35 in the page's adaptive mode)
 *   draft_cost   c >= 0, finite (used by SPEC_ADAPT_SPEEDUP)
 * Errors: SPEC_ERR_INVALID_ARG (host validation, nothing enqueued),
 * SPEC_ERR_HIP.  Calls that share a state or telemetry block must be
 * ordered on one stream.
 * ---------------------------------------------------------------------- */
#define SPEC_ADAPT_MAX_K 32
#define SPEC_ADAPT_STATE_BYTES 64
#define SPEC_ADAPT_TELEMETRY_WORDS 1200
#define SPEC_ADAPT_THRESHOLD 0
#define SPEC_ADAPT_SPEEDUP 1

size_t spec_adapt_state_bytes(int64_t B);
size_t spec_adapt_telemetry_bytes(void);

int spec_adapt(const int32_t* accepted, const int32_t* draft_lens, int64_t B, int K,
               void* state, uint64_t* telemetry, int32_t* next_lens, int k_min, int k_max,
               int window, int policy, double accept_floor, double draft_cost, void* stream);

/* ------------------------------------------------------------------------
 * spec_plan_depth -- HOST function: the draft depth per batch size from a
 * measured verify-cost curve, and the throughput / interactivity frontier.
 *
 * Defined by: agentnet.co.il item on speculative decoding, section "The
 * formula behind the speedup" (speculation pays when the verify time at
 * B(1+D) rows over that at B rows is below the accepted length; the best D
 * depends on B along a Pareto frontier of throughput against
 * interactivity) and section "GEMM-M grows, a small batch suffices"
 * (M = B(1+D)); page "Decode is memory-bound ..." (trefon.com), section
 * "Speculative decoding" (E(a, D) and the draft cost c).
 *
 * With T(M) the measured pass time at M rows (linear between points, flat
 * below the first, the last segment's slope above the last), for batch B
 * and depth D in [0, d_max]:
 *   den = T(B(1+D)) + (D c) T(B)
 *   speedup[B, D] = (E(a, D) T(B)) / den
 *   tokens_per_s[B, D] = (B E(a, D)) / den * 1e6   (t_pts in microseconds)
 *   best_depth[B] = argmax_D speedup (lowest D on ties)
 *   pareto[B, D] = 1 iff no other (B', D') has total tokens/s and
 *                  per-sequence tokens/s (E / den) both >= and one >.
 * Arguments (HOST pointers): m_pts [n_pts] int64 strictly ascending, >= 1;
 * t_pts [n_pts] > 0 finite; batches [n_batches] in [1, 2^31]; d_max in
 * [0, SPEC_MAX_DRAFT]; alpha in [0, 1]; draft_cost >= 0 finite;
 * out_best_depth [n_batches] int32; out_speedup, out_tokens_per_s
 * [n_batches, d_max+1] double, out_pareto [n_batches, d_max+1] uint8, each
 * may be NULL.  Returns SPEC_OK or SPEC_ERR_INVALID_ARG.  Allocates host
 * memory only.
 * ---------------------------------------------------------------------- */
int spec_plan_depth(const int64_t* m_pts, const double* t_pts, int n_pts,
                    const int64_t* batches, int n_batches, int d_max, double alpha,
                    double draft_cost, int32_t* out_best_depth, double* out_speedup,
                    double* out_tokens_per_s, uint8_t* out_pareto);

/* ------------------------------------------------------------------------
 * spec_verify_attention -- attention of a verify pass: the K+1 query
 * positions of each sequence against its KV cache, causal within the
 * verified block, grouped KV heads.
 *
 * Defined by: page "Speculative decoding and early exit: accelerated
 * autoregressive decoding" (reactapp.top), section "Attention structure
 * during decoding" (each step's queries read the sequence's whole key/value
 * memory; one head: Q [8, 1, 128] against K, V [8, 2048, 128]) and section
 * "Speculative decoding: draft first, then verify" (one target pass over
 * K+1 positions); page "Decode is memory-bound ..." (trefon.com), ceiling
 * section (at long context the cache is read in full on every pass).
 *
 * For sequence b with ctx_b cached tokens and L_b drafts (draft_lens[b], K
 * if NULL), query i = 0 .. L_b (the token that ended the previous pass,
 * then the drafts) sits at position ctx_b + i; its key and value must
 * already be in the cache there.  For query head h (KV head g = h / (H/Hkv)):
 *   out[b, i, h, :] = sum_{j <= ctx_b + i} softmax_j(scale * q[b,i,h,:].k[b,g,j,:]) v[b,g,j,:]
 * Rows i > L_b are written as zeros.  fp32 accumulation; the probabilities
 * enter the value product rounded to bf16.
 *
 * Arguments (device pointers, caller-owned, 16-byte aligned):
 *   q          [B, K+1, H, 128] bf16
 *   k_cache, v_cache  [B, Hkv, S, 128] bf16 (S = cache capacity per sequence)
 *   ctx_lens   [B] int32; draft_lens [B] int32 or NULL
 *   B in [0, 65535]; K >= 0; H a multiple of Hkv; (K+1) * (H/Hkv) <= 32;
 *   head_dim == 128; scale finite
 *   out        [B, K+1, H, 128] of out_dtype (SPEC_F32 or SPEC_BF16)
 *   out_status [B] int32 or NULL: SPEC_ROW_BAD_LEN when ctx_b < 0, L_b is
 *              outside [0, K] or ctx_b + L_b + 1 > S (that row's output is
 *              zero); 0 otherwise
 *   workspace  spec_verify_attention_workspace_bytes(B, K, H, Hkv, S) bytes
 *              (0 when the cache is not split across workgroups; may then be
 *              NULL), contents need not be initialised
 * The cache capacity S sets how the keys are split across workgroups:
 * pass the batch's longest ctx_b + L_b + 1 rather than a much larger
 * allocation size for the best split.
 * Errors: SPEC_ERR_INVALID_ARG, SPEC_ERR_WORKSPACE, SPEC_ERR_HIP.
 * ---------------------------------------------------------------------- */
#define SPEC_ATTN_HEAD_DIM 128
#define SPEC_ATTN_MAX_ROWS 32

size_t spec_verify_attention_workspace_bytes(int64_t B, int K, int H, int Hkv, int64_t S);

int spec_verify_attention(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* ctx_lens, const int32_t* draft_lens, int64_t B, int K,
                          int H, int Hkv, int64_t S, int head_dim, float scale, void* out,
                          int out_dtype, int32_t* out_status, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spec_debug_set_wait_bound -- sets how many times a spec_accept workgroup
 * polls its row's decision (a poll is two coherent loads and a short sleep,
 * about 1.5 us) before it gives up on the row and reports SPEC_ROW_STALLED;
 * polls == 0 restores the
 * default (65536, about 0.1 s).  Process-wide, read by each later
 * spec_accept call when it is enqueued.  It exists so that tests can drive
 * the give-up path with every kernel still ending normally: with a bound of
 * 1, workgroups that find no decision on their first poll give up.
 * Returns SPEC_OK, or SPEC_ERR_INVALID_ARG for polls < 0.
 * ---------------------------------------------------------------------- */
int spec_debug_set_wait_bound(int polls);

/* Human-readable text of a return code (static storage). */
const char* spec_status_string(int code);

/* ABI version of this header (incremented on incompatible changes). */
#define SPEC_VERIFY_ABI_VERSION 4
int spec_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
