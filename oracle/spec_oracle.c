/*
 * spec_oracle.c -- plain fp64 CPU oracle for the speculative-decoding
 * verification step (accept/reject over vocabulary distributions).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or constant generator with the HIP implementation; the only
 * things both sides agree on are the published definitions they were each
 * written from (the pages' algorithm and the Philox4x32-10 generator).
 *
 * Sources (cited by page title and section):
 *  [P1] "Speculative decoding and early exit: accelerated autoregressive
 *       decoding" (reactapp.top), section "Speculative decoding: draft first,
 *       then verify", listing `speculative_decode`, accept/reject block.
 *  [P2] "Decode is memory-bound: ~59 tok/s ceiling on an RTX 4090, and how
 *       speculative decoding beats it" (trefon.com), section "Speculative
 *       decoding" (acceptance rule min(1, p(x)/q(x)); greedy longest-prefix
 *       rule) and section "Two things that follow from the math".
 *  [P3] agentnet.co.il news item on speculative decoding, section "How it
 *       works in practice" (accepted length lies in [1, 1+D]).
 *  [PH] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *       1, 2, 3", SC'11: the Philox4x32-10 bijection.
 *
 * Every floating-point step is fp64; inputs arrive as fp32 arrays holding
 * the exact values the GPU receives (bf16 widens to fp32 without rounding).
 * Loops run in plain sequential index order.
 *
 * Readings of the pages taken where they are silent:
 *  - the acceptance ratio has no epsilon: a = min(1, p(x)/q(x)), accept iff
 *    u < a with u in [0,1);  q(x) <= 0 is a data error (ROW_ZERO_Q).
 *  - each (row, position) gets its own Philox block; word 0 drives the
 *    acceptance test and word 1 drives the categorical draw.
 *  - rows are independent; row b verifies L_b drafts and its bonus token is
 *    read at position L_b.
 *  - a categorical draw from weights w uses the inverse CDF: t = u * sum(w),
 *    token = smallest j whose inclusive prefix sum exceeds t.
 *  - an all-zero residual (p == q) falls back to sampling from p and sets
 *    ROW_RESID_ZERO.
 *  - temperature 0 is the greedy limit: argmax with the lowest index on
 *    ties, accept while the draft equals the argmax.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Per-row status bits (the interface's data-error report). */
#define ORC_ROW_NONFINITE   1
#define ORC_ROW_BAD_TOKEN   2
#define ORC_ROW_BAD_LEN     4
#define ORC_ROW_ZERO_Q      8
#define ORC_ROW_RESID_ZERO 16

/* A draw counts as near its threshold inside this window (absolute for the
 * acceptance test, relative to the total weight for a categorical draw). */
#define ORC_NEAR 1e-6

/* Planted-mistake switch used only by the oracle's own pin tests, to show
 * that the statistical pins reject a plausibly wrong implementation.
 * 0 = the method as the pages state it. */
static int g_mutation = 0;
void oracle_set_mutation(int m) { g_mutation = m; }
int oracle_get_mutation(void) { return g_mutation; }

/* ------------------------------------------------------------------------
 * Philox4x32-10 [PH]: a 10-round bijection on a 128-bit counter under a
 * 64-bit key.  Each round multiplies words 0 and 2 by fixed 32-bit
 * multipliers, splits the 64-bit products into high and low halves and
 * recombines them with words 1 and 3 and the round key.  The key is bumped
 * by the two Weyl constants between rounds.
 * ---------------------------------------------------------------------- */
static const uint32_t PH_MUL0 = 0xD2511F53u;
static const uint32_t PH_MUL1 = 0xCD9E8D57u;
static const uint32_t PH_WEYL0 = 0x9E3779B9u; /* golden ratio */
static const uint32_t PH_WEYL1 = 0xBB67AE85u; /* sqrt(3) - 1 */

void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                          uint32_t out[4])
{
    uint32_t x0 = ctr_in[0], x1 = ctr_in[1], x2 = ctr_in[2], x3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PH_WEYL0;
            k1 += PH_WEYL1;
        }
        uint64_t prod0 = (uint64_t)PH_MUL0 * (uint64_t)x0;
        uint64_t prod1 = (uint64_t)PH_MUL1 * (uint64_t)x2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t y0 = hi1 ^ x1 ^ k0;
        uint32_t y1 = lo1;
        uint32_t y2 = hi0 ^ x3 ^ k1;
        uint32_t y3 = lo0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* The two uniforms of (row, position): counter = (position, row,
 * offset_lo, offset_hi), key = (seed_lo, seed_hi); the top 24 bits of a
 * word scaled by 2^-24 give a uniform in [0,1) that is exact in fp32. */
static void uniforms(uint64_t seed, uint64_t offset, uint32_t row,
                     uint32_t pos, double* u_acc, double* u_smp)
{
    uint32_t ctr[4] = {pos, row, (uint32_t)offset, (uint32_t)(offset >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    oracle_philox4x32_10(ctr, key, r);
    *u_acc = (double)(r[0] >> 8) * 0x1p-24;
    *u_smp = (double)(r[1] >> 8) * 0x1p-24;
}

void oracle_uniforms(uint64_t seed, uint64_t offset, uint32_t row,
                     uint32_t pos, double out[2])
{
    uniforms(seed, offset, row, pos, &out[0], &out[1]);
}

/* ------------------------------------------------------------------------
 * Temperature softmax [P1 listing: softmax of the target logits divided by
 * the temperature].  m = max_j z_j; e_j = exp((z_j - m)/T); S = sum_j e_j;
 * p_j = e_j / S.  Returns 0 when the position is finite and has at least one
 * finite logit, else ORC_ROW_NONFINITE (NaN or +Inf anywhere, or every logit
 * -Inf).
 * ---------------------------------------------------------------------- */
static int check_position(const float* z, int64_t V)
{
    int any_finite = 0;
    for (int64_t j = 0; j < V; ++j) {
        double v = (double)z[j];
        if (isnan(v) || (isinf(v) && v > 0)) return ORC_ROW_NONFINITE;
        if (isfinite(v)) any_finite = 1;
    }
    return any_finite ? 0 : ORC_ROW_NONFINITE;
}

static double pos_max(const float* z, int64_t V)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < V; ++j)
        if ((double)z[j] > m) m = (double)z[j];
    return m;
}

/* e_j written to e[] (may be NULL); returns S. */
static double pos_exp(const float* z, int64_t V, double m, double T, double* e)
{
    double S = 0.0;
    for (int64_t j = 0; j < V; ++j) {
        double ej = exp(((double)z[j] - m) / T);
        if (e) e[j] = ej;
        S += ej;
    }
    return S;
}

/* Exported for tests: p = softmax(z / T) of one position, in fp64. */
void oracle_softmax(const float* z, int64_t V, double T, double* p)
{
    double m = pos_max(z, V);
    double S = pos_exp(z, V, m, T, p);
    for (int64_t j = 0; j < V; ++j) p[j] /= S;
}

/* ------------------------------------------------------------------------
 * Categorical draw by inverse CDF.  The pages draw with torch.multinomial
 * [P1 listing], which fixes no mapping from uniforms to tokens; the reading
 * taken: t = u * sum(w); return the smallest j with sum_{k<=j} w_k > t.  A
 * zero-weight token is never chosen.  If rounding leaves no such j, return
 * the last j with w_j > 0.  *near is set when t lies within ORC_NEAR*sum(w)
 * of either prefix sum that brackets the chosen token.
 * ---------------------------------------------------------------------- */
static int64_t inv_cdf(const double* w, int64_t V, double u, int* near)
{
    double total = 0.0;
    for (int64_t j = 0; j < V; ++j) total += w[j];
    double t = u * total;
    double c = 0.0, c_prev = 0.0;
    int64_t chosen = -1;
    for (int64_t j = 0; j < V; ++j) {
        c_prev = c;
        c += w[j];
        if (c > t) { chosen = j; break; }
    }
    if (chosen < 0) {
        for (int64_t j = V - 1; j >= 0; --j)
            if (w[j] > 0.0) { chosen = j; break; }
        c = total;
        c_prev = total;
    }
    *near = (fabs(t - c_prev) < ORC_NEAR * total) || (fabs(c - t) < ORC_NEAR * total);
    return chosen;
}

/* ------------------------------------------------------------------------
 * One row of the batched accept/reject pass.
 * ---------------------------------------------------------------------- */
typedef struct {
    const float* logits;       /* [B, K+1, V] */
    const float* draft_probs;  /* [B, K, V] or NULL when greedy */
    const int32_t* draft_tokens; /* [B, K] */
    const int32_t* draft_lens;   /* [B] or NULL (all K) */
    int64_t B, V;
    int K;
    int64_t row_base;
    double T;
    uint64_t seed, offset;
    int32_t* out_tokens;      /* [B, K+1] */
    int32_t* out_accepted;    /* [B] */
    double* out_p_draft;      /* [B, K] or NULL */
    int32_t* out_status;      /* [B] or NULL */
    int32_t* out_near_acc;    /* [B] or NULL: first near-threshold acceptance position, else -1 */
    int32_t* out_near_smp;    /* [B] or NULL: 1 when the categorical draw was near-threshold */
    double* out_resid_mass;   /* [B] or NULL: S_r at a rejection, else -1 */
} job_t;

static void do_row(const job_t* jb, int64_t b, double* e, double* w)
{
    const int K = jb->K;
    const int64_t V = jb->V;
    const int greedy = (jb->T == 0.0);
    const double T = (g_mutation == 6) ? 1.0 : jb->T; /* 6 = planted */
    int32_t* tok_out = jb->out_tokens + b * (K + 1);
    for (int i = 0; i <= K; ++i) tok_out[i] = -1;
    if (jb->out_p_draft)
        for (int i = 0; i < K; ++i) jb->out_p_draft[b * K + i] = -1.0;
    jb->out_accepted[b] = -1;
    if (jb->out_near_acc) jb->out_near_acc[b] = -1;
    if (jb->out_near_smp) jb->out_near_smp[b] = 0;
    if (jb->out_resid_mass) jb->out_resid_mass[b] = -1.0;

    const int32_t* x = jb->draft_tokens + b * K;
    const float* zrow = jb->logits + b * (int64_t)(K + 1) * V;
    const float* qrow = jb->draft_probs ? jb->draft_probs + b * (int64_t)K * V : NULL;

    /* Step 1: validate the drafted tokens: the length, every token's range
     * and (stochastic mode) q_i(x_i) > 0, for all L drafts. */
    int status = 0;
    int L = jb->draft_lens ? jb->draft_lens[b] : K;
    if (L < 0 || L > K) {
        status |= ORC_ROW_BAD_LEN;
    } else {
        for (int i = 0; i < L; ++i)
            if (x[i] < 0 || (int64_t)x[i] >= V) status |= ORC_ROW_BAD_TOKEN;
        if (!greedy)
            for (int i = 0; i < L; ++i)
                if (x[i] >= 0 && (int64_t)x[i] < V) {
                    double qx = (double)qrow[(int64_t)i * V + x[i]];
                    if (!(qx > 0.0)) status |= ORC_ROW_ZERO_Q;
                }
    }
    if (status) {
        if (jb->out_status) jb->out_status[b] = status;
        return;
    }
    const uint32_t grow = (uint32_t)(jb->row_base + b);

    /* The target's distributions are read in the listing's order: position
     * i only when every draft before it was accepted, and position L (the
     * bonus) only when all L were [P1 listing: the loop breaks at the first
     * rejection].  A position read this way must be finite: a NaN or +Inf
     * logit, or all logits -Inf, makes the row invalid (ROW_NONFINITE);
     * positions after the stop are never read. */
    if (greedy) {
        /* Greedy limit [P2 "Speculative decoding": keep the longest prefix the
         * target agrees with, then take the target's own token]. */
        int a = L;
        for (int i = 0; i <= L; ++i) {
            const float* z = zrow + (int64_t)i * V;
            if (check_position(z, V)) {
                if (jb->out_p_draft)
                    for (int k = 0; k < K; ++k) jb->out_p_draft[b * K + k] = -1.0;
                if (jb->out_status) jb->out_status[b] = ORC_ROW_NONFINITE;
                return;
            }
            if (i == L) break;
            int64_t g = 0;
            for (int64_t j = 1; j < V; ++j)
                if ((double)z[j] > (double)z[g]) g = j;
            if (jb->out_p_draft) jb->out_p_draft[b * K + i] = (x[i] == g) ? 1.0 : 0.0;
            if (x[i] != g) { a = i; break; }
        }
        const float* z = zrow + (int64_t)a * V;
        int64_t g = 0;
        for (int64_t j = 1; j < V; ++j)
            if ((double)z[j] > (double)z[g]) g = j;
        for (int i = 0; i < a; ++i) tok_out[i] = x[i];
        tok_out[a] = (int32_t)g;
        jb->out_accepted[b] = a;
        if (jb->out_status) jb->out_status[b] = 0;
        return;
    }

    /* Steps 2 and 3: at each drafted position in turn, p_i(x_i) and the
     * acceptance test, stopping at the first rejection [P1 listing: accept
     * with probability min(1, p/q), else resample and stop the round; P2
     * "Speculative decoding": acceptance rule]. */
    int a = L;
    int near_acc = -1;
    for (int i = 0; i <= L; ++i) {
        const float* z = zrow + (int64_t)i * V;
        if (check_position(z, V)) {
            if (jb->out_p_draft)
                for (int k = 0; k < K; ++k) jb->out_p_draft[b * K + k] = -1.0;
            if (jb->out_status) jb->out_status[b] = ORC_ROW_NONFINITE;
            return;
        }
        if (i == L) break;
        const float* q = qrow + (int64_t)i * V;
        double m = pos_max(z, V);
        double S = pos_exp(z, V, m, T, NULL);
        double px = exp(((double)z[x[i]] - m) / T) / S;
        if (jb->out_p_draft) jb->out_p_draft[b * K + i] = px;
        double qx = (double)q[x[i]];
        double ratio = (g_mutation == 3) ? qx / px : px / qx;
        double acc = ratio < 1.0 ? ratio : 1.0;
        double u_acc, u_smp;
        uniforms(jb->seed, jb->offset, grow, (uint32_t)i, &u_acc, &u_smp);
        if (near_acc < 0 && fabs(u_acc - acc) < ORC_NEAR) near_acc = i;
        if (g_mutation == 8 && i == 0) continue; /* planted: skip a test */
        if (!(u_acc < acc)) {
            a = i;
            if (g_mutation != 7) break; /* 7 = planted: keep testing */
        }
    }

    /* Step 4: the token at position a -- residual resample after a
     * rejection [P1 listing: normalised relu(p - q)], or the bonus token
     * from p at position L when every draft was accepted [P1 listing: the
     * loop's else-branch]. */
    int smp_pos = (g_mutation == 4 && a == L && L > 0) ? L - 1 : a;
    const float* z = zrow + (int64_t)smp_pos * V;
    double m = pos_max(z, V);
    double S = pos_exp(z, V, m, T, e);
    double u_acc, u_smp;
    uniforms(jb->seed, jb->offset, grow, (uint32_t)a, &u_acc, &u_smp);
    double u_draw = (g_mutation == 5) ? u_acc : u_smp;
    int near_smp = 0;
    int64_t token;
    if (a < L) {
        const float* q = qrow + (int64_t)a * V;
        double Sr = 0.0;
        for (int64_t j = 0; j < V; ++j) {
            double pj = e[j] / S;
            double qj = (double)q[j];
            double rj;
            if (g_mutation == 1) rj = pj;                       /* planted */
            else if (g_mutation == 2) rj = fmax(qj - pj, 0.0);  /* planted */
            else rj = fmax(pj - qj, 0.0);
            w[j] = rj;
            Sr += rj;
        }
        if (jb->out_resid_mass) jb->out_resid_mass[b] = Sr;
        if (Sr > 0.0) {
            token = inv_cdf(w, V, u_draw, &near_smp);
        } else {
            status |= ORC_ROW_RESID_ZERO;
            token = inv_cdf(e, V, u_draw, &near_smp);
        }
    } else {
        token = inv_cdf(e, V, u_draw, &near_smp);
    }
    for (int i = 0; i < a; ++i) tok_out[i] = x[i];
    tok_out[a] = (int32_t)token;
    jb->out_accepted[b] = a;
    if (jb->out_status) jb->out_status[b] = status;
    if (jb->out_near_acc) jb->out_near_acc[b] = near_acc;
    if (jb->out_near_smp) jb->out_near_smp[b] = near_smp;
}

/* Batched accept/reject over B independent rows.  Returns 0, or -1 on an
 * invalid argument (nothing written). */
int oracle_spec_accept(const float* logits, const float* draft_probs,
                       const int32_t* draft_tokens, const int32_t* draft_lens,
                       int64_t B, int K, int64_t V, int64_t row_base,
                       double temperature, uint64_t seed, uint64_t offset,
                       int32_t* out_tokens, int32_t* out_accepted,
                       double* out_p_draft, int32_t* out_status,
                       int32_t* out_near_acc, int32_t* out_near_smp,
                       double* out_resid_mass, int nthreads)
{
    if (!logits || !draft_tokens || !out_tokens || !out_accepted) return -1;
    if (B < 0 || K < 0 || V < 1 || row_base < 0) return -1;
    if (!(temperature >= 0.0) || isinf(temperature)) return -1;
    if (temperature > 0.0 && !draft_probs) return -1;
    job_t jb = {logits, draft_probs, draft_tokens, draft_lens, B, V, K, row_base,
                temperature, seed, offset, out_tokens, out_accepted, out_p_draft,
                out_status, out_near_acc, out_near_smp, out_resid_mass};
    int bad_alloc = 0;
    if (nthreads < 1) nthreads = 1;
#ifdef _OPENMP
#pragma omp parallel num_threads(nthreads) reduction(| : bad_alloc)
#endif
    {
        double* e = (double*)malloc(sizeof(double) * (size_t)V);
        double* w = (double*)malloc(sizeof(double) * (size_t)V);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
        for (int64_t b = 0; b < B; ++b) {
            if (!e || !w) { bad_alloc = 1; continue; }
            do_row(&jb, b, e, w);
        }
        free(e);
        free(w);
    }
    return bad_alloc ? -2 : 0;
}
