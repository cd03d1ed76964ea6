// spec_plan.cpp -- host-side draft-depth planner over a measured verify-cost
// curve.  No GPU work: it turns timings of the verify pass at M rows into
// the depth D to run at each batch size B, and the throughput/interactivity
// frontier over (B, D).
//
// Sources (by page title and section):
//  * "Decode is memory-bound: ~59 tok/s ceiling on an RTX 4090, and how
//    speculative decoding beats it" (trefon.com), section "Speculative
//    decoding": expected tokens per pass E(a, k) = 1 + a + ... + a^k for
//    independent per-draft acceptance a, and the speedup E / (k c + 1) when
//    a draft step costs c of a target pass.
//  * agentnet.co.il item on speculative decoding, section "The formula
//    behind the speedup": speculation pays when the verify time at B(1+D)
//    rows, relative to that at B rows, is below the accepted length; the
//    best D depends on B and moves along a Pareto frontier of throughput
//    against interactivity.  Section "GEMM-M grows, a small batch
//    suffices": every linear layer sees M = B(1+D) rows.
//
// The pass at batch B and depth D costs T(B(1+D)) + D c T(B): the verify
// pass at its widened row count plus D draft steps at batch B.  T is the
// measured curve, linear between points, flat below the first point, and
// continued with the last segment's slope above the last.  All arithmetic is
// fp64 in the order written (built with -ffp-contract=off).
#include <math.h>
#include <stdint.h>

#include <vector>

#include "spec_verify.h"

namespace {

double verify_time(int64_t M, const int64_t* m, const double* t, int n) {
    if (n == 1 || M <= m[0]) return t[0];
    int j = 1;
    while (j < n - 1 && M > m[j]) ++j;
    const double m0 = (double)m[j - 1], m1 = (double)m[j];
    const double t0 = t[j - 1], t1 = t[j];
    return t0 + ((t1 - t0) * ((double)M - m0)) / (m1 - m0);
}

}  // namespace

extern "C" int spec_plan_depth(const int64_t* m_pts, const double* t_pts, int n_pts,
                               const int64_t* batches, int n_batches, int d_max, double alpha,
                               double draft_cost, int32_t* out_best_depth, double* out_speedup,
                               double* out_tokens_per_s, uint8_t* out_pareto) {
    if (!m_pts || !t_pts || n_pts < 1 || !batches || n_batches < 1 || !out_best_depth)
        return SPEC_ERR_INVALID_ARG;
    if (d_max < 0 || d_max > SPEC_MAX_DRAFT) return SPEC_ERR_INVALID_ARG;
    if (!(alpha >= 0.0 && alpha <= 1.0)) return SPEC_ERR_INVALID_ARG;
    if (!(draft_cost >= 0.0) || isinf(draft_cost)) return SPEC_ERR_INVALID_ARG;
    for (int i = 0; i < n_pts; ++i) {
        if (m_pts[i] < 1 || (i > 0 && m_pts[i] <= m_pts[i - 1])) return SPEC_ERR_INVALID_ARG;
        if (!(t_pts[i] > 0.0) || isinf(t_pts[i])) return SPEC_ERR_INVALID_ARG;
    }
    for (int i = 0; i < n_batches; ++i)
        if (batches[i] < 1 || batches[i] > ((int64_t)1 << 31)) return SPEC_ERR_INVALID_ARG;

    const int nd = d_max + 1;
    std::vector<double> rate((size_t)n_batches * nd), user((size_t)n_batches * nd);
    for (int bi = 0; bi < n_batches; ++bi) {
        const int64_t B = batches[bi];
        const double tb = verify_time(B, m_pts, t_pts, n_pts);
        double e = 1.0, term = 1.0, top = -1.0;
        int best = 0;
        for (int D = 0; D <= d_max; ++D) {
            if (D > 0) {
                term = term * alpha;
                e = e + term;
            }
            const double den = verify_time(B * (1 + D), m_pts, t_pts, n_pts) + ((double)D * draft_cost) * tb;
            const double s = (e * tb) / den;
            const size_t o = (size_t)bi * nd + D;
            rate[o] = ((double)B * e) / den * 1e6;
            user[o] = e / den * 1e6;
            if (out_speedup) out_speedup[o] = s;
            if (s > top) {
                top = s;
                best = D;
            }
        }
        out_best_depth[bi] = best;
    }
    if (out_tokens_per_s)
        for (size_t o = 0; o < rate.size(); ++o) out_tokens_per_s[o] = rate[o];
    if (out_pareto) {
        const size_t n = rate.size();
        for (size_t i = 0; i < n; ++i) {
            bool dominated = false;
            for (size_t j = 0; j < n && !dominated; ++j)
                dominated = j != i && rate[j] >= rate[i] && user[j] >= user[i] &&
                            (rate[j] > rate[i] || user[j] > user[i]);
            out_pareto[i] = dominated ? 0 : 1;
        }
    }
    return SPEC_OK;
}
