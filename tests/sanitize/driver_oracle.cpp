// Exercises the C oracle and the library's host-only C++ (the depth planner,
// the status strings) on small inputs covering their edge cases; built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py,
// which fails on any report.  Exit status 0 when every check holds.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "spec_verify.h"

extern "C" {
void oracle_set_mutation(int m);
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]);
void oracle_uniforms(uint64_t seed, uint64_t offset, uint32_t row, uint32_t pos, double out[2]);
void oracle_softmax(const float* z, int64_t V, double T, double* p);
int oracle_spec_accept(const float* logits, const float* draft_probs, const int32_t* draft_tokens,
                       const int32_t* draft_lens, int64_t B, int K, int64_t V, int64_t row_base,
                       double temperature, uint64_t seed, uint64_t offset, int32_t* out_tokens,
                       int32_t* out_accepted, double* out_p_draft, int32_t* out_status,
                       int32_t* out_near_acc, int32_t* out_near_smp, double* out_resid_mass,
                       int nthreads);
}

static int g_fail = 0;
#define CHECK(c)                                                    \
    do {                                                            \
        if (!(c)) {                                                 \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            g_fail = 1;                                             \
        }                                                           \
    } while (0)

static uint32_t lcg(uint64_t& s) {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(s >> 33);
}

static void run_accept(int B, int K, int V, double T, bool ragged, bool with_q, int mutation, uint64_t seed) {
    uint64_t s = seed;
    std::vector<float> z((size_t)B * (K + 1) * V), q((size_t)B * K * V + 1);  // q never empty either
    for (auto& v : z) v = (float)((lcg(s) % 2000) / 250.0 - 4.0);
    for (int r = 0; r < B * K; ++r) {
        double tot = 0;
        for (int j = 0; j < V; ++j) tot += (q[(size_t)r * V + j] = (float)(1 + lcg(s) % 100));
        for (int j = 0; j < V; ++j) q[(size_t)r * V + j] = (float)(q[(size_t)r * V + j] / tot);
    }
    std::vector<int32_t> x((size_t)B * K + 1), L(B);  // never empty: K = 0 still passes a token array
    for (size_t i = 0; i < (size_t)B * K; ++i) x[i] = (int32_t)(lcg(s) % V);
    for (int b = 0; b < B; ++b) L[b] = ragged ? (int32_t)(lcg(s) % (K + 1)) : K;
    if (B > 2 && K > 0) {
        z[(size_t)1 * (K + 1) * V + 0] = NAN;         // row 1, position 0: not finite
        x[(size_t)2 * K] = V + 3;                     // row 2: a token out of range
    }
    if (B > 3) L[3] = K + 1;                          // row 3: bad length
    std::vector<int32_t> tok((size_t)B * (K + 1)), acc(B), st(B), na(B), ns(B);
    std::vector<double> pd((size_t)B * K), rm(B);
    oracle_set_mutation(mutation);
    const int rc = oracle_spec_accept(z.data(), with_q ? q.data() : nullptr, x.data(), L.data(), B, K, V, 7,
                                      T, seed, 3, tok.data(), acc.data(), pd.data(), st.data(), na.data(),
                                      ns.data(), rm.data(), 1);
    oracle_set_mutation(0);
    CHECK(rc == 0);
    for (int b = 0; b < B; ++b) {
        if (acc[b] < 0) continue;
        CHECK(acc[b] <= L[b]);
        CHECK(tok[(size_t)b * (K + 1) + acc[b]] >= 0 && tok[(size_t)b * (K + 1) + acc[b]] < V);
    }
}

int main() {
    // Philox: a bijection sample and determinism
    uint32_t c[4] = {1, 2, 3, 4}, k[2] = {5, 6}, o1[4], o2[4];
    oracle_philox4x32_10(c, k, o1);
    oracle_philox4x32_10(c, k, o2);
    CHECK(memcmp(o1, o2, sizeof(o1)) == 0);
    double u[2];
    oracle_uniforms(~0ull, ~0ull, 0xFFFFFFFFu, 255, u);
    CHECK(u[0] >= 0 && u[0] < 1 && u[1] >= 0 && u[1] < 1);
    // softmax, including -inf entries and one entry
    float zs[5] = {1.f, -INFINITY, 3.f, 0.f, -2.f};
    double p[5];
    oracle_softmax(zs, 5, 0.7, p);
    double tot = 0;
    for (double v : p) tot += v;
    CHECK(fabs(tot - 1.0) < 1e-12 && p[1] == 0.0);
    oracle_softmax(zs, 1, 1.0, p);
    CHECK(p[0] == 1.0);
    // accept/reject: stochastic, greedy, ragged, K = 0, V = 1, every planted mistake
    run_accept(6, 3, 11, 0.8, true, true, 0, 1);
    run_accept(6, 3, 11, 0.0, true, false, 0, 2);
    run_accept(5, 0, 9, 0.9, false, true, 0, 3);
    run_accept(4, 2, 1, 1.0, false, true, 0, 4);
    run_accept(1, 5, 300, 0.6, false, true, 0, 5);
    for (int m = 1; m <= 8; ++m) run_accept(6, 4, 13, 0.7, true, true, m, 10 + m);
    // argument rejection
    float z1 = 0.f;
    int32_t x1 = 0, t1[2], a1;
    double pd1;
    CHECK(oracle_spec_accept(&z1, nullptr, &x1, nullptr, 1, 1, 1, 0, 0.5, 1, 0, t1, &a1, &pd1, nullptr,
                             nullptr, nullptr, nullptr, 1) == -1);
    // the depth planner (host C++): a measured-curve shape, and bad arguments
    const int64_t mp[4] = {1, 32, 256, 1024};
    const double tp[4] = {25.0, 30.0, 46.0, 122.0};
    const int64_t bs[3] = {1, 8, 128};
    int32_t best[3];
    double sp[3 * 8], rate[3 * 8];
    uint8_t par[3 * 8];
    CHECK(spec_plan_depth(mp, tp, 4, bs, 3, 7, 0.8, 0.05, best, sp, rate, par) == SPEC_OK);
    for (int i = 0; i < 3; ++i) CHECK(best[i] >= 0 && best[i] <= 7);
    CHECK(spec_plan_depth(mp, tp, 4, bs, 3, 7, 1.5, 0.05, best, sp, rate, par) == SPEC_ERR_INVALID_ARG);
    CHECK(spec_plan_depth(mp, tp, 0, bs, 3, 7, 0.5, 0.05, best, sp, rate, par) == SPEC_ERR_INVALID_ARG);
    CHECK(spec_plan_depth(mp, tp, 4, bs, 3, 7, 0.5, 0.05, best, nullptr, nullptr, nullptr) == SPEC_OK);
    CHECK(spec_plan_depth(mp, tp, 4, bs, 3, 7, 0.5, 0.05, nullptr, sp, rate, par) == SPEC_ERR_INVALID_ARG);
    // status strings
    for (int code = -5; code <= 2; ++code) CHECK(spec_status_string(code) != nullptr);
    CHECK(spec_abi_version() == SPEC_VERIFY_ABI_VERSION);
    if (!g_fail) printf("sanitized oracle and host code: all checks passed\n");
    return g_fail;
}
