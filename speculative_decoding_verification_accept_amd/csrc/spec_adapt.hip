// spec_adapt.hip -- acceptance telemetry and the adaptive draft depth, on
// the GPU, right after the accept/reject pass that produced out_accepted.
//
// Sources (by page title and section):
//  * "Decode is memory-bound: ~59 tok/s ceiling on an RTX 4090, and how
//    speculative decoding beats it" (trefon.com): section "Two things that
//    follow from the math" (the fork's adaptive mode caps the draft depth
//    once the measured acceptance falls under 35%, where extra drafts add
//    almost nothing); the closing rules (choose the depth from the measured
//    acceptance and keep measuring, since it moves with the text); section
//    "Speculative decoding" (expected tokens per pass 1 + a + ... + a^k and
//    the speedup over (k c + 1) for a draft step costing c).
//  * "Speculative decoding and early exit: accelerated autoregressive
//    decoding" (reactapp.top): section "Production perspective" (acceptance
//    rate and mean accepted length as shipped metrics) and the operational
//    checklist (record acceptance histograms).
//
// One thread per row.  The row's 64-byte record holds a ring of its last 16
// passes as (accepted drafts, tests run) byte pairs; a pass that accepted a
// of L drafts ran a + 1 tests if a < L (the last one failed), else a.  The
// measured acceptance is S / N summed over the last W recorded passes, in
// exact integers.  Telemetry counts are integer sums, first per workgroup
// in LDS (wave ballots for the per-position counts), then added to the
// caller's 64-bit counters with global atomics: the result is independent
// of the order in which rows are visited.  The depth rules' floating point
// is fp64 with no contraction (this file is built with -ffp-contract=off),
// each expression in the order written.
#include <math.h>

#include "device_common.hpp"
#include "spec_verify.h"

namespace specv {
namespace {

constexpr int kThreads = 256;
constexpr int kRing = 16;
constexpr int kMaxK = SPEC_ADAPT_MAX_K;
constexpr int kHistSide = kMaxK + 1;

// telemetry word offsets (uint64 words; the layout is part of the ABI)
constexpr int kRows = 0, kInvalid = 1, kDrafted = 2, kTested = 3, kAccepted = 4, kEmitted = 5,
              kCalls = 6;
constexpr int kTestedAt = 8;
constexpr int kAcceptedAt = kTestedAt + kMaxK;
constexpr int kDepthHist = kAcceptedAt + kMaxK;
constexpr int kHist = kDepthHist + kMaxK + 1;
constexpr int kUsed = kHist + kHistSide * kHistSide;
static_assert(kUsed <= SPEC_ADAPT_TELEMETRY_WORDS, "telemetry layout");

struct AdaptArgs {
    const int32_t* accepted;
    const int32_t* lens;
    uint8_t* state;
    unsigned long long* tel;
    int32_t* next_lens;
    int64_t B;
    int K, k_min, k_max, window, policy;
    double floor, cost;
};

__device__ __forceinline__ uint32_t get_byte(const uint4& r, int s) {
    const uint32_t w = s < 4 ? r.x : s < 8 ? r.y : s < 12 ? r.z : r.w;
    return (w >> ((s & 3) * 8)) & 0xFFu;
}

__device__ __forceinline__ void set_byte(uint4& r, uint32_t slot, uint32_t v) {
    const uint32_t sh = (slot & 3u) * 8u, keep = ~(0xFFu << sh), put = (v & 0xFFu) << sh;
    const uint32_t w = slot >> 2;
    r.x = w == 0 ? (r.x & keep) | put : r.x;
    r.y = w == 1 ? (r.y & keep) | put : r.y;
    r.z = w == 2 ? (r.z & keep) | put : r.z;
    r.w = w == 3 ? (r.w & keep) | put : r.w;
}

// E(a, k) / (k c + 1) maximised over k in [k_min, k_max], lowest k on ties.
__device__ int speedup_depth(double alpha, int k_min, int k_max, double cost) {
    double e = 1.0, term = 1.0;
    for (int k = 1; k < k_min; ++k) {
        term = term * alpha;
        e = e + term;
    }
    int best_k = k_min;
    double best = -1.0;
    for (int k = k_min; k <= k_max; ++k) {
        if (k > 0) {
            term = term * alpha;
            e = e + term;
        }
        const double g = e / ((double)k * cost + 1.0);
        if (g > best) {
            best = g;
            best_k = k;
        }
    }
    return best_k;
}

__global__ __launch_bounds__(kThreads) void k_adapt(AdaptArgs a) {
    __shared__ uint32_t cnt[kUsed];
    const int t = threadIdx.x, lane = t & (kWave - 1);
    for (int i = t; i < kUsed; i += kThreads) cnt[i] = 0;
    __syncthreads();

    for (int64_t base = (int64_t)blockIdx.x * kThreads; base < a.B; base += (int64_t)gridDim.x * kThreads) {
        const int64_t b = base + t;
        const bool active = b < a.B;
        int L = 0, acc = -1, tests = 0;
        bool valid = false;
        if (active) {
            acc = a.accepted[b];
            L = a.lens ? a.lens[b] : a.K;
            valid = L >= 0 && L <= a.K && acc >= 0 && acc <= L;
            uint4* rec = reinterpret_cast<uint4*>(a.state + b * SPEC_ADAPT_STATE_BYTES);
            uint4 succ = rec[0], trials = rec[1], meta = rec[2];
            uint32_t count = meta.x;
            if (valid) {
                tests = acc + (acc < L ? 1 : 0);
                if (tests > 0) {
                    set_byte(succ, count & (kRing - 1), (uint32_t)acc);
                    set_byte(trials, count & (kRing - 1), (uint32_t)tests);
                    count += 1;
                }
            }
            const uint32_t n = min((uint32_t)a.window, min(count, (uint32_t)kRing));
            uint32_t S = 0, N = 0;
#pragma unroll
            for (int s = 0; s < kRing; ++s) {
                const bool in = ((count - 1u - (uint32_t)s) & (kRing - 1)) < n;
                S += in ? get_byte(succ, s) : 0u;
                N += in ? get_byte(trials, s) : 0u;
            }
            int d;
            if (N == 0)
                d = a.k_max;
            else if (a.policy == SPEC_ADAPT_THRESHOLD)
                d = (double)S < a.floor * (double)N ? a.k_min : a.k_max;
            else
                d = speedup_depth((double)S / (double)N, a.k_min, a.k_max, a.cost);
            meta.x = count;
            meta.y = (uint32_t)d;
            rec[0] = succ;
            rec[1] = trials;
            rec[2] = meta;
            a.next_lens[b] = d;
            if (valid) atomicAdd(&cnt[kHist + L * kHistSide + acc], 1u);
            atomicAdd(&cnt[kDepthHist + d], 1u);
        }
        // counts over the wave: one LDS add per wave and counter
        const uint32_t rows = (uint32_t)__popcll(__ballot(valid));
        const uint32_t invalid = (uint32_t)__popcll(__ballot(active && !valid));
        const uint32_t drafted = wave_sum((uint32_t)(valid ? L : 0));
        const uint32_t tested = wave_sum((uint32_t)tests);
        const uint32_t accepted = wave_sum((uint32_t)(valid ? acc : 0));
        if (lane == 0) {
            if (rows) {
                atomicAdd(&cnt[kRows], rows);
                atomicAdd(&cnt[kDrafted], drafted);
                atomicAdd(&cnt[kTested], tested);
                atomicAdd(&cnt[kAccepted], accepted);
                atomicAdd(&cnt[kEmitted], accepted + rows);
            }
            if (invalid) atomicAdd(&cnt[kInvalid], invalid);
        }
        for (int i = 0; i < a.K; ++i) {
            const uint32_t ta = (uint32_t)__popcll(__ballot(tests > i));
            const uint32_t aa = (uint32_t)__popcll(__ballot(valid && acc > i));
            if (lane == 0 && ta) atomicAdd(&cnt[kTestedAt + i], ta);
            if (lane == 0 && aa) atomicAdd(&cnt[kAcceptedAt + i], aa);
        }
    }
    __syncthreads();
    for (int i = t; i < kUsed; i += kThreads) {
        const uint32_t v = cnt[i];
        if (v) atomicAdd(&a.tel[i], (unsigned long long)v);
    }
    if (blockIdx.x == 0 && t == 0) atomicAdd(&a.tel[kCalls], 1ull);
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_adapt_state_bytes(int64_t B) {
    return B < 0 ? 0 : (size_t)B * SPEC_ADAPT_STATE_BYTES;
}

extern "C" size_t spec_adapt_telemetry_bytes(void) {
    return (size_t)SPEC_ADAPT_TELEMETRY_WORDS * sizeof(uint64_t);
}

extern "C" int spec_adapt(const int32_t* accepted, const int32_t* draft_lens, int64_t B, int K,
                          void* state, uint64_t* telemetry, int32_t* next_lens, int k_min,
                          int k_max, int window, int policy, double accept_floor,
                          double draft_cost, void* stream) {
    if (B < 0 || B > ((int64_t)1 << 31) || K < 0 || K > kMaxK) return SPEC_ERR_INVALID_ARG;
    if (k_min < 1 || k_min > k_max || k_max > kMaxK) return SPEC_ERR_INVALID_ARG;
    if (window < 1 || window > kRing) return SPEC_ERR_INVALID_ARG;
    if (policy != SPEC_ADAPT_THRESHOLD && policy != SPEC_ADAPT_SPEEDUP) return SPEC_ERR_INVALID_ARG;
    if (!(accept_floor >= 0.0 && accept_floor <= 1.0)) return SPEC_ERR_INVALID_ARG;
    if (!(draft_cost >= 0.0) || isinf(draft_cost)) return SPEC_ERR_INVALID_ARG;
    if (!telemetry || (reinterpret_cast<uintptr_t>(telemetry) & 7)) return SPEC_ERR_INVALID_ARG;
    if (B > 0 && (!accepted || !next_lens || !state)) return SPEC_ERR_INVALID_ARG;
    if (state && (reinterpret_cast<uintptr_t>(state) & 15)) return SPEC_ERR_INVALID_ARG;
    AdaptArgs a{};
    a.accepted = accepted;
    a.lens = draft_lens;
    a.state = static_cast<uint8_t*>(state);
    a.tel = reinterpret_cast<unsigned long long*>(telemetry);
    a.next_lens = next_lens;
    a.B = B;
    a.K = K;
    a.k_min = k_min;
    a.k_max = k_max;
    a.window = window;
    a.policy = policy;
    a.floor = accept_floor;
    a.cost = draft_cost;
    // a call with B == 0 still counts itself in the telemetry
    const int64_t blocks = B == 0 ? 1 : std::min<int64_t>((B + kThreads - 1) / kThreads, 256);
    hipLaunchKernelGGL(k_adapt, dim3((unsigned)blocks), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
