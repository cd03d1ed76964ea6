// spec_accept_sampled.hip -- accept/reject with the production sampler's
// filters: the draft arrives as logits, and the target's and the draft's
// tempered distributions pass through top-p and min-p before the acceptance
// rule, the residual and the bonus draw.
//
// Sources (by page title and section):
//  * "Decode is memory-bound: ~59 tok/s ceiling on an RTX 4090, and how
//    speculative decoding beats it" (trefon.com), section "Two things that
//    follow from the math": the production sampler (temperature 0.6, top-p
//    0.95, min-p 0.05) and the draft sampler matched to the target's;
//    section "Speculative decoding": accepting with probability
//    min(1, p(x)/q(x)) leaves exactly the target distribution.
//  * "Speculative decoding and early exit ..." (reactapp.top), section
//    "Speculative decoding: draft first, then verify", listing
//    speculative_decode: q is the tempered softmax of the draft's logits;
//    accept/reject, residual resample, bonus token.
//
// Filters.  On softmax(z / T): top-p keeps token j iff the mass of the
// tokens with a strictly larger logit is below top_p; min-p keeps j iff
// p_j >= min_p max p; kept iff both keep it; the kept mass is renormalised.
//
// Two launches, nothing waits:
//  k_stats   one workgroup per distribution row (target positions 0..L_b,
//            draft positions 0..L_b-1).  Pass 1: the max m.  Pass 2 (top-p
//            only): every entry's weight e = 2^(fl(z c - fl(m c))), c =
//            log2(e)/T, in 2^-40 fixed point (exact, order-free integer
//            sums) into a histogram of 512 bins of u = m c - z c (1/16 wide;
//            entries past u = 32 count in the total only), which finds the bin where
//            the mass from the top first reaches top_p of the total; that
//            bin's entries are collected in LDS (one LDS atomic per wave),
//            and a radix select on their order-preserving fp32 keys (4 digits
//            of 8 bits, fixed-point mass histograms) finds the exact logit
//            at which the mass reaches top_p: kept iff key(z) >= that key.
//            Pass 3: the kept mass S' = sum of kept e in fp64, in a fixed
//            order.  A crossing bin of more than 4096 entries (or a cut in
//            the unbinned tail past u = 32) is resolved by the same radix
//            select with each digit's histogram taken by one more pass over
//            the row.
//            With min-p on, one pass instead: the max, the total mass (each
//            thread's fp64 sum relative to a power of two at least its
//            reference max, rescaled exactly as the reference grows; the
//            reference follows the workgroup's running max in LDS), and the
//            entries that can pass min-p against that running max (a superset
//            of those passing against m).  Once m is known their masses are
//            computed in 2^-40 units, top-p is resolved among them by the same
//            radix select (every larger logit passes min-p too), and S' is
//            their integer kept sum.  More than 4096 collected entries: the
//            general passes run.
//  k_accept  one workgroup per (row, chunk of 16 KB of logits).  Every
//            workgroup computes the row's decision itself from the stats and
//            two gathers per position (p'(x_i), q'(x_i) in fp64, the same
//            uniforms as spec_accept), then the draw weights of its chunk
//            at position a_b (residual max(p' - q', 0) after a rejection,
//            p' for the bonus), publishes per-thread fp64 sums and the chunk
//            mass, and counts in; the row's last workgroup draws by inverse
//            CDF in three levels (chunk, thread, entry) and writes the row.
//            Exchange between workgroups uses agent-scope atomic accesses
//            (SC1) and a drain of the workgroup's stores before it counts in.
#include <math.h>

#include <type_traits>

#include "device_common.hpp"
#include "philox.hpp"
#include "spec_verify.h"

namespace specv {
namespace {

typedef uint16_t bf16_t;

constexpr int kT = 256;                     // threads per workgroup
constexpr int kW = kT / kWave;
constexpr int kChunkBytes = 16384;
constexpr int kBins = 512;                  // coarse bins of u, 1/16 wide
constexpr float kBinScale = 16.f;
constexpr int kCand = 4096;                 // entries resolved exactly: the min-p candidates of the
                                            // one-pass reader, or the top-p crossing bin
constexpr int kMaxChunks = 1024;
constexpr int kRowStride = 64;              // ints per row record (256 bytes)
constexpr int kCnt = 0;                     // phase-2 arrivals
constexpr int kInvalid = SPEC_ROW_NONFINITE | SPEC_ROW_BAD_TOKEN | SPEC_ROW_BAD_LEN | SPEC_ROW_ZERO_Q;

template <typename T> constexpr int chunk_of() { return kChunkBytes / (int)sizeof(T); }
template <typename T> constexpr int ept_of() { return chunk_of<T>() / kT; }

__device__ __forceinline__ void co_store(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t co_load(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int co_add(int* p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void co_store32(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void drain_vm() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ uint64_t dbits(double d) { return (uint64_t)__double_as_longlong(d); }
__device__ __forceinline__ double bitsd(uint64_t u) { return __longlong_as_double((long long)u); }

template <typename T>
__device__ __forceinline__ float ld(const T* row, int64_t j) {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(row[j]);
    else return row[j];
}

// order-preserving key of an fp32 value (-0 and +0 share one key)
__device__ __forceinline__ uint32_t fkey(float z) {
    const uint32_t u = __float_as_uint(z == 0.f ? 0.f : z);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// the value of a key (+0 for the shared zero key)
__device__ __forceinline__ float funkey(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// weight of logit z relative to the row max: 2^(fl(z c - fl(m c)))
__device__ __forceinline__ float wexp(float z, float c, float mc) { return hw_exp2(__builtin_fmaf(z, c, -mc)); }

// Stats of one distribution row.
struct Stat {
    float m;        // max logit
    uint32_t tau;   // kept iff fkey(z) >= tau (0: no top-p)
    double s;       // kept mass sum of e
    int flag;       // 1: NaN / +Inf / all -Inf
};

struct Args {
    const void* z;        // target logits [B, K+1, V]
    const void* d;        // draft logits [B, K, V]
    const int32_t* x;     // [B, K]
    const int32_t* lens;  // [B] or null
    int64_t B, V, row_base;
    int K, C;
    float cp, cq;         // log2(e) / T of the target and of the draft
    float top_p, min_p;
    uint64_t seed, offset;
    int32_t* out_tokens;
    int32_t* out_accepted;
    float* out_p_draft;
    int32_t* out_status;
    int* rows;            // [B][kRowStride]
    Stat* stats;          // [B][2K+1]: target 0..K, then draft 0..K-1
    uint64_t* mass;       // [B][C][2]: draw mass, p' mass (for an empty residual)
    uint64_t* tsum;       // [B][C][kT]
};

__device__ __forceinline__ int row_len(const Args& a, int64_t b) { return a.lens ? a.lens[b] : a.K; }

// ---- k_stats ----------------------------------------------------------------------------------
constexpr int kTS = 512;                    // threads of a statistics workgroup
constexpr int kWS = kTS / kWave;
constexpr int kU = 2;                       // 16-byte loads per thread per round
constexpr float kFix40 = 1099511627776.f;   // 2^40: fixed-point unit of the mass histograms

struct StatShared {
    union {
        struct {  // coarse histogram of the top-p pass
            unsigned long long hm[kBins];
            uint32_t hc[kBins];
        };
        struct {  // collected entries: key, mass in 2^-40 units
            uint32_t ck[kCand];
            unsigned long long cq[kCand];
        };
    };
    unsigned long long dig[256];
    unsigned long long red_u[kWS];
    double red_d[kWS];
    float red_f[kWS];
    int red_i[kWS];
    int ncand, bstar;
    uint32_t prefix, mrun;
    double rem;
};

__device__ __forceinline__ void unpack_vec(const uint4& r, float* z, bf16_t) {
    z[0] = bf16_lo(r.x); z[1] = bf16_hi(r.x); z[2] = bf16_lo(r.y); z[3] = bf16_hi(r.y);
    z[4] = bf16_lo(r.z); z[5] = bf16_hi(r.z); z[6] = bf16_lo(r.w); z[7] = bf16_hi(r.w);
}
__device__ __forceinline__ void unpack_vec(const uint4& r, float* z, float) {
    z[0] = __uint_as_float(r.x); z[1] = __uint_as_float(r.y);
    z[2] = __uint_as_float(r.z); z[3] = __uint_as_float(r.w);
}

// Calls f(z, j, valid) for every entry j of a row, in rounds of kU loads per
// thread; a round's loads go out before the previous round is used.  Every thread runs the same rounds and the same
// calls (valid is false past the row): f may use wave-wide operations.
// Loads past the end re-read the last in-range vector instead of branching.
template <typename T, bool VEC, typename F>
__device__ __forceinline__ void row_pass(const T* row, int64_t V, F&& f) {
    const int t = threadIdx.x;
    if constexpr (VEC) {
        constexpr int W = 16 / (int)sizeof(T);
        const int64_t nv = V / W;
        const uint4* p = reinterpret_cast<const uint4*>(row);
        constexpr int64_t kStep = (int64_t)kTS * kU;
        // the next round's loads go out before this round is consumed
        uint4 r[kU], nr[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) r[u] = p[min((int64_t)u * kTS + t, nv - 1)];
        for (int64_t v0 = 0; v0 < nv; v0 += kStep) {
#pragma unroll
            for (int u = 0; u < kU; ++u) nr[u] = p[min(v0 + kStep + (int64_t)u * kTS + t, nv - 1)];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t v = v0 + (int64_t)u * kTS + t;
                float z[W];
                unpack_vec(r[u], z, T{});
#pragma unroll
                for (int k = 0; k < W; ++k) f(z[k], v * W + k, v < nv);
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) r[u] = nr[u];
        }
    } else {
        for (int64_t j0 = 0; j0 < V; j0 += (int64_t)kTS * kU) {
            float z[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) z[u] = ld(row, min(j0 + (int64_t)u * kTS + t, V - 1));
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t j = j0 + (int64_t)u * kTS + t;
                f(z[u], j, j < V);
            }
        }
    }
}

// One round of a thread's entries: kU 16-byte loads, unpacked on each use
// (a bf16 entry is one shift or mask), so the round costs 4 kU registers
// whatever the dtype.
template <typename T>
struct VecRound {
    static constexpr int W = 16 / (int)sizeof(T);
    static constexpr int N = kU * W;
    uint4 r[kU];
    __device__ __forceinline__ float operator[](int e) const {
        const uint4& v = r[e / W];
        const int k = sizeof(T) == 2 ? (e % W) >> 1 : e % W;
        const uint32_t w = k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
        if constexpr (sizeof(T) == 2) return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
        else return __uint_as_float(w);
    }
    // an opaque copy: its entries are unpacked anew where they are used, so
    // values unpacked earlier need not stay live in registers
    __device__ __forceinline__ VecRound fresh() const {
        VecRound c = *this;
#pragma unroll
        for (int u = 0; u < kU; ++u) asm volatile("" : "+v"(c.r[u].x), "+v"(c.r[u].y), "+v"(c.r[u].z), "+v"(c.r[u].w));
        return c;
    }
};
struct ScalarRound {
    static constexpr int N = kU;
    float z[kU];
    __device__ __forceinline__ float operator[](int e) const { return z[e]; }
    __device__ __forceinline__ ScalarRound fresh() const { return *this; }
};

// Calls f(z, ok) once per round with this thread's entries of the round
// (z[e], e < N, N / kU per load) and a bit mask of its loads (bit u for
// entries u N / kU .. (u + 1) N / kU - 1) that lie inside the row.  Every
// thread runs the same rounds.
template <typename T, bool VEC, typename F>
__device__ __forceinline__ void row_rounds(const T* row, int64_t V, F&& f) {
    const int t = threadIdx.x;
    if constexpr (VEC) {
        constexpr int W = VecRound<T>::W;
        const int64_t nv = V / W;
        // buffer loads over the row: the whole byte offset is the per-lane
        // offset (the hardware's range check covers it, not the scalar
        // offset), so reads past the row's end return zeros and never leave
        // the row.  A row holds at most 16 MiB (kMaxChunks chunks), so
        // offsets up to a round past its end fit in 32 bits.
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, (int)(nv * 16), 0x00020000);
        constexpr int64_t kStep = (int64_t)kTS * kU;
        auto ld16 = [&](int64_t v) -> uint4 {
            const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((v + t) * 16), 0, 0);
            return make_uint4(r.x, r.y, r.z, r.w);
        };
        VecRound<T> z, nz;
#pragma unroll
        for (int u = 0; u < kU; ++u) z.r[u] = ld16((int64_t)u * kTS);
        int64_t v0 = 0;
        // whole rounds: every load in the row (a compile-time mask)
        for (; v0 + kStep <= nv; v0 += kStep) {
#pragma unroll
            for (int u = 0; u < kU; ++u) nz.r[u] = ld16(v0 + kStep + (int64_t)u * kTS);
            f(z, std::integral_constant<uint32_t, (1u << kU) - 1u>{});
            z = nz;
        }
        if (v0 < nv) {
            uint32_t ok = 0u;
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (v0 + (int64_t)u * kTS + t < nv) ok |= 1u << u;
            f(z, ok);
        }
    } else {
        for (int64_t j0 = 0; j0 < V; j0 += (int64_t)kTS * kU) {
            ScalarRound z;
            uint32_t ok = 0u;
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                z.z[u] = ld(row, min(j0 + (int64_t)u * kTS + t, V - 1));
                if (j0 + (int64_t)u * kTS + t < V) ok |= 1u << u;
            }
            f(z, ok);
        }
    }
}

// Radix select, descending, over the n collected entries (keys sh.ck, masses
// sh.cq): the key at which the mass, counted from the largest key down and
// taking equal keys together, first reaches rem.  Four 8-bit digits.
// One digit of the radix top-p cut.  dig[] holds the 2^-40 masses of the 256
// digit values at this level; the cut digit is the largest d whose mass at or
// above d reaches rem.  Threads 0..255 hold one digit each; suffix sums in
// waves, then across waves, and a ballot counts the digits that reach rem
// (a prefix of 0..255, as the suffix sums only grow towards digit 0).  The
// thread holding the cut digit writes the extended prefix and rem less the
// mass strictly above the cut; with no such digit (rounding), digit 0 and
// rem less the whole mass.  Every thread of the block calls it; wtot and wcnt
// hold 256 / 64 entries.
__device__ __forceinline__ void pick_digit(const unsigned long long* dig, double rem, uint32_t prefix,
                                           unsigned long long* wtot, int* wcnt, uint32_t* out_prefix,
                                           double* out_rem) {
    constexpr int kDW = 256 / kWave;
    const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
    unsigned long long x = 0ull, v = 0ull;
    if (t < 256) {
        v = dig[t];
        x = v;
        for (int o = 1; o < kWave; o <<= 1) {
            const unsigned long long n = __shfl_down(x, o, kWave);
            if (lane + o < kWave) x += n;
        }
        if (lane == 0) wtot[wv] = x;
    }
    __syncthreads();
    bool f = false;
    if (t < 256) {
        for (int k = wv + 1; k < kDW; ++k) x += wtot[k];
        f = (double)x >= rem;
    }
    const unsigned long long bal = __ballot(f);
    if (t < 256 && lane == 0) wcnt[wv] = __popcll(bal);
    __syncthreads();
    int cnt = 0;
    for (int k = 0; k < kDW; ++k) cnt += wcnt[k];
    const int w = cnt > 0 ? cnt - 1 : 0;
    if (t == w) {
        *out_prefix = (prefix << 8) | (uint32_t)w;
        *out_rem = rem - (double)(cnt > 0 ? x - v : x);
    }
}

__device__ __forceinline__ uint32_t radix_cut(StatShared& sh, int n, double rem) {
    const int t = threadIdx.x;
    uint32_t prefix = 0;
    for (int lvl = 0; lvl < 4; ++lvl) {
        const int shift = 24 - 8 * lvl;
        if (t < 256) sh.dig[t] = 0ull;
        __syncthreads();
        for (int k = t; k < n; k += kTS) {
            const uint32_t key = sh.ck[k];
            if (lvl == 0 || (key >> (shift + 8)) == prefix) atomicAdd(&sh.dig[(key >> shift) & 255u], sh.cq[k]);
        }
        __syncthreads();
        pick_digit(sh.dig, rem, prefix, sh.red_u, sh.red_i, &sh.prefix, &sh.rem);
        __syncthreads();
        prefix = sh.prefix;
        rem = sh.rem;
    }
    return prefix;
}

// Sum over the workgroup of one uint64 per thread (exact, any order).
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, StatShared& sh) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    __syncthreads();
    if (lane == 0) sh.red_u[wv] = v;
    __syncthreads();
    unsigned long long r = 0ull;
    for (int k = 0; k < kWS; ++k) r += sh.red_u[k];
    __syncthreads();
    return r;
}

__device__ __forceinline__ double block_sum_d(double v, StatShared& sh) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    __syncthreads();
    if (lane == 0) sh.red_d[wv] = v;
    __syncthreads();
    double r = 0.0;
    for (int k = 0; k < kWS; ++k) r += sh.red_d[k];
    __syncthreads();
    return r;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kTS) void k_stats(Args a) {
    __shared__ StatShared sh;
    const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
    const int S2 = 2 * a.K + 1;
    const int64_t b = blockIdx.x / S2;
    const int s = (int)(blockIdx.x % S2);
    const int L = row_len(a, b);
    if (L < 0 || L > a.K) return;
    const bool draft = s > a.K;
    const int pos = draft ? s - a.K - 1 : s;
    if (draft ? pos >= L : pos > L) return;
    const int64_t V = a.V;
    const T* row = draft ? static_cast<const T*>(a.d) + (b * a.K + pos) * V
                         : static_cast<const T*>(a.z) + (b * (a.K + 1) + pos) * V;
    const float c = draft ? a.cq : a.cp;
    const float minp = a.min_p;
    Stat st{};

    float mx = -INFINITY;
    int bad = 0;
    double sacc = 0.0;   // min-p pass: this thread's mass relative to 2^(mcref)
    float mcref = 0.f;
    if (minp > 0.f) {
        // One pass: max, non-finite flag, total mass, and the entries that
        // can pass min-p.  Each thread sums its mass relative to 2^kref, kref
        // an integer at least its reference max times c (the reference: its
        // own max so far, raised to the workgroup's running max), so a
        // growing reference rescales the sum exactly by a power of two.  A
        // round is summed against the reference from before it (its entries
        // are unpacked once and used at once); a round whose max lies more
        // than 2^64 above that reference, or that comes before any finite
        // reference, is summed again against the new one.  A NaN entry
        // makes the sum NaN.  An entry can pass min-p against the row max m
        // only if fl(z c - fl(r c)) >= log2(min_p) for any r <= m (fl is
        // monotone); the margin of 1e-4 covers the rounding of the exp2, of
        // log2(min_p) and of the shift to kref.  The collected set is a
        // superset of the entries that pass; their masses are computed once
        // m is known.
        if (t == 0) {
            sh.ncand = 0;
            sh.mrun = fkey(-INFINITY);
        }
        __syncthreads();
        const float lt = log2f(minp) - 1e-4f;
        float ltr = 0.f;  // lt + fl(ref c) - kref
        float gl = -INFINITY;
        row_rounds<T, VEC>(row, V, [&](const auto& z, auto okc) {
            const uint32_t ok = okc;
            constexpr int N = std::remove_reference_t<decltype(z)>::N;
            constexpr int G = N / kU;
            static_assert(N <= 64, "one candidate bit per entry of the round");
            static_assert((kU & (kU - 1)) == 0 && (G & (G - 1)) == 0, "pairwise sums over powers of two");
            // the round's mass against 2^kr (pairwise in fp32 within each
            // load's entries and across the loads, a fixed order) and its max
            auto round_sum = [&](const auto& zz, float kr, float* rmax) {
                float part[kU];
                float rm = -INFINITY;
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    float ev[G];
                    float ru = -INFINITY;
#pragma unroll
                    for (int k = 0; k < G; ++k) {
                        const float v = zz[u * G + k];
                        ru = fmaxf(ru, v);
                        ev[k] = hw_exp2(__builtin_fmaf(v, c, -kr));
                    }
#pragma unroll
                    for (int h = G / 2; h >= 1; h /= 2)
#pragma unroll
                        for (int k = 0; k < h; ++k) ev[k] = ev[k] + ev[k + h];
                    const bool valid = (ok >> u) & 1u;
                    part[u] = valid ? ev[0] : 0.f;
                    rm = valid ? fmaxf(rm, ru) : rm;
                }
#pragma unroll
                for (int h = kU / 2; h >= 1; h /= 2)
#pragma unroll
                    for (int k = 0; k < h; ++k) part[k] = part[k] + part[k + h];
                if (rmax) *rmax = rm;
                return part[0];
            };
            float r;
            const float part = round_sum(z, mcref, &r);
            bad |= r == INFINITY;
            if (r > gl) atomicMax(&sh.mrun, fkey(r));
            const float g = funkey(__hip_atomic_load(&sh.mrun, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
            gl = g;
            const bool redo = !(mx > -INFINITY) || __builtin_fmaf(r, c, -mcref) > 64.f;
            const float nref = fmaxf(fmaxf(mx, r), g);
            if (nref > mx && nref < INFINITY) {
                const float nmc = nref * c;
                const float kr = ceilf(nmc);
                if (!redo) sacc += (double)part;
                sacc = ldexp(sacc, (int)(mcref - kr));
                mx = nref;
                mcref = kr;
                ltr = lt + (nmc - kr);
                if (redo) sacc += (double)round_sum(z.fresh(), mcref, nullptr);
            } else {
                sacc += (double)part;
            }
            // candidates: an entry passes the test only if the round's max
            // does (c > 0), so the per-entry test runs only in waves where
            // some lane's round max passes (about a third of a row's wave
            // rounds on Gaussian logits at min-p 0.05).  Each lane holding
            // candidates takes its slots with one LDS atomic of its own; the
            // order of the collected entries is immaterial (the radix select's
            // mass histograms and the kept sum over them are integer sums)
            const bool hit = mx > -INFINITY && __builtin_fmaf(r, c, -mcref) >= ltr;
            if (__ballot(hit)) {
                const auto zc = z.fresh();
                uint64_t in = 0ull;
                if (hit) {
#pragma unroll
                    for (int e = 0; e < N; ++e)
                        in |= (((ok >> (e / G)) & 1u) && __builtin_fmaf(zc[e], c, -mcref) >= ltr ? 1ull : 0ull) << e;
                }
                const int mine = __popcll(in);
                int slot = 0;
                if (mine) slot = atomicAdd(&sh.ncand, mine);
#pragma unroll
                for (int e = 0; e < N; ++e)
                    if ((in >> e) & 1ull) {
                        if (slot < kCand) sh.ck[slot] = fkey(zc[e]);
                        ++slot;
                    }
            }
        });
    } else {
        // pass 1: max, non-finite flag
        row_pass<T, VEC>(row, V, [&](float z, int64_t, bool ok) {
            if (ok) {
                bad |= (z != z) | (z == INFINITY);
                mx = fmaxf(mx, z);
            }
        });
    }
    const float mthread = mx;
    mx = wave_max(mx);
    bad = wave_or(bad);
    if (lane == 0) {
        sh.red_f[wv] = mx;
        sh.red_i[wv] = bad;
    }
    __syncthreads();
    float m = sh.red_f[0];
    for (int k = 1; k < kWS; ++k) {
        m = fmaxf(m, sh.red_f[k]);
        bad |= sh.red_i[k];
    }
    __syncthreads();
    st.m = m;
    if (bad || m == -INFINITY) {
        if (t == 0) {
            st.flag = 1;
            a.stats[b * S2 + s] = st;
        }
        return;
    }
    const float mc = m * c;

    // min-p on: every entry with a larger logit has a larger e, so top-p is
    // resolved exactly among the collected entries (key, mass in 2^-40
    // units); the kept mass is their integer sum.
    if (minp > 0.f) {
        const double S = block_sum_d(mthread != -INFINITY && sacc != 0.0 ? sacc * exp2((double)mcref - (double)mc) : 0.0, sh);
        if (!(S < INFINITY)) {  // a NaN entry
            if (t == 0) {
                st.flag = 1;
                a.stats[b * S2 + s] = st;
            }
            return;
        }
        const int n = sh.ncand;
        if (n <= kCand) {
            for (int k = t; k < n; k += kTS) {
                const float e = wexp(funkey(sh.ck[k]), c, mc);
                sh.cq[k] = e >= minp ? (unsigned long long)(e * kFix40) : 0ull;
            }
            __syncthreads();
            uint32_t tau = 0;
            if (a.top_p < 1.f) {
                unsigned long long cm = 0ull;
                for (int k = t; k < n; k += kTS) cm += sh.cq[k];
                const unsigned long long C2 = block_sum_u64(cm, sh);
                const double need = (double)a.top_p * S * (double)kFix40;
                if ((double)C2 >= need) tau = radix_cut(sh, n, need);
            }
            unsigned long long kept = 0ull;
            for (int k = t; k < n; k += kTS)
                if (sh.ck[k] >= tau) kept += sh.cq[k];
            const unsigned long long K2 = block_sum_u64(kept, sh);
            if (t == 0) {
                st.tau = tau;
                st.s = (double)K2 / (double)kFix40;
                a.stats[b * S2 + s] = st;
            }
            return;
        }
        // more entries pass min-p than fit: the general passes below
    }

    // pass 2: top-p cut
    uint32_t tau = 0;
    if (a.top_p < 1.f) {
        for (int k = t; k < kBins; k += kTS) {
            sh.hm[k] = 0ull;
            sh.hc[k] = 0u;
        }
        __syncthreads();
        unsigned long long tot = 0ull;
        row_pass<T, VEC>(row, V, [&](float z, int64_t, bool ok) {
            const float w = __builtin_fmaf(z, c, -mc);  // -u
            const unsigned long long q = ok ? (unsigned long long)(hw_exp2(w) * kFix40) : 0ull;
            tot += q;
            const float u = -w;
            if (q && u < 32.f) {
                const int bin = (int)(u * kBinScale);
                atomicAdd(&sh.hm[bin], q);
                atomicAdd(&sh.hc[bin], 1u);
            }
        });
        const unsigned long long S = block_sum_u64(tot, sh);
        if (t == 0) {
            // the crossing bin: the first (from the top) whose cumulative
            // mass reaches need; past the last bin, the unbinned tail
            // (u >= 32), where the rest of the mass lies
            const double need = (double)a.top_p * (double)S;
            unsigned long long acc = 0ull;
            int bs = kBins;
            for (int k = 0; k < kBins; ++k) {
                if ((double)(acc + sh.hm[k]) >= need) {
                    bs = k;
                    break;
                }
                acc += sh.hm[k];
            }
            sh.bstar = bs;
            sh.rem = need - (double)acc;  // > 0: mass still needed inside the bin
            sh.ncand = 0;
        }
        __syncthreads();
        const int bs = sh.bstar;
        const double rem = sh.rem;
        const bool fits = bs < kBins && sh.hc[bs] <= (uint32_t)kCand;
        __syncthreads();  // the entries below overwrite the histogram
        // in the crossing bin: a positive mass and u in the bin (every entry
        // of a higher bin has a strictly larger logit, and equal logits
        // share a bin)
        auto in_bin = [bs](float u, unsigned long long q) {
            return q && (bs < kBins ? (u < 32.f && (int)(u * kBinScale) == bs) : !(u < 32.f));
        };
        if (fits) {
            // collect the crossing bin's entries in LDS, then radix-select there
            row_pass<T, VEC>(row, V, [&](float z, int64_t, bool ok) {
                const float w = __builtin_fmaf(z, c, -mc);
                const unsigned long long q = ok ? (unsigned long long)(hw_exp2(w) * kFix40) : 0ull;
                const bool in = in_bin(-w, q);
                const uint64_t mask = __ballot(in);
                if (mask) {
                    int base = 0;
                    if (lane == 0) base = atomicAdd(&sh.ncand, __popcll(mask));
                    base = __shfl(base, 0, kWave);
                    if (in) {
                        const int slot = base + __popcll(mask & ((1ull << lane) - 1ull));
                        sh.ck[slot] = fkey(z);
                        sh.cq[slot] = q;
                    }
                }
            });
            __syncthreads();
            tau = radix_cut(sh, sh.ncand, rem);
        } else {
            // more entries than LDS holds (or the tail): the same radix
            // select, each 8-bit digit from one more pass over the row.  A
            // thread adds a run of equal digits to the LDS histogram at once.
            uint32_t prefix = 0;
            double r = rem;
            for (int lvl = 0; lvl < 4; ++lvl) {
                const int shift = 24 - 8 * lvl;
                if (t < 256) sh.dig[t] = 0ull;
                __syncthreads();
                uint32_t run_d = 0xFFFFFFFFu;
                unsigned long long run_q = 0ull;
                row_pass<T, VEC>(row, V, [&](float z, int64_t, bool ok) {
                    const float w = __builtin_fmaf(z, c, -mc);
                    const unsigned long long q = ok ? (unsigned long long)(hw_exp2(w) * kFix40) : 0ull;
                    const uint32_t key = fkey(z);
                    if (in_bin(-w, q) && (lvl == 0 || (key >> (shift + 8)) == prefix)) {
                        const uint32_t d = (key >> shift) & 255u;
                        if (d != run_d) {
                            if (run_q) atomicAdd(&sh.dig[run_d], run_q);
                            run_d = d;
                            run_q = 0ull;
                        }
                        run_q += q;
                    }
                });
                if (run_q) atomicAdd(&sh.dig[run_d], run_q);
                __syncthreads();
                pick_digit(sh.dig, r, prefix, sh.red_u, sh.red_i, &sh.prefix, &sh.rem);
                __syncthreads();
                prefix = sh.prefix;
                r = sh.rem;
            }
            tau = prefix;
        }
    }

    // pass 3: kept mass, fp64 per thread, then in thread order
    double sum = 0.0;
    row_pass<T, VEC>(row, V, [&](float z, int64_t, bool ok) {
        const float e = wexp(z, c, mc);
        if (ok && fkey(z) >= tau && e >= minp) sum += (double)e;
    });
    for (int o = kWave / 2; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
    if (lane == 0) sh.red_d[wv] = sum;
    __syncthreads();
    if (t == 0) {
        double S = 0.0;
        for (int k = 0; k < kWS; ++k) S += sh.red_d[k];
        st.tau = tau;
        st.s = S;
        a.stats[b * S2 + s] = st;
    }
}

// ---- k_accept ---------------------------------------------------------------------------------
struct AccShared {
    double red_d[kW];
    int red_x[kW];
    double w[kMaxChunks];
    double scan[kT + 1];
    float px[SPEC_MAX_DRAFT];
    int status, a, cstar, lastpos;
    double tp;
};

// filtered, unnormalised weight of logit z under stats (st, c)
__device__ __forceinline__ float kept_w(float z, float c, const Stat& st, float minp) {
    const float e = wexp(z, c, st.m * c);
    return (fkey(z) >= st.tau && e >= minp) ? e : 0.f;
}

// draw weight of an entry with target logit zp and draft logit zq: the
// residual after a rejection (pmode 0), p' for the bonus (1), p' again (2)
// when the residual is empty
__device__ __forceinline__ float draw_wz(float zp, float zq, int pmode, const Args& a, const Stat& sp,
                                         const Stat& sq, float invp, float invq) {
    const float wp = kept_w(zp, a.cp, sp, a.min_p);
    if (pmode != 0) return wp;
    const float wq = kept_w(zq, a.cq, sq, a.min_p);
    return fmaxf(wp * invp - wq * invq, 0.f);
}
template <typename T>
__device__ __forceinline__ float draw_w(const T* zr, const T* dr, int64_t j, int pmode, const Args& a,
                                        const Stat& sp, const Stat& sq, float invp, float invq) {
    return draw_wz(ld(zr, j), pmode == 0 ? ld(dr, j) : 0.f, pmode, a, sp, sq, invp, invq);
}

__device__ __forceinline__ double block_sum(double v, double* sh) {
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = v;
    __syncthreads();
    double r = 0.0;
    for (int k = 0; k < kW; ++k) r += sh[k];
    __syncthreads();
    return r;
}

// inclusive scan of one double per thread over the workgroup (fixed order)
__device__ __forceinline__ double block_scan(double v, double* sh, double* total) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    for (int o = 1; o < kWave; o <<= 1) {
        const double n = __shfl_up(v, o, kWave);
        if (lane >= o) v += n;
    }
    if (lane == kWave - 1) sh[wv] = v;
    __syncthreads();
    double base = 0.0, tot = 0.0;
    for (int k = 0; k < kW; ++k) {
        if (k < wv) base += sh[k];
        tot += sh[k];
    }
    __syncthreads();
    *total = tot;
    return base + v;
}

// the last index (>= base) whose weight is positive, merged into sh.lastpos
__device__ __forceinline__ void last_positive(bool pos, int base, AccShared& sh) {
    const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
    const uint64_t msk = __ballot(pos);
    if (lane == 0) sh.red_x[wv] = msk ? wv * kWave + 63 - __clzll((long long)msk) : -1;
    __syncthreads();
    if (t == 0) {
        int l = -1;
        for (int k = 0; k < kW; ++k) l = max(l, sh.red_x[k]);
        if (l >= 0) sh.lastpos = max(sh.lastpos, base + l);
    }
    __syncthreads();
}

// The EPT entries [j0, j0 + EPT) of a row, in index order (16-byte loads when
// the rows are aligned); entries past V read as -inf (weight 0).
template <typename T, bool VEC, int EPT>
__device__ __forceinline__ void load_entries(const T* row, int64_t V, int64_t j0, float (&z)[EPT]) {
    if constexpr (VEC) {
        constexpr int W = 16 / (int)sizeof(T);
        const uint4* p = reinterpret_cast<const uint4*>(row + j0);
        uint4 r[EPT / W];
#pragma unroll
        for (int k = 0; k < EPT / W; ++k) r[k] = (j0 + (int64_t)k * W < V) ? p[k] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int k = 0; k < EPT / W; ++k) {
            unpack_vec(r[k], z + k * W, T{});
            if (j0 + (int64_t)k * W >= V)
#pragma unroll
                for (int e = 0; e < W; ++e) z[k * W + e] = -INFINITY;
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) z[e] = (j0 + e < V) ? ld(row, j0 + e) : -INFINITY;
    }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kT) void k_accept(Args a) {
    constexpr int CH = chunk_of<T>(), EPT = ept_of<T>();
    __shared__ AccShared sh;
    const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
    const int64_t b = blockIdx.x / a.C;
    const int ci = (int)(blockIdx.x % a.C);
    const int K = a.K, S2 = 2 * K + 1;
    const int64_t V = a.V;
    const int L = row_len(a, b);
    const bool writer = ci == 0;
    if (L < 0 || L > K) {
        if (writer) {
            for (int i = t; i <= K; i += kT) a.out_tokens[b * (K + 1) + i] = -1;
            if (a.out_p_draft)
                for (int i = t; i < K; i += kT) a.out_p_draft[b * K + i] = -1.f;
            if (t == 0) {
                a.out_accepted[b] = -1;
                if (a.out_status) a.out_status[b] = SPEC_ROW_BAD_LEN;
            }
        }
        return;
    }
    const T* zb = static_cast<const T*>(a.z) + b * (K + 1) * V;
    const T* db = static_cast<const T*>(a.d) + b * K * V;
    const Stat* stb = a.stats + b * S2;
    if (t == 0) {
        sh.status = 0;
        sh.a = L + 1;  // no stop yet
    }
    __syncthreads();
    // The decision, in every workgroup of the row (same inputs, same result),
    // in the listing's order: the row stops at its first rejection, or at
    // the first target position that is not finite (the row is then
    // invalid); target positions after the stop do not count.  The drafted
    // tokens are validated for all L drafts (range, finite draft logits,
    // token in q''s kept set).
    {
        int st = 0;
        bool stop = t <= L && stb[t].flag;  // target position t not finite
        float px = -1.f;
        if (t < L) {
            const int x = a.x[b * K + t];
            if (stb[K + 1 + t].flag) {
                st |= SPEC_ROW_NONFINITE;
            } else if (x < 0 || (int64_t)x >= V) {
                st |= SPEC_ROW_BAD_TOKEN;
            } else {
                const Stat sq = stb[K + 1 + t];
                const float dx = ld(db + (int64_t)t * V, x);
                if (!(kept_w(dx, a.cq, sq, a.min_p) > 0.f)) {
                    st |= SPEC_ROW_ZERO_Q;
                } else if (!stop) {
                    const Stat sp = stb[t];
                    const float zx = ld(zb + (int64_t)t * V, x);
                    const bool kp = kept_w(zx, a.cp, sp, a.min_p) > 0.f;
                    const double p = kp ? exp2((double)zx * (double)a.cp - (double)(sp.m * a.cp)) / sp.s : 0.0;
                    const double q = exp2((double)dx * (double)a.cq - (double)(sq.m * a.cq)) / sq.s;
                    px = (float)p;
                    const double acc = fmin(1.0, p / q);
                    const RowPosUniforms u = row_pos_uniforms(a.seed, a.offset, (uint32_t)(a.row_base + b), (uint32_t)t);
                    stop = !((double)u.acc < acc);
                }
            }
            sh.px[t] = px;
        }
        if (stop) atomicMin(&sh.a, t);
        if (st) atomicOr(&sh.status, st);
    }
    __syncthreads();
    const int ar = min(sh.a, L);
    int status = sh.status | (stb[ar].flag ? SPEC_ROW_NONFINITE : 0);
    const bool invalid = (status & kInvalid) != 0;
    if (writer && a.out_p_draft)
        for (int i = t; i < K; i += kT) a.out_p_draft[b * K + i] = (!invalid && i < L && i <= ar) ? sh.px[i] : -1.f;
    if (invalid) {
        if (writer) {
            for (int i = t; i <= K; i += kT) a.out_tokens[b * (K + 1) + i] = -1;
            if (t == 0) {
                a.out_accepted[b] = -1;
                if (a.out_status) a.out_status[b] = status;
            }
        }
        return;
    }

    // phase 2: this chunk's draw weights at position ar
    const bool reject = ar < L;
    const Stat sp = stb[ar];
    const Stat sq = reject ? stb[K + 1 + ar] : sp;
    const float invp = (float)(1.0 / sp.s), invq = (float)(1.0 / sq.s);
    const T* zr = zb + (int64_t)ar * V;
    const T* dr = db + (int64_t)(reject ? ar : 0) * V;
    const int64_t chunk0 = (int64_t)ci * CH;
    const int64_t j0 = chunk0 + (int64_t)t * EPT;
    double own = 0.0, ownp = 0.0;
    {
        float zz[EPT], dd[EPT];
        load_entries<T, VEC, EPT>(zr, V, j0, zz);
        if (reject) load_entries<T, VEC, EPT>(dr, V, j0, dd);
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            own += (double)draw_wz(zz[e], reject ? dd[e] : 0.f, reject ? 0 : 1, a, sp, sq, invp, invq);
            if (reject) ownp += (double)kept_w(zz[e], a.cp, sp, a.min_p);
        }
    }
    uint64_t* tsrow = a.tsum + b * a.C * kT;
    co_store(tsrow + (int64_t)ci * kT + t, dbits(own));
    const double cm = block_sum(own, sh.red_d);
    const double cmp = reject ? block_sum(ownp, sh.red_d) : 0.0;
    if (t == 0) {
        co_store(a.mass + (b * a.C + ci) * 2, dbits(cm));
        co_store(a.mass + (b * a.C + ci) * 2 + 1, dbits(cmp));
    }
    drain_vm();
    __syncthreads();
    int* rowc = a.rows + b * kRowStride;
    if (t == 0) sh.lastpos = co_add(rowc + kCnt, 1) == a.C - 1;
    __syncthreads();
    if (!sh.lastpos) return;

    // the row's last workgroup draws
    if (t == 0) co_store32(rowc + kCnt, 0);
    const int C = a.C;
    int pmode = reject ? 0 : 1;
    for (int k = t; k < C; k += kT) sh.w[k] = bitsd(co_load(a.mass + (b * C + k) * 2));
    __syncthreads();
    double tot;
    for (;;) {
        double part = 0.0;
        for (int k = t; k < C; k += kT) part += sh.w[k];
        tot = block_sum(part, sh.red_d);
        if (pmode != 0 || tot > 0.0) break;
        pmode = 2;  // empty residual: draw from p'
        status |= SPEC_ROW_RESID_ZERO;
        for (int k = t; k < C; k += kT) sh.w[k] = bitsd(co_load(a.mass + (b * C + k) * 2 + 1));
        __syncthreads();
    }
    const RowPosUniforms u = row_pos_uniforms(a.seed, a.offset, (uint32_t)(a.row_base + b), (uint32_t)ar);
    double tp = (double)u.smp * tot;
    // level 1: the chunk
    if (t == 0) {
        sh.cstar = -1;
        sh.lastpos = -1;
    }
    __syncthreads();
    double carry = 0.0;
    for (int k0 = 0; k0 < C; k0 += kT) {
        const int k = k0 + t;
        const double wk = k < C ? sh.w[k] : 0.0;
        double btot;
        const double incl = carry + block_scan(wk, sh.red_d, &btot);
        sh.scan[t + 1] = incl;
        if (t == 0) sh.scan[0] = carry;
        __syncthreads();
        if (wk > 0.0 && incl > tp && sh.scan[t] <= tp) {
            sh.cstar = k;
            sh.tp = tp - sh.scan[t];
        }
        last_positive(wk > 0.0, k0, sh);
        if (sh.cstar >= 0) break;
        carry += btot;
    }
    int cstar = sh.cstar;
    tp = sh.tp;
    if (cstar < 0) {
        cstar = max(sh.lastpos, 0);
        tp = INFINITY;
    }
    __syncthreads();
    // level 2: the thread of chunk cstar
    const int64_t cb = (int64_t)cstar * CH;
    double ts;
    if (pmode == 2) {
        ts = 0.0;
        float zz[EPT];
        load_entries<T, VEC, EPT>(zr, V, cb + (int64_t)t * EPT, zz);
#pragma unroll
        for (int e = 0; e < EPT; ++e) ts += (double)draw_wz(zz[e], 0.f, 2, a, sp, sq, invp, invq);
    } else {
        ts = bitsd(co_load(tsrow + (int64_t)cstar * kT + t));
    }
    if (t == 0) {
        sh.cstar = -1;
        sh.lastpos = -1;
    }
    __syncthreads();
    double ttot;
    const double incl2 = block_scan(ts, sh.red_d, &ttot);
    sh.scan[t + 1] = incl2;
    if (t == 0) sh.scan[0] = 0.0;
    __syncthreads();
    if (ts > 0.0 && incl2 > tp && sh.scan[t] <= tp) {
        sh.cstar = t;
        sh.tp = tp - sh.scan[t];
    }
    last_positive(ts > 0.0, 0, sh);
    int tstar = sh.cstar;
    tp = sh.tp;
    if (tstar < 0) {
        tstar = max(sh.lastpos, 0);
        tp = INFINITY;
    }
    // level 3: that thread's entries, one per lane of wave 0, in index order
    if (wv == 0) {
        const int64_t jb = cb + (int64_t)tstar * EPT;
        const int64_t j = jb + lane;
        const float wl = (lane < EPT && j < V) ? draw_w(zr, dr, j, pmode, a, sp, sq, invp, invq) : 0.f;
        double incl3 = (double)wl;
        for (int o = 1; o < kWave; o <<= 1) {
            const double n = __shfl_up(incl3, o, kWave);
            if (lane >= o) incl3 += n;
        }
        const uint64_t hit = __ballot(wl > 0.f && incl3 > tp);
        const uint64_t pos = __ballot(wl > 0.f);
        const int sel = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
        if (lane == 0) {
            a.out_tokens[b * (K + 1) + ar] = (int32_t)(jb + sel);
            a.out_accepted[b] = ar;
            if (a.out_status) a.out_status[b] = status;
        }
    }
    for (int i = t; i <= K; i += kT)
        if (i != ar) a.out_tokens[b * (K + 1) + i] = (i < ar) ? a.x[b * K + i] : -1;
}

struct Ws {
    size_t rows_off, stats_off, mass_off, tsum_off, total;
};

Ws ws_layout(int64_t B, int K, int64_t V) {
    const int64_t C = (V + kChunkBytes / 4 - 1) / (kChunkBytes / 4);  // the most chunks of either dtype
    Ws w;
    w.rows_off = 0;
    w.stats_off = align_up((size_t)B * kRowStride * sizeof(int), 256);
    w.mass_off = w.stats_off + align_up((size_t)B * (2 * K + 1) * sizeof(Stat), 256);
    w.tsum_off = w.mass_off + align_up((size_t)B * C * 2 * 8, 256);
    w.total = w.tsum_off + align_up((size_t)B * C * kT * 8, 256);
    return w;
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_accept_sampled_workspace_bytes(int64_t B, int K, int64_t V) {
    if (B < 0 || K < 0 || K > SPEC_MAX_DRAFT || V < 1) return 0;
    return ws_layout(B, K, V).total;
}

extern "C" int spec_accept_sampled(const void* target_logits, const void* draft_logits,
                                   int logits_dtype, const int32_t* draft_tokens,
                                   const int32_t* draft_lens, int64_t B, int K, int64_t V,
                                   int64_t row_base, float temperature, float draft_temperature,
                                   float top_p, float min_p, uint64_t philox_seed,
                                   uint64_t philox_offset, int32_t* out_tokens,
                                   int32_t* out_accepted, float* out_p_draft, int32_t* out_status,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || K < 0 || K > SPEC_MAX_DRAFT || V < 1 || V > 0x7FFFFFFF || row_base < 0)
        return SPEC_ERR_INVALID_ARG;
    if (row_base + B > ((int64_t)1 << 32)) return SPEC_ERR_INVALID_ARG;
    if (logits_dtype != SPEC_F32 && logits_dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
    auto finite_pos = [](float v) { return v > 0.f && v < INFINITY; };
    if (!finite_pos(temperature) || !finite_pos(draft_temperature)) return SPEC_ERR_INVALID_ARG;
    if (!(top_p > 0.f && top_p <= 1.f) || !(min_p >= 0.f && min_p < 1.f)) return SPEC_ERR_INVALID_ARG;
    if (B == 0) return SPEC_OK;
    if (!target_logits || !out_tokens || !out_accepted) return SPEC_ERR_INVALID_ARG;
    if (K > 0 && (!draft_logits || !draft_tokens)) return SPEC_ERR_INVALID_ARG;
    const int64_t CH = logits_dtype == SPEC_BF16 ? chunk_of<bf16_t>() : chunk_of<float>();
    const int64_t C = (V + CH - 1) / CH;
    if (C > kMaxChunks || B * C > ((int64_t)1 << 26) || B * (2 * K + 1) > ((int64_t)1 << 31) - 1)
        return SPEC_ERR_INVALID_ARG;
    const Ws lay = ws_layout(B, K, V);
    if (!workspace || workspace_bytes < lay.total || ((uintptr_t)workspace & 15)) return SPEC_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    Args a{};
    a.z = target_logits;
    a.d = draft_logits;
    a.x = draft_tokens;
    a.lens = draft_lens;
    a.B = B;
    a.V = V;
    a.row_base = row_base;
    a.K = K;
    a.C = (int)C;
    a.cp = (float)(1.4426950408889634074 / (double)temperature);
    a.cq = (float)(1.4426950408889634074 / (double)draft_temperature);
    a.top_p = top_p;
    a.min_p = min_p;
    a.seed = philox_seed;
    a.offset = philox_offset;
    a.out_tokens = out_tokens;
    a.out_accepted = out_accepted;
    a.out_p_draft = out_p_draft;
    a.out_status = out_status;
    a.rows = reinterpret_cast<int*>(ws + lay.rows_off);
    a.stats = reinterpret_cast<Stat*>(ws + lay.stats_off);
    a.mass = reinterpret_cast<uint64_t*>(ws + lay.mass_off);
    a.tsum = reinterpret_cast<uint64_t*>(ws + lay.tsum_off);
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 gs((unsigned)(B * (2 * K + 1))), ga((unsigned)(B * C));
    auto al16 = [](const void* p) { return p == nullptr || ((uintptr_t)p & 15) == 0; };
    const bool rows_aligned = al16(target_logits) && al16(draft_logits);
    if (logits_dtype == SPEC_BF16) {
        if (rows_aligned && V % 8 == 0) {
            hipLaunchKernelGGL((k_stats<bf16_t, true>), gs, dim3(kTS), 0, s, a);
            hipLaunchKernelGGL((k_accept<bf16_t, true>), ga, dim3(kT), 0, s, a);
        } else {
            hipLaunchKernelGGL((k_stats<bf16_t, false>), gs, dim3(kTS), 0, s, a);
            hipLaunchKernelGGL((k_accept<bf16_t, false>), ga, dim3(kT), 0, s, a);
        }
    } else {
        if (rows_aligned && V % 4 == 0) {
            hipLaunchKernelGGL((k_stats<float, true>), gs, dim3(kTS), 0, s, a);
            hipLaunchKernelGGL((k_accept<float, true>), ga, dim3(kT), 0, s, a);
        } else {
            hipLaunchKernelGGL((k_stats<float, false>), gs, dim3(kTS), 0, s, a);
            hipLaunchKernelGGL((k_accept<float, false>), ga, dim3(kT), 0, s, a);
        }
    }
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
