// spec_accept.hip -- batched accept/reject pass of speculative decoding on
// gfx950.
//
// Method: page "Speculative decoding and early exit: accelerated
// autoregressive decoding" (reactapp.top), section "Speculative decoding:
// draft first, then verify", listing `speculative_decode` (accept/reject
// block: temperature softmax of the target logits, acceptance with
// probability min(1, p/q), stop at the first rejection, resample from the
// normalised relu(p - q), bonus token from p when every draft survives);
// page "Decode is memory-bound: ~59 tok/s ceiling on an RTX 4090, and how
// speculative decoding beats it" (trefon.com), section "Speculative
// decoding" (acceptance rule, greedy longest-prefix rule).
//
// The vocabulary is cut into chunks of 4096 entries.  Three launches on the
// caller's stream (two in greedy mode); kernel boundaries order the phases,
// so no workgroup ever waits on, or fences for, another:
//  1. k_stats: single-wave workgroups walk a compact list of (row, position
//     <= L_b, chunk) items (the lengths are prefix-summed in registers), each
//     streaming its 4096 logits from HBM with 16-byte coalesced loads while
//     the next item's loads are already in flight.  Per chunk: max m, then
//     sum_j 2^(fl(z_j c - fl(m c))) with c = log2(e)/T (one FMA and one
//     v_exp_f32 per entry), wave64 butterflies, fp64 across lanes.  Greedy
//     mode keeps (max, lowest index) instead.
//  2. k_decide: one workgroup per (row, chunk).  Each merges the row's chunk
//     partials (fixed order, fp64), runs the acceptance tests (p_i(x_i) in
//     fp64) and finds the first rejection a_b; after a rejection it computes
//     the residual mass sum max(p - q, 0) of its chunk.
//  3. k_sample: one workgroup per row.  Two-level inverse CDF: chunk masses
//     (residual, or p-frame masses from launch 1 for the bonus token) pick
//     the chunk, then one LDS-staged fp64 scan of that chunk picks the token.
// No floating-point atomics: every reduction runs in a fixed order, so the
// output is a deterministic function of the inputs.
#include "spec_verify.h"
#include "device_common.hpp"
#include "philox.hpp"

#include <math.h>

#include <atomic>

namespace specv {
int64_t resident_waves(const void* kernel);
namespace {

constexpr int kChunk = 4096;                 // vocabulary entries per chunk
constexpr int kWEPT = kChunk / kWave;        // entries per lane in k_stats (64)
constexpr int kThreads = 256;                // k_decide / k_sample workgroups
constexpr int kTEPT = kChunk / kThreads;     // entries per thread there (16)
constexpr int kWaves = kThreads / kWave;
constexpr int kRegLens = 4;                  // lengths held in registers by k_stats
constexpr int kCompactMaxB = kWave * kRegLens;
constexpr int kSampleRegs = 4;               // chunk weights held per thread by k_sample
constexpr int kInvalidMask = SPEC_ROW_NONFINITE | SPEC_ROW_BAD_TOKEN | SPEC_ROW_BAD_LEN | SPEC_ROW_ZERO_Q;

struct StatPart {  // stochastic partial of one (row, position, chunk)
    float m;       // chunk max
    int flag;      // 1: NaN or +Inf in the chunk
    double s;      // sum_j 2^(fl(z_j c - fl(m c)))
};
struct ArgPart {  // greedy partial
    float v;
    int flag;
    int idx;
    int pad;
};
struct RowInfo {  // k_decide -> k_sample
    int a;        // first rejection (or L_b)
    int status;   // SPEC_ROW_* bits
    int reject;   // a < L_b
    float M;      // max logit at position a
    double S;     // p-frame normaliser at position a (frame fl(M c))
    double pad;
};
static_assert(sizeof(StatPart) == 16 && sizeof(ArgPart) == 16 && sizeof(RowInfo) == 32, "layout");

typedef uint16_t bf16_t;

// ---- loaders -----------------------------------------------------------------
// Vector width (entries per 16-byte load) of each logits layout.
template <typename T, bool VEC> struct Lay { static constexpr int W = 1; };
template <> struct Lay<bf16_t, true> { static constexpr int W = 8; };
template <> struct Lay<float, true> { static constexpr int W = 4; };

// "Strided" layout over NT threads: vector k of thread t is vector
// (k * NT + t) of the chunk, so consecutive threads read consecutive 16-byte
// vectors.  Register e of thread t holds entry
//   chunk0 + ((e / W) * NT + t) * W + e % W.
template <int W, int NT>
__device__ __forceinline__ int64_t strided_index(int64_t chunk0, int t, int e) {
    return chunk0 + ((int64_t)(e / W) * NT + t) * W + (e % W);
}

__device__ __forceinline__ void unpack8(const uint4 w, float* v) {
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

// One thread's share of a chunk in strided layout, kept as loaded (raw
// 16-byte vectors) so that loads can stay in flight until the values are used.
template <typename T, bool VEC, int NT, int EPT> struct Raw;

template <int NT, int EPT> struct Raw<bf16_t, true, NT, EPT> {
    uint4 r[EPT / 8];
    __device__ __forceinline__ void load(const bf16_t* row, int64_t V, int64_t chunk0, int t) {
        const uint4* p = reinterpret_cast<const uint4*>(row + chunk0) + t;
        if (chunk0 + (int64_t)NT * EPT <= V) {  // whole chunk in range (uniform)
#pragma unroll
            for (int k = 0; k < EPT / 8; ++k) r[k] = p[k * NT];
        } else {
#pragma unroll
            for (int k = 0; k < EPT / 8; ++k)
                r[k] = (chunk0 + ((int64_t)k * NT + t) * 8 < V)
                           ? p[k * NT]
                           : make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
        }
    }
    __device__ __forceinline__ void unpack(float (&v)[EPT]) const {
#pragma unroll
        for (int k = 0; k < EPT / 8; ++k) unpack8(r[k], v + 8 * k);
    }
};

template <int NT, int EPT> struct Raw<float, true, NT, EPT> {
    float4 r[EPT / 4];
    __device__ __forceinline__ void load(const float* row, int64_t V, int64_t chunk0, int t) {
        const float4* p = reinterpret_cast<const float4*>(row + chunk0) + t;
        if (chunk0 + (int64_t)NT * EPT <= V) {  // whole chunk in range (uniform)
#pragma unroll
            for (int k = 0; k < EPT / 4; ++k) r[k] = p[k * NT];
        } else {
#pragma unroll
            for (int k = 0; k < EPT / 4; ++k)
                r[k] = (chunk0 + ((int64_t)k * NT + t) * 4 < V)
                           ? p[k * NT]
                           : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        }
    }
    __device__ __forceinline__ void unpack(float (&v)[EPT]) const {
#pragma unroll
        for (int k = 0; k < EPT / 4; ++k) {
            v[4 * k] = r[k].x; v[4 * k + 1] = r[k].y; v[4 * k + 2] = r[k].z; v[4 * k + 3] = r[k].w;
        }
    }
};

template <typename T, int NT, int EPT> struct Raw<T, false, NT, EPT> {
    float r[EPT];
    __device__ __forceinline__ void load(const T* row, int64_t V, int64_t chunk0, int t) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int64_t j = chunk0 + (int64_t)e * NT + t;
            float x = -INFINITY;
            if (j < V) {
                if constexpr (sizeof(T) == 2) x = bf16_to_f32(row[j]);
                else x = row[j];
            }
            r[e] = x;
        }
    }
    __device__ __forceinline__ void unpack(float (&v)[EPT]) const {
#pragma unroll
        for (int e = 0; e < EPT; ++e) v[e] = r[e];
    }
};

// q entries in the same order as Raw<T, VEC, NT, EPT>; 0 past V.
template <typename T, bool VEC, int NT, int EPT>
__device__ __forceinline__ void load_q_strided(const float* row, int64_t V, int64_t chunk0, int t,
                                               float (&v)[EPT]) {
    constexpr int W = Lay<T, VEC>::W;
    if constexpr (W > 1) {
        const float4* p = reinterpret_cast<const float4*>(row + chunk0) + (int64_t)t * (W / 4);
        const bool full = chunk0 + (int64_t)NT * EPT <= V;  // uniform
#pragma unroll
        for (int k = 0; k < EPT / W; ++k) {
            const bool ok = full || chunk0 + ((int64_t)k * NT + t) * W < V;
#pragma unroll
            for (int h = 0; h < W / 4; ++h) {
                const float4 f = ok ? p[(int64_t)k * NT * (W / 4) + h] : make_float4(0.f, 0.f, 0.f, 0.f);
                v[k * W + 4 * h] = f.x; v[k * W + 4 * h + 1] = f.y;
                v[k * W + 4 * h + 2] = f.z; v[k * W + 4 * h + 3] = f.w;
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int64_t j = chunk0 + (int64_t)e * NT + t;
            v[e] = (j < V) ? row[j] : 0.f;
        }
    }
}

// "Contiguous" layout for the in-chunk scan: the thread owns entries
// [start, start + EPT) in order.
template <typename T, bool VEC, int EPT>
__device__ __forceinline__ void load_contig(const T* row, int64_t V, int64_t start, float (&v)[EPT]) {
    if constexpr (VEC && sizeof(T) == 2) {
        const uint4* p = reinterpret_cast<const uint4*>(row + start);
#pragma unroll
        for (int k = 0; k < EPT / 8; ++k) {
            const uint4 w = (start + 8 * k < V) ? p[k] : make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
            unpack8(w, v + 8 * k);
        }
    } else if constexpr (VEC) {
        const float4* p = reinterpret_cast<const float4*>(row + start);
#pragma unroll
        for (int k = 0; k < EPT / 4; ++k) {
            const float4 f = (start + 4 * k < V) ? p[k] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            v[4 * k] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int64_t j = start + e;
            float x = -INFINITY;
            if (j < V) {
                if constexpr (sizeof(T) == 2) x = bf16_to_f32(row[j]);
                else x = row[j];
            }
            v[e] = x;
        }
    }
}

template <bool VEC, int EPT>
__device__ __forceinline__ void load_q_contig(const float* row, int64_t V, int64_t start, float (&v)[EPT]) {
    if constexpr (VEC) {
        const float4* p = reinterpret_cast<const float4*>(row + start);
#pragma unroll
        for (int k = 0; k < EPT / 4; ++k) {
            const float4 f = (start + 4 * k < V) ? p[k] : make_float4(0.f, 0.f, 0.f, 0.f);
            v[4 * k] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) v[e] = (start + e < V) ? row[start + e] : 0.f;
    }
}

template <typename T>
__device__ __forceinline__ float load_one(const T* row, int64_t j) {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(row[j]);
    else return row[j];
}

// ---- per-entry weights (identical expressions wherever used) -----------------
// p-frame weight of logit z at a position with fl(M c) = mc.
__device__ __forceinline__ float p_weight(float z, float c, float mc) {
    return hw_exp2(__builtin_fmaf(z, c, -mc));
}
// residual weight max(p - q, 0) with p = weight / S, invS = fl(1/S).
__device__ __forceinline__ float r_weight(float z, float q, float c, float mc, float invS) {
    const float p = p_weight(z, c, mc) * invS;
    return fmaxf(p - q, 0.f);
}

// p-frame mass of one chunk partial relative to the position's fl(M c).
__device__ __forceinline__ double chunk_p_mass(const StatPart& e, float c, float mcM) {
    if (e.m == -INFINITY) return 0.0;
    const float mck = e.m * c;
    return e.s * exp2((double)mck - (double)mcM);
}

// ---- workgroup reductions -------------------------------------------------------
__device__ __forceinline__ double block_sum(double v, double* sh) {
    v = wave_sum(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) sh[w] = v;
    __syncthreads();
    double r = sh[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r += sh[k];
    __syncthreads();
    return r;
}

// Inclusive scan of one double per thread across the workgroup (wave64
// shuffle scan, then the wave totals in order); also returns the total.
__device__ __forceinline__ double block_incl_scan(double v, double* sh, double* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double n = __shfl_up(v, o, kWave);
        if (lane >= o) v += n;
    }
    if (lane == kWave - 1) sh[wv] = v;
    __syncthreads();
    double base = 0.0, tot = 0.0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
        if (k < wv) base += sh[k];
        tot += sh[k];
    }
    __syncthreads();
    *total = tot;
    return base + v;
}

__device__ __forceinline__ int wave_incl_scan_int(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int n = __shfl_up(v, o, kWave);
        if (lane >= o) v += n;
    }
    return v;
}

// Merge of the C chunk partials of one position by one wave (lanes over
// chunks, butterfly reductions: a fixed order).  Every kernel that needs a
// position's (M, S) calls this, so they all see the same bits.
struct PosStats {
    float M;
    double S;
    int flag;
};
__device__ __forceinline__ PosStats merge_position(const StatPart* pp, int C, float c) {
    const int lane = threadIdx.x & (kWave - 1);
    float M = -INFINITY;
    int flag = 0;
    for (int k = lane; k < C; k += kWave) {
        M = fmaxf(M, pp[k].m);
        flag |= pp[k].flag;
    }
    M = wave_max(M);
    flag = wave_or(flag);
    if (M == -INFINITY || M == INFINITY) flag = 1;
    const float mcM = M * c;
    double S = 0.0;
    if (!flag)
        for (int k = lane; k < C; k += kWave) S += chunk_p_mass(pp[k], c, mcM);
    S = wave_sum(S);
    return PosStats{M, S, flag};
}

// ---- launch 1: chunk statistics ----------------------------------------------------
// Work list of (row-position rp = b (K+1) + i, chunk).  For B <= 256 the
// list is compact: lane l holds n_b = L_b + 1 (0 for a bad length) for
// b = l + 64 j, prefix-summed across the wave, and item w maps to
// position pos = w / C of the concatenated valid positions.  Larger batches
// walk all B (K+1) positions and skip those past L_b.
struct WorkList {
    int pst[kRegLens];  // exclusive prefix of n_b, b = lane + 64 j
    int64_t B;
    int K, C;
    bool compact;
    const int32_t* lens;
    int64_t nitems;

    __device__ __forceinline__ void init(const int32_t* lens_, int64_t B_, int K_, int C_) {
        lens = lens_;
        B = B_;
        K = K_;
        C = C_;
        compact = B <= kCompactMaxB;
        if (compact) {
            const int lane = threadIdx.x & (kWave - 1);
            int carry = 0;
#pragma unroll
            for (int j = 0; j < kRegLens; ++j) {
                const int64_t b = lane + kWave * j;
                int n = 0;
                if (b < B) {
                    const int L = lens ? lens[b] : K;
                    n = (L >= 0 && L <= K) ? L + 1 : 0;
                }
                const int incl = wave_incl_scan_int(n);
                pst[j] = carry + incl - n;
                carry += __shfl(incl, kWave - 1, kWave);
            }
            nitems = (int64_t)carry * C;
        } else {
            nitems = B * (K + 1) * C;
        }
    }
    // item w -> (rp, chunk); false if the item is past L_b (non-compact only)
    __device__ __forceinline__ bool locate(int64_t w, int64_t& rp, int& ci) const {
        const int64_t pos = w / C;
        ci = (int)(w % C);
        if (compact) {
            const int lane = threadIdx.x & (kWave - 1);
            int cnt = 0;
#pragma unroll
            for (int j = 0; j < kRegLens; ++j)
                cnt += __popcll(__ballot((lane + kWave * j < B) && (int64_t)pst[j] <= pos));
            const int b = cnt - 1;
            const int j = b / kWave;
            static_assert(kRegLens == 4, "select chain below");
            const int sel = (j == 0) ? pst[0] : (j == 1) ? pst[1] : (j == 2) ? pst[2] : pst[3];
            const int base = __shfl(sel, b % kWave, kWave);
            rp = (int64_t)b * (K + 1) + (pos - base);
            return true;
        }
        rp = pos;
        const int64_t b = rp / (K + 1);
        const int i = (int)(rp % (K + 1));
        const int L = lens ? lens[b] : K;
        return L >= 0 && L <= K && i <= L;
    }
    // first valid item at or after w in steps of `stride`
    __device__ __forceinline__ bool next(int64_t& w, int64_t stride, int64_t& rp, int& ci) const {
        while (w < nitems) {
            if (locate(w, rp, ci)) return true;
            w += stride;
        }
        return false;
    }
};

template <typename T, bool VEC, bool GREEDY>
__global__ __launch_bounds__(kWave) void k_stats(const T* __restrict__ logits,
                                                 const int32_t* __restrict__ lens, int64_t B, int K,
                                                 int64_t V, int C, float c, void* __restrict__ part_out) {
    constexpr int W = Lay<T, VEC>::W;
    const int lane = threadIdx.x;
    WorkList wl;
    wl.init(lens, B, K, C);
    const int64_t stride = gridDim.x;
    auto process = [&](const Raw<T, VEC, kWave, kWEPT>& raw, int64_t rp, int ci) {
        float v[kWEPT];
        raw.unpack(v);
        const int64_t pidx = rp * C + ci;
        if constexpr (GREEDY) {
            const int64_t chunk0 = (int64_t)ci * kChunk;
            float best = -INFINITY;
            int bidx = 0x7FFFFFFF, nan = 0;
#pragma unroll
            for (int e = 0; e < kWEPT; ++e) {
                const int64_t j = strided_index<W, kWave>(chunk0, lane, e);
                const float x = v[e];
                if (j < V) {
                    nan |= (x != x);
                    if (x > best || (x == best && (int)j < bidx)) { best = x; bidx = (int)j; }
                }
            }
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) {
                const float ov = __shfl_xor(best, o, kWave);
                const int oi = __shfl_xor(bidx, o, kWave);
                if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
            }
            nan = wave_or(nan);
            if (lane == 0)
                static_cast<ArgPart*>(part_out)[pidx] = ArgPart{best, (nan || best == INFINITY) ? 1 : 0, bidx, 0};
        } else {
            float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
            for (int e = 0; e < kWEPT; e += 2) {
                m0 = fmaxf(m0, v[e]);
                m1 = fmaxf(m1, v[e + 1]);
            }
            const float m = wave_max(fmaxf(m0, m1));
            int flag = 0;
            double s = 0.0;
            if (m == INFINITY) {
                flag = 1;
            } else if (m == -INFINITY) {
                int nan = 0;
#pragma unroll
                for (int e = 0; e < kWEPT; ++e) nan |= (v[e] != v[e]);
                flag = wave_or(nan);
            } else {
                const float mc = m * c;
                float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
                for (int e = 0; e < kWEPT; e += 4) {
                    a0 += p_weight(v[e], c, mc);
                    a1 += p_weight(v[e + 1], c, mc);
                    a2 += p_weight(v[e + 2], c, mc);
                    a3 += p_weight(v[e + 3], c, mc);
                }
                s = wave_sum((double)((a0 + a1) + (a2 + a3)));
                flag = (s != s) ? 1 : 0;
            }
            if (lane == 0) static_cast<StatPart*>(part_out)[pidx] = StatPart{m, flag, s};
        }
    };
    // two register buffers in ping-pong: the next item's loads are issued
    // before the current item is reduced
    Raw<T, VEC, kWave, kWEPT> bufA, bufB;
    int64_t w = blockIdx.x, rpA = 0, rpB = 0;
    int ciA = 0, ciB = 0;
    bool haveA = wl.next(w, stride, rpA, ciA);
    if (haveA) bufA.load(logits + rpA * V, V, (int64_t)ciA * kChunk, lane);
    while (haveA) {
        int64_t w2 = w + stride;
        const bool haveB = wl.next(w2, stride, rpB, ciB);
        if (haveB) bufB.load(logits + rpB * V, V, (int64_t)ciB * kChunk, lane);
        process(bufA, rpA, ciA);
        if (!haveB) break;
        w = w2 + stride;
        haveA = wl.next(w, stride, rpA, ciA);
        if (haveA) bufA.load(logits + rpA * V, V, (int64_t)ciA * kChunk, lane);
        process(bufB, rpB, ciB);
    }
}

// ---- launch 2: decisions and residual chunk masses ----------------------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_decide(
    const T* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ lens, int K, int64_t V, int C, float c, int64_t row_base,
    uint64_t seed, uint64_t offset, const StatPart* __restrict__ part, double* __restrict__ resid,
    RowInfo* __restrict__ info, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_accepted, float* __restrict__ out_p_draft,
    int32_t* __restrict__ out_status) {
    constexpr int kPos = SPEC_MAX_DRAFT + 1;
    __shared__ float s_M[kPos];
    __shared__ double s_S[kPos];
    __shared__ int s_flag[kPos];
    __shared__ float s_zx[kPos];
    __shared__ float s_qx[kPos];
    __shared__ float s_px[kPos];
    __shared__ double sh_d[kWaves];
    __shared__ int s_status, s_a;

    const int64_t b = blockIdx.x / C;
    const int ci = (int)(blockIdx.x % C);
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wv = t / kWave;
    const int x = (t < K) ? tokens[b * K + t] : 0;  // issued with the length load
    const int L = lens ? lens[b] : K;
    const bool len_ok = (L >= 0 && L <= K);
    if (t == 0) {
        s_status = len_ok ? 0 : SPEC_ROW_BAD_LEN;
        s_a = len_ok ? L : 0;
    }
    __syncthreads();

    // gather z_i(x_i) and q_i(x_i) of every drafted position (one thread each)
    if (len_ok && t < L) {
        int st = 0;
        float zx = 0.f, qx = 1.f;
        if (x < 0 || (int64_t)x >= V) {
            st = SPEC_ROW_BAD_TOKEN;
        } else {
            zx = load_one(logits + (b * (K + 1) + t) * V, x);
            qx = q[(b * K + t) * V + x];
            if (!(qx > 0.f)) st = SPEC_ROW_ZERO_Q;
        }
        s_zx[t] = zx;
        s_qx[t] = qx;
        if (st) atomicOr(&s_status, st);
    }
    // merge the chunk partials of each position <= L_b, one wave per position
    if (len_ok) {
        for (int i = wv; i <= L; i += kWaves) {
            const PosStats ps = merge_position(part + (b * (K + 1) + i) * C, C, c);
            if (lane == 0) {
                s_M[i] = ps.M;
                s_S[i] = ps.S;
                s_flag[i] = ps.flag;
                if (ps.flag) atomicOr(&s_status, SPEC_ROW_NONFINITE);
            }
        }
    }
    __syncthreads();
    // acceptance tests, then the first rejection
    if (len_ok && t < L) {
        float px = -1.f;
        int rej = 0;
        const float qx = s_qx[t];
        if (!s_flag[t] && qx > 0.f) {
            const float mcM = s_M[t] * c;
            const double p = exp2((double)s_zx[t] * (double)c - (double)mcM) / s_S[t];
            px = (float)p;
            const double a = fmin(1.0, p / (double)qx);
            const RowPosUniforms u = row_pos_uniforms(seed, offset, (uint32_t)(row_base + b), (uint32_t)t);
            rej = ((double)u.acc < a) ? 0 : 1;
        }
        s_px[t] = px;
        if (rej) atomicMin(&s_a, t);
    }
    __syncthreads();
    const int status = s_status;
    const int a = s_a;
    const bool invalid = (status & kInvalidMask) != 0;
    const bool reject = !invalid && a < L;
    if (ci == 0) {
        if (out_p_draft)
            for (int i = t; i < K; i += kThreads)
                out_p_draft[b * K + i] = (!invalid && i < L) ? s_px[i] : -1.f;
        if (invalid) {
            for (int i = t; i <= K; i += kThreads) out_tokens[b * (K + 1) + i] = -1;
            if (t == 0) {
                out_accepted[b] = -1;
                if (out_status) out_status[b] = status;
            }
        }
        if (t == 0) info[b] = RowInfo{a, status, reject ? 1 : 0, invalid ? 0.f : s_M[a], invalid ? 0.0 : s_S[a], 0.0};
    }
    if (invalid) return;
    const float mcM = s_M[a] * c;
    if (!reject) {
        // the bonus draw uses the p-frame mass of each chunk at position a
        if (t == 0) resid[b * C + ci] = chunk_p_mass(part[(b * (K + 1) + a) * C + ci], c, mcM);
        return;
    }

    // residual mass of this chunk at the rejected position
    const float invS = (float)(1.0 / s_S[a]);
    const T* zrow = logits + (b * (K + 1) + a) * V;
    const float* qrow = q + (b * K + a) * V;
    const int64_t chunk0 = (int64_t)ci * kChunk;
    Raw<T, VEC, kThreads, kTEPT> raw;
    raw.load(zrow, V, chunk0, t);
    float qq[kTEPT], z[kTEPT];
    load_q_strided<T, VEC, kThreads, kTEPT>(qrow, V, chunk0, t, qq);
    raw.unpack(z);
    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
#pragma unroll
    for (int e = 0; e < kTEPT; e += 4) {
        r0 += r_weight(z[e], qq[e], c, mcM, invS);
        r1 += r_weight(z[e + 1], qq[e + 1], c, mcM, invS);
        r2 += r_weight(z[e + 2], qq[e + 2], c, mcM, invS);
        r3 += r_weight(z[e + 3], qq[e + 3], c, mcM, invS);
    }
    const double R = block_sum((double)((r0 + r1) + (r2 + r3)), sh_d);
    if (t == 0) resid[b * C + ci] = R;
}

// ---- launch 3: the categorical draw ------------------------------------------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_sample(
    const T* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ tokens,
    int K, int64_t V, int C, float c, int64_t row_base, uint64_t seed, uint64_t offset,
    const StatPart* __restrict__ part, const double* __restrict__ resid,
    const RowInfo* __restrict__ info, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_accepted, int32_t* __restrict__ out_status) {
    __shared__ double sh_d[kWaves];
    __shared__ double s_scan[kThreads + 1];
    __shared__ double s_tp;
    __shared__ int s_cstar, s_tok, s_lastpos;

    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    // the row's chunk weights and its decision record load together
    double wreg[kSampleRegs];
#pragma unroll
    for (int j = 0; j < kSampleRegs; ++j) {
        const int k = j * kThreads + t;
        wreg[j] = (k < C) ? resid[b * C + k] : 0.0;
    }
    const RowInfo ri = info[b];
    if (ri.status & kInvalidMask) return;  // k_decide wrote this row
    const int a = ri.a;
    int status = ri.status;
    const StatPart* pp = part + (b * (K + 1) + a) * C;
    if (t == 0) {
        s_cstar = 0x7FFFFFFF;
        s_tok = 0x7FFFFFFF;
        s_lastpos = -1;
    }
    const float mcM = ri.M * c;
    const float invS = (float)(1.0 / ri.S);
    const T* zrow = logits + (b * (K + 1) + a) * V;
    const float* qrow = ri.reject ? q + (b * K + a) * V : nullptr;

    // first level: pick the chunk from the chunk masses (residual masses
    // after a rejection, p-frame masses for the bonus token)
    int pmode = ri.reject ? 0 : 1;
    auto chunk_w = [&](int k) -> double {
        if (k >= C) return 0.0;
        const int j = k / kThreads;
        if (pmode == 2 || j >= kSampleRegs) return (pmode == 2) ? chunk_p_mass(pp[k], c, mcM) : resid[b * C + k];
        double r = wreg[0];
#pragma unroll
        for (int jj = 1; jj < kSampleRegs; ++jj) r = (j == jj) ? wreg[jj] : r;
        return r;
    };
    double tot = 0.0;
    for (int k0 = 0; k0 < C; k0 += kThreads) tot += block_sum(chunk_w(k0 + t), sh_d);
    if (!pmode && !(tot > 0.0)) {  // residual is empty: draw from p
        pmode = 2;
        status |= SPEC_ROW_RESID_ZERO;
        tot = 0.0;
        for (int k0 = 0; k0 < C; k0 += kThreads) tot += block_sum(chunk_w(k0 + t), sh_d);
    }
    const RowPosUniforms u = row_pos_uniforms(seed, offset, (uint32_t)(row_base + b), (uint32_t)a);
    const double tt = (double)u.smp * tot;
    double carry = 0.0;
    for (int k0 = 0; k0 < C; k0 += kThreads) {
        const int k = k0 + t;
        const double wk = chunk_w(k);
        double btot;
        const double incl = carry + block_incl_scan(wk, sh_d, &btot);
        s_scan[t + 1] = incl;
        if (t == 0) s_scan[0] = carry;
        __syncthreads();
        if (k < C && wk > 0.0) {
            atomicMax(&s_lastpos, k);
            if (incl > tt && s_scan[t] <= tt) {
                s_cstar = k;  // unique: the scan is non-decreasing
                s_tp = tt - s_scan[t];
            }
        }
        __syncthreads();
        if (s_cstar != 0x7FFFFFFF) break;
        carry += btot;
    }
    int cstar = s_cstar;
    double tp = s_tp;
    if (cstar == 0x7FFFFFFF) {  // rounding left t at or past the total: last positive entry
        cstar = s_lastpos;
        tp = INFINITY;
    }
    __syncthreads();
    if (t == 0) s_lastpos = -1;

    // second level: scan the chosen chunk in index order
    const int64_t start = (int64_t)cstar * kChunk + (int64_t)t * kTEPT;
    float w[kTEPT];
    {
        float z[kTEPT];
        load_contig<T, VEC, kTEPT>(zrow, V, start, z);
        if (pmode) {
#pragma unroll
            for (int e = 0; e < kTEPT; ++e) w[e] = p_weight(z[e], c, mcM);
        } else {
            float qq[kTEPT];
            load_q_contig<VEC, kTEPT>(qrow, V, start, qq);
#pragma unroll
            for (int e = 0; e < kTEPT; ++e) w[e] = r_weight(z[e], qq[e], c, mcM, invS);
        }
    }
    double own = 0.0;
    int lastpos = -1;
#pragma unroll
    for (int e = 0; e < kTEPT; ++e) {
        own += (double)w[e];
        if (w[e] > 0.f) lastpos = e;
    }
    double ctot;
    const double incl = block_incl_scan(own, sh_d, &ctot);
    s_scan[t + 1] = incl;
    if (t == 0) s_scan[0] = 0.0;
    __syncthreads();
    const double lo = s_scan[t], hi = s_scan[t + 1];
    if (lo <= tp && tp < hi) {
        double cum = lo;
        int found = -1;
#pragma unroll
        for (int e = 0; e < kTEPT; ++e) {
            cum += (double)w[e];
            if (found < 0 && w[e] > 0.f && cum > tp) found = e;
        }
        if (found < 0) found = lastpos;
        if (found >= 0) atomicMin(&s_tok, (int)(start + found));
    }
    if (lastpos >= 0) atomicMax(&s_lastpos, (int)(start + lastpos));
    __syncthreads();
    if (t == 0) {
        int tok = s_tok;
        if (tok == 0x7FFFFFFF) tok = s_lastpos;  // t' at or past the chunk total
        out_tokens[b * (K + 1) + a] = tok;
        out_accepted[b] = a;
        if (out_status) out_status[b] = status;
    }
    for (int i = t; i <= K; i += kThreads)
        if (i != a) out_tokens[b * (K + 1) + i] = (i < a) ? tokens[b * K + i] : -1;
}

// ---- greedy finish: one wave per row ---------------------------------------------------
__global__ __launch_bounds__(kWave) void k_greedy_finish(
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ lens, int K, int64_t V, int C,
    const ArgPart* __restrict__ part, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_accepted, float* __restrict__ out_p_draft,
    int32_t* __restrict__ out_status) {
    __shared__ int s_g[SPEC_MAX_DRAFT + 1];
    __shared__ int s_status, s_a;
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    const int L = lens ? lens[b] : K;
    const bool len_ok = (L >= 0 && L <= K);
    if (t == 0) {
        s_status = len_ok ? 0 : SPEC_ROW_BAD_LEN;
        s_a = len_ok ? L : 0;
    }
    __syncthreads();
    if (len_ok) {
        // per position: lanes over chunks, butterfly (max value, lowest index)
        for (int i = 0; i <= L; ++i) {
            const ArgPart* pp = part + ((b * (K + 1) + i) * C);
            float bv = -INFINITY;
            int bi = 0x7FFFFFFF, flag = 0;
            for (int k = t; k < C; k += kWave) {
                const ArgPart e = pp[k];
                flag |= e.flag;
                if (e.v > bv || (e.v == bv && e.idx < bi)) { bv = e.v; bi = e.idx; }
            }
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) {
                const float ov = __shfl_xor(bv, o, kWave);
                const int oi = __shfl_xor(bi, o, kWave);
                if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
            }
            flag = wave_or(flag);
            if (t == 0) {
                s_g[i] = bi;
                if (flag || bv == -INFINITY || bv == INFINITY) s_status |= SPEC_ROW_NONFINITE;
            }
        }
        for (int i = t; i < L; i += kWave) {
            const int x = tokens[b * K + i];
            if (x < 0 || (int64_t)x >= V) atomicOr(&s_status, SPEC_ROW_BAD_TOKEN);
        }
    }
    __syncthreads();
    if (len_ok)
        for (int i = t; i < L; i += kWave)
            if (tokens[b * K + i] != s_g[i]) atomicMin(&s_a, i);
    __syncthreads();
    const int status = s_status;
    const bool invalid = (status & kInvalidMask) != 0;
    const int a = s_a;
    if (out_p_draft)
        for (int i = t; i < K; i += kWave)
            out_p_draft[b * K + i] = (!invalid && i < L) ? (tokens[b * K + i] == s_g[i] ? 1.f : 0.f) : -1.f;
    for (int i = t; i <= K; i += kWave) {
        int v = -1;
        if (!invalid) {
            if (i < a) v = tokens[b * K + i];
            else if (i == a) v = s_g[a];
        }
        out_tokens[b * (K + 1) + i] = v;
    }
    if (t == 0) {
        out_accepted[b] = invalid ? -1 : a;
        if (out_status) out_status[b] = status;
    }
}

// ---- host side ------------------------------------------------------------------------------
struct AcceptWs {
    size_t part_off, resid_off, info_off, total;
};

AcceptWs accept_ws_layout(int64_t B, int K, int64_t V) {
    const int64_t C = (V + kChunk - 1) / kChunk;
    AcceptWs w;
    w.part_off = 0;
    w.resid_off = align_up((size_t)B * (K + 1) * C * sizeof(StatPart), 256);
    w.info_off = w.resid_off + align_up((size_t)B * C * sizeof(double), 256);
    w.total = w.info_off + align_up((size_t)B * sizeof(RowInfo), 256);
    return w;
}

template <typename T, bool VEC>
int launch_accept(const T* logits, const float* q, const int32_t* tokens, const int32_t* lens,
                  int64_t B, int K, int64_t V, int64_t row_base, float temperature, uint64_t seed,
                  uint64_t offset, int32_t* out_tokens, int32_t* out_accepted, float* out_p_draft,
                  int32_t* out_status, char* ws, const AcceptWs& lay, hipStream_t stream) {
    const int C = (int)((V + kChunk - 1) / kChunk);
    const int64_t items = B * (K + 1) * C;
    // k_stats is persistent: one generation of single-wave workgroups that
    // fills the device, each walking several items
    const int64_t cap = temperature == 0.f ? resident_waves((const void*)k_stats<T, VEC, true>)
                                           : resident_waves((const void*)k_stats<T, VEC, false>);
    if (cap <= 0) return SPEC_ERR_HIP;
    const unsigned g1 = (unsigned)(items < cap ? items : cap);
    void* part = ws + lay.part_off;
    if (temperature == 0.f) {
        hipLaunchKernelGGL((k_stats<T, VEC, true>), dim3(g1), dim3(kWave), 0, stream, logits, lens,
                           B, K, V, C, 0.f, part);
        if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
        hipLaunchKernelGGL(k_greedy_finish, dim3((unsigned)B), dim3(kWave), 0, stream, tokens, lens,
                           K, V, C, static_cast<const ArgPart*>(part), out_tokens, out_accepted,
                           out_p_draft, out_status);
        if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
        return SPEC_OK;
    }
    // c = log2(e) / T, rounded once to fp32
    const float c = (float)(1.4426950408889634074 / (double)temperature);
    const StatPart* sp = static_cast<const StatPart*>(part);
    double* resid = reinterpret_cast<double*>(ws + lay.resid_off);
    RowInfo* info = reinterpret_cast<RowInfo*>(ws + lay.info_off);
    hipLaunchKernelGGL((k_stats<T, VEC, false>), dim3(g1), dim3(kWave), 0, stream, logits, lens,
                       B, K, V, C, c, part);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    hipLaunchKernelGGL((k_decide<T, VEC>), dim3((unsigned)(B * C)), dim3(kThreads), 0, stream,
                       logits, q, tokens, lens, K, V, C, c, row_base, seed, offset, sp, resid, info,
                       out_tokens, out_accepted, out_p_draft, out_status);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    hipLaunchKernelGGL((k_sample<T, VEC>), dim3((unsigned)B), dim3(kThreads), 0, stream, logits, q,
                       tokens, K, V, C, c, row_base, seed, offset, sp, resid, info, out_tokens,
                       out_accepted, out_status);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    return SPEC_OK;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

// Number of single-wave workgroups of `kernel` the current device holds at
// once (compute units x resident workgroups per unit); a read-only property
// of the device and the code object, cached per (kernel, device).
int64_t resident_waves(const void* kernel) {
    constexpr int kMaxDev = 64, kMaxKernels = 16;
    static std::atomic<int64_t> cache[kMaxKernels][kMaxDev];
    static std::atomic<const void*> keys[kMaxKernels];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    int slot = -1;
    for (int i = 0; i < kMaxKernels; ++i) {
        const void* k = keys[i].load();
        if (k == kernel) { slot = i; break; }
        if (k == nullptr) {
            const void* expect = nullptr;
            if (keys[i].compare_exchange_strong(expect, kernel) || expect == kernel) { slot = i; break; }
        }
    }
    if (slot >= 0 && dev < kMaxDev) {
        const int64_t v = cache[slot][dev].load();
        if (v > 0) return v;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kWave, 0) != hipSuccess) return -1;
    const int64_t v = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    if (slot >= 0 && dev < kMaxDev) cache[slot][dev].store(v);
    return v;
}
}  // namespace specv

using namespace specv;

extern "C" size_t spec_accept_workspace_bytes(int64_t B, int K, int64_t V) {
    if (B < 0 || K < 0 || K > SPEC_MAX_DRAFT || V < 1) return 0;
    return accept_ws_layout(B, K, V).total;
}

extern "C" int spec_accept(const void* target_logits, int logits_dtype, const float* draft_probs,
                           const int32_t* draft_tokens, const int32_t* draft_lens, int64_t B,
                           int K, int64_t V, int64_t row_base, float temperature,
                           uint64_t philox_seed, uint64_t philox_offset, int32_t* out_tokens,
                           int32_t* out_accepted, float* out_p_draft, int32_t* out_status,
                           void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || K < 0 || K > SPEC_MAX_DRAFT || V < 1 || V > 0x7FFFFFFF || row_base < 0)
        return SPEC_ERR_INVALID_ARG;
    if (row_base + B > ((int64_t)1 << 32)) return SPEC_ERR_INVALID_ARG;
    if (logits_dtype != SPEC_F32 && logits_dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
    if (!(temperature >= 0.f) || isinf(temperature)) return SPEC_ERR_INVALID_ARG;
    if (B == 0) return SPEC_OK;
    if (!target_logits || !out_tokens || !out_accepted) return SPEC_ERR_INVALID_ARG;
    if (K > 0 && !draft_tokens) return SPEC_ERR_INVALID_ARG;
    if (temperature > 0.f && K > 0 && !draft_probs) return SPEC_ERR_INVALID_ARG;
    const int64_t C = (V + kChunk - 1) / kChunk;
    // grid limit: k_decide has B*C workgroups
    if (B * C > ((int64_t)1 << 24) || B * (K + 1) * C > ((int64_t)1 << 40)) return SPEC_ERR_INVALID_ARG;
    const AcceptWs lay = accept_ws_layout(B, K, V);
    if (!workspace || workspace_bytes < lay.total || !aligned16(workspace)) return SPEC_ERR_WORKSPACE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    const float* q = (temperature > 0.f) ? draft_probs : nullptr;
    if (logits_dtype == SPEC_BF16) {
        const bf16_t* z = static_cast<const bf16_t*>(target_logits);
        const bool vec = (V % 8 == 0) && aligned16(z) && (!q || aligned16(q));
        if (vec)
            return launch_accept<bf16_t, true>(z, q, draft_tokens, draft_lens, B, K, V, row_base,
                                               temperature, philox_seed, philox_offset, out_tokens,
                                               out_accepted, out_p_draft, out_status, ws, lay, s);
        return launch_accept<bf16_t, false>(z, q, draft_tokens, draft_lens, B, K, V, row_base,
                                            temperature, philox_seed, philox_offset, out_tokens,
                                            out_accepted, out_p_draft, out_status, ws, lay, s);
    }
    const float* z = static_cast<const float*>(target_logits);
    const bool vec = (V % 4 == 0) && aligned16(z) && (!q || aligned16(q));
    if (vec)
        return launch_accept<float, true>(z, q, draft_tokens, draft_lens, B, K, V, row_base,
                                          temperature, philox_seed, philox_offset, out_tokens,
                                          out_accepted, out_p_draft, out_status, ws, lay, s);
    return launch_accept<float, false>(z, q, draft_tokens, draft_lens, B, K, V, row_base,
                                       temperature, philox_seed, philox_offset, out_tokens,
                                       out_accepted, out_p_draft, out_status, ws, lay, s);
}
