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
// Two launches on the caller's stream:
//  1. k_stats / k_argmax: one workgroup per (row, position <= L_b, chunk of
//     8192 vocabulary entries).  The chunk is streamed from HBM with 16-byte
//     coalesced loads into registers, reduced to its max, then to
//     sum_j 2^(z_j c - fl(m c)) with c = log2(e)/T (one FMA and one v_exp_f32
//     per element), wave64 shuffles + LDS across the workgroup, fp64 across
//     waves.  Greedy mode keeps (max, lowest index) instead.
//  2. k_finish / k_greedy_finish: one workgroup per (row, chunk).  Every
//     workgroup of a row merges the row's chunk partials (fixed order, fp64),
//     runs the acceptance tests (p_i(x_i) in fp64) and finds the first
//     rejection.  After a rejection each workgroup computes the residual mass
//     of its chunk; the last one to arrive (integer atomic counter) picks the
//     chunk by a two-level inverse CDF and scans that one chunk in LDS.  A
//     row with no rejection draws its bonus token from chunk masses it
//     already has (workgroup 0 of the row).
// No floating-point atomics: every reduction runs in a fixed order, so the
// output is a deterministic function of the inputs.
#include "spec_verify.h"
#include "device_common.hpp"
#include "philox.hpp"

#include <math.h>

namespace specv {
namespace {

constexpr int kThreads = 256;
constexpr int kEPT = 32;                     // elements per thread per chunk
constexpr int kChunk = kThreads * kEPT;      // vocabulary entries per chunk
constexpr int kWaves = kThreads / kWave;
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
static_assert(sizeof(StatPart) == 16 && sizeof(ArgPart) == 16, "partial layout");

typedef uint16_t bf16_t;

// ---- chunk loaders --------------------------------------------------------
// "Strided" layout: vector k of thread t is vector (k * kThreads + t) of the
// chunk, so a wave reads consecutive 16-byte vectors (coalesced).  The
// element index of register e is chunk0 + ((e / W) * kThreads + t) * W + e % W.
template <typename T, bool VEC> struct Lay { static constexpr int W = 1; };
template <> struct Lay<bf16_t, true> { static constexpr int W = 8; };
template <> struct Lay<float, true> { static constexpr int W = 4; };

template <int W>
__device__ __forceinline__ int64_t strided_index(int64_t chunk0, int t, int e) {
    return chunk0 + ((int64_t)(e / W) * kThreads + t) * W + (e % W);
}

__device__ __forceinline__ void unpack8(const uint4 w, float* v) {
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

template <typename T, bool VEC>
__device__ __forceinline__ void load_strided(const T* row, int64_t V, int64_t chunk0, int t,
                                             float (&v)[kEPT]) {
    if constexpr (VEC && sizeof(T) == 2) {
        const uint4* p = reinterpret_cast<const uint4*>(row);
        const uint4 ninf = make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
        uint4 w[kEPT / 8];
#pragma unroll
        for (int k = 0; k < kEPT / 8; ++k) {
            const int64_t vi = chunk0 / 8 + (int64_t)k * kThreads + t;
            w[k] = (vi * 8 < V) ? p[vi] : ninf;
        }
#pragma unroll
        for (int k = 0; k < kEPT / 8; ++k) unpack8(w[k], v + 8 * k);
    } else if constexpr (VEC) {
        const float4* p = reinterpret_cast<const float4*>(row);
        const float4 ninf = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
#pragma unroll
        for (int k = 0; k < kEPT / 4; ++k) {
            const int64_t vi = chunk0 / 4 + (int64_t)k * kThreads + t;
            const float4 f = (vi * 4 < V) ? p[vi] : ninf;
            v[4 * k] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kEPT; ++e) {
            const int64_t j = chunk0 + (int64_t)e * kThreads + t;
            float x = -INFINITY;
            if (j < V) {
                if constexpr (sizeof(T) == 2) x = bf16_to_f32(row[j]);
                else x = row[j];
            }
            v[e] = x;
        }
    }
}

// q values matching load_strided<T, VEC>'s element order; 0 past V.
template <typename T, bool VEC>
__device__ __forceinline__ void load_q_strided(const float* row, int64_t V, int64_t chunk0, int t,
                                               float (&v)[kEPT]) {
    constexpr int W = Lay<T, VEC>::W;
    if constexpr (W > 1) {
        const float4* p = reinterpret_cast<const float4*>(row);
#pragma unroll
        for (int k = 0; k < kEPT / W; ++k) {
            const int64_t vi = chunk0 / W + (int64_t)k * kThreads + t;
#pragma unroll
            for (int h = 0; h < W / 4; ++h) {
                const float4 f = (vi * W < V) ? p[vi * (W / 4) + h] : make_float4(0.f, 0.f, 0.f, 0.f);
                v[k * W + 4 * h] = f.x; v[k * W + 4 * h + 1] = f.y;
                v[k * W + 4 * h + 2] = f.z; v[k * W + 4 * h + 3] = f.w;
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < kEPT; ++e) {
            const int64_t j = chunk0 + (int64_t)e * kThreads + t;
            v[e] = (j < V) ? row[j] : 0.f;
        }
    }
}

// "Contiguous" layout for the in-chunk scan: thread t owns entries
// [start + t*kEPT, start + (t+1)*kEPT) in order.
template <typename T, bool VEC>
__device__ __forceinline__ void load_contig(const T* row, int64_t V, int64_t start, float (&v)[kEPT]) {
    if constexpr (VEC && sizeof(T) == 2) {
        const uint4* p = reinterpret_cast<const uint4*>(row + start);
        const uint4 ninf = make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
#pragma unroll
        for (int k = 0; k < kEPT / 8; ++k) {
            const uint4 w = (start + 8 * k < V) ? p[k] : ninf;
            unpack8(w, v + 8 * k);
        }
    } else if constexpr (VEC) {
        const float4* p = reinterpret_cast<const float4*>(row + start);
#pragma unroll
        for (int k = 0; k < kEPT / 4; ++k) {
            const float4 f = (start + 4 * k < V) ? p[k] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            v[4 * k] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kEPT; ++e) {
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

template <bool VEC>
__device__ __forceinline__ void load_q_contig(const float* row, int64_t V, int64_t start, float (&v)[kEPT]) {
    if constexpr (VEC) {
        const float4* p = reinterpret_cast<const float4*>(row + start);
#pragma unroll
        for (int k = 0; k < kEPT / 4; ++k) {
            const float4 f = (start + 4 * k < V) ? p[k] : make_float4(0.f, 0.f, 0.f, 0.f);
            v[4 * k] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kEPT; ++e) v[e] = (start + e < V) ? row[start + e] : 0.f;
    }
}

template <typename T>
__device__ __forceinline__ float load_one(const T* row, int64_t j) {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(row[j]);
    else return row[j];
}

// ---- per-element weights (identical expressions wherever used) -----------
// p-frame weight of logit z at a position with fl(M c) = mc.
__device__ __forceinline__ float p_weight(float z, float c, float mc) {
    return hw_exp2(__builtin_fmaf(z, c, -mc));
}
// residual weight max(p - q, 0) with p = weight / S, invS = fl(1/S).
__device__ __forceinline__ float r_weight(float z, float q, float c, float mc, float invS) {
    const float p = p_weight(z, c, mc) * invS;
    return fmaxf(p - q, 0.f);
}

// ---- workgroup reductions -------------------------------------------------
__device__ __forceinline__ float block_max(float v, float* sh) {
    v = wave_max(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) sh[w] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r = fmaxf(r, sh[k]);
    __syncthreads();
    return r;
}

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

__device__ __forceinline__ int block_or(int v, int* sh) {
    v = wave_or(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) sh[w] = v;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) r |= sh[k];
    __syncthreads();
    return r;
}

// ---- launch 1: chunk statistics --------------------------------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_stats(const T* __restrict__ logits,
                                                    const int32_t* __restrict__ lens, int K,
                                                    int64_t V, int C, float c,
                                                    StatPart* __restrict__ part,
                                                    int32_t* __restrict__ counters) {
    __shared__ float sh_f[kWaves];
    __shared__ double sh_d[kWaves];
    __shared__ int sh_i[kWaves];
    const int64_t bid = blockIdx.x;
    const int ci = (int)(bid % C);
    const int64_t rp = bid / C;
    const int i = (int)(rp % (K + 1));
    const int64_t b = rp / (K + 1);
    const int t = threadIdx.x;
    if (i == 0 && ci == 0 && t == 0) counters[b] = 0;
    const int L = lens ? lens[b] : K;
    if (L < 0 || L > K || i > L) return;

    float v[kEPT];
    load_strided<T, VEC>(logits + rp * V, V, (int64_t)ci * kChunk, t, v);

    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) m = fmaxf(m, v[e]);
    m = block_max(m, sh_f);

    int flag = 0;
    double s = 0.0;
    if (m == INFINITY) {
        flag = 1;
    } else if (m == -INFINITY) {
        int nan = 0;
#pragma unroll
        for (int e = 0; e < kEPT; ++e) nan |= (v[e] != v[e]);
        flag = block_or(nan, sh_i);
    } else {
        const float mc = m * c;
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int e = 0; e < kEPT; e += 4) {
            a0 += p_weight(v[e], c, mc);
            a1 += p_weight(v[e + 1], c, mc);
            a2 += p_weight(v[e + 2], c, mc);
            a3 += p_weight(v[e + 3], c, mc);
        }
        s = block_sum((double)((a0 + a1) + (a2 + a3)), sh_d);
        flag = (s != s) ? 1 : 0;
    }
    if (t == 0) part[bid] = StatPart{m, flag, s};
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_argmax(const T* __restrict__ logits,
                                                     const int32_t* __restrict__ lens, int K,
                                                     int64_t V, int C, ArgPart* __restrict__ part) {
    __shared__ float sh_v[kWaves];
    __shared__ int sh_x[kWaves];
    __shared__ int sh_f[kWaves];
    const int64_t bid = blockIdx.x;
    const int ci = (int)(bid % C);
    const int64_t rp = bid / C;
    const int i = (int)(rp % (K + 1));
    const int64_t b = rp / (K + 1);
    const int t = threadIdx.x;
    const int L = lens ? lens[b] : K;
    if (L < 0 || L > K || i > L) return;

    float v[kEPT];
    const int64_t chunk0 = (int64_t)ci * kChunk;
    load_strided<T, VEC>(logits + rp * V, V, chunk0, t, v);
    constexpr int W = Lay<T, VEC>::W;
    float best = -INFINITY;
    int bidx = 0x7FFFFFFF;
    int nan = 0;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
        const int64_t j = strided_index<W>(chunk0, t, e);
        const float x = v[e];
        if (j < V) {
            nan |= (x != x);
            if (x > best || (x == best && (int)j < bidx)) { best = x; bidx = (int)j; }
        }
    }
    // wave then workgroup reduction of (max, lowest index)
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o, kWave);
        const int oi = __shfl_xor(bidx, o, kWave);
        if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
    }
    nan = wave_or(nan);
    const int w = t / kWave;
    if ((t & (kWave - 1)) == 0) { sh_v[w] = best; sh_x[w] = bidx; sh_f[w] = nan; }
    __syncthreads();
    if (t == 0) {
        float bv = sh_v[0];
        int bi = sh_x[0];
        int f = sh_f[0];
        for (int k = 1; k < kWaves; ++k) {
            if (sh_v[k] > bv || (sh_v[k] == bv && sh_x[k] < bi)) { bv = sh_v[k]; bi = sh_x[k]; }
            f |= sh_f[k];
        }
        if (bv == INFINITY) f = 1;
        part[bid] = ArgPart{bv, f, bi, 0};
    }
}

// ---- launch 2: decisions, residual masses and the draw ----------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_finish(
    const T* __restrict__ logits, const float* __restrict__ q, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ lens, int K, int64_t V, int C, float c, int64_t row_base,
    uint64_t seed, uint64_t offset, const StatPart* __restrict__ part, double* resid,
    int32_t* counters, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_accepted,
    float* __restrict__ out_p_draft, int32_t* __restrict__ out_status) {
    __shared__ float s_M[SPEC_MAX_DRAFT + 1];
    __shared__ double s_S[SPEC_MAX_DRAFT + 1];
    __shared__ int s_acc[SPEC_MAX_DRAFT + 1];
    __shared__ float s_px[SPEC_MAX_DRAFT + 1];
    __shared__ double sh_d[kWaves];
    __shared__ double s_scan[kThreads + 1];
    __shared__ int s_status, s_a, s_last, s_cstar, s_pmode, s_tok, s_lastpos;
    __shared__ double s_tp;

    const int64_t b = blockIdx.x / C;
    const int ci = (int)(blockIdx.x % C);
    const int t = threadIdx.x;
    const int L = lens ? lens[b] : K;
    const bool len_ok = (L >= 0 && L <= K);
    if (t == 0) {
        s_status = len_ok ? 0 : SPEC_ROW_BAD_LEN;
        s_tok = 0x7FFFFFFF;
        s_lastpos = -1;
    }
    __syncthreads();

    // Merge the chunk partials of every position <= L_b and test each draft.
    if (len_ok) {
        for (int i = t; i <= L; i += kThreads) {
            const StatPart* pp = part + ((b * (K + 1) + i) * C);
            float M = -INFINITY;
            int flag = 0;
            for (int k = 0; k < C; ++k) { M = fmaxf(M, pp[k].m); flag |= pp[k].flag; }
            if (M == -INFINITY || M == INFINITY) flag = 1;
            const float mcM = M * c;
            double S = 0.0;
            if (!flag)
                for (int k = 0; k < C; ++k) {
                    const StatPart e = pp[k];
                    if (e.m != -INFINITY) {
                        const float mck = e.m * c;
                        S += e.s * exp2((double)mck - (double)mcM);
                    }
                }
            s_M[i] = M;
            s_S[i] = S;
            int st = flag ? SPEC_ROW_NONFINITE : 0;
            int acc = 1;
            float px = -1.f;
            if (i < L) {
                const int x = tokens[b * K + i];
                if (x < 0 || (int64_t)x >= V) {
                    st |= SPEC_ROW_BAD_TOKEN;
                } else {
                    const float qx = q[(b * K + i) * V + x];
                    if (!(qx > 0.f)) st |= SPEC_ROW_ZERO_Q;
                    if (!flag) {
                        const double zx = (double)load_one(logits + (b * (K + 1) + i) * V, x);
                        const double p = exp2(zx * (double)c - (double)mcM) / S;
                        px = (float)p;
                        if (qx > 0.f) {
                            const double a = fmin(1.0, p / (double)qx);
                            const RowPosUniforms u = row_pos_uniforms(seed, offset, (uint32_t)(row_base + b), (uint32_t)i);
                            acc = ((double)u.acc < a) ? 1 : 0;
                        }
                    }
                }
            }
            s_acc[i] = acc;
            s_px[i] = px;
            if (st) atomicOr(&s_status, st);
        }
    }
    __syncthreads();
    if (t == 0) {
        int a = L;
        if (len_ok)
            for (int i = 0; i < L; ++i)
                if (!s_acc[i]) { a = i; break; }
        s_a = a;
    }
    __syncthreads();
    int status = s_status;
    const int a = s_a;
    const bool invalid = (status & kInvalidMask) != 0;
    if (ci == 0 && out_p_draft)
        for (int i = t; i < K; i += kThreads)
            out_p_draft[b * K + i] = (!invalid && i < L) ? s_px[i] : -1.f;
    if (invalid) {
        if (ci == 0) {
            for (int i = t; i <= K; i += kThreads) out_tokens[b * (K + 1) + i] = -1;
            if (t == 0) {
                out_accepted[b] = -1;
                if (out_status) out_status[b] = status;
            }
        }
        return;
    }

    const bool reject = a < L;
    const float M = s_M[a];
    const double S = s_S[a];
    const float mcM = M * c;
    const float invS = (float)(1.0 / S);
    const T* zrow = logits + (b * (K + 1) + a) * V;
    const float* qrow = reject ? q + (b * K + a) * V : nullptr;

    if (reject) {
        // residual mass of this chunk
        float z[kEPT], qq[kEPT];
        const int64_t chunk0 = (int64_t)ci * kChunk;
        load_strided<T, VEC>(zrow, V, chunk0, t, z);
        load_q_strided<T, VEC>(qrow, V, chunk0, t, qq);
        float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
#pragma unroll
        for (int e = 0; e < kEPT; e += 4) {
            r0 += r_weight(z[e], qq[e], c, mcM, invS);
            r1 += r_weight(z[e + 1], qq[e + 1], c, mcM, invS);
            r2 += r_weight(z[e + 2], qq[e + 2], c, mcM, invS);
            r3 += r_weight(z[e + 3], qq[e + 3], c, mcM, invS);
        }
        const double R = block_sum((double)((r0 + r1) + (r2 + r3)), sh_d);
        if (t == 0) {
            __hip_atomic_store(&resid[b * C + ci], R, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __threadfence();
            const int old = atomicAdd(&counters[b], 1);
            s_last = (old == C - 1) ? 1 : 0;
        }
        __syncthreads();
        if (!s_last) return;
        __threadfence();
    } else if (ci != 0) {
        return;
    }

    // Pick the chunk (first level of the inverse CDF).
    if (t == 0) {
        const RowPosUniforms u = row_pos_uniforms(seed, offset, (uint32_t)(row_base + b), (uint32_t)a);
        int pmode = reject ? 0 : 1;
        double tot = 0.0;
        if (reject) {
            for (int k = 0; k < C; ++k)
                tot += __hip_atomic_load(&resid[b * C + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (!(tot > 0.0)) { pmode = 1; status |= SPEC_ROW_RESID_ZERO; }
        }
        const StatPart* pp = part + ((b * (K + 1) + a) * C);
        auto chunk_w = [&](int k) -> double {
            if (!pmode) return __hip_atomic_load(&resid[b * C + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const StatPart e = pp[k];
            if (e.m == -INFINITY) return 0.0;
            const float mck = e.m * c;
            return e.s * exp2((double)mck - (double)mcM);
        };
        if (pmode) {
            tot = 0.0;
            for (int k = 0; k < C; ++k) tot += chunk_w(k);
        }
        const double tt = (double)u.smp * tot;
        double cum = 0.0;
        int cstar = -1, lastpos = -1;
        double before = 0.0;
        for (int k = 0; k < C; ++k) {
            const double wk = chunk_w(k);
            if (wk > 0.0) lastpos = k;
            if (cstar < 0 && cum + wk > tt) { cstar = k; before = cum; }
            cum += wk;
        }
        double tp = tt - before;
        if (cstar < 0) {  // rounding left t at or past the total: last positive entry overall
            cstar = lastpos;
            tp = INFINITY;
        }
        s_cstar = cstar;
        s_pmode = pmode;
        s_tp = tp;
        s_status = status;
    }
    __syncthreads();
    const int cstar = s_cstar;
    const int pmode = s_pmode;
    const double tp = s_tp;
    status = s_status;

    // Second level: scan the chosen chunk in index order.
    const int64_t start = (int64_t)cstar * kChunk + (int64_t)t * kEPT;
    float w[kEPT];
    {
        float z[kEPT];
        load_contig<T, VEC>(zrow, V, start, z);
        if (pmode) {
#pragma unroll
            for (int e = 0; e < kEPT; ++e) w[e] = p_weight(z[e], c, mcM);
        } else {
            float qq[kEPT];
            load_q_contig<VEC>(qrow, V, start, qq);
#pragma unroll
            for (int e = 0; e < kEPT; ++e) w[e] = r_weight(z[e], qq[e], c, mcM, invS);
        }
    }
    double own = 0.0;
    int lastpos = -1;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
        own += (double)w[e];
        if (w[e] > 0.f) lastpos = e;
    }
    // exclusive scan of the per-thread sums: wave64 shuffle scan, then waves
    {
        const int lane = t & (kWave - 1);
        double inc = own;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const double n = __shfl_up(inc, o, kWave);
            if (lane >= o) inc += n;
        }
        const int wv = t / kWave;
        if (lane == kWave - 1) sh_d[wv] = inc;
        __syncthreads();
        double base = 0.0;
        for (int k = 0; k < wv; ++k) base += sh_d[k];
        s_scan[t + 1] = base + inc;
        if (t == 0) s_scan[0] = 0.0;
    }
    __syncthreads();
    const double lo = s_scan[t], hi = s_scan[t + 1];
    if (lo <= tp && tp < hi) {
        double cum = lo;
        int found = -1;
#pragma unroll
        for (int e = 0; e < kEPT; ++e) {
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
        for (int i = 0; i < a; ++i) out_tokens[b * (K + 1) + i] = tokens[b * K + i];
        out_tokens[b * (K + 1) + a] = tok;
        for (int i = a + 1; i <= K; ++i) out_tokens[b * (K + 1) + i] = -1;
        out_accepted[b] = a;
        if (out_status) out_status[b] = status;
    }
}

__global__ __launch_bounds__(kWave) void k_greedy_finish(
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ lens, int K, int64_t V, int C,
    const ArgPart* __restrict__ part, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_accepted, float* __restrict__ out_p_draft,
    int32_t* __restrict__ out_status) {
    __shared__ int s_g[SPEC_MAX_DRAFT + 1];
    __shared__ int s_match[SPEC_MAX_DRAFT + 1];
    __shared__ int s_status;
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    const int L = lens ? lens[b] : K;
    const bool len_ok = (L >= 0 && L <= K);
    if (t == 0) s_status = len_ok ? 0 : SPEC_ROW_BAD_LEN;
    __syncthreads();
    if (len_ok) {
        for (int i = t; i <= L; i += kWave) {
            const ArgPart* pp = part + ((b * (K + 1) + i) * C);
            float bv = -INFINITY;
            int bi = 0x7FFFFFFF, flag = 0;
            for (int k = 0; k < C; ++k) {
                const ArgPart e = pp[k];
                flag |= e.flag;
                if (e.v > bv || (e.v == bv && e.idx < bi)) { bv = e.v; bi = e.idx; }
            }
            if (bv == -INFINITY || bv == INFINITY) flag = 1;
            int st = flag ? SPEC_ROW_NONFINITE : 0;
            s_g[i] = bi;
            int match = 0;
            if (i < L) {
                const int x = tokens[b * K + i];
                if (x < 0 || (int64_t)x >= V) st |= SPEC_ROW_BAD_TOKEN;
                match = (x == bi) ? 1 : 0;
            }
            s_match[i] = match;
            if (st) atomicOr(&s_status, st);
        }
    }
    __syncthreads();
    const int status = s_status;
    const bool invalid = (status & kInvalidMask) != 0;
    int a = L;
    if (!invalid)
        for (int i = 0; i < L; ++i)
            if (!s_match[i]) { a = i; break; }
    if (out_p_draft)
        for (int i = t; i < K; i += kWave)
            out_p_draft[b * K + i] = (!invalid && i < L) ? (float)s_match[i] : -1.f;
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

// ---- host side ----------------------------------------------------------------
struct AcceptWs {
    size_t part_off, resid_off, count_off, total;
};

AcceptWs accept_ws_layout(int64_t B, int K, int64_t V) {
    const int64_t C = (V + kChunk - 1) / kChunk;
    AcceptWs w;
    w.part_off = 0;
    w.resid_off = align_up((size_t)B * (K + 1) * C * sizeof(StatPart), 256);
    w.count_off = w.resid_off + align_up((size_t)B * C * sizeof(double), 256);
    w.total = w.count_off + align_up((size_t)B * sizeof(int32_t), 256);
    return w;
}

template <typename T, bool VEC>
int launch_accept(const T* logits, const float* q, const int32_t* tokens, const int32_t* lens,
                  int64_t B, int K, int64_t V, int64_t row_base, float temperature, uint64_t seed,
                  uint64_t offset, int32_t* out_tokens, int32_t* out_accepted, float* out_p_draft,
                  int32_t* out_status, char* ws, const AcceptWs& lay, hipStream_t stream) {
    const int C = (int)((V + kChunk - 1) / kChunk);
    const int64_t n1 = B * (K + 1) * C;
    int32_t* counters = reinterpret_cast<int32_t*>(ws + lay.count_off);
    if (temperature == 0.f) {
        ArgPart* part = reinterpret_cast<ArgPart*>(ws + lay.part_off);
        hipLaunchKernelGGL((k_argmax<T, VEC>), dim3((unsigned)n1), dim3(kThreads), 0, stream,
                           logits, lens, K, V, C, part);
        if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
        hipLaunchKernelGGL(k_greedy_finish, dim3((unsigned)B), dim3(kWave), 0, stream, tokens, lens,
                           K, V, C, part, out_tokens, out_accepted, out_p_draft, out_status);
        if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
        return SPEC_OK;
    }
    // c = log2(e) / T, rounded once to fp32
    const float c = (float)(1.4426950408889634074 / (double)temperature);
    StatPart* part = reinterpret_cast<StatPart*>(ws + lay.part_off);
    double* resid = reinterpret_cast<double*>(ws + lay.resid_off);
    hipLaunchKernelGGL((k_stats<T, VEC>), dim3((unsigned)n1), dim3(kThreads), 0, stream, logits,
                       lens, K, V, C, c, part, counters);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    hipLaunchKernelGGL((k_finish<T, VEC>), dim3((unsigned)(B * C)), dim3(kThreads), 0, stream,
                       logits, q, tokens, lens, K, V, C, c, row_base, seed, offset, part, resid,
                       counters, out_tokens, out_accepted, out_p_draft, out_status);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    return SPEC_OK;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace
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
    // grid limits: launch 1 has B(K+1)C workgroups of 256 threads
    if (B * (K + 1) * C > ((int64_t)1 << 24) || B * C > ((int64_t)1 << 24)) return SPEC_ERR_INVALID_ARG;
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
