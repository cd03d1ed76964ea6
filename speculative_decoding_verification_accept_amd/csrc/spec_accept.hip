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
// One launch.  The vocabulary is cut into chunks of 16 KB of logits (8192
// bf16 or 4096 fp32 entries) and one 256-thread workgroup owns one (row b,
// chunk) pair; the C workgroups of a row have consecutive indices.
//  phase 1  the workgroup streams its chunk of the logits at every verified
//           position i <= L_b (16-byte coalesced loads; the next position's
//           loads are in flight while the current one is reduced) and
//           publishes, per position, the chunk max m and
//           sum_j 2^(fl(z_j c - fl(m c))) with c = fl(log2(e) / T): one FMA and
//           one v_exp_f32 per entry, fp64 across lanes (greedy mode: the max
//           and its lowest index).  The workgroup whose chunk holds draft
//           token x_i also gathers z_i(x_i) and q_i(x_i).
//  decide   the last of the row's workgroups to finish phase 1 merges the
//           partials of each position in a fixed order (fp64), runs the
//           acceptance tests, finds the first rejection a_b and publishes
//           the decision.  Greedy mode writes the row's outputs here.
//  phase 2  every workgroup of the row waits for the decision, then publishes
//           its chunk's mass at position a_b: the residual sum of
//           max(p - q, 0) after a rejection, the p-mass for the bonus token.
//  sample   the last of the row's workgroups to publish its mass draws the
//           token by inverse CDF: the chunk masses pick the chunk, then one
//           LDS-staged fp64 scan of that chunk picks the token.
// Rows do not wait for one another: a row with short drafts is in phase 2
// while longer rows still stream phase 1.
//
// Exchange between workgroups of one launch.  Every word one workgroup
// publishes for another is written and read with agent-scope atomic
// accesses, which gfx950 issues with the SC1 bit: the store goes through to
// the device's coherence point and the load is served from it, so the eight
// per-XCD L2 caches never hand out a stale copy.  Before a workgroup counts
// itself in on a row counter it waits for its own stores to complete
// (s_waitcnt vmcnt(0)), so the workgroup that sees the final count also sees
// every published word.  The decision, which waiting workgroups poll, is
// two words with a tag bit each.  The per-row records (two counters and the
// decision words, 256 bytes per row, at the start of the workspace) must be
// zero when a call starts; the workgroup that consumes a record last resets
// it, so a workspace zeroed once stays valid for every later call with the
// same or fewer rows.  Each record has cache lines of its own: device-scope
// atomics on one line serialise.
//
// Progress.  A workgroup waits only for the decision of its own row, which
// needs only phase 1 of that row's workgroups, and phase 1 never waits.
// Workgroups are dispatched in index order, so the lowest unfinished row
// always has all of its workgroups resident.  Each wait is bounded anyway:
// past the bound the workgroup marks its row SPEC_ROW_STALLED and exits.
//
// No floating-point atomics: every reduction runs in a fixed order, so the
// outputs are a deterministic function of the inputs.
#include "spec_verify.h"
#include "device_common.hpp"
#include "philox.hpp"

#include <math.h>

#include <atomic>
#include <mutex>

namespace specv {
namespace {

constexpr int kThreads = 256;                // one workgroup per (row, chunk)
constexpr int kChunkBytes = 16384;           // logits bytes per chunk
constexpr int kWaves = kThreads / kWave;
// Entries per chunk and per thread: 8192 bf16 or 4096 fp32 logits.
template <typename T> constexpr int chunk_of() { return kChunkBytes / (int)sizeof(T); }
template <typename T> constexpr int ept_of() { return chunk_of<T>() / kThreads; }
constexpr int kMinChunk = kChunkBytes / 4;   // the smallest chunk (fp32), for sizing
constexpr int kPos = SPEC_MAX_DRAFT + 1;     // positions per row at most
constexpr int kMaxChunks = 1024;             // chunks per row at most (the sampler keeps their masses in LDS)
constexpr int kMergeRegs = 2;                // chunk partials held per lane by the merge
constexpr int kSpinLimit = 1 << 16;          // polls of one wait (~0.1 s) before giving up (default)
constexpr int kRowStride = 64;               // ints per row-counter record: 256 bytes
constexpr int kInvalidMask = SPEC_ROW_NONFINITE | SPEC_ROW_BAD_TOKEN | SPEC_ROW_BAD_LEN | SPEC_ROW_ZERO_Q;

typedef uint16_t bf16_t;

// Row-counter record (zero between calls): [0] phase-1 arrivals,
// [16] phase-2 arrivals, [32..35] the two tagged decision words, [48] set by
// a workgroup that gave up waiting for the decision.
constexpr int kCnt1 = 0, kCnt2 = 16, kDec = 32, kStall = 48;

// ---- exchange between workgroups -----------------------------------------------
__device__ __forceinline__ void co_store(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t co_load(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void co_store32(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int co_load32(const int* p) {
    return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int co_add(int* p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave has issued has completed
// (vmcnt = 0; expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void drain_vm() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ uint64_t pack2(float lo, uint32_t hi) {
    return (uint64_t)__float_as_uint(lo) | ((uint64_t)hi << 32);
}
__device__ __forceinline__ uint64_t dbits(double d) { return (uint64_t)__double_as_longlong(d); }
__device__ __forceinline__ double bitsd(uint64_t u) { return __longlong_as_double((long long)u); }

// ---- partials --------------------------------------------------------------------
// Stochastic partial of one (row, position, chunk): word 0 = chunk max m
// (low half) and a flag (high half: 1 = NaN or +Inf in the chunk); word 1 =
// fp64 sum_j 2^(fl(z_j c - fl(m c))).  Greedy partial: word 0 = max value
// and flag, word 1 = lowest index of the max.
struct StatPart {
    float m;
    int flag;
    double s;
};
__device__ __forceinline__ void publish_part(uint64_t* p, float m, int flag, uint64_t w1) {
    co_store(p, pack2(m, (uint32_t)flag));
    co_store(p + 1, w1);
}
__device__ __forceinline__ StatPart read_part(const uint64_t* p) {
    const uint64_t w0 = co_load(p), w1 = co_load(p + 1);
    return StatPart{__uint_as_float((uint32_t)w0), (int)(w0 >> 32), bitsd(w1)};
}

// ---- loaders ---------------------------------------------------------------------
template <typename T, bool VEC> struct Lay { static constexpr int W = 1; };
template <> struct Lay<bf16_t, true> { static constexpr int W = 8; };
template <> struct Lay<float, true> { static constexpr int W = 4; };

// "Strided" layout over the workgroup: vector k of thread t is vector
// (k * kThreads + t) of the chunk, so consecutive threads read consecutive
// 16-byte vectors.  Register e of thread t holds entry
//   chunk0 + ((e / W) * kThreads + t) * W + e % W.
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

// One thread's share of a chunk of logits in strided layout, kept as loaded
// so that loads stay in flight until the values are used.  Entries past V
// read as -inf.
template <typename T, bool VEC, int EPT> struct Raw;

template <int EPT> struct Raw<bf16_t, true, EPT> {
    uint4 r[EPT / 8];
    __device__ __forceinline__ void load(const bf16_t* row, int64_t V, int64_t chunk0, int t) {
        const uint4* p = reinterpret_cast<const uint4*>(row + chunk0) + t;
        if (chunk0 + EPT * kThreads <= V) {  // whole chunk in range (uniform)
#pragma unroll
            for (int k = 0; k < EPT / 8; ++k) r[k] = p[k * kThreads];
        } else {
#pragma unroll
            for (int k = 0; k < EPT / 8; ++k)
                r[k] = (chunk0 + ((int64_t)k * kThreads + t) * 8 < V)
                           ? p[k * kThreads]
                           : make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
        }
    }
    __device__ __forceinline__ void unpack(float (&v)[EPT]) const {
#pragma unroll
        for (int k = 0; k < EPT / 8; ++k) unpack8(r[k], v + 8 * k);
    }
};

template <int EPT> struct Raw<float, true, EPT> {
    float4 r[EPT / 4];
    __device__ __forceinline__ void load(const float* row, int64_t V, int64_t chunk0, int t) {
        const float4* p = reinterpret_cast<const float4*>(row + chunk0) + t;
        if (chunk0 + EPT * kThreads <= V) {
#pragma unroll
            for (int k = 0; k < EPT / 4; ++k) r[k] = p[k * kThreads];
        } else {
#pragma unroll
            for (int k = 0; k < EPT / 4; ++k)
                r[k] = (chunk0 + ((int64_t)k * kThreads + t) * 4 < V)
                           ? p[k * kThreads]
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

template <typename T, int EPT> struct Raw<T, false, EPT> {
    float r[EPT];
    __device__ __forceinline__ void load(const T* row, int64_t V, int64_t chunk0, int t) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int64_t j = chunk0 + (int64_t)e * kThreads + t;
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

// q entries in the same order as Raw<T, VEC, EPT>; 0 past V.
template <typename T, bool VEC, int EPT>
__device__ __forceinline__ void load_q_strided(const float* row, int64_t V, int64_t chunk0, int t,
                                               float (&v)[EPT]) {
    constexpr int W = Lay<T, VEC>::W;
    if constexpr (W > 1) {
        const float4* p = reinterpret_cast<const float4*>(row + chunk0) + (int64_t)t * (W / 4);
        const bool full = chunk0 + EPT * kThreads <= V;  // uniform
#pragma unroll
        for (int k = 0; k < EPT / W; ++k) {
            const bool ok = full || chunk0 + ((int64_t)k * kThreads + t) * W < V;
#pragma unroll
            for (int h = 0; h < W / 4; ++h) {
                const float4 f = ok ? p[(int64_t)k * kThreads * (W / 4) + h] : make_float4(0.f, 0.f, 0.f, 0.f);
                v[k * W + 4 * h] = f.x; v[k * W + 4 * h + 1] = f.y;
                v[k * W + 4 * h + 2] = f.z; v[k * W + 4 * h + 3] = f.w;
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int64_t j = chunk0 + (int64_t)e * kThreads + t;
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
__device__ __forceinline__ float block_max(float v, float* sh) {
    v = wave_max(v);
    if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r = fmaxf(r, sh[k]);
    return r;
}
// Fixed-order workgroup sum; the total is valid in every thread.  The caller
// separates consecutive uses of one `sh` with a barrier.
__device__ __forceinline__ double block_sum(double v, double* sh) {
    v = wave_sum(v);
    if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = v;
    __syncthreads();
    double r = sh[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r += sh[k];
    return r;
}
__device__ __forceinline__ int block_or(int v, int* sh) {
    v = wave_or(v);
    if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = v;
    __syncthreads();
    int r = sh[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r |= sh[k];
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

// Merge of the C chunk partials of one position by one wave (lanes over
// chunks, butterfly reductions: a fixed order).
struct PosStats {
    float M;
    double S;
    int flag;
};
__device__ __forceinline__ PosStats merge_position(const uint64_t* pp, int C, float c) {
    const int lane = threadIdx.x & (kWave - 1);
    StatPart e[kMergeRegs];
    float M = -INFINITY;
    int flag = 0;
#pragma unroll
    for (int r = 0; r < kMergeRegs; ++r) {
        const int k = lane + r * kWave;
        e[r] = (k < C) ? read_part(pp + 2 * k) : StatPart{-INFINITY, 0, 0.0};
        M = fmaxf(M, e[r].m);
        flag |= e[r].flag;
    }
    for (int k = lane + kMergeRegs * kWave; k < C; k += kWave) {
        const StatPart x = read_part(pp + 2 * k);
        M = fmaxf(M, x.m);
        flag |= x.flag;
    }
    M = wave_max(M);
    flag = wave_or(flag);
    if (M == -INFINITY || M == INFINITY) flag = 1;
    const float mcM = M * c;
    double S = 0.0;
    if (!flag) {
#pragma unroll
        for (int r = 0; r < kMergeRegs; ++r) S += chunk_p_mass(e[r], c, mcM);
        for (int k = lane + kMergeRegs * kWave; k < C; k += kWave) S += chunk_p_mass(read_part(pp + 2 * k), c, mcM);
    }
    S = wave_sum(S);
    return PosStats{M, S, flag};
}

// Greedy merge: (max value, lowest index) over the chunk partials.
__device__ __forceinline__ void merge_argmax(const uint64_t* pp, int C, float& bv, int& bi, int& flag) {
    const int lane = threadIdx.x & (kWave - 1);
    bv = -INFINITY;
    bi = 0x7FFFFFFF;
    flag = 0;
    for (int k = lane; k < C; k += kWave) {
        const uint64_t w0 = co_load(pp + 2 * k), w1 = co_load(pp + 2 * k + 1);
        const float v = __uint_as_float((uint32_t)w0);
        const int idx = (int)w1;
        flag |= (int)(w0 >> 32);
        if (v > bv || (v == bv && idx < bi)) { bv = v; bi = idx; }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    flag = wave_or(flag);
    if (bv == -INFINITY || bv == INFINITY) flag = 1;
}

// ---- decision words ------------------------------------------------------------------
// word 0: bit 0 tag, bit 1 reject, bits 2..9 status, bits 10..17 a_b,
//         bits 32..63 M (max logit at a_b);  word 1: bit 0 tag, bits 32..63 fl(1/S)
struct Decision {
    int a, status, reject;
    float M, invS;
};
__device__ __forceinline__ uint64_t dec_word0(const Decision& d) {
    return 1ull | ((uint64_t)(d.reject & 1) << 1) | ((uint64_t)(d.status & 0xFF) << 2) |
           ((uint64_t)(d.a & 0xFF) << 10) | ((uint64_t)__float_as_uint(d.M) << 32);
}
__device__ __forceinline__ uint64_t dec_word1(const Decision& d) {
    return 1ull | ((uint64_t)__float_as_uint(d.invS) << 32);
}
__device__ __forceinline__ Decision dec_read(uint64_t w0, uint64_t w1) {
    return Decision{(int)((w0 >> 10) & 0xFF), (int)((w0 >> 2) & 0xFF), (int)((w0 >> 1) & 1),
                    __uint_as_float((uint32_t)(w0 >> 32)), __uint_as_float((uint32_t)(w1 >> 32))};
}

// ---- draw weights at the chosen position ---------------------------------------------
// Weight of entry j: the residual max(p - q, 0) after a rejection (qrow set),
// the p-frame weight otherwise; 0 past V.
template <typename T>
__device__ __forceinline__ float entry_weight(const T* zrow, const float* qrow, int64_t V, int64_t j,
                                              float c, float mcM, float invS) {
    if (j >= V) return 0.f;
    const float z = load_one(zrow, j);
    return qrow ? r_weight(z, qrow[j], c, mcM, invS) : p_weight(z, c, mcM);
}
// Sum, in index order and fp64, of the weights of entries [start, start + EPT):
// the same per-entry expressions as entry_weight.
template <typename T, bool VEC, int EPT>
__device__ __forceinline__ double thread_weight_sum(const T* zrow, const float* qrow, int64_t V,
                                                    int64_t start, float c, float mcM, float invS) {
    float z[EPT];
    load_contig<T, VEC, EPT>(zrow, V, start, z);
    double own = 0.0;
    if (qrow) {
        float qq[EPT];
        load_q_contig<VEC, EPT>(qrow, V, start, qq);
#pragma unroll
        for (int e = 0; e < EPT; ++e) own += (double)r_weight(z[e], qq[e], c, mcM, invS);
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) own += (double)p_weight(z[e], c, mcM);
    }
    return own;
}

// Inclusive scan of one double per lane across a wave.
__device__ __forceinline__ double wave_incl_scan(double v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double n = __shfl_up(v, o, kWave);
        if (lane >= o) v += n;
    }
    return v;
}

// ---- the kernel -----------------------------------------------------------------------------
struct Args {
    const void* logits;
    const float* q;
    const int32_t* tokens;
    const int32_t* lens;
    int64_t B, V, row_base;
    int K, C;
    int spin_limit;  // polls of the decision before a workgroup gives up on its row
    float c;  // log2(e) / T (stochastic)
    uint64_t seed, offset;
    int32_t* out_tokens;
    int32_t* out_accepted;
    float* out_p_draft;
    int32_t* out_status;
    int* rows;       // row-counter records, kRowStride ints per row
    uint64_t* part;  // [B][K+1][C] two words each
    uint64_t* gath;  // [B][K] z_i(x_i) | q_i(x_i) << 32
    uint64_t* mass;  // [B][C] fp64 chunk masses at a_b
    uint64_t* tsum;  // [B][C][kThreads] fp64 per-thread weight sums at a_b
};

struct Shared {
    float red_f[kWaves];
    double red_d[kWaves];
    int red_i[kWaves];
    float red_v[kWaves];
    int red_x[kWaves];
    StatPart own[kPos];  // this workgroup's partial at each position
    union {
        struct {  // decide
            float M[kPos];
            double S[kPos];
            int flag[kPos];
            float px[kPos];
            int gi[kPos];
        } d;
        struct {  // sample
            double w[kMaxChunks];  // chunk masses
            double scan[kThreads + 1];
        } s;
    } u;
    double tp;
    int status, a, last, cstar, lastpos;
    uint64_t w0, w1;
};

// sh.lastpos = max(sh.lastpos, base + the last thread of the workgroup with
// `pos` set): one ballot per wave and one LDS word per wave (same-address LDS
// atomics from every thread would serialise).  Ends with a barrier.
__device__ __forceinline__ void last_positive(bool pos, int base, Shared& sh) {
    const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
    const uint64_t m = __ballot(pos);
    if (lane == 0) sh.red_x[wv] = m ? wv * kWave + 63 - __clzll((long long)m) : -1;
    __syncthreads();
    if (t == 0) {
        int l = -1;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) l = max(l, sh.red_x[k]);
        if (l >= 0) sh.lastpos = max(sh.lastpos, base + l);
    }
    __syncthreads();
}

template <typename T, bool VEC>
__device__ void write_invalid_row(const Args& g, int64_t b, int status, int t) {
    for (int i = t; i <= g.K; i += kThreads) g.out_tokens[b * (g.K + 1) + i] = -1;
    if (g.out_p_draft)
        for (int i = t; i < g.K; i += kThreads) g.out_p_draft[b * g.K + i] = -1.f;
    if (t == 0) {
        g.out_accepted[b] = -1;
        if (g.out_status) g.out_status[b] = status;
    }
}

template <typename T, bool VEC, bool GREEDY>
__global__ __launch_bounds__(kThreads) void k_accept(Args g) {
    constexpr int W = Lay<T, VEC>::W;
    constexpr int EPT = ept_of<T>(), CH = chunk_of<T>();
    __shared__ Shared sh;
    const T* logits = static_cast<const T*>(g.logits);
    const int64_t b = blockIdx.x / g.C;
    const int ci = (int)(blockIdx.x % g.C);
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wv = t / kWave;
    const int K = g.K, C = g.C;
    const int64_t V = g.V;
    const float c = g.c;
    int* rowc = g.rows + b * kRowStride;

    const int L = g.lens ? g.lens[b] : K;
    if (L < 0 || L > K) {  // no counter of this row is touched
        if (ci == 0) write_invalid_row<T, VEC>(g, b, SPEC_ROW_BAD_LEN, t);
        return;
    }
    const int64_t chunk0 = (int64_t)ci * CH;
    const T* zrow0 = logits + b * (K + 1) * V;

    // draft token of position t (t < L); the owner of its chunk gathers
    // z_t(x_t) and q_t(x_t) for the acceptance test
    const int x = (t < L) ? g.tokens[b * K + t] : -1;
    if (!GREEDY && t < L && x >= 0 && (int64_t)x < V && x / CH == ci) {
        const float zx = load_one(zrow0 + (int64_t)t * V, x);
        const float qx = g.q[(b * K + t) * V + x];
        co_store(g.gath + b * K + t, pack2(zx, __float_as_uint(qx)));
    }

    // ---- phase 1: chunk statistics at every position i <= L ----
    uint64_t* prow = g.part + (b * (K + 1)) * C * 2;
    auto reduce = [&](const Raw<T, VEC, EPT>& raw, int i) {
        float v[EPT];
        raw.unpack(v);
        uint64_t* pp = prow + ((int64_t)i * C + ci) * 2;
        if constexpr (GREEDY) {
            float best = -INFINITY;
            int bidx = 0x7FFFFFFF, nan = 0;
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const int64_t j = strided_index<W>(chunk0, t, e);
                const float xv = v[e];
                if (j < V) {
                    nan |= (xv != xv);
                    if (xv > best || (xv == best && (int)j < bidx)) { best = xv; bidx = (int)j; }
                }
            }
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) {
                const float ov = __shfl_xor(best, o, kWave);
                const int oi = __shfl_xor(bidx, o, kWave);
                if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
            }
            nan = wave_or(nan);
            if (lane == 0) {
                sh.red_v[wv] = best;
                sh.red_x[wv] = bidx;
                sh.red_i[wv] = nan;
            }
            __syncthreads();
            if (t == 0) {
                float bv = sh.red_v[0];
                int bi = sh.red_x[0], fl = sh.red_i[0];
#pragma unroll
                for (int k = 1; k < kWaves; ++k) {
                    fl |= sh.red_i[k];
                    if (sh.red_v[k] > bv || (sh.red_v[k] == bv && sh.red_x[k] < bi)) { bv = sh.red_v[k]; bi = sh.red_x[k]; }
                }
                publish_part(pp, bv, (fl || bv == INFINITY) ? 1 : 0, (uint64_t)(uint32_t)bi);
            }
            __syncthreads();
        } else {
            float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
            for (int e = 0; e < EPT; e += 2) {
                m0 = fmaxf(m0, v[e]);
                m1 = fmaxf(m1, v[e + 1]);
            }
            const float m = block_max(fmaxf(m0, m1), sh.red_f);
            int flag = 0;
            double s = 0.0;
            if (m == INFINITY) {
                flag = 1;
            } else if (m == -INFINITY) {
                int nan = 0;
#pragma unroll
                for (int e = 0; e < EPT; ++e) nan |= (v[e] != v[e]);
                flag = block_or(nan, sh.red_i);
            } else {
                const float mc = m * c;
                float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
                for (int e = 0; e < EPT; e += 4) {
                    a0 += p_weight(v[e], c, mc);
                    a1 += p_weight(v[e + 1], c, mc);
                    a2 += p_weight(v[e + 2], c, mc);
                    a3 += p_weight(v[e + 3], c, mc);
                }
                s = block_sum((double)((a0 + a1) + (a2 + a3)), sh.red_d);
                flag = (s != s) ? 1 : 0;
            }
            if (t == 0) {
                publish_part(pp, m, flag, dbits(s));
                sh.own[i] = StatPart{m, flag, s};
            }
            __syncthreads();  // separates this position's reductions from the next
        }
    };
    {
        Raw<T, VEC, EPT> buf0, buf1;
        buf0.load(zrow0, V, chunk0, t);
        if (L >= 1) buf1.load(zrow0 + V, V, chunk0, t);
        for (int i = 0; i <= L; i += 2) {
            reduce(buf0, i);
            if (i + 2 <= L) buf0.load(zrow0 + (int64_t)(i + 2) * V, V, chunk0, t);
            if (i + 1 > L) break;
            reduce(buf1, i + 1);
            if (i + 3 <= L) buf1.load(zrow0 + (int64_t)(i + 3) * V, V, chunk0, t);
        }
    }

    // count in on the row; the last workgroup decides
    drain_vm();
    __syncthreads();
    if (t == 0) sh.last = (co_add(rowc + kCnt1, 1) == C - 1);
    __syncthreads();

    if (sh.last) {
        // ---- decide ----
        if (t == 0) {
            co_store32(rowc + kCnt1, 0);
            sh.status = 0;
            sh.a = L;
        }
        __syncthreads();
        if constexpr (GREEDY) {
            for (int i = wv; i <= L; i += kWaves) {
                float bv;
                int bi, fl;
                merge_argmax(prow + (int64_t)i * C * 2, C, bv, bi, fl);
                if (lane == 0) {
                    sh.u.d.gi[i] = bi;
                    sh.u.d.flag[i] = fl;
                }
            }
            if (t < L && (x < 0 || (int64_t)x >= V)) atomicOr(&sh.status, SPEC_ROW_BAD_TOKEN);
            __syncthreads();
            // the listing's order: the row stops at the first draft that is
            // not the argmax, or at the first position that is not finite
            // (the row is then invalid); positions after the stop do not count
            if ((t < L && x != sh.u.d.gi[t]) || (t <= L && sh.u.d.flag[t])) atomicMin(&sh.a, t);
            __syncthreads();
            const int a = sh.a;
            const int status = sh.status | (sh.u.d.flag[a] ? SPEC_ROW_NONFINITE : 0);
            const bool invalid = (status & kInvalidMask) != 0;
            if (g.out_p_draft)
                for (int i = t; i < K; i += kThreads)
                    g.out_p_draft[b * K + i] =
                        (!invalid && i < L && i <= a) ? (g.tokens[b * K + i] == sh.u.d.gi[i] ? 1.f : 0.f) : -1.f;
            for (int i = t; i <= K; i += kThreads) {
                int v = -1;
                if (!invalid) {
                    if (i < a) v = g.tokens[b * K + i];
                    else if (i == a) v = sh.u.d.gi[a];
                }
                g.out_tokens[b * (K + 1) + i] = v;
            }
            if (t == 0) {
                g.out_accepted[b] = invalid ? -1 : a;
                if (g.out_status) g.out_status[b] = status;
            }
            return;
        } else {
            // gathers and token checks (one thread per drafted position)
            float zx = 0.f, qx = 1.f;
            if (t < L) {
                int st = 0;
                if (x < 0 || (int64_t)x >= V) {
                    st = SPEC_ROW_BAD_TOKEN;
                } else {
                    const uint64_t gw = co_load(g.gath + b * K + t);
                    zx = __uint_as_float((uint32_t)gw);
                    qx = __uint_as_float((uint32_t)(gw >> 32));
                    if (!(qx > 0.f)) st = SPEC_ROW_ZERO_Q;
                }
                if (st) atomicOr(&sh.status, st);
            }
            for (int i = wv; i <= L; i += kWaves) {
                const PosStats ps = merge_position(prow + (int64_t)i * C * 2, C, c);
                if (lane == 0) {
                    sh.u.d.M[i] = ps.M;
                    sh.u.d.S[i] = ps.S;
                    sh.u.d.flag[i] = ps.flag;
                }
            }
            __syncthreads();
            // the listing's order: the row stops at its first rejection, or
            // at the first position that is not finite (the row is then
            // invalid); positions after the stop do not count
            if (t <= L && sh.u.d.flag[t]) atomicMin(&sh.a, t);
            if (t < L) {
                float px = -1.f;
                int rej = 0;
                if (!sh.u.d.flag[t] && qx > 0.f) {
                    const float mcM = sh.u.d.M[t] * c;
                    const double p = exp2((double)zx * (double)c - (double)mcM) / sh.u.d.S[t];
                    px = (float)p;
                    const double acc = fmin(1.0, p / (double)qx);
                    const RowPosUniforms u = row_pos_uniforms(g.seed, g.offset, (uint32_t)(g.row_base + b), (uint32_t)t);
                    rej = ((double)u.acc < acc) ? 0 : 1;
                }
                sh.u.d.px[t] = px;
                if (rej) atomicMin(&sh.a, t);
            }
            __syncthreads();
            const int a = sh.a;
            const int status = sh.status | (sh.u.d.flag[a] ? SPEC_ROW_NONFINITE : 0);
            const bool invalid = (status & kInvalidMask) != 0;
            if (g.out_p_draft)
                for (int i = t; i < K; i += kThreads)
                    g.out_p_draft[b * K + i] = (!invalid && i < L && i <= a) ? sh.u.d.px[i] : -1.f;
            if (invalid) write_invalid_row<T, VEC>(g, b, status, t);
            if (t == 0) {
                Decision d{invalid ? 0 : a, status, (!invalid && a < L) ? 1 : 0,
                           invalid ? 0.f : sh.u.d.M[a], invalid ? 0.f : (float)(1.0 / sh.u.d.S[a])};
                const uint64_t w0 = dec_word0(d), w1 = dec_word1(d);
                co_store(reinterpret_cast<uint64_t*>(rowc + kDec), w0);
                co_store(reinterpret_cast<uint64_t*>(rowc + kDec) + 1, w1);
                sh.w0 = w0;
                sh.w1 = w1;
            }
        }
    } else {
        if constexpr (GREEDY) return;
        // ---- wait for the row's decision ----
        if (t == 0) {
            const uint64_t* dw = reinterpret_cast<const uint64_t*>(rowc + kDec);
            uint64_t w0 = 0, w1 = 0;
            int n = 0;
            for (;;) {
                w0 = co_load(dw);
                w1 = co_load(dw + 1);
                if (w0 & w1 & 1) break;
                if (++n >= g.spin_limit) break;
                __builtin_amdgcn_s_sleep(8);
            }
            sh.w0 = w0;
            sh.w1 = w1;
        }
    }
    __syncthreads();
    // The bound ran out: this workgroup gives up on the row.  It flags the
    // row record and still counts in below, so the row's last workgroup
    // (which writes the row as stalled) resets the record as always.
    const bool stalled = !(sh.w0 & sh.w1 & 1);
    const Decision d = dec_read(sh.w0, sh.w1);
    const bool invalid = (d.status & kInvalidMask) != 0;
    const int a = d.a;
    const float mcM = d.M * c;

    // ---- phase 2: this chunk's draw weights at position a ----
    // Thread t sums the weights of entries [chunk0 + t EPT, + EPT) and
    // publishes that sum (the sampler's second level) and the chunk's total
    // (its first level).
    const T* zrow = zrow0 + (int64_t)a * V;
    const float* qrow = d.reject ? g.q + (b * K + a) * V : nullptr;
    uint64_t* tsrow = g.tsum + b * C * kThreads;  // [C][kThreads]
    double mass = 0.0;
    if (stalled) {
        if (t == 0) co_store32(rowc + kStall, 1);
    } else if (!invalid) {
        const double own = thread_weight_sum<T, VEC, EPT>(zrow, qrow, V, chunk0 + (int64_t)t * EPT, c, mcM, d.invS);
        co_store(tsrow + (int64_t)ci * kThreads + t, dbits(own));
        mass = block_sum(own, sh.red_d);
    }
    if (t == 0 && !stalled) co_store(g.mass + b * C + ci, dbits(mass));
    drain_vm();
    __syncthreads();
    if (t == 0) sh.last = (co_add(rowc + kCnt2, 1) == C - 1);
    __syncthreads();
    if (!sh.last) return;

    // ---- sample (the row's last workgroup) ----
    // Every workgroup of the row has counted in, so none reads the row's
    // record again: reset it for the next call.  A workgroup that gave up
    // flagged the record before counting in; the row is then written as
    // stalled (the decider may never have finished it).
    if (t == 0) {
        sh.last = co_load32(rowc + kStall);
        co_store32(rowc + kCnt2, 0);
        co_store32(rowc + kStall, 0);
        co_store(reinterpret_cast<uint64_t*>(rowc + kDec), 0);
        co_store(reinterpret_cast<uint64_t*>(rowc + kDec) + 1, 0);
    }
    __syncthreads();
    if (sh.last != 0) {
        for (int i = t; i <= K; i += kThreads) g.out_tokens[b * (K + 1) + i] = -1;
        if (t == 0) {
            g.out_accepted[b] = -1;
            if (g.out_status) g.out_status[b] = SPEC_ROW_STALLED;
        }
        return;
    }
    if (invalid) return;  // the decider wrote the row
    int status = d.status;
    int pmode = d.reject ? 0 : 1;  // 0: residual, 1: bonus from p, 2: empty residual, from p
    const uint64_t* pa = prow + (int64_t)a * C * 2;

    // level 1: the chunk.  Chunk masses go to LDS (C <= kMaxChunks); an empty
    // residual is replaced by the p-frame masses of the position's partials.
    for (int k = t; k < C; k += kThreads) sh.u.s.w[k] = bitsd(co_load(g.mass + b * C + k));
    __syncthreads();
    double tot;
    for (;;) {
        double part = 0.0;
        for (int k = t; k < C; k += kThreads) part += sh.u.s.w[k];
        tot = block_sum(part, sh.red_d);
        __syncthreads();
        if (pmode != 0 || tot > 0.0) break;
        pmode = 2;
        status |= SPEC_ROW_RESID_ZERO;
        for (int k = t; k < C; k += kThreads) sh.u.s.w[k] = chunk_p_mass(read_part(pa + 2 * k), c, mcM);
        __syncthreads();
    }
    const RowPosUniforms u = row_pos_uniforms(g.seed, g.offset, (uint32_t)(g.row_base + b), (uint32_t)a);
    double tp = (double)u.smp * tot;
    if (t == 0) {
        sh.cstar = -1;
        sh.lastpos = -1;
    }
    double carry = 0.0;
    for (int k0 = 0; k0 < C; k0 += kThreads) {
        const int k = k0 + t;
        const double wk = (k < C) ? sh.u.s.w[k] : 0.0;
        double btot;
        const double incl = carry + block_incl_scan(wk, sh.red_d, &btot);
        sh.u.s.scan[t + 1] = incl;
        if (t == 0) sh.u.s.scan[0] = carry;
        __syncthreads();
        if (wk > 0.0 && incl > tp && sh.u.s.scan[t] <= tp) {  // unique: the scan is non-decreasing
            sh.cstar = k;
            sh.tp = tp - sh.u.s.scan[t];
        }
        last_positive(wk > 0.0, k0, sh);
        if (sh.cstar >= 0) break;
        carry += btot;
    }
    int cstar = sh.cstar;
    tp = sh.tp;
    if (cstar < 0) {  // rounding left t at or past the total: the last positive chunk
        cstar = max(sh.lastpos, 0);
        tp = INFINITY;
    }
    __syncthreads();

    // level 2: the thread of chunk c* whose entries hold the draw
    const int64_t cbase = (int64_t)cstar * CH;
    const float* qdraw = pmode == 0 ? qrow : nullptr;
    const double ts = (pmode == 2)
                          ? thread_weight_sum<T, VEC, EPT>(zrow, nullptr, V, cbase + (int64_t)t * EPT, c, mcM, d.invS)
                          : bitsd(co_load(tsrow + (int64_t)cstar * kThreads + t));
    if (t == 0) {
        sh.cstar = -1;
        sh.lastpos = -1;
    }
    double ttot;
    const double incl2 = block_incl_scan(ts, sh.red_d, &ttot);
    sh.u.s.scan[t + 1] = incl2;
    if (t == 0) sh.u.s.scan[0] = 0.0;
    __syncthreads();
    if (ts > 0.0 && incl2 > tp && sh.u.s.scan[t] <= tp) {
        sh.cstar = t;
        sh.tp = tp - sh.u.s.scan[t];
    }
    last_positive(ts > 0.0, 0, sh);
    int tstar = sh.cstar;
    tp = sh.tp;
    if (tstar < 0) {
        tstar = max(sh.lastpos, 0);
        tp = INFINITY;
    }

    // level 3: that thread's EPT entries, one per lane of wave 0, in index order
    if (wv == 0) {
        const int64_t j0 = cbase + (int64_t)tstar * EPT;
        const float wl = (lane < EPT) ? entry_weight(zrow, qdraw, V, j0 + lane, c, mcM, d.invS) : 0.f;
        const double incl3 = wave_incl_scan((double)wl);
        const uint64_t hit = __ballot(wl > 0.f && incl3 > tp);
        const uint64_t pos = __ballot(wl > 0.f);
        const int sel = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
        if (lane == 0) {
            g.out_tokens[b * (K + 1) + a] = (int32_t)(j0 + sel);
            g.out_accepted[b] = a;
            if (g.out_status) g.out_status[b] = status;
        }
    }
    for (int i = t; i <= K; i += kThreads)
        if (i != a) g.out_tokens[b * (K + 1) + i] = (i < a) ? g.tokens[b * K + i] : -1;
}

// ---- host side ------------------------------------------------------------------------------
struct AcceptWs {
    size_t rows_off, part_off, gath_off, mass_off, tsum_off, total;
};

AcceptWs accept_ws_layout(int64_t B, int K, int64_t V) {
    const int64_t C = (V + kMinChunk - 1) / kMinChunk;  // the most chunks of either dtype
    AcceptWs w;
    w.rows_off = 0;
    w.part_off = align_up((size_t)B * kRowStride * sizeof(int), 256);
    w.gath_off = w.part_off + align_up((size_t)B * (K + 1) * C * 16, 256);
    w.mass_off = w.gath_off + align_up((size_t)B * K * 8, 256);
    w.tsum_off = w.mass_off + align_up((size_t)B * C * 8, 256);
    w.total = w.tsum_off + align_up((size_t)B * C * kThreads * 8, 256);
    return w;
}

template <typename T, bool VEC>
int launch_accept(const Args& a, hipStream_t stream, bool greedy) {
    const dim3 grid((unsigned)(a.B * a.C));
    if (greedy) hipLaunchKernelGGL((k_accept<T, VEC, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((k_accept<T, VEC, false>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kMaxDevicesNoAlloc = 64;  // devices the allocation-free entry point serves

// Polls of the decision before a workgroup gives up on its row (process-wide;
// only a test of the give-up path changes it).
std::atomic<int> g_wait_bound{kSpinLimit};

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_accept_workspace_bytes(int64_t B, int K, int64_t V) {
    if (B < 0 || K < 0 || K > SPEC_MAX_DRAFT || V < 1) return 0;
    return accept_ws_layout(B, K, V).total;
}

namespace specv {
namespace {

// Host-side validation and argument packing shared by the entry points.
// Returns SPEC_OK with the call packed, kNothing when B == 0, or a negative
// code; it makes no HIP call.
constexpr int kNothing = 1;
struct AcceptCall {
    Args a;
    AcceptWs lay;
    bool bf16, greedy, vec;
};

int accept_prepare(const void* target_logits, int logits_dtype, const float* draft_probs,
                   const int32_t* draft_tokens, const int32_t* draft_lens, int64_t B, int K,
                   int64_t V, int64_t row_base, float temperature, uint64_t philox_seed,
                   uint64_t philox_offset, int32_t* out_tokens, int32_t* out_accepted,
                   float* out_p_draft, int32_t* out_status, AcceptCall& call) {
    if (B < 0 || K < 0 || K > SPEC_MAX_DRAFT || V < 1 || V > 0x7FFFFFFF || row_base < 0)
        return SPEC_ERR_INVALID_ARG;
    if (row_base + B > ((int64_t)1 << 32)) return SPEC_ERR_INVALID_ARG;
    if (logits_dtype != SPEC_F32 && logits_dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
    if (!(temperature >= 0.f) || isinf(temperature)) return SPEC_ERR_INVALID_ARG;
    if (B == 0) return kNothing;
    if (!target_logits || !out_tokens || !out_accepted) return SPEC_ERR_INVALID_ARG;
    if (K > 0 && !draft_tokens) return SPEC_ERR_INVALID_ARG;
    if (temperature > 0.f && K > 0 && !draft_probs) return SPEC_ERR_INVALID_ARG;
    const bool bf16 = logits_dtype == SPEC_BF16;
    const int64_t C = bf16 ? (V + chunk_of<bf16_t>() - 1) / chunk_of<bf16_t>()
                           : (V + chunk_of<float>() - 1) / chunk_of<float>();
    // one workgroup per (row, chunk); the sampler holds a row's chunk masses in LDS
    if (B * C > ((int64_t)1 << 24) || C > kMaxChunks) return SPEC_ERR_INVALID_ARG;
    const bool greedy = temperature == 0.f;
    Args& a = call.a;
    a = Args{};
    a.logits = target_logits;
    a.q = greedy ? nullptr : draft_probs;
    a.tokens = draft_tokens;
    a.lens = draft_lens;
    a.B = B;
    a.V = V;
    a.row_base = row_base;
    a.K = K;
    a.C = (int)C;
    a.spin_limit = g_wait_bound.load(std::memory_order_relaxed);
    // c = log2(e) / T, rounded once to fp32
    a.c = greedy ? 0.f : (float)(1.4426950408889634074 / (double)temperature);
    a.seed = philox_seed;
    a.offset = philox_offset;
    a.out_tokens = out_tokens;
    a.out_accepted = out_accepted;
    a.out_p_draft = out_p_draft;
    a.out_status = out_status;
    call.lay = accept_ws_layout(B, K, V);
    call.bf16 = bf16;
    call.greedy = greedy;
    call.vec = (V % (bf16 ? 8 : 4) == 0) && aligned16(target_logits) && (!a.q || aligned16(a.q));
    return SPEC_OK;
}

// Points the call at its workspace `ws` (device memory of call.lay.total
// bytes whose row records are zero) and launches it on `s`.
int accept_launch(AcceptCall& call, char* ws, hipStream_t s) {
    Args& a = call.a;
    const AcceptWs& lay = call.lay;
    a.rows = reinterpret_cast<int*>(ws + lay.rows_off);
    a.part = reinterpret_cast<uint64_t*>(ws + lay.part_off);
    a.gath = reinterpret_cast<uint64_t*>(ws + lay.gath_off);
    a.mass = reinterpret_cast<uint64_t*>(ws + lay.mass_off);
    a.tsum = reinterpret_cast<uint64_t*>(ws + lay.tsum_off);
    if (call.bf16)
        return call.vec ? launch_accept<bf16_t, true>(a, s, call.greedy) : launch_accept<bf16_t, false>(a, s, call.greedy);
    return call.vec ? launch_accept<float, true>(a, s, call.greedy) : launch_accept<float, false>(a, s, call.greedy);
}

}  // namespace
}  // namespace specv

extern "C" int spec_accept(const void* target_logits, int logits_dtype, const float* draft_probs,
                           const int32_t* draft_tokens, const int32_t* draft_lens, int64_t B,
                           int K, int64_t V, int64_t row_base, float temperature,
                           uint64_t philox_seed, uint64_t philox_offset, int32_t* out_tokens,
                           int32_t* out_accepted, float* out_p_draft, int32_t* out_status,
                           void* workspace, size_t workspace_bytes, void* stream) {
    AcceptCall call;
    const int rc = accept_prepare(target_logits, logits_dtype, draft_probs, draft_tokens, draft_lens, B, K, V,
                                  row_base, temperature, philox_seed, philox_offset, out_tokens, out_accepted,
                                  out_p_draft, out_status, call);
    if (rc == kNothing) return SPEC_OK;
    if (rc != SPEC_OK) return rc;
    if (!workspace || workspace_bytes < call.lay.total || !aligned16(workspace)) return SPEC_ERR_WORKSPACE;
    return accept_launch(call, static_cast<char*>(workspace), reinterpret_cast<hipStream_t>(stream));
}

// ---- the entry point that allocates nothing -------------------------------------------
// Its workspace is this file-scope array, one copy per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device memory: the device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is ever passed on.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace specv {
namespace {

__global__ void k_zero16(uint4* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct ScratchDev {
    std::mutex mu;
    char* ptr = nullptr;  // device address of `scratch` on this device, once set up
};
ScratchDev g_scratch[kMaxDevicesNoAlloc];

// The current device's copy of `scratch`; on first use, its address is taken
// and the whole array is cleared by a fill kernel on `s` (the row records must
// start at zero; every call leaves them zero).  Null on a HIP error.
char* scratch_of_current_device(hipStream_t s) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevicesNoAlloc) return nullptr;
    ScratchDev& sd = g_scratch[dev];
    std::lock_guard<std::mutex> lock(sd.mu);
    if (sd.ptr) return sd.ptr;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    hipLaunchKernelGGL(k_zero16, dim3(1024), dim3(256), 0, s, static_cast<uint4*>(p),
                       (int64_t)(kScratchBytes / sizeof(uint4)));
    if (hipGetLastError() != hipSuccess) return nullptr;
    sd.ptr = static_cast<char*>(p);
    return sd.ptr;
}

}  // namespace
}  // namespace specv

extern "C" int spec_accept_noalloc(const void* target_logits, int logits_dtype, const float* draft_probs,
                                   const int32_t* draft_tokens, const int32_t* draft_lens, int64_t B,
                                   int K, int64_t V, int64_t row_base, float temperature,
                                   uint64_t philox_seed, uint64_t philox_offset, int32_t* out_tokens,
                                   int32_t* out_accepted, float* out_p_draft, int32_t* out_status,
                                   void* stream) {
    AcceptCall call;
    const int rc = accept_prepare(target_logits, logits_dtype, draft_probs, draft_tokens, draft_lens, B, K, V,
                                  row_base, temperature, philox_seed, philox_offset, out_tokens, out_accepted,
                                  out_p_draft, out_status, call);
    if (rc == kNothing) return SPEC_OK;
    if (rc != SPEC_OK) return rc;
    if (call.lay.total > kScratchBytes) return SPEC_ERR_WORKSPACE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = scratch_of_current_device(s);
    if (!ws) return SPEC_ERR_HIP;
    return accept_launch(call, ws, s);
}

extern "C" int spec_debug_set_wait_bound(int polls) {
    if (polls < 0) return SPEC_ERR_INVALID_ARG;
    g_wait_bound.store(polls == 0 ? kSpinLimit : polls, std::memory_order_relaxed);
    return SPEC_OK;
}
