// spec_verify_attention.hip -- attention of a verify pass: the K+1 query
// positions of each sequence (the token that ended the previous pass, then
// its drafts) against the sequence's KV cache, causal within the verified
// block, with grouped KV heads.
//
// Sources (by page title and section):
//  * "Speculative decoding and early exit: accelerated autoregressive
//    decoding" (reactapp.top), section "Attention structure during decoding"
//    (each step's queries read the whole key/value memory; one head: Q
//    [8, 1, 128] against K, V [8, 2048, 128]) and section "Speculative
//    decoding: draft first, then verify" (one target pass over K+1 positions).
//  * "Decode is memory-bound ..." (trefon.com), the ceiling section: at long
//    context the cache is read in full on every pass, next to the weights.
//  * agentnet.co.il item, section "GEMM-M grows, a small batch suffices":
//    verifying D drafts multiplies the rows by 1+D; here those rows share
//    one read of the cache.
//
// Work: one workgroup per (KV-range split s, KV head g, sequence b), of
// eight waves for one 16-row tile of queries and four for two (the larger
// state would spill at eight).  The query rows of (b, g) are R = (K+1) G
// (position-major, then the G query heads of the group), at most 32: one or
// two 16-row tiles.
// Each wave takes 32-key steps of the split, interleaved with the other
// waves, and keeps its own online-softmax state (running max and sum per
// row, unnormalised output) in registers:
//  * scores S^T = K Q^T with v_mfma_f32_16x16x32_bf16.  A lane holds, as the
//    A operand, 8 consecutive head dims of one key row (one 16-byte load):
//    row m of key tile t is key 8 (m / 4) + 4 t + m % 4, so that the score
//    lane (kg, li) receives (rows 4 kg .. 4 kg + 3 of both tiles) covers
//    keys 8 kg .. 8 kg + 7 of query row li;
//  * P V with the same MFMA: those 8 probabilities (bf16) are exactly the A
//    operand of query row li over k-slots 8 kg .. 8 kg + 7.  The B operand
//    needs 8 keys of one head dim; a lane loads keys 8 kg + j (j < 8), dims
//    8 li .. 8 li + 7 (8 loads of 16 bytes) and repacks them in registers
//    into 8 operands, one per dim 8 li + e: output column li of MFMA e is
//    head dim 8 li + e.  No LDS on the streaming path.
// The next two steps' loads are always in flight; their key indices are
// clamped into the split's range, so prefetches past its end re-read the
// last row (a cache hit) instead of branching around the loads.
// The waves' states merge in LDS (log-sum-exp); with one split the
// workgroup writes the normalised output, else an unnormalised partial that
// k_attn_combine merges over the splits (a fixed grouping and order).
#include "spec_verify.h"
#include "device_common.hpp"

namespace specv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = SPEC_ATTN_HEAD_DIM;     // 128
constexpr int kStep = 32;                  // keys per wave step
// Waves of a workgroup: eight for one 16-row tile, four for two (whose
// state needs twice the registers: at eight waves it would spill).
template <int RT> constexpr int attn_waves() { return RT == 1 ? 8 : 4; }
constexpr int kMaxRows = SPEC_ATTN_MAX_ROWS;
constexpr int kSplitTarget = 256;          // workgroups a launch aims for
constexpr int kSplitMinKeys = 256;         // keys per split at least

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

struct AttnArgs {
    const uint16_t* q;    // [B, K+1, H, kD]
    const uint16_t* kc;   // [B, Hkv, S, kD]
    const uint16_t* vc;   // [B, Hkv, S, kD]
    const int32_t* ctx;   // [B]
    const int32_t* lens;  // [B] or null
    void* out;            // [B, K+1, H, kD]
    int32_t* status;      // [B] or null
    float* part_o;        // [B, Hkv, nsplit, R, kD]
    float* part_ml;       // [B, Hkv, nsplit, R, 2]
    int64_t B, S;
    int K, H, Hkv, G, R, nsplit, chunk, out_bf16;
    float c;  // scale * log2(e)
};

// L_b, and T_b = ctx_b + L_b + 1 keys, or -1 (T = 0) for a row whose lengths
// do not fit the cache.
__device__ __forceinline__ int seq_len(const AttnArgs& a, int64_t b, int& ctx, int& T) {
    ctx = a.ctx[b];
    const int L = a.lens ? a.lens[b] : a.K;
    if (ctx < 0 || L < 0 || L > a.K || (int64_t)ctx + L + 1 > a.S) {
        T = 0;
        return -1;
    }
    T = ctx + L + 1;
    return L;
}

struct Stage {
    uint4 k[2][4];  // [key tile][32-dim step]
    uint4 v[8];     // keys 8 kg + j, dims 8 li .. 8 li + 7
};

__device__ __forceinline__ void load_stage(const uint16_t* kh, const uint16_t* vh, int64_t kb,
                                           int64_t last, int kg, int li, Stage& st) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t key = min(kb + 8 * (li >> 2) + 4 * t + (li & 3), last);
        const uint4* p = reinterpret_cast<const uint4*>(kh + key * kD);
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) st.k[t][ds] = p[4 * ds + kg];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t key = min(kb + 8 * kg + j, last);
        st.v[j] = reinterpret_cast<const uint4*>(vh + key * kD)[li];
    }
}

__device__ __forceinline__ uint32_t half_of(const uint4& u, int e) {
    const uint32_t w = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

template <int RT>
struct WaveState {
    uint4 q[RT][4];
    f32x4_t o[RT][8];
    float m[RT], l[RT];
    int lim[RT];  // last key each of this lane's query rows (li) may see
};

template <int RT>
__device__ __forceinline__ void attend_step(const Stage& st, int64_t kb, int64_t hi, bool need_mask,
                                            float c, int kg, int li, WaveState<RT>& ws) {
    f32x4_t s[2][RT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            s[t][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ds = 0; ds < 4; ++ds) s[t][rt] = mfma16(st.k[t][ds], ws.q[rt][ds], s[t][rt]);
        }
    // B operands of P V: head dim 8 li + e of keys 8 kg + j
    uint4 bv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bv[e].x = half_of(st.v[0], e) | (half_of(st.v[1], e) << 16);
        bv[e].y = half_of(st.v[2], e) | (half_of(st.v[3], e) << 16);
        bv[e].z = half_of(st.v[4], e) | (half_of(st.v[5], e) << 16);
        bv[e].w = half_of(st.v[6], e) | (half_of(st.v[7], e) << 16);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float sv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] = s[j >> 2][rt][j & 3] * c;
        if (need_mask) {
            const int64_t lim = min((int64_t)ws.lim[rt], hi - 1);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (kb + 8 * kg + j > lim) sv[j] = -INFINITY;
        }
        float mx = sv[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
        // The running max of a row moves only when one of its scores exceeds
        // it; otherwise every rescale factor is exactly 1 (2^0), so the
        // cross-lane max and the rescale of the outputs are skipped for the
        // whole wave (same results, bit for bit).
        if (__ballot(mx > ws.m[rt])) {
            mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
            const float mnew = fmaxf(ws.m[rt], mx);
            const float alpha = mnew == -INFINITY ? 1.f : hw_exp2(ws.m[rt] - mnew);
            ws.m[rt] = mnew;
            ws.l[rt] *= alpha;
            // rows of the output tile held by this lane: 4 kg + r; their
            // factor lives in lane 4 kg + r (query row = lane % 16)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * kg + r, kWave);
#pragma unroll
                for (int e = 0; e < 8; ++e) ws.o[rt][e][r] *= ar;
            }
        }
        const float mnew = ws.m[rt];
        float p[8], ps = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = sv[j] == -INFINITY ? 0.f : hw_exp2(sv[j] - mnew);
            ps += p[j];
        }
        ws.l[rt] += ps;
        uint4 pa;
        pa.x = (uint32_t)f32_to_bf16(p[0]) | ((uint32_t)f32_to_bf16(p[1]) << 16);
        pa.y = (uint32_t)f32_to_bf16(p[2]) | ((uint32_t)f32_to_bf16(p[3]) << 16);
        pa.z = (uint32_t)f32_to_bf16(p[4]) | ((uint32_t)f32_to_bf16(p[5]) << 16);
        pa.w = (uint32_t)f32_to_bf16(p[6]) | ((uint32_t)f32_to_bf16(p[7]) << 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) ws.o[rt][e] = mfma16(pa, bv[e], ws.o[rt][e]);
    }
}

__device__ __forceinline__ void store_val(void* out, int bf16, int64_t idx, float v) {
    if (bf16) static_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
    else static_cast<float*>(out)[idx] = v;
}

template <int RT>
__global__ __launch_bounds__(attn_waves<RT>() * kWave) void k_attn(AttnArgs a) {
    constexpr int NR = RT * 16;
    constexpr int NWV = attn_waves<RT>(), NTH = NWV * kWave;
    constexpr int kRound = NWV * kStep;  // keys per step of the whole workgroup
    __shared__ float sm[NWV][NR], sl[NWV][NR];
    __shared__ float so[NWV][NR][kD];
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int kg = lane >> 4, li = lane & 15;
    const int s = blockIdx.x, g = blockIdx.y;
    const int64_t b = blockIdx.z;
    int ctx, T;
    const int L = seq_len(a, b, ctx, T);
    const int64_t lo = (int64_t)s * a.chunk, hi = min((int64_t)T, lo + a.chunk);

    WaveState<RT> ws;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = 16 * rt + li;
        const int i = r / a.G, h = g * a.G + r % a.G;
        const bool ok = r < a.R && i <= L;
        const int ic = min(i, a.K);  // padding rows past R: an in-range address, never read
        const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((b * (a.K + 1) + ic) * a.H + h) * kD);
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) ws.q[rt][ds] = ok ? qp[4 * ds + kg] : make_uint4(0u, 0u, 0u, 0u);
        ws.lim[rt] = ok ? ctx + i : -1;
        ws.m[rt] = -INFINITY;
        ws.l[rt] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ws.o[rt][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // this wave's steps: keys lo + 32 (w + NWV n) < hi
    const int64_t first = lo + kStep * w;
    const int nsteps = first < hi ? (int)((hi - first + kRound - 1) / kRound) : 0;
    if (nsteps > 0) {
        const int64_t plane = (b * a.Hkv + g) * a.S * kD;
        const uint16_t* kh = a.kc + plane;
        const uint16_t* vh = a.vc + plane;
        const int64_t last = hi - 1;
        Stage st0, st1;
        load_stage(kh, vh, first, last, kg, li, st0);
        load_stage(kh, vh, first + kRound, last, kg, li, st1);
        for (int n = 0; n < nsteps; n += 2) {
            const int64_t kb = first + (int64_t)n * kRound;
            attend_step<RT>(st0, kb, hi, kb + kStep > ctx || kb + kStep > hi, a.c, kg, li, ws);
            load_stage(kh, vh, kb + 2 * kRound, last, kg, li, st0);
            const int64_t kb1 = kb + kRound;  // past hi on the last odd step: fully masked
            attend_step<RT>(st1, kb1, hi, kb1 + kStep > ctx || kb1 + kStep > hi, a.c, kg, li, ws);
            load_stage(kh, vh, kb1 + 2 * kRound, last, kg, li, st1);
        }
    }

    // merge the waves: running max and sum per row, scaled outputs
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float l = ws.l[rt];
        l += __shfl_xor(l, 16, kWave);
        l += __shfl_xor(l, 32, kWave);
        if (kg == 0) {
            sm[w][16 * rt + li] = ws.m[rt];
            sl[w][16 * rt + li] = l;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int r = 0; r < 4; ++r) so[w][16 * rt + 4 * kg + r][8 * li + e] = ws.o[rt][e][r];
    }
    __syncthreads();
    const bool direct = a.nsplit == 1;
    for (int idx = t; idx < NR * kD; idx += NTH) {
        const int r = idx / kD, dim = idx % kD;
        if (r >= a.R) break;  // rows are visited in order
        float M = sm[0][r];
#pragma unroll
        for (int k = 1; k < NWV; ++k) M = fmaxf(M, sm[k][r]);
        float o = 0.f, ls = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int k = 0; k < NWV; ++k) {
                const float f = sm[k][r] == -INFINITY ? 0.f : hw_exp2(sm[k][r] - M);
                o += so[k][r][dim] * f;
                ls += sl[k][r] * f;
            }
        }
        const int i = r / a.G, h = g * a.G + r % a.G;
        if (direct) {
            const float v = (i <= L && ls > 0.f) ? o / ls : 0.f;
            store_val(a.out, a.out_bf16, ((b * (a.K + 1) + i) * a.H + h) * kD + dim, v);
        } else {
            const int64_t pr = ((b * a.Hkv + g) * a.nsplit + s) * a.R + r;
            a.part_o[pr * kD + dim] = o;
            if (dim == 0) {
                a.part_ml[2 * pr] = M;
                a.part_ml[2 * pr + 1] = ls;
            }
        }
    }
    if (direct && a.status && s == 0 && g == 0 && t == 0) a.status[b] = L < 0 ? SPEC_ROW_BAD_LEN : 0;
}

// One workgroup per (query row r, KV head g, sequence b): ng groups of 128
// threads (thread = head dim; ng = blockDim / 128, at most 4, just enough
// that one batch covers the splits when it can) take the splits
// s = group (mod ng), eight at a time with every load issued before use,
// each keeping a running (max, sum, output); the groups then merge in LDS in
// group order.
constexpr int kCGroups = 4;
constexpr int kCBatch = 8;

__global__ __launch_bounds__(kCGroups * kD) void k_attn_combine(AttnArgs a) {
    __shared__ float cm[kCGroups], cl[kCGroups], co[kCGroups][kD];
    const int dim = threadIdx.x % kD, grp = threadIdx.x / kD, ng = blockDim.x / kD;
    const int r = blockIdx.x, g = blockIdx.y;
    const int64_t b = blockIdx.z;
    int ctx, T;
    const int L = seq_len(a, b, ctx, T);
    const int64_t base = (b * a.Hkv + g) * a.nsplit * a.R + r;  // split s at base + s R
    float m = -INFINITY, l = 0.f, o = 0.f;
    for (int s0 = grp; s0 < a.nsplit; s0 += ng * kCBatch) {
        float ms[kCBatch], ls[kCBatch], os[kCBatch];
#pragma unroll
        for (int k = 0; k < kCBatch; ++k) {
            const int s = s0 + k * ng;
            const int64_t pr = base + (int64_t)min(s, a.nsplit - 1) * a.R;
            ms[k] = a.part_ml[2 * pr];
            ls[k] = a.part_ml[2 * pr + 1];
            os[k] = a.part_o[pr * kD + dim];
            if (s >= a.nsplit) ms[k] = -INFINITY;
        }
#pragma unroll
        for (int k = 0; k < kCBatch; ++k) {
            const float mn = fmaxf(m, ms[k]);
            if (mn == -INFINITY) continue;
            const float fa = m == -INFINITY ? 0.f : hw_exp2(m - mn);
            const float fb = ms[k] == -INFINITY ? 0.f : hw_exp2(ms[k] - mn);
            o = o * fa + os[k] * fb;
            l = l * fa + ls[k] * fb;
            m = mn;
        }
    }
    co[grp][dim] = o;
    if (dim == 0) {
        cm[grp] = m;
        cl[grp] = l;
    }
    __syncthreads();
    if (grp != 0) return;
    float M = cm[0];
    for (int k = 1; k < ng; ++k) M = fmaxf(M, cm[k]);
    float ot = 0.f, lt = 0.f;
    if (M != -INFINITY) {
        for (int k = 0; k < ng; ++k) {
            const float f = cm[k] == -INFINITY ? 0.f : hw_exp2(cm[k] - M);
            ot += co[k][dim] * f;
            lt += cl[k] * f;
        }
    }
    const int i = r / a.G, h = g * a.G + r % a.G;
    const float v = (i <= L && lt > 0.f) ? ot / lt : 0.f;
    store_val(a.out, a.out_bf16, ((b * (a.K + 1) + i) * a.H + h) * kD + dim, v);
    if (a.status && r == 0 && g == 0 && dim == 0) a.status[b] = L < 0 ? SPEC_ROW_BAD_LEN : 0;
}

struct AttnPlan {
    int nsplit, chunk;
    size_t part_o_bytes, part_ml_bytes;
};

AttnPlan attn_plan(int64_t B, int K, int H, int Hkv, int64_t S) {
    AttnPlan p{};
    const int64_t pairs = std::max<int64_t>(B * Hkv, 1);
    int64_t ns = (kSplitTarget + pairs - 1) / pairs;
    ns = std::min<int64_t>(ns, std::max<int64_t>((S + kSplitMinKeys - 1) / kSplitMinKeys, 1));
    ns = std::max<int64_t>(ns, 1);
    int64_t chunk = (S + ns - 1) / ns;
    chunk = (chunk + kStep - 1) / kStep * kStep;
    ns = (S + chunk - 1) / chunk;
    p.nsplit = (int)ns;
    p.chunk = (int)chunk;
    const int64_t R = (int64_t)(K + 1) * (H / Hkv);
    if (ns > 1) {
        p.part_o_bytes = align_up((size_t)(B * Hkv * ns * R * kD) * sizeof(float), 256);
        p.part_ml_bytes = align_up((size_t)(B * Hkv * ns * R * 2) * sizeof(float), 256);
    }
    return p;
}

bool attn_shape_ok(int64_t B, int K, int H, int Hkv, int64_t S, int head_dim) {
    if (B < 0 || B > 65535 || K < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || S < 1) return false;
    if (head_dim != kD || S > ((int64_t)1 << 31)) return false;
    return (int64_t)(K + 1) * (H / Hkv) <= kMaxRows && Hkv <= 65535;
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_verify_attention_workspace_bytes(int64_t B, int K, int H, int Hkv, int64_t S) {
    if (!attn_shape_ok(B, K, H, Hkv, S, kD)) return 0;
    const AttnPlan p = attn_plan(B, K, H, Hkv, S);
    return p.part_o_bytes + p.part_ml_bytes;
}

extern "C" int spec_verify_attention(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* ctx_lens, const int32_t* draft_lens, int64_t B,
                                     int K, int H, int Hkv, int64_t S, int head_dim, float scale,
                                     void* out, int out_dtype, int32_t* out_status, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    if (!attn_shape_ok(B, K, H, Hkv, S, head_dim)) return SPEC_ERR_INVALID_ARG;
    if (out_dtype != SPEC_F32 && out_dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
    if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return SPEC_ERR_INVALID_ARG;
    if (B == 0) return SPEC_OK;
    if (!q || !k_cache || !v_cache || !ctx_lens || !out) return SPEC_ERR_INVALID_ARG;
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    if (!al16(q) || !al16(k_cache) || !al16(v_cache)) return SPEC_ERR_INVALID_ARG;
    const AttnPlan p = attn_plan(B, K, H, Hkv, S);
    const size_t need = p.part_o_bytes + p.part_ml_bytes;
    if (need > 0 && (!workspace || workspace_bytes < need || !al16(workspace))) return SPEC_ERR_WORKSPACE;
    AttnArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.kc = static_cast<const uint16_t*>(k_cache);
    a.vc = static_cast<const uint16_t*>(v_cache);
    a.ctx = ctx_lens;
    a.lens = draft_lens;
    a.out = out;
    a.status = out_status;
    a.B = B;
    a.S = S;
    a.K = K;
    a.H = H;
    a.Hkv = Hkv;
    a.G = H / Hkv;
    a.R = (K + 1) * a.G;
    a.nsplit = p.nsplit;
    a.chunk = p.chunk;
    a.out_bf16 = out_dtype == SPEC_BF16;
    a.c = (float)((double)scale * 1.4426950408889634074);
    if (need > 0) {
        a.part_o = static_cast<float*>(workspace);
        a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.part_o_bytes);
    }
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)p.nsplit, (unsigned)Hkv, (unsigned)B);
    if (a.R <= 16) hipLaunchKernelGGL(k_attn<1>, grid, dim3(attn_waves<1>() * kWave), 0, st, a);
    else hipLaunchKernelGGL(k_attn<2>, grid, dim3(attn_waves<2>() * kWave), 0, st, a);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    if (p.nsplit > 1) {
        const int ng = std::min(kCGroups, (p.nsplit + kCBatch - 1) / kCBatch);
        hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)a.R, (unsigned)Hkv, (unsigned)B),
                           dim3(ng * kD), 0, st, a);
        if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    }
    return SPEC_OK;
}
