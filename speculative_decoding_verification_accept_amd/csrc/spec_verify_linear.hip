// spec_verify_linear.hip -- verify linear layer Y[M, N] = X[M, K] W[K, N] on
// gfx950 bf16 MFMA with fp32 accumulation.
//
// Method: page "New technical post reveals how speculative decoding
// accelerates LLM inference without hurting accuracy" (agentnet.co.il),
// sections "The formula behind the speedup" and "GEMM-M grows, a small batch
// suffices": verifying D drafts turns every linear layer of the target from
// M = B rows into M = B(1+D) rows; weights are read once per pass whatever M
// is, so the layer stays memory-bound until M reaches the machine's
// FLOP-per-byte ridge.
//
// Kernel k_skinny: the product is computed transposed, Y^T = W^T X^T, on
// v_mfma_f32_16x16x32_bf16.  W is stored input-major ([K, N], N contiguous)
// while an MFMA operand wants 8 consecutive k per lane, so each lane loads an
// 8(k) x 8(n) block of W with eight 16-byte row loads (16 lanes cover 256
// contiguous bytes of a row: coalesced) and transposes it in registers with
// v_perm_b32 into the A operands of eight MFMAs whose 16 output rows are the
// strided columns n = nb + 8 i + c.  X (K contiguous) is the B operand as
// stored.  W never goes through LDS; it streams from HBM exactly once per
// m-tile.  Each wave covers 128 columns x 16*MT rows over a slice of K; the
// four waves of a workgroup split K further and are reduced through LDS;
// optional split-K across workgroups writes fp32 partials that the last
// workgroup of a tile (integer atomic counter) sums in a fixed order.
#include "spec_verify.h"
#include "device_common.hpp"

namespace specv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kNT = 128;  // columns per wave tile
constexpr int kKS = 32;   // k per MFMA step
constexpr int kSkinnyWaves = 4;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Column c (0..7) of an 8x8 bf16 block held as 8 row vectors r[0..7]
// (row = k, 8 bf16 columns per uint4) -> 8 k values of that column.
template <int C>
__device__ __forceinline__ uint4 column_of(const uint4 (&r)[8]) {
    constexpr uint32_t sel = (C & 1) ? 0x07060302u : 0x05040100u;
    auto dw = [](const uint4& v) -> uint32_t {
        if constexpr (C / 2 == 0) return v.x;
        else if constexpr (C / 2 == 1) return v.y;
        else if constexpr (C / 2 == 2) return v.z;
        else return v.w;
    };
    uint4 o;
    o.x = __builtin_amdgcn_perm(dw(r[1]), dw(r[0]), sel);
    o.y = __builtin_amdgcn_perm(dw(r[3]), dw(r[2]), sel);
    o.z = __builtin_amdgcn_perm(dw(r[5]), dw(r[4]), sel);
    o.w = __builtin_amdgcn_perm(dw(r[7]), dw(r[6]), sel);
    return o;
}

template <int MT>
struct SkinnyAcc {
    f32x4_t a[8][MT];
};

template <int MT>
__device__ __forceinline__ void skinny_load(const uint16_t* __restrict__ X,
                                            const uint16_t* __restrict__ W, int64_t M, int64_t N,
                                            int64_t K, int64_t m0, int64_t nb, int64_t k0, int lane,
                                            uint4 (&w)[8], uint4 (&x)[MT]) {
    const int kg = lane >> 4;      // k group of 8
    const int li = lane & 15;
    const int64_t ncol = nb + 8 * li;
    const bool nok = ncol < N;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int64_t k = k0 + 8 * kg + r;
        w[r] = (nok && k < K) ? *reinterpret_cast<const uint4*>(W + k * N + ncol)
                              : make_uint4(0u, 0u, 0u, 0u);
    }
    const int64_t kx = k0 + 8 * kg;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = m0 + 16 * mt + li;
        x[mt] = (m < M && kx < K) ? *reinterpret_cast<const uint4*>(X + m * K + kx)
                                  : make_uint4(0u, 0u, 0u, 0u);
    }
}

template <int MT>
__device__ __forceinline__ void skinny_mma(const uint4 (&w)[8], const uint4 (&x)[MT],
                                           SkinnyAcc<MT>& acc) {
    uint4 col[8];
    col[0] = column_of<0>(w); col[1] = column_of<1>(w);
    col[2] = column_of<2>(w); col[3] = column_of<3>(w);
    col[4] = column_of<4>(w); col[5] = column_of<5>(w);
    col[6] = column_of<6>(w); col[7] = column_of<7>(w);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            acc.a[c][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(col[c]),
                                                                   as_bf16x8(x[mt]),
                                                                   acc.a[c][mt], 0, 0, 0);
}

// Output element of accumulator (c, mt, r) at lane l:
//   n = nb + 8 * (4 * (l / 16) + r) + c,  m = m0 + 16 * mt + l % 16.
// For fixed (mt, r) the eight c values are 8 consecutive columns.
template <int MT>
__global__ __launch_bounds__(kSkinnyWaves * kWave) void k_skinny(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y,
    int y_bf16, int64_t M, int64_t N, int64_t K, int splits, float* __restrict__ partial,
    int32_t* __restrict__ counters) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // m-tiles sharing a column strip are adjacent in launch order, so their
    // re-reads of that strip of W hit in cache
    const int64_t mtile = blockIdx.x;
    const int64_t ntile = blockIdx.y;
    const int split = blockIdx.z;
    const int64_t nb = ntile * kNT;
    const int64_t m0 = mtile * (16 * MT);

    const int64_t nsteps = (K + kKS - 1) / kKS;
    const int64_t g = (int64_t)split * kSkinnyWaves + wave;
    const int64_t gtot = (int64_t)splits * kSkinnyWaves;
    const int64_t s0 = g * nsteps / gtot, s1 = (g + 1) * nsteps / gtot;

    SkinnyAcc<MT> acc;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc.a[c][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if (s0 < s1) {
        uint4 w0[8], x0[MT];
        skinny_load<MT>(X, W, M, N, K, m0, nb, s0 * kKS, lane, w0, x0);
        for (int64_t s = s0; s < s1; ++s) {
            uint4 w1[8], x1[MT];
            const bool more = s + 1 < s1;
            if (more) skinny_load<MT>(X, W, M, N, K, m0, nb, (s + 1) * kKS, lane, w1, x1);
            skinny_mma<MT>(w0, x0, acc);
            if (more) {
#pragma unroll
                for (int r = 0; r < 8; ++r) w0[r] = w1[r];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) x0[mt] = x1[mt];
            }
        }
    }

    // reduce the four waves' k-slices through LDS, one 16-row block at a
    // time (fixed order: wave 0 + 1 + 2 + 3)
    __shared__ float lds[(kSkinnyWaves - 1) * 64 * 32];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        if (wave > 0) {
            float* dst = lds + ((wave - 1) * 64 + lane) * 32;
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[c * 4 + r] = acc.a[c][mt][r];
        }
        __syncthreads();
        if (wave == 0) {
            for (int wv = 1; wv < kSkinnyWaves; ++wv) {
                const float* src = lds + ((wv - 1) * 64 + lane) * 32;
#pragma unroll
                for (int c = 0; c < 8; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc.a[c][mt][r] += src[c * 4 + r];
            }
        }
        __syncthreads();
    }
    if (wave != 0) return;

    const int li = lane & 15;
    const int kg = lane >> 4;
    if (splits > 1) {
        // write this split's fp32 partial tile, then the last workgroup of the
        // tile sums all splits in order
        const int64_t Mp = (int64_t)gridDim.x * 16 * MT;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + 16 * mt + li;
                const int64_t n = nb + 8 * (4 * kg + r);
                if (m < M && n < N) {
                    float* p = partial + ((int64_t)split * Mp + m) * N + n;
                    const f32x4_t lo = {acc.a[0][mt][r], acc.a[1][mt][r], acc.a[2][mt][r], acc.a[3][mt][r]};
                    const f32x4_t hi = {acc.a[4][mt][r], acc.a[5][mt][r], acc.a[6][mt][r], acc.a[7][mt][r]};
                    __builtin_nontemporal_store(lo, reinterpret_cast<f32x4_t*>(p));
                    __builtin_nontemporal_store(hi, reinterpret_cast<f32x4_t*>(p + 4));
                }
            }
        __threadfence();
        int last = 0;
        if (lane == 0) {
            const int old = atomicAdd(&counters[ntile * gridDim.x + mtile], 1);
            last = (old == splits - 1);
        }
        last = __shfl(last, 0, kWave);
        if (!last) return;
        __threadfence();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc.a[c][mt][r] = 0.f;
        for (int sp = 0; sp < splits; ++sp) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t m = m0 + 16 * mt + li;
                    const int64_t n = nb + 8 * (4 * kg + r);
                    if (m < M && n < N) {
                        const float* p = partial + ((int64_t)sp * Mp + m) * N + n;
                        const f32x4_t lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
                        const f32x4_t hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + 4));
                        acc.a[0][mt][r] += lo[0]; acc.a[1][mt][r] += lo[1];
                        acc.a[2][mt][r] += lo[2]; acc.a[3][mt][r] += lo[3];
                        acc.a[4][mt][r] += hi[0]; acc.a[5][mt][r] += hi[1];
                        acc.a[6][mt][r] += hi[2]; acc.a[7][mt][r] += hi[3];
                    }
                }
        }
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + 16 * mt + li;
            const int64_t n = nb + 8 * (4 * kg + r);
            if (m >= M || n >= N) continue;
            if (y_bf16) {
                uint4 o;
                o.x = (uint32_t)f32_to_bf16(acc.a[0][mt][r]) | ((uint32_t)f32_to_bf16(acc.a[1][mt][r]) << 16);
                o.y = (uint32_t)f32_to_bf16(acc.a[2][mt][r]) | ((uint32_t)f32_to_bf16(acc.a[3][mt][r]) << 16);
                o.z = (uint32_t)f32_to_bf16(acc.a[4][mt][r]) | ((uint32_t)f32_to_bf16(acc.a[5][mt][r]) << 16);
                o.w = (uint32_t)f32_to_bf16(acc.a[6][mt][r]) | ((uint32_t)f32_to_bf16(acc.a[7][mt][r]) << 16);
                *reinterpret_cast<uint4*>(static_cast<uint16_t*>(Y) + m * N + n) = o;
            } else {
                float* p = static_cast<float*>(Y) + m * N + n;
                *reinterpret_cast<float4*>(p) = make_float4(acc.a[0][mt][r], acc.a[1][mt][r], acc.a[2][mt][r], acc.a[3][mt][r]);
                *reinterpret_cast<float4*>(p + 4) = make_float4(acc.a[4][mt][r], acc.a[5][mt][r], acc.a[6][mt][r], acc.a[7][mt][r]);
            }
        }
}

__global__ void k_zero_i32(int32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// ---- launch plan ----------------------------------------------------------------
struct SkinnyPlan {
    int mt;          // 16-row blocks per wave tile (1, 2 or 4)
    int64_t ntiles, mtiles;
    int splits;
    size_t partial_bytes, counter_bytes;
};

SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K) {
    SkinnyPlan p;
    p.mt = (M <= 16) ? 1 : (M <= 32) ? 2 : 4;
    p.ntiles = (N + kNT - 1) / kNT;
    p.mtiles = (M + 16 * p.mt - 1) / (16 * p.mt);
    const int64_t nsteps = (K + kKS - 1) / kKS;
    const int64_t tiles = p.ntiles * p.mtiles;
    int64_t s = (1024 + tiles - 1) / tiles;                 // aim for >= 1024 workgroups
    s = s < 1 ? 1 : s;
    const int64_t smax = nsteps / (2 * kSkinnyWaves);       // >= 2 MFMA steps per wave
    if (s > smax) s = smax < 1 ? 1 : smax;
    if (s > 32) s = 32;
    p.splits = (int)s;
    const int64_t Mp = p.mtiles * 16 * p.mt;
    p.partial_bytes = p.splits > 1 ? align_up((size_t)p.splits * Mp * N * sizeof(float), 256) : 0;
    p.counter_bytes = p.splits > 1 ? align_up((size_t)tiles * sizeof(int32_t), 256) : 0;
    return p;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_verify_linear_workspace_bytes(int64_t M, int64_t N, int64_t Kd) {
    if (M <= 0 || N <= 0 || Kd <= 0) return 0;
    const SkinnyPlan p = plan_skinny(M, N, Kd);
    return p.partial_bytes + p.counter_bytes;
}

extern "C" int spec_verify_linear(const void* X, const void* W, void* Y, int y_dtype, int64_t M,
                                  int64_t N, int64_t Kd, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    if (M < 0 || N < 1 || Kd < 1 || (N % 8) != 0 || (Kd % 8) != 0) return SPEC_ERR_INVALID_ARG;
    if (y_dtype != SPEC_F32 && y_dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
    if (M == 0) return SPEC_OK;
    if (!X || !W || !Y || !aligned16(X) || !aligned16(W) || !aligned16(Y)) return SPEC_ERR_INVALID_ARG;
    const SkinnyPlan p = plan_skinny(M, N, Kd);
    if (p.ntiles > 65535 || p.mtiles > 0x7FFFFFFF) return SPEC_ERR_INVALID_ARG;
    const size_t need = p.partial_bytes + p.counter_bytes;
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return SPEC_ERR_WORKSPACE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    float* partial = need ? static_cast<float*>(workspace) : nullptr;
    int32_t* counters = need ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + p.partial_bytes) : nullptr;
    if (counters) {
        // tile counters start at zero (a fill kernel, not a memset node, so
        // that the call can be captured in a HIP graph)
        const int64_t n = p.ntiles * p.mtiles;
        hipLaunchKernelGGL(k_zero_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, counters, n);
        if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    }
    const dim3 grid((unsigned)p.mtiles, (unsigned)p.ntiles, (unsigned)p.splits);
    const dim3 block(kSkinnyWaves * kWave);
    const size_t lds = 0;
    const uint16_t* x = static_cast<const uint16_t*>(X);
    const uint16_t* w = static_cast<const uint16_t*>(W);
    const int yb = y_dtype == SPEC_BF16;
    switch (p.mt) {
        case 1: hipLaunchKernelGGL(k_skinny<1>, grid, block, lds, s, x, w, Y, yb, M, N, Kd, p.splits, partial, counters); break;
        case 2: hipLaunchKernelGGL(k_skinny<2>, grid, block, lds, s, x, w, Y, yb, M, N, Kd, p.splits, partial, counters); break;
        default: hipLaunchKernelGGL(k_skinny<4>, grid, block, lds, s, x, w, Y, yb, M, N, Kd, p.splits, partial, counters); break;
    }
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    return SPEC_OK;
}
