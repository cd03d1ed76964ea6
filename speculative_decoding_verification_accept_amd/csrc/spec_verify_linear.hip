// spec_verify_linear.hip -- verify linear layer Y[M, N] = X[M, K] W[K, N] on
// gfx950 bf16 MFMA with fp32 accumulation.
//
// Method: page "New technical post reveals how speculative decoding
// accelerates LLM inference without hurting accuracy" (agentnet.co.il),
// sections "The formula behind the speedup" and "GEMM-M grows, a small batch
// suffices": verifying D drafts turns every linear layer of the target from
// M = B rows into M = B(1+D) rows.  The weights are read once per pass
// whatever M is, so the layer stays memory-bound until M reaches the
// machine's FLOP-per-byte ridge (about 315 on MI355X), then turns
// compute-bound.
//
// W is stored input-major ([K, N], N contiguous) while an MFMA operand wants
// 8 consecutive k per lane; X (K contiguous) is used as stored.  The MFMA
// computes D = A B with A an X fragment and B a W fragment.
//
//  k_strip (M <= 32 when K is not a multiple of 64; memory-bound):
//    one 512-thread workgroup per 64-column
//    strip of W, all M rows, the full K.  Each of its 8 waves takes a slice
//    of K, keeps 4 k-steps of W loads in flight, transposes each lane's 8x4
//    block of W in registers (v_perm_b32) straight into
//    v_mfma_f32_16x16x32_bf16 operands, and the waves' partial tiles are
//    summed through LDS in a fixed order.  W streams from HBM exactly once.
//  k_dma (K a multiple of 64, or of 32 past 32 rows; v_mfma_f32_32x32x16_bf16):
//    a workgroup computes a BM x BN tile; BM is 32 or 64 for a few rows, so
//    that the X rows streamed per W byte stay few.  Tiles of X and W go from HBM
//    straight into an LDS ring of 4-5 stages by loads that write LDS, so the
//    prefetch distance costs no registers; W stays [k][n] in LDS and the
//    transposing LDS read ds_read_b64_tr_b16 builds its MFMA operands.
//    With 129-192 rows and at least 512 columns per compute unit (the
//    lm-head), whole rounds of 192 x 512 tiles (16 waves, a 3-stage ring:
//    half the X bytes per W byte of 192 x 256, 6% faster on the lm-head),
//    then the remaining columns as 192 x 256 tiles.
//  k_tile (other K): the earlier design, W staged through registers and
//    transposed with v_perm_b32 on its way into LDS.
// Split-K (when the tiles alone fill less than half the machine) writes fp32
// partials that k_reduce sums in a fixed order (no atomics).
#include "spec_verify.h"
#include "device_common.hpp"

#include <atomic>
#include <utility>

namespace specv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKS = 32;  // k per MFMA

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// 32x32x16: A lane l = rows l % 32, k 8 (l / 32) .. +7; B likewise by column;
// D register j of lane l = row 8 (j / 4) + 4 (l / 32) + j % 4, column l % 32.
__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// 8 consecutive k of column C from 8 rows (row r = k) whose dword D holds
// columns 2D (low half) and 2D+1 (high half).
template <int C, typename Row>
__device__ __forceinline__ uint4 column_of(const Row (&r)[8]) {
    constexpr uint32_t sel = (C & 1) ? 0x07060302u : 0x05040100u;
    auto dw = [](const Row& v) -> uint32_t {
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

__device__ __forceinline__ void store_out(void* Y, int y_bf16, int64_t idx, f32x4_t v) {
    if (y_bf16) {
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Y) + idx) = o;
    } else {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(Y) + idx) = v;
    }
}

// ---------------------------------------------------------------------------
// k_strip
// Lane l of a wave: li = l % 16 owns columns n0 + 4 li .. +3, kg = l / 16 the
// k rows 8 kg .. 8 kg + 7 of each 32-k step.  MFMA c (c = 0..3) takes as B
// the column n0 + 4 j + c of lane j's block, so accumulator (c, mt) of lane l
// holds Y[m0 + 16 mt + 4 (l / 16) + r][n0 + 4 (l % 16) + c], r = 0..3.
constexpr int kStripN = 64;
constexpr int kStripWaves = 8;
constexpr int kStripDepth = 4;  // k-steps of W loads in flight per wave

template <int MT>
struct StripStage {
    uint2 w[8];
    uint4 x[MT];
};

template <int MT>
__device__ __forceinline__ void strip_load(const uint16_t* __restrict__ X,
                                           const uint16_t* __restrict__ W, int64_t M, int64_t N,
                                           int64_t K, int64_t m0, int64_t n0, int64_t s, int lane,
                                           StripStage<MT>& st) {
    const int kg = lane >> 4, li = lane & 15;
    const int64_t ncol = n0 + 4 * li;
    const int64_t k8 = s * kKS + 8 * kg;  // first of this lane's 8 k (all < K or none, K % 8 == 0)
    const bool wok = ncol < N && k8 < K;
    const uint16_t* wp = W + k8 * N + ncol;
#pragma unroll
    for (int r = 0; r < 8; ++r)
        st.w[r] = wok ? *reinterpret_cast<const uint2*>(wp + (int64_t)r * N) : make_uint2(0u, 0u);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = m0 + 16 * mt + li;
        st.x[mt] = (m < M && k8 < K) ? *reinterpret_cast<const uint4*>(X + m * K + k8)
                                     : make_uint4(0u, 0u, 0u, 0u);
    }
}

template <int MT>
__device__ __forceinline__ void strip_mma(const StripStage<MT>& st, f32x4_t (&acc)[4][MT]) {
    const uint4 c0 = column_of<0>(st.w), c1 = column_of<1>(st.w);
    const uint4 c2 = column_of<2>(st.w), c3 = column_of<3>(st.w);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        acc[0][mt] = mfma(st.x[mt], c0, acc[0][mt]);
        acc[1][mt] = mfma(st.x[mt], c1, acc[1][mt]);
        acc[2][mt] = mfma(st.x[mt], c2, acc[2][mt]);
        acc[3][mt] = mfma(st.x[mt], c3, acc[3][mt]);
    }
}

template <int MT>
__global__ __launch_bounds__(kStripWaves * kWave) void k_strip(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y,
    int y_bf16, int64_t M, int64_t N, int64_t K) {
    __shared__ f32x4_t red[(kStripWaves - 1) * kWave * 4];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t m0 = (int64_t)blockIdx.x * 16 * MT;   // m-tiles of a strip are adjacent
    const int64_t n0 = (int64_t)blockIdx.y * kStripN;
    const int64_t nsteps = (K + kKS - 1) / kKS;
    const int64_t s0 = wave * nsteps / kStripWaves, s1 = (wave + 1) * nsteps / kStripWaves;

    f32x4_t acc[4][MT];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[c][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    StripStage<MT> buf[kStripDepth];
#pragma unroll
    for (int d = 0; d < kStripDepth; ++d)
        if (s0 + d < s1) strip_load<MT>(X, W, M, N, K, m0, n0, s0 + d, lane, buf[d]);
    for (int64_t base = s0; base < s1; base += kStripDepth) {
#pragma unroll
        for (int d = 0; d < kStripDepth; ++d) {
            const int64_t s = base + d;
            if (s < s1) {
                strip_mma<MT>(buf[d], acc);
                if (s + kStripDepth < s1)
                    strip_load<MT>(X, W, M, N, K, m0, n0, s + kStripDepth, lane, buf[d]);
            }
        }
    }

    // fixed-order sum of the 8 waves' k-slices, one 16-row block at a time
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        if (wave > 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c) red[((wave - 1) * kWave + lane) * 4 + c] = acc[c][mt];
        }
        __syncthreads();
        if (wave == 0) {
            for (int wv = 1; wv < kStripWaves; ++wv)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c][mt] += red[((wv - 1) * kWave + lane) * 4 + c];
        }
        __syncthreads();
    }
    if (wave != 0) return;
    const int li = lane & 15, kg = lane >> 4;
    const int64_t n = n0 + 4 * li;
    if (n >= N) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + 16 * mt + 4 * kg + r;
            if (m < M)
                store_out(Y, y_bf16, m * N + n,
                          f32x4_t{acc[0][mt][r], acc[1][mt][r], acc[2][mt][r], acc[3][mt][r]});
        }
}

// ---------------------------------------------------------------------------
// k_tile (v_mfma_f32_32x32x16_bf16: the 16x16x32 shape issues at half its
// rate on gfx950)
// LDS tiles (bf16, rows padded by 8 elements against bank conflicts):
//   Ws[n][k]  BN x (BK + 8): W transposed, 8 consecutive k per 16 bytes
//   Xs[m][k]  BM x (BK + 8)
// Wave (wm, wn) computes rows wm*WM .. +WM and columns wn*WN .. +WN of the
// tile: FM = WM/32 X fragments and FN = WN/32 W fragments per 16-k step.
// Register j of accumulator (fm, fn) of lane l holds
//   Y[m = 32 fm + 8 (j / 4) + 4 (l / 32) + j % 4][n = 32 fn + l % 32].
template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NWM = BM / WM, NWN = BN / WN;
    static constexpr int NT = NWM * NWN * kWave;
    static constexpr int FM = WM / 32, FN = WN / 32;  // 32x32 output blocks per wave
    static constexpr int LDK = BK + 8;
    static constexpr int WBLK_TOTAL = (BK / 8) * (BN / 8);       // 8x8 blocks of W per stage
    static constexpr int WBLK = (WBLK_TOTAL + NT - 1) / NT;      // per thread
    static constexpr int XV_TOTAL = BM * BK / 8;                 // 16-byte vectors of X per stage
    static constexpr int XV = (XV_TOTAL + NT - 1) / NT;
    static constexpr size_t LDS = (size_t)(BN + BM) * LDK * 2;
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile");
    static_assert(BK == 64, "the LDS swizzle assumes 8 groups of 8 k per row");
    static_assert(BN % 128 == 0, "the LDS swizzle assumes 16 column blocks per k-block row");
};

// Physical 16-byte k-group of logical group G in W row n of the LDS tile:
// G ^ ((n >> 4) & 7).  With the 72-element row pitch (36 banks), both the
// transposed stores (16 lanes: rows 8 nb + c, nb = 0..15) and the MFMA
// fragment reads (16 lanes: 16 consecutive rows) then touch 16 disjoint
// 4-bank ranges.
__device__ __forceinline__ int w_group(int G, int n_over_16) { return G ^ (n_over_16 & 7); }

template <typename Cfg>
struct TileRegs {
    uint4 w[Cfg::WBLK][8];
    uint4 x[Cfg::XV];
};

// Loop-invariant per-thread addressing of k_tile.  Global loads are buffer
// loads whose whole byte offset is the per-lane offset: the hardware's range
// check covers that offset and not the scalar one, so an element outside the
// matrix (a column past N, a row past M, a k past K) gets the offset kOOB,
// past the buffer's end, and reads as zero.  The host routes a matrix of
// 2 GiB or more elsewhere, so every in-range offset is below kOOB.
template <typename Cfg>
struct TileAddr {
    __amdgpu_buffer_rsrc_t wr, xr;
    uint32_t wv[Cfg::WBLK];   // W block (8 rows) byte offset at stage 0, row 0 (kOOB past N)
    uint32_t wk[Cfg::WBLK];   // k of the block's row 0 within a stage
    uint32_t xv[Cfg::XV];     // X vector byte offset at stage 0 (kOOB past M)
    uint32_t wlds[Cfg::WBLK]; // LDS byte offset of the block's column 0 (within the W tile)
    uint32_t xlds[Cfg::XV];   // LDS byte offset of the X vector (within the X tile)
    uint32_t row_bytes;       // N * 2
    uint32_t x_kok[Cfg::XV];  // k offset (elements) of the X vector within a stage
};

constexpr uint32_t kOOB = 0x80000000u;  // offset past any buffer below 2 GiB

template <typename Cfg>
__device__ __forceinline__ void tile_addr(const uint16_t* X, const uint16_t* W, int64_t M, int64_t N,
                                          int64_t K, int64_t m0, int64_t n0, int tid,
                                          TileAddr<Cfg>& A) {
    const uint64_t wbytes = (uint64_t)K * N * 2, xbytes = (uint64_t)M * K * 2;
    A.wr = __builtin_amdgcn_make_buffer_rsrc((void*)W, (short)0, (int)(wbytes < kOOB ? wbytes : kOOB - 1), 0x00020000);
    A.xr = __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, (int)(xbytes < kOOB ? xbytes : kOOB - 1), 0x00020000);
    A.row_bytes = (uint32_t)(N * 2);
#pragma unroll
    for (int j = 0; j < Cfg::WBLK; ++j) {
        const int q = tid + j * Cfg::NT;
        const int kb = q / (Cfg::BN / 8), nb = q % (Cfg::BN / 8);
        const int64_t n = n0 + 8 * nb;
        A.wv[j] = (q < Cfg::WBLK_TOTAL && n < N) ? (uint32_t)(((int64_t)8 * kb * N + n) * 2) : kOOB;
        A.wk[j] = (uint32_t)(8 * kb);
        // rows 8 nb .. 8 nb + 7 of the transposed tile share the swizzle (n >> 4) = nb >> 1
        A.wlds[j] = (uint32_t)((8 * nb) * Cfg::LDK * 2 + 16 * w_group(kb, nb >> 1));
    }
#pragma unroll
    for (int j = 0; j < Cfg::XV; ++j) {
        const int v = tid + j * Cfg::NT;
        const int mm = v / (Cfg::BK / 8), kv = v % (Cfg::BK / 8);
        const int64_t m = m0 + mm;
        A.xv[j] = (v < Cfg::XV_TOTAL && m < M) ? (uint32_t)((m * K + 8 * kv) * 2) : kOOB;
        A.xlds[j] = (uint32_t)(mm * Cfg::LDK * 2 + 16 * kv);
        A.x_kok[j] = 8 * kv;
    }
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Global loads of the stage starting at k0.  W rows and X vectors past K
// (only when the stage crosses K, K being a multiple of 8) get the offset
// kOOB and read as zero; no scalar offset is used.
template <typename Cfg>
__device__ __forceinline__ void tile_load(const TileAddr<Cfg>& A, int64_t K, int64_t k0,
                                          TileRegs<Cfg>& R) {
    const uint32_t wst = (uint32_t)(k0 * A.row_bytes);
    const bool tail = k0 + Cfg::BK > K;
#pragma unroll
    for (int j = 0; j < Cfg::WBLK; ++j) {
        // a block's 8 rows are all below K or all at or past it
        const bool wout = A.wv[j] == kOOB || (tail && k0 + A.wk[j] >= K);
#pragma unroll
        for (int r = 0; r < 8; ++r) R.w[j][r] = bload(A.wr, wout ? kOOB : A.wv[j] + wst + r * A.row_bytes, 0u);
    }
#pragma unroll
    for (int j = 0; j < Cfg::XV; ++j) {
        const bool xout = A.xv[j] == kOOB || (tail && k0 + A.x_kok[j] >= K);
        R.x[j] = bload(A.xr, xout ? kOOB : A.xv[j] + (uint32_t)(k0 * 2), 0u);
    }
}

template <typename Cfg>
__device__ __forceinline__ void tile_store(const TileRegs<Cfg>& R, const TileAddr<Cfg>& A,
                                           char* Ws, char* Xs, int tid) {
#pragma unroll
    for (int j = 0; j < Cfg::WBLK; ++j) {
        if (Cfg::WBLK_TOTAL % Cfg::NT != 0 && tid + j * Cfg::NT >= Cfg::WBLK_TOTAL) continue;
        char* base = Ws + A.wlds[j];
        *reinterpret_cast<uint4*>(base + 0 * Cfg::LDK * 2) = column_of<0>(R.w[j]);
        *reinterpret_cast<uint4*>(base + 1 * Cfg::LDK * 2) = column_of<1>(R.w[j]);
        *reinterpret_cast<uint4*>(base + 2 * Cfg::LDK * 2) = column_of<2>(R.w[j]);
        *reinterpret_cast<uint4*>(base + 3 * Cfg::LDK * 2) = column_of<3>(R.w[j]);
        *reinterpret_cast<uint4*>(base + 4 * Cfg::LDK * 2) = column_of<4>(R.w[j]);
        *reinterpret_cast<uint4*>(base + 5 * Cfg::LDK * 2) = column_of<5>(R.w[j]);
        *reinterpret_cast<uint4*>(base + 6 * Cfg::LDK * 2) = column_of<6>(R.w[j]);
        *reinterpret_cast<uint4*>(base + 7 * Cfg::LDK * 2) = column_of<7>(R.w[j]);
    }
#pragma unroll
    for (int j = 0; j < Cfg::XV; ++j) {
        if (Cfg::XV_TOTAL % Cfg::NT != 0 && tid + j * Cfg::NT >= Cfg::XV_TOTAL) continue;
        *reinterpret_cast<uint4*>(Xs + A.xlds[j]) = R.x[j];
    }
}

// MFMAs of one stage.  abase: byte offset of this lane's first X fragment
// row; brow[fn]: byte offset of this lane's W row of fragment fn; bsw[fn]: its
// swizzle (n >> 4) & 7.
template <typename Cfg>
__device__ __forceinline__ void tile_compute(const char* Ws, const char* Xs, uint32_t abase,
                                             const uint32_t (&brow)[Cfg::FN], const int (&bsw)[Cfg::FN],
                                             int g, f32x16_t (&acc)[Cfg::FM][Cfg::FN]) {
#pragma unroll
    for (int k16 = 0; k16 < Cfg::BK / 16; ++k16) {
        uint4 a[Cfg::FM], b[Cfg::FN];
#pragma unroll
        for (int fm = 0; fm < Cfg::FM; ++fm)
            a[fm] = *reinterpret_cast<const uint4*>(Xs + abase + fm * 32 * Cfg::LDK * 2 + k16 * 32);
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn)
            b[fn] = *reinterpret_cast<const uint4*>(Ws + brow[fn] + 16 * ((2 * k16 + g) ^ bsw[fn]));
#pragma unroll
        for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < Cfg::FN; ++fn) acc[fm][fn] = mfma32(a[fm], b[fn], acc[fm][fn]);
    }
}

// D register slots of global loads in flight and two LDS buffers.  Iteration
// st: issue the global loads of stage st + D, multiply stage st out of one
// LDS buffer, write stage st + 1 into the other, one barrier.
template <typename Cfg, int D>
__global__ __launch_bounds__(Cfg::NT) void k_tile(const uint16_t* __restrict__ X,
                                                  const uint16_t* __restrict__ W,
                                                  void* __restrict__ Y, int y_bf16, int64_t M,
                                                  int64_t N, int64_t K, int splits,
                                                  float* __restrict__ partial) {
    static_assert(D % 2 == 0, "the LDS buffer of a stage is fixed by its slot");
    extern __shared__ __align__(16) char lds[];
    constexpr int STAGE = (Cfg::BN + Cfg::BM) * Cfg::LDK * 2;  // bytes
    constexpr int XOFF = Cfg::BN * Cfg::LDK * 2;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave / Cfg::NWN, wn = wave % Cfg::NWN;
    const int64_t m0 = (int64_t)blockIdx.x * Cfg::BM;  // m-tiles of a column strip are adjacent
    const int64_t n0 = (int64_t)blockIdx.y * Cfg::BN;
    const int split = blockIdx.z;
    const int64_t nst = (K + Cfg::BK - 1) / Cfg::BK;
    const int64_t st0 = split * nst / splits, st1 = (split + 1) * nst / splits;

    TileAddr<Cfg> A;
    tile_addr<Cfg>(X, W, M, N, K, m0, n0, tid, A);
    const int l32 = lane & 31, g = lane >> 5;
    const uint32_t abase = (uint32_t)((wm * Cfg::WM + l32) * Cfg::LDK * 2 + 16 * g);
    uint32_t brow[Cfg::FN];
    int bsw[Cfg::FN];
#pragma unroll
    for (int fn = 0; fn < Cfg::FN; ++fn) {
        const int n = wn * Cfg::WN + 32 * fn + l32;
        brow[fn] = (uint32_t)(n * Cfg::LDK * 2);
        bsw[fn] = (n >> 4) & 7;
    }

    f32x16_t acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int a = 0; a < Cfg::FM; ++a)
#pragma unroll
        for (int b = 0; b < Cfg::FN; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.f;

    TileRegs<Cfg> R[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (st0 + d < st1) tile_load<Cfg>(A, K, (st0 + d) * Cfg::BK, R[d]);
    if (st0 < st1) tile_store<Cfg>(R[0], A, lds, lds + XOFF, tid);
    __syncthreads();
    for (int64_t base = st0; base < st1; base += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t st = base + d;
            if (st < st1) {
                // slot d held stage st, already in LDS: refill it with stage st + D
                if (st + D < st1) tile_load<Cfg>(A, K, (st + D) * Cfg::BK, R[d]);
                const char* cur = lds + (d % 2) * STAGE;
                tile_compute<Cfg>(cur, cur + XOFF, abase, brow, bsw, g, acc);
                if (st + 1 < st1) {
                    char* nxt = lds + ((d + 1) % 2) * STAGE;
                    tile_store<Cfg>(R[(d + 1) % D], A, nxt, nxt + XOFF, tid);
                }
                __syncthreads();
            }
        }
    }

    float* dstp = splits > 1 ? partial + (int64_t)split * M * N : nullptr;
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn) {
            const int64_t n = n0 + wn * Cfg::WN + 32 * fn + l32;
            if (n >= N) continue;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int64_t m = m0 + wm * Cfg::WM + 32 * fm + 8 * (j / 4) + 4 * g + (j % 4);
                if (m >= M) continue;
                const float v = acc[fm][fn][j];
                if (dstp) dstp[m * N + n] = v;
                else if (y_bf16) static_cast<uint16_t*>(Y)[m * N + n] = f32_to_bf16(v);
                else static_cast<float*>(Y)[m * N + n] = v;
            }
        }
}


// ---------------------------------------------------------------------------
// k_dma (v_mfma_f32_32x32x16_bf16).  Tiles of X and W go from HBM straight
// into an S-stage LDS ring through buffer loads that write LDS (no register
// staging), S - 1 stages ahead of the MFMAs, so the prefetch distance is
// bounded by LDS capacity rather than by registers.  W stays as stored
// ([k][n], n contiguous): ds_read_b64_tr_b16 gives each lane four
// consecutive k of one column, and two such reads make an MFMA B operand.
// X fragments are plain 16-byte LDS reads.  Both tiles are XOR-swizzled in
// 16-byte groups -- a load's lanes fetch the global groups that the
// permutation places at their LDS slots -- so fragment reads hit distinct
// banks.  K must be a multiple of BK.
//
// ds_read_b64_tr_b16, per group of 16 lanes: lane i receives element i % 4
// of the 8-byte segments addressed by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.
// Pointing lane s at row kb + s/4, columns nb + 4 (s % 4) .. +3 of the W tile
// gives lane i the four values W[kb .. kb+3][nb + i].
template <int BM_, int BN_, int BK_, int NWM_, int NWN_, int S_>
struct DmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, NWM = NWM_, NWN = NWN_, S = S_;
    static constexpr int NW = NWM * NWN, NT = NW * kWave;
    static constexpr int WM = BM / NWM, WN = BN / NWN;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int XBYTES = BM * BK * 2, WBYTES = BK * BN * 2;
    static constexpr int XI = XBYTES / 1024, WI = WBYTES / 1024;  // 1 KB loads per stage
    static constexpr int TI = XI + WI;
    static constexpr int LMAX = (TI + NW - 1) / NW, LMIN = TI / NW;  // loads per wave
    static constexpr int XG = BK / 8, WG = BN / 8;                    // 16-byte groups per row
    static constexpr int XROWS = 1024 / (BK * 2), WROWS = 1024 / (BN * 2);  // rows per load
    static constexpr size_t LDS = (size_t)S * (XBYTES + WBYTES);
    static_assert(BK == 32 || BK == 64, "X swizzle covers 4 or 8 groups per row");
    static_assert(BN == 128 || BN == 256 || BN == 512, "whole W rows per load; W swizzle over 16 groups");
    static_assert(XBYTES % 1024 == 0, "whole X rows per load");
    static_assert(WM % 32 == 0 && WN % 32 == 0 && BM % NWM == 0 && BN % NWN == 0, "wave tile");
    static_assert(S >= 2 && (S - 2) * LMIN < 64, "ring depth / vmcnt range");
    static_assert(LDS <= 160 * 1024, "LDS");
};

// Physical 16-byte group of logical group g in X row r (BK = 32: 4 groups of
// 64-byte rows; BK = 64: 8 groups of 128-byte rows), and in W row kr.
//
// LDS has 64 banks of 4 bytes.  A 16-lane pass of a 16-byte X read covers 16
// rows of one logical group: the XOR spreads them over all 16 slots of 256
// bytes.  A 32-lane pass of a transposed W read covers rows kr .. kr + 3 and
// 4 logical groups 4q .. 4q + 3 (two lanes per group): W rows are a multiple
// of 256 bytes (BN >= 128), so every row starts on bank 0, and XOR-ing the
// group with 4 (kr & 3) gives each row its own 64 bytes of the 256.
template <int XG>
__device__ __forceinline__ int x_group(int g, int r) {
    return XG == 4 ? (g ^ ((r >> 2) & 3)) : (g ^ ((r >> 1) & 7));
}
__device__ __forceinline__ int w_group_tr(int g, int kr) { return g ^ (4 * (kr & 3)); }

// The LDS ring of S stage slots.  The loads that fill it are opaque to the
// compiler (inline assembly with a memory clobber), so it neither waits for
// them nor reuses LDS values across them; every wait is explicit.
template <typename Cfg>
__device__ __forceinline__ char* ring_base() {
    __shared__ __align__(16) char ring[Cfg::S * (Cfg::XBYTES + Cfg::WBYTES)];
    return ring;
}
template <typename Cfg, int D>
__device__ __forceinline__ char* ring_slot() {
    static_assert(D < Cfg::S, "ring slot");
    return ring_base<Cfg>() + D * (Cfg::XBYTES + Cfg::WBYTES);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr16(const char* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (s16x4_t __attribute__((address_space(3)))*)(p)));
}

template <typename Cfg>
struct DmaAddr {
    const char* src[Cfg::LMAX];  // per-lane source of each load at stage 0
    int64_t step[Cfg::LMAX];     // bytes a stage advances it by (uniform)
};

// Global -> LDS loads of the stage at k0 into slot D: lane l of load j writes
// bytes [1024 j + 16 l, + 16) of the slot (lds_dma16).  Lanes whose row or
// column lies outside the matrix read the matrix's first bytes instead; their
// products only reach outputs that are never stored.
template <typename Cfg, int D>
__device__ __forceinline__ uint32_t slot_lds_addr() {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)ring_slot<Cfg, D>();
}

template <typename Cfg, int D>
__device__ __forceinline__ void dma_issue(const DmaAddr<Cfg>& A, int wave, int64_t kstage) {
    const uint32_t slot = slot_lds_addr<Cfg, D>();
#pragma unroll
    for (int i = 0; i < Cfg::LMAX; ++i) {
        const int j = wave + i * Cfg::NW;
        if (Cfg::TI % Cfg::NW != 0 && j >= Cfg::TI) continue;
        lds_dma16(A.src[i] + kstage * A.step[i], __builtin_amdgcn_readfirstlane(slot + 1024 * j));
    }
}

template <typename Cfg, int D>
__device__ __forceinline__ void dma_compute(const uint32_t (&aoff)[Cfg::BK / 16], const uint32_t (&boff)[Cfg::FN],
                                            f32x16_t (&acc)[Cfg::FM][Cfg::FN]) {
    const char* xs = ring_slot<Cfg, D>();
    const char* ws = xs + Cfg::XBYTES;
    constexpr int NK = Cfg::BK / 16;
    // every fragment of the stage is requested before the first MFMA (this
    // measured faster than interleaving reads and MFMAs per k16 step)
    uint4 a[NK][Cfg::FM], b[NK][Cfg::FN];
#pragma unroll
    for (int k16 = 0; k16 < NK; ++k16) {
#pragma unroll
        for (int fm = 0; fm < Cfg::FM; ++fm)
            a[k16][fm] = *reinterpret_cast<const uint4*>(xs + aoff[k16] + fm * 32 * Cfg::BK * 2);
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn) {
            const char* p = ws + boff[fn] + k16 * 16 * Cfg::BN * 2;
            const uint2 lo = lds_tr16(p), hi = lds_tr16(p + 4 * Cfg::BN * 2);
            b[k16][fn] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
    }
#pragma unroll
    for (int k16 = 0; k16 < NK; ++k16)
#pragma unroll
        for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < Cfg::FN; ++fn) acc[fm][fn] = mfma32(a[k16][fm], b[k16][fn], acc[fm][fn]);
}

// One pipeline step: stage st from slot D; stage st + S - 1 into slot D - 1.
template <typename Cfg, int D>
__device__ __forceinline__ void dma_step(const DmaAddr<Cfg>& A, int wave, int64_t st, int64_t st1,
                                         const uint32_t (&aoff)[Cfg::BK / 16],
                                         const uint32_t (&boff)[Cfg::FN], f32x16_t (&acc)[Cfg::FM][Cfg::FN]) {
    if (st >= st1) return;
    // this wave's loads of stage st are done once at most those of the
    // stages issued after it are outstanding; the barrier then publishes
    // every wave's part of the slot (and ends every read of the slot
    // refilled below, made in the previous step)
    if (st + Cfg::S - 2 < st1) wait_vm_lgkm<(Cfg::S - 2) * Cfg::LMIN>();
    else wait_vm_lgkm<0>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (st + Cfg::S - 1 < st1) dma_issue<Cfg, (D + Cfg::S - 1) % Cfg::S>(A, wave, st + Cfg::S - 1);
    dma_compute<Cfg, D>(aoff, boff, acc);
}

template <typename Cfg, int... Ds>
__device__ __forceinline__ void dma_round(const DmaAddr<Cfg>& A, int wave, int64_t base, int64_t st1,
                                          const uint32_t (&aoff)[Cfg::BK / 16],
                                          const uint32_t (&boff)[Cfg::FN], f32x16_t (&acc)[Cfg::FM][Cfg::FN],
                                          std::integer_sequence<int, Ds...>) {
    (dma_step<Cfg, Ds>(A, wave, base + Ds, st1, aoff, boff, acc), ...);
}
template <typename Cfg, int... Ds>
__device__ __forceinline__ void dma_prologue(const DmaAddr<Cfg>& A, int wave, int64_t st0, int64_t st1,
                                             std::integer_sequence<int, Ds...>) {
    ((st0 + Ds < st1 ? dma_issue<Cfg, Ds>(A, wave, st0 + Ds) : void()), ...);
}

// Workgroups are dealt to the XCDs in turn (workgroup id mod kXcds), and
// each XCD has an L2 of its own.  This remap of the (m-tile, n-tile) grid
// gives XCD x a contiguous run of tiles in m-fastest order, so the m-tiles
// that share a column strip of W (and read it at about the same time) run on
// one XCD and fetch it through one L2.  It is a bijection of the grid
// whatever the XCD count, which only decides how well it places tiles.
constexpr int kXcds = 8;
__device__ __forceinline__ void xcd_tile(int64_t& mt, int64_t& nt) {
    const int64_t MT = gridDim.x, T = MT * gridDim.y;
    const int64_t g = mt + MT * nt;  // dispatch order within a split
    const int64_t x = g % kXcds, j = g / kXcds;
    const int64_t per = T / kXcds, rem = T % kXcds;
    const int64_t t = x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
    mt = t % MT;
    nt = t / MT;
}

template <typename Cfg>
__global__ __launch_bounds__(Cfg::NT) void k_dma(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                 void* __restrict__ Y, int y_bf16, int64_t M, int64_t N,
                                                 int64_t K, int splits, float* __restrict__ partial,
                                                 int64_t ntile0, int64_t NP) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // wave-uniform, so the loads' LDS base (M0) and their branches stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / Cfg::NWN, wn = wave % Cfg::NWN;
    int64_t mt = blockIdx.x, nt = blockIdx.y;
    if (gridDim.x > 1) xcd_tile(mt, nt);
    const int64_t m0 = mt * Cfg::BM;
    const int64_t n0 = (nt + ntile0) * Cfg::BN;
    const int split = blockIdx.z;
    const int64_t nst = (K + Cfg::BK - 1) / Cfg::BK;
    const int64_t st0 = split * nst / splits, st1 = (split + 1) * nst / splits;

    // K is a multiple of BK here: every stage lies inside the matrices
    DmaAddr<Cfg> A;
#pragma unroll
    for (int i = 0; i < Cfg::LMAX; ++i) {
        const int j = wave + i * Cfg::NW;
        A.src[i] = reinterpret_cast<const char*>(X);
        A.step[i] = 0;
        if (j < Cfg::XI) {
            const int r = j * Cfg::XROWS + lane / Cfg::XG;
            const int g = x_group<Cfg::XG>(lane % Cfg::XG, r);
            const int64_t m = m0 + r;
            A.step[i] = Cfg::BK * 2;
            if (m < M) A.src[i] = reinterpret_cast<const char*>(X + m * K + 8 * g);
        } else if (j < Cfg::TI) {
            const int kr = (j - Cfg::XI) * Cfg::WROWS + lane / Cfg::WG;
            const int g = w_group_tr(lane % Cfg::WG, kr);
            const int64_t n = n0 + 8 * g;
            A.src[i] = reinterpret_cast<const char*>(W);
            A.step[i] = (int64_t)Cfg::BK * N * 2;
            if (n < N) A.src[i] = reinterpret_cast<const char*>(W + kr * N + n);
        }
    }
    // fragment offsets within a slot
    uint32_t aoff[Cfg::BK / 16], boff[Cfg::FN];
    {
        const int r = wm * Cfg::WM + (lane & 31);
#pragma unroll
        for (int k16 = 0; k16 < Cfg::BK / 16; ++k16)
            aoff[k16] = (uint32_t)(r * Cfg::BK * 2 + 16 * x_group<Cfg::XG>(2 * k16 + (lane >> 5), r));
        const int s = lane & 15;
        const int kr = 8 * (lane >> 5) + (s >> 2);  // k16 = 0, h = 0
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn) {
            const int n = wn * Cfg::WN + 32 * fn + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
            boff[fn] = (uint32_t)(kr * Cfg::BN * 2 + 16 * w_group_tr(n >> 3, kr) + 2 * (n & 7));
        }
    }

    f32x16_t acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int a = 0; a < Cfg::FM; ++a)
#pragma unroll
        for (int b = 0; b < Cfg::FN; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.f;

    dma_prologue<Cfg>(A, wave, st0, st1, std::make_integer_sequence<int, Cfg::S - 1>{});
    for (int64_t base = st0; base < st1; base += Cfg::S)
        dma_round<Cfg>(A, wave, base, st1, aoff, boff, acc, std::make_integer_sequence<int, Cfg::S>{});

    // Stores of 4 consecutive columns per lane: registers 4 jj .. 4 jj + 3
    // of the lanes of a quad form a 4 x 4 block (lane i: column i, register
    // r: row r); transposed inside the quad, lane i holds row i, so one
    // 16-byte store (8 for bf16) replaces four 4-byte ones.  N is a multiple
    // of 8 and a quad's columns start at a multiple of 4: all four are in
    // range or none.
    const int g = lane >> 5, qi = lane & 3, q = (lane & 31) >> 2;
    const int64_t nbase = ntile0 * Cfg::BN;
    float* dstp = splits > 1 ? partial + (int64_t)split * M * NP : nullptr;
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn) {
            const int64_t n = n0 + wn * Cfg::WN + 32 * fn + 4 * q;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float v[4] = {acc[fm][fn][4 * jj], acc[fm][fn][4 * jj + 1], acc[fm][fn][4 * jj + 2],
                              acc[fm][fn][4 * jj + 3]};
                quad_transpose(v, qi);
                const int64_t m = m0 + wm * Cfg::WM + 32 * fm + 8 * jj + 4 * g + qi;
                if (m >= M || n >= N) continue;
                if (dstp) {
                    *reinterpret_cast<float4*>(dstp + m * NP + n - nbase) = make_float4(v[0], v[1], v[2], v[3]);
                } else if (y_bf16) {
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Y) + m * N + n) =
                        make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                                   (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
                } else {
                    *reinterpret_cast<float4*>(static_cast<float*>(Y) + m * N + n) = make_float4(v[0], v[1], v[2], v[3]);
                }
            }
        }
}

// Sum of split-K partials in split order: partial [splits][M][NP] holds
// columns nstart .. nstart + NP - 1 of Y; columns past N are skipped.
__global__ void k_reduce(const float* __restrict__ partial, void* __restrict__ Y, int y_bf16, int64_t M,
                         int64_t N, int64_t nstart, int64_t NP, int splits) {
    const int64_t q = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;  // NP % 4 == 0
    if (q >= M * NP) return;
    const int64_t m = q / NP, c = q % NP;
    if (nstart + c >= N) return;  // N % 8 == 0: all four columns are in range
    f32x4_t s = *reinterpret_cast<const f32x4_t*>(partial + q);
    for (int sp = 1; sp < splits; ++sp) s += *reinterpret_cast<const f32x4_t*>(partial + sp * M * NP + q);
    store_out(Y, y_bf16, m * N + nstart + c, s);
}

// ---- plans ---------------------------------------------------------------------
// Per-M choices, measured on MI355X for K = 4096 and N = 14336 / 151936.
using TileS = TileCfg<128, 128, 64, 32, 64>;   // 8 waves; K not a multiple of 32
using TileL = TileCfg<192, 256, 64, 96, 64>;
using TileB = TileCfg<256, 128, 64, 64, 64>;
using DmaS32 = DmaCfg<32, 128, 64, 1, 4, 4>;  // M <= 32
using DmaS64 = DmaCfg<64, 128, 64, 2, 4, 4>;  // M in (32, 64]
using DmaS = DmaCfg<128, 128, 64, 2, 4, 4>;   // M in (64, 128], or (128, 256] on narrow N
using DmaL = DmaCfg<192, 256, 32, 2, 4, 5>;   // M in (128, 192] on a wide N (lm-head)
using DmaW = DmaCfg<192, 512, 32, 2, 8, 3>;   // M in (128, 192], N >= 512 columns per compute unit
using DmaB = DmaCfg<256, 128, 32, 4, 2, 5>;   // M in (256, 464]
using DmaH = DmaCfg<256, 256, 64, 2, 4, 2>;   // M > 464, K a multiple of 64

enum Kern { kStrip1, kStrip2, kTileS, kTileL, kTileB, kDmaS32, kDmaS64, kDmaS, kDmaL, kDmaB, kDmaH, kDmaWL };

// One or two launches over ranges of n-tiles; each may split K.
struct Launch {
    int64_t t0, t1;  // n-tiles [t0, t1)
    int splits;
};
struct Plan {
    Kern kern;
    int64_t mtiles, ntiles;
    int BN;
    Launch l[2];
    int nl;
    size_t ws_bytes;
};

Plan make_plan(int64_t M, int64_t N, int64_t K, int cus) {
    Plan p{};
    // the strip kernel for up to 32 rows when K is not a multiple of 64;
    // otherwise a tile of 32 or 64 rows streams fewer X bytes per W byte
    // than the 128-row tile and beats the strip kernel too (MI355X, N =
    // 14336, K = 4096: M = 8: 24.2 vs 27.2 us, M = 32: 26.5 vs 33.0 us
    // with the 128-row tile, M = 64: 29.0 vs 36.2 us)
    auto strip_plan = [&]() {
        p.kern = M <= 16 ? kStrip1 : kStrip2;
        const int mt = M <= 16 ? 1 : 2;
        p.mtiles = (M + 16 * mt - 1) / (16 * mt);
        p.ntiles = (N + kStripN - 1) / kStripN;
        p.nl = 1;
        p.l[0] = Launch{0, p.ntiles, 1};
        return p;
    };
    if (M <= 32 && K % 64 != 0) return strip_plan();
    // the lm-head class (128 < M <= 192, at least one 192 x 512 tile per
    // compute unit): whole rounds of 192 x 512 tiles, then the remaining
    // columns as 192 x 256 tiles, split along K when they fill at most half
    // the machine
    if (M > 128 && M <= 192 && K % 32 == 0 && N / DmaW::BN >= cus) {
        const int64_t nst = K / DmaL::BK;
        p.kern = kDmaWL;
        p.mtiles = 1;
        const int64_t tw = N / DmaW::BN / cus * cus;  // 512-column tiles in whole rounds
        const int64_t c0 = tw * DmaW::BN;
        p.l[0] = Launch{0, tw, 1};
        p.nl = 1;
        p.ntiles = tw;
        if (c0 < N) {
            const int64_t t0 = c0 / DmaL::BN, t1 = (N + DmaL::BN - 1) / DmaL::BN, rem = t1 - t0;
            int s2 = 1;
            if (2 * rem <= cus && nst >= 16) s2 = (int)(cus / rem) > 4 ? 4 : (int)(cus / rem);
            p.l[1] = Launch{t0, t1, s2};
            p.nl = 2;
            p.ntiles = t1;
            if (s2 > 1) p.ws_bytes = align_up((size_t)s2 * M * rem * DmaL::BN * sizeof(float), 256);
        }
        return p;
    }
    int BM, BN, BK;
    auto pick = [&](Kern k, int bm, int bn, int bk) { p.kern = k; BM = bm; BN = bn; BK = bk; };
    if (K % 64 == 0 && M <= 32) {
        pick(kDmaS32, DmaS32::BM, DmaS32::BN, DmaS32::BK);
    } else if (K % 64 == 0 && M <= 64) {
        pick(kDmaS64, DmaS64::BM, DmaS64::BN, DmaS64::BK);
    } else if (K % 64 == 0 && M <= 128) {
        pick(kDmaS, DmaS::BM, DmaS::BN, DmaS::BK);
    } else if (K % 32 == 0 && M <= 192 && (N + DmaL::BN - 1) / DmaL::BN >= cus) {
        pick(kDmaL, DmaL::BM, DmaL::BN, DmaL::BK);
    } else if (K % 64 == 0 && M <= 256) {
        pick(kDmaS, DmaS::BM, DmaS::BN, DmaS::BK);
    } else if (K % 32 == 0 && M > 256) {
        // past 464 rows the 256 x 256 tile: at M = 768, N = 14336 its 168
        // tiles fit one round on 256 compute units where the 336 tiles of
        // 256 x 128 need two (measured 111 us against 152 us); at M = 480-512
        // its 112 tiles split in two along K stream fewer bytes per
        // workgroup than 224 tiles of 256 x 128 (79.1 vs 82.4 us at M = 512,
        // slower below 464 rows).  Its stage is 64 deep (half the barriers
        // of 32: 2-3% faster at M = 768 and 1024)
        if (M <= 464 || K % 64 != 0) pick(kDmaB, DmaB::BM, DmaB::BN, DmaB::BK);
        else pick(kDmaH, DmaH::BM, DmaH::BN, DmaH::BK);
    } else if (M > 128 && M <= 192 && (N + TileL::BN - 1) / TileL::BN >= cus) {
        pick(kTileL, TileL::BM, TileL::BN, TileL::BK);
    } else if (M <= 256) {
        pick(kTileS, TileS::BM, TileS::BN, TileS::BK);
    } else {
        pick(kTileB, TileB::BM, TileB::BN, TileB::BK);
    }
    // k_tile addresses its operands with 32-bit buffer offsets below kOOB:
    // a shape that would give it an operand of 2 GiB or more takes the strip
    // kernel (flat loads) instead, whatever M is
    const bool tile = p.kern == kTileS || p.kern == kTileL || p.kern == kTileB;
    if (tile && ((uint64_t)K * N * 2 >= kOOB || (uint64_t)M * K * 2 >= kOOB)) return strip_plan();
    p.BN = BN;
    p.mtiles = (M + BM - 1) / BM;
    p.ntiles = (N + BN - 1) / BN;
    const int64_t tiles = p.mtiles * p.ntiles;
    const int64_t nst = (K + BK - 1) / BK;
    const bool dma = p.kern == kDmaS32 || p.kern == kDmaS64 || p.kern == kDmaS || p.kern == kDmaL ||
                     p.kern == kDmaB || p.kern == kDmaH;
    const int64_t rem = p.ntiles % cus;
    if (dma && p.mtiles == 1 && p.ntiles > cus && rem > 0 && 2 * rem <= cus && nst >= 16) {
        // whole rounds of tiles, then the remainder split along K so that
        // the last round keeps every compute unit streaming
        int s2 = (int)(cus / rem);
        s2 = s2 > 4 ? 4 : s2;
        p.nl = 2;
        p.l[0] = Launch{0, p.ntiles - rem, 1};
        p.l[1] = Launch{p.ntiles - rem, p.ntiles, s2};
        p.ws_bytes = align_up((size_t)s2 * M * rem * BN * sizeof(float), 256);
        return p;
    }
    // split K in two when the tiles alone leave more than half the machine idle
    const int sp = (2 * tiles <= cus && nst >= 8) ? 2 : 1;
    p.nl = 1;
    p.l[0] = Launch{0, p.ntiles, sp};
    p.ws_bytes = sp > 1 ? align_up((size_t)sp * M * p.ntiles * BN * sizeof(float), 256) : 0;
    return p;
}

// NP: row stride of the partials, covering columns l.t0 BN .. l.t0 BN + NP - 1.
int launch_reduce(const Launch& l, int BN, int64_t NP, float* partial, void* Y, int yb, int64_t M,
                  int64_t N, hipStream_t s) {
    if (l.splits <= 1) return SPEC_OK;
    const int64_t nthr = M * NP / 4;
    hipLaunchKernelGGL(k_reduce, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, s, partial, Y, yb, M, N,
                       l.t0 * BN, NP, l.splits);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

template <typename Cfg, int D>
int launch_tile(const Plan& p, const uint16_t* x, const uint16_t* w, void* Y, int yb, int64_t M,
                int64_t N, int64_t K, float* partial, hipStream_t s) {
    constexpr size_t lds = 2 * Cfg::LDS;
    if constexpr (lds > 65536) {
        if (hipFuncSetAttribute((const void*)k_tile<Cfg, D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess)
            return SPEC_ERR_HIP;
    }
    const Launch& l = p.l[0];  // k_tile plans have one launch over every tile
    hipLaunchKernelGGL((k_tile<Cfg, D>), dim3((unsigned)p.mtiles, (unsigned)p.ntiles, (unsigned)l.splits),
                       dim3(Cfg::NT), lds, s, x, w, Y, yb, M, N, K, l.splits, partial);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    return launch_reduce(l, Cfg::BN, N, partial, Y, yb, M, N, s);  // k_tile partials: row stride N
}

// One launch of k_dma<Cfg> over the n-tiles of l (and its split-K reduce).
template <typename Cfg>
int launch_dma_one(const Plan& p, const Launch& l, const uint16_t* x, const uint16_t* w, void* Y, int yb,
                   int64_t M, int64_t N, int64_t K, float* partial, hipStream_t s) {
    const int64_t NP = (l.t1 - l.t0) * Cfg::BN;
    hipLaunchKernelGGL((k_dma<Cfg>), dim3((unsigned)p.mtiles, (unsigned)(l.t1 - l.t0), (unsigned)l.splits),
                       dim3(Cfg::NT), 0, s, x, w, Y, yb, M, N, K, l.splits, partial, l.t0, NP);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    return launch_reduce(l, Cfg::BN, NP, partial, Y, yb, M, N, s);
}

template <typename Cfg>
int launch_dma(const Plan& p, const uint16_t* x, const uint16_t* w, void* Y, int yb, int64_t M, int64_t N,
               int64_t K, float* partial, hipStream_t s) {
    for (int i = 0; i < p.nl; ++i) {
        const int rc = launch_dma_one<Cfg>(p, p.l[i], x, w, Y, yb, M, N, K, partial, s);
        if (rc != SPEC_OK) return rc;
    }
    return SPEC_OK;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

}  // namespace

// Compute units of the current device, queried once per device and cached
// (the plans depend on it; a query per call would cost a runtime round trip).
int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 256;
    cus = cus > 0 ? cus : 256;
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace specv

using namespace specv;

extern "C" size_t spec_verify_linear_workspace_bytes(int64_t M, int64_t N, int64_t Kd) {
    if (M <= 0 || N <= 0 || Kd <= 0) return 0;
    return make_plan(M, N, Kd, device_cus()).ws_bytes;
}

extern "C" int spec_verify_linear(const void* X, const void* W, void* Y, int y_dtype, int64_t M,
                                  int64_t N, int64_t Kd, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    if (M < 0 || N < 1 || Kd < 1 || (N % 8) != 0 || (Kd % 8) != 0) return SPEC_ERR_INVALID_ARG;
    if (y_dtype != SPEC_F32 && y_dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
    if (M == 0) return SPEC_OK;
    if (!X || !W || !Y || !aligned16(X) || !aligned16(W) || !aligned16(Y)) return SPEC_ERR_INVALID_ARG;
    const Plan p = make_plan(M, N, Kd, device_cus());
    if (p.ntiles > 65535 || p.mtiles > 0x7FFFFFFF) return SPEC_ERR_INVALID_ARG;
    if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes || !aligned16(workspace)))
        return SPEC_ERR_WORKSPACE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const uint16_t* x = static_cast<const uint16_t*>(X);
    const uint16_t* w = static_cast<const uint16_t*>(W);
    const int yb = y_dtype == SPEC_BF16;
    float* partial = static_cast<float*>(workspace);
    const dim3 sgrid((unsigned)p.mtiles, (unsigned)p.ntiles);
    const dim3 sblock(kStripWaves * kWave);
    switch (p.kern) {
        case kStrip1: hipLaunchKernelGGL(k_strip<1>, sgrid, sblock, 0, s, x, w, Y, yb, M, N, Kd); break;
        case kStrip2: hipLaunchKernelGGL(k_strip<2>, sgrid, sblock, 0, s, x, w, Y, yb, M, N, Kd); break;
        case kTileS: return launch_tile<TileS, 2>(p, x, w, Y, yb, M, N, Kd, partial, s);
        case kTileL: return launch_tile<TileL, 2>(p, x, w, Y, yb, M, N, Kd, partial, s);
        case kTileB: return launch_tile<TileB, 2>(p, x, w, Y, yb, M, N, Kd, partial, s);
        case kDmaS32: return launch_dma<DmaS32>(p, x, w, Y, yb, M, N, Kd, partial, s);
        case kDmaS64: return launch_dma<DmaS64>(p, x, w, Y, yb, M, N, Kd, partial, s);
        case kDmaS: return launch_dma<DmaS>(p, x, w, Y, yb, M, N, Kd, partial, s);
        case kDmaL: return launch_dma<DmaL>(p, x, w, Y, yb, M, N, Kd, partial, s);
        case kDmaB: return launch_dma<DmaB>(p, x, w, Y, yb, M, N, Kd, partial, s);
        case kDmaH: return launch_dma<DmaH>(p, x, w, Y, yb, M, N, Kd, partial, s);
        case kDmaWL: {
            const int rc = launch_dma_one<DmaW>(p, p.l[0], x, w, Y, yb, M, N, Kd, partial, s);
            if (rc != SPEC_OK || p.nl < 2) return rc;
            return launch_dma_one<DmaL>(p, p.l[1], x, w, Y, yb, M, N, Kd, partial, s);
        }
    }
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    return SPEC_OK;
}
