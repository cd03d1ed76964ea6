// spec_verify_linear_packed.hip -- the verify linear layer Y = X W with W
// stored once in the operand order of v_mfma_f32_16x16x32_bf16 ("packed"),
// for a weight that every verify pass reads whole, such as the lm-head.
//
// Method: page "New technical post reveals how speculative decoding
// accelerates LLM inference without hurting accuracy" (agentnet.co.il),
// sections "The formula behind the speedup" and "GEMM-M grows, a small batch
// suffices": verifying D drafts turns the layer's M = B rows into B(1+D);
// below the machine's FLOP-per-byte ridge the layer is bound by reading W
// once per pass.  The operation is the one spec_verify_linear computes; only
// W's layout in memory differs.
//
// Packed layout (spec_pack_weight).  W [K, N] bf16 (N contiguous) becomes
// 2 KB blocks, one per 32 rows of k and 32 columns: block (s, c) at byte
// (s C + c) 2048, C = ceil(N / 32), k-major so that the workgroups of one
// round read one contiguous span per 32 rows of k.  Inside a block, the 16
// bytes at 16 (64 h + l) (h = 0, 1; lane l < 64) are
// W[32 s + 8 (l / 16) + j][32 c + 16 h + l % 16], j = 0..7: lane l's B
// operand of the MFMA for the 16 columns 32 c + 16 h ...  Columns past N are
// zero.
//
// k_packed<MB>: one 512-thread workgroup per 256-column tile of MB x 16 rows
// (MB = 4, 8 or 12).  Wave w owns the 32 columns of block 8 t + w and loads
// its operands with plain 16-byte loads, two 64-deep k-stages ahead, into
// registers: W never passes through LDS.  X goes through a three-slot LDS
// ring by loads that write LDS (global_load_lds_dwordx4), two stages ahead,
// and every wave reads its A operands from there.  On MI355X this
// streams the lm-head's W faster than the tiles of spec_verify_linear, whose
// W and X both pass through those LDS-writing loads and whose rate is set by
// the bytes each compute unit moves through them.  Loads complete in issue
// order, so a wait for one load also waits for every load issued before it:
// the loads are issued so that the wait for an X slot never drains W loads
// still in flight.
// Whole rounds of tiles run unsplit; the tiles left after the last whole
// round (or every tile, when they fill at most half the machine) are split
// along K into fp32 partials that k_packed_reduce sums in split order.
#include "spec_verify.h"
#include "device_common.hpp"

namespace specv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kPkCols = 256;       // columns per tile: 8 waves x 32
constexpr int kPkStage = 64;       // k per stage
constexpr int kPkThreads = 512;
constexpr int64_t kPkBlock = 2048;  // bytes per (32 k, 32 columns) block

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// X stage slot: MB x 16 rows of 128 bytes (64 k); the 16-byte group g of
// row r sits at group g ^ ((r >> 1) & 7), which spreads the A-operand reads
// (16 rows at one k offset) over the banks.
template <int MB>
__global__ __launch_bounds__(kPkThreads) void k_packed(const uint16_t* __restrict__ X, const uint4* __restrict__ Wp,
                                                       void* __restrict__ Y, int y_bf16, float* __restrict__ partial,
                                                       int64_t M, int64_t N, int64_t K, int64_t tile0, int splits,
                                                       int64_t ncolP) {
    constexpr int SLOT = MB * 16 * 128;
    constexpr int XL = MB / 4;  // LDS-writing loads of X per wave per stage
    static_assert(MB == 4 || MB == 8 || MB == 12, "4, 8 or 12 row blocks");
    __shared__ __align__(1024) char lds[3 * SLOT];
    const int t = threadIdx.x, lane = t & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int64_t C = (N + 31) / 32;
    const int64_t c = (tile0 + blockIdx.x) * 8 + wave;
    const int64_t cl = c < C ? c : C - 1;  // waves past the last block load a real one and store nothing
    const int64_t m0 = (int64_t)blockIdx.y * MB * 16;
    const int z = blockIdx.z;
    const int64_t NT = K / kPkStage;
    const int64_t st0 = z * NT / splits;
    const int NS = (int)((z + 1) * NT / splits - st0);
    const int64_t rowq = C * 128;  // uint4 per 32 rows of k
    const uint4* wp = Wp + cl * 128 + lane + 2 * st0 * rowq;

    f32x4_t acc[MB][2];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) acc[rb][0] = acc[rb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // X load i of this wave covers rows 8 (wave + 8 i) .. +7 of the tile; lane l
    // fills row 8 j + l / 8, slot group l % 8, from the group that maps there.
    // Rows past M read row M - 1 (finite; their outputs are never stored).
    auto xsrc = [&](int i) {
        const int j = wave + 8 * i, r = 8 * j + lane / 8;
        const int64_t row = m0 + r < M ? m0 + r : M - 1;
        const int g = (lane & 7) ^ ((r >> 1) & 7);
        return reinterpret_cast<const char*>(X) + row * K * 2 + st0 * 128 + 16 * g;
    };
    const char* const xs0 = xsrc(0);
    const char* const xs1 = xsrc(XL > 1 ? 1 : 0);
    const char* const xs2 = xsrc(XL > 2 ? 2 : 0);
    const uint32_t lbase = (uint32_t)(uintptr_t)(lds_char*)lds;
#define PK_DMAX(S, SL)                                                                                      \
    do {                                                                                                    \
        lds_dma16(xs0 + (int64_t)(S) * 128, __builtin_amdgcn_readfirstlane(lbase + (SL) * SLOT + 1024 * wave)); \
        if (XL > 1)                                                                                         \
            lds_dma16(xs1 + (int64_t)(S) * 128,                                                             \
                      __builtin_amdgcn_readfirstlane(lbase + (SL) * SLOT + 1024 * (wave + 8)));             \
        if (XL > 2)                                                                                         \
            lds_dma16(xs2 + (int64_t)(S) * 128,                                                             \
                      __builtin_amdgcn_readfirstlane(lbase + (SL) * SLOT + 1024 * (wave + 16)));            \
    } while (0)
    // this wave's B operands of stage S: k rows 32 (2 S) and 32 (2 S + 1) of the
    // split, columns 0-15 and 16-31 of its block
#define PK_LDW(S, W0, W1, W2, W3)                                   \
    do {                                                            \
        const uint4* p_ = wp + (int64_t)(2 * (S)) * rowq;           \
        W0 = p_[0];                                                 \
        W1 = p_[64];                                                \
        W2 = p_[rowq];                                              \
        W3 = p_[rowq + 64];                                         \
    } while (0)
    // A operand of row block rb, k half kk: row 16 rb + l % 16, k 32 kk + 8 (l / 16)
    const int sw = ((lane & 15) >> 1) & 7;
    const uint32_t aoff0 = (lane & 15) * 128 + 16 * ((lane >> 4) ^ sw);
    const uint32_t aoff1 = (lane & 15) * 128 + 16 * ((4 + (lane >> 4)) ^ sw);
    // Row block 0 first, with all four operands: every wait the compiler
    // inserts for this stage's W falls there (see PK_STEP).
#define PK_COMP_A(SL, W0, W1, W2, W3)                                                   \
    do {                                                                                \
        const char* xs_ = lds + (SL) * SLOT;                                            \
        const uint4 p_ = *reinterpret_cast<const uint4*>(xs_ + aoff0);                  \
        const uint4 q_ = *reinterpret_cast<const uint4*>(xs_ + aoff1);                  \
        acc[0][0] = mfma16(p_, W0, acc[0][0]);                                          \
        acc[0][1] = mfma16(p_, W1, acc[0][1]);                                          \
        acc[0][0] = mfma16(q_, W2, acc[0][0]);                                          \
        acc[0][1] = mfma16(q_, W3, acc[0][1]);                                          \
    } while (0)
    // the other row blocks, fragment reads interleaved with the MFMAs: three
    // reads ahead, then one read per two MFMAs
#define PK_COMP_B(SL, W0, W1, W2, W3)                                                   \
    do {                                                                                \
        const char* xs_ = lds + (SL) * SLOT;                                            \
        _Pragma("unroll") for (int rb = 1; rb < MB; ++rb) {                             \
            const uint4 p_ = *reinterpret_cast<const uint4*>(xs_ + aoff0 + rb * 2048);  \
            acc[rb][0] = mfma16(p_, W0, acc[rb][0]);                                    \
            acc[rb][1] = mfma16(p_, W1, acc[rb][1]);                                    \
            const uint4 q_ = *reinterpret_cast<const uint4*>(xs_ + aoff1 + rb * 2048);  \
            acc[rb][0] = mfma16(q_, W2, acc[rb][0]);                                    \
            acc[rb][1] = mfma16(q_, W3, acc[rb][1]);                                    \
        }                                                                               \
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);                              \
        _Pragma("unroll") for (int i_ = 0; i_ < 2 * (MB - 1) - 3; ++i_) {               \
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                          \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                          \
        }                                                                               \
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);                              \
    } while (0)
    // Stage S reads X from slot S % 3 and W from the registers loaded two
    // stages earlier.  The order of a stage's loads keeps the waits exact.
    // Loads complete in issue order, and the compiler, which does not see the
    // LDS-writing loads, waits for W(S) by counting only the W loads issued
    // after it.  That count is right as long as no LDS-writing load is issued
    // between W(S+1) and the last wait for W(S), so row block 0 (which takes
    // all of W(S)) runs first, then X(S+2) goes into slot (S+2) % 3 (freed by
    // the previous barrier), then the other row blocks, then W(S+2) into the
    // registers just used.  Before the barrier X(S+1) must have landed: in
    // the steady state this wave issued W(S+1), X(S+2) and W(S+2) after it,
    // 8 + XL loads (the last steps wait for everything).
#define PK_STEP(S, SL, W0, W1, W2, W3, TAIL)                                  \
    do {                                                                      \
        if (!(TAIL) || (S) < NS) {                                            \
            PK_COMP_A(SL, W0, W1, W2, W3);                                    \
            __builtin_amdgcn_sched_barrier(0);                                \
            if (!(TAIL) || (S) + 2 < NS) PK_DMAX((S) + 2, ((SL) + 2) % 3);    \
            __builtin_amdgcn_sched_barrier(0);                                \
            PK_COMP_B(SL, W0, W1, W2, W3);                                    \
            if (!(TAIL) || (S) + 2 < NS) PK_LDW((S) + 2, W0, W1, W2, W3);     \
            asm volatile("" ::: "memory");                                    \
            __builtin_amdgcn_sched_barrier(0);                                \
            if (TAIL) wait_vm_lgkm<0>();                                      \
            else wait_vm_lgkm<8 + XL>();                                      \
            __builtin_amdgcn_s_barrier();                                     \
            __builtin_amdgcn_sched_barrier(0);                                \
        }                                                                     \
    } while (0)
#define PK_BLOCK(S, TAIL)                             \
    do {                                              \
        PK_STEP(S, 0, a0, a1, a2, a3, TAIL);          \
        PK_STEP((S) + 1, 1, b0, b1, b2, b3, TAIL);    \
        PK_STEP((S) + 2, 2, a0, a1, a2, a3, TAIL);    \
        PK_STEP((S) + 3, 0, b0, b1, b2, b3, TAIL);    \
        PK_STEP((S) + 4, 1, a0, a1, a2, a3, TAIL);    \
        PK_STEP((S) + 5, 2, b0, b1, b2, b3, TAIL);    \
    } while (0)
    uint4 a0, a1, a2, a3, b0, b1, b2, b3;
    PK_DMAX(0, 0);
    if (NS > 1) PK_DMAX(1, 1);
    PK_LDW(0, a0, a1, a2, a3);
    if (NS > 1) PK_LDW(1, b0, b1, b2, b3);
    wait_vm_lgkm<0>();
    __builtin_amdgcn_s_barrier();
    // Blocks of six stages (the period of the three slots and the two W
    // register sets).  A block runs unchecked only if every load it issues is
    // in range (its last stage's loads of stage S + 2 below NS); the stages
    // left over, at most seven, run in two checked blocks.
    int s = 0;
    for (; s + 8 <= NS; s += 6) PK_BLOCK(s, false);
    PK_BLOCK(s, true);
    PK_BLOCK(s + 6, true);
#undef PK_BLOCK
#undef PK_STEP
#undef PK_COMP_A
#undef PK_COMP_B
#undef PK_LDW
#undef PK_DMAX

    if (c >= C) return;  // wave-uniform: the quad exchanges below stay within a wave
    // D register j of lane l: row 4 (l / 16) + j, column l % 16 of the block.
    // With N a multiple of 4, the 4 x 4 block of a quad of lanes (lane i:
    // column i) is transposed inside the quad (lane i: row i), so each lane
    // stores 4 consecutive columns with one 16-byte store (8 for bf16): all
    // four are in range or none.  Otherwise one 4-byte store per element.
    const bool vec = (N & 3) == 0;
    const int g = lane >> 4, qi = lane & 3;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float v[4] = {acc[rb][h][0], acc[rb][h][1], acc[rb][h][2], acc[rb][h][3]};
            if (vec) {
                quad_transpose(v, qi);
                const int64_t n = 32 * c + 16 * h + (lane & 12);
                const int64_t r = m0 + 16 * rb + 4 * g + qi;
                if (r >= M || n >= N) continue;
                if (splits > 1)
                    *reinterpret_cast<float4*>(partial + (z * M + r) * ncolP + (n - tile0 * kPkCols)) =
                        make_float4(v[0], v[1], v[2], v[3]);
                else if (y_bf16)
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Y) + r * N + n) =
                        make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                                   (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
                else
                    *reinterpret_cast<float4*>(static_cast<float*>(Y) + r * N + n) = make_float4(v[0], v[1], v[2], v[3]);
                continue;
            }
            const int64_t n = 32 * c + 16 * h + (lane & 15);
            if (n >= N) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t r = m0 + 16 * rb + 4 * g + j;
                if (r >= M) continue;
                if (splits > 1)
                    partial[(z * M + r) * ncolP + (n - tile0 * kPkCols)] = v[j];
                else if (y_bf16)
                    static_cast<uint16_t*>(Y)[r * N + n] = f32_to_bf16(v[j]);
                else
                    static_cast<float*>(Y)[r * N + n] = v[j];
            }
        }
}

// Y[r, n0 + j] = sum over the splits, in split order, of partial[s][r][j]
// (j < ncols); four columns per thread when N is a multiple of 4 (n0 and the
// partials' row stride always are).
template <bool VEC>
__global__ __launch_bounds__(256) void k_packed_reduce(const float* __restrict__ partial, void* __restrict__ Y,
                                                       int y_bf16, int64_t M, int64_t N, int64_t n0, int64_t ncols,
                                                       int64_t ncolP, int splits) {
    constexpr int V = VEC ? 4 : 1;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_row = ncols / V;
    if (i >= M * per_row) return;
    const int64_t r = i / per_row, j = V * (i % per_row);
    if constexpr (VEC) {
        f32x4_t v = *reinterpret_cast<const f32x4_t*>(partial + r * ncolP + j);
        for (int s = 1; s < splits; ++s) v += *reinterpret_cast<const f32x4_t*>(partial + (s * M + r) * ncolP + j);
        const int64_t o = r * N + n0 + j;
        if (y_bf16)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Y) + o) =
                make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                           (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
        else
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(Y) + o) = v;
    } else {
        float v = partial[r * ncolP + j];
        for (int s = 1; s < splits; ++s) v += partial[(s * M + r) * ncolP + j];
        if (y_bf16)
            static_cast<uint16_t*>(Y)[r * N + n0 + j] = f32_to_bf16(v);
        else
            static_cast<float*>(Y)[r * N + n0 + j] = v;
    }
}

// One thread per 16-byte lane record of the packed layout.
__global__ __launch_bounds__(256) void k_pack_weight(const uint16_t* __restrict__ W, uint4* __restrict__ Wp,
                                                     int64_t K, int64_t N, int64_t total) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= total) return;
    const int64_t C = (N + 31) / 32;
    const int e = (int)(q % 128), h = e / 64, l = e % 64;
    const int64_t blk = q / 128, c = blk % C, s = blk / C;
    const int64_t n = 32 * c + 16 * h + l % 16;
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = n < N ? W[(32 * s + 8 * (l / 16) + j) * N + n] : 0u;
    Wp[q] = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
}

struct PkLaunch {
    int64_t t0, t1;  // tiles [t0, t1)
    int splits;
};
struct PkPlan {
    int mb = 12;
    int64_t mtiles = 0;
    int nl = 0;
    PkLaunch l[2];
    size_t ws_bytes = 0;
};

PkPlan make_packed_plan(int64_t M, int64_t N, int64_t K, int cus) {
    PkPlan p;
    p.mb = M <= 64 ? 4 : M <= 128 ? 8 : 12;
    p.mtiles = (M + p.mb * 16 - 1) / (p.mb * 16);
    const int64_t tiles = (N + kPkCols - 1) / kPkCols;
    const int64_t nst = K / kPkStage;
    auto split_for = [&](int64_t wgs, int64_t min_st) {
        if (2 * wgs > cus || nst < min_st) return 1;
        const int64_t s = cus / wgs;
        return (int)(s > 4 ? 4 : s);
    };
    if (p.mtiles == 1 && tiles > cus) {
        // whole rounds, then the remainder split along K so that the last
        // round keeps the machine streaming
        const int64_t whole = tiles / cus * cus, rem = tiles - whole;
        p.l[0] = PkLaunch{0, whole, 1};
        p.nl = 1;
        if (rem > 0) p.l[p.nl++] = PkLaunch{whole, tiles, split_for(rem, 16)};
    } else {
        p.l[0] = PkLaunch{0, tiles, split_for(tiles * p.mtiles, 8)};
        p.nl = 1;
    }
    for (int i = 0; i < p.nl; ++i)
        if (p.l[i].splits > 1) {
            const size_t b = align_up((size_t)p.l[i].splits * M * (p.l[i].t1 - p.l[i].t0) * kPkCols * sizeof(float), 256);
            p.ws_bytes = b > p.ws_bytes ? b : p.ws_bytes;
        }
    return p;
}

template <int MB>
int launch_packed(const PkPlan& p, const uint16_t* x, const uint4* wp, void* Y, int yb, int64_t M, int64_t N,
                  int64_t K, float* partial, hipStream_t s) {
    for (int i = 0; i < p.nl; ++i) {
        const PkLaunch& l = p.l[i];
        const int64_t nt = l.t1 - l.t0, ncolP = nt * kPkCols;
        hipLaunchKernelGGL(k_packed<MB>, dim3((unsigned)nt, (unsigned)p.mtiles, (unsigned)l.splits),
                           dim3(kPkThreads), 0, s, x, wp, Y, yb, partial, M, N, K, l.t0, l.splits, ncolP);
        if (l.splits > 1) {
            const int64_t n0 = l.t0 * kPkCols, ncols = (N < l.t1 * kPkCols ? N : l.t1 * kPkCols) - n0;
            if (N % 4 == 0) {
                const int64_t n = M * (ncols / 4);
                hipLaunchKernelGGL(k_packed_reduce<true>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                                   partial, Y, yb, M, N, n0, ncols, ncolP, l.splits);
            } else {
                const int64_t n = M * ncols;
                hipLaunchKernelGGL(k_packed_reduce<false>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                                   partial, Y, yb, M, N, n0, ncols, ncolP, l.splits);
            }
        }
    }
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

bool packed_shape_ok(int64_t N, int64_t K) {
    return N >= 1 && K >= kPkStage && K % kPkStage == 0 && K <= (int64_t)1 << 30 && N <= (int64_t)1 << 36;
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_packed_weight_bytes(int64_t K, int64_t N) {
    if (!packed_shape_ok(N, K)) return 0;
    return (size_t)(K / 32) * (size_t)((N + 31) / 32) * (size_t)kPkBlock;
}

extern "C" int spec_pack_weight(const void* W, void* Wp, int64_t K, int64_t N, void* stream) {
    if (!packed_shape_ok(N, K) || !W || !Wp || !aligned16(Wp) || ((uintptr_t)W & 1)) return SPEC_ERR_INVALID_ARG;
    const int64_t total = (K / 32) * ((N + 31) / 32) * 128;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7FFFFFFF) return SPEC_ERR_INVALID_ARG;
    hipLaunchKernelGGL(k_pack_weight, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(W), static_cast<uint4*>(Wp), K, N, total);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

extern "C" size_t spec_verify_linear_packed_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || !packed_shape_ok(N, K)) return 0;
    return make_packed_plan(M, N, K, device_cus()).ws_bytes;
}

extern "C" int spec_verify_linear_packed(const void* X, const void* Wp, void* Y, int y_dtype, int64_t M, int64_t N,
                                         int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
    if (M < 0 || !packed_shape_ok(N, K)) return SPEC_ERR_INVALID_ARG;
    if (y_dtype != SPEC_F32 && y_dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
    if (M == 0) return SPEC_OK;
    if (!X || !Wp || !Y || !aligned16(X) || !aligned16(Wp) || !aligned16(Y)) return SPEC_ERR_INVALID_ARG;
    const PkPlan p = make_packed_plan(M, N, K, device_cus());
    for (int i = 0; i < p.nl; ++i)
        if (p.l[i].t1 - p.l[i].t0 > 0x7FFFFFFF) return SPEC_ERR_INVALID_ARG;
    if (p.mtiles > 65535) return SPEC_ERR_INVALID_ARG;
    if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes || !aligned16(workspace)))
        return SPEC_ERR_WORKSPACE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const uint16_t* x = static_cast<const uint16_t*>(X);
    const uint4* wp = static_cast<const uint4*>(Wp);
    const int yb = y_dtype == SPEC_BF16;
    float* partial = static_cast<float*>(workspace);
    switch (p.mb) {
        case 4: return launch_packed<4>(p, x, wp, Y, yb, M, N, K, partial, s);
        case 8: return launch_packed<8>(p, x, wp, Y, yb, M, N, K, partial, s);
        default: return launch_packed<12>(p, x, wp, Y, yb, M, N, K, partial, s);
    }
}
