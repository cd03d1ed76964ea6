// philox.hpp -- device Philox4x32-10 counter-based generator, written from
// its published definition (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11): ten rounds, each taking the 32x32->64
// products of words 0 and 2 with the two Philox multipliers, with the key
// advanced by the two Weyl increments between rounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

struct PhiloxBlock {
    uint32_t w[4];
};

__device__ __forceinline__ PhiloxBlock philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                     uint32_t c3, uint32_t k0, uint32_t k1) {
    constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
    constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
    // rolled: the generator runs a few times per row, off the streaming path,
    // where a small code footprint matters more than loop overhead
#pragma unroll 1
    for (int r = 0; r < 10; ++r) {
        const uint32_t pa_hi = __umulhi(kMulA, c0), pa_lo = kMulA * c0;
        const uint32_t pb_hi = __umulhi(kMulB, c2), pb_lo = kMulB * c2;
        const uint32_t n0 = pb_hi ^ c1 ^ k0;
        const uint32_t n2 = pa_hi ^ c3 ^ k1;
        c0 = n0;
        c1 = pb_lo;
        c2 = n2;
        c3 = pa_lo;
        k0 += kWeylA;
        k1 += kWeylB;
    }
    return PhiloxBlock{{c0, c1, c2, c3}};
}

// Uniforms of (global row, position): block at counter (pos, row, off_lo,
// off_hi) under key (seed_lo, seed_hi); 24-bit, exact in fp32.
struct RowPosUniforms {
    float acc;  // acceptance test
    float smp;  // categorical draw
};

__device__ __forceinline__ RowPosUniforms row_pos_uniforms(uint64_t seed, uint64_t offset,
                                                           uint32_t row, uint32_t pos) {
    const PhiloxBlock b = philox4x32_10(pos, row, (uint32_t)offset, (uint32_t)(offset >> 32),
                                        (uint32_t)seed, (uint32_t)(seed >> 32));
    constexpr float kScale = 1.0f / 16777216.0f;
    return RowPosUniforms{(float)(b.w[0] >> 8) * kScale, (float)(b.w[1] >> 8) * kScale};
}

}  // namespace specv
