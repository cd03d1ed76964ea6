// device_common.hpp -- small gfx950 device helpers shared by the kernels of
// libspecverify: bf16 unpacking, wave64 reductions, workspace alignment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kWave = 64;

// Host: compute units of the current device (queried once per device and
// cached; the GEMM plans depend on it).  Defined in spec_verify_linear.hip.
int device_cus();

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// bf16 is the top half of an fp32: widening is a shift / mask, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// exp2 on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v |= __shfl_xor(v, o, kWave);
    return v;
}

// Reads of register v from lane l ^ 1 and l ^ 2 of the same quad (DPP quad
// permutations 1,0,3,2 and 2,3,0,1).
__device__ __forceinline__ float quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
// 4 x 4 transpose inside each quad of lanes: lane i (qi = lane & 3) holds
// column i of a block in v[0..3] (v[r] = row r) and ends holding row i
// (v[c] = column c).  Two exchanges: across lane bit 0 the registers whose
// bit 0 differs from the lane's, then across lane bit 1 likewise.  Every
// lane of the wave must take part.
__device__ __forceinline__ void quad_transpose(float (&v)[4], int qi) {
    const bool b0 = qi & 1, b1 = (qi & 2) != 0;
    const float r01 = quad_xor1(b0 ? v[0] : v[1]);
    const float r23 = quad_xor1(b0 ? v[2] : v[3]);
    v[0] = b0 ? r01 : v[0];
    v[1] = b0 ? v[1] : r01;
    v[2] = b0 ? r23 : v[2];
    v[3] = b0 ? v[3] : r23;
    const float r02 = quad_xor2(b1 ? v[0] : v[2]);
    const float r13 = quad_xor2(b1 ? v[1] : v[3]);
    v[0] = b1 ? r02 : v[0];
    v[2] = b1 ? v[2] : r02;
    v[1] = b1 ? r13 : v[1];
    v[3] = b1 ? v[3] : r13;
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt untouched): at most N of this wave's
// vector memory operations still outstanding, no LDS/scalar ones.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// 16 bytes per lane from global memory into LDS at (M0 + 16 lane): the GEMM
// kernels' loads that write LDS (global_load_lds_dwordx4).  Issued as inline
// assembly: the compiler neither tracks these loads nor inserts waits for
// them, so every wait on them is explicit (wait_vm_lgkm).  M0 holds the LDS
// base of the load; that is sound only while the compiler keeps no value of
// its own in M0 in the kernels that use it: in their gfx950 assembly every M0
// access is one of these writes, one per load (checked on every build of the
// test suite, tests/test_isa_m0.py).
__device__ __forceinline__ void lds_dma16(const char* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(src) : "memory", "m0");
}

}  // namespace specv
