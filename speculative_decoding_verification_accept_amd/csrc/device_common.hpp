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
