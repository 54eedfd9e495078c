// rr_device.h -- device-side helpers shared by the librr kernels (gfx950).
//
// Vector types for the CDNA4 bf16 matrix instructions, 16-byte global/LDS
// accesses, bf16 rounding and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rr {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ uint4 as_u4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(uint16_t *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// fp32 -> bf16 bit pattern, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t bf16_bits(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// acc + lo(x) + hi(x) for a packed bf16 pair (v_dot2c_f32_bf16 against 1.0).
__device__ __forceinline__ float add_bf16x2(uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                           __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

// Two fp32 -> packed bf16x2 (low half = a), one v_cvt_pk_bf16_f32 (RNE).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane (lane ^ m) in a 64-wide wave.
__device__ __forceinline__ float xor_lane(float v, int m) { return __shfl_xor(v, m, kWave); }

typedef __attribute__((address_space(3))) char lds_char;

// 16-byte global -> LDS copy without registers (global_load_lds_dwordx4):
// lane i of the wave writes lds_wave_base + 16*i; lds_wave_base must be the
// same for the whole wave.
__device__ __forceinline__ void g2lds16(const void *src, lds_char *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
}

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format,
// no swizzle): byte-addressed, offsets from a VGPR, no range clamping used.
constexpr int kBufFlags = 0x00020000;

// Buffer resource over the bytes starting at p (no range limit).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, -1, kBufFlags);
}

// Buffer resource over the first `bytes` bytes starting at p: a load whose
// byte offset lies at or past `bytes` returns zeros (no memory access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc_n(const void *p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, kBufFlags);
}

// 16-byte buffer -> LDS copy without registers (buffer_load_dwordx4 ... lds):
// lane i reads rsrc base + off and writes lds_wave_base + 16*i.  Unlike the
// flat-encoded global_load_lds, a buffer copy in flight leaves the compiler
// able to count LDS reads in issue order, so fragment reads can run ahead of
// their use without every wait draining all of them.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t r, uint32_t off, lds_char *lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, (int)off, 0, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (<= n pending).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) only (LDS reads of this wave have returned).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Work-group barrier without the memory fence of __syncthreads: the caller
// orders LDS traffic with explicit waits.
__device__ __forceinline__ void bar() { __builtin_amdgcn_s_barrier(); }

// op(x[lane], x[lane ^ 16]) and op(x[lane], x[lane ^ 32]) for every lane
// through v_permlane16_swap / v_permlane32_swap (no LDS round trip).
__device__ __forceinline__ float xor16_max(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Merge two (max, sum-of-2^(x-max)) pairs.  (-inf, 0) is the identity.
__device__ __forceinline__ void merge_max_sum(float &m, float &z, float m2, float z2) {
    float nm = fmaxf(m, m2);
    if (nm == -INFINITY) return;
    z = z * fast_exp2(m - nm) + z2 * fast_exp2(m2 - nm);
    m = nm;
}

}  // namespace rr
