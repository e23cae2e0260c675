// fsa_common.h -- shared device helpers for the gfx950 kernels of libfsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA 16x16x32 operand
typedef __attribute__((ext_vector_type(4))) float f32x4_t;     // MFMA 16x16 accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;  // 16-byte raw load
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;  // 8-byte raw store

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBlockKeys = 64;   // keys per selectable KV block

// C[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulation (gfx950).
// Lane l supplies A[l%16][8*(l/16) + e] and B[8*(l/16) + e][l%16], e = 0..7,
// and holds C[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 (raw bits) -> fp32, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// fp32 pair -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// A wave-uniform 64-bit value.  readfirstlane works on 32 bits and returns a
// signed int, so each half goes through uint32_t (the low half must not be
// sign-extended into the high one).
__device__ __forceinline__ unsigned long long uniform_u64(unsigned long long x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((unsigned long long)hi << 32) | lo;
}

// LDS word read that completes before it returns.  Waves that have
// direct-to-LDS loads in flight read LDS through it: the compiler would make a
// plain LDS read wait for all of those loads.
__device__ __forceinline__ uint32_t lds_load_sync(const void* p) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(v)
                 : "v"((uint32_t)(uintptr_t)p)
                 : "memory");
    return v;
}

// The same for two adjacent words (8-byte aligned).
__device__ __forceinline__ u32x2_t lds_load2_sync(const void* p) {
    u32x2_t v;
    asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(v)
                 : "v"((uint32_t)(uintptr_t)p)
                 : "memory");
    return v;
}

// Workgroup barrier that orders LDS accesses only: global loads in flight
// (prefetches) are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroups are handed to the 8 XCDs round-robin (id % 8).  Give each XCD a
// contiguous range of logical work ids so that work sharing K/V lands on the
// same L2.
__device__ __forceinline__ int xcd_remap(int id, int n) {
    constexpr int kXcd = 8;
    const int q = n / kXcd, r = n % kXcd;
    const int xcd = id % kXcd, k = id / kXcd;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + k;
}

}  // namespace fsa
