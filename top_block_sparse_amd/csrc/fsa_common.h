// fsa_common.h -- shared device helpers for the gfx950 kernels of libfsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

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

// The tokens of m-tile c of a tile of ntok tokens with G query rows each
// (its 16 rows hold tokens 16c/G .. (16c+15)/G), as a bit mask; 0 for
// c >= mtiles.  A union builder computes it once per tile, for c = lane.
__device__ __forceinline__ unsigned long long mtile_token_mask(int c, int G, int ntok, int mtiles) {
    if (c >= mtiles) return 0ull;
    const int tf = (c * 16) / G;
    int tl = (c * 16 + 15) / G;
    tl = tl < ntok - 1 ? tl : ntok - 1;
    const unsigned long long hi = tl >= 63 ? ~0ull : ((1ull << (tl + 1)) - 1ull);
    return tf > tl ? 0ull : (hi & ~((1ull << tf) - 1ull));
}

// The number of m-tiles with a token in m, from the per-lane masks above
// (lane c holds m-tile c's).
__device__ __forceinline__ int mtiles_meeting(unsigned long long m, unsigned long long cm_lane,
                                              int mtiles) {
    int nc = 0;
    for (int c = 0; c < mtiles; ++c) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)cm_lane, c);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(cm_lane >> 32), c);
        nc += (m & (((unsigned long long)hi << 32) | lo)) != 0ull ? 1 : 0;
    }
    return nc;
}

// Bounded waits of the LDS ring protocols.  Every wait polls at most
// `limit` times (a consistent protocol never comes close), so a protocol
// error can only give wrong values, never a hung GPU.  A wait that runs out
// returns false, adds one to the kernel file's device counter of timeouts
// (lane 0, a vector global atomic; the host reads it back with
// fsa_wait_timeouts), raises the workgroup's abort word and lowers the
// wave's own limit to one poll.  A wave still waiting looks at the abort
// word every 1024 polls and gives up too (without counting), so one
// protocol error costs a workgroup about one full wait, not one per block.
// The wave-uniform limit is the loops' only extra live state: a sticky
// per-lane flag and an abort check every 256 polls cost the ring kernels
// 6-8 % (the extra state spilled scalar registers into their loops).
__device__ __forceinline__ void note_wait_timeout(unsigned int* counter, uint32_t* abort_word,
                                                  int& limit, int lane) {
    if (lane == 0) {
        __hip_atomic_store(abort_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    limit = 1;
}

// Wait until two adjacent ready words (one per producer) both reach `target`.
__device__ __forceinline__ bool wait_ready2(const uint32_t* ready, uint32_t target,
                                            unsigned int* counter, uint32_t* abort_word,
                                            int& limit, int lane) {
    for (int sp = 0; sp < limit; ++sp) {
        const u32x2_t r = lds_load2_sync(ready);
        if (r[0] >= target && r[1] >= target) return true;
        if ((sp & 1023) == 1023 && lds_load_sync(abort_word) != 0u) {
            limit = 1;
            return false;
        }
        __builtin_amdgcn_s_sleep(4);
    }
    note_wait_timeout(counter, abort_word, limit, lane);
    return false;
}

// Wait until a done counter reaches `target` (producers: the slot is free).
__device__ __forceinline__ bool wait_done(const uint32_t* done, uint32_t target,
                                          unsigned int* counter, uint32_t* abort_word, int& limit,
                                          int lane) {
    for (int sp = 0; sp < limit; ++sp) {
        if (lds_load_sync(done) >= target) return true;
        if ((sp & 1023) == 1023 && lds_load_sync(abort_word) != 0u) {
            limit = 1;
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    note_wait_timeout(counter, abort_word, limit, lane);
    return false;
}

// Raise a kernel's dynamic LDS limit to 160 KiB on the calling thread's
// current device.  The runtime keeps the attribute per device, so `done`
// holds one bit per device id (< 64) on which it has been set; racing
// threads set the same value.
inline hipError_t ensure_lds_limit(const void* fn, std::atomic<unsigned long long>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = (dev >= 0 && dev < 64) ? 1ull << dev : 0ull;
    if (bit != 0ull && (done.load(std::memory_order_acquire) & bit) != 0ull) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e == hipSuccess && bit != 0ull) done.fetch_or(bit, std::memory_order_release);
    return e;
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
