// Device-side helpers shared by the RAT+ kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rat {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// bf16 <-> fp32.  bf16 -> fp32 is exact (a shift); fp32 -> bf16 rounds to
// nearest even in hardware (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

// Forget gate and its complement for a logit l: g = 1/(1+e^-l), 1-g = 1/(1+e^l),
// with one exp2 and one reciprocal.  Working from e = e^-|l| in [0, 1] keeps
// both outputs free of cancellation and exact at l = +-inf ((1,0) / (0,1)).
__device__ __forceinline__ void forget_gate(float logit, float& g, float& gbar)
{
    const float e = __builtin_amdgcn_exp2f(-fabsf(logit) * kLog2e);
    const float s = __builtin_amdgcn_rcpf(1.0f + e);
    const float es = e * s;
    const bool pos = logit >= 0.0f;
    g = pos ? s : es;
    gbar = pos ? es : s;
}

// The forget gate alone, g = 1/(1 + 2^(-l log2 e)): exactly 0 at l = -inf
// and 1 at l = +inf.  With h = x + g (h - x) -- the same recurrence as
// g h + (1 - g) x -- the complement is never formed.
__device__ __forceinline__ float gate(float logit)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-logit * kLog2e));
}

// Relaxed agent-scope atomics: each 64-bit word carries (value bits, tag) and
// validates itself, so no fence is needed between producer and consumer.
__device__ __forceinline__ void store_tagged(uint64_t* p, float v, uint32_t tag)
{
    uint32_t bits = __float_as_uint(v);
    if ((bits & 0x7fffffffu) > 0x7f800000u) bits = 0x7fc00000u;  // canonical NaN
    __hip_atomic_store(p, ((uint64_t)tag << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool load_tagged(const uint64_t* p, uint32_t tag, float& v)
{
    uint64_t w = __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    v = __uint_as_float((uint32_t)w);
    return (uint32_t)(w >> 32) == tag;
}

// LDS buffers are addressed through generic pointers into the workgroup's
// shared arrays (the compiler keeps them in the LDS address space); the
// builtins that need an explicit LDS pointer get one by an address-space cast.
typedef char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

// vmcnt-only wait (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14])
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at dst + 16 l, dst being wave-uniform (M0).  It is
// issued from inline assembly so that the compiler does not track it as an
// LDS write: its own tracking cannot tell the ring buffers apart and would
// wait for every load in flight before each LDS read.  Completion is
// awaited explicitly (wait_vmcnt + barrier) before the data is read; the
// instruction returns no registers.
__device__ __forceinline__ void dma16(const void* gptr, lds_char* dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)dst);
    // (s_nop: the wait state between the scalar write of M0 and the LDS
    // copy that reads it, which the compiler cannot see inside the asm)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(m0) : "memory");
}

// N global_load_lds_dwordx4 copies issued back to back under one M0 (four
// at most per M0: the immediate offset reaches 4095).  Copy j reads 16
// bytes per lane at base[j] + voff[j] + 1024 (j mod 4) and writes them to
// LDS at m0 + 1024 j + 16 lane: the instruction's immediate offset moves
// both addresses, so the caller passes base[j] already lowered by
// 1024 (j mod 4) and the copies need no M0 write of their own.  The hardware needs 5 wait
// states between a VALU write of an SGPR (a base moved from vector
// registers by readfirstlane) and a copy that reads it, and 1 between the
// write of M0 and the copy; the compiler does not see inside the asm, so
// its leading s_nop provides both for the first copy (later copies' bases
// are older still).
// The bases are uniform by construction; readfirstlane states it to the
// compiler (free when a base already sits in scalar registers), so that a
// base its analysis takes for divergent still lands in scalar registers.
__device__ __forceinline__ uint64_t uniform64(uint64_t x)
{
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x);
    return ((uint64_t)hi << 32) | lo;
}

template <int N>
__device__ __forceinline__ void dma16_group(const uint64_t (&base)[N], const uint32_t (&voff)[N], uint32_t m0);

template <>
__device__ __forceinline__ void dma16_group<2>(const uint64_t (&base_in)[2], const uint32_t (&voff)[2], uint32_t m0)
{
    const uint64_t base[2] = {uniform64(base_in[0]), uniform64(base_in[1])};
    asm volatile("s_nop 4\n\t"
                 "global_load_lds_dwordx4 %0, %2\n\t"
                 "global_load_lds_dwordx4 %1, %3 offset:1024"
                 ::"v"(voff[0]), "v"(voff[1]), "s"(base[0]), "s"(base[1]), "{m0}"(m0) : "memory");
}

template <>
__device__ __forceinline__ void dma16_group<4>(const uint64_t (&base_in)[4], const uint32_t (&voff)[4], uint32_t m0)
{
    const uint64_t base[4] = {uniform64(base_in[0]), uniform64(base_in[1]), uniform64(base_in[2]),
                              uniform64(base_in[3])};
    asm volatile("s_nop 4\n\t"
                 "global_load_lds_dwordx4 %0, %4\n\t"
                 "global_load_lds_dwordx4 %1, %5 offset:1024\n\t"
                 "global_load_lds_dwordx4 %2, %6 offset:2048\n\t"
                 "global_load_lds_dwordx4 %3, %7 offset:3072"
                 ::"v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]),
                   "s"(base[0]), "s"(base[1]), "s"(base[2]), "s"(base[3]), "{m0}"(m0) : "memory");
}

// Eight copies: two groups of four under M0 and M0 + 4096 (each base
// lowered by 1024 (j mod 4) for its immediate offset).
template <>
__device__ __forceinline__ void dma16_group<8>(const uint64_t (&base_in)[8], const uint32_t (&voff)[8], uint32_t m0)
{
    const uint64_t b0[4] = {base_in[0], base_in[1], base_in[2], base_in[3]};
    const uint64_t b1[4] = {base_in[4], base_in[5], base_in[6], base_in[7]};
    const uint32_t v0[4] = {voff[0], voff[1], voff[2], voff[3]};
    const uint32_t v1[4] = {voff[4], voff[5], voff[6], voff[7]};
    dma16_group<4>(b0, v0, m0);
    dma16_group<4>(b1, v1, m0 + 4096);
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads()
// it does not wait for outstanding global memory operations, so direct
// global -> LDS copies stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 16 bytes of one token row: CPL = 16 / sizeof(E) adjacent channels.
template <typename E> struct Row16;
template <> struct Row16<uint16_t> {
    static constexpr int CPL = 8;
    static __device__ __forceinline__ float get(const u32x4& r, int j)
    {
        return (j & 1) ? bf16_hi(r[j >> 1]) : bf16_lo(r[j >> 1]);
    }
    static __device__ __forceinline__ u32x4 pack(const float (&x)[8])
    {
        return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7])};
    }
};
template <> struct Row16<float> {
    static constexpr int CPL = 4;
    static __device__ __forceinline__ float get(const u32x4& r, int j) { return __uint_as_float(r[j]); }
    static __device__ __forceinline__ u32x4 pack(const float (&x)[4])
    {
        return u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
    }
};

// A compile-time bool for the two forms of a kernel's inner loops.
template <bool B> struct BoolC { static constexpr bool value = B; };

}  // namespace rat
