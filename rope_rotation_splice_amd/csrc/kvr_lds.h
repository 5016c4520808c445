// LDS and direct-load helpers shared by the decode kernels (device code only).
#pragma once

#include "kvr_device.h"

namespace kvr {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) v4u lds_v4u;
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2u lds_v2u;

__device__ __forceinline__ v8bf as_bf(v4u x) { return __builtin_bit_cast(v8bf, x); }

// LDS accesses at byte offsets (the swizzled addresses are formed as integers)
__device__ __forceinline__ v4u lds16_at(uint32_t off) { return *(const lds_v4u*)(size_t)off; }
__device__ __forceinline__ v2u lds8_at(uint32_t off) { return *(const lds_v2u*)(size_t)off; }
__device__ __forceinline__ void lds8_put(uint32_t off, v2u v) { *(lds_v2u*)(size_t)off = v; }
__device__ __forceinline__ v4s lds_tr_at(uint32_t off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(size_t)off);
}

// A pointer the whole wave agrees on, in scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const char*)(((uint64_t)hi << 32) | lo);
}

// One direct global -> LDS load: lane l reads 16 bytes at base + off (base
// wave-uniform, off per lane) and they land at LDS address lds + 16 l.  M0
// carries the (wave-uniform) LDS address; the compiler sets M0 itself before
// every use it makes, so the value left here is never relied upon.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Combine the values of lanes l and l ^ 32 (v_permlane32_swap leaves one
// copy of each half's value in each of its two results).
__device__ __forceinline__ float max_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace
}  // namespace kvr
