// Device helpers shared by the relocation kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvr {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 16-byte global accesses.  Streaming traffic uses the nontemporal hint so
// the bulk rows do not evict the small, re-read tables from L2/MALL.
__device__ __forceinline__ v4u ld16(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
}
__device__ __forceinline__ void st16(char* p, v4u v) {
    __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(p));
}

// bf16 <-> f32.  Widening is exact (bf16 is the top half of an f32).
// Narrowing uses the hardware round-to-nearest-even pack (v_cvt_pk_bf16_f32),
// which also keeps NaN a NaN.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// One rotation pair in fp32: (xl, xh) -> (xl c - xh s, xl s + xh c).
__device__ __forceinline__ void rot2(float xl, float xh, float c, float s, float& yl, float& yh) {
    yl = fmaf(xl, c, -(xh * s));
    yh = fmaf(xl, s, xh * c);
}

// Rotate the 8 bf16 pairs held in a 16-byte "lo" chunk (x_j..x_{j+7}) and its
// "hi" partner (x_{j+h}..x_{j+h+7}); cs[e] = (cos, sin) of pair j+e.
__device__ __forceinline__ void rot_bf16x8(v4u& lo, v4u& hi, const float2* cs) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float2 c0 = cs[2 * w], c1 = cs[2 * w + 1];
        float a0, b0, a1, b1;
        rot2(bf_lo(lo[w]), bf_lo(hi[w]), c0.x, c0.y, a0, b0);
        rot2(bf_hi(lo[w]), bf_hi(hi[w]), c1.x, c1.y, a1, b1);
        lo[w] = pack_bf16(a0, a1);
        hi[w] = pack_bf16(b0, b1);
    }
}

// Same for 4 fp32 pairs per 16-byte chunk.
__device__ __forceinline__ void rot_f32x4(v4u& lo, v4u& hi, const float2* cs) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float a, b;
        rot2(__uint_as_float(lo[w]), __uint_as_float(hi[w]), cs[w].x, cs[w].y, a, b);
        lo[w] = __float_as_uint(a);
        hi[w] = __float_as_uint(b);
    }
}

// (cos, sin) of the angle shift * theta_j for j < n_pairs, written to LDS by
// the first n_pairs threads.  omega_j = theta_j / (2 pi) is the frequency in
// revolutions per position (float64).  The angle is reduced in float64:
// u = shift * omega_j (relative error ~2^-52), and its fractional part
// f = u - rint(u) in [-1/2, 1/2] is exact.  Only the reduced angle 2 pi f,
// |2 pi f| <= pi, goes to float32 sincos, so the error stays ~2e-7 absolute at
// any |shift| (a float32 product shift * theta would lose ~|shift| * 2^-24 rad).
// The caller must __syncthreads() before reading `cs`.  angle_table_from
// takes omega[tid] already loaded (so that a kernel can request it before
// its row loads and not wait behind them).
__device__ __forceinline__ void angle_table_from(float2* cs, double omega_tid, int n_pairs, int shift, int tid) {
    if (tid < n_pairs) {
        const double u = (double)shift * omega_tid;
        const double f = u - rint(u);
        float s, c;
        sincosf((float)(f * 6.283185307179586476925), &s, &c);
        cs[tid] = make_float2(c, s);
    }
}
__device__ __forceinline__ void angle_table(float2* cs, const double* omega, int n_pairs,
                                            int shift, int tid) {
    angle_table_from(cs, tid < n_pairs ? omega[tid] : 0.0, n_pairs, shift, tid);
}

// Workgroups reach the 8 XCDs round-robin (workgroup b runs on XCD b % 8,
// each with its own L2).  This remap gives each XCD a contiguous range of
// logical workgroup ids, so neighbouring logical workgroups share an L2.
__device__ __forceinline__ int xcd_contiguous(int b, int n) {
    const int x = b & 7, k = b >> 3, q = n >> 3, r = n & 7;
    return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// Relaxed device-scope atomics (coherent across the XCDs' L2 caches).
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every vector-memory load this thread issued has returned data.
// The "memory" clobber also keeps the compiler from sinking loads below it.
__device__ __forceinline__ void wait_loads() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace kvr
