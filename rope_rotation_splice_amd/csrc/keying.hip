// Registry keying of token streams (Irminsul, section 2.2): content-defined
// chunks cut by a Gear rolling hash over 64-token windows, fingerprinted with
// xxHash64, plus the S1 fallback's fixed windows inside each chunk.
//
// 1. gear_kernel: one thread per token.  The 64-bit Gear state shifts a
//    token's contribution out after 64 steps, so h_i is the sum over the
//    last 64 tokens of gear[tok] * 2^age: every position is computed
//    independently from a window of Gear values staged in LDS (Horner order,
//    oldest first, clipped at the stream start).  Candidates (h_i below the
//    threshold) become a bitmask, one wave ballot per 64 tokens.
// 2. cut_kernel: one wave per stream walks the chunk rule; the first
//    candidate in [p + min_len - 1, p + max_len - 1] is found by scanning 64
//    bitmask words (4096 tokens) per step.
// 3. fp_kernel: one thread per chunk computes xxHash64 of the chunk's token
//    ids (little-endian int32 bytes) and of its S1 windows.  xxHash64 follows
//    its published specification (XXH64: four lanes over 32-byte stripes,
//    merge, 8- and 4-byte tail steps, avalanche).
#include "kvr_device.h"
#include "kvr_internal.h"

#include "../../include/kvreloc.h"

namespace kvr {

__device__ uint32_t g_errors_keys;

namespace {

constexpr uint64_t P1 = 11400714785074694791ull;
constexpr uint64_t P2 = 14029467366897019727ull;
constexpr uint64_t P3 = 1609587929392839161ull;
constexpr uint64_t P4 = 9650029242287828579ull;
constexpr uint64_t P5 = 2870177450012600261ull;

__device__ __forceinline__ void raise_error(uint32_t bit) {
    __hip_atomic_fetch_or(&g_errors_keys, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t rotl64(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
__device__ __forceinline__ uint64_t xround(uint64_t acc, uint64_t lane) { return rotl64(acc + lane * P2, 31) * P1; }
__device__ __forceinline__ uint64_t xmerge(uint64_t acc, uint64_t v) { return (acc ^ xround(0, v)) * P1 + P4; }

// 8 bytes = two consecutive token ids, little-endian
__device__ __forceinline__ uint64_t two_tokens(const int32_t* t) {
    return (uint64_t)(uint32_t)t[0] | ((uint64_t)(uint32_t)t[1] << 32);
}

// xxHash64 of n token ids (4 n bytes)
__device__ uint64_t xxh64_tokens(const int32_t* t, int n, uint64_t seed) {
    int i = 0;
    uint64_t h;
    if (n >= 8) {
        uint64_t v1 = seed + P1 + P2, v2 = seed + P2, v3 = seed, v4 = seed - P1;
        for (; i + 8 <= n; i += 8) {
            v1 = xround(v1, two_tokens(t + i));
            v2 = xround(v2, two_tokens(t + i + 2));
            v3 = xround(v3, two_tokens(t + i + 4));
            v4 = xround(v4, two_tokens(t + i + 6));
        }
        h = rotl64(v1, 1) + rotl64(v2, 7) + rotl64(v3, 12) + rotl64(v4, 18);
        h = xmerge(h, v1);
        h = xmerge(h, v2);
        h = xmerge(h, v3);
        h = xmerge(h, v4);
    } else {
        h = seed + P5;
    }
    h += 4ull * (uint64_t)n;
    for (; i + 2 <= n; i += 2) {
        h ^= xround(0, two_tokens(t + i));
        h = rotl64(h, 27) * P1 + P4;
    }
    if (i < n) {
        h ^= (uint64_t)(uint32_t)t[i] * P1;
        h = rotl64(h, 23) * P2 + P3;
    }
    h ^= h >> 33;
    h *= P2;
    h ^= h >> 29;
    h *= P3;
    h ^= h >> 32;
    return h;
}

__device__ __forceinline__ int64_t stream_start(const KeyArgs& A, int64_t i) {
    int lo = 0, hi = A.n_streams - 1;        // last stream whose start <= i
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (A.offsets[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return A.offsets[lo];
}

__global__ __launch_bounds__(256) void gear_kernel(const KeyArgs A) {
    __shared__ uint64_t g[256 + 64];
    const int tid = threadIdx.x;
    const int64_t base = A.offsets[0] + (int64_t)blockIdx.x * 256;
    for (int j = tid; j < 320; j += 256) {
        const int64_t p = base - 64 + j;
        uint64_t v = 0;
        if (p >= A.offsets[0] && p < A.total) {
            const int32_t t = A.tokens[p];
            if ((uint32_t)t < (uint32_t)A.vocab) v = A.gear[t];
            else if (j >= 64) raise_error(KVR_DEV_BAD_TOKEN);      // reported once, by its own tile
        }
        g[j] = v;
    }
    __syncthreads();
    const int64_t i = base + tid;
    bool cand = false;
    if (i < A.total) {
        const int kmax = (int)min<int64_t>(63, i - stream_start(A, i));
        uint64_t h = 0;
        for (int k = kmax; k >= 0; --k) h = (h << 1) + g[tid + 64 - k];
        if (A.hash) A.hash[i] = h;
        cand = h < A.threshold;
    }
    const uint64_t m = __ballot(cand);
    const int64_t w0 = base + (tid & ~63);
    if ((tid & 63) == 0 && w0 < A.total) A.cand[(w0 - A.offsets[0]) >> 6] = m;
}

__global__ __launch_bounds__(64) void cut_kernel(const KeyArgs A) {
    const int s = blockIdx.x, lane = threadIdx.x;
    const int64_t S = A.offsets[s], E = A.offsets[s + 1], O = A.offsets[0];
    int64_t p = S;
    int k = 0;
    while (p < E) {
        const int64_t lo = p + A.min_len - 1, hi = min(p + A.max_len, E) - 1;
        int64_t end = hi + 1;
        if (lo <= hi) {
            // bitmask words hold tokens O + 64 w .. O + 64 w + 63
            const int64_t wlo = (lo - O) >> 6, whi = (hi - O) >> 6;
            for (int64_t w0 = wlo; w0 <= whi; w0 += 64) {
                const int64_t w = w0 + lane;
                uint64_t bits = 0;
                if (w <= whi) {
                    bits = A.cand[w];
                    if (w == wlo) bits &= ~0ull << ((lo - O) & 63);
                    const int top = (int)((hi - O) & 63);
                    if (w == whi && top < 63) bits &= (2ull << top) - 1;
                }
                const uint64_t any = __ballot(bits != 0);
                if (any) {
                    const int first = __ffsll((unsigned long long)any) - 1;
                    const uint32_t blo = __shfl((uint32_t)bits, first), bhi = __shfl((uint32_t)(bits >> 32), first);
                    const uint64_t fb = (uint64_t)blo | ((uint64_t)bhi << 32);
                    end = O + ((w0 + first) << 6) + (__ffsll((unsigned long long)fb) - 1) + 1;
                    break;
                }
            }
        }
        if (k >= A.cap) {                    // cannot happen with a valid cap
            if (lane == 0) raise_error(KVR_DEV_RANGE);
            break;
        }
        if (lane == 0) A.chunk_end[(int64_t)s * A.cap + k] = (int32_t)(end - S);
        ++k;
        p = end;
    }
    if (lane == 0) A.n_chunks[s] = k;
}

__global__ __launch_bounds__(256) void fp_kernel(const KeyArgs A) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t s = gid / A.cap;
    const int k = (int)(gid - s * A.cap);
    if (s >= A.n_streams || k >= A.n_chunks[s]) return;
    const int32_t* ce = A.chunk_end + s * A.cap;
    const int start = k == 0 ? 0 : ce[k - 1], end = ce[k];
    const int32_t* t = A.tokens + A.offsets[s];
    A.chunk_fp[s * A.cap + k] = xxh64_tokens(t + start, end - start, A.seed);
    if (A.s1_fp) {
        uint64_t* o = A.s1_fp + (s * A.cap + k) * A.s1_slots;
        for (int w = 0; w < A.s1_slots; ++w) {
            const int a = start + w * A.s1_window;
            o[w] = a < end ? xxh64_tokens(t + a, min(A.s1_window, end - a), A.seed) : 0;
        }
    }
}

}  // namespace

hipError_t launch_keys(const KeyArgs& a, hipStream_t s) {
    if (a.n_streams <= 0) return hipSuccess;
    const int64_t n = a.total - a.offsets[0];
    if (n > 0) {
        hipLaunchKernelGGL(gear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(cut_kernel, dim3(a.n_streams), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t slots = (int64_t)a.n_streams * a.cap;
    hipLaunchKernelGGL(fp_kernel, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

uint32_t read_and_clear_errors_keys() {
    uint32_t v = 0, z = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_errors_keys), sizeof(v)) != hipSuccess) return 0xffffffffu;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_errors_keys), &z, sizeof(z)) != hipSuccess) return 0xffffffffu;
    return v;
}

}  // namespace kvr
