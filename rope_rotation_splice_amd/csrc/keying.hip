// Registry keying of token streams (Irminsul, section 2.2): content-defined
// chunks cut by a Gear rolling hash over 64-token windows, fingerprinted with
// xxHash64, plus the S1 fallback's fixed windows inside each chunk.
//
// 1. gear_kernel: one lane per token.  The 64-bit Gear state shifts a
//    token's contribution out after 64 steps, so h_i is the sum over the
//    last 64 tokens of gear[tok] * 2^age (clipped at the stream start).  A
//    64-token tile is a segmented scan under (a, b) -> (a << d) + b, six
//    shift-add steps across the wave (DPP row shifts, then row broadcasts)
//    that restart at stream starts, plus the
//    previous tile's last h shifted by lane + 1 where no start intervenes.
//    Candidates (h_i below the threshold) become a bitmask, one wave ballot
//    per 64 tokens.
// 2. cut_kernel: one wave per stream walks the chunk rule (the first
//    candidate in [p + min_len - 1, p + max_len - 1] ends the chunk from p).
//    The chunk that follows each candidate is found for all candidates at
//    once, so the walk reads one table entry per chunk; streams with too many
//    candidates or too long for the LDS window scan 64 bitmask words per step
//    instead.
// 3. fp_kernel: one wave per chunk computes xxHash64 of its tokens' ids
//    (little-endian int32 bytes) and of its S1 windows, four lanes (the four
//    stripe accumulators) per hash, 16 hashes side by side.  xxHash64 follows
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

// Starting value of stripe accumulator a (0..3).
__device__ __forceinline__ uint64_t xxh_init(int a, uint64_t seed) {
    return a == 0 ? seed + P1 + P2 : a == 1 ? seed + P2 : a == 2 ? seed : seed - P1;
}

__device__ __forceinline__ uint64_t xxh_converge(uint64_t v1, uint64_t v2, uint64_t v3, uint64_t v4) {
    uint64_t h = rotl64(v1, 1) + rotl64(v2, 7) + rotl64(v3, 12) + rotl64(v4, 18);
    h = xmerge(h, v1);
    h = xmerge(h, v2);
    h = xmerge(h, v3);
    return xmerge(h, v4);
}

// Length, the rem (< 8 after the stripes) trailing token ids at t, avalanche.
__device__ __forceinline__ uint64_t xxh_tail(uint64_t h, const int32_t* t, int rem, int n) {
    h += 4ull * (uint64_t)n;
    int i = 0;
    for (; i + 2 <= rem; i += 2) {
        h ^= xround(0, two_tokens(t + i));
        h = rotl64(h, 27) * P1 + P4;
    }
    if (i < rem) {
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

// Each wave takes kGearTiles consecutive 64-token tiles (one position per
// lane), after one warm-up tile that only supplies the carry-in.  All the
// span's token ids and Gear values are loaded before the scans.
constexpr int kGearTiles = 8;

// A 64-bit DPP move: lane i takes the value the DPP control names (0 where
// its source lane is outside the row or the wave).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, true);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
    return (uint64_t)lo | ((uint64_t)hi << 32);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return (uint64_t)lo | ((uint64_t)hi << 32);
}

__global__ __launch_bounds__(256) void gear_kernel(const KeyArgs A) {
    // the stream starts, staged in LDS: the searches below read them there
    // instead of through the scalar cache
    __shared__ int64_t s_off[kKeyMaxStreams + 1];
    for (int i = threadIdx.x; i <= A.n_streams; i += 256) s_off[i] = A.offsets[i];
    const int lane = threadIdx.x & 63;
    const int64_t O = A.offsets[0];
    const int64_t ntiles = (A.total - O + 63) >> 6;
    const int64_t t0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kGearTiles;
    __syncthreads();
    if (t0 >= ntiles) return;
    const int64_t tw = t0 > 0 ? t0 - 1 : 0;  // first tile scanned (the warm-up one unless t0 == 0)
    const int nt = (int)(min<int64_t>(t0 + kGearTiles, ntiles) - tw);
    // Loads are unconditional (addresses clamped into range, values masked
    // afterwards) so that all of them are in flight together.
    int32_t tk[kGearTiles + 1];
    uint64_t gv[kGearTiles + 1];
#pragma unroll
    for (int j = 0; j < kGearTiles + 1; ++j) {
        const int64_t i = O + ((tw + j) << 6) + lane;
        tk[j] = A.tokens[min(i, A.total - 1)];
    }
#pragma unroll
    for (int j = 0; j < kGearTiles + 1; ++j)
        gv[j] = A.gear[(uint32_t)tk[j] < (uint32_t)A.vocab ? tk[j] : 0];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kGearTiles + 1; ++j) {
        const int64_t i = O + ((tw + j) << 6) + lane;
        const bool in = j < nt && i < A.total;
        const bool ok = (uint32_t)tk[j] < (uint32_t)A.vocab;
        if (!(in && ok)) gv[j] = 0;
        bad |= in && !ok && tw + j >= t0;    // reported by the span that owns the tile
    }
    if (bad) raise_error(KVR_DEV_BAD_TOKEN);
    // first stream start at or after the first scanned tile
    const int64_t first = O + (tw << 6);
    int sidx = 0, shi = A.n_streams;
    while (sidx < shi) {
        const int mid = (sidx + shi) >> 1;
        if (s_off[mid] < first) sidx = mid + 1; else shi = mid;
    }
    uint64_t carry = 0;                      // h just before the tile
#pragma unroll
    for (int j = 0; j < kGearTiles + 1; ++j) {
        if (j < nt) {
            const int64_t tile0 = O + ((tw + j) << 6);
            uint64_t F = 0;                      // stream starts inside the tile
            while (sidx < A.n_streams && s_off[sidx] < tile0 + 64) {
                F |= 1ull << (s_off[sidx] - tile0);
                ++sidx;
            }
            const uint64_t m = lane == 63 ? F : F & ((2ull << lane) - 1);
            const int hd = m ? 63 - __clzll((long long)m) : -1;    // this position's stream start in the tile
            // segmented scan: v = sum over [max(hd, 0), lane] of g_j 2^(lane - j)
            // within each 16-lane row by row shifts (row_shr 1, 2, 4, 8), then
            // across rows: lane 15 of rows 0 and 2 into rows 1 and 3
            // (row_bcast 15), lane 31 into rows 2 and 3 (row_bcast 31); a
            // source before this position's stream start adds nothing
            uint64_t v = gv[j];
            const int li = lane & 15;
            { const uint64_t u = dpp64<0x111>(v); if (li >= 1 && lane - 1 >= hd) v += u << 1; }
            { const uint64_t u = dpp64<0x112>(v); if (li >= 2 && lane - 2 >= hd) v += u << 2; }
            { const uint64_t u = dpp64<0x114>(v); if (li >= 4 && lane - 4 >= hd) v += u << 4; }
            { const uint64_t u = dpp64<0x118>(v); if (li >= 8 && lane - 8 >= hd) v += u << 8; }
            {
                const uint64_t u = dpp64<0x142>(v);
                const int src = (lane & ~15) - 1;
                if (((lane >> 4) & 1) && src >= hd) v += u << (lane - src);
            }
            { const uint64_t u = dpp64<0x143>(v); if (lane >= 32 && 31 >= hd) v += u << (lane - 31); }
            if (hd < 0 && lane < 63) v += carry << (lane + 1);
            carry = readlane64(v, 63);
            if (tw + j >= t0) {
                const int64_t i = tile0 + lane;
                const bool ok = i < A.total;
                if (A.hash && ok) A.hash[i] = v;
                const uint64_t bm = __ballot(ok && v < A.threshold);
                if (lane == 0) A.cand[(tile0 - O) >> 6] = bm;
            }
        }
    }
}

// The walk reads the stream's bitmask from an LDS window of kCutWords words.
// A stream whose bitmask fits the window and has at most kCutCands
// candidates is walked through a table: for every candidate c, the chunk end
// that follows a cut at c (the first candidate in [c + min_len, c + max_len],
// plus one, else the forced end) is found in parallel by binary search over
// the sorted candidate positions, and the walk then reads one table entry per
// chunk.  Other streams take the scan: from the window, refilled (coalesced)
// whenever it needs words past it, 64 words per step by ballot.  Positions
// are 32-bit and relative to the stream start (a stream is shorter than 2^31
// tokens); the walk's state stays wave-uniform.
constexpr int kCutWords = 4096;
constexpr int kCutCands = 4096;

__global__ __launch_bounds__(64) void cut_kernel(const KeyArgs A) {
    __shared__ uint64_t win[kCutWords];
    __shared__ int32_t cpos[kCutCands];      // candidate token positions, ascending
    __shared__ int2 cnext[kCutCands];        // after a cut at candidate i: (next candidate or -1, its chunk end)
    const int s = blockIdx.x, lane = threadIdx.x;
    const int64_t O = A.offsets[0], S = A.offsets[s];
    const int L = (int)(A.offsets[s + 1] - S);
    const int64_t ws = (S - O) >> 6;         // first bitmask word of the stream
    const int sh = (int)((S - O) & 63);      // bit of the stream's first token in it
    const int wlast = L > 0 ? (sh + L - 1) >> 6 : -1;    // last word, stream-relative
    const int minl = A.min_len, maxl = A.max_len;
    int32_t* ce = A.chunk_end + (int64_t)s * A.cap;
    int p = 0, k = 0;

    // ---- table walk -----------------------------------------------------------
    int nc = -1;                             // candidates, or -1: take the scan
    if (L > 0 && wlast < kCutWords) {
        // the stream's words, bits outside [0, L) cleared
        for (int w = lane; w <= wlast; w += 64) {
            uint64_t v = A.cand[ws + w];
            if (w == 0) v &= ~0ull << sh;
            const int top = (sh + L - 1) & 63;
            if (w == wlast && top < 63) v &= (2ull << top) - 1;
            win[w] = v;
        }
        __syncthreads();
        // lane l counts words [l m, (l + 1) m), then writes their candidates in order
        const int m = (wlast + 64) >> 6;
        const int w0 = lane * m, w1 = min(w0 + m, wlast + 1);
        int cnt = 0;
        for (int w = w0; w < w1; ++w) cnt += __popcll(win[w]);
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(incl, d);
            if (lane >= d) incl += u;
        }
        nc = __shfl(incl, 63);
        if (nc <= kCutCands) {
            int o = incl - cnt;
            for (int w = w0; w < w1; ++w) {
                uint64_t v = win[w];
                while (v) {
                    const int bit = __ffsll((unsigned long long)v) - 1;
                    v &= v - 1;
                    cpos[o++] = (w << 6) + bit - sh;
                }
            }
            __syncthreads();
            // first candidate index >= x among [from, nc)
            auto first_at = [&](int from, int x) __attribute__((always_inline)) {
                int lo = from, hi = nc;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (cpos[mid] < x) lo = mid + 1; else hi = mid;
                }
                return lo;
            };
            // the chunk that starts at q: (its ending candidate or -1, its end)
            auto chunk_from = [&](int q, int from) __attribute__((always_inline)) -> int2 {
                const int lo = q + minl - 1, hi = min(q + maxl, L) - 1;
                if (lo > hi) return make_int2(-1, hi + 1);
                const int j = first_at(from, lo);
                if (j < nc && cpos[j] <= hi) return make_int2(j, cpos[j] + 1);
                return make_int2(-1, hi + 1);
            };
            for (int i = lane; i < nc; i += 64) cnext[i] = chunk_from(cpos[i] + 1, i + 1);
            __syncthreads();
            // the walk: a table entry per chunk after a candidate cut, a search
            // after the start and after a forced cut.  Chunk ends collect in
            // LDS (the window's words are no longer needed) and leave in
            // coalesced batches.
            int32_t* ends = reinterpret_cast<int32_t*>(win);
            constexpr int kEnds = kCutWords * 2;
            int nb = 0, kb = 0;
            auto flush = [&]() __attribute__((always_inline)) {
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                for (int i = lane; i < nb; i += 64) ce[kb + i] = ends[i];
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                kb += nb;
                nb = 0;
            };
            // (the walk's state in scalar registers)
            const int2 c0 = chunk_from(0, 0);
            int cx = __builtin_amdgcn_readfirstlane(c0.x), cy = __builtin_amdgcn_readfirstlane(c0.y);
            while (p < L) {
                if (k >= A.cap) {            // cannot happen with a valid cap
                    if (lane == 0) raise_error(KVR_DEV_RANGE);
                    break;
                }
                ends[nb] = cy;               // every lane writes the same value
                ++nb;
                ++k;
                p = cy;
                if (nb == kEnds) flush();
                if (p >= L) break;
                const int2 v = cx >= 0 ? cnext[cx] : chunk_from(p, 0);
                cx = __builtin_amdgcn_readfirstlane(v.x);
                cy = __builtin_amdgcn_readfirstlane(v.y);
            }
            flush();
        }
        __syncthreads();                     // the scan below refills the window
    }

    // ---- scan walk --------------------------------------------------------------
    if (nc < 0 || nc > kCutCands) {
        int wb = -kCutWords;                 // first word held in win (none yet)
        while (p < L) {
            const int lo = p + minl - 1, hi = min(p + maxl, L) - 1;
            int end = hi + 1;
            if (lo <= hi) {
                const int wlo = (sh + lo) >> 6, whi = (sh + hi) >> 6;
                const int blo = (sh + lo) & 63, bhi = (sh + hi) & 63;
                for (int w0 = wlo; w0 <= whi; w0 += 64) {
                    if (w0 < wb || w0 + 64 > wb + kCutWords) {
                        __syncthreads();
                        // 16 loads in flight per lane; batches past the stream's end are skipped
                        for (int j0 = 0; j0 < kCutWords && w0 + j0 <= wlast; j0 += 64 * 16) {
                            uint64_t r[16];
#pragma unroll
                            for (int i = 0; i < 16; ++i) {   // clamped: unconditional loads
                                const int j = j0 + 64 * i + lane;
                                r[i] = A.cand[ws + min(w0 + j, wlast)];
                                if (w0 + j > wlast) r[i] = 0;
                            }
#pragma unroll
                            for (int i = 0; i < 16; ++i) win[j0 + 64 * i + lane] = r[i];
                        }
                        __syncthreads();
                        wb = w0;
                    }
                    const int w = w0 + lane;
                    uint64_t bits = 0;
                    if (w <= whi) {
                        bits = win[w - wb];
                        if (w == wlo) bits &= ~0ull << blo;
                        if (w == whi && bhi < 63) bits &= (2ull << bhi) - 1;
                    }
                    const uint64_t any = __ballot(bits != 0);
                    if (any) {
                        const int first = __ffsll((unsigned long long)any) - 1;
                        const uint32_t flo = __builtin_amdgcn_readlane((int)(uint32_t)bits, first);
                        const uint32_t fhi = __builtin_amdgcn_readlane((int)(uint32_t)(bits >> 32), first);
                        const int bit = flo ? __ffs(flo) - 1 : 31 + __ffs(fhi);
                        end = ((w0 + first) << 6) + bit - sh + 1;
                        break;
                    }
                }
            }
            if (k >= A.cap) {                // cannot happen with a valid cap
                if (lane == 0) raise_error(KVR_DEV_RANGE);
                break;
            }
            if (lane == 0) ce[k] = end;
            ++k;
            p = end;
        }
    }
    if (lane == 0) A.n_chunks[s] = k;
}

// One wave per chunk.  Each workgroup first scans n_chunks into a prefix in
// LDS, then takes chunks g = blockIdx.x, blockIdx.x + gridDim.x, ... of the
// concatenated chunk list, so the work is spread evenly whatever the chunk
// counts per stream.  A chunk's hashes are items: item 0 the chunk, item
// 1 + w its S1 window w.  Each item takes four lanes, one per stripe
// accumulator, so a pass runs 16 items side by side.  The pass's token range
// is staged in LDS kFpPiece tokens at a time, with kFpHalo tokens on either
// side so that a stripe starting in the piece, and a tail ending in it, read
// only staged tokens.  An item is finished (accumulators merged, tail,
// avalanche) in the piece that holds its last token.
constexpr int kFpPiece = 2048;
constexpr int kFpHalo = 8;
constexpr int kFpGrid = 4096;
constexpr int kFpUnroll = 8;            // stripes whose words are read ahead of their rounds

__global__ __launch_bounds__(64) void fp_kernel(const KeyArgs A) {
    __shared__ int32_t buf[kFpPiece + 2 * kFpHalo];
    __shared__ int pre[kKeyMaxStreams + 1];
    const int lane = threadIdx.x, acc = lane & 3, grp = lane >> 2;
    int carry = 0;
    for (int s0 = 0; s0 < A.n_streams; s0 += 64) {
        int v = s0 + lane < A.n_streams ? A.n_chunks[s0 + lane] : 0;
        for (int dd = 1; dd < 64; dd <<= 1) {
            const int u = __shfl_up(v, dd);
            if (lane >= dd) v += u;
        }
        if (s0 + lane < A.n_streams) pre[s0 + lane + 1] = carry + v;
        carry += __shfl(v, 63);
    }
    if (lane == 0) pre[0] = 0;
    __syncthreads();
    const int total = pre[A.n_streams];
    const int W = A.s1_window;
    for (int g = blockIdx.x; g < total; g += gridDim.x) {
        int s = 0, hi = A.n_streams - 1;        // last stream with pre[s] <= g
        while (s < hi) {
            const int mid = (s + hi + 1) >> 1;
            if (pre[mid] <= g) s = mid; else hi = mid - 1;
        }
        const int k = g - pre[s];
        const int64_t c = (int64_t)s * A.cap + k;
        const int32_t* ce = A.chunk_end + (int64_t)s * A.cap;
        const int start = k == 0 ? 0 : ce[k - 1];
        const int len = ce[k] - start;
        const int32_t* t = A.tokens + A.offsets[s] + start;
        const int nw = A.s1_fp ? min(A.s1_slots, (len + W - 1) / W) : 0;
        const int items = 1 + nw;
        for (int i0 = 0; i0 < items; i0 += 16) {
            const int it = i0 + grp;
            const bool act = it < items;
            const int st = !act || it == 0 ? 0 : (it - 1) * W;            // item's first token
            const int nt = !act ? 0 : it == 0 ? len : min(W, len - st);   // and its length
            const int ns = nt >> 3;                                       // whole stripes
            const int last = st + nt - 1;
            const int ilast = min(items, i0 + 16) - 1;
            const int r0 = i0 == 0 ? 0 : (i0 - 1) * W;                    // the pass's token range
            const int r1 = i0 == 0 ? len : min(len, ilast * W);
            uint64_t v = xxh_init(acc, A.seed);
            for (int base = r0; base < r1; base += kFpPiece) {
                const int lo = max(0, base - kFpHalo), hi2 = min(len, base + kFpPiece + kFpHalo);
                int32_t* b0 = buf + kFpHalo - base;                       // b0[x] holds token x
                __syncthreads();
                for (int j0 = 0; j0 < hi2 - lo; j0 += 64 * 8) {          // 8 loads in flight per lane
                    int32_t r[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) r[i] = t[min(lo + j0 + 64 * i + lane, hi2 - 1)];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int x = lo + j0 + 64 * i + lane;
                        if (x < hi2) b0[x] = r[i];
                    }
                }
                __syncthreads();
                const int d0 = base - st, d1 = base + kFpPiece - st;
                const int q0 = d0 <= 0 ? 0 : (d0 + 7) >> 3;
                const int q1 = d1 <= 0 ? 0 : min(ns, (d1 + 7) >> 3);
                // the lane words of kFpUnroll stripes are read from LDS before their
                // rounds run, so the dependent rounds do not wait on each read
                int q = q0;
                for (; q + kFpUnroll <= q1; q += kFpUnroll) {
                    uint64_t wv[kFpUnroll];
#pragma unroll
                    for (int u = 0; u < kFpUnroll; ++u) wv[u] = two_tokens(b0 + st + 8 * (q + u) + 2 * acc);
#pragma unroll
                    for (int u = 0; u < kFpUnroll; ++u) v = xround(v, wv[u]);
                }
                for (; q < q1; ++q) v = xround(v, two_tokens(b0 + st + 8 * q + 2 * acc));
                const uint32_t vlo = (uint32_t)v, vhi = (uint32_t)(v >> 32);
                uint64_t va[4];
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    va[b] = (uint64_t)__shfl(vlo, (lane & ~3) + b) | ((uint64_t)__shfl(vhi, (lane & ~3) + b) << 32);
                if (act && acc == 0 && last >= base && last < base + kFpPiece) {
                    uint64_t h = ns > 0 ? xxh_converge(va[0], va[1], va[2], va[3]) : A.seed + P5;
                    h = xxh_tail(h, b0 + st + 8 * ns, nt - 8 * ns, nt);
                    if (it == 0) A.chunk_fp[c] = h;
                    else A.s1_fp[c * A.s1_slots + (it - 1)] = h;
                }
            }
        }
        if (A.s1_fp)
            for (int w = nw + lane; w < A.s1_slots; w += 64) A.s1_fp[c * A.s1_slots + w] = 0;
    }
}

}  // namespace

hipError_t launch_keys(const KeyArgs& a, hipStream_t s) {
    if (a.n_streams <= 0) return hipSuccess;
    const int64_t n = a.total - a.offsets[0];
    if (n > 0) {
        const int64_t waves = ((n + 63) / 64 + kGearTiles - 1) / kGearTiles;
        hipLaunchKernelGGL(gear_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(cut_kernel, dim3(a.n_streams), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t slots = (int64_t)a.n_streams * a.cap;
    hipLaunchKernelGGL(fp_kernel, dim3((unsigned)std::min<int64_t>(slots, kFpGrid)), dim3(64), 0, s, a);
    return hipGetLastError();
}

uint32_t read_and_clear_errors_keys() {
    uint32_t v = 0, z = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_errors_keys), sizeof(v)) != hipSuccess) return 0xffffffffu;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_errors_keys), &z, sizeof(z)) != hipSuccess) return 0xffffffffu;
    return v;
}

}  // namespace kvr
