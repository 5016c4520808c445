// Band mover: the in-place splice of Leyline (sections 2.1-2.3) without any
// ordering between workgroups, for calls small enough to be bound by latency
// (a single sequence, a few layers); large batched calls take the ticketed
// mover of relocate.hip, which streams better.
//
// Let L = |Delta| and number the moved rows 0..M-1 in processing order
// (increasing slots for Delta < 0, decreasing for Delta > 0).  Row i lands on
// the slot that row i - L occupied.  Group the rows by offset o = i mod L: the
// rows of one offset form a chain o, o + L, o + 2L, ..., and each row's
// destination is its predecessor's source.  The K = ceil(M / L) rows o + kL of
// all offsets form band k.  A workgroup owns a range of offsets and every row
// of their chains, so the whole write-after-read ordering of the move -- a row
// stored over its chain predecessor's source -- stays inside one workgroup:
// no atomics, flags or waits between workgroups.
//
// Rows are moved as in the ticketed mover (relocate.hip): the position-free
// part as raw 16-byte chunks (bit-exact), the rotary part as (lo, hi) chunk
// pairs rotated in fp32 inside one thread and rounded once.
#include "kvr_device.h"
#include "kvr_internal.h"

#include "../../include/kvreloc.h"

namespace kvr {

__device__ uint32_t g_errors_band;

namespace {

__device__ __forceinline__ void raise_error(uint32_t bit) {
    __hip_atomic_fetch_or(&g_errors_band, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// floor(a / b) for 0 <= a < 2^21 from r = the fp32 reciprocal of b (within
// an ulp): (a + 1/2) / b lies at least 1/(2b) from an integer, while the fp32
// product errs by at most 3 * 2^-24 * a / b.
__device__ __forceinline__ int div_small(int a, float r) { return (int)(((float)a + 0.5f) * r); }

// a * b + c with 32-bit a, b (one v_mad_u64_u32)
__device__ __forceinline__ uint64_t mad64(uint32_t a, uint32_t b, uint64_t c) { return (uint64_t)a * b + c; }

// ---- chain tiles -------------------------------------------------------------
//
// Workgroups of an item (sequence): per layer, `move_tiles` chain tiles, then
// stub workgroups (TR stub rows each); per layer and item the launch holds
// `tiles` of them.  A chain tile owns TO = max(1, TR / K) offsets and takes
// every band of their chains, G = min(K, TR) bands at a time: it loads the
// group's rows (about TR rows, all at once), waits for them, passes a barrier
// and stores them.  A
// row's destination is the source of the previous row of its chain, read in
// the same group before the barrier or in an earlier group.  The block ids of
// the tile's bands (first and last row of each, source and destination) and
// the first row's row within its block are staged in LDS; a band of TO <= TR
// <= block size consecutive slots spans at most two blocks.
// For Delta > 0 the stub rows [|S|, |S| + min(L, M)) land on the sources of
// the last row of each chain; a tile copies the ones of its offsets after its
// last group.  All other stub rows overlap no source and are copied by the
// stub workgroups.
//
// One-item launches (ONE: a single sequence, the common small call) skip the
// search for the workgroup's item and take the item's (cos, sin) table from
// the arguments.  Both would otherwise be chains of dependent reads of the
// argument block before the first row load: on MI355X they cost about 0.9
// and 0.4 us of a 6.5 us single-sequence splice.
//
// The values the block-table staging needs come first, as scalar arguments
// (the item's table row, its slots, shift, moved rows and tile counts, the
// tile height and the block size).  Built with kernarg preloading, they
// arrive in scalar registers at launch, so a one-item launch issues its
// staging lookups at once, while the argument block is still being read.
// Launches of several items pass their first item's values and ignore them.
template <int PFI, int RS, bool RF32, bool ONE>
__global__ __launch_bounds__(kThreads) void band_kernel(const int32_t* lead_bt, int32_t lead_a, int32_t lead_b,
                                                        int32_t lead_shift, int32_t lead_moved, int32_t lead_tiles,
                                                        int32_t lead_move_tiles, int32_t lead_r_len, int32_t lead_tr,
                                                        int32_t lead_bs, const RelocArgs A) {
    __shared__ float2 s_cs[kMaxPairs];
    __shared__ int32_t s_blk[4 * kBandMaxBands];
    __shared__ int32_t s_r0[2 * kBandMaxBands];

    const int tid = threadIdx.x;
    const int bid = blockIdx.x;
    const Pool& P = A.pool;
    int it = 0;
    if (!ONE) {
#pragma unroll
        for (int i = 1; i < kMaxItems; ++i) it += bid >= A.offs[i] ? 1 : 0;
    }
    const Item& I = A.items[it];
    // the item's scalars: from the leading arguments in a one-item launch
    const int Ia = ONE ? lead_a : I.a, Ib = ONE ? lead_b : I.b, Ishift = ONE ? lead_shift : I.shift;
    const int Imoved = ONE ? lead_moved : I.moved, Itiles = ONE ? lead_tiles : I.tiles;
    const int Imove_tiles = ONE ? lead_move_tiles : I.move_tiles, Ir_len = ONE ? lead_r_len : I.r_len;
    const int Bsz = ONE ? lead_bs : P.block_size;
    const int bs_shift = ONE ? ((Bsz & (Bsz - 1)) == 0 ? __builtin_ctz((unsigned)Bsz) : -1) : P.bs_shift;
    const int local = ONE ? bid : bid - I.wg_off;
    const int layer = local / Itiles;
    const int t = local - layer * Itiles;
    const int32_t* bt = ONE ? lead_bt : A.bt + I.bt_off;
    const unsigned nb = (unsigned)P.n_blocks;
    auto bt_index = [&](int slot) { return bs_shift >= 0 ? (slot >> bs_shift) : slot / Bsz; };
    auto in_block = [&](int slot) {
        return bs_shift >= 0 ? (slot & (Bsz - 1)) : slot - (slot / Bsz) * Bsz;
    };
    const char* pfl = P.pf + (int64_t)layer * P.pf_l;
    const char* rpl = P.rp + (int64_t)layer * P.rp_l;
    const uint32_t pf_b = (uint32_t)P.pf_b, pf_r = (uint32_t)P.pf_r;    // host-checked < 2^32
    const uint32_t rp_b = (uint32_t)P.rp_b, rp_r = (uint32_t)P.rp_r;
    const int pfc = P.pf_chunks, ri = P.rope_items;
    const int L = Ishift < 0 ? -Ishift : Ishift;
    const int M = Imoved;
    const int span = min(L, M);
    const int S = Ia - Ib;                 // |S|: stub row S + i lands on moved row i's source slot
    const bool mirror = Ishift > 0;
    const int TR = ONE ? lead_tr : A.tile_rows;

    // this thread's items: 16-byte chunks of the position-free part and (lo,
    // hi) chunk pairs of the rotary part of tile rows 0..TR-1 (row TR: none)
    int pf_row[PFI], pf_c[PFI];
    {
        const float r = __builtin_amdgcn_rcpf((float)pfc);
#pragma unroll
        for (int k = 0; k < PFI; ++k) {
            const int q = tid + k * kThreads;
            const int row = div_small(q, r);
            pf_row[k] = q < TR * pfc ? row : TR;
            pf_c[k] = q - row * pfc;
        }
    }
    int rp_row[RS], rp_off[RS], rp_hc[RS];
    {
        const float r = __builtin_amdgcn_rcpf((float)ri), rh = __builtin_amdgcn_rcpf((float)P.half_chunks);
#pragma unroll
        for (int k = 0; k < RS; ++k) {
            const int q = tid + k * kThreads;
            const int row = div_small(q, r), item = q - row * ri;
            const int head = div_small(item, rh), hc = item - head * P.half_chunks;
            rp_row[k] = q < TR * ri ? row : TR;
            rp_off[k] = head * P.head_bytes + hc * 16;
            rp_hc[k] = hc;
        }
    }

    const int B = Bsz;
    if (t >= Imove_tiles) {
        // ---- stub rows that overlap no source --------------------------------
        // Rows [r0, r0 + n) of the stub land on consecutive slots from
        // Ib + r0, in at most two blocks (TR <= block size).
        const int r0 = (t - Imove_tiles) * TR;
        const int n = min(TR, Ir_len - r0);
        if (tid < 2) {
            const int slot = Ib + r0 + (tid ? n - 1 : 0);
            int b = bt[bt_index(slot)];
            if ((unsigned)b >= nb) { raise_error(KVR_DEV_BAD_BLOCK); b = -1; }
            s_blk[tid] = b;
            if (tid == 0) s_r0[0] = in_block(slot);
        }
        __syncthreads();
        const char* spf = I.src.pf + (int64_t)layer * I.src.pf_l;
        const char* srp = I.src.rp + (int64_t)layer * I.src.rp_l;
        const int br0 = __builtin_amdgcn_readfirstlane(s_r0[0]);
        const int b0 = __builtin_amdgcn_readfirstlane(s_blk[0]), b1 = __builtin_amdgcn_readfirstlane(s_blk[1]);
        // destination of stub row r0 + row, or false when this workgroup does
        // not write it (past the stub, a bad block, or a row that lands on a
        // chain's source and is written by that chain's tile)
        auto dst = [&](int row, int& blk, int& rib) __attribute__((always_inline)) -> bool {
            const int r = br0 + row;
            const bool second = r >= B;
            rib = second ? r - B : r;
            blk = second ? b1 : b0;
            const int sr = r0 + row;
            return row < n && blk >= 0 && !(mirror && sr >= S && sr < S + span);
        };
        v4u pv[PFI], lo[RS], hi[RS];
#pragma unroll
        for (int k = 0; k < PFI; ++k) {
            const int row = pf_row[k] < n ? pf_row[k] : 0;
            pv[k] = ld16(spf + (int64_t)(r0 + row) * I.src.pf_r + pf_c[k] * 16);
        }
#pragma unroll
        for (int k = 0; k < RS; ++k) {
            const int row = rp_row[k] < n ? rp_row[k] : 0;
            const char* q = srp + (int64_t)(r0 + row) * I.src.rp_r + rp_off[k];
            lo[k] = ld16(q);
            hi[k] = ld16(q + P.half_bytes);
        }
#pragma unroll
        for (int k = 0; k < PFI; ++k) {
            int blk, rib;
            if (dst(pf_row[k], blk, rib)) st16((char*)pfl + mad64(blk, pf_b, mad64(rib, pf_r, pf_c[k] * 16)), pv[k]);
        }
#pragma unroll
        for (int k = 0; k < RS; ++k) {
            int blk, rib;
            if (dst(rp_row[k], blk, rib)) {
                char* q = (char*)rpl + mad64(blk, rp_b, mad64(rib, rp_r, rp_off[k]));
                st16(q, lo[k]);
                st16(q + P.half_bytes, hi[k]);
            }
        }
        return;
    }

    // ---- chain tile ------------------------------------------------------------
    const int K = (M + L - 1) / L;             // bands of the unit
    const int TO = K >= TR ? 1 : TR / K;       // offsets per tile
    const int G = min(K, TR);                  // bands per group
    const int o0 = t * TO;
    const int nrow = min(TO, span - o0);
    const int Kt = (M - o0 + L - 1) / L;       // bands of offset o0 (the most of any offset here)
    // processing-order row -> moved row (slot Ia + moved row)
    auto moved_row = [&](int ip) { return mirror ? M - 1 - ip : ip; };
    if (tid < 4 * Kt) {
        // block ids of band k's first (w & 1 == 0) and last row, source (w < 2)
        // or destination, and the first row's row within its block
        const int k = tid >> 2, w = tid & 3;
        const int ip = o0 + k * L + ((w & 1) ? min(nrow, M - o0 - k * L) - 1 : 0);
        const int slot = Ia + moved_row(ip) + ((w & 2) ? Ishift : 0);
        int b = bt[bt_index(slot)];
        if ((unsigned)b >= nb) { raise_error(KVR_DEV_BAD_BLOCK); b = -1; }
        s_blk[tid] = b;
        if (!(w & 1)) s_r0[2 * k + (w >> 1)] = in_block(slot);
    }
    if (ONE) {
        if (tid < P.n_pairs) s_cs[tid] = make_float2(A.cs[2 * tid], A.cs[2 * tid + 1]);
    } else {
        angle_table(s_cs, A.omega, P.n_pairs, Ishift, tid);
    }
    __syncthreads();

    // tile row -> (band within the group, offset within the tile)
    int pf_g[PFI], pf_o[PFI], rp_g[RS], rp_o[RS];
    {
        const float r = __builtin_amdgcn_rcpf((float)TO);
#pragma unroll
        for (int j = 0; j < PFI; ++j) { pf_g[j] = div_small(pf_row[j], r); pf_o[j] = pf_row[j] - pf_g[j] * TO; }
#pragma unroll
        for (int j = 0; j < RS; ++j) { rp_g[j] = div_small(rp_row[j], r); rp_o[j] = rp_row[j] - rp_g[j] * TO; }
    }

    // Location of offset `o` in band k, source or destination: a band's rows
    // are consecutive slots (ascending for Delta < 0, descending for
    // Delta > 0), offset o at r0 +- o within the first block or past its edge
    // in the second.  Rows outside the tile (past a chain's end, bands past
    // Kt, padding rows) and rows of a bad block take row 0 of band
    // min(k, Kt - 1), or block 0, and report false: their loads are harmless
    // and their stores are skipped, so every load is issued unconditionally.
    auto locate = [&](int g, int o, int k, int dst, int& blk, int& rib) -> bool {
        const int kc = min(k, Kt - 1);
        const bool ok = g < G && k < Kt && o < nrow && o0 + kc * L + o < M;
        const int rr = ok ? o : 0;
        const int r0 = s_r0[2 * kc + dst];
        const int r = mirror ? r0 - rr : r0 + rr;
        const bool second = mirror ? r < 0 : r >= B;
        rib = second ? (mirror ? r + B : r - B) : r;
        const int b = s_blk[4 * kc + 2 * dst + (second ? 1 : 0)];
        blk = b >= 0 ? b : 0;
        return ok && b >= 0;
    };
    v4u pv[PFI], lo[RS], hi[RS];
    for (int g0 = 0; g0 < Kt; g0 += G) {
        uint32_t src_ok = 0;
#pragma unroll
        for (int j = 0; j < PFI; ++j) {
            int blk, rib;
            src_ok |= (uint32_t)locate(pf_g[j], pf_o[j], g0 + pf_g[j], 0, blk, rib) << j;
            pv[j] = ld16(pfl + mad64(blk, pf_b, mad64(rib, pf_r, pf_c[j] * 16)));
        }
#pragma unroll
        for (int j = 0; j < RS; ++j) {
            int blk, rib;
            src_ok |= (uint32_t)locate(rp_g[j], rp_o[j], g0 + rp_g[j], 0, blk, rib) << (PFI + j);
            const char* q = rpl + mad64(blk, rp_b, mad64(rib, rp_r, rp_off[j]));
            lo[j] = ld16(q);
            hi[j] = ld16(q + P.half_bytes);
        }
        wait_loads();
        __syncthreads();               // every row of the group is in registers
#pragma unroll
        for (int j = 0; j < PFI; ++j) {
            int blk, rib;
            const bool ok = locate(pf_g[j], pf_o[j], g0 + pf_g[j], 1, blk, rib) && ((src_ok >> j) & 1);
            if (ok) st16((char*)pfl + mad64(blk, pf_b, mad64(rib, pf_r, pf_c[j] * 16)), pv[j]);
        }
#pragma unroll
        for (int j = 0; j < RS; ++j) {
            int blk, rib;
            const bool ok = locate(rp_g[j], rp_o[j], g0 + rp_g[j], 1, blk, rib) && ((src_ok >> (PFI + j)) & 1);
            const float2* cs = s_cs + rp_hc[j] * P.pairs_per_chunk;
            if (RF32) rot_f32x4(lo[j], hi[j], cs);
            else      rot_bf16x8(lo[j], hi[j], cs);
            if (ok) {
                char* q = (char*)rpl + mad64(blk, rp_b, mad64(rib, rp_r, rp_off[j]));
                st16(q, lo[j]);
                st16(q + P.half_bytes, hi[j]);
            }
        }
    }


    // ---- Delta > 0: stub rows that land on the last row of each chain -------
    // Every chain's last row was read before the last group's stores.  Tile
    // rows 0..TO-1 (band 0 of a group) stand for the tile's offsets here.
    if (mirror && Ir_len > 0) {
        const char* spf = I.src.pf + (int64_t)layer * I.src.pf_l;
        const char* srp = I.src.rp + (int64_t)layer * I.src.rp_l;
        // offset o's last row is moved row (M - 1 - o) mod L, in band kl; the
        // stub row S + that index lands on its source slot
        auto last_row = [&](int row, int& blk, int& rib) -> int {
            if (row >= nrow) return -1;
            const int i = (M - 1 - (o0 + row)) % L;
            const int kl = (M - 1 - (o0 + row)) / L;
            const int r = s_r0[2 * kl] - row;    // the band's slots descend from its first row
            const bool second = r < 0;
            blk = s_blk[4 * kl + (second ? 1 : 0)];
            rib = second ? r + B : r;
            return blk >= 0 ? S + i : -1;
        };
#pragma unroll
        for (int j = 0; j < PFI; ++j) {
            int blk, rib;
            const int r = pf_g[j] == 0 ? last_row(pf_o[j], blk, rib) : -1;
            if (r >= 0)
                st16((char*)pfl + mad64(blk, pf_b, mad64(rib, pf_r, pf_c[j] * 16)),
                     ld16(spf + (int64_t)r * I.src.pf_r + pf_c[j] * 16));
        }
#pragma unroll
        for (int j = 0; j < RS; ++j) {
            int blk, rib;
            const int r = rp_g[j] == 0 ? last_row(rp_o[j], blk, rib) : -1;
            if (r >= 0) {
                const char* s = srp + (int64_t)r * I.src.rp_r + rp_off[j];
                char* q = (char*)rpl + mad64(blk, rp_b, mad64(rib, rp_r, rp_off[j]));
                const v4u a = ld16(s), b = ld16(s + P.half_bytes);
                st16(q, a);
                st16(q + P.half_bytes, b);
            }
        }
    }
}

template <int PFI, int RS, bool RF32, bool ONE>
void launch_band_kernel(const RelocArgs& a, hipStream_t s) {
    const Item& I = a.items[0];
    hipLaunchKernelGGL((band_kernel<PFI, RS, RF32, ONE>), dim3(a.n_wg), dim3(kThreads), 0, s, a.bt + I.bt_off, I.a,
                       I.b, I.shift, I.moved, I.tiles, I.move_tiles, I.r_len, a.tile_rows, a.pool.block_size, a);
}

template <int PFI, int RS, bool ONE>
hipError_t launch_band_one(const RelocArgs& a, bool f32, hipStream_t s) {
    if (f32) launch_band_kernel<PFI, RS, true, ONE>(a, s);
    else     launch_band_kernel<PFI, RS, false, ONE>(a, s);
    return hipGetLastError();
}

// Instantiated shapes: rotary slots RS in {1, 2, 4} (fp32 keys: {1, 2}),
// RS <= PFI; the host lowers the tile height until its shape is one of them.
template <int PFI, bool ONE>
hipError_t launch_band_rs(const RelocArgs& a, int rs, bool f32, hipStream_t s) {
    switch (rs) {
        case 1: return launch_band_one<PFI, 1, ONE>(a, f32, s);
        case 2: if (PFI >= 2) return launch_band_one<PFI, (PFI >= 2 ? 2 : 1), ONE>(a, f32, s); break;
        case 4:
            if (PFI >= 4 && !f32) {
                launch_band_kernel<PFI, (PFI >= 4 ? 4 : 1), false, ONE>(a, s);
                return hipGetLastError();
            }
            break;
    }
    return hipErrorInvalidValue;
}

template <bool ONE>
hipError_t launch_band_pfi(const RelocArgs& a, int pfi, int rs, bool f32, hipStream_t s) {
    switch (pfi) {
        case 1: return launch_band_rs<1, ONE>(a, rs, f32, s);
        case 2: return launch_band_rs<2, ONE>(a, rs, f32, s);
        case 4: return launch_band_rs<4, ONE>(a, rs, f32, s);
        case 8: return launch_band_rs<8, ONE>(a, rs, f32, s);
        case 16: return launch_band_rs<16, ONE>(a, rs, f32, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_band(const RelocArgs& a, int pfi, int rs, bool f32, bool one_item, hipStream_t s) {
    return one_item ? launch_band_pfi<true>(a, pfi, rs, f32, s) : launch_band_pfi<false>(a, pfi, rs, f32, s);
}

uint32_t read_and_clear_errors_band() {
    uint32_t v = 0, z = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_errors_band), sizeof(v)) != hipSuccess) return 0xffffffffu;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_errors_band), &z, sizeof(z)) != hipSuccess) return 0xffffffffu;
    return v;
}

}  // namespace kvr
