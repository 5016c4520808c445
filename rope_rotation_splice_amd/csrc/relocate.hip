// Row movers with fused delta-rotation: the in-place splice of Leyline
// (sections 2.1-2.3) and the relocating gather of Irminsul (section 2.2).
//
// A workgroup handles one tile of up to `tile_rows` consecutive token rows of
// one (item, layer) unit.  Per row the position-free part is moved as raw
// 16-byte chunks (bit-exact, dtype-agnostic) and the rotary part is loaded
// as (lo, hi) 16-byte chunk pairs that hold the two halves x_j and x_{j+d/2}
// of 8 (bf16) or 4 (f32) rotation pairs, so each pair is rotated inside one
// thread without shuffles.  The whole tile is held in registers between the
// loads and the stores.
//
// In-place splice ordering (ticket form).  Downstream rows move by Delta
// within their own sequence, so a tile's destination may overlap the sources
// of other tiles.  Tiles of a unit are ordered in the safe direction
// (increasing slots for Delta < 0, decreasing for Delta > 0) by a ticket
// taken from a per-unit atomic counter when the workgroup starts -- so a
// ticket holder is resident.  Every workgroup takes exactly one ticket, and
// the one that takes the last resets the counter, so a launch always leaves
// its counters zeroed.  A tile loads its whole source first, publishes
// "sources read" (flag = launch epoch), then waits only for the earlier tiles
// whose sources overlap its destination, and stores.  No tile waits before
// publishing, so every wait ends; waits are bounded anyway.  A ticket out of
// range (a workspace that was not zeroed) or a wait that runs out raises a
// device error bit and marks the launch aborted (g_abort_epoch = epoch):
// from then on its tiles skip their stores, so no tile overwrites a source
// that may not have been read.  Stub tiles take the last tickets and wait
// for the move tiles whose sources overlap the stub's destination (only
// possible when Delta > 0).
#include "kvr_device.h"
#include "kvr_internal.h"

#include "../../include/kvreloc.h"

namespace kvr {

__device__ uint32_t g_errors_relocate;
__device__ uint32_t g_abort_epoch;      // epoch of a splice launch that hit a ticket or wait error

namespace {

constexpr uint32_t kSpinLimit = 1u << 22;   // polls (each ~1-2 us with the sleep)

__device__ __forceinline__ void raise_error(uint32_t bit) {
    __hip_atomic_fetch_or(&g_errors_relocate, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool aborted(uint32_t epoch) { return ld_dev(&g_abort_epoch) == epoch; }
__device__ __forceinline__ void abort_launch(uint32_t bit, uint32_t epoch) {
    raise_error(bit);
    st_dev(&g_abort_epoch, epoch);
}

__device__ __forceinline__ int floor_div(int a, int b) {
    int q = a / b;
    return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}
__device__ __forceinline__ int ceil_div(int a, int b) { return -floor_div(-a, b); }

enum Mode { kSplice = 0, kGather = 1 };

template <int MODE, int PFI, int RS, bool RF32>
__global__ __launch_bounds__(kThreads) void reloc_kernel(const RelocArgs A) {
    __shared__ float2 s_cs[kMaxPairs];
    __shared__ int32_t s_src_blk[kMaxTileRows], s_src_row[kMaxTileRows];
    __shared__ int32_t s_dst_blk[kMaxTileRows], s_dst_row[kMaxTileRows];
    __shared__ int32_t s_ticket;
    __shared__ int32_t s_store;      // splice: 0 when this tile must not store

    const int tid = threadIdx.x;
    const int bid = blockIdx.x;
    const Pool& P = A.pool;

    // ---- which unit (item, layer) and which tile --------------------------
    // last item whose first workgroup (splice) or tile (gather) is <= x: the
    // offsets are ascending and padded with INT32_MAX, so a count suffices
    auto item_at = [&](int x) __attribute__((always_inline)) {
        int n = 0;
#pragma unroll
        for (int i = 1; i < kMaxItems; ++i) n += x >= A.offs[i] ? 1 : 0;
        return n;
    };
    int it, t, layer;
    if (MODE == kGather) {
        // layer after layer, tiles numbered item after item within a layer
        layer = bid / A.n_tiles;
        const int k = bid - layer * A.n_tiles;
        it = item_at(k);
        t = k - A.offs[it];
    } else {
        it = item_at(bid);
    }
    const Item& I = A.items[it];
    if (MODE == kSplice) {
        const int local = bid - I.wg_off;
        layer = local / I.tiles;
        if (tid == 0) {
            // every workgroup takes exactly one ticket, whatever happened
            // before, so the counter returns to zero at the end of the launch
            uint32_t* cnt = A.counters + it * P.n_layers + layer;
            int tk = (int)__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tk == I.tiles - 1) st_dev(cnt, 0u);     // all tickets taken: leave it zeroed
            if (tk < 0 || tk >= I.tiles) { abort_launch(KVR_DEV_BAD_TICKET, A.epoch); tk = -1; }
            s_ticket = tk;
        }
        __syncthreads();
        t = s_ticket;
        if (t < 0) return;
    }

    const int T = A.tile_rows;
    const bool is_move = (MODE == kGather) || t < I.move_tiles;
    int r0, r1;                     // rows [r0, r1) of the moved range / entry / stub
    if (MODE == kGather) {
        r0 = t * T; r1 = min(r0 + T, I.moved);
    } else if (is_move) {
        if (I.shift < 0) { r0 = t * T; r1 = min(r0 + T, I.moved); }
        else             { r1 = I.moved - t * T; r0 = max(r1 - T, 0); }
    } else {
        r0 = (t - I.move_tiles) * T; r1 = min(r0 + T, I.r_len);
    }
    const int nrows = r1 - r0;
    const bool src_in_pool = (MODE == kSplice) && is_move;
    const bool rotate = is_move && I.shift != 0;
    const int32_t* bt = A.bt + I.bt_off;
    // destination slot of row i of this tile's range
    const int dbase = (MODE == kGather) ? I.a : (is_move ? I.a + I.shift : I.b);

    // ---- block-table lookups ----------------------------------------------
    // Vector-memory loads complete in order, so each row's block-table entry
    // is requested before any row data: using it later never waits behind a
    // row load.  The splice stages one entry per row in LDS; its source rows
    // of a move live in the pool and need their entries before the data loads
    // (one round trip + barrier).  Registry and stub rows are contiguous and
    // load at once.
    auto bt_index = [&](int slot) { return P.bs_shift >= 0 ? (slot >> P.bs_shift) : slot / P.block_size; };
    auto in_block = [&](int slot) {
        return P.bs_shift >= 0 ? (slot & (P.block_size - 1)) : slot - (slot / P.block_size) * P.block_size;
    };
    // theta_j / 2 pi of this thread's pair, requested ahead of every row load
    const double om = rotate && tid < P.n_pairs ? A.omega[tid] : 0.0;
    const int sbase = I.a + r0;            // source slot of row 0 (splice move tiles)
    const int dslot0 = dbase + r0;
    const unsigned nb = (unsigned)P.n_blocks;
    int my_db = 0, my_sb = 0;
    if (MODE == kSplice && tid < nrows) {
        my_db = bt[bt_index(dslot0 + tid)];
        if (src_in_pool) my_sb = bt[bt_index(sbase + tid)];
    }
    if (src_in_pool) {
        if (tid < nrows) {
            const bool ok = (unsigned)my_sb < nb;
            if (!ok) raise_error(KVR_DEV_BAD_BLOCK);
            s_src_blk[tid] = ok ? my_sb : -1;
            s_src_row[tid] = in_block(sbase + tid);
        }
        __syncthreads();
    }

    // ---- this thread's items: 16-byte chunks of the position-free part and
    // (lo, hi) chunk pairs of the rotary part, and the rows they belong to
    const int pfc = P.pf_chunks;
    const int pf_total = nrows * pfc;
    const int step_row = kThreads / pfc, step_c = kThreads % pfc;
    const int ri = P.rope_items;
    const int rp_total = nrows * ri;
    int pf_row[PFI], pf_c[PFI];
    {
        int row = tid / pfc, c = tid - (tid / pfc) * pfc;
#pragma unroll
        for (int k = 0; k < PFI; ++k) {
            const bool ok = tid + k * kThreads < pf_total && (!src_in_pool || s_src_blk[row] >= 0);
            pf_row[k] = ok ? row : -1;
            pf_c[k] = c;
            row += step_row; c += step_c;
            if (c >= pfc) { c -= pfc; ++row; }
        }
    }
    int rp_row[RS], rp_off[RS];
#pragma unroll
    for (int k = 0; k < RS; ++k) {
        const int q = tid + k * kThreads;
        rp_row[k] = -1;
        rp_off[k] = 0;
        if (q < rp_total) {
            const int row = q / ri, item = q - row * ri;
            if (!src_in_pool || s_src_blk[row] >= 0) {
                const int head = item / P.half_chunks, hc = item - head * P.half_chunks;
                rp_row[k] = row;
                rp_off[k] = head * P.head_bytes + hc * 16;
            }
        }
    }
    // Gather: every thread looks up the destination block of its own items'
    // rows (lanes of a wave mostly share one entry), before its row loads, so
    // the waves store independently, with no barrier between loads and stores.
    int pf_db[PFI], rp_db[RS];
    if (MODE == kGather) {
#pragma unroll
        for (int k = 0; k < PFI; ++k) pf_db[k] = pf_row[k] >= 0 ? bt[bt_index(dslot0 + pf_row[k])] : -1;
#pragma unroll
        for (int k = 0; k < RS; ++k) rp_db[k] = rp_row[k] >= 0 ? bt[bt_index(dslot0 + rp_row[k])] : -1;
    }

    // ---- row loads ---------------------------------------------------------
    const char* spf = src_in_pool ? P.pf + (int64_t)layer * P.pf_l : I.src.pf + (int64_t)layer * I.src.pf_l;
    const char* srp = src_in_pool ? P.rp + (int64_t)layer * P.rp_l : I.src.rp + (int64_t)layer * I.src.rp_l;
    v4u pv[PFI];
#pragma unroll
    for (int k = 0; k < PFI; ++k) {
        const int row = pf_row[k];
        if (row >= 0) {
            const char* p = src_in_pool
                ? spf + (int64_t)s_src_blk[row] * P.pf_b + (int64_t)s_src_row[row] * P.pf_r
                : spf + (int64_t)(r0 + row) * I.src.pf_r;
            pv[k] = ld16(p + pf_c[k] * 16);
        }
    }
    v4u lo[RS], hi[RS];
#pragma unroll
    for (int k = 0; k < RS; ++k) {
        const int row = rp_row[k];
        if (row >= 0) {
            const char* p = src_in_pool
                ? srp + (int64_t)s_src_blk[row] * P.rp_b + (int64_t)s_src_row[row] * P.rp_r
                : srp + (int64_t)(r0 + row) * I.src.rp_r;
            lo[k] = ld16(p + rp_off[k]);
            hi[k] = ld16(p + rp_off[k] + P.half_bytes);
        }
    }

    // ---- while the rows are in flight: destination rows, angle table -------
    if (MODE == kSplice && tid < nrows) {
        const bool ok = (unsigned)my_db < nb;
        if (!ok) raise_error(KVR_DEV_BAD_BLOCK);
        s_dst_blk[tid] = ok ? my_db : -1;
        s_dst_row[tid] = in_block(dslot0 + tid);
    }
    if (rotate) angle_table_from(s_cs, om, P.n_pairs, I.shift, tid);

    if (MODE == kSplice) {
        wait_loads();
        __syncthreads();                 // destination rows and angle table ready;
                                         // every source row is in registers
    } else if (rotate) {
        // the angle table is ready; when its writers and every rotation item
        // sit in wave 0, a wave-level fence is enough
        if (P.n_pairs <= 64 && rp_total <= 64) {
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();
        } else {
            __syncthreads();
        }
    }
    if (MODE == kSplice && is_move && tid == 0)
        st_dev(A.flags + (I.wg_off + layer * I.tiles) + t, A.epoch);

    // ---- rotation (fp32, round to nearest even on store) -------------------
    if (rotate) {
#pragma unroll
        for (int k = 0; k < RS; ++k) {
            if (rp_row[k] >= 0) {
                const int q = tid + k * kThreads;
                const int item = q % ri;
                const int hc = item % P.half_chunks;
                const float2* cs = s_cs + hc * P.pairs_per_chunk;
                if (RF32) rot_f32x4(lo[k], hi[k], cs);
                else      rot_bf16x8(lo[k], hi[k], cs);
            }
        }
    }

    // ---- wait for the tiles whose sources this tile overwrites -------------
    if (MODE == kSplice) {
        if (tid == 0) {
            int j0, j1;                   // inclusive range of move-tile tickets
            const int L = I.shift < 0 ? -I.shift : I.shift;
            const int M = I.moved;
            if (is_move) {
                // mirrored coordinates: rows counted in processing order, the
                // destination of row i is row i - L in the same coordinates
                const int a = t * T, b = min((t + 1) * T, M);
                j0 = max(0, floor_div(a - L, T));
                j1 = min(t - 1, ceil_div(b - L, T) - 1);
            } else {
                // stub rows [r0, r1) land on slots s_start + r; moved source row
                // i sits at slot s_end + i
                const int i0 = max(0, I.b + r0 - I.a), i1 = min(M, I.b + r1 - I.a);
                if (i0 >= i1 || I.move_tiles == 0) { j0 = 0; j1 = -1; }
                else if (I.shift < 0) { j0 = i0 / T; j1 = (i1 - 1) / T; }
                else { j0 = (M - i1) / T; j1 = (M - 1 - i0) / T; }
                j1 = min(j1, I.move_tiles - 1);
            }
            const uint32_t* f = A.flags + (I.wg_off + layer * I.tiles);
            bool ok = true;
            for (int j = j0; j <= j1 && ok; ++j) {
                uint32_t n = 0;
                while (ld_dev(f + j) != A.epoch) {
                    __builtin_amdgcn_s_sleep(2);
                    if (aborted(A.epoch)) { ok = false; break; }
                    if (++n >= kSpinLimit) { abort_launch(KVR_DEV_SPIN_LIMIT, A.epoch); ok = false; break; }
                }
            }
            // a tile whose wait did not end normally, or of an aborted
            // launch, stores nothing: its destination may hold unread sources
            s_store = ok && !aborted(A.epoch);
        }
        __syncthreads();
        if (!s_store) return;
    }

    // ---- stores -----------------------------------------------------------
    const int64_t dpf = (int64_t)layer * P.pf_l, drp = (int64_t)layer * P.rp_l;
    auto dst_block = [&](int row, int db) __attribute__((always_inline)) -> int {
        if (MODE == kSplice) return s_dst_blk[row];
        if ((unsigned)db >= nb) { raise_error(KVR_DEV_BAD_BLOCK); return -1; }
        return db;
    };
    auto dst_row = [&](int row) __attribute__((always_inline)) -> int {
        return MODE == kSplice ? s_dst_row[row] : in_block(dslot0 + row);
    };
#pragma unroll
    for (int k = 0; k < PFI; ++k) {
        const int row = pf_row[k];
        if (row >= 0) {
            const int db = dst_block(row, MODE == kGather ? pf_db[k] : 0);
            if (db >= 0)
                st16(P.pf + dpf + (int64_t)db * P.pf_b + (int64_t)dst_row(row) * P.pf_r + pf_c[k] * 16, pv[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < RS; ++k) {
        const int row = rp_row[k];
        if (row >= 0) {
            const int db = dst_block(row, MODE == kGather ? rp_db[k] : 0);
            if (db >= 0) {
                char* p = P.rp + drp + (int64_t)db * P.rp_b + (int64_t)dst_row(row) * P.rp_r + rp_off[k];
                st16(p, lo[k]);
                st16(p + P.half_bytes, hi[k]);
            }
        }
    }
}

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

template <int MODE, int PFI, int RS>
hipError_t launch_one(const RelocArgs& a, bool f32, hipStream_t s) {
    if (f32) hipLaunchKernelGGL((reloc_kernel<MODE, PFI, RS, true>), dim3(a.n_wg), dim3(kThreads), 0, s, a);
    else     hipLaunchKernelGGL((reloc_kernel<MODE, PFI, RS, false>), dim3(a.n_wg), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

// Instantiated shapes: (PFI, RS) with RS <= PFI for every power of two up to
// 16 (the host picks PFI >= RS).
template <int MODE, int PFI>
hipError_t launch_rs(const RelocArgs& a, int rs, bool f32, hipStream_t s) {
    switch (rs) {
        case 1: return launch_one<MODE, PFI, 1>(a, f32, s);
        case 2: if (PFI >= 2) return launch_one<MODE, PFI, (PFI >= 2 ? 2 : 1)>(a, f32, s); break;
        case 4: if (PFI >= 4) return launch_one<MODE, PFI, (PFI >= 4 ? 4 : 1)>(a, f32, s); break;
        case 8: if (PFI >= 8) return launch_one<MODE, PFI, (PFI >= 8 ? 8 : 1)>(a, f32, s); break;
        case 16: if (PFI >= 16) return launch_one<MODE, PFI, 16>(a, f32, s); break;
    }
    return hipErrorInvalidValue;
}

template <int MODE>
hipError_t launch(const RelocArgs& a, int pfi, int rs, bool f32, hipStream_t s) {
    switch (pfi) {
        case 1: return launch_rs<MODE, 1>(a, rs, f32, s);
        case 2: return launch_rs<MODE, 2>(a, rs, f32, s);
        case 4: return launch_rs<MODE, 4>(a, rs, f32, s);
        case 8: return launch_rs<MODE, 8>(a, rs, f32, s);
        case 16: return launch_rs<MODE, 16>(a, rs, f32, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_splice(const RelocArgs& a, int pfi, int rs, bool f32, hipStream_t s) {
    return launch<kSplice>(a, pfi, rs, f32, s);
}
hipError_t launch_gather(const RelocArgs& a, int pfi, int rs, bool f32, hipStream_t s) {
    return launch<kGather>(a, pfi, rs, f32, s);
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    unsigned blocks = (unsigned)((n + 255) / 256);
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, s, (uint32_t*)p, n);
    return hipGetLastError();
}

uint32_t read_and_clear_errors_relocate() {
    uint32_t v = 0, z = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_errors_relocate), sizeof(v)) != hipSuccess) return 0xffffffffu;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_errors_relocate), &z, sizeof(z)) != hipSuccess) return 0xffffffffu;
    return v;
}

}  // namespace kvr
