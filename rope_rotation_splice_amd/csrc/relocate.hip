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
// In-place splice ordering.  Downstream rows move by Delta within their own
// sequence, so a tile's destination may overlap the sources of other tiles.
// Tiles of a unit are ordered in the safe direction (increasing slots for
// Delta < 0, decreasing for Delta > 0) by a ticket taken from a per-unit
// atomic counter when the workgroup starts -- so a ticket holder is resident.
// A tile loads its whole source first, publishes "sources read" (flag =
// launch epoch), then waits only for the earlier tiles whose sources overlap
// its destination, and stores.  No tile waits before publishing, so every
// wait ends; waits are bounded anyway and report KVR_DEV_SPIN_LIMIT instead
// of hanging.  Stub tiles take the last tickets and wait for the move tiles
// whose sources overlap the stub's destination (only possible when Delta > 0).
#include "kvr_device.h"
#include "kvr_internal.h"

#include "../../include/kvreloc.h"

namespace kvr {

__device__ uint32_t g_errors_relocate;

namespace {

constexpr uint32_t kSpinLimit = 1u << 22;   // polls (each ~1-2 us with the sleep)

__device__ __forceinline__ void raise_error(uint32_t bit) {
    __hip_atomic_fetch_or(&g_errors_relocate, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int floor_div(int a, int b) {
    int q = a / b;
    return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}
__device__ __forceinline__ int ceil_div(int a, int b) { return -floor_div(-a, b); }

enum Mode { kSplice = 0, kGather = 1 };

template <int MODE, int RS, bool RF32>
__global__ __launch_bounds__(kThreads) void reloc_kernel(const RelocArgs A) {
    __shared__ float2 s_cs[kMaxPairs];
    __shared__ int32_t s_src_blk[kMaxTileRows], s_src_row[kMaxTileRows];
    __shared__ int32_t s_dst_blk[kMaxTileRows], s_dst_row[kMaxTileRows];
    __shared__ int32_t s_ticket;

    const int tid = threadIdx.x;
    const int bid = blockIdx.x;
    const Pool& P = A.pool;

    // ---- which unit (item, layer) and which tile --------------------------
    int it = 0;
    while (it + 1 < A.n_items && bid >= A.items[it + 1].wg_off) ++it;
    const Item& I = A.items[it];
    const int local = bid - I.wg_off;
    const int layer = local / I.tiles;
    int t;
    if (MODE == kSplice) {
        if (tid == 0) {
            int tk = -1;
            if ((__hip_atomic_load(&g_errors_relocate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                 (KVR_DEV_SPIN_LIMIT | KVR_DEV_BAD_TICKET)) == 0) {
                uint32_t* cnt = A.counters + it * P.n_layers + layer;
                tk = (int)__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (tk == I.tiles - 1) st_dev(cnt, 0u);     // all tickets taken: leave it zeroed
                if (tk < 0 || tk >= I.tiles) { raise_error(KVR_DEV_BAD_TICKET); tk = -1; }
            }
            s_ticket = tk;
        }
        __syncthreads();
        t = s_ticket;
        if (t < 0) return;
    } else {
        t = local - layer * I.tiles;
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

    // ---- row tables (block-table lookups staged in LDS) -------------------
    if (tid < nrows) {
        const int i = r0 + tid;
        const int32_t* bt = A.bt + I.bt_off;
        const int B = P.block_size;
        const int dslot = (MODE == kGather) ? I.a + i : (is_move ? I.a + i + I.shift : I.b + i);
        int db = bt[dslot / B];
        bool ok = (unsigned)db < (unsigned)P.n_blocks;
        int sb = 0, sr = i;
        if (src_in_pool) {
            const int sslot = I.a + i;
            sb = bt[sslot / B];
            sr = sslot % B;
            ok = ok && (unsigned)sb < (unsigned)P.n_blocks;
        }
        if (!ok) { raise_error(KVR_DEV_BAD_BLOCK); db = -1; }
        s_dst_blk[tid] = db;
        s_dst_row[tid] = dslot % B;
        s_src_blk[tid] = sb;
        s_src_row[tid] = sr;
    }
    if (rotate) angle_table(s_cs, A.theta, P.n_pairs, I.shift, tid);
    __syncthreads();

    // ---- loads ------------------------------------------------------------
    const int64_t lpf = (int64_t)layer * (src_in_pool ? P.pf_l : I.src.pf_l);
    const int64_t lrp = (int64_t)layer * (src_in_pool ? P.rp_l : I.src.rp_l);
    auto src_pf = [&](int row) -> const char* {
        return src_in_pool ? P.pf + lpf + (int64_t)s_src_blk[row] * P.pf_b + (int64_t)s_src_row[row] * P.pf_r
                           : I.src.pf + lpf + (int64_t)(r0 + row) * I.src.pf_r;
    };
    auto src_rp = [&](int row) -> const char* {
        return src_in_pool ? P.rp + lrp + (int64_t)s_src_blk[row] * P.rp_b + (int64_t)s_src_row[row] * P.rp_r
                           : I.src.rp + lrp + (int64_t)(r0 + row) * I.src.rp_r;
    };

    const int pfc = P.pf_chunks;
    const int pf_total = nrows * pfc;
    const int step_row = kThreads / pfc, step_c = kThreads % pfc;
    v4u pv[kPfItems];
    {
        int row = tid / pfc, c = tid % pfc;
#pragma unroll
        for (int k = 0; k < kPfItems; ++k) {
            const int q = tid + k * kThreads;
            if (q < pf_total && s_dst_blk[row] >= 0) pv[k] = ld16(src_pf(row) + c * 16);
            row += step_row; c += step_c;
            if (c >= pfc) { c -= pfc; ++row; }
        }
    }
    const int ri = P.rope_items;
    const int rp_total = nrows * ri;
    v4u lo[RS], hi[RS];
#pragma unroll
    for (int k = 0; k < RS; ++k) {
        const int q = tid + k * kThreads;
        if (q < rp_total) {
            const int row = q / ri, item = q - row * ri;
            const int head = item / P.half_chunks, hc = item - head * P.half_chunks;
            if (s_dst_blk[row] >= 0) {
                const char* p = src_rp(row) + head * P.head_bytes + hc * 16;
                lo[k] = ld16(p);
                hi[k] = ld16(p + P.half_bytes);
            }
        }
    }

    if (MODE == kSplice) {
        wait_loads();
        __syncthreads();                 // every source row of this tile is in registers
        if (is_move && tid == 0)
            st_dev(A.flags + (I.wg_off + layer * I.tiles) + t, A.epoch);
    }

    // ---- rotation (fp32, round to nearest even on store) -------------------
    if (rotate) {
#pragma unroll
        for (int k = 0; k < RS; ++k) {
            const int q = tid + k * kThreads;
            if (q < rp_total) {
                const int row = q / ri, item = q - row * ri;
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
            for (int j = j0; j <= j1; ++j) {
                uint32_t n = 0;
                while (ld_dev(f + j) != A.epoch) {
                    __builtin_amdgcn_s_sleep(2);
                    if (++n >= kSpinLimit ||
                        (__hip_atomic_load(&g_errors_relocate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                         (KVR_DEV_SPIN_LIMIT | KVR_DEV_BAD_TICKET))) {
                        raise_error(KVR_DEV_SPIN_LIMIT);
                        break;
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- stores -----------------------------------------------------------
    const int64_t dpf = (int64_t)layer * P.pf_l, drp = (int64_t)layer * P.rp_l;
    {
        int row = tid / pfc, c = tid % pfc;
#pragma unroll
        for (int k = 0; k < kPfItems; ++k) {
            const int q = tid + k * kThreads;
            if (q < pf_total && s_dst_blk[row] >= 0)
                st16(P.pf + dpf + (int64_t)s_dst_blk[row] * P.pf_b + (int64_t)s_dst_row[row] * P.pf_r + c * 16, pv[k]);
            row += step_row; c += step_c;
            if (c >= pfc) { c -= pfc; ++row; }
        }
    }
#pragma unroll
    for (int k = 0; k < RS; ++k) {
        const int q = tid + k * kThreads;
        if (q < rp_total) {
            const int row = q / ri, item = q - row * ri;
            const int head = item / P.half_chunks, hc = item - head * P.half_chunks;
            if (s_dst_blk[row] >= 0) {
                char* p = P.rp + drp + (int64_t)s_dst_blk[row] * P.rp_b + (int64_t)s_dst_row[row] * P.rp_r +
                          head * P.head_bytes + hc * 16;
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

template <int MODE>
hipError_t launch(const RelocArgs& a, int rs, bool f32, hipStream_t s) {
    dim3 grid(a.n_wg), block(kThreads);
#define KVR_CASE(R)                                                                              \
    case R:                                                                                      \
        if (f32) hipLaunchKernelGGL((reloc_kernel<MODE, R, true>), grid, block, 0, s, a);         \
        else     hipLaunchKernelGGL((reloc_kernel<MODE, R, false>), grid, block, 0, s, a);        \
        break;
    switch (rs) {
        KVR_CASE(1)
        KVR_CASE(2)
        KVR_CASE(4)
        KVR_CASE(8)
        KVR_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef KVR_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_splice(const RelocArgs& a, int rs, bool f32, hipStream_t s) { return launch<kSplice>(a, rs, f32, s); }
hipError_t launch_gather(const RelocArgs& a, int rs, bool f32, hipStream_t s) { return launch<kGather>(a, rs, f32, s); }

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
