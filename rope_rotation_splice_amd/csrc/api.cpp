// Host side of the C ABI: argument validation, Delta/delta bookkeeping,
// tiling, workspace layout and kernel launches.  Nothing here touches device
// memory before every argument of a call has been validated.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/kvreloc.h"
#include "kvr_internal.h"

using namespace kvr;

namespace {

thread_local int32_t t_last_hip = 0;
std::atomic<uint32_t> g_epoch{1};

uint32_t next_epoch() {
    uint32_t e = g_epoch.fetch_add(1);
    if (e == 0) e = g_epoch.fetch_add(1);    // 0 is the value of a cleared flag
    return e;
}

kvr_status hip_fail(hipError_t e) {
    t_last_hip = (int32_t)e;
    return KVR_E_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool mult16(int64_t v) { return (v % 16) == 0; }
int esize(int32_t dtype) { return dtype == KVR_BF16 ? 2 : (dtype == KVR_F32 ? 4 : 0); }

// Validate a cache descriptor and build the byte-addressed pool view and the
// frequency table (omega_j = theta_j / 2 pi, revolutions per position).
kvr_status make_pool(const kvr_cache* c, Pool& P, double* omega) {
    if (!c) return KVR_E_ARG;
    const int pe = esize(c->pf_dtype), re = esize(c->rope_dtype);
    if (!pe || !re) return KVR_E_ARG;
    if (c->n_layers < 1 || c->block_size < 1 || c->n_blocks < 1) return KVR_E_ARG;
    if (c->pf_width < 1 || c->rope_heads < 1 || c->rope_dim < 2 || (c->rope_dim & 1)) return KVR_E_ARG;
    if (c->rope_dim / 2 > kMaxPairs || (int64_t)c->rope_heads * c->rope_dim > 4096) return KVR_E_ARG;
    const int64_t pf_bytes = (int64_t)c->pf_width * pe;
    const int64_t half_bytes = (int64_t)(c->rope_dim / 2) * re;
    if (!mult16(pf_bytes) || !mult16(half_bytes) || pf_bytes / 16 > kThreads) return KVR_E_ARG;
    if (!c->pf.base || !c->rope.base || !aligned16(c->pf.base) || !aligned16(c->rope.base)) return KVR_E_ARG;
    const int64_t s[6] = {c->pf.layer_stride * pe, c->pf.block_stride * pe, c->pf.row_stride * pe,
                          c->rope.layer_stride * re, c->rope.block_stride * re, c->rope.row_stride * re};
    for (int64_t v : s)
        if (v < 0 || !mult16(v)) return KVR_E_ARG;
    if (!c->inv_freq && !(c->rope_base > 0.0)) return KVR_E_ARG;

    P.pf = (char*)c->pf.base;   P.pf_l = s[0]; P.pf_b = s[1]; P.pf_r = s[2];
    P.rp = (char*)c->rope.base; P.rp_l = s[3]; P.rp_b = s[4]; P.rp_r = s[5];
    P.block_size = c->block_size;
    P.bs_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((1 << sh) == c->block_size) P.bs_shift = sh;
    P.n_blocks = c->n_blocks;
    P.n_layers = c->n_layers;
    P.pf_chunks = (int32_t)(pf_bytes / 16);
    P.half_chunks = (int32_t)(half_bytes / 16);
    P.rope_items = c->rope_heads * P.half_chunks;
    P.head_bytes = (int32_t)(2 * half_bytes);
    P.half_bytes = (int32_t)half_bytes;
    P.n_pairs = c->rope_dim / 2;
    P.pairs_per_chunk = 16 / re;
    for (int j = 0; j < kMaxPairs; ++j) omega[j] = 0.0;
    for (int j = 0; j < P.n_pairs; ++j) {
        const double th = c->inv_freq ? c->inv_freq[j]
                                      : std::pow(c->rope_base, -2.0 * (double)j / (double)c->rope_dim);
        if (!std::isfinite(th)) return KVR_E_ARG;
        omega[j] = th / (2.0 * M_PI);     // revolutions per position
    }
    return KVR_OK;
}

// Tile shape: rows per tile T, and the per-thread counts of position-free
// chunks (pfi) and rotation items (rs) it needs, both powers of two <= 16.
// Measured on MI355X (61-layer MLA rows): the gather streams best with about
// 9 KB of row data per workgroup (many short-lived workgroups), the ticketed
// in-place splice with about 36 KB (its per-tile ticket and flag round trips
// need more bytes per workgroup to hide).
struct TileShape { int T, pfi, rs; };

int pow2_at_least(int v) { int p = 1; while (p < v) p *= 2; return p; }
int pow2_at_most(int v) { int p = 1; while (p * 2 <= v) p *= 2; return p; }

TileShape shape_for(const Pool& P, int T) {
    for (;;) {
        TileShape s{T, pow2_at_least((T * P.pf_chunks + kThreads - 1) / kThreads),
                    pow2_at_least((T * P.rope_items + kThreads - 1) / kThreads)};
        s.pfi = std::max(s.pfi, s.rs);
        if (s.pfi <= kPfItems || T == 1) return s;
        T = std::max(1, T / 2);
    }
}

TileShape choose_tile(const Pool& P, bool rope_f32, bool splice) {
    const int row_bytes = 16 * (P.pf_chunks + 2 * P.rope_items);
    int T = pow2_at_most(std::max(1, (splice ? 36864 : 9216) / row_bytes));
    T = std::min(T, kMaxTileRows);
    if (rope_f32) T = std::min(kMaxTileRows, (kThreads * kPfItems) / P.pf_chunks);
    TileShape s = shape_for(P, T);
    if (rope_f32) s.pfi = kPfItems;          // fp32 keys: one register shape only
    return s;
}

// Chain tiles of the band mover hold about 4.5 KB of rows (4 MLA rows), and
// at most a block of rows, so that the rows a tile takes from one band span at
// most two blocks.  Latency-bound calls finish sooner in many small tiles:
// the single 4096-slot splice (2,296 rows, one-item launch with preloaded
// arguments) took a median of 5.24, 5.12, 4.96 and 5.86 us on MI355X with
// tiles of 16, 8, 4 and 2 rows.
constexpr int kBandBytes = 4608;
// Calls that move fewer rows than this (all layers; 256 compute units x 8
// workgroups x 32 rows) are bound by latency and take the band mover; larger
// ones stream through the ticketed mover.  Measured on MI355X: the single
// splice takes 10.0 us ticketed; the 64-sequence batch takes 21.5 ms ticketed
// against 25.2 ms in chain tiles.
constexpr int64_t kBandMaxRows = 65536;

TileShape choose_band(const Pool& P, bool rope_f32) {
    const int row_bytes = 16 * (P.pf_chunks + 2 * P.rope_items);
    int T = pow2_at_most(std::max(1, kBandBytes / row_bytes));
    T = std::min({T, kMaxTileRows, pow2_at_most(P.block_size)});
    // the band kernel is built for at most 4 rotation items per thread (2 for fp32 keys)
    for (;;) {
        const TileShape s = shape_for(P, T);
        if (s.rs <= (rope_f32 ? 2 : 4) || T == 1) return s;
        T /= 2;
    }
}

kvr_status check_rows(const kvr_rows& r, const kvr_cache* c) {
    const int pe = esize(c->pf_dtype), re = esize(c->rope_dtype);
    if (!r.pf || !r.rope || !aligned16(r.pf) || !aligned16(r.rope)) return KVR_E_ARG;
    const int64_t s[4] = {r.pf_layer_stride * pe, r.pf_row_stride * pe, r.rope_layer_stride * re,
                          r.rope_row_stride * re};
    for (int64_t v : s)
        if (v < 0 || !mult16(v)) return KVR_E_ARG;
    if (s[1] > INT32_MAX || s[3] > INT32_MAX) return KVR_E_ARG;
    return KVR_OK;
}

SrcRows src_rows(const kvr_rows& r, const kvr_cache* c) {
    const int pe = esize(c->pf_dtype), re = esize(c->rope_dtype);
    SrcRows s;
    s.pf = (const char*)r.pf;
    s.rp = (const char*)r.rope;
    s.pf_l = r.pf_layer_stride * pe;
    s.rp_l = r.rope_layer_stride * re;
    s.pf_r = (int32_t)(r.pf_row_stride * pe);
    s.rp_r = (int32_t)(r.rope_row_stride * re);
    return s;
}

// ------------------------------------------------------------------ splice --

struct SpliceSeq {
    int32_t seq;
    Item item;
};

struct SplicePlan {
    Pool pool;
    double omega[kMaxPairs];
    TileShape tile{1, 1, 1};          // ticketed tiles
    TileShape band{1, 1, 1};          // band mover (chain tiles)
    std::vector<std::vector<SpliceSeq>> launches;        // ticketed launches
    std::vector<std::vector<SpliceSeq>> band_launches;
    size_t counters_bytes = 0, flags_bytes = 0;
    bool forget = false;
    std::vector<int64_t> new_lens;
};

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Optional ownership checks (environment KVR_DEBUG_CHECKS=1).  The host
// cannot see the block tables, so the callers' preconditions -- every block a
// call writes is held by that one logical block of one sequence, and no block
// id is out of range -- are otherwise only caught (in part) by the kernels'
// device error bits.  With the checks on, the tables are copied to the host,
// which waits for the stream, before anything is enqueued.
bool debug_checks() {
    const char* e = std::getenv("KVR_DEBUG_CHECKS");
    return e && std::atoi(e) != 0;
}

// Per table: the logical blocks [0, live) the sequence holds, and the ranges
// [lo, hi) of logical blocks the call writes.
struct TableUse {
    int64_t live = 0;
    std::vector<std::pair<int64_t, int64_t>> written;
};

kvr_status check_ownership(const int32_t* d_tables, int32_t stride, const std::vector<TableUse>& use,
                           int32_t n_blocks, hipStream_t stream) {
    if (use.empty()) return KVR_OK;
    std::vector<int32_t> h((size_t)use.size() * stride);
    hipError_t e = hipMemcpyAsync(h.data(), d_tables, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e);
    std::unordered_map<int32_t, int> holders;    // physical block -> logical blocks naming it
    std::vector<int32_t> written;
    for (size_t b = 0; b < use.size(); ++b) {
        std::set<int64_t> logical;
        for (int64_t k = 0; k < use[b].live; ++k) logical.insert(k);
        for (const auto& r : use[b].written)
            for (int64_t k = r.first; k < r.second; ++k) {
                logical.insert(k);
                written.push_back(h[b * stride + k]);
            }
        for (int64_t k : logical) {
            const int32_t id = h[b * stride + k];
            if (id < 0 || id >= n_blocks) return KVR_E_RANGE;
            ++holders[id];
        }
    }
    for (int32_t id : written)
        if (holders[id] > 1) return KVR_E_OVERLAP;
    return KVR_OK;
}

// Group items into launches of at most kMaxItems items and < 2^31 workgroups;
// wg_off is each item's first workgroup within its launch.
void pack_launches(std::vector<SpliceSeq>& items, int n_layers, std::vector<std::vector<SpliceSeq>>& out) {
    std::vector<SpliceSeq> cur;
    int64_t wg = 0;
    for (SpliceSeq& s : items) {
        const int64_t add = (int64_t)s.item.tiles * n_layers;
        if ((int)cur.size() == kMaxItems || wg + add >= ((int64_t)1 << 31)) {
            out.push_back(cur);
            cur.clear();
            wg = 0;
        }
        s.item.wg_off = (int32_t)wg;
        wg += add;
        cur.push_back(s);
    }
    if (!cur.empty()) out.push_back(cur);
}

kvr_status plan_splice(const kvr_cache* c, int32_t bt_stride, int32_t n_seq, const int64_t* seq_lens,
                       const kvr_directive* dirs, const kvr_rows* stubs, SplicePlan& pl) {
    kvr_status st = make_pool(c, pl.pool, pl.omega);
    if (st != KVR_OK) return st;
    if (n_seq < 0 || bt_stride < 1) return KVR_E_ARG;
    if (n_seq > 0 && (!seq_lens || !dirs)) return KVR_E_ARG;
    const int64_t capacity = (int64_t)bt_stride * c->block_size;
    if (capacity >= (int64_t)1 << 31) return KVR_E_ARG;
    pl.tile = choose_tile(pl.pool, c->rope_dtype == KVR_F32, true);
    const int T = pl.tile.T;
    pl.new_lens.assign(n_seq, 0);
    std::vector<SpliceSeq> ticketed, banded;
    std::vector<int64_t> bands;                       // per banded item: bands its chains hold
    // rows the call moves, all layers: a small call takes the band mover
    int64_t rows = 0;
    for (int32_t b = 0; b < n_seq; ++b)
        if (dirs[b].mode == KVR_AMORTIZE && dirs[b].s_end >= 0 && dirs[b].s_end <= seq_lens[b] &&
            dirs[b].r_len != dirs[b].s_end - dirs[b].s_start)
            rows += seq_lens[b] - dirs[b].s_end;
    const bool small = rows * c->n_layers < kBandMaxRows;
    for (int32_t b = 0; b < n_seq; ++b) {
        const kvr_directive& d = dirs[b];
        const int64_t N = seq_lens[b];
        if (d.mode != KVR_AMORTIZE && d.mode != KVR_FORGET) return KVR_E_ARG;
        if (N < 0 || N > capacity || d.s_start < 0 || d.s_start > d.s_end || d.s_end > N || d.r_len < 0)
            return KVR_E_RANGE;
        if (d.mode == KVR_FORGET) {
            pl.new_lens[b] = d.s_start;
            pl.forget = true;
            continue;
        }
        const int64_t delta = d.r_len - (d.s_end - d.s_start);
        if (N + delta > capacity) return KVR_E_CAPACITY;
        pl.new_lens[b] = N + delta;
        const bool has_stub = stubs && stubs[b].pf;
        if (has_stub) {
            st = check_rows(stubs[b], c);
            if (st != KVR_OK) return st;
            if (stubs[b].len != d.r_len) return KVR_E_RANGE;
        }
        Item it{};
        if (has_stub) it.src = src_rows(stubs[b], c);
        it.a = (int32_t)d.s_end;
        it.b = (int32_t)d.s_start;
        it.shift = (int32_t)delta;
        it.moved = (int32_t)(N - d.s_end);
        it.r_len = has_stub ? (int32_t)d.r_len : 0;
        it.bt_off = b * bt_stride;
        const int64_t L = delta < 0 ? -delta : delta;
        const bool moves = delta != 0 && it.moved > 0;
        // the band mover takes a sequence whose chains are at most
        // kBandMaxBands rows long; shorter shifts go through tickets
        const int64_t K = moves ? (it.moved + L - 1) / L : 0;
        // the band mover addresses rows with 32-bit block and row strides
        const bool strides32 = pl.pool.pf_b < ((int64_t)1 << 32) && pl.pool.pf_r < ((int64_t)1 << 32) &&
                               pl.pool.rp_b < ((int64_t)1 << 32) && pl.pool.rp_r < ((int64_t)1 << 32);
        if (small && K <= kBandMaxBands && strides32) {
            if (!moves && it.r_len == 0) continue;
            banded.push_back({b, it});
            bands.push_back(K);
        } else {
            it.move_tiles = (it.moved + T - 1) / T;
            it.tiles = it.move_tiles + (it.r_len + T - 1) / T;
            ticketed.push_back({b, it});
        }
    }
    // chain tiles take all K bands of max(1, TB / K) offsets each
    pl.band = choose_band(pl.pool, c->rope_dtype == KVR_F32);
    const int TB = pl.band.T;
    for (size_t i = 0; i < banded.size(); ++i) {
        Item& it = banded[i].item;
        const int64_t K = bands[i];
        const int64_t L = it.shift < 0 ? -(int64_t)it.shift : it.shift;
        const int64_t TO = K >= TB ? 1 : TB / std::max<int64_t>(K, 1);
        it.move_tiles = K ? (int32_t)((std::min<int64_t>(L, it.moved) + TO - 1) / TO) : 0;
        it.tiles = it.move_tiles + (it.r_len + TB - 1) / TB;
    }
    // longest chains first, so that they do not trail at the end of a launch
    std::vector<size_t> order(banded.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return bands[x] > bands[y]; });
    std::vector<SpliceSeq> sorted;
    for (size_t i : order) sorted.push_back(banded[i]);
    pack_launches(sorted, c->n_layers, pl.band_launches);
    pack_launches(ticketed, c->n_layers, pl.launches);
    size_t maxc = 0, maxf = 0;
    for (auto& L : pl.launches) {
        size_t nwg = 0;
        for (auto& s : L) nwg += (size_t)s.item.tiles * c->n_layers;
        maxc = std::max(maxc, L.size() * (size_t)c->n_layers * 4);
        maxf = std::max(maxf, nwg * 4);
    }
    pl.counters_bytes = maxc ? round_up(maxc) : 0;
    pl.flags_bytes = maxf ? round_up(maxf) : 0;
    return KVR_OK;
}


// ------------------------------------------------------------------- patch --

// The fused patch path needs bf16 parts, position-free rows of whole 64-feature
// (128-byte) pairs of groups, rotary heads made of whole 32-feature halves,
// and rope_dim / 2 <= kPatchMaxPairs.
kvr_status check_patch_cache(const kvr_cache* c) {
    if (c->pf_dtype != KVR_BF16 || c->rope_dtype != KVR_BF16) return KVR_E_UNSUPPORTED;
    if (c->pf_width % 64 || c->rope_dim % 64 || c->rope_dim / 2 > kPatchMaxPairs) return KVR_E_UNSUPPORTED;
    return KVR_OK;
}

kvr_status check_lowrank(const kvr_lowrank* f, int64_t len, int32_t width) {
    (void)width;
    if (!f || f->rank == 0 || len == 0) return KVR_OK;
    if (f->rank < 0 || f->rank > 64 || (f->rank % 4)) return KVR_E_ARG;
    if (!f->U || !f->V || !aligned16(f->U) || !aligned16(f->V)) return KVR_E_ARG;
    if (f->u_layer_stride < 0 || f->v_layer_stride < 0 || (f->u_layer_stride % 4) || (f->v_layer_stride % 4))
        return KVR_E_ARG;
    return KVR_OK;
}

void set_factors(const kvr_lowrank* f, const float*& U, const float*& V, int64_t& ul, int64_t& vl, int32_t& rank) {
    if (f && f->rank > 0) {
        U = f->U; V = f->V; ul = f->u_layer_stride; vl = f->v_layer_stride; rank = f->rank;
    } else {
        U = nullptr; V = nullptr; ul = vl = 0; rank = 0;
    }
}

// Enqueue patch-kernel launches for `items` (at most kPatchMaxItems each).
kvr_status run_patch(const Pool& pool, const double* omega, const int32_t* d_bt, std::vector<PatchItem>& items,
                     int n_layers, bool inplace, bool do_rope, bool do_pf, hipStream_t stream) {
    // The streaming kernel takes bf16 rows in 256-byte units (128-dimension
    // rotary heads), ranks up to 16, power-of-two blocks of at least 16 rows
    // and items of at most 4 x kPatchDmaMaxStages x 16 rows; anything else
    // goes to the tiled kernel.
    bool dma = pool.bs_shift >= 4 && (!do_rope || (pool.head_bytes == 256 && pool.pairs_per_chunk == 8)) &&
               (!do_pf || pool.pf_chunks % 16 == 0);
    for (const PatchItem& it : items)
        if (it.len > 4 * kPatchDmaMaxStages * 16 || it.rank_rp > 16 || it.rank_pf > 16) dma = false;
    const int n_ru = do_rope ? pool.rope_items / pool.half_chunks : 0;
    const int n_units = n_ru + (do_pf ? pool.pf_chunks / 16 : 0);
    size_t i = 0;
    while (i < items.size()) {
        PatchArgs a;
        std::memset(&a, 0, sizeof(a));
        a.pool = pool;
        a.bt = d_bt;
        a.tile_rows = kPatchTileRows;
        a.do_rope = do_rope;
        a.do_pf = do_pf;
        a.dma = dma;
        a.n_units = n_units;
        a.n_rope_units = n_ru;
        std::memcpy(a.omega, omega, sizeof(a.omega));
        int64_t wg = 0;
        int n = 0;
        for (; i < items.size() && n < kPatchMaxItems; ++i) {
            PatchItem it = items[i];
            const int64_t add = (int64_t)(dma ? n_units : it.tiles) * n_layers;
            if (n > 0 && wg + add >= ((int64_t)1 << 31)) break;
            it.wg_off = (int32_t)wg;
            wg += add;
            a.items[n++] = it;
        }
        a.n_items = n;
        a.n_wg = (int32_t)wg;
        hipError_t e = launch_patch(a, inplace, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    return KVR_OK;
}

}  // namespace

int32_t kvr::record_hip_error(hipError_t e) { return hip_fail(e); }

extern "C" {

int32_t kvr_abi_version(void) { return KVR_ABI_VERSION; }

const char* kvr_status_str(kvr_status s) {
    switch (s) {
        case KVR_OK: return "ok";
        case KVR_FORGET_NEEDS_PREFILL: return "FORGET directive: re-prefill from s_start";
        case KVR_E_ARG: return "invalid argument (pointer, alignment, dtype, shape or stride)";
        case KVR_E_RANGE: return "position or length out of range";
        case KVR_E_CAPACITY: return "result exceeds block-table capacity";
        case KVR_E_OVERLAP: return "target ranges overlap";
        case KVR_E_HIP: return "HIP runtime error";
        case KVR_E_WORKSPACE: return "workspace missing, misaligned or too small";
        case KVR_E_UNSUPPORTED: return "unsupported configuration";
        case KVR_E_SCRATCH: return "call needs more device scratch than the no-allocation entry point holds";
        default: return "unknown status";
    }
}

int32_t kvr_last_hip_error(void) { return t_last_hip; }

kvr_status kvr_device_errors(uint32_t* flags) {
    if (!flags) return KVR_E_ARG;
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e);
    const uint32_t v = read_and_clear_errors_relocate();
    const uint32_t w = read_and_clear_errors_patch();
    const uint32_t x = read_and_clear_errors_decode();
    const uint32_t y = read_and_clear_errors_lazy();
    const uint32_t z = read_and_clear_errors_keys();
    const uint32_t u = read_and_clear_errors_gqa_decode();
    const uint32_t b = read_and_clear_errors_band();
    if (v == 0xffffffffu || w == 0xffffffffu || x == 0xffffffffu || y == 0xffffffffu || z == 0xffffffffu ||
        u == 0xffffffffu || b == 0xffffffffu)
        return hip_fail(hipErrorUnknown);
    *flags = v | w | x | y | z | u | b;
    return KVR_OK;
}

kvr_status kvr_workspace_clear(void* d_ws, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return KVR_OK;
    if (!d_ws || (reinterpret_cast<uintptr_t>(d_ws) & 3u) || (bytes & 3u)) return KVR_E_ARG;
    hipError_t e = launch_fill_zero(d_ws, bytes, stream);
    return e == hipSuccess ? KVR_OK : hip_fail(e);
}

size_t kvr_splice_workspace_bytes(const kvr_cache* cache, int32_t n_seq, const int64_t* seq_lens,
                                  const kvr_directive* dirs) {
    SplicePlan pl;
    // The block-table stride only bounds capacity; use the largest so that
    // the query never fails on it.  Stubs do not change the tile count bound
    // (every stub row counts as if present).
    std::vector<kvr_rows> fake;
    if (!cache || n_seq < 0 || (n_seq > 0 && (!seq_lens || !dirs))) return 0;
    fake.resize(n_seq);
    for (int32_t b = 0; b < n_seq; ++b) {
        std::memset(&fake[b], 0, sizeof(kvr_rows));
        fake[b].pf = cache->pf.base;
        fake[b].rope = cache->rope.base;
        fake[b].len = dirs[b].r_len;
    }
    const int32_t bt_stride = (int32_t)std::max<int64_t>(1, ((int64_t)1 << 31) / std::max(1, cache->block_size) - 1);
    if (plan_splice(cache, bt_stride, n_seq, seq_lens, dirs, fake.data(), pl) != KVR_OK) return 0;
    return pl.counters_bytes + pl.flags_bytes;
}

kvr_status leyline_splice(const kvr_cache* cache, const int32_t* d_block_tables, int32_t bt_stride,
                          int32_t n_seq, const int64_t* seq_lens, const kvr_directive* dirs,
                          const kvr_rows* stubs, int64_t* new_lens, void* d_ws, size_t ws_bytes,
                          hipStream_t stream) {
    if (!d_block_tables || (reinterpret_cast<uintptr_t>(d_block_tables) & 3u)) return KVR_E_ARG;
    if (n_seq > 0 && !new_lens) return KVR_E_ARG;
    SplicePlan pl;
    kvr_status st = plan_splice(cache, bt_stride, n_seq, seq_lens, dirs, stubs, pl);
    if (st != KVR_OK) return st;
    const size_t need = pl.counters_bytes + pl.flags_bytes;
    if (!pl.launches.empty()) {
        if (!d_ws || (reinterpret_cast<uintptr_t>(d_ws) % kAlign) || ws_bytes < need) return KVR_E_WORKSPACE;
    }
    if (debug_checks()) {
        // a sequence holds the blocks of max(N, new_len) slots and writes [s_start, new_len)
        const int64_t B = cache->block_size;
        std::vector<TableUse> use(n_seq);
        for (int32_t b = 0; b < n_seq; ++b) {
            const int64_t n = seq_lens[b], nl = pl.new_lens[b];
            use[b].live = (std::max(n, nl) + B - 1) / B;
            if (dirs[b].mode == KVR_AMORTIZE && nl > dirs[b].s_start)
                use[b].written.push_back({dirs[b].s_start / B, (nl + B - 1) / B});
        }
        st = check_ownership(d_block_tables, bt_stride, use, cache->n_blocks, stream);
        if (st != KVR_OK) return st;
    }
    for (int32_t b = 0; b < n_seq; ++b) new_lens[b] = pl.new_lens[b];
    for (auto& L : pl.band_launches) {
        RelocArgs a;
        std::memset(&a, 0, sizeof(a));
        a.pool = pl.pool;
        a.bt = d_block_tables;
        a.n_items = (int32_t)L.size();
        a.tile_rows = pl.band.T;
        std::memcpy(a.omega, pl.omega, sizeof(a.omega));
        int64_t nwg = 0;
        for (int i = 0; i < kMaxItems; ++i) a.offs[i] = INT32_MAX;
        for (size_t i = 0; i < L.size(); ++i) {
            a.items[i] = L[i].item;
            a.offs[i] = L[i].item.wg_off;
            nwg += (int64_t)L[i].item.tiles * cache->n_layers;
        }
        a.n_wg = (int32_t)nwg;
        const bool one = L.size() == 1;
        if (one) {
            // the item's (cos, sin) per pair, reduced and evaluated in float64
            // (the kernel's own table reduces in float64 and evaluates in float32)
            const double shift = L[0].item.shift;
            for (int j = 0; j < kMaxPairs; ++j) {
                const double u = shift * pl.omega[j];
                const double f = u - std::nearbyint(u);
                a.cs[2 * j] = (float)std::cos(2.0 * M_PI * f);
                a.cs[2 * j + 1] = (float)std::sin(2.0 * M_PI * f);
            }
        }
        hipError_t e = launch_band(a, pl.band.pfi, pl.band.rs, cache->rope_dtype == KVR_F32, one, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    for (auto& L : pl.launches) {
        RelocArgs a;
        std::memset(&a, 0, sizeof(a));
        a.pool = pl.pool;
        a.bt = d_block_tables;
        a.counters = (uint32_t*)d_ws;
        a.flags = (uint32_t*)((char*)d_ws + pl.counters_bytes);
        a.n_items = (int32_t)L.size();
        a.tile_rows = pl.tile.T;
        a.epoch = next_epoch();
        std::memcpy(a.omega, pl.omega, sizeof(a.omega));
        int64_t nwg = 0;
        for (int i = 0; i < kMaxItems; ++i) a.offs[i] = INT32_MAX;
        for (size_t i = 0; i < L.size(); ++i) {
            a.items[i] = L[i].item;
            a.offs[i] = L[i].item.wg_off;
            nwg += (int64_t)L[i].item.tiles * cache->n_layers;
        }
        a.n_wg = (int32_t)nwg;
        hipError_t e = launch_splice(a, pl.tile.pfi, pl.tile.rs, cache->rope_dtype == KVR_F32, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    return pl.forget ? KVR_FORGET_NEEDS_PREFILL : KVR_OK;
}

// ------------------------------------------------------------------ gather --

kvr_status kv_relocate_gather(const kvr_cache* dst, const int32_t* d_block_table, int32_t bt_len,
                              const kvr_rows* entries, const int64_t* p_target, int32_t n,
                              const kvr_lowrank* patch_rope, const kvr_lowrank* patch_pf,
                              hipStream_t stream) {
    Pool pool;
    double omega[kMaxPairs];
    kvr_status st = make_pool(dst, pool, omega);
    if (st != KVR_OK) return st;
    if (!d_block_table || (reinterpret_cast<uintptr_t>(d_block_table) & 3u) || bt_len < 1 || n < 0)
        return KVR_E_ARG;
    if (n > 0 && (!entries || !p_target)) return KVR_E_ARG;
    const int64_t capacity = (int64_t)bt_len * dst->block_size;
    if (capacity >= (int64_t)1 << 31) return KVR_E_ARG;
    std::vector<std::pair<int64_t, int64_t>> rng;
    for (int32_t i = 0; i < n; ++i) {
        if (entries[i].len > 0) {
            st = check_rows(entries[i], dst);
            if (st != KVR_OK) return st;
        }
        const int64_t len = entries[i].len, p = p_target[i];
        if (len < 0 || p < 0 || p + len > capacity) return KVR_E_RANGE;
        const int64_t delta = p - entries[i].base_pos;
        if (delta > INT32_MAX || delta < -(int64_t)INT32_MAX) return KVR_E_RANGE;
        if (len > 0) rng.push_back({p, p + len});
    }
    std::sort(rng.begin(), rng.end());
    for (size_t i = 1; i < rng.size(); ++i)
        if (rng[i].first < rng[i - 1].second) return KVR_E_OVERLAP;
    if (debug_checks()) {
        // the destination blocks must be distinct physical blocks
        const int64_t B = dst->block_size;
        std::vector<TableUse> use(1);
        for (const auto& r : rng) use[0].written.push_back({r.first / B, (r.second + B - 1) / B});
        st = check_ownership(d_block_table, bt_len, use, dst->n_blocks, stream);
        if (st != KVR_OK) return st;
    }
    bool any_patch = false;
    for (int32_t i = 0; i < n; ++i) {
        if (patch_rope && patch_rope[i].rank) any_patch = true;
        if (patch_pf && patch_pf[i].rank) any_patch = true;
    }
    if (any_patch) {
        st = check_patch_cache(dst);
        if (st != KVR_OK) return st;
        for (int32_t i = 0; i < n; ++i) {
            st = check_lowrank(patch_rope ? &patch_rope[i] : nullptr, entries[i].len, dst->rope_heads * dst->rope_dim);
            if (st != KVR_OK) return st;
            st = check_lowrank(patch_pf ? &patch_pf[i] : nullptr, entries[i].len, dst->pf_width);
            if (st != KVR_OK) return st;
        }
        std::vector<PatchItem> items;
        for (int32_t i = 0; i < n; ++i) {
            if (entries[i].len == 0) continue;
            PatchItem it{};
            const SrcRows s = src_rows(entries[i], dst);
            it.src_pf = s.pf; it.src_rp = s.rp;
            it.src_pf_l = s.pf_l; it.src_rp_l = s.rp_l;
            it.src_pf_r = s.pf_r; it.src_rp_r = s.rp_r;
            set_factors(patch_rope ? &patch_rope[i] : nullptr, it.U_rp, it.V_rp, it.u_rp_l, it.v_rp_l, it.rank_rp);
            set_factors(patch_pf ? &patch_pf[i] : nullptr, it.U_pf, it.V_pf, it.u_pf_l, it.v_pf_l, it.rank_pf);
            it.dst0 = (int32_t)p_target[i];
            it.shift = (int32_t)(p_target[i] - entries[i].base_pos);
            it.len = (int32_t)entries[i].len;
            it.tiles = (it.len + kPatchTileRows - 1) / kPatchTileRows;
            items.push_back(it);
        }
        return run_patch(pool, omega, d_block_table, items, dst->n_layers, false, true, true, stream);
    }

    const TileShape tile = choose_tile(pool, dst->rope_dtype == KVR_F32, false);
    const int T = tile.T;
    // Workgroups go layer after layer, each layer's tiles item after item.
    std::vector<Item> cur;
    int64_t tiles = 0;               // of the batch, per layer
    auto flush = [&]() -> kvr_status {
        if (cur.empty()) return KVR_OK;
        RelocArgs a;
        std::memset(&a, 0, sizeof(a));
        a.pool = pool;
        a.bt = d_block_table;
        a.n_items = (int32_t)cur.size();
        a.tile_rows = T;
        a.n_tiles = (int32_t)tiles;
        a.n_wg = (int32_t)(tiles * dst->n_layers);
        std::memcpy(a.omega, omega, sizeof(omega));
        for (int i = 0; i < kMaxItems; ++i) a.offs[i] = INT32_MAX;
        for (size_t i = 0; i < cur.size(); ++i) {
            a.items[i] = cur[i];
            a.offs[i] = cur[i].wg_off;
        }
        hipError_t e = launch_gather(a, tile.pfi, tile.rs, dst->rope_dtype == KVR_F32, stream);
        cur.clear();
        tiles = 0;
        return e == hipSuccess ? KVR_OK : hip_fail(e);
    };
    for (int32_t i = 0; i < n; ++i) {
        if (entries[i].len == 0) continue;
        Item it{};
        it.src = src_rows(entries[i], dst);
        it.a = (int32_t)p_target[i];
        it.shift = (int32_t)(p_target[i] - entries[i].base_pos);
        it.moved = (int32_t)entries[i].len;
        it.move_tiles = (it.moved + T - 1) / T;
        it.tiles = it.move_tiles;
        it.bt_off = 0;
        if ((int64_t)it.tiles * dst->n_layers >= ((int64_t)1 << 31)) return KVR_E_RANGE;
        if ((int)cur.size() == kMaxItems || (tiles + it.tiles) * dst->n_layers >= ((int64_t)1 << 31)) {
            st = flush();
            if (st != KVR_OK) return st;
        }
        it.wg_off = (int32_t)tiles;
        tiles += it.tiles;
        cur.push_back(it);
    }
    return flush();
}

kvr_status kv_patch_lowrank(const kvr_cache* cache, const int32_t* d_block_table, int32_t bt_len, int32_t part,
                            const int64_t* p_start, const int64_t* len, const kvr_lowrank* f, int32_t n,
                            hipStream_t stream) {
    Pool pool;
    double omega[kMaxPairs];
    kvr_status st = make_pool(cache, pool, omega);
    if (st != KVR_OK) return st;
    if (!d_block_table || (reinterpret_cast<uintptr_t>(d_block_table) & 3u) || bt_len < 1 || n < 0) return KVR_E_ARG;
    if (part != 0 && part != 1) return KVR_E_ARG;
    if (n > 0 && (!p_start || !len || !f)) return KVR_E_ARG;
    st = check_patch_cache(cache);
    if (st != KVR_OK) return st;
    const int64_t capacity = (int64_t)bt_len * cache->block_size;
    if (capacity >= (int64_t)1 << 31) return KVR_E_ARG;
    std::vector<std::pair<int64_t, int64_t>> rng;
    for (int32_t i = 0; i < n; ++i) {
        if (len[i] < 0 || p_start[i] < 0 || p_start[i] + len[i] > capacity) return KVR_E_RANGE;
        st = check_lowrank(&f[i], len[i], part ? cache->rope_heads * cache->rope_dim : cache->pf_width);
        if (st != KVR_OK) return st;
        if (len[i] > 0) rng.push_back({p_start[i], p_start[i] + len[i]});
    }
    std::sort(rng.begin(), rng.end());
    for (size_t i = 1; i < rng.size(); ++i)
        if (rng[i].first < rng[i - 1].second) return KVR_E_OVERLAP;
    std::vector<PatchItem> items;
    for (int32_t i = 0; i < n; ++i) {
        if (len[i] == 0 || f[i].rank == 0) continue;
        PatchItem it{};
        if (part == 1) set_factors(&f[i], it.U_rp, it.V_rp, it.u_rp_l, it.v_rp_l, it.rank_rp);
        else           set_factors(&f[i], it.U_pf, it.V_pf, it.u_pf_l, it.v_pf_l, it.rank_pf);
        it.dst0 = (int32_t)p_start[i];
        it.len = (int32_t)len[i];
        it.tiles = (it.len + kPatchTileRows - 1) / kPatchTileRows;
        items.push_back(it);
    }
    return run_patch(pool, omega, d_block_table, items, cache->n_layers, true, part == 1, part == 0, stream);
}

// Splits per sequence: enough workgroups to cover the 256 compute units,
// at most kDecMaxBlocks KV blocks per split.
static void decode_split(int32_t batch, int32_t max_seq_len, int32_t& n_split, int32_t& bps) {
    const int32_t blocks = std::max(1, (max_seq_len + kDecBlockTokens - 1) / kDecBlockTokens);
    n_split = std::max<int32_t>(1, (256 + batch - 1) / std::max(1, batch));
    n_split = std::max(n_split, (blocks + kDecMaxBlocks - 1) / kDecMaxBlocks);
    n_split = std::min(n_split, blocks);
    bps = (blocks + n_split - 1) / n_split;
    n_split = (blocks + bps - 1) / bps;
}

size_t kvr_decode_workspace_bytes(int32_t batch, int32_t heads, int32_t max_seq_len) {
    if (batch < 1 || heads < 32 || heads % 32 || heads > 128 || max_seq_len < 0) return 0;
    int32_t n_split, bps;
    decode_split(batch, max_seq_len, n_split, bps);
    const size_t po = (size_t)batch * n_split  * heads * 512 * 4;
    const size_t pm = (size_t)batch * n_split  * heads * 8;
    return round_up(po) + round_up(pm);
}

kvr_status mla_decode_rotate_on_read(const void* q_nope, const void* q_rope, int32_t batch, int32_t heads,
                                     const kvr_cache* cache, int32_t layer, const int32_t* d_block_tables,
                                     const int32_t* d_pending_delta, int32_t bt_stride, const int32_t* d_seq_lens,
                                     int32_t max_seq_len, float scale, void* out, float* lse, void* d_ws,
                                     size_t ws_bytes, hipStream_t stream) {
    Pool pool;
    double omega[kMaxPairs];
    kvr_status st = make_pool(cache, pool, omega);
    if (st != KVR_OK) return st;
    if (cache->pf_dtype != KVR_BF16 || cache->rope_dtype != KVR_BF16 || cache->pf_width != 512 ||
        cache->rope_heads != 1 || cache->rope_dim != 64 || cache->block_size != kDecBlockTokens)
        return KVR_E_UNSUPPORTED;
    if (batch < 1 || heads < 32 || heads % 32 || heads > 128) return KVR_E_UNSUPPORTED;
    if (layer < 0 || layer >= cache->n_layers) return KVR_E_RANGE;
    if (!q_nope || !q_rope || !aligned16(q_nope) || !aligned16(q_rope) || !out || !lse) return KVR_E_ARG;
    if (!d_block_tables || !d_pending_delta || !d_seq_lens || bt_stride < 1) return KVR_E_ARG;
    if ((reinterpret_cast<uintptr_t>(d_block_tables) | reinterpret_cast<uintptr_t>(d_pending_delta) |
         reinterpret_cast<uintptr_t>(d_seq_lens) | reinterpret_cast<uintptr_t>(lse)) & 3u)
        return KVR_E_ARG;
    if ((reinterpret_cast<uintptr_t>(out) & 1u) || !std::isfinite(scale)) return KVR_E_ARG;
    if (max_seq_len < 0 || (int64_t)max_seq_len > (int64_t)bt_stride * kDecBlockTokens) return KVR_E_RANGE;
    const size_t need = kvr_decode_workspace_bytes(batch, heads, max_seq_len);
    if (!d_ws || (reinterpret_cast<uintptr_t>(d_ws) % kAlign) || ws_bytes < need) return KVR_E_WORKSPACE;

    DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.ckv = pool.pf + (int64_t)layer * pool.pf_l;
    a.ckv_b = pool.pf_b;
    a.ckv_r = pool.pf_r;
    a.kr = pool.rp + (int64_t)layer * pool.rp_l;
    a.kr_b = pool.rp_b;
    a.kr_r = pool.rp_r;
    a.n_blocks = pool.n_blocks;
    a.q_nope = (const uint16_t*)q_nope;
    a.q_rope = (const uint16_t*)q_rope;
    a.bt = d_block_tables;
    a.pend = d_pending_delta;
    a.seq_lens = d_seq_lens;
    a.bt_stride = bt_stride;
    a.max_len = max_seq_len;
    a.batch = batch;
    a.heads = heads;
    decode_split(batch, max_seq_len, a.n_split, a.blocks_per_split);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.part_o = (float*)d_ws;
    a.part_ml = (float*)((char*)d_ws + round_up((size_t)batch * a.n_split  * heads * 512 * 4));
    std::memcpy(a.omega, omega, sizeof(a.omega));
    hipError_t e = launch_decode(a, (uint16_t*)out, lse, stream);
    return e == hipSuccess ? KVR_OK : hip_fail(e);
}

// Splits of the GQA decode: about 2048 single-wave workgroups in all, at most
// kGqaMaxBlocks blocks per split.
static void gqa_split(int32_t batch, int32_t kv_heads, int32_t max_seq_len, int32_t& n_split, int32_t& bps) {
    const int32_t blocks = std::max(1, (max_seq_len + kDecBlockTokens - 1) / kDecBlockTokens);
    const int32_t pairs = std::max(1, batch * kv_heads);
    n_split = std::max<int32_t>(1, (2048 + pairs - 1) / pairs);
    n_split = std::max(n_split, (blocks + kGqaMaxBlocks - 1) / kGqaMaxBlocks);
    n_split = std::min(n_split, blocks);
    bps = (blocks + n_split - 1) / n_split;
    n_split = (blocks + bps - 1) / bps;
}

size_t kvr_gqa_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t max_seq_len) {
    if (batch < 1 || kv_heads < 1 || q_heads < kv_heads || q_heads % kv_heads ||
        q_heads / kv_heads > kGqaMaxGroup || max_seq_len < 0)
        return 0;
    int32_t n_split, bps;
    gqa_split(batch, kv_heads, max_seq_len, n_split, bps);
    const size_t rows = (size_t)batch * n_split * q_heads;
    return round_up(rows * kGqaDim * 4) + round_up(rows * 8);
}

kvr_status gqa_decode_rotate_on_read(const void* q, int32_t batch, int32_t q_heads, const kvr_cache* cache,
                                     int32_t layer, const int32_t* d_block_tables, const int32_t* d_pending_delta,
                                     int32_t bt_stride, const int32_t* d_seq_lens, int32_t max_seq_len, float scale,
                                     void* out, float* lse, void* d_ws, size_t ws_bytes, hipStream_t stream) {
    Pool pool;
    double omega[kMaxPairs];
    kvr_status st = make_pool(cache, pool, omega);
    if (st != KVR_OK) return st;
    const int32_t G = cache->rope_heads;
    if (cache->pf_dtype != KVR_BF16 || cache->rope_dtype != KVR_BF16 || cache->rope_dim != kGqaDim ||
        cache->pf_width != G * kGqaDim || cache->block_size != kDecBlockTokens)
        return KVR_E_UNSUPPORTED;
    if (batch < 1 || q_heads < G || q_heads % G || q_heads / G > kGqaMaxGroup) return KVR_E_UNSUPPORTED;
    if (layer < 0 || layer >= cache->n_layers) return KVR_E_RANGE;
    if (!q || !aligned16(q) || !out || !lse) return KVR_E_ARG;
    if (!d_block_tables || !d_pending_delta || !d_seq_lens || bt_stride < 1) return KVR_E_ARG;
    if ((reinterpret_cast<uintptr_t>(d_block_tables) | reinterpret_cast<uintptr_t>(d_pending_delta) |
         reinterpret_cast<uintptr_t>(d_seq_lens) | reinterpret_cast<uintptr_t>(lse)) & 3u)
        return KVR_E_ARG;
    if ((reinterpret_cast<uintptr_t>(out) & 1u) || !std::isfinite(scale)) return KVR_E_ARG;
    // the direct loads address rows with 32-bit offsets from a block's row
    if (pool.pf_r > (1 << 24) || pool.rp_r > (1 << 24)) return KVR_E_UNSUPPORTED;
    if (max_seq_len < 0 || (int64_t)max_seq_len > (int64_t)bt_stride * kDecBlockTokens) return KVR_E_RANGE;
    const size_t need = kvr_gqa_decode_workspace_bytes(batch, q_heads, G, max_seq_len);
    if (!d_ws || (reinterpret_cast<uintptr_t>(d_ws) % kAlign) || ws_bytes < need) return KVR_E_WORKSPACE;

    GqaDecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.k = pool.rp + (int64_t)layer * pool.rp_l;
    a.k_b = pool.rp_b;
    a.k_r = pool.rp_r;
    a.v = pool.pf + (int64_t)layer * pool.pf_l;
    a.v_b = pool.pf_b;
    a.v_r = pool.pf_r;
    a.n_blocks = pool.n_blocks;
    a.q = (const uint16_t*)q;
    a.bt = d_block_tables;
    a.pend = d_pending_delta;
    a.seq_lens = d_seq_lens;
    a.bt_stride = bt_stride;
    a.max_len = max_seq_len;
    a.batch = batch;
    a.q_heads = q_heads;
    a.kv_heads = G;
    a.group = q_heads / G;
    gqa_split(batch, G, max_seq_len, a.n_split, a.blocks_per_split);
    a.scale_log2 = scale * 1.4426950408889634f;
    const size_t rows = (size_t)batch * a.n_split * q_heads;
    a.part_o = (float*)d_ws;
    a.part_ml = (float*)((char*)d_ws + round_up(rows * kGqaDim * 4));
    for (int j = 0; j < kGqaDim / 2; ++j) a.omega[j] = omega[j];
    hipError_t e = launch_gqa_decode(a, (uint16_t*)out, lse, stream);
    return e == hipSuccess ? KVR_OK : hip_fail(e);
}

size_t kvr_patch_factors_workspace_bytes(int32_t n, int32_t orders, int32_t rows, int32_t cols) {
    if (n < 0 || orders < 1 || rows < 1 || cols < 1) return 0;
    const size_t y = round_up((size_t)n * rows * kFormSketch * 4);
    const size_t z = round_up((size_t)n * cols * kFormSketch * 4);
    const size_t m = orders > 1 ? round_up((size_t)n * rows * cols * 4) : 0;
    return std::max<size_t>(kAlign, y + z + m);
}

kvr_status kamera_patch_factors(const float* d_deficits, int32_t n, int32_t orders, int32_t rows, int32_t cols,
                                int32_t rank, const float* d_omega, float* d_U, float* d_V, float* d_sigma,
                                void* d_ws, size_t ws_bytes, hipStream_t stream) {
    if (n < 0 || orders < 1) return KVR_E_ARG;
    if (rank < 1 || rank > kFormMaxRank) return KVR_E_UNSUPPORTED;
    if (rows < 64 || cols < 64 || rows % 64 || cols % 64 || rows > 16384 || cols > 16384) return KVR_E_UNSUPPORTED;
    if (n == 0) return KVR_OK;
    if ((int64_t)n * (std::max(rows, cols) / 64) >= ((int64_t)1 << 31)) return KVR_E_RANGE;
    if (!d_deficits || !d_omega || !d_U || !d_V || !d_sigma) return KVR_E_ARG;
    if (!aligned16(d_deficits) || !aligned16(d_omega) || (reinterpret_cast<uintptr_t>(d_U) & 3u) ||
        (reinterpret_cast<uintptr_t>(d_V) & 3u) || (reinterpret_cast<uintptr_t>(d_sigma) & 3u))
        return KVR_E_ARG;
    const size_t need = kvr_patch_factors_workspace_bytes(n, orders, rows, cols);
    if (!d_ws || (reinterpret_cast<uintptr_t>(d_ws) % kAlign) || ws_bytes < need) return KVR_E_WORKSPACE;
    float* Y = (float*)d_ws;
    float* Z = (float*)((char*)d_ws + round_up((size_t)n * rows * kFormSketch * 4));
    const float* D = d_deficits;
    const int64_t per = (int64_t)rows * cols;
    hipError_t e;
    if (orders > 1) {
        float* Dm = (float*)((char*)Z + round_up((size_t)n * cols * kFormSketch * 4));
        e = launch_form_mean(d_deficits, orders, per, n, Dm, stream);
        if (e != hipSuccess) return hip_fail(e);
        D = Dm;
    }
    FormGemmArgs g;
    std::memset(&g, 0, sizeof(g));
    g.D = D;
    g.d_stride = per;
    g.n = n;
    g.rows = rows;
    g.cols = cols;
    // Y = D Omega; twice: Z = D^T Y, Z = orth(Z), Y = D Z.  For widths the
    // one-pass kernel takes, each Z = D^T (D X) is one pass over D (X = Omega,
    // then the orthonormalized Z) and only the last Y is formed.
    const bool one_pass = cols % 256 == 0 && cols <= kFormPowerMaxCols;
    FormOrthArgs o{Z, cols};
    if (one_pass) {
        g.X = d_omega; g.x_stride = 0; g.Y = Z; g.y_stride = (int64_t)cols * kFormSketch;
        if ((e = launch_form_power(g, stream)) != hipSuccess) return hip_fail(e);
        if ((e = launch_form_orth(o, n, stream)) != hipSuccess) return hip_fail(e);
        g.X = Z; g.x_stride = (int64_t)cols * kFormSketch;       // in place: a wave reads its rows of X
        if ((e = launch_form_power(g, stream)) != hipSuccess) return hip_fail(e);   // before it writes them
        if ((e = launch_form_orth(o, n, stream)) != hipSuccess) return hip_fail(e);
        g.Y = Y; g.y_stride = (int64_t)rows * kFormSketch;
        if ((e = launch_form_gemm(g, false, stream)) != hipSuccess) return hip_fail(e);
    } else {
        g.X = d_omega; g.x_stride = 0; g.Y = Y; g.y_stride = (int64_t)rows * kFormSketch;
        if ((e = launch_form_gemm(g, false, stream)) != hipSuccess) return hip_fail(e);
        for (int step = 0; step < 2; ++step) {
            g.X = Y; g.x_stride = (int64_t)rows * kFormSketch; g.Y = Z; g.y_stride = (int64_t)cols * kFormSketch;
            if ((e = launch_form_gemm(g, true, stream)) != hipSuccess) return hip_fail(e);
            if ((e = launch_form_orth(o, n, stream)) != hipSuccess) return hip_fail(e);
            g.X = Z; g.x_stride = (int64_t)cols * kFormSketch; g.Y = Y; g.y_stride = (int64_t)rows * kFormSketch;
            if ((e = launch_form_gemm(g, false, stream)) != hipSuccess) return hip_fail(e);
        }
    }
    FormEigArgs ea{Y, Z, d_U, d_V, d_sigma, rows, cols, rank};
    e = launch_form_eig(ea, n, stream);
    return e == hipSuccess ? KVR_OK : hip_fail(e);
}

kvr_status leyline_splice_lazy(int32_t block_size, int32_t* d_block_tables, int32_t* d_pending_delta,
                               int32_t bt_stride, int32_t n_seq, const int64_t* seq_lens,
                               const kvr_directive* dirs, const int32_t* d_stub_blocks,
                               int32_t* d_freed_blocks, int64_t* new_lens, hipStream_t stream) {
    if (block_size <= 0 || bt_stride <= 0 || bt_stride > kLazyMaxBlocks || n_seq < 0) return KVR_E_ARG;
    if (n_seq > 0 && (!d_block_tables || !d_pending_delta || !seq_lens || !dirs || !new_lens)) return KVR_E_ARG;
    const int64_t B = block_size, cap = (int64_t)bt_stride * B;
    // validate everything first: no table is touched unless all sequences pass
    int64_t n_stub = 0, n_free = 0;
    bool forget = false;
    std::vector<int64_t> out(n_seq);
    for (int32_t b = 0; b < n_seq; ++b) {
        const kvr_directive& d = dirs[b];
        const int64_t N = seq_lens[b];
        if (d.mode != KVR_AMORTIZE && d.mode != KVR_FORGET) return KVR_E_ARG;
        if (N < 0 || N > cap || d.s_start < 0 || d.s_start > d.s_end || d.s_end > N || d.r_len < 0)
            return KVR_E_RANGE;
        if (d.mode == KVR_FORGET) {
            out[b] = d.s_start;
            forget = true;
            continue;
        }
        if (d.s_start % B || d.s_end % B || d.r_len % B) return KVR_E_ARG;
        const int64_t delta = d.r_len - (d.s_end - d.s_start);
        if (N + delta > cap) return KVR_E_CAPACITY;
        out[b] = N + delta;
        n_stub += d.r_len / B;
        n_free += (d.s_end - d.s_start) / B;
    }
    if ((n_stub > 0 && !d_stub_blocks) || (n_free > 0 && !d_freed_blocks)) return KVR_E_ARG;
    if (n_stub >= ((int64_t)1 << 31) || n_free >= ((int64_t)1 << 31)) return KVR_E_RANGE;

    LazyArgs a;
    std::memset(&a, 0, sizeof(a));
    a.bt = d_block_tables;
    a.pend = d_pending_delta;
    a.stubs = d_stub_blocks;
    a.freed = d_freed_blocks;
    a.bt_stride = bt_stride;
    a.block_size = block_size;
    int32_t stub_off = 0, free_off = 0;
    auto flush = [&]() -> kvr_status {
        hipError_t e = launch_lazy(a, stream);
        a.n_seq = 0;
        return e == hipSuccess ? KVR_OK : hip_fail(e);
    };
    for (int32_t b = 0; b < n_seq; ++b) {
        const kvr_directive& d = dirs[b];
        if (d.mode == KVR_FORGET) continue;
        const int64_t N = seq_lens[b];
        LazySeq s;
        s.row = b;
        s.n_old = (int32_t)((N + B - 1) / B);
        s.n_new = (int32_t)((out[b] + B - 1) / B);
        s.s0b = (int32_t)(d.s_start / B);
        s.s1b = (int32_t)(d.s_end / B);
        s.rb = (int32_t)(d.r_len / B);
        s.delta = (int32_t)(out[b] - N);
        s.stub_off = stub_off;
        s.free_off = free_off;
        stub_off += s.rb;
        free_off += s.s1b - s.s0b;
        a.seqs[a.n_seq++] = s;
        if (a.n_seq == kLazyMaxSeq) {
            kvr_status st = flush();
            if (st != KVR_OK) return st;
        }
    }
    if (a.n_seq > 0) {
        kvr_status st = flush();
        if (st != KVR_OK) return st;
    }
    for (int32_t b = 0; b < n_seq; ++b) new_lens[b] = out[b];
    return forget ? KVR_FORGET_NEEDS_PREFILL : KVR_OK;
}

kvr_status kv_relocate_gather_lazy(int32_t block_size, int32_t* d_block_tables, int32_t* d_pending_delta,
                                   int32_t bt_stride, int32_t n_seq, const kvr_lazy_entry* entries, int32_t n,
                                   int32_t* d_replaced, hipStream_t stream) {
    if (block_size <= 0 || bt_stride <= 0 || bt_stride > kLazyMaxBlocks || n < 0 || n_seq < 0) return KVR_E_ARG;
    if (n == 0) return KVR_OK;
    if (!d_block_tables || !d_pending_delta || !entries) return KVR_E_ARG;
    const int64_t B = block_size, cap = (int64_t)bt_stride * B;
    // validate everything first: no table is touched unless all entries pass
    std::vector<std::vector<std::pair<int64_t, int64_t>>> used(n_seq);   // block ranges per sequence
    int64_t total = 0;
    for (int32_t e = 0; e < n; ++e) {
        const kvr_lazy_entry& E = entries[e];
        if (E.seq < 0 || E.seq >= n_seq) return KVR_E_ARG;
        if (E.len < 0 || E.p_target < 0 || E.p_target > cap - E.len) return KVR_E_RANGE;
        if (E.p_target % B) return KVR_E_ARG;
        // |p_target - base_pos| < 2^31 (p_target <= 2^44, so neither bound overflows)
        if (E.base_pos <= E.p_target - ((int64_t)1 << 31) || E.base_pos >= E.p_target + ((int64_t)1 << 31))
            return KVR_E_RANGE;
        const int64_t nb = (E.len + B - 1) / B;
        if (nb > 0 && !E.d_blocks) return KVR_E_ARG;
        if (nb > 0) used[E.seq].push_back({E.p_target / B, E.p_target / B + nb});
        total += nb;
    }
    for (auto& v : used) {
        std::sort(v.begin(), v.end());
        for (size_t i = 1; i < v.size(); ++i)
            if (v[i].first < v[i - 1].second) return KVR_E_OVERLAP;   // non-empty, sorted by start
    }
    if (total >= ((int64_t)1 << 31)) return KVR_E_RANGE;

    LazyGatherArgs a;
    std::memset(&a, 0, sizeof(a));
    a.bt = d_block_tables;
    a.pend = d_pending_delta;
    a.replaced = d_replaced;
    a.bt_stride = bt_stride;
    int32_t off = 0;
    for (int32_t e = 0; e < n; ++e) {
        const kvr_lazy_entry& E = entries[e];
        const int32_t nb = (int32_t)((E.len + B - 1) / B);
        if (nb > 0) {
            LazyEntry& L = a.ents[a.n++];
            L.blocks = E.d_blocks;
            L.pend = E.d_pend;
            L.row = E.seq;
            L.slot0 = (int32_t)(E.p_target / B);
            L.nb = nb;
            L.delta = (int32_t)(E.p_target - E.base_pos);
            L.rep_off = off;
        }
        off += nb;
        if (a.n == kLazyMaxEntries || (e == n - 1 && a.n > 0)) {
            hipError_t err = launch_lazy_gather(a, stream);
            if (err != hipSuccess) return hip_fail(err);
            a.n = 0;
        }
    }
    return KVR_OK;
}

size_t kvr_keys_workspace_bytes(int64_t total_tokens) {
    if (total_tokens <= 0) return kAlign;
    return round_up((size_t)((total_tokens + 63) / 64) * 8);
}

kvr_status registry_chunk_keys(const int32_t* d_tokens, const int64_t* offsets, int32_t n_streams,
                               const uint64_t* d_gear, int32_t vocab, const kvr_cdc_params* params,
                               uint64_t* d_hash, int32_t* d_chunk_end, int32_t chunk_cap, int32_t* d_n_chunks,
                               uint64_t* d_chunk_fp, uint64_t* d_s1_fp, void* d_ws, size_t ws_bytes,
                               hipStream_t stream) {
    if (n_streams < 0 || !params) return KVR_E_ARG;
    if (n_streams > kKeyMaxStreams) return KVR_E_UNSUPPORTED;
    if (n_streams == 0) return KVR_OK;
    if (!offsets || !d_tokens || !d_gear || vocab <= 0 || !d_chunk_end || !d_n_chunks || !d_chunk_fp)
        return KVR_E_ARG;
    const kvr_cdc_params& P = *params;
    if (P.min_len < 1 || P.max_len < P.min_len || P.s1_window < 1) return KVR_E_ARG;
    if (offsets[0] < 0) return KVR_E_RANGE;
    for (int32_t s = 0; s < n_streams; ++s) {
        const int64_t len = offsets[s + 1] - offsets[s];
        if (len < 0 || len >= ((int64_t)1 << 31)) return KVR_E_RANGE;
        if (chunk_cap < (len + P.min_len - 1) / P.min_len) return KVR_E_ARG;
    }
    if (chunk_cap < 1 || (int64_t)chunk_cap * n_streams >= ((int64_t)1 << 31)) return KVR_E_ARG;
    const int64_t n_tok = offsets[n_streams] - offsets[0];
    const size_t need = kvr_keys_workspace_bytes(n_tok);
    if (!d_ws || (reinterpret_cast<uintptr_t>(d_ws) % kAlign) || ws_bytes < need) return KVR_E_WORKSPACE;
    KeyArgs a;
    std::memset(&a, 0, sizeof(a));
    a.tokens = d_tokens;
    a.gear = d_gear;
    a.hash = d_hash;
    a.cand = (uint64_t*)d_ws;
    a.chunk_end = d_chunk_end;
    a.n_chunks = d_n_chunks;
    a.chunk_fp = d_chunk_fp;
    a.s1_fp = d_s1_fp;
    a.threshold = P.threshold;
    a.seed = P.seed;
    a.total = offsets[n_streams];
    a.vocab = vocab;
    a.min_len = P.min_len;
    a.max_len = P.max_len;
    a.s1_window = P.s1_window;
    a.s1_slots = (P.max_len + P.s1_window - 1) / P.s1_window;
    a.cap = chunk_cap;
    a.n_streams = n_streams;
    for (int32_t s = 0; s <= n_streams; ++s) a.offsets[s] = offsets[s];
    hipError_t e = launch_keys(a, stream);
    return e == hipSuccess ? KVR_OK : hip_fail(e);
}

}  // extern "C"
