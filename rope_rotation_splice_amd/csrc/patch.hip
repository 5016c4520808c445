// Kamera's reuse operator with its rank-m conditioning patch (section 2):
//   K_out = R(delta) K + U V^T,   V_out = V + U' V'^T
// fused into the relocating gather (registry rows -> paged destination), and
// the same patch applied in place to rows already in the cache.
//
// The low-rank product is a contraction over the rank (K dimension 4..64), so
// it runs on the fp32 matrix cores: v_mfma_f32_16x16x4f32 with the features
// as the M dimension and 16 tokens as N.  In that instruction lane l holds
// output rows 4*(l/16) + r (r < 4) of column l % 16.  Two instructions per
// 32-feature group with interleaved feature orders (set a: 8*(i/4) + i%4,
// set b: the same + 4) leave lane l = (token l%16, g = l/16) holding features
// 8g .. 8g+7 of the group -- exactly the 16-byte bf16 chunk that lane loads
// from memory, so the patch is added in registers, with no LDS transpose,
// after the fp32 rotation and before the single rounding to bf16.  The K
// dimension is walked in blocks of 16: in step kk lane q = l/16 supplies rank
// index 16*kb + 4q + kk, so every operand is one float4 load.
//
// The rotary part is processed in pairs of 32-feature groups (lo half x_j and
// hi half x_{j+d/2} of a head) so each rotation pair stays inside one lane.
#include "kvr_device.h"
#include "kvr_internal.h"

#include "../../include/kvreloc.h"

namespace kvr {

__device__ uint32_t g_errors_patch;

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void raise_error(uint32_t bit) {
    __hip_atomic_fetch_or(&g_errors_patch, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Accumulate the patch of one 32-feature group for this lane's token:
// acc_a / acc_b receive features 8g..8g+3 / 8g+4..8g+7 (g = lane/16).
// Vg points at the factor row of feature 0 of the group (rank floats per row),
// Ut at the U row of this lane's token (nullptr for a token outside the tile).
__device__ __forceinline__ void group_patch(const float* __restrict__ Vg, const float* __restrict__ Ut,
                                            int rank, int lane, v4f& acc_a, v4f& acc_b) {
    const int i = lane & 15, q = lane >> 4;
    const int fa = 8 * (i >> 2) + (i & 3);           // feature of A row i in set a
    const float* va = Vg + (int64_t)fa * rank;
    const float* vb = Vg + (int64_t)(fa + 4) * rank;
    for (int k0 = 0; k0 < rank; k0 += 16) {
        const int k = k0 + 4 * q;
        v4f a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0}, b = {0, 0, 0, 0};
        if (k < rank) {
            a0 = *reinterpret_cast<const v4f*>(va + k);
            a1 = *reinterpret_cast<const v4f*>(vb + k);
            if (Ut) b = *reinterpret_cast<const v4f*>(Ut + k);
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            acc_a = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[kk], b[kk], acc_a, 0, 0, 0);
            acc_b = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[kk], b[kk], acc_b, 0, 0, 0);
        }
    }
}

// 8 bf16 of a chunk + 8 fp32 patch values -> 8 bf16 (one rounding).
__device__ __forceinline__ v4u add_patch(v4u x, v4f pa, v4f pb) {
    v4u y;
    y[0] = pack_bf16(bf_lo(x[0]) + pa[0], bf_hi(x[0]) + pa[1]);
    y[1] = pack_bf16(bf_lo(x[1]) + pa[2], bf_hi(x[1]) + pa[3]);
    y[2] = pack_bf16(bf_lo(x[2]) + pb[0], bf_hi(x[2]) + pb[1]);
    y[3] = pack_bf16(bf_lo(x[3]) + pb[2], bf_hi(x[3]) + pb[3]);
    return y;
}

// Rotate a lo/hi chunk pair in fp32, add the patches (if any), round once to
// bf16.  With neither a rotation nor a patch the chunks are left untouched.
__device__ __forceinline__ void rot_patch(v4u& lo, v4u& hi, const float2* cs, bool rotate, bool patched,
                                          v4f pla, v4f plb, v4f pha, v4f phb) {
    if (!rotate && !patched) return;
    float xl[8], xh[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        xl[2 * w] = bf_lo(lo[w]); xl[2 * w + 1] = bf_hi(lo[w]);
        xh[2 * w] = bf_lo(hi[w]); xh[2 * w + 1] = bf_hi(hi[w]);
    }
    if (rotate) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a, b;
            rot2(xl[e], xh[e], cs[e].x, cs[e].y, a, b);
            xl[e] = a; xh[e] = b;
        }
    }
    if (patched) {
        const float pl[8] = {pla[0], pla[1], pla[2], pla[3], plb[0], plb[1], plb[2], plb[3]};
        const float ph[8] = {pha[0], pha[1], pha[2], pha[3], phb[0], phb[1], phb[2], phb[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) { xl[e] += pl[e]; xh[e] += ph[e]; }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        lo[w] = pack_bf16(xl[2 * w], xl[2 * w + 1]);
        hi[w] = pack_bf16(xh[2 * w], xh[2 * w + 1]);
    }
}

// Every tile of an (item, layer) re-reads that layer's factors: with
// xcd_contiguous the tiles of one (item, layer) share one XCD's L2.

template <bool INPLACE>
__global__ __launch_bounds__(kThreads) void patch_kernel(const PatchArgs A) {
    __shared__ float2 s_cs[kPatchMaxPairs];
    __shared__ int32_t s_blk[kMaxTileRows], s_row[kMaxTileRows];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bid = xcd_contiguous(blockIdx.x, gridDim.x);
    const Pool& P = A.pool;

    int it = 0;
    {
        int hi = A.n_items - 1;
        while (it < hi) {
            const int mid = (it + hi + 1) >> 1;
            if (bid >= A.items[mid].wg_off) it = mid; else hi = mid - 1;
        }
    }
    const PatchItem& I = A.items[it];
    const int local = bid - I.wg_off;
    const int layer = local / I.tiles;
    const int t = local - layer * I.tiles;
    const int T = A.tile_rows;
    const int r0 = t * T;
    const int nrows = min(T, I.len - r0);
    const int dslot0 = I.dst0 + r0;
    const int32_t* bt = A.bt;

    if (tid < nrows) {
        const int slot = dslot0 + tid;
        const int idx = P.bs_shift >= 0 ? (slot >> P.bs_shift) : slot / P.block_size;
        const int blk = bt[idx];
        const bool ok = (unsigned)blk < (unsigned)P.n_blocks;
        if (!ok) raise_error(KVR_DEV_BAD_BLOCK);
        s_blk[tid] = ok ? blk : -1;
        s_row[tid] = slot - idx * P.block_size;
    }
    const bool rotate = !INPLACE && I.shift != 0;
    if (rotate) angle_table(s_cs, A.omega, P.n_pairs, I.shift, tid);
    __syncthreads();

    const int tok = lane & 15, g = lane >> 4;
    const int64_t lpf = (int64_t)layer * P.pf_l, lrp = (int64_t)layer * P.rp_l;

    // Work of a wave: whole rotary heads (every 32-feature group of the head,
    // so the two 64-byte halves of each 128-byte line are read and written by
    // the same wave in consecutive instructions) and pairs of position-free
    // groups (128 bytes).  The tile's four sub-tiles of 16 tokens are taken at once:
    // all their loads are issued before the matrix cores run.  For rank <= 16
    // (one K block) the U rows of this lane's token stay in registers for the
    // whole tile and each group's factor rows are loaded once per unit; larger
    // ranks walk the K blocks with operand reloads (group_patch).
    constexpr int NS = kPatchTileRows / 16;
    constexpr int NB = 4;                      // sub-tiles per batch
    constexpr int MAXG = 4;                    // groups per unit (a 128-dim head)

    auto load_u = [&](const float* Ul, int rank, v4f* ub) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int row = s * 16 + tok;
            ub[s] = v4f{0, 0, 0, 0};
            if (row < nrows && 4 * g < rank) ub[s] = *reinterpret_cast<const v4f*>(Ul + (int64_t)(r0 + row) * rank + 4 * g);
        }
    };
    auto load_f = [&](const float* Vl, int f0, int rank, v4f& fa, v4f& fb) {
        fa = v4f{0, 0, 0, 0};
        fb = fa;
        if (4 * g < rank) {
            const int fr = f0 + 8 * (tok >> 2) + (tok & 3);
            fa = *reinterpret_cast<const v4f*>(Vl + (int64_t)fr * rank + 4 * g);
            fb = *reinterpret_cast<const v4f*>(Vl + (int64_t)(fr + 4) * rank + 4 * g);
        }
    };
    auto mfma16 = [&](v4f fa, v4f fb, v4f u, v4f& pa, v4f& pb) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            pa = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[kk], u[kk], pa, 0, 0, 0);
            pb = __builtin_amdgcn_mfma_f32_16x16x4f32(fb[kk], u[kk], pb, 0, 0, 0);
        }
    };

    // ---- rotary part: units = heads -----------------------------------------
    if (A.do_rope) {
        const int gph = P.head_bytes / 64;           // 32-feature groups per head (2 or 4)
        const int hg = gph / 2;                      // groups per half head
        const int heads = P.rope_items / P.half_chunks;
        const float* Ul = I.U_rp ? I.U_rp + (int64_t)layer * I.u_rp_l : nullptr;
        const float* Vl = I.V_rp ? I.V_rp + (int64_t)layer * I.v_rp_l : nullptr;
        const int rank = I.rank_rp;
        const bool small = rank > 0 && rank <= 16;
        v4f ub[NS];
        if (small) load_u(Ul, rank, ub);
        for (int head = wave; head < heads; head += kThreads / 64) {
            const int f_head = head * gph * 32;
            v4f fa[MAXG], fb[MAXG];
            if (small) {
#pragma unroll
                for (int gi = 0; gi < MAXG; ++gi)
                    if (gi < gph) load_f(Vl, f_head + gi * 32, rank, fa[gi], fb[gi]);
            }
#pragma unroll
            for (int sb = 0; sb < NS; sb += NB) {
                if (sb * 16 >= nrows) break;
                v4u x[NB][MAXG];
                char* dst[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int row = (sb + b) * 16 + tok;
                    dst[b] = nullptr;
                    if (row < nrows && s_blk[row] >= 0) {
                        dst[b] = P.rp + lrp + (int64_t)s_blk[row] * P.rp_b + (int64_t)s_row[row] * P.rp_r +
                                 head * P.head_bytes + g * 16;
                        const char* src = INPLACE ? dst[b]
                                                  : I.src_rp + (int64_t)layer * I.src_rp_l +
                                                        (int64_t)(r0 + row) * I.src_rp_r + head * P.head_bytes + g * 16;
#pragma unroll
                        for (int gi = 0; gi < MAXG; ++gi)
                            if (gi < gph) x[b][gi] = ld16(src + gi * 64);
                    }
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int s = sb + b;
                    if (s * 16 >= nrows) break;
#pragma unroll
                    for (int gl = 0; gl < MAXG / 2; ++gl) {
                        if (gl >= hg) break;
                        // hi group of this pair: gl + hg (hg is 1 or 2; indices stay compile-time)
                        const int gh = gl + hg;
                        v4f pla = {0, 0, 0, 0}, plb = pla, pha = pla, phb = pla;
                        if (small) {
                            mfma16(fa[gl], fb[gl], ub[s], pla, plb);
                            mfma16(hg == 1 ? fa[gl + 1] : fa[gl + 2], hg == 1 ? fb[gl + 1] : fb[gl + 2], ub[s], pha, phb);
                        } else if (rank > 0) {
                            const int row = s * 16 + tok;
                            const float* Ut = (row < nrows) ? Ul + (int64_t)(r0 + row) * rank : nullptr;
                            group_patch(Vl + (int64_t)(f_head + gl * 32) * rank, Ut, rank, lane, pla, plb);
                            group_patch(Vl + (int64_t)(f_head + gh * 32) * rank, Ut, rank, lane, pha, phb);
                        }
                        if (dst[b] && (rotate || rank > 0 || !INPLACE)) {
                            v4u lo = x[b][gl], hi = hg == 1 ? x[b][gl + 1] : x[b][gl + 2];
                            rot_patch(lo, hi, s_cs + gl * 32 + g * 8, rotate, rank > 0, pla, plb, pha, phb);
                            st16(dst[b] + gl * 64, lo);
                            st16(dst[b] + gh * 64, hi);
                        }
                    }
                }
            }
        }
    }

    // ---- position-free part: units = pairs of 32-feature groups (128 B) ------
    if (A.do_pf) {
        const int pairs = P.pf_chunks / 8;
        const float* Ul = I.U_pf ? I.U_pf + (int64_t)layer * I.u_pf_l : nullptr;
        const float* Vl = I.V_pf ? I.V_pf + (int64_t)layer * I.v_pf_l : nullptr;
        const int rank = I.rank_pf;
        const bool small = rank > 0 && rank <= 16;
        v4f ub[NS];
        if (small) load_u(Ul, rank, ub);
        for (int q = wave; q < pairs; q += kThreads / 64) {
            v4f fa[2], fb[2];
            if (small) {
                load_f(Vl, q * 64, rank, fa[0], fb[0]);
                load_f(Vl, q * 64 + 32, rank, fa[1], fb[1]);
            }
#pragma unroll
            for (int sb = 0; sb < NS; sb += NB) {
                if (sb * 16 >= nrows) break;
                v4u x[NB][2];
                char* dst[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int row = (sb + b) * 16 + tok;
                    dst[b] = nullptr;
                    if (row < nrows && s_blk[row] >= 0) {
                        dst[b] = P.pf + lpf + (int64_t)s_blk[row] * P.pf_b + (int64_t)s_row[row] * P.pf_r + q * 128 + g * 16;
                        const char* src = INPLACE ? dst[b]
                                                  : I.src_pf + (int64_t)layer * I.src_pf_l +
                                                        (int64_t)(r0 + row) * I.src_pf_r + q * 128 + g * 16;
                        x[b][0] = ld16(src);
                        x[b][1] = ld16(src + 64);
                    }
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int s = sb + b;
                    if (s * 16 >= nrows) break;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        if (rank > 0) {
                            v4f pa = {0, 0, 0, 0}, pb = pa;
                            if (small) {
                                mfma16(fa[h], fb[h], ub[s], pa, pb);
                            } else {
                                const int row = s * 16 + tok;
                                const float* Ut = (row < nrows) ? Ul + (int64_t)(r0 + row) * rank : nullptr;
                                group_patch(Vl + (int64_t)(q * 64 + h * 32) * rank, Ut, rank, lane, pa, pb);
                            }
                            if (dst[b]) st16(dst[b] + h * 64, add_patch(x[b][h], pa, pb));
                        } else if (dst[b] && !INPLACE) {
                            st16(dst[b] + h * 64, x[b][h]);      // no patch: bit-exact copy
                        }
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming form.  One workgroup per (item, layer, unit), a unit being 256
// bytes of the row: a 128-dimension rotary head or 128 position-free
// features.  The unit's feature-side factor rows are loaded into registers
// once; each wave then streams its 16-row sub-tiles (wave w takes sub-tiles
// w, w + 4, ...) global -> LDS directly, data and U rows, 3 stages ahead,
// from inline assembly (no registers hold data in flight, no barriers: a
// wave reads only what it loaded itself).  Results are written back to
// their LDS slots and stored row by row, so every store covers whole
// 128-byte lines.  Every stage issues exactly 5
// direct loads and 4 stores, so the vmcnt waits are exact: rows outside the
// item or behind a bad block id load a clamped in-range row and store into
// g_patch_sink instead of being skipped.
constexpr int kDmaRows = 16;                        // rows per stage (one MFMA sub-tile)
constexpr int kDmaBuf = 4;                          // stage buffers per wave (3 loads ahead)
constexpr int kDmaDataB = kDmaRows * 256;           // 4 KB of row data per stage
constexpr int kDmaUB = 1024;                        // U rows of a stage (16 x at most 16 floats)
constexpr int kDmaStageB = kDmaDataB + kDmaUB;
constexpr int kDmaWaveB = kDmaBuf * kDmaStageB;     // 20 KB per wave

__device__ v4u g_patch_sink[64];

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Direct global -> LDS load from a per-lane 64-bit address: 16 bytes of lane
// l land at LDS address lds + 16 l (lds wave-uniform, carried in M0).
__device__ __forceinline__ void dma16_va(const char* p, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(p), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

typedef __attribute__((address_space(3))) v4u lds_v4u_t;
typedef __attribute__((address_space(3))) v4f lds_v4f_t;

template <bool INPLACE>
__global__ __launch_bounds__(kThreads) void patch_dma_kernel(const PatchArgs A) {
    __shared__ __attribute__((aligned(1024))) char smem[(kThreads / 64) * kDmaWaveB];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bid = xcd_contiguous(blockIdx.x, gridDim.x);
    const Pool& P = A.pool;

    int it = 0;
    {
        int hi = A.n_items - 1;
        while (it < hi) {
            const int mid = (it + hi + 1) >> 1;
            if (bid >= A.items[mid].wg_off) it = mid; else hi = mid - 1;
        }
    }
    const PatchItem& I = A.items[it];
    const int local = bid - I.wg_off;
    const int layer = local / A.n_units, unit = local - layer * A.n_units;
    const bool rope = unit < A.n_rope_units;
    const int uo = rope ? unit : unit - A.n_rope_units;
    const char* dst_base = rope ? P.rp + (int64_t)layer * P.rp_l : P.pf + (int64_t)layer * P.pf_l;
    const int64_t dst_b = rope ? P.rp_b : P.pf_b, dst_r = rope ? P.rp_r : P.pf_r;
    const int unit_off = uo * 256;
    const char* src_base = INPLACE ? nullptr
                                   : (rope ? I.src_rp + (int64_t)layer * I.src_rp_l : I.src_pf + (int64_t)layer * I.src_pf_l);
    const int64_t src_r = rope ? I.src_rp_r : I.src_pf_r;
    const int rank = rope ? I.rank_rp : I.rank_pf;
    const float* U = rank ? (rope ? I.U_rp + (int64_t)layer * I.u_rp_l : I.U_pf + (int64_t)layer * I.u_pf_l) : nullptr;
    const float* V = rank ? (rope ? I.V_rp + (int64_t)layer * I.v_rp_l : I.V_pf + (int64_t)layer * I.v_pf_l) : nullptr;
    const bool rotate = rope && !INPLACE && I.shift != 0;
    const int len = I.len;
    const int n_sub = (len + kDmaRows - 1) / kDmaRows;
    const int n_st = n_sub > wave ? (n_sub - wave + 3) / 4 : 0;       // this wave's stages
    const int bs = P.bs_shift;
    const int bmask = P.block_size - 1;
    const int tok = lane & 15, g = lane >> 4;

    // feature-side factor rows of the unit's 4 groups (A operands)
    v4f fa[4], fb[4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
        fa[gi] = v4f{0, 0, 0, 0};
        fb[gi] = fa[gi];
        if (4 * g < rank) {
            const int fr = uo * 128 + gi * 32 + 8 * (tok >> 2) + (tok & 3);
            fa[gi] = *reinterpret_cast<const v4f*>(V + (int64_t)fr * rank + 4 * g);
            fb[gi] = *reinterpret_cast<const v4f*>(V + (int64_t)(fr + 4) * rank + 4 * g);
        }
    }
    // block ids of this wave's stages: lane k holds those of stage k (first
    // and last row of the sub-tile; -1 for a bad id)
    int id0 = -1, id1 = -1;
    if (lane < n_st) {
        const int r0 = kDmaRows * (wave + 4 * lane);
        const int s0 = I.dst0 + r0, s1 = I.dst0 + min(r0 + kDmaRows, len) - 1;
        id0 = A.bt[s0 >> bs];
        id1 = A.bt[s1 >> bs];
        if ((unsigned)id0 >= (unsigned)P.n_blocks) { raise_error(KVR_DEV_BAD_BLOCK); id0 = -1; }
        if ((unsigned)id1 >= (unsigned)P.n_blocks) { raise_error(KVR_DEV_BAD_BLOCK); id1 = -1; }
    }
    // (cos, sin) of this lane's pairs j = 32 gl + 8 g + e (gl < 2, e < 8)
    float2 cs[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) cs[k] = make_float2(1.f, 0.f);
    if (rotate) {
        double om[16];                               // all loads first, then the angles
#pragma unroll
        for (int k = 0; k < 16; ++k) om[k] = A.omega[32 * (k >> 3) + 8 * g + (k & 7)];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const double u = (double)I.shift * om[k];
            const double f = u - rint(u);
            float s, c;
            sincosf((float)(f * 6.283185307179586476925), &s, &c);
            cs[k] = make_float2(c, s);
        }
    }
    // every load so far has landed (the compiler accounts for this wait, so
    // it adds none later that would drain the direct loads)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (n_st == 0) return;

    const uint32_t lds_w = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem + wave * kDmaWaveB;
    const char* sink = reinterpret_cast<const char*>(&g_patch_sink[lane]);

    // physical row of item row `row` of stage k (whose ids are i0 / i1), or
    // nullptr when the row's block id is bad
    auto row_addr = [&](int k, int row, int i0, int i1) __attribute__((always_inline)) -> const char* {
        const int slot = I.dst0 + row;
        const int first = (I.dst0 + kDmaRows * (wave + 4 * k)) >> bs;
        const int id = (slot >> bs) == first ? i0 : i1;
        return id < 0 ? nullptr : dst_base + (int64_t)id * dst_b + (int64_t)(slot & bmask) * dst_r + unit_off;
    };
    // direct loads of stage kk: 4 x (4 rows x 256 B) of data, then 16 U rows
    auto issue = [&](int kk) __attribute__((always_inline)) {
        const int k = min(kk, n_st - 1);
        const int r0 = kDmaRows * (wave + 4 * k);
        const uint32_t buf = lds_w + (uint32_t)(kk % kDmaBuf) * kDmaStageB;
        const int i0 = __builtin_amdgcn_readlane(id0, k), i1 = __builtin_amdgcn_readlane(id1, k);
        const char* first_addr = nullptr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * i + (lane >> 4);
            const int row = min(r0 + r, len - 1);
            const uint32_t c = (uint32_t)(lane & 15) ^ (uint32_t)r;
            const char* a;
            if (INPLACE) {
                const char* ra = row_addr(k, row, i0, i1);
                a = (ra ? ra : dst_base + unit_off) + 16 * c;      // bad block: any in-range row
            } else {
                a = src_base + (int64_t)row * src_r + unit_off + 16 * c;
            }
            if (i == 0) first_addr = a;
            dma16_va(a, buf + 1024 * i);
        }
        const char* ua = first_addr;
        if (rank) {
            const int64_t left = (int64_t)(len - r0) * rank * 4 - 16;   // last 16 bytes of the item's U
            ua = reinterpret_cast<const char*>(U + (int64_t)r0 * rank) + min<int64_t>(16 * lane, left);
        }
        dma16_va(ua, buf + kDmaDataB);
    };

    for (int kk = 0; kk < 3; ++kk) issue(kk);
    wait_vm<10>();                                   // stage 0 landed
    for (int k = 0; k < n_st; ++k) {
        const uint32_t buf = lds_w + (uint32_t)(k % kDmaBuf) * kDmaStageB;
        const int r0 = kDmaRows * (wave + 4 * k);
        const int i0 = __builtin_amdgcn_readlane(id0, k), i1 = __builtin_amdgcn_readlane(id1, k);
        v4f u = v4f{0, 0, 0, 0};
        if (4 * g < rank) u = *(const lds_v4f_t*)(size_t)(buf + kDmaDataB + 4 * (tok * rank + 4 * g));
        v4u x[4];
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
            x[gi] = *(const lds_v4u_t*)(size_t)(buf + tok * 256 + 16 * ((uint32_t)(4 * gi + g) ^ (uint32_t)tok));
        v4f pa[4], pb[4];
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            pa[gi] = v4f{0, 0, 0, 0};
            pb[gi] = pa[gi];
            if (rank) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    pa[gi] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[gi][kk], u[kk], pa[gi], 0, 0, 0);
                    pb[gi] = __builtin_amdgcn_mfma_f32_16x16x4f32(fb[gi][kk], u[kk], pb[gi], 0, 0, 0);
                }
            }
        }
        if (rope) {
#pragma unroll
            for (int gl = 0; gl < 2; ++gl)
                rot_patch(x[gl], x[gl + 2], cs + 8 * gl, rotate, rank > 0, pa[gl], pb[gl], pa[gl + 2], pb[gl + 2]);
        } else if (rank) {
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) x[gi] = add_patch(x[gi], pa[gi], pb[gi]);
        }
        // Results go back to their own LDS slots and leave row-major: store i
        // writes rows 4i..4i+3, 256 contiguous bytes each (whole 128-byte
        // lines), lane l taking chunk position l % 16 of row 4i + l / 16.
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
            *(lds_v4u_t*)(size_t)(buf + tok * 256 + 16 * ((uint32_t)(4 * gi + g) ^ (uint32_t)tok)) = x[gi];
        // other lanes' results are read next: order the reads after the writes
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * i + (lane >> 4);
            const uint32_t p = (uint32_t)(lane & 15);
            const v4u y = *(const lds_v4u_t*)(size_t)(buf + r * 256 + 16 * p);
            const char* ra = r0 + r < len ? row_addr(k, r0 + r, i0, i1) : nullptr;
            st16(const_cast<char*>(ra ? ra + 16 * (p ^ (uint32_t)r) : sink), y);
        }
        issue(k + 3);
        if (k == 0) wait_vm<14>();                   // stage k + 1 landed
        else        wait_vm<18>();
    }
    wait_vm<0>();                                    // no load may land in LDS after this
}

}  // namespace

hipError_t launch_patch(const PatchArgs& a, bool inplace, hipStream_t s) {
    if (a.dma) {
        if (inplace) hipLaunchKernelGGL(patch_dma_kernel<true>, dim3(a.n_wg), dim3(kThreads), 0, s, a);
        else         hipLaunchKernelGGL(patch_dma_kernel<false>, dim3(a.n_wg), dim3(kThreads), 0, s, a);
    } else {
        if (inplace) hipLaunchKernelGGL(patch_kernel<true>, dim3(a.n_wg), dim3(kThreads), 0, s, a);
        else         hipLaunchKernelGGL(patch_kernel<false>, dim3(a.n_wg), dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

uint32_t read_and_clear_errors_patch() {
    uint32_t v = 0, z = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_errors_patch), sizeof(v)) != hipSuccess) return 0xffffffffu;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_errors_patch), &z, sizeof(z)) != hipSuccess) return 0xffffffffu;
    return v;
}

}  // namespace kvr
