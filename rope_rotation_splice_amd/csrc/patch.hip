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

// Workgroups reach the 8 XCDs round-robin (workgroup b runs on XCD b % 8,
// each with its own L2).  Every tile of an (item, layer) re-reads that
// layer's feature-side factors, so each XCD is given a contiguous range of
// logical workgroups: the tiles of one (item, layer) then share one L2.
__device__ __forceinline__ int xcd_contiguous(int b, int n) {
    const int x = b & 7, k = b >> 3, q = n >> 3, r = n & 7;
    return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

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

}  // namespace

hipError_t launch_patch(const PatchArgs& a, bool inplace, hipStream_t s) {
    if (inplace) hipLaunchKernelGGL(patch_kernel<true>, dim3(a.n_wg), dim3(kThreads), 0, s, a);
    else         hipLaunchKernelGGL(patch_kernel<false>, dim3(a.n_wg), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

uint32_t read_and_clear_errors_patch() {
    uint32_t v = 0, z = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_errors_patch), sizeof(v)) != hipSuccess) return 0xffffffffu;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_errors_patch), &z, sizeof(z)) != hipSuccess) return 0xffffffffu;
    return v;
}

}  // namespace kvr
