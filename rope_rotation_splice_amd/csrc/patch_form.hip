// Kamera patch formation (section 2: the m leading factors of the deficit
// Delta = KV(B|A) - KV(B|empty) from an SVD; section 3: one orbit patch,
// formed from the deficit averaged over the sampled orders, serves every
// order of a cached set).
//
// Randomized range finder with two power steps on Delta^T Delta (a
// 32-column sketch Omega, m <= 16):
//   Y = Delta Omega
//   twice:  Z = Delta^T Y,  V = orth(Z),  Y = Delta V
//   Y^T Y = W Lambda W^T (Jacobi),  order by decreasing eigenvalue
//   V_m = V W_m,  U_m Sigma_m = Y W_m,  sigma = sqrt(Lambda_m)
// so that U V^T is the best rank-m approximation of Delta up to the
// sketch's error ((sigma_33 / sigma_m)^5 per power step pair) and float32
// rounding.  Omega is drawn by the caller.  For deficits of 256, 512, 768 or
// 1024 columns each power step Z = Delta^T (Delta X) is one pass over Delta
// (power_kernel, X = Omega and then the orthonormalized Z): three passes
// over every deficit instead of five.
//
// Kernels:
// * power_kernel<NCT>: Z = Delta^T (Delta X), cols = 256 NCT, Y never leaves
//   the chip.  One workgroup of 8 waves per deficit; wave w owns the column
//   slice c0 = 32 NCT w .. + 32 NCT - 1: its rows of X (B operand of the Y
//   step) and of Z (accumulators) stay in registers for the whole deficit.
//   Delta is walked in stages of 16 rows (all columns), global -> LDS
//   directly, one stage ahead.  Per stage: each wave multiplies its
//   16 x 32 NCT slice by its X rows (v_mfma_f32_16x16x4f32) into a partial
//   Y; the 8 partials are summed through LDS; then Z[slice] += slice^T Y on
//   v_mfma_f32_32x32x16_bf16 with both operands split exactly into three
//   bf16 parts (six of the nine part products: float32 accuracy).  Stage
//   rows are laid out in LDS with chunk c of row r at (c & ~15) |
//   ((c & 15) ^ swz(r)), swz(r) = (r & 15) ^ 8 (r & 1): the row reads of the
//   Y step and the column reads of the Z step touch every bank once.
// * sketch_gemm_kernel<TRANS>: Y = Delta X (or Delta^T X) for every
//   deficit, X with 32 columns.  One workgroup per (deficit, 64 output
//   rows); K is walked in stages of 64 rows whose Delta block (16 KB) and X
//   block (8 KB) go global -> LDS directly, kNs - 1 stages ahead, with one
//   barrier per stage.  v_mfma_f32_16x16x4f32, wave w on output rows
//   16 w .. 16 w + 15.  LDS layouts (16-byte chunks permuted so that every
//   operand read touches each bank once):
//     Delta, Y = Delta X: row m (256 bytes), chunk c at c ^ (m mod 16); lane
//       (i, q) reads a float4 covering K = 16 kb + 4 q .. + 3.
//     Delta, Z = Delta^T Y: K row t (256 bytes), chunk c at c ^ 4 (t mod 4);
//       lane (i, q) reads one float at K = 4 ks + q.
//     X: K row k (128 bytes) in slot row k ^ ((k >> 2) & 1) with chunk c at
//       c ^ 4 ((k >> 3) & 1) (Y = Delta X), or in row k with chunk c at
//       c ^ 4 ((k >> 1) & 1) (Z = Delta^T Y).
//   The direct loads come from inline assembly with exact vmcnt waits, and
//   the loop holds no other memory access the compiler would wait on.
// * orth_kernel: shifted CholeskyQR3 of Z (cols x 32) in place -- Gram on
//   the matrix cores (float64 in the second pass), Cholesky and the
//   triangular inverse in float64 in the registers of one wave (a row per
//   lane, other rows' entries broadcast by readlane), the update Z L^-T on
//   the float32 matrix cores;
//   the first pass adds the shift 11 (n k + k (k + 1)) u ||Z||_F^2 to the
//   Gram diagonal, and columns whose pivot falls to u^2 of the largest are
//   dropped (a deficit of rank below 32 gives a sketch of lower rank: the
//   basis then has zero columns).  A sketch that meets the test matrix
//   badly is ill-conditioned (condition ~1e5 and more): after the shifted
//   pass its weakest genuine direction leaves a pivot below float32
//   rounding (~1e-8 of the largest), which a float32 factorization could
//   turn negative and drop for good; in float64 it is kept.
// * eig_kernel: Gram of Y, cyclic Jacobi (tournament ordering: 16 disjoint
//   rotations per round, 31 rounds per sweep; each thread applies a round to
//   one 2 x 2 block of the Gram matrix and to two entry pairs of W;
//   negligible rotations are skipped and the sweeps stop once a whole sweep
//   skips them all), eigenvalues ordered, then the factors V W_m and Y W_m
//   on the matrix cores, and sigma.
// * mean_kernel: the orbit deficit, the mean of each matrix's orders.
#include "kvr_device.h"
#include "kvr_internal.h"
#include "kvr_lds.h"

#include "../../include/kvreloc.h"

namespace kvr {

namespace {

constexpr int kSk = kFormSketch;     // sketch columns
constexpr int kTm = 64;              // output rows per workgroup
constexpr int kTk = 64;              // K rows per stage
constexpr int kNs = 3;               // stage buffers (loads run kNs - 1 stages ahead)
constexpr int kDeltaB = kTm * kTk * 4;                // Delta block of a stage
constexpr int kStageB = kDeltaB + kTk * kSk * 4;      // + X block
constexpr int kSweeps = 8;

// value of v in lane l (l uniform)
__device__ __forceinline__ float rl(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <bool TRANS>
__global__ __launch_bounds__(256) void sketch_gemm_kernel(const FormGemmArgs A) {
    __shared__ __attribute__((aligned(1024))) char smem[kNs * kStageB];
    const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;
    const int M = TRANS ? A.cols : A.rows, K = TRANS ? A.rows : A.cols;
    const int tiles = M / kTm;
    const int bid = xcd_contiguous(blockIdx.x, gridDim.x);
    const int b = bid / tiles, m0 = (bid - b * tiles) * kTm;
    const char* D = reinterpret_cast<const char*>(A.D + (int64_t)b * A.d_stride);
    const char* X = reinterpret_cast<const char*>(A.X + (int64_t)b * A.x_stride);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 15, q = lane >> 4;
    const int nk = K / kTk;

    // Direct loads of stage s (K rows k0 = 64 s .. k0 + 63) into buffer s % kNs:
    // 16 KB of Delta (16 loads of 1 KB) and 8 KB of X (8 loads); wave w
    // issues Delta loads w, w + 4, w + 8, w + 12 and X loads w, w + 4.
    // Stages past the end reload the last one into a buffer nobody reads
    // again, so every stage issues the same loads.
    auto issue = [&](int s) __attribute__((always_inline)) {
        const int k0 = kTk * min(s, nk - 1);
        const uint32_t buf = lds0 + (uint32_t)(s % kNs) * kStageB;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int u = w + 4 * v;
            const int r = 4 * u + (lane >> 4), p = lane & 15;
            if (!TRANS) {
                // row m0 + r, 16-byte chunk c of its 64 K-floats
                const uint32_t c = (uint32_t)(p ^ (r & 15));
                dma16(D + ((int64_t)m0 * A.cols + k0) * 4, (uint32_t)(r * A.cols) * 4u + 16u * c, buf + 1024u * u);
            } else {
                // K row k0 + r, 16-byte chunk c of its 64 M-floats
                const uint32_t c = (uint32_t)(p ^ (4 * (r & 3)));
                dma16(D + ((int64_t)k0 * A.cols + m0) * 4, (uint32_t)(r * A.cols) * 4u + 16u * c, buf + 1024u * u);
            }
        }
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int u = w + 4 * v;
            const int ks = 8 * u + (lane >> 3), cs = lane & 7;       // LDS slot (row, chunk)
            const int k = TRANS ? ks : ks ^ ((ks >> 2) & 1);
            const int c = TRANS ? cs ^ (4 * ((ks >> 1) & 1)) : cs ^ (4 * ((k >> 3) & 1));
            dma16(X + (int64_t)k0 * (kSk * 4), (uint32_t)(k * kSk + 4 * c) * 4u, buf + kDeltaB + 1024u * u);
        }
    };
    // LDS byte offsets of the operands (see the layouts above)
    auto x_at = [&](uint32_t buf, int k, int n) __attribute__((always_inline)) -> uint32_t {
        const int c = n >> 2;
        const uint32_t slot = TRANS ? (uint32_t)(8 * k + (c ^ (4 * ((k >> 1) & 1))))
                                    : (uint32_t)(8 * (k ^ ((k >> 2) & 1)) + (c ^ (4 * ((k >> 3) & 1))));
        return buf + kDeltaB + 16u * slot + 4u * (n & 3);
    };

    v4f acc0 = {0, 0, 0, 0}, acc1 = acc0;
#pragma unroll
    for (int s = 0; s < kNs - 1; ++s) issue(s);
    for (int j = 0; j < nk; ++j) {
        wait_vmcnt<6 * (kNs - 2)>();        // stage j landed (this wave's part)
        __syncthreads();                     // every wave's part; stage j - 1 consumed
        issue(j + kNs - 1);
        const uint32_t buf = lds0 + (uint32_t)(j % kNs) * kStageB;
        // the stage's operands are read into registers first, then the 32
        // MFMAs run back to back
        typedef const __attribute__((address_space(3))) float* lds_f;
        typedef const __attribute__((address_space(3))) v4f* lds_f4;
        float av[16], b0[16], b1[16];
        if (!TRANS) {
            // lane (i, q) supplies K index 16 kb + 4 q + kk: a float4 of row 16 w + i
            const uint32_t arow = buf + (uint32_t)(16 * w + i) * 256u;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const v4f v = *(lds_f4)(size_t)(arow + 16u * (uint32_t)((4 * kb + q) ^ i));
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int k = 16 * kb + 4 * q + kk;
                    av[4 * kb + kk] = v[kk];
                    b0[4 * kb + kk] = *(lds_f)(size_t)x_at(buf, k, i);
                    b1[4 * kb + kk] = *(lds_f)(size_t)x_at(buf, k, 16 + i);
                }
            }
        } else {
            // lane (i, q) supplies K index 4 ks + q: Delta[k0 + t][m0 + 16 w + i]
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
                const int t = 4 * ks + q;
                const uint32_t ca = (uint32_t)((4 * w + (i >> 2)) ^ (4 * (t & 3)));
                av[ks] = *(lds_f)(size_t)(buf + (uint32_t)t * 256u + 16u * ca + 4u * (i & 3));
                b0[ks] = *(lds_f)(size_t)x_at(buf, t, i);
                b1[ks] = *(lds_f)(size_t)x_at(buf, t, 16 + i);
            }
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            acc0 = mfma4(av[u], b0[u], acc0);
            acc1 = mfma4(av[u], b1[u], acc1);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, TRANS ? 48 : 36, 0);    // every LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);                 // then the MFMAs
    }
    wait_vmcnt<0>();                         // no direct load may land after the workgroup ends
    // output row 4 q + r of this wave's 16, column i (+ 16)
    float* Y = A.Y + (int64_t)b * A.y_stride + (int64_t)(m0 + 16 * w + 4 * q) * kSk + i;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        Y[r * kSk] = acc0[r];
        Y[r * kSk + 16] = acc1[r];
    }
}

// One power step Z = Delta^T (Delta X) in a single pass over Delta
// (power_kernel in the header).
constexpr int kPwWaves = 8;
constexpr int kPwRows = 16;                                   // Delta rows per stage
constexpr int kPwStageB = kPwRows * kFormPowerMaxCols * 4;    // 64 KB
constexpr int kPwEPitch = 36;                                 // floats per row of a partial Y
constexpr int kPwEOff = 2 * kPwStageB;
constexpr int kPwFOff = kPwEOff + kPwWaves * kPwRows * kPwEPitch * 4;
constexpr int kPwFPitch = 20;                                // floats per column of Y (rows 0..15 used)
constexpr int kPwSmem = kPwFOff + kSk * kPwFPitch * 4;
static_assert(kPwSmem <= 160 * 1024, "LDS budget");

// chunk permutation of stage row r (a bijection of 0..15)
__device__ __forceinline__ uint32_t pw_swz(int r) { return (uint32_t)((r & 15) ^ ((r & 1) << 3)); }
__device__ __forceinline__ uint32_t pw_pos(int c, int r) { return (uint32_t)(c & ~15) | (((uint32_t)c & 15u) ^ pw_swz(r)); }

typedef float v16f __attribute__((ext_vector_type(16)));

// The high halves of two floats as one pair of bf16 (a in the low half).
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// x = h + m + l exactly, each part a bf16: h keeps x's leading 8
// significant bits (truncated), m the leading 8 of the remainder and l the
// at most 8 bits left.  A product x y then equals the sum of the nine part
// products; the six kept (hh, hm, mh, hl, lh, mm) leave out terms below
// 2^-23 |x y|.
__device__ __forceinline__ void split3(const float (&x)[8], v8bf& h, v8bf& m, v8bf& l) {
    v4u H, M, L;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t xa = __float_as_uint(x[2 * p]), xb = __float_as_uint(x[2 * p + 1]);
        const float ra = x[2 * p] - __uint_as_float(xa & 0xffff0000u);
        const float rb = x[2 * p + 1] - __uint_as_float(xb & 0xffff0000u);
        const uint32_t ma = __float_as_uint(ra), mb = __float_as_uint(rb);
        const float la = ra - __uint_as_float(ma & 0xffff0000u);
        const float lb = rb - __uint_as_float(mb & 0xffff0000u);
        H[p] = hi_pair(xa, xb);
        M[p] = hi_pair(ma, mb);
        L[p] = hi_pair(__float_as_uint(la), __float_as_uint(lb));
    }
    h = as_bf(H);
    m = as_bf(M);
    l = as_bf(L);
}

template <int NCT>
__global__ __launch_bounds__(kPwWaves * 64) void power_kernel(const FormGemmArgs A) {
    __shared__ __attribute__((aligned(1024))) char smem[kPwSmem];
    const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;
    constexpr int kCols = 256 * NCT, kChunks = kCols / 4;        // 16-byte chunks per row
    constexpr uint32_t kRowB = 4u * kCols;
    typedef const __attribute__((address_space(3))) float* lds_f;
    typedef const __attribute__((address_space(3))) v4f* lds_f4;
    typedef __attribute__((address_space(3))) float* lds_fw;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 15, q = lane >> 4;          // 16 x 16 x 4 operand coordinates
    const int n32 = lane & 31, h = lane >> 5;        // 32 x 32 x 2 operand coordinates
    const int b = blockIdx.x;
    const char* D = reinterpret_cast<const char*>(A.D + (int64_t)b * A.d_stride);
    const float* X = A.X + (int64_t)b * A.x_stride;
    const int c0 = 32 * NCT * w;
    const int nst = A.rows / kPwRows;

    // X rows of the slice, B operand of the Y step: lane (i, q) supplies
    // K index c0 + 16 kb + 4 q + kk of columns i and 16 + i
    float xb[2][2 * NCT][4];
#pragma unroll
    for (int kb = 0; kb < 2 * NCT; ++kb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const float* xr = X + (int64_t)(c0 + 16 * kb + 4 * q + kk) * kSk;
            xb[0][kb][kk] = xr[i];
            xb[1][kb][kk] = xr[16 + i];
        }
    // every load so far has landed (a wait the compiler also accounts for,
    // so it adds none later that would drain the direct loads)
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // Direct loads of stage s: the stage (16 rows, all columns) is 4 KB x
    // NCT per row; wave w's load u fills LDS slots 64 (8 u + w) .. + 63, slot
    // g holding chunk pw_pos(g % kChunks, r) of row r = g / kChunks.
    auto issue = [&](int s) __attribute__((always_inline)) {
        const uint32_t buf = lds0 + (uint32_t)(s & 1) * kPwStageB;
        const char* base = D + (int64_t)s * kPwRows * kRowB;
#pragma unroll
        for (int u = 0; u < 2 * NCT; ++u) {
            const int g = 64 * (8 * u + w) + lane;
            const int r = g / kChunks, p = g - r * kChunks;
            dma16(base, (uint32_t)r * kRowB + 16u * pw_pos(p, r), buf + 1024u * (uint32_t)(8 * u + w));
        }
    };

    v16f zacc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) zacc[ct] = v16f{};
    lds_fw E = (lds_fw)(size_t)(lds0 + kPwEOff);
    lds_fw F = (lds_fw)(size_t)(lds0 + kPwFOff);

    issue(0);
    for (int s = 0; s < nst; ++s) {
        wait_vmcnt<0>();                 // this wave's part of stage s landed
        __syncthreads();                 // every wave's part; stage s - 1's buffer is free
        if (s + 1 < nst) issue(s + 1);
        const uint32_t buf = lds0 + (uint32_t)(s & 1) * kPwStageB;

        // Y step: partial Y (16 x 32) of this slice; lane (i, q) reads a float4
        // of row i covering K indices c0 + 16 kb + 4 q .. + 3
        v4f y0 = {0, 0, 0, 0}, y1 = y0;
        {
            v4f av[2 * NCT];
            const uint32_t arow = buf + (uint32_t)i * kRowB;
#pragma unroll
            for (int kb = 0; kb < 2 * NCT; ++kb)
                av[kb] = *(lds_f4)(size_t)(arow + 16u * pw_pos(c0 / 4 + 4 * kb + q, i));
#pragma unroll
            for (int kb = 0; kb < 2 * NCT; ++kb)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    y0 = mfma4(av[kb][kk], xb[0][kb][kk], y0);
                    y1 = mfma4(av[kb][kk], xb[1][kb][kk], y1);
                }
        }
        // rows 4 q + r, columns i and 16 + i of this wave's partial
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            E[(w * kPwRows + 4 * q + r) * kPwEPitch + i] = y0[r];
            E[(w * kPwRows + 4 * q + r) * kPwEPitch + 16 + i] = y1[r];
        }
        __syncthreads();
        // Y = the sum of the 8 partials; thread (w, lane) forms row w + 8 h, column n32
        {
            const int rr = w + 8 * h;
            float acc = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < kPwWaves; ++w2) acc += E[(w2 * kPwRows + rr) * kPwEPitch + n32];
            F[n32 * kPwFPitch + rr] = acc;
        }
        __syncthreads();

        // Z step: Z[slice] += slice^T Y, K = the 16 rows, on
        // v_mfma_f32_32x32x16_bf16 with both operands split in three (six
        // products per tile).  Lane (n32, h) supplies rows 8 h .. 8 h + 7 of
        // column c0 + 32 ct + n32 (A) and of Y's column n32 (B).
        v8bf bh, bm, bl;
        {
            const v4f y0v = *(lds_f4)(size_t)(lds0 + kPwFOff + 4u * (uint32_t)(n32 * kPwFPitch + 8 * h));
            const v4f y1v = *(lds_f4)(size_t)(lds0 + kPwFOff + 4u * (uint32_t)(n32 * kPwFPitch + 8 * h + 4));
            const float yv[8] = {y0v[0], y0v[1], y0v[2], y0v[3], y1v[0], y1v[1], y1v[2], y1v[3]};
            split3(yv, bh, bm, bl);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            float a[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int r = 8 * h + t;
                a[t] = *(lds_f)(size_t)(buf + (uint32_t)r * kRowB +
                                        16u * pw_pos(c0 / 4 + 8 * ct + (n32 >> 2), r) + 4u * (uint32_t)(n32 & 3));
            }
            v8bf ah, am, al;
            split3(a, ah, am, al);
            v16f z = zacc[ct];
            z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, z, 0, 0, 0);
            z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, z, 0, 0, 0);
            z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bm, z, 0, 0, 0);
            z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bh, z, 0, 0, 0);
            z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bm, z, 0, 0, 0);
            zacc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, z, 0, 0, 0);
        }
    }
    wait_vmcnt<0>();                     // no direct load may land after the workgroup ends

    // Z rows c0 + 32 ct + 8 (e / 4) + 4 h + e % 4, column n32
    float* Z = A.Y + (int64_t)b * A.y_stride;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            Z[(int64_t)(c0 + 32 * ct + 8 * (e >> 2) + 4 * h + (e & 3)) * kSk + n32] = zacc[ct][e];
}

// Gram G = Z^T Z of a [n x 32] matrix (n a multiple of 64) into sG
// (32 x 33): wave w computes the 16 x 16 tile (w / 2, w % 2); the loads of
// 64 rows are in flight together.
__device__ __forceinline__ void gram32(const float* Z, int n, float (*sG)[33], int tid) {
    const int lane = tid & 63, w = tid >> 6, i = lane & 15, q = lane >> 4;
    const int ma = 16 * (w >> 1) + i, nb = 16 * (w & 1) + i;
    v4f acc = {0, 0, 0, 0};
    for (int k0 = 0; k0 < n; k0 += 64) {
        float a[16], b[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float* row = Z + (int64_t)(k0 + 16 * (u >> 2) + 4 * q + (u & 3)) * kSk;
            a[u] = row[ma];
            b[u] = row[nb];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) acc = mfma4(a[u], b[u], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sG[16 * (w >> 1) + 4 * q + r][16 * (w & 1) + i] = acc[r];
}

// The same Gram matrix accumulated in float64 (v_mfma_f64_16x16x4f64, the
// products of the float32 entries are exact): its pivots keep their
// meaning far below float32 rounding.  That instruction leaves output rows
// q + 4 r (not 4 q + r) of column i in lane (i, q).
typedef double v4d __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void gram32_f64(const float* Z, int n, double (*sG)[33], int tid) {
    const int lane = tid & 63, w = tid >> 6, i = lane & 15, q = lane >> 4;
    const int ma = 16 * (w >> 1) + i, nb = 16 * (w & 1) + i;
    v4d acc = {0, 0, 0, 0};
    for (int k0 = 0; k0 < n; k0 += 64) {
        float a[16], b[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float* row = Z + (int64_t)(k0 + 16 * (u >> 2) + 4 * q + (u & 3)) * kSk;
            a[u] = row[ma];
            b[u] = row[nb];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a[u], (double)b[u], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sG[16 * (w >> 1) + q + 4 * r][16 * (w & 1) + i] = acc[r];
}

// value of v in lane l (l uniform), float64
__device__ __forceinline__ double rld(double v, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// One wave factors a 32 x 32 Gram matrix in float64 registers and writes
// L^-1 to sLi (float): lane i (< 32) holds row i in g[], and the values a
// step needs from other rows are broadcast with readlane (lanes 32..63
// mirror lanes 0..31 and store nothing).  `shift` adds the first pass's
// diagonal shift.
__device__ __forceinline__ void chol_inverse(double (&g)[32], float (*sLi)[36], int n, bool shift, int lane) {
    const int ri = lane & 31;
    if (shift) {
        // shift 11 (n k + k (k + 1)) u tr(G), u = 2^-24 (Z is float32), k = 32
        double tr = 0;
#pragma unroll
        for (int k = 0; k < 32; ++k) tr += rld(g[k], k);
        const double sh = 11.0 * (double)(n * 32 + 32 * 33) * 0x1p-24 * tr;
#pragma unroll
        for (int k = 0; k < 32; ++k)
            if (k == ri) g[k] += sh;
    }
    // Cholesky G = L L^T, right-looking, lower triangle.  A pivot --
    // the squared norm of column j orthogonal to the earlier columns
    // -- at or below u^2 = 2^-48 of the largest diagonal entry (Z's own
    // float32 rounding) marks column j as dependent: it is dropped
    // (its row of L^-1 is zero, so Z's column j becomes 0).
    double dmax = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k) dmax = fmax(dmax, rld(g[k], k));
    const double tau = 0x1p-48 * dmax;
    uint32_t dead = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const double piv = rld(g[j], j);
        if (piv <= tau) {
            dead |= 1u << j;
            g[j] = ri == j ? 1.0 : (ri > j ? 0.0 : g[j]);
            continue;
        }
        const double dj = sqrt(piv);
        const double lij = g[j] / dj;
        g[j] = ri == j ? dj : (ri > j ? lij : g[j]);
#pragma unroll
        for (int k = j + 1; k < 32; ++k) {
            const double lkj = rld(g[j], k);        // L[k][j]
            if (ri >= k) g[k] -= lij * lkj;
        }
    }
    // L^-1 by forward substitution, lane c builds column c; rows of
    // dropped columns are zero
    double x[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        double s = r == ri ? 1.0 : 0.0;
#pragma unroll
        for (int k = 0; k < r; ++k) s -= rld(g[k], r) * x[k];     // L[r][k]
        x[r] = (r < ri || ((dead >> r) & 1u)) ? 0.0 : s / rld(g[r], r);
    }
    if (lane < 32) {
#pragma unroll
        for (int r = 0; r < 32; ++r) sLi[r][lane] = (float)x[r];
    }
}

__global__ __launch_bounds__(256) void orth_kernel(const FormOrthArgs A) {
    __shared__ float sGf[32][33];
    __shared__ double sGd[32][33];
    __shared__ __attribute__((aligned(16))) float sLi[32][36];
    const int tid = threadIdx.x, lane = tid & 63;
    float* Z = A.Z + (int64_t)blockIdx.x * A.n * kSk;
    for (int pass = 0; pass < 3; ++pass) {
        // The factorization runs in float64.  The second pass's Gram matrix
        // -- of the shifted pass's output, whose weakest genuine directions
        // may sit below float32 rounding -- is accumulated in float64 too;
        // the first (shifted) and last (near-orthonormal) ones in float32.
        if (pass == 1) gram32_f64(Z, A.n, sGd, tid);
        else           gram32(Z, A.n, sGf, tid);
        __syncthreads();
        if (tid < 64) {
            const int ri = lane & 31;
            double g[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) g[k] = pass == 1 ? sGd[ri][k] : (double)sGf[ri][k];
            chol_inverse(g, sLi, A.n, pass == 0, lane);
        }
        __syncthreads();
        // Z <- Z L^-T on the matrix cores: Z'[row][j] = sum_c Z[row][c] Li[j][c].
        // Wave w takes 16-row tiles w, w + 4, ...; lane (i, q) supplies
        // K index c = 16 kb + 4 q + kk.
        {
            const int w = tid >> 6, i = lane & 15, q = lane >> 4;
            float bl[2][2][4];                   // [N tile][kb][kk]: Li[16 nt + i][16 kb + 4 q + kk]
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const v4f v = *reinterpret_cast<const v4f*>(&sLi[16 * nt + i][16 * kb + 4 * q]);
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) bl[nt][kb][kk] = v[kk];
                }
            for (int m0 = 16 * w; m0 < A.n; m0 += 64) {
                const v4f* zr = reinterpret_cast<const v4f*>(Z + (int64_t)(m0 + i) * kSk);
                const v4f a0 = zr[q], a1 = zr[4 + q];
                v4f c0 = {0, 0, 0, 0}, c1 = c0;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    c0 = mfma4(a0[kk], bl[0][0][kk], c0);
                    c1 = mfma4(a0[kk], bl[1][0][kk], c1);
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    c0 = mfma4(a1[kk], bl[0][1][kk], c0);
                    c1 = mfma4(a1[kk], bl[1][1][kk], c1);
                }
                // every lane of the wave has read the tile before it is overwritten
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                __builtin_amdgcn_wave_barrier();
                float* zo = Z + (int64_t)(m0 + 4 * q) * kSk + i;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    zo[r * kSk] = c0[r];
                    zo[r * kSk + 16] = c1[r];
                }
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void eig_kernel(const FormEigArgs A) {
    __shared__ float sG[32][33];
    __shared__ float sW[32][33];
    __shared__ float s_c[16], s_s[16];
    __shared__ int s_p[16], s_q[16];
    __shared__ int s_idx[32];
    __shared__ float s_lam[32];
    const int tid = threadIdx.x, lane = tid & 63;
    const int b = blockIdx.x;
    const float* Y = A.Y + (int64_t)b * A.rows * kSk;
    const float* V = A.V + (int64_t)b * A.cols * kSk;
    gram32(Y, A.rows, sG, tid);
    for (int e = tid; e < 32 * 32; e += 256) sW[e >> 5][e & 31] = (e >> 5) == (e & 31) ? 1.f : 0.f;
    __syncthreads();
    // Cyclic Jacobi, tournament ordering: in round r, position 0 holds index
    // 0 and position i >= 1 index ((i - 1 + r) mod 31) + 1; pair k joins
    // positions k and 31 - k.  The 16 rotations of a round are disjoint.
    // Threads 0..15 form them; then thread t applies G <- J^T G J to the
    // 2 x 2 block (pair t / 16 of rows, pair t % 16 of columns) and W <- W J
    // to two (row, pair) items.  A rotation whose off-diagonal entry is at
    // most 2^-24 sqrt(|app aqq|) is skipped, and the sweeps stop after one in
    // which every rotation was skipped (the matrix is diagonal to working
    // precision).
    for (int sweep = 0; sweep < kSweeps; ++sweep) {
        int rotated = 0;
        for (int r = 0; r < 31; ++r) {
            if (tid < 16) {
                const int p = tid == 0 ? 0 : ((tid - 1 + r) % 31) + 1;
                const int qq = ((30 - tid + r) % 31) + 1;
                const float app = sG[p][p], aqq = sG[qq][qq], apq = sG[p][qq];
                float c = 1.f, s = 0.f;
                if (fabsf(apq) > 0x1p-24f * sqrtf(fabsf(app)) * sqrtf(fabsf(aqq))) {
                    rotated = 1;
                    const float th = (aqq - app) / (2.f * apq);
                    const float t = fabsf(th) > 1e18f ? 0.5f / th
                                                      : copysignf(1.f, th) / (fabsf(th) + sqrtf(th * th + 1.f));
                    c = 1.f / sqrtf(t * t + 1.f);
                    s = t * c;
                }
                s_c[tid] = c;
                s_s[tid] = s;
                s_p[tid] = p;
                s_q[tid] = qq;
            }
            __syncthreads();
            {
                const int kr = tid >> 4, kc = tid & 15;
                const int pr = s_p[kr], qr = s_q[kr], pc = s_p[kc], qc = s_q[kc];
                const float cr = s_c[kr], sr = s_s[kr], cc = s_c[kc], sc = s_s[kc];
                const float g00 = sG[pr][pc], g01 = sG[pr][qc], g10 = sG[qr][pc], g11 = sG[qr][qc];
                const float h00 = cr * g00 - sr * g10, h01 = cr * g01 - sr * g11;
                const float h10 = sr * g00 + cr * g10, h11 = sr * g01 + cr * g11;
                sG[pr][pc] = cc * h00 - sc * h01;
                sG[pr][qc] = sc * h00 + cc * h01;
                sG[qr][pc] = cc * h10 - sc * h11;
                sG[qr][qc] = sc * h10 + cc * h11;
                const int row = tid >> 3;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int k = 2 * (tid & 7) + u;
                    const int pk = s_p[k], qk = s_q[k];
                    const float c = s_c[k], s = s_s[k];
                    const float x = sW[row][pk], y = sW[row][qk];
                    sW[row][pk] = c * x - s * y;
                    sW[row][qk] = s * x + c * y;
                }
            }
            __syncthreads();
        }
        if (!__syncthreads_or(rotated)) break;
    }
    // order by decreasing eigenvalue (ties by index)
    if (tid < 32) {
        const float l = sG[tid][tid];
        int pos = 0;
        for (int j = 0; j < 32; ++j) {
            const float o = sG[j][j];
            pos += (o > l) || (o == l && j < tid);
        }
        s_idx[pos] = tid;
        s_lam[pos] = l;
    }
    __syncthreads();
    const int m = A.rank;
    if (tid < m) A.sigma[(int64_t)b * m + tid] = sqrtf(fmaxf(s_lam[tid], 0.f));
    // V_m = V W_m (cols x m) and U_m Sigma_m = Y W_m (rows x m) on the matrix
    // cores, 16-row tiles spread over the waves: B[k][j] = W[k][idx_j] (zero
    // for j >= m); lane (i, q) supplies K index 16 kb + 4 q + kk
    {
        const int w = tid >> 6, i = lane & 15, q = lane >> 4;
        const int col = i < m ? s_idx[i] : 0;
        float bw[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) bw[kb][kk] = i < m ? sW[16 * kb + 4 * q + kk][col] : 0.f;
        const int tiles_v = A.cols / 16, tiles = tiles_v + A.rows / 16;
        for (int t = w; t < tiles; t += 4) {
            const bool isv = t < tiles_v;
            const int m0 = 16 * (isv ? t : t - tiles_v);
            const v4f* src = reinterpret_cast<const v4f*>((isv ? V : Y) + (int64_t)(m0 + i) * kSk);
            const v4f a0 = src[q], a1 = src[4 + q];
            v4f c = {0, 0, 0, 0};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) c = mfma4(a0[kk], bw[0][kk], c);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) c = mfma4(a1[kk], bw[1][kk], c);
            float* out = isv ? A.Vout + (int64_t)b * A.cols * m : A.Uout + (int64_t)b * A.rows * m;
            if (i < m) {
#pragma unroll
                for (int r = 0; r < 4; ++r) out[(int64_t)(m0 + 4 * q + r) * m + i] = c[r];
            }
        }
    }
}

// Workgroup w takes 1024 float4 of matrix w / chunks; each thread streams
// four of them with every order's loads unrolled ahead of the sums (read
// once: nontemporal).
__global__ __launch_bounds__(256) void mean_kernel(const float* D, int orders, int64_t per4, int chunks, float* out) {
    const int wg = blockIdx.x;
    const int b = wg / chunks, c = wg - b * chunks;
    const float inv = 1.f / (float)orders;
    const v4f* src = reinterpret_cast<const v4f*>(D) + (int64_t)b * orders * per4;
    v4f* dst = reinterpret_cast<v4f*>(out) + (int64_t)b * per4;
    const int64_t u0 = (int64_t)c * 1024 + threadIdx.x;
    v4f s[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t u = u0 + 256 * k;
        s[k] = u < per4 ? __builtin_nontemporal_load(src + u) : v4f{0, 0, 0, 0};
    }
#pragma unroll 3
    for (int p = 1; p < orders; ++p) {
        v4f x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t u = u0 + 256 * k;
            x[k] = u < per4 ? __builtin_nontemporal_load(src + (int64_t)p * per4 + u) : v4f{0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) s[k] += x[k];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t u = u0 + 256 * k;
        if (u < per4) __builtin_nontemporal_store(s[k] * inv, dst + u);
    }
}

}  // namespace

hipError_t launch_form_gemm(const FormGemmArgs& a, bool trans, hipStream_t s) {
    const int M = trans ? a.cols : a.rows;
    const dim3 grid((unsigned)((int64_t)a.n * (M / kTm)));
    if (trans) hipLaunchKernelGGL(sketch_gemm_kernel<true>, grid, dim3(256), 0, s, a);
    else       hipLaunchKernelGGL(sketch_gemm_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_form_power(const FormGemmArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)a.n), block(kPwWaves * 64);
    switch (a.cols) {
        case 256: hipLaunchKernelGGL(power_kernel<1>, grid, block, 0, s, a); break;
        case 512: hipLaunchKernelGGL(power_kernel<2>, grid, block, 0, s, a); break;
        case 768: hipLaunchKernelGGL(power_kernel<3>, grid, block, 0, s, a); break;
        case 1024: hipLaunchKernelGGL(power_kernel<4>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_form_orth(const FormOrthArgs& a, int count, hipStream_t s) {
    hipLaunchKernelGGL(orth_kernel, dim3((unsigned)count), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_form_eig(const FormEigArgs& a, int count, hipStream_t s) {
    hipLaunchKernelGGL(eig_kernel, dim3((unsigned)count), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_form_mean(const float* d, int orders, int64_t per, int64_t n, float* out, hipStream_t s) {
    const int64_t per4 = per / 4;
    const int chunks = (int)((per4 + 1023) / 1024);
    const int64_t batch = std::max<int64_t>(1, ((int64_t)1 << 30) / chunks);     // matrices per launch
    for (int64_t b0 = 0; b0 < n; b0 += batch) {
        const int64_t nb = std::min(batch, n - b0);
        hipLaunchKernelGGL(mean_kernel, dim3((unsigned)(nb * chunks)), dim3(256), 0, s, d + b0 * orders * per, orders,
                           per4, chunks, out + b0 * per);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kvr
