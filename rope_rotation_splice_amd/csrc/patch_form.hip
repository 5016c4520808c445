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
// rounding.  Omega is drawn by the caller.
//
// Kernels:
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
//   the matrix cores, Cholesky and the triangular inverse in the registers
//   of one wave (a row per lane, other rows' entries broadcast by readlane),
//   the update Z L^-T on the matrix cores; the first pass adds the shift
//   11 (n k + k (k + 1)) u ||Z||_F^2 to the Gram diagonal, which keeps the
//   Cholesky factorization defined for any conditioning, and columns whose
//   pivot falls to 1e-8 of the largest are dropped (a deficit of rank below
//   32 gives a sketch of lower rank: the basis then has zero columns).
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

__global__ __launch_bounds__(256) void orth_kernel(const FormOrthArgs A) {
    __shared__ float sG[32][33];
    __shared__ __attribute__((aligned(16))) float sLi[32][36];
    const int tid = threadIdx.x, lane = tid & 63;
    float* Z = A.Z + (int64_t)blockIdx.x * A.n * kSk;
    for (int pass = 0; pass < 3; ++pass) {
        gram32(Z, A.n, sG, tid);
        __syncthreads();
        if (tid < 64) {
            // One wave factors the 32 x 32 Gram matrix in registers: lane i
            // (< 32) holds row i in g[], and the values a step needs from
            // other rows are broadcast with readlane (lanes 32..63 mirror
            // lanes 0..31 and store nothing).
            const int ri = lane & 31;
            float g[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) g[k] = sG[ri][k];
            if (pass == 0) {
                // shift 11 (n k + k (k + 1)) u tr(G), u = 2^-24, k = 32
                float tr = 0.f;
#pragma unroll
                for (int k = 0; k < 32; ++k) tr += rl(g[k], k);
                const float sh = 11.f * (float)(A.n * 32 + 32 * 33) * 5.9604645e-8f * tr;
#pragma unroll
                for (int k = 0; k < 32; ++k)
                    if (k == ri) g[k] += sh;
            }
            // Cholesky G = L L^T, right-looking, lower triangle.  A pivot --
            // the squared norm of column j orthogonal to the earlier columns
            // -- at or below 1e-8 of the largest diagonal entry marks column
            // j as dependent: it is dropped (its row of L^-1 is zero, so Z's
            // column j becomes 0).
            float dmax = 0.f;
#pragma unroll
            for (int k = 0; k < 32; ++k) dmax = fmaxf(dmax, rl(g[k], k));
            const float tau = 1e-8f * dmax;
            uint32_t dead = 0;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const float piv = rl(g[j], j);
                if (piv <= tau) {
                    dead |= 1u << j;
                    g[j] = ri == j ? 1.f : (ri > j ? 0.f : g[j]);
                    continue;
                }
                const float dj = sqrtf(piv);
                const float lij = g[j] / dj;
                g[j] = ri == j ? dj : (ri > j ? lij : g[j]);
#pragma unroll
                for (int k = j + 1; k < 32; ++k) {
                    const float lkj = rl(g[j], k);          // L[k][j]
                    if (ri >= k) g[k] -= lij * lkj;
                }
            }
            // L^-1 by forward substitution, lane c builds column c; rows of
            // dropped columns are zero
            float x[32];
#pragma unroll
            for (int r = 0; r < 32; ++r) {
                float s = r == ri ? 1.f : 0.f;
#pragma unroll
                for (int k = 0; k < r; ++k) s -= rl(g[k], r) * x[k];      // L[r][k]
                x[r] = (r < ri || ((dead >> r) & 1u)) ? 0.f : s / rl(g[r], r);
            }
            if (lane < 32) {
#pragma unroll
                for (int r = 0; r < 32; ++r) sLi[r][lane] = x[r];
            }
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
