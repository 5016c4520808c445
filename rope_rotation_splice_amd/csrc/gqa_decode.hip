// One decode step of GQA attention over a paged cache whose blocks carry a
// pending rotary shift (Kamera, section 2: in GQA all of K is rotary and is
// re-rotated, V is position-free; Irminsul, sections 2.2 and 4: the shift is
// applied inside attention, on the load path, and never written back).
//
//   s_t = scale * q_h . R(delta_blk(t)) k_{t,g},   g = h / group
//   O_h = sum_t softmax(s)_t v_{t,g},   LSE_h = ln sum_t exp(s_t)
//
// The rotation is moved to the query: q . R(d) k = (R(-d) q) . k, because
// R(d) is orthogonal with transpose R(-d).  A 64-token block has one shift,
// so a group's queries are re-rotated once per block instead of rotating
// every key.  The re-rotated query q' is split into two bf16 terms, hi =
// bf16(q') and lo = bf16(q' - hi), which both go through the matrix core: the
// scores then carry about 16 bits of q' instead of 8.
//
// Work split (flash-decoding): one single-wave workgroup per (sequence,
// split, KV head), KV heads fastest so that neighbouring workgroups read
// neighbouring 256-byte pieces of the same rows.  A split is walked in stages
// of 32 tokens; a stage's K and V rows go global -> LDS directly (16 bytes
// per lane), 3 stages ahead, issued from inline assembly with exact vmcnt
// waits.  One wave needs no barrier: its LDS accesses complete in order, and
// a direct load has landed in LDS once vmcnt has retired it.
//
// Matrix cores (v_mfma_f32_16x16x32_bf16; output lane l holds column l%16,
// rows 4(l/16)..4(l/16)+3):
// * S^T = K q'^T: two 16-token tiles per stage, 4 K-steps of 32 dimensions,
//   each with the hi and the lo query term.  Tile A's row m is token
//   8(m/4) + m%4 of the stage and tile B's row m token 8(m/4) + 4 + m%4, so
//   lane (n, c) ends up holding tokens 8c..8c+7 of query head n: exactly the
//   B operand (P^T) of the next product, with no data movement.
// * O^T += V^T P^T: 8 feature tiles of 16 per stage; V^T is read from the
//   row-major V rows with the LDS transpose read ds_read_b64_tr_b16 (source
//   lane s addresses row K0 + s/4, columns C + 4(s%4); destination lane d of
//   the 16-lane group receives rows K0..K0+3 of column C + d).
// Softmax is online, in base 2 with the scale folded in; O is rescaled only
// when some head's maximum moved (a wave-uniform test).
//
// LDS rows (256 bytes = 16 chunks of 16 bytes; r = row within the stage):
// * K: chunk c at position c ^ kkey(r), kkey(r) = 4(r/8) + r%4, which is
//   one-to-one on each tile's 16 rows, so the row reads of a K-step touch
//   every bank once per 16 lanes.
// * V: chunk c at position c ^ 2 vkey(r), vkey(r) = r%4 + 4((r/8)%2): a
//   transpose read (16 rows x 32 bytes) then falls on each 32-byte bank group
//   twice, the minimum for 512 bytes.
// A direct load writes position p of a row from lane p, so that lane fetches
// the chunk that belongs there.
#include "kvr_device.h"
#include "kvr_internal.h"
#include "kvr_lds.h"

#include "../../include/kvreloc.h"

namespace kvr {

__device__ uint32_t g_errors_gqa_decode;

namespace {

constexpr int kBlk = kDecBlockTokens;                    // tokens per KV block
constexpr int kStage = 32;                              // tokens per stage
constexpr int kNBuf = 4;                                // stage buffers (3 loads ahead)
constexpr int kRowB = kGqaDim * 2;                      // bytes per row and head
constexpr int kStageB = kStage * kRowB;                 // 8 KB of K (or V) per stage
constexpr int kKOff = 0;
constexpr int kVOff = kNBuf * kStageB;
constexpr int kBlkOff = 2 * kNBuf * kStageB;            // block ids of the split
constexpr int kPendOff = kBlkOff + kGqaMaxBlocks * 4;   // pending shifts of the split
constexpr int kOmegaOff = kPendOff + kGqaMaxBlocks * 4; // theta_j / 2 pi, float64
constexpr int kCsOff = kOmegaOff + (kGqaDim / 2) * 8;   // (cos, sin) of the current block
constexpr int kSmem = kCsOff + (kGqaDim / 2) * 8;
constexpr int kLoadsK = kStageB / 1024;                 // direct loads per stage: 1 KB each
constexpr int kPerStage = 2 * kLoadsK;
constexpr int kAhead = kNBuf - 1;
static_assert(kSmem <= 80 * 1024, "two workgroups per CU");
static_assert(kPerStage * kAhead <= 63, "vmcnt range");
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ uint32_t kkey(int r) { return 4u * (uint32_t)(r >> 3) + (uint32_t)(r & 3); }
__device__ __forceinline__ uint32_t vkey(int r) { return (uint32_t)(r & 3) | ((uint32_t)((r >> 3) & 1) << 2); }

__device__ __forceinline__ void raise_error(uint32_t bit) {
    __hip_atomic_fetch_or(&g_errors_gqa_decode, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float bf_at(const v4u& v, int e) {
    return (e & 1) ? bf_hi(v[e >> 1]) : bf_lo(v[e >> 1]);
}

__global__ __launch_bounds__(64) void gqa_decode_kernel(const GqaDecodeArgs A) {
    __shared__ __attribute__((aligned(1024))) char smem[kSmem];
    const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;
    int32_t* s_blk = reinterpret_cast<int32_t*>(smem + kBlkOff);
    int32_t* s_pend = reinterpret_cast<int32_t*>(smem + kPendOff);
    double* s_omega = reinterpret_cast<double*>(smem + kOmegaOff);
    float2* s_cs = reinterpret_cast<float2*>(smem + kCsOff);

    const int lane = threadIdx.x;
    const int n = lane & 15, c4 = lane >> 4;             // column (query head of the group), row group
    const int g = blockIdx.x % A.kv_heads;
    const int bs = blockIdx.x / A.kv_heads;
    const int sp = bs % A.n_split, b = bs / A.n_split;

    const int len = max(0, min(A.seq_lens[b], A.max_len));
    const int nblk_seq = (len + kBlk - 1) / kBlk;
    const int blk0 = sp * A.blocks_per_split;
    const int nb = max(0, min(A.blocks_per_split, nblk_seq - blk0));
    // stages holding at least one token of the sequence
    const int n_st = nb > 0 ? min(2 * nb, (len - blk0 * kBlk + kStage - 1) / kStage) : 0;

    // ---- per-split tables; theta table --------------------------------------
    for (int e = lane; e < nb; e += 64) {
        int id = A.bt[(int64_t)b * A.bt_stride + blk0 + e];
        if ((unsigned)id >= (unsigned)A.n_blocks) { raise_error(KVR_DEV_BAD_BLOCK); id = -1; }
        s_blk[e] = id;
        s_pend[e] = A.pend[(int64_t)b * A.bt_stride + blk0 + e];
    }
    s_omega[lane] = A.omega[lane];

    // ---- this lane's query dimensions 32s + 8 c4 + e (s < 4, e < 8) ----------
    v4u qraw[4];
    {
        const bool real = n < A.group;
        const int64_t qrow = (int64_t)b * A.q_heads + g * A.group + (real ? n : 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            qraw[s] = *reinterpret_cast<const v4u*>(A.q + qrow * kGqaDim + 32 * s + 8 * c4);
            if (!real) qraw[s] = v4u{0, 0, 0, 0};
        }
    }
    // every load so far has landed (the compiler accounts for this wait too,
    // so it adds none later that would drain the direct loads)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // Direct loads of stage jj into buffer jj % kNBuf: K rows 4i..4i+3 for
    // i < kLoadsK, then V rows.  Stages past the split reload its last stage
    // (into a buffer nobody reads again) and a bad block id loads block 0
    // (those rows are masked, and V zeroed, once landed), so every iteration
    // issues the same number of loads.
    auto issue = [&](int jj) __attribute__((always_inline)) {
        const int j = min(jj, n_st - 1);
        const int id = max(0, __builtin_amdgcn_readfirstlane(s_blk[j >> 1]));
        const int64_t row0 = kStage * (j & 1);
        const char* kb = A.k + (int64_t)id * A.k_b + row0 * A.k_r + g * kRowB;
        const char* vb = A.v + (int64_t)id * A.v_b + row0 * A.v_r + g * kRowB;
        const int rr = lane >> 4, p = lane & 15;
        const uint32_t buf = (uint32_t)(jj % kNBuf) * kStageB;
#pragma unroll
        for (int i = 0; i < kLoadsK; ++i) {
            const int r = 4 * i + rr;
            dma16(kb + (int64_t)(4 * i) * A.k_r, (uint32_t)rr * (uint32_t)A.k_r + 16u * ((uint32_t)p ^ kkey(r)),
                  lds0 + kKOff + buf + 1024 * i);
        }
#pragma unroll
        for (int i = 0; i < kLoadsK; ++i) {
            const int r = 4 * i + rr;
            dma16(vb + (int64_t)(4 * i) * A.v_r, (uint32_t)rr * (uint32_t)A.v_r + 16u * ((uint32_t)p ^ (2u * vkey(r))),
                  lds0 + kVOff + buf + 1024 * i);
        }
    };
    // V rows of stage j at or past the sequence end (all rows if the block id
    // is bad) are zeroed: their P is 0, and 0 * (NaN left in an unused cache
    // row) would still poison O.
    auto zero_tail = [&](int j) __attribute__((always_inline)) {
        const int valid = __builtin_amdgcn_readfirstlane((int)(s_blk[j >> 1] >= 0));
        const int first = valid ? max(0, len - (blk0 * kBlk + kStage * j)) : 0;
        if (first >= kStage) return;
        const uint32_t vb = lds0 + kVOff + (uint32_t)(j % kNBuf) * kStageB;
        for (int e = first * 16 + lane; e < kStage * 16; e += 64)
            *(lds_v4u*)(size_t)(vb + 16 * e) = v4u{0, 0, 0, 0};
    };

    // ---- query re-rotation for block i: q' = R(-delta_i) q, hi and lo -------
    v8bf qhi[4], qlo[4];
    auto rotate_q = [&](int i) __attribute__((always_inline)) {
        // lane l: (cos, sin) of pair l, the angle reduced in float64 to a
        // fraction of a revolution (the hardware sine and cosine take those)
        {
            const double u = (double)s_pend[i] * s_omega[lane];
            const float f = (float)(u - rint(u));
            s_cs[lane] = make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
        }
        // the other lanes' entries are read next: order them after the writes
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        // pair j = 32s + 8 c4 + e (s < 2) couples qraw[s][e] and qraw[s + 2][e]
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float2 cs = s_cs[32 * s + 8 * c4 + e];
                const float x = bf_at(qraw[s], e), y = bf_at(qraw[s + 2], e);
                const float xr = x * cs.x + y * cs.y;          // R(-delta): sin -> -sin
                const float yr = y * cs.x - x * cs.y;
                const __bf16 xh = (__bf16)xr, yh = (__bf16)yr;
                qhi[s][e] = xh;
                qhi[s + 2][e] = yh;
                qlo[s][e] = (__bf16)(xr - (float)xh);
                qlo[s + 2][e] = (__bf16)(yr - (float)yh);
            }
        }
    };

    v4f acc[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;   // l_run: this lane's share (tokens 8 c4 .. 8 c4 + 7)

    auto stage = [&](int j) __attribute__((always_inline)) {
        // S^T for tiles A and B
        const uint32_t kbuf = lds0 + kKOff + (uint32_t)(j % kNBuf) * kStageB;
        const uint32_t ra = kbuf + (uint32_t)(8 * (n >> 2) + (n & 3)) * kRowB;   // kkey of both rows is n
        const uint32_t rb = ra + 4 * kRowB;
        v4f sa = v4f{0.f, 0.f, 0.f, 0.f}, sb = sa;
        v4u ka[4], kb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t off = 16u * ((uint32_t)(4 * s + c4) ^ (uint32_t)n);
            ka[s] = lds16_at(ra + off);
            kb[s] = lds16_at(rb + off);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(ka[s]), qhi[s], sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(kb[s]), qhi[s], sb, 0, 0, 0);
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(ka[s]), qlo[s], sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(kb[s]), qlo[s], sb, 0, 0, 0);
        }
        issue(j + kAhead);

        // softmax over this lane's 8 tokens 8 c4 + e (tile A: e < 4, tile B: e >= 4)
        const bool valid = __builtin_amdgcn_readfirstlane((int)(s_blk[j >> 1] >= 0)) != 0;
        const int tok_base = blk0 * kBlk + kStage * j;
        const bool full = valid && tok_base + kStage <= len;
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = sa[e] * A.scale_log2;
            x[e + 4] = sb[e] * A.scale_log2;
        }
        if (!full) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (!valid || tok_base + 8 * c4 + e >= len) x[e] = kNegInf;
        }
        float mt = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mt = fmaxf(mt, x[e]);
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = max_halves(mt);
        const float m_new = fmaxf(m_run, mt);
        const float mr = m_new == kNegInf ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - mr);   // 0 while m_run = -inf
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int f = 0; f < 8; ++f) acc[f] *= alpha;
        }
        l_run *= alpha;
        m_run = m_new;
        // P in bf16, summed from the same bf16 values so that numerator and
        // denominator agree
        v8bf pb;
        const v2bf ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const v2bf pr = {(__bf16)__builtin_amdgcn_exp2f(x[e] - mr), (__bf16)__builtin_amdgcn_exp2f(x[e + 1] - mr)};
            pb[e] = pr[0];
            pb[e + 1] = pr[1];
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
        }

        // O^T += V^T P^T: this lane addresses rows r1 = 8 c4 + sl/4 (tokens
        // 8 c4 .. 8 c4 + 3 of the group) and r2 = r1 + 4, 8 bytes at columns
        // 16 f + 4 (sl % 4)
        const uint32_t vbuf = lds0 + kVOff + (uint32_t)(j % kNBuf) * kStageB;
        const int sl = lane & 15;
        const int r1 = 8 * c4 + (sl >> 2), r2 = r1 + 4;
        const uint32_t cl = (uint32_t)((sl & 3) >> 1), hb = 8u * (uint32_t)(sl & 1);
        const uint32_t a1 = vbuf + (uint32_t)r1 * kRowB + hb, a2 = vbuf + (uint32_t)r2 * kRowB + hb;
        const uint32_t k1 = 2u * vkey(r1), k2 = 2u * vkey(r2);
        v4s w1[8], w2[8];
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            w1[f] = lds_tr_at(a1 + 16u * ((2u * f + cl) ^ k1));
            w2[f] = lds_tr_at(a2 + 16u * ((2u * f + cl) ^ k2));
        }
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            const v8bf va = __builtin_bit_cast(v8bf, __builtin_shufflevector(w1[f], w2[f], 0, 1, 2, 3, 4, 5, 6, 7));
            acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[f], 0, 0, 0);
        }
    };

    if (n_st > 0) {
        for (int jj = 0; jj < kAhead; ++jj) issue(jj);
        wait_vmcnt<kPerStage * (kAhead - 1)>();     // stage 0 landed
        zero_tail(0);
        int cur = -1;
        for (int j = 0; j < n_st; ++j) {
            if ((j >> 1) != cur) {
                cur = j >> 1;
                rotate_q(cur);
            }
            stage(j);
            wait_vmcnt<kPerStage * (kAhead - 1)>(); // stage j + 1 landed
            if (j + 1 < n_st) zero_tail(j + 1);
        }
        wait_vmcnt<0>();                            // no load may land in LDS after this
    }

    // ---- unnormalized partials: this head's features 16 f + 4 c4 + i --------
    l_run += __shfl_xor(l_run, 16);
    l_run = sum_halves(l_run);
    if (n < A.group) {
        const int64_t row = (((int64_t)b * A.kv_heads + g) * A.n_split + sp) * A.group + n;
        float* po = A.part_o + row * kGqaDim;
#pragma unroll
        for (int f = 0; f < 8; ++f) *reinterpret_cast<v4f*>(po + 16 * f + 4 * c4) = acc[f];
        if (c4 == 0) reinterpret_cast<float2*>(A.part_ml)[row] = make_float2(m_run, l_run);
    }
}

// Merge the splits: O = sum_s 2^(m_s - M) O_s / L, L = sum_s 2^(m_s - M) l_s,
// LSE = ln 2 * (M + log2 L).  One workgroup per (sequence, query head), one
// thread per feature; the split loops are unrolled so their loads overlap.
__global__ __launch_bounds__(kGqaDim) void gqa_decode_combine(const GqaDecodeArgs A, uint16_t* out, float* lse) {
    const int h = blockIdx.x % A.q_heads, b = blockIdx.x / A.q_heads;
    const int g = h / A.group, i = h - g * A.group;
    const int f = threadIdx.x;
    const int64_t base = ((int64_t)b * A.kv_heads + g) * A.n_split;      // row = (base + s) * group + i
    const float2* pm = reinterpret_cast<const float2*>(A.part_ml);
    float M = kNegInf;
#pragma unroll 8
    for (int s = 0; s < A.n_split; ++s) M = fmaxf(M, pm[(base + s) * A.group + i].x);
    float L = 0.f, o = 0.f;
#pragma unroll 8
    for (int s = 0; s < A.n_split; ++s) {
        const int64_t row = (base + s) * A.group + i;
        const float2 ml = pm[row];
        const float w = ml.x == kNegInf ? 0.f : exp2f(ml.x - M);
        L += w * ml.y;
        o += w * A.part_o[row * kGqaDim + f];
    }
    const int64_t oh = (int64_t)b * A.q_heads + h;
    out[oh * kGqaDim + f] = __builtin_bit_cast(uint16_t, (__bf16)(L > 0.f ? o / L : 0.f));
    if (f == 0) lse[oh] = L > 0.f ? 0.6931471805599453f * (M + log2f(L)) : kNegInf;
}

}  // namespace

hipError_t launch_gqa_decode(const GqaDecodeArgs& a, uint16_t* out, float* lse, hipStream_t s) {
    hipLaunchKernelGGL(gqa_decode_kernel, dim3((unsigned)(a.batch * a.n_split * a.kv_heads)), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gqa_decode_combine, dim3((unsigned)(a.batch * a.q_heads)), dim3(kGqaDim), 0, s, a, out, lse);
    return hipGetLastError();
}

uint32_t read_and_clear_errors_gqa_decode() {
    uint32_t v = 0, z = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_errors_gqa_decode), sizeof(v)) != hipSuccess) return 0xffffffffu;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_errors_gqa_decode), &z, sizeof(z)) != hipSuccess) return 0xffffffffu;
    return v;
}

}  // namespace kvr
