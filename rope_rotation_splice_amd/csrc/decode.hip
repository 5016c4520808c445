// One decode step of absorbed-form MLA attention over a paged cache whose
// blocks carry a pending rotary shift, with the delta-rotation applied while
// the keys are loaded (Irminsul, sections 2.2 and 4: the rotation is fused
// into attention on the HBM -> on-chip path; section 5: absorbed matmul form).
//
//   s_t = scale * (q_nope . cKV_t + q_rope . R(delta_blk(t)) k_r_t)
//   O   = sum_t softmax(s)_t cKV_t,     LSE = ln sum_t exp(s_t)
//
// Work split (flash-decoding): one workgroup per (sequence, KV split), one
// wave per 32 query heads (4 waves = 128 heads), q held in registers for the
// whole split.  Nothing rotated is written back to HBM.
//
// Load pipeline.  A split is walked in stages of 32 tokens (half a 64-token
// block).  Both parts of a stage's rows go global -> LDS directly (16 bytes
// per lane, no registers): the cKV rows into one of 4 stage buffers, the raw
// k_r rows into one of 4 k_r buffers.  Loads run 3 stages ahead.  At the end
// of stage j each wave waits until only the loads of stages j+2 and j+3 are
// outstanding (vmcnt retires loads in order), the workgroup rotates stage
// j+1's k_r in place in fp32 by its block's pending delta, and one barrier
// publishes stage j+1.  The direct loads are issued from inline assembly:
// the compiler would otherwise wait for every outstanding direct load before
// any later LDS read, which serializes the pipeline; the waits here are
// explicit and exact instead.  (cos, sin) of each block's shift live in a
// 4-block ring filled 3 stages before use.
//
// LDS layouts.  cKV rows are unpadded (1024 bytes) with their 16-byte chunks
// permuted: chunk c of row r sits at position c ^ swz(r), where swz maps r
// mod 16 one-to-one onto 0..15 and puts r's two low bits into position bits
// 2-3.  The K-row reads (16 rows x one chunk per 16 lanes) and the transpose
// reads (4 rows x 64 contiguous bytes per 32 lanes) then each touch every LDS
// bank once.  k_r rows (128 bytes) use chunk c at position c ^ ((r >> 1) & 7),
// which spreads 16 consecutive rows' chunk reads over all banks.  A direct
// load writes position l from lane l, so lane l fetches the chunk that
// belongs there.
//
// Matrix cores (v_mfma_f32_32x32x16_bf16, lane l holds output rows
// 8*(r/4) + 4*(l/32) + r%4 of column l%32):
// * S^T = K Q^T per stage: K rows (A) read from LDS, q (B) from registers.
//   Lane l then holds 16 tokens of head l%32, so the per-head softmax
//   statistics need one cross-lane exchange (lanes l and l^32).
// * O^T += V^T P^T per 16-token step: P (B) comes straight from the S^T
//   registers -- the K-dimension slots are matched to the tokens a lane holds
//   -- and V^T (A) is read from the row-major cKV tile with the LDS transpose
//   read ds_read_b64_tr_b16 (source lane s addresses row K0 + s/4, columns
//   C + 4*(s%4); destination lane d of the 16-lane group receives rows
//   K0..K0+3 of column C + d).  O^T keeps head l%32 in lane l, the same head
//   as the softmax statistics, so rescaling is lane-local.
// LDS operands stream through 4-deep register windows ahead of the MFMAs.
// Softmax runs in base 2 with the scale folded in.  The 256 accumulators of a
// wave live in AGPRs and the main loop touches them only through the matrix
// cores (any VALU access there makes the compiler spill): each head keeps a
// fixed reference maximum (its first stage's maximum) and P = 2^(x - m_ref)
// may exceed 1 by up to 2^48 (fp32 and bf16 share the exponent range).  If a
// stage overshoots that headroom, the workgroup finishes the stage, abandons
// the pass and restarts the split with the observed maxima as references (at
// most kPasses passes; then KVR_DEV_RANGE is raised and the last pass
// completes).  Splits write unnormalized partials (lane-native layout) that a
// combine kernel merges.
#include <type_traits>

#include "kvr_device.h"
#include "kvr_internal.h"
#include "kvr_lds.h"

#include "../../include/kvreloc.h"

namespace kvr {

__device__ uint32_t g_errors_decode;

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int kBlk = kDecBlockTokens;                    // tokens per KV block
constexpr int kStage = 32;                              // tokens per pipeline stage
constexpr int kNBuf = 4;                                // stage buffers (3 loads ahead)
constexpr int kCkvRow = 1024;                           // LDS bytes per cKV row (chunk-swizzled)
constexpr int kKrRow = 128;                             // LDS bytes per k_r row (chunk-swizzled)
constexpr int kCkvStageB = kStage * kCkvRow;
constexpr int kKrStageB = kStage * kKrRow;
constexpr int kKrOff = kNBuf * kCkvStageB;
constexpr int kCsOff = kKrOff + kNBuf * kKrStageB;      // (cos, sin) ring: 4 blocks x 32 pairs
constexpr int kBlkOff = kCsOff + 4 * 32 * 8;            // block ids of the split
constexpr int kPendOff = kBlkOff + kDecMaxBlocks * 4;   // pending shifts of the split
constexpr int kOmegaOff = kPendOff + kDecMaxBlocks * 4; // theta_j / 2 pi, float64
constexpr int kFlagOff = kOmegaOff + 32 * 8;            // restart flag
constexpr int kSmem = kFlagOff + 16;
static_assert(kSmem <= 160 * 1024, "LDS budget");
constexpr float kNegInf = -__builtin_inff();

// chunk permutations of the rows in LDS
__device__ __forceinline__ uint32_t swz(int r) { return 4u * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ uint32_t swz_kr(int r) { return (uint32_t)(r >> 1) & 7u; }

__device__ __forceinline__ void raise_error(uint32_t bit) {
    __hip_atomic_fetch_or(&g_errors_decode, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Rotate 4 bf16 pairs: lo holds x_j..x_{j+3}, hi holds x_{j+h}..x_{j+h+3}.
__device__ __forceinline__ void rot_bf16x4(v2u& lo, v2u& hi, const float2* cs) {
    float a0, b0, a1, b1, a2, b2, a3, b3;
    rot2(bf_lo(lo.x), bf_lo(hi.x), cs[0].x, cs[0].y, a0, b0);
    rot2(bf_hi(lo.x), bf_hi(hi.x), cs[1].x, cs[1].y, a1, b1);
    rot2(bf_lo(lo.y), bf_lo(hi.y), cs[2].x, cs[2].y, a2, b2);
    rot2(bf_hi(lo.y), bf_hi(hi.y), cs[3].x, cs[3].y, a3, b3);
    lo = v2u{pack_bf16(a0, a1), pack_bf16(a2, a3)};
    hi = v2u{pack_bf16(b0, b1), pack_bf16(b2, b3)};
}

constexpr float kHeadroom = 48.f;      // log2 of the largest P before a restart
constexpr int kPasses = 3;

template <int NW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_kernel(const DecodeArgs A) {
    // the only LDS variable, so its 1024-byte alignment makes every row base
    // a multiple of the row size and the chunk swizzles plain XORs of offsets
    __shared__ __attribute__((aligned(1024))) char smem[kSmem];
    const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;
    float2* cs_s = reinterpret_cast<float2*>(smem + kCsOff);
    int32_t* s_blk = reinterpret_cast<int32_t*>(smem + kBlkOff);
    int32_t* s_pend = reinterpret_cast<int32_t*>(smem + kPendOff);
    double* s_omega = reinterpret_cast<double*>(smem + kOmegaOff);
    int& s_overshoot = *reinterpret_cast<int*>(smem + kFlagOff);

    const int tid = threadIdx.x, nthr = NW * 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n = lane & 31, half = lane >> 5;
    const int b = blockIdx.x / A.n_split, sp = blockIdx.x - b * A.n_split;
    const int head = wave * 32 + n;

    const int len = max(0, min(A.seq_lens[b], A.max_len));
    const int nblk_seq = (len + kBlk - 1) / kBlk;
    const int blk0 = sp * A.blocks_per_split;
    const int nb = max(0, min(A.blocks_per_split, nblk_seq - blk0));
    // stages holding at least one token of the sequence
    const int n_st = nb > 0 ? min(2 * nb, (len - blk0 * kBlk + kStage - 1) / kStage) : 0;

    // ---- per-split tables: block ids and pending shifts ---------------------
    for (int e = tid; e < nb; e += nthr) {
        int id = A.bt[(int64_t)b * A.bt_stride + blk0 + e];
        if ((unsigned)id >= (unsigned)A.n_blocks) { raise_error(KVR_DEV_BAD_BLOCK); id = -1; }
        s_blk[e] = id;
        s_pend[e] = A.pend[(int64_t)b * A.bt_stride + blk0 + e];
    }
    if (tid < 32) s_omega[tid] = A.omega[tid];

    // ---- q for this lane's head: B operand of S^T = K Q^T, 36 K-steps -------
    v8bf q[36];
    {
        const int64_t qh = (int64_t)b * A.heads + head;
#pragma unroll
        for (int s = 0; s < 32; ++s)
            q[s] = as_bf(*reinterpret_cast<const v4u*>(A.q_nope + qh * 512 + 16 * s + 8 * half));
#pragma unroll
        for (int s = 0; s < 4; ++s)
            q[32 + s] = as_bf(*reinterpret_cast<const v4u*>(A.q_rope + qh * 64 + 16 * s + 8 * half));
    }
    // all loads so far have landed (a wait the compiler also accounts for, so
    // it adds none later that would drain the direct loads)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // a stage is live if it exists and its block id is valid (uniform)
    auto live = [&](int j) __attribute__((always_inline)) -> bool {
        return __builtin_amdgcn_readfirstlane((int)(j < n_st && s_blk[j >> 1] >= 0)) != 0;
    };
    // (cos, sin) of block i's shift into ring slot i % 4: threads 0..31.
    // The angle is reduced in float64 to f in [-1/2, 1/2] revolution; the
    // hardware sine and cosine take revolutions, so f goes in directly.
    // Every wave computes them (lanes share pairs); threads 0..31 store.
    auto angles = [&](int i) __attribute__((always_inline)) {
        const double u = (double)s_pend[i] * s_omega[tid & 31];
        const float f = (float)(u - rint(u));
        const float2 v = make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
        if (tid < 32) cs_s[(i & 3) * 32 + tid] = v;
    };
    // Direct loads of stage j, as items of this wave: cKV rows r = wave + k NW
    // (k < nc), then k_r row groups g = wave + (k - nc) NW (8 rows of 128
    // bytes per instruction).  With NW dividing both counts every wave has
    // the same items and their kinds are known at compile time.  Stages past
    // the split reload its last stage (into a buffer nobody reads again, from
    // L2) and a bad block id loads block 0 (its rows are zeroed once landed),
    // so every iteration issues the same loads and no branch splits the
    // matrix-core loop.
    constexpr bool kEven = (kStage % NW == 0) && ((kStage / 8) % NW == 0);
    const int nc = kEven ? kStage / NW : (kStage - wave + NW - 1) / NW;
    const int n_items = kEven ? kStage / NW + (kStage / 8) / NW : nc + (kStage / 8 - wave + NW - 1) / NW;
    // The source rows of stage jj are looked up once, before its loads are
    // issued: the direct loads clobber memory as far as the compiler knows,
    // so a table read between them would be repeated, and each repeat waits
    // for every LDS read in flight.
    struct StageSrc { const char* ck; const char* kr; };
    auto stage_src = [&](int jj) __attribute__((always_inline)) -> StageSrc {
        const int j = min(jj, n_st - 1);
        const int id = max(0, __builtin_amdgcn_readfirstlane(s_blk[j >> 1]));
        const int64_t row0 = 32 * (j & 1);
        return {A.ckv + (int64_t)id * A.ckv_b + row0 * A.ckv_r, A.kr + (int64_t)id * A.kr_b + row0 * A.kr_r};
    };
    auto issue_item = [&](int jj, const StageSrc& src, int k) __attribute__((always_inline)) {
        if (k < nc) {
            const int r = wave + NW * k;
            dma16(src.ck + r * A.ckv_r, 16u * (lane ^ swz(r)), lds0 + (jj & 3) * kCkvStageB + r * kCkvRow);
        } else {
            const int g = wave + NW * (k - nc);
            const int r = 8 * g + (lane >> 3);
            dma16(src.kr + 8 * g * A.kr_r,
                  (uint32_t)(lane >> 3) * (uint32_t)A.kr_r + 16u * ((lane & 7) ^ swz_kr(r)),
                  lds0 + kKrOff + (jj & 3) * kKrStageB + g * 1024);
        }
    };
    auto issue_all = [&](int j) __attribute__((always_inline)) {
        const StageSrc src = stage_src(j);
        for (int k = 0; k < n_items; ++k) issue_item(j, src, k);
    };
    // rotate stage j's k_r in place: item e = (row e/8, 8-byte unit e%8 of
    // the lo half and its partner in the hi half)
    auto rotate_kr = [&](int j) __attribute__((always_inline)) {
        const uint32_t kb = lds0 + kKrOff + (j & 3) * kKrStageB;
        const float2* cs = cs_s + ((j >> 1) & 3) * 32;
#pragma unroll
        for (int k = 0; k < (kStage * 8 + nthr - 1) / nthr; ++k) {
            const int e = tid + k * nthr;
            if ((kStage * 8) % nthr != 0 && e >= kStage * 8) break;
            const int r = e >> 3, u = e & 7;
            const uint32_t rb = kb + r * kKrRow + 8 * (u & 1);
            const uint32_t plo = rb + 16 * ((uint32_t)(u >> 1) ^ swz_kr(r));
            const uint32_t phi = rb + 16 * ((uint32_t)((u >> 1) + 4) ^ swz_kr(r));
            v2u lo = lds8_at(plo), hi = lds8_at(phi);
            rot_bf16x4(lo, hi, cs + 4 * u);
            lds8_put(plo, lo);
            lds8_put(phi, hi);
        }
    };
    // cKV rows of stage j at or past the sequence end (all rows if the block
    // id is bad) are zeroed: their P is 0, and 0 * (NaN left in an unused
    // cache row) would still poison O.
    auto zero_tail = [&](int j) __attribute__((always_inline)) {
        const int valid = __builtin_amdgcn_readfirstlane((int)(s_blk[j >> 1] >= 0));
        const int first = valid ? max(0, len - (blk0 * kBlk + kStage * j)) : 0;
        if (first >= kStage) return;
        const uint32_t cb = lds0 + (j & 3) * kCkvStageB;
        for (int e = first * 64 + tid; e < kStage * 64; e += nthr)
            *(lds_v4u*)(size_t)(cb + 16 * e) = v4u{0, 0, 0, 0};
    };
    // loads per stage and wave: the fewest any wave issues
    constexpr int kPerStage = kStage / NW + (kStage / 8) / NW;
    constexpr int kItemsMax = (kStage + NW - 1) / NW + (kStage / 8 + NW - 1) / NW;
    constexpr int kSlot = 36 / kItemsMax;                 // S^T steps per load issued
    constexpr int kW1 = kPerStage < 63 ? kPerStage : 63;

    v16f acc[16];
    float m_run = kNegInf, l_run = 0.f;
    float m_hint = kNegInf;                 // references carried into a restarted pass

    // softmax of stage j from its S^T: P (bf16) and the running statistics
    auto softmax = [&](int j, const v16f& sacc, bool last_pass, v8bf* pb) __attribute__((always_inline)) {
        const bool valid = __builtin_amdgcn_readfirstlane((int)(s_blk[j >> 1] >= 0)) != 0;
        const int tok_base = blk0 * kBlk + kStage * j;
        // a stage wholly inside the sequence needs no mask (uniform)
        const bool full = valid && tok_base + kStage <= len;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = sacc[r] * A.scale_log2;
        if (!full) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int t = 8 * (r >> 2) + 4 * half + (r & 3);
                if (!valid || tok_base + t >= len) x[r] = kNegInf;
            }
        }
        float mt = x[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
        mt = max_halves(mt);
        // the first live stage of a head fixes its reference; an overshoot
        // beyond the headroom abandons this pass (decided per workgroup at
        // the end of the stage)
        if (m_run == kNegInf) m_run = mt;
        if (mt > m_run + kHeadroom) {
            m_hint = fmaxf(m_hint, mt);
            if (!last_pass) s_overshoot = 1;
            else raise_error(KVR_DEV_RANGE);
        }
        m_hint = fmaxf(m_hint, m_run);
        // P in bf16, summed from the same bf16 values so that numerator and
        // denominator agree.  P <= 2^48 and exp2 of anything below -126 may
        // flush to zero, so the bare hardware exp2 is exact enough.  A head
        // with no live token yet has m_run = x = -inf: P = exp2(-inf) = 0.
        const float mr = m_run == kNegInf ? 0.f : m_run;
        const v2bf ones = {(__bf16)1.f, (__bf16)1.f};
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const v2bf pr = {(__bf16)__builtin_amdgcn_exp2f(x[r] - mr), (__bf16)__builtin_amdgcn_exp2f(x[r + 1] - mr)};
            pb[r >> 3][r & 7] = pr[0];
            pb[r >> 3][(r & 7) + 1] = pr[1];
            ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls, false);
        }
        ls = sum_halves(ls);
        l_run += ls;
    };

    // One stage of attention: S^T, softmax, O^T += V^T P^T.  The loads of
    // stage j+3 are spread over the S^T steps; between the two O^T steps
    // stage j+1's k_r is rotated and block (j+3)/2's angles are computed.
    // Stage j+1's k_r landed before the last barrier; stages beyond the
    // split only touch buffers and ring slots nobody reads again.
    auto compute = [&](int j, bool last_pass) __attribute__((always_inline)) {
        const uint32_t ck = lds0 + (j & 3) * kCkvStageB;
        const uint32_t kq = lds0 + kKrOff + (j & 3) * kKrStageB;

        // S^T: rows = 32 tokens, columns = 32 heads.  Chunk 2s + half of cKV
        // row n sits at position (2s) ^ (half ^ swz(n)); chunk 2s' + half of
        // k_r row n at (2s') ^ (half ^ swz_kr(n)).
        const uint32_t krow = ck + n * kCkvRow + 16 * (half ^ swz(n));
        const uint32_t rrow = kq + n * kKrRow + 16 * (half ^ swz_kr(n));
        auto kop = [&](int s) __attribute__((always_inline)) {
            return s < 32 ? lds16_at((krow ^ (32u * (s & 7))) + 256u * (s >> 3)) : lds16_at(rrow ^ (32u * (s - 32)));
        };
        const StageSrc src3 = stage_src(j + 3);
        v16f sacc = v16f{};
        constexpr int kWin = 4;             // K-row reads in flight ahead of the MFMAs
        v4u kw[kWin];
#pragma unroll
        for (int s = 0; s < kWin; ++s) kw[s] = kop(s);
        __builtin_amdgcn_sched_group_barrier(0x100, kWin, 0);
#pragma unroll
        for (int s = 0; s < 36; ++s) {
            const v4u cur = kw[s % kWin];
            if (s + kWin < 36) kw[s % kWin] = kop(s + kWin);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(cur), q[s], sacc, 0, 0, 0);
            if (s % kSlot == 0 && s / kSlot < kItemsMax && (kEven || s / kSlot < n_items)) issue_item(j + 3, src3, s / kSlot);
            // keep the window: each K-row read is issued before the MFMA
            // that precedes its use by kWin steps
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (s + kWin < 36) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }

        v8bf pb[2];
        softmax(j, sacc, last_pass, pb);

        // O^T += V^T P^T over two 16-token steps; transpose reads run 4
        // feature tiles ahead of the matrix core
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (s == 1) {
                // between the two steps no read window is live
                rotate_kr(j + 1);
                angles(min((j + 3) >> 1, nb - 1));
            }
            // this lane's 8 bytes of feature tile f (64 bytes per row) start
            // at byte 64f + 16cl + 8(sl&1) of rows ka and ka + 8
            const int sl = lane & 15;
            const int ka = 16 * s + 4 * half + (sl >> 2);
            const uint32_t cl = 2 * ((lane >> 4) & 1) + ((sl & 3) >> 1);
            const uint32_t ra = ck + ka * kCkvRow + 16 * (cl ^ swz(ka)) + 8 * (sl & 1);
            const uint32_t rb = ck + (ka + 8) * kCkvRow + 16 * (cl ^ swz(ka + 8)) + 8 * (sl & 1);
            auto tr = [&](uint32_t base, int f) __attribute__((always_inline)) {
                return lds_tr_at((base ^ (64u * (f & 3))) + 256u * (f >> 2));
            };
            v4s wa[4], wb[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) { wa[f] = tr(ra, f); wb[f] = tr(rb, f); }
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int f = 0; f < 16; ++f) {
                const v4s ta = wa[f & 3], tb = wb[f & 3];
                if (f + 4 < 16) { wa[f & 3] = tr(ra, f + 4); wb[f & 3] = tr(rb, f + 4); }
                const v8bf va = __builtin_bit_cast(v8bf, __builtin_shufflevector(ta, tb, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[s], acc[f], 0, 0, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (f + 4 < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        }
    };

    for (int pass = 0; pass < kPasses; ++pass) {
#pragma unroll
        for (int f = 0; f < 16; ++f) acc[f] = v16f{};
        m_run = m_hint;
        l_run = 0.f;
        const bool last_pass = pass + 1 == kPasses;
        __syncthreads();                    // everyone has read the previous flag
        if (tid == 0) s_overshoot = 0;
        // prologue: angles of blocks 0 and 1, loads of stages 0..2; stage 0
        // ready (landed, tail zeroed, k_r rotated) and stage 1 landed
        if (nb > 0) angles(0);
        if (nb > 1) angles(1);
        if (n_st > 0) { issue_all(0); issue_all(1); issue_all(2); }
        wait_vmcnt<kW1>();
        __syncthreads();
        if (0 < n_st) { zero_tail(0); rotate_kr(0); }
        __syncthreads();

        // Iteration j: attention over stage j, with stage j+1's k_r rotated
        // and stage j+3's loads issued on the way; at the end stage j+2 has
        // landed and one barrier makes stages j+1 and j+2 visible.
        bool restart = false;
        for (int j = 0; !restart && j < n_st; ++j) {
            if (j + 1 < n_st) zero_tail(j + 1);
            compute(j, last_pass);
            wait_vmcnt<kW1>();              // stage j+2 landed
            __syncthreads();
            restart = __builtin_amdgcn_readfirstlane(s_overshoot) != 0;
        }
        wait_vmcnt<0>();                    // no load may land in LDS after this
        if (!restart) break;
    }

    // ---- unnormalized partials in the lane-native layout ---------------------
    float* po = A.part_o + (((int64_t)b * A.n_split + sp) * NW + wave) * (16 * 16 * 64);
#pragma unroll
    for (int f = 0; f < 16; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) po[(f * 16 + r) * 64 + lane] = acc[f][r];
    if (half == 0) {
        float2* pm = reinterpret_cast<float2*>(A.part_ml) + ((int64_t)b * A.n_split + sp) * A.heads + head;
        *pm = make_float2(m_run, l_run);
    }
}

// Merge the splits: O = sum_s 2^(m_s - M) O_s / L, L = sum_s 2^(m_s - M) l_s,
// LSE = ln 2 * (M + log2 L).  One workgroup per (sequence, wave's 32 heads,
// quarter of the 512 features = 4 feature tiles).  Partials are read in
// their lane-native order as float4 (coalesced), the merged values go
// through LDS as [head][feature] bf16, and leave as 256-byte row segments.
constexpr int kCombineSplitChunk = 256;     // split weights staged in LDS at a time

__global__ __launch_bounds__(256) void mla_decode_combine(const DecodeArgs A, uint16_t* out, float* lse) {
    __shared__ float s_w[kCombineSplitChunk][32];
    __shared__ float s_M[32], s_L[32];
    __shared__ uint16_t s_o[32][128 + 8];
    const int tid = threadIdx.x;
    const int n_waves = A.heads / 32;
    const int q = blockIdx.x & 3;                        // feature quarter: tiles 4q .. 4q+3
    const int bw = blockIdx.x >> 2;
    const int b = bw / n_waves, wave = bw - b * n_waves;
    const float2* pm = reinterpret_cast<const float2*>(A.part_ml) + (int64_t)b * A.n_split * A.heads + wave * 32;

    if (tid < 32) {
        float M = kNegInf;
        for (int s = 0; s < A.n_split; ++s) M = fmaxf(M, pm[(int64_t)s * A.heads + tid].x);
        float L = 0.f;
        if (M != kNegInf)
            for (int s = 0; s < A.n_split; ++s) {
                const float2 ml = pm[(int64_t)s * A.heads + tid];
                if (ml.x != kNegInf) L += exp2f(ml.x - M) * ml.y;
            }
        s_M[tid] = M;
        s_L[tid] = L;
    }
    // this thread's float4 units u = tid + 256 k (k < 4) of the quarter's
    // 4 x 16 x 64 lane-native floats: element e = 4u + i has tile f = e / 1024,
    // row r = (e / 64) % 16, lane (e % 64)
    v4f acc[4] = {};
    const int64_t base0 = (((int64_t)b * A.n_split) * n_waves + wave) * (16 * 16 * 64) + (int64_t)q * 4 * 1024;
    const int64_t split_stride = (int64_t)n_waves * 16 * 16 * 64;
    for (int c0 = 0; c0 < A.n_split; c0 += kCombineSplitChunk) {
        const int nc = min(kCombineSplitChunk, A.n_split - c0);
        __syncthreads();                                   // s_M ready; previous chunk consumed
        for (int e = tid; e < nc * 32; e += 256) {
            const int s = e >> 5, h = e & 31;
            const float m = pm[(int64_t)(c0 + s) * A.heads + h].x;
            s_w[s][h] = (m == kNegInf || s_M[h] == kNegInf) ? 0.f : exp2f(m - s_M[h]);
        }
        __syncthreads();
        for (int s = 0; s < nc; ++s) {
            const v4f* src = reinterpret_cast<const v4f*>(A.part_o + base0 + (int64_t)(c0 + s) * split_stride);
            v4f x[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = src[tid + 256 * k];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int lane0 = (4 * (tid + 256 * k)) & 63;   // 4 consecutive lanes, same half
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[k][i] += s_w[s][(lane0 + i) & 31] * x[k][i];
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e0 = 4 * (tid + 256 * k);
        const int f = e0 >> 10, r = (e0 >> 6) & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lane = (e0 + i) & 63, h = lane & 31;
            const int feat = 32 * f + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);   // within the quarter
            const float v = s_L[h] > 0.f ? acc[k][i] / s_L[h] : 0.f;
            s_o[h][feat] = __builtin_bit_cast(uint16_t, (__bf16)v);
        }
    }
    __syncthreads();
    // 32 heads x 128 features = 512 runs of 8 bf16 (16 bytes); 2 per thread
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int unit = tid + 256 * k, h = unit >> 4, c = (unit & 15) * 8;
        uint4 v;
        v.x = s_o[h][c] | ((uint32_t)s_o[h][c + 1] << 16);
        v.y = s_o[h][c + 2] | ((uint32_t)s_o[h][c + 3] << 16);
        v.z = s_o[h][c + 4] | ((uint32_t)s_o[h][c + 5] << 16);
        v.w = s_o[h][c + 6] | ((uint32_t)s_o[h][c + 7] << 16);
        *reinterpret_cast<uint4*>(out + ((int64_t)b * A.heads + wave * 32 + h) * 512 + 128 * q + c) = v;
    }
    if (q == 0 && tid < 32)
        lse[(int64_t)b * A.heads + wave * 32 + tid] =
            s_L[tid] > 0.f ? 0.6931471805599453f * (s_M[tid] + log2f(s_L[tid])) : kNegInf;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, uint16_t* out, float* lse, hipStream_t s) {
    const dim3 grid(a.batch * a.n_split), block(a.heads * 2);
    switch (a.heads / 32) {
        case 1: hipLaunchKernelGGL(mla_decode_kernel<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(mla_decode_kernel<2>, grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL(mla_decode_kernel<3>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(mla_decode_kernel<4>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mla_decode_combine, dim3((unsigned)(a.batch * (a.heads / 32) * 4)), dim3(256), 0, s, a, out, lse);
    return hipGetLastError();
}

uint32_t read_and_clear_errors_decode() {
    uint32_t v = 0, z = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_errors_decode), sizeof(v)) != hipSuccess) return 0xffffffffu;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_errors_decode), &z, sizeof(z)) != hipSuccess) return 0xffffffffu;
    return v;
}

}  // namespace kvr
