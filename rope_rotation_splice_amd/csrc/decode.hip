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
// whole split.  KV blocks of 64 tokens are double-buffered in LDS: cKV rows go
// global -> LDS directly (16 bytes per lane, no registers); the 64-d k_r rows
// pass through registers, are rotated in fp32 by the block's pending delta
// and land in LDS as bf16.  Nothing rotated is written back to HBM.
//
// cKV rows sit in LDS unpadded (1024 bytes) with their 16-byte chunks
// permuted: chunk c of row r is stored at position c ^ swz(r), where swz
// maps r mod 16 one-to-one onto 0..15 and puts r's two low bits into
// position bits 2-3.  The K-row reads (16 rows x one chunk per 16 lanes) and
// the transpose reads (4 rows x 64 contiguous bytes per 32 lanes) then each
// touch every LDS bank once.  The direct global->LDS load writes position l
// from lane l, so lane l fetches chunk l ^ swz(r).
//
// Matrix cores (v_mfma_f32_32x32x16_bf16, lane l holds output rows
// 8*(r/4) + 4*(l/32) + r%4 of column l%32):
// * S^T = K Q^T per 32-token tile: K rows (A) read from LDS, q (B) from
//   registers.  Lane l then holds 16 tokens of head l%32, so the per-head
//   softmax statistics need one cross-lane exchange (lanes l and l^32).
// * O^T += V^T P^T per 16-token step: P (B) comes straight from the S^T
//   registers -- the K-dimension slots are matched to the tokens a lane holds
//   -- and V^T (A) is read from the row-major cKV tile with the LDS transpose
//   read ds_read_b64_tr_b16 (source lane s addresses row K0 + s/4, columns
//   C + 4*(s%4); destination lane d of the 16-lane group receives rows
//   K0..K0+3 of column C + d).  O^T keeps head l%32 in lane l, the same head
//   as the softmax statistics, so rescaling is lane-local.
// Softmax runs in base 2 with the scale folded in.  The 256 accumulators of a
// wave live in AGPRs and the main loop touches them only through the matrix
// cores (any VALU access there makes the compiler spill): each head keeps a
// fixed reference maximum (its first tile's maximum) and P = 2^(x - m_ref) may
// exceed 1 by up to 2^48 (fp32 and bf16 share the exponent range).  If a tile
// overshoots that headroom, the workgroup finishes the block, abandons the
// pass and restarts the split from its first block with the observed maxima
// as references (at most kPasses passes; then KVR_DEV_RANGE is raised and the
// last pass completes).  Splits write unnormalized partials (lane-native
// layout) that a combine kernel merges.
#include "kvr_device.h"
#include "kvr_internal.h"

#include "../../include/kvreloc.h"

namespace kvr {

__device__ uint32_t g_errors_decode;

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int kBlk = kDecBlockTokens;                    // tokens per KV block
constexpr int kCkvStride = 1024;                        // LDS bytes per cKV row (chunk-swizzled)
constexpr int kKrStride = 144;                          // LDS bytes per k_r row (128 + 16)
constexpr int kCkvBuf = kBlk * kCkvStride;
constexpr int kKrBuf = kBlk * kKrStride;
constexpr int kCsOff = 2 * kCkvBuf + 2 * kKrBuf;        // (cos, sin) per block and pair
constexpr int kBlkOff = kCsOff + kDecMaxBlocks * 32 * 8; // block ids of the split
constexpr int kFlagOff = kBlkOff + kDecMaxBlocks * 4;   // restart flag
constexpr int kSmem = kFlagOff + 16;
static_assert(kSmem <= 160 * 1024, "LDS budget");

// chunk permutation of a cKV row in LDS (row r mod 16 -> 0..15, one to one)
__device__ __forceinline__ uint32_t swz(int r) { return 4u * (r & 3) + ((r >> 2) & 3); }
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ void raise_error(uint32_t bit) {
    __hip_atomic_fetch_or(&g_errors_decode, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ v8bf as_bf(v4u x) { return __builtin_bit_cast(v8bf, x); }

typedef __attribute__((address_space(3))) v4u lds_v4u;

__device__ __forceinline__ v4u lds16(const char* p) { return *reinterpret_cast<const v4u*>(p); }

// reads at LDS byte offsets (the swizzled addresses are formed as integers)
__device__ __forceinline__ v4u lds16_at(uint32_t off) { return *(const lds_v4u*)(size_t)off; }
__device__ __forceinline__ v4s lds_tr_at(uint32_t off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(size_t)off);
}

// cKV rows of one block straight into LDS: one wave instruction per row
// (64 lanes x 16 bytes = the 1024-byte row).
__device__ __forceinline__ void stage_ckv(const DecodeArgs& A, int blk_id, char* dst, int wave, int n_waves,
                                          int lane) {
    const char* src = A.ckv + (int64_t)blk_id * A.ckv_b;
    for (int r = wave; r < kBlk; r += n_waves)
        __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)r * A.ckv_r + 16 * (lane ^ swz(r))),
                                         (void __attribute__((address_space(3)))*)(dst + r * kCkvStride), 16, 0, 0);
}

constexpr float kHeadroom = 48.f;      // log2 of the largest P before a restart
constexpr int kPasses = 3;

template <int NW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_kernel(const DecodeArgs A) {
    // the only LDS variable, so its 1024-byte alignment makes the cKV row
    // bases multiples of 1024 and the chunk swizzle a plain XOR of offsets
    __shared__ __attribute__((aligned(1024))) char smem[kSmem];
    char* ckv_s = smem;
    char* kr_s = smem + 2 * kCkvBuf;
    float2* cs_s = reinterpret_cast<float2*>(smem + kCsOff);
    int32_t* s_blk = reinterpret_cast<int32_t*>(smem + kBlkOff);
    int& s_overshoot = *reinterpret_cast<int*>(smem + kFlagOff);
    const uint32_t ckv_off = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)smem;

    const int tid = threadIdx.x, nthr = NW * 64;
    const int wave = tid >> 6, lane = tid & 63, n_waves = NW;
    const int n = lane & 31, half = lane >> 5;
    const int b = blockIdx.x / A.n_split, sp = blockIdx.x - b * A.n_split;
    const int head = wave * 32 + n;

    const int len = max(0, min(A.seq_lens[b], A.max_len));
    const int nblk_seq = (len + kBlk - 1) / kBlk;
    const int blk0 = sp * A.blocks_per_split;
    const int nb = max(0, min(A.blocks_per_split, nblk_seq - blk0));

    // ---- per-split tables: block ids and (cos, sin) of every pending shift --
    for (int e = tid; e < nb; e += nthr) {
        int id = A.bt[(int64_t)b * A.bt_stride + blk0 + e];
        if ((unsigned)id >= (unsigned)A.n_blocks) { raise_error(KVR_DEV_BAD_BLOCK); id = -1; }
        s_blk[e] = id;
    }
    for (int e = tid; e < nb * 32; e += nthr) {
        const int d = A.pend[(int64_t)b * A.bt_stride + blk0 + (e >> 5)];
        const double u = (double)d * A.omega[e & 31];
        float s, c;
        sincosf((float)((u - rint(u)) * 6.283185307179586476925), &s, &c);
        cs_s[e] = make_float2(c, s);
    }

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

    v16f acc[16];
    float m_run = kNegInf, l_run = 0.f;
    float m_hint = kNegInf;                 // references carried into a restarted pass

    __syncthreads();

    // k_r staging: item e < 256 is (token e/4, 16-byte chunk e%4) of the lo
    // half plus its partner chunk in the hi half; thread tid owns items
    // tid + k * nthr (k < 4).
    constexpr int KRI = (4 + NW - 1) / NW;
    auto load_kr = [&](int i, v4u* lo, v4u* hi) -> bool {
        const int id = s_blk[i];
        if (id < 0) return false;
#pragma unroll
        for (int k = 0; k < KRI; ++k) {
            const int e = tid + k * nthr;
            if (e < kBlk * 4) {
                const char* p = A.kr + (int64_t)id * A.kr_b + (int64_t)(e >> 2) * A.kr_r + (e & 3) * 16;
                lo[k] = *reinterpret_cast<const v4u*>(p);
                hi[k] = *reinterpret_cast<const v4u*>(p + 64);
            }
        }
        return true;
    };
    auto store_kr = [&](int i, v4u* lo, v4u* hi, char* dst) {
#pragma unroll
        for (int k = 0; k < KRI; ++k) {
            const int e = tid + k * nthr;
            if (e < kBlk * 4) {
                rot_bf16x8(lo[k], hi[k], cs_s + i * 32 + (e & 3) * 8);
                char* p = dst + (e >> 2) * kKrStride + (e & 3) * 16;
                *reinterpret_cast<v4u*>(p) = lo[k];
                *reinterpret_cast<v4u*>(p + 64) = hi[k];
            }
        }
    };

    for (int pass = 0; pass < kPasses; ++pass) {
#pragma unroll
    for (int f = 0; f < 16; ++f) acc[f] = v16f{};
    m_run = m_hint;
    l_run = 0.f;
    if (tid == 0) s_overshoot = 0;
    if (nb > 0) {
        v4u lo[KRI], hi[KRI];
        if (s_blk[0] >= 0) stage_ckv(A, s_blk[0], ckv_s, wave, n_waves, lane);
        if (load_kr(0, lo, hi)) store_kr(0, lo, hi, kr_s);
    }
    wait_loads();
    __syncthreads();
    const bool last_pass = pass + 1 == kPasses;
    bool restart = false;

    for (int i = 0; i < nb; ++i) {
        const int cur = i & 1;
        const uint32_t ck = ckv_off + cur * kCkvBuf;
        const char* kq = kr_s + cur * kKrBuf;
        v4u nlo[KRI], nhi[KRI];
        bool nkr = false;
        if (i + 1 < nb) {
            if (s_blk[i + 1] >= 0) stage_ckv(A, s_blk[i + 1], ckv_s + (cur ^ 1) * kCkvBuf, wave, n_waves, lane);
            nkr = load_kr(i + 1, nlo, nhi);
        }
        const bool valid = s_blk[i] >= 0;
        const int tok_base = (blk0 + i) * kBlk;

#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            const int t0 = tile * 32;
            // S^T tile: rows = 32 tokens, columns = 32 heads
            v16f sacc = v16f{};
            // chunk 2s + half of row t0 + n sits at position (2s) ^ (half ^ swz(n))
            const uint32_t krow = ck + (t0 + n) * kCkvStride + 16 * (half ^ swz(n));
            const char* rrow = kq + (t0 + n) * kKrStride + 16 * half;
            // K-row operands stream from LDS through a 4-deep window so the
            // matrix core never waits for a read it could have issued earlier
            auto kop = [&](int s) {
                return s < 32 ? lds16_at((krow ^ (32u * (s & 7))) + 256u * (s >> 3)) : lds16(rrow + 32 * (s - 32));
            };
            v4u kw[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) kw[s] = kop(s);
#pragma unroll
            for (int s = 0; s < 36; ++s) {
                const v4u cur = kw[s & 3];
                if (s + 4 < 36) kw[s & 3] = kop(s + 4);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(cur), q[s], sacc, 0, 0, 0);
            }

            // scores (base 2), masking, tile maximum over the head's 32 tokens
            float x[16];
            float mt = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int t = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
                x[r] = (valid && tok_base + t < len) ? sacc[r] * A.scale_log2 : kNegInf;
                mt = fmaxf(mt, x[r]);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            // first valid tile of a head fixes its reference; an overshoot
            // beyond the headroom abandons this pass (decided per workgroup
            // at the end of the block)
            if (m_run == kNegInf) m_run = mt;
            if (mt > m_run + kHeadroom) {
                m_hint = fmaxf(m_hint, mt);
                if (!last_pass) s_overshoot = 1;
                else raise_error(KVR_DEV_RANGE);
            }
            m_hint = fmaxf(m_hint, m_run);
            // P in bf16 (also summed in bf16 so numerator and denominator agree)
            v8bf pb[2];
            float ls = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = (m_run == kNegInf) ? 0.f : exp2f(x[r] - m_run);
                const __bf16 pr = (__bf16)p;
                pb[r >> 3][r & 7] = pr;
                ls += (float)pr;
            }
            ls += __shfl_xor(ls, 32);
            l_run += ls;

            // O^T += V^T P^T over two 16-token steps; transpose reads run
            // 4 feature tiles ahead of the matrix core
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                // this lane's 8 bytes of feature tile f (64 bytes per row)
                // start at byte 64f + 16cl + 8(sl&1) of rows ka and ka + 8
                const int sl = lane & 15;
                const int ka = t0 + 16 * s + 4 * half + (sl >> 2);
                const uint32_t cl = 2 * ((lane >> 4) & 1) + ((sl & 3) >> 1);
                const uint32_t ra = ck + ka * kCkvStride + 16 * (cl ^ swz(ka)) + 8 * (sl & 1);
                const uint32_t rb = ck + (ka + 8) * kCkvStride + 16 * (cl ^ swz(ka + 8)) + 8 * (sl & 1);
                auto tr = [&](uint32_t base, int f) { return lds_tr_at((base ^ (64u * (f & 3))) + 256u * (f >> 2)); };
                v4s wa[4], wb[4];
#pragma unroll
                for (int f = 0; f < 4; ++f) { wa[f] = tr(ra, f); wb[f] = tr(rb, f); }
#pragma unroll
                for (int f = 0; f < 16; ++f) {
                    const v4s ta = wa[f & 3], tb = wb[f & 3];
                    if (f + 4 < 16) { wa[f & 3] = tr(ra, f + 4); wb[f & 3] = tr(rb, f + 4); }
                    const v8bf va = __builtin_bit_cast(v8bf, __builtin_shufflevector(ta, tb, 0, 1, 2, 3, 4, 5, 6, 7));
                    acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[s], acc[f], 0, 0, 0);
                }
            }
        }

        if (nkr) store_kr(i + 1, nlo, nhi, kr_s + (cur ^ 1) * kKrBuf);
        wait_loads();
        __syncthreads();
        if (s_overshoot) { restart = true; break; }
    }
    if (!restart) break;
    __syncthreads();                        // everyone has read the flag before it is cleared
    }

    // ---- unnormalized partials in the lane-native layout ---------------------
    float* po = A.part_o + (((int64_t)b * A.n_split + sp) * n_waves + wave) * (16 * 16 * 64);
#pragma unroll
    for (int f = 0; f < 16; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) po[(f * 16 + r) * 64 + lane] = acc[f][r];
    if (half == 0) {
        float2* pm = reinterpret_cast<float2*>(A.part_ml) + ((int64_t)b * A.n_split + sp) * A.heads + head;
        *pm = make_float2(m_run, l_run);
    }
}

// Merge the splits of one (sequence, head group): O = sum_s 2^(m_s - M) O_s / L,
// L = sum_s 2^(m_s - M) l_s, LSE = ln 2 * (M + log2 L).  One thread per
// (lane-native position) of a wave's 32 heads x 512 features.
__global__ __launch_bounds__(256) void mla_decode_combine(const DecodeArgs A, uint16_t* out, float* lse) {
    const int n_waves = A.heads / 32;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;     // over b, wave, f, r, lane
    const int64_t per_b = (int64_t)n_waves * 16 * 16 * 64;
    if (idx >= (int64_t)gridDim.x * 256 || idx >= per_b * A.batch) return;
    const int b = (int)(idx / per_b);
    int64_t rem = idx - b * per_b;
    const int wave = (int)(rem / (16 * 16 * 64));
    rem -= (int64_t)wave * (16 * 16 * 64);
    const int f = (int)(rem / (16 * 64));
    const int r = (int)((rem / 64) % 16);
    const int lane = (int)(rem % 64);
    const int head = wave * 32 + (lane & 31);
    const int feat = 32 * f + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);

    const float2* pm = reinterpret_cast<const float2*>(A.part_ml);
    float M = kNegInf;
    for (int s = 0; s < A.n_split; ++s) M = fmaxf(M, pm[((int64_t)b * A.n_split + s) * A.heads + head].x);
    float L = 0.f, o = 0.f;
    if (M != kNegInf) {
        for (int s = 0; s < A.n_split; ++s) {
            const float2 ml = pm[((int64_t)b * A.n_split + s) * A.heads + head];
            if (ml.x == kNegInf) continue;
            const float w = exp2f(ml.x - M);
            L += w * ml.y;
            o += w * A.part_o[(((int64_t)b * A.n_split + s) * n_waves + wave) * (16 * 16 * 64) + rem];
        }
    }
    const float v = L > 0.f ? o / L : 0.f;
    out[((int64_t)b * A.heads + head) * 512 + feat] = __builtin_bit_cast(uint16_t, (__bf16)v);
    if (f == 0 && r == 0 && (lane >> 5) == 0)
        lse[(int64_t)b * A.heads + head] = L > 0.f ? 0.6931471805599453f * (M + log2f(L)) : kNegInf;
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
    const int64_t total = (int64_t)a.batch * (a.heads / 32) * 16 * 16 * 64;
    hipLaunchKernelGGL(mla_decode_combine, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, out, lse);
    return hipGetLastError();
}

uint32_t read_and_clear_errors_decode() {
    uint32_t v = 0, z = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_errors_decode), sizeof(v)) != hipSuccess) return 0xffffffffu;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_errors_decode), &z, sizeof(z)) != hipSuccess) return 0xffffffffu;
    return v;
}

}  // namespace kvr
