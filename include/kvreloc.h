/*
 * kvreloc.h -- C ABI of the KV-relocation library (HIP, gfx950 / MI355X).
 *
 * The library relocates cached KV rows to new absolute positions without a
 * re-prefill.  For every moved token row the position-free part (the MLA cKV
 * latent, or V in GQA) is copied bit for bit, and the rotary key part (MLA
 * k_rope, or the whole GQA K) is re-rotated in closed form, K <- R(delta) K,
 * using the RoPE closure R(a) R(b) = R(a + b).
 *
 * Sources (technical summaries on gist.science):
 *   Leyline  -- "Leyline : Directives de Cache KV pour l'Inference Agentique"
 *               (directive D = (s_start, s_end, R, m), AMORTIZE / FORGET,
 *               delta-rotation of the downstream K_pe band: sections 2.1-2.3).
 *   Irminsul -- "Irminsul: Cache Independente de Posicao Nativo para MLA ..."
 *               (registry entry (cKV, k_r, base_pos), delta = p_target -
 *               p_source, rotation fused into MLA attention: sections 2.1-2.2).
 *   Kamera   -- "Kamera : Un KV Cache Multimodal Unifie et Invariant a la
 *               Position ..." (reuse operator R(delta) KV + U_m V_m^T, GQA
 *               re-rotates all of K and patches K and V: section 2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Device pointers are caller-owned (typically PyTorch allocations).  The
 *   library allocates and frees no device memory in these calls; scratch
 *   memory comes in through a caller-provided workspace.
 * - Host arrays are read before the call returns; they need not outlive it.
 * - Every call validates all arguments on the host first.  A validation error
 *   returns before anything is enqueued, so device memory is untouched (no
 *   partial edits).  On success the work is enqueued on `stream` and the call
 *   returns without synchronizing.
 * - Kernels bounds-check every block-table entry against the pool
 *   (0 <= id < n_blocks).  A bad entry is never dereferenced: the affected
 *   rows are skipped and a bit is set in the device error word, read (and
 *   cleared) with kvr_device_errors().
 * - Debug checks (environment variable KVR_DEBUG_CHECKS=1): leyline_splice
 *   and kv_relocate_gather first copy the block tables to the host, waiting
 *   for `stream`.  They return KVR_E_OVERLAP if a block the call would write
 *   is named by more than one logical block of the call's sequences (a
 *   splice's sequence holds its first max(N, new_len) slots), and
 *   KVR_E_RANGE for such a block id outside the pool, before enqueuing
 *   anything.  Off by default: the copy synchronizes the stream.
 * - RoPE (the reading taken here; the pages give no formula): within each
 *   head of rotary dimension d, pairs (x_j, x_{j+d/2}), j < d/2, rotate by
 *   phi = p * theta_j with theta_j = base^(-2j/d) (or the caller's inv_freq):
 *   y_j = x_j cos(phi) - x_{j+d/2} sin(phi), y_{j+d/2} = x_j sin(phi) +
 *   x_{j+d/2} cos(phi).  phi is formed and reduced in float64; the rotation
 *   itself runs in float32 and bf16 results are rounded to nearest even.
 *   A shift of 0 is the identity: rows are copied bit for bit.
 * - Paged layout: logical slot s of a sequence lives in physical row
 *   (bt[s / block_size], s % block_size) of the pool; a contiguous cache is
 *   a pool of one block (block_size = capacity) with block table {0}.
 */
#ifndef KVRELOC_H
#define KVRELOC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVR_ABI_VERSION 1

typedef int32_t kvr_status;
#define KVR_OK                    0
#define KVR_FORGET_NEEDS_PREFILL  1   /* informational: a FORGET directive was seen */
#define KVR_E_ARG                (-1) /* null/misaligned pointer, bad dtype, shape or stride */
#define KVR_E_RANGE              (-2) /* a position or length outside its sequence */
#define KVR_E_CAPACITY           (-3) /* result does not fit the block table */
#define KVR_E_OVERLAP            (-4) /* gather targets overlap each other */
#define KVR_E_HIP                (-5) /* HIP runtime/launch error: kvr_last_hip_error() */
#define KVR_E_WORKSPACE          (-6) /* workspace missing, misaligned or too small */
#define KVR_E_UNSUPPORTED        (-7) /* valid request this build does not implement */
#define KVR_E_SCRATCH            (-8) /* leyline_splice_noalloc: call needs more than its scratch */

/* Device error word bits (kvr_device_errors). */
#define KVR_DEV_BAD_BLOCK   1u  /* a block-table entry was outside [0, n_blocks) */
#define KVR_DEV_SPIN_LIMIT  2u  /* a splice ordering wait hit its bound (workspace misuse) */
#define KVR_DEV_BAD_TICKET  4u  /* a splice ticket was out of range (workspace not zeroed) */
#define KVR_DEV_RANGE       8u  /* decode: scores kept outgrowing the softmax headroom (2^48);
                                    lazy splice: a shift left int32; keying: chunk list overflow */
#define KVR_DEV_BAD_TOKEN  16u  /* keying: a token id outside [0, vocab) */

/* Directive modes m (Leyline 2.1). */
#define KVR_AMORTIZE 0
#define KVR_FORGET   1

/* Element types. */
#define KVR_BF16 0
#define KVR_F32  1

/* One part (position-free or rotary) of a paged KV pool.  Element
 * [layer][block][row][col] is at base + layer*layer_stride +
 * block*block_stride + row*row_stride + col (strides in elements).  base and
 * every row start must be 16-byte aligned. */
typedef struct kvr_part {
    void*   base;
    int64_t layer_stride;
    int64_t block_stride;
    int64_t row_stride;
} kvr_part;

/* A paged KV cache: the position-free part is moved as raw words, the rotary
 * part is rotated.  MLA (Irminsul 2.1): pf = cKV, pf_width 512; rope = k_r,
 * rope_heads 1, rope_dim 64.  GQA (Kamera 2): pf = V, pf_width heads*dim;
 * rope = K, rope_heads = KV heads, rope_dim = head dim.
 * Requirements: pf_width * sizeof(pf word) a multiple of 16 bytes;
 * rope_dim even, (rope_dim/2) * sizeof(rope elt) a multiple of 16 bytes;
 * rope_heads * rope_dim <= 4096. */
typedef struct kvr_cache {
    int32_t  n_layers;
    int32_t  block_size;     /* rows per block, >= 1 */
    int32_t  n_blocks;       /* physical blocks per layer (valid block ids) */
    int32_t  pf_width;       /* elements of the position-free part per row */
    int32_t  pf_dtype;       /* KVR_BF16 (2-byte words) or KVR_F32 (4-byte words) */
    int32_t  rope_heads;
    int32_t  rope_dim;       /* rotary dimension per head */
    int32_t  rope_dtype;     /* KVR_BF16 or KVR_F32 */
    double   rope_base;      /* theta_j = rope_base^(-2j/rope_dim) */
    const double* inv_freq;  /* host, optional: rope_dim/2 entries overriding theta_j */
    kvr_part pf;
    kvr_part rope;
} kvr_cache;

/* Directive D = (s_start, s_end, R, m) of Leyline 2.1: replace the half-open
 * token range [s_start, s_end) by r_len = |R| replacement tokens. */
typedef struct kvr_directive {
    int64_t s_start;
    int64_t s_end;
    int64_t r_len;
    int32_t mode;            /* KVR_AMORTIZE or KVR_FORGET */
    int32_t reserved;
} kvr_directive;

/* Token rows outside the pool, for every layer: row t of layer l is at
 * pf + l*pf_layer_stride + t*pf_row_stride (elements, same dtypes and widths
 * as the cache parts).  Used for a registry entry (cKV, k_r, base_pos) of
 * Irminsul 2.2, whose rotary part was computed at absolute positions
 * base_pos + t, and for a splice stub (already-prefilled replacement rows,
 * Leyline 2.3; base_pos ignored).  Must not alias rows the call writes. */
typedef struct kvr_rows {
    const void* pf;
    int64_t     pf_layer_stride;
    int64_t     pf_row_stride;
    const void* rope;
    int64_t     rope_layer_stride;
    int64_t     rope_row_stride;
    int64_t     len;
    int64_t     base_pos;
} kvr_rows;

/* Rank-m factors of Kamera's conditioning patch U_m V_m^T for one chunk and
 * every layer, float32: U[l][t][k] at U + l*u_layer_stride + t*rank + k,
 * V[l][f][k] at V + l*v_layer_stride + f*rank + k.  The patch of element
 * (t, f) is sum_k U[t][k] V[f][k]; f is the flattened feature index
 * (head*head_dim + dim).  rank 0 means "no patch". */
typedef struct kvr_lowrank {
    const float* U;
    int64_t      u_layer_stride;
    const float* V;
    int64_t      v_layer_stride;
    int32_t      rank;       /* 0, or a multiple of 4 up to 64 (else KVR_E_ARG) */
    int32_t      reserved;
} kvr_lowrank;

/* Content-defined chunking parameters (registry_chunk_keys). */
typedef struct kvr_cdc_params {
    uint64_t threshold;  /* a candidate boundary follows token i when its Gear hash < threshold */
    int32_t  min_len;    /* chunk length bounds in tokens, 1 <= min_len <= max_len */
    int32_t  max_len;
    int32_t  s1_window;  /* S1 fallback window in tokens (>= 1) */
    int32_t  reserved;
    uint64_t seed;       /* xxHash64 seed */
} kvr_cdc_params;

/* ------------------------------------------------------------------------
 * leyline_splice -- in-place AMORTIZE splice of n_seq sequences (Leyline
 * 2.1-2.3).  For sequence b of current length N = seq_lens[b] and directive
 * dirs[b]: Delta = r_len - (s_end - s_start); old slots [s_end, N) move to
 * [s_end + Delta, N + Delta) in every layer, their position-free part copied
 * bit for bit and their rotary part rotated by R(Delta); then the stub rows
 * stubs[b] (if stubs != NULL and stubs[b].pf != NULL) are copied, unrotated,
 * into [s_start, s_start + r_len).  The prefix [0, s_start) is untouched.
 * new_lens[b] = N + Delta.  Rows in [N + Delta, N) after a shrink are left
 * as they are ("don't care").
 * FORGET directives move nothing: new_lens[b] = s_start and the call returns
 * KVR_FORGET_NEEDS_PREFILL (after enqueuing the AMORTIZE sequences of the
 * same batch); the caller re-prefills from there.
 *
 *   d_block_tables : device int32 [n_seq][bt_stride]; capacity of each
 *                    sequence = bt_stride * block_size slots.  The blocks a
 *                    splice writes must belong to that sequence only.
 *   seq_lens, dirs : host [n_seq]
 *   stubs          : host [n_seq] or NULL; stubs[b].len must equal r_len
 *   new_lens       : host out [n_seq]
 *   d_workspace    : device, kvr_splice_workspace_bytes() bytes, 256-byte
 *                    aligned, zero-filled before its first use (every call
 *                    leaves it zero-filled).  Calls sharing a workspace must
 *                    be ordered on one stream.
 * Errors: KVR_E_ARG, KVR_E_RANGE (0 <= s_start <= s_end <= N <= capacity
 * violated, r_len < 0), KVR_E_CAPACITY (N + Delta > capacity),
 * KVR_E_WORKSPACE, KVR_E_HIP.
 * ---------------------------------------------------------------------- */
size_t kvr_splice_workspace_bytes(const kvr_cache* cache, int32_t n_seq,
                                  const int64_t* seq_lens, const kvr_directive* dirs);

kvr_status leyline_splice(const kvr_cache* cache, const int32_t* d_block_tables,
                          int32_t bt_stride, int32_t n_seq, const int64_t* seq_lens,
                          const kvr_directive* dirs, const kvr_rows* stubs,
                          int64_t* new_lens, void* d_workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * leyline_splice_noalloc -- leyline_splice for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same splices, arguments and results, with no
 * workspace argument.  The ticketed mover's counters and flags live in a
 * device array of the library, kvr_noalloc_scratch_bytes() bytes (8 MiB:
 * ~2M workgroups per launch, e.g. 64 sequences x 32K slots x 61 layers) that
 * each GPU the library runs on holds until the process ends.  The call
 * allocates nothing: it clears the part of the array it uses with a kernel
 * and launches as leyline_splice does.  Every call on one GPU shares that
 * GPU's array, so calls that overlap on one GPU (different streams, other
 * host threads) race and must be ordered by the caller.
 * Errors: as leyline_splice, and KVR_E_SCRATCH when the call needs more than
 * the array holds.
 * ---------------------------------------------------------------------- */
kvr_status leyline_splice_noalloc(const kvr_cache* cache, const int32_t* d_block_tables,
                                  int32_t bt_stride, int32_t n_seq, const int64_t* seq_lens,
                                  const kvr_directive* dirs, const kvr_rows* stubs,
                                  int64_t* new_lens, hipStream_t stream);
size_t     kvr_noalloc_scratch_bytes(void);

/* ------------------------------------------------------------------------
 * kv_relocate_gather -- copy n registry entries into one paged destination
 * sequence (Irminsul 2.2; Kamera 2).  Entry i's row t lands on logical slot
 * p_target[i] + t of every layer: position-free part bit for bit, rotary
 * part rotated by delta_i = p_target[i] - entries[i].base_pos.  With
 * patch_rope / patch_pf (host arrays [n], or NULL) the rank-m patch of
 * Kamera's operator is added after the rotation, before rounding:
 * K_out = R(delta) K + U V^T, V_out = V + U' V'^T.
 *
 *   d_block_table : device int32 [bt_len]; capacity = bt_len * block_size
 *   entries, p_target : host [n]
 * Errors: KVR_E_ARG, KVR_E_RANGE (p_target < 0 or p_target + len beyond
 * capacity, len < 0), KVR_E_OVERLAP (two targets share a slot), KVR_E_HIP.
 * ---------------------------------------------------------------------- */
kvr_status kv_relocate_gather(const kvr_cache* dst, const int32_t* d_block_table,
                              int32_t bt_len, const kvr_rows* entries,
                              const int64_t* p_target, int32_t n,
                              const kvr_lowrank* patch_rope, const kvr_lowrank* patch_pf,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * kv_patch_lowrank -- add Kamera's rank-m patch in place to rows already in
 * the cache (Kamera 2): for item i, logical slots [p_start[i], p_start[i] +
 * len[i]) of every layer, X += U_i V_i^T on the chosen part (0 = position-
 * free, 1 = rotary), computed in float32 and rounded once.  No rotation.
 *   d_block_table : device int32 [bt_len]
 *   p_start, len, f : host [n]; f[i].U rows correspond to the len[i] slots
 * Errors: KVR_E_ARG, KVR_E_RANGE, KVR_E_OVERLAP, KVR_E_HIP.
 * ---------------------------------------------------------------------- */
kvr_status kv_patch_lowrank(const kvr_cache* cache, const int32_t* d_block_table,
                            int32_t bt_len, int32_t part, const int64_t* p_start,
                            const int64_t* len, const kvr_lowrank* f, int32_t n,
                            hipStream_t stream);

/* ------------------------------------------------------------------------
 * mla_decode_rotate_on_read -- one decode step of absorbed-form MLA attention
 * over a paged cache whose blocks carry a pending rotary shift (Irminsul 2.2
 * and 4: the delta-rotation is fused into attention on the load path; 5: the
 * absorbed-matmul form).  For sequence b and head h:
 *   s_t = scale * (q_nope[b][h] . cKV_t + q_rope[b][h] . (R(delta_blk(t)) k_r_t))
 *   out[b][h] = sum_t softmax(s)_t cKV_t,   lse[b][h] = ln sum_t exp(s_t)
 * over t < seq_lens[b]; delta_blk(t) = d_pending_delta[b][t / block_size].
 * The rotated key is formed in registers and never written back.
 *   cache          : MLA layout (pf_width 512 bf16, rope 1 x 64 bf16)
 *   q_nope, q_rope : device bf16 [batch][heads][512], [batch][heads][64]
 *   d_block_tables, d_pending_delta : device int32 [batch][bt_stride]
 *   d_seq_lens     : device int32 [batch]; max_seq_len (host) bounds them
 *   out            : device bf16 [batch][heads][512]; lse : device f32 [batch][heads]
 *   d_workspace    : kvr_decode_workspace_bytes() bytes, 256-byte aligned
 * heads must be 32, 64, 96 or 128; the cache's block_size must be 64.
 * Errors: KVR_E_ARG, KVR_E_RANGE, KVR_E_WORKSPACE, KVR_E_UNSUPPORTED, KVR_E_HIP.
 * ---------------------------------------------------------------------- */
size_t kvr_decode_workspace_bytes(int32_t batch, int32_t heads, int32_t max_seq_len);

kvr_status mla_decode_rotate_on_read(const void* q_nope, const void* q_rope,
                                     int32_t batch, int32_t heads,
                                     const kvr_cache* cache, int32_t layer,
                                     const int32_t* d_block_tables,
                                     const int32_t* d_pending_delta, int32_t bt_stride,
                                     const int32_t* d_seq_lens, int32_t max_seq_len,
                                     float scale, void* out, float* lse,
                                     void* d_workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * gqa_decode_rotate_on_read -- one decode step of GQA attention over a paged
 * cache whose blocks carry a pending rotary shift (Kamera, section 2: in GQA
 * all of K is rotary and is re-rotated, V is position-free; Irminsul,
 * sections 2.2 and 4: the shift is applied inside attention, on the load
 * path, and never written back).  For sequence b and query head h, with G =
 * cache->rope_heads KV heads and g = h / (q_heads / G):
 *   s_t = scale * q[b][h] . (R(delta_blk(t)) K_t[g])
 *   out[b][h] = sum_t softmax(s)_t V_t[g],   lse[b][h] = ln sum_t exp(s_t)
 * over t < seq_lens[b]; delta_blk(t) = d_pending_delta[b][t / block_size].
 * The kernel applies R(-delta) to the query once per block (the same scores,
 * R being orthogonal) and keeps the rotated query to about 16 bits.
 *   q              : device bf16 [batch][q_heads][128], 16-byte aligned
 *   cache          : GQA layout: rope = K with rope_heads = G and rope_dim 128,
 *                    pf = V with pf_width = G * 128, both bf16; block_size 64
 *   q_heads        : a multiple of G, at most 16 query heads per KV head
 *   d_block_tables, d_pending_delta : device int32 [batch][bt_stride]
 *   d_seq_lens     : device int32 [batch]; max_seq_len (host) bounds them
 *   out            : device bf16 [batch][q_heads][128]; lse : device f32 [batch][q_heads]
 *                    (a sequence of length 0 gives out 0 and lse -inf)
 *   d_workspace    : kvr_gqa_decode_workspace_bytes() bytes, 256-byte aligned
 * Device errors: KVR_DEV_BAD_BLOCK for a block id outside [0, n_blocks) (its
 * tokens are skipped).
 * Errors: KVR_E_ARG, KVR_E_RANGE (layer, max_seq_len past the table),
 * KVR_E_WORKSPACE, KVR_E_UNSUPPORTED (other layouts, dtypes, head counts,
 * row strides above 16 MiB), KVR_E_HIP.
 * ---------------------------------------------------------------------- */
size_t kvr_gqa_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t max_seq_len);

kvr_status gqa_decode_rotate_on_read(const void* q, int32_t batch, int32_t q_heads,
                                     const kvr_cache* cache, int32_t layer,
                                     const int32_t* d_block_tables,
                                     const int32_t* d_pending_delta, int32_t bt_stride,
                                     const int32_t* d_seq_lens, int32_t max_seq_len,
                                     float scale, void* out, float* lse,
                                     void* d_workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * kamera_patch_factors -- Kamera's patch formation (section 2: the m
 * leading SVD factors of the conditioning deficit
 * Delta = KV(B|A) - KV(B|empty); section 3: the orbit patch, from the deficit
 * averaged over the sampled orders of a cached set).  For every deficit b:
 *   D_b = mean over the `orders` matrices of b (orders = 1: the matrix itself)
 *   U_b [rows x rank] = U_m Sigma_m,  V_b [cols x rank] = V_m,  sigma_b [rank]
 * so that U_b V_b^T is the best rank-m approximation of D_b: the factors the
 * reuse operator adds (kvr_lowrank layout U[t][k], V[f][k]).  Computed by a
 * randomized range finder with a 32-column sketch and two power steps in
 * float32 (accurate when sigma_33 << sigma_m).
 *   d_deficits : device float32 [n][orders][rows][cols], 16-byte aligned
 *   d_omega    : device float32 [cols][32], the range finder's random test
 *                matrix (caller-drawn, e.g. N(0,1))
 *   rows, cols : multiples of 64 in 64..16384;  rank : 1..16
 *   d_U, d_V, d_sigma : device float32 outputs as above
 *   d_workspace: kvr_patch_factors_workspace_bytes() bytes, 256-byte aligned
 * Errors: KVR_E_ARG (null or misaligned pointer, n < 0, orders < 1),
 * KVR_E_UNSUPPORTED (shapes, rank), KVR_E_RANGE, KVR_E_WORKSPACE, KVR_E_HIP.
 * ---------------------------------------------------------------------- */
size_t kvr_patch_factors_workspace_bytes(int32_t n, int32_t orders, int32_t rows, int32_t cols);

kvr_status kamera_patch_factors(const float* d_deficits, int32_t n, int32_t orders, int32_t rows, int32_t cols,
                                int32_t rank, const float* d_omega, float* d_U, float* d_V, float* d_sigma,
                                void* d_workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * leyline_splice_lazy -- a block-aligned AMORTIZE splice done as an edit of
 * the block table and of the per-block pending shifts; no KV byte moves.
 * (Leyline, sections 2.2-2.3: the downstream slots are re-indexed and owe
 * R(Delta); rotations compose, so Delta is added to each moved block's
 * pending shift and applied once, on read, by mla_decode_rotate_on_read --
 * Irminsul, sections 2.2 and 4.)  Repeated splices then round the keys once
 * instead of once per splice.
 *
 * Per sequence b with directive (s_start, s_end, r_len, mode), B = block_size,
 * Delta = r_len - (s_end - s_start), all of s_start, s_end, r_len multiples
 * of B, N = seq_lens[b]:
 *   - logical blocks below s_start/B keep their entries;
 *   - blocks s_start/B .. s_start/B + r_len/B - 1 take the next r_len/B ids
 *     of d_stub_blocks (blocks the caller has prefilled with R at its final
 *     positions) with pending shift 0;
 *   - blocks up to ceil((N + Delta)/B) - 1 take the entry of old block
 *     k - Delta/B, its pending shift increased by Delta;
 *   - entries from ceil((N + Delta)/B) up to ceil(N/B) - 1 become -1 with
 *     shift 0; entries past both counts are left alone;
 *   - the ids of old blocks s_start/B .. s_end/B - 1 are written to
 *     d_freed_blocks, sequences concatenated in order; the caller owns them.
 * FORGET changes nothing: KVR_FORGET_NEEDS_PREFILL, new_lens[b] = s_start.
 *   block_size      : slots per block, > 0
 *   d_block_tables  : device int32 [n_seq][bt_stride], edited in place
 *   d_pending_delta : device int32 [n_seq][bt_stride], edited in place
 *   bt_stride       : 1 .. 8192 blocks; capacity = bt_stride * block_size
 *   seq_lens, dirs  : host [n_seq]
 *   d_stub_blocks   : device int32 [sum of r_len/B]; NULL when that sum is 0
 *   d_freed_blocks  : device int32 out [sum of (s_end - s_start)/B]; NULL when 0
 *   new_lens        : host out [n_seq]
 * A shift that would leave the int32 range raises KVR_DEV_RANGE (see
 * kvr_device_errors) and that entry keeps its unshifted value.
 * Errors: KVR_E_ARG (null pointer, block_size <= 0, bt_stride outside
 * 1..8192, a range not on block boundaries, unknown mode), KVR_E_RANGE
 * (0 <= s_start <= s_end <= N <= capacity violated, r_len < 0),
 * KVR_E_CAPACITY (N + Delta > capacity), KVR_E_HIP.  Nothing is enqueued
 * unless every sequence validates.
 * ---------------------------------------------------------------------- */
kvr_status leyline_splice_lazy(int32_t block_size, int32_t* d_block_tables, int32_t* d_pending_delta,
                               int32_t bt_stride, int32_t n_seq, const int64_t* seq_lens,
                               const kvr_directive* dirs, const int32_t* d_stub_blocks,
                               int32_t* d_freed_blocks, int64_t* new_lens, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kv_relocate_gather_lazy -- registry entries placed by reference.  A
 * registry hit reuses a chunk's KV at a new position and owes
 * R(p_target - p_source) (Irminsul, section 2.2); when the entry is kept in
 * pool blocks from row 0 of its first block and p_target is a multiple of
 * the block size, the placement is an edit of the destination's block table
 * and per-block pending shifts, and mla_decode_rotate_on_read applies the
 * shift on read (Irminsul, sections 2.2 and 4).  No KV byte moves.
 *
 * For entry e, B = block_size, nb = ceil(len / B), k < nb, slot =
 * p_target / B + k in row `seq` of the tables:
 *   d_replaced[off_e + k] = the old d_block_tables[seq][slot]   (off_e = the
 *                           nb of the earlier entries, summed; skipped when
 *                           d_replaced is NULL)
 *   d_block_tables[seq][slot]  = d_blocks[k]
 *   d_pending_delta[seq][slot] = (d_pend ? d_pend[k] : 0) + p_target - base_pos
 * The entry's blocks are then shared by the registry and the sequence; the
 * replaced ids pass to the caller.  Rows of a ragged last block past len
 * are the entry block's own rows, so an entry whose len is not a multiple of
 * B must be the last thing in its sequence up to that block's end.
 *   block_size      : slots per block, > 0
 *   d_block_tables,
 *   d_pending_delta : device int32 [n_seq][bt_stride], edited in place
 *   bt_stride       : 1 .. 8192 blocks; capacity = bt_stride * block_size
 *   entries         : host [n]; d_blocks and d_pend are device int32 [nb]
 *   d_replaced      : device int32 out [sum of nb], or NULL
 * A pending shift that would leave the int32 range raises KVR_DEV_RANGE (see
 * kvr_device_errors) and that slot keeps the entry block's own shift.
 * Errors: KVR_E_ARG (null tables, entries or d_blocks where needed,
 * block_size <= 0, bt_stride outside 1..8192, n < 0, seq outside
 * 0..n_seq-1, p_target not a multiple of B), KVR_E_RANGE (len < 0,
 * p_target < 0, p_target + len > capacity, |p_target - base_pos| >= 2^31),
 * KVR_E_OVERLAP (two entries of one sequence covering one logical block),
 * KVR_E_HIP.  Nothing is enqueued unless every entry validates.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t seq;                /* row of the block and shift tables */
    const int32_t* d_blocks;    /* device int32 [nb]: pool blocks holding the entry, in order */
    const int32_t* d_pend;      /* device int32 [nb]: shifts those blocks already owe, or NULL for 0 */
    int64_t len, base_pos, p_target;
} kvr_lazy_entry;

kvr_status kv_relocate_gather_lazy(int32_t block_size, int32_t* d_block_tables, int32_t* d_pending_delta,
                                   int32_t bt_stride, int32_t n_seq, const kvr_lazy_entry* entries, int32_t n,
                                   int32_t* d_replaced, hipStream_t stream);

/* ------------------------------------------------------------------------
 * registry_chunk_keys -- registry keying of token streams (Irminsul, section
 * 2.2): content-defined chunks cut by a Gear rolling hash over 64-token
 * windows, each fingerprinted with xxHash64, plus the S1 fallback's fixed
 * windows inside every chunk.
 *
 * Per stream s = tokens [offsets[s], offsets[s+1]) of d_tokens:
 *   h_i = (2 h_{i-1} + gear[tok_i]) mod 2^64, h = 0 before the stream start
 *         (= sum over the last 64 tokens of gear[tok] * 2^age);
 *   the chunk starting at p ends after the first i in
 *   [p + min_len - 1, p + max_len - 1] with h_i < threshold, else after
 *   p + max_len - 1; the last chunk ends at the stream end;
 *   fingerprint = xxHash64(token ids as little-endian int32 bytes, seed);
 *   S1 window w of a chunk [a, b) = [a + w s1, min(a + (w+1) s1, b)).
 *   d_tokens     : device int32 [offsets[n_streams]]
 *   offsets      : host int64 [n_streams + 1], non-decreasing, offsets[0] >= 0;
 *                  each stream shorter than 2^31 tokens
 *   n_streams    : 0 .. 240
 *   d_gear       : device uint64 [vocab] (the Gear table, caller-drawn)
 *   d_hash       : device uint64 out [total] (h_i per token) or NULL
 *   d_chunk_end  : device int32 out [n_streams][chunk_cap]: chunk ends
 *                  relative to the stream start, in order
 *   chunk_cap    : >= ceil(len / min_len) for every stream
 *   d_n_chunks   : device int32 out [n_streams]
 *   d_chunk_fp   : device uint64 out [n_streams][chunk_cap]
 *   d_s1_fp      : device uint64 out [n_streams][chunk_cap][ceil(max_len / s1_window)]
 *                  (a chunk's unused windows 0) or NULL
 *   Entries of d_chunk_end, d_chunk_fp and d_s1_fp at chunk k >= n_chunks[s]
 *   are not written; d_hash is written at [offsets[0], total) only.
 *   d_workspace  : kvr_keys_workspace_bytes(total) bytes, 256-byte aligned
 * Device errors: KVR_DEV_BAD_TOKEN for an id outside [0, vocab) (its Gear
 * value counts as 0).
 * Errors: KVR_E_ARG (null pointer, bad parameters, chunk_cap too small),
 * KVR_E_RANGE (offsets), KVR_E_UNSUPPORTED (n_streams > 240),
 * KVR_E_WORKSPACE, KVR_E_HIP.
 * ---------------------------------------------------------------------- */
size_t kvr_keys_workspace_bytes(int64_t total_tokens);
kvr_status registry_chunk_keys(const int32_t* d_tokens, const int64_t* offsets, int32_t n_streams,
                               const uint64_t* d_gear, int32_t vocab, const kvr_cdc_params* params,
                               uint64_t* d_hash, int32_t* d_chunk_end, int32_t chunk_cap, int32_t* d_n_chunks,
                               uint64_t* d_chunk_fp, uint64_t* d_s1_fp, void* d_workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* ------------------------------------------------------------------------
 * Utilities.
 * ---------------------------------------------------------------------- */
int32_t     kvr_abi_version(void);
const char* kvr_status_str(kvr_status s);
/* hipError_t of the last KVR_E_HIP returned on this thread (0 if none). */
int32_t     kvr_last_hip_error(void);
/* Synchronize the current device, return its device error word (KVR_DEV_*
 * bits, OR-ed over all calls since the last read) in *flags, and clear it. */
kvr_status  kvr_device_errors(uint32_t* flags);
/* Zero-fill a workspace on `stream` (a plain fill kernel, graph-safe). */
kvr_status  kvr_workspace_clear(void* d_workspace, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVRELOC_H */
