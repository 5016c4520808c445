// Internal launch descriptors shared by the host entry points (api.cpp) and
// the kernels.  Everything here is passed by value as kernel arguments, so a
// launch needs no descriptor upload (no host->device copy before the kernel).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kvr {

constexpr int kThreads = 256;        // threads per workgroup (4 wave64)
constexpr int kPfItems = 16;         // max 16-byte position-free chunks held per thread
constexpr int kMaxTileRows = 128;    // rows per tile (LDS row tables)
constexpr int kMaxPairs = 128;       // rotation pairs per head (rope_dim <= 256)
constexpr int kMaxItems = 32;        // sequences / entries per launch
constexpr int kBandMaxBands = 64;    // bands one band-mover workgroup walks (4 block ids each in LDS)

// Byte-addressed view of the two parts of a paged pool.
struct Pool {
    char* pf;  int64_t pf_l, pf_b, pf_r;     // strides in bytes
    char* rp;  int64_t rp_l, rp_b, rp_r;
    int32_t block_size, n_blocks, n_layers;
    int32_t bs_shift;       // log2(block_size) if a power of two, else -1
    int32_t pf_chunks;      // 16-byte chunks of the position-free part per row
    int32_t rope_items;     // rotation items per row: heads * half_chunks
    int32_t half_chunks;    // 16-byte chunks in half a head
    int32_t head_bytes;     // bytes of one rotary head
    int32_t half_bytes;     // bytes of half a head
    int32_t n_pairs;        // rope_dim / 2
    int32_t pairs_per_chunk;  // 8 (bf16) or 4 (f32)
};

// Rows living outside the pool: a registry entry or a splice stub.
struct SrcRows {
    const char* pf;
    const char* rp;
    int64_t pf_l, rp_l;                      // layer strides, bytes
    int32_t pf_r, rp_r;                      // row strides, bytes
};

// One sequence (splice) or one registry entry (gather) of a launch.
struct Item {
    SrcRows src;
    int32_t a;            // splice: s_end (first moved slot); gather: p_target
    int32_t b;            // splice: s_start (first stub slot)
    int32_t shift;        // rotation shift (Delta or delta)
    int32_t moved;        // splice: rows moved; gather: entry length
    int32_t r_len;        // splice: stub rows written (0 = none)
    int32_t move_tiles;   // per layer
    int32_t tiles;        // per layer: move tiles, then stub tiles
    int32_t bt_off;       // element offset of this item's block-table row
    int32_t wg_off;       // splice: first workgroup of this item (all layers);
                          // gather: first tile of this item (per layer)
};

struct RelocArgs {
    Pool pool;
    const int32_t* bt;
    uint32_t* counters;   // splice: one ticket counter per (item, layer)
    uint32_t* flags;      // splice: one "sources read" flag per tile
    int32_t n_items;
    int32_t tile_rows;
    uint32_t epoch;       // value a flag takes when set in this launch
    int32_t n_wg;
    int32_t n_tiles;      // gather: tiles per layer, all items
    union {
        double omega[kMaxPairs];   // theta_j / (2 pi): revolutions per position
        float cs[2 * kMaxPairs];   // one-item band mover: (cos, sin) of its item's shift per pair,
                                   // formed on the host in float64
    };
    Item items[kMaxItems];
    int32_t offs[kMaxItems];   // items[i].wg_off side by side, INT32_MAX past n_items:
                               // a workgroup finds its item in one scalar pass
};
static_assert(sizeof(RelocArgs) <= 4000, "row mover arguments too large");

// One registry entry (gather with patch) or one slot range (in-place patch).
constexpr int kPatchMaxPairs = 64;   // rope_dim <= 128 on the patch path
constexpr int kPatchTileRows = 64;   // tokens per workgroup on the patch path (4 x 16)
constexpr int kPatchMaxItems = 16;

struct PatchItem {
    const char* src_pf; const char* src_rp;    // entry rows (gather); unused in place
    int64_t src_pf_l, src_rp_l;                // bytes
    int32_t src_pf_r, src_rp_r;                // bytes
    const float* U_rp; const float* V_rp;      // rotary-part factors (or null)
    int64_t u_rp_l, v_rp_l;                    // layer strides, floats
    const float* U_pf; const float* V_pf;      // position-free-part factors (or null)
    int64_t u_pf_l, v_pf_l;
    int32_t rank_rp, rank_pf;                  // 0 = no patch
    int32_t dst0;                              // destination slot of row 0
    int32_t shift;                             // rotation (gather); 0 in place
    int32_t len;                               // rows
    int32_t tiles;                             // tiles per layer
    int32_t wg_off;                            // first workgroup of this item
};

// Streaming form of the patch kernel (patch_dma_kernel): one workgroup per
// (item, layer, 256-byte unit of the row), each wave streaming 16-row stages.
constexpr int kPatchDmaMaxStages = 64;   // stages per wave: items of at most 4 x 64 x 16 rows

struct PatchArgs {
    Pool pool;
    const int32_t* bt;
    int32_t n_items, tile_rows, n_wg;
    int32_t do_rope, do_pf;
    int32_t dma;                               // 1: patch_dma_kernel (items' wg counts are layers x units)
    int32_t n_units, n_rope_units;             // units per row; the first n_rope_units are rotary heads
    double omega[kPatchMaxPairs];
    PatchItem items[kPatchMaxItems];
};
static_assert(sizeof(PatchArgs) <= 4000, "patch kernel arguments too large");

// Rotate-on-read MLA decode (decode.hip).
constexpr int kDecBlockTokens = 64;  // paged block size the decode kernel reads
constexpr int kDecMaxBlocks = 64;    // KV blocks per split (block and shift tables in LDS)

struct DecodeArgs {
    const char* ckv; int64_t ckv_b, ckv_r;     // layer applied; bytes
    const char* kr;  int64_t kr_b, kr_r;
    int32_t n_blocks;
    const uint16_t* q_nope;                    // bf16 [batch][heads][512]
    const uint16_t* q_rope;                    // bf16 [batch][heads][64]
    const int32_t* bt;                         // [batch][bt_stride]
    const int32_t* pend;                       // [batch][bt_stride]
    const int32_t* seq_lens;                   // [batch]
    int32_t bt_stride, max_len;
    int32_t batch, heads, n_split, blocks_per_split;
    float scale_log2;                          // softmax scale * log2(e)
    float* part_o;                             // [batch][n_split][heads/32][16*16*64]
    float* part_ml;                            // [batch][n_split][heads] x (max, sum)
    double omega[32];
};

// GQA decode (gqa_decode.hip): one wave per (sequence, KV head, split).
constexpr int kGqaDim = 128;          // head dimension the GQA decode reads
constexpr int kGqaMaxGroup = 16;      // query heads per KV head
constexpr int kGqaMaxBlocks = 64;     // KV blocks per split (tables in LDS)

struct GqaDecodeArgs {
    const char* k; int64_t k_b, k_r;          // K pool, layer applied; bytes
    const char* v; int64_t v_b, v_r;          // V pool, layer applied; bytes
    int32_t n_blocks;
    const uint16_t* q;                         // bf16 [batch][q_heads][128]
    const int32_t* bt;                         // [batch][bt_stride]
    const int32_t* pend;                       // [batch][bt_stride]
    const int32_t* seq_lens;                   // [batch]
    int32_t bt_stride, max_len;
    int32_t batch, q_heads, kv_heads, group, n_split, blocks_per_split;
    float scale_log2;                          // softmax scale * log2(e)
    float* part_o;                             // [batch][kv_heads][n_split][group][128]
    float* part_ml;                            // [batch][kv_heads][n_split][group] x (max, sum)
    double omega[kGqaDim / 2];
};

// Patch formation (patch_form.hip).
constexpr int kFormSketch = 32;       // columns of the range finder's sketch
constexpr int kFormMaxRank = 16;
constexpr int kFormPowerMaxCols = 1024;  // widest deficit the one-pass power step takes

struct FormGemmArgs {
    const float* D; int64_t d_stride;          // deficits, [n][rows][cols], stride in floats
    const float* X; int64_t x_stride;          // [n][K][32] (stride 0: one X for all)
    float* Y; int64_t y_stride;                // [n][M][32]
    int32_t n, rows, cols;
};
struct FormOrthArgs { float* Z; int32_t n; };  // [count][n][32], orthonormalized in place
struct FormEigArgs {
    const float* Y; const float* V;            // [count][rows][32], [count][cols][32]
    float* Uout; float* Vout; float* sigma;    // [count][rows][m], [count][cols][m], [count][m]
    int32_t rows, cols, rank;
};

// Block-table splice (lazy.hip): one workgroup per sequence.
constexpr int kLazyMaxBlocks = 8192;  // table entries a workgroup stages in LDS
constexpr int kLazyMaxSeq = 96;       // sequences per launch

struct LazySeq {
    int32_t row;                      // sequence index (row of the tables)
    int32_t n_old, n_new;             // blocks before / after
    int32_t s0b, s1b, rb;             // replaced range and stub count, in blocks
    int32_t delta;                    // slots (a multiple of the block size)
    int32_t stub_off, free_off;       // offsets into the stub / freed id lists
};

struct LazyArgs {
    int32_t* bt;
    int32_t* pend;
    const int32_t* stubs;
    int32_t* freed;
    int32_t bt_stride, block_size, n_seq;
    LazySeq seqs[kLazyMaxSeq];
};
static_assert(sizeof(LazyArgs) <= 4000, "lazy splice arguments too large");

// Block-table gather (lazy.hip): one workgroup per entry.
constexpr int kLazyMaxEntries = 80;   // entries per launch
struct LazyEntry {
    const int32_t* blocks;            // the entry's pool blocks
    const int32_t* pend;              // their own pending shifts, or null
    int32_t row;                      // sequence (row of the tables)
    int32_t slot0, nb;                // first logical block, block count
    int32_t delta;                    // p_target - base_pos
    int32_t rep_off;                  // offset into the replaced-id list
};
struct LazyGatherArgs {
    int32_t* bt;
    int32_t* pend;
    int32_t* replaced;                // or null
    int32_t bt_stride, n;
    LazyEntry ents[kLazyMaxEntries];
};
static_assert(sizeof(LazyGatherArgs) <= 4000, "lazy gather arguments too large");
static_assert(sizeof(GqaDecodeArgs) <= 4000, "GQA decode arguments too large");

// Registry keying (keying.hip).
constexpr int kKeyMaxStreams = 240;

struct KeyArgs {
    const int32_t* tokens;
    const uint64_t* gear;
    uint64_t* hash;                   // optional Gear hash per token
    uint64_t* cand;                   // candidate bitmask, one bit per token
    int32_t* chunk_end;
    int32_t* n_chunks;
    uint64_t* chunk_fp;
    uint64_t* s1_fp;                  // optional
    uint64_t threshold, seed;
    int64_t total;
    int32_t vocab, min_len, max_len, s1_window, s1_slots, cap, n_streams;
    int64_t offsets[kKeyMaxStreams + 1];
};
static_assert(sizeof(KeyArgs) <= 4000, "keying arguments too large");

// Kernel arguments must stay within the 4 KB kernarg budget.
static_assert(sizeof(RelocArgs) <= 4000, "relocation kernel arguments too large");

// Device scratch of the no-allocation splice (noalloc.hip): the ticketed
// mover's counters and flags for up to ~2M workgroups per launch.
#ifndef KVR_NOALLOC_SCRATCH_BYTES
#define KVR_NOALLOC_SCRATCH_BYTES (8u << 20)
#endif

// Records a HIP error for kvr_last_hip_error() and returns KVR_E_HIP (api.cpp).
int32_t record_hip_error(hipError_t e);

// Launchers (relocate.hip).  pf_slots / rope_slots are the per-thread counts
// of 16-byte position-free chunks and of rotation items a tile needs (powers
// of two up to 16, rope_slots <= pf_slots); rope_f32 selects fp32 keys.
hipError_t launch_splice(const RelocArgs& a, int pf_slots, int rope_slots, bool rope_f32, hipStream_t s);
// Band mover (in-place splice without cross-workgroup ordering): tile_rows
// is the band height (<= block size), the slot counts as above.  one_item:
// the launch holds a single item and carries its (cos, sin) table in cs.
hipError_t launch_band(const RelocArgs& a, int pf_slots, int rope_slots, bool rope_f32, bool one_item, hipStream_t s);
uint32_t read_and_clear_errors_band();
hipError_t launch_gather(const RelocArgs& a, int pf_slots, int rope_slots, bool rope_f32, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
uint32_t read_and_clear_errors_relocate();
// Patch kernel (patch.hip): fused gather + patch, or in-place patch.
hipError_t launch_patch(const PatchArgs& a, bool inplace, hipStream_t s);
uint32_t read_and_clear_errors_patch();
// Decode (decode.hip): split kernel + combine kernel.
hipError_t launch_decode(const DecodeArgs& a, uint16_t* out, float* lse, hipStream_t s);
uint32_t read_and_clear_errors_decode();
// Patch formation (patch_form.hip).
hipError_t launch_form_gemm(const FormGemmArgs& a, bool trans, hipStream_t s);
hipError_t launch_form_power(const FormGemmArgs& a, hipStream_t s);   // Z = D^T (D X), cols 256 k, k <= 4
hipError_t launch_form_orth(const FormOrthArgs& a, int count, hipStream_t s);
hipError_t launch_form_eig(const FormEigArgs& a, int count, hipStream_t s);
hipError_t launch_form_mean(const float* d, int orders, int64_t per, int64_t n, float* out, hipStream_t s);
// GQA decode (gqa_decode.hip): split kernel + combine kernel.
hipError_t launch_gqa_decode(const GqaDecodeArgs& a, uint16_t* out, float* lse, hipStream_t s);
uint32_t read_and_clear_errors_gqa_decode();
// Block-table splice (lazy.hip).
hipError_t launch_lazy(const LazyArgs& a, hipStream_t s);
hipError_t launch_lazy_gather(const LazyGatherArgs& a, hipStream_t s);
uint32_t read_and_clear_errors_lazy();
// Registry keying (keying.hip): Gear hashes and candidates, cuts, fingerprints.
hipError_t launch_keys(const KeyArgs& a, hipStream_t s);
uint32_t read_and_clear_errors_keys();

}  // namespace kvr
