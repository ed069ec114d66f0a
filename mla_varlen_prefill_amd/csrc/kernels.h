// Internal interface between the C-ABI host code (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Tile shape of the attention kernel: one workgroup owns FWD_BM query rows of
// one (sequence, head) and walks the visible keys in tiles of FWD_BN.
constexpr int FWD_BM = 256;
constexpr int FWD_BN = 64;
constexpr int FWD_THREADS = 512;
constexpr int ROPE_DIM = 64;    // rope part, fixed by the operator definition
constexpr int MASK_TILE = 512;  // side of the MASK_FREE tile

// Per-sequence record of the work list (int32 x 4).
struct SeqRec {
    int32_t q_off;   // first query row of the sequence in Q / attenOut
    int32_t kv_off;  // first key row in K / KRope / V (packed offset or b * max_seq)
    int32_t q_len;
    int32_t kv_len;
};

// Query rows of one workgroup's task: FWD_BM / 2^pack_shift rows of each of
// 2^pack_shift query heads that share one KV head, so every K/V tile staged
// in LDS serves all of them (pack_shift = 0 without head grouping).
constexpr int FWD_MAX_PACK_SHIFT = 3;

// One work item: q_rows (= FWD_BM >> pack_shift) query rows starting at
// q_row0 of sequence b, and the number of FWD_BN-key tiles (from key 0) that
// any of them can see.
struct WorkItem {
    int32_t b;
    int32_t q_row0;
    int32_t kv_tiles;
    int32_t q_rows;
};

// One workgroup's task: key tiles [kt0, kt1) of a work item for its query
// heads head .. head + 2^pack_shift - 1. A task holding only part of the
// item's tiles writes a partial result into partial slot `part` (-1: the task
// holds all of them and writes the output). item == -1 marks an empty
// padding task.
struct Task {
    int32_t item;
    int32_t head;
    int32_t kt0, kt1;
    int32_t part;
};

// MI355X: 8 XCDs of 32 CUs; consecutive workgroups of a launch go to
// consecutive XCDs.
constexpr int MLA_XCDS = 8;
constexpr int MLA_CUS_PER_XCD = 32;

// What one workgroup of the attention launch runs, flattened so that the
// kernel reads it with a single scalar load: a work item (q rows of one
// sequence) for 2^pack_shift query heads from `head`. head == -1 marks an
// empty padding workgroup.
// A task over key tiles [kt0, kt1) of its item is run as the item over the
// sequence's keys from kt0 * FWD_BN on: kv_off and kv_len are shifted by that
// many keys, which leaves every row's causal position relative to the keys
// unchanged (position - k0 = (kv_len - k0) - rows + row), and, since the
// planner cuts only at multiples of 512 keys under MASK_FREE, its 512-key
// blocks too.
struct LaunchRec {
    int32_t q_tok0;    // first query row of the item in Q / attenOut (sequence offset + row in the sequence)
    int32_t kv_tiles;  // FWD_BN-key tiles (from the task's first key) any of its rows can see
    int32_t head;      // first query head; -1: padding
    int32_t kv_head;   // the KV head of those query heads
    int32_t q_left;    // query rows of the sequence from the item's first row on
    int32_t kv_off;    // contiguous K/V: row of the task's first key; paged: the sequence index, plus the
                       // task's first tile (FWD_BN keys) of the sequence << PAGED_SEQ_BITS
    int32_t kv_len;    // keys of the sequence from the task's first key on
    int32_t part;      // -1: write attenOut; else the partial slot (normalised fp32 rows and log-sum-exp)
};
static_assert(sizeof(LaunchRec) == 32, "one scalar load per workgroup");

// Partial results of tasks holding part of an item's key tiles: slot s holds,
// for each of the FWD_BM wave rows (wave slot w = 0..7, row r = 0..31, the
// kernel's row order), the row's attention output over the task's keys
// alone in fp32 (head_dim values) and the log-sum-exp of its scaled, masked
// scores over those keys (-inf: no visible key among them). The merge
// combines the n_parts slots part0.. of one (item, head pack) into attenOut.
struct MergeRec {
    int32_t part0;
    int32_t n_parts;
    int32_t head;    // first query head
    int32_t q_tok0;  // as in LaunchRec
    int32_t q_left;
    int32_t pad[3];
};
static_assert(sizeof(MergeRec) == 32, "merge record size");
constexpr int PART_ROWS = FWD_BM;

struct FwdParams {
    const void *q;        // [nq, H, D]
    const void *q_rope;   // [nq, H, 64]
    const void *k;        // rows of Hkv * D
    const void *k_rope;   // rows of Hkv * 64
    const void *v;        // rows of Hkv * D
    const void *mask;     // [512, 512] or nullptr
    // MASK_FREE: class of each (tile row, 64-key block) of the mask tile,
    // uint8 [512][8] (MASK_CLS_*), or nullptr (every diagonal-block tile then
    // takes the per-element path)
    const uint8_t *mask_cls;
    void *out;            // [nq, H, D]
    const LaunchRec *launch;  // one record per workgroup
    float *part_o;            // partial rows: [parts, PART_ROWS, head_dim] fp32 (tasks with part >= 0)
    float *part_lse;          // [parts, PART_ROWS]
    int32_t heads;
    int32_t kv_heads;
    int32_t group;        // heads / kv_heads
    int32_t mask_type;    // enum mla_mask_type
    int32_t mask_is_bf16; // dtype of the MASK_FREE tile
    int32_t n_tasks;      // workgroups to launch
    int32_t pack_shift;   // log2 of the query heads one workgroup runs
    int32_t head_dim;     // embeddimV: 64 or 128
    float qk_scale;       // qkScale as given (any finite value, 0 included)
    // Paged K/V (launch_mla_fwd with paged = true): k, k_rope and v point at
    // ND caches [num_blocks, block_size, Hkv, D | 64 | D]; key t of
    // sequence b is slot t % block_size of block block_tables[b][t / block_size].
    const int32_t *block_tables;  // [batch, bt_stride]
    int32_t bt_stride;
    int32_t block_size;           // a multiple of FWD_BN
    int32_t num_blocks;
};

// Key tiles of one sequence the paged kernel can address (its per-tile table
// lives in LDS): PAGED_MAX_TILES * FWD_BN keys.
constexpr int PAGED_MAX_TILES = 2048;
// A paged launch record's kv_off: sequence index in the low PAGED_SEQ_BITS
// bits, the task's first tile above them (below PAGED_MAX_TILES = 2^11).
constexpr int PAGED_SEQ_BITS = 20;
static_assert(PAGED_MAX_TILES <= (1 << (31 - PAGED_SEQ_BITS)), "first tile must fit above the sequence index");

// dtype: 1 = fp16, 2 = bf16 (enum mla_dtype). One workgroup per task.
hipError_t launch_mla_fwd(const FwdParams &p, int dtype, bool paged, hipStream_t stream);

// Classes of the MASK_FREE tile's 64-entry row blocks: every entry +-0, every
// entry -inf, or anything else.
constexpr uint8_t MASK_CLS_ZERO = 0, MASK_CLS_MIXED = 1, MASK_CLS_DEAD = 2;
constexpr int MASK_CLS_BYTES = 512 * 8;
hipError_t launch_mask_classify(const void *mask, int mask_is_bf16, uint8_t *cls, hipStream_t stream);

struct MergeParams {
    const MergeRec *merges;
    const float *part_o;
    const float *part_lse;
    void *out;  // attenOut [nq, heads, head_dim]
    int32_t n_merges;
    int32_t heads;
    int32_t pack_shift;
    int32_t head_dim;
};

// Combine the partial results of split tasks into attenOut (dtype as above).
hipError_t launch_mla_merge(const MergeParams &p, int dtype, hipStream_t stream);

struct GatherParams {
    const void *key_cache;
    const void *value_cache;  // may be null
    void *key;
    void *value;              // null iff value_cache is null
    const int32_t *block_tables;
    const int32_t *context_lens;
    const int32_t *seq_starts; // null unless has_seq_starts
    int64_t num_blocks;
    int64_t block_size;
    int64_t max_blocks;       // columns of block_tables
    int64_t num_tokens;       // rows of key / value
    int64_t row_bytes_k;      // bytes of one token row (heads * head_size_k * elem)
    int64_t row_bytes_v;
    int32_t batch;
    int32_t ctx_entries;      // batch or batch + 1
    int32_t cumsum;
    int32_t has_seq_starts;
    // NZ layout: caches [num_blocks, chunks, block_size, 32 bytes], outputs
    // [num_tokens, chunks * 32 bytes]; row_bytes_* = chunks_* * 32.
    int32_t nz;
    int64_t chunks_k;
    int64_t chunks_v;
};

constexpr int GATHER_MAX_BATCH = 8192;  // offsets table in LDS: (batch + 1) * 8 bytes

hipError_t launch_paged_gather(const GatherParams &p, hipStream_t stream);

// ---- MLA prolog (non-quantised): products of bf16 activations [M, K] with
// bf16 weights [K, N] (both row-major), in output tiles of PROLOG_BN columns x
// PROLOG_BM rows, with an epilogue per column range.
constexpr int PROLOG_BN = 512;  // one head / one normalised row per tile
constexpr int PROLOG_BM = 128;
constexpr int PROLOG_BK = 32;   // k per pipeline stage
constexpr int PROLOG_K_MULTIPLE = 128;  // K must be a multiple (4 stages)
constexpr int PROLOG_ROPE = 64; // rope_dim: the tile's last 64 columns

enum PrologEpilogue : int32_t {
    PROLOG_STORE_F32 = 0,  // out (fp32) = product
    PROLOG_NORM_ROPE = 1,  // out (bf16) = rope(RmsNorm over the tile's 512 columns (* gamma))
};

struct PrologSegment {
    const void *w;       // bf16 (int8 with PrologGemmParams::int8) [K, ldw]; tile j reads columns j*512 .. j*512+511
    int64_t ldw;         // row stride of w, elements
    void *wp;            // packed copy of w (launch_prolog_pack): n_tiles * (K / stage k) blocks of 32 KB
    int32_t n_tiles;     // 512-column tiles of this segment
    int32_t epilogue;    // PrologEpilogue
    void *out;           // tile j of rows m: out + m * ld_out + j * 512 (elements of the epilogue's type)
    int64_t ld_out;
    const void *gamma;   // bf16 [n_tiles * 512] or null (weight 1); PROLOG_NORM_ROPE only
};

struct PrologGemmParams {
    const void *a;       // bf16 [M, lda], or int8 with int8 set
    int64_t lda;
    int32_t m;           // rows
    int32_t k;           // a multiple of PROLOG_K_MULTIPLE (bf16) or PROLOG_K_MULTIPLE_I8 (int8)
    PrologSegment seg[2];  // tiles 0 .. seg[0].n_tiles - 1 from seg[0], the rest from seg[1]
    const void *rope_cos;  // bf16 [M, 64]
    const void *rope_sin;
    float eps;
    // int8 operands (a and the weights), int32 products: the tile epilogue
    // first scales product (m, n) by row_scale[m] * col_scale[n] (fp32);
    // PROLOG_NORM_ROPE only
    int32_t int8;
    const float *row_scale;  // [M]
    const float *col_scale;  // [N], column n of the segment's weights
    // Split over K (bf16 only; few output tiles): with k_splits > 1 each
    // tile runs as k_splits workgroups, workgroup s over stages
    // [s * nk / k_splits, (s + 1) * nk / k_splits) of the nk = k / PROLOG_BK;
    // nk / k_splits must be a multiple of 4. Each writes its raw fp32 sums to
    // part + s * m * ld_part, tile n of the two segments together at column
    // n * PROLOG_BN, and launch_prolog_split_reduce adds the parts and
    // applies the segments' epilogues.
    int32_t k_splits;
    float *part;
    int64_t ld_part;
    // bf16 only, k_splits 1: when a1 is set, seg[1] reads its own activation
    // a1 [M, lda1] over K = k1 (a multiple of PROLOG_K_MULTIPLE, its packed
    // weights laid out for k1), and its workgroups come first in the launch.
    // launch_prolog_pack does not take this form (pack such a segment with
    // its own a, lda and k).
    const void *a1;
    int64_t lda1;
    int32_t k1;
};
// An int8 stage is 64 k: the same 64 bytes per row as a bf16 stage of 32 k.
constexpr int PROLOG_K_MULTIPLE_I8 = 256;

// Bytes of a segment's packed weights: one 32 KB block per 512-column tile and
// 32-row stage of K.
constexpr int64_t PROLOG_PACK_BLOCK = PROLOG_BN * PROLOG_BK * 2;
inline int64_t prolog_packed_bytes(int32_t n_tiles, int32_t k, bool int8 = false) {
    return (int64_t)n_tiles * (k / (int8 ? 2 * PROLOG_BK : PROLOG_BK)) * PROLOG_PACK_BLOCK;
}

// Writes seg.wp from seg.w for each segment with tiles: block (j, kt) is the
// stage image the product kernel reads (see prolog.hip).
hipError_t launch_prolog_pack(const PrologGemmParams &p, hipStream_t stream);
hipError_t launch_prolog_gemm(const PrologGemmParams &p, hipStream_t stream);
// The epilogues of a product run with k_splits > 1, on the sum of its parts.
hipError_t launch_prolog_split_reduce(const PrologGemmParams &p, hipStream_t stream);

// y fp32 [rows, cols] (row stride ld_y) -> out bf16 [rows, cols] (row stride
// ld_out) = RmsNorm over each row * gamma; cols a multiple of 256.
hipError_t launch_prolog_rms_rows(const float *y, int64_t ld_y, const void *gamma, void *out, int64_t ld_out,
                                  int32_t rows, int32_t cols, float eps, hipStream_t stream);

// y fp32 [rows, cols] -> c = RmsNorm over each row * gamma, quantised per row:
// scale[row] = max |c| / 127 (fp32), codes int8 [rows, cols] (row stride
// ld_codes) = c / scale rounded to nearest, ties to even (0 for a zero row);
// cols a multiple of 256, at most PROLOG_QUANT_MAX_COLS.
constexpr int PROLOG_QUANT_MAX_COLS = 2048;
hipError_t launch_prolog_quant_rows(const float *y, int64_t ld_y, const void *gamma, void *codes, int64_t ld_codes,
                                    float *scale, int32_t rows, int32_t cols, float eps, hipStream_t stream);

}  // namespace mla
