/*
 * mla_prefill.h -- C ABI of the MI355X (gfx950) MLA varlen-prefill library.
 *
 * The operations below, each defined by one page: two Ascend Transformer
 * Boost C API pages, and the MlaProlog operator notes (further down):
 *
 *   mla_prefill_get_workspace_size / mla_prefill
 *     "MLA Prefill" page, Definition and the AtbMLAPreFillGetWorkspaceSize
 *     Members table. For every sequence b of a variable-length batch and every
 *     query head h it computes
 *         S  = qkScale * (Q . K^T + QRope . KRope^T) + mask
 *         O  = softmax_rows(S) . V
 *     with a split head: an embeddimV-element "nope" part (Q, K, V) and a
 *     64-element rope part (QRope, KRope). The page's two-phase protocol
 *     (plan the workspace, then run) is kept; the page's atb::Operation and
 *     atb::Context handles are replaced by a stateless call that takes the
 *     same arguments twice plus a HIP stream.
 *
 *   paged_cache_load
 *     "PagedCacheLoadOperation" page, Definition and Members table. Copies the
 *     tokens of each sequence out of a block-paged K/V cache into packed
 *     key/value tensors. The page's plan phase is folded in: the gather needs
 *     no workspace.
 *
 * Conventions shared by every entry point
 *   - Tensors are passed as mla_tensor descriptors: a data pointer, a dtype
 *     code and a row-major shape. Every tensor is dense and row-major ("ND"
 *     on the pages). Device tensors must be 16-byte aligned.
 *   - Ownership: the caller owns every tensor, the workspace and the stream.
 *     The library allocates and frees no device memory and keeps no pointer
 *     after a call returns. Host arrays are read before the call returns.
 *     (Exception: mla_prefill_no_alloc's fixed per-GPU work-list array, a
 *     static device array of the library, looked up once per device.)
 *   - Calls that take a stream only enqueue work on it (hipStream_t passed as
 *     void*; NULL is the default stream) and return without synchronising.
 *   - Return value: MLA_OK (0) or a negative MLA_ERR_* code. Arguments are
 *     validated completely before any HIP call: on an error nothing is
 *     enqueued and no output is touched. mla_last_error() returns a
 *     thread-local message describing the last failure of the calling thread.
 *   - The library holds no other state and is safe to call from several
 *     threads (mla_prefill_no_alloc: see its note on overlapping calls).
 */
#ifndef MLA_PREFILL_H
#define MLA_PREFILL_H

#include <stdbool.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. The pages allow float16/bf16 for attention data and
 * float16/bf16/int8 for paged caches; int32 is used for lengths and tables,
 * float32 for the quantised prolog's scales. */
enum mla_dtype {
    MLA_FP16 = 1,
    MLA_BF16 = 2,
    MLA_INT8 = 3,
    MLA_INT32 = 4,
    MLA_FP32 = 5
};

/* maskType. The "MLA Prefill" page names the modes (Members table, rows
 * Mask and maskType) but prints no integer values; these are ours.
 *   MLA_MASK_UNDEFINED  all-zero mask: every key of the sequence is visible.
 *   MLA_MASK_SPEC       causal, bottom-right aligned (query i of a sequence
 *                       sits at key position kvSeqLen - qSeqLen + i and sees
 *                       keys 0..that position). With qSeqLen == 1 the single
 *                       query sees every key, i.e. the mask only acts when
 *                       qSeqLen > 1.
 *   MLA_MASK_CAUSAL     same visibility rule as MLA_MASK_SPEC.
 *   MLA_MASK_FREE       a 512 x 512 tile (argument mask) placed on the
 *                       diagonal 512-blocks of key-position space: for a
 *                       query at position p and key j, blocks with
 *                       j/512 < p/512 are fully visible, j/512 > p/512 fully
 *                       masked, and j/512 == p/512 adds
 *                       mask[p % 512][j % 512]. A causal tile (0 on and below
 *                       the diagonal, -inf above) reproduces MLA_MASK_CAUSAL. */
enum mla_mask_type {
    MLA_MASK_UNDEFINED = 0,
    MLA_MASK_SPEC = 1,
    MLA_MASK_CAUSAL = 2,
    MLA_MASK_FREE = 3
};

/* kvCacheCfg ("PagedCacheLoadOperation" page, Members table): NZ = 0 is the
 * page's default, ND = 1. Both layouts are implemented (see paged_cache_load). */
enum mla_kv_cache_cfg {
    MLA_KV_CACHE_NZ = 0,
    MLA_KV_CACHE_ND = 1
};

/* Status codes (0 = success, like atb::Status on the pages). */
enum mla_status {
    MLA_OK = 0,
    MLA_ERR_NULL = -1,        /* a required pointer or descriptor is NULL */
    MLA_ERR_SHAPE = -2,       /* a shape disagrees with the others or with the lengths */
    MLA_ERR_DTYPE = -3,       /* a dtype is not allowed or dtypes disagree */
    MLA_ERR_VALUE = -4,       /* a scalar argument or length is out of range */
    MLA_ERR_UNSUPPORTED = -5, /* a valid request this build does not implement */
    MLA_ERR_WORKSPACE = -6,   /* workspace NULL, too small or misaligned */
    MLA_ERR_RUNTIME = -7      /* a HIP call failed (no device, launch error, ...) */
};

/* Dense row-major tensor. shape[0..ndim-1] are used; ndim is 1..4. */
typedef struct mla_tensor {
    void *data;
    int32_t dtype;     /* enum mla_dtype */
    int32_t ndim;
    int64_t shape[4];
} mla_tensor;

/*
 * mla_prefill_get_workspace_size -- plan phase of "MLA Prefill"
 * (AtbMLAPreFillGetWorkspaceSize on the page). Host only: no HIP call.
 *
 * Arguments (the page's Members table, same order):
 *   q          device, [nTokens, headNum*D] or [nTokens, headNum, D], fp16/bf16.
 *              nTokens = sum of q_seqlen. D = embeddimV: 64 or 128 here (other
 *              values return MLA_ERR_UNSUPPORTED).
 *   q_rope     device, [nTokens, headNum*64] or [nTokens, headNum, 64], same dtype.
 *   k          device, packed [sum kv_seqlen, kvHeadNum, D], or padded
 *              [batch, max_seq, kvHeadNum*D] (sequence b's keys start at row
 *              b*max_seq). A shape valid both ways is read as packed.
 *   k_rope     device, like k with 64 in place of D.
 *   v          device, like k.
 *   q_seqlen   HOST int32 [batch], each >= 0.
 *   kv_seqlen  HOST int32 [batch], each >= 0. qSeqLen may exceed kvSeqLen;
 *              under a causal mode the rows with no visible key return 0.
 *   mask       device [512, 512] fp16/bf16, additive; required for
 *              MLA_MASK_FREE, ignored (may be NULL) otherwise. Its dtype may
 *              differ from the data dtype.
 *   head_num   query heads (> 0).
 *   qk_scale   finite float multiplying the whole 192-deep product, rope
 *              term included, before the mask is added.
 *   kv_head_num  KV heads (> 0, divides head_num). Query head h reads KV
 *              head h / (head_num / kv_head_num).
 *   mask_type  enum mla_mask_type.
 *   cache_mode only 0 (K/V given as contiguous tensors) is accepted; the page
 *              documents no other value. Other values: MLA_ERR_UNSUPPORTED.
 *   atten_out  device, [nTokens, headNum*D] or [nTokens, headNum, D], same dtype as q.
 *   workspace_size  out: bytes of device workspace mla_prefill needs.
 * A row of a sequence that sees no key (kv_seqlen 0, or fully masked) is
 * written as zeros.
 */
int mla_prefill_get_workspace_size(const mla_tensor *q, const mla_tensor *q_rope,
                                   const mla_tensor *k, const mla_tensor *k_rope,
                                   const mla_tensor *v, const mla_tensor *q_seqlen,
                                   const mla_tensor *kv_seqlen, const mla_tensor *mask,
                                   int32_t head_num, float qk_scale, int32_t kv_head_num,
                                   int32_t mask_type, uint8_t cache_mode,
                                   const mla_tensor *atten_out, uint64_t *workspace_size);

/*
 * mla_prefill -- run phase of "MLA Prefill" (AtbMLAPreFill on the page).
 * The first 14 arguments are those of mla_prefill_get_workspace_size, with
 * the same values. workspace: device memory of at least the planned size,
 * 16-byte aligned (NULL allowed when the planned size is 0). The call copies
 * a work list built from the host lengths into the workspace and enqueues the
 * attention kernel on stream; the workspace must stay untouched until that
 * work has run. When the problem holds little work for the GPU's 256 compute
 * units (few heads or sequences), items longer than an even share of it are
 * cut into runs of consecutive key tiles, each run a workgroup of its own;
 * such a workgroup writes its rows over its own keys in fp32 with their
 * log-sum-exp into the workspace (head_dim * 4 + 4 bytes per row and run),
 * and a second kernel on the same stream combines the runs of each row. The
 * result then differs from an unsplit run only by rounding. Under
 * MLA_MASK_FREE the workspace also ends with 4 KiB in which a small kernel,
 * enqueued first, records for each 64-entry block of a mask row whether it
 * is all zero, all -inf or neither; the attention kernel uses this to skip
 * the per-element mask on all-zero blocks and to skip all -inf blocks, with
 * the same result bit for bit. Errors:
 * validation codes as above, MLA_ERR_WORKSPACE, MLA_ERR_RUNTIME when a HIP
 * call fails.
 */
int mla_prefill(const mla_tensor *q, const mla_tensor *q_rope, const mla_tensor *k,
                const mla_tensor *k_rope, const mla_tensor *v, const mla_tensor *q_seqlen,
                const mla_tensor *kv_seqlen, const mla_tensor *mask, int32_t head_num,
                float qk_scale, int32_t kv_head_num, int32_t mask_type, uint8_t cache_mode,
                const mla_tensor *atten_out, void *workspace, uint64_t workspace_size,
                void *stream);

/*
 * mla_prefill_no_alloc -- mla_prefill for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same first 14 arguments and stream as mla_prefill, and no
 * workspace: the work list goes into a fixed array in device memory that the
 * library holds, MLA_NO_ALLOC_WORKSPACE_BYTES (4 MiB = 131072 launch records)
 * on each GPU it runs on, until the process ends. The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine). It never splits an
 * item (mla_prefill may, where little work is spread over many compute
 * units), so its work list is one 32-byte launch record per workgroup, and
 * its result can differ from mla_prefill's by rounding where mla_prefill
 * splits. A problem whose work list is larger than the array returns
 * MLA_ERR_WORKSPACE before anything is enqueued; at 128 heads the limit is
 * reached near 256K query rows. The first call on a device looks the array's
 * address up with that device current (the tensors and the stream must belong
 * to the current device, as for mla_prefill).
 * Every call on one GPU uses that GPU's single array, which keeps the last
 * call's work list: calls on one stream are ordered and safe, but calls that
 * overlap on one GPU (several streams, or threads without ordering) race and
 * can compute wrong results. Errors: as mla_prefill.
 */
#define MLA_NO_ALLOC_WORKSPACE_BYTES (4u << 20)
int mla_prefill_no_alloc(const mla_tensor *q, const mla_tensor *q_rope, const mla_tensor *k,
                         const mla_tensor *k_rope, const mla_tensor *v, const mla_tensor *q_seqlen,
                         const mla_tensor *kv_seqlen, const mla_tensor *mask, int32_t head_num,
                         float qk_scale, int32_t kv_head_num, int32_t mask_type, uint8_t cache_mode,
                         const mla_tensor *atten_out, void *stream);

/*
 * paged_cache_load -- "PagedCacheLoadOperation" page (AtbPagedCacheLoad).
 *
 *   key_cache     device ND [num_blocks, block_size, num_heads, head_size_k],
 *                 fp16/bf16/int8.
 *   value_cache   device ND [num_blocks, block_size, num_heads, head_size_v], same
 *                 dtype, num_blocks and block_size; or NULL to gather keys only
 *                 (then value must be NULL too).
 *   block_tables  device int32 [batch, max_blocks]: block ids of each sequence.
 *   context_lens  device int32. Plain mode: [batch] token counts (their sum
 *                 may pass 2^31; the device sums them in 64 bits). Cumulative
 *                 mode (is_seq_lens_cumsum_type): running totals, either
 *                 [batch + 1] starting with 0 or [batch] inclusive totals.
 *   key, value    device outputs [num_tokens, num_heads, head_size_k / _v] of the
 *                 cache dtype, num_tokens = total tokens gathered; sequence b's
 *                 tokens are packed in batch order.
 *   seq_starts    device int32 [batch]: token offset of each sequence inside its
 *                 block table's logical space. Read only when has_seq_starts;
 *                 otherwise every sequence starts at 0 and it may be NULL.
 *   kv_cache_cfg  MLA_KV_CACHE_ND (1), or MLA_KV_CACHE_NZ (0), the layout of the
 *                 page's dimension table, NZ column: caches
 *                 [num_blocks, num_heads*head_size / E, block_size, E] with E = 32
 *                 for int8 and 16 for fp16/bf16 (32-byte chunks), outputs 2-D
 *                 [num_tokens, num_heads*head_size]; chunk c of the token in
 *                 slot s of block k is cache[k][c][s]. The page allows seqStarts
 *                 and cumulative lengths in the ND layout only: with NZ they return
 *                 MLA_ERR_UNSUPPORTED.
 *
 * Token t of sequence b is logical position s_b + t, found in block
 * block_tables[b][(s_b + t) / block_size] at slot (s_b + t) % block_size. The
 * copy is bit-exact. Lengths and tables live on the device, so the host cannot
 * check them: a token whose output row lies beyond num_tokens, whose table
 * column lies beyond max_blocks, or whose block id lies outside
 * [0, num_blocks) is not written.
 */
int paged_cache_load(const mla_tensor *key_cache, const mla_tensor *value_cache,
                     const mla_tensor *block_tables, const mla_tensor *context_lens,
                     const mla_tensor *key, const mla_tensor *value,
                     const mla_tensor *seq_starts, int8_t kv_cache_cfg,
                     bool is_seq_lens_cumsum_type, bool has_seq_starts, void *stream);

/*
 * mla_prefill_paged_get_workspace_size / mla_prefill_paged -- "MLA Prefill"
 * with K, KRope and V read in place from paged caches. The result equals
 * paged_cache_load ("PagedCacheLoadOperation" page, Members table: ND caches,
 * plain contextLens, no seqStarts) of K, KRope and V followed by mla_prefill
 * (cache_mode 0) on the gathered tensors, without materialising them.
 *
 *   q, q_rope, q_seqlen, mask, head_num, qk_scale, kv_head_num, mask_type,
 *   atten_out   as for mla_prefill.
 *   key_cache     device ND [num_blocks, block_size, kvHeadNum, D], dtype of q.
 *   krope_cache   device ND [num_blocks, block_size, kvHeadNum, 64], dtype of q.
 *   value_cache   device ND [num_blocks, block_size, kvHeadNum, D], dtype of q.
 *   block_tables  device int32 [batch, max_blocks]: key t of sequence b is slot
 *                 t % block_size of block block_tables[b][t / block_size]
 *                 (every sequence starts at position 0 of its table row).
 *   kv_seqlen     HOST int32 [batch]: keys (context length) of each sequence.
 * Supported here: block_size a multiple of MLA_PLAN_KV_COLS (64), at most
 * MLA_PAGED_MAX_KEYS keys per sequence, num_blocks * block_size < 2^31, at
 * most 2^20 sequences; otherwise MLA_ERR_UNSUPPORTED. max_blocks must cover ceil(kv_len /
 * block_size) for every sequence (else MLA_ERR_SHAPE). Block ids live on the
 * device and are not checked by the host: a 64-key tile whose block id lies
 * outside [0, num_blocks) reads as zeros (those keys contribute exp(0 - max)
 * weight with a zero value row; they are not an error signal). Workspace
 * (including the split of long items over runs of keys and its merge),
 * stream and error behaviour as for mla_prefill; the plan equals
 * mla_prefill's for the same lengths, so the two paths agree bit for bit.
 */
#define MLA_PAGED_MAX_KEYS (2048 * 64)
int mla_prefill_paged_get_workspace_size(const mla_tensor *q, const mla_tensor *q_rope,
                                         const mla_tensor *key_cache, const mla_tensor *krope_cache,
                                         const mla_tensor *value_cache, const mla_tensor *block_tables,
                                         const mla_tensor *q_seqlen, const mla_tensor *kv_seqlen,
                                         const mla_tensor *mask, int32_t head_num, float qk_scale,
                                         int32_t kv_head_num, int32_t mask_type,
                                         const mla_tensor *atten_out, uint64_t *workspace_size);
int mla_prefill_paged(const mla_tensor *q, const mla_tensor *q_rope, const mla_tensor *key_cache,
                      const mla_tensor *krope_cache, const mla_tensor *value_cache,
                      const mla_tensor *block_tables, const mla_tensor *q_seqlen,
                      const mla_tensor *kv_seqlen, const mla_tensor *mask, int32_t head_num,
                      float qk_scale, int32_t kv_head_num, int32_t mask_type,
                      const mla_tensor *atten_out, void *workspace, uint64_t workspace_size,
                      void *stream);

/*
 * mla_prolog_get_workspace_size / mla_prolog -- the "MlaProlog" operator
 * (cann-recipes-infer operator notes: formula section, parameter and return
 * lists, constraints), non-quantised. From hidden states x it computes
 *     c^Q = RmsNorm(x . wq_a) * gamma_cq
 *     q   = RmsNorm(c^Q . wq_b), over each head's head_dim values, weight 1
 *     kv  = RmsNorm(x . wkv) * gamma_ckv
 * and then rotates the last rope_dim values of every q head and of kv with the
 * interleaved rope: elements 2i and 2i + 1 of that slice become
 *     x[2i] cos[2i] - x[2i+1] sin[2i],   x[2i+1] cos[2i+1] + x[2i] sin[2i+1]
 * with cos / sin taken from the token's row of rope_cos / rope_sin. RmsNorm(y)
 * = y / sqrt(mean(y^2) + eps). The page documents the int8 variant (int8
 * wq_b with a per-column scale, int8 c^Q with a per-token scale) and leaves
 * the non-quantised one to an example: here wq_b is bf16 and the third output
 * is c^Q in bf16.
 *
 *   token_x     device bf16 [t, h]
 *   wq_a        device bf16 [h, q_lora_rank]                (row-major, "ND")
 *   wq_b        device bf16 [q_lora_rank, num_heads * head_dim]
 *   wkv         device bf16 [h, head_dim]
 *   rope_cos    device bf16 [t, rope_dim]
 *   rope_sin    device bf16 [t, rope_dim]
 *   gamma_cq    device bf16 [q_lora_rank]
 *   gamma_ckv   device bf16 [head_dim]
 *   eps         RmsNorm epsilon (the page gives none; 1e-6 is customary), > 0
 *   q_out       device bf16 [t, num_heads, head_dim] or [t, num_heads * head_dim]
 *   kv_out      device bf16 [t, head_dim]
 *   qr_out      device bf16 [t, q_lora_rank]: c^Q
 *   workspace_size  out: bytes of device workspace mla_prolog needs: the
 *               fp32 product x . wq_a before its norm (t * q_lora_rank * 4,
 *               rounded up to 256 bytes), then copies of wq_a, wkv and wq_b
 *               rearranged for the product kernel (2 bytes per weight, each
 *               rounded up to 256 bytes), then, when x . [wq_a | wkv] has
 *               fewer than 128 tiles of 128 rows x 512 columns and is split
 *               over K into S runs (S the smallest divisor of h / 128 that
 *               brings S * tiles to 128, or h / 128), the runs' fp32 sums
 *               (S * t * (q_lora_rank + 512) * 4 bytes, rounded up to 256);
 *               0 when t = 0.
 * Supported (the page's constraints fix head_dim 512, h 4096, q_lora_rank
 * 1024, num_heads 64, rope_dim 64, t up to 64k): head_dim = 512,
 * rope_dim = 64, h a multiple of 128, q_lora_rank a multiple of 512, any
 * num_heads >= 1 and t >= 0; other sizes return MLA_ERR_UNSUPPORTED.
 * num_heads is read from wq_b's width. Outputs are rounded to nearest even
 * from fp32; products accumulate in fp32; c^Q is rounded to bf16 before it
 * enters the second product.
 * mla_prolog enqueues six kernels on stream (the rearrangements of wq_a and
 * of wkv, x . [wq_a | wkv] with the kv epilogue, the c^Q norm, the
 * rearrangement of wq_b, c^Q . wq_b with the q epilogue), and a seventh
 * that adds the runs of a split first product and applies its epilogues.
 * The result then differs from an unsplit call only by rounding. The workspace
 * (16-byte aligned, at least the planned size) must stay untouched until they
 * have run. Errors as for mla_prefill.
 */
int mla_prolog_get_workspace_size(const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
                                  const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                                  const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, float eps,
                                  const mla_tensor *q_out, const mla_tensor *kv_out, const mla_tensor *qr_out,
                                  uint64_t *workspace_size);
int mla_prolog(const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
               const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
               const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, float eps, const mla_tensor *q_out,
               const mla_tensor *kv_out, const mla_tensor *qr_out, void *workspace, uint64_t workspace_size,
               void *stream);

/*
 * mla_prolog_quant_get_workspace_size / mla_prolog_quant -- the quantised
 * "MlaProlog" operator (cann-recipes-infer operator notes: the prototype
 * mla_prolog_quant, formula section, parameter and return lists,
 * constraints). As mla_prolog, except that wq_b is int8 with a per-column
 * dequantisation scale and c^Q leaves as int8 codes with a per-token scale:
 *     c^Q     = RmsNorm(x . wq_a) * gamma_cq                  (fp32)
 *     s[t]    = max |c^Q[t, :]| / 127
 *     qr[t,k] = c^Q[t,k] / s[t] rounded to nearest, ties to even (|qr| <= 127)
 *     q       = RmsNorm((qr . wq_b)[t, n] * s[t] * wq_b_scale[n]), per head, weight 1
 *     kv      = RmsNorm(x . wkv) * gamma_ckv
 * then the interleaved rope on the last rope_dim values of every q head and
 * of kv, as in mla_prolog. The page names qr_out and qr_scale_out and their
 * types but not the rounding rule or the scale's form: the symmetric
 * max / 127 scale with c^Q ~ qr_out * qr_scale_out and ties to even is the
 * reading taken; a row of zeros gets scale 0 and codes 0. qr . wq_b is exact
 * (int32 accumulation).
 *
 *   token_x, wq_a, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps,
 *   q_out, kv_out     as for mla_prolog
 *   wq_b          device int8 [q_lora_rank, num_heads * head_dim]
 *   wq_b_scale    device fp32 [num_heads * head_dim, 1] or [num_heads * head_dim]
 *   qr_out        device int8 [t, q_lora_rank]: the codes of c^Q
 *   qr_scale_out  device fp32 [t, 1] or [t]: the per-token scale s
 *   workspace_size  out: bytes of device workspace mla_prolog_quant needs:
 *               t * q_lora_rank * 4 for x . wq_a, then the rearranged copies
 *               of wq_a and wkv (2 bytes per weight) and of wq_b (1 byte per
 *               weight), then the split first product's sums as for
 *               mla_prolog, each rounded up to 256 bytes; 0 when t = 0.
 * Supported: as mla_prolog, with q_lora_rank one of 512, 1024, 1536, 2048
 * (the page fixes 1024). mla_prolog_quant enqueues six kernels on stream
 * (the rearrangements of wq_a and wkv, x . [wq_a | wkv] with the kv
 * epilogue, the c^Q norm and quantisation, the rearrangement of wq_b, and
 * qr . wq_b with the dequantisation, per-head norm and rope epilogue), and
 * the sum of a split first product as mla_prolog does; the workspace must
 * stay valid until they have run. Errors as for mla_prefill.
 */
int mla_prolog_quant_get_workspace_size(const mla_tensor *token_x, const mla_tensor *wq_a,
                                        const mla_tensor *wq_b, const mla_tensor *wkv,
                                        const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                                        const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv,
                                        const mla_tensor *wq_b_scale, float eps, const mla_tensor *q_out,
                                        const mla_tensor *kv_out, const mla_tensor *qr_out,
                                        const mla_tensor *qr_scale_out, uint64_t *workspace_size);
int mla_prolog_quant(const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
                     const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                     const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, const mla_tensor *wq_b_scale,
                     float eps, const mla_tensor *q_out, const mla_tensor *kv_out, const mla_tensor *qr_out,
                     const mla_tensor *qr_scale_out, void *workspace, uint64_t workspace_size, void *stream);

/*
 * Prolog weights packed once -- for callers that run the prolog many times
 * with the same weights (every inference deployment). mla_prolog and
 * mla_prolog_quant rearrange wq_a, wkv and wq_b into the product kernel's
 * stage layout on every call (a third of a call at 64 tokens, 2-3% at
 * 16384); these entry points do it once.
 *
 *   mla_prolog_weights_size  host only: *packed_size = bytes of the packed
 *       weights: the rearranged copies of wq_a [h, q_lora_rank] and wkv
 *       [h, 512] (2 bytes per weight) and of wq_b [q_lora_rank, num_heads *
 *       512] (2 bytes per weight in bf16, 1 in int8), each rounded up to 256
 *       bytes. Shapes, dtypes and supported sizes as for mla_prolog (wq_b
 *       int8 selects the quantised layout).
 *   mla_prolog_pack_weights  enqueues the rearrangement into packed (device,
 *       16-byte aligned, at least *packed_size bytes, owned by the caller) on
 *       stream. The packed buffer depends only on the weights: it stays
 *       valid for any number of calls while the weights are unchanged.
 *   mla_prolog_prepacked_workspace_size  host only: the workspace of the two
 *       prepacked operators for token_x [t, h] and wq_a [h, q_lora_rank]:
 *       t * q_lora_rank * 4 bytes for x . wq_a, then the split first
 *       product's sums as for mla_prolog, each rounded up to 256; 0 when
 *       t = 0.
 *   mla_prolog_prepacked / mla_prolog_quant_prepacked  as mla_prolog /
 *       mla_prolog_quant with the same arguments, plus the packed buffer of
 *       these weights (packed_size bytes); the weight descriptors are still
 *       validated, their data is not read. Outputs equal those of the
 *       packing operators bit for bit. Errors as for mla_prolog, and
 *       MLA_ERR_WORKSPACE for a packed buffer smaller than the weights need.
 */
int mla_prolog_weights_size(const mla_tensor *wq_a, const mla_tensor *wq_b, const mla_tensor *wkv,
                            uint64_t *packed_size);
int mla_prolog_pack_weights(const mla_tensor *wq_a, const mla_tensor *wq_b, const mla_tensor *wkv, void *packed,
                            uint64_t packed_size, void *stream);
int mla_prolog_prepacked_workspace_size(const mla_tensor *token_x, const mla_tensor *wq_a,
                                        uint64_t *workspace_size);
int mla_prolog_prepacked(const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
                         const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                         const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, float eps, const mla_tensor *q_out,
                         const mla_tensor *kv_out, const mla_tensor *qr_out, const void *packed,
                         uint64_t packed_size, void *workspace, uint64_t workspace_size, void *stream);
int mla_prolog_quant_prepacked(const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
                               const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                               const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, const mla_tensor *wq_b_scale,
                               float eps, const mla_tensor *q_out, const mla_tensor *kv_out,
                               const mla_tensor *qr_out, const mla_tensor *qr_scale_out, const void *packed,
                               uint64_t packed_size, void *workspace, uint64_t workspace_size, void *stream);

/* Message describing the last failed call on this thread ("" if none). */
const char *mla_last_error(void);

/*
 * mla_prefill_plan_host -- host-only view of the work list mla_prefill builds,
 * for inspection and tests. No HIP call. (mla_prefill folds each task with its
 * item and batch record into one 32-byte launch record per workgroup, which
 * is what its workspace holds.) Writes, into buf (host memory of buf_size
 * bytes), three arrays each starting on a 256-byte boundary:
 *   batch records  {q_offset, kv_offset, q_len, kv_len}  int32 x 4, batch of them
 *   work items     {batch, first_q_row, kv_tiles, q_rows} int32 x 4, *n_items of them
 *   tasks          {item, first_head, first_tile, end_tile} int32 x 4, *n_tasks of them
 * A task runs P = MLA_PLAN_Q_ROWS / q_rows query heads, first_head ..
 * first_head + P - 1, which share one KV head: P is the largest power of two
 * up to 8 that divides head_num / kv_head_num (1 without head grouping). One
 * work item covers q_rows = MLA_PLAN_Q_ROWS / P query rows of a sequence;
 * kv_tiles counts the tiles of MLA_PLAN_KV_COLS keys (from key 0) those rows
 * can see. A task covers the item's tiles [first_tile, end_tile): all of
 * them, or one run of an item that mla_prefill splits (see there). Task i is
 * the work of workgroup i of the launch (item -1: an empty padding task).
 * kv_padded_max_seq: 0 for packed K/V, else max_seq of the padded layout.
 * Returns MLA_ERR_WORKSPACE if buf is too small, MLA_ERR_VALUE for bad
 * lengths or head counts.
 */
#define MLA_PLAN_Q_ROWS 256
#define MLA_PLAN_KV_COLS 64
int mla_prefill_plan_host(const int32_t *q_seqlen, const int32_t *kv_seqlen, int32_t batch,
                          int32_t head_num, int32_t kv_head_num, int32_t mask_type,
                          int64_t kv_padded_max_seq, void *buf, uint64_t buf_size,
                          int32_t *n_items, int32_t *n_tasks);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PREFILL_H */
