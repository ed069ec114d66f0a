// C ABI of the MLA varlen-prefill library: argument validation, the host work
// planner, and the launches. Operations and argument meanings follow the
// Ascend Transformer Boost C API pages "MLA Prefill" and
// "PagedCacheLoadOperation" (Definition and Members tables).
#include "mla_prefill.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

using mla::FWD_BM;
using mla::FWD_BN;
using mla::MASK_TILE;
using mla::ROPE_DIM;
using mla::SeqRec;
using mla::MLA_CUS_PER_XCD;
using mla::MLA_XCDS;
using mla::PAGED_MAX_TILES;
using mla::MergeRec;
using mla::PART_ROWS;
using mla::Task;
using mla::WorkItem;

#ifndef MLA_PLAN_BATCH_TASKS
#define MLA_PLAN_BATCH_TASKS (2 * MLA_CUS_PER_XCD)
#endif
constexpr int PLAN_BATCH_TASKS = MLA_PLAN_BATCH_TASKS;  // minimum tasks per launch-order batch of an XCD queue
#ifndef MLA_PLAN_EVEN_BATCH_TASKS
#define MLA_PLAN_EVEN_BATCH_TASKS (MLA_CUS_PER_XCD / 2)
#endif
constexpr int PLAN_EVEN_BATCH_TASKS = MLA_PLAN_EVEN_BATCH_TASKS;  // the same when the tasks are about equal
#ifndef MLA_SPLIT_MIN_TILES
#define MLA_SPLIT_MIN_TILES 16
#endif
constexpr int32_t SPLIT_MIN_TILES = MLA_SPLIT_MIN_TILES;  // no piece of a split item is cut shorter than this
#ifndef MLA_SPLIT_SHARE_PERCENT
#define MLA_SPLIT_SHARE_PERCENT 100
#endif
constexpr int64_t SPLIT_SHARE_PERCENT = MLA_SPLIT_SHARE_PERCENT;  // longest run, in percent of the even share
constexpr int64_t TASK_FIXED_TILES = 2;  // a workgroup's fixed work (Q load, pipeline fill, epilogue) in tiles
#ifndef MLA_MAX_PACK_SHIFT
#define MLA_MAX_PACK_SHIFT 3
#endif
static_assert(MLA_MAX_PACK_SHIFT >= 0 && MLA_MAX_PACK_SHIFT <= mla::FWD_MAX_PACK_SHIFT, "at most 8 heads per task");
static_assert(MLA_PLAN_Q_ROWS == FWD_BM, "plan row count must match the kernel tile");
static_assert(MLA_PLAN_KV_COLS == FWD_BN, "plan key count must match the kernel tile");
static_assert(MLA_PAGED_MAX_KEYS == PAGED_MAX_TILES * FWD_BN, "paged key limit must match the kernel table");

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return MLA_OK;
}

int64_t numel(const mla_tensor *t) {
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
    return n;
}

size_t elem_size(int dtype) {
    switch (dtype) {
        case MLA_FP16:
        case MLA_BF16: return 2;
        case MLA_INT8: return 1;
        case MLA_INT32:
        case MLA_FP32: return 4;
        default: return 0;
    }
}

// Structural checks shared by every tensor argument.
int check_tensor(const mla_tensor *t, const char *name, bool device) {
    if (t == nullptr) return fail(MLA_ERR_NULL, "%s: descriptor is NULL", name);
    if (t->ndim < 1 || t->ndim > 4) return fail(MLA_ERR_SHAPE, "%s: ndim %d not in 1..4", name, t->ndim);
    for (int i = 0; i < t->ndim; ++i)
        if (t->shape[i] < 0) return fail(MLA_ERR_SHAPE, "%s: negative extent", name);
    if (elem_size(t->dtype) == 0) return fail(MLA_ERR_DTYPE, "%s: unknown dtype code %d", name, t->dtype);
    if (numel(t) > 0 && t->data == nullptr) return fail(MLA_ERR_NULL, "%s: data is NULL", name);
    if (device && numel(t) > 0 && (reinterpret_cast<uintptr_t>(t->data) & 15) != 0)
        return fail(MLA_ERR_VALUE, "%s: device data must be 16-byte aligned", name);
    return MLA_OK;
}

bool is_half(int dtype) { return dtype == MLA_FP16 || dtype == MLA_BF16; }

// [n, heads * dim] or [n, heads, dim]; returns dim through *dim_out (0 if the
// shape does not fit).
bool token_head_shape(const mla_tensor *t, int64_t heads, int64_t *n_out, int64_t *dim_out) {
    if (t->ndim == 3 && t->shape[1] == heads) {
        *n_out = t->shape[0];
        *dim_out = t->shape[2];
        return true;
    }
    if (t->ndim == 2 && heads > 0 && t->shape[1] % heads == 0) {
        *n_out = t->shape[0];
        *dim_out = t->shape[1] / heads;
        return true;
    }
    return false;
}

struct Problem {
    int dtype = 0;
    int32_t batch = 0;
    int32_t heads = 0;
    int32_t kv_heads = 0;
    int64_t n_q = 0;
    int64_t n_kv = 0;
    int64_t kv_padded_max_seq = 0;  // 0: packed
    int mask_type = 0;
    int mask_dtype = 0;
    int64_t head_dim = 0;  // embeddimV
    const int32_t *q_seqlen = nullptr;
    const int32_t *kv_seqlen = nullptr;
};

// KV tensor layout: packed [sum kv, Hkv, dim] or padded [batch, max_seq, Hkv * dim].
int kv_layout(const mla_tensor *t, const char *name, const Problem &pr, int64_t dim, int32_t max_kv,
              int64_t *padded_max_seq) {
    if (t->ndim != 3) return fail(MLA_ERR_SHAPE, "%s: expected 3 dimensions", name);
    if (t->shape[0] == pr.n_kv && t->shape[1] == pr.kv_heads && t->shape[2] == dim) {
        *padded_max_seq = 0;
        return MLA_OK;
    }
    if (t->shape[0] == pr.batch && t->shape[2] == (int64_t)pr.kv_heads * dim && t->shape[1] >= max_kv) {
        *padded_max_seq = t->shape[1];
        return MLA_OK;
    }
    return fail(MLA_ERR_SHAPE,
                "%s: shape must be packed [%lld, %d, %lld] or padded [%d, max_seq >= %d, %lld]", name,
                (long long)pr.n_kv, pr.kv_heads, (long long)dim, pr.batch, max_kv,
                (long long)pr.kv_heads * dim);
}

int validate_prefill(const mla_tensor *q, const mla_tensor *q_rope, const mla_tensor *k,
                     const mla_tensor *k_rope, const mla_tensor *v, const mla_tensor *q_seqlen,
                     const mla_tensor *kv_seqlen, const mla_tensor *mask, int32_t head_num,
                     float qk_scale, int32_t kv_head_num, int32_t mask_type, uint8_t cache_mode,
                     const mla_tensor *out, Problem *pr) {
    int rc;
    if ((rc = check_tensor(q, "q", true)) || (rc = check_tensor(q_rope, "q_rope", true)) ||
        (rc = check_tensor(k, "k", true)) || (rc = check_tensor(k_rope, "k_rope", true)) ||
        (rc = check_tensor(v, "v", true)) || (rc = check_tensor(q_seqlen, "q_seqlen", false)) ||
        (rc = check_tensor(kv_seqlen, "kv_seqlen", false)) ||
        (rc = check_tensor(out, "atten_out", true)))
        return rc;
    if (head_num <= 0) return fail(MLA_ERR_VALUE, "headNum must be > 0 (got %d)", head_num);
    if (kv_head_num <= 0) return fail(MLA_ERR_VALUE, "kvHeadNum must be > 0 (got %d)", kv_head_num);
    if (head_num % kv_head_num != 0)
        return fail(MLA_ERR_VALUE, "headNum %d is not a multiple of kvHeadNum %d", head_num, kv_head_num);
    if (!std::isfinite(qk_scale)) return fail(MLA_ERR_VALUE, "qkScale must be finite");
    if (mask_type < MLA_MASK_UNDEFINED || mask_type > MLA_MASK_FREE)
        return fail(MLA_ERR_VALUE, "maskType %d is not a known mask type", mask_type);
    if (cache_mode != 0)
        return fail(MLA_ERR_UNSUPPORTED, "cacheMode %d: only 0 (contiguous K/V) is implemented", cache_mode);

    // dtypes
    if (!is_half(q->dtype)) return fail(MLA_ERR_DTYPE, "q: dtype must be fp16 or bf16");
    const mla_tensor *same[] = {q_rope, k, k_rope, v, out};
    const char *same_names[] = {"q_rope", "k", "k_rope", "v", "atten_out"};
    for (int i = 0; i < 5; ++i)
        if (same[i]->dtype != q->dtype) return fail(MLA_ERR_DTYPE, "%s: dtype differs from q", same_names[i]);
    if (q_seqlen->dtype != MLA_INT32 || kv_seqlen->dtype != MLA_INT32)
        return fail(MLA_ERR_DTYPE, "q_seqlen / kv_seqlen must be int32");

    // lengths
    if (q_seqlen->ndim != 1 || kv_seqlen->ndim != 1 || q_seqlen->shape[0] != kv_seqlen->shape[0])
        return fail(MLA_ERR_SHAPE, "q_seqlen and kv_seqlen must both be [batch]");
    if (q_seqlen->shape[0] > INT32_MAX) return fail(MLA_ERR_VALUE, "batch too large");
    pr->batch = (int32_t)q_seqlen->shape[0];
    pr->heads = head_num;
    pr->kv_heads = kv_head_num;
    pr->dtype = q->dtype;
    pr->mask_type = mask_type;
    pr->q_seqlen = static_cast<const int32_t *>(q_seqlen->data);
    pr->kv_seqlen = static_cast<const int32_t *>(kv_seqlen->data);
    int64_t sum_q = 0, sum_kv = 0;
    int32_t max_kv = 0;
    for (int32_t b = 0; b < pr->batch; ++b) {
        int32_t ql = pr->q_seqlen[b], kl = pr->kv_seqlen[b];
        if (ql < 0 || kl < 0) return fail(MLA_ERR_VALUE, "sequence %d has a negative length", b);
        sum_q += ql;
        sum_kv += kl;
        max_kv = std::max(max_kv, kl);
    }
    if (sum_q > INT32_MAX || sum_kv > INT32_MAX)
        return fail(MLA_ERR_VALUE, "total tokens exceed 2^31 - 1");
    pr->n_q = sum_q;
    pr->n_kv = sum_kv;

    // Q, QRope, attenOut
    int64_t nq, dq, nqr, dqr, no, dout;
    if (!token_head_shape(q, head_num, &nq, &dq))
        return fail(MLA_ERR_SHAPE, "q: expected [nTokens, headNum*D] or [nTokens, headNum, D]");
    if (!token_head_shape(q_rope, head_num, &nqr, &dqr))
        return fail(MLA_ERR_SHAPE, "q_rope: expected [nTokens, headNum*64] or [nTokens, headNum, 64]");
    if (!token_head_shape(out, head_num, &no, &dout))
        return fail(MLA_ERR_SHAPE, "atten_out: expected [nTokens, headNum*D] or [nTokens, headNum, D]");
    if (nq != sum_q || nqr != sum_q || no != sum_q)
        return fail(MLA_ERR_SHAPE, "q / q_rope / atten_out rows must equal sum(qSeqLen) = %lld",
                    (long long)sum_q);
    if (dqr != ROPE_DIM) return fail(MLA_ERR_SHAPE, "q_rope: rope dimension must be 64 (got %lld)", (long long)dqr);
    if (dout != dq) return fail(MLA_ERR_SHAPE, "atten_out: head dimension %lld differs from q's %lld",
                                (long long)dout, (long long)dq);

    // K, KRope, V share one layout
    int64_t pad_k, pad_kr, pad_v;
    if ((rc = kv_layout(k, "k", *pr, dq, max_kv, &pad_k)) ||
        (rc = kv_layout(k_rope, "k_rope", *pr, ROPE_DIM, max_kv, &pad_kr)) ||
        (rc = kv_layout(v, "v", *pr, dq, max_kv, &pad_v)))
        return rc;
    if (pad_k != pad_kr || pad_k != pad_v)
        return fail(MLA_ERR_SHAPE, "k, k_rope and v must share one layout (packed or padded)");
    pr->kv_padded_max_seq = pad_k;
    if (pad_k && (int64_t)pr->batch * pad_k > INT32_MAX)
        return fail(MLA_ERR_VALUE, "padded K/V rows exceed 2^31 - 1");

    if (mask_type == MLA_MASK_FREE) {
        if (mask == nullptr) return fail(MLA_ERR_NULL, "mask: required for MASK_FREE");
        if ((rc = check_tensor(mask, "mask", true))) return rc;
        if (!is_half(mask->dtype)) return fail(MLA_ERR_DTYPE, "mask: dtype must be fp16 or bf16");
        if (mask->ndim != 2 || mask->shape[0] != MASK_TILE || mask->shape[1] != MASK_TILE)
            return fail(MLA_ERR_SHAPE, "mask: expected [512, 512]");
        pr->mask_dtype = mask->dtype;
    }
    if (dq != 64 && dq != 128)
        return fail(MLA_ERR_UNSUPPORTED, "embeddimV %lld: the kernel implements 64 and 128", (long long)dq);
    pr->head_dim = dq;
    if ((int64_t)head_num > 65535) return fail(MLA_ERR_UNSUPPORTED, "headNum above 65535");
    return MLA_OK;
}

// Paged K/V: ND caches [num_blocks, block_size, Hkv, dim] and a device block
// table [batch, max_blocks]. Q, lengths, mask and output are checked as for
// the contiguous form (through validate_prefill with stand-in K/V
// descriptors of the packed shape).
struct PagedProblem {
    int64_t num_blocks = 0;
    int64_t block_size = 0;
    int64_t bt_stride = 0;
};

int validate_paged(const mla_tensor *q, const mla_tensor *q_rope, const mla_tensor *key_cache,
                   const mla_tensor *krope_cache, const mla_tensor *value_cache,
                   const mla_tensor *block_tables, const mla_tensor *q_seqlen,
                   const mla_tensor *kv_seqlen, const mla_tensor *mask, int32_t head_num, float qk_scale,
                   int32_t kv_head_num, int32_t mask_type, const mla_tensor *out, Problem *pr,
                   PagedProblem *pg) {
    int rc;
    if ((rc = check_tensor(key_cache, "key_cache", true)) ||
        (rc = check_tensor(krope_cache, "krope_cache", true)) ||
        (rc = check_tensor(value_cache, "value_cache", true)) ||
        (rc = check_tensor(block_tables, "block_tables", true)) ||
        (rc = check_tensor(kv_seqlen, "kv_seqlen", false)))
        return rc;
    if (kv_seqlen->ndim != 1) return fail(MLA_ERR_SHAPE, "kv_seqlen must be [batch]");
    if (kv_seqlen->dtype != MLA_INT32) return fail(MLA_ERR_DTYPE, "q_seqlen / kv_seqlen must be int32");
    int64_t sum_kv = 0;
    for (int64_t b = 0; b < kv_seqlen->shape[0]; ++b) sum_kv += std::max(0, static_cast<const int32_t *>(kv_seqlen->data)[b]);
    // stand-in descriptors of the packed shape: the shared checks then apply
    mla_tensor k = *key_cache, kr = *krope_cache, v = *value_cache;
    k.ndim = kr.ndim = v.ndim = 3;
    k.shape[0] = kr.shape[0] = v.shape[0] = sum_kv;
    k.shape[1] = kr.shape[1] = v.shape[1] = kv_head_num;
    k.shape[2] = key_cache->shape[key_cache->ndim - 1];
    kr.shape[2] = krope_cache->shape[krope_cache->ndim - 1];
    v.shape[2] = value_cache->shape[value_cache->ndim - 1];
    if ((rc = validate_prefill(q, q_rope, &k, &kr, &v, q_seqlen, kv_seqlen, mask, head_num, qk_scale, kv_head_num,
                               mask_type, 0, out, pr)))
        return rc;
    if (pr->kv_padded_max_seq != 0) return fail(MLA_ERR_SHAPE, "caches: unexpected shape");
    const mla_tensor *caches[] = {key_cache, krope_cache, value_cache};
    const char *names[] = {"key_cache", "krope_cache", "value_cache"};
    const int64_t dims[] = {pr->head_dim, ROPE_DIM, pr->head_dim};
    for (int i = 0; i < 3; ++i) {
        const mla_tensor *c = caches[i];
        if (c->ndim != 4 || c->shape[2] != kv_head_num || c->shape[3] != dims[i] ||
            c->shape[0] != key_cache->shape[0] || c->shape[1] != key_cache->shape[1])
            return fail(MLA_ERR_SHAPE, "%s: expected ND [num_blocks, block_size, %d, %lld] like key_cache", names[i],
                        kv_head_num, (long long)dims[i]);
    }
    pg->num_blocks = key_cache->shape[0];
    pg->block_size = key_cache->shape[1];
    if (pg->num_blocks <= 0 || pg->block_size <= 0) return fail(MLA_ERR_SHAPE, "caches: empty");
    if (pg->block_size % FWD_BN != 0)
        return fail(MLA_ERR_UNSUPPORTED, "block_size %lld: the fused path needs a multiple of %d",
                    (long long)pg->block_size, FWD_BN);
    if (pg->num_blocks * pg->block_size > INT32_MAX)
        return fail(MLA_ERR_UNSUPPORTED, "caches of more than 2^31 - 1 token slots");
    if (block_tables->dtype != MLA_INT32) return fail(MLA_ERR_DTYPE, "block_tables must be int32");
    if (pr->batch > (1 << mla::PAGED_SEQ_BITS))
        return fail(MLA_ERR_UNSUPPORTED, "batch %d: the fused path takes at most %d sequences", pr->batch,
                    1 << mla::PAGED_SEQ_BITS);
    if (block_tables->ndim != 2 || block_tables->shape[0] != pr->batch)
        return fail(MLA_ERR_SHAPE, "block_tables: expected [batch = %d, max_blocks]", pr->batch);
    pg->bt_stride = block_tables->shape[1];
    if (pg->bt_stride > INT32_MAX) return fail(MLA_ERR_SHAPE, "block_tables: too many columns");
    for (int32_t b = 0; b < pr->batch; ++b) {
        const int64_t kl = pr->kv_seqlen[b];
        if ((kl + pg->block_size - 1) / pg->block_size > pg->bt_stride)
            return fail(MLA_ERR_SHAPE, "block_tables: sequence %d needs %lld blocks, the table has %lld columns", b,
                        (long long)((kl + pg->block_size - 1) / pg->block_size), (long long)pg->bt_stride);
        if ((kl + FWD_BN - 1) / FWD_BN > PAGED_MAX_TILES)
            return fail(MLA_ERR_UNSUPPORTED, "sequence %d: %lld keys exceed the fused path's %d", b, (long long)kl,
                        PAGED_MAX_TILES * FWD_BN);
    }
    return MLA_OK;
}

// Number of FWD_BN-key tiles (counted from key 0) that query rows
// [q_row0, q_end) of a sequence can see under mask_type.
int32_t visible_tiles(int mask_type, int32_t q_len, int32_t kv_len, int32_t q_end) {
    int64_t visible;
    int64_t p_last = (int64_t)kv_len - q_len + q_end - 1;  // key position of the last row
    switch (mask_type) {
        case MLA_MASK_UNDEFINED: visible = kv_len; break;
        case MLA_MASK_SPEC:
        case MLA_MASK_CAUSAL: visible = std::min<int64_t>(kv_len, std::max<int64_t>(p_last + 1, 0)); break;
        default:  // MLA_MASK_FREE: every key up to the end of the last row's 512-block
            visible = p_last < 0 ? 0 : std::min<int64_t>(kv_len, (p_last / MASK_TILE + 1) * MASK_TILE);
    }
    return (int32_t)((visible + FWD_BN - 1) / FWD_BN);
}

// Relative cost of a task over key tiles [kt0, kt1): its tiles plus one for
// the fixed per-workgroup work (Q load, pipeline fill, epilogue).
int64_t tiles_work(int32_t kt0, int32_t kt1) { return (int64_t)(kt1 - kt0) + 1; }

// A run of key tiles [kt0, kt1) of one work item; piece k of n of the item
// (n = 1: the whole item).
struct Piece {
    int32_t item, kt0, kt1, k, n;
};

struct Plan {
    std::vector<SeqRec> seqs;
    std::vector<WorkItem> items;
    std::vector<Task> tasks;  // one per workgroup, in launch order
    std::vector<MergeRec> merges;  // one per (split item, head pack)
    int32_t n_parts = 0;           // partial slots of the split tasks
    bool mask_free = false;        // MASK_FREE: the workspace may end with the tile's classes
};

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// Host view of the work list (mla_prefill_plan_host): batch records, items,
// tasks {item, first head, first tile, end tile}, each array on a 256-byte
// boundary.
constexpr uint64_t VIEW_TASK_BYTES = 16;
uint64_t items_offset(const Plan &p) { return align256(p.seqs.size() * sizeof(SeqRec)); }
uint64_t tasks_offset(const Plan &p) { return items_offset(p) + align256(p.items.size() * sizeof(WorkItem)); }

uint64_t view_bytes(const Plan &p) {
    if (p.items.empty()) return 0;
    return tasks_offset(p) + p.tasks.size() * VIEW_TASK_BYTES;
}

// Device workspace: one LaunchRec per workgroup; with split items, then the
// merge records, the partial log-sum-exps and the partial rows, each on a
// 256-byte boundary.
uint64_t merges_offset(const Plan &p) { return align256(p.tasks.size() * sizeof(mla::LaunchRec)); }
uint64_t lse_offset(const Plan &p) { return merges_offset(p) + align256(p.merges.size() * sizeof(MergeRec)); }
uint64_t part_o_offset(const Plan &p) { return lse_offset(p) + align256((uint64_t)p.n_parts * PART_ROWS * 4); }
// bytes of the records copied from the host
uint64_t records_bytes(const Plan &p) {
    if (p.merges.empty()) return p.tasks.size() * sizeof(mla::LaunchRec);
    return merges_offset(p) + p.merges.size() * sizeof(MergeRec);
}
uint64_t plan_bytes_no_cls(const Plan &p, int64_t head_dim) {
    if (p.items.empty()) return 0;
    if (p.n_parts == 0) return records_bytes(p);
    return part_o_offset(p) + (uint64_t)p.n_parts * PART_ROWS * (uint64_t)head_dim * 4;
}
// MASK_FREE: the classes of the tile's 64-key row blocks (MASK_CLS_BYTES)
// follow, 256-byte aligned (not in mla_prefill_no_alloc's array: without
// them every diagonal-block tile takes the per-element path, with the same
// result bit for bit).
uint64_t cls_offset(const Plan &p, int64_t head_dim) { return align256(plan_bytes_no_cls(p, head_dim)); }
uint64_t plan_bytes(const Plan &p, int64_t head_dim, bool with_cls = true) {
    const uint64_t base = plan_bytes_no_cls(p, head_dim);
    if (base == 0 || !with_cls || !p.mask_free) return base;
    return cls_offset(p, head_dim) + mla::MASK_CLS_BYTES;
}

// log2 of the query heads one task runs: the largest power of two, at most
// 8, dividing the group size headNum / kvHeadNum. The heads of a task then
// share one KV head.
int32_t pack_shift_for(int32_t heads, int32_t kv_heads) {
    const int32_t group = kv_heads > 0 ? heads / kv_heads : 1;
    int32_t ps = 0;
    while (ps < MLA_MAX_PACK_SHIFT && group % (2 << ps) == 0) ++ps;
    return ps;
}

// Work list.
//  * Items: one per FWD_BM >> pack_shift query rows of each sequence, with the
//    number of key tiles its rows can see.
//  * Split items (allow_split: not in mla_prefill_no_alloc): when the launch holds
//    little work for the CUs -- few heads, few sequences -- the longest items
//    would set its duration alone. Let W be the work of all tasks (tiles plus
//    TASK_FIXED_TILES each) spread evenly over the CUs. If the longest item
//    has more than 1.5 W tiles, every item with more than
//    max(W, SPLIT_MIN_TILES) tiles is cut into runs of at most about that
//    many consecutive key tiles (at multiples of 512 keys under MASK_FREE,
//    so the tile's blocks stay aligned), each a task of its own. Such a task
//    writes its rows over its own keys with their log-sum-exp into a partial
//    slot, and a merge kernel combines the pieces of each (item, head pack)
//    afterwards. (The part runs at a power-limited clock: once every CU has
//    work, evening out the tasks mostly trades idle CUs for a lower clock,
//    and the partial rows and the merge cost more than they save. Measured
//    at 4096 causal rows: 8 heads 105 -> 80 us, 16 heads 129 -> 124 us, 24
//    heads 140 -> 170 us, so 24 heads, whose longest item is 1.2 W, is not
//    split.)
//  * Tasks: one workgroup each, a piece (or all) of an item for 2^pack_shift
//    consecutive query heads of one KV head (its rows of each of them).
//  * Launch order. Tasks that read the same K/V stream (same sequence and KV
//    head) form a group. Groups are dealt, heaviest first, to the XCD queue
//    with the least work so far. If that leaves an XCD more than 5% above the
//    mean (few KV heads, or one long sequence), groups holding more than 1/32
//    of the launch's work are cut into consecutive pieces of at most that
//    much and dealt again, so that every XCD gets a share. Block i of the
//    launch is taken from queue i % MLA_XCDS (the hardware hands consecutive
//    workgroups to consecutive XCDs). Each queue is cut into batches of whole
//    groups holding at least twice as many tasks as the XCD has CUs -- or
//    half as many when most of the work is in groups whose tasks are within
//    a factor 2 of each other -- and each batch is ordered heaviest task
//    first. The tasks of a
//    group thus run together on one XCD and share its L2 while they stream
//    the same keys, and the heaviest first order inside a batch keeps the
//    XCD's CUs evenly loaded to the end. Short queues are padded with empty
//    tasks.
void build_plan(const int32_t *q_seqlen, const int32_t *kv_seqlen, int32_t batch, int32_t heads,
                int32_t kv_heads, int mask_type, int64_t kv_padded_max_seq, bool allow_split, Plan *plan) {
    plan->seqs.resize(batch);
    plan->items.clear();
    plan->tasks.clear();
    plan->merges.clear();
    plan->n_parts = 0;
    plan->mask_free = mask_type == MLA_MASK_FREE;
    const int32_t group = kv_heads > 0 ? heads / kv_heads : 1;
    const int32_t ps = pack_shift_for(heads, kv_heads);
    const int32_t rows = FWD_BM >> ps;
    const int32_t tasks_per_item = group >> ps;
    std::vector<int32_t> seq_item_first(batch + 1, 0);  // items of sequence b: [seq_item_first[b], .. [b + 1])
    int64_t q_off = 0, kv_off = 0;
    for (int32_t b = 0; b < batch; ++b) {
        SeqRec &s = plan->seqs[b];
        s.q_off = (int32_t)q_off;
        s.kv_off = (int32_t)(kv_padded_max_seq ? (int64_t)b * kv_padded_max_seq : kv_off);
        s.q_len = q_seqlen[b];
        s.kv_len = kv_seqlen[b];
        q_off += s.q_len;
        kv_off += s.kv_len;
        seq_item_first[b] = (int32_t)plan->items.size();
        for (int32_t r = 0; r < s.q_len; r += rows) {
            int32_t q_end = std::min(s.q_len, r + rows);
            plan->items.push_back(WorkItem{b, r, visible_tiles(mask_type, s.q_len, s.kv_len, q_end), rows});
        }
    }
    seq_item_first[batch] = (int32_t)plan->items.size();
    // the longest run of key tiles a task may hold (rule above)
    int32_t cap = INT32_MAX;
    const int32_t gran = mask_type == MLA_MASK_FREE ? MASK_TILE / FWD_BN : 1;
    if (allow_split) {
        int64_t total = 0, longest = 0;
        for (const WorkItem &it : plan->items) {
            total += ((int64_t)it.kv_tiles + TASK_FIXED_TILES);
            longest = std::max<int64_t>(longest, it.kv_tiles);
        }
        total *= (int64_t)kv_heads * tasks_per_item;
        const int64_t cus = (int64_t)MLA_XCDS * MLA_CUS_PER_XCD;
        const int64_t share = (total + cus - 1) / cus;
        if (2 * longest > 3 * share)
            cap = (int32_t)std::min<int64_t>(INT32_MAX,
                                             std::max<int64_t>(SPLIT_MIN_TILES, share * SPLIT_SHARE_PERCENT / 100));
    }
    // pieces of each item, in item order (so each sequence's are consecutive)
    std::vector<Piece> pieces;
    std::vector<int32_t> seq_piece_first(batch + 1, 0);  // pieces of sequence b: [seq_piece_first[b], .. [b + 1])
    std::vector<int32_t> item_part_base(plan->items.size(), -1), item_pieces(plan->items.size(), 1);
    for (int32_t b = 0; b < batch; ++b) {
        seq_piece_first[b] = (int32_t)pieces.size();
        for (int32_t i = seq_item_first[b]; i < seq_item_first[b + 1]; ++i) {
            const int32_t nt = plan->items[i].kv_tiles;
            // cut points k * nt / n, rounded down to the granularity and kept increasing
            std::vector<int32_t> cuts{0};
            const int32_t want = nt > cap ? (nt + cap - 1) / cap : 1;
            for (int32_t k = 1; k < want; ++k) {
                const int32_t c = (int32_t)((int64_t)nt * k / want) / gran * gran;
                if (c > cuts.back() && c < nt) cuts.push_back(c);
            }
            cuts.push_back(nt);
            const int32_t n = (int32_t)cuts.size() - 1;
            item_pieces[i] = n;
            if (n > 1) {
                item_part_base[i] = plan->n_parts;
                plan->n_parts += n * kv_heads * tasks_per_item;
            }
            for (int32_t k = 0; k < n; ++k) pieces.push_back(Piece{i, cuts[k], cuts[k + 1], k, n});
        }
    }
    seq_piece_first[batch] = (int32_t)pieces.size();
    // merge records: (item, KV head, head pack) in the order of their partial slots
    for (int32_t i = 0; i < (int32_t)plan->items.size(); ++i) {
        if (item_part_base[i] < 0) continue;
        const WorkItem &it = plan->items[i];
        const SeqRec &sq = plan->seqs[it.b];
        const int32_t n = item_pieces[i];
        for (int32_t hk = 0; hk < kv_heads; ++hk)
            for (int32_t pk = 0; pk < tasks_per_item; ++pk) {
                MergeRec m{};
                m.part0 = item_part_base[i] + (hk * tasks_per_item + pk) * n;
                m.n_parts = n;
                m.head = hk * group + pk * (1 << ps);
                m.q_tok0 = sq.q_off + it.q_row0;
                m.q_left = sq.q_len - it.q_row0;
                plan->merges.push_back(m);
            }
    }
    // the task of group slot t (t < group's piece count * tasks_per_item)
    auto make_task = [&](int32_t b, int32_t hk, int32_t t) -> Task {
        const Piece &pc = pieces[seq_piece_first[b] + t / tasks_per_item];
        const int32_t pk = t % tasks_per_item;
        const int32_t part = pc.n > 1 ? item_part_base[pc.item] + (hk * tasks_per_item + pk) * pc.n + pc.k : -1;
        return Task{pc.item, hk * group + pk * (1 << ps), pc.kt0, pc.kt1, part};
    };
    auto slot_work = [&](int32_t b, int32_t t) -> int64_t {
        const Piece &pc = pieces[seq_piece_first[b] + t / tasks_per_item];
        return tiles_work(pc.kt0, pc.kt1);
    };
    struct Group {
        int64_t work;
        int32_t b, hk;
        int32_t t0, t1;  // tasks [t0, t1) of the group: task t = piece t / tasks_per_item, head pack t % tasks_per_item
    };
    std::vector<Group> groups;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t seq_work = 0;
        for (int32_t j = seq_piece_first[b]; j < seq_piece_first[b + 1]; ++j)
            seq_work += tiles_work(pieces[j].kt0, pieces[j].kt1);
        const int32_t n_tasks = (seq_piece_first[b + 1] - seq_piece_first[b]) * tasks_per_item;
        if (seq_work > 0)
            for (int32_t hk = 0; hk < kv_heads; ++hk) groups.push_back({seq_work * tasks_per_item, b, hk, 0, n_tasks});
    }
    std::vector<std::vector<Group>> xcd_groups;
    std::vector<int64_t> load;
    auto deal = [&]() {
        std::stable_sort(groups.begin(), groups.end(), [](const Group &x, const Group &y) { return x.work > y.work; });
        xcd_groups.assign(MLA_XCDS, {});
        load.assign(MLA_XCDS, 0);
        for (const Group &gr : groups) {
            const int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
            load[x] += gr.work;
            xcd_groups[x].push_back(gr);
        }
    };
    deal();
    int64_t total = 0;
    for (const Group &gr : groups) total += gr.work;
    // If some XCD got more than 5% above the mean (few KV streams, or one long
    // sequence), cut groups heavier than 1/32 of the total into consecutive
    // pieces and deal again.
    if (20 * MLA_XCDS * *std::max_element(load.begin(), load.end()) > 21 * total) {
        const int64_t gcap = std::max<int64_t>(1, (total + 4 * MLA_XCDS - 1) / (4 * MLA_XCDS));
        std::vector<Group> cut;
        for (const Group &gr : groups) {
            if (gr.work <= gcap) {
                cut.push_back(gr);
                continue;
            }
            Group piece{0, gr.b, gr.hk, gr.t0, gr.t0};
            for (int32_t t = gr.t0; t < gr.t1; ++t) {
                piece.work += slot_work(gr.b, t);
                piece.t1 = t + 1;
                if (piece.work >= gcap || t + 1 == gr.t1) {
                    cut.push_back(piece);
                    piece = Group{0, gr.b, gr.hk, t + 1, t + 1};
                }
            }
        }
        groups.swap(cut);
        deal();
    }
    // Batch size of the launch order (below). Large batches let the
    // heaviest-first order balance the CUs when a group's tasks differ a lot
    // in length (causal items over their own keys); when they are about
    // equal (query rows at the end of a long key range), balance comes by
    // itself and small batches keep fewer K/V streams in flight per XCD, so
    // more of them hit in its L2.
    size_t batch_tasks = PLAN_BATCH_TASKS;
    {
        int64_t uneven = 0, even = 0;
        for (const Group &gr : groups) {
            int64_t lo = INT64_MAX, hi = 0;
            for (int32_t t = gr.t0; t < gr.t1; ++t) {
                const int64_t w = slot_work(gr.b, t);
                lo = std::min(lo, w);
                hi = std::max(hi, w);
            }
            if (gr.t1 > gr.t0) (hi > 2 * lo ? uneven : even) += gr.work;
        }
        if (even > uneven) batch_tasks = PLAN_EVEN_BATCH_TASKS;
    }
    std::vector<std::vector<Task>> queue(MLA_XCDS);
    std::vector<Task> pending;
    for (int x = 0; x < MLA_XCDS; ++x) {
        auto flush = [&]() {
            std::stable_sort(pending.begin(), pending.end(), [&](const Task &u, const Task &v) {
                return tiles_work(u.kt0, u.kt1) > tiles_work(v.kt0, v.kt1);
            });
            queue[x].insert(queue[x].end(), pending.begin(), pending.end());
            pending.clear();
        };
        for (const Group &gr : xcd_groups[x]) {
            for (int32_t t = gr.t0; t < gr.t1; ++t) pending.push_back(make_task(gr.b, gr.hk, t));
            if (pending.size() >= batch_tasks) flush();
        }
        flush();
    }
    size_t longest = 0;
    for (const auto &q : queue) longest = std::max(longest, q.size());
    plan->tasks.assign(longest * MLA_XCDS, Task{-1, 0, 0, 0, -1});
    for (int x = 0; x < MLA_XCDS; ++x)
        for (size_t k = 0; k < queue[x].size(); ++k) plan->tasks[k * MLA_XCDS + x] = queue[x][k];
}

void write_plan_view(const Plan &p, uint8_t *dst) {
    std::memcpy(dst, p.seqs.data(), p.seqs.size() * sizeof(SeqRec));
    std::memcpy(dst + items_offset(p), p.items.data(), p.items.size() * sizeof(WorkItem));
    int32_t *t = reinterpret_cast<int32_t *>(dst + tasks_offset(p));
    for (const Task &x : p.tasks) {
        t[0] = x.item;
        t[1] = x.head;
        t[2] = x.kt0;
        t[3] = x.kt1;
        t += VIEW_TASK_BYTES / 4;
    }
}

// The launch records the kernel reads: each task with its item and sequence
// folded in. Paged K/V carry the sequence index (its block-table row) where
// contiguous K/V carry the row of the task's first key (pieces of a split
// item start at key kt0 * FWD_BN); paged K/V carry the sequence index with
// kt0 above it.
void write_launch(const Plan &p, int32_t group, bool paged, mla::LaunchRec *dst) {
    for (size_t i = 0; i < p.tasks.size(); ++i) {
        const Task &t = p.tasks[i];
        mla::LaunchRec r{};
        if (t.item < 0) {
            r.head = -1;
            r.part = -1;
        } else {
            const WorkItem &it = p.items[t.item];
            const SeqRec &sq = p.seqs[it.b];
            const int32_t k0 = t.kt0 * FWD_BN;
            r.q_tok0 = sq.q_off + it.q_row0;
            r.q_left = sq.q_len - it.q_row0;
            r.kv_tiles = t.kt1 - t.kt0;
            r.head = t.head;
            r.kv_head = t.head / group;
            r.kv_off = paged ? (it.b | (t.kt0 << mla::PAGED_SEQ_BITS)) : sq.kv_off + k0;
            r.kv_len = sq.kv_len - k0;
            r.part = t.part;
        }
        dst[i] = r;
    }
}

// Launch records of mla_prefill_no_alloc: a fixed array in device memory, one
// copy per GPU, held until the process ends. On the host the name `scratch`
// stands for a host-side stand-in, not a device address: host code only ever
// uses the address hipGetSymbolAddress returns for the current device.
static_assert(MLA_NO_ALLOC_WORKSPACE_BYTES % sizeof(mla::LaunchRec) == 0, "whole launch records");
static __device__ __align__(256) unsigned char scratch[MLA_NO_ALLOC_WORKSPACE_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};  // device address of `scratch`, per device ordinal

// The current device's copy of `scratch`; its address is looked up once per
// device, with that device current.
int scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
        return fail(MLA_ERR_UNSUPPORTED, "device ordinal %d beyond the %d this library tracks", dev,
                    SCRATCH_MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        if (ptr == nullptr) return fail(MLA_ERR_RUNTIME, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MLA_OK;
}

// Plan on the host, copy the work list into the workspace, launch. pg and
// block_tables are null for contiguous K/V. With use_scratch the workspace
// arguments are ignored and the work list goes into the current device's
// `scratch` array instead.
int plan_and_launch(const Problem &pr, const PagedProblem *pg, const int32_t *block_tables, const mla_tensor *q,
                    const mla_tensor *q_rope, const void *k, const void *k_rope, const void *v,
                    const mla_tensor *mask, float qk_scale, const mla_tensor *atten_out, void *workspace,
                    uint64_t workspace_size, bool use_scratch, void *stream) {
    // Items are split only where the workspace is the caller's (not the fixed
    // array of mla_prefill_no_alloc).
    Plan plan;
    build_plan(pr.q_seqlen, pr.kv_seqlen, pr.batch, pr.heads, pr.kv_heads, pr.mask_type, pr.kv_padded_max_seq,
               !use_scratch, &plan);
    const bool with_cls = !use_scratch && pr.mask_type == MLA_MASK_FREE;
    const uint64_t need = plan_bytes(plan, pr.head_dim, with_cls);
    if (need == 0) return ok();  // no query rows: nothing to write
    if (use_scratch) {
        if (need > MLA_NO_ALLOC_WORKSPACE_BYTES)
            return fail(MLA_ERR_WORKSPACE,
                        "the work list needs %llu bytes (%zu launch records); mla_prefill_no_alloc holds at most "
                        "%llu bytes: use mla_prefill with a workspace",
                        (unsigned long long)need, plan.tasks.size(), (unsigned long long)MLA_NO_ALLOC_WORKSPACE_BYTES);
        int rc = scratch_on_current_device(&workspace);
        if (rc) return rc;
        workspace_size = MLA_NO_ALLOC_WORKSPACE_BYTES;
    }
    if (workspace == nullptr || workspace_size < need)
        return fail(MLA_ERR_WORKSPACE, "workspace of %llu bytes needed, %llu given",
                    (unsigned long long)need, (unsigned long long)workspace_size);
    if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
        return fail(MLA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (plan.tasks.size() > (size_t)INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "too many work items");

    const uint64_t rec_bytes = records_bytes(plan);
    std::vector<uint8_t> host(rec_bytes);
    write_launch(plan, pr.heads / pr.kv_heads, pg != nullptr, reinterpret_cast<mla::LaunchRec *>(host.data()));
    if (!plan.merges.empty())
        std::memcpy(host.data() + merges_offset(plan), plan.merges.data(), plan.merges.size() * sizeof(MergeRec));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(workspace, host.data(), rec_bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "hipMemcpyAsync: %s", hipGetErrorString(e));
    unsigned char *ws = static_cast<unsigned char *>(workspace);

    mla::FwdParams p{};
    p.q = q->data;
    p.q_rope = q_rope->data;
    p.k = k;
    p.k_rope = k_rope;
    p.v = v;
    p.mask = (pr.mask_type == MLA_MASK_FREE) ? mask->data : nullptr;
    if (with_cls) {
        uint8_t *cls = ws + cls_offset(plan, pr.head_dim);
        e = mla::launch_mask_classify(mask->data, mask->dtype == MLA_BF16 ? 1 : 0, cls, s);
        if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "mask tile classes: %s", hipGetErrorString(e));
        p.mask_cls = cls;
    }
    p.out = atten_out->data;
    p.launch = static_cast<const mla::LaunchRec *>(workspace);
    if (plan.n_parts > 0) {
        p.part_lse = reinterpret_cast<float *>(ws + lse_offset(plan));
        p.part_o = reinterpret_cast<float *>(ws + part_o_offset(plan));
    }
    p.heads = pr.heads;
    p.kv_heads = pr.kv_heads;
    p.group = pr.heads / pr.kv_heads;
    p.pack_shift = pack_shift_for(pr.heads, pr.kv_heads);
    p.head_dim = (int32_t)pr.head_dim;
    p.n_tasks = (int32_t)plan.tasks.size();
    p.mask_type = pr.mask_type;
    p.mask_is_bf16 = (pr.mask_type == MLA_MASK_FREE && mask->dtype == MLA_BF16) ? 1 : 0;
    p.qk_scale = qk_scale;
    if (pg) {
        p.block_tables = block_tables;
        p.bt_stride = (int32_t)pg->bt_stride;
        p.block_size = (int32_t)pg->block_size;
        p.num_blocks = (int32_t)pg->num_blocks;
    }
    e = mla::launch_mla_fwd(p, pr.dtype, pg != nullptr, s);
    if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "attention launch: %s", hipGetErrorString(e));
    if (!plan.merges.empty()) {
        mla::MergeParams mp{};
        mp.merges = reinterpret_cast<const MergeRec *>(ws + merges_offset(plan));
        mp.part_o = p.part_o;
        mp.part_lse = p.part_lse;
        mp.out = atten_out->data;
        mp.n_merges = (int32_t)plan.merges.size();
        mp.heads = pr.heads;
        mp.pack_shift = p.pack_shift;
        mp.head_dim = p.head_dim;
        e = mla::launch_mla_merge(mp, pr.dtype, s);
        if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "merge launch: %s", hipGetErrorString(e));
    }
    return ok();
}


// ---- MLA prolog ("MlaProlog" operator notes: parameter and return lists,
// constraints), non-quantised.
struct PrologProblem {
    int64_t t = 0, h = 0, r = 0, heads = 0;
};

int check_bf16(const mla_tensor *x, const char *name, int ndim) {
    int rc = check_tensor(x, name, true);
    if (rc) return rc;
    if (x->dtype != MLA_BF16) return fail(MLA_ERR_DTYPE, "%s must be bf16", name);
    if (x->ndim != ndim) return fail(MLA_ERR_SHAPE, "%s: expected %d dimensions, got %d", name, ndim, x->ndim);
    return MLA_OK;
}

int check_dtype(const mla_tensor *x, const char *name, int dtype, const char *dname, int ndim) {
    int rc = check_tensor(x, name, true);
    if (rc) return rc;
    if (x->dtype != dtype) return fail(MLA_ERR_DTYPE, "%s must be %s", name, dname);
    if (x->ndim != ndim) return fail(MLA_ERR_SHAPE, "%s: expected %d dimensions, got %d", name, ndim, x->ndim);
    return MLA_OK;
}

// [n, 1] or [n] fp32 (the quantised prolog's scales)
int check_scale_vector(const mla_tensor *x, const char *name, int64_t n) {
    int rc = check_tensor(x, name, true);
    if (rc) return rc;
    if (x->dtype != MLA_FP32) return fail(MLA_ERR_DTYPE, "%s must be float32", name);
    const bool ok_shape = (x->ndim == 1 && x->shape[0] == n) || (x->ndim == 2 && x->shape[0] == n && x->shape[1] == 1);
    if (!ok_shape) return fail(MLA_ERR_SHAPE, "%s: expected [%lld, 1] or [%lld]", name, (long long)n, (long long)n);
    return MLA_OK;
}

// quant: wq_b and qr_out are int8 (mla_prolog_quant); the scale tensors are
// checked by the caller
int validate_prolog(const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
                    const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                    const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, float eps, const mla_tensor *q_out,
                    const mla_tensor *kv_out, const mla_tensor *qr_out, PrologProblem *pp, bool quant = false) {
    int rc;
    if ((rc = check_bf16(token_x, "token_x", 2)) || (rc = check_bf16(wq_a, "wq_a", 2)) ||
        (rc = quant ? check_dtype(wq_b, "wq_b", MLA_INT8, "int8", 2) : check_bf16(wq_b, "wq_b", 2)) ||
        (rc = check_bf16(wkv, "wkv", 2)) || (rc = check_bf16(rope_cos, "rope_cos", 2)) ||
        (rc = check_bf16(rope_sin, "rope_sin", 2)) || (rc = check_bf16(gamma_cq, "gamma_cq", 1)) ||
        (rc = check_bf16(gamma_ckv, "gamma_ckv", 1)) || (rc = check_bf16(kv_out, "kv_out", 2)) ||
        (rc = quant ? check_dtype(qr_out, "qr_out", MLA_INT8, "int8", 2) : check_bf16(qr_out, "qr_out", 2)))
        return rc;
    if ((rc = check_tensor(q_out, "q_out", true))) return rc;
    if (q_out->dtype != MLA_BF16) return fail(MLA_ERR_DTYPE, "q_out must be bf16");
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(MLA_ERR_VALUE, "eps must be finite and > 0");
    const int64_t t = token_x->shape[0], h = token_x->shape[1];
    const int64_t r = wq_a->shape[1], hd = wkv->shape[1], rd = rope_cos->shape[1];
    if (wq_a->shape[0] != h) return fail(MLA_ERR_SHAPE, "wq_a: expected [h = %lld, q_lora_rank]", (long long)h);
    if (wkv->shape[0] != h) return fail(MLA_ERR_SHAPE, "wkv: expected [h = %lld, head_dim]", (long long)h);
    if (wq_b->shape[0] != r)
        return fail(MLA_ERR_SHAPE, "wq_b: expected [q_lora_rank = %lld, num_heads * head_dim]", (long long)r);
    if (hd <= 0 || wq_b->shape[1] % hd != 0 || wq_b->shape[1] == 0)
        return fail(MLA_ERR_SHAPE, "wq_b: width %lld is not num_heads * head_dim (%lld)",
                    (long long)wq_b->shape[1], (long long)hd);
    const int64_t heads = wq_b->shape[1] / hd;
    if (rope_cos->shape[0] != t || rope_sin->ndim != 2 || rope_sin->shape[0] != t || rope_sin->shape[1] != rd)
        return fail(MLA_ERR_SHAPE, "rope_cos / rope_sin: expected [t = %lld, rope_dim] each", (long long)t);
    if (gamma_cq->shape[0] != r) return fail(MLA_ERR_SHAPE, "gamma_cq: expected [q_lora_rank = %lld]", (long long)r);
    if (gamma_ckv->shape[0] != hd) return fail(MLA_ERR_SHAPE, "gamma_ckv: expected [head_dim = %lld]", (long long)hd);
    if (kv_out->shape[0] != t || kv_out->shape[1] != hd)
        return fail(MLA_ERR_SHAPE, "kv_out: expected [t = %lld, head_dim = %lld]", (long long)t, (long long)hd);
    if (qr_out->shape[0] != t || qr_out->shape[1] != r)
        return fail(MLA_ERR_SHAPE, "qr_out: expected [t = %lld, q_lora_rank = %lld]", (long long)t, (long long)r);
    const bool q3 = q_out->ndim == 3 && q_out->shape[0] == t && q_out->shape[1] == heads && q_out->shape[2] == hd;
    const bool q2 = q_out->ndim == 2 && q_out->shape[0] == t && q_out->shape[1] == heads * hd;
    if (!q3 && !q2)
        return fail(MLA_ERR_SHAPE, "q_out: expected [t, %lld, %lld] or [t, %lld]", (long long)heads, (long long)hd,
                    (long long)(heads * hd));
    if (hd != mla::PROLOG_BN) return fail(MLA_ERR_UNSUPPORTED, "head_dim %lld: only 512 is supported", (long long)hd);
    if (rd != mla::PROLOG_ROPE) return fail(MLA_ERR_UNSUPPORTED, "rope_dim %lld: only 64 is supported", (long long)rd);
    if (h <= 0 || h % mla::PROLOG_K_MULTIPLE != 0)
        return fail(MLA_ERR_UNSUPPORTED, "h %lld: a positive multiple of %d is required", (long long)h,
                    mla::PROLOG_K_MULTIPLE);
    if (r <= 0 || r % mla::PROLOG_BN != 0)
        return fail(MLA_ERR_UNSUPPORTED, "q_lora_rank %lld: a positive multiple of %d is required", (long long)r,
                    mla::PROLOG_BN);
    if (quant && r > mla::PROLOG_QUANT_MAX_COLS)
        return fail(MLA_ERR_UNSUPPORTED, "q_lora_rank %lld: at most %d in the quantised prolog", (long long)r,
                    mla::PROLOG_QUANT_MAX_COLS);
    // buffer resources address at most 4 GB from a tile's start; weights and
    // a 128-row tile of any operand stay far below that in every supported case
    if (r * heads * hd * 2 >= (int64_t)1 << 31 || h * r * 2 >= (int64_t)1 << 31 ||
        (int64_t)mla::PROLOG_BM * heads * hd * 2 >= (int64_t)1 << 31 || t > INT32_MAX / 2)
        return fail(MLA_ERR_UNSUPPORTED, "operand too large for 32-bit tile offsets");
    pp->t = t;
    pp->h = h;
    pp->r = r;
    pp->heads = heads;
    return MLA_OK;
}

// Workspace of mla_prolog: the fp32 rows of x . wq_a, then the packed copies
// of wq_a, wkv and wq_b (each 256-byte aligned).
uint64_t prolog_yq_bytes(const PrologProblem &pp) { return align256((uint64_t)pp.t * pp.r * 4); }
uint64_t prolog_pack_a_bytes(const PrologProblem &pp) {
    return align256((uint64_t)mla::prolog_packed_bytes((int32_t)(pp.r / mla::PROLOG_BN), (int32_t)pp.h));
}
uint64_t prolog_pack_kv_bytes(const PrologProblem &pp) {
    return align256((uint64_t)mla::prolog_packed_bytes(1, (int32_t)pp.h));
}
uint64_t prolog_pack_b_bytes(const PrologProblem &pp) {
    return align256((uint64_t)mla::prolog_packed_bytes((int32_t)pp.heads, (int32_t)pp.r));
}
uint64_t prolog_pack_b_i8_bytes(const PrologProblem &pp) {
    return align256((uint64_t)mla::prolog_packed_bytes((int32_t)pp.heads, (int32_t)pp.r, true));
}
// The first product's split over K. With few rows its output is a handful
// of 512-column tiles (3 at q_lora_rank 1024 below 129 rows), and so few
// workgroups cannot pull the 2 * h * (q_lora_rank + 512) bytes of weights at
// any useful rate. The K stages are then shared out, in runs of a multiple of
// 4 stages, until the launch has at least 128 workgroups; the runs' fp32 sums
// go to the workspace and a second kernel adds them and applies the tiles'
// epilogues.
constexpr int64_t PROLOG_SPLIT_MIN_WORKGROUPS = 128;
int32_t prolog_first_splits(const PrologProblem &pp) {
    const int64_t tiles = ((pp.t + mla::PROLOG_BM - 1) / mla::PROLOG_BM) * (pp.r / mla::PROLOG_BN + 1);
    const int64_t runs = pp.h / mla::PROLOG_BK / 4;  // K in runs of 4 stages
    int64_t ks = 1;
    while (tiles * ks < PROLOG_SPLIT_MIN_WORKGROUPS && ks < runs) {
        ++ks;
        while (runs % ks != 0) ++ks;  // the next divisor of runs (runs itself at the latest)
    }
    return (int32_t)ks;
}
// The kv tile (x . wkv) moves from the first product's launch to the
// second's, its workgroups first, where that takes a round of workgroups off
// the first launch: one product workgroup fills a CU (its LDS ring), so the
// first launch runs ceil(tiles * row tiles / CUs) rounds of workgroups over
// K = h, and its kv tiles then cost the second launch (many rounds over
// K = q_lora_rank) their share, row tiles / CUs of such a round. bf16 only
// (the quantised second product is int8), and never with a split first
// product. The kv tile's arithmetic is the same either way.
bool prolog_kv_with_second(const PrologProblem &pp, bool quant) {
    if (quant || prolog_first_splits(pp) > 1) return false;
    const int64_t cus = (int64_t)MLA_XCDS * MLA_CUS_PER_XCD;
    const int64_t m_tiles = (pp.t + mla::PROLOG_BM - 1) / mla::PROLOG_BM;
    const int64_t a_tiles = pp.r / mla::PROLOG_BN;
    auto rounds = [&](int64_t tiles) { return (tiles * m_tiles + cus - 1) / cus; };
    return rounds(a_tiles + 1) > rounds(a_tiles) && m_tiles < cus;
}
uint64_t prolog_part_bytes(const PrologProblem &pp) {
    const int32_t ks = prolog_first_splits(pp);
    if (ks <= 1) return 0;
    return align256((uint64_t)ks * pp.t * (pp.r + mla::PROLOG_BN) * 4);
}
uint64_t prolog_workspace_bytes(const PrologProblem &pp, bool quant = false) {
    if (pp.t == 0) return 0;  // nothing to compute
    return prolog_yq_bytes(pp) + prolog_pack_a_bytes(pp) + prolog_pack_kv_bytes(pp) +
           (quant ? prolog_pack_b_i8_bytes(pp) : prolog_pack_b_bytes(pp)) + prolog_part_bytes(pp);
}

// The first product, x . [wq_a | wkv], shared by both prolog operators: the
// wq_a tiles store fp32 rows for the c^Q norm, the wkv tile is the kv row
// (norm * gamma_ckv, rope). With kv_later the wkv tile is packed here but
// not run (the second product's launch runs it).
int prolog_first_product(const PrologProblem &pp, const mla_tensor *token_x, const mla_tensor *wq_a,
                         const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                         const mla_tensor *gamma_ckv, float eps, const mla_tensor *kv_out, float *y_q,
                         unsigned char *pack_a, unsigned char *pack_kv, float *part, bool pack, bool kv_later,
                         hipStream_t s) {
    mla::PrologGemmParams g1{};
    g1.a = token_x->data;
    g1.lda = pp.h;
    g1.m = (int32_t)pp.t;
    g1.k = (int32_t)pp.h;
    g1.seg[0] = {wq_a->data, pp.r, pack_a, (int32_t)(pp.r / mla::PROLOG_BN), mla::PROLOG_STORE_F32, y_q, pp.r,
                 nullptr};
    g1.seg[1] = {wkv->data, mla::PROLOG_BN, pack_kv, 1, mla::PROLOG_NORM_ROPE, kv_out->data, mla::PROLOG_BN,
                 gamma_ckv->data};
    g1.rope_cos = rope_cos->data;
    g1.rope_sin = rope_sin->data;
    g1.eps = eps;
    g1.k_splits = prolog_first_splits(pp);
    g1.part = part;
    g1.ld_part = pp.r + mla::PROLOG_BN;
    hipError_t e = hipSuccess;
    if (pack) {
        e = mla::launch_prolog_pack(g1, s);
        if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "prolog weight packing 1: %s", hipGetErrorString(e));
    }
    if (kv_later) g1.seg[1].n_tiles = 0;
    e = mla::launch_prolog_gemm(g1, s);
    if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "prolog product 1: %s", hipGetErrorString(e));
    if (g1.k_splits > 1) {
        e = mla::launch_prolog_split_reduce(g1, s);
        if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "prolog product 1 split sums: %s", hipGetErrorString(e));
    }
    return MLA_OK;
}

// The weight operands alone (mla_prolog_weights_size / pack_weights): the
// same checks as validate_prolog; wq_b bf16 or int8 (then *quant).
int validate_prolog_weights(const mla_tensor *wq_a, const mla_tensor *wq_b, const mla_tensor *wkv,
                            PrologProblem *pp, bool *quant) {
    int rc;
    if ((rc = check_bf16(wq_a, "wq_a", 2)) || (rc = check_bf16(wkv, "wkv", 2)) ||
        (rc = check_tensor(wq_b, "wq_b", true)))
        return rc;
    if (wq_b->dtype != MLA_BF16 && wq_b->dtype != MLA_INT8) return fail(MLA_ERR_DTYPE, "wq_b must be bf16 or int8");
    if (wq_b->ndim != 2) return fail(MLA_ERR_SHAPE, "wq_b: expected 2 dimensions, got %d", wq_b->ndim);
    *quant = wq_b->dtype == MLA_INT8;
    const int64_t h = wq_a->shape[0], r = wq_a->shape[1], hd = wkv->shape[1];
    if (wkv->shape[0] != h) return fail(MLA_ERR_SHAPE, "wkv: expected [h = %lld, head_dim]", (long long)h);
    if (wq_b->shape[0] != r)
        return fail(MLA_ERR_SHAPE, "wq_b: expected [q_lora_rank = %lld, num_heads * head_dim]", (long long)r);
    if (hd != mla::PROLOG_BN) return fail(MLA_ERR_UNSUPPORTED, "head_dim %lld: only 512 is supported", (long long)hd);
    if (wq_b->shape[1] % hd != 0 || wq_b->shape[1] == 0)
        return fail(MLA_ERR_SHAPE, "wq_b: width %lld is not num_heads * head_dim (%lld)",
                    (long long)wq_b->shape[1], (long long)hd);
    const int64_t heads = wq_b->shape[1] / hd;
    if (h <= 0 || h % mla::PROLOG_K_MULTIPLE != 0)
        return fail(MLA_ERR_UNSUPPORTED, "h %lld: a positive multiple of %d is required", (long long)h,
                    mla::PROLOG_K_MULTIPLE);
    if (r <= 0 || r % mla::PROLOG_BN != 0)
        return fail(MLA_ERR_UNSUPPORTED, "q_lora_rank %lld: a positive multiple of %d is required", (long long)r,
                    mla::PROLOG_BN);
    if (*quant && r > mla::PROLOG_QUANT_MAX_COLS)
        return fail(MLA_ERR_UNSUPPORTED, "q_lora_rank %lld: at most %d in the quantised prolog", (long long)r,
                    mla::PROLOG_QUANT_MAX_COLS);
    if (r * heads * hd * 2 >= (int64_t)1 << 31 || h * r * 2 >= (int64_t)1 << 31 ||
        (int64_t)mla::PROLOG_BM * heads * hd * 2 >= (int64_t)1 << 31)
        return fail(MLA_ERR_UNSUPPORTED, "operand too large for 32-bit tile offsets");
    pp->t = 0;
    pp->h = h;
    pp->r = r;
    pp->heads = heads;
    return MLA_OK;
}

// Packed weights: the copies of wq_a, wkv and wq_b the product kernel reads,
// in that order, each 256-byte aligned.
uint64_t prolog_packed_weights_bytes(const PrologProblem &pp, bool quant) {
    return prolog_pack_a_bytes(pp) + prolog_pack_kv_bytes(pp) +
           (quant ? prolog_pack_b_i8_bytes(pp) : prolog_pack_b_bytes(pp));
}
// Workspace of the prepacked operators: the fp32 rows of x . wq_a and the
// split first product's sums.
uint64_t prolog_prepacked_workspace_bytes(const PrologProblem &pp) {
    if (pp.t == 0) return 0;
    return prolog_yq_bytes(pp) + prolog_part_bytes(pp);
}

// The four prolog operators: quant selects int8 wq_b (qr_out int8, the two
// scale tensors); packed == nullptr packs the weights into the workspace on
// every call, else they are read from packed (mla_prolog_pack_weights).
int prolog_call(bool quant, const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
                const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, const mla_tensor *wq_b_scale, float eps,
                const mla_tensor *q_out, const mla_tensor *kv_out, const mla_tensor *qr_out,
                const mla_tensor *qr_scale_out, const void *packed, uint64_t packed_size, void *workspace,
                uint64_t workspace_size, void *stream) {
    PrologProblem pp;
    int rc = validate_prolog(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q_out, kv_out,
                             qr_out, &pp, quant);
    if (rc) return rc;
    if (quant && ((rc = check_scale_vector(wq_b_scale, "wq_b_scale", pp.heads * mla::PROLOG_BN)) ||
                  (rc = check_scale_vector(qr_scale_out, "qr_scale_out", pp.t))))
        return rc;
    const bool pack = packed == nullptr;
    if (!pack) {
        const uint64_t pneed = prolog_packed_weights_bytes(pp, quant);
        if (packed_size < pneed)
            return fail(MLA_ERR_WORKSPACE, "packed weights of %llu bytes needed, %llu given",
                        (unsigned long long)pneed, (unsigned long long)packed_size);
        if ((reinterpret_cast<uintptr_t>(packed) & 15) != 0)
            return fail(MLA_ERR_WORKSPACE, "packed weights must be 16-byte aligned");
    }
    if (pp.t == 0) return ok();
    const uint64_t need = pack ? prolog_workspace_bytes(pp, quant) : prolog_prepacked_workspace_bytes(pp);
    if (workspace == nullptr || workspace_size < need)
        return fail(MLA_ERR_WORKSPACE, "workspace of %llu bytes needed, %llu given", (unsigned long long)need,
                    (unsigned long long)workspace_size);
    if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
        return fail(MLA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned char *wsb = static_cast<unsigned char *>(workspace);
    float *y_q = reinterpret_cast<float *>(wsb);
    unsigned char *pack_a, *pack_kv, *pack_b;
    float *part;
    if (pack) {
        pack_a = wsb + prolog_yq_bytes(pp);
        pack_kv = pack_a + prolog_pack_a_bytes(pp);
        pack_b = pack_kv + prolog_pack_kv_bytes(pp);
        part = reinterpret_cast<float *>(pack_b + (quant ? prolog_pack_b_i8_bytes(pp) : prolog_pack_b_bytes(pp)));
    } else {
        pack_a = const_cast<unsigned char *>(static_cast<const unsigned char *>(packed));
        pack_kv = pack_a + prolog_pack_a_bytes(pp);
        pack_b = pack_kv + prolog_pack_kv_bytes(pp);
        part = reinterpret_cast<float *>(wsb + prolog_yq_bytes(pp));
    }

    const bool kv_later = prolog_kv_with_second(pp, quant);
    rc = prolog_first_product(pp, token_x, wq_a, wkv, rope_cos, rope_sin, gamma_ckv, eps, kv_out, y_q, pack_a,
                              pack_kv, part, pack, kv_later, s);
    if (rc) return rc;
    hipError_t e;
    float *scale = quant ? static_cast<float *>(qr_scale_out->data) : nullptr;
    if (quant)
        e = mla::launch_prolog_quant_rows(y_q, pp.r, gamma_cq->data, qr_out->data, pp.r, scale, (int32_t)pp.t,
                                          (int32_t)pp.r, eps, s);
    else
        e = mla::launch_prolog_rms_rows(y_q, pp.r, gamma_cq->data, qr_out->data, pp.r, (int32_t)pp.t, (int32_t)pp.r,
                                        eps, s);
    if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "prolog c^Q norm: %s", hipGetErrorString(e));
    // c^Q . wq_b (int8 with quant: dequantisation first): one tile per head
    // (norm per head, weight 1, rope); with kv_later also the kv tile, on x
    mla::PrologGemmParams g2{};
    g2.a = qr_out->data;
    g2.lda = pp.r;
    g2.m = (int32_t)pp.t;
    g2.k = (int32_t)pp.r;
    g2.seg[0] = {wq_b->data, pp.heads * mla::PROLOG_BN, pack_b, (int32_t)pp.heads, mla::PROLOG_NORM_ROPE,
                 q_out->data, pp.heads * mla::PROLOG_BN, nullptr};
    g2.seg[1] = {nullptr, 0, nullptr, 0, mla::PROLOG_NORM_ROPE, nullptr, 0, nullptr};
    g2.rope_cos = rope_cos->data;
    g2.rope_sin = rope_sin->data;
    g2.eps = eps;
    if (quant) {
        g2.int8 = 1;
        g2.row_scale = scale;
        g2.col_scale = static_cast<const float *>(wq_b_scale->data);
    }
    if (pack) {
        e = mla::launch_prolog_pack(g2, s);
        if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "prolog weight packing 2: %s", hipGetErrorString(e));
    }
    if (kv_later) {
        g2.seg[1] = {wkv->data, mla::PROLOG_BN, pack_kv, 1, mla::PROLOG_NORM_ROPE, kv_out->data, mla::PROLOG_BN,
                     gamma_ckv->data};
        g2.a1 = token_x->data;
        g2.lda1 = pp.h;
        g2.k1 = (int32_t)pp.h;
    }
    e = mla::launch_prolog_gemm(g2, s);
    if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "prolog product 2: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char *mla_last_error(void) { return g_last_error.c_str(); }

int mla_prefill_plan_host(const int32_t *q_seqlen, const int32_t *kv_seqlen, int32_t batch, int32_t head_num,
                          int32_t kv_head_num, int32_t mask_type, int64_t kv_padded_max_seq, void *buf,
                          uint64_t buf_size, int32_t *n_items, int32_t *n_tasks) {
    if (batch < 0) return fail(MLA_ERR_VALUE, "batch must be >= 0");
    if (batch > 0 && (q_seqlen == nullptr || kv_seqlen == nullptr))
        return fail(MLA_ERR_NULL, "length arrays are NULL");
    if (n_items == nullptr || n_tasks == nullptr) return fail(MLA_ERR_NULL, "n_items / n_tasks is NULL");
    if (head_num <= 0 || kv_head_num <= 0 || head_num % kv_head_num != 0)
        return fail(MLA_ERR_VALUE, "headNum / kvHeadNum invalid");
    if (mask_type < MLA_MASK_UNDEFINED || mask_type > MLA_MASK_FREE)
        return fail(MLA_ERR_VALUE, "maskType %d is not a known mask type", mask_type);
    for (int32_t b = 0; b < batch; ++b)
        if (q_seqlen[b] < 0 || kv_seqlen[b] < 0) return fail(MLA_ERR_VALUE, "negative length");
    Plan plan;
    build_plan(q_seqlen, kv_seqlen, batch, head_num, kv_head_num, mask_type, kv_padded_max_seq, true, &plan);
    *n_items = (int32_t)plan.items.size();
    *n_tasks = (int32_t)plan.tasks.size();
    uint64_t need = view_bytes(plan);
    if (need > 0) {
        if (buf == nullptr || buf_size < need)
            return fail(MLA_ERR_WORKSPACE, "plan needs %llu bytes", (unsigned long long)need);
        write_plan_view(plan, static_cast<uint8_t *>(buf));
    }
    return ok();
}

int mla_prefill_get_workspace_size(const mla_tensor *q, const mla_tensor *q_rope,
                                   const mla_tensor *k, const mla_tensor *k_rope,
                                   const mla_tensor *v, const mla_tensor *q_seqlen,
                                   const mla_tensor *kv_seqlen, const mla_tensor *mask,
                                   int32_t head_num, float qk_scale, int32_t kv_head_num,
                                   int32_t mask_type, uint8_t cache_mode,
                                   const mla_tensor *atten_out, uint64_t *workspace_size) {
    if (workspace_size == nullptr) return fail(MLA_ERR_NULL, "workspace_size is NULL");
    Problem pr;
    int rc = validate_prefill(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale,
                              kv_head_num, mask_type, cache_mode, atten_out, &pr);
    if (rc) return rc;
    Plan plan;
    build_plan(pr.q_seqlen, pr.kv_seqlen, pr.batch, pr.heads, pr.kv_heads, pr.mask_type, pr.kv_padded_max_seq,
               true, &plan);
    *workspace_size = plan_bytes(plan, pr.head_dim);
    return ok();
}

int mla_prefill(const mla_tensor *q, const mla_tensor *q_rope, const mla_tensor *k,
                const mla_tensor *k_rope, const mla_tensor *v, const mla_tensor *q_seqlen,
                const mla_tensor *kv_seqlen, const mla_tensor *mask, int32_t head_num,
                float qk_scale, int32_t kv_head_num, int32_t mask_type, uint8_t cache_mode,
                const mla_tensor *atten_out, void *workspace, uint64_t workspace_size,
                void *stream) {
    Problem pr;
    int rc = validate_prefill(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale,
                              kv_head_num, mask_type, cache_mode, atten_out, &pr);
    if (rc) return rc;
    return plan_and_launch(pr, nullptr, nullptr, q, q_rope, k->data, k_rope->data, v->data, mask, qk_scale,
                           atten_out, workspace, workspace_size, false, stream);
}

int mla_prefill_no_alloc(const mla_tensor *q, const mla_tensor *q_rope, const mla_tensor *k,
                         const mla_tensor *k_rope, const mla_tensor *v, const mla_tensor *q_seqlen,
                         const mla_tensor *kv_seqlen, const mla_tensor *mask, int32_t head_num,
                         float qk_scale, int32_t kv_head_num, int32_t mask_type, uint8_t cache_mode,
                         const mla_tensor *atten_out, void *stream) {
    Problem pr;
    int rc = validate_prefill(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale,
                              kv_head_num, mask_type, cache_mode, atten_out, &pr);
    if (rc) return rc;
    return plan_and_launch(pr, nullptr, nullptr, q, q_rope, k->data, k_rope->data, v->data, mask, qk_scale,
                           atten_out, nullptr, 0, true, stream);
}

int mla_prefill_paged_get_workspace_size(const mla_tensor *q, const mla_tensor *q_rope,
                                         const mla_tensor *key_cache, const mla_tensor *krope_cache,
                                         const mla_tensor *value_cache, const mla_tensor *block_tables,
                                         const mla_tensor *q_seqlen, const mla_tensor *kv_seqlen,
                                         const mla_tensor *mask, int32_t head_num, float qk_scale,
                                         int32_t kv_head_num, int32_t mask_type, const mla_tensor *atten_out,
                                         uint64_t *workspace_size) {
    if (workspace_size == nullptr) return fail(MLA_ERR_NULL, "workspace_size is NULL");
    Problem pr;
    PagedProblem pg;
    int rc = validate_paged(q, q_rope, key_cache, krope_cache, value_cache, block_tables, q_seqlen, kv_seqlen,
                            mask, head_num, qk_scale, kv_head_num, mask_type, atten_out, &pr, &pg);
    if (rc) return rc;
    Plan plan;
    build_plan(pr.q_seqlen, pr.kv_seqlen, pr.batch, pr.heads, pr.kv_heads, pr.mask_type, 0, true, &plan);
    *workspace_size = plan_bytes(plan, pr.head_dim);
    return ok();
}

int mla_prefill_paged(const mla_tensor *q, const mla_tensor *q_rope, const mla_tensor *key_cache,
                      const mla_tensor *krope_cache, const mla_tensor *value_cache,
                      const mla_tensor *block_tables, const mla_tensor *q_seqlen,
                      const mla_tensor *kv_seqlen, const mla_tensor *mask, int32_t head_num,
                      float qk_scale, int32_t kv_head_num, int32_t mask_type,
                      const mla_tensor *atten_out, void *workspace, uint64_t workspace_size,
                      void *stream) {
    Problem pr;
    PagedProblem pg;
    int rc = validate_paged(q, q_rope, key_cache, krope_cache, value_cache, block_tables, q_seqlen, kv_seqlen,
                            mask, head_num, qk_scale, kv_head_num, mask_type, atten_out, &pr, &pg);
    if (rc) return rc;
    return plan_and_launch(pr, &pg, static_cast<const int32_t *>(block_tables->data), q, q_rope, key_cache->data,
                           krope_cache->data, value_cache->data, mask, qk_scale, atten_out, workspace,
                           workspace_size, false, stream);
}

int paged_cache_load(const mla_tensor *key_cache, const mla_tensor *value_cache,
                     const mla_tensor *block_tables, const mla_tensor *context_lens,
                     const mla_tensor *key, const mla_tensor *value, const mla_tensor *seq_starts,
                     int8_t kv_cache_cfg, bool is_seq_lens_cumsum_type, bool has_seq_starts,
                     void *stream) {
    int rc;
    if ((rc = check_tensor(key_cache, "key_cache", true)) || (rc = check_tensor(key, "key", true)) ||
        (rc = check_tensor(block_tables, "block_tables", true)) ||
        (rc = check_tensor(context_lens, "context_lens", true)))
        return rc;
    if ((value_cache == nullptr) != (value == nullptr))
        return fail(MLA_ERR_NULL, "value_cache and value must both be given or both be NULL");
    if (value_cache && ((rc = check_tensor(value_cache, "value_cache", true)) ||
                        (rc = check_tensor(value, "value", true))))
        return rc;
    if (kv_cache_cfg != MLA_KV_CACHE_ND && kv_cache_cfg != MLA_KV_CACHE_NZ)
        return fail(MLA_ERR_VALUE, "kvCacheCfg %d is unknown", kv_cache_cfg);
    const bool nz = kv_cache_cfg == MLA_KV_CACHE_NZ;
    if (nz && (is_seq_lens_cumsum_type || has_seq_starts))
        return fail(MLA_ERR_UNSUPPORTED, "kvCacheCfg NZ: cumulative lengths and seqStarts are ND-only");

    const int dt = key_cache->dtype;
    if (!(dt == MLA_FP16 || dt == MLA_BF16 || dt == MLA_INT8))
        return fail(MLA_ERR_DTYPE, "key_cache: dtype must be fp16, bf16 or int8");
    if (key->dtype != dt) return fail(MLA_ERR_DTYPE, "key: dtype differs from key_cache");
    if (value_cache && (value_cache->dtype != dt || value->dtype != dt))
        return fail(MLA_ERR_DTYPE, "value_cache / value: dtype differs from key_cache");
    if (block_tables->dtype != MLA_INT32 || context_lens->dtype != MLA_INT32)
        return fail(MLA_ERR_DTYPE, "block_tables / context_lens must be int32");

    int64_t nb, bs, heads = 0, chunks_k = 0, chunks_v = 0;
    if (nz) {
        // NZ: cache [num_blocks, heads*head_size / E, block_size, E], E = 32 int8 / 16 fp16-bf16
        // (32 bytes); gathered tensor [num_tokens, heads*head_size]
        const int64_t e = dt == MLA_INT8 ? 32 : 16;
        if (key_cache->ndim != 4 || key_cache->shape[3] != e)
            return fail(MLA_ERR_SHAPE, "key_cache: expected NZ [num_blocks, chunks, block_size, %lld]", (long long)e);
        nb = key_cache->shape[0];
        bs = key_cache->shape[2];
        chunks_k = key_cache->shape[1];
        if (bs <= 0) return fail(MLA_ERR_SHAPE, "key_cache: block_size must be > 0");
        if (key->ndim != 2 || key->shape[1] != chunks_k * e)
            return fail(MLA_ERR_SHAPE, "key: expected [num_tokens, %lld]", (long long)(chunks_k * e));
        if (value_cache) {
            if (value_cache->ndim != 4 || value_cache->shape[0] != nb || value_cache->shape[2] != bs ||
                value_cache->shape[3] != e)
                return fail(MLA_ERR_SHAPE, "value_cache: expected NZ [%lld, chunks, %lld, %lld]", (long long)nb,
                            (long long)bs, (long long)e);
            chunks_v = value_cache->shape[1];
            if (value->ndim != 2 || value->shape[0] != key->shape[0] || value->shape[1] != chunks_v * e)
                return fail(MLA_ERR_SHAPE, "value: expected [%lld, %lld]", (long long)key->shape[0],
                            (long long)(chunks_v * e));
        }
    } else {
        if (key_cache->ndim != 4) return fail(MLA_ERR_SHAPE, "key_cache: expected ND [num_blocks, block_size, heads, head_size]");
        nb = key_cache->shape[0];
        bs = key_cache->shape[1];
        heads = key_cache->shape[2];
        if (bs <= 0) return fail(MLA_ERR_SHAPE, "key_cache: block_size must be > 0");
        if (key->ndim != 3 || key->shape[1] != heads || key->shape[2] != key_cache->shape[3])
            return fail(MLA_ERR_SHAPE, "key: expected [num_tokens, %lld, %lld]", (long long)heads,
                        (long long)key_cache->shape[3]);
        if (value_cache) {
            if (value_cache->ndim != 4 || value_cache->shape[0] != nb || value_cache->shape[1] != bs ||
                value_cache->shape[2] != heads)
                return fail(MLA_ERR_SHAPE, "value_cache: expected [%lld, %lld, %lld, head_size_v]", (long long)nb,
                            (long long)bs, (long long)heads);
            if (value->ndim != 3 || value->shape[0] != key->shape[0] || value->shape[1] != heads ||
                value->shape[2] != value_cache->shape[3])
                return fail(MLA_ERR_SHAPE, "value: expected [%lld, %lld, %lld]", (long long)key->shape[0],
                            (long long)heads, (long long)value_cache->shape[3]);
        }
    }
    const int64_t num_tokens = key->shape[0];
    if (block_tables->ndim != 2) return fail(MLA_ERR_SHAPE, "block_tables: expected [batch, max_blocks]");
    const int64_t batch = block_tables->shape[0];
    if (batch > mla::GATHER_MAX_BATCH)
        return fail(MLA_ERR_UNSUPPORTED, "batch above %d", mla::GATHER_MAX_BATCH);
    if (context_lens->ndim != 1) return fail(MLA_ERR_SHAPE, "context_lens: expected one dimension");
    const int64_t n_ctx = context_lens->shape[0];
    if (!(n_ctx == batch || (is_seq_lens_cumsum_type && n_ctx == batch + 1)))
        return fail(MLA_ERR_SHAPE, "context_lens: expected [batch]%s", is_seq_lens_cumsum_type ? " or [batch + 1]" : "");
    if (has_seq_starts) {
        if (seq_starts == nullptr) return fail(MLA_ERR_NULL, "seq_starts: required when has_seq_starts");
        if ((rc = check_tensor(seq_starts, "seq_starts", true))) return rc;
        if (seq_starts->dtype != MLA_INT32) return fail(MLA_ERR_DTYPE, "seq_starts must be int32");
        if (seq_starts->ndim != 1 || seq_starts->shape[0] != batch)
            return fail(MLA_ERR_SHAPE, "seq_starts: expected [batch]");
    }
    if (num_tokens == 0 || batch == 0) return ok();

    mla::GatherParams p{};
    p.key_cache = key_cache->data;
    p.value_cache = value_cache ? value_cache->data : nullptr;
    p.key = key->data;
    p.value = value ? value->data : nullptr;
    p.block_tables = static_cast<const int32_t *>(block_tables->data);
    p.context_lens = static_cast<const int32_t *>(context_lens->data);
    p.seq_starts = has_seq_starts ? static_cast<const int32_t *>(seq_starts->data) : nullptr;
    p.num_blocks = nb;
    p.block_size = bs;
    p.max_blocks = block_tables->shape[1];
    p.num_tokens = num_tokens;
    if (nz) {
        p.nz = 1;
        p.chunks_k = chunks_k;
        p.chunks_v = chunks_v;
        p.row_bytes_k = chunks_k * 32;
        p.row_bytes_v = chunks_v * 32;
    } else {
        p.row_bytes_k = heads * key_cache->shape[3] * (int64_t)elem_size(dt);
        p.row_bytes_v = value_cache ? heads * value_cache->shape[3] * (int64_t)elem_size(dt) : 0;
    }
    p.batch = (int32_t)batch;
    p.ctx_entries = (int32_t)n_ctx;
    p.cumsum = is_seq_lens_cumsum_type ? 1 : 0;
    p.has_seq_starts = has_seq_starts ? 1 : 0;
    hipError_t e = mla::launch_paged_gather(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "gather launch: %s", hipGetErrorString(e));
    return ok();
}


int mla_prolog_get_workspace_size(const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
                                  const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                                  const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, float eps,
                                  const mla_tensor *q_out, const mla_tensor *kv_out, const mla_tensor *qr_out,
                                  uint64_t *workspace_size) {
    if (workspace_size == nullptr) return fail(MLA_ERR_NULL, "workspace_size is NULL");
    PrologProblem pp;
    int rc = validate_prolog(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q_out, kv_out,
                             qr_out, &pp);
    if (rc) return rc;
    *workspace_size = prolog_workspace_bytes(pp);
    return ok();
}

int mla_prolog(const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
               const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
               const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, float eps, const mla_tensor *q_out,
               const mla_tensor *kv_out, const mla_tensor *qr_out, void *workspace, uint64_t workspace_size,
               void *stream) {
    return prolog_call(false, token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, nullptr, eps, q_out,
                       kv_out, qr_out, nullptr, nullptr, 0, workspace, workspace_size, stream);
}

int mla_prolog_quant_get_workspace_size(const mla_tensor *token_x, const mla_tensor *wq_a,
                                        const mla_tensor *wq_b, const mla_tensor *wkv,
                                        const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                                        const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv,
                                        const mla_tensor *wq_b_scale, float eps, const mla_tensor *q_out,
                                        const mla_tensor *kv_out, const mla_tensor *qr_out,
                                        const mla_tensor *qr_scale_out, uint64_t *workspace_size) {
    if (workspace_size == nullptr) return fail(MLA_ERR_NULL, "workspace_size is NULL");
    PrologProblem pp;
    int rc = validate_prolog(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q_out, kv_out,
                             qr_out, &pp, true);
    if (rc) return rc;
    if ((rc = check_scale_vector(wq_b_scale, "wq_b_scale", pp.heads * mla::PROLOG_BN)) ||
        (rc = check_scale_vector(qr_scale_out, "qr_scale_out", pp.t)))
        return rc;
    *workspace_size = prolog_workspace_bytes(pp, true);
    return ok();
}

int mla_prolog_quant(const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
                     const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                     const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, const mla_tensor *wq_b_scale,
                     float eps, const mla_tensor *q_out, const mla_tensor *kv_out, const mla_tensor *qr_out,
                     const mla_tensor *qr_scale_out, void *workspace, uint64_t workspace_size, void *stream) {
    return prolog_call(true, token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, eps, q_out,
                       kv_out, qr_out, qr_scale_out, nullptr, 0, workspace, workspace_size, stream);
}

int mla_prolog_weights_size(const mla_tensor *wq_a, const mla_tensor *wq_b, const mla_tensor *wkv,
                            uint64_t *packed_size) {
    if (packed_size == nullptr) return fail(MLA_ERR_NULL, "packed_size is NULL");
    PrologProblem pp;
    bool quant = false;
    int rc = validate_prolog_weights(wq_a, wq_b, wkv, &pp, &quant);
    if (rc) return rc;
    *packed_size = prolog_packed_weights_bytes(pp, quant);
    return ok();
}

int mla_prolog_pack_weights(const mla_tensor *wq_a, const mla_tensor *wq_b, const mla_tensor *wkv, void *packed,
                            uint64_t packed_size, void *stream) {
    PrologProblem pp;
    bool quant = false;
    int rc = validate_prolog_weights(wq_a, wq_b, wkv, &pp, &quant);
    if (rc) return rc;
    const uint64_t need = prolog_packed_weights_bytes(pp, quant);
    if (packed == nullptr || packed_size < need)
        return fail(MLA_ERR_WORKSPACE, "packed weights need %llu bytes, %llu given", (unsigned long long)need,
                    (unsigned long long)packed_size);
    if ((reinterpret_cast<uintptr_t>(packed) & 15) != 0)
        return fail(MLA_ERR_WORKSPACE, "packed weights must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned char *pb = static_cast<unsigned char *>(packed);
    mla::PrologGemmParams g1{};
    g1.k = (int32_t)pp.h;
    g1.seg[0] = {wq_a->data, pp.r, pb, (int32_t)(pp.r / mla::PROLOG_BN), mla::PROLOG_STORE_F32, nullptr, 0, nullptr};
    g1.seg[1] = {wkv->data, mla::PROLOG_BN, pb + prolog_pack_a_bytes(pp), 1, mla::PROLOG_NORM_ROPE, nullptr, 0,
                 nullptr};
    hipError_t e = mla::launch_prolog_pack(g1, s);
    if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "prolog weight packing 1: %s", hipGetErrorString(e));
    mla::PrologGemmParams g2{};
    g2.k = (int32_t)pp.r;
    g2.int8 = quant ? 1 : 0;
    g2.seg[0] = {wq_b->data, pp.heads * mla::PROLOG_BN, pb + prolog_pack_a_bytes(pp) + prolog_pack_kv_bytes(pp),
                 (int32_t)pp.heads, mla::PROLOG_NORM_ROPE, nullptr, 0, nullptr};
    e = mla::launch_prolog_pack(g2, s);
    if (e != hipSuccess) return fail(MLA_ERR_RUNTIME, "prolog weight packing 2: %s", hipGetErrorString(e));
    return ok();
}

int mla_prolog_prepacked_workspace_size(const mla_tensor *token_x, const mla_tensor *wq_a, uint64_t *workspace_size) {
    if (workspace_size == nullptr) return fail(MLA_ERR_NULL, "workspace_size is NULL");
    int rc;
    if ((rc = check_tensor(token_x, "token_x", true)) || (rc = check_tensor(wq_a, "wq_a", true))) return rc;
    if (token_x->ndim != 2 || wq_a->ndim != 2 || wq_a->shape[0] != token_x->shape[1])
        return fail(MLA_ERR_SHAPE, "token_x [t, h] and wq_a [h, q_lora_rank] expected");
    PrologProblem pp;
    pp.t = token_x->shape[0];
    pp.h = token_x->shape[1];
    pp.r = wq_a->shape[1];
    if (pp.h <= 0 || pp.h % mla::PROLOG_K_MULTIPLE != 0 || pp.r <= 0 || pp.r % mla::PROLOG_BN != 0)
        return fail(MLA_ERR_UNSUPPORTED, "h must be a positive multiple of %d and q_lora_rank of %d",
                    mla::PROLOG_K_MULTIPLE, mla::PROLOG_BN);
    *workspace_size = prolog_prepacked_workspace_bytes(pp);
    return ok();
}

int mla_prolog_prepacked(const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
                         const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                         const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, float eps, const mla_tensor *q_out,
                         const mla_tensor *kv_out, const mla_tensor *qr_out, const void *packed,
                         uint64_t packed_size, void *workspace, uint64_t workspace_size, void *stream) {
    if (packed == nullptr) return fail(MLA_ERR_NULL, "packed is NULL");
    return prolog_call(false, token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, nullptr, eps, q_out,
                       kv_out, qr_out, nullptr, packed, packed_size, workspace, workspace_size, stream);
}

int mla_prolog_quant_prepacked(const mla_tensor *token_x, const mla_tensor *wq_a, const mla_tensor *wq_b,
                               const mla_tensor *wkv, const mla_tensor *rope_cos, const mla_tensor *rope_sin,
                               const mla_tensor *gamma_cq, const mla_tensor *gamma_ckv, const mla_tensor *wq_b_scale,
                               float eps, const mla_tensor *q_out, const mla_tensor *kv_out,
                               const mla_tensor *qr_out, const mla_tensor *qr_scale_out, const void *packed,
                               uint64_t packed_size, void *workspace, uint64_t workspace_size, void *stream) {
    if (packed == nullptr) return fail(MLA_ERR_NULL, "packed is NULL");
    return prolog_call(true, token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, eps, q_out,
                       kv_out, qr_out, qr_scale_out, packed, packed_size, workspace, workspace_size, stream);
}

}  // extern "C"
