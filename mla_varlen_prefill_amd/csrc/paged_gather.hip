// Paged K/V gather for gfx950 (Ascend Transformer Boost
// "PagedCacheLoadOperation" page, Members table; ND cache layout).
//
// Token t of sequence b is logical position s_b + t of that sequence's block
// table: block block_tables[b][(s_b + t) / block_size], slot
// (s_b + t) % block_size. Its row of heads * head_size elements is copied
// verbatim to output row off_b + t.
//
// The copy is HBM-bound, so the kernel is built around bytes in flight:
//  * every workgroup first rebuilds the per-sequence output offsets in LDS
//    (a block-wide scan of context_lens, or the running totals as given);
//  * it then walks its share of output tokens, resolving each token's source
//    row once (binary search over the offsets), and copies the key row and the
//    value row with 16-byte non-temporal loads and stores, eight of them in
//    flight per thread before the first store;
//  * rows that are not a multiple of 16 bytes, or unaligned ones, fall back to
//    a byte copy.
// Tokens whose output row is past num_tokens, whose table column is past
// max_blocks or whose block id is outside [0, num_blocks) are skipped.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mla {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int G_THREADS = 256;
constexpr int G_TOKENS = 4;  // tokens resolved per workgroup step
constexpr int G_UNROLL = 8;  // 16-byte loads in flight per thread and row

__device__ __forceinline__ void copy_row16(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                           int64_t n16, int tid) {
    int64_t c = tid;
    for (; c + (G_UNROLL - 1) * G_THREADS < n16; c += G_UNROLL * G_THREADS) {
        u32x4 r[G_UNROLL];
#pragma unroll
        for (int u = 0; u < G_UNROLL; ++u) r[u] = __builtin_nontemporal_load(src + c + u * G_THREADS);
#pragma unroll
        for (int u = 0; u < G_UNROLL; ++u) __builtin_nontemporal_store(r[u], dst + c + u * G_THREADS);
    }
    for (; c < n16; c += G_THREADS) __builtin_nontemporal_store(__builtin_nontemporal_load(src + c), dst + c);
}

__device__ __forceinline__ void copy_row_bytes(const unsigned char *src, unsigned char *dst, int64_t n,
                                               int tid) {
    for (int64_t c = tid; c < n; c += G_THREADS) dst[c] = src[c];
}

__global__ __launch_bounds__(G_THREADS) void paged_gather_kernel(const GatherParams p) {
    extern __shared__ int32_t s_off[];  // [batch + 1] output offsets
    __shared__ int64_t s_src[G_TOKENS];  // source slot (block * block_size + offset), -1 to skip
    __shared__ int32_t s_partial[G_THREADS];
    const int tid = threadIdx.x;
    const int B = p.batch;

    // ---- output offsets of every sequence
    if (p.cumsum) {
        if (p.ctx_entries == B + 1) {  // [0, c1, c1 + c2, ...]
            for (int i = tid; i <= B; i += G_THREADS) s_off[i] = p.context_lens[i];
        } else {                        // inclusive totals [c1, c1 + c2, ...]
            for (int i = tid; i <= B; i += G_THREADS) s_off[i] = i == 0 ? 0 : p.context_lens[i - 1];
        }
        __syncthreads();
    } else {
        // block-wide exclusive scan: each thread sums a contiguous chunk
        const int chunk = (B + G_THREADS - 1) / G_THREADS;
        const int lo = tid * chunk, hi = min(B, lo + chunk);
        int32_t sum = 0;
        for (int i = lo; i < hi; ++i) sum += p.context_lens[i];
        s_partial[tid] = sum;
        __syncthreads();
        if (tid == 0) {
            int32_t run = 0;
            for (int t = 0; t < G_THREADS; ++t) {
                const int32_t x = s_partial[t];
                s_partial[t] = run;
                run += x;
            }
        }
        __syncthreads();
        int32_t run = s_partial[tid];
        for (int i = lo; i < hi; ++i) {
            s_off[i] = run;
            run += p.context_lens[i];
        }
        if (hi == B && lo < hi) s_off[B] = run;  // the thread holding the last sequence
        __syncthreads();
    }

    const bool vec = ((p.row_bytes_k | p.row_bytes_v) & 15) == 0 &&
                     ((reinterpret_cast<uintptr_t>(p.key_cache) | reinterpret_cast<uintptr_t>(p.key) |
                       reinterpret_cast<uintptr_t>(p.value_cache) | reinterpret_cast<uintptr_t>(p.value)) &
                      15) == 0;
    const int64_t total = p.num_tokens;
    const unsigned char *kc = static_cast<const unsigned char *>(p.key_cache);
    const unsigned char *vc = static_cast<const unsigned char *>(p.value_cache);
    unsigned char *ko = static_cast<unsigned char *>(p.key);
    unsigned char *vo = static_cast<unsigned char *>(p.value);

    for (int64_t n0 = (int64_t)blockIdx.x * G_TOKENS; n0 < total; n0 += (int64_t)gridDim.x * G_TOKENS) {
        // ---- resolve the source rows of tokens n0 .. n0 + G_TOKENS - 1
        if (tid < G_TOKENS) {
            const int64_t n = n0 + tid;
            int64_t src = -1;
            if (n < total && n < s_off[B]) {
                // last sequence b with s_off[b] <= n
                int lo = 0, hi = B;  // invariant: s_off[lo] <= n < s_off[hi]
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (s_off[mid] <= n) lo = mid; else hi = mid;
                }
                const int b = lo;
                const int64_t t = n - s_off[b];
                const int64_t lpos = t + (p.has_seq_starts ? p.seq_starts[b] : 0);
                if (lpos >= 0) {
                    const int64_t col = lpos / p.block_size;
                    if (col < p.max_blocks) {
                        const int64_t blk = p.block_tables[(int64_t)b * p.max_blocks + col];
                        if (blk >= 0 && blk < p.num_blocks) src = blk * p.block_size + lpos % p.block_size;
                    }
                }
            }
            s_src[tid] = src;
        }
        __syncthreads();
        for (int i = 0; i < G_TOKENS; ++i) {
            const int64_t n = n0 + i;
            const int64_t src = s_src[i];
            if (n >= total || src < 0) continue;
            if (vec) {
                copy_row16(reinterpret_cast<const u32x4 *>(kc + src * p.row_bytes_k),
                           reinterpret_cast<u32x4 *>(ko + n * p.row_bytes_k), p.row_bytes_k >> 4, tid);
                if (vc)
                    copy_row16(reinterpret_cast<const u32x4 *>(vc + src * p.row_bytes_v),
                               reinterpret_cast<u32x4 *>(vo + n * p.row_bytes_v), p.row_bytes_v >> 4, tid);
            } else {
                copy_row_bytes(kc + src * p.row_bytes_k, ko + n * p.row_bytes_k, p.row_bytes_k, tid);
                if (vc) copy_row_bytes(vc + src * p.row_bytes_v, vo + n * p.row_bytes_v, p.row_bytes_v, tid);
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_paged_gather(const GatherParams &p, hipStream_t stream) {
    if (p.num_tokens <= 0 || p.batch <= 0) return hipSuccess;
    int64_t steps = (p.num_tokens + G_TOKENS - 1) / G_TOKENS;
    int grid = (int)(steps < 8192 ? steps : 8192);
    size_t shmem = sizeof(int32_t) * ((size_t)p.batch + 1);
    hipLaunchKernelGGL(paged_gather_kernel, dim3(grid), dim3(G_THREADS), shmem, stream, p);
    return hipGetLastError();
}

}  // namespace mla
