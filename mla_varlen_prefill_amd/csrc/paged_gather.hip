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
//
// NZ layout (the page's dimension table, NZ column): a token's row is cut into
// 32-byte chunks (16 fp16/bf16 or 32 int8 elements) and chunk c of slot s of
// block k sits at cache[k][c][s]. For one chunk, consecutive slots are
// adjacent; for one token, consecutive chunks are block_size * 32 bytes apart.
// So the NZ kernel transposes through LDS: a workgroup owns 44 output tokens;
// for each group of 32 chunks, every read instruction takes one chunk of 32
// consecutive tokens (one contiguous kilobyte when they share a block), the
// tile is stored in LDS by token (rows padded by 16 bytes against bank
// conflicts), and every write instruction then stores one kilobyte of one
// token's output row. The next group's loads are in flight while a group goes
// from LDS to the output. The 44 x 32 tile (45 KB of LDS, three workgroups
// per CU) measured 71-74% of the HBM peak for the paged workload's K+V and
// 71-72% for its KRope, against 67-69% for 64 x 32 (66 KB, two per CU);
// 36, 40 and 48 tokens were within a point or two of 44, and 32 x 16, 32 x 32,
// 64 x 16, 64 x 24, 48 x 40, 128 x 8, 128 x 16 and 16 x 64 lower.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mla {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int G_THREADS = 256;
constexpr int G_TOKENS = 4;  // tokens resolved per workgroup step (16 measured 12% slower on 16 KB rows)
constexpr int G_GRID = 8192;  // at most this many workgroups (they stride over the steps)
constexpr int G_UNROLL = 8;  // 16-byte loads in flight per thread and row

// Every pass issues all of a thread's loads (up to G_UNROLL) before its first
// store, also for rows shorter than G_UNROLL * G_THREADS pieces (a 16 KB
// KRope row is 4 pieces per thread): a load-store loop there keeps only one
// load per thread in flight.
//
// Measured on the paged workload (one call gathers K and V, 32 KB rows each;
// a second call KRope, 16 KB rows): K+V at 79-81% of the 8 TB/s peak, KRope
// at 65-68%, where a plain device copy of the KRope bytes (torch copy_) runs
// at 57-63%, and at any size from 2 to 64 GB. K alone (one stream of 32 KB
// rows) and two 16 KB caches in one call run at 65-66% too: only two 32 KB
// rows per token reach 80%. Not faster on KRope, and 2-15% slower on K+V:
// the eight loads taken across the four tokens of a step; 2, 8 or 16 tokens
// per step; 2048 to 65536 workgroups; plain instead of non-temporal loads or
// stores; one wave per row with 16 loads per lane and no workgroup barriers;
// a KRope-only call taking each step's tokens from both halves of the token
// range (two read and two write streams, as K+V has).
__device__ __forceinline__ void copy_row16(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                           int64_t n16, int tid) {
    for (int64_t c = tid; c < n16; c += G_UNROLL * G_THREADS) {
        u32x4 r[G_UNROLL];
#pragma unroll
        for (int u = 0; u < G_UNROLL; ++u)
            if (c + u * G_THREADS < n16) r[u] = __builtin_nontemporal_load(src + c + u * G_THREADS);
#pragma unroll
        for (int u = 0; u < G_UNROLL; ++u)
            if (c + u * G_THREADS < n16) __builtin_nontemporal_store(r[u], dst + c + u * G_THREADS);
    }
}

__device__ __forceinline__ void copy_row_bytes(const unsigned char *src, unsigned char *dst, int64_t n,
                                               int tid) {
    for (int64_t c = tid; c < n; c += G_THREADS) dst[c] = src[c];
}

// Output offset of every sequence into s_off[0 .. batch]: a block-wide scan
// of context_lens, or the running totals as given. The scan is 64-bit: the
// lengths are device data the host never sees, and their total may pass
// 2^31 (rows at or past num_tokens are then skipped, not wrapped).
__device__ void build_offsets(const GatherParams &p, int64_t *s_off, int64_t *s_partial, int tid) {
    const int B = p.batch;
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
        int64_t sum = 0;
        for (int i = lo; i < hi; ++i) sum += p.context_lens[i];
        s_partial[tid] = sum;
        __syncthreads();
        if (tid == 0) {
            int64_t run = 0;
            for (int t = 0; t < G_THREADS; ++t) {
                const int64_t x = s_partial[t];
                s_partial[t] = run;
                run += x;
            }
        }
        __syncthreads();
        int64_t run = s_partial[tid];
        for (int i = lo; i < hi; ++i) {
            s_off[i] = run;
            run += p.context_lens[i];
        }
        if (hi == B && lo < hi) s_off[B] = run;  // the thread holding the last sequence
        __syncthreads();
    }
}

// Source slot of output token n (block * block_size + position in the block),
// or -1 when the token is to be skipped.
__device__ int64_t source_slot(const GatherParams &p, const int64_t *s_off, int64_t n) {
    const int B = p.batch;
    if (n >= p.num_tokens || n >= s_off[B]) return -1;
    int lo = 0, hi = B;  // last sequence b with s_off[b] <= n: s_off[lo] <= n < s_off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= n) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int64_t lpos = n - s_off[b] + (p.has_seq_starts ? p.seq_starts[b] : 0);
    if (lpos < 0) return -1;
    const int64_t col = lpos / p.block_size;
    if (col >= p.max_blocks) return -1;
    const int64_t blk = p.block_tables[(int64_t)b * p.max_blocks + col];
    if (blk < 0 || blk >= p.num_blocks) return -1;
    return blk * p.block_size + lpos % p.block_size;
}

__global__ __launch_bounds__(G_THREADS) void paged_gather_kernel(const GatherParams p) {
    extern __shared__ int64_t s_off[];  // [batch + 1] output offsets
    __shared__ int64_t s_src[G_TOKENS];  // source slot (block * block_size + offset), -1 to skip
    __shared__ int64_t s_partial[G_THREADS];
    const int tid = threadIdx.x;

    build_offsets(p, s_off, s_partial, tid);

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
            // source_slot returns -1 past num_tokens, so every token to copy has n < total
            const int64_t src = source_slot(p, s_off, n0 + tid);
            s_src[tid] = src;
        }
        __syncthreads();
        for (int i = 0; i < G_TOKENS; ++i) {
            const int64_t n = n0 + i;
            const int64_t src = s_src[i];
            if (src < 0) continue;
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


// ---- NZ layout
#ifndef MLA_NZ_TOKENS
#define MLA_NZ_TOKENS 44
#endif
#ifndef MLA_NZ_CHUNKS
#define MLA_NZ_CHUNKS 32
#endif
constexpr int NZ_TOKENS = MLA_NZ_TOKENS;      // output tokens per workgroup
constexpr int NZ_CHUNKS = MLA_NZ_CHUNKS;      // 32-byte chunks per tile
constexpr int NZ_ROW = NZ_CHUNKS * 32 + 16;   // LDS bytes per token row of the tile
constexpr int NZ_PER_THREAD = NZ_TOKENS * NZ_CHUNKS * 2 / G_THREADS;  // 16-byte pieces per thread and tile
static_assert(NZ_PER_THREAD * G_THREADS == NZ_TOKENS * NZ_CHUNKS * 2, "whole pieces per thread");

// One cache (key or value): output token rows n0 .. n0 + NZ_TOKENS - 1 of
// chunks [0, chunks), through LDS tiles of NZ_TOKENS tokens x NZ_CHUNKS chunks.
__global__ __launch_bounds__(G_THREADS) void paged_gather_nz_kernel(const GatherParams p, const void *cache_,
                                                                    void *out_, int64_t chunks) {
    extern __shared__ int64_t s_off[];  // [batch + 1] output offsets
    __shared__ int64_t s_base[NZ_TOKENS];  // byte offset of chunk 0 of each token, -1 to skip
    __shared__ int64_t s_partial[G_THREADS];
    __shared__ __attribute__((aligned(16))) unsigned char tile[NZ_TOKENS * NZ_ROW];
    const int tid = threadIdx.x;
    const unsigned char *cache = static_cast<const unsigned char *>(cache_);
    unsigned char *out = static_cast<unsigned char *>(out_);

    build_offsets(p, s_off, s_partial, tid);
    const int64_t n0 = (int64_t)blockIdx.x * NZ_TOKENS;
    if (tid < NZ_TOKENS) {
        const int64_t slot = source_slot(p, s_off, n0 + tid);  // block * block_size + position
        if (slot < 0) {
            s_base[tid] = -1;
        } else {
            const int64_t blk = slot / p.block_size, pos = slot - blk * p.block_size;
            s_base[tid] = ((blk * chunks) * p.block_size + pos) * 32;
        }
    }
    __syncthreads();
    const int64_t chunk_stride = (int64_t)p.block_size * 32;  // bytes between chunk c and c + 1 of one slot
    const int64_t row_bytes = chunks * 32;
    // Software pipeline: the loads of chunk group g + 1 are in flight while
    // group g goes from LDS to the output.
    u32x4 r[NZ_PER_THREAD];
    auto load_group = [&](int64_t c0) __attribute__((always_inline)) {
        // piece q is chunk q / (2 * NZ_TOKENS) of the tile, token (q / 2) % NZ_TOKENS, half q % 2
#pragma unroll
        for (int u = 0; u < NZ_PER_THREAD; ++u) {
            const int q = tid + G_THREADS * u;
            const int cl = q / (2 * NZ_TOKENS), tok = (q >> 1) % NZ_TOKENS, half = q & 1;
            const int64_t base = s_base[tok];
            r[u] = (u32x4){0u, 0u, 0u, 0u};
            if (base >= 0 && c0 + cl < chunks)
                r[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(cache + base + (c0 + cl) * chunk_stride + half * 16));
        }
    };
    load_group(0);
    for (int64_t c0 = 0; c0 < chunks; c0 += NZ_CHUNKS) {
#pragma unroll
        for (int u = 0; u < NZ_PER_THREAD; ++u) {
            const int q = tid + G_THREADS * u;
            const int cl = q / (2 * NZ_TOKENS), tok = (q >> 1) % NZ_TOKENS, half = q & 1;
            *reinterpret_cast<u32x4 *>(tile + tok * NZ_ROW + cl * 32 + half * 16) = r[u];
        }
        __syncthreads();
        if (c0 + NZ_CHUNKS < chunks) load_group(c0 + NZ_CHUNKS);
        // LDS -> output: piece q is token q / (2 * NZ_CHUNKS), chunk (q / 2) % NZ_CHUNKS, half q % 2
#pragma unroll
        for (int u = 0; u < NZ_PER_THREAD; ++u) {
            const int q = tid + G_THREADS * u;
            const int tok = q / (2 * NZ_CHUNKS), cl = (q >> 1) % NZ_CHUNKS, half = q & 1;
            const int64_t n = n0 + tok;
            if (s_base[tok] >= 0 && c0 + cl < chunks)
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(tile + tok * NZ_ROW + cl * 32 + half * 16),
                                            reinterpret_cast<u32x4 *>(out + n * row_bytes + (c0 + cl) * 32 + half * 16));
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_paged_gather(const GatherParams &p, hipStream_t stream) {
    if (p.num_tokens <= 0 || p.batch <= 0) return hipSuccess;
    if (p.nz) {
        const int64_t grid = (p.num_tokens + NZ_TOKENS - 1) / NZ_TOKENS;
        if (grid > INT32_MAX) return hipErrorInvalidValue;
        const size_t shmem = sizeof(int64_t) * ((size_t)p.batch + 1);
        hipLaunchKernelGGL(paged_gather_nz_kernel, dim3((unsigned)grid), dim3(G_THREADS), shmem, stream, p,
                           p.key_cache, p.key, p.chunks_k);
        if (p.value_cache)
            hipLaunchKernelGGL(paged_gather_nz_kernel, dim3((unsigned)grid), dim3(G_THREADS), shmem, stream, p,
                               p.value_cache, p.value, p.chunks_v);
        return hipGetLastError();
    }
    size_t shmem = sizeof(int64_t) * ((size_t)p.batch + 1);
    int64_t steps = (p.num_tokens + G_TOKENS - 1) / G_TOKENS;
    int grid = (int)(steps < G_GRID ? steps : G_GRID);
    hipLaunchKernelGGL(paged_gather_kernel, dim3(grid), dim3(G_THREADS), shmem, stream, p);
    return hipGetLastError();
}

}  // namespace mla
