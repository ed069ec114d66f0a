// MLA varlen prefill attention for gfx950 (MI355X).
//
// Computes, for each sequence of a packed variable-length batch and each
// query head (Ascend Transformer Boost "MLA Prefill" page, Members table rows
// Q, QRope, K, kRope, V, qkScale, Mask, maskType):
//     S = qkScale * (Q . K^T + QRope . KRope^T) + mask,   O = softmax_rows(S) . V
//
// One workgroup = 8 waves = FWD_BM = 256 query rows: 256 rows of one
// (sequence, head), or, when several query heads share a KV head (the page's
// kvHeadNum < headNum), 256 / P rows of each of P = 2, 4 or 8 heads of one
// group, so that every K/V tile staged in LDS is used by all of them.
//
//  * The head dim D (embeddimV) is a template parameter, 64 or 128; the text
//    below gives sizes for D = 128.
//  * Each wave owns 32 query rows of one head. Their Q (32 x 128) and QRope
//    (32 x 64) arrive by DMA into LDS, whole rows per instruction, and are
//    read once into VGPRs, where they stay as the B operand of
//    v_mfma_f32_32x32x16 (8 + 4 k-steps of 16).
//  * Keys are walked in tiles of FWD_BN = 64 through a 3-stage LDS ring. K-nope
//    (64 x 128) and K-rope (64 x 64) of a tile are copied HBM -> LDS by the
//    buffer-load-to-LDS DMA path; so is V (64 x 128), into one of two raw
//    buffers, from which it is transposed LDS -> LDS into the ring stage's
//    V^T (128 x 64), as (key, key + 1) dword pairs. Key rows past the
//    sequence end fall outside the buffer range and arrive as zeros.
//  * LDS rows are XOR-swizzled in 16-byte chunks so that every MFMA operand is
//    one conflict-free 16-byte read per lane, without padding.
//  * Scores are computed transposed, S^T = K . Q^T: the accumulator holds one
//    query row per lane (lanes l and l + 32 share it), so row max / row sum
//    take one cross-lane swap, and the probabilities already sit in the
//    B-operand layout of O^T = V^T . P^T. K rows are stored with bits 2 and 3
//    of the key index swapped, which makes each lane's 8 probabilities of a
//    16-key step consecutive keys, the k-order of a V^T operand read.
//  * Ping-pong schedule. The waves form two groups, one wave of each per
//    SIMD. Workgroup barriers cut time into intervals; in every interval one
//    group runs a matrix block (O += P_j V_j, then S_{j+1} = K_{j+1} Q^T: 40
//    MFMAs fed from LDS a few operands ahead) while the other runs a vector
//    block (mask, row max, online-softmax update and probabilities of one
//    tile), and the roles swap at each barrier. The matrix core of each SIMD
//    is thus fed by one wave while the other wave's softmax runs on the VALU.
//    The leading group issues the K loads during its matrix blocks, the
//    trailing group the V loads and the V transpose during its own, so the
//    vector blocks carry no memory instructions.
//  * The workgroup's work item comes from one 32-byte launch record (one
//    scalar load); only Q and tile 0 are loaded before the first barrier.
//  * Online softmax in fp32 with exp2 (log2(e) folded into the scale), its
//    steps in independent phases (max tree, exponent arguments, exponentials,
//    packing and row sum) so that no instruction waits on the one before. The
//    running max is only moved -- and O rescaled -- when a tile raises some
//    row's max by more than 2^8 in probability units, so most tiles skip the
//    rescale; probabilities stay <= 256 and are rounded to the input dtype for
//    the second product; O is normalised once at the end and rounded to
//    nearest even.
//  * Causal / MASK_FREE: the host work list stops each workgroup at its last
//    visible tile; blocks of tiles a wave cannot see are skipped; only tiles
//    that cut through a wave's rows pay the per-element mask.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernels.h"

namespace mla {
namespace {

constexpr int BM = FWD_BM;
constexpr int BN = FWD_BN;
constexpr int NT = FWD_THREADS;
constexpr int DR = ROPE_DIM;
constexpr int STAGES = 3;
#ifndef MLA_PREFETCH
#define MLA_PREFETCH 2
#endif
#ifndef MLA_LOAD_SPACING
#define MLA_LOAD_SPACING 4
#endif
constexpr int LOAD_SPACING = MLA_LOAD_SPACING;  // MFMAs between the tile loads a matrix block issues
constexpr int PREFETCH = MLA_PREFETCH;  // LDS operands in flight ahead of the MFMA using them
constexpr int KR_BYTES = BN * DR * 2;  // 8 KB
// LDS of a head dim D (embeddimV: 64 or 128). A ring stage holds K-nope
// (64 keys x D), K-rope (64 x 64) and V^T (D x 64 keys); two buffers of raw
// V tiles (64 keys x D, as loaded) follow the ring. D = 128: 40 KB stages,
// 152 KB in all.
template <int D>
struct Geom {
    static constexpr int KN_BYTES = BN * D * 2;
    static constexpr int V_BYTES = BN * D * 2;
    static constexpr int STAGE_BYTES = KN_BYTES + KR_BYTES + V_BYTES;
    static constexpr int VRAW_OFFSET = STAGES * STAGE_BYTES;
    static constexpr int LDS_BYTES = VRAW_OFFSET + 2 * V_BYTES;
    // Q and Q-rope of the 8 waves pass through LDS once, at the start: 32 rows
    // of D + 64 values per wave (a slot). D = 128, inside the ring: a leading
    // wave's slot lies in the K half of stage 1 or 2 (tiles 1 and 2's K lands
    // there after the first barrier, so it is read back before); a trailing
    // wave's slot lies in the V^T half of a stage or in the second raw V
    // buffer, which nothing writes before interval 1, so the trailing group
    // reads its Q back during interval 0 and the first barrier does not wait
    // for it. Tile 0's K (stage 0's K half) and raw V (first raw buffer) load
    // meanwhile. D = 64: past everything else.
    static constexpr int QSLOT_BYTES = 32 * (D + 64) * 2;
    static constexpr int QSTAGE_OFFSET = LDS_BYTES + PAGED_MAX_TILES * 4;
    static constexpr int SMEM_MIN = D == 128 ? 0 : QSTAGE_OFFSET + 8 * QSLOT_BYTES;
    static constexpr int qslot_offset(int grp, int w) {
        return D == 128 ? (grp == 0 ? STAGE_BYTES * (1 + (w >> 1)) + (w & 1) * QSLOT_BYTES
                                    : (w < 3 ? STAGE_BYTES * w + KN_BYTES + KR_BYTES : VRAW_OFFSET + V_BYTES))
                        : QSTAGE_OFFSET + (2 * w + grp) * QSLOT_BYTES;
    }
};
static_assert(2 * Geom<128>::QSLOT_BYTES <= Geom<128>::KN_BYTES + KR_BYTES, "two leading Q slots per K half");
static_assert(Geom<128>::QSLOT_BYTES <= Geom<128>::V_BYTES, "a trailing Q slot per V^T half or raw buffer");
// 16-byte chunk swizzle of an LDS row of D * 2 bytes (K-nope rows, output
// staging rows): chunk c of row r sits at c ^ swz(r), which makes the 16-byte
// reads of 16 consecutive rows (and 8-byte writes of 32) conflict-free.
template <int D>
__device__ __forceinline__ int row_swizzle(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
// The running max moves only when a row's max rises by more than this many
// natural-log units (2^8 in probability), so probabilities stay <= 256.
constexpr float RESCALE_THRESHOLD = 5.545177444479562f;  // 8 ln 2
constexpr float LOG2E = 1.4426950408889634f;

constexpr int MASK_UNDEFINED = 0;
constexpr int MASK_FREE = 3;

// which tile loads a matrix block issues
constexpr int ISS_NONE = 0, ISS_K = 1, ISS_V = 2, ISS_K2 = 3;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned int *lds_u32_ptr;

// Cache policy of a buffer access whose data is used once: non-temporal, so
// that it leaves L2 early instead of the K/V tiles that the items of a head
// share. Set on the Q loads and the output stores (single workload: 1.30 ->
// 1.26 GB of L2 misses per launch, 1.2% faster).
constexpr int CPOL_NT = 2;

// Buffer load with the LDS-DMA bit: lane l's `size` bytes land at lds + l*size.
extern "C" __device__ void mla_raw_buffer_load_lds(i32x4 rsrc, lds_u32_ptr lds, int size, int voffset,
                                                   int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");
extern "C" __device__ i32x4 mla_raw_buffer_load_b128(i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
extern "C" __device__ void mla_raw_buffer_store_b128(i32x4 data, i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.store.v4i32");

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct Bf16 {
    typedef bf16x8 vec8;
    typedef bf16x4 vec4;
    typedef bf16x2 pair;
    typedef __bf16 scalar;
    static __device__ __forceinline__ pair pack(float a, float b) {
        return pair{static_cast<__bf16>(a), static_cast<__bf16>(b)};
    }
    // sum of the two values of a packed pair, in fp32 (exact widening)
    static __device__ __forceinline__ float pair_sum(unsigned w) {
        return __uint_as_float(w << 16) + __uint_as_float(w & 0xffff0000u);
    }
    static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
struct Fp16 {
    typedef f16x8 vec8;
    typedef f16x4 vec4;
    typedef f16x2 pair;
    typedef _Float16 scalar;
    static __device__ __forceinline__ pair pack(float a, float b) {
        return pair{static_cast<_Float16>(a), static_cast<_Float16>(b)};
    }
    static __device__ __forceinline__ float pair_sum(unsigned w) {
        const pair x = __builtin_bit_cast(pair, w);
        return static_cast<float>(x[0]) + static_cast<float>(x[1]);
    }
    static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// Buffer resource over [base, base + bytes): loads past the end return 0,
// stores past the end are dropped. Every argument must be wave-uniform; the
// fields are read from the first lane so the resource lives in SGPRs.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
    r[3] = 0x00020000;
    return r;
}

__device__ __forceinline__ float bits_to_float_bf16(unsigned short b) {
    return __uint_as_float(static_cast<unsigned>(b) << 16);
}
__device__ __forceinline__ float bits_to_float_f16(unsigned short b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max of three scores straight from the MFMA (no NaN canonicalisation)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// max of x over lanes l and l ^ 32
__device__ __forceinline__ float max_with_partner(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return fmaxf(__int_as_float(s[0]), __int_as_float(s[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(s[0]) + __int_as_float(s[1]);
}

// Workgroup barrier without the memory fence __syncthreads() carries: that
// fence makes the compiler wait for every outstanding buffer load, including
// LDS-DMA prefetches still meant to be in flight. Visibility is handled
// explicitly instead: a thread waits (vmcnt) for its own DMA writes before
// the barrier that publishes them, and every LDS read has returned (lgkmcnt)
// before a barrier after which its buffer may be overwritten. The signal
// fences only stop the compiler from moving memory accesses across.
__device__ __forceinline__ void block_sync() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// PAGED: K, KRope and V are read from ND caches through the block table; a
// table of the first cache row of each of the sequence's key tiles sits in
// the LDS past the ring.
constexpr int TILE_TABLE_BYTES = PAGED_MAX_TILES * 4;

// MF: the MASK_FREE instance (the 512 x 512 tile is read on diagonal blocks);
// the other mask types share the other instance.
template <typename T, bool PAGED, int DN, bool MF>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void mla_fwd_kernel(const FwdParams p) {
    constexpr int KN_BYTES = Geom<DN>::KN_BYTES;
    constexpr int STAGE_BYTES = Geom<DN>::STAGE_BYTES;
    constexpr int VRAW_OFFSET = Geom<DN>::VRAW_OFFSET;
    constexpr int V_BYTES = Geom<DN>::V_BYTES;
    constexpr int LDS_BYTES = Geom<DN>::LDS_BYTES;
    constexpr int KN_ROW = DN * 2;      // LDS bytes of a K-nope row
    constexpr int NKS = DN / 16;        // k-steps of the nope product
    constexpr int NDB = DN / 32;        // 32-column blocks of O
    constexpr int NV = 4 * NDB;         // V^T operands of a matrix block (4 key steps x NDB)
    constexpr int KN_LOADS = DN / 32;   // K-nope DMA per leading thread and tile
    constexpr int CPT = DN / 64;        // V column chunk pairs per leading thread
    constexpr int V_LOADS = 2 * CPT;    // raw V DMA per trailing thread and tile
    constexpr int SMEM_BYTES = LDS_BYTES + (PAGED ? TILE_TABLE_BYTES : 0) > Geom<DN>::SMEM_MIN
                                   ? LDS_BYTES + (PAGED ? TILE_TABLE_BYTES : 0)
                                   : Geom<DN>::SMEM_MIN;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM_BYTES];
    typedef typename T::vec8 vec8;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int grp = wave >> 2;  // 0: leading group, 1: trailing group (one interval behind)
    const int g = lane >> 5;    // which 8 of each 16 k-slots this lane carries
    const int r32 = lane & 31;  // query row within the wave

    // The host's task list says which work item and head this workgroup runs
    // (launch order and XCD placement are chosen there); padding tasks exit.
    const LaunchRec task = p.launch[blockIdx.x];
    if (task.head < 0) return;
    // The wave's 32-row slot: slot s holds head task.head + s % P and rows
    // 32 * (s / P) .. + 31 of the item (P = 2^pack_shift heads per task). The
    // two waves sharing a SIMD (w, w + 4) take slots 2(w & 3) and 2(w & 3) + 1:
    // adjacent row blocks, or the same rows of two heads, so both groups see
    // the same share of diagonal tiles.
    const int ps = p.pack_shift;
    const int slot = (wave & 3) * 2 + grp;
    const int h = task.head + (slot & ((1 << ps) - 1));
    const int hk = task.kv_head;
    const int H = p.heads, HKV = p.kv_heads;
    const int q_left = task.q_left;  // rows of the sequence from the item's first row on
    const int kv_len = task.kv_len;
    const int n_kt = task.kv_tiles;
    const int mask_type = MF ? MASK_FREE : p.mask_type;
    const bool causal_like = !MF && mask_type != MASK_UNDEFINED;

    const int lrow0 = (slot >> ps) * 32;            // first row of this wave within the item
    const int wpos0 = kv_len - q_left + lrow0;      // key positions of the wave's rows
    const int pos = wpos0 + r32;                    // ... and of this lane's row
    const int wpos1 = wpos0 + 31;

    // MASK_FREE: this lane's row of the tile classes (see the tile visibility
    // below), loaded ahead of the DMA so that its latency overlaps theirs
    uint64_t mask_cls_row = 0;
    if (MF && p.mask_cls != nullptr)
        mask_cls_row = *reinterpret_cast<const uint64_t *>(p.mask_cls + (size_t)(pos & (MASK_TILE - 1)) * 8);

    // ---- Q and Q-rope of the wave's 32 rows go HBM -> LDS by DMA, whole rows
    // per instruction (4 rows of Q-nope, or 8 of Q-rope, per 1 KB), into the
    // wave's staging slot; they are read back into VGPRs below as the B
    // operand of S^T = K . Q^T (lane: row r32, k-slots g*8 .. g*8+7 of each
    // 16-wide k-step). A direct VGPR load would touch 32 rows, 32 bytes each,
    // per instruction. Chunk c of staged row r sits at c ^ swizzle(r), which
    // keeps the read-back conflict-free. Rows past the end read as 0.
    constexpr int QN_INSTR = DN / 16;          // 1 KB DMA instructions for Q-nope
    constexpr int QN_CPR = DN / 8;             // 16-byte chunks of a Q-nope row
    unsigned char *qslot = smem + Geom<DN>::qslot_offset(grp, wave & 3);
    {
        const int rows = max(0, min(32, q_left - lrow0));
        const int64_t tok = (int64_t)task.q_tok0 + lrow0;
        const i32x4 rq = make_rsrc(static_cast<const unsigned char *>(p.q) + (tok * H + h) * (DN * 2),
                                   (uint32_t)rows * H * DN * 2);
        const i32x4 rr = make_rsrc(static_cast<const unsigned char *>(p.q_rope) + (tok * H + h) * (DR * 2),
                                   (uint32_t)rows * H * DR * 2);
#pragma unroll
        for (int u = 0; u < QN_INSTR; ++u) {
            const int r = u * (64 / QN_CPR) + lane / QN_CPR, c = (lane % QN_CPR) ^ row_swizzle<DN>(r);
            mla_raw_buffer_load_lds(rq, (lds_u32_ptr)(qslot + u * 1024), 16, (uint32_t)r * H * DN * 2 + c * 16, 0,
                                    0, CPOL_NT);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = u * 8 + lane / 8, c = (lane % 8) ^ ((r >> 1) & 7);
            mla_raw_buffer_load_lds(rr, (lds_u32_ptr)(qslot + 32 * DN * 2 + u * 1024), 16,
                                    (uint32_t)r * H * DR * 2 + c * 16, 0, 0, CPOL_NT);
        }
    }
    constexpr int Q_LOADS = QN_INSTR + 4;
    vec8 qreg[NKS], qrreg[4];

    // ---- paged K/V: first cache row of each key tile of the task (block
    // size is a multiple of the tile, so a tile never straddles two blocks);
    // -1 for a tile whose block id lies outside the cache, which then reads
    // as zeros like rows past the sequence end. A run of a split item starts
    // at tile kt0 of its sequence.
    int32_t *tile_row = reinterpret_cast<int32_t *>(smem + LDS_BYTES);
    const int n_tiles_seq = min((kv_len + BN - 1) / BN, PAGED_MAX_TILES);
    if (PAGED) {
        const int tpb = p.block_size / BN;
        const int seq = task.kv_off & ((1 << PAGED_SEQ_BITS) - 1), kt0 = task.kv_off >> PAGED_SEQ_BITS;
        const int32_t *bt = p.block_tables + (int64_t)seq * p.bt_stride;
        for (int i = tid; i < n_tiles_seq; i += NT) {
            const int gi = i + kt0, bi = gi / tpb;
            const int blk = bt[bi];
            tile_row[i] = (blk >= 0 && blk < p.num_blocks) ? blk * p.block_size + (gi - bi * tpb) * BN : -1;
        }
        block_sync();
    }

    // ---- K / V tile streaming. Tile kt lives in ring stage kt % 3.
    //  * K-nope and K-rope go HBM -> LDS by DMA. Row m of the K tile holds key
    //    perm(m), perm swapping bits 2 and 3 of the key index, so that after
    //    S^T = K . Q^T each lane's probabilities of a 16-key step are 8
    //    consecutive keys (what the V^T operand read below needs).
    //  * V goes HBM -> LDS by DMA too, into a raw buffer, and is transposed
    //    into V^T[d][key] of its stage one interval later.
    const unsigned char *kbase = static_cast<const unsigned char *>(p.k);
    const unsigned char *krbase = static_cast<const unsigned char *>(p.k_rope);
    const unsigned char *vbase = static_cast<const unsigned char *>(p.v);
    const uint32_t kn_row = (uint32_t)HKV * DN * 2;  // bytes between consecutive keys
    const uint32_t kr_row = (uint32_t)HKV * DR * 2;
    auto perm_key = [](int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); };
    // Per tile, the leading group (waves 0-3, threads 0..LT-1) issues the K
    // DMA, six per thread: K-nope in four (slot tid + LT*u: row slot / 16,
    // chunk slot % 16), K-rope in two (row slot / 8, chunk slot % 8); the
    // trailing group issues the raw V DMA (below). In the loop they go out one
    // every four MFMAs of the group's matrix block, so no wave stalls behind a
    // burst of address work in the texture unit and the vector blocks issue
    // no memory instruction at all.
    constexpr int LT = NT / 2;
    uint32_t off_kn[KN_LOADS], off_kr[2];
#pragma unroll
    for (int u = 0; u < KN_LOADS; ++u) {
        const int slot = tid + LT * u;
        const int m = slot / (DN / 8);  // tile row; DN / 8 chunks of 16 bytes each
        off_kn[u] = perm_key(m) * kn_row + (((slot % (DN / 8)) ^ row_swizzle<DN>(m)) << 4);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int slot = tid + LT * u;
        const int m = slot >> 3;
        off_kr[u] = perm_key(m) * kr_row + (((slot & 7) ^ ((m >> 1) & 7)) << 4);
    }
    // Raw V tiles land by DMA in one of two LDS buffers (tile kt in buffer
    // kt % 2) in their global row order; 16-byte chunk c of key row m sits at
    // chunk position c ^ vswz(m), so that the transposing reads below, 16 keys
    // of one chunk per quarter wave, are conflict-free (D = 128). Either group
    // issues them: load j of thread i of a group (i = tid % LT) fills LDS slot
    // j * LT + i of the buffer.
    const int kp = tid & 31, dg = (tid >> 5) & 7;  // V^T writer: keys 2kp, 2kp + 1; column chunks of dg
    constexpr int CPR = DN / 8;  // 16-byte chunks of a V row
    auto vswz = [](int m) { return (m >> 1) & (CPR - 1); };
    uint32_t off_vr[V_LOADS];
#pragma unroll
    for (int u = 0; u < V_LOADS; ++u) {
        const int slot = (tid & (LT - 1)) + LT * u;
        const int m = slot / CPR;
        off_vr[u] = m * kn_row + (((slot % CPR) ^ vswz(m)) << 4);
    }
    struct TileLoad {
        i32x4 rk, rr, rv;
        unsigned char *st;  // ring stage
        unsigned char *vr;  // raw V buffer
    };
    // paged: first cache row of tile kt (-1: none), read from the LDS table
    // ahead of prep_tile so the read's latency stays off the matrix block
    auto cache_row_ld = [&](int kt) __attribute__((always_inline)) -> int {
        if (!PAGED) return 0;
        return kt < n_tiles_seq ? tile_row[kt] : -1;
    };
    auto cache_row = [&](int kt) __attribute__((always_inline)) -> int {
        if (!PAGED) return 0;
        return __builtin_amdgcn_readfirstlane(cache_row_ld(kt));
    };
    auto prep_tile = [&](int kt, int r) __attribute__((always_inline)) -> TileLoad {
        int64_t rowi;     // first key row of the tile, this head
        uint32_t nvalid;  // rows that hold keys of the sequence
        if (PAGED) {
            rowi = r >= 0 ? (int64_t)r * HKV + hk : 0;
            nvalid = r >= 0 ? (uint32_t)max(0, min(kv_len - kt * BN, BN)) : 0u;
        } else {
            rowi = ((int64_t)task.kv_off + (int64_t)kt * BN) * HKV + hk;
            nvalid = (uint32_t)max(0, min(kv_len - kt * BN, BN));
        }
        TileLoad tl;
        tl.rk = make_rsrc(kbase + rowi * (DN * 2), nvalid * kn_row);
        tl.rr = make_rsrc(krbase + rowi * (DR * 2), nvalid * kr_row);
        tl.rv = make_rsrc(vbase + rowi * (DN * 2), nvalid * kn_row);
        tl.st = smem + (kt % STAGES) * STAGE_BYTES;
        tl.vr = smem + VRAW_OFFSET + (kt & 1) * V_BYTES;
        return tl;
    };
    // A leading thread's loads of a tile: six K DMA (K_LOADS) and four V loads
    // (V_LOADS). V load j lands in vst[j]: key 2kp + (j & 1), column chunk
    // 2dg + (j >> 1).
    constexpr int K_LOADS = KN_LOADS + 2;
    // every load of a matrix block has an MFMA slot
    static_assert(K_LOADS * LOAD_SPACING <= NV + 2 * (NKS + 4), "matrix block too short for its loads");
    static_assert(V_LOADS * LOAD_SPACING <= 2 * (NKS + 4), "scores-only block too short for the V loads");
    static_assert(V_LOADS * LT * 16 == V_BYTES, "raw V DMA must fill the buffer");
    auto issue_k = [&](const TileLoad &tl, int i) __attribute__((always_inline)) {
        const int wofs = wave * 64 * 16;
        if (i < KN_LOADS)
            mla_raw_buffer_load_lds(tl.rk, (lds_u32_ptr)(tl.st + i * LT * 16 + wofs), 16, off_kn[i], 0, 0, 0);
        else
            mla_raw_buffer_load_lds(tl.rr, (lds_u32_ptr)(tl.st + KN_BYTES + (i - KN_LOADS) * LT * 16 + wofs), 16,
                                    off_kr[i - KN_LOADS], 0, 0, 0);
    };
    auto issue_v = [&](const TileLoad &tl, int j) __attribute__((always_inline)) {
        mla_raw_buffer_load_lds(tl.rv, (lds_u32_ptr)(tl.vr + j * LT * 16 + (wave & 3) * 64 * 16), 16, off_vr[j],
                                0, 0, 0);
    };
    // The transposing read: a leading thread (kp, dg) takes the 16-byte chunks
    // it writes as V^T below from a raw buffer; chunk j is key 2kp + (j & 1),
    // column chunk CPT dg + (j >> 1).
    auto read_vraw = [&](const unsigned char *vr, uint4 *vst) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < V_LOADS; ++j) {
            const int m = 2 * kp + (j & 1), cc = CPT * dg + (j >> 1);
            vst[j] = *reinterpret_cast<const uint4 *>(vr + m * (DN * 2) + ((cc ^ vswz(m)) << 4));
        }
    };
    // V^T region of a stage: row d (128 B = 64 keys), 16-byte chunk c (8 keys)
    // at position c ^ ((d >> 1) & 7). A leading thread writes the dwords
    // (key 2kp, 2kp + 1) of rows 16dg .. 16dg + 15: for d = 16dg + 8h + 2dd (+1),
    // (d >> 1) & 7 = 4h + dd, so the offset is vw_base ^ ((4h + dd) << 4) plus
    // 1024h + 256dd (+128).
    // (DN = 64: one chunk per thread, d = 8dg + 2dd; (d >> 1) & 7 = 4(dg & 1) + dd,
    // so the 4(dg & 1) part goes into the base.)
    const uint32_t vw_base = KN_BYTES + KR_BYTES + dg * (CPT * 1024) +
                             (((kp >> 2) ^ (CPT == 1 ? 4 * (dg & 1) : 0)) << 4) + (kp & 3) * 4;
    // piece q = 4h + dd of the V^T write: dword dd of chunk pair h, keys
    // 2kp (vst[2h]) and 2kp + 1 (vst[2h + 1]) -> two V^T rows
    constexpr int VT_PIECES = 4 * CPT;
    auto write_vt_piece = [&](unsigned char *st, uint32_t vwb, int q, const uint4 *vst)
                              __attribute__((always_inline)) {
        const int h = q >> 2, dd = q & 3;
        const unsigned a = reinterpret_cast<const unsigned *>(&vst[2 * h])[dd];
        const unsigned b = reinterpret_cast<const unsigned *>(&vst[2 * h + 1])[dd];
        const uint32_t w = (vwb ^ ((4 * h + dd) << 4)) + h * 1024 + dd * 256;
        *reinterpret_cast<unsigned *>(st + w) = __builtin_amdgcn_perm(b, a, 0x05040100u);
        *reinterpret_cast<unsigned *>(st + w + 128) = __builtin_amdgcn_perm(b, a, 0x07060302u);
    };
    // the transpose and the next raw V loads alone, for a trailing wave that
    // runs no matrix block
    auto transpose_v = [&](const unsigned char *vr, uint32_t st, const TileLoad &tl) __attribute__((always_inline)) {
        uint4 vst[V_LOADS];
        read_vraw(vr, vst);
        uint32_t vwb = vw_base + st;
        asm volatile("" : "+v"(vwb));
#pragma unroll
        for (int q = 0; q < VT_PIECES; ++q) write_vt_piece(smem, vwb, q, vst);
#pragma unroll
        for (int i = 0; i < V_LOADS; ++i) issue_v(tl, i);
    };

    // Loads of a tile past the last one have no valid rows (they return
    // zeros) and land in a ring stage or raw buffer no longer read, so they
    // are issued unconditionally.
    // Tile t's K goes out (leading group) four intervals before its first
    // scores: a stage's K region is free once the trailing group has scored
    // the tile before. Its raw V goes out (trailing group) right after the
    // transpose of tile t-1, two intervals before its own.
    // Q read back from the wave's own staging slot once its own DMA has
    // landed. A negative scale is folded into Q so the row max can be taken on
    // raw scores: Q-nope and Q-rope are negated in registers.
    auto read_q = [&]() __attribute__((always_inline)) {
        const uint32_t qn = (uint32_t)r32 * (DN * 2) + ((g ^ row_swizzle<DN>(r32)) << 4);
        const uint32_t qr = 32 * DN * 2 + (uint32_t)r32 * 128 + ((g ^ ((r32 >> 1) & 7)) << 4);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qreg[ks] = __builtin_bit_cast(vec8, *reinterpret_cast<const uint4 *>(qslot + (qn ^ (ks << 5))));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qrreg[ks] = __builtin_bit_cast(vec8, *reinterpret_cast<const uint4 *>(qslot + (qr ^ (ks << 5))));
        if (p.qk_scale < 0.f) {
#pragma unroll
            for (int ks = 0; ks < NKS + 4; ++ks) {
                vec8 &q = ks < NKS ? qreg[ks] : qrreg[ks - NKS];
                i32x4 w = __builtin_bit_cast(i32x4, q);
                w ^= (int)0x80008000;
                q = __builtin_bit_cast(vec8, w);
            }
        }
    };
    // Before the first barrier only what interval 0 needs is loaded: the
    // leading group's Q and tile 0's K (the leading group scores it); tile 0's
    // raw V goes out too and is waited for at the end of interval 0. The
    // trailing group waits for its own Q during interval 0. The K of tiles 1
    // and 2 goes out during interval 0 (into ring stages that hold the leading
    // group's Q staging until the first barrier).
    if (grp == 0) {
        const TileLoad t0 = prep_tile(0, cache_row(0));
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) issue_k(t0, i);
#pragma unroll
        for (int j = 0; j < V_LOADS; ++j) issue_v(t0, j);
        __builtin_amdgcn_s_waitcnt(0x0F70 | V_LOADS);  // Q, Q-rope and K of tile 0 landed
        read_q();
    }
    static_assert(Q_LOADS + K_LOADS + V_LOADS <= 63, "vmcnt range");

    // natural-log units per unit of the raw dot product, and log2 units. A zero
    // scale is taken as 1e-30, so that a masked -inf times the scale stays
    // -inf: every score it yields is then so small that exp2 rounds it to
    // exactly 1, as 0 would.
    const float c_nat = fmaxf(fabsf(p.qk_scale), 1e-30f);
    const float c2 = c_nat * LOG2E;

    // ---- per-wave tile visibility. Under every mask mode the tiles some row
    // of the wave can see, and the tiles every row sees whole, are prefixes of
    // the item's tile range, so two wave-uniform counts decide both questions
    // with one compare each.
    //  * visible: causal modes, key0 <= wpos1; MASK_FREE, the key block (512
    //    keys) is not after the last row's block; UNDEFINED, every tile.
    //  * whole: the tile lies inside the sequence (key0 + 64 <= kv_len) and,
    //    for the causal modes, its last key is <= wpos0; for MASK_FREE its
    //    512-key block lies before the first row's block.
    int kt_vis = n_kt, kt_full = kv_len / BN;
    if (causal_like) {
        kt_vis = min(n_kt, wpos1 >= 0 ? wpos1 / BN + 1 : 0);
        kt_full = min(kt_full, max(0, (wpos0 + 1) / BN));
    } else if (MF) {
        kt_vis = min(n_kt, wpos1 >= 0 ? ((wpos1 >> 9) + 1) * (MASK_TILE / BN) : 0);
        kt_full = min(kt_full, wpos0 >= 0 ? (wpos0 >> 9) * (MASK_TILE / BN) : 0);
    }
    // MASK_FREE with a classified tile, the wave's rows all in one 512-key
    // block: within that block, a leading run of 64-key tiles whose tile
    // entries are 0 for every row of the wave is whole (a zero entry gives
    // the unmasked arguments bit for bit), and tiles past the last one with
    // any entry other than -inf for some row are invisible (such a tile
    // changes no row's state). With the causal tile this gives the causal
    // mode's counts.
    if (MF && p.mask_cls != nullptr && wpos0 >= 0 && (wpos0 >> 9) == (wpos1 >> 9)) {
        uint64_t zero_bits = 0, live_bits = 0;  // tile k of the block: zero for every row / live for some row
#pragma unroll
        for (int k = 0; k < MASK_TILE / BN; ++k) {
            const uint32_t c = (uint32_t)(mask_cls_row >> (8 * k)) & 0xffu;
            if (__builtin_amdgcn_ballot_w64(c == MASK_CLS_ZERO) == ~0ull) zero_bits |= 1ull << k;
            if (__builtin_amdgcn_ballot_w64(c != MASK_CLS_DEAD) != 0ull) live_bits |= 1ull << k;
        }
        const int diag0 = (wpos0 >> 9) * (MASK_TILE / BN);
        const int run = __builtin_ctzll(~zero_bits);  // leading tiles zero for every row (at most 8)
        const int live = live_bits != 0 ? 63 - __builtin_clzll(live_bits) : -1;  // last live tile, or -1
        kt_full = min(kv_len / BN, diag0 + run);
        kt_vis = min(kt_vis, diag0 + live + 1);
    }
    kt_vis = __builtin_amdgcn_readfirstlane(kt_vis);
    kt_full = __builtin_amdgcn_readfirstlane(kt_full);
    // can any of the wave's rows see any key of tile kt?
    auto wave_active = [&](int kt) __attribute__((always_inline)) -> bool {
        return (unsigned)kt < (unsigned)kt_vis;
    };
    // does every row of the wave see every key of it (no per-element mask)?
    auto wave_full = [&](int kt) __attribute__((always_inline)) -> bool { return kt < kt_full; };

    // ---- per-lane LDS read offsets. With the XOR swizzles, the offset of
    // step k (k-step, or 16-key step for V^T) is base ^ (k << 5) for one base
    // per operand kind; the key block / column block adds a multiple of 4 KB
    // or 8 KB. Each matrix block forms its addresses from an opaque copy of
    // the bases (one VALU op per read) instead of keeping 24 of them live.
    //  K-nope (A of S^T): tile row kb*32 + r32, chunk 2*ks + g, swizzle ^ (row & 15)
    //  K-rope:            row kb*32 + r32, chunk 2*ks + g, swizzle ^ ((row >> 1) & 7)
    //  V^T (A of O^T):    row d = 32*db + r32, chunk 2*st4 + g, swizzle ^ ((d >> 1) & 7)
    const uint32_t kn_base = r32 * KN_ROW + ((g ^ row_swizzle<DN>(r32)) << 4);
    const uint32_t kr_base = KN_BYTES + r32 * 128 + ((g ^ ((r32 >> 1) & 7)) << 4);
    const uint32_t vt_base = KN_BYTES + KR_BYTES + r32 * 128 + ((g ^ ((r32 >> 1) & 7)) << 4);

    auto lds16 = [](const unsigned char *a) __attribute__((always_inline)) -> vec8 {
        return __builtin_bit_cast(vec8, *reinterpret_cast<const uint4 *>(a));
    };
    // operand n of a matrix block: n < NV -> V^T of (16-key step n / NDB, column
    // block n % NDB) from stage sv; n >= NV -> K of (k-step (n - NV) / 2, key
    // block (n - NV) % 2) from sk, the first NKS k-steps nope, the last 4 rope
    // The bases passed in carry their stage's byte offset (a multiple of 8 KB,
    // so it never meets the XOR-ed bits).
    auto load_operand = [&](int n, uint32_t knb, uint32_t krb, uint32_t vtb) __attribute__((always_inline)) -> vec8 {
        if (n < NV) return lds16(smem + (vtb ^ ((n / NDB) << 5)) + (n % NDB) * 32 * 128);
        const int ks = (n - NV) >> 1, kb = (n - NV) & 1;
        if (ks < NKS) return lds16(smem + (knb ^ (ks << 5)) + kb * 32 * KN_ROW);
        return lds16(smem + (krb ^ ((ks - NKS) << 5)) + kb * 32 * 128);
    };
    static_assert(STAGE_BYTES % 8192 == 0 && (KN_BYTES + KR_BYTES) % 8192 == 0, "stage offsets must clear the swizzle bits");

    // ---- softmax state
    float m_run = -INFINITY;  // running row max, natural-log units (same in both lanes of a row)
    float l_run = 0.f;        // this lane's share of the running row sum
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
    // scores of one tile; element e of block kb is key
    // kb*32 + 16*(e/8) + 8*g + (e%8) of the tile (see perm_key)
    f32x16 s[2];
    vec8 pb[4];  // P^T operands of the four 16-key steps

    // ---- matrix block: O += P . V (tile in stage sv) then S = K . Q^T (tile in
    // stage sk); either half may be switched off. Operands are read ahead.
    // ISS: ISS_K issues the K loads of tile tlk, ISS_V the raw V loads of tile
    // tlv, one load every LOAD_SPACING MFMAs (after MFMAs LOAD_SPACING - 1,
    // 2 LOAD_SPACING - 1, ...). VT:
    // transpose the raw V tile in buffer vt_src into V^T of stage vt_st: the
    // raw chunks are read ahead of the first MFMA, and the V^T writes go out
    // one piece after each of the first MFMAs (a burst of these writes ahead
    // of the block held back its first MFMA).
    auto mfma_block = [&](uint32_t sv, uint32_t sk, auto do_pv, auto do_qk, auto do_iss, auto do_vt,
                          const TileLoad &tlv, const TileLoad &tlk, const unsigned char *vt_src, uint32_t vt_st)
                          __attribute__((always_inline)) {
        constexpr bool PV = decltype(do_pv)::value, QK = decltype(do_qk)::value;
        constexpr int ISS = decltype(do_iss)::value;
        constexpr bool VT = decltype(do_vt)::value;
        // ISS_K2 (tile 0's scores only): the K of two tiles, tlv's then tlk's,
        // one load every other MFMA
        constexpr int NLOADS = ISS == ISS_K ? K_LOADS : (ISS == ISS_V ? V_LOADS : (ISS == ISS_K2 ? 2 * K_LOADS : 0));
        constexpr int SPACING = ISS == ISS_K2 ? 2 : LOAD_SPACING;
        constexpr int n0 = PV ? 0 : NV, n1 = QK ? NV + 2 * (NKS + 4) : NV;
        static_assert(NLOADS * SPACING <= n1 - n0, "matrix block too short for its loads");
        // the wave feeding the matrix core wins issue arbitration against the
        // other wave of its SIMD, which runs a vector block meanwhile
        __builtin_amdgcn_s_setprio(1);
        if (QK) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
        }
        uint32_t knb = kn_base + sk, krb = kr_base + sk, vtb = vt_base + sv, vwb = vw_base + vt_st;
        asm volatile("" : "+v"(knb), "+v"(krb), "+v"(vtb));
        if (VT) asm volatile("" : "+v"(vwb));
        // raw V chunks first: LDS returns in order, so they have landed by the
        // time the first ring operand is waited for
        uint4 vst[V_LOADS];
        if (VT) read_vraw(vt_src, vst);
        vec8 ring[PREFETCH + 1];
#pragma unroll
        for (int d = 0; d < PREFETCH; ++d)
            if (n0 + d < n1) ring[d] = load_operand(n0 + d, knb, krb, vtb);
#pragma unroll
        for (int n = n0; n < n1; ++n) {
            if (n + PREFETCH < n1)
                ring[(n + PREFETCH - n0) % (PREFETCH + 1)] = load_operand(n + PREFETCH, knb, krb, vtb);
            __builtin_amdgcn_sched_barrier(0);
            const vec8 a = ring[(n - n0) % (PREFETCH + 1)];
            if (n < NV) {
                o[n % NDB] = T::mfma(a, pb[n / NDB], o[n % NDB]);
            } else {
                const int ks = (n - NV) >> 1, kb = (n - NV) & 1;
                s[kb] = T::mfma(a, ks < NKS ? qreg[ks] : qrreg[ks - NKS], s[kb]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (VT && n - n0 < VT_PIECES) {
                write_vt_piece(smem, vwb, n - n0, vst);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (NLOADS && (n - n0) % SPACING == SPACING - 1 && (n - n0) / SPACING < NLOADS) {
                const int li = (n - n0) / SPACING;
                if (ISS == ISS_V) issue_v(tlv, li);
                else if (ISS == ISS_K2 && li < K_LOADS) issue_k(tlv, li);
                else if (ISS == ISS_K2) issue_k(tlk, li - K_LOADS);
                else issue_k(tlk, li);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- vector block for tile kt: mask (if needed), row max, lazy rescale,
    // probabilities -> pb, row sums. The running max m_run is kept in
    // natural-log units (|qkScale| * dot + tile entry). The scores stay raw dot
    // products, rewritten in place: the causal and undefined masks set masked
    // keys to -inf; the row max of the raw scores, scaled, is the tile's max;
    // the exponent arguments are one fma, s * c2 - m_run * log2(e). A
    // MASK_FREE tile on the diagonal block takes its max on
    // fma(s, |qkScale|, entry) over the visible keys and its arguments are
    // fma(s, c2, (entry - m_run) * log2(e)), -inf where masked: with a zero
    // entry that is the plain fma bit for bit (so MASK_FREE with a causal tile
    // equals CAUSAL exactly), a tile entry is never divided by the scale, and
    // an entry near the largest finite value only meets a running max of its
    // own size. Every path rewrites the scores in place: with a separate
    // result per path the compiler copied all 32 scores where they merge.
    const i32x4 mask_rsrc = make_rsrc(p.mask, MF ? MASK_TILE * MASK_TILE * 2 : 0);
    auto valu_block = [&](int kt) __attribute__((always_inline)) {
        const bool full = wave_full(kt);
        // Masked tile: element e is key key0 + 8g + off(e), visible iff
        // off(e) <= lim (one limit per lane). Key j is visible iff j <= min(pos,
        // kv_len - 1) (causal modes) or j <= kv_len - 1 (UNDEFINED). MASK_FREE:
        // a 64-key tile lies inside one 512-key block, so the block rule gives
        // one limit too: keys of an earlier block are visible (up to kv_len - 1),
        // of a later one not; on the diagonal block the row of the 512 x 512
        // tile is added, read as four 16-byte runs of 8 entries (the keys
        // 8g + 32kb + 16h + 0..7; the host accepts only 16-byte aligned tiles).
        // Lanes off the diagonal block read past the tile's end, which returns
        // zeros, so the entry is 0 there without a branch.
        auto off_of = [](int e) { return (e >> 4) * 32 + 16 * ((e & 15) >> 3) + (e & 7); };
        int lim = 0;
        uint32_t mw[16];
        auto entry = [&](int e) __attribute__((always_inline)) -> float {
            const uint32_t w = mw[e >> 1];
            const unsigned short b = (unsigned short)(w >> (16 * (e & 1)));
            return p.mask_is_bf16 ? bits_to_float_bf16(b) : bits_to_float_f16(b);
        };
        if (!full) {
            const int key0 = kt * BN;
            if (!MF) {
                lim = (causal_like ? min(pos, kv_len - 1) : kv_len - 1) - key0 - 8 * g;
#pragma unroll
                for (int e = 0; e < 32; ++e) s[e >> 4][e & 15] = off_of(e) <= lim ? s[e >> 4][e & 15] : -INFINITY;
            } else {
                const int jb = key0 >> 9, pblk = pos >> 9;
                lim = (pos < 0 || jb > pblk) ? -1 : kv_len - 1 - key0 - 8 * g;
                int pp = pos;  // formed here: kept live across the loop it would cost registers
                asm volatile("" : "+v"(pp));
                const uint32_t mo = (pp >= 0 && jb == pblk)
                                        ? (uint32_t)(((pp & (MASK_TILE - 1)) * MASK_TILE + (key0 & (MASK_TILE - 1)) +
                                                      8 * g) * 2)
                                        : 0x40000000u;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const i32x4 w = mla_raw_buffer_load_b128(mask_rsrc, mo + (q >> 1) * 64 + (q & 1) * 32, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) mw[4 * q + i] = (uint32_t)w[i];
                }
            }
        }
        // Row max as a tree of three-input maxima (no NaN canonicalisation: the
        // scores come straight from the MFMA), in natural-log units.
        float lane_max = 0.f;  // this lane's own max (before its partner's), as max_tree takes it
        auto max_tree = [&](auto val) __attribute__((always_inline)) -> float {
            float t[11];
#pragma unroll
            for (int i = 0; i < 10; ++i) t[i] = max3f(val(3 * i), val(3 * i + 1), val(3 * i + 2));
            const float v31 = val(31);
            t[10] = max3f(val(30), v31, v31);
            const float u0 = max3f(t[0], t[1], t[2]), u1 = max3f(t[3], t[4], t[5]), u2 = max3f(t[6], t[7], t[8]);
            const float u3 = max3f(t[9], t[10], u2);
            lane_max = max3f(u0, u1, u3);
            return max_with_partner(lane_max);
        };
        const bool mf_masked = MF && !full;
        float mx;
        if (!mf_masked) {
            // the scale is > 0, so it commutes with the max (and keeps -inf)
            mx = max_tree([&](int e) { return s[e >> 4][e & 15]; }) * c_nat;
        } else {
            mx = max_tree([&](int e) {
                return off_of(e) <= lim ? __builtin_fmaf(s[e >> 4][e & 15], c_nat, entry(e)) : -INFINITY;
            });
        }
        // move the running max only if some row of the wave rose past the threshold
        const bool need = mx - m_run > RESCALE_THRESHOLD;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2((m_run - m_new) * LOG2E);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
            m_run = m_new;
        }
        const float mr = (m_run == -INFINITY) ? 0.f : m_run;
        // Probabilities in independent phases -- all exponent arguments, then
        // all exponentials, then the packing and the row sum -- so that no
        // instruction waits on the one just before it.
        const float m2 = mr * LOG2E;
        float pm_arg;  // exponent argument of the lane's largest probability (for the row sum below)
        if (!mf_masked) {
            pm_arg = __builtin_fmaf(lane_max, c2, -m2);
#pragma unroll
            for (int t = 0; t < 32; ++t) s[t >> 4][t & 15] = __builtin_fmaf(s[t >> 4][t & 15], c2, -m2);
        } else {
#pragma unroll
            for (int t = 0; t < 32; ++t)
                s[t >> 4][t & 15] = off_of(t) <= lim
                                        ? __builtin_fmaf(s[t >> 4][t & 15], c2, (entry(t) - mr) * LOG2E)
                                        : -INFINITY;
            // the fma is monotone in the score, so with zero entries this is
            // the other path's value bit for bit
            (void)max_tree([&](int e) { return s[e >> 4][e & 15]; });
            pm_arg = lane_max;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 32; ++t) s[t >> 4][t & 15] = fast_exp2(s[t >> 4][t & 15]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 32; t += 2) {
            const int kb = t >> 4, e = t & 15;
            const typename T::pair pr = T::pack(s[kb][e], s[kb][e + 1]);
            pb[kb * 2 + (e >> 3)][e & 7] = pr[0];
            pb[kb * 2 + (e >> 3)][(e & 7) + 1] = pr[1];
        }
        {
            // Row sum in fp32. The P.V product sees each probability rounded to
            // the input dtype; for the lane's largest one the sum takes the
            // rounded value too, so a row whose weight sits on one key returns
            // that key's values whatever the rounding (with bf16 and a large
            // scale that rounding error, up to 2^-8 of the output, was the
            // largest one). The other probabilities' rounding errors weigh
            // with their (smaller) share of the row.
            float a[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) a[i] = s[(2 * i) >> 4][(2 * i) & 15] + s[(2 * i + 1) >> 4][(2 * i + 1) & 15];
#pragma unroll
            for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
                for (int i = 0; i < w; ++i) a[i] += a[i + w];
            {
                const float pm = fast_exp2(pm_arg);  // that probability, bit for bit
                const typename T::pair pr = T::pack(pm, 0.f);
                a[0] += T::pair_sum(__builtin_bit_cast(unsigned, pr)) - pm;
            }
            l_run += a[0];
        }
    };

    const std::integral_constant<bool, true> yes{};
    const std::integral_constant<bool, false> no{};
    const TileLoad none{};  // placeholder for blocks that issue nothing
    const std::integral_constant<int, ISS_NONE> iss_none{};
    const std::integral_constant<int, ISS_K> iss_k{};
    const std::integral_constant<int, ISS_V> iss_v{};
    const std::integral_constant<int, ISS_K2> iss_k2{};
    // byte offset of ring stage r
    auto soff = [&](int r) __attribute__((always_inline)) -> uint32_t { return (uint32_t)r * STAGE_BYTES; };

    // ---- schedule. Interval 0: leading group scores tile 0. Then for each tile
    // j two intervals:
    //   2j+1: leading: vector block j        trailing: PV j-1 + scores j
    //   2j+2: leading: PV j + scores j+1     trailing: vector block j
    // and a last interval in which the trailing group does PV of the last tile.
    // Tile t's K DMA goes out during interval 2t-4 (leading group's matrix
    // block) and is waited for at the end of interval 2t-1. Its raw V DMA goes
    // out during interval 2t-1 (trailing group's matrix block, after the
    // transpose of tile t-1) and is waited for at the end of interval 2t; the
    // trailing group transposes it into V^T of tile t in interval 2t+1. (Tile
    // 0: K and V from the prologue, V^T in interval 1; raw V of tile 1 goes
    // out in interval 1.) K is first read in interval 2t, V^T in interval
    // 2t+2. The K DMA of tile t overwrites only the K half of a stage, whose
    // last reader (trailing scores of tile t-3) finished in interval 2t-5; the
    // V^T half was last read by P.V of tile t-3 in interval 2t-3; raw buffer
    // t % 2 last held tile t-2, transposed in interval 2t-3.
    // A wave's visible tiles are a prefix of the tile range, so a matrix block
    // runs whenever its PV tile is visible; scores it computes for a tile the
    // wave cannot see (or past the last tile) are dropped. Each group runs its
    // own copy of the schedule with the same barrier sequence.
    block_sync();
    if (grp != 0) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // own Q and Q-rope landed
        read_q();
    }

    // one tile's two intervals; r0 = ring stage of tile j (a runtime value, so
    // that each group's loop holds one copy of its matrix and vector blocks)
    // paged, trailing group: cache row of the tile whose raw V goes out next,
    // read from the LDS table in the vector interval before, like the leading
    // group's rows, so that the read's latency stays off the matrix block
    int trail_row_v = 0;
    TileLoad trail_tv{};  // trailing group: raw V load of the next tile, prepared in the vector interval before
    auto tile_pair = [&](int j, int r0, auto LEAD) __attribute__((always_inline)) {
        constexpr bool lead = decltype(LEAD)::value;
        const int rprev = r0 == 0 ? STAGES - 1 : r0 - 1, rnext = r0 == STAGES - 1 ? 0 : r0 + 1;
        block_sync();
        // interval 2j + 1
        int row_k = 0;  // paged: cache row of the tile whose K goes out next interval
        TileLoad tk{};  // leading group: that K load, prepared here, off the matrix block
        if (lead) {
            // paged: the table read goes out first and is taken after the
            // softmax, so its latency does not hold the vector block up
            const int row_k_ld = cache_row_ld(j + 3);
            // a leading wave past its last visible tile still runs its matrix
            // blocks (they carry the group's loads), with P = 0
            if (wave_active(j)) {
                valu_block(j);
            } else {
#pragma unroll
                for (int st4 = 0; st4 < 4; ++st4) pb[st4] = vec8{};
            }
            if (PAGED) row_k = __builtin_amdgcn_readfirstlane(row_k_ld);
            tk = prep_tile(j + 3, row_k);
            // K of tile j+1 and everything before it landed; K of tile j+2 may
            // still fly
            __builtin_amdgcn_s_waitcnt(0x0F70 | K_LOADS);
        } else {
            // the trailing group writes V^T of tile j (its raw V landed at the
            // end of interval 2j) and sends out raw V of tile j+1, with its
            // matrix block or alone
            unsigned char *vr = smem + VRAW_OFFSET + (j & 1) * V_BYTES;
            const TileLoad tv = trail_tv;
            if (wave_active(j - 1))
                mfma_block(soff(rprev), soff(r0), yes, yes, iss_v, yes, tv, none, vr, soff(r0));
            else
                transpose_v(vr, soff(r0), tv);
        }
        block_sync();
        // interval 2j + 2: the leading group sends out K of tile j+3 during its
        // matrix block
        if (lead) {
            mfma_block(soff(r0), soff(rnext), yes, yes, iss_k, no, none, tk, nullptr, 0);
        } else {
            const int row_v_ld = cache_row_ld(j + 2);
            if (wave_active(j)) valu_block(j);
            if (PAGED) trail_row_v = __builtin_amdgcn_readfirstlane(row_v_ld);
            trail_tv = prep_tile(j + 2, trail_row_v);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // raw V of tile j+1 landed
        }
    };
    if (grp == 0) {
        // interval 0: scores of tile 0, and the K of tiles 1 and 2 goes out;
        // tile 0's raw V (issued before them) has landed at its end
        {
            const TileLoad t1 = prep_tile(1, cache_row(1)), t2 = prep_tile(2, cache_row(2));
            if (wave_active(0)) {
                mfma_block(0, 0, no, yes, iss_k2, no, t1, t2, nullptr, 0);
            } else {
#pragma unroll
                for (int i = 0; i < K_LOADS; ++i) issue_k(t1, i);
#pragma unroll
                for (int i = 0; i < K_LOADS; ++i) issue_k(t2, i);
            }
            __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * K_LOADS));
        }
        int r = 0;
#pragma clang loop unroll(disable)
        for (int j = 0; j < n_kt; ++j) {
            tile_pair(j, r, yes);
            r = r == STAGES - 1 ? 0 : r + 1;
        }
        block_sync();
    } else if (n_kt > 0) {
        // tile 0 peeled: in its first interval the leading group scores tile 0
        // and the trailing group takes its Q into registers
        block_sync();
        // (and V^T of tile 0, whose raw V the barrier before the schedule
        // published; raw V of tile 1 goes out)
        {
            const TileLoad tv = prep_tile(1, cache_row(1));
            if (wave_active(0))
                mfma_block(0, 0, no, yes, iss_v, yes, tv, none, smem + VRAW_OFFSET, 0);
            else
                transpose_v(smem + VRAW_OFFSET, 0, tv);
        }
        block_sync();
        trail_row_v = cache_row(2);
        trail_tv = prep_tile(2, trail_row_v);
        if (wave_active(0)) valu_block(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // raw V of tile 1 landed
        int r = 1;
#pragma clang loop unroll(disable)
        for (int j = 1; j < n_kt; ++j) {
            tile_pair(j, r, no);
            r = r == STAGES - 1 ? 0 : r + 1;
        }
        block_sync();
        if (wave_active(n_kt - 1)) {
            const uint32_t sl = soff((n_kt - 1) % STAGES);
            mfma_block(sl, sl, yes, no, iss_none, no, none, none, nullptr, 0);
        }
    } else {
        block_sync();
    }

    // ---- epilogue: combine the two lanes' row sums, normalise, round, store.
    // The rows leave through LDS so that each store instruction writes whole
    // 256-byte head slices of 4 rows: straight from the accumulators every
    // instruction would write 16 bytes into each of 32 rows, and such
    // partial-line writes cost far more than their bytes. Each wave stages its
    // 32 rows (half a V tile of bytes) where no other wave reads or writes any
    // more, so no barrier is needed and the leading group stores while the
    // trailing group still runs its last P.V: a leading wave in the raw V
    // buffers (the last raw V DMA landed and the last transpose ran before the
    // barrier that ended the loop), a trailing wave in the V^T half of ring
    // stage n_kt % 3 or (n_kt + 1) % 3 (the last P.V reads stage
    // (n_kt - 1) % 3; K DMA writes only K halves). The wave's own DMA must have
    // landed before its LDS is released.
    const float l_tot = sum_with_partner(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if (task.part >= 0) {
        // The task holds part of the item's keys: its rows over those keys in
        // fp32, and their log-sum-exp (the running max is in natural-log
        // units and the row sum is taken relative to it), for the merge. Both
        // lanes of a row hold 4 consecutive values of each 8-value group.
        const int64_t prow = ((int64_t)task.part * 8 + slot) * 32 + r32;
        float *po = p.part_o + prow * DN;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 v = {o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
                                  o[db][4 * i + 3] * inv};
                *reinterpret_cast<float4 *>(po + db * 32 + i * 8 + g * 4) = v;
            }
        if (g == 0) p.part_lse[prow] = l_tot > 0.f ? m_run + logf(l_tot) : -INFINITY;
        return;
    }
    {
        const int w4 = wave & 3;
        unsigned char *stg =
            smem + (grp == 0 ? VRAW_OFFSET + w4 * (V_BYTES / 2)
                             : ((n_kt + (w4 >> 1)) % STAGES) * STAGE_BYTES + KN_BYTES + KR_BYTES +
                                   (w4 & 1) * (V_BYTES / 2));
        // staging row r32 (DN * 2 bytes), 16-byte chunk c (8 values of d) at
        // c ^ row_swizzle(r32)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                typename T::vec4 v4;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) v4[jj] = static_cast<typename T::scalar>(o[db][4 * i + jj] * inv);
                *reinterpret_cast<typename T::vec4 *>(stg + r32 * KN_ROW +
                                                      (((4 * db + i) ^ row_swizzle<DN>(r32)) << 4) + g * 8) = v4;
            }
        const int rows = max(0, min(32, q_left - lrow0));
        const int64_t tok = (int64_t)task.q_tok0 + lrow0;
        const i32x4 ro = make_rsrc(static_cast<unsigned char *>(p.out) + (tok * H + h) * (DN * 2),
                                   (uint32_t)rows * H * DN * 2);
        constexpr int CPR = DN / 8;      // 16-byte chunks of a row
        constexpr int RPI = 64 / CPR;    // rows one instruction stores
        const int ch = lane % CPR;
#pragma unroll
        for (int k = 0; k < 32 / RPI; ++k) {
            const int r = RPI * k + lane / CPR;  // row of the wave
            const i32x4 v = *reinterpret_cast<const i32x4 *>(stg + r * KN_ROW + ((ch ^ row_swizzle<DN>(r)) << 4));
            mla_raw_buffer_store_b128(v, ro, (uint32_t)r * H * DN * 2 + ch * 16, 0, CPOL_NT);
        }
    }
}

// ---- merge of split tasks: attenOut row = sum_i w_i O_i / sum_i w_i with
// w_i = exp(lse_i - max_j lse_j), over the partial results O_i (each
// normalised over its own keys) of one row; a row no part sees gives 0. The
// sum is taken in one pass, rescaled whenever a larger lse arrives, so that
// the loads of several parts can be in flight together. A workgroup takes
// 256 / (DN / 4) rows of one wave slot of one merge record, DN / 4 lanes per
// row, 4 values per lane.
template <int DN>
struct MergeShape {
    static constexpr int LPR = DN / 4;          // lanes per row
    static constexpr int RPB = 256 / LPR;       // rows per workgroup
    static constexpr int BPS = 32 / RPB;        // workgroups per wave slot
};

template <typename T, int DN>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void mla_merge_kernel(const MergeParams p) {
    typedef MergeShape<DN> S;
    const MergeRec m = p.merges[blockIdx.x / (8 * S::BPS)];
    const int sub = blockIdx.x % (8 * S::BPS);
    const int slot = sub / S::BPS;
    const int ps = p.pack_shift;
    const int h = m.head + (slot & ((1 << ps) - 1));
    const int lrow0 = (slot >> ps) * 32;
    const int r = (sub % S::BPS) * S::RPB + (int)threadIdx.x / S::LPR;  // row of the wave slot
    if (r >= m.q_left - lrow0) return;
    const int c = threadIdx.x % S::LPR;
    const int64_t row0 = ((int64_t)m.part0 * 8 + slot) * 32 + r;  // partial row of part 0
    constexpr int64_t PSTRIDE = 8 * 32;                          // rows between consecutive parts
    float mx = -INFINITY, wsum = 0.f;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    auto add = [&](float li, float4 v) {
        if (li > mx) {
            const float sc = expf(mx - li);  // 0 while mx is -inf
            wsum *= sc;
#pragma unroll
            for (int k = 0; k < 4; ++k) a[k] *= sc;
            mx = li;
        }
        if (li > -INFINITY) {
            const float w = expf(li - mx);
            wsum += w;
            a[0] += w * v.x;
            a[1] += w * v.y;
            a[2] += w * v.z;
            a[3] += w * v.w;
        }
    };
    int i = 0;
    for (; i + 4 <= m.n_parts; i += 4) {
        float li[4];
        float4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t pr = row0 + (int64_t)(i + k) * PSTRIDE;
            li[k] = p.part_lse[pr];
            v[k] = *reinterpret_cast<const float4 *>(p.part_o + pr * DN + 4 * c);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) add(li[k], v[k]);
    }
    for (; i < m.n_parts; ++i) {
        const int64_t pr = row0 + (int64_t)i * PSTRIDE;
        add(p.part_lse[pr], *reinterpret_cast<const float4 *>(p.part_o + pr * DN + 4 * c));
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    typename T::vec4 o4;
#pragma unroll
    for (int k = 0; k < 4; ++k) o4[k] = static_cast<typename T::scalar>(a[k] * inv);
    const int64_t tok = (int64_t)m.q_tok0 + lrow0 + r;
    *reinterpret_cast<typename T::vec4 *>(static_cast<unsigned char *>(p.out) +
                                          ((tok * p.heads + h) * DN + 4 * c) * 2) = o4;
}

// ---- MASK_FREE tile classes: thread (row, block) looks at the 64 entries
// of its row block (128 bytes) and writes MASK_CLS_ZERO if all are +-0,
// MASK_CLS_DEAD if all are -inf, else MASK_CLS_MIXED.
__global__ __launch_bounds__(256) void mask_classify_kernel(const unsigned short *mask, int is_bf16, uint8_t *cls) {
    const int q = blockIdx.x * 256 + threadIdx.x;  // row * 8 + block
    if (q >= MASK_TILE * (MASK_TILE / BN)) return;
    const unsigned short ninf = is_bf16 ? 0xff80u : 0xfc00u;
    const uint4 *src = reinterpret_cast<const uint4 *>(mask + (size_t)(q >> 3) * MASK_TILE + (q & 7) * BN);
    bool zero = true, dead = true;
#pragma unroll
    for (int i = 0; i < BN / 8; ++i) {
        const uint4 v = src[i];
        const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const unsigned short lo = (unsigned short)(w[j] & 0xffffu), hi = (unsigned short)(w[j] >> 16);
            zero = zero && (lo & 0x7fffu) == 0 && (hi & 0x7fffu) == 0;
            dead = dead && lo == ninf && hi == ninf;
        }
    }
    cls[q] = zero ? MASK_CLS_ZERO : (dead ? MASK_CLS_DEAD : MASK_CLS_MIXED);
}

}  // namespace

hipError_t launch_mask_classify(const void *mask, int mask_is_bf16, uint8_t *cls, hipStream_t stream) {
    hipLaunchKernelGGL(mask_classify_kernel, dim3(MASK_TILE * (MASK_TILE / BN) / 256), dim3(256), 0, stream,
                       static_cast<const unsigned short *>(mask), mask_is_bf16, cls);
    return hipGetLastError();
}

hipError_t launch_mla_merge(const MergeParams &p, int dtype, hipStream_t stream) {
    if (p.n_merges <= 0) return hipSuccess;
    const unsigned per_rec = 8u * (p.head_dim == 64 ? MergeShape<64>::BPS : MergeShape<128>::BPS);
    dim3 grid((unsigned)p.n_merges * per_rec), block(256);
    if (p.head_dim == 64) {
        if (dtype == 2) hipLaunchKernelGGL((mla_merge_kernel<Bf16, 64>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((mla_merge_kernel<Fp16, 64>), grid, block, 0, stream, p);
    } else {
        if (dtype == 2) hipLaunchKernelGGL((mla_merge_kernel<Bf16, 128>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((mla_merge_kernel<Fp16, 128>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_mla_fwd(const FwdParams &p, int dtype, bool paged, hipStream_t stream) {
    if (p.n_tasks <= 0) return hipSuccess;
    dim3 grid((unsigned)p.n_tasks);
    dim3 block(FWD_THREADS);
    const bool mf = p.mask_type == MASK_FREE;
#define MLA_LAUNCH(TT, PG, D, M) hipLaunchKernelGGL((mla_fwd_kernel<TT, PG, D, M>), grid, block, 0, stream, p)
#define MLA_LAUNCH_MF(TT, PG, D) \
    do {                         \
        if (mf)                  \
            MLA_LAUNCH(TT, PG, D, true); \
        else                     \
            MLA_LAUNCH(TT, PG, D, false); \
    } while (0)
#define MLA_LAUNCH_PAGED(TT, D) \
    do {                        \
        if (paged)              \
            MLA_LAUNCH_MF(TT, true, D); \
        else                    \
            MLA_LAUNCH_MF(TT, false, D); \
    } while (0)
    if (p.head_dim == 64) {
        if (dtype == 2) MLA_LAUNCH_PAGED(Bf16, 64);
        else MLA_LAUNCH_PAGED(Fp16, 64);
    } else {
        if (dtype == 2) MLA_LAUNCH_PAGED(Bf16, 128);
        else MLA_LAUNCH_PAGED(Fp16, 128);
    }
#undef MLA_LAUNCH_PAGED
#undef MLA_LAUNCH_MF
#undef MLA_LAUNCH
    return hipGetLastError();
}

}  // namespace mla
