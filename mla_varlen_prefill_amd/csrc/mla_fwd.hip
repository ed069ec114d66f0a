// MLA varlen prefill attention for gfx950 (MI355X).
//
// Computes, for each sequence of a packed variable-length batch and each
// query head (Ascend Transformer Boost "MLA Prefill" page, Members table rows
// Q, QRope, K, kRope, V, qkScale, Mask, maskType):
//     S = qkScale * (Q . K^T + QRope . KRope^T) + mask,   O = softmax_rows(S) . V
//
// One workgroup = 8 waves = FWD_BM = 256 query rows of one (sequence, head).
//
//  * Each wave owns 32 query rows. Their Q | QRope (32 x 192) stay in VGPRs as
//    the B operand of v_mfma_f32_32x32x16 (12 k-steps of 16: 8 nope, 4 rope).
//  * Keys are walked in tiles of FWD_BN = 64. K-nope (64 x 128), K-rope
//    (64 x 64) and V (64 x 128) of a tile are copied HBM -> LDS by the
//    buffer-load-to-LDS DMA path (no VGPR staging), into a 3-stage ring.
//    Key rows past the sequence end fall outside the buffer range and
//    arrive as zeros.
//  * LDS rows are XOR-swizzled in 16-byte chunks so that both the 16-byte
//    reads of K (one key row per lane) and the transposing 8-byte reads of V
//    are free of bank conflicts without padding.
//  * Scores are computed transposed, S^T = K . Q^T: the accumulator holds one
//    query row per lane (lanes l and l + 32 share it), so row max / row sum
//    take one cross-lane swap, and the probabilities already sit in the
//    B-operand layout of O^T = V^T . P^T. V^T operands come straight from the
//    row-major V tile through ds_read_b64_tr_b16.
//  * Ping-pong schedule. The waves form two groups, one wave of each per
//    SIMD. Workgroup barriers cut time into intervals; in every interval one
//    group runs a matrix block (O += P_j V_j, then S_{j+1} = K_{j+1} Q^T: 40
//    MFMAs fed from LDS two operands ahead) while the other runs a vector
//    block (mask, row max, online-softmax update and probabilities of one
//    tile), and the roles swap at each barrier. The matrix core of each SIMD
//    is thus fed by one wave while the other wave's softmax runs on the VALU.
//  * Online softmax in fp32 with exp2 (log2(e) folded into the scale). The
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
constexpr int DN = HEAD_DIM;
constexpr int DR = ROPE_DIM;
constexpr int STAGES = 3;
#ifndef MLA_PREFETCH
#define MLA_PREFETCH 2
#endif
constexpr int PREFETCH = MLA_PREFETCH;  // LDS operands in flight ahead of the MFMA using them
constexpr int KN_BYTES = BN * DN * 2;  // 16 KB
constexpr int KR_BYTES = BN * DR * 2;  // 8 KB
constexpr int V_BYTES = BN * DN * 2;   // 16 KB
constexpr int STAGE_BYTES = KN_BYTES + KR_BYTES + V_BYTES;
constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units
constexpr float LOG2E = 1.4426950408889634f;

constexpr int MASK_UNDEFINED = 0;
constexpr int MASK_FREE = 3;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned int *lds_u32_ptr;

// Buffer load with the LDS-DMA bit: lane l's `size` bytes land at lds + l*size.
extern "C" __device__ void mla_raw_buffer_load_lds(i32x4 rsrc, lds_u32_ptr lds, int size, int voffset,
                                                   int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");
extern "C" __device__ i32x4 mla_raw_buffer_load_b128(i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
extern "C" __device__ void mla_raw_buffer_store_b64(i16x4 data, i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.store.v4i16");

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
    // acc + x[0] + x[1], products and sum in fp32
    static __device__ __forceinline__ float dot2_ones(pair x, float acc) {
        const pair one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
        return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
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
    static __device__ __forceinline__ float dot2_ones(pair x, float acc) {
        const pair one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
        return __builtin_amdgcn_fdot2(x, one, acc, false);
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

__device__ __forceinline__ i16x4 lds_read_tr16(const unsigned char *p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

template <typename T>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void mla_fwd_kernel(const FwdParams p) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGES * STAGE_BYTES];
    typedef typename T::vec8 vec8;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int grp = wave >> 2;  // 0: leading group, 1: trailing group (one interval behind)
    const int g = lane >> 5;    // which 8 of each 16 k-slots this lane carries
    const int r32 = lane & 31;  // query row within the wave

    // The host's task list says which work item and head this workgroup runs
    // (launch order and XCD placement are chosen there); padding tasks exit.
    const Task task = p.tasks[blockIdx.x];
    if (task.item < 0) return;
    const int h = task.head;
    const WorkItem item = p.items[task.item];
    const SeqRec seq = p.seqs[item.b];
    const int hk = h / p.group;
    const int H = p.heads, HKV = p.kv_heads;
    const int q_len = seq.q_len;
    const int kv_len = seq.kv_len;
    const int n_kt = item.kv_tiles;
    const int mask_type = p.mask_type;
    const bool causal_like = mask_type != MASK_UNDEFINED && mask_type != MASK_FREE;

    // The two waves sharing a SIMD (w, w + 4) take adjacent 32-row blocks, so
    // both groups see the same share of diagonal tiles.
    const int row0 = item.q_row0 + (wave & 3) * 64 + grp * 32;  // first query row of this wave
    const int qi = row0 + r32;                                  // this lane's query row
    const int pos = kv_len - q_len + qi;                        // its key position
    const int wpos0 = kv_len - q_len + row0;                    // key positions of the wave's rows
    const int wpos1 = wpos0 + 31;

    // ---- Q^T operand (B of S^T = K . Q^T): lane holds row r32, k-slots g*8..g*8+7.
    // Rows past the sequence end read as zeros.
    vec8 qreg[12];
    {
        const int rows = max(0, min(32, q_len - row0));
        const int64_t tok = (int64_t)seq.q_off + row0;
        const i32x4 rq = make_rsrc(static_cast<const unsigned char *>(p.q) + (tok * H + h) * (DN * 2),
                                   (uint32_t)rows * H * DN * 2);
        const i32x4 rqr = make_rsrc(static_cast<const unsigned char *>(p.q_rope) + (tok * H + h) * (DR * 2),
                                    (uint32_t)rows * H * DR * 2);
        const uint32_t qo = (uint32_t)r32 * H * DN * 2 + g * 16;
        const uint32_t qro = (uint32_t)r32 * H * DR * 2 + g * 16;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qreg[ks] = __builtin_bit_cast(vec8, mla_raw_buffer_load_b128(rq, qo + ks * 32, 0, 0));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qreg[8 + ks] = __builtin_bit_cast(vec8, mla_raw_buffer_load_b128(rqr, qro + ks * 32, 0, 0));
    }

    // ---- K / V tile streaming (LDS-DMA). Tile kt -> ring stage kt % 3.
    const unsigned char *kbase = static_cast<const unsigned char *>(p.k);
    const unsigned char *krbase = static_cast<const unsigned char *>(p.k_rope);
    const unsigned char *vbase = static_cast<const unsigned char *>(p.v);
    const uint32_t kn_row = (uint32_t)HKV * DN * 2;  // bytes between consecutive keys
    const uint32_t kr_row = (uint32_t)HKV * DR * 2;
    // per-thread source offsets (fixed across tiles): LDS slot -> (key, swizzled chunk)
    uint32_t off_kn[2], off_v[2], off_kr;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int slot = tid + NT * u;
        const int key = slot >> 4;
        off_kn[u] = key * kn_row + (((slot & 15) ^ (key & 15)) << 4);
        off_v[u] = key * kn_row + (((slot & 15) ^ ((key & 3) << 2)) << 4);
    }
    {
        const int key = tid >> 3;
        off_kr = key * kr_row + (((tid & 7) ^ ((key >> 1) & 7)) << 4);
    }
    auto issue_tile = [&](int kt) __attribute__((always_inline)) {
        unsigned char *st = smem + (kt % STAGES) * STAGE_BYTES;
        const int64_t rowi = ((int64_t)seq.kv_off + (int64_t)kt * BN) * HKV + hk;  // first key row, this head
        const uint32_t nvalid = (uint32_t)min(kv_len - kt * BN, BN);
        const i32x4 rk = make_rsrc(kbase + rowi * (DN * 2), nvalid * kn_row);
        const i32x4 rr = make_rsrc(krbase + rowi * (DR * 2), nvalid * kr_row);
        const i32x4 rv = make_rsrc(vbase + rowi * (DN * 2), nvalid * kn_row);
        const int wofs = wave * 64 * 16;
#pragma unroll
        for (int u = 0; u < 2; ++u)
            mla_raw_buffer_load_lds(rk, (lds_u32_ptr)(st + u * NT * 16 + wofs), 16, off_kn[u], 0, 0, 0);
        mla_raw_buffer_load_lds(rr, (lds_u32_ptr)(st + KN_BYTES + wofs), 16, off_kr, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 2; ++u)
            mla_raw_buffer_load_lds(rv, (lds_u32_ptr)(st + KN_BYTES + KR_BYTES + u * NT * 16 + wofs), 16,
                                    off_v[u], 0, 0, 0);
    };
    constexpr int LOADS_PER_TILE = 5;  // DMA instructions per thread and tile

    if (n_kt > 0) issue_tile(0);
    if (n_kt > 1) issue_tile(1);

    // A negative scale is folded into Q so the row max can be taken on raw scores.
    const float c = fabsf(p.scale_log2);
    if (p.scale_log2 < 0.f) {
#pragma unroll
        for (int ks = 0; ks < 12; ++ks) {
            i32x4 w = __builtin_bit_cast(i32x4, qreg[ks]);
            w ^= (int)0x80008000;
            qreg[ks] = __builtin_bit_cast(vec8, w);
        }
    }

    // ---- per-wave tile visibility
    // can any of the wave's rows see any key of tile kt?
    auto wave_active = [&](int kt) __attribute__((always_inline)) -> bool {
        if (kt < 0 || kt >= n_kt) return false;
        const int key0 = kt * BN;
        if (causal_like) return key0 <= wpos1;
        if (mask_type == MASK_FREE) return wpos1 >= 0 && (key0 >> 9) <= (wpos1 >> 9);
        return true;
    };
    // does every row of the wave see every key of it (no per-element mask)?
    auto wave_full = [&](int kt) __attribute__((always_inline)) -> bool {
        const int key0 = kt * BN;
        bool full = key0 + BN <= kv_len;
        if (causal_like) full = full && key0 + BN - 1 <= wpos0;
        else if (mask_type == MASK_FREE) full = full && wpos0 >= 0 && ((key0 + BN - 1) >> 9) < (wpos0 >> 9);
        return full;
    };

    // ---- per-lane LDS read offsets: every operand read is one of these lane
    // offsets plus a compile-time immediate (ring stage, key block, step).
    // K (A operand of S^T): lane reads key kb*32 + r32, 16-byte chunk 2*ks + g.
    // With the chunk swizzles c ^ (key & 15) (nope) and c ^ ((key >> 1) & 7)
    // (rope) and key & 31 == r32, the lane offset depends on ks but not kb.
    uint32_t k_off[12];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) k_off[ks] = r32 * 256 + (((2 * ks + g) ^ (r32 & 15)) << 4);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) k_off[8 + ks] = KN_BYTES + r32 * 128 + (((2 * ks + g) ^ ((r32 >> 1) & 7)) << 4);
    // V^T (A operand of O^T, transposing read): within a 16-lane group, lane sl
    // points at 4 consecutive columns of key 4*(group/2) + sl/4; the chunk
    // swizzle c ^ ((key & 3) << 2) then depends on the column block db only.
    uint32_t v_off[4];
    {
        const int lg = lane >> 4, sl = lane & 15;
        const int vk = 4 * (lg >> 1) + (sl >> 2);
        const int vcl = 2 * (lg & 1) + ((sl & 3) >> 1);
#pragma unroll
        for (int db = 0; db < 4; ++db)
            v_off[db] = KN_BYTES + KR_BYTES + vk * 256 + (((db * 4 + vcl) ^ ((vk & 3) << 2)) << 4) + (sl & 1) * 8;
    }
    // operand n of a matrix block: n < 16 -> V^T of (16-key step n/4, column block
    // n%4) from stage sv; n >= 16 -> K of (k-step (n-16)/2, key block (n-16)%2) from sk
    auto load_operand = [&](const unsigned char *sv, const unsigned char *sk, int n) __attribute__((always_inline))
        -> vec8 {
        if (n < 16) {
            const int st4 = n >> 2, db = n & 3;
            const i16x4 lo = lds_read_tr16(sv + v_off[db] + st4 * 16 * 256);
            const i16x4 hi = lds_read_tr16(sv + v_off[db] + st4 * 16 * 256 + 8 * 256);
            const i16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(vec8, a);
        }
        const int ks = (n - 16) >> 1, kb = (n - 16) & 1;
        const int row_step = ks < 8 ? 256 : 128;
        const uint4 u = *reinterpret_cast<const uint4 *>(sk + k_off[ks] + kb * 32 * row_step);
        return __builtin_bit_cast(vec8, u);
    };

    // ---- softmax state
    float m_run = -INFINITY;  // running row max of raw scores (same in both lanes of a row)
    float l_run = 0.f;        // this lane's share of the running row sum
    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
    f32x16 s[2];  // scores of one tile; element e of block kb is key kb*32 + 8*(e/4) + 4*g + e%4
    vec8 pb[4];   // P^T operands of the four 16-key steps

    // ---- matrix block: O += P . V (tile in stage sv) then S = K . Q^T (tile in
    // stage sk); either half may be switched off. Operands are read two ahead.
    auto mfma_block = [&](const unsigned char *sv, const unsigned char *sk, auto do_pv, auto do_qk)
        __attribute__((always_inline)) {
        constexpr bool PV = decltype(do_pv)::value, QK = decltype(do_qk)::value;
        constexpr int n0 = PV ? 0 : 16, n1 = QK ? 40 : 16;
        if (QK) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
        }
        vec8 ring[PREFETCH + 1];
#pragma unroll
        for (int d = 0; d < PREFETCH; ++d)
            if (n0 + d < n1) ring[d] = load_operand(sv, sk, n0 + d);
#pragma unroll
        for (int n = n0; n < n1; ++n) {
            if (n + PREFETCH < n1) ring[(n + PREFETCH - n0) % (PREFETCH + 1)] = load_operand(sv, sk, n + PREFETCH);
            __builtin_amdgcn_sched_barrier(0);
            const vec8 a = ring[(n - n0) % (PREFETCH + 1)];
            if (n < 16) {
                o[n & 3] = T::mfma(a, pb[n >> 2], o[n & 3]);
            } else {
                const int ks = (n - 16) >> 1, kb = (n - 16) & 1;
                s[kb] = T::mfma(a, qreg[ks], s[kb]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- vector block for tile kt: mask (if needed), row max, lazy rescale,
    // probabilities -> pb, row sums.
    const float inv_c = 1.f / c;
    auto valu_block = [&](int kt) __attribute__((always_inline)) {
        float mx = -INFINITY;
        if (wave_full(kt)) {
            float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int t = 0; t < 32; ++t) m4[t & 3] = fmaxf(m4[t & 3], s[t >> 4][t & 15]);
            mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        } else {
            const int key0 = kt * BN;
            const unsigned short *mrow = nullptr;
            if (mask_type == MASK_FREE)
                mrow = static_cast<const unsigned short *>(p.mask) + (pos & (MASK_TILE - 1)) * MASK_TILE;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int j = key0 + kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                    float x = s[kb][e];
                    bool vis = j < kv_len;
                    if (causal_like) {
                        vis = vis && j <= pos;
                    } else if (mask_type == MASK_FREE) {
                        vis = vis && pos >= 0 && (j >> 9) <= (pos >> 9);
                        if (vis && (j >> 9) == (pos >> 9)) {
                            // tile entry m is added as m * log2(e) / c, so the
                            // fma with c below turns it into m * log2(e)
                            const unsigned short mbits = mrow[j & (MASK_TILE - 1)];
                            const float mv = p.mask_is_bf16 ? bits_to_float_bf16(mbits) : bits_to_float_f16(mbits);
                            x += mv * LOG2E * inv_c;
                        }
                    }
                    x = vis ? x : -INFINITY;
                    s[kb][e] = x;
                    mx = fmaxf(mx, x);
                }
        }
        mx = max_with_partner(mx);
        // move the running max only if some row of the wave rose past the threshold
        const bool need = (mx - m_run) * c > RESCALE_THRESHOLD;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2((m_run - m_new) * c);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
            m_run = m_new;
        }
        const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
        // probabilities, rounded to the input dtype; the row sum is taken over
        // the rounded values (the ones the PV product uses) with dot2 against
        // (1, 1), in four independent partial sums
        float lsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 32; t += 2) {
            const int kb = t >> 4, e = t & 15;
            const float p0 = fast_exp2(__builtin_fmaf(s[kb][e], c, -mc));
            const float p1 = fast_exp2(__builtin_fmaf(s[kb][e + 1], c, -mc));
            const typename T::pair pr = T::pack(p0, p1);
            lsum[(t >> 1) & 3] = T::dot2_ones(pr, lsum[(t >> 1) & 3]);
            pb[kb * 2 + (e >> 3)][e & 7] = pr[0];
            pb[kb * 2 + (e >> 3)][(e & 7) + 1] = pr[1];
        }
        l_run += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    };

    const std::integral_constant<bool, true> yes{};
    const std::integral_constant<bool, false> no{};
    auto stage_ptr = [&](int r) __attribute__((always_inline)) -> const unsigned char * {
        return smem + r * STAGE_BYTES;
    };
    // ---- schedule. Interval 0: leading group scores tile 0. Then for each tile
    // j two intervals:
    //   2j+1: leading: vector block j        trailing: PV j-1 + scores j
    //   2j+2: leading: PV j + scores j+1     trailing: vector block j
    // and a last interval in which the trailing group does PV of the last tile.
    // Tile t's DMA is issued at the start of interval 2t-2 and waited for
    // before interval 2t, the first that reads it.
    // A wave's visible tiles are a prefix of the tile range, so a matrix block
    // runs whenever its PV tile is visible; scores it computes for a tile the
    // wave cannot see (or past the last tile) are dropped. Each group runs its
    // own copy of the schedule with the same barrier sequence.
    if (n_kt > 1)
        __builtin_amdgcn_s_waitcnt(0x0F70 | LOADS_PER_TILE);  // tile 0 landed, tile 1 may fly
    else
        __builtin_amdgcn_s_waitcnt(0x0F70);
    block_sync();

    // one tile's two intervals; R = ring stage of tile j
    auto tile_pair = [&](int j, auto R, auto LEAD) __attribute__((always_inline)) {
        constexpr int r0 = decltype(R)::value;
        constexpr bool lead = decltype(LEAD)::value;
        constexpr int rprev = (r0 + STAGES - 1) % STAGES, rnext = (r0 + 1) % STAGES;
        block_sync();
        // interval 2j + 1
        if (lead) {
            if (wave_active(j)) valu_block(j);
        } else {
            if (wave_active(j - 1)) mfma_block(stage_ptr(rprev), stage_ptr(r0), yes, yes);
        }
        if (j + 1 < n_kt) __builtin_amdgcn_s_waitcnt(0x0F70);  // own DMA of tile j+1 landed
        block_sync();
        // interval 2j + 2
        if (j + 2 < n_kt) issue_tile(j + 2);
        if (lead) {
            if (wave_active(j)) mfma_block(stage_ptr(r0), stage_ptr(rnext), yes, yes);
        } else {
            if (wave_active(j)) valu_block(j);
        }
    };
    if (grp == 0) {
        if (wave_active(0)) mfma_block(stage_ptr(0), stage_ptr(0), no, yes);
        for (int j = 0; j < n_kt; j += STAGES) {
            tile_pair(j, std::integral_constant<int, 0>{}, yes);
            if (j + 1 < n_kt) tile_pair(j + 1, std::integral_constant<int, 1>{}, yes);
            if (j + 2 < n_kt) tile_pair(j + 2, std::integral_constant<int, 2>{}, yes);
        }
        block_sync();
    } else if (n_kt > 0) {
        // tile 0 peeled: its first interval only scores tile 0
        block_sync();
        if (wave_active(0)) mfma_block(stage_ptr(0), stage_ptr(0), no, yes);
        if (1 < n_kt) __builtin_amdgcn_s_waitcnt(0x0F70);
        block_sync();
        if (2 < n_kt) issue_tile(2);
        if (wave_active(0)) valu_block(0);
        for (int j = 1; j < n_kt; j += STAGES) {
            tile_pair(j, std::integral_constant<int, 1>{}, no);
            if (j + 1 < n_kt) tile_pair(j + 1, std::integral_constant<int, 2>{}, no);
            if (j + 2 < n_kt) tile_pair(j + 2, std::integral_constant<int, 0>{}, no);
        }
        block_sync();
        if (wave_active(n_kt - 1)) {
            const int r = (n_kt - 1) % STAGES;
            if (r == 0) mfma_block(stage_ptr(0), stage_ptr(0), yes, no);
            else if (r == 1) mfma_block(stage_ptr(1), stage_ptr(1), yes, no);
            else mfma_block(stage_ptr(2), stage_ptr(2), yes, no);
        }
    } else {
        block_sync();
    }

    // ---- epilogue: combine the two lanes' row sums, normalise, round, store
    const float l_tot = sum_with_partner(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    {
        const int rows = max(0, min(32, q_len - row0));
        const int64_t tok = (int64_t)seq.q_off + row0;
        const i32x4 ro = make_rsrc(static_cast<unsigned char *>(p.out) + (tok * H + h) * (DN * 2),
                                   (uint32_t)rows * H * DN * 2);
        const uint32_t base = (uint32_t)r32 * H * DN * 2 + g * 8;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                typename T::vec4 v4;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) v4[jj] = static_cast<typename T::scalar>(o[db][4 * i + jj] * inv);
                mla_raw_buffer_store_b64(__builtin_bit_cast(i16x4, v4), ro, base + (db * 32 + 8 * i) * 2, 0, 0);
            }
    }
}

}  // namespace

hipError_t launch_mla_fwd(const FwdParams &p, int dtype, hipStream_t stream) {
    if (p.n_tasks <= 0) return hipSuccess;
    dim3 grid((unsigned)p.n_tasks);
    dim3 block(FWD_THREADS);
    if (dtype == 2)
        hipLaunchKernelGGL(mla_fwd_kernel<Bf16>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(mla_fwd_kernel<Fp16>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
