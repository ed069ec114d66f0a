// MLA prolog, non-quantised, for gfx950 (MI355X).
//
// The "MlaProlog" operator (cann-recipes-infer notes, formula section) turns
// hidden states x [t, h] into the attention inputs:
//     c^Q = RmsNorm(x . wq_a) * gamma_cq                    [t, q_lora_rank]
//     q   = rope(RmsNorm(c^Q . wq_b)), the norm per head     [t, heads, 512]
//     kv  = rope(RmsNorm(x . wkv) * gamma_ckv)               [t, 512]
// where rope rotates adjacent pairs of the last 64 values of each row.
//
// Two kernels:
//  * prolog_gemm_kernel: out = a . w for bf16 a [M, K] and bf16 w [K, N]
//    (row-major, as the page gives the weights), one workgroup per tile of
//    512 output columns x 128 rows, fp32 accumulation on
//    v_mfma_f32_32x32x16_bf16. A 512-column tile is exactly one head of q (or
//    the kv row), so the tile's epilogue can apply the RmsNorm over its
//    columns, gamma and the rope, and store bf16; or it stores fp32.
//  * prolog_rms_rows_kernel: RmsNorm * gamma of the fp32 rows x . wq_a
//    (q_lora_rank = 1024 columns, two tiles of the product), stored as the
//    bf16 c^Q that is both an output and the next product's input.
//
// Tile kernel design:
//  * The product is computed transposed, out^T = w^T . a^T: the MFMA A operand
//    is a 32-column block of w^T, B a 32-row block of a, so each lane of the
//    accumulator holds one output row and 16 of its columns in runs of 4 --
//    the rope's adjacent pairs sit in one lane.
//  * 8 waves = 4 column quarters (128 columns) x 2 row halves (64 rows):
//    4 x 2 accumulator blocks of 32 x 32 per wave.
//  * K is walked in stages of 32 through a 4-stage LDS ring (40 KB a stage),
//    loaded three stages ahead by DMA (buffer loads straight into LDS, no
//    register round trip). The operand needs 8 consecutive k per column,
//    and the weights are k-major in memory, so prolog_pack_kernel first
//    rewrites each weight into blocks of 32 KB -- one per 512-column tile and
//    32-row stage -- that are exactly the stage's LDS image: column n, 16-byte
//    chunk c (k 8c .. 8c + 7) at byte n * 64 + ((c ^ ((n >> 2) & 3)) << 4).
//    Every weight DMA instruction then reads one contiguous kilobyte. The
//    activation stage (128 rows x 64 bytes) is DMA'd from the row-major
//    activations with the same XOR swizzle applied on the global side. Both
//    swizzles make the 16-byte operand reads conflict-free. (Loading the
//    weights k-major through registers, the lanes of one load instruction
//    spread over eight rows, and transposing them with v_perm before an LDS
//    write took 1.53 ms for the 16384-token workload's main product, against
//    1.15-1.29 ms for this path; the whole prolog went from 29% to 34% of the
//    bf16 peak. Counters on this path: matrix cores busy 49% of the cycles
//    at 1.85 GHz; bank conflicts are a quarter of the LDS-active count, the
//    same with the weight rows permuted and with 4-byte DMA (which fills 256
//    contiguous bytes per instruction and ran 6% slower), so they come
//    from neither the operand reads nor the DMA writes.)
//  * Each ring slot is an LDS array of its own, so the compiler can tell a
//    slot being read from the slots the DMA is filling and waits only where
//    the pipeline says so.
//  * Column tiles are spread so that the 32 CUs of an XCD work on the same
//    weight tile at the same time (it stays in that XCD's L2).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernels.h"

namespace mla {
namespace {

constexpr int BN = PROLOG_BN;
constexpr int BM = PROLOG_BM;
constexpr int BK = PROLOG_BK;
constexpr int NT = 512;
constexpr int STAGES = 4;
constexpr int X_BYTES = BM * BK * 2;  // 8 KB of activations
constexpr int W_BYTES = BN * BK * 2;  // 32 KB of transposed weights
constexpr int LDS_BYTES = STAGES * (X_BYTES + W_BYTES);  // 160 KB

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

extern "C" __device__ i32x4 prolog_raw_buffer_load_b128(i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
extern "C" __device__ i16x4 prolog_raw_buffer_load_b64(i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i16");
extern "C" __device__ float prolog_raw_buffer_load_f32(i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.f32");
typedef __attribute__((address_space(3))) unsigned int *lds_u32_ptr;
// Buffer load with the LDS-DMA bit: lane l's `size` bytes land at lds + l*size.
extern "C" __device__ void prolog_raw_buffer_load_lds(i32x4 rsrc, lds_u32_ptr lds, int size, int voffset,
                                                      int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");
extern "C" __device__ void prolog_raw_buffer_store_b128(i32x4 data, i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.store.v4i32");

// Cache policy of the output stores: non-temporal, since no kernel of the
// product reads them back and the weight tiles the XCD's CUs share should stay
// in L2 (16384-token prolog: -2.3%, quantised -3.5%).
constexpr int CPOL_NT = 2;

// Buffer resource over [base, base + bytes): loads past the end return 0,
// stores past the end are dropped. Arguments must be wave-uniform.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
    r[3] = 0x00020000;
    return r;
}

// Barrier without __syncthreads()'s fence (which would make every thread
// wait for its prefetches still in flight); LDS reads and writes of this
// thread have completed (lgkmcnt) before it.
__device__ __forceinline__ void block_sync() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float bf16_bits_to_float(unsigned short b) {
    return __uint_as_float(static_cast<unsigned>(b) << 16);
}

// Packs the weights of one segment tile stage: workgroup (j, kt) reads the KR
// k rows of stage kt (32 bf16 or 64 int8 rows), columns 512 j .. 512 j + 511
// of w (coalesced, into LDS k-major) and writes block j * nk + kt of wp in the
// stage layout the product kernel reads: column n, 16-byte chunk c (the k
// values 8c .. 8c + 7 of the stage in bf16, 16c .. 16c + 15 in int8) at byte
// n * 64 + ((c ^ ((n >> 2) & 3)) << 4).
template <bool I8>
__global__ __launch_bounds__(256) void prolog_pack_kernel(const unsigned char *w, int64_t ldw, int32_t nk,
                                                          unsigned char *wp) {
    constexpr int ESZ = I8 ? 1 : 2;         // bytes per element
    constexpr int KR = 64 / ESZ;            // k rows per stage
    constexpr int ROW = BN * ESZ + 16;      // LDS bytes per k row (padded)
    constexpr int CPR = BN * ESZ / 16;      // 16-byte chunks per k row
    __shared__ __attribute__((aligned(16))) unsigned char t[KR * ROW];
    const int tid = threadIdx.x;
    const int j = blockIdx.x / nk, kt = blockIdx.x % nk;
    const unsigned char *src = w + ((int64_t)kt * KR * ldw + (int64_t)j * BN) * ESZ;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int q = tid + 256 * u, row = q / CPR, ch = q % CPR;
        *reinterpret_cast<uint4 *>(t + row * ROW + ch * 16) =
            *reinterpret_cast<const uint4 *>(src + (int64_t)row * ldw * ESZ + ch * 16);
    }
    __syncthreads();
    unsigned char *dst = wp + ((int64_t)j * nk + kt) * PROLOG_PACK_BLOCK;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int s16 = tid + 256 * u;  // 16-byte slot of the block: column n, physical chunk pc
        const int n = s16 >> 2, pc = s16 & 3, c = pc ^ ((n >> 2) & 3);
        uint4 o;
        if (I8) {
            unsigned b[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) b[i] = t[(16 * c + i) * ROW + n];
            o.x = b[0] | b[1] << 8 | b[2] << 16 | b[3] << 24;
            o.y = b[4] | b[5] << 8 | b[6] << 16 | b[7] << 24;
            o.z = b[8] | b[9] << 8 | b[10] << 16 | b[11] << 24;
            o.w = b[12] | b[13] << 8 | b[14] << 16 | b[15] << 24;
        } else {
            unsigned short v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = *reinterpret_cast<const unsigned short *>(t + (8 * c + i) * ROW + n * 2);
            o.x = v[0] | (unsigned)v[1] << 16;
            o.y = v[2] | (unsigned)v[3] << 16;
            o.z = v[4] | (unsigned)v[5] << 16;
            o.w = v[6] | (unsigned)v[7] << 16;
        }
        *reinterpret_cast<uint4 *>(dst + s16 * 16) = o;
    }
}

// I8: int8 operands, v_mfma_i32_32x32x32_i8, a stage of 64 k (the same 64
// bytes per row as a bf16 stage of 32 k, so the ring, the DMA and the operand
// reads are the same); the epilogue scales the int32 products to fp32 first.
template <bool I8>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void prolog_gemm_kernel(const PrologGemmParams p) {
    constexpr int ESZ = I8 ? 1 : 2;  // bytes per element
    // one array per ring slot (see the design notes above)
    __shared__ __attribute__((aligned(1024))) unsigned char xs0[X_BYTES], xs1[X_BYTES], xs2[X_BYTES], xs3[X_BYTES];
    __shared__ __attribute__((aligned(1024))) unsigned char ws0[W_BYTES], ws1[W_BYTES], ws2[W_BYTES], ws3[W_BYTES];
    auto WS = [&](int i) __attribute__((always_inline)) -> unsigned char * {
        return i == 0 ? ws0 : i == 1 ? ws1 : i == 2 ? ws2 : ws3;
    };
    auto XS = [&](int i) __attribute__((always_inline)) -> unsigned char * {
        return i == 0 ? xs0 : i == 1 ? xs1 : i == 2 ? xs2 : xs3;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 3;   // column quarter: columns 128 wn .. + 127 of the tile
    const int wt = wave >> 2;  // row half: rows 64 wt .. + 63
    const int g = lane >> 5;
    const int r32 = lane & 31;

    // ---- which tile. When the column tiles split evenly over the 8 XCDs,
    // XCD x takes column tiles x, x + 8, ... one after another, all row
    // tiles of each: its CUs then share one weight tile in L2. A second
    // segment with an operand of its own (a1) goes first, tile by tile: its
    // workgroups are the launch's longest, and a multiple of 8 of them keeps
    // the first segment's blocks on the same XCDs.
    const bool lead = !I8 && p.a1 != nullptr;
    const int n_tiles = lead ? p.seg[0].n_tiles : p.seg[0].n_tiles + p.seg[1].n_tiles;
    const int m_tiles = (p.m + BM - 1) / BM;
    const int lead_blocks = lead ? p.seg[1].n_tiles * m_tiles : 0;
    // split over K: the k_splits workgroups of a tile are consecutive
    const bool split_k = !I8 && p.k_splits > 1;
    const int n_splits = split_k ? p.k_splits : 1;
    const int split = (int)blockIdx.x % n_splits;
    int blk = (int)blockIdx.x / n_splits;
    int tn, tm;
    if (blk < lead_blocks) {
        tn = p.seg[0].n_tiles + blk / m_tiles;
        tm = blk % m_tiles;
    } else if ((blk -= lead_blocks, n_tiles % 8 == 0)) {
        const int s = blk >> 3;
        tn = (blk & 7) + 8 * (s / m_tiles);
        tm = s % m_tiles;
    } else {
        tn = blk % n_tiles;
        tm = blk / n_tiles;
    }
    const bool second = tn >= p.seg[0].n_tiles;
    const bool own_a = lead && second;
    const void *a_ptr = own_a ? p.a1 : p.a;
    const int64_t lda = own_a ? p.lda1 : p.lda;
    const int32_t k_len = own_a ? p.k1 : p.k;
    const int tj = second ? tn - p.seg[0].n_tiles : tn;
    const unsigned char *wpk = static_cast<const unsigned char *>(second ? p.seg[1].wp : p.seg[0].wp);
    const int epilogue = second ? p.seg[1].epilogue : p.seg[0].epilogue;
    void *out_base = second ? p.seg[1].out : p.seg[0].out;
    const int64_t ld_out = second ? p.seg[1].ld_out : p.seg[0].ld_out;
    const unsigned char *gamma = static_cast<const unsigned char *>(second ? p.seg[1].gamma : p.seg[0].gamma);
    const int m0 = tm * BM;
    const int rows = min(BM, p.m - m0);
    const int nk_all = k_len * ESZ / (BK * 2);  // 64-byte stages
    const int nk = nk_all / n_splits;         // this workgroup's stages: [kbase, kbase + nk)
    const int kbase = split * nk;
    // int8: the dequantisation scales go out now and are used by the
    // epilogue -- thread tid takes the scale of the tile's column tid, a lane
    // those of its two output rows (rows past the end read 0)
    float cs_pre = 0.f, rs_pre[2] = {0.f, 0.f};
    if constexpr (I8) {
        cs_pre = p.col_scale[(int64_t)tj * BN + tid];
        const i32x4 rsr = make_rsrc(p.row_scale + m0, (uint32_t)rows * 4);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
            rs_pre[tb] = prolog_raw_buffer_load_f32(rsr, (uint32_t)(64 * wt + 32 * tb + r32) * 4, 0, 0);
    }

    // ---- activation stage: 128 rows x 64 bytes; LDS slot tid (row tid / 4,
    // physical chunk tid % 4) receives logical chunk (tid % 4) ^ ((row >> 2)
    // & 3). Rows past the end read as zeros.
    const i32x4 ra = make_rsrc(static_cast<const unsigned char *>(a_ptr) + (int64_t)m0 * lda * ESZ + (int64_t)kbase * 64,
                               (uint32_t)rows * (uint32_t)lda * ESZ - (uint32_t)kbase * 64);
    const int xr = tid >> 2;
    const uint32_t xoff = (uint32_t)xr * (uint32_t)lda * ESZ + ((((tid & 3) ^ ((xr >> 2) & 3))) << 4);
    // ---- weight stage: block kt of this tile's packed weights, 2048 16-byte
    // slots; load r of a thread takes slot 512 r + tid. Stages past K read
    // as zeros (a split's activation stages past its end read real values,
    // which meet those zero weights).
    const i32x4 rw = make_rsrc(wpk + ((int64_t)tj * nk_all + kbase) * PROLOG_PACK_BLOCK, (uint32_t)nk * PROLOG_PACK_BLOCK);
    // DMA of stage kt into ring slot kt % STAGES: lane l's 16 bytes land at
    // base + 16 l, so a wave's base is its first slot.
    auto issue = [&](int kt, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            prolog_raw_buffer_load_lds(rw, (lds_u32_ptr)(WS(slot) + (r * 512 + wave * 64) * 16), 16,
                                       (uint32_t)kt * PROLOG_PACK_BLOCK + (uint32_t)(r * 512 + tid) * 16, 0, 0, 0);
        prolog_raw_buffer_load_lds(ra, (lds_u32_ptr)(XS(slot) + wave * 64 * 16), 16, xoff + (uint32_t)kt * BK * 2,
                                   0, 0, 0);
    };

    // ---- operand read offsets (within a stage). Weight column block nb of
    // the wave: column n = 128 wn + 32 nb + r32; k chunk 2 ks + g. Activation
    // row block tb: row 64 wt + 32 tb + r32, chunk 2 ks + g. Both are base ^
    // (ks << 5) plus a multiple of 2 KB.
    const int n_l = 128 * wn + r32;
    const uint32_t wb = (uint32_t)(n_l * 64) | ((uint32_t)(g ^ ((n_l >> 2) & 3)) << 4);
    const int xrow = 64 * wt + r32;
    const uint32_t xb = (uint32_t)(xrow * 64) | ((uint32_t)(g ^ ((xrow >> 2) & 3)) << 4);

    typedef std::conditional_t<I8, i32x16, f32x16> acc_t;
    acc_t acc[4][2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[nb][tb][e] = 0;

    // Operands of one k-step: av = 4 weight column blocks, bv = 2 activation
    // row blocks. Operand o < 4 is av[o], o >= 4 is bv[o - 4]. The products of
    // a k-step run row block first (n -> column block n % 4, row block n / 4),
    // so each operand is done with early and the next k-step's value is read
    // into its registers while the remaining products run: bv[0] after product
    // 3, av[0..2] after products 4..6, av[3] and bv[1] after product 7.
    bf16x8 av[4], bv[2];
    auto read_op = [&](int slot, int ks, int o) __attribute__((always_inline)) {
        if (o < 4)
            av[o] = __builtin_bit_cast(bf16x8,
                                       *reinterpret_cast<const uint4 *>(WS(slot) + ((wb ^ (ks << 5)) + o * 2048)));
        else
            bv[o - 4] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4 *>(XS(slot) + ((xb ^ (ks << 5)) + (o - 4) * 2048)));
    };
    auto product = [&](int n) __attribute__((always_inline)) {
        const int nb = n & 3, tb = n >> 2;
        if constexpr (I8)
            acc[nb][tb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, av[nb]),
                                                                __builtin_bit_cast(i32x4, bv[tb]), acc[nb][tb], 0, 0,
                                                                0);
        else
            acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[nb], bv[tb], acc[nb][tb], 0, 0, 0);
    };
    // operands of the next k-step read after product n of this one
    auto read_after = [&](int slot, int ks, int n) __attribute__((always_inline)) {
        if (n == 3) read_op(slot, ks, 4);
        if (n >= 4) read_op(slot, ks, n - 4);
        if (n == 7) read_op(slot, ks, 5);
    };

    // ---- pipeline. Stage kt lives in ring slot kt % 4. Iteration kt sends
    // out the DMA of stage kt+3 (into the slot of stage kt-1, which every
    // wave finished reading before the last barrier), so each stage has two
    // iterations to arrive. Within iteration kt: k-step 0's products, with
    // k-step 1's operand reads in between; k-step 1's first five products;
    // the DMA of stage kt+3; a wait until stage kt+1 has landed (vmcnt(10):
    // only the loads of stages kt+2 and kt+3 may still fly); the barrier that
    // publishes it; k-step 1's last three products with k-step 0's operand
    // reads of slot kt+1 in between, so the matrix core has work while the
    // first reads after the barrier are in flight. Every iteration
    // issues exactly five loads per thread (stages past K read zeros), so
    // the counts hold on every iteration. The loop is unrolled by the ring
    // depth so every slot is a compile-time constant.
    issue(0, 0);
    issue(1, 1);
    issue(2, 2);
    __builtin_amdgcn_s_waitcnt(0x0F70 | 10);  // stage 0 landed (stages 1 and 2 may fly)
    block_sync();
#pragma unroll
    for (int o = 0; o < 6; ++o) read_op(0, 0, o);
    auto step = [&](int kt, auto SLOT) __attribute__((always_inline)) {
        constexpr int sl = decltype(SLOT)::value;
        constexpr int ns = (sl + 1) % STAGES;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            product(n);
            read_after(sl, 1, n);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int n = 0; n < 5; ++n) {
            product(n);
            __builtin_amdgcn_sched_barrier(0);
        }
        issue(kt + 3, (sl + 3) % STAGES);
        __builtin_amdgcn_s_waitcnt(0x0F70 | 10);  // stage kt+1 landed: only stages kt+2 and kt+3 may fly
        block_sync();
        // k-step 1's last three products need no operand read: the next
        // slot's k-step 0 operands are read between them (bv[0] and av[0]
        // are free after product 4)
        read_op(ns, 0, 4);
        read_op(ns, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 5; n < 8; ++n) {
            product(n);
            read_after(ns, 0, n);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // K is a multiple of 4 stages: every iteration runs all four steps
    for (int kt = 0; kt < nk; kt += STAGES) {
        step(kt, std::integral_constant<int, 0>{});
        step(kt + 1, std::integral_constant<int, 1>{});
        step(kt + 2, std::integral_constant<int, 2>{});
        step(kt + 3, std::integral_constant<int, 3>{});
    }
    // The DMA of the three stages past the end (zeros) may still be landing
    // in the ring, which the epilogue reuses: wait for all of it, then for
    // every wave to be past the last stage.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    block_sync();

    // ---- epilogue. Lane: output row 64 wt + 32 tb + r32 of the tile; element
    // 4i + j of block nb is column 128 wn + 32 nb + 8i + 4g + j.
    // Output tiles leave through LDS (the weight ring, free now) so that each
    // store instruction writes whole rows: 16 bytes per lane straight from
    // the accumulators would touch 32 rows 16 bytes at a time, and the
    // partial-line writes cost several times the bytes.
    if (!I8 && (split_k || epilogue == PROLOG_STORE_F32)) {
        // fp32 rows are 2 KB: two passes of 64 rows (tb = 0, 1). Row lr of a
        // pass (= 32 wt + r32) holds chunk c (4 columns) at c ^ ((lr & 7) << 1).
        // A split's raw sums go to its part, at the tile's column over both
        // segments.
        float *out = split_k ? p.part + (int64_t)split * p.m * p.ld_part : static_cast<float *>(out_base);
        const int64_t ldo = split_k ? p.ld_part : ld_out;
        const int64_t col0 = (int64_t)(split_k ? tn : tj) * BN;
        const i32x4 ro = make_rsrc(out + (int64_t)m0 * ldo + col0, (uint32_t)(((int64_t)rows * ldo - col0) * 4));
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            if (tb == 1) block_sync();  // the first pass's rows have been read
            const int lr = 32 * wt + r32;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 32 * wn + 8 * nb + 2 * i + g;
                    float4 v;
                    v.x = acc[nb][tb][4 * i];
                    v.y = acc[nb][tb][4 * i + 1];
                    v.z = acc[nb][tb][4 * i + 2];
                    v.w = acc[nb][tb][4 * i + 3];
                    *reinterpret_cast<float4 *>(WS(lr >> 4) + (lr & 15) * 2048 + ((c ^ ((lr & 7) << 1)) << 4)) = v;
                }
            block_sync();
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int q = 8 * wave + (u >> 1);        // pass row
                const int ch = (u & 1) * 64 + lane;       // logical 16-byte chunk
                const int row = 64 * (q >> 5) + 32 * tb + (q & 31);
                const i32x4 v =
                    *reinterpret_cast<const i32x4 *>(WS(q >> 4) + (q & 15) * 2048 + ((ch ^ ((q & 7) << 1)) << 4));
                prolog_raw_buffer_store_b128(v, ro, (uint32_t)row * (uint32_t)ldo * 4 + ch * 16, 0, CPOL_NT);
            }
        }
        return;
    }

    // Every load of the epilogue (gamma, and the rope's cos / sin for the
    // quarter holding columns 448 .. 511) goes out first: a load placed after
    // one of the output stores would have to wait for it (they may alias), and
    // the latency would be paid once per store. They land while the row sums
    // are reduced.
    uint2 gw[4][4];  // gamma of columns n .. n + 3 for (nb, i), bf16 pairs
    if (!I8 && gamma != nullptr) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                gw[nb][i] = *reinterpret_cast<const uint2 *>(
                    gamma + ((int64_t)tj * BN + 128 * wn + 32 * nb + 8 * i + 4 * g) * 2);
    }
    const bool rope_wave = wn == 3;  // its blocks nb = 2, 3 are columns 448 .. 511
    i16x4 rcos[2][4][2], rsin[2][4][2];  // [nb - 2][i][tb]
    if (rope_wave) {
        const i32x4 rc = make_rsrc(static_cast<const unsigned char *>(p.rope_cos) + (int64_t)m0 * PROLOG_ROPE * 2,
                                   (uint32_t)rows * PROLOG_ROPE * 2);
        const i32x4 rs = make_rsrc(static_cast<const unsigned char *>(p.rope_sin) + (int64_t)m0 * PROLOG_ROPE * 2,
                                   (uint32_t)rows * PROLOG_ROPE * 2);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    const int row = 64 * wt + 32 * tb + r32;
                    const uint32_t co = (uint32_t)(row * PROLOG_ROPE + 32 * nb + 8 * i + 4 * g) * 2;
                    rcos[nb][i][tb] = prolog_raw_buffer_load_b64(rc, co, 0, 0);
                    rsin[nb][i][tb] = prolog_raw_buffer_load_b64(rs, co, 0, 0);
                }
    }

    // int8: the products scaled to fp32 by their row's and column's scales
    // (the column scales pass through the free ring, so that a lane does not
    // hold its 64 of them); bf16: as they are.
    f32x16 fa[4][2];
    if constexpr (I8) {
        float *csl = reinterpret_cast<float *>(xs1);  // [512] column scales of the tile
        csl[tid] = cs_pre;
        block_sync();
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 c4 = *reinterpret_cast<const float4 *>(csl + 128 * wn + 32 * nb + 8 * i + 4 * g);
                const float cj[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        fa[nb][tb][4 * i + j] = static_cast<float>(acc[nb][tb][4 * i + j]) * (rs_pre[tb] * cj[j]);
            }
    } else {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) fa[nb][tb] = acc[nb][tb];
    }

    // RmsNorm over the tile's 512 columns: per-lane partial sums of squares,
    // the lane pair (l, l ^ 32) of a row, then the 4 column quarters in LDS.
    float ssq[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                s0 = __builtin_fmaf(fa[nb][tb][e], fa[nb][tb][e], s0);
                s1 = __builtin_fmaf(fa[nb][tb][e + 1], fa[nb][tb][e + 1], s1);
            }
        const float sm = s0 + s1;
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(sm), __float_as_int(sm), false, false);
        ssq[tb] = __int_as_float(sw[0]) + __int_as_float(sw[1]);
    }
    float *red = reinterpret_cast<float *>(xs0);  // [4 quarters][128 rows]
    if (g == 0) {
        red[wn * BM + 64 * wt + r32] = ssq[0];
        red[wn * BM + 64 * wt + 32 + r32] = ssq[1];
    }
    block_sync();
    float inv[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int row = 64 * wt + 32 * tb + r32;
        const float tot = ((red[row] + red[BM + row]) + red[2 * BM + row]) + red[3 * BM + row];
        inv[tb] = 1.0f / sqrtf(tot * (1.0f / BN) + p.eps);
    }

    __bf16 *out = static_cast<__bf16 *>(out_base);
    const i32x4 ro = make_rsrc(out + (int64_t)m0 * ld_out + (int64_t)tj * BN,
                               (uint32_t)(((int64_t)rows * ld_out - (int64_t)tj * BN) * 2));
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = 128 * wn + 32 * nb + 8 * i + 4 * g;
            float gm[4] = {1.f, 1.f, 1.f, 1.f};
            if (!I8 && gamma != nullptr) {
                gm[0] = bf16_bits_to_float(gw[nb][i].x & 0xffff);
                gm[1] = bf16_bits_to_float(gw[nb][i].x >> 16);
                gm[2] = bf16_bits_to_float(gw[nb][i].y & 0xffff);
                gm[3] = bf16_bits_to_float(gw[nb][i].y >> 16);
            }
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const int row = 64 * wt + 32 * tb + r32;
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = fa[nb][tb][4 * i + j] * inv[tb] * gm[j];
                if (nb >= 2 && rope_wave) {
                    float cs[4], sn[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        cs[j] = bf16_bits_to_float((unsigned short)rcos[nb - 2][i][tb][j]);
                        sn[j] = bf16_bits_to_float((unsigned short)rsin[nb - 2][i][tb][j]);
                    }
                    const float a0 = v[0] * cs[0] - v[1] * sn[0];
                    const float a1 = v[1] * cs[1] + v[0] * sn[1];
                    const float a2 = v[2] * cs[2] - v[3] * sn[2];
                    const float a3 = v[3] * cs[3] + v[2] * sn[3];
                    v[0] = a0;
                    v[1] = a1;
                    v[2] = a2;
                    v[3] = a3;
                }
                bf16x4 o4;
#pragma unroll
                for (int j = 0; j < 4; ++j) o4[j] = static_cast<__bf16>(v[j]);
                // tile row r (1 KB) holds 16-byte chunk c (8 columns) at c ^ (r & 15)
                *reinterpret_cast<bf16x4 *>(WS(row >> 5) + (row & 31) * 1024 + (((n >> 3) ^ (row & 15)) << 4) + g * 8) =
                    o4;
            }
        }
    block_sync();
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int row = 16 * wave + u;
        const i32x4 v = *reinterpret_cast<const i32x4 *>(WS(row >> 5) + (row & 31) * 1024 + ((lane ^ (row & 15)) << 4));
        prolog_raw_buffer_store_b128(v, ro, (uint32_t)row * (uint32_t)ld_out * 2 + lane * 16, 0, CPOL_NT);
    }
}

// The epilogues of a product run split over K: one wave per (row, tile),
// 8 columns per lane. The lane adds the parts' raw sums of its columns, then
// applies the tile's segment epilogue as the product kernel does: the fp32
// row (PROLOG_STORE_F32), or RmsNorm over the tile's 512 columns times gamma,
// the rope on columns 448 .. 511 (pairs (2i, 2i + 1) with the row's cos /
// sin of both columns) and bf16 (PROLOG_NORM_ROPE).
__global__ __launch_bounds__(256) void prolog_split_reduce_kernel(const PrologGemmParams p) {
    const int lane = threadIdx.x & 63;
    const int n_tiles = p.seg[0].n_tiles + p.seg[1].n_tiles;
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= p.m * n_tiles) return;
    const int row = w / n_tiles, tn = w % n_tiles;
    const bool second = tn >= p.seg[0].n_tiles;
    const PrologSegment &sg = second ? p.seg[1] : p.seg[0];
    const int tj = second ? tn - p.seg[0].n_tiles : tn;
    const int c0 = 8 * lane;  // first column of the lane within the tile
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float *src = p.part + (int64_t)row * p.ld_part + (int64_t)tn * BN + c0;
    for (int s = 0; s < p.k_splits; ++s) {
        const float4 a = *reinterpret_cast<const float4 *>(src);
        const float4 b = *reinterpret_cast<const float4 *>(src + 4);
        v[0] += a.x;
        v[1] += a.y;
        v[2] += a.z;
        v[3] += a.w;
        v[4] += b.x;
        v[5] += b.y;
        v[6] += b.z;
        v[7] += b.w;
        src += (int64_t)p.m * p.ld_part;
    }
    if (sg.epilogue == PROLOG_STORE_F32) {
        float *o = static_cast<float *>(sg.out) + (int64_t)row * sg.ld_out + (int64_t)tj * BN + c0;
        *reinterpret_cast<float4 *>(o) = float4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<float4 *>(o + 4) = float4{v[4], v[5], v[6], v[7]};
        return;
    }
    float ssq = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ssq = __builtin_fmaf(v[j], v[j], ssq);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ssq += __shfl_xor(ssq, o, 64);
    const float inv = 1.0f / sqrtf(ssq * (1.0f / BN) + p.eps);
    const __bf16 *gamma = static_cast<const __bf16 *>(sg.gamma);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float gm = gamma != nullptr ? static_cast<float>(gamma[(int64_t)tj * BN + c0 + j]) : 1.f;
        v[j] = v[j] * inv * gm;
    }
    if (c0 >= BN - PROLOG_ROPE) {
        const __bf16 *cs = static_cast<const __bf16 *>(p.rope_cos) + (int64_t)row * PROLOG_ROPE + (c0 - (BN - PROLOG_ROPE));
        const __bf16 *sn = static_cast<const __bf16 *>(p.rope_sin) + (int64_t)row * PROLOG_ROPE + (c0 - (BN - PROLOG_ROPE));
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            const float a0 = v[j] * static_cast<float>(cs[j]) - v[j + 1] * static_cast<float>(sn[j]);
            const float a1 = v[j + 1] * static_cast<float>(cs[j + 1]) + v[j] * static_cast<float>(sn[j + 1]);
            v[j] = a0;
            v[j + 1] = a1;
        }
    }
    bf16x4 lo, hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        lo[j] = static_cast<__bf16>(v[j]);
        hi[j] = static_cast<__bf16>(v[4 + j]);
    }
    __bf16 *o = static_cast<__bf16 *>(sg.out) + (int64_t)row * sg.ld_out + (int64_t)tj * BN + c0;
    *reinterpret_cast<bf16x4 *>(o) = lo;
    *reinterpret_cast<bf16x4 *>(o + 4) = hi;
}

// One wave per row: RmsNorm over cols fp32 values, times gamma, to bf16.
__global__ __launch_bounds__(256) void prolog_rms_rows_kernel(const float *y, int64_t ld_y, const __bf16 *gamma,
                                                              __bf16 *out, int64_t ld_out, int32_t rows,
                                                              int32_t cols, float eps) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float *yr = y + (int64_t)row * ld_y;
    float s = 0.f;
    for (int c = lane * 4; c < cols; c += 256) {
        const float4 v = *reinterpret_cast<const float4 *>(yr + c);
        s = __builtin_fmaf(v.x, v.x, s);
        s = __builtin_fmaf(v.y, v.y, s);
        s = __builtin_fmaf(v.z, v.z, s);
        s = __builtin_fmaf(v.w, v.w, s);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    const float inv = 1.0f / sqrtf(s / (float)cols + eps);
    __bf16 *orow = out + (int64_t)row * ld_out;
    for (int c = lane * 4; c < cols; c += 256) {
        const float4 v = *reinterpret_cast<const float4 *>(yr + c);
        const uint2 gw = *reinterpret_cast<const uint2 *>(gamma + c);
        bf16x4 o4;
        o4[0] = static_cast<__bf16>(v.x * inv * bf16_bits_to_float(gw.x & 0xffff));
        o4[1] = static_cast<__bf16>(v.y * inv * bf16_bits_to_float(gw.x >> 16));
        o4[2] = static_cast<__bf16>(v.z * inv * bf16_bits_to_float(gw.y & 0xffff));
        o4[3] = static_cast<__bf16>(v.w * inv * bf16_bits_to_float(gw.y >> 16));
        *reinterpret_cast<bf16x4 *>(orow + c) = o4;
    }
}

// One wave per row: c = RmsNorm over the row's cols = 256 NV fp32 values
// (kept in registers) * gamma, computed as in prolog_rms_rows_kernel; then the
// row's largest |c|, its scale max / 127, and the int8 codes c / scale
// rounded to nearest, ties to even (so within [-127, 127]); a zero row gets
// scale 0 and codes 0.
template <int NV>
__global__ __launch_bounds__(256) void prolog_quant_rows_kernel(const float *y, int64_t ld_y, const __bf16 *gamma,
                                                                signed char *codes, int64_t ld_codes, float *scale,
                                                                int32_t rows, float eps) {
    constexpr int COLS = 256 * NV;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float *yr = y + (int64_t)row * ld_y;
    float4 v[NV];
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        v[u] = *reinterpret_cast<const float4 *>(yr + lane * 4 + 256 * u);
        s = __builtin_fmaf(v[u].x, v[u].x, s);
        s = __builtin_fmaf(v[u].y, v[u].y, s);
        s = __builtin_fmaf(v[u].z, v[u].z, s);
        s = __builtin_fmaf(v[u].w, v[u].w, s);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    const float inv = 1.0f / sqrtf(s / (float)COLS + eps);
    float amax = 0.f;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const uint2 gw = *reinterpret_cast<const uint2 *>(gamma + lane * 4 + 256 * u);
        v[u].x = v[u].x * inv * bf16_bits_to_float(gw.x & 0xffff);
        v[u].y = v[u].y * inv * bf16_bits_to_float(gw.x >> 16);
        v[u].z = v[u].z * inv * bf16_bits_to_float(gw.y & 0xffff);
        v[u].w = v[u].w * inv * bf16_bits_to_float(gw.y >> 16);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const float sc = amax / 127.0f;
    signed char *crow = codes + (int64_t)row * ld_codes;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const float c4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        unsigned packed = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = sc > 0.f ? static_cast<int>(rintf(c4[j] / sc)) : 0;
            packed |= (static_cast<unsigned>(q) & 0xffu) << (8 * j);
        }
        *reinterpret_cast<unsigned *>(crow + lane * 4 + 256 * u) = packed;
    }
    if (lane == 0) scale[row] = sc;
}

}  // namespace

hipError_t launch_prolog_pack(const PrologGemmParams &p, hipStream_t stream) {
    if (p.a1 != nullptr) return hipErrorInvalidValue;
    const int32_t nk = p.k / (p.int8 ? 2 * PROLOG_BK : PROLOG_BK);
    for (int i = 0; i < 2; ++i) {
        const PrologSegment &sg = p.seg[i];
        if (sg.n_tiles <= 0) continue;
        if (p.int8)
            hipLaunchKernelGGL(prolog_pack_kernel<true>, dim3((unsigned)(sg.n_tiles * nk)), dim3(256), 0, stream,
                               static_cast<const unsigned char *>(sg.w), sg.ldw, nk,
                               static_cast<unsigned char *>(sg.wp));
        else
            hipLaunchKernelGGL(prolog_pack_kernel<false>, dim3((unsigned)(sg.n_tiles * nk)), dim3(256), 0, stream,
                               static_cast<const unsigned char *>(sg.w), sg.ldw, nk,
                               static_cast<unsigned char *>(sg.wp));
    }
    return hipGetLastError();
}

hipError_t launch_prolog_gemm(const PrologGemmParams &p, hipStream_t stream) {
    const int n_tiles = p.seg[0].n_tiles + p.seg[1].n_tiles;
    const int m_tiles = (p.m + PROLOG_BM - 1) / PROLOG_BM;
    if (p.m <= 0 || n_tiles <= 0) return hipSuccess;
    const unsigned splits = (!p.int8 && p.k_splits > 1) ? (unsigned)p.k_splits : 1u;
    if (p.a1 != nullptr && (p.int8 || splits > 1 || p.seg[1].n_tiles <= 0)) return hipErrorInvalidValue;
    if (p.int8)
        hipLaunchKernelGGL(prolog_gemm_kernel<true>, dim3((unsigned)(n_tiles * m_tiles)), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL(prolog_gemm_kernel<false>, dim3((unsigned)(n_tiles * m_tiles) * splits), dim3(NT), 0,
                           stream, p);
    return hipGetLastError();
}

hipError_t launch_prolog_split_reduce(const PrologGemmParams &p, hipStream_t stream) {
    const int64_t waves = (int64_t)p.m * (p.seg[0].n_tiles + p.seg[1].n_tiles);
    if (waves <= 0) return hipSuccess;
    hipLaunchKernelGGL(prolog_split_reduce_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_prolog_rms_rows(const float *y, int64_t ld_y, const void *gamma, void *out, int64_t ld_out,
                                  int32_t rows, int32_t cols, float eps, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(prolog_rms_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, y, ld_y,
                       static_cast<const __bf16 *>(gamma), static_cast<__bf16 *>(out), ld_out, rows, cols, eps);
    return hipGetLastError();
}

hipError_t launch_prolog_quant_rows(const float *y, int64_t ld_y, const void *gamma, void *codes, int64_t ld_codes,
                                    float *scale, int32_t rows, int32_t cols, float eps, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + 3) / 4));
    const __bf16 *g = static_cast<const __bf16 *>(gamma);
    signed char *c = static_cast<signed char *>(codes);
    switch (cols) {
        case 512:
            hipLaunchKernelGGL(prolog_quant_rows_kernel<2>, grid, dim3(256), 0, stream, y, ld_y, g, c, ld_codes, scale,
                               rows, eps);
            break;
        case 1024:
            hipLaunchKernelGGL(prolog_quant_rows_kernel<4>, grid, dim3(256), 0, stream, y, ld_y, g, c, ld_codes, scale,
                               rows, eps);
            break;
        case 1536:
            hipLaunchKernelGGL(prolog_quant_rows_kernel<6>, grid, dim3(256), 0, stream, y, ld_y, g, c, ld_codes, scale,
                               rows, eps);
            break;
        case 2048:
            hipLaunchKernelGGL(prolog_quant_rows_kernel<8>, grid, dim3(256), 0, stream, y, ld_y, g, c, ld_codes, scale,
                               rows, eps);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mla
