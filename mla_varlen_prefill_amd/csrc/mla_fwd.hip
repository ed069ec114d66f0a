// MLA varlen prefill attention for gfx950 (MI355X).
//
// Computes, for each sequence of a packed variable-length batch and each
// query head (Ascend Transformer Boost "MLA Prefill" page, Members table rows
// Q, QRope, K, kRope, V, qkScale, Mask, maskType):
//     S = qkScale * (Q . K^T + QRope . KRope^T) + mask,   O = softmax_rows(S) . V
//
// Design (one workgroup = 4 waves = FWD_BM = 128 query rows of one head):
//  * Each wave owns 32 query rows. Q and QRope of those rows stay in VGPRs as
//    the B operand of v_mfma_f32_32x32x16 (12 k-steps of 16: 8 nope + 4 rope).
//  * Keys are walked in tiles of FWD_BN = 64. K | KRope (64 x 192) and V
//    (64 x 128) are copied from HBM into LDS with 16-byte coalesced loads; the
//    next tile's loads are issued before the current tile's math so their
//    latency hides under it.
//  * Scores are computed transposed, S^T = K . Q^T: the accumulator then puts
//    one query row per lane (lanes l and l + 32 share a row), so row max and
//    row sum need one cross-lane step, and the probabilities already sit in
//    the B-operand layout of the second product O^T = V^T . P^T -- no LDS
//    round trip for P.
//  * V^T is read from the row-major V tile with ds_read_b64_tr_b16, which
//    transposes 16-bit elements across each group of 16 lanes.
//  * Online softmax in fp32 with exp2 (log2(e) folded into the scale);
//    probabilities rounded to the input dtype for the second product; the
//    output is normalised once at the end and rounded to nearest even.
//  * Causal / MASK_FREE: the host work list stops each workgroup at its last
//    visible tile; fully visible tiles skip the per-element mask; tiles a
//    whole wave cannot see skip the math.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mla {
namespace {

constexpr int BM = FWD_BM;
constexpr int BN = FWD_BN;
constexpr int DN = HEAD_DIM;
constexpr int DR = ROPE_DIM;
constexpr int DQK = DN + DR;
// LDS row strides in 16-bit elements. 400-byte K rows make the 16 rows read by
// one quarter-wave of ds_read_b128 land on distinct banks; 320-byte V rows do
// the same for the 8 rows touched by each half-wave of the transposing read.
constexpr int K_STRIDE = DQK + 8;
constexpr int V_STRIDE = DN + 32;

constexpr int MASK_UNDEFINED = 0;
constexpr int MASK_FREE = 3;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

struct Bf16 {
    typedef bf16x8 vec8;
    typedef bf16x4 vec4;
    typedef __bf16 scalar;
    static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
struct Fp16 {
    typedef f16x8 vec8;
    typedef f16x4 vec4;
    typedef _Float16 scalar;
    static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ float bits_to_float_bf16(unsigned short b) {
    return __uint_as_float(static_cast<unsigned>(b) << 16);
}
__device__ __forceinline__ float bits_to_float_f16(unsigned short b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ typename T::vec8 as_vec8(uint4 u) {
    return __builtin_bit_cast(typename T::vec8, u);
}

// Transposing LDS read: see the header comment.
__device__ __forceinline__ i16x4 lds_read_tr16(const unsigned short *p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

template <typename T>
__global__ __launch_bounds__(FWD_THREADS, 2) void mla_fwd_kernel(const FwdParams p) {
    __shared__ __attribute__((aligned(16))) unsigned short smem[BN * K_STRIDE + BN * V_STRIDE];
    unsigned short *Ks = smem;                  // [BN][K_STRIDE]: nope 0..127, rope 128..191
    unsigned short *Vs = smem + BN * K_STRIDE;  // [BN][V_STRIDE]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 5;     // which half of the k-slots this lane carries
    const int r32 = lane & 31;   // query row within the wave

    const WorkItem item = p.items[blockIdx.x];
    const SeqRec seq = p.seqs[item.b];
    const int h = blockIdx.y;
    const int hk = h / p.group;
    const int q_len = seq.q_len;
    const int kv_len = seq.kv_len;
    const int qi = item.q_row0 + wave * 32 + r32;  // query row within the sequence
    const bool row_ok = qi < q_len;
    const int pos = kv_len - q_len + qi;           // key position of this query row
    const int wave_pos0 = kv_len - q_len + item.q_row0 + wave * 32;
    const int wave_pos1 = wave_pos0 + 31;
    const int mask_type = p.mask_type;
    const bool causal_like = mask_type != MASK_UNDEFINED && mask_type != MASK_FREE;

    // ---- Q^T operand: lane holds row r32, k-slots g*8 .. g*8+7 of each 16-wide step
    typename T::vec8 qreg[12];
    {
        const uint4 zero = {0, 0, 0, 0};
        const int64_t tok = (int64_t)seq.q_off + qi;
        const unsigned short *qp = static_cast<const unsigned short *>(p.q) + (tok * p.heads + h) * DN + g * 8;
        const unsigned short *qrp =
            static_cast<const unsigned short *>(p.q_rope) + (tok * p.heads + h) * DR + g * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qreg[ks] = as_vec8<T>(row_ok ? *reinterpret_cast<const uint4 *>(qp + ks * 16) : zero);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qreg[8 + ks] = as_vec8<T>(row_ok ? *reinterpret_cast<const uint4 *>(qrp + ks * 16) : zero);
    }

    // ---- tile staging: thread copies 4 x 16 B of K-nope, 2 of K-rope, 4 of V
    const unsigned short *kbase = static_cast<const unsigned short *>(p.k);
    const unsigned short *krbase = static_cast<const unsigned short *>(p.k_rope);
    const unsigned short *vbase = static_cast<const unsigned short *>(p.v);
    uint4 kn[4], kr[2], vv[4];

    auto global_load = [&](int kt) {
        const uint4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = tid + FWD_THREADS * u;
            const int key = c >> 4, ch = c & 15;
            const int j = kt * BN + key;
            if (j < kv_len) {
                const int64_t row = ((int64_t)seq.kv_off + j) * p.kv_heads + hk;
                kn[u] = *reinterpret_cast<const uint4 *>(kbase + row * DN + ch * 8);
                vv[u] = *reinterpret_cast<const uint4 *>(vbase + row * DN + ch * 8);
            } else {
                kn[u] = zero;
                vv[u] = zero;
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = tid + FWD_THREADS * u;
            const int key = c >> 3, ch = c & 7;
            const int j = kt * BN + key;
            if (j < kv_len) {
                const int64_t row = ((int64_t)seq.kv_off + j) * p.kv_heads + hk;
                kr[u] = *reinterpret_cast<const uint4 *>(krbase + row * DR + ch * 8);
            } else {
                kr[u] = zero;
            }
        }
    };
    auto lds_store = [&]() {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = tid + FWD_THREADS * u;
            const int key = c >> 4, ch = c & 15;
            *reinterpret_cast<uint4 *>(Ks + key * K_STRIDE + ch * 8) = kn[u];
            *reinterpret_cast<uint4 *>(Vs + key * V_STRIDE + ch * 8) = vv[u];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = tid + FWD_THREADS * u;
            const int key = c >> 3, ch = c & 7;
            *reinterpret_cast<uint4 *>(Ks + key * K_STRIDE + DN + ch * 8) = kr[u];
        }
    };

    float m_run = -INFINITY;  // running row max (log2 units), same in both lanes of a row
    float l_run = 0.f;        // this lane's share of the running row sum
    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = 0.f;

    const int n_kt = item.kv_tiles;
    if (n_kt > 0) {
        global_load(0);
        lds_store();
    }
    __syncthreads();

    // fixed per-lane offsets of the transposing V read (see header comment)
    const int grp = lane >> 4, sl = lane & 15;
    const int v_row = 4 * (grp >> 1) + (sl >> 2);
    const int v_col = 16 * (grp & 1) + 4 * (sl & 3);

    for (int kt = 0; kt < n_kt; ++kt) {
        if (kt + 1 < n_kt) global_load(kt + 1);
        const int key0 = kt * BN;

        bool active = true;  // can any row of this wave see any key of the tile?
        if (causal_like) active = key0 <= wave_pos1;
        else if (mask_type == MASK_FREE) active = wave_pos1 >= 0 && (key0 >> 9) <= (wave_pos1 >> 9);

        if (active) {
            // ---- S^T = K . Q^T  (two 32-key blocks)
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
                const unsigned short *krow = Ks + (kb * 32 + r32) * K_STRIDE + g * 8;
#pragma unroll
                for (int ks = 0; ks < 12; ++ks) {
                    const uint4 a = *reinterpret_cast<const uint4 *>(krow + ks * 16);
                    s[kb] = T::mfma(as_vec8<T>(a), qreg[ks], s[kb]);
                }
            }

            // ---- scale and mask. Element e of block kb is key key0 + kb*32 + 8*(e/4) + 4*g + e%4.
            bool full = key0 + BN <= kv_len;
            if (causal_like) full = full && key0 + BN - 1 <= wave_pos0;
            else if (mask_type == MASK_FREE)
                full = full && wave_pos0 >= 0 && ((key0 + BN - 1) >> 9) < (wave_pos0 >> 9);
            float mx = -INFINITY;
            if (full) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        s[kb][e] *= p.scale_log2;
                        mx = fmaxf(mx, s[kb][e]);
                    }
            } else {
                const unsigned short *mrow = nullptr;
                if (mask_type == MASK_FREE && pos >= 0)
                    mrow = static_cast<const unsigned short *>(p.mask) + (pos & (MASK_TILE - 1)) * MASK_TILE;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int j = key0 + kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                        float x = s[kb][e] * p.scale_log2;
                        bool vis = j < kv_len;
                        if (causal_like) {
                            vis = vis && j <= pos;
                        } else if (mask_type == MASK_FREE) {
                            vis = vis && pos >= 0 && (j >> 9) <= (pos >> 9);
                            if (vis && (j >> 9) == (pos >> 9)) {
                                const unsigned short mb = mrow[j & (MASK_TILE - 1)];
                                const float mv = p.mask_is_bf16 ? bits_to_float_bf16(mb) : bits_to_float_f16(mb);
                                x += mv * 1.4426950408889634f;
                            }
                        }
                        x = vis ? x : -INFINITY;
                        s[kb][e] = x;
                        mx = fmaxf(mx, x);
                    }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));

            // ---- online softmax update
            const float m_new = fmaxf(m_run, mx);
            const float base = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - base);
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float pe = fast_exp2(s[kb][e] - base);
                    s[kb][e] = pe;
                    lsum += pe;
                }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[db][e] *= alpha;

            // ---- O^T += V^T . P^T, four 16-key steps
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int kb = st >> 1, half = st & 1;
                typename T::vec8 pb;
#pragma unroll
                for (int t = 0; t < 8; ++t) pb[t] = static_cast<typename T::scalar>(s[kb][8 * half + t]);
                const unsigned short *vrow = Vs + (st * 16 + v_row) * V_STRIDE + v_col;
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const i16x4 lo = lds_read_tr16(vrow + db * 32);
                    const i16x4 hi = lds_read_tr16(vrow + 8 * V_STRIDE + db * 32);
                    const i16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    o[db] = T::mfma(__builtin_bit_cast(typename T::vec8, a), pb, o[db]);
                }
            }
        }

        __syncthreads();
        if (kt + 1 < n_kt) lds_store();
        __syncthreads();
    }

    // ---- epilogue: combine the two lanes' row sums, normalise, round, store
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (row_ok) {
        unsigned short *op = static_cast<unsigned short *>(p.out) +
                             (((int64_t)seq.q_off + qi) * p.heads + h) * DN;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                typename T::vec4 v4;
#pragma unroll
                for (int j = 0; j < 4; ++j) v4[j] = static_cast<typename T::scalar>(o[db][4 * i + j] * inv);
                *reinterpret_cast<uint2 *>(op + db * 32 + 8 * i + 4 * g) = __builtin_bit_cast(uint2, v4);
            }
    }
}

}  // namespace

hipError_t launch_mla_fwd(const FwdParams &p, int dtype, int n_items, hipStream_t stream) {
    if (n_items <= 0) return hipSuccess;
    dim3 grid(n_items, p.heads);
    dim3 block(FWD_THREADS);
    if (dtype == 2)
        hipLaunchKernelGGL(mla_fwd_kernel<Bf16>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(mla_fwd_kernel<Fp16>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
