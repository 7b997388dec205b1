// splitkv_valu.hip -- partial split-KV pass on the vector ALUs (few query rows per KV head).
//
// What it computes (per work unit = split s, KV head h, sequence b): for the R = G * q_len query
// rows that read head h (the G query heads hq = h*G + g of every query token t, packed as in the
// PyTorch Inductor flex_decode.py.jinja template), the attention restricted to the keys of the
// split's range, as a normalised partial output o_s = acc / l and a natural-log LSE
// (mslk splitk_kernels.py, _fwd_kernel_splitK epilogue). The online softmax keeps scores in
// base-2 units, q.k * scale * log2(e), and rescales with exp2 (the same page's qk_scale and
// exp2 update; FlashInfer mla.cuh update_mdo_states_).
//
// Why VALU and not MFMA: with at most 8 rows per KV head the step reads 256-512 B of K/V per key
// and does ~4 flop/B, far under the fp32-vector ridge; padding 4 rows to an MFMA tile of 16 would
// only move the bottleneck to operand shuffles. The kernel is built to keep HBM busy:
//
//   * 8 lanes share one K/V row; each lane loads 16-byte pieces, so one wave-wide load covers 8
//     rows x 128 contiguous bytes (full cache lines). The 8 lanes of a row reduce their partial
//     dot products with 3 DPP adds (quad_perm 1032, quad_perm 2301, row_half_mirror).
//   * Each of the 8 row-slots of a wave runs its own online softmax over the keys it loads, so
//     the hot loop has no cross-slot traffic; slots and waves are combined once, at the end.
//   * Software pipeline per wave: V loads of step i and K loads of step i+1 are in flight while
//     step i's scores and P.V are computed.
//   * bf16 scores use v_dot2 (bf16 pairs, fp32 accumulate); q stays exact bf16 and the scale is
//     applied to the fp32 dot. P.V accumulates in fp32 with P kept in fp32.
//   * Page ids (paged cache) and listed block ids (block-sparse) of the split are staged in LDS
//     once, so address generation never waits on a global load behind the K/V stream.
//   * Masked keys are never read: their loads are redirected to the unit's own query row (always
//     valid, finite memory) and their probability is forced to 0, so NaN/Inf in unused cache
//     slots cannot leak into the result.
#include "ad_internal.h"

#include <math.h>

namespace ad {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLanesPerRow = 8;               // lanes sharing one K/V row
constexpr int kSlots = 64 / kLanesPerRow;     // rows one wave-wide load covers

template <typename T>
struct Elem;
template <>
struct Elem<float> {
    static constexpr int kPer16 = 4;
};
template <>
struct Elem<uint16_t> {  // bf16 bit patterns
    static constexpr int kPer16 = 8;
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 lanes of a row-slot; every lane of the slot gets the total.
__device__ __forceinline__ float slot_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8
    return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Reinterpretations take the 32-bit word BY VALUE: hipcc miscompiles __builtin_bit_cast applied
// directly to an element of an ext_vector_type lvalue (it reads the wrong element), so vector
// elements always pass through a plain uint32_t first.
__device__ __forceinline__ float as_f32(uint32_t w) { return __uint_as_float(w); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T, int D, int RP, int MODE, int U>
__global__ void __launch_bounds__(kThreads) partial_valu_kernel(const PartialParams p) {
    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int kPer16 = Elem<T>::kPer16;
    constexpr int kPieces = D * (int)sizeof(T) / (16 * kLanesPerRow);  // 16-B pieces per lane per row
    static_assert(kPieces >= 1, "row too short for 8 lanes of 16 bytes");
    constexpr int kEPL = kPieces * kPer16;  // elements per lane per row
    constexpr int kStep = kSlots * U;       // keys per wave per step

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = lane / kLanesPerRow, c = lane % kLanesPerRow;
    const int G = p.group, Q = p.q_len, R = G * Q, S = p.num_splits, Dv = p.head_dim_v;
    const int L = p.seq_lens ? p.seq_lens[b] : p.kv_len_max;

    int vlen = L;  // length of the key range the splits partition
    if constexpr (MODE == KV_SPARSE) {
        const int nb = p.num_blocks[b * p.nb_s[0] + h * p.nb_s[1]];
        vlen = nb << p.block_shift;
    }
    const int t0 = split * p.chunk;
    const int t1 = min(t0 + p.chunk, vlen);

    auto out_row = [&](int r) -> int64_t {
        const int t = r / G, g = r - t * G;
        return (int64_t)(b * Q + t) * p.num_q_heads + h * G + g;
    };

    if (t0 >= t1) {  // uniform over the work group
        if (p.write_empty) {
            for (int i = tid; i < R * Dv; i += kThreads) {
                const int r = i / Dv, d = i - r * Dv;
                p.part_o[(out_row(r) * S + split) * Dv + d] = 0.f;
            }
            for (int r = tid; r < R; r += kThreads) p.part_lse[out_row(r) * S + split] = -INFINITY;
        }
        return;
    }

    __shared__ int s_map[kMapCapacity];
    __shared__ float s_acc[kWaves][RP][D];
    __shared__ float s_m[kWaves][RP];
    __shared__ float s_l[kWaves][RP];

    int map_first = 0;
    if constexpr (MODE == KV_PAGED) {
        map_first = t0 >> p.page_shift;
        const int n = ((t1 - 1) >> p.page_shift) - map_first + 1;
        const int32_t *bt = p.block_table + b * p.bt_stride + map_first;
        for (int i = tid; i < n; i += kThreads) s_map[i] = bt[i];
    } else if constexpr (MODE == KV_SPARSE) {
        map_first = t0 >> p.block_shift;
        const int n = ((t1 - 1) >> p.block_shift) - map_first + 1;
        const int32_t *ix = p.block_idx + b * p.ix_s[0] + h * p.ix_s[1];
        for (int i = tid; i < n; i += kThreads) s_map[i] = ix[(int64_t)(map_first + i) * p.ix_s[2]];
    }
    if constexpr (MODE != KV_CONTIG) __syncthreads();

    // ---- query rows of this unit: row r = t*G + g (hq = h*G + g)
    const T *qbase = static_cast<const T *>(p.q) + b * p.q_s[0] + (int64_t)(h * G) * p.q_s[2];
    u32x4 qv[RP][kPieces];
    int qpos[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        const int t = r / G, g = r - t * G;
        qpos[r] = L - Q + t;
        const T *qr = qbase + t * p.q_s[1] + g * p.q_s[2];
#pragma unroll
        for (int i = 0; i < kPieces; ++i) qv[r][i] = u32x4{0, 0, 0, 0};
        if (r < R) {
#pragma unroll
            for (int i = 0; i < kPieces; ++i) qv[r][i] = ld16(qr + (i * kLanesPerRow + c) * kPer16);
        }
    }
    float qf[kBf16 ? 1 : RP][kBf16 ? 1 : kEPL];  // fp32 queries, prescaled by scale*log2(e)
    if constexpr (!kBf16) {
#pragma unroll
        for (int r = 0; r < RP; ++r)
#pragma unroll
            for (int i = 0; i < kPieces; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) qf[r][i * 4 + j] = as_f32(qv[r][i][j]) * p.scale_log2;
    }

    // ---- key addressing
    const T *kbase = static_cast<const T *>(p.k) + (int64_t)h * p.k_s[2];
    const T *vbase = static_cast<const T *>(p.v) + (int64_t)h * p.v_s[2];
    if constexpr (MODE != KV_PAGED) {
        kbase += b * p.k_s[0];
        vbase += b * p.v_s[0];
    }
    const T *safe = qbase;  // a finite, always-readable row for masked lanes
    const int page_mask = (1 << p.page_shift) - 1;
    const int block_mask = (1 << p.block_shift) - 1;

    float m[RP], l[RP], acc[RP][kEPL];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < kEPL; ++e) acc[r][e] = 0.f;
    }

    u32x4 kr[U][kPieces];
    const T *vptr[U];
    int kpos[U];
    bool kval[U];

    auto fetch_k = [&](int base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tok = base + u * kSlots + slot;
            bool valid = tok < t1;
            const int tt = valid ? tok : t0;
            int pos = tt;
            const T *kp;
            const T *vp;
            if constexpr (MODE == KV_PAGED) {
                const int64_t page = s_map[(tt >> p.page_shift) - map_first];
                const int sl = tt & page_mask;
                kp = kbase + page * p.k_s[0] + sl * p.k_s[1];
                vp = vbase + page * p.v_s[0] + sl * p.v_s[1];
            } else {
                if constexpr (MODE == KV_SPARSE) {
                    pos = (s_map[(tt >> p.block_shift) - map_first] << p.block_shift) + (tt & block_mask);
                    valid = valid && pos < L;
                }
                kp = kbase + (int64_t)pos * p.k_s[1];
                vp = vbase + (int64_t)pos * p.v_s[1];
            }
            if (!valid) {
                kp = safe;
                vp = safe;
            }
            kpos[u] = pos;
            kval[u] = valid;
            vptr[u] = vp;
#pragma unroll
            for (int i = 0; i < kPieces; ++i) kr[u][i] = ld16(kp + (i * kLanesPerRow + c) * kPer16);
        }
    };

    const int stride = kWaves * kStep;
    int base = t0 + wave * kStep;
    if (base < t1) fetch_k(base);
    while (base < t1) {
        // V of this step: in flight while the scores are computed
        u32x4 vr[U][kPieces];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < kPieces; ++i) vr[u][i] = ld16(vptr[u] + (i * kLanesPerRow + c) * kPer16);

        float sc[U][RP];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                float d = 0.f;
                if constexpr (kBf16) {
#pragma unroll
                    for (int i = 0; i < kPieces; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[r][i][j]), as_bf16x2(kr[u][i][j]), d,
                                                                false);
                } else {
#pragma unroll
                    for (int i = 0; i < kPieces; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) d += qf[r][i * 4 + j] * as_f32(kr[u][i][j]);
                }
                d = slot_sum(d);
                if constexpr (kBf16) d *= p.scale_log2;
                bool vis = kval[u];
                if (p.causal) vis = vis && kpos[u] <= qpos[r];
                if (p.window) vis = vis && qpos[r] - kpos[u] < p.window;
                sc[u][r] = vis ? d : -INFINITY;
            }
        }

        const int next = base + stride;
        if (next < t1) fetch_k(next);  // K of the next step: in flight during P.V

#pragma unroll
        for (int r = 0; r < RP; ++r) {
            float mx = sc[0][r];
#pragma unroll
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][r]);
            const float mn = fmaxf(m[r], mx);
            const float ms = (mn == -INFINITY) ? 0.f : mn;
            const float alpha = exp2_fast(m[r] - ms);
            m[r] = mn;
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                sc[u][r] = exp2_fast(sc[u][r] - ms);  // exp2(-inf) = 0 for masked keys
                ps += sc[u][r];
            }
            l[r] = l[r] * alpha + ps;
#pragma unroll
            for (int e = 0; e < kEPL; ++e) acc[r][e] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[kEPL];
#pragma unroll
            for (int i = 0; i < kPieces; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (kBf16) {
                        vf[i * 8 + 2 * j] = bf16_lo(vr[u][i][j]);
                        vf[i * 8 + 2 * j + 1] = bf16_hi(vr[u][i][j]);
                    } else {
                        vf[i * 4 + j] = as_f32(vr[u][i][j]);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < RP; ++r)
#pragma unroll
                for (int e = 0; e < kEPL; ++e) acc[r][e] += sc[u][r] * vf[e];
        }
        base = next;
    }

    // ---- combine the 8 row-slots of the wave (lanes c, c+8, ..., c+56)
#pragma unroll
    for (int off = kLanesPerRow; off < 64; off <<= 1) {
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const float mo = __shfl_xor(m[r], off);
            const float lo = __shfl_xor(l[r], off);
            const float mn = fmaxf(m[r], mo);
            const float ms = (mn == -INFINITY) ? 0.f : mn;
            const float a = exp2_fast(m[r] - ms), bb = exp2_fast(mo - ms);
            l[r] = l[r] * a + lo * bb;
            m[r] = mn;
#pragma unroll
            for (int e = 0; e < kEPL; ++e) acc[r][e] = acc[r][e] * a + __shfl_xor(acc[r][e], off) * bb;
        }
    }
    if (slot == 0) {
#pragma unroll
        for (int r = 0; r < RP; ++r) {
#pragma unroll
            for (int i = 0; i < kPieces; ++i)
#pragma unroll
                for (int j = 0; j < kPer16; ++j) s_acc[wave][r][(i * kLanesPerRow + c) * kPer16 + j] = acc[r][i * kPer16 + j];
            if (c == 0) {
                s_m[wave][r] = m[r];
                s_l[wave][r] = l[r];
            }
        }
    }
    __syncthreads();

    // ---- combine the waves and write o_s = acc / l, lse_s = (m + log2 l) * ln 2
    for (int i = tid; i < R * D; i += kThreads) {
        const int r = i / D, d = i - r * D;
        float M = s_m[0][r];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][r]);
        const float ms = (M == -INFINITY) ? 0.f : M;
        float lsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = exp2_fast(s_m[w][r] - ms);
            lsum += s_l[w][r] * f;
            o += s_acc[w][r][d] * f;
        }
        const int64_t row = out_row(r);
        p.part_o[(row * S + split) * Dv + d] = lsum > 0.f ? o / lsum : 0.f;
        if (d == 0)
            p.part_lse[row * S + split] = lsum > 0.f ? (M + __builtin_amdgcn_logf(lsum)) * 0.69314718055994531f : -INFINITY;
    }
}

template <typename T, int D, int RP, int MODE>
hipError_t launch_t(const PartialParams &p, hipStream_t stream) {
    constexpr int U = RP <= 4 ? 4 : 2;
    dim3 grid(p.num_splits, p.num_kv_heads, p.batch);
    hipLaunchKernelGGL((partial_valu_kernel<T, D, RP, MODE, U>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D, int RP>
hipError_t by_mode(const PartialParams &p, int mode, hipStream_t s) {
    switch (mode) {
        case KV_CONTIG: return launch_t<T, D, RP, KV_CONTIG>(p, s);
        case KV_PAGED: return launch_t<T, D, RP, KV_PAGED>(p, s);
        default: return launch_t<T, D, RP, KV_SPARSE>(p, s);
    }
}

template <typename T, int D>
hipError_t by_rows(const PartialParams &p, int rows_padded, int mode, hipStream_t s) {
    switch (rows_padded) {
        case 1: return by_mode<T, D, 1>(p, mode, s);
        case 2: return by_mode<T, D, 2>(p, mode, s);
        case 4: return by_mode<T, D, 4>(p, mode, s);
        default: return by_mode<T, D, 8>(p, mode, s);
    }
}

}  // namespace

hipError_t launch_partial_valu(const PartialParams &p, int dtype, int head_dim, int rows_padded, int mode,
                               hipStream_t stream) {
    if (dtype == DT_F32) {
        return head_dim == 64 ? by_rows<float, 64>(p, rows_padded, mode, stream)
                              : by_rows<float, 128>(p, rows_padded, mode, stream);
    }
    return head_dim == 64 ? by_rows<uint16_t, 64>(p, rows_padded, mode, stream)
                          : by_rows<uint16_t, 128>(p, rows_padded, mode, stream);
}

}  // namespace ad
