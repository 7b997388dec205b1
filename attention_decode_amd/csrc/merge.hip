// merge.hip -- LSE-weighted combine of split partials (mslk splitk_kernels.py, _splitK_reduce):
//
//   M = max_s lse_s,  w_s = exp(lse_s - M),  out = sum_s w_s o_s / sum_s w_s,
//   lse = M + ln sum_s w_s;   M = -inf  ->  out = 0, lse = -inf.
//
// One wave per output row; lane l owns head_dim_v / 64 consecutive output columns, so every
// partial row is read with one coalesced wave-wide load. The split weights are wave-uniform:
// the row index is made uniform with readfirstlane, so the LSE reads become scalar loads and the
// exponentials are computed once per split per lane without any cross-lane traffic beyond the
// max. Ragged batches merge only the splits that hold keys: ceil(L_b / chunk) on the whole-step
// paths, or the caller's count per sequence (splits_per_batch) on the public merge. With
// variable query lengths the rows of tokens past a sequence's count are skipped, and the others
// are written to their packed output rows.
#include "ad_internal.h"

#include <math.h>

namespace ad {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

template <int VEC, bool OUT_BF16>
__global__ void __launch_bounds__(64 * kRowsPerBlock) merge_kernel(const MergeParams p) {
    const int lane = threadIdx.x & 63;
    const int row = __builtin_amdgcn_readfirstlane(blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6));
    if (row >= p.rows) return;
    const int t = (row / p.num_q_heads) % p.q_len;
    const int b = row / (p.num_q_heads * p.q_len);
    const int Dv = p.head_dim_v;
    if (p.q_starts && t >= q_rows(p.q_starts, p.q_len, b).n) return;  // uniform: no such token
    const OutIdx oi = out_index(p.q_starts, p.q_len, p.num_q_heads, p.out_s, row);

    int S = p.num_splits;
    if (p.count_by_len) {
        const int Lb = p.seq_lens ? p.seq_lens[b] : p.kv_len_max;
        const int Sb = Lb > 0 ? (Lb + p.chunk - 1) / p.chunk : 0;
        S = min(S, Sb);
    }
    if (p.splits_per_batch) S = min(S, max(p.splits_per_batch[b], 0));
    const float *ls = p.part_lse + (int64_t)row * p.num_splits;
    const float *po = p.part_o + (int64_t)row * p.num_splits * Dv + lane * VEC;
    // The partial rows of the first 4 splits are loaded before the LSEs are read, so that both
    // round trips overlap; later splits follow 4 at a time. Splits are summed in ascending order.
    float x[4][VEC];
    auto load4 = [&](int s0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float *src = po + (int64_t)(s0 + j) * Dv;
            if (s0 + j < S) {
                if constexpr (VEC % 4 == 0) {
#pragma unroll
                    for (int k = 0; k < VEC; k += 4) {
                        const float4 v = *reinterpret_cast<const float4 *>(src + k);
                        x[j][k] = v.x;
                        x[j][k + 1] = v.y;
                        x[j][k + 2] = v.z;
                        x[j][k + 3] = v.w;
                    }
                } else if constexpr (VEC == 2) {
                    const float2 v = *reinterpret_cast<const float2 *>(src);
                    x[j][0] = v.x;
                    x[j][1] = v.y;
                } else {
                    x[j][0] = src[0];
                }
            } else {
#pragma unroll
                for (int k = 0; k < VEC; ++k) x[j][k] = 0.f;
            }
        }
    };
    load4(0);
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ls[s]);
    const float ms = (M == -INFINITY) ? 0.f : M;

    float o[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) o[j] = 0.f;
    float W = 0.f;
    for (int s0 = 0; s0 < S; s0 += 4) {
        if (s0 > 0) load4(s0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (s0 + j < S) {
                const float w = __builtin_amdgcn_exp2f((ls[s0 + j] - ms) * kLog2e);
                W += w;
#pragma unroll
                for (int k = 0; k < VEC; ++k) o[k] += w * x[j][k];
            }
        }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    char *dst = static_cast<char *>(p.out) + (oi.off + lane * VEC) * (OUT_BF16 ? 2 : 4);
    if constexpr (OUT_BF16) {
        __bf16 *d = reinterpret_cast<__bf16 *>(dst);
#pragma unroll
        for (int j = 0; j < VEC; ++j) d[j] = (__bf16)(o[j] * inv);
    } else {
        float *d = reinterpret_cast<float *>(dst);
#pragma unroll
        for (int j = 0; j < VEC; ++j) d[j] = o[j] * inv;
    }
    if (p.lse && lane == 0) p.lse[oi.lse] = W > 0.f ? M + __builtin_amdgcn_logf(W) * kLn2 : -INFINITY;
}

template <int VEC>
hipError_t launch_vec(const MergeParams &p, hipStream_t stream) {
    dim3 grid((p.rows + kRowsPerBlock - 1) / kRowsPerBlock);
    if (p.out_dtype == DT_BF16)
        hipLaunchKernelGGL((merge_kernel<VEC, true>), grid, dim3(64 * kRowsPerBlock), 0, stream, p);
    else
        hipLaunchKernelGGL((merge_kernel<VEC, false>), grid, dim3(64 * kRowsPerBlock), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeParams &p, hipStream_t stream) {
    switch (p.head_dim_v) {
        case 64: return launch_vec<1>(p, stream);
        case 128: return launch_vec<2>(p, stream);
        case 256: return launch_vec<4>(p, stream);
        case 512: return launch_vec<8>(p, stream);
        default: return launch_vec<16>(p, stream);
    }
}

}  // namespace ad
