// fused_merge.h -- the split merge run inside the partial pass, so that a decode step is one
// launch.
//
// Every work group of a work unit (sequence b, KV head h, block of query rows) whose split holds
// keys stores its partial rows (o_s, lse_s) exactly as in the two-pass path, then arrives on the
// unit's counter. The group that completes the count merges all splits of the unit's rows with
// the arithmetic of the separate merge kernel (mslk splitk_kernels.py, _splitK_reduce):
//
//   M = max_s lse_s,  w_s = exp(lse_s - M),  out = sum_s w_s o_s / sum_s w_s,
//   lse = M + ln sum_s w_s;   M = -inf  ->  out = 0, lse = -inf,
//
// with the splits summed in the same order, so the result equals the two-pass result bit for bit.
// The election of the last group by a counter that wraps back to zero on the last arrival is the
// multi-block mode of the TensorRT-LLM xqa kernel (mha.cu, the semaphore increment that picks the
// last CTA to merge): the counters need to be zero once, before their first use, and every launch
// leaves them zero again.
//
// Visibility across the chip: each XCD has its own L2, which does not see the other XCDs' ordinary
// stores. The partials therefore travel as agent-scope accesses: stores that write through to the
// device-coherent level and loads that read from it (store_partial / load_partial). An arriving
// group waits until its stores are acknowledged, synchronises, and one lane increments the
// counter with a device-scope atomic; the elected group reads the partials with coherent loads.
// No fence is needed: a fence at agent scope would write back and invalidate the whole L2 of the
// XCD under the other groups' streaming loads, which costs far more than the merge saves.
#pragma once

#include "ad_internal.h"

#include <math.h>

namespace ad {

constexpr float kFusedLog2e = 1.4426950408889634f;
constexpr float kFusedLn2 = 0.69314718055994531f;
// s_waitcnt vmcnt(0) with no wait on the other counters (gfx9 encoding): this wave's stores are done.
constexpr int kWaitStores = (7 << 4) | (15 << 8);

// A partial value stored / loaded at agent scope (coherent across the XCDs' L2 caches).
__device__ __forceinline__ void store_partial(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_partial(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Output element offset (column 0) and LSE index of padded row `row` (packed rows with q_starts).
__device__ __forceinline__ OutIdx out_index(const PartialParams &p, int row) {
    return out_index(p.q_starts, p.q_len, p.num_q_heads, p.out_s, row);
}

__device__ __forceinline__ void store_out(const PartialParams &p, int64_t off, float v) {
    if (p.out_dtype == DT_BF16)
        static_cast<__bf16 *>(p.out)[off] = (__bf16)v;
    else
        static_cast<float *>(p.out)[off] = v;
}

// Writes out = 0 and lse = -inf for rows r < nr (a unit without any key: no split arrives).
// Both helpers are always inlined: a call would pass the kernel's parameter block by address,
// which moves it to scratch and turns every load of the calling kernel into a flat load.
template <int NTHREADS, int DV, typename RowFn>
__device__ __forceinline__ void fused_write_empty(const PartialParams &p, int nr, RowFn out_row) {
    for (int r = 0; r < nr; ++r) {
        const OutIdx oi = out_index(p, (int)out_row(r));
        for (int d = threadIdx.x; d < DV; d += NTHREADS) store_out(p, oi.off + d, 0.f);
        if (p.lse && threadIdx.x == 0) p.lse[oi.lse] = -INFINITY;
    }
}

// Arrival of a work group that has stored its partial rows with store_partial; the last of the
// unit's nsplit groups merges rows r < nr (<= 64; flat output rows out_row(r)). DV: head_dim_v.
// EPT: elements of the nr x DV output each thread owns at most (ceil(max rows * DV / NTHREADS)).
// weights: LDS scratch of at least nr * nsplit floats that the caller no longer needs. Every
// thread of the group must call it.
template <int NTHREADS, int DV, int EPT, typename RowFn>
__device__ __forceinline__ void fused_arrive_merge(const PartialParams &p, int unit, int nsplit, int nr, RowFn out_row,
                                                   float *weights) {
    __shared__ int s_last;
    __shared__ int s_row[64];                // per row: LSE index
    __shared__ float s_inv[64], s_lse[64];   // per row: 1 / sum_s w_s and the merged LSE
    __shared__ int64_t s_off[64];            // per row: output element offset of column 0
    __builtin_amdgcn_s_waitcnt(kWaitStores);  // this wave's partial stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t last = (uint32_t)(nsplit - 1);
        s_last = __builtin_amdgcn_atomic_inc32(p.counters + unit, last, __ATOMIC_RELAXED, "agent") == last;
    }
    __syncthreads();
    if (!s_last) return;  // uniform

    // Every load of the merge is issued at once: the LSEs of all splits and, per owned element
    // i = tid + e * NTHREADS (e < EPT), the partial outputs of the first 4 splits (later splits
    // follow 4 at a time). Each element sums its splits in ascending order.
    const int S = p.num_splits, n = nr * DV;
    const float *src[EPT];
    float o[EPT], x[EPT][4];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = threadIdx.x + e * NTHREADS;
        const int r = i < n ? i / DV : 0, d = i - r * DV;
        src[e] = p.part_o + (int64_t)(int)out_row(r) * S * DV + d;
        o[e] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[e][j] = (i < n && j < nsplit) ? load_partial(src[e] + (int64_t)j * DV) : 0.f;
    }
    for (int i = threadIdx.x; i < nr * nsplit; i += NTHREADS) {
        const int r = i / nsplit, s = i - r * nsplit;
        weights[i] = load_partial(p.part_lse + (int64_t)(int)out_row(r) * S + s);
    }
    for (int r = threadIdx.x; r < nr; r += NTHREADS) {
        const OutIdx oi = out_index(p, (int)out_row(r));
        s_row[r] = oi.lse;
        s_off[r] = oi.off;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < nr; r += NTHREADS) {
        float *w = weights + r * nsplit;
        float M = -INFINITY;
        for (int s = 0; s < nsplit; ++s) M = fmaxf(M, w[s]);
        const float ms = (M == -INFINITY) ? 0.f : M;
        float W = 0.f;
        for (int s = 0; s < nsplit; ++s) {
            const float e = __builtin_amdgcn_exp2f((w[s] - ms) * kFusedLog2e);
            W += e;
            w[s] = e;
        }
        s_inv[r] = W > 0.f ? 1.f / W : 0.f;
        s_lse[r] = W > 0.f ? M + __builtin_amdgcn_logf(W) * kFusedLn2 : -INFINITY;
    }
    __syncthreads();
    for (int s0 = 0; s0 < nsplit; s0 += 4) {
        if (s0 > 0) {
#pragma unroll
            for (int e = 0; e < EPT; ++e)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    x[e][j] = (threadIdx.x + e * NTHREADS < n && s0 + j < nsplit)
                                  ? load_partial(src[e] + (int64_t)(s0 + j) * DV) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int r = (threadIdx.x + e * NTHREADS) / DV;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (s0 + j < nsplit && r < nr) o[e] += weights[r * nsplit + s0 + j] * x[e][j];
        }
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = threadIdx.x + e * NTHREADS;
        if (i >= n) continue;
        const int r = i / DV, d = i - r * DV;
        store_out(p, s_off[r] + d, o[e] * s_inv[r]);
        if (p.lse && d == 0) p.lse[s_row[r]] = s_lse[r];
    }
}

}  // namespace ad
