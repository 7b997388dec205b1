// splitkv_mfma.hip -- partial split-KV pass on the matrix cores (bf16, more than 8 query rows per
// KV head: grouped heads times speculative query tokens).
//
// What it computes is the same as the vector-ALU pass: per work unit (split s, block of up to 32
// query rows of KV head h, sequence b), the attention of those rows restricted to the split's keys,
// written as o_s = acc / l and a natural-log LSE (mslk splitk_kernels.py, _fwd_kernel_splitK
// epilogue), with the online softmax kept in base-2 units (same page, qk_scale and exp2 update).
// Rows r = t*G + g are the G query heads of every query token that read head h, packed as in the
// PyTorch Inductor flex_decode.py.jinja template; the bottom-right causal position of token t is
// L - q_len + t (mslk splitk_kernels.py, causal mask of the speculative-decode path).
//
// Layout on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16; operand lane maps measured on gfx950):
//
//   * Scores are computed transposed, S^T = K Q^T: K is the A operand (lane l holds 8 consecutive
//     head-dim elements of key l%32), loaded straight from HBM as 16-byte pieces; Q is the B
//     operand and stays in registers for the whole unit. The result leaves each lane with 16 keys
//     of ONE query row (row l%32; lanes l and l^32 split the tile's keys), so the row max and row
//     sum are an in-lane reduction plus one v_permlane32_swap.
//   * That accumulator already is the A operand of P.V once converted to bf16: the MFMA reduction
//     index k of lane l maps to key 16t + 8(i/4) + 4(l/32) + i%4 (t = k-step, i = element), and
//     the V operand is built with the same key order.
//   * V is the B operand of P.V and must be read key-major per lane, while memory holds it
//     head-dim-major. Each wave stores its V tile in a private LDS region (16-byte chunks
//     XOR-swizzled by row so that both the stores and the transposing reads avoid bank
//     conflicts) and reads it back with ds_read_b64_tr_b16, which hands every lane four keys of
//     one column.
//   * A wave handles 32-key tiles; the 4 waves of a work group take every 4th tile of the split,
//     each with its own running max / sum / accumulator, combined once through LDS at the end.
//     Loads of the next tile are issued before the arithmetic of the current one (two register
//     buffers, loop unrolled by two).
//   * Keys outside the split, past the sequence, in no visible range of any row of the unit, or in
//     unlisted blocks are never read: their loads are redirected to the unit's own query row and
//     their probability is exactly 0. Tiles that are fully visible to every row skip all masking.
//   * Lazy rescaling as in the vector pass: a row's reference max only moves when a score clears
//     it by more than 2^8; the accumulator rows are rescaled through a small LDS exchange because
//     the output layout spreads a row over other lanes than the score layout does.
//   * P is rounded to bf16 for the P.V product and the output normaliser sums the rounded values
//     (TensorRT-LLM mha.cu computeRowSum; FlashInfer mla.cuh compute_mla_pv); the LSE uses the
//     fp32 sum.
//   * An fp8 (OCP E4M3) cache with fp32 row scales (TensorRT-LLM mha.cu, kvCacheScale; mslk
//     splitk_kernels.py, _process_fp8_quantization): a lane loads its key's bytes as 16-byte
//     pieces at 32j + 16*half and converts each into two k-steps of bf16 operands exactly; Q is
//     loaded in the same head-dim order (the reduction order over the head dim is free as long
//     as both operands share it). V is converted into the same bf16 LDS tile. The key scales
//     multiply the fp32 scores; the value scales go into P before its bf16 rounding, and the
//     normaliser sums the rounded products divided by their scales again.
#include "ad_internal.h"
#include "fused_merge.h"
#include "mfma_util.h"

#include <limits.h>
#include <math.h>

#include <type_traits>

namespace ad {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;   // keys per wave per step
constexpr int kRows = 32;   // query rows per work unit

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

template <int D, int MODE, bool FP8, bool ROWS>
__global__ void __launch_bounds__(kThreads) partial_mfma_kernel(const PartialParams p) {
    static_assert(!(ROWS && FP8), "whole-row loads are built for bf16 caches");
    constexpr int kKs = D / 16;    // k-steps of the score product
    constexpr int kSlabs = D / 32; // 32-column slabs of the output
    constexpr int kRowBytes = D * 2;  // one bf16 row of the LDS V tile
    constexpr int kLoads = FP8 ? kKs / 2 : kKs;  // 16-byte pieces of K (and of V) per lane and key

    const UnitId wu = p.lpt ? decode_unit_lpt<kThreads>(p) : decode_unit(p);
    const int split = wu.split, rb = wu.rb, h = wu.h, b = wu.b;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;
    const int G = p.group, Q = p.q_len, S = p.num_splits, Dv = p.head_dim_v;
    // this sequence's query tokens (fewer than q_len with variable query lengths)
    const QRows qrows = q_rows(p.q_starts, Q, b);
    const int Qb = qrows.n, R = G * Qb;
    const int r0 = rb * kRows, nr = min(kRows, R - r0);
    if (nr <= 0) return;  // uniform: a row block past the sequence's last token
    const int L = p.seq_lens ? p.seq_lens[b] : p.kv_len_max;

    int vlen = L;
    if constexpr (MODE == KV_SPARSE) vlen = p.num_blocks[b * p.nb_s[0] + h * p.nb_s[1]] << p.block_shift;
    const int t0 = split * p.chunk;
    const int t1 = min(t0 + p.chunk, vlen);

    auto out_row = [&](int r) -> int64_t {  // r: row inside the unit
        const int ra = r0 + r, t = ra / G, g = ra - t * G;
        return (int64_t)(b * Q + t) * p.num_q_heads + h * G + g;
    };

    if (t0 >= t1) {  // uniform
        if (p.counters) {  // fused merge: only a unit without keys writes here (out = 0, lse = -inf)
            if (vlen <= 0 && split == 0) fused_write_empty<kThreads, D>(p, nr, out_row);
            return;
        }
        if (p.write_empty) {
            for (int i = tid; i < nr * Dv; i += kThreads) {
                const int r = i / Dv, d = i - r * Dv;
                p.part_o[(out_row(r) * S + split) * Dv + d] = 0.f;
            }
            for (int r = tid; r < nr; r += kThreads) p.part_lse[out_row(r) * S + split] = -INFINITY;
        }
        return;
    }

    __shared__ int s_map[kMapCapacity];
    // Per-wave V tiles (and K tiles, ROWS form) during the loop; per-wave fp32 accumulators for
    // the final combine.
    __shared__ __attribute__((aligned(16))) unsigned char s_buf[kWaves * kRows * D * 4];
    __shared__ __attribute__((aligned(16))) float s_alpha[kWaves][kRows];
    __shared__ float s_m[kWaves][kRows], s_l[kWaves][kRows], s_lf[kWaves][kRows];
    __shared__ float s_fw[kWaves][kRows], s_inv[kRows];  // combine weights of the waves' partials, 1 / l
    // fp8 cache: the scales of a wave's 32 tile keys, read back in the score accumulator's key order
    __shared__ __attribute__((aligned(16))) float s_ks[FP8 ? kWaves : 1][kTile], s_vs[FP8 ? kWaves : 1][kTile];

    const int map_shift = MODE == KV_PAGED ? p.page_shift : p.block_shift;
    const int map_first = (MODE == KV_CONTIG) ? 0 : (t0 >> map_shift);
    if constexpr (MODE == KV_PAGED) {
        const int n = ((t1 - 1) >> map_shift) - map_first + 1;
        const int32_t *bt = p.block_table + b * p.bt_stride + map_first;
        for (int i = tid; i < n; i += kThreads) s_map[i] = bt[i];
    } else if constexpr (MODE == KV_SPARSE) {
        const int n = ((t1 - 1) >> map_shift) - map_first + 1;
        const int32_t *ix = p.block_idx + b * p.ix_s[0] + h * p.ix_s[1];
        for (int i = tid; i < n; i += kThreads) s_map[i] = ix[(int64_t)(map_first + i) * p.ix_s[2]];
    }
    if constexpr (MODE != KV_CONTIG) __syncthreads();
    const int map_mask = (1 << map_shift) - 1;

    // ---- this lane's query row (row col of the unit) as the B operand, and its visible range
    const uint16_t *qbase = static_cast<const uint16_t *>(p.q) +
                            (p.q_starts ? (int64_t)qrows.first * p.q_s[1] : b * p.q_s[0]) +
                            (int64_t)(h * G) * p.q_s[2];
    u32x4 qb[kKs];
    int lo_r = INT_MIN, hi_r = INT_MAX;
    // Tree mask: the last Qb keys are the drafts; this lane's row sees draft i only with bit i of
    // its token's mask row (tm0: drafts 0-31, tm1: 32-63).
    const int first_draft = L - Qb;
    uint32_t tm0 = ~0u, tm1 = ~0u;
    {
        const int ra = r0 + col;
        const int t = ra / G, g = ra - t * G;
        if (col < nr) {
            const uint16_t *qr = qbase + t * p.q_s[1] + g * p.q_s[2];
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks)  // fp8: the head-dim order of the fp8 K operand
                qb[ks] = ld16(qr + (FP8 ? 32 * (ks / 2) + 16 * half + 8 * (ks % 2) : 16 * ks + 8 * half));
            const int qpos = L - Qb + t;
            if (p.causal) hi_r = qpos + 1;
            if (p.window) lo_r = qpos - p.window + 1;
            if (p.tree_mask) {
                const uint32_t *mr = p.tree_mask + (int64_t)(qrows.first + t) * p.mask_words;
                tm0 = mr[0];
                tm1 = p.mask_words > 1 ? mr[1] : 0u;
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) qb[ks] = u32x4{0, 0, 0, 0};
        }
    }
    // Visible range of the unit: keys outside [lo_min, hi_max) are seen by no row; keys inside
    // [lo_max, hi_min) by every row.
    const int t_first = __builtin_amdgcn_readfirstlane(r0 / G);
    const int t_last = __builtin_amdgcn_readfirstlane((r0 + nr - 1) / G);
    // (tree mask: keys from the first draft on are never seen by every row for certain)
    const int hi_min = min(p.causal ? L - Qb + t_first + 1 : INT_MAX, p.tree_mask ? first_draft : INT_MAX);
    const int hi_max = p.causal ? L - Qb + t_last + 1 : INT_MAX;
    const int lo_min = p.window ? L - Qb + t_first - p.window + 1 : INT_MIN;
    const int lo_max = p.window ? L - Qb + t_last - p.window + 1 : INT_MIN;

    // ---- key addressing: virtual key index v (position in the split's key range) -> logical
    // position and row offsets. Only called with v < t1.
    using KV = std::conditional_t<FP8, uint8_t, uint16_t>;  // one K / V element
    const KV *kbase = static_cast<const KV *>(p.k) + (int64_t)h * p.k_s[2];
    const KV *vbase = static_cast<const KV *>(p.v) + (int64_t)h * p.v_s[2];
    const float *ksbase = p.k_scale + (int64_t)h * p.ks_s[2];  // fp8: row scales, indexed like the rows
    const float *vsbase = p.v_scale + (int64_t)h * p.vs_s[2];
    if constexpr (MODE != KV_PAGED) {
        kbase += b * p.k_s[0];
        vbase += b * p.v_s[0];
        if constexpr (FP8) {
            ksbase += b * p.ks_s[0];
            vsbase += b * p.vs_s[0];
        }
    }
    auto logical = [&](int v) -> int {
        if constexpr (MODE == KV_SPARSE) return (s_map[(v >> map_shift) - map_first] << map_shift) + (v & map_mask);
        return v;
    };
    // finite (bf16), always readable, at least D elements; an fp8 cache's bytes read from it may
    // be NaN codes, which never reach the sums (masked scores, zeroed values)
    const KV *safe = reinterpret_cast<const KV *>(qbase);

    struct Buf {
        u32x4 k[kLoads];
        u32x4 v[kLoads];
        float ks, vs;  // fp8: this lane's key scales as loaded (any value for a key that is not read)
        bool live;     // fp8: this lane's key is read
        int base;
    };
    auto fetch = [&](Buf &f, int base) {
        f.base = base;
        const int v = base + col;
        const KV *kp = safe, *vp = safe;
        const float *ksp = p.k_scale, *vsp = p.v_scale;  // the arrays' first scales: always readable
        if (v < t1) {
            if constexpr (MODE == KV_PAGED) {  // logical position = v, and v < t1 <= L
                if (v >= lo_min && v < hi_max) {
                    const int64_t page = s_map[(v >> map_shift) - map_first];
                    const int slot = v & map_mask;
                    kp = kbase + page * p.k_s[0] + slot * p.k_s[1];
                    vp = vbase + page * p.v_s[0] + slot * p.v_s[1];
                    if constexpr (FP8) {
                        ksp = ksbase + page * p.ks_s[0] + slot * p.ks_s[1];
                        vsp = vsbase + page * p.vs_s[0] + slot * p.vs_s[1];
                    }
                }
            } else {
                const int pos = logical(v);
                if (pos < L && pos >= lo_min && pos < hi_max) {
                    kp = kbase + (int64_t)pos * p.k_s[1];
                    vp = vbase + (int64_t)pos * p.v_s[1];
                    if constexpr (FP8) {
                        ksp = ksbase + (int64_t)pos * p.ks_s[1];
                        vsp = vsbase + (int64_t)pos * p.vs_s[1];
                    }
                }
            }
        }
        if constexpr (FP8) {
#pragma unroll
            for (int j = 0; j < kLoads; ++j)
                f.k[j] = j % 4 == 3 ? ld16_last(kp + 32 * j + 16 * half) : ld16(kp + 32 * j + 16 * half);
#pragma unroll
            for (int j = 0; j < kLoads; ++j)
                f.v[j] = j % 4 == 3 ? ld16_last(vp + 32 * j + 16 * half) : ld16(vp + 32 * j + 16 * half);
            // used only once this buffer is current (a select here would wait for the prefetch)
            f.ks = *ksp;
            f.vs = *vsp;
            f.live = kp != safe;
        } else if constexpr (!ROWS) {
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) f.k[ks] = ld16(kp + 16 * ks + 8 * half);
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) f.v[ks] = ld16(vp + 16 * ks + 8 * half);
        }
    };
    // ROWS form: kRowLanes lanes share a row (16 B each), a wave-wide load covers kRowsPerLoad
    // rows and kKs loads the tile's 32 keys, for K and again for V; the rows go to the wave's LDS
    // tiles, from which the matrix cores read K as the A operand and V transposed.
    constexpr int kRowLanes = D * 2 / 16;
    constexpr int kRowsPerLoad = 64 / kRowLanes;
    static_assert(kRowsPerLoad * kKs == kTile, "the loads of a tile cover its keys");
    const int lrow = lane / kRowLanes, lpiece = lane % kRowLanes;  // row within a load, 16-B piece
    // element offsets of the K and V rows of key v from kbase / vbase; ok false: not read
    struct RowOff {
        int64_t k, v;
        bool ok;
    };
    auto rows_of = [&](int v) -> RowOff {
        RowOff r{0, 0, false};
        if (v >= t1) return r;
        if constexpr (MODE == KV_PAGED) {  // logical position = v, and v < t1 <= L
            if (v < lo_min || v >= hi_max) return r;
            const int64_t page = s_map[(v >> map_shift) - map_first];
            const int slot = v & map_mask;
            r.k = page * p.k_s[0] + slot * p.k_s[1];
            r.v = page * p.v_s[0] + slot * p.v_s[1];
        } else {
            const int pos = logical(v);
            if (pos >= L || pos < lo_min || pos >= hi_max) return r;
            r.k = (int64_t)pos * p.k_s[1];
            r.v = (int64_t)pos * p.v_s[1];
        }
        r.ok = true;
        return r;
    };
    auto fetch_rows = [&](Buf &f, int base) {
        f.base = base;
#pragma unroll
        for (int i = 0; i < kKs; ++i) {
            const RowOff r = rows_of(base + kRowsPerLoad * i + lrow);
            const KV *kp = r.ok ? kbase + r.k : safe;
            const KV *vp = r.ok ? vbase + r.v : safe;
            f.k[i] = ld16_stream(kp + 8 * lpiece);
            f.v[i] = ld16_stream(vp + 8 * lpiece);
        }
    };

    lds_u8 *vw = (lds_u8 *)s_buf + wave * kTile * kRowBytes;             // this wave's V tile
    lds_u8 *kw = (lds_u8 *)s_buf + (kWaves + wave) * kTile * kRowBytes;  // and its K tile (ROWS form)
    // Transposing-read addresses (bytes in vw) of this lane, for k-step t, read rd and slab s:
    // row 16t + 8rd + 4*half + (lane&15)/4, chunk 4s + 2*((lane>>4)&1) + (lane&3)/2, half-chunk lane&1.
    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int tr_byte = (lane & 1) << 3;

    float m = -INFINITY, l = 0.f, lf = 0.f;  // row col's running state (this lane's keys)
    f32x16 o[kSlabs];
#pragma unroll
    for (int s = 0; s < kSlabs; ++s)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[s][j] = 0.f;

    auto compute = [&](const Buf &cur, bool full) {
        // V tile -> LDS (row col, chunk 2ks + half); fp8: converted to bf16, chunks 4j + 2*half (+1)
        if constexpr (FP8) {
#pragma unroll
            for (int j = 0; j < kLoads; ++j) {
                u32x4 w = cur.v[j];
                if (!full && !cur.live) w = u32x4{0, 0, 0, 0};  // a key that is not read may hold NaN codes
                const int c0 = 4 * j + 2 * half;
                *(__attribute__((address_space(3))) u32x4 *)(vw + col * kRowBytes + ((c0 ^ swz<D>(col)) << 4)) =
                    e4m3_x8(w[0], w[1]);
                *(__attribute__((address_space(3))) u32x4 *)(vw + col * kRowBytes + (((c0 + 1) ^ swz<D>(col)) << 4)) =
                    e4m3_x8(w[2], w[3]);
            }
            if (half == 0) {  // a key that is not read takes scale 0
                s_ks[wave][col] = cur.live ? cur.ks : 0.f;
                s_vs[wave][col] = cur.live ? cur.vs : 0.f;
            }
        } else if constexpr (ROWS) {  // load i: chunk lpiece of row kRowsPerLoad * i + lrow, K and V
#pragma unroll
            for (int i = 0; i < kKs; ++i) {
                const int kk = kRowsPerLoad * i + lrow;
                const int at = kk * kRowBytes + ((lpiece ^ swz<D>(kk)) << 4);
                *(__attribute__((address_space(3))) u32x4 *)(kw + at) = cur.k[i];
                *(__attribute__((address_space(3))) u32x4 *)(vw + at) = cur.v[i];
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks)
                *(__attribute__((address_space(3))) u32x4 *)(vw + col * kRowBytes + (((2 * ks + half) ^ swz<D>(col)) << 4)) =
                    cur.v[ks];
        }
        // S^T = K Q^T
        f32x16 sc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[j] = 0.f;
        if constexpr (FP8) {
#pragma unroll
            for (int j = 0; j < kLoads; ++j) {
                const u32x4 w = cur.k[j];
                sc = mfma(e4m3_x8(w[0], w[1]), qb[2 * j], sc);
                sc = mfma(e4m3_x8(w[2], w[3]), qb[2 * j + 1], sc);
            }
        } else if constexpr (ROWS) {  // the A operand of k-step ks: row col, chunk 2 ks + half of the K tile
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {
                const u32x4 a = *(__attribute__((address_space(3))) u32x4 *)(kw + col * kRowBytes +
                                                                                (((2 * ks + half) ^ swz<D>(col)) << 4));
                sc = mfma(a, qb[ks], sc);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) sc = mfma(cur.k[ks], qb[ks], sc);
        }
        float sv[16];
        f32x4 vs4[FP8 ? 4 : 1];  // fp8: value scales of this lane's keys 8*q4 + 4*half + e
        if constexpr (FP8) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 k4 = *(const f32x4 *)&s_ks[wave][8 * q4 + 4 * half];
                vs4[q4] = *(const f32x4 *)&s_vs[wave][8 * q4 + 4 * half];
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[4 * q4 + e] = sc[4 * q4 + e] * (p.scale_log2 * k4[e]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) sv[j] = sc[j] * p.scale_log2;
        }
        if (!full) {  // uniform
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int v4 = cur.base + 8 * q4 + 4 * half;  // keys v4 .. v4+3 share a page / block
                const int pos4 = v4 < t1 ? logical(v4) : 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int pos = pos4 + e;
                    bool vis = v4 + e < t1 && pos < L && pos >= lo_r && pos < hi_r;
                    if (p.tree_mask && vis && pos >= first_draft) {
                        const int i = pos - first_draft;  // < Qb <= 64: a visible key lies below L
                        vis = ((i < 32 ? tm0 : tm1) >> (i & 31)) & 1u;
                    }
                    sv[4 * q4 + e] = vis ? sv[4 * q4 + e] : -INFINITY;
                }
            }
        }
        float mx = sv[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sv[j]);
        mx = pair_max(mx);
        const bool raise = mx > m + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform
            // Rows that do not move keep factor 1 exactly (exp2(m - m) is NaN while m = -inf).
            const float alpha = raise ? exp2_fast(m - mx) : 1.f;
            m = raise ? mx : m;
            l *= alpha;
            lf *= alpha;
            if (half == 0) s_alpha[wave][col] = alpha;
            // output rows of this lane: 8*(j/4) + 4*half + j%4
            f32x4 a4[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) a4[q4] = *(const f32x4 *)&s_alpha[wave][8 * q4 + 4 * half];
#pragma unroll
            for (int s = 0; s < kSlabs; ++s)
#pragma unroll
                for (int j = 0; j < 16; ++j) o[s][j] *= a4[j / 4][j % 4];
        }
        const float ms = (m == -INFINITY) ? 0.f : m;
        uint32_t pk[8];
        const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p0 = exp2_fast(sv[2 * i] - ms), p1 = exp2_fast(sv[2 * i + 1] - ms);  // exp2(-inf) = 0
            if constexpr (FP8) {  // value scales into P; normaliser from the rounded products / scales
                const float vs0 = vs4[i / 2][(2 * i) % 4], vs1 = vs4[i / 2][(2 * i + 1) % 4];
                pk[i] = pack_bf16(p0 * vs0, p1 * vs1);
                const float r0 = __uint_as_float(pk[i] << 16), r1 = __uint_as_float(pk[i] & 0xFFFF0000u);
                l += (vs0 != 0.f ? r0 * __builtin_amdgcn_rcpf(vs0) : p0) +
                     (vs1 != 0.f ? r1 * __builtin_amdgcn_rcpf(vs1) : p1);
            } else {
                pk[i] = pack_bf16(p0, p1);
                l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]), ones, l, false);
            }
            lf += p0 + p1;
        }
        // O += P V over the tile's two 16-key k-steps
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const u32x4 pa = u32x4{pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]};
#pragma unroll
            for (int s = 0; s < kSlabs; ++s) {
                s16x4 part[2];
#pragma unroll
                for (int rd = 0; rd < 2; ++rd) {
                    const int row = 16 * t + 8 * rd + tr_row;
                    const int chunk = 4 * s + tr_chunk;
                    part[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4 *)(vw + row * kRowBytes +
                                                                    ((chunk ^ swz<D>(row)) << 4) + tr_byte));
                }
                const s16x8 vb = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
                o[s] = mfma(pa, __builtin_bit_cast(u32x4, vb), o[s]);
            }
        }
    };

    constexpr int kStride = kWaves * kTile;
    auto prefetch = [&](Buf &f, int base) {
        if constexpr (ROWS)
            fetch_rows(f, base);
        else
            fetch(f, base);
    };
    auto iterate = [&](Buf &cur, Buf &nxt) {
        prefetch(nxt, cur.base + kStride);
        __builtin_amdgcn_sched_barrier(0);
        bool full = cur.base + kTile <= t1;
        if (full) {
            const int pf = logical(cur.base), pl = logical(cur.base + kTile - 1);
            full = pl - pf == kTile - 1 && pl < L && pf >= lo_max && pl < hi_min;
        }
        compute(cur, full);
    };

    // This wave's tiles start at first + i * kStride < t1. The loop runs pairs of tiles with its
    // only exit test at the back edge, so the loads in flight are the same on every path into the
    // loop and the compiler waits for no more of them than a tile needs (an exit test between the
    // two halves made it wait for every load at the loop head); an odd last tile follows the loop.
    const int first = t0 + wave * kTile;
    const int ntiles = first < t1 ? (t1 - first + kStride - 1) / kStride : 0;
    Buf A, B;
    prefetch(A, first);
    int i = 0;
    for (; i + 2 <= ntiles; i += 2) {
        iterate(A, B);
        iterate(B, A);
    }
    if (i < ntiles) iterate(A, B);

    // ---- combine the waves: o_s = acc / l, lse_s = (m + log2 lf) * ln 2
    l = pair_sum(l);
    lf = pair_sum(lf);
    __syncthreads();  // every wave is done with its tiles: s_buf now holds the accumulators
    float *s_o = reinterpret_cast<float *>(s_buf) + wave * kRows * D;
    if (half == 0) {
        s_m[wave][col] = m;
        s_l[wave][col] = l;
        s_lf[wave][col] = lf;
    }
#pragma unroll
    for (int s = 0; s < kSlabs; ++s)
#pragma unroll
        for (int j = 0; j < 16; ++j) s_o[(8 * (j / 4) + 4 * half + (j % 4)) * D + 32 * s + col] = o[s][j];
    __syncthreads();

    // Per-row factors, once per row: the weight of each wave's partial and 1 / l. Stores are
    // agent-scope: a merging group on another XCD reads them (fused merge).
    if (tid < nr) {
        const int r = tid;
        float M = s_m[0][r];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][r]);
        const float ms = (M == -INFINITY) ? 0.f : M;
        float lsum = 0.f, lfsum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = exp2_fast(s_m[w][r] - ms);
            s_fw[w][r] = f;
            lsum += s_l[w][r] * f;
            lfsum += s_lf[w][r] * f;
        }
        s_inv[r] = lsum > 0.f ? 1.f / lsum : 0.f;
        store_partial(p.part_lse + out_row(r) * S + split,
                      lsum > 0.f ? (ms + __builtin_amdgcn_logf(lfsum)) * 0.69314718055994531f : -INFINITY);
    }
    __syncthreads();
    const float *s_all = reinterpret_cast<const float *>(s_buf);
    for (int i = tid; i < nr * D; i += kThreads) {
        const int r = i / D, d = i - r * D;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) acc += s_all[(w * kRows + r) * D + d] * s_fw[w][r];
        store_partial(p.part_o + (out_row(r) * S + split) * Dv + d, acc * s_inv[r]);
    }
    if (p.counters) {  // one launch per step: the unit's last split merges (s_buf is free now)
        const int nsplit = min(S, (vlen + p.chunk - 1) / p.chunk);
        constexpr int kPerThread = (kRows * D + kThreads - 1) / kThreads;
        fused_arrive_merge<kThreads, D, kPerThread>(p, wu.unit, nsplit, nr, out_row,
                                                 reinterpret_cast<float *>(s_buf));
    }
}

template <int D, int MODE, bool FP8>
hipError_t launch_t(const PartialParams &p, hipStream_t stream) {
    const dim3 grid(p.num_splits * p.batch * p.num_kv_heads * p.row_blocks);  // see decode_unit
    if constexpr (!FP8)
        if (p.mfma_rows) {
            hipLaunchKernelGGL((partial_mfma_kernel<D, MODE, false, true>), grid, dim3(kThreads), 0, stream, p);
            return hipGetLastError();
        }
    hipLaunchKernelGGL((partial_mfma_kernel<D, MODE, FP8, false>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool FP8 = false>
hipError_t by_mode(const PartialParams &p, int mode, hipStream_t s) {
    switch (mode) {
        case KV_CONTIG: return launch_t<D, KV_CONTIG, FP8>(p, s);
        case KV_PAGED: return launch_t<D, KV_PAGED, FP8>(p, s);
        default: return launch_t<D, KV_SPARSE, FP8>(p, s);
    }
}

}  // namespace

hipError_t launch_partial_mfma(const PartialParams &p, int head_dim, int mode, hipStream_t stream) {
    if (p.kv_int4) return hipErrorInvalidValue;  // int4 caches run on the vector kernel only
    if (p.kv_fp8) {  // the host admits an fp8 cache with head dim 128 only
        if (head_dim != 128) return hipErrorInvalidValue;
        return by_mode<128, true>(p, mode, stream);
    }
    return head_dim == 64 ? by_mode<64>(p, mode, stream) : by_mode<128>(p, mode, stream);
}

}  // namespace ad
