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
// Why VALU and not MFMA: with at most 8 rows per KV head a key costs 256-512 B of K/V and ~4
// flop/B; the step is bound by HBM and by VALU issue, and MFMA would add operand transposes of V.
// The kernel is built to keep HBM busy with as few VALU instructions per key as possible:
//
//   * LPT lanes share one K/V row; each lane loads 16-byte pieces, so one wave-wide load covers
//     64/LPT rows x 16*LPT contiguous bytes (whole cache lines). The lanes of a row reduce their
//     partial dot products with DPP adds (quad_perm 1032, quad_perm 2301, row_half_mirror,
//     row_mirror).
//   * Each row-slot of a wave runs its own online softmax over the keys it loads, so the hot
//     loop has no cross-slot traffic; slots and waves are combined once, at the end.
//   * A step is 64/LPT * U consecutive keys (<= 16), so it never straddles a page of the paged
//     cache or a listed block of the block-sparse cache: the page / block id is one LDS read per
//     step, and the step's keys are one contiguous run.
//   * Prefetch depth one step: the K and V loads of step i+1 are issued before step i's
//     arithmetic; two register buffers alternate (loop unrolled by two) so no register moves are
//     needed, and a scheduling fence keeps the loads where they are issued.
//   * Steps wholly inside the visible range (every key in the split, inside the sequence, not
//     cut by causal or window bounds) skip all masking; only boundary steps evaluate masks.
//   * Lazy rescaling: the running max of a row is only raised when a score exceeds it by more
//     than 2^8, so the accumulator rescale is rare; probabilities stay <= 256, the result is the
//     same softmax with a different (exactly cancelled) reference point.
//   * bf16: scores use v_dot2 on bf16 pairs (q stays exact, scale applied to the fp32 dot); P is
//     rounded to bf16 and P.V uses v_dot2 over key pairs (V words re-paired with v_perm), with
//     the row sum taken from the same rounded P, as the xqa (TensorRT-LLM mha.cu, toFp16 /
//     computeRowSum) and FlashInfer (mla.cuh compute_mla_pv) kernels do. fp32 keeps P in fp32.
//   * Masked keys are never read: their loads are redirected to the unit's own query row (always
//     valid, finite memory) and their probability is exactly 0, so NaN/Inf in unused cache slots
//     cannot leak into the result.
#include "ad_internal.h"
#include "fused_merge.h"

#include <limits.h>
#include <math.h>

#include <type_traits>

namespace ad {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLazyRescale = 8.f;  // log2 units

// Tuning: lanes that share one K/V row (4, 8 or 16; capped at row bytes / 16) and keys each
// row-slot loads per step (even for bf16).
#ifndef AD_VALU_LANES_PER_ROW
#define AD_VALU_LANES_PER_ROW 8
#endif
#ifndef AD_VALU_KEYS_PER_SLOT
#define AD_VALU_KEYS_PER_SLOT 2
#endif


template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPT consecutive lanes of a row-slot; every lane of the slot gets the total.
template <int LPT>
__device__ __forceinline__ float slot_sum(float x) {
    x += dpp<0xB1>(x);                            // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);                            // quad_perm [2,3,0,1]
    if constexpr (LPT >= 8) x += dpp<0x141>(x);   // row_half_mirror: the other quad of the 8
    if constexpr (LPT >= 16) x += dpp<0x140>(x);  // row_mirror: the other half of the 16
    return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Every 16-B load of this kernel is nontemporal: the 8 lanes sharing a row read whole 128-B lines
// in one instruction and nothing is read twice, so the lines need not stay in the caches
// (measured: 224 -> 205 us on the ragged paged cache of 64 sequences, 56.7 -> 52.7 us on the
// contiguous 16 x 4096 cache).
__device__ __forceinline__ u32x4 ld16(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Reinterpretations take the 32-bit word BY VALUE: hipcc miscompiles __builtin_bit_cast applied
// directly to an element of an ext_vector_type lvalue (it reads the wrong element), so vector
// elements always pass through a plain uint32_t first.
__device__ __forceinline__ float as_f32(uint32_t w) { return __uint_as_float(w); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }
__device__ __forceinline__ bf16x2 pack_bf16(float lo, float hi) {  // round to nearest even
    bf16x2 r;
    r.x = (__bf16)lo;
    r.y = (__bf16)hi;
    return r;
}
__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}
// Two OCP E4M3 bytes of w (bytes 0-1, or 2-3 with HI) as a bf16 pair, exactly (every E4M3 value
// is a bf16 value; the conversion's own scale is 1).
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3_pair(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}

// FP8: k and v hold OCP E4M3 bytes with fp32 row scales (bf16 queries); K / V elements are then
// bytes, each lane still owns 16 of a row, and its query values for them are two 16-B words.
// INT4: k and v hold rows of 32-bit words, kv_groups coefficient words (fp16 scale s low, fp16
// shift m high) and then D / 8 words of 4-bit fields f (field d % 8 of word d / 8); 16 lanes share
// a row and each owns 8 consecutive dimensions, all in one group (one value word and the group's
// coefficient word), so that a wave-wide load covers 4 keys and a step 16.
// q.k over them is s * sum q (128 + f) + (m - 128 s) * sum q: the fields become bf16 pairs
// 128 + f by masking in an exponent (exact), multiplied with v_dot2 against the queries paired
// the same way, and the per-row query sums fix the offset in fp32. P.V keeps P unrounded:
// acc += (p s) f in fp32 with f converted from bytes, and p m is summed once per row and added
// at the end.
template <typename T, int D, int RP, int MODE, int U, int LPT, bool FP8, bool INT4>
__device__ __forceinline__ void partial_valu_body(const PartialParams &p) {
    constexpr bool kBf16 = sizeof(T) == 2;
    static_assert(!(FP8 || INT4) || kBf16, "a quantised cache is read with bf16 queries");
    static_assert(!INT4 || (D == 128 && (LPT == 8 || LPT == 16)), "the int4 lane map: 8 or 16 lanes per row");
    using KV = std::conditional_t<FP8, uint8_t, std::conditional_t<INT4, uint32_t, T>>;  // one K / V element
    constexpr int kPer16 = INT4 ? D / LPT : 16 / (int)sizeof(KV);  // K / V elements per 16-B piece (int4: per lane)
    constexpr int kIW = INT4 ? D / (8 * LPT) : 1;                 // int4: packed value words per lane
    constexpr int kSlots = 64 / LPT;                           // rows per wave-wide load
    constexpr int kPieces = INT4 ? 1 : D * (int)sizeof(KV) / (16 * LPT);  // 16-B pieces per lane per row
    constexpr int kEPL = kPieces * kPer16;                     // elements per lane per row
    constexpr int kQv = FP8 ? 2 * kPieces : INT4 ? kPer16 / 8 : kPieces;  // 16-B query words per lane per row
    constexpr int kStep = kSlots * U;                         // keys per wave per step
    static_assert(kPieces >= 1, "row too short for the lanes sharing it");
    static_assert(MODE == KV_CONTIG || (kStep <= 16 && 16 % kStep == 0),
                  "a step must stay inside one page / listed block (both are >= 16 keys)");
    static_assert(!kBf16 || INT4 || U % 2 == 0, "bf16 P.V pairs keys");

    const UnitId wu = p.lpt ? decode_unit_lpt<kThreads>(p) : decode_unit(p);
    const int split = wu.split, rb = wu.rb, h = wu.h, b = wu.b;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps step bases scalar
    const int slot = lane / LPT, c = lane % LPT;
    const int G = p.group, Q = p.q_len, S = p.num_splits, Dv = p.head_dim_v;
    // this sequence's query tokens (fewer than q_len with variable query lengths)
    const QRows qr = q_rows(p.q_starts, Q, b);
    const int Qb = qr.n, R = G * Qb;
    const int r0 = rb * RP, nr = min(RP, R - r0);  // this unit's rows: r0 .. r0 + nr - 1
    if (nr <= 0) return;  // uniform: a row block past the sequence's last token
    const int L = p.seq_lens ? p.seq_lens[b] : p.kv_len_max;

    int vlen = L;  // length of the key range the splits partition
    if constexpr (MODE == KV_SPARSE) {
        const int nb = p.num_blocks[b * p.nb_s[0] + h * p.nb_s[1]];
        vlen = nb << p.block_shift;
    }
    const int t0 = split * p.chunk;
    const int t1 = min(t0 + p.chunk, vlen);

    auto out_row = [&](int r) -> int64_t {  // r: row inside the unit
        const int ra = r0 + r, t = ra / G, g = ra - t * G;
        return (int64_t)(b * Q + t) * p.num_q_heads + h * G + g;
    };

    if (t0 >= t1) {  // uniform over the work group
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
    __shared__ float s_acc[kWaves][RP][D];
    __shared__ float s_m[kWaves][RP];
    __shared__ float s_l[kWaves][RP];
    __shared__ float s_lf[kWaves][RP];
    __shared__ uint32_t s_tree[RP][2];  // tree mask words of each row's token

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

    // ---- query rows of this unit: row r0 + r = t*G + g (hq = h*G + g)
    const T *qbase = static_cast<const T *>(p.q) + (p.q_starts ? (int64_t)qr.first * p.q_s[1] : b * p.q_s[0]) +
                     (int64_t)(h * G) * p.q_s[2];
    // Tree mask: the last Qb keys are the drafts; a row sees draft i only with bit i of its token's
    // mask row. Steps that reach the drafts take the masked path.
    const int first_draft = L - Qb;
    if (p.tree_mask) {
        if (tid < RP * 2) {
            const int r = tid >> 1, w = tid & 1;
            const int t = (r0 + min(r, nr - 1)) / G;
            s_tree[r][w] = w < p.mask_words ? p.tree_mask[(int64_t)(qr.first + t) * p.mask_words + w] : 0u;
        }
        __syncthreads();
    }
    u32x4 qv[RP][kQv];
    int lo[RP], hi[RP];  // visible key positions of row r: [lo, hi)
    int lo_max = INT_MIN, hi_min = p.tree_mask ? first_draft : INT_MAX;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        const int ra = r0 + r, t = ra / G, g = ra - t * G;
        const int qpos = L - Qb + t;
        hi[r] = p.causal ? qpos + 1 : INT_MAX;
        lo[r] = p.window ? qpos - p.window + 1 : INT_MIN;
        if (r < nr) {
            hi_min = min(hi_min, hi[r]);
            lo_max = max(lo_max, lo[r]);
        }
        const T *qr = qbase + t * p.q_s[1] + g * p.q_s[2];
#pragma unroll
        for (int i = 0; i < kQv; ++i) qv[r][i] = u32x4{0, 0, 0, 0};
        if (r < nr) {
#pragma unroll
            for (int i = 0; i < kPieces; ++i) {
                const T *src = qr + (i * LPT + c) * kPer16;  // the lane's elements of piece i
                if constexpr (FP8) {
                    qv[r][2 * i] = ld16(src);
                    qv[r][2 * i + 1] = ld16(src + 8);
                } else if constexpr (INT4) {
#pragma unroll
                    for (int qi = 0; qi < kQv; ++qi) qv[r][qi] = ld16(src + 8 * qi);
                } else {
                    qv[r][i] = ld16(src);
                }
            }
        }
    }
    // int4: the lane's query values as pairs (dim 8w + j, dim 8w + j + 4), the order in which the
    // fields of its packed word w come out two at a time, and their fp32 sum
    bf16x2 qp[INT4 ? RP : 1][INT4 ? 4 * kIW : 1];
    float qsum[INT4 ? RP : 1];
    if constexpr (INT4) {
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            qsum[r] = 0.f;
#pragma unroll
            for (int w = 0; w < kIW; ++w)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t a = qv[r][w][j / 2], b = qv[r][w][2 + j / 2];  // dims j and j + 4
                    const uint32_t pr = j % 2 ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
                    qp[r][4 * w + j] = as_bf16x2(pr);
                    qsum[r] += __uint_as_float(pr << 16) + __uint_as_float(pr & 0xFFFF0000u);
                }
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

    const Int4Consts i4k = [] {
        if constexpr (INT4) return int4_consts();
        else return Int4Consts{0u, 0u};
    }();

    // ---- key addressing
    const KV *kbase = static_cast<const KV *>(p.k) + (int64_t)h * p.k_s[2];
    const KV *vbase = static_cast<const KV *>(p.v) + (int64_t)h * p.v_s[2];
    // row scales of an fp8 cache, indexed like the rows
    const float *ksbase = p.k_scale + (int64_t)h * p.ks_s[2];
    const float *vsbase = p.v_scale + (int64_t)h * p.vs_s[2];
    if constexpr (MODE != KV_PAGED) {
        kbase += b * p.k_s[0];
        vbase += b * p.v_s[0];
        if constexpr (FP8) {
            ksbase += b * p.ks_s[0];
            vsbase += b * p.vs_s[0];
        }
    }
    // an always-readable row for lanes whose key is not visible (the unit's own query row; for
    // an fp8 cache its bytes may decode to NaN, which the arithmetic keeps away from the sums)
    const KV *safe = reinterpret_cast<const KV *>(qbase);
    const int map_mask = (1 << map_shift) - 1;
    const int lane_piece = c * kPer16;
    // int4: this lane's value words and its group's coefficient word inside a row (a query row
    // read instead is 64 words long, more than the largest offset, 8 + 15)
    const int i4_vals = INT4 ? p.kv_groups + kIW * c : 0;
    const int i4_coef = INT4 ? (kPer16 * c) * p.kv_groups / D : 0;

    // l: row sum of the probabilities as multiplied into acc (the rounded P for bf16), the output
    // normaliser; lf: the same sum in full fp32, which gives the LSE.
    // int4: pm = sum of p * shift of the lane's group, added to every accumulator at the end
    float m[RP], l[RP], lf[RP], acc[RP][kEPL], pm[INT4 ? RP : 1];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
        lf[r] = 0.f;
        if constexpr (INT4) pm[r] = 0.f;
#pragma unroll
        for (int e = 0; e < kEPL; ++e) acc[r][e] = 0.f;
    }

    // One step's K and V registers and the facts about its keys.
    struct Buf {
        u32x4 k[U][kPieces];
        u32x4 v[U][kPieces];
        float ks[U], vs[U];  // fp8 cache: the keys' row scales as loaded (used only where val[u])
        bool val[U];
        int base, pos0;
    };

    auto fetch = [&](Buf &f, int base) {
        f.base = base;
        int pos0 = base;
        const KV *krow = kbase;
        const KV *vrow = vbase;
        const float *ksrow = ksbase, *vsrow = vsbase;
        const bool live = base < t1;  // uniform; a step past the end reads the safe row only
        if (live) {
            if constexpr (MODE == KV_PAGED) {
                const int64_t page = __builtin_amdgcn_readfirstlane(s_map[(base >> map_shift) - map_first]);
                const int slot0 = base & map_mask;
                krow = kbase + page * p.k_s[0] + slot0 * p.k_s[1];
                vrow = vbase + page * p.v_s[0] + slot0 * p.v_s[1];
                if constexpr (FP8) {
                    ksrow = ksbase + page * p.ks_s[0] + slot0 * p.ks_s[1];
                    vsrow = vsbase + page * p.vs_s[0] + slot0 * p.vs_s[1];
                }
            } else {
                if constexpr (MODE == KV_SPARSE)
                    pos0 = (__builtin_amdgcn_readfirstlane(s_map[(base >> map_shift) - map_first]) << map_shift) +
                           (base & map_mask);
                krow = kbase + (int64_t)pos0 * p.k_s[1];
                vrow = vbase + (int64_t)pos0 * p.v_s[1];
                if constexpr (FP8) {
                    ksrow = ksbase + (int64_t)pos0 * p.ks_s[1];
                    vsrow = vsbase + (int64_t)pos0 * p.vs_s[1];
                }
            }
        }
        f.pos0 = pos0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int off = u * kSlots + slot;  // key offset inside the step
            bool valid = live && base + off < t1;
            if constexpr (MODE == KV_SPARSE) valid = valid && pos0 + off < L;
            const KV *kp = valid ? krow + off * p.k_s[1] : safe;
            const KV *vp = valid ? vrow + off * p.v_s[1] : safe;
            if constexpr (FP8) {
                // A key that is not read loads the array's first scale (always inside the array,
                // though it may belong to an unused row and hold anything); the arithmetic gives it
                // scale 0 once this buffer is current (a select here would wait for the prefetch).
                f.ks[u] = *(valid ? ksrow + off * p.ks_s[1] : p.k_scale);
                f.vs[u] = *(valid ? vsrow + off * p.vs_s[1] : p.v_scale);
            }
            f.val[u] = valid;
            if constexpr (INT4) {  // dword loads: int4 rows are only 4-byte aligned; coefficient in .z
                f.k[u][0] = u32x4{kp[i4_vals], kIW > 1 ? kp[i4_vals + 1] : 0u, kp[i4_coef], 0u};
                f.v[u][0] = u32x4{vp[i4_vals], kIW > 1 ? vp[i4_vals + 1] : 0u, vp[i4_coef], 0u};
            } else {
#pragma unroll
                for (int i = 0; i < kPieces; ++i) f.k[u][i] = ld16(kp + i * LPT * kPer16 + lane_piece);
#pragma unroll
                for (int i = 0; i < kPieces; ++i) f.v[u][i] = ld16(vp + i * LPT * kPer16 + lane_piece);
            }
        }
    };

    // int4: scale and shift of a coefficient word (w.z of a lane's loaded words)
    auto int4_coef = [](uint32_t cw, float &sc, float &sh) {
        sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(cw & 0xFFFFu));
        sh = (float)__builtin_bit_cast(_Float16, (uint16_t)(cw >> 16));
    };

    // Arithmetic of one step on its loaded K and V.
    auto compute = [&](const Buf &cur, auto masked_tag) {
        constexpr bool kMasked = decltype(masked_tag)::value;
        float sc[U][RP];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // int4 cache: the key's fields as bf16 pairs 128 + f (dims 8w + j, 8w + j + 4), once per key
            bf16x2 kf[INT4 ? 4 * kIW : 1];
            float ksc = 0.f, koff = 0.f;  // s and m - 128 s of the lane's group
            if constexpr (INT4) {
#pragma unroll
                for (int w = 0; w < kIW; ++w)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        kf[4 * w + j] = as_bf16x2(((cur.k[u][0][w] >> (4 * j)) & i4k.mask) | i4k.bits);
                float sh;
                int4_coef(cur.k[u][0][2], ksc, sh);
                koff = fmaf(-128.f, ksc, sh);
            }
            bf16x2 kp8[FP8 ? kPieces : 1][8];  // fp8 cache: the keys' bytes as bf16 pairs, once per key
            if constexpr (FP8) {
#pragma unroll
                for (int i = 0; i < kPieces; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t w = cur.k[u][i][j];
                        kp8[i][2 * j] = e4m3_pair<false>(w);
                        kp8[i][2 * j + 1] = e4m3_pair<true>(w);
                    }
            }
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                float d = 0.f;
                if constexpr (FP8) {
#pragma unroll
                    for (int i = 0; i < kPieces; ++i)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            d = dot2(as_bf16x2(qv[r][2 * i + e / 4][e % 4]), kp8[i][e], d);
                } else if constexpr (INT4) {
#pragma unroll
                    for (int i = 0; i < 4 * kIW; ++i) d = dot2(qp[r][i], kf[i], d);
                    d = fmaf(ksc, d, koff * qsum[r]);
                } else if constexpr (kBf16) {
#pragma unroll
                    for (int i = 0; i < kPieces; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) d = dot2(as_bf16x2(qv[r][i][j]), as_bf16x2(cur.k[u][i][j]), d);
                } else {
#pragma unroll
                    for (int i = 0; i < kPieces; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) d += qf[r][i * 4 + j] * as_f32(cur.k[u][i][j]);
                }
                d = slot_sum<LPT>(d);
                if constexpr (FP8)
                    d *= p.scale_log2 * (cur.val[u] ? cur.ks[u] : 0.f);
                else if constexpr (kBf16)
                    d *= p.scale_log2;
                if constexpr (kMasked) {
                    const int pos = cur.pos0 + u * kSlots + slot;
                    bool vis = cur.val[u] && pos >= lo[r] && pos < hi[r];
                    if (p.tree_mask && vis && pos >= first_draft) {
                        const int i = pos - first_draft;  // < Qb <= 64: a visible key lies below L
                        vis = (s_tree[r][i >> 5] >> (i & 31)) & 1u;
                    }
                    d = vis ? d : -INFINITY;
                }
                sc[u][r] = d;
            }
        }
        // lazy running max: raise a row's reference only when a score clears it by > 2^8
        bool need = false;
        float mx[RP];
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            mx[r] = sc[0][r];
#pragma unroll
            for (int u = 1; u < U; ++u) mx[r] = fmaxf(mx[r], sc[u][r]);
            need = need || (mx[r] > m[r] + kLazyRescale);
        }
        if (__builtin_amdgcn_ballot_w64(need) != 0) {  // wave-uniform
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                // A row (or slot) that does not need it keeps factor 1 exactly: exp2(m - m) would be
                // NaN while m is still -inf. A raised row starting from -inf gets exp2(-inf) = 0.
                const bool raise = mx[r] > m[r] + kLazyRescale;
                const float alpha = raise ? exp2_fast(m[r] - mx[r]) : 1.f;
                m[r] = raise ? mx[r] : m[r];
                l[r] *= alpha;
                lf[r] *= alpha;
                if constexpr (INT4) pm[r] *= alpha;
#pragma unroll
                for (int e = 0; e < kEPL; ++e) acc[r][e] *= alpha;
            }
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const float ms = (m[r] == -INFINITY) ? 0.f : m[r];  // m = -inf only while every score is -inf
#pragma unroll
            for (int u = 0; u < U; ++u) sc[u][r] = exp2_fast(sc[u][r] - ms);  // exp2(-inf) = 0
        }
        if constexpr (FP8) {
            // P.V over key pairs (u, u+1): each key's V scale goes into its probability before the
            // bf16 rounding, and the normaliser sums the rounded products divided by their scales
            // again, so that a row's weights sum exactly as they are multiplied into acc (as the
            // bf16 path sums its rounded P); a zero scale contributes its probability itself. The
            // LSE keeps the fp32 sum of the unrounded probabilities.
#pragma unroll
            for (int u = 0; u < U; u += 2) {
                const float vs0 = cur.val[u] ? cur.vs[u] : 0.f, vs1 = cur.val[u + 1] ? cur.vs[u + 1] : 0.f;
                const float inv0 = __builtin_amdgcn_rcpf(vs0), inv1 = __builtin_amdgcn_rcpf(vs1);
                bf16x2 pk[RP];
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    pk[r] = pack_bf16(sc[u][r] * vs0, sc[u + 1][r] * vs1);
                    const uint32_t w = __builtin_bit_cast(uint32_t, pk[r]);
                    const float r0 = __uint_as_float(w << 16), r1 = __uint_as_float(w & 0xFFFF0000u);
                    l[r] += (vs0 != 0.f ? r0 * inv0 : sc[u][r]) + (vs1 != 0.f ? r1 * inv1 : sc[u + 1][r]);
                    lf[r] += sc[u][r] + sc[u + 1][r];
                }
#pragma unroll
                for (int i = 0; i < kPieces; ++i) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        uint32_t w0 = cur.v[u][i][j], w1 = cur.v[u + 1][i][j];  // elements 4j..4j+3
                        if constexpr (kMasked) {  // a key that was not read may hold NaN codes: 0 * NaN
                            w0 = cur.val[u] ? w0 : 0u;
                            w1 = cur.val[u + 1] ? w1 : 0u;
                        }
                        // bytes interleaved by key: (u[4j], u1[4j], u[4j+1], u1[4j+1]), then 4j+2, 4j+3
                        const uint32_t a = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
                        const uint32_t bq = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
                        const bf16x2 v0 = e4m3_pair<false>(a), v1 = e4m3_pair<true>(a);
                        const bf16x2 v2 = e4m3_pair<false>(bq), v3 = e4m3_pair<true>(bq);
#pragma unroll
                        for (int r = 0; r < RP; ++r) {
                            float *o = &acc[r][i * 16 + 4 * j];
                            o[0] = dot2(pk[r], v0, o[0]);
                            o[1] = dot2(pk[r], v1, o[1]);
                            o[2] = dot2(pk[r], v2, o[2]);
                            o[3] = dot2(pk[r], v3, o[3]);
                        }
                    }
                }
            }
        } else if constexpr (INT4) {
            // fp32 P.V with the unrounded P: acc += (p s) f and pm += p m; a key that was not read
            // has all its words zeroed (scale and shift 0) so that the row it read stays out
#pragma unroll
            for (int u = 0; u < U; ++u) {
                u32x4 w = cur.v[u][0];
                if constexpr (kMasked) w = cur.val[u] ? w : u32x4{0u, 0u, 0u, 0u};
                float f[kEPL];  // fields of dims 8w + 2k (low nibble of byte k) and 8w + 2k + 1 (high)
#pragma unroll
                for (int ww = 0; ww < kIW; ++ww) {
                    const uint32_t lo = w[ww] & 0x0F0F0F0Fu, hi = (w[ww] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        f[8 * ww + 2 * k] = (float)((lo >> (8 * k)) & 0xFFu);
                        f[8 * ww + 2 * k + 1] = (float)((hi >> (8 * k)) & 0xFFu);
                    }
                }
                float vsc, vsh;
                int4_coef(w[2], vsc, vsh);
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    const float pr = sc[u][r], ps = pr * vsc;
                    l[r] += pr;
                    lf[r] += pr;
                    pm[r] = fmaf(pr, vsh, pm[r]);
#pragma unroll
                    for (int e = 0; e < kEPL; ++e) acc[r][e] = fmaf(ps, f[e], acc[r][e]);
                }
            }
        } else if constexpr (kBf16) {
            const bf16x2 ones = as_bf16x2(0x3F803F80u);
#pragma unroll
            for (int u = 0; u < U; u += 2) {
                bf16x2 pk[RP];
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    pk[r] = pack_bf16(sc[u][r], sc[u + 1][r]);
                    l[r] = dot2(pk[r], ones, l[r]);  // row sum of the rounded P
                    lf[r] += sc[u][r] + sc[u + 1][r];
                }
#pragma unroll
                for (int i = 0; i < kPieces; ++i) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t w0 = cur.v[u][i][j], w1 = cur.v[u + 1][i][j];
                        const bf16x2 vlo = as_bf16x2(__builtin_amdgcn_perm(w1, w0, 0x05040100u));
                        const bf16x2 vhi = as_bf16x2(__builtin_amdgcn_perm(w1, w0, 0x07060302u));
#pragma unroll
                        for (int r = 0; r < RP; ++r) {
                            acc[r][i * 8 + 2 * j] = dot2(pk[r], vlo, acc[r][i * 8 + 2 * j]);
                            acc[r][i * 8 + 2 * j + 1] = dot2(pk[r], vhi, acc[r][i * 8 + 2 * j + 1]);
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int r = 0; r < RP; ++r) l[r] += sc[u][r];
#pragma unroll
                for (int i = 0; i < kPieces; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float vf = as_f32(cur.v[u][i][j]);
#pragma unroll
                        for (int r = 0; r < RP; ++r) acc[r][i * 4 + j] += sc[u][r] * vf;
                    }
            }
        }
    };

    const int stride = kWaves * kStep;
    // One step: issue K and V of step i+1, then the arithmetic of step i (whose loads were issued
    // one step earlier). Returns false past the end.
    auto iterate = [&](Buf &cur, Buf &nxt) -> bool {
        if (cur.base >= t1) return false;
        fetch(nxt, cur.base + stride);
        // Keep the issue here: the register-pressure scheduler would otherwise sink the loads below
        // the arithmetic, and every step would wait a full memory round trip.
        __builtin_amdgcn_sched_barrier(0);
        const bool full = cur.base + kStep <= t1 && cur.pos0 >= lo_max && cur.pos0 + kStep <= hi_min &&
                          (MODE != KV_SPARSE || cur.pos0 + kStep <= L);
        if (full)
            compute(cur, std::integral_constant<bool, false>{});
        else
            compute(cur, std::integral_constant<bool, true>{});
        return true;
    };

    Buf A, B;
    fetch(A, t0 + wave * kStep);
    while (iterate(A, B) && iterate(B, A)) {
    }

    if constexpr (INT4) {  // the shifts' share of the lane's accumulators
#pragma unroll
        for (int r = 0; r < RP; ++r)
#pragma unroll
            for (int e = 0; e < kEPL; ++e) acc[r][e] += pm[r];
    }
    // ---- combine the row-slots of the wave (lanes c, c+LPT, ...)
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const float mo = __shfl_xor(m[r], off);
            const float lo_ = __shfl_xor(l[r], off);
            const float lfo = kBf16 ? __shfl_xor(lf[r], off) : 0.f;
            const float mn = fmaxf(m[r], mo);
            const float ms = (mn == -INFINITY) ? 0.f : mn;
            const float a = exp2_fast(m[r] - ms), bb = exp2_fast(mo - ms);
            l[r] = l[r] * a + lo_ * bb;
            if constexpr (kBf16) lf[r] = lf[r] * a + lfo * bb;
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
                for (int j = 0; j < kPer16; ++j) s_acc[wave][r][(i * LPT + c) * kPer16 + j] = acc[r][i * kPer16 + j];
            if (c == 0) {
                s_m[wave][r] = m[r];
                s_l[wave][r] = l[r];
                s_lf[wave][r] = kBf16 ? lf[r] : l[r];
            }
        }
    }
    __syncthreads();

    // ---- combine the waves and write o_s = acc / l, lse_s = (m + log2 l) * ln 2
    for (int i = tid; i < nr * D; i += kThreads) {
        const int r = i / D, d = i - r * D;
        float M = s_m[0][r];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][r]);
        const float ms = (M == -INFINITY) ? 0.f : M;
        float lsum = 0.f, lfsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = exp2_fast(s_m[w][r] - ms);
            lsum += s_l[w][r] * f;
            lfsum += s_lf[w][r] * f;
            o += s_acc[w][r][d] * f;
        }
        const int64_t row = out_row(r);
        // agent-scope stores: a merging group on another XCD reads them (fused merge)
        store_partial(p.part_o + (row * S + split) * Dv + d, lsum > 0.f ? o / lsum : 0.f);
        if (d == 0)
            store_partial(p.part_lse + row * S + split,
                          lsum > 0.f ? (ms + __builtin_amdgcn_logf(lfsum)) * 0.69314718055994531f : -INFINITY);
    }
    if (p.counters) {  // one launch per step: the unit's last split merges (s_acc is free now)
        const int nsplit = min(S, (vlen + p.chunk - 1) / p.chunk);
        constexpr int kPerThread = (RP * D + kThreads - 1) / kThreads;
        fused_arrive_merge<kThreads, D, kPerThread>(p, wu.unit, nsplit, nr, out_row,
                                                 &s_acc[0][0][0]);
    }
}

template <typename T, int D, int RP, int MODE, int U, int LPT, bool FP8, bool INT4>
__global__ void __launch_bounds__(kThreads) partial_valu_kernel(const PartialParams p) {
    partial_valu_body<T, D, RP, MODE, U, LPT, FP8, INT4>(p);
}

// The int4 form is bound by memory latency at one wave per SIMD; held to two (256 registers), a
// second wave's loads and arithmetic overlap the first's wait.
template <typename T, int D, int RP, int MODE, int U, int LPT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
partial_valu_kernel_int4(const PartialParams p) {
    partial_valu_body<T, D, RP, MODE, U, LPT, false, true>(p);
}

template <typename T, int D, int RP, int MODE, bool FP8, bool INT4>
hipError_t launch_t(const PartialParams &p, hipStream_t stream) {
    constexpr int kRowLanes = D * (FP8 ? 1 : (int)sizeof(T)) / 16;
    // int4: 16 lanes per row (8 dimensions each) and 4 keys per slot, a 16-key step in few registers
    constexpr int LPT = INT4 ? 16 : AD_VALU_LANES_PER_ROW < kRowLanes ? AD_VALU_LANES_PER_ROW : kRowLanes;
    constexpr int U = INT4 ? 4 : AD_VALU_KEYS_PER_SLOT;
    const dim3 grid(p.num_splits * p.batch * p.num_kv_heads * p.row_blocks);  // see decode_unit
    if constexpr (INT4)
        hipLaunchKernelGGL((partial_valu_kernel_int4<T, D, RP, MODE, U, LPT>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((partial_valu_kernel<T, D, RP, MODE, U, LPT, FP8, INT4>), grid, dim3(kThreads), 0, stream,
                           p);
    return hipGetLastError();
}

template <typename T, int D, int RP, bool FP8, bool INT4>
hipError_t by_mode(const PartialParams &p, int mode, hipStream_t s) {
    switch (mode) {
        case KV_CONTIG: return launch_t<T, D, RP, KV_CONTIG, FP8, INT4>(p, s);
        case KV_PAGED: return launch_t<T, D, RP, KV_PAGED, FP8, INT4>(p, s);
        default: return launch_t<T, D, RP, KV_SPARSE, FP8, INT4>(p, s);
    }
}

// An fp8 or int4 unit holds at most 4 rows (the host plans so): 8 rows would need more registers
// than a lane has, and those instantiations are not built.
template <typename T, int D, bool FP8 = false, bool INT4 = false>
hipError_t by_rows(const PartialParams &p, int rows_padded, int mode, hipStream_t s) {
    constexpr int kMaxRows = (FP8 || INT4) ? 4 : 8;
    if (rows_padded > kMaxRows) return hipErrorInvalidValue;
    switch (rows_padded) {
        case 1: return by_mode<T, D, 1, FP8, INT4>(p, mode, s);
        case 2: return by_mode<T, D, 2, FP8, INT4>(p, mode, s);
        case 4: return by_mode<T, D, 4, FP8, INT4>(p, mode, s);
        default: return by_mode<T, D, kMaxRows, FP8, INT4>(p, mode, s);
    }
}

}  // namespace

hipError_t launch_partial_valu(const PartialParams &p, int dtype, int head_dim, int rows_padded, int mode,
                               hipStream_t stream) {
    if (p.kv_fp8) {  // the host admits an fp8 cache with bf16 queries and head dim 128 only
        if (dtype != DT_BF16 || head_dim != 128) return hipErrorInvalidValue;
        return by_rows<uint16_t, 128, true>(p, rows_padded, mode, stream);
    }
    if (p.kv_int4) {  // likewise for an int4 cache
        if (dtype != DT_BF16 || head_dim != 128) return hipErrorInvalidValue;
        return by_rows<uint16_t, 128, false, true>(p, rows_padded, mode, stream);
    }
    if (dtype == DT_F32) {
        return head_dim == 64 ? by_rows<float, 64>(p, rows_padded, mode, stream)
                              : by_rows<float, 128>(p, rows_padded, mode, stream);
    }
    return head_dim == 64 ? by_rows<uint16_t, 64>(p, rows_padded, mode, stream)
                          : by_rows<uint16_t, 128>(p, rows_padded, mode, stream);
}

}  // namespace ad
