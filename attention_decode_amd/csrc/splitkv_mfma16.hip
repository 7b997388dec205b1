// splitkv_mfma16.hip -- partial split-KV pass on the matrix cores for work units of at most 16 query
// rows (bf16, fp8 or one-group int4 caches): small GQA groups times speculative tokens, e.g. 4
// query heads per KV head over an fp8 or int4 cache.
//
// It computes what the 32-row matrix-core pass (splitkv_mfma.hip) computes: per work unit (split s,
// block of up to 16 query rows r = t*G + g of KV head h, sequence b) the attention of those rows
// restricted to the split's keys, stored as o_s = acc / l with a natural-log LSE (mslk
// splitk_kernels.py, _fwd_kernel_splitK epilogue), online softmax in base-2 units. The group of
// query heads sharing a KV head is padded to 16 rows rather than 32 (TensorRT-LLM mha.cu rounds its
// warp tile of heads x tokens up to a multiple of 16), so a 4-row group makes 4x the needed
// matrix-core products instead of 8x, and a wave needs half the registers: several work groups
// share a compute unit and cover each other's arithmetic with their loads.
//
// Layout on v_mfma_f32_16x16x32_bf16 (A: lane l holds row l%16 and 8 reduction elements chosen by
// l/16; B likewise with column l%16; C: lane l holds column l%16 of rows 4(l/16) .. +3):
//
//   * Scores transposed, S^T = K Q^T, per 16-key block kb of a 32-key tile: K is the A operand, a
//     lane holding 8 head-dim elements of key 16kb + l%16 straight from HBM; Q is the B operand,
//     lane l holding query row l%16, in registers for the whole unit. The result leaves lane l with
//     keys 16kb + 4(l/16) .. +3 of query row l%16: 8 keys per tile, so the row max and sum are an
//     in-lane reduction and two lane swaps (l^16, l^32).
//   * Those 8 probabilities, rounded to bf16, are the A operand of P.V as they stand: reduction
//     index 8(l/16) + i of lane l is key 16(i/4) + 4(l/16) + i%4. V is the B operand with the same
//     key order, read from a per-wave LDS tile with ds_read_b64_tr_b16 (the tile's 16-byte chunks
//     XOR-swizzled by row as in the 32-row pass: both the stores of 16 rows and the transposing
//     reads of 4 rows x 2 chunks are free of bank conflicts).
//   * Head-dim order of the score reduction: k-step ks of a bf16 cache covers elements 32ks ..
//     32ks+31, lane group l/16 taking 8 of them; an fp8 operand takes 16 bytes (elements 64j +
//     16(l/16) .. +15) into k-steps 2j and 2j+1, loaded straight into the operand (half rows) or,
//     by default, loaded as whole 128-byte rows and read back from a per-wave LDS tile (ROWS);
//     an int4 operand takes a lane's 4 words of fields in the order int4_x8 produces. Q is loaded
//     in the same order (the order of a reduction is free as long as both operands share it).
//   * Everything else follows the 32-row pass: a work group of 4 waves each taking every 4th 32-key
//     tile with loads one tile ahead; keys outside the split, past the sequence, seen by no row of
//     the unit or in unlisted blocks never read (their loads go to the unit's own query row, their
//     probability is 0); masking only on tiles that are not fully visible; lazy rescaling through a
//     small LDS exchange; P rounded to bf16 with the normaliser summing the rounded values
//     (TensorRT-LLM mha.cu computeRowSum) and the LSE the fp32 ones; fp8 (OCP E4M3) rows times
//     their fp32 scales (TensorRT-LLM mha.cu kvCacheScale; mslk splitk_kernels.py,
//     _process_fp8_quantization), key scales on the fp32 scores, value scales in P before its bf16
//     rounding, the normaliser summing each rounded product divided by its scale; the 4 waves
//     combined once through LDS; the in-pass merge when the host asks for one launch.
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
constexpr int kTile = 32;  // keys per wave per step: two 16-key blocks
constexpr int kRows = 16;  // query rows per work unit

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// 16-byte LDS store and load.
__device__ __forceinline__ void st_lds16(lds_u8 *at, u32x4 x) { *(__attribute__((address_space(3))) u32x4 *)at = x; }
__device__ __forceinline__ u32x4 ld_lds16(const lds_u8 *at) {
    return *(const __attribute__((address_space(3))) u32x4 *)at;
}

// All four lanes l, l^16, l^32, l^48 get the max / sum of their four values.
__device__ __forceinline__ float quad_max(float x) { return pair_max(pair16_max(x)); }
__device__ __forceinline__ float quad_sum(float x) { return pair_sum(pair16_sum(x)); }

// 8 int4 fields of a word as bf16 values 128 + f, in the order fields 0, 4, 1, 5, 2, 6, 3, 7 (each
// pair (j, j + 4) is the word shifted by 4 j, masked and ORed with the exponent pattern, one
// v_and_or_b32 with Int4Consts: exact, since 128 + f needs 8 significant bits).
__device__ __forceinline__ u32x4 int4_x8(uint32_t w, Int4Consts k) {
    return u32x4{(w & k.mask) | k.bits, ((w >> 4) & k.mask) | k.bits, ((w >> 8) & k.mask) | k.bits,
                 ((w >> 12) & k.mask) | k.bits};
}
// The query's 8 bf16 values of the same 8 dimensions (a 16-byte load q), in that order.
__device__ __forceinline__ u32x4 int4_order(u32x4 q) {
    return u32x4{(q[0] & 0xFFFFu) | (q[2] << 16), (q[0] >> 16) | (q[2] & 0xFFFF0000u), (q[1] & 0xFFFFu) | (q[3] << 16),
                 (q[1] >> 16) | (q[3] & 0xFFFF0000u)};
}
// Dimension of the output column 16 c + i of the value product on an int4 cache: the LDS value
// tile keeps each word's 8 fields in int4_x8's order.
__device__ __forceinline__ int int4_dim(int col) {
    const int q = col & 7;
    return (col & ~7) + (q >> 1) + 4 * (q & 1);
}
// Scale (low half) and shift (high half) of an int4 coefficient word, both fp16.
__device__ __forceinline__ void int4_coef(uint32_t cw, float &scale, float &shift) {
    scale = (float)__builtin_bit_cast(_Float16, (uint16_t)(cw & 0xFFFFu));
    shift = (float)__builtin_bit_cast(_Float16, (uint16_t)(cw >> 16));
}

// QF: the cache format, bf16 (kQfBf16), OCP E4M3 with fp32 row scales (kQfFp8), or int4 rows with
// one fp16 scale / shift pair (kQfInt4).
enum { kQfBf16 = 0, kQfFp8 = 1, kQfInt4 = 2 };

// ROWS (fp8): each load instruction reads whole 128-byte rows (lane l: byte piece l%8 of key
// l/8 of an 8-key group) instead of half rows of 16 keys, and K goes through a per-wave LDS tile
// to the matrix operand; see the load forms below.
template <int D, int MODE, int QF, bool ROWS>
__global__ void __launch_bounds__(kThreads) partial_mfma16_kernel(const PartialParams p) {
    constexpr bool FP8 = QF == kQfFp8, INT4 = QF == kQfInt4, QUANT = FP8 || INT4;
    static_assert(!ROWS || FP8, "the whole-row form is built for fp8 caches");
    constexpr int kKs = D / 32;                   // k-steps of the score product
    constexpr int kCols = D / 16;                 // 16-column blocks of the output
    constexpr int kRowBytes = D * 2;              // one bf16 row of the LDS V tile
    // 16-byte pieces per lane, key block and operand (int4: the lane's 4 words of fields)
    constexpr int kLoads = FP8 ? D / 64 : INT4 ? 1 : kKs;
    static_assert(!QUANT || D == 128, "a quantised cache has head dim 128");

    const UnitId wu = p.lpt ? decode_unit_lpt<kThreads>(p) : decode_unit(p);
    const int split = wu.split, rb = wu.rb, h = wu.h, b = wu.b;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, grp = lane >> 4;
    const int G = p.group, Q = p.q_len, S = p.num_splits, Dv = p.head_dim_v;
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
    // per-wave V tiles during the loop, per-wave fp32 accumulators for the final combine
    constexpr int kBufBytes = kWaves * kRows * D * 4 > kWaves * kTile * kRowBytes ? kWaves * kRows * D * 4
                                                                                  : kWaves * kTile * kRowBytes;
    __shared__ __attribute__((aligned(16))) unsigned char s_buf[kBufBytes];
    __shared__ __attribute__((aligned(16))) float s_alpha[kWaves][kRows];
    __shared__ float s_m[kWaves][kRows], s_l[kWaves][kRows], s_lf[kWaves][kRows];
    __shared__ float s_fw[kWaves][kRows], s_inv[kRows];  // combine weights of the waves' partials, 1 / l
    // Quantised cache: per wave and tile key, the key scale times scale * log2(e) (the scores'
    // base-2 units), the value scale and its reciprocal (int4: and the key's (shift - 128 scale)
    // times scale * log2(e), the value's shift), 0 for a key that is not read, read back in the
    // score accumulator's key order
    constexpr int kQW = QUANT ? kWaves : 1, kIW = INT4 ? kWaves : 1;
    const Int4Consts i4k = [] {
        if constexpr (INT4) return int4_consts();
        else return Int4Consts{0u, 0u};
    }();
    __shared__ __attribute__((aligned(16))) float s_ks[kQW][kTile], s_vs[kQW][kTile], s_vr[kQW][kTile];
    __shared__ __attribute__((aligned(16))) float s_kz[kIW][kTile], s_vz[kIW][kTile];
    __shared__ float s_corr[kIW][kRows];  // int4: the shifts' share of each wave's rows
    // ROWS: the wave's K tile as loaded (32 keys x 128 bytes), piece c of key k at c ^ (k % 8)
    __shared__ __attribute__((aligned(16))) unsigned char s_kt[ROWS ? kWaves : 1][ROWS ? kTile * 128 : 16];

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

    // ---- this lane's query row (row c16 of the unit) as the B operand, and its visible range
    const uint16_t *qbase = static_cast<const uint16_t *>(p.q) +
                            (p.q_starts ? (int64_t)qrows.first * p.q_s[1] : b * p.q_s[0]) +
                            (int64_t)(h * G) * p.q_s[2];
    u32x4 qb[kKs];
    float qsum = 0.f;  // int4: the sum of the row's query values (this lane's share until reduced)
    int lo_r = INT_MIN, hi_r = INT_MAX;
    // Tree mask: the last Qb keys are the drafts; this lane's row sees draft i only with bit i of
    // its token's mask row (tm0: drafts 0-31, tm1: 32-63).
    const int first_draft = L - Qb;
    uint32_t tm0 = ~0u, tm1 = ~0u;
    {
        const int ra = r0 + c16;
        const int t = ra / G, g = ra - t * G;
        if (c16 < nr) {
            const uint16_t *qr = qbase + t * p.q_s[1] + g * p.q_s[2];
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {  // quantised: the head-dim order of the K operand
                if constexpr (INT4) {  // word 4 grp + ks of the row: dims 8 (4 grp + ks) .. + 7
                    const u32x4 q8 = ld16(qr + 8 * (4 * grp + ks));
                    qb[ks] = int4_order(q8);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        qsum += __uint_as_float(q8[j] << 16) + __uint_as_float(q8[j] & 0xFFFF0000u);
                } else {
                    qb[ks] = ld16(qr + (FP8 ? 64 * (ks / 2) + 16 * grp + 8 * (ks % 2) : 32 * ks + 8 * grp));
                }
            }
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
    if constexpr (INT4) qsum = quad_sum(qsum);
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
    // one K / V element (int4: a 32-bit word, the unit of the int4 strides)
    using KV = std::conditional_t<FP8, uint8_t, std::conditional_t<INT4, uint32_t, uint16_t>>;
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
    // finite (bf16), always readable, at least D bf16 values (int4: 1 + D / 8 words); an fp8 cache's
    // bytes read from it may be NaN codes and an int4 coefficient word NaN halves, which never
    // reach the sums (masked scores, zeroed values and coefficients)
    const KV *safe = reinterpret_cast<const KV *>(qbase);

    // Lane l loads key 16 kb + l%16 of the tile for kb = 0, 1: bf16 pieces at elements 32 ks +
    // 8 (l/16), fp8 pieces at bytes 64 j + 16 (l/16), int4 words 1 + 4 (l/16) .. + 3 (after the
    // coefficient word) and the coefficient word. ROWS: lane l loads bytes 16 (l%8) .. + 15 of
    // keys 16 kb + 8 jr + l/8 for jr = 0, 1 (8 lanes read a whole row in one instruction).
    constexpr int kR = ROWS ? 2 : 1;  // keys per lane and 16-key block
    struct Buf {
        u32x4 k[2][kLoads];
        u32x4 v[2][kLoads];
        float ks[2], vs[2];  // fp8: the scales of key l % 16 as loaded (any value for a key that is not read)
        bool slive[2];       // fp8: that key is read
        uint32_t kc[2], vc[2];  // int4: the coefficient words
        bool live[2][kR];      // quantised: the lane's key is read
        int base;
    };
    // ROWS: a block wholly inside the split and the unit's visible range lies in one page or one
    // listed block (both at least 16 keys, aligned): one lookup and one row address for the wave,
    // and each lane's row i of the block at i times the row stride from it, one 32 x 32 -> 64-bit
    // multiply-add (strides below 2^26 elements; other strides, and the other blocks, address key by
    // key). That saves the per-key lookups and 64-bit arithmetic of a lane's two rows per block (fp8
    // 106.6 -> 104.5 us per step on the ragged fp8 workload); with one row per lane and block the
    // wait for the wave-wide lookup costs more than it saves (int4 77.5 -> 81.5 us), so the other
    // forms address key by key. ROWS: the lane's rows are keys 8 jr + l / 8 and its scales those of
    // key l % 16; otherwise both are key l % 16.
    const int lane_key = ROWS ? (lane >> 3) : c16;
    constexpr uint64_t kNarrow = uint64_t(1) << 26;
    const bool narrow = ROWS && (uint64_t)p.k_s[1] < kNarrow && (uint64_t)p.v_s[1] < kNarrow &&
                        (!FP8 || ((uint64_t)p.ks_s[1] < kNarrow && (uint64_t)p.vs_s[1] < kNarrow));
    auto row_at = [](const auto *base, int i, int64_t stride) { return base + (uint64_t)(uint32_t)i * (uint32_t)stride; };
    auto fetch = [&](Buf &f, int base) {
        f.base = base;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int vb = base + 16 * kb;  // uniform, a multiple of 16
            const KV *kp[kR], *vp[kR];
            const float *ksp = p.k_scale, *vsp = p.v_scale;  // the arrays' first scales: always readable
            bool slive = false;                                // the scales' key is read
            // Only addresses are formed here; the loads below are issued on every path.
            bool whole = ROWS && narrow && vb + 16 <= t1;  // uniform
            int64_t page = 0;
            int pos0 = vb;
            if constexpr (MODE == KV_SPARSE) {
                if (whole) pos0 = __builtin_amdgcn_readfirstlane(logical(vb));
                whole = whole && pos0 + 16 <= L;
            }
            whole = whole && pos0 >= lo_min && pos0 + 16 <= hi_max;
            if constexpr (MODE == KV_PAGED)
                if (whole) page = __builtin_amdgcn_readfirstlane(s_map[(vb >> map_shift) - map_first]);
            if (whole) {
                const int slot = MODE == KV_PAGED ? (vb & map_mask) : pos0;
                const int64_t pk = MODE == KV_PAGED ? page * p.k_s[0] : 0, pv = MODE == KV_PAGED ? page * p.v_s[0] : 0;
#pragma unroll
                for (int jr = 0; jr < kR; ++jr) {
                    kp[jr] = row_at(kbase + pk + (int64_t)(slot + 8 * jr) * p.k_s[1], lane_key, p.k_s[1]);
                    vp[jr] = row_at(vbase + pv + (int64_t)(slot + 8 * jr) * p.v_s[1], lane_key, p.v_s[1]);
                }
                if constexpr (FP8) {
                    const int64_t pks = MODE == KV_PAGED ? page * p.ks_s[0] : 0;
                    const int64_t pvs = MODE == KV_PAGED ? page * p.vs_s[0] : 0;
                    ksp = row_at(ksbase + pks + (int64_t)slot * p.ks_s[1], c16, p.ks_s[1]);
                    vsp = row_at(vsbase + pvs + (int64_t)slot * p.vs_s[1], c16, p.vs_s[1]);
                }
                slive = true;
            } else {
                // key v's row offsets (64-bit), or false for a key that is not read
                auto rows_of = [&](int v, int64_t &rk, int64_t &rv, int64_t &rks, int64_t &rvs) -> bool {
                    if (v >= t1) return false;
                    if constexpr (MODE == KV_PAGED) {  // logical position = v, and v < t1 <= L
                        if (v < lo_min || v >= hi_max) return false;
                        const int64_t pg = s_map[(v >> map_shift) - map_first];
                        const int slot = v & map_mask;
                        rk = pg * p.k_s[0] + slot * p.k_s[1];
                        rv = pg * p.v_s[0] + slot * p.v_s[1];
                        rks = pg * p.ks_s[0] + slot * p.ks_s[1];
                        rvs = pg * p.vs_s[0] + slot * p.vs_s[1];
                    } else {
                        const int pos = logical(v);
                        if (pos >= L || pos < lo_min || pos >= hi_max) return false;
                        rk = (int64_t)pos * p.k_s[1];
                        rv = (int64_t)pos * p.v_s[1];
                        rks = (int64_t)pos * p.ks_s[1];
                        rvs = (int64_t)pos * p.vs_s[1];
                    }
                    return true;
                };
#pragma unroll
                for (int jr = 0; jr < kR; ++jr) {
                    int64_t rk = 0, rv = 0, rks = 0, rvs = 0;
                    const bool live = rows_of(vb + 8 * jr + lane_key, rk, rv, rks, rvs);
                    kp[jr] = live ? kbase + rk : safe;
                    vp[jr] = live ? vbase + rv : safe;
                    if constexpr (FP8 && !ROWS) {
                        if (live) {
                            ksp = ksbase + rks;
                            vsp = vsbase + rvs;
                        }
                        slive = live;
                    }
                }
                if constexpr (FP8 && ROWS) {
                    int64_t rk = 0, rv = 0, rks = 0, rvs = 0;
                    slive = rows_of(vb + c16, rk, rv, rks, rvs);
                    if (slive) {
                        ksp = ksbase + rks;
                        vsp = vsbase + rvs;
                    }
                }
            }
            if constexpr (FP8) {  // used only once this buffer is current (a select there would wait)
                f.ks[kb] = *ksp;
                f.vs[kb] = *vsp;
                f.slive[kb] = slive;
            }
#pragma unroll
            for (int jr = 0; jr < kR; ++jr) {
                if constexpr (INT4) {  // rows are 4-byte aligned only: word loads
                    const uint32_t *kw = kp[0] + 1 + 4 * grp, *vw = vp[0] + 1 + 4 * grp;
                    f.k[kb][0] = u32x4{kw[0], kw[1], kw[2], kw[3]};
                    f.v[kb][0] = u32x4{vw[0], vw[1], vw[2], vw[3]};
                    f.kc[kb] = kp[0][0];
                    f.vc[kb] = vp[0][0];
                    f.live[kb][0] = kp[0] != safe;
                } else if constexpr (ROWS) {
                    f.k[kb][jr] = ld16_stream(kp[jr] + 16 * (lane & 7));
                    f.v[kb][jr] = ld16_stream(vp[jr] + 16 * (lane & 7));
                    f.live[kb][jr] = kp[jr] != safe;
                } else if constexpr (FP8) {
#pragma unroll
                    for (int j = 0; j < kLoads; ++j)
                        f.k[kb][j] = j == kLoads - 1 ? ld16_last(kp[0] + 64 * j + 16 * grp) : ld16(kp[0] + 64 * j + 16 * grp);
#pragma unroll
                    for (int j = 0; j < kLoads; ++j)
                        f.v[kb][j] = j == kLoads - 1 ? ld16_last(vp[0] + 64 * j + 16 * grp) : ld16(vp[0] + 64 * j + 16 * grp);
                    f.live[kb][0] = kp[0] != safe;
                } else {
#pragma unroll
                    for (int ks = 0; ks < kKs; ++ks) f.k[kb][ks] = ld16(kp[0] + 32 * ks + 8 * grp);
#pragma unroll
                    for (int ks = 0; ks < kKs; ++ks) f.v[kb][ks] = ld16(vp[0] + 32 * ks + 8 * grp);
                }
            }
        }
    };

    lds_u8 *vw = (lds_u8 *)s_buf + wave * kTile * kRowBytes;  // this wave's V tile
    lds_u8 *kt = (lds_u8 *)s_kt[ROWS ? wave : 0];                 // and its K tile (ROWS)
    // Transposing-read address of this lane for read rd and output block c: row 16 rd + 4 grp +
    // (lane&15)/4, chunk 2c + (lane&3)/2, half-chunk lane&1.
    const int tr_row = 4 * grp + (c16 >> 2);
    const int tr_chunk = (lane & 3) >> 1;
    const int tr_byte = (lane & 1) << 3;

    float m = -INFINITY, l = 0.f, lf = 0.f;  // row c16's running state (this lane's keys)
    float corr = 0.f;  // int4: sum over this lane's keys of w (shift) - 128 P' (w: the key's weight)
    f32x4 o[kCols];
#pragma unroll
    for (int c = 0; c < kCols; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Buf &cur, bool full) {
        if constexpr (ROWS) {  // K as loaded and V converted to bf16 -> LDS: row 16 kb + 8 jr + lane / 8
            const int pc = lane & 7;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int jr = 0; jr < kR; ++jr) {
                    const int row = 16 * kb + 8 * jr + (lane >> 3);
                    const bool live = cur.live[kb][jr];
                    st_lds16(kt + row * 128 + ((pc ^ (row & 7)) << 4), cur.k[kb][jr]);
                    u32x4 w = cur.v[kb][jr];
                    if (!full && !live) w = u32x4{0, 0, 0, 0};  // a key that is not read may hold NaN codes
                    lds_u8 *vr = vw + row * kRowBytes;
                    st_lds16(vr + (((2 * pc) ^ swz<D>(row)) << 4), e4m3_x8(w[0], w[1]));
                    st_lds16(vr + (((2 * pc + 1) ^ swz<D>(row)) << 4), e4m3_x8(w[2], w[3]));
                }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (grp == 0) {  // key 16 kb + c16's scales; a key that is not read takes scale 0
                    const int row = 16 * kb + c16;
                    const float vsv = cur.slive[kb] ? cur.vs[kb] : 0.f;
                    s_ks[wave][row] = cur.slive[kb] ? cur.ks[kb] * p.scale_log2 : 0.f;
                    s_vs[wave][row] = vsv;
                    s_vr[wave][row] = vsv != 0.f ? __builtin_amdgcn_rcpf(vsv) : 0.f;
                }
        }
        // Other forms: V tile -> LDS, row 16 kb + c16; bf16 chunk 4 ks + grp; fp8 piece j as chunks
        // 8 j + 2 grp (+1)
        if constexpr (!ROWS) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int row = 16 * kb + c16;
                lds_u8 *vr = vw + row * kRowBytes;
                if constexpr (INT4) {  // word j of the lane's 4 as chunk 4 grp + j (fields in int4_x8 order)
                    const u32x4 w = cur.v[kb][0];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *(__attribute__((address_space(3))) u32x4 *)(vr + (((4 * grp + j) ^ swz<D>(row)) << 4)) =
                            int4_x8(w[j], i4k);
                    if (grp == 0) {  // a key that is not read takes scales and shifts 0
                        const bool live = cur.live[kb][0];
                        float ksc, ksh, vsc, vsh;
                        int4_coef(cur.kc[kb], ksc, ksh);
                        int4_coef(cur.vc[kb], vsc, vsh);
                        s_ks[wave][row] = live ? ksc * p.scale_log2 : 0.f;
                        s_kz[wave][row] = live ? fmaf(-128.f, ksc, ksh) * p.scale_log2 : 0.f;
                        s_vs[wave][row] = live ? vsc : 0.f;
                        s_vr[wave][row] = live && vsc != 0.f ? __builtin_amdgcn_rcpf(vsc) : 0.f;
                        s_vz[wave][row] = live ? vsh : 0.f;
                    }
                } else if constexpr (FP8) {
#pragma unroll
                    for (int j = 0; j < kLoads; ++j) {
                        u32x4 w = cur.v[kb][j];
                        if (!full && !cur.live[kb][0]) w = u32x4{0, 0, 0, 0};  // a key not read may hold NaN codes
                        const int c0 = 8 * j + 2 * grp;
                        st_lds16(vr + ((c0 ^ swz<D>(row)) << 4), e4m3_x8(w[0], w[1]));
                        st_lds16(vr + (((c0 + 1) ^ swz<D>(row)) << 4), e4m3_x8(w[2], w[3]));
                    }
                    if (grp == 0) {  // a key that is not read takes scale 0
                        const float vsv = cur.slive[kb] ? cur.vs[kb] : 0.f;
                        s_ks[wave][row] = cur.slive[kb] ? cur.ks[kb] * p.scale_log2 : 0.f;
                        s_vs[wave][row] = vsv;
                        s_vr[wave][row] = vsv != 0.f ? __builtin_amdgcn_rcpf(vsv) : 0.f;
                    }
                } else {
#pragma unroll
                    for (int ks = 0; ks < kKs; ++ks)
                        *(__attribute__((address_space(3))) u32x4 *)(vr + (((4 * ks + grp) ^ swz<D>(row)) << 4)) =
                            cur.v[kb][ks];
                }
            }
        }
        // S^T = K Q^T, one 16-key block at a time
        f32x4 sc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (INT4) {
#pragma unroll
                for (int ks = 0; ks < kKs; ++ks) sc[kb] = mfma16(int4_x8(cur.k[kb][0][ks], i4k), qb[ks], sc[kb]);
            } else if constexpr (FP8) {
#pragma unroll
                for (int j = 0; j < kLoads; ++j) {
                    // ROWS: bytes 64 j + 16 grp of key 16 kb + c16 from the LDS tile
                    const int key = 16 * kb + c16;
                    const u32x4 w = ROWS ? ld_lds16(kt + key * 128 + (((4 * j + grp) ^ (key & 7)) << 4)) : cur.k[kb][j];
                    sc[kb] = mfma16(e4m3_x8(w[0], w[1]), qb[2 * j], sc[kb]);
                    sc[kb] = mfma16(e4m3_x8(w[2], w[3]), qb[2 * j + 1], sc[kb]);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < kKs; ++ks) sc[kb] = mfma16(cur.k[kb][ks], qb[ks], sc[kb]);
            }
        }
        // this lane's keys: 16 kb + 4 grp + e of the tile
        float sv[2][4];
        f32x4 vs4[QUANT ? 2 : 1], vr4[QUANT ? 2 : 1], vz4[INT4 ? 2 : 1];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if constexpr (INT4) {  // s (128 + f).q + (shift - 128 s) sum q
                const f32x4 k4 = *(const f32x4 *)&s_ks[wave][16 * kb + 4 * grp];
                const f32x4 z4 = *(const f32x4 *)&s_kz[wave][16 * kb + 4 * grp];
                vs4[kb] = *(const f32x4 *)&s_vs[wave][16 * kb + 4 * grp];
                vr4[kb] = *(const f32x4 *)&s_vr[wave][16 * kb + 4 * grp];
                vz4[kb] = *(const f32x4 *)&s_vz[wave][16 * kb + 4 * grp];
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[kb][e] = fmaf(sc[kb][e], k4[e], z4[e] * qsum);
            } else if constexpr (FP8) {
                const f32x4 k4 = *(const f32x4 *)&s_ks[wave][16 * kb + 4 * grp];
                vs4[kb] = *(const f32x4 *)&s_vs[wave][16 * kb + 4 * grp];
                vr4[kb] = *(const f32x4 *)&s_vr[wave][16 * kb + 4 * grp];
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[kb][e] = sc[kb][e] * k4[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[kb][e] = sc[kb][e] * p.scale_log2;
            }
        }
        if (!full) {  // uniform
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int v4 = cur.base + 16 * kb + 4 * grp;  // keys v4 .. v4+3 share a page / block
                const int pos4 = v4 < t1 ? logical(v4) : 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int pos = pos4 + e;
                    bool vis = v4 + e < t1 && pos < L && pos >= lo_r && pos < hi_r;
                    if (p.tree_mask && vis && pos >= first_draft) {
                        const int i = pos - first_draft;  // < Qb <= 64: a visible key lies below L
                        vis = ((i < 32 ? tm0 : tm1) >> (i & 31)) & 1u;
                    }
                    sv[kb][e] = vis ? sv[kb][e] : -INFINITY;
                }
            }
        }
        float mx = sv[0][0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j / 4][j % 4]);
        mx = quad_max(mx);
        const bool raise = mx > m + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform
            // Rows that do not move keep factor 1 exactly (exp2(m - m) is NaN while m = -inf).
            const float alpha = raise ? exp2_fast(m - mx) : 1.f;
            m = raise ? mx : m;
            l *= alpha;
            lf *= alpha;
            if constexpr (INT4) corr *= alpha;
            if (grp == 0) s_alpha[wave][c16] = alpha;
            // output rows of this lane: 4 grp + j
            const f32x4 a4 = *(const f32x4 *)&s_alpha[wave][4 * grp];
#pragma unroll
            for (int c = 0; c < kCols; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) o[c][j] *= a4[j];
        }
        const float ms = (m == -INFINITY) ? 0.f : m;
        uint32_t pk[4];
        const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kb = i / 2, e = 2 * (i % 2);
            const float p0 = exp2_fast(sv[kb][e] - ms), p1 = exp2_fast(sv[kb][e + 1] - ms);  // exp2(-inf) = 0
            if constexpr (QUANT) {  // value scales into P; normaliser from the rounded products / scales
                const float vs0 = vs4[kb][e], vs1 = vs4[kb][e + 1];
                pk[i] = pack_bf16(p0 * vs0, p1 * vs1);
                const float q0 = __uint_as_float(pk[i] << 16), q1 = __uint_as_float(pk[i] & 0xFFFF0000u);
                const float w0 = vs0 != 0.f ? q0 * vr4[kb][e] : p0, w1 = vs1 != 0.f ? q1 * vr4[kb][e + 1] : p1;
                l += w0 + w1;
                if constexpr (INT4)  // the fields enter the product as 128 + f
                    corr += fmaf(w0, vz4[kb][e], -128.f * q0) + fmaf(w1, vz4[kb][e + 1], -128.f * q1);
            } else {
                pk[i] = pack_bf16(p0, p1);
                l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]), ones, l, false);
            }
            lf += p0 + p1;
        }
        // O += P V over the tile's 32 keys, one 16-column block at a time
        const u32x4 pa = u32x4{pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
        for (int c = 0; c < kCols; ++c) {
            s16x4 part[2];
#pragma unroll
            for (int rd = 0; rd < 2; ++rd) {
                const int row = 16 * rd + tr_row;
                const int chunk = 2 * c + tr_chunk;
                part[rd] = ds_read_tr(vw + row * kRowBytes + ((chunk ^ swz<D>(row)) << 4) + tr_byte);
            }
            const s16x8 vb = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
            o[c] = mfma16(pa, __builtin_bit_cast(u32x4, vb), o[c]);
        }
    };

    constexpr int kStride = kWaves * kTile;
    auto iterate = [&](Buf &cur, Buf &nxt) {
        fetch(nxt, cur.base + kStride);
        __builtin_amdgcn_sched_barrier(0);
        bool full = cur.base + kTile <= t1;
        if (full) {
            const int pf = logical(cur.base), pl = logical(cur.base + kTile - 1);
            full = pl - pf == kTile - 1 && pl < L && pf >= lo_max && pl < hi_min;
        }
        compute(cur, full);
    };

    // Pairs of tiles with the loop's only exit test at the back edge (the loads in flight are the
    // same on every path into the loop), and an odd last tile after it. One tile in flight per
    // wave: at two waves per SIMD a third buffer (two tiles ahead) spills or halves the occupancy
    // with bf16 and fp8 tiles, and measured no faster with the smaller int4 tiles.
    const int first = t0 + wave * kTile;
    const int ntiles = first < t1 ? (t1 - first + kStride - 1) / kStride : 0;
    Buf A, B;
    fetch(A, first);
    int i = 0;
    for (; i + 2 <= ntiles; i += 2) {
        iterate(A, B);
        iterate(B, A);
    }
    if (i < ntiles) iterate(A, B);

    // ---- combine the waves: o_s = acc / l, lse_s = (m + log2 lf) * ln 2
    l = quad_sum(l);
    lf = quad_sum(lf);
    if constexpr (INT4) corr = quad_sum(corr);
    __syncthreads();  // every wave is done with its tiles: s_buf now holds the accumulators
    float *s_o = reinterpret_cast<float *>(s_buf) + wave * kRows * D;
    if (grp == 0) {
        s_m[wave][c16] = m;
        s_l[wave][c16] = l;
        s_lf[wave][c16] = lf;
        if constexpr (INT4) s_corr[wave][c16] = corr;
    }
#pragma unroll
    for (int c = 0; c < kCols; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s_o[(4 * grp + j) * D + (INT4 ? int4_dim(16 * c + c16) : 16 * c + c16)] = o[c][j];
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
        for (int w = 0; w < kWaves; ++w) {
            if constexpr (INT4)
                acc += (s_all[(w * kRows + r) * D + d] + s_corr[w][r]) * s_fw[w][r];
            else
                acc += s_all[(w * kRows + r) * D + d] * s_fw[w][r];
        }
        store_partial(p.part_o + (out_row(r) * S + split) * Dv + d, acc * s_inv[r]);
    }
    if (p.counters) {  // one launch per step: the unit's last split merges (s_buf is free now)
        const int nsplit = min(S, (vlen + p.chunk - 1) / p.chunk);
        constexpr int kPerThread = (kRows * D + kThreads - 1) / kThreads;
        fused_arrive_merge<kThreads, D, kPerThread>(p, wu.unit, nsplit, nr, out_row,
                                                 reinterpret_cast<float *>(s_buf));
    }
}

template <int D, int QF, bool ROWS = false>
hipError_t by_mode(const PartialParams &p, int mode, hipStream_t s) {
    const dim3 grid(p.num_splits * p.batch * p.num_kv_heads * p.row_blocks);  // see decode_unit
    switch (mode) {
        case KV_CONTIG:
            hipLaunchKernelGGL((partial_mfma16_kernel<D, KV_CONTIG, QF, ROWS>), grid, dim3(kThreads), 0, s, p);
            break;
        case KV_PAGED:
            hipLaunchKernelGGL((partial_mfma16_kernel<D, KV_PAGED, QF, ROWS>), grid, dim3(kThreads), 0, s, p);
            break;
        default:
            hipLaunchKernelGGL((partial_mfma16_kernel<D, KV_SPARSE, QF, ROWS>), grid, dim3(kThreads), 0, s, p);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_partial_mfma16(const PartialParams &p, int head_dim, int mode, hipStream_t stream) {
    // the host admits quantised caches with head dim 128 only, and int4 rows of one coefficient group
    if (p.kv_int4) {
        if (head_dim != 128 || p.kv_groups != 1) return hipErrorInvalidValue;
        return by_mode<128, kQfInt4>(p, mode, stream);
    }
    if (p.kv_fp8) {
        if (head_dim != 128) return hipErrorInvalidValue;
        return p.mfma_rows ? by_mode<128, kQfFp8, true>(p, mode, stream) : by_mode<128, kQfFp8>(p, mode, stream);
    }
    return head_dim == 64 ? by_mode<64, kQfBf16>(p, mode, stream) : by_mode<128, kQfBf16>(p, mode, stream);
}

}  // namespace ad
