// ad_internal.h -- parameter blocks shared by the host entry points (api.cpp) and the kernel
// launchers (*.hip). Not installed; the public interface is include/attn_decode.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ad {

enum KvMode : int { KV_CONTIG = 0, KV_PAGED = 1, KV_SPARSE = 2 };
enum Dtype : int { DT_F32 = 0, DT_BF16 = 1 };

// Largest page-id / block-id window one work unit stages in LDS (tokens per split / page + 2).
constexpr int kMapCapacity = 1040;

// One partial pass: every work unit is (split s, KV head h, sequence b).
struct PartialParams {
    const void *q;
    int64_t q_s[3];       // {b, t, hq}
    const void *k;
    int64_t k_s[3];       // contiguous {b, token, h}; paged {page, slot, h}
    const void *v;
    int64_t v_s[3];
    const int32_t *seq_lens;  // nullable: every sequence has kv_len_max keys
    int32_t kv_len_max;
    // paged
    const int32_t *block_table;
    int64_t bt_stride;
    int32_t page_shift;
    // block-sparse
    const int32_t *num_blocks;
    const int32_t *block_idx;
    int64_t nb_s[2];
    int64_t ix_s[3];
    int32_t block_shift;
    // shape
    int32_t batch, q_len, num_q_heads, num_kv_heads, group, head_dim_v;
    int32_t row_blocks;   // work units per KV head along its G * q_len query rows (grid y = Hkv * row_blocks)
    int32_t mfma_rows;    // matrix-core kernel, bf16: whole-row loads staged through LDS (grids of several rounds)
    float scale_log2;     // softmax scale * log2(e): scores are kept in base-2 units
    int32_t causal, window;
    int32_t num_splits, chunk;  // split s covers [s*chunk, (s+1)*chunk) of the (virtual) key range
    int32_t write_empty;        // 1: splits past the end still write (0, -inf); 0: they do nothing
    float *part_o;              // [rows][num_splits][head_dim_v]
    float *part_lse;            // [rows][num_splits]
    // One launch per step: when counters is set, the last split of each work unit (b, KV head,
    // row block) to finish merges the unit's rows into out / lse. counters[unit] counts arrivals;
    // zero before the launch, and zero again after it.
    uint32_t *counters;
    void *out;
    int64_t out_s[3];
    int32_t out_dtype;
    float *lse;
    // Quantised cache: k / v hold OCP E4M3 bytes (k_s / v_s count bytes), each element times the
    // fp32 scale of its row, k_scale[b|page * ks_s[0] + token|slot * ks_s[1] + h * ks_s[2]].
    int32_t kv_fp8;
    const float *k_scale;
    int64_t ks_s[3];
    const float *v_scale;
    int64_t vs_s[3];
    // Int4 cache: k / v rows of 32-bit words (k_s / v_s count words), kv_groups coefficient words
    // (fp16 scale low, fp16 shift high) then D / 8 words of 4-bit fields.
    int32_t kv_int4, kv_groups;
    // Speculative decoding: packed query rows of variable count per sequence (q_starts, nullable)
    // and a tree mask over each sequence's last Q_b keys, mask_words 32-bit words per token row.
    const int32_t *q_starts;
    const uint32_t *tree_mask;
    int32_t mask_words;
    // MLA second score part (rope): q_pe rows and kpe rows, 64 columns
    const void *q2;
    int64_t q2_s[3];
    const void *k2;
    int64_t k2_s[3];
    // Longest-piece-first placement (decode_unit_lpt): set by the host for ragged lengths.
    int32_t lpt;
};

// Work-group placement of the GQA partial passes: a 1-D grid of (units x splits) groups, unit =
// (b, KV head, row block), with the split index slowest. The dispatcher deals group L to XCD
// L % 8, so every XCD gets an equal share of every split index (the later splits of a ragged
// batch are often empty, and a split-fastest order would pile the full ones onto some XCDs), and
// the fullest splits are dispatched first.
struct UnitId {
    int split, unit, rb, h, b;
};
__device__ __forceinline__ UnitId decode_unit(const PartialParams &p) {
    const int units = p.batch * p.num_kv_heads * p.row_blocks;
    UnitId u;
    u.split = blockIdx.x / units;
    u.unit = blockIdx.x - u.split * units;
    u.rb = u.unit % p.row_blocks;
    const int bh = u.unit / p.row_blocks;
    u.h = bh % p.num_kv_heads;
    u.b = bh / p.num_kv_heads;
    return u;
}

// Longest-piece-first placement, for per-sequence (ragged) lengths on grids of several rounds. A
// piece is (sequence b, split s), and its Hkv x row_blocks work groups are consecutive in the grid.
// Pieces go out in order of decreasing size, the classic longest-processing-time order for
// scheduling jobs on identical machines: every full split (chunk keys) first, sequence by
// sequence, then each sequence's remainder split from the longest down (ties by sequence), then
// the empty splits. The dispatcher hands the groups out in grid order, so the short remainders
// fill the last gaps instead of long splits starting last. Every work group ranks the pieces
// itself from the lengths with the same arithmetic (no launch before the pass), so the groups
// cover every piece exactly once. The host sets p.lpt only with seq_lens given, no block list, at
// most kLptMaxBatch sequences, and more work groups than compute units. Every thread of the work
// group (NT threads) must call it; it synchronises the group.
constexpr int kLptMaxBatch = 256;

__device__ __forceinline__ int wave_incl_sum(int x) {  // inclusive prefix sum over the wave's lanes
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

template <int NT>
__device__ __forceinline__ UnitId decode_unit_lpt(const PartialParams &p) {
    static_assert(NT >= kLptMaxBatch, "one thread per sequence");
    constexpr int kW = NT / 64;
    __shared__ int s_rem[kLptMaxBatch];  // remainder keys per sequence (0: none)
    __shared__ int s_tot[3][kW];          // per wave: full splits, empty splits, remainders
    __shared__ int s_piece[2];            // (b, split) of this group's piece
    const int tid = threadIdx.x, wave = tid >> 6;
    const int B = p.batch, S = p.num_splits, C = p.chunk;
    const int U = p.num_kv_heads * p.row_blocks;
    const int k = blockIdx.x / U, sub = blockIdx.x - k * U;
    // thread tid = sequence tid: full splits n, remainder keys r (in split n), first empty split e
    int n = 0, r = 0;
    if (tid < B) {
        const int L = max(p.seq_lens[tid], 0);
        n = min(L / C, S);
        r = n < S ? L - n * C : 0;
    }
    const int e = n + (r > 0), ne = tid < B ? S - e : 0;
    if (tid < kLptMaxBatch) s_rem[tid] = r;
    const int pn = wave_incl_sum(n), pe = wave_incl_sum(ne);
    const int nr = __builtin_popcountll(__builtin_amdgcn_ballot_w64(r > 0));
    if ((tid & 63) == 63) {
        s_tot[0][wave] = pn;
        s_tot[1][wave] = pe;
    }
    if ((tid & 63) == 0) s_tot[2][wave] = nr;
    if (tid == 0) {  // overwritten below by the one thread whose piece has rank k (always in range)
        s_piece[0] = 0;
        s_piece[1] = 0;
    }
    __syncthreads();
    int F = 0, R = 0, bn = 0, be = 0;  // totals, and the sums of the waves before this one
#pragma unroll
    for (int w = 0; w < kW; ++w) {
        F += s_tot[0][w];
        R += s_tot[2][w];
        if (w < wave) {
            bn += s_tot[0][w];
            be += s_tot[1][w];
        }
    }
    const int first_n = bn + pn - n, first_e = be + pe - ne;  // exclusive prefixes
    if (k < F) {  // uniform: the full split k - first_n of this sequence
        if (k >= first_n && k < first_n + n) {
            s_piece[0] = tid;
            s_piece[1] = k - first_n;
        }
    } else if (k < F + R) {  // uniform: the remainder of rank k - F
        if (r > 0) {
            int rank = 0;
            for (int b = 0; b < B; ++b) {
                const int rb = s_rem[b];
                rank += (rb > r) | ((rb == r) & (b < tid));
            }
            if (rank == k - F) {
                s_piece[0] = tid;
                s_piece[1] = n;
            }
        }
    } else {  // the empty split k - F - R - first_e past this sequence's keys
        const int j = k - F - R;
        if (j >= first_e && j < first_e + ne) {
            s_piece[0] = tid;
            s_piece[1] = e + (j - first_e);
        }
    }
    __syncthreads();
    UnitId u;
    u.b = s_piece[0];
    u.split = s_piece[1];
    u.rb = sub % p.row_blocks;
    u.h = sub / p.row_blocks;
    u.unit = (u.b * p.num_kv_heads + u.h) * p.row_blocks + u.rb;
    return u;
}

// An int4 cache's fields become bf16 pairs 128 + f as ((word >> 4 j) & mask) | bits, with mask
// 0x000F000F (fields j and j + 4 of the word) and bits 0x43004300 (the exponent of 128 in each
// half). A three-operand instruction takes no literal on this architecture, so with the two
// constants as literals the compiler splits each mask-and-OR in two; held in registers they make
// one v_and_or_b32. The empty asm keeps them in registers, out of reach of constant folding.
struct Int4Consts {
    uint32_t mask, bits;
};
__device__ __forceinline__ Int4Consts int4_consts() {
    Int4Consts k{0x000F000Fu, 0x43004300u};
    asm volatile("" : "+v"(k.mask), "+v"(k.bits));
    return k;
}

// Query tokens of sequence b and the packed row of its token 0: q_len tokens at row b * q_len, or
// with q_starts the count q_starts[b+1] - q_starts[b] clamped to [0, q_len] (so that the padded
// partial rows stay in bounds) at row q_starts[b].
struct QRows {
    int n;
    int first;
};
__device__ __forceinline__ QRows q_rows(const int32_t *q_starts, int q_len, int b) {
    if (!q_starts) return QRows{q_len, b * q_len};
    const int s0 = q_starts[b];
    return QRows{min(max(q_starts[b + 1] - s0, 0), q_len), s0};
}

// Output element offset and LSE index of padded row `row` = (b * q_len + t) * num_q_heads + hq
// (the host keeps the row count below 2^31); t must be < the sequence's token count.
struct OutIdx {
    int64_t off;
    int lse;
};
__device__ __forceinline__ OutIdx out_index(const int32_t *q_starts, int q_len, int num_q_heads,
                                            const int64_t out_s[3], int row) {
    const int hq = row % num_q_heads, tq = row / num_q_heads;
    const int t = tq % q_len, b = tq / q_len;
    if (q_starts) {
        const int n = q_starts[b] + t;
        return OutIdx{(int64_t)n * out_s[1] + hq * out_s[2], n * num_q_heads + hq};
    }
    return OutIdx{b * out_s[0] + t * out_s[1] + hq * out_s[2], row};
}

struct MergeParams {
    const float *part_o;
    const float *part_lse;
    int32_t num_splits;
    int32_t rows;             // batch * q_len * num_q_heads
    int32_t head_dim_v;
    int32_t q_len, num_q_heads;
    // count_by_len: row b merges only min(num_splits, ceil(L_b / chunk)) splits, L_b = seq_lens[b]
    // (or kv_len_max when seq_lens is NULL) -- the splits a paged pass actually wrote.
    int32_t count_by_len;
    const int32_t *seq_lens;
    int32_t kv_len_max;
    int32_t chunk;
    int32_t out_dtype;
    void *out;
    int64_t out_s[3];
    float *lse;
    const int32_t *q_starts;  // nullable: rows of tokens t >= Q_b are skipped, out / lse packed
    // nullable: row b merges only its first splits_per_batch[b] splits (clamped to [0, num_splits])
    const int32_t *splits_per_batch;
};

// Launchers (hipSuccess or the launch error). They assume the host checks already passed.
hipError_t launch_partial_valu(const PartialParams &p, int dtype, int head_dim, int rows_padded, int mode,
                               hipStream_t stream);
hipError_t launch_partial_mfma(const PartialParams &p, int head_dim, int mode, hipStream_t stream);
hipError_t launch_partial_mfma16(const PartialParams &p, int head_dim, int mode, hipStream_t stream);
hipError_t launch_partial_mla(const PartialParams &p, hipStream_t stream);
hipError_t launch_merge(const MergeParams &p, hipStream_t stream);
hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, int groups, hipStream_t stream);

}  // namespace ad
