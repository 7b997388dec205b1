// mla_mfma.hip -- partial split-KV pass of multi-head latent attention (MLA) on the matrix cores.
//
// What it computes (FlashInfer mla.cuh, the MLA decode kernel): one shared latent KV head per
// token, ckv (512 values) and kpe (64 rotary values). A query head's score is
//   s = scale * (q_nope . ckv + q_pe . kpe)
// and its value vector is the same ckv row. Per work unit (split s, block of up to 128 query rows,
// sequence b) the kernel writes the attention of those rows over the split's keys as a normalised
// partial o_s = acc / l (512 values) and a natural-log LSE, like the other split-KV passes
// (mslk splitk_kernels.py, _fwd_kernel_splitK epilogue). Rows are r = t * H + h.
//
// Design for CDNA4:
//
//   * 128 query heads per work group, 32 per wave: every wave keeps its Q (576 bf16 per head) in
//     registers as the B operand of S^T = K Q^T and its 32 x 512 fp32 output in the accumulation
//     registers. The KV tile (32 keys x 1152 B) is shared by the 4 waves through LDS, so HBM
//     delivers each key once per unit and LDS feeds the matrix cores.
//   * Tiles are copied HBM -> LDS with buffer_load ... lds (no register staging) into a 4-slot
//     ring: while tile i is computed, tiles i+1 .. i+3 are in flight. Each slot is its own LDS
//     object and the loop is unrolled by 4, so the compiler knows which copies a read depends
//     on; a wave waits for its own copies of tile i (vmcnt) and a barrier publishes everybody's.
//   * A key row in LDS is 72 chunks of 16 B (64 latent + 8 rotary); chunk c of key k sits at
//     position c ^ f(k). With f(k) = 4*bit1(k) + bits2..3(k), the score operand reads
//     (ds_read_b128: 16 keys, one chunk) and the transposing value reads (ds_read_b64_tr_b16:
//     4 keys x 4 chunks per 32 lanes) are both free of bank conflicts.
//   * Scores, online softmax (base 2, lazy rescale), P rounding and the P.V product follow the
//     generic matrix-core pass: lane l ends with 16 keys of query row l%32, P in bf16 is the A
//     operand of P.V with the matching key order, V comes from the transposing LDS reads.
//   * Keys past the split or the sequence are never read from the cache (their copies read the
//     unit's own query row) and get probability 0.
#include "ad_internal.h"

#include <limits.h>
#include <math.h>

namespace ad {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kRows = kWaves * kRowsPerWave;      // query rows per work unit
constexpr int kTile = 32;                         // keys per tile
constexpr int kLatent = 512, kRope = 64;
constexpr int kLatBytes = kTile * kLatent * 2;    // latent part of a ring slot: 32 rows x 1 KB
constexpr int kRopeBytes = kTile * kRope * 2;     // rotary part: 32 rows x 128 B
constexpr int kCopiesPerWave = kTile / kWaves + 1;  // latent row copies + one rotary copy, per tile and wave
constexpr int kKs = (kLatent + kRope) / 16;       // k-steps (16 values) of the score product
constexpr int kLatKs = kLatent / 16;
constexpr int kSlabs = kLatent / 32;              // 32-column slabs of the output
constexpr int kStoreSlabs = 4;                     // slabs per transposed store group
constexpr int kStageStride = 32 * kStoreSlabs + 4; // floats per staged row (the pad spreads banks)
// All matrix-core accumulators of a kernel live in one register file (the accumulation registers
// here), which holds 256 per lane: 15 output slabs plus the score accumulator fill it exactly. The
// last output slab is therefore summed in ordinary registers: each tile's product for it goes
// into a fresh accumulator (the score accumulator's registers, free by then) and is added.
constexpr int kAccSlabs = kSlabs - 1;
// A row's reference max is fixed at its first tile with a visible key; later scores may exceed it
// by up to 2^64 (probabilities up to 2^64 stay finite in bf16 and in the fp32 sums). A row that
// goes further makes the work group recompute its unit exactly: one pass for every row's true
// max, then the main pass with that max as the reference. The accumulators are never rescaled.
constexpr float kHeadroom = 64.f;
constexpr int kPipe = 4;  // LDS operand reads in flight ahead of the matrix products

// s_waitcnt with vmcnt(n) and no wait on the other counters (gfx9 encoding).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// Buffer descriptor word 3 for raw (untyped, unswizzled) buffer accesses on the gfx9 family.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {  // round to nearest even
    bf16x2 r;
    r.x = (__bf16)lo;
    r.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// LDS layout of a ring slot. Latent chunk c (16 B) of key k sits at k*1024 + 16*(c ^ F(k)) of the
// slot's latent object; rotary chunk c of key k at k*128 + 16*(c ^ Hr(k)) of its rotary object. With these permutations the score
// operand reads (ds_read_b128: 16 keys, one chunk) and the transposing value reads
// (ds_read_b64_tr_b16: 4 keys x 4 chunks per 32 lanes) hit distinct banks.
// The 64-bit value held as (hi, lo) words in lane `l`. The lane read returns a signed int: each
// word is widened as unsigned, or a low word with bit 31 set would fill the high word with ones.
__device__ __forceinline__ uint64_t lane_u64(uint32_t hi, uint32_t lo, int l) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, l) << 32) |
           (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lo, l);
}

__device__ __forceinline__ int swz_lat(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }
__device__ __forceinline__ int swz_rope(int k) { return (k >> 1) & 7; }

// Work-group placement. The dispatcher deals work groups to the 8 XCDs round robin (group L to
// XCD L % 8), and each XCD has its own L2. Unit u = (b * row_blocks + rb) * splits + split is
// given to the group that makes consecutive units share an XCD: the splits of a sequence then
// read its queries (4.7 MB for 128 heads) through one L2 instead of eight. A bijection of [0, N).
__device__ __forceinline__ int xcd_unit(int L, int N) {
    constexpr int kXcds = 8;
    const int per = N / kXcds, rem = N % kXcds, x = L % kXcds;
    return x * per + min(x, rem) + L / kXcds;
}

__global__ void __launch_bounds__(kThreads) mla_partial_kernel(const PartialParams p) {
    const int unit = xcd_unit(blockIdx.x, gridDim.x);
    const int split = unit % p.num_splits;
    const int rb = (unit / p.num_splits) % p.row_blocks;
    const int b = unit / (p.num_splits * p.row_blocks);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;
    const int H = p.group, Q = p.q_len, R = H * Q, S = p.num_splits;
    const int r0 = rb * kRows + wave * kRowsPerWave;   // this wave's first row
    const int nr = max(0, min(kRowsPerWave, R - r0));  // its valid rows
    const int L = p.seq_lens ? p.seq_lens[b] : p.kv_len_max;
    const int t0 = split * p.chunk;
    const int t1 = min(t0 + p.chunk, L);

    auto out_row = [&](int r) -> int64_t {  // r: row of this wave
        const int ra = r0 + r, t = ra / H, g = ra - t * H;
        return (int64_t)(b * Q + t) * p.num_q_heads + g;
    };

    if (t0 >= t1) {  // uniform over the work group
        if (p.write_empty) {
            for (int i = lane; i < nr * kLatent; i += 64) {
                const int r = i / kLatent, d = i - r * kLatent;
                p.part_o[(out_row(r) * S + split) * kLatent + d] = 0.f;
            }
            for (int r = lane; r < nr; r += 64) p.part_lse[out_row(r) * S + split] = -INFINITY;
        }
        return;
    }

    __shared__ int s_map[kMapCapacity];
    // Ring slots: separate LDS objects, so that the compiler can tell which copies a read or a
    // store depends on (the rotary parts are written by ordinary stores, never by copies).
    __shared__ __attribute__((aligned(16))) unsigned char s_lat0[kLatBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_lat1[kLatBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_lat2[kLatBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_lat3[kLatBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_rope0[kRopeBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_rope1[kRopeBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_rope2[kRopeBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_rope3[kRopeBytes];
    __shared__ float s_x[kWaves][kRowsPerWave];  // per-row exchange inside a wave
    __shared__ int s_flag[kWaves];

    const int map_shift = p.page_shift, map_mask = (1 << map_shift) - 1;
    const int map_first = t0 >> map_shift;
    {
        const int n = ((t1 - 1) >> map_shift) - map_first + 1;
        const int32_t *bt = p.block_table + b * p.bt_stride + map_first;
        for (int i = tid; i < n; i += kThreads) s_map[i] = bt[i];
    }
    __syncthreads();

    // ---- this lane's query row (row col of the wave): B operand, 32 latent + 4 rotary k-steps
    const uint16_t *q_nope = static_cast<const uint16_t *>(p.q);
    const uint16_t *q_pe = static_cast<const uint16_t *>(p.q2);
    const uint16_t *safe_n = q_nope + b * p.q_s[0];  // row (b, 0, 0): finite, always readable
    const uint16_t *safe_p = q_pe + b * p.q2_s[0];
    u32x4 qb[kKs];
    int lo_r = INT_MIN, hi_r = INT_MAX;
    if (col < nr) {
        const int ra = r0 + col, t = ra / H, g = ra - t * H;
        const uint16_t *qn = q_nope + b * p.q_s[0] + t * p.q_s[1] + g * p.q_s[2];
        const uint16_t *qp = q_pe + b * p.q2_s[0] + t * p.q2_s[1] + g * p.q2_s[2];
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks)
            qb[ks] = ks < kLatKs ? ld16(qn + 16 * ks + 8 * half) : ld16(qp + 16 * (ks - kLatKs) + 8 * half);
        const int qpos = L - Q + t;
        if (p.causal) hi_r = qpos + 1;
        if (p.window) lo_r = qpos - p.window + 1;
    } else {
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) qb[ks] = u32x4{0, 0, 0, 0};
    }
    // keys [lo_max, hi_min) are visible to every row of the unit
    const int t_first = __builtin_amdgcn_readfirstlane((rb * kRows) / H);
    const int t_last = __builtin_amdgcn_readfirstlane((min(R, (rb + 1) * kRows) - 1) / H);
    const int hi_min = p.causal ? L - Q + t_first + 1 : INT_MAX;
    const int lo_max = p.window ? L - Q + t_last - p.window + 1 : INT_MIN;

    const uint16_t *ckv = static_cast<const uint16_t *>(p.k);
    const uint16_t *kpe = static_cast<const uint16_t *>(p.k2);

    // ---- copy tile [base, base + 32) of the split into a ring slot, HBM -> LDS with
    // buffer_load ... lds (no register staging). Wave w copies the latent rows of keys w, w+4, ..,
    // w+28 (one 1-KB copy per row, lane i bringing chunk i ^ F(key)) and the rotary rows of keys
    // 8w .. 8w+7 (lane i: key 8w + i/8, chunk (i%8) ^ Hr(key)). Those 8 keys lie in one page:
    // tiles start at multiples of 16 and pages hold 16, 32 or 64 keys. Every descriptor covers
    // only rows the copy may read, so the hardware range check confines it: a latent row is
    // 1 KB, a rotary group ends after its last key inside the split; lanes beyond read zeros
    // (the scores of those keys are masked). Latent rows past the split read the unit's query
    // row instead. The buffer form of the LDS copy matters: the compiler treats the global form
    // as a possible LDS access of unknown order and would make every LDS read wait for all.
    // The copies are nontemporal (cache-policy bit 1 of the buffer instruction): each reads whole
    // lines once: 128 -> 113 us for 32 sequences of 8192 keys under 128 heads.
    constexpr int kStreamPolicy = 2;
    const int64_t rope_stride = p.k2_s[1] * 2;  // bytes between the rotary rows of two slots of a page
    auto issue = [&](lds_u8 *lat_slot, lds_u8 *rope_slot, int base) {
        // Row addresses of key base + i in lane i (i < 32), computed once per tile on the vector
        // unit; each copy takes its row with a lane read. Keys past the split get the query row.
        const int vl = base + (lane & 31);
        const int vlc = min(vl, t1 - 1);
        const int64_t pg = s_map[(vlc >> map_shift) - map_first];
        const int sl = vlc & map_mask;
        const uint64_t lat_row = vl < t1 ? (uint64_t)(ckv + pg * p.k_s[0] + sl * p.k_s[1]) : (uint64_t)safe_n;
        const uint64_t rope_row = vl < t1 ? (uint64_t)(kpe + pg * p.k2_s[0] + sl * p.k2_s[1]) : (uint64_t)safe_p;
        const uint32_t lat_lo = (uint32_t)lat_row, lat_hi = (uint32_t)(lat_row >> 32);
        const uint32_t rope_lo = (uint32_t)rope_row, rope_hi = (uint32_t)(rope_row >> 32);
#pragma unroll
        for (int j = 0; j < kTile / kWaves; ++j) {
            const int kk = wave + kWaves * j;  // uniform
            const uint64_t row = lane_u64(lat_hi, lat_lo, kk);
            const __amdgpu_buffer_rsrc_t rsrc =
                __builtin_amdgcn_make_buffer_rsrc((void *)row, (short)0, kLatent * 2, kBufferFlags);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void *)(lat_slot + kk * 1024), 16, (lane ^ swz_lat(kk)) << 4,
                0, 0, kStreamPolicy);
        }
        const int v0 = base + 8 * wave;  // uniform: first key of this wave's rotary group
        const int nv = min(max(t1 - v0, 0), 8);
        const uint64_t row = lane_u64(rope_hi, rope_lo, 8 * wave);
        const int k = 8 * wave + (lane >> 3);
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void *)row, (short)0, nv > 0 ? (int)((nv - 1) * rope_stride) + kRope * 2 : 0, kBufferFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void *)(rope_slot + wave * 1024), 16,
            (int)((lane >> 3) * rope_stride) + (((lane & 7) ^ swz_rope(k)) << 4), 0, 0, kStreamPolicy);
    };

    // Per-lane LDS offsets inside a slot; every read adds a compile-time offset that fits the DS
    // instruction's immediate field.
    //   score operand, k-step ks < 32: key col, latent chunk 2ks + half = k_off[ks % 8] + 256 (ks / 8)
    //   score operand, k-step 32 + i:  key col, rotary chunk 2i + half  = r_off[i]
    //   value read (k-step t, read rd, slab s): key 16t + 8rd + tr_row, chunk 4s + tr_chunk
    //                                          = v_off[4rd + s % 4] + (16t + 8rd) * 1024 + 256 (s / 4)
    int k_off[8], r_off[4], v_off[8];
    {
        const int tr_row = 4 * half + ((lane & 15) >> 2);
        const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) k_off[i] = col * 1024 + (((2 * i + half) ^ swz_lat(col)) << 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) r_off[i] = col * 128 + (((2 * i + half) ^ swz_rope(col)) << 4);
#pragma unroll
        for (int rd = 0; rd < 2; ++rd)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v_off[4 * rd + i] = tr_row * 1024 + (((4 * i + tr_chunk) ^ swz_lat(8 * rd + tr_row)) << 4) + ((lane & 1) << 3);
    }

    float m = -INFINITY, l = 0.f, lf = 0.f;  // row col's reference max and sums (this lane's keys)
    bool overflow = false;
    f32x16 o[kSlabs];  // o[0 .. kAccSlabs-1]: matrix-core accumulators; o[kAccSlabs]: summed by the VALU
    // Zeros are produced as a product with zero operands: every value that reaches the loop-carried
    // accumulators then comes out of the matrix core, and the compiler keeps them in the
    // accumulation registers for the whole loop (a plain 0.f start made it carry all 240 in
    // ordinary registers and copy them over at every iteration, spilling the queries).
    auto clear = [&]() {
#pragma unroll
        for (int s = 0; s < kAccSlabs; ++s) o[s] = mfma(u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}, f32x16{});
#pragma unroll
        for (int j = 0; j < 16; ++j) o[kAccSlabs][j] = 0.f;
    };
    clear();

    // Scores of tile `base` (base-2 units, masked) for row col, 16 keys of this lane.
    // LDS operand reads run kPipe matrix products ahead of their use: a read issued right before
    // the product that needs it would stall every product for the full LDS latency.
    auto k_operand = [&](const lds_u8 *cur, const lds_u8 *rcur, int ks) -> u32x4 {
        const lds_u8 *at = ks < kLatKs ? cur + k_off[ks & 7] + 256 * (ks >> 3) : rcur + r_off[ks - kLatKs];
        return *(const __attribute__((address_space(3))) u32x4 *)at;
    };
    auto scores = [&](const lds_u8 *cur, const lds_u8 *rcur, int base, float (&sv)[16]) {
        f32x16 sc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[j] = 0.f;
        u32x4 ka[kPipe];
#pragma unroll
        for (int i = 0; i < kPipe; ++i) ka[i] = k_operand(cur, rcur, i);
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            sc = mfma(ka[ks % kPipe], qb[ks], sc);
            if (ks + kPipe < kKs) ka[ks % kPipe] = k_operand(cur, rcur, ks + kPipe);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) sv[j] = sc[j] * p.scale_log2;
        const bool full = base + kTile <= t1 && base >= lo_max && base + kTile <= hi_min;  // uniform
        if (!full) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int pos = base + 8 * (j / 4) + 4 * half + (j % 4);
                const bool vis = pos < t1 && pos >= lo_r && pos < hi_r;
                sv[j] = vis ? sv[j] : -INFINITY;
            }
        }
    };

    auto v_operand = [&](const lds_u8 *cur, int t, int s) -> u32x4 {
        s16x4 part[2];
#pragma unroll
        for (int rd = 0; rd < 2; ++rd)
            part[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(cur + v_off[4 * rd + (s & 3)] + (16 * t + 8 * rd) * 1024 +
                                                            256 * (s >> 2)));
        return __builtin_bit_cast(u32x4, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto compute = [&](const lds_u8 *cur, const lds_u8 *rcur, int base) {
        float sv[16];
        scores(cur, rcur, base, sv);
        u32x4 vb_pipe[kPipe];  // first value operands, loading while the softmax runs
#pragma unroll
        for (int i = 0; i < kPipe; ++i) vb_pipe[i] = v_operand(cur, i / kAccSlabs, i % kAccSlabs);
        float mx = sv[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sv[j]);
        mx = pair_max(mx);
        if (m == -INFINITY) m = mx;  // first visible key of the row: o, l and lf are still exactly 0
        overflow = overflow || mx > m + kHeadroom;
        const float ms = (m == -INFINITY) ? 0.f : m;
        uint32_t pk[8];
        const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p0 = exp2_fast(sv[2 * i] - ms), p1 = exp2_fast(sv[2 * i + 1] - ms);  // exp2(-inf) = 0
            pk[i] = pack_bf16(p0, p1);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]), ones, l, false);
            lf += p0 + p1;
        }
        // products in order: (t, s) for s < kAccSlabs, t = 0 then 1; then the summed slab, t = 0, 1
        constexpr int kProducts = 2 * kSlabs;
        auto prod_t = [](int i) { return i < 2 * kAccSlabs ? i / kAccSlabs : i - 2 * kAccSlabs; };
        auto prod_s = [](int i) { return i < 2 * kAccSlabs ? i % kAccSlabs : kAccSlabs; };
        u32x4 pa[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) pa[t] = u32x4{pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]};
        f32x16 part;
#pragma unroll
        for (int i = 0; i < kProducts; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            const int t = prod_t(i), s = prod_s(i);
            const u32x4 vb = vb_pipe[i % kPipe];
            if (i + kPipe < kProducts) vb_pipe[i % kPipe] = v_operand(cur, prod_t(i + kPipe), prod_s(i + kPipe));
            if (s < kAccSlabs)
                o[s] = mfma(pa[t], vb, o[s]);
            else
                part = mfma(pa[t], vb, t == 0 ? f32x16{} : part);
        }
        o[kAccSlabs] += part;
    };

    auto max_only = [&](const lds_u8 *cur, const lds_u8 *rcur, int base) {
        float sv[16];
        scores(cur, rcur, base, sv);
        float mx = sv[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sv[j]);
        m = fmaxf(m, pair_max(mx));
    };

    // The ring over the split (4 slots, 3 tiles in flight): before tile `base` is used, each wave
    // waits for its own copies of it (vmcnt: the copies of the next two tiles may stay in flight)
    // and a barrier publishes all of them; the barrier also ends every read of the slot the copy
    // of tile base + 3*32 then overwrites. Copies past the end read nothing or the query row, so
    // every step issues the same number of copies and the vmcnt count is exact. At the end every
    // copy has landed and every read is done.
    auto run = [&](auto body) {
        lds_u8 *l0 = (lds_u8 *)s_lat0, *l1 = (lds_u8 *)s_lat1, *l2 = (lds_u8 *)s_lat2, *l3 = (lds_u8 *)s_lat3;
        lds_u8 *q0 = (lds_u8 *)s_rope0, *q1 = (lds_u8 *)s_rope1, *q2 = (lds_u8 *)s_rope2, *q3 = (lds_u8 *)s_rope3;
        auto step = [&](lds_u8 *cur, lds_u8 *qcur, lds_u8 *nxt, lds_u8 *qnxt, int base) -> bool {
            if (base >= t1) return false;  // uniform
            __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kCopiesPerWave));
            asm volatile("s_barrier" ::: "memory");
            issue(nxt, qnxt, base + 3 * kTile);
            body(cur, qcur, base);
            return true;
        };
        issue(l0, q0, t0);
        issue(l1, q1, t0 + kTile);
        issue(l2, q2, t0 + 2 * kTile);
        for (int base = t0;; base += 4 * kTile) {
            if (!step(l0, q0, l3, q3, base)) break;
            if (!step(l1, q1, l0, q0, base + kTile)) break;
            if (!step(l2, q2, l1, q1, base + 2 * kTile)) break;
            if (!step(l3, q3, l2, q2, base + 3 * kTile)) break;
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        __syncthreads();
    };

    run(compute);
    if (lane == 0) s_flag[wave] = __builtin_amdgcn_ballot_w64(overflow) != 0;
    __syncthreads();
    if (s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3]) {  // uniform; rare: recompute exactly
        m = -INFINITY;
        run(max_only);
        l = lf = 0.f;
        clear();
        run(compute);  // m is every row's true max: no score exceeds it
    }

    // ---- o_s = acc / l, lse_s = (m + log2 lf) * ln 2 for this wave's rows
    l = pair_sum(l);
    lf = pair_sum(lf);
    if (half == 0) s_x[wave][col] = l;
    float lr[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) lr[j] = s_x[wave][8 * (j / 4) + 4 * half + (j % 4)];
    float inv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) inv[j] = lr[j] > 0.f ? 1.f / lr[j] : 0.f;
    // The accumulators hold one column per lane; the partial rows go out as 16-byte stores of
    // four columns, transposed through this wave's ring slot (free since the loop's last
    // barrier): kStoreSlabs slabs at a time as 32 rows of kStageStride floats.
    lds_u8 *slot = wave == 0 ? (lds_u8 *)s_lat0 : wave == 1 ? (lds_u8 *)s_lat1 : wave == 2 ? (lds_u8 *)s_lat2 : (lds_u8 *)s_lat3;
    __attribute__((address_space(3))) float *stage = (__attribute__((address_space(3))) float *)slot;
    static_assert(kRowsPerWave * kStageStride * 4 <= kLatBytes, "a slab group fits a ring slot");
#pragma unroll
    for (int g = 0; g < kSlabs / kStoreSlabs; ++g) {
#pragma unroll
        for (int sl = 0; sl < kStoreSlabs; ++sl)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                stage[(8 * (j / 4) + 4 * half + (j % 4)) * kStageStride + 32 * sl + col] =
                    o[kStoreSlabs * g + sl][j] * inv[j];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < kRowsPerWave / 2; ++i) {
            const int r = 2 * i + half;  // lanes 0-31 row 2i, lanes 32-63 row 2i + 1: 4 columns each
            const f32x4 v = *(const __attribute__((address_space(3))) f32x4 *)(stage + r * kStageStride + 4 * col);
            if (r < nr)
                *reinterpret_cast<f32x4 *>(p.part_o + (out_row(r) * S + split) * kLatent +
                                           32 * kStoreSlabs * g + 4 * col) = v;
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (half == 0 && col < nr) {
        const float ms = (m == -INFINITY) ? 0.f : m;
        p.part_lse[out_row(col) * S + split] =
            l > 0.f ? (ms + __builtin_amdgcn_logf(lf)) * 0.69314718055994531f : -INFINITY;
    }
}

}  // namespace

hipError_t launch_partial_mla(const PartialParams &p, hipStream_t stream) {
    const dim3 grid(p.num_splits * p.row_blocks * p.batch);
    hipLaunchKernelGGL(mla_partial_kernel, grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ad
