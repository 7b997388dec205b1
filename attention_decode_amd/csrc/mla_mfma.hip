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
// Design for CDNA4 (LDS layout and copy addressing: mla_layout.h):
//
//   * Scores by rows, values by columns. Wave w computes the scores of rows 32w .. 32w + 31: it
//     keeps their Q (576 bf16 per row) in registers as the B operand of S^T = K Q^T and reads K
//     from LDS. The value product is split the other way: wave w accumulates output columns
//     128w .. 128w + 127 of ALL 128 rows, reading only its quarter of each V row from LDS. The
//     probabilities cross between the waves through LDS once per tile (8 KB of bf16 A operands),
//     the sharding of mla.cuh's compute_mla_pv (QK_SHARD), where each warpgroup multiplies its
//     own slice of the 512 latent columns with the gathered P. Every V element read from LDS then
//     feeds 4 row blocks instead of 1: per 32-key tile and compute unit the transposing V reads
//     drop from 128 KB to 32 KB, the reads the LDS serves slowest.
//   * Each row's reference max is fixed at its first tile with a visible key and never moves, so
//     the value accumulators are never rescaled, and a wave can accumulate rows whose scores
//     another wave computed without any per-tile exchange of maxima. Later scores may exceed the
//     reference by up to 2^64 (probabilities up to 2^64 stay finite in bf16 and fp32); a row that
//     goes further makes the work group recompute its unit exactly: one pass for every row's true
//     max, then the main pass with that max.
//   * Tiles (32 keys: 32 KB latent + 4 KB rotary) are copied HBM -> LDS with buffer_load ... lds
//     (no register staging) into a 4-slot ring: while tile i is computed, tiles i+1 .. i+3 are in
//     flight. Each slot is its own LDS object and the loop is unrolled by 4, so the compiler knows
//     which copies a read depends on; a wave waits for its own copies of tile i (vmcnt) and a
//     barrier publishes everybody's. A second barrier per tile publishes the probabilities.
//   * Keys past the split or the sequence are never read from the cache (their copies read the
//     unit's own query row) and get probability 0.
#include "ad_internal.h"
#include "mla_layout.h"

#include <limits.h>
#include <math.h>

namespace ad {
namespace {

using namespace mla;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kKs = (kLatent + kRope) / 16;  // k-steps (16 values) of the score product
constexpr int kLatKs = kLatent / 16;
constexpr int kBlocks = kWaves;              // row blocks of 32 rows
// Value accumulators: 4 row blocks x 4 slabs of 32 columns. All matrix-core accumulators of a
// kernel live in one register file (the accumulation registers here), which holds 256 per lane:
// 15 of the 16 blocks plus the score accumulator fill it exactly. The last block (row block 3,
// slab 3) is summed in ordinary registers: each tile's products for it go into a fresh
// accumulator (the score accumulator's registers, free by then) and are added.
constexpr int kAcc = kBlocks * kSlabsPerWave;
constexpr int kVgprAcc = kAcc - 1;
constexpr float kHeadroom = 64.f;
constexpr int kPipe = 4;  // score-operand reads in flight ahead of the matrix products

// s_waitcnt with vmcnt(n) and no wait on the other counters (gfx9 encoding).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// s_waitcnt lgkmcnt(0) with no wait on the other counters.
constexpr int kLgkmZero = 15 | (3 << 14) | (7 << 4);
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
__device__ __forceinline__ u32x4 lds16(const lds_u8 *p) { return *(const __attribute__((address_space(3))) u32x4 *)p; }

// The 64-bit value held as (hi, lo) words in lane `l`. The lane read returns a signed int: each
// word is widened as unsigned, or a low word with bit 31 set would fill the high word with ones.
__device__ __forceinline__ uint64_t lane_u64(uint32_t hi, uint32_t lo, int l) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, l) << 32) |
           (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lo, l);
}

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
    const int L = p.seq_lens ? p.seq_lens[b] : p.kv_len_max;
    const int t0 = split * p.chunk;
    const int t1 = min(t0 + p.chunk, L);
    // valid rows of row block hb (32 rows each) of this unit
    auto rows_of = [&](int hb) { return max(0, min(kRowsPerWave, R - (rb * kRows + hb * kRowsPerWave))); };
    auto out_row = [&](int hb, int r) -> int64_t {  // r: row inside row block hb
        const int ra = rb * kRows + hb * kRowsPerWave + r, t = ra / H, g = ra - t * H;
        return (int64_t)(b * Q + t) * p.num_q_heads + g;
    };
    const int nr = rows_of(wave);  // rows whose scores this wave computes

    if (t0 >= t1) {  // uniform over the work group
        if (p.write_empty) {
            for (int i = lane; i < nr * kLatent; i += 64) {
                const int r = i / kLatent, d = i - r * kLatent;
                p.part_o[(out_row(wave, r) * S + split) * kLatent + d] = 0.f;
            }
            for (int r = lane; r < nr; r += 64) p.part_lse[out_row(wave, r) * S + split] = -INFINITY;
        }
        return;
    }

    __shared__ int s_map[mla::kMapCapacity];
    // Ring slots: separate LDS objects, so that the compiler can tell which copies a read or a
    // store depends on.
    __shared__ __attribute__((aligned(16))) unsigned char s_lat0[kLatBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_lat1[kLatBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_lat2[kLatBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_lat3[kLatBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_rope0[kRopeBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_rope1[kRopeBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_rope2[kRopeBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_rope3[kRopeBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_p[kPBytes];  // probabilities, all rows
    __shared__ float s_l[kRows];                                          // row sums, all rows
    __shared__ int s_flag[kWaves];

    const int map_shift = p.page_shift, map_mask = (1 << map_shift) - 1;
    const int map_first = t0 >> map_shift;
    {
        const int n = ((t1 - 1) >> map_shift) - map_first + 1;  // <= kMapCapacity (host plan)
        const int32_t *bt = p.block_table + b * p.bt_stride + map_first;
        for (int i = tid; i < n; i += kThreads) s_map[i] = bt[i];
    }
    __syncthreads();

    // ---- this lane's query row (row col of this wave's block): B operand, 32 latent + 4 rotary k-steps
    const uint16_t *q_nope = static_cast<const uint16_t *>(p.q);
    const uint16_t *q_pe = static_cast<const uint16_t *>(p.q2);
    const uint16_t *safe_n = q_nope + b * p.q_s[0];  // row (b, 0, 0): finite, always readable, 1 KB
    const uint16_t *safe_p = q_pe + b * p.q2_s[0];
    u32x4 qb[kKs];
    int lo_r = INT_MIN, hi_r = INT_MAX;
    if (col < nr) {
        const int ra = rb * kRows + wave * kRowsPerWave + col, t = ra / H, g = ra - t * H;
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
    const int r_first = rb * kRows, r_last = min(R, (rb + 1) * kRows) - 1;
    const int hi_min = p.causal ? L - Q + r_first / H + 1 : INT_MAX;
    const int lo_max = p.window ? L - Q + r_last / H - p.window + 1 : INT_MIN;

    const uint16_t *ckv = static_cast<const uint16_t *>(p.k);
    const uint16_t *kpe = static_cast<const uint16_t *>(p.k2);

    // ---- copy tile [base, base + 32) of the split into a ring slot, HBM -> LDS with
    // buffer_load ... lds (mla_layout.h: lat_copy_*, rope_copy_*). Every descriptor covers only the
    // rows the copy may read, so the hardware range check confines it. Latent rows past the split
    // read the unit's query row instead. The buffer form of the LDS copy matters: the compiler
    // treats the global form as a possible LDS access of unknown order and would make every LDS
    // read wait for all. The copies are nontemporal (cache-policy bit 1): each reads whole lines
    // once.
    constexpr int kStreamPolicy = 2;
    const int64_t rope_stride = p.k2_s[1] * 2;  // bytes between the rotary rows of two slots of a page
    auto issue = [&](lds_u8 *lat_slot, lds_u8 *rope_slot, int base) {
        // Row addresses of key base + i in lane i (i < 32), computed once per tile on the vector
        // unit; each copy takes its row with a lane read. Keys past the split get the query row.
        const int vl = base + col;
        const int vlc = min(vl, t1 - 1);
        const int64_t pg = s_map[(vlc >> map_shift) - map_first];
        const int sl = vlc & map_mask;
        const uint64_t lat_row = vl < t1 ? (uint64_t)(ckv + pg * p.k_s[0] + sl * p.k_s[1]) : (uint64_t)safe_n;
        const uint64_t rope_row = vl < t1 ? (uint64_t)(kpe + pg * p.k2_s[0] + sl * p.k2_s[1]) : (uint64_t)safe_p;
        const uint32_t lat_lo = (uint32_t)lat_row, lat_hi = (uint32_t)(lat_row >> 32);
        const uint32_t rope_lo = (uint32_t)rope_row, rope_hi = (uint32_t)(rope_row >> 32);
#pragma unroll
        for (int j = 0; j < kLatCopiesPerWave; ++j) {
            const int kk = lat_copy_key(wave, j);  // uniform
            const uint64_t row = lane_u64(lat_hi, lat_lo, kk);
            const __amdgpu_buffer_rsrc_t rsrc =
                __builtin_amdgcn_make_buffer_rsrc((void *)row, (short)0, kLatRowBytes, kBufferFlags);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void *)(lat_slot + lat_copy_lds(kk)), 16,
                lat_copy_src(kk, lane), 0, 0, kStreamPolicy);
        }
        const int v0 = base + rope_copy_key(wave, 0);  // uniform: first key of this wave's rotary group
        const int nv = min(max(t1 - v0, 0), 8);
        const uint64_t row = lane_u64(rope_hi, rope_lo, rope_copy_key(wave, 0));
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void *)row, (short)0, (int)rope_copy_records(nv, rope_stride), kBufferFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void *)(rope_slot + rope_copy_lds(wave)), 16,
            (int)rope_copy_src(wave, lane, rope_stride), 0, 0, kStreamPolicy);
    };

    // Per-lane LDS offsets inside a slot (mla_layout.h, the split forms): a base and a rotation per
    // lane, one XOR and one shifted add per read, and a compile-time offset that fits the DS
    // instruction's immediate field.
    // The values pass through an empty asm statement at every tile (opaque()), so that the
    // compiler computes each read's offset at the read instead of hoisting all of them out of the
    // loop into registers it does not have.
    int klb = k_lat_base(lane), klr = k_lat_rot(lane);
    int krb = k_rope_base(lane), krr = k_rope_rot(lane);
    int vb_0 = v_base(lane, 0) + 256 * wave, vb_1 = v_base(lane, 1) + 256 * wave, vr = v_rot(lane);
    auto opaque = [&]() {
        asm volatile("" : "+v"(klb), "+v"(klr), "+v"(krb), "+v"(krr), "+v"(vb_0), "+v"(vb_1), "+v"(vr));
    };

    float m = -INFINITY, l = 0.f, lf = 0.f;  // row col's reference max and sums (this lane's keys)
    bool overflow = false;
    // o[hb * 4 + s]: row block hb, slab s (columns 128 wave + 32 s ..); o[0 .. kVgprAcc-1] are
    // matrix-core accumulators, o[kVgprAcc] is summed by the VALU.
    f32x16 o[kAcc];
    // Zeros are produced as a product with zero operands: every value that reaches the loop-carried
    // accumulators then comes out of the matrix core, and the compiler keeps them in the
    // accumulation registers for the whole loop (a plain 0.f start made it carry them in ordinary
    // registers and copy them over at every iteration).
    auto clear = [&]() {
#pragma unroll
        for (int a = 0; a < kVgprAcc; ++a) o[a] = mfma(u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}, f32x16{});
#pragma unroll
        for (int j = 0; j < 16; ++j) o[kVgprAcc][j] = 0.f;
    };
    clear();

    // Scores of tile `base` (base-2 units, masked) for row col of this wave's block, 16 keys of
    // this lane. LDS operand reads run kPipe matrix products ahead of their use.
    auto k_operand = [&](const lds_u8 *cur, const lds_u8 *rcur, int ks) -> u32x4 {
        return lds16(ks < kLatKs ? cur + (klb + 32 * ((ks & 7) ^ klr)) + 256 * (ks >> 3)
                                 : rcur + (krb + 32 * ((ks - kLatKs) ^ krr)));
    };
    auto scores = [&](const lds_u8 *cur, const lds_u8 *rcur, int base, float (&sv)[16]) {
        opaque();
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
            // key of element j: base + acc_row(lane, j) = (base + 4 half) + 8 (j / 4) + j % 4
            const int pos0 = base + 4 * half;
            const int lim = min(t1, hi_r);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int pos = pos0 + 8 * (j >> 2) + (j & 3);
                sv[j] = (pos < lim && pos >= lo_r) ? sv[j] : -INFINITY;
            }
        }
    };

    // value operand of key step t, slab s of this wave's columns (global slab 4 wave + s)
    auto v_operand = [&](const lds_u8 *cur, int t, int s) -> u32x4 {
        const int rot = 64 * (s ^ vr);
        s16x4 part[2];
#pragma unroll
        for (int rd = 0; rd < 2; ++rd)
            part[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(cur + ((rd ? vb_1 : vb_0) + rot) + 16384 * t));
        return __builtin_bit_cast(u32x4, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    lds_u8 *const pbuf = (lds_u8 *)s_p;

    auto compute = [&](const lds_u8 *cur, const lds_u8 *rcur, int base) {
        float sv[16];
        scores(cur, rcur, base, sv);
        // the first value operands do not depend on P: they load while the softmax runs
        u32x4 vb0 = v_operand(cur, 0, 0), vb1 = v_operand(cur, 0, 1);
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
        // this wave's rows' P, as the A operands of key steps 0 and 1, to every wave
#pragma unroll
        for (int t = 0; t < kKeySteps; ++t)
            *(__attribute__((address_space(3))) u32x4 *)(pbuf + p_off(wave, t, lane)) =
                u32x4{pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]};
        __builtin_amdgcn_s_waitcnt(kLgkmZero);
        asm volatile("s_barrier" ::: "memory");
        // products in order: key step t, slab s, row block hb (i = 16 t + 4 s + hb); the value
        // operand (t, s) serves 4 consecutive products, the P operands of step t all 16. Each
        // value operand is read two slabs ahead; each P operand of step 1 replaces its step-0
        // operand right after that operand's last product.
        u32x4 pa[kBlocks];
#pragma unroll
        for (int hb = 0; hb < kBlocks; ++hb) pa[hb] = lds16(pbuf + p_off(hb, 0, lane));
        f32x16 part;
#pragma unroll
        for (int t = 0; t < kKeySteps; ++t) {
#pragma unroll
            for (int s = 0; s < kSlabsPerWave; ++s) {
                const u32x4 vb = s % 2 ? vb1 : vb0;
#pragma unroll
                for (int hb = 0; hb < kBlocks; ++hb) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int a = hb * kSlabsPerWave + s;
                    if (a < kVgprAcc)
                        o[a] = mfma(pa[hb], vb, o[a]);
                    else
                        part = mfma(pa[hb], vb, t == 0 ? f32x16{} : part);
                    if (t + 1 < kKeySteps && s == kSlabsPerWave - 1) pa[hb] = lds16(pbuf + p_off(hb, t + 1, lane));
                }
                const int nt = t + (s + 2) / kSlabsPerWave, ns = (s + 2) % kSlabsPerWave;
                if (nt < kKeySteps) {
                    if (s % 2)
                        vb1 = v_operand(cur, nt, ns);
                    else
                        vb0 = v_operand(cur, nt, ns);
                }
            }
        }
        o[kVgprAcc] += part;
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
    // of tile base + 3*32 then overwrites, and every read of the probabilities of the previous
    // tile. Copies past the end read nothing or the query row, so every step issues the same
    // number of copies and the vmcnt count is exact. At the end every copy has landed and every
    // read is done.
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

    // ---- row sums of every row, then o_s = acc / l for this wave's columns of all rows and
    // lse_s = (m + log2 lf) * ln 2 for this wave's score rows
    l = pair_sum(l);
    lf = pair_sum(lf);
    if (half == 0) s_l[wave * kRowsPerWave + col] = l;
    if (half == 0 && col < nr) {
        const float ms = (m == -INFINITY) ? 0.f : m;
        p.part_lse[out_row(wave, col) * S + split] =
            l > 0.f ? (ms + __builtin_amdgcn_logf(lf)) * 0.69314718055994531f : -INFINITY;
    }
    __syncthreads();
    // The accumulators hold one column per lane; the partial rows go out as 16-byte stores of four
    // columns, transposed through this wave's ring slot (free since the loop's last barrier): one
    // row block (32 rows x 128 columns) at a time.
    lds_u8 *slot = wave == 0 ? (lds_u8 *)s_lat0 : wave == 1 ? (lds_u8 *)s_lat1 : wave == 2 ? (lds_u8 *)s_lat2 : (lds_u8 *)s_lat3;
#pragma unroll
    for (int hb = 0; hb < kBlocks; ++hb) {
        const int nb = rows_of(hb);
        float inv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float lr = s_l[hb * kRowsPerWave + acc_row(lane, j)];
            inv[j] = lr > 0.f ? 1.f / lr : 0.f;
        }
#pragma unroll
        for (int s = 0; s < kSlabsPerWave; ++s)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                *(__attribute__((address_space(3))) float *)(slot + stage_write_off(lane, j, s)) =
                    o[hb * kSlabsPerWave + s][j] * inv[j];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < kRowsPerWave / 2; ++i) {
            const int r = 2 * i + half;
            const f32x4 v = *(const __attribute__((address_space(3))) f32x4 *)(slot + stage_read_off(lane, i));
            if (r < nb)
                *reinterpret_cast<f32x4 *>(p.part_o + (out_row(hb, r) * S + split) * kLatent + kColsPerWave * wave +
                                           4 * col) = v;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace

hipError_t launch_partial_mla(const PartialParams &p, hipStream_t stream) {
    const dim3 grid(p.num_splits * p.row_blocks * p.batch);
    hipLaunchKernelGGL(mla_partial_kernel, grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ad
