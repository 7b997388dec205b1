// mla_mfma.hip -- partial split-KV pass of multi-head latent attention (MLA) on the matrix cores.
//
// What it computes (FlashInfer mla.cuh, the MLA decode kernel): one shared latent KV head per
// token, ckv (512 values) and kpe (64 rotary values). A query head's score is
//   s = scale * (q_nope . ckv + q_pe . kpe)
// and its value vector is the same ckv row. Per work unit (split s, block of up to 64 query rows,
// sequence b) the kernel writes the attention of those rows over the split's keys as a normalised
// partial o_s = acc / l (512 values) and a natural-log LSE, like the other split-KV passes
// (mslk splitk_kernels.py, _fwd_kernel_splitK epilogue). Rows are r = t * H + h.
//
// Design for CDNA4 (LDS layout and copy addressing: mla_layout.h):
//
//   * Two waves per SIMD. A unit's state is its queries (1152 bytes per row) and its value
//     accumulators (2048 bytes per row); at 64 rows per unit that is 200 KB, and 8 waves of 256
//     registers hold it with room for the operands, so the two waves of a SIMD cover each
//     other's softmax, barriers and copy issue with their matrix products. (At 128 rows the state
//     alone takes 400 of the compute unit's 512 KB of registers: one wave per SIMD.)
//   * Scores by row and key blocks, values by columns. Wave w scores query rows 16 (w % 4) .. + 15
//     against keys 16 (w / 4) .. + 15 of each 32-key tile on v_mfma_f32_16x16x32_bf16: its Q
//     (576 bf16 per row) is the B operand in 72 registers, K comes from LDS as the A operand. The
//     value product is split the other way: wave w accumulates output columns 64 w .. 64 w + 63
//     of all 64 rows on v_mfma_f32_32x32x16_bf16, reading its slice of each V row from LDS. The
//     probabilities cross between the waves through LDS once per tile (4 KB of bf16 A operands),
//     the sharding of mla.cuh's compute_mla_pv, where each warpgroup multiplies its own slice of
//     the 512 latent columns with the gathered P.
//   * The two row blocks of a (sequence, split) piece are consecutive work units on one XCD: they
//     run side by side and the second reads the piece's keys from that XCD's L2.
//   * Each row's reference max is fixed at its first tile with a visible key and never moves, so
//     the value accumulators are never rescaled, and a wave can accumulate rows whose scores
//     another wave computed without any per-tile exchange of maxima. The two waves scoring a row
//     (one per key half) exchange their maxima through LDS on the tiles where a row may first see
//     a key, so both take the same reference. Later scores may exceed it by up to 2^64
//     (probabilities up to 2^64 stay finite in bf16 and fp32); a row that goes further makes the
//     work group recompute its unit exactly: one pass for every row's true max, then the main
//     pass with that max.
//   * Tiles (32 keys: 32 KB latent + 4 KB rotary) are copied HBM -> LDS with buffer_load ... lds
//     (no register staging) into a 4-slot ring. The loop is software-pipelined with one barrier
//     per tile: step i computes tile i's scores and softmax and tile i-1's value products, whose
//     probabilities that step's barrier published (two probability buffers, even and odd tiles),
//     so the softmax's vector work and the copy issue run beside matrix products. Slots hold tile
//     i-1 (values), tile i (scores) and tiles i+1, i+2 (in flight). A wave waits for its own copies
//     of tile i (vmcnt) and the barrier publishes everybody's.
//   * Keys past the split or the sequence are never read from the cache (their copies read the
//     unit's own query row) and get probability 0.
#include "ad_internal.h"
#include "mfma_util.h"
#include "mla_layout.h"

#include <limits.h>
#include <math.h>

namespace ad {
namespace {

using namespace mla;

constexpr int kKs = (kLatent + kRope) / 32;  // k-steps (32 values) of the score product
constexpr int kLatKs = kLatent / 32;
constexpr float kHeadroom = 64.f;
// Score-operand reads in flight ahead of the matrix products (6 or 8 measured no faster).
constexpr int kPipe = 4;
// The score product after which a step issues its copies (after the 9th or 13th measured slower).
constexpr int kIssueAt = 3;
// Independent accumulation chains of the score product (2 or 3 measured no faster).
constexpr int kChains = 1;

// s_waitcnt with vmcnt(n) and no wait on the other counters (gfx9 encoding).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// s_waitcnt lgkmcnt(0) with no wait on the other counters.
constexpr int kLgkmZero = 15 | (3 << 14) | (7 << 4);
// Buffer descriptor word 3 for raw (untyped, unswizzled) buffer accesses on the gfx9 family.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ u32x4 lds16(const lds_u8 *p) { return *(const __attribute__((address_space(3))) u32x4 *)p; }

// HBM -> LDS copy of 16 bytes per lane: lane i's bytes at `voffset` inside the buffer go to LDS
// bytes [16 i, 16 i + 16) after `lds` (M0), nontemporal (each line is read once). Written as
// inline assembly so that the compiler's wait insertion does not track the copy: this kernel
// waits for its copies itself (vmcnt, then a barrier) before any LDS read of the slot they fill,
// and the compiler, unable to follow the ring's slots through its loop, otherwise made reads wait
// for later tiles' copies as well (and for every copy in flight where only some waves copy). The
// copy writes no register. Copies unknown to the compiler only make its own vmcnt waits for its
// loads and stores stricter (the counter retires them in order). The descriptor's words come from
// lane reads (the vector unit writing scalar registers), which a buffer instruction may read only
// 5 wait states later; M0 needs 1: the s_nop provides both, since the compiler's hazard checks do
// not look inside the assembly.
__device__ __forceinline__ void copy_to_lds(u32x4 rsrc, int voffset, const lds_u8 *lds) {
    const uint32_t m0 = (uint32_t)(uintptr_t)lds;
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voffset), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}
// Raw buffer descriptor (gfx9 family): base address, stride 0, num_records bytes, raw access.
__device__ __forceinline__ u32x4 buffer_rsrc(uint64_t base, uint32_t num_records) {
    return u32x4{(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, num_records, (uint32_t)kBufferFlags};
}

// The 64-bit value held as (hi, lo) words in lane `l`. The lane read returns a signed int: each
// word is widened as unsigned, or a low word with bit 31 set would fill the high word with ones.
__device__ __forceinline__ uint64_t lane_u64(uint32_t hi, uint32_t lo, int l) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, l) << 32) |
           (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lo, l);
}

// Work-group placement. The dispatcher deals work groups to the 8 XCDs round robin (group L to
// XCD L % 8), and each XCD has its own L2. Unit u = ((b * splits + split) * row_blocks + rb) is
// given to the group that makes consecutive units share an XCD: the row blocks of a piece read
// its keys, and the splits of a sequence its queries, through one L2. A bijection of [0, N).
__device__ __forceinline__ int xcd_unit(int L, int N) {
    constexpr int kXcds = 8;
    const int per = N / kXcds, rem = N % kXcds, x = L % kXcds;
    return x * per + min(x, rem) + L / kXcds;
}

__global__ void __launch_bounds__(kThreads) mla_partial_kernel(const PartialParams p) {
    const int unit = xcd_unit(blockIdx.x, gridDim.x);
    const int rb = unit % p.row_blocks;
    const int split = (unit / p.row_blocks) % p.num_splits;
    const int b = unit / (p.row_blocks * p.num_splits);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rblk = wave % kScoreBlocks, kh = wave / kScoreBlocks;  // score rows and key half
    const int c16 = lane & 15, grp = lane >> 4;
    const int H = p.group, Q = p.q_len, R = H * Q, S = p.num_splits;
    const int L = p.seq_lens ? p.seq_lens[b] : p.kv_len_max;
    const int t0 = split * p.chunk;
    const int t1 = min(t0 + p.chunk, L);
    const int nrows = max(0, min(kRows, R - rb * kRows));  // valid rows of the unit
    auto out_row = [&](int r) -> int64_t {                  // r: row inside the unit
        const int ra = rb * kRows + r, t = ra / H, g = ra - t * H;
        return (int64_t)(b * Q + t) * p.num_q_heads + g;
    };

    if (t0 >= t1) {  // uniform over the work group
        if (p.write_empty) {
            for (int i = tid; i < nrows * kLatent; i += kThreads) {
                const int r = i / kLatent, d = i - r * kLatent;
                p.part_o[(out_row(r) * S + split) * kLatent + d] = 0.f;
            }
            for (int r = tid; r < nrows; r += kThreads) p.part_lse[out_row(r) * S + split] = -INFINITY;
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
    // probabilities of all rows, of even and odd tiles
    __shared__ __attribute__((aligned(16))) unsigned char s_p0[kPBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_p1[kPBytes];
    __shared__ float s_hmax[kKeyHalves][kRows];  // row maxima of each key half
    __shared__ float s_sum[2][kKeyHalves][kRows];  // row sums (bf16-rounded and fp32) of each key half
    __shared__ int s_flag[kWaves];

    const int map_shift = p.page_shift, map_mask = (1 << map_shift) - 1;
    const int map_first = t0 >> map_shift;
    {
        const int n = ((t1 - 1) >> map_shift) - map_first + 1;  // <= kMapCapacity (host plan)
        const int32_t *bt = p.block_table + b * p.bt_stride + map_first;
        for (int i = tid; i < n; i += kThreads) s_map[i] = bt[i];
    }
    __syncthreads();

    // ---- this lane's query row (row c16 of this wave's score block): B operand, 16 latent + 2
    // rotary k-steps, lane group grp taking 8 of each step's 32 values
    const uint16_t *q_nope = static_cast<const uint16_t *>(p.q);
    const uint16_t *q_pe = static_cast<const uint16_t *>(p.q2);
    const uint16_t *safe_n = q_nope + b * p.q_s[0];  // row (b, 0, 0): finite, always readable, 1 KB
    const uint16_t *safe_p = q_pe + b * p.q2_s[0];
    const int myrow = rblk * kScoreRows + c16;
    u32x4 qb[kKs];
    int lo_r = INT_MIN, hi_r = INT_MAX;
    if (myrow < nrows) {
        const int ra = rb * kRows + myrow, t = ra / H, g = ra - t * H;
        const uint16_t *qn = q_nope + b * p.q_s[0] + t * p.q_s[1] + g * p.q_s[2];
        const uint16_t *qp = q_pe + b * p.q2_s[0] + t * p.q2_s[1] + g * p.q2_s[2];
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks)
            qb[ks] = ks < kLatKs ? ld16(qn + 32 * ks + 8 * grp) : ld16(qp + 32 * (ks - kLatKs) + 8 * grp);
        const int qpos = L - Q + t;
        if (p.causal) hi_r = qpos + 1;
        if (p.window) lo_r = qpos - p.window + 1;
    } else {
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) qb[ks] = u32x4{0, 0, 0, 0};
    }
    // keys [lo_max, hi_min) are visible to every row of the unit
    const int r_first = rb * kRows, r_last = rb * kRows + nrows - 1;
    const int hi_min = p.causal ? L - Q + r_first / H + 1 : INT_MAX;
    const int lo_max = p.window ? L - Q + r_last / H - p.window + 1 : INT_MIN;
    // Every row that sees a key of the split sees one at or before exch_last (its first visible
    // key is max(t0, its window start) <= max(t0, lo_max)): tiles from there on need no exchange.
    int exch_last = max(t0, lo_max);

    // Q has landed before the first copy is issued. The compiler does not see the copies; seeing
    // Q's loads possibly in flight, it would wait for them inside the loop with counts that then
    // also wait for every copy in flight.
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));

    const uint16_t *ckv = static_cast<const uint16_t *>(p.k);
    const uint16_t *kpe = static_cast<const uint16_t *>(p.k2);

    // ---- copy tile [base, base + 32) of the split into a ring slot, HBM -> LDS with
    // buffer_load ... lds (mla_layout.h: lat_copy_*, rope_copy_*). Every descriptor covers only the
    // rows the copy may read, so the hardware range check confines it. Latent rows past the split
    // read the unit's query row instead. The buffer form of the LDS copy matters: the compiler
    // treats the global form as a possible LDS access of unknown order and would make every LDS
    // read wait for all. The copies are nontemporal (cache-policy bit 1): each reads whole lines
    // once.
    const int64_t rope_stride = p.k2_s[1] * 2;  // bytes between the rotary rows of two slots of a page
    // Page id of key base + i in lane i (i < 32; the last key of the split past its end), read one
    // step before the tile's copies are issued so that its LDS round trip is off their path.
    auto lookup = [&](int base) -> int {
        const int vlc = min(base + (lane & 31), t1 - 1);
        return s_map[(vlc >> map_shift) - map_first];
    };
    // Byte strides of the two pools; with all four below 2^32 (any page of up to 4 GB) a row
    // address is two 32 x 32 -> 64-bit multiply-adds.
    const uint64_t ks0 = 2 * (uint64_t)p.k_s[0], ks1 = 2 * (uint64_t)p.k_s[1];
    const uint64_t ks20 = 2 * (uint64_t)p.k2_s[0], ks21 = 2 * (uint64_t)p.k2_s[1];
    const bool narrow = ((ks0 | ks1 | ks20 | ks21) >> 32) == 0;  // uniform
    auto row_at = [&](const uint16_t *pool, uint64_t s0, uint64_t s1, int pg, int sl) -> uint64_t {
        if (narrow)
            return (uint64_t)(uint32_t)pg * (uint32_t)s0 + ((uint64_t)(uint32_t)sl * (uint32_t)s1 + (uint64_t)pool);
        return (uint64_t)pool + (uint64_t)(uint32_t)pg * s0 + (uint64_t)(uint32_t)sl * s1;
    };
    auto issue = [&](lds_u8 *lat_slot, lds_u8 *rope_slot, int base, int pg) {
        // Row addresses of key base + i in lane i (i < 32), computed once per tile on the vector
        // unit; each copy takes its row with a lane read. Keys past the split get the query row.
        // Block-table entries name pool pages, so they are non-negative.
        const int vl = base + (lane & 31);
        const int vlc = min(vl, t1 - 1);
        const int sl = vlc & map_mask;
        const uint64_t lat_row = vl < t1 ? row_at(ckv, ks0, ks1, pg, sl) : (uint64_t)safe_n;
        const uint32_t lat_lo = (uint32_t)lat_row, lat_hi = (uint32_t)(lat_row >> 32);
#pragma unroll
        for (int j = 0; j < kLatCopiesPerWave; ++j) {
            const int kk = lat_copy_key(wave, j);  // uniform
            const uint64_t row = lane_u64(lat_hi, lat_lo, kk);
            copy_to_lds(buffer_rsrc(row, kLatRowBytes), lat_copy_src(kk, lane), lat_slot + lat_copy_lds(kk));
        }
        if (wave < kRopeWaves) {  // uniform
            const uint64_t rope_row = vl < t1 ? row_at(kpe, ks20, ks21, pg, sl) : (uint64_t)safe_p;
            const int k0 = rope_copy_key(wave, 0);  // first key of this wave's rotary group
            const int nv = min(max(t1 - (base + k0), 0), 8);
            const uint64_t row = lane_u64((uint32_t)(rope_row >> 32), (uint32_t)rope_row, k0);
            copy_to_lds(buffer_rsrc(row, (uint32_t)rope_copy_records(nv, rope_stride)),
                            (int)rope_copy_src(wave, lane, rope_stride), rope_slot + rope_copy_lds(wave));
        }
    };

    // Wait until at most `tiles` tiles of this wave's copies are in flight (waves 0 .. 3 make one
    // more copy per tile than the others: their rotary group).
    auto wait_copies = [&](int tiles) {
        if (wave < kRopeWaves) {  // uniform
            if (tiles == 1)
                __builtin_amdgcn_s_waitcnt(vmcnt_only(kLatCopiesPerWave + 1));
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * (kLatCopiesPerWave + 1)));
        } else {
            if (tiles == 1)
                __builtin_amdgcn_s_waitcnt(vmcnt_only(kLatCopiesPerWave));
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kLatCopiesPerWave));
        }
    };

    // Per-lane LDS offsets inside a slot (mla_layout.h: k_lat_lane, k_rope_off, v_lane).
    int kl[4], kr[2], vo[2][kSlabsPerWave];
#pragma unroll
    for (int j = 0; j < 4; ++j) kl[j] = k_lat_lane(kh, lane, j);
#pragma unroll
    for (int i = 0; i < 2; ++i) kr[i] = k_rope_off(kh, lane, i);
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int sl = 0; sl < kSlabsPerWave; ++sl) vo[rd][sl] = v_lane(wave, lane, rd, sl);
    const int pw = p_write_off(wave, lane);

    float m = -INFINITY;                      // row myrow's reference max
    float runmax = -INFINITY;                 // largest score of this lane's keys so far
    float l = 0.f, lf = 0.f;                  // row sums of this lane's keys (bf16-rounded P, fp32 P)
    // o[hb][sl]: 32-row block hb, slab sl (columns 64 wave + 32 sl ..)
    f32x16 o[kValueBlocks][kSlabsPerWave];
    auto clear = [&]() {
#pragma unroll
        for (int hb = 0; hb < kValueBlocks; ++hb)
#pragma unroll
            for (int sl = 0; sl < kSlabsPerWave; ++sl) o[hb][sl] = f32x16{};
    };
    clear();

    // Scores of this wave's 16 keys of the tile for row c16 of its block: element i is key
    // 16 kh + 4 grp + i. LDS operand reads run kPipe matrix products ahead of their use.
    auto scores = [&](const lds_u8 *cur, const lds_u8 *rcur, int base, float (&sv)[4], auto &&hook) {
        auto k_operand = [&](int ks) -> u32x4 {
            return ks < kLatKs ? lds16(cur + kl[ks & 3] + 256 * (ks >> 2)) : lds16(rcur + kr[ks - kLatKs]);
        };
        // k-step ks accumulates into chain ks % kChains
        f32x4 sc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) sc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 ka[kPipe];
#pragma unroll
        for (int i = 0; i < kPipe; ++i) ka[i] = k_operand(i);
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
            // keeps the reads kPipe products ahead (left alone, the scheduler kept one or two)
            __builtin_amdgcn_sched_barrier(0);
            sc[ks % kChains] = mfma16(ka[ks % kPipe], qb[ks], sc[ks % kChains]);
            if (ks + kPipe < kKs) ka[ks % kPipe] = k_operand(ks + kPipe);
            // the copy issue's vector and scalar work runs while the matrix core works on the chain
            if (ks == kIssueAt) hook();
        }
#pragma unroll
        for (int c = 1; c < kChains; ++c) sc[0] += sc[c];
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = sc[0][i] * p.scale_log2;
        const bool full = base + kTile <= t1 && base >= lo_max && base + kTile <= hi_min;  // uniform
        if (!full) {
            const int pos0 = base + 16 * kh + 4 * grp;
            const int lim = min(t1, hi_r);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pos = pos0 + i;
                sv[i] = (pos < lim && pos >= lo_r) ? sv[i] : -INFINITY;
            }
        }
        runmax = fmaxf(runmax, fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    };

    // Both waves scoring row myrow take the max over the row's 32 keys of this tile (the
    // work group synchronises; uniform).
    auto exchange_max = [&](float mx) -> float {
        mx = pair16_max(pair_max(mx));  // lanes c16, c16 + 16, + 32, + 48: this wave's 16 keys
        if (grp == 0) s_hmax[kh][myrow] = mx;
        __builtin_amdgcn_s_waitcnt(kLgkmZero);  // an LDS-only barrier: the copies in flight stay in flight
        asm volatile("s_barrier" ::: "memory");
        return fmaxf(mx, s_hmax[kh ^ 1][myrow]);
    };

    // value operand of key step t, slab sl of this wave's columns
    auto v_operand = [&](const lds_u8 *cur, int t, int sl) -> u32x4 {
        s16x4 part[2];
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) part[rd] = ds_read_tr(cur + vo[rd][sl] + 16384 * t);
        return __builtin_bit_cast(u32x4, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // Softmax of one tile's scores against the row's reference max, and this lane's 4 probabilities
    // into the A operands of every wave's value product (pout).
    auto softmax = [&](const float (&sv)[4], int base, lds_u8 *pout) {
        if (base <= exch_last) {  // uniform
            const float mx = exchange_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
            if (m == -INFINITY) m = mx;  // first visible key of the row: o, l and lf are still exactly 0
        }
        const float ms = (m == -INFINITY) ? 0.f : m;
        const float p0 = exp2_fast(sv[0] - ms), p1 = exp2_fast(sv[1] - ms);  // exp2(-inf) = 0
        const float p2 = exp2_fast(sv[2] - ms), p3 = exp2_fast(sv[3] - ms);
        const uint32_t pk0 = pack_bf16(p0, p1), pk1 = pack_bf16(p2, p3);
        const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk0), ones, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk1), ones, l, false);
        lf += (p0 + p1) + (p2 + p3);
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *(__attribute__((address_space(3))) u32x2 *)(pout + pw) = u32x2{pk0, pk1};
    };
    // Value products of one tile: P of all rows from pin, V (this wave's columns) from the tile's
    // latent slot.
    auto values = [&](const lds_u8 *prev, const lds_u8 *pin) {
        u32x4 pa[kValueBlocks][kKeySteps], vb[kKeySteps][kSlabsPerWave];
#pragma unroll
        for (int t = 0; t < kKeySteps; ++t) {
#pragma unroll
            for (int hb = 0; hb < kValueBlocks; ++hb) pa[hb][t] = lds16(pin + p_off(hb, t, lane));
#pragma unroll
            for (int sl = 0; sl < kSlabsPerWave; ++sl) vb[t][sl] = v_operand(prev, t, sl);
        }
#pragma unroll
        for (int t = 0; t < kKeySteps; ++t)
#pragma unroll
            for (int sl = 0; sl < kSlabsPerWave; ++sl)
#pragma unroll
                for (int hb = 0; hb < kValueBlocks; ++hb) o[hb][sl] = mfma32(pa[hb][t], vb[t][sl], o[hb][sl]);
    };

    lds_u8 *const l0 = (lds_u8 *)s_lat0, *const l1 = (lds_u8 *)s_lat1, *const l2 = (lds_u8 *)s_lat2,
                 *const l3 = (lds_u8 *)s_lat3;
    lds_u8 *const q0 = (lds_u8 *)s_rope0, *const q1 = (lds_u8 *)s_rope1, *const q2 = (lds_u8 *)s_rope2,
                 *const q3 = (lds_u8 *)s_rope3;
    lds_u8 *const pb0 = (lds_u8 *)s_p0, *const pb1 = (lds_u8 *)s_p1;

    // The main pass, software-pipelined over a 4-slot ring with one barrier per tile. Step i
    // computes tile i's scores and softmax and tile i-1's value products (their probabilities were
    // published by this step's barrier), so that the softmax's vector work and the copy issue run
    // beside matrix products. Before the barrier each wave waits for its own copies of tile i
    // (vmcnt: those of tile i+1 may stay in flight) and for its probability writes of tile i-1; the
    // barrier also ends every read of tile i-2's slot, into which the step then copies tile i+2,
    // and every read of the probability buffer this step writes (tile i-2's). Copies past the end
    // read nothing or the query row, so every step issues the same number of copies and the vmcnt
    // count is exact. The first tile has no value products before it (base == t0); the last
    // tile's follow the loop.
    auto run_main = [&]() {
        int pg_next = 0;  // page ids of the next tile to copy (lookup)
        auto step = [&](lds_u8 *cur, lds_u8 *qcur, lds_u8 *prev, lds_u8 *fill, lds_u8 *qfill, lds_u8 *pout,
                        lds_u8 *pin, int base, bool has_prev) -> bool {
            if (base >= t1) return false;  // uniform
            wait_copies(1);
            __builtin_amdgcn_s_waitcnt(kLgkmZero);
            asm volatile("s_barrier" ::: "memory");
            float sv[4];
            scores(cur, qcur, base, sv, [&]() {
                issue(fill, qfill, base + 2 * kTile, pg_next);
                pg_next = lookup(base + 3 * kTile);
            });
            __builtin_amdgcn_sched_barrier(0);
            if (has_prev && base > t0) values(prev, pin);  // uniform
            softmax(sv, base, pout);
            return true;
        };
        auto round = [&](int base, bool first) -> bool {
            return step(l0, q0, l3, l2, q2, pb0, pb1, base, !first) &&
                   step(l1, q1, l0, l3, q3, pb1, pb0, base + kTile, true) &&
                   step(l2, q2, l1, l0, q0, pb0, pb1, base + 2 * kTile, true) &&
                   step(l3, q3, l2, l1, q1, pb1, pb0, base + 3 * kTile, true);
        };
        issue(l0, q0, t0, lookup(t0));
        issue(l1, q1, t0 + kTile, lookup(t0 + kTile));
        pg_next = lookup(t0 + 2 * kTile);
        for (int base = t0; round(base, false); base += 4 * kTile) {
        }
        // the last tile's value products
        const int last = (t1 - 1 - t0) / kTile;  // its index: slot last % 4, probabilities last % 2
        __builtin_amdgcn_s_waitcnt(kLgkmZero);
        asm volatile("s_barrier" ::: "memory");
        values((last & 3) == 0 ? l0 : (last & 3) == 1 ? l1 : (last & 3) == 2 ? l2 : l3, (last & 1) ? pb1 : pb0);
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        __syncthreads();
    };

    // Scores only, for the exact pass's maxima: the same ring with one barrier per tile and three
    // tiles in flight.
    auto run_max = [&]() {
        int pg_next = 0;
        auto step = [&](lds_u8 *cur, lds_u8 *qcur, lds_u8 *nxt, lds_u8 *qnxt, int base) -> bool {
            if (base >= t1) return false;  // uniform
            wait_copies(2);
            asm volatile("s_barrier" ::: "memory");
            float sv[4];
            scores(cur, qcur, base, sv, [&]() {
                issue(nxt, qnxt, base + 3 * kTile, pg_next);
                pg_next = lookup(base + 4 * kTile);
            });
            return true;
        };
        issue(l0, q0, t0, lookup(t0));
        issue(l1, q1, t0 + kTile, lookup(t0 + kTile));
        issue(l2, q2, t0 + 2 * kTile, lookup(t0 + 2 * kTile));
        pg_next = lookup(t0 + 3 * kTile);
        for (int base = t0;; base += 4 * kTile) {
            if (!step(l0, q0, l3, q3, base)) break;
            if (!step(l1, q1, l0, q0, base + kTile)) break;
            if (!step(l2, q2, l1, q1, base + 2 * kTile)) break;
            if (!step(l3, q3, l2, q2, base + 3 * kTile)) break;
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        __syncthreads();
    };

    for (int pass = 0;; ++pass) {
        run_main();
        // rows with no visible key keep m = runmax = -inf: -inf > -inf + 64 is false. The vote is
        // taken by every lane (each holds its own keys' largest score), then stored by one.
        const bool overflow = __builtin_amdgcn_ballot_w64(runmax > m + kHeadroom) != 0;
        if (lane == 0) s_flag[wave] = overflow;
        __syncthreads();
        int any = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) any |= s_flag[w];
        if (!any || pass > 0) break;  // uniform
        // rare: recompute exactly, with every row's true max over the split as its reference (no
        // score exceeds it, so the second main pass sets no reference and exchanges nothing)
        __syncthreads();  // every wave has read the flags
        runmax = -INFINITY;
        run_max();
        m = exchange_max(runmax);
        exch_last = INT_MIN;
        l = lf = 0.f;
        clear();
    }

    // ---- row sums of every row, then o_s = acc / l for this wave's columns of all rows and
    // lse_s = (m + log2 lf) * ln 2 for the score rows of the waves of key half 0
    l = pair16_sum(pair_sum(l));
    lf = pair16_sum(pair_sum(lf));
    if (grp == 0) {
        s_sum[0][kh][myrow] = l;
        s_sum[1][kh][myrow] = lf;
    }
    __syncthreads();
    if (kh == 0 && grp == 0 && myrow < nrows) {
        const float lt = s_sum[0][0][myrow] + s_sum[0][1][myrow];
        const float lft = s_sum[1][0][myrow] + s_sum[1][1][myrow];
        const float ms = (m == -INFINITY) ? 0.f : m;
        p.part_lse[out_row(myrow) * S + split] =
            lt > 0.f ? (ms + __builtin_amdgcn_logf(lft)) * 0.69314718055994531f : -INFINITY;
    }
    // The accumulators hold one column per lane; the partial rows go out as 16-byte stores of four
    // columns, transposed through half a ring slot per wave (free since the loop's last barrier):
    // one 32-row block at a time.
    lds_u8 *const slot = (wave >> 1) == 0   ? (lds_u8 *)s_lat0
                         : (wave >> 1) == 1 ? (lds_u8 *)s_lat1
                         : (wave >> 1) == 2 ? (lds_u8 *)s_lat2
                                            : (lds_u8 *)s_lat3;
    lds_u8 *const stage = slot + (wave & 1) * kStageHalf;
#pragma unroll
    for (int hb = 0; hb < kValueBlocks; ++hb) {
        float inv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int r = 32 * hb + acc_row(lane, j);
            const float lr = s_sum[0][0][r] + s_sum[0][1][r];
            inv[j] = lr > 0.f ? 1.f / lr : 0.f;
        }
#pragma unroll
        for (int sl = 0; sl < kSlabsPerWave; ++sl)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                *(__attribute__((address_space(3))) float *)(stage + stage_write_off(lane, j, sl)) =
                    o[hb][sl][j] * inv[j];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 32 * hb + 4 * i + grp;
            const f32x4 v = *(const __attribute__((address_space(3))) f32x4 *)(stage + stage_read_off(lane, i));
            if (r < nrows)
                *reinterpret_cast<f32x4 *>(p.part_o + (out_row(r) * S + split) * kLatent + kColsPerWave * wave +
                                           4 * c16) = v;
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
