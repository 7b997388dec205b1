// mla_layout.h -- where the MLA partial pass puts things in LDS and where its copies read from.
//
// The kernel (mla_mfma.hip) and a host-side bounds check (tests/mla_layout_check.cpp) both take
// every offset from these functions, so the check covers exactly the arithmetic the kernel runs:
// that each HBM -> LDS copy reads only inside the key row it is meant to read and lands inside
// its ring slot, that every chunk a copy brings is where the operand reads look for it, and that
// every operand read, probability exchange and staging access stays inside its LDS object.
//
// A work unit is 64 query rows of one sequence and split, on 8 waves (two per SIMD). Wave w
// scores query rows 16 (w % 4) .. + 15 against keys 16 (w / 4) .. + 15 of each 32-key tile
// (v_mfma_f32_16x16x32_bf16, K as the A operand from LDS, Q as the B operand in registers), and
// accumulates value columns 64 w .. 64 w + 63 of all 64 rows (v_mfma_f32_32x32x16_bf16, the
// probabilities of every wave as the A operand from LDS, V as the B operand from LDS).
//
// A ring slot holds one tile of kTile keys: the latent rows (512 bf16 = 64 chunks of 16 bytes per
// key) in one LDS object and the rotary rows (64 bf16 = 8 chunks per key) in another. Chunk c of
// key k sits at position c ^ lat_swz(k) (latent) or c ^ rope_swz(k) (rotary) of the key's row, so
// that the score-operand reads (16 keys, one chunk each, per 16 lanes) and the transposing value
// reads (4 keys x 4 chunks per 32 lanes) hit distinct banks in a model of 32 or of 64 banks.
#pragma once

#include <stdint.h>

#ifdef __HIP__
#define AD_HD __host__ __device__ __forceinline__
#else
#define AD_HD inline
#endif

namespace ad {
namespace mla {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 64;                         // query rows per work unit
constexpr int kScoreRows = 16;                    // query rows a wave scores
constexpr int kScoreBlocks = kRows / kScoreRows;  // 4: wave w scores row block w % 4 ...
constexpr int kKeyHalves = 2;                     // ... against key half w / 4 of each tile
constexpr int kTile = 32;                         // keys per tile
constexpr int kLatent = 512, kRope = 64;          // latent (= value) and rotary widths
constexpr int kLatRowBytes = kLatent * 2;         // 1024
constexpr int kRopeRowBytes = kRope * 2;          // 128
constexpr int kLatBytes = kTile * kLatRowBytes;   // latent object of a slot: 32 KB
constexpr int kRopeBytes = kTile * kRopeRowBytes; // rotary object of a slot: 4 KB
// Ring depth: the main loop has two tiles in use (value products, scores) and two in flight; the
// exact pass's score-only loop one in use and three in flight.
constexpr int kSlots = 4;
constexpr int kColsPerWave = kLatent / kWaves;    // value columns whose products a wave accumulates (64)
constexpr int kSlabsPerWave = kColsPerWave / 32;  // 32-column output slabs per wave (2)
constexpr int kValueBlocks = kRows / 32;          // 32-row blocks of the value product (2)
constexpr int kKeySteps = kTile / 16;             // 16-key steps of the value product per tile (2)
// P exchange: the probabilities of all 64 rows as the A operands of the value product (one
// 16-byte word per lane, 32-row block and key step): 2 x 2 x 64 x 16 bytes.
constexpr int kPBytes = kValueBlocks * kKeySteps * 64 * 16;
// Staging of one 32-row block of a wave's output columns for the stores: 32 rows of
// kStageStride floats, in half a latent slot (wave w: slot w / 2, half w % 2).
constexpr int kStageStride = kColsPerWave + 4;
constexpr int kStageBytes = 32 * kStageStride * 4;
constexpr int kStageHalf = kLatBytes / 2;
// Page ids one split stages (the host plans splits so that a split's pages fit).
constexpr int kMapCapacity = 260;
// Copies per tile: wave w copies latent rows w, w + 8, w + 16, w + 24 (16 bytes per lane); waves
// 0 .. 3 also copy one group of 8 rotary rows each (16 bytes per lane).
constexpr int kLatCopiesPerWave = kTile / kWaves;
constexpr int kRopeWaves = kTile / 8;

static_assert(kStageBytes <= kStageHalf, "a staged row block fits half a latent slot");
static_assert(kWaves <= 2 * kSlots, "two waves stage in each latent slot");
static_assert(kTile % 16 == 0, "tiles start on 16-key boundaries, so a rotary group of 8 keys stays in one page");

// Latent: a permutation of 0..15 over any 16 consecutive keys whose low 3 bits are a permutation
// over any 8 (the score-operand reads of 16 keys at one chunk are conflict-free in a model that
// serves 8 and in one that serves 16 lanes of 16 bytes per cycle), and whose bits 1-2 and bits 2-3
// are each distinct over keys 4j .. 4j + 3 (the transposing reads of 4 keys x 2 or 4 chunks
// likewise).
AD_HD int lat_swz(int k) {
    constexpr int kBase = (0 << 0) | (6 << 4) | (10 << 8) | (12 << 12);  // 0, 6, 10, 12 by k % 4
    return ((kBase >> (4 * (k & 3))) & 15) ^ ((k >> 2) & 3);
}
// Rotary (rows of 8 chunks, so 2 keys per 256 bytes): distinct over any 8 consecutive keys, and
// over the 8 even (odd) keys of any 16.
AD_HD int rope_swz(int k) { return (k & 7) ^ ((k >> 3) & 1); }

// ---- HBM -> LDS copies (16 bytes per lane; lane i of a copy writes LDS bytes [16 i, 16 i + 16)
// after the copy's LDS base)
// Latent copy j of wave w copies key lat_copy_key(w, j) of the tile.
AD_HD int lat_copy_key(int wave, int j) { return wave + kWaves * j; }
// LDS base of that copy inside the latent object, and the byte its lane i reads inside the key's
// 1 KB latent row (the copy's buffer range is that row: kLatRowBytes).
AD_HD int lat_copy_lds(int key) { return key * kLatRowBytes; }
AD_HD int lat_copy_src(int key, int lane) { return (lane ^ lat_swz(key)) << 4; }
// Rotary copy of wave w < kRopeWaves: keys 8w .. 8w + 7 of the tile, lane i bringing chunk
// (i % 8) of key 8w + i / 8. Those keys are consecutive slots of one page, so the source is the
// rotary row of key 8w plus (i / 8) slot strides. Its buffer range ends after the last key inside
// the split (rope_copy_records); lanes past it read zeros.
AD_HD int rope_copy_key(int wave, int lane) { return 8 * wave + (lane >> 3); }
AD_HD int rope_copy_lds(int wave) { return wave * 8 * kRopeRowBytes; }
AD_HD int64_t rope_copy_src(int wave, int lane, int64_t slot_stride_bytes) {
    return (int64_t)(lane >> 3) * slot_stride_bytes + (((lane & 7) ^ rope_swz(rope_copy_key(wave, lane))) << 4);
}
// nv: keys of the group inside the split (0 .. 8)
AD_HD int64_t rope_copy_records(int nv, int64_t slot_stride_bytes) {
    return nv > 0 ? (int64_t)(nv - 1) * slot_stride_bytes + kRopeRowBytes : 0;
}

// ---- operand reads
// Score operand (A of S^T = K Q^T) of the wave scoring key half kh: lane l, k-step ks < 16 reads
// latent chunk 4 ks + l / 16 of key 16 kh + l % 16; k-step 16 + i reads rotary chunk 4 i + l / 16.
// 16 bytes each.
AD_HD int k_lat_off(int kh, int lane, int ks) {
    const int key = 16 * kh + (lane & 15), chunk = 4 * ks + (lane >> 4);
    return key * kLatRowBytes + ((chunk ^ lat_swz(key)) << 4);
}
AD_HD int k_rope_off(int kh, int lane, int i) {
    const int key = 16 * kh + (lane & 15), chunk = 4 * i + (lane >> 4);
    return key * kRopeRowBytes + ((chunk ^ rope_swz(key)) << 4);
}
// The latent offsets from four per-lane values (the kernel keeps them in registers; the 256-byte
// steps fit the DS instruction's immediate field):
//   k_lat_off(kh, l, ks) = k_lat_lane(kh, l, ks % 4) + 256 (ks / 4)
AD_HD int k_lat_lane(int kh, int lane, int j) {
    const int key = 16 * kh + (lane & 15), sw = lat_swz(key);
    return key * kLatRowBytes + (((lane >> 4) ^ (sw & 3)) << 4) + 64 * (j ^ (sw >> 2));
}
// Value operand (B of O += P V) of key step t (keys 16 t .. 16 t + 15) and global output slab s
// (columns 32 s .. 32 s + 31), as two transposing 8-byte reads rd = 0, 1 (ds_read_b64_tr_b16:
// keys 16 t + 8 rd + (0..7) of the step); the key order matches the P operand's.
AD_HD int v_off(int lane, int t, int rd, int s) {
    const int half = lane >> 5;
    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int key = 16 * t + 8 * rd + tr_row;
    const int chunk = 4 * s + tr_chunk;
    return key * kLatRowBytes + ((chunk ^ lat_swz(key)) << 4) + ((lane & 1) << 3);
}
// The same for slab sl of wave w's columns, from one per-lane value per (rd, sl):
//   v_off(l, t, rd, 2 w + sl) = v_lane(w, l, rd, sl) + 16384 t
AD_HD int v_lane(int wave, int lane, int rd, int sl) {
    const int half = lane >> 5;
    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int key = 8 * rd + tr_row, sw = lat_swz(key), s = kSlabsPerWave * wave + sl;
    return key * kLatRowBytes + ((tr_chunk ^ (sw & 3)) << 4) + ((lane & 1) << 3) + 64 * ((s & 3) ^ (sw >> 2)) +
           256 * (s >> 2);
}
// P exchange: the 16-byte A operand of 32-row block hb and key step t for lane l (row l % 32 of
// the block; reduction elements e = 0..7 are keys 16 t + 8 (e / 4) + 4 (l / 32) + e % 4).
AD_HD int p_off(int hb, int t, int lane) { return ((hb * kKeySteps + t) * 64 + lane) << 4; }
// Where lane l of wave w writes its 4 probabilities (keys 16 (w / 4) + 4 (l / 16) + 0..3 of query
// row 16 (w % 4) + l % 16, 8 bytes): inside the word of that row and key step.
AD_HD int p_write_off(int wave, int lane) {
    const int rblk = wave & 3, g = lane >> 4;
    const int word = 16 * (rblk & 1) + (lane & 15) + 32 * (g & 1);
    return p_off(rblk >> 1, wave >> 2, word) + 8 * (g >> 1);
}

// ---- output staging (half a latent slot of the ring, free after the loop)
// Value accumulator element j of lane l in slab sl: row 8 (j / 4) + 4 (l / 32) + j % 4 of the
// 32-row block, column 32 sl + l % 32 of the wave's columns.
AD_HD int acc_row(int lane, int j) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }
AD_HD int stage_write_off(int lane, int j, int sl) {
    return (acc_row(lane, j) * kStageStride + 32 * sl + (lane & 31)) * 4;
}
// Read-back for the stores: pass i < 8, lane l takes row 4 i + l / 16, columns 4 (l % 16) .. + 3.
AD_HD int stage_read_off(int lane, int i) { return ((4 * i + (lane >> 4)) * kStageStride + 4 * (lane & 15)) * 4; }

}  // namespace mla
}  // namespace ad
