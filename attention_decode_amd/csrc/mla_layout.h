// mla_layout.h -- where the MLA partial pass puts things in LDS and where its copies read from.
//
// The kernel (mla_mfma.hip) and a host-side bounds check (tests/mla_layout_check.cpp) both take
// every offset from these functions, so the check covers exactly the arithmetic the kernel runs:
// that each HBM -> LDS copy reads only inside the key row it is meant to read and lands inside
// its ring slot, and that every operand read, operand exchange and staging access stays inside
// its LDS object.
//
// A ring slot holds one tile of kTile keys: the latent rows (512 bf16 = 64 chunks of 16 bytes per
// key) in one LDS object and the rotary rows (64 bf16 = 8 chunks per key) in another. Chunk c of
// key k sits at position c ^ lat_swz(k) (latent) or c ^ rope_swz(k) (rotary) of the key's row, so
// that the score-operand reads (16 keys, one chunk each) and the transposing value reads (4 keys x
// 4 chunks per 32 lanes) hit distinct banks.
#pragma once

#include <stdint.h>

#ifdef __HIP__
#define AD_HD __host__ __device__ __forceinline__
#else
#define AD_HD inline
#endif

namespace ad {
namespace mla {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;                  // query rows whose scores a wave computes
constexpr int kRows = kWaves * kRowsPerWave;      // query rows per work unit
constexpr int kTile = 32;                         // keys per tile
constexpr int kLatent = 512, kRope = 64;          // latent (= value) and rotary widths
constexpr int kLatRowBytes = kLatent * 2;         // 1024
constexpr int kRopeRowBytes = kRope * 2;          // 128
constexpr int kLatBytes = kTile * kLatRowBytes;   // latent object of a slot: 32 KB
constexpr int kRopeBytes = kTile * kRopeRowBytes; // rotary object of a slot: 4 KB
constexpr int kSlots = 4;                         // ring depth: one tile in use, three in flight
constexpr int kColsPerWave = kLatent / kWaves;    // value columns whose products a wave accumulates
constexpr int kSlabsPerWave = kColsPerWave / 32;  // 32-column output slabs per wave (4)
constexpr int kKeySteps = kTile / 16;             // 16-key steps of the value product per tile (2)
// P exchange: every wave's probabilities of its 32 rows, as the A operands of the value product
// (one 16-byte word per lane and key step), for all 4 row blocks: 4 x 2 x 64 x 16 bytes.
constexpr int kPBytes = kWaves * kKeySteps * 64 * 16;
// Staging of one row block's output columns for the stores: 32 rows of kStageStride floats.
constexpr int kStageStride = kColsPerWave + 4;
// Page ids one split stages (the host plans splits so that a split's pages fit).
constexpr int kMapCapacity = 260;
// Copies one wave issues per tile: 8 latent rows and one rotary group of 8 keys.
constexpr int kLatCopiesPerWave = kTile / kWaves;
constexpr int kCopiesPerWave = kLatCopiesPerWave + 1;

static_assert(kRowsPerWave * kStageStride * 4 <= kLatBytes, "a staged row block fits a latent slot");
static_assert(kTile % 16 == 0, "tiles start on 16-key boundaries, so a rotary group of 8 keys stays in one page");

AD_HD int lat_swz(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }  // < 16, depends on k % 16
AD_HD int rope_swz(int k) { return (k >> 1) & 7; }                     // < 8, depends on k % 16

// ---- HBM -> LDS copies (16 bytes per lane; lane i of a copy writes LDS bytes [16 i, 16 i + 16)
// after the copy's LDS base)
// Latent copy j of wave w copies key lat_copy_key(w, j) of the tile.
AD_HD int lat_copy_key(int wave, int j) { return wave + kWaves * j; }
// LDS base of that copy inside the latent object, and the byte its lane i reads inside the key's
// 1 KB latent row (the copy's buffer range is that row: kLatRowBytes).
AD_HD int lat_copy_lds(int key) { return key * kLatRowBytes; }
AD_HD int lat_copy_src(int key, int lane) { return (lane ^ lat_swz(key)) << 4; }
// Rotary copy of wave w: keys 8w .. 8w + 7 of the tile, lane i bringing chunk (i % 8) of key
// 8w + i / 8. Those keys are consecutive slots of one page, so the source is the rotary row of key
// 8w plus (i / 8) slot strides. Its buffer range ends after the last key inside the split
// (rope_copy_records); lanes past it read zeros.
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
// Score operand (A of S^T = K Q^T): lane l, k-step ks < 32 reads latent chunk 2 ks + l / 32 of key
// l % 32; k-step 32 + i reads rotary chunk 2 i + l / 32. 16 bytes each.
AD_HD int k_lat_off(int lane, int ks) {
    const int key = lane & 31, chunk = 2 * ks + (lane >> 5);
    return key * kLatRowBytes + ((chunk ^ lat_swz(key)) << 4);
}
AD_HD int k_rope_off(int lane, int i) {
    const int key = lane & 31, chunk = 2 * i + (lane >> 5);
    return key * kRopeRowBytes + ((chunk ^ rope_swz(key)) << 4);
}
// Value operand (B of O += P V) of key step t (keys 16 t .. 16 t + 15) and output slab s
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
// The same offsets from two per-lane values each, as the kernel computes them (one XOR and one
// shifted add per read instead of a table of offsets per lane):
//   k_lat_off(l, ks)     = k_lat_base(l) + 32 ((ks % 8) ^ k_lat_rot(l)) + 256 (ks / 8)
//   k_rope_off(l, i)     = k_rope_base(l) + 32 (i ^ k_rope_rot(l))
//   v_off(l, t, rd, s)   = v_base(l, rd) + 64 ((s % 4) ^ v_rot(l)) + 16384 t + 256 (s / 4)
AD_HD int k_lat_base(int lane) {
    const int key = lane & 31;
    return key * kLatRowBytes + (((lane >> 5) ^ (lat_swz(key) & 1)) << 4);
}
AD_HD int k_lat_rot(int lane) { return lat_swz(lane & 31) >> 1; }
AD_HD int k_lat_off_split(int lane, int ks) {
    return k_lat_base(lane) + 32 * ((ks & 7) ^ k_lat_rot(lane)) + 256 * (ks >> 3);
}
AD_HD int k_rope_base(int lane) {
    const int key = lane & 31;
    return key * kRopeRowBytes + (((lane >> 5) ^ (rope_swz(key) & 1)) << 4);
}
AD_HD int k_rope_rot(int lane) { return rope_swz(lane & 31) >> 1; }
AD_HD int k_rope_off_split(int lane, int i) { return k_rope_base(lane) + 32 * (i ^ k_rope_rot(lane)); }
AD_HD int v_base(int lane, int rd) {
    const int half = lane >> 5;
    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int key = 8 * rd + tr_row;
    return key * kLatRowBytes + ((tr_chunk ^ (lat_swz(key) & 3)) << 4) + ((lane & 1) << 3);
}
AD_HD int v_rot(int lane) { return lat_swz(4 * (lane >> 5) + ((lane & 15) >> 2)) >> 2; }
AD_HD int v_off_split(int lane, int t, int rd, int s) {
    return v_base(lane, rd) + 64 * ((s & 3) ^ v_rot(lane)) + 16384 * t + 256 * (s >> 2);
}
// P exchange: the 16-byte A operand of row block hb, key step t, lane l.
AD_HD int p_off(int hb, int t, int lane) { return ((hb * kKeySteps + t) * 64 + lane) << 4; }

// ---- output staging (a latent slot of the ring, free after the loop)
// Value accumulator element j of lane l in slab s: row 8 (j / 4) + 4 (l / 32) + j % 4, column
// 32 s + l % 32 of the wave's columns.
AD_HD int acc_row(int lane, int j) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }
AD_HD int stage_write_off(int lane, int j, int s) {
    return (acc_row(lane, j) * kStageStride + 32 * s + (lane & 31)) * 4;
}
// Read-back for the stores: pass i, lane l takes row 2 i + l / 32, columns 4 (l % 32) .. + 3.
AD_HD int stage_read_off(int lane, int i) { return ((2 * i + (lane >> 5)) * kStageStride + 4 * (lane & 31)) * 4; }

}  // namespace mla
}  // namespace ad
