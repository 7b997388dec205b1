// Host-side bounds check of the MLA partial pass's copies and LDS accesses, using the kernel's
// own offset functions (attention_decode_amd/csrc/mla_layout.h) and the kernel's address
// arithmetic restated for the host. For every work unit (sequence, split) of a problem and every
// tile the ring copies (three past the split's end included, as the kernel issues them), wave and
// lane, it checks:
//   - the page-id map a split stages fits its LDS array and every lookup stays inside it;
//   - every HBM -> LDS copy reads 16 bytes inside the row it is meant to read: the latent or rotary
//     row of the right key of the right page, or the unit's query row for keys past the split; a
//     rotary lane past its group's last key lies wholly outside the descriptor's range (it reads
//     zeros and touches no memory);
//   - every copy lands inside its ring slot, and every latent or rotary chunk it brings is where
//     the score operand reads expect it; every value operand read takes the key and chunk its
//     lane is meant to hold;
//   - every probability a wave writes is the one the value product's readers take for that row
//     and key, and no two writes land on one place;
//   - every operand read, probability exchange and staging access stays inside its LDS object,
//     and the per-lane forms of the offsets the kernel keeps in registers equal the plain ones;
//   - the score-operand and value-operand reads are free of bank conflicts in models of 32 and of
//     64 banks.
// Built with g++ and called through ctypes by tests/test_mla_layout.py; no GPU involved.
#include <stdint.h>
#include <stdio.h>

#include "mla_layout.h"

using namespace ad::mla;

namespace {

struct Geometry {
    int32_t batch, num_splits, chunk, page_size;
    const int32_t *seq_lens;     // [batch]
    const int32_t *block_table;  // [batch, bt_stride]
    int64_t bt_stride;
    int64_t pool_pages;
    int64_t ckv_s[2];   // element strides {page, slot} of the latent pool (bf16)
    int64_t kpe_s[2];   // of the rotary pool
    int64_t ckv_elems, kpe_elems;  // sizes of the pools in elements
    int64_t q_s0;       // element stride between sequences of q_nope (and q_pe: q2_s0)
    int64_t q2_s0;
    int64_t q_elems, q2_elems;
};

char *g_msg;
int g_len;
long g_checks;

bool bad(const char *what, int b, int split, int base, int wave, int lane, long long a, long long c) {
    snprintf(g_msg, g_len, "%s: b=%d split=%d tile=%d wave=%d lane=%d (%lld vs %lld)", what, b, split, base, wave,
             lane, a, c);
    return false;
}

// byte range [off, off + n) inside [lo, hi)
bool inside(long long off, long long n, long long lo, long long hi) { return off >= lo && off + n <= hi; }

bool check_lds(int wave) {
    const int kh = wave / kScoreBlocks;
    for (int lane = 0; lane < 64; ++lane) {
        for (int ks = 0; ks < kLatent / 32; ++ks) {
            const int o = k_lat_off(kh, lane, ks);
            const int split = k_lat_lane(kh, lane, ks & 3) + 256 * (ks >> 2);
            ++g_checks;
            if (o != split) return bad("score operand split form", 0, 0, ks, wave, lane, split, o);
            if (!inside(o, 16, 0, kLatBytes)) return bad("score operand outside the latent slot", 0, 0, ks, wave, lane, o, kLatBytes);
        }
        for (int i = 0; i < kRope / 32; ++i) {
            const int o = k_rope_off(kh, lane, i);
            if (!inside(o, 16, 0, kRopeBytes)) return bad("rotary operand outside the rotary slot", 0, 0, i, wave, lane, o, kRopeBytes);
        }
        for (int t = 0; t < kKeySteps; ++t)
            for (int rd = 0; rd < 2; ++rd)
                for (int sl = 0; sl < kSlabsPerWave; ++sl) {
                    const int o = v_lane(wave, lane, rd, sl) + 16384 * t;  // the kernel's form
                    const int want = v_off(lane, t, rd, kSlabsPerWave * wave + sl);
                    ++g_checks;
                    if (o != want) return bad("value operand split form", 0, 0, t, wave, lane, o, want);
                    if (!inside(o, 8, 0, kLatBytes)) return bad("value operand outside the latent slot", 0, 0, t, wave, lane, o, kLatBytes);
                }
        for (int hb = 0; hb < kValueBlocks; ++hb)
            for (int t = 0; t < kKeySteps; ++t)
                if (!inside(p_off(hb, t, lane), 16, 0, kPBytes)) return bad("probability exchange read", 0, 0, t, hb, lane, p_off(hb, t, lane), kPBytes);
        if (!inside(p_write_off(wave, lane), 8, 0, kPBytes)) return bad("probability exchange write", 0, 0, 0, wave, lane, p_write_off(wave, lane), kPBytes);
        const int stage = (wave & 1) * kStageHalf;  // wave w stages in half w % 2 of latent slot w / 2
        for (int sl = 0; sl < kSlabsPerWave; ++sl)
            for (int j = 0; j < 16; ++j)
                if (!inside(stage + stage_write_off(lane, j, sl), 4, stage, stage + kStageHalf)) return bad("staging store", 0, 0, j, wave, lane, stage_write_off(lane, j, sl), kStageHalf);
        for (int i = 0; i < 8; ++i)
            if (!inside(stage + stage_read_off(lane, i), 16, stage, stage + kStageHalf)) return bad("staging read", 0, 0, i, wave, lane, stage_read_off(lane, i), kStageHalf);
    }
    return true;
}

// Bank conflicts of one wave-wide read of `bytes` per lane: the lanes are served in consecutive
// groups that move 4 * banks bytes; the degree is the largest number of distinct 4-byte words of
// one group that fall in one bank (1: conflict-free).
int conflict_degree(const int *addr, int bytes, int banks) {
    const int per = 4 * banks / bytes;
    int worst = 1;
    for (int g = 0; g < 64; g += per) {
        int words[64][16], nw[64] = {0};
        for (int l = g; l < g + per; ++l)
            for (int w = addr[l] / 4; w < (addr[l] + bytes) / 4; ++w) {
                const int b = w % banks;
                bool seen = false;
                for (int i = 0; i < nw[b]; ++i) seen = seen || words[b][i] == w;
                if (!seen && nw[b] < 16) words[b][nw[b]++] = w;
                if (nw[b] > worst) worst = nw[b];
            }
    }
    return worst;
}

// The score-operand reads (latent and rotary) and the transposing value reads are free of bank
// conflicts in a model of 32 banks (128 bytes per cycle) and in one of 64 (256 bytes per cycle).
bool check_banks() {
    int a[64];
    for (int banks = 32; banks <= 64; banks *= 2) {
        for (int kh = 0; kh < kKeyHalves; ++kh) {
            for (int ks = 0; ks < kLatent / 32; ++ks) {
                for (int l = 0; l < 64; ++l) a[l] = k_lat_off(kh, l, ks);
                ++g_checks;
                if (conflict_degree(a, 16, banks) != 1) return bad("score operand bank conflict", 0, 0, ks, kh, banks, conflict_degree(a, 16, banks), 1);
            }
            for (int i = 0; i < kRope / 32; ++i) {
                for (int l = 0; l < 64; ++l) a[l] = k_rope_off(kh, l, i);
                ++g_checks;
                if (conflict_degree(a, 16, banks) != 1) return bad("rotary operand bank conflict", 0, 0, i, kh, banks, conflict_degree(a, 16, banks), 1);
            }
        }
        for (int t = 0; t < kKeySteps; ++t)
            for (int rd = 0; rd < 2; ++rd)
                for (int sg = 0; sg < kLatent / 32; ++sg) {
                    for (int l = 0; l < 64; ++l) a[l] = v_off(l, t, rd, sg);
                    ++g_checks;
                    if (conflict_degree(a, 8, banks) != 1) return bad("value operand bank conflict", 0, 0, t, sg, banks, conflict_degree(a, 8, banks), 1);
                }
    }
    return true;
}

// Every (key, chunk) a copy brings sits where the operand reads look for it, and every
// probability a wave writes is the one its readers take for that row and key.
bool check_roundtrips() {
    for (int key = 0; key < kTile; ++key)
        for (int lane = 0; lane < 64; ++lane) {
            const int chunk = lat_copy_src(key, lane) >> 4;  // the latent chunk lane `lane` copies
            const int at = lat_copy_lds(key) + 16 * lane;    // where it lands
            // score operand: wave of key half key / 16, lane key % 16 + 16 (chunk % 4), k-step chunk / 4
            const int reader = (key & 15) + 16 * (chunk & 3);
            ++g_checks;
            if (k_lat_off(key >> 4, reader, chunk >> 2) != at)
                return bad("latent copy and score operand disagree", 0, 0, key, 0, lane, at, k_lat_off(key >> 4, reader, chunk >> 2));
        }
    for (int w = 0; w < kRopeWaves; ++w)
        for (int lane = 0; lane < 64; ++lane) {
            const int key = rope_copy_key(w, lane), chunk = (lane & 7) ^ rope_swz(key);
            const int at = rope_copy_lds(w) + 16 * lane;
            const int reader = (key & 15) + 16 * (chunk & 3);
            ++g_checks;
            if (k_rope_off(key >> 4, reader, chunk >> 2) != at)
                return bad("rotary copy and score operand disagree", 0, 0, key, w, lane, at, k_rope_off(key >> 4, reader, chunk >> 2));
        }
    // value operand: recover (key, chunk) from each read's offset through the copies' placement
    for (int t = 0; t < kKeySteps; ++t)
        for (int rd = 0; rd < 2; ++rd)
            for (int s = 0; s < kLatent / 32; ++s)
                for (int lane = 0; lane < 64; ++lane) {
                    const int o = v_off(lane, t, rd, s), key = o / kLatRowBytes;
                    const int chunk = ((o % kLatRowBytes) >> 4) ^ lat_swz(key);
                    const int want_key = 16 * t + 8 * rd + 4 * (lane >> 5) + ((lane & 15) >> 2);
                    const int want_chunk = 4 * s + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
                    ++g_checks;
                    if (key != want_key || chunk != want_chunk) return bad("value operand reads the wrong chunk", 0, 0, t, s, lane, key * 64 + chunk, want_key * 64 + want_chunk);
                }
    // probabilities: wave w, lane l writes keys 16 (w / 4) + 4 (l / 16) + i (i < 4) of row
    // 16 (w % 4) + l % 16; the reader of block hb, step t, lane L, element e takes row 32 hb + L % 32
    // and key 16 t + 8 (e / 4) + 4 (L / 32) + e % 4
    static int row_of[kPBytes / 2], key_of[kPBytes / 2];
    for (int i = 0; i < kPBytes / 2; ++i) row_of[i] = key_of[i] = -1;
    for (int w = 0; w < kWaves; ++w)
        for (int lane = 0; lane < 64; ++lane)
            for (int i = 0; i < 4; ++i) {
                const int e = (p_write_off(w, lane) >> 1) + i;  // bf16 element
                if (row_of[e] != -1) return bad("two probabilities written to one place", 0, 0, i, w, lane, e, row_of[e]);
                row_of[e] = 16 * (w & 3) + (lane & 15);
                key_of[e] = 16 * (w >> 2) + 4 * (lane >> 4) + i;
            }
    for (int hb = 0; hb < kValueBlocks; ++hb)
        for (int t = 0; t < kKeySteps; ++t)
            for (int lane = 0; lane < 64; ++lane)
                for (int e = 0; e < 8; ++e) {
                    const int el = (p_off(hb, t, lane) >> 1) + e;
                    const int row = 32 * hb + (lane & 31), key = 16 * t + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    ++g_checks;
                    if (row_of[el] != row || key_of[el] != key)
                        return bad("probability read is not the one written", 0, 0, t, hb, lane, row_of[el] * 64 + key_of[el], row * 64 + key);
                }
    return true;
}

bool check_unit(const Geometry &g, int b, int split) {
    const int L = g.seq_lens[b];
    const int t0 = split * g.chunk, t1 = t0 + g.chunk < L ? t0 + g.chunk : L;
    if (t0 >= t1) return true;  // the kernel returns before staging or copying anything
    int shift = 0;
    while ((1 << shift) < g.page_size) ++shift;
    const int mask = (1 << shift) - 1;
    const int map_first = t0 >> shift;
    const int n = ((t1 - 1) >> shift) - map_first + 1;
    if (n > kMapCapacity) return bad("page map larger than its LDS array", b, split, t0, 0, 0, n, kMapCapacity);
    const long long lat_bytes = 2LL * g.ckv_elems, rope_bytes = 2LL * g.kpe_elems;
    const long long rope_stride = 2LL * g.kpe_s[1];
    // addresses are (array, byte offset): latent pool 0, rotary pool 1, q_nope 2, q_pe 3
    const int ntiles = (t1 - t0 + kTile - 1) / kTile;
    for (int i = 0; i < ntiles + kSlots - 1; ++i) {
        const int base = t0 + i * kTile;
        // per key of the tile (lane i < 32 of the kernel): its latent and rotary row
        int lat_arr[kTile], rope_arr[kTile];
        long long lat_row[kTile], rope_row[kTile];
        for (int k = 0; k < kTile; ++k) {
            const int vl = base + k, vlc = vl < t1 - 1 ? vl : t1 - 1;
            const int mi = (vlc >> shift) - map_first;
            ++g_checks;
            if (mi < 0 || mi >= n) return bad("page map lookup outside the staged ids", b, split, base, 0, k, mi, n);
            const long long pg = g.block_table[b * g.bt_stride + map_first + mi];
            const int sl = vlc & mask;
            if (vl < t1) {
                if (pg < 0 || pg >= g.pool_pages) return bad("page id outside the pool", b, split, base, 0, k, pg, g.pool_pages);
                lat_arr[k] = 0, lat_row[k] = 2 * (pg * g.ckv_s[0] + sl * g.ckv_s[1]);
                rope_arr[k] = 1, rope_row[k] = 2 * (pg * g.kpe_s[0] + sl * g.kpe_s[1]);
            } else {
                lat_arr[k] = 2, lat_row[k] = 2 * (b * g.q_s0);
                rope_arr[k] = 3, rope_row[k] = 2 * (b * g.q2_s0);
            }
        }
        for (int wave = 0; wave < kWaves; ++wave) {
            for (int j = 0; j < kLatCopiesPerWave; ++j) {
                const int kk = lat_copy_key(wave, j);
                const long long arr_bytes = lat_arr[kk] == 0 ? lat_bytes : 2LL * g.q_elems;
                for (int lane = 0; lane < 64; ++lane) {
                    const long long src = lat_row[kk] + lat_copy_src(kk, lane);
                    ++g_checks;
                    if (!inside(lat_copy_src(kk, lane), 16, 0, kLatRowBytes))
                        return bad("latent copy outside its 1 KB row", b, split, base, wave, lane, lat_copy_src(kk, lane), kLatRowBytes);
                    if (!inside(src, 16, 0, arr_bytes)) return bad("latent copy outside its array", b, split, base, wave, lane, src, arr_bytes);
                    if (!inside(lat_copy_lds(kk) + 16 * lane, 16, 0, kLatBytes))
                        return bad("latent copy lands outside its slot", b, split, base, wave, lane, lat_copy_lds(kk) + 16 * lane, kLatBytes);
                }
            }
            // rotary group of waves 0 .. 3: keys 8 wave .. 8 wave + 7 from the row of its first key
            if (wave >= kRopeWaves) continue;
            const int k0 = rope_copy_key(wave, 0), v0 = base + k0;
            int nv = t1 - v0;
            nv = nv < 0 ? 0 : nv > 8 ? 8 : nv;
            const long long records = rope_copy_records(nv, rope_stride);
            for (int lane = 0; lane < 64; ++lane) {
                const long long off = rope_copy_src(wave, lane, rope_stride);
                ++g_checks;
                if (!inside(rope_copy_lds(wave) + 16 * lane, 16, 0, kRopeBytes))
                    return bad("rotary copy lands outside its slot", b, split, base, wave, lane, rope_copy_lds(wave) + 16 * lane, kRopeBytes);
                if (off + 16 <= records) {
                    // in range: must be exactly the rotary row of key k0 + lane / 8 of this page
                    const int kk = rope_copy_key(wave, lane);
                    if (base + kk >= t1) return bad("rotary lane in range past the split", b, split, base, wave, lane, base + kk, t1);
                    if (rope_arr[k0] != 1 || rope_arr[kk] != 1) return bad("rotary group row kind", b, split, base, wave, lane, rope_arr[k0], 1);
                    const long long want = rope_row[kk] + (((lane & 7) ^ rope_swz(kk)) << 4);
                    if (rope_row[k0] + off != want) return bad("rotary copy reads another key's row", b, split, base, wave, lane, rope_row[k0] + off, want);
                    if (!inside(want, 16, rope_row[kk], rope_row[kk] + kRopeRowBytes) || !inside(want, 16, 0, rope_bytes))
                        return bad("rotary copy outside its row", b, split, base, wave, lane, want, rope_bytes);
                } else if (off < records) {
                    return bad("rotary copy straddles its range", b, split, base, wave, lane, off, records);
                }
            }
        }
    }
    return true;
}

}  // namespace

extern "C" int mla_layout_check(const Geometry *g, char *msg, int msg_len, long *checks) {
    g_msg = msg;
    g_len = msg_len;
    g_checks = 0;
    msg[0] = 0;
    for (int w = 0; w < kWaves; ++w)
        if (!check_lds(w)) return 1;
    if (!check_roundtrips()) return 1;
    if (!check_banks()) return 1;
    for (int b = 0; b < g->batch; ++b)
        for (int s = 0; s < g->num_splits; ++s)
            if (!check_unit(*g, b, s)) return 1;
    *checks = g_checks;
    return 0;
}
