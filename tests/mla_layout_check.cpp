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
//   - every copy lands inside its ring slot, and the latent chunk it brings is where the score
//     operand reads expect it;
//   - every operand read, probability exchange and staging access stays inside its LDS object,
//     and the per-lane split forms of the offsets equal the plain ones.
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
    for (int lane = 0; lane < 64; ++lane) {
        for (int ks = 0; ks < kLatent / 16; ++ks) {
            const int o = k_lat_off_split(lane, ks);
            ++g_checks;
            if (o != k_lat_off(lane, ks)) return bad("score operand split form", 0, 0, ks, wave, lane, o, k_lat_off(lane, ks));
            if (!inside(o, 16, 0, kLatBytes)) return bad("score operand outside the latent slot", 0, 0, ks, wave, lane, o, kLatBytes);
        }
        for (int i = 0; i < kRope / 16; ++i) {
            const int o = k_rope_off_split(lane, i);
            if (o != k_rope_off(lane, i)) return bad("rotary operand split form", 0, 0, i, wave, lane, o, k_rope_off(lane, i));
            if (!inside(o, 16, 0, kRopeBytes)) return bad("rotary operand outside the rotary slot", 0, 0, i, wave, lane, o, kRopeBytes);
        }
        for (int t = 0; t < kKeySteps; ++t)
            for (int rd = 0; rd < 2; ++rd)
                for (int s = 0; s < kSlabsPerWave; ++s) {
                    const int sg = kSlabsPerWave * wave + s;  // the wave's slab s: global slab
                    // the kernel's form: v_base + 256 wave + 64 (s ^ v_rot) + 16384 t
                    const int o = v_base(lane, rd) + 256 * wave + 64 * (s ^ v_rot(lane)) + 16384 * t;
                    ++g_checks;
                    if (o != v_off(lane, t, rd, sg) || o != v_off_split(lane, t, rd, sg))
                        return bad("value operand split form", 0, 0, t, wave, lane, o, v_off(lane, t, rd, sg));
                    if (!inside(o, 8, 0, kLatBytes)) return bad("value operand outside the latent slot", 0, 0, t, wave, lane, o, kLatBytes);
                }
        for (int hb = 0; hb < kWaves; ++hb)
            for (int t = 0; t < kKeySteps; ++t)
                if (!inside(p_off(hb, t, lane), 16, 0, kPBytes)) return bad("probability exchange", 0, 0, t, hb, lane, p_off(hb, t, lane), kPBytes);
        for (int s = 0; s < kSlabsPerWave; ++s)
            for (int j = 0; j < 16; ++j)
                if (!inside(stage_write_off(lane, j, s), 4, 0, kLatBytes)) return bad("staging store", 0, 0, j, wave, lane, stage_write_off(lane, j, s), kLatBytes);
        for (int i = 0; i < kRowsPerWave / 2; ++i)
            if (!inside(stage_read_off(lane, i), 16, 0, kLatBytes)) return bad("staging read", 0, 0, i, wave, lane, stage_read_off(lane, i), kLatBytes);
    }
    // every (key, latent chunk) a copy brings sits where the score operand reads look for it
    for (int key = 0; key < kTile; ++key)
        for (int lane = 0; lane < 64; ++lane) {
            const int chunk = lat_copy_src(key, lane) >> 4;  // the global chunk lane `lane` copies
            const int at = lat_copy_lds(key) + 16 * lane;    // where it lands
            // score operand: lane l = key + 32 (chunk % 2) reads chunk 2 ks + l / 32 with ks = chunk / 2
            const int reader = key + 32 * (chunk & 1);
            if (k_lat_off(reader, chunk >> 1) != at) return bad("latent copy and score operand disagree", 0, 0, key, 0, lane, at, k_lat_off(reader, chunk >> 1));
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
            // rotary group: keys 8 wave .. 8 wave + 7 from the row of its first key
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
    for (int b = 0; b < g->batch; ++b)
        for (int s = 0; s < g->num_splits; ++s)
            if (!check_unit(*g, b, s)) return 1;
    *checks = g_checks;
    return 0;
}
