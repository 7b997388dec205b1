// api.cpp -- host side of the C ABI declared in include/attn_decode.h.
//
// Every entry point validates its arguments completely on the host before touching the HIP
// runtime, so every rejection path is observable without a GPU. Then it plans the split, fills a
// parameter block and enqueues the kernels on the caller's stream. Nothing here allocates,
// synchronises or throws.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <climits>
#include <mutex>
#include <cmath>
#include <string>

#include "ad_internal.h"
#include "attn_decode.h"
#include "mla_layout.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    g_error = std::string(what) + ": " + hipGetErrorString(e);
    return (int)e;
}

int ok() {
    g_error.clear();
    return AD_OK;
}

constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == AD_F32 ? 4 : 2; }

bool strides_aligned(const int64_t s[3], int es) {
    for (int i = 0; i < 3; ++i)
        if ((s[i] * es) % 16 != 0) return false;
    return true;
}

int log2_exact(int x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return (1 << s) == x ? s : -1;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Testing aids (AD_NUM_SPLITS, AD_PARTIAL_KERNEL, AD_MFMA_ROWS, AD_FUSED_MERGE) are read only when
// AD_TEST_KNOBS=1 is set, so that a stray variable in a serving process cannot change kernels or
// plans; every call reads them afresh, so a test can switch them between calls.
const char *knob(const char *name) {
    const char *on = getenv("AD_TEST_KNOBS");
    if (!on || strcmp(on, "1") != 0) return nullptr;
    const char *v = getenv(name);
    return (v && *v) ? v : nullptr;
}

int knob_int(const char *name) {
    const char *s = knob(name);
    return s ? atoi(s) : 0;
}

// ------------------------------------------------------------------ validation
enum class Path { Contig, Paged, Mla };

int check_args(const ad_decode_args *a, Path path, bool need_out) {
    if (!a) return fail(AD_E_NULL, "args is NULL");
    if (a->dtype != AD_F32 && a->dtype != AD_BF16) return fail(AD_E_DTYPE, "dtype %d is not AD_F32 or AD_BF16", a->dtype);
    if (a->batch < 0 || a->q_len < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1)
        return fail(AD_E_SHAPE, "batch must be >= 0 and q_len, num_q_heads, num_kv_heads >= 1");
    if (a->num_q_heads % a->num_kv_heads)
        return fail(AD_E_SHAPE, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)", a->num_q_heads,
                    a->num_kv_heads);
    if (a->kv_len_max < 0) return fail(AD_E_RANGE, "kv_len_max must be >= 0");
    if (a->window < 0) return fail(AD_E_RANGE, "window must be >= 0");
    if (a->causal != 0 && a->causal != 1) return fail(AD_E_RANGE, "causal must be 0 or 1");
    if (!(std::isfinite(a->scale))) return fail(AD_E_RANGE, "scale must be finite");
    if (a->kv_format != AD_KV_SAME && a->kv_format != AD_KV_FP8_E4M3 && a->kv_format != AD_KV_INT4)
        return fail(AD_E_DTYPE, "kv_format %d is not AD_KV_SAME, AD_KV_FP8_E4M3 or AD_KV_INT4", a->kv_format);
    if (a->tree_mask && a->q_len > 64)
        return fail(AD_E_UNSUPPORTED, "a tree mask covers at most 64 query tokens (q_len %d)", a->q_len);
    if ((reinterpret_cast<uintptr_t>(a->q_starts) & 3u) || (reinterpret_cast<uintptr_t>(a->tree_mask) & 3u))
        return fail(AD_E_ALIGN, "q_starts and tree_mask must be 4-byte aligned");
    if (a->batch == 0) return AD_OK;  // nothing is read or written: no pointer is needed
    if (path == Path::Mla) {
        if (a->q_starts || a->tree_mask)
            return fail(AD_E_UNSUPPORTED, "MLA takes neither variable query lengths nor a tree mask");
        if (a->dtype != AD_BF16) return fail(AD_E_UNSUPPORTED, "MLA supports bf16 only");
        if (a->head_dim_qk != 576 || a->head_dim_v != 512 || a->num_kv_heads != 1)
            return fail(AD_E_UNSUPPORTED, "MLA needs head_dim_qk 576, head_dim_v 512 and one KV head");
        if (a->v && a->v != a->k)
            return fail(AD_E_UNSUPPORTED, "MLA reads values from the latent cache: v must be NULL or equal k");
        if (a->kv_format != AD_KV_SAME) return fail(AD_E_UNSUPPORTED, "MLA does not take a quantised cache");
    } else {
        if (a->head_dim_qk != a->head_dim_v) return fail(AD_E_UNSUPPORTED, "head_dim_qk must equal head_dim_v");
        if (a->head_dim_qk != 64 && a->head_dim_qk != 128)
            return fail(AD_E_UNSUPPORTED, "head dim %d not supported (64 or 128)", a->head_dim_qk);
        if (!a->v) return fail(AD_E_NULL, "v is NULL");
        if (a->kv_format == AD_KV_FP8_E4M3) {
            if (a->dtype != AD_BF16) return fail(AD_E_UNSUPPORTED, "an fp8 cache is read with bf16 q and out");
            if (a->head_dim_qk != 128) return fail(AD_E_UNSUPPORTED, "an fp8 cache needs head dim 128");
            if (!a->k_scale || !a->v_scale) return fail(AD_E_NULL, "k_scale or v_scale is NULL");
            if ((reinterpret_cast<uintptr_t>(a->k_scale) & 3u) || (reinterpret_cast<uintptr_t>(a->v_scale) & 3u))
                return fail(AD_E_ALIGN, "k_scale and v_scale must be 4-byte aligned");
        }
        if (a->kv_format == AD_KV_INT4) {
            if (a->dtype != AD_BF16) return fail(AD_E_UNSUPPORTED, "an int4 cache is read with bf16 q and out");
            if (a->head_dim_qk != 128) return fail(AD_E_UNSUPPORTED, "an int4 cache needs head dim 128");
            const int g = a->kv_groups;
            if (g != 1 && g != 2 && g != 4 && g != 8) return fail(AD_E_RANGE, "kv_groups %d is not 1, 2, 4 or 8", g);
        }
    }
    if (!a->q || !a->k) return fail(AD_E_NULL, "q or k is NULL");
    const int es = elem_bytes(a->dtype);
    const bool int4 = a->kv_format == AD_KV_INT4;
    const int kv_es = a->kv_format == AD_KV_FP8_E4M3 ? 1 : es;  // bytes per K / V element
    const uintptr_t kv_align = int4 ? 3u : 15u;                  // int4 rows are read as words
    if (!aligned16(a->q) || (reinterpret_cast<uintptr_t>(a->k) & kv_align) ||
        (a->v && (reinterpret_cast<uintptr_t>(a->v) & kv_align)))
        return fail(AD_E_ALIGN, int4 ? "q must be 16-byte and k, v 4-byte aligned" : "q, k and v must be 16-byte aligned");
    if (!strides_aligned(a->q_stride, es) ||
        (!int4 && (!strides_aligned(a->k_stride, kv_es) || (a->v && !strides_aligned(a->v_stride, kv_es)))))
        return fail(AD_E_ALIGN, "q/k/v strides must keep every row 16-byte aligned");
    if (need_out) {
        if (!a->out) return fail(AD_E_NULL, "out is NULL");
        if (!aligned16(a->out) || !strides_aligned(a->out_stride, es))
            return fail(AD_E_ALIGN, "out rows must be 16-byte aligned");
        if (a->lse && (reinterpret_cast<uintptr_t>(a->lse) & 3u)) return fail(AD_E_ALIGN, "lse must be 4-byte aligned");
    }
    return AD_OK;
}

int check_paged(const ad_decode_args *a, const ad_paged *pg) {
    if (!pg) return fail(AD_E_NULL, "paged is NULL");
    if (!pg->block_table) return fail(AD_E_NULL, "block_table is NULL");
    if (pg->page_size != 16 && pg->page_size != 32 && pg->page_size != 64)
        return fail(AD_E_RANGE, "page_size %d is not 16, 32 or 64", pg->page_size);
    if (pg->bt_stride < cdiv(a->kv_len_max, pg->page_size))
        return fail(AD_E_RANGE, "bt_stride %lld is smaller than ceil(kv_len_max / page_size)",
                    (long long)pg->bt_stride);
    return AD_OK;
}

int check_sparse(const ad_sparse *sp) {
    if (!sp->num_blocks || !sp->block_idx) return fail(AD_E_NULL, "num_blocks or block_idx is NULL");
    const int sh = log2_exact(sp->block_size);
    if (sh < 4 || sh > 12) return fail(AD_E_RANGE, "block_size %d is not a power of two in [16, 4096]", sp->block_size);
    if (sp->max_blocks < 0) return fail(AD_E_RANGE, "max_blocks must be >= 0");
    return AD_OK;
}

// ------------------------------------------------------------------ planning
// The latent-attention kernel takes 64 query rows (heads x query tokens) per work unit.
int mla_row_blocks(const ad_decode_args *a) { return (int)cdiv((int64_t)a->num_q_heads * a->q_len, ad::mla::kRows); }

// Which partial kernel runs, and how the G * q_len query rows of one KV head are blocked into work
// units: the matrix-core kernels (bf16 with more than 8 rows, any fp8 cache, and an int4 cache of
// one coefficient group per row) take 16 rows per unit when the rows fit 16 and 32 otherwise (an
// int4 cache always 16); the vector kernel takes up to 8 (4 with an fp8 or int4 cache; an int4
// cache of 2, 4 or 8 groups per row always runs there). AD_PARTIAL_KERNEL=valu|mfma overrides the
// choice of kernel where both exist, and AD_MFMA_TILE=16|32 the matrix-core tile (testing aids).
struct Rows {
    bool mfma;
    bool tile16;   // matrix cores, 16-row units (v_mfma_f32_16x16x32_bf16)
    int per_unit;  // rows one unit holds (the vector kernel's padded row count)
    int blocks;    // units per KV head
};

Rows row_plan(const ad_decode_args *a) {
    const int r = (a->num_q_heads / a->num_kv_heads) * a->q_len;
    const char *force = knob("AD_PARTIAL_KERNEL");
    // quantised caches take the matrix cores by default (the vector path converts every key's
    // values once per row block, and is bound by its ALUs)
    const bool fp8 = a->kv_format == AD_KV_FP8_E4M3, int4 = a->kv_format == AD_KV_INT4;
    const bool int4_mfma = int4 && a->kv_groups == 1;  // the matrix-core int4 form: one group per row
    bool mfma = a->dtype == AD_BF16 && (r > 8 || fp8 || int4_mfma) && (!int4 || int4_mfma);
    if (force && a->dtype == AD_BF16 && (!int4 || int4_mfma)) {
        if (!strcmp(force, "mfma")) mfma = true;
        if (!strcmp(force, "valu")) mfma = false;
    }
    Rows x{};
    x.mfma = mfma;
    if (mfma) {
        // 16-row units when the rows fit them: a unit of r <= 16 rows padded to 32 makes twice the
        // matrix-core products and holds twice the registers of the 16-row form
        x.tile16 = r <= 16;
        if (const char *t = knob("AD_MFMA_TILE")) x.tile16 = !strcmp(t, "16");
        if (int4) x.tile16 = true;  // the int4 form exists in 16-row units only
        x.per_unit = x.tile16 ? 16 : 32;
    } else {
        // an fp8 or int4 unit takes at most 4 rows (8 would exceed a lane's registers)
        const int valu_max = (fp8 || int4) ? 4 : 8;
        x.per_unit = std::min(valu_max, r <= 1 ? 1 : r <= 2 ? 2 : r <= 4 ? 4 : 8);
    }
    x.blocks = (int)cdiv(r, x.per_unit);
    return x;
}

int device_cus(int *cus) {
    static int cache[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev >= 0 && dev < 64 && cache[dev] > 0) {
        *cus = cache[dev];
        return AD_OK;
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    if (dev >= 0 && dev < 64) cache[dev] = n;
    *cus = n;
    return AD_OK;
}


struct Plan {
    int splits;
    int chunk;
};

// Largest key range the splits partition (virtual for a block list).
int64_t key_span(const ad_decode_args *a, const ad_sparse *sp) {
    return sp ? (int64_t)sp->max_blocks * sp->block_size : (int64_t)a->kv_len_max;
}

// Keys per split at most when lengths may be ragged. Measured on 64 paged sequences of
// 128..8192 keys (8 KV heads, 4 query rows each), repeated same-box runs: the vector kernel takes
// 191.8 us at 1664 keys (5 splits), 198.0 at 2048, 196.0 at 1366; the 32-row matrix-core kernel,
// whose work group costs more to start and to combine, 224.3 us at 4096 keys (2 splits) against
// 230.0 at 2048 with 1-8 draft tokens (32 rows per KV head). The 16-row matrix-core kernel, two
// work groups per compute unit, with longest-first placement: fp8 with whole-row loads 109.1 us
// at 2048 keys (4 splits), 105.8 at 2736, 121.8 at 4096 (with half-row loads 114.1 at 2048, 113.3
// at 1648, 114.5 at 2736); int4, whose keys are half as many bytes, 85.5 at 2048, 81.9 at 2736,
// 95.2 at 4096. The vector kernel's shorter bound applies only to grids of several rounds at
// 2048, where shorter splits even out the ragged tail; a grid of one round would spill into a
// second (16 sequences of 4096 keys: 50 -> 56 us). Other paths (MLA) keep 2048.
constexpr int64_t kRaggedChunkVector = 1664;
constexpr int64_t kRaggedChunkMatrix = 4096;
constexpr int64_t kRaggedChunkQuant = 3072;
constexpr int64_t kRaggedChunk = 2048;

// fp8 caches on the 16-row kernel: each load reads whole 128-byte rows and K reaches the matrix
// cores through LDS (109.1 us against 114.1 on the ragged fp8 workload above, both at 2048 keys),
// or each reads half rows of 16 keys straight into the operand registers. AD_MFMA_ROWS=0/1 forces
// either (testing aid).
bool fp8_whole_rows() { return knob("AD_MFMA_ROWS") ? knob_int("AD_MFMA_ROWS") != 0 : true; }

int plan_splits(const ad_decode_args *a, const ad_paged *pg, const ad_sparse *sp, Path path, int requested,
                Plan *out) {
    const int64_t span = key_span(a, sp);
    const int grain = pg ? pg->page_size : (sp ? sp->block_size : 16);
    // page / block ids one split can stage (the MLA kernel keeps a smaller map: its LDS holds the ring)
    const int map_capacity = path == Path::Mla ? ad::mla::kMapCapacity : ad::kMapCapacity;
    int S = requested > 0 ? requested : knob_int("AD_NUM_SPLITS");
    if (S < 0 || S > AD_MAX_SPLITS) return fail(AD_E_RANGE, "num_splits %d outside [0, %d]", S, AD_MAX_SPLITS);
    if (S == 0) {
        int cus = 0;
        int rc = device_cus(&cus);
        if (rc != AD_OK) return rc;
        const int64_t units =
            (int64_t)a->batch * (path == Path::Mla ? mla_row_blocks(a) : (int64_t)a->num_kv_heads * row_plan(a).blocks);
        // Few, long splits: a work group streams its keys most efficiently as one long run, and
        // one group per compute unit already saturates HBM. Two splits per sequence (one for short
        // caches), doubled until every compute unit has a work group, never below 256 keys each.
        S = span >= 2048 ? 2 : 1;
        while (units * S < cus && span / (2 * S) >= 256 && S * 2 <= AD_MAX_SPLITS) S *= 2;
        // Per-sequence lengths may be ragged: splits of a bounded length (the bounds above) keep
        // the longest work group near the average share of a compute unit (a uniform cache is
        // best served by the fewest splits that fill the compute units, as above).
        if (a->seq_lens) {
            int64_t most = kRaggedChunk;
            if (path != Path::Mla) {
                const Rows rows = row_plan(a);
                if (rows.mfma && !rows.tile16)
                    most = kRaggedChunkMatrix;
                else if (rows.mfma)
                    most = a->kv_format == AD_KV_INT4 || (a->kv_format == AD_KV_FP8_E4M3 && fp8_whole_rows())
                               ? kRaggedChunkQuant
                               : kRaggedChunk;
                else if (units * std::max<int64_t>(S, cdiv(span, kRaggedChunk)) >= 2 * (int64_t)cus)
                    most = kRaggedChunkVector;
            }
            S = (int)std::min<int64_t>(std::max<int64_t>(S, cdiv(span, most)), AD_MAX_SPLITS);
        }
        // A split over a paged cache or a block list stages its page / block ids in LDS: never
        // more of them than the map holds, whatever the bounds above chose (a multiple of 16).
        if (pg || sp)
            S = (int)std::min<int64_t>(std::max<int64_t>(S, cdiv(span, (int64_t)(map_capacity - 2) * grain)),
                                       AD_MAX_SPLITS);
    }
    int64_t chunk = cdiv(std::max<int64_t>(span, 1), S);
    chunk = std::max<int64_t>(cdiv(chunk, 16) * 16, 16);
    if (pg || sp) {
        if (cdiv(chunk, grain) + 2 > map_capacity)
            return fail(AD_E_RANGE, "%d splits leave %lld keys per split; at most %d pages/blocks per split", S,
                        (long long)chunk, map_capacity - 2);
    }
    if (chunk > (1 << 30)) return fail(AD_E_RANGE, "key range too long");
    out->splits = S;
    out->chunk = (int)chunk;
    return AD_OK;
}

ad::PartialParams base_params(const ad_decode_args *a, const Plan &pl) {
    ad::PartialParams p{};
    p.q = a->q;
    p.k = a->k;
    p.v = a->v ? a->v : a->k;
    for (int i = 0; i < 3; ++i) {
        p.q_s[i] = a->q_stride[i];
        p.k_s[i] = a->k_stride[i];
        p.v_s[i] = a->v ? a->v_stride[i] : a->k_stride[i];
    }
    p.seq_lens = a->seq_lens;
    p.kv_len_max = a->kv_len_max;
    p.batch = a->batch;
    p.q_len = a->q_len;
    p.num_q_heads = a->num_q_heads;
    p.num_kv_heads = a->num_kv_heads;
    p.group = a->num_q_heads / a->num_kv_heads;
    p.head_dim_v = a->head_dim_v;
    p.scale_log2 = a->scale * kLog2e;
    p.causal = a->causal;
    p.window = a->window;
    p.num_splits = pl.splits;
    p.chunk = pl.chunk;
    p.q_starts = a->q_starts;
    p.tree_mask = a->tree_mask;
    p.mask_words = (a->q_len + 31) / 32;
    if (a->kv_format == AD_KV_INT4) {
        p.kv_int4 = 1;
        p.kv_groups = a->kv_groups;
    }
    if (a->kv_format == AD_KV_FP8_E4M3) {
        p.kv_fp8 = 1;
        p.k_scale = a->k_scale;
        p.v_scale = a->v_scale;
        for (int i = 0; i < 3; ++i) {
            p.ks_s[i] = a->k_scale_stride[i];
            p.vs_s[i] = a->v_scale_stride[i];
        }
    }
    return p;
}

hipError_t launch_partial(const ad_decode_args *a, ad::PartialParams &p, int mode, hipStream_t stream) {
    // The kernels pick their element format from these flags: a block that disagrees with the
    // arguments would read a byte-strided cache as 16-bit elements, past the end of its allocation.
    if ((a->kv_format == AD_KV_FP8_E4M3) != (p.kv_fp8 != 0) || (a->kv_format == AD_KV_INT4) != (p.kv_int4 != 0))
        return hipErrorInvalidValue;
    const Rows rows = row_plan(a);
    p.row_blocks = rows.blocks;
    // one work group per (split, b, KV head, row block) on a 1-D grid
    const int64_t groups = (int64_t)p.num_splits * a->batch * a->num_kv_heads * rows.blocks;
    if (groups > INT_MAX) return hipErrorInvalidConfiguration;
    // Longest-piece-first placement (decode_unit_lpt) for per-sequence lengths on grids of more
    // work groups than compute units (a grid of one round runs every group at once, and the order
    // is moot); not with a block list, whose lengths differ per KV head. Measured on 64 ragged
    // paged sequences: 191.2 -> 185.8 us (bf16), 122.7 -> 114.1 (fp8), 97.0 -> 82.3 (int4),
    // 224.5 -> 207.6 (1-8 drafts). AD_LPT=0/1 forces it where it applies (testing aid).
    const bool lpt_ok = a->seq_lens && mode != ad::KV_SPARSE && a->batch <= ad::kLptMaxBatch;
    if (knob("AD_LPT")) {
        p.lpt = lpt_ok && knob_int("AD_LPT") != 0;
    } else {
        int cus = 0;
        if (device_cus(&cus) != AD_OK) return hipErrorInvalidDevice;
        p.lpt = lpt_ok && groups > cus;
    }
    if (rows.mfma && rows.tile16) {
        p.mfma_rows = a->kv_format == AD_KV_FP8_E4M3 && fp8_whole_rows();
        return ad::launch_partial_mfma16(p, a->head_dim_qk, mode, stream);
    }
    if (rows.mfma && a->kv_format == AD_KV_SAME) {
        // Whole-row loads staged through LDS (bf16 caches): every load reads whole lines once, at
        // the price of a round trip through LDS per tile. That pays when a compute unit runs
        // several work groups in turn (2048 groups: 258 -> 238 us) and costs when each runs one
        // (256 groups: 33.9 -> 35.5 us). AD_MFMA_ROWS=0/1 forces the choice (testing aid).
        if (knob("AD_MFMA_ROWS")) {
            p.mfma_rows = knob_int("AD_MFMA_ROWS") != 0;
        } else {
            int cus = 0;
            if (device_cus(&cus) != AD_OK) return hipErrorInvalidDevice;
            p.mfma_rows = groups > cus;
        }
    }
    if (rows.mfma) return ad::launch_partial_mfma(p, a->head_dim_qk, mode, stream);
    return ad::launch_partial_valu(p, a->dtype, a->head_dim_qk, rows.per_unit, mode, stream);  // fp8: p.kv_fp8
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t partial_bytes(const ad_decode_args *a, int S, size_t *lse_offset) {
    const size_t rows = (size_t)a->batch * a->q_len * a->num_q_heads;
    const size_t o = align256(rows * S * a->head_dim_v * sizeof(float));
    if (lse_offset) *lse_offset = o;
    return o + align256(rows * S * sizeof(float));
}

// Work units of the partial pass: (b, KV head, row block), or (b, row block) for MLA.
int64_t work_units(const ad_decode_args *a, Path path) {
    if (path == Path::Mla) return (int64_t)a->batch * mla_row_blocks(a);
    return (int64_t)a->batch * a->num_kv_heads * row_plan(a).blocks;
}

// Workspace of a whole decode step: a fixed region of arrival counters (one per work unit of the
// single-launch merge) first, then the partial outputs and LSEs. The counter region has the same
// place and size for every shape and split count, so partials never land on counters and one
// zero fill lasts for the workspace's life.
constexpr size_t kCounterBytes = size_t(1) << 20;
constexpr int64_t kMaxUnits = (int64_t)(kCounterBytes / sizeof(uint32_t));

size_t step_bytes(const ad_decode_args *a, int S, size_t *lse_offset) {
    size_t lse = 0;
    const size_t n = kCounterBytes + partial_bytes(a, S, &lse);
    if (lse_offset) *lse_offset = kCounterBytes + lse;
    return n;
}

// Whether attn_decode merges inside the partial pass (one launch) or with the merge kernel. The
// in-pass merge makes every work group wait for its stores and an atomic round trip before it
// leaves, and puts the unit's merge behind its last split; a merge launch costs a few
// microseconds of launch gap and its own run. One launch wins when the grid is a single round
// (at most one group per compute unit, so no group waits for a slot) and a unit holds few rows
// (at most 8, so its merge is short); otherwise two launches. AD_FUSED_MERGE=0/1 forces the
// choice (testing aid).
int fuse_merge(const ad_decode_args *a, Path path, int S, bool *fused) {
    if (knob("AD_FUSED_MERGE")) {
        *fused = knob_int("AD_FUSED_MERGE") != 0;
        return AD_OK;
    }
    int cus = 0;
    int rc = device_cus(&cus);
    if (rc != AD_OK) return rc;
    const Rows rows = row_plan(a);
    const int r = (a->num_q_heads / a->num_kv_heads) * a->q_len;
    *fused = std::min(r, rows.per_unit) <= 8 && work_units(a, path) * S <= cus;
    return AD_OK;
}

// Fills the cache addressing of p for a paged cache or a block list (contiguous otherwise) and
// returns the kernel mode.
int kv_mode(ad::PartialParams &p, const ad_paged *paged, const ad_sparse *sparse) {
    if (sparse) {
        p.num_blocks = sparse->num_blocks;
        p.block_idx = sparse->block_idx;
        p.nb_s[0] = sparse->nb_stride[0];
        p.nb_s[1] = sparse->nb_stride[1];
        for (int i = 0; i < 3; ++i) p.ix_s[i] = sparse->idx_stride[i];
        p.block_shift = log2_exact(sparse->block_size);
        return ad::KV_SPARSE;
    }
    if (paged) {
        p.block_table = paged->block_table;
        p.bt_stride = paged->bt_stride;
        p.page_shift = log2_exact(paged->page_size);
        return ad::KV_PAGED;
    }
    return ad::KV_CONTIG;
}

int run_merge(const ad_decode_args *a, const float *po, const float *pl, int S, bool count_by_len, int chunk,
              hipStream_t stream, const int32_t *splits_per_batch = nullptr) {
    ad::MergeParams m{};
    m.part_o = po;
    m.part_lse = pl;
    m.num_splits = S;
    m.rows = a->batch * a->q_len * a->num_q_heads;
    m.head_dim_v = a->head_dim_v;
    m.q_len = a->q_len;
    m.num_q_heads = a->num_q_heads;
    m.count_by_len = count_by_len ? 1 : 0;
    m.seq_lens = a->seq_lens;
    m.kv_len_max = a->kv_len_max;
    m.chunk = chunk;
    m.out_dtype = a->dtype;
    m.out = a->out;
    for (int i = 0; i < 3; ++i) m.out_s[i] = a->out_stride[i];
    m.lse = a->lse;
    m.q_starts = a->q_starts;
    m.splits_per_batch = splits_per_batch;
    hipError_t e = ad::launch_merge(m, stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return AD_OK;
}

// ------------------------------------------------------------------ library-owned scratch
// attn_decode_noalloc's workspace: a file-scope device array, one copy per GPU, held until the
// process ends. Its address on the current device comes from hipGetSymbolAddress, taken once per
// device at the first call there; host code never passes the array's own name to a kernel (in
// host code that name is a stand-in, not a device address). The first call on a device also
// clears the arrival counters with a fill kernel on its stream (every call leaves them at zero).
constexpr size_t kScratchBytes = AD_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes > kCounterBytes, "room for partials after the counters");

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static __global__ void clear_words_kernel(uint32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

int scratch_of_device(hipStream_t stream, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(AD_E_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        constexpr int words = (int)(kCounterBytes / sizeof(uint32_t));
        hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                           static_cast<uint32_t *>(ptr), words);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "scratch counter clear");
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return AD_OK;
}

int decode_step(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse, int32_t num_splits,
                void *workspace, size_t workspace_bytes, void *stream, bool library_scratch) {
    const Path path = paged ? Path::Paged : Path::Contig;
    int rc = check_args(args, path, true);
    if (rc != AD_OK) return rc;
    if (paged && sparse) return fail(AD_E_UNSUPPORTED, "a block list over a paged cache is not supported");
    if (args->batch == 0) return ok();
    if (paged && (rc = check_paged(args, paged)) != AD_OK) return rc;
    if (sparse && (rc = check_sparse(sparse)) != AD_OK) return rc;
    if (num_splits < 0 || num_splits > AD_MAX_SPLITS)
        return fail(AD_E_RANGE, "num_splits %d outside [0, %d]", num_splits, AD_MAX_SPLITS);
    if (!library_scratch) {
        if (!workspace) return fail(AD_E_WORKSPACE, "workspace is NULL");
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(AD_E_ALIGN, "workspace must be 256-byte aligned");
    }
    Plan pl{};
    if ((rc = plan_splits(args, paged, sparse, path, num_splits, &pl)) != AD_OK) return rc;
    if ((int64_t)args->batch * args->q_len * args->num_q_heads > INT_MAX)
        return fail(AD_E_UNSUPPORTED, "batch x q_len x num_q_heads must stay below 2^31");
    if (work_units(args, path) > kMaxUnits)
        return fail(AD_E_UNSUPPORTED, "%lld work units (batch x KV heads x query-row blocks) exceed %lld",
                    (long long)work_units(args, path), (long long)kMaxUnits);
    size_t lse_off = 0;
    const size_t need = step_bytes(args, pl.splits, &lse_off);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (library_scratch) {
        if (need > kScratchBytes)
            return fail(AD_E_RANGE, "this step needs %zu bytes of workspace (%d splits); the library's own "
                        "scratch holds %zu: use attn_decode with a workspace",
                        need, pl.splits, kScratchBytes);
        if ((rc = scratch_of_device(s, &workspace)) != AD_OK) return rc;
    } else if (workspace_bytes < need) {
        return fail(AD_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed for %d splits",
                    workspace_bytes, need, pl.splits);
    }
    char *ws = static_cast<char *>(workspace);
    ad::PartialParams p = base_params(args, pl);
    const int mode = kv_mode(p, paged, sparse);
    p.part_o = reinterpret_cast<float *>(ws + kCounterBytes);
    p.part_lse = reinterpret_cast<float *>(ws + lse_off);
    bool fused = false;
    if ((rc = fuse_merge(args, path, pl.splits, &fused)) != AD_OK) return rc;
    if (fused) {
        p.write_empty = 0;
        p.counters = reinterpret_cast<uint32_t *>(ws);
        p.out = args->out;
        for (int i = 0; i < 3; ++i) p.out_s[i] = args->out_stride[i];
        p.out_dtype = args->dtype == AD_BF16 ? ad::DT_BF16 : ad::DT_F32;
        p.lse = args->lse;
        hipError_t e = launch_partial(args, p, mode, s);
        if (e != hipSuccess) return hip_fail(e, "decode launch");
        return ok();
    }
    // Two launches. A block list's length varies per (b, KV head), so every split slot is written
    // and merged; otherwise splits past a sequence's end write nothing and row b merges only
    // ceil(L_b / chunk) of them.
    p.write_empty = sparse ? 1 : 0;
    hipError_t e = launch_partial(args, p, mode, s);
    if (e != hipSuccess) return hip_fail(e, "split-KV launch");
    rc = run_merge(args, p.part_o, p.part_lse, pl.splits, !sparse, pl.chunk, s);
    return rc == AD_OK ? ok() : rc;
}


}  // namespace

extern "C" {

int attn_decode_plan(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse, int32_t *num_splits,
                     int32_t *chunk) {
    const bool mla = args && args->head_dim_qk == 576 && args->head_dim_v == 512;
    const Path path = mla ? Path::Mla : (paged ? Path::Paged : Path::Contig);
    int rc = check_args(args, path, false);
    if (rc != AD_OK) return rc;
    if (paged && (rc = check_paged(args, paged)) != AD_OK) return rc;
    if (sparse && (rc = check_sparse(sparse)) != AD_OK) return rc;
    Plan pl{};
    if ((rc = plan_splits(args, paged, sparse, path, 0, &pl)) != AD_OK) return rc;
    if (num_splits) *num_splits = pl.splits;
    if (chunk) *chunk = pl.chunk;
    return ok();
}

size_t attn_decode_workspace_size(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse,
                                  int32_t num_splits) {
    const bool mla = args && args->head_dim_qk == 576 && args->head_dim_v == 512;
    const Path path = mla ? Path::Mla : (paged ? Path::Paged : Path::Contig);
    if (check_args(args, path, false) != AD_OK) return 0;
    if (paged && sparse) {
        fail(AD_E_UNSUPPORTED, "a block list over a paged cache is not supported");
        return 0;
    }
    if (paged && check_paged(args, paged) != AD_OK) return 0;
    if (sparse && check_sparse(sparse) != AD_OK) return 0;
    Plan pl{};
    if (plan_splits(args, paged, sparse, path, num_splits, &pl) != AD_OK) return 0;
    ok();
    return step_bytes(args, pl.splits, nullptr);
}

int attn_decode_splitkv(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse,
                        int32_t num_splits, float *part_o, float *part_lse, void *stream) {
    int rc = check_args(args, paged ? Path::Paged : Path::Contig, false);
    if (rc != AD_OK) return rc;
    if (paged && sparse) return fail(AD_E_UNSUPPORTED, "a block list over a paged cache is not supported");
    if (args->batch == 0) return ok();
    if (paged && (rc = check_paged(args, paged)) != AD_OK) return rc;
    if (sparse && (rc = check_sparse(sparse)) != AD_OK) return rc;
    if (!part_o || !part_lse) return fail(AD_E_NULL, "part_o or part_lse is NULL");
    if (!aligned16(part_o) || (reinterpret_cast<uintptr_t>(part_lse) & 3u))
        return fail(AD_E_ALIGN, "part_o must be 16-byte and part_lse 4-byte aligned");
    if (num_splits < 0 || num_splits > AD_MAX_SPLITS)
        return fail(AD_E_RANGE, "num_splits %d outside [0, %d]", num_splits, AD_MAX_SPLITS);
    Plan pl{};
    if ((rc = plan_splits(args, paged, sparse, paged ? Path::Paged : Path::Contig, num_splits, &pl)) != AD_OK)
        return rc;
    ad::PartialParams p = base_params(args, pl);
    const int mode = kv_mode(p, paged, sparse);
    p.write_empty = 1;
    p.part_o = part_o;
    p.part_lse = part_lse;
    hipError_t e = launch_partial(args, p, mode, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "split-KV launch");
    return ok();
}

int attn_decode_merge(const float *part_o, const float *part_lse, const int32_t *splits_per_batch,
                      int32_t num_splits, int32_t batch, int32_t q_len, int32_t num_q_heads, int32_t head_dim_v,
                      int32_t out_dtype, void *out, const int64_t out_stride[3], float *lse, void *stream) {
    if (out_dtype != AD_F32 && out_dtype != AD_BF16) return fail(AD_E_DTYPE, "out_dtype %d unknown", out_dtype);
    if (num_splits < 1 || num_splits > AD_MAX_SPLITS)
        return fail(AD_E_RANGE, "num_splits %d outside [1, %d]", num_splits, AD_MAX_SPLITS);
    if (batch < 0 || q_len < 1 || num_q_heads < 1) return fail(AD_E_SHAPE, "bad batch / q_len / num_q_heads");
    if (batch == 0) return ok();
    if (!part_o || !part_lse || !out || !out_stride) return fail(AD_E_NULL, "part_o, part_lse, out or out_stride is NULL");
    if (head_dim_v != 64 && head_dim_v != 128 && head_dim_v != 256 && head_dim_v != 512 && head_dim_v != 1024)
        return fail(AD_E_UNSUPPORTED, "head_dim_v %d not in {64, 128, 256, 512, 1024}", head_dim_v);
    if (!aligned16(part_o) || (reinterpret_cast<uintptr_t>(part_lse) & 3u) || !aligned16(out) ||
        !strides_aligned(out_stride, elem_bytes(out_dtype)) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) ||
        (reinterpret_cast<uintptr_t>(splits_per_batch) & 3u))
        return fail(AD_E_ALIGN, "misaligned part_o / part_lse / splits_per_batch / out / lse");
    ad_decode_args a{};
    a.dtype = out_dtype;
    a.batch = batch;
    a.q_len = q_len;
    a.num_q_heads = num_q_heads;
    a.head_dim_v = head_dim_v;
    a.out = out;
    for (int i = 0; i < 3; ++i) a.out_stride[i] = out_stride[i];
    a.lse = lse;
    int rc = run_merge(&a, part_o, part_lse, num_splits, false, 1, static_cast<hipStream_t>(stream), splits_per_batch);
    return rc == AD_OK ? ok() : rc;
}

int attn_decode(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse, int32_t num_splits,
                void *workspace, size_t workspace_bytes, void *stream) {
    return decode_step(args, paged, sparse, num_splits, workspace, workspace_bytes, stream, false);
}

int attn_decode_noalloc(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse,
                        int32_t num_splits, void *stream) {
    return decode_step(args, paged, sparse, num_splits, nullptr, 0, stream, true);
}

int attn_decode_launches(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse,
                         int32_t num_splits, int32_t *launches) {
    if (!launches) return fail(AD_E_NULL, "launches is NULL");
    const bool mla = args && args->head_dim_qk == 576 && args->head_dim_v == 512;
    const Path path = mla ? Path::Mla : paged ? Path::Paged : Path::Contig;
    int rc = check_args(args, path, false);
    if (rc != AD_OK) return rc;
    if (paged && sparse) return fail(AD_E_UNSUPPORTED, "a block list over a paged cache is not supported");
    if (mla && (!paged || sparse)) return fail(AD_E_UNSUPPORTED, "MLA reads a paged cache without a block list");
    if (paged && (rc = check_paged(args, paged)) != AD_OK) return rc;
    if (sparse && (rc = check_sparse(sparse)) != AD_OK) return rc;
    if (args->batch == 0) {
        *launches = 0;
        return ok();
    }
    Plan pl{};
    if ((rc = plan_splits(args, paged, sparse, path, num_splits, &pl)) != AD_OK) return rc;
    bool fused = false;  // the MLA step is always the partial pass and the merge kernel
    if (!mla && (rc = fuse_merge(args, path, pl.splits, &fused)) != AD_OK) return rc;
    *launches = fused ? 1 : 2;
    return ok();
}

int attn_decode_kernel(const ad_decode_args *args, int32_t *kind) {
    if (!kind) return fail(AD_E_NULL, "kind is NULL");
    if (!args) return fail(AD_E_NULL, "args is NULL");
    const bool mla = args->head_dim_qk == 576 && args->head_dim_v == 512;
    const int rc = check_args(args, mla ? Path::Mla : Path::Contig, false);
    if (rc != AD_OK) return rc;
    if (mla) {
        *kind = AD_KERNEL_MLA;
    } else {
        const Rows rows = row_plan(args);
        *kind = !rows.mfma ? AD_KERNEL_VECTOR : rows.tile16 ? AD_KERNEL_MATRIX16 : AD_KERNEL_MATRIX;
    }
    return ok();
}

int attn_decode_paged(const ad_decode_args *args, const ad_paged *paged, int32_t num_splits, void *workspace,
                      size_t workspace_bytes, void *stream) {
    if (!paged) return fail(AD_E_NULL, "paged is NULL");
    return attn_decode(args, paged, nullptr, num_splits, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Checks shared by the two MLA entry points; on success fills *pl and *p (partials not set).
int mla_prepare(const ad_decode_args *args, const void *kpe, const int64_t kpe_stride[3], const void *q_pe,
                const int64_t q_pe_stride[3], const ad_paged *paged, int32_t num_splits, bool need_out, Plan *pl,
                ad::PartialParams *p) {
    int rc = check_args(args, Path::Mla, need_out);
    if (rc != AD_OK) return rc;
    if (args->batch == 0) return AD_OK;
    if ((rc = check_paged(args, paged)) != AD_OK) return rc;
    if (!kpe || !q_pe || !kpe_stride || !q_pe_stride) return fail(AD_E_NULL, "kpe / q_pe or their strides are NULL");
    if (!aligned16(kpe) || !aligned16(q_pe) || !strides_aligned(kpe_stride, 2) || !strides_aligned(q_pe_stride, 2))
        return fail(AD_E_ALIGN, "kpe and q_pe rows must be 16-byte aligned");
    if (num_splits < 0 || num_splits > AD_MAX_SPLITS)
        return fail(AD_E_RANGE, "num_splits %d outside [0, %d]", num_splits, AD_MAX_SPLITS);
    if ((rc = plan_splits(args, paged, nullptr, Path::Mla, num_splits, pl)) != AD_OK) return rc;
    if ((int64_t)pl->splits * mla_row_blocks(args) * args->batch > INT32_MAX)
        return fail(AD_E_RANGE, "batch x row blocks x splits exceeds the launch grid");
    *p = base_params(args, *pl);
    p->q2 = q_pe;
    p->k2 = kpe;
    for (int i = 0; i < 3; ++i) {
        p->q2_s[i] = q_pe_stride[i];
        p->k2_s[i] = kpe_stride[i];
    }
    p->block_table = paged->block_table;
    p->bt_stride = paged->bt_stride;
    p->page_shift = log2_exact(paged->page_size);
    p->row_blocks = mla_row_blocks(args);
    return AD_OK;
}

}  // namespace

extern "C" {

int attn_decode_mla(const ad_decode_args *args, const void *kpe, const int64_t kpe_stride[3], const void *q_pe,
                    const int64_t q_pe_stride[3], const ad_paged *paged, int32_t num_splits, void *workspace,
                    size_t workspace_bytes, void *stream) {
    Plan pl{};
    ad::PartialParams p{};
    int rc = mla_prepare(args, kpe, kpe_stride, q_pe, q_pe_stride, paged, num_splits, true, &pl, &p);
    if (rc != AD_OK) return rc;
    if (args->batch == 0) return ok();
    if (!workspace) return fail(AD_E_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(AD_E_ALIGN, "workspace must be 256-byte aligned");
    size_t lse_off = 0;
    const size_t need = step_bytes(args, pl.splits, &lse_off);
    if (workspace_bytes < need)
        return fail(AD_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
    // the partials go where every whole-step entry puts them: after the counter region
    float *po = reinterpret_cast<float *>(static_cast<char *>(workspace) + kCounterBytes);
    float *plse = reinterpret_cast<float *>(static_cast<char *>(workspace) + lse_off);
    p.write_empty = 0;
    p.part_o = po;
    p.part_lse = plse;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = ad::launch_partial_mla(p, s);
    if (e != hipSuccess) return hip_fail(e, "MLA split-KV launch");
    // Splits past a sequence's end wrote nothing: row b merges only ceil(L_b / chunk) of them.
    rc = run_merge(args, po, plse, pl.splits, true, pl.chunk, s);
    return rc == AD_OK ? ok() : rc;
}

int attn_decode_mla_splitkv(const ad_decode_args *args, const void *kpe, const int64_t kpe_stride[3],
                            const void *q_pe, const int64_t q_pe_stride[3], const ad_paged *paged,
                            int32_t num_splits, float *part_o, float *part_lse, void *stream) {
    Plan pl{};
    ad::PartialParams p{};
    int rc = mla_prepare(args, kpe, kpe_stride, q_pe, q_pe_stride, paged, num_splits, false, &pl, &p);
    if (rc != AD_OK) return rc;
    if (args->batch == 0) return ok();
    if (!part_o || !part_lse) return fail(AD_E_NULL, "part_o or part_lse is NULL");
    if (!aligned16(part_o) || (reinterpret_cast<uintptr_t>(part_lse) & 3u))
        return fail(AD_E_ALIGN, "part_o must be 16-byte and part_lse 4-byte aligned");
    p.write_empty = 1;
    p.part_o = part_o;
    p.part_lse = part_lse;
    hipError_t e = ad::launch_partial_mla(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "MLA split-KV launch");
    return ok();
}

int attn_decode_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    if (!src || !sink) return fail(AD_E_NULL, "src or sink is NULL");
    if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u))
        return fail(AD_E_ALIGN, "src must be 16-byte and sink 4-byte aligned");
    if (bytes == 0 || bytes % 16 || bytes > (size_t(1) << 40))
        return fail(AD_E_RANGE, "bytes must be a nonzero multiple of 16 (at most 2^40)");
    hipError_t e = ad::launch_read_probe(src, (int64_t)bytes, sink, AD_PROBE_SINK_WORDS / 4,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "read probe launch");
    return ok();
}

const char *attn_decode_last_error(void) { return g_error.c_str(); }

}  // extern "C"
