/*
 * oracle.c -- plain fp64 CPU reference for single-step decode attention.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry file and the
 * CPU-baseline leg of the benchmark may load or run this library. The HIP library never
 * links, includes or calls it, and it shares no code, header, table or helper with it.
 *
 * It computes the plain definition with no tiling, no split and no online softmax. For every
 * query row (b, t, hq):
 *
 *   hkv   = hq / G,   G = num_q_heads / num_kv_heads             (GQA: G consecutive query heads
 *                                                              share one KV head; PyTorch Inductor
 *                                                              flex_decode.py.jinja, the
 *                                                              "hq = hkv*G + g" head packing)
 *   L     = seq_lens[b],   pos = L - q_len + t                   (query t sits at the tail of its
 *                                                              sequence; mslk splitk_kernels.py,
 *                                                              the causal-mask comment in
 *                                                              _fwd_kernel_splitK)
 *   s_j   = scale * sum_d q[d] * k_j[d]                          (plus the second part
 *                                                              q2 . k2_j when present: the MLA
 *                                                              score is q_nope.ckv + q_pe.kpe,
 *                                                              FlashInfer attention/mla.cuh,
 *                                                              compute_mla_qk)
 *   out   = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m)
 *   lse   = m + ln sum_j exp(s_j - m)                            (natural-log LSE as written by
 *                                                              mslk splitk_kernels.py at the end
 *                                                              of _fwd_kernel_splitK)
 *
 * over the visible keys j, with m their largest score.
 *
 * Variable query lengths (TensorRT-LLM xqa mha.cu, qCuSeqLens; mslk splitk_kernels.py,
 * Seq_starts_q): with q_starts, sequence b has Q_b = q_starts[b+1] - q_starts[b] query tokens
 * (at most q_len) and its token t is packed row n = q_starts[b] + t of q, out and lse; it sits at
 * position L - Q_b + t. Without it every sequence has q_len tokens and n = b*q_len + t.
 *
 * Tree mask (TensorRT-LLM xqa mha.cu, the SPEC_DEC input mask): the last Q_b keys of sequence b
 * are its draft tokens, draft key i at position L - Q_b + i. Token row n sees draft key i only if
 * bit i % 32 of word tree_mask[n * ceil(q_len / 32) + i / 32] is set; the keys before the drafts
 * are not affected. It combines with the other conditions below (all must hold). A row with no visible key gets out = 0 and
 * lse = -inf (mslk splitk_kernels.py, the l == 0 guard of the split epilogue and the lse_max ==
 * -inf guard of _splitK_reduce).
 *
 * Key j is visible to row (b, t, hq) iff all of:
 *   0 <= j < L;
 *   key_lo <= j < key_hi when a key range is given (a split's own token range);
 *   not causal, or j <= pos     (bottom-right causal: FlashInfer mla.cuh logits_mask_ masks
 *                                kv_idx + qo_len > kv_len + q_idx);
 *   window == 0, or pos - j < window   (the window keeps `window` keys ending at the query's own
 *                                position: TensorRT-LLM xqa mha.cu skips the first len - W cache
 *                                tokens; equal to mslk's WINDOW_LEFT = window - 1);
 *   no block list, or j / block_size is one of the listed blocks of (b, hkv)   (PyTorch Inductor
 *                                flex_decode.py.jinja, KV_NUM_BLKS / KV_IDX);
 *   no tree mask, or j < L - Q_b, or the tree-mask bit of (n, j - (L - Q_b)) is set.
 *
 * K and V rows are found through the same address map the cache uses:
 *   contiguous: base + b*st[0] + j*st[1] + hkv*st[2]
 *   paged:      base + block_table[b][j / page_size]*st[0] + (j % page_size)*st[1] + hkv*st[2]
 *               (mslk splitk_kernels.py paged branch; TensorRT-LLM xqa page list)
 * The last dimension is contiguous. Elements are fp64, fp32 or bf16 (raw 16-bit patterns), all
 * widened exactly to fp64, or, for K and V only, fp8 bytes of a quantised cache (see below).
 *
 * Quantised cache (TensorRT-LLM xqa mha.cu: an e4m3 cache with one kvCacheScale for K and V;
 * mslk splitk_kernels.py, _process_fp8_quantization: row-wise fp8 with a scale per row): every K
 * (V) element is an OCP E4M3 byte, decoded exactly and multiplied by the fp32 scale of its row,
 * k_scale[kv_row(scale strides, b, hkv, j)] (the scale array is indexed like the cache rows; a zero
 * stride broadcasts, all zero is one scale per tensor). The attention then runs on those values.
 * E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits): exponent field e > 0 gives
 * (1 + m/8) 2^(e-7), e = 0 gives the subnormal m 2^-9, and S.1111.111 is NaN (no infinities), so
 * the largest finite magnitude is 1.75 * 2^8 = 448.
 *
 * Int4 cache (mslk splitk_kernels.py, the int4 branch of dequantize / _process_int4_quantization):
 * every K (V) row of dim_qk (dim_v) values is stored as 32-bit words, n_groups coefficient words
 * followed by the packed values, 8 per word. Dimension d belongs to group g = d / (dim / n_groups)
 * and is the unsigned 4-bit field (d % 8) of packed word d / 8 (bits 4(d % 8) .. 4(d % 8) + 3);
 * coefficient word g holds two IEEE half floats, the scale in its low 16 bits and the shift in its
 * high 16 bits, and the value is field * scale + shift. Row strides then count 32-bit words.
 *
 * oracle_merge() is the LSE-weighted combine of per-split (o_s, lse_s) pairs written out in fp64
 * (mslk splitk_kernels.py, _splitK_reduce): M = max_s lse_s, w_s = exp(lse_s - M),
 * out = sum_s w_s o_s / sum_s w_s, lse = M + ln sum_s w_s; M = -inf gives out 0, lse -inf.
 *
 * Every function here is pinned by the oracle tests (closed forms, a library attention routine,
 * hand-listed visibility sets, paging and split invariants); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2, ORC_E4M3 = 3, ORC_INT4 = 4 };

typedef struct {
    int32_t batch, q_len, num_q_heads, num_kv_heads;
    int32_t dim_qk;   /* first score part (all of it for plain attention; the 512 latent dims for MLA) */
    int32_t dim_qk2;  /* second score part (the 64 rope dims for MLA); 0 when absent */
    int32_t dim_v;
    double scale;
    int32_t q_type, kv_type; /* ORC_F64 / ORC_F32 / ORC_BF16 */
    const void *q;  int64_t q_stride[3];  /* [b][t][hq] */
    const void *q2; int64_t q2_stride[3]; /* [b][t][hq] */
    const void *k;  int64_t k_stride[3];  /* contiguous [b][j][hkv]; paged [page][slot][hkv] */
    const void *k2; int64_t k2_stride[3]; /* same indexing as k */
    const void *v;  int64_t v_stride[3];  /* same indexing as k */
    const int32_t *seq_lens;              /* [batch]; NULL: every sequence has kv_len keys */
    int32_t kv_len;
    const int32_t *block_table; int64_t bt_stride; int32_t page_size; /* NULL: contiguous */
    const int32_t *num_blocks; int64_t nb_stride[2];                   /* NULL: no block list */
    const int32_t *block_idx; int64_t idx_stride[3]; int32_t block_size;
    int32_t causal, window;
    int32_t key_lo, key_hi; /* key_hi < 0: no range restriction */
    /* kv_type ORC_E4M3: fp32 scale of every K / V row, indexed like the rows */
    const float *k_scale; int64_t ks_stride[3];
    const float *v_scale; int64_t vs_stride[3];
    /* variable query lengths: [batch + 1] packed token offsets (q and q2 rows n use
     * n * q_stride[1] + hq * q_stride[2]); NULL: q_len tokens per sequence */
    const int32_t *q_starts;
    const uint32_t *tree_mask; /* [token rows][ceil(q_len / 32)] words; NULL: none */
    int32_t n_groups;          /* kv_type ORC_INT4: coefficient words per row (1, 2, 4 or 8) */
} oracle_problem;

/* Value of one OCP E4M3 byte, from the format's definition. */
static double e4m3(uint8_t x)
{
    const int sign = x >> 7, e = (x >> 3) & 15, m = x & 7;
    double mag;
    if (e == 15 && m == 7)
        mag = NAN;
    else if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* IEEE binary16 value of a 16-bit pattern, from the format's definition. */
static double half_value(uint32_t h)
{
    const int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double mag;
    if (e == 31)
        mag = m ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)m, -24);
    else
        mag = ldexp(1.0 + m / 1024.0, e - 15);
    return sign ? -mag : mag;
}

/* Value of dimension d of the int4 row that starts at word `row` (dim values per row). */
static double int4_value(const void *base, int64_t row, int64_t d, int64_t dim, int32_t n_groups)
{
    const uint32_t *w = (const uint32_t *)base + row;
    const uint32_t coef = w[d / (dim / n_groups)];
    const uint32_t field = (w[n_groups + d / 8] >> (4 * (d % 8))) & 15u;
    return (double)field * half_value(coef & 0xFFFFu) + half_value(coef >> 16);
}

static double widen(const void *base, int32_t type, int64_t i)
{
    if (type == ORC_F64) return ((const double *)base)[i];
    if (type == ORC_F32) return (double)((const float *)base)[i];
    if (type == ORC_E4M3) return e4m3(((const uint8_t *)base)[i]);
    /* bf16 is the upper half of an IEEE binary32 pattern */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Offset (in elements) of the row of key j of head hkv of sequence b. */
static int64_t kv_row(const oracle_problem *P, const int64_t st[3], int64_t b, int64_t hkv, int64_t j)
{
    if (P->block_table) {
        int64_t page = P->block_table[b * P->bt_stride + j / P->page_size];
        return page * st[0] + (j % P->page_size) * st[1] + hkv * st[2];
    }
    return b * st[0] + j * st[1] + hkv * st[2];
}

static int block_listed(const oracle_problem *P, int64_t b, int64_t hkv, int64_t j)
{
    if (!P->num_blocks) return 1;
    int64_t n = P->num_blocks[b * P->nb_stride[0] + hkv * P->nb_stride[1]];
    int64_t blk = j / P->block_size;
    for (int64_t i = 0; i < n; i++)
        if (P->block_idx[b * P->idx_stride[0] + hkv * P->idx_stride[1] + i * P->idx_stride[2]] == blk)
            return 1;
    return 0;
}

/* Query tokens of sequence b, and the packed row of its token t. */
static int64_t q_tokens(const oracle_problem *P, int64_t b)
{
    return P->q_starts ? (int64_t)P->q_starts[b + 1] - P->q_starts[b] : P->q_len;
}
static int64_t q_row(const oracle_problem *P, int64_t b, int64_t t)
{
    return P->q_starts ? (int64_t)P->q_starts[b] + t : b * P->q_len + t;
}
static int64_t q_offset(const oracle_problem *P, const int64_t st[3], int64_t b, int64_t t, int64_t hq)
{
    if (P->q_starts) return q_row(P, b, t) * st[1] + hq * st[2];
    return b * st[0] + t * st[1] + hq * st[2];
}

static int tree_allows(const oracle_problem *P, int64_t b, int64_t t, int64_t L, int64_t j)
{
    if (!P->tree_mask) return 1;
    const int64_t first_draft = L - q_tokens(P, b);
    if (j < first_draft) return 1;
    const int64_t i = j - first_draft, words = (P->q_len + 31) / 32;
    return (int)((P->tree_mask[q_row(P, b, t) * words + i / 32] >> (i % 32)) & 1u);
}

static int key_visible(const oracle_problem *P, int64_t b, int64_t t, int64_t hkv, int64_t L, int64_t j)
{
    int64_t pos = L - q_tokens(P, b) + t;
    if (j < 0 || j >= L) return 0;
    if (P->key_hi >= 0 && (j < P->key_lo || j >= P->key_hi)) return 0;
    if (P->causal && j > pos) return 0;
    if (P->window > 0 && pos - j >= P->window) return 0;
    if (!tree_allows(P, b, t, L, j)) return 0;
    return block_listed(P, b, hkv, j);
}

static double score(const oracle_problem *P, int64_t b, int64_t t, int64_t hq, int64_t hkv, int64_t j)
{
    double acc = 0.0;
    int64_t qo = q_offset(P, P->q_stride, b, t, hq);
    int64_t ko = kv_row(P, P->k_stride, b, hkv, j);
    const double ks = P->kv_type == ORC_E4M3 ? (double)P->k_scale[kv_row(P, P->ks_stride, b, hkv, j)] : 1.0;
    for (int64_t d = 0; d < P->dim_qk; d++) {
        const double kd = P->kv_type == ORC_INT4 ? int4_value(P->k, ko, d, P->dim_qk, P->n_groups)
                                                 : widen(P->k, P->kv_type, ko + d) * ks;
        acc += widen(P->q, P->q_type, qo + d) * kd;
    }
    if (P->dim_qk2 > 0) {
        int64_t qo2 = q_offset(P, P->q2_stride, b, t, hq);
        int64_t ko2 = kv_row(P, P->k2_stride, b, hkv, j);
        for (int64_t d = 0; d < P->dim_qk2; d++)
            acc += widen(P->q2, P->q_type, qo2 + d) * widen(P->k2, P->kv_type, ko2 + d);
    }
    return P->scale * acc;
}

static int check_problem(const oracle_problem *P)
{
    if (!P || P->batch < 0 || P->q_len <= 0 || P->num_q_heads <= 0 || P->num_kv_heads <= 0) return -1;
    if (P->num_q_heads % P->num_kv_heads) return -1;
    if (P->dim_qk <= 0 || P->dim_v <= 0 || P->dim_qk2 < 0) return -1;
    if (!P->q || !P->k || !P->v) return -1;
    if (P->dim_qk2 > 0 && (!P->q2 || !P->k2)) return -1;
    if (P->block_table && P->page_size <= 0) return -1;
    if (P->num_blocks && (!P->block_idx || P->block_size <= 0)) return -1;
    if (P->window < 0) return -1;
    if (P->q_type == ORC_E4M3) return -1;
    if (P->kv_type == ORC_E4M3 && (!P->k_scale || !P->v_scale || P->dim_qk2 > 0)) return -1;
    if (P->kv_type == ORC_INT4) {
        const int32_t g = P->n_groups;
        if (P->dim_qk2 > 0 || (g != 1 && g != 2 && g != 4 && g != 8)) return -1;
        if (P->dim_qk % (8 * g) || P->dim_v % (8 * g)) return -1;
    }
    if (P->q_type == ORC_INT4) return -1;
    if (P->q_starts) {
        if (P->q_starts[0] < 0) return -1;
        for (int64_t b = 0; b < P->batch; b++)
            if (q_tokens(P, b) < 0 || q_tokens(P, b) > P->q_len) return -1;
    }
    return 0;
}

static int n_threads = 0; /* 0: OpenMP default */

void oracle_set_threads(int n) { n_threads = n; }

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return n_threads > 0 ? n_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Attention for the listed rows (row = n*num_q_heads + hq for packed token row n, i.e.
 * (b*q_len + t)*num_q_heads + hq without q_starts), or for every row in that order when
 * rows == NULL. out is [nrows][dim_v], lse is [nrows]. With q_starts, a token row below
 * q_starts[0] belongs to no sequence and gets out = 0, lse = -inf. Returns 0, or -1 on a
 * malformed problem.
 */
int oracle_attend(const oracle_problem *P, const int64_t *rows, int64_t nrows, double *out, double *lse)
{
    if (check_problem(P) || !out || !lse) return -1;
    const int64_t G = P->num_q_heads / P->num_kv_heads;
    const int64_t tokens = P->q_starts ? (int64_t)P->q_starts[P->batch] : (int64_t)P->batch * P->q_len;
    const int64_t total = tokens * P->num_q_heads;
    if (!rows) nrows = total;
    for (int64_t i = 0; rows && i < nrows; i++)
        if (rows[i] < 0 || rows[i] >= total) return -1;

    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(oracle_get_threads())
    for (int64_t i = 0; i < nrows; i++) {
        const int64_t r = rows ? rows[i] : i;
        const int64_t hq = r % P->num_q_heads, n = r / P->num_q_heads;
        int64_t b = n / P->q_len, t = n % P->q_len;
        double *o = out + i * P->dim_v;
        if (P->q_starts) {  /* the sequence whose packed rows hold n */
            b = -1;
            for (int64_t c = 0; c < P->batch; c++)
                if (P->q_starts[c] <= n && n < P->q_starts[c + 1]) b = c;
            if (b < 0) {
                for (int64_t d = 0; d < P->dim_v; d++) o[d] = 0.0;
                lse[i] = -INFINITY;
                continue;
            }
            t = n - P->q_starts[b];
        }
        const int64_t hkv = hq / G;
        const int64_t L = P->seq_lens ? P->seq_lens[b] : P->kv_len;

        double *s = (double *)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
        char *vis = (char *)malloc((size_t)(L > 0 ? L : 1));
        if (!s || !vis) {
            free(s);
            free(vis);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        double m = -INFINITY;
        int64_t n_vis = 0;
        for (int64_t j = 0; j < L; j++) {
            vis[j] = (char)key_visible(P, b, t, hkv, L, j);
            if (!vis[j]) continue;
            s[j] = score(P, b, t, hq, hkv, j);
            if (s[j] > m) m = s[j];
            n_vis++;
        }
        for (int64_t d = 0; d < P->dim_v; d++) o[d] = 0.0;
        if (n_vis == 0) {
            lse[i] = -INFINITY;
            free(s);
            free(vis);
            continue;
        }
        double l = 0.0;
        for (int64_t j = 0; j < L; j++) {
            if (!vis[j]) continue;
            double w = exp(s[j] - m);
            int64_t vo = kv_row(P, P->v_stride, b, hkv, j);
            const double vs =
                P->kv_type == ORC_E4M3 ? (double)P->v_scale[kv_row(P, P->vs_stride, b, hkv, j)] : 1.0;
            l += w;
            for (int64_t d = 0; d < P->dim_v; d++) {
                const double vd = P->kv_type == ORC_INT4 ? int4_value(P->v, vo, d, P->dim_v, P->n_groups)
                                                         : widen(P->v, P->kv_type, vo + d) * vs;
                o[d] += w * vd;
            }
        }
        for (int64_t d = 0; d < P->dim_v; d++) o[d] /= l;
        lse[i] = m + log(l);
        free(s);
        free(vis);
    }
    return bad ? -1 : 0;
}

/*
 * LSE-weighted merge of `splits` partial results per row.
 * part_o is [rows][splits][dim_v], part_lse is [rows][splits]; out is [rows][dim_v], lse [rows].
 */
int oracle_merge(int64_t rows, int32_t splits, int32_t dim_v, const double *part_o, const double *part_lse,
                 double *out, double *lse)
{
    if (rows < 0 || splits <= 0 || dim_v <= 0 || !part_o || !part_lse || !out || !lse) return -1;
    for (int64_t r = 0; r < rows; r++) {
        const double *ls = part_lse + r * splits;
        double *o = out + r * dim_v;
        double M = -INFINITY;
        for (int32_t s = 0; s < splits; s++)
            if (ls[s] > M) M = ls[s];
        for (int32_t d = 0; d < dim_v; d++) o[d] = 0.0;
        if (M == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double W = 0.0;
        for (int32_t s = 0; s < splits; s++) {
            double w = exp(ls[s] - M);
            const double *os = part_o + (r * splits + s) * dim_v;
            W += w;
            for (int32_t d = 0; d < dim_v; d++) o[d] += w * os[d];
        }
        for (int32_t d = 0; d < dim_v; d++) o[d] /= W;
        lse[r] = M + log(W);
    }
    return 0;
}
