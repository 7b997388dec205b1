/*
 * attn_decode.h -- C ABI of the MI355X (gfx950) single-step decode-attention library.
 *
 * One decode step computes, for every query row (b, t, hq),
 *
 *     out = softmax(scale * q . K^T + mask) . V        lse = ln sum_j exp(scale * q . k_j)
 *
 * for a few query rows per KV head (GQA: query head hq reads KV head hq / G, G = Hq / Hkv; the G
 * heads x q_len tokens of one KV head are packed into one work tile, as in the PyTorch Inductor
 * flex_decode.py.jinja template's GQA_SHARED_HEADS packing) against a long KV cache that is
 * contiguous, paged or block-sparse. The work is split along the KV length into partial passes
 * that each emit a normalised partial output and a natural-log LSE (mslk splitk_kernels.py,
 * _fwd_kernel_splitK epilogue), followed by an LSE-weighted merge (the same page,
 * _splitK_reduce). An MLA variant reads one shared latent KV head whose first 512 columns are
 * also the values (FlashInfer attention/mla.cuh, compute_mla_qk / compute_mla_pv).
 *
 * Conventions for every entry point:
 *   - Every tensor pointer is DEVICE memory owned by the caller; descriptors (the structs and
 *     the stride arrays) are HOST memory, read during the call only. The library allocates no
 *     device memory, never synchronises and never throws. Work is enqueued on `stream` (a
 *     hipStream_t; NULL = the default stream) and runs asynchronously. This is the launch
 *     contract of the pages' kernels: TensorRT-LLM xqa mha.cu's launchMHA takes its semaphores
 *     and scratch buffers from the caller and enqueues on the caller's stream, and FlashInfer
 *     attention/mla.cuh's BatchMLAPagedAttention takes partial_o / partial_lse inside its Params
 *     and launches on the given stream. Where xqa throws (runtime_error on an unsupported input),
 *     this C ABI returns a status instead, as mla.cuh's launcher returns a cudaError_t.
 *   - Strides are in ELEMENTS (bytes for an fp8 cache, 32-bit words for an int4 cache). The
 *     last (feature) dimension of every tensor is contiguous, and every row start must be
 *     16-byte aligned (int4 cache rows: 4-byte aligned).
 *   - Return value: AD_OK (0), a negative AD_E_* code when the arguments were rejected on the
 *     host before anything was enqueued, or a positive hipError_t when a launch failed (the
 *     status-code style of FlashInfer mla.cuh's BatchMLAPagedAttention, which returns
 *     cudaErrorNotSupported with a message for a configuration it has no kernel for).
 *     attn_decode_last_error() gives a message for the calling thread's last non-OK return.
 *   - Testing aids: the environment variables AD_NUM_SPLITS (split count, cf. xqa's
 *     XQA_NB_SUB_SEQ), AD_PARTIAL_KERNEL, AD_MFMA_TILE, AD_MFMA_ROWS, AD_FUSED_MERGE and AD_LPT
 *     (kernel forms and work-group placement, named at the calls they affect) are read only while AD_TEST_KNOBS=1 is set; otherwise the
 *     environment changes nothing.
 *   - Data contracts that are NOT checked (they live in device memory): seq_lens[b] <=
 *     kv_len_max and >= the sequence's query tokens; q_starts nondecreasing with counts of at
 *     most q_len; block-table entries for the pages a sequence covers lie in
 *     [0, pages of the pool) (entries past the sequence are never read and may hold -1);
 *     listed sparse blocks are < ceil(kv_len_max / block_size). Keys outside a sequence, past
 *     its last page slot, in unlisted blocks or in unreferenced pages are never read into the
 *     result and may hold any bits (NaN included).
 */
#ifndef ATTN_DECODE_H
#define ATTN_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------------------------ */
#define AD_OK 0
#define AD_E_NULL (-1)        /* a required pointer is NULL */
#define AD_E_DTYPE (-2)       /* unknown or unsupported element type */
#define AD_E_SHAPE (-3)       /* inconsistent sizes (e.g. Hq % Hkv != 0, non-positive sizes) */
#define AD_E_ALIGN (-4)       /* a row start or the last dimension is not 16-byte aligned/contiguous */
#define AD_E_UNSUPPORTED (-5) /* a valid request the library has no kernel for (e.g. head dim 96) */
#define AD_E_WORKSPACE (-6)   /* workspace missing or smaller than attn_decode_workspace_size() */
#define AD_E_RANGE (-7)       /* a count out of range (num_splits, page size, window, ...) */

/* ---- element types (Q, K, V and the output share one, unless kv_format quantises K / V) ---- */
#define AD_F32 0
#define AD_BF16 1

/* Cache element formats (ad_decode_args.kv_format). */
#define AD_KV_SAME 0     /* k and v hold `dtype` elements */
#define AD_KV_FP8_E4M3 1 /* k and v hold OCP E4M3 bytes with fp32 row scales */
#define AD_KV_INT4 2     /* k and v hold rows of 4-bit fields with fp16 scale / shift per group */

#define AD_MAX_SPLITS 256

/*
 * One decode step.
 *   q      [batch, q_len, num_q_heads, head_dim_qk]    (MLA: the latent part q_nope, 512 cols)
 *   k, v   contiguous cache: logical [batch, kv_len_max, num_kv_heads, D], strides
 *          {per batch, per token, per head}; a head-major cache [B, Hkv, L, D] is expressed by
 *          its strides. Paged cache: logical [pages, page_size, num_kv_heads, D] with strides
 *          {per page, per slot, per head}, addressed through ad_paged.block_table.
 *   out    [batch, q_len, num_q_heads, head_dim_v] in `dtype` (bf16 rounded to nearest even).
 *   lse    [batch, q_len, num_q_heads] fp32, natural log, contiguous; NULL to skip. A row with
 *          no visible key gets out = 0 and lse = -inf.
 * Query t of a q_len-token query sits at position L_b - q_len + t of its sequence (its own K/V
 * are already in the cache). With `causal`, it sees keys j <= that position (bottom-right
 * alignment: FlashInfer mla.cuh logits_mask_; mslk splitk_kernels.py causal comment). With
 * window W > 0 it sees only keys with position - j < W: the W most recent keys up to and
 * including its own (TensorRT-LLM xqa mha.cu sliding window). `scale` multiplies q . k in
 * natural-exp units and is never derived from the head dim (xqa passes qScale separately;
 * mla.cuh and splitk_kernels.py take sm_scale).
 */
typedef struct ad_decode_args {
    int32_t dtype;
    int32_t batch, q_len, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v;
    float scale;
    const void *q;
    int64_t q_stride[3];
    const void *k;
    int64_t k_stride[3];
    const void *v;
    int64_t v_stride[3];
    const int32_t *seq_lens; /* [batch] KV lengths (incl. the q_len new tokens); NULL: all kv_len_max */
    int32_t kv_len_max;      /* host-side bound on every seq_lens[b]; a contiguous cache's capacity */
    int32_t causal;
    int32_t window;          /* 0: none */
    void *out;
    int64_t out_stride[3];
    float *lse;
    /* Quantised cache (TensorRT-LLM xqa mha.cu: an e4m3 cache with one kvCacheScale; mslk
     * splitk_kernels.py, _process_fp8_quantization: fp8 rows with a scale per row). With
     * AD_KV_FP8_E4M3, k and v hold OCP E4M3 bytes (their strides count bytes) and every element
     * is dequantised as its decoded value times the fp32 scale of its row,
     * k_scale[b * k_scale_stride[0] + j * k_scale_stride[1] + h * k_scale_stride[2]] (paged:
     * page, slot, head), likewise for v. Zero strides broadcast; all zero is one scale per tensor,
     * xqa's form. Supported with bf16 q / out and head dim 128 on both partial kernels (the
     * matrix-core kernel by default, the vector kernel in blocks of at most 4 rows); not with MLA.
     * AD_KV_SAME (a zero-filled struct) ignores the rest. */
    int32_t kv_format;
    const float *k_scale;
    int64_t k_scale_stride[3];
    const float *v_scale;
    int64_t v_scale_stride[3];
    /* Speculative decoding (TensorRT-LLM xqa mha.cu SPEC_DEC: qCuSeqLens and the packed input
     * mask; mslk splitk_kernels.py Seq_starts_q). Both NULL in a zero-filled struct: off.
     *
     * q_starts [batch + 1] (device): variable query lengths. Sequence b has
     * Q_b = q_starts[b+1] - q_starts[b] query tokens, 0 <= Q_b <= q_len (q_len is then the
     * largest count), and its token t is packed row n = q_starts[b] + t: q row at
     * q + n*q_stride[1] + hq*q_stride[2] (q_stride[0] is not used), out row likewise with
     * out_stride, lse[n*num_q_heads + hq]. The token sits at position L_b - Q_b + t. Rows of
     * tokens t >= Q_b do not exist: nothing is read or written for them (the partial layout of
     * attn_decode_splitkv keeps its [batch, q_len, ...] rows; those stay unwritten). The counts
     * are the caller's contract, like a block table: they are clamped to [0, q_len] for the
     * library's own buffers, but q / out / lse rows are addressed through q_starts as given.
     *
     * tree_mask (device): the last Q_b keys of sequence b are its draft tokens, draft key i at
     * position L_b - Q_b + i. Token row n (q_starts[b] + t, or b*q_len + t without q_starts)
     * sees draft key i only if bit i % 32 of tree_mask[n * ceil(q_len / 32) + i / 32] is set;
     * keys before the drafts are not affected, and the mask combines (AND) with causal, window
     * and block lists. q_len <= 64 with a tree mask. Neither field is supported with MLA. */
    const int32_t *q_starts;
    const uint32_t *tree_mask;
    /* Int4 cache (mslk splitk_kernels.py, the int4 path of dequantize /
     * _process_int4_quantization). With AD_KV_INT4, every K (V) row is kv_groups + D/8 32-bit
     * words: kv_groups coefficient words, each an fp16 scale in its low half and an fp16 shift in
     * its high half, then the packed values, dimension d being the unsigned 4-bit field d % 8
     * (bits 4*(d % 8) upwards) of packed word d / 8. Dimension d belongs to group
     * d / (D / kv_groups) and its value is field * scale + shift. k / v point at those words
     * (4-byte aligned) and their strides count words. kv_groups is 1, 2, 4 or 8; head dim 128
     * (qk == v), bf16 q / out; not with MLA. Runs on the vector path in units of at most 4 rows,
     * in fp32 arithmetic. Ignored unless kv_format == AD_KV_INT4. */
    int32_t kv_groups;
} ad_decode_args;

/* Paged cache: logical page p of sequence b is pool page block_table[b * bt_stride + p]
 * (mslk splitk_kernels.py paged branch; TensorRT-LLM xqa page list). page_size is 16, 32 or 64. */
typedef struct ad_paged {
    const int32_t *block_table;
    int64_t bt_stride;
    int32_t page_size;
} ad_paged;

/* Block-sparse KV (PyTorch Inductor flex_decode.py.jinja, KV_NUM_BLKS / KV_IDX): for each
 * (b, KV head), num_blocks[b*nb_stride[0] + h*nb_stride[1]] blocks of block_size keys are listed
 * in block_idx[b*idx_stride[0] + h*idx_stride[1] + i*idx_stride[2]], i < num_blocks, ascending.
 * A stride of 0 broadcasts one list over that dimension. Key j contributes iff its block is
 * listed AND the causal/window masks admit it. max_blocks bounds every num_blocks entry.
 * block_size is a power of two in [16, 4096]. */
typedef struct ad_sparse {
    const int32_t *num_blocks;
    const int32_t *block_idx;
    int64_t nb_stride[2];
    int64_t idx_stride[3];
    int32_t block_size;
    int32_t max_blocks;
} ad_sparse;

/*
 * Split planner. Writes the split count the library would choose for this step (num_splits = 0
 * on the calls below) to *num_splits, and the tokens per split to *chunk (either may be NULL).
 * `paged` and `sparse` are nullable and select the path; MLA is selected by head_dim_qk == 576
 * with head_dim_v == 512. The choice fills every compute unit with work units of a few hundred
 * tokens or more (cf. TensorRT-LLM xqa launchMHA: sub-sequences = min(SMs / (batch * kv heads),
 * tiles per sequence)); with per-sequence lengths (seq_lens != NULL, possibly ragged) it also
 * bounds the split length, so that no work group is much longer than the average: 2048 keys,
 * 1664 on the vector kernel when that grid already takes several rounds of work groups, 4096 on
 * the 32-row matrix-core kernel (whose work groups cost more to start and finish), 3072 for
 * fp8 and int4 caches on the 16-row kernel (keys of fewer bytes, read as whole rows). A split of a
 * paged cache or a block list never covers more than 1038 pages or blocks (258 pages for MLA:
 * the ids it stages), which raises the count for very long caches of small pages. AD_NUM_SPLITS
 * forces the count (testing aid, see the conventions above).
 */
int attn_decode_plan(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse,
                     int32_t *num_splits, int32_t *chunk);

/* Bytes of workspace attn_decode / attn_decode_paged / attn_decode_mla need for `num_splits`
 * splits (0: the planner's choice) with the same `paged` / `sparse` (both nullable; a block list
 * changes the planner's choice, so pass the one the call will carry). The caller owns and sizes
 * this memory, as TensorRT-LLM xqa mha.cu's caller provides the `scratch` buffer of its
 * multi-block mode and FlashInfer mla.cuh's caller the partial_o / partial_lse arrays of Params.
 * Layout, the same for every entry point, shape and split count: AD_COUNTER_BYTES of arrival
 * counters (one 4-byte counter per work unit = sequence x KV head x block of query rows, at most
 * AD_COUNTER_BYTES / 4 units per call; xqa's `semaphores`), then the partials,
 * rows * splits * (head_dim_v + 1) * 4 bytes in 256-byte aligned parts. Returns 0, with a message
 * for attn_decode_last_error(), for arguments the calls would reject. */
#define AD_COUNTER_BYTES (1u << 20)
size_t attn_decode_workspace_size(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse,
                                  int32_t num_splits);

/*
 * Partial pass. The cache is contiguous (paged == NULL) or paged; a contiguous cache may carry a
 * block list (sparse; paged and sparse together are rejected). Split s covers keys
 * [s*c, (s+1)*c) with c = ceil(kv_len_max / num_splits) rounded up to 16 (for a block list: the
 * same ranges over the concatenation of the listed blocks, of length max_blocks*block_size).
 * Writes EVERY slot, also of splits that lie past a short sequence's end:
 *   part_o   [batch, q_len, num_q_heads, num_splits, head_dim_v] fp32, o_s = acc_s / l_s
 *   part_lse [batch, q_len, num_q_heads, num_splits] fp32, natural log; a split with no visible
 *            key gets o_s = 0, lse_s = -inf (mslk splitk_kernels.py: zeros when l == 0).
 * args->out and args->lse are ignored. num_splits in [1, AD_MAX_SPLITS]; 0 = the planner's
 * choice. Supported: head dims 64 and 128 (qk == v), fp32 or bf16, any G * q_len (bf16 with
 * more than 8 rows per KV head, every fp8 cache and an int4 cache of one coefficient group per row
 * run on the matrix cores, 16 or 32 rows per work unit; otherwise the vector ALUs take up to 8 rows
 * per work unit; attn_decode_kernel tells which). With per-sequence lengths (seq_lens, no block
 * list, at most 256 sequences) on a grid of more work groups than compute units, the work groups
 * take the (sequence, split) pieces longest first (full splits, then the remainders by length,
 * then empty splits), the longest-processing-time order for identical machines; which group
 * computes a piece changes, the values do not (AD_LPT=0/1 forces the order, testing aid).
 */
int attn_decode_splitkv(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse,
                        int32_t num_splits, float *part_o, float *part_lse, void *stream);

/*
 * LSE-weighted merge of num_splits partials per row (mslk splitk_kernels.py, _splitK_reduce):
 *   M = max_s lse_s,  w_s = exp(lse_s - M),  out = sum_s w_s o_s / sum_s w_s,
 *   lse = M + ln sum_s w_s;  M = -inf gives out = 0, lse = -inf.
 * part_o / part_lse use the layout attn_decode_splitkv writes. splits_per_batch (device, [batch],
 * nullable) gives the number of leading splits of each sequence that hold partials: row b merges
 * splits 0 .. min(splits_per_batch[b], num_splits) - 1 and never reads the others, so a ragged
 * batch whose short sequences left later slots unwritten merges correctly (a count <= 0 gives
 * out = 0, lse = -inf). NULL merges all num_splits slots of every row. out [batch, q_len,
 * num_q_heads, head_dim_v] in out_dtype with element strides out_stride {b, t, hq}; lse nullable,
 * contiguous. head_dim_v is 64, 128, 256, 512 or 1024.
 */
int attn_decode_merge(const float *part_o, const float *part_lse, const int32_t *splits_per_batch,
                      int32_t num_splits, int32_t batch, int32_t q_len, int32_t num_q_heads, int32_t head_dim_v,
                      int32_t out_dtype, void *out, const int64_t out_stride[3], float *lse, void *stream);

/*
 * Whole decode step, writing args->out / args->lse: the partial pass of attn_decode_splitkv
 * (contiguous cache, paged cache or a block list over a contiguous cache) and the merge of
 * attn_decode_merge, in ONE launch where that is faster: the last split of each work unit to
 * finish merges the unit's splits (same arithmetic, same order: the result is the two-launch
 * result bit for bit), elected by a counter per work unit that wraps back to zero on the last
 * arrival (the multi-block mode of TensorRT-LLM xqa mha.cu: a semaphore increment picks the last
 * CTA, which merges). One launch is used when the step is a single round of work groups (at most
 * one group per compute unit) whose units hold at most 8 query rows, else the
 * partial pass and the merge kernel run as two launches in the same workspace. AD_FUSED_MERGE=0 / 1
 * forces two launches / one launch (testing aid, see the conventions above).
 * workspace: device memory of at least attn_decode_workspace_size(args, paged, sparse, num_splits)
 * bytes, 256-byte aligned. Its first AD_COUNTER_BYTES MUST be zero before its first use (zero
 * the allocation once); every call leaves them zero and writes its partials only after them, so
 * the workspace is reused as is by any later call, of any shape or split count, and by
 * attn_decode_mla. One workspace serves one call at a time (calls that overlap on it race).
 * num_splits 0 = the planner's choice. Ragged seq_lens are handled per sequence: a split past the
 * end of its sequence does no work, and a sequence without keys gets out = 0, lse = -inf. More
 * than AD_COUNTER_BYTES / 4 work units: AD_E_UNSUPPORTED.
 */
int attn_decode(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse, int32_t num_splits,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode for callers that cannot allocate or pass device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same step, kernels, plan and
 * result bit for bit as attn_decode with the same arguments, but the workspace is the library's
 * own: a static device array of AD_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, held
 * until the process ends. The call allocates nothing (no hipMalloc / hipFree, no allocating
 * library routine). A step that needs more workspace than that (attn_decode_workspace_size
 * tells: AD_COUNTER_BYTES plus the partials) is rejected with AD_E_RANGE before anything is
 * enqueued. The first call on a device looks the array up there and clears its arrival counters
 * with a small kernel on `stream`; every call leaves them at zero. All calls on one GPU share the
 * array: calls that overlap on one GPU (other streams, other threads) race and give wrong
 * results; serialise them.
 */
#define AD_NOALLOC_SCRATCH_BYTES (32u << 20)
int attn_decode_noalloc(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse,
                        int32_t num_splits, void *stream);

/* Number of kernel launches attn_decode (or, for MLA head dims 576 / 512, attn_decode_mla: always
 * 2) makes for these arguments and num_splits (0 = the planner's choice): 1 when the merge runs
 * inside the partial pass, 2 when the merge kernel follows, 0 for an empty batch (e.g. to plan
 * graph capture, or to time the partial kernel on its own). Checks the arguments as the call does
 * (out is not needed). */
int attn_decode_launches(const ad_decode_args *args, const ad_paged *paged, const ad_sparse *sparse,
                         int32_t num_splits, int32_t *launches);

/* Which partial-pass kernel the calls above run for these arguments (e.g. to name it in a
 * profile): AD_KERNEL_VECTOR (vector ALUs, up to 8 query rows per work unit), the matrix cores
 * for bf16 with more than 8 rows per KV head and for every fp8 cache, as AD_KERNEL_MATRIX16
 * (16 rows per unit, when G * q_len <= 16) or AD_KERNEL_MATRIX (32 rows per unit), or
 * AD_KERNEL_MLA (head_dim_qk 576 with head_dim_v 512). The rows of a KV head's group padded to
 * 16 are the warp tile of TensorRT-LLM mha.cu (heads x tokens rounded up to a multiple of 16).
 * Honours AD_PARTIAL_KERNEL=valu / mfma and AD_MFMA_TILE=16 / 32 as the calls do (testing aids).
 * Checks the arguments as the calls do (out is not needed). On a bf16 cache the 32-row kernel
 * reads whole K / V rows and stages K through LDS when the grid holds more work groups than
 * compute units, else K goes from HBM straight to the matrix cores; both give the same bits, and
 * AD_MFMA_ROWS=0 / 1 forces either (testing aid). On an fp8 cache the 16-row kernel reads whole
 * rows and stages K through LDS unless AD_MFMA_ROWS=0 asks for half rows of 16 keys straight into
 * the operand registers (same bits again). */
#define AD_KERNEL_VECTOR 0
#define AD_KERNEL_MATRIX 1
#define AD_KERNEL_MLA 2
#define AD_KERNEL_MATRIX16 3
int attn_decode_kernel(const ad_decode_args *args, int32_t *kind);

/* attn_decode over a paged cache (paged must not be NULL); the same workspace contract. */
int attn_decode_paged(const ad_decode_args *args, const ad_paged *paged, int32_t num_splits,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * MLA decode step (FlashInfer attention/mla.cuh, BatchMLAPagedAttention): one shared latent KV
 * head (num_kv_heads = 1), head_dim_qk = 576 = 512 latent + 64 rope, head_dim_v = 512.
 *   args->q      q_nope [batch, q_len, num_q_heads, 512]
 *   args->k      ckv pool [pages, page_size, 1, 512] (strides {page, slot, head}); the values are
 *                the same latent rows, so args->v must be NULL or equal to args->k.
 *   q_pe         [batch, q_len, num_q_heads, 64] with strides q_pe_stride {b, t, hq}
 *   kpe          [pages, page_size, 1, 64] with strides kpe_stride {page, slot, head}
 * The score is scale * (q_nope . ckv_j + q_pe . kpe_j). Partial pass + merge (two launches);
 * workspace of attn_decode_workspace_size bytes, 256-byte aligned; the call needs no initial
 * contents, writes only after the counter region and leaves that region as it found it.
 */
int attn_decode_mla(const ad_decode_args *args, const void *kpe, const int64_t kpe_stride[3],
                    const void *q_pe, const int64_t q_pe_stride[3], const ad_paged *paged,
                    int32_t num_splits, void *workspace, size_t workspace_bytes, void *stream);

/*
 * MLA partial pass alone: the first half of attn_decode_mla with the same arguments, writing
 * caller-owned partials in the layout of attn_decode_splitkv (part_o [batch, q_len, num_q_heads,
 * num_splits, 512], part_lse [batch, q_len, num_q_heads, num_splits]), every slot included (a
 * split past a short sequence's end gets o = 0, lse = -inf). attn_decode_merge finishes the step.
 * args->out and args->lse are ignored.
 */
int attn_decode_mla_splitkv(const ad_decode_args *args, const void *kpe, const int64_t kpe_stride[3],
                            const void *q_pe, const int64_t q_pe_stride[3], const ad_paged *paged,
                            int32_t num_splits, float *part_o, float *part_lse, void *stream);

/*
 * Measurement aid, not part of a decode step: reads `bytes` of device memory at `src` (16-byte
 * aligned, a nonzero multiple of 16) with the load form of the partial passes -- every work group
 * streams its own contiguous region with 16-byte nontemporal loads, a wave instruction covering
 * whole 128-byte lines -- and writes AD_PROBE_SINK_WORDS 32-bit words of XOR-folded data to
 * `sink` (device) so that no load is dropped. The time of the call divided into `bytes` is the HBM
 * read rate this access form reaches, the practical ceiling the decode kernels are compared with
 * beside the published peak (the pages' kernels are likewise judged by their share of the
 * bandwidth their loads can reach).
 */
#define AD_PROBE_SINK_WORDS 4096
int attn_decode_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Message for the calling thread's last non-OK return ("" if none; every successful call clears
 * it). Valid until the thread's next call into the library. The message is the text FlashInfer
 * mla.cuh's launcher raises with its error code (the shared-memory configuration it cannot
 * serve) and TensorRT-LLM xqa mha.cu throws; a C ABI keeps it per thread instead, beside the
 * status the call returned. Never NULL; owned by the library. */
const char *attn_decode_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DECODE_H */
