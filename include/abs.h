/*
 * abs.h -- C ABI of the AB-Sparse decode library for AMD Instinct MI355X (gfx950).
 *
 * AB-Sparse ("AB-Sparse: Sparse Attention with Adaptive Block Size for
 * Accurate and Efficient Long-Context Inference", arXiv 2605.12110, Pith
 * review page) is block-sparse decode attention in which every KV head has
 * its own block size.  Figure 1 of the page fixes the pipeline: one
 * representative vector (centroid) per block, a dot-product estimate of each
 * block's importance against the query, top-K selection, and exact attention
 * over the selected blocks only.  Figure 8 and the mapping figure after it
 * fix the storage: centroids quantized to INT4 (asymmetric, per channel) and
 * 16-token physical pages grouped into per-head logical blocks of
 * stride = pages per block, each head reading the same number of pages.
 * Figure 5's text fixes that block sizes are static per head (changing one
 * means rebuilding its centroids).
 *
 * Conventions for every call:
 *   - All pointers marked "device" are HIP device memory; "host" pointers are
 *     read on the host during the call only.  The caller owns every buffer;
 *     the library never allocates, frees or synchronizes (the debug checks of
 *     abs_set_debug_checks, off by default, synchronize).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Outputs are valid once that stream reaches the point
 *     after the call.
 *   - Host-side arguments are validated before anything is enqueued; on any
 *     status other than ABS_OK nothing is enqueued and no output is written,
 *     except ABS_ERR_HIP, which reports a failed launch (outputs undefined).
 *   - Device contents are trusted: page ids, selections and counts must obey
 *     the layouts below.  Kernels clamp or skip out-of-range ids rather than
 *     fault, but results are then undefined.
 *   - Calls are thread-safe; calls that share a workspace or output buffer
 *     must be ordered by the caller (same stream, or events).
 *   - No C++ exception crosses this interface.
 */
#ifndef ABS_H
#define ABS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every enum of this interface is a 32-bit integer.  Compiled as C++ its
 * underlying type is int32_t, so that any value a C caller passes (an
 * out-of-range op or status included) is a value of the type, which the
 * calls can check and reject; compiled as C it is the usual enum. */
#ifdef __cplusplus
#define ABS_ENUM(name) enum name : int32_t
#else
#define ABS_ENUM(name) enum name
#endif

typedef ABS_ENUM(abs_status) {
    ABS_OK = 0,
    ABS_ERR_INVALID_ARG = 1,  /* null pointer, bad dimension, too-small capacity */
    ABS_ERR_UNSUPPORTED = 2,  /* valid but not built: head_dim, page size, block size, group size, N */
    ABS_ERR_WORKSPACE = 3,    /* workspace smaller than abs_workspace_bytes() */
    ABS_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} abs_status;

typedef ABS_ENUM(abs_dtype) {
    ABS_F32 = 0,   /* IEEE binary32 */
    ABS_BF16 = 1   /* bfloat16 (upper half of binary32) */
} abs_dtype;

typedef ABS_ENUM(abs_op) {
    ABS_OP_BUILD = 0,    /* abs_build_centroids */
    ABS_OP_SELECT = 1,   /* abs_score_select */
    ABS_OP_DECODE = 2,   /* abs_sparse_decode */
    ABS_OP_SELECT_DECODE = 3   /* abs_select_decode */
} abs_op;

/*
 * Paged KV cache of one layer (the paged layout of the mapping figure after
 * Figure 8; PagedAttention in the page's references).
 *   k_cache, v_cache: device, [num_pages][num_kv_heads][page_size][head_dim]
 *       in kv_dtype: each (page, KV head) is one contiguous page_size x
 *       head_dim tile.
 *   page_table: device, int32 [num_seqs][max_pages_per_seq]; token t of
 *       sequence b lives in physical page page_table[b][t / 16], slot t % 16.
 *       Entries past a sequence's ceil(L_b / 16) pages are never read.
 *   seq_lens: device, int32 [num_seqs], L_b = cached tokens of sequence b,
 *       the current decode token included.  seq_lens_host: the same values on
 *       the host (launch sizes and every buffer size are computed from it; it
 *       must equal seq_lens).  The kernels clamp a device length into
 *       [1, max_b seq_lens_host[b]], so a mismatch cannot index past a
 *       buffer, but its results are undefined; abs_set_debug_checks(1)
 *       makes every call compare the two (and the page ids) first.
 * Supported: page_size 16, head_dim 64 or 128, num_kv_heads <= 64,
 * num_seqs * num_kv_heads <= 65536, num_q_heads / num_kv_heads in 1..8,
 * 1 <= L_b <= max_pages_per_seq * 16.
 */
typedef struct abs_paged_kv {
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t max_pages_per_seq;
    int64_t num_pages;
    int32_t kv_dtype;            /* abs_dtype */
    int32_t reserved0;           /* must be 0 */
    const void *k_cache;
    const void *v_cache;
    const int32_t *page_table;
    const int32_t *seq_lens;
    const int32_t *seq_lens_host;
} abs_paged_kv;

/*
 * Block-size map of one layer (the per-head block-size heatmap printed after
 * Figure 3; static per Figure 5's text).
 *   block_size_host: host int32 [num_kv_heads], each in {16, 32, 64};
 *       bs_h / 16 is the head's page stride.  The kernels take the sizes from
 *       it (they travel in the launch arguments).
 *   block_size: device int32 [num_kv_heads] or NULL.  The kernels never read
 *       it; when given, the debug checks (abs_set_debug_checks) compare it
 *       with block_size_host.
 *   centroid_off: device int64 [num_seqs * num_kv_heads + 1]; the first
 *       centroid row of (b, h) is centroid_off[b * num_kv_heads + h], with
 *       N_{b,h} = ceil(L_b / bs_h) rows.  Fill it with abs_centroid_offsets().
 */
typedef struct abs_block_map {
    const int32_t *block_size_host;
    const int32_t *block_size;
    const int64_t *centroid_off;
} abs_block_map;

/*
 * Centroid storage formats.  Figure 8 of the page compares centroid
 * precisions and keeps INT4 asymmetric per channel (ABS_CENT_INT4, the
 * default); the others are there to measure that trade-off.  Per (b, h) over
 * its blocks j, per channel d, with c the fp32 mean key:
 *   ABS_CENT_INT4: lo = min_j c, scale = (max_j c - lo) / 15,
 *       code = clamp(rint((c - lo) / scale), 0, 15); 4 bits per channel.
 *   ABS_CENT_INT4_SYM: scale = max_j |c| / 7, q = clamp(rint(c / scale),
 *       -7, 7), code = q + 8; lo = -8 * scale, so code * scale + lo = q * scale.
 *   ABS_CENT_INT8: as ABS_CENT_INT4 with 255 levels; 8 bits per channel.
 *   ABS_CENT_INT4_TENSOR: as ABS_CENT_INT4 with one range for the whole
 *       (b, h): lo and scale from the min/max over every block and channel
 *       (stored per channel, all equal).
 *   ABS_CENT_BF16: code = the bf16 bit pattern of c (round to nearest, ties
 *       to even); scale and lo are written as 0 and not used.
 * Every step that decides a code is an fp32 operation; a scale of 0 gives
 * code 0 (ABS_CENT_INT4_SYM: q = 0).
 */
typedef ABS_ENUM(abs_centroid_format) {
    ABS_CENT_INT4 = 0,
    ABS_CENT_INT4_SYM = 1,
    ABS_CENT_INT8 = 2,
    ABS_CENT_INT4_TENSOR = 3,
    ABS_CENT_BF16 = 4
} abs_centroid_format;

/*
 * Centroid store.
 *   codes: device [total_blocks][row bytes] (abs_centroid_row_bytes), 16-byte
 *       aligned.  4-bit formats: channel 2i in the low nibble of byte i,
 *       channel 2i+1 in the high nibble; ABS_CENT_INT8: one byte per channel;
 *       ABS_CENT_BF16: one little-endian uint16 per channel.
 *   scale, lo: device f32 [num_seqs][num_kv_heads][head_dim]; the
 *       dequantized centroid is code * scale + lo (ABS_CENT_BF16: the bf16
 *       value itself).
 *   format: abs_centroid_format; a zero-filled struct means ABS_CENT_INT4.
 *   reserved0: must be 0.
 */
typedef struct abs_centroids {
    uint8_t *codes;
    float *scale;
    float *lo;
    int32_t format;
    int32_t reserved0;
} abs_centroids;

/* Static text for a status code. */
const char *abs_status_str(abs_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char *abs_last_error(void);

/* Sum over (b, h) of N_{b,h} = ceil(L_b / bs_h), the number of centroid rows. */
abs_status abs_total_blocks(const abs_paged_kv *kv, const abs_block_map *map, int64_t *total);

/* Host: fill off_host[num_seqs * num_kv_heads + 1] with the running sum of
 * N_{b,h}, b-major then h (only map->block_size_host is read). */
abs_status abs_centroid_offsets(const abs_paged_kv *kv, const abs_block_map *map, int64_t *off_host);

/* Host: like abs_centroid_offsets, but every (b, h) gets room for
 * ceil(capacity_tokens / bs_h) rows, so the rows of blocks that later
 * appends create (abs_update_centroids) already exist; the centroid store
 * then needs off_host[num_seqs * num_kv_heads] rows.  capacity_tokens must be
 * at least every L_b, else ABS_ERR_INVALID_ARG. */
abs_status abs_centroid_offsets_capacity(const abs_paged_kv *kv, const abs_block_map *map,
                                         int32_t capacity_tokens, int64_t *off_host);

/* Bytes of one centroid row: head_dim / 2 (4-bit formats), head_dim
 * (ABS_CENT_INT8) or 2 * head_dim (ABS_CENT_BF16).  ABS_ERR_INVALID_ARG for
 * an unknown format or head_dim < 1. */
abs_status abs_centroid_row_bytes(int32_t head_dim, int32_t format, int64_t *bytes);

/* Largest K_{b,h} = min(N_{b,h}, max(1, floor(token_budget / bs_h))) over all
 * (b, h): the smallest row length (sel_cap) a selection buffer may have. */
abs_status abs_select_capacity(const abs_paged_kv *kv, const abs_block_map *map,
                               int32_t token_budget, int32_t *sel_cap);

/* Workspace bytes that `op` needs for these descriptors and budget (the
 * budget is ignored for ABS_OP_BUILD). */
abs_status abs_workspace_bytes(const abs_paged_kv *kv, const abs_block_map *map,
                               int32_t token_budget, abs_op op, size_t *bytes);

/*
 * Centroid build + quantization, for every (b, h) of the layer.
 * Centroid of block j of (b, h) = mean of the keys of its valid tokens
 * [j*bs_h, min((j+1)*bs_h, L_b)) (Figure 1's block representation; mean key),
 * rounded once to fp32, then coded in out->format (ABS_CENT_INT4: per (b, h,
 * channel d): lo = min_j c_j[d], scale = (max_j c_j[d] - lo) / 15 (fp32),
 * code = clamp(rint((c - lo) / scale), 0, 15) in fp32, 0 if scale == 0).
 * Writes out->codes (all total_blocks rows), out->scale, out->lo.
 */
abs_status abs_build_centroids(const abs_paged_kv *kv, const abs_block_map *map,
                               const abs_centroids *out, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Keep the centroids current while decoding.  The page fixes static per-head
 * block sizes (Figure 5's text) and INT4 per-channel centroids (Figure 8) but
 * not how they follow appended tokens; this call reads it as: after the last
 * `appended` tokens of every sequence were written to the cache (L_b counts
 * them), every block holding one of the tokens [L_b - appended - 1, L_b) --
 * always at least the last, possibly partial block -- gets its centroid
 * recomputed (mean of its valid tokens, as abs_build_centroids) and coded
 * with the (scale, lo) already in cents, clamped to the format's code range
 * (cents->format must be the format the store was built in).  The range is not
 * widened: a caller rebuilds the layer (abs_build_centroids) when it wants a
 * new one, e.g. when out_of_range grows.
 *   cents: the store written by abs_build_centroids for this layer; block j
 *       of (b, h) is row centroid_off[b * num_kv_heads + h] + j, so the
 *       offsets must leave room for blocks that appends create (use
 *       abs_centroid_offsets_capacity).
 *   appended: >= 0, the same for every sequence (0 redoes the last block).
 *   out_of_range: device int32 [num_seqs][num_kv_heads] or NULL; receives the
 *       number of (block, channel) codes of this call that were clamped (the
 *       rounded quotient outside the code range, or, for a channel with
 *       scale 0, a centroid other than lo; ABS_CENT_BF16: a finite centroid
 *       that rounds to an infinity).
 * No workspace; one launch.
 */
abs_status abs_update_centroids(const abs_paged_kv *kv, const abs_block_map *map,
                                const abs_centroids *cents, int32_t appended, int32_t *out_of_range,
                                void *stream);

/*
 * Dot-product estimation + top-K (Figure 1; the "Estimation" and "Top-K"
 * stages of the per-stage latency figure after Figure 13).  For each (b, h):
 * qbar = sum of the query heads h*G .. h*G+G-1 (G = num_q_heads /
 * num_kv_heads), score_j = qbar . (code_j * scale + lo) (ABS_CENT_BF16:
 * qbar . centroid_j), rounded to fp32; keep the K_{b,h} best blocks ranked
 * by (score desc, index asc).  bf16 centroids are evaluated in fp64; the
 * 4- and 8-bit formats as exact integer sums of code x weight after each
 * weight qbar_d * scale_d is rounded to a 30-bit multiple of a power of two
 * (one per 32 channels for 4-bit codes, per 16 for 8-bit), which moves a
 * score by at most 2.4e-7 M, M = sum_d |qbar_d| max(|lo_d|, |hi_d|) (a
 * bound on every |score|).  Equal centroids give equal scores.
 *   q: device [num_seqs][num_q_heads][head_dim] in kv_dtype.
 *   sel: device int32 [num_seqs][num_kv_heads][sel_cap]; row (b, h) gets its
 *       K_{b,h} block indices in ascending order; slots past K are not written.
 *   sel_count: device int32 [num_seqs][num_kv_heads], receives K_{b,h}.
 *   sel_cap >= abs_select_capacity(); N_{b,h} <= 65536 is supported.
 */
abs_status abs_score_select(const abs_paged_kv *kv, const abs_block_map *map,
                            const abs_centroids *cents, const void *q, int32_t token_budget,
                            int32_t *sel, int32_t sel_cap, int32_t *sel_count,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Exact attention over the selected blocks only (Figure 1's sparse attention;
 * the "Attention" stage of the figure after Figure 13), split over pages with
 * an fp32 online softmax and a log-sum-exp merge (FlashAttention, in the
 * page's references); one kernel launch, in which the last workgroup to
 * finish a (b, h) merges that head's partials.
 * For query head i of KV head h = i / G: the kept tokens are the union of
 * [j*bs_h, min((j+1)*bs_h, L_b)) over the first sel_count[b][h] entries j of
 * sel row (b, h); z_t = sm_scale * q_i . k_t;
 * out_i = sum_t softmax(z)_t v_t; lse_i = ln sum_t exp(z_t).
 *   token_budget: the budget the selection was made with (sizes the launch;
 *       sel_count[b][h] must not exceed K_{b,h} for it).
 *   out: device [num_seqs][num_q_heads][head_dim] in kv_dtype.
 *   lse: device f32 [num_seqs][num_q_heads], natural log; may be NULL.
 *   workspace: >= abs_workspace_bytes(ABS_OP_DECODE) bytes: per-(b, h)
 *       arrival counters, then fp32 partials.  The counters must be zero
 *       before the call: zero-fill the workspace before its first use, or
 *       call abs_reset_workspace(ABS_OP_DECODE).  Every completed call leaves
 *       them at zero, so a workspace keeps working as long as nothing else
 *       writes to it; after a call that did not complete (an error on the
 *       stream), reset it.  Calls that share a workspace must not overlap in
 *       time.
 */
abs_status abs_sparse_decode(const abs_paged_kv *kv, const abs_block_map *map, const void *q,
                             const int32_t *sel, int32_t sel_cap, const int32_t *sel_count,
                             int32_t token_budget, float sm_scale, void *out, float *lse,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * abs_score_select followed by abs_sparse_decode on the same query, in fewer
 * launches: the scores in one launch, then the top-K inside the decode's
 * split launch (every workgroup of a head selects the head's blocks itself
 * from the scores, keeps the positions its pages cover, and the first one
 * writes sel and sel_count).  sel, sel_count, out and lse are written as the
 * two calls write them, with the same values (the same arithmetic).  The
 * fused launch serves bf16 caches with head_dim 128 and up to 4 query heads
 * per KV head (and a split decode of at least 8 pages per workgroup), where
 * it measured faster than the separate launches: heads of at most 4096
 * blocks; heads of at most 8192 blocks with a split grid of at most two
 * workgroups per compute unit of the device; heads of up to 16384 blocks
 * with the grid within the compute units and at most 6144 blocks per head
 * on average.  Other layers run the two calls' launches, with the same
 * results.
 *   Arguments: as abs_score_select and abs_sparse_decode (token_budget is
 *   both the selection budget and the decode's).
 *   workspace: >= abs_workspace_bytes(ABS_OP_SELECT_DECODE) bytes: the select
 *       workspace (abs_workspace_bytes(ABS_OP_SELECT) bytes), then the
 *       decode workspace.  No zero-filling is needed: the first launch of
 *       the call zero-fills the decode's arrival counters.  Calls that share
 *       a workspace must not overlap in time.
 * abs_describe_launch() reports which form a layer gets and its launch shape.
 */
abs_status abs_select_decode(const abs_paged_kv *kv, const abs_block_map *map, const abs_centroids *cents,
                             const void *q, int32_t token_budget, float sm_scale, int32_t *sel,
                             int32_t sel_cap, int32_t *sel_count, void *out, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * abs_select_decode in two calls, one per side of the page's per-stage
 * latency split (the figure after Figure 13: Estimation, then Top-K and
 * Attention).  abs_estimate computes every block's score (the estimation of
 * abs_score_select) into the select region of an abs_select_decode
 * workspace; abs_topk_decode then runs the top-K and the sparse attention
 * from those scores.  The two calls on one workspace, in this order on one
 * stream, enqueue exactly the launches of abs_select_decode and give the
 * same results bit for bit; in between, the workspace holds the scores of
 * this layer and query (abs_topk_decode on any other contents gives
 * undefined results).  Arguments as abs_select_decode; abs_estimate zero-fills
 * the decode's arrival counters, so neither call needs a zero-filled
 * workspace.
 */
abs_status abs_estimate(const abs_paged_kv *kv, const abs_block_map *map, const abs_centroids *cents,
                        const void *q, int32_t token_budget, void *workspace, size_t workspace_bytes,
                        void *stream);

abs_status abs_topk_decode(const abs_paged_kv *kv, const abs_block_map *map, const void *q,
                           int32_t token_budget, float sm_scale, int32_t *sel, int32_t sel_cap,
                           int32_t *sel_count, void *out, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * abs_select_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The library keeps one scratch array of
 * ABS_STATIC_SCRATCH_BYTES in device memory per GPU, for the life of the
 * process; this call works on the current device's array and allocates
 * nothing.  Arguments, outputs and results are those of abs_select_decode
 * (bit for bit); the call clears the state that must start at zero itself.
 *   ABS_ERR_WORKSPACE, nothing enqueued, when the layer needs more than
 *   ABS_STATIC_SCRATCH_BYTES (abs_workspace_bytes(ABS_OP_SELECT_DECODE));
 *   ABS_ERR_HIP if the array's address cannot be obtained on this device.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.
 */
#define ABS_STATIC_SCRATCH_BYTES ((size_t)16 << 20)

abs_status abs_select_decode_static(const abs_paged_kv *kv, const abs_block_map *map, const abs_centroids *cents,
                                    const void *q, int32_t token_budget, float sm_scale, int32_t *sel,
                                    int32_t sel_cap, int32_t *sel_count, void *out, float *lse, void *stream);

/*
 * Launch shape of abs_select_decode / abs_sparse_decode for these
 * descriptors and budget on the current device (host only; nothing is
 * enqueued).  The decode splits each (b, h)'s selected pages over `splits`
 * workgroups of at most `pages_per_wg` pages (the page-level work unit of the
 * mapping figure after Figure 8: every head reads budget / 16 pages).
 */
typedef struct abs_launch_plan {
    int32_t splits;            /* split workgroups per (b, h) */
    int32_t pages_per_wg;      /* selected pages one split workgroup reads */
    int32_t chunk;             /* pages in registers at a time (1, 2, 4 or 8) */
    int32_t pipelined;         /* 1: the double-buffered layout */
    int32_t fused;             /* 1: abs_select_decode runs the top-K inside the decode launch */
    int32_t score_workgroups;  /* workgroups of the score launch */
    int32_t max_blocks;        /* largest N_{b,h} */
    int32_t sel_cap;           /* largest K_{b,h} */
    int32_t compute_units;     /* of the current device, as the library sized the launch for */
    int32_t reserved[7];
} abs_launch_plan;

abs_status abs_describe_launch(const abs_paged_kv *kv, const abs_block_map *map, int32_t token_budget,
                               abs_launch_plan *plan);

/*
 * Zero-fill the arrival counters of a decode workspace (op = ABS_OP_DECODE:
 * a workspace of abs_sparse_decode; ABS_OP_SELECT_DECODE: of
 * abs_select_decode), enqueued on `stream` as one small kernel (no memset, so
 * it can be captured in a graph).  Needed before the first abs_sparse_decode
 * on a workspace that was not zero-filled, and after a call that did not
 * complete.  ABS_ERR_WORKSPACE if the workspace is smaller than op needs.
 */
abs_status abs_reset_workspace(const abs_paged_kv *kv, const abs_block_map *map, int32_t token_budget, abs_op op,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Debug checks, off by default (process-wide; returns the previous setting).
 * When on, every call that enqueues work first reads back the device
 * seq_lens, the page-table entries of each sequence's pages and (when given)
 * the device block sizes, synchronizing the stream, and returns
 * ABS_ERR_INVALID_ARG, enqueuing nothing, if a length or block size differs
 * from its host copy or a page id lies outside [0, num_pages).
 */
int32_t abs_set_debug_checks(int32_t enable);

/*
 * Offline block-size calibration (Figure 3 of the page: per-head recall at
 * block sizes 16, 32 and 64, normalized by the recall at 16; the heatmap
 * after it: the resulting per-head map).  The page does not define its
 * sensitivity metric; these two calls implement this reading of it:
 *   recall of a selection for query head i = the share of i's exact
 *   attention over all L_b tokens that falls on the kept tokens; a KV head's
 *   recall at block size s = the mean of that share over the sequences and
 *   the head's query group, when every head uses block size s;
 *   a head gets the largest block size whose recall divided by its recall
 *   at 16 is at least a threshold, else 16.
 * A caller measures the recall with the calls above: for each s, a layer
 * descriptor with every block size = s, abs_build_centroids,
 * abs_score_select and abs_sparse_decode (lse -> lse_sel); once, the decode
 * with every block selected (token_budget >= every L_b, lse -> lse_full).
 */

/* recall: device f32 [num_kv_heads] = mean over b and g < G of
 * exp(lse_sel[b][h*G + g] - lse_full[b][h*G + g]) (fp64 inside).
 * lse_sel, lse_full: device f32 [num_seqs][num_q_heads] as abs_sparse_decode
 * writes them.  Only kv's num_seqs, num_q_heads and num_kv_heads are read.
 * One launch, no workspace. */
abs_status abs_head_recall(const abs_paged_kv *kv, const float *lse_sel, const float *lse_full, float *recall,
                           void *stream);

/* Host: block_size_host[h] = the largest s in {32, 64} with
 * recall_host[k(s)][h] / recall_host[0][h] >= threshold (a ratio of 1 when
 * the recall at 16 is 0), else 16; k(16) = 0, k(32) = 1, k(64) = 2.
 * recall_host: [3][num_kv_heads], each in [0, 1] (else
 * ABS_ERR_INVALID_ARG); threshold: finite, > 0. */
abs_status abs_assign_block_sizes(int32_t num_kv_heads, const float *recall_host, float threshold,
                                  int32_t *block_size_host);

/*
 * Measurement, not part of the decode step: the K/V gather of the split
 * decode (its page loop reads, for each selected page of a head, the
 * page's K and V tiles of [page_size][head_dim] storage elements) with none
 * of its arithmetic, for timing the decode's page loop against the rate at
 * which the GPU gathers the same bytes.
 *
 * Reads num_tiles tiles of tile_bytes bytes at the device addresses
 * tile_addr[0 .. num_tiles) (device u64 array; each address 16-byte
 * aligned) with the decode's non-temporal 16-byte loads: workgroups
 * workgroups of 256 threads, each wavefront a contiguous run of
 * ceil(num_tiles / (4 * workgroups)) tiles of the list, in_flight tiles
 * (1, 2, 4 or 8) in flight at a time.  xor_out (device u32 [workgroups]):
 * entry g = the XOR of every 32-bit word of the tiles workgroup g read, so
 * the XOR of all entries is the XOR of all words of all listed tiles
 * (a tile listed twice cancels).  tile_bytes must be 4096 (bf16,
 * head_dim 128, 16-token pages); num_tiles >= 1; 1 <= workgroups <= 65535;
 * otherwise ABS_ERR_INVALID_ARG.  One launch, no workspace, asynchronous on
 * `stream`.
 */
abs_status abs_gather_tiles(const uint64_t *tile_addr, int32_t num_tiles, int32_t tile_bytes, int32_t workgroups,
                            int32_t in_flight, uint32_t *xor_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ABS_H */
