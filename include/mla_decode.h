/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) absorbed-MLA decode library.
 *
 * The operation (FlashMLA new-kernel deep dive, "Theoretical analysis"; the
 * "matrices, attention & GPU" explainer, sections 5-7; FlashMLA README,
 * "Usage"): after the MLA up-projections are absorbed into the query and the
 * output projection, decoding is multi-query attention.  Every query token
 * has h_q heads of width d_qk = 576 (512 latent + 64 RoPE) and attends to one
 * shared KV head read from a paged latent cache; K is all 576 dims of a cached
 * row and V its first d_v = 512 dims:
 *
 *     out[b, i, h, :] = softmax_t(scale * q[b, i, h, :] . K_t) V_t
 *     lse[b, h, i]    = ln sum_t exp(scale * q[b, i, h, :] . K_t)
 *
 * with t ranging over the visible cache tokens (dense: the first
 * cache_seqlens[b] tokens through block_table, bottom-right causal when
 * requested; sparse: the valid top-k indices).  A query that sees no token
 * gets out = 0 and lse = -inf.
 *
 * Optional arguments (FlashMLA README, sparse attention arguments):
 *  - attn_sink [h_q] float32: a per-head sink logit; every output row is
 *    scaled by exp(lse) / (exp(lse) + exp(attn_sink[h])).  lse itself is
 *    unchanged.  NULL: no sink.
 *  - topk_length [batch, s_q] int32 (sparse only): query token (b, i) attends
 *    only to its first topk_length[b, i] index entries (values are clamped
 *    to [0, topk]).  NULL: all topk entries.  The README gives the argument
 *    per query token of its prefill call; here it is per decode query token.
 *
 * Conventions for every entry point:
 *  - Device pointers point to contiguous, row-major device memory owned by the
 *    caller; the library allocates no device memory and keeps no state other
 *    than a per-device cache of the compute-unit count.
 *  - Work is enqueued on ``stream`` (a hipStream_t; NULL = the null stream) and
 *    is asynchronous; device-side faults surface at the caller's next sync.
 *  - Argument, shape and alignment errors are reported synchronously, before
 *    anything is launched, by the returned status.  q, kv_cache, out,
 *    workspace and the metadata buffer must be 16-byte aligned.
 *  - Entry points are thread-safe; calls that share a workspace or metadata
 *    buffer must be ordered by the caller (same stream or events).
 *  - Debug mode: with the environment variable MLA_DEBUG set to "1", every
 *    entry point that reads metadata, lengths, a block table or top-k indices
 *    first synchronises ``stream``, copies those device arrays to the host and
 *    runs the checks of mla_check_inputs on them (the scheduler also checks
 *    the schedule it has just written; mla_combine checks that split_offsets
 *    is a prefix sum from 0).  A failed check prints the first offending entry
 *    to stderr and returns INVALID_ARG before anything is launched.  The mode
 *    is for eager calls: on a stream that is capturing a graph it returns
 *    INVALID_ARG.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_DECODE_ABI_VERSION 6

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1,          /* null/misaligned pointer, bad size or flag */
    MLA_ERR_UNSUPPORTED = 2,          /* well-formed but outside the supported set */
    MLA_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < mla_workspace_bytes() */
    MLA_ERR_METADATA_MISMATCH = 4,    /* metadata planned for another problem */
    MLA_ERR_HIP = 5                   /* a HIP runtime call failed */
} mla_status_t;

typedef enum {
    MLA_KV_BF16_576 = 0,  /* 576 bfloat16 per token (1152 B)                        */
    MLA_KV_FP8_656 = 1,   /* 512 e4m3fn | 4 float32 scales (1 per 128) | 64 bf16   */
    /* 512 e4m3fn | 16 float8_e8m0 scales (1 per 32 values): the 512-wide head of
     * the README copy's newer model, RoPE dims quantised too (README copy, "FP8 /
     * FP4 KV Cache Format").  d_qk = d_v = 512 (K and V are the same 512
     * values), q is [batch, s_q, h_q, 512]; top-k sparse problems only. */
    MLA_KV_FP8_528 = 2,
    /* 256 bytes of e2m1 pairs (512 values, the even-indexed one in the low
     * nibble) | 32 float8_e4m3fn scales (1 per 16 values): the FP4 record of
     * the same 512-wide head (README copy, "FP8 / FP4 KV Cache Format", where it
     * serves as the extra cache beside a 528-byte one; here a sparse cache
     * format of its own).  Same shapes and restrictions as MLA_KV_FP8_528. */
    MLA_KV_FP4_288 = 3
} mla_kv_format_t;

typedef enum { MLA_OUT_BF16 = 0, MLA_OUT_FP32 = 1 } mla_out_dtype_t;

/* Problem shape.  Supported: h_kv = 1, d_qk = 576 (512 for MLA_KV_FP8_528 and MLA_KV_FP4_288), d_v = 512, block_size = 64
 * (FlashMLA README: the key cache has one head; d_v can only be 512).  Tensor
 * layouts:
 *   q            [batch, s_q, h_q, 576]              bfloat16 ([.., 512] for the 512-wide head)
 *   kv_cache     [num_blocks, 64, 1, 576] bfloat16   or
 *                [num_blocks, 64, 1, 656] uint8 (MLA_KV_FP8_656) or
 *                [num_blocks, 64, 1, 528] uint8 (MLA_KV_FP8_528) or
 *                [num_blocks, 64, 1, 288] uint8 (MLA_KV_FP4_288)
 *   block_table  [batch, max_blocks_per_seq]         int32 page ids
 *   cache_seqlens[batch]                             int32, in [0, 64*max_blocks_per_seq]
 *   indices      [batch, s_q, topk]                  int32 page*64 + offset; -1 invalid
 *   out          [batch, s_q, h_q, 512]              bfloat16 or float32
 *   lse          [batch, h_q, s_q]                   float32 (natural log)
 */
typedef struct {
    int32_t batch;
    int32_t s_q;
    int32_t h_q;
    int32_t h_kv;
    int32_t d_qk;
    int32_t d_v;
    int32_t block_size;
    int32_t num_blocks;
    int32_t max_blocks_per_seq;  /* dense: block_table columns; may be 0 for sparse */
    int32_t topk;                /* 0 = dense decode; > 0 = top-k sparse decode     */
    int32_t causal;              /* dense only: bottom-right causal over the s_q tokens */
    int32_t kv_format;           /* mla_kv_format_t */
    int32_t out_dtype;           /* mla_out_dtype_t */
    float softmax_scale;         /* > 0; multiplies q . k before the softmax */
    /* Online-softmax running max (the flash-attention sparse-MLA note on the
     * exact running max, "threshold branch" and "measurements").  0: exact
     * running max, raised whenever a tile holds a larger score.  tau in
     * (0, 30]: lazy rescale, the running max of a row is raised only when a
     * tile's max exceeds it by more than tau, in log2 units of the scaled
     * scores, so probabilities reach up to 2^tau and the output rescale runs
     * rarely.  The result is the same softmax up to rounding; the pages
     * measure a coherent bf16 gain error on rows dominated by one key that is
     * processed last.  Not part of the metadata signature. */
    float rescale_threshold;
} mla_problem_t;

/* Split-KV schedule for one problem shape.  ``mla_plan`` fills everything
 * except ``dev``; the caller allocates ``bytes`` of device memory for ``dev``
 * and reuses the filled buffer for every call (every layer) of one decode
 * step (FlashMLA README, "Usage": metadata is made once before the layer loop).
 * Device layout of ``dev`` (int32): 8-word header, num_partitions records of 5
 * words (begin_item, begin_tile, end_item, end_tile, first_split_slot), then
 * split_offsets[batch*s_q + 1]. */
typedef struct {
    mla_problem_t sig;           /* problem the plan was made for */
    int32_t num_partitions;      /* P: workgroup columns of the split-KV grid */
    int32_t num_head_blocks;     /* ceil(h_q / 64) for dense decode over a bf16 cache, else ceil(h_q / 128) */
    int32_t fixed_overhead;      /* F: per-item cost added by the scheduler */
    int32_t max_splits;          /* upper bound of split slots: batch*s_q + P */
    void *dev;                   /* caller-owned device buffer, >= bytes */
    size_t bytes;                /* size of the device metadata */
} mla_metadata_t;

/* Library ABI version (MLA_DECODE_ABI_VERSION). */
int32_t mla_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char *mla_status_string(mla_status_t status);

/* Validate ``problem`` and fill ``meta`` (all fields but ``dev``) for a device
 * with ``num_cus`` compute units; num_cus = 0 queries the current device.
 * Pure host computation when num_cus > 0.  Errors: INVALID_ARG for null
 * pointers or impossible sizes, UNSUPPORTED for shapes outside the supported
 * set, HIP if the device query fails. */
mla_status_t mla_plan(const mla_problem_t *problem, int32_t num_cus, mla_metadata_t *meta);

/* Bytes of the split-partial workspace a decode call with this plan needs:
 * max_splits * h_q * (512 + 1) float32.  0 if ``meta`` is NULL.  Its contents
 * are internal to a decode call: with an fp32 output the partials are float32
 * (the layout mla_combine takes); with a bf16 output they are float16 scaled
 * per lane by a power of two, with the scales in the unused half. */
size_t mla_workspace_bytes(const mla_metadata_t *meta);

/* Split-KV tile scheduler.  Writes meta->dev on ``stream`` from
 * cache_seqlens (device, [batch]; dense only, ignored and may be NULL when
 * topk > 0) or, for sparse problems, topk_length (device, [batch, s_q], or
 * NULL when every query token uses all topk entries; ignored when dense).
 * The decode call must be given the same topk_length.
 * The scheduler balances KV tiles of 64 tokens (plus a fixed per-item cost)
 * over the partitions in contiguous ranges (FlashMLA new-kernel deep dive,
 * "Other performance improvements": the tile scheduler spreads requests and
 * blocks evenly over the compute units).  Errors: INVALID_ARG, UNSUPPORTED,
 * METADATA_MISMATCH if meta was planned for another problem, HIP. */
mla_status_t mla_get_decode_metadata(const mla_problem_t *problem, const int32_t *cache_seqlens,
                                     const int32_t *topk_length, mla_metadata_t *meta, void *stream);

/* Dense decode over the paged cache through block_table and
 * cache_seqlens (both device).  problem->topk must be 0.  Writes out and lse.
 * ``workspace`` holds split partials (device, >= mla_workspace_bytes(meta)).
 * The caller keeps ``meta->dev`` current: reusing metadata made from other
 * cache_seqlens silently mis-splits (the pages give the same warning).
 * attn_sink: device [h_q] float32 or NULL (see the top of this file).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, METADATA_MISMATCH, HIP. */
mla_status_t mla_decode_fwd(const mla_problem_t *problem, const void *q, const void *kv_cache,
                            const int32_t *block_table, const int32_t *cache_seqlens, const float *attn_sink,
                            const mla_metadata_t *meta, void *workspace, size_t workspace_bytes,
                            void *out, float *lse, void *stream);

/* Top-k sparse decode (DeepSeek Sparse Attention): each query token attends
 * to the cache rows listed in indices[b, i, :] (device int32, page*64 +
 * offset; block_table is not used, FlashMLA README "indices Tensor").  Entries
 * < 0 or >= num_blocks*64 are masked (the pages mark -1 invalid and do no
 * upper-bound check; this library masks instead of faulting).  problem->topk
 * must be > 0 and problem->causal 0.  topk_length (device [batch, s_q] int32
 * or NULL) and attn_sink (device [h_q] float32 or NULL) as at the top of
 * this file; the metadata must have been made with the same topk_length.
 * Same errors as mla_decode_fwd. */
mla_status_t mla_sparse_decode_fwd(const mla_problem_t *problem, const void *q, const void *kv_cache,
                                   const int32_t *indices, const int32_t *topk_length, const float *attn_sink,
                                   const mla_metadata_t *meta, void *workspace, size_t workspace_bytes,
                                   void *out, float *lse, void *stream);

/* Top-k sparse prefill (README copy, "DSA Prefill", flash_mla_sparse_fwd):
 * every query row s of q [s_q, h_q, 576] attends to the rows
 * indices[s, 0, :] (device int32 [s_q, 1, topk]; entries < 0 or >= s_kv are
 * invalid) of a flat, unpaged cache kv [s_kv, 1, 576] bfloat16 (or
 * [s_kv, 1, 656 | 528 | 288] uint8 records, problem->kv_format telling which;
 * q is [s_q, h_q, 512] with the 528- and 288-byte records), writing out [s_q, h_q, 512] and lse
 * [h_q, s_q].  It is the sparse decode of one request with s_q query tokens:
 * ``problem`` has batch = 1, s_q = the number of query rows (at most 16384
 * per call), topk > 0, causal 0 and num_blocks >= ceil(s_kv / 64); plan and
 * metadata are made as for mla_sparse_decode_fwd; topk_length ([s_q]) and
 * attn_sink ([h_q]) are optional.  The README copy gives this call on the
 * 512-wide head of its newer model; here it serves the 576-wide latent head
 * of the decode path as well as that 512-wide head.  Errors: as mla_sparse_decode_fwd, plus INVALID_ARG
 * when batch != 1 or s_kv is not in [1, num_blocks*64]. */
mla_status_t mla_sparse_prefill_fwd(const mla_problem_t *problem, int32_t s_kv, const void *q, const void *kv,
                                    const int32_t *indices, const int32_t *topk_length, const float *attn_sink,
                                    const mla_metadata_t *meta, void *workspace, size_t workspace_bytes,
                                    void *out, float *lse, void *stream);

/* LSE merge of split partials ("matrices, attention & GPU" explainer,
 * split-KV section: m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m),
 * o = (o1 l1 e^(m1-m) + o2 l2 e^(m2-m)) / l).  Item j = b*s_q + i owns the
 * split slots [split_offsets[j], split_offsets[j+1]) of
 *   o_part   [slots, h_q, 512] float32 (normalised partial outputs)
 *   lse_part [slots, h_q]      float32 (natural-log lse, -inf = empty)
 * and receives out[b, i, :, :] and lse[b, :, i].  An item with no slot, or
 * whose partials are all -inf, gets out = 0 and lse = -inf.  attn_sink
 * ([h_q] float32 or NULL) scales each merged row as at the top of this file.
 * All pointers are device memory.  Errors: INVALID_ARG, UNSUPPORTED when
 * num_items * h_q is 2^29 or more, HIP. */
mla_status_t mla_combine(int32_t num_items, int32_t h_q, int32_t s_q, const float *o_part,
                         const float *lse_part, const int32_t *split_offsets, const float *attn_sink,
                         int32_t out_dtype, void *out, float *lse, void *stream);

/* Test and measurement hook: the partial-attention kernel of mla_decode_fwd /
 * mla_sparse_decode_fwd alone, without the LSE combine.  Items whose KV range
 * lies in one partition get out and lse as usual; every other item leaves its
 * normalised partials in ``workspace`` and its out/lse untouched.
 * partial_format 0: float32 partials in the layout mla_combine takes (o_part
 * first, then lse_part at float offset max_splits*h_q*512).  partial_format 1:
 * the format mla_decode_fwd itself writes before its combine (float16 scaled
 * per lane by a power of two when the output is bf16, float32 otherwise), so
 * that the launch is the one mla_decode_fwd makes.  partial_format 2: the
 * launch mla_decode_step makes -- format 1, with the schedule computed inside
 * the kernel and written to meta->dev where mla_decode_step does that
 * (batch * s_q <= 256), format 1 otherwise.  ``table_or_indices`` is
 * block_table (dense) or indices (sparse); cache_seqlens is ignored for sparse
 * problems, topk_length for dense ones; attn_sink applies to the outputs this
 * call writes.  Same errors as mla_decode_fwd, plus INVALID_ARG for another
 * partial_format. */
mla_status_t mla_debug_decode_partial(const mla_problem_t *problem, const void *q, const void *kv_cache,
                                      const int32_t *table_or_indices, const int32_t *cache_seqlens,
                                      const int32_t *topk_length, const float *attn_sink,
                                      const mla_metadata_t *meta, void *workspace, size_t workspace_bytes,
                                      void *out, float *lse, int32_t partial_format, void *stream);

/* Test hook for the row resolution: writes, for every item j and KV slot t < tiles_j*64, the
 * physical cache row the decode kernels read for that slot, or -1 where the
 * slot is masked; rows_out is device int32 [batch*s_q, row_stride] with
 * row_stride = 64*max_blocks_per_seq (dense) or 64*ceil(topk/64) (sparse);
 * columns past an item's tiles are left untouched.  ``table_or_indices`` is
 * block_table (dense) or indices (sparse); slots past a sparse item's
 * topk_length (when given) are masked.  Errors: INVALID_ARG, UNSUPPORTED, HIP. */
mla_status_t mla_debug_gather_rows(const mla_problem_t *problem, const int32_t *table_or_indices,
                                   const int32_t *cache_seqlens, const int32_t *topk_length,
                                   int32_t *rows_out, void *stream);

/* One whole decode step in a single call: the split-KV schedule for the
 * current lengths, the partial-attention kernel and the combine.  The pages'
 * newer interface makes the metadata call a placeholder and lets the first
 * decode call compute the schedule on the device and keep it for the layers
 * and steps that follow (the "matrices, attention & GPU" explainer, split-KV
 * section; FlashMLA README, "Usage", DSA decoding); this call does the same every time it runs and
 * writes the schedule to meta->dev, so later mla_decode_fwd /
 * mla_sparse_decode_fwd calls with the same lengths can reuse ``meta``.
 * Problems with batch * s_q <= 256 (every cache format, dense or sparse)
 * compute the schedule inside the partial-attention kernel (no scheduler
 * launch); larger batches run mla_get_decode_metadata first.  Either way meta->dev ends up holding the
 * words mla_get_decode_metadata would write, and out/lse are bit-identical to
 * that call followed by the decode call.  Arguments as for those calls:
 * table_or_indices is block_table (dense, with cache_seqlens) or indices
 * (sparse, with topk_length optional); ``meta`` comes from mla_plan and must
 * have meta->dev set.  Errors: theirs. */
mla_status_t mla_decode_step(const mla_problem_t *problem, const void *q, const void *kv_cache,
                             const int32_t *table_or_indices, const int32_t *cache_seqlens,
                             const int32_t *topk_length, const float *attn_sink, const mla_metadata_t *meta,
                             void *workspace, size_t workspace_bytes, void *out, float *lse, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one whole
 * decode step -- mla_plan with ``num_cus`` (0: the device's compute units),
 * then mla_decode_step (dense, problem->topk == 0: table_or_indices =
 * block_table, cache_seqlens required; sparse: table_or_indices = indices,
 * topk_length optional) -- with the metadata and the split partials in a
 * scratch area the library holds in device memory (128 MiB per device,
 * reserved when the library is loaded on that device and kept until the
 * process ends) instead of a metadata buffer and a workspace.  The caller
 * passes inputs and outputs as for that call; the call allocates nothing
 * and makes the same kernel launches as mla_decode_step, so its outputs
 * equal those of mla_decode_step, and of the metadata call followed by the
 * decode call, bit for bit.  Every call on a device shares that device's scratch:
 * calls that may overlap on one device (different streams, threads or
 * processes without ordering) race and must be serialised by the caller.
 * Errors: those of mla_plan and mla_decode_step;
 * WORKSPACE_TOO_SMALL, before anything touches the device, when the plan
 * needs more than 64 KiB of metadata or more than 128 MiB - 64 KiB of
 * partials (mla_workspace_bytes), e.g. more than about 500 split slots of
 * 128 heads. */
mla_status_t mla_decode_step_noalloc(const mla_problem_t *problem, int32_t num_cus, const void *q,
                                     const void *kv_cache, const int32_t *table_or_indices,
                                     const int32_t *cache_seqlens, const int32_t *topk_length,
                                     const float *attn_sink, void *out, float *lse, void *stream);

/* Host-side check of the arrays a decode call reads; every pointer is host
 * memory (the MLA_DEBUG=1 mode runs it on copies of the device arrays).
 *   meta_words       the metadata buffer's int32 words as written by
 *                    mla_get_decode_metadata for ``meta`` (NULL: not checked).
 *                    They must hold the schedule of the current lengths: every
 *                    KV tile of every query token covered once, in order, with
 *                    split counts, split offsets and first split slots that
 *                    agree (reused metadata from other lengths fails here).
 *   cache_seqlens    dense: [batch], each in [0, 64*max_blocks_per_seq]
 *   table_or_indices dense: block_table, whose pages in use (the first
 *                    ceil(cache_seqlens[b]/64) of row b) lie in [0, num_blocks);
 *                    sparse: indices, whose entries before the token's top-k
 *                    length are -1 or a row in [0, num_rows) (NULL: not checked)
 *   topk_length      sparse: [batch*s_q] in [0, topk], or NULL
 *   num_rows         rows the indices may name (0: num_blocks*64; s_kv for
 *                    the prefill)
 * The decode calls mask what this check rejects (see mla_sparse_decode_fwd)
 * or clamp it (lengths); the check reports it as a caller error.  On a
 * failure ``msg`` (if not NULL) receives a one-line description of the first
 * offending entry.  Errors: INVALID_ARG (a check failed or a bad argument),
 * UNSUPPORTED (the problem), METADATA_MISMATCH (``meta`` planned for another
 * problem). */
mla_status_t mla_check_inputs(const mla_problem_t *problem, const mla_metadata_t *meta,
                              const int32_t *meta_words, const int32_t *cache_seqlens,
                              const int32_t *table_or_indices, const int32_t *topk_length, int64_t num_rows,
                              char *msg, size_t msg_len);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
