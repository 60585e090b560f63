/*
 * lit.h -- C ABI of liblit.so: the sparse-attention step of a DeepSeek-V3.2 /
 * V4.1-style model on one AMD Instinct MI355X (gfx950).
 *
 * The step has three parts, each a call below, plus a fused call:
 *   1. lit_indexer_scores : the lightning indexer scores every visible
 *      compressed-KV row for every query (head-weighted ReLU of q.k over e4m3
 *      codes with one ue8m0 scale per 32 values; lit_indexer_scores_fmt also
 *      takes fp4 e2m1 codes with the same scales);
 *   2. lit_topk           : a per-query selector keeps the index_topk best rows
 *      (lit_candidate_blocks / lit_topk_candidates: the two-level form);
 *   3. lit_sparse_attn    : attention with an online softmax over the sliding
 *      window and the selected compressed rows, one shared KV head (K = V);
 *      lit_sparse_attn_layers runs several layers over one shared list.
 *   lit_window_indices builds the window row lists; lit_sparse_step runs 1-3
 *   (window rows derived in-kernel) as one stream-ordered sequence, for one
 *   layer or several layers that share the top-k.  lit_sparse_attn_fmt reads
 *   quantised KV caches; lit_compress_append / lit_window_append write them
 *   (the cache writes of a decode step), lit_compress_chunk / lit_window_chunk
 *   those of a chunk (prefill).
 *
 * Sources (page title, symbol):
 *   [V4.1] DeepSeek-V4.1-Flash-NVFP4, inference/model.py -- module globals
 *          (fp8 and fp4 block size 32, ue8m0 scales), get_window_topk_idxs,
 *          Indexer.__init__/forward, Attention._window_kv/_compress_kv/forward
 *          (the sparse_attn call and its int32 [b, m, topk] index lists),
 *          select_candidate_blocks.
 *   [V3.2] DeepSeek-V3.2-Exp, inference/model.py -- Indexer.forward
 *          (fp8_index over e4m3 key cache + block scales), MLA.forward.
 *
 * Conventions for every call:
 *   - Pointers marked (device) are HIP device pointers, 16-byte aligned; the
 *     caller owns every buffer and keeps it alive until the stream reaches the
 *     work.  Nothing is allocated or freed inside a call.
 *   - All layouts are dense row-major in the order the brackets give.
 *     "bf16" buffers hold bfloat16 bit patterns (uint16).
 *   - stream is a hipStream_t (NULL = the default stream).  Every launch is
 *     asynchronous on it; no call synchronises the host.
 *   - Arguments are validated on the host before anything is launched; a
 *     refused call launches nothing and returns the status saying why.
 *     LIT_E_HIP reports a launch failure (the HIP error is then cleared).
 *   - Calls are thread-safe and keep no state between calls.
 */
#ifndef LIT_H
#define LIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LIT_ABI_VERSION 2

typedef enum {
    LIT_OK = 0,
    LIT_E_NULL = 1,        /* a required pointer is NULL                       */
    LIT_E_SHAPE = 2,       /* a size is negative, zero where it must not be,   */
                           /* or sizes are inconsistent with each other        */
    LIT_E_ALIGN = 3,       /* a pointer or leading dimension is misaligned     */
    LIT_E_UNSUPPORTED = 4, /* valid, but outside what the kernels implement    */
    LIT_E_WORKSPACE = 5,   /* workspace NULL or smaller than required          */
    LIT_E_HIP = 6          /* a HIP launch failed                              */
} lit_status;

/* Human-readable name of a status (static string, never NULL). */
const char *lit_status_str(int status);

/* LIT_ABI_VERSION of the loaded library. */
int lit_abi_version(void);

/*
 * lit_topk_width -- [V4.1] Indexer.forward: the number of entries of each top-k
 * row, k_eff = min(index_topk, (start_pos + S) / ratio) (integer division), or 0
 * when ratio < 1 or index_topk < 1.  Every lit_topk / lit_topk_candidates /
 * lit_sparse_step output list has this width; a query that sees fewer rows pads
 * its list with -1.  No device work; never fails.
 */
int lit_topk_width(int S, int start_pos, int ratio, int index_topk);

/*
 * lit_indexer_scores -- [V4.1] Indexer.forward (score einsum, ReLU, head-weighted
 * sum, then the -inf mask of rows a query cannot see yet); [V3.2] fp8_index.
 *
 *   scores[b,i,t] = sum_h w[b,i,h] * relu( sum_d qhat[b,i,h,d] * khat[b,t,d] )
 *   qhat = e4m3(q8) * 2^(q_sc - 127), khat = e4m3(k8) * 2^(k_sc - 127), one
 *   scale byte per 32 consecutive d.
 *
 * Row t of the compressed cache stands for tokens t*ratio .. t*ratio+ratio-1; a
 * query at position P = start_pos + i sees rows t < (P + 1) / ratio.
 *
 *   q8    (device) u8   [B, S, Hi, Di]   e4m3 codes of the index queries
 *   q_sc  (device) u8   [B, S, Hi, Di/32] ue8m0 scale bytes
 *   w     (device) f32  [B, S, Hi]       final head weights (every constant
 *                                        factor already folded in)
 *   k8    (device) u8   [B, T_cap, Di]   e4m3 index-key cache
 *   k_sc  (device) u8   [B, T_cap, Di/32] ue8m0 scale bytes of the cache
 *   scores(device) f32  [B, S, ld_scores] output; columns t < T are written,
 *                       T = (start_pos + S) / ratio; t >= visible -> -inf.
 * Requirements: Di in {64, 128}; Hi a multiple of 16, at most 64; B*S <= 65535; ratio >= 1;
 * T <= T_cap; ld_scores >= T and a multiple of 4.  A scale byte of 255 (NaN)
 * or a NaN e4m3 code gives unspecified scores.
 */
lit_status lit_indexer_scores(const uint8_t *q8, const uint8_t *q_sc, const float *w,
                              const uint8_t *k8, const uint8_t *k_sc, int B, int S,
                              int Hi, int Di, int T_cap, int start_pos, int ratio,
                              float *scores, int ld_scores, void *stream);

/*
 * Index-code formats.  Both carry one ue8m0 scale byte per 32 elements.
 *   LIT_INDEX_E4M3: one e4m3 byte per element, rows of Di bytes.
 *   LIT_INDEX_E2M1: fp4 -- [V4.1] Indexer.forward quantises the index queries
 *                   and keys to fp4 with 32-element ue8m0 blocks (fp4_act_quant
 *                   with the module's fp4 block size); two e2m1 codes per byte,
 *                   element 2j in the low nibble of byte j, rows of Di/2 bytes.
 */
typedef enum { LIT_INDEX_E4M3 = 0, LIT_INDEX_E2M1 = 1 } lit_index_format;

/*
 * lit_indexer_scores_fmt -- lit_indexer_scores with the code format of q8 and k8
 * given by index_format (a lit_index_format; q and k share it).  With
 * LIT_INDEX_E2M1, q8 is [B, S, Hi, Di/2] and k8 is [B, T_cap, Di/2] bytes; every
 * other argument, requirement and result is as above (Di is the element count).
 * An unknown format is refused with LIT_E_UNSUPPORTED.
 */
lit_status lit_indexer_scores_fmt(int index_format, const uint8_t *q8, const uint8_t *q_sc,
                                  const float *w, const uint8_t *k8, const uint8_t *k_sc, int B,
                                  int S, int Hi, int Di, int T_cap, int start_pos, int ratio,
                                  float *scores, int ld_scores, void *stream);

/*
 * lit_topk -- [V4.1] Indexer.forward (top-k, re-sorted into position order,
 * unreachable picks -> -1); [V3.2] Indexer.forward (topk of min(index_topk, T)).
 *
 * Every row (b, i) gets k_eff = min(index_topk, (start_pos + S) / ratio) entries:
 * the row numbers of its k_eff highest scores among its visible rows
 * t < (start_pos + i + 1) / ratio, in ascending order, followed by -1 in the
 * slots a short row cannot fill.  Equal scores are taken lowest row first.
 *
 *   scores (device) f32 [B, S, ld_scores]  (only visible columns are read)
 *   idx    (device) i32 [B, S, k_eff]      output
 *   ws, ws_bytes    workspace; lit_topk_workspace_bytes() gives the size
 *                   (currently 0: NULL is accepted)
 * Requirements: ld_scores multiple of 4 and >= T; NaN scores unspecified.
 */
lit_status lit_topk(const float *scores, int ld_scores, int B, int S, int start_pos,
                    int ratio, int index_topk, int32_t *idx, void *ws, size_t ws_bytes,
                    void *stream);
size_t lit_topk_workspace_bytes(int B, int S, int start_pos, int ratio, int index_topk);

/*
 * Two-level top-k ([V4.1] select_candidate_blocks and Indexer.forward with
 * candidate layers): one layer (the candidate source) keeps, per query, the
 * topk_blocks best blocks of block_size consecutive rows; the layers that use
 * them score as usual but treat every row outside those blocks as -inf before
 * their own top-k.
 *
 * lit_candidate_blocks -- level one.  A block scores the max of its visible
 * scores; the block holding the query's newest visible row, (n_vis-1)/block_size,
 * is always kept; of the others the best are kept (equal block scores: lower
 * block first) up to kb = min(topk_blocks, ceil(T / block_size)) blocks.  Blocks
 * a query cannot see are never kept.  Output per query: the kept block numbers
 * in ascending order, -1 in the slots a query with fewer visible blocks cannot
 * fill.
 *
 *   scores (device) f32 [B, S, ld_scores]  as lit_indexer_scores writes them
 *                                          (only visible columns are read)
 *   blocks (device) i32 [B, S, kb]         output
 *   ws, ws_bytes    workspace of lit_candidate_blocks_workspace_bytes() bytes
 *                   (the block scores), 16-byte aligned
 * Requirements: block_size >= 1, topk_blocks >= 0, ld_scores >= T and a multiple
 * of 4.
 */
lit_status lit_candidate_blocks(const float *scores, int ld_scores, int B, int S, int start_pos,
                                int ratio, int topk_blocks, int block_size, int32_t *blocks,
                                void *ws, size_t ws_bytes, void *stream);
size_t lit_candidate_blocks_workspace_bytes(int B, int S, int start_pos, int ratio,
                                            int block_size);
int lit_candidate_blocks_width(int S, int start_pos, int ratio, int topk_blocks,
                               int block_size);

/*
 * lit_topk_candidates -- level two: lit_topk over the scores with every row
 * outside the blocks listed for its query counted as -inf.  The result follows
 * lit_topk's contract (k_eff entries, ascending, -1 padded); when a query has
 * fewer than k_eff rows inside its blocks, the remaining picks are its lowest
 * visible rows outside them (they score -inf, and equal scores go to the lower
 * row), as a top-k over the masked scores gives.
 *
 *   blocks (device) i32 [B, S, kb]  block numbers of block_size rows, or -1;
 *                                   entries out of range are ignored
 * Requirements: as lit_topk; block_size >= 1; ceil(T / block_size) <= 65536.
 */
lit_status lit_topk_candidates(const float *scores, int ld_scores, int B, int S, int start_pos,
                               int ratio, int index_topk, const int32_t *blocks, int kb,
                               int block_size, int32_t *idx, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * lit_window_indices -- [V4.1] get_window_topk_idxs, generalised to a chunk
 * that starts after position 0.
 *
 * The window source is a ring of R slots holding position p in slot p mod R.
 * The query at P = start_pos + i attends to positions max(0, P-W+1) .. P:
 *   start_pos == 0: width min(S, W); entry j is position max(0, i-W+1) + j, or -1
 *                   when that lies past the query;
 *   start_pos  > 0: width W; entry j is position P-W+1+j (oldest first), or -1
 *                   when that is before the sequence start.
 * Each listed position is written as its slot p mod R.
 *
 *   win_idx (device) i32 [B, S, width] output (same for every b)
 * Requirements: R >= the span of needed positions (S when start_pos == 0,
 * else min(start_pos + S, W + S - 1)).
 */
lit_status lit_window_indices(int B, int S, int start_pos, int W, int R, int32_t *win_idx,
                              void *stream);
int lit_window_width(int S, int start_pos, int W);

/*
 * lit_sparse_attn -- [V4.1] Attention.forward's sparse_attn call over the window
 * KV and the compressed KV; [V3.2] MLA.forward gives the dense equivalent.
 *
 * For each (b, i, h) the row set J is the window slots listed in win_idx
 * followed by the compressed rows listed in comp_idx (-1 entries skipped,
 * repeats kept).  One bf16 row serves as key and value:
 *   l_j = scale * sum_{d<D} q[b,i,h,d] * row_j[d]
 *   out[b,i,h,d] = sum_j e^(l_j) row_j[d] / (sum_j e^(l_j) + e^(sink[h])), d < dv
 * The sink (nullable) is an extra logit per head that enters only the
 * normaliser.  An empty J gives 0.
 *
 *   q        (device) bf16 [B, S, H, D]  post-RoPE queries
 *   win_kv   (device) bf16 [B, R, D]     window source (ring slots); NULL if W == 0
 *   win_idx  (device) i32  [B, S, W]     slots, or -1
 *   comp_kv  (device) bf16 [B, T_cap, D] compressed KV; NULL if K == 0
 *   comp_idx (device) i32  [B, S, K]     rows, or -1
 *   sink     (device) f32  [H] or NULL
 *   out      (device) bf16 [B, S, H, dv] output
 *   ws, ws_bytes  workspace, lit_sparse_attn_workspace_bytes() bytes
 * Requirements: H == 16; D in {64, 128, 192, 256}; B*S <= 65535; dv a multiple of 16 and
 * <= D; R*D*2 and T_cap*D*2 (one sequence's sources in bytes) below 2^31, else
 * LIT_E_UNSUPPORTED; every listed slot < R and row < T_cap (checked on the device: an
 * out-of-range entry is treated as -1).
 */
lit_status lit_sparse_attn(const uint16_t *q, int B, int S, int H, int D, int dv,
                           const uint16_t *win_kv, int R, const int32_t *win_idx, int W,
                           const uint16_t *comp_kv, int T_cap, const int32_t *comp_idx,
                           int K, const float *sink, float scale, uint16_t *out, void *ws,
                           size_t ws_bytes, void *stream);
size_t lit_sparse_attn_workspace_bytes(int B, int S, int H, int dv, int W, int K);

/*
 * KV row formats of the attention sources ([V4.1] Attention._window_kv keeps the
 * window KV as e4m3 with the module's ue8m0 scales per 32; Attention._compress_kv
 * stores the compressed KV as fp4 in groups of 16 with e4m3 scales):
 *   LIT_KV_BF16: bf16 rows of D (the form lit_sparse_attn takes);
 *   LIT_KV_E4M3: e4m3 codes [*, D] plus ue8m0 scale bytes [*, D/32];
 *   LIT_KV_E2M1: e2m1 codes [*, D/2] (element 2j in the low nibble of byte j) plus
 *                e4m3 scale bytes [*, D/16].
 * A row's values are code * scale; they are dequantised to bf16 (exactly) as they
 * are gathered.
 */
typedef enum { LIT_KV_BF16 = 0, LIT_KV_E4M3 = 1, LIT_KV_E2M1 = 2 } lit_kv_format;

/*
 * lit_sparse_attn_fmt -- lit_sparse_attn with each source in a lit_kv_format:
 * the window source bf16 or LIT_KV_E4M3, the compressed source bf16 or
 * LIT_KV_E2M1 (others: LIT_E_UNSUPPORTED).  win_kv / comp_kv point at the
 * codes (or bf16 rows), win_scales / comp_scales at the scale bytes (NULL for
 * bf16).  The workspace is lit_sparse_attn_workspace_bytes().
 */
lit_status lit_sparse_attn_fmt(const uint16_t *q, int B, int S, int H, int D, int dv,
                               int win_format, const void *win_kv, const uint8_t *win_scales,
                               int R, const int32_t *win_idx, int W, int comp_format,
                               const void *comp_kv, const uint8_t *comp_scales, int T_cap,
                               const int32_t *comp_idx, int K, const float *sink, float scale,
                               uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/*
 * lit_sparse_attn_layers -- lit_sparse_attn for L layers that share one row list
 * and one compressed KV: [V4.1] Attention.forward / _compress_topk_idxs, where
 * the layers between index sources reuse the source's top-k list
 * (index_source_layers) and the shared compressed cache (kv_source_layers), each
 * with its own queries, window KV and sink.  Layer l's output is exactly what
 * lit_sparse_attn gives for q[l], win_kv[l], sink[l] and the shared lists.
 *
 *   q        (device) bf16 [L, B, S, H, D]
 *   win_kv   (device) bf16 [L, B, R, D]   each layer's window source; NULL if W == 0
 *   win_idx  (device) i32  [B, S, W]      shared; or NULL with W > 0: the window of
 *                                         size W is derived from start_pos, as
 *                                         lit_window_indices lists it (R must cover
 *                                         it as there)
 *   comp_kv  (device) bf16 [B, T_cap, D]  shared
 *   comp_idx (device) i32  [B, S, K]      shared
 *   sink     (device) f32  [L, H] or NULL
 *   out      (device) bf16 [L, B, S, H, dv]
 *   ws, ws_bytes  lit_sparse_attn_layers_workspace_bytes() bytes
 * Requirements: as lit_sparse_attn; L >= 1 and L*B*S <= 65535.  The workgroups of
 * one query's layers are launched side by side, so rows one layer gathers are
 * cache hits for the others.
 */
lit_status lit_sparse_attn_layers(int L, const uint16_t *q, int B, int S, int H, int D, int dv,
                                  const uint16_t *win_kv, int R, const int32_t *win_idx, int W,
                                  int start_pos, const uint16_t *comp_kv, int T_cap, const int32_t *comp_idx,
                                  int K, const float *sink, float scale, uint16_t *out, void *ws,
                                  size_t ws_bytes, void *stream);
/* W here is the window list's width (lit_window_width for a derived window). */
size_t lit_sparse_attn_layers_workspace_bytes(int L, int B, int S, int H, int dv, int W, int K);

/*
 * lit_compress_writes_row -- [V4.1] Compressor.forward (decode branch): whether
 * the decode token at start_pos completes its group of ratio tokens, so that
 * lit_compress_append writes compressed row start_pos / ratio: 1 when
 * (start_pos + 1) % ratio == 0, else 0 (also 0 for ratio < 1 or start_pos < 0).
 * No device work; never fails.
 */
int lit_compress_writes_row(int start_pos, int ratio);

/*
 * Producer side: the cache writes of one decode step ([V4.1] Compressor.forward,
 * RMSNorm.forward, apply_rotary_emb, Attention._compress_kv and _window_kv).  The
 * projections that make their inputs (wkv, wgate, kv_norm) are outside the path.
 * Quantiser readings (their kernels are not on the pages): fp4 scale = the
 * smallest e4m3 value s with 6 s >= the group's amax (amax 0: e4m3 code 1),
 * codes to the nearest e2m1 value, ties to the even code; e4m3 scale = the
 * smallest 2^e with amax <= 448 * 2^e, codes to the nearest e4m3 value, ties to
 * the even code.
 *
 * lit_compress_append -- one decode token per sequence into the compressor.  The
 * token's kv / score fill slot start_pos % ratio of kv_state / score_state; when
 * (start_pos + 1) % ratio == 0 the group's latent -- sum over the slots of
 * kv_state * softmax(score_state over the slots), per feature, cast to bf16 and
 * RMS-normalised with norm_w (fp32 math, bf16 result); for ratio 1 the norm of
 * the token's kv -- is rotated on its last rd dims at position
 * start_pos + 1 - ratio, quantised to LIT_KV_E2M1 and written to cache row
 * start_pos / ratio.  Nothing is written to the cache otherwise.
 *
 *   kv, score    (device) f32 [B, D]          the token's compressor inputs
 *   kv_state     (device) f32 [B, ratio, D]   state (ratio > 1; NULL for ratio 1);
 *   score_state  (device) f32 [B, ratio, D]   initialise kv 0, score -inf
 *   norm_w       (device) f32 [D]
 *   freqs        (device) f32 [n_pos, rd/2, 2] rotary table (cos, sin) per position
 *   codes        (device) u8  [B, T_cap, D/2] compressed cache (LIT_KV_E2M1)
 *   scales       (device) u8  [B, T_cap, D/16]
 *   latent       (device) bf16 [B, D] or NULL: the pre-rotation latent (the
 *                indexer's key projection reads it), written with the row
 * Requirements: D a multiple of 32, at most 256; rd even, <= D; the rotation
 * position < n_pos and the row < T_cap when a row is written.
 */
lit_status lit_compress_append(int B, int D, int ratio, int start_pos, const float *kv,
                               const float *score, float *kv_state, float *score_state,
                               const float *norm_w, float eps, const float *freqs, int n_pos,
                               int rd, uint8_t *codes, uint8_t *scales, int T_cap,
                               uint16_t *latent, void *stream);

/*
 * lit_window_append -- one decode token per sequence into the window ring: the
 * bf16 row kv (after kv_norm) is rotated on its last rd dims at start_pos,
 * quantised to LIT_KV_E4M3 and written to slot start_pos % R.
 *
 *   kv     (device) bf16 [B, D]
 *   freqs  (device) f32  [n_pos, rd/2, 2]
 *   codes  (device) u8   [B, R, D];  scales (device) u8 [B, R, D/32]
 * Requirements: D a multiple of 32, at most 256; rd even, <= D; start_pos < n_pos.
 */
lit_status lit_window_append(int B, int D, int start_pos, const uint16_t *kv, const float *freqs,
                             int n_pos, int rd, uint8_t *codes, uint8_t *scales, int R,
                             void *stream);

/*
 * Chunks (chunked prefill): S tokens per sequence at positions start_pos ..
 * start_pos + S - 1, by definition the S decode steps above in order, in one launch.
 * At start_pos 0 this is the pages' prefill branch ([V4.1] Compressor.forward with
 * start_pos == 0: whole groups pooled at once, the S % ratio remaining tokens left in
 * the state; Attention._window_kv prefill: the ring seeded with the chunk's last rows).
 *
 * lit_compress_chunk -- writes compressed rows start_pos / ratio ..
 * (start_pos + S) / ratio - 1 (lit_compress_chunk_rows of them): group g pooled over
 * positions g*ratio .. g*ratio + ratio - 1 (those before start_pos from the state),
 * normalised, rotated at g*ratio and quantised as in lit_compress_append.  Afterwards
 * slot r of the state holds the chunk's last token at a position = r (mod ratio), where
 * the chunk has one (the slots a later decode step reads).
 *
 *   kv, score  (device) f32 [B, S, D]
 *   latent     (device) bf16 [B, rows, D] or NULL: each written row's pre-rotation latent
 *   others as in lit_compress_append
 * Requirements: those of lit_compress_append; every rotation position < n_pos and
 * every written row < T_cap.
 *
 * lit_window_chunk -- the chunk's window rows: position p = start_pos + t rotated at p,
 * quantised to LIT_KV_E4M3 and written to slot p % R, for the last min(S, R) rows (an
 * earlier row's slot is taken again within the chunk).
 *
 *   kv     (device) bf16 [B, S, D]
 *   others as in lit_window_append; start_pos + S - 1 < n_pos.
 */
int lit_compress_chunk_rows(int start_pos, int S, int ratio);
lit_status lit_compress_chunk(int B, int S, int D, int ratio, int start_pos, const float *kv,
                              const float *score, float *kv_state, float *score_state,
                              const float *norm_w, float eps, const float *freqs, int n_pos,
                              int rd, uint8_t *codes, uint8_t *scales, int T_cap,
                              uint16_t *latent, void *stream);
lit_status lit_window_chunk(int B, int S, int D, int start_pos, const uint16_t *kv,
                            const float *freqs, int n_pos, int rd, uint8_t *codes,
                            uint8_t *scales, int R, void *stream);

/*
 * lit_sparse_step -- the whole step for one layer: lit_indexer_scores, lit_topk
 * and lit_sparse_attn, with the window rows of lit_window_indices derived
 * in-kernel from (start_pos, W, R).  [V4.1] Attention.forward with
 * _compress_topk_idxs; the -1 / position-order contract of the top-k list is
 * that of lit_topk.  Scores and attention partials live in the workspace.
 *
 * With cand_in / cand_out set the layer also takes part in the two-level top-k:
 * as the candidate source it writes lit_candidate_blocks of its own scores (its
 * own top-k stays the plain one), as a level-two layer its top-k is
 * lit_topk_candidates over cand_in.
 *
 * Decode-sized batches (B*S queries that fit the device's co-resident
 * workgroups) run as ONE kernel: a team of workgroups per query scores, selects,
 * gathers and merges, exchanging scores and partial attention states through the
 * workspace and synchronising through flags in the state buffer.  Larger
 * batches (chunked prefill) run the indexer, top-k and attention kernels in turn.
 * flags & LIT_STEP_UNFUSED forces the multi-kernel form.
 *
 * Workspace: lit_sparse_step_workspace_bytes() bytes of scratch, 256-byte
 * aligned, contents irrelevant.
 *
 * State (fused form only): lit_sparse_step_state_bytes() bytes, 256-byte
 * aligned, ZERO-FILLED ONCE before first use and afterwards passed only to
 * fused calls.  It holds, per query, a launch count and the teams' barrier
 * flags, which every fused call leaves consistent for the next, so one state
 * buffer serves calls of any shape on one stream (its size must cover the
 * largest).  With state == NULL (or too small) the step uses the multi-kernel
 * form.  State bytes [0, 4) are a sticky error word: nonzero means a fused
 * call's team did not assemble within its bounded wait (its workgroups were not
 * all resident, e.g. another kernel held compute units); that call's outputs
 * are undefined.  Zero the whole state to clear it.  Calls that share a
 * workspace or a state must be ordered on one stream.
 */
#define LIT_STEP_UNFUSED 1
typedef struct lit_step_args {
    /* positions */
    int B, S, start_pos, ratio;
    /* indexer (code rows are Di bytes, or Di/2 with index_format LIT_INDEX_E2M1) */
    int Hi, Di, index_topk, T_cap;
    const uint8_t *q8;   /* [B,S,Hi,Di]      */
    const uint8_t *q_sc; /* [B,S,Hi,Di/32]   */
    const float *w;      /* [B,S,Hi]         */
    const uint8_t *k8;   /* [B,T_cap,Di]     */
    const uint8_t *k_sc; /* [B,T_cap,Di/32]  */
    /* attention */
    int H, D, dv, W, R;
    const uint16_t *q;       /* [B,S,H,D] bf16     */
    const uint16_t *win_kv;  /* [B,R,D] bf16       */
    const uint16_t *comp_kv; /* [B,T_cap,D] bf16   */
    const float *sink;       /* [H] or NULL        */
    float scale;
    /* outputs */
    int32_t *topk_idx; /* [B,S,k_eff]  (device) */
    uint16_t *out;     /* [B,S,H,dv] bf16        */
    /* optional timing: hipEvent_t handles (each may be NULL) recorded on the stream
     * before the indexer, after the indexer, after the top-k and after the
     * attention, so a caller can time the stages without a profiler */
    void *stage_events[4];
    /* fused-form state (see above); NULL selects the multi-kernel form */
    void *state;
    size_t state_bytes;
    int flags; /* LIT_STEP_* bits */
    int index_format; /* lit_index_format of q8 / k8 (0 = LIT_INDEX_E4M3) */
    /* two-level top-k (lit_candidate_blocks / lit_topk_candidates); unused when
     * cand_in and cand_out are both NULL.  A level-two layer with 1..2048 blocks per
     * query can run fused; so can a candidate source whose cand_block_size divides
     * the fused members' score chunks (any divisor of 256 does): the fused kernel
     * writes the block maxima and one top-k kernel over them follows it. */
    const int32_t *cand_in; /* [B,S,cand_k]: level two -- this layer's rows outside
                               these blocks count as -inf before its top-k */
    int cand_k;
    int32_t *cand_out;      /* [B,S,kb]: candidate source -- this layer writes its
                               kept blocks (kb = lit_candidate_blocks_width) */
    int cand_topk_blocks;
    int cand_block_size;    /* rows per block, for cand_in and cand_out */
    /* quantised attention KV (lit_kv_format; 0 = bf16): win_kv / comp_kv then hold the
     * codes (cast to the field's type) and these the scale bytes.  Both sources
     * quantised (window LIT_KV_E4M3, compressed LIT_KV_E2M1) run fused, with or
     * without level two and layers; one quantised source alone runs as kernels. */
    int win_kv_format;
    const uint8_t *win_kv_scales;
    int comp_kv_format;
    const uint8_t *comp_kv_scales;
    /* layers sharing this step's top-k (0 or 1: one).  With layers = L > 1, q, win_kv
     * (and win_kv_scales), sink and out hold L layers back to back -- q [L,B,S,H,D],
     * win_kv [L,B,R,*], sink [L,H], out [L,B,S,H,dv] -- and every layer attends over the
     * one top-k list and comp_kv ([V4.1] index_source_layers / kv_source_layers).  They
     * run fused with either KV format and with or without level two. */
    int layers;
} lit_step_args;

lit_status lit_sparse_step(const lit_step_args *args, void *ws, size_t ws_bytes, void *stream);
size_t lit_sparse_step_workspace_bytes(const lit_step_args *args);
/* State bytes the fused form needs for these sizes (0 when it does not apply). */
size_t lit_sparse_step_state_bytes(const lit_step_args *args);

/*
 * lit_sparse_step_noalloc -- lit_sparse_step for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the workspace and the fused form's state are the library's own scratch,
 * a 16 MiB device array per GPU that lives until the process ends.  The call allocates
 * and frees nothing.  args->state / state_bytes are ignored.
 *
 *   err_word  (device) u32, or NULL: a fused team timeout ORs a nonzero value into it
 *             (the caller zero-fills it; NULL: such a timeout is not reported and that
 *             call's outputs are undefined)
 *
 * The first MiB holds the fused form's state (shapes whose state needs more run as
 * kernels); the remaining 15 MiB are the workspace: a shape whose
 * lit_sparse_step_workspace_bytes exceeds 15 MiB (e.g. a 4096-query prefill chunk) is
 * refused with LIT_E_WORKSPACE before anything is launched.  Every call on one GPU
 * shares that GPU's scratch, which keeps the last call's contents: calls that overlap
 * on one GPU (other streams, other host threads) race and must be ordered by the caller.
 */
lit_status lit_sparse_step_noalloc(const lit_step_args *args, uint32_t *err_word, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIT_H */
