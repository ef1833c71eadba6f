/*
 * pic.h -- C ABI of the position-independent KV splicing library (libpic.so, gfx950).
 *
 * The library runs the link phase of LegoLink / seam-window selective recompute on
 * one GPU.  The path of one attention layer:
 *
 *   1. pic_build_index     host planner: chunk offsets, the recompute index (the first
 *                          min(k, L_c) tokens of every chunk except chunk 0, then every
 *                          query token) and the launch schedule of the kernels.
 *   2. pic_rope_delta      in place, rotates the cached K of every chunk from its local
 *                          RoPE positions to its global offset with one direct rotation
 *                          R(delta_c) per row (pic_rope_apply: RoPE at the global
 *                          positions for a position-free cache).
 *   3. pic_splice          copies the fresh K/V of the recomputed rows into the spliced
 *                          buffers at their global positions (pic_rope_splice: steps 2
 *                          and 3 as one launch).
 *   4. pic_selective_attn  causal attention of the recomputed rows (global positions)
 *                          over every spliced key j <= p_r, GQA, flash-style on MFMA.
 *
 * Around it: pic_selective_attn_paged (steps 2-4 over chunks stored once in a shared
 * paged pool, rotation folded into the query), pic_rope_splice_pool (steps 2-3 from such a
 * pool into contiguous buffers, for pic_selective_attn), pic_decode_attn_paged (the next token of
 * every request over the same pool), pic_qkv_rope / pic_out_proj / pic_link (the
 * recomputed rows' projections and the multi-layer link) and pic_state_compose (the
 * state of a linear-attention layer composed over cached chunk summaries).
 *
 * Sources (page title and section):
 *   [EPIC]  "EPIC: Efficient Position-Independent Caching for Serving Large Language
 *           Models" walkthrough: worked 4+5+5+3 example; link_legolink Steps 1-3.
 *   [RoPE-C] 10100.com article on RoPE and prefix caching: 2.2 (RoPE rotates pairs of
 *           neighbouring dimensions by position-proportional angles), 3.3 (scheme C,
 *           rotary correction by the delta rotation, one direct kernel rather than two
 *           stacked rotations), footnote 3 (inv_freq = base^(-2i/D)).
 *   [HYPIC] joto.ai article on HYPIC: 2.1 composition of linear-layer states, 2.2 seam
 *           window (k = w = 8 per internal segment).
 *   [KV-scratch] "KV cache 从零实现：两层 Decoder、位置偏移与正确性验证": offset mask
 *           allowed[i, j] = [j <= P + i].
 *
 * Conventions shared by every call
 *   - Ownership: the caller owns every buffer, host and device (EPIC's explicit-cache
 *     API leaves cache lifetime to the user).  The library allocates no memory and
 *     keeps no state between calls, so calls are reentrant.
 *   - Streams: device calls are asynchronous on the caller's HIP stream (hipStream_t
 *     passed as void*, NULL = legacy default stream).  No call synchronises.
 *   - Errors: every argument check runs before any launch.  On a non-zero status
 *     nothing was launched and no buffer was touched.  PIC_EDEVICE reports a HIP
 *     launch error; faults inside kernels surface at the caller's next synchronise.
 *   - Layouts: token-major.  K/V buffers are [n_tokens, h_kv, head_dim]; request b
 *     owns rows req_tok_ptr[b] .. req_tok_ptr[b+1]-1; within a request the chunks'
 *     cached rows come first in chunk order, then q_b query rows.  Fresh K/V are
 *     [n_rows, h_kv, head_dim], Q and O are [n_rows, h_q, head_dim], all in the order
 *     of the recompute index (ascending position within each request, requests in
 *     order).  Elements are dense, innermost dimension contiguous.
 *   - RoPE: pair i of a head (i < D/2) is (2i, 2i+1) for PIC_ROPE_ADJACENT (the
 *     [RoPE-C] 2.2 wording) or (i, i + D/2) for PIC_ROPE_HALF (the HF layout of
 *     footnote 3); theta_i = base^(-2i/D); pair (a, b) at angle phi becomes
 *     (a cos phi - b sin phi, a sin phi + b cos phi).
 */
#ifndef PIC_H
#define PIC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  PIC_OK = 0,
  PIC_EINVAL = -1,       /* bad argument (null pointer, negative size, bad shape) */
  PIC_ENOSPC = -2,       /* caller buffer too small; the needed size is reported */
  PIC_EUNSUPPORTED = -3, /* valid but not implemented (e.g. head_dim outside the set) */
  PIC_EDEVICE = -4       /* HIP runtime error at launch */
};

/* Element types of K, V, Q, O (storage; arithmetic is fp32 on the device). */
enum { PIC_F32 = 0, PIC_BF16 = 1 };

/* RoPE pair layouts. */
enum { PIC_ROPE_ADJACENT = 0, PIC_ROPE_HALF = 1 };

/* What pic_rope_splice does to the kept cached rows: the pic_rope_delta rotation or
 * the pic_rope_apply RoPE at the target positions. */
enum { PIC_ROPE_BY_DELTA = 0, PIC_ROPE_AT_POSITION = 1 };

/* ------------------------------------------------------------------------------
 * Plan: one int32 array written by pic_build_index.  A header of
 * PIC_PLAN_HEADER_WORDS words, then sections at the word offsets the header gives.
 * ---------------------------------------------------------------------------- */
#define PIC_PLAN_MAGIC 0x31434950 /* "PIC1" */
#define PIC_PLAN_HEADER_WORDS 48
#define PIC_ATTN_TILE_M 128 /* query vectors (row, head) per attention tile */
#define PIC_ROPE_TILE_ROWS 32
#define PIC_DECODE_COLS 64   /* query columns (use, head) of one decode item */
#define PIC_DECODE_BLOCK 32    /* keys per decode block (the unit the grid is split in) */
#define PIC_DECODE_WG_PER_CU 4 /* decode workgroups resident per compute unit */

enum {
  PIC_H_MAGIC = 0,
  PIC_H_WORDS,        /* total words of the plan */
  PIC_H_N_REQ,        /* requests */
  PIC_H_N_CHUNKS,     /* chunks over all requests */
  PIC_H_N_ROWS,       /* recomputed rows over all requests (sum of R_b) */
  PIC_H_N_TOKENS,     /* spliced tokens over all requests (sum of N_b) */
  PIC_H_K,            /* recompute count per chunk c >= 1 */
  PIC_H_POS_BASE,     /* local RoPE position of each chunk's first cached row */
  PIC_H_H_Q,
  PIC_H_H_KV,
  PIC_H_TILE_ROWS,    /* recompute rows per attention tile = PIC_ATTN_TILE_M / (h_q/h_kv) */
  PIC_H_N_ROPE_TILES,
  PIC_H_N_ATTN_TILES,
  PIC_H_N_ATTN_ITEMS,
  PIC_H_N_MERGE,
  PIC_H_N_PARTIALS,   /* split-KV partial slots the attention workspace must hold */
  PIC_H_MAX_TOKENS,   /* largest N_b */
  PIC_H_O_REQ_CHUNK_PTR, /* [n_req+1] copy of the input CSR */
  PIC_H_O_CHUNK_OFF,  /* [n_chunks+n_req] per request b: off_0..off_{n_b} (last = ctx_b) */
  PIC_H_O_REQ_TOK_PTR,/* [n_req+1] first K/V row of each request; last = n_tokens */
  PIC_H_O_REQ_ROW_PTR,/* [n_req+1] first recomputed row of each request; last = n_rows */
  PIC_H_O_ROWS,       /* [n_rows] request-local global position p_r of each recomputed row */
  PIC_H_O_ROW_TOK,    /* [n_rows] K/V buffer row of each recomputed row (req_tok_ptr[b] + p_r) */
  PIC_H_O_ROPE_TILES, /* [n_rope_tiles][4]: first K row, row count, delta, global position
                         of the first row; every cached row that keeps its K, <= 32 rows
                         of one chunk per tile (tiles with delta 0 included) */
  PIC_H_O_ATTN_TILES, /* [n_attn_tiles][8]: req, first row, row count, req_tok_ptr[req],
                         p_first, p_last, req_row_ptr[req], recomputed rows of req */
  PIC_H_O_ATTN_ITEMS, /* [n_attn_items][8]: tile, kv head, key_begin, key_end,
                         partial slot (-1: writes O directly), 0, 0, 0.  Paged plans
                         store a key-block range [key_begin, key_end) instead */
  PIC_H_O_MERGE,      /* [n_merge][4]: tile, kv head, first slot, slot count */
  PIC_H_PAGED,        /* 1: chunks live in a shared paged pool (chunk_ids given) */
  PIC_H_O_SEGS,       /* paged: [n_chunks][8] off_c, L_c, n_seam_c, pool chunk id, delta_c,
                         request, 0, 0 */
  PIC_H_N_KBLOCKS,    /* paged: key blocks over all requests */
  PIC_H_O_KBLOCKS,    /* paged: [n_kblocks][4] chunk (global chunk index, or -1 for the
                         request's fresh rows), first local key (t0, or fresh row offset),
                         position of the first key, 0; per request the fresh blocks
                         come first, then the pool blocks in position order */
  PIC_H_N_DEC_ITEMS,  /* paged: decode items (0 when h_q/h_kv > PIC_DECODE_COLS) */
  PIC_H_O_DEC_ITEMS,  /* paged: [n_dec_items][4] source (pool chunk id >= 0, or -1-b for
                         the fresh rows of request b), key count, first use, use count;
                         items of one pool chunk are adjacent */
  PIC_H_N_DEC_USES,
  PIC_H_O_DEC_USES,   /* paged: [n_dec_uses] per use, the global chunk index c reading the
                         item's pool chunk (or -1-b for fresh rows); at most
                         PIC_DECODE_COLS / (h_q/h_kv) uses per item */
  PIC_H_N_DEC_RECS,   /* paged: decode partial records, each (m, l, O) of the G query
                         heads of one (piece, use) */
  PIC_H_O_DEC_REC_PTR,/* paged: [n_req * h_kv + 1] records of request b and kv head g are
                         [ptr[b*h_kv+g], ptr[b*h_kv+g+1]) */
  PIC_H_N_DEC_PIECES, /* paged: decode pieces */
  PIC_H_O_DEC_PIECES, /* paged: [n_dec_pieces][8] item, kv head, first key, end key, offset
                         of its records in piece_recs, 0, 0, 0.  The (item, kv head) units,
                         in item order, are cut into PIC_DECODE_BLOCK-key blocks and the
                         block sequence into n_dec_wg equal runs; a piece is one unit's part
                         of one run */
  PIC_H_O_DEC_PIECE_RECS, /* paged: per piece, the record of each of its item's uses */
  PIC_H_N_DEC_WG,     /* paged: decode workgroups, min(blocks, n_cu * PIC_DECODE_WG_PER_CU) */
  PIC_H_O_DEC_WG_PTR, /* paged: [n_dec_wg + 1] pieces of workgroup w are
                         pieces[ptr[w] .. ptr[w+1]) */
  PIC_H_RESERVED7
};

/*
 * pic_build_index -- host planner (integer, exact).                 [EPIC] Step 1-2
 *
 * Requests b = 0..n_req-1 hold chunks req_chunk_ptr[b] .. req_chunk_ptr[b+1]-1 with
 * lengths chunk_lens[] (>= 0) and q_lens[b] (>= 0) query tokens.  off_0 = 0,
 * off_{c+1} = off_c + L_c, ctx = off_n, N_b = ctx + q_b.  The recompute index of a
 * request lists, for c = 1..n_b-1 and j < min(k, L_c), position off_c + j, then
 * positions ctx .. N_b-1 (k >= 0; k = 0 keeps only the query rows).  Chunk 0 is never
 * recomputed.  pos_base is the local position of the first cached row of every chunk
 * (0 after a plain compile; delta_c = off_c - pos_base may be negative).
 * h_q/h_kv fix the GQA group G = h_q / h_kv (must divide PIC_ATTN_TILE_M).  n_cu is
 * the compute-unit count used to size split-KV (<= 0 selects 256).
 *
 * chunk_ids: NULL for spliced contiguous K/V buffers.  Otherwise the chunks are stored
 * once in a shared paged pool and chunk_ids[c] (>= 0) names the pool chunk of request
 * chunk c (chunk_lens[c] must be its length, the same wherever the id appears, else
 * PIC_EINVAL): the plan then has no rope tiles (the pool
 * is read-only; pic_selective_attn_paged rotates on load), and attention items walk
 * per-request key blocks (fresh rows first, then pool rows chunk by chunk).
 *
 * plan: caller-owned int32 host array of plan_cap words, or NULL to query the size.
 * *plan_words receives the size the plan needs.  Returns PIC_ENOSPC (plan untouched)
 * when plan_cap is too small, PIC_EINVAL on bad input (null pointers, negative values,
 * req_chunk_ptr not starting at 0 or decreasing, h_q % h_kv != 0, totals beyond int32)
 * and PIC_EUNSUPPORTED when G does not divide PIC_ATTN_TILE_M or some |delta_c| > 2^24.
 * A request may have no chunks (only query rows) or no query tokens.
 */
int pic_build_index(int32_t n_req, const int32_t *req_chunk_ptr, const int32_t *chunk_lens,
                    const int32_t *q_lens, const int32_t *chunk_ids, int32_t k,
                    int32_t pos_base, int32_t h_q, int32_t h_kv, int32_t n_cu, int32_t *plan,
                    int64_t plan_cap, int64_t *plan_words);

/*
 * pic_rope_delta -- rotary correction of cached K in place.          [RoPE-C] 3.3
 *
 * For every rope tile of the plan with delta_c != 0 (cached rows that are not
 * recomputed), each pair of each head of each row is rotated by the angle
 * delta_c * theta_i: one direct rotation, fp32 arithmetic with a double-float
 * angle (theta_i from fp64 on the host, exact product, Cody-Waite reduction),
 * result rounded to the storage type (RNE).  Rows that the splice overwrites and
 * chunks with delta 0 are skipped; V is never touched.
 *
 * plan_host / plan_dev: the same plan on the host and on the device.  k: device
 * buffer [n_tokens, h_kv, head_dim] of dtype.  head_dim even, head_dim % 8 == 0 for
 * PIC_ROPE_ADJACENT and head_dim % 16 == 0 for PIC_ROPE_HALF, 8 <= head_dim <= 256.
 */
int pic_rope_delta(const int32_t *plan_host, const int32_t *plan_dev, void *k, int32_t dtype,
                   int32_t head_dim, int32_t rope_layout, double rope_base, void *stream);

/*
 * pic_rope_apply -- RoPE at the target positions for a position-free cache.
 *                                                                   [RoPE-C] 3.2
 * Scheme B: the cache holds K before RoPE ("nope"); on a hit every cached row that is
 * not recomputed gets RoPE at its global position p = off_c + t (t = row within its
 * chunk; pos_base plays no role): each pair is rotated by p * theta_i, with the same
 * double-float fp32 angle, pair layouts, sizes and rounding as pic_rope_delta.  Rows
 * that the splice overwrites are skipped; V is never touched.  Arguments and errors
 * as pic_rope_delta, plus PIC_EUNSUPPORTED when a kept row sits at position >= 2^24; k
 * holds the nope rows on entry and the rotated rows on return.
 */
int pic_rope_apply(const int32_t *plan_host, const int32_t *plan_dev, void *k, int32_t dtype,
                   int32_t head_dim, int32_t rope_layout, double rope_base, void *stream);

/*
 * pic_splice -- overwrite the recomputed rows with their fresh K/V.  [EPIC] Step 3
 *
 * For every recomputed row r: k[row_tok[r]] = k_fresh[r], v[row_tok[r]] = v_fresh[r]
 * (bit copies, all h_kv heads).  k, v: device [n_tokens, h_kv, head_dim];
 * k_fresh, v_fresh: device [n_rows, h_kv, head_dim]; head_dim % 8 == 0.
 */
int pic_splice(const int32_t *plan_host, const int32_t *plan_dev, void *k, void *v,
               const void *k_fresh, const void *v_fresh, int32_t dtype, int32_t head_dim,
               void *stream);

/*
 * pic_rope_splice -- pic_rope_delta (rope_mode PIC_ROPE_BY_DELTA) or pic_rope_apply
 * (PIC_ROPE_AT_POSITION), then pic_splice, as one kernel launch.
 *                                                      [RoPE-C] 3.2-3.3, [EPIC] Step 3
 * The result is bit-identical to the two calls in that order: the rotation skips every
 * recomputed row, so the rows it rewrites and the rows the splice writes are disjoint
 * and one launch needs no ordering between them.  Arguments, sizes and errors as the
 * two calls (every check of both runs before the launch); PIC_EINVAL for another
 * rope_mode.  Plans beyond 2^22 workgroups of work run as the two launches.
 */
int pic_rope_splice(const int32_t *plan_host, const int32_t *plan_dev, void *k, void *v,
                    const void *k_fresh, const void *v_fresh, int32_t dtype, int32_t head_dim,
                    int32_t rope_layout, double rope_base, int32_t rope_mode, void *stream);

/*
 * pic_rope_splice_pool -- rotation + splice from a shared paged pool into contiguous
 * spliced K/V.                                 [RoPE-C] 3.3, [EPIC] Step 3, [HYPIC] 2.2
 * The pool (chunks stored once, carrying RoPE at local positions pos_base..; layout and
 * block table as pic_selective_attn_paged) is only read.  For a paged plan (built with
 * chunk_ids), every row of the contiguous buffers k, v [n_tokens][h_kv][head_dim] is
 * written: kept row t of request chunk c (t >= min(k, L_c), chunk 0 entirely) becomes
 * R(delta_c) applied to the pool chunk's row t (delta_c = off_c - pos_base, same angle,
 * pair layout and rounding as pic_rope_delta) and V the pool row copied; every
 * recomputed row gets its fresh K/V (bit copies).  The result is what pic_rope_delta +
 * pic_splice would leave on the gathered chunks, so pic_selective_attn with a plan
 * built from the same chunk lengths, query lengths, k and pos_base without chunk_ids
 * (whose token layout is the same) runs over it.  Rows whose pool block the chunk's
 * block-table row does not list, or whose id is outside the pool, are written as zeros.
 * One launch; no size limit on the pool (64-bit offsets).  head_dim even,
 * head_dim % 8 == 0 (PIC_ROPE_ADJACENT) or % 16 == 0 (PIC_ROPE_HALF), <= 256; bf16 or
 * f32.  Errors: PIC_EINVAL (not a paged plan, a chunk id >= n_pool_chunks, null
 * pointers, bad layout/base), PIC_EUNSUPPORTED (block_size != 16, head_dim, plans
 * beyond 2^22 workgroups), PIC_EDEVICE.
 */
int pic_rope_splice_pool(const int32_t *plan_host, const int32_t *plan_dev, const void *pool_k,
                         const void *pool_v, int64_t pool_blocks, int32_t block_size,
                         const int32_t *chunk_block_ptr, int32_t n_pool_chunks,
                         const int32_t *block_ids, void *k, void *v, const void *k_fresh,
                         const void *v_fresh, int32_t dtype, int32_t head_dim,
                         int32_t rope_layout, double rope_base, void *stream);

/* Bytes of workspace pic_selective_attn (split-KV partials; 0 if the plan has no split
 * tile) or pic_selective_attn_paged (partials, per-chunk angle table, per-key-block
 * records) needs.  Returns 0 on a bad plan as well; the attention call checks again. */
size_t pic_attn_workspace_bytes(const int32_t *plan_host, int32_t head_dim);

/*
 * pic_selective_attn -- causal attention of the recomputed rows.   [EPIC] Step 3
 *                                                      [KV-scratch] offset mask
 * For recomputed row r of request b at position p = rows[r] and query head h
 * (kv head g = h / (h_q/h_kv)):
 *   O[r, h] = sum_{j <= p} softmax_j(Q[r, h] . K[tok_b + j, g] * scale) V[tok_b + j, g]
 * over the spliced K/V of request b only.  q: device [n_rows, h_q, head_dim] (already
 * rotated at p); k, v: spliced device buffers; out: device [n_rows, h_q, head_dim]
 * of dtype.  scale: the softmax scale; a value <= 0 selects 1/sqrt(head_dim) (NaN or
 * infinity is PIC_EINVAL).  bf16 runs bf16 MFMA with fp32
 * accumulation and an fp32 online softmax; f32 runs fp32 MFMA.  head_dim in {64, 128}
 * for bf16, {16, 32, 64, 128} for f32.  workspace: device, >= pic_attn_workspace_bytes
 * (may be NULL when that is 0); contents on entry are ignored.  A paged plan (built with
 * chunk_ids) is rejected with PIC_EINVAL: it needs pic_selective_attn_paged.  A request
 * whose K (or V) rows take more than 0x7fff0000 bytes (N_b * h_kv * head_dim * dtype
 * size) is PIC_EUNSUPPORTED (32-bit buffer offsets).
 */
int pic_selective_attn(const int32_t *plan_host, const int32_t *plan_dev, const void *q,
                       const void *k, const void *v, void *out, int32_t dtype,
                       int32_t head_dim, float scale, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * pic_selective_attn_noalloc -- pic_selective_attn without a workspace argument.
 *
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same computation, arguments,
 * result bits and errors as pic_selective_attn, with the split-KV partials kept in a
 * scratch array of PIC_ATTN_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends.  The call allocates nothing.  A plan whose partials need
 * more (pic_attn_workspace_bytes > PIC_ATTN_SCRATCH_BYTES) is refused with
 * PIC_ENOSPC before anything runs; PIC_EDEVICE if the array's address cannot be
 * obtained.  Calls on one GPU share the array: calls that may overlap on one GPU
 * (several streams or threads) race and must be serialised by the caller.
 */
#define PIC_ATTN_SCRATCH_BYTES (128u << 20) /* 128 MiB per GPU */
int pic_selective_attn_noalloc(const int32_t *plan_host, const int32_t *plan_dev, const void *q,
                               const void *k, const void *v, void *out, int32_t dtype,
                               int32_t head_dim, float scale, void *stream);

/*
 * pic_selective_attn_paged -- selective attention over a shared paged chunk pool.
 *                                  [EPIC] Step 3; [RoPE-C] 3.3; [HYPIC] 2.2
 * Same result as pic_rope_delta + pic_splice + pic_selective_attn on the gathered
 * chunks, without modifying the pool: chunks are stored once, carrying RoPE at local
 * positions pos_base.., in pool_k/pool_v [pool_blocks][block_size = 16][h_kv][head_dim];
 * pool chunk i occupies the blocks block_ids[chunk_block_ptr[i] .. chunk_block_ptr[i+1]-1]
 * in order (the last one partially); chunk_block_ptr is device [n_pool_chunks + 1] and
 * block_ids device int32.  The plan must come from pic_build_index with chunk_ids, all
 * of them < n_pool_chunks (checked on the host).  chunk_block_ptr must be a CSR over
 * block_ids (non-decreasing, its last entry at most the length of block_ids).  Not
 * checkable on the host and left to the caller: each listed chunk has at least
 * ceil(L_c / 16) blocks (blocks its table row does not list read as zeros, never the
 * next row's ids), and block ids are < pool_blocks (a larger or negative id reads
 * zeros: the pool loads are range-checked).
 * k_fresh/v_fresh [n_rows][h_kv][head_dim] hold the recomputed rows (RoPE'd at their
 * global positions) and are read in place; q/out as in pic_selective_attn.  bf16: cached
 * keys of chunk c are scored in their local frame against the query rotated by -delta_c
 * (bf16 MFMA, head_dim in {64, 128}); fp32: each staged pool key is rotated by delta_c
 * into the global frame (fp32 MFMA, head_dim in {16, 32, 64, 128}); same theta and pair
 * layout as pic_rope_delta.  32-bit buffer offsets: the pool at most 0x7fff0000 bytes
 * less one 16-row block, the fresh K (and V) at most 0x7fff0000 bytes.  Pool slots past
 * a chunk's length may hold anything (NaN included).  workspace >= pic_attn_workspace_bytes(plan_host, head_dim):
 * partials, the angle table and one 32-byte record per key block (a small kernel fills
 * them from the block table before the attention kernel runs).  Errors: PIC_EINVAL (not
 * a paged plan, null pointers, a chunk id >= n_pool_chunks, NaN/infinite scale (<= 0
 * selects 1/sqrt(head_dim)), bad base/layout),
 * PIC_EUNSUPPORTED (dtype, head_dim, block_size != 16, sizes), PIC_ENOSPC (workspace),
 * PIC_EDEVICE.
 */
int pic_selective_attn_paged(const int32_t *plan_host, const int32_t *plan_dev, const void *q,
                             const void *pool_k, const void *pool_v, int64_t pool_blocks,
                             int32_t block_size, const int32_t *chunk_block_ptr,
                             int32_t n_pool_chunks, const int32_t *block_ids, const void *k_fresh, const void *v_fresh,
                             void *out, int32_t dtype, int32_t head_dim, int32_t rope_layout,
                             double rope_base, float scale, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * pic_decode_attn_paged -- one decode step over the spliced KV of a shared pool.
 *                        [EPIC] decode after the link; [HYPIC] 2.2; [RoPE-C] 3.3
 * For every request b of a paged plan, its next token (position N_b, right after its
 * q_b query tokens) attends causally over all of the request's keys: its pool chunks
 * (as pic_selective_attn_paged sees them: rotated by delta_c, seam rows replaced by
 * the fresh rows), its recomputed rows (k_fresh/v_fresh, the link's fresh buffer) and
 * itself:  out[b, h] = sum_j softmax_j(q_new[b, h] . K_b[j, g] * scale) V_b[j, g]
 * (scale <= 0 selects 1/sqrt(head_dim)).
 * Work is chunk-major: each pool chunk is read once per call for all request chunks
 * that use it (the plan's decode items), on a resident grid that walks the plan's
 * decode units.  q_new/out: device [n_req][h_q][head_dim];
 * k_new/v_new: device [n_req][h_kv][head_dim], RoPE'd at N_b; pool and fresh arguments
 * as pic_selective_attn_paged, without its fresh-row size limit.  Later decode
 * steps append the generated rows to the fresh buffer through a plan with longer
 * queries.  bf16 only, head_dim in {64, 128}, h_q/h_kv <= PIC_DECODE_COLS.
 * workspace >= pic_decode_workspace_bytes (partials + angle table).  Errors as
 * pic_selective_attn_paged, without the size cases.
 */
size_t pic_decode_workspace_bytes(const int32_t *plan_host, int32_t head_dim);
int pic_decode_attn_paged(const int32_t *plan_host, const int32_t *plan_dev, const void *q_new,
                          const void *k_new, const void *v_new, const void *pool_k,
                          const void *pool_v, int64_t pool_blocks, int32_t block_size,
                          const int32_t *chunk_block_ptr, int32_t n_pool_chunks,
                          const int32_t *block_ids, const void *k_fresh, const void *v_fresh,
                          void *out, int32_t dtype, int32_t head_dim, int32_t rope_layout,
                          double rope_base, float scale, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * pic_qkv_rope -- compute_qkv of the recomputed rows.                [EPIC] Step 2-3
 * The rows' Q, K and V from their hidden states, with RoPE at their global positions:
 * y = x W^T for x [n_rows][d_model] (bf16, plan row order) and w_qkv
 * [(h_q + 2 h_kv) * head_dim][d_model] (bf16, one row per output feature: Q heads,
 * then K heads, then V heads); q [n_rows][h_q][head_dim], k_fresh/v_fresh
 * [n_rows][h_kv][head_dim] receive bf16 results, Q and K rotated at p_r (the plan's
 * rows) with theta_i = rope_base^(-2i/head_dim) in rope_layout, V not rotated.  fp32
 * accumulation; RoPE applied before the one bf16 rounding.  workspace >=
 * pic_qkv_workspace_bytes (per-row cos/sin table).  bf16 only, head_dim in {64, 128},
 * d_model % 64 == 0, h_q*head_dim and h_kv*head_dim multiples of 128, positions < 2^24;
 * else PIC_EUNSUPPORTED.  Errors: PIC_EINVAL (null pointers, bad layout/base),
 * PIC_ENOSPC (workspace), PIC_EDEVICE.  Device pointers; caller-owned buffers.
 */
size_t pic_qkv_workspace_bytes(const int32_t *plan_host, int32_t head_dim);
int pic_qkv_rope(const int32_t *plan_host, const int32_t *plan_dev, const void *x,
                 const void *w_qkv, void *q, void *k_fresh, void *v_fresh, int32_t dtype,
                 int32_t d_model, int32_t head_dim, int32_t rope_layout, double rope_base,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * pic_out_proj -- next hidden state of the recomputed rows.          [EPIC] Step 3
 * x <- x + O W_o^T in place: o [n_rows][h_q][head_dim] (the attention output, read as
 * [n_rows][h_q*head_dim]), w_o [d_model][h_q*head_dim] (bf16, one row per output
 * feature), x [n_rows][d_model] bf16; fp32 accumulation and residual add, one bf16
 * rounding.  The pages show only compute_qkv, the splice and the attention of a
 * layer; this output projection plus residual is the plainest block that carries
 * the rows to the next layer.  bf16 only; d_model % 128 == 0, h_q*head_dim % 64 == 0;
 * else PIC_EUNSUPPORTED.  Errors as pic_qkv_rope.
 */
int pic_out_proj(const int32_t *plan_host, const void *o, const void *w_o, void *x,
                 int32_t dtype, int32_t d_model, int32_t head_dim, void *stream);

/*
 * pic_link -- the whole link over n_layers layers (contiguous K/V).  [EPIC] Step 1-3
 * For l = 0 .. n_layers-1 on one stream: pic_rope_delta(k_cache[l]);
 * pic_qkv_rope(x, w_qkv[l]) -> q, k_fresh, v_fresh; pic_splice(k_cache[l], v_cache[l]);
 * pic_selective_attn(q, k_cache[l], v_cache[l]) -> o; pic_out_proj(o, w_o[l], x).
 * w_qkv, w_o, k_cache, v_cache: host arrays of n_layers device pointers (each layer's
 * weights, and its spliced K/V buffers [n_tokens][h_kv][head_dim] holding the cached
 * chunks at their local positions, which are rotated and spliced in place).  x: the
 * rows' hidden states entering layer 0, [n_rows][d_model], updated in place to the
 * last layer's output.  q/k_fresh/v_fresh/o: caller scratch of the per-layer shapes.
 * workspace >= pic_link_workspace_bytes; scale as pic_selective_attn (<= 0 selects
 * 1/sqrt(head_dim)).  Every argument check of the per-layer calls
 * runs before the first launch; errors as those calls.  bf16 only.
 */
size_t pic_link_workspace_bytes(const int32_t *plan_host, int32_t head_dim);
int pic_link(const int32_t *plan_host, const int32_t *plan_dev, int32_t n_layers, void *x,
             const void *const *w_qkv, const void *const *w_o, void *const *k_cache,
             void *const *v_cache, void *q, void *k_fresh, void *v_fresh, void *o,
             int32_t dtype, int32_t d_model, int32_t head_dim, int32_t rope_layout,
             double rope_base, float scale, void *workspace, size_t workspace_bytes,
             void *stream);

/*
 * pic_state_compose -- linear-layer states over the chunks of every request.
 *                                                                  [HYPIC] 2.1
 * A linear-attention head keeps one state S [d_k][d_v]; a cached chunk is its
 * cumulative transition T_C [d_k][d_k] (the product of its tokens' transitions, the
 * latest on the left) and its state from a zero start S(C|0).  For every request b of
 * a paged plan and head h, over the request's chunks c in prompt order (pool chunk
 * id_c from the plan): S_c = T_{id_c} S_{c-1} + S_{id_c}(0), with S_{-1} = s_init[b][h]
 * (zero when s_init is NULL).  t_pool [n_pool_chunks][n_heads][d_k][d_k] and s_pool
 * [n_pool_chunks][n_heads][d_k][d_v] (device, fp32, row-major); prefix_out
 * [n_chunks][n_heads][d_k][d_v] receives S_c after every chunk of every request (in
 * plan chunk order; NULL skips it); final_out [n_req][n_heads][d_k][d_v] the state
 * after each request's last chunk (s_init, or zero, for a request without chunks).
 * fp32 only, d_k = d_v = 128; else PIC_EUNSUPPORTED.  Errors: PIC_EINVAL (not a paged
 * plan, a chunk id >= n_pool_chunks, null pointers, sizes <= 0), PIC_EDEVICE.
 */
int pic_state_compose(const int32_t *plan_host, const int32_t *plan_dev, int32_t n_heads,
                      int32_t d_k, int32_t d_v, const void *t_pool, const void *s_pool,
                      int32_t n_pool_chunks, const void *s_init, void *prefix_out,
                      void *final_out, int32_t dtype, void *stream);

/* Short static description of a status code. */
const char *pic_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* PIC_H */
