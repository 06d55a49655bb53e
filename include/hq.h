/*
 * hq.h -- C ABI of the hybrid K4V4/FP16 decode-attention library (libhq.so).
 *
 * The method (HyQuant: hybrid-precision quantization for LLM attention) keeps
 * a small set of "vertical-line" key positions and the most recent window of
 * W tokens in FP16, stores every other cached token as packed 4-bit keys and
 * values (K4V4), and fuses the dequantisation into the decode attention scan
 * so no full-precision cache is ever materialised.  Sources, by page title:
 *   - agihunt.info digest "HyQuant: Hybrid-Precision Quantization for LLM
 *     Attention", method paragraph: the three-way key partition (vertical
 *     lines / recent window / quantised rest), the column-attention-mass
 *     score, top-rho over the non-window prefix (default 5 %), at most 64
 *     buffered FP16 queries, a lightweight reduction every 64 tokens;
 *     decode paragraph: dequantisation fused into the attention scan, the
 *     vertical-line set chosen on prefill-tail queries and kept fixed during
 *     decode, new tokens staged first and then merged into the hybrid layout.
 *   - HyQuant README, "Overview" items 1 and 3 (running column-mass score;
 *     K4V4 + FP16 cache, online softmax over quantised blocks), "Overhead"
 *     and "Mode reference" (window_size, top_ratio).
 *
 * 4-bit layout (the pages say only "K4V4"; this library fixes it): per token
 * and per group of 32 consecutive head_dim elements, asymmetric uint4 codes
 * with an fp16 {scale, min}: scale = fp16_rne((max - min) / 15), code =
 * clamp(round_half_even((x - min) / scale), 0, 15) (all 0 when scale == 0),
 * x_hat = code * scale + min.  Byte j of a packed row holds element 2j in the
 * low nibble and element 2j+1 in the high nibble.  b-bit codes (b = 2, 8)
 * follow the same rule with 2^b - 1 in place of 15, 8/b codes per byte, the
 * lower element in the lower bits.
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major,
 *     16-byte aligned (HQ_ERR_ALIGN otherwise), except the cache's int32
 *     position arrays and counters (q_pos, vl_pos, n_q, n_vl, n_stg), which
 *     need 4 bytes, so that one sequence's slice of a batch cache is a
 *     valid B = 1 cache.  fp16 data is passed as the
 *     raw uint16_t bit patterns.  The library allocates nothing and keeps no
 *     state between calls.
 *   - Calls are asynchronous on `stream`.  All argument checks run on the host
 *     before anything is launched; on an error nothing is launched and no
 *     output is touched.  A launch failure returns HQ_ERR_HIP.
 *   - head_dim d must be 128 (HQ_ERR_UNSUPPORTED otherwise); Hq % Hkv == 0;
 *     B * Hkv <= 65535 (HQ_ERR_ARG otherwise);
 *     query head h uses KV head h / (Hq / Hkv).  A "unit" is one
 *     (sequence b, KV head) pair; units are independent.
 *   - The softmax scale is 1/sqrt(d); logsumexp outputs are natural-log.
 *   - Calls that write the same cache or workspace must not run concurrently
 *     on different streams.
 */
#ifndef HQ_H
#define HQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HQ_OK               0
#define HQ_ERR_ARG         -1   /* null pointer, bad shape or out-of-range scalar */
#define HQ_ERR_UNSUPPORTED -2   /* head_dim other than 128, or a code width other than 2/4/8 */
#define HQ_ERR_ALIGN       -3   /* a tensor pointer not 16-byte aligned */
#define HQ_ERR_CAPACITY    -4   /* a cache region too small for the request */
#define HQ_ERR_WORKSPACE   -5   /* workspace missing or smaller than required */
#define HQ_ERR_HIP         -6   /* a HIP launch or runtime call failed */
#define HQ_ERR_SCRATCH     -7   /* request larger than hq_decode_attn_noalloc's static scratch */

/* Problem shape: batch, query/KV heads, head_dim, window W, vertical-line
 * ratio rho in [0, 1], the capacities (tokens per unit) of the quantised,
 * vertical-line and staging regions of a cache, and the code widths of the
 * quantised keys and values: 2, 4 or 8 bits each (0 means 4).  K4V4 is the
 * method's cache; K8V8, K4V2 and K2V4 are the other strict low-bit caches of
 * the README's mode table, with or without vertical lines.  A caller with
 * per-layer value widths passes each layer's dims. */
typedef struct {
  int32_t B, Hq, Hkv, d;
  int32_t W;
  double rho;
  int32_t cap_q, cap_vl, cap_stg;
  int32_t k_bits, v_bits;
} hq_dims;

/* One layer's hybrid cache.  u = b * Hkv + kv_head indexes the units.
 *   kq, vq        [B][Hkv][cap_q][d*k_bits/8], [..][d*v_bits/8]
 *                                          packed K and V codes (d/2 bytes
 *                                          a token at 4 bits)
 *   kq_meta,      [B][Hkv][cap_q][d/32][2] fp16 {scale, min} per group
 *   vq_meta
 *   q_pos         [B][Hkv][cap_q]          source position of each K4V4 slot;
 *                                          slots are in ascending position
 *   kvl, vvl      [B][Hkv][cap_vl][d]      fp16 vertical-line tokens
 *   vl_pos        [B][Hkv][cap_vl]         their positions
 *   kwin, vwin    [B][Hkv][W][d]           fp16 window ring, slot = pos mod W
 *   kstg, vstg    [B][Hkv][cap_stg][d]     fp16 staging (the newest token)
 *   n_q, n_vl,    [B][Hkv]                 device counters: tokens held in the
 *   n_stg                                  K4V4, vertical-line and staging
 *                                          regions of each unit
 *   k4_pages      [B][Hkv][cap_q/32] or NULL: paged K4V4 slots (below)
 * kwin/vwin may be NULL when W == 0.
 *
 * Paged K4V4 slots: with k4_pages set, kq, vq, kq_meta, vq_meta and q_pos are
 * pools of 32-slot blocks shared by all units ([P*32][...] with the same
 * per-slot rows), and slot s of unit u lives in pool block
 * k4_pages[u][s / 32], row s mod 32.  cap_q must then be a multiple of 32.
 * The caller allocates the pool and assigns the blocks (each block to at
 * most one (unit, index) pair, every index below P); a sequence's units
 * need blocks only for the slots their positions can reach, so a ragged
 * batch does not reserve every sequence's K4V4 region for the longest
 * one.  Every entry point reads and writes the slots through the table. */
typedef struct {
  uint8_t *kq, *vq;
  uint16_t *kq_meta, *vq_meta;
  int32_t *q_pos;
  uint16_t *kvl, *vvl;
  int32_t *vl_pos;
  uint16_t *kwin, *vwin;
  uint16_t *kstg, *vstg;
  int32_t *n_q, *n_vl, *n_stg;
  int32_t *k4_pages;
} hq_cache;

/* Operation ids for hq_workspace_bytes. */
#define HQ_OP_SELECT 1
#define HQ_OP_DECODE 2
#define HQ_OP_PREFILL 3

/*
 * hq_select_vertical -- column-mass score and top-rho vertical-line set
 * (agihunt digest, method paragraph; README Overview item 1).
 *
 * For every unit, each buffered query j (position p_j = L - nb + j) of each
 * query head of the unit's group has a causal softmax row over keys 0..p_j.
 * The row's probabilities at the non-window columns i < L - W are summed over
 * heads and queries and ADDED to score_inout[b][kvh][i] (a running score;
 * zero it before the first refresh).  Columns i >= L - W are left unchanged.
 * Then the n_vl = floor(rho * (L - W) + 1e-6) columns of [0, L - W) with the
 * largest accumulated score are selected, ties going to the lower position.
 *
 *   qbuf        [B][Hq][nb][d] fp16, 1 <= nb <= min(64, L)
 *   k           [B][Hkv][L][d] fp16 dense keys of the prefix
 *   lse_or_null [B][Hq][nb] fp32 natural-log LSE of each buffered row, or
 *               NULL to compute it here (a first pass over the keys)
 *   score_inout [B][Hkv][L] fp32
 *   vl_idx      [B][Hkv][n_vl] int32 out: selected positions, ascending
 *   vl_flag     [B][Hkv][L] uint8 out: 1 at selected positions, else 0
 *   ws          device workspace of at least
 *               hq_workspace_bytes(dims, HQ_OP_SELECT, L) bytes (scratch:
 *               no initial contents are required)
 * Only dims->B, Hq, Hkv, d, W, rho are read.  Requires L >= 1.
 */
int hq_select_vertical(const hq_dims* dims, const uint16_t* qbuf, int32_t nb,
                       const uint16_t* k, int32_t L, const float* lse_or_null,
                       float* score_inout, int32_t* vl_idx, uint8_t* vl_flag,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hq_quant_pack -- build the hybrid cache of a prefix 0..L-1 (agihunt
 * digest, decode paragraph; README Overview item 3).
 *
 * Window positions [max(0, L-W), L) are copied to ring slot (pos mod W).
 * Non-window positions flagged in vl_flag [B][Hkv][L] are copied in
 * ascending position to the vertical-line region (the first cap_vl of them;
 * any beyond cap_vl are treated as unflagged).  Every other non-window
 * position is quantised and stored in ascending position in the K4V4 region.
 * Counters are set; nothing is staged (n_stg = 0).
 * Requires cap_q >= max(0, L - W) (HQ_ERR_CAPACITY) and L >= 0.
 */
int hq_quant_pack(const hq_dims* dims, const uint16_t* k, const uint16_t* v,
                  int32_t L, const uint8_t* vl_flag, const hq_cache* cache,
                  hipStream_t stream);

/*
 * hq_append_merge -- stage the token at position t and merge the one staged
 * before it (agihunt digest, decode paragraph).
 *
 * If a token is staged (position t-1): with W > 0 it moves to ring slot
 * (t-1) mod W, and the token that slot held (position t-1-W, when >= 0)
 * leaves the window; with W == 0 the staged token itself leaves.  A leaving
 * token goes to the vertical-line region when evict_is_vl[u] is nonzero and
 * the region has room, else it is quantised and appended to the K4V4 region.
 * Then k_new/v_new [B][Hkv][d] fp16 are staged (n_stg = 1).
 * evict_is_vl_or_null: [B][Hkv] uint8, or NULL for all zero (the fixed
 * vertical-line set of the pages).  Requires cap_stg >= 1 and
 * cap_q >= max(0, t - W) (HQ_ERR_CAPACITY), t >= 0.
 */
int hq_append_merge(const hq_dims* dims, const hq_cache* cache, int32_t t,
                    const uint16_t* k_new, const uint16_t* v_new,
                    const uint8_t* evict_is_vl_or_null, hipStream_t stream);

/*
 * hq_decode_attn -- one decode query per head over the hybrid cache
 * (agihunt digest, decode paragraph; README Overview item 3).
 *
 * Query q [B][Hq][d] fp16 at position L attends to the unit's K4V4 slots
 * (dequantised in registers), its vertical-line tokens, the window ring
 * positions [max(0, L-W), L) and the staged tokens, in one online softmax
 * split over the sequence and merged by log-sum-exp.  Writes
 * out [B][Hq][d] fp16 and, if lse_or_null is not NULL, the natural-log
 * logsumexp [B][Hq] fp32.  A head with no keys at all gets out = 0 and
 * lse = -inf.
 *
 * ws: at least hq_workspace_bytes(dims, HQ_OP_DECODE, L) bytes.  Its first
 * 128*B*Hkv bytes hold the arrival counters (one int32 per unit, 128 bytes
 * apart), which must be zero before the first call that uses this workspace
 * (allocate it zero-filled); every completed call leaves them zero again.
 * Requires L >= 0.
 */
int hq_decode_attn(const hq_dims* dims, const hq_cache* cache, int32_t L,
                   const uint16_t* q, uint16_t* out, float* lse_or_null,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hq_decode_attn_noalloc -- hq_decode_attn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): no workspace argument; the arrival counters and
 * partial records live in a static device array of the library, 8 MiB per
 * GPU, held until the process ends.  Arguments, result and the other errors
 * as hq_decode_attn.
 *   - Limit: at most 4096 units (B * Hkv), and the records of the call's
 *     split plan (units * splits * Hq/Hkv * 528 bytes) within the
 *     7.5 MiB after the counters; larger requests return HQ_ERR_SCRATCH
 *     before anything is launched.  (The Qwen3-32B-shaped layer at B = 32
 *     and L = 32K needs 2.2 MB.)
 *   - The first call on a GPU looks the array up (hipGetSymbolAddress, with
 *     that GPU current) and clears its counters with a fill kernel on
 *     `stream`; every completed call leaves them zero again.
 *   - Every call on one GPU uses the same array: calls that overlap on one
 *     GPU (concurrent streams, host threads) race and must not be issued.
 * Calls no hipMalloc, hipFree or other allocating routine.
 */
int hq_decode_attn_noalloc(const hq_dims* dims, const hq_cache* cache, int32_t L,
                           const uint16_t* q, uint16_t* out, float* lse_or_null,
                           hipStream_t stream);

/*
 * hq_refresh_hybrid -- decode-time refresh of the running vertical-line
 * score over the hybrid cache, and the cut-off a leaving token must reach
 * (agihunt digest, method paragraph: the column-mass score is a running
 * estimate over at most 64 buffered FP16 queries, refreshed every 64 tokens;
 * README Overview item 1).
 *
 * The cache is the one at decode position t, as hq_quant_pack and
 * hq_append_merge leave it: the K4V4 and vertical-line regions hold the
 * positions below t - W, the window ring positions max(0, t - W) .. t - 1,
 * and the staging region the token at t (at most one staged token is read).
 * A K4V4 key is code * scale + min; the kernel rounds each element of it to
 * fp16 for the matrix cores (relative error at most 2^-11).  Buffered
 * query j of each query head (position p_j = t - nb + 1 + j) adds, for every
 * cached key at a position i <= p_j, exp(q.k_i / sqrt(d) - lse_j) to
 * score_inout[b][kvh][i], summed over the unit's heads and queries; lse_j is
 * the row's natural-log logsumexp from its own decode step.  Then the
 * n_vl = floor(rho * (t - W) + 1e-6) positions of [0, t - W) with the largest
 * running score are selected (ties to the lower position) into vl_idx and
 * vl_flag, and cut_out receives the n_vl-th largest running score (+inf
 * when n_vl = 0): hq_append_merge_scored promotes a leaving token whose score
 * reaches it.
 *
 *   qbuf        [B][Hq][nb][d] fp16, the last nb decode queries, 1 <= nb <= 64,
 *               nb <= t + 1
 *   lse         [B][Hq][nb] fp32
 *   score_inout [B][Hkv][score_ld] fp32, score_ld >= t + 1 (a running score;
 *               zero it before the first refresh)
 *   vl_idx      [B][Hkv][n_vl] int32 out, ascending (may be NULL when n_vl = 0)
 *   vl_flag     [B][Hkv][score_ld] uint8 out: 1 at selected positions, else 0
 *   cut_out     [B][Hkv] fp32 out
 * Keys a cache holds beyond positions 0..t are not scored; positions outside
 * [0, score_ld) are skipped.  Requires t >= 0.
 */
int hq_refresh_hybrid(const hq_dims* dims, const hq_cache* cache, int32_t t,
                      const uint16_t* qbuf, int32_t nb, const float* lse,
                      float* score_inout, int32_t score_ld, int32_t* vl_idx,
                      uint8_t* vl_flag, float* cut_out, hipStream_t stream);

/*
 * hq_append_merge_scored -- hq_append_merge where the token leaving the
 * window becomes a vertical line exactly when its running score reaches the
 * unit's cut-off: score[b][kvh][pos] >= cut[b][kvh] (agihunt digest, method
 * and decode paragraphs; README Overview item 1).
 *
 *   score [B][Hkv][score_ld] fp32, score_ld >= max(t, 1)
 *   cut   [B][Hkv] fp32 (from hq_refresh_hybrid)
 * Everything else, including the capacity rules, is as in hq_append_merge.
 */
int hq_append_merge_scored(const hq_dims* dims, const hq_cache* cache, int32_t t,
                           const uint16_t* k_new, const uint16_t* v_new,
                           const float* score, int32_t score_ld, const float* cut,
                           hipStream_t stream);

/*
 * hq_append_merge_ragged, hq_decode_attn_ragged -- the per-step operations
 * of a ragged batch, each sequence at its own position (a serving batch of
 * sequences of different lengths; the 32K-prefix batch-capacity runs of the
 * agihunt digest, results paragraph, and the HyQuant README, Highlights).
 *
 *   t_seq / L_seq  [B] int32 DEVICE array: sequence b's new token / query
 *                  position; values are clamped to [0, t_max] / [0, L_max]
 *   t_max / L_max  host bound on every sequence's position: the capacity
 *                  checks and the decode's split plan use it
 * Otherwise exactly hq_append_merge / hq_decode_attn (the decode's workspace
 * is hq_workspace_bytes(dims, HQ_OP_DECODE, L_max)).  Sequences shorter than
 * their cache's capacity simply use fewer slots; to build the cache of a
 * ragged batch, hq_quant_pack (and hq_select_vertical) run per sequence on
 * B = 1 views of the cache (pointers advanced by b * Hkv units).
 */
int hq_append_merge_ragged(const hq_dims* dims, const hq_cache* cache, const int32_t* t_seq,
                           int32_t t_max, const uint16_t* k_new, const uint16_t* v_new,
                           const uint8_t* evict_is_vl_or_null, hipStream_t stream);
int hq_decode_attn_ragged(const hq_dims* dims, const hq_cache* cache, const int32_t* L_seq,
                          int32_t L_max, const uint16_t* q, uint16_t* out, float* lse_or_null,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hq_decode_step -- one decode step in one launch: hq_append_merge of the
 * token at position t followed by hq_decode_attn at t, with the same result
 * (agihunt digest on HyQuant, decode paragraph: new tokens are staged, then
 * merged into the hybrid layout; the attention scan dequantises in place).
 *
 *   t            position of the new token (the query's position)
 *   k_new, v_new [B][Hkv][d] fp16 rows of the new token
 *   evict_is_vl_or_null [B][Hkv] u8: the token leaving the window becomes a
 *                vertical line (as in hq_append_merge)
 *   q, out, lse_or_null, ws, ws_bytes  as in hq_decode_attn
 * The query attends to the cache's K4V4 slots, vertical lines and window
 * (positions max(0, t-W) .. t-1) and to the new token itself.  Afterwards
 * the token at t - W (with W = 0: the new token) has left the window (into
 * the next K4V4 slot, or the vertical-line region when flagged) and the new
 * token sits in the ring at slot t mod W, so that nothing is staged.
 * Precondition: nothing is staged (n_stg = 0, as after hq_quant_pack or a
 * previous hq_decode_step); the window holds positions max(0, t-W) .. t-1.
 * Mixing with hq_append_merge / hq_decode_attn is allowed in that state: a
 * plain hq_append_merge at t then stages t and moves nothing.  The staging
 * count lives on the device, so the precondition is checked there: a unit
 * with a staged token is refused, its out rows and lse entries are set to
 * NaN and its cache is left unchanged (the other units step normally).
 * Errors: as hq_decode_attn; HQ_ERR_CAPACITY when cap_q < t + 1 - W.
 */
int hq_decode_step(const hq_dims* dims, const hq_cache* cache, int32_t t, const uint16_t* k_new,
                   const uint16_t* v_new, const uint8_t* evict_is_vl_or_null, const uint16_t* q,
                   uint16_t* out, float* lse_or_null, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hq_decode_step_ragged -- hq_decode_step with each sequence at its own
 * position: t_seq [B] int32 device array (clamped to [0, t_max]), t_max a
 * host bound on every entry (capacity check, split plan, workspace as for
 * hq_decode_attn at t_max).  Same passages, arguments and errors otherwise.
 */
int hq_decode_step_ragged(const hq_dims* dims, const hq_cache* cache, const int32_t* t_seq,
                          int32_t t_max, const uint16_t* k_new, const uint16_t* v_new,
                          const uint8_t* evict_is_vl_or_null, const uint16_t* q, uint16_t* out,
                          float* lse_or_null, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hq_quant_int8 -- symmetric INT8 of 128-element fp16 rows, the low-bit
 * operand of the prefill's QK product (agihunt digest on HyQuant, method
 * paragraph, prefill sentences; HyQuant README, Overview item 2, and the ops
 * listing's INT8-QK + FP16-PV prefill attention).
 *
 *   x       [rows][128] fp16
 *   codes   [rows][128] int8 out: round-half-even(127 x / amax) of the row
 *           (the decision is exact); all 0 when amax = 0
 *   scales  [rows] fp32 out: fp32(amax / 127), 0 for an all-zero row
 * rows may be 0 (nothing happens).  Errors: HQ_ERR_ARG (negative rows, null
 * pointers), HQ_ERR_ALIGN.
 */
int hq_quant_int8(const uint16_t* x, int64_t rows, int8_t* codes, float* scales, hipStream_t stream);

/*
 * hq_prefill_attn -- causal prefill attention of the whole prefix in one
 * online softmax with hybrid-precision logits (same passages as above).
 *
 *   q            [B][Hq][L][d] fp16 queries of positions 0..L-1
 *   k, v         [B][Hkv][L][d] fp16 keys and values
 *   vl_flag_or_null [B][Hkv][L] u8: nonzero marks a vertical-line key
 *                position (e.g. hq_select_vertical's vl_flag); null: none
 *   out          [B][Hq][L][d] fp16 out
 *   lse_or_null  [B][Hq][L] fp32 out: natural-log log-sum-exp of each
 *                query's logits (hq_select_vertical accepts the last nb rows
 *                of a unit's heads as its lse)
 *   ws           hq_workspace_bytes(dims, HQ_OP_PREFILL, L) bytes (INT8
 *                codes and scales of q and k, the vertical-line lists)
 * Query p (query head h, KV head h / G) attends to keys 0..p.  The logit of
 * key i is tau q.k in FP16 when i is a vertical line or p - i < W (the
 * query's own window, itself included), else tau (q8 . k8) s_q s_k with the
 * hq_quant_int8 codes and scales of the two rows; tau = 1/sqrt(d).  P V uses
 * the FP16 values of every key.  dims->rho, cap_* and the bit widths are not
 * used.  L = 0 does nothing; L is at most 65535 blocks of 32 (G a multiple
 * of 4), 64 (G even) or 128 positions (HQ_ERR_UNSUPPORTED beyond).
 * Errors: HQ_ERR_ARG, HQ_ERR_UNSUPPORTED (d, L),
 * HQ_ERR_ALIGN, HQ_ERR_WORKSPACE, HQ_ERR_HIP.
 */
int hq_prefill_attn(const hq_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    int32_t L, const uint8_t* vl_flag_or_null, uint16_t* out, float* lse_or_null,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Size of the vertical-line set of n_nw candidate (non-window) positions:
 * floor(rho * n_nw + 1e-6), 0 when n_nw <= 0 (agihunt digest, method
 * paragraph: the top-rho of the non-window prefix; the 1e-6 absorbs the
 * binary representation of rho, e.g. 0.29 * 100).  The count every entry
 * point uses; rho outside [0, 1] or NaN gives 0. */
int32_t hq_n_vertical(double rho, int32_t n_nw);

/* Workspace bytes an operation needs for any prefix length up to L_max;
 * 0 for an invalid request. */
size_t hq_workspace_bytes(const hq_dims* dims, int op, int32_t L_max);

/* Static description of a status code. */
const char* hq_status_string(int status);

/* Library ABI version (incremented on any change of this header). */
int hq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HQ_H */
