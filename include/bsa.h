/*
 * bsa.h -- C ABI of the MI355X (gfx950) sparse decode-attention library.
 *
 * One decode step per layer, per unit = one (sequence b, KV head h):
 *
 *   score_scan   score every cached key from a 4-bit copy (block mode) or a
 *                rank-r projected copy (token mode)
 *   select_topk  choose the budget per KV head: top blocks of 128 tokens (plus
 *                the forced BF16 tail pages) or top tokens
 *   sparse_decode_attn
 *                softmax(sigma q K^T) V over the chosen rows only, read in
 *                place from the FP16 cache, FP32 accumulation, split into
 *                num_splits partials per query head
 *   combine      log-sum-exp merge of the partials
 *
 * and, off the timed path, pack_kv_cache builds the 4-bit key copy or the
 * projected-key copy.
 *
 * Sources: "Jet-QSparse: Accelerating Agentic LLM Inference with 4-Bit Sparse
 * Attention", abstract -- NVFP4 key cache, a dense scan over the whole history,
 * selection of 128-token blocks with a budget per KV head, FP16 products summed
 * in FP32 over the chosen values, calibrated key centering, up to two newest
 * pages per sequence kept in BF16; "Joint Subspace Sparse Attention for
 * Efficient Long-Context Decoding" (JSSA), Abstract and Figure 1 -- the group's
 * mean query scores a projected-key cache,
 * one top-B token set per KV head shared by its query heads, attention that
 * reads the selected rows of the standard GQA cache without gathering them.
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers are device memory of the current HIP
 *     device; the caller owns every buffer; the library allocates nothing,
 *     frees nothing and keeps no state between calls (apart from the scratch
 *     that bsa_decode_step_noalloc keeps on each GPU, described there).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns without waiting for it. Inputs must stay valid and outputs
 *     unread until the stream reaches the work.
 *   - Same inputs give the same output bits (no float atomics; fixed orders).
 *   - Return value: BSA_OK, or a negative code with a message readable from
 *     bsa_last_error() on the calling thread. Argument checks happen before
 *     anything is enqueued; nothing is enqueued when a check fails.
 *   - Contents of device buffers are not validated (the library cannot read
 *     them without synchronizing): seq_lens must lie in [0, max_tokens],
 *     global_scale must be finite and > 0, idx entries must be -1 or valid.
 *     Out-of-range seq_lens are clamped to [0, max_tokens]; idx entries outside
 *     the valid range are skipped; no such input makes a kernel read or write
 *     outside the buffers described here.
 */
#ifndef BSA_H_
#define BSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = -1, /* null pointer, inconsistent sizes or strides */
  BSA_ERR_UNSUPPORTED = -2, /* head_dim or block_size other than 128, group > 16, ... */
  BSA_ERR_HIP = -3,         /* a HIP launch failed (message names the HIP error) */
  BSA_ERR_WORKSPACE = -4    /* workspace missing or smaller than bsa_workspace_size() */
};

enum { BSA_DTYPE_F16 = 0, BSA_DTYPE_BF16 = 1 };
/* BLOCK: 128-token blocks of a 4-bit key copy (Jet-QSparse); TOKEN: tokens
 * of a projected-key copy (JSSA); CLUSTER: coarse semantic blocks of
 * noncontiguous tokens, picked by their centroids (Coarse Semantic Blocks
 * abstract; the calls at the end of this header). */
enum { BSA_GRANULARITY_BLOCK = 0, BSA_GRANULARITY_TOKEN = 1, BSA_GRANULARITY_CLUSTER = 2 };

/* Storage of the projected-key cache (TOKEN mode; JSSA Figure 10 evaluates
 * both): BF16, or FP8 as OCP E4M3FN bytes. */
enum { BSA_PROJ_BF16 = 0, BSA_PROJ_FP8 = 1 };

/* The query the block scan scores with (Jet-QSparse abstract: the scan's
 * query-key products run natively in FP4). F16: the step's query as given.
 * NVFP4: each query head quantized as a key is packed (no centering; per-head
 * FP32 scale s_q = amax / 2688, one E4M3 scale per 16 channels, E2M1 elements,
 * each step one correctly rounded float32 operation; a head of zeros stays
 * zero), and the dequantized query qtilde replaces q in both terms of the
 * score. The attention always uses the FP16 query. */
enum { BSA_QUERY_F16 = 0, BSA_QUERY_NVFP4 = 1 };

/* Where the attention reads the values (Jet-QSparse abstract: an NVFP4
 * persistent cache, whose capacity gain needs 4-bit values as well as keys).
 * CACHE: v is the standard cache below, in kv_dtype. NVFP4: v is a 4-bit value
 * store (layout further below) in every entry point that reads or writes V,
 * and the attention aggregates its dequantized values. */
enum { BSA_VALUE_CACHE = 0, BSA_VALUE_NVFP4 = 1 };

/* Standard GQA KV cache: K and V are [batch][num_kv_heads][max_tokens][head_dim]
 * through the strides below (in elements, head_dim contiguous). Query head hq
 * belongs to KV head hq / (num_q_heads / num_kv_heads). */
typedef struct bsa_kv_layout {
  int32_t batch;        /* B >= 1 */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t num_q_heads;  /* Hq, a multiple of Hkv; group G = Hq/Hkv in 1..16 */
  int32_t head_dim;     /* must be 128 */
  int32_t block_size;   /* must be 128 */
  int32_t max_tokens;   /* Tmax: capacity per unit, a multiple of 128 */
  int64_t kv_stride_b;  /* elements between sequences */
  int64_t kv_stride_h;  /* elements between KV heads */
  int64_t kv_stride_t;  /* elements between tokens, >= head_dim, multiple of 8 */
  int32_t kv_dtype;     /* BSA_DTYPE_F16 or BSA_DTYPE_BF16 (K and V alike) */
  int32_t value_dtype;  /* BSA_VALUE_CACHE (V in this layout) or BSA_VALUE_NVFP4 */
} bsa_kv_layout;

/* Selection rule of the step. */
typedef struct bsa_select_cfg {
  int32_t granularity;  /* BSA_GRANULARITY_BLOCK or BSA_GRANULARITY_TOKEN */
  int32_t budget;       /* per unit: blocks (forced tail pages included) or tokens (TOKEN,
                           CLUSTER: the token budget the chosen blocks fit in) */
  int32_t n_tail_pages; /* BLOCK: 0..2 newest pages kept in a BF16 store and always
                           selected (Jet-QSparse abstract); TOKEN: must be 0 */
  int32_t proj_rank;    /* TOKEN: r in {8, 16, 32, 64, 128} (16 .. 128 for FP8); BLOCK: ignored */
  float softmax_scale;  /* sigma, > 0 (1/sqrt(128) for the standard scale) */
  int32_t proj_dtype;   /* TOKEN: BSA_PROJ_BF16 or BSA_PROJ_FP8; BLOCK: must be BSA_PROJ_BF16 (0) */
  int32_t query_dtype;  /* BLOCK: BSA_QUERY_F16 or BSA_QUERY_NVFP4; TOKEN: must be BSA_QUERY_F16 (0) */
  float top_p;          /* TOKEN: 0 keeps the fixed budget; in (0, 1] the budget adapts (top-p
                           retrieval, RaBitQCache abstract): of the budget best tokens, the
                           fewest top-ranked ones whose softmax shares of the unit's scores
                           (over all t < L_b) reach top_p are kept; NaN and -inf weigh
                           nothing, +inf scores share the whole mass, and with no weight at
                           all the budget stays. Needs budget <= 4096. BLOCK: must be 0. */
  int32_t num_clusters; /* CLUSTER: C, coarse blocks per unit, 1..4096; else ignored */
} bsa_select_cfg;

/* ---------------------------------------------------------------------------
 * Layout of the 4-bit key copy (BLOCK mode)
 *
 * codes  : uint8 [B][Hkv][max_tokens/128][8192]
 * scales : uint8 [B][Hkv][max_tokens/128][1024]
 * For token tau = 16 i + n (i < 8, n < 16) of a block and channel d = 32 j + e
 * (j < 4, e < 32), scale group g = d / 16 = 2 j + s (s < 2):
 *   E2M1 code of (tau, d)   at byte ((i*4 + j)*16 + n)*16 + e/2 of the code
 *                           record, low nibble for even e, high nibble for odd e
 *   E4M3 scale of (tau, g)  at byte ((j*16 + n)*8 + i)*2 + s of the scale record
 * The order lets one 64-lane wave load 16 tokens x 128 channels with one
 * contiguous 16-byte load per lane, already in the matrix-core operand order.
 *
 * Number format (NVFP4, named by the Jet-QSparse abstract): E2M1 elements,
 * one E4M3 (OCP E4M3FN) scale per 16 channels, one FP32 scale s_t per KV head.
 * Packing of key row k with centering vector c:
 *   y   = fl32(fl32(k) - c[h])
 *   sb  = E4M3_rne_sat( fl32( max|y over the group| / fl32(6 * s_t[h]) ) )
 *   S   = fl32(E4M3(sb) * s_t[h])
 *   code= S > 0 ? E2M1_rne_sat(fl32(y / S)) : 0     (sign copied from y)
 * The dequantized key is s_t[h] * E2M1(code) * E4M3(sb) + c[h].
 * ------------------------------------------------------------------------- */

/* ---------------------------------------------------------------------------
 * Layout of the 4-bit value store (value_dtype = BSA_VALUE_NVFP4)
 *
 * One device buffer of bsa_value_store_size() bytes, 16-byte aligned; with
 * R = B * Hkv * max_tokens rows, row (b, h, t) = (b * Hkv + h) * max_tokens + t:
 *   codes  uint8 [R][64] at byte 0: E2M1 code of channel d at byte d/2 of the
 *          row, low nibble for even d
 *   scales uint8 [R][8] at byte 64 R: E4M3 scale of channels 16 g .. 16 g + 15
 *          at byte g of the row
 *   s_v    float [Hkv] at byte 72 R: the FP32 scale of each KV head
 * A value row v is packed as a key row is, with no centering and s_v in place
 * of s_t: sb = E4M3_rne_sat(fl32(max|v over the group| / fl32(6 * s_v))),
 * S = fl32(E4M3(sb) * s_v), code = S > 0 ? E2M1_rne_sat(fl32(v / S)) : 0. The
 * attention reads the value E2M1(code) * S (= s_v * E2M1 * E4M3 up to one
 * float32 rounding of S). The tail store of BLOCK mode stays BF16.
 * ------------------------------------------------------------------------- */

/* Bytes of the value store: 72 * B * Hkv * max_tokens + 4 * Hkv (0 for a bad
 * layout). */
size_t bsa_value_store_size(const bsa_kv_layout* layout);

/* Pack values into the store for tokens [128*block_begin, 128*block_end) of
 * every unit, and set the store's s_v from value_scale (device float [Hkv],
 * finite > 0; the caller's calibration, e.g. the largest |v| of the KV head
 * over 2688 = 6 * 448, so that no group scale saturates).
 * v: device, kv_dtype, the K/V layout's strides (the full-precision values;
 * value_dtype is not read). store: bsa_value_store_size() bytes. Requires
 * 0 <= block_begin <= block_end <= max_tokens/128; an empty range only sets
 * s_v. */
int bsa_pack_values(const bsa_kv_layout* layout, const void* v, const float* value_scale,
                    int32_t block_begin, int32_t block_end, void* store, void* stream);

/* Build the key copy for blocks [block_begin, block_end) of every unit.
 *
 * BLOCK: k (device, kv_dtype, layout above), key_center (device float
 *   [Hkv][128], or NULL for no centering), global_scale (device float [Hkv],
 *   finite > 0) -> codes, scales (device, layout above). proj and kproj unused.
 * TOKEN: k and proj (device float [Hkv][128][r]) -> kproj [B][Hkv][max_tokens][r]
 *   for tokens [128*block_begin, 128*block_end), from acc, the float32 sum over
 *   d = 0..127 in ascending order of fl32(P[h][d][j] * k[t][d]), each addition
 *   rounded to float32 (JSSA Figure 1: projected-key cache; Figure 10: BF16 or
 *   FP8 storage):
 *     BSA_PROJ_BF16: uint16 bfloat16 bits, kproj[t][j] = BF16_rne(acc);
 *     BSA_PROJ_FP8:  uint8 E4M3FN codes, kproj[t][j] = nearest E4M3FN value
 *                    to acc (ties to the even code, saturating at 448, sign
 *                    bit copied from acc; no further scale).
 * Packing all tokens of the blocks regardless of sequence length is the
 * caller's choice: blocks past a sequence's end are never read by the scan.
 * Requires 0 <= block_begin <= block_end <= max_tokens/128. */
int bsa_pack_kv_cache(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                      const void* k, const float* key_center, const float* global_scale,
                      const float* proj, int32_t block_begin, int32_t block_end,
                      uint8_t* codes, uint8_t* scales, void* kproj, void* stream);

/* Append one decode step's token to every sequence's cache (the cache
 * lifecycle of the Jet-QSparse abstract: the newest pages kept in BF16, the key
 * copy packed straight from the full-precision keys; JSSA Figure 1: projected
 * keys of new tokens).
 *
 * For each sequence b with length L_b = seq_lens[b] before the append
 * (0 <= L_b < max_tokens; other sequences are left unchanged) and KV head h,
 * with k_new, v_new device [B][Hkv][128] in kv_dtype (16-byte aligned):
 *   k[b][h][L_b] = k_new[b][h], v[b][h][L_b] = v_new[b][h] (with a 4-bit value
 *     store: v_new[b][h] packed into its row (b, h, L_b), as bsa_pack_values
 *     packs it, with the store's s_v);
 *   BLOCK: the token's E2M1 codes and E4M3 scales in codes, scales, exactly as
 *     bsa_pack_kv_cache packs that token (a token's records depend on its own
 *     row only), from key_center (or NULL) and global_scale;
 *   BLOCK with n_tail_pages > 0: the BF16 tail store (tail_k, tail_v, layout
 *     as in bsa_sparse_decode_attn: slot s holds page ceil(L/128) -
 *     n_tail_pages + s) is kept in step: a token that starts a new page
 *     (L_b % 128 == 0) shifts the slots down by one and clears the last slot;
 *     then the last slot's row L_b % 128 takes the BF16 (round to nearest
 *     even) of the new key and value;
 *   TOKEN: kproj[b][h][L_b] = the projected key of k_new, exactly as
 *     bsa_pack_kv_cache forms it (proj required).
 * seq_lens is read, not written: the caller advances it after the call. */
int bsa_append_token(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* k_new,
                     const void* v_new, const int32_t* seq_lens, void* k, void* v,
                     const float* key_center, const float* global_scale, const float* proj,
                     uint8_t* codes, uint8_t* scales, void* kproj, uint16_t* tail_k,
                     uint16_t* tail_v, void* stream);

/* Score the cache for one decode step.
 *
 * q: device fp16 [B][Hq][128] contiguous. seq_lens: device int32 [B].
 * BLOCK (Jet-QSparse abstract: dense scan of the whole history, 128-token
 *   blocks): for block n < P_b = ceil(L_b/128) - n_tail_pages,
 *     scores[b][h][n] = max over query heads hq of KV head h and tokens t of
 *       block n with t < L_b of  sigma * (s_t[h] * q_hq . (E2M1 * E4M3)(t)
 *                                           + q_hq . c[h])
 *   (the centering vector is added back so the estimate targets q . k;
 *   key_center NULL means c = 0); every other block scores -inf. With
 *   query_dtype = BSA_QUERY_NVFP4, q_hq is replaced in both terms by its NVFP4
 *   form qtilde_hq (defined at BSA_QUERY_NVFP4).
 *   codes, scales, global_scale required; kproj, proj unused.
 * TOKEN (JSSA Figure 1): qbar = mean of the group's query heads,
 *   p = P[h]^T qbar, scores[b][h][t] = sigma * p . kproj[b][h][t] for t < L_b,
 *   -inf beyond. kproj, proj required; codes, scales, global_scale unused.
 * scores: device float [B][Hkv][max_tokens/128] (BLOCK) or [B][Hkv][max_tokens]
 * (TOKEN, 16-byte aligned); every entry is written. */
int bsa_score_scan(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* q,
                   const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                   const float* key_center, const void* kproj, const float* proj,
                   const int32_t* seq_lens, float* scores, void* stream);

/* Bytes of device workspace bsa_select_topk needs for this layout and cfg
 * (0 for BLOCK granularity). */
size_t bsa_workspace_size(const bsa_kv_layout* layout, const bsa_select_cfg* cfg);

/* Choose the budget per unit (Jet-QSparse abstract: top blocks per KV head;
 * JSSA Figure 1 and Table 15: top-B tokens per KV head, shared by its query heads).
 *
 * BLOCK: candidates are blocks n < P_b (see score_scan); the
 *   (budget - n_tail_pages) highest-scoring candidates are taken, plus the
 *   forced pages max(0, N_b - n_tail_pages) .. N_b - 1, N_b = ceil(L_b/128).
 * TOKEN: candidates are tokens t < L_b; the budget highest-scoring are taken.
 * Equal scores go to the lower index; NaN ranks below every number; -0 == +0.
 * idx: device int32 [B][Hkv][budget], ascending, padded with -1.
 * count: device int32 [B][Hkv], the number of valid idx entries.
 * workspace: device memory of at least bsa_workspace_size() bytes (may be NULL
 * when that is 0). TOKEN: zero-fill it before its first use; every call that
 * completes leaves the parts that must start at zero (histograms, arrival
 * counters) zeroed again, so it is reused as is; calls that share it must not
 * run concurrently. Its size depends on the cfg: with budget <= 2048 and
 * max_tokens <= 131072 (a multiple of 4) the selection runs in one launch
 * and also needs room for per-unit candidate lists. */
int bsa_select_topk(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                    const float* scores, const int32_t* seq_lens, void* workspace,
                    size_t workspace_bytes, int32_t* idx, int32_t* count, void* stream);

/* Sparse attention over the selected rows, as split partials (Jet-QSparse
 * abstract: FP16 aggregation with FP32 accumulation over contiguous block
 * tiles; JSSA Figure 1: gather-free reads of the selected rows).
 *
 * For query head hq of KV head h and split s, with n = count (clamped to
 * [0, budget]) and per = ceil(n/S), the rows are those of idx entries
 * [s*per, min((s+1)*per, n)) (entries that are -1 are skipped):
 *   BLOCK: the tokens t of each selected block with t < L_b; a block that is one
 *     of the n_tail_pages newest pages (n >= N_b - n_tail_pages) is read from
 *     the BF16 tail store, slot n - (N_b - n_tail_pages), else from k, v.
 *   TOKEN: the tokens idx[...] (those >= L_b are skipped).
 *   part_o[b][hq][s][:]  = sum_t softmax_t(sigma q . k_t) v_t over the split's rows
 *   part_lse[b][hq][s]   = log sum_t exp(sigma q . k_t)
 *   (an empty split writes 0 and -inf).
 * q: device fp16 [B][Hq][128]. k, v: device, kv_dtype, the layout above (v:
 * the 4-bit value store when value_dtype = BSA_VALUE_NVFP4; its rows are then
 * the dequantized values, the tail store's stay BF16).
 * tail_k, tail_v: device bfloat16 bits [B][Hkv][n_tail_pages][128][128], or
 * NULL when n_tail_pages is 0. idx, count: as written by bsa_select_topk (the
 * selection's entries first, then -1 padding); the splits share the count's
 * entries evenly.
 * part_o: device float [B][Hq][S][128]; part_lse: device float [B][Hq][S];
 * 1 <= num_splits <= budget. */
int bsa_sparse_decode_attn(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                           const void* q, const void* k, const void* v,
                           const int32_t* seq_lens, const int32_t* idx, const int32_t* count,
                           const uint16_t* tail_k, const uint16_t* tail_v, int32_t num_splits,
                           float* part_o, float* part_lse, void* stream);

/* Log-sum-exp merge of split partials (the pages aggregate each KV head's
 * chosen rows into one softmax-weighted sum with FP32 accumulation,
 * Jet-QSparse abstract; JSSA Figure 1: one attention over the selected rows
 * per query head; split into S parts for parallelism, that sum is recovered
 * exactly by this identity, the reading this library uses), per row r (a
 * (sequence, query head)):
 *   lse[r] = log sum_s exp(part_lse[r][s]),
 *   out[r] = sum_s exp(part_lse[r][s] - lse[r]) * part_o[r][s][:];
 * rows whose splits are all empty get out = 0 and lse = -inf.
 * part_o: device float [rows][num_splits][head_dim]; part_lse: device float
 * [rows][num_splits]; out: device float [rows][head_dim]; out_lse: device
 * float [rows] (may be NULL). head_dim must be 128. */
int bsa_combine(int32_t rows, int32_t num_splits, int32_t head_dim, const float* part_o,
                const float* part_lse, float* out, float* out_lse, void* stream);

/* ---------------------------------------------------------------------------
 * Combined forms of the step (same results, fewer calls)
 *
 * bsa_score_select = bsa_score_scan followed by bsa_select_topk, and
 * bsa_attend_combine = bsa_sparse_decode_attn followed by bsa_combine over the
 * num_splits partials of each (sequence, query head), with identical outputs.
 * With at most 8 splits bsa_attend_combine merges in the last attention
 * work-group of each unit to finish, so the merge hides behind other units'
 * attention (with more it launches the merge separately). That group is found
 * with one arrival counter per unit in `counters` (device, bsa_counters_size
 * bytes): it must be zero-filled before its first use, every call that
 * completes leaves it zero, and calls that share it must not run
 * concurrently. No work-group ever waits for another.
 * ------------------------------------------------------------------------- */

/* Bytes of the counters: 4 * batch * num_kv_heads (0 for a bad layout). */
size_t bsa_counters_size(const bsa_kv_layout* layout);

/* bsa_score_scan then bsa_select_topk; arguments as there. In token mode the
 * scan also counts the selection's first radix digits into the workspace as it
 * stores the scores, so the selection skips its own pass over them. */
int bsa_score_select(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* q,
                     const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                     const float* key_center, const void* kproj, const float* proj,
                     const int32_t* seq_lens, float* scores, void* workspace,
                     size_t workspace_bytes, int32_t* idx, int32_t* count, void* stream);

/* bsa_sparse_decode_attn then bsa_combine: part_o / part_lse are filled as by
 * bsa_sparse_decode_attn, out [B][Hq][128] and out_lse [B][Hq] (may be NULL) as
 * by bsa_combine. */
int bsa_attend_combine(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* q,
                       const void* k, const void* v, const int32_t* seq_lens,
                       const int32_t* idx, const int32_t* count, const uint16_t* tail_k,
                       const uint16_t* tail_v, int32_t num_splits, float* part_o,
                       float* part_lse, uint32_t* counters, float* out, float* out_lse,
                       void* stream);

/* bsa_select_topk then bsa_attend_combine, with identical outputs: idx and count
 * as written by bsa_select_topk, part_o / part_lse / out / out_lse as by
 * bsa_attend_combine. In block mode with budget <= 1024 a single attention
 * launch does both: every work-group of a unit makes the unit's selection in
 * its prologue (Jet-QSparse abstract: selection by score, then sparse
 * aggregation), and the split-0 group writes idx and count. Otherwise (token
 * mode, larger budgets) it runs the two calls; workspace is bsa_select_topk's. */
int bsa_select_attend_combine(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                              const void* q, const void* k, const void* v,
                              const int32_t* seq_lens, const float* scores, void* workspace,
                              size_t workspace_bytes, const uint16_t* tail_k,
                              const uint16_t* tail_v, int32_t num_splits, int32_t* idx,
                              int32_t* count, float* part_o, float* part_lse,
                              uint32_t* counters, float* out, float* out_lse, void* stream);

/* One whole decode step: bsa_score_scan, bsa_select_topk and
 * bsa_attend_combine, with identical outputs (scores, idx, count, part_o,
 * part_lse, out, out_lse); arguments as there, the block-mode key copy (codes,
 * scales, global_scale, key_center) or the token-mode one (kproj, proj) as the
 * granularity needs. counters: bsa_counters_size bytes, zero-filled before the
 * first use.
 *
 * In block mode with budget <= 1024 this is two launches (Jet-QSparse
 * abstract: a dense scan of the 4-bit keys, then a per-KV-head block selection
 * and sparse aggregation of the chosen blocks): the scan, then the attention
 * launch with the selection in its prologue, as bsa_select_attend_combine.
 * Otherwise (token mode, larger budgets) it runs the scan, the selection and
 * the attention in turn; workspace is bsa_select_topk's (unused in block
 * mode). Calls sharing counters or a workspace must not run concurrently. */
int bsa_decode_step(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* q,
                    const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                    const float* key_center, const void* kproj, const float* proj,
                    const void* k, const void* v, const int32_t* seq_lens,
                    const uint16_t* tail_k, const uint16_t* tail_v, int32_t num_splits,
                    float* scores, void* workspace, size_t workspace_bytes, int32_t* idx,
                    int32_t* count, float* part_o, float* part_lse, uint32_t* counters,
                    float* out, float* out_lse, void* stream);

/* bsa_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Inputs and out / out_lse as in bsa_decode_step; the intermediates that call
 * takes from the caller (scores, idx, count, part_o, part_lse, the arrival
 * counters and the token selection's workspace) live instead in a scratch
 * array of 64 MiB that the library holds on each GPU it runs on until the
 * process ends. No call allocates or frees memory.
 *
 * The scratch of the current HIP device is used (its address is looked up on
 * the first call on that device; stream must belong to it). A step whose
 * intermediates exceed 64 MiB returns BSA_ERR_WORKSPACE with the size needed
 * (token mode at 128K context reaches that near 128 units of 128K tokens).
 * Each call first clears the counters and the workspace in the scratch, so no
 * set-up is needed, but all calls on one GPU share the one scratch: calls that
 * overlap on one GPU (other streams, other host threads) race and must not be
 * made. The intermediates are not readable by the caller. */
int bsa_decode_step_noalloc(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                            const void* q, const uint8_t* codes, const uint8_t* scales,
                            const float* global_scale, const float* key_center,
                            const void* kproj, const float* proj, const void* k, const void* v,
                            const int32_t* seq_lens, const uint16_t* tail_k,
                            const uint16_t* tail_v, int32_t num_splits, float* out,
                            float* out_lse, void* stream);

/* ---------------------------------------------------------------------------
 * Coarse semantic blocks (granularity BSA_GRANULARITY_CLUSTER)
 *
 * Coarse Semantic Blocks abstract: the keys are clustered into large blocks
 * of noncontiguous tokens; a query picks blocks by scoring their centroids
 * and attends the original keys and values of the picked blocks. The
 * clustering itself is the caller's (the abstract names no method): the index
 * is built from a token -> block assignment. Index of one unit:
 *   centroids float [B][Hkv][C][128]: block c's centroid, the mean of its
 *             tokens' keys (FP32 sum over the tokens in ascending order, then
 *             one division); zero for a block with no token;
 *   offsets   int32 [B][Hkv][C + 1]: block c's tokens are
 *             members[offsets[c] .. offsets[c + 1]);
 *   members   int32 [B][Hkv][max_tokens]: the tokens, block after block,
 *             ascending within a block (the first offsets[C] entries).
 * The step, per unit (reading of the abstract: the KV head's query heads pick
 * one block set together, as in the other modes):
 *   score_c = max over the group's query heads hq of sigma * q_hq . centroid_c
 *             (-inf for a block with no token);
 *   the blocks ranked by score (descending, the lower block id first among
 *   equal scores, NaN last); the chosen blocks are the longest prefix of the
 *   ranking whose sizes add up to at most the token budget (whole blocks);
 *   idx = their tokens, block after block in ranking order, ascending within a
 *   block, padded with -1 to budget; count = their number.
 * The attention then reads those tokens in place, as in token mode:
 * bsa_sparse_decode_attn and bsa_attend_combine accept CLUSTER with this idx
 * and count. The other calls reject CLUSTER (BSA_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------- */

/* Build the index from assign (device int32 [B][Hkv][max_tokens]: the block
 * of each token, -1 or any value outside [0, C) for none; tokens t >= L_b are
 * not indexed) and the keys k (kv_dtype, the layout above). Off the decode
 * step. centroids, offsets, members: as above (device, 16-byte aligned). */
int bsa_build_cluster_index(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                            const void* k, const int32_t* assign, const int32_t* seq_lens,
                            float* centroids, int32_t* offsets, int32_t* members, void* stream);

/* The centroids' scores: scores device float [B][Hkv][C]. q: device fp16
 * [B][Hq][128]. */
int bsa_score_clusters(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* q,
                       const float* centroids, const int32_t* offsets, float* scores,
                       void* stream);

/* The choice from given scores: idx device int32 [B][Hkv][budget], count
 * device int32 [B][Hkv]. */
int bsa_select_clusters(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                        const float* scores, const int32_t* offsets, const int32_t* members,
                        int32_t* idx, int32_t* count, void* stream);

/* bsa_score_clusters then bsa_select_clusters, in one call. */
int bsa_score_select_clusters(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                              const void* q, const float* centroids, const int32_t* offsets,
                              const int32_t* members, float* scores, int32_t* idx,
                              int32_t* count, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* bsa_last_error(void);

/* Library version string. */
const char* bsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H_ */
