/*
 * kvq.h -- C ABI of libkvq, the MI355X (gfx950) KV-cache quantization library.
 *
 * Three schemes, each a quantize -> bit-pack -> unpack -> dequantize path over
 * fp16 key/value tensors already resident in device memory:
 *   - symmetric per-(token, head) q8 / q6 / q4 on paged storage
 *     [MTPLX pull request #267, "feat(kv-cache): add q6 paged KV quantization",
 *      PR description];
 *   - KIVI asymmetric min/max group round trip
 *     ["veloxquant_mlx.cache.kivi_cache" module source, KIVIKVCache];
 *   - KVQuant-style non-uniform quantization with dense-and-sparse outliers and
 *     attention-sink tokens ["veloxquant_mlx.cache.kvquant_cache module"].
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE memory owned by the caller unless marked [host]. The
 *     library allocates no device memory and keeps no device data between
 *     calls; its only device objects are the auxiliary stream and two events
 *     that kvq_nuq_fit_quant creates once per device (see there).
 *   - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream. Work
 *     is enqueued on it; no entry point synchronises.
 *   - All validation happens on the host before any HIP call: a bad argument
 *     returns a kvq_status != KVQ_OK and enqueues nothing. Device-side data
 *     that the host cannot see (slot mappings, block tables, sequence lengths)
 *     is range-checked inside the kernels: out-of-range entries are skipped as
 *     documented per call, never dereferenced.
 *   - kvq_last_error() returns a thread-local description of the last failure.
 *   - There is no fallback path: if the GPU code cannot run, the call fails
 *     with KVQ_ERR_HIP.
 *   - Base pointers of fp16 and code buffers must be 16-byte aligned
 *     (KVQ_ERR_ALIGN otherwise); fp32/int32 buffers 4-byte aligned.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_NULL = 1,     /* a required pointer is NULL */
  KVQ_ERR_BITS = 2,     /* bit width not in the scheme's table */
  KVQ_ERR_SHAPE = 3,    /* sizes inconsistent or out of range */
  KVQ_ERR_ALIGN = 4,    /* pointer not aligned as required */
  KVQ_ERR_CAPACITY = 5, /* an output or workspace is too small */
  KVQ_ERR_HIP = 6,      /* the HIP runtime reported an error (text in kvq_last_error) */
  KVQ_ERR_MODE = 7,     /* unknown or rejected mode string */
  KVQ_ERR_ARG = 8       /* other invalid scalar argument */
} kvq_status;

/* [host] Thread-local text of the most recent failure on this thread ("" if none). */
const char *kvq_last_error(void);

/* [host] Library version string. */
const char *kvq_version(void);

/* ------------------------------------------------------------------ symmetric
 * [MTPLX PR #267, PR description] One symmetric quantizer per (token, KV head)
 * row of head_dim values with one fp16 scale. qmax is an explicit table
 * {8: 127, 6: 31, 4: 7}; any other width is rejected, never mapped to a
 * neighbour. q6 codes are biased by +32 into 6-bit fields packed four per
 * three bytes, little-endian, per the page's byte equations; q4 codes are
 * biased by +8, two per byte, even element in the low nibble; q8 codes are
 * int8 two's complement, one per byte.
 *
 * Per row x[0..D): a = max|x_i|; scale = fp16(a / qmax) (binary32 division,
 * round-to-nearest-even); s = float(scale); q_i = 0 when s == 0, else
 * clamp(rint(x_i * (1/s)), -qmax, qmax) with 1/s and the product in binary32
 * and rint ties-to-even. Dequantization: x_i' = fp16(q_i * s).
 */

/* [host] Parse a mode name. Accepts "q8", "q6", "q4", "8", "6", "4", and the
 * q6 aliases "6bit", "int6", "uint6"; case-sensitive. Rejects everything
 * else, including "q6_k" and "q6_0" (a different format), with KVQ_ERR_MODE.
 * *bits receives 8, 6 or 4.
 * [MTPLX PR #267, PR description: q6 aliases kept narrow, q6_k/q6_0 rejected] */
int kvq_parse_mode(const char *mode, int32_t *bits);

/* [host] qmax for a width: 127, 31, 7; -1 for any other width. */
int32_t kvq_sym_qmax(int32_t bits);

/* [host] Bytes of packed codes per row: D*bits/8. -1 if bits is not 8/6/4,
 * D <= 0, q6 with D % 4 != 0, or q4 with odd D. [MTPLX PR #267: packed_dim] */
int64_t kvq_packed_dim(int32_t head_dim, int32_t bits);

/* [host] Bytes of a K+V cache of `tokens` tokens: 2 * tokens * layers *
 * kv_heads * (packed_dim + 2) (codes + one fp16 scale per row); bits == 16
 * gives the unquantised fp16 size. -1 on invalid widths/shapes.
 * [MTPLX PR #267, PR description: storage arithmetic] */
int64_t kvq_sym_cache_bytes(int64_t tokens, int32_t layers, int32_t kv_heads, int32_t head_dim,
                            int32_t bits);

/* Geometry of a paged symmetric pool. One pool holds `layers` layers; each
 * layer has num_pages pages of page_size token slots. Codes of layer l are
 * uint8 [num_pages][page_size][kv_heads][packed_dim] starting at
 * codes + l * num_pages*page_size*kv_heads*packed_dim; scales (fp16) are
 * [num_pages][page_size][kv_heads] per layer. K and V use two pools of the
 * same geometry. */
typedef struct kvq_paged_layout {
  int32_t layers;
  int32_t num_pages;
  int32_t page_size;
  int32_t kv_heads;
  int32_t head_dim;
  int32_t bits; /* 8, 6 or 4 */
} kvq_paged_layout;

/* Quantize and pack tokens into the paged pools (write path).
 *   k, v         fp16 [n_layers][n_tokens][kv_heads][head_dim], contiguous;
 *                layer i of the input goes to pool layer layer0 + i.
 *   slot_mapping int32 [n_tokens]: global slot page*page_size + slot of each
 *                token (same for every layer). A negative entry, or one >=
 *                num_pages*page_size, leaves that token unwritten.
 *   k_codes/k_scales, v_codes/v_scales: the pools (updated in place).
 * Either side may be skipped by passing NULL for its input AND both of its
 * pool pointers. n_tokens == 0 or n_layers == 0 is a no-op.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_BITS, KVQ_ERR_SHAPE (layer range outside the
 * pool, bad geometry), KVQ_ERR_ALIGN, KVQ_ERR_HIP. */
int kvq_quant_sym(const kvq_paged_layout *layout, const uint16_t *k, const uint16_t *v,
                  int32_t layer0, int32_t n_layers, int32_t n_tokens,
                  const int32_t *slot_mapping, uint8_t *k_codes, uint16_t *k_scales,
                  uint8_t *v_codes, uint16_t *v_scales, void *stream);

/* Unpack and dequantize sequences out of the paged pools (read path).
 *   block_table  int32 [n_seqs][max_blocks]: page id of each block of each sequence.
 *   seq_lens     int32 [n_seqs]: tokens held by each sequence.
 *   k_out, v_out fp16 [n_layers][n_seqs][max_len][kv_heads][head_dim].
 * Position p of sequence s reads page block_table[s][p / page_size], slot
 * p % page_size. Rows at p >= seq_lens[s], p >= max_blocks*page_size, or whose
 * page id is outside [0, num_pages), are written as +0.
 * Either side may be skipped by passing NULL for its pool pointers AND output.
 * Errors: as kvq_quant_sym. */
int kvq_dequant_sym(const kvq_paged_layout *layout, const uint8_t *k_codes,
                    const uint16_t *k_scales, const uint8_t *v_codes, const uint16_t *v_scales,
                    int32_t layer0, int32_t n_layers, const int32_t *block_table,
                    int32_t max_blocks, const int32_t *seq_lens, int32_t n_seqs, int32_t max_len,
                    uint16_t *k_out, uint16_t *v_out, void *stream);

/* ------------------------------------------------------------------ decode attention
 * [MTPLX pull request #267, "feat(kv-cache): add q6 paged KV quantization",
 *  PR description: the cached rows are dequantized (code x fp16 scale) and
 *  passed to scaled-dot-product attention] -- here one call reads the packed
 *  codes and scales directly (no fp16 copy of the cache).
 */

/* [host] Bytes of device workspace kvq_attn_decode_sym needs:
 * n_seqs * ceil(max_len / 256) * q_heads * (head_dim + 2) * 4 (one chunk when
 * max_len is 0). -1 on a negative size or non-positive q_heads / head_dim. */
int64_t kvq_attn_workspace_bytes(int32_t n_seqs, int32_t q_heads, int32_t head_dim, int32_t max_len);

/* One decode step of attention for one layer of a paged symmetric pool.
 *   out[s][h][:] = sum_t softmax_t(softmax_scale * q[s][h] . k[s][t]) v[s][t]
 * over positions t < min(seq_lens[s], max_len) of sequence s, where k, v are
 * the rows of KV head h / (q_heads / kv_heads) dequantized exactly as
 * kvq_dequant_sym does; positions p >= max_blocks * page_size and positions
 * whose block-table entry is outside [0, num_pages) are left out of the
 * softmax; a sequence with no position left gives 0.
 * q fp16 [n_seqs][q_heads][head_dim]; out fp16 [n_seqs][q_heads][head_dim];
 * block_table / seq_lens / pools as in kvq_dequant_sym; layer indexes the
 * pool. head_dim 64, 128 or 256; q_heads a multiple of kv_heads with at most
 * 16 query heads per KV head. Scores and the softmax are fp32 (scores from
 * fp16 products accumulated in fp32), the probabilities are rounded to fp16
 * for the weighted sum of V, accumulated in fp32; the result is rounded to
 * fp16 once.
 * workspace: caller-owned device memory of kvq_attn_workspace_bytes bytes,
 * 16-byte aligned, contents irrelevant on entry. All pointers device memory,
 * caller-owned; code pools and q 16-byte aligned. Errors: KVQ_ERR_SHAPE /
 * _NULL / _ALIGN / _CAPACITY / _ARG as for the other calls. Asynchronous on
 * `stream`. */
int kvq_attn_decode_sym(const kvq_paged_layout *layout, const uint8_t *k_codes, const uint16_t *k_scales,
                        const uint8_t *v_codes, const uint16_t *v_scales, int32_t layer, const uint16_t *q,
                        int32_t q_heads, const int32_t *block_table, int32_t max_blocks,
                        const int32_t *seq_lens, int32_t n_seqs, int32_t max_len, float softmax_scale,
                        uint16_t *out, void *workspace, int64_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ KIVI
 * ["veloxquant_mlx.cache.kivi_cache", KIVIKVCache._quant_dequant_along]
 * Asymmetric min/max round trip in binary32: for each group,
 * levels = 2^bits - 1, scale = max((max - min)/levels, eps),
 * code = clamp(rint((x - min)/scale), 0, levels) (IEEE division, ties to
 * even), x' = fp16(code*scale + min) (product then sum, not fused).
 * Keys are grouped per channel along tokens (groups of group_size tokens
 * starting at lo); values per token along channels (groups of group_size
 * channels starting at channel 0). A last group shorter than group_size is
 * its own group (equivalent to the page's edge-replicating pad). */

/* [host] Quantization frontier: max(0, offset - residual_length) rounded down
 * to a multiple of group_size ["kivi_cache", _quantization_boundary].
 * -1 if group_size <= 0 or residual_length < 0 or offset < 0. */
int64_t kvq_kivi_boundary(int64_t offset, int32_t residual_length, int32_t group_size);

/* In-place KIVI round trip of tokens [lo, hi) of keys and values.
 *   keys, values fp16 [B][H][S_cap][D] (batch and layers folded into B);
 *                tokens outside [lo, hi) are not touched. Either may be NULL
 *                to skip that side (its optional outputs must then be NULL).
 *   bits         2, 4 or 8.  group_size >= 1.  eps > 0 (the page uses 1e-8).
 *   Optional outputs (NULL to skip; each side independently):
 *     *_codes    uint8 [B][H][hi-lo][D*bits/8], codes packed LSB-first along D
 *                (requires D*bits % 8 == 0);
 *     k_scale/k_min fp32 [B][H][ceil((hi-lo)/group_size)][D];
 *     v_scale/v_min fp32 [B][H][hi-lo][ceil(D/group_size)].
 *   Codes, scale and min reproduce the written fp16 values exactly.
 * hi == lo is a no-op. Errors: KVQ_ERR_NULL, KVQ_ERR_BITS, KVQ_ERR_SHAPE,
 * KVQ_ERR_ARG (eps), KVQ_ERR_ALIGN, KVQ_ERR_HIP. */
int kvq_kivi_quant_dequant(uint16_t *keys, uint16_t *values, int32_t B, int32_t H, int32_t S_cap,
                           int32_t D, int32_t lo, int32_t hi, int32_t bits, int32_t group_size,
                           float eps, uint8_t *k_codes, float *k_scale, float *k_min,
                           uint8_t *v_codes, float *v_scale, float *v_min, void *stream);

/* Packed KIVI storage ["veloxquant_mlx.cache.kivi_cache", module docstring
 * on per-token storage at bit-width b and group size g, and
 * _quantized_bytes]: b-bit codes plus one fp16 (scale, zero) pair per
 * group, the storage the page's byte accounting charges for. Group math as
 * kvq_kivi_quant_dequant with the pair rounded to fp16 before use:
 * scale = max((max - min)/levels, eps) rounded to fp16 toward zero (so that
 * zero + levels*scale never exceeds the group's max) and raised to 2^-24 if
 * that gives 0 (eps = 1e-8 is below the smallest fp16); zero = min (exact,
 * -0 stored as +0); code = clamp(rint((x - zero)/scale), 0, levels) with the
 * fp16 scale; reconstruction fp16(code*scale + zero), product then sum.
 * Storage is indexed by absolute token so that successive flushes fill it in
 * place (the fp16 side may be a window of the sequence, see x_rows / x_t0
 * and out_rows / out_t0):
 *   codes   uint8 [B][H][S_cap][D*bits/8], LSB-first along D;
 *   keys    groups of group_size tokens from token 0 (lo must be a multiple
 *           of group_size): scale, zero fp16 [B][H][ceil(S_cap/group_size)][D];
 *   values  groups of group_size channels: scale, zero fp16
 *           [B][H][S_cap][ceil(D/group_size)].
 * Requires D % 8 == 0 and group_size a positive multiple of 8; bits 2, 4,
 * 8; all pointers device memory, caller-owned, 16-byte aligned. */

/* Quantize tokens [lo, hi) of keys and/or values into packed storage; the
 * other tokens' storage is not touched. keys / values: fp16
 * [B][H][x_rows][D], not modified, row r holding token x_t0 + r (so a
 * residual window can be packed without copying it into a full-length
 * buffer; x_rows = S_cap, x_t0 = 0 for a full-length buffer); needs
 * 0 <= x_t0 <= lo and hi <= x_t0 + x_rows. keys or values may be NULL to skip
 * that side (its outputs are then unused); a given side needs all three
 * outputs. hi == lo is a no-op.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_BITS, KVQ_ERR_SHAPE, KVQ_ERR_ARG (eps),
 * KVQ_ERR_ALIGN, KVQ_ERR_HIP. Asynchronous on `stream`. */
int kvq_kivi_pack(const uint16_t *keys, const uint16_t *values, int32_t B, int32_t H, int32_t S_cap, int32_t D,
                  int32_t lo, int32_t hi, int32_t bits, int32_t group_size, float eps, uint8_t *k_codes,
                  uint16_t *k_scale, uint16_t *k_zero, uint8_t *v_codes, uint16_t *v_scale, uint16_t *v_zero,
                  int32_t x_rows, int32_t x_t0, void *stream);

/* Reconstruct tokens [lo, hi) from packed storage into k_out / v_out, fp16
 * [B][H][out_rows][D] with token t written to row t - out_t0 (needs
 * 0 <= out_t0 <= lo and hi <= out_t0 + out_rows; other rows not written).
 * Either output may be NULL to skip that side. Errors as kvq_kivi_pack
 * (no eps). Asynchronous on `stream`. */
int kvq_kivi_unpack(const uint8_t *k_codes, const uint16_t *k_scale, const uint16_t *k_zero, const uint8_t *v_codes,
                    const uint16_t *v_scale, const uint16_t *v_zero, int32_t B, int32_t H, int32_t S_cap, int32_t D,
                    int32_t lo, int32_t hi, int32_t bits, int32_t group_size, uint16_t *k_out, uint16_t *v_out,
                    int32_t out_rows, int32_t out_t0, void *stream);

/* ------------------------------------------------------------------ NUQ
 * ["veloxquant_mlx.cache.kvquant_cache module", module docstring] KVQuant-style
 * non-uniform quantization. Keys get one table of L = 2^bits levels per
 * channel (samples: the channel's values over tokens), values one table per
 * token (samples: the token's D channels). Per vector of n samples:
 *   k = floor(frac * n) with frac a binary64 number and one binary64 product
 *   (the page's outlier fraction is a Python float: 1% of 100 samples is 1);
 *   tau = the (k+1)-th largest |x|; samples
 *   with |x| > tau are outliers (at most k), kept exact in a side channel;
 *   the inliers are fit by `lloyd_iters` Lloyd-Max iterations (unweighted
 *   1-D k-means) from linear-interpolated quantiles at probabilities
 *   (j + 1/2)/L; a sample's code is its nearest level (ties to the lower
 *   index); an empty cell keeps its level; a level is the binary32 rounding
 *   of its cell's exact mean (sums are exact: int64 in 2^-24 units for key
 *   fits, double for value fits of at most 256 samples); after each
 *   update the table is sorted ascending (an ordered "signpost" table).
 * Attention sinks: when start_pos == 0 the first n_sink tokens of the call
 * are sinks: exact, code 0, excluded from every fit and threshold, and their
 * value-level rows are 0 (module docstring, "Attention Sink-Aware").
 * Level lifecycle ("Level lifecycle"): fit_keys = 1 fits key levels and
 * |key| thresholds on this call's non-sink tokens and writes them to
 * key_levels / key_thresh (prefill); fit_keys = 0 reads them as given (frozen)
 * and a key is an outlier iff |x| > key_thresh of its channel. Value levels
 * are fit on every call.
 * Outputs: codes packed LSB-first along D, [BH][S][D*bits/8] (outliers and
 * sinks: code 0); outlier lists of (int32 flat index into this call's
 * [BH][S][D], fp16 value) in ascending index order, keys and values
 * separately, counts in out_counts[0] (keys) and [1] (values); optional
 * reconstructions fp16 [BH][S][D] (inliers: fp16 of their level; outliers and
 * sinks: x). */

/* [host] Upper bound on the outlier-list length of one call (which = 0 keys,
 * 1 values): keys fit_keys ? BH*D*floor(frac*n_fit) : BH*n_fit*D, values
 * BH*n_fit*floor(frac*D), with n_fit = S minus the call's sink tokens.
 * -1 on invalid arguments. */
int64_t kvq_nuq_outlier_bound(int32_t BH, int32_t S, int32_t D, int32_t start_pos, int32_t n_sink,
                              double frac, int32_t fit_keys, int32_t which);

/* [host] Bytes of device workspace kvq_nuq_fit_quant needs for these sizes
 * (scratch: per-block outlier counts and their per-64-block sums, value
 * outlier staging, the key outliers (a bitmap of one bit per key element, or
 * staging slots in a call of at most 256 vectors), and for a key fit over
 * more than 8,192 tokens one byte per key sample).
 * -1 on invalid arguments. */
int64_t kvq_nuq_workspace_bytes(int32_t BH, int32_t S, int32_t D, int32_t bits, int32_t start_pos,
                                int32_t n_sink, double frac, int32_t fit_keys);

/* One NUQ call over fp16 keys and values [BH][S][D] (BH = batch*kv_heads).
 *   bits 1..4 (L = 2^bits); D in {32, 64, 128, 256}; 0 <= frac < 1;
 *   0 <= lloyd_iters <= 1000; a key fit (fit_keys = 1) covers at most
 *   1,048,576 (2^20) non-sink tokens per call (its per-bucket significand
 *   sums stay below 2^32); BH*S*D < 2^31 (int32 outlier positions).
 *   key_levels fp32 [BH][D][L] and key_thresh fp16 [BH][D]: written when
 *   fit_keys = 1, read otherwise (each channel's table ascending, as a fit
 *   leaves it). value_levels fp32 [BH][S][L] (written).
 *   k_codes/v_codes uint8 [BH][S][D*bits/8]. k_opos/k_oval, v_opos/v_oval:
 *   out_cap entries each; out_cap must be >= kvq_nuq_outlier_bound for both
 *   lists (else KVQ_ERR_CAPACITY). out_counts int64 [2] (device).
 *   k_recon / v_recon: optional (NULL to skip).
 *   workspace: device memory of at least kvq_nuq_workspace_bytes, owned by
 *   the caller, 16-byte aligned; its contents on entry do not matter.
 * Calls that share a workspace must not overlap.
 * Streams: when BH*S > 4096 the value fit runs on a second stream of the
 * current device, forked from `stream` after the call's first kernel and
 * joined back into it before the last (event record / stream wait), so the
 * call stays ordered on `stream` like every other. That stream (non-blocking,
 * default priority) and its two events are created on the first such call
 * on each device and kept until the process ends; concurrent host threads
 * are serialised around the fork and join.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_BITS, KVQ_ERR_SHAPE, KVQ_ERR_ARG (frac,
 * iters), KVQ_ERR_CAPACITY, KVQ_ERR_ALIGN, KVQ_ERR_HIP. */
int kvq_nuq_fit_quant(const uint16_t *keys, const uint16_t *values, int32_t BH, int32_t S, int32_t D,
                      int32_t start_pos, int32_t bits, double frac, int32_t lloyd_iters, int32_t n_sink,
                      int32_t fit_keys, float *key_levels, uint16_t *key_thresh, float *value_levels,
                      uint8_t *k_codes, uint8_t *v_codes, int32_t *k_opos, uint16_t *k_oval,
                      int32_t *v_opos, uint16_t *v_oval, int64_t out_cap, int64_t *out_counts,
                      uint16_t *k_recon, uint16_t *v_recon, void *workspace, int64_t workspace_bytes,
                      void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, serving loops that forbid allocation, harnesses that do not allow
 * hipMalloc: kvq_nuq_fit_quant without the workspace argument. The workspace
 * is a static device array of KVQ_NUQ_NOALLOC_WORKSPACE_BYTES (32 MiB) built
 * into the library: every device the library runs on holds one copy until
 * the process ends, looked up (hipGetSymbolAddress) on the first call made
 * with that device current. The call allocates nothing, creates no stream or
 * event, and runs every kernel on `stream` (no auxiliary stream); counters
 * in the array are cleared by the call's first kernel. Arguments, outputs and
 * errors as kvq_nuq_fit_quant, plus KVQ_ERR_CAPACITY when the call needs more
 * workspace than the array holds (kvq_nuq_workspace_bytes gives the need:
 * e.g. 32 (batch, head) vectors x 4096 tokens x D = 128 need about 3 MiB).
 * All calls on one device share the one array: calls that overlap on a
 * device (other streams, other host threads) race and must be serialised by
 * the caller. */
#define KVQ_NUQ_NOALLOC_WORKSPACE_BYTES (32u << 20)
int kvq_nuq_fit_quant_noalloc(const uint16_t *keys, const uint16_t *values, int32_t BH, int32_t S, int32_t D,
                              int32_t start_pos, int32_t bits, double frac, int32_t lloyd_iters, int32_t n_sink,
                              int32_t fit_keys, float *key_levels, uint16_t *key_thresh, float *value_levels,
                              uint8_t *k_codes, uint8_t *v_codes, int32_t *k_opos, uint16_t *k_oval,
                              int32_t *v_opos, uint16_t *v_oval, int64_t out_cap, int64_t *out_counts,
                              uint16_t *k_recon, uint16_t *v_recon, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
