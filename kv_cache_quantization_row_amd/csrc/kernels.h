// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct SymQuantArgs {
  const uint16_t *k, *v;           // fp16 [n_layers][n_tokens][H][D]
  uint8_t *k_codes, *v_codes;      // pools
  uint16_t *k_scales, *v_scales;
  const int32_t *slot_mapping;     // [n_tokens]
  int64_t n_slots;                 // num_pages * page_size
  int64_t code_layer_stride;       // bytes per pool layer
  int64_t scale_layer_stride;      // scales per pool layer
  uint32_t rows_per_layer;         // n_tokens * H
  int32_t layer0, H, D, h_shift;   // h_shift = log2(H) when H is a power of two, else -1
};

struct SymDequantArgs {
  const uint8_t *k_codes, *v_codes;
  const uint16_t *k_scales, *v_scales;
  uint16_t *k_out, *v_out;         // fp16 [n_layers][n_seqs][max_len][H][D]
  const int32_t *block_table;      // [n_seqs][max_blocks]
  const int32_t *seq_lens;         // [n_seqs]
  int64_t code_layer_stride, scale_layer_stride;
  int32_t layer0, H, D, h_shift;
  int32_t num_pages, page_size, max_blocks, n_seqs, max_len;
  int32_t ppb;                     // positions per workgroup (set by the launcher)
};

hipError_t launch_sym_quant(const SymQuantArgs &a, int bits, int n_layers, hipStream_t st);
hipError_t launch_sym_dequant(const SymDequantArgs &a, int bits, int n_layers, hipStream_t st);

struct KiviArgs {
  uint16_t *keys, *values;         // fp16 [B][H][S_cap][D], in place on [lo, hi) (read only when packed)
  uint8_t *k_codes, *v_codes;      // optional (required when packed)
  float *k_scale, *k_min, *v_scale, *v_min;        // binary32 parameters (round trip)
  uint16_t *k_s16, *k_z16, *v_s16, *v_z16;         // fp16 parameters (packed)
  int64_t BH;
  int32_t S_cap, D, lo, hi, bits, gs;
  float eps;
  int32_t packed;      // 1: fp16 parameters (scale rounded toward zero), no reconstruction written
  int32_t code_rows;   // code / value-parameter rows per (b, h): hi - lo, or S_cap when packed
  int32_t code_t0;     // token of row 0: lo, or 0 when packed
  int32_t kgrp_rows;   // key parameter groups per (b, h): ceil((hi-lo)/gs), or ceil(S_cap/gs)
  int32_t kgrp0;       // group index of the first group (0, or lo/gs when packed)
  int32_t x_rows;      // fp16 rows per (b, h) of keys / values (S_cap in place)
  int32_t x_t0;        // token held by fp16 row 0 (0 in place)
};

hipError_t launch_kivi(const KiviArgs &a, hipStream_t st);

struct KiviUnpackArgs {
  const uint8_t *codes;            // [BH][S_cap][D*bits/8]
  const uint16_t *scale, *zero;    // fp16: keys [BH][ceil(S_cap/gs)][D], values [BH][S_cap][ceil(D/gs)]
  uint16_t *out;                   // fp16 [BH][out_rows][D]: token t in row t - out_t0, tokens [lo, hi) written
  int64_t BH;
  int32_t S_cap, D, lo, hi, bits, gs, per_channel;
  int32_t out_rows, out_t0;
  int32_t chunk_shift, gs_shift;   // log2(D/8), log2(gs) when powers of two, else -1 (set by the launcher)
};
hipError_t launch_kivi_unpack(KiviUnpackArgs a, hipStream_t st);

struct NuqArgs {
  const uint16_t *keys, *values;   // fp16 [BH][S][D]
  int32_t BH, S, D, bits, iters, fit_keys, n_sink_eff;
  int32_t k_key, k_val;            // outliers per vector: floor(frac * n) for a key fit (n = non-sink tokens), a value token (n = D)
  float *key_levels;               // [BH][D][L]
  uint16_t *key_thresh;            // [BH][D]
  float *value_levels;             // [BH][S][L]
  uint8_t *k_codes, *v_codes;      // [BH][S][D*bits/8]
  int32_t *k_opos, *v_opos;
  uint16_t *k_oval, *v_oval;
  int64_t *out_counts;             // [2]
  uint16_t *k_recon, *v_recon;     // optional
  // workspace
  uint32_t *ws_kblk, *ws_vblk;     // per workgroup (staging base, count)
  uint32_t *ws_ksup, *ws_vsup;     // per 64 workgroups: sum of their counts
  int32_t *ws_kpos, *ws_vpos;      // staging
  uint8_t *ws_kdat;                // key fit over more than 8192 tokens: bucketed key bytes [BH][D][round16(n)]
  uint8_t *ws_kbits;               // calls that are not small: key outlier bitmap [BH][S][D/8], bit e of byte g
                                   // for channel 8g+e (each key producer writes its bytes; no staging)
  int64_t k_cap, v_cap;            // list entries (the outlier bounds)
  int64_t k_scap;                  // key staging entries: BH*S*D for a small call, else 0 (the bitmap)
  int32_t small;                   // 1: a small call (one fused kernel, then one placement workgroup); key
                                   // workgroups stage at the flat index of their first element, nothing
                                   // needs a zeroed counter
  int64_t v_scap;                  // value staging entries: k_val slots for every token of every value workgroup
                                   // (writes past any of these bounds are dropped)
  uint16_t *ws_kval, *ws_vval;
  int64_t k_blk_x, v_nblk;         // key-quant workgroups along S (16384/D rows each); value workgroups
};

// fork: run a many-token value fit on the device's auxiliary stream (false:
// every kernel on `st`, no stream or event is created)
// Key fit: channels of at most NUQ_KFIT_LDS_N non-sink tokens keep their
// bucketed samples in LDS, longer ones in the workspace; a key fit covers at
// most NUQ_KFIT_MAX_N tokens (its per-bucket significand sums stay below 2^32
// and its exact sums below 2^63).
constexpr int NUQ_KFIT_LDS_N = 8192;
constexpr int NUQ_KFIT_MAX_N = 1 << 20;
hipError_t launch_nuq(const NuqArgs &a, int key_cpc, int val_cpc, bool fork, hipStream_t st);

// Attention chunks are whole blocks of 16 positions and never shorter than
// ATTN_MIN_CHUNK positions, so a sequence of max_len positions has at most
// ceil(max_len / ATTN_MIN_CHUNK) chunk partials in the workspace.
constexpr int ATTN_MIN_CHUNK = 256;
struct AttnArgs {
  const uint8_t *k_codes, *v_codes;      // pools as in SymDequantArgs
  const uint16_t *k_scales, *v_scales;
  int64_t code_layer_stride, scale_layer_stride;
  int32_t layer, num_pages, page_size, kv_heads, head_dim, bits;
  const uint16_t *q;                     // fp16 [n_seqs][q_heads][D]
  int32_t q_heads, group;                // group = q_heads / kv_heads (<= 16)
  const int32_t *block_table;            // [n_seqs][max_blocks]
  int32_t max_blocks;
  const int32_t *seq_lens;               // [n_seqs]
  int32_t n_seqs, max_len;
  int32_t n_chunks, chunk_blocks;        // set by launch_attn_decode
  float scale_log2;                      // softmax scale * log2(e)
  float *ws;                             // [n_seqs][n_chunks][q_heads][D + 2]
  uint16_t *out;                         // fp16 [n_seqs][q_heads][D]
};
hipError_t launch_attn_decode(AttnArgs a, hipStream_t st);

}  // namespace kvq
