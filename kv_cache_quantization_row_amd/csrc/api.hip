// C-ABI entry points of libkvq: host-side validation, then kernel launch on
// the caller's stream. Declarations and argument documentation: include/kvq.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>

#include "../../include/kvq.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return KVQ_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// product of non-negative sizes is below `limit` (false also when the product
// does not fit in 64 bits)
bool product_below(std::initializer_list<int64_t> factors, int64_t limit) {
  int64_t r = 1;
  for (const int64_t f : factors)
    if (__builtin_mul_overflow(r, f, &r)) return false;
  return r < limit;
}

int32_t qmax_of(int32_t bits) {
  switch (bits) {  // explicit table; unknown widths are not mapped to a neighbour
    case 8: return 127;
    case 6: return 31;
    case 4: return 7;
    default: return -1;
  }
}

int64_t packed(int32_t D, int32_t bits) {
  if (D <= 0 || qmax_of(bits) < 0) return -1;
  if (bits == 6 && D % 4) return -1;
  if (bits == 4 && D % 2) return -1;
  return (int64_t)D * bits / 8;
}

int h_shift_of(int32_t H) {
  if (H <= 0 || (H & (H - 1))) return -1;
  int s = 0;
  while ((1 << s) < H) ++s;
  return s;
}

int check_layout(const kvq_paged_layout *L) {
  if (!L) return fail(KVQ_ERR_NULL, "layout is NULL");
  if (qmax_of(L->bits) < 0) return fail(KVQ_ERR_BITS, "bits=%d is not one of 8, 6, 4", L->bits);
  if (packed(L->head_dim, L->bits) < 0)
    return fail(KVQ_ERR_SHAPE, "head_dim=%d is not valid for q%d (q6 needs D%%4==0, q4 even D)",
                L->head_dim, L->bits);
  if (L->layers <= 0 || L->num_pages <= 0 || L->page_size <= 0 || L->kv_heads <= 0)
    return fail(KVQ_ERR_SHAPE, "layout sizes must be positive (layers=%d pages=%d page_size=%d heads=%d)",
                L->layers, L->num_pages, L->page_size, L->kv_heads);
  const int64_t slots = (int64_t)L->num_pages * L->page_size;
  int64_t rows = 0;
  if (__builtin_mul_overflow(slots, (int64_t)L->kv_heads, &rows) || rows >= ((int64_t)1 << 40))
    return fail(KVQ_ERR_SHAPE, "pool too large");
  return KVQ_OK;
}

}  // namespace

extern "C" {

const char *kvq_last_error(void) { return g_err.c_str(); }

const char *kvq_version(void) { return "kvq 0.1 gfx950"; }

int kvq_parse_mode(const char *mode, int32_t *bits) {
  if (!mode || !bits) return fail(KVQ_ERR_NULL, "mode or bits is NULL");
  static const struct {
    const char *name;
    int32_t bits;
  } table[] = {{"q8", 8}, {"8", 8}, {"q6", 6}, {"6", 6}, {"6bit", 6}, {"int6", 6},
               {"uint6", 6}, {"q4", 4}, {"4", 4}};
  for (const auto &e : table)
    if (std::strcmp(mode, e.name) == 0) {
      *bits = e.bits;
      return ok();
    }
  return fail(KVQ_ERR_MODE, "unknown KV quantization mode '%s'", mode);
}

int32_t kvq_sym_qmax(int32_t bits) { return qmax_of(bits); }

int64_t kvq_packed_dim(int32_t head_dim, int32_t bits) { return packed(head_dim, bits); }

int64_t kvq_sym_cache_bytes(int64_t tokens, int32_t layers, int32_t kv_heads, int32_t head_dim,
                            int32_t bits) {
  if (tokens < 0 || layers <= 0 || kv_heads <= 0 || head_dim <= 0) return -1;
  int64_t row;
  if (bits == 16) {
    row = 2 * (int64_t)head_dim;
  } else {
    const int64_t pd = packed(head_dim, bits);
    if (pd < 0) return -1;
    row = pd + 2;
  }
  int64_t r = 2 * row;
  for (const int64_t f : {tokens, (int64_t)layers, (int64_t)kv_heads})
    if (__builtin_mul_overflow(r, f, &r)) return -1;  // not representable
  return r;
}

int kvq_quant_sym(const kvq_paged_layout *layout, const uint16_t *k, const uint16_t *v,
                  int32_t layer0, int32_t n_layers, int32_t n_tokens,
                  const int32_t *slot_mapping, uint8_t *k_codes, uint16_t *k_scales,
                  uint8_t *v_codes, uint16_t *v_scales, void *stream) {
  int rc = check_layout(layout);
  if (rc) return rc;
  const kvq_paged_layout &L = *layout;
  if (n_tokens < 0 || n_layers < 0) return fail(KVQ_ERR_SHAPE, "negative n_tokens/n_layers");
  if (layer0 < 0 || (int64_t)layer0 + n_layers > L.layers)
    return fail(KVQ_ERR_SHAPE, "layers [%d, %lld) outside the pool's %d layers", layer0,
                (long long)layer0 + n_layers, L.layers);
  const bool do_k = k || k_codes || k_scales, do_v = v || v_codes || v_scales;
  if (do_k && (!k || !k_codes || !k_scales))
    return fail(KVQ_ERR_NULL, "K side needs k, k_codes and k_scales together");
  if (do_v && (!v || !v_codes || !v_scales))
    return fail(KVQ_ERR_NULL, "V side needs v, v_codes and v_scales together");
  if (!do_k && !do_v) return fail(KVQ_ERR_NULL, "neither K nor V given");
  if (n_tokens == 0 || n_layers == 0) return ok();
  if (!slot_mapping) return fail(KVQ_ERR_NULL, "slot_mapping is NULL");
  const int64_t rows = (int64_t)n_tokens * L.kv_heads;
  if (rows >= ((int64_t)1 << 31)) return fail(KVQ_ERR_SHAPE, "n_tokens*kv_heads must be < 2^31");
  if (n_layers > 65535) return fail(KVQ_ERR_SHAPE, "at most 65535 layers per call");
  for (const void *p : {(const void *)k, (const void *)v, (const void *)k_codes, (const void *)v_codes})
    if (p && !aligned(p, 16)) return fail(KVQ_ERR_ALIGN, "fp16 input and code pools need 16-byte alignment");
  for (const void *p : {(const void *)k_scales, (const void *)v_scales})
    if (p && !aligned(p, 2)) return fail(KVQ_ERR_ALIGN, "scales need 2-byte alignment");
  if (!aligned(slot_mapping, 4)) return fail(KVQ_ERR_ALIGN, "slot_mapping needs 4-byte alignment");

  const int64_t pd = packed(L.head_dim, L.bits);
  const int64_t slots = (int64_t)L.num_pages * L.page_size;
  kvq::SymQuantArgs a{};
  a.k = do_k ? k : nullptr;
  a.v = do_v ? v : nullptr;
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.slot_mapping = slot_mapping;
  a.n_slots = slots;
  a.code_layer_stride = slots * L.kv_heads * pd;
  a.scale_layer_stride = slots * L.kv_heads;
  a.rows_per_layer = (uint32_t)rows;
  a.layer0 = layer0;
  a.H = L.kv_heads;
  a.D = L.head_dim;
  a.h_shift = h_shift_of(L.kv_heads);
  return hip_status(kvq::launch_sym_quant(a, L.bits, n_layers, (hipStream_t)stream), "kvq_quant_sym launch");
}

int kvq_dequant_sym(const kvq_paged_layout *layout, const uint8_t *k_codes,
                    const uint16_t *k_scales, const uint8_t *v_codes, const uint16_t *v_scales,
                    int32_t layer0, int32_t n_layers, const int32_t *block_table,
                    int32_t max_blocks, const int32_t *seq_lens, int32_t n_seqs, int32_t max_len,
                    uint16_t *k_out, uint16_t *v_out, void *stream) {
  int rc = check_layout(layout);
  if (rc) return rc;
  const kvq_paged_layout &L = *layout;
  if (n_seqs < 0 || n_layers < 0 || max_len < 0 || max_blocks < 0)
    return fail(KVQ_ERR_SHAPE, "negative size");
  if (layer0 < 0 || (int64_t)layer0 + n_layers > L.layers)
    return fail(KVQ_ERR_SHAPE, "layers [%d, %lld) outside the pool's %d layers", layer0,
                (long long)layer0 + n_layers, L.layers);
  const bool do_k = k_out || k_codes || k_scales, do_v = v_out || v_codes || v_scales;
  if (do_k && (!k_out || !k_codes || !k_scales))
    return fail(KVQ_ERR_NULL, "K side needs k_codes, k_scales and k_out together");
  if (do_v && (!v_out || !v_codes || !v_scales))
    return fail(KVQ_ERR_NULL, "V side needs v_codes, v_scales and v_out together");
  if (!do_k && !do_v) return fail(KVQ_ERR_NULL, "neither K nor V given");
  if (n_seqs == 0 || n_layers == 0 || max_len == 0) return ok();
  if (!block_table || !seq_lens) return fail(KVQ_ERR_NULL, "block_table or seq_lens is NULL");
  if (max_blocks == 0) return fail(KVQ_ERR_SHAPE, "max_blocks must be positive");
  if ((int64_t)max_len * L.kv_heads >= ((int64_t)1 << 31))
    return fail(KVQ_ERR_SHAPE, "max_len*kv_heads must be < 2^31");
  if (n_seqs > 65535 || 2 * (int64_t)n_layers > 65535)
    return fail(KVQ_ERR_SHAPE, "at most 65535 sequences and 32767 layers per call");
  for (const void *p : {(const void *)k_out, (const void *)v_out, (const void *)k_codes, (const void *)v_codes})
    if (p && !aligned(p, 16)) return fail(KVQ_ERR_ALIGN, "fp16 output and code pools need 16-byte alignment");
  for (const void *p : {(const void *)k_scales, (const void *)v_scales})
    if (p && !aligned(p, 2)) return fail(KVQ_ERR_ALIGN, "scales need 2-byte alignment");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4))
    return fail(KVQ_ERR_ALIGN, "block_table/seq_lens need 4-byte alignment");

  const int64_t pd = packed(L.head_dim, L.bits);
  const int64_t slots = (int64_t)L.num_pages * L.page_size;
  kvq::SymDequantArgs a{};
  a.k_codes = do_k ? k_codes : nullptr;
  a.v_codes = do_v ? v_codes : nullptr;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.k_out = do_k ? k_out : nullptr;
  a.v_out = do_v ? v_out : nullptr;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.code_layer_stride = slots * L.kv_heads * pd;
  a.scale_layer_stride = slots * L.kv_heads;
  a.layer0 = layer0;
  a.H = L.kv_heads;
  a.D = L.head_dim;
  a.h_shift = h_shift_of(L.kv_heads);
  a.num_pages = L.num_pages;
  a.page_size = L.page_size;
  a.max_blocks = max_blocks;
  a.n_seqs = n_seqs;
  a.max_len = max_len;
  return hip_status(kvq::launch_sym_dequant(a, L.bits, n_layers, (hipStream_t)stream),
                    "kvq_dequant_sym launch");
}

int64_t kvq_attn_workspace_bytes(int32_t n_seqs, int32_t q_heads, int32_t head_dim, int32_t max_len) {
  if (n_seqs < 0 || q_heads <= 0 || head_dim <= 0 || max_len < 0) return -1;
  const int64_t chunks = max_len > 0 ? ((int64_t)max_len + kvq::ATTN_MIN_CHUNK - 1) / kvq::ATTN_MIN_CHUNK : 1;
  int64_t r = 4 * ((int64_t)head_dim + 2);  // fp32 partial output + running max and sum per chunk and head
  for (const int64_t f : {(int64_t)n_seqs, chunks, (int64_t)q_heads})
    if (__builtin_mul_overflow(r, f, &r)) return -1;  // not representable: no valid call has these sizes
  return r;
}

int kvq_attn_decode_sym(const kvq_paged_layout *layout, const uint8_t *k_codes, const uint16_t *k_scales,
                        const uint8_t *v_codes, const uint16_t *v_scales, int32_t layer, const uint16_t *q,
                        int32_t q_heads, const int32_t *block_table, int32_t max_blocks,
                        const int32_t *seq_lens, int32_t n_seqs, int32_t max_len, float softmax_scale,
                        uint16_t *out, void *workspace, int64_t workspace_bytes, void *stream) {
  int rc = check_layout(layout);
  if (rc) return rc;
  const kvq_paged_layout &L = *layout;
  if (L.head_dim != 64 && L.head_dim != 128 && L.head_dim != 256)
    return fail(KVQ_ERR_SHAPE, "attention head_dim must be 64, 128 or 256 (got %d)", L.head_dim);
  if (q_heads <= 0 || q_heads % L.kv_heads != 0 || q_heads / L.kv_heads > 16)
    return fail(KVQ_ERR_SHAPE, "q_heads=%d must be a multiple of kv_heads=%d, at most 16 per KV head", q_heads,
                L.kv_heads);
  if (layer < 0 || layer >= L.layers) return fail(KVQ_ERR_SHAPE, "layer %d outside the pool's %d layers", layer,
                                                  L.layers);
  if (n_seqs < 0 || max_len < 0 || max_blocks < 0) return fail(KVQ_ERR_SHAPE, "negative size");
  if (n_seqs == 0) return ok();
  if (n_seqs > 65535) return fail(KVQ_ERR_SHAPE, "at most 65535 sequences per call");
  if (!(softmax_scale == softmax_scale) || softmax_scale == __builtin_inff() || softmax_scale == -__builtin_inff())
    return fail(KVQ_ERR_ARG, "softmax_scale must be finite");
  if (!k_codes || !k_scales || !v_codes || !v_scales || !q || !out || !seq_lens || !workspace)
    return fail(KVQ_ERR_NULL, "a required attention pointer is NULL");
  if (max_len > 0 && (!block_table || max_blocks == 0))
    return fail(KVQ_ERR_NULL, "block_table is NULL or max_blocks is 0");
  for (const void *p : {(const void *)k_codes, (const void *)v_codes, (const void *)q, (const void *)workspace})
    if (!aligned(p, 16)) return fail(KVQ_ERR_ALIGN, "code pools, q and the workspace need 16-byte alignment");
  if (!aligned(k_scales, 2) || !aligned(v_scales, 2) || !aligned(out, 2) || !aligned(seq_lens, 4) ||
      (block_table && !aligned(block_table, 4)))
    return fail(KVQ_ERR_ALIGN, "misaligned scales, output, block table or lengths");
  const int64_t need = kvq_attn_workspace_bytes(n_seqs, q_heads, L.head_dim, max_len);
  if (workspace_bytes < need)
    return fail(KVQ_ERR_CAPACITY, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                (long long)need);
  const int64_t pd = packed(L.head_dim, L.bits);
  const int64_t slots = (int64_t)L.num_pages * L.page_size;
  kvq::AttnArgs a{};
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.code_layer_stride = slots * L.kv_heads * pd;
  a.scale_layer_stride = slots * L.kv_heads;
  a.layer = layer;
  a.num_pages = L.num_pages;
  a.page_size = L.page_size;
  a.kv_heads = L.kv_heads;
  a.head_dim = L.head_dim;
  a.bits = L.bits;
  a.q = q;
  a.q_heads = q_heads;
  a.group = q_heads / L.kv_heads;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.n_seqs = n_seqs;
  a.max_len = max_len;
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);  // log2(e)
  a.ws = static_cast<float *>(workspace);
  a.out = out;
  return hip_status(kvq::launch_attn_decode(a, (hipStream_t)stream), "kvq_attn_decode_sym launch");
}

int64_t kvq_kivi_boundary(int64_t offset, int32_t residual_length, int32_t group_size) {
  if (group_size <= 0 || residual_length < 0 || offset < 0) return -1;
  int64_t aged = offset - residual_length;
  if (aged < 0) aged = 0;
  return (aged / group_size) * group_size;
}

int kvq_kivi_quant_dequant(uint16_t *keys, uint16_t *values, int32_t B, int32_t H, int32_t S_cap,
                           int32_t D, int32_t lo, int32_t hi, int32_t bits, int32_t group_size,
                           float eps, uint8_t *k_codes, float *k_scale, float *k_min,
                           uint8_t *v_codes, float *v_scale, float *v_min, void *stream) {
  if (!keys && !values) return fail(KVQ_ERR_NULL, "neither keys nor values given");
  if (!keys && (k_codes || k_scale || k_min))
    return fail(KVQ_ERR_NULL, "key outputs given without keys");
  if (!values && (v_codes || v_scale || v_min))
    return fail(KVQ_ERR_NULL, "value outputs given without values");
  if (bits != 2 && bits != 4 && bits != 8) return fail(KVQ_ERR_BITS, "bits=%d is not one of 2, 4, 8", bits);
  if (B < 0 || H < 0 || S_cap < 0 || D <= 0) return fail(KVQ_ERR_SHAPE, "bad B/H/S_cap/D");
  if (lo < 0 || hi < lo || hi > S_cap) return fail(KVQ_ERR_SHAPE, "need 0 <= lo <= hi <= S_cap");
  if (group_size <= 0) return fail(KVQ_ERR_SHAPE, "group_size must be positive");
  if (!(eps > 0.0f) || !(eps < 3.0e38f)) return fail(KVQ_ERR_ARG, "eps must be positive and finite");
  if ((k_codes || v_codes) && (D % 8 || group_size % 8))
    return fail(KVQ_ERR_SHAPE, "packed code output needs D %% 8 == 0 and group_size %% 8 == 0");
  for (const void *p : {(const void *)keys, (const void *)values, (const void *)k_codes, (const void *)v_codes})
    if (p && !aligned(p, 16)) return fail(KVQ_ERR_ALIGN, "fp16 tensors and code buffers need 16-byte alignment");
  for (const void *p : {(const void *)k_scale, (const void *)k_min, (const void *)v_scale, (const void *)v_min})
    if (p && !aligned(p, 4)) return fail(KVQ_ERR_ALIGN, "scale/min buffers need 4-byte alignment");
  const int64_t BH = (int64_t)B * H;
  if (hi == lo || BH == 0) return ok();
  const int64_t n = hi - lo;
  if (!product_below({BH, n, (int64_t)D}, (int64_t)1 << 46)) return fail(KVQ_ERR_SHAPE, "tensor too large");
  if ((BH * n + 255) / 256 * 64 >= ((int64_t)1 << 31)) return fail(KVQ_ERR_SHAPE, "too many rows");
  kvq::KiviArgs a{};
  a.keys = keys;
  a.values = values;
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_scale = k_scale;
  a.k_min = k_min;
  a.v_scale = v_scale;
  a.v_min = v_min;
  a.BH = BH;
  a.S_cap = S_cap;
  a.D = D;
  a.lo = lo;
  a.hi = hi;
  a.bits = bits;
  a.gs = group_size;
  a.eps = eps;
  a.packed = 0;
  a.code_rows = (int32_t)n;
  a.code_t0 = lo;
  a.kgrp_rows = (int32_t)((n + group_size - 1) / group_size);
  a.kgrp0 = 0;
  a.x_rows = S_cap;
  a.x_t0 = 0;
  return hip_status(kvq::launch_kivi(a, (hipStream_t)stream), "kvq_kivi_quant_dequant launch");
}

int kvq_kivi_pack(const uint16_t *keys, const uint16_t *values, int32_t B, int32_t H, int32_t S_cap, int32_t D,
                  int32_t lo, int32_t hi, int32_t bits, int32_t group_size, float eps, uint8_t *k_codes,
                  uint16_t *k_scale, uint16_t *k_zero, uint8_t *v_codes, uint16_t *v_scale, uint16_t *v_zero,
                  int32_t x_rows, int32_t x_t0, void *stream) {
  if (!keys && !values) return fail(KVQ_ERR_NULL, "neither keys nor values given");
  if (keys && (!k_codes || !k_scale || !k_zero)) return fail(KVQ_ERR_NULL, "key codes, scale and zero are required");
  if (values && (!v_codes || !v_scale || !v_zero))
    return fail(KVQ_ERR_NULL, "value codes, scale and zero are required");
  if (bits != 2 && bits != 4 && bits != 8) return fail(KVQ_ERR_BITS, "bits=%d is not one of 2, 4, 8", bits);
  if (B < 0 || H < 0 || S_cap < 0 || D <= 0) return fail(KVQ_ERR_SHAPE, "bad B/H/S_cap/D");
  if (lo < 0 || hi < lo || hi > S_cap) return fail(KVQ_ERR_SHAPE, "need 0 <= lo <= hi <= S_cap");
  if (group_size <= 0 || group_size % 8 || D % 8)
    return fail(KVQ_ERR_SHAPE, "packed storage needs D %% 8 == 0 and group_size a positive multiple of 8");
  if (keys && lo % group_size)
    return fail(KVQ_ERR_SHAPE, "key groups start at token 0: lo=%d must be a multiple of group_size", lo);
  if (x_rows < 0 || x_t0 < 0 || (hi > lo && (x_t0 > lo || (int64_t)hi > (int64_t)x_t0 + x_rows)))
    return fail(KVQ_ERR_SHAPE, "input rows [%d, %d + %d) do not hold tokens [%d, %d)", x_t0, x_t0, x_rows, lo, hi);
  if (!(eps > 0.0f) || !(eps < 3.0e38f)) return fail(KVQ_ERR_ARG, "eps must be positive and finite");
  for (const void *p : {(const void *)keys, (const void *)values, (const void *)k_codes, (const void *)v_codes,
                        (const void *)k_scale, (const void *)k_zero, (const void *)v_scale, (const void *)v_zero})
    if (p && !aligned(p, 16)) return fail(KVQ_ERR_ALIGN, "packed KIVI tensors need 16-byte alignment");
  const int64_t BH = (int64_t)B * H;
  if (hi == lo || BH == 0) return ok();
  const int64_t n = hi - lo;
  if (!product_below({BH, (int64_t)S_cap, (int64_t)D}, (int64_t)1 << 46) ||
      !product_below({BH, (int64_t)x_rows, (int64_t)D}, (int64_t)1 << 46))
    return fail(KVQ_ERR_SHAPE, "tensor too large");
  if ((BH * n + 255) / 256 * 64 >= ((int64_t)1 << 31)) return fail(KVQ_ERR_SHAPE, "too many rows");
  kvq::KiviArgs a{};
  a.keys = const_cast<uint16_t *>(keys);  // read only: packed mode writes no reconstruction
  a.values = const_cast<uint16_t *>(values);
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_s16 = k_scale;
  a.k_z16 = k_zero;
  a.v_s16 = v_scale;
  a.v_z16 = v_zero;
  a.BH = BH;
  a.S_cap = S_cap;
  a.D = D;
  a.lo = lo;
  a.hi = hi;
  a.bits = bits;
  a.gs = group_size;
  a.eps = eps;
  a.packed = 1;
  a.code_rows = S_cap;
  a.code_t0 = 0;
  a.kgrp_rows = (int32_t)(((int64_t)S_cap + group_size - 1) / group_size);
  a.kgrp0 = lo / group_size;
  a.x_rows = x_rows;
  a.x_t0 = x_t0;
  return hip_status(kvq::launch_kivi(a, (hipStream_t)stream), "kvq_kivi_pack launch");
}

int kvq_kivi_unpack(const uint8_t *k_codes, const uint16_t *k_scale, const uint16_t *k_zero, const uint8_t *v_codes,
                    const uint16_t *v_scale, const uint16_t *v_zero, int32_t B, int32_t H, int32_t S_cap, int32_t D,
                    int32_t lo, int32_t hi, int32_t bits, int32_t group_size, uint16_t *k_out, uint16_t *v_out,
                    int32_t out_rows, int32_t out_t0, void *stream) {
  if (!k_out && !v_out) return fail(KVQ_ERR_NULL, "neither key nor value output given");
  if (k_out && (!k_codes || !k_scale || !k_zero)) return fail(KVQ_ERR_NULL, "key codes, scale and zero are required");
  if (v_out && (!v_codes || !v_scale || !v_zero))
    return fail(KVQ_ERR_NULL, "value codes, scale and zero are required");
  if (bits != 2 && bits != 4 && bits != 8) return fail(KVQ_ERR_BITS, "bits=%d is not one of 2, 4, 8", bits);
  if (B < 0 || H < 0 || S_cap < 0 || D <= 0) return fail(KVQ_ERR_SHAPE, "bad B/H/S_cap/D");
  if (lo < 0 || hi < lo || hi > S_cap) return fail(KVQ_ERR_SHAPE, "need 0 <= lo <= hi <= S_cap");
  if (group_size <= 0 || group_size % 8 || D % 8)
    return fail(KVQ_ERR_SHAPE, "packed storage needs D %% 8 == 0 and group_size a positive multiple of 8");
  if (out_rows < 0 || out_t0 < 0 || (hi > lo && (out_t0 > lo || (int64_t)hi > (int64_t)out_t0 + out_rows)))
    return fail(KVQ_ERR_SHAPE, "output rows [%d, %d + %d) do not hold tokens [%d, %d)", out_t0, out_t0, out_rows, lo,
                hi);
  for (const void *p : {(const void *)k_codes, (const void *)v_codes, (const void *)k_scale, (const void *)k_zero,
                        (const void *)v_scale, (const void *)v_zero, (const void *)k_out, (const void *)v_out})
    if (p && !aligned(p, 16)) return fail(KVQ_ERR_ALIGN, "packed KIVI tensors need 16-byte alignment");
  const int64_t BH = (int64_t)B * H;
  if (hi == lo || BH == 0) return ok();
  if (!product_below({BH, (int64_t)S_cap, (int64_t)D}, (int64_t)1 << 46) ||
      !product_below({BH, (int64_t)out_rows, (int64_t)D}, (int64_t)1 << 46))
    return fail(KVQ_ERR_SHAPE, "tensor too large");
  if ((int64_t)(hi - lo) * (D / 8) >= ((int64_t)1 << 31) - 256 || (BH + 65534) / 65535 > 65535)
    return fail(KVQ_ERR_SHAPE, "too many rows");
  kvq::KiviUnpackArgs a{};
  a.BH = BH;
  a.S_cap = S_cap;
  a.D = D;
  a.lo = lo;
  a.hi = hi;
  a.bits = bits;
  a.gs = group_size;
  a.out_rows = out_rows;
  a.out_t0 = out_t0;
  for (int side = 0; side < 2; ++side) {
    uint16_t *out = side ? v_out : k_out;
    if (!out) continue;
    a.codes = side ? v_codes : k_codes;
    a.scale = side ? v_scale : k_scale;
    a.zero = side ? v_zero : k_zero;
    a.out = out;
    a.per_channel = side == 0;
    const int rc = hip_status(kvq::launch_kivi_unpack(a, (hipStream_t)stream), "kvq_kivi_unpack launch");
    if (rc) return rc;
  }
  return ok();
}

// ------------------------------------------------------------------ NUQ
namespace {
struct NuqPlan {
  int n_sink_eff, n_fit, key_cpc, val_cpc;
  int64_t kb, vb;  // outlier bounds
  int64_t vs;      // value staging slots: k_val per token of every value workgroup
  int64_t ks;      // key staging slots: BH*S*D for a small call, else none (the outlier bitmap)
  bool small;      // at most 256 (batch, head, token) vectors: one fused kernel and one placement workgroup
  int64_t k_blk_x, v_nblk;
  int64_t off_kblk, off_vblk, off_ksup, off_vsup, off_kpos, off_kval, off_vpos, off_vval, off_kdat, off_kbits,
      total;
};

// outliers per vector of n samples: floor(frac * n), one binary64 product
int64_t floor_frac(double frac, int64_t n) { return (int64_t)std::floor(frac * (double)n); }

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

int nuq_plan(int32_t BH, int32_t S, int32_t D, int32_t bits, int32_t start_pos, int32_t n_sink,
             double frac, int32_t fit_keys, NuqPlan &p) {
  if (bits < 1 || bits > 4) return fail(KVQ_ERR_BITS, "NUQ bits=%d is not in 1..4", bits);
  if (BH <= 0 || S <= 0) return fail(KVQ_ERR_SHAPE, "BH and S must be positive");
  if (D != 32 && D != 64 && D != 128 && D != 256) return fail(KVQ_ERR_SHAPE, "NUQ head_dim must be 32, 64, 128 or 256 (got %d)", D);
  if (!(frac >= 0.0 && frac < 1.0)) return fail(KVQ_ERR_ARG, "outlier fraction must be in [0, 1)");
  if (start_pos < 0 || n_sink < 0) return fail(KVQ_ERR_ARG, "start_pos and n_sink must be >= 0");
  if (BH > 65535) return fail(KVQ_ERR_SHAPE, "BH must be <= 65535");
  if ((int64_t)BH * S * D >= ((int64_t)1 << 31)) return fail(KVQ_ERR_SHAPE, "BH*S*D must be < 2^31 (int32 outlier positions)");
  p.n_sink_eff = start_pos == 0 ? (n_sink < S ? n_sink : S) : 0;
  p.n_fit = S - p.n_sink_eff;
  if (fit_keys && p.n_fit > kvq::NUQ_KFIT_MAX_N)
    return fail(KVQ_ERR_SHAPE, "a key fit covers at most %d non-sink tokens per call (got %d)", kvq::NUQ_KFIT_MAX_N,
                p.n_fit);
  int chunks = (p.n_fit + 127) / 128, cpc = 1;
  while (cpc < chunks) cpc <<= 1;
  p.key_cpc = cpc;
  // values: one wave per token for up to 4096 tokens (latency), else one
  // lane (D <= 128) or two lanes (D = 256) per token (throughput)
  p.val_cpc = (int64_t)BH * S <= 4096 ? 0 : (D <= 128 ? 1 : 2);
  p.kb = fit_keys ? (int64_t)BH * D * floor_frac(frac, p.n_fit) : (int64_t)BH * p.n_fit * D;
  p.vb = (int64_t)BH * p.n_fit * floor_frac(frac, D);
  const int rpb = 16384 / D;  // key-quant rows per workgroup: 4 waves x 8 steps x 512/D rows
  p.k_blk_x = (S + rpb - 1) / rpb;
  p.v_nblk = p.val_cpc == 0 ? (int64_t)BH * S : ((int64_t)BH * S + (64 / p.val_cpc) - 1) / (64 / p.val_cpc);
  int64_t o = 0;
  p.off_kblk = o; o = align256(o + p.k_blk_x * BH * 8);
  p.off_vblk = o; o = align256(o + p.v_nblk * 8);
  p.off_ksup = o; o = align256(o + (p.k_blk_x * BH + 63) / 64 * 4);
  p.off_vsup = o; o = align256(o + (p.v_nblk + 63) / 64 * 4);
  // a small call's key workgroups stage at the flat index of their first
  // element (no shared counter to clear); other calls mark key outliers in a
  // bitmap, from which the placement emits them in flat order
  p.small = p.val_cpc == 0 && (int64_t)BH * S <= 256;
  p.ks = p.small ? (int64_t)BH * S * D : 0;
  p.off_kpos = o; o = align256(o + p.ks * 4);
  p.off_kval = o; o = align256(o + p.ks * 2);
  // value workgroups stage their outliers at fixed offsets (no shared
  // counter): k_val slots for each token they cover, sinks and padding too
  p.vs = (p.val_cpc == 0 ? (int64_t)BH * S : p.v_nblk * (64 / p.val_cpc)) * floor_frac(frac, D);
  p.off_vpos = o; o = align256(o + p.vs * 4);
  p.off_vval = o; o = align256(o + p.vs * 2);
  // a key fit over more tokens than fit in LDS keeps its bucketed samples here
  const int64_t kdat = fit_keys && p.n_fit > kvq::NUQ_KFIT_LDS_N ? (int64_t)BH * D * ((p.n_fit + 15) / 16 * 16) : 0;
  p.off_kdat = o; o = align256(o + kdat);
  p.off_kbits = o; o = align256(o + (p.small ? 0 : (int64_t)BH * S * (D / 8)));
  p.total = o;
  return KVQ_OK;
}
}  // namespace

int64_t kvq_nuq_outlier_bound(int32_t BH, int32_t S, int32_t D, int32_t start_pos, int32_t n_sink,
                              double frac, int32_t fit_keys, int32_t which) {
  NuqPlan p;
  if (nuq_plan(BH, S, D, 1, start_pos, n_sink, frac, fit_keys, p) != KVQ_OK) return -1;
  return which == 0 ? p.kb : (which == 1 ? p.vb : -1);
}

int64_t kvq_nuq_workspace_bytes(int32_t BH, int32_t S, int32_t D, int32_t bits, int32_t start_pos,
                                int32_t n_sink, double frac, int32_t fit_keys) {
  NuqPlan p;
  if (nuq_plan(BH, S, D, bits, start_pos, n_sink, frac, fit_keys, p) != KVQ_OK) return -1;
  return p.total;
}

}  // extern "C"

namespace {
// One NUQ call with a given workspace: host validation, then the launches.
int nuq_call(const uint16_t *keys, const uint16_t *values, int32_t BH, int32_t S, int32_t D, int32_t start_pos,
             int32_t bits, double frac, int32_t lloyd_iters, int32_t n_sink, int32_t fit_keys, float *key_levels,
             uint16_t *key_thresh, float *value_levels, uint8_t *k_codes, uint8_t *v_codes, int32_t *k_opos,
             uint16_t *k_oval, int32_t *v_opos, uint16_t *v_oval, int64_t out_cap, int64_t *out_counts,
             uint16_t *k_recon, uint16_t *v_recon, const NuqPlan &p, void *workspace, bool fork, void *stream,
             const char *what) {
  if (lloyd_iters < 0 || lloyd_iters > 1000) return fail(KVQ_ERR_ARG, "lloyd_iters must be in [0, 1000]");
  if (!keys || !values || !key_levels || !key_thresh || !value_levels || !k_codes || !v_codes ||
      !k_opos || !k_oval || !v_opos || !v_oval || !out_counts || !workspace)
    return fail(KVQ_ERR_NULL, "a required NUQ pointer is NULL");
  if (out_cap < p.kb || out_cap < p.vb)
    return fail(KVQ_ERR_CAPACITY, "out_cap=%lld below the outlier bound (keys %lld, values %lld)",
                (long long)out_cap, (long long)p.kb, (long long)p.vb);
  for (const void *q : {(const void *)keys, (const void *)values, (const void *)k_codes, (const void *)v_codes,
                        (const void *)k_recon, (const void *)v_recon, (const void *)workspace})
    if (q && !aligned(q, 16)) return fail(KVQ_ERR_ALIGN, "fp16 tensors, code buffers and the workspace need 16-byte alignment");
  for (const void *q : {(const void *)key_levels, (const void *)value_levels, (const void *)k_opos, (const void *)v_opos})
    if (!aligned(q, 4)) return fail(KVQ_ERR_ALIGN, "level tables and position lists need 4-byte alignment");
  if (!aligned(key_thresh, 2) || !aligned(k_oval, 2) || !aligned(v_oval, 2) || !aligned(out_counts, 8))
    return fail(KVQ_ERR_ALIGN, "misaligned threshold, value list or counts");
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  kvq::NuqArgs a{};
  a.keys = keys;
  a.values = values;
  a.BH = BH;
  a.S = S;
  a.D = D;
  a.bits = bits;
  a.iters = lloyd_iters;
  a.fit_keys = fit_keys ? 1 : 0;
  a.n_sink_eff = p.n_sink_eff;
  a.k_key = (int32_t)floor_frac(frac, p.n_fit);
  a.k_val = (int32_t)floor_frac(frac, D);
  a.key_levels = key_levels;
  a.key_thresh = key_thresh;
  a.value_levels = value_levels;
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_opos = k_opos;
  a.v_opos = v_opos;
  a.k_oval = k_oval;
  a.v_oval = v_oval;
  a.out_counts = out_counts;
  a.k_recon = k_recon;
  a.v_recon = v_recon;
  a.ws_kblk = reinterpret_cast<uint32_t *>(ws + p.off_kblk);
  a.ws_vblk = reinterpret_cast<uint32_t *>(ws + p.off_vblk);
  a.ws_ksup = reinterpret_cast<uint32_t *>(ws + p.off_ksup);
  a.ws_vsup = reinterpret_cast<uint32_t *>(ws + p.off_vsup);
  a.ws_kpos = reinterpret_cast<int32_t *>(ws + p.off_kpos);
  a.ws_kval = reinterpret_cast<uint16_t *>(ws + p.off_kval);
  a.ws_vpos = reinterpret_cast<int32_t *>(ws + p.off_vpos);
  a.ws_vval = reinterpret_cast<uint16_t *>(ws + p.off_vval);
  a.ws_kdat = ws + p.off_kdat;
  a.ws_kbits = ws + p.off_kbits;
  a.k_cap = p.kb;
  a.k_scap = p.ks;
  a.small = p.small ? 1 : 0;
  a.v_cap = p.vb;
  a.v_scap = p.vs;
  a.k_blk_x = p.k_blk_x;
  a.v_nblk = p.v_nblk;
  return hip_status(kvq::launch_nuq(a, p.key_cpc, p.val_cpc, fork, (hipStream_t)stream), what);
}

// Workspace of kvq_nuq_fit_quant_noalloc: a file-scope device array, one copy
// per device, addressed through the pointer hipGetSymbolAddress gives for it
// on that device (the array's name in host code is a host-side stand-in, not
// a device address, and is never passed to a kernel or a copy).
static __device__ __align__(256) uint8_t scratch[KVQ_NUQ_NOALLOC_WORKSPACE_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64];  // address of `scratch` on device i, looked up once with that device current

int scratch_on_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(KVQ_ERR_HIP, "device %d is outside the 64 devices supported", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(KVQ_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVQ_OK;
}
}  // namespace

extern "C" {

int kvq_nuq_fit_quant(const uint16_t *keys, const uint16_t *values, int32_t BH, int32_t S, int32_t D,
                      int32_t start_pos, int32_t bits, double frac, int32_t lloyd_iters, int32_t n_sink,
                      int32_t fit_keys, float *key_levels, uint16_t *key_thresh, float *value_levels,
                      uint8_t *k_codes, uint8_t *v_codes, int32_t *k_opos, uint16_t *k_oval,
                      int32_t *v_opos, uint16_t *v_oval, int64_t out_cap, int64_t *out_counts,
                      uint16_t *k_recon, uint16_t *v_recon, void *workspace, int64_t workspace_bytes,
                      void *stream) {
  NuqPlan p;
  int rc = nuq_plan(BH, S, D, bits, start_pos, n_sink, frac, fit_keys, p);
  if (rc) return rc;
  if (workspace && workspace_bytes < p.total)
    return fail(KVQ_ERR_CAPACITY, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                (long long)p.total);
  return nuq_call(keys, values, BH, S, D, start_pos, bits, frac, lloyd_iters, n_sink, fit_keys, key_levels,
                  key_thresh, value_levels, k_codes, v_codes, k_opos, k_oval, v_opos, v_oval, out_cap, out_counts,
                  k_recon, v_recon, p, workspace, true, stream, "kvq_nuq_fit_quant launch");
}

int kvq_nuq_fit_quant_noalloc(const uint16_t *keys, const uint16_t *values, int32_t BH, int32_t S, int32_t D,
                              int32_t start_pos, int32_t bits, double frac, int32_t lloyd_iters, int32_t n_sink,
                              int32_t fit_keys, float *key_levels, uint16_t *key_thresh, float *value_levels,
                              uint8_t *k_codes, uint8_t *v_codes, int32_t *k_opos, uint16_t *k_oval,
                              int32_t *v_opos, uint16_t *v_oval, int64_t out_cap, int64_t *out_counts,
                              uint16_t *k_recon, uint16_t *v_recon, void *stream) {
  NuqPlan p;
  int rc = nuq_plan(BH, S, D, bits, start_pos, n_sink, frac, fit_keys, p);
  if (rc) return rc;
  if (p.total > (int64_t)KVQ_NUQ_NOALLOC_WORKSPACE_BYTES)
    return fail(KVQ_ERR_CAPACITY,
                "this call needs %lld bytes of workspace, above the %lld bytes of the built-in one "
                "(use kvq_nuq_fit_quant with a workspace)",
                (long long)p.total, (long long)KVQ_NUQ_NOALLOC_WORKSPACE_BYTES);
  if (lloyd_iters < 0 || lloyd_iters > 1000) return fail(KVQ_ERR_ARG, "lloyd_iters must be in [0, 1000]");
  if (!keys || !values || !key_levels || !key_thresh || !value_levels || !k_codes || !v_codes || !k_opos ||
      !k_oval || !v_opos || !v_oval || !out_counts)
    return fail(KVQ_ERR_NULL, "a required NUQ pointer is NULL");
  void *ws = nullptr;
  if ((rc = scratch_on_current_device(&ws)) != KVQ_OK) return rc;
  return nuq_call(keys, values, BH, S, D, start_pos, bits, frac, lloyd_iters, n_sink, fit_keys, key_levels,
                  key_thresh, value_levels, k_codes, v_codes, k_opos, k_oval, v_opos, v_oval, out_cap, out_counts,
                  k_recon, v_recon, p, ws, false, stream, "kvq_nuq_fit_quant_noalloc launch");
}

}  // extern "C"
