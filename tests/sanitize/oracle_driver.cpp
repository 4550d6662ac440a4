// Host sanitizer driver for the CPU oracle (test infrastructure).
//
// Built together with oracle/kvq_oracle.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer (every finding fatal) by tests/test_sanitizers.py,
// it runs the oracle's exported functions on small inputs that reach the
// edges: ragged group tails, single-element groups, sinks covering the whole
// call, empty key fits, zero outlier fractions, tiny and huge fp16 values,
// every width. A memory or undefined-behaviour error aborts the process; the
// driver itself only checks return codes.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
float orc_h2f(uint16_t h);
uint16_t orc_f2h(float f);
long long orc_packed_dim(int D, int bits);
long long orc_sym_cache_bytes(long long tokens, int layers, int kv_heads, int D, int bits);
int orc_sym_quant_rows(const uint16_t *x, long long n_rows, int D, int bits, uint8_t *codes, uint16_t *scales);
int orc_sym_dequant_rows(const uint8_t *codes, const uint16_t *scales, long long n_rows, int D, int bits,
                         uint16_t *out);
int orc_sym_quant_paged(const uint16_t *x, int n_tokens, int H, int D, int bits, const int32_t *slot_mapping,
                        long long n_slots, uint8_t *codes, uint16_t *scales);
int orc_sym_dequant_paged(const uint8_t *codes, const uint16_t *scales, int num_pages, int page_size, int H, int D,
                          int bits, const int32_t *block_table, int max_blocks, const int32_t *seq_lens, int n_seqs,
                          int max_len, uint16_t *out);
long long orc_kivi_boundary(long long offset, int residual_length, int group_size);
int orc_kivi_round_trip(uint16_t *x, int B, int H, int S_cap, int D, int lo, int hi, int per_channel, int bits,
                        int gs, float eps, uint8_t *codes, float *scale_out, float *min_out);
int orc_kivi_pack(const uint16_t *x, int B, int H, int S_cap, int D, int lo, int hi, int per_channel, int bits,
                  int gs, float eps, uint8_t *codes, uint16_t *scale, uint16_t *zero);
int orc_kivi_unpack(const uint8_t *codes, const uint16_t *scale, const uint16_t *zero, int B, int H, int S_cap, int D,
                    int lo, int hi, int per_channel, int bits, int gs, uint16_t *out);
void orc_nuq_fit(const uint16_t *u, int m, int L, int iters, float *lev);
uint16_t orc_nuq_threshold(const uint16_t *x, int n, double frac);
int orc_nuq_fit_quant(const uint16_t *keys, const uint16_t *values, int BH, int S, int D, int start_pos, int bits,
                      double frac, int iters, int n_sink, int fit_keys, float *key_levels, uint16_t *key_thresh,
                      float *value_levels, uint8_t *k_codes, uint8_t *v_codes, int32_t *k_opos, uint16_t *k_oval,
                      int32_t *v_opos, uint16_t *v_oval, long long out_cap, long long *out_counts,
                      uint16_t *k_recon, uint16_t *v_recon);
}

static int failures = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static std::mt19937 rng(12345);

static std::vector<uint16_t> fp16_data(size_t n, float scale) {
  std::normal_distribution<float> nd(0.0f, scale);
  std::vector<uint16_t> v(n);
  for (auto &x : v) x = orc_f2h(nd(rng));
  // a few extremes: subnormals, signed zeros, the largest finite values
  const uint16_t special[] = {0x0001, 0x8001, 0x0000, 0x8000, 0x7bff, 0xfbff, 0x03ff, 0x8400};
  for (size_t i = 0; i < n && i < 8 * 7; i += 7) v[i] = special[(i / 7) % 8];
  return v;
}

int main() {
  // fp16 conversions over every pattern
  for (uint32_t h = 0; h < 65536; ++h) {
    const float f = orc_h2f((uint16_t)h);
    if (f == f) (void)orc_f2h(f);
  }
  (void)orc_f2h(1e30f);
  (void)orc_f2h(-1e-30f);
  // symmetric rows, every width, every multiple-of-4 head dim up to 260
  for (int bits : {8, 6, 4}) {
    for (int D : {4, 8, 12, 64, 256, 260}) {
      const long long pd = orc_packed_dim(D, bits);
      CHECK(pd > 0);
      const int rows = 13;
      auto x = fp16_data((size_t)rows * D, 3.0f);
      std::vector<uint8_t> codes((size_t)rows * pd);
      std::vector<uint16_t> sc(rows), out((size_t)rows * D);
      CHECK(orc_sym_quant_rows(x.data(), rows, D, bits, codes.data(), sc.data()) == 0);
      CHECK(orc_sym_dequant_rows(codes.data(), sc.data(), rows, D, bits, out.data()) == 0);
      // paged: slots out of range and negative, sequences past their pages
      const int P = 4, pages = 5, T = 9, H = 1;
      std::vector<int32_t> slot = {0, 19, -1, 20, 3, 7, 100000, 2, 11};
      std::vector<uint8_t> pc((size_t)pages * P * H * pd);
      std::vector<uint16_t> ps((size_t)pages * P * H);
      CHECK(orc_sym_quant_paged(x.data(), T, H, D, bits, slot.data(), pages * P, pc.data(), ps.data()) == 0);
      std::vector<int32_t> bt = {0, 4, -3, 2, 9, 1};
      std::vector<int32_t> lens = {7, 12};
      std::vector<uint16_t> po((size_t)2 * 14 * H * D);
      CHECK(orc_sym_dequant_paged(pc.data(), ps.data(), pages, P, H, D, bits, bt.data(), 3, lens.data(), 2, 14,
                                  po.data()) == 0);
    }
  }
  CHECK(orc_packed_dim(6, 6) < 0 && orc_packed_dim(5, 4) < 0 && orc_packed_dim(8, 5) < 0);
  CHECK(orc_sym_cache_bytes(262144, 16, 4, 256, 6) == 6509559808LL);
  // KIVI: ragged tails on both axes, one-element groups, every width
  for (int bits : {2, 4, 8}) {
    for (int gs : {1, 3, 8, 32}) {
      for (int per_channel : {0, 1}) {
        const int B = 2, H = 1, S = 37, D = 24, lo = 5, hi = 36;
        auto x = fp16_data((size_t)B * H * S * D, 2.0f);
        const int n = hi - lo;
        const int cpr = (D * bits + 7) / 8;
        const int ngk = (n + gs - 1) / gs, ngv = (D + gs - 1) / gs;
        std::vector<uint8_t> codes((size_t)B * H * n * cpr);
        std::vector<float> s((size_t)B * H * (per_channel ? ngk * D : n * ngv)), m(s.size());
        CHECK(orc_kivi_round_trip(x.data(), B, H, S, D, lo, hi, per_channel, bits, gs, 1e-8f, codes.data(),
                                  s.data(), m.data()) == 0);
        if (gs % 8 == 0) {
          const int lo2 = per_channel ? gs : 5;  // key groups start at a multiple of gs
          std::vector<uint8_t> pc((size_t)B * H * S * D * bits / 8);
          const size_t np = (size_t)B * H * (per_channel ? ((S + gs - 1) / gs) * D : S * ngv);
          std::vector<uint16_t> ps(np), pz(np), out((size_t)B * H * S * D);
          CHECK(orc_kivi_pack(x.data(), B, H, S, D, lo2, hi, per_channel, bits, gs, 1e-8f, pc.data(), ps.data(),
                              pz.data()) == 0);
          CHECK(orc_kivi_unpack(pc.data(), ps.data(), pz.data(), B, H, S, D, lo2, hi, per_channel, bits, gs,
                                out.data()) == 0);
        }
      }
    }
  }
  for (long long off : {0LL, 1LL, 127LL, 128LL, 160LL, 1LL << 40}) (void)orc_kivi_boundary(off, 128, 32);
  // NUQ: fits over 0..9 samples, thresholds at several fractions, whole calls
  for (int m = 0; m < 10; ++m) {
    auto u = fp16_data((size_t)m + 1, 4.0f);
    for (int L : {2, 4, 8, 16}) {
      std::vector<float> lev(L);
      orc_nuq_fit(u.data(), m, L, 5, lev.data());
    }
    if (m > 0)
      for (double f : {0.0, 0.01, 0.5, 0.99}) (void)orc_nuq_threshold(u.data(), m, f);
  }
  for (int bits = 1; bits <= 4; ++bits) {
    for (int S : {1, 3, 4, 5, 40}) {
      for (int fit : {1, 0}) {
        const int BH = 2, D = 16, L = 1 << bits;
        const int cpr = D * bits / 8;
        auto k = fp16_data((size_t)BH * S * D, 3.0f);
        auto v = fp16_data((size_t)BH * S * D, 3.0f);
        std::vector<float> kl((size_t)BH * D * L, 0.5f), vl((size_t)BH * S * L);
        std::vector<uint16_t> kt((size_t)BH * D, 0x3c00);
        std::vector<uint8_t> kc((size_t)BH * S * cpr), vc(kc.size());
        const long long cap = (long long)BH * S * D;
        std::vector<int32_t> kp(cap), vp(cap);
        std::vector<uint16_t> kv(cap), vv(cap), kr((size_t)BH * S * D), vr(kr.size());
        long long counts[2];
        for (int sp : {0, 7})
          CHECK(orc_nuq_fit_quant(k.data(), v.data(), BH, S, D, sp, bits, 0.05, 8, 4, fit, kl.data(), kt.data(),
                                  vl.data(), kc.data(), vc.data(), kp.data(), kv.data(), vp.data(), vv.data(), cap,
                                  counts, kr.data(), vr.data()) == 0);
        // a capacity too small for the lists is refused, not overrun
        CHECK(orc_nuq_fit_quant(k.data(), v.data(), BH, S, D, 9, bits, 0.05, 8, 4, 0, kl.data(), kt.data(),
                                vl.data(), kc.data(), vc.data(), kp.data(), kv.data(), vp.data(), vv.data(), 0,
                                counts, kr.data(), vr.data()) != 0 ||
              counts[0] == 0);
      }
    }
  }
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("oracle driver ok\n");
  return 0;
}
