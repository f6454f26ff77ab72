// Host check of the CPU oracle (oracle/msa_oracle.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer: every exported function on small seeded
// problems with ragged shapes (S_k not a multiple of the block, S_q < S_k,
// several groups and batches), one and several threads, plus the argument
// checks.  Expectations: the calls succeed, results are finite, each
// selection holds the query's local block, bf16-input and fp64-input entries
// agree, and bad arguments are rejected.  Exits 0 when all hold.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

extern "C" {
typedef struct oracle_dims {
  int64_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim, index_dim, block_size, topk;
  double softmax_scale;
} oracle_dims;
int oracle_block_scores(const oracle_dims*, const uint16_t*, const uint16_t*, const int64_t*, int64_t, double*, int);
int oracle_select(const oracle_dims*, const int64_t*, int64_t, const double*, int32_t*);
int oracle_attention(const oracle_dims*, const uint16_t*, const uint16_t*, const uint16_t*, const int64_t*, int64_t,
                     const int32_t*, double*, double*, int);
int oracle_attention_f64(const oracle_dims*, const double*, const double*, const double*, const int64_t*, int64_t,
                         const int32_t*, double*, double*, int);
int oracle_forward(const oracle_dims*, const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                   const uint16_t*, const int64_t*, int64_t, double*, int32_t*, double*, double*, int);
int oracle_kl_rows(const oracle_dims*, const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                   const int64_t*, int64_t, const int32_t*, double*, int);
int oracle_kl_rows_f64(const oracle_dims*, const double*, const double*, const double*, const double*,
                       const int64_t*, int64_t, const int32_t*, double*, int);
int oracle_attention_bwd(const oracle_dims*, const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                         const int64_t*, int64_t, const int32_t*, double*, double*, double*, int);
int oracle_attention_bwd_f64(const oracle_dims*, const double*, const double*, const double*, const double*,
                             const int64_t*, int64_t, const int32_t*, double*, double*, double*, int);
int oracle_kl_bwd(const oracle_dims*, const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                  const int64_t*, int64_t, const int32_t*, double*, double*, double*, int);
int oracle_kl_bwd_f64(const oracle_dims*, const double*, const double*, const double*, const double*,
                      const int64_t*, int64_t, const int32_t*, double*, double*, double*, int);
int oracle_default_threads(void);
}

namespace {

int failures = 0;
#define EXPECT(cond)                                                                       \
  do {                                                                                     \
    if (!(cond)) {                                                                         \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                                          \
    }                                                                                      \
  } while (0)

uint64_t state = 0x243F6A8885A308D3ull;
uint64_t next_u64() {  // xorshift64*: any seeded stream does for shapes this small
  state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
  return state * 0x2545F4914F6CDD1Dull;
}
// bf16 bits of a value on a coarse grid (exact in bf16): integers for index
// inputs, multiples of 1/8 in [-2, 2] for the main branch.
uint16_t bits_of(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}
double value_of(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

struct Case {
  oracle_dims d;
  std::vector<uint16_t> q, k, v, qi, ki, dout;
};

Case make_case(int64_t B, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv, int64_t D, int64_t Didx, int64_t bs,
               int64_t topk) {
  Case c;
  c.d = {B, Sq, Sk, Hq, Hkv, D, Didx, bs, topk, 0.0};
  auto fill = [](std::vector<uint16_t>& a, size_t n, bool integer) {
    a.resize(n);
    for (auto& x : a)
      x = bits_of(integer ? (float)((int)(next_u64() % 7) - 3) : (float)((int)(next_u64() % 33) - 16) / 8.f);
  };
  fill(c.q, B * Sq * Hq * D, false);
  fill(c.k, B * Sk * Hkv * D, false);
  fill(c.v, B * Sk * Hkv * D, false);
  fill(c.dout, B * Sq * Hq * D, false);
  fill(c.qi, B * Sq * Hkv * Didx, true);
  fill(c.ki, B * Sk * Didx, true);
  return c;
}

std::vector<double> widen(const std::vector<uint16_t>& a) {
  std::vector<double> out(a.size());
  for (size_t i = 0; i < a.size(); ++i) out[i] = value_of(a[i]);
  return out;
}

bool finite(const std::vector<double>& a) {
  for (double x : a)
    if (!std::isfinite(x)) return false;
  return true;
}

double max_diff(const std::vector<double>& a, const std::vector<double>& b) {
  double m = 0;
  for (size_t i = 0; i < a.size(); ++i) m = std::fmax(m, std::fabs(a[i] - b[i]));
  return m;
}

void run(const Case& c, int threads) {
  const oracle_dims& d = c.d;
  const int64_t G = d.heads_q / d.heads_kv, nb = (d.seqlen_k + d.block_size - 1) / d.block_size;
  std::vector<int64_t> rows;
  for (int64_t b = 0; b < d.batch; ++b)
    for (int64_t i = 0; i < d.seqlen_q; ++i)
      for (int64_t g = 0; g < d.heads_kv; ++g) rows.insert(rows.end(), {b, i, g});
  const int64_t n = (int64_t)rows.size() / 3;
  std::vector<double> bm(n * nb), out(n * G * d.head_dim), lse(n * G);
  std::vector<int32_t> sel(n * d.topk);
  EXPECT(oracle_forward(&d, c.q.data(), c.k.data(), c.v.data(), c.qi.data(), c.ki.data(), rows.data(), n,
                        bm.data(), sel.data(), out.data(), lse.data(), threads) == 0);
  EXPECT(finite(out) && finite(lse));
  for (int64_t r = 0; r < n; ++r) {
    const int64_t local = (rows[3 * r + 1] + d.seqlen_k - d.seqlen_q) / d.block_size;
    bool has = false;
    for (int64_t e = 0; e < d.topk; ++e) has |= sel[r * d.topk + e] == local;
    EXPECT(has);
  }
  // fp64 entries on the widened inputs give the same results
  const auto q = widen(c.q), k = widen(c.k), v = widen(c.v), qi = widen(c.qi), ki = widen(c.ki),
             dout = widen(c.dout);
  std::vector<double> out2(out.size()), lse2(lse.size());
  EXPECT(oracle_attention_f64(&d, q.data(), k.data(), v.data(), rows.data(), n, sel.data(), out2.data(),
                              lse2.data(), threads) == 0);
  EXPECT(max_diff(out, out2) < 1e-12 && max_diff(lse, lse2) < 1e-12);
  std::vector<double> kl(n), kl2(n);
  EXPECT(oracle_kl_rows(&d, c.q.data(), c.k.data(), c.qi.data(), c.ki.data(), rows.data(), n, sel.data(),
                        kl.data(), threads) == 0);
  EXPECT(oracle_kl_rows_f64(&d, q.data(), k.data(), qi.data(), ki.data(), rows.data(), n, sel.data(), kl2.data(),
                            threads) == 0);
  EXPECT(finite(kl) && max_diff(kl, kl2) < 1e-9);
  std::vector<double> dq(out.size()), dk(d.batch * d.seqlen_k * d.heads_kv * d.head_dim),
      dv(dk.size()), dq2(dq.size()), dk2(dk.size()), dv2(dk.size());
  EXPECT(oracle_attention_bwd(&d, c.q.data(), c.k.data(), c.v.data(), c.dout.data(), rows.data(), n, sel.data(),
                              dq.data(), dk.data(), dv.data(), threads) == 0);
  EXPECT(oracle_attention_bwd_f64(&d, q.data(), k.data(), v.data(), dout.data(), rows.data(), n, sel.data(),
                                  dq2.data(), dk2.data(), dv2.data(), threads) == 0);
  EXPECT(finite(dq) && finite(dk) && finite(dv));
  EXPECT(max_diff(dq, dq2) < 1e-9 && max_diff(dk, dk2) < 1e-9 && max_diff(dv, dv2) < 1e-9);
  std::vector<double> dqi(n * d.index_dim), dki(d.batch * d.seqlen_k * d.index_dim), lz(n), dqi2(dqi.size()),
      dki2(dki.size());
  EXPECT(oracle_kl_bwd(&d, c.q.data(), c.k.data(), c.qi.data(), c.ki.data(), rows.data(), n, sel.data(), dqi.data(),
                       dki.data(), lz.data(), threads) == 0);
  EXPECT(oracle_kl_bwd_f64(&d, q.data(), k.data(), qi.data(), ki.data(), rows.data(), n, sel.data(), dqi2.data(),
                           dki2.data(), nullptr, threads) == 0);
  EXPECT(finite(dqi) && finite(dki) && finite(lz) && max_diff(dqi, dqi2) < 1e-9 && max_diff(dki, dki2) < 1e-9);
  // the optional outputs may be null
  EXPECT(oracle_attention_bwd(&d, c.q.data(), c.k.data(), c.v.data(), c.dout.data(), rows.data(), n, sel.data(),
                              dq.data(), nullptr, nullptr, threads) == 0);
  EXPECT(oracle_forward(&d, c.q.data(), c.k.data(), c.v.data(), c.qi.data(), c.ki.data(), rows.data(), n, nullptr,
                        sel.data(), out.data(), lse.data(), threads) == 0);
  // block scores and selection on their own agree with the forward's
  std::vector<double> bm2(bm.size());
  std::vector<int32_t> sel2(sel.size());
  EXPECT(oracle_block_scores(&d, c.qi.data(), c.ki.data(), rows.data(), n, bm2.data(), threads) == 0);
  EXPECT(oracle_select(&d, rows.data(), n, bm2.data(), sel2.data()) == 0);
  EXPECT(sel == sel2);
}

void run_rejections(const Case& c) {
  const oracle_dims& d = c.d;
  int64_t bad_rows[3] = {0, d.seqlen_q, 0};  // query past S_q
  double bm[4096];
  int32_t sel[64];
  double out[4096], lse[64];
  EXPECT(oracle_block_scores(&d, c.qi.data(), c.ki.data(), bad_rows, 1, bm, 1) == -1);
  EXPECT(oracle_block_scores(&d, nullptr, c.ki.data(), bad_rows, 1, bm, 1) == -1);
  int64_t row[3] = {0, 0, 0};
  for (int64_t e = 0; e < d.topk; ++e) sel[e] = -1;  // no local block: rejected
  EXPECT(oracle_attention(&d, c.q.data(), c.k.data(), c.v.data(), row, 1, sel, out, lse, 1) == -1);
  EXPECT(oracle_forward(&d, c.q.data(), c.k.data(), c.v.data(), c.qi.data(), c.ki.data(), row, -1, nullptr, sel,
                        out, lse, 1) == -1);
}

}  // namespace

int main() {
  const Case cases[] = {make_case(2, 40, 300, 4, 2, 16, 8, 32, 3),  // ragged S_k, S_q < S_k, G = 2
                        make_case(1, 70, 70, 8, 1, 8, 4, 16, 4),     // G = 8, every query a prefix
                        make_case(3, 1, 500, 2, 2, 8, 8, 64, 5),     // decode-shaped, G = 1
                        make_case(1, 33, 200, 4, 4, 8, 16, 8, 40)};  // topk beyond the blocks
  for (const Case& c : cases) {
    run(c, 1);
    run(c, 4);
    run_rejections(c);
  }
  EXPECT(oracle_default_threads() >= 1);
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("oracle host check ok\n");
  return 0;
}
