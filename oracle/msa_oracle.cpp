// Plain, slow CPU oracle of the MSA forward path.  TEST INFRASTRUCTURE ONLY:
// only the tests, the package smoke check and the benchmark's CPU-baseline leg
// may load it.  It shares no code, header, table or helper with the device
// library.
//
// It restates the method from its description, one step at a time, in fp64:
//
//   Sparse Attention Part II (mtreviso.github.io), section 3.2 "MiniMax's MSA":
//     for each query and group, the index query is dotted with the single
//     index key that all groups share, over causally visible keys; a block's
//     score is the largest token score inside it; Top-k keeps 16 blocks of 128
//     tokens per group, the block holding the query always among them and the
//     other 15 picked by score; each query head of the group then runs its own
//     attention over the causally visible tokens of those blocks.
//   Same page, section 2: sparse-trained models normalise the softmax inside
//     the selection; exactness means reproducing that operator.
//   Same page, section 4.1: P = softmax(Q K^T / sqrt(d)), O = P V.
//   Same page, section 4.2: an exact top-k must break equal scores one fixed way
//     (here: higher score first, then lower block index).
//   MiniMax Sparse Attention (api.staik.se blog): the Top-k selects on raw
//     scores (exp-free), per GQA group.
//   Sparse Attention Part II, section 3.2, alignment loss: on the tokens of a
//     row's selected blocks, KL(teacher || student) with the teacher the mean
//     of the group's per-head attention probabilities (each head normalised
//     over those tokens) and the student the softmax of the index token
//     scores there; the loss averages the term over N * H_kv rows.
//
// Readings where the pages are silent (each also listed in the design notes):
//   - index score = raw dot product (no scale, no activation);
//   - queries are the last S_q positions: t_i = i + S_k - S_q;
//   - the local block does not compete: k-1 blocks are ranked among strictly
//     earlier blocks; with fewer than k-1 earlier blocks all of them are kept;
//   - the selection is emitted in ascending block order, padded with -1;
//   - query head h uses KV head / group floor(h / (H_q / H_kv)).
//
// Inputs are bf16 bit patterns (uint16), widened exactly to fp64.  Index
// scores accumulate in fp64, which is exact for integer-valued inputs.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

struct Dims {
  int64_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim, index_dim,
      block_size, topk;
  double softmax_scale;  // 0 => 1/sqrt(head_dim)
};

double widen_bf16(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  std::memcpy(&f, &w, sizeof f);
  return (double)f;
}

int64_t n_blocks(const Dims& d) {
  return (d.seqlen_k + d.block_size - 1) / d.block_size;
}

// Absolute position of query i (bottom-right causal alignment).
int64_t position(const Dims& d, int64_t i) { return i + d.seqlen_k - d.seqlen_q; }

bool dims_ok(const Dims* d) {
  return d && d->batch > 0 && d->seqlen_q > 0 && d->seqlen_k >= d->seqlen_q &&
         d->heads_kv > 0 && d->heads_q > 0 && d->heads_q % d->heads_kv == 0 &&
         d->head_dim > 0 && d->index_dim > 0 && d->block_size > 0 && d->topk > 0;
}

bool row_ok(const Dims& d, const int64_t* r) {
  return r[0] >= 0 && r[0] < d.batch && r[1] >= 0 && r[1] < d.seqlen_q &&
         r[2] >= 0 && r[2] < d.heads_kv;
}

// Runs fn(row) for every row on `threads` worker threads (0: all cores).
template <class Fn>
void for_rows(int64_t n_rows, int threads, Fn fn) {
  int t = threads > 0 ? threads : (int)std::thread::hardware_concurrency();
  if (t < 1) t = 1;
  if (t > n_rows) t = (int)std::max<int64_t>(n_rows, 1);
  std::vector<std::thread> pool;
  for (int w = 0; w < t; ++w)
    pool.emplace_back([=, &fn] {
      for (int64_t r = w; r < n_rows; r += t) fn(r);
    });
  for (auto& th : pool) th.join();
}

// Step 1-3: token index scores of query (b, i) for group g against every
// visible key, max-pooled per block; -inf for blocks with no visible key.
void block_scores_row(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx,
                      int64_t b, int64_t i, int64_t g, double* bm) {
  const int64_t nb = n_blocks(d);
  const int64_t t = position(d, i);
  const double neg_inf = -std::numeric_limits<double>::infinity();
  std::vector<double> q(d.index_dim);
  const uint16_t* qrow =
      q_idx + ((b * d.seqlen_q + i) * d.heads_kv + g) * d.index_dim;
  for (int64_t c = 0; c < d.index_dim; ++c) q[c] = widen_bf16(qrow[c]);
  for (int64_t j = 0; j < nb; ++j) bm[j] = neg_inf;
  for (int64_t s = 0; s <= t; ++s) {
    const uint16_t* krow = k_idx + (b * d.seqlen_k + s) * d.index_dim;
    double z = 0.0;
    for (int64_t c = 0; c < d.index_dim; ++c) z += q[c] * widen_bf16(krow[c]);
    int64_t j = s / d.block_size;
    if (z > bm[j]) bm[j] = z;
  }
}

// Step 4: the local block plus the best k-1 earlier blocks, ascending, -1 pad.
void select_row(const Dims& d, int64_t i, const double* bm, int32_t* sel) {
  const int64_t local = position(d, i) / d.block_size;
  std::vector<int64_t> cand(local);
  for (int64_t j = 0; j < local; ++j) cand[j] = j;
  const int64_t keep = std::min<int64_t>(d.topk - 1, local);
  std::sort(cand.begin(), cand.end(), [bm](int64_t a, int64_t b) {
    if (bm[a] != bm[b]) return bm[a] > bm[b];
    return a < b;
  });
  std::vector<int64_t> chosen(cand.begin(), cand.begin() + keep);
  chosen.push_back(local);
  std::sort(chosen.begin(), chosen.end());
  for (int64_t e = 0; e < d.topk; ++e)
    sel[e] = e < (int64_t)chosen.size() ? (int32_t)chosen[e] : -1;
}

// Step 5: every head of group g attends to the visible tokens of the selected
// blocks; softmax normalised over that set; fp64 throughout.
void attention_row(const Dims& d, const uint16_t* q, const uint16_t* k,
                   const uint16_t* v, int64_t b, int64_t i, int64_t g,
                   const int32_t* sel, double* out, double* lse) {
  const int64_t G = d.heads_q / d.heads_kv;
  const int64_t D = d.head_dim;
  const int64_t t = position(d, i);
  const double scale =
      d.softmax_scale != 0.0 ? d.softmax_scale : 1.0 / std::sqrt((double)D);
  std::vector<int64_t> tokens;
  for (int64_t e = 0; e < d.topk; ++e) {
    if (sel[e] < 0) continue;
    for (int64_t s = (int64_t)sel[e] * d.block_size;
         s < ((int64_t)sel[e] + 1) * d.block_size && s <= t; ++s)
      tokens.push_back(s);
  }
  std::vector<double> a(tokens.size());
  for (int64_t hh = 0; hh < G; ++hh) {
    const int64_t h = g * G + hh;
    const uint16_t* qrow = q + ((b * d.seqlen_q + i) * d.heads_q + h) * D;
    double m = -std::numeric_limits<double>::infinity();
    for (size_t n = 0; n < tokens.size(); ++n) {
      const uint16_t* krow = k + ((b * d.seqlen_k + tokens[n]) * d.heads_kv + g) * D;
      double dot = 0.0;
      for (int64_t c = 0; c < D; ++c) dot += widen_bf16(qrow[c]) * widen_bf16(krow[c]);
      a[n] = dot * scale;
      m = std::max(m, a[n]);
    }
    double sum = 0.0;
    double* o = out + hh * D;
    for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
    for (size_t n = 0; n < tokens.size(); ++n) {
      const double w = std::exp(a[n] - m);
      sum += w;
      const uint16_t* vrow = v + ((b * d.seqlen_k + tokens[n]) * d.heads_kv + g) * D;
      for (int64_t c = 0; c < D; ++c) o[c] += w * widen_bf16(vrow[c]);
    }
    for (int64_t c = 0; c < D; ++c) o[c] /= sum;
    lse[hh] = m + std::log(sum);
  }
}

// Auxiliary loss of the index branch, forward value, for one (query, group)
// row (Sparse Attention Part II, section 3.2): on the row's token set T (the
// visible tokens of its selected blocks), the teacher P averages the group's
// per-head attention probabilities, each head normalised over T; the student
// P_idx is the softmax over T of the index token scores; the row's term is
// KL(P || P_idx) = sum over T of P ln(P / P_idx).  Index scores enter the
// softmax as raw dot products (the pages give them no scale; a reading).
double kl_row(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* q_idx,
              const uint16_t* k_idx, int64_t b, int64_t i, int64_t g, const int32_t* sel) {
  const int64_t G = d.heads_q / d.heads_kv;
  const int64_t D = d.head_dim;
  const int64_t t = position(d, i);
  const double scale =
      d.softmax_scale != 0.0 ? d.softmax_scale : 1.0 / std::sqrt((double)D);
  std::vector<int64_t> tokens;
  for (int64_t e = 0; e < d.topk; ++e) {
    if (sel[e] < 0) continue;
    for (int64_t s = (int64_t)sel[e] * d.block_size;
         s < ((int64_t)sel[e] + 1) * d.block_size && s <= t; ++s)
      tokens.push_back(s);
  }
  const size_t n = tokens.size();
  // Teacher: mean over the group's heads of each head's softmax over T.
  std::vector<double> teacher(n, 0.0), a(n);
  for (int64_t hh = 0; hh < G; ++hh) {
    const uint16_t* qrow = q + ((b * d.seqlen_q + i) * d.heads_q + g * G + hh) * D;
    double m = -std::numeric_limits<double>::infinity();
    for (size_t x = 0; x < n; ++x) {
      const uint16_t* krow = k + ((b * d.seqlen_k + tokens[x]) * d.heads_kv + g) * D;
      double dot = 0.0;
      for (int64_t c = 0; c < D; ++c) dot += widen_bf16(qrow[c]) * widen_bf16(krow[c]);
      a[x] = dot * scale;
      m = std::max(m, a[x]);
    }
    double sum = 0.0;
    for (size_t x = 0; x < n; ++x) sum += std::exp(a[x] - m);
    for (size_t x = 0; x < n; ++x) teacher[x] += std::exp(a[x] - m) / sum / (double)G;
  }
  // Student: softmax over T of the raw index scores.
  std::vector<double> z(n);
  const uint16_t* qi = q_idx + ((b * d.seqlen_q + i) * d.heads_kv + g) * d.index_dim;
  double zm = -std::numeric_limits<double>::infinity();
  for (size_t x = 0; x < n; ++x) {
    const uint16_t* krow = k_idx + (b * d.seqlen_k + tokens[x]) * d.index_dim;
    double dot = 0.0;
    for (int64_t c = 0; c < d.index_dim; ++c) dot += widen_bf16(qi[c]) * widen_bf16(krow[c]);
    z[x] = dot;
    zm = std::max(zm, dot);
  }
  double zs = 0.0;
  for (size_t x = 0; x < n; ++x) zs += std::exp(z[x] - zm);
  const double log_zs = zm + std::log(zs);
  double kl = 0.0;
  for (size_t x = 0; x < n; ++x)
    if (teacher[x] > 0.0) kl += teacher[x] * (std::log(teacher[x]) - (z[x] - log_zs));
  return kl;
}

}  // namespace

extern "C" {

typedef struct oracle_dims {
  int64_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim, index_dim,
      block_size, topk;
  double softmax_scale;
} oracle_dims;

// Block scores for the listed rows.  rows: n_rows triples (b, i, g).
// bm: n_rows x n_blk doubles.  Returns 0, or -1 on a bad argument.
int oracle_block_scores(const oracle_dims* od, const uint16_t* q_idx,
                        const uint16_t* k_idx, const int64_t* rows,
                        int64_t n_rows, double* bm, int threads) {
  const Dims* d = reinterpret_cast<const Dims*>(od);
  if (!dims_ok(d) || !q_idx || !k_idx || !rows || !bm || n_rows < 0) return -1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (!row_ok(*d, rows + 3 * r)) return -1;
  const int64_t nb = n_blocks(*d);
  for_rows(n_rows, threads, [&](int64_t r) {
    const int64_t* rw = rows + 3 * r;
    block_scores_row(*d, q_idx, k_idx, rw[0], rw[1], rw[2], bm + r * nb);
  });
  return 0;
}

// Selection for the listed rows from their block scores (n_rows x n_blk).
// sel: n_rows x topk int32.
int oracle_select(const oracle_dims* od, const int64_t* rows, int64_t n_rows,
                  const double* bm, int32_t* sel) {
  const Dims* d = reinterpret_cast<const Dims*>(od);
  if (!dims_ok(d) || !rows || !bm || !sel || n_rows < 0) return -1;
  const int64_t nb = n_blocks(*d);
  for (int64_t r = 0; r < n_rows; ++r) {
    if (!row_ok(*d, rows + 3 * r)) return -1;
    select_row(*d, rows[3 * r + 1], bm + r * nb, sel + r * d->topk);
  }
  return 0;
}

// Main-branch attention of the listed rows over their selections.
// sel: n_rows x topk; out: n_rows x G x D doubles; lse: n_rows x G doubles.
int oracle_attention(const oracle_dims* od, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const int64_t* rows, int64_t n_rows,
                     const int32_t* sel, double* out, double* lse, int threads) {
  const Dims* d = reinterpret_cast<const Dims*>(od);
  if (!dims_ok(d) || !q || !k || !v || !rows || !sel || !out || !lse || n_rows < 0)
    return -1;
  const int64_t G = d->heads_q / d->heads_kv;
  const int64_t nb = n_blocks(*d);
  for (int64_t r = 0; r < n_rows; ++r) {
    if (!row_ok(*d, rows + 3 * r)) return -1;
    const int64_t local = position(*d, rows[3 * r + 1]) / d->block_size;
    bool has_local = false;
    for (int64_t e = 0; e < d->topk; ++e) {
      const int32_t j = sel[r * d->topk + e];
      if (j < -1 || j >= nb || j > local) return -1;
      has_local |= (j == local);
    }
    if (!has_local) return -1;  // the visible set would be empty
  }
  for_rows(n_rows, threads, [&](int64_t r) {
    const int64_t* rw = rows + 3 * r;
    attention_row(*d, q, k, v, rw[0], rw[1], rw[2], sel + r * d->topk,
                  out + r * G * d->head_dim, lse + r * G);
  });
  return 0;
}

// The three steps in order for the listed rows; bm may be NULL.
int oracle_forward(const oracle_dims* od, const uint16_t* q, const uint16_t* k,
                   const uint16_t* v, const uint16_t* q_idx,
                   const uint16_t* k_idx, const int64_t* rows, int64_t n_rows,
                   double* bm, int32_t* sel, double* out, double* lse,
                   int threads) {
  const Dims* d = reinterpret_cast<const Dims*>(od);
  if (!dims_ok(d) || n_rows < 0) return -1;
  std::vector<double> own;
  if (!bm) {
    own.resize((size_t)(n_rows * n_blocks(*d)));
    bm = own.data();
  }
  int rc = oracle_block_scores(od, q_idx, k_idx, rows, n_rows, bm, threads);
  if (rc) return rc;
  rc = oracle_select(od, rows, n_rows, bm, sel);
  if (rc) return rc;
  return oracle_attention(od, q, k, v, rows, n_rows, sel, out, lse, threads);
}

// KL-alignment loss terms of the listed rows over their selections (section
// 3.2); kl: n_rows doubles.  The loss is their mean over all N * H_kv rows.
int oracle_kl_rows(const oracle_dims* od, const uint16_t* q, const uint16_t* k,
                   const uint16_t* q_idx, const uint16_t* k_idx, const int64_t* rows,
                   int64_t n_rows, const int32_t* sel, double* kl, int threads) {
  const Dims* d = reinterpret_cast<const Dims*>(od);
  if (!dims_ok(d) || !q || !k || !q_idx || !k_idx || !rows || !sel || !kl || n_rows < 0)
    return -1;
  const int64_t nb = n_blocks(*d);
  for (int64_t r = 0; r < n_rows; ++r) {
    if (!row_ok(*d, rows + 3 * r)) return -1;
    const int64_t local = position(*d, rows[3 * r + 1]) / d->block_size;
    bool has_local = false;
    for (int64_t e = 0; e < d->topk; ++e) {
      const int32_t j = sel[r * d->topk + e];
      if (j < -1 || j >= nb || j > local) return -1;
      has_local |= (j == local);
    }
    if (!has_local) return -1;
  }
  for_rows(n_rows, threads, [&](int64_t r) {
    const int64_t* rw = rows + 3 * r;
    kl[r] = kl_row(*d, q, k, q_idx, k_idx, rw[0], rw[1], rw[2], sel + r * d->topk);
  });
  return 0;
}

// Threads the oracle uses when asked for "all cores".
int oracle_default_threads(void) {
  int t = (int)std::thread::hardware_concurrency();
  return t > 0 ? t : 1;
}

}  // extern "C"
