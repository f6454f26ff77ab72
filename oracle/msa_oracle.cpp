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
//   Gradients (the backward the MSA kernel notes describe): the selection is
//     a discrete choice with no gradient; inside it the main branch is a
//     softmax attention over the selected visible tokens, differentiated the
//     usual way; the alignment term reaches only the index inputs (its
//     teacher is detached, section 3.2), with d KL / d z = Pidx - P.
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

// Inputs arrive as bf16 bit patterns or, for the finite-difference checks of
// the gradients, as fp64 values; every formula below reads them through val().
inline double val(const uint16_t* p, int64_t i) { return widen_bf16(p[i]); }
inline double val(const double* p, int64_t i) { return p[i]; }

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

// T: the visible tokens of the selected blocks of query i, ascending within
// each block, blocks in selection order.
std::vector<int64_t> token_set(const Dims& d, int64_t i, const int32_t* sel) {
  const int64_t t = position(d, i);
  std::vector<int64_t> tokens;
  for (int64_t e = 0; e < d.topk; ++e) {
    if (sel[e] < 0) continue;
    for (int64_t s = (int64_t)sel[e] * d.block_size;
         s < ((int64_t)sel[e] + 1) * d.block_size && s <= t; ++s)
      tokens.push_back(s);
  }
  return tokens;
}

double scale_of(const Dims& d) {
  return d.softmax_scale != 0.0 ? d.softmax_scale : 1.0 / std::sqrt((double)d.head_dim);
}

// Step 5: every head of group g attends to the visible tokens of the selected
// blocks; softmax normalised over that set; fp64 throughout.
template <class T>
void attention_row(const Dims& d, const T* q, const T* k, const T* v, int64_t b, int64_t i,
                   int64_t g, const int32_t* sel, double* out, double* lse) {
  const int64_t G = d.heads_q / d.heads_kv;
  const int64_t D = d.head_dim;
  const double scale = scale_of(d);
  const std::vector<int64_t> tokens = token_set(d, i, sel);
  std::vector<double> a(tokens.size());
  for (int64_t hh = 0; hh < G; ++hh) {
    const int64_t h = g * G + hh;
    const int64_t qrow = ((b * d.seqlen_q + i) * d.heads_q + h) * D;
    double m = -std::numeric_limits<double>::infinity();
    for (size_t n = 0; n < tokens.size(); ++n) {
      const int64_t krow = ((b * d.seqlen_k + tokens[n]) * d.heads_kv + g) * D;
      double dot = 0.0;
      for (int64_t c = 0; c < D; ++c) dot += val(q, qrow + c) * val(k, krow + c);
      a[n] = dot * scale;
      m = std::max(m, a[n]);
    }
    double sum = 0.0;
    double* o = out + hh * D;
    for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
    for (size_t n = 0; n < tokens.size(); ++n) {
      const double w = std::exp(a[n] - m);
      sum += w;
      const int64_t vrow = ((b * d.seqlen_k + tokens[n]) * d.heads_kv + g) * D;
      for (int64_t c = 0; c < D; ++c) o[c] += w * val(v, vrow + c);
    }
    for (int64_t c = 0; c < D; ++c) o[c] /= sum;
    lse[hh] = m + std::log(sum);
  }
}

// Gradient of the main branch for one (query, group) row, given the upstream
// gradient dO of its G output rows.  The selection is a discrete choice and
// carries no gradient; inside it the attention is an ordinary softmax
// attention over T (Sparse Attention Part II, section 2: the normalisation is
// over the selected set), so for each head, with P the softmax over T,
//   dV_s += P_s dO,  dP_s = dO . v_s,  dS_s = P_s (dP_s - sum_u P_u dP_u),
//   dq = scale sum_s dS_s k_s,  dK_s += scale dS_s q.
// sum_u P_u dP_u equals dO . O.  dq: G x D; dk, dv: [B][S_k][H_kv][D]
// accumulators (may be null).
template <class T>
void attention_bwd_row(const Dims& d, const T* q, const T* k, const T* v, const T* dout,
                       int64_t b, int64_t i, int64_t g, const int32_t* sel, double* dq,
                       double* dk, double* dv) {
  const int64_t G = d.heads_q / d.heads_kv;
  const int64_t D = d.head_dim;
  const double scale = scale_of(d);
  const std::vector<int64_t> tokens = token_set(d, i, sel);
  const size_t n = tokens.size();
  std::vector<double> p(n), dp(n);
  for (int64_t hh = 0; hh < G; ++hh) {
    const int64_t h = g * G + hh;
    const int64_t qrow = ((b * d.seqlen_q + i) * d.heads_q + h) * D;
    double m = -std::numeric_limits<double>::infinity();
    for (size_t x = 0; x < n; ++x) {
      const int64_t krow = ((b * d.seqlen_k + tokens[x]) * d.heads_kv + g) * D;
      double dot = 0.0;
      for (int64_t c = 0; c < D; ++c) dot += val(q, qrow + c) * val(k, krow + c);
      p[x] = dot * scale;
      m = std::max(m, p[x]);
    }
    double sum = 0.0;
    for (size_t x = 0; x < n; ++x) sum += (p[x] = std::exp(p[x] - m));
    double pdp = 0.0;  // sum_s P_s dP_s
    for (size_t x = 0; x < n; ++x) {
      p[x] /= sum;
      const int64_t vrow = ((b * d.seqlen_k + tokens[x]) * d.heads_kv + g) * D;
      double dot = 0.0;
      for (int64_t c = 0; c < D; ++c) dot += val(dout, qrow + c) * val(v, vrow + c);
      dp[x] = dot;
      pdp += p[x] * dot;
    }
    double* dqh = dq + hh * D;
    for (int64_t c = 0; c < D; ++c) dqh[c] = 0.0;
    for (size_t x = 0; x < n; ++x) {
      const double ds = p[x] * (dp[x] - pdp);
      const int64_t krow = ((b * d.seqlen_k + tokens[x]) * d.heads_kv + g) * D;
      for (int64_t c = 0; c < D; ++c) dqh[c] += scale * ds * val(k, krow + c);
      if (dk)
        for (int64_t c = 0; c < D; ++c) dk[krow + c] += scale * ds * val(q, qrow + c);
      if (dv)
        for (int64_t c = 0; c < D; ++c) dv[krow + c] += p[x] * val(dout, qrow + c);
    }
  }
}

// Auxiliary loss of the index branch, forward value, for one (query, group)
// row (Sparse Attention Part II, section 3.2): on the row's token set T (the
// visible tokens of its selected blocks), the teacher P averages the group's
// per-head attention probabilities, each head normalised over T; the student
// P_idx is the softmax over T of the index token scores; the row's term is
// KL(P || P_idx) = sum over T of P ln(P / P_idx).  Index scores enter the
// softmax as raw dot products (the pages give them no scale; a reading).
// Teacher and student of one row over its token set T: the mean over the
// group's heads of each head's softmax over T, and the raw index scores z
// with their log-sum-exp over T.
template <class T>
void kl_parts(const Dims& d, const T* q, const T* k, const T* q_idx, const T* k_idx, int64_t b,
              int64_t i, int64_t g, const std::vector<int64_t>& tokens,
              std::vector<double>& teacher, std::vector<double>& z, double& lse_z) {
  const int64_t G = d.heads_q / d.heads_kv;
  const int64_t D = d.head_dim;
  const double scale = scale_of(d);
  const size_t n = tokens.size();
  teacher.assign(n, 0.0);
  std::vector<double> a(n);
  for (int64_t hh = 0; hh < G; ++hh) {
    const int64_t qrow = ((b * d.seqlen_q + i) * d.heads_q + g * G + hh) * D;
    double m = -std::numeric_limits<double>::infinity();
    for (size_t x = 0; x < n; ++x) {
      const int64_t krow = ((b * d.seqlen_k + tokens[x]) * d.heads_kv + g) * D;
      double dot = 0.0;
      for (int64_t c = 0; c < D; ++c) dot += val(q, qrow + c) * val(k, krow + c);
      a[x] = dot * scale;
      m = std::max(m, a[x]);
    }
    double sum = 0.0;
    for (size_t x = 0; x < n; ++x) sum += std::exp(a[x] - m);
    for (size_t x = 0; x < n; ++x) teacher[x] += std::exp(a[x] - m) / sum / (double)G;
  }
  z.assign(n, 0.0);
  const int64_t qi = ((b * d.seqlen_q + i) * d.heads_kv + g) * d.index_dim;
  double zm = -std::numeric_limits<double>::infinity();
  for (size_t x = 0; x < n; ++x) {
    const int64_t krow = (b * d.seqlen_k + tokens[x]) * d.index_dim;
    double dot = 0.0;
    for (int64_t c = 0; c < d.index_dim; ++c) dot += val(q_idx, qi + c) * val(k_idx, krow + c);
    z[x] = dot;
    zm = std::max(zm, dot);
  }
  double zs = 0.0;
  for (size_t x = 0; x < n; ++x) zs += std::exp(z[x] - zm);
  lse_z = zm + std::log(zs);
}

template <class T>
double kl_row(const Dims& d, const T* q, const T* k, const T* q_idx, const T* k_idx, int64_t b,
              int64_t i, int64_t g, const int32_t* sel) {
  const std::vector<int64_t> tokens = token_set(d, i, sel);
  std::vector<double> teacher, z;
  double lse_z;
  kl_parts(d, q, k, q_idx, k_idx, b, i, g, tokens, teacher, z, lse_z);
  double kl = 0.0;
  for (size_t x = 0; x < tokens.size(); ++x)
    if (teacher[x] > 0.0) kl += teacher[x] * (std::log(teacher[x]) - (z[x] - lse_z));
  return kl;
}

// Gradient of one row's term with respect to the index inputs (the teacher
// is held fixed: section 3.2 detaches it).  d KL / d z_s = Pidx_s - P_s, so
//   dq_idx = sum_s (Pidx_s - P_s) k_idx_s,  dk_idx_s += (Pidx_s - P_s) q_idx.
// dq_idx: D_idx values; dk_idx: [B][S_k][D_idx] accumulator (may be null).
// Also returns the row's log-sum-exp of the index scores over T.
template <class T>
double kl_bwd_row(const Dims& d, const T* q, const T* k, const T* q_idx, const T* k_idx,
                  int64_t b, int64_t i, int64_t g, const int32_t* sel, double* dq_idx,
                  double* dk_idx) {
  const std::vector<int64_t> tokens = token_set(d, i, sel);
  std::vector<double> teacher, z;
  double lse_z;
  kl_parts(d, q, k, q_idx, k_idx, b, i, g, tokens, teacher, z, lse_z);
  const int64_t qi = ((b * d.seqlen_q + i) * d.heads_kv + g) * d.index_dim;
  for (int64_t c = 0; c < d.index_dim; ++c) dq_idx[c] = 0.0;
  for (size_t x = 0; x < tokens.size(); ++x) {
    const double gz = std::exp(z[x] - lse_z) - teacher[x];
    const int64_t krow = (b * d.seqlen_k + tokens[x]) * d.index_dim;
    for (int64_t c = 0; c < d.index_dim; ++c) dq_idx[c] += gz * val(k_idx, krow + c);
    if (dk_idx)
      for (int64_t c = 0; c < d.index_dim; ++c) dk_idx[krow + c] += gz * val(q_idx, qi + c);
  }
  return lse_z;
}

// Like for_rows, with the worker's index passed along: fn(row, worker).
template <class Fn>
int for_rows_w(int64_t n_rows, int threads, Fn fn) {
  int t = threads > 0 ? threads : (int)std::thread::hardware_concurrency();
  if (t < 1) t = 1;
  if (t > n_rows) t = (int)std::max<int64_t>(n_rows, 1);
  std::vector<std::thread> pool;
  for (int w = 0; w < t; ++w)
    pool.emplace_back([=, &fn] {
      for (int64_t r = w; r < n_rows; r += t) fn(r, w);
    });
  for (auto& th : pool) th.join();
  return t;
}

// Checks rows and selections the way the attention entry points do.
bool rows_and_sel_ok(const Dims& d, const int64_t* rows, int64_t n_rows, const int32_t* sel) {
  const int64_t nb = n_blocks(d);
  for (int64_t r = 0; r < n_rows; ++r) {
    if (!row_ok(d, rows + 3 * r)) return false;
    const int64_t local = position(d, rows[3 * r + 1]) / d.block_size;
    bool has_local = false;
    for (int64_t e = 0; e < d.topk; ++e) {
      const int32_t j = sel[r * d.topk + e];
      if (j < -1 || j >= nb || j > local) return false;
      has_local |= (j == local);
    }
    if (!has_local) return false;
  }
  return true;
}

// Runs a per-row gradient over the listed rows.  Full-size accumulators
// (acc_n doubles each, may be null) get one private copy per worker, summed
// in worker order at the end, so the result does not depend on scheduling.
template <class RowFn>
void rows_with_accumulators(int64_t n_rows, int threads, size_t acc_n, double* acc0, double* acc1,
                            RowFn fn) {
  int t = threads > 0 ? threads : (int)std::thread::hardware_concurrency();
  if (t < 1) t = 1;
  if (t > n_rows) t = (int)std::max<int64_t>(n_rows, 1);
  std::vector<std::vector<double>> a0(acc0 ? t : 0), a1(acc1 ? t : 0);
  for (auto& x : a0) x.assign(acc_n, 0.0);
  for (auto& x : a1) x.assign(acc_n, 0.0);
  for_rows_w(n_rows, t, [&](int64_t r, int w) {
    fn(r, acc0 ? a0[w].data() : nullptr, acc1 ? a1[w].data() : nullptr);
  });
  if (acc0) {
    std::fill(acc0, acc0 + acc_n, 0.0);
    for (auto& x : a0)
      for (size_t e = 0; e < acc_n; ++e) acc0[e] += x[e];
  }
  if (acc1) {
    std::fill(acc1, acc1 + acc_n, 0.0);
    for (auto& x : a1)
      for (size_t e = 0; e < acc_n; ++e) acc1[e] += x[e];
  }
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

}  // extern "C"

namespace {

template <class T>
int attention_rows(const oracle_dims* od, const T* q, const T* k, const T* v, const int64_t* rows,
                   int64_t n_rows, const int32_t* sel, double* out, double* lse, int threads) {
  const Dims* d = reinterpret_cast<const Dims*>(od);
  if (!dims_ok(d) || !q || !k || !v || !rows || !sel || !out || !lse || n_rows < 0)
    return -1;
  // Every selection must hold the local block: the visible set is then never empty.
  if (!rows_and_sel_ok(*d, rows, n_rows, sel)) return -1;
  const int64_t G = d->heads_q / d->heads_kv;
  for_rows(n_rows, threads, [&](int64_t r) {
    const int64_t* rw = rows + 3 * r;
    attention_row(*d, q, k, v, rw[0], rw[1], rw[2], sel + r * d->topk,
                  out + r * G * d->head_dim, lse + r * G);
  });
  return 0;
}

template <class T>
int attention_bwd_rows(const oracle_dims* od, const T* q, const T* k, const T* v, const T* dout,
                       const int64_t* rows, int64_t n_rows, const int32_t* sel, double* dq,
                       double* dk, double* dv, int threads) {
  const Dims* d = reinterpret_cast<const Dims*>(od);
  if (!dims_ok(d) || !q || !k || !v || !dout || !rows || !sel || !dq || n_rows < 0) return -1;
  if (!rows_and_sel_ok(*d, rows, n_rows, sel)) return -1;
  const int64_t G = d->heads_q / d->heads_kv;
  const size_t acc_n = (size_t)(d->batch * d->seqlen_k * d->heads_kv * d->head_dim);
  rows_with_accumulators(n_rows, threads, acc_n, dk, dv, [&](int64_t r, double* dkw, double* dvw) {
    const int64_t* rw = rows + 3 * r;
    attention_bwd_row(*d, q, k, v, dout, rw[0], rw[1], rw[2], sel + r * d->topk,
                      dq + r * G * d->head_dim, dkw, dvw);
  });
  return 0;
}

template <class T>
int kl_rows_impl(const oracle_dims* od, const T* q, const T* k, const T* q_idx, const T* k_idx,
                 const int64_t* rows, int64_t n_rows, const int32_t* sel, double* kl, int threads) {
  const Dims* d = reinterpret_cast<const Dims*>(od);
  if (!dims_ok(d) || !q || !k || !q_idx || !k_idx || !rows || !sel || !kl || n_rows < 0)
    return -1;
  if (!rows_and_sel_ok(*d, rows, n_rows, sel)) return -1;
  for_rows(n_rows, threads, [&](int64_t r) {
    const int64_t* rw = rows + 3 * r;
    kl[r] = kl_row(*d, q, k, q_idx, k_idx, rw[0], rw[1], rw[2], sel + r * d->topk);
  });
  return 0;
}

template <class T>
int kl_bwd_rows(const oracle_dims* od, const T* q, const T* k, const T* q_idx, const T* k_idx,
                const int64_t* rows, int64_t n_rows, const int32_t* sel, double* dq_idx,
                double* dk_idx, double* lse_z, int threads) {
  const Dims* d = reinterpret_cast<const Dims*>(od);
  if (!dims_ok(d) || !q || !k || !q_idx || !k_idx || !rows || !sel || !dq_idx || n_rows < 0)
    return -1;
  if (!rows_and_sel_ok(*d, rows, n_rows, sel)) return -1;
  const size_t acc_n = (size_t)(d->batch * d->seqlen_k * d->index_dim);
  rows_with_accumulators(n_rows, threads, acc_n, dk_idx, nullptr, [&](int64_t r, double* dkw, double*) {
    const int64_t* rw = rows + 3 * r;
    const double l = kl_bwd_row(*d, q, k, q_idx, k_idx, rw[0], rw[1], rw[2], sel + r * d->topk,
                                dq_idx + r * d->index_dim, dkw);
    if (lse_z) lse_z[r] = l;
  });
  return 0;
}

}  // namespace

extern "C" {

// Main-branch attention of the listed rows over their selections.
// sel: n_rows x topk; out: n_rows x G x D doubles; lse: n_rows x G doubles.
int oracle_attention(const oracle_dims* od, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const int64_t* rows, int64_t n_rows,
                     const int32_t* sel, double* out, double* lse, int threads) {
  return attention_rows(od, q, k, v, rows, n_rows, sel, out, lse, threads);
}

// The same on fp64 inputs (finite-difference checks of the gradients).
int oracle_attention_f64(const oracle_dims* od, const double* q, const double* k,
                         const double* v, const int64_t* rows, int64_t n_rows,
                         const int32_t* sel, double* out, double* lse, int threads) {
  return attention_rows(od, q, k, v, rows, n_rows, sel, out, lse, threads);
}

// Gradient of the main branch for the listed rows, given dO ([B][S_q][H_q][D],
// same layout as q).  dq: n_rows x G x D; dk, dv: [B][S_k][H_kv][D], summed
// over the listed rows (each may be null).
int oracle_attention_bwd(const oracle_dims* od, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const uint16_t* dout, const int64_t* rows,
                         int64_t n_rows, const int32_t* sel, double* dq, double* dk, double* dv,
                         int threads) {
  return attention_bwd_rows(od, q, k, v, dout, rows, n_rows, sel, dq, dk, dv, threads);
}

int oracle_attention_bwd_f64(const oracle_dims* od, const double* q, const double* k,
                             const double* v, const double* dout, const int64_t* rows,
                             int64_t n_rows, const int32_t* sel, double* dq, double* dk,
                             double* dv, int threads) {
  return attention_bwd_rows(od, q, k, v, dout, rows, n_rows, sel, dq, dk, dv, threads);
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
  return kl_rows_impl(od, q, k, q_idx, k_idx, rows, n_rows, sel, kl, threads);
}

int oracle_kl_rows_f64(const oracle_dims* od, const double* q, const double* k,
                       const double* q_idx, const double* k_idx, const int64_t* rows,
                       int64_t n_rows, const int32_t* sel, double* kl, int threads) {
  return kl_rows_impl(od, q, k, q_idx, k_idx, rows, n_rows, sel, kl, threads);
}

// Gradient of the listed rows' terms with respect to q_idx and k_idx (teacher
// held fixed).  dq_idx: n_rows x D_idx; dk_idx: [B][S_k][D_idx] summed over
// the listed rows (may be null); lse_z: n_rows log-sum-exps of the index
// scores over T (may be null).  Unscaled: the loss's 1/(N H_kv) is the
// caller's.
int oracle_kl_bwd(const oracle_dims* od, const uint16_t* q, const uint16_t* k,
                  const uint16_t* q_idx, const uint16_t* k_idx, const int64_t* rows,
                  int64_t n_rows, const int32_t* sel, double* dq_idx, double* dk_idx,
                  double* lse_z, int threads) {
  return kl_bwd_rows(od, q, k, q_idx, k_idx, rows, n_rows, sel, dq_idx, dk_idx, lse_z, threads);
}

int oracle_kl_bwd_f64(const oracle_dims* od, const double* q, const double* k,
                      const double* q_idx, const double* k_idx, const int64_t* rows,
                      int64_t n_rows, const int32_t* sel, double* dq_idx, double* dk_idx,
                      double* lse_z, int threads) {
  return kl_bwd_rows(od, q, k, q_idx, k_idx, rows, n_rows, sel, dq_idx, dk_idx, lse_z, threads);
}

// Threads the oracle uses when asked for "all cores".
int oracle_default_threads(void) {
  int t = (int)std::thread::hardware_concurrency();
  return t > 0 ? t : 1;
}

}  // extern "C"
