// h3_oracle_skip.cpp — fp64 CPU oracle for dense (unquantized) attention with
// Skip-Softmax, the "Skip-Softmax-only" control.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or calls
// this code; only the tests and the benchmark do.  It shares no source with the GPU path.
//
// Pages: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
// (Chinese translation of the vLLM blog post), §4.3 and figure 6: Skip-Softmax takes a
// tile-level decision from the QK result and bypasses the softmax and P x V work of the
// tiles it judges unimportant; a higher threshold skips more.  The blog's draft pull
// request keeps dense and Skip-Softmax-only (no FP8) controls beside the SAGE rows.
//
// What it computes, in fp64, for each valid query row i of each head (the readings of
// what the pages leave open are those of the FP8 oracle's Skip-Softmax):
//   - scores s_ij = scale * q_i . k_j over the valid keys j < N;
//   - the keys are walked in tiles of T consecutive keys (T = p_tile), keeping the
//     running maximum m of the kept tiles' scores; tile t >= 1 is dropped when
//     exp(max over the tile of s_ij - m) < lambda, m being the running maximum before
//     the tile; tile 0 is always kept; lambda = 0 drops nothing;
//   - o_i = sum over the kept keys of exp(s_ij - M) v_j / sum over the kept keys of
//     exp(s_ij - M), M the largest kept score (a plain softmax over the kept keys);
//   - wmax_i (optional) = the largest normalised weight of the row, 1 / that sum;
//   - rows in [N, S) are zero.
// The layer form normalises and rotates Q and K with the fp64 prologue of h3_oracle.cpp
// first (no bf16 rounding, as the dense oracle).
// Parity status: pinned by the closed forms in tests/test_oracle_skip_pins.py.
#include "h3_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <memory>
#include <thread>
#include <vector>

namespace {

template <class F>
void run_parallel(int64_t n, int threads, F fn) {
  if (threads < 1) threads = 1;
  if (threads == 1 || n < 2) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> pool;
  const int64_t per = (n + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    const int64_t lo = t * per, hi = std::min(n, lo + per);
    if (lo < hi) pool.emplace_back(fn, lo, hi);
  }
  for (auto& th : pool) th.join();
}

// q: [n_rows][heads][d] for the rows (row_valid[r] says whether row r is < N);
// k, v: [N][heads][d].  out: [n_rows][heads][d]; wmax: [n_rows][heads] or null.
void skip_attention(const double* q, const bool* row_valid, const double* k, const double* v,
                    int64_t n_rows, int64_t N, int64_t heads, int64_t d, double scale,
                    int64_t p_tile, double skip_threshold, int threads, double* out,
                    double* wmax) {
  const double skip_log = skip_threshold > 0.0 ? std::log(skip_threshold) : -INFINITY;
  run_parallel(n_rows * heads, threads, [&](int64_t lo, int64_t hi) {
    std::vector<double> s((size_t)std::max<int64_t>(N, 1));
    std::vector<char> kept((size_t)std::max<int64_t>(N, 1));
    for (int64_t rh = lo; rh < hi; ++rh) {
      const int64_t r = rh / heads, h = rh % heads;
      double* o = out + (r * heads + h) * d;
      if (wmax) wmax[r * heads + h] = 0.0;
      if (!row_valid[r] || N == 0) {
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        continue;
      }
      const double* qr = q + (r * heads + h) * d;
      for (int64_t j = 0; j < N; ++j) {
        const double* kj = k + (j * heads + h) * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qr[c] * kj[c];
        s[(size_t)j] = scale * dot;
      }
      // the tile walk: which tiles are kept
      double m = -INFINITY;
      for (int64_t t0 = 0; t0 < N; t0 += p_tile) {
        const int64_t t1 = std::min(N, t0 + p_tile);
        double tmax = -INFINITY;
        for (int64_t j = t0; j < t1; ++j) tmax = std::max(tmax, s[(size_t)j]);
        const bool keep = t0 == 0 || !(tmax - m < skip_log);
        for (int64_t j = t0; j < t1; ++j) kept[(size_t)j] = keep;
        if (keep) m = std::max(m, tmax);
      }
      // softmax over the kept keys (m is their largest score)
      double l = 0.0;
      for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
      for (int64_t j = 0; j < N; ++j) {
        if (!kept[(size_t)j]) continue;
        const double p = std::exp(s[(size_t)j] - m);
        l += p;
        const double* vj = v + (j * heads + h) * d;
        for (int64_t c = 0; c < d; ++c) o[c] += p * vj[c];
      }
      for (int64_t c = 0; c < d; ++c) o[c] /= l;
      if (wmax) wmax[r * heads + h] = 1.0 / l;
    }
  });
}

double widen1(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

bool args_ok(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_buf,
             int64_t n_valid, int64_t heads, int64_t d, int64_t p_tile, double skip_threshold,
             const int64_t* rows, int64_t n_rows, const double* out) {
  if (!q || !k || !v || !out || (n_rows > 0 && !rows)) return false;
  if (heads <= 0 || d <= 0 || n_valid < 0 || n_valid > seq_buf || p_tile < 1) return false;
  if (!(skip_threshold >= 0.0 && skip_threshold < 1.0)) return false;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= seq_buf) return false;
  return true;
}

}  // namespace

extern "C" {

int h3o_attn_varlen_skip(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         int64_t seq_buf, int64_t n_valid, int64_t heads, int64_t d,
                         int64_t row_stride, double scale, int64_t p_tile,
                         double skip_threshold, const int64_t* rows, int64_t n_rows,
                         int threads, double* out, double* wmax) {
  if (!args_ok(q, k, v, seq_buf, n_valid, heads, d, p_tile, skip_threshold, rows, n_rows, out))
    return H3O_ERR_ARG;
  const int64_t N = n_valid, hd = heads * d;
  std::vector<double> qq((size_t)(n_rows * hd)), kk((size_t)(N * hd)), vv((size_t)(N * hd));
  std::vector<char> valid((size_t)std::max<int64_t>(n_rows, 1));
  for (int64_t r = 0; r < n_rows; ++r) {
    valid[(size_t)r] = rows[r] < N;
    if (rows[r] < N)
      for (int64_t c = 0; c < hd; ++c) qq[(size_t)(r * hd + c)] = widen1(q[rows[r] * row_stride + c]);
  }
  for (int64_t j = 0; j < N; ++j)
    for (int64_t c = 0; c < hd; ++c) {
      kk[(size_t)(j * hd + c)] = widen1(k[j * row_stride + c]);
      vv[(size_t)(j * hd + c)] = widen1(v[j * row_stride + c]);
    }
  std::unique_ptr<bool[]> vbits(new bool[(size_t)std::max<int64_t>(n_rows, 1)]);
  for (int64_t r = 0; r < n_rows; ++r) vbits[(size_t)r] = valid[(size_t)r] != 0;
  skip_attention(qq.data(), vbits.get(), kk.data(), vv.data(), n_rows, N, heads, d, scale,
                 p_tile, skip_threshold, threads, out, wmax);
  return H3O_OK;
}

int h3o_attn_layer_skip(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        int64_t seq_buf, int64_t n_valid, int64_t heads, int64_t d,
                        int64_t row_stride, const uint16_t* w_q, const uint16_t* w_k,
                        int64_t w_head_stride, double eps, const h3o_rope* rope, double scale,
                        int64_t p_tile, double skip_threshold, const int64_t* rows,
                        int64_t n_rows, int threads, double* out, double* wmax) {
  if (!args_ok(q, k, v, seq_buf, n_valid, heads, d, p_tile, skip_threshold, rows, n_rows, out) ||
      !w_q || !w_k || !rope)
    return H3O_ERR_ARG;
  const int64_t N = n_valid, hd = heads * d;
  // normalised, rotated Q of the valid requested rows and K of every valid row (fp64)
  std::vector<int64_t> qrows, all((size_t)N);
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < N) qrows.push_back(rows[r]);
  for (int64_t j = 0; j < N; ++j) all[(size_t)j] = j;
  std::vector<double> qn((size_t)(qrows.size() * hd)), kk((size_t)(N * hd)), vv((size_t)(N * hd));
  int rc = h3o_prologue(q, heads, d, row_stride, N, w_q, w_head_stride, eps, rope, qrows.data(),
                        (int64_t)qrows.size(), threads, qn.data());
  if (rc != H3O_OK) return rc;
  rc = h3o_prologue(k, heads, d, row_stride, N, w_k, w_head_stride, eps, rope, all.data(), N,
                    threads, kk.data());
  if (rc != H3O_OK) return rc;
  for (int64_t j = 0; j < N; ++j)
    for (int64_t c = 0; c < hd; ++c) vv[(size_t)(j * hd + c)] = widen1(v[j * row_stride + c]);
  std::vector<double> qq((size_t)(n_rows * hd), 0.0);
  std::unique_ptr<bool[]> vbits(new bool[(size_t)std::max<int64_t>(n_rows, 1)]);
  for (int64_t r = 0, i = 0; r < n_rows; ++r) {
    vbits[(size_t)r] = rows[r] < N;
    if (rows[r] < N) {
      std::memcpy(&qq[(size_t)(r * hd)], &qn[(size_t)(i * hd)], sizeof(double) * hd);
      ++i;
    }
  }
  skip_attention(qq.data(), vbits.get(), kk.data(), vv.data(), n_rows, N, heads, d, scale,
                 p_tile, skip_threshold, threads, out, wmax);
  return H3O_OK;
}

}  // extern "C"
