// h3_oracle_fp8.cpp — fp64 CPU oracle for the FP8 ("SAGE") variant of the attention.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or calls
// this code; only the tests, the smoke check and the benchmark's CPU baseline do.  It
// shares no source with the GPU path.
//
// Pages: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
// (Chinese translation of the vLLM blog post), §4.3 and its figure 6: SAGE quantization
// takes Q, K, P and V to FP8 for both attention products, and Skip-Softmax drops the
// softmax and P x V work of key tiles it judges unimportant, by a tile-level decision
// taken from the QK result; the draft pull request of the same post names the measured
// configuration "K16" without defining it.
//
// The method as this oracle computes it, every step in fp64 (the readings of what the
// pages leave open are marked):
//   - FP8 is E4M3 in its OCP "fn" form: bias 7, largest finite value 448, subnormals
//     down to 2^-9, no infinities; rounding to nearest, ties to even; values beyond 448
//     saturate to 448.  (reading: the format the pages' FP8 hardware uses)
//   - Q is quantized with one scale per token (row), K with one scale per block of 16
//     consecutive valid tokens ("K16"), V with one scale per channel over the N valid
//     tokens; each per head.  (reading)  A group's scale is amax / 448 and an element's
//     code is E4M3(x * 448 / amax): the group's largest element maps to +-448.
//   - scores s_ij = scale * sq_i * sk_block(j) * sum_c Qq_ic Kq_jc, the dot product of
//     the decoded codes (exact in fp64: each product has at most 8 significant bits).
//   - P.  Figure 6 places both the FP8 P and the Skip-Softmax decision inside an
//     attention that walks the keys tile by tile: each tile's weights exist only
//     against the row maximum known when that tile is reached.  So the valid keys are
//     taken in tiles of T consecutive keys (T = p_tile; the width is a parameter, the
//     pages give none), a running maximum m_t = max(m_(t-1), max over tile t of s_ij)
//     is kept, the tile's weights are P_ij = E4M3(256 * exp(s_ij - m_t)) (at most 256:
//     the largest power of two in E4M3's range, so the factor divides out exactly), and
//     the sums of earlier tiles are carried to the new maximum by exp(m_(t-1) - m_t).
//     A single tile (T >= N) gives P_ij = E4M3(256 exp(s_ij - max_j s_ij)).
//   - o_ic = sv_c * sum_j w_j P_ij Vq_jc / sum_j w_j P_ij with w_j = exp(m_t(j) - m_last):
//     the normaliser is the sum of the quantized weights, so each output is a weighted
//     mean of dequantized V (reading).  Rows in [N, S) are zero.
//   - Skip-Softmax with threshold lambda in [0, 1): tile t >= 1 is dropped for row i
//     when exp(max over the tile of s_ij - m_(t-1)) < lambda, m_(t-1) being the running
//     maximum before the tile; a dropped tile adds nothing and leaves the maximum as it
//     is.  lambda = 0 never drops a tile.  (reading: the pages give no threshold rule
//     beyond "a higher threshold skips more")
//   - optional `wmax`, one value per (row, head): the row's largest normalised weight
//     w_j P_ij / sum_j w_j P_ij, the quantity the FP8 comparison bar is stated in.
// Parity status: pinned by the closed forms in tests/test_oracle_fp8_pins.py.
#include "h3_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace {

double widen1(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

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

// One-scale group quantization: codes (as their E4M3 values) and the scale amax / 448.
void quantize(const double* x, int64_t n, double* codes, double* scale) {
  double amax = 0.0;
  for (int64_t i = 0; i < n; ++i) amax = std::max(amax, std::fabs(x[i]));
  if (!(amax > 0.0)) {
    for (int64_t i = 0; i < n; ++i) codes[i] = 0.0;
    *scale = 0.0;
    return;
  }
  for (int64_t i = 0; i < n; ++i) codes[i] = h3o_e4m3(x[i] * 448.0 / amax);
  *scale = amax / 448.0;
}

}  // namespace

extern "C" {

double h3o_e4m3(double x) {
  if (std::isnan(x)) return x;
  const double a = std::fabs(x);
  if (a >= 448.0) return std::copysign(448.0, x);
  // quantum: 2^(E-3) for normal values with exponent E >= -6, 2^-9 below
  double q;
  if (a < std::ldexp(1.0, -6)) {
    q = std::ldexp(1.0, -9);
  } else {
    int e;
    std::frexp(a, &e);  // a = f * 2^e, f in [0.5, 1)
    q = std::ldexp(1.0, (e - 1) - 3);
  }
  const double t = a / q;  // exact: q is a power of two
  double n = std::floor(t);
  const double frac = t - n;
  if (frac > 0.5 || (frac == 0.5 && std::fmod(n, 2.0) != 0.0)) n += 1.0;
  return std::copysign(n * q, x);
}

void h3o_quantize_group(const float* x, int64_t n, double* codes, double* scale) {
  std::vector<double> xd((size_t)std::max<int64_t>(n, 0));
  for (int64_t i = 0; i < n; ++i) xd[(size_t)i] = x[i];
  quantize(xd.data(), n, codes, scale);
}

uint16_t h3o_round_bf16(double x) {
  // nearest bf16 (8 significant bits), ties to even, computed from the double directly
  if (std::isnan(x)) return 0x7FC0;
  const double a = std::fabs(x);
  uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);                              // a = f * 2^e, f in [0.5, 1)
  const int ee = std::max(e - 1, -126);           // exponent of the leading bit (or subnormal)
  const double q = std::ldexp(1.0, ee - 7);       // quantum
  const double t = a / q;
  double n = std::floor(t);
  const double frac = t - n;
  if (frac > 0.5 || (frac == 0.5 && std::fmod(n, 2.0) != 0.0)) n += 1.0;
  const double r = n * q;
  if (r >= std::ldexp(1.0, 128)) return sign | 0x7F80;  // overflow to infinity
  const float f = (float)r;                       // exact: r has at most 8 significant bits
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

int h3o_attn_varlen_fp8(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        int64_t seq_buf, int64_t n_valid, int64_t heads, int64_t d,
                        int64_t row_stride, double scale, int64_t p_tile, double skip_threshold,
                        const int64_t* rows, int64_t n_rows, int threads, double* out,
                        double* wmax) {
  if (!q || !k || !v || !out || (n_rows > 0 && !rows)) return H3O_ERR_ARG;
  if (heads <= 0 || d <= 0 || n_valid < 0 || n_valid > seq_buf || p_tile < 1)
    return H3O_ERR_ARG;
  if (!(skip_threshold >= 0.0 && skip_threshold < 1.0)) return H3O_ERR_ARG;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= seq_buf) return H3O_ERR_ARG;
  const int64_t N = n_valid;
  // a tile is dropped when its maximum lies below the running maximum by more than this
  const double skip_log = skip_threshold > 0.0 ? std::log(skip_threshold) : -INFINITY;
  for (int64_t h = 0; h < heads; ++h) {
    // K: blocks of 16 valid tokens; V: per channel over the valid tokens
    std::vector<double> kq((size_t)(N * d)), ks((size_t)((N + 15) / 16));
    {
      std::vector<double> buf((size_t)(16 * d));
      for (int64_t b = 0; b * 16 < N; ++b) {
        const int64_t lo = b * 16, hi = std::min(N, lo + 16);
        for (int64_t j = lo; j < hi; ++j)
          for (int64_t c = 0; c < d; ++c)
            buf[(size_t)((j - lo) * d + c)] = widen1(k[j * row_stride + h * d + c]);
        quantize(buf.data(), (hi - lo) * d, kq.data() + lo * d, &ks[(size_t)b]);
      }
    }
    std::vector<double> vq((size_t)(N * d)), vs((size_t)d);
    {
      std::vector<double> col((size_t)N), cq((size_t)N);
      for (int64_t c = 0; c < d; ++c) {
        for (int64_t j = 0; j < N; ++j) col[(size_t)j] = widen1(v[j * row_stride + h * d + c]);
        quantize(col.data(), N, cq.data(), &vs[(size_t)c]);
        for (int64_t j = 0; j < N; ++j) vq[(size_t)(j * d + c)] = cq[(size_t)j];
      }
    }
    run_parallel(n_rows, threads, [&](int64_t lo, int64_t hi) {
      std::vector<double> qrow((size_t)d), qq((size_t)d), acc((size_t)d),
          s((size_t)std::max<int64_t>(N, 1));
      for (int64_t r = lo; r < hi; ++r) {
        double* o = out + (r * heads + h) * d;
        const int64_t i = rows[r];
        if (wmax) wmax[r * heads + h] = 0.0;
        if (i >= N || N == 0) {
          for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
          continue;
        }
        for (int64_t c = 0; c < d; ++c) qrow[(size_t)c] = widen1(q[i * row_stride + h * d + c]);
        double sq;
        quantize(qrow.data(), d, qq.data(), &sq);
        // scores of every valid key
        for (int64_t j = 0; j < N; ++j) {
          double dot = 0.0;
          for (int64_t c = 0; c < d; ++c) dot += qq[(size_t)c] * kq[(size_t)(j * d + c)];
          s[(size_t)j] = scale * sq * ks[(size_t)(j / 16)] * dot;
        }
        // key tiles: running maximum, weights quantized against it, sums carried over
        double m = -INFINITY, l = 0.0, pmax = 0.0;  // pmax: largest carried weight
        std::fill(acc.begin(), acc.end(), 0.0);
        for (int64_t t0 = 0; t0 < N; t0 += p_tile) {
          const int64_t t1 = std::min(N, t0 + p_tile);
          double tmax = -INFINITY;
          for (int64_t j = t0; j < t1; ++j) tmax = std::max(tmax, s[(size_t)j]);
          if (t0 > 0 && tmax - m < skip_log) continue;  // Skip-Softmax: tile dropped
          const double mt = std::max(m, tmax);
          const double carry = (m == -INFINITY) ? 0.0 : std::exp(m - mt);
          l *= carry;
          pmax *= carry;
          for (int64_t c = 0; c < d; ++c) acc[(size_t)c] *= carry;
          for (int64_t j = t0; j < t1; ++j) {
            const double p = h3o_e4m3(256.0 * std::exp(s[(size_t)j] - mt));
            l += p;
            pmax = std::max(pmax, p);
            for (int64_t c = 0; c < d; ++c) acc[(size_t)c] += p * vq[(size_t)(j * d + c)];
          }
          m = mt;
        }
        for (int64_t c = 0; c < d; ++c) o[c] = vs[(size_t)c] * acc[(size_t)c] / l;
        if (wmax) wmax[r * heads + h] = pmax / l;
      }
    });
  }
  return H3O_OK;
}

int h3o_attn_layer_fp8(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_buf,
                       int64_t n_valid, int64_t heads, int64_t d, int64_t row_stride,
                       const uint16_t* w_q, const uint16_t* w_k, int64_t w_head_stride,
                       double eps, const h3o_rope* rope, double scale, int64_t p_tile,
                       double skip_threshold, const int64_t* rows, int64_t n_rows, int threads,
                       double* out, double* wmax) {
  if (!q || !k || !v || !w_q || !w_k || !rope || !out) return H3O_ERR_ARG;
  if (heads <= 0 || d <= 0 || n_valid < 0 || n_valid > seq_buf) return H3O_ERR_ARG;
  // Normalised, rotated Q and K of every valid token, rounded to bf16 (the type the
  // fused operator hands to attention), then the FP8 attention on them.
  const int64_t N = n_valid, hd = heads * d;
  std::vector<uint16_t> qn((size_t)(seq_buf * hd), 0), kn((size_t)(seq_buf * hd), 0),
      vv((size_t)(seq_buf * hd), 0);
  std::vector<int64_t> all((size_t)N);
  for (int64_t i = 0; i < N; ++i) all[(size_t)i] = i;
  std::vector<double> tmp((size_t)(N * hd));
  for (int pass = 0; pass < 2; ++pass) {
    const uint16_t* x = pass ? k : q;
    const uint16_t* w = pass ? w_k : w_q;
    std::vector<uint16_t>& dst = pass ? kn : qn;
    const int rc = h3o_prologue(x, heads, d, row_stride, N, w, w_head_stride, eps, rope,
                                all.data(), N, threads, tmp.data());
    if (rc != H3O_OK) return rc;
    for (int64_t i = 0; i < N * hd; ++i) dst[(size_t)i] = h3o_round_bf16(tmp[(size_t)i]);
  }
  for (int64_t i = 0; i < N; ++i)
    for (int64_t c = 0; c < hd; ++c) vv[(size_t)(i * hd + c)] = v[i * row_stride + c];
  return h3o_attn_varlen_fp8(qn.data(), kn.data(), vv.data(), seq_buf, N, heads, d, hd, scale,
                             p_tile, skip_threshold, rows, n_rows, threads, out, wmax);
}

}  // extern "C"
