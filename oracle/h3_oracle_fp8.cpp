// h3_oracle_fp8.cpp — fp64 CPU oracle for the FP8 ("SAGE") variant of the attention.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or calls
// this code; only the tests, the smoke check and the benchmark's CPU baseline do.  It
// shares no source with the GPU path.
//
// Pages: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
// (Chinese translation of the vLLM blog post), §4.3 and its figure 6: SAGE quantization
// takes Q, K, P and V to FP8 for both attention products; the draft pull request of the
// same post names the measured configuration "K16" without defining it.
//
// The method as this oracle computes it (the readings of what the pages leave open):
//   - FP8 is E4M3 in its OCP "fn" form: bias 7, largest finite value 448, subnormals
//     down to 2^-9, no infinities; rounding to nearest, ties to even; values beyond 448
//     saturate to 448.
//   - Q is quantized with one scale per token (row), K with one scale per block of 16
//     consecutive valid tokens ("K16"), V with one scale per channel over the N valid
//     tokens; each per head.  A group's scale is amax / 448, so its largest element maps
//     to +-448.  The quantization decision is taken in fp32 (inverse scale 448 / amax,
//     one product, then rounding), the precision the kernel takes it in.
//   - scores s_ij = scale * sq_i * sk_block(j) * sum_c Qq_ic Kq_jc;
//   - P is produced the way a streaming (online-softmax) attention produces it: the
//     valid keys are taken in tiles of T consecutive keys (T = p_tile), a running row
//     maximum m_t = max(m_(t-1), max over tile t of s_ij) is kept, the weights of tile t
//     are P_ij = E4M3(256 * exp(s_ij - m_t)) (at most 256), and the sums of earlier
//     tiles are carried over by the factor exp(m_(t-1) - m_t).  When a row's maximum
//     lies in its first tile (or N <= T) this is P_ij = E4M3(256 exp(s_ij - max_j s_ij))
//     for every key;
//   - the P codes are quantization decisions, so their argument is formed in fp32, the
//     kernel's precision, in base 2: x_ij = fl(raw_ij * c_ib) with the raw score
//     raw_ij = fl(fl(dot over channels 0..63) + dot over channels 64..127) of the codes,
//     c_ib = fl(fl(scale * log2 e) * fl(amax_q / 448)) * fl(amax_kb / 448), the running
//     maximum m kept in fp32 in the same units, and P = E4M3(exp2f(fmaf(raw, c, 8 - m)));
//     the carries and all sums are fp64;
//   - optional `allow`: the FP8 product of the matrix cores accumulates its 64 terms with
//     less than fp32 precision (measured: errors up to 2^-11.2 of the largest term of a
//     single product), so a P code whose argument lies that close to an E4M3 rounding
//     midpoint may legitimately come out one step apart.  With a score error bound of
//     2^-9 times the row's largest |q_c k_c| term (two chained products, margin 2) for
//     the key and for the running maximum, every code that can change within that window
//     (and every tile whose Skip-Softmax decision can change) contributes its change,
//     carried to the row's final maximum, times |v - o| to a per-element allowance.
//   - o_ic = sv_c * sum_j w_j P_ij Vq_jc / sum_j w_j P_ij with w_j = exp(m_t(j) - m_last)
//     (the normaliser is the sum of the quantized weights); rows in [N, S) are zero.
//   - Skip-Softmax (same section: a tile-level decision taken from the QK result drops
//     the softmax and P V work of unimportant tiles; a higher threshold skips more):
//     with threshold lambda in [0, 1), tile t (t >= 1) is dropped for row i when
//     exp(max over the tile of s_ij - m_(t-1)) < lambda, m_(t-1) being the running
//     maximum before the tile; a dropped tile adds nothing and leaves the maximum as
//     it is.  lambda = 0 never drops a tile.  The decision is per query row, taken in
//     fp32 like the P codes: x_max < m + fl(log2 lambda).
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

// Quantize n fp32 values with one scale: codes (as their E4M3 values), the scale and
// (optionally) the fp32 amax.
void quantize(const float* x, int64_t n, double* codes, double* scale, float* amax_out = nullptr) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) amax = std::max(amax, std::fabs(x[i]));
  if (amax_out) *amax_out = amax;
  if (!(amax > 0.0f)) {
    for (int64_t i = 0; i < n; ++i) codes[i] = 0.0;
    *scale = 0.0;
    return;
  }
  const float inv = 448.0f / amax;
  for (int64_t i = 0; i < n; ++i) {
    float y = x[i] * inv;
    y = std::min(448.0f, std::max(-448.0f, y));
    codes[i] = h3o_e4m3(y);
  }
  *scale = (double)amax / 448.0;
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
  quantize(x, n, codes, scale);
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
                        double* allow) {
  if (!q || !k || !v || !out || (n_rows > 0 && !rows)) return H3O_ERR_ARG;
  if (heads <= 0 || d <= 0 || n_valid < 0 || n_valid > seq_buf || p_tile < 1)
    return H3O_ERR_ARG;
  if (!(skip_threshold >= 0.0 && skip_threshold < 1.0)) return H3O_ERR_ARG;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= seq_buf) return H3O_ERR_ARG;
  const int64_t N = n_valid;
  for (int64_t h = 0; h < heads; ++h) {
    // K: blocks of 16 valid tokens; V: per channel over the valid tokens
    std::vector<double> kq((size_t)(N * d)), ks((size_t)((N + 15) / 16));
    std::vector<float> ka((size_t)((N + 15) / 16));
    std::vector<float> buf((size_t)(16 * d));
    for (int64_t b = 0; b * 16 < N; ++b) {
      const int64_t lo = b * 16, hi = std::min(N, lo + 16);
      for (int64_t j = lo; j < hi; ++j)
        for (int64_t c = 0; c < d; ++c)
          buf[(size_t)((j - lo) * d + c)] = (float)widen1(k[j * row_stride + h * d + c]);
      quantize(buf.data(), (hi - lo) * d, kq.data() + lo * d, &ks[(size_t)b], &ka[(size_t)b]);
    }
    const float c_scale = (float)scale * 1.4426950408889634f;  // fl(scale * log2 e)
    const float skip_log2 = skip_threshold > 0.0 ? (float)std::log2(skip_threshold) : -INFINITY;
    std::vector<double> vq((size_t)(N * d)), vs((size_t)d);
    {
      std::vector<float> col((size_t)N);
      std::vector<double> cq((size_t)N);
      for (int64_t c = 0; c < d; ++c) {
        for (int64_t j = 0; j < N; ++j) col[(size_t)j] = (float)widen1(v[j * row_stride + h * d + c]);
        quantize(col.data(), N, cq.data(), &vs[(size_t)c]);
        for (int64_t j = 0; j < N; ++j) vq[(size_t)(j * d + c)] = cq[(size_t)j];
      }
    }
    run_parallel(n_rows, threads, [&](int64_t lo, int64_t hi) {
      std::vector<float> qrow((size_t)d), raw((size_t)std::max<int64_t>(N, 1)),
          cb((size_t)ka.size());
      std::vector<double> qq((size_t)d), acc((size_t)d), err((size_t)std::max<int64_t>(N, 1));
      struct Amb { int64_t j; double dp; float mt; };
      std::vector<Amb> amb;
      for (int64_t r = lo; r < hi; ++r) {
        double* o = out + (r * heads + h) * d;
        double* al = allow ? allow + (r * heads + h) * d : nullptr;
        const int64_t i = rows[r];
        if (al)
          for (int64_t c = 0; c < d; ++c) al[c] = 0.0;
        if (i >= N || N == 0) {
          for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
          continue;
        }
        for (int64_t c = 0; c < d; ++c) qrow[(size_t)c] = (float)widen1(q[i * row_stride + h * d + c]);
        double sq;
        float qa;
        quantize(qrow.data(), d, qq.data(), &sq, &qa);
        // multipliers of the raw scores in base 2, per 16-key block (fp32)
        const float c_row = c_scale * (qa / 448.0f);
        for (size_t b = 0; b < cb.size(); ++b) cb[b] = c_row * (ka[b] / 448.0f);
        // raw scores: exact dot products of the codes over channels [0, 64) and the rest,
        // each rounded once to fp32 as it is accumulated
        const int64_t half = std::min<int64_t>(64, d);
        for (int64_t j = 0; j < N; ++j) {
          double d0 = 0.0, d1 = 0.0, big = 0.0;
          for (int64_t c = 0; c < half; ++c) d0 += qq[(size_t)c] * kq[(size_t)(j * d + c)];
          for (int64_t c = half; c < d; ++c) d1 += qq[(size_t)c] * kq[(size_t)(j * d + c)];
          raw[(size_t)j] = (float)((double)(float)d0 + d1);
          if (allow) {
            for (int64_t c = 0; c < d; ++c)
              big = std::max(big, std::fabs(qq[(size_t)c] * kq[(size_t)(j * d + c)]));
            err[(size_t)j] = std::ldexp(big, -9) * (double)cb[(size_t)(j / 16)];  // log2 units
          }
        }
        amb.clear();
        double em = 0.0;  // error bound of the running maximum
        // tiles of p_tile keys, running maximum (fp32, base 2), carried sums (fp64)
        float m = -INFINITY;
        double l = 0.0;
        std::fill(acc.begin(), acc.end(), 0.0);
        for (int64_t t0 = 0; t0 < N; t0 += p_tile) {
          const int64_t t1 = std::min(N, t0 + p_tile);
          float local = -INFINITY;
          int64_t jmax = t0;
          for (int64_t j = t0; j < t1; ++j) {
            const float xj = raw[(size_t)j] * cb[(size_t)(j / 16)];
            if (xj > local) {
              local = xj;
              jmax = j;
            }
          }
          // a Skip-Softmax decision within the error window of its threshold may go either
          // way: the tile's weights (against the current maximum) enter the allowance
          const bool edge = allow && m != -INFINITY && skip_log2 != -INFINITY &&
                            std::fabs((double)local - ((double)m + skip_log2)) <=
                                err[(size_t)jmax] + em;
          if (local < m + skip_log2) {  // dropped (never when m = -inf or lambda = 0)
            if (edge)
              for (int64_t j = t0; j < t1; ++j) {
                const float arg = std::fmaf(raw[(size_t)j], cb[(size_t)(j / 16)], 8.0f - m);
                amb.push_back({j, h3o_e4m3((double)std::exp2f(arg)), m});
              }
            continue;
          }
          const float mt = local > m ? local : m;
          if (local > m) em = allow ? err[(size_t)jmax] : 0.0;
          const double carry = (m == -INFINITY) ? 0.0 : std::exp2((double)m - (double)mt);
          l *= carry;
          for (int64_t c = 0; c < d; ++c) acc[(size_t)c] *= carry;
          for (int64_t j = t0; j < t1; ++j) {
            const float arg = std::fmaf(raw[(size_t)j], cb[(size_t)(j / 16)], 8.0f - mt);
            const double p = h3o_e4m3((double)std::exp2f(arg));
            l += p;
            for (int64_t c = 0; c < d; ++c) acc[(size_t)c] += p * vq[(size_t)(j * d + c)];
            if (allow) {
              double dp = edge ? p : 0.0;
              const double wdw = err[(size_t)j] + em;
              const double plo = h3o_e4m3(std::exp2((double)arg - wdw));
              const double phi = h3o_e4m3(std::exp2((double)arg + wdw));
              dp = std::max(dp, std::max(std::fabs(phi - p), std::fabs(p - plo)));
              if (dp > 0.0) amb.push_back({j, dp, mt});
            }
          }
          m = mt;
        }
        for (int64_t c = 0; c < d; ++c) o[c] = vs[(size_t)c] * acc[(size_t)c] / l;
        if (al && !amb.empty()) {
          // each ambiguous weight carried to the final maximum; bound the normaliser below
          double total = 0.0;
          for (auto& e : amb) {
            e.dp *= std::exp2((double)e.mt - (double)m);
            total += e.dp;
          }
          const double lmin = std::max(l - total, 0.5 * l);
          for (const auto& e : amb)
            for (int64_t c = 0; c < d; ++c)
              al[c] += e.dp * std::fabs(vs[(size_t)c] * vq[(size_t)(e.j * d + c)] - o[c]) / lmin;
        }
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
                       double* out, double* allow) {
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
                             p_tile, skip_threshold, rows, n_rows, threads, out, allow);
}

}  // extern "C"
