// h3_oracle.cpp — fp64 CPU oracle for the packed-sequence DiT attention layer.
//
// TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
// benchmark's CPU baseline, never by the product library.  Plain definitions in
// fp64, written for checking by eye rather than for speed.  The only
// concession to speed is that independent rows run on separate std::threads;
// every individual sum is still accumulated in its natural index order.
//
// Pages cited (see h3_oracle.h for what each passage fixes):
//   [Blog] "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务",
//          §1, §3.1 "长序列注意力与通信", §3.2 "融合的 DiT 算子", §3.5.
#include "h3_oracle.h"

#include <cmath>
#include <cstring>
#include <thread>
#include <vector>
#include <algorithm>

namespace {

// Runs fn(lo, hi) over [0, n) split into `threads` contiguous chunks.
template <class F>
void parallel_for(int64_t n, int threads, F fn) {
  if (threads < 1) threads = 1;
  if (n <= 0) return;
  if (threads == 1 || n == 1) {
    fn(int64_t(0), n);
    return;
  }
  int64_t nt = std::min<int64_t>(threads, n);
  std::vector<std::thread> pool;
  pool.reserve(nt);
  for (int64_t t = 0; t < nt; ++t) {
    int64_t lo = n * t / nt, hi = n * (t + 1) / nt;
    pool.emplace_back([=]() { fn(lo, hi); });
  }
  for (auto& th : pool) th.join();
}

double widen(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return double(f);
}

// Rotates the pair (a, b) = (y[j], y[j + half]) by angle `ang` (rotate-half form):
//   a' = a cos - b sin,   b' = b cos + a sin.
void rotate_pair(double a, double b, double ang, double* a_out, double* b_out) {
  double c = std::cos(ang), s = std::sin(ang);
  *a_out = a * c - b * s;
  *b_out = b * c + a * s;
}

// Softmax attention of one head for query rows [lo, hi) (one thread's share).
//   q:   [n_rows][d]   query vectors       k, v: [n][d]   keys and values
//   out: [n_rows][d]
// Definition, per row r:
//   s_rj = scale * sum_c q_r[c] k_j[c]          (summed over c = 0, 1, ..., d-1)
//   m_r  = max_j s_rj                            (pass 1)
//   p_rj = exp(s_rj - m_r),  l_r = sum_j p_rj,  o_r = sum_j p_rj v_j / l_r   (pass 2,
//                                                summed over j = 0, 1, ..., n-1)
// The key loop is the outer loop so that one pass over K (and one over V) serves
// all of this thread's rows; every sum above still runs in the order written.
__attribute__((target_clones("avx2", "default")))
void attend_rows(const double* q, const double* k, const double* v, int64_t lo, int64_t hi,
                 int64_t n, int64_t d, double scale, double* out) {
  const int64_t R = hi - lo;
  if (R <= 0) return;
  for (int64_t r = 0; r < R; ++r)
    for (int64_t c = 0; c < d; ++c) out[(lo + r) * d + c] = 0.0;
  if (n == 0) return;
  std::vector<double> q_t(size_t(d * R));  // this thread's queries, channel-major
  for (int64_t r = 0; r < R; ++r)
    for (int64_t c = 0; c < d; ++c) q_t[c * R + r] = q[(lo + r) * d + c];
  std::vector<double> s(size_t(R * n));  // scores, key-major: s[j * R + r]
  std::vector<double> acc(static_cast<size_t>(R)), m(static_cast<size_t>(R)),
      l(static_cast<size_t>(R));
  // scores
  for (int64_t j = 0; j < n; ++j) {
    const double* kj = k + j * d;
    for (int64_t r = 0; r < R; ++r) acc[r] = 0.0;
    for (int64_t c = 0; c < d; ++c) {
      const double kc = kj[c];
      const double* qc = q_t.data() + c * R;
      for (int64_t r = 0; r < R; ++r) acc[r] += qc[r] * kc;
    }
    for (int64_t r = 0; r < R; ++r) s[j * R + r] = scale * acc[r];
  }
  // pass 1: row maxima
  for (int64_t r = 0; r < R; ++r) {
    m[r] = s[r];
    l[r] = 0.0;
  }
  for (int64_t j = 1; j < n; ++j)
    for (int64_t r = 0; r < R; ++r) m[r] = std::max(m[r], s[j * R + r]);
  // pass 2: exponentials, their sums, and the weighted sums of values
  for (int64_t j = 0; j < n; ++j) {
    const double* vj = v + j * d;
    for (int64_t r = 0; r < R; ++r) {
      const double p = std::exp(s[j * R + r] - m[r]);
      l[r] += p;
      double* o = out + (lo + r) * d;
      for (int64_t c = 0; c < d; ++c) o[c] += p * vj[c];
    }
  }
  for (int64_t r = 0; r < R; ++r) {
    double* o = out + (lo + r) * d;
    for (int64_t c = 0; c < d; ++c) o[c] /= l[r];
  }
}

// One head's attention for all n_rows query rows, rows split across threads.
void attend_head(const double* q, const double* k, const double* v, int64_t n_rows,
                 int64_t n, int64_t d, double scale, int threads, double* out) {
  parallel_for(n_rows, threads, [&](int64_t lo, int64_t hi) {
    attend_rows(q, k, v, lo, hi, n, d, scale, out);
  });
}

// Shared driver of the two bf16 entry points.  `prep_q` / `prep_k` produce one
// head row (fp64) of Q or K for token t; V rows are widened as they are.
template <class PrepQ, class PrepK>
int attn_bf16(const uint16_t* v, int64_t seq_buf, int64_t n_valid, int64_t heads, int64_t d,
              int64_t row_stride, double scale, const int64_t* rows, int64_t n_rows,
              int threads, double* out, PrepQ prep_q, PrepK prep_k) {
  if (n_valid < 0 || n_valid > seq_buf || heads <= 0 || d <= 0 || row_stride < heads * d)
    return H3O_ERR_ARG;
  if (n_rows > 0 && (!rows || !out)) return H3O_ERR_ARG;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= seq_buf) return H3O_ERR_ARG;
  // Valid query rows get attention; rows in [n_valid, seq_buf) are exact zeros.
  std::vector<int64_t> live;
  for (int64_t r = 0; r < n_rows; ++r) {
    if (rows[r] < n_valid) live.push_back(r);
    for (int64_t i = 0; i < heads * d; ++i) out[r * heads * d + i] = 0.0;
  }
  const int64_t nl = int64_t(live.size());
  std::vector<double> qh(size_t(nl * d)), oh(size_t(nl * d));
  std::vector<double> kh(size_t(n_valid * d)), vh(size_t(n_valid * d));
  int bad = 0;
  for (int64_t h = 0; h < heads; ++h) {
    parallel_for(n_valid, threads, [&](int64_t lo, int64_t hi) {
      for (int64_t j = lo; j < hi; ++j) {
        if (!prep_k(j, h, kh.data() + j * d)) bad = 1;
        h3o_widen_bf16(v + j * row_stride + h * d, d, vh.data() + j * d);
      }
    });
    parallel_for(nl, threads, [&](int64_t lo, int64_t hi) {
      for (int64_t i = lo; i < hi; ++i)
        if (!prep_q(rows[live[i]], h, qh.data() + i * d)) bad = 1;
    });
    if (bad) return H3O_ERR_ARG;
    attend_head(qh.data(), kh.data(), vh.data(), nl, n_valid, d, scale, threads, oh.data());
    for (int64_t i = 0; i < nl; ++i)
      for (int64_t c = 0; c < d; ++c) out[(live[i] * heads + h) * d + c] = oh[i * d + c];
  }
  return H3O_OK;
}

}  // namespace

extern "C" {

void h3o_widen_bf16(const uint16_t* src, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = widen(src[i]);
}

// [Blog §3.2] per-head Q/K RMSNorm: normalise by the root mean square over the
// head's channels (eps added to the mean square, inside the square root), then
// multiply channel-wise by the learned weight.
void h3o_rmsnorm_row(const double* x, const double* w, int64_t d, double eps, double* y) {
  double ss = 0.0;
  for (int64_t c = 0; c < d; ++c) ss += x[c] * x[c];
  const double ms = ss / double(d);
  const double inv = 1.0 / std::sqrt(ms + eps);
  for (int64_t c = 0; c < d; ++c) y[c] = x[c] * inv * w[c];
}

// [Blog §3.1, §3.2] rotary embedding of one head row ("RoPE rows").
int h3o_rope_row(const double* in, int64_t d, int mode, const double pos[3],
                 const int32_t sections[3], double theta, double* out) {
  if (d <= 0 || (d % 2) != 0) return H3O_ERR_ARG;
  std::vector<double> y(in, in + d);
  if (mode == 0) {
    const int64_t half = d / 2;
    for (int64_t j = 0; j < half; ++j) {
      const double freq = std::pow(theta, -2.0 * double(j) / double(d));
      rotate_pair(y[j], y[j + half], pos[0] * freq, &out[j], &out[j + half]);
    }
    return H3O_OK;
  }
  if (mode != 1) return H3O_ERR_ARG;
  int64_t total = 0;
  for (int s = 0; s < 3; ++s) {
    if (sections[s] < 0 || (sections[s] % 2) != 0) return H3O_ERR_ARG;
    total += sections[s];
  }
  if (total != d) return H3O_ERR_ARG;
  int64_t off = 0;
  for (int s = 0; s < 3; ++s) {
    const int64_t ds = sections[s], half = ds / 2;
    for (int64_t j = 0; j < half; ++j) {
      const double freq = std::pow(theta, -2.0 * double(j) / double(ds));
      rotate_pair(y[off + j], y[off + j + half], pos[s] * freq, &out[off + j],
                  &out[off + j + half]);
    }
    off += ds;
  }
  return H3O_OK;
}

int h3o_token_position(const h3o_rope* r, int64_t i, int* mode, double pos[3]) {
  if (i < 0) return H3O_ERR_ARG;
  if (i < r->n_1d) {
    *mode = 0;
    pos[0] = double(i);
    pos[1] = pos[2] = 0.0;
    return H3O_OK;
  }
  const int64_t gt = r->grid_t, gh = r->grid_h, gw = r->grid_w;
  if (gt <= 0 || gh <= 0 || gw <= 0) return H3O_ERR_ARG;
  const int64_t k = i - r->n_1d;
  if (k >= gt * gh * gw) return H3O_ERR_ARG;
  *mode = 1;
  pos[0] = double(k / (gh * gw));
  pos[1] = double((k / gw) % gh);
  pos[2] = double(k % gw);
  return H3O_OK;
}

int h3o_prologue(const uint16_t* x, int64_t heads, int64_t d, int64_t row_stride,
                 int64_t n_valid, const uint16_t* w, int64_t w_head_stride, double eps,
                 const h3o_rope* rope, const int64_t* rows, int64_t n_rows, int threads,
                 double* out) {
  if (!x || !w || !rope || (n_rows > 0 && (!rows || !out))) return H3O_ERR_ARG;
  if (heads <= 0 || d <= 0 || row_stride < heads * d) return H3O_ERR_ARG;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= n_valid) return H3O_ERR_ARG;
  int bad = 0;
  parallel_for(n_rows, threads, [&](int64_t lo, int64_t hi) {
    std::vector<double> xr(d), wr(d), y(d);
    for (int64_t r = lo; r < hi; ++r) {
      const int64_t t = rows[r];
      int mode;
      double pos[3];
      if (h3o_token_position(rope, t, &mode, pos) != H3O_OK) {
        bad = 1;
        continue;
      }
      for (int64_t h = 0; h < heads; ++h) {
        h3o_widen_bf16(x + t * row_stride + h * d, d, xr.data());
        h3o_widen_bf16(w + h * w_head_stride, d, wr.data());
        h3o_rmsnorm_row(xr.data(), wr.data(), d, eps, y.data());
        if (h3o_rope_row(y.data(), d, mode, pos, rope->sections, rope->theta,
                         out + (r * heads + h) * d) != H3O_OK)
          bad = 1;
      }
    }
  });
  return bad ? H3O_ERR_ARG : H3O_OK;
}

int h3o_attention(const double* q, const double* k, const double* v, int64_t n_rows,
                  int64_t n_valid, int64_t heads, int64_t d, double scale, int threads,
                  double* out) {
  if (n_rows < 0 || n_valid < 0 || heads <= 0 || d <= 0) return H3O_ERR_ARG;
  if (n_rows > 0 && (!q || !out)) return H3O_ERR_ARG;
  if (n_valid > 0 && (!k || !v)) return H3O_ERR_ARG;
  std::vector<double> qh(size_t(n_rows * d)), oh(size_t(n_rows * d));
  std::vector<double> kh(size_t(n_valid * d)), vh(size_t(n_valid * d));
  for (int64_t h = 0; h < heads; ++h) {
    for (int64_t r = 0; r < n_rows; ++r)
      for (int64_t c = 0; c < d; ++c) qh[r * d + c] = q[(r * heads + h) * d + c];
    for (int64_t j = 0; j < n_valid; ++j)
      for (int64_t c = 0; c < d; ++c) {
        kh[j * d + c] = k[(j * heads + h) * d + c];
        vh[j * d + c] = v[(j * heads + h) * d + c];
      }
    attend_head(qh.data(), kh.data(), vh.data(), n_rows, n_valid, d, scale, threads,
                oh.data());
    for (int64_t r = 0; r < n_rows; ++r)
      for (int64_t c = 0; c < d; ++c) out[(r * heads + h) * d + c] = oh[r * d + c];
  }
  return H3O_OK;
}


int h3o_attn_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_buf,
                    int64_t n_valid, int64_t heads, int64_t d, int64_t row_stride,
                    double scale, const int64_t* rows, int64_t n_rows, int threads,
                    double* out) {
  if (!q || !k || !v) return H3O_ERR_ARG;
  auto plain = [&](const uint16_t* x) {
    return [=](int64_t t, int64_t h, double* dst) {
      h3o_widen_bf16(x + t * row_stride + h * d, d, dst);
      return true;
    };
  };
  return attn_bf16(v, seq_buf, n_valid, heads, d, row_stride, scale, rows, n_rows, threads,
                   out, plain(q), plain(k));
}

int h3o_attn_layer(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_buf,
                   int64_t n_valid, int64_t heads, int64_t d, int64_t row_stride,
                   const uint16_t* w_q, const uint16_t* w_k, int64_t w_head_stride,
                   double eps, const h3o_rope* rope, double scale, const int64_t* rows,
                   int64_t n_rows, int threads, double* out) {
  if (!q || !k || !v || !w_q || !w_k || !rope) return H3O_ERR_ARG;
  // RMSNorm, then RoPE, of token t head h of buffer x with weights wt.
  auto normed = [&](const uint16_t* x, const uint16_t* wt) {
    return [=](int64_t t, int64_t h, double* dst) {
      std::vector<double> xr(d), wr(d), y(d);
      int mode;
      double pos[3];
      if (h3o_token_position(rope, t, &mode, pos) != H3O_OK) return false;
      h3o_widen_bf16(x + t * row_stride + h * d, d, xr.data());
      h3o_widen_bf16(wt + h * w_head_stride, d, wr.data());
      h3o_rmsnorm_row(xr.data(), wr.data(), d, eps, y.data());
      return h3o_rope_row(y.data(), d, mode, pos, rope->sections, rope->theta, dst) ==
             H3O_OK;
    };
  };
  return attn_bf16(v, seq_buf, n_valid, heads, d, row_stride, scale, rows, n_rows, threads,
                   out, normed(q, w_q), normed(k, w_k));
}

}  // extern "C"
