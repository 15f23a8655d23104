// h3_oracle_block.cpp — fp64 CPU oracle for the DiT block steps on either side of the
// attention: gated residual update, normalization and modulation.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or calls
// this code; only the tests, the smoke check and the benchmark's CPU baseline do.  It
// shares no source with the GPU path.
//
// Page: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
// (Chinese translation of the vLLM blog post), §3.2: around the matrix products the
// DiT's small FP32 steps (modulation, normalization, residual) are merged into one
// operation.  The pages give no formula; the reading taken here is the plain adaLN form
// of a DiT block:
//   - residual (when a branch output a is given): x <- x + gate * a, per channel, in the
//     fp32 residual stream (gate absent: 1);
//   - normalization: LayerNorm over the hidden channels without an affine part,
//     n = (x - mean) / sqrt(var + eps), with the population variance;
//   - modulation: y = n * (1 + scale) + shift, rounded to bf16 for the next product.
// Rows in [N, S) are not read; their y is 0 and their x is left as it is.
// Parity status: pinned by closed forms in tests/test_oracle_block_pins.py.
#include "h3_oracle.h"

#include <cmath>
#include <cstring>
#include <vector>

namespace {

double widen(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

}  // namespace

extern "C" {

int h3o_residual_norm_modulate(const float* x, const uint16_t* a, const float* gate,
                               const float* shift, const float* scale, int64_t seq_buf,
                               int64_t n_valid, int64_t hidden, double eps, double* x_out,
                               double* y_out) {
  if (!x || !shift || !scale || !x_out || !y_out) return H3O_ERR_ARG;
  if (hidden <= 0 || n_valid < 0 || n_valid > seq_buf || !(eps >= 0.0)) return H3O_ERR_ARG;
  std::vector<double> r((size_t)hidden);
  for (int64_t t = 0; t < seq_buf; ++t) {
    const float* xr = x + t * hidden;
    double* xo = x_out + t * hidden;
    double* yo = y_out + t * hidden;
    if (t >= n_valid) {
      for (int64_t c = 0; c < hidden; ++c) {
        xo[c] = xr[c];
        yo[c] = 0.0;
      }
      continue;
    }
    // residual update
    for (int64_t c = 0; c < hidden; ++c) {
      double v = xr[c];
      if (a) v += (gate ? (double)gate[c] : 1.0) * widen(a[t * hidden + c]);
      r[(size_t)c] = v;
      xo[c] = v;
    }
    // LayerNorm, two passes
    double mean = 0.0;
    for (int64_t c = 0; c < hidden; ++c) mean += r[(size_t)c];
    mean /= (double)hidden;
    double var = 0.0;
    for (int64_t c = 0; c < hidden; ++c) {
      const double d = r[(size_t)c] - mean;
      var += d * d;
    }
    var /= (double)hidden;
    const double inv = 1.0 / std::sqrt(var + eps);
    // modulation
    for (int64_t c = 0; c < hidden; ++c)
      yo[c] = (r[(size_t)c] - mean) * inv * (1.0 + (double)scale[c]) + (double)shift[c];
  }
  return H3O_OK;
}

}  // extern "C"
