// block.hpp — the DiT block steps on either side of the attention, fused into one pass
// over the fp32 residual stream: gated residual update, LayerNorm, modulation.
//
// Page: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
// (Chinese translation of the vLLM blog post), §3.2: the DiT's small FP32 steps
// (modulation, normalization, residual) are merged into one operation.  The formula is
// the plain adaLN reading (the pages give none):
//   x <- x + gate * a        (when the branch output a is given; gate absent: 1)
//   y  = (x - mean) / sqrt(var + eps) * (1 + scale) + shift      (bf16 out)
// over the `hidden` channels of each valid token, with the population variance.
//
// One workgroup of 256 threads per group of consecutive tokens, taken one after the
// other: 4 with the residual update, whose threads then keep their channels' gate,
// shift and scale in registers for the whole group (read once per group, not per
// token), 1 without it (measured: holding them costs the lighter variant more in
// occupancy than it saves).  Each thread holds up to kMaxChunks chunks of 8 channels of
// the current row, so the row is read from HBM once and the variance is taken in a
// second pass over registers (no cancellation).
// HBM-bound: per token it reads 4C bytes of x (+ 2C of a) and writes 2C of y (+ 4C of x).
#pragma once

#include "common.hpp"

namespace h3 {

struct BlockArgs {
  float* x;              // [S, C] fp32 residual stream (updated when a is given)
  const __bf16* a;       // [S, C] branch output, or NULL
  const float* gate;     // [C] or NULL (gate 1)
  const float* shift;    // [C]
  const float* scale;    // [C]
  __bf16* y;             // [S, C]
  int64_t hidden;        // C, a multiple of 8, at most 8 * 256 * kMaxChunks
  int64_t n_valid;
  int64_t seq_buf;       // S
  float eps;
};

namespace blk {
constexpr int kThreads = 256;
constexpr int kMaxChunks = 4;  // 8-channel chunks per thread: C <= 8,192
constexpr int kRowsResidual = 4;  // rows per workgroup with the residual update
constexpr int kRowsPlain = 1;     // rows per workgroup without it
}  // namespace blk

// Sum over the workgroup (256 threads = 4 waves), identical in every thread.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // `red` may still be read from the previous reduction
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// kRows consecutive rows per workgroup.  With kRows > 1 each thread loads its slices of
// gate, shift and scale once and keeps them in registers for all the rows; with
// kRows = 1 it loads them where they are used (fewer live registers, more waves).
template <bool kResidual, bool kGate, int kRows>
__global__ __launch_bounds__(blk::kThreads) void residual_norm_modulate_kernel(BlockArgs a) {
  using namespace blk;
  constexpr bool kHold = kRows > 1;
  const int tid = threadIdx.x;
  const int nchunk = (int)(a.hidden / 8);
  __shared__ float red[4];

  // 8 consecutive fp32 values of a modulation vector
  auto load8 = [&](const float* p, int c, float* out) __attribute__((always_inline)) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p + c * 8);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(p + c * 8 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[e] = lo[e];
      out[4 + e] = hi[e];
    }
  };
  float g[kMaxChunks][8], sh[kMaxChunks][8], sc[kMaxChunks][8];
  if (kHold) {
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int c = tid + i * kThreads;
      if (c < nchunk) {
        if (kGate) load8(a.gate, c, g[i]);
        load8(a.shift, c, sh[i]);
        load8(a.scale, c, sc[i]);
      }
    }
  }

  const float inv_c = 1.0f / (float)a.hidden;
  for (int k = 0; k < kRows; ++k) {
    const int64_t row = (int64_t)blockIdx.x * kRows + k;  // uniform
    if (row >= a.seq_buf) break;
    __bf16* yrow = a.y + row * a.hidden;
    if (row >= a.n_valid) {  // rows past the valid length: y = 0, x untouched
      for (int c = tid; c < nchunk; c += kThreads)
        *reinterpret_cast<u32x4*>(yrow + c * 8) = u32x4{0u, 0u, 0u, 0u};
      continue;
    }
    float* xrow = a.x + row * a.hidden;
    float v[kMaxChunks][8];
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int c = tid + i * kThreads;
      if (c < nchunk) {
        load8(xrow, c, v[i]);
        if (kResidual) {
          float br[8];
          unpack8(*reinterpret_cast<const u32x4*>(a.a + row * a.hidden + c * 8), br);
          float gi[8];
          if (kGate && !kHold) load8(a.gate, c, gi);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            v[i][e] = kGate ? __builtin_fmaf(kHold ? g[i][e] : gi[e], br[e], v[i][e])
                            : v[i][e] + br[e];
          *reinterpret_cast<f32x4*>(xrow + c * 8) = f32x4{v[i][0], v[i][1], v[i][2], v[i][3]};
          *reinterpret_cast<f32x4*>(xrow + c * 8 + 4) = f32x4{v[i][4], v[i][5], v[i][6], v[i][7]};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += v[i][e];
      }
    }
    const float mean = block_sum(sum, red) * inv_c;
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int c = tid + i * kThreads;
      if (c < nchunk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = v[i][e] - mean;
          ss = __builtin_fmaf(d, d, ss);
        }
    }
    const float var = block_sum(ss, red) * inv_c;
    const float inv = 1.0f / sqrtf(var + a.eps);
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int c = tid + i * kThreads;
      if (c < nchunk) {
        float sci[8], shi[8];
        if (!kHold) {
          load8(a.scale, c, sci);
          load8(a.shift, c, shi);
        }
        float out[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          out[e] = __builtin_fmaf((v[i][e] - mean) * inv, 1.0f + (kHold ? sc[i][e] : sci[e]),
                                  kHold ? sh[i][e] : shi[e]);
        *reinterpret_cast<u32x4*>(yrow + c * 8) = pack8(out);
      }
    }
  }
}

}  // namespace h3
