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
// One workgroup of 256 threads per token; each thread holds up to kMaxChunks chunks of
// 8 channels in registers, so the row is read from HBM once and the variance is taken
// in a second pass over registers (no cancellation).  HBM-bound: per token it reads
// 4C bytes of x (+ 2C of a) and writes 2C of y (+ 4C of x).
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
  float eps;
};

namespace blk {
constexpr int kThreads = 256;
constexpr int kMaxChunks = 4;  // 8-channel chunks per thread: C <= 8,192
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

template <bool kResidual, bool kGate>
__global__ __launch_bounds__(blk::kThreads) void residual_norm_modulate_kernel(BlockArgs a) {
  using namespace blk;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nchunk = (int)(a.hidden / 8);
  __bf16* yrow = a.y + row * a.hidden;
  if (row >= a.n_valid) {  // rows past the valid length: y = 0, x untouched
    for (int c = tid; c < nchunk; c += kThreads)
      *reinterpret_cast<u32x4*>(yrow + c * 8) = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  float* xrow = a.x + row * a.hidden;
  __shared__ float red[4];

  float v[kMaxChunks][8];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = tid + i * kThreads;
    if (c < nchunk) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(xrow + c * 8);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(xrow + c * 8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[i][e] = x0[e];
        v[i][4 + e] = x1[e];
      }
      if (kResidual) {
        float br[8];
        unpack8(*reinterpret_cast<const u32x4*>(a.a + row * a.hidden + c * 8), br);
        float g[8];
        if (kGate) {
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(a.gate + c * 8);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(a.gate + c * 8 + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            g[e] = g0[e];
            g[4 + e] = g1[e];
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[i][e] = kGate ? __builtin_fmaf(g[e], br[e], v[i][e]) : v[i][e] + br[e];
        *reinterpret_cast<f32x4*>(xrow + c * 8) = f32x4{v[i][0], v[i][1], v[i][2], v[i][3]};
        *reinterpret_cast<f32x4*>(xrow + c * 8 + 4) = f32x4{v[i][4], v[i][5], v[i][6], v[i][7]};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += v[i][e];
    }
  }
  const float inv_c = 1.0f / (float)a.hidden;
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
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(a.scale + c * 8);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(a.scale + c * 8 + 4);
      const f32x4 h0 = *reinterpret_cast<const f32x4*>(a.shift + c * 8);
      const f32x4 h1 = *reinterpret_cast<const f32x4*>(a.shift + c * 8 + 4);
      float out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float sc = e < 4 ? s0[e] : s1[e - 4];
        const float sh = e < 4 ? h0[e] : h1[e - 4];
        out[e] = __builtin_fmaf((v[i][e] - mean) * inv, 1.0f + sc, sh);
      }
      *reinterpret_cast<u32x4*>(yrow + c * 8) = pack8(out);
    }
  }
}

}  // namespace h3
