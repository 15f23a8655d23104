// attention.hpp — dense non-causal softmax attention over the valid tokens of a packed,
// aligned buffer, bf16 MFMA on gfx950.
//
// Pages: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
// (Chinese translation of the vLLM blog post), §3.1: attention receives the valid
// sequence length and the structural tail padding is not computed; §3.2: the Q/K
// RMSNorm + RoPE prologue is fused (here: the Q half in registers).
//
// Structure (one workgroup = 4 waves = one head x BM query rows, BM = 4 * 32 * RB):
//   * Q: each wave holds RB blocks of 32 query rows in registers as MFMA B operands
//     (optionally normalised + rotated on load).
//   * K/V: 64-key tiles, prepared by kv_pack_kernel as swizzled 16 KiB images, are
//     copied linearly into a double-buffered LDS ring (2 x 32 KiB).
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16.  Lane l of a wave owns query row
//     l % 32 of each row block; K rows are read in the order swap23(l % 32) so that the
//     accumulator registers come out in the exact order of the P^T B operand of the
//     second product (no cross-lane shuffles between the two products).
//   * Online softmax in fp32, base-2, with the softmax scale folded into the exponent;
//     the running max is only raised when a new score exceeds it by more than kTau
//     (log2 units), so the O rescale is skipped almost always.
//   * O^T += V^T P^T with the same MFMA; V^T chunks come straight from the V image.
//   * Epilogue: O / l -> bf16; rows in [N, S) are written as zeros.
#pragma once

#include "common.hpp"
#include "prologue.hpp"

namespace h3 {

struct AttnArgs {
  const __bf16* q;
  __bf16* o;
  const char* k_img;
  const char* v_img;
  int64_t tiles_per_head;
  int64_t in_stride, out_stride;
  int64_t n_valid, seq_buf;
  int heads;
  int m_tiles;            // ceil(seq_buf / BM)
  float scale_log2;       // softmax_scale * log2(e)
  // fused Q prologue
  const __bf16* w_q;
  int64_t w_head_stride;
  float eps;
  RopeArgs rope;
};

// Raise the running max only when a score exceeds it by more than this (log2 units):
// exponentials stay <= 2^kTau, far inside fp32 and bf16 range.
constexpr float kTau = 8.0f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Waves per SIMD the register budget is sized for: two workgroups per CU with one
// 32-row block per wave (<= 256 registers), one with two blocks (<= 512).
template <int RB>
struct AttnOccupancy {
  static constexpr int kWavesPerEU = RB == 1 ? 2 : 1;
};

template <int RB, bool kFusedQ>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(AttnOccupancy<RB>::kWavesPerEU,
                                   AttnOccupancy<RB>::kWavesPerEU))) void
attn_fwd_kernel(AttnArgs a) {
  constexpr int kWaves = 4;
  constexpr int BM = kWaves * RB * 32;
  __shared__ __attribute__((aligned(16))) char smem[2][2 * kTileBytes];
  __shared__ FreqTable ft;

  const int logical = xcd_remap(blockIdx.x, a.heads * a.m_tiles);
  const int head = logical / a.m_tiles;
  const int64_t m0 = (int64_t)(logical % a.m_tiles) * BM;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5, l32 = lane & 31;
  const int64_t hoff = (int64_t)head * kHeadDim;

  // Workgroups entirely past the valid length only zero their output rows.
  if (m0 >= a.n_valid) {
    const int64_t rows = (a.seq_buf - m0) < BM ? (a.seq_buf - m0) : BM;
    for (int64_t i = tid; i < rows * kChunks; i += 256) {
      const int64_t r = m0 + i / kChunks;
      *reinterpret_cast<u32x4*>(a.o + r * a.out_stride + hoff + (i % kChunks) * 8) =
          u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }

  if (kFusedQ) {
    fill_freq_table(&ft, a.rope, tid, 256);
    __syncthreads();
  }

  // ---- Q rows -> registers (B operand: lane holds row l32, channels 16ks + 8hl .. +8)
  bf16x8 qreg[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t row = m0 + (wave * RB + rb) * 32 + l32;
    const bool valid = row < a.n_valid;
    const __bf16* qrow = a.q + row * a.in_stride + hoff;
    u32x4 raw[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      raw[ks] = valid ? *reinterpret_cast<const u32x4*>(qrow + (2 * ks + hl) * 8)
                      : u32x4{0u, 0u, 0u, 0u};
    if (kFusedQ) {
      // RMS over the row: partials of the 8 own chunks, the other 8 from lane l^32,
      // combined in the canonical pairwise tree (chunks c, c^1, then c^2, c^4, c^8).
      float part[8], other[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        float x[8];
        unpack8(raw[ks], x);
        part[ks] = chunk_sumsq(x);
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) other[ks] = other_half(part[ks]);
      // chunk 2ks is even, 2ks+1 odd: level-1 sums p[2ks] + p[2ks+1]
      float s1[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s1[ks] = hl ? other[ks] + part[ks] : part[ks] + other[ks];
      const float s2[4] = {s1[0] + s1[1], s1[2] + s1[3], s1[4] + s1[5], s1[6] + s1[7]};
      const float s3[2] = {s2[0] + s2[1], s2[2] + s2[3]};
      const float ss = s3[0] + s3[1];
      const float inv = inv_rms(ss, a.eps);
      const __bf16* w = a.w_q + (int64_t)head * a.w_head_stride;
#pragma unroll 1
      for (int ks = 0; ks < 8; ++ks) {
        const int cc = 2 * ks + hl;
        const ChunkRot cr = chunk_rotation(a.rope, row, cc);
        float x[8], xp[8], wv[8], wpv[8], y[8];
        unpack8(raw[ks], x);
        const u32x4 praw = valid ? *reinterpret_cast<const u32x4*>(qrow + cr.partner * 8)
                                 : u32x4{0u, 0u, 0u, 0u};
        unpack8(praw, xp);
        unpack8(*reinterpret_cast<const u32x4*>(w + cc * 8), wv);
        unpack8(*reinterpret_cast<const u32x4*>(w + cr.partner * 8), wpv);
        norm_rotate_chunk(x, xp, wv, wpv, inv, cr, &ft, y);
        raw[ks] = pack8(y);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[rb][ks] = __builtin_bit_cast(bf16x8, raw[ks]);
  }

  // ---- main loop over 64-key tiles
  const int64_t n_tiles = (a.n_valid + kTileKeys - 1) / kTileKeys;
  const char* kimg = a.k_img + (int64_t)head * a.tiles_per_head * kTileBytes;
  const char* vimg = a.v_img + (int64_t)head * a.tiles_per_head * kTileBytes;
  const int tail_keys = (int)(a.n_valid - (n_tiles - 1) * kTileKeys);  // 1..64

  float m_run[RB], l_run[RB];
  f32x16 oacc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[rb][db] = f32x16{};
  }

  // staging: each thread copies 4 x 16 B of the K image and 4 x 16 B of the V image
  u32x4 stage[8];
  auto load_tile = [&](int64_t kt) {
    const char* ks = kimg + kt * kTileBytes;
    const char* vs = vimg + kt * kTileBytes;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      stage[p] = *reinterpret_cast<const u32x4*>(ks + (p * 256 + tid) * 16);
      stage[4 + p] = *reinterpret_cast<const u32x4*>(vs + (p * 256 + tid) * 16);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      *reinterpret_cast<u32x4*>(&smem[buf][(p * 256 + tid) * 16]) = stage[p];
      *reinterpret_cast<u32x4*>(&smem[buf][kTileBytes + (p * 256 + tid) * 16]) = stage[4 + p];
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  // LDS read offsets (bytes) within one buffer.
  // K: A operand row kb*32 + swap23(l32), chunk 2ks + hl, slot row*16 + (chunk ^ (l32 & 15)).
  const int krow = swap23(l32);
  // V: A operand row d = db*32 + l32, chunk 2t + hl, slot d*8 + (chunk ^ vswz(d)).
  const int vx = vswz(l32);
  const float c2 = a.scale_log2;

  for (int64_t kt = 0; kt < n_tiles; ++kt) {
    const bool has_next = kt + 1 < n_tiles;
    if (has_next) load_tile(kt + 1);
    const char* kl = smem[kt & 1];
    const char* vl = kl + kTileBytes;

    // S^T (keys x rows) for two 32-key blocks
    f32x16 sacc[2][RB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[kb][rb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = kb * 32 + krow;
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(
            kl + (r * 16 + ((2 * ks + hl) ^ (l32 & 15))) * 16);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sacc[kb][rb] = mfma32(kop, qreg[rb][ks], sacc[kb][rb]);
      }
    }

    // mask keys >= N (last tile only).  Register 4i+j of block kb holds key
    // kb*32 + 16(i>>1) + 8hl + 4(i&1) + j of the tile.
    if (kt == n_tiles - 1 && tail_keys < kTileKeys) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kb * 32 + 16 * (i >> 1) + 8 * hl + 4 * (i & 1) + j;
            if (key >= tail_keys)
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) sacc[kb][rb][4 * i + j] = -INFINITY;
          }
    }

    // online softmax, P^T as bf16 B operands
    bf16x8 preg[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = sacc[0][rb][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][rb][e]);
      mx = pair_max(mx);
      const bool raise = mx * c2 > m_run[rb] * c2 + kTau || m_run[rb] == -INFINITY;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float m_new = raise ? fmaxf(mx, m_run[rb]) : m_run[rb];
        const float alpha = __builtin_amdgcn_exp2f((m_run[rb] - m_new) * c2);
        m_run[rb] = m_new;
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[rb][db][e] *= alpha;
      }
      const float mc = m_run[rb] * c2;
      float lsum = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[t >> 1][rb][8 * (t & 1) + e], c2, -mc));
          lsum += p[e];
        }
        preg[rb][t] = __builtin_bit_cast(bf16x8, pack8(p));
      }
      l_run[rb] += lsum;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + l32;
        const bf16x8 vop = *reinterpret_cast<const bf16x8*>(
            vl + (d * 8 + ((2 * t + hl) ^ vx)) * 16);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = mfma32(vop, preg[rb][t], oacc[rb][db]);
      }
    }

    if (has_next) store_tile((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds O[row l32][d = db*32 + 8i + 4hl + j] at register 4i+j
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t row = m0 + (wave * RB + rb) * 32 + l32;
    if (row >= a.seq_buf) continue;
    const float l = pair_sum(l_run[rb]);
    const bool valid = row < a.n_valid;
    const float inv = 1.0f / l;
    __bf16* orow = a.o + row * a.out_stride + hoff;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w = {0u, 0u};  // rows in [N, S): exact +0
        if (valid) {
          w[0] = pack_bf16x2(oacc[rb][db][4 * i] * inv, oacc[rb][db][4 * i + 1] * inv);
          w[1] = pack_bf16x2(oacc[rb][db][4 * i + 2] * inv, oacc[rb][db][4 * i + 3] * inv);
        }
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * i + 4 * hl) = w;
      }
  }
}

}  // namespace h3
