// attention_pipelined.hpp — dense non-causal softmax attention over the valid tokens of
// a packed, aligned buffer; software-pipelined for gfx950.
//
// Pages: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
// (Chinese translation of the vLLM blog post), §3.1: attention receives the valid
// sequence length and the structural tail padding is not computed; §3.2: the Q/K
// RMSNorm + RoPE prologue is fused (the Q half here, in registers).
//
// Why the pipeline.  On gfx950 a wave can issue VALU work while its own MFMA runs, but
// only a few instructions' worth per MFMA (about two v_exp_f32 or four full-rate ops per
// 32x32x16 MFMA are hidden); VALU work of another wave on the same SIMD overlaps much
// less.  So each wave interleaves the softmax of one 64-key tile with the matrix
// products of its neighbours.  Per tile j, for the wave's 32 query rows:
//
//   B1: QK(j+1)  MFMA x16  ||  E(j)          (32 exp2)
//   B2: PV(j)    MFMA x16  ||  C(j), M(j+1)   (bf16 convert + row sums, row max + check)
//       -- stage tile j+2 into LDS; barrier; load tile j+3 --
//
// QK: S^T = K Q^T (two 32-key halves); M: row max of the new scores, raising the running
// max where it is exceeded (rare branch); E: p = exp2(s); C: p -> bf16 and row sums;
// PV: O^T += V^T P^T.  The scores of tiles j and j+1 live in two register sets used
// alternately (loop unrolled by two).
//
// Arithmetic.  Q is pre-scaled by softmax_scale*log2(e), so scores are in log2 units, and
// the QK accumulation starts from -m (the running max) as its C operand: the
// accumulator holds s - m directly and p = exp2(acc) costs one instruction.  The running
// max is raised only when a score exceeds it by more than kTauP (log2 units), so p <= 2^8
// and the O rescale is rare.  Keys >= N in the last tile start from -inf instead.  Row sums
// use v_dot2_f32_bf16 on the bf16-rounded p, so the normaliser matches the weights fed to
// the PV product exactly.
//
// Memory.  Eight waves (256 query rows) share each K/V tile.  Tiles (prepared by
// kv_pack_kernel as swizzled 16 KiB images) go through a 3-slot LDS ring (96 KiB): tile j
// is read from B1(j-1) to B2(j).  Tile j+2 is copied global -> LDS directly (no staging
// registers) during step j into the slot tile j-1 left, and waited for at the step's end,
// before its one barrier.  Everything fits in 256 VGPRs per lane, two waves per SIMD.
#pragma once

#include "attention.hpp"
#include "common.hpp"
#include "prologue.hpp"

#include <type_traits>

namespace h3 {

constexpr float kTauP = 8.0f;  // log2 units

namespace pipe {

constexpr int kSlots = 3;
constexpr int kSlotBytes = 2 * kTileBytes;  // K image + V image
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;           // query rows per workgroup

struct Wave {
  bf16x8 q[8];      // Q^T B operands (pre-scaled)
  f32x16 o[4];      // O^T accumulators per 32-channel block
  bf16x8 p[4];      // P^T B operands per 16-key step
  f32x16 negm;      // C operand of QK: -m, splat
  float m, l;       // running max (log2 units), row-sum partial over this lane's keys
};

// S^T (64 keys x 32 rows, as two 32-key halves) from the K image at `kl`; the
// accumulation starts from c0[kb].
__device__ __forceinline__ void qk(const Wave& w, f32x16* s, const char* kl, const f32x16* c0,
                                   int krow, int l15, int hl) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int r = kb * 32 + krow;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(
          kl + (r * 16 + ((2 * ks + hl) ^ l15)) * 16);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.q[ks], ks == 0 ? c0[kb] : s[kb], 0,
                                                      0, 0);
    }
  }
}

// O^T += V^T P^T from the V image at `vl`.
__device__ __forceinline__ void pv(Wave& w, const char* vl, int l32, int vx, int hl) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + l32;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vl + (d * 8 + ((2 * t + hl) ^ vx)) * 16);
      w.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.p[t], w.o[db], 0, 0, 0);
    }
  }
}

// E: p = exp2(acc), in place.
__device__ __forceinline__ void ex(f32x16* s) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = __builtin_amdgcn_exp2f(s[kb][e]);
}

// C: p -> bf16 operands; row sum of the rounded values (v_dot2_f32_bf16 with (1, 1)).
__device__ __forceinline__ void cv(Wave& w, const f32x16* s) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float acc0 = w.l, acc1 = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    bf16x2 pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 f = {s[t >> 1][8 * (t & 1) + 2 * i], s[t >> 1][8 * (t & 1) + 2 * i + 1]};
      pr[i] = __builtin_convertvector(f, bf16x2);
    }
    acc0 = __builtin_amdgcn_fdot2_f32_bf16(pr[0], ones, acc0, false);
    acc1 = __builtin_amdgcn_fdot2_f32_bf16(pr[1], ones, acc1, false);
    acc0 = __builtin_amdgcn_fdot2_f32_bf16(pr[2], ones, acc0, false);
    acc1 = __builtin_amdgcn_fdot2_f32_bf16(pr[3], ones, acc1, false);
    const bf16x8 pv8 = {pr[0][0], pr[0][1], pr[1][0], pr[1][1],
                        pr[2][0], pr[2][1], pr[3][0], pr[3][1]};
    w.p[t] = pv8;
  }
  w.l = acc0 + acc1;
}

// M: tile row max of acc; raise the running max where it is exceeded by more than kTauP
// (always on the first tile).  Rare path: rescale O and l, shift acc and -m.
template <bool kFirst>
__device__ __forceinline__ void mx(Wave& w, f32x16* s) {
  float v = s[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) v = fmaxf(v, s[kb][e]);
  v = pair_max(v);
  const bool need = kFirst || v > kTauP;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float delta = need ? v : 0.0f;
    w.m += delta;
    if (!kFirst) {
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      w.l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) w.o[db][e] *= alpha;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) w.negm[e] = -w.m;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] -= delta;
  }
}

}  // namespace pipe

template <bool kFusedQ>
__global__ __launch_bounds__(pipe::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_pipelined_kernel(AttnArgs a) {
  using namespace pipe;
  __shared__ __attribute__((aligned(16))) char smem[kSlots * kSlotBytes];
  __shared__ FreqTable ft;

  const int logical = xcd_remap(blockIdx.x, a.heads * a.m_tiles);
  const int head = logical / a.m_tiles;
  const int64_t m0 = (int64_t)(logical % a.m_tiles) * kRows;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5, l32 = lane & 31;
  const int64_t hoff = (int64_t)head * kHeadDim;

  if (m0 >= a.n_valid) {  // rows past the valid length: zeros only
    const int64_t rows = (a.seq_buf - m0) < kRows ? (a.seq_buf - m0) : kRows;
    for (int64_t i = tid; i < rows * kChunks; i += kThreads) {
      const int64_t r = m0 + i / kChunks;
      *reinterpret_cast<u32x4*>(a.o + r * a.out_stride + hoff + (i % kChunks) * 8) =
          u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  if (kFusedQ) {
    fill_freq_table(&ft, a.rope, tid, kThreads);
    __syncthreads();
  }

  Wave w;
  const float c2 = a.scale_log2;
  const int64_t row = m0 + wave * 32 + l32;
  const bool row_valid = row < a.n_valid;

  // ---- Q row -> B operands (lane: channels 16ks + 8hl .. +8), scaled by scale*log2(e)
  {
    const __bf16* qrow = a.q + row * a.in_stride + hoff;
    u32x4 raw[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      raw[ks] = row_valid ? *reinterpret_cast<const u32x4*>(qrow + (2 * ks + hl) * 8)
                          : u32x4{0u, 0u, 0u, 0u};
    if (kFusedQ) {
      // RMS of the row: partials of the 8 own chunks, the other 8 from lane l^32, combined
      // in the canonical pairwise tree (chunks c, c^1, then c^2, c^4, c^8).
      float part[8], other[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        float x[8];
        unpack8(raw[ks], x);
        part[ks] = chunk_sumsq(x);
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) other[ks] = other_half(part[ks]);
      float s1[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s1[ks] = hl ? other[ks] + part[ks] : part[ks] + other[ks];
      const float s2[4] = {s1[0] + s1[1], s1[2] + s1[3], s1[4] + s1[5], s1[6] + s1[7]};
      const float s3[2] = {s2[0] + s2[1], s2[2] + s2[3]};
      const float inv = inv_rms(s3[0] + s3[1], a.eps);
      const __bf16* wq = a.w_q + (int64_t)head * a.w_head_stride;
#pragma unroll 1
      for (int ks = 0; ks < 8; ++ks) {
        const int cc = 2 * ks + hl;
        const ChunkRot cr = chunk_rotation(a.rope, row, cc);
        float x[8], xp[8], wv[8], wpv[8], y[8];
        unpack8(raw[ks], x);
        const u32x4 praw = row_valid ? *reinterpret_cast<const u32x4*>(qrow + cr.partner * 8)
                                     : u32x4{0u, 0u, 0u, 0u};
        unpack8(praw, xp);
        unpack8(*reinterpret_cast<const u32x4*>(wq + cc * 8), wv);
        unpack8(*reinterpret_cast<const u32x4*>(wq + cr.partner * 8), wpv);
        norm_rotate_chunk(x, xp, wv, wpv, inv, cr, &ft, y);
        raw[ks] = pack8(y);  // the same bf16 values h3_qk_rmsnorm_rope writes
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      float x[8];
      unpack8(raw[ks], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= c2;
      w.q[ks] = __builtin_bit_cast(bf16x8, pack8(x));
    }
  }
  w.m = 0.0f;
  w.l = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) w.negm[e] = 0.0f;
#pragma unroll
  for (int db = 0; db < 4; ++db) w.o[db] = f32x16{};

  const int nt = (int)((a.n_valid + kTileKeys - 1) / kTileKeys);
  const char* kimg = a.k_img + (int64_t)head * a.tiles_per_head * kTileBytes;
  const char* vimg = a.v_img + (int64_t)head * a.tiles_per_head * kTileBytes;
  const int tail = (int)(a.n_valid - (int64_t)(nt - 1) * kTileKeys);  // valid keys, last tile

  // Tiles go straight from global memory into their LDS slot (global_load_lds_dwordx4: lane
  // i of a wave writes 16 bytes at the wave's LDS base + 16 i, a linear copy of the image).
  auto slot = [&](int t) { return smem + (t % kSlots) * kSlotBytes; };
  auto load = [&](int t) {
    const char* ks = kimg + (int64_t)t * kTileBytes;
    const char* vs = vimg + (int64_t)t * kTileBytes;
    char* dst = slot(t);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int off = p * kThreads * 16 + wave * 1024;  // wave-uniform LDS offset
      __builtin_amdgcn_global_load_lds(ks + off + lane * 16,
                                       (__attribute__((address_space(3))) void*)(dst + off), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds(
          vs + off + lane * 16,
          (__attribute__((address_space(3))) void*)(dst + kTileBytes + off), 16, 0, 0);
    }
  };
  // all of this thread's tile loads have landed in LDS
  auto loads_done = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ };

  const int krow = swap23(l32);
  const int l15 = l32 & 15;
  const int vx = vswz(l32);

  // QK of tile t into s.  kMask (the last tile): the C operand is -inf for keys >= tail;
  // register 4i+j of half kb holds key kb*32 + 16(i>>1) + 8hl + 4(i&1) + j.  Decided at
  // compile time so that no branch separates the products from the work they overlap.
  auto qk_tile = [&](f32x16* s, int t, auto mask_tag) {
    constexpr bool kMask = decltype(mask_tag)::value;
    const char* kl = slot(t);
    f32x16 c[2] = {w.negm, w.negm};
    if (kMask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kb * 32 + 16 * (i >> 1) + 8 * hl + 4 * (i & 1) + j;
            if (key >= tail) c[kb][4 * i + j] = -INFINITY;
          }
    }
    qk(w, s, kl, c, krow, l15, hl);
  };

  // One pipeline step for tile j: `cur` holds acc of tile j (max already applied), `nxt`
  // receives tile j+1.  kNext: tile j+1 exists; kMaskNext: it is the last tile.
  auto step = [&](f32x16* cur, f32x16* nxt, int j, auto next_tag, auto mask_tag) {
    constexpr bool kNext = decltype(next_tag)::value;
    if (j + 2 < nt) load(j + 2);               // into the slot tile j-1 left
    if (kNext) qk_tile(nxt, j + 1, mask_tag);  // B1
    ex(cur);
    cv(w, cur);                                // B2
    pv(w, slot(j) + kTileBytes, l32, vx, hl);
    if (kNext) mx<false>(w, nxt);
    loads_done();
    __syncthreads();
  };
  using T = std::true_type;
  using F = std::false_type;

  // ---- pipeline fill: tiles 0 and 1
  load(0);
  if (nt > 1) load(1);
  loads_done();
  __syncthreads();
  f32x16 sa[2], sb[2];
  if (nt == 1)
    qk_tile(sa, 0, T{});
  else
    qk_tile(sa, 0, F{});
  mx<true>(w, sa);
  // steady steps: tile j+1 exists and is not the last (j <= nt-3), two at a time
  int j = 0;
  for (; j + 4 <= nt; j += 2) {
    step(sa, sb, j, T{}, F{});
    step(sb, sa, j + 1, T{}, F{});
  }
  // the last one to three steps; `sa` holds the current tile here
  const int r = nt - j;
  if (r == 3) {
    step(sa, sb, j, T{}, F{});
    step(sb, sa, j + 1, T{}, T{});
    step(sa, sb, j + 2, F{}, F{});
  } else if (r == 2) {
    step(sa, sb, j, T{}, T{});
    step(sb, sa, j + 1, F{}, F{});
  } else {
    step(sa, sb, j, F{}, F{});
  }

  // ---- epilogue: lane holds O[row][d = db*32 + 8i + 4hl + j] at register 4i+j
  if (row < a.seq_buf) {
    const float inv = 1.0f / pair_sum(w.l);
    __bf16* orow = a.o + row * a.out_stride + hoff;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 v = {0u, 0u};  // rows in [N, S): exact +0
        if (row_valid) {
          v[0] = pack_bf16x2(w.o[db][4 * i] * inv, w.o[db][4 * i + 1] * inv);
          v[1] = pack_bf16x2(w.o[db][4 * i + 2] * inv, w.o[db][4 * i + 3] * inv);
        }
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * i + 4 * hl) = v;
      }
  }
}

}  // namespace h3
