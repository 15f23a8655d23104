// attention.hpp — dense non-causal softmax attention over the valid tokens of a packed,
// aligned buffer; software-pipelined for gfx950.
//
// Pages: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
// (Chinese translation of the vLLM blog post), §3.1: attention receives the valid
// sequence length and the structural tail padding is not computed; §3.2: the Q/K
// RMSNorm + RoPE prologue is fused (the Q half here, in registers).
//
// Where the time goes (measured on gfx950).  With 32 query rows per wave, every
// 32x32x16 MFMA consumes one 1 KiB operand read from LDS.  That is under half of what
// the LDS delivers (about 190 B per clock per CU with 8 waves), but the reads, the
// softmax VALU work and the MFMAs compete for issue: MFMA chains with both the reads and
// this kernel's VALU mix reach about 1,430 TFLOP/s in isolation, and this kernel adds
// the tile copies into LDS and one barrier per tile on top.  Holding 64 rows per wave
// halves the LDS reads per MFMA but needs one wave per SIMD, which leaves every barrier
// and memory wait unhidden; it measured slower.  Spreading the softmax work evenly over
// all 32 MFMA slots of a step, reading operands further ahead, spreading the tile
// copies over the step, or summing the rows with plain adds instead of
// v_dot2_f32_bf16 measured no faster either.
//
// The pipeline.  Two waves per SIMD; each wave interleaves the softmax of one 64-key
// tile with the matrix products of its neighbours.  Per tile j, for its 32 query rows:
//
//   B1: QK(j+1)  MFMA x16  ||  E(j), C(j) of the first groups   (fma + exp2, convert)
//   B2: PV(j)    MFMA x16  ||  C(j) of the last group, M(j+1) if checked
//       -- tile j+2 lands in LDS; barrier; the copy of tile j+3 starts --
//
// QK: S^T = K Q^T (two 32-key halves); M: row max of the new scores, raising the running
// max where it is exceeded (rare branch); E: p = exp2(c (s - m)); C: p -> bf16 operands
// and row sums; PV: O^T += V^T P^T.  The scores of tiles j and j+1 live in two register
// sets used alternately (loop unrolled by two).
//
// In the fast pass the second wave of each SIMD (waves 4-7) runs the same work in
// another order instead: per step its 32 MFMAs back to back (QK(j+1), PV(j)), then E and
// C of tile j+1 as one VALU block, with a single score set.  Paired with an interleaving
// wave, whose VALU work sits in its QK half, the two keep the matrix pipe busier than
// two interleaving waves do.
//
// Arithmetic.  Scores are exact bf16 products summed in fp32.  Two forms, chosen per
// launch from the factor the K tiles were stored with:
//  - prescaled K (the layer path: the pre-pass multiplies the normalised fp32 K rows by
//    c = softmax_scale * log2(e) before their one rounding to bf16): the QK
//    accumulation of a tile starts at -m, so the matrix cores return c s - m and
//    p = exp2 of it, with no per-score VALU work besides the exp2 (the fast pass);
//  - K as given (bf16 input, where scaling would round it a second time): the
//    accumulation starts at 0 and p = exp2(fma(s, c, -m c)), c applied in fp32.
// The running max m is raised only when a score exceeds it by more than kTauP / c, so
// p <= 2^8 and the O rescale is rare.  Keys >= N of the last tile get -inf scores.
// P is rounded to bf16 for the PV product, and the row sums add exactly
// those rounded values (v_dot2_f32_bf16 with (1, 1)), so every output row is a true
// weighted average of V rows; summing the unrounded fp32 p instead costs up to 2^-9
// relative error on strongly peaked rows.
//
// Memory.  Eight waves (256 query rows) share each K/V tile.  Tiles (prepared by
// kv_pack_kernel as padded 35 KiB images, layout in common.hpp) go through a 3-slot LDS
// ring: tile j is read from step j-1 (QK) to step j (PV).  Tile j+2 is copied
// global -> LDS directly (global_load_lds_dwordx4, no staging registers) during step j
// into the slot tile j-1 left, and waited for at the step's end, before its one
// barrier.  Every operand read is one base register plus an immediate offset.
// Everything fits in 256 VGPRs per lane, two waves per SIMD.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "prologue.hpp"

namespace h3 {

struct AttnArgs {
  const __bf16* q;
  __bf16* o;
  const char* img;        // packed K/V tile images, [head][tile]
  int64_t tiles_per_head;
  int64_t in_stride, out_stride;
  int64_t n_valid, seq_buf;
  int heads;
  int m_tiles;            // ceil(seq_buf / rows per workgroup)
  float scale_log2;       // softmax_scale * log2(e)
  int* wg_checked;        // per workgroup: 1 = left to the checked pass (Skip-Softmax
                          // launches: the wave tiles the workgroup skipped)
  float skip_log2;        // Skip-Softmax launches: log2 of the threshold
  // Key ranges per query block.  1: each workgroup takes every key and writes O.  k > 1:
  // workgroup (head, split, block) takes tiles [nt*split/k, nt*(split+1)/k) and writes
  // its unnormalised O (fp32, part + ((split*heads + head)*seq_buf + row)*128) and its
  // running maximum (log2 units) and row sum (part_ml, same index times 2);
  // attn_merge_kernel combines them.
  int splits;
  float* part;
  float* part_ml;
  // fused Q prologue
  const __bf16* w_q;
  int64_t w_head_stride;
  float eps;
  RopeArgs rope;
};

constexpr float kTauP = 8.0f;  // log2 units

namespace attn {

constexpr int kSlots = 3;                    // LDS ring depth (tiles)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;           // query rows per workgroup
constexpr int kImageChunks = kTileImageBytes / 1024;  // 1 KiB DMA chunks per tile (35)
static_assert(kTileImageBytes % 1024 == 0, "tile image must be whole 1 KiB chunks");

// 16 bytes per lane at LDS byte address base + off.  Operand addresses are formed as
// a scalar slot base plus one per-lane offset, with the constant part `off` folded into
// the read instruction's offset field.
__device__ __forceinline__ bf16x8 lds16(uint32_t base, int off) {
  typedef __attribute__((address_space(3))) const char lds_char;
  return *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(
      (lds_char*)(uintptr_t)base + off);
}

struct Wave {
  bf16x8 q[8];      // Q^T B operands
  f32x16 o[4];      // O^T accumulators per 32-channel block
  bf16x8 p[4];      // P^T B operands per 16-key step
  f32x16 nm;        // prescaled K: -m in every register, the QK accumulation's start
  float m;          // running max (raw score units)
  float nmc;        // -m * c, the exp2 offset
  float mt;         // m + kTauP / c: scores above it raise the running max
  float l;          // row-sum partial over this lane's keys
  float c;          // raw score units -> exp2 units (1 for prescaled K)
  float tau;        // kTauP / c: the running-max slack in raw units
};

// S^T (64 keys x 32 rows, as two 32-key halves).  `kb_base` = this lane's K operand
// address in the slot: key row l32, channel chunk hl; the (kb, ks) operand sits at
// + kb*32 rows + ks*32 bytes.
__device__ __forceinline__ void qk(const Wave& w, f32x16* s, uint32_t kb_base) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 a = lds16(kb_base, kb * 32 * kKRowPitch + ks * 32);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.q[ks], ks == 0 ? f32x16{} : s[kb], 0,
                                                      0, 0);
    }
  }
}

// O^T += V^T P^T.  `vb_base` = this lane's V operand address: channel row l32, key chunk hl;
// the (db, t) operand sits at + db*32 rows + t*32 bytes.
__device__ __forceinline__ void pv(Wave& w, uint32_t vb_base) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const bf16x8 a = lds16(vb_base, db * 32 * kVRowPitch + t * 32);
      w.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.p[t], w.o[db], 0, 0, 0);
    }
  }
}

// E: p = exp2(c (s - m)), in place.  kPre (K prescaled by c): the scores already are
// c s - m, and p = exp2(s).
template <bool kPre>
__device__ __forceinline__ float ex1(const Wave& w, float s) {
  return kPre ? __builtin_amdgcn_exp2f(s) : __builtin_amdgcn_exp2f(__builtin_fmaf(s, w.c, w.nmc));
}
template <bool kPre>
__device__ __forceinline__ void ex(const Wave& w, f32x16* s) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = ex1<kPre>(w, s[kb][e]);
}

// Set the running max to v where `need` (wave-uniform call); with kRescale, scale O and
// l by exp2(c (m_old - m_new)) for those rows.
template <bool kRescale>
__device__ __forceinline__ void raise_max(Wave& w, bool need, float v) {
  const float m_new = need ? v : w.m;
  if (kRescale) {
    const float alpha = __builtin_amdgcn_exp2f((w.m - m_new) * w.c);
    w.l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) w.o[db][e] *= alpha;
  }
  w.m = m_new;
  w.nmc = -m_new * w.c;
  w.mt = m_new + w.tau;
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

// Prescaled K (fast pass only): the scores of the first tile are made relative to the
// running max (shifted by -d = -m), and the QK accumulation of later tiles starts at -m.
__device__ __forceinline__ void shift_scores(Wave& w, f32x16* s, float d) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] -= d;
#pragma unroll
  for (int e = 0; e < 16; ++e) w.nm[e] = -w.m;
}

// M on the first tile: the running max starts at the tile's row max.
__device__ __forceinline__ void mx_first(Wave& w, const f32x16* s) {
  float v = s[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) v = fmaxf(v, s[kb][e]);
  raise_max<false>(w, true, pair_max(v));
}

// One steady-state step as an explicit instruction order.  kCheck: also take the row
// max of tile j+1 for the running-max check (not needed when the wave's scores are
// provably bounded, see the kernel).  QK(j+1) and PV(j) are 32
// MFMAs; after each MFMA comes the operand read of the MFMA three places later and the
// VALU work that the MFMA hides:
//   QK MFMA i:  exp2 of values 2i, 2i+1 of tile j; from i = 4 on, two convert/sum ops of
//               the 8-value group finished four MFMAs earlier;
//   PV MFMA i:  the last group's convert/sum ops (i < 4), one max3 of tile j+1's scores.
// A scheduling barrier after each group keeps the compiler from clustering the VALU
// work (which it otherwise does, leaving MFMAs waiting on reads and VALU unhidden).
template <bool kCheck, bool kPre>
__device__ __forceinline__ void steady_step(Wave& w, f32x16* cur, f32x16* nxt,
                                            uint32_t kbase, uint32_t vbase,
                                            float& vmax) {
  bf16x8 kop[16], vop[16];
  auto read_k = [&](int i) {  // operand of QK MFMA i: kb = i & 1, ks = i >> 1
    kop[i] = lds16(kbase, (i & 1) * 32 * kKRowPitch + (i >> 1) * 32);
  };
  auto read_v = [&](int i) {  // operand of PV MFMA i: t = i >> 2, db = i & 3
    vop[i] = lds16(vbase, (i & 3) * 32 * kVRowPitch + (i >> 2) * 32);
  };
  auto read = [&](int i) {  // operand i of the step's 32 MFMAs
    if (i < 16)
      read_k(i);
    else if (i < 32)
      read_v(i - 16);
  };
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float acc0 = w.l, acc1 = 0.0f;
  bf16x2 pr[4][4];
  // convert/sum op k (0..7) of 16-key group t: k < 4 converts pair k, k >= 4 adds it
  auto cv_op = [&](int t, int k) {
    if (k < 4) {
      const int i = k;
      const f32x2 f = {cur[t >> 1][8 * (t & 1) + 2 * i], cur[t >> 1][8 * (t & 1) + 2 * i + 1]};
      pr[t][i] = __builtin_convertvector(f, bf16x2);
    } else {
      const int i = k - 4;
      // the empty asm keeps the compiler from sinking the sum to the end of the step
      if (i & 1) {
        acc1 = __builtin_amdgcn_fdot2_f32_bf16(pr[t][i], ones, acc1, false);
        asm volatile("" : "+v"(acc1));
      } else {
        acc0 = __builtin_amdgcn_fdot2_f32_bf16(pr[t][i], ones, acc0, false);
        asm volatile("" : "+v"(acc0));
      }
      if (i == 3) {
        const bf16x8 pv8 = {pr[t][0][0], pr[t][0][1], pr[t][1][0], pr[t][1][1],
                            pr[t][2][0], pr[t][2][1], pr[t][3][0], pr[t][3][1]};
        w.p[t] = pv8;
      }
    }
  };
  read(0);
  read(1);
  read(2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // QK(j+1) || exp(j), convert/sum(j)
    const int kb = i & 1, ks = i >> 1;
    nxt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        kop[i], w.q[ks], ks == 0 ? (kPre ? w.nm : f32x16{}) : nxt[kb], 0, 0, 0);
    read(i + 3);
    cur[(2 * i) >> 4][(2 * i) & 15] = ex1<kPre>(w, cur[(2 * i) >> 4][(2 * i) & 15]);
    cur[(2 * i + 1) >> 4][(2 * i + 1) & 15] = ex1<kPre>(w, cur[(2 * i + 1) >> 4][(2 * i + 1) & 15]);
    if (i >= 4) {
      cv_op((i - 4) >> 2, 2 * ((i - 4) & 3));
      cv_op((i - 4) >> 2, 2 * ((i - 4) & 3) + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  float v = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // PV(j) || convert/sum(j), max(j+1)
    const int t = i >> 2, db = i & 3;
    w.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[i], w.p[t], w.o[db], 0, 0, 0);
    read(i + 19);
    if (i < 4) {
      cv_op(3, 2 * i);
      cv_op(3, 2 * i + 1);
    }
    if (kCheck) {  // tile j+1 scores: values 2i, 2i+1 of nxt
      v = fmaxf(fmaxf(v, nxt[(2 * i) >> 4][(2 * i) & 15]), nxt[(2 * i + 1) >> 4][(2 * i + 1) & 15]);
      asm volatile("" : "+v"(v));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  w.l = acc0 + acc1;
  vmax = v;
}

// MFMA-first form of a step (fast pass; see the kernel for which waves take it): the
// step's 32 MFMAs back to back, QK(j+1) into s (kNext) then PV(j) with the P operands of
// tile j, each operand read three MFMAs ahead; then (valu_block) the P operands and row
// sums of the new scores.  One score set suffices: a tile's scores become P operands
// before the next QK overwrites them.  kPre as in steady_step.
template <bool kNext, bool kPre, bool kPV = true>
__device__ __forceinline__ void mfma_block(Wave& w, f32x16* s, uint32_t kbase,
                                           uint32_t vbase) {
  constexpr int nq = kNext ? 16 : 0;
  constexpr int n = nq + (kPV ? 16 : 0);
  bf16x8 op[32];
  auto read = [&](int i) {
    if (i < nq) {
      op[i] = lds16(kbase, (i & 1) * 32 * kKRowPitch + (i >> 1) * 32);
    } else if (i < n) {
      const int k = i - nq;
      op[i] = lds16(vbase, (k & 3) * 32 * kVRowPitch + (k >> 2) * 32);
    }
  };
  read(0);
  read(1);
  read(2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < n; ++i) {
    if (i < nq) {
      const int kb = i & 1, ks = i >> 1;
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          op[i], w.q[ks], ks == 0 ? (kPre ? w.nm : f32x16{}) : s[kb], 0, 0, 0);
    } else {
      const int k = i - nq, t = k >> 2, db = k & 3;
      w.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], w.p[t], w.o[db], 0, 0, 0);
    }
    read(i + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool kPre>
__device__ __forceinline__ void valu_block(Wave& w, f32x16* s) {
  ex<kPre>(w, s);
  cv(w, s);
  __builtin_amdgcn_sched_barrier(0);
}

// valu_block of the multiply-add form with this row's exp2 offset `off` (-inf: the row
// drops the tile, so its P is exactly 0).
__device__ __forceinline__ void valu_block_off(Wave& w, f32x16* s, float off) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      s[kb][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], w.c, off));
  cv(w, s);
  __builtin_amdgcn_sched_barrier(0);
}

// Rest of M after steady_step: row max across the lane pair; raise the running max
// where it is exceeded by more than kTauP / c (rare branch).
__device__ __forceinline__ void mx_finish(Wave& w, float v) {
  v = pair_max(v);
  const bool need = v > w.mt;
  if (__builtin_amdgcn_ballot_w64(need)) raise_max<true>(w, need, v);
}

}  // namespace attn

// The 8 Q^T B operands of one query row (lane: channels 16ks + 8hl .. +8), as bf16;
// zeros for rows >= N.  With kFusedQ the row is RMS-normalised and rotated on the way,
// with the same helpers, operation order and pairwise-tree RMS sum as
// qk_norm_rope_kernel, so the values are the ones h3_qk_rmsnorm_rope writes.  All 64
// lanes must be active (lane pairs l, l^32 share the row).
template <bool kFusedQ>
__device__ __forceinline__ void load_q_operands(const AttnArgs& a, int64_t row, int head, int hl,
                                                const FreqTable* ft, bf16x8* q) {
  const bool row_valid = row < a.n_valid;
  const __bf16* qrow = a.q + row * a.in_stride + (int64_t)head * kHeadDim;
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
      norm_rotate_chunk(x, xp, wv, wpv, inv, cr, ft, y);
      raw[ks] = pack8(y);
    }
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) q[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
}

// Workgroups whose rows all lie in [N, S): write zeros (the caller returns after).
__device__ __forceinline__ void zero_rows(const AttnArgs& a, int64_t m0, int rows_per_wg,
                                          int head, int tid, int nthreads) {
  const int64_t rows = (a.seq_buf - m0) < rows_per_wg ? (a.seq_buf - m0) : rows_per_wg;
  const int64_t hoff = (int64_t)head * kHeadDim;
  for (int64_t i = tid; i < rows * kChunks; i += nthreads) {
    const int64_t r = m0 + i / kChunks;
    *reinterpret_cast<u32x4*>(a.o + r * a.out_stride + hoff + (i % kChunks) * 8) =
        u32x4{0u, 0u, 0u, 0u};
  }
}

// Largest K row norm over the head's nt tiles (from the tile images' pads), every lane.
__device__ __forceinline__ float head_kmax(const char* img, int nt, int lane) {
  float kmax = 0.0f;
  for (int t = lane; t < nt; t += 64)
    kmax = fmaxf(kmax, *reinterpret_cast<const float*>(img + (int64_t)t * kTileImageBytes +
                                                        kKNormOffset));
  for (int off = 32; off >= 1; off >>= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, off, 64));
  return kmax;
}

// |q|^2 of this lane's row from its 8 B operands (the other half comes from lane l^32).
__device__ __forceinline__ float q_norm2(const bf16x8* q) {
  float q2 = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) q2 = fmaf((float)q[ks][e], (float)q[ks][e], q2);
  return pair_sum(q2);
}

// kCheck = false: the fast pass; workgroups whose scores are not provably bounded are
// flagged in wg_checked and left alone.  kCheck = true: the second pass; runs the flagged
// workgroups with the per-tile running-max check and returns at once for the others.
// kSkip (with kCheck): dense attention with Skip-Softmax, a launch of its own that runs
// every workgroup (see skip_steps below).
template <bool kFusedQ, bool kCheck, bool kSkip = false>
__global__ __launch_bounds__(attn::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_fwd_kernel(AttnArgs a) {
  static_assert(kCheck || !kSkip, "Skip-Softmax runs in the checked pass's arithmetic");
  using namespace attn;
  __shared__ __attribute__((aligned(16))) char smem[kSlots * kTileImageBytes];
  __shared__ FreqTable ft;

  // logical workgroup = (head, split, query block), so the workgroups resident on one
  // XCD stream the same key range of one head
  const int logical = xcd_remap(blockIdx.x, a.heads * a.m_tiles * a.splits);
  const int hs = logical / a.m_tiles;
  const int head = hs / a.splits, split = hs % a.splits;
  const int64_t m0 = (int64_t)(logical % a.m_tiles) * kRows;
  const int tid = threadIdx.x;
  // the wave index is uniform across the wave: keep it in a scalar register
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hl = lane >> 5, l32 = lane & 31;
  const int64_t hoff = (int64_t)head * kHeadDim;

  const int wg = logical;
  if (kCheck && !kSkip && a.wg_checked[wg] == 0) return;  // done by the fast pass
  if (m0 >= a.n_valid) {  // rows past the valid length: zeros only (the merge writes
    if (tid == 0) a.wg_checked[wg] = 0;  // them when the keys are split)
    if (a.splits == 1) zero_rows(a, m0, kRows, head, tid, kThreads);
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

  load_q_operands<kFusedQ>(a, row, head, hl, &ft, w.q);
  w.m = 0.0f;
  w.nmc = 0.0f;
  w.mt = 0.0f;
  w.l = 0.0f;
#pragma unroll
  for (int db = 0; db < 4; ++db) w.o[db] = f32x16{};

  // this workgroup's key tiles [t_lo, t_hi) (all of them unless the keys are split; the
  // host keeps splits <= tiles, so every range holds at least one tile)
  const int nt_all = (int)((a.n_valid + kTileKeys - 1) / kTileKeys);
  const int t_lo = (int)((int64_t)nt_all * split / a.splits);
  const int t_hi = (int)((int64_t)nt_all * (split + 1) / a.splits);
  const int nt = t_hi - t_lo;
  const char* img = a.img + ((int64_t)head * a.tiles_per_head + t_lo) * kTileImageBytes;
  // valid keys of the range's last tile
  const int tail = t_hi == nt_all ? (int)(a.n_valid - (int64_t)(nt_all - 1) * kTileKeys)
                                  : kTileKeys;

  // The factor the stored K rows carry (tile 0's pad; the same for every tile).  When it
  // is c2 itself, the scores leave the matrix cores in exp2 units: the QK accumulation
  // then starts at -m and p = exp2(score), with no per-score multiply-add (kPre).
  const float kmul = __int_as_float(
      __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(img + kKMulOffset)));
  const bool prescaled = kmul == c2;
  w.c = prescaled ? 1.0f : c2 / kmul;
  w.tau = kTauP / w.c;

  // Tiles go straight from global memory into their LDS slot (global_load_lds_dwordx4:
  // lane i of a wave writes 16 bytes at the wave's LDS base + 16 i).  Only waves 0-3, one
  // per SIMD (waves w and w + 4 share a SIMD), issue copies: wave w < 4 copies the 1 KiB
  // chunks w, w + 4, ... of the 35 KiB image.  In the prescaled fast pass these are the
  // interleaving waves, and their MFMA-first partners then never stop for copy issue:
  // 2.4-3.2 % faster than copies from all eight waves in interleaved A/Bs (the same
  // output bits); copies from waves 4-7 gained 1.3 %, from waves 0-1 or 0, 2, 4, 6 lost.
  auto slot = [&](int t) __attribute__((always_inline)) { return smem + (t % kSlots) * kTileImageBytes; };
  // LDS byte address of tile t's slot, on the scalar unit
  const uint32_t smem_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  auto slot_addr = [&](int t) __attribute__((always_inline)) {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(smem_addr + ((unsigned)t % (unsigned)kSlots) * (unsigned)kTileImageBytes));
  };
  const uint32_t lane_off = lane * 16;
  constexpr int kCopyWaves = kWaves / 2;
  auto load = [&](int t) __attribute__((always_inline)) {
    if (wave >= kCopyWaves) return;
    const char* src = img + (int64_t)t * kTileImageBytes;
    char* dst = slot(t);
#pragma unroll
    for (int i = 0; i < (kImageChunks + kCopyWaves - 1) / kCopyWaves; ++i) {
      const int c = wave + i * kCopyWaves;
      if (c < kImageChunks)
        dma_to_lds16(src + c * 1024, lane_off,
                     (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(dst + c * 1024));
    }
  };
  // All of this thread's tile loads have landed in LDS (s_waitcnt vmcnt(0)).
  auto loads_done = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0x0F70); };


  // per-lane operand offsets within a slot (see qk / pv)
  const uint32_t k_lane = l32 * kKRowPitch + hl * 16;
  const uint32_t v_lane = kKImageBytes + l32 * kVRowPitch + hl * 16;

  // Keys >= tail of the last tile get -inf scores (so p = 0); register 4i+j of half kb
  // holds key kb*32 + 8i + 4hl + j.  Applied after the product, once per workgroup.
  auto mask_tail = [&](f32x16* s) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int key = kb * 32 + 8 * i + 4 * hl + jj;
          s[kb][4 * i + jj] = key >= tail ? -INFINITY : s[kb][4 * i + jj];
        }
  };

  // One pipeline step for tile j: `cur` holds acc of tile j (max already applied), `nxt`
  // receives tile j+1.  kNext: tile j+1 exists; kMask: it is the last tile.  The
  // choices are compile-time so that no branch separates the products from the work
  // they overlap.
  auto step = [&](f32x16* cur, f32x16* nxt, int j, auto next_tag, auto mask_tag,
                  auto check_tag, auto pre_tag) __attribute__((always_inline)) {
    constexpr bool kNext = decltype(next_tag)::value;
    constexpr bool kMask = decltype(mask_tag)::value;
    constexpr bool kChk = decltype(check_tag)::value;
    constexpr bool kPre = decltype(pre_tag)::value;
    static_assert(!(kChk && kPre), "the running max is never raised with prescaled K");
    if (j + kSlots - 1 < nt) load(j + kSlots - 1);  // into the slot tile j-1 left
    if (kNext) {
      float v;
      steady_step<kChk, kPre>(w, cur, nxt, slot_addr(j + 1) + k_lane, slot_addr(j) + v_lane, v);
      if (kMask) {
        mask_tail(nxt);
        if (kChk) {  // the max taken in the step saw the masked keys: take it again
          v = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) v = fmaxf(v, nxt[kb][e]);
        }
      }
      if (kChk) mx_finish(w, v);
    } else {  // last tile: no next scores
      ex<kPre>(w, cur);
      cv(w, cur);
      pv(w, slot_addr(j) + v_lane);
    }
    loads_done();  // tile j+2 in LDS before the next step
    __syncthreads();
  };
  using T = std::true_type;
  using F = std::false_type;

  // ---- pipeline fill: tiles 0 .. kSlots-2
#pragma unroll
  for (int t = 0; t < kSlots - 1; ++t)
    if (t < nt) load(t);
  loads_done();
  __syncthreads();
  f32x16 sa[2], sb[2];
  qk(w, sa, slot_addr(0) + k_lane);
  if (nt == 1) mask_tail(sa);
  mx_first(w, sa);  // the running max starts at tile 0's row max

  // Score bound.  Every score of this lane's row satisfies s <= |q| * max_j |k_j|
  // (Cauchy-Schwarz), and the running max starts at tile 0's row maximum m0, a lower
  // bound of the row's true maximum.  If c (|q| max|k| - m0) <= 64 for every row of the
  // workgroup, no exponent exceeds 64, the row's largest term is >= 1
  // (so l >= 1), and l <= 2^84 for up to 2^20 keys: the fp32 sums stay far from overflow
  // and, bf16 and fp32 precision being relative, the result is as accurate as with the
  // exact running max.  Then the fast pass runs without the per-tile max and its branch;
  // otherwise the workgroup is left to the checked pass.
  if (!kCheck) {
    const float kmax = head_kmax(img, nt, lane);
    const float bound = sqrtf(q_norm2(w.q)) * 1.0001f * kmax;
    const bool ok = (bound - w.m) * w.c <= 64.0f;  // false for NaN as well
    __shared__ int wave_fail[kWaves];
    if (lane == 0) wave_fail[wave] = __builtin_amdgcn_ballot_w64(!ok) != 0;
    __syncthreads();
    int fail = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) fail |= wave_fail[i];
    if (tid == 0) a.wg_checked[wg] = fail;
    if (fail) return;
  }

  // Steps.  Step j (tile j current, tile j+1 next) for j < nt-2 is a steady step; then
  // come step nt-2 (its next tile is the last, masked) and step nt-1 (no next tile).
  // The score sets alternate sa -> sb -> sa; for every path to reach the loop with the
  // current tile in sa and leave it with the same, an odd count of steady steps peels
  // one first.
  // kPre: the tile-0 scores are first made relative to the running max.
  using Check = std::integral_constant<bool, kCheck>;
  auto steps = [&](auto pre_tag) __attribute__((always_inline)) {
    using Pre = decltype(pre_tag);
    if (Pre::value) shift_scores(w, sa, w.m);
    if (nt == 1) {
      step(sa, sb, 0, F{}, F{}, Check{}, Pre{});
    } else {
      int j = 0;
      if (nt & 1) {
        step(sa, sb, 0, T{}, F{}, Check{}, Pre{});
        sa[0] = sb[0];
        sa[1] = sb[1];
        j = 1;
      }
      for (; j < nt - 2; j += 2) {
        step(sa, sb, j, T{}, F{}, Check{}, Pre{});
        step(sb, sa, j + 1, T{}, F{}, Check{}, Pre{});
      }
      step(sa, sb, nt - 2, T{}, T{}, Check{}, Pre{});
      step(sb, sa, nt - 1, F{}, F{}, Check{}, Pre{});
    }
  };
  // MFMA-first steps (fast pass): per step the 32 MFMAs, then the VALU work of the new
  // tile; exactly nt barriers, as in `steps`.
  auto mfma_first_steps = [&](auto pre_tag) __attribute__((always_inline)) {
    constexpr bool kPre = decltype(pre_tag)::value;
    static_assert(!(kCheck && kPre), "the running max is never raised with prescaled K");
    if (kPre) shift_scores(w, sa, w.m);
    auto kaddr = [&](int t) __attribute__((always_inline)) { return slot_addr(t) + k_lane; };
    auto vaddr = [&](int t) __attribute__((always_inline)) { return slot_addr(t) + v_lane; };
    auto body = [&](int j, auto mask_tag) __attribute__((always_inline)) {
      if (j + kSlots - 1 < nt) load(j + kSlots - 1);
      mfma_block<true, kPre>(w, sa, kaddr(j + 1), vaddr(j));
      if (decltype(mask_tag)::value) mask_tail(sa);
      if (kCheck) {  // M of tile j+1 (the maximum is exact, so the order does not matter)
        float v = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) v = fmaxf(v, sa[kb][e]);
        mx_finish(w, v);
      }
      valu_block<kPre>(w, sa);
      loads_done();
      __syncthreads();
    };
    valu_block<kPre>(w, sa);  // P operands of tile 0
    for (int j = 0; j < nt - 2; ++j) body(j, F{});
    if (nt >= 2) body(nt - 2, T{});
    mfma_block<false, kPre>(w, sa, 0, vaddr(nt - 1));
    loads_done();
    __syncthreads();
  };
  // Skip-Softmax ([Blog] §4.3, figure 6: a tile-level decision from the QK result drops
  // the softmax and P V work of unimportant tiles): tile t >= 1 is dropped for a row when
  // exp(tile max - running max of the kept tiles) < threshold.  The checked pass's
  // arithmetic with, besides its lazy running max (the exp2 reference), the exact running
  // max of the kept tiles for the decision; a dropping row gets P = 0 for the tile
  // (exp2 offset -inf) and keeps its maxima.  Every wave runs the MFMA-first step, whose
  // VALU block and PV products stand apart from the QK products: when all 32 rows of a
  // wave drop a tile, the wave skips that tile's VALU block and its 16 PV MFMAs.  Rows
  // >= N always drop, so they never hold a wave back.
  uint32_t skipped = 0;  // wave tiles this wave skipped
  auto skip_steps = [&]() __attribute__((always_inline)) {
    auto kaddr = [&](int t) __attribute__((always_inline)) { return slot_addr(t) + k_lane; };
    auto vaddr = [&](int t) __attribute__((always_inline)) { return slot_addr(t) + v_lane; };
    float mx = w.m;         // exact running max of the kept tiles (tile 0's row max)
    bool skip_all = false;  // the whole wave drops the tile whose P is in w.p
    auto body = [&](int j, auto mask_tag) __attribute__((always_inline)) {
      if (j + kSlots - 1 < nt) load(j + kSlots - 1);
      if (skip_all)
        mfma_block<true, false, false>(w, sa, kaddr(j + 1), 0);
      else
        mfma_block<true, false>(w, sa, kaddr(j + 1), vaddr(j));
      if (decltype(mask_tag)::value) mask_tail(sa);
      float v = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) v = fmaxf(v, sa[kb][e]);
      v = pair_max(v);
      const bool skip = !row_valid || (v - mx) * w.c < a.skip_log2;
      skip_all = __builtin_amdgcn_ballot_w64(!skip) == 0;
      skipped += skip_all ? 1u : 0u;
      if (!skip) mx = fmaxf(mx, v);
      const bool need = !skip && v > w.mt;  // a dropped tile never raises the maximum
      if (__builtin_amdgcn_ballot_w64(need)) raise_max<true>(w, need, v);
      if (!skip_all) valu_block_off(w, sa, skip ? -INFINITY : w.nmc);
      loads_done();
      __syncthreads();
    };
    valu_block<false>(w, sa);  // tile 0 is always kept
    for (int j = 0; j < nt - 2; ++j) body(j, F{});
    if (nt >= 2) body(nt - 2, T{});
    if (!skip_all) mfma_block<false, false>(w, sa, 0, vaddr(nt - 1));
    loads_done();
    __syncthreads();
  };

  // Fast pass: waves 0-3 take the interleaved steps and waves 4-7 the MFMA-first ones.
  // A workgroup's waves are placed on the SIMDs in turn, so waves w and w + 4 share a
  // SIMD: while one runs the exp2 work that the interleaved form packs into its QK half,
  // the other keeps the matrix pipe busy (prescaled K: 1.1-1.3 % faster than both waves
  // interleaved; the multiply-add form, with the copies from waves 0-3: 1.7 %; in
  // interleaved A/Bs, the same output bits).  The checked pass pairs its waves the same
  // way and takes the multiply-add path for either kind of K (c = 1 for prescaled K):
  // the rare raise of the running max needs registers the kPre path would spill.
  if constexpr (kSkip) {
    skip_steps();
    __shared__ uint32_t wave_skipped[kWaves];
    if (lane == 0) wave_skipped[wave] = skipped;
    __syncthreads();
    if (tid == 0) {
      uint32_t total = 0;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) total += wave_skipped[i];
      a.wg_checked[wg] = (int)total;
    }
  } else if constexpr (!kCheck) {
    if (prescaled) {
      if (wave >= kWaves / 2)
        mfma_first_steps(T{});
      else
        steps(T{});
    } else {
      if (wave >= kWaves / 2)
        mfma_first_steps(F{});
      else
        steps(F{});
    }
  } else {
    if (wave >= kWaves / 2)
      mfma_first_steps(F{});
    else
      steps(F{});
  }

  // ---- epilogue: lane holds O[row][d = db*32 + 8i + 4hl + j] at register 4i+j
  if (a.splits > 1) {  // this key range's partial result; rows >= N are the merge's
    if (row_valid) {
      const float l = pair_sum(w.l);
      const int64_t idx = ((int64_t)split * a.heads + head) * a.seq_buf + row;
      float* po = a.part + idx * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<f32x4*>(po + db * 32 + 8 * i + 4 * hl) =
              f32x4{w.o[db][4 * i], w.o[db][4 * i + 1], w.o[db][4 * i + 2], w.o[db][4 * i + 3]};
      if (hl == 0) *reinterpret_cast<f32x2*>(a.part_ml + 2 * idx) = f32x2{w.m * w.c, l};
    }
    return;
  }
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

// Combines the key ranges of a split launch: per (row, head), with m_s and l_s the
// ranges' running maxima (log2 units) and row sums and O_s their unnormalised outputs,
// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s, the ranges taken in
// order (deterministic); rows in [N, S) get zeros.  16 rows x 16 chunks of 8 channels
// per 256-thread workgroup.
struct MergeArgs {
  const float* part;
  const float* part_ml;
  __bf16* o;
  int64_t out_stride;
  int64_t n_valid, seq_buf;
  int heads, splits;
};

__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int head = blockIdx.y, cc = threadIdx.x & 15;
  if (row >= a.seq_buf) return;
  u32x4 res = {0u, 0u, 0u, 0u};
  if (row < a.n_valid) {
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s)
      mx = fmaxf(mx, a.part_ml[2 * (((int64_t)s * a.heads + head) * a.seq_buf + row)]);
    float l = 0.0f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.splits; ++s) {
      const int64_t idx = ((int64_t)s * a.heads + head) * a.seq_buf + row;
      const f32x2 ml = *reinterpret_cast<const f32x2*>(a.part_ml + 2 * idx);
      const float f = __builtin_amdgcn_exp2f(ml[0] - mx);
      l = __builtin_fmaf(f, ml[1], l);
      const f32x4* po = reinterpret_cast<const f32x4*>(a.part + idx * kHeadDim + cc * 8);
      const f32x4 lo = po[0], hi = po[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = __builtin_fmaf(f, lo[e], acc[e]);
        acc[4 + e] = __builtin_fmaf(f, hi[e], acc[4 + e]);
      }
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    res = pack8(acc);
  }
  *reinterpret_cast<u32x4*>(a.o + row * a.out_stride + (int64_t)head * kHeadDim + cc * 8) = res;
}

}  // namespace h3
