// attention_fp8.hpp — the FP8 ("SAGE") variant of the attention: Q, K, P and V in FP8
// E4M3 for both products, on the gfx950 matrix cores' FP8 instruction (32x32x64, twice
// the bf16 rate).
//
// Pages: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
// (Chinese translation of the vLLM blog post), §4.3 and figure 6: SAGE quantizes Q, K,
// P and V to FP8 for the QK and PV products; the post's draft pull request calls the
// measured configuration "K16".
//
// What is computed (the readings of what the pages leave open):
//   Q: one scale per token, amax/448, applied in registers on load (after the fused
//      RMSNorm + RoPE when it is on);  K: one scale per block of 16 keys ("K16"),
//      computed by the pre-pass; V: one scale per channel over the valid tokens (a
//      separate max pass); every code is the E4M3 rounding (to nearest, ties to even) of
//      the exact x * 448 / amax (see quant4 for why the arithmetic used decides it
//      exactly).
//   P: the weights of a streaming softmax: per 64-key tile t, with m_t the running row
//      maximum of the scaled scores through tile t (log2 units, c = softmax_scale *
//      log2(e) * sq * sk), P = E4M3(2^(8 + c s - m_t)) <= 256; O and the row sums are
//      carried to a new maximum by 2^(m_(t-1) - m_t).  The row sums are the sums of the
//      quantized P, taken by one extra matrix product of P with an all-ones operand
//      (FP4 E2M1 ones, exact, half the registers of FP8 ones).
//   O = s_v * (P V) / l, rounded to bf16; rows in [N, S) are zero.
//   Skip-Softmax (same section: tiles judged unimportant from the QK result skip the
//      softmax and the P V product; a higher threshold skips more): with threshold
//      lambda, tile t >= 1 is dropped for a row when 2^(tile max - m_(t-1)) < lambda
//      (scaled scores in log2 units, m_(t-1) the running maximum before the tile); the
//      row's P for that tile is then 0 and its maximum unchanged.  A wave whose 32 rows
//      all drop a tile skips that tile's softmax, PV and row-sum products.
//
// FP8 tile image (64 keys, 19,456 bytes):
//   K part: key r, channel c at byte r*144 + c (128 bytes of codes + 16 bytes pad; row
//           0's pad holds the four 16-key block scales as floats, the others are zero);
//   V part: channel d at byte 9216 + d*80: bytes 32h + b (h = 0, 1; b = 0..31) hold the
//           code of key 32(b/16) + 8((b%16)/4) + 4h + b%4 (the order in which the QK
//           product leaves P in a lane's registers), then 16 bytes of pad.
// The FP8 product's reduction dimension may be ordered freely within a lane as long as
// both operands agree (measured); these orders make both products shuffle free.
#pragma once

#include "attention.hpp"

namespace h3 {
namespace fp8 {

typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int kKPitch = kHeadDim + 16;          // 144
constexpr int kVPitch = kTileKeys + 16;         // 80
constexpr int kKBytes = kTileKeys * kKPitch;    // 9,216
constexpr int kVBytes = kHeadDim * kVPitch;     // 10,240
constexpr int kTileBytes = kKBytes + kVBytes;   // 19,456 = 19 KiB
constexpr int kScaleOffset = kHeadDim;          // K row 0's pad: 4 block scales
constexpr int kImgChunks = kTileBytes / 1024;   // 19 DMA chunks
static_assert(kTileBytes % 1024 == 0, "FP8 tile image must be whole 1 KiB chunks");
constexpr float kMax = 448.0f;                  // largest finite E4M3

// Two fp32 values -> E4M3 codes (round to nearest even) in bytes 2w, 2w+1 of `old`.
template <bool kHi>
__device__ __forceinline__ uint32_t cvt2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHi);
}

// Inverse of a group's scale for quant4: 448 / amax in fp64 (0 for an all-zero group).
__device__ __forceinline__ double code_inverse(float amax) {
  return amax > 0.0f ? 448.0 / (double)amax : 0.0;
}

// Four values of one group -> one dword of E4M3 codes (byte i = value i), each code the
// rounding to nearest even of the exact t = x * 448 / amax.  x and amax are bf16 values
// (at most 8 significant bits), so t is either exactly an E4M3 rounding midpoint or at
// least 2^-14 of its magnitude away from every midpoint (with x = X 2^a, amax = A 2^b,
// X and A odd and below 256, t - M 2^e is a multiple of 2^min(a-b+6, e) over A, and
// M < 32 for any neighbouring midpoint M 2^e).  Formed as an fp64 product with the fp64
// inverse (relative error below 2^-51) and rounded once to fp32 (2^-24): a midpoint, with
// its 5 significant bits, comes back exactly and the conversion breaks the tie to even;
// any other t stays on its side of every midpoint.  |t| <= 448, so no clamp is needed;
// the conversion is exact on [-448, 448].
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, double inv) {
  auto q = [&](float x) { return (float)((double)x * inv); };
  return cvt2<true>(q(c), q(d), cvt2<false>(q(a), q(b), 0u));
}

// Column sums of b: FP4 (E2M1) A operand `ones` x E4M3 B, unit scales.
__device__ __forceinline__ f32x16 mfma_ones(i32x8 ones, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, b, c, 4, 0, 0, 127, 0, 127);
}

// max(a, b) for scores that are finite or -inf: the NaN-propagating maximum
// (v_maximum3_f32) then equals fmaxf, and unlike fmaxf needs no input canonicalization.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// vmax over the lane pair (l, l ^ 32); identical bits in both lanes.
__device__ __forceinline__ float pair_vmax(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                            false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  // E4M3 x E4M3, no block scaling (unit E8M0 scales)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

}  // namespace fp8

// ---------------------------------------------------------------------------------
// Pre-passes: per-channel V amax, then the FP8 tile images.

// dst[i] = 0 for i < n (graph-capturable clear).
__global__ void fill_zero_kernel(uint32_t* dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = 0u;
}

struct Fp8StatsArgs {
  const __bf16* v;
  int64_t in_stride;
  int64_t n_valid;
  uint32_t* vamax;  // [head][128] as float bits (non-negative floats order as integers)
};

constexpr int kStatKeys = 512;  // keys per workgroup of v_amax_kernel

// 512 keys of one head per workgroup, 256 threads (16 lanes per 256-byte row, 16 rows
// per pass): the largest |V| of each channel, reduced in LDS, then merged across
// workgroups with atomicMax (order independent, so the result is deterministic).
__global__ __launch_bounds__(256) void v_amax_kernel(Fp8StatsArgs a) {
  const int64_t key0 = (int64_t)blockIdx.x * kStatKeys;
  const int h = blockIdx.y, tid = threadIdx.x, cc = tid & 15, rg = tid >> 4;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = rg; r < kStatKeys; r += 16) {
    const int64_t key = key0 + r;
    if (key < a.n_valid) {
      float x[8];
      unpack8(*reinterpret_cast<const u32x4*>(a.v + key * a.in_stride + (int64_t)h * kHeadDim +
                                              cc * 8),
              x);
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(x[i]));
    }
  }
  __shared__ float red[16][kHeadDim];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rg][cc * 8 + i] = m[i];
  __syncthreads();
  if (tid < kHeadDim) {
    float mm = 0.0f;
#pragma unroll
    for (int g = 0; g < 16; ++g) mm = fmaxf(mm, red[g][tid]);
    if (mm > 0.0f) atomicMax(a.vamax + h * kHeadDim + tid, __float_as_uint(mm));
  }
}

struct Fp8PackArgs {
  const __bf16* k;
  const __bf16* v;
  const __bf16* w_k;
  int64_t w_head_stride;
  int64_t in_stride;
  int64_t n_valid;
  int64_t tiles_per_head;
  float eps;
  RopeArgs rope;
  const uint32_t* vamax;  // [head][128]
  char* img;              // [head][tile] x fp8::kTileBytes
};

// One 64-key tile of one head per workgroup, 256 threads: K rows (normalised and
// rotated when kNorm, rounded to bf16 as the bf16 path does) and V rows staged in LDS,
// then K quantized per 16-key block and V per channel into the image.
template <bool kNorm>
__global__ __launch_bounds__(256) void kv_pack_fp8_kernel(Fp8PackArgs a) {
  using namespace fp8;
  const int64_t kt = blockIdx.x;
  const int h = blockIdx.y, tid = threadIdx.x;
  __shared__ FreqTable ft;
  __shared__ __attribute__((aligned(16))) __bf16 ks[kTileKeys][kHeadDim];
  __shared__ __attribute__((aligned(16))) __bf16 vs[kTileKeys][kHeadDim];
  if (kNorm) {
    fill_freq_table(&ft, a.rope, tid, blockDim.x);
    __syncthreads();
  }
  const int64_t key0 = kt * kTileKeys;
  const int64_t hoff = (int64_t)h * kHeadDim;
  char* img = a.img + ((int64_t)h * a.tiles_per_head + kt) * kTileBytes;

  // stage K (16 lanes per row, 16 rows per pass) and V (same shape)
  const int cc = tid & 15;
  for (int r = tid >> 4; r < kTileKeys; r += 16) {
    const int64_t key = key0 + r;
    u32x4 kout = {0u, 0u, 0u, 0u}, vout = {0u, 0u, 0u, 0u};
    if (key < a.n_valid) {  // the whole 16-lane row group takes the same branch
      const __bf16* row = a.k + key * a.in_stride + hoff;
      if (kNorm) {
        const ChunkRot cr = chunk_rotation(a.rope, key, cc);
        float y[8];
        norm_rotate_row16(row, a.w_k + (int64_t)h * a.w_head_stride, a.eps, cr, cc, &ft, y);
        kout = pack8(y);
      } else {
        kout = *reinterpret_cast<const u32x4*>(row + cc * 8);
      }
      vout = *reinterpret_cast<const u32x4*>(a.v + key * a.in_stride + hoff + cc * 8);
    }
    *reinterpret_cast<u32x4*>(&ks[r][cc * 8]) = kout;
    *reinterpret_cast<u32x4*>(&vs[r][cc * 8]) = vout;
  }
  __syncthreads();

  // K: wave w quantizes block w (keys 16w .. 16w+15); lane: key 16w + lane/4, channels
  // 32 (lane%4) .. +32
  {
    const int w = tid >> 6, lane = tid & 63;
    const int r = 16 * w + (lane >> 2), c0 = 32 * (lane & 3);
    float x[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack8(*reinterpret_cast<const u32x4*>(&ks[r][c0 + 8 * i]), x + 8 * i);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(x[i]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const double inv = code_inverse(m);
    u32x4 q0, q1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q0[i] = quant4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3], inv);
      q1[i] = quant4(x[16 + 4 * i], x[16 + 4 * i + 1], x[16 + 4 * i + 2], x[16 + 4 * i + 3], inv);
    }
    *reinterpret_cast<u32x4*>(img + r * kKPitch + c0) = q0;
    *reinterpret_cast<u32x4*>(img + r * kKPitch + c0 + 16) = q1;
    __shared__ float bscale[4];
    if (lane == 0) bscale[w] = m / kMax;
    __syncthreads();
    if (tid < kTileKeys) {  // row pads: row 0 carries the four block scales
      u32x4 pad = {0u, 0u, 0u, 0u};
      if (tid == 0)
        pad = u32x4{__float_as_uint(bscale[0]), __float_as_uint(bscale[1]),
                    __float_as_uint(bscale[2]), __float_as_uint(bscale[3])};
      *reinterpret_cast<u32x4*>(img + tid * kKPitch + kScaleOffset) = pad;
    }
  }

  // V: thread (channel d, half hh) writes the 32 codes of bytes 32hh .. 32hh+31
  {
    const int d = tid >> 1, hh = tid & 1;
    const float amax = __uint_as_float(a.vamax[h * kHeadDim + d]);
    const double inv = code_inverse(amax);
    float x[32];
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      const int key = 32 * (b >> 4) + 8 * ((b & 15) >> 2) + 4 * hh + (b & 3);
      x[b] = (float)vs[key][d];
    }
    u32x4 q0, q1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q0[i] = quant4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3], inv);
      q1[i] = quant4(x[16 + 4 * i], x[16 + 4 * i + 1], x[16 + 4 * i + 2], x[16 + 4 * i + 3], inv);
    }
    char* vrow = img + kKBytes + d * kVPitch;
    *reinterpret_cast<u32x4*>(vrow + 32 * hh) = q0;
    *reinterpret_cast<u32x4*>(vrow + 32 * hh + 16) = q1;
    if (hh == 0) *reinterpret_cast<u32x4*>(vrow + 64) = u32x4{0u, 0u, 0u, 0u};
  }
}

// ---------------------------------------------------------------------------------
// Attention.

struct Fp8AttnArgs {
  const __bf16* q;
  __bf16* o;
  const char* img;          // FP8 tile images, [head][tile]
  const uint32_t* vamax;    // [head][128]
  int64_t tiles_per_head;
  int64_t in_stride, out_stride;
  int64_t n_valid, seq_buf;
  int heads;
  int m_tiles;              // ceil(seq_buf / 256)
  float scale_log2;         // softmax_scale * log2(e)
  const __bf16* w_q;        // fused Q prologue (NULL: Q used as is)
  int64_t w_head_stride;
  float eps;
  RopeArgs rope;
  float skip_log2;          // log2(Skip-Softmax threshold); -inf: never skip
  uint32_t* skipped;        // [head * m_tiles]: wave tiles skipped by each workgroup
};

namespace fp8 {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;
constexpr int kSlots = 3;

struct Wave {
  i32x8 q[2];        // Q codes, B operand: channels 64 ks + 32 hl + b at byte b
  f32x16 o[4];       // O^T accumulators per 32-channel block
  f32x16 l;          // row sums (every register holds the lane's row sum)
  i32x8 p;           // P codes, B operand (byte b = value b of the tile, see the image)
  float m;           // running max (log2 units)
  float c;           // softmax_scale * log2(e) * sq (this row's Q scale)
  bool skip;         // this row drops the current tile (Skip-Softmax)
  bool skip_all;     // every row of the wave drops it (wave-uniform)
  uint32_t skipped;  // wave tiles skipped so far
};

}  // namespace fp8

// 8 waves x 32 query rows per workgroup, two waves per SIMD; per 64-key tile and wave:
// 4 QK products, the softmax of the previous tile, 4 PV products and the row-sum
// product.  One barrier per tile; tiles are copied global -> LDS into a 3-slot ring.
// Waves 0-3 interleave the softmax of tile j with the QK products of tile j+1; their
// SIMD partners (waves 4-7) run the same arithmetic MFMA-first: the step's 9 products
// back to back, then the max and P codes of the new tile as one VALU block.  Two
// interleaving waves on a SIMD want the VALU at the same time and the younger one waits
// (the older wave wins issue); the MFMA-first partner takes the matrix pipe while the
// interleaving wave runs its softmax.  Same operations in the same order per row, so
// the same output bits.
template <bool kFusedQ, bool kSkip>
__global__ __launch_bounds__(fp8::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_fp8_kernel(Fp8AttnArgs a) {
  using namespace fp8;
  __shared__ __attribute__((aligned(16))) char smem[kSlots * kTileBytes];
  __shared__ FreqTable ft;

  const int logical = xcd_remap(blockIdx.x, a.heads * a.m_tiles);
  const int head = logical / a.m_tiles;
  const int64_t m0 = (int64_t)(logical % a.m_tiles) * kRows;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hl = lane >> 5, l32 = lane & 31;
  const int64_t hoff = (int64_t)head * kHeadDim;
  if (m0 >= a.n_valid) {  // rows past the valid length: zeros only
    if (tid == 0) a.skipped[logical] = 0u;
    const int64_t rows = (a.seq_buf - m0) < kRows ? (a.seq_buf - m0) : kRows;
    for (int64_t i = tid; i < rows * h3::kChunks; i += kThreads) {
      const int64_t r = m0 + i / h3::kChunks;
      *reinterpret_cast<u32x4*>(a.o + r * a.out_stride + hoff + (i % h3::kChunks) * 8) =
          u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  if (kFusedQ) {
    fill_freq_table(&ft, a.rope, tid, kThreads);
    __syncthreads();
  }

  Wave w;
  const int64_t row = m0 + wave * 32 + l32;
  // ---- Q: bf16 operands as the bf16 path builds them (lane half hl holds chunks
  // 2k + hl), regrouped so that half hl holds chunks 4hl..4hl+3 and 8+4hl..8+4hl+3,
  // then quantized with the row's scale.
  {
    AttnArgs qa{};
    qa.q = a.q;
    qa.in_stride = a.in_stride;
    qa.n_valid = a.n_valid;
    qa.w_q = a.w_q;
    qa.w_head_stride = a.w_head_stride;
    qa.eps = a.eps;
    qa.rope = a.rope;
    bf16x8 qb[8];
    load_q_operands<kFusedQ>(qa, row, head, hl, &ft, qb);
    // Half h holds chunks 2s + h in slot s; the FP8 product wants chunks 8ks + 4h + i
    // (i = 0..3) in half h.  v_permlane32_swap of slots (4ks + p, 4ks + 2 + p) swaps
    // the upper half of the first with the lower half of the second, which leaves
    // chunk i = 2p in the first result and i = 2p + 1 in the second, in both halves.
    float x[2][32];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const u32x4 lo = __builtin_bit_cast(u32x4, qb[4 * ks + pp]);
        const u32x4 hi = __builtin_bit_cast(u32x4, qb[4 * ks + 2 + pp]);
        u32x4 first, second;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto r = __builtin_amdgcn_permlane32_swap(lo[e], hi[e], false, false);
          first[e] = r[0];
          second[e] = r[1];
        }
        unpack8(first, &x[ks][16 * pp]);
        unpack8(second, &x[ks][16 * pp + 8]);
      }
    float amax = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[ks][i]));
    amax = pair_max(amax);
    const double inv = code_inverse(amax);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w.q[ks][i] = (int)quant4(x[ks][4 * i], x[ks][4 * i + 1], x[ks][4 * i + 2],
                                 x[ks][4 * i + 3], inv);
    w.c = a.scale_log2 * (amax / kMax);
  }
  w.m = -INFINITY;
  w.skip = false;
  w.skip_all = false;
  w.skipped = 0u;
  const bool row_valid = row < a.n_valid;
#pragma unroll
  for (int db = 0; db < 4; ++db) w.o[db] = f32x16{};
  w.l = f32x16{};
  // the row-sum product's A operand: 1.0 in FP4 E2M1 (code 0x2) in every nibble; an FP4
  // operand occupies the first 4 dwords
  const i32x8 ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};

  const int nt = (int)((a.n_valid + kTileKeys - 1) / kTileKeys);
  const char* img = a.img + (int64_t)head * a.tiles_per_head * kTileBytes;
  const int tail = (int)(a.n_valid - (int64_t)(nt - 1) * kTileKeys);

  // LDS byte address of tile t's slot, kept on the scalar unit; operand reads add one
  // per-lane offset to it and fold their constant offsets into the read instruction
  typedef __attribute__((address_space(3))) const char lds_char;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  auto slot_addr = [&](int t) __attribute__((always_inline)) {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(smem_addr + ((unsigned)t % (unsigned)kSlots) * (unsigned)kTileBytes));
  };
  auto slot = [&](int t) __attribute__((always_inline)) {
    return smem + ((unsigned)t % (unsigned)kSlots) * (unsigned)kTileBytes;
  };
  const uint32_t lane_off = lane * 16;
  // Copies from waves 0-3 only, one per SIMD, as in the bf16 kernel (+1.2 % in an
  // interleaved A/B, the same output bits).
  constexpr int kCopyWaves = kWaves / 2;
  auto load = [&](int t) __attribute__((always_inline)) {
    if (wave >= kCopyWaves) return;
    const char* src = img + (int64_t)t * kTileBytes;
    const uint32_t dst = slot_addr(t);
#pragma unroll
    for (int i = 0; i < (kImgChunks + kCopyWaves - 1) / kCopyWaves; ++i) {
      const int c = wave + i * kCopyWaves;
      if (c < kImgChunks) dma_to_lds16(src + c * 1024, lane_off, dst + c * 1024);
    }
  };
  auto loads_done = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0x0F70); };
  // per-lane operand offsets within a slot
  const uint32_t k_lane = l32 * kKPitch + 32 * hl;
  const uint32_t v_lane = kKBytes + l32 * kVPitch + 32 * hl;
  // 32 bytes at LDS address base + off (off a compile-time constant after unrolling)
  auto read32 = [&](uint32_t base, int off) __attribute__((always_inline)) {
    lds_char* p = (lds_char*)(uintptr_t)base + off;
    const u32x4 lo = *reinterpret_cast<__attribute__((address_space(3))) const u32x4*>(p);
    const u32x4 hi = *reinterpret_cast<__attribute__((address_space(3))) const u32x4*>(p + 16);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // S^T of tile t: s[kb] (32 keys x 32 rows), register 4i+j = key kb*32 + 8i + 4hl + j
  auto qk = [&](f32x16* s, int t) __attribute__((always_inline)) {
    const uint32_t kb0 = slot_addr(t) + k_lane;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = fp8::mfma8(read32(kb0, kb * 32 * kKPitch), w.q[0], f32x16{});
      s[kb] = fp8::mfma8(read32(kb0, kb * 32 * kKPitch + 64), w.q[1], s[kb]);
    }
  };
  // per-register multipliers c * sk(block): registers 0-7 of half kb are block 2kb,
  // 8-15 block 2kb+1
  auto block_c = [&](int t, float* cb) __attribute__((always_inline)) {
    const u32x4 sc = *reinterpret_cast<const u32x4*>(slot(t) + kScaleOffset);
#pragma unroll
    for (int b = 0; b < 4; ++b) cb[b] = w.c * __uint_as_float(sc[b]);
  };
  // key of register r of half kb (this lane's half hl)
  auto key_of = [&](int kb, int r) __attribute__((always_inline)) {
    return kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
  };
  // Row max of tile t's scaled scores; raise the running max where the tile exceeds it
  // (wave-uniform branch), carrying O and the row sums over to the new maximum.  kMask (the
  // last tile): keys >= tail are left out, after scaling, since a block with no valid
  // key has scale 0.  Block scales are >= 0, so max(s) * c is the max of s * c.
  auto update_max = [&](const f32x16* s, const float* cb, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    float v = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        if (kMask) {
#pragma unroll
          for (int r = 8 * g; r < 8 * g + 8; ++r)
            v = fmaxf(v, key_of(kb, r) < tail ? s[kb][r] * cb[2 * kb + g] : -INFINITY);
        } else {
          float gm = s[kb][8 * g];
#pragma unroll
          for (int r = 8 * g + 1; r < 8 * g + 8; ++r) gm = fp8::vmax(gm, s[kb][r]);
          v = fp8::vmax(v, gm * cb[2 * kb + g]);
        }
      }
    v = fp8::pair_vmax(v);
    if (kSkip) {  // decided against the maximum before this tile; rows >= N never block
      w.skip = !row_valid || v < w.m + a.skip_log2;
      w.skip_all = __builtin_amdgcn_ballot_w64(!w.skip) == 0;
    }
    const bool need = v > w.m;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? v : w.m;
      const float alpha = __builtin_amdgcn_exp2f(w.m - m_new);  // 0 on the first tile
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) w.o[db][e] *= alpha;
#pragma unroll
      for (int e = 0; e < 16; ++e) w.l[e] *= alpha;
      w.m = m_new;
    }
  };
  // P codes of one 32-key half kb of a tile: 2^(8 + s c - m) <= 256;
  // kMask: keys >= tail get 0.  Writes bytes 16kb .. 16kb+15 of the P operand.
  auto softmax_half = [&](const f32x16& s, const float* cb, int kb, auto mask_tag)
      __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    // a row that drops the tile gets p = exp2(-inf) = 0
    const float off = (kSkip && w.skip) ? -INFINITY : 8.0f - w.m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float p[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 4 * i + jj;
        const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], cb[2 * kb + (r >> 3)], off));
        p[jj] = (kMask && key_of(kb, r) >= tail) ? 0.0f : x;
      }
      // both halves of the word are written: the previous codes serve as the untouched
      // half of the first conversion, which saves clearing a register
      w.p[4 * kb + i] = (int)fp8::cvt2<true>(
          p[2], p[3], fp8::cvt2<false>(p[0], p[1], (uint32_t)w.p[4 * kb + i]));
    }
  };

  // O^T += V^T P^T and the row sums l += 1^T P^T (exact sums of the quantized weights)
  auto pv = [&](int t) __attribute__((always_inline)) {
    const uint32_t vb = slot_addr(t) + v_lane;
#pragma unroll
    for (int db = 0; db < 4; ++db) w.o[db] = fp8::mfma8(read32(vb, db * 32 * kVPitch), w.p, w.o[db]);
    w.l = fp8::mfma_ones(ones, w.p, w.l);
  };

  // One step for tile j: `cur` holds tile j's scores (its max already applied), `nxt`
  // receives tile j+1's.  Three phases, kept apart with scheduling barriers so that only
  // one phase's operands are in registers at a time: (A) channels 0-63 of the QK
  // products of tile j+1 and the P codes of keys 0-31 of tile j; (B) channels 64-127 and
  // keys 32-63; (C) the PV and row-sum products of tile j, then the max of tile j+1.  kLast: no tile j+1;
  // kMaskNext: tile j+1 is the last one.
  auto step = [&](f32x16* cur, f32x16* nxt, const float* cbc, float* cbn, int j, auto last_tag,
                  auto mask_next_tag) __attribute__((always_inline)) {
    constexpr bool kLast = decltype(last_tag)::value;
    constexpr bool kMaskNext = decltype(mask_next_tag)::value;
    if (j + kSlots - 1 < nt) load(j + kSlots - 1);  // into the slot tile j-1 left
    const uint32_t kb0 = slot_addr(j + 1) + k_lane;
    // every row of the wave drops tile j: no softmax, PV or row-sum products for it
    const bool run = !(kSkip && w.skip_all);
    if (!run) ++w.skipped;
    // phase p: channel half p of the QK products of both key halves of tile j+1 (two
    // independent products), then the P codes of key half p of tile j
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (!kLast) {
        nxt[0] = fp8::mfma8(read32(kb0, 64 * p), w.q[p], p ? nxt[0] : f32x16{});
        nxt[1] = fp8::mfma8(read32(kb0, 32 * kKPitch + 64 * p), w.q[p], p ? nxt[1] : f32x16{});
      }
      if (run) softmax_half(cur[p], cbc, p, std::integral_constant<bool, kLast>{});
      __builtin_amdgcn_sched_barrier(0);
    }
    if (run) pv(j);
    if (!kLast) {
      block_c(j + 1, cbn);
      update_max(nxt, cbn, std::integral_constant<bool, kMaskNext>{});
    }
    loads_done();  // tile j+2 in LDS before the next step
    __syncthreads();
  };

  using T = std::true_type;
  using F = std::false_type;
  // ---- fill, then one step per tile
#pragma unroll
  for (int t = 0; t < kSlots - 1; ++t)
    if (t < nt) load(t);
  loads_done();
  __syncthreads();

  // MFMA-first step for tile j: the QK products of tile j+1 and the PV and row-sum
  // products of tile j back to back (operands read two products ahead), then the max
  // and the P codes of tile j+1 (kLast: no tile j+1; kMaskNext: tile j+1 is the last).
  // One score set: tile j+1's scores become P codes before the next QK overwrites them.
  auto mf_step = [&](f32x16* s, float* cbv, int j, auto last_tag, auto mask_next_tag)
      __attribute__((always_inline)) {
    constexpr bool kLast = decltype(last_tag)::value;
    constexpr bool kMaskNext = decltype(mask_next_tag)::value;
    using MN = std::integral_constant<bool, kMaskNext>;
    if (j + kSlots - 1 < nt) load(j + kSlots - 1);
    const bool run = !(kSkip && w.skip_all);
    if (!run) ++w.skipped;
    {
      // operand i: QK (i < 4: key half i & 1, channel half i >> 1), PV (4 <= i < 8:
      // channel block i - 4)
      const uint32_t kb0 = slot_addr(j + 1) + k_lane;
      const uint32_t vb0 = slot_addr(j) + v_lane;
      constexpr int i0 = kLast ? 4 : 0;
      i32x8 op[8];
      auto rd = [&](int i) __attribute__((always_inline)) {
        if (i < 4)
          op[i] = read32(kb0, (i & 1) * 32 * kKPitch + (i >> 1) * 64);
        else if (i < 8)
          op[i] = read32(vb0, (i - 4) * 32 * kVPitch);
      };
      if (i0 < 4 || run) {
        rd(i0);
        rd(i0 + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = i0; i < 9; ++i) {
        if (i < 4) {
          s[i & 1] = fp8::mfma8(op[i], w.q[i >> 1], (i >> 1) ? s[i & 1] : f32x16{});
          if (i + 2 < 4 || run) rd(i + 2);
        } else if (run) {
          if (i < 8) {
            w.o[i - 4] = fp8::mfma8(op[i], w.p, w.o[i - 4]);
            rd(i + 2);
          } else {
            w.l = fp8::mfma_ones(ones, w.p, w.l);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!kLast) {
      block_c(j + 1, cbv);
      update_max(s, cbv, MN{});
      if (!(kSkip && w.skip_all)) {
        softmax_half(s[0], cbv, 0, MN{});
        softmax_half(s[1], cbv, 1, MN{});
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    loads_done();  // tile j+2 in LDS before the next step
    __syncthreads();
  };

  if (wave >= kCopyWaves) {
    // the empty asm keeps the compiler from hoisting either form's first LDS reads above
    // the branch (which lengthened their live ranges into a spill)
    asm volatile("" ::: "memory");
    f32x16 s1[2];
    float cbv[4];
    qk(s1, 0);
    block_c(0, cbv);
    auto first = [&](auto mask_tag) __attribute__((always_inline)) {
      update_max(s1, cbv, mask_tag);
      if (!(kSkip && w.skip_all)) {
        softmax_half(s1[0], cbv, 0, mask_tag);
        softmax_half(s1[1], cbv, 1, mask_tag);
      }
    };
    if (nt == 1) {
      first(T{});
      mf_step(s1, cbv, 0, T{}, F{});
    } else {
      first(F{});
      for (int j = 0; j < nt - 2; ++j) mf_step(s1, cbv, j, F{}, F{});
      mf_step(s1, cbv, nt - 2, F{}, T{});
      mf_step(s1, cbv, nt - 1, T{}, F{});
    }
  } else {
  asm volatile("" ::: "memory");
  f32x16 sa[2], sb[2];
  float ca[4], cb[4];
  qk(sa, 0);
  block_c(0, ca);
  if (nt == 1)
    update_max(sa, ca, T{});
  else
    update_max(sa, ca, F{});
  // Steady steps j < nt-2, then step nt-2 (its next tile is the last) and step nt-1.
  // Score sets alternate sa -> sb -> sa; an odd count of steady steps peels one first so
  // that the loop always starts and ends with the current tile in sa.
  if (nt == 1) {
    step(sa, sb, ca, cb, 0, T{}, F{});
  } else {
    int j = 0;
    if (nt & 1) {
      step(sa, sb, ca, cb, 0, F{}, F{});
      sa[0] = sb[0];
      sa[1] = sb[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) ca[i] = cb[i];
      j = 1;
    }
    for (; j < nt - 2; j += 2) {
      step(sa, sb, ca, cb, j, F{}, F{});
      step(sb, sa, cb, ca, j + 1, F{}, F{});
    }
    step(sa, sb, ca, cb, nt - 2, F{}, T{});
    step(sb, sa, cb, ca, nt - 1, T{}, F{});
  }
  }  // interleaving waves

  if (kSkip) {  // wave tiles this workgroup skipped
    __shared__ uint32_t wave_skipped[kWaves];
    if (lane == 0) wave_skipped[wave] = w.skipped;
    __syncthreads();
    if (tid == 0) {
      uint32_t total = 0;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) total += wave_skipped[i];
      a.skipped[logical] = total;
    }
  } else if (tid == 0) {
    a.skipped[logical] = 0u;
  }

  // ---- epilogue: lane holds O^T[d = db*32 + 8i + 4hl + j][row] at register 4i+j
  if (row < a.seq_buf) {
    const float inv_l = 1.0f / w.l[0];
    __bf16* orow = a.o + row * a.out_stride + hoff;
    const uint32_t* vm = a.vamax + head * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * hl;
        u32x2 v = {0u, 0u};
        if (row < a.n_valid) {
          float y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            y[j] = w.o[db][4 * i + j] * (__uint_as_float(vm[d0 + j]) / kMax) * inv_l;
          v[0] = pack_bf16x2(y[0], y[1]);
          v[1] = pack_bf16x2(y[2], y[3]);
        }
        *reinterpret_cast<u32x2*>(orow + d0) = v;
      }
  }
}

}  // namespace h3
