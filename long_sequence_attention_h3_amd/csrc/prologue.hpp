// prologue.hpp — per-head RMSNorm + rotary embedding for Q and K, and the K/V
// repacking pre-pass of the attention kernel.
//
// Pages: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
// (Chinese translation of the vLLM blog post), §3.2 (Q/K RMSNorm and RoPE fused into
// one operator) and §3.1 (RoPE rows are built per token; the packed sequence keeps
// only its valid tokens).
//
// Every kernel that normalises and rotates a head row goes through the helpers in
// this file with the same operation order, so the standalone prologue, the K pre-pass
// and the Q prologue fused into attention produce bit-identical bf16 values.
#pragma once

#include "common.hpp"

namespace h3 {

// ---------------------------------------------------------------------------------
// Rotary geometry.
//
// 1-D tokens: pair (j, j + 64), j = 0..63, frequency theta^(-2j/128), position = token.
// 3-axis tokens: channel sections (s0, s1, s2) at offsets (0, s0, s0 + s1); inside a
// section of size s, pair (off + j, off + j + s/2), frequency theta^(-2j/s), position
// pt / ph / pw.  With sections that are multiples of 16 every 8-channel chunk lies in
// one section and one half of it, so a chunk's rotation partner is a whole chunk.
// Pairs are numbered 0..63 globally: 1-D pair j is j; 3-axis pair j of the section at
// offset off is off/2 + j.

// Frequencies divided by 2*pi ("revolutions per position unit") for the 64 pairs of
// each mode, computed in fp64 once per workgroup into LDS.
struct FreqTable {
  double one_d[64];
  double three[64];
};

__device__ __forceinline__ void fill_freq_table(FreqTable* t, const RopeArgs& r, int tid,
                                                int nthreads) {
  const double inv_2pi = 0.15915494309189533577;  // 1 / (2 pi)
  for (int i = tid; i < 128; i += nthreads) {
    const int p = i & 63;
    if (i < 64) {
      t->one_d[p] = pow(r.theta, -2.0 * (double)p / 128.0) * inv_2pi;
    } else {
      int off = 0, s = r.sec[0];
      if (2 * p >= r.sec[0] + r.sec[1]) {
        off = r.sec[0] + r.sec[1];
        s = r.sec[2];
      } else if (2 * p >= r.sec[0]) {
        off = r.sec[0];
        s = r.sec[1];
      }
      const int j = p - off / 2;
      t->three[p] = (s > 0) ? pow(r.theta, -2.0 * (double)j / (double)s) * inv_2pi : 0.0;
    }
  }
}

// Where one 8-channel chunk of a token's row sits in the rotation.
struct ChunkRot {
  int partner;      // chunk holding the other member of each pair
  int pair0;        // global pair index of the chunk's first channel
  bool first;       // chunk holds the first members (y_j) rather than y_{j+s/2}
  bool three_axis;  // 3-axis table and position
  double pos;       // position along the chunk's axis
};

// Tokens past n_1d without a 3-axis layout (sections zero) only occur as query rows in
// the buffer tail, whose results are discarded; they take the 1-D path so every table
// index stays inside the 64 pairs.
__device__ __forceinline__ ChunkRot chunk_rotation(const RopeArgs& r, int64_t token, int cc) {
  ChunkRot c;
  if (token < r.n_1d || r.sec[0] == 0) {
    c.three_axis = false;
    c.first = cc < 8;
    c.partner = cc ^ 8;
    c.pair0 = (cc & 7) * 8;
    c.pos = (double)token;
    return c;
  }
  c.three_axis = true;
  const int64_t k = token - r.n_1d;
  const int64_t hw = (int64_t)r.gh * r.gw;
  const int64_t pt = k / hw, ph = (k / r.gw) % r.gh, pw = k % r.gw;
  const int ch = cc * 8;
  int off, s;
  int64_t pos;
  if (ch < r.sec[0]) {
    off = 0; s = r.sec[0]; pos = pt;
  } else if (ch < r.sec[0] + r.sec[1]) {
    off = r.sec[0]; s = r.sec[1]; pos = ph;
  } else {
    off = r.sec[0] + r.sec[1]; s = r.sec[2]; pos = pw;
  }
  const int half = s / 2, u = ch - off;
  c.first = u < half;
  c.partner = c.first ? cc + half / 8 : cc - half / 8;
  c.pair0 = off / 2 + (c.first ? u : u - half);
  c.pos = (double)pos;
  return c;
}

// cos and sin of 2*pi*frac(pos * f): the product and its reduction to one revolution in
// fp64 (positions reach ~1e5, where an fp32 angle would be off by ~1e-2 rad), the
// trigonometry on the reduced fp32 argument.
__device__ __forceinline__ void rope_cos_sin(double pos, double f, float* c, float* s) {
  const double rev = pos * f;
  const float fr = (float)(rev - rint(rev));
  *c = __builtin_amdgcn_cosf(fr);  // cos(2*pi*fr)
  *s = __builtin_amdgcn_sinf(fr);  // sin(2*pi*fr)
}

// Sum of squares of one chunk (8 values), accumulated in index order.
__device__ __forceinline__ float chunk_sumsq(const float* x) {
  float p = x[0] * x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) p = fmaf(x[e], x[e], p);
  return p;
}

// The row's inverse RMS from its sum of squares.  The sum over the 16 chunk partials
// is always formed as the pairwise tree ((p0+p1)+(p2+p3)) + ... , i.e. partials of
// chunks c and c^1 first, then c^2, c^4, c^8; callers reproduce that tree exactly.
__device__ __forceinline__ float inv_rms(float sumsq, float eps) {
  return __builtin_amdgcn_rsqf(sumsq * (1.0f / kHeadDim) + eps);
}

// Normalise and rotate one chunk.  x / xp: own and partner chunk values; w / wp: their
// weights; returns the 8 rotated values.
__device__ __forceinline__ void norm_rotate_chunk(const float* x, const float* xp,
                                                  const float* w, const float* wp,
                                                  float inv, const ChunkRot& cr,
                                                  const FreqTable* ft, float* out) {
  const double* tab = cr.three_axis ? ft->three : ft->one_d;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y = (x[e] * inv) * w[e];
    const float yp = (xp[e] * inv) * wp[e];
    float c, s;
    rope_cos_sin(cr.pos, tab[cr.pair0 + e], &c, &s);
    // first member:  y_j cos - y_{j+s/2} sin;  second member:  y_{j+s/2} cos + y_j sin
    out[e] = cr.first ? fmaf(y, c, -(yp * s)) : fmaf(y, c, yp * s);
  }
}

// ---------------------------------------------------------------------------------
// One (token, head) row handled by 16 consecutive lanes, lane `cc` owning chunk cc.
// Normalises and rotates the row whose chunk cc the lane holds in `raw` and returns the
// lane's 8 output values; `w` points at the head's 128 weights.  All 16 lanes must be
// active.
__device__ __forceinline__ void norm_rotate_raw16(const u32x4 raw, const __bf16* w, float eps,
                                                  const ChunkRot& cr, int cc,
                                                  const FreqTable* ft, float* out) {
  float x[8];
  unpack8(raw, x);
  float ss = chunk_sumsq(x);
  ss += __shfl_xor(ss, 1, 16);
  ss += __shfl_xor(ss, 2, 16);
  ss += __shfl_xor(ss, 4, 16);
  ss += __shfl_xor(ss, 8, 16);
  const float inv = inv_rms(ss, eps);
  // partner chunk's values from the lane that owns it
  const int base = (threadIdx.x & 63) & ~15;
  u32x4 praw;
#pragma unroll
  for (int i = 0; i < 4; ++i) praw[i] = __shfl(raw[i], base + cr.partner, 64);
  float xp[8], wv[8], wpv[8];
  unpack8(praw, xp);
  unpack8(*reinterpret_cast<const u32x4*>(w + cc * 8), wv);
  unpack8(*reinterpret_cast<const u32x4*>(w + cr.partner * 8), wpv);
  norm_rotate_chunk(x, xp, wv, wpv, inv, cr, ft, out);
}

// The same, loading chunk cc of the row at `row` (the head's 128 inputs).
__device__ __forceinline__ void norm_rotate_row16(const __bf16* row, const __bf16* w,
                                                  float eps, const ChunkRot& cr, int cc,
                                                  const FreqTable* ft, float* out) {
  norm_rotate_raw16(*reinterpret_cast<const u32x4*>(row + cc * 8), w, eps, cr, cc, ft, out);
}

struct PrologueArgs {
  const __bf16* q_in;
  const __bf16* k_in;
  __bf16* q_out;
  __bf16* k_out;
  const __bf16* w_q;
  const __bf16* w_k;
  int64_t w_head_stride;  // elements; 0 = shared
  int64_t in_stride, out_stride;  // row strides, elements
  int64_t n_valid;
  int heads;
  float eps;
  RopeArgs rope;
};

// Standalone fused Q/K RMSNorm + RoPE.  One workgroup per token: the rotation of a
// token is the same for every head, so it is set up once and reused for 2*H rows.
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(PrologueArgs a) {
  const int64_t t = blockIdx.x;
  if (t >= a.n_valid) return;
  __shared__ FreqTable ft;
  fill_freq_table(&ft, a.rope, threadIdx.x, blockDim.x);
  __syncthreads();
  const int cc = threadIdx.x & 15;
  const ChunkRot cr = chunk_rotation(a.rope, t, cc);
  for (int r = threadIdx.x >> 4; r < 2 * a.heads; r += blockDim.x >> 4) {
    const bool is_q = r < a.heads;
    const int h = is_q ? r : r - a.heads;
    const __bf16* in = (is_q ? a.q_in : a.k_in) + t * a.in_stride + (int64_t)h * kHeadDim;
    const __bf16* w = (is_q ? a.w_q : a.w_k) + (int64_t)h * a.w_head_stride;
    float y[8];
    norm_rotate_row16(in, w, a.eps, cr, cc, &ft, y);
    __bf16* out = (is_q ? a.q_out : a.k_out) + t * a.out_stride + (int64_t)h * kHeadDim;
    // every lane has read its partner chunk before any lane of the row stores (the
    // shuffles above are complete), so in-place operation is safe
    *reinterpret_cast<u32x4*>(out + cc * 8) = pack8(y);
  }
}

// ---------------------------------------------------------------------------------
// K/V pre-pass of the attention kernel.
//
// For head h and key tile kt (keys 64 kt .. 64 kt + 63) it writes one contiguous tile
// image (layout in common.hpp) that the attention kernel copies linearly into LDS:
//   K part: key r, channels 8c .. 8c+7 at byte r*272 + 16c;
//   V part: channel d, key chunk c at byte 17408 + d*144 + 16c, where chunk c holds, in
//           order, the keys 16(c/2) + 4(c%2) + {0,1,2,3} and 16(c/2) + 8 + 4(c%2) + {0,1,2,3}.
// The pad after K row 0 holds the tile's largest K row norm (the attention kernel bounds
// its scores with it) and the factor k_mul.  With `norm` set, K rows are RMS-normalised
// and rotated on the way (the layer path) and multiplied by k_mul in fp32 before their
// one rounding to bf16: the attention kernel passes softmax_scale * log2(e), so its
// scores come out of the matrix cores in exp2 units.  Without `norm`, K is copied as
// given and k_mul is 1 (scaling bf16 input would round it a second time).
// The V key order inside each 16-key group (bits 2 and 3 of the key index exchanged)
// is the order in which the QK product leaves the probabilities in registers, so the PV
// product consumes them without shuffles.  Keys >= N are written as zeros.
struct PackArgs {
  const __bf16* k;
  const __bf16* v;
  const __bf16* w_k;
  int64_t w_head_stride;
  int64_t in_stride;
  int64_t n_valid;
  int64_t tiles_per_head;  // capacity of the image array per head
  float eps;
  float k_mul;             // applied to normalised K rows before rounding (1 without norm)
  RopeArgs rope;
  char* img;               // [head][tile] x kTileImageBytes
};

template <bool kNorm>
__global__ __launch_bounds__(128) void kv_pack_kernel(PackArgs a) {
  const int64_t kt = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ FreqTable ft;
  if (kNorm) {
    fill_freq_table(&ft, a.rope, tid, blockDim.x);
    __syncthreads();
  }
  const int64_t key0 = kt * kTileKeys;
  char* img = a.img + ((int64_t)h * a.tiles_per_head + kt) * kTileImageBytes;
  const int64_t hoff = (int64_t)h * kHeadDim;

  // K: 64 rows x 16 chunks; 8 rows per pass (16 lanes per row).  All 8 rows of a lane are
  // loaded before the first image store: the compiler cannot tell the image from K, so
  // with a load per iteration every load would wait for the previous row's store.
  const int cc = tid & 15;
  float norm2_max = 0.0f;  // largest squared row norm seen by this thread's row group
  u32x4 kraw[kTileKeys / 8];
#pragma unroll
  for (int i = 0; i < kTileKeys / 8; ++i) {
    const int64_t key = key0 + (tid >> 4) + 8 * i;
    kraw[i] = key < a.n_valid
                  ? *reinterpret_cast<const u32x4*>(a.k + key * a.in_stride + hoff + cc * 8)
                  : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < kTileKeys / 8; ++i) {
    const int r = (tid >> 4) + 8 * i;
    const int64_t key = key0 + r;
    u32x4 out = {0u, 0u, 0u, 0u};
    // the whole 16-lane row group takes the same branch (one key per group)
    if (key < a.n_valid) {
      if (kNorm) {
        const ChunkRot cr = chunk_rotation(a.rope, key, cc);
        float y[8];
        norm_rotate_raw16(kraw[i], a.w_k + (int64_t)h * a.w_head_stride, a.eps, cr, cc, &ft,
                          y);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] *= a.k_mul;
        out = pack8(y);
      } else {
        out = kraw[i];
      }
    }
    *reinterpret_cast<u32x4*>(img + r * kKRowPitch + cc * 16) = out;
    float x[8];
    unpack8(out, x);
    float n2 = chunk_sumsq(x);
    n2 += __shfl_xor(n2, 1, 16);
    n2 += __shfl_xor(n2, 2, 16);
    n2 += __shfl_xor(n2, 4, 16);
    n2 += __shfl_xor(n2, 8, 16);
    norm2_max = fmaxf(norm2_max, n2);
  }
  __shared__ float row_max[8];
  if (cc == 0) row_max[tid >> 4] = norm2_max;
  __syncthreads();
  // the K row pads: row 0's carries the tile's largest row norm (rounded up a little so
  // that it bounds the fp32 norm of every row) and k_mul, the others are zero
  if (tid < kTileKeys) {
    u32x4 pad = {0u, 0u, 0u, 0u};
    if (tid == 0) {
      float m2 = row_max[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) m2 = fmaxf(m2, row_max[i]);
      pad[0] = __float_as_uint(sqrtf(m2) * 1.0001f);
      pad[1] = __float_as_uint(kNorm ? a.k_mul : 1.0f);
    }
    *reinterpret_cast<u32x4*>(img + tid * kKRowPitch + kKNormOffset) = pad;
  }

  // V: thread (key chunk c, channel chunk cg) gathers the chunk's 8 keys at channels
  // 8cg .. 8cg+7 and writes 8 image chunks (one per channel, 8 keys each).
  {
    char* vimg = img + kKImageBytes;
    const int c = tid & 7, cg = tid >> 3;  // 8 x 16 = 128 threads
    uint32_t x[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kin = 16 * (c >> 1) + 8 * (e >> 2) + 4 * (c & 1) + (e & 3);
      const int64_t key = key0 + kin;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (key < a.n_valid)
        raw = *reinterpret_cast<const u32x4*>(a.v + key * a.in_stride + hoff + cg * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[e][i] = raw[i];
    }
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {  // channel 8cg + ch
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // keys 2i and 2i+1 of channel ch: 16-bit halves (ch & 1) of dword ch/2
        const uint32_t lo = x[2 * i][ch >> 1], hi = x[2 * i + 1][ch >> 1];
        o[i] = (ch & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                        : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      }
      const int d = cg * 8 + ch;
      *reinterpret_cast<u32x4*>(vimg + d * kVRowPitch + c * 16) = o;
    }
    // zero the V row pads
    *reinterpret_cast<u32x4*>(vimg + tid * kVRowPitch + 128) = u32x4{};
  }
}

}  // namespace h3
