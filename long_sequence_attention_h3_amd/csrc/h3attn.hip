// h3attn.hip — libh3attn: C ABI entry points (declared in include/h3attn.h), argument
// validation and kernel launches.  Kernels live in prologue.hpp, attention.hpp,
// attention_fp8.hpp and block.hpp.
//
// Pages: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
// (Chinese translation of the vLLM blog post), §3.1 (valid-length attention over an
// aligned packed buffer, per-token RoPE rows), §3.2 (fused Q/K RMSNorm + RoPE; the merged
// FP32 modulation, normalization and residual steps) and §4.3 (the FP8 "SAGE" variant of
// the attention and Skip-Softmax).
#include "h3attn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "attention.hpp"
#include "attention_fp8.hpp"
#include "block.hpp"
#include "prologue.hpp"

namespace {

using namespace h3;

constexpr int kBM = attn::kRows;  // query rows per attention workgroup

// ---------------------------------------------------------------- device check
// Per-device verdict of "is this a gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

h3_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return H3_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int v = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (v == 1) return H3_OK;
    if (v == 2) return H3_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return H3_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? H3_OK : H3_ERR_DEVICE;
}

// ---------------------------------------------------------------- validation
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

h3_status check_shape(const h3_shape* s, int64_t* max_valid) {
  if (!s || !s->seq_valid) return H3_ERR_NULL;
  if (s->batch < 1 || s->num_heads < 1 || s->seq_buf < 0) return H3_ERR_SHAPE;
  if (s->head_dim != kHeadDim) return H3_ERR_UNSUPPORTED;
  const int64_t hd = (int64_t)s->num_heads * kHeadDim;
  if (s->in_row_stride < hd || s->out_row_stride < hd) return H3_ERR_SHAPE;
  if ((s->in_row_stride % 8) != 0 || (s->out_row_stride % 8) != 0) return H3_ERR_ALIGN;
  // the grids index rows and heads with 32-bit block ids
  if (s->seq_buf > (int64_t)1 << 30 || s->num_heads > (1 << 16)) return H3_ERR_SHAPE;
  int64_t mx = 0;
  for (int b = 0; b < s->batch; ++b) {
    const int64_t n = s->seq_valid[b];
    if (n < 0 || n > s->seq_buf) return H3_ERR_SHAPE;
    if (n > mx) mx = n;
  }
  *max_valid = mx;
  return H3_OK;
}

h3_status check_rope(const h3_rope* r, int64_t max_valid, RopeArgs* out) {
  if (!r) return H3_ERR_NULL;
  if (!(r->theta > 0.0) || !std::isfinite(r->theta) || r->n_1d < 0) return H3_ERR_UNSUPPORTED;
  out->theta = r->theta;
  out->n_1d = r->n_1d;
  for (int i = 0; i < 3; ++i) out->sec[i] = r->sections[i];
  out->gt = r->grid_t;
  out->gh = r->grid_h;
  out->gw = r->grid_w;
  if (max_valid <= r->n_1d) {  // every valid token is 1-D
    out->sec[0] = out->sec[1] = out->sec[2] = 0;
    out->gt = out->gh = out->gw = 1;
    return H3_OK;
  }
  int sum = 0;
  for (int i = 0; i < 3; ++i) {
    // each 8-channel chunk must sit inside one half of one section
    if (r->sections[i] <= 0 || (r->sections[i] % 16) != 0) return H3_ERR_UNSUPPORTED;
    sum += r->sections[i];
  }
  if (sum != kHeadDim) return H3_ERR_UNSUPPORTED;
  if (r->grid_t <= 0 || r->grid_h <= 0 || r->grid_w <= 0) return H3_ERR_UNSUPPORTED;
  const int64_t cells = (int64_t)r->grid_t * r->grid_h * r->grid_w;
  if (max_valid - r->n_1d > cells) return H3_ERR_UNSUPPORTED;
  return H3_OK;
}

h3_status check_weights(const void* w_q, const void* w_k, int64_t w_head_stride) {
  if (!w_q || !w_k) return H3_ERR_NULL;
  if (!aligned16(w_q) || !aligned16(w_k)) return H3_ERR_ALIGN;
  if (w_head_stride != 0 && w_head_stride < kHeadDim) return H3_ERR_SHAPE;
  if ((w_head_stride % 8) != 0) return H3_ERR_ALIGN;
  return H3_OK;
}

int64_t tiles_per_head(const h3_shape* s) { return (s->seq_buf + kTileKeys - 1) / kTileKeys; }

int64_t attn_workgroups(const h3_shape* s) {
  return (int64_t)s->num_heads * ((s->seq_buf + kBM - 1) / kBM);
}

// Key ranges per query block.  A launch takes ceil(W / CUs) rounds of equally long
// workgroups for W workgroups (one resident per compute unit), so a grid of few rounds
// loses much of its last one: the 6-head, 58,816-row layer has 1,380 workgroups, 5.4
// rounds on 256 compute units.  Splitting each block's keys into k ranges (merged by
// attn_merge_kernel) gives ceil(k W / CUs) rounds of 1/k the length.  The k in 1..8
// (at most the number of key tiles) with the least ceil(k W / CUs) / k * (1 + 0.02 (k-1))
// is taken (the last factor prices the merge and each range's own start-up); ties go
// to the smaller k.  The compute-unit count is gfx950's (MI355X); it only steers the
// schedule, never the result's correctness.
constexpr int kMaxSplits = 8;
constexpr int kComputeUnits = 256;

int attn_splits(const h3_shape* s, int64_t n) {
  const int64_t W = attn_workgroups(s);
  const int64_t nt = (n + kTileKeys - 1) / kTileKeys;
  int best = 1;
  double best_cost = (double)((W + kComputeUnits - 1) / kComputeUnits);
  for (int k = 2; k <= kMaxSplits && k <= nt; ++k) {
    const double cost = (double)((k * W + kComputeUnits - 1) / kComputeUnits) / k *
                        (1.0 + 0.02 * (k - 1));
    if (cost < best_cost) {
      best = k;
      best_cost = cost;
    }
  }
  return best;
}

int max_splits(const h3_shape* s) {
  int k = 1;
  for (int b = 0; b < s->batch; ++b) {
    const int kb = attn_splits(s, s->seq_valid[b]);
    if (kb > k) k = kb;
  }
  return k;
}

// Workspace layout: packed K/V tile images, [batch][head][tile] x kTileImageBytes; then
// one int per attention workgroup (which pass handles it), [batch][kMaxSplits x W] with
// workgroup (head, split, block) at (head * k + split) * blocks + block; then, when some
// batch splits its keys, the partial results of one batch (reused batch after batch):
// O as [k][head][row][128] floats, then (m, l) as [k][head][row][2] floats.
size_t batch_ws_bytes(const h3_shape* s) {
  return (size_t)s->num_heads * (size_t)tiles_per_head(s) * (size_t)kTileImageBytes;
}
size_t flags_bytes(const h3_shape* s) {
  return ((size_t)s->batch * kMaxSplits * (size_t)attn_workgroups(s) * sizeof(int) + 255) &
         ~size_t(255);
}
size_t part_rows(const h3_shape* s) {
  const int k = max_splits(s);
  return k > 1 ? (size_t)k * (size_t)s->num_heads * (size_t)s->seq_buf : 0;
}
size_t part_o_bytes(const h3_shape* s) { return part_rows(s) * kHeadDim * sizeof(float); }
size_t part_bytes(const h3_shape* s) {
  return part_o_bytes(s) + ((part_rows(s) * 2 * sizeof(float) + 255) & ~size_t(255));
}
size_t workspace_bytes(const h3_shape* s) {
  return (size_t)s->batch * batch_ws_bytes(s) + flags_bytes(s) + part_bytes(s);
}

h3_status launched() { return hipGetLastError() == hipSuccess ? H3_OK : H3_ERR_LAUNCH; }

#define H3_TRY(expr)                   \
  do {                                 \
    const h3_status st_ = (expr);      \
    if (st_ != H3_OK) return st_;      \
  } while (0)

// FP8 workspace: tile images, [batch][head][tile] x fp8::kTileBytes, then the per-channel
// V maxima, [batch][head][128] floats, then one skipped-tile count per attention
// workgroup, [batch][head][ceil(S/256)] uint32; each part rounded up to 256 bytes.
size_t fp8_batch_img_bytes(const h3_shape* s) {
  return (size_t)s->num_heads * (size_t)tiles_per_head(s) * (size_t)fp8::kTileBytes;
}
size_t fp8_vamax_words(const h3_shape* s) {
  return (size_t)s->batch * (size_t)s->num_heads * kHeadDim;
}
size_t fp8_vamax_bytes(const h3_shape* s) { return (fp8_vamax_words(s) * 4 + 255) & ~size_t(255); }
size_t fp8_count_words(const h3_shape* s) {
  return (size_t)s->batch * (size_t)s->num_heads * (size_t)((s->seq_buf + fp8::kRows - 1) / fp8::kRows);
}
size_t fp8_workspace_bytes(const h3_shape* s) {
  return (size_t)s->batch * fp8_batch_img_bytes(s) + fp8_vamax_bytes(s) +
         ((fp8_count_words(s) * 4 + 255) & ~size_t(255));
}

h3_status check_workspace(const h3_shape* s, const void* ws, size_t bytes, bool is_fp8 = false) {
  const size_t need = is_fp8 ? fp8_workspace_bytes(s) : workspace_bytes(s);
  if (need > 0 && (!ws || bytes < need)) return H3_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return H3_ERR_ALIGN;
  return H3_OK;
}

h3_status check_norm(const void* w, int64_t w_head_stride, float eps, const h3_rope* rope,
                     int64_t max_valid, RopeArgs* ra) {
  H3_TRY(check_weights(w, w, w_head_stride));
  H3_TRY(check_rope(rope, max_valid, ra));
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return H3_ERR_SHAPE;
  return H3_OK;
}

// ---------------------------------------------------------------- stage 1: K/V pack
// The attention kernels' exp2 scale; the layer path also stores normalised K times it.
float exp2_scale(float softmax_scale) { return softmax_scale * 1.4426950408889634f; }

// Factor for normalised K rows: the exp2 scale, unless it is so small or large that K
// times it could leave bf16's normal range; then 1 (K stored as given), and the
// attention kernel applies the scale per score instead (it reads the factor from the
// tiles).
float prescale_factor(float softmax_scale) {
  const float c = exp2_scale(softmax_scale);
  return (c >= 0x1p-32f && c <= 0x1p32f) ? c : 1.0f;
}

h3_status do_kv_pack(const void* k, const void* v, const void* w_k, int64_t w_head_stride,
                     float eps, const h3_rope* rope, float softmax_scale, const h3_shape* shp,
                     void* workspace, size_t ws_bytes, hipStream_t stream) {
  int64_t max_valid = 0;
  H3_TRY(check_shape(shp, &max_valid));
  if (!k || !v) return H3_ERR_NULL;
  if (!aligned16(k) || !aligned16(v)) return H3_ERR_ALIGN;
  const bool norm = w_k != nullptr;
  RopeArgs ra{};
  if (norm) {
    H3_TRY(check_norm(w_k, w_head_stride, eps, rope, max_valid, &ra));
    if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return H3_ERR_SHAPE;
  }
  H3_TRY(check_workspace(shp, workspace, ws_bytes));
  H3_TRY(check_device());
  const int64_t S = shp->seq_buf, tph = tiles_per_head(shp);
  const size_t per_batch = batch_ws_bytes(shp);
  for (int b = 0; b < shp->batch; ++b) {
    const int64_t n = shp->seq_valid[b];
    if (n == 0) continue;
    char* ws = static_cast<char*>(workspace) + b * per_batch;
    PackArgs pa{};
    pa.k = static_cast<const __bf16*>(k) + b * S * shp->in_row_stride;
    pa.v = static_cast<const __bf16*>(v) + b * S * shp->in_row_stride;
    pa.w_k = static_cast<const __bf16*>(w_k);
    pa.w_head_stride = w_head_stride;
    pa.in_stride = shp->in_row_stride;
    pa.n_valid = n;
    pa.tiles_per_head = tph;
    pa.eps = eps;
    pa.k_mul = norm ? prescale_factor(softmax_scale) : 1.0f;
    pa.rope = ra;
    pa.img = ws;
    const dim3 grid((unsigned)((n + kTileKeys - 1) / kTileKeys), (unsigned)shp->num_heads);
    if (norm)
      kv_pack_kernel<true><<<grid, 128, 0, stream>>>(pa);
    else
      kv_pack_kernel<false><<<grid, 128, 0, stream>>>(pa);
    H3_TRY(launched());
  }
  return H3_OK;
}

// ---------------------------------------------------------------- stage 2: attention
// skip_threshold > 0: dense attention with Skip-Softmax (one launch over every
// workgroup, keys never split: the rule walks each row's tiles from the first).
h3_status do_attn_packed(const void* q, void* o, const void* w_q, int64_t w_head_stride,
                         float eps, const h3_rope* rope, float softmax_scale,
                         const h3_shape* shp, void* workspace, size_t ws_bytes,
                         hipStream_t stream, float skip_threshold = 0.0f) {
  if (!(skip_threshold >= 0.0f && skip_threshold < 1.0f)) return H3_ERR_SHAPE;
  const bool skip = skip_threshold > 0.0f;
  int64_t max_valid = 0;
  H3_TRY(check_shape(shp, &max_valid));
  if (!q || !o) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(o)) return H3_ERR_ALIGN;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return H3_ERR_SHAPE;
  const bool norm = w_q != nullptr;
  RopeArgs ra{};
  if (norm) H3_TRY(check_norm(w_q, w_head_stride, eps, rope, max_valid, &ra));
  H3_TRY(check_workspace(shp, workspace, ws_bytes));
  H3_TRY(check_device());
  const int H = shp->num_heads;
  const int64_t S = shp->seq_buf;
  if (S == 0) return H3_OK;
  const int m_tiles = (int)((S + kBM - 1) / kBM);
  const size_t per_batch = batch_ws_bytes(shp);
  char* after_images = static_cast<char*>(workspace) + shp->batch * per_batch;
  int* flags = reinterpret_cast<int*>(after_images);
  float* part = reinterpret_cast<float*>(after_images + flags_bytes(shp));
  float* part_ml = reinterpret_cast<float*>(after_images + flags_bytes(shp) + part_o_bytes(shp));
  for (int b = 0; b < shp->batch; ++b) {
    const char* ws = static_cast<const char*>(workspace) + b * per_batch;
    const int splits = skip ? 1 : attn_splits(shp, shp->seq_valid[b]);
    AttnArgs aa{};
    aa.wg_checked = flags + (size_t)b * kMaxSplits * attn_workgroups(shp);
    aa.splits = splits;
    aa.part = part;
    aa.part_ml = part_ml;
    aa.q = static_cast<const __bf16*>(q) + b * S * shp->in_row_stride;
    aa.o = static_cast<__bf16*>(o) + b * S * shp->out_row_stride;
    aa.img = ws;
    aa.tiles_per_head = tiles_per_head(shp);
    aa.in_stride = shp->in_row_stride;
    aa.out_stride = shp->out_row_stride;
    aa.n_valid = shp->seq_valid[b];
    aa.seq_buf = S;
    aa.heads = H;
    aa.m_tiles = m_tiles;
    aa.scale_log2 = exp2_scale(softmax_scale);
    aa.w_q = static_cast<const __bf16*>(w_q);
    aa.w_head_stride = w_head_stride;
    aa.eps = eps;
    aa.rope = ra;
    aa.skip_log2 = skip ? std::log2(skip_threshold) : -INFINITY;
    const unsigned blocks = (unsigned)((int64_t)H * m_tiles * splits);
    if (skip) {
      if (norm)
        attn_fwd_kernel<true, true, true><<<blocks, attn::kThreads, 0, stream>>>(aa);
      else
        attn_fwd_kernel<false, true, true><<<blocks, attn::kThreads, 0, stream>>>(aa);
      H3_TRY(launched());
      continue;
    }
    // fast pass, then the checked pass for the workgroups the fast pass flagged
    if (norm) {
      attn_fwd_kernel<true, false><<<blocks, attn::kThreads, 0, stream>>>(aa);
      attn_fwd_kernel<true, true><<<blocks, attn::kThreads, 0, stream>>>(aa);
    } else {
      attn_fwd_kernel<false, false><<<blocks, attn::kThreads, 0, stream>>>(aa);
      attn_fwd_kernel<false, true><<<blocks, attn::kThreads, 0, stream>>>(aa);
    }
    H3_TRY(launched());
    if (splits > 1) {
      MergeArgs ma{};
      ma.part = part;
      ma.part_ml = part_ml;
      ma.o = aa.o;
      ma.out_stride = aa.out_stride;
      ma.n_valid = aa.n_valid;
      ma.seq_buf = S;
      ma.heads = H;
      ma.splits = splits;
      attn_merge_kernel<<<dim3((unsigned)((S + 15) / 16), (unsigned)H), 256, 0, stream>>>(ma);
      H3_TRY(launched());
    }
  }
  return H3_OK;
}

// ---------------------------------------------------------------- FP8 stage 1
h3_status do_kv_pack_fp8(const void* k, const void* v, const void* w_k, int64_t w_head_stride,
                         float eps, const h3_rope* rope, const h3_shape* shp, void* workspace,
                         size_t ws_bytes, hipStream_t stream) {
  int64_t max_valid = 0;
  H3_TRY(check_shape(shp, &max_valid));
  if (!k || !v) return H3_ERR_NULL;
  if (!aligned16(k) || !aligned16(v)) return H3_ERR_ALIGN;
  const bool norm = w_k != nullptr;
  RopeArgs ra{};
  if (norm) H3_TRY(check_norm(w_k, w_head_stride, eps, rope, max_valid, &ra));
  H3_TRY(check_workspace(shp, workspace, ws_bytes, true));
  H3_TRY(check_device());
  const int64_t S = shp->seq_buf, tph = tiles_per_head(shp);
  const int H = shp->num_heads;
  const size_t per_batch = fp8_batch_img_bytes(shp);
  uint32_t* vamax =
      reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + shp->batch * per_batch);
  const int64_t words = (int64_t)fp8_vamax_words(shp);
  fill_zero_kernel<<<(unsigned)((words + 255) / 256), 256, 0, stream>>>(vamax, words);
  H3_TRY(launched());
  for (int b = 0; b < shp->batch; ++b) {
    const int64_t n = shp->seq_valid[b];
    if (n == 0) continue;
    Fp8StatsArgs sa{};
    sa.v = static_cast<const __bf16*>(v) + b * S * shp->in_row_stride;
    sa.in_stride = shp->in_row_stride;
    sa.n_valid = n;
    sa.vamax = vamax + (int64_t)b * H * kHeadDim;
    v_amax_kernel<<<dim3((unsigned)((n + kStatKeys - 1) / kStatKeys), (unsigned)H), 256, 0,
                    stream>>>(sa);
    H3_TRY(launched());
    Fp8PackArgs pa{};
    pa.k = static_cast<const __bf16*>(k) + b * S * shp->in_row_stride;
    pa.v = sa.v;
    pa.w_k = static_cast<const __bf16*>(w_k);
    pa.w_head_stride = w_head_stride;
    pa.in_stride = shp->in_row_stride;
    pa.n_valid = n;
    pa.tiles_per_head = tph;
    pa.eps = eps;
    pa.rope = ra;
    pa.vamax = sa.vamax;
    pa.img = static_cast<char*>(workspace) + b * per_batch;
    const dim3 grid((unsigned)((n + kTileKeys - 1) / kTileKeys), (unsigned)H);
    if (norm)
      kv_pack_fp8_kernel<true><<<grid, 256, 0, stream>>>(pa);
    else
      kv_pack_fp8_kernel<false><<<grid, 256, 0, stream>>>(pa);
    H3_TRY(launched());
  }
  return H3_OK;
}

// ---------------------------------------------------------------- FP8 stage 2
h3_status do_attn_packed_fp8(const void* q, void* o, const void* w_q, int64_t w_head_stride,
                             float eps, const h3_rope* rope, float softmax_scale,
                             float skip_threshold, const h3_shape* shp, void* workspace,
                             size_t ws_bytes, hipStream_t stream) {
  int64_t max_valid = 0;
  H3_TRY(check_shape(shp, &max_valid));
  if (!q || !o) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(o)) return H3_ERR_ALIGN;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return H3_ERR_SHAPE;
  if (!(skip_threshold >= 0.0f && skip_threshold < 1.0f)) return H3_ERR_SHAPE;
  const bool norm = w_q != nullptr;
  RopeArgs ra{};
  if (norm) H3_TRY(check_norm(w_q, w_head_stride, eps, rope, max_valid, &ra));
  H3_TRY(check_workspace(shp, workspace, ws_bytes, true));
  H3_TRY(check_device());
  const int H = shp->num_heads;
  const int64_t S = shp->seq_buf;
  if (S == 0) return H3_OK;
  const int m_tiles = (int)((S + fp8::kRows - 1) / fp8::kRows);
  const size_t per_batch = fp8_batch_img_bytes(shp);
  const uint32_t* vamax = reinterpret_cast<const uint32_t*>(
      static_cast<const char*>(workspace) + shp->batch * per_batch);
  uint32_t* counts = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) +
                                                 shp->batch * per_batch + fp8_vamax_bytes(shp));
  const bool skip = skip_threshold > 0.0f;
  for (int b = 0; b < shp->batch; ++b) {
    Fp8AttnArgs aa{};
    aa.skip_log2 = skip ? (float)std::log2((double)skip_threshold) : -INFINITY;
    aa.skipped = counts + (int64_t)b * H * m_tiles;
    aa.q = static_cast<const __bf16*>(q) + b * S * shp->in_row_stride;
    aa.o = static_cast<__bf16*>(o) + b * S * shp->out_row_stride;
    aa.img = static_cast<const char*>(workspace) + b * per_batch;
    aa.vamax = vamax + (int64_t)b * H * kHeadDim;
    aa.tiles_per_head = tiles_per_head(shp);
    aa.in_stride = shp->in_row_stride;
    aa.out_stride = shp->out_row_stride;
    aa.n_valid = shp->seq_valid[b];
    aa.seq_buf = S;
    aa.heads = H;
    aa.m_tiles = m_tiles;
    aa.scale_log2 = exp2_scale(softmax_scale);
    aa.w_q = static_cast<const __bf16*>(w_q);
    aa.w_head_stride = w_head_stride;
    aa.eps = eps;
    aa.rope = ra;
    const unsigned blocks = (unsigned)((int64_t)H * m_tiles);
    if (norm && skip)
      attn_fp8_kernel<true, true><<<blocks, fp8::kThreads, 0, stream>>>(aa);
    else if (norm)
      attn_fp8_kernel<true, false><<<blocks, fp8::kThreads, 0, stream>>>(aa);
    else if (skip)
      attn_fp8_kernel<false, true><<<blocks, fp8::kThreads, 0, stream>>>(aa);
    else
      attn_fp8_kernel<false, false><<<blocks, fp8::kThreads, 0, stream>>>(aa);
    H3_TRY(launched());
  }
  return H3_OK;
}

// ---------------------------------------------------------------- allocation-free entry
// Workspace of h3_attn_layer_noalloc: a static device array, one per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is used.
constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// This device's address of `scratch` (looked up on the first call on the device).
h3_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return H3_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return H3_ERR_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return H3_OK;
}

}  // namespace

extern "C" {

const char* h3_status_string(h3_status s) {
  switch (s) {
    case H3_OK: return "H3_OK";
    case H3_ERR_NULL: return "H3_ERR_NULL: a required pointer is NULL";
    case H3_ERR_SHAPE: return "H3_ERR_SHAPE: inconsistent sizes or arguments";
    case H3_ERR_ALIGN: return "H3_ERR_ALIGN: pointer or stride not 16-byte aligned";
    case H3_ERR_UNSUPPORTED: return "H3_ERR_UNSUPPORTED: head_dim or RoPE layout not supported";
    case H3_ERR_DEVICE: return "H3_ERR_DEVICE: no current gfx950 device";
    case H3_ERR_LAUNCH: return "H3_ERR_LAUNCH: kernel launch failed";
    case H3_ERR_WORKSPACE: return "H3_ERR_WORKSPACE: workspace missing or too small";
    case H3_ERR_SCRATCH_LIMIT:
      return "H3_ERR_SCRATCH_LIMIT: the problem needs more workspace than the static "
             "scratch of the allocation-free entry point holds";
  }
  return "unknown h3_status";
}

int h3_version(void) { return 100; }

h3_status h3_qk_rmsnorm_rope(const void* q_in, const void* k_in, void* q_out, void* k_out,
                             const void* w_q, const void* w_k, int64_t w_head_stride,
                             float eps, const h3_rope* rope, const h3_shape* shape,
                             hipStream_t stream) {
  int64_t max_valid = 0;
  H3_TRY(check_shape(shape, &max_valid));
  if (!q_in || !k_in || !q_out || !k_out) return H3_ERR_NULL;
  if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(q_out) || !aligned16(k_out))
    return H3_ERR_ALIGN;
  H3_TRY(check_weights(w_q, w_k, w_head_stride));
  RopeArgs ra{};
  H3_TRY(check_rope(rope, max_valid, &ra));
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return H3_ERR_SHAPE;
  if ((q_out == q_in || k_out == k_in) && shape->in_row_stride != shape->out_row_stride)
    return H3_ERR_SHAPE;
  H3_TRY(check_device());
  const int64_t S = shape->seq_buf;
  for (int b = 0; b < shape->batch; ++b) {
    const int64_t n = shape->seq_valid[b];
    if (n == 0) continue;
    PrologueArgs pa{};
    pa.q_in = static_cast<const __bf16*>(q_in) + b * S * shape->in_row_stride;
    pa.k_in = static_cast<const __bf16*>(k_in) + b * S * shape->in_row_stride;
    pa.q_out = static_cast<__bf16*>(q_out) + b * S * shape->out_row_stride;
    pa.k_out = static_cast<__bf16*>(k_out) + b * S * shape->out_row_stride;
    pa.w_q = static_cast<const __bf16*>(w_q);
    pa.w_k = static_cast<const __bf16*>(w_k);
    pa.w_head_stride = w_head_stride;
    pa.in_stride = shape->in_row_stride;
    pa.out_stride = shape->out_row_stride;
    pa.n_valid = n;
    pa.heads = shape->num_heads;
    pa.eps = eps;
    pa.rope = ra;
    qk_norm_rope_kernel<<<(unsigned)n, 256, 0, stream>>>(pa);
    H3_TRY(launched());
  }
  return H3_OK;
}

size_t h3_attn_workspace_size(const h3_shape* shape) {
  int64_t max_valid = 0;
  if (check_shape(shape, &max_valid) != H3_OK) return 0;
  return workspace_bytes(shape);
}

h3_status h3_kv_pack(const void* k, const void* v, const void* w_k, int64_t w_head_stride,
                     float eps, const h3_rope* rope, float softmax_scale, const h3_shape* shape,
                     void* workspace, size_t workspace_bytes_, hipStream_t stream) {
  return do_kv_pack(k, v, w_k, w_head_stride, eps, rope, softmax_scale, shape, workspace,
                    workspace_bytes_, stream);
}

h3_status h3_attn_packed(const void* q, void* o, const void* w_q, int64_t w_head_stride,
                         float eps, const h3_rope* rope, float softmax_scale,
                         const h3_shape* shape, void* workspace, size_t workspace_bytes_,
                         hipStream_t stream) {
  return do_attn_packed(q, o, w_q, w_head_stride, eps, rope, softmax_scale, shape, workspace,
                        workspace_bytes_, stream);
}

h3_status h3_attn_varlen(const void* q, const void* k, const void* v, void* o,
                         float softmax_scale, const h3_shape* shape, void* workspace,
                         size_t workspace_bytes_, hipStream_t stream) {
  // validate everything the second stage needs before launching the first
  if (!q || !o) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(o)) return H3_ERR_ALIGN;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return H3_ERR_SHAPE;
  H3_TRY(do_kv_pack(k, v, nullptr, 0, 0.0f, nullptr, softmax_scale, shape, workspace,
                    workspace_bytes_, stream));
  return do_attn_packed(q, o, nullptr, 0, 0.0f, nullptr, softmax_scale, shape, workspace,
                        workspace_bytes_, stream);
}

h3_status h3_attn_layer(const void* q, const void* k, const void* v, void* o,
                        const void* w_q, const void* w_k, int64_t w_head_stride, float eps,
                        const h3_rope* rope, float softmax_scale, const h3_shape* shape,
                        void* workspace, size_t workspace_bytes_, hipStream_t stream) {
  if (!q || !o || !w_q || !w_k) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(o)) return H3_ERR_ALIGN;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return H3_ERR_SHAPE;
  H3_TRY(check_weights(w_q, w_k, w_head_stride));
  H3_TRY(do_kv_pack(k, v, w_k, w_head_stride, eps, rope, softmax_scale, shape, workspace,
                    workspace_bytes_, stream));
  return do_attn_packed(q, o, w_q, w_head_stride, eps, rope, softmax_scale, shape, workspace,
                        workspace_bytes_, stream);
}

h3_status h3_attn_varlen_skip(const void* q, const void* k, const void* v, void* o,
                              float softmax_scale, float skip_threshold, const h3_shape* shape,
                              void* workspace, size_t workspace_bytes_, hipStream_t stream) {
  if (!q || !o) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(o)) return H3_ERR_ALIGN;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return H3_ERR_SHAPE;
  if (!(skip_threshold > 0.0f && skip_threshold < 1.0f)) return H3_ERR_SHAPE;
  H3_TRY(do_kv_pack(k, v, nullptr, 0, 0.0f, nullptr, softmax_scale, shape, workspace,
                    workspace_bytes_, stream));
  return do_attn_packed(q, o, nullptr, 0, 0.0f, nullptr, softmax_scale, shape, workspace,
                        workspace_bytes_, stream, skip_threshold);
}

h3_status h3_attn_layer_skip(const void* q, const void* k, const void* v, void* o,
                             const void* w_q, const void* w_k, int64_t w_head_stride, float eps,
                             const h3_rope* rope, float softmax_scale, float skip_threshold,
                             const h3_shape* shape, void* workspace, size_t workspace_bytes_,
                             hipStream_t stream) {
  if (!q || !o || !w_q || !w_k) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(o)) return H3_ERR_ALIGN;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return H3_ERR_SHAPE;
  if (!(skip_threshold > 0.0f && skip_threshold < 1.0f)) return H3_ERR_SHAPE;
  H3_TRY(check_weights(w_q, w_k, w_head_stride));
  H3_TRY(do_kv_pack(k, v, w_k, w_head_stride, eps, rope, softmax_scale, shape, workspace,
                    workspace_bytes_, stream));
  return do_attn_packed(q, o, w_q, w_head_stride, eps, rope, softmax_scale, shape, workspace,
                        workspace_bytes_, stream, skip_threshold);
}

size_t h3_attn_layer_noalloc_max_workspace(void) { return kScratchBytes; }

h3_status h3_attn_layer_noalloc(const void* q, const void* k, const void* v, void* o,
                                const void* w_q, const void* w_k, int64_t w_head_stride,
                                float eps, const h3_rope* rope, float softmax_scale,
                                const h3_shape* shape, hipStream_t stream) {
  int64_t max_valid = 0;
  H3_TRY(check_shape(shape, &max_valid));
  if (workspace_bytes(shape) > kScratchBytes) return H3_ERR_SCRATCH_LIMIT;
  H3_TRY(check_device());
  void* ws = nullptr;
  H3_TRY(scratch_address(&ws));
  // The same two stages as h3_attn_layer, with the static scratch as their workspace.
  // Nothing in it needs clearing: kv_pack writes every tile image the attention reads,
  // and the fast pass writes every pass flag before the checked pass reads it.
  return h3_attn_layer(q, k, v, o, w_q, w_k, w_head_stride, eps, rope, softmax_scale, shape,
                       ws, kScratchBytes, stream);
}

int h3_attn_splits(const h3_shape* shape, int batch) {
  int64_t max_valid = 0;
  if (check_shape(shape, &max_valid) != H3_OK || batch < 0 || batch >= shape->batch) return 0;
  return attn_splits(shape, shape->seq_valid[batch]);
}

size_t h3_attn_fp8_workspace_size(const h3_shape* shape) {
  int64_t max_valid = 0;
  if (check_shape(shape, &max_valid) != H3_OK) return 0;
  return fp8_workspace_bytes(shape);
}

h3_status h3_kv_pack_fp8(const void* k, const void* v, const void* w_k, int64_t w_head_stride,
                         float eps, const h3_rope* rope, const h3_shape* shape, void* workspace,
                         size_t workspace_bytes_, hipStream_t stream) {
  return do_kv_pack_fp8(k, v, w_k, w_head_stride, eps, rope, shape, workspace,
                        workspace_bytes_, stream);
}

h3_status h3_attn_packed_fp8(const void* q, void* o, const void* w_q, int64_t w_head_stride,
                             float eps, const h3_rope* rope, float softmax_scale,
                             float skip_threshold, const h3_shape* shape, void* workspace,
                             size_t workspace_bytes_, hipStream_t stream) {
  return do_attn_packed_fp8(q, o, w_q, w_head_stride, eps, rope, softmax_scale, skip_threshold,
                            shape, workspace, workspace_bytes_, stream);
}

h3_status h3_attn_varlen_fp8(const void* q, const void* k, const void* v, void* o,
                             float softmax_scale, float skip_threshold, const h3_shape* shape,
                             void* workspace, size_t workspace_bytes_, hipStream_t stream) {
  if (!q || !o) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(o)) return H3_ERR_ALIGN;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return H3_ERR_SHAPE;
  if (!(skip_threshold >= 0.0f && skip_threshold < 1.0f)) return H3_ERR_SHAPE;
  H3_TRY(do_kv_pack_fp8(k, v, nullptr, 0, 0.0f, nullptr, shape, workspace, workspace_bytes_,
                        stream));
  return do_attn_packed_fp8(q, o, nullptr, 0, 0.0f, nullptr, softmax_scale, skip_threshold,
                            shape, workspace, workspace_bytes_, stream);
}

h3_status h3_attn_layer_fp8(const void* q, const void* k, const void* v, void* o,
                            const void* w_q, const void* w_k, int64_t w_head_stride, float eps,
                            const h3_rope* rope, float softmax_scale, float skip_threshold,
                            const h3_shape* shape, void* workspace, size_t workspace_bytes_,
                            hipStream_t stream) {
  if (!q || !o || !w_q || !w_k) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(o)) return H3_ERR_ALIGN;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return H3_ERR_SHAPE;
  if (!(skip_threshold >= 0.0f && skip_threshold < 1.0f)) return H3_ERR_SHAPE;
  H3_TRY(check_weights(w_q, w_k, w_head_stride));
  H3_TRY(do_kv_pack_fp8(k, v, w_k, w_head_stride, eps, rope, shape, workspace,
                        workspace_bytes_, stream));
  return do_attn_packed_fp8(q, o, w_q, w_head_stride, eps, rope, softmax_scale, skip_threshold,
                            shape, workspace, workspace_bytes_, stream);
}

h3_status h3_residual_norm_modulate(void* x, const void* a, const float* gate,
                                    const float* shift, const float* scale,
                                    int64_t mod_batch_stride, float eps, void* y,
                                    const h3_rows* rows, hipStream_t stream) {
  if (!rows || !rows->seq_valid || !x || !y || !shift || !scale) return H3_ERR_NULL;
  if (rows->batch < 1 || rows->seq_buf < 0 || rows->hidden < 8) return H3_ERR_SHAPE;
  if ((rows->hidden % 8) != 0 || rows->hidden > 8 * blk::kThreads * blk::kMaxChunks)
    return H3_ERR_UNSUPPORTED;
  if (rows->seq_buf > ((int64_t)1 << 31) - 1) return H3_ERR_SHAPE;
  if (mod_batch_stride != 0 && mod_batch_stride < rows->hidden) return H3_ERR_SHAPE;
  if ((mod_batch_stride % 4) != 0) return H3_ERR_ALIGN;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return H3_ERR_SHAPE;
  for (int b = 0; b < rows->batch; ++b)
    if (rows->seq_valid[b] < 0 || rows->seq_valid[b] > rows->seq_buf) return H3_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(y) || !aligned16(shift) || !aligned16(scale) ||
      (a && !aligned16(a)) || (gate && !aligned16(gate)))
    return H3_ERR_ALIGN;
  H3_TRY(check_device());
  const int64_t S = rows->seq_buf, C = rows->hidden;
  if (S == 0) return H3_OK;
  for (int b = 0; b < rows->batch; ++b) {
    BlockArgs ba{};
    ba.x = static_cast<float*>(x) + b * S * C;
    ba.a = a ? static_cast<const __bf16*>(a) + b * S * C : nullptr;
    ba.gate = gate ? gate + b * mod_batch_stride : nullptr;
    ba.shift = shift + b * mod_batch_stride;
    ba.scale = scale + b * mod_batch_stride;
    ba.y = static_cast<__bf16*>(y) + b * S * C;
    ba.hidden = C;
    ba.n_valid = rows->seq_valid[b];
    ba.seq_buf = S;
    ba.eps = eps;
    constexpr int RR = blk::kRowsResidual, RP = blk::kRowsPlain;
    const unsigned grid_r = (unsigned)((S + RR - 1) / RR);
    const unsigned grid_p = (unsigned)((S + RP - 1) / RP);
    if (a && gate)
      residual_norm_modulate_kernel<true, true, RR><<<grid_r, blk::kThreads, 0, stream>>>(ba);
    else if (a)
      residual_norm_modulate_kernel<true, false, RR><<<grid_r, blk::kThreads, 0, stream>>>(ba);
    else
      residual_norm_modulate_kernel<false, false, RP><<<grid_p, blk::kThreads, 0, stream>>>(ba);
    H3_TRY(launched());
  }
  return H3_OK;
}

}  // extern "C"
