/*
 * h3attn.h — C ABI of libh3attn: the self-attention layer of a joint audio/video
 * DiT over a packed text+audio+video token sequence, on AMD MI355X (gfx950).
 *
 * Pages cited:
 *   [Blog] "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
 *          (Chinese translation of the vLLM blog post on serving MiniMax H3).
 *     §1    text, audio and video tokens form one packed sequence, denoised jointly;
 *     §3.1  "长序列注意力与通信": the packed sequence sits in an aligned buffer
 *           (58,758 valid tokens of 58,816); attention receives the valid length and
 *           the structural tail padding is dropped; RoPE rows are built per token;
 *           heads are 128-channel projections of a 5,376-channel hidden state;
 *     §3.2  "融合的 DiT 算子": Q/K RMSNorm and RoPE are one fused operator; the FP32
 *           modulation, normalization and residual steps are merged into one;
 *     §3.5  speed-ups are "lossless" but not bitwise identical to other kernels;
 *     §4.3  (figure 6) SAGE attention: Q, K, P and V quantized to FP8 for both
 *           attention products; the measured configuration is called "K16".
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every entry point
 *
 *  - Tensors are bf16, in caller-owned DEVICE memory, laid out [B, S, H, D]:
 *    token t of batch b, head h, channel c at  base + b*S*stride + t*stride + h*D + c
 *    (element offsets), where stride is the row stride in elements (>= H*D; a fused
 *    [S, 3, H, D] QKV buffer is addressed with stride 3*H*D).
 *  - Only D = 128 is supported.  Every pointer and every row stride must be
 *    16-byte aligned (stride a multiple of 8 elements).
 *  - Rows [N_b, S) of every input may hold anything, NaN included; they never
 *    enter the arithmetic.  Output rows [N_b, S) of an attention call are written
 *    as exact zeros.  N_b = 0 is valid.
 *  - Valid rows must be finite.  The attention sums are accumulated in fp32 with each
 *    softmax term at most 2^64 times the row's first-tile maximum term (at most 2^8 on
 *    the workgroups that fail the fast pass's score bound), so for any length the
 *    interface accepts (S <= 2^30) no accumulator overflows while max |V| < 2^34.
 *  - All work is enqueued asynchronously on `stream` (NULL: the default stream).
 *    The status reports argument validation and launch errors only; faults on the
 *    device surface at the caller's next synchronisation.  Nothing is allocated
 *    on the device: the attention calls take a caller-provided workspace.
 *  - No state is kept between calls; calls on different streams are independent
 *    as long as their output and workspace buffers do not overlap.
 *  - No C++ exception crosses this interface.
 */
#ifndef H3ATTN_H
#define H3ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  H3_OK = 0,
  H3_ERR_NULL = 1,         /* a required pointer is NULL                            */
  H3_ERR_SHAPE = 2,        /* inconsistent sizes (N > S, N < 0, stride < H*D, ...)  */
  H3_ERR_ALIGN = 3,        /* pointer or stride not 16-byte aligned                 */
  H3_ERR_UNSUPPORTED = 4,  /* head_dim != 128, bad RoPE sections or grid            */
  H3_ERR_DEVICE = 5,       /* no current HIP device, or it is not gfx950            */
  H3_ERR_LAUNCH = 6,       /* a kernel launch failed                                */
  H3_ERR_WORKSPACE = 7,    /* workspace missing or smaller than h3_attn_workspace_size */
  H3_ERR_SCRATCH_LIMIT = 8 /* h3_attn_layer_noalloc: the problem needs more workspace than
                              h3_attn_layer_noalloc_max_workspace() bytes            */
} h3_status;

/* One packed, aligned buffer ([Blog §3.1]: a valid length inside an aligned buffer). */
typedef struct {
  int32_t batch;             /* B >= 1                                              */
  int32_t num_heads;         /* H >= 1                                              */
  int32_t head_dim;          /* D; must be 128                                      */
  int64_t seq_buf;           /* S: rows allocated per sequence                      */
  const int64_t* seq_valid;  /* HOST array [B]: N_b, 0 <= N_b <= S                  */
  int64_t in_row_stride;     /* row stride (elements) of Q, K, V and prologue inputs */
  int64_t out_row_stride;    /* row stride (elements) of O and prologue outputs      */
} h3_shape;

/* Rotary descriptor: the per-token "RoPE rows" of [Blog §3.1].
 * Tokens t < n_1d rotate as 1-D RoPE at position t over all D channels: pairs
 * (j, j + D/2), angle t * theta^(-2j/D).  Tokens t >= n_1d (video) rotate as 3-axis
 * RoPE: k = t - n_1d, (pt, ph, pw) = (k / (gh*gw), (k / gw) % gh, k % gw); channel
 * sections of sizes sections[0..2] at offsets 0, s0, s0+s1 rotate by pt, ph, pw,
 * pairs (off + j, off + j + s/2), angle p * theta^(-2j/s).  When every valid token is
 * 1-D (n_1d >= N) the sections and grid are ignored; otherwise each section size must
 * be even and positive with s0 + s1 + s2 = D, and the grid must hold N - n_1d tokens. */
typedef struct {
  double theta;              /* base, e.g. 10000                                    */
  int64_t n_1d;
  int32_t sections[3];       /* e.g. {32, 48, 48}                                   */
  int32_t grid_t, grid_h, grid_w;
} h3_rope;

/* Human-readable name of a status code (static storage, never NULL). */
const char* h3_status_string(h3_status s);

/* Library version, as MAJOR*10000 + MINOR*100 + PATCH. */
int h3_version(void);

/* Fused per-head Q/K RMSNorm + RoPE  ([Blog §3.2]).
 * For every valid token t < N_b and head h, independently for X in {Q, K}:
 *   y = x / sqrt(mean_c x_c^2 + eps) * w[h*w_head_stride + c]   (fp32 arithmetic)
 *   out = RoPE_t(y)   (descriptor above), rounded to bf16 (nearest even).
 * q_in/k_in are read with in_row_stride, q_out/k_out written with out_row_stride.
 * Output rows [N_b, S) are left untouched.  In place (q_out == q_in, equal strides)
 * is allowed; partially overlapping buffers are not.
 * w_q, w_k: bf16 device arrays, [D] when w_head_stride == 0, [H][w_head_stride] else.
 * Errors: H3_ERR_NULL, H3_ERR_SHAPE, H3_ERR_ALIGN, H3_ERR_UNSUPPORTED, H3_ERR_DEVICE,
 * H3_ERR_LAUNCH. */
h3_status h3_qk_rmsnorm_rope(const void* q_in, const void* k_in, void* q_out, void* k_out,
                             const void* w_q, const void* w_k, int64_t w_head_stride,
                             float eps, const h3_rope* rope, const h3_shape* shape,
                             hipStream_t stream);

/* Bytes of device workspace an attention call with this shape needs (0 if the shape
 * is invalid).  The workspace holds the key and value operands of every batch repacked
 * for the attention kernel as 64-key tiles of 35,840 bytes each,
 * B * H * ceil(S / 64) * 35840 bytes (about 1.09x the bf16 size of K plus V), followed
 * by one 4-byte word per 256 query rows of every head and batch, rounded up to 256
 * bytes: round_up(B * H * ceil(S / 256) * 4, 256) bytes.  After an attention call,
 * word (b * H + h) * ceil(S / 256) + i tells which pass handled rows [256 i, 256 i + 256)
 * of head h, batch b: 0 the fast pass (scores provably bounded), 1 the checked pass. */
size_t h3_attn_workspace_size(const h3_shape* shape);

/* Stage 1 of attention: repack K and V of every batch into `workspace` (keys of 64-key
 * tiles as the attention kernel reads them; keys >= N_b stored as zeros).  With w_k
 * non-NULL each K row is first RMS-normalised (weights w_k, w_head_stride, eps) and
 * rotated (rope) with the arithmetic of h3_qk_rmsnorm_rope, then multiplied in fp32 by
 * c = softmax_scale * log2(e) (when 2^-32 <= c <= 2^32; otherwise by 1, so that K
 * stays in bf16's normal range) and rounded once to bf16, so that the attention kernel's
 * scores come out of the matrix cores in exp2 units (the layer's K operand is thus
 * bf16(k * softmax_scale * log2 e) rather than bf16(k): the same relative rounding,
 * of a different value).  With w_k NULL, K is stored as given and rope, eps and
 * softmax_scale are ignored.  The tiles record the factor used, and h3_attn_packed
 * accepts either kind with any softmax_scale.  Reads K and V with in_row_stride.  The
 * packed workspace stays valid for any number of h3_attn_packed calls with the same
 * shape.
 * Errors: H3_ERR_NULL, H3_ERR_SHAPE (also softmax_scale not positive and finite when w_k
 * is non-NULL), H3_ERR_ALIGN, H3_ERR_UNSUPPORTED, H3_ERR_DEVICE, H3_ERR_LAUNCH,
 * H3_ERR_WORKSPACE. */
h3_status h3_kv_pack(const void* k, const void* v, const void* w_k, int64_t w_head_stride,
                     float eps, const h3_rope* rope, float softmax_scale,
                     const h3_shape* shape, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Stage 2 of attention: O = softmax(scale * Q K^T) V over the valid keys, with K and V
 * taken from a workspace filled by h3_kv_pack for the same shape.  With w_q non-NULL
 * each Q row is RMS-normalised and rotated in registers on load (same arithmetic as
 * h3_qk_rmsnorm_rope); with w_q NULL, Q is used as is.  Output rows [N_b, S) are zero.
 * The tile images are only read; the pass words after them are written, so two calls
 * sharing one workspace must not overlap in time.
 * Errors: as h3_kv_pack. */
h3_status h3_attn_packed(const void* q, void* o, const void* w_q, int64_t w_head_stride,
                         float eps, const h3_rope* rope, float softmax_scale,
                         const h3_shape* shape, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Dense non-causal softmax attention over the valid tokens ([Blog §3.1]), with Q and
 * K already normalised and rotated:
 *   O[t, h, :] = sum_{j<N} softmax_j(scale * Q[t,h,:] . K[j,h,:]) V[j, h, :]   t < N
 *   O[t, h, :] = 0                                                           N <= t < S
 * Products in bf16 on the matrix cores with fp32 accumulation; softmax in fp32;
 * output rounded to bf16.  The result is deterministic run to run.  Equivalent to
 * h3_kv_pack (w_k NULL) followed by h3_attn_packed (w_q NULL).
 * workspace: device buffer of at least h3_attn_workspace_size(shape) bytes, 256-byte
 * aligned, not shared with a concurrent call.
 * Errors: as h3_qk_rmsnorm_rope, plus H3_ERR_WORKSPACE. */
h3_status h3_attn_varlen(const void* q, const void* k, const void* v, void* o,
                         float softmax_scale, const h3_shape* shape, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* The whole layer ([Blog §3.1]: attention over the valid tokens of an aligned packed
 * buffer, RoPE rows built per token; [Blog §3.2]: Q/K RMSNorm and RoPE as one fused
 * operator): per-head Q/K RMSNorm + RoPE fused into the attention prologue,
 * then attention as in h3_attn_varlen, with normalised Q and K never round-tripping
 * through a bf16 [S, H, D] buffer: K is prepared once into the workspace (h3_kv_pack
 * with w_k, which stores it times softmax_scale * log2(e), rounded once), Q in registers
 * (h3_attn_packed with w_q).  The Q operands are bit-identical to what
 * h3_qk_rmsnorm_rope writes; the K operands are bf16(k * softmax_scale * log2 e) instead
 * of bf16(k), so the result agrees with h3_qk_rmsnorm_rope + h3_attn_varlen to within
 * bf16 rounding, not bit for bit.  Inputs are not modified.
 * Errors: as h3_attn_varlen. */
h3_status h3_attn_layer(const void* q, const void* k, const void* v, void* o,
                        const void* w_q, const void* w_k, int64_t w_head_stride, float eps,
                        const h3_rope* rope, float softmax_scale, const h3_shape* shape,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Dense (bf16) attention with Skip-Softmax, the "Skip-Softmax-only" control ([Blog §4.3],
 * figure 6: a tile-level decision from the QK result drops the softmax and P x V work of
 * unimportant tiles; a higher threshold drops more): skip_threshold in (0, 1).  For each
 * query row the valid keys are walked in 64-key tiles; tile t >= 1 is dropped when
 * exp(tile maximum - running maximum of the kept tiles) < skip_threshold (scores
 * s = softmax_scale * q . k), and the row is a softmax over the kept keys.  The result
 * depends only on each row's own scores; work is saved where all 32 rows of a wave drop
 * a tile.  Products and softmax as in h3_attn_varlen (its per-tile running-maximum
 * form).  After the call, the workspace's pass-flag word of each 256-row workgroup
 * (layout at h3_attn_workspace_size) holds the number of 32-row x 64-key wave tiles it
 * skipped.  Same arguments as h3_attn_varlen / h3_attn_layer plus skip_threshold;
 * H3_ERR_SHAPE for a threshold outside (0, 1). */
h3_status h3_attn_varlen_skip(const void* q, const void* k, const void* v, void* o,
                              float softmax_scale, float skip_threshold, const h3_shape* shape,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);
h3_status h3_attn_layer_skip(const void* q, const void* k, const void* v, void* o,
                             const void* w_q, const void* w_k, int64_t w_head_stride, float eps,
                             const h3_rope* rope, float softmax_scale, float skip_threshold,
                             const h3_shape* shape, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* The same layer for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): h3_attn_layer with its
 * workspace in a static 64 MiB device array inside the library instead of a caller
 * buffer.  It calls no hipMalloc, hipFree or allocating library routine; each GPU the
 * library runs on holds its own copy of the array from first use until the process
 * ends.  The caller still passes every input and output.  Output and errors as
 * h3_attn_layer (bit-identical results), plus H3_ERR_SCRATCH_LIMIT, returned before any
 * launch, when h3_attn_workspace_size(shape) exceeds
 * h3_attn_layer_noalloc_max_workspace() (e.g. 8 heads x 8,192 tokens fit, 6 heads x
 * 58,816 do not).  Every call on one GPU shares that GPU's array, so calls that overlap
 * on one GPU (concurrent streams or threads) race; serialise them. */
h3_status h3_attn_layer_noalloc(const void* q, const void* k, const void* v, void* o,
                                const void* w_q, const void* w_k, int64_t w_head_stride,
                                float eps, const h3_rope* rope, float softmax_scale,
                                const h3_shape* shape, hipStream_t stream);

/* Key ranges each 256-row query block of batch `batch` is split into by the attention
 * calls (1: none; 0 for an invalid shape or batch).  Grids of few rounds on the chip's
 * compute units split the keys so that every unit stays busy; the ranges' partial
 * results are combined in a fixed order, so results stay deterministic. */
int h3_attn_splits(const h3_shape* shape, int batch);

/* Bytes of the static scratch behind h3_attn_layer_noalloc (the largest
 * h3_attn_workspace_size it accepts). */
size_t h3_attn_layer_noalloc_max_workspace(void);

/* ---------------------------------------------------------------------------
 * FP8 ("SAGE") attention  ([Blog §4.3], figure 6): the same attention with Q, K, P and
 * V quantized to FP8 E4M3 (OCP "fn": largest finite 448, round to nearest even) for
 * both products on the FP8 matrix cores.  The quantization groups (the reading of
 * "K16"): one scale per Q row, per block of 16 consecutive keys, and per V channel over
 * the N_b valid tokens, each per head; a group's scale is amax / 448 and an element's
 * code is the E4M3 rounding of the exact x * 448 / amax.  The softmax weights
 * are those of a streaming softmax over 64-key tiles: P = E4M3(256 exp(s - m_t)) with
 * m_t the running row maximum through the key's tile, earlier sums carried over by
 * exp(m_(t-1) - m_t); each row is normalised by the sum of its quantized weights.
 * Products accumulate into fp32 (the FP8 matrix cores sum each 64-term product with
 * an error of up to about 2^-11 of its largest term); output rounded to bf16.
 * Deterministic run to run.
 * Accuracy: a few percent relative to exact attention (FP8 keeps 4 significant bits).
 *
 * Skip-Softmax ([Blog §4.3], figure 6: a tile-level decision from the QK result skips
 * the softmax and P x V work of unimportant tiles; a higher threshold skips more):
 * skip_threshold in [0, 1).  For each query row, a 64-key tile after the first is
 * dropped when exp(tile maximum - running maximum before the tile) < skip_threshold
 * (scores s = softmax_scale * q . k); a dropped tile contributes nothing.  The result
 * depends only on each row's own scores (not on how rows are grouped); work is saved
 * where all 32 rows of a wave drop a tile.  0 disables it (dense FP8 attention). */

/* Workspace bytes of the FP8 calls: 64-key tiles of 19,456 bytes,
 * B * H * ceil(S / 64) * 19456 bytes (about 0.59x the bf16 size of K plus V), then the
 * per-channel V maxima, round_up(B * H * 128 * 4, 256) bytes, then the skip counts,
 * round_up(B * H * ceil(S / 256) * 4, 256) bytes: one uint32 per 256 query rows of each
 * head and batch, in that order ([batch][head][row block]), holding the number of
 * (32-row x 64-key) tiles whose work the last h3_attn_packed_fp8 call on this
 * workspace skipped (0 without Skip-Softmax).  0 if the shape is invalid. */
size_t h3_attn_fp8_workspace_size(const h3_shape* shape);

/* FP8 stage 1: quantize K (normalised and rotated first, rounded to bf16, when w_k is
 * non-NULL, exactly as h3_kv_pack) and V of every batch into `workspace` as FP8 tiles
 * with their scales.  Keys >= N_b are stored as zero codes.  Same arguments and errors
 * as h3_kv_pack, with an FP8 workspace (h3_attn_fp8_workspace_size). */
h3_status h3_kv_pack_fp8(const void* k, const void* v, const void* w_k, int64_t w_head_stride,
                         float eps, const h3_rope* rope, const h3_shape* shape, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* FP8 stage 2: attention of Q (normalised and rotated in registers when w_q is non-NULL,
 * then quantized per row) against a workspace filled by h3_kv_pack_fp8 for the same
 * shape, with Skip-Softmax threshold skip_threshold (0: dense).  The tile images are
 * only read; the skip counts after them are written, so two calls sharing one
 * workspace must not overlap in time.  Output rows [N_b, S) are zero.
 * Errors: as h3_kv_pack; H3_ERR_SHAPE for skip_threshold outside [0, 1). */
h3_status h3_attn_packed_fp8(const void* q, void* o, const void* w_q, int64_t w_head_stride,
                             float eps, const h3_rope* rope, float softmax_scale,
                             float skip_threshold, const h3_shape* shape, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* FP8 attention with Q and K already normalised and rotated: h3_kv_pack_fp8 (w_k NULL)
 * then h3_attn_packed_fp8 (w_q NULL).  Arguments and errors as h3_attn_varlen, with an
 * FP8 workspace and the Skip-Softmax threshold (0: dense). */
h3_status h3_attn_varlen_fp8(const void* q, const void* k, const void* v, void* o,
                             float softmax_scale, float skip_threshold, const h3_shape* shape,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The whole layer in FP8: Q/K RMSNorm + RoPE fused (results rounded to bf16, as
 * h3_qk_rmsnorm_rope writes them), then FP8 attention.  Arguments and errors as
 * h3_attn_layer, with an FP8 workspace and the Skip-Softmax threshold (0: dense). */
h3_status h3_attn_layer_fp8(const void* q, const void* k, const void* v, void* o,
                            const void* w_q, const void* w_k, int64_t w_head_stride, float eps,
                            const h3_rope* rope, float softmax_scale, float skip_threshold,
                            const h3_shape* shape, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * DiT block steps around the attention ([Blog §3.2]: the FP32 modulation,
 * normalization and residual computations are merged into one operation).  The pages
 * give no formula; this is the plain adaLN form of a DiT block. */

/* Rows of one or more sequences: x, a and y are [B, S, hidden], contiguous. */
typedef struct {
  int32_t batch;             /* B >= 1                                              */
  int64_t seq_buf;           /* S: rows allocated per sequence                      */
  const int64_t* seq_valid;  /* HOST array [B]: N_b, 0 <= N_b <= S                  */
  int64_t hidden;            /* channels per row: a multiple of 8, at most 8,192    */
} h3_rows;

/* For every valid row t < N_b of batch b, over its `hidden` channels c:
 *   if a != NULL:  x[c] <- x[c] + gate[c] * a[c]   (fp32 fused multiply-add; gate NULL:
 *                  gate 1), written back into x
 *   y[c] = bf16( (x[c] - mean) / sqrt(var + eps) * (1 + scale[c]) + shift[c] )
 * with mean and var the mean and population variance of the row's x (after the
 * update), in fp32.  Rows [N_b, S): y written as +0, x neither read nor written.
 * x: fp32 device [B, S, hidden], read (and updated when a != NULL).  a: bf16 device
 * [B, S, hidden] (e.g. the attention output after its projection) or NULL.  gate,
 * shift, scale: fp32 device vectors of batch b at base + b * mod_batch_stride
 * (mod_batch_stride 0: shared by all batches, else >= hidden and a multiple of 4).
 * y: bf16 device [B, S, hidden]; must not overlap x or a.  All pointers 16-byte aligned.
 * Errors: H3_ERR_NULL, H3_ERR_SHAPE, H3_ERR_ALIGN, H3_ERR_UNSUPPORTED (hidden not a
 * multiple of 8 or above 8,192), H3_ERR_DEVICE, H3_ERR_LAUNCH. */
h3_status h3_residual_norm_modulate(void* x, const void* a, const float* gate,
                                    const float* shift, const float* scale,
                                    int64_t mod_batch_stride, float eps, void* y,
                                    const h3_rows* rows, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_H */
