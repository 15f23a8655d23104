/*
 * h3_oracle.h — fp64 CPU oracle for the packed-sequence DiT attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this code; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no source with the GPU path.
 *
 * What it computes (plain definitions, fp64 throughout, inputs are bf16 bit
 * patterns widened exactly):
 *   1. per-head RMSNorm of Q and K over head_dim, eps inside the square root,
 *      elementwise weight;
 *   2. rotary position embedding, rotate-half pairing (j, j + d/2), either 1-D
 *      (position = packed token index) or 3-axis (channel sections t/h/w,
 *      positions from a row-major (t, h, w) grid);
 *   3. dense non-causal softmax attention over the valid tokens [0, N) only,
 *      two-pass softmax (max, then exp and sum);
 *   4. output rows in [N, S) are exactly zero.
 *
 * Pages cited:
 *   [Blog]  "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
 *           (Chinese translation of the vLLM blog post on serving MiniMax H3).
 *   §1   text, audio and video tokens are denoised jointly as one packed sequence;
 *   §3.1 "长序列注意力与通信": 58,758 valid tokens in a 58,816-token aligned buffer,
 *        attention receives the valid length and the structural tail padding is
 *        removed; only local embedding/RoPE rows are built; 128-channel head
 *        projections versus the 5,376-channel hidden state;
 *   §3.2 "融合的 DiT 算子": Q/K RMSNorm and RoPE form one fused operator;
 *   §3.5 "基础 H3 的实测结果": "lossless" speed-ups are not bitwise identical,
 *        so GPU results are compared to this oracle within a tolerance.
 * The numeric conventions the pages leave open (eps = 1e-6, RoPE theta = 1e4,
 * half-split pairing, softmax scale 1/sqrt(head_dim), 3-axis sections 32/48/48)
 * are the layer's stated workload parameters; they are passed in, not assumed.
 *
 * Parity status: every function here is pinned by closed-form tests
 * (tests/test_oracle_pins.py); none is "parity unpinned".
 */
#ifndef H3_ORACLE_H
#define H3_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Rotary descriptor, oracle-side.  Tokens [0, n_1d) use 1-D rotation at
 * position = token index over all head_dim channels.  Tokens i >= n_1d use the
 * 3-axis rotation: k = i - n_1d, (t, h, w) = (k / (gh*gw), (k / gw) % gh, k % gw);
 * channel sections of sizes sections[0..2] at consecutive offsets rotate by the
 * t, h and w positions respectively. */
typedef struct {
  double theta;
  int64_t n_1d;
  int32_t sections[3];
  int32_t grid_t, grid_h, grid_w;
} h3o_rope;

/* Return codes. */
enum { H3O_OK = 0, H3O_ERR_ARG = 1 };

/* bf16 bit patterns -> double, exact. */
void h3o_widen_bf16(const uint16_t* src, int64_t n, double* dst);

/* RMSNorm of one row of length d: y_c = x_c / sqrt(mean(x^2) + eps) * w_c. */
void h3o_rmsnorm_row(const double* x, const double* w, int64_t d, double eps, double* y);

/* Rotary embedding of one row of length d (in -> out, may alias).
 * mode 0: 1-D at position pos[0] over all d channels (pairs (j, j + d/2),
 *         frequency theta^(-2j/d)).
 * mode 1: 3-axis; section s covers sections[s] channels starting after the
 *         previous sections, pairs (off + j, off + j + sections[s]/2), frequency
 *         theta^(-2j/sections[s]), angle pos[s] * frequency. */
int h3o_rope_row(const double* in, int64_t d, int mode, const double pos[3],
                 const int32_t sections[3], double theta, double* out);

/* Position of packed token i under descriptor r: writes mode (0: 1-D, 1: 3-axis)
 * and pos[3].  Returns H3O_ERR_ARG if i lies beyond the 3-axis grid. */
int h3o_token_position(const h3o_rope* r, int64_t i, int* mode, double pos[3]);

/* RMSNorm then RoPE of selected tokens, all heads.
 * x: bf16 bits, token t head h channel c at x[t*row_stride + h*d + c].
 * w: bf16 bits, head h channel c at w[h*w_head_stride + c] (w_head_stride 0: shared).
 * rows[n_rows]: token indices, each < n_valid.  out: [n_rows][heads][d]. */
int h3o_prologue(const uint16_t* x, int64_t heads, int64_t d, int64_t row_stride,
                 int64_t n_valid, const uint16_t* w, int64_t w_head_stride, double eps,
                 const h3o_rope* rope, const int64_t* rows, int64_t n_rows, int threads,
                 double* out);

/* Softmax attention on already-prepared fp64 operands.
 * q: [n_rows][heads][d] (query rows), k, v: [n_valid][heads][d] (all valid keys).
 * out: [n_rows][heads][d];  o = sum_j exp(s_j - max s) v_j / sum_j exp(s_j - max s),
 * s_j = scale * q . k_j.  n_valid == 0 gives zeros. */
int h3o_attention(const double* q, const double* k, const double* v, int64_t n_rows,
                  int64_t n_valid, int64_t heads, int64_t d, double scale, int threads,
                  double* out);

/* Attention on bf16 buffers whose Q and K are already normalised and rotated.
 * q, k, v: bf16 bits, [S rows][row_stride].  rows[n_rows] in [0, S): rows >= n_valid
 * give exact zeros.  out: [n_rows][heads][d]. */
int h3o_attn_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_buf,
                    int64_t n_valid, int64_t heads, int64_t d, int64_t row_stride,
                    double scale, const int64_t* rows, int64_t n_rows, int threads,
                    double* out);

/* The whole layer: prologue of Q (selected rows) and K (all valid rows), then
 * attention.  Same layouts as above; rows >= n_valid give exact zeros. */
int h3o_attn_layer(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_buf,
                   int64_t n_valid, int64_t heads, int64_t d, int64_t row_stride,
                   const uint16_t* w_q, const uint16_t* w_k, int64_t w_head_stride,
                   double eps, const h3o_rope* rope, double scale, const int64_t* rows,
                   int64_t n_rows, int threads, double* out);

/* ---- FP8 ("SAGE") variant: see h3_oracle_fp8.cpp for the method and its readings. */

/* Nearest FP8 E4M3 value (OCP "fn": bias 7, max 448, subnormals), ties to even,
 * saturating at +-448.  NaN stays NaN. */
double h3o_e4m3(double x);

/* Nearest bf16 of x (ties to even), as bits. */
uint16_t h3o_round_bf16(double x);

/* Quantize n values (bf16 values passed as fp32, so exact) with one scale: codes[i] =
 * E4M3(x[i] * 448 / amax) as values, evaluated in fp64; *scale = amax / 448 (0 if all
 * zero). */
void h3o_quantize_group(const float* x, int64_t n, double* codes, double* scale);

/* FP8 attention on bf16 buffers whose Q and K are already normalised and rotated
 * (same layouts and row semantics as h3o_attn_varlen), fp64 throughout: Q quantized per
 * token, K per 16-key block, V per channel; the weights P quantized against the running
 * row maximum of tiles of p_tile keys; with skip_threshold > 0 a tile whose maximum is
 * below the running maximum by a factor under skip_threshold is dropped for that row
 * (Skip-Softmax).  wmax (optional, [n_rows][heads]): each row's largest normalised
 * weight (0 for rows >= n_valid). */
int h3o_attn_varlen_fp8(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        int64_t seq_buf, int64_t n_valid, int64_t heads, int64_t d,
                        int64_t row_stride, double scale, int64_t p_tile, double skip_threshold,
                        const int64_t* rows, int64_t n_rows, int threads, double* out,
                        double* wmax);

/* The FP8 layer: prologue of Q and K (fp64, rounded to bf16), then h3o_attn_varlen_fp8. */
int h3o_attn_layer_fp8(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t seq_buf,
                       int64_t n_valid, int64_t heads, int64_t d, int64_t row_stride,
                       const uint16_t* w_q, const uint16_t* w_k, int64_t w_head_stride,
                       double eps, const h3o_rope* rope, double scale, int64_t p_tile,
                       double skip_threshold, const int64_t* rows, int64_t n_rows, int threads,
                       double* out, double* wmax);

/* ---- Dense attention with Skip-Softmax (the "Skip-Softmax-only" control): see
 * h3_oracle_skip.cpp.  Same layouts and row semantics as h3o_attn_varlen; the keys are
 * walked in tiles of p_tile keys and tile t >= 1 is dropped for a row when
 * exp(tile max - running max of the kept tiles) < skip_threshold; the row is a softmax
 * over the kept keys.  wmax (optional, [n_rows][heads]): each row's largest normalised
 * weight.  The layer form applies the fp64 prologue (h3o_prologue) to Q and K first. */
int h3o_attn_varlen_skip(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         int64_t seq_buf, int64_t n_valid, int64_t heads, int64_t d,
                         int64_t row_stride, double scale, int64_t p_tile,
                         double skip_threshold, const int64_t* rows, int64_t n_rows,
                         int threads, double* out, double* wmax);
int h3o_attn_layer_skip(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        int64_t seq_buf, int64_t n_valid, int64_t heads, int64_t d,
                        int64_t row_stride, const uint16_t* w_q, const uint16_t* w_k,
                        int64_t w_head_stride, double eps, const h3o_rope* rope, double scale,
                        int64_t p_tile, double skip_threshold, const int64_t* rows,
                        int64_t n_rows, int threads, double* out, double* wmax);

/* ---- DiT block steps around attention: see h3_oracle_block.cpp for the reading. */

/* One sequence of seq_buf rows of `hidden` channels: for rows t < n_valid,
 * x_out = x + gate * a (a bf16 bits; a NULL: x; gate NULL: 1), y = LayerNorm(x_out)
 * * (1 + scale) + shift (population variance, eps inside the square root); rows
 * t >= n_valid: x_out = x, y = 0.  fp64 throughout. */
int h3o_residual_norm_modulate(const float* x, const uint16_t* a, const float* gate,
                               const float* shift, const float* scale, int64_t seq_buf,
                               int64_t n_valid, int64_t hidden, double eps, double* x_out,
                               double* y_out);

#ifdef __cplusplus
}
#endif

#endif /* H3_ORACLE_H */
