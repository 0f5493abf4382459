/*
 * CPU oracle for MLA decode — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It is a plain, slow, float64 implementation of what an
 * MLA decode step computes, written from the pages' statement of the method,
 * and it shares no code with the GPU library.
 *
 * Parity status of every function is listed in oracle.c's header.
 */
#ifndef MLA_ORACLE_H
#define MLA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage formats understood by the oracle's element decoder */
enum {
  ORACLE_F32 = 0,  /* IEEE-754 binary32 */
  ORACLE_BF16 = 1, /* upper 16 bits of binary32 */
  ORACLE_E4M3 = 2, /* OCP FP8 E4M3 (bias 7, no Inf, S.1111.111 = NaN) */
  ORACLE_F64 = 3   /* IEEE-754 binary64 */
};

typedef struct {
  int32_t B, H, d_nope, d_rope, d_latent, d_v;
  double scale; /* softmax scale; <= 0 selects 1/sqrt(d_nope + d_rope) */
  const void* q_nope; /* [B][H][d_nope] */
  const void* q_rope; /* [B][H][d_rope] */
  int32_t q_dtype;
  const void* w_uk; /* [H][d_nope][d_latent] */
  const void* w_uv; /* [H][d_v][d_latent] */
  int32_t w_dtype;
  const void* rows; /* cache rows of d_latent + d_rope elements: [c_KV | k_R] */
  const float* row_scale; /* E4M3 cache: one factor per row, else NULL */
  int32_t cache_dtype;
  int32_t page_size;          /* 0: row of token t of seq b = b*seq_stride + t */
  int64_t seq_stride;
  const int32_t* block_table; /* paged: row = block_table[b*max_pages + t/ps]*ps + t%ps */
  int32_t max_pages;
  const int32_t* seq_lens; /* [B] */
  int32_t ring; /* contiguous only: 1 = each sequence's seq_stride rows are a ring */
} oracle_mla_problem;

/* Naive decode: rebuild K and V per cached token, then textbook attention.
 * sel_b/sel_h (n_sel pairs) choose the outputs; NULL computes all B*H in
 * (b, h) order.  t_begin/t_end (per sequence, may be NULL) restrict the
 * attended tokens to [t_begin[b], t_end[b]).  Outputs per selected pair:
 * o [d_v], lse (natural log; -inf when no token is attended), and optionally
 * u [d_latent] = softmax-weighted mean of the cached latents.  Returns 0, or
 * a negative value on a bad argument. */
int oracle_mla_decode(const oracle_mla_problem* P, const int32_t* sel_b,
                      const int32_t* sel_h, int32_t n_sel, const int32_t* t_begin,
                      const int32_t* t_end, double* o, double* lse, double* u);

/* The naive form's per-head keys and values of sequence b's tokens
 * [t_begin, t_end): k [H][n_t][d_nope + d_rope] = [W_UK[h] c_t ; k_R,t],
 * v [H][n_t][d_v] = W_UV[h] c_t, float64. */
int oracle_rebuild_kv(const oracle_mla_problem* P, int32_t b, int32_t t_begin, int32_t t_end,
                      double* k, double* v);

/* Absorbed-form attention for a given absorbed query q_abs
 * [B][H][d_latent + d_rope] (q_dtype; E4M3 with one factor per (b, h) in
 * q_scale): s_t = scale * q_abs . row_t over the whole cached row, softmax,
 * u = sum_t p_t c_KV,t / sum_t p_t, lse = log sum_t e^{s_t}, and optionally
 * o = W_UV[h] u.  P gives the cache, d_latent, d_rope, d_v, the scale (d_nope
 * only for the default 1/sqrt(d_nope + d_rope)) and W_UV; its query fields are
 * not read.  Selection and token ranges as in oracle_mla_decode. */
int oracle_absorbed_decode(const oracle_mla_problem* P, const void* q_abs, int32_t q_dtype,
                           const float* q_scale, const int32_t* sel_b, const int32_t* sel_h,
                           int32_t n_sel, const int32_t* t_begin, const int32_t* t_end,
                           double* u, double* lse, double* o);

/* E4M3 rows with one fp32 factor each, the rule of oracle_cache_append's E4M3
 * cache: x [n][w] binary32 -> codes [n][w], scale [n]. */
int oracle_quantize_e4m3_rows(int64_t n, int32_t w, const float* x, uint8_t* codes,
                              float* scale);

/* q_abs[b][h][:d_latent] = sum_n q_nope[b][h][n] * W_UK[h][n][:] ;
 * q_abs[b][h][d_latent:] = q_rope[b][h][:]  (float64 out) */
int oracle_absorb_q(int32_t B, int32_t H, int32_t d_nope, int32_t d_rope,
                    int32_t d_latent, const void* q_nope, const void* q_rope,
                    int32_t q_dtype, const void* w_uk, int32_t w_dtype,
                    double* q_abs);

/* Merge S partial softmax results: lse = log sum_p exp(lse_p),
 * u = sum_p exp(lse_p - lse) u_p.  u_part [B][S][H][D], lse_part [B][S][H]. */
int oracle_combine(int32_t B, int32_t S, int32_t H, int32_t D,
                   const double* u_part, const double* lse_part, double* u,
                   double* lse);

/* o[b][h][v] = sum_c W_UV[h][v][c] * u[b][h][c] */
int oracle_up_proj(int32_t B, int32_t H, int32_t d_v, int32_t d_latent,
                   const double* u, const void* w_uv, int32_t w_dtype, double* o);

/* Append one token per sequence to the cache ([V2] §2.3: per token only the
 * latent c_KV and the shared RoPE key k_R are cached; [DSA]: the 128K cache is
 * kept in FP8).  For every b with 0 <= positions[b] < capacity (contiguous:
 * seq_stride rows per sequence; paged: max_pages * page_size), the row of
 * token positions[b] (same row map as oracle_mla_problem) becomes
 * [c_kv[b][0:d_latent] | k_r[b][0:d_rope]] in the cache dtype:
 *   F32   the input value (exact from F32 or BF16 input);
 *   BF16  the input rounded to nearest even (a copy for BF16 input);
 *   E4M3  one fp32 factor per row, s = fl32(max(amax, 2^-126) / 448) with amax
 *         the largest |value| of the row, stored in row_scale[row]; each code is
 *         the E4M3 value nearest to fl32(x / s) (ties to even mantissa), with
 *         |fl32(x / s)| first clamped to 448.
 * Other positions, and positions whose page id is negative, are skipped; no
 * other row is touched.  Inputs [B][d] in
 * src_dtype (F32 or BF16), finite.  Returns 0, or a negative value on a bad
 * argument. */
int oracle_cache_append(int32_t B, int32_t d_latent, int32_t d_rope, const void* c_kv,
                        const void* k_r, int32_t src_dtype, const int32_t* positions,
                        void* rows, int32_t cache_dtype, float* row_scale, int32_t page_size,
                        int64_t seq_stride, const int32_t* block_table, int32_t max_pages,
                        int32_t ring);

int oracle_ring_grow(int32_t B, int32_t row_bytes, const int32_t* seq_lens, const void* src,
                     const float* src_scale, int64_t src_cap, void* dst, float* dst_scale,
                     int64_t dst_cap);

/* Multi-head attention decode over a full per-head K/V cache, the baseline
 * the latent cache replaces ([LAT] §2.1 textbook attention
 * softmax(q k^T / sqrt(d_k)) v; [V2] §1.1 the MHA cache holds K and V of
 * every head):
 *   o[b][i] = sum_t p_t v[b][i][t] / sum_t p_t,  p_t = exp(s_t - max s),
 *   s_t = scale * q[b][i] . k[b][i][t],  t < seq_lens[b],
 * scale <= 0 means 1/sqrt(d_qk).  q [B][H][d_qk]; k [B][H][seq_stride][d_qk]
 * and v [B][H][seq_stride][d_v] (head-major) in dtype; o [B][H][d_v] and
 * lse [B][H] (natural log, -inf for an empty sequence) in float64.  Returns 0,
 * or a negative value on a bad argument. */
int oracle_mha_decode(int32_t B, int32_t H, int32_t d_qk, int32_t d_v, const void* q,
                      const void* k, const void* v, int32_t dtype, const int32_t* seq_lens,
                      int64_t seq_stride, double scale, double* o, double* lse);

/* Decoupled RoPE of the positional query ([V2] §2.2: only q_R and k_R are
 * rotated, q_C is left as it is; frequencies 1/10000^(2i/d) as in the
 * listings of [V2] and [LAT]; the [LAT] listing repeats the d/2 frequencies
 * over both halves, so element i pairs with element i + d/2, rotate-half):
 *   inv_freq[i] = binary32 nearest to base^(-2i/d_r), i < d_r/2,
 *   theta_i     = binary32 product position * inv_freq[i] (the listings work
 *                 in float32),
 *   out[i]          = x[i] cos theta_i - x[i + d_r/2] sin theta_i,
 *   out[i + d_r/2]  = x[i + d_r/2] cos theta_i + x[i] sin theta_i,
 * cos and sin in float64.  x [B][H][d_r] in dtype, positions [B] (one per
 * sequence: every head of a token shares its position); out float64.
 * Returns 0, or a negative value on a bad argument. */
int oracle_gqa_decode(int32_t B, int32_t H, int32_t H_kv, int32_t d_qk, int32_t d_v,
                      const void* q, const void* k, const void* v, int32_t dtype,
                      const int32_t* seq_lens, int64_t seq_stride, double scale, double* o,
                      double* lse);

int oracle_rope(int32_t B, int32_t H, int32_t d_r, const void* x, int32_t dtype,
                const int32_t* positions, double base, double* out);

/* inv_freq[i] of oracle_rope for i < d_r/2 */
void oracle_rope_inv_freq(int32_t d_r, double base, float* inv_freq);

/* The E4M3 code nearest to the binary32 value y (|y| <= 448, finite), ties to
 * the even mantissa. */
uint8_t oracle_encode_e4m3(float y);

/* element decoders (exact) */
double oracle_decode_bf16(uint16_t bits);
double oracle_decode_e4m3(uint8_t code);
void oracle_decode_array(const void* src, int32_t dtype, int64_t n, double* dst);

/* cache-size arithmetic */
int64_t oracle_mla_cache_bytes_per_token(int32_t d_latent, int32_t d_rope,
                                         int32_t elem_bytes, int32_t scale_bytes);
int64_t oracle_mha_cache_bytes(int64_t layers, int64_t seq_len, int64_t heads,
                               int64_t head_dim, int64_t elem_bytes);

int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
