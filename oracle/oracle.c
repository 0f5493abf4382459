/*
 * CPU oracle for MLA decode — TEST INFRASTRUCTURE ONLY.
 *
 * Callers: the tests, the smoke check and the benchmark's CPU-baseline leg.
 * Nothing on the product path may load it.  It shares no code, header, table
 * or helper with the GPU library.
 *
 * What it computes is the plain, non-absorbed MLA decode, in float64:
 * for every cached token the full key and value of each head are rebuilt from
 * the token's latent, then textbook softmax attention runs over them.  The
 * pages:
 *   [V2]  "DeepSeek V2的MLA注意力机制：如何用低秩压缩技术降低KV Cache显存消耗？"
 *         (snabindia.com) — §2.1 low-rank reconstruction K = W_U^K·KV_comp,
 *         V = W_U^V·KV_comp; §2.2 decoupled RoPE: a content query q_C, a
 *         positional query q_R and ONE positional key k_R shared by all heads;
 *         §2.3 only KV_comp and k_R are cached, the score is the product of the
 *         concatenations (q_C q_R)(K_C K_R)^T over sqrt(d), and absorbing W_U^K
 *         into the query / W_U^V into the output is exact algebra;
 *         §1.1 MHA cache size 2 x layers x seq x h x d (x bytes).
 *   [LAT] "Multi-Head Latent Attention（MLA）：大模型KV Cache显存优化原理与实操"
 *         (CSDN mirror) — §2.1 Attention(Q,K,V) = softmax(QK^T/sqrt(d_k)) V and
 *         the MHA cache bytes per token; §3.2 the latent cache is a 2-D
 *         [seq, latent] array per sequence, read by slicing.
 *   [DSA] "engineering DeepSeek sparse attention long context inference"
 *         (blog.hotdry.top) — the MLA module listing: cache the latent, rebuild
 *         k and v with the up-projections, then attention.
 * Readings taken where the pages are silent (the softmax scale is
 * 1/sqrt(d_nope + d_rope); W_UK is [h][d_nope][d_latent] and W_UV is
 * [h][d_v][d_latent], the nn.Linear layout of the [DSA] listing; one 576-wide
 * row per token holds [c_KV | k_R]; e4m3 rows carry one fp32 factor; every
 * cached token is attended, no mask) are listed with the tests that pin them.
 * Ring cache ([V2] §4.1 keeps the KV cache in a ring buffer so that it can
 * grow): a sequence's seq_stride rows are a ring of that capacity C, token t
 * sits in row t mod C, so the ring holds the last min(L, C) tokens and those
 * are the ones attended (a window of C tokens once L > C); growing moves that
 * window into a larger ring, token t to row t mod C'.
 *
 * Pins (tests/test_oracle_*.py): library SDPA over explicitly rebuilt K/V,
 * the absorbed-form identity, closed forms (one token, zero query, dominant
 * key), invariants (score shift, token and head permutation, split+merge,
 * paged vs contiguous, unread NaN slots, linearity in W_UV), exhaustive codec
 * tables against torch's bfloat16 / float8_e4m3fn, and the pages' printed
 * cache sizes.  No function here is "parity unpinned".
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- decoders */

double oracle_decode_bf16(uint16_t bits) {
  /* bfloat16 is the upper half of an IEEE-754 binary32 */
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double oracle_decode_e4m3(uint8_t code) {
  /* OCP 8-bit floating point spec, E4M3: 1 sign, 4 exponent (bias 7),
   * 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
   * there are no infinities. */
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, 1 - 7);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

static double load_elem(const void* base, int32_t dtype, int64_t i) {
  switch (dtype) {
    case ORACLE_F32: return (double)((const float*)base)[i];
    case ORACLE_BF16: return oracle_decode_bf16(((const uint16_t*)base)[i]);
    case ORACLE_E4M3: return oracle_decode_e4m3(((const uint8_t*)base)[i]);
    case ORACLE_F64: return ((const double*)base)[i];
    default: return NAN;
  }
}

void oracle_decode_array(const void* src, int32_t dtype, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, dtype, i);
}

static int valid_dtype(int32_t d) { return d >= ORACLE_F32 && d <= ORACLE_F64; }

/* --------------------------------------------------------- cache addressing */

/* physical row of token t of sequence b: contiguous [b][seq_stride] rows, or a
 * page of page_size rows named by the block table ([V2] §1.2/§3.3 paging) */
static int64_t row_of(const oracle_mla_problem* P, int32_t b, int64_t t) {
  if (P->ring) return (int64_t)b * P->seq_stride + t % P->seq_stride;
  if (P->page_size > 0) {
    int64_t page = P->block_table[(int64_t)b * P->max_pages + t / P->page_size];
    return page * P->page_size + t % P->page_size;
  }
  return (int64_t)b * P->seq_stride + t;
}

/* decode one cached row [c_KV | k_R] to float64; e4m3 rows are multiplied by
 * their per-row factor */
static void load_row(const oracle_mla_problem* P, int64_t r, double* c) {
  const int32_t w = P->d_latent + P->d_rope;
  double f = 1.0;
  if (P->cache_dtype == ORACLE_E4M3) f = (double)P->row_scale[r];
  for (int32_t j = 0; j < w; ++j) c[j] = load_elem(P->rows, P->cache_dtype, r * w + j) * f;
}

/* ----------------------------------------------------------- naive decode */

int oracle_mla_decode(const oracle_mla_problem* P, const int32_t* sel_b,
                      const int32_t* sel_h, int32_t n_sel, const int32_t* t_begin,
                      const int32_t* t_end, double* o, double* lse, double* u) {
  if (!P || !o || !lse) return -1;
  if (P->B < 0 || P->H <= 0 || P->d_nope <= 0 || P->d_rope < 0 || P->d_latent <= 0 ||
      P->d_v <= 0)
    return -2;
  if (!valid_dtype(P->q_dtype) || !valid_dtype(P->w_dtype) || !valid_dtype(P->cache_dtype))
    return -3;
  if (P->cache_dtype == ORACLE_E4M3 && !P->row_scale) return -4;
  if (P->page_size > 0 && !P->block_table) return -5;
  if (P->ring && (P->page_size > 0 || P->seq_stride < 1)) return -7;
  const int32_t all = (sel_b == NULL);
  const int64_t n = all ? (int64_t)P->B * P->H : n_sel;
  const double scale =
      P->scale > 0 ? P->scale : 1.0 / sqrt((double)(P->d_nope + P->d_rope));
  const int32_t dn = P->d_nope, dr = P->d_rope, dl = P->d_latent, dv = P->d_v;
  int err = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t idx = 0; idx < n; ++idx) {
    const int32_t b = all ? (int32_t)(idx / P->H) : sel_b[idx];
    const int32_t h = all ? (int32_t)(idx % P->H) : sel_h[idx];
    if (b < 0 || b >= P->B || h < 0 || h >= P->H) {
      err = -6;
      continue;
    }
    int64_t L = P->seq_lens[b];
    int64_t t0 = t_begin ? t_begin[b] : 0;
    int64_t t1 = t_end ? t_end[b] : L;
    if (t0 < 0) t0 = 0;
    if (t1 > L) t1 = L;
    /* a ring of C rows keeps only the last C tokens */
    if (P->ring && t0 < L - P->seq_stride) t0 = L - P->seq_stride;
    double* out_o = o + idx * dv;
    double* out_u = u ? u + idx * dl : NULL;
    for (int32_t v = 0; v < dv; ++v) out_o[v] = 0.0;
    if (out_u)
      for (int32_t j = 0; j < dl; ++j) out_u[j] = 0.0;
    if (t1 <= t0) {
      lse[idx] = -INFINITY;
      continue;
    }
    const int64_t nt = t1 - t0;
    double* Wk = malloc(sizeof(double) * dn * dl);
    double* Wv = malloc(sizeof(double) * dv * dl);
    double* qc = malloc(sizeof(double) * dn);
    double* qr = malloc(sizeof(double) * (dr > 0 ? dr : 1));
    double* c = malloc(sizeof(double) * (dl + dr));
    double* k = malloc(sizeof(double) * dn);
    double* vv = malloc(sizeof(double) * dv);
    double* s = malloc(sizeof(double) * nt);
    for (int64_t i = 0; i < (int64_t)dn * dl; ++i)
      Wk[i] = load_elem(P->w_uk, P->w_dtype, (int64_t)h * dn * dl + i);
    for (int64_t i = 0; i < (int64_t)dv * dl; ++i)
      Wv[i] = load_elem(P->w_uv, P->w_dtype, (int64_t)h * dv * dl + i);
    for (int32_t i = 0; i < dn; ++i)
      qc[i] = load_elem(P->q_nope, P->q_dtype, ((int64_t)b * P->H + h) * dn + i);
    for (int32_t i = 0; i < dr; ++i)
      qr[i] = load_elem(P->q_rope, P->q_dtype, ((int64_t)b * P->H + h) * dr + i);

    /* pass 1: scores.  The key of head h for token t is the concatenation of
     * the rebuilt content key W_UK[h]·c_t ([V2] §2.1) and the shared
     * positional key k_R,t ([V2] §2.2); the query is [q_C ; q_R]; the score is
     * their dot product times the softmax scale ([V2] §2.3, [LAT] §2.1). */
    for (int64_t t = 0; t < nt; ++t) {
      load_row(P, row_of(P, b, t0 + t), c);
      for (int32_t i = 0; i < dn; ++i) {
        double acc = 0.0;
        const double* wr = Wk + (int64_t)i * dl;
        for (int32_t j = 0; j < dl; ++j) acc += wr[j] * c[j];
        k[i] = acc;
      }
      double dot = 0.0;
      for (int32_t i = 0; i < dn; ++i) dot += qc[i] * k[i];
      for (int32_t i = 0; i < dr; ++i) dot += qr[i] * c[dl + i];
      s[t] = scale * dot;
    }
    /* softmax over the attended tokens ([LAT] §2.1) */
    double m = -INFINITY;
    for (int64_t t = 0; t < nt; ++t)
      if (s[t] > m) m = s[t];
    double l = 0.0;
    for (int64_t t = 0; t < nt; ++t) {
      s[t] = exp(s[t] - m);
      l += s[t];
    }
    /* pass 2: weighted sum of the rebuilt values W_UV[h]·c_t ([V2] §2.1) */
    for (int64_t t = 0; t < nt; ++t) {
      load_row(P, row_of(P, b, t0 + t), c);
      for (int32_t i = 0; i < dv; ++i) {
        double acc = 0.0;
        const double* wr = Wv + (int64_t)i * dl;
        for (int32_t j = 0; j < dl; ++j) acc += wr[j] * c[j];
        vv[i] = acc;
      }
      for (int32_t i = 0; i < dv; ++i) out_o[i] += s[t] * vv[i];
      if (out_u)
        for (int32_t j = 0; j < dl; ++j) out_u[j] += s[t] * c[j];
    }
    for (int32_t i = 0; i < dv; ++i) out_o[i] /= l;
    if (out_u)
      for (int32_t j = 0; j < dl; ++j) out_u[j] /= l;
    lse[idx] = m + log(l);
    free(Wk); free(Wv); free(qc); free(qr); free(c); free(k); free(vv); free(s);
  }
  return err;
}

/* The naive form's rebuild ([V2] §2.1, [DSA]'s MLA listing): for sequence b
 * and every cached token t in [t_begin, t_end), each head's key is the
 * concatenation of the rebuilt content key W_UK[h]·c_t and the shared k_R,t
 * ([V2] §2.2), and its value W_UV[h]·c_t.  k [H][n_t][d_nope + d_rope],
 * v [H][n_t][d_v], n_t = t_end - t_begin, float64. */
int oracle_rebuild_kv(const oracle_mla_problem* P, int32_t b, int32_t t_begin, int32_t t_end,
                      double* k, double* v) {
  if (!P || !k || !v || b < 0 || b >= P->B || t_begin < 0 || t_end < t_begin) return -1;
  const int32_t dn = P->d_nope, dr = P->d_rope, dl = P->d_latent, dv = P->d_v;
  const int64_t nt = t_end - t_begin;
  double* c = malloc(sizeof(double) * (dl + dr));
  if (!c) return -5;
  for (int64_t t = 0; t < nt; ++t) {
    load_row(P, row_of(P, b, t_begin + t), c);
    for (int32_t h = 0; h < P->H; ++h) {
      double* kr = k + ((int64_t)h * nt + t) * (dn + dr);
      double* vr = v + ((int64_t)h * nt + t) * dv;
      for (int32_t i = 0; i < dn; ++i) {
        double acc = 0.0;
        for (int32_t j = 0; j < dl; ++j)
          acc += load_elem(P->w_uk, P->w_dtype, ((int64_t)h * dn + i) * dl + j) * c[j];
        kr[i] = acc;
      }
      for (int32_t i = 0; i < dr; ++i) kr[dn + i] = c[dl + i];
      for (int32_t i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int32_t j = 0; j < dl; ++j)
          acc += load_elem(P->w_uv, P->w_dtype, ((int64_t)h * dv + i) * dl + j) * c[j];
        vr[i] = acc;
      }
    }
  }
  free(c);
  return 0;
}

/* Attention of an absorbed query over the cached latent rows ([V2] §2.3:
 * with W_UK folded into the query the score of token t is the dot product of
 * the query row [q~ | q_R] with the cached row [c_KV | k_R], times the softmax
 * scale; the weights multiply c_KV itself, and W_UV is applied to the weighted
 * mean afterwards).  q_abs [B][H][d_latent + d_rope] in q_dtype; an E4M3
 * query carries one factor per (b, h) in q_scale (value = code x factor, the
 * rows' own convention).  Cache, selection and token ranges as in
 * oracle_mla_decode.  Outputs per selected pair: u [d_latent], lse, and
 * o [d_v] = W_UV[h] u when o is not NULL (P->w_uv, P->w_dtype). */
int oracle_absorbed_decode(const oracle_mla_problem* P, const void* q_abs, int32_t q_dtype,
                           const float* q_scale, const int32_t* sel_b, const int32_t* sel_h,
                           int32_t n_sel, const int32_t* t_begin, const int32_t* t_end,
                           double* u, double* lse, double* o) {
  if (!P || !q_abs || !u || !lse) return -1;
  if (P->B < 0 || P->H <= 0 || P->d_rope < 0 || P->d_latent <= 0 || (o && P->d_v <= 0)) return -2;
  if (!valid_dtype(q_dtype) || !valid_dtype(P->cache_dtype) || (o && !valid_dtype(P->w_dtype)))
    return -3;
  if ((q_dtype == ORACLE_E4M3 && !q_scale) || (P->cache_dtype == ORACLE_E4M3 && !P->row_scale))
    return -4;
  if (P->page_size > 0 && !P->block_table) return -5;
  if (P->ring && (P->page_size > 0 || P->seq_stride < 1)) return -7;
  if (o && !P->w_uv) return -1;
  const int32_t all = (sel_b == NULL);
  const int64_t n = all ? (int64_t)P->B * P->H : n_sel;
  const double scale =
      P->scale > 0 ? P->scale : 1.0 / sqrt((double)P->d_nope + (double)P->d_rope);
  const int32_t dl = P->d_latent, w = P->d_latent + P->d_rope;
  int err = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t idx = 0; idx < n; ++idx) {
    const int32_t b = all ? (int32_t)(idx / P->H) : sel_b[idx];
    const int32_t h = all ? (int32_t)(idx % P->H) : sel_h[idx];
    if (b < 0 || b >= P->B || h < 0 || h >= P->H) {
      err = -6;
      continue;
    }
    int64_t L = P->seq_lens[b];
    int64_t t0 = t_begin ? t_begin[b] : 0;
    int64_t t1 = t_end ? t_end[b] : L;
    if (t0 < 0) t0 = 0;
    if (t1 > L) t1 = L;
    if (P->ring && L - t0 > P->seq_stride) t0 = L - P->seq_stride; /* ring window */
    double* out_u = u + idx * dl;
    for (int32_t j = 0; j < dl; ++j) out_u[j] = 0.0;
    if (o)
      for (int32_t v = 0; v < P->d_v; ++v) o[idx * P->d_v + v] = 0.0;
    if (t1 <= t0) {
      lse[idx] = -INFINITY;
      continue;
    }
    const int64_t nt = t1 - t0;
    double* q = malloc(sizeof(double) * w);
    double* c = malloc(sizeof(double) * w);
    double* s = malloc(sizeof(double) * nt);
    const int64_t qrow = (int64_t)b * P->H + h;
    const double qf = q_dtype == ORACLE_E4M3 ? (double)q_scale[qrow] : 1.0;
    for (int32_t j = 0; j < w; ++j) q[j] = load_elem(q_abs, q_dtype, qrow * w + j) * qf;
    /* scores over the whole 576-wide rows */
    for (int64_t t = 0; t < nt; ++t) {
      load_row(P, row_of(P, b, t0 + t), c);
      double dot = 0.0;
      for (int32_t j = 0; j < w; ++j) dot += q[j] * c[j];
      s[t] = scale * dot;
    }
    double m = -INFINITY;
    for (int64_t t = 0; t < nt; ++t)
      if (s[t] > m) m = s[t];
    double l = 0.0;
    for (int64_t t = 0; t < nt; ++t) {
      s[t] = exp(s[t] - m);
      l += s[t];
    }
    /* weighted mean of the latents c_KV */
    for (int64_t t = 0; t < nt; ++t) {
      load_row(P, row_of(P, b, t0 + t), c);
      for (int32_t j = 0; j < dl; ++j) out_u[j] += s[t] * c[j];
    }
    for (int32_t j = 0; j < dl; ++j) out_u[j] /= l;
    lse[idx] = log(l) + m;
    if (o)
      for (int32_t v = 0; v < P->d_v; ++v) {
        double acc = 0.0;
        for (int32_t j = 0; j < dl; ++j)
          acc += load_elem(P->w_uv, P->w_dtype, ((int64_t)h * P->d_v + v) * dl + j) * out_u[j];
        o[idx * P->d_v + v] = acc;
      }
    free(q); free(c); free(s);
  }
  return err;
}

/* ------------------------------------------------------- the other calls */

/* Absorbing W_UK into the query ([V2] §2.3, §4.1): the content score
 * q_C·(W_UK c) equals (W_UK^T q_C)·c, so the absorbed query is
 * sum_n q_C[n] W_UK[n][:]; the RoPE part is carried unchanged. */
int oracle_absorb_q(int32_t B, int32_t H, int32_t d_nope, int32_t d_rope,
                    int32_t d_latent, const void* q_nope, const void* q_rope,
                    int32_t q_dtype, const void* w_uk, int32_t w_dtype,
                    double* q_abs) {
  if (B < 0 || H <= 0 || d_nope <= 0 || d_rope < 0 || d_latent <= 0 || !q_abs) return -1;
  if (!valid_dtype(q_dtype) || !valid_dtype(w_dtype)) return -3;
  const int32_t w = d_latent + d_rope;
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
    const int64_t h = bh % H;
    double* out = q_abs + bh * w;
    for (int32_t j = 0; j < d_latent; ++j) out[j] = 0.0;
    for (int32_t n = 0; n < d_nope; ++n) {
      const double q = load_elem(q_nope, q_dtype, bh * d_nope + n);
      for (int32_t j = 0; j < d_latent; ++j)
        out[j] += q * load_elem(w_uk, w_dtype, (h * d_nope + n) * d_latent + j);
    }
    for (int32_t j = 0; j < d_rope; ++j)
      out[d_latent + j] = load_elem(q_rope, q_dtype, bh * d_rope + j);
  }
  return 0;
}

/* Merging softmax results computed over disjoint token sets: each part p
 * holds u_p = sum_{t in p} e^{s_t} x_t / Z_p with lse_p = log Z_p; the whole
 * is Z = sum_p Z_p and u = sum_p (Z_p / Z) u_p.  Parts with lse_p = -inf
 * attended nothing and carry no weight. */
int oracle_combine(int32_t B, int32_t S, int32_t H, int32_t D,
                   const double* u_part, const double* lse_part, double* u,
                   double* lse) {
  if (B < 0 || S <= 0 || H <= 0 || D <= 0 || !u_part || !lse_part || !u) return -1;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h) {
      double m = -INFINITY;
      for (int64_t p = 0; p < S; ++p) {
        double x = lse_part[(b * S + p) * H + h];
        if (x > m) m = x;
      }
      double* out = u + (b * H + h) * D;
      for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
      if (m == -INFINITY) {
        if (lse) lse[b * H + h] = -INFINITY;
        continue;
      }
      double z = 0.0;
      for (int64_t p = 0; p < S; ++p) z += exp(lse_part[(b * S + p) * H + h] - m);
      const double L = m + log(z);
      for (int64_t p = 0; p < S; ++p) {
        const double wgt = exp(lse_part[(b * S + p) * H + h] - L);
        if (wgt == 0.0) continue;
        const double* up = u_part + ((b * S + p) * H + h) * D;
        for (int32_t d = 0; d < D; ++d) out[d] += wgt * up[d];
      }
      if (lse) lse[b * H + h] = L;
    }
  return 0;
}

/* Applying W_UV after the weighted sum ([V2] §2.3): the attention output of
 * head h is W_UV[h] · (sum_t p_t c_t). */
int oracle_up_proj(int32_t B, int32_t H, int32_t d_v, int32_t d_latent,
                   const double* u, const void* w_uv, int32_t w_dtype, double* o) {
  if (B < 0 || H <= 0 || d_v <= 0 || d_latent <= 0 || !u || !o) return -1;
  if (!valid_dtype(w_dtype)) return -3;
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
    const int64_t h = bh % H;
    for (int32_t v = 0; v < d_v; ++v) {
      double acc = 0.0;
      for (int32_t c = 0; c < d_latent; ++c)
        acc += load_elem(w_uv, w_dtype, (h * d_v + v) * d_latent + c) * u[bh * d_latent + c];
      o[bh * d_v + v] = acc;
    }
  }
  return 0;
}

/* ------------------------------------------------------ cache append */

/* OCP E4M3: value = 2^(e-7) * (1 + m/8) for exponent field e in 1..15 (field
 * 15 with mantissa 7 is NaN, so the largest value is 448), and m * 2^-9 for
 * e = 0.  The representable values are spaced 2^(k-3) in the binade
 * [2^k, 2^(k+1)) for k >= -6 and 2^-9 below 2^-6, so the nearest one is
 * found by scaling |y| to units of that spacing (exact: a power of two) and
 * rounding to the nearest integer, ties to even (rint in the default
 * rounding mode).  A binade's count of 16 spacings is the next binade's
 * first value. */
uint8_t oracle_encode_e4m3(float y) {
  const uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs((double)y);
  if (a > 448.0) a = 448.0;
  if (a < ldexp(1.0, -6)) {                 /* subnormal spacing 2^-9 */
    const double q = rint(ldexp(a, 9));     /* 0 .. 8; 8 is the code of 2^-6 */
    return (uint8_t)(sign | (uint8_t)q);
  }
  int k;
  (void)frexp(a, &k);                       /* a = f * 2^k, f in [0.5, 1) */
  k -= 1;                                   /* a in [2^k, 2^(k+1)) */
  double q = rint(ldexp(a, 3 - k));         /* 8 .. 16 spacings of 2^(k-3) */
  if (q == 16.0) {
    q = 8.0;
    k += 1;
  }
  return (uint8_t)(sign | (uint8_t)(((k + 7) << 3) | ((int)q - 8)));
}

/* One row of w binary32 values in E4M3 with one fp32 factor ([DSA]'s FP8
 * cache; the factor maps the row's largest magnitude onto E4M3's largest
 * finite value 448): s = fl32(max(amax, 2^-126) / 448), each code the E4M3
 * value nearest to fl32(x / s) after clamping to +-448. */
static void quantize_row_e4m3(const float* x, int32_t w, uint8_t* codes, float* scale) {
  float amax = 0.0f;
  for (int32_t j = 0; j < w; ++j) amax = fmaxf(amax, fabsf(x[j]));
  const float s = fmaxf(amax, 0x1p-126f) / 448.0f;
  *scale = s;
  for (int32_t j = 0; j < w; ++j) {
    float y = x[j] / s;
    if (y > 448.0f) y = 448.0f;
    if (y < -448.0f) y = -448.0f;
    codes[j] = oracle_encode_e4m3(y);
  }
}

static void round_bf16(float x, uint16_t* out) {
  /* nearest bf16 (the binary32 values whose low 16 bits are zero), ties to
   * the even one: compare with the two neighbours in double */
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  const uint32_t lo = u & 0xFFFF0000u, hi = lo + 0x10000u;
  float flo, fhi;
  memcpy(&flo, &lo, sizeof flo);
  memcpy(&fhi, &hi, sizeof fhi);
  const double dlo = fabs((double)x - (double)flo), dhi = fabs((double)fhi - (double)x);
  uint32_t r = lo;
  if (dhi < dlo || (dhi == dlo && ((lo >> 16) & 1u))) r = hi;
  *out = (uint16_t)(r >> 16);
}

int oracle_cache_append(int32_t B, int32_t d_latent, int32_t d_rope, const void* c_kv,
                        const void* k_r, int32_t src_dtype, const int32_t* positions,
                        void* rows, int32_t cache_dtype, float* row_scale, int32_t page_size,
                        int64_t seq_stride, const int32_t* block_table, int32_t max_pages,
                        int32_t ring) {
  if (B < 0 || d_latent <= 0 || d_rope < 0 || !positions || !rows) return -1;
  if (B > 0 && (!c_kv || (d_rope > 0 && !k_r))) return -1;
  if (src_dtype != ORACLE_F32 && src_dtype != ORACLE_BF16) return -3;
  if (cache_dtype != ORACLE_F32 && cache_dtype != ORACLE_BF16 && cache_dtype != ORACLE_E4M3)
    return -3;
  if (cache_dtype == ORACLE_E4M3 && !row_scale) return -4;
  if (page_size < 0 || (page_size > 0 && (!block_table || max_pages < 1))) return -2;
  if (page_size == 0 && seq_stride < 1) return -2;
  if (ring && page_size != 0) return -2;
  const int32_t w = d_latent + d_rope;
  const int64_t capacity = page_size ? (int64_t)max_pages * page_size : seq_stride;
  float* x = (float*)malloc(sizeof(float) * (size_t)w);
  if (!x) return -5;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t t = positions[b];
    if (t < 0 || (!ring && t >= capacity)) continue;
    const int64_t page = page_size ? block_table[(int64_t)b * max_pages + t / page_size] : 0;
    if (page < 0) continue; /* no page mapped */
    /* a ring overwrites the token C positions back */
    const int64_t slot = ring ? t % seq_stride : t;
    const int64_t row = page_size ? page * page_size + t % page_size : (int64_t)b * seq_stride + slot;
    /* the new row as binary32 values (both input formats convert exactly) */
    for (int32_t j = 0; j < d_latent; ++j)
      x[j] = (float)load_elem(c_kv, src_dtype, (int64_t)b * d_latent + j);
    for (int32_t j = 0; j < d_rope; ++j)
      x[d_latent + j] = (float)load_elem(k_r, src_dtype, (int64_t)b * d_rope + j);
    if (cache_dtype == ORACLE_F32) {
      memcpy((float*)rows + row * w, x, sizeof(float) * (size_t)w);
    } else if (cache_dtype == ORACLE_BF16) {
      for (int32_t j = 0; j < w; ++j) round_bf16(x[j], (uint16_t*)rows + row * w + j);
    } else {
      quantize_row_e4m3(x, w, (uint8_t*)rows + row * w, row_scale + row);
    }
  }
  free(x);
  return 0;
}

int oracle_quantize_e4m3_rows(int64_t n, int32_t w, const float* x, uint8_t* codes,
                              float* scale) {
  if (n < 0 || w <= 0 || (n > 0 && (!x || !codes || !scale))) return -1;
  for (int64_t r = 0; r < n; ++r) quantize_row_e4m3(x + r * w, w, codes + r * w, scale + r);
  return 0;
}

/* Growing a ring ([V2] §4.1): the tokens a sequence's ring of src_cap rows
 * holds, the last min(L, src_cap), move to a ring of dst_cap rows, token t to
 * row t mod dst_cap; a smaller ring keeps the last dst_cap of them.  Rows are
 * moved as bytes (any cache dtype), with their fp32 factor when given. */
int oracle_ring_grow(int32_t B, int32_t row_bytes, const int32_t* seq_lens, const void* src,
                     const float* src_scale, int64_t src_cap, void* dst, float* dst_scale,
                     int64_t dst_cap) {
  if (B < 0 || row_bytes < 1 || src_cap < 1 || dst_cap < 1) return -1;
  if (B > 0 && (!seq_lens || !src || !dst)) return -1;
  if ((src_scale == NULL) != (dst_scale == NULL)) return -1;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t L = seq_lens[b];
    if (L < 0) return -2;
    int64_t keep = L < src_cap ? L : src_cap;
    if (keep > dst_cap) keep = dst_cap;
    for (int64_t t = L - keep; t < L; ++t) {
      const int64_t rs = (int64_t)b * src_cap + t % src_cap;
      const int64_t rd = (int64_t)b * dst_cap + t % dst_cap;
      memcpy((uint8_t*)dst + rd * row_bytes, (const uint8_t*)src + rs * row_bytes,
             (size_t)row_bytes);
      if (dst_scale) dst_scale[rd] = src_scale[rs];
    }
  }
  return 0;
}

/* ------------------------------------------------------ MHA baseline */

/* Grouped-query attention decode ([LAT] §2.2: query heads in groups, each
 * group sharing one key/value head; [V2] §1.2 lists MQA/GQA as the cache
 * reductions MLA is compared with).  The H query heads form H_kv contiguous
 * groups of G = H / H_kv: query head h reads key/value head h / G.  H_kv = H
 * is multi-head attention, H_kv = 1 multi-query attention. */
int oracle_gqa_decode(int32_t B, int32_t H, int32_t H_kv, int32_t d_qk, int32_t d_v,
                      const void* q, const void* k, const void* v, int32_t dtype,
                      const int32_t* seq_lens, int64_t seq_stride, double scale, double* o,
                      double* lse) {
  if (B < 0 || H <= 0 || H_kv <= 0 || d_qk <= 0 || d_v <= 0 || !q || !k || !v || !seq_lens ||
      !o || !lse)
    return -1;
  if (H % H_kv != 0) return -2;
  if (!valid_dtype(dtype)) return -3;
  if (seq_stride < 0) return -2;
  const int64_t G = H / H_kv;
  const double sc = scale > 0.0 ? scale : 1.0 / sqrt((double)d_qk);
  int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
    const int64_t b = bh / H, h = bh % H;
    const int64_t kvh = h / G;                  /* the group's key/value head */
    const int64_t kv = b * H_kv + kvh;          /* its rows: [b][kvh][seq_stride] */
    const int64_t L = seq_lens[b];
    double* out = o + bh * d_v;
    for (int32_t j = 0; j < d_v; ++j) out[j] = 0.0;
    if (L < 0 || L > seq_stride) {
      bad = 1;
      continue;
    }
    if (L == 0) {
      lse[bh] = -INFINITY;
      continue;
    }
    double* s = (double*)malloc(sizeof(double) * (size_t)L);
    if (!s) {
      bad = 1;
      continue;
    }
    /* scores */
    double m = -INFINITY;
    for (int64_t t = 0; t < L; ++t) {
      double dot = 0.0;
      for (int32_t j = 0; j < d_qk; ++j)
        dot += load_elem(q, dtype, bh * d_qk + j) * load_elem(k, dtype, (kv * seq_stride + t) * d_qk + j);
      s[t] = sc * dot;
      if (s[t] > m) m = s[t];
    }
    /* softmax weights and the weighted sum of the values */
    double l = 0.0;
    for (int64_t t = 0; t < L; ++t) {
      const double p = exp(s[t] - m);
      l += p;
      for (int32_t j = 0; j < d_v; ++j) out[j] += p * load_elem(v, dtype, (kv * seq_stride + t) * d_v + j);
    }
    for (int32_t j = 0; j < d_v; ++j) out[j] /= l;
    lse[bh] = m + log(l);
    free(s);
  }
  return bad ? -2 : 0;
}

/* Multi-head attention decode: every query head has its own key/value head. */
int oracle_mha_decode(int32_t B, int32_t H, int32_t d_qk, int32_t d_v, const void* q,
                      const void* k, const void* v, int32_t dtype, const int32_t* seq_lens,
                      int64_t seq_stride, double scale, double* o, double* lse) {
  return oracle_gqa_decode(B, H, H, d_qk, d_v, q, k, v, dtype, seq_lens, seq_stride, scale, o, lse);
}

/* ------------------------------------------------------ decoupled RoPE */

void oracle_rope_inv_freq(int32_t d_r, double base, float* inv_freq) {
  for (int32_t i = 0; i < d_r / 2; ++i)
    inv_freq[i] = (float)pow(base, -(2.0 * (double)i) / (double)d_r);
}

int oracle_rope(int32_t B, int32_t H, int32_t d_r, const void* x, int32_t dtype,
                const int32_t* positions, double base, double* out) {
  if (B < 0 || H <= 0 || d_r <= 0 || (d_r & 1) || !x || !positions || !out) return -1;
  if (!valid_dtype(dtype)) return -3;
  if (!(base > 1.0)) return -2;
  const int32_t half = d_r / 2;
  float* inv_freq = (float*)malloc(sizeof(float) * (size_t)half);
  if (!inv_freq) return -5;
  oracle_rope_inv_freq(d_r, base, inv_freq);
  for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
    const float pos = (float)positions[bh / H];
    for (int32_t i = 0; i < half; ++i) {
      const float theta = pos * inv_freq[i]; /* binary32 product */
      const double c = cos((double)theta), s = sin((double)theta);
      const double a = load_elem(x, dtype, bh * d_r + i);
      const double b = load_elem(x, dtype, bh * d_r + i + half);
      out[bh * d_r + i] = a * c - b * s;
      out[bh * d_r + i + half] = b * c + a * s;
    }
  }
  free(inv_freq);
  return 0;
}

/* ------------------------------------------------------ size arithmetic */

/* [V2] §2.3: per token and layer only KV_comp (d_latent) and k_R (d_rope)
 * are cached; an e4m3 row adds its scale factor. */
int64_t oracle_mla_cache_bytes_per_token(int32_t d_latent, int32_t d_rope,
                                         int32_t elem_bytes, int32_t scale_bytes) {
  return (int64_t)(d_latent + d_rope) * elem_bytes + scale_bytes;
}

/* [V2] §1.1: MHA caches K and V of every head: 2 x layers x seq x h x d
 * elements. */
int64_t oracle_mha_cache_bytes(int64_t layers, int64_t seq_len, int64_t heads,
                               int64_t head_dim, int64_t elem_bytes) {
  return 2 * layers * seq_len * heads * head_dim * elem_bytes;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
