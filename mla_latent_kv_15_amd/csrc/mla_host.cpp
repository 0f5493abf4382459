// Host-side argument validation of the MLA decode library (no HIP calls).
#include "mla_host.h"

#include <math.h>

namespace mla {

namespace {

bool valid_dtype(int32_t dt) {
  return dt == MLA_F32 || dt == MLA_BF16 || dt == MLA_FP8_E4M3;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

int32_t split_chunk(int32_t max_seq_len, int32_t num_splits) {
  if (max_seq_len <= 0 || num_splits <= 0) return 0;
  const int64_t per_tile = static_cast<int64_t>(kTileTokens) * num_splits;
  const int64_t tiles = (static_cast<int64_t>(max_seq_len) + per_tile - 1) / per_tile;
  return static_cast<int32_t>(tiles * kTileTokens);
}

float effective_scale(const mla_dims_t* dims) {
  if (dims->softmax_scale > 0.0f) return dims->softmax_scale;
  return static_cast<float>(1.0 / sqrt(static_cast<double>(dims->d_nope + dims->d_rope)));
}

mla_status_t check_dims(const mla_dims_t* dims) {
  if (!dims) return MLA_E_ARG;
  if (dims->heads < 1 || dims->d_nope < 1 || dims->d_v < 1 || dims->d_rope < 0 ||
      dims->d_latent < 1)
    return MLA_E_ARG;
  if (!(dims->softmax_scale == dims->softmax_scale)) return MLA_E_ARG;  // NaN
  if (dims->d_latent != kDLatent || dims->d_rope != kDRope) return MLA_E_SHAPE;
  if (dims->d_nope > kMaxDHead || dims->d_v > kMaxDHead) return MLA_E_SHAPE;
  return MLA_OK;
}

mla_status_t check_absorb(const mla_dims_t* dims, int32_t B, const void* q_nope,
                          const void* q_rope, int32_t q_dt, const void* w_uk,
                          int32_t w_dt, const void* q_abs, int32_t q_abs_dt,
                          const float* q_abs_scale) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (B < 0) return MLA_E_ARG;
  if (!valid_dtype(q_dt) || !valid_dtype(w_dt) || !valid_dtype(q_abs_dt)) return MLA_E_ARG;
  if (B == 0) return MLA_OK;
  if (!q_nope || !q_rope || !w_uk || !q_abs) return MLA_E_ARG;
  if (q_dt == MLA_FP8_E4M3 || w_dt == MLA_FP8_E4M3) return MLA_E_DTYPE;
  if (q_abs_dt == MLA_FP8_E4M3) {
    if (!q_abs_scale) return MLA_E_ARG;
  } else if (q_abs_scale) {
    return MLA_E_ARG;
  }
  if (!aligned(q_abs, 16)) return MLA_E_ALIGN;
  return MLA_OK;
}

mla_status_t check_decode(const mla_dims_t* dims, int32_t B, const void* q_abs,
                          int32_t q_abs_dt, const float* q_abs_scale,
                          const mla_cache_t* cache, int32_t num_splits,
                          const void* u_part, int32_t part_dt, const float* lse_part) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!cache) return MLA_E_ARG;
  if (B < 0 || num_splits < 1 || num_splits > kMaxSplits) return MLA_E_ARG;
  if (!valid_dtype(q_abs_dt) || !valid_dtype(part_dt) || !valid_dtype(cache->dtype))
    return MLA_E_ARG;
  if (cache->max_seq_len < 0) return MLA_E_ARG;
  if (cache->page_size != 0 && cache->page_size != kPageSize) return MLA_E_SHAPE;
  if (cache->ring != 0 && cache->ring != 1) return MLA_E_ARG;
  if (cache->ring && cache->page_size != 0) return MLA_E_ARG;
  if (B == 0) return MLA_OK;
  if (!q_abs || !u_part || !lse_part || !cache->rows || !cache->seq_lens) return MLA_E_ARG;
  if (part_dt == MLA_FP8_E4M3) return MLA_E_DTYPE;
  // provided (cache, q_abs) pairs
  const int32_t cd = cache->dtype;
  const bool pair_ok = (cd == MLA_F32 && q_abs_dt == MLA_F32) ||
                       (cd == MLA_BF16 && q_abs_dt == MLA_BF16) ||
                       (cd == MLA_FP8_E4M3 && (q_abs_dt == MLA_BF16 || q_abs_dt == MLA_FP8_E4M3));
  if (!pair_ok) return MLA_E_DTYPE;
  if (q_abs_dt == MLA_FP8_E4M3) {
    if (!q_abs_scale) return MLA_E_ARG;
  } else if (q_abs_scale) {
    return MLA_E_ARG;
  }
  if (cd == MLA_FP8_E4M3) {
    if (!cache->row_scale) return MLA_E_ARG;
  } else if (cache->row_scale) {
    return MLA_E_ARG;
  }
  if (cache->page_size == 0) {
    // a ring holds the last seq_stride tokens: lengths may exceed it
    if (cache->seq_stride < (cache->ring ? 1 : cache->max_seq_len)) return MLA_E_ARG;
  } else {
    if (!cache->block_table || cache->max_pages < 1) return MLA_E_ARG;
    const int64_t need = (static_cast<int64_t>(cache->max_seq_len) + kPageSize - 1) / kPageSize;
    if (cache->max_pages < need) return MLA_E_ARG;
  }
  if (cd != MLA_F32 && dims->heads % kHeadsPerWave != 0) return MLA_E_SHAPE;
  if (!aligned(cache->rows, 16) || !aligned(q_abs, 16) || !aligned(u_part, 16) ||
      !aligned(lse_part, 4))
    return MLA_E_ALIGN;
  return MLA_OK;
}

mla_status_t check_combine(const mla_dims_t* dims, int32_t B, int32_t num_splits,
                           const void* u_part, int32_t part_dt, const float* lse_part,
                           const void* u, int32_t u_dt) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (B < 0 || num_splits < 1 || num_splits > kMaxSplits) return MLA_E_ARG;
  if (!valid_dtype(part_dt) || !valid_dtype(u_dt)) return MLA_E_ARG;
  if (B == 0) return MLA_OK;
  if (!u_part || !lse_part || !u) return MLA_E_ARG;
  if (part_dt == MLA_FP8_E4M3 || u_dt == MLA_FP8_E4M3) return MLA_E_DTYPE;
  if (!aligned(u_part, 16) || !aligned(u, 16)) return MLA_E_ALIGN;
  return MLA_OK;
}

mla_status_t check_up_proj(const mla_dims_t* dims, int32_t B, const void* u,
                           int32_t u_dt, const void* w_uv, int32_t w_dt, const void* o,
                           int32_t o_dt) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (B < 0) return MLA_E_ARG;
  if (!valid_dtype(u_dt) || !valid_dtype(w_dt) || !valid_dtype(o_dt)) return MLA_E_ARG;
  if (B == 0) return MLA_OK;
  if (!u || !w_uv || !o) return MLA_E_ARG;
  if (u_dt == MLA_FP8_E4M3 || w_dt == MLA_FP8_E4M3 || o_dt == MLA_FP8_E4M3)
    return MLA_E_DTYPE;
  if (!aligned(u, 16) || !aligned(w_uv, 16)) return MLA_E_ALIGN;
  return MLA_OK;
}

mla_status_t check_combine_up_proj(const mla_dims_t* dims, int32_t B, int32_t num_splits,
                                   const void* u_part, int32_t part_dt, const float* lse_part,
                                   const void* w_uv, int32_t w_dt, const void* o, int32_t o_dt,
                                   const void* u) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (B < 0 || num_splits < 1 || num_splits > kMaxSplits) return MLA_E_ARG;
  if (!valid_dtype(part_dt) || !valid_dtype(w_dt) || !valid_dtype(o_dt)) return MLA_E_ARG;
  if (B == 0) return MLA_OK;
  if (!u_part || !lse_part || !w_uv || !o) return MLA_E_ARG;
  if (part_dt == MLA_FP8_E4M3 || o_dt == MLA_FP8_E4M3) return MLA_E_DTYPE;
  if (w_dt != MLA_BF16) return MLA_E_DTYPE;
  if (dims->d_v % 16 != 0) return MLA_E_SHAPE;
  if (!aligned(u_part, 16) || !aligned(w_uv, 16) || (u && !aligned(u, 16))) return MLA_E_ALIGN;
  return MLA_OK;
}

mla_status_t check_cache_append(const mla_dims_t* dims, int32_t B, const void* c_kv,
                                const void* k_r, int32_t src_dt, const int32_t* positions,
                                const mla_cache_t* cache) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!cache || B < 0) return MLA_E_ARG;
  if (!valid_dtype(src_dt) || !valid_dtype(cache->dtype)) return MLA_E_ARG;
  if (cache->page_size != 0 && cache->page_size != kPageSize) return MLA_E_SHAPE;
  if (cache->ring != 0 && cache->ring != 1) return MLA_E_ARG;
  if (cache->ring && cache->page_size != 0) return MLA_E_ARG;
  if (B == 0) return MLA_OK;
  if (!c_kv || !k_r || !positions || !cache->rows) return MLA_E_ARG;
  if (src_dt == MLA_FP8_E4M3) return MLA_E_DTYPE;
  if (cache->dtype == MLA_FP8_E4M3) {
    if (!cache->row_scale) return MLA_E_ARG;
  } else if (cache->row_scale) {
    return MLA_E_ARG;
  }
  if (cache->page_size == 0) {
    if (cache->seq_stride < 1) return MLA_E_ARG;
  } else {
    if (!cache->block_table || cache->max_pages < 1) return MLA_E_ARG;
  }
  if (!aligned(cache->rows, 16)) return MLA_E_ALIGN;
  return MLA_OK;
}

mla_status_t check_ring_grow(int32_t B, const mla_cache_t* src, const mla_cache_t* dst) {
  if (!src || !dst || B < 0) return MLA_E_ARG;
  if (src->ring != 1 || dst->ring != 1 || src->page_size != 0 || dst->page_size != 0)
    return MLA_E_ARG;
  if (src->seq_stride < 1 || dst->seq_stride < 1 || src->max_seq_len < 0) return MLA_E_ARG;
  if (!valid_dtype(src->dtype) || !valid_dtype(dst->dtype)) return MLA_E_ARG;
  if (src->dtype != dst->dtype) return MLA_E_DTYPE;
  if (B == 0) return MLA_OK;
  if (!src->rows || !dst->rows || !src->seq_lens) return MLA_E_ARG;
  const bool fp8 = src->dtype == MLA_FP8_E4M3;
  if (fp8 != (src->row_scale != nullptr) || fp8 != (dst->row_scale != nullptr)) return MLA_E_ARG;
  if (!aligned(src->rows, 16) || !aligned(dst->rows, 16)) return MLA_E_ALIGN;
  return MLA_OK;
}

mla_status_t check_mha_decode(int32_t B, int32_t heads, int32_t d_head, const void* q,
                              const void* k_cache, const void* v_cache, int32_t dt,
                              const int32_t* seq_lens, int64_t seq_stride, int32_t max_seq_len,
                              float softmax_scale, const void* o, int32_t o_dt) {
  if (B < 0 || heads < 1 || d_head < 1 || max_seq_len < 0) return MLA_E_ARG;
  if (!(softmax_scale == softmax_scale)) return MLA_E_ARG;  // NaN
  if (!valid_dtype(dt) || !valid_dtype(o_dt)) return MLA_E_ARG;
  if (d_head != kMhaHeadDim) return MLA_E_SHAPE;
  if (seq_stride < max_seq_len || seq_stride < 1) return MLA_E_ARG;
  if (B == 0) return MLA_OK;
  if (!q || !k_cache || !v_cache || !seq_lens || !o) return MLA_E_ARG;
  if (dt != MLA_BF16 || o_dt == MLA_FP8_E4M3) return MLA_E_DTYPE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16)) return MLA_E_ALIGN;
  return MLA_OK;
}

}  // namespace mla

extern "C" const char* mla_status_str(mla_status_t status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_E_ARG: return "invalid argument";
    case MLA_E_DTYPE: return "dtype combination not provided";
    case MLA_E_SHAPE: return "dimension outside the compiled geometry";
    case MLA_E_ALIGN: return "pointer or stride misaligned";
    case MLA_E_HIP: return "HIP runtime error at launch";
    case MLA_E_UNSUPPORTED: return "request not provided by this library";
    case MLA_E_SCRATCH: return "request larger than the library's static scratch";
  }
  return "unknown status";
}

extern "C" int32_t mla_version(void) { return 100; }
