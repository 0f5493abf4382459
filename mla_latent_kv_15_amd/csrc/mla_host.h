// Host-side argument validation and launch geometry of the MLA decode library.
// Pure C++ (no HIP calls), so every error path can be exercised without a GPU.
#pragma once

#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

// Compiled geometry (DeepSeek V2 page §3.1: latent d_c = 512, RoPE width 64).
constexpr int32_t kDLatent = 512;
constexpr int32_t kDRope = 64;
constexpr int32_t kRowElems = kDLatent + kDRope;  // one cached row [c_KV | k_R]
constexpr int32_t kTileTokens = 32;               // split ranges are whole tiles
constexpr int32_t kPageSize = 64;
constexpr int32_t kMaxSplits = 1024;
constexpr int32_t kMaxDHead = 256;  // d_nope / d_v bound of absorb and up-projection
constexpr int32_t kHeadsPerWave = 32;
constexpr int32_t kMhaHeadDim = 128;  // head dimension of the MHA baseline kernel
constexpr int32_t kMaxQueryTokens = 16;  // query tokens per sequence in mla_decode_multi

inline int32_t dtype_bytes(int32_t dt) {
  return dt == MLA_F32 ? 4 : dt == MLA_BF16 ? 2 : dt == MLA_FP8_E4M3 ? 1 : 0;
}

// Tokens per split range: 32 * ceil(max_seq_len / (32 * num_splits)); 0 when
// max_seq_len == 0.
int32_t split_chunk(int32_t max_seq_len, int32_t num_splits);

// softmax scale actually used (dims->softmax_scale, or 1/sqrt(d_nope+d_rope)).
float effective_scale(const mla_dims_t* dims);

mla_status_t check_dims(const mla_dims_t* dims);

mla_status_t check_absorb(const mla_dims_t* dims, int32_t B, const void* q_nope,
                          const void* q_rope, int32_t q_dt, const void* w_uk,
                          int32_t w_dt, const void* q_abs, int32_t q_abs_dt,
                          const float* q_abs_scale);

mla_status_t check_decode(const mla_dims_t* dims, int32_t B, const void* q_abs,
                          int32_t q_abs_dt, const float* q_abs_scale,
                          const mla_cache_t* cache, int32_t num_splits,
                          const void* u_part, int32_t part_dt, const float* lse_part);

mla_status_t check_combine(const mla_dims_t* dims, int32_t B, int32_t num_splits,
                           const void* u_part, int32_t part_dt, const float* lse_part,
                           const void* u, int32_t u_dt);

mla_status_t check_up_proj(const mla_dims_t* dims, int32_t B, const void* u,
                           int32_t u_dt, const void* w_uv, int32_t w_dt, const void* o,
                           int32_t o_dt);

mla_status_t check_combine_up_proj(const mla_dims_t* dims, int32_t B, int32_t num_splits,
                                   const void* u_part, int32_t part_dt, const float* lse_part,
                                   const void* w_uv, int32_t w_dt, const void* o, int32_t o_dt,
                                   const void* u);

mla_status_t check_cache_append(const mla_dims_t* dims, int32_t B, const void* c_kv,
                                const void* k_r, int32_t src_dt, const int32_t* positions,
                                const mla_cache_t* cache);

mla_status_t check_ring_grow(int32_t B, const mla_cache_t* src, const mla_cache_t* dst);

mla_status_t check_mha_decode(int32_t B, int32_t heads, int32_t d_head, const void* q,
                              const void* k_cache, const void* v_cache, int32_t dt,
                              const int32_t* seq_lens, int64_t seq_stride, int32_t max_seq_len,
                              float softmax_scale, const void* o, int32_t o_dt);

}  // namespace mla
