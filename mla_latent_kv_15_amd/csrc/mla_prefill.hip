// Chunked prefill in the naive (rebuild) form, for gfx950 (CDNA4).
//
// "Multi-Head Latent Attention（MLA）：大模型KV Cache显存优化原理与实操" page, §4.2
// (the varlen flash-attention call with causal=True) and §4.3 (prefill of long
// passages); "KV Cache 革命…" page, "2. 分块并行计算" (the prompt processed in
// chunks).  A chunk of n_b new tokens of sequence b sits at the end of its
// cache, at positions L_b - n_b .. L_b - 1; query token j attends the cached
// tokens 0 .. L_b - n_b + j.  In the naive form of MLA ("DeepSeek V2的MLA注意力
// 机制…" page, §2.1) every head's keys and values are rebuilt from the latent:
//   K[b][h][t] = [W_UK[h] c_t ; k_R,t]   (192 wide),   V[b][h][t] = W_UV[h] c_t
// and attention runs over them with the un-absorbed query [q_C ; q_R] -- a
// compute-bound matrix-core workload, unlike the decode.
//
//   rebuild_kv_kernel  : K and V^T of one head for 128 cached tokens per workgroup
//   prefill_attn_kernel: causal attention of 128 query tokens of one head
//
// Matrix-core layout of v_mfma_f32_32x32x16_bf16 used throughout: lane l holds
// A[m = l % 32][k = 8 (l / 32) + i] and B[k = 8 (l / 32) + i][n = l % 32],
// i = 0..7; the accumulator D[m][n] sits in lane n + 32 g, register r with
// m = 8 (r / 4) + 4 g + r % 4.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/mla.h"
#include "mla_device.h"
#include "mla_host.h"

namespace mla {
namespace {

constexpr int kPfThreads = 256;
constexpr int kPfNope = 128;                 // d_nope of the prefill kernels
constexpr int kPfDv = 128;                   // d_v
constexpr int kPfQk = kPfNope + kDRope;      // 192: query / key width
constexpr int kPfQkBytes = kPfQk * 2;        // 384
constexpr int kRebuildTokens = 128;          // cached tokens per rebuild workgroup
constexpr int kPfQueries = 128;              // query tokens per attention workgroup
constexpr int kPfKeys = 32;                  // keys per block of the attention loop

__device__ inline int64_t cache_row(const int32_t* block_table, int32_t max_pages,
                                    int64_t seq_stride, bool paged, int b, int t) {
  if (paged) {
    const int64_t page = block_table[static_cast<int64_t>(b) * max_pages + (t >> 6)];
    return page * kPageSize + (t & 63);
  }
  return static_cast<int64_t>(b) * seq_stride + t;
}

__device__ inline bf16x8_t load_bf16x8(const void* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

// ---------------------------------------------------------------- rebuild
//
// Workgroup (token tile, head h, sequence b), 4 waves; wave w takes the 64
// tokens 64 (w & 1) .. +63 of the tile and computes either the content keys
// (w < 2) or the values (w >= 2) of head h for them, two 32-token blocks x
// four 32-wide output blocks = 8 accumulators, over the 512 latent columns in
// 32 steps of 16.  Operands come straight from memory in matrix-core layout:
// a cached row gives 16 contiguous bytes per lane (8 latent columns of one
// token), a weight row likewise (8 columns of one output row), so no LDS is
// needed; W_UK[h] / W_UV[h] (128 KB each) are shared by the tile's waves and
// by all tiles of the head through the caches.
//   keys   D[token][n]  = sum_c c[token][c] W_UK[h][n][c]   (A = rows, B = weights)
//   values D[dv][token] = sum_c W_UV[h][dv][c] c[token][c]  (A = weights, B = rows)
// so both accumulators store 32 consecutive elements per register: key rows
// [t][192] (the 64 RoPE elements copied from the cached row) and value columns
// of V^T [dv][kv_stride].
struct RebuildParams {
  const uint16_t* rows;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* rebuild_from;
  int64_t seq_stride;
  int32_t max_pages;
  int32_t paged;
  int32_t max_seq_len;
  int32_t H;
  const uint16_t* w_uk;
  const uint16_t* w_uv;
  uint16_t* k;
  uint16_t* vt;
  int64_t kv_stride;
};

__global__ __attribute__((amdgpu_flat_work_group_size(kPfThreads, kPfThreads), amdgpu_waves_per_eu(2, 2)))
void rebuild_kv_kernel(RebuildParams P) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int L = min(max(P.seq_lens[b], 0), P.max_seq_len);
  const int from = P.rebuild_from ? max(P.rebuild_from[b], 0) : 0;
  const int tile0 = blockIdx.x * kRebuildTokens;
  if (tile0 >= L || tile0 + kRebuildTokens <= from) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const bool values = wave >= 2;  // wave-uniform
  const int t_w = tile0 + 64 * (wave & 1);
  const bool paged = P.paged != 0;
  // the two 32-token blocks of this wave: lane's token row (tokens past the
  // end read the last token's row: finite data, never stored)
  const uint16_t* crow[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = min(t_w + 32 * tb + l32, L - 1);
    crow[tb] = P.rows + cache_row(P.block_table, P.max_pages, P.seq_stride, paged, b, t) * kRowElems +
               8 * g;
  }
  const uint16_t* W = (values ? P.w_uv : P.w_uk) + static_cast<int64_t>(h) * kPfNope * kDLatent + 8 * g;
  f32x16_t acc[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ob = 0; ob < 4; ++ob)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tb][ob][r] = 0.0f;

  // two steps in flight: set 0 for even steps, set 1 for odd ones
  bf16x8_t cf[2][2], wf[2][4];
  auto load = [&](int ks, auto slot) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) cf[slot][tb] = load_bf16x8(crow[tb] + 16 * ks);
#pragma unroll
    for (int ob = 0; ob < 4; ++ob)
      wf[slot][ob] = load_bf16x8(W + static_cast<int64_t>(32 * ob + l32) * kDLatent + 16 * ks);
  };
  auto run = [&](auto is_values) {
    auto step = [&](auto slot) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) {
          if constexpr (decltype(is_values)::value)
            acc[tb][ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[slot][ob], cf[slot][tb], acc[tb][ob], 0, 0, 0);
          else
            acc[tb][ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cf[slot][tb], wf[slot][ob], acc[tb][ob], 0, 0, 0);
        }
    };
    constexpr std::integral_constant<int, 0> s0{};
    constexpr std::integral_constant<int, 1> s1{};
    load(0, s0);
    for (int ks = 0; ks < kDLatent / 16; ks += 2) {
      load(ks + 1, s1);
      step(s0);
      if (ks + 2 < kDLatent / 16) load(ks + 2, s0);
      step(s1);
    }
  };
  if (values)
    run(std::true_type{});
  else
    run(std::false_type{});
  const int64_t bh = static_cast<int64_t>(b) * P.H + h;
  if (!values) {
    // keys: register r of block (tb, ob) is token t_w + 32 tb + 8 (r/4) + 4 g + r%4,
    // column n = 32 ob + l32
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t_w + 32 * tb + 8 * (r >> 2) + 4 * g + (r & 3);
        if (t < from || t >= L) continue;
        uint16_t* krow = P.k + (bh * P.kv_stride + t) * kPfQk;
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) krow[32 * ob + l32] = f32_to_bf16(acc[tb][ob][r]);
      }
    // the RoPE part of each key is the token's own k_R: 64 tokens x 8 chunks
    // of 16 bytes, 8 per lane
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = i * 64 + lane, tl = q >> 3, ch = q & 7;
      const int t = t_w + tl;
      if (t < from || t >= L) continue;
      const uint16_t* src =
          P.rows + cache_row(P.block_table, P.max_pages, P.seq_stride, paged, b, t) * kRowElems +
          kDLatent + 8 * ch;
      *reinterpret_cast<u32x4_t*>(P.k + (bh * P.kv_stride + t) * kPfQk + kPfNope + 8 * ch) =
          *reinterpret_cast<const u32x4_t*>(src);
    }
  } else {
    // values: register r of block (tb, ob) is value row dv = 32 ob + 8 (r/4) +
    // 4 g + r%4 of token t_w + 32 tb + l32
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int t = t_w + 32 * tb + l32;
      if (t < from || t >= L) continue;
#pragma unroll
      for (int ob = 0; ob < 4; ++ob)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dv = 32 * ob + 8 * (r >> 2) + 4 * g + (r & 3);
          P.vt[(bh * kPfDv + dv) * P.kv_stride + t] = f32_to_bf16(acc[tb][ob][r]);
        }
    }
  }
}

// ---------------------------------------------------------------- attention
//
// Workgroup (query tile of 128, head h, sequence b), 4 waves of 32 query
// tokens; the key blocks of 32 are staged once per workgroup in LDS (keys
// [32][192] and values V^T [128][32], double-buffered) and shared by the four
// waves.  Per key block a wave computes the transposed scores
//   S^T[key][query] = sum_d K[key][d] Q[query][d]      (12 steps of 16)
// with its 32 queries held in registers as the B operand, so that each lane
// owns one query (lane l and l + 32 hold the same query, other keys): the
// causal mask, the running maximum and the sum are lane-local (one exchange
// with lane l ^ 32).  The probabilities are already the B operand of
//   O^T[dv][query] += sum_key V^T[dv][key] P^T[key][query]   (4 x 2 steps)
// once the key order inside each 16-key step is taken as the accumulator's:
// lanes 0-31 hold keys 0-3 and 8-11, lanes 32-63 keys 4-7 and 12-15; the
// values are read from LDS in that same order (two 8-byte reads per step).
// Scores use base 2 with log2(e) folded into the scale; the rescale of the
// running output by 2^(m_old - m_new) is a per-lane scalar.  Keys past the
// sequence are masked by selection (their staged values are zeroed, so stale
// memory contributes exactly 0 x 0).
constexpr int kKRow = kPfQkBytes + 16;          // LDS key row stride (bytes), padded
constexpr int kVRow = kPfKeys * 2 + 16;         // LDS value row stride: 32 keys + pad
constexpr int kKBuf = kPfKeys * kKRow;          // 12800
constexpr int kVBuf = kPfDv * kVRow;            // 10240

struct AttnParams {
  const uint16_t* q;        // [B][QL][H][192]
  const int32_t* q_lens;    // [B]
  const uint16_t* k;        // [B][H][kv_stride][192]
  const uint16_t* vt;       // [B][H][128][kv_stride]
  const int32_t* seq_lens;  // [B]
  int64_t kv_stride;
  int32_t QL, H, max_seq_len;
  float scale_log2;
  void* o;                  // [B][QL][H][128]
  float* lse;               // [B][QL][H] or null
};

template <int O_DT>
__global__ __attribute__((amdgpu_flat_work_group_size(kPfThreads, kPfThreads), amdgpu_waves_per_eu(2, 2)))
void prefill_attn_kernel(AttnParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (kKBuf + kVBuf)];
  const int b = blockIdx.z, h = blockIdx.y;
  const int qt = gridDim.x - 1 - blockIdx.x;  // the longest query tiles first
  const int nq = min(max(P.q_lens[b], 0), P.QL);
  const int L = min(max(P.seq_lens[b], 0), P.max_seq_len);
  const int j0 = qt * kPfQueries;
  if (j0 >= nq) return;
  const int base = L - nq;  // position of query token 0 of the chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int j = j0 + 32 * wave + l32;  // this lane's query token
  const bool qvalid = j < nq;
  const int pos = base + j;            // attends keys t <= pos (and t < L)
  const int j_last = min(j0 + kPfQueries - 1, nq - 1);
  const int kend = max(min(L, base + j_last + 1), 0);  // keys of the tile: [0, kend)
  const int nblk = (kend + kPfKeys - 1) / kPfKeys;
  const int64_t bh = static_cast<int64_t>(b) * P.H + h;

  // queries: B operand, query l32 of the wave, 8 elements per step
  bf16x8_t qf[kPfQk / 16];
  {
    const uint16_t* qrow = P.q + ((static_cast<int64_t>(b) * P.QL + (qvalid ? j : 0)) * P.H + h) * kPfQk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kPfQk / 16; ++ks) qf[ks] = qvalid ? load_bf16x8(qrow + 16 * ks) : bf16x8_t{};
  }
  f32x16_t acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  // staging of key block kb: 768 key chunks and 512 value chunks of 16 bytes
  u32x4_t kst[3], vst[2];
  const uint16_t* kbase = P.k + bh * P.kv_stride * kPfQk;
  const uint16_t* vbase = P.vt + bh * kPfDv * P.kv_stride;
  auto stage_load = [&](int kb) {
    const int t0 = kb * kPfKeys;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int c = i * kPfThreads + tid, row = c / 24, col = c % 24;
      kst[i] = *reinterpret_cast<const u32x4_t*>(kbase + static_cast<int64_t>(t0 + row) * kPfQk + 8 * col);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = i * kPfThreads + tid, dv = c >> 2, ch = c & 3;
      const int tk = t0 + 8 * ch;
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(vbase + static_cast<int64_t>(dv) * P.kv_stride + tk);
      if (tk + 8 > L) {  // keys past the sequence: exact zeros
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (tk + 2 * e < L) ? 0x0000FFFFu : 0u;
          const uint32_t hi = (tk + 2 * e + 1 < L) ? 0xFFFF0000u : 0u;
          v[e] &= (lo | hi);
        }
      }
      vst[i] = v;
    }
  };
  auto stage_store = [&](int buf) {
    uint8_t* K = smem + buf * (kKBuf + kVBuf);
    uint8_t* V = K + kKBuf;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int c = i * kPfThreads + tid, row = c / 24, col = c % 24;
      *reinterpret_cast<u32x4_t*>(K + row * kKRow + 16 * col) = kst[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = i * kPfThreads + tid, dv = c >> 2, ch = c & 3;
      *reinterpret_cast<u32x4_t*>(V + dv * kVRow + 16 * ch) = vst[i];
    }
  };

  if (nblk > 0) stage_load(0);
  for (int kb = 0; kb < nblk; ++kb) {
    const int buf = kb & 1;
    stage_store(buf);
    __syncthreads();  // block kb staged; block kb - 2 in this buffer fully read
    if (kb + 1 < nblk) stage_load(kb + 1);
    const uint8_t* K = smem + buf * (kKBuf + kVBuf);
    const uint8_t* V = K + kKBuf;
    const int t0 = kb * kPfKeys;
    // S^T: key l32 of the block (A), query l32 of the wave (B)
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
    const uint8_t* krow = K + l32 * kKRow + 16 * g;
#pragma unroll
    for (int ks = 0; ks < kPfQk / 16; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_bf16x8(krow + 32 * ks), qf[ks], s, 0, 0, 0);
    // register r: key t0 + 8 (r/4) + 4 g + r%4 of this lane's query
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + 8 * (r >> 2) + 4 * g + (r & 3);
      s[r] = (t <= pos && t < L) ? s[r] * P.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;  // nothing attended yet
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    // the accumulators are rescaled only when some query's maximum moved: an
    // unchanged maximum gives alpha = 1 (and a query with nothing attended yet
    // has nothing accumulated), so skipping is exact
    if (__any(m_new != m)) {
      l *= alpha;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
    }
    m = m_new;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
      l += p[r];
    }
    bf16x8_t pk[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[8 * kk + 2 * e], p[8 * kk + 2 * e + 1]);
      __builtin_memcpy(&pk[kk], w, 16);
    }
    // O^T: value rows 32 cb + l32 (A, keys in the accumulator's order), P^T (B)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const uint8_t* vrow = V + (32 * cb + l32) * kVRow + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow + 32 * kk);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 32 * kk + 16);
        const u32x4_t a4 = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        bf16x8_t a;
        __builtin_memcpy(&a, &a4, 16);
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kk], acc[cb], 0, 0, 0);
      }
    }
  }
  // the query's total weight: this lane's keys and lane l ^ 32's
  const float l_tot = l + __shfl_xor(l, 32);
  if (!qvalid) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int64_t orow = ((static_cast<int64_t>(b) * P.QL + j) * P.H + h) * kPfDv;
  // register r of block cb: value element 32 cb + 8 (r/4) + 4 g + r%4
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dv = 32 * cb + 8 * r4 + 4 * g;
      const float v0 = acc[cb][4 * r4] * inv, v1 = acc[cb][4 * r4 + 1] * inv;
      const float v2 = acc[cb][4 * r4 + 2] * inv, v3 = acc[cb][4 * r4 + 3] * inv;
      if constexpr (O_DT == MLA_F32)
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(P.o) + orow + dv) = f32x4_t{v0, v1, v2, v3};
      else
        *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(P.o) + orow + dv) =
            u32x2_t{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
    }
  if (P.lse && g == 0)
    P.lse[(static_cast<int64_t>(b) * P.QL + j) * P.H + h] =
        l_tot > 0.0f ? (m + log2f(l_tot)) * kLn2 : -INFINITY;
}

mla_status_t launch_status() { return hipGetLastError() == hipSuccess ? MLA_OK : MLA_E_HIP; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" mla_status_t mla_prefill_rebuild_kv(const mla_dims_t* dims, int32_t B,
                                               const mla_cache_t* cache,
                                               const int32_t* rebuild_from, const void* w_uk,
                                               const void* w_uv, int32_t w_dt, void* k, void* vt,
                                               int64_t kv_stride, void* stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!cache || B < 0 || cache->max_seq_len < 0) return MLA_E_ARG;
  if (dims->d_nope != kPfNope || dims->d_v != kPfDv) return MLA_E_SHAPE;
  if (cache->page_size != 0 && cache->page_size != kPageSize) return MLA_E_SHAPE;
  if (kv_stride < cache->max_seq_len || kv_stride % 32 != 0) return MLA_E_ARG;
  if (B == 0 || cache->max_seq_len == 0) return MLA_OK;
  if (!cache->rows || !cache->seq_lens || !w_uk || !w_uv || !k || !vt) return MLA_E_ARG;
  if (cache->dtype != MLA_BF16 || w_dt != MLA_BF16) return MLA_E_DTYPE;
  if (cache->ring) return MLA_E_UNSUPPORTED;
  if (cache->page_size == 0 && cache->seq_stride < cache->max_seq_len) return MLA_E_ARG;
  if (cache->page_size != 0) {
    const int64_t need = (static_cast<int64_t>(cache->max_seq_len) + kPageSize - 1) / kPageSize;
    if (!cache->block_table || cache->max_pages < need) return MLA_E_ARG;
  }
  if (!aligned16(cache->rows) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(k) ||
      !aligned16(vt))
    return MLA_E_ALIGN;
  if (B > 65535 || dims->heads > 65535) return MLA_E_SHAPE;
  RebuildParams P{static_cast<const uint16_t*>(cache->rows), cache->block_table, cache->seq_lens,
                  rebuild_from, cache->seq_stride, cache->max_pages, cache->page_size != 0,
                  cache->max_seq_len, dims->heads, static_cast<const uint16_t*>(w_uk),
                  static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(k),
                  static_cast<uint16_t*>(vt), kv_stride};
  const dim3 grid((cache->max_seq_len + kRebuildTokens - 1) / kRebuildTokens, dims->heads, B);
  rebuild_kv_kernel<<<grid, kPfThreads, 0, static_cast<hipStream_t>(stream)>>>(P);
  return launch_status();
}

extern "C" mla_status_t mla_prefill_attn(const mla_dims_t* dims, int32_t B, int32_t q_len,
                                         const int32_t* q_lens, const void* q, int32_t q_dt,
                                         const void* k, const void* vt, int64_t kv_stride,
                                         const int32_t* seq_lens, int32_t max_seq_len, void* o,
                                         int32_t o_dt, float* lse, void* stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (B < 0 || q_len < 0 || max_seq_len < 0) return MLA_E_ARG;
  if (dims->d_nope != kPfNope || dims->d_v != kPfDv) return MLA_E_SHAPE;
  if (kv_stride < max_seq_len || kv_stride % 32 != 0) return MLA_E_ARG;
  if (B == 0 || q_len == 0) return MLA_OK;
  if (!q_lens || !q || !k || !vt || !seq_lens || !o) return MLA_E_ARG;
  if (q_dt != MLA_BF16 || (o_dt != MLA_BF16 && o_dt != MLA_F32)) return MLA_E_DTYPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o)) return MLA_E_ALIGN;
  const int64_t tiles = (static_cast<int64_t>(q_len) + kPfQueries - 1) / kPfQueries;
  if (B > 65535 || dims->heads > 65535 || tiles > 0x7FFFFFFF) return MLA_E_SHAPE;
  AttnParams P{static_cast<const uint16_t*>(q), q_lens, static_cast<const uint16_t*>(k),
               static_cast<const uint16_t*>(vt), seq_lens, kv_stride, q_len, dims->heads,
               max_seq_len, effective_scale(dims) * kLog2e, o, lse};
  const dim3 grid(static_cast<unsigned>(tiles), dims->heads, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (o_dt == MLA_F32)
    prefill_attn_kernel<MLA_F32><<<grid, kPfThreads, 0, s>>>(P);
  else
    prefill_attn_kernel<MLA_BF16><<<grid, kPfThreads, 0, s>>>(P);
  return launch_status();
}
