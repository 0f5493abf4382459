// HIP kernels and C entry points of the MLA decode library, for gfx950 (CDNA4).
//
// The decode step follows the absorbed form of multi-head latent attention
// ("DeepSeek V2的MLA注意力机制…" page, §2.3 and §4.1): W_UK is folded into the
// query (mla_absorb_q), attention runs directly over the cached latent rows
// [c_KV | k_R] (mla_decode), split partials are merged with log-sum-exp
// weights (mla_combine), and W_UV is applied after the weighted sum
// (mla_up_proj).  Full per-head keys and values are never formed.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mla.h"
#include "mla_host.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------ element codecs

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// binary32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// OCP E4M3 code -> value.  Placing the 7 magnitude bits at binary32 bit 20
// gives exponent field e and mantissa m/8 (or, for e = 0, the binary32
// subnormal m*2^-129); multiplying by 2^120 rebases the exponent from bias 127
// to bias 7, which is exact for normal and subnormal codes alike.
__device__ inline float e4m3_to_f32(uint32_t code) {
  float f = __uint_as_float((code & 0x7Fu) << 20) * 0x1p120f;
  f = (code & 0x80u) ? -f : f;
  return ((code & 0x7Fu) == 0x7Fu) ? __uint_as_float(0x7FC00000u) : f;
}

// 4 codes (one 32-bit word) -> 4 bf16 (two 32-bit words).  E4M3 values have at
// most 4 significant bits, so the bf16 truncation of the binary32 is exact.
__device__ inline u32x2_t e4m3x4_to_bf16x4(uint32_t w) {
  u32x2_t r;
  const uint32_t b0 = __float_as_uint(e4m3_to_f32(w & 0xFFu)) >> 16;
  const uint32_t b1 = __float_as_uint(e4m3_to_f32((w >> 8) & 0xFFu)) >> 16;
  const uint32_t b2 = __float_as_uint(e4m3_to_f32((w >> 16) & 0xFFu)) >> 16;
  const uint32_t b3 = __float_as_uint(e4m3_to_f32(w >> 24)) >> 16;
  r.x = b0 | (b1 << 16);
  r.y = b2 | (b3 << 16);
  return r;
}

template <int DT>
__device__ inline float load_elem(const void* p, int64_t i) {
  if constexpr (DT == MLA_F32) return static_cast<const float*>(p)[i];
  else return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <int DT>
__device__ inline void store_elem(void* p, int64_t i, float v) {
  if constexpr (DT == MLA_F32) static_cast<float*>(p)[i] = v;
  else static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
}

// Workgroups are dispatched round-robin over the 8 XCDs (block x runs on XCD
// x % 8).  Give every XCD one contiguous range of logical work ids, so that the
// split ranges of one sequence, which all read the same absorbed query rows,
// share that XCD's L2.
__device__ inline int xcd_remap(int bid, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = bid & 7, k = bid >> 3;
  return x * per + (x < rem ? x : rem) + k;
}

// Physical row of the first token of a 32-token tile (tiles never straddle a
// 64-row page because every split range starts at a multiple of 32).
__device__ inline int64_t tile_row0(const int32_t* block_table, int32_t max_pages,
                                    int64_t seq_stride, bool paged, int b, int t) {
  if (paged) {
    const int64_t page = block_table[static_cast<int64_t>(b) * max_pages + (t >> 6)];
    return page * kPageSize + (t & 63);
  }
  return static_cast<int64_t>(b) * seq_stride + t;
}

// ================================================================ decode (MFMA)
//
// One workgroup = one (sequence b, split range p, group of up to 128 heads);
// 4 waves, wave w owns 32 heads.  Per 32-token tile:
//   * the 32 cached rows are staged once in LDS as bf16 and shared by all
//     waves.  bf16 rows travel HBM -> LDS directly (global_load_lds_dwordx4,
//     16 bytes per lane, no VGPR staging); fp8 rows are loaded into VGPRs and
//     widened exactly to bf16 on the way.  Rows are stored unpadded with the
//     16-byte chunks of token t permuted by XOR (t & 7), which spreads both
//     read patterns below over the LDS banks;
//   * QK:  Sᵀ[t][h] = Σ_k tile[t][k] · q_abs[h][k]  — v_mfma_f32_32x32x16_bf16
//     with the tile as A (k-contiguous 16-byte LDS reads) and the wave's
//     absorbed queries as B, held in VGPRs for the whole range;
//   * online softmax in the base-2 domain.  In the Sᵀ accumulator layout each
//     lane owns one head (column = lane % 32), so the running max and sum need
//     one cross-half exchange only.  The accumulator is rescaled only when a
//     head's maximum grows by more than 2^8 (exact: numerator and denominator
//     always share the same reference maximum);
//   * PV:  Uᵀ[c][h] += Σ_t tile[t][c] · P[t][h] — the probabilities stay in the
//     registers they were computed in (B operand); the latent, contracted over
//     tokens here, is read from the same LDS tile with ds_read_b64_tr_b16
//     transposing reads (A operand).
// Tiles are double-buffered: the next tile's loads are in flight while the
// current one is computed.  Tokens past the end of the range are loaded from
// the range's first row instead (finite data; their probability is zero).

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kHeadsPerBlock = kWaves * kHeadsPerWave;  // 128
constexpr int kRowBytes = kRowElems * 2;                // 1152: bf16 row in LDS
constexpr int kRowChunks = kRowBytes / 16;              // 72
constexpr int kTileBytes = kTileTokens * kRowBytes;     // 36864
constexpr int kBf16Chunks = kTileTokens * kRowChunks;   // 2304 x 16 B
constexpr int kDmaPerWave = kBf16Chunks / 64 / kWaves;  // 9 wave-loads of 1 KB
constexpr int kFp8RowChunks = kRowElems / 16;           // 36 x 16 B per fp8 row
constexpr int kFp8Chunks = kTileTokens * kFp8RowChunks;               // 1152
constexpr int kFp8PerThread = (kFp8Chunks + kThreads - 1) / kThreads;  // 5
constexpr float kRefSlack = 64.0f;  // log2 units, see the softmax reference note

typedef __attribute__((address_space(3))) void lds_void_t;

struct DecodeParams {
  const void* q_abs;        // [B][H][576] bf16
  const uint8_t* rows;      // cache rows
  const float* row_scale;   // fp8 only
  const int32_t* block_table;
  const int32_t* seq_lens;
  int64_t seq_stride;
  int32_t max_pages;
  int32_t paged;
  int32_t B, H, S, HG, chunk;
  int32_t max_seq_len;
  float scale_log2;
  void* u_part;
  float* lse_part;
};

// byte offset in an LDS tile of 16-byte chunk c of token t
__device__ inline int lds_chunk(int t, int c) { return t * kRowBytes + ((c ^ (t & 7)) << 4); }

// bf16 tile: wave w fills LDS chunk slots [(4i + w)*64, +64) for i = 0..8;
// slot s holds chunk (s % 72) ^ (t & 7) of token t = s / 72.  The per-lane
// source offsets are recomputed for every tile from an opaque copy of the lane
// id, so the compiler does not keep nine of them alive across the loop.
__device__ inline void tile_dma_bf16(const DecodeParams& P, uint8_t* T, int b, int t0, int nvalid,
                                     int wave, int lane) {
  const int64_t row0 = tile_row0(P.block_table, P.max_pages, P.seq_stride, P.paged != 0, b, t0);
  const uint8_t* base = P.rows + row0 * kRowBytes;
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int slot = (i * kWaves + wave) * 64 + ln;
    const int t = slot / kRowChunks;
    const int c = (slot - t * kRowChunks) ^ (t & 7);
    const uint32_t off = static_cast<uint32_t>(((t < nvalid) ? t : 0) * kRowBytes + c * 16);
    __builtin_amdgcn_global_load_lds(base + off, (lds_void_t*)(T + (i * kWaves + wave) * 1024),
                                     16, 0, 0);
  }
}

struct Fp8Regs {
  u32x4_t r[kFp8PerThread];
  float scale;
};

__device__ inline void tile_load_fp8(Fp8Regs& R, const DecodeParams& P, int b, int t0, int nvalid,
                                     int tid) {
  const int64_t row0 = tile_row0(P.block_table, P.max_pages, P.seq_stride, P.paged != 0, b, t0);
  const uint8_t* base = P.rows + row0 * kRowElems;
#pragma unroll
  for (int i = 0; i < kFp8PerThread; ++i) {
    const int q = i * kThreads + tid;
    const int t = q / kFp8RowChunks;
    if (q < kFp8Chunks && t < nvalid)
      R.r[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base) + q);
    else
      R.r[i] = u32x4_t{0u, 0u, 0u, 0u};
  }
  R.scale = (tid < nvalid) ? P.row_scale[row0 + tid] : 0.0f;
}

__device__ inline void tile_store_fp8(const Fp8Regs& R, uint8_t* T, float* tscale, int tid) {
#pragma unroll
  for (int i = 0; i < kFp8PerThread; ++i) {
    const int q = i * kThreads + tid;
    if (q < kFp8Chunks) {
      const int t = q / kFp8RowChunks, cc = q % kFp8RowChunks;
      const u32x2_t a = e4m3x4_to_bf16x4(R.r[i].x), bb = e4m3x4_to_bf16x4(R.r[i].y);
      const u32x2_t c = e4m3x4_to_bf16x4(R.r[i].z), d = e4m3x4_to_bf16x4(R.r[i].w);
      *reinterpret_cast<u32x4_t*>(T + lds_chunk(t, 2 * cc)) = u32x4_t{a.x, a.y, bb.x, bb.y};
      *reinterpret_cast<u32x4_t*>(T + lds_chunk(t, 2 * cc + 1)) = u32x4_t{c.x, c.y, d.x, d.y};
    }
  }
  if (tid < kTileTokens) tscale[tid] = R.scale;
}

template <bool FP8, int PART_DT>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(DecodeParams P) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kTileBytes];
  __shared__ __attribute__((aligned(16))) float sscale[2][kTileTokens];

  const int nwork = P.B * P.S * P.HG;
  const int wid = xcd_remap(blockIdx.x, nwork);
  const int hg = wid % P.HG;
  const int bp = wid / P.HG;
  const int p = bp % P.S;
  const int b = bp / P.S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane & 31;  // head within the wave (column of Sᵀ and Uᵀ)
  const int g = lane >> 5;   // k-slot half
  const int h0 = hg * kHeadsPerBlock + wave * kHeadsPerWave;
  const bool active = h0 < P.H;  // wave-uniform
  const int h = h0 + hl;

  // lengths are clamped to [0, max_seq_len]: the cache is never read past it
  const int L = min(max(P.seq_lens[b], 0), P.max_seq_len);
  const int t_begin = p * P.chunk;
  const int t_end = min(t_begin + P.chunk, L);
  const int64_t out_row = (static_cast<int64_t>(b) * P.S + p) * P.H + h;

  if (t_begin >= t_end) {  // empty range: u = 0, lse = -inf
    if (active) {
      for (int c = g; c < kDLatent; c += 2) store_elem<PART_DT>(P.u_part, out_row * kDLatent + c, 0.0f);
      if (g == 0) P.lse_part[out_row] = -INFINITY;
    }
    return;
  }

  // absorbed queries of this wave's 32 heads as the B operand:
  // lane (hl, g) holds q_abs[h][16*kk + 8*g .. +7] for kk = 0..35
  bf16x8_t qreg[kRowElems / 16];
  if (active) {
    const bf16x8_t* qrow = reinterpret_cast<const bf16x8_t*>(
        static_cast<const uint16_t*>(P.q_abs) + (static_cast<int64_t>(b) * P.H + h) * kRowElems);
#pragma unroll
    for (int kk = 0; kk < kRowElems / 16; ++kk) qreg[kk] = qrow[2 * kk + g];
  }

  // transposing-read geometry: lane (G = lane/16, e, q4) reads rows
  // 16*j + 4*(G/2) + e and +8, columns 32*cb + 16*(G%2) + 4*q4 .. +3
  const int G = lane >> 4, e = (lane >> 2) & 3, q4 = lane & 3;
  const int tr_row = 4 * (G >> 1) + e;
  const int tr_key = tr_row & 7;
  const int tr_x = 2 * (G & 1) + (q4 >> 1);
  const int tr_byte = 8 * (q4 & 1);
  // column chunk 4*cb + tr_x: its low 3 bits are 4*(cb & 1) + tr_x
  const int tr_off[2] = {((0 + tr_x) ^ tr_key) << 4, ((4 + tr_x) ^ tr_key) << 4};
  // QK chunk 2*kk + g of token hl: its low 3 bits are 2*(kk & 3) + g
  int qk_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) qk_off[i] = ((2 * i + g) ^ (hl & 7)) << 4;

  const int ntiles = (t_end - t_begin + kTileTokens - 1) / kTileTokens;

  // Softmax reference.  The probabilities are taken relative to a reference
  // maximum m_ref (log2 domain) fixed at the first tile instead of the running
  // maximum, so the accumulators are never rescaled.  A later score may exceed
  // m_ref by up to kRefSlack: probabilities then stay below 2^kRefSlack, far
  // from the bf16/fp32 range limits.  If any score exceeds it (no realistic
  // logit spread does), the range is recomputed once with m_ref set to the
  // true maximum found by the first pass.  Either way numerator and
  // denominator share one reference, so the result is exact.
  float m_ref = -INFINITY;
  float m_seen = -INFINITY;  // true running max of head h
  float l_run = 0.0f;        // this lane's share of the sum of probabilities
  f32x16_t acc[kDLatent / 32];

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int cb = 0; cb < kDLatent / 32; ++cb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][r] = 0.0f;
      asm volatile("" : "+a"(acc[cb]));
    }
    // The PV MFMAs are inline asm, so the compiler cannot see the hazard
    // between these accumulator writes and their first matrix-core read.
    asm volatile("s_nop 4");
    l_run = 0.0f;
    int overflow = 0;

    Fp8Regs R;
    if constexpr (FP8) {
      tile_load_fp8(R, P, b, t_begin, min(kTileTokens, t_end - t_begin), tid);
      tile_store_fp8(R, smem, sscale[0], tid);
      if (ntiles > 1) {
        const int t1 = t_begin + kTileTokens;
        tile_load_fp8(R, P, b, t1, min(kTileTokens, t_end - t1), tid);
      }
    } else {
      tile_dma_bf16(P, smem, b, t_begin, min(kTileTokens, t_end - t_begin), wave, lane);
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
      const int buf = it & 1;
      uint8_t* T = smem + buf * kTileBytes;
      const int t0 = t_begin + it * kTileTokens;
      if constexpr (!FP8) {
        if (it + 1 < ntiles) {
          const int t1 = t0 + kTileTokens;
          tile_dma_bf16(P, smem + (buf ^ 1) * kTileBytes, b, t1, min(kTileTokens, t_end - t1),
                        wave, lane);
        }
      }
      if (active) {
        // ---- QK: Sᵀ (32 tokens x 32 heads) over the 576-wide row.  Issued as
        //      inline asm so that Sᵀ lives in VGPRs: the 256 AGPRs hold Uᵀ.
        f32x16_t s;
        const uint8_t* arow = T + hl * kRowBytes;
        auto qk_read = [&](int kk) {
          return *reinterpret_cast<const bf16x8_t*>(arow + qk_off[kk & 3] + (kk >> 2) * 128);
        };
        bf16x8_t a0 = qk_read(0), a1 = qk_read(1);
#pragma unroll
        for (int kk = 0; kk < kRowElems / 16; kk += 2) {
          bf16x8_t n0 = a0, n1 = a1;
          if (kk + 2 < kRowElems / 16) {
            n0 = qk_read(kk + 2);
            n1 = qk_read(kk + 3);
          }
          if (kk == 0)
            asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(s) : "v"(a0), "v"(qreg[kk]));
          else
            asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a0), "v"(qreg[kk]));
          asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a1), "v"(qreg[kk + 1]));
          __builtin_amdgcn_sched_barrier(0);
          a0 = n0;
          a1 = n1;
        }
        // the compiler does not see the asm results as MFMA writes: wait out
        // the matrix-core-write -> VALU-read hazard before Sᵀ is read
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
        // ---- softmax.  Register r of lane (hl, g) holds token
        //      8*(r/4) + 4*g + r%4 of the tile, head h.
        const int nvalid = t_end - t0;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s[r] * P.scale_log2;
          if constexpr (FP8) v *= sscale[buf][8 * (r >> 2) + 4 * g + (r & 3)];
          s[r] = v;
        }
        if (nvalid < kTileTokens) {  // partial last tile: drop absent tokens
          const int nv = nvalid - 4 * g;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[r] = (8 * (r >> 2) + (r & 3) < nv) ? s[r] : -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (pass == 0 && it == 0) m_ref = mx;
        m_seen = fmaxf(m_seen, mx);
        overflow |= (mx > m_ref + kRefSlack);
        bf16x8_t pk[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = exp2f(s[r] - m_ref);
          l_run += pr;
          if constexpr (FP8) pr *= sscale[buf][8 * (r >> 2) + 4 * g + (r & 3)];
          pk[r >> 3][r & 7] = static_cast<__bf16>(pr);
        }
        // ---- PV: Uᵀ[c][h] += Σ_t tile[t][c] P[t][h]: 16 column blocks x 2
        //      token blocks of 16
        const uint8_t* r0 = T + tr_row * kRowBytes + tr_byte;
        auto tr_read = [&](int j, int hi, int cb) {
          const uint8_t* ptr =
              r0 + tr_off[cb & 1] + (cb >> 1) * 128 + (16 * j + 8 * hi) * kRowBytes;
          return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)ptr);
        };
        // VALU-written probabilities -> matrix-core read
        asm volatile("s_nop 4" : "+v"(pk[0]), "+v"(pk[1]));
        bf16x4_t c00 = tr_read(0, 0, 0), c01 = tr_read(0, 1, 0);
        bf16x4_t c10 = tr_read(1, 0, 0), c11 = tr_read(1, 1, 0);
#pragma unroll
        for (int cb = 0; cb < kDLatent / 32; ++cb) {
          bf16x4_t n00 = c00, n01 = c01, n10 = c10, n11 = c11;
          if (cb + 1 < kDLatent / 32) {
            n00 = tr_read(0, 0, cb + 1);
            n01 = tr_read(0, 1, cb + 1);
            n10 = tr_read(1, 0, cb + 1);
            n11 = tr_read(1, 1, cb + 1);
          }
          const bf16x8_t A0 = {c00[0], c00[1], c00[2], c00[3], c01[0], c01[1], c01[2], c01[3]};
          const bf16x8_t A1 = {c10[0], c10[1], c10[2], c10[3], c11[0], c11[1], c11[2], c11[3]};
          asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[cb]) : "v"(A0), "v"(pk[0]));
          asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[cb]) : "v"(A1), "v"(pk[1]));
          __builtin_amdgcn_sched_barrier(0);
          c00 = n00;
          c01 = n01;
          c10 = n10;
          c11 = n11;
        }
      }
      if constexpr (FP8) {
        if (it + 1 < ntiles) {
          tile_store_fp8(R, smem + (buf ^ 1) * kTileBytes, sscale[buf ^ 1], tid);
          if (it + 2 < ntiles) {
            const int t2 = t_begin + (it + 2) * kTileTokens;
            tile_load_fp8(R, P, b, t2, min(kTileTokens, t_end - t2), tid);
          }
        }
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      __syncthreads();
    }
    // every wave takes the same number of passes (the tile loop has barriers)
    if (!__syncthreads_or(overflow)) break;
    m_ref = m_seen;
  }

  if (active) {
    // matrix-core accumulator writes -> VALU reads (the MFMAs are inline asm)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    // Uᵀ register r of block cb in lane (hl, g) is column 32*cb + 8*(r/4) + 4*g + r%4
    const int64_t obase = out_row * kDLatent;
#pragma unroll
    for (int cb = 0; cb < kDLatent / 32; ++cb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int c = 32 * cb + 8 * r4 + 4 * g;
        const float v0 = acc[cb][4 * r4 + 0] * inv, v1 = acc[cb][4 * r4 + 1] * inv;
        const float v2 = acc[cb][4 * r4 + 2] * inv, v3 = acc[cb][4 * r4 + 3] * inv;
        if constexpr (PART_DT == MLA_F32) {
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(P.u_part) + obase + c) =
              f32x4_t{v0, v1, v2, v3};
        } else {
          const uint32_t w0 = f32_to_bf16(v0) | (static_cast<uint32_t>(f32_to_bf16(v1)) << 16);
          const uint32_t w1 = f32_to_bf16(v2) | (static_cast<uint32_t>(f32_to_bf16(v3)) << 16);
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(P.u_part) + obase + c) =
              u32x2_t{w0, w1};
        }
      }
    }
    if (g == 0) P.lse_part[out_row] = (m_ref + log2f(l_tot)) * kLn2;
  }
}

// ================================================================ decode (fp32)
//
// Plain fp32 path for fp32 caches: one workgroup per (b, split, head), 256
// threads.  Scores of 256 tokens at a time (one token per thread), exact
// online softmax across those blocks, and the weighted row sum with each
// thread owning two latent columns.

constexpr int kF32Threads = 256;

struct DecodeF32Params {
  const float* q_abs;
  const float* rows;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int64_t seq_stride;
  int32_t max_pages;
  int32_t paged;
  int32_t B, H, S, chunk;
  int32_t max_seq_len;
  float scale;
  void* u_part;
  float* lse_part;
};

__device__ inline int64_t token_row(const DecodeF32Params& P, int b, int t) {
  if (P.paged) {
    const int64_t page = P.block_table[static_cast<int64_t>(b) * P.max_pages + (t >> 6)];
    return page * kPageSize + (t & 63);
  }
  return static_cast<int64_t>(b) * P.seq_stride + t;
}

__device__ inline float block_reduce_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  v = red[0];
  for (int i = 1; i < kF32Threads / 64; ++i) v = fmaxf(v, red[i]);
  return v;
}

__device__ inline float block_reduce_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  v = red[0];
  for (int i = 1; i < kF32Threads / 64; ++i) v += red[i];
  return v;
}

template <int PART_DT>
__global__ __launch_bounds__(kF32Threads) void decode_f32_kernel(DecodeF32Params P) {
  __shared__ float q[kRowElems];
  __shared__ float pw[kF32Threads];
  __shared__ float red[kF32Threads / 64];
  const int h = blockIdx.x % P.H;
  const int p = (blockIdx.x / P.H) % P.S;
  const int b = blockIdx.x / (P.H * P.S);
  const int tid = threadIdx.x;
  const int L = min(max(P.seq_lens[b], 0), P.max_seq_len);
  const int t_begin = p * P.chunk;
  const int t_end = min(t_begin + P.chunk, L);
  const int64_t out_row = (static_cast<int64_t>(b) * P.S + p) * P.H + h;
  for (int k = tid; k < kRowElems; k += kF32Threads)
    q[k] = P.q_abs[(static_cast<int64_t>(b) * P.H + h) * kRowElems + k];
  __syncthreads();

  float m = -INFINITY, l = 0.0f;
  float u0 = 0.0f, u1 = 0.0f;  // columns tid and tid + 256
  for (int tb = t_begin; tb < t_end; tb += kF32Threads) {
    const int t = tb + tid;
    float s = -INFINITY;
    if (t < t_end) {
      const float* row = P.rows + token_row(P, b, t) * kRowElems;
      float acc = 0.0f;
      for (int k = 0; k < kRowElems; ++k) acc = fmaf(q[k], row[k], acc);
      s = acc * P.scale;
    }
    const float mt = block_reduce_max(s, red);
    const float m_new = fmaxf(m, mt);
    const float alpha = (m == -INFINITY) ? 0.0f : expf(m - m_new);
    const float e = (t < t_end) ? expf(s - m_new) : 0.0f;
    const float lt = block_reduce_sum(e, red);
    l = l * alpha + lt;
    u0 *= alpha;
    u1 *= alpha;
    m = m_new;
    pw[tid] = e;
    __syncthreads();
    const int n = min(kF32Threads, t_end - tb);
    for (int j = 0; j < n; ++j) {
      const float* row = P.rows + token_row(P, b, tb + j) * kRowElems;
      u0 = fmaf(pw[j], row[tid], u0);
      u1 = fmaf(pw[j], row[tid + kF32Threads], u1);
    }
    __syncthreads();
  }
  const bool empty = t_begin >= t_end;
  const float inv = empty ? 0.0f : 1.0f / l;
  store_elem<PART_DT>(P.u_part, out_row * kDLatent + tid, u0 * inv);
  store_elem<PART_DT>(P.u_part, out_row * kDLatent + tid + kF32Threads, u1 * inv);
  if (tid == 0) P.lse_part[out_row] = empty ? -INFINITY : m + logf(l);
}

// ================================================================ combine
//
// One workgroup of 128 threads per (b, head): log-sum-exp weights of the S
// partials, then each thread sums four latent columns over the partials.

constexpr int kCombThreads = 128;

template <int PART_DT, int U_DT>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const void* u_part,
                                                              const float* lse_part, void* u,
                                                              float* lse, int H, int S) {
  extern __shared__ float wts[];  // [S]
  __shared__ float red[2];
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x;
  float mx = -INFINITY;
  for (int p = tid; p < S; p += kCombThreads)
    mx = fmaxf(mx, lse_part[(static_cast<int64_t>(b) * S + p) * H + h]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  __syncthreads();
  float z = 0.0f;
  for (int p = tid; p < S; p += kCombThreads) {
    const float lp = lse_part[(static_cast<int64_t>(b) * S + p) * H + h];
    const float w = (mx == -INFINITY) ? 0.0f : expf(lp - mx);
    wts[p] = w;
    z += w;
  }
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
  if ((tid & 63) == 0) red[tid >> 6] = z;
  __syncthreads();
  z = red[0] + red[1];
  const float inv = (z > 0.0f) ? 1.0f / z : 0.0f;
  float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int c0 = tid * 4;
  for (int p = 0; p < S; ++p) {
    const float w = wts[p];
    if (w == 0.0f) continue;
    const int64_t base = ((static_cast<int64_t>(b) * S + p) * H + h) * kDLatent + c0;
    if constexpr (PART_DT == MLA_F32) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(u_part) + base);
      a[0] = fmaf(w, v[0], a[0]);
      a[1] = fmaf(w, v[1], a[1]);
      a[2] = fmaf(w, v[2], a[2]);
      a[3] = fmaf(w, v[3], a[3]);
    } else {
      const u32x2_t v = *reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(u_part) + base);
      a[0] = fmaf(w, __uint_as_float(v.x << 16), a[0]);
      a[1] = fmaf(w, __uint_as_float(v.x & 0xFFFF0000u), a[1]);
      a[2] = fmaf(w, __uint_as_float(v.y << 16), a[2]);
      a[3] = fmaf(w, __uint_as_float(v.y & 0xFFFF0000u), a[3]);
    }
  }
  const int64_t ob = (static_cast<int64_t>(b) * H + h) * kDLatent + c0;
#pragma unroll
  for (int i = 0; i < 4; ++i) store_elem<U_DT>(u, ob + i, a[i] * inv);
  if (lse && tid == 0) lse[static_cast<int64_t>(b) * H + h] = (z > 0.0f) ? mx + logf(z) : -INFINITY;
}

// ================================================================ absorb
//
// q_abs[b][h][c] = Σ_n q_nope[b][h][n] W_UK[h][n][c] for a block of up to 8
// sequences per workgroup; thread t owns latent columns 2t and 2t+1 and
// streams the head's W_UK rows (coalesced across the workgroup).

constexpr int kAbsThreads = 256;
constexpr int kAbsBatch = 8;

template <int Q_DT, int W_DT, int OUT_DT>
__global__ __launch_bounds__(kAbsThreads) void absorb_kernel(const void* q_nope, const void* q_rope,
                                                            const void* w_uk, void* q_abs,
                                                            float* q_abs_scale, int B, int H,
                                                            int d_nope) {
  __shared__ float qs[kAbsBatch][kMaxDHead];
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * kAbsBatch;
  const int nb = min(kAbsBatch, B - b0);
  const int tid = threadIdx.x;
  for (int i = tid; i < nb * d_nope; i += kAbsThreads) {
    const int bb = i / d_nope, n = i % d_nope;
    qs[bb][n] = load_elem<Q_DT>(q_nope, (static_cast<int64_t>(b0 + bb) * H + h) * d_nope + n);
  }
  __syncthreads();
  float acc[kAbsBatch][2];
#pragma unroll
  for (int bb = 0; bb < kAbsBatch; ++bb) acc[bb][0] = acc[bb][1] = 0.0f;
  const int c = 2 * tid;
  for (int n = 0; n < d_nope; ++n) {
    const int64_t wi = (static_cast<int64_t>(h) * d_nope + n) * kDLatent + c;
    const float w0 = load_elem<W_DT>(w_uk, wi), w1 = load_elem<W_DT>(w_uk, wi + 1);
#pragma unroll
    for (int bb = 0; bb < kAbsBatch; ++bb) {
      acc[bb][0] = fmaf(qs[bb][n], w0, acc[bb][0]);
      acc[bb][1] = fmaf(qs[bb][n], w1, acc[bb][1]);
    }
  }
  for (int bb = 0; bb < nb; ++bb) {
    const int64_t ob = (static_cast<int64_t>(b0 + bb) * H + h) * kRowElems;
    float r0 = 0.0f;  // RoPE element handled by this thread (tid < 64)
    if (tid < kDRope)
      r0 = load_elem<Q_DT>(q_rope, (static_cast<int64_t>(b0 + bb) * H + h) * kDRope + tid);
    if constexpr (OUT_DT == MLA_FP8_E4M3) {
      // the fp8 absorbed query is not provided yet
      (void)q_abs_scale;
    } else {
      store_elem<OUT_DT>(q_abs, ob + c, acc[bb][0]);
      store_elem<OUT_DT>(q_abs, ob + c + 1, acc[bb][1]);
      if (tid < kDRope) store_elem<OUT_DT>(q_abs, ob + kDLatent + tid, r0);
    }
  }
}

// ================================================================ up-projection
//
// o[b][h][v] = Σ_c W_UV[h][v][c] u[b][h][c]: one workgroup per (head, block of
// 8 sequences); the u rows sit in LDS (read as broadcasts), thread v streams
// row v of W_UV[h] 16 bytes at a time.

constexpr int kUpBatch = 8;

template <int U_DT, int W_DT, int O_DT>
__global__ __launch_bounds__(kMaxDHead) void up_proj_kernel(const void* u, const void* w_uv, void* o,
                                                           int B, int H, int d_v) {
  __shared__ float us[kUpBatch][kDLatent];
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * kUpBatch;
  const int nb = min(kUpBatch, B - b0);
  const int tid = threadIdx.x;
  for (int i = tid; i < kUpBatch * kDLatent; i += blockDim.x) {
    const int bb = i / kDLatent, c = i % kDLatent;
    us[bb][c] = (bb < nb) ? load_elem<U_DT>(u, (static_cast<int64_t>(b0 + bb) * H + h) * kDLatent + c) : 0.0f;
  }
  __syncthreads();
  const int v = tid;
  if (v >= d_v) return;
  float acc[kUpBatch];
#pragma unroll
  for (int bb = 0; bb < kUpBatch; ++bb) acc[bb] = 0.0f;
  const int64_t wrow = (static_cast<int64_t>(h) * d_v + v) * kDLatent;
  for (int c = 0; c < kDLatent; c += 8) {
    float w[8];
    if constexpr (W_DT == MLA_F32) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(w_uv) + wrow + c);
      const f32x4_t bq = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(w_uv) + wrow + c + 4);
      w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
      w[4] = bq[0]; w[5] = bq[1]; w[6] = bq[2]; w[7] = bq[3];
    } else {
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(w_uv) + wrow + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[2 * i] = __uint_as_float(a[i] << 16);
        w[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int bb = 0; bb < kUpBatch; ++bb)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[bb] = fmaf(w[i], us[bb][c + i], acc[bb]);
  }
  for (int bb = 0; bb < nb; ++bb)
    store_elem<O_DT>(o, (static_cast<int64_t>(b0 + bb) * H + h) * d_v + v, acc[bb]);
}

mla_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_E_HIP;
}

}  // namespace
}  // namespace mla

using namespace mla;

// ================================================================ entry points

extern "C" mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t B, const void* q_nope,
                                     const void* q_rope, int32_t q_dt, const void* w_uk,
                                     int32_t w_dt, void* q_abs, int32_t q_abs_dt,
                                     float* q_abs_scale, void* stream) {
  mla_status_t st = check_absorb(dims, B, q_nope, q_rope, q_dt, w_uk, w_dt, q_abs, q_abs_dt,
                                 q_abs_scale);
  if (st != MLA_OK || B == 0) return st;
  if (q_abs_dt == MLA_FP8_E4M3) return MLA_E_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(dims->heads, (B + kAbsBatch - 1) / kAbsBatch);
  const int H = dims->heads, dn = dims->d_nope;
#define MLA_ABS(QD, WD, OD)                                                                     \
  if (q_dt == QD && w_dt == WD && q_abs_dt == OD) {                                             \
    absorb_kernel<QD, WD, OD><<<grid, kAbsThreads, 0, s>>>(q_nope, q_rope, w_uk, q_abs,         \
                                                           q_abs_scale, B, H, dn);              \
    return launch_status();                                                                     \
  }
  MLA_ABS(MLA_F32, MLA_F32, MLA_F32)
  MLA_ABS(MLA_F32, MLA_F32, MLA_BF16)
  MLA_ABS(MLA_BF16, MLA_BF16, MLA_BF16)
  MLA_ABS(MLA_BF16, MLA_BF16, MLA_F32)
  MLA_ABS(MLA_F32, MLA_BF16, MLA_BF16)
  MLA_ABS(MLA_BF16, MLA_F32, MLA_BF16)
#undef MLA_ABS
  return MLA_E_DTYPE;
}

extern "C" mla_status_t mla_decode(const mla_dims_t* dims, int32_t B, const void* q_abs,
                                   int32_t q_abs_dt, const float* q_abs_scale,
                                   const mla_cache_t* cache, int32_t num_splits, void* u_part,
                                   int32_t part_dt, float* lse_part, void* stream) {
  mla_status_t st = check_decode(dims, B, q_abs, q_abs_dt, q_abs_scale, cache, num_splits,
                                 u_part, part_dt, lse_part);
  if (st != MLA_OK || B == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t H = dims->heads;
  // with max_seq_len == 0 every range is empty; a chunk of 32 keeps the
  // kernels' range arithmetic well defined
  const int32_t chunk = max(split_chunk(cache->max_seq_len, num_splits), kTileTokens);
  const float scale = effective_scale(dims);
  if (cache->dtype == MLA_F32) {
    DecodeF32Params P{static_cast<const float*>(q_abs), static_cast<const float*>(cache->rows),
                      cache->block_table, cache->seq_lens, cache->seq_stride, cache->max_pages,
                      cache->page_size != 0, B, H, num_splits, chunk, cache->max_seq_len, scale,
                      u_part, lse_part};
    const int64_t nblk = static_cast<int64_t>(B) * num_splits * H;
    if (nblk > 0x7FFFFFFF) return MLA_E_SHAPE;
    if (part_dt == MLA_F32)
      decode_f32_kernel<MLA_F32><<<static_cast<unsigned>(nblk), kF32Threads, 0, s>>>(P);
    else
      decode_f32_kernel<MLA_BF16><<<static_cast<unsigned>(nblk), kF32Threads, 0, s>>>(P);
    return launch_status();
  }
  const int32_t HG = (H + kHeadsPerBlock - 1) / kHeadsPerBlock;
  DecodeParams P{q_abs, static_cast<const uint8_t*>(cache->rows), cache->row_scale,
                 cache->block_table, cache->seq_lens, cache->seq_stride, cache->max_pages,
                 cache->page_size != 0, B, H, num_splits, HG, chunk, cache->max_seq_len,
                 scale * kLog2e, u_part, lse_part};
  const int64_t nblk = static_cast<int64_t>(B) * num_splits * HG;
  if (nblk > 0x7FFFFFFF) return MLA_E_SHAPE;
  const unsigned grid = static_cast<unsigned>(nblk);
  const bool fp8 = cache->dtype == MLA_FP8_E4M3;
  if (!fp8 && part_dt == MLA_F32) decode_mfma_kernel<false, MLA_F32><<<grid, kThreads, 0, s>>>(P);
  else if (!fp8) decode_mfma_kernel<false, MLA_BF16><<<grid, kThreads, 0, s>>>(P);
  else if (part_dt == MLA_F32) decode_mfma_kernel<true, MLA_F32><<<grid, kThreads, 0, s>>>(P);
  else decode_mfma_kernel<true, MLA_BF16><<<grid, kThreads, 0, s>>>(P);
  return launch_status();
}

extern "C" mla_status_t mla_combine(const mla_dims_t* dims, int32_t B, int32_t num_splits,
                                    const void* u_part, int32_t part_dt, const float* lse_part,
                                    void* u, int32_t u_dt, float* lse, void* stream) {
  mla_status_t st = check_combine(dims, B, num_splits, u_part, part_dt, lse_part, u, u_dt);
  if (st != MLA_OK || B == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = dims->heads;
  const int64_t nblk = static_cast<int64_t>(B) * H;
  if (nblk > 0x7FFFFFFF) return MLA_E_SHAPE;
  const size_t shm = sizeof(float) * num_splits;
  const unsigned grid = static_cast<unsigned>(nblk);
#define MLA_COMB(PD, UD)                                                                       \
  if (part_dt == PD && u_dt == UD) {                                                           \
    combine_kernel<PD, UD><<<grid, kCombThreads, shm, s>>>(u_part, lse_part, u, lse, H,        \
                                                           num_splits);                        \
    return launch_status();                                                                    \
  }
  MLA_COMB(MLA_F32, MLA_F32)
  MLA_COMB(MLA_F32, MLA_BF16)
  MLA_COMB(MLA_BF16, MLA_F32)
  MLA_COMB(MLA_BF16, MLA_BF16)
#undef MLA_COMB
  return MLA_E_DTYPE;
}

extern "C" mla_status_t mla_up_proj(const mla_dims_t* dims, int32_t B, const void* u,
                                    int32_t u_dt, const void* w_uv, int32_t w_dt, void* o,
                                    int32_t o_dt, void* stream) {
  mla_status_t st = check_up_proj(dims, B, u, u_dt, w_uv, w_dt, o, o_dt);
  if (st != MLA_OK || B == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = dims->heads, dv = dims->d_v;
  const dim3 grid(H, (B + kUpBatch - 1) / kUpBatch);
#define MLA_UP(UD, WD, OD)                                                                      \
  if (u_dt == UD && w_dt == WD && o_dt == OD) {                                                 \
    up_proj_kernel<UD, WD, OD><<<grid, kMaxDHead, 0, s>>>(u, w_uv, o, B, H, dv);                \
    return launch_status();                                                                     \
  }
  MLA_UP(MLA_F32, MLA_F32, MLA_F32)
  MLA_UP(MLA_F32, MLA_BF16, MLA_F32)
  MLA_UP(MLA_F32, MLA_BF16, MLA_BF16)
  MLA_UP(MLA_BF16, MLA_BF16, MLA_BF16)
  MLA_UP(MLA_BF16, MLA_BF16, MLA_F32)
  MLA_UP(MLA_F32, MLA_F32, MLA_BF16)
#undef MLA_UP
  return MLA_E_DTYPE;
}
