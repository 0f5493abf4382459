// Tile layout, DMA and parameter block shared by the MLA decode kernels
// (gfx950): the bf16 and fp8 kernels stage their tiles with the same LDS-DMA
// plan and token-group layout.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mla_device.h"
#include "mla_host.h"

namespace mla {

// Arguments of the MLA decode kernels (one per launch, passed by value).
struct DecodeParams {
  const void* q_abs;        // [B][QL][H][576] bf16, or E4M3 codes
  const uint8_t* rows;      // cache rows
  const float* row_scale;   // fp8 only
  const int32_t* block_table;
  const int32_t* seq_lens;
  int64_t seq_stride;
  int32_t max_pages;
  int32_t paged;
  int32_t B, H, S, HG, chunk;
  int32_t max_seq_len;
  int32_t QL;  // query tokens per sequence (1: plain decode)
  float scale_log2;
  void* u_part;
  float* lse_part;
  int32_t ring;  // contiguous rows used as a ring of seq_stride slots
  const float* q_scale;  // E4M3 query: one factor per (b, query token, head)
  // split slots per row of u_part / lse_part (>= S): when the host merges R
  // consecutive split ranges into one range per workgroup, S counts the merged
  // ranges and slots S .. S_out - 1 are empty (lse = -inf)
  int32_t S_out;
};

// fp8 cache and fp8 absorbed query, on the fp8 matrix cores (one workgroup
// per (sequence, query token, group of consecutive split ranges, 64 heads))
mla_status_t decode_fp8q_launch(const DecodeParams& P, int32_t part_dt, hipStream_t s);

namespace {

constexpr int kRowBytes = kRowElems * 2;             // 1152: bf16 row in LDS
constexpr int kTileBytes = kTileTokens * kRowBytes;  // 36864
constexpr int kDmaPerWave = kTileBytes / 1024 / 4;   // 9 wave-loads of 1 KB per wave of 4
constexpr int kNBuf = 4;                             // LDS tile buffers
// Softmax reference.  The probabilities are taken relative to a reference
// maximum m_ref (log2 domain) fixed at the first tile of the range instead of
// the running maximum, so the accumulators are never rescaled.  A later score
// may exceed m_ref by up to kRefSlack: probabilities then stay below
// 2^kRefSlack, far from the bf16/fp32 range limits.  If any score exceeds it
// (no realistic logit spread does), the range is computed again with m_ref set
// to the true maximum found by the first pass.  Either way numerator and
// denominator share one reference, so the result is exact.
constexpr float kRefSlack = 64.0f;  // log2 units

typedef __attribute__((address_space(3))) void lds_void_t;


// Tokens of sequence b that the decode attends: its length, clamped to the
// host bound; a ring of C slots holds (and attends) only the last C, which
// sit in its first min(L, C) rows -- attention does not depend on their order.
__device__ inline int attended_len(const int32_t* seq_lens, int b, int max_seq_len,
                                   int ring, int64_t seq_stride) {
  int L = min(max(seq_lens[b], 0), max_seq_len);
  if (ring) L = static_cast<int>(min(static_cast<int64_t>(L), seq_stride));
  return L;
}

__device__ inline uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}

// ================================================================ decode: tile layout
//
// The work unit is (sequence b, split range p, group of up to 64 heads);
// tiles of 32 tokens sit in LDS as bf16 in the token-group layout below.

constexpr int kH64 = 64;                 // heads per workgroup
constexpr int kH64Blocks = 2;            // head blocks of 32
constexpr int kQkSteps = kRowElems / 32;  // 18 k-steps of 32
constexpr int kP64Bytes = 4096;           // bf16 probabilities, 64 heads x 32 tokens
constexpr int kX64Off = kNBuf * kTileBytes + 2 * kP64Bytes;  // exchange area (float[2][64] + votes)

// Token-group tile layout: tokens in groups of 8 and 16-byte chunks in groups
// of 8, token t / chunk c at
//   (t / 8) * 9216 + (c / 8) * 1024 + (t % 8) * 128 + ((c % 8) ^ swzg(t)) * 16,
//   swzg(t) = (5 (t % 8) mod 8) xor (2 (t & 2)).
// One 1 KB LDS-DMA wave instruction moves 8 tokens x 8 chunks, i.e. 8 whole
// 128-byte lines of the cache, and a lane's source offset is the same for all
// 9 instructions of a wave (only the scalar base and M0 advance).  The XOR key
// was chosen by measurement (SQ_LDS_BANK_CONFLICT on gfx950, one read pattern
// per kernel): with it neither operand read has bank conflicts -- the 16x16x32
// QK read (16 lanes = one chunk of 8 rows in each of two groups) nor the
// transposing PV read (per half-wave 4 rows x 4 chunks: rows t and t + 2 need
// keys that differ in bit 2, which 5t mod 8 alone does not give; it cost two
// extra LDS cycles per ds_read_b64_tr_b16).
constexpr int kTokGroupBytes = 8 * kRowBytes;  // 9216

__device__ inline int swzg(int t) { return ((5 * t) & 7) ^ ((t & 2) << 1); }

// DMA of 32 rows of 1152 bytes starting at `base` (rows consecutive in
// memory) into an LDS tile in the token-group layout; wave w moves rows
// 8w..8w+7, rows >= nvalid are replaced by row 0.
// The 9 wave instructions can be issued one at a time (rows_dma_issue), spread
// between other work: the vector memory unit of a CU accepts about 64 bytes
// per clock, so the 36 instructions of a tile occupy it for ~600 clocks.
struct RowsDma {
  const uint8_t* base;  // wave-uniform
  uint32_t off;         // per lane
  uint32_t m0;          // wave-uniform
};

__device__ inline RowsDma rows_dma_plan(const uint8_t* base, uint32_t lds_tile, int nvalid, int wave) {
  int ln;  // volatile: recomputed per call rather than kept live across the loop
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  const int k = ln >> 3, j = ln & 7;
  const int t = 8 * wave + k;
  RowsDma d;
  d.base = base;
  d.off = static_cast<uint32_t>(((t < nvalid) ? t : 0) * kRowBytes + ((j ^ swzg(t)) << 4));
  d.m0 = lds_tile + wave * kTokGroupBytes;
  return d;
}

__device__ inline void rows_dma_issue(const RowsDma& d, int i) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(d.off), "s"(d.base + 128 * i),
               "{m0}"(d.m0 + 1024 * i) : "memory");
}

__device__ inline void rows_dma_g8(const uint8_t* base, uint32_t lds_tile, int nvalid, int wave) {
  const RowsDma d = rows_dma_plan(base, lds_tile, nvalid, wave);
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) rows_dma_issue(d, i);
}

}  // namespace
}  // namespace mla
