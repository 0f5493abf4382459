// MLA decode for an E4M3 latent cache with an E4M3 absorbed query, on the fp8
// matrix cores of gfx950 (v_mfma_f32_32x32x64_f8f6f4 and its block-scaled
// form).
//
// What is computed is the absorbed form of multi-head latent attention ("DeepSeek
// V2的MLA注意力机制…" page, §2.3): the score of token t for head h is the dot
// product of the absorbed query row [q~ | q_R] with the cached row [c_KV | k_R]
// times the softmax scale, and the split partial is the softmax-weighted sum
// of c_KV.  The rows are stored in FP8 with one fp32 factor per token (the FP8
// KV cache of the "engineering DeepSeek sparse attention long context
// inference" page), and so is the query, with one factor per head.
//
// Work decomposition, roles and barriers are those of the bf16
// warp-specialised decode (one workgroup per (sequence, query token, split
// range, 64 heads); 8 waves, 4 QK + 4 PV, two per SIMD).  What differs:
//   * a tile holds 64 tokens: 64 rows of 576 codes = 36 KB, the bf16 tile's
//     size, moved by the same LDS-DMA plan with each pair of 576-byte rows
//     (tokens 2r, 2r + 1: 1152 contiguous bytes in every cache layout, pages
//     being 64 tokens long) in place of one bf16 row;
//   * QK: S^T[t][h] for 32 tokens x 32 heads per wave with 9 fp8 MFMAs
//     (K = 64 codes each), the raw row codes as A and the query codes, held
//     in AGPRs, as B.  The scores are then multiplied by the token's row
//     factor, the head's query factor and the softmax scale;
//   * PV: U^T[c][h] += sum_t V[t][c] P'[t][h] with P' = p x row factor on the
//     block-scaled fp8 MFMA.  P' goes to E4M3 with one power-of-two factor per
//     (head, 32-token half) -- the instruction's E8M0 operand scale, applied
//     exactly -- chosen so that the half's largest value lands in [128, 256);
//     V is the raw codes, read with transposing byte reads (ds_read_b64_tr_b8).
//     The partial is normalised by the sum of the weights the product used
//     (each rounded P' over its row factor), so that it stays a convex
//     combination of the rows: one dominant token gives its row exactly
//     instead of the row times its rounding error (up to 2^-4).  The
//     log-sum-exp, which weights the ranges in the combine, sums the
//     unrounded p.
// No code is widened: the LDS holds the codes as they are in HBM.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/mla.h"
#include "mla_decode_tile.h"
#include "mla_device.h"
#include "mla_host.h"

namespace mla {
namespace {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

constexpr int kF8Threads = 512;
constexpr int kF8Tok = 64;                  // tokens per tile
constexpr int kF8Steps = kRowElems / 64;    // 9 QK k-steps of 64 codes
constexpr int kF8PBytes = kH64 * kF8Tok;    // P' codes of one tile: 64 heads x 64 tokens
// LDS map past the 4 tile buffers
constexpr int kF8POff = kNBuf * kTileBytes;             // P' [2 tiles][hb][half][lane][16 B]
constexpr int kF8SOff = kF8POff + 2 * kF8PBytes;        // P' factors [2 tiles][hb][half][32] (E8M0)
constexpr int kF8ROff = kF8SOff + 2 * 128;              // row factors [kNBuf][64] fp32
constexpr int kF8XOff = kF8ROff + kNBuf * kF8Tok * 4;   // exchange float[2][2][64], linv float[64], votes int[8]
constexpr int kF8Lds = kF8XOff + 1024 + 256 + 32;
static_assert(kF8Lds <= 160 * 1024, "fp8 decode LDS");
// vector-memory instructions per tile and PV wave: 9 row lines + 1 factor load
// (the s_waitcnt vmcnt counts below are multiples of it)
static_assert(kDmaPerWave + 1 == 10, "fp8 decode wait counts");

// Byte offset in a tile buffer of 16-byte chunk c (0..35) of element row e (a
// token of the tile, or a head of the staged queries): rows e = 2r, 2r + 1
// together take the place of 1152-byte row r of the token-group layout.  With
// this map the QK operand reads (8 lanes: 4 pairs x both rows, one chunk) and
// the transposing PV reads (16 lanes: 4 pairs x both rows, one chunk) each
// touch 8 distinct 16-byte slots of the 128-byte bank row: the pair's second
// row sits 36 chunks on, which flips bit 2 of the slot, and the key of
// swzg differs in bits 0-1 for 4 consecutive pair rows.
__device__ inline int f8_chunk(int e, int c) {
  const int r = e >> 1, pc = 36 * (e & 1) + c;
  return (r >> 3) * kTokGroupBytes + (pc >> 3) * 1024 + (r & 7) * 128 + (((pc & 7) ^ swzg(r)) << 4);
}

// LDS DMA of the 64 rows of a tile (or of 64 query rows) whose element 0 is at
// `base`: wave w moves pair rows 8w..8w+7.  Elements >= nvalid are never
// read: a pair past the end reads pair 0, and the second row of a pair whose
// first row is the last valid one reads that first row again, so every byte
// read belongs to the sequence (the rows after it may be unwritten or past
// the allocation).  Line i of a pair row holds chunks 8i..8i+7; chunks 36
// and up are the pair's second row, so lines 0-3 never move it, line 4 does
// for slots 4-7, and lines 5-8 always.  Each group of lines keeps its own
// non-negative lane offset from its own scalar base.
struct F8Dma {
  const uint8_t* base;
  uint32_t off[3];  // lines 0-3 (from base + 128 i), line 4 (from base), 5-8 (from base + 128 (i - 5))
  uint32_t m0;
};

__device__ inline F8Dma f8_dma_plan(const uint8_t* base, uint32_t lds_tile, int nvalid, int wave) {
  int ln;  // volatile: recomputed per call rather than kept live across the loop
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  const int t = 8 * wave + (ln >> 3);
  const int slot = (ln & 7) ^ swzg(t);
  const int src = (2 * t < nvalid) ? t : 0;
  const uint32_t back = (2 * src + 1 < nvalid) ? 0u : 576u;
  const uint32_t o = static_cast<uint32_t>(src * kRowBytes + (slot << 4));
  F8Dma d;
  d.base = base;
  d.off[0] = o;
  d.off[1] = o + 512u - (slot >= 4 ? back : 0u);
  d.off[2] = o + 640u - back;
  d.m0 = lds_tile + wave * kTokGroupBytes;
  return d;
}

__device__ inline void f8_dma_issue(const F8Dma& d, int i) {
  const uint32_t off = i < 4 ? d.off[0] : (i == 4 ? d.off[1] : d.off[2]);
  const uint8_t* sb = d.base + 128 * (i < 4 ? i : (i == 4 ? 0 : i - 5));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sb), "{m0}"(d.m0 + 1024 * i)
               : "memory");
}

// Row factors of tokens 16w..16w+15 of a tile (lanes 0-15 of PV wave w, one
// dword each, into factors[16w..]); tokens >= nvalid read token 0's.
__device__ inline void f8_factor_issue(const float* tile_scale, uint32_t lds_factors, int nvalid,
                                       int wave, int lane) {
  if (lane < 16) {
    const int t = 16 * wave + lane;
    const uint32_t off = static_cast<uint32_t>((t < nvalid ? t : 0) * 4);
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(tile_scale),
                 "{m0}"(lds_factors + 64 * wave)
                 : "memory");
  }
}

template <int PART_DT>
__global__ __attribute__((amdgpu_flat_work_group_size(kF8Threads, kF8Threads),
                          amdgpu_waves_per_eu(2, 2)))
void decode_f8q_kernel(DecodeParams P, const int32_t* __restrict__ block_table) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kF8Lds];
  float* rfac = reinterpret_cast<float*>(smem + kF8ROff);  // [kNBuf][64] row factors
  float* xch = reinterpret_cast<float*>(smem + kF8XOff);   // [2][2][64] per-head exchange
  float* linv = xch + 256;                                 // [64] 1 / normaliser per head
  int* votes = reinterpret_cast<int*>(smem + kF8XOff + 1280);

  // work id -> (head group, query token j, split range p, sequence b; the
  // consecutive ranges that the host merged count as one), the head groups and
  // query tokens of one range adjacent (same XCD: they share each tile through
  // L2)
  const int nwork = P.B * P.QL * P.S * P.HG;
  const int wid = xcd_remap(blockIdx.x, nwork);
  const int hg = wid % P.HG;
  const int r1 = wid / P.HG;
  const int qj = r1 % P.QL;
  const int r2 = r1 / P.QL;
  const int p = r2 % P.S;  // the split (a range the host merged from several is one)
  const int b = r2 / P.S;
  const int bj = b * P.QL + qj;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool is_qk = wave < 4;
  const int rw = wave & 3;
  const int hbase = hg * kH64;
  const int nhb = min(kH64Blocks, (P.H - hbase) / kHeadsPerWave);

  const int L = max(attended_len(P.seq_lens, b, P.max_seq_len, P.ring, P.seq_stride) -
                        (P.QL - 1 - qj), 0);
  // the workgroup's range covers tokens [T0, T1): K consecutive 64-token tiles
  const int T0 = p * P.chunk;
  const int T1 = min((p + 1) * P.chunk, L);
  const int K = T1 > T0 ? (T1 - T0 + kF8Tok - 1) / kF8Tok : 0;
  const int k0 = 0, k1 = K;  // the range's tiles
  auto row_base = [&](int sp) { return (static_cast<int64_t>(bj) * P.S_out + sp) * P.H + hbase; };

  // splits without tokens (PV waves): lse = -inf, and u = 0 unless lse_only
  // (the slots past merged range groups: mla_combine does not read the u of a
  // split with lse = -inf)
  auto write_empty = [&](int sp, bool lse_only = false) {
    const int pt = tid - 256;
    if (!lse_only)
      for (int idx = pt; idx < nhb * kHeadsPerWave * kDLatent; idx += 256)
        store_elem<PART_DT>(P.u_part, row_base(sp) * kDLatent + idx, 0.0f);
    if (pt < nhb * kHeadsPerWave) P.lse_part[row_base(sp) + pt] = -INFINITY;
  };
  // the workgroup of the last range also marks the slots past the ranges
  if (!is_qk && p + 1 == P.S)
    for (int q = P.S; q < P.S_out; ++q) write_empty(q, true);
  if (K == 0) {
    if (!is_qk) write_empty(p);
    return;
  }

  // s_barriers, issued by both roles in the same order:
  //   Q1 Q2 T0 | [pass 0: AM AM] B_0 .. B_K-1 V1 V2
  //   [redo: AM AM T0 B_0 .. B_K-1 V1 V2] E1 E2
  auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  if (is_qk) {
    // ------------------------------------------------------------ QK role
    // wave (qhb, th): heads 32 qhb + n, tokens 32 th .. 32 th + 31 of each tile
    const int qhb = rw & 1, th = rw >> 1;
    const bool active = qhb < nhb;
    const int n = lane & 31, gq = lane >> 5;
    const float qf = active ? P.q_scale[static_cast<int64_t>(bj) * P.H + hbase + 32 * qhb + n] *
                                  P.scale_log2
                            : 0.0f;
    // A operand of k-step ks: chunks 4 ks + gq and 4 ks + 2 + gq of token
    // 32 th + n; the chunk pair of k-step ks sits (ks / 2) KB past that of
    // k-step ks % 2 (the pair row's line advances by one every 8 chunks)
    int abase[2][2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int j = 0; j < 2; ++j) abase[e][j] = f8_chunk(32 * th + n, 4 * e + 2 * j + gq);
    // l_run: sum of p (the log-sum-exp); l_used: sum of the weights the value
    // product multiplies, rounded P' / row factor (the normalisation of u)
    float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.0f, l_used = 0.0f;
    i32x8_t qb[kF8Steps];  // B operands: the query codes of head 32 qhb + n

    barrier();  // Q1: the queries are staged in tile buffer 3
    if (active) {
      const uint8_t* Q = smem + 3 * kTileBytes;
#pragma unroll
      for (int ks = 0; ks < kF8Steps; ++ks) {
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(Q + f8_chunk(32 * qhb + n, 4 * ks + gq));
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(Q + f8_chunk(32 * qhb + n, 4 * ks + 2 + gq));
        qb[ks] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        asm volatile("" : "+a"(qb[ks]));
      }
    }
    barrier();  // Q2: staging buffer free

    auto ld_a = [&](const uint8_t* T, int ks) {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(T + abase[ks & 1][0] + (ks >> 1) * 1024);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(T + abase[ks & 1][1] + (ks >> 1) * 1024);
      return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    // raw scores of the wave's 32 tokens x 32 heads: lane (n, gq), register r
    // holds token 32 th + 8 (r / 4) + 4 gq + r % 4 of head 32 qhb + n
    auto qk_tile = [&](const uint8_t* T, f32x16_t& s) {
      constexpr int kRing = 3;
      i32x8_t ring[kRing];
#pragma unroll
      for (int k = 0; k < kRing; ++k) ring[k] = ld_a(T, k);
#pragma unroll
      for (int ks = 0; ks < kF8Steps; ++ks) {
        const i32x8_t a = ring[ks % kRing];
        if (ks + kRing < kF8Steps) ring[ks % kRing] = ld_a(T, ks + kRing);
        if (ks == 0)
          asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=v"(s) : "v"(a), "a"(qb[ks]));
        else
          asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(s) : "v"(a), "a"(qb[ks]));
        __builtin_amdgcn_sched_barrier(0);
      }
      // matrix-core result -> VALU reads (16-pass MFMA)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
    };
    // row factors of the lane's 16 tokens of tile buffer buf
    auto load_factors = [&](float (&rs)[16], int buf) {
      const float* rp = rfac + buf * kF8Tok + 32 * th + 4 * gq;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(rp + 8 * s4);
#pragma unroll
        for (int q = 0; q < 4; ++q) rs[4 * s4 + q] = v[q];
      }
    };
    // scores in the log2 domain: raw x row factor x query factor x scale;
    // tokens past the range end (nvalid tokens in the tile) -> -inf
    // rs: the tile's row factors (load_factors)
    auto scale_scores = [&](f32x16_t& s, const float (&rs)[16], int nvalid) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] *= qf * rs[r];
      if (nvalid < kF8Tok) {
        int first = 32 * th + 4 * gq;
        asm volatile("" : "+v"(first));
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[r] = (first + 8 * (r >> 2) + (r & 3) < nvalid) ? s[r] : -INFINITY;
      }
    };
    // rs: the row factors scale_scores loaded for the same tile
    auto softmax_publish = [&](const f32x16_t& s, const float (&rs)[16], int& overflow, int k) {
      uint8_t* PB = smem + kF8POff + (k & 1) * kF8PBytes;
      uint8_t* SB = smem + kF8SOff + (k & 1) * 128;
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      m_seen = fmaxf(m_seen, mx);
      overflow |= (mx > m_ref + kRefSlack);
      float pp[16], pmax = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(s[r] - m_ref);  // v_exp_f32
        l_run += pr;
        pp[r] = pr * rs[r];  // the value product takes the raw codes
        pmax = fmaxf(pmax, pp[r]);
      }
      {  // head n over the wave's 32 tokens: v_permlane32_swap exchanges the
         // upper half of pa with the lower half of pb, leaving pa = the lower
         // half's value and pb = the upper half's in every lane (no LDS trip)
        float pa = pmax, pb = pmax;
        asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(pa), "+v"(pb));
        pmax = fmaxf(pa, pb);
      }
      // power-of-two factor 2^se putting the largest value in [128, 256)
      const int se = min(max(__builtin_amdgcn_frexp_expf(pmax) - 8, -127), 127);
      const float f = __builtin_ldexpf(1.0f, -se);
      float lu = 0.0f;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(pp[4 * s4] * f, pp[4 * s4 + 1] * f, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(pp[4 * s4 + 2] * f, pp[4 * s4 + 3] * f, w, true);
        // the weights as the value product sees them: code / f / row factor
        const f32x2_t c01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        const f32x2_t c23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        lu += c01[0] * __builtin_amdgcn_rcpf(rs[4 * s4]) + c01[1] * __builtin_amdgcn_rcpf(rs[4 * s4 + 1]) +
              c23[0] * __builtin_amdgcn_rcpf(rs[4 * s4 + 2]) + c23[1] * __builtin_amdgcn_rcpf(rs[4 * s4 + 3]);
        // tokens 8 s4 + 4 gq .. +3 of the half: lane n + 32 (s4 / 2) of the
        // B operand, bytes 8 (s4 % 2) + 4 gq
        *reinterpret_cast<int*>(PB + ((qhb * 2 + th) * 64 + n + 32 * (s4 >> 1)) * 16 + 8 * (s4 & 1) +
                                4 * gq) = w;
      }
      if (gq == 0) SB[(qhb * 2 + th) * 32 + n] = static_cast<uint8_t>(127 + se);
      l_used += __builtin_ldexpf(lu, se);
    };
    // per-head maximum over the two token halves
    auto agree_max = [&](float& m) {
      m = fmaxf(m, __shfl_xor(m, 32));
      if (active && gq == 0) xch[th * 64 + qhb * 32 + n] = m;
      barrier();  // AM
      if (active) m = fmaxf(m, xch[(th ^ 1) * 64 + qhb * 32 + n]);
      barrier();  // AM
    };

    barrier();  // T0: the first tile landed
    {
      auto nvalid = [&](int k) { return T1 - (T0 + k * kF8Tok); };
      m_ref = -INFINITY;
      m_seen = -INFINITY;
      for (int pass = 0; pass < 2; ++pass) {
        l_run = 0.0f;
        l_used = 0.0f;
        int overflow = 0;
        if (pass > 0) barrier();  // T0: the range's first tile loaded again
        f32x16_t s;
        float rs[16];
        if (active) {
          load_factors(rs, k0 & (kNBuf - 1));
          qk_tile(smem + (k0 & (kNBuf - 1)) * kTileBytes, s);
          scale_scores(s, rs, nvalid(k0));
        }
        if (pass == 0) {  // reference: maximum of the range's first tile
          float mx = -INFINITY;
          if (active) {
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
          }
          agree_max(mx);
          m_ref = mx;
        }
        if (active) softmax_publish(s, rs, overflow, k0);
        for (int k = k0; k < k1; ++k) {
          barrier();  // B_k: P'(k) published, tile k+1 landed
          if (active && k + 1 < k1) {
            const int buf = (k + 1) & (kNBuf - 1);
            load_factors(rs, buf);  // in flight during the products
            qk_tile(smem + buf * kTileBytes, s);
            scale_scores(s, rs, nvalid(k + 1));
            softmax_publish(s, rs, overflow, k + 1);
          }
        }
        const int vote = __any(overflow) ? 1 : 0;
        if (lane == 0) votes[wave] = vote;
        barrier();  // V1
        int again = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) again |= votes[w];
        barrier();  // V2
        if (!again) break;
        agree_max(m_seen);  // redo the range with the range maximum as reference
        m_ref = m_seen;
      }
      l_run += __shfl_xor(l_run, 32);
      l_used += __shfl_xor(l_used, 32);
      if (active && gq == 0) {
        xch[th * 64 + qhb * 32 + n] = l_run;
        xch[128 + th * 64 + qhb * 32 + n] = l_used;
      }
      barrier();  // E1
      if (active && th == 0 && gq == 0) {
        const int hx = qhb * 32 + n;
        const float l_tot = xch[hx] + xch[64 + hx];
        linv[hx] = 1.0f / (xch[128 + hx] + xch[192 + hx]);
        P.lse_part[row_base(p) + hx] = (m_ref + log2f(l_tot)) * kLn2;
      }
      barrier();  // E2
    }
    return;
  }

  // -------------------------------------------------------------- PV role
  // wave rw: latent columns 128 rw .. 128 rw + 127 (column blocks cb = 4 rw +
  // cbl of 32) of all 64 heads
  const int hl = lane & 31, g = lane >> 5;
  // transposing read rd (0..3) of column block cbl: this lane names the
  // 8-byte half (lane & 1) of chunk 2 cb + (lane / 16) % 2 of token
  // 32 (rd / 2) + 16 g + 8 (rd % 2) + (lane % 16) / 2; lane c of each 16 then
  // receives column c of the chunk for those 8 tokens.  A-operand byte 8 rd + k
  // of lane (c, g) is thus token 32 (rd / 2) + 16 g + 8 (rd % 2) + k: bytes
  // 0-15 are tokens 16 g .. 16 g + 15 of the first half, bytes 16-31 the same
  // of the second, the order in which the QK role writes P'.
  int trb[4][4];
#pragma unroll
  for (int rd = 0; rd < 4; ++rd)
#pragma unroll
    for (int cbl = 0; cbl < 4; ++cbl)
      trb[rd][cbl] = f8_chunk(32 * (rd >> 1) + 16 * g + 8 * (rd & 1) + ((lane & 15) >> 1),
                              2 * (4 * rw + cbl) + ((lane >> 4) & 1)) +
                     8 * (lane & 1);
  int one = 127;  // E8M0 1.0: the codes' own scale
  asm volatile("" : "+v"(one));
  f32x16_t acc[kH64Blocks * 4];

  auto zero_acc = [&] {
#pragma unroll
    for (int k = 0; k < kH64Blocks * 4; ++k) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[k][r] = 0.0f;
      asm volatile("" : "+a"(acc[k]));
    }
    asm volatile("s_nop 4");  // accumulator writes -> first (inline-asm) MFMA read
  };
  // U^T += V(k)^T P'(k): 8 block-scaled MFMAs; after_mfma(st) runs after MFMA st
  auto pv_tile = [&](int k, auto&& after_mfma) {
    const uint8_t* T = smem + (k & (kNBuf - 1)) * kTileBytes;
    const uint8_t* PB = smem + kF8POff + (k & 1) * kF8PBytes;
    const uint8_t* SB = smem + kF8SOff + (k & 1) * 128;
    i32x8_t av[4];
#pragma unroll
    for (int cbl = 0; cbl < 4; ++cbl)
#pragma unroll
      for (int rd = 0; rd < 4; ++rd) {
        const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(T + trb[rd][cbl]));
        av[cbl][2 * rd] = v[0];
        av[cbl][2 * rd + 1] = v[1];
      }
    i32x8_t pb[2];
    int sb[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(PB + ((hb * 2 + 0) * 64 + lane) * 16);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(PB + ((hb * 2 + 1) * 64 + lane) * 16);
      pb[hb] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      // the B scale of lane (n, g) is that of K block g: the 32 tokens of half g
      sb[hb] = SB[(hb * 2 + g) * 32 + hl];
    }
    // MFMA st: column block st / 2, head block st % 2.  Head blocks beyond
    // nhb multiply stale data into accumulators that are never stored.
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int cbl = st >> 1, hb = st & 1;
      asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
          : "+a"(acc[4 * hb + cbl])
          : "v"(av[cbl]), "v"(pb[hb]), "v"(one), "v"(sb[hb]));
      after_mfma(st);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const uint8_t* qsrc = static_cast<const uint8_t*>(P.q_abs) +
                        (static_cast<int64_t>(bj) * P.H + hbase) * kRowElems;
  struct TileDma {
    F8Dma rows;
    const float* scale;
    int nvalid;
  };
  // tile k of the workgroup: tokens T0 + 64 k .., all attended (T1 <= L)
  auto dma_plan = [&](int k) {
    const int tt = T0 + k * kF8Tok;
    const int64_t row0 = tile_row0(block_table, P.max_pages, P.seq_stride, P.paged != 0, b, tt);
    const int nvalid = min(kF8Tok, T1 - tt);
    TileDma d;
    d.rows = f8_dma_plan(P.rows + row0 * kRowElems,
                         lds_addr(smem) + (k & (kNBuf - 1)) * kTileBytes, nvalid, rw);
    d.scale = P.row_scale + row0;
    d.nvalid = nvalid;
    return d;
  };
  auto dma_factors = [&](const TileDma& d, int k) {
    f8_factor_issue(d.scale, lds_addr(rfac) + (k & (kNBuf - 1)) * kF8Tok * 4, d.nvalid, rw, lane);
  };
  auto dma = [&](int k) {
    const TileDma d = dma_plan(k);
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) f8_dma_issue(d.rows, i);
    dma_factors(d, k);
  };
  // wait until tile k has landed, when tiles up to min(k + 2, K - 1) were
  // issued (and nothing after them)
  auto wait_tile = [&](int k) {
    const int later = min(K - 1, k + 2) - k;  // 0, 1 or 2 tiles issued after k
    if (later >= 2)
      asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // queries (one tile buffer: 64 heads x 576 codes), then tiles 0-2
  {
    const F8Dma dq = f8_dma_plan(qsrc, lds_addr(smem) + 3 * kTileBytes, nhb * kHeadsPerWave, rw);
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) f8_dma_issue(dq, i);
  }
  dma(0);
  if (K > 1) dma(1);
  wait_tile(0);  // at least the queries (issued first) have landed
  barrier();  // Q1
  barrier();  // Q2: buffer 3 free
  if (K > 2) dma(2);
  wait_tile(0);
  barrier();  // T0

  {
    for (int pass = 0; pass < 2; ++pass) {
      zero_acc();
      if (pass > 0) {  // the range again: its first tiles back into the buffers
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        dma(k0);
        if (k0 + 1 < K) dma(k0 + 1);
        if (k0 + 2 < K) dma(k0 + 2);
        wait_tile(k0);
        barrier();  // T0
      } else {
        barrier();  // AM
        barrier();  // AM
      }
      for (int k = k0; k < k1; ++k) {
        // tiles up to min(k + 2, K - 1) are issued: tile k + 1 lands
        if (k + 2 < K)
          asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier();  // B_k
        // tile k+3 into tile k-1's buffer: one row line after each MFMA, the
        // last line and the row factors after the last
        const bool dnext = k + 3 < K;  // workgroup-uniform
        TileDma dp{};
        if (dnext) dp = dma_plan(k + 3);
        pv_tile(k, [&](int st) {
          if (dnext) {
            f8_dma_issue(dp.rows, st);
            if (st == 7) {
              f8_dma_issue(dp.rows, 8);
              dma_factors(dp, k + 3);
            }
          }
        });
      }
      if (lane == 0) votes[wave] = 0;
      barrier();  // V1
      int again = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) again |= votes[w];
      barrier();  // V2
      if (!again) break;
      barrier();  // AM
      barrier();  // AM
    }
    barrier();  // E1
    barrier();  // E2: linv ready
    // matrix-core accumulator writes -> VALU reads
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
    // U^T register r of block (hb, cbl) in lane (hl, g) is column
    // 128 rw + 32 cbl + 8 (r / 4) + 4 g + r % 4 of head hbase + 32 hb + hl;
    // each wave stages one head block (32 rows x 128 columns) at a time in its
    // own region of the range's last tile buffer (free: no tile is loaded
    // after it) and writes 256 contiguous bytes per row.
    constexpr int kEsz = PART_DT == MLA_F32 ? 4 : 2;
    constexpr int kColsRound = 256 / kEsz;
    constexpr int kStageRow = kColsRound * kEsz + 16;
    // the lane index recomputed here (volatile), so that the epilogue's
    // addresses are formed in place rather than held across the tile loop
    int eln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(eln));
    const int hl = eln & 31, g = eln >> 5;
    uint8_t* W = smem + ((k1 - 1) & (kNBuf - 1)) * kTileBytes + rw * kHeadsPerWave * kStageRow;
#pragma unroll
    for (int hb = 0; hb < kH64Blocks; ++hb) {
      if (hb < nhb) {
        const float inv = linv[hb * kHeadsPerWave + hl];
#pragma unroll
        for (int half = 0; half < 128 / kColsRound; ++half) {
#pragma unroll
          for (int cbl2 = 0; cbl2 < kColsRound / 32; ++cbl2) {
            const int cbl = half * (kColsRound / 32) + cbl2;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int c = 32 * cbl2 + 8 * r4 + 4 * g;
              const f32x16_t& A = acc[4 * hb + cbl];
              const float v0 = A[4 * r4 + 0] * inv, v1 = A[4 * r4 + 1] * inv;
              const float v2 = A[4 * r4 + 2] * inv, v3 = A[4 * r4 + 3] * inv;
              uint8_t* wp = W + hl * kStageRow + c * kEsz;
              if constexpr (PART_DT == MLA_F32) {
                *reinterpret_cast<f32x4_t*>(wp) = f32x4_t{v0, v1, v2, v3};
              } else {
                *reinterpret_cast<u32x2_t*>(wp) = u32x2_t{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
              }
            }
          }
          asm volatile("" ::: "memory");
          uint8_t* dst = static_cast<uint8_t*>(P.u_part) +
                         ((row_base(p) + hb * kHeadsPerWave) * kDLatent + 128 * rw) * kEsz +
                         half * (kColsRound * kEsz);
#pragma unroll
          for (int i = 0; i < kHeadsPerWave / 4; ++i) {
            const int row = 4 * i + (eln >> 4);
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(W + row * kStageRow + (eln & 15) * 16);
            *reinterpret_cast<u32x4_t*>(dst + static_cast<int64_t>(row) * (kDLatent * kEsz) +
                                        (eln & 15) * 16) = v;
          }
          asm volatile("" ::: "memory");
        }
      }
    }
  }
}

}  // namespace

mla_status_t decode_fp8q_launch(const DecodeParams& P0, int32_t part_dt, hipStream_t s) {
  // R consecutive split ranges per workgroup (enough workgroups to fill the
  // 256 CUs once), merged into one range: the workgroup streams their tokens
  // with one softmax and writes one partial, to slot g of its group g; slots
  // from ceil(S / R) on hold lse = -inf
  const int64_t units = static_cast<int64_t>(P0.B) * P0.QL * P0.S * P0.HG;
  const int64_t per_cu = units / 256;
  const int R = static_cast<int>(per_cu < 1 ? 1 : (per_cu > P0.S ? P0.S : per_cu));
  DecodeParams P = P0;
  P.S = (P0.S + R - 1) / R;
  P.chunk = P0.chunk * R;
  P.S_out = P0.S;
  const int64_t nblk = static_cast<int64_t>(P.B) * P.QL * P.S * P.HG;
  if (nblk > 0x7FFFFFFF) return MLA_E_SHAPE;
  const unsigned grid = static_cast<unsigned>(nblk);
  if (part_dt == MLA_F32)
    decode_f8q_kernel<MLA_F32><<<grid, kF8Threads, 0, s>>>(P, P.block_table);
  else
    decode_f8q_kernel<MLA_BF16><<<grid, kF8Threads, 0, s>>>(P, P.block_table);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_E_HIP;
}

}  // namespace mla
