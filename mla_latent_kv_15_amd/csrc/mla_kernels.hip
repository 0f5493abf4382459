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
#include <cmath>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "../../include/mla.h"
#include "mla_decode_tile.h"
#include "mla_device.h"
#include "mla_host.h"

namespace mla {
namespace {

// ================================================================ decode (MFMA)
//
// The bf16 and fp8 cache paths share one kernel design: one workgroup per
// (sequence b, split range p, group of up to 64 heads).  Per 32-token tile:
//   * the 32 cached rows are staged once in LDS as bf16 and shared by all
//     heads of the workgroup.  bf16 rows travel HBM -> LDS directly
//     (global_load_lds_dwordx4, no VGPR staging); fp8 rows pass through
//     registers and are widened exactly to bf16 on their way in;
//   * QK:  S[t][h] = sum_k tile[t][k] q_abs[h][k] on the matrix cores, the
//     absorbed queries held in registers for the whole range;
//   * a softmax with one reference maximum per head and range (below), in
//     the base-2 domain;
//   * PV:  Uᵀ[c][h] += sum_t tile[t][c] P[t][h] on the matrix cores, the
//     latent read from the same LDS tile with transposing reads.
// Tokens past the end of the range are loaded from the tile's first row
// (finite data; their probability is zero).

// ================================================================ decode (warp-specialised)
//
// One workgroup per (sequence b, split range p, 64 heads), 8 waves, two per
// SIMD, in two roles:
//   * QK waves 0..3 (head block w & 1, token half w >> 1) hold their absorbed
//     queries in AGPRs, compute the scores of tile i+1 with
//     v_mfma_f32_16x16x32_bf16, run the softmax and publish the bf16
//     probabilities;
//   * PV waves 4..7 (latent columns 128(w-4)..+127 of all 64 heads) stream the
//     tiles into LDS and accumulate U^T of tile i in AGPRs with
//     v_mfma_f32_32x32x16_bf16.
// Each SIMD runs one wave of each role, so the matrix core alternates between
// the two while the other role waits on LDS or runs the softmax.  The roles
// meet at one barrier per tile; their register footprints (queries vs
// accumulators) share the same AGPRs because each role's code is a separate
// region of the kernel.
//
// fp8 caches (FP8 = true): the PV waves load the codes of tile i+4 into
// registers while the MFMAs of tile i run, and widen tile i+2 (loaded two
// tiles earlier) into the same bf16 layout; the row scales go to a small LDS
// array.  The scores are multiplied by the row scales after the QK product,
// and the published probabilities carry them into the PV product.

constexpr int kWsThreads = 512;
constexpr int kBalancedWorkgroups = 256;  // one 64-head workgroup per CU
constexpr int kBalancedMaxRows = kWsThreads;  // the plan takes one row per thread
constexpr int kRowStartTiles = 5;  // a piece's start, in tiles of streaming (measured ~4.5 us)
constexpr int kWalkOff = kX64Off + 1536;  // the balanced piece list, after the exchange area

// fp8 rows in flight in a PV wave's registers: lane (k = lane / 8, j = lane % 8)
// of PV wave w holds, for i = 0..8, the 8 codes of bf16 chunk 8 i + (j ^ swzg(t))
// of row t = 8 w + k (the chunk that the token-group layout puts at slot j of
// line (i, t)), and that row's scale
struct Fp8Rows {
  u32x2_t w[kDmaPerWave];
  float sc;
};

template <bool FP8, int PART_DT, bool BAL = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kWsThreads, kWsThreads),
                          amdgpu_waves_per_eu(2, 2)))
void decode_ws_kernel(DecodeParams P, const int32_t* __restrict__ block_table) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kWalkOff + (FP8 || !BAL ? 0 : 12 * kBalancedMaxRows)];
  uint8_t* pbuf = smem + kNBuf * kTileBytes;
  float* xch = reinterpret_cast<float*>(smem + kX64Off);  // [2][64] per-head exchange
  int* votes = reinterpret_cast<int*>(smem + kX64Off + 512);
  float* linv = reinterpret_cast<float*>(smem + kX64Off + 768);  // epilogue: 1 / l per head
  float* tscale = reinterpret_cast<float*>(smem + kX64Off + 1024);  // fp8: [kNBuf][32] row scales

  // Work id -> head group hg (adjacent work ids, same XCD, share each tile
  // through L2) and r1: in the fixed partition (query token j, split range p,
  // sequence b; consecutive ranges that the host merged count as one); in the
  // balanced one the worker.
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int hg = wid % P.HG;
  const int r1 = wid / P.HG;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const bool is_qk = wave < 4;                                // wave-uniform
  const int rw = wave & 3;                                    // index within the role
  const int hbase = hg * kH64;
  const int nhb = min(kH64Blocks, (P.H - hbase) / kHeadsPerWave);  // 1 or 2
  auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  // first partial row of split p of row bj = b * QL + qj of q_abs / u_part
  auto row_base = [&](int bj, int p) { return (static_cast<int64_t>(bj) * P.S_out + p) * P.H + hbase; };
  // a split without tokens (PV waves): lse = -inf, and u = 0 unless
  // lse_only (a slot past merged range groups, an empty split of the balanced
  // partition: mla_combine does not read the u of a split with lse = -inf)
  auto write_empty = [&](int bj, int p, bool lse_only = false) {
    if (is_qk) return;
    constexpr int kEsz = PART_DT == MLA_F32 ? 4 : 2;
    const int64_t rb = row_base(bj, p);
    const int pt = tid - 256;
    if (!lse_only) {  // the split's rows of this head group are contiguous: 16-byte stores
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(P.u_part) + rb * kDLatent * kEsz);
      for (int i = pt; i < nhb * kHeadsPerWave * kDLatent * kEsz / 16; i += 256)
        dst[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
    if (pt < nhb * kHeadsPerWave) P.lse_part[rb + pt] = -INFINITY;
  };
  // tokens attended by row v = b * QL + qj: query token qj of QL new tokens
  // (the last QL cached rows) sees the cached rows up to and including its
  // own, the first L - (QL - 1 - qj)
  auto attended = [&](int v) {
    const int b = v / P.QL, qj = v - (v / P.QL) * P.QL;
    return max(attended_len(P.seq_lens, b, P.max_seq_len, P.ring, P.seq_stride) - (P.QL - 1 - qj), 0);
  };

  // One unit of work: split p of row bj, tokens [T0, T1) of its attended ones
  // as K consecutive 32-token tiles (a range the host merged from several
  // split ranges is one range here).
  auto unit = [&](const int bj, const int p, const int T0, const int T1, const int lane,
                  const int tid) {
  const int b = bj / P.QL;
  const int K = T1 > T0 ? (T1 - T0 + kTileTokens - 1) / kTileTokens : 0;
  if (K == 0) {
    write_empty(bj, p);
    return;
  }
  // fp8: the PV loop runs in pairs of tiles (one register set each), so an
  // odd range gets one more tile: it is loaded from the range's first rows
  // and all of its tokens are masked, which adds exact zeros
  const int ntp = FP8 ? ((K + 1) & ~1) : K;
  const int k1 = ntp;  // the range's tiles 0 .. k1 - 1

  // all s_barriers below are issued by both roles in the same order:
  //   Q1 Q2 T0 | [pass 0: AM AM] B_0..B_k1-1 V1 V2
  //   [redo: AM AM T0 B_0..B_k1-1 V1 V2] E1 E2

  if (is_qk) {
    // ------------------------------------------------------------ QK role
    const int qhb = rw & 1, th = rw >> 1;
    const bool active = qhb < nhb;  // wave-uniform
    const int n16 = lane & 15, kg = lane >> 4;
    const int qk_row = ((n16 >> 3) * kTokGroupBytes) + (n16 & 7) * 128;
    const int qk_key = swzg(n16);  // row n16 % 8 of group n16 / 8 of a 16-row half
    const int qk_off[2] = {(kg ^ qk_key) << 4, ((4 + kg) ^ qk_key) << 4};
    auto qk_addr = [&](int half, int ks) {
      return 2 * half * kTokGroupBytes + qk_row + qk_off[ks & 1] + (ks >> 1) * 1024;
    };
    float m_ref[2] = {-INFINITY, -INFINITY}, m_seen[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.0f, 0.0f};
    // B operands: k-steps < kQkAgpr in AGPRs (the PV role's accumulators use
    // the same 128 AGPRs), the rest in VGPRs; the fp8 cache's row scales take
    // VGPRs, so that variant moves two more k-steps to AGPRs
    constexpr int kQkAgpr = FP8 ? 16 : 14;
    bf16x8_t qa[kQkAgpr][2];
    bf16x8_t qv[kQkSteps - kQkAgpr][2];

    barrier();  // Q1: the queries are staged in tile buffers 2 and 3
    if (active) {
      const uint8_t* Q = smem + (2 + qhb) * kTileBytes;
#pragma unroll
      for (int ks = 0; ks < kQkSteps; ++ks)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          if (ks < kQkAgpr) {
            qa[ks][hh] = *reinterpret_cast<const bf16x8_t*>(Q + qk_addr(hh, ks));
            asm volatile("" : "+a"(qa[ks][hh]));
          } else {
            qv[ks - kQkAgpr][hh] = *reinterpret_cast<const bf16x8_t*>(Q + qk_addr(hh, ks));
            asm volatile("" : "+v"(qv[ks - kQkAgpr][hh]));
          }
        }
    }
    barrier();  // Q2: staging buffers free

    constexpr int kRing = 6;
    auto qk_tile = [&](const uint8_t* T, f32x4_t (&s)[2]) {
      bf16x8_t ring[kRing];
#pragma unroll
      for (int k = 0; k < kRing; ++k) ring[k] = *reinterpret_cast<const bf16x8_t*>(T + qk_addr(th, k));
#pragma unroll
      for (int ks = 0; ks < kQkSteps; ++ks) {
        const bf16x8_t a = ring[ks % kRing];
        if (ks + kRing < kQkSteps)
          ring[ks % kRing] = *reinterpret_cast<const bf16x8_t*>(T + qk_addr(th, ks + kRing));
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          if (ks == 0)
            asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(s[hh]) : "v"(a), "a"(qa[ks][hh]));
          else if (ks < kQkAgpr)
            asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(s[hh]) : "v"(a), "a"(qa[ks][hh]));
          else
            asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                : "+v"(s[hh]) : "v"(a), "v"(qv[ks - kQkAgpr][hh]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
    };
    // fp8: scores of the raw codes times the row scales of tokens
    // 16 th + 4 kg + r; returns the scales for the probabilities
    auto row_scale = [&](f32x4_t (&s)[2], int buf) {
      const f32x4_t sc = *reinterpret_cast<const f32x4_t*>(tscale + buf * kTileTokens + 16 * th + 4 * kg);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[hh][r] *= sc[r];
      return sc;
    };
    auto softmax_publish = [&](f32x4_t (&s)[2], const f32x4_t& sc, int nvalid, int& overflow,
                               uint8_t* PB) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[hh][r] *= P.scale_log2;
      if (nvalid < kTileTokens) {  // partial last tile: token 16 th + 4 kg + r present?
        int first = 16 * th + 4 * kg;
        asm volatile("" : "+v"(first));
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[hh][r] = (first + r < nvalid) ? s[hh][r] : -INFINITY;
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float mx = fmaxf(fmaxf(s[hh][0], s[hh][1]), fmaxf(s[hh][2], s[hh][3]));
        m_seen[hh] = fmaxf(m_seen[hh], mx);
        overflow |= (mx > m_ref[hh] + kRefSlack);
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = __builtin_amdgcn_exp2f(s[hh][r] - m_ref[hh]);  // v_exp_f32
          l_run[hh] += pr[r];
        }
        // fp8: the PV product takes the raw codes, so the probability carries
        // the row scale (the sum l does not)
        if constexpr (FP8) {
#pragma unroll
          for (int r = 0; r < 4; ++r) pr[r] *= sc[r];
        }
        // B-operand slot of token 16th + 4kg + r: k-step th, lane group kg & 1,
        // slots 4 (kg >> 1) + r of head 32 qhb + 16 hh + n16
        *reinterpret_cast<u32x2_t*>(PB + (((th * 2 + qhb) * 2 + (kg & 1)) * 32 + 16 * hh + n16) * 16 +
                                    8 * (kg >> 1)) =
            u32x2_t{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
      }
    };
    // per-head maximum over the lane groups and the two token halves
    auto agree_max = [&](float (&m)[2]) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        m[hh] = fmaxf(m[hh], __shfl_xor(m[hh], 16));
        m[hh] = fmaxf(m[hh], __shfl_xor(m[hh], 32));
      }
      if (active && kg == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) xch[th * 64 + qhb * 32 + 16 * hh + n16] = m[hh];
      }
      barrier();  // AM
      if (active) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          m[hh] = fmaxf(m[hh], xch[(th ^ 1) * 64 + qhb * 32 + 16 * hh + n16]);
      }
      barrier();  // AM
    };

    barrier();  // T0: the first tile landed
    {
      const int k0 = 0;
      auto nvalid = [&](int k) { return T1 - (T0 + k * kTileTokens); };
      m_ref[0] = m_ref[1] = m_seen[0] = m_seen[1] = -INFINITY;
      for (int pass = 0; pass < 2; ++pass) {
        l_run[0] = l_run[1] = 0.0f;
        int overflow = 0;
        if (pass > 0) barrier();  // T0: the range's first tiles loaded again
        f32x4_t s[2];
        f32x4_t sc = {1.0f, 1.0f, 1.0f, 1.0f};
        const int buf0 = k0 & (kNBuf - 1);
        if (active) {
          qk_tile(smem + buf0 * kTileBytes, s);
          if constexpr (FP8) sc = row_scale(s, buf0);
        }
        if (pass == 0) {  // reference: maximum of the range's first tile
          float mx[2] = {-INFINITY, -INFINITY};
          if (active) {
            const int nv = nvalid(k0);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (16 * th + 4 * kg + r < nv) mx[hh] = fmaxf(mx[hh], s[hh][r] * P.scale_log2);
          }
          agree_max(mx);
          m_ref[0] = mx[0];
          m_ref[1] = mx[1];
        }
        if (active) softmax_publish(s, sc, nvalid(k0), overflow, pbuf + (k0 & 1) * kP64Bytes);
        for (int k = k0; k < k1; ++k) {
          barrier();  // B_k: P(k) published, tile k+1 landed
          if (active && k + 1 < k1) {
            const int buf = (k + 1) & (kNBuf - 1);
            qk_tile(smem + buf * kTileBytes, s);
            if constexpr (FP8) sc = row_scale(s, buf);
            softmax_publish(s, sc, nvalid(k + 1), overflow, pbuf + ((k + 1) & 1) * kP64Bytes);
          }
        }
        // the vote over all lanes, taken before the branch that stores it
        // (inside `lane == 0` it would see lane 0's flag only)
        const int vote = __any(overflow) ? 1 : 0;
        if (lane == 0) votes[wave] = vote;
        barrier();  // V1
        int again = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) again |= votes[w];
        barrier();  // V2
        if (!again) break;
        agree_max(m_seen);  // redo the range with the range maximum as reference
        m_ref[0] = m_seen[0];
        m_ref[1] = m_seen[1];
      }
      // l per head: lane groups, then the two token halves
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        l_run[hh] += __shfl_xor(l_run[hh], 16);
        l_run[hh] += __shfl_xor(l_run[hh], 32);
      }
      if (active && kg == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) xch[th * 64 + qhb * 32 + 16 * hh + n16] = l_run[hh];
      }
      barrier();  // E1
      if (active && th == 0 && kg == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int hx = qhb * 32 + 16 * hh + n16;
          const float l_tot = xch[hx] + xch[64 + hx];
          linv[hx] = 1.0f / l_tot;
          P.lse_part[row_base(bj, p) + hx] = (m_ref[hh] + log2f(l_tot)) * kLn2;
        }
      }
      barrier();  // E2
    }
    return;
  }

  // -------------------------------------------------------------- PV role
  const int G = lane >> 4, e = (lane >> 2) & 3, q4 = lane & 3;
  const int tr_row = 4 * (G >> 1) + e;
  const int tr_key = swzg(tr_row);
  const int tr_x = 2 * (G & 1) + (q4 >> 1);
  const int tr_byte = 8 * (q4 & 1);
  const int tr_off[2] = {((0 + tr_x) ^ tr_key) << 4, ((4 + tr_x) ^ tr_key) << 4};
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
  // Uᵀ += tile i ⋅ P(i): 16 MFMAs; after_mfma(st) runs after MFMA st (the
  // staging of a later tile is spread between them)
  auto pv_tile = [&](int i, auto&& after_mfma) {
    const uint8_t* T = smem + (i & (kNBuf - 1)) * kTileBytes;
    const uint8_t* PB = pbuf + (i & 1) * kP64Bytes;
    const uint8_t* r0 = T + tr_row * 128 + tr_byte;
    auto load_av = [&](int cbl, int j) {
      const int cb = 4 * rw + cbl;
      const uint8_t* ptr = r0 + tr_off[cb & 1] + (cb >> 1) * 1024 + 2 * j * kTokGroupBytes;
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)ptr);
      const bf16x4_t hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(ptr + kTokGroupBytes));
      return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    bf16x8_t pb[2][2];  // [token half j][head block]
    bf16x8_t av[4][2];  // [column block][token half j]
#pragma unroll
    for (int cbl = 0; cbl < 4; ++cbl) {
      av[cbl][0] = load_av(cbl, 0);
      av[cbl][1] = load_av(cbl, 1);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        pb[j][hb] = *reinterpret_cast<const bf16x8_t*>(PB + ((j * 2 + hb) * 64 + lane) * 16);
    // MFMA st: column block st / 4, token half (st / 2) % 2, head block st % 2.
    // Head blocks beyond nhb multiply stale probabilities into accumulators
    // that are never stored.
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int cbl = st >> 2, j = (st >> 1) & 1, hb = st & 1;
      asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
          : "+a"(acc[4 * hb + cbl]) : "v"(av[cbl][j]), "v"(pb[j][hb]));
      after_mfma(st);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // the partial of one range: U^T / l, staged per wave (32 rows x 128
  // columns) in `stage` (a tile buffer no DMA is writing) and written as 256
  // contiguous bytes per row at rows rb + head
  auto write_partial = [&](int64_t rb, uint8_t* stage) {
    // matrix-core accumulator writes -> VALU reads (the MFMAs are inline asm)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
    // U^T register r of block (hb, cbl) in lane (hl, g) is column
    // 128*rw + 32*cbl + 8*(r/4) + 4*g + r%4 of head hbase + 32*hb + hl.  Each
    // wave stages one head block (32 rows x 128 columns) at a time in its own
    // region of `stage` and writes 256 contiguous bytes per row.
    constexpr int kEsz = PART_DT == MLA_F32 ? 4 : 2;
    constexpr int kColsRound = 256 / kEsz;             // 128 bf16 / 64 fp32 columns
    constexpr int kStageRow = kColsRound * kEsz + 16;  // padded: rows start 4 banks apart
    // the lane index recomputed here (volatile), so that the epilogue's
    // addresses are formed in place rather than held across the tile loop
    int eln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(eln));
    const int hl = eln & 31, g = eln >> 5;
    uint8_t* W = stage + rw * kHeadsPerWave * kStageRow;
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
          // one wave's LDS operations complete in order: no barrier is needed
          asm volatile("" ::: "memory");
          // 32 rows x 256 bytes: 4 rows per wave instruction, 16 bytes per lane
          uint8_t* dst = static_cast<uint8_t*>(P.u_part) +
                         ((rb + hb * kHeadsPerWave) * kDLatent + 128 * rw) * kEsz +
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
  };

  // the queries of both head blocks (32 rows each) go into tile buffers 2 and 3
  const uint8_t* qsrc = static_cast<const uint8_t*>(P.q_abs) +
                        (static_cast<int64_t>(bj) * P.H + hbase) * kRowBytes;
  auto stage_q = [&] {
    for (int hb = 0; hb < nhb; ++hb)
      rows_dma_g8(qsrc + hb * kHeadsPerWave * kRowBytes, lds_addr(smem) + (2 + hb) * kTileBytes,
                  kTileTokens, rw);
  };

  if constexpr (!FP8) {
    // tile k of the workgroup: tokens T0 + 32 k .., all attended (T1 is at most the row's length)
    auto dma_plan = [&](int k) {
      const int tt = T0 + k * kTileTokens;
      const int64_t row0 = tile_row0(block_table, P.max_pages, P.seq_stride, P.paged != 0, b, tt);
      return rows_dma_plan(P.rows + row0 * kRowBytes, lds_addr(smem) + (k & (kNBuf - 1)) * kTileBytes,
                           min(kTileTokens, T1 - tt), rw);
    };
    auto dma = [&](int k) {
      const RowsDma d = dma_plan(k);
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) rows_dma_issue(d, i);
    };
    // wait until tile k has landed, when tiles up to min(k + 2, K - 1) were
    // issued (and nothing after them)
    auto wait_tile = [&](int k) {
      const int later = min(K - 1, k + 2) - k;
      if (later >= 2)
        asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
      else if (later == 1)
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    // queries, then tiles 0 and 1 (tile 2 once the staging buffers are free)
    stage_q();
    dma(0);
    if (K > 1) dma(1);
    if (K > 1)
      asm volatile("s_waitcnt vmcnt(18)" ::: "memory");  // the queries landed
    else
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    barrier();  // Q1
    barrier();  // Q2
    if (K > 2) dma(2);
    wait_tile(0);
    barrier();  // T0

    {
      const int k0 = 0;
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
            asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
          else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          barrier();  // B_k
          // tile k+3 into tile k-1's buffer, one wave instruction per MFMA
          const bool dnext = k + 3 < K;  // workgroup-uniform
          RowsDma dp{};
          if (dnext) dp = dma_plan(k + 3);
          pv_tile(k, [&](int st) {
            if (dnext && st < kDmaPerWave) rows_dma_issue(dp, st);
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
      // the range's last tile buffer: no tile is loaded after it
      write_partial(row_base(bj, p), smem + ((k1 - 1) & (kNBuf - 1)) * kTileBytes);
    }
  } else {
    // one range per workgroup
    const int t_begin = T0, t_end = T1, ntiles = K;
    // fp8 rows travel through registers: tile k is loaded two tiles ahead of
    // its conversion, into register set k % 2, and widened to bf16 on its way
    // into the same token-group layout as the bf16 path
    auto f8_load = [&](Fp8Rows& S, int tile) {
      // tiles past the range (the padding tile, and the loads issued ahead of
      // the last iterations, whose registers are never read) read the last
      // tile again: every wave then issues the same loads in every iteration,
      // which keeps the compiler's wait counts exact
      const int tc = min(tile, ntiles - 1);
      const int tt = t_begin + tc * kTileTokens;
      const int64_t row0 = tile_row0(block_table, P.max_pages, P.seq_stride, P.paged != 0, b, tt);
      const int nvalid = min(kTileTokens, t_end - tt);
      int ln;  // volatile: recomputed per call rather than kept live across the loop
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const int t = 8 * rw + (ln >> 3);
      const int tr = t < nvalid ? t : 0;  // rows past the end: the tile's first row
      const uint8_t* base = P.rows + row0 * kRowElems;  // wave-uniform
      const uint32_t off = static_cast<uint32_t>(tr * kRowElems + ((ln & 7) ^ swzg(t)) * 8);
      S.sc = (P.row_scale + row0)[tr];
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i)
        S.w[i] = *reinterpret_cast<const u32x2_t*>(base + off + 64 * i);
    };
    auto f8_store_chunk = [&](const Fp8Rows& S, int buf, int i) {
      uint8_t* T = smem + buf * kTileBytes + rw * kTokGroupBytes + 1024 * i + lane * 16;
      const u32x2_t lo = e4m3x4_to_bf16x4(S.w[i].x), hi = e4m3x4_to_bf16x4(S.w[i].y);
      *reinterpret_cast<u32x4_t*>(T) = u32x4_t{lo.x, lo.y, hi.x, hi.y};
    };
    auto f8_store_scale = [&](const Fp8Rows& S, int buf) {
      if ((lane & 7) == 0) tscale[buf * kTileTokens + 8 * rw + (lane >> 3)] = S.sc;
    };
    auto f8_store = [&](const Fp8Rows& S, int buf) {
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) f8_store_chunk(S, buf, i);
      f8_store_scale(S, buf);
    };
    // iteration i: Uᵀ of tile i, tile i+2 from set S into LDS, then tile i+4
    // into S.  With a set in flight for each of the next two tiles, the
    // compiler's waits before each conversion leave the other set's loads
    // outstanding.
    auto f8_iter = [&](int i, Fp8Rows& S) {
      barrier();  // B_i
      const bool conv = i + 2 < ntp;  // workgroup-uniform
      const int cb = (i + 2) & (kNBuf - 1);
      pv_tile(i, [&](int st) {
        if (conv && st == 0) f8_store_scale(S, cb);
        if (conv && st < kDmaPerWave) f8_store_chunk(S, cb, st);
        if (st == kDmaPerWave + 1) f8_load(S, i + 4);
      });
    };

    Fp8Rows A, B;
    stage_q();
    f8_load(A, 0);
    f8_load(B, 1);
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");  // queries (and tile 0) landed
    barrier();  // Q1
    barrier();  // Q2

    for (int pass = 0; pass < 2; ++pass) {
      zero_acc();
      if (pass > 0) {
        f8_load(A, 0);
        f8_load(B, 1);
      }
      f8_store(A, 0);
      f8_load(A, 2);
      barrier();  // T0
      if (pass == 0) {
        barrier();  // AM
        barrier();  // AM
      }
      f8_store(B, 1);
      f8_load(B, 3);
      for (int i = 0; i < ntp; i += 2) {
        f8_iter(i, A);
        f8_iter(i + 1, B);
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
    write_partial(row_base(bj, p), smem);  // no tile is in flight in LDS
  }
  };  // unit

  // Balanced partition (bf16 cache): the rows laid end to end, row v weighing
  // kRowStartTiles + n_v (n_v = ceil(L_v / 32) tiles; 0 for an empty row), its
  // tiles after its start weight, N in all, are cut into G equal spans
  // [w N / G, (w + 1) N / G), worker w taking span w; G = min(workers
  // launched, N / ceil(n_max / (S - 1))) with n_max the largest row weight, so
  // no row meets more than S spans.  The piece of row v in span w is its
  // split w - (the span of v's first tile); splits after v's last piece, and
  // every split of an empty row, are written empty by the worker whose span
  // holds v's last tile (the span of v's position, the last span if none).
  constexpr bool balanced = !FP8 && BAL;
  // the worker's pieces (balanced): kBalancedMaxRows entries of (row |
  // split << 16, first token, end token), kept in LDS for the whole kernel
  int* plist = reinterpret_cast<int*>(smem + kWalkOff);
  int npieces = 1;
  if constexpr (balanced) {
    // thread t plans row t (B * QL <= 512, checked on the host)
    const int V = P.B * P.QL;
    const int A = tid < V ? attended(tid) : 0;
    const int n = (A + kTileTokens - 1) / kTileTokens;
    // a row's weight: its tiles plus kRowStartTiles for the start of a piece
    // (query staging, the first tiles' latency), so that spans holding more
    // row starts take fewer tiles
    const int nw = n > 0 ? n + kRowStartTiles : 0;
    int* red = reinterpret_cast<int*>(pbuf);  // P buffers: free until the first piece
    auto wave_scan = [&](int x) {  // inclusive prefix over the wave's lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(x, d);
        if (lane >= d) x += t;
      }
      return x;
    };
    // weight before row t (pre), all weight (N), the largest row weight (n_max)
    const int incl = wave_scan(nw);
    int mx = nw;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mx = max(mx, __shfl_xor(mx, d));
    if (lane == 63) red[wave] = incl;
    if (lane == 0) red[8 + wave] = mx;
    barrier();
    int pre = incl - nw, N = 0, nmax = 0;
#pragma unroll
    for (int w2 = 0; w2 < 8; ++w2) {
      const int t = red[w2];
      pre += w2 < wave ? t : 0;
      N += t;
      nmax = max(nmax, red[8 + w2]);
    }
    N = __builtin_amdgcn_readfirstlane(N);
    nmax = __builtin_amdgcn_readfirstlane(nmax);
    const int G_launch = static_cast<int>(gridDim.x) / P.HG;
    const int G = N > 0 ? min(G_launch, max(1, N / ((nmax + P.S - 2) / (P.S - 1)))) : 1;
    if (r1 >= G) return;  // more workers launched than the spans need
    const int lo = static_cast<int>(static_cast<int64_t>(r1) * N / G);
    const int hi = static_cast<int>(static_cast<int64_t>(r1 + 1) * N / G);
    // row t's tiles sit at [f0, f0 + n) after its start weight; its piece in
    // this span (its split: this span minus the span of its first tile), and
    // the empty splits this worker writes for row t
    const int f0 = pre + (n > 0 ? kRowStartTiles : 0);
    bool piece = tid < V && n > 0 && f0 < hi && f0 + n > lo;
    int slot = 0, first_empty = P.S;
    if (piece) {
      slot = r1 - min(G - 1, static_cast<int>((static_cast<int64_t>(f0 + 1) * G - 1) / N));
      piece = slot < P.S;  // always (G bounds the spans a row meets); keeps writes in bounds
      if (f0 + n <= hi) first_empty = slot + 1;  // the row ends in this span
    } else if (tid < V && n == 0 && ((pre >= lo && pre < hi) || (r1 == G - 1 && pre == N))) {
      first_empty = 0;  // an empty row at this span's position
    }
    const bool job = first_empty < P.S;
    // list positions: pieces and empty-split jobs in row order
    const int pin = wave_scan(piece ? 1 : 0), jin = wave_scan(job ? 1 : 0);
    if (lane == 63) {
      red[16 + wave] = pin;
      red[24 + wave] = jin;
    }
    barrier();
    int pidx = pin - (piece ? 1 : 0), jidx = jin - (job ? 1 : 0), np = 0, nj = 0;
#pragma unroll
    for (int w2 = 0; w2 < 8; ++w2) {
      const int tp = red[16 + w2], tj = red[24 + w2];
      pidx += w2 < wave ? tp : 0;
      jidx += w2 < wave ? tj : 0;
      np += tp;
      nj += tj;
    }
    int* jobs = red + 64;  // (row, first empty split)
    if (piece) {
      plist[3 * pidx + 0] = tid | (slot << 16);
      plist[3 * pidx + 1] = kTileTokens * (max(lo, f0) - f0);
      plist[3 * pidx + 2] = min(kTileTokens * (min(hi, f0 + n) - f0), A);
    }
    if (job) {
      jobs[2 * jidx + 0] = tid;
      jobs[2 * jidx + 1] = first_empty;
    }
    barrier();
    npieces = __builtin_amdgcn_readfirstlane(np);
    nj = __builtin_amdgcn_readfirstlane(nj);
    for (int j = 0; j < nj; ++j) {
      const int v = __builtin_amdgcn_readfirstlane(jobs[2 * j]);
      const int f = __builtin_amdgcn_readfirstlane(jobs[2 * j + 1]);
      for (int p = f; p < P.S; ++p) write_empty(v, p, true);
    }
    barrier();  // the P buffers are free again
  }

  // the pieces of this workgroup: its range (fixed partition) or the
  // worker's pieces in row order (balanced); a barrier between two pieces
  // (the previous one's partial staging vs the next one's first loads)
  for (int it = 0;; ++it) {
    int bj, pf, T0, T1;
    if constexpr (!balanced) {
      if (it > 0) break;
      const int qj = r1 % P.QL;
      const int r2 = r1 / P.QL;
      const int b = r2 / P.S;
      bj = b * P.QL + qj;
      pf = r2 % P.S;
      if (pf + 1 == P.S)  // the last range's workgroup marks the slots past the ranges
        for (int p = P.S; p < P.S_out; ++p) write_empty(bj, p, true);
      T0 = pf * P.chunk;
      T1 = min((pf + 1) * P.chunk, attended(bj));
    } else {
      if (it >= npieces) break;
      const int e0 = __builtin_amdgcn_readfirstlane(plist[3 * it]);
      bj = e0 & 0xFFFF;
      pf = e0 >> 16;
      T0 = __builtin_amdgcn_readfirstlane(plist[3 * it + 1]);
      T1 = __builtin_amdgcn_readfirstlane(plist[3 * it + 2]);
    }
    if (it > 0) barrier();
    // balanced: the lane ids pass through an opaque copy per piece, so that
    // the addresses derived from them are formed inside the piece rather
    // than held across all of them
    int lane_i = lane, tid_i = tid;
    if constexpr (balanced) asm volatile("" : "+v"(lane_i), "+v"(tid_i));
    unit(bj, pf, T0, T1, lane_i, tid_i);
  }
}

// ================================================================ stream probe
//
// The decode's tile stream alone, the ceiling its HBM fraction is read
// against: workgroups of 8 waves, 4 of which stream 32-row bf16 tiles (36 KB)
// into a ring of 4 LDS tile buffers with the decode's DMA plan and counted
// waits (2 tiles in flight), one barrier per tile, no compute.  With `paired`
// the two workgroups of adjacent work ids (one XCD) read the same tiles, as the
// two head groups of a decode range do.
__global__ __attribute__((amdgpu_flat_work_group_size(kWsThreads, kWsThreads)))
void stream_probe_kernel(const uint8_t* __restrict__ src, int tiles, int paired, int32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNBuf * kTileBytes];
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const uint8_t* base = src + static_cast<int64_t>(paired ? wid >> 1 : wid) * tiles * kTileBytes;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool issuer = wave >= 4;
  auto dma = [&](int t) {
    rows_dma_g8(base + static_cast<int64_t>(t) * kTileBytes,
                lds_addr(smem) + (t & (kNBuf - 1)) * kTileBytes, kTileTokens, wave & 3);
  };
  if (issuer) {
    dma(0);
    if (tiles > 1) dma(1);
  }
  for (int t = 0; t < tiles; ++t) {
    if (issuer) {  // tile t landed (tile t + 1 may be in flight)
      if (t + 1 < tiles)
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (issuer && t + 2 < tiles) dma(t + 2);  // into the buffer of tile t - 2
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = smem[wid & 1023];
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
  int32_t ring;
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
  const int L = attended_len(P.seq_lens, b, P.max_seq_len, P.ring, P.seq_stride);
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
// One wave per (b, head); lane l owns latent columns 8l .. 8l+7 (16 bytes of
// each bf16 partial).  The first group of partial loads is issued before the
// log-sum-exp weights are computed, so the two do not form a chain.

constexpr int kCombThreads = 64;

template <int PART_DT>
struct PartVec {  // 8 columns of one partial
  static constexpr int kWords = PART_DT == MLA_F32 ? 8 : 4;
  uint32_t w[kWords];
};

template <int PART_DT>
__device__ inline PartVec<PART_DT> load_part(const void* u_part, int64_t elem) {
  PartVec<PART_DT> v;
  if constexpr (PART_DT == MLA_F32) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(u_part) + elem);
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(u_part) + elem + 4);
    v.w[0] = a.x; v.w[1] = a.y; v.w[2] = a.z; v.w[3] = a.w;
    v.w[4] = c.x; v.w[5] = c.y; v.w[6] = c.z; v.w[7] = c.w;
  } else {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(u_part) + elem);
    v.w[0] = a.x; v.w[1] = a.y; v.w[2] = a.z; v.w[3] = a.w;
  }
  return v;
}

template <int PART_DT>
__device__ inline float part_elem(const PartVec<PART_DT>& v, int k) {
  if constexpr (PART_DT == MLA_F32) return __uint_as_float(v.w[k]);
  else return __uint_as_float((k & 1) ? (v.w[k >> 1] & 0xFFFF0000u) : (v.w[k >> 1] << 16));
}

template <int PART_DT, int U_DT>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const void* u_part,
                                                              const float* lse_part, void* u,
                                                              float* lse, int H, int S) {
  constexpr int kG = PART_DT == MLA_F32 ? 8 : 16;  // partials in flight per lane
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int lane = threadIdx.x;
  const int c0 = lane * 8;
  auto part_at = [&](int p) {
    return ((static_cast<int64_t>(b) * S + p) * H + h) * kDLatent + c0;
  };
  auto lse_at = [&](int p) { return lse_part[(static_cast<int64_t>(b) * S + p) * H + h]; };
  // log-sum-exp weights (parts with lse = -inf carry no weight and their
  // u is not read: an empty split's u is not written), and the last split
  // with a finite or NaN log-sum-exp
  float mx = -INFINITY;
  int last = -1;
  for (int p = lane; p < S; p += 64) {
    const float x = lse_at(p);
    mx = max_nan(mx, x);
    last = x != -INFINITY ? p : last;
  }
  for (int o = 32; o > 0; o >>= 1) {
    mx = max_nan(mx, __shfl_xor(mx, o));
    last = max(last, __shfl_xor(last, o));
  }
  float z = 0.0f;
  if (mx != -INFINITY)
    for (int p = lane; p < S; p += 64) z += expf(lse_at(p) - mx);
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
  const bool live = z > 0.0f || z != z;  // not every range empty (a NaN sum stays NaN)
  const float inv = live ? 1.0f / z : 0.0f;
  const int np = last + 1;  // splits that are read
  PartVec<PART_DT> v[kG];
#pragma unroll
  for (int i = 0; i < kG; ++i)
    if (i < np) v[i] = load_part<PART_DT>(u_part, part_at(i));
  float a[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int p0 = 0; p0 < np; p0 += kG) {
    // weight of partial p0 + i sits in lane i
    const int pl = p0 + (lane & (kG - 1));
    const float wl = (pl < np && mx != -INFINITY) ? expf(lse_at(pl) - mx) : 0.0f;
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      const float w = __shfl(wl, i);
      if (p0 + i < np && w != 0.0f) {  // an empty split before the last: not read
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = fmaf(w, part_elem<PART_DT>(v[i], k), a[k]);
      }
    }
#pragma unroll
    for (int i = 0; i < kG; ++i)
      if (p0 + kG + i < np) v[i] = load_part<PART_DT>(u_part, part_at(p0 + kG + i));
  }
  const int64_t ob = (static_cast<int64_t>(b) * H + h) * kDLatent + c0;
  if constexpr (U_DT == MLA_F32) {
    float* dst = static_cast<float*>(u) + ob;
    *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv};
    *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{a[4] * inv, a[5] * inv, a[6] * inv, a[7] * inv};
  } else {
    u32x4_t w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = pack_bf16x2(a[2 * k] * inv, a[2 * k + 1] * inv);
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(u) + ob) = w;
  }
  if (lse && lane == 0) lse[static_cast<int64_t>(b) * H + h] = live ? mx + logf(z) : -INFINITY;
}

// ================================================================ decoupled RoPE
//
// Rotation of the positional query q_R by the sequence's position (the
// content part q_C is not rotated): element i pairs with element i + d_r/2,
//   out[i]         = x[i] cos t_i - x[i + d_r/2] sin t_i,
//   out[i + d_r/2] = x[i + d_r/2] cos t_i + x[i] sin t_i,
// t_i = position * inv_freq[i] in binary32, inv_freq[i] = base^(-2i/d_r)
// rounded once to binary32 on the host.

struct RopeArgs {
  const int32_t* positions;  // [B]; nullptr: q_R is carried unchanged
  float inv_freq[kDRope / 2];
};

// element j of the rotated row whose element j is xj and element j ^ 32 is xp
__device__ inline float rope_elem(const RopeArgs& R, int pos, int j, float xj, float xp) {
  const float t = static_cast<float>(pos) * R.inv_freq[j & (kDRope / 2 - 1)];
  float sn, cs;
  sincosf(t, &sn, &cs);
  return j < kDRope / 2 ? xj * cs - xp * sn : xj * cs + xp * sn;
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
                                                            int d_nope, RopeArgs R) {
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
    if (tid < kDRope) {
      const int64_t rb = (static_cast<int64_t>(b0 + bb) * H + h) * kDRope;
      r0 = load_elem<Q_DT>(q_rope, rb + tid);
      if (R.positions)
        r0 = rope_elem(R, R.positions[b0 + bb], tid, r0, load_elem<Q_DT>(q_rope, rb + (tid ^ 32)));
    }
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

// ================================================================ absorb (MFMA)
//
// bf16 queries and W_UK: per head h, q̃ᵀ[c][b] = Σ_n W_UK[h][n][c] q_nope[b][h][n] on
// v_mfma_f32_32x32x16_bf16 (M = 32 latent columns, N = 32 sequences, K = n).  The
// contraction runs over W_UK's row axis, so a [d_nope x 128] column slab of W_UK[h]
// is staged in LDS (rows padded to 288 B) and read with transposing LDS reads; the
// query operand is 16 contiguous bytes of q_nope per lane.  Grid: (head, 4 slabs of
// 128 columns); wave w owns columns 32w..32w+31 of its slab.

constexpr int kProjThreads = 256;
constexpr int kAbsRowBytes = 128 * 2 + 32;
// output stage of the staged-query case (d_nope <= 128): past a 128-row W_UK
// slab and 32 query rows of 128 elements; 32 rows x (512 + 16) bytes at most
constexpr int kAbsOutOff = 128 * kAbsRowBytes + 32 * (2 * 128 + 16);
static_assert(kAbsOutOff + 32 * (128 * 4 + 16) <= kMaxDHead * kAbsRowBytes, "absorb LDS stage");

template <int OUT_DT>
__global__ __launch_bounds__(kProjThreads) void absorb_mfma_kernel(const uint16_t* q_nope,
                                                                  const void* q_rope,
                                                                  const uint16_t* w_uk, void* q_abs,
                                                                  int B, int H, int d_nope,
                                                                  RopeArgs R) {
  __shared__ __attribute__((aligned(16))) uint8_t wt[kMaxDHead * kAbsRowBytes];
  const int h = blockIdx.x;
  const int c_slab = blockIdx.y * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, bl = lane & 31;
  // Every independent load is issued before the first wait: the W_UK slab
  // W_UK[h][0:d_nope][c_slab : c_slab+128] (16 chunks of 16 B per row), the
  // query operands of the first tile of 32 sequences, and (slab 0) the RoPE
  // rows that are copied through.
  const uint16_t* wsrc = w_uk + static_cast<int64_t>(h) * d_nope * kDLatent + c_slab;
  constexpr int kStage = kMaxDHead * 16 / kProjThreads;  // 16 chunks per thread at most
  u32x4_t st[kStage];
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int q = i * kProjThreads + tid;
    if (q < d_nope * 16)
      st[i] = *reinterpret_cast<const u32x4_t*>(wsrc + static_cast<int64_t>(q >> 4) * kDLatent +
                                                 (q & 15) * 8);
  }
  // Lanes of sequences past B read sequence 0 (their output columns are not
  // stored) and k-steps past d_nope are never multiplied, so every load is
  // unconditional: no zero fill that would have to wait for a load in flight.
  auto load_q = [&](bf16x8_t (&bq)[kMaxDHead / 16], int b0) {
    const int b = b0 + bl;
    const uint16_t* qrow = q_nope + (static_cast<int64_t>(b < B ? b : 0) * H + h) * d_nope + 8 * g;
#pragma unroll
    for (int k = 0; k < kMaxDHead / 16; ++k)
      if (16 * k < d_nope) bq[k] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * k);
  };
  // With d_nope <= 128 the W_UK rows fill half of the LDS buffer, and the
  // query rows of a tile of 32 sequences (which all 4 waves multiply) are
  // staged once in the other half instead of being loaded by every wave:
  // thread tid moves 16-byte chunks tid and tid + 256 of the tile.
  const bool q_lds = d_nope <= kMaxDHead / 2;  // workgroup-uniform
  const int qcpr = d_nope / 8;                 // 16-byte chunks per query row
  const int q_stride = 2 * d_nope + 16;        // padded LDS row
  uint8_t* qs = wt + d_nope * kAbsRowBytes;
  auto q_chunk = [&](int i, int b0) {  // i-th chunk of this thread: (row, column) of the tile
    const int c = tid + i * kProjThreads;
    const int row = c / qcpr, col = 8 * (c % qcpr);
    const int b = b0 + row;
    return *reinterpret_cast<const u32x4_t*>(q_nope + (static_cast<int64_t>(b < B ? b : 0) * H + h) * d_nope + col);
  };
  auto q_store = [&](int i, const u32x4_t& v) {
    const int c = tid + i * kProjThreads;
    if (c < 32 * qcpr) *reinterpret_cast<u32x4_t*>(qs + (c / qcpr) * q_stride + 16 * (c % qcpr)) = v;
  };
  bf16x8_t bq[kMaxDHead / 16];
  u32x4_t qv[2], qn[2];
  if (q_lds) {
    qv[0] = q_chunk(0, 0);
    qv[1] = q_chunk(1, 0);
    if (B > 32) {  // the next tile's rows, staged while this one is multiplied
      qn[0] = q_chunk(0, 32);
      qn[1] = q_chunk(1, 32);
    }
  } else {
    load_q(bq, 0);
  }
  // RoPE rows: 8 chunks of 16 B per sequence, chunks tid and tid + 256 loaded
  // here (all of them for B <= 64), the rest where they are copied
  u32x4_t rv[2] = {u32x4_t{0u, 0u, 0u, 0u}, u32x4_t{0u, 0u, 0u, 0u}};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + k * kProjThreads;
    if (blockIdx.y == 0 && i < B * (kDRope / 8))
      rv[k] = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(q_rope) +
                                                (static_cast<int64_t>(i >> 3) * H + h) * kDRope +
                                                8 * (i & 7));
  }
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int q = i * kProjThreads + tid;
    if (q < d_nope * 16) *reinterpret_cast<u32x4_t*>(wt + (q >> 4) * kAbsRowBytes + (q & 15) * 16) = st[i];
  }
  if (q_lds) {
    q_store(0, qv[0]);
    q_store(1, qv[1]);
  }
  __syncthreads();
  // A operand (M = c, K = n) by transposing reads: lane (G, e, q4) points at
  // row n0 + 8*(G/2) + e (+4), columns 32*wave + 16*(G%2) + 4*q4
  const int G = lane >> 4, e = (lane >> 2) & 3, q4 = lane & 3;
  const uint8_t* abase = wt + (8 * (G >> 1) + e) * kAbsRowBytes + (32 * wave + 16 * (G & 1) + 4 * q4) * 2;
  for (int b0 = 0; b0 < B; b0 += 32) {
    if (q_lds) {
      if (b0 > 0) {  // the next tile of sequences replaces the staged rows
        __syncthreads();
        q_store(0, qn[0]);
        q_store(1, qn[1]);
        __syncthreads();
        if (b0 + 32 < B) {
          qn[0] = q_chunk(0, b0 + 32);
          qn[1] = q_chunk(1, b0 + 32);
        }
      }
      // B operand: lane (sequence bl, half g) reads elements 16k + 8g .. +7
#pragma unroll
      for (int k = 0; k < kMaxDHead / 16; ++k)
        if (16 * k < d_nope)
          bq[k] = *reinterpret_cast<const bf16x8_t*>(qs + bl * q_stride + 32 * k + 16 * g);
    } else if (b0 > 0) {
      load_q(bq, b0);
    }
    const int b = b0 + bl;
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxDHead / 16; ++k) {
      if (16 * k < d_nope) {
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4_t*)(abase + 16 * k * kAbsRowBytes));
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4_t*)(abase + (16 * k + 4) * kAbsRowBytes));
        const bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[k], acc, 0, 0, 0);
      }
    }
    // accumulator: column b, rows c = 8*(r/4) + 4*g + r%4 of the wave's 32 columns
    if (q_lds) {
      // the 32 x 128 output tile goes through LDS (past the W_UK slab and the
      // query rows), so that each store writes 16 bytes per lane along whole
      // 256-byte (bf16) or 512-byte (fp32) row segments instead of 8 or 16
      // bytes at a 1152-byte stride
      constexpr int kEsz = OUT_DT == MLA_F32 ? 4 : 2;
      constexpr int kOStride = 128 * kEsz + 16;
      constexpr int kOChunks = 128 * kEsz / 16;  // 16-byte chunks per row
      uint8_t* os = wt + kAbsOutOff;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint8_t* wp = os + bl * kOStride + (32 * wave + 8 * r4 + 4 * g) * kEsz;
        if constexpr (OUT_DT == MLA_F32) {
          *reinterpret_cast<f32x4_t*>(wp) = f32x4_t{acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
        } else {
          *reinterpret_cast<u32x2_t*>(wp) =
              u32x2_t{pack_bf16x2(acc[4 * r4], acc[4 * r4 + 1]), pack_bf16x2(acc[4 * r4 + 2], acc[4 * r4 + 3])};
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 32 * kOChunks / kProjThreads; ++i) {
        const int q = i * kProjThreads + tid, row = q / kOChunks, ch = q % kOChunks;
        if (b0 + row < B) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(os + row * kOStride + 16 * ch);
          uint8_t* dst = static_cast<uint8_t*>(q_abs) +
                         ((static_cast<int64_t>(b0 + row) * H + h) * kRowElems + c_slab) * kEsz;
          *reinterpret_cast<u32x4_t*>(dst + 16 * ch) = v;
        }
      }
      // the next tile's first barrier (before its query rows are staged)
      // orders these reads before the next tile's writes to the stage
    } else if (b < B) {
      const int64_t ob = (static_cast<int64_t>(b) * H + h) * kRowElems + c_slab + 32 * wave;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int c = 8 * r4 + 4 * g;
        if constexpr (OUT_DT == MLA_F32) {
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(q_abs) + ob + c) =
              f32x4_t{acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
        } else {
          const uint32_t w0 = pack_bf16x2(acc[4 * r4], acc[4 * r4 + 1]);
          const uint32_t w1 = pack_bf16x2(acc[4 * r4 + 2], acc[4 * r4 + 3]);
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(q_abs) + ob + c) = u32x2_t{w0, w1};
        }
      }
    }
  }
  // the RoPE part: slab 0 carries it (more rows than threads only when
  // B > 32), rotated by the sequence's position when positions are given
  if (blockIdx.y == 0) {
    for (int i = tid; i < B * (kDRope / 8); i += kProjThreads) {
      const int b = i >> 3, j = 8 * (i & 7);
      const uint16_t* rrow = static_cast<const uint16_t*>(q_rope) + (static_cast<int64_t>(b) * H + h) * kDRope;
      u32x4_t v = i == tid ? rv[0]
                  : i == tid + kProjThreads ? rv[1]
                                            : *reinterpret_cast<const u32x4_t*>(rrow + j);
      if (R.positions) {  // pair with the chunk 32 elements away
        const u32x4_t vp = *reinterpret_cast<const u32x4_t*>(rrow + (j ^ 32));
        const int pos = R.positions[b];
        float y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t wv = v[k >> 1], wp = vp[k >> 1];
          const float xj = __uint_as_float((k & 1) ? (wv & 0xFFFF0000u) : (wv << 16));
          const float xq = __uint_as_float((k & 1) ? (wp & 0xFFFF0000u) : (wp << 16));
          y[k] = rope_elem(R, pos, j + k, xj, xq);
        }
        const int64_t ob = (static_cast<int64_t>(b) * H + h) * kRowElems + kDLatent + j;
        if constexpr (OUT_DT == MLA_F32) {
          float* dst = static_cast<float*>(q_abs) + ob;
          *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{y[0], y[1], y[2], y[3]};
          *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{y[4], y[5], y[6], y[7]};
        } else {
          *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(q_abs) + ob) =
              u32x4_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                      pack_bf16x2(y[6], y[7])};
        }
        continue;
      }
      const int64_t ob = (static_cast<int64_t>(b) * H + h) * kRowElems + kDLatent + j;
      if constexpr (OUT_DT == MLA_F32) {
        float* dst = static_cast<float*>(q_abs) + ob;
        *reinterpret_cast<f32x4_t*>(dst) =
            f32x4_t{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                    __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u)};
        *reinterpret_cast<f32x4_t*>(dst + 4) =
            f32x4_t{__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xFFFF0000u),
                    __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xFFFF0000u)};
      } else {
        *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(q_abs) + ob) = v;
      }
    }
  }
}

// ================================================================ absorb with an E4M3 output
//
// The fp8 decode takes the absorbed query in E4M3 with one fp32 factor per
// (sequence, head), by the rule of the fp8 cache rows: the factor maps the
// row's largest magnitude over all 576 elements onto 448, each code is the
// correctly rounded quotient x / factor rounded to the nearest E4M3 value
// (ties to even, by the hardware conversion).  The factor needs the whole row
// in one workgroup: one workgroup per (head, 32 sequences), 16 waves.
// W_UK[h] (d_nope x 512 bf16, d_nope <= 128) is staged whole in LDS; wave w
// computes latent columns 32w..32w+31 of the 32 sequences on
// v_mfma_f32_32x32x16_bf16 (A = W_UK^T by transposing reads, B = the query
// rows, as in absorb_mfma_kernel); the first 256 threads carry the RoPE part
// (rotated when positions are given); the row maxima meet in LDS; the codes
// are staged in LDS over the W_UK slab, which is no longer read, and leave as
// whole 576-byte rows.
constexpr int kAf8Threads = 1024;
constexpr int kAf8Row = kDLatent * 2 + 16;               // padded LDS row of W_UK[h]
constexpr int kAf8QStride = 2 * 128 + 16;                // padded query row (d_nope <= 128)
constexpr int kAf8QOff = 128 * kAf8Row;
constexpr int kAf8RedOff = kAf8QOff + 32 * kAf8QStride;  // float [32][24]: row maxima
constexpr int kAf8ScOff = kAf8RedOff + 32 * 24 * 4;      // float [32]: factors
constexpr int kAf8Lds = kAf8ScOff + 32 * 4;
constexpr int kAf8Out = kRowElems + 16;                  // staged code row
static_assert(32 * kAf8Out <= kAf8QOff, "absorb fp8 output stage");
static_assert(kAf8Lds <= 160 * 1024, "absorb fp8 LDS");

__global__ __launch_bounds__(kAf8Threads) void absorb_f8_kernel(const uint16_t* q_nope,
                                                               const uint16_t* q_rope,
                                                               const uint16_t* w_uk, uint8_t* q_abs,
                                                               float* q_scale, int B, int H,
                                                               int d_nope, RopeArgs R) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[kAf8Lds];
  float* red = reinterpret_cast<float*>(sm + kAf8RedOff);
  float* fac = reinterpret_cast<float*>(sm + kAf8ScOff);
  const int h = blockIdx.x, b0 = blockIdx.y * 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, bl = lane & 31;
  // every load before the first wait: W_UK[h] (d_nope rows of 64 chunks of
  // 16 B, 8 per thread), the 32 query rows (one chunk per thread), the RoPE
  // rows (threads < 256: 8 elements of sequence b0 + tid / 8)
  const uint16_t* wsrc = w_uk + static_cast<int64_t>(h) * d_nope * kDLatent;
  constexpr int kSt = 128 * 64 / kAf8Threads;
  u32x4_t st[kSt];
#pragma unroll
  for (int i = 0; i < kSt; ++i) {
    const int q = i * kAf8Threads + tid;
    if (q < d_nope * 64) st[i] = *reinterpret_cast<const u32x4_t*>(wsrc + (q >> 6) * kDLatent + (q & 63) * 8);
  }
  const int qcpr = d_nope / 8;
  const int qrow = tid / qcpr, qcol = tid % qcpr;
  const bool q_thread = tid < 32 * qcpr;
  u32x4_t qv = u32x4_t{0u, 0u, 0u, 0u};
  if (q_thread) {
    const int b = b0 + qrow;
    qv = *reinterpret_cast<const u32x4_t*>(q_nope + (static_cast<int64_t>(b < B ? b : 0) * H + h) * d_nope + 8 * qcol);
  }
  const bool rope_thread = tid < 256;
  const int rb = b0 + (tid >> 3), rj = 8 * (tid & 7);
  float y[8];
  if (rope_thread) {
    const uint16_t* rrow = q_rope + (static_cast<int64_t>(rb < B ? rb : 0) * H + h) * kDRope;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(rrow + rj);
    if (R.positions) {  // pair with the chunk 32 elements away
      const u32x4_t vp = *reinterpret_cast<const u32x4_t*>(rrow + (rj ^ 32));
      const int pos = R.positions[rb < B ? rb : 0];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t wv = v[k >> 1], wp = vp[k >> 1];
        const float xj = __uint_as_float((k & 1) ? (wv & 0xFFFF0000u) : (wv << 16));
        const float xq = __uint_as_float((k & 1) ? (wp & 0xFFFF0000u) : (wp << 16));
        y[k] = rope_elem(R, pos, rj + k, xj, xq);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t wv = v[k >> 1];
        y[k] = __uint_as_float((k & 1) ? (wv & 0xFFFF0000u) : (wv << 16));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kSt; ++i) {
    const int q = i * kAf8Threads + tid;
    if (q < d_nope * 64) *reinterpret_cast<u32x4_t*>(sm + (q >> 6) * kAf8Row + (q & 63) * 16) = st[i];
  }
  uint8_t* qs = sm + kAf8QOff;
  if (q_thread) *reinterpret_cast<u32x4_t*>(qs + qrow * kAf8QStride + 16 * qcol) = qv;
  __syncthreads();

  // columns 32 wave .. 32 wave + 31; accumulator: column
  // 32 wave + 8 (r / 4) + 4 g + r % 4 of sequence b0 + bl
  const int G = lane >> 4, e = (lane >> 2) & 3, q4 = lane & 3;
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  for (int k = 0; k < d_nope / 16; ++k) {
    const bf16x8_t bq = *reinterpret_cast<const bf16x8_t*>(qs + bl * kAf8QStride + 32 * k + 16 * g);
    const uint8_t* ab = sm + (16 * k + 8 * (G >> 1) + e) * kAf8Row +
                        (32 * wave + 16 * (G & 1) + 4 * q4) * 2;
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)ab);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(ab + 4 * kAf8Row));
    const bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, acc, 0, 0, 0);
  }
  // row maxima: 16 waves, and 8 RoPE chunks, per sequence
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[r]));
  m = fmaxf(m, __shfl_xor(m, 32));
  if (g == 0) red[bl * 24 + wave] = m;
  if (rope_thread) {
    float mr = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) mr = fmaxf(mr, fabsf(y[k]));
    red[(tid >> 3) * 24 + 16 + (tid & 7)] = mr;
  }
  __syncthreads();
  if (tid < 32) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 24; ++i) amax = fmaxf(amax, red[tid * 24 + i]);
    const float f = fmaxf(amax, 0x1p-126f) / 448.0f;
    fac[tid] = f;
    if (b0 + tid < B) q_scale[static_cast<int64_t>(b0 + tid) * H + h] = f;
  }
  __syncthreads();
  // codes, staged over the W_UK slab (every wave is past its last read)
  {
    const float f = fac[bl];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = fminf(fmaxf(acc[4 * r4 + q] / f, -448.0f), 448.0f);
      // v_cvt_pk_fp8_f32: OCP E4M3, round to nearest even (the same codes as
      // e4m3_encode for |x| <= 448)
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
      *reinterpret_cast<int*>(sm + bl * kAf8Out + 32 * wave + 8 * r4 + 4 * g) = w;
    }
  }
  if (rope_thread) {
    const float f = fac[tid >> 3];
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = fminf(fmaxf(y[k] / f, -448.0f), 448.0f);
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], w1, true);
    *reinterpret_cast<u32x2_t*>(sm + (tid >> 3) * kAf8Out + kDLatent + rj) =
        u32x2_t{static_cast<uint32_t>(w0), static_cast<uint32_t>(w1)};
  }
  __syncthreads();
  // 32 rows x 36 chunks of 16 B
  for (int i = tid; i < 32 * (kRowElems / 16); i += kAf8Threads) {
    const int row = i / (kRowElems / 16), ch = i % (kRowElems / 16);
    if (b0 + row < B)
      *reinterpret_cast<u32x4_t*>(q_abs + (static_cast<int64_t>(b0 + row) * H + h) * kRowElems + 16 * ch) =
          *reinterpret_cast<const u32x4_t*>(sm + row * kAf8Out + 16 * ch);
  }
}

// ================================================================ up-projection (MFMA)
//
// bf16 u and W_UV: per head h, oᵀ[v][b] = Σ_c W_UV[h][v][c] u[b][h][c] on
// v_mfma_f32_32x32x16_bf16 (M = 32 value rows, N = 32 sequences, K = c).  Both
// operands are contiguous along c.  One workgroup (2 waves) per (head, 64
// value rows): each wave keeps its 32 rows of W_UV (32 x 512) in VGPRs, loaded
// straight from global memory, while the 32 x 512 tile of u rows is staged in
// LDS (rows padded by 16 bytes) by both waves; all of these loads are issued
// before the first wait.  Sequences are walked in tiles of 32.

constexpr int kUpThreads = 128;
constexpr int kUpRow = kDLatent * 2 + 16;  // padded LDS row of u

template <int O_DT>
__global__ __launch_bounds__(kUpThreads) void up_proj_mfma_kernel(const uint16_t* u,
                                                                 const uint16_t* w_uv, void* o,
                                                                 int B, int H, int d_v) {
  __shared__ __attribute__((aligned(16))) uint8_t us[32 * kUpRow];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int v0 = blockIdx.y * 64 + wave * 32;
  const int v = v0 + l32;
  const bool vv = v < d_v;
  bf16x8_t wa[kDLatent / 16];
  const uint16_t* wrow = w_uv + (static_cast<int64_t>(h) * d_v + (vv ? v : 0)) * kDLatent + 8 * g;
#pragma unroll
  for (int k = 0; k < kDLatent / 16; ++k)
    wa[k] = vv ? *reinterpret_cast<const bf16x8_t*>(wrow + 16 * k) : bf16x8_t{};
  for (int b0 = 0; b0 < B; b0 += 32) {
    // stage u rows b0 .. b0+31 of head h: 32 x 64 chunks of 16 B, 16 per thread
    u32x4_t st[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = i * kUpThreads + tid, r = q >> 6, cc = q & 63;
      st[i] = (b0 + r < B) ? *reinterpret_cast<const u32x4_t*>(
                                 u + (static_cast<int64_t>(b0 + r) * H + h) * kDLatent + cc * 8)
                           : u32x4_t{0u, 0u, 0u, 0u};
    }
    if (b0 > 0) __syncthreads();  // previous tile fully read
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = i * kUpThreads + tid, r = q >> 6, cc = q & 63;
      *reinterpret_cast<u32x4_t*>(us + r * kUpRow + cc * 16) = st[i];
    }
    __syncthreads();
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const uint8_t* urow = us + l32 * kUpRow + 16 * g;
#pragma unroll
    for (int k = 0; k < kDLatent / 16; ++k)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          wa[k], *reinterpret_cast<const bf16x8_t*>(urow + 32 * k), acc, 0, 0, 0);
    // accumulator: column b = b0 + l32, rows v0 + 8*(r/4) + 4*g + r%4
    const int b = b0 + l32;
    if (b < B) {
      const int64_t ob = (static_cast<int64_t>(b) * H + h) * d_v;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int vr = v0 + 8 * r4 + 4 * g;
        if (vr + 3 < d_v && (d_v & 3) == 0) {
          if constexpr (O_DT == MLA_F32) {
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(o) + ob + vr) =
                f32x4_t{acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
          } else {
            const uint32_t w0 = pack_bf16x2(acc[4 * r4], acc[4 * r4 + 1]);
            const uint32_t w1 = pack_bf16x2(acc[4 * r4 + 2], acc[4 * r4 + 3]);
            *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(o) + ob + vr) = u32x2_t{w0, w1};
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (vr + k < d_v) store_elem<O_DT>(o, ob + vr + k, acc[4 * r4 + k]);
        }
      }
    }
  }
}

// ================================================================ combine + up-projection
//
// mla_combine followed by mla_up_proj in one kernel, for bf16 W_UV: one
// workgroup of 8 waves per (head h, 16 consecutive sequences).
//   1. the u rows of the 16 sequences are merged from the split partials with
//      log-sum-exp weights (32 lanes per row and split phase, 16 latent
//      columns per lane; fewer sequences get more phases) and rounded to bf16
//      into LDS — the values mla_combine stores, up to summation order;
//   2. o[b][h][:] = W_UV[h] u[b] on v_mfma_f32_16x16x32_bf16 (M = 16
//      sequences, N = 16 value rows per wave, K = 32 latent columns): A = u
//      from LDS, B = rows of W_UV, 16 contiguous bytes per lane from global
//      memory.
// Every independent load is issued first: the wave's W_UV rows, then the
// first splits' partial rows, then the log-sum-exp inputs; later splits are
// requested one batch ahead of their use.

constexpr int kCuThreads = 512;
constexpr int kCuRows = 16;                // sequences per workgroup
constexpr int kCuRow = kDLatent * 2 + 16;  // padded LDS row of u (bf16)
constexpr int kCuBatch = 4;                // splits per batch of partial loads

template <int PART_DT, int O_DT, int VS, int LSE_BLK, bool EARLY_W>
__global__ __launch_bounds__(kCuThreads) void combine_up_kernel(
    const void* u_part, const float* lse_part, const uint16_t* w_uv, void* o, uint16_t* u_out,
    float* lse_out, int B, int H, int S, int d_v, int rows) {
  // u rows (bf16), then the per-group fp32 sums of the phase reduction
  __shared__ __attribute__((aligned(16))) uint8_t us[kCuRows * kCuRow + kCuRows * 32 * 64];
  // `rows` (a power of two <= 16) consecutive sequences of one head per
  // workgroup: fewer than 16 when the batch is small, so the grid still
  // covers the CUs.  With one sequence per workgroup and still too few
  // workgroups, VS = 2 workgroups share a (head, sequence): each merges all
  // of its partials and multiplies by its half of the value rows.
  static_assert(VS == 1 || VS == 2, "value split");
  const int nbt = (B + rows - 1) / rows;
  const int wid = xcd_remap(blockIdx.x, H * nbt * VS);
  const int vs = wid % VS;  // adjacent: the halves read the partials through one L2
  const int h = wid / VS / nbt;  // the sequence tiles of one head share W_UV[h] in L2
  const int b0 = (wid / VS % nbt) * rows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, kg = lane >> 4;
  const int nnb = d_v / 16;  // value blocks of 16 rows
  const int nbper = (nnb + VS - 1) / VS;
  const int nb0 = vs * nbper, nb1 = min(nnb, nb0 + nbper);  // this workgroup's value blocks
  constexpr int kWaves = kCuThreads / 64;
  constexpr int kKs = kDLatent / 32;  // k-steps

  // ---- 1. merge: 16 groups of 32 lanes, 16 latent columns per lane.  With
  // nrows sequences in the workgroup, group g takes sequence r = g % nrows
  // and every nph-th split from ph = g / nrows, so small batches still keep
  // all 512 threads' loads in flight; the groups of a sequence are summed in
  // LDS afterwards, in phase order.
  const int nrows = min(rows, B - b0);  // >= 1
  const int nph = kCuRows / nrows;         // split phases per sequence
  const int grp = tid >> 5, cg = tid & 31;
  const int r = grp % nrows, ph = grp / nrows;
  // this group's splits: all of its phase at first; once the log-sum-exp
  // inputs are in, only those below the last non-empty split
  int ns = (ph < nph && ph < S) ? (S - ph + nph - 1) / nph : 0;
  const int b = b0 + r;
  const int64_t prow = (static_cast<int64_t>(b) * S) * H + h;  // (b, p = 0, h)
  auto split = [&](int kk) { return ph + nph * kk; };

  // Every independent load is issued before the first wait, and all of them
  // unconditionally (clamped to valid addresses) so that the compiler's wait
  // counts stay exact: the log-sum-exp inputs of splits cg + 32 j (all a lane
  // needs when S <= 32 kCuLse), the wave's W_UV rows, the first batch of
  // partials.  LSE_BLK = 1 (S <= 32) or 8 (S <= 256) registers of them.
  constexpr int kCuLse = LSE_BLK;
  const bool lse_reg = S <= 32 * kCuLse;  // workgroup-uniform
  float lse_l[kCuLse];
#pragma unroll
  for (int j = 0; j < kCuLse; ++j)
    lse_l[j] = lse_part[prow + static_cast<int64_t>(min(cg + 32 * j, S - 1)) * H];
  auto wrow = [&](int nb) {
    return w_uv + (static_cast<int64_t>(h) * d_v + 16 * nb + n16) * kDLatent + 8 * kg;
  };
  // EARLY_W: the wave's W_UV rows are loaded with the first loads (64 more
  // VGPRs: one 512-thread workgroup per CU); else once the partials are
  // summed, in flight during the merge's LDS steps (two workgroups per CU,
  // for grids of more workgroups than CUs)
  bf16x8_t wk[kKs];
  if (EARLY_W && (VS == 1 || nb0 + wave < nb1)) {  // wave-uniform
    const uint16_t* wr = wrow(min(nb0 + wave, nb1 - 1));
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) wk[ks] = *reinterpret_cast<const bf16x8_t*>(wr + 32 * ks);
  }
  // splits per batch of partial loads: fp32 partials take twice the registers
  constexpr int kBatch = PART_DT == MLA_F32 ? kCuBatch / 2 : kCuBatch;
  constexpr int kEl = PART_DT == MLA_F32 ? 4 : 8;  // elements per 16-byte load
  constexpr int kLd = 16 / kEl;                     // loads per split
  auto load_batch = [&](u32x4_t (&v)[kBatch][kLd], int k0) {
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int p = ns > 0 ? split(min(k0 + q, ns - 1)) : 0;
      const int64_t e = (prow + static_cast<int64_t>(p) * H) * kDLatent + 16 * cg;
#pragma unroll
      for (int i = 0; i < kLd; ++i) {
        if constexpr (PART_DT == MLA_F32)
          v[q][i] = *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(u_part) + e + 4 * i);
        else
          v[q][i] = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(u_part) + e + 8 * i);
      }
    }
  };
  u32x4_t va[kBatch][kLd], vb[kBatch][kLd];
  load_batch(va, 0);
  // log-sum-exp weights over all splits of the sequence (every group of the
  // sequence computes the same values)
  float mx = -INFINITY, z = 0.0f;
  float e_l[kCuLse];  // S <= 32 kCuLse: weights of splits cg + 32 j
  int last = -1;       // last split with a finite log-sum-exp
  if (lse_reg) {
#pragma unroll
    for (int j = 0; j < kCuLse; ++j) {
      lse_l[j] = cg + 32 * j < S ? lse_l[j] : -INFINITY;
      mx = max_nan(mx, lse_l[j]);
      last = lse_l[j] != -INFINITY ? cg + 32 * j : last;
    }
#pragma unroll
    for (int o2 = 1; o2 < 32; o2 <<= 1) mx = max_nan(mx, __shfl_xor(mx, o2));
#pragma unroll
    for (int j = 0; j < kCuLse; ++j) {
      e_l[j] = (mx != -INFINITY) ? expf(lse_l[j] - mx) : 0.0f;
      z += e_l[j];
    }
  } else {
    for (int p = cg; p < S; p += 32) {
      const float x = lse_part[prow + static_cast<int64_t>(p) * H];
      mx = max_nan(mx, x);
      last = x != -INFINITY ? p : last;
    }
#pragma unroll
    for (int o2 = 1; o2 < 32; o2 <<= 1) mx = max_nan(mx, __shfl_xor(mx, o2));
    if (mx != -INFINITY)
      for (int p = cg; p < S; p += 32) z += expf(lse_part[prow + static_cast<int64_t>(p) * H] - mx);
  }
#pragma unroll
  for (int o2 = 1; o2 < 32; o2 <<= 1) {
    z += __shfl_xor(z, o2);
    last = max(last, __shfl_xor(last, o2));
  }
  const bool live = z > 0.0f || z != z;  // not every range empty (a NaN sum stays NaN)
  const float inv = live ? 1.0f / z : 0.0f;
  // Splits past the last finite log-sum-exp are empty ranges (the trailing
  // ranges of a short sequence, the slots past merged range groups): weight 0,
  // and their partials are not read (an empty split's u is not written).
  ns = min(ns, ph <= last ? (last - ph) / nph + 1 : 0);
  float acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = 0.0f;
  float wl = 0.0f;  // S > 32: weight of the group's split 32 * (k / 32) + (lane % 32)
  auto accumulate = [&](const u32x4_t (&v)[kBatch][kLd], int k0) {
    if (!lse_reg && (k0 & 31) == 0) {
      const int kl = k0 + cg;
      wl = (kl < ns && mx != -INFINITY)
               ? expf(lse_part[prow + static_cast<int64_t>(split(kl)) * H] - mx)
               : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      float w;
      if (lse_reg) {  // split p's weight: lane p % 32, register p / 32
        const int sp = split(k0 + q);
        float ev = e_l[0];
#pragma unroll
        for (int j = 1; j < kCuLse; ++j) ev = (sp >> 5) == j ? e_l[j] : ev;
        w = __shfl(ev, (lane & ~31) | (sp & 31));
      } else {
        w = __shfl(wl, (lane & ~31) | ((k0 + q) & 31));
      }
      if (k0 + q < ns && w != 0.0f) {  // an empty split before the last: its u is not read
#pragma unroll
        for (int i = 0; i < kLd; ++i)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if constexpr (PART_DT == MLA_F32) {
              acc[4 * i + k] = fmaf(w, __uint_as_float(v[q][i][k]), acc[4 * i + k]);
            } else {
              acc[8 * i + 2 * k] = fmaf(w, __uint_as_float(v[q][i][k] << 16), acc[8 * i + 2 * k]);
              acc[8 * i + 2 * k + 1] = fmaf(w, __uint_as_float(v[q][i][k] & 0xFFFF0000u), acc[8 * i + 2 * k + 1]);
            }
          }
      }
    }
  };
  // batches of kBatch splits, the next batch in flight while one is summed
  for (int k0 = 0; k0 < ns; k0 += 2 * kBatch) {
    if (k0 + kBatch < ns) load_batch(vb, k0 + kBatch);
    accumulate(va, k0);
    if (k0 + kBatch < ns) {
      if (k0 + 2 * kBatch < ns) load_batch(va, k0 + 2 * kBatch);
      accumulate(vb, k0 + kBatch);
    }
  }
  if (!EARLY_W && (VS == 1 || nb0 + wave < nb1)) {  // wave-uniform
    const uint16_t* wr = wrow(min(nb0 + wave, nb1 - 1));
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) wk[ks] = *reinterpret_cast<const bf16x8_t*>(wr + 32 * ks);
  }
  if (nph > 1) {  // workgroup-uniform: sum the phases of each sequence
    f32x4_t* red = reinterpret_cast<f32x4_t*>(us + kCuRows * kCuRow);  // [group][4][lane]
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
      red[(grp * 4 + k4) * 32 + cg] = f32x4_t{acc[4 * k4], acc[4 * k4 + 1], acc[4 * k4 + 2], acc[4 * k4 + 3]};
    __syncthreads();
    if (ph == 0) {
      for (int j = 1; j < nph; ++j) {
        const int g2 = j * nrows + r;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const f32x4_t x = red[(g2 * 4 + k4) * 32 + cg];
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[4 * k4 + k] += x[k];
        }
      }
    }
  }
  if (ph == 0) {
    const u32x4_t u0 = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                        pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
    const u32x4_t u1 = {pack_bf16x2(acc[8] * inv, acc[9] * inv), pack_bf16x2(acc[10] * inv, acc[11] * inv),
                        pack_bf16x2(acc[12] * inv, acc[13] * inv), pack_bf16x2(acc[14] * inv, acc[15] * inv)};
    *reinterpret_cast<u32x4_t*>(us + r * kCuRow + cg * 32) = u0;
    *reinterpret_cast<u32x4_t*>(us + r * kCuRow + cg * 32 + 16) = u1;
    if (u_out && vs == 0) {
      uint16_t* dst = u_out + (static_cast<int64_t>(b) * H + h) * kDLatent + 16 * cg;
      *reinterpret_cast<u32x4_t*>(dst) = u0;
      *reinterpret_cast<u32x4_t*>(dst + 8) = u1;
    }
    if (lse_out && cg == 0 && vs == 0) lse_out[static_cast<int64_t>(b) * H + h] = live ? mx + logf(z) : -INFINITY;
  }
  __syncthreads();

  // ---- 2. o = u W_UV^T on the matrix cores
  // A: row n16 (sequence), k group kg.  Rows past the batch are never written;
  // they only reach D rows that are not stored.
  const uint8_t* arow = us + n16 * kCuRow + 16 * kg;
  for (int nb = nb0 + wave; nb < nb1; nb += kWaves) {
    if (nb != nb0 + wave) {
      const uint16_t* wr = wrow(nb);
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) wk[ks] = *reinterpret_cast<const bf16x8_t*>(wr + 32 * ks);
    }
    f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(arow + 64 * ks);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, wk[ks], d, 0, 0, 0);
    }
    // D: column n16 = value row 16 nb + n16, rows 4 kg + i = sequences (only
    // the workgroup's own nrows are stored)
    const int v = 16 * nb + n16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * kg + i;
      if (rr < nrows)
        store_elem<O_DT>(o, (static_cast<int64_t>(b0 + rr) * H + h) * d_v + v, d[i]);
    }
  }
}

// ================================================================ MHA / GQA baseline decode
//
// Multi-head (and grouped-query) attention decode over a full bf16 K/V cache
// (head-major [B][h_kv][seq_stride][128]), the baselines the latent cache
// replaces.  Query head h reads key/value head h / G (G = h / h_kv query heads
// per group); the G workgroups of a group are adjacent in the work order and
// so run on one XCD, where its L2 serves the K/V rows to all of them after one
// HBM read.  One workgroup of 4 waves per (b, query head); wave w streams a contiguous quarter of
// the tokens with its own online softmax.  Per step a wave takes 16 tokens:
// lane group g (16 lanes) owns tokens 4u + g, lane k of a group holds
// elements 8k..8k+7 of a key and a value row (16-byte loads, 256 contiguous
// bytes per token), the dot products reduce over the 16 lanes, one maximum
// per step rescales the accumulators.  The next step's 8 loads per lane are
// in flight while a step is summed.  The four waves merge in LDS.  No matrix
// cores: one query row per head has nothing to reuse, the kernel is a stream.

constexpr int kMhaThreads = 256;
constexpr int kMhaD = 128;

template <int O_DT>
__global__ __launch_bounds__(kMhaThreads) void mha_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ seq_lens, int64_t seq_stride, int32_t max_seq_len, int H,
    int G, float scale_log2, void* o, float* lse) {
  __shared__ float red_m[4], red_l[4];
  __shared__ __attribute__((aligned(16))) float red_acc[4][kMhaD];
  // work id (b, query head): consecutive ids, one group's heads, on one XCD
  const int bh = G > 1 ? xcd_remap(blockIdx.x, gridDim.x) : blockIdx.x;
  const int b = bh / H;
  const int kv = b * (H / G) + (bh % H) / G;  // (b, key/value head) row block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, k = lane & 15;
  const int L = min(max(seq_lens[b], 0), max_seq_len);
  const int chunk = ((L + 3) / 4 + 15) & ~15;  // tokens per wave, a multiple of 16
  const int t0 = min(wave * chunk, L), t1 = min(t0 + chunk, L);
  const int64_t rowbase = static_cast<int64_t>(kv) * seq_stride;

  float qv[8];
  {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(q + static_cast<int64_t>(bh) * kMhaD + 8 * k);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[2 * i] = __uint_as_float(w[i] << 16) * scale_log2;
      qv[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u) * scale_log2;
    }
  }
  float m = -INFINITY, l = 0.0f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;

  // rows of tokens past the wave's range are replaced by its first row
  // (finite data, weight zero); a wave with no tokens loads nothing
  auto load = [&](u32x4_t (&kr)[4], u32x4_t (&vr)[4], int ts) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = ts + 4 * u + g;
      const int64_t r = (rowbase + (t < t1 ? t : t0)) * kMhaD + 8 * k;
      kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kc + r));
      vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vc + r));
    }
  };
  auto step = [&](const u32x4_t (&kr)[4], const u32x4_t (&vr)[4], int ts) {
    float sc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d = fmaf(qv[2 * i], __uint_as_float(kr[u][i] << 16), d);
        d = fmaf(qv[2 * i + 1], __uint_as_float(kr[u][i] & 0xFFFF0000u), d);
      }
#pragma unroll
      for (int o2 = 8; o2 >= 1; o2 >>= 1) d += __shfl_xor(d, o2);
      sc[u] = (ts + 4 * u + g < t1) ? d : -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);  // finite: every step holds at least one token
    const float r = __builtin_amdgcn_exp2f(m - mn);
    l *= r;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= r;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float p = __builtin_amdgcn_exp2f(sc[u] - mn);
      l += p;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(p, __uint_as_float(vr[u][i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(p, __uint_as_float(vr[u][i] & 0xFFFF0000u), acc[2 * i + 1]);
      }
    }
    m = mn;
  };
  if (t0 < t1) {
    u32x4_t ka[4], va[4], kb[4], vb[4];
    load(ka, va, t0);
    for (int ts = t0; ts < t1; ts += 32) {
      if (ts + 16 < t1) load(kb, vb, ts + 16);
      step(ka, va, ts);
      if (ts + 16 < t1) {
        if (ts + 32 < t1) load(ka, va, ts + 32);
        step(kb, vb, ts + 16);
      }
    }
  }
  // the four lane groups: the sums of their own tokens (m is common)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i] += __shfl_xor(acc[i], 16);
    acc[i] += __shfl_xor(acc[i], 32);
  }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (lane < 16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red_acc[wave][8 * lane + i] = acc[i];
  }
  if (lane == 0) {
    red_m[wave] = m;
    red_l[wave] = l;
  }
  __syncthreads();
  if (wave == 0 && lane < 16) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w]);
    float lt = 0.0f, ot[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ot[i] = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = __builtin_amdgcn_exp2f(red_m[w] - M);  // 0 for a wave without tokens
        lt += f * red_l[w];
#pragma unroll
        for (int i = 0; i < 8; ++i) ot[i] += f * red_acc[w][8 * lane + i];
      }
    }
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) store_elem<O_DT>(o, static_cast<int64_t>(bh) * kMhaD + 8 * lane + i, ot[i] * inv);
    if (lse && lane == 0) lse[bh] = lt > 0.0f ? (M + log2f(lt)) * kLn2 : -INFINITY;
  }
}

// ================================================================ cache append
//
// One wave per sequence writes the new token's row (576 elements: lane l
// takes elements l + 64 j, so every store instruction covers 64 consecutive
// elements).  For an E4M3 cache the row maximum is reduced across the wave,
// the factor s = max(amax, 2^-126) / 448 and the quotients x / s are
// correctly rounded binary32 divisions (the library is built without fast
// math), and each quotient is rounded to E4M3 by e4m3_encode.

constexpr int kAppendThreads = 256;  // 4 sequences per workgroup

template <int SRC_DT, int CACHE_DT>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    const void* c_kv, const void* k_r, const int32_t* positions, void* rows, float* row_scale,
    const int32_t* block_table, int32_t max_pages, int32_t paged, int64_t seq_stride, int ring,
    int B) {
  const int b = blockIdx.x * (kAppendThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= B) return;
  const int64_t t = positions[b];
  const int64_t capacity = paged ? static_cast<int64_t>(max_pages) * kPageSize : seq_stride;
  if (t < 0 || (!ring && t >= capacity)) return;  // a ring overwrites, it has no end
  int64_t row;
  if (paged) {
    const int64_t page = block_table[static_cast<int64_t>(b) * max_pages + (t >> 6)];
    if (page < 0) return;
    row = page * kPageSize + (t & 63);
  } else {
    row = static_cast<int64_t>(b) * seq_stride + (ring ? t % seq_stride : t);
  }
  constexpr int kPer = kRowElems / 64;  // 9
  float x[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + 64 * j;
    x[j] = e < kDLatent ? load_elem<SRC_DT>(c_kv, static_cast<int64_t>(b) * kDLatent + e)
                        : load_elem<SRC_DT>(k_r, static_cast<int64_t>(b) * kDRope + (e - kDLatent));
  }
  const int64_t base = row * kRowElems;
  if constexpr (CACHE_DT == MLA_FP8_E4M3) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float sc = fmaxf(amax, 0x1p-126f) / 448.0f;
    uint8_t* dst = static_cast<uint8_t*>(rows) + base;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float y = fminf(fmaxf(x[j] / sc, -448.0f), 448.0f);
      dst[lane + 64 * j] = static_cast<uint8_t>(e4m3_encode(y));
    }
    if (lane == 0) row_scale[row] = sc;
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) store_elem<CACHE_DT>(rows, base + lane + 64 * j, x[j]);
  }
}

// Ring grow: workgroup (b, y) copies rows k = 16y .. 16y+15 of sequence b's
// live window, the last `keep` tokens, token t = L - keep + k from row t % Cs
// of the source ring to row t % Cd of the destination, as 16-byte chunks
// (and the row factor of an fp8 cache).
constexpr int kGrowThreads = 256;
constexpr int kGrowRows = 16;

__global__ __launch_bounds__(kGrowThreads) void ring_grow_kernel(
    const uint8_t* src, const float* src_scale, int64_t src_cap, uint8_t* dst, float* dst_scale,
    int64_t dst_cap, const int32_t* seq_lens, int max_seq_len, int row_chunks) {
  const int b = blockIdx.x;
  const int64_t L = min(max(seq_lens[b], 0), max_seq_len);
  const int64_t keep = min(L, min(src_cap, dst_cap));
  const int64_t row_bytes = static_cast<int64_t>(row_chunks) * 16;
  for (int idx = threadIdx.x; idx < kGrowRows * row_chunks; idx += kGrowThreads) {
    const int64_t k = static_cast<int64_t>(blockIdx.y) * kGrowRows + idx / row_chunks;
    const int c = idx % row_chunks;
    if (k >= keep) continue;
    const int64_t t = L - keep + k;
    const int64_t rs = static_cast<int64_t>(b) * src_cap + t % src_cap;
    const int64_t rd = static_cast<int64_t>(b) * dst_cap + t % dst_cap;
    *reinterpret_cast<u32x4_t*>(dst + rd * row_bytes + 16 * c) =
        *reinterpret_cast<const u32x4_t*>(src + rs * row_bytes + 16 * c);
    if (c == 0 && dst_scale) dst_scale[rd] = src_scale[rs];
  }
}

mla_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_E_HIP;
}

}  // namespace
}  // namespace mla

using namespace mla;

// ================================================================ entry points

static mla_status_t absorb_launch(const mla_dims_t* dims, int32_t B, const void* q_nope,
                                  const void* q_rope, int32_t q_dt, const void* w_uk, int32_t w_dt,
                                  void* q_abs, int32_t q_abs_dt, float* q_abs_scale,
                                  const RopeArgs& R, hipStream_t s) {
  const int H = dims->heads, dn = dims->d_nope;
  if (q_abs_dt == MLA_FP8_E4M3) {  // bf16 inputs only, whole W_UK[h] in LDS
    if (q_dt != MLA_BF16 || w_dt != MLA_BF16 || dn % 16 != 0 || dn > 128 || !q_abs_scale ||
        reinterpret_cast<uintptr_t>(q_nope) % 16 != 0 || reinterpret_cast<uintptr_t>(w_uk) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(q_rope) % 16 != 0)
      return MLA_E_UNSUPPORTED;
    const dim3 grid(H, (B + 31) / 32);
    absorb_f8_kernel<<<grid, kAf8Threads, 0, s>>>(
        static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope),
        static_cast<const uint16_t*>(w_uk), static_cast<uint8_t*>(q_abs), q_abs_scale, B, H, dn, R);
    return launch_status();
  }
  if (q_dt == MLA_BF16 && w_dt == MLA_BF16 && dn % 16 == 0 &&
      (q_abs_dt == MLA_BF16 || q_abs_dt == MLA_F32) &&
      reinterpret_cast<uintptr_t>(q_nope) % 16 == 0 && reinterpret_cast<uintptr_t>(w_uk) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(q_rope) % 16 == 0) {
    const dim3 g2(H, kDLatent / 128);
    if (q_abs_dt == MLA_BF16)
      absorb_mfma_kernel<MLA_BF16><<<g2, kProjThreads, 0, s>>>(
          static_cast<const uint16_t*>(q_nope), q_rope, static_cast<const uint16_t*>(w_uk), q_abs, B, H, dn, R);
    else
      absorb_mfma_kernel<MLA_F32><<<g2, kProjThreads, 0, s>>>(
          static_cast<const uint16_t*>(q_nope), q_rope, static_cast<const uint16_t*>(w_uk), q_abs, B, H, dn, R);
    return launch_status();
  }
  const dim3 grid(dims->heads, (B + kAbsBatch - 1) / kAbsBatch);
#define MLA_ABS(QD, WD, OD)                                                                     \
  if (q_dt == QD && w_dt == WD && q_abs_dt == OD) {                                             \
    absorb_kernel<QD, WD, OD><<<grid, kAbsThreads, 0, s>>>(q_nope, q_rope, w_uk, q_abs,         \
                                                           nullptr, B, H, dn, R);               \
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

extern "C" mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t B, const void* q_nope,
                                     const void* q_rope, int32_t q_dt, const void* w_uk,
                                     int32_t w_dt, void* q_abs, int32_t q_abs_dt,
                                     float* q_abs_scale, void* stream) {
  mla_status_t st = check_absorb(dims, B, q_nope, q_rope, q_dt, w_uk, w_dt, q_abs, q_abs_dt,
                                 q_abs_scale);
  if (st != MLA_OK || B == 0) return st;
  RopeArgs R{};
  R.positions = nullptr;
  return absorb_launch(dims, B, q_nope, q_rope, q_dt, w_uk, w_dt, q_abs, q_abs_dt, q_abs_scale, R,
                       static_cast<hipStream_t>(stream));
}

extern "C" mla_status_t mla_absorb_q_rope(const mla_dims_t* dims, int32_t B, const void* q_nope,
                                          const void* q_rope, int32_t q_dt, const void* w_uk,
                                          int32_t w_dt, const int32_t* positions, float rope_base,
                                          void* q_abs, int32_t q_abs_dt, void* stream) {
  mla_status_t st = check_absorb(dims, B, q_nope, q_rope, q_dt, w_uk, w_dt, q_abs, q_abs_dt,
                                 nullptr);
  if (st != MLA_OK) return st;
  if (!(rope_base > 1.0f) || !(rope_base < INFINITY)) return MLA_E_ARG;
  if (B == 0) return MLA_OK;
  if (!positions) return MLA_E_ARG;
  if (q_abs_dt == MLA_FP8_E4M3) return MLA_E_UNSUPPORTED;
  RopeArgs R{};
  R.positions = positions;
  for (int i = 0; i < kDRope / 2; ++i)
    R.inv_freq[i] = static_cast<float>(std::pow(static_cast<double>(rope_base),
                                                -2.0 * static_cast<double>(i) / kDRope));
  return absorb_launch(dims, B, q_nope, q_rope, q_dt, w_uk, w_dt, q_abs, q_abs_dt, nullptr, R,
                       static_cast<hipStream_t>(stream));
}

static mla_status_t decode_launch(const mla_dims_t* dims, int32_t B, int32_t q_len,
                                  const void* q_abs, int32_t q_abs_dt, const float* q_abs_scale,
                                  const mla_cache_t* cache, int32_t num_splits, void* u_part,
                                  int32_t part_dt, float* lse_part, int32_t kernel, hipStream_t s) {
  const int32_t H = dims->heads;
  // with max_seq_len == 0 every range is empty; a chunk of 32 keeps the
  // kernels' range arithmetic well defined
  // a ring attends at most seq_stride tokens per sequence
  const int32_t span = cache->ring ? static_cast<int32_t>(min(static_cast<int64_t>(cache->max_seq_len),
                                                              cache->seq_stride))
                                   : cache->max_seq_len;
  const int32_t chunk = max(split_chunk(span, num_splits), kTileTokens);
  const float scale = effective_scale(dims);
  if (cache->ring && q_len != 1) return MLA_E_UNSUPPORTED;
  // values 2 and 3 named the retired 128-head workgroups
  if (kernel == 2 || kernel == 3) return MLA_E_UNSUPPORTED;
  if (kernel != MLA_KERNEL_AUTO && kernel != MLA_KERNEL_H64 && kernel != MLA_KERNEL_H64_BALANCED)
    return MLA_E_ARG;
  if (cache->dtype == MLA_F32) {
    if (q_len != 1 || kernel == MLA_KERNEL_H64_BALANCED) return MLA_E_UNSUPPORTED;
    DecodeF32Params P{static_cast<const float*>(q_abs), static_cast<const float*>(cache->rows),
                      cache->block_table, cache->seq_lens, cache->seq_stride, cache->max_pages,
                      cache->page_size != 0, B, H, num_splits, chunk, cache->max_seq_len, scale,
                      u_part, lse_part, cache->ring};
    const int64_t nblk = static_cast<int64_t>(B) * num_splits * H;
    if (nblk > 0x7FFFFFFF) return MLA_E_SHAPE;
    if (part_dt == MLA_F32)
      decode_f32_kernel<MLA_F32><<<static_cast<unsigned>(nblk), kF32Threads, 0, s>>>(P);
    else
      decode_f32_kernel<MLA_BF16><<<static_cast<unsigned>(nblk), kF32Threads, 0, s>>>(P);
    return launch_status();
  }
  // workgroups of 64 heads of one query token
  const int32_t HG64 = (H + kH64 - 1) / kH64;
  if (q_abs_dt == MLA_FP8_E4M3) {  // fp8 cache and query: 64-token tiles on the fp8 matrix cores
    if (kernel != MLA_KERNEL_AUTO && kernel != MLA_KERNEL_H64) return MLA_E_UNSUPPORTED;
    const int32_t per = 2 * kTileTokens * num_splits;
    const int32_t chunk64 = max((span + per - 1) / per, 1) * (2 * kTileTokens);
    DecodeParams Q{q_abs, static_cast<const uint8_t*>(cache->rows), cache->row_scale,
                   cache->block_table, cache->seq_lens, cache->seq_stride, cache->max_pages,
                   cache->page_size != 0, B, H, num_splits, HG64, chunk64, cache->max_seq_len,
                   q_len, scale * kLog2e, u_part, lse_part, cache->ring, q_abs_scale, num_splits};
    return decode_fp8q_launch(Q, part_dt, s);
  }
  const int64_t nblk64 = static_cast<int64_t>(B) * q_len * num_splits * HG64;
  if (nblk64 > 0x7FFFFFFF) return MLA_E_SHAPE;
  const unsigned grid64 = static_cast<unsigned>(nblk64);
  DecodeParams P{q_abs, static_cast<const uint8_t*>(cache->rows), cache->row_scale,
                 cache->block_table, cache->seq_lens, cache->seq_stride, cache->max_pages,
                 cache->page_size != 0, B, H, num_splits, HG64, chunk, cache->max_seq_len,
                 q_len, scale * kLog2e, u_part, lse_part, cache->ring, nullptr, num_splits};
  const bool fp8 = cache->dtype == MLA_FP8_E4M3;
  // balanced partition (bf16 cache): one worker of HG64 workgroups per two
  // CUs' worth of 64-head workgroups (256 workgroups of 64 heads in all, one
  // per CU), each taking an equal share of the batch's tiles
  if (kernel == MLA_KERNEL_H64_BALANCED) {
    const int64_t V = static_cast<int64_t>(B) * q_len;
    const int64_t tiles_max =
        V * ((static_cast<int64_t>(span) + kTileTokens - 1) / kTileTokens + kRowStartTiles);
    if (fp8 || num_splits < 2 || V > kBalancedMaxRows || tiles_max > 0x7FFFFFFF)
      return MLA_E_UNSUPPORTED;
    if (V == 0) return MLA_OK;
    const unsigned gridB = static_cast<unsigned>(max(1, kBalancedWorkgroups / HG64) * HG64);
    if (part_dt == MLA_F32)
      decode_ws_kernel<false, MLA_F32, true><<<gridB, kWsThreads, 0, s>>>(P, cache->block_table);
    else
      decode_ws_kernel<false, MLA_BF16, true><<<gridB, kWsThreads, 0, s>>>(P, cache->block_table);
    return launch_status();
  }
  // automatic choice: the 64-head kernel over the fixed split ranges
  if (kernel == MLA_KERNEL_AUTO) kernel = MLA_KERNEL_H64;
  // bf16 cache with many splits per sequence (S >= 32): R consecutive split
  // ranges per workgroup, enough workgroups to fill the 256 CUs once, merged
  // into one range: the workgroup streams their tokens with one softmax and
  // writes one partial, to slot g of its group g; slots from ceil(S / R) on
  // hold lse = -inf.  Fewer splits (long ranges, ragged batches) keep one
  // range per workgroup, so that the dispatcher balances ranges of different
  // lengths; the fp8 (widening) kernel always runs one.
  int R = 1;
  if (!fp8 && num_splits >= 32) {
    const int64_t per_cu = nblk64 / 256;
    R = static_cast<int>(per_cu < 1 ? 1 : (per_cu > num_splits ? num_splits : per_cu));
  }
  P.S = (num_splits + R - 1) / R;
  P.chunk = chunk * R;
  const unsigned gridR = static_cast<unsigned>(static_cast<int64_t>(B) * q_len * P.S * HG64);
  if (fp8 && part_dt == MLA_F32)
    decode_ws_kernel<true, MLA_F32><<<grid64, kWsThreads, 0, s>>>(P, cache->block_table);
  else if (fp8)
    decode_ws_kernel<true, MLA_BF16><<<grid64, kWsThreads, 0, s>>>(P, cache->block_table);
  else if (part_dt == MLA_F32)
    decode_ws_kernel<false, MLA_F32><<<gridR, kWsThreads, 0, s>>>(P, cache->block_table);
  else
    decode_ws_kernel<false, MLA_BF16><<<gridR, kWsThreads, 0, s>>>(P, cache->block_table);
  return launch_status();
}

extern "C" mla_status_t mla_decode(const mla_dims_t* dims, int32_t B, const void* q_abs,
                                   int32_t q_abs_dt, const float* q_abs_scale,
                                   const mla_cache_t* cache, int32_t num_splits, void* u_part,
                                   int32_t part_dt, float* lse_part, void* stream) {
  mla_status_t st = check_decode(dims, B, q_abs, q_abs_dt, q_abs_scale, cache, num_splits,
                                 u_part, part_dt, lse_part);
  if (st != MLA_OK || B == 0) return st;
  return decode_launch(dims, B, 1, q_abs, q_abs_dt, q_abs_scale, cache, num_splits, u_part,
                       part_dt, lse_part, MLA_KERNEL_AUTO, static_cast<hipStream_t>(stream));
}

extern "C" mla_status_t mla_decode_multi(const mla_dims_t* dims, int32_t B, int32_t q_len,
                                         const void* q_abs, int32_t q_abs_dt,
                                         const mla_cache_t* cache, int32_t num_splits,
                                         void* u_part, int32_t part_dt, float* lse_part,
                                         void* stream) {
  if (q_len < 1 || q_len > kMaxQueryTokens) return MLA_E_ARG;
  mla_status_t st = check_decode(dims, B, q_abs, q_abs_dt, nullptr, cache, num_splits, u_part,
                                 part_dt, lse_part);
  if (st != MLA_OK || B == 0) return st;
  if (static_cast<int64_t>(B) * q_len > 0x7FFFFFFF) return MLA_E_SHAPE;
  return decode_launch(dims, B, q_len, q_abs, q_abs_dt, nullptr, cache, num_splits, u_part,
                       part_dt, lse_part, MLA_KERNEL_AUTO, static_cast<hipStream_t>(stream));
}

extern "C" mla_status_t mla_decode_ex(const mla_dims_t* dims, int32_t B, int32_t q_len,
                                      const void* q_abs, int32_t q_abs_dt,
                                      const mla_cache_t* cache, int32_t num_splits,
                                      void* u_part, int32_t part_dt, float* lse_part,
                                      int32_t kernel, void* stream) {
  if (q_len < 1 || q_len > kMaxQueryTokens) return MLA_E_ARG;
  mla_status_t st = check_decode(dims, B, q_abs, q_abs_dt, nullptr, cache, num_splits, u_part,
                                 part_dt, lse_part);
  if (st != MLA_OK || B == 0) return st;
  if (static_cast<int64_t>(B) * q_len > 0x7FFFFFFF) return MLA_E_SHAPE;
  return decode_launch(dims, B, q_len, q_abs, q_abs_dt, nullptr, cache, num_splits, u_part,
                       part_dt, lse_part, kernel, static_cast<hipStream_t>(stream));
}

extern "C" mla_status_t mla_stream_probe(const void* src, int64_t src_bytes, int32_t workgroups,
                                         int32_t tiles, int32_t paired, int32_t* sink,
                                         void* stream) {
  if (!src || !sink || workgroups < 1 || tiles < 1 || (paired && (workgroups & 1)))
    return MLA_E_ARG;
  if (reinterpret_cast<uintptr_t>(src) % 16) return MLA_E_ALIGN;
  const int64_t streams = paired ? workgroups / 2 : workgroups;
  if (src_bytes < 0 || streams * tiles > src_bytes / kTileBytes) return MLA_E_SHAPE;
  stream_probe_kernel<<<workgroups, kWsThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t*>(src), tiles, paired ? 1 : 0, sink);
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
  const unsigned grid = static_cast<unsigned>(nblk);
#define MLA_COMB(PD, UD)                                                                       \
  if (part_dt == PD && u_dt == UD) {                                                           \
    combine_kernel<PD, UD><<<grid, kCombThreads, 0, s>>>(u_part, lse_part, u, lse, H,          \
                                                         num_splits);                          \
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
  if (u_dt == MLA_BF16 && w_dt == MLA_BF16 && reinterpret_cast<uintptr_t>(u) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(w_uv) % 16 == 0) {
    const dim3 g2(H, (dv + 63) / 64);
    if (o_dt == MLA_BF16)
      up_proj_mfma_kernel<MLA_BF16><<<g2, kUpThreads, 0, s>>>(
          static_cast<const uint16_t*>(u), static_cast<const uint16_t*>(w_uv), o, B, H, dv);
    else
      up_proj_mfma_kernel<MLA_F32><<<g2, kUpThreads, 0, s>>>(
          static_cast<const uint16_t*>(u), static_cast<const uint16_t*>(w_uv), o, B, H, dv);
    return launch_status();
  }
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

static mla_status_t combine_up_launch(const mla_dims_t* dims, int32_t B, int32_t num_splits,
                                      const void* u_part, int32_t part_dt, const float* lse_part,
                                      const void* w_uv, void* o, int32_t o_dt, void* u, float* lse,
                                      hipStream_t s) {
  const int H = dims->heads;
  // sequences per workgroup: 16, halved while the grid would not cover the
  // 256 CUs (small batches)
  int rows = kCuRows;
  while (rows > 1 && static_cast<int64_t>(H) * ((B + rows - 1) / rows) < 256) rows >>= 1;
  // one sequence per workgroup and still fewer workgroups than CUs (B = 1 at
  // 128 heads): two workgroups per (head, sequence), each with half the value rows
  const int vsplit = (static_cast<int64_t>(H) * B < 256 && dims->d_v >= 32) ? 2 : 1;  // VS
  const int64_t nblk = static_cast<int64_t>(H) * ((B + rows - 1) / rows) * vsplit;
  if (nblk > 0x7FFFFFFF) return MLA_E_SHAPE;
  const unsigned grid = static_cast<unsigned>(nblk);
  // one workgroup per CU holds the W_UV rows from the start; a larger grid
  // runs two per CU with them loaded after the merge (fewer registers)
  const bool early_w = nblk <= 256;
  uint16_t* ub = static_cast<uint16_t*>(u);
  const uint16_t* w = static_cast<const uint16_t*>(w_uv);
#define MLA_CU_K(PD, OD, EW)                                                                       \
  if (vsplit == 2 && num_splits <= 32)                                                             \
    combine_up_kernel<PD, OD, 2, 1, EW><<<grid, kCuThreads, 0, s>>>(u_part, lse_part, w, o, ub, lse, \
                                                                    B, H, num_splits, dims->d_v, rows); \
  else if (vsplit == 2)                                                                            \
    combine_up_kernel<PD, OD, 2, 8, EW><<<grid, kCuThreads, 0, s>>>(u_part, lse_part, w, o, ub, lse, \
                                                                    B, H, num_splits, dims->d_v, rows); \
  else if (num_splits <= 32)                                                                       \
    combine_up_kernel<PD, OD, 1, 1, EW><<<grid, kCuThreads, 0, s>>>(u_part, lse_part, w, o, ub, lse, \
                                                                    B, H, num_splits, dims->d_v, rows); \
  else                                                                                             \
    combine_up_kernel<PD, OD, 1, 8, EW><<<grid, kCuThreads, 0, s>>>(u_part, lse_part, w, o, ub, lse, \
                                                                    B, H, num_splits, dims->d_v, rows);
#define MLA_CU(PD, OD)                                                                             \
  if (part_dt == PD && o_dt == OD) {                                                               \
    if (early_w) {                                                                                 \
      MLA_CU_K(PD, OD, true)                                                                       \
    } else {                                                                                       \
      MLA_CU_K(PD, OD, false)                                                                      \
    }                                                                                              \
    return launch_status();                                                                        \
  }
  MLA_CU(MLA_BF16, MLA_BF16)
  MLA_CU(MLA_BF16, MLA_F32)
  MLA_CU(MLA_F32, MLA_BF16)
  MLA_CU(MLA_F32, MLA_F32)
#undef MLA_CU
#undef MLA_CU_K
  return MLA_E_DTYPE;
}

extern "C" mla_status_t mla_combine_up_proj(const mla_dims_t* dims, int32_t B, int32_t num_splits,
                                            const void* u_part, int32_t part_dt,
                                            const float* lse_part, const void* w_uv, int32_t w_dt,
                                            void* o, int32_t o_dt, void* u, float* lse,
                                            void* stream) {
  mla_status_t st = check_combine_up_proj(dims, B, num_splits, u_part, part_dt, lse_part, w_uv,
                                          w_dt, o, o_dt, u);
  if (st != MLA_OK || B == 0) return st;
  return combine_up_launch(dims, B, num_splits, u_part, part_dt, lse_part, w_uv, o, o_dt, u, lse,
                           static_cast<hipStream_t>(stream));
}

// ================================================================ no-allocation decode + tail
//
// Callers that cannot allocate (code under HIP graph capture, serving loops
// that forbid hipMalloc) get the split partials in a buffer the library owns:
// a file-scope device array, one copy per GPU, held until the process ends.
// In host code `scratch` only names the symbol; its device address on the
// current GPU is looked up once per device (hipGetSymbolAddress) and only that
// address is passed to kernels.  Layout: bf16 partials [rows][512], then the
// fp32 log-sum-exps [rows], rows = B * num_splits * heads <= kScratchRows.

constexpr int64_t kScratchRows = 65536;
constexpr int64_t kScratchPartBytes = kScratchRows * kDLatent * 2;  // 64 MiB
constexpr int64_t kScratchBytes = kScratchPartBytes + kScratchRows * 4;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// device address of this GPU's scratch array, looked up on the first call on
// the device (with that device current); nullptr if the lookup failed
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchSlot& sl = g_scratch[dev];
  std::call_once(sl.once, [&sl] {
    void* p = nullptr;
    sl.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (sl.err == hipSuccess) sl.ptr = p;
  });
  return sl.err == hipSuccess ? sl.ptr : nullptr;
}
}  // namespace

extern "C" mla_status_t mla_decode_combine_up_proj_noalloc(
    const mla_dims_t* dims, int32_t B, const void* q_abs, int32_t q_abs_dt,
    const mla_cache_t* cache, int32_t num_splits, const void* w_uv, int32_t w_dt, void* o,
    int32_t o_dt, void* u, float* lse, void* stream) {
  // the partial buffers are the library's: validate with a stand-in address
  // (any 256-byte aligned non-null value) and substitute the real one after
  const void* stand_in = reinterpret_cast<const void*>(static_cast<uintptr_t>(256));
  mla_status_t st = check_decode(dims, B, q_abs, q_abs_dt, nullptr, cache, num_splits, stand_in,
                                 MLA_BF16, static_cast<const float*>(stand_in));
  if (st != MLA_OK) return st;
  st = check_combine_up_proj(dims, B, num_splits, stand_in, MLA_BF16,
                             static_cast<const float*>(stand_in), w_uv, w_dt, o, o_dt, u);
  if (st != MLA_OK || B == 0) return st;
  if (static_cast<int64_t>(B) * num_splits * dims->heads > kScratchRows) return MLA_E_SCRATCH;
  uint8_t* base = static_cast<uint8_t*>(scratch_on_current_device());
  if (!base) return MLA_E_HIP;
  void* u_part = base;
  float* lse_part = reinterpret_cast<float*>(base + kScratchPartBytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the decode writes every (sequence, split, head) row it is asked for (an
  // empty range writes u = 0 and lse = -inf), so nothing needs clearing
  st = decode_launch(dims, B, 1, q_abs, q_abs_dt, nullptr, cache, num_splits, u_part, MLA_BF16,
                     lse_part, MLA_KERNEL_AUTO, s);
  if (st != MLA_OK) return st;
  return combine_up_launch(dims, B, num_splits, u_part, MLA_BF16, lse_part, w_uv, o, o_dt, u, lse,
                           s);
}

extern "C" mla_status_t mla_cache_append(const mla_dims_t* dims, int32_t B, const void* c_kv,
                                         const void* k_r, int32_t src_dt,
                                         const int32_t* positions, const mla_cache_t* cache,
                                         void* stream) {
  mla_status_t st = check_cache_append(dims, B, c_kv, k_r, src_dt, positions, cache);
  if (st != MLA_OK || B == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = static_cast<unsigned>((B + kAppendThreads / 64 - 1) / (kAppendThreads / 64));
  // the cache is written through: the caller passes writable buffers
  void* rows = const_cast<void*>(cache->rows);
  float* scale = const_cast<float*>(cache->row_scale);
  const int32_t paged = cache->page_size != 0;
#define MLA_AP(SD, CD)                                                                          \
  if (src_dt == SD && cache->dtype == CD) {                                                    \
    append_kernel<SD, CD><<<grid, kAppendThreads, 0, s>>>(c_kv, k_r, positions, rows, scale,   \
                                                          cache->block_table, cache->max_pages, \
                                                          paged, cache->seq_stride, cache->ring, B); \
    return launch_status();                                                                   \
  }
  MLA_AP(MLA_F32, MLA_F32)
  MLA_AP(MLA_F32, MLA_BF16)
  MLA_AP(MLA_F32, MLA_FP8_E4M3)
  MLA_AP(MLA_BF16, MLA_F32)
  MLA_AP(MLA_BF16, MLA_BF16)
  MLA_AP(MLA_BF16, MLA_FP8_E4M3)
#undef MLA_AP
  return MLA_E_DTYPE;
}

extern "C" mla_status_t mla_cache_ring_grow(int32_t B, const mla_cache_t* src,
                                            const mla_cache_t* dst, void* stream) {
  mla_status_t st = check_ring_grow(B, src, dst);
  if (st != MLA_OK || B == 0) return st;
  const int64_t keep = min(static_cast<int64_t>(src->max_seq_len),
                           min(src->seq_stride, dst->seq_stride));
  if (keep == 0) return MLA_OK;
  const int64_t ys = (keep + kGrowRows - 1) / kGrowRows;
  if (ys > 65535) return MLA_E_SHAPE;
  const int row_chunks = kRowElems * dtype_bytes(src->dtype) / 16;
  const dim3 grid(static_cast<unsigned>(B), static_cast<unsigned>(ys));
  ring_grow_kernel<<<grid, kGrowThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t*>(src->rows), src->row_scale, src->seq_stride,
      static_cast<uint8_t*>(const_cast<void*>(dst->rows)), const_cast<float*>(dst->row_scale),
      dst->seq_stride, src->seq_lens, src->max_seq_len, row_chunks);
  return launch_status();
}

extern "C" mla_status_t mla_gqa_decode(int32_t B, int32_t heads, int32_t kv_heads,
                                       int32_t d_head, const void* q, const void* k_cache,
                                       const void* v_cache, int32_t dt, const int32_t* seq_lens,
                                       int64_t seq_stride, int32_t max_seq_len,
                                       float softmax_scale, void* o, int32_t o_dt, float* lse,
                                       void* stream) {
  mla_status_t st = check_mha_decode(B, heads, d_head, q, k_cache, v_cache, dt, seq_lens,
                                     seq_stride, max_seq_len, softmax_scale, o, o_dt);
  if (st != MLA_OK) return st;
  if (kv_heads < 1 || heads % kv_heads != 0) return MLA_E_ARG;
  if (B == 0) return MLA_OK;
  const int64_t nblk = static_cast<int64_t>(B) * heads;
  if (nblk > 0x7FFFFFFF) return MLA_E_SHAPE;
  const int G = heads / kv_heads;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(d_head));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* qp = static_cast<const uint16_t*>(q);
  const auto* kp = static_cast<const uint16_t*>(k_cache);
  const auto* vp = static_cast<const uint16_t*>(v_cache);
  if (o_dt == MLA_F32)
    mha_decode_kernel<MLA_F32><<<static_cast<unsigned>(nblk), kMhaThreads, 0, s>>>(
        qp, kp, vp, seq_lens, seq_stride, max_seq_len, heads, G, scale * kLog2e, o, lse);
  else
    mha_decode_kernel<MLA_BF16><<<static_cast<unsigned>(nblk), kMhaThreads, 0, s>>>(
        qp, kp, vp, seq_lens, seq_stride, max_seq_len, heads, G, scale * kLog2e, o, lse);
  return launch_status();
}

extern "C" mla_status_t mla_mha_decode(int32_t B, int32_t heads, int32_t d_head, const void* q,
                                       const void* k_cache, const void* v_cache, int32_t dt,
                                       const int32_t* seq_lens, int64_t seq_stride,
                                       int32_t max_seq_len, float softmax_scale, void* o,
                                       int32_t o_dt, float* lse, void* stream) {
  return mla_gqa_decode(B, heads, heads, d_head, q, k_cache, v_cache, dt, seq_lens, seq_stride,
                        max_seq_len, softmax_scale, o, o_dt, lse, stream);
}
