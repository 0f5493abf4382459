// Device-side helpers shared by the HIP sources of the MLA library (gfx950):
// vector types, element codecs, the XCD-aware work order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_host.h"

namespace mla {

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

// two floats -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), low half first
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  uint32_t r;
  __builtin_memcpy(&r, &v, 4);
  return r;
}

// binary32 -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ inline uint16_t f32_to_bf16(float f) { return static_cast<uint16_t>(pack_bf16x2(f, 0.0f)); }

// 4 OCP E4M3 codes (one 32-bit word, first code in the low byte) -> 4 bf16
// (two words, same order) with v_cvt_scalef32_pk_bf16_fp8 at unit scale.
// Exact: every E4M3 value, subnormals included, is a bf16 value; the two NaN
// codes give NaN.
__device__ inline u32x2_t e4m3x4_to_bf16x4(uint32_t w) {
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  uint32_t x, y;
  __builtin_memcpy(&x, &lo, 4);
  __builtin_memcpy(&y, &hi, 4);
  return u32x2_t{x, y};
}

// Nearest E4M3 code to y (|y| <= 448 after clamping), ties to the even
// mantissa, from the format's spacing: 2^-9 below 2^-6, and 2^(k-3) in the
// binade [2^k, 2^(k+1)).  Scaling |y| by that spacing is exact, so
// v_rndne_f32 makes the decision; a count of 16 is the next binade's first
// value.  The sign is kept (-0 gives 0x80).
__device__ inline uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.0f);
  if (a < 0x1p-6f) return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  int k = static_cast<int>((__float_as_uint(a) >> 23) & 0xFFu) - 127;
  int q = static_cast<int>(__builtin_rintf(__builtin_ldexpf(a, 3 - k)));
  if (q == 16) {
    q = 8;
    ++k;
  }
  return sign | static_cast<uint32_t>(((k + 7) << 3) | (q - 8));
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

// maximum that keeps a NaN (fmaxf drops it): a NaN split log-sum-exp must make
// the merged result NaN, not be skipped
__device__ inline float max_nan(float a, float b) { return (a != a) ? a : ((b != b) ? b : fmaxf(a, b)); }

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

}  // namespace mla
