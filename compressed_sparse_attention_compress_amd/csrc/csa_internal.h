// Internal helpers shared by the HIP translation units of libcsa (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned short v8us __attribute__((ext_vector_type(8)));

#define CSA_TRY_LAUNCH()                                   \
  do {                                                     \
    if (hipGetLastError() != hipSuccess) return CSA_ERR_HIP; \
  } while (0)

static inline bool csa_aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// ---------------------------------------------------------------- scans ----

// First query position of sequence b: pos0 for every sequence, or, with
// per-sequence positions, pos[b] clamped into [0, pos0] (pos0 is then the
// bound the launch plan and the workspace were sized for).
__device__ inline int64_t query_base(const int64_t* pos, int64_t pos0, int b) {
  if (!pos) return pos0;
  const int64_t p = pos[b];
  return p < 0 ? 0 : (p > pos0 ? pos0 : p);
}

// Cross-lane moves within a wave by DPP (a few cycles each, against ~130 for
// an LDS-routed shuffle): row_shr:n moves lane i - n to lane i inside each
// row of 16 lanes; row_bcast:15 / row_bcast:31 copy lane 15 of each row /
// lane 31 into the following rows selected by the row mask. Lanes with no
// source (or in rows the mask leaves out) take `fill`.
template <int CTRL, int ROW_MASK>
__device__ inline int dpp_move(int x, int fill) {
  return __builtin_amdgcn_update_dpp(fill, x, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum across the 64 lanes of one wave (Hillis-Steele inside
// each row of 16, then the row totals carried across rows).
__device__ inline int wave_scan_incl(int x) {
  x += dpp_move<0x111, 0xf>(x, 0);  // row_shr:1
  x += dpp_move<0x112, 0xf>(x, 0);  // row_shr:2
  x += dpp_move<0x114, 0xf>(x, 0);  // row_shr:4
  x += dpp_move<0x118, 0xf>(x, 0);  // row_shr:8
  x += dpp_move<0x142, 0xa>(x, 0);  // row_bcast:15 into rows 1 and 3
  x += dpp_move<0x143, 0xc>(x, 0);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Largest / smallest value over the 64 lanes of a wave, in every lane.
// Sum over the wave (every lane gets it).
__device__ inline int wave_sum(int x) { return __builtin_amdgcn_readlane(wave_scan_incl(x), 63); }

__device__ inline int wave_max(int x) {
  constexpr int lo = (int)0x80000000;
  x = max(x, dpp_move<0x111, 0xf>(x, lo));
  x = max(x, dpp_move<0x112, 0xf>(x, lo));
  x = max(x, dpp_move<0x114, 0xf>(x, lo));
  x = max(x, dpp_move<0x118, 0xf>(x, lo));
  x = max(x, dpp_move<0x142, 0xa>(x, lo));
  x = max(x, dpp_move<0x143, 0xc>(x, lo));
  return __builtin_amdgcn_readlane(x, 63);
}
__device__ inline int wave_min(int x) { return -wave_max(-x); }  // (x > INT_MIN)

// Inclusive prefix sum over the NT threads of a workgroup (NT multiple of
// 64). `tmp` must hold NT/64 ints of LDS. Returns the inclusive prefix and
// writes the workgroup total to *total. Contains two barriers.
template <int NT>
__device__ inline int wg_scan_incl(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int x = wave_scan_incl(v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int wv = 0; wv < NT / 64; ++wv) {
    int s = tmp[wv];
    pre += (wv < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return x + pre;
}

// ------------------------------------------------------------ MXFP4 -----

// E8M0 byte -> float32 scale 2^(s-127). Byte 0 is 2^-127, a float32
// subnormal.
__device__ inline float e8m0_to_f32(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// Eight E2M1 codes (a 32-bit word, channel 2i in the low nibble of byte i)
// times 2^(s-127) -> eight bfloat16 values, using the gfx950 scaled FP4
// conversion (exact: every result is representable in bfloat16).
__device__ inline v8bf fp4x8_to_bf16(uint32_t word, float scale) {
  v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
  v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
  v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
  v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
  v8bf r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Same to float16 (exact while the scaled values stay in float16 range).
__device__ inline v8h fp4x8_to_f16(uint32_t word, float scale) {
  v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, scale, 0);
  v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, scale, 1);
  v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, scale, 2);
  v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, scale, 3);
  v8h r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// ---------------------------------------------- FP4 with E4M3 scales -----

// Non-negative OCP E4M3 byte (0 .. 0x7E) -> float32, exact: exponent field
// bits 6..3 (bias 7), mantissa bits 2..0, exponent field 0 subnormal.
__device__ inline float e4m3_to_f32(uint32_t b) {
  const int e = (b >> 3) & 15, mnt = b & 7;
  return e ? ldexpf((float)(8 + mnt), e - 10) : ldexpf((float)mnt, -9);
}

// Eight E2M1 codes times an E4M3 scale. The scale is not a power of two, so
// the codes are converted unscaled and multiplied in float32; E2M1 (2
// significant bits) times E4M3 (4 bits) is exact in float32, bfloat16 and
// float16 over the whole E4M3 range.
__device__ inline v8bf fp4x8_to_bf16_mul(uint32_t word, float scale) {
  const v8bf u = fp4x8_to_bf16(word, 1.0f);
  v8bf r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)((float)u[i] * scale);
  return r;
}

__device__ inline v8h fp4x8_to_f16_mul(uint32_t word, float scale) {
  const v8h u = fp4x8_to_f16(word, 1.0f);
  v8h r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (_Float16)((float)u[i] * scale);
  return r;
}

// Both at once, for the attention staging: the products are formed in
// float16 (exact: at most 5 significant bits, magnitudes 2^-10 .. 2688), and
// the bfloat16 copy is converted from them. (The gfx950 scaled FP4
// conversions use only the exponent of their scale operand, so they cannot
// apply an E4M3 scale themselves.)
__device__ inline void fp4x8_e4m3_both(uint32_t word, _Float16 scale, v8h& h, v8bf& bf) {
  h = fp4x8_to_f16(word, 1.0f) * scale;
#pragma unroll
  for (int i = 0; i < 8; ++i) bf[i] = (__bf16)(float)h[i];
}

// ----------------------------------------------------------- indexer ----

// Monotone (non-decreasing) map of a non-negative int32 score to one of 512
// histogram bins: 0 for 0, otherwise the float32 exponent and top 4 mantissa
// bits (16 bins per octave).
__device__ inline int score_bin512(int s) {
  if (s <= 0) return 0;
  return (int)(__float_as_uint((float)s) >> 19) - 2031;
}

// 256 bins, 8 per octave.
__device__ inline int score_bin256(int s) {
  if (s <= 0) return 0;
  return (int)(__float_as_uint((float)s) >> 20) - 1015;
}
