// Block compression + MXFP4 quantisation, and MXFP4 dequantisation.
//
// Method: "Frontier Architecture Decoding Notes (4): DeepSeek V4", section 1
// (the KV is summarised per 4-token block for CSA, up to 128 tokens for HCA)
// and the podcast transcript "DeepSeek-V4.1-Flash: Pushing the Limits of KV
// Cache Compression", cue 16 (MXFP4 main cache). Pooling rule: softmax over
// the block's gate logits, weighted sum of the token latents. Quantisation:
// OCP MX v1.0 MXFP4 (E8M0 per 32, exponent floor(log2 amax) - 2, RNE on the
// E2M1 grid with saturation, sign kept on zero).
//
// The pooled value is computed in float64 with the multiply and the add
// rounded separately, tokens in order, so the decision of every code is taken
// on the same float64 value a plain float64 evaluation produces (the only
// difference left is the last bit of exp()). HBM-bound: one wave reads a
// block's m x d float32 latents with 32-byte loads per lane.
#include "csa_internal.h"

#pragma clang fp contract(off)

namespace {

// Pools the n tokens of one block over this lane's 8 channels: gate_at(j) is
// token j's gate logit, row_at(j, a, c) loads its 8 channels.
template <class GateAt, class RowAt>
__device__ inline void pool8(int n, GateAt gate_at, RowAt row_at, double p[8]) {
  double gmax = (double)gate_at(0);
  for (int j = 1; j < n; ++j) gmax = fmax(gmax, (double)gate_at(j));
  double den = exp((double)gate_at(0) - gmax);
  for (int j = 1; j < n; ++j) den = den + exp((double)gate_at(j) - gmax);
  {
    const double w0 = exp((double)gate_at(0) - gmax) / den;
    float4 a, c;
    row_at(0, a, c);
    p[0] = w0 * (double)a.x; p[1] = w0 * (double)a.y;
    p[2] = w0 * (double)a.z; p[3] = w0 * (double)a.w;
    p[4] = w0 * (double)c.x; p[5] = w0 * (double)c.y;
    p[6] = w0 * (double)c.z; p[7] = w0 * (double)c.w;
  }
  for (int j = 1; j < n; ++j) {
    const double wj = exp((double)gate_at(j) - gmax) / den;
    float4 a, c;
    row_at(j, a, c);
    p[0] = p[0] + wj * (double)a.x; p[1] = p[1] + wj * (double)a.y;
    p[2] = p[2] + wj * (double)a.z; p[3] = p[3] + wj * (double)a.w;
    p[4] = p[4] + wj * (double)c.x; p[5] = p[5] + wj * (double)c.y;
    p[6] = p[6] + wj * (double)c.z; p[7] = p[7] + wj * (double)c.w;
  }
}

// Lane j of each aligned 4-lane quad receives quad lane J's value.
template <int J>
__device__ inline double quad_bcast(double v) {
  constexpr int CTRL = J | (J << 2) | (J << 4) | (J << 6);  // quad_perm [J,J,J,J]
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

// pool8 for a full 4-token block, the same operations in the same order, with
// the four gate exponentials and weight divisions spread over the lanes of
// each quad (lane j of a quad takes token j) and broadcast back, and every row
// load issued before the arithmetic. The quads of a block's lane group all hold
// the same gates, so each quad computes the weights on its own.
__device__ inline void pool4_quad(const float* __restrict__ g, const float* __restrict__ x,
                                  int64_t ld, int lane, double p[8]) {
  const float gl = g[lane & 3];
  float4 a[4], c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = *reinterpret_cast<const float4*>(x + j * ld);
    c[j] = *reinterpret_cast<const float4*>(x + j * ld + 4);
  }
  const double gd = (double)gl;
  double gmax = fmax(quad_bcast<0>(gd), quad_bcast<1>(gd));
  gmax = fmax(gmax, quad_bcast<2>(gd));
  gmax = fmax(gmax, quad_bcast<3>(gd));
  const double e = exp(gd - gmax);
  double den = quad_bcast<0>(e);
  den = den + quad_bcast<1>(e);
  den = den + quad_bcast<2>(e);
  den = den + quad_bcast<3>(e);
  const double wl = e / den;
  double w[4];
  w[0] = quad_bcast<0>(wl);
  w[1] = quad_bcast<1>(wl);
  w[2] = quad_bcast<2>(wl);
  w[3] = quad_bcast<3>(wl);
  p[0] = w[0] * (double)a[0].x; p[1] = w[0] * (double)a[0].y;
  p[2] = w[0] * (double)a[0].z; p[3] = w[0] * (double)a[0].w;
  p[4] = w[0] * (double)c[0].x; p[5] = w[0] * (double)c[0].y;
  p[6] = w[0] * (double)c[0].z; p[7] = w[0] * (double)c[0].w;
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    p[0] = p[0] + w[j] * (double)a[j].x; p[1] = p[1] + w[j] * (double)a[j].y;
    p[2] = p[2] + w[j] * (double)a[j].z; p[3] = p[3] + w[j] * (double)a[j].w;
    p[4] = p[4] + w[j] * (double)c[j].x; p[5] = p[5] + w[j] * (double)c[j].y;
    p[6] = p[6] + w[j] * (double)c[j].z; p[7] = p[7] + w[j] * (double)c[j].w;
  }
}

// MXFP4 (E8M0 per 32): the 4 lanes of a scale group call it together.
// Returns the 8 packed codes; *sbyte = the scale byte (exponent + 127).
__device__ inline uint32_t quantize8_e8m0(const double p[8], uint32_t* sbyte) {
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmax(amax, fabs(p[i]));
  amax = fmax(amax, __shfl_xor(amax, 1, 64));
  amax = fmax(amax, __shfl_xor(amax, 2, 64));
  int e = -127;
  if (amax > 0.0) {
    int ex;
    (void)frexp(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1)
    e = ex - 1 - 2;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double y = ldexp(p[i], -e);
    const double a = fabs(y);
    uint32_t mag = (a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) +
                   (a >= 3.5) + (a > 5.0);
    uint32_t code = (signbit(y) ? 8u : 0u) | mag;
    word |= code << (4 * i);
  }
  *sbyte = (uint32_t)(e + 127);
  return word;
}

__device__ inline double e4m3_f64(int b) {
  const int e = (b >> 3) & 15, mnt = b & 7;
  return e ? ldexp((double)(8 + mnt), e - 10) : ldexp((double)mnt, -9);
}

// FP4 with one E4M3 scale per 16 channels: the 2 lanes of a scale group call
// it together. The scale is the E4M3 value nearest to amax / 6 (ties to the
// even byte, saturating at 448), found without dividing: a binary search for
// the largest byte with 6 v <= amax, then amax against 3 (v + v_next). The
// codes round to the nearest multiple of the scale by comparing |p| with the
// scale times each midpoint of the E2M1 grid (exact products in float64).
__device__ inline uint32_t quantize8_e4m3(const double p[8], uint32_t* sbyte) {
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmax(amax, fabs(p[i]));
  amax = fmax(amax, __shfl_xor(amax, 1, 64));
  int lo = 0, hi = 0x7E;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (6.0 * e4m3_f64(mid) <= amax) lo = mid;
    else hi = mid - 1;
  }
  int b = lo;
  if (lo < 0x7E) {
    const double mid6 = 3.0 * (e4m3_f64(lo) + e4m3_f64(lo + 1));
    if (amax > mid6 || (amax == mid6 && (lo & 1))) b = lo + 1;
  }
  const double sc = e4m3_f64(b);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double a = fabs(p[i]);
    uint32_t mag = sc == 0.0 ? 0u
                             : (a > sc * 0.25) + (a >= sc * 0.75) + (a > sc * 1.25) +
                                   (a >= sc * 1.75) + (a > sc * 2.5) + (a >= sc * 3.5) +
                                   (a > sc * 5.0);
    uint32_t code = (signbit(p[i]) ? 8u : 0u) | mag;
    word |= code << (4 * i);
  }
  *sbyte = (uint32_t)b;
  return word;
}

// Writes one lane's 8 codes and, from the first lane of its scale group, the
// scale byte of entry `row`.
template <int D, int FMT>
__device__ inline void store_entry(const double p[8], int seg, int64_t row,
                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  uint32_t sb;
  const uint32_t word = FMT == CSA_SCALE_E4M3_16 ? quantize8_e4m3(p, &sb) : quantize8_e8m0(p, &sb);
  *reinterpret_cast<uint32_t*>(codes + row * (D / 2) + seg * 4) = word;
  if (FMT == CSA_SCALE_E4M3_16) {
    if ((seg & 1) == 0) scales[row * (D / 16) + seg / 2] = (uint8_t)sb;
  } else {
    if ((seg & 3) == 0) scales[row * (D / 32) + seg / 4] = (uint8_t)sb;
  }
}

// One lane owns 8 consecutive channels of one block; D/8 lanes cover a block
// row, so a wave holds 64/(D/8) blocks. Grid: x over a sequence's blocks,
// y over sequences. M4: m == 4, full blocks take pool4_quad (D/8 is a
// multiple of 4, so quads never straddle blocks).
template <int D, int FMT, bool M4>
__global__ __launch_bounds__(256) void k_compress_quantize(
    const float* __restrict__ kv, int64_t kv_ld, const float* __restrict__ gate,
    int64_t n_tok, int m, int64_t nblk, int64_t blk_first,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t blk_cap) {
  constexpr int LPB = D / 8;
  constexpr int BPW = 64 / LPB;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t bi = ((int64_t)blockIdx.x * 4 + wave) * BPW + lane / LPB;
  if (bi >= nblk) return;  // whole 4-lane groups leave together
  const int64_t b = blockIdx.y;
  const int64_t j0 = bi * m;
  const int n = (int)((n_tok - j0) < m ? (n_tok - j0) : m);
  const int seg = lane % LPB;
  const float* g = gate + b * n_tok + j0;
  const float* x = kv + (b * n_tok + j0) * kv_ld + seg * 8;
  double p[8];
  if (M4 && n == 4) {
    pool4_quad(g, x, kv_ld, lane, p);
  } else {
    pool8(
        n, [&](int j) { return g[j]; },
        [&](int j, float4& a, float4& c) {
          const float* xj = x + (int64_t)j * kv_ld;
          a = *reinterpret_cast<const float4*>(xj);
          c = *reinterpret_cast<const float4*>(xj + 4);
        },
        p);
  }
  store_entry<D, FMT>(p, seg, b * blk_cap + blk_first + bi, codes, scales);
}

// Decode append: one new token per sequence, at its own position pos[b]
// (sequences with pos[b] < 0 are skipped). The token goes to the bf16 ring
// slot pos % Wcap and, in float32, to the staging row pos % m; when it is the
// block's m-th token the block is pooled from the m staged rows (this token
// from registers) and quantised into entry pos / m, with the same arithmetic
// as k_compress_quantize. Lanes as in k_compress_quantize, one sequence per
// D/8 lanes.
template <int D, int FMT>
__global__ __launch_bounds__(256) void k_decode_append(
    const float* __restrict__ kv, int64_t kv_ld, const float* __restrict__ gate,
    const int64_t* __restrict__ pos, int B, int m, float* __restrict__ stage,
    float* __restrict__ stage_gate, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    int64_t blk_cap, uint16_t* __restrict__ win, int Wcap) {
  constexpr int LPB = D / 8;
  constexpr int BPW = 64 / LPB;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t b = ((int64_t)blockIdx.x * 4 + wave) * BPW + lane / LPB;
  if (b >= B) return;  // whole sequences leave together
  const int64_t t = pos[b];
  const int seg = lane % LPB;
  const float* x = kv + b * kv_ld + seg * 8;
  const float4 xa = *reinterpret_cast<const float4*>(x);
  const float4 xc = *reinterpret_cast<const float4*>(x + 4);
  const float gt = gate[b];
  // m = 4: the block's staged rows and gates are requested with the token, so
  // they need not wait for the position (their addresses do not depend on it;
  // the row this token overwrites is taken from registers below)
  float* st = stage + b * m * D;
  float4 pa[4], pc[4];
  float pg[4];
  if (m == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* sr = st + (int64_t)i * D + seg * 8;
      pa[i] = *reinterpret_cast<const float4*>(sr);
      pc[i] = *reinterpret_cast<const float4*>(sr + 4);
      pg[i] = stage_gate[b * 4 + i];
    }
  }
  if (t < 0) return;

  // bf16 ring row (round to nearest even)
  {
    v8bf v;
    v[0] = (__bf16)xa.x; v[1] = (__bf16)xa.y; v[2] = (__bf16)xa.z; v[3] = (__bf16)xa.w;
    v[4] = (__bf16)xc.x; v[5] = (__bf16)xc.y; v[6] = (__bf16)xc.z; v[7] = (__bf16)xc.w;
    *reinterpret_cast<v8bf*>(win + (b * Wcap + t % Wcap) * D + seg * 8) = v;
  }
  // staging row of the block being filled
  const int j = (int)(t % m);
  {
    float* sr = st + (int64_t)j * D + seg * 8;
    *reinterpret_cast<float4*>(sr) = xa;
    *reinterpret_cast<float4*>(sr + 4) = xc;
    if (seg == 0) stage_gate[b * m + j] = gt;
  }
  if (j != m - 1) return;
  const int64_t blk = t / m;
  if (blk >= blk_cap) return;
  const float* sg = stage_gate + b * m;
  double p[8];
  if (m == 4) {
    // (j == 3 here: the token is the block's last row)
    pool8(
        4, [&](int i) { return i == 3 ? gt : pg[i]; },
        [&](int i, float4& a, float4& c) {
          a = i == 3 ? xa : pa[i];
          c = i == 3 ? xc : pc[i];
        },
        p);
    store_entry<D, FMT>(p, seg, b * blk_cap + blk, codes, scales);
    return;
  }
  pool8(
      m, [&](int i) { return i == j ? gt : sg[i]; },
      [&](int i, float4& a, float4& c) {
        if (i == j) {
          a = xa;
          c = xc;
        } else {
          const float* sr = st + (int64_t)i * D + seg * 8;
          a = *reinterpret_cast<const float4*>(sr);
          c = *reinterpret_cast<const float4*>(sr + 4);
        }
      },
      p);
  store_entry<D, FMT>(p, seg, b * blk_cap + blk, codes, scales);
}

template <int OUT, int FMT>
__global__ __launch_bounds__(256) void k_dequantize(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t blk_cap,
    int64_t blk0, int64_t n_blk, int d, int64_t total, void* __restrict__ out) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= total) return;
  const int segs = d / 8;
  const int64_t row = u / segs;
  const int seg = (int)(u - row * segs);
  const int64_t b = row / n_blk;
  const int64_t bi = row - b * n_blk;
  const int64_t src = b * blk_cap + blk0 + bi;
  const uint32_t word = *reinterpret_cast<const uint32_t*>(codes + src * (d / 2) + seg * 4);
  const bool e4 = FMT == CSA_SCALE_E4M3_16;
  const float sc = e4 ? e4m3_to_f32(scales[src * (d / 16) + seg / 2])
                      : e8m0_to_f32(scales[src * (d / 32) + seg / 4]);
  if (OUT == CSA_BF16) {
    v8bf v = e4 ? fp4x8_to_bf16_mul(word, sc) : fp4x8_to_bf16(word, sc);
    *reinterpret_cast<v8bf*>(reinterpret_cast<__bf16*>(out) + u * 8) = v;
  } else if (OUT == CSA_F16) {
    v8h v = e4 ? fp4x8_to_f16_mul(word, sc) : fp4x8_to_f16(word, sc);
    *reinterpret_cast<v8h*>(reinterpret_cast<_Float16*>(out) + u * 8) = v;
  } else {
    v8bf v = e4 ? fp4x8_to_bf16_mul(word, sc) : fp4x8_to_bf16(word, sc);
    float* o = reinterpret_cast<float*>(out) + u * 8;
    float4 a, c;
    a.x = (float)v[0]; a.y = (float)v[1]; a.z = (float)v[2]; a.w = (float)v[3];
    c.x = (float)v[4]; c.y = (float)v[5]; c.z = (float)v[6]; c.w = (float)v[7];
    reinterpret_cast<float4*>(o)[0] = a;
    reinterpret_cast<float4*>(o)[1] = c;
  }
}

}  // namespace

static inline bool valid_fmt(int f) { return f == CSA_SCALE_E8M0_32 || f == CSA_SCALE_E4M3_16; }

extern "C" int64_t csa_cache_bytes(int64_t n_tokens, int d, int m, int scale_fmt) {
  if (n_tokens < 0 || m < 1 || d <= 0 || d % 32 || !valid_fmt(scale_fmt)) return -1;
  const int sb = scale_fmt == CSA_SCALE_E4M3_16 ? d / 16 : d / 32;
  return ((n_tokens + m - 1) / m) * (int64_t)(d / 2 + sb);
}

extern "C" int csa_compress_quantize(const float* kv, int64_t kv_ld, const float* gate, int B,
                                     int64_t tok0, int64_t n_tok, int d, int m, uint8_t* codes,
                                     uint8_t* scales, int64_t blk_cap, int scale_fmt,
                                     hipStream_t stream) {
  if (!valid_fmt(scale_fmt)) return CSA_ERR_DTYPE;
  if (B < 0 || n_tok < 0 || tok0 < 0 || blk_cap < 0) return CSA_ERR_SHAPE;
  if (m < 1 || m > 128) return CSA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 128 && d != 256 && d != 512) return CSA_ERR_SHAPE;
  if (kv_ld < d || kv_ld % 4) return CSA_ERR_ALIGN;
  if (tok0 % m) return CSA_ERR_RANGE;
  if (B == 0 || n_tok == 0) return CSA_OK;
  if (!kv || !gate || !codes || !scales) return CSA_ERR_NULL;
  if (!csa_aligned(kv, 16) || !csa_aligned(codes, 4)) return CSA_ERR_ALIGN;
  const int64_t blk_first = tok0 / m;
  const int64_t nblk = (n_tok + m - 1) / m;
  if (blk_first + nblk > blk_cap) return CSA_ERR_RANGE;
  const int bpwg = 4 * (64 / (d / 8));
  const int64_t grid = (nblk + bpwg - 1) / bpwg;
  if (grid > 0x7fffffff) return CSA_ERR_SHAPE;
  const int scale_bytes = scale_fmt == CSA_SCALE_E4M3_16 ? d / 16 : d / 32;
  // sequences go on grid y, at most 65535 per launch
  for (int b0 = 0; b0 < B; b0 += 65535) {
    const int nb = B - b0 < 65535 ? B - b0 : 65535;
    const float* kv_b = kv + (int64_t)b0 * n_tok * kv_ld;
    const float* gate_b = gate + (int64_t)b0 * n_tok;
    uint8_t* codes_b = codes + (int64_t)b0 * blk_cap * (d / 2);
    uint8_t* scales_b = scales + (int64_t)b0 * blk_cap * scale_bytes;
#define CSA_LAUNCH_COMPRESS2(DD, FF, M4)                                                   \
  hipLaunchKernelGGL((k_compress_quantize<DD, FF, M4>), dim3((unsigned)grid, (unsigned)nb), \
                     dim3(256), 0, stream, kv_b, kv_ld, gate_b, n_tok, m, nblk, blk_first,  \
                     codes_b, scales_b, blk_cap)
#define CSA_LAUNCH_COMPRESS1(DD, FF)                \
  do {                                              \
    if (m == 4) CSA_LAUNCH_COMPRESS2(DD, FF, true); \
    else CSA_LAUNCH_COMPRESS2(DD, FF, false);       \
  } while (0)
#define CSA_LAUNCH_COMPRESS(DD)                                         \
  if (scale_fmt == CSA_SCALE_E4M3_16) CSA_LAUNCH_COMPRESS1(DD, CSA_SCALE_E4M3_16); \
  else CSA_LAUNCH_COMPRESS1(DD, CSA_SCALE_E8M0_32)
    switch (d) {
      case 32: CSA_LAUNCH_COMPRESS(32); break;
      case 64: CSA_LAUNCH_COMPRESS(64); break;
      case 128: CSA_LAUNCH_COMPRESS(128); break;
      case 256: CSA_LAUNCH_COMPRESS(256); break;
      default: CSA_LAUNCH_COMPRESS(512); break;
    }
#undef CSA_LAUNCH_COMPRESS
#undef CSA_LAUNCH_COMPRESS1
#undef CSA_LAUNCH_COMPRESS2
    CSA_TRY_LAUNCH();
  }
  return CSA_OK;
}

extern "C" int csa_decode_append(const float* kv, int64_t kv_ld, const float* gate,
                                 const int64_t* pos, int B, int d, int m, float* stage,
                                 float* stage_gate, uint8_t* codes, uint8_t* scales,
                                 int64_t blk_cap, uint16_t* win, int Wcap, int scale_fmt,
                                 hipStream_t stream) {
  if (!valid_fmt(scale_fmt)) return CSA_ERR_DTYPE;
  if (B < 0 || blk_cap < 0 || Wcap < 1) return CSA_ERR_SHAPE;
  if (m < 1 || m > 128) return CSA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 128 && d != 256 && d != 512) return CSA_ERR_SHAPE;
  if (kv_ld < d || kv_ld % 4) return CSA_ERR_ALIGN;
  if (B == 0) return CSA_OK;
  if (!kv || !gate || !pos || !stage || !stage_gate || !win) return CSA_ERR_NULL;
  if (blk_cap > 0 && (!codes || !scales)) return CSA_ERR_NULL;
  if (!csa_aligned(kv, 16) || !csa_aligned(stage, 16) || !csa_aligned(win, 16) ||
      !csa_aligned(pos, 8) || (blk_cap > 0 && !csa_aligned(codes, 4)))
    return CSA_ERR_ALIGN;
  const int spw = 4 * (64 / (d / 8));  // sequences per workgroup
  const int grid = (B + spw - 1) / spw;
#define CSA_LAUNCH_APPEND1(DD, FF)                                                          \
  hipLaunchKernelGGL((k_decode_append<DD, FF>), dim3(grid), dim3(256), 0, stream, kv, kv_ld,  \
                     gate, pos, B, m, stage, stage_gate, codes, scales, blk_cap, win, Wcap)
#define CSA_LAUNCH_APPEND(DD)                                                       \
  if (scale_fmt == CSA_SCALE_E4M3_16) CSA_LAUNCH_APPEND1(DD, CSA_SCALE_E4M3_16); \
  else CSA_LAUNCH_APPEND1(DD, CSA_SCALE_E8M0_32)
  switch (d) {
    case 32: CSA_LAUNCH_APPEND(32); break;
    case 64: CSA_LAUNCH_APPEND(64); break;
    case 128: CSA_LAUNCH_APPEND(128); break;
    case 256: CSA_LAUNCH_APPEND(256); break;
    default: CSA_LAUNCH_APPEND(512); break;
  }
#undef CSA_LAUNCH_APPEND
#undef CSA_LAUNCH_APPEND1
  CSA_TRY_LAUNCH();
  return CSA_OK;
}

extern "C" int csa_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t blk_cap, int B,
                              int64_t blk0, int64_t n_blk, int d, void* out, int out_dtype,
                              int scale_fmt, hipStream_t stream) {
  if (!valid_fmt(scale_fmt)) return CSA_ERR_DTYPE;
  if (B < 0 || blk0 < 0 || n_blk < 0 || blk_cap < 0) return CSA_ERR_SHAPE;
  if (d <= 0 || d % 32 || d > 4096) return CSA_ERR_SHAPE;
  if (out_dtype != CSA_BF16 && out_dtype != CSA_F16 && out_dtype != CSA_F32) return CSA_ERR_DTYPE;
  if (blk0 + n_blk > blk_cap) return CSA_ERR_RANGE;
  if (B == 0 || n_blk == 0) return CSA_OK;
  if (!codes || !scales || !out) return CSA_ERR_NULL;
  if (!csa_aligned(codes, 4) || !csa_aligned(out, 16)) return CSA_ERR_ALIGN;
  const int64_t total = (int64_t)B * n_blk * (d / 8);
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7fffffff) return CSA_ERR_SHAPE;
#define CSA_LAUNCH_DEQ(OO)                                                                   \
  if (scale_fmt == CSA_SCALE_E4M3_16)                                                        \
    hipLaunchKernelGGL((k_dequantize<OO, CSA_SCALE_E4M3_16>), dim3((unsigned)grid), dim3(256), \
                       0, stream, codes, scales, blk_cap, blk0, n_blk, d, total, out);        \
  else                                                                                       \
    hipLaunchKernelGGL((k_dequantize<OO, CSA_SCALE_E8M0_32>), dim3((unsigned)grid), dim3(256), \
                       0, stream, codes, scales, blk_cap, blk0, n_blk, d, total, out)
  if (out_dtype == CSA_BF16) {
    CSA_LAUNCH_DEQ(CSA_BF16);
  } else if (out_dtype == CSA_F16) {
    CSA_LAUNCH_DEQ(CSA_F16);
  } else {
    CSA_LAUNCH_DEQ(CSA_F32);
  }
#undef CSA_LAUNCH_DEQ
  CSA_TRY_LAUNCH();
  return CSA_OK;
}
