// Gather attention over selected MXFP4 entries plus the bf16 sliding window.
//
// Method: "Frontier Architecture Decoding Notes (4): DeepSeek V4", section 1
// (top-k compressed blocks, HCA's dense compressed entries, and the newest
// 128 tokens uncompressed, combined) and the podcast transcript
// "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", cue 8
// (every query head reads one shared latent entry) and cue 16 (the FP4 cache
// is dequantised right before attention, no FP4 arithmetic needed).
//
// One workgroup = one query (all H <= 64 heads, 16 per wave) x one range of
// slots; slots are the selected entries followed by the W window tokens, and
// all of them share one softmax. Slots are processed 32 at a time: the
// workgroup gathers the 32 rows, dequantises each value once into LDS in two
// layouts (entry-major bf16 for q.k, channel-major fp16 for p.v), then every
// wave runs S^T = K Q^T (16x16x32 bf16 MFMA, K = d) and O^T += V^T P^T
// (16x16x32 fp16 MFMA, K = 32 slots) with an online softmax whose head index
// is the lane's column in both products, so no register shuffles are needed
// between them. Ranges of slots of one query can be split over workgroups
// (decode); their partial (o, max, sum) are merged in a fixed order.
#include "csa_internal.h"

namespace {

constexpr int CH = 32;                     // slots per LDS chunk
constexpr int VST = 36;                    // channel-major row stride (halfs)
constexpr int SLOT_INVALID = -1;           // slot code: nothing there
// slot code >= 0: compressed block id; <= -2: window ring row (-2 - row)

template <int D, int NW, bool DENSE>
__global__ __launch_bounds__(NW * 64) void k_attn(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int64_t blk_cap, const int32_t* __restrict__ idx, int k,
    int m, const uint16_t* __restrict__ win, int Wcap, int W, int T, int H, int64_t pos0,
    float scale_log2, int nsplit, int spl, void* __restrict__ out, int out_dtype,
    float* __restrict__ lse, float* __restrict__ part_o, float2* __restrict__ part_ml) {
  constexpr int NT = NW * 64;
  constexpr int KST = D + 8;  // entry-major row stride (bf16)
  constexpr int KSTEPS = D / 32;
  constexpr int CT = D / 16;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[CH * KST];
  __shared__ __attribute__((aligned(16))) _Float16 Vs[D * VST];
  __shared__ int s_code[CH];

  const int split = blockIdx.x % nsplit;
  const int qi = blockIdx.x / nsplit;
  const int b = qi / T;
  const int64_t t = pos0 + (qi - b * T);
  int64_t nsel = k;
  if (DENSE) {
    nsel = (t + 1) / m;
    nsel = nsel < blk_cap ? nsel : blk_cap;
  }
  const int64_t n_slots = nsel + W;
  const int64_t s_begin = (int64_t)split * spl;
  const int64_t s_end = (s_begin + spl < n_slots) ? s_begin + spl : n_slots;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int head = wave * 16 + i16;

  v8bf Qop[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    if (head < H)
      Qop[kk] = *reinterpret_cast<const v8bf*>(q + ((int64_t)qi * H + head) * D + 32 * kk + 8 * g);
    else
      Qop[kk] = v8bf{};
  }
  v4f O[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) O[ct] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int64_t c0 = s_begin; c0 < s_end; c0 += CH) {
    if (threadIdx.x < CH) {
      const int64_t slot = c0 + threadIdx.x;
      int code = SLOT_INVALID;
      if (slot < s_end) {
        if (slot < nsel) {
          const int64_t blk = DENSE ? slot : (int64_t)idx[(int64_t)qi * k + slot];
          if (blk >= 0 && blk < blk_cap) code = (int)blk;
        } else {
          const int64_t p = t - W + 1 + (slot - nsel);
          if (p >= 0) code = -2 - (int)(p % Wcap);
        }
      }
      s_code[threadIdx.x] = code;
    }
    __syncthreads();

    // gather + dequantise: task = (group of 4 slots, 16-channel segment)
    for (int task = threadIdx.x; task < 8 * (D / 16); task += NT) {
      const int sg = task / (D / 16);
      const int cs = task - sg * (D / 16);
      v8h vh[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int slot = 4 * sg + u;
        const int code = s_code[slot];
        v8bf k0, k1;
        if (code >= 0) {
          const int64_t row = (int64_t)b * blk_cap + code;
          const uint2 cw = *reinterpret_cast<const uint2*>(codes + row * (D / 2) + cs * 8);
          const float sc = e8m0_to_f32(scales[row * (D / 32) + cs / 2]);
          k0 = fp4x8_to_bf16(cw.x, sc);
          k1 = fp4x8_to_bf16(cw.y, sc);
          vh[u][0] = fp4x8_to_f16(cw.x, sc);
          vh[u][1] = fp4x8_to_f16(cw.y, sc);
        } else if (code <= -2) {
          const uint16_t* src = win + ((int64_t)b * Wcap + (-2 - code)) * D + cs * 16;
          k0 = *reinterpret_cast<const v8bf*>(src);
          k1 = *reinterpret_cast<const v8bf*>(src + 8);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            vh[u][0][i] = (_Float16)(float)k0[i];
            vh[u][1][i] = (_Float16)(float)k1[i];
          }
        } else {
          k0 = v8bf{};
          k1 = v8bf{};
          vh[u][0] = v8h{};
          vh[u][1] = v8h{};
        }
        *reinterpret_cast<v8bf*>(&Ks[slot * KST + cs * 16]) = k0;
        *reinterpret_cast<v8bf*>(&Ks[slot * KST + cs * 16 + 8]) = k1;
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        v4h col;
        col[0] = vh[0][c >> 3][c & 7];
        col[1] = vh[1][c >> 3][c & 7];
        col[2] = vh[2][c >> 3][c & 7];
        col[3] = vh[3][c >> 3][c & 7];
        *reinterpret_cast<v4h*>(&Vs[(cs * 16 + c) * VST + 4 * sg]) = col;
      }
    }
    __syncthreads();

    // S^T[entry][head] for two 16-entry tiles
    v4f S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const v8bf a0 = *reinterpret_cast<const v8bf*>(&Ks[i16 * KST + 32 * kk + 8 * g]);
      const v8bf a1 = *reinterpret_cast<const v8bf*>(&Ks[(16 + i16) * KST + 32 * kk + 8 * g]);
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, Qop[kk], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, Qop[kk], S1, 0, 0, 0);
    }
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = s_code[4 * g + r] != SLOT_INVALID ? S0[r] * scale_log2 : -INFINITY;
      x[4 + r] = s_code[16 + 4 * g + r] != SLOT_INVALID ? S1[r] * scale_log2 : -INFINITY;
    }
    float cmax = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cmax = fmaxf(cmax, x[i]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m_run, cmax);
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    v8h P;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = none ? 0.f : exp2f(x[i] - m_new);
      psum += p;
      P[i] = (_Float16)p;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      O[ct] *= alpha;
      const _Float16* vrow = &Vs[(ct * 16 + i16) * VST];
      const v4h lo = *reinterpret_cast<const v4h*>(vrow + 4 * g);
      const v4h hi = *reinterpret_cast<const v4h*>(vrow + 16 + 4 * g);
      v8h A;
      A[0] = lo[0]; A[1] = lo[1]; A[2] = lo[2]; A[3] = lo[3];
      A[4] = hi[0]; A[5] = hi[1]; A[6] = hi[2]; A[7] = hi[3];
      O[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, P, O[ct], 0, 0, 0);
    }
    __syncthreads();
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (head >= H) return;
  if (nsplit == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t base = ((int64_t)qi * H + head) * D;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = ct * 16 + 4 * g;
      if (out_dtype == CSA_F32) {
        float4 v;
        v.x = O[ct][0] * inv; v.y = O[ct][1] * inv; v.z = O[ct][2] * inv; v.w = O[ct][3] * inv;
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + base + c) = v;
      } else {
        typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
        v4bf v;
        v[0] = (__bf16)(O[ct][0] * inv); v[1] = (__bf16)(O[ct][1] * inv);
        v[2] = (__bf16)(O[ct][2] * inv); v[3] = (__bf16)(O[ct][3] * inv);
        *reinterpret_cast<v4bf*>(reinterpret_cast<__bf16*>(out) + base + c) = v;
      }
    }
    if (lse && g == 0) lse[(int64_t)qi * H + head] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
  } else {
    const int64_t pbase = (((int64_t)qi * nsplit + split) * H + head);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = ct * 16 + 4 * g;
      float4 v;
      v.x = O[ct][0]; v.y = O[ct][1]; v.z = O[ct][2]; v.w = O[ct][3];
      *reinterpret_cast<float4*>(part_o + pbase * D + c) = v;
    }
    if (g == 0) part_ml[pbase] = float2{m_run, l_tot};
  }
}

// Merge of the split partials of one (query, head), splits in index order.
template <int D>
__global__ __launch_bounds__(D / 4) void k_attn_merge(const float* __restrict__ part_o,
                                                      const float2* __restrict__ part_ml,
                                                      int nsplit, int H, void* __restrict__ out,
                                                      int out_dtype, float* __restrict__ lse) {
  const int64_t qh = blockIdx.x;
  const int64_t qi = qh / H;
  const int h = (int)(qh - qi * H);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[(qi * nsplit + s) * H + h].x);
  float L = 0.f;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const float2 ml = part_ml[(qi * nsplit + s) * H + h];
    if (ml.x == -INFINITY) continue;
    const float f = exp2f(ml.x - M);
    L += ml.y * f;
    const float4 o =
        *reinterpret_cast<const float4*>(part_o + ((qi * nsplit + s) * H + h) * D + 4 * threadIdx.x);
    acc.x += o.x * f; acc.y += o.y * f; acc.z += o.z * f; acc.w += o.w * f;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int64_t base = qh * D + 4 * threadIdx.x;
  if (out_dtype == CSA_F32) {
    float4 v;
    v.x = acc.x * inv; v.y = acc.y * inv; v.z = acc.z * inv; v.w = acc.w * inv;
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + base) = v;
  } else {
    typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
    v4bf v;
    v[0] = (__bf16)(acc.x * inv); v[1] = (__bf16)(acc.y * inv);
    v[2] = (__bf16)(acc.z * inv); v[3] = (__bf16)(acc.w * inv);
    *reinterpret_cast<v4bf*>(reinterpret_cast<__bf16*>(out) + base) = v;
  }
  if (lse && threadIdx.x == 0) lse[qh] = (M + log2f(L)) * 0.69314718055994531f;
}

struct AttnPlan {
  int nsplit, spl;
  int64_t ws_bytes;
};

static AttnPlan attn_plan(int B, int T, int H, int d, int64_t n_slots) {
  AttnPlan p;
  if (T >= 16 || n_slots <= 128) {
    p.nsplit = 1;
    p.spl = (int)(((n_slots + CH - 1) / CH) * CH);
    if (p.spl < CH) p.spl = CH;
  } else {
    int64_t spl = (n_slots + 15) / 16;
    spl = ((spl + CH - 1) / CH) * CH;
    if (spl < 128) spl = 128;
    p.spl = (int)spl;
    p.nsplit = (int)((n_slots + spl - 1) / spl);
  }
  p.ws_bytes = 0;
  if (p.nsplit > 1) {
    const int64_t units = (int64_t)B * T * p.nsplit * H;
    p.ws_bytes = units * d * 4 + 256 + units * 8;
  }
  return p;
}

struct AttnArgs {
  const uint16_t* q; const uint8_t* codes; const uint8_t* scales; int64_t blk_cap;
  const int32_t* idx; int k; int m; const uint16_t* win; int Wcap, W, B, T, H, d;
  int64_t pos0; float softmax_scale; void* out; int out_dtype; float* lse; void* ws;
  int64_t ws_bytes; hipStream_t stream;
};

template <int D, bool DENSE>
static void launch_attn(const AttnArgs& a, const AttnPlan& p, float* part_o, float2* part_ml) {
  const int nw = (a.H + 15) / 16;
  const dim3 grid((unsigned)((int64_t)a.B * a.T * p.nsplit));
  const float sl2 = a.softmax_scale * 1.4426950408889634f;
#define CSA_LAUNCH_ATTN(NW)                                                                  \
  hipLaunchKernelGGL((k_attn<D, NW, DENSE>), grid, dim3(NW * 64), 0, a.stream, a.q, a.codes, \
                     a.scales, a.blk_cap, a.idx, a.k, a.m, a.win, a.Wcap, a.W, a.T, a.H, a.pos0, \
                     sl2, p.nsplit, p.spl, a.out, a.out_dtype, a.lse, part_o, part_ml)
  switch (nw) {
    case 1: CSA_LAUNCH_ATTN(1); break;
    case 2: CSA_LAUNCH_ATTN(2); break;
    case 3: CSA_LAUNCH_ATTN(3); break;
    default: CSA_LAUNCH_ATTN(4); break;
  }
#undef CSA_LAUNCH_ATTN
  if (p.nsplit > 1)
    hipLaunchKernelGGL(k_attn_merge<D>, dim3((unsigned)((int64_t)a.B * a.T * a.H)), dim3(D / 4),
                       0, a.stream, part_o, part_ml, p.nsplit, a.H, a.out, a.out_dtype, a.lse);
}

static int attn_run(const AttnArgs& a, bool dense) {
  if (a.B < 0 || a.T < 0 || a.blk_cap < 0 || a.pos0 < 0) return CSA_ERR_SHAPE;
  if (a.d != 128 && a.d != 256 && a.d != 512) return CSA_ERR_SHAPE;
  if (a.H < 1 || a.H > 64) return CSA_ERR_SHAPE;
  if (a.W < 1 || a.Wcap < a.W) return CSA_ERR_SHAPE;
  if ((int64_t)a.Wcap < (int64_t)a.W + a.T - 1) return CSA_ERR_RANGE;
  if (!dense && a.k < 0) return CSA_ERR_SHAPE;
  if (dense && (a.m < 1 || a.m > 1 << 20)) return CSA_ERR_SHAPE;
  if (a.out_dtype != CSA_BF16 && a.out_dtype != CSA_F32) return CSA_ERR_DTYPE;
  if (a.B == 0 || a.T == 0) return CSA_OK;
  if (!a.q || !a.win || !a.out) return CSA_ERR_NULL;
  if (!dense && a.k > 0 && !a.idx) return CSA_ERR_NULL;
  int64_t nsel = a.k;
  if (dense) {
    nsel = (a.pos0 + a.T) / a.m;
    nsel = nsel < a.blk_cap ? nsel : a.blk_cap;
  }
  if (nsel > 0 && (!a.codes || !a.scales)) return CSA_ERR_NULL;
  if (nsel > 0x3fffffff) return CSA_ERR_SHAPE;
  if (!csa_aligned(a.q, 16) || !csa_aligned(a.win, 16) || !csa_aligned(a.out, 16)) return CSA_ERR_ALIGN;
  if (nsel > 0 && !csa_aligned(a.codes, 8)) return CSA_ERR_ALIGN;
  const AttnPlan p = attn_plan(a.B, a.T, a.H, a.d, nsel + a.W);
  if ((int64_t)a.B * a.T * p.nsplit > 0x7fffffffLL) return CSA_ERR_SHAPE;
  float* part_o = nullptr;
  float2* part_ml = nullptr;
  if (p.nsplit > 1) {
    if (!a.ws || a.ws_bytes < p.ws_bytes) return CSA_ERR_WORKSPACE;
    if (!csa_aligned(a.ws, 256)) return CSA_ERR_ALIGN;
    const int64_t units = (int64_t)a.B * a.T * p.nsplit * a.H;
    part_o = reinterpret_cast<float*>(a.ws);
    part_ml = reinterpret_cast<float2*>(reinterpret_cast<char*>(a.ws) +
                                        ((units * a.d * 4 + 255) / 256) * 256);
  }
  if (dense) {
    if (a.d == 128) launch_attn<128, true>(a, p, part_o, part_ml);
    else if (a.d == 256) launch_attn<256, true>(a, p, part_o, part_ml);
    else launch_attn<512, true>(a, p, part_o, part_ml);
  } else {
    if (a.d == 128) launch_attn<128, false>(a, p, part_o, part_ml);
    else if (a.d == 256) launch_attn<256, false>(a, p, part_o, part_ml);
    else launch_attn<512, false>(a, p, part_o, part_ml);
  }
  CSA_TRY_LAUNCH();
  return CSA_OK;
}

}  // namespace

extern "C" int64_t csa_attn_workspace(int B, int T, int H, int d, int64_t n_slots) {
  if (B < 0 || T < 0 || H < 1 || d < 1 || n_slots < 0) return -1;
  return attn_plan(B, T, H, d, n_slots).ws_bytes;
}

extern "C" int csa_sparse_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                               int64_t blk_cap, const int32_t* idx, int k, const uint16_t* win,
                               int Wcap, int W, int B, int T, int H, int d, int64_t pos0,
                               float softmax_scale, void* out, int out_dtype, float* lse,
                               void* workspace, int64_t ws_bytes, hipStream_t stream) {
  AttnArgs a{q, codes, scales, blk_cap, idx, k, 1, win, Wcap, W, B, T, H, d, pos0,
             softmax_scale, out, out_dtype, lse, workspace, ws_bytes, stream};
  return attn_run(a, false);
}

extern "C" int hca_dense_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                              int64_t blk_cap, int m, const uint16_t* win, int Wcap, int W, int B,
                              int T, int H, int d, int64_t pos0, float softmax_scale, void* out,
                              int out_dtype, float* lse, void* workspace, int64_t ws_bytes,
                              hipStream_t stream) {
  AttnArgs a{q, codes, scales, blk_cap, nullptr, 0, m, win, Wcap, W, B, T, H, d, pos0,
             softmax_scale, out, out_dtype, lse, workspace, ws_bytes, stream};
  return attn_run(a, true);
}
