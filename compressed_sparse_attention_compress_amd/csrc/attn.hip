// Gather attention over selected MXFP4 entries plus the bf16 sliding window.
//
// Method: "Frontier Architecture Decoding Notes (4): DeepSeek V4", section 1
// (top-k compressed blocks, HCA's dense compressed entries, and the newest
// 128 tokens uncompressed, combined) and the podcast transcript
// "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", cue 8
// (every query head reads one shared latent entry) and cue 16 (the FP4 cache
// is dequantised right before attention, no FP4 arithmetic needed).
//
// One workgroup = one query (all H <= 64 heads) x one range of slots; slots
// are the selected entries followed by the W window tokens, and all of them
// share one softmax. Slots are processed 64 at a time: the workgroup gathers
// the 64 rows and dequantises each value once into LDS in two layouts
// (entry-major bf16 for q.k, channel-major fp16 for p.v). Two waves serve
// each group of 16 heads: for q.k each takes 32 of the 64 slots over all d
// channels (S^T = K Q^T, 16x16x32 bf16 MFMA); the pair exchanges its
// per-head maxima and its P^T operands through LDS; for p.v each takes half
// of the d channels over all 64 slots (O^T += V^T P^T, 16x16x32 fp16 MFMA).
// The head index is the lane's column in both products, so no register
// shuffles are needed between them, and every LDS byte of a pass is read by
// four waves at most. O is rescaled only in passes where some head's running
// maximum grew. Ranges of slots of one query can be split over workgroups
// (decode); their partial (o, max, sum) are merged in a fixed order.
#include "csa_internal.h"

#include <type_traits>

namespace {

constexpr int CH = 64;        // slots per staging pass (two 32-slot MFMA k-steps)
// channel-major row stride (halfs): 34 dwords. Measured on the LDS bank
// conflict counter against 36 (and against a store order that pairs
// channels 8 apart), this layout conflicts least.
constexpr int VST = CH + 4;
constexpr int IDX_CAP = 1024; // entry block ids cached in LDS per refill
constexpr float RESCALE_LOG2 = 0.f;  // rescale whenever a head's max grows (see below)

// Raw bytes of the 4 slots of one staging task (16 channels each): an MXFP4
// entry uses lo.x, lo.y (8 code bytes) and lo.z (its scale byte); a window
// token uses lo and hi (16 bf16).
struct RawSlots {
  uint4 lo[4], hi[4];
};

template <int D, int NW, bool DENSE, int FMT>
__global__ __launch_bounds__(NW * 128) void k_attn(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int64_t blk_cap, const int32_t* __restrict__ idx, int k,
    int m, const uint16_t* __restrict__ win, int Wcap, int W, int T, int H, int64_t pos0,
    const int64_t* __restrict__ qpos, float scale_log2, int nsplit, int spl, int n_queries,
    void* __restrict__ out, int out_dtype,
    float* __restrict__ lse, float* __restrict__ part_o, float2* __restrict__ part_ml) {
  constexpr int NWV = 2 * NW;                 // waves: (head group, half)
  constexpr int NT = NWV * 64;
  constexpr int KST = D + 8;                  // entry-major row stride (bf16)
  // 16-byte chunk c of entry row r sits at chunk c ^ ((r >> 4) & 3): a q.k
  // operand load (16 consecutive rows, one chunk) and a staging store (rows
  // 4 apart, 4 row groups) both touch 16 distinct 4-bank groups
  auto ks_at = [](int r, int c) { return r * KST + ((c ^ ((r >> 4) & 3)) << 3); };
  constexpr int KSTEPS = D / 32;              // q.k k-steps of 32 channels
  constexpr int CTH = D / 32;                 // 16-channel output tiles of one half of d
  constexpr int SG = CH / 4;                  // slot groups of 4 per pass
  constexpr int TASKS = SG * (D / 16);
  constexpr int TPT = (TASKS + NT - 1) / NT;  // staging tasks per thread
  __shared__ __attribute__((aligned(16))) __bf16 Ks[CH * KST];
  __shared__ __attribute__((aligned(16))) _Float16 Vs[D * VST];
  __shared__ int s_blk[IDX_CAP];
  __shared__ __attribute__((aligned(16))) v8h s_p[NWV][64];  // each wave's P^T operand
  __shared__ float s_x[NWV][16];                             // per-head max / sum exchange

  // Workgroups are dealt to the 8 XCDs round-robin by id; all splits of a
  // query are mapped onto one XCD so its q rows are fetched from HBM once and
  // then served by that XCD's L2.
  const int xcd = blockIdx.x & 7;
  const int jx = blockIdx.x >> 3;
  const int qi = xcd + 8 * (jx / nsplit);
  const int split = jx % nsplit;
  if (qi >= n_queries) return;
  const int b = qi / T;
  const int64_t t = query_base(qpos, pos0, b) + (qi - b * T);
  int64_t nsel = k;
  if (DENSE) {
    nsel = (t + 1) / m;
    nsel = nsel < blk_cap ? nsel : blk_cap;
  }
  const int64_t n_slots = nsel + W;
  const int64_t s_begin = (int64_t)split * spl;
  const int64_t s_end = (s_begin + spl < n_slots) ? s_begin + spl : n_slots;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hg = wave >> 1, half = wave & 1, partner = wave ^ 1;
  const int i16 = lane & 15, g = lane >> 4;
  const int head = hg * 16 + i16;

  // q rows are loaded after the first entry ids and raw entries have been
  // requested, so that waiting for those does not wait for q as well
  v8bf Qop[KSTEPS];
  bool q_loaded = false;
  auto load_q = [&]() {
    if (q_loaded) return;
    q_loaded = true;
    const int hq = head < H ? head : H - 1;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      Qop[kk] = *reinterpret_cast<const v8bf*>(q + ((int64_t)qi * H + hq) * D + 32 * kk + 8 * g);
  };
  v4f O[CTH];
#pragma unroll
  for (int ct = 0; ct < CTH; ++ct) O[ct] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const uint8_t* cbase = codes + (int64_t)b * blk_cap * (D / 2);
  constexpr bool E4 = FMT == CSA_SCALE_E4M3_16;
  constexpr int SPE = E4 ? D / 16 : D / 32;  // scale bytes per entry
  const uint8_t* sbase = scales + (int64_t)b * blk_cap * SPE;
  const uint16_t* wbase = win + (int64_t)b * Wcap * D;
  const int32_t* ibase = DENSE ? nullptr : idx + (int64_t)qi * k;

  // One homogeneous phase: entries (IS_WIN false) or window tokens, slots
  // [p0, p1). Loads are unconditional (clamped rows), validity is applied to
  // the logits; in the entry phase the next pass's raw bytes are fetched
  // while the current pass is in the matrix cores.
  auto phase = [&](auto is_win_tag, int64_t p0, int64_t p1) {
    constexpr bool IS_WIN = decltype(is_win_tag)::value;
    if (p0 >= p1) return;
    int64_t tab0 = p0;  // first slot whose block id sits in s_blk[0]
    // entry ids of slots [from, from + IDX_CAP) into LDS; all loads issued
    // before the first is used (addresses clamped into the phase)
    auto refill = [&](int64_t from) {
      constexpr int RPT = (IDX_CAP + NT - 1) / NT;
      __syncthreads();
      tab0 = from;
      int64_t v[RPT];
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int64_t sl = from + threadIdx.x + r * NT;
        v[r] = DENSE ? sl : (int64_t)ibase[sl < p1 ? sl : p1 - 1];
      }
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int i = threadIdx.x + r * NT;
        const int64_t sl = from + i;
        if (i < IDX_CAP) s_blk[i] = (sl < p1 && v[r] >= 0 && v[r] < blk_cap) ? (int)v[r] : -1;
      }
      __syncthreads();
    };
    if (!IS_WIN) refill(p0);
    // task -> (slot group sg, 16-channel segment cs), sg fastest across lanes
    // so that the channel-major writes of a wave spread over all LDS banks
    auto load_task = [&](RawSlots& r, int task, int64_t c0) {
      const int sg = (task < TASKS ? task : 0) % SG;
      const int cs = (task < TASKS ? task : 0) / SG;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t sl = c0 + 4 * sg + u;
        if (IS_WIN) {
          int64_t p = t - W + 1 + (sl - nsel);
          p = p < 0 ? 0 : p;
          const uint16_t* src = wbase + (p % Wcap) * D + cs * 16;
          r.lo[u] = *reinterpret_cast<const uint4*>(src);
          r.hi[u] = *reinterpret_cast<const uint4*>(src + 8);
        } else {
          int blk = (sl < p1 && sl - tab0 < IDX_CAP) ? s_blk[sl - tab0] : -1;
          blk = blk < 0 ? 0 : blk;
          const uint2 cw =
              *reinterpret_cast<const uint2*>(cbase + (int64_t)blk * (D / 2) + cs * 8);
          r.lo[u].x = cw.x;
          r.lo[u].y = cw.y;
          r.lo[u].z = sbase[(int64_t)blk * SPE + (E4 ? cs : cs / 2)];
        }
      }
    };
    auto convert_task = [&](const RawSlots& r, int task) {
      const int sg = task % SG;
      const int cs = task / SG;
      v8h vh[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int slot = 4 * sg + u;
        v8bf k0, k1;
        if (IS_WIN) {
          k0 = __builtin_bit_cast(v8bf, r.lo[u]);
          k1 = __builtin_bit_cast(v8bf, r.hi[u]);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            vh[u][0][i] = (_Float16)(float)k0[i];
            vh[u][1][i] = (_Float16)(float)k1[i];
          }
        } else {
          if (E4) {
            const _Float16 sc = (_Float16)e4m3_to_f32(r.lo[u].z & 0xffu);
            fp4x8_e4m3_both(r.lo[u].x, sc, vh[u][0], k0);
            fp4x8_e4m3_both(r.lo[u].y, sc, vh[u][1], k1);
          } else {
            const float sc = e8m0_to_f32(r.lo[u].z & 0xffu);
            k0 = fp4x8_to_bf16(r.lo[u].x, sc);
            k1 = fp4x8_to_bf16(r.lo[u].y, sc);
            vh[u][0] = fp4x8_to_f16(r.lo[u].x, sc);
            vh[u][1] = fp4x8_to_f16(r.lo[u].y, sc);
          }
        }
        *reinterpret_cast<v8bf*>(&Ks[ks_at(slot, 2 * cs)]) = k0;
        *reinterpret_cast<v8bf*>(&Ks[ks_at(slot, 2 * cs + 1)]) = k1;
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
    };
    // prefetch (whole pass ahead) only where the raw bytes are small
    // (entries) and a thread owns at most two tasks; otherwise each task is
    // loaded right before it is converted
    constexpr bool PREFETCH = !IS_WIN && TPT <= 2;
    constexpr int NRAW = PREFETCH ? TPT : 1;
    RawSlots raw[NRAW];
    auto load_all = [&](int64_t c0) {
#pragma unroll
      for (int tt = 0; tt < NRAW; ++tt) load_task(raw[tt], threadIdx.x + tt * NT, c0);
    };
    if (PREFETCH) load_all(p0);
    load_q();
    for (int64_t c0 = p0; c0 < p1; c0 += CH) {
      if (!IS_WIN && c0 + CH > tab0 + IDX_CAP) {
        refill(c0);
        if (PREFETCH) load_all(c0);
      }
      // convert the raw bytes into LDS: entry-major bf16 and channel-major fp16
#pragma unroll
      for (int tt = 0; tt < TPT; ++tt) {
        const int task = threadIdx.x + tt * NT;
        if (task < TASKS) {
          if (PREFETCH) {
            convert_task(raw[tt < NRAW ? tt : 0], task);
          } else {
            load_task(raw[0], task, c0);
            convert_task(raw[0], task);
          }
        }
      }
      // validity of this lane's logit slots: this wave's half, tile et, row 4g + r
      const int64_t h0 = c0 + 32 * half;
      bool ok[2][4];
#pragma unroll
      for (int et = 0; et < 2; ++et)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t sl = h0 + 16 * et + 4 * g + r;
          if (IS_WIN)
            ok[et][r] = sl < p1 && t - W + 1 + (sl - nsel) >= 0;
          else
            ok[et][r] = sl < p1 && s_blk[sl - tab0] >= 0;
        }
      if (PREFETCH && c0 + CH < p1 && c0 + 2 * CH <= tab0 + IDX_CAP) load_all(c0 + CH);
      __syncthreads();

      // S^T[slot][head] for this wave's 32 slots (two independent 16-slot
      // tiles) over all d channels
      v4f S[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
        for (int et = 0; et < 2; ++et) {
          const v8bf a = *reinterpret_cast<const v8bf*>(
              &Ks[ks_at(32 * half + 16 * et + i16, 4 * kk + g)]);
          S[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Qop[kk], S[et], 0, 0, 0);
        }
      float x[2][4];
      float cmax = -INFINITY;
#pragma unroll
      for (int et = 0; et < 2; ++et)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[et][r] = ok[et][r] ? S[et][r] * scale_log2 : -INFINITY;
          cmax = fmaxf(cmax, x[et][r]);
        }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      if (g == 0) s_x[wave][i16] = cmax;
      __syncthreads();
      cmax = fmaxf(cmax, s_x[partner][i16]);
      // online-softmax rescale, skipped when no head of the wave saw its max
      // grow (the branch is wave-uniform, and both waves of a head group see
      // the same maxima; heads whose max did not grow get alpha = 1). Letting
      // the reference max lag (p up to 2^k in fp16) was measured to raise the
      // p.v error steadily with k, so it never lags.
      if (__ballot(cmax > m_run + RESCALE_LOG2)) {
        const float m_new = fmaxf(m_run, cmax);
        const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int ct = 0; ct < CTH; ++ct) O[ct] *= alpha;
        m_run = m_new;
      }
      const bool none = m_run == -INFINITY;
      // P^T operand of the k-step over this half's 32 slots: element s of
      // lane (j + 16g) is slot (s < 4 ? 4g + s : 16 + 4g + s - 4), head j
      v8h P;
      float psum = 0.f;
#pragma unroll
      for (int et = 0; et < 2; ++et)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = none ? 0.f : exp2f(x[et][r] - m_run);
          psum += pv;
          P[et * 4 + r] = (_Float16)pv;
        }
      l_run += psum;
      s_p[wave][lane] = P;
      __syncthreads();
      const v8h Pq = s_p[partner][lane];
      // O^T[channel][head] += V^T P^T over both halves' slots, for this
      // wave's half of the channels
#pragma unroll
      for (int ct = 0; ct < CTH; ++ct) {
        const _Float16* vrow = &Vs[(half * (D / 2) + ct * 16 + i16) * VST];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const v4h lo = *reinterpret_cast<const v4h*>(vrow + 32 * kh + 4 * g);
          const v4h hi = *reinterpret_cast<const v4h*>(vrow + 32 * kh + 16 + 4 * g);
          v8h A;
          A[0] = lo[0]; A[1] = lo[1]; A[2] = lo[2]; A[3] = lo[3];
          A[4] = hi[0]; A[5] = hi[1]; A[6] = hi[2]; A[7] = hi[3];
          O[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, kh == half ? P : Pq, O[ct], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  };
  phase(std::false_type{}, s_begin, s_end < nsel ? s_end : nsel);
  phase(std::true_type{}, s_begin > nsel ? s_begin : nsel, s_end);

  // softmax denominator: this lane's slots, then the wave's, then the pair's
  float l_own = l_run + __shfl_xor(l_run, 16, 64);
  l_own += __shfl_xor(l_own, 32, 64);
  if (g == 0) s_x[wave][i16] = l_own;
  __syncthreads();
  const float l_tot = l_own + s_x[partner][i16];
  if (head >= H) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (nsplit == 1) {
    const int64_t base = ((int64_t)qi * H + head) * D + half * (D / 2);
#pragma unroll
    for (int ct = 0; ct < CTH; ++ct) {
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
    if (lse && half == 0 && g == 0)
      lse[(int64_t)qi * H + head] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
  } else {
    // normalised partial output in float32, stored in register order
    // [query][split][head group][column tile][lane][4] (the two halves of a
    // head group hold column tiles 0..CTH-1 and CTH..2CTH-1), so every store
    // of a wave is 1 KB contiguous; m and l in float32
    float* pw = part_o + ((((int64_t)qi * nsplit + split) * NWV + wave) * CTH) * 256 + lane * 4;
#pragma unroll
    for (int ct = 0; ct < CTH; ++ct) {
      float4 v;
      v.x = O[ct][0] * inv; v.y = O[ct][1] * inv; v.z = O[ct][2] * inv; v.w = O[ct][3] * inv;
      *reinterpret_cast<float4*>(pw + ct * 256) = v;
    }
    if (half == 0 && g == 0)
      part_ml[((int64_t)qi * nsplit + split) * H + head] = float2{m_run, l_tot};
  }
}

// Merge of the split partials, one workgroup per (query, 16-head block, 4
// column tiles), one thread per (column tile, lane), splits in index order: weights l_s * 2^(m_s - M) / L on the normalised
// partial outputs. The partials are read in the register order the attention
// kernel wrote them ([ct][lane][4] per 16-head block), 512 contiguous bytes
// per wave load; lane (j + 16g) of column tile ct holds head j, channels
// 16ct + 4g .. +3.
constexpr int MERGE_MAX = 256;  // splits per query handled by the merge
template <int D>
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ part_o,
                                                    const float2* __restrict__ part_ml,
                                                    int nsplit, int H, int NW, int n_queries,
                                                    void* __restrict__ out, int out_dtype,
                                                    float* __restrict__ lse) {
  constexpr int CT = D / 16;
  __shared__ float s_m[16][MERGE_MAX], s_f[16][MERGE_MAX];
  __shared__ float s_inv[16];
  // workgroup -> (query, 16-head block, group of 4 column tiles); thread ->
  // one (ct, lane) pair. Workgroups are dealt to the XCDs round-robin; every
  // workgroup of query qi goes to XCD qi % 8, where the attention kernel
  // wrote that query's partials, so they are read from that XCD's L2.
  constexpr int CG = CT / 4;
  const int per_q = NW * CG;
  const int xcd = blockIdx.x & 7;
  const int jx = blockIdx.x >> 3;
  const int64_t qi = xcd + 8 * (int64_t)(jx / per_q);
  if (qi >= n_queries) return;
  const int r = jx % per_q;
  const int cg = r % CG;
  const int w = r / CG;
  const int pr = cg * 256 + threadIdx.x;
  const int ct = pr >> 6, ln = pr & 63;
  const int j = ln & 15, g = ln >> 4;
  const int h = w * 16 + j;
  const int64_t split_stride = (int64_t)NW * CT * 256;
  const float* src = part_o + (qi * nsplit * NW + w) * CT * 256 + ct * 256 + ln * 4;
  // the first PB partials are requested before the (max, sum) staging so that
  // both rounds of loads overlap (indices clamped; surplus ones get weight 0)
  constexpr int PB = 8;
  float4 pre[PB];
#pragma unroll
  for (int u = 0; u < PB; ++u)
    pre[u] = *reinterpret_cast<const float4*>(src + (int64_t)(u < nsplit ? u : 0) * split_stride);
  // stage every (max, sum) of the block's 16 heads, two loads per thread in
  // flight per round
  for (int i0 = threadIdx.x; i0 < 16 * nsplit; i0 += 512) {
    float2 ml[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = i0 + 256 * r;
      const int jj = i & 15, sp = i >> 4;
      const int hh = w * 16 + jj;
      ml[r] = (i < 16 * nsplit && hh < H) ? part_ml[(qi * nsplit + sp) * H + hh]
                                          : float2{-INFINITY, 0.f};
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = i0 + 256 * r;
      if (i < 16 * nsplit) {
        s_m[i & 15][i >> 4] = ml[r].x;
        s_f[i & 15][i >> 4] = ml[r].y;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const int jj = threadIdx.x;
    const int hh = w * 16 + jj;
    float M = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, s_m[jj][sp]);
    float L = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float f = s_m[jj][sp] == -INFINITY ? 0.f : s_f[jj][sp] * exp2f(s_m[jj][sp] - M);
      s_f[jj][sp] = f;
      L += f;
    }
    s_inv[jj] = L > 0.f ? 1.f / L : 0.f;
    if (lse && cg == 0 && hh < H) lse[qi * H + hh] = (M + log2f(L)) * 0.69314718055994531f;
  }
  __syncthreads();
  {
    float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const float f = u < nsplit ? s_f[j][u] : 0.f;
      acc.x += pre[u].x * f; acc.y += pre[u].y * f;
      acc.z += pre[u].z * f; acc.w += pre[u].w * f;
    }
    for (int s0 = PB; s0 < nsplit; s0 += PB) {
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const int sp = s0 + u < nsplit ? s0 + u : 0;
        pre[u] = *reinterpret_cast<const float4*>(src + (int64_t)sp * split_stride);
      }
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const float f = s0 + u < nsplit ? s_f[j][s0 + u] : 0.f;
        acc.x += pre[u].x * f; acc.y += pre[u].y * f;
        acc.z += pre[u].z * f; acc.w += pre[u].w * f;
      }
    }
    if (h >= H) return;
    const float inv = s_inv[j];
    const int64_t o_off = (qi * H + h) * D + ct * 16 + 4 * g;
    if (out_dtype == CSA_F32) {
      float4 v;
      v.x = acc.x * inv; v.y = acc.y * inv; v.z = acc.z * inv; v.w = acc.w * inv;
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + o_off) = v;
    } else {
      typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
      v4bf v;
      v[0] = (__bf16)(acc.x * inv); v[1] = (__bf16)(acc.y * inv);
      v[2] = (__bf16)(acc.z * inv); v[3] = (__bf16)(acc.w * inv);
      *reinterpret_cast<v4bf*>(reinterpret_cast<__bf16*>(out) + o_off) = v;
    }
  }
}

struct AttnPlan {
  int nsplit, spl;
  int64_t ws_bytes;
};

// Decode (T < 16): the slots of a query are split over workgroups in whole
// 64-slot passes, at most ~32 per query (>= n/16 slots for very long dense
// ranges, where the partials would otherwise dominate), and no more than it
// takes to give every compute unit one workgroup: with many queries each
// workgroup takes more passes instead, which keeps the partial outputs (128
// KiB per workgroup at 64 heads x 512) small. A sequence's output is
// therefore the same in any batch of up to 256 / (most splits) queries.
// Longer query runs take one workgroup per query.
static AttnPlan attn_plan(int B, int T, int H, int d, int64_t n_slots) {
  AttnPlan p;
  if (T >= 16 || n_slots <= CH) {
    p.nsplit = 1;
    p.spl = (int)(((n_slots + CH - 1) / CH) * CH);
    if (p.spl < CH) p.spl = CH;
  } else {
    const int64_t div = n_slots > 4096 ? 16 : 32;
    int64_t spl = ((n_slots + div - 1) / div + CH - 1) / CH * CH;
    const int64_t most = (n_slots + spl - 1) / spl;
    const int64_t nq = (int64_t)B * T;
    const int64_t fill = nq > 0 ? (256 + nq - 1) / nq : most;
    const int64_t ns = most < fill ? most : fill;
    spl = ((n_slots + ns - 1) / ns + CH - 1) / CH * CH;
    p.spl = (int)spl;
    p.nsplit = (int)((n_slots + spl - 1) / spl);
  }
  p.ws_bytes = 0;
  if (p.nsplit > 1) {
    const int64_t units = (int64_t)B * T * p.nsplit;
    const int64_t hpad = 16 * ((H + 15) / 16);
    p.ws_bytes = ((units * hpad * d * 4 + 255) / 256) * 256 + units * H * 8;
  }
  return p;
}

struct AttnArgs {
  const uint16_t* q; const uint8_t* codes; const uint8_t* scales; int64_t blk_cap;
  const int32_t* idx; int k; int m; const uint16_t* win; int Wcap, W, B, T, H, d;
  int64_t pos0; float softmax_scale; void* out; int out_dtype; float* lse; void* ws;
  int64_t ws_bytes; hipStream_t stream;
  const int64_t* pos = nullptr;  // per-sequence first positions (pos0 = their bound) or null
  int scale_fmt = CSA_SCALE_E8M0_32;
};

template <int D, bool DENSE, int FMT>
static void launch_attn(const AttnArgs& a, const AttnPlan& p, float* part_o, float2* part_ml) {
  const int nw = (a.H + 15) / 16;
  const int64_t nq = (int64_t)a.B * a.T;
  const dim3 grid((unsigned)(((nq + 7) / 8) * 8 * p.nsplit));
  const float sl2 = a.softmax_scale * 1.4426950408889634f;
#define CSA_LAUNCH_ATTN(NW)                                                                  \
  hipLaunchKernelGGL((k_attn<D, NW, DENSE, FMT>), grid, dim3(NW * 128), 0, a.stream, a.q, a.codes, \
                     a.scales, a.blk_cap, a.idx, a.k, a.m, a.win, a.Wcap, a.W, a.T, a.H, a.pos0, \
                     a.pos, sl2, p.nsplit, p.spl, (int)nq, a.out, a.out_dtype, a.lse, part_o, part_ml)
  switch (nw) {
    case 1: CSA_LAUNCH_ATTN(1); break;
    case 2: CSA_LAUNCH_ATTN(2); break;
    case 3: CSA_LAUNCH_ATTN(3); break;
    default: CSA_LAUNCH_ATTN(4); break;
  }
#undef CSA_LAUNCH_ATTN
  if (p.nsplit > 1)
    hipLaunchKernelGGL(k_attn_merge<D>, dim3((unsigned)(((nq + 7) / 8) * 8 * nw * (D / 64))),
                       dim3(256), 0, a.stream, part_o, part_ml, p.nsplit, a.H, nw, (int)nq, a.out,
                       a.out_dtype, a.lse);
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
  if (a.scale_fmt != CSA_SCALE_E8M0_32 && a.scale_fmt != CSA_SCALE_E4M3_16) return CSA_ERR_DTYPE;
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
  if (((int64_t)a.B * a.T + 7) / 8 * 8 * p.nsplit > 0x7fffffffLL) return CSA_ERR_SHAPE;
  float* part_o = nullptr;
  float2* part_ml = nullptr;
  if (p.nsplit > 1) {
    if (!a.ws || a.ws_bytes < p.ws_bytes) return CSA_ERR_WORKSPACE;
    if (!csa_aligned(a.ws, 256)) return CSA_ERR_ALIGN;
    const int64_t units = (int64_t)a.B * a.T * p.nsplit;
    const int64_t hpad = 16 * ((a.H + 15) / 16);
    part_o = reinterpret_cast<float*>(a.ws);
    part_ml = reinterpret_cast<float2*>(reinterpret_cast<char*>(a.ws) +
                                        ((units * hpad * a.d * 4 + 255) / 256) * 256);
  }
#define CSA_ATTN_D(DN, FF)                                             \
  if (a.d == 128) launch_attn<128, DN, FF>(a, p, part_o, part_ml);      \
  else if (a.d == 256) launch_attn<256, DN, FF>(a, p, part_o, part_ml); \
  else launch_attn<512, DN, FF>(a, p, part_o, part_ml)
  if (a.scale_fmt == CSA_SCALE_E4M3_16) {
    if (dense) { CSA_ATTN_D(true, CSA_SCALE_E4M3_16); }
    else { CSA_ATTN_D(false, CSA_SCALE_E4M3_16); }
  } else {
    if (dense) { CSA_ATTN_D(true, CSA_SCALE_E8M0_32); }
    else { CSA_ATTN_D(false, CSA_SCALE_E8M0_32); }
  }
#undef CSA_ATTN_D
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
                               void* workspace, int64_t ws_bytes, int scale_fmt,
                               hipStream_t stream) {
  AttnArgs a{q, codes, scales, blk_cap, idx, k, 1, win, Wcap, W, B, T, H, d, pos0,
             softmax_scale, out, out_dtype, lse, workspace, ws_bytes, stream};
  a.scale_fmt = scale_fmt;
  return attn_run(a, false);
}

extern "C" int hca_dense_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                              int64_t blk_cap, int m, const uint16_t* win, int Wcap, int W, int B,
                              int T, int H, int d, int64_t pos0, float softmax_scale, void* out,
                              int out_dtype, float* lse, void* workspace, int64_t ws_bytes,
                              int scale_fmt, hipStream_t stream) {
  AttnArgs a{q, codes, scales, blk_cap, nullptr, 0, m, win, Wcap, W, B, T, H, d, pos0,
             softmax_scale, out, out_dtype, lse, workspace, ws_bytes, stream};
  a.scale_fmt = scale_fmt;
  return attn_run(a, true);
}

extern "C" int csa_sparse_attn_ragged(const uint16_t* q, const uint8_t* codes,
                                      const uint8_t* scales, int64_t blk_cap, const int32_t* idx,
                                      int k, const uint16_t* win, int Wcap, int W, int B, int T,
                                      int H, int d, const int64_t* pos, int64_t pos_max,
                                      float softmax_scale, void* out, int out_dtype, float* lse,
                                      void* workspace, int64_t ws_bytes, int scale_fmt,
                                      hipStream_t stream) {
  if (B > 0 && T > 0 && !pos) return CSA_ERR_NULL;
  if (pos && !csa_aligned(pos, 8)) return CSA_ERR_ALIGN;
  AttnArgs a{q, codes, scales, blk_cap, idx, k, 1, win, Wcap, W, B, T, H, d, pos_max,
             softmax_scale, out, out_dtype, lse, workspace, ws_bytes, stream};
  a.pos = pos;
  a.scale_fmt = scale_fmt;
  return attn_run(a, false);
}

extern "C" int hca_dense_attn_ragged(const uint16_t* q, const uint8_t* codes,
                                     const uint8_t* scales, int64_t blk_cap, int m,
                                     const uint16_t* win, int Wcap, int W, int B, int T, int H,
                                     int d, const int64_t* pos, int64_t pos_max,
                                     float softmax_scale, void* out, int out_dtype, float* lse,
                                     void* workspace, int64_t ws_bytes, int scale_fmt,
                                     hipStream_t stream) {
  if (B > 0 && T > 0 && !pos) return CSA_ERR_NULL;
  if (pos && !csa_aligned(pos, 8)) return CSA_ERR_ALIGN;
  AttnArgs a{q, codes, scales, blk_cap, nullptr, 0, m, win, Wcap, W, B, T, H, d, pos_max,
             softmax_scale, out, out_dtype, lse, workspace, ws_bytes, stream};
  a.pos = pos;
  a.scale_fmt = scale_fmt;
  return attn_run(a, true);
}
