// Exact top-k selection over indexer scores: device functions shared by the
// indexer kernels (indexer.hip) and the fused selection + attention kernel
// (attn.hip), plus the index workspace layout both sides address.
//
// Method: podcast transcript "DeepSeek-V4.1-Flash: Pushing the Limits of KV
// Cache Compression", cue 14 (each query keeps the top-k of the indexer
// scores over every causally visible entry). Order: score descending, then
// the lower entry; the selected entries are emitted in ascending entry order.
//
// How a selection is resolved without sorting: a 512-bin monotone histogram
// of the scores (kept by the scan) gives the threshold bin T1 whose count
// from the top first reaches k; candidates at or above T1 (collected per
// 2048-entry tile, in entry order) are narrowed to the exact k-th score tau
// by radix refinement inside T1, and one prefix scan of the packed
// (greater-than-tau, equal-to-tau) counts in entry order gives every
// selected entry its output position (the first take_eq entries equal to tau
// are the ones kept).
#pragma once

#include "csa_internal.h"

namespace csa_topk {

constexpr int TILE = 2048;       // entries per scan tile
constexpr int NB1 = 512;         // histogram bins
constexpr int MAX_TILES = 2048;  // n_max <= TILE * MAX_TILES
constexpr int POOL_G = 8;        // entries per group of the blockwise pool
constexpr int PICK_MAX = 8192;   // candidates a one-workgroup pick handles
constexpr int SPEC_SLOTS = 4096; // speculative candidates staged per query
constexpr int FUSED_CAP = 4096;  // compaction slots of an in-kernel selection
constexpr int LIST_CAP = 32;     // entries a scan unit lists (whole top bins)
constexpr int LIST_MIN = 8;      // smallest list kept (more units: no lists)
constexpr int FLAT_PER = 32;     // candidates per thread of the final pass's flat register path

// LDS scratch of a selection: ints and counters the 256 threads share.
struct SelShared {
  int* cs;        // candidate scores   [cap]
  int* ce;        // candidate entries  [cap]
  uint32_t* bh;   // refinement histogram [256]
  int* tmp;       // scan scratch [4]
  int* s_red;     // reductions [8]
};

// Exclusive prefix sum, in place, of an LDS array of n <= 2048 ints, by a
// 256-thread workgroup. Ends with a barrier.
__device__ inline void lds_excl_scan(int* a, int n, int* tmp) {
  const int base = threadIdx.x * 8;
  int loc[8];
  int s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    loc[j] = (base + j < n) ? a[base + j] : 0;
    s += loc[j];
  }
  int tot;
  int run = wg_scan_incl<256>(s, tmp, &tot) - s;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (base + j < n) a[base + j] = run;
    run += loc[j];
  }
  __syncthreads();
}

// Threshold bin of a query from the two histogram bins this thread owns
// (c_hi = bin 511 - 2j, c_lo = bin 510 - 2j for thread j): T1 is the bin
// where the count from the top first reaches k_eff = min(k, total), A1 the
// count above it. Returns k_eff; T1 and A1 come back through s_red[0..1]
// (valid if k_eff > 0). Ends with a barrier.
__device__ inline int threshold_from_bins(int c_hi, int c_lo, int k, int* tmp, int* s_red) {
  const int hb = NB1 - 1 - 2 * (int)threadIdx.x;
  int total;
  const int incl = wg_scan_incl<256>(c_hi + c_lo, tmp, &total);
  const int excl = incl - c_hi - c_lo;
  const int keff = k < total ? k : total;
  if (keff > 0) {
    if (excl + c_hi >= keff && excl < keff) {
      s_red[0] = hb;
      s_red[1] = excl;
    }
    if (incl >= keff && excl + c_hi < keff) {
      s_red[0] = hb - 1;
      s_red[1] = excl + c_hi;
    }
  }
  __syncthreads();
  return keff;
}

__device__ inline int threshold_bin(const uint32_t* hq, int k, int* tmp, int* s_red) {
  const int hb = NB1 - 1 - 2 * (int)threadIdx.x;
  return threshold_from_bins((int)hq[hb], (int)hq[hb - 1], k, tmp, s_red);
}

// Smallest and largest score of bin T1 over the workgroup, from each
// thread's partial (vmin, vmax); returns them through *lo / *hi. Two
// barriers; s_red is free again afterwards.
__device__ inline void bin_range(int vmin, int vmax, int* s_red, int* lo, int* hi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  vmin = wave_min(vmin);
  vmax = wave_max(vmax);
  if (lane == 0) {
    s_red[wave] = vmin;
    s_red[4 + wave] = vmax;
  }
  __syncthreads();
  *lo = min(min(s_red[0], s_red[1]), min(s_red[2], s_red[3]));
  *hi = max(max(s_red[4], s_red[5]), max(s_red[6], s_red[7]));
  __syncthreads();
}

// The integer scores a histogram bin can hold, in closed form (no pass over
// the candidates): bin b >= 1 covers the float32 values [2^e (1 + j/16),
// 2^e (1 + (j+1)/16)) of the scores; above 2^24 the int -> float rounding can
// move a score across a boundary by up to an ulp, so the range is widened by
// one ulp there (the refinement only counts scores actually in the bin, so a
// wider range costs nothing but empty histogram bins). Bin 0 holds 0 only.
__device__ inline void bin_bounds(int T1, int* lo, int* hi) {
  if (T1 <= 0) {
    *lo = 0;
    *hi = 0;
    return;
  }
  const double b_lo = (double)__uint_as_float((uint32_t)(T1 + 2031) << 19);
  const double b_hi = (double)__uint_as_float((uint32_t)(T1 + 2032) << 19);
  const double pad = b_lo >= 16777216.0 ? b_lo * (1.0 / 8388608.0) : 0.0;
  double l = floor(b_lo - pad), h = ceil(b_hi + pad);
  l = l < 0.0 ? 0.0 : l;
  h = h > 2147483647.0 ? 2147483647.0 : h;
  *lo = (int)l;
  *hi = (int)h;
}

// Exact k-th score among LDS candidates: cs[0..M) holds scores (negative =
// no candidate), those in bin T1 span [lo, hi], and `need` of them are still
// to be taken. Radix refinement over (score - lo): a 256-bin histogram of
// the remaining range per round, narrowed to the bin where the count from
// the top reaches need. Returns tau; *take_eq = how many candidates equal to
// tau are taken. All 256 threads call it; it ends with a barrier.
__device__ inline int refine_tau(const int* cs, int M, int T1, int lo, int hi, int need,
                                 uint32_t* bh, int* tmp, int* s_red, int* take_eq) {
  int R = hi - lo;
  while (R > 0) {
    const int bits = 32 - __clz(R);
    const int shift = bits > 8 ? bits - 8 : 0;
    bh[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < M; i += 256) {
      const int sv = cs[i];
      if (score_bin512(sv) == T1 && sv >= lo && sv - lo <= R)
        atomicAdd(&bh[(sv - lo) >> shift], 1u);
    }
    __syncthreads();
    const int v = (int)bh[255 - threadIdx.x];
    int tot;
    const int inc = wg_scan_incl<256>(v, tmp, &tot);
    if (inc >= need && inc - v < need) {
      s_red[0] = 255 - (int)threadIdx.x;
      s_red[1] = need - (inc - v);
    }
    __syncthreads();
    const int beta = s_red[0];
    need = s_red[1];
    __syncthreads();
    lo += beta << shift;
    R = shift ? min(R - (beta << shift), (1 << shift) - 1) : 0;
  }
  *take_eq = need;
  return lo;
}

// Ordered emission of the selected candidates of cs/ce[0..M) (kept in entry
// order; negative scores are holes): thread j owns slots [8j, 8j + 8) of
// each 2048-slot round; one scan of the packed (greater, equal) counts gives
// every slot its output position: #greater before it + min(#equal before
// it, take_eq). emit(pos, ce[i], cs[i]) for the keff selected ones.
template <class Emit>
__device__ inline void emit_ordered(const int* cs, const int* ce, int M, int tau, int take_eq,
                                    int keff, int* tmp, Emit emit) {
  int run_gt = 0, run_eq = 0;
  for (int r0 = 0; r0 < M; r0 += 2048) {
    const int i0 = r0 + 8 * (int)threadIdx.x;
    int sv[8];
    int gtc = 0, eqc = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sv[j] = i0 + j < M ? cs[i0 + j] : -1;
      gtc += sv[j] > tau;
      eqc += sv[j] == tau;
    }
    const int mine = (gtc << 16) | eqc;
    int tot;
    const int before = wg_scan_incl<256>(mine, tmp, &tot) - mine;
    int gb = run_gt + (before >> 16), eb = run_eq + (before & 0xffff);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int pos = -1;
      if (sv[j] > tau) {
        pos = gb + min(eb, take_eq);
        ++gb;
      } else if (sv[j] == tau) {
        if (eb < take_eq) pos = gb + eb;
        ++eb;
      }
      if (pos >= 0 && pos < keff) emit(pos, ce[i0 + j], sv[j]);
    }
    run_gt += tot >> 16;
    run_eq += tot & 0xffff;
  }
}

// ------------------------------------------------------------------------
// Register-resident selection: thread j holds PER candidate scores in
// entry order (thread-major, so the workgroup's candidates are in entry
// order as a whole); negative scores are holes. With T1 known and `need`
// candidates of bin T1 still to take:
//  * refine_regs: the exact k-th score tau by radix refinement over the
//    registers (a 256-bin LDS histogram of bin T1's values per round; only
//    bin-T1 values touch LDS, one round while T1 spans <= 256 values);
//  * emit_regs: one scan of the packed (greater, equal) counts gives each
//    selected candidate its output position; emit(pos, j, score) for
//    register j of this thread.
// ------------------------------------------------------------------------
template <int PER>
__device__ inline int refine_regs(const int (&sv)[PER], int T1, int need, SelShared s,
                                  int* take_eq) {
  int lo, hi;
  bin_bounds(T1, &lo, &hi);
  int nd = need;
  int R = hi - lo;
  while (R > 0) {
    const int bits = 32 - __clz(R);
    const int shift = bits > 8 ? bits - 8 : 0;
    s.bh[threadIdx.x] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int v = sv[j];
      if (v >= 0 && score_bin512(v) == T1 && v >= lo && v - lo <= R)
        atomicAdd(&s.bh[(v - lo) >> shift], 1u);
    }
    __syncthreads();
    const int c = (int)s.bh[255 - threadIdx.x];
    int tot;
    const int inc = wg_scan_incl<256>(c, s.tmp, &tot);
    if (inc >= nd && inc - c < nd) {
      s.s_red[0] = 255 - (int)threadIdx.x;
      s.s_red[1] = nd - (inc - c);
    }
    __syncthreads();
    const int beta = s.s_red[0];
    nd = s.s_red[1];
    __syncthreads();
    lo += beta << shift;
    R = shift ? min(R - (beta << shift), (1 << shift) - 1) : 0;
  }
  *take_eq = nd;
  return lo;
}

template <int PER, class Emit>
__device__ inline void emit_regs(const int (&sv)[PER], int p0, int tau, int take_eq, int keff,
                                 int* tmp, Emit emit) {
  (void)p0;
  int gtc = 0, eqc = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    gtc += sv[j] > tau;
    eqc += sv[j] == tau;
  }
  const int mine = (gtc << 16) | eqc;
  int tot;
  const int before = wg_scan_incl<256>(mine, tmp, &tot) - mine;
  int gb = before >> 16, eb = before & 0xffff;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    int pos = -1;
    if (sv[j] > tau) {
      pos = gb + min(eb, take_eq);
      ++gb;
    } else if (sv[j] == tau) {
      if (eb < take_eq) pos = gb + eb;
      ++eb;
    }
    if (pos >= 0 && pos < keff) emit(pos, j, sv[j]);
  }
}

// ------------------------------------------------------------------------
// One-workgroup selection over a whole score row (at most PICK_MAX
// candidates: a small Reindex pool, a short context). Thread j holds scores
// [PER j, PER j + PER) of sq[0..N) in registers; the threshold bin comes from
// the histogram, the rest from refine_regs / emit_regs (no LDS staging: at
// one or two waves per SIMD every LDS round trip of a loop is exposed).
// emit(pos, row index, score) for the keff selected ones; returns keff. The
// histogram is only read; SelShared's cs / ce are not used. With a candidate
// pool `ids` (the row's entry ids), each thread loads its rows' ids with their
// scores, and emit receives the id instead of the row index (no dependent load
// per selected entry).
// ------------------------------------------------------------------------
template <int PER, class Emit>
__device__ inline int pick_select(const int32_t* sq, const int32_t* ids, const uint32_t* hq,
                                  int N, int k, SelShared s, Emit emit) {
  const int p0 = PER * (int)threadIdx.x;
  int sv[PER];  // issued before the histogram scan so that both loads overlap
  int cid[PER];
  // (a pool row starts 16-byte aligned only when the pool length is a
  // multiple of 4; otherwise its ids are loaded one by one)
  const bool ids_vec = ids && ((reinterpret_cast<uintptr_t>(ids) & 15) == 0);
  if (p0 + PER <= N) {
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
      const int4 v = *reinterpret_cast<const int4*>(sq + p0 + j);
      sv[j] = v.x; sv[j + 1] = v.y; sv[j + 2] = v.z; sv[j + 3] = v.w;
    }
    if (ids_vec) {
#pragma unroll
      for (int j = 0; j < PER; j += 4) {
        const int4 v = *reinterpret_cast<const int4*>(ids + p0 + j);
        cid[j] = v.x; cid[j + 1] = v.y; cid[j + 2] = v.z; cid[j + 3] = v.w;
      }
    } else if (ids) {
#pragma unroll
      for (int j = 0; j < PER; ++j) cid[j] = ids[p0 + j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) sv[j] = p0 + j < N ? sq[p0 + j] : -1;
    if (ids) {
#pragma unroll
      for (int j = 0; j < PER; ++j) cid[j] = p0 + j < N ? ids[p0 + j] : -1;
    }
  }
  const int keff = threshold_bin(hq, k, s.tmp, s.s_red);
  if (keff == 0) return 0;
  const int T1 = s.s_red[0];
  const int need = keff - s.s_red[1];
  __syncthreads();
  int take_eq;
  const int tau = refine_regs<PER>(sv, T1, need, s, &take_eq);
  emit_regs<PER>(sv, p0, tau, take_eq, keff, s.tmp, [&](int pos, int j, int v) {
    emit(pos, ids ? cid[j] : p0 + j, v);
  });
  return keff;
}

// ------------------------------------------------------------------------
// Selection from per-segment candidate lists (the select pass's per-tile
// lists, or the batched scan's quarter-tile lists): segment t of the query
// holds cnt[t] (score, entry) pairs at or above the threshold bin, in entry
// order, at cq[t << seg_shift ...]; segments follow each other in entry
// order, and "tile" below means a segment.
//
// One round of loads brings the histogram bins, the tile counts and the
// first 2^spec_shift candidates of each of the first spec_tiles tiles
// (speculatively, before the counts are known) into LDS. Then:
//  * every tile staged and none holding more than 2^spec_shift candidates
//    (the usual case): the stage itself, tile-major with holes, is already in
//    entry order, so the refinement and the ordered emission run over it in
//    registers (refine_regs, emit_regs);
//  * else, at most `cap` candidates: they are compacted into LDS (from the
//    stage, or from global memory past it) by a prefix over the tile counts;
//  * else (massive ties): the per-tile lists are walked in global memory.
// emit(pos, entry, score) for the keff selected ones; returns keff. The
// histogram is only read.
//
// LDS (`smem`, 16-byte aligned): t_off [toff_n] ints, then the compaction
// area cs/ce [cap] ints each (2 cap >= 4 toff_n, for the walk's per-tile
// arrays), then the stage's scores and entries [spec_tiles << spec_shift]
// ints each.
// ------------------------------------------------------------------------
// n_tiles candidate lists (segments), list t at cq[t << seg_shift] with its
// count at cntq[t]: the select pass's per-tile lists (seg_shift = log2 TILE),
// or the batched scan's quarter-tile lists (log2 TILE / 4)
struct FinalPlan {
  int n_tiles, k, spec_tiles, spec_shift, cap, toff_n, seg_shift;
};

__host__ __device__ inline size_t final_lds_bytes(const FinalPlan& p) {
  return (size_t)(p.toff_n + 2 * p.cap + 2 * (p.spec_tiles << p.spec_shift)) * sizeof(int);
}

template <bool FLAT, class Emit>
__device__ inline int final_select(const uint32_t* hq, const int32_t* cntq, const int2* cq,
                                   const FinalPlan& P, int* smem, uint32_t* bh, int* tmp,
                                   int* s_red, Emit emit) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_tiles = P.n_tiles, cap = P.cap;
  int* t_off = smem;
  int* area = smem + P.toff_n;
  const int nspec = P.spec_tiles << P.spec_shift;
  const int spt = 1 << P.spec_shift;
  int* sp_s = area + 2 * cap;
  int* sp_e = sp_s + nspec;

  // ---- one round of independent loads: histogram bins, the stage's
  // candidates (thread j: slots [16 j, 16 j + 16), so the workgroup's slots
  // run tile-major in entry order), the counts of their tiles, all tile counts
  const int hb = NB1 - 1 - 2 * (int)threadIdx.x;
  const int c_hi = (int)hq[hb];
  const int c_lo = (int)hq[hb - 1];
  constexpr int SPT = SPEC_SLOTS / 256;  // 16
  const int i0 = SPT * (int)threadIdx.x;
  int2 r[SPT];
#pragma unroll
  for (int u = 0; u < SPT; u += 2) {  // pairs of slots: one 16-byte load each
    const int i = i0 + u < nspec ? i0 + u : 0;
    const int4 v = *reinterpret_cast<const int4*>(
        cq + ((int64_t)(i >> P.spec_shift) << P.seg_shift) + (i & (spt - 1)));
    r[u] = int2{v.x, v.y};
    r[u + 1] = int2{v.z, v.w};
  }
  // the thread's slots span at most two tiles (at least 8 slots per tile)
  const int tl_a = (i0 < nspec ? i0 : 0) >> P.spec_shift;
  const int tl_b = (i0 + SPT - 1 < nspec ? i0 + SPT - 1 : 0) >> P.spec_shift;
  const int rc_a = cntq[tl_a], rc_b = cntq[tl_b];
  int cr[MAX_TILES / 256];
#pragma unroll
  for (int u = 0; u < MAX_TILES / 256; ++u) {
    const int i = threadIdx.x + 256 * u;
    cr[u] = i < n_tiles ? cntq[i] : 0;
  }
  const int keff = threshold_from_bins(c_hi, c_lo, P.k, tmp, s_red);
  if (keff == 0) return 0;
  const int T1 = s_red[0], A1 = s_red[1];
  int need = keff - A1;  // threshold-bin candidates still to take
  // a tile with more candidates than its staged slots (or one not staged)
  bool spill = P.spec_tiles < n_tiles;
#pragma unroll
  for (int u = 0; u < MAX_TILES / 256; ++u) spill |= cr[u] > spt;
  const bool direct = __syncthreads_or(spill ? 1 : 0) == 0;  // (also orders s_red reads)

  if (direct) {
    // ---- the stage in registers: slot (t, j) holds candidate j of tile t,
    // or a hole (score -1) past the tile's count
    int sv[SPT];
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int i = i0 + u;
      const int cnt_t = (i >> P.spec_shift) == tl_a ? rc_a : rc_b;
      sv[u] = (i < nspec && (i & (spt - 1)) < cnt_t) ? r[u].x : -1;
    }
    const SelShared sh{nullptr, nullptr, bh, tmp, s_red};
    int take_eq;
    const int tau = refine_regs<SPT>(sv, T1, need, sh, &take_eq);
    emit_regs<SPT>(sv, i0, tau, take_eq, keff, tmp,
                   [&](int pos, int u, int v) { emit(pos, r[u].y, v); });
    return keff;
  }

  // ---- flat register path: with at most 256 lists and FLAT_PER * 256
  // candidates, the list offsets come from one scan of the per-thread list
  // counts, and thread j loads positions [FLAT_PER j, FLAT_PER j + FLAT_PER)
  // of the concatenated lists (entry order) straight into registers; the
  // refinement and the ordered emission then run as on the direct path (the
  // LDS compaction, refinement and emission below cost about twice as much).
  // Compiled only where asked (FLAT): its registers would cost the launches of
  // many queries, which share a compute unit four workgroups at a time.
  if (FLAT && n_tiles <= 256) {
    const int c_me = (int)threadIdx.x < n_tiles ? cr[0] : 0;
    int tot;
    const int incl = wg_scan_incl<256>(c_me, tmp, &tot);
    if (tot <= FLAT_PER * 256) {  // (uniform)
      if ((int)threadIdx.x < n_tiles) t_off[threadIdx.x] = incl - c_me;
      __syncthreads();
      const int p0 = FLAT_PER * (int)threadIdx.x;
      // the list holding position p0: the last one starting at or before it
      int tl = 0;
      if (p0 < tot) {
        int lo = 0, hi = n_tiles - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (t_off[mid] <= p0) lo = mid;
          else hi = mid - 1;
        }
        tl = lo;
      }
      int nxt = tl + 1 < n_tiles ? t_off[tl + 1] : tot;
      int base = t_off[tl];
      int2 v[FLAT_PER];
#pragma unroll
      for (int u = 0; u < FLAT_PER; ++u) {
        const int p = p0 + u;
        while (p < tot && p >= nxt) {  // (lists with no candidate are skipped)
          ++tl;
          base = nxt;
          nxt = tl + 1 < n_tiles ? t_off[tl + 1] : tot;
        }
        const int pc = p < tot ? p : 0;
        const int tc = p < tot ? tl : 0;
        v[u] = cq[((int64_t)tc << P.seg_shift) + (p < tot ? pc - base : 0)];
      }
      int sv[FLAT_PER];
#pragma unroll
      for (int u = 0; u < FLAT_PER; ++u) sv[u] = p0 + u < tot ? v[u].x : -1;
      const SelShared sh{nullptr, nullptr, bh, tmp, s_red};
      int take_eq;
      const int tau = refine_regs<FLAT_PER>(sv, T1, need, sh, &take_eq);
      emit_regs<FLAT_PER>(sv, p0, tau, take_eq, keff, tmp,
                          [&](int pos, int u, int val) { emit(pos, v[u].y, val); });
      return keff;
    }
  }

  // ---- per-tile offsets of the candidates; the stage goes to LDS as well
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int i = i0 + u;
    if (i < nspec) {
      sp_s[i] = r[u].x;
      sp_e[i] = r[u].y;
    }
  }
#pragma unroll
  for (int u = 0; u < MAX_TILES / 256; ++u) {
    const int i = threadIdx.x + 256 * u;
    if (i < n_tiles) t_off[i] = cr[u];
  }
  __syncthreads();
  const int last_cnt = t_off[n_tiles - 1];
  __syncthreads();
  lds_excl_scan(t_off, n_tiles, tmp);
  const int M = t_off[n_tiles - 1] + last_cnt;

  if (M <= cap) {
    // ---- every candidate compacted into LDS, entry order kept: two threads
    // per tile copy its candidates (from the stage, or from global memory
    // past it) and track the score range of the threshold bin
    int* cs = area;
    int* ce = area + cap;
    int vmin = 0x7fffffff, vmax = -1;
    for (int tl = threadIdx.x >> 1; tl < n_tiles; tl += 128) {
      const int base = t_off[tl];
      const int c = (tl + 1 < n_tiles ? t_off[tl + 1] : M) - base;
      for (int j = threadIdx.x & 1; j < c; j += 2) {
        int sv, ev;
        if (tl < P.spec_tiles && j < spt) {
          sv = sp_s[(tl << P.spec_shift) + j];
          ev = sp_e[(tl << P.spec_shift) + j];
        } else {
          const int2 v = cq[((int64_t)tl << P.seg_shift) + j];
          sv = v.x;
          ev = v.y;
        }
        cs[base + j] = sv;
        ce[base + j] = ev;
        if (score_bin512(sv) == T1) {
          vmin = min(vmin, sv);
          vmax = max(vmax, sv);
        }
      }
    }
    int lo, hi;
    bin_range(vmin, vmax, s_red, &lo, &hi);
    int take_eq;
    const int tau = refine_tau(cs, M, T1, lo, hi, need, bh, tmp, s_red, &take_eq);
    emit_ordered(cs, ce, M, tau, take_eq, keff, tmp, emit);
    return keff;
  }

  // ---- per-tile lists in global memory (arrays alias the area)
  int* t_cnt = area;
  int* t_gt = area + P.toff_n;
  int* t_eq = area + 2 * P.toff_n;
  int* t_eqb = area + 3 * P.toff_n;
  for (int i = threadIdx.x; i < n_tiles; i += 256) t_cnt[i] = cntq[i];
  __syncthreads();
  int vmin = 0x7fffffff, vmax = -1;
  for (int tl = wave; tl < n_tiles; tl += 4) {
    const int c = t_cnt[tl];
    for (int j = lane; j < c; j += 64) {
      const int sv = cq[((int64_t)tl << P.seg_shift) + j].x;
      if (score_bin512(sv) == T1) {
        vmin = min(vmin, sv);
        vmax = max(vmax, sv);
      }
    }
  }
  int lo, hi;
  bin_range(vmin, vmax, s_red, &lo, &hi);
  int R = hi - lo;
  while (R > 0) {
    const int bits = 32 - __clz(R);
    const int shift = bits > 8 ? bits - 8 : 0;
    bh[threadIdx.x] = 0;
    __syncthreads();
    for (int tl = wave; tl < n_tiles; tl += 4) {
      const int c = t_cnt[tl];
      for (int j = lane; j < c; j += 64) {
        const int sv = cq[((int64_t)tl << P.seg_shift) + j].x;
        if (score_bin512(sv) == T1 && sv >= lo && sv - lo <= R)
          atomicAdd(&bh[(sv - lo) >> shift], 1u);
      }
    }
    __syncthreads();
    const int v = (int)bh[255 - threadIdx.x];
    int tot;
    const int inc = wg_scan_incl<256>(v, tmp, &tot);
    if (inc >= need && inc - v < need) {
      s_red[0] = 255 - (int)threadIdx.x;
      s_red[1] = need - (inc - v);
    }
    __syncthreads();
    const int beta = s_red[0];
    need = s_red[1];
    __syncthreads();
    lo += beta << shift;
    R = shift ? min(R - (beta << shift), (1 << shift) - 1) : 0;
  }
  const int tau = lo;
  const int take_eq = need;
  for (int tl = wave; tl < n_tiles; tl += 4) {
    const int c = t_cnt[tl];
    int gt = 0, eq = 0;
    for (int j = lane; j < c; j += 64) {
      const int sv = cq[((int64_t)tl << P.seg_shift) + j].x;
      gt += sv > tau;
      eq += sv == tau;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      gt += __shfl_xor(gt, off, 64);
      eq += __shfl_xor(eq, off, 64);
    }
    if (lane == 0) {
      t_gt[tl] = gt;
      t_eq[tl] = eq;
      t_eqb[tl] = eq;
    }
  }
  __syncthreads();
  lds_excl_scan(t_eqb, n_tiles, tmp);
  for (int tl = threadIdx.x; tl < n_tiles; tl += 256) {
    int take = take_eq - t_eqb[tl];
    take = take < 0 ? 0 : (take > t_eq[tl] ? t_eq[tl] : take);
    t_gt[tl] += take;  // selected count of the tile
  }
  __syncthreads();
  lds_excl_scan(t_gt, n_tiles, tmp);  // -> output offset of each tile
  for (int tl = wave; tl < n_tiles; tl += 4) {
    const int c = t_cnt[tl];
    int eq_run = t_eqb[tl];
    int out_run = t_gt[tl];
    for (int j0 = 0; j0 < c; j0 += 64) {
      const int j = j0 + lane;
      int2 v = int2{-1, -1};
      if (j < c) v = cq[((int64_t)tl << P.seg_shift) + j];
      const bool is_eq = j < c && v.x == tau;
      const uint64_t meq = __ballot(is_eq);
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      const int eq_rank = eq_run + __popcll(meq & below);
      const bool take = j < c && (v.x > tau || (is_eq && eq_rank < take_eq));
      const uint64_t mt = __ballot(take);
      if (take) {
        const int pos = out_run + __popcll(mt & below);
        if (pos < keff) emit(pos, v.y, v.x);
      }
      eq_run += __popcll(meq);
      out_run += __popcll(mt);
    }
  }
  __syncthreads();
  return keff;
}

// ------------------------------------------------------------------------
// Where a selection reads a query's scores: its row of the score slab, or,
// where the scan wrote none (the list path of csa_index_attn), recomputed
// from the keys as the scan computes them: the sum over the Hi heads of
// w_h * max(0, q_h . key), in int32 (int8 products and their sums are exact,
// so the order of the additions does not matter).
// ------------------------------------------------------------------------
template <int DI>
__device__ inline int score_from_key(const int8_t* key, const int* q_lds, int Hi) {
  int4 kv[DI / 16];
#pragma unroll
  for (int c = 0; c < DI / 16; ++c) kv[c] = reinterpret_cast<const int4*>(key)[c];
  const int* wl = q_lds + Hi * (DI / 4);
  int s = 0;
  for (int h = 0; h < Hi; ++h) {
    int d = 0;
#pragma unroll
    for (int c = 0; c < DI / 16; ++c) {
      const int4 qv = *reinterpret_cast<const int4*>(q_lds + h * (DI / 4) + 4 * c);
      d = __builtin_amdgcn_sdot4(qv.x, kv[c].x, d, false);
      d = __builtin_amdgcn_sdot4(qv.y, kv[c].y, d, false);
      d = __builtin_amdgcn_sdot4(qv.z, kv[c].z, d, false);
      d = __builtin_amdgcn_sdot4(qv.w, kv[c].w, d, false);
    }
    s += wl[h] * max(d, 0);
  }
  return s;
}

struct ScoreSrc {
  const int32_t* sq;   // the query's slab row, or null: recompute
  const int8_t* keys;  // the sequence's keys [blk_cap][Di] (recompute)
  const int8_t* q;     // the query's indexer rows [Hi][Di] (recompute)
  const int8_t* w;     // its head weights [Hi] (recompute)
  int Hi, Di;
  int* q_lds;          // 16-byte aligned LDS: Hi * Di / 4 words of q, then Hi weights

  // q and w into LDS (recompute only; every thread calls it; ends with a
  // barrier when it stages)
  __device__ inline void stage() const {
    if (sq) return;
    const int nq = Hi * Di / 4;
    for (int i = threadIdx.x; i < nq; i += 256) q_lds[i] = reinterpret_cast<const int*>(q)[i];
    if ((int)threadIdx.x < Hi) q_lds[nq + threadIdx.x] = (int)w[threadIdx.x];
    __syncthreads();
  }
  // scores of entries e0 .. e0 + 7, -1 at and past N
  __device__ inline void load8(int64_t e0, int64_t N, int (&v)[8]) const {
    if (sq) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = e0 + j < N ? sq[e0 + j] : -1;
      return;
    }
    for (int j = 0; j < 8; ++j) {
      const int64_t e = e0 + j;
      int sc = -1;
      if (e < N) {
        const int8_t* key = keys + e * Di;
        sc = Di == 32 ? score_from_key<32>(key, q_lds, Hi)
                      : (Di == 64 ? score_from_key<64>(key, q_lds, Hi)
                                  : score_from_key<128>(key, q_lds, Hi));
      }
      v[j] = sc;
    }
  }
};

// ------------------------------------------------------------------------
// Exact selection by walking a query's whole score row (src: the slab row in
// global memory, or the scores recomputed from the keys; negative scores are
// holes), given its threshold bin T1 and the `need` candidates of T1 still to
// take: the bin's score range, the radix refinement of tau, then the ordered
// emission in rounds of 2048 entries. The slow path of the list selection (a
// threshold bin that even the wide lists do not cover: massive ties).
// ------------------------------------------------------------------------
template <class Emit>
__device__ inline void row_walk_select(const ScoreSrc& src, int N, int keff, int T1, int need,
                                       SelShared s, Emit emit) {
  int vmin = 0x7fffffff, vmax = -1;
  for (int64_t b0 = 8 * (int64_t)threadIdx.x; b0 < N; b0 += 2048) {
    int v[8];
    src.load8(b0, N, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (v[j] >= 0 && score_bin512(v[j]) == T1) {
        vmin = min(vmin, v[j]);
        vmax = max(vmax, v[j]);
      }
    }
  }
  int lo, hi;
  bin_range(vmin, vmax, s.s_red, &lo, &hi);
  int R = hi - lo;
  while (R > 0) {
    const int bits = 32 - __clz(R);
    const int shift = bits > 8 ? bits - 8 : 0;
    s.bh[threadIdx.x] = 0;
    __syncthreads();
    for (int64_t b0 = 8 * (int64_t)threadIdx.x; b0 < N; b0 += 2048) {
      int v[8];
      src.load8(b0, N, v);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (v[j] >= 0 && score_bin512(v[j]) == T1 && v[j] >= lo && v[j] - lo <= R)
          atomicAdd(&s.bh[(v[j] - lo) >> shift], 1u);
    }
    __syncthreads();
    const int c = (int)s.bh[255 - threadIdx.x];
    int tot;
    const int inc = wg_scan_incl<256>(c, s.tmp, &tot);
    if (inc >= need && inc - c < need) {
      s.s_red[0] = 255 - (int)threadIdx.x;
      s.s_red[1] = need - (inc - c);
    }
    __syncthreads();
    const int beta = s.s_red[0];
    need = s.s_red[1];
    __syncthreads();
    lo += beta << shift;
    R = shift ? min(R - (beta << shift), (1 << shift) - 1) : 0;
  }
  const int tau = lo, take_eq = need;
  int run_gt = 0, run_eq = 0;
  for (int r0 = 0; r0 < N; r0 += 2048) {
    const int b0 = r0 + 8 * (int)threadIdx.x;
    int sv[8];
    src.load8(b0, N, sv);
    int gtc = 0, eqc = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      gtc += sv[j] > tau;
      eqc += sv[j] == tau;
    }
    const int mine = (gtc << 16) | eqc;
    int tot;
    const int before = wg_scan_incl<256>(mine, s.tmp, &tot) - mine;
    int gb = run_gt + (before >> 16), eb = run_eq + (before & 0xffff);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int pos = -1;
      if (sv[j] > tau) {
        pos = gb + min(eb, take_eq);
        ++gb;
      } else if (sv[j] == tau) {
        if (eb < take_eq) pos = gb + eb;
        ++eb;
      }
      if (pos >= 0 && pos < keff) emit(pos, b0 + j, sv[j]);
    }
    run_gt += tot >> 16;
    run_eq += tot & 0xffff;
  }
}

// ------------------------------------------------------------------------
// Selection from the scan's own short lists (no select pass, ListsLoad): scan unit u
// of the query listed all cnt_u of its entries whose bin is at least its cut
// bin c_u (whole bins, at most lcap entries, entry order) at comp[u * lcap].
// With the query's threshold bin T1 from the histogram, unit u holds every
// one of its entries at or above T1 whenever c_u <= T1; then the candidates
// are the listed entries of bin >= T1 and the selection runs in registers
// (thread j: slots [16 j, 16 j + 16) of the units' lists, tile-major, so in
// entry order). A unit with c_u > T1 sends the query to row_walk_select over
// its score row. emit(pos, entry, score); returns keff.
// ------------------------------------------------------------------------
struct ListsPlan {
  int units, lshift;  // lcap = 2^lshift entries per unit; units * lcap <= SPEC_SLOTS, lcap >= LIST_MIN
  int ushift;         // a unit covers entries [u << ushift, (u + 1) << ushift)
};

// lists_select in two steps, so that a kernel can issue these loads before
// its other ones (vector loads complete in order: a wait for these then does
// not wait for loads issued later).
struct ListsLoad {
  static constexpr int SPT = SPEC_SLOTS / 256;  // 16 slots per thread
  int c_hi, c_lo;   // the thread's two histogram bins
  int2 r[SPT];      // its slots (score, entry)
  int2 ia, ib;      // (count, cut) of the units its slots lie in
  int i0, ua, ub, nslot;

  __device__ inline void load(const uint32_t* hq, const int2* tinfo, const int2* comp,
                              ListsPlan P) {
    const int hb = NB1 - 1 - 2 * (int)threadIdx.x;
    c_hi = (int)hq[hb];
    c_lo = (int)hq[hb - 1];
    nslot = P.units << P.lshift;
    i0 = SPT * (int)threadIdx.x;
#pragma unroll
    for (int u = 0; u < SPT; u += 2) {
      const int i = i0 + u < nslot ? i0 + u : 0;
      const int4 v = *reinterpret_cast<const int4*>(comp + i);
      r[u] = int2{v.x, v.y};
      r[u + 1] = int2{v.z, v.w};
    }
    // the thread's slots span at most two units (lcap >= 8)
    ua = (i0 < nslot ? i0 : 0) >> P.lshift;
    ub = (i0 + SPT - 1 < nslot ? i0 + SPT - 1 : 0) >> P.lshift;
    ia = tinfo[ua];
    ib = tinfo[ub];
  }

  // A unit whose list stops above T1 (cut > T1) takes its candidates from its
  // wide list instead (2 lcap entries of its top bins); the candidates of
  // all units (bin >= T1) are compacted into LDS in entry order (area: 2 *
  // units ints, then scores and entries, cap each), then refined and emitted
  // as in the final pass's compaction path. Returns false, having emitted
  // nothing, when a wide list also stops above T1 or the candidates exceed
  // cap.
  template <class Emit>
  __device__ inline bool spill_select(const int2* tinfo_q, const int2* tinfo2_q,
                                      const int2* comp2_q, int keff, int T1, int need,
                                      ListsPlan P, int* area, int cap, SelShared s, Emit emit) {
    const int U = P.units;
    const int lcap2 = 2 << P.lshift;
    int* u_off = area;         // per unit: candidate count, then its offset
    int* u_base = area + U;    // per listed unit: rank of its first slot among listed candidates
    int* cs = area + 2 * U;
    int* ce = cs + cap;
    __shared__ int s_sp[SPEC_SLOTS / LIST_MIN];  // the spilled units
    __shared__ int s_nsp, s_deep;
    for (int u = threadIdx.x; u < U; u += 256) u_off[u] = 0;
    if (threadIdx.x == 0) {
      s_nsp = 0;
      s_deep = 0;
    }
    __syncthreads();
    for (int u = threadIdx.x; u < U; u += 256) {
      if (tinfo_q[u].y > T1) {
        s_sp[atomicAdd(&s_nsp, 1)] = u;
        if (tinfo2_q[u].y > T1) s_deep = 1;  // even the wide list misses part of bin T1
      }
    }
    // this thread's listed candidates: slots of units that did not spill
    const int lmask = (1 << P.lshift) - 1;
    bool q[SPT];
    int ca = 0, cb = 0;
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int i = i0 + u;
      const bool in_a = (i >> P.lshift) == ua;
      const int2 inf = in_a ? ia : ib;
      q[u] = i < nslot && inf.y <= T1 && (i & lmask) < inf.x && score_bin512(r[u].x) >= T1;
      ca += q[u] && in_a;
      cb += q[u] && !in_a;
    }
    if (ca) atomicAdd(&u_off[ua], ca);
    if (cb) atomicAdd(&u_off[ub], cb);
    __syncthreads();
    if (s_deep) return false;
    const int nsp = s_nsp;
    // the spilled units' counts, from their wide lists (a wave per unit)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int j = wave; j < nsp; j += 4) {
      const int u = s_sp[j];
      const int cnt2 = tinfo2_q[u].x;
      int c = 0;
      for (int i = lane; i < cnt2; i += 64) c += score_bin512(comp2_q[u * lcap2 + i].x) >= T1;
      c = wave_sum(c);
      if (lane == 0) u_off[u] = c;
    }
    __syncthreads();
    const int last_cnt = u_off[U - 1];
    __syncthreads();
    lds_excl_scan(u_off, U, s.tmp);
    const int M = u_off[U - 1] + last_cnt;
    if (M > cap) return false;
    // ranks of the listed candidates: a scan over the threads (slots are in
    // unit order), each unit's first slot recording where the unit starts
    int tot;
    int rank = wg_scan_incl<256>(ca + cb, s.tmp, &tot) - (ca + cb);
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int i = i0 + u;
      if (i < nslot && (i & lmask) == 0) u_base[i >> P.lshift] = rank;
      rank += q[u];
    }
    __syncthreads();
    int vmin = 0x7fffffff, vmax = -1;
    rank -= ca + cb;
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      if (q[u]) {
        const int un = (i0 + u) >> P.lshift;
        const int at = u_off[un] + rank - u_base[un];
        cs[at] = r[u].x;
        ce[at] = r[u].y;
        if (score_bin512(r[u].x) == T1) {
          vmin = min(vmin, r[u].x);
          vmax = max(vmax, r[u].x);
        }
        ++rank;
      }
    }
    // the spilled units' candidates from their wide lists (entry order), a
    // wave per unit with a ballot for the ranks
    for (int j = wave; j < nsp; j += 4) {
      const int u = s_sp[j];
      const int cnt2 = tinfo2_q[u].x;
      int at = u_off[u];
      for (int i0w = 0; i0w < cnt2; i0w += 64) {
        const int i = i0w + lane;
        const int2 ent = i < cnt2 ? comp2_q[u * lcap2 + i] : int2{-1, 0};
        const bool take = i < cnt2 && score_bin512(ent.x) >= T1;
        const uint64_t m = __ballot(take);
        if (take) {
          const int pos = at + __popcll(m & ((1ull << lane) - 1));
          cs[pos] = ent.x;
          ce[pos] = ent.y;
          if (score_bin512(ent.x) == T1) {
            vmin = min(vmin, ent.x);
            vmax = max(vmax, ent.x);
          }
        }
        at += __popcll(m);
      }
    }
    int lo, hi;
    bin_range(vmin, vmax, s.s_red, &lo, &hi);  // (its barrier orders the writes above)
    int take_eq;
    const int tau = refine_tau(cs, M, T1, lo, hi, need, s.bh, s.tmp, s.s_red, &take_eq);
    emit_ordered(cs, ce, M, tau, take_eq, keff, s.tmp, emit);
    return true;
  }

  // area/cap: LDS for the spill path (see spill_select); tinfo_q / tinfo2_q /
  // comp2_q: the query's (count, cut) per unit and its wide lists; src: its
  // scores for the whole-row walk (slab row, or recomputed from the keys)
  template <class Emit>
  __device__ inline int resolve(const ScoreSrc& src, int N, int k, ListsPlan P, SelShared s,
                                const int2* tinfo_q, const int2* tinfo2_q, const int2* comp2_q,
                                int* area, int cap, Emit emit) {
    const int keff = threshold_from_bins(c_hi, c_lo, k, s.tmp, s.s_red);
    if (keff == 0) return 0;
    const int T1 = s.s_red[0];
    const int need = keff - s.s_red[1];
    const bool spill = i0 < nslot && (ia.y > T1 || ib.y > T1);
    if (__syncthreads_or(spill ? 1 : 0)) {  // (also orders the s_red reads)
      if (!spill_select(tinfo_q, tinfo2_q, comp2_q, keff, T1, need, P, area, cap, s, emit)) {
        __syncthreads();  // the spill path's LDS reads are done before the walk stages q
        src.stage();
        row_walk_select(src, N, keff, T1, need, s, emit);
      }
      return keff;
    }
    int sv[SPT];
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int i = i0 + u;
      const int cnt_u = (i >> P.lshift) == ua ? ia.x : ib.x;
      const bool ok = i < nslot && (i & ((1 << P.lshift) - 1)) < cnt_u &&
                      score_bin512(r[u].x) >= T1;
      sv[u] = ok ? r[u].x : -1;
    }
    int take_eq;
    const int tau = refine_regs<SPT>(sv, T1, need, s, &take_eq);
    emit_regs<SPT>(sv, i0, tau, take_eq, keff, s.tmp,
                   [&](int pos, int u, int v) { emit(pos, r[u].y, v); });
    return keff;
  }
};

// ------------------------------------------------------------------------
// host side: the index workspace layout and the final-pass plan
// ------------------------------------------------------------------------
struct IdxLayout {
  int n_tiles, g_tiles;  // entry tiles; group tiles (0 without a pool)
  int64_t npad, gpad;
  int64_t off_hist, off_ghist, off_cnt, off_slab, off_cbuf, off_gcnt, off_gslab, off_gcbuf;
  // scan-side lists (csa_index_attn): per scan unit its (count, cut bin)
  // and its top entries [units][lcap] (score, entry); units = 0 without them
  int sub, units, lcap;
  int64_t off_tinfo, off_comp, off_tinfo2, off_comp2, bytes;  // (2: the wide lists, 2 lcap)
};

// Scan workgroups per 2048-entry tile: enough workgroups (about 1024, four
// per compute unit) to stream the keys at full rate.
inline int scan_sub(int n_tiles, int64_t BT) {
  const int64_t nwg = (int64_t)n_tiles * BT;
  return nwg >= 1024 ? 1 : (nwg >= 512 ? 2 : 4);
}

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Head (per-query histograms, kept zero between calls; depends on B*T only)
// then the body every call rewrites: per-tile candidate counts, the score
// slab [BT][npad] and the per-tile candidate lists [BT][npad] (score, entry),
// and the same three again for the groups of a blockwise pool.
inline IdxLayout idx_layout(int64_t BT, int64_t n_max, bool pool, bool lists = false) {
  IdxLayout L;
  int64_t nt = (n_max + TILE - 1) / TILE;
  L.n_tiles = (int)(nt < 1 ? 1 : nt);
  L.npad = (int64_t)L.n_tiles * TILE;
  L.g_tiles = pool ? (int)((L.npad / POOL_G + TILE - 1) / TILE) : 0;
  L.gpad = (int64_t)L.g_tiles * TILE;
  int64_t o = 0;
  L.off_hist = o; o = align_up(o + BT * NB1 * 4, 256);
  L.off_ghist = o; o = align_up(o + BT * NB1 * 4, 256);
  L.off_cnt = o; o = align_up(o + BT * L.n_tiles * 4, 256);
  L.off_slab = o; o = align_up(o + BT * L.npad * 4, 256);
  L.off_cbuf = o; o = align_up(o + BT * L.npad * 8, 256);
  L.off_gcnt = o; o = align_up(o + BT * L.g_tiles * 4, 256);
  L.off_gslab = o; o = align_up(o + BT * L.gpad * 4, 256);
  L.off_gcbuf = o; o = align_up(o + BT * L.gpad * 8, 256);
  // scan-side lists: each scan unit keeps its entries of the top bins (at
  // most lcap, whole bins); a query's lists fill at most SPEC_SLOTS slots
  L.sub = scan_sub(L.n_tiles, BT);
  L.units = 0;
  L.lcap = 0;
  if (lists) {
    const int units = L.n_tiles * L.sub;
    int lcap = LIST_CAP;
    while (lcap > LIST_MIN && (int64_t)units * lcap > SPEC_SLOTS) lcap >>= 1;
    if ((int64_t)units * lcap <= SPEC_SLOTS) {
      L.units = units;
      L.lcap = lcap;
    }
  }
  L.off_tinfo = o; o = align_up(o + BT * L.units * 8, 256);
  L.off_comp = o; o = align_up(o + BT * L.units * L.lcap * 8, 256);
  L.off_tinfo2 = o; o = align_up(o + BT * L.units * 8, 256);
  L.off_comp2 = o; o = align_up(o + BT * L.units * 2 * L.lcap * 8, 256);
  L.bytes = o;
  return L;
}

// Candidates compacted into LDS when the direct path does not apply: about
// twice k (the entries above the threshold bin plus that bin), at least
// `least`, at most 8192, and enough for the global walk's per-tile arrays
// (2 cap >= 4 toff_n).
inline int select_cap(int k, int toff_n, int least) {
  int c = least;
  while (c < 2 * k && c < 8192) c *= 2;
  return c > 2 * toff_n ? c : 2 * toff_n;
}

// Speculative first-round candidates: a stage of `slots` shared out evenly,
// a power of two per list between 8 and the list's capacity `seg` (at least 8
// so that every list of a context up to slots/8 lists is staged and the
// direct path can apply).
inline void spec_plan(int n_tiles, int slots, int* spec_tiles, int* spec_shift, int seg = TILE) {
  int sh = 3;
  while ((1 << (sh + 1)) <= seg && ((int64_t)n_tiles << (sh + 1)) <= slots) ++sh;
  *spec_shift = sh;
  *spec_tiles = n_tiles < (slots >> sh) ? n_tiles : (slots >> sh);
}

// The attention half of a fused index + attention call (csa_index_attn),
// implemented with the attention kernels: the workspace holds the indexer's
// histograms, score rows and (sel = 1) the scan's short lists.
struct FusedAttn {
  const uint16_t* q; const uint8_t* codes; const uint8_t* scales; int64_t blk_cap; int k;
  const uint16_t* win; int Wcap, W, B, T, H, d; int64_t pos0; const int64_t* pos;
  float softmax_scale; void* out; int out_dtype; float* lse; void* ws; int64_t ws_bytes;
  int scale_fmt; hipStream_t stream;
  int sel;  // 1: the scan's short lists, 2: whole score rows
  uint32_t* hist; const int2* tinfo; const int2* comp; const int32_t* slab;
  int64_t npad; ListsPlan lp; const int32_t* cand; int C, m_idx;
  int32_t* out_idx; int32_t* out_score;
  int64_t alg_bytes;  // the query's algorithmic bytes (indexer + attention), for the split plan
  // the wide lists, and what recomputes a score where the scan wrote no slab
  const int2* tinfo2 = nullptr; const int2* comp2 = nullptr;
  const int8_t* q_idx = nullptr; const int8_t* w = nullptr; const int8_t* keys = nullptr;
  int Hi = 0, Di = 0;
  bool slab_ok = true;
};
// Algorithmic HBM bytes of one query of the fused call: its indexer keys (or
// pool rows), indexer query and weights, the selected entries, the window,
// q and out.
inline int64_t fused_alg_bytes(int64_t n_max, int Hi, int Di, int k, int W, int H, int d) {
  return n_max * Di + (int64_t)Hi * Di + Hi + (int64_t)k * (d / 2 + d / 32) +
         (int64_t)W * 2 * d + 2 * (int64_t)H * d * 2;
}
int64_t fused_attn_workspace(int B, int T, int H, int d, int64_t n_slots, int64_t alg_bytes);
bool fused_attn_fits(int T, int64_t n_slots);
int fused_attn_check(const FusedAttn& f);
int fused_attn_launch(const FusedAttn& f);

}  // namespace csa_topk
