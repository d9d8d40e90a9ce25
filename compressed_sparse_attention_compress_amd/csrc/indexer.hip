// Indexer scores + exact top-k over compressed blocks.
//
// Method: podcast transcript "DeepSeek-V4.1-Flash: Pushing the Limits of KV
// Cache Compression", cue 12 (Full layers run their own indexer and keep
// their own top-k; Reindex layers rescore a shared pool) and cue 14 (the
// indexer scores every causally visible position; the pool makes later
// layers' cost independent of the context length); "Frontier Architecture
// Decoding Notes (4)", section 1 (top-k over 4-token blocks).
// Score of block b: s = sum_h w[h] * max(0, q[h] . key[b]), int8 inputs, exact
// int32 accumulation on the int8 matrix cores (v_mfma_i32_16x16x64_i8).
// Selection order: score descending, then lower block index; output ascending.
//
// Plan: the entry range of every query is cut into 2048-entry tiles.
//  * phase 1 scores every tile. Few queries per sequence, or a candidate
//    pool: k_idx_scan, one workgroup per (query, tile, or part of a tile),
//    streams the int8 keys once (HBM-bound: every load is issued
//    unconditionally and double-buffered). Runs of >= 16 queries per sequence
//    (prefill chunks): k_idx_bscan, one workgroup per (group of 8-32
//    consecutive queries, tile), so each key loaded feeds the whole group.
//    Both add a 512-bin monotone histogram of the scores into a per-query
//    global histogram and (up to SLAB_SCAN_MAX entries) write each score to a
//    slab.
//  * k_idx_select (one workgroup per query and tile) reads the finished
//    histogram, derives the threshold bin and keeps the tile's entries at or
//    above it, in index order. A batched scan over more entries keeps no
//    slab: k_idx_thresh turns each histogram into a threshold score and a
//    second k_idx_bscan pass rescores the keys and keeps each query's
//    entries at or above it, per quarter tile, in index order.
//  * k_idx_final (one workgroup per query) gathers those candidates into LDS,
//    narrows the threshold to the exact k-th score by radix refinement and
//    writes the ascending list.
// Kernel boundaries, not fences, order the hand-offs: an agent-scope fence
// inside a workgroup writes back and invalidates the XCD's whole L2.
#include "csa_internal.h"
#include "topk_device.h"

#include <mutex>

namespace {

using namespace csa_topk;
constexpr int PREFILL_MIN_T = 16;
// Batched scans over more entries than this keep no score slab: they score
// every tile twice (histograms, then each query's candidates), since storing
// and re-reading 4 B per (query, entry) costs more than the second scoring
// pass. Smaller ones keep the slab (the one-workgroup pick reads it).
constexpr int64_t SLAB_SCAN_MAX = PICK_MAX;

// One 16-entry column tile: A = indexer queries (rows = heads), B = keys
// (columns = entries). Lane (j + 16g) holds D[head 4g + r][entry j] in
// acc[r] and returns its four heads' part of entry j's score: the weighted
// ReLU as 24-bit multiplies (an int8 weight times a ReLU'd product of at most
// DI x 2^14 fits).
template <int KS>
__device__ inline int score_part(const v4i (&A)[KS], const v4i (&Bk)[KS], const int (&wr)[4]) {
  v4i acc = {0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[ks], Bk[ks], acc, 0, 0, 0);
  return __mul24(wr[0], max(acc[0], 0)) + __mul24(wr[1], max(acc[1], 0)) +
         __mul24(wr[2], max(acc[2], 0)) + __mul24(wr[3], max(acc[3], 0));
}

// The parts of four column tiles (p[u] in every lane group) summed over the
// lane groups by a transpose: 16-lane rows of tiles 0/1 and 2/3 trade
// places, then 32-lane halves of the two pairs, and the sums leave lane
// (j + 16g) the whole score of tile g, entry j.
__device__ inline int quad_scores(int p0, int p1, int p2, int p3) {
  const auto a = __builtin_amdgcn_permlane16_swap(p0, p1, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(p2, p3, false, false);
  const auto h = __builtin_amdgcn_permlane32_swap((int)a[0] + (int)a[1], (int)c[0] + (int)c[1],
                                                  false, false);
  return (int)h[0] + (int)h[1];
}

// The scan unit's short lists (k_idx_scan's LISTS tail). Its cut bin is the
// lowest bin whose suffix count (entries in it and above) is at most lcap
// (NB1, an empty list, when no bin qualifies); the list holds its entries of
// the bins at or above the cut in entry order, with (count, cut). The wide
// list does the same for 2 lcap entries: a selection whose threshold bin lies
// below a unit's cut reads that unit's candidates there. Every workgroup of
// the scan runs this at the same time, at its end, so it is kept to two
// barriers: one wave finds both cuts (8 bins per lane, a wave scan from the
// top), and the entries' ranks come from wave scans plus the four wave totals.
// Returns the lowest bin the unit must add into the query's histogram: the
// bin of its kflush-th largest score (0 when it has fewer, or kflush <= 0).
// The query's kflush-th largest score is at least every unit's, so its
// threshold bin is at or above every unit's, and those bins stay exact; the
// total still reaches kflush whenever some unit has kflush scores.
__device__ __attribute__((always_inline)) inline int scan_unit_list(
    const uint32_t* lh, const int* ssc, const uint16_t* sbn, int span, int64_t wg0, int64_t N,
    int2* lq, int2* info, int2* lq2, int2* info2, int lcap, int kflush) {
  __shared__ int l_cut[3];
  __shared__ int l_wtot[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    // lane l: bins NB1 - 1 - 8 l - u, u = 0..7 (from the top down)
    int c[8];
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      c[u] = (int)lh[NB1 - 1 - 8 * lane - u];
      sum += c[u];
    }
    int run = wave_scan_incl(sum) - sum;  // entries in the bins above this lane's
    int cut = NB1, cut2 = NB1, kb = -1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      run += c[u];  // entries in bin NB1 - 1 - 8 lane - u and above
      const int bn = NB1 - 1 - 8 * lane - u;
      if (run <= lcap) cut = bn;
      if (run <= 2 * lcap) cut2 = bn;
      if (run >= kflush && kb < 0) kb = bn;  // the highest bin reaching kflush
    }
    cut = wave_min(cut);
    cut2 = wave_min(cut2);
    kb = wave_max(kb);
    if (lane == 0) {
      l_cut[0] = cut;
      l_cut[1] = cut2;
      l_cut[2] = kflush > 0 && kb > 0 ? kb : 0;
    }
  }
  __syncthreads();
  const int cut = l_cut[0], cut2 = l_cut[1];
  // the listed entries in entry order: thread j takes [8 j, 8 j + 8) of the
  // span (threads past it list nothing and read slot 0); entries at or past N
  // are not listed. sbn holds each staged score's bin + 1 (0: no score), so
  // "bin >= cut" is "sbn > cut", with both loads unconditional.
  const int j0 = threadIdx.x * 8;
  const int64_t rem64 = N - (wg0 + j0);
  const int rem = j0 < span ? (rem64 < 0 ? 0 : (rem64 > 8 ? 8 : (int)rem64)) : 0;
  const int jr = j0 < span ? j0 : 0;
  const uint4 bw = *reinterpret_cast<const uint4*>(sbn + jr);
  const int4 ra = *reinterpret_cast<const int4*>(ssc + jr);
  const int4 rb = *reinterpret_cast<const int4*>(ssc + jr + 4);
  const uint32_t bwd[4] = {bw.x, bw.y, bw.z, bw.w};
  const int v[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
  bool l1[8], l2[8];
  int f = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int b1 = j < rem ? (int)((bwd[j >> 1] >> (16 * (j & 1))) & 0xffffu) : 0;
    l1[j] = b1 > cut;
    l2[j] = b1 > cut2;
    f += (l1[j] ? 1 << 16 : 0) + (l2[j] ? 1 : 0);
  }
  const int x = wave_scan_incl(f);
  if (lane == 63) l_wtot[wave] = x;
  __syncthreads();
  int pre = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int t = l_wtot[w];
    pre += w < wave ? t : 0;
    total += t;
  }
  const int before = x - f + pre;
  int at = before >> 16, at2 = before & 0xffff;
  const int e0 = (int)(wg0 + j0);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int2 ent = int2{v[j], e0 + j};
    if (l1[j]) lq[at++] = ent;
    if (l2[j]) lq2[at2++] = ent;
  }
  if (threadIdx.x == 0) {
    *info = int2{total >> 16, cut};
    *info2 = int2{total & 0xffff, cut2};
  }
  return l_cut[2];
}

// ------------------------------------------------------------------------
// split scan, phase 1: scores -> slab, per-query score histogram
// ------------------------------------------------------------------------
// Every load is unconditional (addresses clamped into the buffers, invalid
// entries masked after the product) and double-buffered, so that a wave keeps
// 8 column tiles of keys in flight while the previous 8 are scored; scores
// are staged in LDS and written to the slab at the end.
// POOL: the tile's scores are also reduced to the best score of each group of
// POOL_G consecutive entries (group slab + group histogram), for the
// blockwise candidate pool.
// (keys carries no restrict: loads through it then stay ordered with the
// empty asm statement that paces the batches below)
// LISTS: the workgroup also lists its entries of the top bins (all entries
// of the bins above its cut, at most lcap, in entry order) with their count
// and the cut bin, so that a later selection needs no select pass.
template <int DI, bool CAND, int SUB, bool POOL, bool LISTS>
__global__ __launch_bounds__(256, DI <= 64 ? 4 : 2) void k_idx_scan(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ w,
    const int8_t* keys, int64_t blk_cap, int T, int Hi, int m, int64_t pos0,
    const int64_t* __restrict__ qpos, const int32_t* __restrict__ cand, int C, int64_t npad,
    int32_t* __restrict__ slab,
    uint32_t* __restrict__ hist, int64_t gpad, int32_t* __restrict__ gslab,
    uint32_t* __restrict__ ghist, int2* __restrict__ tinfo, int2* __restrict__ comp, int lcap,
    int2* __restrict__ tinfo2, int2* __restrict__ comp2, int write_slab, int kflush) {
  constexpr int KS = (DI + 63) / 64;
  constexpr int BATCH = 8;
  constexpr int SPAN = TILE / SUB;  // entries per workgroup (SUB workgroups per tile)
  __shared__ uint32_t lh[NB1];
  __shared__ uint32_t lhg[POOL ? NB1 : 1];
  __shared__ __attribute__((aligned(16))) int ssc[SPAN];
  // (LISTS) each staged score's histogram bin + 1, 0 where there is no score
  __shared__ __attribute__((aligned(16))) uint16_t sbn[LISTS ? SPAN : 8];
  const int64_t wg0 = (int64_t)blockIdx.x * SPAN;  // first entry of the workgroup
  const int qi = blockIdx.y;
  const int b = qi / T;
  const int64_t t = query_base(qpos, pos0, b) + (qi - b * T);
  int64_t nv = (t + 1) / m;
  nv = nv < blk_cap ? nv : blk_cap;
  const int64_t N = CAND ? (int64_t)C : nv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;

  for (int i = threadIdx.x; i < NB1; i += 256) {
    lh[i] = 0;
    if (POOL) lhg[i] = 0;
  }

  // query rows and head weights: every load unconditional (indexes clamped
  // into the row, padding masked afterwards), so that all of them are in
  // flight together instead of one round trip each. A row past the last head
  // holds a copy of that head's row: its products land in output rows whose
  // weight is 0, so it needs no mask, and with DI a multiple of 64 nothing
  // reads the q rows before the first products (a mask here made every wave
  // wait for its q row before it sent most of its first batch of key loads).
  v4i A[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c0 = ks * 64 + 16 * g;
    const int hr = i16 < Hi ? i16 : Hi - 1;
    const v4i v = *reinterpret_cast<const v4i*>(q_idx + ((int64_t)qi * Hi + hr) * DI +
                                                (c0 < DI ? c0 : 0));
    if constexpr (DI % 64 == 0) A[ks] = v;
    else A[ks] = c0 < DI ? v : v4i{0, 0, 0, 0};
  }
  int wr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g + r;
    const int wv = (int)w[(int64_t)qi * Hi + (h < Hi ? h : Hi - 1)];
    wr[r] = h < Hi ? wv : 0;
  }
  __syncthreads();

  // column tile u of batch bt of this wave: the workgroup's 4 waves take
  // interleaved 16-entry tiles, so each batch of the workgroup reads one
  // contiguous 4 x BATCH KiB stretch of keys
  auto tile_e = [&](int bt, int u) -> int64_t {
    return wg0 + ((int64_t)(bt * BATCH + u) * 4 + wave) * 16;
  };
  const int8_t* kb = keys + (int64_t)b * blk_cap * DI;
  const int32_t* cq = CAND ? cand + (int64_t)qi * C : nullptr;
  int32_t* sq = slab + (int64_t)qi * npad;
  // lanes with c0 >= DI (only when DI == 32) load a duplicate in-bounds chunk;
  // their A operand is zero, so the product does not see it
  int coff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) coff[ks] = (ks * 64 + 16 * g) % DI;
  // with no visible key row to clamp to (a pool query before its first
  // block completes) every entry scores -1 and no key is read; otherwise the
  // loads below carry no condition, so they issue back to back
  if (wg0 < N && nv == 0) {
    for (int j = threadIdx.x; j < SPAN; j += 256) {
      ssc[j] = -1;
      if (LISTS) sbn[j] = 0;
    }
  } else if (wg0 < N) {
    // two register buffers: the keys of batch bt + 1 are in flight while
    // batch bt is in the matrix cores
    constexpr int NBT = SPAN / 4 / 16 / BATCH;  // batches of BATCH column tiles per wave
    v4i Bk[2][BATCH][KS];
    bool valid[2][BATCH];
    // pool entries: every block id of the wave is requested up front, so the
    // key loads of a batch do not wait for its ids
    int cid[CAND ? NBT : 1][BATCH];
    if (CAND) {
#pragma unroll
      for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int64_t e = tile_e(bt, u) + i16;
          cid[CAND ? bt : 0][u] = cq[e < N ? e : N - 1];
        }
    }
    auto issue = [&](int buf, int bt) {
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int64_t e = tile_e(bt, u) + i16;
        int64_t blk;
        if (CAND) {
          const int64_t c = cid[CAND ? bt : 0][u];
          valid[buf][u] = e < N && c >= 0 && c < nv;
          blk = valid[buf][u] ? c : 0;
        } else {
          valid[buf][u] = e < nv;
          blk = valid[buf][u] ? e : nv - 1;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          Bk[buf][u][ks] = __builtin_nontemporal_load(
              reinterpret_cast<const v4i*>(kb + blk * DI + coff[ks]));
      }
    };
    auto consume = [&](int buf, int bt, const v4i (&Aq)[KS]) {
      // an invalid entry's part is -2^28 in every lane group (validity does
      // not depend on the group), so its sum is negative and stored as -1;
      // a valid entry's parts are >= 0 and their sum is its score
      // lane (j + 16g) takes tile 4h+g, entry j
#pragma unroll
      for (int h = 0; h < BATCH / 4; ++h) {
        int sc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int s = score_part<KS>(Aq, Bk[buf][4 * h + u], wr);
          sc[u] = valid[buf][4 * h + u] ? s : -(1 << 28);
        }
        const int v = max(quad_scores(sc[0], sc[1], sc[2], sc[3]), -1);
        const int64_t e = tile_e(bt, 4 * h + g) + i16;
        if (e < N) {
          ssc[e - wg0] = v;
          const int bv = score_bin512(v);
          if (v >= 0) atomicAdd(&lh[bv], 1u);
          if (LISTS) sbn[e - wg0] = (uint16_t)(v >= 0 ? bv + 1 : 0);
        }
      }
    };
    issue(0, 0);
#pragma unroll
    for (int bt = 0; bt < NBT; ++bt) {
      if (bt + 1 < NBT) issue((bt + 1) & 1, bt + 1);
      // the compiler would otherwise sink the next batch's loads below this
      // batch's products, and the in-order load counter would then wait for
      // both batches together: the empty statement orders the key loads
      // before it (memory clobber) and the products after it (their query
      // operand takes a zero it yields)
      asm volatile("" : "+v"(A[0])::"memory");
      consume(bt & 1, bt, A);
    }
  }
  __syncthreads();
  // the scores leave in one burst of 16-byte stores once every key load is
  // done (stores issued between loads would be waited on with them); entries
  // at or past N are never read, so whole 8-entry runs past it are not stored
  const int64_t e0 = wg0 + threadIdx.x * 8;
  if ((!LISTS || write_slab) && threadIdx.x * 8 < SPAN && e0 < N) {
    const int j0 = threadIdx.x * 8;
    int v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = e0 + j < N ? ssc[j0 + j] : -1;
    int4* d = reinterpret_cast<int4*>(sq + e0);
    d[0] = int4{v[0], v[1], v[2], v[3]};
    d[1] = int4{v[4], v[5], v[6], v[7]};
    if (POOL) {  // this thread's 8 entries are exactly one group
      int mx = v[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = max(mx, v[j]);
      gslab[(int64_t)qi * gpad + e0 / POOL_G] = mx;
      if (mx >= 0) atomicAdd(&lhg[score_bin512(mx)], 1u);
    }
  }
  if (POOL) __syncthreads();
  // the lists (whose selection needs only the bins at or above the query's
  // threshold bin) come first: their unit's kflush-th bin bounds the bins it
  // adds into the query's histogram
  int kcut = 0;
  if constexpr (LISTS) {
    const int64_t unit = (int64_t)qi * gridDim.x + blockIdx.x;
    kcut = scan_unit_list(lh, ssc, sbn, SPAN, wg0, N, comp + unit * lcap, tinfo + unit,
                          comp2 + unit * 2 * lcap, tinfo2 + unit, lcap, kflush);
  }
  uint32_t* hq = hist + (int64_t)qi * NB1;
  for (int i = threadIdx.x; i < NB1; i += 256) {
    if (i >= kcut && lh[i]) atomicAdd(&hq[i], lh[i]);
    if (POOL && lhg[i]) atomicAdd(&ghist[(int64_t)qi * NB1 + i], lhg[i]);
  }
}

// ------------------------------------------------------------------------
// split scan, phase 1 for runs of consecutive queries (prefill chunks): one
// workgroup = QG queries of one sequence x one 2048-entry tile, so every key
// loaded feeds QG queries. Rows of an MFMA tile are (query, head) pairs:
// QPT = 16 / HP queries per row tile, RT row tiles per wave, all waves share
// the queries and split the tile's entries. Scores go straight to the slab
// (entries a query cannot see yet get -1), the per-query histograms to LDS
// and then to the global histogram.
// ------------------------------------------------------------------------
// byte r of a packed word of int8 head weights, sign-extended
__device__ inline int wbyte(uint32_t pk, int r) { return (int)(int8_t)(pk >> (8 * r)); }

// MODE: 0 scores to the slab and the histograms; 1 the histograms only; 2
// (after k_idx_thresh) each query's candidates, its entries whose score
// reaches its threshold score s1q (the first score of its threshold bin), as
// (score, entry) in entry order, one list per wave's quarter of the tile at
// cbuf[row][tile * TILE + wave * TILE / 4 ..] with its count in
// cnt4[row][tile][wave] (k_idx_concat then joins the quarters), so that no
// score row is written or read back.
template <int DI, int HP, int MODE>
__global__ __launch_bounds__(256, DI <= 64 ? (MODE == 2 || HP == 16 ? 3 : 4) : 1) void k_idx_bscan(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ w,
    const int8_t* __restrict__ keys, int64_t blk_cap, int T, int Hi, int m, int64_t pos0,
    const int64_t* __restrict__ qpos, int64_t npad, int n_groups, int32_t* __restrict__ slab,
    uint32_t* __restrict__ hist, const int* __restrict__ s1q, int2* __restrict__ cbuf,
    int32_t* __restrict__ cnt4, int n_tiles) {
  constexpr int KS = (DI + 63) / 64;
  constexpr int QPT = 16 / HP;
  constexpr int RT = 8 / KS;
  constexpr int QG = RT * QPT;
  constexpr int GPQ = HP / 4;  // lane groups per query in the score layout
  constexpr int BATCH = 4;     // column tiles per load round
  __shared__ uint32_t lh[MODE == 2 ? 1 : QG][NB1];
  const int tile = blockIdx.x;
  const int b = blockIdx.y / n_groups;
  const int t0 = (blockIdx.y - b * n_groups) * QG;  // first query (index within T)
  const int64_t base = query_base(qpos, pos0, b);     // position of query 0
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;

  if (MODE != 2)
    for (int i = threadIdx.x; i < QG * NB1; i += 256) (&lh[0][0])[i] = 0;

  // Query rows and head weights: unconditional loads with clamped indexes.
  // A row of a padding query or head keeps the clamped row: its product is
  // multiplied by a zero weight. Only chunks past DI (DI = 32) are zeroed. The
  // weights of this lane's four output rows (four consecutive heads of one
  // query) are packed as int8 in one word, loaded as one word when Hi is a
  // multiple of 4.
  v4i A[RT][KS];
  uint32_t wr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int ti = t0 + rt * QPT + i16 / HP;
    const int h = i16 % HP;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = ks * 64 + 16 * g;
      const int tc = ti < T ? ti : T - 1, hc = h < Hi ? h : Hi - 1;
      const v4i v = *reinterpret_cast<const v4i*>(
          q_idx + (((int64_t)b * T + tc) * Hi + hc) * DI + (c0 < DI ? c0 : 0));
      A[rt][ks] = (DI >= 64 || c0 < DI) ? v : v4i{0, 0, 0, 0};
    }
  }
  if ((Hi & 3) == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int tq = t0 + rt * QPT + (4 * g) / HP;
      const int hh0 = (4 * g) % HP;
      const uint32_t wv = *reinterpret_cast<const uint32_t*>(
          w + ((int64_t)b * T + (tq < T ? tq : T - 1)) * Hi + (hh0 < Hi ? hh0 : 0));
      wr[rt] = (tq < T && hh0 < Hi) ? wv : 0u;
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      uint32_t pk = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;
        const int tq = t0 + rt * QPT + row / HP;
        const int hh = row % HP;
        const uint32_t wv =
            (uint8_t)w[((int64_t)b * T + (tq < T ? tq : T - 1)) * Hi + (hh < Hi ? hh : Hi - 1)];
        pk |= ((tq < T && hh < Hi) ? wv : 0u) << (8 * r);
      }
      wr[rt] = pk;
    }
  }
  // The score lanes. Lane group g's MFMA rows are four heads of query g / GPQ
  // of each row tile. The head sums go through a transpose: swapping 16-lane
  // rows between the partial sums of two row tiles (then, for 16 heads, 32-lane
  // halves between two such pairs) and adding leaves every lane a whole score,
  // RJ of them, the j-th of row tile GPQ * j + g % GPQ's query g / GPQ. So
  // lane group g owns the group's query row 4 j + lrow (lrow below) for each
  // j, and the per-score work after the sums runs on every lane.
  constexpr int RJ = RT / GPQ;
  const int lrow = (g % GPQ) * QPT + g / GPQ;
  // 32-bit per row: visible entries past this wave's first entry (negative
  // when none), so that nothing 64-bit is kept (or recomputed) per score
  const int64_t e_wave = (int64_t)tile * TILE + wave * (TILE / 4);
  const int nv_w = (int)(e_wave < 0x7fffffff ? e_wave : 0x7fffffff);
  int my_nv[RJ];
  bool my_real[RJ];  // padding queries of the last group store nothing
  int s1[RJ], run[RJ];  // emit: threshold score (above every score for padding
                        // queries) and the running candidate count of the quarter
#pragma unroll
  for (int j = 0; j < RJ; ++j) {
    const int ti = t0 + 4 * j + lrow;
    int64_t nv = (base + ti + 1) / m;
    nv = nv < blk_cap ? nv : blk_cap;
    my_real[j] = ti < T;
    my_nv[j] = ti < T ? (int)nv - nv_w : -1;
    const int sv = MODE == 2 ? s1q[(int64_t)b * T + (ti < T ? ti : T - 1)] : 0;
    s1[j] = ti < T ? sv : 0x7fffffff;
    run[j] = 0;
  }
  const int t_last = (t0 + QG < T ? t0 + QG : T) - 1;
  int64_t n_end = (base + t_last + 1) / m;  // entries any query of the group can see
  n_end = n_end < blk_cap ? n_end : blk_cap;
  __syncthreads();

  // this lane's first score row (slab, or candidate lists), from this wave's
  // first entry on; row 4 j + lrow is 4 j rows further
  int32_t* const slab_w =
      MODE == 0 ? slab + ((int64_t)b * T + t0 + lrow) * npad + e_wave : nullptr;
  int2* const cbuf_w = MODE == 2 ? cbuf + ((int64_t)b * T + t0 + lrow) * npad + e_wave : nullptr;
  uint32_t* const lh_w = &lh[MODE == 2 ? 0 : lrow][0];
  const int8_t* kb = keys + (int64_t)b * blk_cap * DI;
  int coff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) coff[ks] = (ks * 64 + 16 * g) % DI;
  if (n_end > 0 && e_wave < n_end) {
    constexpr int NBT = TILE / 4 / 16 / BATCH;
    v4i Bk[2][BATCH][KS];
    auto issue = [&](int buf, int bt) {
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        int64_t e = e_wave + (int64_t)(bt * BATCH + u) * 16 + i16;
        e = e < n_end ? e : n_end - 1;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          Bk[buf][u][ks] = *reinterpret_cast<const v4i*>(kb + e * DI + coff[ks]);
      }
    };
    // Per score the vector work is kept small (it, not the matrix cores,
    // bounds this kernel): 24-bit multiplies (an int8 weight times a ReLU'd
    // product of at most DI x 2^14 fits), the head sums as lane swaps, 32-bit
    // store offsets; e < npad always holds inside the tile.
    auto consume = [&](int buf, int bt) {
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int el = (bt * BATCH + u) * 16 + i16;  // entry within the wave's range
        // the RT products of the column tile first (independent MFMAs), then
        // their head sums, then the stores
        int p[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          v4i acc = {0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[rt][ks], Bk[buf][u][ks], acc, 0, 0, 0);
          p[rt] = __mul24(wbyte(wr[rt], 0), max(acc[0], 0)) +
                  __mul24(wbyte(wr[rt], 1), max(acc[1], 0)) +
                  __mul24(wbyte(wr[rt], 2), max(acc[2], 0)) +
                  __mul24(wbyte(wr[rt], 3), max(acc[3], 0));
        }
        int sj[RJ];
        if constexpr (GPQ == 1) {
#pragma unroll
          for (int j = 0; j < RJ; ++j) sj[j] = p[j];
        } else {
          // rows 16-31 of p[2i] trade places with rows 0-15 of p[2i + 1] (and
          // 48-63 with 32-47): the sum holds row tile 2i + (g & 1)
          int h[RT / 2];
#pragma unroll
          for (int i = 0; i < RT / 2; ++i) {
            const auto r = __builtin_amdgcn_permlane16_swap(p[2 * i], p[2 * i + 1], false, false);
            h[i] = (int)r[0] + (int)r[1];
          }
          if constexpr (GPQ == 2) {
#pragma unroll
            for (int j = 0; j < RJ; ++j) sj[j] = h[j];
          } else {
            // lanes 32-63 of h[2j] trade places with lanes 0-31 of h[2j + 1]:
            // the sum holds row tile 4j + g
#pragma unroll
            for (int j = 0; j < RJ; ++j) {
              const auto r = __builtin_amdgcn_permlane32_swap(h[2 * j], h[2 * j + 1], false, false);
              sj[j] = (int)r[0] + (int)r[1];
            }
          }
        }
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
          if constexpr (MODE == 2) {
            // the row's candidates of this column tile (the threshold score
            // is >= 0, so an invisible entry's -1 never passes), ranked
            // within its 16 lanes by a ballot
            const int sc = el < my_nv[j] ? sj[j] : -1;
            const bool c = sc >= s1[j];
            const uint32_t gb = (uint32_t)(__ballot(c) >> (16 * g)) & 0xffffu;
            if (c)
              cbuf_w[4 * j * (int)npad + run[j] + __popc(gb & ((1u << i16) - 1u))] =
                  int2{sc, (int)(e_wave + el)};
            run[j] += __popc(gb);
          } else {
            // An entry the row cannot see yet is counted in bin 0 (its score
            // taken as 0) and taken out of it again after the loop, so no
            // branch is needed; its slab value is never read (reads stop at
            // the row's visible entries). Scores are >= 0, so the bin is
            // max(float bits >> 19, 2031) - 2031 (score_bin512 without its
            // test for s <= 0).
            const int sc = el < my_nv[j] ? sj[j] : 0;
            if (MODE == 0 && my_real[j]) slab_w[4 * j * (int)npad + el] = sj[j];
            const uint32_t bk = max(__float_as_uint((float)(uint32_t)sc) >> 19, 2031u) - 2031u;
            atomicAdd(&lh_w[4 * j * NB1 + (int)bk], 1u);
          }
        }
      }
    };
    issue(0, 0);
#pragma unroll
    for (int bt = 0; bt < NBT; ++bt) {
      if (bt + 1 < NBT) issue((bt + 1) & 1, bt + 1);
      consume(bt & 1, bt);
    }
    if constexpr (MODE != 2) {
      // the wave's TILE / 4 entries each row could not see, counted in bin 0
#pragma unroll
      for (int j = 0; j < RJ; ++j) {
        const int vis = my_nv[j] < 0 ? 0 : (my_nv[j] > TILE / 4 ? TILE / 4 : my_nv[j]);
        if (i16 == 0 && vis < TILE / 4) atomicSub(&lh_w[4 * j * NB1], (uint32_t)(TILE / 4 - vis));
      }
    }
  }
  if constexpr (MODE == 2) {
    // every real row's count of this quarter (zero where the wave saw nothing)
#pragma unroll
    for (int j = 0; j < RJ; ++j)
      if (i16 == 0 && my_real[j])
        cnt4[(((int64_t)b * T + t0 + 4 * j + lrow) * n_tiles + tile) * 4 + wave] = run[j];
    return;
  }
  // (slab entries past a query's visible range are never read)
  __syncthreads();
  for (int i = threadIdx.x; i < QG * NB1; i += 256) {
    const int ql = i / NB1;
    const uint32_t c = (&lh[0][0])[i];
    if (c && t0 + ql < T) atomicAdd(&hist[((int64_t)b * T + t0 + ql) * NB1 + (i % NB1)], c);
  }
}

// Each query's threshold score for the candidate pass of k_idx_bscan: the
// least score whose bin reaches the query's threshold bin (the bin where the
// count from the top reaches min(k, visible entries)), found by bisection on
// the monotone bin map, so that "score >= it" is exactly "bin >= threshold
// bin"; INT_MAX (above every score) when the query sees no entry.
__global__ __launch_bounds__(256) void k_idx_thresh(const uint32_t* __restrict__ hist, int k,
                                                    int* __restrict__ s1q) {
  __shared__ int tmp[4];
  __shared__ int s_red[2];
  const int qi = blockIdx.x;
  const int keff = threshold_bin(hist + (int64_t)qi * NB1, k, tmp, s_red);
  if (threadIdx.x != 0) return;
  if (keff == 0) {
    s1q[qi] = 0x7fffffff;
    return;
  }
  const int T1 = s_red[0];
  int lo = 0, hi = 0x7fffffff;  // bin(hi) >= T1 holds or hi is the sentinel
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (score_bin512(mid) >= T1) hi = mid;
    else lo = mid + 1;
  }
  s1q[qi] = lo;
}

// Joins the four quarter lists of a (query, tile) that the candidate pass of
// k_idx_bscan wrote into one list in entry order at the tile's start, with
// its count, as k_idx_select would have left them for k_idx_final. The moved
// quarters go through LDS, so every read precedes every write.
__global__ __launch_bounds__(256) void k_idx_concat(int2* __restrict__ cbuf,
                                                    const int32_t* __restrict__ cnt4,
                                                    int32_t* __restrict__ cnt, int64_t npad,
                                                    int n_tiles) {
  constexpr int QL = TILE / 4;  // entries of a quarter
  __shared__ int2 st[TILE];
  const int tile = blockIdx.x, qi = blockIdx.y;
  const int4 c = *reinterpret_cast<const int4*>(cnt4 + ((int64_t)qi * n_tiles + tile) * 4);
  const int total = c.x + c.y + c.z + c.w;
  if (threadIdx.x == 0) cnt[(int64_t)qi * n_tiles + tile] = total;
  if (total == c.x) return;  // the first quarter's list is the whole list, in place
  int2* base = cbuf + (int64_t)qi * npad + (int64_t)tile * TILE;
  // wave q moves quarter q (q >= 1) behind the quarters before it
  const int wq = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cw = wq == 1 ? c.y : (wq == 2 ? c.z : c.w);
  const int pre = c.x + (wq >= 2 ? c.y : 0) + (wq >= 3 ? c.z : 0);
  if (wq > 0)
    for (int j = lane; j < cw; j += 64) st[pre + j] = base[wq * QL + j];
  __syncthreads();
  for (int j = c.x + (int)threadIdx.x; j < total; j += 256) base[j] = st[j];
}

// One selection of the select and final passes: over the entries themselves,
// or (gshift > 0) over groups of 2^gshift consecutive entries, each scored by
// its best visible entry, whose kept groups are written out entry by entry.
struct Level {
  const int32_t* slab;  // [BT][npad] scores
  int2* cbuf;           // [BT][npad] (score, index) candidates per tile
  int32_t* cnt;         // [BT][n_tiles] candidate counts
  uint32_t* hist;       // [BT][NB1] score histogram
  int64_t npad;
  int n_tiles, k, gshift;
  int spec_tiles, spec_shift;
  int32_t* out;         // [BT][k << gshift]
  int32_t* out_score;   // [BT][k] or null (entries only)
  int seg_shift = 11;   // the final pass's lists: cbuf[row][t << seg_shift], cnt[row][t]
};

// ------------------------------------------------------------------------
// split scan, phase 2a: per tile, the entries at or above the threshold bin
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_idx_select(int T, int m, int64_t pos0,
                                                    const int64_t* __restrict__ qpos,
                                                    int64_t blk_cap, int C, bool cand_mode,
                                                    Level L0, Level L1) {
  __shared__ int tmp[4];
  __shared__ int s_red[2];
  // tiles of the entry selection first, then those of the group selection
  const bool lv1 = (int)blockIdx.x >= L0.n_tiles;
  const Level L = lv1 ? L1 : L0;
  const int tile = lv1 ? blockIdx.x - L0.n_tiles : blockIdx.x;
  const int n_tiles = L.n_tiles, k = L.k;
  const int64_t npad = L.npad;
  int2* cbuf = L.cbuf;
  int32_t* cnt = L.cnt;
  const uint32_t* hist = L.hist;
  const int qi = blockIdx.y;
  const int b = qi / T;
  const int64_t t = query_base(qpos, pos0, b) + (qi - b * T);
  int64_t nv = (t + 1) / m;
  nv = nv < blk_cap ? nv : blk_cap;
  const int64_t N = lv1 ? (nv + (1 << L.gshift) - 1) >> L.gshift : (cand_mode ? (int64_t)C : nv);
  const int64_t e0 = (int64_t)tile * TILE + threadIdx.x * 8;
  const int32_t* sq = L.slab + (int64_t)qi * npad;
  int s[8];  // issued before the histogram scan so both loads overlap
  if (e0 + 8 <= N) {
    const int4 a = *reinterpret_cast<const int4*>(sq + e0);
    const int4 c = *reinterpret_cast<const int4*>(sq + e0 + 4);
    s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w;
    s[4] = c.x; s[5] = c.y; s[6] = c.z; s[7] = c.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = (e0 + j < N) ? sq[e0 + j] : -1;
  }
  const int keff = threshold_bin(hist + (int64_t)qi * NB1, k, tmp, s_red);
  if (keff == 0) return;
  const int T1 = s_red[0];
  int f = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) f += (s[j] >= 0 && score_bin512(s[j]) >= T1);
  int total;
  int pos = wg_scan_incl<256>(f, tmp, &total) - f;
  int2* dst = cbuf + (int64_t)qi * npad + (int64_t)tile * TILE;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (s[j] >= 0 && score_bin512(s[j]) >= T1) dst[pos++] = int2{s[j], (int)(e0 + j)};
  if (threadIdx.x == 0) cnt[(int64_t)qi * n_tiles + tile] = total;
}

// ------------------------------------------------------------------------
// small selections, phase 2: one workgroup per query
// ------------------------------------------------------------------------
// When a query has at most PICK_MAX candidates (a small Reindex pool, or a
// context of at most PICK_MAX entries) the per-tile select pass is not
// needed: one workgroup per query reads the query's whole score row and
// histogram (left by k_idx_scan) and selects in registers (pick_select).
// It clears the histogram for the next call. PER = entries per thread.
template <int PER>
__global__ __launch_bounds__(256) void k_idx_pick(int T, int m, int64_t pos0,
                                                  const int64_t* __restrict__ qpos,
                                                  int64_t blk_cap, int C, int k, int64_t npad,
                                                  const int32_t* __restrict__ slab,
                                                  uint32_t* __restrict__ hist,
                                                  const int32_t* __restrict__ cand,
                                                  int32_t* __restrict__ out_idx,
                                                  int32_t* __restrict__ out_score) {
  __shared__ uint32_t bh[256];
  __shared__ int tmp[4];
  __shared__ int s_red[8];
  const int qi = blockIdx.x;
  int N;  // candidates of the query: the pool, or its visible entries
  {
    const int b = qi / T;
    int64_t nv = (query_base(qpos, pos0, b) + (qi - b * T) + 1) / m;
    nv = nv < blk_cap ? nv : blk_cap;
    N = cand ? C : (int)nv;
  }
  uint32_t* hq = hist + (int64_t)qi * NB1;
  const int32_t* cq = cand ? cand + (int64_t)qi * C : nullptr;
  int32_t* oi = out_idx + (int64_t)qi * k;
  int32_t* os = out_score ? out_score + (int64_t)qi * k : nullptr;
  const int keff = pick_select<PER>(slab + (int64_t)qi * npad, cq, hq, N, k,
                                    SelShared{nullptr, nullptr, bh, tmp, s_red},
                                    [&](int pos, int id, int v) {
                                      oi[pos] = id;
                                      if (os) os[pos] = v;
                                    });
  // histogram consumed (every read of it precedes the barriers inside the
  // selection): clear it for the next call (thread j owns two bins)
  hq[NB1 - 1 - 2 * (int)threadIdx.x] = 0u;
  hq[NB1 - 2 - 2 * (int)threadIdx.x] = 0u;
  for (int i = keff + threadIdx.x; i < k; i += 256) {
    oi[i] = -1;
    if (os) os[i] = -1;
  }
}

// ------------------------------------------------------------------------
// split scan, phase 2b: one workgroup per query resolves the exact k-th score
// among the per-tile candidates and writes the ascending index list
// (final_select); a group level writes each kept group entry by entry.
// Dynamic LDS as final_select lays it out. The histogram of the query is
// cleared for the next call.
// ------------------------------------------------------------------------
template <bool FLAT>
__global__ __launch_bounds__(256) void k_idx_final(int T, int m, int64_t pos0,
                                                   const int64_t* __restrict__ qpos,
                                                   int64_t blk_cap,
                                                   const int32_t* __restrict__ cand, int C,
                                                   int cap_lds, int toff_n, int BT, Level L0,
                                                   Level L1) {
  extern __shared__ __attribute__((aligned(16))) int smem[];
  __shared__ int tmp[4];
  __shared__ uint32_t bh[256];
  __shared__ int s_red[8];
  // queries of the entry selection first, then those of the group selection
  const bool lv1 = (int)blockIdx.x >= BT;
  const Level L = lv1 ? L1 : L0;
  const int qi = lv1 ? blockIdx.x - BT : blockIdx.x;
  const int k = L.k, gs = L.gshift;
  int64_t nv;  // visible entries of the query (bounds the expanded groups)
  {
    const int b = qi / T;
    nv = (query_base(qpos, pos0, b) + (qi - b * T) + 1) / m;
    nv = nv < blk_cap ? nv : blk_cap;
  }
  uint32_t* hq = L.hist + (int64_t)qi * NB1;
  int32_t* oi = L.out + ((int64_t)qi * k << gs);
  int32_t* os = L.out_score ? L.out_score + (int64_t)qi * k : nullptr;
  const int32_t* cqq = cand ? cand + (int64_t)qi * C : nullptr;
  const FinalPlan P{L.n_tiles, k, L.spec_tiles, L.spec_shift, cap_lds, toff_n, L.seg_shift};
  const int keff = final_select<FLAT>(
      hq, L.cnt + (int64_t)qi * L.n_tiles, L.cbuf + (int64_t)qi * L.npad, P, smem, bh, tmp, s_red,
      [&](int pos, int e, int sv) {
        if (gs == 0) {
          oi[pos] = cqq ? cqq[e] : e;
          if (os) os[pos] = sv;
        } else {
          for (int r = 0; r < (1 << gs); ++r) {
            const int64_t ent = ((int64_t)e << gs) + r;
            oi[(pos << gs) + r] = ent < nv ? (int)ent : -1;
          }
        }
      });
  // histogram consumed: clear it for the next call
  hq[NB1 - 1 - 2 * (int)threadIdx.x] = 0u;
  hq[NB1 - 2 - 2 * (int)threadIdx.x] = 0u;
  for (int i = (keff << gs) + threadIdx.x; i < (k << gs); i += 256) oi[i] = -1;
  if (os)
    for (int i = keff + threadIdx.x; i < k; i += 256) os[i] = -1;
}

// ------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------
// A launch of at least this many queries has workgroups to spare: its final
// pass uses the compact LDS budget (2,048 candidates, as many speculative
// slots), which lets four workgroups share a compute unit at k <= 1024.
constexpr int FINAL_COMPACT_BT = 1024;

// Raise the dynamic LDS limit of both k_idx_final variants once per device
// (to the largest size asked so far), so calls inside a graph capture make no
// attribute call.
static bool final_lds_allow(size_t lds) {
  static std::mutex mu;
  static size_t allowed[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  std::lock_guard<std::mutex> lock(mu);
  if (allowed[dev] >= lds) return true;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_idx_final<true>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess ||
      hipFuncSetAttribute(reinterpret_cast<const void*>(k_idx_final<false>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return false;
  allowed[dev] = lds;
  return true;
}

struct IdxArgs {
  const int8_t* q_idx; const int8_t* w; const int8_t* keys; int64_t blk_cap;
  int B, T, Hi, Di, m; int64_t pos0; const int32_t* cand; int C, k;
  int32_t* out_idx; int32_t* out_score; void* ws; int64_t ws_bytes; hipStream_t stream;
  const int64_t* pos = nullptr;  // per-sequence first positions (pos0 = their bound) or null
  int n_keep = 0;              // blockwise pool: groups kept (0 = no pool)
  int32_t* out_pool = nullptr;  // [B][T][POOL_G * n_keep]
  bool lists = false;          // the workspace has the scan-side lists (csa_index_attn)
  bool write_slab = true;      // false: a list scan whose scores only the lists carry on
};

// Runs of at least PREFILL_MIN_T queries per sequence (prefill chunks) are
// scored by the batched scan; fewer queries, a candidate pool or a blockwise
// pool by the one-query scan. All feed the same select and final passes.
static bool batched_plan(const IdxArgs& a) {
  return a.cand == nullptr && a.out_pool == nullptr && a.T >= PREFILL_MIN_T;
}

static int idx_check(const IdxArgs& a, int64_t* n_max) {
  if (a.B < 0 || a.T < 0 || a.blk_cap < 0 || a.pos0 < 0) return CSA_ERR_SHAPE;
  if (a.Hi < 1 || a.Hi > 16) return CSA_ERR_SHAPE;
  if (a.Di != 32 && a.Di != 64 && a.Di != 128) return CSA_ERR_SHAPE;
  if (a.Hi * a.Di > 1024) return CSA_ERR_SHAPE;
  if (a.m < 1 || a.k < 1) return CSA_ERR_SHAPE;
  if (a.cand && a.C < 0) return CSA_ERR_SHAPE;
  if (a.out_pool && (a.cand || a.n_keep < 1)) return CSA_ERR_SHAPE;
  if ((int64_t)a.n_keep * POOL_G > 0x7fffffff || a.k > 0x7fffffff / 2) return CSA_ERR_SHAPE;
  if ((int64_t)a.B * a.T > 65535) return CSA_ERR_SHAPE;  // queries per call (grid y)
  if (a.pos0 + a.T > (int64_t)1 << 40) return CSA_ERR_RANGE;
  if (a.B == 0 || a.T == 0) return CSA_OK;
  if (!a.q_idx || !a.w || !a.keys || !a.out_idx) return CSA_ERR_NULL;
  if (!csa_aligned(a.q_idx, 16) || !csa_aligned(a.keys, 16)) return CSA_ERR_ALIGN;
  int64_t nv = (a.pos0 + a.T) / a.m;
  nv = nv < a.blk_cap ? nv : a.blk_cap;
  *n_max = a.cand ? (int64_t)a.C : nv;
  if (*n_max > (int64_t)TILE * MAX_TILES) return CSA_ERR_SHAPE;
  if (nv > 0x7fffffff) return CSA_ERR_SHAPE;
  return CSA_OK;
}

static int idx_phase(const IdxArgs& a, int phase) {
  int64_t n_max = 0;
  int st = idx_check(a, &n_max);
  if (st != CSA_OK || a.B == 0 || a.T == 0) return st;
  const int BT = a.B * a.T;
  const bool pool = a.out_pool != nullptr;
  IdxLayout L = idx_layout(BT, n_max, pool, a.lists);
  if (!a.ws) return CSA_ERR_WORKSPACE;
  if (a.ws_bytes < L.bytes) return CSA_ERR_WORKSPACE;
  if (!csa_aligned(a.ws, 256)) return CSA_ERR_ALIGN;
  char* ws = reinterpret_cast<char*>(a.ws);
  int32_t* slab = reinterpret_cast<int32_t*>(ws + L.off_slab);
  int2* cbuf = reinterpret_cast<int2*>(ws + L.off_cbuf);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.off_hist);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + L.off_cnt);
  int32_t* gslab = reinterpret_cast<int32_t*>(ws + L.off_gslab);
  int2* gcbuf = reinterpret_cast<int2*>(ws + L.off_gcbuf);
  uint32_t* ghist = reinterpret_cast<uint32_t*>(ws + L.off_ghist);
  int32_t* gcnt = reinterpret_cast<int32_t*>(ws + L.off_gcnt);
  const int C = a.cand ? a.C : 0;
  // a query with at most PICK_MAX candidates: the select and final passes in
  // one workgroup per query
  if (!pool && n_max > 0 && n_max <= PICK_MAX && phase == 1) {
    if (n_max <= PICK_MAX / 2)
      hipLaunchKernelGGL(k_idx_pick<PICK_MAX / 512>, dim3(BT), dim3(256), 0, a.stream, a.T, a.m,
                         a.pos0, a.pos, a.blk_cap, C, a.k, L.npad, slab, hist, a.cand, a.out_idx,
                         a.out_score);
    else
      hipLaunchKernelGGL(k_idx_pick<PICK_MAX / 256>, dim3(BT), dim3(256), 0, a.stream, a.T, a.m,
                         a.pos0, a.pos, a.blk_cap, C, a.k, L.npad, slab, hist, a.cand, a.out_idx,
                         a.out_score);
    CSA_TRY_LAUNCH();
    return CSA_OK;
  }
  // a batched scan without the slab (SLAB_SCAN_MAX): the slab's space holds
  // each query's threshold score [BT], then its per-quarter candidate counts
  // [BT][n_tiles][4]
  const bool rescan = batched_plan(a) && n_max > SLAB_SCAN_MAX;
  int* s1q = slab;
  int32_t* cnt4 = slab + align_up(BT, 64);
  // the final pass takes the quarter lists as they are while their number
  // fits its per-list registers (MAX_TILES); beyond that they are joined per
  // tile first
  const bool quarters = rescan && 4 * (int64_t)L.n_tiles <= MAX_TILES;
  if (phase == 0 && batched_plan(a)) {
    const int HP = a.Hi <= 4 ? 4 : (a.Hi <= 8 ? 8 : 16);
    const int KS = (a.Di + 63) / 64;
    const int QG = (8 / KS) * (16 / HP);
    const int n_groups = (a.T + QG - 1) / QG;
    const dim3 bgrid(L.n_tiles, a.B * n_groups);
#define CSA_LAUNCH_BSCAN(DD, HH, MM)                                                           \
  hipLaunchKernelGGL((k_idx_bscan<DD, HH, MM>), bgrid, dim3(256), 0, a.stream, a.q_idx, a.w,  \
                     a.keys, a.blk_cap, a.T, a.Hi, a.m, a.pos0, a.pos, L.npad, n_groups, slab,  \
                     hist, s1q, cbuf, cnt4, L.n_tiles)
#define CSA_LAUNCH_BSCAN_H(DD, MM)                                                  \
  do {                                                                              \
    if (HP == 4) CSA_LAUNCH_BSCAN(DD, 4, MM);                                       \
    else if (HP == 8) CSA_LAUNCH_BSCAN(DD, 8, MM);                                  \
    else CSA_LAUNCH_BSCAN(DD, 16, MM);                                              \
  } while (0)
#define CSA_LAUNCH_BSCAN_D(MM)                                                      \
  do {                                                                              \
    if (a.Di == 32) CSA_LAUNCH_BSCAN_H(32, MM);                                     \
    else if (a.Di == 64) CSA_LAUNCH_BSCAN_H(64, MM);                                \
    else CSA_LAUNCH_BSCAN_H(128, MM);                                               \
  } while (0)
    if (!rescan) {
      CSA_LAUNCH_BSCAN_D(0);
    } else {
      // histograms; each query's threshold score; its candidates per wave
      // quarter (joined per tile, as the select pass leaves them, only past
      // MAX_TILES / 4 tiles)
      CSA_LAUNCH_BSCAN_D(1);
      hipLaunchKernelGGL(k_idx_thresh, dim3(BT), dim3(256), 0, a.stream, hist, a.k, s1q);
      CSA_LAUNCH_BSCAN_D(2);
      if (!quarters)
        hipLaunchKernelGGL(k_idx_concat, dim3(L.n_tiles, BT), dim3(256), 0, a.stream, cbuf,
                           cnt4, cnt, L.npad, L.n_tiles);
    }
#undef CSA_LAUNCH_BSCAN_D
#undef CSA_LAUNCH_BSCAN_H
#undef CSA_LAUNCH_BSCAN
  } else if (phase == 0) {
    // small scans split each tile over 2 or 4 workgroups so that about 1024
    // workgroups (four per compute unit, all resident at once) stream the keys
    const int sub = L.sub;
    const dim3 sgrid(L.n_tiles * sub, BT);
    int2* tinfo = reinterpret_cast<int2*>(ws + L.off_tinfo);
    int2* comp = reinterpret_cast<int2*>(ws + L.off_comp);
    int2* tinfo2 = reinterpret_cast<int2*>(ws + L.off_tinfo2);
    int2* comp2 = reinterpret_cast<int2*>(ws + L.off_comp2);
    const bool lists = a.lists && L.units > 0 && !a.cand && !pool;
#define CSA_LAUNCH_SCAN1(DD, CC, SS, PP, LL)                                                     \
  hipLaunchKernelGGL((k_idx_scan<DD, CC, SS, PP, LL>), sgrid, dim3(256), 0, a.stream, a.q_idx,  \
                     a.w, a.keys, a.blk_cap, a.T, a.Hi, a.m, a.pos0, a.pos, a.cand, C, L.npad,    \
                     slab, hist, L.gpad, gslab, ghist, tinfo, comp, L.lcap, tinfo2, comp2,  \
                     a.write_slab ? 1 : 0, a.k)
#define CSA_LAUNCH_SCAN(DD, CC, SS, PP)                               \
  do {                                                                \
    if (!CC && !PP && lists) CSA_LAUNCH_SCAN1(DD, CC, SS, PP, true);  \
    else CSA_LAUNCH_SCAN1(DD, CC, SS, PP, false);                     \
  } while (0)
#define CSA_LAUNCH_SCAN_S(DD, CC, PP)                  \
  do {                                                \
    if (sub == 1) CSA_LAUNCH_SCAN(DD, CC, 1, PP);     \
    else if (sub == 2) CSA_LAUNCH_SCAN(DD, CC, 2, PP); \
    else CSA_LAUNCH_SCAN(DD, CC, 4, PP);              \
  } while (0)
    if (a.cand) {
      if (a.Di == 32) CSA_LAUNCH_SCAN_S(32, true, false);
      else if (a.Di == 64) CSA_LAUNCH_SCAN_S(64, true, false);
      else CSA_LAUNCH_SCAN_S(128, true, false);
    } else if (pool) {
      if (a.Di == 32) CSA_LAUNCH_SCAN_S(32, false, true);
      else if (a.Di == 64) CSA_LAUNCH_SCAN_S(64, false, true);
      else CSA_LAUNCH_SCAN_S(128, false, true);
    } else {
      if (a.Di == 32) CSA_LAUNCH_SCAN_S(32, false, false);
      else if (a.Di == 64) CSA_LAUNCH_SCAN_S(64, false, false);
      else CSA_LAUNCH_SCAN_S(128, false, false);
    }
#undef CSA_LAUNCH_SCAN_S
#undef CSA_LAUNCH_SCAN
#undef CSA_LAUNCH_SCAN1
  } else if (phase == 1) {
    Level L0{slab, cbuf, cnt, hist, L.npad, L.n_tiles, a.k, 0, 0, 0, a.out_idx, a.out_score};
    Level L1{gslab, gcbuf, gcnt, ghist, L.gpad, L.g_tiles, a.n_keep, 3, 0, 0, a.out_pool,
             nullptr};
    if (quarters) {  // the scan's quarter-tile lists and counts
      L0.cnt = cnt4;
      L0.n_tiles = 4 * L.n_tiles;
      L0.seg_shift = __builtin_ctz(TILE / 4);
    }
    const bool compact = BT >= FINAL_COMPACT_BT;
    const int toff_n = ((L0.n_tiles > L.g_tiles ? L0.n_tiles : L.g_tiles) + 3) / 4 * 4;
    const int cap_lds = select_cap(pool && a.n_keep > a.k ? a.n_keep : a.k, toff_n,
                                   compact ? 2048 : 4096);
    const int slots = compact && cap_lds < SPEC_SLOTS ? cap_lds : SPEC_SLOTS;
    spec_plan(L0.n_tiles, slots, &L0.spec_tiles, &L0.spec_shift, TILE >> (quarters ? 2 : 0));
    if (pool) spec_plan(L.g_tiles, slots, &L1.spec_tiles, &L1.spec_shift);
    if (!rescan)  // (the candidate pass of a rescan left the lists already)
      hipLaunchKernelGGL(k_idx_select, dim3(L.n_tiles + L.g_tiles, BT), dim3(256), 0, a.stream,
                         a.T, a.m, a.pos0, a.pos, a.blk_cap, C, a.cand != nullptr, L0, L1);
    const int spec_slots = (L0.spec_tiles << L0.spec_shift) >
                                   (pool ? (L1.spec_tiles << L1.spec_shift) : 0)
                               ? (L0.spec_tiles << L0.spec_shift)
                               : (L1.spec_tiles << L1.spec_shift);
    const size_t lds = (size_t)(toff_n + 2 * cap_lds) * sizeof(int) +
                       (size_t)spec_slots * sizeof(int2);
    if (lds > 65536 && !final_lds_allow(lds)) return CSA_ERR_HIP;
    // launches of few queries (a workgroup per compute unit) take the flat
    // register path; compact ones keep the leaner kernel
    if (compact)
      hipLaunchKernelGGL(k_idx_final<false>, dim3(BT * (pool ? 2 : 1)), dim3(256), lds, a.stream,
                         a.T, a.m, a.pos0, a.pos, a.blk_cap, a.cand, C, cap_lds, toff_n, BT, L0,
                         L1);
    else
      hipLaunchKernelGGL(k_idx_final<true>, dim3(BT * (pool ? 2 : 1)), dim3(256), lds, a.stream,
                         a.T, a.m, a.pos0, a.pos, a.blk_cap, a.cand, C, cap_lds, toff_n, BT, L0,
                         L1);
  }
  CSA_TRY_LAUNCH();
  return CSA_OK;
}

__global__ void k_fill_zero(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t j = i; j < n; j += stride) p[j] = 0u;
}

}  // namespace

extern "C" int64_t csa_index_topk_workspace(int B, int T, int64_t n_max, int k, int cand_given) {
  (void)k;
  (void)cand_given;
  if (B < 0 || T < 0 || n_max < 0) return -1;
  return idx_layout((int64_t)B * T, n_max, false).bytes;
}

extern "C" int64_t csa_index_topk_pool_workspace(int B, int T, int64_t n_max) {
  if (B < 0 || T < 0 || n_max < 0) return -1;
  return idx_layout((int64_t)B * T, n_max, true).bytes;
}

#define CSA_IDX_ARGS                                                                      \
  IdxArgs a{q_idx, w, keys, blk_cap, B, T, Hi, Di, m, pos0, cand, C, k, out_idx, out_score, \
            workspace, ws_bytes, stream}

extern "C" int csa_index_scan(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                              int64_t blk_cap, int B, int T, int Hi, int Di, int m, int64_t pos0,
                              const int32_t* cand, int C, int k, int32_t* out_idx,
                              int32_t* out_score, void* workspace, int64_t ws_bytes,
                              hipStream_t stream) {
  CSA_IDX_ARGS;
  return idx_phase(a, 0);
}

extern "C" int csa_index_select(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                                int64_t blk_cap, int B, int T, int Hi, int Di, int m,
                                int64_t pos0, const int32_t* cand, int C, int k,
                                int32_t* out_idx, int32_t* out_score, void* workspace,
                                int64_t ws_bytes, hipStream_t stream) {
  CSA_IDX_ARGS;
  return idx_phase(a, 1);
}

extern "C" int csa_index_topk(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                              int64_t blk_cap, int B, int T, int Hi, int Di, int m, int64_t pos0,
                              const int32_t* cand, int C, int k, int32_t* out_idx,
                              int32_t* out_score, void* workspace, int64_t ws_bytes,
                              hipStream_t stream) {
  CSA_IDX_ARGS;
  int st = idx_phase(a, 0);
  if (st != CSA_OK) return st;
  return idx_phase(a, 1);
}

static int ragged_phases(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                         int64_t blk_cap, int B, int T, int Hi, int Di, int m,
                         const int64_t* pos, int64_t pos_max, const int32_t* cand, int C, int k,
                         int32_t* out_idx, int32_t* out_score, void* workspace,
                         int64_t ws_bytes, hipStream_t stream, int first, int last) {
  if (B > 0 && T > 0 && !pos) return CSA_ERR_NULL;
  if (pos && !csa_aligned(pos, 8)) return CSA_ERR_ALIGN;
  IdxArgs a{q_idx, w, keys, blk_cap, B, T, Hi, Di, m, pos_max, cand, C, k, out_idx, out_score,
            workspace, ws_bytes, stream};
  a.pos = pos;
  for (int ph = first; ph <= last; ++ph) {
    const int st = idx_phase(a, ph);
    if (st != CSA_OK) return st;
  }
  return CSA_OK;
}

#define CSA_RAGGED_PARAMS                                                                     \
  const int8_t *q_idx, const int8_t *w, const int8_t *keys, int64_t blk_cap, int B, int T,    \
      int Hi, int Di, int m, const int64_t *pos, int64_t pos_max, const int32_t *cand, int C,  \
      int k, int32_t *out_idx, int32_t *out_score, void *workspace, int64_t ws_bytes,          \
      hipStream_t stream
#define CSA_RAGGED_ARGS                                                                      \
  q_idx, w, keys, blk_cap, B, T, Hi, Di, m, pos, pos_max, cand, C, k, out_idx, out_score,    \
      workspace, ws_bytes, stream

extern "C" int csa_index_topk_ragged(CSA_RAGGED_PARAMS) {
  return ragged_phases(CSA_RAGGED_ARGS, 0, 1);
}
extern "C" int csa_index_scan_ragged(CSA_RAGGED_PARAMS) {
  return ragged_phases(CSA_RAGGED_ARGS, 0, 0);
}
extern "C" int csa_index_select_ragged(CSA_RAGGED_PARAMS) {
  return ragged_phases(CSA_RAGGED_ARGS, 1, 1);
}

#undef CSA_RAGGED_ARGS
#undef CSA_RAGGED_PARAMS

static int pool_phases(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                       int64_t blk_cap, int B, int T, int Hi, int Di, int m, int64_t pos0, int k,
                       int32_t* out_idx, int32_t* out_score, int group, int n_keep,
                       int32_t* out_pool, void* workspace, int64_t ws_bytes, hipStream_t stream,
                       int first, int last) {
  if (group != POOL_G || n_keep < 1) return CSA_ERR_SHAPE;
  if (!out_pool && B > 0 && T > 0) return CSA_ERR_NULL;
  IdxArgs a{q_idx, w, keys, blk_cap, B, T, Hi, Di, m, pos0, nullptr, 0, k, out_idx, out_score,
            workspace, ws_bytes, stream};
  a.n_keep = n_keep;
  a.out_pool = out_pool;
  for (int ph = first; ph <= last; ++ph) {
    const int st = idx_phase(a, ph);
    if (st != CSA_OK) return st;
  }
  return CSA_OK;
}

#define CSA_POOL_PARAMS                                                                       \
  const int8_t *q_idx, const int8_t *w, const int8_t *keys, int64_t blk_cap, int B, int T,    \
      int Hi, int Di, int m, int64_t pos0, int k, int32_t *out_idx, int32_t *out_score,        \
      int group, int n_keep, int32_t *out_pool, void *workspace, int64_t ws_bytes,             \
      hipStream_t stream
#define CSA_POOL_ARGS                                                                        \
  q_idx, w, keys, blk_cap, B, T, Hi, Di, m, pos0, k, out_idx, out_score, group, n_keep,      \
      out_pool, workspace, ws_bytes, stream

extern "C" int csa_index_topk_pool(CSA_POOL_PARAMS) { return pool_phases(CSA_POOL_ARGS, 0, 1); }
extern "C" int csa_index_pool_scan(CSA_POOL_PARAMS) { return pool_phases(CSA_POOL_ARGS, 0, 0); }
extern "C" int csa_index_pool_select(CSA_POOL_PARAMS) { return pool_phases(CSA_POOL_ARGS, 1, 1); }

#undef CSA_POOL_ARGS
#undef CSA_POOL_PARAMS

extern "C" int csa_workspace_clear(void* ws, int64_t bytes, hipStream_t stream) {
  if (bytes < 0 || bytes % 4) return CSA_ERR_SHAPE;
  if (bytes == 0) return CSA_OK;
  if (!ws) return CSA_ERR_NULL;
  if (!csa_aligned(ws, 4)) return CSA_ERR_ALIGN;
  const int64_t n = bytes / 4;
  int64_t grid = (n + 255) / 256;
  grid = grid > 65536 ? 65536 : grid;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<uint32_t*>(ws), n);
  CSA_TRY_LAUNCH();
  return CSA_OK;
}

// ---------------------------------------------------------------------------
// Indexer + top-k + sparse attention in one call (one CSA layer's decode
// step). Few queries per sequence: the scan (which also leaves each unit's
// short list of top-bin entries), then the attention kernel in which every
// workgroup resolves its query's top-k for its own slots from those lists
// or, with at most PICK_MAX candidates, from the whole score row (no select
// or final pass, no id round trip through memory), then the merge. Runs of
// queries: the separate index and attention launches.
// ---------------------------------------------------------------------------
extern "C" int64_t csa_index_attn_workspace(int B, int T, int64_t n_max, int k, int H, int d,
                                            int W) {
  if (B < 0 || T < 0 || n_max < 0 || k < 1 || H < 1 || d < 1 || W < 0) return -1;
  const int64_t ib =
      align_up(idx_layout((int64_t)B * T, n_max, false, n_max > PICK_MAX).bytes, 256);
  const int64_t ns = (int64_t)k + W;
  // (the fused plan's partials depend on the indexer shape only through n_max;
  // Hi = 16 is the largest the indexer takes, so the size covers every Hi)
  // (a call with a candidate pool takes the uncapped plan: the larger of the two)
  int64_t ab = csa_attn_workspace(B, T, H, d, ns);
  if (fused_attn_fits(T, ns)) {
    const int64_t capped =
        fused_attn_workspace(B, T, H, d, ns, fused_alg_bytes(n_max, 16, 128, k, W, H, d));
    const int64_t pooled = fused_attn_workspace(B, T, H, d, ns, 0);
    ab = ab > capped ? ab : capped;
    ab = ab > pooled ? ab : pooled;
  }
  return ab < 0 ? -1 : ib + ab;
}

#define CSA_INDEX_ATTN_PARAMS                                                                 \
  const int8_t *q_idx, const int8_t *w, const int8_t *keys, int64_t blk_cap, int B, int T,     \
      int Hi, int Di, int m, int64_t pos0, const int64_t *pos, const int32_t *cand, int C,     \
      int k, const uint16_t *q, const uint8_t *codes, const uint8_t *scales,                   \
      const uint16_t *win, int Wcap, int W, int H, int d, float softmax_scale,                 \
      int32_t *out_idx, int32_t *out_score, void *out, int out_dtype, float *lse,              \
      void *workspace, int64_t ws_bytes, int scale_fmt, hipStream_t stream
#define CSA_INDEX_ATTN_ARGS                                                                  \
  q_idx, w, keys, blk_cap, B, T, Hi, Di, m, pos0, pos, cand, C, k, q, codes, scales, win,     \
      Wcap, W, H, d, softmax_scale, out_idx, out_score, out, out_dtype, lse, workspace,      \
      ws_bytes, scale_fmt, stream

// scan_only: every check, then only the first launch (the indexer scan)
static int index_attn(CSA_INDEX_ATTN_PARAMS, bool scan_only) {
  if (pos && !csa_aligned(pos, 8)) return CSA_ERR_ALIGN;
  IdxArgs a{q_idx, w, keys, blk_cap, B, T, Hi, Di, m, pos0, cand, C, k, out_idx, out_score,
            workspace, ws_bytes, stream};
  a.pos = pos;
  int64_t n_max = 0;
  int st = idx_check(a, &n_max);
  if (st != CSA_OK) return st;
  if (B == 0 || T == 0) return CSA_OK;
  const int BT = B * T;
  // the scan's short lists serve queries with more than PICK_MAX candidates
  // and no pool (smaller ones select from their whole score row)
  a.lists = !cand && n_max > PICK_MAX;
  const IdxLayout L = idx_layout(BT, n_max, false, a.lists);
  const int64_t ib = align_up(L.bytes, 256);
  const int64_t ns = (int64_t)k + W;
  // in-kernel selection: from whole score rows (at most PICK_MAX candidates)
  // or from the scan's short lists (when the layout could give every unit
  // one); otherwise the separate passes
  const bool fused = fused_attn_fits(T, ns) && (n_max <= PICK_MAX || (!cand && L.units > 0));
  char* ws = reinterpret_cast<char*>(workspace);
  FusedAttn f{q, codes, scales, blk_cap, k, win, Wcap, W, B, T, H, d, pos0, pos,
              softmax_scale, out, out_dtype, lse, nullptr, 0, scale_fmt, stream,
              0, reinterpret_cast<uint32_t*>(ws + L.off_hist),
              reinterpret_cast<const int2*>(ws + L.off_tinfo),
              reinterpret_cast<const int2*>(ws + L.off_comp),
              reinterpret_cast<const int32_t*>(ws + L.off_slab), L.npad,
              ListsPlan{L.units, __builtin_ctz(L.lcap > 0 ? L.lcap : 1),
                        __builtin_ctz(TILE / L.sub)},
              cand, cand ? C : 0, m,
              out_idx, out_score, cand ? 0 : fused_alg_bytes(n_max, Hi, Di, k, W, H, d)};
  // the fused list path keeps its scores in the lists (the whole-row walk of
  // massive ties recomputes them from the keys), so its scan writes no slab
  a.write_slab = !(fused && a.lists);
  f.tinfo2 = reinterpret_cast<const int2*>(ws + L.off_tinfo2);
  f.comp2 = reinterpret_cast<const int2*>(ws + L.off_comp2);
  f.q_idx = q_idx;
  f.w = w;
  f.keys = keys;
  f.Hi = Hi;
  f.Di = Di;
  f.slab_ok = a.write_slab;
  // every argument is checked before anything is launched
  st = fused_attn_check(f);
  if (st != CSA_OK) return st;
  const int64_t ab = fused ? fused_attn_workspace(B, T, H, d, ns, f.alg_bytes)
                           : csa_attn_workspace(B, T, H, d, ns);
  if (ab < 0) return CSA_ERR_SHAPE;
  if (!workspace || ws_bytes < ib + ab) return CSA_ERR_WORKSPACE;
  if (!csa_aligned(workspace, 256)) return CSA_ERR_ALIGN;
  f.ws = ab > 0 ? ws + ib : nullptr;
  f.ws_bytes = ws_bytes - ib;
  st = idx_phase(a, 0);
  if (st != CSA_OK || scan_only) return st;
  if (!fused) {
    st = idx_phase(a, 1);
    if (st != CSA_OK) return st;
    if (pos)
      return csa_sparse_attn_ragged(q, codes, scales, blk_cap, out_idx, k, win, Wcap, W, B, T, H, d,
                                    pos, pos0, softmax_scale, out, out_dtype, lse, f.ws,
                                    f.ws_bytes, scale_fmt, stream);
    return csa_sparse_attn(q, codes, scales, blk_cap, out_idx, k, win, Wcap, W, B, T, H, d, pos0,
                           softmax_scale, out, out_dtype, lse, f.ws, f.ws_bytes, scale_fmt,
                           stream);
  }
  f.sel = n_max <= PICK_MAX ? 2 : 1;  // whole score rows, or the scan's lists
  return fused_attn_launch(f);
}

extern "C" int csa_index_attn(CSA_INDEX_ATTN_PARAMS) {
  return index_attn(CSA_INDEX_ATTN_ARGS, false);
}

extern "C" int csa_index_attn_scan(CSA_INDEX_ATTN_PARAMS) {
  return index_attn(CSA_INDEX_ATTN_ARGS, true);
}

#undef CSA_INDEX_ATTN_PARAMS
#undef CSA_INDEX_ATTN_ARGS
