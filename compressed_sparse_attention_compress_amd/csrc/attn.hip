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
// the 64 rows and dequantises each once into LDS as float16, entry-major.
// Keys and values are the same latent rows, so that one copy feeds both
// products: q.k reads it row-wise, p.v reads it through the gfx950
// transposing LDS load, so no transposed second copy is written. Two waves
// serve each group of 32 heads with 32x32x16 f16 MFMA tiles (every LDS byte
// read serves 32 heads): for q.k each takes 32 of the 64 slots over all d
// channels (S^T = K Q^T); the pair exchanges its per-head maxima and its P^T
// operands through LDS; for p.v each takes half of the d channels over all
// 64 slots (O^T += V^T P^T). The head index is the lane's column in both
// products, so no register shuffles are needed between them. The stage is
// double-buffered: the next 64 rows are converted while the current q.k is
// in the matrix cores. O is rescaled only in passes where some head's
// running maximum grew. Ranges of slots of one query can be split over
// workgroups (decode); their partial (o, max, sum) are merged in a fixed
// order.
#include "csa_internal.h"
#include "topk_device.h"

#include <mutex>
#include <type_traits>

namespace {

using csa_topk::FinalPlan;
using csa_topk::NB1;

constexpr int CH = 64;        // slots per staging pass (two 32-slot halves)
constexpr int IDX_CAP = 1024; // entry block ids cached in LDS per refill
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Row stride of the float16 stage, in halfs: d plus 24 (three 16-byte chunks
// past a multiple of the 64 LDS banks). Under this stride the q.k operand
// reads (32 rows, two chunks each) and the staging writes (4 rows x 16 chunks
// 4 apart) spread evenly over the banks and the transposed p.v reads (8 rows x
// 4 chunks) take 1.5x their minimum; with d + 16 the staging writes took 2x
// (measured: the larger part of the kernel's LDS bank-conflict cycles).
template <int D>
constexpr int row_stride() { return D + 24; }

// Transposing LDS read: within each 16-lane group, lane i receives element
// i % 4 of the 4-half words addressed by lanes 4j + i / 4 (j = 0..3).
__device__ inline v4h lds_read_tr(const _Float16* p) {
  return __builtin_bit_cast(
      v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(const_cast<_Float16*>(p))));
}

// bfloat16 bits -> float16 (exact in float16's normal range)
__device__ inline _Float16 bf16_to_f16(uint32_t bits) {
  return (_Float16)__uint_as_float(bits << 16);
}

// Where the entry ids of a query come from: SEL_IDX, an id list the caller
// gives (csa_sparse_attn); SEL_LISTS, the indexer scan's short per-unit
// lists, resolved to the top-k by every workgroup for its own slots
// (lists_select, whose slow path walks the score row); SEL_ROW, the
// indexer's whole score row of a query with few candidates (pick_select).
// With a selection in the kernel, each workgroup writes the out_idx /
// out_score positions of its own slots.
enum { SEL_IDX = 0, SEL_LISTS = 1, SEL_ROW = 2 };

struct SelArgs {
  uint32_t* hist;         // [queries][NB1] score histograms (cleared after use)
  const int2* tinfo;      // [queries][units] (count, cut bin) of the lists (SEL_LISTS)
  const int2* comp;       // [queries][units][lcap] listed (score, entry) (SEL_LISTS)
  const int32_t* slab;    // [queries][npad] scores
  int64_t npad;
  csa_topk::ListsPlan lp; // units, log2 of the list length (SEL_LISTS)
  const int32_t* cand;    // [queries][C] pool, or null
  int C, m_idx;           // pool size; block size of the indexed cache
  int32_t* out_idx;       // [queries][k]
  int32_t* out_score;     // [queries][k] or null
  const int2* tinfo2;     // [queries][units] (count, cut bin) of the wide lists (SEL_LISTS)
  const int2* comp2;      // [queries][units][2 lcap] wide lists (SEL_LISTS)
  const int8_t* q_idx;    // [queries][Hi][Di] indexer rows, w [queries][Hi] and keys
  const int8_t* w;        // [B][blk_cap][Di]: a score of the whole-row walk is recomputed
  const int8_t* keys;     // from them where the scan wrote no slab (slab_ok false)
  int Hi, Di;
  bool slab_ok;
};


// One workgroup per compute unit is all the LDS allows at d = 512, so the
// compiler is told to schedule for one wave per SIMD (registers for LDS
// reads in flight rather than for occupancy).
template <int D, int NG, bool DENSE, int FMT, bool WF, int SEL>
__global__ __launch_bounds__(NG * 128) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_attn(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int64_t blk_cap, const int32_t* __restrict__ idx, int k,
    int m, const uint16_t* __restrict__ win, int Wcap, int W, int T, int H, int64_t pos0,
    const int64_t* __restrict__ qpos, float scale_log2, int nsplit, int spl, int n_queries,
    void* __restrict__ out, int out_dtype,
    float* __restrict__ lse, float* __restrict__ part_o, float2* __restrict__ part_ml,
    SelArgs sa) {
  constexpr int NWV = 2 * NG;                 // waves: (head group, half)
  constexpr int NT = NWV * 64;
  constexpr int RS = row_stride<D>();
  constexpr int KS2 = D / 32;                 // q.k k-steps of 16 channels in one half of d
  constexpr int CT = D / 64;                  // 32-channel output tiles of one half of d
  constexpr int CHUNKS = D / 32;              // 32-channel chunks of a row
  constexpr int TASKS = CH * CHUNKS;          // staging tasks (slot, chunk) per pass
  constexpr int TPT = TASKS / NT;             // staging tasks per thread
  static_assert(TASKS % NT == 0, "tasks must divide evenly");
  constexpr bool E4 = FMT == CSA_SCALE_E4M3_16;
  constexpr int SPE = E4 ? D / 16 : D / 32;   // scale bytes per entry
  static_assert(SEL == SEL_IDX || NT == 256, "the in-kernel selection needs 256 threads");
  // the stage (rows of a pass) and each wave's partial logits of both 32-slot
  // tiles, in register order (a plain vector type: the HIP float4 struct was
  // read back as single dwords, four bank-conflicted reads per value instead
  // of one)
  constexpr int STAGE_BYTES = CH * RS * 2;
  constexpr int LOGIT_BYTES = NWV * 2 * 4 * 64 * 16;
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[STAGE_BYTES + LOGIT_BYTES];
  _Float16* const Rs = reinterpret_cast<_Float16*>(s_raw);
  v4f (*const s_S)[2][4][64] = reinterpret_cast<v4f (*)[2][4][64]>(s_raw + STAGE_BYTES);
  __shared__ int s_blk[IDX_CAP];
  __shared__ unsigned long long s_valid;      // entry slots of the staged pass that are valid

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
  const int i32 = lane & 31, gg = lane >> 5;
  const int head = hg * 32 + i32;

  const int32_t* ibase = (DENSE || SEL != SEL_IDX) ? nullptr : idx + (int64_t)qi * k;
  // entry ids of the first table (slots [s_begin, s_begin + IDX_CAP) of the
  // entry range), requested before the q rows so that both latencies overlap
  constexpr int RPT = (IDX_CAP + NT - 1) / NT;
  const int64_t e_end = s_end < nsel ? s_end : nsel;
  int64_t first_ids[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int64_t sl = s_begin + threadIdx.x + r * NT;
    first_ids[r] = (DENSE || SEL != SEL_IDX || s_begin >= e_end)
                       ? sl
                       : (int64_t)ibase[sl < e_end ? sl : e_end - 1];
  }
  // q.k operand: the two waves of a head group split d; lane (i + 32 gg) of
  // wave half h holds head i's channels h d/2 + 16 kk + 8 gg .. +7 of every
  // k-step kk, as float16
  v8h Qop[KS2];
  const uint8_t* cbase = codes + (int64_t)b * blk_cap * (D / 2);
  const uint8_t* sbase = scales + (int64_t)b * blk_cap * SPE;
  const uint16_t* wbase = win + (int64_t)b * Wcap * D;
  const int64_t ep0 = s_begin, ep1 = e_end;                          // entry slots
  const int64_t wp0 = s_begin > nsel ? s_begin : nsel, wp1 = s_end;  // window slots
  // window staging task (slot c0 + s, 32-channel chunk c): 64 bytes of a row
  struct RawW {
    uint4 w[4];
  };
  auto load_win = [&](RawW& r, int task, int64_t c0) {
    const int c = task % CHUNKS, s = task / CHUNKS;
    const int64_t sl = c0 + s;
    int64_t p = t - W + 1 + (sl - nsel);
    p = p < 0 ? 0 : p;
    // positions and the ring size are below 2^31 (checked at the entry
    // points), so the ring slot takes a 32-bit remainder, not a 64-bit one
    const uint32_t ring = (uint32_t)p % (uint32_t)Wcap;
    const uint4* src = reinterpret_cast<const uint4*>(wbase + (int64_t)ring * D + 32 * c);
#pragma unroll
    for (int u = 0; u < 4; ++u) r.w[u] = src[u];
  };
  constexpr int NPRE = TPT < 2 ? TPT : 2;
  struct RawE {
    uint4 w;
    uint32_t sc;
  };
  RawE eraw[TPT];          // raw bytes of the next entry pass to be staged
  bool eraw_ok = false;    // eraw holds the entry phase's first pass
  RawW wpre[NPRE];  // the first window tasks, requested with the q rows
  bool sel_done = false;   // the in-kernel selection put this range's ids in s_blk
  // an in-kernel selection's loads go out first, before the q rows
  csa_topk::ListsLoad sel_ld;
  if constexpr (SEL == SEL_LISTS) {
    if (ep0 < ep1) {
      const int64_t nu = sa.lp.units;
      sel_ld.load(sa.hist + (int64_t)qi * NB1, sa.tinfo + qi * nu,
                  sa.comp + ((qi * nu) << sa.lp.lshift), sa.lp);
    }
  }
  {
    const int hq = head < H ? head : H - 1;
    const uint16_t* qr = q + ((int64_t)qi * H + hq) * D + half * (D / 2) + 8 * gg;
    v8us raw[KS2];
#pragma unroll
    for (int kk = 0; kk < KS2; ++kk) raw[kk] = *reinterpret_cast<const v8us*>(qr + 16 * kk);
    if (WF && wp0 < wp1) {
#pragma unroll
      for (int u = 0; u < NPRE; ++u) load_win(wpre[u], threadIdx.x + u * NT, wp0);
    }
    // dense attention needs no ids (slot = block), so its first entry pass is
    // requested with the q rows as well (slots past the range read row ep0
    // and are masked like any invalid slot)
    if constexpr (DENSE && !WF && TPT <= 4) {
      if (ep0 < ep1) {
#pragma unroll
        for (int tt = 0; tt < TPT; ++tt) {
          const int task = threadIdx.x + tt * NT;
          const int c = task % CHUNKS;
          const int64_t sl = ep0 + task / CHUNKS;
          const int64_t blk = sl < ep1 ? sl : ep0;
          eraw[tt].w = *reinterpret_cast<const uint4*>(cbase + blk * (D / 2) + 16 * c);
          const uint8_t* sp = sbase + blk * SPE + (E4 ? 2 * c : c);
          eraw[tt].sc = E4 ? ((uint32_t)sp[0] | ((uint32_t)sp[1] << 8)) : (uint32_t)sp[0];
        }
        eraw_ok = true;
      }
    }
    if constexpr (SEL != SEL_IDX) {
      // the query's top-k, resolved here (its loads go out with the q rows);
      // this workgroup keeps the ids of its own entry slots [ep0, ep1) and
      // writes those positions of out_idx / out_score
      if (ep0 < ep1) {
        const uint32_t* hq = sa.hist + (int64_t)qi * NB1;
        const int32_t* cq = sa.cand ? sa.cand + (int64_t)qi * sa.C : nullptr;
        int32_t* oi = sa.out_idx + (int64_t)qi * k;
        int32_t* os = sa.out_score ? sa.out_score + (int64_t)qi * k : nullptr;
        __shared__ uint32_t sel_bh[256];
        __shared__ int sel_tmp[4];
        __shared__ int sel_red[8];
        // emit takes a candidate index (the lists path); emit_id the entry id
        // itself (the whole-row pick loads a pool's ids with the scores)
        auto emit = [&](int pos, int e, int v) {
          if (pos >= ep0 && pos < ep1) {
            int id = cq ? cq[e] : e;
            id = (id >= 0 && id < blk_cap) ? id : -1;
            s_blk[pos - ep0] = id;
            oi[pos] = id;
            if (os) os[pos] = v;
          }
        };
        auto emit_id = [&](int pos, int id, int v) {
          if (pos >= ep0 && pos < ep1) {
            id = (id >= 0 && id < blk_cap) ? id : -1;
            s_blk[pos - ep0] = id;
            oi[pos] = id;
            if (os) os[pos] = v;
          }
        };
        int keff;
        int64_t nv = (t + 1) / sa.m_idx;
        nv = nv < blk_cap ? nv : blk_cap;
        const csa_topk::SelShared sh{nullptr, nullptr, sel_bh, sel_tmp, sel_red};
        if constexpr (SEL == SEL_LISTS) {
          // a spilled selection compacts its candidates into the (still unused) stage
          const int cap = ((STAGE_BYTES + LOGIT_BYTES) / 4 - 2 * sa.lp.units) / 2;
          const int64_t nu = sa.lp.units;
          const csa_topk::ScoreSrc src{
              sa.slab_ok ? sa.slab + (int64_t)qi * sa.npad : nullptr,
              sa.keys + (int64_t)b * blk_cap * sa.Di, sa.q_idx + (int64_t)qi * sa.Hi * sa.Di,
              sa.w + (int64_t)qi * sa.Hi, sa.Hi, sa.Di, reinterpret_cast<int*>(s_raw)};
          keff = sel_ld.resolve(src, (int)nv, k, sa.lp, sh, sa.tinfo + qi * nu,
                                sa.tinfo2 + qi * nu, sa.comp2 + ((qi * nu) << (sa.lp.lshift + 1)),
                                reinterpret_cast<int*>(s_raw), cap, emit);
        } else {
          const int N = cq ? sa.C : (int)nv;
          if (N <= csa_topk::PICK_MAX / 2)
            keff = csa_topk::pick_select<csa_topk::PICK_MAX / 512>(
                sa.slab + (int64_t)qi * sa.npad, cq, hq, N, k, sh, emit_id);
          else
            keff = csa_topk::pick_select<csa_topk::PICK_MAX / 256>(
                sa.slab + (int64_t)qi * sa.npad, cq, hq, N, k, sh, emit_id);
        }
        for (int64_t pos = (keff > ep0 ? keff : ep0) + threadIdx.x; pos < ep1; pos += NT) {
          s_blk[pos - ep0] = -1;
          oi[pos] = -1;
          if (os) os[pos] = -1;
        }
        // the ids are in place and the selection's LDS is free for the stage;
        // a workgroup that is the query's only reader of its histogram clears
        // it for the next call (otherwise the merge does)
        __syncthreads();
        if (nsplit == 1) {
          uint32_t* hw = sa.hist + (int64_t)qi * NB1;
          hw[NB1 - 1 - 2 * (int)threadIdx.x] = 0u;
          hw[NB1 - 2 - 2 * (int)threadIdx.x] = 0u;
        }
        sel_done = true;
      }
    }
#pragma unroll
    for (int kk = 0; kk < KS2; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) Qop[kk][e] = bf16_to_f16(raw[kk][e]);
  }
  v16f O[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[ct][r] = 0.f;
  // running max and sum; both waves of a head group compute the same values
  float m_run = -INFINITY, l_run = 0.f;
  // set when a staged row leaves float16's range: an E8M0 entry with a scale
  // byte above 140 (its largest codes overflow), or a window value of
  // magnitude 2^16 or more (or not finite); the query's output is then NaN
  bool out_of_range = false;

  // The window phase runs first: its rows need no ids, so their loads go out
  // with the q rows and the ids; the first entry gather is then issued during
  // the window passes (its ids are in LDS by then) and converted when the
  // entry phase starts.
  bool ids_stored = sel_done; // s_blk holds the entry phase's first table
  // entry ids of slots [from, from + IDX_CAP) into LDS
  auto store_ids = [&](int64_t from, const int64_t* v) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = threadIdx.x + r * NT;
      const int64_t sl = from + i;
      if (i < IDX_CAP) s_blk[i] = (sl < ep1 && v[r] >= 0 && v[r] < blk_cap) ? (int)v[r] : -1;
    }
  };
  // raw bytes of entry task (slot c0 + s, 32-channel chunk c), chunk fastest
  // across lanes so that 16 lanes (d = 512) read one entry's 256 code bytes
  // contiguously; tab0 is the first slot of the id table in s_blk
  auto load_entry = [&](RawE& r, int task, int64_t c0, int64_t tab0) {
    const int c = task % CHUNKS, s = task / CHUNKS;
    const int64_t sl = c0 + s;
    int blk = (sl < ep1 && sl - tab0 < IDX_CAP) ? s_blk[sl - tab0] : -1;
    const bool used = blk >= 0;
    blk = used ? blk : 0;
    r.w = *reinterpret_cast<const uint4*>(cbase + (int64_t)blk * (D / 2) + 16 * c);
    const uint8_t* sp = sbase + (int64_t)blk * SPE + (E4 ? 2 * c : c);
    const uint32_t sb = E4 ? ((uint32_t)sp[0] | ((uint32_t)sp[1] << 8)) : (uint32_t)sp[0];
    // an unused slot (masked later) stages row 0 at scale 1, so its scale
    // byte never raises the range flag
    r.sc = (E4 || used) ? sb : 127u;
  };

  // One homogeneous phase: window tokens (IS_WIN true) or entries, slots
  // [p0, p1). Loads are unconditional (clamped rows), validity is applied to
  // the logits.
  auto phase = [&](auto is_win_tag, int64_t p0, int64_t p1) {
    constexpr bool IS_WIN = decltype(is_win_tag)::value;
    if (p0 >= p1) return;
    int64_t tab0 = p0;  // first slot whose block id sits in s_blk[0]
    // a later id table: all loads issued before the first is used
    // (addresses clamped into the phase)
    auto refill = [&](int64_t from) {
      __syncthreads();
      tab0 = from;
      int64_t v[RPT];
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int64_t sl = from + threadIdx.x + r * NT;
        v[r] = DENSE ? sl : (int64_t)ibase[sl < p1 ? sl : p1 - 1];
      }
      store_ids(from, v);
      __syncthreads();
    };
    using Raw = typename std::conditional<IS_WIN, RawW, RawE>::type;
    auto load_task = [&](Raw& r, int task, int64_t c0) {
      if constexpr (IS_WIN)
        load_win(r, task, c0);
      else
        load_entry(r, task, c0, tab0);
    };
    auto convert_task = [&](const Raw& r, int task) {
      const int c = task % CHUNKS, s = task / CHUNKS;
      v8h h[4];
      if constexpr (IS_WIN) {
        // largest exponent field of the 32 bfloat16 values (packed halves)
        typedef unsigned short v2us __attribute__((ext_vector_type(2)));
        v2us emax = {0, 0};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t wv[4] = {r.w[u].x, r.w[u].y, r.w[u].z, r.w[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            emax = __builtin_elementwise_max(emax,
                                             __builtin_bit_cast(v2us, wv[e] & 0x7f807f80u));
        }
        out_of_range |= (emax[0] >= 0x4780 || emax[1] >= 0x4780);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t wd[4] = {r.w[u].x, r.w[u].y, r.w[u].z, r.w[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            h[u][2 * e] = bf16_to_f16(wd[e] & 0xffffu);
            h[u][2 * e + 1] = bf16_to_f16(wd[e] >> 16);
          }
        }
      } else if (E4) {
        // E2M1 times an E4M3 scale, formed in float16 (exact: at most 5
        // significant bits, magnitudes 2^-10 .. 2688)
        const _Float16 s0 = (_Float16)e4m3_to_f32(r.sc & 0xffu);
        const _Float16 s1 = (_Float16)e4m3_to_f32(r.sc >> 8);
        h[0] = fp4x8_to_f16(r.w.x, 1.0f) * s0;
        h[1] = fp4x8_to_f16(r.w.y, 1.0f) * s0;
        h[2] = fp4x8_to_f16(r.w.z, 1.0f) * s1;
        h[3] = fp4x8_to_f16(r.w.w, 1.0f) * s1;
      } else {
        out_of_range |= r.sc > 140u;
        const float sc = e8m0_to_f32(r.sc);
        h[0] = fp4x8_to_f16(r.w.x, sc);
        h[1] = fp4x8_to_f16(r.w.y, sc);
        h[2] = fp4x8_to_f16(r.w.z, sc);
        h[3] = fp4x8_to_f16(r.w.w, sc);
      }
      v8h* dst = reinterpret_cast<v8h*>(Rs + s * RS + 32 * c);
#pragma unroll
      for (int u = 0; u < 4; ++u) dst[u] = h[u];
    };
    // entries: raw bytes prefetched one pass ahead (they are small); window
    // rows: loaded right before they are converted, two tasks in flight (the
    // first two tasks of the phase's first pass were issued at kernel start)
    RawE (&raw)[TPT] = eraw;
    bool& have_raw = eraw_ok;  // raw[] holds the pass to be staged (entries only)
    auto stage = [&](int64_t c0, auto first_tag) {
      constexpr bool FIRST = decltype(first_tag)::value;
      if constexpr (IS_WIN) {
        Raw wr[2];
        if constexpr (WF && FIRST) {
#pragma unroll
          for (int u = 0; u < NPRE; ++u) wr[u] = wpre[u];
        } else {
          load_task(wr[0], threadIdx.x, c0);
        }
#pragma unroll
        for (int tt = 0; tt < TPT; ++tt) {
          if (tt + 1 < TPT && !(WF && FIRST && tt + 1 < NPRE))
            load_task(wr[(tt + 1) & 1], threadIdx.x + (tt + 1) * NT, c0);
          convert_task(wr[tt & 1], threadIdx.x + tt * NT);
        }
      } else {
      if (!have_raw) {
#pragma unroll
        for (int tt = 0; tt < TPT; ++tt) load_task(raw[tt], threadIdx.x + tt * NT, c0);
      }
#pragma unroll
      for (int tt = 0; tt < TPT; ++tt) convert_task(raw[tt], threadIdx.x + tt * NT);
      // validity of the staged slots as one 64-bit mask
      if (wave == 0) {
        const int64_t sl = c0 + lane;
        const unsigned long long vm = __ballot(sl < p1 && s_blk[sl - tab0] >= 0);
        if (lane == 0) s_valid = vm;
      }
      // the next pass's raw entries, if its ids are in the table
      have_raw = false;
      if (c0 + CH < p1 && c0 + 2 * CH <= tab0 + IDX_CAP) {
#pragma unroll
        for (int tt = 0; tt < TPT; ++tt) load_task(raw[tt], threadIdx.x + tt * NT, c0 + CH);
        have_raw = true;
      }
      }
    };
    if constexpr (!IS_WIN) {
      // the first table (unless the window phase wrote it): the entry range
      // starts at s_begin, its ids were loaded at kernel start
      if (!ids_stored) {
        store_ids(p0, first_ids);
        ids_stored = true;
        __syncthreads();
      }
    }
    stage(p0, std::true_type{});
    if constexpr (IS_WIN && WF) {
      // the entry phase's first id table, once the window rows are requested
      // (made visible by the barrier below)
      if (ep0 < ep1) {
        store_ids(ep0, first_ids);
        ids_stored = true;
      }
    }
    for (int64_t c0 = p0; c0 < p1; c0 += CH) {
      __syncthreads();  // this pass's rows are staged
      if constexpr (IS_WIN && WF && TPT <= 4) {
        // the entry phase's first gather, in flight during the window passes
        // (not with 8 tasks per thread: their registers would spill)
        if (ids_stored && !eraw_ok) {
#pragma unroll
          for (int tt = 0; tt < TPT; ++tt) load_entry(eraw[tt], threadIdx.x + tt * NT, ep0, ep0);
          eraw_ok = true;
        }
      }
      // validity of this lane's logit slots: tile et, register r holds slot
      // 32 et + 8 (r / 4) + 4 gg + r % 4 of the pass; bit 16 et + r
      uint32_t okm = 0;
      if (IS_WIN) {
#pragma unroll
        for (int r = 0; r < 32; ++r) {
          const int64_t sl = c0 + 32 * (r >> 4) + 8 * ((r >> 2) & 3) + 4 * gg + (r & 3);
          okm |= (uint32_t)(sl < p1 && t - W + 1 + (sl - nsel) >= 0) << r;
        }
      } else {
        const unsigned long long vm = s_valid >> (4 * gg);
#pragma unroll
        for (int n = 0; n < 8; ++n)
          okm |= (uint32_t)((vm >> (32 * (n >> 2) + 8 * (n & 3))) & 0xfu) << (4 * n);
      }
      // partial S^T[slot][head] of both 32-slot tiles over this wave's half of d
      v16f S[2];
#pragma unroll
      for (int et = 0; et < 2; ++et)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[et][r] = 0.f;
      const _Float16* krow = Rs + i32 * RS + half * (D / 2) + 8 * gg;
      // key operands read 8 at a time ahead of their products, so that the
      // LDS latency is paid once per batch
#pragma unroll
      for (int k0 = 0; k0 < KS2; k0 += 4) {
        v8h ka[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int et = 0; et < 2; ++et)
            ka[u][et] = *reinterpret_cast<const v8h*>(krow + 32 * et * RS + 16 * (k0 + u));
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int et = 0; et < 2; ++et)
            S[et] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[u][et], Qop[k0 + u], S[et], 0, 0, 0);
      }
#pragma unroll
      for (int et = 0; et < 2; ++et)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          s_S[wave][et][q4][lane] = v4f{S[et][4 * q4], S[et][4 * q4 + 1], S[et][4 * q4 + 2],
                                           S[et][4 * q4 + 3]};
      __syncthreads();
      // full logits of the 64 slots (own half of d + the partner's)
      float x[32];
      float cmax = -INFINITY;
#pragma unroll
      for (int et = 0; et < 2; ++et)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const v4f o = s_S[partner][et][q4][lane];
          const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * et + 4 * q4 + e;
            // the same sum in both waves: lower half of d first
            const float sv = half == 0 ? S[et][4 * q4 + e] + ov[e] : ov[e] + S[et][4 * q4 + e];
            x[r] = (okm >> r) & 1u ? sv * scale_log2 : -INFINITY;
            cmax = fmaxf(cmax, x[r]);
          }
        }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      // online-softmax rescale (128 accumulator values in AGPRs per lane),
      // skipped unless some head of the wave saw its max grow by more than
      // four (log2 units), so the reference max lags by at most 4 and p stays
      // at most 16 in fp16 (the branch is wave-uniform; heads whose max did
      // not grow get alpha = 1). With p as two float16 terms the measured
      // attention errors are the same for a lag of 1 and of 4 (with one term
      // a lag of 2 or 4 had raised them).
      if (__ballot(cmax > m_run + 4.0f)) {
        const float m_new = fmaxf(m_run, cmax);
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        // a head that has seen no finite logit yet has O = 0, so the multiply
        // is skipped while that holds for every head of the wave (the first
        // pass of every workgroup)
        if (__ballot(m_run != -INFINITY)) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) O[ct] *= alpha;
        }
        m_run = m_new;
      }
      const bool none = m_run == -INFINITY;
      // P^T operands of the four 16-slot k-steps: element e of lane
      // (i + 32 gg) in k-step ks = 2 et + s is slot 32 et + 16 s + 8 (e / 4) +
      // 4 gg + e % 4, head i (logit registers 8 s .. 8 s + 7 of tile et)
      // p goes into the product as two float16 terms, p = ph + pl with pl the
      // float16 rounding of p - ph (exact in float32), so each weight carries
      // about 22 significant bits: one float16 term alone moves up to 2^-11 of
      // a weight between value rows, which for a query with a few slots of
      // large, different values exceeds the output tolerance.
      v8h P[4], Pl[4];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        // hardware exp2 (results below 2^-126 flush to 0, far under the
        // weights' resolution)
        const float pv = none ? 0.f : __builtin_amdgcn_exp2f(x[r] - m_run);
        const _Float16 ph = (_Float16)pv;
        P[r >> 3][r & 7] = ph;
        Pl[r >> 3][r & 7] = (_Float16)(pv - (float)ph);
        psum += pv;
      }
      l_run += psum;
      // O^T[channel][head] += V^T P^T over the 64 slots, for this wave's half
      // of the channels. V^T operand of k-step ks (slots 16 ks ..): lane
      // (i + 32 gg) needs slot 16 ks + 8 a + 4 gg + j of channel i for a = 0, 1
      // and j = 0..3; in the transposing read, lane 16 G + 4 j + c (G = lane /
      // 16) addresses row 16 ks + 8 a + 4 (G / 2) + j, channels 16 (G % 2) + 4 c
      // .. + 3 of the tile.
      const int G = lane >> 4, jj = (lane >> 2) & 3, cc = lane & 3;
      const _Float16* vbase = Rs + (4 * (G >> 1) + jj) * RS + half * (D / 2) + 16 * (G & 1) + 4 * cc;
      // one k-step at a time: the scheduler is kept from hoisting every
      // transposed read of the pass (their registers would push the q.k
      // operands out of the VGPRs)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const _Float16* vp = vbase + 16 * ks * RS + 32 * ct;
          const v4h lo = lds_read_tr(vp);
          const v4h hi = lds_read_tr(vp + 8 * RS);
          const v8h A = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, P[ks], O[ct], 0, 0, 0);
          O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, Pl[ks], O[ct], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c0 + CH < p1) {
        __syncthreads();  // every read of this pass's rows is done
        if (!IS_WIN && SEL == SEL_IDX && c0 + 2 * CH > tab0 + IDX_CAP) refill(c0 + CH);
        stage(c0 + CH, std::false_type{});
      }
    }
    __syncthreads();  // the stage may be rewritten by the next phase
  };
  if constexpr (WF) {
    phase(std::true_type{}, wp0, wp1);
    phase(std::false_type{}, ep0, ep1);
  } else {
    phase(std::false_type{}, ep0, ep1);
    phase(std::true_type{}, wp0, wp1);
  }

  // softmax denominator: the two lanes of a head hold the two halves of the slots
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  // a row outside float16's range anywhere in the workgroup makes the whole
  // output of the query NaN (a split's NaN partial carries into the merge)
  const bool bad = __syncthreads_or(out_of_range ? 1 : 0) != 0;
  const float inv = bad ? __builtin_nanf("") : (l_tot > 0.f ? 1.f / l_tot : 0.f);
  // output register r of tile ct: channel half (d/2) + 32 ct + 8 (r / 4) + 4 gg + r % 4
  if (nsplit == 1 && out_dtype != CSA_F32) {
    // bfloat16 output of a whole query through LDS (the stage is free now):
    // each lane's 8-byte pieces sit 1 KB apart in the output (one head per
    // lane), so they are written into a head-major copy first and then leave
    // in 16-byte pieces, 1 KB contiguous per wave instruction
    constexpr int OROW = D + 8;  // bfloat16 per LDS row (16 B past the row)
    static_assert(NWV * 32 / 2 * OROW * 2 <= STAGE_BYTES + LOGIT_BYTES, "output rows fit");
    __bf16* ol = reinterpret_cast<__bf16*>(s_raw);
    typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
    const int hl = hg * 32 + i32;  // the lane's head within the workgroup
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = half * (D / 2) + 32 * ct + 8 * q4 + 4 * gg;
        const v4bf v = {(__bf16)(O[ct][4 * q4] * inv), (__bf16)(O[ct][4 * q4 + 1] * inv),
                        (__bf16)(O[ct][4 * q4 + 2] * inv), (__bf16)(O[ct][4 * q4 + 3] * inv)};
        *reinterpret_cast<v4bf*>(ol + hl * OROW + c) = v;
      }
    __syncthreads();
    constexpr int CPR = D / 8;               // 16-byte pieces per row
    constexpr int PIECES = NWV * 16 * CPR;   // rows = NG * 32 heads
    __bf16* ob = reinterpret_cast<__bf16*>(out) + (int64_t)qi * H * D;
#pragma unroll
    for (int i = threadIdx.x; i < PIECES; i += NT) {
      const int row = i / CPR, cp = i % CPR;
      if (row < H)
        *reinterpret_cast<uint4*>(ob + (int64_t)row * D + 8 * cp) =
            *reinterpret_cast<const uint4*>(ol + row * OROW + 8 * cp);
    }
    if (lse && head < H && half == 0 && gg == 0)
      lse[(int64_t)qi * H + head] =
          bad ? __builtin_nanf("") : (m_run + log2f(l_tot)) * 0.69314718055994531f;
    return;
  }
  if (head >= H) return;
  if (nsplit == 1) {
    const int64_t base = ((int64_t)qi * H + head) * D + half * (D / 2) + 4 * gg;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = 32 * ct + 8 * q4;
        const float v0 = O[ct][4 * q4] * inv, v1 = O[ct][4 * q4 + 1] * inv;
        const float v2 = O[ct][4 * q4 + 2] * inv, v3 = O[ct][4 * q4 + 3] * inv;
        if (out_dtype == CSA_F32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + base + c) =
              float4{v0, v1, v2, v3};
        } else {
          typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
          const v4bf v = {(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
          *reinterpret_cast<v4bf*>(reinterpret_cast<__bf16*>(out) + base + c) = v;
        }
      }
    if (lse && half == 0 && gg == 0)
      lse[(int64_t)qi * H + head] =
          bad ? __builtin_nanf("") : (m_run + log2f(l_tot)) * 0.69314718055994531f;
  } else {
    // the split's partial output sum p v (not divided by its l: the merge
    // weights it by 2^(m - M) alone) in float32, stored in register order
    // [query][split][wave][column tile][r / 4][lane][4], so every store of a
    // wave is 1 KB contiguous; m and l in float32 (NaN for a row out of
    // float16's range, which the merge carries into the query's output)
    float* pw = part_o + (((int64_t)qi * nsplit + split) * NWV + wave) * (CT * 1024) + lane * 4;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(pw + (4 * ct + q4) * 256) =
            float4{O[ct][4 * q4], O[ct][4 * q4 + 1], O[ct][4 * q4 + 2], O[ct][4 * q4 + 3]};
    if (half == 0 && gg == 0)
      part_ml[((int64_t)qi * nsplit + split) * H + head] =
          bad ? float2{__builtin_nanf(""), __builtin_nanf("")} : float2{m_run, l_tot};
  }
}

// Merge of the split partials, one workgroup per (query, 32-head group,
// 32-channel tile), one thread per (register quad, lane) of that tile: weights
// 2^(m_s - M) / L on the partial outputs (L = sum of l_s 2^(m_s - M)), summed
// in split order. The partials are read in the register order the attention kernel
// wrote them, 4 KB contiguous per split; thread (q4, lane) holds head lane %
// 32 and channels 8 q4 + 4 (lane / 32) .. +3 of the tile. Every thread loads
// its head's (max, sum) of all splits and its partials of all splits in one
// round (indices clamped, surplus splits weighted 0), so the merge is one
// memory round trip with no LDS and no barrier.
constexpr int MERGE_MAX = 32;  // splits per query handled by the merge
template <int D, int NS>       // NS >= nsplit loads in flight per thread
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ part_o,
                                                    const float2* __restrict__ part_ml,
                                                    int nsplit, int H, int NG, int n_queries,
                                                    void* __restrict__ out, int out_dtype,
                                                    float* __restrict__ lse,
                                                    uint32_t* __restrict__ hist_clear) {
  constexpr int CT = D / 64;      // tiles per wave (half of d)
  constexpr int TILES = D / 32;   // tiles of a head group
  // Workgroups are dealt to the XCDs round-robin; every workgroup of query qi
  // goes to XCD qi % 8, where the attention kernel wrote that query's
  // partials, so they are read from that XCD's L2.
  const int per_q = NG * TILES;
  const int xcd = blockIdx.x & 7;
  const int jx = blockIdx.x >> 3;
  const int64_t qi = xcd + 8 * (int64_t)(jx / per_q);
  if (qi >= n_queries) return;
  const int rr = jx % per_q;
  // an in-kernel selection read the query's indexer histogram in every split:
  // the first merge workgroup of the query clears it for the next call
  if (hist_clear && rr == 0) {
    uint32_t* hq = hist_clear + qi * NB1;
    hq[NB1 - 1 - 2 * (int)threadIdx.x] = 0u;
    hq[NB1 - 2 - 2 * (int)threadIdx.x] = 0u;
  }
  const int tile = rr % TILES, hg = rr / TILES;
  const int hf = tile / CT, ct = tile % CT;
  const int wave = 2 * hg + hf;
  const int q4 = threadIdx.x >> 6, ln = threadIdx.x & 63;
  const int j = ln & 31, gg = ln >> 5;
  const int h = hg * 32 + j;
  const int hc = h < H ? h : H - 1;
  const int NWV = 2 * NG;
  const int64_t split_stride = (int64_t)NWV * CT * 1024;
  const float* src = part_o + (qi * nsplit * NWV + wave) * (CT * 1024) + (4 * ct + q4) * 256 + ln * 4;
  const float2* mls = part_ml + qi * nsplit * H + hc;
  float2 ml[NS];
  float4 po[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int sp = s < nsplit ? s : 0;
    ml[s] = mls[(int64_t)sp * H];
    po[s] = *reinterpret_cast<const float4*>(src + (int64_t)sp * split_stride);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nsplit) M = fmaxf(M, ml[s].x);
  float L = 0.f;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float f = (s >= nsplit || ml[s].x == -INFINITY) ? 0.f : exp2f(ml[s].x - M);
    L += ml[s].y * f;
    acc.x += po[s].x * f; acc.y += po[s].y * f;
    acc.z += po[s].z * f; acc.w += po[s].w * f;
  }
  if (h >= H) return;
  if (lse && tile == 0 && q4 == 0 && gg == 0)
    lse[qi * H + h] = (M + log2f(L)) * 0.69314718055994531f;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int64_t o_off = (qi * H + h) * D + hf * (D / 2) + 32 * ct + 8 * q4 + 4 * gg;
  if (out_dtype == CSA_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + o_off) =
        float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  } else {
    typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
    const v4bf v = {(__bf16)(acc.x * inv), (__bf16)(acc.y * inv), (__bf16)(acc.z * inv),
                    (__bf16)(acc.w * inv)};
    *reinterpret_cast<v4bf*>(reinterpret_cast<__bf16*>(out) + o_off) = v;
  }
}

struct AttnPlan {
  int nsplit, spl;
  int64_t ws_bytes;
};

// Decode (T < 16): the slots of a query are split over workgroups in whole
// 64-slot passes, at most ~32 splits per query (~16 for very long dense
// ranges, >= n/16 slots each, where the partials would otherwise dominate).
// The plan depends on the query's slot count only, never on the batch: a
// sequence's output bits are the same in any batch ("batch invariant
// kernels"). Longer query runs take one workgroup per query. two_groups:
// the kernel runs both 32-head groups whatever H is (in-kernel selection),
// so the partials hold 64 heads. alg_bytes > 0 (the fused call, which knows
// the query's whole algorithmic traffic): the splits are also capped so that
// their partials, written and read back, cost about the query's own
// algorithmic HBM bytes at most (rounded up to a whole split: a 1M-token
// query may split into 1-pass ranges; a 32K-token query keeps a few
// multi-pass ranges).
static AttnPlan attn_plan(int B, int T, int H, int d, int64_t n_slots, bool two_groups = false,
                          int64_t alg_bytes = 0) {
  AttnPlan p;
  const int64_t hpad = two_groups ? 64 : 32 * ((H + 31) / 32);
  if (T >= 16 || n_slots <= CH) {
    p.nsplit = 1;
    p.spl = (int)(((n_slots + CH - 1) / CH) * CH);
    if (p.spl < CH) p.spl = CH;
  } else {
    const int64_t div = n_slots > 4096 ? 16 : 32;
    int64_t spl = ((n_slots + div - 1) / div + CH - 1) / CH * CH;
    if (alg_bytes > 0) {
      const int64_t prt = 2 * hpad * d * 4;  // a split's partial, written and read back
      int64_t cap = (alg_bytes + prt - 1) / prt;
      cap = cap < 1 ? 1 : cap;
      const int64_t spl_cap = ((n_slots + cap - 1) / cap + CH - 1) / CH * CH;
      spl = spl > spl_cap ? spl : spl_cap;
    }
    p.spl = (int)spl;
    p.nsplit = (int)((n_slots + spl - 1) / spl);
  }
  p.ws_bytes = 0;
  if (p.nsplit > 1) {
    const int64_t units = (int64_t)B * T * p.nsplit;
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
  int sel = SEL_IDX;             // where the entry ids come from
  SelArgs sa{};                  // the indexer's results, for an in-kernel selection
  int64_t alg_bytes = 0;         // per-query algorithmic bytes (fused call), for the plan
};

template <int D, bool DENSE, int FMT>
static void launch_attn(const AttnArgs& a, const AttnPlan& p, float* part_o, float2* part_ml) {
  // an in-kernel selection runs in 256 threads (two head groups)
  const int ng = a.sel != SEL_IDX ? 2 : (a.H + 31) / 32;
  const int64_t nq = (int64_t)a.B * a.T;
  const dim3 grid((unsigned)(((nq + 7) / 8) * 8 * p.nsplit));
  const float sl2 = a.softmax_scale * 1.4426950408889634f;
#define CSA_LAUNCH_ATTN_S(NG, WF, SS)                                                         \
  hipLaunchKernelGGL((k_attn<D, NG, DENSE, FMT, WF, SS>), grid, dim3(NG * 128), 0, a.stream,     \
                     a.q, a.codes, a.scales, a.blk_cap, a.idx, a.k, a.m, a.win, a.Wcap, a.W, a.T, \
                     a.H, a.pos0, a.pos, sl2, p.nsplit, p.spl, (int)nq, a.out, a.out_dtype, a.lse, \
                     part_o, part_ml, a.sa)
#define CSA_LAUNCH_ATTN(NG, WF) CSA_LAUNCH_ATTN_S(NG, WF, SEL_IDX)
  // a workgroup that takes a whole query (runs of queries) stages the window
  // first so that its start-up loads overlap; split queries keep the entries
  // first (measured faster there)
  if constexpr (!DENSE) {
    if (a.sel == SEL_LISTS) {
      CSA_LAUNCH_ATTN_S(2, false, SEL_LISTS);
    } else if (a.sel == SEL_ROW) {
      CSA_LAUNCH_ATTN_S(2, false, SEL_ROW);
    }
  }
  if (a.sel != SEL_IDX) {
    // launched above
  } else if (p.nsplit == 1) {
    if (ng == 1) CSA_LAUNCH_ATTN(1, true);
    else CSA_LAUNCH_ATTN(2, true);
  } else {
    if (ng == 1) CSA_LAUNCH_ATTN(1, false);
    else CSA_LAUNCH_ATTN(2, false);
  }
#undef CSA_LAUNCH_ATTN
#undef CSA_LAUNCH_ATTN_S
  if (p.nsplit > 1) {
    const dim3 mgrid((unsigned)(((nq + 7) / 8) * 8 * ng * (D / 32)));
#define CSA_LAUNCH_MERGE(NS)                                                                 \
  hipLaunchKernelGGL((k_attn_merge<D, NS>), mgrid, dim3(256), 0, a.stream, part_o, part_ml, \
                     p.nsplit, a.H, ng, (int)nq, a.out, a.out_dtype, a.lse,                 \
                     a.sel != SEL_IDX ? a.sa.hist : nullptr)
    if (p.nsplit <= 8) CSA_LAUNCH_MERGE(8);
    else if (p.nsplit <= 16) CSA_LAUNCH_MERGE(16);
    else if (p.nsplit <= 24) CSA_LAUNCH_MERGE(24);
    else CSA_LAUNCH_MERGE(MERGE_MAX);
#undef CSA_LAUNCH_MERGE
  }
}

// Host argument checks of attn_run (everything but the workspace); on
// success *nsel is the number of entry slots per query.
static int attn_validate(const AttnArgs& a, bool dense, int64_t* nsel_out) {
  if (a.B < 0 || a.T < 0 || a.blk_cap < 0 || a.pos0 < 0) return CSA_ERR_SHAPE;
  if (a.d != 128 && a.d != 256 && a.d != 512) return CSA_ERR_SHAPE;
  if (a.H < 1 || a.H > 64) return CSA_ERR_SHAPE;
  if (a.W < 1 || a.Wcap < a.W) return CSA_ERR_SHAPE;
  if ((int64_t)a.Wcap < (int64_t)a.W + a.T - 1) return CSA_ERR_RANGE;
  if (a.pos0 > 0x7fffffffLL - a.T) return CSA_ERR_RANGE;  // positions fit 31 bits
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
  if (nsel > 0 && !csa_aligned(a.codes, 16)) return CSA_ERR_ALIGN;
  *nsel_out = nsel;
  return CSA_OK;
}

static int attn_run(const AttnArgs& a, bool dense) {
  int64_t nsel = 0;
  const int st = attn_validate(a, dense, &nsel);
  if (st != CSA_OK || a.B == 0 || a.T == 0) return st;
  const bool two = a.sel != SEL_IDX;
  const AttnPlan p = attn_plan(a.B, a.T, a.H, a.d, nsel + a.W, two, a.alg_bytes);
  if (((int64_t)a.B * a.T + 7) / 8 * 8 * p.nsplit > 0x7fffffffLL) return CSA_ERR_SHAPE;
  if (p.nsplit > MERGE_MAX) return CSA_ERR_SHAPE;  // the plan keeps it at <= 32
  float* part_o = nullptr;
  float2* part_ml = nullptr;
  if (p.nsplit > 1) {
    if (!a.ws || a.ws_bytes < p.ws_bytes) return CSA_ERR_WORKSPACE;
    if (!csa_aligned(a.ws, 256)) return CSA_ERR_ALIGN;
    const int64_t units = (int64_t)a.B * a.T * p.nsplit;
    const int64_t hpad = two ? 64 : 32 * ((a.H + 31) / 32);
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

namespace csa_topk {

// The attention half of csa_index_attn: every workgroup resolves its query's
// top-k from the indexer results in the workspace, then attends.
static AttnArgs fused_args(const FusedAttn& f) {
  // (idx: the call's out_idx, which the kernels write rather than read)
  AttnArgs a{f.q, f.codes, f.scales, f.blk_cap, f.out_idx, f.k, 1, f.win, f.Wcap, f.W, f.B, f.T,
             f.H, f.d, f.pos0, f.softmax_scale, f.out, f.out_dtype, f.lse, f.ws, f.ws_bytes,
             f.stream};
  a.pos = f.pos;
  a.scale_fmt = f.scale_fmt;
  a.sel = f.sel;
  a.sa = SelArgs{f.hist,    f.tinfo,   f.comp,  f.slab,  f.npad,  f.lp,   f.cand,
                 f.C,       f.m_idx,   f.out_idx, f.out_score, f.tinfo2, f.comp2, f.q_idx,
                 f.w,       f.keys,    f.Hi,    f.Di,    f.slab_ok};
  a.alg_bytes = f.alg_bytes;
  return a;
}

int64_t fused_attn_workspace(int B, int T, int H, int d, int64_t n_slots, int64_t alg_bytes) {
  return attn_plan(B, T, H, d, n_slots, true, alg_bytes).ws_bytes;
}

bool fused_attn_fits(int T, int64_t n_slots) {
  // one id table per workgroup (IDX_CAP slots) and at most MERGE_MAX splits
  return T < 16 && n_slots <= (int64_t)IDX_CAP * MERGE_MAX;
}

int fused_attn_check(const FusedAttn& f) {
  int64_t nsel = 0;
  return attn_validate(fused_args(f), false, &nsel);
}

int fused_attn_launch(const FusedAttn& f) { return attn_run(fused_args(f), false); }

}  // namespace csa_topk

// Scratch of csa_sparse_attn_noalloc: the split partials live in this
// file-scope device array instead of a caller workspace. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in);
// the device address is looked up once per device with hipGetSymbolAddress
// and kept.
constexpr int64_t NOALLOC_SCRATCH_BYTES = (int64_t)CSA_NOALLOC_SCRATCH_MAX;
__device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device (looked up on the first
// call per device), or null if the lookup failed.
static void* noalloc_scratch() {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

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

extern "C" int csa_sparse_attn_noalloc(const uint16_t* q, const uint8_t* codes,
                                       const uint8_t* scales, int64_t blk_cap, const int32_t* idx,
                                       int k, const uint16_t* win, int Wcap, int W, int B, int T,
                                       int H, int d, int64_t pos0, float softmax_scale, void* out,
                                       int out_dtype, float* lse, int scale_fmt,
                                       hipStream_t stream) {
  AttnArgs a{q, codes, scales, blk_cap, idx, k, 1, win, Wcap, W, B, T, H, d, pos0,
             softmax_scale, out, out_dtype, lse, nullptr, 0, stream};
  a.scale_fmt = scale_fmt;
  // argument errors first, then the plan's scratch against the static array,
  // all before the array's address is looked up or anything is launched
  int64_t nsel = 0;
  const int st = attn_validate(a, false, &nsel);
  if (st != CSA_OK || B == 0 || T == 0) return st;
  const int64_t need = attn_plan(B, T, H, d, nsel + W).ws_bytes;
  if (need > NOALLOC_SCRATCH_BYTES) return CSA_ERR_SCRATCH;
  if (need > 0) {
    a.ws = noalloc_scratch();
    if (!a.ws) return CSA_ERR_HIP;
    a.ws_bytes = NOALLOC_SCRATCH_BYTES;
  }
  return attn_run(a, false);
}
