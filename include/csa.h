/*
 * csa.h -- C ABI of the MI355X (gfx950) compressed sparse attention library.
 *
 * The method (DeepSeek-V4-style compressed sparse attention) as described on
 * the public pages this library follows:
 *  - "Frontier Architecture Decoding Notes (4): DeepSeek V4", section 1
 *    "Attention: CSA + HCA Hybrid": the KV is compressed into 4-token blocks
 *    and a top-k of blocks is attended (CSA); a much heavier compression (up
 *    to 128 tokens per entry) is attended densely (HCA); the newest 128
 *    tokens are attended uncompressed.
 *  - "Recent Developments in LLM Architectures: KV Sharing, mHC, and
 *    Compressed Attention", section "Data": the cache is shortened along the
 *    sequence by summarising groups of tokens.
 *  - podcast transcript "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
 *    Compression": cue 8 (one shared latent entry serves every query head),
 *    cue 12 (Full / Reindex / Reuse layer modes), cue 14 (the indexer scores
 *    every causally visible entry; Reindex layers search a shared candidate
 *    pool), cue 16 (the main cache is MXFP4 with E2M1 elements and is
 *    dequantised just before attention).
 * Steps the pages leave open are fixed as follows: a block's entry is the
 * softmax-gated weighted sum of its m token latents (one gate logit per
 * token); MXFP4 follows the OCP MX v1.0 rule (one E8M0 scale per 32
 * elements, exponent floor(log2 amax) - 2, round-to-nearest-even on the E2M1
 * grid, saturating); the indexer score of block b is
 * sum_h w[h] * max(0, q[h] . key[b]) in exact int32, ties broken toward the
 * lower block index; all selected entries and the window share one softmax,
 * keys and values both being the latent row.
 *
 * Conventions for every call:
 *  - All data pointers are DEVICE pointers on the current HIP device. The
 *    caller owns every buffer; the library allocates nothing.
 *  - Calls are asynchronous: they enqueue kernels on `stream` and return.
 *    Argument errors are detected on the host before anything is launched
 *    and return a negative csa_status; a failed launch returns CSA_ERR_HIP.
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - bfloat16 data is passed as uint16_t bit patterns.
 *  - Layouts are dense and row-major in the order the brackets give.
 *  - Calls that share a workspace must not overlap in time (same stream, or
 *    externally ordered). Calls with distinct workspaces are independent.
 */
#ifndef CSA_H
#define CSA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum csa_status {
  CSA_OK = 0,
  CSA_ERR_NULL = -1,       /* a required pointer is NULL                     */
  CSA_ERR_SHAPE = -2,      /* unsupported or inconsistent sizes              */
  CSA_ERR_RANGE = -3,      /* positions / block ranges outside the buffers   */
  CSA_ERR_WORKSPACE = -4,  /* workspace missing or smaller than required     */
  CSA_ERR_DTYPE = -5,      /* unknown dtype code                             */
  CSA_ERR_HIP = -6,        /* a HIP launch or runtime call failed            */
  CSA_ERR_ALIGN = -7,      /* a pointer or stride breaks the stated alignment */
  CSA_ERR_SCRATCH = -8     /* the call needs more scratch than the library's
                              static buffer holds (csa_sparse_attn_noalloc) */
};

/* Size of the static device scratch of csa_sparse_attn_noalloc, in bytes. */
#define CSA_NOALLOC_SCRATCH_MAX (64 << 20)

enum csa_dtype { CSA_BF16 = 0, CSA_F32 = 1, CSA_F16 = 2 };

/* Scale format of the FP4 cache (every call that reads or writes codes and
 * scales takes one; an unknown value returns CSA_ERR_DTYPE):
 *  CSA_SCALE_E8M0_32  one E8M0 byte per 32 channels, the OCP MX v1.0 MXFP4
 *                     rule: exponent floor(log2 amax) - 2; scales [..][d/32].
 *  CSA_SCALE_E4M3_16  one OCP E4M3 byte per 16 channels, no global scale
 *                     (podcast cue 16 names E4M3 scales per 16 channels): the
 *                     E4M3 value nearest to amax / 6, ties to the even byte,
 *                     saturating at 448; codes round to the nearest multiple
 *                     of the scale on the E2M1 grid, ties to even, saturating
 *                     at 6; a zero scale gives zero codes; scales [..][d/16].
 * Both formats dequantise exactly to bfloat16, and to float16 (E8M0 only for
 * scale bytes in [104, 140], E4M3 over its whole range). */
enum csa_scale_fmt { CSA_SCALE_E8M0_32 = 0, CSA_SCALE_E4M3_16 = 1 };

/* Human-readable name of a status code (static string, never NULL). */
const char* csa_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int csa_version(void);

/* Closed form, host only: bytes of FP4 codes + scales for n_tokens tokens
 * compressed m tokens per entry, d channels: ceil(n_tokens/m) * (d/2 + d/32)
 * (E8M0 scales) or ceil(n_tokens/m) * (d/2 + d/16) (E4M3 scales). Returns -1
 * for n_tokens < 0, m < 1, d not a positive multiple of 32 or an unknown
 * scale format. */
int64_t csa_cache_bytes(int64_t n_tokens, int d, int m, int scale_fmt);

/* ---------------------------------------------------------------------------
 * Block compression + FP4 quantisation (the compressed cache write).
 * Summarises tokens [tok0, tok0 + n_tok) of each of B sequences into entries
 * tok0/m .. ceil((tok0 + n_tok)/m) - 1 ("Frontier Architecture Decoding
 * Notes (4)", section 1: 4-token CSA blocks, up to 128 for HCA; podcast
 * cue 16: FP4 cache). For each block, w = softmax(gate over its tokens) and
 * p = sum_j w_j * kv_j, computed in float64; then p is quantised to FP4 in
 * scale_fmt (every 32-channel group with an E8M0 scale, or every 16-channel
 * group with an E4M3 scale). A final partial block pools the tokens present.
 *   kv     float32 [B][n_tok][kv_ld] (first d columns used), 16-byte aligned,
 *          kv_ld % 4 == 0
 *   gate   float32 [B][n_tok]
 *   codes  uint8  [B][blk_cap][d/2]  E2M1 codes, channel 2i in the low nibble
 *          of byte i (sign in bit 3); 4-byte aligned
 *   scales uint8  [B][blk_cap][d/32] E8M0 exponents (value 2^(byte-127)), or
 *          [B][blk_cap][d/16] E4M3 scales
 * Requires 1 <= m <= 128, tok0 % m == 0, d in {32, 64, 128, 256, 512},
 * n_tok >= 0, and the last entry < blk_cap (else CSA_ERR_RANGE).
 * Inputs must be finite. Entries outside the range are left untouched.
 * ------------------------------------------------------------------------- */
int csa_compress_quantize(const float* kv, int64_t kv_ld, const float* gate,
                          int B, int64_t tok0, int64_t n_tok, int d, int m,
                          uint8_t* codes, uint8_t* scales, int64_t blk_cap,
                          int scale_fmt, hipStream_t stream);

/* Dequantise entries [blk0, blk0 + n_blk) of each sequence (podcast cue 16:
 * the cache is expanded just before attention) with the same conversion the
 * attention kernels use. out: [B][n_blk][d] in out_dtype (CSA_BF16, CSA_F16
 * or CSA_F32). E8M0: BF16 and F32 are exact for scale bytes up to 252 (the
 * largest a finite float32 input can produce; above it large codes overflow
 * to +-inf); F16 is exact for scale bytes in [104, 140]. E4M3: exact in all
 * three. */
int csa_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t blk_cap,
                   int B, int64_t blk0, int64_t n_blk, int d,
                   void* out, int out_dtype, int scale_fmt, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Decode append: one new token for each of B sequences, each at its own
 * position ("Frontier Architecture Decoding Notes (4)", section 1: finished
 * 4-token blocks are compressed, the newest 128 tokens stay uncompressed).
 * For sequence b with t = pos[b] >= 0 (sequences with pos[b] < 0 are left
 * untouched):
 *   - the token's bf16 rounding (nearest, ties to even) goes to win[b][t % Wcap];
 *   - its float32 latent and gate go to the staging row stage[b][t % m];
 *   - if t % m == m - 1, the block's m staged tokens are pooled and quantised
 *     into entry t / m exactly as csa_compress_quantize would (skipped when
 *     t / m >= blk_cap).
 * A block still being filled gets no entry (no query can see it). After a
 * one-shot csa_compress_quantize of tokens 0 .. P-1 that ends inside a
 * block, the caller copies that block's P % m tokens and gates into staging
 * rows 0 .. P % m - 1 before the first append.
 *   kv     float32 [B][kv_ld] (first d used), 16-byte aligned, kv_ld % 4 == 0
 *   gate   float32 [B]
 *   pos    int64 [B] DEVICE array, 8-byte aligned
 *   stage  float32 [B][m][d], 16-byte aligned;  stage_gate float32 [B][m]
 *   codes / scales  as in csa_compress_quantize;  win bf16 [B][Wcap][d], 16-byte aligned
 * Requires 1 <= m <= 128, d in {32, 64, 128, 256, 512}, Wcap >= 1.
 * ------------------------------------------------------------------------- */
int csa_decode_append(const float* kv, int64_t kv_ld, const float* gate,
                      const int64_t* pos, int B, int d, int m,
                      float* stage, float* stage_gate,
                      uint8_t* codes, uint8_t* scales, int64_t blk_cap,
                      uint16_t* win, int Wcap, int scale_fmt, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Indexer + top-k (podcast cues 12 and 14: a light indexer scores every
 * causally visible compressed entry and keeps the top-k; a Reindex layer
 * scores only a candidate pool that an earlier Full layer chose).
 * Queries sit at positions pos0 .. pos0 + T - 1 of every sequence. Block b is
 * visible to position t when (b + 1) * m - 1 <= t (and b < blk_cap).
 *   q_idx  int8 [B][T][Hi][Di]        indexer queries, 16-byte aligned
 *   w      int8 [B][T][Hi]            head weights, must lie in [0, 127]
 *   keys   int8 [B][blk_cap][Di]      one key per entry, 16-byte aligned
 *   cand   int32 [B][T][C] or NULL    Reindex pool: block ids in ascending
 *          order, -1 entries anywhere are ignored, and so are blocks that are
 *          not visible. The tie-break then follows the pool order, which for
 *          an ascending pool is the block order.
 *   out_idx   int32 [B][T][k]  the k_eff = min(k, #candidates) best blocks in
 *             ascending block order, then -1
 *   out_score int32 [B][T][k] or NULL: their scores (-1 in padding)
 * Score: s(b) = sum_h w[h] * max(0, sum_c q_idx[h][c] * keys[b][c]), exact in
 * int32 (Hi * Di <= 1024 keeps it below 2^31). Order: score descending, then
 * lower block index. Supports 1 <= Hi <= 16, Di in {32, 64, 128}, k >= 1,
 * B*T <= 65535 queries per call.
 * Workspace: csa_index_topk_workspace(...) bytes of device memory. Its head
 * holds per-query counters and histograms whose layout depends on B*T only:
 * zero-fill the workspace (csa_workspace_clear) after allocating it, again
 * whenever B*T changes, and after any failed call. A successful call leaves
 * that head zero again, so a decode loop with a fixed B*T reuses one
 * workspace without clearing, whatever n_max does. n_max is the largest
 * number of candidates a query can have: C when a pool is given, else
 * min(blk_cap, (pos0+T)/m). The size is about B*T*n_max*12 bytes (a score
 * and a candidate slot per entry), e.g. 3 GiB for an 8192-query chunk at
 * 32,768 visible blocks (a run that keeps no scores uses the score part only
 * for per-query thresholds and per-list counts).
 * ------------------------------------------------------------------------- */
int64_t csa_index_topk_workspace(int B, int T, int64_t n_max, int k, int cand_given);

int csa_index_topk(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                   int64_t blk_cap, int B, int T, int Hi, int Di, int m, int64_t pos0,
                   const int32_t* cand, int C, int k,
                   int32_t* out_idx, int32_t* out_score,
                   void* workspace, int64_t ws_bytes, hipStream_t stream);

/* csa_index_topk for a batch whose sequences sit at different positions:
 * the queries of sequence b are at pos[b] .. pos[b] + T - 1, with pos an
 * int64 [B] DEVICE array (8-byte aligned) read by the kernels, so a decode
 * loop can advance it on the device. pos_max bounds every pos[b] (values
 * outside [0, pos_max] are clamped into it); the launch plan and the
 * workspace (n_max = min(blk_cap, (pos_max + T) / m) without a pool) are
 * sized for it. Results per query are those of csa_index_topk at its own
 * position. */
int csa_index_topk_ragged(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                          int64_t blk_cap, int B, int T, int Hi, int Di, int m,
                          const int64_t* pos, int64_t pos_max,
                          const int32_t* cand, int C, int k,
                          int32_t* out_idx, int32_t* out_score,
                          void* workspace, int64_t ws_bytes, hipStream_t stream);
/* Its two launches, as csa_index_scan / csa_index_select below. */
int csa_index_scan_ragged(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                          int64_t blk_cap, int B, int T, int Hi, int Di, int m,
                          const int64_t* pos, int64_t pos_max,
                          const int32_t* cand, int C, int k,
                          int32_t* out_idx, int32_t* out_score,
                          void* workspace, int64_t ws_bytes, hipStream_t stream);
int csa_index_select_ragged(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                            int64_t blk_cap, int B, int T, int Hi, int Di, int m,
                            const int64_t* pos, int64_t pos_max,
                            const int32_t* cand, int C, int k,
                            int32_t* out_idx, int32_t* out_score,
                            void* workspace, int64_t ws_bytes, hipStream_t stream);

/* The two phases csa_index_topk runs, exposed so a caller can place events
 * or other work between them: csa_index_topk == csa_index_scan followed by
 * csa_index_select with identical arguments (the workspace carries state from
 * one to the other, so k and every other argument must match). Scan computes
 * every exact score (one key stream per query for T < 16 or a pool; for runs
 * of T >= 16 queries one key stream per group of 8-32 queries) and a
 * per-query score histogram, and keeps the scores in the workspace; select
 * turns them into the sorted index list. A run of T >= 16 queries over more
 * than 8,192 entries keeps no scores: its scan scores the keys twice (the
 * histograms, then each query's entries at or above its threshold bin as
 * candidate lists) and its select is the final selection alone. For at most
 * 8,192 candidates (a pool, or a short context), select is one workgroup per
 * query that reads the query's whole score row (one launch instead of two). */
int csa_index_scan(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                   int64_t blk_cap, int B, int T, int Hi, int Di, int m, int64_t pos0,
                   const int32_t* cand, int C, int k,
                   int32_t* out_idx, int32_t* out_score,
                   void* workspace, int64_t ws_bytes, hipStream_t stream);
int csa_index_select(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                     int64_t blk_cap, int B, int T, int Hi, int Di, int m, int64_t pos0,
                     const int32_t* cand, int C, int k,
                     int32_t* out_idx, int32_t* out_score,
                     void* workspace, int64_t ws_bytes, hipStream_t stream);

/* Full-mode top-k plus a blockwise candidate pool in one pass over the keys
 * (podcast cue 14: the best score of each block of positions decides which
 * blocks a later Reindex layer may choose from). Same arguments, layouts and
 * top-k result as csa_index_topk without a pool (cand = NULL), and:
 *   group     entries per group; must be 8 (CSA_ERR_SHAPE otherwise)
 *   n_keep    groups kept, >= 1
 *   out_pool  int32 [B][T][group * n_keep]  kept group i (ascending group
 *             order) fills slots i*group .. i*group + group - 1 with its
 *             entry ids, -1 for entries not visible yet; slots of groups
 *             beyond the number of visible groups are -1. Ascending, so it
 *             is a valid `cand` for csa_index_topk.
 * The causally visible entries are cut into groups of 8 consecutive entries
 * (the last may be partial); a group's score is the largest score of its
 * visible entries; groups are ordered by score descending, then lower group
 * index. Runs of queries use the one-query scan (no batched prefill scan).
 * Workspace: csa_index_topk_pool_workspace(B, T, n_max) bytes, with the same
 * head rules as csa_index_topk (the head layout depends on B*T only and is the
 * same for both calls, so one workspace serves both). */
int64_t csa_index_topk_pool_workspace(int B, int T, int64_t n_max);
int csa_index_topk_pool(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                        int64_t blk_cap, int B, int T, int Hi, int Di, int m, int64_t pos0,
                        int k, int32_t* out_idx, int32_t* out_score,
                        int group, int n_keep, int32_t* out_pool,
                        void* workspace, int64_t ws_bytes, hipStream_t stream);

/* The two launches of csa_index_topk_pool (scan: entry scores and group
 * maxima with their histograms; select: both selections), with identical
 * arguments, so a caller can place events or other work between them. */
int csa_index_pool_scan(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                        int64_t blk_cap, int B, int T, int Hi, int Di, int m, int64_t pos0,
                        int k, int32_t* out_idx, int32_t* out_score,
                        int group, int n_keep, int32_t* out_pool,
                        void* workspace, int64_t ws_bytes, hipStream_t stream);
int csa_index_pool_select(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                          int64_t blk_cap, int B, int T, int Hi, int Di, int m, int64_t pos0,
                          int k, int32_t* out_idx, int32_t* out_score,
                          int group, int n_keep, int32_t* out_pool,
                          void* workspace, int64_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * One CSA layer's index + attention step in a single call: csa_index_topk
 * (no candidate pool, or a Reindex pool `cand`) followed by csa_sparse_attn
 * over the selected entries plus the window, with the same results as those
 * two calls (podcast cues 12 and 14: a Full or Reindex layer selects its
 * top-k, then attends to it; "Frontier Architecture Decoding Notes (4)",
 * section 1: selected compressed blocks plus the newest 128 tokens under one
 * softmax). For decode (T < 16 queries per sequence, k + W <= 32768) the
 * top-k is resolved inside the attention kernel: every workgroup selects for
 * its own slots, so no separate final pass or id list round trip is needed.
 * Arguments are those of csa_index_topk and csa_sparse_attn:
 *   q_idx, w, keys, blk_cap, B, T, Hi, Di, m, cand, C, k, out_idx, out_score
 *     as in csa_index_topk (keys and the FP4 cache share blk_cap);
 *   q, codes, scales, win, Wcap, W, H, d, softmax_scale, out, out_dtype, lse,
 *     scale_fmt as in csa_sparse_attn;
 *   pos0: the queries' first position; or, with pos (int64 [B] DEVICE array,
 *     8-byte aligned, may be NULL), the bound of the per-sequence positions
 *     as in the *_ragged calls.
 * out_idx is always written (ascending, -1 padded). Workspace:
 * csa_index_attn_workspace(B, T, n_max, k, H, d, W) bytes, n_max as for
 * csa_index_topk_workspace, 256-byte aligned; its head (the first part, laid
 * out by B*T only) follows the csa_index_topk rules: zero before the first
 * call and after a B*T change or a failed call, left zero by every
 * successful call. Every argument is checked before the first launch. */
int64_t csa_index_attn_workspace(int B, int T, int64_t n_max, int k, int H, int d, int W);
int csa_index_attn(const int8_t* q_idx, const int8_t* w, const int8_t* keys, int64_t blk_cap,
                   int B, int T, int Hi, int Di, int m, int64_t pos0, const int64_t* pos,
                   const int32_t* cand, int C, int k,
                   const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                   const uint16_t* win, int Wcap, int W, int H, int d, float softmax_scale,
                   int32_t* out_idx, int32_t* out_score, void* out, int out_dtype, float* lse,
                   void* workspace, int64_t ws_bytes, int scale_fmt, hipStream_t stream);
/* The first launch of csa_index_attn alone, so a caller can time the key scan
 * by itself: identical arguments and checks, then only the indexer scan (the
 * exact scores and histograms, and for queries with more than 8192 candidates
 * and no pool the per-unit short lists the attention kernel selects from).
 * out_idx, out_score, out and lse are not written. The scan adds into the
 * workspace head, which only the rest of csa_index_attn returns to zero:
 * clear it (csa_workspace_clear) before the workspace serves another call. */
int csa_index_attn_scan(const int8_t* q_idx, const int8_t* w, const int8_t* keys,
                        int64_t blk_cap, int B, int T, int Hi, int Di, int m, int64_t pos0,
                        const int64_t* pos, const int32_t* cand, int C, int k,
                        const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                        const uint16_t* win, int Wcap, int W, int H, int d, float softmax_scale,
                        int32_t* out_idx, int32_t* out_score, void* out, int out_dtype,
                        float* lse, void* workspace, int64_t ws_bytes, int scale_fmt,
                        hipStream_t stream);

/* Zero-fill a workspace with a kernel on `stream` (no hipMemset, so it may be
 * captured in a graph). bytes must be a multiple of 4 and ws 4-byte aligned. */
int csa_workspace_clear(void* ws, int64_t bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Sparse attention with sliding window ("Frontier Architecture Decoding
 * Notes (4)", section 1; podcast cues 12 and 16). For the query at position
 * t = pos0 + i of sequence b, every one of the H heads attends, under ONE
 * softmax, to
 *   - the entries idx[b][i][0..k) (-1 or out-of-range slots are skipped;
 *     order is irrelevant; a Reuse layer passes an earlier layer's idx), each
 *     dequantised from MXFP4, and
 *   - the window tokens max(0, t-W+1) .. t, read from the bfloat16 ring
 *     win[b][p % Wcap].
 * Keys and values are both the latent row; logit = softmax_scale * <q_h, row>.
 *   q    bf16 [B][T][H][d]         16-byte aligned
 *   win  bf16 [B][Wcap][d]         16-byte aligned; Wcap >= W + T - 1
 *   out  [B][T][H][d] in out_dtype (CSA_BF16 or CSA_F32)
 *   lse  float32 [B][T][H] or NULL: natural-log log-sum-exp of the logits
 * Supports d in {128, 256, 512}, 1 <= H <= 64, 1 <= W <= Wcap, k >= 0,
 * pos0 + T <= 2^31 - 1 (else CSA_ERR_RANGE).
 * codes must be 16-byte aligned here (one entry's codes are read as 16-byte
 * words). Numerics: q, the dequantised entries and the window rows enter both
 * products as float16 (exact for values in float16's normal range: bfloat16
 * values of magnitude 2^-14 .. 65504, and entries while their scale byte lies
 * in [104, 140]; q values below 2^-14 keep float16's subnormal resolution of
 * 2^-24); q.k and p.v accumulate in float32, probabilities enter p.v as
 * two float16 terms (about 22 significant bits), taken against a running
 * max that lags the true one by at most a factor of 2^4, so they stay at
 * most 16; when the slots of a query are split over workgroups (few queries
 * per sequence), the partial outputs are kept in float32 and merged in a
 * fixed order. Rows outside float16's range are not attended silently: a query
 * any of whose staged rows is an E8M0 entry with a scale byte above 140 (a
 * 32-channel group with amax >= 2^16, whose largest codes overflow float16),
 * or a window value of magnitude 2^16 or more or not finite, gets NaN in
 * every head of its output and lse. Entries with scale bytes below 104 (every
 * value below 2^-21 in magnitude) are staged with float16's reduced subnormal
 * precision (absolute error below 2^-21 per element); a zero group (byte 0,
 * zero codes) is exact.
 * Workspace: csa_attn_workspace(...) bytes (no initialisation
 * needed); it may be NULL when that size is 0.
 * ------------------------------------------------------------------------- */
int64_t csa_attn_workspace(int B, int T, int H, int d, int64_t n_slots);

int csa_sparse_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                    int64_t blk_cap, const int32_t* idx, int k,
                    const uint16_t* win, int Wcap, int W,
                    int B, int T, int H, int d, int64_t pos0, float softmax_scale,
                    void* out, int out_dtype, float* lse,
                    void* workspace, int64_t ws_bytes, int scale_fmt, hipStream_t stream);

/* Heavily compressed (dense) attention: csa_sparse_attn with the entry set =
 * every visible block of an m-token cache, b with (b + 1) * m - 1 <= t
 * ("Frontier Architecture Decoding Notes (4)", section 1: HCA, up to 128
 * tokens per entry, attended densely). n_slots for the workspace query is
 * min(blk_cap, (pos0 + T) / m) + W. */
int hca_dense_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                   int64_t blk_cap, int m,
                   const uint16_t* win, int Wcap, int W,
                   int B, int T, int H, int d, int64_t pos0, float softmax_scale,
                   void* out, int out_dtype, float* lse,
                   void* workspace, int64_t ws_bytes, int scale_fmt, hipStream_t stream);

/* csa_sparse_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same call without a workspace argument. The split partials (the only
 * scratch csa_sparse_attn needs) live in a static device array of
 * CSA_NOALLOC_SCRATCH_MAX bytes inside the library, one per GPU the library
 * runs on, held until the process ends; its device address is looked up on
 * the first call on each device. The call allocates nothing and its results
 * are bit-identical to csa_sparse_attn's. A call whose launch plan needs more
 * scratch than the array holds returns CSA_ERR_SCRATCH before launching
 * (csa_attn_workspace(B, T, H, d, k + W) gives the need; it is 0 for runs of
 * 16 or more queries per sequence, and e.g. 18.9 MB for 8 decode queries
 * with k = 1024, d = 512, 64 heads). The scratch needs no initialisation.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (different streams, or different host threads without ordering)
 * race on it and give undefined results; order them (one stream) instead. */
int csa_sparse_attn_noalloc(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                            int64_t blk_cap, const int32_t* idx, int k,
                            const uint16_t* win, int Wcap, int W,
                            int B, int T, int H, int d, int64_t pos0, float softmax_scale,
                            void* out, int out_dtype, float* lse, int scale_fmt,
                            hipStream_t stream);

/* csa_sparse_attn and hca_dense_attn for sequences at different positions:
 * the queries of sequence b are at pos[b] .. pos[b] + T - 1 (pos: int64 [B]
 * DEVICE array, 8-byte aligned; values outside [0, pos_max] are clamped into
 * it). The split plan and the workspace are those of a batch at pos_max
 * (csa_attn_workspace with n_slots = k + W, or min(blk_cap, (pos_max + T) /
 * m) + W for the dense call). */
int csa_sparse_attn_ragged(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                           int64_t blk_cap, const int32_t* idx, int k,
                           const uint16_t* win, int Wcap, int W,
                           int B, int T, int H, int d, const int64_t* pos, int64_t pos_max,
                           float softmax_scale, void* out, int out_dtype, float* lse,
                           void* workspace, int64_t ws_bytes, int scale_fmt, hipStream_t stream);
int hca_dense_attn_ragged(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                          int64_t blk_cap, int m,
                          const uint16_t* win, int Wcap, int W,
                          int B, int T, int H, int d, const int64_t* pos, int64_t pos_max,
                          float softmax_scale, void* out, int out_dtype, float* lse,
                          void* workspace, int64_t ws_bytes, int scale_fmt, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
