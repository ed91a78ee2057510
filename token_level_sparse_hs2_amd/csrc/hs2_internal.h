// hs2_internal.h - internals shared by the host planner and the gfx950 kernels
// of the token-level sparse attention library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs2 {

// ---------------------------------------------------------------------------
// Fixed shapes and tuning constants
// ---------------------------------------------------------------------------
constexpr int kHeadDim = 128;   // d (the only supported head size)
constexpr int kKeyTile = 64;    // keys per LDS tile in the selection sweeps
constexpr int kSampleStride = 8;  // sample sweep visits key tiles 0, 8, 16, ...
constexpr int kBins = 256;        // histogram bins per row (8 per octave of S)
constexpr int kSelThreads = 256;  // threads of every selection workgroup
constexpr int kTopkBins = 2048;   // radix bins per pass of the top-K select (11 bits)
constexpr int kMinCandCap = 2048;  // candidate slots per row: max(2048, 2K) ...
constexpr int kMaxRankedK = 2048;  // ... held in registers by the top-K wave (<= 64 per lane);
                                   // a larger K is ranked by exact_kernel from the lists
constexpr int kMaxListK = 8192;    // largest K ranked from candidate lists (2K slots per row),
                                   // when some row is longer than 4K; otherwise, and above
                                   // it, every row takes the dense exact path
constexpr int64_t kCandBudgetBytes = 4LL << 30;  // candidate buffer cap per chunk
constexpr int64_t kDenseBudgetBytes = 16LL << 30;  // dense score rows (exact path) per chunk
constexpr int kFallbackBlocks = 1280;            // persistent grid of the exact path (5 per CU)
constexpr int kExactListCap = 1024;              // boundary-bin values the exact path ranks in LDS
constexpr int kBlockTokens = 64;                 // tokens per block in block selection (= kKeyTile)
// sampled threshold: rank r = ceil(kTauAlpha * K * n_sample / n_cand) + kTauBeta
constexpr float kTauAlpha = 1.2f;
constexpr int kTauBeta = 24;

// Scoring workgroups: 4 waves x 16 * score_row_tiles(G) MFMA rows (tokens x heads);
// tokens per selection task (one workgroup): 64, 64, 64, 32, 16 for G = 1..16.
__host__ __device__ constexpr int score_row_tiles(int G) { return G >= 4 ? 4 : G; }
__host__ __device__ constexpr int tokens_per_task(int G) { return 4 * 16 * score_row_tiles(G) / G; }

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Position-decaying budget (Stem page, Token Position-Decay paragraph): query
// position t of a sequence of L tokens keeps K - floor((K - k_end) t / (L - 1))
// candidates, K at the first position down to k_end at the last (k_end == K: none).
__host__ __device__ inline int row_budget(int K, int k_end, int t, int L) {
  if (L <= 1 || k_end == K) return K;
  return K - (int)(((int64_t)(K - k_end) * t) / (L - 1));
}

// ---------------------------------------------------------------------------
// Varlen task order (host and device): tasks are (sequence, tile of `tok`
// tokens). Tiles further into a sequence cost more (more causal keys), so the
// order is tile index descending, then sequence ascending: a greedy
// longest-first assignment when the hardware dispatches workgroups in order.
// P(q) = number of tasks with tile index > q = sum_i max(0, n_i - q - 1).
// ---------------------------------------------------------------------------
__host__ __device__ inline int64_t plan_tasks_above(const int32_t* cu, int B, int tok, int q) {
  int64_t s = 0;
  for (int i = 0; i < B; i++) {
    int n = ceil_div(cu[i + 1] - cu[i], tok);
    if (n - q - 1 > 0) s += n - q - 1;
  }
  return s;
}

__host__ __device__ inline void plan_decode(const int32_t* cu, int B, int tok, int max_tiles,
                                            int64_t task, int* seq, int* tile) {
  int lo = 0, hi = max_tiles - 1;  // smallest q with P(q) <= task
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (plan_tasks_above(cu, B, tok, mid) <= task) hi = mid; else lo = mid + 1;
  }
  int q = lo;
  int64_t r = task - plan_tasks_above(cu, B, tok, q);
  int s = 0;
  for (int i = 0; i < B; i++) {
    int n = ceil_div(cu[i + 1] - cu[i], tok);
    if (n > q) {
      if (r == 0) { s = i; break; }
      r--;
    }
  }
  *seq = s;
  *tile = q;
}

// ---------------------------------------------------------------------------
// Kernel parameter blocks
// ---------------------------------------------------------------------------
struct ScoreParams {
  const uint16_t* q;    // [T, Hq, 128] bf16
  const uint16_t* k;    // [T, Hkv, 128] bf16
  const int32_t* cu;    // [B+1]
  int B, Hq, Hkv, K, W;
  int k_end;            // budget at a sequence's last position (K: no decay)
  int max_tiles;        // tiles of the longest sequence
  int64_t task_begin;   // first task of this chunk
  float c;              // softmax_scale * log2(e)
  int bin_base;         // (bits(G/max(1, k_end)) >> 20) - (kBins - 1)
  const uint32_t* kmax; // [B * Hkv] largest key norm of each (sequence, group), float bits
  int cand_cap;         // C
  uint32_t flags;
  int list_rank;        // K > kMaxRankedK: rows within [K, C] candidates go to exact_kernel too
  int block;            // 0, or kBlockTokens: block selection (candidates are block scores)
  const float* vw;      // [T, Hkv] log2 key weights beta * max(0, log2 |v|), or null (plain score)
  const uint32_t* vwmax;  // [B * Hkv] largest weight of each (sequence, group), float bits
  float* lse2;          // [T, Hq] log2-domain log-sum-exp of each full-layer row
  int lse_given;        // 1: lse2 holds the rows' statistics already (no statistics sweep)
  uint64_t* cand;       // [chunk rows, C]: (S bits << 32) | position
  int32_t* cand_count;  // [chunk rows]: count, or -1 = exact path
  int32_t* flag_list;   // [chunk rows]: slots sent to the exact path
  int32_t* flag_count;  // [1]
  int2* task_map;       // [chunk tasks]: (sequence, tile) of each task, read by the top-K kernel
  float* dense_out;     // exact-path rows: [chunk rows, dense_ld] S of every candidate, or null
  int64_t dense_ld;
};

struct TopkParams {
  int64_t n_rows;       // rows of this chunk
  const int32_t* cu;
  int B, Hq, Hkv, K, W;
  int k_end;            // budget at a sequence's last position (K: no decay)
  int max_tiles;
  int64_t task_begin;
  int tok;              // tokens per task (a power of two)
  int tok_shift;        // log2(tok)
  const int2* task_map; // [chunk tasks]: (sequence, tile), written by the scores kernel
  const float* dense_rows;  // [chunk rows, dense_ld] S of every candidate (scores kernel), or
  int64_t dense_ld;         // null: the exact path then recomputes the scores
  int block;            // 0, or kBlockTokens: candidates are (block score, block index)
  int list_rank;        // rows with a candidate count >= 0 are ranked by exact_kernel
  int cand_cap;
  int bitmap_words;     // words per bitmap in LDS (covers max_seqlen)
  int sbuf_words;       // per-wave LDS staging of the selected positions (min(K, kMaxRankedK))
  float c;
  const uint64_t* cand;
  const int32_t* cand_count;
  const int32_t* flag_list;
  const int32_t* flag_count;
  // exact path
  const uint16_t* q;
  const uint16_t* k;
  const float* lse2;
  uint32_t* dense;      // [kFallbackBlocks, max_seqlen] S bits
  int max_seqlen;
  const float* vw;      // [T, Hkv] log2 key weights, or null
  // outputs
  int32_t* idx;         // [T, Hkv, K+W]
  float* kth;           // [T, Hkv] or null
};

struct SparseParams {
  const uint16_t* q;    // [T, Hq, 128] (decode: [B, Hq, 128])
  const uint16_t* k;    // [T, Hkv, 128]
  const uint16_t* v;
  const int32_t* idx;   // [T, Hkv, KW] (decode: [B, Hkv, KW])
  const int32_t* cu;
  int B, Hq, Hkv, KW;
  int64_t T;            // query rows: tokens, or sequences when decoding
  float c;              // softmax_scale * log2(e)
  void* out;            // [T, Hq, 128] bf16 or f32
  int decode;           // query row r is sequence r at its last position
  // FP8 KV cache (E4M3 codes, per-tensor scales): k8 / v8 [T, Hkv, 128] replace
  // k / v; the key scale is folded into c, the value scale multiplies the output
  const uint8_t* k8;
  const uint8_t* v8;
  float v_scale;
  // split rows (decode): n_part waves share a row's index entries, each writing
  // an unnormalised partial that sparse_combine merges
  int n_part;           // 1 = one wave per row, output written directly
  float* part_o;        // [T * n_part * Hkv, G, 128] partial P.V (fp32)
  float2* part_ml;      // [T * n_part * Hkv, G] (reference, sum) of each partial
  // shared-gather plan (prefill): one wave per (token group, g) walks the union of
  // the group's index rows (see SparsePlan); plist null = one wave per (token, g)
  const uint32_t* plist;  // [n_grp * Hkv, pcap] row - base0 | token mask << 24
  const int32_t* pcount;  // [n_grp * Hkv] entries of each union
  int pcap;
  int64_t n_grp;
};

// Shared-gather plan. Consecutive query tokens select largely the same rows (the
// forced window, and keys that score high for all of them), so the NT = 16 / G
// (at most 8) tokens t0 .. t0 + NT - 1 of the packed batch are served by one wave:
// the sorted union of their index rows is gathered once, and the S^T tiles take
// the NT * G (token, head) columns. An entry is one word: the row relative to the
// sequence base of token t0 (below max_seqlen + 16 < 2^24) in bits 0-23 and the
// mask of the tokens whose row holds it in bits 24-31.
__host__ __device__ constexpr int plan_tokens(int G) { return G >= 2 ? 16 / G : 8; }
constexpr uint32_t kPlanRowMask = 0xFFFFFFu;
constexpr int kPlanChunk = 8192;  // row positions per bitmap pass of the plan kernel

struct PlanParams {
  const int32_t* idx;   // [T, Hkv, KW] rows as written by the selection
  const int32_t* cu;
  int B, Hkv, KW;
  int64_t T;
  int64_t n_grp;        // ceil(T / NT)
  int cap;              // NT * KW entries per union
  uint32_t* list;       // [n_grp * Hkv, cap]
  int32_t* count;       // [n_grp * Hkv]
};

// Decode step: one query per sequence at its last cached position.
// cached key bytes per logits workgroup: 256 bf16 or 512 FP8 rows of 128 elements
constexpr int kDecodeSplitBytes = 65536;
__host__ __device__ constexpr int decode_split_len(bool fp8) {
  return kDecodeSplitBytes / (kHeadDim * (fp8 ? 1 : 2));
}
constexpr int kDecodeCandCap = 4096;  // candidates ranked in LDS per decode row

struct DecodeParams {
  const uint16_t* q;    // [B, Hq, 128]
  const uint16_t* k;    // [T, Hkv, 128] cache
  const uint8_t* k8;    // or an FP8 key cache (E4M3 codes; the scale is folded into c)
  const int32_t* cu;    // [B+1] cache offsets
  int B, Hq, Hkv, K, W;
  int max_seqlen;
  int split_len;        // cached keys per logits workgroup, decode_split_len
  int n_split;          // ceil(max_seqlen / split_len)
  int bitmap_words;     // ceil(max_seqlen / 32)
  float c;              // softmax_scale * log2(e)
  int64_t T;            // cached tokens
  float* z2;            // [Hkv, T, G]: c * q.k of every cached key and the group's heads
  float2* part;         // [B, Hkv, n_split, G]: per split (max, sum of exp2(z2 - max))
  uint32_t* dense;      // [B * Hkv, max_seqlen] S bits
  float* lse2;          // [B * Hkv, G] log-sum-exp (log2 domain) of each head over the cache
  uint32_t* tau;        // [B * Hkv] sampled threshold (S bits)
  int32_t* n_pass;      // [B * Hkv] scores reaching tau
  uint32_t* cand;       // [B * Hkv, 2, kDecodeCandCap] S bits, then positions, of those scores
  int32_t* idx;         // [B, Hkv, K+W]
  float* kth;           // [B, Hkv] or null
};

// The full layer's output sweep: 4 waves x 32 MFMA rows per workgroup.
__host__ __device__ constexpr int full_out_tokens(int G) { return 4 * 32 / G; }

struct FullOutParams {
  const uint16_t* q;    // [T, Hq, 128] the full layer's queries
  const uint16_t* k;    // [T, Hkv, 128]
  const uint16_t* v;
  const int32_t* cu;
  int B, Hq, Hkv;
  int max_tiles;        // tiles of full_out_tokens(G) tokens in the longest sequence
  float c;              // softmax_scale * log2(e)
  float* lse2;          // [T, Hq] out: log2-domain log-sum-exp of every row (nullable)
  void* out;            // [T, Hq, 128] bf16 or f32
};

// launchers (defined in the .hip files)
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
hipError_t launch_key_norms(const uint16_t* k, const int32_t* cu, int B, int Hkv, int64_t T,
                            uint32_t* kmax, hipStream_t s);
hipError_t launch_value_weights(const uint16_t* v, const int32_t* cu, int B, int Hkv, int64_t T,
                                float beta, float* vw, uint32_t* vwmax, hipStream_t s);
hipError_t launch_scores(int G, const ScoreParams& p, int n_blocks, hipStream_t s);
hipError_t launch_topk(int G, const TopkParams& p, int n_tasks, int rows_per_block, hipStream_t s);
hipError_t launch_fallback(int G, const TopkParams& p, size_t lds_bytes, hipStream_t s);
hipError_t launch_sparse(int G, bool precise, bool fp8, const SparseParams& p, hipStream_t s);
// Device address of the no-allocation entry point's scratch array on the current
// device (looked up once per device and kept).
constexpr size_t kNoAllocScratchBytes = (size_t)20 << 20;
hipError_t noalloc_scratch(void** out);
hipError_t launch_sparse_plan(int G, const PlanParams& p, hipStream_t s);
// dst[i] = E4M3(float(src[i]) * inv_scale), round to nearest even, saturating at +-448
hipError_t launch_quantize_fp8(const uint16_t* src, uint8_t* dst, int64_t n, float inv_scale,
                               hipStream_t s);
hipError_t launch_decode_logits(int G, const DecodeParams& p, hipStream_t s);
hipError_t launch_full_out(int G, bool precise, const FullOutParams& p, int64_t n_tasks,
                           hipStream_t s);
hipError_t launch_decode_select(int G, const DecodeParams& p, size_t lds_bytes, hipStream_t s);

}  // namespace hs2
