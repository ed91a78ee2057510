// hs2_api.cpp - the C ABI (include/hs2.h): validation, workspace layout,
// chunking of the selection work, and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hs2.h"
#include "hs2_internal.h"

namespace {

thread_local char g_hip_msg[256] = "no HIP error recorded";

int hip_fail(hipError_t e, const char* what) {
  std::snprintf(g_hip_msg, sizeof(g_hip_msg), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return HS2_ERR_HIP;
}

constexpr size_t kAlign = 256;
constexpr int kPlanShortRows = 32768;  // hs2_prefill_block plans one layer up to this length
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Geometry {
  int G = 0, tok = 0;
  int64_t T = 0;
  int B = 0;
  int max_len = 0;      // longest sequence
  int max_tiles = 0;    // tiles of the longest sequence
  int64_t n_tasks = 0;  // (sequence, tile) pairs
  int cand_cap = 0;
  int64_t tasks_per_chunk = 0;
  int64_t rows_per_chunk = 0;
  int bitmap_words = 0;
  // workspace offsets
  size_t off_lse = 0, off_cand = 0, off_count = 0, off_flags = 0, off_nflag = 0, off_dense = 0,
         off_kmax = 0, off_vw = 0, off_vwmax = 0, off_tmap = 0;
  size_t select_bytes = 0;
  size_t exact_lds = 0;
  int topk_rows_per_block = 4;
  int sbuf_words = 0;
  bool exact_only = false;  // K above the list-ranked limit: every row takes the exact path
  bool list_rank = false;   // K above the register-ranked limit: candidate lists ranked by
                            // exact_kernel instead of the top-K waves
  bool dense = false;       // every ranked row takes the exact path: dense score rows
  int block = 0;            // block selection: tokens per block
  // shared-gather plan of the sparse layers (usable when plan_ok)
  bool plan_ok = false;
  int64_t n_grp = 0;        // token groups of plan_tokens(G)
  int plan_cap = 0;         // union entries per (group, KV group)
  size_t off_pcount = 0, plan_bytes = 0;
  int Hq = 0, Hkv = 0;
};

// Selection workspace for `tpc` tasks per chunk: only the candidate rows, their
// counts and the exact-path row list scale with the chunk.
void layout_select(Geometry* geo, int64_t tpc) {
  geo->tasks_per_chunk = tpc;
  geo->rows_per_chunk = tpc * geo->Hkv * geo->tok;
  size_t off = 0;
  geo->off_lse = off;
  off = align_up(off + (size_t)geo->T * geo->Hq * sizeof(float));
  geo->off_cand = off;
  off = align_up(off + (size_t)geo->rows_per_chunk * geo->cand_cap * sizeof(uint64_t));
  geo->off_count = off;
  off = align_up(off + (size_t)geo->rows_per_chunk * sizeof(int32_t));
  geo->off_flags = off;
  off = align_up(off + (size_t)geo->rows_per_chunk * sizeof(int32_t));
  geo->off_tmap = off;  // (sequence, tile) of each task of the chunk
  off = align_up(off + (size_t)tpc * 2 * sizeof(int32_t));
  geo->off_nflag = off;
  off = align_up(off + sizeof(int32_t));
  geo->off_dense = off;
  off = align_up(off + (size_t)hs2::kFallbackBlocks * std::max(1, geo->max_len) * sizeof(uint32_t));
  geo->off_kmax = off;
  off = align_up(off + (size_t)geo->B * geo->Hkv * sizeof(uint32_t));
  geo->off_vw = off;  // output-aware metric: key weights and their maxima
  off = align_up(off + (size_t)geo->T * geo->Hkv * sizeof(float));
  geo->off_vwmax = off;
  off = align_up(off + (size_t)geo->B * geo->Hkv * sizeof(uint32_t));
  geo->select_bytes = off;
}

bool g_supported(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

int validate(const hs2_dims* d, const hs2_varlen* v, Geometry* geo) {
  if (!d || !v) return HS2_ERR_INVALID_ARG;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads)
    return HS2_ERR_INVALID_ARG;
  if (d->top_k < 0 || d->window < 0 || (int64_t)d->top_k + d->window < 1 ||
      (int64_t)d->top_k + d->window > (1 << 24))
    return HS2_ERR_INVALID_ARG;
  if (!(std::isfinite(d->softmax_scale) && d->softmax_scale > 0.f)) return HS2_ERR_INVALID_ARG;
  if (d->flags & ~(uint32_t)(HS2_FLAG_EXACT_SELECT | HS2_FLAG_BLOCK_SELECT)) return HS2_ERR_INVALID_ARG;
  if ((d->flags & HS2_FLAG_BLOCK_SELECT) && d->top_k % hs2::kBlockTokens) return HS2_ERR_INVALID_ARG;
  if (v->batch < 0) return HS2_ERR_INVALID_ARG;
  if (d->head_dim != hs2::kHeadDim) return HS2_ERR_UNSUPPORTED;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (!g_supported(G)) return HS2_ERR_UNSUPPORTED;
  geo->G = G;
  geo->tok = hs2::tokens_per_task(G);
  geo->B = v->batch;
  if (v->batch == 0) {
    if (v->total_tokens != 0) return HS2_ERR_INVALID_ARG;
    geo->T = 0;
    return HS2_OK;
  }
  if (!v->cu_seqlens || !v->cu_seqlens_host) return HS2_ERR_INVALID_ARG;
  const int32_t* cu = v->cu_seqlens_host;
  if (cu[0] != 0) return HS2_ERR_INVALID_ARG;
  int max_len = 0;
  int64_t n_tasks = 0;
  for (int i = 0; i < v->batch; i++) {
    if (cu[i + 1] < cu[i]) return HS2_ERR_INVALID_ARG;
    const int L = cu[i + 1] - cu[i];
    max_len = std::max(max_len, L);
    n_tasks += hs2::ceil_div(L, geo->tok);
  }
  if ((int64_t)cu[v->batch] != v->total_tokens) return HS2_ERR_INVALID_ARG;
  if (v->max_seqlen < max_len || v->max_seqlen > HS2_MAX_SEQLEN) return HS2_ERR_INVALID_ARG;
  // kernels address K/V rows within one sequence with 32-bit byte offsets
  if ((int64_t)max_len * d->num_kv_heads * hs2::kHeadDim * 2 >= (1LL << 32)) return HS2_ERR_UNSUPPORTED;
  geo->T = v->total_tokens;
  geo->max_len = max_len;
  geo->max_tiles = std::max(1, hs2::ceil_div(max_len, geo->tok));
  geo->n_tasks = n_tasks;

  // candidate rows: C slots each; chunks of whole tasks under the byte budget
  const int K = d->top_k;
  geo->block = (d->flags & HS2_FLAG_BLOCK_SELECT) ? hs2::kBlockTokens : 0;
  int64_t cap = std::max<int64_t>(hs2::kMinCandCap, 2LL * K);
  // K above the register-ranked limit: the rows are ranked from their candidate lists
  // (up to 2K each) when the longest row exceeds two lists; with shorter rows a list is
  // most of its row at twice the bytes per entry, and the dense rows measured faster
  // (8k tokens, K = 3000: 1.73 against 1.98 ms)
  const bool big = !geo->block && K > hs2::kMaxRankedK;
  geo->exact_only = big && (K > hs2::kMaxListK || (int64_t)max_len <= 2 * cap);
  geo->dense = !geo->block && (geo->exact_only || (d->flags & HS2_FLAG_EXACT_SELECT));
  geo->list_rank = big && !geo->dense;
  if (geo->block)  // one entry per candidate block of the longest row (<= 4096, ranked in registers)
    cap = std::max<int64_t>(64, hs2::ceil_div(std::max(1, max_len), hs2::kBlockTokens));
  if (geo->dense)  // the candidate rows hold one fp32 score per position (two per 8-byte slot)
    cap = std::max<int64_t>(64, hs2::ceil_div(std::max(1, max_len), 2));
  cap = (cap + 63) / 64 * 64;
  geo->cand_cap = (int)cap;
  const int64_t rows_per_task = (int64_t)d->num_kv_heads * geo->tok;
  const int64_t row_bytes = cap * 8;
  const int64_t budget = geo->dense ? hs2::kDenseBudgetBytes : hs2::kCandBudgetBytes;
  int64_t tpc = budget / (rows_per_task * row_bytes);
  tpc = std::max<int64_t>(1, std::min<int64_t>(tpc, std::max<int64_t>(1, n_tasks)));
  geo->bitmap_words = hs2::ceil_div(std::max(1, max_len), 32);
  geo->Hq = d->num_q_heads;
  geo->Hkv = d->num_kv_heads;
  layout_select(geo, tpc);
  // exact path: histogram, scratch words, two bitmaps, then G query rows in fp32 or
  // (after them) the boundary-bin list of keys and positions
  geo->exact_lds = (hs2::kTopkBins + 16 + 2 * (size_t)geo->bitmap_words +
                    std::max<size_t>(16 * hs2::kHeadDim, 2 * (size_t)hs2::kExactListCap)) *
                   sizeof(uint32_t);
  // top-K waves: a 256-bin histogram and one bitmap each; up to 4 waves per block
  // a 256-bin histogram, a bitmap and the staging of the selected positions
  geo->sbuf_words = std::min(d->top_k, hs2::kMaxRankedK);
  const size_t per_wave =
      (256 + (size_t)geo->bitmap_words + (size_t)geo->sbuf_words) * sizeof(uint32_t);
  // 1, 2 or 4 waves (rows) per block: a block's rows are consecutive tokens of one task
  const size_t rpb = std::max<size_t>(1, std::min<size_t>(4, 40960 / per_wave));
  geo->topk_rows_per_block = rpb >= 4 ? 4 : (rpb >= 2 ? 2 : 1);
  // shared-gather plan: union rows are relative to a group's first sequence and lie
  // below its last token, so they stay under max_len + 16 (32-bit byte offsets)
  const int nt = hs2::plan_tokens(geo->G);
  const int64_t kw = (int64_t)d->top_k + d->window;
  geo->n_grp = (geo->T + nt - 1) / nt;
  geo->plan_cap = (int)std::min<int64_t>(kw * nt, INT32_MAX);
  geo->plan_ok = kw * nt <= INT32_MAX &&
                 ((int64_t)max_len + 16) * d->num_kv_heads * hs2::kHeadDim * 2 < (1LL << 32);
  if (geo->plan_ok) {
    const size_t lists = (size_t)geo->n_grp * d->num_kv_heads;
    geo->off_pcount = align_up(lists * (size_t)geo->plan_cap * sizeof(uint32_t));
    geo->plan_bytes = align_up(geo->off_pcount + lists * sizeof(int32_t));
  }
  return HS2_OK;
}

// Decode step: the varlen struct describes the cache; every sequence holds >= 1 token.
struct DecodeGeometry {
  Geometry geo;
  int n_split = 0, bitmap_words = 0;
  size_t off_z2 = 0, off_part = 0, off_dense = 0, off_lse = 0, off_tau = 0, off_npass = 0,
         off_cand = 0, bytes = 0, lds = 0;
  // sparse layer: n_part waves per (sequence, group) row and their partials
  int n_part = 1;
  size_t off_po = 0, off_pml = 0, sparse_bytes = 0;
};

int validate_decode(const hs2_dims* d, const hs2_varlen* v, DecodeGeometry* dg) {
  int st = validate(d, v, &dg->geo);
  if (st != HS2_OK) return st;
  if (d->flags & HS2_FLAG_BLOCK_SELECT) return HS2_ERR_UNSUPPORTED;  // decode selects tokens
  const Geometry& g = dg->geo;
  if (g.B == 0) return HS2_OK;
  for (int i = 0; i < v->batch; i++)
    if (v->cu_seqlens_host[i + 1] - v->cu_seqlens_host[i] < 1) return HS2_ERR_INVALID_ARG;
  if (v->batch > 65535 || d->num_kv_heads > 65535) return HS2_ERR_UNSUPPORTED;  // grid y/z
  const int max_len = std::max(1, g.max_len);
  // the bf16 cache's (shorter) split sizes the partials for both caches
  dg->n_split = hs2::ceil_div(max_len, hs2::decode_split_len(false));
  dg->bitmap_words = hs2::ceil_div(max_len, 32);
  size_t off = 0;
  dg->off_z2 = off;
  off = align_up(off + (size_t)g.T * d->num_q_heads * sizeof(float));
  dg->off_part = off;
  off = align_up(off + (size_t)v->batch * d->num_kv_heads * dg->n_split * g.G * 2 * sizeof(float));
  dg->off_dense = off;
  off = align_up(off + (size_t)v->batch * d->num_kv_heads * max_len * sizeof(uint32_t));
  const size_t rows_kv = (size_t)v->batch * d->num_kv_heads;
  dg->off_lse = off;
  off = align_up(off + (size_t)v->batch * d->num_q_heads * sizeof(float));
  dg->off_tau = off;
  off = align_up(off + rows_kv * sizeof(uint32_t));
  dg->off_npass = off;
  off = align_up(off + rows_kv * sizeof(int32_t));
  dg->off_cand = off;
  off = align_up(off + rows_kv * 2 * hs2::kDecodeCandCap * sizeof(uint32_t));
  dg->bytes = off;
  // histogram, scratch words, two bitmaps of the row's candidates, compacted candidates
  dg->lds = (hs2::kTopkBins + 16 + 2 * (size_t)dg->bitmap_words + 2 * (size_t)hs2::kDecodeCandCap) *
            sizeof(uint32_t);
  // sparse layer: spread the B * Hkv rows over about 1024 waves, >= 4 index steps each
  const int64_t rows = (int64_t)v->batch * d->num_kv_heads;
  const int n_steps = hs2::ceil_div(d->top_k + d->window, 32);
  const int64_t want = (1024 + rows - 1) / rows;
  dg->n_part = (int)std::max<int64_t>(
      1, std::min<int64_t>({want, (int64_t)hs2::ceil_div(n_steps, 4), (int64_t)32}));  // <= kMaxParts
  if (dg->n_part > 1) {
    const size_t slots = (size_t)rows * dg->n_part;
    size_t o2 = 0;
    dg->off_po = o2;
    o2 = align_up(o2 + slots * g.G * hs2::kHeadDim * sizeof(float));
    dg->off_pml = o2;
    o2 = align_up(o2 + slots * g.G * 2 * sizeof(float));
    dg->sparse_bytes = o2;
  }
  return HS2_OK;
}

// Smallest selection workspace: one task per chunk.
size_t min_select_bytes(const Geometry& geo) {
  Geometry g1 = geo;
  layout_select(&g1, 1);
  return g1.select_bytes;
}

// The selection runs in chunks of whole tasks whose candidate rows fit the given
// workspace: the full size of hs2_workspace_size(HS2_OP_SELECT), or fewer tasks
// per chunk in a smaller workspace down to min_select_bytes.
int fit_workspace(Geometry* geo, void* ws, size_t bytes) {
  if (geo->select_bytes == 0) return HS2_OK;
  if (!ws) return HS2_ERR_WORKSPACE;
  if (bytes >= geo->select_bytes) return HS2_OK;
  const size_t min_bytes = min_select_bytes(*geo);
  if (bytes < min_bytes) return HS2_ERR_WORKSPACE;
  const size_t per_task = (size_t)geo->Hkv * geo->tok * ((size_t)geo->cand_cap * 8 + 8) + 8;
  int64_t tpc = std::min<int64_t>(geo->tasks_per_chunk, 1 + (int64_t)((bytes - min_bytes) / per_task));
  layout_select(geo, tpc);
  while (tpc > 1 && geo->select_bytes > bytes) layout_select(geo, --tpc);
  return geo->select_bytes <= bytes ? HS2_OK : HS2_ERR_WORKSPACE;
}

// hs2_prefill_block runs its layers from one shared-gather plan when the plan pays
// for itself: two or more layers, or one layer over rows up to kPlanShortRows
// tokens (the plan's cost grows with row positions; a single layer over longer
// rows does not recover it).
bool plan_pays(const Geometry& geo, int n_sparse) {
  return geo.plan_ok && (n_sparse >= 2 || (n_sparse == 1 && geo.max_len <= kPlanShortRows));
}

float scale_log2(const hs2_dims* d) { return d->softmax_scale * 1.4426950408889634f; }

int run_select(const hs2_dims* d, const hs2_varlen* v, const Geometry& geo, const void* q,
               const void* k, int32_t* idx_out, float* kth_out, void* ws, hipStream_t s,
               const void* vv = nullptr, float oam_beta = 0.f, int k_end = -1,
               bool lse_given = false) {
  if (geo.T == 0) return HS2_OK;
  if (k_end < 0) k_end = d->top_k;  // no decay
  char* w = static_cast<char*>(ws);
  float* lse2 = reinterpret_cast<float*>(w + geo.off_lse);
  uint64_t* cand = reinterpret_cast<uint64_t*>(w + geo.off_cand);
  int32_t* count = reinterpret_cast<int32_t*>(w + geo.off_count);
  int32_t* flags = reinterpret_cast<int32_t*>(w + geo.off_flags);
  int32_t* nflag = reinterpret_cast<int32_t*>(w + geo.off_nflag);
  uint32_t* dense = reinterpret_cast<uint32_t*>(w + geo.off_dense);
  uint32_t* kmax = reinterpret_cast<uint32_t*>(w + geo.off_kmax);
  int2* tmap = reinterpret_cast<int2*>(w + geo.off_tmap);

  const int G = geo.G;
  const float gk = (float)G / (float)std::max(1, k_end);
  uint32_t gk_bits;
  std::memcpy(&gk_bits, &gk, 4);

  hs2::ScoreParams sp{};
  sp.q = static_cast<const uint16_t*>(q);
  sp.k = static_cast<const uint16_t*>(k);
  sp.cu = v->cu_seqlens;
  sp.B = v->batch;
  sp.Hq = d->num_q_heads;
  sp.Hkv = d->num_kv_heads;
  sp.K = d->top_k;
  sp.W = d->window;
  sp.k_end = k_end;
  sp.max_tiles = geo.max_tiles;
  sp.c = scale_log2(d);
  sp.bin_base = (int)(gk_bits >> 20) - (hs2::kBins - 1);
  sp.cand_cap = geo.cand_cap;
  sp.flags = d->flags | (geo.exact_only ? (uint32_t)HS2_FLAG_EXACT_SELECT : 0u);
  sp.block = geo.block;
  sp.list_rank = geo.list_rank ? 1 : 0;
  sp.lse2 = lse2;
  sp.lse_given = lse_given ? 1 : 0;
  sp.cand = cand;
  sp.cand_count = count;
  sp.flag_list = flags;
  sp.flag_count = nflag;
  sp.kmax = kmax;
  sp.task_map = tmap;
  sp.dense_out = geo.dense ? reinterpret_cast<float*>(cand) : nullptr;
  sp.dense_ld = 2 * (int64_t)geo.cand_cap;

  hs2::TopkParams tp{};
  tp.cu = v->cu_seqlens;
  tp.B = v->batch;
  tp.Hq = d->num_q_heads;
  tp.Hkv = d->num_kv_heads;
  tp.K = d->top_k;
  tp.W = d->window;
  tp.k_end = k_end;
  tp.max_tiles = geo.max_tiles;
  tp.tok = geo.tok;
  tp.tok_shift = __builtin_ctz((unsigned)geo.tok);
  tp.task_map = tmap;
  tp.dense_rows = sp.dense_out;
  tp.dense_ld = sp.dense_ld;
  tp.block = geo.block;
  tp.list_rank = geo.list_rank ? 1 : 0;
  tp.cand_cap = geo.cand_cap;
  tp.bitmap_words = geo.bitmap_words;
  tp.sbuf_words = geo.sbuf_words;
  tp.c = sp.c;
  tp.cand = cand;
  tp.cand_count = count;
  tp.flag_list = flags;
  tp.flag_count = nflag;
  tp.q = sp.q;
  tp.k = sp.k;
  tp.lse2 = lse2;
  tp.dense = dense;
  tp.max_seqlen = std::max(1, geo.max_len);
  tp.idx = idx_out;
  tp.kth = kth_out;

  hipError_t ek = hipSuccess;
  if (!lse_given) {  // the statistics sweep's reference needs the key norms
    ek = hs2::launch_key_norms(sp.k, v->cu_seqlens, v->batch, d->num_kv_heads, geo.T, kmax, s);
    if (ek != hipSuccess) return hip_fail(ek, "key norm kernel");
  }
  if (oam_beta > 0.f) {
    float* vw = reinterpret_cast<float*>(w + geo.off_vw);
    uint32_t* vwmax = reinterpret_cast<uint32_t*>(w + geo.off_vwmax);
    ek = hs2::launch_value_weights(static_cast<const uint16_t*>(vv), v->cu_seqlens, v->batch,
                                   d->num_kv_heads, geo.T, oam_beta, vw, vwmax, s);
    if (ek != hipSuccess) return hip_fail(ek, "value weight kernel");
    sp.vw = vw;
    sp.vwmax = vwmax;
    tp.vw = vw;
  }
  for (int64_t t0 = 0; t0 < geo.n_tasks; t0 += geo.tasks_per_chunk) {
    const int64_t nt = std::min(geo.tasks_per_chunk, geo.n_tasks - t0);
    const int64_t blocks = nt * d->num_kv_heads;
    const int64_t rows = blocks * geo.tok;
    if (blocks > 0x7FFFFFFF || rows > 0x7FFFFFFF) return HS2_ERR_UNSUPPORTED;
    sp.task_begin = t0;
    tp.task_begin = t0;
    tp.n_rows = rows;
    hipError_t e = hs2::launch_zero_i32(nflag, 1, s);
    if (e != hipSuccess) return hip_fail(e, "zero flag counter");
    e = hs2::launch_scores(G, sp, (int)blocks, s);
    if (e != hipSuccess) return hip_fail(e, "scores kernel");
    e = hs2::launch_topk(G, tp, (int)nt, geo.topk_rows_per_block, s);
    if (e != hipSuccess) return hip_fail(e, "top-k kernel");
    e = hs2::launch_fallback(G, tp, geo.exact_lds, s);
    if (e != hipSuccess) return hip_fail(e, "exact-select kernel");
  }
  return HS2_OK;
}

// The full layer's own output over all causal keys (one sweep with a running
// row maximum); lse2 (nullable) receives every row's log2-domain log-sum-exp.
int run_full_out(const hs2_dims* d, const hs2_varlen* v, const Geometry& geo, const void* q,
                 const void* k, const void* vv, void* out, int out_dtype, float* lse2,
                 hipStream_t s) {
  const int tok = hs2::full_out_tokens(geo.G);
  int64_t n_tasks = 0;
  for (int i = 0; i < v->batch; i++)
    n_tasks += hs2::ceil_div(v->cu_seqlens_host[i + 1] - v->cu_seqlens_host[i], tok);
  hs2::FullOutParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(vv);
  p.cu = v->cu_seqlens;
  p.B = v->batch;
  p.Hq = d->num_q_heads;
  p.Hkv = d->num_kv_heads;
  p.max_tiles = std::max(1, hs2::ceil_div(geo.max_len, tok));
  p.c = scale_log2(d);
  p.lse2 = lse2;
  p.out = out;
  hipError_t e = hs2::launch_full_out(geo.G, out_dtype == HS2_OUT_F32, p, n_tasks, s);
  if (e != hipSuccess) return hip_fail(e, "full-layer output kernel");
  return HS2_OK;
}

// K/V of a sparse launch: bf16 rows, or (fp8_scales = {k_scale, v_scale}) E4M3 codes
void set_kv(hs2::SparseParams* p, const void* k, const void* v, const float* fp8_scales) {
  if (fp8_scales) {
    p->k8 = static_cast<const uint8_t*>(k);
    p->v8 = static_cast<const uint8_t*>(v);
    p->v_scale = fp8_scales[1];
  } else {
    p->k = static_cast<const uint16_t*>(k);
    p->v = static_cast<const uint16_t*>(v);
  }
}

// FP8 scales: finite and > 0; code rows are read 8 bytes at a time
int check_fp8(const void* k8, const void* v8, float k_scale, float v_scale) {
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return HS2_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k8) | reinterpret_cast<uintptr_t>(v8)) & 7u)
    return HS2_ERR_INVALID_ARG;
  return HS2_OK;
}

// The shared-gather plan of idx (rows as written by the selection) into plan.
int run_plan(const hs2_dims* d, const hs2_varlen* v, const Geometry& geo, const int32_t* idx,
             void* plan, hipStream_t s) {
  hs2::PlanParams pp{};
  pp.idx = idx;
  pp.cu = v->cu_seqlens;
  pp.B = v->batch;
  pp.Hkv = d->num_kv_heads;
  pp.KW = d->top_k + d->window;
  pp.T = geo.T;
  pp.n_grp = geo.n_grp;
  pp.cap = geo.plan_cap;
  pp.list = static_cast<uint32_t*>(plan);
  pp.count = reinterpret_cast<int32_t*>(static_cast<char*>(plan) + geo.off_pcount);
  hipError_t e = hs2::launch_sparse_plan(geo.G, pp, s);
  if (e != hipSuccess) return hip_fail(e, "sparse plan kernel");
  return HS2_OK;
}

// One sparse layer: one wave per (token, KV group) over idx, or, with a plan
// (from run_plan), one wave per (token group, KV group) over the plan's unions.
int run_sparse(const hs2_dims* d, const hs2_varlen* v, const Geometry& geo, const void* q,
               const void* k, const void* vv, const int32_t* idx, void* out, int out_dtype,
               hipStream_t s, const float* fp8_scales = nullptr, const void* plan = nullptr) {
  if (geo.T == 0) return HS2_OK;
  hs2::SparseParams p{};
  if (plan) {
    p.plist = static_cast<const uint32_t*>(plan);
    p.pcount = reinterpret_cast<const int32_t*>(static_cast<const char*>(plan) + geo.off_pcount);
    p.pcap = geo.plan_cap;
    p.n_grp = geo.n_grp;
  }
  p.q = static_cast<const uint16_t*>(q);
  set_kv(&p, k, vv, fp8_scales);
  p.idx = idx;
  p.cu = v->cu_seqlens;
  p.B = v->batch;
  p.Hq = d->num_q_heads;
  p.Hkv = d->num_kv_heads;
  p.KW = d->top_k + d->window;
  p.T = geo.T;
  p.c = scale_log2(d) * (fp8_scales ? fp8_scales[0] : 1.f);
  p.out = out;
  p.n_part = 1;
  hipError_t e = hs2::launch_sparse(geo.G, out_dtype == HS2_OUT_F32, fp8_scales != nullptr, p, s);
  if (e != hipSuccess) return hip_fail(e, "sparse attention kernel");
  return HS2_OK;
}

int run_planned(const hs2_dims* dims, const hs2_varlen* varlen, const void* q, const void* k,
                const void* v, const void* plan, size_t plan_bytes, void* out, int out_dtype,
                void* stream, const float* fp8_scales) {
  Geometry geo;
  int st = validate(dims, varlen, &geo);
  if (st != HS2_OK) return st;
  if (out_dtype != HS2_OUT_BF16 && out_dtype != HS2_OUT_F32) return HS2_ERR_INVALID_ARG;
  if (fp8_scales && check_fp8(k, v, fp8_scales[0], fp8_scales[1]) != HS2_OK)
    return HS2_ERR_INVALID_ARG;
  if (geo.T == 0) return HS2_OK;
  if (!geo.plan_ok) return HS2_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out) return HS2_ERR_INVALID_ARG;
  if (!plan || plan_bytes < geo.plan_bytes) return HS2_ERR_WORKSPACE;
  return run_sparse(dims, varlen, geo, q, k, v, nullptr, out, out_dtype,
                    static_cast<hipStream_t>(stream), fp8_scales, plan);
}

}  // namespace

extern "C" {

int hs2_version(void) { return 2 * 10000 + 0 * 100 + 0; }

const char* hs2_status_string(int status) {
  switch (status) {
    case HS2_OK: return "ok";
    case HS2_ERR_INVALID_ARG: return "invalid argument";
    case HS2_ERR_UNSUPPORTED: return "unsupported configuration (head_dim must be 128, Hq/Hkv in {1,2,4,8,16})";
    case HS2_ERR_WORKSPACE: return "workspace missing or too small";
    case HS2_ERR_HIP: return g_hip_msg;
    case HS2_ERR_SCRATCH: return "the call needs more than the no-allocation scratch holds";
    default: return "unknown status";
  }
}

int hs2_workspace_size(const hs2_dims* dims, const hs2_varlen* varlen, int op, int n_sparse,
                       size_t* bytes_out) {
  if (!bytes_out) return HS2_ERR_INVALID_ARG;
  if (op == HS2_OP_DECODE_SELECT || op == HS2_OP_DECODE_SPARSE) {
    DecodeGeometry dg;
    int st = validate_decode(dims, varlen, &dg);
    if (st != HS2_OK) return st;
    *bytes_out = dg.geo.B == 0 ? 0 : (op == HS2_OP_DECODE_SPARSE ? dg.sparse_bytes : dg.bytes);
    return HS2_OK;
  }
  if (op != HS2_OP_SELECT && op != HS2_OP_SPARSE && op != HS2_OP_PREFILL_BLOCK &&
      op != HS2_OP_SPARSE_PLAN && op != HS2_OP_SELECT_MIN)
    return HS2_ERR_INVALID_ARG;
  if (op == HS2_OP_PREFILL_BLOCK && n_sparse < 0) return HS2_ERR_INVALID_ARG;
  Geometry geo;
  int st = validate(dims, varlen, &geo);
  if (st != HS2_OK) return st;
  if (geo.T == 0 || op == HS2_OP_SPARSE) {
    *bytes_out = 0;
  } else if (op == HS2_OP_SPARSE_PLAN) {
    if (!geo.plan_ok) return HS2_ERR_UNSUPPORTED;
    *bytes_out = geo.plan_bytes;
  } else if (op == HS2_OP_PREFILL_BLOCK) {
    *bytes_out = std::max(geo.select_bytes, plan_pays(geo, n_sparse) ? geo.plan_bytes : 0);
  } else if (op == HS2_OP_SELECT_MIN) {
    *bytes_out = min_select_bytes(geo);
  } else {
    *bytes_out = geo.select_bytes;
  }
  return HS2_OK;
}

int hs2_select(const hs2_dims* dims, const hs2_varlen* varlen, const void* q, const void* k,
               int32_t* idx_out, float* kth_score_out, void* workspace, size_t workspace_bytes,
               void* stream) {
  Geometry geo;
  int st = validate(dims, varlen, &geo);
  if (st != HS2_OK) return st;
  if (geo.T == 0) return HS2_OK;
  if (!q || !k || !idx_out) return HS2_ERR_INVALID_ARG;
  st = fit_workspace(&geo, workspace, workspace_bytes);
  if (st != HS2_OK) return st;
  return run_select(dims, varlen, geo, q, k, idx_out, kth_score_out, workspace,
                    static_cast<hipStream_t>(stream));
}

int hs2_sparse_attn(const hs2_dims* dims, const hs2_varlen* varlen, const void* q, const void* k,
                    const void* v, const int32_t* idx, void* out, int out_dtype, void* stream) {
  Geometry geo;
  int st = validate(dims, varlen, &geo);
  if (st != HS2_OK) return st;
  if (out_dtype != HS2_OUT_BF16 && out_dtype != HS2_OUT_F32) return HS2_ERR_INVALID_ARG;
  if (geo.T == 0) return HS2_OK;
  if (!q || !k || !v || !idx || !out) return HS2_ERR_INVALID_ARG;
  return run_sparse(dims, varlen, geo, q, k, v, idx, out, out_dtype,
                    static_cast<hipStream_t>(stream));
}

int hs2_sparse_plan(const hs2_dims* dims, const hs2_varlen* varlen, const int32_t* idx,
                    void* plan, size_t plan_bytes, void* stream) {
  Geometry geo;
  int st = validate(dims, varlen, &geo);
  if (st != HS2_OK) return st;
  if (geo.T == 0) return HS2_OK;
  if (!geo.plan_ok) return HS2_ERR_UNSUPPORTED;
  if (!idx) return HS2_ERR_INVALID_ARG;
  if (!plan || plan_bytes < geo.plan_bytes) return HS2_ERR_WORKSPACE;
  return run_plan(dims, varlen, geo, idx, plan, static_cast<hipStream_t>(stream));
}


int hs2_sparse_attn_planned(const hs2_dims* dims, const hs2_varlen* varlen, const void* q,
                            const void* k, const void* v, const void* plan, size_t plan_bytes,
                            void* out, int out_dtype, void* stream) {
  return run_planned(dims, varlen, q, k, v, plan, plan_bytes, out, out_dtype, stream, nullptr);
}

int hs2_sparse_attn_planned_fp8(const hs2_dims* dims, const hs2_varlen* varlen, const void* q,
                                const uint8_t* k8, const uint8_t* v8, float k_scale,
                                float v_scale, const void* plan, size_t plan_bytes, void* out,
                                int out_dtype, void* stream) {
  const float scales[2] = {k_scale, v_scale};
  return run_planned(dims, varlen, q, k8, v8, plan, plan_bytes, out, out_dtype, stream, scales);
}

int hs2_prefill_block(const hs2_dims* dims, const hs2_varlen* varlen, const void* q_full,
                      const void* k, const void* v, int n_sparse,
                      const void* const* q_sparse_host_array, void* const* out_sparse_host_array,
                      int out_dtype, int32_t* idx_out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  Geometry geo;
  int st = validate(dims, varlen, &geo);
  if (st != HS2_OK) return st;
  if (n_sparse < 0) return HS2_ERR_INVALID_ARG;
  if (out_dtype != HS2_OUT_BF16 && out_dtype != HS2_OUT_F32) return HS2_ERR_INVALID_ARG;
  if (geo.T == 0) return HS2_OK;
  if (!q_full || !k || !v || !idx_out) return HS2_ERR_INVALID_ARG;
  if (n_sparse > 0 && (!q_sparse_host_array || !out_sparse_host_array)) return HS2_ERR_INVALID_ARG;
  for (int i = 0; i < n_sparse; i++)
    if (!q_sparse_host_array[i] || !out_sparse_host_array[i]) return HS2_ERR_INVALID_ARG;
  st = fit_workspace(&geo, workspace, workspace_bytes);
  if (st != HS2_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_select(dims, varlen, geo, q_full, k, idx_out, nullptr, workspace, s);
  if (st != HS2_OK) return st;
  // the sparse layers share one gather plan, written over the selection's scratch
  // (stream order: the selection is done with it) when the workspace holds it. The
  // plan's cost grows with row positions: on rows up to kPlanShortRows it pays for
  // itself within one layer, on longer ones it takes two
  const void* plan = nullptr;
  if (plan_pays(geo, n_sparse) && workspace_bytes >= geo.plan_bytes) {
    st = run_plan(dims, varlen, geo, idx_out, workspace, s);
    if (st != HS2_OK) return st;
    plan = workspace;
  }
  for (int i = 0; i < n_sparse; i++) {
    st = run_sparse(dims, varlen, geo, q_sparse_host_array[i], k, v, idx_out,
                    out_sparse_host_array[i], out_dtype, s, nullptr, plan);
    if (st != HS2_OK) return st;
  }
  return HS2_OK;
}

int hs2_select_ex(const hs2_dims* dims, const hs2_varlen* varlen, const hs2_select_options* opts,
                  const void* q, const void* k, const void* v, int32_t* idx_out,
                  float* kth_score_out, void* workspace, size_t workspace_bytes, void* stream) {
  Geometry geo;
  int st = validate(dims, varlen, &geo);
  if (st != HS2_OK) return st;
  float beta = 0.f;
  int k_end = dims->top_k;
  if (opts) {
    beta = opts->oam_beta;
    if (!(std::isfinite(beta) && beta >= 0.f)) return HS2_ERR_INVALID_ARG;
    const float mu = opts->decay_mu;
    if (!(mu == 0.f || (mu > 0.f && mu <= 1.f))) return HS2_ERR_INVALID_ARG;
    for (float r : opts->reserved)
      if (r != 0.f) return HS2_ERR_INVALID_ARG;
    if (mu > 0.f) {
      if (geo.block) return HS2_ERR_UNSUPPORTED;  // blocks are ranked with one budget
      k_end = (int)std::floor((double)mu * dims->top_k + 0.5);
    }
  }
  if (geo.T == 0) return HS2_OK;
  if (!q || !k || !idx_out || (beta > 0.f && !v)) return HS2_ERR_INVALID_ARG;
  st = fit_workspace(&geo, workspace, workspace_bytes);
  if (st != HS2_OK) return st;
  return run_select(dims, varlen, geo, q, k, idx_out, kth_score_out, workspace,
                    static_cast<hipStream_t>(stream), v, beta, k_end);
}

int hs2_select_full(const hs2_dims* dims, const hs2_varlen* varlen, const void* q, const void* k,
                    const void* v, int32_t* idx_out, float* kth_score_out, void* out_full,
                    int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  Geometry geo;
  int st = validate(dims, varlen, &geo);
  if (st != HS2_OK) return st;
  if (out_dtype != HS2_OUT_BF16 && out_dtype != HS2_OUT_F32) return HS2_ERR_INVALID_ARG;
  if (geo.T == 0) return HS2_OK;
  if (!q || !k || !v || !idx_out || !out_full) return HS2_ERR_INVALID_ARG;
  st = fit_workspace(&geo, workspace, workspace_bytes);
  if (st != HS2_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the output sweep first: it also writes every row's log-sum-exp, which the
  // selection then takes instead of running its own statistics sweep
  st = run_full_out(dims, varlen, geo, q, k, v, out_full, out_dtype,
                    reinterpret_cast<float*>(static_cast<char*>(workspace) + geo.off_lse), s);
  if (st != HS2_OK) return st;
  return run_select(dims, varlen, geo, q, k, idx_out, kth_score_out, workspace, s, nullptr, 0.f, -1,
                    true);
}

int hs2_full_attn(const hs2_dims* dims, const hs2_varlen* varlen, const void* q, const void* k,
                  const void* v, void* out, int out_dtype, float* lse2_out, void* stream) {
  Geometry geo;
  int st = validate(dims, varlen, &geo);
  if (st != HS2_OK) return st;
  if (out_dtype != HS2_OUT_BF16 && out_dtype != HS2_OUT_F32) return HS2_ERR_INVALID_ARG;
  if (geo.T == 0) return HS2_OK;
  if (!q || !k || !v || !out) return HS2_ERR_INVALID_ARG;
  return run_full_out(dims, varlen, geo, q, k, v, out, out_dtype, lse2_out,
                      static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Decode selection; k8 set: the keys are an FP8 cache of scale k_scale
int run_decode_select(const hs2_dims* dims, const hs2_varlen* cache, const void* q, const void* k,
                      const uint8_t* k8, float k_scale, int32_t* idx_out, float* kth_score_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  DecodeGeometry dg;
  int st = validate_decode(dims, cache, &dg);
  if (st != HS2_OK) return st;
  if (k8 && check_fp8(k8, k8, k_scale, 1.f) != HS2_OK) return HS2_ERR_INVALID_ARG;
  if (dg.geo.B == 0) return HS2_OK;
  if (!q || !(k || k8) || !idx_out) return HS2_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < dg.bytes) return HS2_ERR_WORKSPACE;
  char* w = static_cast<char*>(workspace);
  hs2::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.k8 = k8;
  p.cu = cache->cu_seqlens;
  p.B = cache->batch;
  p.Hq = dims->num_q_heads;
  p.Hkv = dims->num_kv_heads;
  p.K = dims->top_k;
  p.W = dims->window;
  p.max_seqlen = std::max(1, dg.geo.max_len);
  p.T = dg.geo.T;
  p.split_len = hs2::decode_split_len(k8 != nullptr);
  p.n_split = hs2::ceil_div(p.max_seqlen, p.split_len);
  p.bitmap_words = dg.bitmap_words;
  p.c = scale_log2(dims) * (k8 ? k_scale : 1.f);
  p.z2 = reinterpret_cast<float*>(w + dg.off_z2);
  p.part = reinterpret_cast<float2*>(w + dg.off_part);
  p.dense = reinterpret_cast<uint32_t*>(w + dg.off_dense);
  p.lse2 = reinterpret_cast<float*>(w + dg.off_lse);
  p.tau = reinterpret_cast<uint32_t*>(w + dg.off_tau);
  p.n_pass = reinterpret_cast<int32_t*>(w + dg.off_npass);
  p.cand = reinterpret_cast<uint32_t*>(w + dg.off_cand);
  p.idx = idx_out;
  p.kth = kth_score_out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hs2::launch_decode_logits(dg.geo.G, p, s);
  if (e != hipSuccess) return hip_fail(e, "decode logits kernel");
  e = hs2::launch_decode_select(dg.geo.G, p, dg.lds, s);
  if (e != hipSuccess) return hip_fail(e, "decode select kernel");
  return HS2_OK;
}

}  // namespace

extern "C" {

int hs2_decode_select(const hs2_dims* dims, const hs2_varlen* cache, const void* q, const void* k,
                      int32_t* idx_out, float* kth_score_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return run_decode_select(dims, cache, q, k, nullptr, 1.f, idx_out, kth_score_out, workspace,
                           workspace_bytes, stream);
}

int hs2_decode_select_fp8(const hs2_dims* dims, const hs2_varlen* cache, const void* q,
                          const uint8_t* k8, float k_scale, int32_t* idx_out, float* kth_score_out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return run_decode_select(dims, cache, q, nullptr, k8, k_scale, idx_out, kth_score_out,
                           workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

int run_decode_sparse(const hs2_dims* dims, const hs2_varlen* cache, const void* q, const void* k,
                      const void* v, const int32_t* idx, void* out, int out_dtype, void* workspace,
                      size_t workspace_bytes, void* stream, const float* fp8_scales) {
  DecodeGeometry dg;
  int st = validate_decode(dims, cache, &dg);
  if (st != HS2_OK) return st;
  if (out_dtype != HS2_OUT_BF16 && out_dtype != HS2_OUT_F32) return HS2_ERR_INVALID_ARG;
  if (fp8_scales && check_fp8(k, v, fp8_scales[0], fp8_scales[1]) != HS2_OK)
    return HS2_ERR_INVALID_ARG;
  if (dg.geo.B == 0) return HS2_OK;
  if (!q || !k || !v || !idx || !out) return HS2_ERR_INVALID_ARG;
  if (dg.sparse_bytes > 0 && (!workspace || workspace_bytes < dg.sparse_bytes))
    return HS2_ERR_WORKSPACE;
  hs2::SparseParams p{};
  p.q = static_cast<const uint16_t*>(q);
  set_kv(&p, k, v, fp8_scales);
  p.idx = idx;
  p.cu = cache->cu_seqlens;
  p.B = cache->batch;
  p.Hq = dims->num_q_heads;
  p.Hkv = dims->num_kv_heads;
  p.KW = dims->top_k + dims->window;
  p.T = cache->batch;
  p.c = scale_log2(dims) * (fp8_scales ? fp8_scales[0] : 1.f);
  p.out = out;
  p.decode = 1;
  p.n_part = dg.n_part;
  if (dg.n_part > 1) {
    char* w = static_cast<char*>(workspace);
    p.part_o = reinterpret_cast<float*>(w + dg.off_po);
    p.part_ml = reinterpret_cast<float2*>(w + dg.off_pml);
  }
  hipError_t e = hs2::launch_sparse(dg.geo.G, out_dtype == HS2_OUT_F32, fp8_scales != nullptr, p,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode sparse attention kernel");
  return HS2_OK;
}

}  // namespace

extern "C" {

int hs2_decode_sparse_attn(const hs2_dims* dims, const hs2_varlen* cache, const void* q,
                           const void* k, const void* v, const int32_t* idx, void* out,
                           int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return run_decode_sparse(dims, cache, q, k, v, idx, out, out_dtype, workspace, workspace_bytes,
                           stream, nullptr);
}

int hs2_decode_sparse_attn_noalloc(const hs2_dims* dims, const hs2_varlen* cache, const void* q,
                                   const void* k, const void* v, const int32_t* idx, void* out,
                                   int out_dtype, void* stream) {
  static_assert(hs2::kNoAllocScratchBytes == HS2_NOALLOC_SCRATCH_BYTES, "one scratch size");
  DecodeGeometry dg;
  int st = validate_decode(dims, cache, &dg);
  if (st != HS2_OK) return st;
  if (dg.sparse_bytes > hs2::kNoAllocScratchBytes) return HS2_ERR_SCRATCH;
  void* scratch = nullptr;
  if (dg.geo.B > 0 && dg.sparse_bytes > 0) {
    hipError_t e = hs2::noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e, "no-allocation scratch lookup");
  }
  return run_decode_sparse(dims, cache, q, k, v, idx, out, out_dtype, scratch,
                           hs2::kNoAllocScratchBytes, stream, nullptr);
}

int hs2_decode_sparse_attn_fp8(const hs2_dims* dims, const hs2_varlen* cache, const void* q,
                               const uint8_t* k8, const uint8_t* v8, float k_scale, float v_scale,
                               const int32_t* idx, void* out, int out_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  const float sc[2] = {k_scale, v_scale};
  return run_decode_sparse(dims, cache, q, k8, v8, idx, out, out_dtype, workspace,
                           workspace_bytes, stream, sc);
}

int hs2_sparse_attn_fp8(const hs2_dims* dims, const hs2_varlen* varlen, const void* q,
                        const uint8_t* k8, const uint8_t* v8, float k_scale, float v_scale,
                        const int32_t* idx, void* out, int out_dtype, void* stream) {
  Geometry geo;
  int st = validate(dims, varlen, &geo);
  if (st != HS2_OK) return st;
  if (out_dtype != HS2_OUT_BF16 && out_dtype != HS2_OUT_F32) return HS2_ERR_INVALID_ARG;
  if (check_fp8(k8, v8, k_scale, v_scale) != HS2_OK) return HS2_ERR_INVALID_ARG;
  if (geo.T == 0) return HS2_OK;
  if (!q || !k8 || !v8 || !idx || !out) return HS2_ERR_INVALID_ARG;
  const float sc[2] = {k_scale, v_scale};
  return run_sparse(dims, varlen, geo, q, k8, v8, idx, out, out_dtype,
                    static_cast<hipStream_t>(stream), sc);
}

int hs2_quantize_fp8(const void* src, uint8_t* dst, int64_t n, float inv_scale, void* stream) {
  if (n < 0 || !(std::isfinite(inv_scale) && inv_scale > 0.f)) return HS2_ERR_INVALID_ARG;
  if (n == 0) return HS2_OK;
  if (!src || !dst) return HS2_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 7u))
    return HS2_ERR_INVALID_ARG;
  hipError_t e = hs2::launch_quantize_fp8(static_cast<const uint16_t*>(src), dst, n, inv_scale,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 quantize kernel");
  return HS2_OK;
}

int64_t hs2_plan_task(const int32_t* cu_seqlens_host, int32_t batch, int32_t rows_per_task,
                      int64_t task, int32_t* seq_out, int32_t* tile_out) {
  if (!cu_seqlens_host || batch < 0 || rows_per_task < 1) return HS2_ERR_INVALID_ARG;
  if (batch > 0 && cu_seqlens_host[0] != 0) return HS2_ERR_INVALID_ARG;
  int64_t n_tasks = 0;
  int max_len = 0;
  for (int i = 0; i < batch; i++) {
    if (cu_seqlens_host[i + 1] < cu_seqlens_host[i]) return HS2_ERR_INVALID_ARG;
    const int L = cu_seqlens_host[i + 1] - cu_seqlens_host[i];
    max_len = std::max(max_len, L);
    n_tasks += hs2::ceil_div(L, rows_per_task);
  }
  if (task >= 0 && task < n_tasks) {
    int seq = 0, tile = 0;
    hs2::plan_decode(cu_seqlens_host, batch, rows_per_task,
                     std::max(1, hs2::ceil_div(max_len, rows_per_task)), task, &seq, &tile);
    if (seq_out) *seq_out = seq;
    if (tile_out) *tile_out = tile;
  }
  return n_tasks;
}

}  // extern "C"
