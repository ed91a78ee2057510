/*
 * hs2.h - C ABI of the token-level sparse attention prefill library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (HySparse2 news summary of the MiMo-V3 architecture; paragraph
 * on two-level KV sharing, forced-recent paragraph, token-granularity
 * paragraph, ablation paragraph):
 *   - a hybrid module is one full-attention layer followed by sparse layers;
 *     the sparse layers reuse the full layer's KV cache and its token
 *     selection ("KV Reuse");
 *   - the full layer's complete attention scores choose the tokens: per query
 *     token t and KV group g, the K = 1024 best single tokens ("global") plus
 *     the W = 128 most recent tokens, which are always kept;
 *   - each sparse layer attends, with its own queries, only to the selected
 *     positions, renormalising the softmax over them (masking before the
 *     softmax, SHARP walkthrough section 2.3).
 *
 * Exact definitions used by this library (readings where the pages are silent):
 *   z[t,h,j] = softmax_scale * <q[t,h], k[j,g(h)]>, j <= t, g(h) = h / (Hq/Hkv)
 *   S[t,g,j] = sum_{h in g} exp(z[t,h,j] - m[t,h]) / l[t,h]
 *              (m, l: max and sum of exp over all causal keys of head h)
 *   candidates C_t = [0, t-W]; window W_t = [max(0, t-W+1), t]
 *   T_t = all of C_t if |C_t| <= K, else the K best by (S desc, position asc)
 *   I_t = ascending(T_t U W_t): n_t = min(t+1, K+W) entries, then -1 to K+W
 *   sparse layer: o[t,h] = sum_{j in I_t} softmax_j(scale * <q'[t,h], k[j,g]>) v[j,g]
 *
 * Conventions
 *   - Pointers are device pointers unless the name ends in _host.
 *   - bf16 tensors are raw 16-bit storage (uint16_t bit patterns).
 *   - Layouts are contiguous and token-major over the packed varlen batch:
 *       Q, O   [T, Hq,  head_dim]       K, V   [T, Hkv, head_dim]
 *       idx    [T, Hkv, top_k + window] int32, local positions (0-based within
 *              the token's own sequence), ascending, -1 padded.
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only
 *     enqueues work on it: no call synchronises, allocates device memory or
 *     keeps state between calls, so calls are thread-safe. Inputs must stay
 *     valid and outputs unread until the stream has passed the call.
 *   - The caller owns every buffer, including the workspace
 *     (size from hs2_workspace_size). Workspace contents need no initialisation.
 *   - Errors: all validation happens before anything is enqueued; on a
 *     validation error nothing is written. A HIP launch failure returns
 *     HS2_ERR_HIP (detail from hs2_status_string, per thread).
 *   - NaN/Inf in the inputs is outside the contract: outputs are then
 *     unspecified, but idx entries stay in range and no access goes out of
 *     bounds.
 */
#ifndef HS2_H_
#define HS2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  HS2_OK = 0,
  HS2_ERR_INVALID_ARG = -1, /* a pointer, size or cu_seqlens entry is invalid */
  HS2_ERR_UNSUPPORTED = -2, /* valid but not implemented: head_dim != 128, Hq/Hkv not in
                               {1,2,4,8,16}, or one sequence's K (L * Hkv * 256 bytes) >= 4 GiB */
  HS2_ERR_WORKSPACE = -3,   /* workspace pointer NULL or smaller than hs2_workspace_size */
  HS2_ERR_HIP = -4,         /* a HIP runtime call failed */
  HS2_ERR_SCRATCH = -5      /* the call needs more than the library's own scratch holds
                               (hs2_decode_sparse_attn_noalloc) */
};

/* Output element type of the sparse attention. */
enum {
  HS2_OUT_BF16 = 0, /* bf16 output (round to nearest even); P.V with P as two bf16 parts */
  HS2_OUT_F32 = 1   /* fp32 output; P.V with P as three bf16 parts (~fp32 precision)
                       -- the precise mode */
};

/* Operation selector for hs2_workspace_size. */
enum {
  HS2_OP_SELECT = 1,
  HS2_OP_SPARSE = 2,
  HS2_OP_PREFILL_BLOCK = 3,
  HS2_OP_DECODE_SELECT = 4,
  HS2_OP_DECODE_SPARSE = 5,
  HS2_OP_SPARSE_PLAN = 6, /* the plan buffer of hs2_sparse_plan */
  HS2_OP_SELECT_MIN = 7   /* the smallest workspace the selection accepts (see below) */
};

/* Flags of hs2_dims.flags. */
enum {
  /* Skip the sampled threshold: every row with more than top_k candidates is
     selected by the exact full-row path (the score of every candidate written to
     a dense row, then a full-row radix select; slower; results obey the same rule). */
  HS2_FLAG_EXACT_SELECT = 1u,
  /* Select aligned 64-token blocks instead of single tokens (the previous
     generation's granularity, the baseline of the pages' block-vs-token
     ablation: HySparse2 news summary, ablation paragraph): the candidates
     [0, t-W] are cut into blocks [64i, 64i+63]; a block scores the sum of S over
     its candidate tokens; the top_k/64 best blocks (score desc, block asc) are
     taken whole, then the window. top_k must be a multiple of 64; kth_score is
     the lowest selected block's score. Prefill only (hs2_select,
     hs2_prefill_block); every block row is ranked exactly. */
  HS2_FLAG_BLOCK_SELECT = 2u
};

typedef struct {
  int32_t num_q_heads;  /* Hq >= 1 */
  int32_t num_kv_heads; /* Hkv >= 1, Hq % Hkv == 0; G = Hq / Hkv in {1, 2, 4, 8, 16} */
  int32_t head_dim;     /* must be 128 */
  int32_t top_k;        /* K >= 0 global tokens per (t, g) */
  int32_t window;       /* W >= 0 forced recent tokens (includes t itself); K + W >= 1 */
  float softmax_scale;  /* finite, > 0; usually 1/sqrt(head_dim) */
  uint32_t flags;       /* HS2_FLAG_* bits, 0 by default */
} hs2_dims;

typedef struct {
  int32_t batch;                  /* B >= 0 sequences */
  const int32_t* cu_seqlens;      /* device [B+1]: cu[0] = 0, non-decreasing */
  const int32_t* cu_seqlens_host; /* host copy of the same [B+1] */
  int32_t max_seqlen;             /* >= every L_i and <= HS2_MAX_SEQLEN */
  int64_t total_tokens;           /* T = cu[B] */
} hs2_varlen;

#define HS2_MAX_SEQLEN 262144

/*
 * Bytes of workspace an operation needs for these dimensions.
 * op:
 *   HS2_OP_SELECT       the selection (hs2_select, hs2_select_ex, hs2_select_full):
 *                       per-row statistics, candidate rows of one chunk of tasks
 *                       (at most 4 GiB of candidates, 2 * top_k slots per row when
 *                       top_k > 1024; with the exact flag or top_k above 8192, dense
 *                       score rows of at most 16 GiB), exact-path
 *                       scratch. A smaller
 *                       workspace, down to HS2_OP_SELECT_MIN bytes, is accepted too:
 *                       the selection then runs in more, smaller chunks with the
 *                       same results.
 *   HS2_OP_SELECT_MIN   the smallest selection workspace (one task per chunk).
 *   HS2_OP_SPARSE       0: the per-token sparse layer needs no workspace.
 *   HS2_OP_PREFILL_BLOCK  for hs2_prefill_block with n_sparse layers (n_sparse >= 0):
 *                       the selection's size, or the plan's when larger and the
 *                       block will plan its layers (n_sparse >= 2, or n_sparse == 1
 *                       and no sequence longer than 32768 tokens).
 *   HS2_OP_SPARSE_PLAN  the plan buffer of hs2_sparse_plan (HS2_ERR_UNSUPPORTED when
 *                       no plan is possible for these dimensions).
 *   HS2_OP_DECODE_SELECT, HS2_OP_DECODE_SPARSE  the decode ops (`varlen` describes
 *                       the cache).
 * n_sparse is read for HS2_OP_PREFILL_BLOCK only. Returns HS2_OK and writes
 * *bytes_out, or a validation error (nothing written).
 */
int hs2_workspace_size(const hs2_dims* dims, const hs2_varlen* varlen, int op, int n_sparse,
                       size_t* bytes_out);

/*
 * Token selection of the full-attention layer. HySparse2 news summary: the
 * paragraph on two-level KV sharing (the full layer's complete attention scores
 * pick the tokens the sparse layers attend to), the token-granularity paragraph
 * (single tokens, not blocks: 1024 global tokens plus the 128 most recent) and
 * the forced-recent paragraph (the recent window is always kept); scores as the
 * softmax of the SHARP walkthrough, section 1.1. Steps: per-head row statistics
 * (m, l), group probability score S, top-K of the candidates [0, t-W], window
 * forcing, ascending index row (definitions at the top of this file).
 * q [T,Hq,128] bf16 (the full layer's queries), k [T,Hkv,128] bf16 in;
 * idx_out [T,Hkv,K+W] int32 out. kth_score_out (nullable, device [T,Hkv] float):
 * the score S of the lowest-ranked selected global candidate, or -1 when every
 * candidate was taken. workspace: at least hs2_workspace_size(HS2_OP_SELECT_MIN)
 * bytes, caller-owned, no initialisation needed. Errors: HS2_ERR_INVALID_ARG
 * (a NULL q, k or idx_out with T > 0, or invalid dims / varlen),
 * HS2_ERR_UNSUPPORTED, HS2_ERR_WORKSPACE, HS2_ERR_HIP.
 */
int hs2_select(const hs2_dims* dims, const hs2_varlen* varlen, const void* q, const void* k,
               int32_t* idx_out, float* kth_score_out, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * One sparse attention layer over given index rows. HySparse2 news summary, the
 * KV Reuse paragraph: a sparse layer keeps no cache of its own and attends, with
 * its own queries, over the positions the full layer selected in the full
 * layer's K/V; the softmax is renormalised over those positions only (masking
 * before the softmax, SHARP walkthrough section 2.3).
 * q [T,Hq,128] bf16 (the layer's own queries), k, v [T,Hkv,128] bf16 (the
 * shared cache), idx [T,Hkv,K+W] int32 (any order; repeats count twice).
 * Entries outside [0, t] are ignored; a row with no valid entry gives a zero
 * output. out [T,Hq,128]: bf16 (HS2_OUT_BF16) or float (HS2_OUT_F32), written
 * for every token. Needs no workspace. Errors: HS2_ERR_INVALID_ARG (a NULL
 * pointer with T > 0, a bad out_dtype, invalid dims / varlen),
 * HS2_ERR_UNSUPPORTED, HS2_ERR_HIP.
 */
int hs2_sparse_attn(const hs2_dims* dims, const hs2_varlen* varlen, const void* q, const void* k,
                    const void* v, const int32_t* idx, void* out, int out_dtype, void* stream);

/*
 * Shared-gather plan of a selection's index rows, for the sparse layers that
 * reuse them (HySparse2 news summary, KV Reuse paragraph: every sparse layer of
 * the module attends over the same positions of the same cache). Consecutive
 * tokens select largely the same rows -- the forced window, and keys that score
 * high for all of them -- so the tokens t0 .. t0 + NT - 1 of the packed batch
 * (NT = 16 / G, at most 8; G = Hq / Hkv) are served together: for each such
 * group and KV group the plan
 * holds the sorted union of their rows, each with the set of tokens that hold
 * it, and a planned layer gathers every union row once for all of them.
 * idx [T,Hkv,K+W] int32 in the selection's format (hs2_select, hs2_select_ex,
 * hs2_select_full): each row ascending, no repeats, then -1 padding; entries
 * past t are skipped, and rows in another order are not supported (entries
 * below an earlier one are dropped). plan: device buffer of
 * hs2_workspace_size(HS2_OP_SPARSE_PLAN) bytes, owned by the caller, written
 * here and read by the planned layers (its layout is internal); it stays valid
 * while idx and cu_seqlens are unchanged. Errors: HS2_ERR_INVALID_ARG (idx NULL),
 * HS2_ERR_WORKSPACE (plan NULL or too small), HS2_ERR_UNSUPPORTED (sequences so
 * long that (max_seqlen + 16) * Hkv * 256 >= 2^32).
 */
int hs2_sparse_plan(const hs2_dims* dims, const hs2_varlen* varlen, const int32_t* idx,
                    void* plan, size_t plan_bytes, void* stream);

/*
 * hs2_sparse_attn over a plan from hs2_sparse_plan (the same dims, varlen and
 * rows): the same outputs (to fp32 rounding order), each union row gathered
 * once per token group. q, k, v, out, out_dtype as for hs2_sparse_attn.
 */
int hs2_sparse_attn_planned(const hs2_dims* dims, const hs2_varlen* varlen, const void* q,
                            const void* k, const void* v, const void* plan, size_t plan_bytes,
                            void* out, int out_dtype, void* stream);

/*
 * One hybrid module in prefill (HySparse2 news summary, paragraph on two-level
 * KV sharing: one full-attention layer followed by sparse layers that reuse its
 * KV cache and its token selection): hs2_select on (q_full, k) into idx_out,
 * then n_sparse >= 0 sparse layers, layer i reading q_sparse_host_array[i]
 * (device pointer) and writing out_sparse_host_array[i], all sharing k, v and
 * idx. The two pointer arrays live on the host and are read during the call.
 * With a workspace of hs2_workspace_size(HS2_OP_PREFILL_BLOCK, n_sparse) bytes
 * the layers run from one shared-gather plan (as hs2_sparse_plan +
 * hs2_sparse_attn_planned, the plan written over the selection's scratch) when
 * n_sparse >= 2, or n_sparse == 1 and no sequence is longer than 32768 tokens
 * (the plan's cost grows with the row positions; a single layer over longer
 * rows does not recover it); otherwise, or with a workspace too small for the
 * plan, they run as hs2_sparse_attn. Errors as hs2_select and hs2_sparse_attn
 * (HS2_ERR_INVALID_ARG also for n_sparse < 0 or a NULL layer pointer); all are
 * detected before anything is enqueued.
 */
int hs2_prefill_block(const hs2_dims* dims, const hs2_varlen* varlen, const void* q_full,
                      const void* k, const void* v, int n_sparse,
                      const void* const* q_sparse_host_array, void* const* out_sparse_host_array,
                      int out_dtype, int32_t* idx_out, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Selection variants for hs2_select_ex. */
typedef struct {
  /* Output-aware metric (Stem page, OAM paragraph: add beta * max(0, log |v_j|_2)
     to the selection logit): key j's group score is weighted,
       S'[t,g,j] = S[t,g,j] * max(1, |v[j,g]|_2)^oam_beta,
     and S' replaces S in the selection (tokens or blocks) and in kth_score.
     Finite, >= 0; 0 = the plain score. */
  float oam_beta;
  /* Position-decaying budget (Stem page, Token Position-Decay paragraph): query
     position t of a sequence of L tokens keeps
       K_t = top_k - floor((top_k - k_end) * t / (L - 1)),  k_end = floor(decay_mu * top_k + 0.5)
     candidates, top_k at the first position down to k_end at the last. Rows stay
     top_k + window wide; a smaller budget leaves more -1 padding. 0 = no decay,
     else in (0, 1]. Token selection only (HS2_ERR_UNSUPPORTED with
     HS2_FLAG_BLOCK_SELECT). To keep the total of a uniform budget K0, pass
     top_k = 2 K0 / (1 + decay_mu). */
  float decay_mu;
  float reserved[2]; /* must be 0 */
} hs2_select_options;

/*
 * hs2_select with the options above (opts NULL = hs2_select). v [T,Hkv,128]
 * bf16 is read when oam_beta > 0 (may be NULL otherwise). Workspace as for
 * HS2_OP_SELECT.
 */
int hs2_select_ex(const hs2_dims* dims, const hs2_varlen* varlen, const hs2_select_options* opts,
                  const void* q, const void* k, const void* v, int32_t* idx_out,
                  float* kth_score_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * hs2_select plus the full layer's own attention output (the full layer is a
 * real layer of the module; its softmax is the one whose scores select):
 *   out_full[t,h] = sum_{j <= t} softmax_j(softmax_scale <q[t,h], k[j,g]>) v[j,g]
 * q, k, v [T,*,128] bf16; out_full [T,Hq,128] bf16 (HS2_OUT_BF16, P as one bf16
 * part) or float (HS2_OUT_F32, P as three parts). The output sweep reuses the
 * selection's per-row log-sum-exp, so it needs no running maximum (it divides by
 * the sum of the P it accumulated). Workspace as for HS2_OP_SELECT.
 */
int hs2_select_full(const hs2_dims* dims, const hs2_varlen* varlen, const void* q, const void* k,
                    const void* v, int32_t* idx_out, float* kth_score_out, void* out_full,
                    int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The full layer's own attention output alone, without the selection (the
 * first sweep of hs2_select_full; the full layer's softmax as in the SHARP
 * walkthrough, section 1.1):
 *   out[t,h] = sum_{j <= t} softmax_j(softmax_scale <q[t,h], k[j,g]>) v[j,g]
 * q [T,Hq,128], k, v [T,Hkv,128] bf16; out [T,Hq,128] bf16 (HS2_OUT_BF16, P as
 * one bf16 part) or float (HS2_OUT_F32, P as three parts). lse2_out (nullable,
 * device [T,Hq] float): each row's base-2 log-sum-exp of the scaled logits,
 * log2 sum_{j <= t} 2^(c <q[t,h], k[j,g]>) with c = softmax_scale * log2(e)
 * (the natural-log value times 1/ln 2). Needs no workspace. Errors:
 * HS2_ERR_INVALID_ARG (a NULL q, k, v or out with T > 0, a bad out_dtype,
 * invalid dims / varlen), HS2_ERR_UNSUPPORTED, HS2_ERR_HIP.
 */
int hs2_full_attn(const hs2_dims* dims, const hs2_varlen* varlen, const void* q, const void* k,
                  const void* v, void* out, int out_dtype, float* lse2_out, void* stream);

/*
 * Decode step: one new token per sequence after the prompt (the cross-decoder
 * work HySparse2 moves to generation: HySparse2 news summary, early-exit
 * paragraph). `cache` describes the KV cache: sequence b holds L_b >= 1
 * tokens, the newest (position L_b - 1) being the new token itself, whose K/V
 * rows are already appended. q [B,Hq,128] bf16 are the full layer's queries of
 * the new tokens (row b). The selection of row b is exactly the prefill rule
 * for position t = L_b - 1: per-head softmax over all L_b cached keys, group
 * score S, top-K of [0, t-W] (S desc, position asc), the window [t-W+1, t],
 * ascending. idx_out [B,Hkv,K+W] int32 (row b*Hkv + g), kth_score_out nullable
 * [B,Hkv]. Every row is ranked exactly over all its candidates (no sampled
 * threshold). A sequence with L_b = 0 is an HS2_ERR_INVALID_ARG.
 */
int hs2_decode_select(const hs2_dims* dims, const hs2_varlen* cache, const void* q, const void* k,
                      int32_t* idx_out, float* kth_score_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * One sparse layer of the decode step: q [B,Hq,128] bf16 (the layer's own
 * queries of the new tokens), k, v the cache, idx [B,Hkv,K+W] (positions are
 * local to each sequence; entries outside [0, L_b - 1] are ignored); out
 * [B,Hq,128] bf16 or float as in hs2_sparse_attn. The few rows of a decode
 * step are split over several wavefronts whose partial results are merged, so
 * it takes a workspace of hs2_workspace_size(HS2_OP_DECODE_SPARSE) bytes
 * (0 when no split is needed; then workspace may be NULL).
 */
int hs2_decode_sparse_attn(const hs2_dims* dims, const hs2_varlen* cache, const void* q,
                           const void* k, const void* v, const int32_t* idx, void* out,
                           int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 KV cache (HySparse2 news summary, cost paragraph: the KV cache kept in
 * FP8). Codes are OCP FP8 E4M3 ("e4m3fn": bias 7, subnormals m * 2^-9, largest
 * finite 448, S.1111.111 NaN, no infinities) with one fp32 scale per tensor:
 *   k[j,g,e] = k_scale * E4M3(k8[j,g,e]),  v[j,g,e] = v_scale * E4M3(v8[j,g,e]).
 * k8, v8 [T,Hkv,128] uint8 device arrays, 8-byte aligned; scales finite, > 0.
 *
 * hs2_quantize_fp8 writes a cache: dst[i] = E4M3(float(src[i]) * inv_scale) for
 * n bf16 values src (16-byte aligned) into dst (8-byte aligned): the product
 * rounded to float, then to the nearest code (ties to even), saturating at
 * +-448; NaN gives a NaN code. Pass inv_scale = 1 / scale.
 */
int hs2_quantize_fp8(const void* src, uint8_t* dst, int64_t n, float inv_scale, void* stream);

/* hs2_sparse_attn over an FP8 cache (same q, idx, out and errors; no workspace). */
int hs2_sparse_attn_fp8(const hs2_dims* dims, const hs2_varlen* varlen, const void* q,
                        const uint8_t* k8, const uint8_t* v8, float k_scale, float v_scale,
                        const int32_t* idx, void* out, int out_dtype, void* stream);

/* hs2_sparse_attn_planned over an FP8 cache (same plan, q, out and errors; scales
 * as for hs2_sparse_attn_fp8). */
int hs2_sparse_attn_planned_fp8(const hs2_dims* dims, const hs2_varlen* varlen, const void* q,
                                const uint8_t* k8, const uint8_t* v8, float k_scale,
                                float v_scale, const void* plan, size_t plan_bytes, void* out,
                                int out_dtype, void* stream);

/* hs2_decode_select over an FP8 key cache: the full layer's decode queries
 * against k = k_scale * E4M3(k8) (same idx, kth, workspace and errors). */
int hs2_decode_select_fp8(const hs2_dims* dims, const hs2_varlen* cache, const void* q,
                          const uint8_t* k8, float k_scale, int32_t* idx_out, float* kth_score_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * hs2_decode_sparse_attn for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments (without the workspace), results and errors as
 * hs2_decode_sparse_attn; the call allocates nothing. The partials of the split
 * rows go to a library-owned device array of HS2_NOALLOC_SCRATCH_BYTES, one per
 * GPU, which that GPU keeps until the process ends; its address is looked up
 * on the first call made on each device (with that device current). The device
 * current on the calling thread must be the one `stream` belongs to. A call
 * whose partials would need more (hs2_workspace_size(HS2_OP_DECODE_SPARSE) >
 * HS2_NOALLOC_SCRATCH_BYTES; no configuration of this library's limits does)
 * returns HS2_ERR_SCRATCH before anything is enqueued. Every call on one GPU
 * shares its array and leaves its own partials there (nothing needs clearing:
 * each call writes every partial it reads): calls on one stream are ordered and
 * safe, calls that overlap on one GPU (concurrent streams, threads) race.
 */
#define HS2_NOALLOC_SCRATCH_BYTES (20u << 20)
int hs2_decode_sparse_attn_noalloc(const hs2_dims* dims, const hs2_varlen* cache, const void* q,
                                   const void* k, const void* v, const int32_t* idx, void* out,
                                   int out_dtype, void* stream);

/* hs2_decode_sparse_attn over an FP8 cache (same workspace as HS2_OP_DECODE_SPARSE). */
int hs2_decode_sparse_attn_fp8(const hs2_dims* dims, const hs2_varlen* cache, const void* q,
                               const uint8_t* k8, const uint8_t* v8, float k_scale, float v_scale,
                               const int32_t* idx, void* out, int out_dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Static text for a status; for HS2_ERR_HIP the last HIP error of this thread. */
const char* hs2_status_string(int status);

/*
 * Planner query (host only, no GPU needed): the selection work of a varlen
 * batch is cut into tasks of `rows_per_task` tokens of one sequence, ordered by
 * decreasing cost (tile index within its sequence, descending; then sequence
 * ascending). For task index `task` in [0, n_tasks) writes its sequence and
 * tile index. Returns the number of tasks (>= 0), or a negative status.
 */
int64_t hs2_plan_task(const int32_t* cu_seqlens_host, int32_t batch, int32_t rows_per_task,
                      int64_t task, int32_t* seq_out, int32_t* tile_out);

/* Library version: major * 10000 + minor * 100 + patch. */
int hs2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HS2_H_ */
