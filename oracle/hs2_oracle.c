/*
 * hs2_oracle.c - TEST INFRASTRUCTURE ONLY. Plain, slow, fp64 CPU reference of
 * HySparse2-style token-level sparse attention in prefill. Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load this library; the
 * GPU library never calls it and shares no code with it.
 *
 * What it computes (each point cites the page it follows):
 *  - A hybrid module is one full-attention layer followed by sparse layers that
 *    reuse the full layer's KV cache and its token-selection result
 *    ("KV Reuse"; HySparse2 news summary of the MiMo-V3 architecture, the
 *    two-level KV sharing paragraph).
 *  - The full layer's complete attention scores pick the tokens for the later
 *    sparse layers (same page, ablation paragraph, last sentences).
 *  - Selection is per single token: 1024 global tokens plus the 128 most recent
 *    tokens forced in (same page, token-granularity paragraph; forcing recent
 *    tokens replaces the old sliding-window branch, forced-recent paragraph).
 *  - Attention is softmax(Q K^T / sqrt(d)) V (SHARP walkthrough, section 1.1).
 *    Restricting attention to a set by setting the other logits to -inf before
 *    the softmax renormalises over the set (SHARP walkthrough, section 2.3).
 *
 * Readings taken where the pages are silent (each is listed in the design doc):
 *  R1 selection is per query token t and KV group g;
 *  R2 the group score sums each head's normalised probability:
 *       S[t,g,j] = sum_{h in g} exp(z[t,h,j] - m[t,h]) / l[t,h],
 *     z = scale * <q[t,h], k[j,g]>, m = max_{j<=t} z, l = sum_{j<=t} exp(z - m);
 *  R3 the K global tokens are chosen outside the window: candidates
 *     C_t = [0, t-W], window W_t = [max(0, t-W+1), t] (includes t itself);
 *  R4 if |C_t| <= K all candidates are taken; otherwise the K best by
 *     (S descending, position ascending);
 *  R5 the index row is ascending(T_t U W_t), n_t = min(t+1, K+W) entries,
 *     padded with -1 to K+W;
 *  R6 sparse layers take a fresh Q' and attend over I_t only (renormalised).
 *  Heads are grouped contiguously: head h belongs to KV group h / (Hq/Hkv).
 *  Varlen: rows of sequence i see only sequence i; positions are local.
 *
 * All arithmetic is in double. bf16 inputs convert exactly. Work is split over
 * threads by rows; every row is computed independently, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf2d(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* double -> bf16 bits, round to nearest even (own implementation). */
static uint16_t d2bf(double x) {
  if (isnan(x)) return 0x7FC0u;
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  double ax = fabs(x);
  if (isinf(x) || ax >= 3.3961775292304e38) return (uint16_t)(sign | 0x7F80u);
  if (ax < 1.1754943508222875e-38) { /* bf16 subnormal range: step 2^-133 */
    double s = ax * 1.0889035741470030830827987437817e40; /* 2^133 */
    double fl = floor(s), rem = s - fl;
    uint32_t m = (uint32_t)fl;
    if (rem > 0.5 || (rem == 0.5 && (m & 1u))) m++;
    return (uint16_t)(sign | m);
  }
  int e;
  double fr = frexp(ax, &e); /* ax = fr * 2^e, fr in [0.5, 1) */
  /* bf16 keeps 8 significant bits: scale to [128, 256) */
  double s = ldexp(fr, 8);
  double fl = floor(s), rem = s - fl;
  uint32_t m = (uint32_t)fl; /* 128..255 */
  if (rem > 0.5 || (rem == 0.5 && (m & 1u))) m++;
  if (m == 256) { m = 128; e++; }
  int be = e - 1 + 127; /* value = (m/128) * 2^(e-1) */
  if (be >= 255) return (uint16_t)(sign | 0x7F80u);
  return (uint16_t)(sign | ((uint32_t)be << 7) | (m - 128));
}

/* ---- FP8 KV cache ----
 * The pages store the KV cache in FP8 (HySparse2 news summary, cost paragraph:
 * the cache size at 1M tokens with an FP8 cache) without naming the encoding;
 * reading: OCP 8-bit floating point E4M3 ("e4m3fn"): sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; S.1111.111
 * is NaN; there are no infinities, the largest finite value is 448. One fp32
 * scale per tensor: value = scale * e4m3(code). */
static double e4m3_to_d(uint8_t b) {
  const int e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return (b & 0x80) ? -v : v;
}

/* float -> E4M3, rounded to nearest (ties to an even code), saturating at
 * +-448; NaN -> 0x7F. */
static uint8_t f_to_e4m3(float x) {
  if (isnan(x)) return 0x7F;
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  const double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  int e2;
  frexp(a, &e2); /* a in [2^(e2-1), 2^e2) */
  int ue = e2 - 1;
  if (ue < -6) ue = -6; /* subnormals share the spacing of the lowest binade */
  const double s = ldexp(a, 3 - ue); /* a in units of the spacing 2^(ue-3) */
  const double fl = floor(s), rem = s - fl;
  uint32_t n = (uint32_t)fl;
  if (rem > 0.5 || (rem == 0.5 && (n & 1u))) n++;
  if (n < 8) return (uint8_t)(sign | n); /* subnormal (or zero): ue == -6 */
  if (n == 16) { n = 8; ue++; }
  return (uint8_t)(sign | ((uint32_t)(ue + 7) << 3) | (n - 8));
}

typedef struct {
  int B, Hq, Hkv, d, K, W;
  double scale;
  const int32_t* cu;
  int block; /* 0: single-token selection; > 0: blocks of this many tokens (K a multiple) */
  double oam_beta; /* > 0: S_j is weighted by max(1, |v_j|_2)^beta (needs v) */
  int k_end;       /* budget at a sequence's last position (K: no decay) */
} dims_t;

/* Position-decaying budget (Stem page, Token Position-Decay paragraph): the
 * top-k budget of query position t falls linearly from K at the first position
 * of its sequence to k_end at the last one (L tokens). Reading: the decrement
 * (K - k_end) * t / (L - 1) is rounded down, so K_t is exact in integers. */
static int row_budget(const dims_t* D, int64_t t, int64_t L) {
  if (L <= 1 || D->k_end == D->K) return D->K;
  return D->K - (int)(((int64_t)(D->K - D->k_end) * t) / (L - 1));
}

static int find_seq(const dims_t* D, int64_t t_global) {
  int lo = 0, hi = D->B - 1;
  while (lo < hi) { /* last i with cu[i] <= t_global */
    int mid = (lo + hi + 1) / 2;
    if (D->cu[mid] <= t_global) lo = mid; else hi = mid - 1;
  }
  return lo;
}

/* ---- O1 + O2: per-head row statistics and the group score of one row ---- */
/* Row (t, g) of the sequence starting at token `base`; qt holds the query
 * token's Hq query rows [Hq, d]. Keys are bf16 (k), or with k8 set FP8 codes of
 * value k_scale * E4M3(code). S_out[j] for j in [0, t]; scratch z holds
 * G*(t+1) doubles. */
static void row_group_scores(const dims_t* D, const uint16_t* qt, const uint16_t* k,
                             const uint8_t* k8, double k_scale, int64_t base, int64_t t, int g,
                             double* z, double* S_out, double* m_out, double* l_out) {
  const int G = D->Hq / D->Hkv, d = D->d;
  const int64_t n = t + 1;
  for (int hh = 0; hh < G; hh++) {
    const int h = g * G + hh;
    const uint16_t* qr = qt + (size_t)h * d;
    double qd[1024];
    for (int e = 0; e < d; e++) qd[e] = bf2d(qr[e]);
    double* zr = z + (size_t)hh * n;
    double m = -INFINITY;
    for (int64_t j = 0; j < n; j++) { /* causal keys j <= t */
      const size_t off = ((size_t)(base + j) * D->Hkv + g) * d;
      double acc = 0.0;
      if (k8)
        for (int e = 0; e < d; e++) acc += qd[e] * (k_scale * e4m3_to_d(k8[off + e]));
      else
        for (int e = 0; e < d; e++) acc += qd[e] * bf2d(k[off + e]);
      zr[j] = D->scale * acc;
      if (zr[j] > m) m = zr[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; j++) l += exp(zr[j] - m);
    if (m_out) m_out[hh] = m;
    if (l_out) l_out[hh] = l;
    for (int64_t j = 0; j < n; j++) {
      double p = exp(zr[j] - m) / l;
      if (hh == 0) S_out[j] = p; else S_out[j] += p;
    }
  }
}

typedef struct { double s; int64_t j; } cand_t;

static int cmp_cand(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->s > y->s) return -1; /* higher score first */
  if (x->s < y->s) return 1;
  if (x->j < y->j) return -1; /* then lower position */
  if (x->j > y->j) return 1;
  return 0;
}

/* ---- O3..O6 for one row: window, candidates, top-K, ascending index row ---- */
static void row_select(const dims_t* D, const double* S, int64_t t, int64_t L, int32_t* idx_row,
                       double* kth, cand_t* cbuf, uint8_t* mark) {
  const int K = row_budget(D, t, L), W = D->W, KW = D->K + D->W;
  const int64_t n_cand = t - W + 1 > 0 ? t - W + 1 : 0; /* C_t = [0, t-W] */
  memset(mark, 0, (size_t)(t + 1));
  for (int64_t j = (t - W + 1 > 0 ? t - W + 1 : 0); j <= t; j++) mark[j] = 1; /* W_t */
  if (n_cand <= K || K == 0) {
    /* all candidates fit in the budget (or the budget is empty) */
    if (n_cand <= K)
      for (int64_t j = 0; j < n_cand; j++) mark[j] = 1;
    *kth = -1.0;
  } else if (D->block > 0) {
    /* block selection (the previous generation's granularity, HySparse2 news
     * summary, block-vs-token paragraph and ablation): the candidates are cut
     * into aligned blocks of D->block tokens; a block scores the sum of S over
     * its candidate tokens; the K / block best blocks (score desc, block asc)
     * are taken whole. */
    const int bs = D->block;
    const int64_t nb = (n_cand + bs - 1) / bs;
    const int n_sel = K / bs;
    for (int64_t b = 0; b < nb; b++) {
      double sum = 0.0;
      for (int64_t j = b * bs; j < (b + 1) * bs && j < n_cand; j++) sum += S[j];
      cbuf[b].s = sum;
      cbuf[b].j = b;
    }
    qsort(cbuf, (size_t)nb, sizeof(cand_t), cmp_cand);
    for (int i = 0; i < n_sel; i++)
      for (int64_t j = cbuf[i].j * bs; j < (cbuf[i].j + 1) * bs && j < n_cand; j++) mark[j] = 1;
    *kth = n_sel > 0 ? cbuf[n_sel - 1].s : -1.0;
  } else {
    for (int64_t j = 0; j < n_cand; j++) { cbuf[j].s = S[j]; cbuf[j].j = j; }
    qsort(cbuf, (size_t)n_cand, sizeof(cand_t), cmp_cand);
    for (int i = 0; i < K; i++) mark[cbuf[i].j] = 1;
    *kth = cbuf[K - 1].s;
  }
  int c = 0;
  for (int64_t j = 0; j <= t; j++)
    if (mark[j]) idx_row[c++] = (int32_t)j;
  for (; c < KW; c++) idx_row[c] = -1;
}

/* ------------------------------ threading -------------------------------- */
typedef struct {
  const dims_t* D;
  const uint16_t *q, *k, *v;
  const int64_t* rows;
  int64_t n_rows;
  /* select */
  int32_t* idx_out;
  double* kth_out;
  /* sparse */
  const int32_t* idx_in;
  double* o64;
  uint16_t* o16;
  int64_t next;
  pthread_mutex_t mu;
  int max_len;
  /* decode: one query per sequence (q, idx and outputs indexed by sequence),
     at the sequence's last position */
  int decode;
  /* FP8 KV cache (sparse attention): codes and per-tensor scales, used instead
     of k / v when k8 is set */
  const uint8_t *k8, *v8;
  double k_scale, v_scale;
} job_t;

/* One K (is_v = 0) or V row of d values starting at element `off`, in double. */
static void kv_row(const job_t* J, int is_v, size_t off, int d, double* out) {
  if (J->k8) {
    const uint8_t* p = (is_v ? J->v8 : J->k8) + off;
    const double sc = is_v ? J->v_scale : J->k_scale;
    for (int c = 0; c < d; c++) out[c] = sc * e4m3_to_d(p[c]);
  } else {
    const uint16_t* p = (is_v ? J->v : J->k) + off;
    for (int c = 0; c < d; c++) out[c] = bf2d(p[c]);
  }
}

static int64_t take(job_t* J, int64_t chunk, int64_t* end) {
  pthread_mutex_lock(&J->mu);
  int64_t s = J->next;
  J->next += chunk;
  pthread_mutex_unlock(&J->mu);
  *end = s + chunk < J->n_rows ? s + chunk : J->n_rows;
  return s;
}

static void* select_worker(void* arg) {
  job_t* J = (job_t*)arg;
  const dims_t* D = J->D;
  const int G = D->Hq / D->Hkv, KW = D->K + D->W;
  size_t L = (size_t)J->max_len;
  double* z = (double*)malloc(sizeof(double) * (size_t)G * L);
  double* S = (double*)malloc(sizeof(double) * L);
  cand_t* cb = (cand_t*)malloc(sizeof(cand_t) * L);
  uint8_t* mark = (uint8_t*)malloc(L);
  for (;;) {
    int64_t e, s = take(J, 8, &e);
    if (s >= J->n_rows) break;
    for (int64_t r = s; r < e; r++) {
      int64_t row = J->rows ? J->rows[r] : r; /* row = t_global * Hkv + g (decode: b * Hkv + g) */
      int64_t tg = row / D->Hkv;
      int g = (int)(row % D->Hkv);
      int64_t base, t, L;
      const uint16_t* qt;
      if (J->decode) {
        base = D->cu[tg];
        L = D->cu[tg + 1] - base;
        t = L - 1;
        qt = J->q + (size_t)tg * D->Hq * D->d;
      } else {
        int i = find_seq(D, tg);
        base = D->cu[i];
        L = D->cu[i + 1] - base;
        t = tg - base;
        qt = J->q + (size_t)tg * D->Hq * D->d;
      }
      row_group_scores(D, qt, J->k, J->k8, J->k_scale, base, t, g, z, S, NULL, NULL);
      if (D->oam_beta > 0.0) {
        /* output-aware metric (Stem page, OAM paragraph): the logit term
         * beta * max(0, log |v_j|_2) multiplies key j's probability, and so its
         * group score, by max(1, |v_j|_2)^beta */
        for (int64_t j = 0; j <= t; j++) {
          const uint16_t* vr = J->v + ((size_t)(base + j) * D->Hkv + g) * D->d;
          double n2 = 0.0;
          for (int c = 0; c < D->d; c++) n2 += bf2d(vr[c]) * bf2d(vr[c]);
          const double nv = sqrt(n2);
          S[j] *= pow(nv > 1.0 ? nv : 1.0, D->oam_beta);
        }
      }
      double kth;
      row_select(D, S, t, L, J->idx_out + (size_t)r * KW, &kth, cb, mark);
      if (J->kth_out) J->kth_out[r] = kth;
    }
  }
  free(z); free(S); free(cb); free(mark);
  return NULL;
}

/* ---- O7: sparse attention of one token over its index rows (all heads) ---- */
static void* sparse_worker(void* arg) {
  job_t* J = (job_t*)arg;
  const dims_t* D = J->D;
  const int G = D->Hq / D->Hkv, KW = D->K + D->W, d = D->d;
  double* y = (double*)malloc(sizeof(double) * (size_t)KW);
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  double qd[1024], rd[1024];
  for (;;) {
    int64_t e, s = take(J, 16, &e);
    if (s >= J->n_rows) break;
    for (int64_t r = s; r < e; r++) {
      int64_t tg = J->rows ? J->rows[r] : r; /* decode: the sequence */
      int64_t base, t;
      if (J->decode) {
        base = D->cu[tg];
        t = D->cu[tg + 1] - base - 1;
      } else {
        int i = find_seq(D, tg);
        base = D->cu[i];
        t = tg - base;
      }
      for (int h = 0; h < D->Hq; h++) {
        const int g = h / G;
        const int32_t* ir = J->idx_in + ((size_t)tg * D->Hkv + g) * KW;
        const uint16_t* qr = J->q + ((size_t)tg * D->Hq + h) * d;
        for (int c = 0; c < d; c++) qd[c] = bf2d(qr[c]);
        double mu = -INFINITY;
        for (int a = 0; a < KW; a++) {
          int32_t j = ir[a];
          if (j < 0 || j > t) { y[a] = -INFINITY; continue; } /* not in I_t */
          kv_row(J, 0, ((size_t)(base + j) * D->Hkv + g) * d, d, rd);
          double dot = 0.0;
          for (int c = 0; c < d; c++) dot += qd[c] * rd[c];
          y[a] = D->scale * dot;
          if (y[a] > mu) mu = y[a];
        }
        double den = 0.0;
        for (int c = 0; c < d; c++) acc[c] = 0.0;
        if (mu > -INFINITY) {
          for (int a = 0; a < KW; a++) {
            if (y[a] == -INFINITY) continue;
            double w = exp(y[a] - mu);
            den += w;
            kv_row(J, 1, ((size_t)(base + ir[a]) * D->Hkv + g) * d, d, rd);
            for (int c = 0; c < d; c++) acc[c] += w * rd[c];
          }
        }
        size_t o = ((size_t)r * D->Hq + h) * d;
        for (int c = 0; c < d; c++) {
          double val = den > 0.0 ? acc[c] / den : 0.0;
          if (J->o64) J->o64[o + c] = val;
          if (J->o16) J->o16[o + c] = d2bf(val);
        }
      }
    }
  }
  free(y); free(acc);
  return NULL;
}

static int check_dims(const dims_t* D) {
  if (D->B < 1 || D->Hq < 1 || D->Hkv < 1 || D->Hq % D->Hkv || D->d < 1 || D->d > 1024) return -1;
  if (D->K < 0 || D->W < 0 || D->K + D->W < 1) return -1;
  if (D->block < 0 || (D->block > 0 && D->K % D->block)) return -1;
  if (D->k_end < 0 || D->k_end > D->K || (D->block > 0 && D->k_end != D->K)) return -1;
  if (D->cu[0] != 0) return -1;
  for (int i = 0; i < D->B; i++)
    if (D->cu[i + 1] < D->cu[i]) return -1;
  return 0;
}

static int run(job_t* J, void* (*fn)(void*), int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_mutex_init(&J->mu, NULL);
  J->next = 0;
  pthread_t th[256];
  int n = 0;
  for (int i = 0; i < nthreads; i++) {
    if (pthread_create(&th[i], NULL, fn, J) != 0) break;
    n++;
  }
  if (n == 0) fn(J);
  for (int i = 0; i < n; i++) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&J->mu);
  return 0;
}

static int max_len(const dims_t* D) {
  int m = 1;
  for (int i = 0; i < D->B; i++)
    if (D->cu[i + 1] - D->cu[i] > m) m = D->cu[i + 1] - D->cu[i];
  return m;
}

/*
 * Selection (O1..O6). rows: list of row ids t_global*Hkv + g, or NULL for all
 * T*Hkv rows in order. idx_out [n_rows, K+W] int32; kth_out [n_rows] (nullable):
 * the score of the lowest-ranked selected global candidate, -1 when all were taken
 * (or when K = 0, so none is).
 */
int hs2o_select(const uint16_t* q, const uint16_t* k, const int32_t* cu, int B, int Hq, int Hkv,
                int d, double scale, int K, int W, const int64_t* rows, int64_t n_rows,
                int32_t* idx_out, double* kth_out, int nthreads) {
  dims_t D = {B, Hq, Hkv, d, K, W, scale, cu, 0, 0.0, K};
  if (!q || !k || !cu || !idx_out || check_dims(&D)) return -1;
  int64_t T = cu[B];
  if (!rows) n_rows = T * Hkv;
  for (int64_t r = 0; rows && r < n_rows; r++)
    if (rows[r] < 0 || rows[r] >= T * Hkv) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.D = &D; J.q = q; J.k = k; J.rows = rows; J.n_rows = n_rows;
  J.idx_out = idx_out; J.kth_out = kth_out; J.max_len = max_len(&D);
  return run(&J, select_worker, nthreads);
}

/* hs2o_select with block selection: blocks of `block` tokens (K a multiple of
 * it); kth_out is the score of the lowest-ranked selected block. block = 0 is
 * hs2o_select. */
int hs2o_select_blocks(const uint16_t* q, const uint16_t* k, const int32_t* cu, int B, int Hq,
                       int Hkv, int d, double scale, int K, int W, int block, const int64_t* rows,
                       int64_t n_rows, int32_t* idx_out, double* kth_out, int nthreads) {
  dims_t D = {B, Hq, Hkv, d, K, W, scale, cu, block, 0.0, K};
  if (!q || !k || !cu || !idx_out || check_dims(&D)) return -1;
  int64_t T = cu[B];
  if (!rows) n_rows = T * Hkv;
  for (int64_t r = 0; rows && r < n_rows; r++)
    if (rows[r] < 0 || rows[r] >= T * Hkv) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.D = &D; J.q = q; J.k = k; J.rows = rows; J.n_rows = n_rows;
  J.idx_out = idx_out; J.kth_out = kth_out; J.max_len = max_len(&D);
  return run(&J, select_worker, nthreads);
}

/* Selection with the variants: the output-aware metric S'_j = S_j *
 * max(1, |v_j|_2)^beta (beta >= 0; v [T, Hkv, d], may be NULL when beta = 0),
 * the position-decaying budget from K down to k_end (0 <= k_end <= K; k_end = K
 * is no decay; token selection only), and block selection as in
 * hs2o_select_blocks. kth_out is the score (S' with beta > 0) of the
 * lowest-ranked selected candidate (or block). Rows are K + W wide; a row with
 * a smaller budget holds fewer entries and more -1 padding. */
int hs2o_select_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* cu,
                   int B, int Hq, int Hkv, int d, double scale, int K, int W, int block,
                   double beta, int k_end, const int64_t* rows, int64_t n_rows, int32_t* idx_out,
                   double* kth_out, int nthreads) {
  dims_t D = {B, Hq, Hkv, d, K, W, scale, cu, block, beta, k_end};
  if (!q || !k || !cu || !idx_out || check_dims(&D) || !(beta >= 0.0)) return -1;
  if (beta > 0.0 && !v) return -1;
  int64_t T = cu[B];
  if (!rows) n_rows = T * Hkv;
  for (int64_t r = 0; rows && r < n_rows; r++)
    if (rows[r] < 0 || rows[r] >= T * Hkv) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.D = &D; J.q = q; J.k = k; J.v = v; J.rows = rows; J.n_rows = n_rows;
  J.idx_out = idx_out; J.kth_out = kth_out; J.max_len = max_len(&D);
  return run(&J, select_worker, nthreads);
}

/* The group score row S[t,g,0..t] (O1+O2) of one row, plus per-head m and l (nullable, [G]). */
int hs2o_group_scores(const uint16_t* q, const uint16_t* k, const int32_t* cu, int B, int Hq,
                      int Hkv, int d, double scale, int64_t t_global, int g, double* S_out,
                      double* m_out, double* l_out) {
  dims_t D = {B, Hq, Hkv, d, 1, 0, scale, cu, 0, 0.0, 1};
  if (!q || !k || !cu || !S_out || check_dims(&D) || g < 0 || g >= Hkv) return -1;
  if (t_global < 0 || t_global >= cu[B]) return -1;
  int i = find_seq(&D, t_global);
  int64_t base = cu[i], t = t_global - base;
  double* z = (double*)malloc(sizeof(double) * (size_t)(Hq / Hkv) * (size_t)(t + 1));
  if (!z) return -1;
  row_group_scores(&D, q + (size_t)t_global * Hq * d, k, NULL, 1.0, base, t, g, z, S_out, m_out,
                   l_out);
  free(z);
  return 0;
}

/*
 * Sparse attention (O7) with the index rows idx [T, Hkv, KW] (entries outside
 * [0, t] are ignored). tokens: list of global token ids or NULL for all T.
 * o64 [n, Hq, d] double (nullable), o16 [n, Hq, d] bf16 RNE (nullable).
 * A token whose row holds no valid entry gets a zero output.
 */
int hs2o_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* cu,
                     int B, int Hq, int Hkv, int d, double scale, int KW, const int32_t* idx,
                     const int64_t* tokens, int64_t n_tokens, double* o64, uint16_t* o16,
                     int nthreads) {
  dims_t D = {B, Hq, Hkv, d, KW, 0, scale, cu, 0, 0.0, KW};
  if (!q || !k || !v || !cu || !idx || check_dims(&D) || KW < 1) return -1;
  int64_t T = cu[B];
  if (!tokens) n_tokens = T;
  for (int64_t r = 0; tokens && r < n_tokens; r++)
    if (tokens[r] < 0 || tokens[r] >= T) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.D = &D; J.q = q; J.k = k; J.v = v; J.rows = tokens; J.n_rows = n_tokens;
  J.idx_in = idx; J.o64 = o64; J.o16 = o16;
  return run(&J, sparse_worker, nthreads);
}

/*
 * Decode step (one new query per sequence). cu describes the cache: sequence b
 * holds L_b >= 1 tokens and its query sits at its last position t = L_b - 1,
 * so row (b, g) is exactly prefill row (t, g) with q_dec[b] as the query.
 * q_dec [B, Hq, d]; idx_out [B*Hkv, K+W] (row b*Hkv + g); kth_out [B*Hkv] nullable.
 */
int hs2o_decode_select(const uint16_t* q_dec, const uint16_t* k, const int32_t* cu, int B, int Hq,
                       int Hkv, int d, double scale, int K, int W, int32_t* idx_out,
                       double* kth_out, int nthreads) {
  dims_t D = {B, Hq, Hkv, d, K, W, scale, cu, 0, 0.0, K};
  if (!q_dec || !k || !cu || !idx_out || check_dims(&D)) return -1;
  for (int b = 0; b < B; b++)
    if (cu[b + 1] - cu[b] < 1) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.D = &D; J.q = q_dec; J.k = k; J.n_rows = (int64_t)B * Hkv; J.decode = 1;
  J.idx_out = idx_out; J.kth_out = kth_out; J.max_len = max_len(&D);
  return run(&J, select_worker, nthreads);
}

/* Decode-step selection over an FP8 key cache (k = k_scale * E4M3(k8)); as
 * hs2o_decode_select otherwise. */
int hs2o_decode_select_fp8(const uint16_t* q_dec, const uint8_t* k8, double k_scale,
                           const int32_t* cu, int B, int Hq, int Hkv, int d, double scale, int K,
                           int W, int32_t* idx_out, double* kth_out, int nthreads) {
  dims_t D = {B, Hq, Hkv, d, K, W, scale, cu, 0, 0.0, K};
  if (!q_dec || !k8 || !cu || !idx_out || check_dims(&D)) return -1;
  for (int b = 0; b < B; b++)
    if (cu[b + 1] - cu[b] < 1) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.D = &D; J.q = q_dec; J.k8 = k8; J.k_scale = k_scale; J.n_rows = (int64_t)B * Hkv;
  J.decode = 1; J.idx_out = idx_out; J.kth_out = kth_out; J.max_len = max_len(&D);
  return run(&J, select_worker, nthreads);
}

/* Sparse attention of the decode queries q_dec [B, Hq, d] over idx [B, Hkv, KW];
 * o64 / o16 [B, Hq, d] (nullable). */
int hs2o_decode_sparse_attn(const uint16_t* q_dec, const uint16_t* k, const uint16_t* v,
                            const int32_t* cu, int B, int Hq, int Hkv, int d, double scale, int KW,
                            const int32_t* idx, double* o64, uint16_t* o16, int nthreads) {
  dims_t D = {B, Hq, Hkv, d, KW, 0, scale, cu, 0, 0.0, KW};
  if (!q_dec || !k || !v || !cu || !idx || check_dims(&D) || KW < 1) return -1;
  for (int b = 0; b < B; b++)
    if (cu[b + 1] - cu[b] < 1) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.D = &D; J.q = q_dec; J.k = k; J.v = v; J.n_rows = B; J.decode = 1;
  J.idx_in = idx; J.o64 = o64; J.o16 = o16;
  return run(&J, sparse_worker, nthreads);
}

/*
 * The full layer's own attention output (dense causal softmax attention over
 * [0, t] with the full layer's queries; SHARP walkthrough, section 1.1):
 * o[t,h] = sum_{j <= t} softmax_j(scale <q[t,h], k[j,g]>) v[j,g]. tokens: global
 * token ids or NULL for all T; o64 / o16 [n, Hq, d] (nullable).
 */
static void* full_worker(void* arg) {
  job_t* J = (job_t*)arg;
  const dims_t* D = J->D;
  const int G = D->Hq / D->Hkv, d = D->d;
  double* y = (double*)malloc(sizeof(double) * (size_t)J->max_len);
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  double qd[1024];
  for (;;) {
    int64_t e, s = take(J, 4, &e);
    if (s >= J->n_rows) break;
    for (int64_t r = s; r < e; r++) {
      int64_t tg = J->rows ? J->rows[r] : r;
      int i = find_seq(D, tg);
      int64_t base = D->cu[i], t = tg - base;
      for (int h = 0; h < D->Hq; h++) {
        const int g = h / G;
        const uint16_t* qr = J->q + ((size_t)tg * D->Hq + h) * d;
        for (int c = 0; c < d; c++) qd[c] = bf2d(qr[c]);
        double mu = -INFINITY;
        for (int64_t j = 0; j <= t; j++) {
          const uint16_t* kr = J->k + ((size_t)(base + j) * D->Hkv + g) * d;
          double dot = 0.0;
          for (int c = 0; c < d; c++) dot += qd[c] * bf2d(kr[c]);
          y[j] = D->scale * dot;
          if (y[j] > mu) mu = y[j];
        }
        double den = 0.0;
        for (int c = 0; c < d; c++) acc[c] = 0.0;
        for (int64_t j = 0; j <= t; j++) {
          double w = exp(y[j] - mu);
          den += w;
          const uint16_t* vr = J->v + ((size_t)(base + j) * D->Hkv + g) * d;
          for (int c = 0; c < d; c++) acc[c] += w * bf2d(vr[c]);
        }
        size_t o = ((size_t)r * D->Hq + h) * d;
        for (int c = 0; c < d; c++) {
          double val = acc[c] / den;
          if (J->o64) J->o64[o + c] = val;
          if (J->o16) J->o16[o + c] = d2bf(val);
        }
      }
    }
  }
  free(y); free(acc);
  return NULL;
}

int hs2o_full_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* cu,
                   int B, int Hq, int Hkv, int d, double scale, const int64_t* tokens,
                   int64_t n_tokens, double* o64, uint16_t* o16, int nthreads) {
  dims_t D = {B, Hq, Hkv, d, 1, 0, scale, cu, 0, 0.0, 1};
  if (!q || !k || !v || !cu || check_dims(&D)) return -1;
  int64_t T = cu[B];
  if (!tokens) n_tokens = T;
  for (int64_t r = 0; tokens && r < n_tokens; r++)
    if (tokens[r] < 0 || tokens[r] >= T) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.D = &D; J.q = q; J.k = k; J.v = v; J.rows = tokens; J.n_rows = n_tokens;
  J.o64 = o64; J.o16 = o16; J.max_len = max_len(&D);
  return run(&J, full_worker, nthreads);
}

/* double -> bf16 RNE, exported for tests of the rounding itself. */
uint16_t hs2o_bf16_round(double x) { return d2bf(x); }

/* E4M3 code <-> value, exported for tests of the encoding itself. */
double hs2o_fp8_value(uint8_t code) { return e4m3_to_d(code); }
uint8_t hs2o_fp8_encode(float x) { return f_to_e4m3(x); }

/* Writing the FP8 cache: dst[i] = E4M3(float(src[i]) * inv_scale), the product
 * rounded to float first, then to the nearest code (saturating at +-448). */
int hs2o_quantize_fp8(const uint16_t* src, uint8_t* dst, int64_t n, float inv_scale) {
  if (n < 0 || (n > 0 && (!src || !dst))) return -1;
  for (int64_t i = 0; i < n; i++) {
    const float v = (float)bf2d(src[i]) * inv_scale;
    dst[i] = f_to_e4m3(v);
  }
  return 0;
}

/* Sparse attention (O7) over an FP8 KV cache: as hs2o_sparse_attn with
 * k = k_scale * E4M3(k8), v = v_scale * E4M3(v8). */
int hs2o_sparse_attn_fp8(const uint16_t* q, const uint8_t* k8, const uint8_t* v8, double k_scale,
                         double v_scale, const int32_t* cu, int B, int Hq, int Hkv, int d,
                         double scale, int KW, const int32_t* idx, const int64_t* tokens,
                         int64_t n_tokens, double* o64, uint16_t* o16, int nthreads) {
  dims_t D = {B, Hq, Hkv, d, KW, 0, scale, cu, 0, 0.0, KW};
  if (!q || !k8 || !v8 || !cu || !idx || check_dims(&D) || KW < 1) return -1;
  int64_t T = cu[B];
  if (!tokens) n_tokens = T;
  for (int64_t r = 0; tokens && r < n_tokens; r++)
    if (tokens[r] < 0 || tokens[r] >= T) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.D = &D; J.q = q; J.k8 = k8; J.v8 = v8; J.k_scale = k_scale; J.v_scale = v_scale;
  J.rows = tokens; J.n_rows = n_tokens; J.idx_in = idx; J.o64 = o64; J.o16 = o16;
  return run(&J, sparse_worker, nthreads);
}

/* Decode-step sparse attention over an FP8 KV cache (as hs2o_decode_sparse_attn). */
int hs2o_decode_sparse_attn_fp8(const uint16_t* q_dec, const uint8_t* k8, const uint8_t* v8,
                                double k_scale, double v_scale, const int32_t* cu, int B, int Hq,
                                int Hkv, int d, double scale, int KW, const int32_t* idx,
                                double* o64, uint16_t* o16, int nthreads) {
  dims_t D = {B, Hq, Hkv, d, KW, 0, scale, cu, 0, 0.0, KW};
  if (!q_dec || !k8 || !v8 || !cu || !idx || check_dims(&D) || KW < 1) return -1;
  for (int b = 0; b < B; b++)
    if (cu[b + 1] - cu[b] < 1) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.D = &D; J.q = q_dec; J.k8 = k8; J.v8 = v8; J.k_scale = k_scale; J.v_scale = v_scale;
  J.n_rows = B; J.decode = 1; J.idx_in = idx; J.o64 = o64; J.o16 = o16;
  return run(&J, sparse_worker, nthreads);
}
