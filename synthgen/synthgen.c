/*
 * synthgen.c - seeded synthetic inputs for token-level sparse attention prefill.
 *
 * This module holds none of the attention method's arithmetic. It only makes
 * the input bytes (bf16 Q/K/V, needle keys, varlen lengths) that both the CPU
 * oracle and the GPU library consume, so that the two sides see identical data.
 *
 * Random numbers:
 *   SplitMix64 (S. Vigna, "Further scramblings of Marsaglia's xorshift
 *   generators", and the public-domain splitmix64.c) used as a counter-based
 *   generator: output c of stream `key` is mix64(key + GAMMA * (c + 1)).
 *   Normals by the Box-Muller transform (Box & Muller, 1958): from two
 *   uniforms u1 in (0,1], u2 in [0,1): r = sqrt(-2 ln u1), n0 = r cos(2 pi u2),
 *   n1 = r sin(2 pi u2). Element 2p of a tensor takes n0 of pair p, 2p+1 n1.
 *   Values are rounded double -> bf16 with round-to-nearest-even, directly
 *   (no intermediate float, so no double rounding).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SG_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sg_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Stream key for (seed, tensor id). */
uint64_t sg_stream_key(uint64_t seed, uint64_t tensor_id) {
  return sg_mix64(sg_mix64(seed + SG_GAMMA) ^ (tensor_id * 0xD1B54A32D192ED03ULL + 1ULL));
}

/* Counter-based SplitMix64 output number c of a stream. */
uint64_t sg_u64(uint64_t key, uint64_t c) { return sg_mix64(key + SG_GAMMA * (c + 1ULL)); }

static inline void sg_pair(uint64_t key, uint64_t p, double* n0, double* n1) {
  uint64_t a = sg_u64(key, 2 * p), b = sg_u64(key, 2 * p + 1);
  double u1 = (double)((a >> 11) + 1ULL) * (1.0 / 9007199254740992.0); /* (0,1] */
  double u2 = (double)(b >> 11) * (1.0 / 9007199254740992.0);          /* [0,1) */
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  *n0 = r * cos(th);
  *n1 = r * sin(th);
}

/* double -> bf16 bits, round to nearest even, computed from the double's bits. */
uint16_t sg_bf16_from_double(double x) {
  uint64_t bits;
  memcpy(&bits, &x, 8);
  uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
  int exp = (int)((bits >> 52) & 0x7FF);
  uint64_t mant = bits & 0xFFFFFFFFFFFFFULL;
  if (exp == 0x7FF) return (uint16_t)(sign | 0x7F80u | (mant ? 0x40u : 0u)); /* inf / nan */
  int e = exp - 1023; /* unbiased */
  if (exp == 0 || e < -133) return sign; /* far below the bf16 subnormal range */
  if (e < -126) {
    /* bf16 subnormal: value = m * 2^-133, m in [0,127]. Round |x| * 2^133. */
    double ax = fabs(x) * 1.0889035741470030830827987437817e40; /* 2^133 */
    double fl = floor(ax);
    double rem = ax - fl;
    uint32_t m = (uint32_t)fl;
    if (rem > 0.5 || (rem == 0.5 && (m & 1u))) m++;
    return (uint16_t)(sign | m); /* m == 128 becomes the smallest normal */
  }
  /* normal: keep 7 mantissa bits, round at bit 45 */
  uint64_t keep = mant >> 45;
  uint64_t rem = mant & ((1ULL << 45) - 1);
  uint64_t half = 1ULL << 44;
  uint32_t be = (uint32_t)(e + 127);
  uint32_t v = (be << 7) | (uint32_t)keep;
  if (rem > half || (rem == half && (keep & 1ULL))) v++; /* carries into exponent */
  if (v >= 0x7F80u) return (uint16_t)(sign | 0x7F80u);   /* overflow to inf */
  return (uint16_t)(sign | v);
}

typedef struct {
  uint64_t key, start, n;
  uint16_t* out16;
  double* out64;
} sg_job;

static void sg_fill_range(uint64_t key, uint64_t start, uint64_t n, uint16_t* o16, double* o64) {
  uint64_t e = start, end = start + n;
  while (e < end) {
    double n0, n1;
    uint64_t p = e >> 1;
    sg_pair(key, p, &n0, &n1);
    if ((e & 1ULL) == 0) {
      if (o16) o16[e - start] = sg_bf16_from_double(n0);
      if (o64) o64[e - start] = n0;
      e++;
      if (e >= end) break;
    }
    if (o16) o16[e - start] = sg_bf16_from_double(n1);
    if (o64) o64[e - start] = n1;
    e++;
  }
}

static void* sg_worker(void* arg) {
  sg_job* j = (sg_job*)arg;
  sg_fill_range(j->key, j->start, j->n, j->out16, j->out64);
  return NULL;
}

static void sg_fill(uint64_t seed, uint64_t tensor_id, uint64_t start, uint64_t n, uint16_t* o16,
                    double* o64, int nthreads) {
  uint64_t key = sg_stream_key(seed, tensor_id);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (n < 65536 || nthreads == 1) {
    sg_fill_range(key, start, n, o16, o64);
    return;
  }
  pthread_t th[256];
  sg_job jobs[256];
  uint64_t per = (n + nthreads - 1) / nthreads;
  int launched = 0;
  for (int i = 0; i < nthreads; i++) {
    uint64_t s = (uint64_t)i * per;
    if (s >= n) break;
    uint64_t m = (n - s < per) ? n - s : per;
    jobs[i].key = key;
    jobs[i].start = start + s;
    jobs[i].n = m;
    jobs[i].out16 = o16 ? o16 + s : NULL;
    jobs[i].out64 = o64 ? o64 + s : NULL;
    if (pthread_create(&th[i], NULL, sg_worker, &jobs[i]) != 0) {
      sg_worker(&jobs[i]);
      th[i] = 0;
    }
    launched = i + 1;
  }
  for (int i = 0; i < launched; i++)
    if (th[i]) pthread_join(th[i], NULL);
}

/* Elements [start, start+n) of the N(0,1) stream (seed, tensor_id), as bf16 bits. */
void sg_normal_bf16(uint64_t seed, uint64_t tensor_id, uint64_t start, uint64_t n, uint16_t* out,
                    int nthreads) {
  sg_fill(seed, tensor_id, start, n, out, NULL, nthreads);
}

/* Same stream as doubles (unrounded). */
void sg_normal_f64(uint64_t seed, uint64_t tensor_id, uint64_t start, uint64_t n, double* out,
                   int nthreads) {
  sg_fill(seed, tensor_id, start, n, NULL, out, nthreads);
}

static inline double sg_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/*
 * Needle keys for one sequence of length L (bf16 q [L, Hq, d], k [L, Hkv, d],
 * k modified in place). For each KV group g and each query block b >= 1 of
 * `block` tokens: u = unit(sum over tokens of block b and heads of group g of
 * q); pick `per_block` distinct key positions uniformly from [0, block*b - W)
 * not used before as needles of group g; set k[j, g] = bf16(mag * u + eps),
 * eps ~ N(0, I_d) from stream (seed, eps_tid). Positions come from stream
 * (seed, pos_tid). Groups are contiguous: head h belongs to group h / (Hq/Hkv).
 * Returns the number of needles written, or -1 on bad arguments.
 */
int64_t sg_add_needles(const uint16_t* q, uint16_t* k, int64_t L, int Hq, int Hkv, int d, int block,
                       int per_block, int W, double mag, uint64_t seed, uint64_t pos_tid,
                       uint64_t eps_tid, int32_t* needle_pos_out /* nullable [Hkv*nblk*per_block] */) {
  if (!q || !k || L <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || block <= 0 || per_block < 0)
    return -1;
  int G = Hq / Hkv;
  int64_t nblk = (L + block - 1) / block;
  uint8_t* used = (uint8_t*)calloc((size_t)L, 1);
  double* u = (double*)malloc(sizeof(double) * (size_t)d);
  double* eps = (double*)malloc(sizeof(double) * (size_t)d);
  if (!used || !u || !eps) {
    free(used); free(u); free(eps);
    return -1;
  }
  uint64_t pkey = sg_stream_key(seed, pos_tid);
  uint64_t pctr = 0;
  int64_t written = 0, slot = 0;
  for (int g = 0; g < Hkv; g++) {
    memset(used, 0, (size_t)L);
    for (int64_t b = 1; b < nblk; b++) {
      int64_t t_lo = b * block, t_hi = (b + 1) * block < L ? (b + 1) * block : L;
      for (int e = 0; e < d; e++) u[e] = 0.0;
      for (int64_t t = t_lo; t < t_hi; t++)
        for (int hh = 0; hh < G; hh++) {
          const uint16_t* qr = q + ((size_t)t * Hq + (size_t)g * G + hh) * d;
          for (int e = 0; e < d; e++) u[e] += sg_bf16_to_double(qr[e]);
        }
      double nrm = 0.0;
      for (int e = 0; e < d; e++) nrm += u[e] * u[e];
      nrm = sqrt(nrm);
      int64_t range = b * block - W;
      if (nrm == 0.0 || range <= 0) {
        if (needle_pos_out)
          for (int n = 0; n < per_block; n++) needle_pos_out[slot + n] = -1;
        slot += per_block;
        continue;
      }
      int64_t free_left = 0;
      for (int64_t j = 0; j < range; j++) free_left += used[j] ? 0 : 1;
      int want = per_block < free_left ? per_block : (int)free_left;
      for (int n = 0; n < want; n++) {
        int64_t j;
        do {
          uint64_t r = sg_u64(pkey, pctr++);
          j = (int64_t)(((unsigned __int128)r * (unsigned __int128)range) >> 64);
        } while (used[j]);
        used[j] = 1;
        sg_normal_f64(seed, eps_tid, ((uint64_t)g * (uint64_t)L + (uint64_t)j) * (uint64_t)d,
                      (uint64_t)d, eps, 1);
        uint16_t* kr = k + ((size_t)j * Hkv + g) * d;
        for (int e = 0; e < d; e++) kr[e] = sg_bf16_from_double(mag * u[e] / nrm + eps[e]);
        if (needle_pos_out) needle_pos_out[slot + n] = (int32_t)j;
        written++;
      }
      if (needle_pos_out)
        for (int n = want; n < per_block; n++) needle_pos_out[slot + n] = -1;
      slot += per_block;
    }
  }
  free(used); free(u); free(eps);
  return written;
}
