// select_topk.hip - exact top-K of each (t, g) row and index assembly on gfx950.
//
// Selection rule (HySparse2 news summary, token-granularity paragraph: single
// tokens, not 64-token blocks; forced-recent paragraph: the W most recent
// tokens are always in): among the candidates C_t = [0, t-W] keep the K with
// the largest group score S, ties to the lower position; then
//   I_t = ascending(T_t U [t-W+1, t]), padded with -1 to K+W.
//
// topk_kernel: one wavefront per row of a chunk. Its candidates (S >= tau,
//   collected by the scoring sweep) sit in registers and are ranked by a radix
//   select on the fp32 bit pattern of S (monotone for S >= 0), starting below
//   the bits all candidates share, 8 bits per pass; it yields the K-th largest
//   value and how many of the values equal to it to take (lowest positions
//   first). Selected positions go into an LDS bitmap, so the compaction into
//   the index row comes out in ascending order.
// exact_kernel: persistent workgroups over the rows the sweep could not settle
//   (too many / too few candidates, or the exact flag). S of the whole row comes
//   from the dense rows the scoring kernel wrote (exact flag, or K above the
//   register-ranked limit) or is recomputed into a scratch row; then a workgroup
//   radix select and the same assembly run.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

struct TopkShared {
  uint32_t* hist;   // [kTopkBins]
  int32_t* misc;    // [16]
  uint32_t* sel;    // [bitmap_words]
  uint32_t* tie;    // [bitmap_words]
  uint32_t* keys;   // [cand_cap] (candidate path only)
  float* qf;        // [16 * 128] (exact path only)
};

// Exclusive prefix sum over the 256 threads; *total gets the sum. Uses misc[8..11].
__device__ int block_excl_scan(int v, int32_t* misc, int* total) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  int x = wave_incl_scan(v, l);
  if (l == 63) misc[8 + w] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int s = misc[8 + i];
    if (i < w) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// The digit passes of radix_kth for keys that all share the bits in mask (equal to
// prefix); hi is the highest bit below them.
template <class KeyFn>
__device__ uint32_t radix_digits(KeyFn key, int n, int k, const TopkShared& sh, int* krem, int hi,
                                 uint32_t mask, uint32_t prefix, int max_passes = 3) {
  const int tid = threadIdx.x;
  int kr = k;
  constexpr int kPer = kTopkBins / kSelThreads;  // bins per thread in the scan
  for (int pass = 0; hi >= 0 && pass < max_passes; pass++) {
    const int lo = max(0, hi - 10);
    const int nb = hi - lo + 1;
    const uint32_t dmask = (1u << nb) - 1u;
    for (int i = tid; i < kTopkBins; i += kSelThreads) sh.hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
      const uint32_t b = key(i);
      if ((b & mask) == prefix) atomicAdd(&sh.hist[(b >> lo) & dmask], 1u);
    }
    __syncthreads();
    // suffix counts over bins: thread tid owns bins [kPer*tid, kPer*tid + kPer)
    uint32_t h[kPer];
    int local = 0;
#pragma unroll
    for (int u = 0; u < kPer; u++) {
      h[u] = sh.hist[kPer * tid + u];
      local += (int)h[u];
    }
    int total;
    const int excl = block_excl_scan(local, sh.misc, &total);
    const int above = total - excl - local;  // elements in bins above this thread's
    if (above < kr && kr <= above + local) {
      int a = above, d = kPer * tid;
#pragma unroll
      for (int u = kPer - 1; u >= 0; u--) {
        if (a + (int)h[u] >= kr) { d = kPer * tid + u; break; }
        a += (int)h[u];
      }
      sh.misc[0] = d;
      sh.misc[1] = a;
    }
    __syncthreads();
    const uint32_t d = (uint32_t)sh.misc[0];
    kr -= sh.misc[1];
    prefix |= d << lo;
    mask |= dmask << lo;
    hi = lo - 1;
    __syncthreads();
  }
  *krem = kr;
  return prefix;
}

// K-th largest key among key(i), i < n (1 <= k <= n). Returns the key and, in
// *krem, how many elements equal to it belong to the top k. Radix select on the
// bits below the keys' common prefix, up to 11 bits (2048 bins) per pass. With
// max_passes, it stops early and returns the lower edge of the bin that holds the
// K-th largest key (at least k keys reach it; *krem is then meaningless).
template <class KeyFn>
__device__ uint32_t radix_kth(KeyFn key, int n, int k, const TopkShared& sh, int* krem,
                              int max_passes = 3) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = tid; i < n; i += kSelThreads) {
    const uint32_t b = key(i);
    mn = min(mn, b);
    mx = max(mx, b);
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (l == 0) {
    sh.misc[4 + w] = (int)mn;
    sh.misc[8 + w] = (int)mx;
  }
  __syncthreads();
  mn = (uint32_t)sh.misc[4];
  mx = (uint32_t)sh.misc[8];
#pragma unroll
  for (int i = 1; i < 4; i++) {
    mn = min(mn, (uint32_t)sh.misc[4 + i]);
    mx = max(mx, (uint32_t)sh.misc[8 + i]);
  }
  __syncthreads();
  if (mn == mx) {
    *krem = k;
    return mn;
  }
  const int hi = 31 - __clz(mn ^ mx);  // highest bit where the keys differ
  const uint32_t mask = (hi == 31) ? 0u : ~((2u << hi) - 1u);
  return radix_digits(key, n, k, sh, krem, hi, mask, mx & mask, max_passes);
}

// Marks in sh.sel every position whose key is above kth, plus the krem lowest
// positions whose key equals kth.
template <class KeyFn, class PosFn>
__device__ void mark_selected(KeyFn key, PosFn pos, int n, uint32_t kth, int krem, int nwords,
                              const TopkShared& sh, bool keep_sel = false) {
  const int tid = threadIdx.x;
  for (int i = tid; i < nwords; i += kSelThreads) {
    if (!keep_sel) sh.sel[i] = 0u;
    sh.tie[i] = 0u;
  }
  if (tid == 0) sh.misc[2] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kSelThreads) {
    const uint32_t b = key(i);
    if (b >= kth) {
      const uint32_t p = pos(i);
      if (b > kth) {
        atomicOr(&sh.sel[p >> 5], 1u << (p & 31));
      } else {
        atomicOr(&sh.tie[p >> 5], 1u << (p & 31));
        atomicAdd(&sh.misc[2], 1);
      }
    }
  }
  __syncthreads();
  const int n_eq = sh.misc[2];
  const int per = ceil_div(nwords, kSelThreads);
  const int w0 = min(tid * per, nwords), w1 = min(w0 + per, nwords);
  if (n_eq == krem) {
    for (int i = w0; i < w1; i++) sh.sel[i] |= sh.tie[i];
  } else {
    int cnt = 0;
    for (int i = w0; i < w1; i++) cnt += __popc(sh.tie[i]);
    int total;
    int off = block_excl_scan(cnt, sh.misc, &total);
    for (int i = w0; i < w1 && off < krem; i++) {
      uint32_t m = sh.tie[i];
      while (m && off < krem) {
        const uint32_t bit = m & (0u - m);
        sh.sel[i] |= bit;
        m ^= bit;
        off++;
      }
    }
  }
  __syncthreads();
}

// Writes the index row: the selected positions (ascending, from sh.sel), then
// the window [n_c, t], then -1 up to K + W (a decaying budget leaves room).
__device__ void write_selected_row(int nwords, int n_c, int t, int KW, int32_t* row,
                                   const TopkShared& sh) {
  const int tid = threadIdx.x;
  const int per = ceil_div(nwords, kSelThreads);
  const int w0 = min(tid * per, nwords), w1 = min(w0 + per, nwords);
  int cnt = 0;
  for (int i = w0; i < w1; i++) cnt += __popc(sh.sel[i]);
  int total;
  int off = block_excl_scan(cnt, sh.misc, &total);
  for (int i = w0; i < w1; i++) {
    uint32_t m = sh.sel[i];
    while (m) {
      const int b = __ffs(m) - 1;
      m &= m - 1;
      if (off < KW) row[off] = i * 32 + b;
      off++;
    }
  }
  for (int j = n_c + tid; j <= t; j += kSelThreads) {
    const int o = total + (j - n_c);
    if (o < KW) row[o] = j;
  }
  for (int o = total + (t - n_c + 1) + tid; o < KW; o += kSelThreads) row[o] = -1;
}

// Rows needing no ranking: all candidates fit (n_c <= K) -> [0, t];
// K == 0 -> the window only. Pads with -1.
__device__ void write_trivial_row(int n_c, int K, int t, int KW, int32_t* row) {
  const int start = (n_c <= K) ? 0 : n_c;
  const int n = t - start + 1;
  for (int o = threadIdx.x; o < KW; o += kSelThreads) row[o] = (o < n) ? start + o : -1;
}

struct RowInfo {
  int seq, base, L, t, g;
};

__device__ __forceinline__ RowInfo decode_slot(const TopkParams& p, int64_t slot) {
  RowInfo r;
  const int64_t blk = slot / p.tok;
  const int tl = (int)(slot % p.tok);
  r.g = (int)(blk % p.Hkv);
  int seq, tile;
  plan_decode(p.cu, p.B, p.tok, p.max_tiles, p.task_begin + blk / p.Hkv, &seq, &tile);
  r.seq = seq;
  r.base = p.cu[seq];
  r.L = p.cu[seq + 1] - r.base;
  r.t = tile * p.tok + tl;
  return r;
}

__device__ __forceinline__ TopkShared carve_lds(uint32_t* smem, const TopkParams& p, bool exact) {
  TopkShared sh;
  sh.hist = smem;
  sh.misc = reinterpret_cast<int32_t*>(smem + kTopkBins);
  sh.sel = smem + kTopkBins + 16;
  sh.tie = sh.sel + p.bitmap_words;
  sh.keys = sh.tie + p.bitmap_words;
  sh.qf = reinterpret_cast<float*>(sh.keys);
  (void)exact;
  return sh;
}

// ---------------------------------------------------------------------------
// Candidate path: one wavefront per row, no workgroup barriers. The row's
// candidates (at most 64 * NREG) sit in registers: lane l holds entries l + 64 s.
// LDS per wave: a 256-bin histogram and a bitmap of the row's candidate range.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
  return v;
}

// A wave-uniform value the compiler has to take as new at each call: the register
// loops below compare their index against their own copy of the row's register
// count, so those comparisons are made at each branch instead of being hoisted and
// kept live in SGPR pairs across the kernel.
__device__ __forceinline__ int fresh_uniform(int x) {
  asm volatile("" : "+s"(x));
  return x;
}

template <int NREG>
__global__ __launch_bounds__(256) void topk_kernel(TopkParams p) {
  extern __shared__ uint32_t smem[];
  // the wave index is wave-uniform, so everything derived from it stays in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int wshift = (blockDim.x >> 6) >> 1;  // log2 of the waves per block: 1, 2 or 4 waves
  uint32_t* hist = smem + (size_t)w * (256 + p.bitmap_words + p.sbuf_words);
  uint32_t* bm = hist + 256;
  // grid (chunk tasks * tok / waves, Hkv): block x holds `waves` consecutive tokens of
  // one task, block y is the KV group; rows are numbered as the scores kernel wrote them
  const int sub_shift = p.tok_shift - wshift;
  const int tq = blockIdx.x >> sub_shift;
  const int tl = ((blockIdx.x & ((1 << sub_shift) - 1)) << wshift) + w;
  const int64_t slot = (((int64_t)tq * p.Hkv + blockIdx.y) << p.tok_shift) + tl;
  if (slot >= p.n_rows) return;
  const int2 tm = p.task_map[tq];
  RowInfo r;
  r.seq = tm.x;
  r.base = p.cu[tm.x];
  r.L = p.cu[tm.x + 1] - r.base;
  r.t = tm.y * p.tok + tl;
  r.g = blockIdx.y;
  if (r.t >= r.L) return;
  const int KW = p.K + p.W;
  const int n_c = r.t - p.W + 1;
  const int Kt = row_budget(p.K, p.k_end, r.t, r.L);  // this row's budget
  int32_t* row = p.idx + ((size_t)(r.base + r.t) * p.Hkv + r.g) * KW;
  float* kth_out = p.kth ? p.kth + (size_t)(r.base + r.t) * p.Hkv + r.g : nullptr;
  if (Kt == 0 || n_c <= Kt) {  // nothing to rank: [0, t] or the window only
    const int start = (n_c <= Kt) ? 0 : n_c;
    const int n = r.t - start + 1;
    for (int o = l; o < KW; o += 64) row[o] = (o < n) ? start + o : -1;
    if (kth_out && l == 0) *kth_out = -1.f;
    return;
  }
  const int count = p.cand_count[slot];
  if (count < 0 || p.list_rank) return;  // settled by exact_kernel
  const uint64_t* cand = p.cand + (size_t)slot * p.cand_cap;
  uint32_t key[NREG], pos[NREG];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  // every load of the row is issued before the first use (a use right after each
  // load would wait out one memory latency per load); the guard is wave-uniform
  const int count_u = __builtin_amdgcn_readfirstlane(count);
  const int nreg = (count_u + 63) >> 6;  // registers that hold candidates (wave-uniform)
  uint64_t ev[NREG];
#pragma unroll
  for (int s = 0; s < NREG; s++) {
    ev[s] = 0u;
    if (64 * s < count_u) ev[s] = cand[min(l + 64 * s, p.cand_cap - 1)];
  }
  // a slot past the row's count holds the key kNoKey, which matches no prefix of a
  // valid key (scores are >= 0, so their bit 31 is clear) and equals none of them
  constexpr uint32_t kNoKey = 0xFFFFFFFFu;
#pragma unroll
  for (int s = 0; s < NREG; s++) {
    const bool in = l + 64 * s < count_u;
    key[s] = in ? (uint32_t)(ev[s] >> 32) : kNoKey;
    pos[s] = in ? (uint32_t)ev[s] : 0u;
    if (in) {
      mn = min(mn, key[s]);
      mx = max(mx, key[s]);
    }
  }
  mn = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_min_u32(mn));
  mx = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_max_u32(mx));
  // radix select of the K-th largest key below the common prefix, 8 bits per pass
  // (block mode: the (K / 64)-th largest block score). The loops over the lane's
  // registers stop at the row's count (wave-uniform), and the passes stop once the
  // bin holding the K-th key is taken whole: then the K-th key is that bin's smallest
  // and every key equal to it is taken.
  const int k_sel = p.block ? p.K / p.block : Kt;
  uint32_t prefix = mx, mask = 0xFFFFFFFFu;
  int kr = k_sel;
  bool all_ties = false;
  if (mn != mx) {
    int hi = 31 - __clz(mn ^ mx);
    mask = (hi == 31) ? 0u : ~((2u << hi) - 1u);
    prefix = mx & mask;
    while (hi >= 0) {
      const int lo = max(0, hi - 7);
      const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
#pragma unroll
      for (int u = 0; u < 4; u++) hist[l + 64 * u] = 0u;
      wave_lds_fence();
      const int nr = fresh_uniform(nreg);
#pragma unroll
      for (int s = 0; s < NREG; s++) {
        if (s < nr)  // keys outside the prefix (sentinels included) add zero
          atomicAdd(&hist[(key[s] >> lo) & dmask], (key[s] & mask) == prefix ? 1u : 0u);
      }
      wave_lds_fence();
      // lane l owns bins 4l .. 4l+3; inclusive suffix sums over lanes
      uint32_t h[4];
#pragma unroll
      for (int u = 0; u < 4; u++) h[u] = hist[4 * l + u];
      const uint32_t local = h[0] + h[1] + h[2] + h[3];
      const uint32_t incl = (uint32_t)wave_incl_scan((int)local, l);
      const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      const uint32_t suf = total - incl + local;  // this lane's bins and all above
      const uint32_t above = suf - local;
      const bool mine = above < (uint32_t)kr && (uint32_t)kr <= suf;
      int d = 0;
      uint32_t a = above, hd = 0;
      if (mine) {
        if (a + h[3] >= (uint32_t)kr) { d = 4 * l + 3; hd = h[3]; }
        else if ((a += h[3]) + h[2] >= (uint32_t)kr) { d = 4 * l + 2; hd = h[2]; }
        else if ((a += h[2]) + h[1] >= (uint32_t)kr) { d = 4 * l + 1; hd = h[1]; }
        else { a += h[1]; d = 4 * l; hd = h[0]; }
      }
      // the bin, the count above it and its size, from the lane that holds it (wave-uniform)
      const int src = max(0, __ffsll((unsigned long long)__ballot(mine)) - 1);
      d = __builtin_amdgcn_readlane(d, src);
      a = (uint32_t)__builtin_amdgcn_readlane((int)a, src);
      hd = (uint32_t)__builtin_amdgcn_readlane((int)hd, src);
      kr -= (int)a;
      prefix |= (uint32_t)d << lo;
      mask |= dmask << lo;
      hi = lo - 1;
      wave_lds_fence();
      if (hi >= 0 && hd == (uint32_t)kr) {  // the whole bin is taken: its smallest key
        uint32_t m = 0xFFFFFFFFu;
        const int nr = fresh_uniform(nreg);
#pragma unroll
        for (int s = 0; s < NREG; s++) {
          if (s < nr && (key[s] & mask) == prefix) m = min(m, key[s]);
        }
        prefix = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_min_u32(m));
        all_ties = true;
        break;
      }
    }
  }
  const uint32_t kth = prefix;  // K-th largest key; kr of the keys equal to it are taken
  // ties at the boundary: take the kr lowest positions (binary search on position)
  uint32_t n_eq = 0;
  {
    const int nr = fresh_uniform(nreg);
#pragma unroll
    for (int s = 0; s < NREG; s++) {
      if (s < nr) n_eq += (key[s] == kth) ? 1u : 0u;
    }
  }
  n_eq = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_sum_u32(n_eq));
  if (all_ties) kr = (int)n_eq;  // the bin was taken whole: every key equal to its minimum
  uint32_t pos_cut = 0xFFFFFFFFu;  // ties with pos <= pos_cut are taken
  if (n_eq != (uint32_t)kr) {
    // smallest cut with >= kr ties at or below it (positions, or block indices)
    uint32_t lo = 0, hi = (uint32_t)(p.block ? count : n_c) - 1;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      uint32_t c = 0;
      const int nr = fresh_uniform(nreg);
#pragma unroll
      for (int s = 0; s < NREG; s++) {
        if (s < nr) c += (key[s] == kth && pos[s] <= mid) ? 1u : 0u;
      }
      c = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_sum_u32(c));
      if (c >= (uint32_t)kr) hi = mid; else lo = mid + 1;
    }
    pos_cut = lo;
  }
  // bitmap of the selected positions, then ascending compaction
  const int nwords = ceil_div(n_c, 32);
  for (int i = l; i < nwords; i += 64) bm[i] = 0u;
  wave_lds_fence();
  if (p.block) {  // the block's candidate tokens [64 b, min(64 b + 64, n_c)): its own two words
    const int nr = fresh_uniform(nreg);
#pragma unroll
    for (int s = 0; s < NREG; s++) {
      if (s < nr && key[s] != kNoKey &&
          (key[s] > kth || (key[s] == kth && pos[s] <= pos_cut))) {
        const int j0 = p.block * (int)pos[s], j1 = min(j0 + p.block, n_c);
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int nbits = min(max(j1 - (j0 + 32 * h), 0), 32);
          if (nbits > 0) bm[(j0 >> 5) + h] = nbits == 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u);
        }
      }
    }
  } else {  // a slot not taken ORs a zero word (sentinel slots hold position 0)
    const int nr = fresh_uniform(nreg);
#pragma unroll
    for (int s = 0; s < NREG; s++) {
      if (s < nr) {
        const bool take =
            key[s] != kNoKey && (key[s] > kth || (key[s] == kth && pos[s] <= pos_cut));
        atomicOr(&bm[pos[s] >> 5], take ? 1u << (pos[s] & 31) : 0u);
      }
    }
  }
  wave_lds_fence();
  // Ascending compaction, 64 consecutive words per step (lane l reads word c + l, so
  // the LDS reads do not conflict): a wave scan of the words' popcounts gives each
  // lane its first output slot, then the lanes emit their positions in as many rounds
  // as the fullest word has bits. The positions go to the wave's LDS staging and leave
  // in coalesced stores. Plain selection takes Kt positions, block selection at most K.
  uint32_t* sbuf = bm + p.bitmap_words;
  const int sbw = p.sbuf_words;
  const bool stage = (p.block ? p.K : Kt) <= sbw;  // wave-uniform
  int base = 0;  // positions emitted so far (wave-uniform)
  for (int c = 0; c < nwords; c += 64) {
    const int i = c + l;
    uint32_t mm = i < nwords ? bm[i] : 0u;
    const int cnt = __popc(mm);
    const int incl = wave_incl_scan(cnt, l);
    int off = base + incl - cnt;
    base += __builtin_amdgcn_readlane(incl, 63);
    const int rounds = __builtin_amdgcn_readlane(wave_incl_max(cnt), 63);
    for (int it = 0; it < rounds; it++) {
      const bool has = mm != 0u;
      const uint32_t v = (uint32_t)(i * 32 + __ffs(mm) - 1);
      mm &= mm - 1u;
      if (stage) {  // a lane without a bit left writes the dead histogram instead
        *((has && off < sbw) ? sbuf + off : hist + l) = v;
      } else if (has && off < KW) {
        row[off] = (int32_t)v;
      }
      off += has ? 1 : 0;
    }
  }
  if (stage) {
    wave_lds_fence();
    const int n = min(base, sbw);
    for (int o = l; o < n; o += 64) row[o] = (int32_t)sbuf[o];
  }
  for (int j = n_c + l; j <= r.t; j += 64) {
    const int o = base + (j - n_c);
    if (o < KW) row[o] = j;
  }
  for (int o = base + (r.t - n_c + 1) + l; o < KW; o += 64) row[o] = -1;
  if (kth_out && l == 0) *kth_out = __uint_as_float(kth);
}

// The exact path's ranking of one row of (position, score) entries (a dense row, or a
// candidate list) in two passes over it: a histogram of
// the top bits of S (S >= 0, so bits 30..20: exponent and 3 mantissa bits) gives
// the bin d1 holding the kt-th largest value and how many lie above it; the second
// pass marks every value above d1 as selected and copies the values of d1, with their
// positions, into an LDS list, where the radix select finishes and the ties take the
// lowest positions. Returns false (nothing changed but the histogram) when kt is
// outside (0, n), or d1 holds more than kExactListCap values: then the whole-row
// radix select runs instead. On true, sh.sel holds the kt selected positions.
// fn(i, row[i]) for every i < n, spread over the workgroup; the body reads the row
// 16 bytes per lane with kSweepLoads loads in flight per lane (row is 4-byte aligned).
constexpr int kSweepLoads = 8;
template <class Fn>
__device__ __forceinline__ void sweep_row(const uint32_t* row, int n, Fn fn) {
  const int tid = threadIdx.x;
  const int head = min(n, (int)(((16u - ((uint32_t)(uintptr_t)row & 15u)) & 15u) >> 2));
  if (tid < head) fn(tid, row[tid]);
  const int nv = (n - head) >> 2;
  const uint4* v = reinterpret_cast<const uint4*>(row + head);
  for (int j0 = 0; j0 < nv; j0 += kSweepLoads * kSelThreads) {
    uint4 x[kSweepLoads];
#pragma unroll
    for (int u = 0; u < kSweepLoads; u++)  // (clamped, not branched: all loads in flight)
      x[u] = v[min(j0 + u * kSelThreads + tid, nv - 1)];
#pragma unroll
    for (int u = 0; u < kSweepLoads; u++) {
      const int j = j0 + u * kSelThreads + tid;
      if (j < nv) {
        const int i = head + 4 * j;
        fn(i, x[u].x); fn(i + 1, x[u].y); fn(i + 2, x[u].z); fn(i + 3, x[u].w);
      }
    }
  }
  for (int i = head + 4 * nv + tid; i < n; i += kSelThreads) fn(i, row[i]);
}

// fn(position, S bits) for every entry of a candidate list (8-byte entries: the
// position in the low word, S in the high word; the list is 16-byte aligned)
template <class Fn>
__device__ __forceinline__ void sweep_cand(const uint64_t* list, int n, Fn fn) {
  const int tid = threadIdx.x;
  const int nv = n >> 1;
  const uint4* v = reinterpret_cast<const uint4*>(list);
  for (int j0 = 0; j0 < nv; j0 += kSweepLoads * kSelThreads) {
    uint4 x[kSweepLoads];
#pragma unroll
    for (int u = 0; u < kSweepLoads; u++)  // (clamped, not branched: all loads in flight)
      x[u] = v[min(j0 + u * kSelThreads + tid, nv - 1)];
#pragma unroll
    for (int u = 0; u < kSweepLoads; u++) {
      if (j0 + u * kSelThreads + tid < nv) {
        fn(x[u].x, x[u].y);
        fn(x[u].z, x[u].w);
      }
    }
  }
  if ((n & 1) && tid == 0) {
    const uint2 e = reinterpret_cast<const uint2*>(list)[n - 1];
    fn(e.x, e.y);
  }
}

// Top digit of a score's bits for the exact path's first pass (scores are >= 0;
// anything with the sign bit set lands in the last bin, which keeps the order).
__device__ __forceinline__ uint32_t top_digit(uint32_t b) {
  return min(b >> 20, (uint32_t)kTopkBins - 1u);
}

template <class SweepFn>
__device__ bool rank_via_list(SweepFn sweep, int n, int kt, int nwords, const TopkShared& sh,
                              uint32_t* kth_out, int* krem_out) {
  if (kt <= 0 || kt >= n) return false;
  const int tid = threadIdx.x;
  for (int i = tid; i < kTopkBins; i += kSelThreads) sh.hist[i] = 0u;
  __syncthreads();
  sweep([&](uint32_t, uint32_t b) { atomicAdd(&sh.hist[top_digit(b)], 1u); });
  __syncthreads();
  constexpr int kPer = kTopkBins / kSelThreads;
  uint32_t h[kPer];
  int local = 0;
#pragma unroll
  for (int u = 0; u < kPer; u++) {
    h[u] = sh.hist[kPer * tid + u];
    local += (int)h[u];
  }
  int total;
  const int excl = block_excl_scan(local, sh.misc, &total);
  const int above = total - excl - local;
  if (above < kt && kt <= above + local) {
    int a = above, d = kPer * tid;
#pragma unroll
    for (int u = kPer - 1; u >= 0; u--) {
      if (a + (int)h[u] >= kt) { d = kPer * tid + u; break; }
      a += (int)h[u];
    }
    sh.misc[0] = d;
    sh.misc[1] = a;
  }
  __syncthreads();
  const uint32_t d1 = (uint32_t)sh.misc[0];
  const int a1 = sh.misc[1];
  const int n1 = (int)sh.hist[d1];
  if (n1 > kExactListCap) return false;  // (uniform: every thread read the same words)
  uint32_t* lkey = sh.keys;
  uint32_t* lpos = sh.keys + kExactListCap;
  for (int i = tid; i < nwords; i += kSelThreads) sh.sel[i] = 0u;
  if (tid == 0) sh.misc[3] = 0;
  __syncthreads();
  sweep([&](uint32_t i, uint32_t b) {
    const uint32_t dg = top_digit(b);
    if (dg > d1) {
      atomicOr(&sh.sel[i >> 5], 1u << (i & 31));
    } else if (dg == d1) {
      const int slot = atomicAdd(&sh.misc[3], 1);
      lkey[slot] = b;
      lpos[slot] = i;
    }
  });
  __syncthreads();
  // the kt - a1 largest of the list (1 <= kt - a1 <= n1); below the last bin the
  // list's keys share their top 12 bits (d1 and a clear sign bit)
  int krem;
  const auto lk = [&](int i) { return lkey[i]; };
  const uint32_t kth =
      d1 < (uint32_t)kTopkBins - 1u
          ? radix_digits(lk, n1, kt - a1, sh, &krem, 19, 0xFFF00000u, d1 << 20)
          : radix_kth(lk, n1, kt - a1, sh, &krem);
  mark_selected(lk, [&](int i) { return lpos[i]; }, n1, kth, krem, nwords, sh,
                /*keep_sel=*/true);
  *kth_out = kth;
  *krem_out = krem;
  return true;
}

template <int G>
__global__ __launch_bounds__(kSelThreads) void exact_kernel(TopkParams p) {
  extern __shared__ uint32_t smem[];
  const TopkShared sh = carve_lds(smem, p, true);
  const int nflag = *p.flag_count;
  const int KW = p.K + p.W;
  uint32_t* scratch = p.dense + (size_t)blockIdx.x * p.max_seqlen;
  for (int f = blockIdx.x; f < nflag; f += gridDim.x) {
    const int64_t slot = p.flag_list[f];
    const RowInfo r = decode_slot(p, slot);
    const int n_c = r.t - p.W + 1;
    int32_t* row = p.idx + ((size_t)(r.base + r.t) * p.Hkv + r.g) * KW;
    const int kt = row_budget(p.K, p.k_end, r.t, r.L);
    const int nwords = ceil_div(n_c, 32);
    int krem;
    uint32_t kth;
    const int count = p.list_rank ? p.cand_count[slot] : -1;
    if (count >= 0) {
      // a candidate list of count entries, kt <= count <= C (budgets above the
      // register-ranked limit): ranked here from the list, not from dense scores
      const uint64_t* list = p.cand + (size_t)slot * p.cand_cap;
      if (!rank_via_list([&](auto fn) { sweep_cand(list, count, fn); }, count, kt, nwords, sh,
                         &kth, &krem)) {
        kth = radix_kth([&](int i) { return (uint32_t)(list[i] >> 32); }, count, kt, sh, &krem);
        mark_selected([&](int i) { return (uint32_t)(list[i] >> 32); },
                      [&](int i) { return (uint32_t)list[i]; }, count, kth, krem, nwords, sh);
      }
      write_selected_row(nwords, n_c, r.t, KW, row, sh);
      if (p.kth && threadIdx.x == 0)
        p.kth[(size_t)(r.base + r.t) * p.Hkv + r.g] = __uint_as_float(kth);
      __syncthreads();
      continue;
    }
    // the row's scores: written by the scores kernel, or recomputed here
    const uint32_t* dense = p.dense_rows
        ? reinterpret_cast<const uint32_t*>(p.dense_rows + (size_t)slot * p.dense_ld)
        : scratch;
    if (!p.dense_rows) {
      // queries of the group's heads (fp32) and their lse2
      for (int i = threadIdx.x; i < G * kHeadDim; i += kSelThreads) {
        const int hh = i / kHeadDim, e = i % kHeadDim;
        sh.qf[i] = bf16_bits_to_f32(
            p.q[((size_t)(r.base + r.t) * p.Hq + r.g * G + hh) * kHeadDim + e]);
      }
      __syncthreads();
      float lse[G];
#pragma unroll
      for (int hh = 0; hh < G; hh++) lse[hh] = p.lse2[(size_t)(r.base + r.t) * p.Hq + r.g * G + hh];
      // S[j] for every candidate, recomputed with fp32 dot products
      for (int j = threadIdx.x; j < n_c; j += kSelThreads) {
        const uint16_t* kr = p.k + ((size_t)(r.base + j) * p.Hkv + r.g) * kHeadDim;
        float dot[G];
#pragma unroll
        for (int hh = 0; hh < G; hh++) dot[hh] = 0.f;
        for (int e8 = 0; e8 < kHeadDim / 8; e8++) {
          const uint4 kv = ldg128(kr + e8 * 8);
          const uint32_t wv[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
          for (int u = 0; u < 4; u++) {
            const float k0 = __uint_as_float(wv[u] << 16), k1 = __uint_as_float(wv[u] & 0xFFFF0000u);
#pragma unroll
            for (int hh = 0; hh < G; hh++) {
              dot[hh] = fmaf(sh.qf[hh * kHeadDim + e8 * 8 + 2 * u], k0, dot[hh]);
              dot[hh] = fmaf(sh.qf[hh * kHeadDim + e8 * 8 + 2 * u + 1], k1, dot[hh]);
            }
          }
        }
        // output-aware metric: the key's log2 weight joins every head's exponent
        const float lwj = p.vw ? p.vw[(size_t)(r.base + j) * p.Hkv + r.g] : 0.f;
        float s = 0.f;
#pragma unroll
        for (int hh = 0; hh < G; hh++) s += fast_exp2(fmaf(dot[hh], p.c, lwj - lse[hh]));
        scratch[j] = __float_as_uint(s);
      }
      __syncthreads();
    }
    if (!rank_via_list([&](auto fn) { sweep_row(dense, n_c, fn); }, n_c, kt, nwords, sh, &kth,
                       &krem)) {
      kth = radix_kth([&](int i) { return dense[i]; }, n_c, kt, sh, &krem);
      mark_selected([&](int i) { return dense[i]; }, [&](int i) { return (uint32_t)i; }, n_c, kth,
                    krem, nwords, sh);
    }
    write_selected_row(nwords, n_c, r.t, KW, row, sh);
    if (p.kth && threadIdx.x == 0)
      p.kth[(size_t)(r.base + r.t) * p.Hkv + r.g] = __uint_as_float(kth);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Decode step, selection: three launches per step, so that the pass over every
// cached score runs on many workgroups instead of one per row.
//  decode_tau_kernel (one workgroup per (KV group, sequence) row): each head's
//    log-sum-exp over all cached keys, from the split partials, and a threshold
//    tau, the r-th largest S of a 1-in-stride sample of the candidates
//    j <= t - W (t = L_b - 1).
//  decode_dense_kernel (a grid of chunks per row): S[j] of every candidate into
//    a scratch row; the scores that reach tau are appended to the row's
//    candidate list (one counter per row; slot order is arbitrary).
//  decode_rank_kernel (one workgroup per row): if at least K and at most
//    kDecodeCandCap scores reach tau, the top K all do, so only the list goes
//    through the exact radix select; otherwise the whole scratch row does. The
//    positions are marked in a bitmap, so the result is the exact top K, ties to
//    the lower position, in whatever order the list was filled.
// ---------------------------------------------------------------------------
constexpr int kDecodeSampleStride = 16;   // densest sampling
constexpr int kDecodeSampleCap = 8192;    // sampled scores held in LDS

// S bits of one candidate: the sum over the group's heads of exp2(z2 - lse2).
template <int G>
__device__ __forceinline__ uint32_t decode_score(const float (&z)[G], const float (&lse)[G]) {
  float sum = 0.f;
#pragma unroll
  for (int h = 0; h < G; h++) sum += fast_exp2(z[h] - lse[h]);
  return __float_as_uint(sum);
}

// candidates handled per thread and pass: enough independent loads in flight
template <int G>
constexpr int decode_batch() { return G >= 16 ? 2 : 32 / G; }

// rows with nothing to rank: [0, t] (all candidates fit) or the window only
__device__ __forceinline__ bool decode_trivial(const DecodeParams& p, int n_c) {
  return p.K == 0 || n_c <= p.K;
}

template <int G>
__global__ __launch_bounds__(kSelThreads) void decode_tau_kernel(DecodeParams p) {
  extern __shared__ uint32_t smem[];
  __shared__ float lse_s[G];
  TopkShared sh{};
  sh.hist = smem;
  sh.misc = reinterpret_cast<int32_t*>(smem + kTopkBins);
  sh.keys = smem + kTopkBins + 16;  // [kDecodeSampleCap] the sample
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int base = p.cu[b], L = p.cu[b + 1] - base, n_c = L - p.W;
  const size_t rowi = (size_t)b * p.Hkv + g;
  if (decode_trivial(p, n_c)) return;
  // log-sum-exp of each head: one wave per head, lanes over the splits
  const int n_sp = ceil_div(L, p.split_len);
  for (int h = w; h < G; h += kSelThreads / 64) {
    const float2* pr = p.part + rowi * p.n_split * G + h;
    float m = -INFINITY, s = 0.f;
    for (int i = l; i < n_sp; i += 64) {
      const float2 v = pr[(size_t)i * G];
      const float mn = fmaxf(m, v.x);
      s = s * fast_exp2(m - mn) + v.y * fast_exp2(v.x - mn);
      m = mn;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float mo = shfl_xor_f(m, off), so = shfl_xor_f(s, off);
      const float mn = fmaxf(m, mo);
      s = mn == -INFINITY ? 0.f : s * fast_exp2(m - mn) + so * fast_exp2(mo - mn);
      m = mn;
    }
    if (l == 0) {
      const float v = m + fast_log2(s);
      lse_s[h] = v;
      p.lse2[rowi * G + h] = v;
    }
  }
  __syncthreads();
  float lse[G];
#pragma unroll
  for (int h = 0; h < G; h++) lse[h] = lse_s[h];
  // the sample: every stride-th candidate, at most kDecodeSampleCap of them
  const int stride = max(kDecodeSampleStride, ceil_div(n_c, kDecodeSampleCap));
  const int n_s = ceil_div(n_c, stride);
  const float* zg = p.z2 + ((size_t)g * p.T + base) * G;
  constexpr int E = decode_batch<G>();
  for (int i0 = 0; i0 < n_s; i0 += E * kSelThreads) {
    float z[E][G];
#pragma unroll
    for (int u = 0; u < E; u++) {  // every load issued before the first use
      const size_t j = (size_t)min(i0 + u * kSelThreads + tid, n_s - 1) * stride;
#pragma unroll
      for (int h = 0; h < G; h++) z[u][h] = zg[j * G + h];
    }
#pragma unroll
    for (int u = 0; u < E; u++) {
      const int i = i0 + u * kSelThreads + tid;
      if (i < n_s) sh.keys[i] = decode_score<G>(z[u], lse);
    }
  }
  __syncthreads();
  // r ~ 1.5 K n_s / n_c + 16: about 1.5 K scores of the row are expected to reach
  // tau. One histogram pass suffices: tau is the lower edge of the 11-bit bin that
  // holds the sample's r-th largest score (any tau is correct, this one is close)
  const int r = min(n_s, (int)ceilf(1.5f * (float)p.K * (float)n_s / (float)n_c) + 16);
  int krem;
  const uint32_t tau = radix_kth([&](int i) { return sh.keys[i]; }, n_s, r, sh, &krem, 1);
  if (tid == 0) {
    p.tau[rowi] = tau;
    p.n_pass[rowi] = 0;
  }
}

template <int G>
__global__ __launch_bounds__(kSelThreads) void decode_dense_kernel(DecodeParams p) {
  __shared__ int32_t misc[16];
  constexpr int E = decode_batch<G>();
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int base = p.cu[b], L = p.cu[b + 1] - base, n_c = L - p.W;
  const int j0 = blockIdx.x * (E * kSelThreads);
  if (decode_trivial(p, n_c) || j0 >= n_c) return;
  const size_t rowi = (size_t)b * p.Hkv + g;
  float lse[G];
#pragma unroll
  for (int h = 0; h < G; h++) lse[h] = p.lse2[rowi * G + h];
  const uint32_t tau = p.tau[rowi];
  const float* zg = p.z2 + ((size_t)g * p.T + base) * G;
  float z[E][G];
#pragma unroll
  for (int u = 0; u < E; u++) {  // every load issued before the first use
    const size_t j = (size_t)min(j0 + u * kSelThreads + tid, n_c - 1);
#pragma unroll
    for (int h = 0; h < G; h++) z[u][h] = zg[j * G + h];
  }
  uint32_t* dense = p.dense + rowi * p.max_seqlen;
  uint32_t sv[E];
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < E; u++) {
    const int j = j0 + u * kSelThreads + tid;
    sv[u] = decode_score<G>(z[u], lse);
    if (j < n_c) {
      dense[j] = sv[u];
      cnt += sv[u] >= tau ? 1 : 0;
    }
  }
  int total;
  const int off = block_excl_scan(cnt, misc, &total);
  if (total == 0) return;
  if (tid == 0) misc[0] = atomicAdd(&p.n_pass[rowi], total);
  __syncthreads();
  int o = misc[0] + off;
  uint32_t* ck = p.cand + rowi * (2 * kDecodeCandCap);
#pragma unroll
  for (int u = 0; u < E; u++) {
    const int j = j0 + u * kSelThreads + tid;
    if (j < n_c && sv[u] >= tau) {
      if (o < kDecodeCandCap) {
        ck[o] = sv[u];
        ck[kDecodeCandCap + o] = (uint32_t)j;
      }
      o++;
    }
  }
}

template <int G>
__global__ __launch_bounds__(kSelThreads) void decode_rank_kernel(DecodeParams p) {
  extern __shared__ uint32_t smem[];
  TopkShared sh{};
  sh.hist = smem;
  sh.misc = reinterpret_cast<int32_t*>(smem + kTopkBins);
  sh.sel = smem + kTopkBins + 16;
  sh.tie = sh.sel + p.bitmap_words;
  sh.keys = sh.tie + p.bitmap_words;                   // [kDecodeCandCap] candidate S bits
  uint32_t* cpos = sh.keys + kDecodeCandCap;           // [kDecodeCandCap] their positions
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int base = p.cu[b], L = p.cu[b + 1] - base;
  const int t = L - 1, n_c = t - p.W + 1, KW = p.K + p.W;
  const size_t rowi = (size_t)b * p.Hkv + g;
  int32_t* row = p.idx + rowi * KW;
  float* kth_out = p.kth ? p.kth + rowi : nullptr;
  if (decode_trivial(p, n_c)) {
    write_trivial_row(n_c, p.K, t, KW, row);
    if (kth_out && tid == 0) *kth_out = -1.f;
    return;
  }
  const int n_pass = p.n_pass[rowi];
  int krem;
  uint32_t kth;
  if (n_pass >= p.K && n_pass <= kDecodeCandCap) {
    const uint32_t* ck = p.cand + rowi * (2 * kDecodeCandCap);
    constexpr int kB = 4;
    for (int i0 = 0; i0 < n_pass; i0 += kB * kSelThreads) {
      uint32_t kv[kB], pv[kB];
#pragma unroll
      for (int u = 0; u < kB; u++) {  // every load issued before the first store
        const int i = min(i0 + u * kSelThreads + tid, n_pass - 1);
        kv[u] = ck[i];
        pv[u] = ck[kDecodeCandCap + i];
      }
#pragma unroll
      for (int u = 0; u < kB; u++) {
        const int i = i0 + u * kSelThreads + tid;
        if (i < n_pass) { sh.keys[i] = kv[u]; cpos[i] = pv[u]; }
      }
    }
    __syncthreads();
    kth = radix_kth([&](int i) { return sh.keys[i]; }, n_pass, p.K, sh, &krem);
    mark_selected([&](int i) { return sh.keys[i]; }, [&](int i) { return cpos[i]; }, n_pass, kth,
                  krem, ceil_div(n_c, 32), sh);
  } else {  // the sample misled: rank the whole row
    const uint32_t* dense = p.dense + rowi * p.max_seqlen;
    kth = radix_kth([&](int i) { return dense[i]; }, n_c, p.K, sh, &krem);
    mark_selected([&](int i) { return dense[i]; }, [&](int i) { return (uint32_t)i; }, n_c, kth,
                  krem, ceil_div(n_c, 32), sh);
  }
  write_selected_row(ceil_div(n_c, 32), n_c, t, KW, row, sh);
  if (kth_out && tid == 0) *kth_out = __uint_as_float(kth);
}

template <class Kern>
static hipError_t allow_lds(Kern k, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <int G>
static hipError_t launch_decode_select_g(const DecodeParams& p, size_t lds, hipStream_t s) {
  constexpr int E = decode_batch<G>();
  const size_t lds_tau = (size_t)(kTopkBins + 16 + kDecodeSampleCap) * sizeof(uint32_t);
  hipError_t e = allow_lds(decode_tau_kernel<G>, lds_tau);
  if (e != hipSuccess) return e;
  e = allow_lds(decode_rank_kernel<G>, lds);
  if (e != hipSuccess) return e;
  const dim3 rows(p.Hkv, p.B), block(kSelThreads);
  hipLaunchKernelGGL(decode_tau_kernel<G>, rows, block, lds_tau, s, p);
  const dim3 chunks(ceil_div(p.max_seqlen, E * kSelThreads), p.Hkv, p.B);
  hipLaunchKernelGGL(decode_dense_kernel<G>, chunks, block, 0, s, p);
  hipLaunchKernelGGL(decode_rank_kernel<G>, rows, block, lds, s, p);
  return hipGetLastError();
}

hipError_t launch_decode_select(int G, const DecodeParams& p, size_t lds_bytes, hipStream_t s) {
  if (p.B <= 0) return hipSuccess;
  switch (G) {
    case 1: return launch_decode_select_g<1>(p, lds_bytes, s);
    case 2: return launch_decode_select_g<2>(p, lds_bytes, s);
    case 4: return launch_decode_select_g<4>(p, lds_bytes, s);
    case 8: return launch_decode_select_g<8>(p, lds_bytes, s);
    case 16: return launch_decode_select_g<16>(p, lds_bytes, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_topk(int G, const TopkParams& p, int n_tasks, int rows_per_block, hipStream_t s) {
  (void)G;
  if (n_tasks <= 0) return hipSuccess;
  // blocks of 1, 2 or 4 rows (consecutive tokens of one task; tok is a power of two >= 16)
  if ((rows_per_block != 1 && rows_per_block != 2 && rows_per_block != 4) ||
      p.tok != (1 << p.tok_shift) || p.tok < rows_per_block)
    return hipErrorInvalidValue;
  const size_t lds =
      (size_t)rows_per_block * (256 + p.bitmap_words + p.sbuf_words) * sizeof(uint32_t);
  const dim3 grid((unsigned)n_tasks * (unsigned)(p.tok / rows_per_block), (unsigned)p.Hkv),
      block(64 * rows_per_block);
  const int nreg = p.list_rank ? 32 : p.cand_cap / 64;  // (list-ranked rows are not read)
  if (nreg <= 32) {
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<32>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(topk_kernel<32>, grid, block, lds, s, p);
  } else {
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<64>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(topk_kernel<64>, grid, block, lds, s, p);
  }
  return hipGetLastError();
}

template <int G>
static hipError_t launch_exact_g(const TopkParams& p, size_t lds_bytes, hipStream_t s) {
  if (lds_bytes > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)exact_kernel<G>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(exact_kernel<G>, dim3(kFallbackBlocks), dim3(kSelThreads), lds_bytes, s, p);
  return hipGetLastError();
}

hipError_t launch_fallback(int G, const TopkParams& p, size_t lds_bytes, hipStream_t s) {
  switch (G) {
    case 1: return launch_exact_g<1>(p, lds_bytes, s);
    case 2: return launch_exact_g<2>(p, lds_bytes, s);
    case 4: return launch_exact_g<4>(p, lds_bytes, s);
    case 8: return launch_exact_g<8>(p, lds_bytes, s);
    case 16: return launch_exact_g<16>(p, lds_bytes, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hs2
