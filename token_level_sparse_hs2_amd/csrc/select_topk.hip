// select_topk.hip - exact top-K of each (t, g) row and index assembly on gfx950.
//
// Selection rule (HySparse2 news summary, token-granularity paragraph: single
// tokens, not 64-token blocks; forced-recent paragraph: the W most recent
// tokens are always in): among the candidates C_t = [0, t-W] keep the K with
// the largest group score S, ties to the lower position; then
//   I_t = ascending(T_t U [t-W+1, t]), padded with -1 to K+W.
//
// topk_kernel: one 256-thread workgroup per row of a chunk. Its candidates
//   (S >= tau, collected by the scoring sweep) are ranked by a 4-pass 8-bit
//   radix select on the fp32 bit pattern of S (monotone for S >= 0), which
//   yields the K-th largest value and how many of the values equal to it to
//   take. Selected positions go into an LDS bitmap, so the compaction into the
//   index row comes out in ascending order.
// exact_kernel: persistent workgroups over the rows the sweep could not settle
//   (too many / too few candidates, or the exact flag). S is recomputed for the
//   whole row into a scratch row, then the same select and assembly run.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

struct TopkShared {
  uint32_t* hist;   // [256]
  int32_t* misc;    // [16]
  uint32_t* sel;    // [bitmap_words]
  uint32_t* tie;    // [bitmap_words]
  uint32_t* keys;   // [cand_cap] (candidate path only)
  float* qf;        // [16 * 128] (exact path only)
};

__device__ __forceinline__ int wave_incl_scan(int x, int l) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (l >= off) x += y;
  }
  return x;
}

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

// K-th largest key among key(i), i < n (1 <= k <= n). Returns the key and, in
// *krem, how many elements equal to it belong to the top k.
template <class KeyFn>
__device__ uint32_t radix_kth(KeyFn key, int n, int k, const TopkShared& sh, int* krem) {
  const int tid = threadIdx.x, l = tid & 63;
  uint32_t prefix = 0u, mask = 0u;
  int kr = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    sh.hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
      const uint32_t b = key(i);
      if ((b & mask) == prefix) atomicAdd(&sh.hist[(b >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const uint32_t h0 = sh.hist[4 * l], h1 = sh.hist[4 * l + 1], h2 = sh.hist[4 * l + 2],
                     h3 = sh.hist[4 * l + 3];
      const uint32_t local = h0 + h1 + h2 + h3;
      uint32_t suf = local;  // inclusive suffix sum over lanes
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(suf, off, 64);
        if (l + off < 64) suf += v;
      }
      const uint32_t above = suf - local;
      if (above < (uint32_t)kr && (uint32_t)kr <= suf) {
        uint32_t a = above;
        int d;
        if (a + h3 >= (uint32_t)kr) d = 4 * l + 3;
        else if ((a += h3) + h2 >= (uint32_t)kr) d = 4 * l + 2;
        else if ((a += h2) + h1 >= (uint32_t)kr) d = 4 * l + 1;
        else { a += h1; d = 4 * l; }
        sh.misc[0] = d;
        sh.misc[1] = (int)a;
      }
    }
    __syncthreads();
    const int d = sh.misc[0];
    kr -= sh.misc[1];
    prefix |= (uint32_t)d << shift;
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  *krem = kr;
  return prefix;
}

// Marks in sh.sel every position whose key is above kth, plus the krem lowest
// positions whose key equals kth.
template <class KeyFn, class PosFn>
__device__ void mark_selected(KeyFn key, PosFn pos, int n, uint32_t kth, int krem, int nwords,
                              const TopkShared& sh) {
  const int tid = threadIdx.x;
  for (int i = tid; i < nwords; i += kSelThreads) { sh.sel[i] = 0u; sh.tie[i] = 0u; }
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
// the window [n_c, t]; n_sel + window == K + W here, so no padding.
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
  sh.misc = reinterpret_cast<int32_t*>(smem + 256);
  sh.sel = smem + 256 + 16;
  sh.tie = sh.sel + p.bitmap_words;
  sh.keys = sh.tie + p.bitmap_words;
  sh.qf = reinterpret_cast<float*>(sh.keys);
  (void)exact;
  return sh;
}

__global__ __launch_bounds__(kSelThreads) void topk_kernel(TopkParams p) {
  extern __shared__ uint32_t smem[];
  const TopkShared sh = carve_lds(smem, p, false);
  const int64_t slot = blockIdx.x;
  const RowInfo r = decode_slot(p, slot);
  if (r.t >= r.L) return;
  const int KW = p.K + p.W;
  const int n_c = r.t - p.W + 1;
  int32_t* row = p.idx + ((size_t)(r.base + r.t) * p.Hkv + r.g) * KW;
  float* kth_out = p.kth ? p.kth + (size_t)(r.base + r.t) * p.Hkv + r.g : nullptr;
  if (p.K == 0 || n_c <= p.K) {
    write_trivial_row(n_c, p.K, r.t, KW, row);
    if (kth_out && threadIdx.x == 0) *kth_out = -1.f;
    return;
  }
  const int count = p.cand_count[slot];
  if (count < 0) return;  // settled by exact_kernel
  const uint64_t* cand = p.cand + (size_t)slot * p.cand_cap;
  for (int i = threadIdx.x; i < count; i += kSelThreads) sh.keys[i] = (uint32_t)(cand[i] >> 32);
  __syncthreads();
  int krem;
  const uint32_t kth = radix_kth([&](int i) { return sh.keys[i]; }, count, p.K, sh, &krem);
  const int nwords = ceil_div(n_c, 32);
  mark_selected([&](int i) { return sh.keys[i]; },
                [&](int i) { return (uint32_t)(cand[i] & 0xFFFFFFFFu); }, count, kth, krem, nwords,
                sh);
  write_selected_row(nwords, n_c, r.t, KW, row, sh);
  if (kth_out && threadIdx.x == 0) *kth_out = __uint_as_float(kth);
}

template <int G>
__global__ __launch_bounds__(kSelThreads) void exact_kernel(TopkParams p) {
  extern __shared__ uint32_t smem[];
  const TopkShared sh = carve_lds(smem, p, true);
  const int nflag = *p.flag_count;
  const int KW = p.K + p.W;
  uint32_t* dense = p.dense + (size_t)blockIdx.x * p.max_seqlen;
  for (int f = blockIdx.x; f < nflag; f += gridDim.x) {
    const int64_t slot = p.flag_list[f];
    const RowInfo r = decode_slot(p, slot);
    const int n_c = r.t - p.W + 1;
    int32_t* row = p.idx + ((size_t)(r.base + r.t) * p.Hkv + r.g) * KW;
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
      float s = 0.f;
#pragma unroll
      for (int hh = 0; hh < G; hh++) s += fast_exp2(dot[hh] * p.c - lse[hh]);
      dense[j] = __float_as_uint(s);
    }
    __syncthreads();
    int krem;
    const uint32_t kth = radix_kth([&](int i) { return dense[i]; }, n_c, p.K, sh, &krem);
    const int nwords = ceil_div(n_c, 32);
    mark_selected([&](int i) { return dense[i]; }, [&](int i) { return (uint32_t)i; }, n_c, kth,
                  krem, nwords, sh);
    write_selected_row(nwords, n_c, r.t, KW, row, sh);
    if (p.kth && threadIdx.x == 0)
      p.kth[(size_t)(r.base + r.t) * p.Hkv + r.g] = __uint_as_float(kth);
    __syncthreads();
  }
}

hipError_t launch_topk(int G, const TopkParams& p, int n_rows, size_t lds_bytes, hipStream_t s) {
  (void)G;
  if (n_rows <= 0) return hipSuccess;
  if (lds_bytes > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topk_kernel, dim3(n_rows), dim3(kSelThreads), lds_bytes, s, p);
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
