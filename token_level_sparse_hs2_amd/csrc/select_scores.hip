// select_scores.hip - the full-attention layer's scoring sweeps on gfx950.
//
// One workgroup owns TOK consecutive query tokens of one sequence and one KV
// group g: all G query heads of the group, 4 waves x 16 * RT MFMA rows in
// token-major, head-minor order, so the 4 accumulator rows a lane holds are the
// heads of whole tokens (G <= 4) or a share of one token (G = 8, 16; joined with
// the partner lane groups). It sweeps the causal keys in 64-key tiles streamed
// through an LDS ring, with bf16 v_mfma_f32_16x16x32_bf16 and fp32 accumulation:
//
//  1. row statistics: per (t, h) the log2-domain log-sum-exp lse2 of the full
//     layer's softmax over all causal keys with scale 1/sqrt(d) (attention as in
//     the SHARP walkthrough, section 1.1). The exponents are taken against a
//     fixed per-row reference, the Cauchy-Schwarz bound c * |q| * max_j |k_j|,
//     which the MFMAs subtract as their initial accumulator, so the sweep needs
//     no running maximum; if that bound is too loose for some row (sum below
//     2^-60) the workgroup first finds each row's exact maximum and sums again.
//  2. sample: on every 8th key tile, the group score
//       S[t,g,j] = sum_{h in g} exp2(z2[t,h,j] - lse2[t,h])
//     (the full layer's probabilities, summed over the group whose KV cache
//     and selection the sparse layers reuse -- HySparse2 news summary, KV
//     Reuse and ablation paragraphs) goes into a per-token LDS histogram, from
//     which a threshold tau just below the top-K boundary is estimated.
//  3. collect: on all candidate tiles (keys j <= t - W; the W most recent
//     tokens are forced in separately, forced-recent paragraph), every S >= tau
//     is appended as (S, j) to the token's candidate row in global memory.
//
// A row whose candidates are too many (> C) or too few (< K) is sent to the
// exact path (select_topk.hip), so the result never depends on the sample.
#include <type_traits>

#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

enum : int { kModeTrivial = 0, kModeEmit = 1, kModeExact = 2, kModeSample = 3 };

template <int G>
struct ScoreCfg {
  static constexpr int RT = score_row_tiles(G);   // 16-row tiles per wave
  static constexpr int ROWS_W = 16 * RT;          // MFMA rows per wave
  static constexpr int TOK = tokens_per_task(G);  // tokens per workgroup
  // tokens whose rows a lane holds per accumulator tile: 4 (G = 1), 2 (G = 2), else 1
  static constexpr int NT = G >= 4 ? 1 : 4 / G;
};

constexpr int kRing = 4;  // K tiles in flight: compute tile kt while kt+1..kt+3 load

template <int TOK>
struct ScoreSmem {
  // A ring of kRing 64-key x 256-byte K tiles (XOR-swizzled 16-byte chunks). The
  // sample sweep uses tiles 0-1 only and keeps its histogram where tiles 2-3 live.
  union {
    uint4 ktile[kRing][kKeyTile][16];
    struct {
      uint4 ktile2[2][kKeyTile][16];
      uint32_t hist[TOK][kBins / 2];  // two 16-bit bin counters per word
    } s;
  } u;
  float nref[256];                   // minus the reference of each MFMA row
  // output-aware metric: log2 key weights of each ring slot's tile, one copy per wave
  float lw[kRing][kSelThreads / 64][kKeyTile];
  float tau[TOK];
  int32_t cnt[TOK];
  int32_t mode[TOK];
  int32_t any_sample, any_emit, unsafe;
};

__global__ void zero_i32_kernel(int32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

// Largest key norm of each (sequence, KV group). A workgroup takes 256 tokens of
// one group, 16 lanes per key row (coalesced 256-byte rows); when its tokens lie
// in one sequence it reduces to one atomic max on the float bits (norms are >= 0),
// else each row does its own. kmax must be zeroed first.
__global__ __launch_bounds__(256) void key_norm_kernel(const uint16_t* k, const int32_t* cu, int B,
                                                       int Hkv, int64_t T, uint32_t* kmax) {
  __shared__ float wmax[4];
  const int g = blockIdx.y, tid = threadIdx.x, lane16 = tid & 15, sub = tid >> 4;
  const int64_t t_first = (int64_t)blockIdx.x * 256;
  const int64_t t_last = min(T, t_first + 256) - 1;
  const int s_first = find_seq(cu, B, t_first), s_last = find_seq(cu, B, t_last);
  const bool one_seq = s_first == s_last;
  float m = 0.f;
  for (int it = 0; it < 16; it++) {
    const int64_t tok = t_first + 16 * it + sub;
    float n2 = 0.f;
    if (tok <= t_last) {
      const uint4 v = ldg128(k + ((size_t)tok * Hkv + g) * kHeadDim + 8 * lane16);
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const float a = __uint_as_float(wv[u] << 16), b = __uint_as_float(wv[u] & 0xFFFF0000u);
        n2 = fmaf(a, a, fmaf(b, b, n2));
      }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) n2 += shfl_xor_f(n2, off);
    const float nrm = sqrtf(n2);
    if (one_seq) m = fmaxf(m, nrm);
    else if (lane16 == 0 && tok <= t_last)
      atomicMax(&kmax[find_seq(cu, B, tok) * Hkv + g], __float_as_uint(nrm));
  }
  if (!one_seq) return;  // uniform over the workgroup
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) m = fmaxf(m, shfl_xor_f(m, off));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  if (tid == 0)
    atomicMax(&kmax[s_first * Hkv + g],
              __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
}

hipError_t launch_key_norms(const uint16_t* k, const int32_t* cu, int B, int Hkv, int64_t T,
                            uint32_t* kmax, hipStream_t s) {
  hipError_t e = launch_zero_i32(reinterpret_cast<int32_t*>(kmax), B * Hkv, s);
  if (e != hipSuccess) return e;
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(key_norm_kernel, dim3((unsigned)((T + 255) / 256), (unsigned)Hkv), dim3(256), 0,
                     s, k, cu, B, Hkv, T, kmax);
  return hipGetLastError();
}

// Key weights of the output-aware metric, max(1, |v[j,g]|_2)^beta: vw[j, g] holds
// their log2, beta * max(0, log2 |v|), and vwmax the largest weight of each
// (sequence, group) itself, as float bits (weights are >= 1; vwmax zeroed first).
// Same geometry and single-sequence reduction as key_norm_kernel.
__global__ __launch_bounds__(256) void value_weight_kernel(const uint16_t* v, const int32_t* cu,
                                                           int B, int Hkv, int64_t T, float beta,
                                                           float* vw, uint32_t* vwmax) {
  __shared__ float wmax[4];
  const int g = blockIdx.y, tid = threadIdx.x, lane16 = tid & 15, sub = tid >> 4;
  const int64_t t_first = (int64_t)blockIdx.x * 256;
  const int64_t t_last = min(T, t_first + 256) - 1;
  const int s_first = find_seq(cu, B, t_first), s_last = find_seq(cu, B, t_last);
  const bool one_seq = s_first == s_last;
  float m = 1.f;
  for (int it = 0; it < 16; it++) {
    const int64_t tok = t_first + 16 * it + sub;
    float n2 = 0.f;
    if (tok <= t_last) {
      const uint4 x = ldg128(v + ((size_t)tok * Hkv + g) * kHeadDim + 8 * lane16);
      const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const float a = __uint_as_float(wv[u] << 16), b = __uint_as_float(wv[u] & 0xFFFF0000u);
        n2 = fmaf(a, a, fmaf(b, b, n2));
      }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) n2 += shfl_xor_f(n2, off);
    // n2 <= 1 gives weight 1
    const float lw = n2 > 1.f ? beta * 0.5f * fast_log2(n2) : 0.f;
    const float wgt = fast_exp2(lw);
    if (lane16 == 0 && tok <= t_last) {
      vw[(size_t)tok * Hkv + g] = lw;
      if (!one_seq) atomicMax(&vwmax[find_seq(cu, B, tok) * Hkv + g], __float_as_uint(wgt));
    }
    if (tok <= t_last) m = fmaxf(m, wgt);
  }
  if (!one_seq) return;  // uniform over the workgroup
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) m = fmaxf(m, shfl_xor_f(m, off));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  if (tid == 0)
    atomicMax(&vwmax[s_first * Hkv + g],
              __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
}

hipError_t launch_value_weights(const uint16_t* v, const int32_t* cu, int B, int Hkv, int64_t T,
                                float beta, float* vw, uint32_t* vwmax, hipStream_t s) {
  hipError_t e = launch_zero_i32(reinterpret_cast<int32_t*>(vwmax), B * Hkv, s);
  if (e != hipSuccess || T <= 0) return e;
  hipLaunchKernelGGL(value_weight_kernel, dim3((unsigned)((T + 255) / 256), (unsigned)Hkv), dim3(256),
                     0, s, v, cu, B, Hkv, T, beta, vw, vwmax);
  return hipGetLastError();
}

// DENSE: the rows the exact path ranks (every ranked row, with the exact flag or a
// budget above the register-ranked limit) get the score of every candidate written
// to p.dense_out, from which exact_kernel selects; the other rows are unchanged.
template <int G, bool DENSE>
__global__ __launch_bounds__(kSelThreads, 2) void scores_kernel(ScoreParams p) {
  using Cfg = ScoreCfg<G>;
  constexpr int RT = Cfg::RT, TOK = Cfg::TOK, ROWS_W = Cfg::ROWS_W, NT = Cfg::NT;
  static_assert(TOK <= 64, "the histogram overlays two ring slots");
  __shared__ ScoreSmem<TOK> sm;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int lq = l >> 4, lc = l & 15;
  const int g = blockIdx.x % p.Hkv;
  const int64_t task = p.task_begin + blockIdx.x / p.Hkv;
  int seq, tile;
  plan_decode(p.cu, p.B, TOK, p.max_tiles, task, &seq, &tile);
  // the top-K kernel of this chunk finds each row's task here instead of searching again
  if (tid == 0 && g == 0) p.task_map[blockIdx.x / p.Hkv] = make_int2(seq, tile);
  const int base = p.cu[seq];
  const int L = p.cu[seq + 1] - base;
  const int t0 = tile * TOK;
  const int ntok = min(TOK, L - t0);
  const int64_t slot0 = (int64_t)blockIdx.x * TOK;
  const int Hq = p.Hq, Hkv = p.Hkv, K = p.K, W = p.W;
  const float c = p.c;

  // accumulator element i of row tile rt: wave row 16 rt + 4 lq + i, key lc of its
  // 16-key column tile
  auto row_of = [&](int rt, int i) HS2_INLINE { return w * ROWS_W + 16 * rt + 4 * lq + i; };
  // local token of the lane's u-th token in row tile rt
  auto token_of = [&](int rt, int u) HS2_INLINE { return (w * ROWS_W + 16 * rt + 4 * lq) / G + u; };
  // lanes holding a token's first rows (G = 8 and 16 spread a token over lane groups)
  const bool owner = (G <= 4) || (G == 8 ? ((lq & 1) == 0) : (lq == 0));

  // ---- Q operands (A): row ra (token-major, head-minor), d = 32 ks + 8 lq .. +7 ----
  // all loads first (rows past the sequence read its last token and are zeroed
  // afterwards), so their latencies overlap
  bf16x8 qa[RT][4];
  u32x4 qv[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; rt++) {
    const int ra = w * ROWS_W + 16 * rt + lc;
    const int ta = min(ra / G, ntok - 1), ha = ra % G;
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
      qv[rt][ks] = to_u32x4(ldg128(p.q + ((size_t)(base + t0 + ta) * Hq + g * G + ha) * kHeadDim +
                                   32 * ks + 8 * lq));
  }
  const float kmax = p.lse_given ? 0.f : __uint_as_float(p.kmax[seq * Hkv + g]);
#pragma unroll
  for (int rt = 0; rt < RT; rt++) {
    const int ra = w * ROWS_W + 16 * rt + lc;
    const bool live = ra / G < ntok;
    float qn2 = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      u32x4 v = qv[rt][ks];
      if (!live) v = u32x4{0u, 0u, 0u, 0u};
      qa[rt][ks] = as_bf16x8(v);
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const float a = __uint_as_float(v[u] << 16), b = __uint_as_float(v[u] & 0xFFFF0000u);
        qn2 = fmaf(a, a, fmaf(b, b, qn2));
      }
    }
    qn2 += shfl_xor_f(qn2, 16);
    qn2 += shfl_xor_f(qn2, 32);
    // reference of sweep 1: the Cauchy-Schwarz bound |q| * max_j |k_j| >= q . k_j
    if (lq == 0) sm.nref[ra] = -(sqrtf(qn2) * kmax);
  }

  // K tiles go global -> LDS directly (no staging registers). One load moves 4
  // keys x 256 bytes: lane l lands at LDS slot (key 4r + (l >> 4), chunk l & 15)
  // and fetches the logical chunk (l & 15) ^ (key & 15), which realises the XOR
  // swizzle. Keys at or past kend read row kend - 1 (masked later). The load is
  // issued from inline asm so that the compiler, which cannot tell ring slots
  // apart, does not drain every load in flight before each LDS read; the sweeps
  // wait for exactly the tile they need with vmcnt and an LDS-only barrier.
  const uint16_t* kbase = p.k + (size_t)g * kHeadDim;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t lds_ring = (uint32_t)(uintptr_t)&sm.u.ktile[0][0][0];
  const uint32_t lds_lw = (uint32_t)(uintptr_t)&sm.lw[0][0][0];
  // With wts (the output-aware metric) a fifth load per wave brings the tile's 64
  // log2 key weights into the wave's own copy, so the ring waits cover them too.
  // A whole tile (every key below kend) loads from a wave-uniform tile base in
  // SGPRs plus fixed 32-bit lane offsets, so its addresses cost no vector ALU work;
  // only a partial last tile clamps each key to kend - 1.
  const size_t krow_bytes = (size_t)Hkv * kHeadDim * sizeof(uint16_t);
  uint32_t koff[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int key = 16 * w + 4 * r + lq;
    koff[r] = (uint32_t)(key * krow_bytes) + 16u * (lc ^ (key & 15));
  }
  const uint32_t wofs = (uint32_t)(l * Hkv) * (uint32_t)sizeof(float);
  auto dma_tile = [&](int kt, int kend, int buf, bool wts) HS2_INLINE {
    if (kt * kKeyTile + kKeyTile <= kend) {
      const uint16_t* tb = uniform_ptr(kbase + (size_t)(base + kt * kKeyTile) * Hkv * kHeadDim);
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const uint32_t dst = lds_ring + (uint32_t)(buf * kKeyTile + 16 * wu + 4 * r) * 256u;
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(koff[r]), "s"(tb), "{m0}"(dst)
                     : "memory");
      }
      if (wts) {
        const float* wb = uniform_ptr(p.vw + (size_t)(base + kt * kKeyTile) * Hkv + g);
        const uint32_t dst = lds_lw + (uint32_t)(buf * (kSelThreads / 64) + wu) * (kKeyTile * 4u);
        asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(wofs), "s"(wb), "{m0}"(dst)
                     : "memory");
      }
      return;
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int key = 16 * w + 4 * r + lq;
      const int j = min(kt * kKeyTile + key, kend - 1);
      const int ch = lc ^ (key & 15);
      const uint16_t* src = kbase + (size_t)(base + j) * Hkv * kHeadDim + ch * 8;
      const uint32_t dst = lds_ring + (uint32_t)(buf * kKeyTile + 16 * wu + 4 * r) * 256u;
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(dst) : "memory");
    }
    if (wts) {
      const float* src = p.vw + (size_t)(base + min(kt * kKeyTile + l, kend - 1)) * Hkv + g;
      const uint32_t dst = lds_lw + (uint32_t)(buf * (kSelThreads / 64) + wu) * (kKeyTile * 4u);
      asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(dst) : "memory");
    }
  };
  auto lds_barrier = [&]() HS2_INLINE {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  // Wait until the oldest outstanding tile has landed while `younger` later tiles
  // (4 loads each, 5 with weights; at most 2 of them) may still be in flight, then
  // the barrier. Loads complete in issue order, so vmcnt <= loads * younger
  // suffices; global stores issued in between only make the wait stricter.
  auto ring_ready = [&](int younger, bool wts) HS2_INLINE {
    // s_waitcnt immediate: vmcnt in bits 3:0, expcnt 6:4 = 7 and lgkmcnt 11:8 = 15 (no wait)
    if (younger >= 2) {
      if (wts) __builtin_amdgcn_s_waitcnt(0x0F7A);  // vmcnt(10)
      else __builtin_amdgcn_s_waitcnt(0x0F78);      // vmcnt(8)
    } else if (younger == 1) {
      if (wts) __builtin_amdgcn_s_waitcnt(0x0F75);  // vmcnt(5)
      else __builtin_amdgcn_s_waitcnt(0x0F74);      // vmcnt(4)
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    lds_barrier();
  };
  // Streams tiles first, first + step, ... (n of them) of keys below kend through
  // NS ring slots, NS - 1 tiles ahead; body(kt, slot). Ends with every load landed
  // and every wave past its last LDS read.
  auto sweep = [&](int n, int first, int step, int kend, auto NSc, bool wts,
                   auto&& body) HS2_INLINE {
    constexpr int NS = decltype(NSc)::value;
    static_assert(NS <= 4, "ring_ready waits for at most 2 younger tiles");
#pragma unroll
    for (int i = 0; i < NS - 1; i++)
      if (i < n) dma_tile(first + i * step, kend, i, wts);
    for (int i = 0; i < n; i++) {
      ring_ready(min(NS - 2, n - 1 - i), wts);
      // every wave is past tile i - 1, so its slot can take tile i + NS - 1
      if (i + NS - 1 < n) dma_tile(first + (i + NS - 1) * step, kend, (i + NS - 1) % NS, wts);
      body(first + i * step, i % NS);
    }
    lds_barrier();
  };
  // acc = q . k - rref[row]: the first MFMA of each chain starts from -rref
  f32x4 acc[RT][4];
  f32x4 nref4[RT];
  auto load_nref = [&]() HS2_INLINE {
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
      nref4[rt] = *reinterpret_cast<const f32x4*>(&sm.nref[w * ROWS_W + 16 * rt + 4 * lq]);
  };
  // the MFMAs of column tile ct (16 keys) for every row tile
  auto compute_ct = [&](int buf, int ct) HS2_INLINE {
    const int kk = 16 * ct + lc;  // kk & 15 == lc
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const bf16x8 b = as_bf16x8(to_u32x4(sm.u.ktile[buf][kk][(4 * ks + lq) ^ lc]));
#pragma unroll
      for (int rt = 0; rt < RT; rt++)
        acc[rt][ct] = mfma16x16x32(qa[rt][ks], b, ks == 0 ? nref4[rt] : acc[rt][ct]);
    }
  };
  auto compute = [&](int buf) HS2_INLINE {
    // the wave's matrix block issues at raised priority, so that the other wave on
    // the SIMD fills the matrix core's busy cycles with its exponentials
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ct = 0; ct < 4; ct++) compute_ct(buf, ct);
    __builtin_amdgcn_s_setprio(0);
  };
  // keys beyond a row's token are -inf (only tiles that reach past t0)
  auto mask_causal = [&](int kt) HS2_INLINE {
    if (kt * kKeyTile + kKeyTile - 1 <= t0) return;
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int t = t0 + row_of(rt, i) / G;
#pragma unroll
        for (int ct = 0; ct < 4; ct++)
          if (kt * kKeyTile + 16 * ct + lc > t) acc[rt][ct][i] = -INFINITY;
      }
  };
  using Ring = std::integral_constant<int, kRing>;
  using Pair = std::integral_constant<int, 2>;

  // ======================= sweep 1: row statistics ==========================
  // lsum = sum_j exp2(c (q . k_j - rref)) over the causal keys; a row's 16 lanes
  // (one per key column) are summed at the end.
  const int kend1 = t0 + ntok;
  const int n_kt1 = ceil_div(kend1, kKeyTile);
  float lsum[RT][4];
  auto sum_sweep = [&]() HS2_INLINE {
    lds_barrier();  // nref
    load_nref();
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int i = 0; i < 4; i++) lsum[rt][i] = 0.f;
    auto sum_ct = [&](int ct) HS2_INLINE {
#pragma unroll
      for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int i = 0; i < 4; i++) lsum[rt][i] += fast_exp2(acc[rt][ct][i] * c);
    };
    sweep(n_kt1, 0, 1, kend1, Ring{}, false, [&](int kt, int buf) HS2_INLINE {
      compute(buf);
      mask_causal(kt);
#pragma unroll
      for (int ct = 0; ct < 4; ct++) sum_ct(ct);
    });
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float s = lsum[rt][i];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) s += shfl_xor_f(s, off);
        lsum[rt][i] = s;
      }
  };
  if (p.lse_given) {
    // the row statistics come with the call (the full layer's output sweep wrote
    // them): rref = lse2 / c, so exp2(c * acc) is the full layer's probability.
    // The bound-based references written above must land first.
    __syncthreads();
    for (int row = tid; row < 4 * ROWS_W; row += kSelThreads) {
      const int tl = row / G;
      sm.nref[row] =
          tl < ntok ? -p.lse2[(size_t)(base + t0 + tl) * Hq + g * G + row % G] / c : 0.f;
    }
    __syncthreads();
  } else {
    sum_sweep();
    {
      bool bad = false;
  #pragma unroll
      for (int rt = 0; rt < RT; rt++)
  #pragma unroll
        for (int i = 0; i < 4; i++) bad |= (row_of(rt, i) / G < ntok) && !(lsum[rt][i] >= 0x1p-60f);
      if (tid == 0) sm.unsafe = 0;
      __syncthreads();
      if (bad) sm.unsafe = 1;
      __syncthreads();
    }
    if (sm.unsafe) {
      // the bound is too loose for some row: rref <- the row's exact maximum of
      // q . k_j, then the sum again
      float mx[RT][4];
  #pragma unroll
      for (int rt = 0; rt < RT; rt++)
  #pragma unroll
        for (int i = 0; i < 4; i++) mx[rt][i] = -INFINITY;
      sweep(n_kt1, 0, 1, kend1, Ring{}, false, [&](int kt, int buf) HS2_INLINE {
        compute(buf);
        mask_causal(kt);
  #pragma unroll
        for (int rt = 0; rt < RT; rt++)
  #pragma unroll
          for (int i = 0; i < 4; i++)
            mx[rt][i] = fmaxf(mx[rt][i], fmaxf(fmaxf(acc[rt][0][i], acc[rt][1][i]),
                                               fmaxf(acc[rt][2][i], acc[rt][3][i])));
      });
  #pragma unroll
      for (int rt = 0; rt < RT; rt++)
  #pragma unroll
        for (int i = 0; i < 4; i++) {
          float m = mx[rt][i];
  #pragma unroll
          for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, shfl_xor_f(m, off));
          // acc held q . k - rref, so the new reference is rref + m
          if (lc == 0) sm.nref[row_of(rt, i)] -= m;
        }
      sum_sweep();
    }
    // lse2 = c * rref + log2(lsum); from here on rref = lse2 / c, so that
    // exp2(c * acc) is the full layer's probability
    lds_barrier();
  #pragma unroll
    for (int rt = 0; rt < RT; rt++)
  #pragma unroll
      for (int i = 0; i < 4; i++) lsum[rt][i] = fmaf(-c, nref4[rt][i], fast_log2(lsum[rt][i]));
    lds_barrier();
  #pragma unroll
    for (int rt = 0; rt < RT; rt++)
  #pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = row_of(rt, i);
        if (lc == 0) {
          sm.nref[row] = -lsum[rt][i] / c;
          if (row / G < ntok) p.lse2[(size_t)(base + t0 + row / G) * Hq + g * G + row % G] = lsum[rt][i];
        }
      }
  }

  // ===================== per-token selection mode ===========================
  const int cand_end = t0 + ntok - W;  // candidates of the last token are [0, cand_end)
  const int n_kt2 = cand_end > 0 ? ceil_div(cand_end, kKeyTile) : 0;
  if (tid < TOK) {
    const int t = t0 + tid;
    const int n_c = t - W + 1;
    const int Kt = row_budget(K, p.k_end, t, L);
    int mode = kModeTrivial;
    if (tid < ntok && Kt > 0 && n_c > Kt) {
      if (p.block) mode = kModeEmit;  // block scores: one entry per candidate block, no sample
      else if (p.flags & 1u) mode = kModeExact;
      else if (n_c <= p.cand_cap) mode = kModeEmit;
      else mode = kModeSample;
    }
    sm.mode[tid] = mode;
    sm.tau[tid] = 0.f;
    sm.cnt[tid] = 0;
  }
  if (tid == 0) { sm.any_sample = 0; sm.any_emit = 0; }
  for (int i = tid; i < TOK * (kBins / 2); i += kSelThreads) (&sm.u.s.hist[0][0])[i] = 0u;
  __syncthreads();
  if (tid < TOK) {
    if (sm.mode[tid] == kModeSample) atomicOr(&sm.any_sample, 1);
    if (sm.mode[tid] == kModeEmit) atomicOr(&sm.any_emit, 1);
  }
  __syncthreads();
  load_nref();

  // Histogram range: 8 bins per octave below G/K_t (the largest a K_t-th score
  // can be; K_t >= k_end); with key weights, below G * max weight / k_end.
  int bin_base = p.bin_base;
  if (p.vw) {
    const float top = (float)G * __uint_as_float(p.vwmax[seq * Hkv + g]) / (float)max(1, p.k_end);
    bin_base = (int)(__float_as_uint(top) >> 20) - (kBins - 1);
  }
  // output-aware metric: the log2 weight of the lane's key (column lc of tile ct)
  // enters every head's exponent, so S comes out multiplied by the key's weight
  const bool wts = p.vw != nullptr;
  float lw[4] = {0.f, 0.f, 0.f, 0.f};
  auto read_weights = [&](int buf) HS2_INLINE {
    if (!wts) return;
#pragma unroll
    for (int ct = 0; ct < 4; ct++) lw[ct] = sm.lw[buf][w][16 * ct + lc];
  };

  // group scores of accumulator tile (rt, ct): S[u] for the lane's tokens
  auto group_scores = [&](int rt, int ct, float (&S)[NT]) HS2_INLINE {
    float e[4];
#pragma unroll
    for (int i = 0; i < 4; i++) e[i] = fast_exp2(fmaf(acc[rt][ct][i], c, lw[ct]));
    if constexpr (G == 1) {
#pragma unroll
      for (int u = 0; u < 4; u++) S[u] = e[u];
    } else if constexpr (G == 2) {
      S[0] = e[0] + e[1];
      S[1] = e[2] + e[3];
    } else {
      float s = (e[0] + e[1]) + (e[2] + e[3]);
      if constexpr (G >= 8) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s),
                                                         false, false);
        s = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      if constexpr (G >= 16) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s),
                                                         false, false);
        s = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      S[0] = s;
    }
  };

  // ========================= sweep 2: sample ================================
  if (sm.any_sample) {
    // which of the lane's tokens take part, and their last candidate key, read once:
    // the modes do not change during this sweep, and reading them between the
    // histogram atomics would make every key group wait for the previous atomics
    bool samp[RT][NT];
    int jlim[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int u = 0; u < NT; u++) {
        const int tl = token_of(rt, u);
        samp[rt][u] = owner && tl < TOK && sm.mode[tl] == kModeSample;
        jlim[rt][u] = t0 + tl - W;
      }
    sweep(ceil_div(n_kt2, kSampleStride), 0, kSampleStride, cand_end, Pair{}, wts,
          [&](int kt, int buf) HS2_INLINE {
      read_weights(buf);
      compute(buf);
      // every group score and bin of the tile first, then the atomics
      uint32_t addr[RT][4][NT], inc[RT][4][NT];
#pragma unroll
      for (int rt = 0; rt < RT; rt++) {
#pragma unroll
        for (int ct = 0; ct < 4; ct++) {
          float S[NT];
          group_scores(rt, ct, S);
          const int j = kt * kKeyTile + 16 * ct + lc;
#pragma unroll
          for (int u = 0; u < NT; u++) {
            const int tl = token_of(rt, u);
            int bin = (int)(__float_as_uint(S[u]) >> 20) - bin_base;
            bin = min(max(bin, 0), kBins - 1);
            addr[rt][ct][u] = (uint32_t)(tl * (kBins / 2) + (bin >> 1));
            inc[rt][ct][u] = (samp[rt][u] && j <= jlim[rt][u]) ? ((bin & 1) ? 65536u : 1u) : 0u;
          }
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int ct = 0; ct < 4; ct++)
#pragma unroll
          for (int u = 0; u < NT; u++)
            if (inc[rt][ct][u]) atomicAdd(&sm.u.s.hist[0][0] + addr[rt][ct][u], inc[rt][ct][u]);
    });
    // threshold: interpolated where the sample's top count reaches r
    if (tid < TOK && sm.mode[tid] == kModeSample) {
      const int t = t0 + tid, n_c = t - W + 1;
      const int Kt = row_budget(K, p.k_end, t, L);
      int n_s = 0;
      for (int kt = 0; kt < n_kt2; kt += kSampleStride) n_s += min(max(n_c - kt * kKeyTile, 0), kKeyTile);
      const int r = (int)ceilf(kTauAlpha * (float)Kt * (float)n_s / (float)n_c) + kTauBeta;
      int mode = kModeExact;
      float tau = 0.f;
      if (r <= n_s) {
        int cum = 0;
        for (int b = kBins - 1; b >= 1; b--) {
          const uint32_t wd = sm.u.s.hist[tid][b >> 1];
          const int h = (b & 1) ? (int)(wd >> 16) : (int)(wd & 0xFFFFu);
          cum += h;
          if (cum >= r) {
            // the r-th sample lies (r - (cum - h)) / h deep into bin b from its top;
            // interpolate linearly in the bit pattern (bins are 1/8 octave)
            const float depth = (float)(r - (cum - h)) / (float)h;
            const uint32_t lo_bits = (uint32_t)(b + bin_base) << 20;
            tau = __uint_as_float(lo_bits + (uint32_t)((1.f - depth) * (float)(1u << 20)));
            mode = kModeEmit;
            break;
          }
        }
      }
      sm.mode[tid] = mode;
      sm.tau[tid] = tau;
      if (mode == kModeEmit) atomicOr(&sm.any_emit, 1);
    }
    __syncthreads();
  }

  // ================= block mode: the score of every candidate block =========
  // Block kt (keys 64 kt .. 64 kt + 63, one key tile) of token t scores the sum
  // of S over its candidate keys j <= t - W; every token with n_c > K gets one
  // entry (score bits << 32 | kt) per candidate block, ranked by the top-K kernel.
  if (p.block && sm.any_emit) {
    uint64_t* cand = p.cand;
    const int C = p.cand_cap;
    sweep(n_kt2, 0, 1, cand_end, Ring{}, wts, [&](int kt, int buf) HS2_INLINE {
      read_weights(buf);
      compute(buf);
#pragma unroll
      for (int rt = 0; rt < RT; rt++) {
        float bsum[NT];
#pragma unroll
        for (int u = 0; u < NT; u++) bsum[u] = 0.f;
#pragma unroll
        for (int ct = 0; ct < 4; ct++) {
          float S[NT];
          group_scores(rt, ct, S);
          const int j = kt * kKeyTile + 16 * ct + lc;
#pragma unroll
          for (int u = 0; u < NT; u++)
            if (j <= t0 + token_of(rt, u) - W) bsum[u] += S[u];
        }
#pragma unroll
        for (int u = 0; u < NT; u++) {
          float b = bsum[u];
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) b += shfl_xor_f(b, off);  // the token's 16 key lanes
          const int tl = token_of(rt, u);
          if (owner && lc == 0 && tl < TOK && sm.mode[tl] == kModeEmit &&
              kt * kKeyTile <= t0 + tl - W)
            cand[(size_t)(slot0 + tl) * C + kt] = ((uint64_t)__float_as_uint(b) << 32) | (uint32_t)kt;
        }
      }
    });
    if (tid < TOK && sm.mode[tid] == kModeEmit) sm.cnt[tid] = ceil_div(t0 + tid - W + 1, kKeyTile);
    __syncthreads();
  }

  // ================= dense rows: every candidate's score (exact path) ========
  if constexpr (DENSE) {
    if (n_kt2 > 0) {
      sweep(n_kt2, 0, 1, cand_end, Ring{}, wts, [&](int kt, int buf) HS2_INLINE {
        read_weights(buf);
        compute(buf);
#pragma unroll
        for (int rt = 0; rt < RT; rt++) {
#pragma unroll
          for (int ct = 0; ct < 4; ct++) {
            float S[NT];
            group_scores(rt, ct, S);
            const int j = kt * kKeyTile + 16 * ct + lc;
#pragma unroll
            for (int u = 0; u < NT; u++) {
              const int tl = token_of(rt, u);
              if (owner && tl < TOK && sm.mode[tl] == kModeExact && j <= t0 + tl - W)
                p.dense_out[(size_t)(slot0 + tl) * p.dense_ld + j] = S[u];
            }
          }
        }
      });
    }
  }

  // ========================= sweep 3: collect ===============================
  if (!p.block && sm.any_emit) {
    float tau_r[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int u = 0; u < NT; u++) {
        const int tl = token_of(rt, u);
        const bool emit = owner && tl < TOK && sm.mode[tl] == kModeEmit;
        tau_r[rt][u] = emit ? sm.tau[tl] : INFINITY;
      }
    // per (row tile, token): the last candidate position and the candidate row
    int lim_r[RT][NT];
    uint2* dst_r[RT][NT];
    const int C = p.cand_cap;
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int u = 0; u < NT; u++) {
        const int tl = token_of(rt, u);
        lim_r[rt][u] = t0 + tl - W;
        dst_r[rt][u] = reinterpret_cast<uint2*>(p.cand + (size_t)(slot0 + min(tl, TOK - 1)) * C);
      }
    // per (row tile, token): the candidates appended so far. A token's keys all sit in
    // the 16 lanes of one row group of one wave, so each lane's first slot is the
    // count so far plus a prefix sum over that row (no LDS atomics); every lane of the
    // row keeps the same count.
    int cnt_r[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int u = 0; u < NT; u++) cnt_r[rt][u] = 0;
    sweep(n_kt2, 0, 1, cand_end, Ring{}, wts, [&](int kt, int buf) HS2_INLINE {
      read_weights(buf);
      compute(buf);
      int jc[4];
#pragma unroll
      for (int ct = 0; ct < 4; ct++) jc[ct] = kt * kKeyTile + 16 * ct + lc;
#pragma unroll
      for (int rt = 0; rt < RT; rt++) {
        float Sv[4][NT];
        bool ok[4][NT];
#pragma unroll
        for (int ct = 0; ct < 4; ct++) {
          group_scores(rt, ct, Sv[ct]);
          // both tests always evaluated (no short circuit): S >= tau, key a candidate
#pragma unroll
          for (int u = 0; u < NT; u++)
            ok[ct][u] = (Sv[ct][u] >= tau_r[rt][u]) & (jc[ct] <= lim_r[rt][u]);
        }
        // the lane's (up to 4) passing keys go to consecutive slots after those of the
        // lanes before it in the row; an entry is stored as the words (position, S
        // bits), i.e. (S bits << 32) | position
#pragma unroll
        for (int u = 0; u < NT; u++) {
          const int n = (int)ok[0][u] + (int)ok[1][u] + (int)ok[2][u] + (int)ok[3][u];
          const int incl = row_incl_scan(n);
          int pos = cnt_r[rt][u] + incl - n;
          cnt_r[rt][u] += __shfl(incl, l | 15, 64);  // the row's total
#pragma unroll
          for (int ct = 0; ct < 4; ct++) {
            if (ok[ct][u]) {
              if (pos < C) dst_r[rt][u][pos] = make_uint2((uint32_t)jc[ct], __float_as_uint(Sv[ct][u]));
              pos++;
            }
          }
        }
      }
    });
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int u = 0; u < NT; u++) {
        const int tl = token_of(rt, u);
        if (owner && lc == 0 && sm.mode[tl] == kModeEmit) sm.cnt[tl] = cnt_r[rt][u];
      }
    __syncthreads();
  }

  // ============================ row verdicts ================================
  if (tid < TOK) {
    const int mode = sm.mode[tid];
    int count = 0;
    if (mode == kModeExact) {
      count = -1;
    } else if (mode == kModeEmit) {
      count = sm.cnt[tid];
      // block mode: ceil(n_c / 64) > K / 64 block entries, always within C
      if (!p.block && (count > p.cand_cap || count < row_budget(K, p.k_end, t0 + tid, L)))
        count = -1;
    }
    p.cand_count[slot0 + tid] = count;
    if (count < 0 || (p.list_rank && mode == kModeEmit)) {
      const int f = atomicAdd(p.flag_count, 1);
      p.flag_list[f] = (int32_t)(slot0 + tid);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode step, logits. Sequence b's query (its newest token, at position
// L_b - 1) against every cached key: z2[j, h] = c * <q[b,h], k[j,g]> for the
// group's heads, written to p.z2 in the [Hkv, T, G] layout (each group's run
// is contiguous for the selection kernels' reads), and per split the
// (max, sum of exp2(z2 - max)) of each head, from which decode_tau_kernel forms
// the full layer's log-sum-exp. Grid (split, g, b): p.split_len keys per
// workgroup, 4 waves x 16 keys per step on v_mfma_f32_16x16x32_bf16 with the
// group's G heads as the 16-row A operand (rows >= G are zero).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void merge_max_sum(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  s = s * fast_exp2(m - mn) + s2 * fast_exp2(m2 - mn);
  m = mn;
}

template <int G, bool FP8>
__global__ __launch_bounds__(256) void decode_logits_kernel(DecodeParams p) {
  __shared__ float2 red[4][16];
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int base = p.cu[b], L = p.cu[b + 1] - base;
  const int j0 = split * p.split_len;
  if (j0 >= L) return;  // the whole workgroup: this split is past the sequence
  const int j1 = min(L, j0 + p.split_len);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l >> 4, lc = l & 15;
  const int Hq = p.Hq, Hkv = p.Hkv;
  const float c = p.c;

  // A operand: row lc = head lc of the group, d = 32 ks + 8 lq .. +7
  bf16x8 qa[4];
  {
    const uint16_t* qrow = p.q + ((size_t)b * Hq + g * G + min(lc, G - 1)) * kHeadDim;
    u32x4 v[4];
#pragma unroll
    for (int ks = 0; ks < 4; ks++) v[ks] = to_u32x4(ldg128(qrow + 32 * ks + 8 * lq));
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      if (lc >= G) v[ks] = u32x4{0u, 0u, 0u, 0u};
      qa[ks] = as_bf16x8(v[ks]);
    }
  }
  // running (max, sum) of rows (heads) 4 lq + i over the lane's keys
  float m[4], sm[4];
#pragma unroll
  for (int i = 0; i < 4; i++) { m[i] = -INFINITY; sm[i] = 0.f; }
  const size_t kstride = (size_t)Hkv * kHeadDim;  // elements per cached token
  const size_t kbase = ((size_t)base * Hkv + g) * kHeadDim;
  // B operand: key jt + lc (clamped to the split; masked below), d = 32 ks + 8 lq:
  // 16 bytes of a bf16 row, or 8 bytes of an FP8 one widened exactly to bf16.
  // The next step's rows are in flight while this step computes (the loads are
  // unconditional, clamped, so the compiler's wait leaves them in flight).
  using Raw = std::conditional_t<FP8, uint2, uint4>;
  auto load_keys = [&](int jt, Raw (&kv)[4]) {
    const size_t row = kbase + (size_t)min(jt + lc, j1 - 1) * kstride;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      if constexpr (FP8) kv[ks] = ldg64(p.k8 + row + 32 * ks + 8 * lq);
      else kv[ks] = ldg128(p.k + row + 32 * ks + 8 * lq);
    }
  };
  auto widen = [&](const Raw& x) HS2_INLINE -> u32x4 {
    if constexpr (FP8)
      return u32x4{e4m3x2_to_bf16x2<false>(x.x), e4m3x2_to_bf16x2<true>(x.x),
                   e4m3x2_to_bf16x2<false>(x.y), e4m3x2_to_bf16x2<true>(x.y)};
    else
      return to_u32x4(x);
  };
  Raw kn[4];
  load_keys(j0 + 16 * w, kn);
  for (int jt = j0 + 16 * w; jt < j1; jt += 64) {
    u32x4 kv[4];
#pragma unroll
    for (int ks = 0; ks < 4; ks++) kv[ks] = widen(kn[ks]);
    load_keys(jt + 64, kn);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ks++) acc = mfma16x16x32(qa[ks], as_bf16x8(kv[ks]), acc);
    const bool kval = jt + lc < j1;
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; i++) z[i] = kval ? acc[i] * c : -INFINITY;
    if (kval && 4 * lq < G) {  // heads 4 lq .. of key jt + lc
      float* dst = p.z2 + ((size_t)g * p.T + base + jt + lc) * G + 4 * lq;
      if constexpr (G >= 4) {
        *reinterpret_cast<float4*>(dst) = make_float4(z[0], z[1], z[2], z[3]);
      } else {
#pragma unroll
        for (int i = 0; i < G; i++) dst[i] = z[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) merge_max_sum(m[i], sm[i], z[i], kval ? 1.f : 0.f);
  }
  // the 16 lanes of a lane group hold the same heads: merge them, then the waves
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const float m2 = shfl_xor_f(m[i], off), s2 = shfl_xor_f(sm[i], off);
      merge_max_sum(m[i], sm[i], m2, s2);
    }
    if (lc == 0) red[w][4 * lq + i] = make_float2(m[i], sm[i]);
  }
  __syncthreads();
  if (tid < G) {
    float mm = -INFINITY, ss = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ww++) merge_max_sum(mm, ss, red[ww][tid].x, red[ww][tid].y);
    p.part[(((size_t)b * Hkv + g) * p.n_split + split) * G + tid] = make_float2(mm, ss);
  }
}

template <bool FP8>
static hipError_t launch_decode_logits_t(int G, const DecodeParams& p, hipStream_t s) {
  if (p.B <= 0) return hipSuccess;
  const dim3 grid(p.n_split, p.Hkv, p.B), block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_logits_kernel<1, FP8>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_logits_kernel<2, FP8>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_logits_kernel<4, FP8>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((decode_logits_kernel<8, FP8>), grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL((decode_logits_kernel<16, FP8>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_logits(int G, const DecodeParams& p, hipStream_t s) {
  return p.k8 ? launch_decode_logits_t<true>(G, p, s) : launch_decode_logits_t<false>(G, p, s);
}

template <int G>
static void launch_scores_g(bool dense, dim3 grid, dim3 block, const ScoreParams& p,
                            hipStream_t s) {
  if (dense) hipLaunchKernelGGL((scores_kernel<G, true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((scores_kernel<G, false>), grid, block, 0, s, p);
}

hipError_t launch_scores(int G, const ScoreParams& p, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  dim3 grid(n_blocks), block(kSelThreads);
  const bool dense = p.dense_out != nullptr;
  switch (G) {
    case 1: launch_scores_g<1>(dense, grid, block, p, s); break;
    case 2: launch_scores_g<2>(dense, grid, block, p, s); break;
    case 4: launch_scores_g<4>(dense, grid, block, p, s); break;
    case 8: launch_scores_g<8>(dense, grid, block, p, s); break;
    case 16: launch_scores_g<16>(dense, grid, block, p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hs2
