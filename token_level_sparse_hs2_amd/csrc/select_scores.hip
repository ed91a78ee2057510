// select_scores.hip - the full-attention layer's scoring sweeps on gfx950.
//
// One workgroup owns TOK consecutive query tokens of one sequence and one KV
// group g (all G query heads of the group: 64*RT MFMA rows, token-major,
// head-minor, so a lane's accumulator rows are the heads of one token). It
// sweeps the causal keys in 64-key tiles staged through LDS, with bf16 MFMA
// QK^T tiles and fp32 accumulation, three times:
//
//  1. row statistics: per (t, h) the max m and sum l of exp over all causal
//     keys (online, log2 domain), giving lse2 = m + log2 l. The full layer's
//     softmax is taken over all causal keys, scale 1/sqrt(d) (attention as in
//     the SHARP walkthrough, section 1.1).
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
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

enum : int { kModeTrivial = 0, kModeEmit = 1, kModeExact = 2, kModeSample = 3 };

template <int G>
struct ScoreCfg {
  static constexpr int RT = row_tiles(G);
  static constexpr int TOK = tokens_per_task(G);
  static constexpr int ROWS_W = 16 * RT;
  static constexpr int NT = G >= 4 ? 1 : 4 / G;  // tokens per lane per row tile
};

struct ScoreSmem {
  uint4 ktile[2][kKeyTile][16];       // two 64-key x 256-byte tiles (XOR-swizzled chunks)
  uint32_t hist[64][kBins / 2];       // two 16-bit bin counters per word
  float tau[64];
  int32_t cnt[64];
  int32_t mode[64];
  int32_t any_sample, any_emit;
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

template <int G>
__global__ __launch_bounds__(kSelThreads, 2) void scores_kernel(ScoreParams p) {
  using C = ScoreCfg<G>;
  constexpr int RT = C::RT, TOK = C::TOK, ROWS_W = C::ROWS_W, NT = C::NT;
  __shared__ ScoreSmem sm;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int lq = l >> 4, lc = l & 15;
  const int g = blockIdx.x % p.Hkv;
  const int64_t task = p.task_begin + blockIdx.x / p.Hkv;
  int seq, tile;
  plan_decode(p.cu, p.B, TOK, p.max_tiles, task, &seq, &tile);
  const int base = p.cu[seq];
  const int L = p.cu[seq + 1] - base;
  const int t0 = tile * TOK;
  const int ntok = min(TOK, L - t0);
  const int64_t slot0 = (int64_t)blockIdx.x * TOK;
  const int Hq = p.Hq, Hkv = p.Hkv, K = p.K, W = p.W;
  const float c = p.c;

  // ---- Q operands (A): row ra = token-major, head-minor ----
  bf16x8 qa[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; rt++) {
    const int ra = w * ROWS_W + 16 * rt + lc;
    const int ta = ra / G, ha = ra % G;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ta < ntok)
        v = to_u32x4(ldg128(p.q + ((size_t)(base + t0 + ta) * Hq + g * G + ha) * kHeadDim +
                            32 * ks + 8 * lq));
      qa[rt][ks] = as_bf16x8(v);
    }
  }

  const uint16_t* kbase = p.k + (size_t)g * kHeadDim;
  auto load_tile = [&](int kt, int kend, uint4 (&reg)[4]) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int kk = (tid >> 4) + 16 * r;
      const int j = kt * kKeyTile + kk;
      reg[r] = make_uint4(0u, 0u, 0u, 0u);
      if (j < kend) reg[r] = ldg128(kbase + (size_t)(base + j) * Hkv * kHeadDim + (tid & 15) * 8);
    }
  };
  auto store_tile = [&](int buf, const uint4 (&reg)[4]) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int kk = (tid >> 4) + 16 * r;
      sm.ktile[buf][kk][(tid & 15) ^ (kk & 15)] = reg[r];
    }
  };
  f32x4 acc[RT][4];
  auto compute = [&](int buf) {
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int ct = 0; ct < 4; ct++) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < 4; ct++) {
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        const int kk = 16 * ct + lc;
        const bf16x8 b = as_bf16x8(to_u32x4(sm.ktile[buf][kk][(4 * ks + lq) ^ lc]));
#pragma unroll
        for (int rt = 0; rt < RT; rt++) acc[rt][ct] = mfma16x16x32(qa[rt][ks], b, acc[rt][ct]);
      }
    }
  };

  // ======================= sweep 1: row statistics ==========================
  float m_run[RT][4], l_run[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; rt++)
#pragma unroll
    for (int i = 0; i < 4; i++) { m_run[rt][i] = -1e30f; l_run[rt][i] = 0.f; }  // finite: no inf-inf

  {
    const int kend = t0 + ntok;
    const int n_kt = ceil_div(kend, kKeyTile);
    uint4 reg[4];
    load_tile(0, kend, reg);
    store_tile(0, reg);
    __syncthreads();
    constexpr float kSlack = 8.f;  // log2 units a score may exceed the row reference
    for (int kt = 0; kt < n_kt; kt++) {
      if (kt + 1 < n_kt) load_tile(kt + 1, kend, reg);
      compute(kt & 1);
      const bool diag = kt * kKeyTile + kKeyTile - 1 > t0;  // some key may lie beyond a token
      if (diag) {
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int t = t0 + (w * ROWS_W + 16 * rt + 4 * lq + i) / G;
#pragma unroll
            for (int ct = 0; ct < 4; ct++)
              if (kt * kKeyTile + 16 * ct + lc > t) acc[rt][ct][i] = -INFINITY;
          }
      }
      // the row reference m only moves when a score passes it by the slack (so no
      // term exceeds 2^slack); moving it rescales l. Raw accumulators compare
      // directly since the scale c is positive.
      bool move = false;
      float mx[RT][4];
#pragma unroll
      for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          mx[rt][i] = fmaxf(fmaxf(acc[rt][0][i], acc[rt][1][i]), fmaxf(acc[rt][2][i], acc[rt][3][i])) * c;
          move |= mx[rt][i] > m_run[rt][i] + kSlack;
        }
      if (__any(move)) {
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float mn = fmaxf(m_run[rt][i], mx[rt][i]);
            l_run[rt][i] *= fast_exp2(m_run[rt][i] - mn);
            m_run[rt][i] = mn;
          }
      }
#pragma unroll
      for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float mneg = -m_run[rt][i];
          float sum = 0.f;
#pragma unroll
          for (int ct = 0; ct < 4; ct++) sum += fast_exp2(fmaf(acc[rt][ct][i], c, mneg));
          l_run[rt][i] += sum;
        }
      if (kt + 1 < n_kt) store_tile((kt + 1) & 1, reg);
      __syncthreads();
    }
  }

  // combine the 16 lanes that share a row, then lse2 = m + log2(l)
  float lse[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; rt++) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float m = m_run[rt][i], s = l_run[rt][i];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const float mo = shfl_xor_f(m, off), so = shfl_xor_f(s, off);
        const float mn = fmaxf(m, mo);
        const float a = s * fast_exp2(m - mn);  // m, mo finite (>= -1e30)
        const float b = so * fast_exp2(mo - mn);
        s = a + b;
        m = mn;
      }
      lse[rt][i] = m + fast_log2(s);
      const int r = w * ROWS_W + 16 * rt + 4 * lq + i;
      const int tl = r / G, hl = r % G;
      if (lc == 0 && tl < ntok) p.lse2[(size_t)(base + t0 + tl) * Hq + g * G + hl] = lse[rt][i];
    }
  }

  // ===================== per-token selection mode ===========================
  const int cand_end = t0 + ntok - W;  // candidates of the last token are [0, cand_end)
  const int n_kt2 = cand_end > 0 ? ceil_div(cand_end, kKeyTile) : 0;
  if (tid < TOK) {
    const int t = t0 + tid;
    const int n_c = t - W + 1;
    int mode = kModeTrivial;
    if (tid < ntok && K > 0 && n_c > K) {
      if (p.flags & 1u) mode = kModeExact;
      else if (n_c <= p.cand_cap) mode = kModeEmit;
      else mode = kModeSample;
    }
    sm.mode[tid] = mode;
    sm.tau[tid] = 0.f;
    sm.cnt[tid] = 0;
  }
  if (tid == 0) { sm.any_sample = 0; sm.any_emit = 0; }
  for (int i = tid; i < 64 * (kBins / 2); i += kSelThreads) (&sm.hist[0][0])[i] = 0u;
  __syncthreads();
  if (tid < TOK) {
    if (sm.mode[tid] == kModeSample) atomicOr(&sm.any_sample, 1);
    if (sm.mode[tid] == kModeEmit) atomicOr(&sm.any_emit, 1);
  }
  __syncthreads();

  // group score of the lane's token(s) for accumulator (rt, ct); emits per token u
  auto group_scores = [&](int rt, int ct, float (&S)[NT]) {
    float e[4];
#pragma unroll
    for (int i = 0; i < 4; i++) e[i] = fast_exp2(fmaf(acc[rt][ct][i], c, -lse[rt][i]));
    if constexpr (G == 1) {
#pragma unroll
      for (int u = 0; u < NT; u++) S[u] = e[u];
    } else if constexpr (G == 2) {
      S[0] = e[0] + e[1];
      S[1] = e[2] + e[3];
    } else {
      float part = (e[0] + e[1]) + (e[2] + e[3]);
      if constexpr (G >= 8) part += shfl_xor_f(part, 16);
      if constexpr (G >= 16) part += shfl_xor_f(part, 32);
      S[0] = part;
    }
  };
  // local token index of the lane's u-th token in row tile rt; owner lanes only
  auto token_of = [&](int rt, int u) { return (w * ROWS_W + 16 * rt + 4 * lq) / G + u; };
  const bool owner = (G <= 4) || (G == 8 ? ((lq & 1) == 0) : (lq == 0));

  // ========================= sweep 2: sample ================================
  if (sm.any_sample) {
    for (int kt = 0; kt < n_kt2; kt += kSampleStride) {
      uint4 reg[4];
      load_tile(kt, cand_end, reg);
      store_tile(0, reg);
      __syncthreads();
      compute(0);
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
            if (owner && tl < TOK && sm.mode[tl] == kModeSample && j <= t0 + tl - W) {
              int bin = (int)(__float_as_uint(S[u]) >> 20) - p.bin_base;
              bin = min(max(bin, 0), kBins - 1);
              atomicAdd(&sm.hist[tl][bin >> 1], (bin & 1) ? 65536u : 1u);
            }
          }
        }
      }
      __syncthreads();
    }
    // threshold: lower edge of the bin where the top count reaches r
    if (tid < TOK && sm.mode[tid] == kModeSample) {
      const int t = t0 + tid, n_c = t - W + 1;
      int n_s = 0;
      for (int kt = 0; kt < n_kt2; kt += kSampleStride) n_s += min(max(n_c - kt * kKeyTile, 0), kKeyTile);
      const int r = (int)ceilf(kTauAlpha * (float)K * (float)n_s / (float)n_c) + kTauBeta;
      int mode = kModeExact;
      float tau = 0.f;
      if (r <= n_s) {
        int cum = 0;
        for (int b = kBins - 1; b >= 1; b--) {
          const uint32_t wd = sm.hist[tid][b >> 1];
          const int h = (b & 1) ? (int)(wd >> 16) : (int)(wd & 0xFFFFu);
          cum += h;
          if (cum >= r) {
            // the r-th sample lies (r - (cum - h)) / h deep into bin b from its top;
            // interpolate linearly in the bit pattern (bins are 1/8 octave)
            const float depth = (float)(r - (cum - h)) / (float)h;
            const uint32_t lo_bits = (uint32_t)(b + p.bin_base) << 20;
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

  // ========================= sweep 3: collect ===============================
  if (sm.any_emit) {
    float tau_r[RT][NT];
    int nc_r[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
      for (int u = 0; u < NT; u++) {
        const int tl = token_of(rt, u);
        const bool emit = owner && tl < TOK && sm.mode[tl] == kModeEmit;
        tau_r[rt][u] = emit ? sm.tau[tl] : INFINITY;
        nc_r[rt][u] = emit ? t0 + tl - W + 1 : 0;
      }
    uint64_t* cand = p.cand;
    const int C = p.cand_cap;
    uint4 reg[4];
    load_tile(0, cand_end, reg);
    store_tile(0, reg);
    __syncthreads();
    for (int kt = 0; kt < n_kt2; kt++) {
      if (kt + 1 < n_kt2) load_tile(kt + 1, cand_end, reg);
      compute(kt & 1);
#pragma unroll
      for (int rt = 0; rt < RT; rt++) {
        float Sv[4][NT];
        uint32_t pass[NT];
#pragma unroll
        for (int u = 0; u < NT; u++) pass[u] = 0u;
#pragma unroll
        for (int ct = 0; ct < 4; ct++) {
          float S[NT];
          group_scores(rt, ct, S);
          const int j = kt * kKeyTile + 16 * ct + lc;
#pragma unroll
          for (int u = 0; u < NT; u++) {
            Sv[ct][u] = S[u];
            pass[u] |= (S[u] >= tau_r[rt][u] && j < nc_r[rt][u]) ? (1u << ct) : 0u;
          }
        }
        // one LDS atomic per lane and token for its (up to 4) passing keys
#pragma unroll
        for (int u = 0; u < NT; u++) {
          if (pass[u]) {
            const int tl = token_of(rt, u);
            int pos = atomicAdd(&sm.cnt[tl], __popc(pass[u]));
            uint64_t* dst = cand + (size_t)(slot0 + tl) * C;
#pragma unroll
            for (int ct = 0; ct < 4; ct++) {
              if ((pass[u] >> ct) & 1u) {
                if (pos < C)
                  dst[pos] = ((uint64_t)__float_as_uint(Sv[ct][u]) << 32) |
                             (uint32_t)(kt * kKeyTile + 16 * ct + lc);
                pos++;
              }
            }
          }
        }
      }
      if (kt + 1 < n_kt2) store_tile((kt + 1) & 1, reg);
      __syncthreads();
    }
  }

  // ============================ row verdicts ================================
  if (tid < TOK) {
    const int mode = sm.mode[tid];
    int count = 0;
    if (mode == kModeExact) {
      count = -1;
    } else if (mode == kModeEmit) {
      count = sm.cnt[tid];
      if (count > p.cand_cap || count < K) count = -1;
    }
    p.cand_count[slot0 + tid] = count;
    if (count < 0) {
      const int f = atomicAdd(p.flag_count, 1);
      p.flag_list[f] = (int32_t)(slot0 + tid);
    }
  }
}

hipError_t launch_scores(int G, const ScoreParams& p, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  dim3 grid(n_blocks), block(kSelThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL(scores_kernel<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(scores_kernel<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(scores_kernel<4>, grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL(scores_kernel<8>, grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL(scores_kernel<16>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hs2
