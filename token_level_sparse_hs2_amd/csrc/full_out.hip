// full_out.hip - the full-attention layer's own output on gfx950.
//
// The full layer of a hybrid module is a real attention layer (HySparse2 news
// summary, two-level KV sharing paragraph: the full-attention layers keep their
// own projections and outputs; its scores also pick the sparse layers' tokens):
//   o[t,h] = sum_{j <= t} P[t,h,j] v[j,g],  P = softmax_j(scale <q[t,h], k[j,g]>)
// (attention as in the SHARP walkthrough, section 1.1). One sweep over the causal
// keys with a running maximum per row (log2 domain, moved lazily: only when a
// 64-key tile passes it by 2^8, which rescales the row's sum and output), and
// the row's log2-domain log-sum-exp lse2 = m + log2(sum) written as a by-product:
// the selection then takes its row statistics from here and skips its own
// statistics sweep, so the full layer's output costs one QK^T pass, not two.
//
// One workgroup owns TOK tokens of one sequence and one KV group: 4 wavefronts
// x 32 MFMA rows (token-major, head-minor). Each 64-key tile of K and of V
// streams into a 2-slot LDS ring with global_load_lds (16-byte chunks
// XOR-swizzled by which chunk each lane fetches). Per wave and tile:
//   S^T = K Q^T (keys x rows), v_mfma_f32_16x16x32_bf16, A = K from LDS, B = Q
//   in registers;
//   P^T = exp2(c S^T - m) in the accumulator layout; two 16-key subtiles side by
//   side are the B operand of one v_mfma_f32_16x16x32_bf16 (its k slots taken in
//   the order those scores sit in the accumulators);
//   O^T += V^T P^T with V^T read transposed from LDS (ds_read_b64_tr_b16), the
//   A operand's k slots in the same key order.
// P enters as one bf16 part for bf16 output and three (~24 bits) for fp32.
#include <type_traits>

#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

namespace {

constexpr int kOutRT = 2;                  // 16-row tiles per wave
constexpr int kOutRowsW = 16 * kOutRT;     // MFMA rows per wave
constexpr int kOutSlots = 2;               // ring depth (K and V each)


struct OutSmem {
  uint4 k[kOutSlots][kKeyTile][16];  // K rows: chunk c of key r at c ^ (r & 15)
  uint4 v[kOutSlots][kKeyTile][16];  // V rows: chunk c of key r at c ^ (2 (r & 7))
};

}  // namespace

template <int G, bool PRECISE>
__global__ __launch_bounds__(256, 2) void full_out_kernel(FullOutParams p) {
  constexpr int TOK = full_out_tokens(G);
  constexpr int NSPLIT = PRECISE ? 3 : 1;
  __shared__ OutSmem sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int lq = l >> 4, lc = l & 15;
  const int g = blockIdx.x % p.Hkv;
  int seq, tile;
  plan_decode(p.cu, p.B, TOK, p.max_tiles, blockIdx.x / p.Hkv, &seq, &tile);
  const int base = p.cu[seq];
  const int L = p.cu[seq + 1] - base;
  const int t0 = tile * TOK;
  const int ntok = min(TOK, L - t0);
  const int Hq = p.Hq, Hkv = p.Hkv;
  const float c = p.c;

  // B operand Q^T: column = row (lc) of row tile rt, k = d chunk 4 ks + lq (rows
  // past the sequence take zero queries and are not written)
  bf16x8 qb[kOutRT][4];
  {
    u32x4 v[kOutRT][4];
#pragma unroll
    for (int rt = 0; rt < kOutRT; rt++) {
      const int row = w * kOutRowsW + 16 * rt + lc;
      const int ta = min(row / G, ntok - 1), ha = row % G;
#pragma unroll
      for (int ks = 0; ks < 4; ks++)
        v[rt][ks] = to_u32x4(ldg128(p.q + ((size_t)(base + t0 + ta) * Hq + g * G + ha) * kHeadDim +
                                    32 * ks + 8 * lq));
    }
#pragma unroll
    for (int rt = 0; rt < kOutRT; rt++) {
      const bool live = (w * kOutRowsW + 16 * rt + lc) / G < ntok;
#pragma unroll
      for (int ks = 0; ks < 4; ks++) qb[rt][ks] = as_bf16x8(live ? v[rt][ks] : u32x4{0u, 0u, 0u, 0u});
    }
  }

  // ---- K / V tiles: global -> LDS ring, waits by vmcnt (loads complete in order) ----
  const size_t row_elems = (size_t)Hkv * kHeadDim;
  const uint16_t* kbase = p.k + (size_t)base * row_elems + (size_t)g * kHeadDim;
  const uint16_t* vbase = p.v + (size_t)base * row_elems + (size_t)g * kHeadDim;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t lds_k = (uint32_t)(uintptr_t)&sm.k[0][0][0];
  const uint32_t lds_v = (uint32_t)(uintptr_t)&sm.v[0][0][0];
  const int kend = t0 + ntok;  // keys [0, kend) cover every row's causal range
  // A whole tile (keys below kend) loads from a wave-uniform tile base in SGPRs plus
  // fixed 32-bit lane offsets, so the addresses cost no vector ALU work per tile;
  // only the last, partial tile clamps each key to kend - 1 (those keys are masked).
  const size_t row_bytes = row_elems * sizeof(uint16_t);
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int key = 16 * w + 4 * r + lq;
    koff[r] = (uint32_t)(key * row_bytes) + 16u * (lc ^ (key & 15));
    voff[r] = (uint32_t)(key * row_bytes) + 16u * (lc ^ (2 * (key & 7)));
  }
  auto dma_tile = [&](int kt, int buf) HS2_INLINE {
    if (kt * kKeyTile + kKeyTile <= kend) {
      const size_t tb = (size_t)kt * kKeyTile * row_bytes;
      const uint16_t* kt_base = uniform_ptr(reinterpret_cast<const uint16_t*>(
          reinterpret_cast<const char*>(kbase) + tb));
      const uint16_t* vt_base = uniform_ptr(reinterpret_cast<const uint16_t*>(
          reinterpret_cast<const char*>(vbase) + tb));
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const uint32_t off = (uint32_t)(buf * kKeyTile + 16 * wu + 4 * r) * 256u;
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(koff[r]), "s"(kt_base),
                     "{m0}"(lds_k + off) : "memory");
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff[r]), "s"(vt_base),
                     "{m0}"(lds_v + off) : "memory");
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int key = 16 * w + 4 * r + lq;
        const int j = min(kt * kKeyTile + key, kend - 1);
        const uint16_t* ks = kbase + (size_t)j * row_elems + 8 * (lc ^ (key & 15));
        const uint16_t* vs = vbase + (size_t)j * row_elems + 8 * (lc ^ (2 * (key & 7)));
        const uint32_t off = (uint32_t)(buf * kKeyTile + 16 * wu + 4 * r) * 256u;
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(ks), "{m0}"(lds_k + off) : "memory");
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(vs), "{m0}"(lds_v + off) : "memory");
      }
    }
  };
  auto lds_barrier = [&]() HS2_INLINE {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  constexpr float kRescaleSlack = 8.f;  // log2 units the running maximum may lag behind
  f32x4 o[8][kOutRT];
  float lsum[kOutRT] = {};
  float m[kOutRT] = {};  // set from the first tile
#pragma unroll
  for (int dt = 0; dt < 8; dt++)
#pragma unroll
    for (int rt = 0; rt < kOutRT; rt++) o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_kt = ceil_div(kend, kKeyTile);
  dma_tile(0, 0);
  for (int kt = 0; kt < n_kt; kt++) {
    const int buf = kt & 1;
    // tile kt landed (the 8 loads of tile kt + 1, issued below, may stay in flight)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): only tile kt is outstanding here
    lds_barrier();
    if (kt + 1 < n_kt) dma_tile(kt + 1, buf ^ 1);
    const bool diag = kt * kKeyTile + kKeyTile - 1 > t0;
    // S^T of the tile's four 16-key subtiles (keys 16 kk + 4 lq + i, row lc of each
    // row tile) in the log2 domain relative to the row's running maximum m:
    // z = c S - m, then keys past a row's token at -inf
    f32x4 z[4][kOutRT];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const int kr = 16 * kk + lc;  // A operand row (key) of this lane
      bf16x8 ka[4];
#pragma unroll
      for (int ks = 0; ks < 4; ks++) ka[ks] = as_bf16x8(to_u32x4(sm.k[buf][kr][(4 * ks + lq) ^ (kr & 15)]));
#pragma unroll
      for (int rt = 0; rt < kOutRT; rt++) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ks++) acc = mfma16x16x32(ka[ks], qb[rt][ks], acc);
#pragma unroll
        for (int i = 0; i < 4; i++) z[kk][rt][i] = fmaf(acc[i], c, -m[rt]);
      }
    }
    if (diag) {  // only the last tile or two hold keys past some row's token
      asm volatile("");  // keeps this a branch: selects on every tile cost ~90 VALU ops
#pragma unroll
      for (int rt = 0; rt < kOutRT; rt++) {
        const int t = t0 + (w * kOutRowsW + 16 * rt + lc) / G;
#pragma unroll
        for (int kk = 0; kk < 4; kk++)
#pragma unroll
          for (int i = 0; i < 4; i++)
            if (kt * kKeyTile + 16 * kk + 4 * lq + i > t) z[kk][rt][i] = -INFINITY;
      }
    }
    // the row's maximum over the tile relative to m (16 values per lane, then its 4
    // lane groups). The first tile sets m to the row's exact maximum there (key 0 is
    // in it for every row, so that is finite); later tiles move m only when a score
    // passes it by the slack, rescaling the row's sum and output.
#pragma unroll
    for (int rt = 0; rt < kOutRT; rt++) {
      const float a0 = max3_f32(z[0][rt][0], z[0][rt][1], z[0][rt][2]);
      const float a1 = max3_f32(z[0][rt][3], z[1][rt][0], z[1][rt][1]);
      const float a2 = max3_f32(z[1][rt][2], z[1][rt][3], z[2][rt][0]);
      const float a3 = max3_f32(z[2][rt][1], z[2][rt][2], z[2][rt][3]);
      const float a4 = max3_f32(z[3][rt][0], z[3][rt][1], z[3][rt][2]);
      float mx = max3_f32(max3_f32(a0, a1, a2), max3_f32(a3, a4, z[3][rt][3]), -INFINITY);
      mx = max_xor32_raw(max_xor16_raw(mx));
      const bool first = kt == 0;
      if (first || __any(mx > kRescaleSlack)) {
        const float dm = first ? mx : fmaxf(mx, 0.f);
        if (!first) {
          const float alpha = fast_exp2(-dm);
          lsum[rt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 8; dt++) o[dt][rt] *= alpha;
        }
        m[rt] += dm;
#pragma unroll
        for (int kk = 0; kk < 4; kk++) z[kk][rt] -= dm;
      }
    }
#pragma unroll
    for (int kp = 0; kp < 2; kp++) {  // pairs of 16-key subtiles: 32 keys per MFMA
      // P^T as the B operand of the 16x16x32 product: k slot 4 h + i of lane group lq
      // holds key 16 (2 kp + h) + 4 lq + i, the accumulator position of that score
      uint32_t pk[kOutRT][NSPLIT][4];
#pragma unroll
      for (int rt = 0; rt < kOutRT; rt++) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
          float pv[4];
#pragma unroll
          for (int i = 0; i < 4; i++) pv[i] = fast_exp2(z[2 * kp + h][rt][i]);
          lsum[rt] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
#pragma unroll
          for (int part = 0; part < NSPLIT; part++) {
            const uint32_t lo = pack_bf16x2(pv[0], pv[1]), hi = pack_bf16x2(pv[2], pv[3]);
            pk[rt][part][2 * h] = lo;
            pk[rt][part][2 * h + 1] = hi;
            if (part + 1 < NSPLIT) {
              pv[0] -= bf16_bits_to_f32(lo & 0xFFFFu);
              pv[1] -= __uint_as_float(lo & 0xFFFF0000u);
              pv[2] -= bf16_bits_to_f32(hi & 0xFFFFu);
              pv[3] -= __uint_as_float(hi & 0xFFFF0000u);
            }
          }
        }
      }
      // O^T += V^T P^T: the A operand's k slots 4 h + e are V[16 (2 kp + h) + 4 lq + e]
      // [16 dt + lc], one transposing read per half: lane j of the group addresses key
      // 16 (2 kp + h) + 4 lq + (j >> 2), d = 16 dt + 4 (j & 3)
#pragma unroll
      for (int dt = 0; dt < 8; dt++) {
        const int d0 = 16 * dt + 4 * (lc & 3);
        uint2 hv[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int key = 16 * (2 * kp + h) + 4 * lq + (lc >> 2);
          const int phys = (d0 >> 3) ^ (2 * (key & 7));
          const short* src = reinterpret_cast<const short*>(&sm.v[buf][key][phys]) + (d0 & 7);
          hv[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                (s16x4 __attribute__((address_space(3)))*)(src)));
        }
        const bf16x8 va = as_bf16x8(u32x4{hv[0].x, hv[0].y, hv[1].x, hv[1].y});
#pragma unroll
        for (int rt = 0; rt < kOutRT; rt++)
#pragma unroll
          for (int part = 0; part < NSPLIT; part++)
            o[dt][rt] = mfma16x16x32(va, as_bf16x8(u32x4{pk[rt][part][0], pk[rt][part][1],
                                                         pk[rt][part][2], pk[rt][part][3]}),
                                     o[dt][rt]);
      }
    }
  }

  // lane holds O^T[d = 16 dt + 4 lq + i][row lc of each row tile]; a row's keys
  // are spread over the 4 lane groups
#pragma unroll
  for (int rt = 0; rt < kOutRT; rt++) {
    float ls = lsum[rt];
    ls += shfl_xor_f(ls, 16);
    ls += shfl_xor_f(ls, 32);
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) o[dt][rt] *= inv;
    // the row's log2-domain log-sum-exp, for the selection
    const int row = w * kOutRowsW + 16 * rt + lc;
    if (p.lse2 && lq == 0 && row / G < ntok)
      p.lse2[(size_t)(base + t0 + row / G) * Hq + g * G + row % G] = m[rt] + fast_log2(ls);
  }
#pragma unroll
  for (int rt = 0; rt < kOutRT; rt++) {
    const int row = w * kOutRowsW + 16 * rt + lc;
    if (row / G >= ntok) continue;
    const size_t ob = ((size_t)(base + t0 + row / G) * Hq + g * G + row % G) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      const int d0 = 16 * dt + 4 * lq;
      if constexpr (PRECISE) {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + ob + d0) =
            make_float4(o[dt][rt][0], o[dt][rt][1], o[dt][rt][2], o[dt][rt][3]);
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + ob + d0) =
            make_uint2(pack_bf16x2(o[dt][rt][0], o[dt][rt][1]), pack_bf16x2(o[dt][rt][2], o[dt][rt][3]));
      }
    }
  }
}

template <int G>
static hipError_t launch_full_out_g(bool precise, const FullOutParams& p, int64_t blocks,
                                    hipStream_t s) {
  if (precise)
    hipLaunchKernelGGL((full_out_kernel<G, true>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((full_out_kernel<G, false>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_full_out(int G, bool precise, const FullOutParams& p, int64_t n_tasks,
                           hipStream_t s) {
  const int64_t blocks = n_tasks * p.Hkv;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  switch (G) {
    case 1: return launch_full_out_g<1>(precise, p, blocks, s);
    case 2: return launch_full_out_g<2>(precise, p, blocks, s);
    case 4: return launch_full_out_g<4>(precise, p, blocks, s);
    case 8: return launch_full_out_g<8>(precise, p, blocks, s);
    case 16: return launch_full_out_g<16>(precise, p, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hs2
