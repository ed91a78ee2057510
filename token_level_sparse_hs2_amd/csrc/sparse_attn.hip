// sparse_attn.hip - one sparse attention layer over the selected positions, gfx950.
//
// Each sparse layer of a hybrid module reuses the full layer's KV cache and its
// token selection (HySparse2 news summary, KV Reuse paragraph; token-granularity
// paragraph: "subsequent sparse layers keep reusing these positions and their
// cache"), with its own queries. Attention over a subset is the softmax with
// every other logit at -inf, i.e. renormalised over the subset (SHARP
// walkthrough, section 2.3):
//   o[t,h] = sum_{j in I_t} exp(y_j - mu) v[j,g] / sum_{j in I_t} exp(y_j - mu),
//   y_j = scale * <q'[t,h], k[j,g]>, g = h / G.
//
// One wavefront per (token, KV group): the K rows of a 32-entry chunk of I_t
// are gathered straight into MFMA A operands (S^T = K_sel Q'^T, keys x heads,
// all G heads of the group share the gather); the V rows are staged in the
// wave's LDS slice and read back transposed as the A operand of
// O^T = V^T P^T. Online softmax in the log2 domain, fp32 accumulation. P enters
// the matrix product as a sum of bf16 parts (two parts: ~16 mantissa bits; three
// in the precise mode: ~24 bits), so rounding P to bf16 adds no visible error.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

constexpr int kChunk = 32;  // index entries per step

template <int G, bool PRECISE>
__global__ __launch_bounds__(256) void sparse_attn_kernel(SparseParams p) {
  __shared__ uint4 vlds[4][kChunk][16];  // per wave: 32 keys x 256 B, swizzled 16-byte chunks
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int lq = l >> 4, lc = l & 15;
  const int Hkv = p.Hkv, Hq = p.Hq, KW = p.KW;
  const int g = blockIdx.x % Hkv;
  const int64_t tg = (int64_t)(blockIdx.x / Hkv) * 4 + w;
  if (tg >= p.T) return;
  const int seq = find_seq(p.cu, p.B, tg);
  const int base = p.cu[seq];
  const int t = (int)(tg - base);
  const int32_t* irow = p.idx + ((size_t)tg * Hkv + g) * KW;
  const float c = p.c;

  // Q'^T operand (B): column = head (lane & 15) < G, k = d slice
  bf16x8 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ks++) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (lc < G)
      v = to_u32x4(ldg128(p.q + ((size_t)tg * Hq + g * G + lc) * kHeadDim + 32 * ks + 8 * lq));
    qb[ks] = as_bf16x8(v);
  }

  float m = -INFINITY, lsum = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; i++) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* kb = p.k + (size_t)g * kHeadDim;
  const uint16_t* vb = p.v + (size_t)g * kHeadDim;
  uint4(*vl)[16] = vlds[w];

  for (int c0 = 0; c0 < KW; c0 += kChunk) {
    // index entries for the lane's two A rows
    int j0 = -1, j1 = -1;
    if (c0 + lc < KW) j0 = irow[c0 + lc];
    if (c0 + 16 + lc < KW) j1 = irow[c0 + 16 + lc];
    const bool ok0 = (j0 >= 0) && (j0 <= t), ok1 = (j1 >= 0) && (j1 <= t);
    const uint64_t bal0 = __ballot(ok0), bal1 = __ballot(ok1);
    if ((bal0 | bal1) == 0) continue;
    const size_t r0 = (size_t)(base + (ok0 ? j0 : 0)) * Hkv * kHeadDim;
    const size_t r1 = (size_t)(base + (ok1 ? j1 : 0)) * Hkv * kHeadDim;

    // gather K rows into A operands and V rows into LDS
    bf16x8 ka[2][4];
    uint4 vr[2][4];
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      ka[0][ks] = as_bf16x8(to_u32x4(ldg128(kb + r0 + 32 * ks + 8 * lq)));
      ka[1][ks] = as_bf16x8(to_u32x4(ldg128(kb + r1 + 32 * ks + 8 * lq)));
      vr[0][ks] = ldg128(vb + r0 + 32 * ks + 8 * lq);
      vr[1][ks] = ldg128(vb + r1 + 32 * ks + 8 * lq);
    }
    wave_lds_fence();  // previous chunk's reads of vl are done
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const int key = 16 * mt + lc;
      const int swz = 2 * ((key >> 2) & 3);
#pragma unroll
      for (int ks = 0; ks < 4; ks++) vl[key][(4 * ks + lq) ^ swz] = vr[mt][ks];
    }

    // scores S^T (keys x heads)
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ks++) s[mt] = mfma16x16x32(ka[mt][ks], qb[ks], s[mt]);
    }
    // entry 16*mt + 4*lq + i is valid iff bit (4*lq + i) of the ballot
    float v2[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const uint64_t bal = mt ? bal1 : bal0;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const bool ok = (bal >> (4 * lq + i)) & 1ull;
        v2[mt][i] = ok ? s[mt][i] * c : -INFINITY;
        mx = fmaxf(mx, v2[mt][i]);
      }
    }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m, mx);  // finite: the chunk has a valid entry
    const float alpha = fast_exp2(m - m_new);
    float pv[2][4];
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        pv[mt][i] = fast_exp2(v2[mt][i] - m_new);
        psum += pv[mt][i];
      }
    lsum = lsum * alpha + psum;
    m = m_new;
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] *= alpha;

    // P^T operand (B): column = head, k slot s <-> key (s < 4 ? 4lq + s : 16 + 4lq + s - 4).
    // P is split into bf16 parts p = p0 + p1 (+ p2 in the precise mode), each the
    // bf16 rounding of what the previous parts leave, so P.V keeps ~16 (~24)
    // mantissa bits of P; V is bf16 already, so every product is exact.
    constexpr int NSPLIT = PRECISE ? 3 : 2;
    bf16x8 pb[NSPLIT];
    {
      float rem[8];
#pragma unroll
      for (int sidx = 0; sidx < 8; sidx++) rem[sidx] = pv[sidx >> 2][sidx & 3];
#pragma unroll
      for (int part = 0; part < NSPLIT; part++) {
        u32x4 pk;
#pragma unroll
        for (int u = 0; u < 4; u++) pk[u] = pack_bf16x2(rem[2 * u], rem[2 * u + 1]);
        pb[part] = as_bf16x8(pk);
        if (part + 1 < NSPLIT) {
#pragma unroll
          for (int u = 0; u < 4; u++) {
            rem[2 * u] -= bf16_bits_to_f32(pk[u] & 0xFFFFu);
            rem[2 * u + 1] -= bf16_bits_to_f32(pk[u] >> 16);
          }
        }
      }
    }

    wave_lds_fence();  // this chunk's V rows are in LDS
    // V^T operand (A): row d = 16*dt + lc, k slot s <-> key as above
    const uint16_t* vls = reinterpret_cast<const uint16_t*>(&vl[0][0]);
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      const int d = 16 * dt + lc;
      const int ch = d >> 3, within = d & 7;
      uint32_t a[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        uint32_t pair[2];
#pragma unroll
        for (int e = 0; e < 2; e++) {
          const int sidx = 2 * u + e;
          const int key = sidx < 4 ? 4 * lq + sidx : 16 + 4 * lq + (sidx - 4);
          const int swz = 2 * ((key >> 2) & 3);
          pair[e] = vls[(key * 16 + (ch ^ swz)) * 8 + within];
        }
        a[u] = pair[0] | (pair[1] << 16);
      }
      u32x4 av;
      av[0] = a[0]; av[1] = a[1]; av[2] = a[2]; av[3] = a[3];
      const bf16x8 va = as_bf16x8(av);
#pragma unroll
      for (int part = 0; part < NSPLIT; part++) o[dt] = mfma16x16x32(va, pb[part], o[dt]);
    }
  }

  lsum += shfl_xor_f(lsum, 16);
  lsum += shfl_xor_f(lsum, 32);
  if (lc < G) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const size_t ob = ((size_t)tg * Hq + g * G + lc) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      const int d0 = 16 * dt + 4 * lq;
      if constexpr (PRECISE) {
        float4 r = make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + ob + d0) = r;
      } else {
        uint2 r = make_uint2(pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv),
                             pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + ob + d0) = r;
      }
    }
  }
}

template <int G>
static hipError_t launch_sparse_g(bool precise, const SparseParams& p, hipStream_t s) {
  const int64_t blocks = ((p.T + 3) / 4) * p.Hkv;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (precise)
    hipLaunchKernelGGL((sparse_attn_kernel<G, true>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((sparse_attn_kernel<G, false>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_sparse(int G, bool precise, const SparseParams& p, hipStream_t s) {
  switch (G) {
    case 1: return launch_sparse_g<1>(precise, p, s);
    case 2: return launch_sparse_g<2>(precise, p, s);
    case 4: return launch_sparse_g<4>(precise, p, s);
    case 8: return launch_sparse_g<8>(precise, p, s);
    case 16: return launch_sparse_g<16>(precise, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hs2
