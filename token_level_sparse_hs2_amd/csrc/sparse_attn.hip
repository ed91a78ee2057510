// sparse_attn.hip - one sparse attention layer over the selected positions, gfx950.
//
// Each sparse layer of a hybrid module reuses the full layer's KV cache and its
// token selection (HySparse2 news summary, KV Reuse paragraph; token-granularity
// paragraph: the later sparse layers go on using the same positions and cache),
// with its own queries. Attention over a subset is the softmax with
// every other logit at -inf, i.e. renormalised over the subset (SHARP
// walkthrough, section 2.3):
//   o[t,h] = sum_{j in I_t} exp(y_j - mu) v[j,g] / sum_{j in I_t} exp(y_j - mu),
//   y_j = scale * <q'[t,h], k[j,g]>, g = h / G.
//
// One wavefront per (token, KV group), CH index entries per step: the step's K
// and V rows are gathered with full-row coalesced loads (16 lanes per 256-byte
// row) into registers one step ahead, staged in the wave's LDS slice, and read
// back as the A operands of S^T = K_sel Q'^T (keys x heads; all G heads of the
// group share the gather) and, transposed, of O^T = V^T P^T. Online softmax in the log2 domain, fp32 accumulation. P enters
// the matrix product as a sum of bf16 parts (two parts: ~16 mantissa bits; three
// in the precise mode: ~24 bits), so rounding P to bf16 adds no visible error.
//
// Shared gather (PLAN): consecutive tokens select largely the same rows (the
// forced window, and keys that score high for all of them), so a wave can serve
// the NT = min(16 / G, 8) tokens of a group over the sorted union of their rows,
// built once per selection by sparse_plan_kernel: each union row is gathered once
// and the S^T tiles take all NT * G (token, head) columns, an entry counting only
// for the tokens whose row holds it, so each token's attention is unchanged.
//
// FP8 KV cache (HySparse2 news summary, cost paragraph: the cache kept in FP8):
// E4M3 codes with one fp32 scale per tensor. A lane gathers its 8 codes of a
// 128-byte row (the elements of its 16-byte chunk of the bf16 layout) and widens
// them with v_cvt_scalef32_pk_bf16_fp8 at scale 1, which is exact (every E4M3 value
// is a bf16 value), so the LDS layout and the matrix code are those of the bf16
// cache; the key scale is folded into the softmax constant and the value scale
// into the output.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

constexpr int kMaxParts = 32;  // partials merged per row (split rows of a decode step)

// DPP row rotates between the 4-lane banks of each 16-lane row (lanes 4a .. 4a+3
// form bank a). to_bank<A>: the lanes of bank A take src from lane - 4A of their
// row (bank 0); the other lanes keep old. from_bank<A>: the lanes of bank 0 take
// src from lane + 4A (bank A); the other lanes keep old.
template <int A>
__device__ __forceinline__ float to_bank(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src),
                                                    0x120 + 4 * A, 0xF, 1 << A, false));
}
template <int A>
__device__ __forceinline__ uint32_t from_bank(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, 0x120 + ((16 - 4 * A) & 15), 0xF,
                                               0x1, false);
}
// every lane takes the value of lane (lane & ~12) (its row's bank-0 lane of the same position)
__device__ __forceinline__ float bank_bcast(float x) {
  return to_bank<3>(to_bank<2>(to_bank<1>(x, x), x), x);
}

// CH index entries per step: 32 for a bf16 cache; 16 for an FP8 one, which halves
// the LDS slice and the staging registers so that four waves per SIMD fit (measured
// 5% faster there; a bf16 cache at 16 entries and three waves was 1.6% slower).
// MT = CH / 16 key tiles per step. PLAN: one wave per (token group, g) over the
// group's shared-gather union (SparseParams::plist); the S^T columns are the NT
// tokens' G heads, and an entry counts for the tokens in its mask only.
template <int G, bool PRECISE, bool FP8, int CH, bool PLAN>
__global__ __launch_bounds__(256, CH == 16 ? (FP8 && !PLAN ? 4 : 3) : 2) void sparse_attn_kernel(
    SparseParams p) {
  constexpr int MT = CH / 16, NR = CH / 4;
  constexpr int NT = PLAN ? plan_tokens(G) : 1;  // query tokens per wave
  __shared__ uint4 klds[4][CH][16];  // per wave: CH K rows x 256 B, swizzled 16-byte chunks
  __shared__ uint4 vlds[4][CH][16];  // per wave: CH V rows
  // the wave index is uniform: row, sequence and K/V row pointers live in SGPRs,
  // so the gathers take a scalar base and a 32-bit lane offset
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int lq = l >> 4, lc = l & 15;
  const int Hkv = p.Hkv, Hq = p.Hq, KW = p.KW;
  const int g = blockIdx.x % Hkv;
  const int64_t vr = (int64_t)(blockIdx.x / Hkv) * 4 + w;  // row x part, or token group
  if (vr >= (PLAN ? p.n_grp : p.T * p.n_part)) return;
  const int64_t tg = PLAN ? vr * NT : vr / p.n_part;  // the (first) query row
  const int part = PLAN ? 0 : (int)(vr % p.n_part);
  // query row tg: a token of the packed batch, or (decode) sequence tg at its
  // last cached position (PLAN: rows of the union are relative to this base)
  const int seq = p.decode ? (int)tg : find_seq(p.cu, p.B, tg);
  const int base = p.cu[seq];
  const int t = p.decode ? p.cu[seq + 1] - base - 1 : (int)(tg - base);
  const int32_t* irow = p.idx + ((size_t)tg * Hkv + g) * KW;
  const uint32_t* prow = PLAN ? p.plist + ((size_t)vr * Hkv + g) * p.pcap : nullptr;
  const int n_ent = PLAN ? p.pcount[(size_t)vr * Hkv + g] : KW;  // index entries of the wave
  const float c = p.c;
  // S^T column lc: head lc < G of token tg, or (PLAN) head lc % G of token tg + lc / G
  const int col_tok = PLAN ? lc / G : 0;
  const bool col_ok = PLAN ? lc < NT * G && tg + col_tok < p.T : lc < G;

  // Q'^T operand (B): column lc, k = d slice (loads first, columns without a
  // (token, head) zeroed afterwards)
  bf16x8 qb[4];
  {
    const int64_t qrow = PLAN ? min(tg + min(col_tok, NT - 1), p.T - 1) : tg;
    const int qh = PLAN ? lc % G : min(lc, G - 1);
    u32x4 v[4];
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
      v[ks] = to_u32x4(ldg128(p.q + ((size_t)qrow * Hq + g * G + qh) * kHeadDim + 32 * ks + 8 * lq));
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      if (!col_ok) v[ks] = u32x4{0u, 0u, 0u, 0u};
      qb[ks] = as_bf16x8(v[ks]);
    }
  }

  // Compact softmax (G <= 4, 32-entry steps): the step's valid scores sit in lanes
  // (lq, h < 4) of the S^T tiles, 8 per lane. Bank a of each row takes the pair
  // (2a, 2a + 1) of lane (lq, h) with a DPP row rotate, so the exponentials and
  // the bf16 split run on 2 values per lane instead of 8; the packed pairs return
  // to lanes (lq, h), the B operand of P.V, the same way. lsum then holds each
  // lane's share (reduced over the banks at the end) and mc the reference m of
  // head (lane & 3). (16-entry steps keep the plain layout: there the saving is
  // smaller and the extra registers spill under four waves per SIMD.)
  constexpr bool kCompact = !PLAN && G <= 4 && MT == 2;
  float m = -INFINITY, mc = -INFINITY, lsum = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; i++) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this sequence's K/V rows of group g; row j starts at byte j * row_stride
  constexpr int kElemBytes = FP8 ? 1 : 2;
  const char* kseq = FP8 ? reinterpret_cast<const char*>(p.k8) : reinterpret_cast<const char*>(p.k);
  const char* vseq = FP8 ? reinterpret_cast<const char*>(p.v8) : reinterpret_cast<const char*>(p.v);
  kseq += ((size_t)base * Hkv + g) * kHeadDim * kElemBytes;
  vseq += ((size_t)base * Hkv + g) * kHeadDim * kElemBytes;
  const uint32_t row_stride = (uint32_t)Hkv * kHeadDim * kElemBytes;
  uint4(*vl)[16] = vlds[w];
  const int n_chunks = (n_ent + CH - 1) / CH;
  // this wave's steps: all of them, or its part's share
  const int per_part = (n_chunks + p.n_part - 1) / p.n_part;
  const int c_begin = part * per_part, c_end = min(n_chunks, c_begin + per_part);

  // Index entries of chunk c for the lane's MT A rows (keys 16*mt + lc). The raw
  // load is unconditional (clamped to a valid entry) and its value is only used
  // two chunks later by valid_idx(); loads skipped on some path, or consumed at
  // once, would make the compiler drain the gather in flight behind them.
  // (PLAN: an entry is (row, token mask); mk gets the mask, 0 for no entry)
  using Raw = std::conditional_t<PLAN, uint32_t, int>;
  auto load_raw = [&](int c, Raw (&r)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      if constexpr (PLAN) r[mt] = prow[max(0, min(c * CH + 16 * mt + lc, n_ent - 1))];
      else r[mt] = irow[min(c * CH + 16 * mt + lc, KW - 1)];
    }
  };
  auto valid_idx = [&](int c, const Raw (&r)[MT], int (&j)[MT], uint32_t (&mk)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const bool ok = c < c_end && c * CH + 16 * mt + lc < n_ent;
      if constexpr (PLAN) {
        j[mt] = ok ? (int)(r[mt] & kPlanRowMask) : -1;
        mk[mt] = ok ? r[mt] >> 24 : 0u;
      } else {
        j[mt] = ok ? r[mt] : -1;
        mk[mt] = 0u;
      }
    }
  };
  // an entry to gather: PLAN rows are valid by construction, others lie in [0, t]
  auto entry_ok = [&](int j) HS2_INLINE { return PLAN ? j >= 0 : (j >= 0 && j <= t); };
  // gather the chunk's K and V rows, fully coalesced: load r covers keys
  // 4r .. 4r+3, 16 lanes per row (lane: key 4r + lq, elements 8 lc .. 8 lc + 7:
  // 16 bytes of a bf16 row, 8 bytes of an FP8 one)
  using Piece = std::conditional_t<FP8, uint2, uint4>;
  struct Gather {
    Piece kr[NR];
    Piece vr[NR];
  };
  auto gather = [&](const int (&j)[MT], Gather& gb) {
    // byte offset of the row of each of the lane's entries (row 0 if invalid)
    int roff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
      roff[mt] = (int)((uint32_t)(entry_ok(j[mt]) ? j[mt] : 0) * row_stride);
#pragma unroll
    for (int r = 0; r < NR; r++) {
      const int key = 4 * r + lq;  // entry of the chunk; its offset is held by lane (key & 15)
      const uint32_t off =
          (uint32_t)__shfl(roff[key >> 4], key & 15, 64) + (8u * kElemBytes) * lc;
      if constexpr (FP8) {
        gb.kr[r] = ldg64(kseq + off);
        gb.vr[r] = ldg64(vseq + off);
      } else {
        gb.kr[r] = ldg128(kseq + off);
        gb.vr[r] = ldg128(vseq + off);
      }
    }
  };
  // a gathered piece as 8 bf16 (FP8: widened exactly)
  auto widen = [&](const Piece& x) HS2_INLINE -> uint4 {
    if constexpr (FP8)
      return make_uint4(e4m3x2_to_bf16x2<false>(x.x), e4m3x2_to_bf16x2<true>(x.x),
                        e4m3x2_to_bf16x2<false>(x.y), e4m3x2_to_bf16x2<true>(x.y));
    else
      return x;
  };
  uint4(*kl)[16] = klds[w];

  constexpr int NSPLIT = PRECISE ? 3 : 2;
  constexpr float kRescaleSlack = 8.f;  // log2 units the running max may lag behind

  auto consume = [&](const int (&j)[MT], const uint32_t (&mk)[MT], const Gather& gb) {
    uint64_t bal[MT], any = 0, all = ~0ull;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      bal[mt] = __ballot(entry_ok(j[mt]));
      any |= bal[mt];
      all &= bal[mt];
    }
    if (any == 0) return;
    const bool full = all == ~0ull;
    wave_lds_fence();  // previous chunk's reads of kl / vl are done
    // rows into LDS. K: 16-byte chunk ch of key r at physical chunk ch ^ (r & 15);
    // V: at ch ^ (2 * (r & 7)) (suits the transposing reads below)
#pragma unroll
    for (int r = 0; r < NR; r++) {
      const int key = 4 * r + lq;
      kl[key][lc ^ (key & 15)] = widen(gb.kr[r]);
      vl[key][lc ^ (2 * (key & 7))] = widen(gb.vr[r]);
    }
    wave_lds_fence();
    // raw scores S^T (keys x heads); lane: head lc, keys 16*mt + 4*lq + i
    f32x4 s[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = 16 * mt + lc;
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        const bf16x8 ka = as_bf16x8(to_u32x4(kl[key][(4 * ks + lq) ^ (key & 15)]));
        s[mt] = mfma16x16x32(ka, qb[ks], s[mt]);
      }
    }
    if constexpr (PLAN && NT * 16 <= 64) {
      // entry 16*mt + e (lane lc = e holds its word) counts for column lc iff its mask
      // holds token col_tok: the tokens' ballots over lanes 0..15, packed into one scalar
      // word (bit 16*a + e), give each lane its four entries' bits with one shift
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const uint64_t ok = __ballot(entry_ok(j[mt]));
        uint64_t tm = 0;
#pragma unroll
        for (int a = 0; a < NT; a++)
          tm |= ((__ballot((mk[mt] >> a) & 1u) & ok) & 0xFFFFull) << (16 * a);
        const uint32_t bits = (uint32_t)(tm >> (16 * col_tok + 4 * lq)) & 0xFu;
#pragma unroll
        for (int i = 0; i < 4; i++)
          if (!((bits >> i) & 1u)) s[mt][i] = -INFINITY;
      }
    } else if constexpr (PLAN) {
      // entry 16*mt + 4*lq + i counts for column lc iff its mask holds token col_tok:
      // bit (4*lq + i) of that token's ballot
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        uint64_t mine = 0;
#pragma unroll
        for (int a = 0; a < NT; a++) {
          const uint64_t b = __ballot(entry_ok(j[mt]) && ((mk[mt] >> a) & 1u));
          mine = col_tok == a ? b : mine;
        }
        const uint32_t bits = (uint32_t)(mine >> (4 * lq)) & 0xFu;
#pragma unroll
        for (int i = 0; i < 4; i++)
          if (!((bits >> i) & 1u)) s[mt][i] = -INFINITY;
      }
    } else if (!full) {  // entry 16*mt + 4*lq + i is valid iff bit (4*lq + i) of the ballot
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
#pragma unroll
        for (int i = 0; i < 4; i++)
          if (!((bal[mt] >> (4 * lq + i)) & 1ull)) s[mt][i] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
    if constexpr (MT == 2)
      mx = fmaxf(mx, fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = max_xor32(max_xor16(mx));
    mx *= c;  // finite when the column has an entry in the chunk (always, unless PLAN)
    // the reference m only moves when a score passes it by the slack (never
    // overflows: terms stay below 2^slack); moving it rescales l and O. (PLAN: a
    // column without entries so far keeps m = -inf, alpha 1.)
    if (__any(mx > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = m_new == m ? 1.f : fast_exp2(m - m_new);
#pragma unroll
      for (int i = 0; i < 8; i++) o[i] *= alpha;
      m = m_new;
      if constexpr (kCompact) {
        lsum *= bank_bcast(alpha);
        mc = bank_bcast(m);
      } else {
        lsum *= alpha;
      }
    }

    // P^T operand (B): column = head, k slot s <-> key (s < 4 ? 4lq + s : 16 + 4lq + s - 4).
    // P is split into bf16 parts p = p0 + p1 (+ p2 in the precise mode), each the
    // bf16 rounding of what the previous parts leave, so P.V keeps ~16 (~24)
    // mantissa bits of P; V is bf16 already, so every product is exact.
    // (MT = 1: 16x16x16 MFMA, k slot s <-> key 4lq + s.)
    uint32_t pk[NSPLIT][2 * MT];
    if constexpr (kCompact) {
      // bank a <- pair a: (s[0][0], s[0][1]), (s[0][2], s[0][3]), (s[1][0], s[1][1]), ...
      float t0 = to_bank<1>(s[0][0], s[0][2]), t1 = to_bank<1>(s[0][1], s[0][3]);
      t0 = to_bank<2>(t0, s[MT - 1][0]);
      t1 = to_bank<2>(t1, s[MT - 1][1]);
      t0 = to_bank<3>(t0, s[MT - 1][2]);
      t1 = to_bank<3>(t1, s[MT - 1][3]);
      float p0 = fast_exp2(fmaf(t0, c, -mc)), p1 = fast_exp2(fmaf(t1, c, -mc));
      lsum += p0 + p1;
#pragma unroll
      for (int part = 0; part < NSPLIT; part++) {
        const uint32_t pc = pack_bf16x2(p0, p1);
        if (part + 1 < NSPLIT) {
          p0 -= bf16_bits_to_f32(pc & 0xFFFFu);
          p1 -= __uint_as_float(pc & 0xFFFF0000u);
        }
        pk[part][0] = pc;
        pk[part][1] = from_bank<1>(pc, pc);
        pk[part][MT] = from_bank<2>(pc, pc);
        pk[part][2 * MT - 1] = from_bank<3>(pc, pc);
      }
    } else {
      // (PLAN: a column still at m = -inf has only -inf scores here; weight 0)
      const float mref = PLAN ? (m > -INFINITY ? m : 0.f) : m;
      float pv[4 * MT];
      float psum = 0.f;
#pragma unroll
      for (int sidx = 0; sidx < 4 * MT; sidx++) {
        pv[sidx] = fast_exp2(fmaf(s[sidx >> 2][sidx & 3], c, -mref));
        psum += pv[sidx];
      }
      lsum += psum;
#pragma unroll
      for (int part = 0; part < NSPLIT; part++) {
#pragma unroll
        for (int u = 0; u < 2 * MT; u++) pk[part][u] = pack_bf16x2(pv[2 * u], pv[2 * u + 1]);
        if (part + 1 < NSPLIT) {
#pragma unroll
          for (int u = 0; u < 2 * MT; u++) {
            pv[2 * u] -= bf16_bits_to_f32(pk[part][u] & 0xFFFFu);
            pv[2 * u + 1] -= __uint_as_float(pk[part][u] & 0xFFFF0000u);
          }
        }
      }
    }

    // V^T operand (A): row d = 16*dt + lc, k slots 4h..4h+3 <-> keys 16h + 4lq + e.
    // One transposing LDS read per half: within each 16-lane group, lane i gets
    // element (i & 3) of the 8-byte pieces read by lanes (i >> 2) + 4e, so lane j
    // reads key 16h + 4lq + (j >> 2), d = 16dt + 4(j & 3) .. +3.
    const int key_lo = 4 * lq + (lc >> 2);
    const int dsub = 4 * (lc & 3);
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      typedef short i16x4 __attribute__((ext_vector_type(4)));
      uint2 hv[MT];
#pragma unroll
      for (int h = 0; h < MT; h++) {
        const int key = 16 * h + key_lo;
        const int d0 = 16 * dt + dsub;
        const int phys = (d0 >> 3) ^ (2 * (key & 7));
        const short* src = reinterpret_cast<const short*>(&vl[key][phys]) + (d0 & 7);
        hv[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                              (i16x4 __attribute__((address_space(3)))*)(src)));
      }
      if constexpr (MT == 2) {
        const bf16x8 va = as_bf16x8(u32x4{hv[0].x, hv[0].y, hv[1].x, hv[1].y});
#pragma unroll
        for (int part = 0; part < NSPLIT; part++)
          o[dt] = mfma16x16x32(va, as_bf16x8(u32x4{pk[part][0], pk[part][1], pk[part][2],
                                                   pk[part][3]}),
                               o[dt]);
      } else {
        const s16x4 va = __builtin_bit_cast(s16x4, hv[0]);
#pragma unroll
        for (int part = 0; part < NSPLIT; part++)
          o[dt] = mfma16x16x16(va, __builtin_bit_cast(s16x4, make_uint2(pk[part][0], pk[part][1])),
                               o[dt]);
      }
    }
  };

  // software pipeline: while chunk c computes, the gather of chunk c+1 and the
  // index entries of chunks c+2 and c+3 are in flight. Entries past the row are
  // -1: their gathers read row 0 and are skipped.
  Raw r0[MT], r1[MT], r2[MT];
  int ja[MT], jb[MT];
  uint32_t ma[MT], mb[MT];
  Gather ga, gb;
  load_raw(c_begin, r0);
  load_raw(c_begin + 1, r1);
  load_raw(c_begin + 2, r2);
  // keep this issue order (as in the loop body: idx entries older than the gather
  // behind them), so the loop's waits can leave the gather in flight
  __builtin_amdgcn_sched_barrier(0);
  valid_idx(c_begin, r0, ja, ma);
  gather(ja, ga);
  for (int c = c_begin; c < c_end; c += 2) {
    valid_idx(c + 1, r1, jb, mb);
    gather(jb, gb);
    load_raw(c + 3, r1);
    consume(ja, ma, ga);
    // no early exit here: a chunk past the row has no valid entry and is skipped
    // by consume(), and one exit keeps every path through the loop issuing the
    // same loads in the same order
    valid_idx(c + 2, r2, ja, ma);
    gather(ja, ga);
    load_raw(c + 4, r2);
    consume(jb, mb, gb);
  }
  if constexpr (kCompact) {  // the banks' shares of each head
    lsum += shfl_xor_f(lsum, 4);
    lsum += shfl_xor_f(lsum, 8);
  }
  lsum += shfl_xor_f(lsum, 16);
  lsum += shfl_xor_f(lsum, 32);
  const float osc = FP8 ? p.v_scale : 1.f;  // the value scale, outside the sums
  if (!PLAN && p.n_part > 1) {  // unnormalised partial of this part (m = -inf, sum 0 if it had none)
    if (lc < G) {
      const size_t slot = (size_t)vr * Hkv + g;
      float* po = p.part_o + (slot * G + lc) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 8; dt++)
        *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * lq) = FP8 ? o[dt] * osc : o[dt];
      if (lq == 0) p.part_ml[slot * G + lc] = make_float2(m, lsum);
    }
    return;
  }
  if (col_ok) {
    const float inv = lsum > 0.f ? osc / lsum : 0.f;
    const size_t ob = ((size_t)(tg + col_tok) * Hq + g * G + (PLAN ? lc % G : lc)) * kHeadDim;
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

// Merges the n_part (<= kMaxParts) partials of each (row, group): per head and d,
// o = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), M = max_s m_s (0 if no part
// saw a valid entry). One workgroup per (row, group, head), one thread per d: the
// parts' outputs and their (m, l) are all loaded before the first use, so the
// merge waits out one memory round trip.
template <int G, bool PRECISE>
__global__ __launch_bounds__(kHeadDim) void sparse_combine_kernel(SparseParams p) {
  __shared__ float2 ml[kMaxParts];
  const int64_t row = blockIdx.x / G;  // (query row, group)
  const int h = (int)(blockIdx.x % G);
  const int64_t tg = row / p.Hkv;
  const int g = (int)(row % p.Hkv);
  const int d = threadIdx.x, np = p.n_part;
  auto slot = [&](int s) { return (size_t)(tg * np + s) * p.Hkv + g; };
  float v[kMaxParts];
#pragma unroll
  for (int s = 0; s < kMaxParts; s++)
    v[s] = s < np ? p.part_o[(slot(s) * G + h) * kHeadDim + d] : 0.f;
  if (d < np) ml[d] = p.part_ml[slot(d) * G + h];
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < np; s++) M = fmaxf(M, ml[s].x);
  float den = 0.f, val = 0.f;
  if (M > -INFINITY) {
#pragma unroll
    for (int s = 0; s < kMaxParts; s++) {
      if (s < np) {
        const float2 e = ml[s];
        const float wgt = fast_exp2(e.x - M);  // 0 for a part without valid entries
        den += e.y * wgt;
        val = fmaf(v[s], wgt, val);
      }
    }
  }
  val = den > 0.f ? val / den : 0.f;
  const size_t o = ((size_t)tg * p.Hq + g * G + h) * kHeadDim + d;
  if constexpr (PRECISE) static_cast<float*>(p.out)[o] = val;
  else static_cast<__bf16*>(p.out)[o] = (__bf16)val;
}

template <int G, bool PLAN>
static void launch_sparse_kernel(bool precise, bool fp8, dim3 grid, const SparseParams& p,
                                 hipStream_t s) {
  const dim3 block(256);
  if (fp8) {
    if (precise) hipLaunchKernelGGL((sparse_attn_kernel<G, true, true, 16, PLAN>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((sparse_attn_kernel<G, false, true, 16, PLAN>), grid, block, 0, s, p);
  } else {
    if (precise) hipLaunchKernelGGL((sparse_attn_kernel<G, true, false, 32, PLAN>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((sparse_attn_kernel<G, false, false, 32, PLAN>), grid, block, 0, s, p);
  }
}

template <int G>
static hipError_t launch_sparse_g(bool precise, bool fp8, const SparseParams& p, hipStream_t s) {
  if (p.plist) {  // shared-gather plan: 4 token groups per workgroup, one KV group each
    if (p.n_part != 1) return hipErrorInvalidValue;
    const int64_t blocks = ((p.n_grp + 3) / 4) * p.Hkv;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    launch_sparse_kernel<G, true>(precise, fp8, dim3((unsigned)blocks), p, s);
    return hipGetLastError();
  }
  const int64_t blocks = ((p.T * p.n_part + 3) / 4) * p.Hkv;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  launch_sparse_kernel<G, false>(precise, fp8, dim3((unsigned)blocks), p, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_part <= 1) return e;
  const int64_t blocks_c = p.T * p.Hkv * G;  // (row, group, head)
  if (blocks_c > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid_c((unsigned)blocks_c), block_c(kHeadDim);
  if (precise) hipLaunchKernelGGL((sparse_combine_kernel<G, true>), grid_c, block_c, 0, s, p);
  else hipLaunchKernelGGL((sparse_combine_kernel<G, false>), grid_c, block_c, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_sparse(int G, bool precise, bool fp8, const SparseParams& p, hipStream_t s) {
  switch (G) {
    case 1: return launch_sparse_g<1>(precise, fp8, p, s);
    case 2: return launch_sparse_g<2>(precise, fp8, p, s);
    case 4: return launch_sparse_g<4>(precise, fp8, p, s);
    case 8: return launch_sparse_g<8>(precise, fp8, p, s);
    case 16: return launch_sparse_g<16>(precise, fp8, p, s);
    default: return hipErrorInvalidValue;
  }
}

// Shared-gather plan: one wavefront per (token group, KV group g). The group's
// rows are walked in windows of kPlanChunk positions (relative to base0, the
// sequence base of its first token): each token's entries of the window set bits
// in its LDS bitmap, then the union of the bitmaps is compacted in ascending
// order with one wave scan, each entry carrying the mask of the tokens that hold
// it. A row is ascending, so a cursor per token marks where the next window
// starts; -1 ends a row, entries past t are stepped over. Each round loads the
// next 256 entries of every unfinished row (4 per lane, all issued before any
// use), so a window costs about one memory round trip. The union is written by
// rank, 64 entries at a time: lane l takes entry base + l (its word: the words
// whose first entry falls in the block mark their slot, and a max scan over the
// slots gives every rank the last word started at or before it; its bit by a
// popcount select), so the work is balanced over the lanes however the entries
// cluster, and the stores are coalesced.
template <int NT>
__global__ __launch_bounds__(256) void sparse_plan_kernel(PlanParams p) {
  constexpr int kWords = kPlanChunk / 32;
  __shared__ uint32_t bms[4][NT][kWords];
  __shared__ uint32_t uws[4][kWords];   // union words of the window
  __shared__ int32_t pres[4][kWords];   // entries of the union in the words before
  __shared__ int32_t slots[4][64];      // word starting at each rank of a block, or -1
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  uint32_t(*bm)[kWords] = bms[w];
  uint32_t* uw = uws[w];
  int32_t* pre = pres[w];
  int32_t* slot = slots[w];
  const int64_t wid = (int64_t)blockIdx.x * 4 + w;  // grp * Hkv + g
  if (wid >= p.n_grp * p.Hkv) return;
  const int64_t grp = wid / p.Hkv;
  const int g = (int)(wid % p.Hkv);
  const int64_t tg0 = grp * NT;
  const int nt = (int)min<int64_t>(NT, p.T - tg0);
  const int base0 = p.cu[find_seq(p.cu, p.B, tg0)];
  const int KW = p.KW;
  // token a: its row, its position t and its sequence base relative to base0
  const int32_t* row[NT];
  int t_of[NT], off[NT], cur[NT];
#pragma unroll
  for (int a = 0; a < NT; a++) {
    const int64_t tg = tg0 + min(a, nt - 1);
    const int base = p.cu[find_seq(p.cu, p.B, tg)];
    row[a] = p.idx + ((size_t)tg * p.Hkv + g) * KW;
    t_of[a] = (int)(tg - base);
    off[a] = base - base0;
    cur[a] = a < nt ? 0 : KW;  // tokens past the batch hold nothing
  }
  const int rel_max = (int)(tg0 + nt - 1 - base0);  // no entry lies past the last token
  uint32_t* list = p.list + (size_t)wid * p.cap;
  int out = 0;
  for (int lo = 0; lo <= rel_max; lo += kPlanChunk) {
    const int hi = lo + kPlanChunk;
#pragma unroll
    for (int a = 0; a < NT; a++)
      for (int i = l; i < kWords; i += 64) bm[a][i] = 0u;
    wave_lds_fence();
    bool pending[NT];
#pragma unroll
    for (int a = 0; a < NT; a++) pending[a] = cur[a] < KW;
    for (;;) {
      bool any = false;
#pragma unroll
      for (int a = 0; a < NT; a++) any |= pending[a];
      if (!any) break;
      // entries cur + 64 i + l of every pending row
      int j[NT][4];
#pragma unroll
      for (int a = 0; a < NT; a++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int e = cur[a] + 64 * i + l;
          j[a][i] = pending[a] && e < KW ? row[a][e] : -1;
        }
#pragma unroll
      for (int a = 0; a < NT; a++) {
        if (!pending[a]) continue;
        int n_lead = 0;
        bool stopped = false;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int jj = j[a][i];
          const int rel = off[a] + jj;
          const bool in = jj >= 0 && jj <= t_of[a] && rel < hi;
          if (in && rel >= lo) atomicOr(&bm[a][(rel - lo) >> 5], 1u << ((rel - lo) & 31));
          const uint64_t lead = __ballot(in);
          if (!stopped) {
            if (lead == ~0ull) {
              n_lead += 64;
            } else {
              n_lead += __builtin_ctzll(~lead);
              stopped = true;
            }
          }
        }
        const int stop = cur[a] + n_lead;  // the entry that ended the run (uniform)
        if (!stopped) {  // all 256 below hi: another round
          cur[a] = stop;
          continue;
        }
        // the stopping entry was loaded: entry n_lead of this round
        const int si = n_lead >> 6;
        const int sv = si == 0 ? j[a][0] : si == 1 ? j[a][1] : si == 2 ? j[a][2] : j[a][3];
        const int js = __shfl(sv, n_lead & 63, 64);
        if (js < 0) {  // -1 padding (or the end): the row is done
          cur[a] = KW;
          pending[a] = false;
        } else if (js <= t_of[a]) {  // at or past hi: the next window starts here
          cur[a] = stop;
          pending[a] = false;
        } else {  // past t: step over it
          cur[a] = stop + 1;
          pending[a] = cur[a] < KW;
        }
      }
    }
    wave_lds_fence();
    // lane l owns words [l * per, l * per + per) of the union
    constexpr int per = kWords / 64;
    uint32_t u[per];
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < per; q++) {
      uint32_t x = 0u;
#pragma unroll
      for (int a = 0; a < NT; a++) x |= bm[a][per * l + q];
      u[q] = x;
      cnt += __popc(x);
    }
    const int incl = wave_incl_scan(cnt, l);
    const int total = __shfl(incl, 63, 64);
    int pq[per];
    {
      int o = incl - cnt;
#pragma unroll
      for (int q = 0; q < per; q++) {
        uw[per * l + q] = u[q];
        pre[per * l + q] = o;
        pq[q] = o;
        o += __popc(u[q]);
      }
    }
    int carry = -1;  // the last word started before the block
    for (int base = 0; base < total; base += 64) {
      slot[l] = -1;
      wave_lds_fence();
#pragma unroll
      for (int q = 0; q < per; q++)
        if (u[q] != 0u && pq[q] >= base && pq[q] < base + 64) slot[pq[q] - base] = per * l + q;
      wave_lds_fence();
      const int wlo = max(wave_incl_max(slot[l]), carry);  // the word holding entry base + l
      carry = __shfl(wlo, 63, 64);
      const int r = base + l;
      if (r < total) {
        uint32_t x = uw[wlo];
        int k = r - pre[wlo], b = 0;  // the k-th set bit of x
#pragma unroll
        for (int width = 16; width >= 1; width >>= 1) {
          const int c = __popc(x & ((1u << width) - 1u));
          if (k >= c) {
            k -= c;
            x >>= width;
            b += width;
          }
        }
        uint32_t mask = 0u;
#pragma unroll
        for (int a = 0; a < NT; a++) mask |= ((bm[a][wlo] >> b) & 1u) << a;
        if (out + r < p.cap) list[out + r] = (uint32_t)(lo + 32 * wlo + b) | mask << 24;
      }
      wave_lds_fence();  // the slots are read before the next block resets them
    }
    out += total;
    wave_lds_fence();
  }
  if (l == 0) p.count[wid] = min(out, p.cap);
}

template <int NT>
static hipError_t launch_plan_nt(const PlanParams& p, hipStream_t s) {
  const int64_t waves = p.n_grp * p.Hkv;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sparse_plan_kernel<NT>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_sparse_plan(int G, const PlanParams& p, hipStream_t s) {
  switch (G) {
    case 1: return launch_plan_nt<8>(p, s);
    case 2: return launch_plan_nt<8>(p, s);
    case 4: return launch_plan_nt<4>(p, s);
    case 8: return launch_plan_nt<2>(p, s);
    case 16: return launch_plan_nt<1>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Writing the FP8 cache: 8 elements per thread (one 16-byte load, one 8-byte
// store), grid-stride; the product with inv_scale is rounded to fp32, clamped to
// +-448 (NaN stays NaN: the comparisons fail) and rounded to the nearest E4M3
// code by v_cvt_pk_fp8_f32. A tail of n % 8 elements is done one by one.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* src, uint8_t* dst,
                                                           int64_t n, float inv_scale) {
  auto q = [&](float x) HS2_INLINE {
    const float y = x * inv_scale;
    return y > 448.f ? 448.f : (y < -448.f ? -448.f : y);
  };
  const int64_t n8 = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 x = ldg128(src + 8 * i);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      int r = 0;
      r = __builtin_amdgcn_cvt_pk_fp8_f32(q(bf16_bits_to_f32(w[2 * h] & 0xFFFFu)),
                                          q(__uint_as_float(w[2 * h] & 0xFFFF0000u)), r, false);
      r = __builtin_amdgcn_cvt_pk_fp8_f32(q(bf16_bits_to_f32(w[2 * h + 1] & 0xFFFFu)),
                                          q(__uint_as_float(w[2 * h + 1] & 0xFFFF0000u)), r, true);
      out[h] = (uint32_t)r;
    }
    *reinterpret_cast<uint2*>(dst + 8 * i) = make_uint2(out[0], out[1]);
  }
  if (blockIdx.x == 0 && threadIdx.x < (int)(n - 8 * n8)) {
    const int64_t i = 8 * n8 + threadIdx.x;
    const int r = __builtin_amdgcn_cvt_pk_fp8_f32(q(bf16_bits_to_f32(src[i])), 0.f, 0, false);
    dst[i] = (uint8_t)(r & 0xFF);
  }
}

hipError_t launch_quantize_fp8(const uint16_t* src, uint8_t* dst, int64_t n, float inv_scale,
                               hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n / 8 + 255) / 256;
  const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>(want, 4096));
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3(blocks), dim3(256), 0, s, src, dst, n, inv_scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the entry point that allocates nothing (hs2_decode_sparse_attn_noalloc):
// the split rows' partials (sparse_attn_kernel with n_part > 1, read back by
// sparse_combine_kernel) live in this file-scope device array instead of a caller
// workspace. Every GPU holds its own copy at its own address; host code must not
// pass the array's name to a kernel (that is a host-side stand-in), only the
// address looked up here, once per device with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

}  // namespace hs2
