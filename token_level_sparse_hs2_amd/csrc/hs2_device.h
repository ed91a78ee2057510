// hs2_device.h - small device helpers for the gfx950 kernels: bf16 vectors,
// MFMA wrappers, lane utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// lambdas that capture register arrays must be inlined, or the arrays go to scratch
#define HS2_INLINE __attribute__((always_inline))

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (lo in bits 0-15), hardware round-to-nearest-even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// C[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulation.
// Lane l supplies A row (l & 15), k = 8*(l >> 4) .. +7; B column (l & 15), same k;
// receives C column (l & 15), rows 4*(l >> 4) .. +3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two E4M3 codes (bytes 2 HI, 2 HI + 1 of x) -> two bf16 in a word, at scale 1:
// exact, every E4M3 value being a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x, 1.0f, HI));
}

__device__ __forceinline__ uint2 ldg64(const void* p) {
  return *reinterpret_cast<const uint2*>(p);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
// v_mfma_f32_16x16x16_bf16: A lane l = row l & 15, k = 4 (l >> 4) .. +3; B lane l =
// column l & 15, same k; C as for 16x16x32
__device__ __forceinline__ f32x4 mfma16x16x16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ldg128(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ u32x4 to_u32x4(uint4 v) {
  u32x4 r;
  r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
  return r;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// max(v[l], v[l ^ 16]) and max(v[l], v[l ^ 32]) with the gfx950 lane-swap ops
// (v_permlane16_swap / v_permlane32_swap: VALU, no LDS round trip). Called with
// the same register as both operands, the pair returned holds v[l] and v[l ^ 16]
// (resp. v[l ^ 32]) in some order.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// max of three floats / of a lane pair as one v_max3_f32 / v_max_f32 from inline
// asm: fmaxf in IEEE mode first quiets each operand the compiler cannot prove is
// not a signalling NaN (one extra v_max per operand); scores and -inf are never NaN.
__device__ __forceinline__ float max3_f32(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2_f32(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_xor16_raw(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2_f32(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32_raw(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2_f32(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// A pointer the caller knows to be wave-uniform, moved into SGPRs (for the saddr
// form of global loads).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round trip):
// scans within each 16-lane row, then row broadcasts of lanes 15 and 31.
__device__ __forceinline__ int wave_incl_scan(int x, int l) {
  (void)l;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Inclusive prefix sum within each 16-lane row (the first four moves of
// wave_incl_scan).
__device__ __forceinline__ int row_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  return x;
}

// Inclusive max scan over the 64 lanes (values >= -1), the DPP moves of
// wave_incl_scan with -1 where a move brings nothing.
__device__ __forceinline__ int wave_incl_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x111, 0xF, 0xF, false));  // row_shr:1
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x112, 0xF, 0xF, false));  // row_shr:2
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x114, 0xF, 0xF, false));  // row_shr:4
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x118, 0xF, 0xF, false));  // row_shr:8
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return x;
}

// Order LDS traffic of one wavefront (its own writes become visible to its own
// later reads); a barrier for the compiler and the memory model, not a
// workgroup barrier.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Sequence of global token tg: last i with cu[i] <= tg.
__device__ __forceinline__ int find_seq(const int32_t* cu, int B, int64_t tg) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= tg) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace hs2
