// Device helpers shared by the gfx950 kernels: element types, 8-element operand fragments and
// the 16x16 MFMA wrappers.
//
// Fragment convention. Every MFMA here is a 16x16 output tile with a 32-deep contraction, and
// every lane supplies 8 consecutive contraction elements of one operand row (A) or column (B):
// lane l covers row/column (l % 16) and contraction elements [8 * (l / 16), 8 * (l / 16) + 8).
// For bf16 that is exactly one v_mfma_f32_16x16x32_bf16. For fp32 the same 8 elements feed eight
// v_mfma_f32_16x16x4_f32, the s-th taking element s of every lane, so lane group g supplies
// contraction index 8 g + s; summing over s and g covers all 32 in both cases, and operands A and
// B always pair the same elements. The output tile puts element (row 4 (l / 16) + e, column
// l % 16) in register e of lane l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkc {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct f32x8 {
  floatx4 lo, hi;
};

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

// ---- 8-element loads (16 B for bf16, 32 B for fp32; addresses are 16-byte aligned) ----------

__device__ __forceinline__ bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 load8(const float* p) {
  f32x8 r;
  r.lo = *reinterpret_cast<const floatx4*>(p);
  r.hi = *reinterpret_cast<const floatx4*>(p + 4);
  return r;
}

// Streaming loads (non-temporal hint): data read once per launch, such as the cached K/V pages,
// so that what every launch re-reads (block tables, shared positional tables) stays in L2.
__device__ __forceinline__ bf16x8 load8_stream(const bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
}
__device__ __forceinline__ f32x8 load8_stream(const float* p) {
  f32x8 r;
  r.lo = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
  r.hi = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p + 4));
  return r;
}

// Transposing LDS read (ds_read_b64_tr_b16, gfx950): within each group of 16 lanes, the four
// 8-byte rows addressed by lanes 4 r .. 4 r + 3 form row r of a 4 x 16 matrix of 16-bit values,
// and lane i receives its column i. Two reads (rows lo and hi) give 8 elements: [lo col, hi col].
typedef short lds_short4 __attribute__((ext_vector_type(4)));
typedef short lds_short8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 load8_tr(const bf16* lo, const bf16* hi) {
  typedef __attribute__((address_space(3))) lds_short4 LdsShort4;
  const lds_short4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsShort4*)(lo));
  const lds_short4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsShort4*)(hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Direct global -> LDS load (global_load_lds_dwordx4, gfx950): every lane reads 16 bytes at its
// own src, and lane l's bytes land at lds + 16 l (lds is the same for the whole wave). The
// builtin exists only for the device; the host pass, which never runs a kernel body, sees none
// (a host compile of it drops the whole kernel, stub included).
__device__ __forceinline__ void load_lds16(const void* src, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#endif
}

__device__ __forceinline__ void store8(bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ __forceinline__ void store8(float* p, f32x8 v) {
  *reinterpret_cast<floatx4*>(p) = v.lo;
  *reinterpret_cast<floatx4*>(p + 4) = v.hi;
}

__device__ __forceinline__ float get(const bf16x8& v, int e) { return (float)v[e]; }
__device__ __forceinline__ float get(const f32x8& v, int e) { return e < 4 ? v.lo[e] : v.hi[e - 4]; }
__device__ __forceinline__ void set(bf16x8& v, int e, float x) { v[e] = (bf16)x; }
__device__ __forceinline__ void set(f32x8& v, int e, float x) {
  if (e < 4) v.lo[e] = x; else v.hi[e - 4] = x;
}

template <typename T> __device__ __forceinline__ typename Frag<T>::type zero8() {
  typename Frag<T>::type v;
#pragma unroll
  for (int e = 0; e < 8; ++e) set(v, e, 0.f);
  return v;
}

// Zero the elements at positions >= n (any n; <= 0 clears all, >= 8 keeps all) of four
// fragments. bf16 works on whole 32-bit words, so nothing is unpacked.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void zero_from(bf16x8 (&v)[4], int n) {
  u32x4 keep;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    keep[w] = (2 * w < n ? 0x0000ffffu : 0u) | (2 * w + 1 < n ? 0xffff0000u : 0u);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    v[dt] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, v[dt]) & keep);
}
__device__ __forceinline__ void zero_from(f32x8 (&v)[4], int n) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 8; ++e) set(v[dt], e, e < n ? get(v[dt], e) : 0.f);
}

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f(float x) { return (T)x; }

// ---- 16x16x32 products ------------------------------------------------------------------------

__device__ __forceinline__ floatx4 mma(const bf16x8& a, const bf16x8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma(const f32x8& a, const f32x8& b, floatx4 c) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[s], b.lo[s], c, 0, 0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[s], b.hi[s], c, 0, 0, 0);
  return c;
}

// ---- wave-level helpers -----------------------------------------------------------------------

__device__ __forceinline__ float xor_max(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask, 64));
}
__device__ __forceinline__ float xor_sum(float x, int mask) { return x + __shfl_xor(x, mask, 64); }

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one column of a 16x16 MFMA tile) with
// the gfx950 row-swap instructions: v_permlane16_swap / v_permlane32_swap with both operands the
// same register leave, in every lane, the two values of its pair (lower row first), so all four
// lanes combine the same operands in the same order and end with identical results.
__device__ __forceinline__ float pair16_max(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float column_max(float x) { return pair32_max(pair16_max(x)); }
__device__ __forceinline__ float column_sum(float x) { return pair32_sum(pair16_sum(x)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Division by a launch-invariant divisor d (1 <= d < 2^31) as a multiply-high, an add and a shift
// (Granlund and Montgomery, "Division by Invariant Integers using Multiplication", 1994, the
// round-up method): with s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1 < 2^32, the
// quotient n / d is (mulhi(n, m) + n) >> s for 0 <= n < 2^31 (the sum stays below 2^32). The host
// makes the pair once per launch; it replaces the reciprocal-and-correct sequence of a runtime
// division at kernel start.
struct FastDiv {
  uint32_t m, s;
};
inline FastDiv make_fastdiv(int d) {
  uint32_t s = 0;
  while ((1u << s) < (uint32_t)d) ++s;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - (uint64_t)d)) / (uint64_t)d + 1;
  return FastDiv{(uint32_t)m, s};
}
__device__ __forceinline__ int fdiv(int n, FastDiv f) {
  return (int)((__umulhi((uint32_t)n, f.m) + (uint32_t)n) >> f.s);
}

}  // namespace pkc
