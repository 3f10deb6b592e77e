// The 32-key attention step shared by the paged chunk kernel and the packed varlen kernel.
//
// Layout convention (16x16 MFMA tiles whose columns are the 16 queries of a tile): a lane holds
// query column m16 = lane % 16 and, after the score tiles, the 8 consecutive keys
// 8 kg + [0, 8) of the step, kg = key_group(lane / 16) (tile 0 row 4a + e is key 8 kg(a) + e, tile 1
// row 4a + e is key 8 kg(a) + 4 + e), which are exactly the contraction elements it feeds to the
// PV product in slots 8 (lane / 16) + [0, 8). Scores are in log2 units (the softmax scale and
// log2 e are folded into q + u and q + v).
//
// Relative position: the band product G^T[r][i] = p_r . (q_i + v) for the 48 table rows
// [rb, rb + 48) of the step, rb = R0 + j0 - (q0 + 15) (table row of query i and key j is
// R0 + j - i), gives Bd[i][j] = G^T[j - j0 + 15 - (i - q0)][i]: a shift inside each query column,
// done through a per-wave LDS tile.
#pragma once

#include <math.h>

#include "pkc_device.h"

namespace pkc {

constexpr int kD = 64;                  // head_dim of the attention kernels
constexpr int kSkewPitch = 52;          // floats per query column of the skew tile (48 rows used;
                                        // 52 puts the 16-byte writes of 8 columns on distinct banks)
constexpr int kSkewFloats = kSkewPitch * 16;
constexpr float kRescaleLog2 = 8.f;     // headroom before the running max moves

// Key group of lane group g (lanes 16 g .. 16 g + 15) inside a 32-key step: g itself, or with
// kPermGrp groups 1 and 2 swapped. Swapped, the two lane groups of a half-wave hold keys 16 apart,
// and their reads of the shifted position values (one column, rows 16 apart, any odd column
// pitch) fall on distinct banks; with the natural order the rows are 8 apart and half of them
// pair up on a bank (measured on gfx950).
template <bool kPermGrp>
__device__ __forceinline__ int key_group(int g) {
  return kPermGrp ? (((g & 1) << 1) | (g >> 1)) : g;
}

// Running softmax state of one lane (one query column, 8 keys of each step): m the running
// maximum (the per-key steps; the folded steps keep theirs in RunRef), l this lane's part of the
// row sum, o the output accumulators. The packed kernel keeps the row sum in ls instead: the
// product of an all-ones operand with the step's probabilities on the MFMA, the same value in
// every register (the column's sum of the bf16-rounded probabilities that also weight the values).
struct Softmax {
  float m, l;
  floatx4 o[4];
  floatx4 ls;
};

template <typename T> __device__ __forceinline__ typename Frag<T>::type ones8() {
  typename Frag<T>::type v;
#pragma unroll
  for (int e = 0; e < 8; ++e) set(v, e, 1.f);
  return v;
}

// Scores of one 32-key step, WeNet convention (no shift): the table has one row per key, in the
// same permuted order as the key tiles, and S^T = K (q+u)^T + P (q+v)^T.
template <typename T>
__device__ __forceinline__ void per_key_scores(const typename Frag<T>::type (&kf)[2][2],
                                               const typename Frag<T>::type (&pf)[2][2],
                                               const typename Frag<T>::type (&qu)[2],
                                               const typename Frag<T>::type (&qv)[2],
                                               float (&x)[2][4]) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    floatx4 sc = mma(kf[tt][0], qu[0], floatx4{0.f, 0.f, 0.f, 0.f});
    sc = mma(kf[tt][1], qu[1], sc);
    sc = mma(pf[tt][0], qv[0], sc);
    sc = mma(pf[tt][1], qv[1], sc);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[tt][e] = sc[e];
  }
}

// Online softmax and PV of one step from its scores. kMask: only keys k_lo <= key < k_hi of the
// step count for this lane's query column (bounds may differ between columns); a column with no
// key seen yet contributes nothing.
template <typename T, bool kMask, bool kPermGrp = false>
__device__ __forceinline__ void softmax_pv(Softmax& st, float (&x)[2][4],
                                           const typename Frag<T>::type (&vf)[4], int k_lo,
                                           int k_hi) {
  typedef typename Frag<T>::type F;
  const int kg = key_group<kPermGrp>((threadIdx.x & 63) >> 4);
  float mx = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = 8 * kg + 4 * tt + e;
      if (kMask) x[tt][e] = (key >= k_lo && key < k_hi) ? x[tt][e] : -INFINITY;
      mx = fmaxf(mx, x[tt][e]);
    }
  mx = column_max(mx);
  const bool move = mx > st.m + kRescaleLog2;
  if (__ballot(move) != 0) {
    const float m_new = move ? mx : st.m;
    // (a column that does not move keeps its scale; computing it as exp2(m - m) would give NaN
    // for a column that has seen no key yet, m = -inf)
    const float alpha = move ? fast_exp2(st.m - m_new) : 1.f;
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.o[dt] *= alpha;
    st.m = m_new;
  }
  // (with a mask, a column may still have seen nothing: its max is -inf, and every probability
  // of it must be 0, not exp2(-inf - -inf))
  const float m_ref = (kMask && st.m == -INFINITY) ? 0.f : st.m;
  F pf;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pe = fast_exp2(x[tt][e] - m_ref);
      st.l += pe;
      set(pf, 4 * tt + e, pe);
    }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) st.o[dt] = mma(vf[dt], pf, st.o[dt]);
}

// Running-max reference of a query column in the folded form (step_fold, and the packed kernel's
// multi-tile step). m is the running maximum (log2 units, -inf before the column's first visible
// key); scores are formed relative to r = m, or 0 while m = -inf: -r starts the accumulation of
// every band product, and each score reads exactly one band value, so a score is x - r without a
// subtraction. thr is the score (relative to r) past which the lazy rescale must run:
// kRescaleLog2, or -inf while m = -inf (the first visible key must set m).
struct RunRef {
  float m, r, thr;
  floatx4 nr;   // {-r, -r, -r, -r}: the band products' accumulator start
};

__device__ __forceinline__ void runref_init(RunRef& rr) {
  rr.m = -INFINITY;
  rr.r = 0.f;
  rr.thr = -INFINITY;
  rr.nr = floatx4{0.f, 0.f, 0.f, 0.f};
}

// A new running maximum for the column from this lane's maximum lm over its keys (relative to
// r): the rescale of the accumulators when the column moves, and the shift d = r_new - r that
// every value still relative to the old reference must drop. Call from a branch uniform over the
// wave (the column maximum is a cross-lane reduction).
// (l: the row sum, per-lane partial or the MFMA's floatx4)
template <typename L>
__device__ __forceinline__ float runref_move(RunRef& rr, float lm, floatx4 (&o)[4], L& l) {
  const float mx = column_max(lm) + rr.r;   // the column's maximum
  const bool mv = mx > rr.m + kRescaleLog2;
  const float m_new = mv ? mx : rr.m;
  // (a column that does not move keeps its scale; one that moves for the first time has nothing
  // accumulated yet, exp2(-inf) = 0)
  const float alpha = mv ? fast_exp2(rr.m - m_new) : 1.f;
  l *= alpha;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
  const float r_new = m_new == -INFINITY ? 0.f : m_new;
  const float d = r_new - rr.r;
  rr.m = m_new;
  rr.r = r_new;
  rr.thr = m_new == -INFINITY ? -INFINITY : kRescaleLog2;
  rr.nr = floatx4{-r_new, -r_new, -r_new, -r_new};
  return d;
}

// One whole 32-key Transformer-XL step with the running-max reference folded in: g0, g1 and g2
// were accumulated onto rr.nr, so the shifted band values, and the scores with them, come out
// relative to r, and the probabilities are exp2 of the scores. The lazy-rescale decision is a
// per-lane test against rr.thr and one ballot; the column maxima, the rescale and the re-basing
// of the scores and of g2 (the carried band product of the next step) run only in that rare
// branch. The decisions are those of the plain form (rescale when a column maximum passes m by
// kRescaleLog2). kMask: keys at or past valid_keys are excluded
// (never all of a step's keys). The row sums stay per-lane in st.l (column_sum at the end).
template <typename T, bool kMask, bool kPermGrp = false>
__device__ __forceinline__ void step_fold(Softmax& st, RunRef& rr,
                                          const typename Frag<T>::type (&kf)[2][2],
                                          const typename Frag<T>::type (&vf)[4],
                                          const typename Frag<T>::type (&qu)[2],
                                          const floatx4& g0, const floatx4& g1, floatx4& g2,
                                          float* s_g, int valid_keys) {
  typedef typename Frag<T>::type F;
  const int lane = threadIdx.x & 63;
  const int m16 = lane & 15;
  const int grp = lane >> 4;
  floatx4 sc[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    sc[tt] = mma(kf[tt][0], qu[0], floatx4{0.f, 0.f, 0.f, 0.f});
    sc[tt] = mma(kf[tt][1], qu[1], sc[tt]);
  }
  float* colw = s_g + m16 * kSkewPitch + 4 * grp;
  *reinterpret_cast<floatx4*>(colw) = g0;
  *reinterpret_cast<floatx4*>(colw + 16) = g1;
  *reinterpret_cast<floatx4*>(colw + 32) = g2;
  __builtin_amdgcn_wave_barrier();
  const int kg = key_group<kPermGrp>(grp);
  const float* colr = s_g + m16 * kSkewPitch + 15 - m16 + 8 * kg;
  float x[2][4];
  float lm = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = sc[tt][e] + colr[4 * tt + e];
      if (kMask) v = (8 * kg + 4 * tt + e < valid_keys) ? v : -INFINITY;
      x[tt][e] = v;
      lm = fmaxf(lm, v);
    }
  __builtin_amdgcn_wave_barrier();
  if (__ballot(lm > rr.thr) != 0) {
    const float d = runref_move(rr, lm, st.o, st.l);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[tt][e] -= d;
    g2 -= d;
  }
  F pf;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pe = fast_exp2(x[tt][e]);
      st.l += pe;
      set(pf, 4 * tt + e, pe);
    }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) st.o[dt] = mma(vf[dt], pf, st.o[dt]);
}

}  // namespace pkc
