// Packed varlen relative-position attention for gfx950 (the offline forward).
//
// Sources: OASR docs, "Model Layer", "The engine-facing surface" (forward_offline_packed: gapless
// varlen rows, attention inside each utterance); "ASR Engine", section 4.1 (sequence packing);
// "Model Layer", fixed_attention_window declaration (Transformer-XL distances i - j). Each
// utterance of length L is the chunk case with no cache and C = L: query i and key j read table
// row L - 1 + j - i of the utterance's 2 L - 1 rows.
//
// Work decomposition. One workgroup of 4 waves per (utterance, head, 64-query tile); wave w owns
// queries [64 t + 16 w, + 16) outright (its own online softmax, no merge). The workgroup walks the
// utterance's keys in 32-key steps: every step's K rows and V rows are staged once in
// double-buffered LDS and read by all four waves, while each wave fetches its own
// band rows (the table rows its 16 queries touch) one step ahead. The per-step math is the shared
// step engine of pkc_step.h. MFMA-bound in principle (6 L^2 D FLOP per utterance and head).
//
// V staging. For bf16, V rows stay in their natural [key][head_dim] order in LDS (one 16-byte
// write per thread) and the PV operand - 8 consecutive keys of one dimension per lane - comes
// from two transposing reads; the 4-dimension chunks of row r are XOR-swizzled by
// 4 ((r & 3) ^ ((r >> 3) & 1)), which gives each of the 8 rows one read of 32 lanes touches its
// own 32-byte bank slot. fp32 stages V transposed to [head_dim][key].
//
// chunked_limited mask ("Model Layer", Nemotron encoder notes; kLimited): query i sees only the
// keys of its own chunk of `chunk` frames and of the `left` chunks before it. A workgroup then
// walks only the keys its 64 queries can see - its own frames plus the trained history, as one
// streaming step per query block - and each query column masks to its own range.
#include "pkc_device.h"
#include "pkc_launch.h"
#include "pkc_step.h"

namespace pkc {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQTile = 16 * kWaves;     // queries per workgroup

template <typename T> constexpr int kKP = kD + 16 / (int)sizeof(T);   // K tile row pitch
template <typename T> constexpr int kVP = 32 + 16 / (int)sizeof(T);   // V^T tile row pitch (fp32)
template <typename T> constexpr bool kTrV = sizeof(T) == 2;            // natural V rows + tr reads
// swizzle of the 4-dimension chunks of natural V row r (bf16)
__device__ __forceinline__ int v_swz(int r) { return 4 * ((r & 3) ^ ((r >> 3) & 1)); }

template <typename T>
struct VarlenArgs {
  const T* q;
  const T* k;
  const T* v;
  const int32_t* cu;
  const T* pos;
  const T* u;
  const T* w;
  T* out;
  int H, Hk, qtiles, total;
  int chunk, left;            // chunked_limited mask (kLimited)
  float scale_log2;
};

template <typename T, bool kLimited>
__global__ void __launch_bounds__(kThreads)
varlen_attn_kernel(VarlenArgs<T> a) {
  typedef typename Frag<T>::type F;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NV = kD / VEC;
  constexpr int KP = kKP<T>;
  constexpr int VP = kVP<T>;
  constexpr int TILE = 32 * KP + (kTrV<T> ? 32 * kD : kD * VP);   // elements of one K + V stage

  __shared__ __align__(16) T s_kv[2 * TILE];
  __shared__ __align__(16) float s_skew[kWaves * kSkewFloats];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m16 = lane & 15;
  const int grp = lane >> 4;

  int id = blockIdx.x;
  const int qt = id % a.qtiles;
  id /= a.qtiles;
  const int h = id % a.H;
  const int s = id / a.H;
  const int lo = clampi(a.cu[s], 0, a.total);
  const int L = clampi(a.cu[s + 1], lo, a.total) - lo;
  if (qt * kQTile >= L) return;  // uniform over the workgroup
  const int hk = h / (a.H / a.Hk);
  const size_t krow = (size_t)a.Hk * kD;      // elements between consecutive frames of k / v
  const T* kseg = a.k + (size_t)lo * krow + (size_t)hk * kD;
  const T* vseg = a.v + (size_t)lo * krow + (size_t)hk * kD;
  const size_t prow = (size_t)a.H * kD;
  const T* ptab = a.pos + (size_t)(2 * lo) * prow + (size_t)h * kD;
  const int q0 = qt * kQTile + 16 * wave;       // this wave's first query
  const int R0 = L - 1;                         // table row of (i, j) is R0 + j - i
  const int rlo = 0, rhi = 2 * L - 2;
  const int qlast = q0 + 15;
  auto band_row = [&](int r) { return ptab + (size_t)(uint32_t)clampi(r, rlo, rhi) * prow; };

  // queries with the biases, pre-scaled into log2 units
  F qu[2], qv[2];
  {
    const T* qrow = a.q + ((size_t)(lo + min(q0 + m16, L - 1)) * a.H + h) * kD;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int d0 = 32 * half + 8 * grp;
      const F qq = load8(qrow + d0);
      const F uu = load8(a.u + h * kD + d0);
      const F ww = load8(a.w + h * kD + d0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        set(qu[half], e, (get(qq, e) + get(uu, e)) * a.scale_log2);
        set(qv[half], e, (get(qq, e) + get(ww, e)) * a.scale_log2);
      }
    }
  }

  // cooperative staging of one 32-key step: 32 K rows and the same 32 V rows, transposed
  // (keys past L are zero in V, so masked probabilities meet finite values)
  constexpr int NLD = (32 * NV + kThreads - 1) / kThreads;   // 16-byte vectors per thread per tensor
  struct Rows { uint4 k[NLD], v[NLD]; };
  Rows ra, rb;   // two steps in flight
  auto fetch = [&](Rows& rr, int j0) {
    uint4* kr = rr.k;
    uint4* vr = rr.v;
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int idx = tid + kThreads * it;
      const int r = idx / NV;
      const int dv = (idx % NV) * VEC;
      kr[it] = uint4{0u, 0u, 0u, 0u};
      vr[it] = uint4{0u, 0u, 0u, 0u};
      if (idx < 32 * NV && j0 + r < L) {
        kr[it] = *reinterpret_cast<const uint4*>(kseg + (size_t)(j0 + r) * krow + dv);
        vr[it] = *reinterpret_cast<const uint4*>(vseg + (size_t)(j0 + r) * krow + dv);
      }
    }
  };
  auto stash = [&](const Rows& rr, T* st) {
    const uint4* kr = rr.k;
    const uint4* vr = rr.v;
    T* sk = st;
    T* sv = st + 32 * KP;
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int idx = tid + kThreads * it;
      if (idx >= 32 * NV) continue;
      const int r = idx / NV;
      const int dv = (idx % NV) * VEC;
      *reinterpret_cast<uint4*>(sk + r * KP + dv) = kr[it];
      if constexpr (kTrV<T>) {
        *reinterpret_cast<uint4*>(sv + r * kD + 4 * ((dv >> 2) ^ v_swz(r))) = vr[it];
      } else {
        const T* e = reinterpret_cast<const T*>(&vr[it]);
#pragma unroll
        for (int c = 0; c < VEC; ++c) sv[(dv + c) * VP + r] = e[c];
      }
    }
  };
  // band tiles 1 and 2 of a step (tile 0 is the previous step's tile 2)
  F pb[2][2];
  auto fetch_band = [&](int j0) {
    const int rb = R0 + j0 - qlast;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const T* row = band_row(rb + 16 * (t + 1) + m16) + 8 * grp;
      pb[t][0] = load8(row);
      pb[t][1] = load8(row + 32);
    }
  };

  Softmax st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) st.o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float* s_g = s_skew + wave * kSkewFloats;

  // the keys this workgroup's queries can see: all of the utterance, or with the chunked_limited
  // mask the first visible key of its first query to the last of its last query; and per query
  // column (this lane's query, clamped into the utterance) its own range [k_lo_q, k_hi_q)
  int j_first = 0, j_end = L, k_lo_q = 0, k_hi_q = L;
  if constexpr (kLimited) {
    const int left = min(a.left, L);   // more chunks than frames sees everything anyway
    const int tq0 = qt * kQTile;
    const int tq1 = min(tq0 + kQTile, L) - 1;
    j_first = max(0, (tq0 / a.chunk - left) * a.chunk);
    j_end = min(L, (tq1 / a.chunk + 1) * a.chunk);
    const int iq = min(q0 + m16, L - 1);
    k_lo_q = max(0, (iq / a.chunk - left) * a.chunk);
    k_hi_q = min(L, (iq / a.chunk + 1) * a.chunk);
  }
  const int s_first = j_first >> 5;
  const int nsteps = ((j_end + 31) >> 5) - s_first;
  floatx4 g_prev;
  {
    const T* row = band_row(R0 + 32 * s_first - qlast + m16) + 8 * grp;
    const F p_lo = load8(row);
    const F p_hi = load8(row + 32);
    g_prev = mma(p_lo, qv[0], floatx4{0.f, 0.f, 0.f, 0.f});
    g_prev = mma(p_hi, qv[1], g_prev);
  }
  fetch(ra, 32 * s_first);
  if (nsteps > 1) fetch(rb, 32 * s_first + 32);
  fetch_band(32 * s_first);
  stash(ra, s_kv);
  __syncthreads();
  // one step (index `step` from the first visible one): registers `nxt` already hold step + 1,
  // `fre` receives step + 2
  auto do_step = [&](int step, Rows& nxt, Rows& fre) {
    const int j0 = 32 * (s_first + step);
    const T* cur = s_kv + (step & 1) * TILE;
    if (step + 2 < nsteps) fetch(fre, j0 + 64);
    F kf[2][2], vf[4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const T* row = cur + (8 * (m16 >> 2) + 4 * tt + (m16 & 3)) * KP + 8 * grp;
      kf[tt][0] = load8(row);
      kf[tt][1] = load8(row + 32);
    }
    if constexpr (kTrV<T>) {
      // lane m16 of the group addresses row 8 grp + m16 / 4 (+ 4), dimensions 16 dt + 4 (m16 % 4)
      const int r = 8 * grp + (m16 >> 2);
      const T* lo = cur + 32 * KP + r * kD;
      const int sw = v_swz(r);   // the same for row r + 4
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int c = 4 * (((4 * dt) + (m16 & 3)) ^ sw);
        vf[dt] = load8_tr(lo + c, lo + 4 * kD + c);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vf[dt] = load8(cur + 32 * KP + (16 * dt + m16) * VP + 8 * grp);
    }
    floatx4 g1 = mma(pb[0][0], qv[0], floatx4{0.f, 0.f, 0.f, 0.f});
    g1 = mma(pb[0][1], qv[1], g1);
    floatx4 g2 = mma(pb[1][0], qv[0], floatx4{0.f, 0.f, 0.f, 0.f});
    g2 = mma(pb[1][1], qv[1], g2);
    if (step + 1 < nsteps) fetch_band(j0 + 32);
    if constexpr (kLimited) {
      float x[2][4];
      skew_scores<T>(kf, qu, g_prev, g1, g2, s_g, x);
      softmax_pv<T, true>(st, x, vf, k_lo_q - j0, k_hi_q - j0);
    } else if (j0 + 32 <= L) {
      step_compute<T, false>(st, kf, vf, qu, g_prev, g1, g2, s_g, 32);
    } else {
      step_compute<T, true>(st, kf, vf, qu, g_prev, g1, g2, s_g, L - j0);
    }
    g_prev = g2;
    if (step + 1 < nsteps) stash(nxt, s_kv + ((step + 1) & 1) * TILE);
    __syncthreads();
  };
  for (int step = 0; step < nsteps; step += 2) {
    do_step(step, rb, ra);
    if (step + 1 < nsteps) do_step(step + 1, ra, rb);
  }

  // finish: every wave owns its 16 queries
  st.l = column_sum(st.l);
  const float inv = 1.f / st.l;
  const int i = q0 + m16;
  if (i < L) {
    T* dst = a.out + ((size_t)(lo + i) * a.H + h) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[16 * dt + 4 * grp + e] = from_f<T>(st.o[dt][e] * inv);
  }
}

template <typename T>
hipError_t launch_varlen_t(const VarlenParams& p, hipStream_t stream) {
  VarlenArgs<T> a;
  a.q = (const T*)p.q;
  a.k = (const T*)p.k;
  a.v = (const T*)p.v;
  a.cu = p.cu_seqlens;
  a.pos = (const T*)p.pos;
  a.u = (const T*)p.pos_bias_u;
  a.w = (const T*)p.pos_bias_v;
  a.out = (T*)p.out;
  a.H = p.n_head;
  a.Hk = p.n_kv_head;
  a.qtiles = (p.max_seqlen + kQTile - 1) / kQTile;
  a.total = p.total;
  const float scale = p.softmax_scale > 0.f ? p.softmax_scale : 1.f / sqrtf((float)p.head_dim);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.chunk = p.mask_chunk;
  a.left = p.mask_left_chunks;
  const dim3 grid((unsigned)p.num_seqs * p.n_head * a.qtiles);
  if (p.mask_chunk > 0)
    hipLaunchKernelGGL((varlen_attn_kernel<T, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((varlen_attn_kernel<T, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_varlen_attn(pkc_dtype dtype, const VarlenParams& p, hipStream_t stream) {
  return dtype == PKC_BF16 ? launch_varlen_t<bf16>(p, stream) : launch_varlen_t<float>(p, stream);
}

}  // namespace pkc
