// Packed varlen relative-position attention for gfx950 (the offline forward).
//
// Sources: OASR docs, "Model Layer", "The engine-facing surface" (forward_offline_packed: gapless
// varlen rows, attention inside each utterance); "ASR Engine", section 4.1 (sequence packing);
// "Model Layer", fixed_attention_window declaration (Transformer-XL distances i - j). Each
// utterance of length L is the chunk case with no cache and C = L.
//
// Work decomposition. One workgroup of kWaves wavefronts per (utterance, head, 16-query tile). The T keys are cut into 32-key steps; wave w takes steps w, w + kWaves, ... and keeps its
// own online-softmax state; the waves merge through LDS at the end in a fixed order, so a row's
// result depends only on its own length (never on the cohort or the batch width).
//
// Per step the wave computes, with 16x16 MFMA tiles whose columns are the 16 queries:
//   S^T = K . (q + u)^T          two tiles (32 keys x 16 queries), contraction over head_dim
//   G^T = P_band . (q + v)^T     three tiles: the 47 table rows this step can touch
//   O^T += V^T . softmax(S + Bd)^T
// Key order inside a step is permuted so that the 8 scores a lane holds after the S^T tiles are
// exactly the 8 consecutive keys it must feed to the PV product (tile 0 row 4a + e is key 8a + e,
// tile 1 row 4a + e is key 8a + 4 + e). V pages are stored transposed, so the V^T operand is one
// 16-byte load of 8 consecutive frames per lane. The relative shift Bd[i][j] = G[i][j + 15 - i']
// (i' = query inside the tile) moves data between lanes of the same query column; it goes through
// a per-wave LDS tile.
//
// Table geometry: the row for (query i, key j) is R0 + j - i, where R0 = centre - cache. Only rows
// [R0 - (C - 1), R0 + T - 1] are ever read.
#include <math.h>

#include "pkc_device.h"
#include "pkc_launch.h"

namespace pkc {

namespace {

constexpr int kD = 64;          // head_dim of these kernels
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kWaveLds = kD * 16 + 32;  // floats per wave: O^T tile + m + l (band tile aliases it)

// ------------------------------------------------------------------------------------------------
// Key/value sources
// ------------------------------------------------------------------------------------------------

// Keys of one packed utterance, rows [0, T_len) starting at k / v (stride Hk * D per frame).
template <typename T>
struct PackedSource {
  const T* k;
  const T* v;
  int Hk, hk, T_len;

  __device__ __forceinline__ const T* k_row(int key) const {
    return k + ((size_t)key * Hk + hk) * kD;
  }
  __device__ __forceinline__ bool v_whole(int) const { return false; }
  __device__ __forceinline__ const T* v_group(int) const { return v; }
  __device__ __forceinline__ size_t v_dim_stride() const { return 1; }
  __device__ __forceinline__ float v_elem(int key, int d) const {
    return to_f(v[((size_t)key * Hk + hk) * kD + d]);
  }
};

// ------------------------------------------------------------------------------------------------
// One 32-key step
// ------------------------------------------------------------------------------------------------

template <typename T>
struct StepData {
  typedef typename Frag<T>::type F;
  F k[2][2];   // [key tile][head_dim half]
  F v[4];      // [16-dim tile]
  F p[3][2];   // [band tile][head_dim half]
};

template <typename T, typename Src>
__device__ __forceinline__ void load_step(StepData<T>& sd, const Src& src, int j0, const T* ptab,
                                          size_t prow_stride, int band0, int rlo, int rhi,
                                          int lane) {
  const int m16 = lane & 15;
  const int grp = lane >> 4;
  const int T_len = src.T_len;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int key = min(j0 + 8 * (m16 >> 2) + 4 * tt + (m16 & 3), T_len - 1);
    const T* row = src.k_row(key);
    sd.k[tt][0] = load8(row + 8 * grp);
    sd.k[tt][1] = load8(row + 32 + 8 * grp);
  }
  const int kg = j0 + 8 * grp;
  if (src.v_whole(kg)) {
    const T* base = src.v_group(kg);
    const size_t ds = src.v_dim_stride();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) sd.v[dt] = load8(base + (size_t)(16 * dt + m16) * ds);
  } else {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kg + e;
        set(sd.v[dt], e, key < T_len ? src.v_elem(key, 16 * dt + m16) : 0.f);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int r = clampi(band0 + 16 * t + m16, rlo, rhi);
    const T* row = ptab + (size_t)r * prow_stride;
    sd.p[t][0] = load8(row + 8 * grp);
    sd.p[t][1] = load8(row + 32 + 8 * grp);
  }
}

// Attention of one 16-query tile (queries q0 .. q0 + 15 of C) over the T keys of `src`, written
// to out_row0 + i * out_stride. q_row0 + i * q_stride is query row i.
template <typename T, typename Src>
__device__ __forceinline__ void attend_tile(const Src& src, const T* q_row0, size_t q_stride,
                                            const T* u_h, const T* w_h, const T* ptab,
                                            size_t prow_stride, int R0, int C, int q0,
                                            float scale_log2, T* out_row0, size_t out_stride,
                                            float* s_wave) {
  typedef typename Frag<T>::type F;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m16 = lane & 15;
  const int grp = lane >> 4;
  const int T_len = src.T_len;

  F qu[2], qv[2];
  {
    const T* qrow = q_row0 + (size_t)min(q0 + m16, C - 1) * q_stride;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int d0 = 32 * half + 8 * grp;
      const F qq = load8(qrow + d0);
      const F uu = load8(u_h + d0);
      const F ww = load8(w_h + d0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        set(qu[half], e, get(qq, e) + get(uu, e));
        set(qv[half], e, get(qq, e) + get(ww, e));
      }
    }
  }
  const int rlo = R0 - (C - 1);
  const int rhi = R0 + T_len - 1;
  const int qlast = q0 + 15;

  float* s_g = s_wave + wave * kWaveLds;
  const int nsteps = (T_len + 31) / 32;
  float m_run = -INFINITY;
  float l_run = 0.f;
  floatx4 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  StepData<T> cur, nxt;
  int s = wave;
  if (s < nsteps) load_step(cur, src, 32 * s, ptab, prow_stride, R0 + 32 * s - qlast, rlo, rhi, lane);
  for (; s < nsteps; s += kWaves) {
    const int j0 = 32 * s;
    const int sn = s + kWaves;
    if (sn < nsteps)
      load_step(nxt, src, 32 * sn, ptab, prow_stride, R0 + 32 * sn - qlast, rlo, rhi, lane);
    floatx4 sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sc[tt] = mma(cur.k[tt][0], qu[0], floatx4{0.f, 0.f, 0.f, 0.f});
      sc[tt] = mma(cur.k[tt][1], qu[1], sc[tt]);
    }
    floatx4 gb[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      gb[t] = mma(cur.p[t][0], qv[0], floatx4{0.f, 0.f, 0.f, 0.f});
      gb[t] = mma(cur.p[t][1], qv[1], gb[t]);
    }
    // Relative shift through LDS: G^T[row][query] -> s_g[row * 16 + query].
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_g[(16 * t + 4 * grp + e) * 16 + m16] = gb[t][e];
    __builtin_amdgcn_wave_barrier();
    float sv[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int koff = 8 * grp + 4 * tt + e;
        const float bd = s_g[(koff + 15 - m16) * 16 + m16];
        float x = (sc[tt][e] + bd) * scale_log2;
        x = (j0 + koff < T_len) ? x : -INFINITY;
        sv[tt][e] = x;
        mx = fmaxf(mx, x);
      }
    __builtin_amdgcn_wave_barrier();
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    F pf;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = fast_exp2(sv[tt][e] - m_new);
        l_run += pe;
        set(pf, 4 * tt + e, pe);
      }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = mma(cur.v[dt], pf, o[dt]);
    m_run = m_new;
    cur = nxt;
  }

  // Merge the waves' partial states in a fixed order.
  l_run = xor_sum(l_run, 16);
  l_run = xor_sum(l_run, 32);
  float* s_o = s_wave + wave * kWaveLds;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[(16 * dt + 4 * grp + e) * 16 + m16] = o[dt][e];
  if (grp == 0) {
    s_o[kD * 16 + m16] = m_run;
    s_o[kD * 16 + 16 + m16] = l_run;
  }
  __syncthreads();
  for (int x = threadIdx.x; x < 16 * (kD / 4); x += kThreads) {
    const int il = x & 15;
    const int d0 = (x >> 4) * 4;
    const int i = q0 + il;
    if (i >= C) continue;
    float mmax = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mmax = fmaxf(mmax, s_wave[w * kWaveLds + kD * 16 + il]);
    float lsum = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* so = s_wave + w * kWaveLds;
      const float f = fast_exp2(so[kD * 16 + il] - mmax);
      lsum += f * so[kD * 16 + 16 + il];
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] += f * so[(d0 + k) * 16 + il];
    }
    const float inv = 1.f / lsum;
    T* dst = out_row0 + (size_t)i * out_stride + d0;
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = from_f<T>(acc[k] * inv);
  }
}

// ------------------------------------------------------------------------------------------------
// Packed varlen kernel: each utterance is the chunk case with cache 0 and C = L.
// ------------------------------------------------------------------------------------------------

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
  float scale_log2;
};

template <typename T>
__global__ void __launch_bounds__(kThreads)
varlen_attn_kernel(VarlenArgs<T> a) {
  extern __shared__ float smem[];
  int id = blockIdx.x;
  const int qt = id % a.qtiles;
  id /= a.qtiles;
  const int h = id % a.H;
  const int s = id / a.H;
  const int lo = clampi(a.cu[s], 0, a.total);
  const int L = clampi(a.cu[s + 1], lo, a.total) - lo;
  if (qt * 16 >= L) return;  // uniform over the workgroup
  const int hk = h / (a.H / a.Hk);
  PackedSource<T> src;
  src.k = a.k + (size_t)lo * a.Hk * kD;
  src.v = a.v + (size_t)lo * a.Hk * kD;
  src.Hk = a.Hk;
  src.hk = hk;
  src.T_len = L;
  const T* ptab = a.pos + (size_t)(2 * lo) * a.H * kD + (size_t)h * kD;
  const size_t stride = (size_t)a.H * kD;
  attend_tile<T>(src, a.q + ((size_t)lo * a.H + h) * kD, stride, a.u + h * kD, a.w + h * kD, ptab,
                 stride, L - 1, L, qt * 16, a.scale_log2, a.out + ((size_t)lo * a.H + h) * kD,
                 stride, smem);
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
  a.qtiles = (p.max_seqlen + 15) / 16;
  a.total = p.total;
  const float scale = p.softmax_scale > 0.f ? p.softmax_scale : 1.f / sqrtf((float)p.head_dim);
  a.scale_log2 = scale * 1.4426950408889634f;
  const size_t smem = (size_t)kWaves * kWaveLds * sizeof(float);
  const dim3 grid((unsigned)p.num_seqs * p.n_head * a.qtiles);
  hipLaunchKernelGGL(varlen_attn_kernel<T>, grid, dim3(kThreads), smem, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_varlen_attn(pkc_dtype dtype, const VarlenParams& p, hipStream_t stream) {
  return dtype == PKC_BF16 ? launch_varlen_t<bf16>(p, stream) : launch_varlen_t<float>(p, stream);
}

}  // namespace pkc
