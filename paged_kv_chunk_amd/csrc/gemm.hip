// The GEMMs either side of the paged attention, for gfx950: y = x W^T (+ b) on MFMA.
//
// Sources: OASR docs, "Model Layer", the decoder notes (WeNet's linear_q / linear_k / linear_v /
// linear_out over the attention core, an activation folded into the GEMM epilogue) and "Heads";
// "ASR Engine", section 9 (the positional projection of the relative-position table, sized by the
// cache rung) and "Model Layer", "Three optional encoder declarations" (one shared table, or a
// projection per row); "ASR Engine", section 4.3 (the chunk's K/V go into the stream's pages
// before the attention reads them).
//
// One kernel, three uses, picked at compile time:
//   plain       y[M, N] = x[M, K] W[N, K]^T + b                       (linear_out, any linear)
//   Q/K/V       the chunk's fused projection; the epilogue writes q [B, C, H, D] and appends the
//               K/V rows straight into the stream's pages (column-blocked K, transposed V), the
//               way paged_kv_append does, so the chunk's K/V never go through HBM twice
//   positional  x is the sinusoidal table itself, generated in registers (row m = t rows + r
//               holds position pos_start[t] + step r), so only W is read: linear_pos
//
// Work decomposition. A workgroup of 4 waves computes a BM x BN tile of y (128 x 128, 128 x 64
// or 64 x 64: whichever gives the least work on the busiest CU when all tiles run at once), each
// wave a quarter. The contraction runs in 32-deep stages, each stage's x and W rows staged once in
// LDS and read by the waves that share them. W is the MFMA's first operand: a lane ends with 4
// consecutive output features of one row, stored with one 8-byte (bf16) or 16-byte (fp32) write.
//
// Staging, bf16 with d_model 256, 512 or 1024 (the projections of the streaming cohorts): direct
// global -> LDS loads (global_load_lds_dwordx4; each lane's 16 bytes land at the wave's LDS base
// + 16 lane, probed on the GPU) into a ring of 3 stages, 2 in flight. A stage is 64 dims deep,
// so each row's whole 128-byte line is one request; it is a run of 1 KB blocks of 8 rows, the
// 16-byte chunk c of row r (within its group of 16) at chunk c ^ (((r >> 1) ^ (r << 2)) & 7), so
// the 16 rows of a fragment read fall on distinct banks (for 32 banks per quarter-wave and 64 per
// half-wave alike; checked on the CPU). The stage loop is unrolled at compile
// time (the stage count is a template argument): every ring slot is its own LDS array and every
// wait names its exact count, so the compiler can tell a slot being read from one being filled.
// Otherwise (fp32, the generated sinusoid, other widths) the rows go through registers, two
// stages ahead, into double-buffered LDS with a padded row pitch.
#include <math.h>

#include "pkc_device.h"
#include "pkc_launch.h"

namespace pkc {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;   // contraction depth of one stage

enum Epilogue { kPlain = 0, kQKV = 1 };

template <typename T> constexpr int kLP = kBK + 16 / (int)sizeof(T);   // LDS row pitch (elements)

template <typename T>
struct GemmArgs {
  const T* x;             // [M, K]; unused for the positional source
  const T* w;             // [N, K]
  const T* bias;          // [N] or null
  T* y;                   // [M, N]; the Q/K/V epilogue: q [B, C, H, D], its first H D columns
  int M, N, K, tiles_n;
  // positional source: row m = t rows + r holds position pos0 + step r, pos0 = pos_start[t] or
  // pos_first; column 2 i / 2 i + 1 is sin / cos of position 10000^(-2 i / K)
  const int32_t* pos_start;
  int pos_first, pos_step, rows;
  float neg_log2_base_per_col;   // -log2(10000) / K
  // Q/K/V epilogue
  T* k_pool;
  T* v_pool;
  const int32_t* bt;
  const int32_t* cs;
  const int32_t* lens;
  const int32_t* ws;
  int C, HD, Hk, D, S, num_blocks, max_blocks, max_cache;
};

template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&v)[4]);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, const float (&v)[4]) {
  bf16x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
  *reinterpret_cast<bf16x4*>(p) = o;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const float (&v)[4]) {
  *reinterpret_cast<floatx4*>(p) = floatx4{v[0], v[1], v[2], v[3]};
}

// Tile of a workgroup. Workgroups go to the 8 XCDs round-robin (block b to XCD b % 8); each XCD
// takes one contiguous run of the row-major tile order instead, so the x rows of a tile row are
// read into one XCD's L2 (only the small W is read by every XCD).
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int xcd = b & 7, local = b >> 3;
  const int per = total >> 3, extra = total & 7;
  const int logical = xcd < extra ? xcd * (per + 1) + local
                                  : extra * (per + 1) + (xcd - extra) * per + local;
  tm = logical / tiles_n;
  tn = logical - tm * tiles_n;
}

// Epilogue: the lane holds y[m][n .. n + 3] of every 16 x 16 product tile (rows mb + 16 fm + m16,
// features nb + 16 fn + 4 grp); plain rows, or the Q/K/V split with the K/V rows appended into
// the pages. Two neighbouring tiles go out together: after one row swap between lane groups
// (v_permlane16_swap: groups 0 <-> 1 and 2 <-> 3), every lane holds 8 consecutive features of
// its row - tile fn's [0, 8) or [8, 16) for groups 0 and 2, tile fn + 1's for groups 1 and 3 -
// stored with one 16-byte write (two in fp32), so a row's 32 features leave as 64 (128)
// contiguous bytes. V (transposed pages: consecutive features are S slots apart) is written
// element by element.

// 8 consecutive features: v[0..3] of tile A and of tile B before the swap, the lane's 8 after
template <typename T>
__device__ __forceinline__ void swap_pair(const float (&va)[4], const float (&vb)[4], T* dst);
template <>
__device__ __forceinline__ void swap_pair<bf16>(const float (&va)[4], const float (&vb)[4], bf16* dst) {
  uint32_t a[2], b[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    bf16x2_t pa{(bf16)va[2 * h], (bf16)va[2 * h + 1]};
    bf16x2_t pb{(bf16)vb[2 * h], (bf16)vb[2 * h + 1]};
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, pa),
                                                    __builtin_bit_cast(uint32_t, pb), false, false);
    a[h] = r[0];
    b[h] = r[1];
  }
  *reinterpret_cast<u32x4*>(dst) = u32x4{a[0], a[1], b[0], b[1]};
}
template <>
__device__ __forceinline__ void swap_pair<float>(const float (&va)[4], const float (&vb)[4], float* dst) {
  float a[4], b[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(va[e]), __float_as_uint(vb[e]),
                                                    false, false);
    a[e] = __uint_as_float(r[0]);
    b[e] = __uint_as_float(r[1]);
  }
  *reinterpret_cast<floatx4*>(dst) = floatx4{a[0], a[1], a[2], a[3]};
  *reinterpret_cast<floatx4*>(dst + 4) = floatx4{b[0], b[1], b[2], b[3]};
}

template <typename T, int kEpi, int FM, int FN>
__device__ __forceinline__ void store_tiles(const GemmArgs<T>& a, const floatx4 (&acc)[FN][FM],
                                            int mb, int nb, int m16, int grp) {
  static_assert(FN % 2 == 0, "tiles go out in pairs");
  // this lane's 8 features after the swap, relative to the pair's first column
  const int sw_col = 16 * (grp & 1) + 8 * (grp >> 1);
#pragma unroll
  for (int fp = 0; fp < FN; fp += 2) {
    const int np = nb + fp * 16;         // the pair's first feature (a multiple of 32)
    if (np >= a.N) continue;             // (N is a multiple of 16: a pair is in or out whole...
    const bool second = np + 16 < a.N;   // ...but its second tile may be past N)
    float bias[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = np + 16 * h + 4 * grp + e;
        bias[h][e] = (a.bias && n < a.N) ? to_f(a.bias[n]) : 0.f;
      }
    // the region of the pair (the Q/K/V boundaries are multiples of 32)
    const bool is_v = kEpi == kQKV && np >= a.HD + a.Hk * a.D;
    const bool is_k = kEpi == kQKV && !is_v && np >= a.HD;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = mb + fm * 16 + m16;
      float va[4], vb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        va[e] = acc[fp][fm][e] + bias[0][e];
        vb[e] = acc[fp + 1][fm][e] + bias[1][e];
      }
      if (!is_v) {
        // every lane takes part in the swap (rows past M included); only the store is masked
        T tmp[8];
        swap_pair<T>(va, vb, tmp);
        const int n = np + sw_col;
        if (m >= a.M || (!second && n >= np + 16)) continue;
        T* dst;
        if constexpr (kEpi == kPlain) {
          dst = a.y + (size_t)m * a.N + n;
        } else if (!is_k) {
          dst = a.y + (size_t)m * a.HD + n;
        } else {
          const int b = m / a.C;
          const int t = m - b * a.C;
          const int n_real = a.lens ? clampi(a.lens[b], 0, a.C) : a.C;
          if (t >= n_real) continue;   // frames past the stream's real ones are not appended
          const int start = a.ws ? max(a.ws[b], 0) / a.S * a.S : 0;
          const int frame = start + clampi(a.cs[b], 0, a.max_cache) + t;
          const int blk = clampi(a.bt[(size_t)b * a.max_blocks + (frame / a.S) % a.max_blocks], 0,
                                 a.num_blocks - 1);
          const int slot = frame % a.S;
          const int kv = n - a.HD;
          const int g = kv / a.D, d = kv - g * a.D;
          // K pages in 32-dim column blocks: dim d of slot s at ((d / 32) S + s) 32 + d % 32
          dst = a.k_pool + ((size_t)blk * a.Hk + g) * a.S * a.D + ((d >> 5) * a.S + slot) * 32 + (d & 31);
        }
#pragma unroll
        for (int e = 0; e < 8; e += 16 / (int)sizeof(T))
          *reinterpret_cast<u32x4*>(dst + e) = *reinterpret_cast<const u32x4*>(tmp + e);
      } else {
        if (m >= a.M) continue;
        const int b = m / a.C;
        const int t = m - b * a.C;
        const int n_real = a.lens ? clampi(a.lens[b], 0, a.C) : a.C;
        if (t >= n_real) continue;
        const int start = a.ws ? max(a.ws[b], 0) / a.S * a.S : 0;
        const int frame = start + clampi(a.cs[b], 0, a.max_cache) + t;
        const int blk = clampi(a.bt[(size_t)b * a.max_blocks + (frame / a.S) % a.max_blocks], 0,
                               a.num_blocks - 1);
        const int slot = frame % a.S;
        const int hkd = a.Hk * a.D;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1 && !second) continue;
          const int kv = np + 16 * h + 4 * grp - a.HD - hkd;
          const int g = kv / a.D, d = kv - g * a.D;
          T* col = a.v_pool + (((size_t)blk * a.Hk + g) * a.D + d) * a.S + slot;
#pragma unroll
          for (int e = 0; e < 4; ++e) col[(size_t)e * a.S] = from_f<T>(h ? vb[e] : va[e]);
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int kEpi, bool kSin>
__global__ void __launch_bounds__(kThreads)
gemm_kernel(GemmArgs<T> a) {
  typedef typename Frag<T>::type F;
  constexpr int VEC = 16 / sizeof(T);          // elements per 16-byte vector
  constexpr int RV = kBK / VEC;                // vectors per staged row
  constexpr int LP = kLP<T>;
  constexpr int WM = BM / 2, WN = BN / 2;      // wave tile (2 x 2 waves)
  constexpr int FM = WM / 16, FN = WN / 16;    // 16 x 16 products per wave
  constexpr int NX = kSin ? 0 : BM * RV / kThreads;   // x vectors per thread per stage
  constexpr int NW = BN * RV / kThreads;              // W vectors per thread per stage
  static_assert((kSin || NX * kThreads == BM * RV) && NW * kThreads == BN * RV, "staging covers the tiles");

  __shared__ __align__(16) T s_x[kSin ? 1 : 2 * BM * LP];
  __shared__ __align__(16) T s_w[2 * BN * LP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m16 = lane & 15;
  const int grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, (a.M + BM - 1) / BM, a.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = a.K / kBK;

  struct Regs { u32x4 x[NX > 0 ? NX : 1], w[NW]; };
  // rows past M or N read the last row (their results are never stored)
  auto fetch = [&](Regs& r, int s) {
    const int k0 = kBK * s;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int idx = tid + kThreads * i;
      const int row = min(m0 + idx / RV, a.M - 1);
      r.x[i] = *reinterpret_cast<const u32x4*>(a.x + (size_t)row * a.K + k0 + (idx % RV) * VEC);
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int idx = tid + kThreads * i;
      const int row = min(n0 + idx / RV, a.N - 1);
      r.w[i] = *reinterpret_cast<const u32x4*>(a.w + (size_t)row * a.K + k0 + (idx % RV) * VEC);
    }
  };
  auto stash = [&](const Regs& r, int buf) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int idx = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(s_x + buf * BM * LP + (idx / RV) * LP + (idx % RV) * VEC) = r.x[i];
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int idx = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(s_w + buf * BN * LP + (idx / RV) * LP + (idx % RV) * VEC) = r.w[i];
    }
  };

  // positional source: this lane's positions (one per row fragment)
  float pos[FM];
  if constexpr (kSin) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = min(m0 + wm * WM + fm * 16 + m16, a.M - 1);
      const int t = m / a.rows;
      const int r = m - t * a.rows;
      pos[fm] = (float)((a.pos_start ? a.pos_start[t] : a.pos_first) + a.pos_step * r);
    }
  }

  floatx4 acc[FN][FM];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int s, int buf) {
    F xf[FM], wf[FN];
    if constexpr (kSin) {
      // columns k0 + 8 grp + [0, 8): four (sin, cos) pairs, frequencies 10000^(-2 i / K)
      const int i0 = (kBK * s + 8 * grp) >> 1;
      float freq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) freq[e] = exp2f((float)(2 * (i0 + e)) * a.neg_log2_base_per_col);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float sn, cs;
          sincosf(pos[fm] * freq[e], &sn, &cs);
          set(xf[fm], 2 * e, sn);
          set(xf[fm], 2 * e + 1, cs);
        }
    } else {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        xf[fm] = load8(s_x + buf * BM * LP + (wm * WM + fm * 16 + m16) * LP + 8 * grp);
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      wf[fn] = load8(s_w + buf * BN * LP + (wn * WN + fn * 16 + m16) * LP + 8 * grp);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mma(wf[fn], xf[fm], acc[fn][fm]);
  };

  Regs ra, rb;
  fetch(ra, 0);
  fetch(rb, min(1, nk - 1));
  stash(ra, 0);
  __syncthreads();
  // stage s: registers `nxt` hold stage s + 1, `fre` receives stage s + 2
  auto step = [&](int s, Regs& nxt, Regs& fre) {
    fetch(fre, min(s + 2, nk - 1));
    compute(s, s & 1);
    if (s + 1 < nk) stash(nxt, (s + 1) & 1);
    __syncthreads();
  };
  for (int s = 0; s < nk; s += 2) {
    step(s, rb, ra);
    if (s + 1 < nk) step(s + 1, ra, rb);
  }

  store_tiles<T, kEpi, FM, FN>(a, acc, m0 + wm * WM, n0 + wn * WN, m16, grp);
}

// ---- bf16, direct global -> LDS staging, NK stages unrolled ------------------------------------

constexpr int kDK = 64;   // contraction depth of one directly loaded stage: a row's whole 128-byte
                          // line per request

__device__ __forceinline__ int dma_swz(int r) { return ((r >> 1) ^ (r << 2)) & 7; }

// Wait until at most N of this wave's direct loads are in flight and its LDS accesses are done
// (s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4 left at 7, lgkmcnt 11:8 at 0).
template <int N>
__device__ __forceinline__ void wait_stage() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
}

template <int BM, int BN, int kEpi, int NK>
__global__ void __launch_bounds__(kThreads)
gemm_dma_kernel(GemmArgs<bf16> a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int NBX = BM / 8, NB = (BM + BN) / 8;   // 1 KB blocks (8 rows x 64 dims) per stage
  constexpr int DPW = NB / 4;                        // direct loads per wave per stage
  constexpr int SLOT = NB * 512;                     // bf16 elements of one ring slot
  static_assert(DPW * 4 == NB, "blocks split evenly over the waves");

  // a ring of 3 stages (2 in flight), each slot its own array
  __shared__ __align__(16) bf16 s0[SLOT];
  __shared__ __align__(16) bf16 s1[SLOT];
  __shared__ __align__(16) bf16 s2[SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m16 = lane & 15;
  const int grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, (a.M + BM - 1) / BM, a.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // this wave's blocks: lane l loads row l / 8 of the block, the 16-byte chunk that belongs at
  // chunk position l % 8 (rows past M or N read the last row; their results are never stored)
  const bf16* src[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int blk = wave * DPW + i;
    const int r = 8 * blk + (lane >> 3);               // row of the stage (x rows, then W rows)
    const int c = (lane & 7) ^ dma_swz(r & 15);
    if (blk < NBX) {
      src[i] = a.x + (size_t)min(m0 + r, a.M - 1) * a.K + 8 * c;
    } else {
      src[i] = a.w + (size_t)min(n0 + r - BM, a.N - 1) * a.K + 8 * c;
    }
  }
  auto slot = [&](int k) -> bf16* {
    switch (k % 3) {
      case 0: return s0;
      case 1: return s1;
      default: return s2;
    }
  };
  auto issue = [&](int s) {
    bf16* base = slot(s);
#pragma unroll
    for (int i = 0; i < DPW; ++i) load_lds16(src[i] + kDK * s, base + (wave * DPW + i) * 512);
  };
  // fragment reads: row m16 of a 16-row group (block m16 / 8, row m16 % 8 of it), the 16-byte
  // chunk 4 kk + grp of contraction half kk at its swizzled position
  int fo[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    fo[kk] = (m16 >> 3) * 512 + (m16 & 7) * 64 + 8 * ((4 * kk + grp) ^ dma_swz(m16));

  floatx4 acc[FN][FM];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = floatx4{0.f, 0.f, 0.f, 0.f};

  issue(0);
  if (NK > 1) issue(1);
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    // stage s in LDS for every wave (this wave's loads: all but the next stage's), and every
    // wave done reading the slot stage s + 2 refills
    if (s + 1 < NK) wait_stage<DPW>();
    else wait_stage<0>();
    // (the empty asm statements keep the compiler from moving LDS accesses across the barrier,
    // which it would otherwise treat as touching no memory)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s + 2 < NK) issue(s + 2);
    const bf16* cur = slot(s);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 xf[FM], wf[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) xf[fm] = load8(cur + ((wm * WM) / 16 + fm) * 1024 + fo[kk]);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) wf[fn] = load8(cur + (BM / 16 + (wn * WN) / 16 + fn) * 1024 + fo[kk]);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mma(wf[fn], xf[fm], acc[fn][fm]);
    }
  }
  store_tiles<bf16, kEpi, FM, FN>(a, acc, m0 + wm * WM, n0 + wn * WN, m16, grp);
}

// Tile shape: the least work on the busiest CU with every tile resident at once (ties: the larger
// tile, which re-reads less), over 128 x 128, 128 x 64 and 64 x 64.
inline int pick_tile(int M, int N) {
  const int cand[3][2] = {{128, 128}, {128, 64}, {64, 64}};
  int best = 0;
  long best_cost = -1;
  for (int i = 0; i < 3; ++i) {
    const long tiles = (long)((M + cand[i][0] - 1) / cand[i][0]) * ((N + cand[i][1] - 1) / cand[i][1]);
    const long cost = ((tiles + 255) / 256) * cand[i][0] * cand[i][1];
    if (best_cost < 0 || cost < best_cost) {
      best = i;
      best_cost = cost;
    }
  }
  return best;
}

template <int BM, int BN, int kEpi>
hipError_t launch_dma(GemmArgs<bf16>& a, dim3 grid, hipStream_t stream) {
  switch (a.K / kDK) {
    case 4: hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, kEpi, 4>), grid, dim3(kThreads), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, kEpi, 8>), grid, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, kEpi, 16>), grid, dim3(kThreads), 0, stream, a); break;
  }
  return hipGetLastError();
}

template <typename T, int BM, int BN, int kEpi, bool kSin>
hipError_t launch_shape(GemmArgs<T> a, hipStream_t stream) {
  a.tiles_n = (a.N + BN - 1) / BN;
  const dim3 grid((unsigned)(((a.M + BM - 1) / BM) * a.tiles_n));
  if constexpr (sizeof(T) == 2 && !kSin) {
    if (a.K == 256 || a.K == 512 || a.K == 1024) return launch_dma<BM, BN, kEpi>(a, grid, stream);
  }
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, kEpi, kSin>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int kEpi, bool kSin>
hipError_t launch_tiles(GemmArgs<T> a, hipStream_t stream) {
  switch (pick_tile(a.M, a.N)) {
    case 0: return launch_shape<T, 128, 128, kEpi, kSin>(a, stream);
    case 1: return launch_shape<T, 128, 64, kEpi, kSin>(a, stream);
    default: return launch_shape<T, 64, 64, kEpi, kSin>(a, stream);
  }
}

template <typename T>
GemmArgs<T> base_args(const GemmParams& p) {
  GemmArgs<T> a{};
  a.x = (const T*)p.x;
  a.w = (const T*)p.w;
  a.bias = (const T*)p.bias;
  a.y = (T*)p.y;
  a.M = p.M;
  a.N = p.N;
  a.K = p.K;
  return a;
}

template <typename T>
hipError_t launch_linear_t(const GemmParams& p, hipStream_t stream) {
  return launch_tiles<T, kPlain, false>(base_args<T>(p), stream);
}

template <typename T>
hipError_t launch_qkv_t(const QkvParams& q, hipStream_t stream) {
  GemmParams g{q.x, q.w, q.bias, q.q_out, q.batch * q.chunk,
               (q.n_head + 2 * q.n_kv_head) * q.head_dim, q.d_model};
  GemmArgs<T> a = base_args<T>(g);
  a.k_pool = (T*)q.k_pool;
  a.v_pool = (T*)q.v_pool;
  a.bt = q.block_tables;
  a.cs = q.cache_seqlens;
  a.lens = q.chunk_lens;
  a.ws = q.window_start;
  a.C = q.chunk;
  a.HD = q.n_head * q.head_dim;
  a.Hk = q.n_kv_head;
  a.D = q.head_dim;
  a.S = q.block_size;
  a.num_blocks = q.num_blocks;
  a.max_blocks = q.max_blocks;
  a.max_cache = q.max_cache;
  return launch_tiles<T, kQKV, false>(a, stream);
}

template <typename T>
hipError_t launch_pos_t(const PosProjParams& q, hipStream_t stream) {
  GemmParams g{nullptr, q.w, nullptr, q.out, q.n_tables * q.rows, q.out_features, q.d_model};
  GemmArgs<T> a = base_args<T>(g);
  a.pos_start = q.pos_start;
  a.pos_first = q.pos_first;
  a.pos_step = q.pos_step;
  a.rows = q.rows;
  a.neg_log2_base_per_col = -13.287712379549449f / (float)q.d_model;   // log2(10000) = 13.2877...
  return launch_tiles<T, kPlain, true>(a, stream);
}

}  // namespace

hipError_t launch_linear(pkc_dtype dtype, const GemmParams& p, hipStream_t stream) {
  return dtype == PKC_BF16 ? launch_linear_t<bf16>(p, stream) : launch_linear_t<float>(p, stream);
}

hipError_t launch_qkv_append(pkc_dtype dtype, const QkvParams& p, hipStream_t stream) {
  return dtype == PKC_BF16 ? launch_qkv_t<bf16>(p, stream) : launch_qkv_t<float>(p, stream);
}

hipError_t launch_pos_projection(pkc_dtype dtype, const PosProjParams& p, hipStream_t stream) {
  return dtype == PKC_BF16 ? launch_pos_t<bf16>(p, stream) : launch_pos_t<float>(p, stream);
}

}  // namespace pkc
