// Memory-path ceiling of the fused append + chunk attention (gfx950): a kernel that moves exactly
// the bytes one fused launch moves, through the same block tables and page layouts, with no
// arithmetic. Its launch time is what the access pattern itself costs at a given launch shape; the
// attention kernel is measured against it.
//
// Source of the access pattern: OASR docs, "ASR Engine", section 4.3 "Batched paged forward" (the
// chunk's K/V written into the stream's pages through its block-table row, the cached frames read
// back through it) and "Model Layer", "Three optional encoder declarations",
// fixed_attention_window (the positional rows a chunk touches: distances cache + i - j, one
// shared table for a uniform cache, one table per row otherwise).
//
// Per (stream b, head h) unit, split over `split` workgroups of kWaves (1, 4 or 8) waves:
//   reads   the 16 queries, u and v, the chunk's K/V (k_new, v_new), the cached K/V pages
//           [0, cache) in 32-key steps, and the positional band rows of each step, all with the
//           attention kernel's own per-lane addresses;
//   writes  the chunk's K/V into the pool exactly as paged_kv_append does (same slots, same
//           bits), and one 16-byte word per output element group of out[b][i][h][:] (the XOR of
//           what the unit read: garbage, never an attention result).
// Every load of a wave's step group is issued before the first wait: the block IDs, then the
// pages. Split variants (split > 1) omit the cross-workgroup merge a split attention would need,
// so they bound such a design from below. With reads = 0 the same grid only writes its output
// rows: the floor that launching, dispatching and retiring this grid costs.
#include "pkc_device.h"
#include "pkc_launch.h"

namespace pkc {

namespace {

struct GatherArgs {
  const bf16* q;
  const bf16* u;
  const bf16* w;
  const bf16* k_new;
  const bf16* v_new;
  bf16* k_pool;
  bf16* v_pool;
  const int32_t* bt;
  const int32_t* cs;
  const bf16* pos;
  bf16* out;
  int C, H, Hk, S, logS, N, M, max_cache, pos_len, per_row, split, reads;
  int band_rs, band_hs, band_hd;   // positional table strides: row, 32-dim half, head
  FastDiv div_split, div_H, div_group;
};

constexpr int kD = 64;          // head_dim
constexpr int kStepLoads = 12;   // 16-byte loads of one lane per 32-key step: K 4, V 4, band 4

template <int kWaves>
__global__ void __launch_bounds__(kWaves * 64)
gather_read_kernel(GatherArgs a) {
  constexpr int kThreads = kWaves * 64;
  __shared__ u32x4 s_x[kWaves][64];
  __shared__ __align__(16) bf16 s_vt[kD][16 + 8];   // the chunk's V, transposed

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m16 = lane & 15;
  const int grp = lane >> 4;

  const int id = blockIdx.x;
  const int unit = fdiv(id, a.div_split);
  const int part = id - unit * a.split;
  const int b = fdiv(unit, a.div_H);
  const int h = unit - b * a.H;
  const int hk = fdiv(h, a.div_group);
  if (!a.reads) {
    // the launch floor: the same grid writing its output rows, reading nothing
    for (int f = tid >> 3; part == 0 && f < a.C; f += kThreads / 8)
      *reinterpret_cast<u32x4*>(a.out + (((size_t)b * a.C + f) * a.H + h) * kD + (tid & 7) * 8) =
          u32x4{(uint32_t)id, 0u, 0u, 0u};
    return;
  }
  const int cs_raw = a.cs[b];
  __builtin_amdgcn_sched_barrier(0);
  const int32_t* bt = a.bt + (size_t)b * a.M;

  // requests that need no cache length: queries, u, v and the chunk's frames
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 qv[6];
  {
    const int iq = min(m16, a.C - 1);
    const bf16* qrow = a.q + (((size_t)b * a.C + iq) * a.H + h) * kD + 8 * grp;
    qv[0] = *reinterpret_cast<const u32x4*>(qrow);
    qv[1] = *reinterpret_cast<const u32x4*>(qrow + 32);
    qv[2] = *reinterpret_cast<const u32x4*>(a.u + h * kD + 8 * grp);
    qv[3] = *reinterpret_cast<const u32x4*>(a.u + h * kD + 32 + 8 * grp);
    qv[4] = *reinterpret_cast<const u32x4*>(a.w + h * kD + 8 * grp);
    qv[5] = *reinterpret_cast<const u32x4*>(a.w + h * kD + 32 + 8 * grp);
  }
  const bool chunk_owner = part == 0;
  // chunk frames of this thread (8 vectors per row): ft, ft + kThreads / 8, ... (at most 16)
  constexpr int NF = (16 * 8 + kThreads - 1) / kThreads;
  u32x4 nk[NF], nv[NF];
  const int ft = tid >> 3;
  const int fdv = (tid & 7) * 8;
#pragma unroll
  for (int it = 0; it < NF; ++it) {
    nk[it] = nv[it] = u32x4{0u, 0u, 0u, 0u};
    const int f = ft + it * (kThreads / 8);
    if (chunk_owner && f < a.C) {
      const size_t row = ((size_t)(b * a.C + f) * a.Hk + hk) * kD + fdv;
      nk[it] = *reinterpret_cast<const u32x4*>(a.k_new + row);
      nv[it] = *reinterpret_cast<const u32x4*>(a.v_new + row);
    }
  }

  const int cache = clampi(cs_raw, 0, a.max_cache);
  const int T_len = cache + a.C;
  const int nbody = (cache + 31) >> 5;
  const int G = a.split * kWaves;
  const int gw = part * kWaves + wave;
  const int s_begin = (gw * nbody) / G;
  const int s_end = ((gw + 1) * nbody) / G;
  const uint32_t blk_stride = (uint32_t)(a.Hk * a.S * kD);
  const bf16* kp = a.k_pool + (size_t)hk * a.S * kD;
  const bf16* vp = a.v_pool + (size_t)hk * a.S * kD;
  const int center = a.per_row ? (cache + a.C - 1) : (a.pos_len - 1) / 2;
  const int R0 = center - cache;
  const int rlo = R0 - (a.C - 1);
  const int rhi = R0 + T_len - 1;
  const size_t prow = (size_t)a.band_rs;
  const bf16* ptab = a.pos + (a.per_row ? (size_t)b * a.pos_len * a.H * kD : 0) + (size_t)h * a.band_hd;
  auto band = [&](int r) {
    return *reinterpret_cast<const u32x4*>(ptab + (size_t)(uint32_t)clampi(r, rlo, rhi) * prow + 8 * grp);
  };
  auto page_id = [&](int pg) { return clampi(pg, 0, a.M - 1); };

  // the positional rows of the wave's first step (tile 0) and of the chunk's own step
  if (s_begin < s_end) {
    const int r = R0 + 32 * s_begin - 15 + m16;
    acc ^= band(r);
  }
  if (chunk_owner && wave == 0) {
#pragma unroll
    for (int t = 0; t < 3; ++t) acc ^= band(R0 + cache - 15 + 16 * t + m16);
  }

  // body steps in groups of two: both steps' block IDs, then every load of both steps
  for (int s = s_begin; s < s_end; s += 2) {
    const int ns = min(2, s_end - s);
    int kb[2], vb[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j0 = 32 * (s + min(k, ns - 1));
      kb[k] = bt[page_id((j0 + 8 * (m16 >> 2)) >> a.logS)];
      vb[k] = bt[page_id((j0 + 8 * grp) >> a.logS)];
    }
    u32x4 r[2][kStepLoads];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j0 = 32 * (s + min(k, ns - 1));
      const int key = j0 + 8 * (m16 >> 2) + (m16 & 3);
      const bf16* krow = kp + (uint64_t)clampi(kb[k], 0, a.N - 1) * blk_stride +
                         (uint32_t)((key & (a.S - 1)) * 32 + 8 * grp);
      r[k][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow));
      r[k][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow + a.S * 32));
      r[k][2] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow + 4 * 32));
      r[k][3] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow + a.S * 32 + 4 * 32));
      const int kg = j0 + 8 * grp;
      const bf16* vrow = vp + (uint64_t)clampi(vb[k], 0, a.N - 1) * blk_stride +
                         (uint32_t)(m16 * a.S + (kg & (a.S - 1)));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        r[k][4 + dt] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vrow + 16 * dt * a.S));
      const int rb = R0 + j0 - 15;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16* row = ptab + (size_t)(uint32_t)clampi(rb + 16 * (t + 1) + m16, rlo, rhi) * prow + 8 * grp;
        r[k][8 + 2 * t] = *reinterpret_cast<const u32x4*>(row);
        r[k][9 + 2 * t] = *reinterpret_cast<const u32x4*>(row + a.band_hs);
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int x = 0; x < kStepLoads; ++x) acc ^= r[k][x];
  }
#pragma unroll
  for (int x = 0; x < 6; ++x) acc ^= qv[x];

  // the append: the chunk's K rows into their column-blocked slots, V transposed through LDS
  const bool append = chunk_owner && h == hk * (a.H / a.Hk);
#pragma unroll
  for (int it = 0; it < NF; ++it) {
    const int f = ft + it * (kThreads / 8);
    if (append && f < a.C) {
      const int key = cache + f;
      bf16* dst = a.k_pool + (size_t)hk * a.S * kD +
                  (uint64_t)clampi(bt[page_id(key >> a.logS)], 0, a.N - 1) * blk_stride +
                  (uint32_t)(((fdv >> 5) * a.S + (key & (a.S - 1))) * 32 + (fdv & 31));
      *reinterpret_cast<u32x4*>(dst) = nk[it];
      const uint32_t wd[4] = {nv[it][0], nv[it][1], nv[it][2], nv[it][3]};
#pragma unroll
      for (int c = 0; c < 8; ++c)
        reinterpret_cast<uint16_t*>(&s_vt[fdv + c][0])[f] = (uint16_t)(wd[c >> 1] >> (16 * (c & 1)));
    }
  }
  s_x[wave][lane] = acc;
  __syncthreads();
  if (append) {
    for (int x = tid; x < kD * a.C; x += kThreads) {
      const int d = x % kD;
      const int t = x / kD;
      const int key = cache + t;
      bf16* dst = a.v_pool + (size_t)hk * a.S * kD +
                  (uint64_t)clampi(bt[page_id(key >> a.logS)], 0, a.N - 1) * blk_stride +
                  (uint32_t)(d * a.S + (key & (a.S - 1)));
      if ((key & 7) == 0 && (t & 7) == 0 && t + 8 <= a.C) {
        *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(&s_vt[d][t]);
      } else if ((key & 7) == 0 || t == 0) {
        // a run not aligned to 8 frames: element stores up to the next 8-frame boundary
        for (int c = t; c < a.C && (c == t || ((cache + c) & 7) != 0); ++c) {
          const int kc = cache + c;
          bf16* dc = a.v_pool + (size_t)hk * a.S * kD +
                     (uint64_t)clampi(bt[page_id(kc >> a.logS)], 0, a.N - 1) * blk_stride +
                     (uint32_t)(d * a.S + (kc & (a.S - 1)));
          *dc = s_vt[d][c];
        }
      }
    }
  }
  u32x4 o = s_x[0][tid & 63];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) o ^= s_x[w][tid & 63];
#pragma unroll
  for (int it = 0; it < NF; ++it) {
    const int f = ft + it * (kThreads / 8);
    if (chunk_owner && f < a.C)
      *reinterpret_cast<u32x4*>(a.out + (((size_t)b * a.C + f) * a.H + h) * kD + fdv) = o;
  }
}

}  // namespace

LaunchGrid gather_read_grid(int batch, int n_head, int split, int waves) {
  return {mul_sat(mul_sat(batch, n_head), split), waves * 64};
}

hipError_t launch_gather_read(const GatherParams& p, hipStream_t stream) {
  GatherArgs a;
  a.q = (const bf16*)p.q;
  a.u = (const bf16*)p.pos_bias_u;
  a.w = (const bf16*)p.pos_bias_v;
  a.k_new = (const bf16*)p.k_new;
  a.v_new = (const bf16*)p.v_new;
  a.k_pool = (bf16*)p.k_pool;
  a.v_pool = (bf16*)p.v_pool;
  a.bt = p.block_tables;
  a.cs = p.cache_seqlens;
  a.pos = (const bf16*)p.pos;
  a.out = (bf16*)p.out;
  a.C = p.chunk;
  a.H = p.n_head;
  a.Hk = p.n_kv_head;
  a.S = p.block_size;
  a.logS = 0;
  while ((1 << a.logS) < p.block_size) ++a.logS;
  a.N = p.num_blocks;
  a.M = p.max_blocks;
  a.max_cache = p.max_cache;
  a.pos_len = p.pos_len;
  a.per_row = (p.pos_layout & PKC_POS_PER_ROW) != 0;
  const bool blocked = (p.pos_layout & PKC_POS_COL_BLOCKED) != 0;
  a.band_rs = blocked ? 32 : p.n_head * kD;
  a.band_hs = blocked ? 32 * p.pos_len : 32;
  a.band_hd = blocked ? kD * p.pos_len : kD;
  a.split = p.split;
  a.reads = p.reads;
  a.div_split = make_fastdiv(p.split);
  a.div_H = make_fastdiv(p.n_head);
  a.div_group = make_fastdiv(p.n_head / p.n_kv_head);
  const dim3 grid((unsigned)gather_read_grid(p.batch, p.n_head, p.split, p.waves).workgroups);
  if (p.waves == 8) hipLaunchKernelGGL(gather_read_kernel<8>, grid, dim3(512), 0, stream, a);
  else if (p.waves == 1) hipLaunchKernelGGL(gather_read_kernel<1>, grid, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL(gather_read_kernel<4>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkc
