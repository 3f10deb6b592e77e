// Chunk attention over a paged K/V pool with a Transformer-XL relative-position term (gfx950).
//
// Sources: OASR docs, "Scheduler", section 4.3 "Heterogeneous-offset batching" (attention over the
// paged pool, per-stream lengths from cache_seqlens, matrix_bd / sqrt(d_k) added to the scores);
// "Model Layer", fixed_attention_window declaration (distances cache + i - j; one shared table for
// a uniform cache, one table per row otherwise); "ASR Engine", section 4.3 (the append of the
// chunk's K/V that precedes the attention, fused into this kernel when k_new is given).
//
// Work decomposition. One workgroup of kWaves wavefronts per (stream b, head h, 16-query tile).
// The T = cache + C keys split into
//   * the body, the cached keys [0, cache): 32-key steps read straight from the pool pages; the
//     last one is masked when cache is not a multiple of 32 (its V past cache zeroed);
//   * the tail, the chunk's own frames [cache, T): staged into LDS - K rows and V transposed,
//     taken from k_new / v_new when fused and from the pool otherwise, zero past T - and
//     processed as masked steps.
// The split and the step-to-wave assignment depend only on the cache length, so the fused and the
// unfused entries do identical arithmetic on identical values.
// Each wave takes a contiguous range of body steps (so one band tile carries over from step to
// step) and every kWaves-th tail step, keeps its own online-softmax state, and the waves merge
// through LDS in a fixed order: a stream's result depends only on its own cache length.
//
// Latency. Everything a wave needs is requested before it first waits: the block IDs of the
// stream's first 128 pages (into a wave-private LDS window, no workgroup barrier), the queries,
// the chunk's frames (short fused chunks), the band rows and the first two body steps; later
// steps are fetched two steps ahead into alternating register sets, and the band rows of the
// wave's tail step into the set the body frees last. The chunk's K/V are written into the pool
// only at the very end: on CDNA global stores share the in-order vector-memory counter with
// loads, so a store issued early would hold up every later load wait. The softmax scale (and
// log2 e) is folded into q + u and q + v, and the running max moves only when a score exceeds it
// by 2^8 (the probabilities stay <= 256, exact after the final division), which keeps the
// rescale of the accumulator out of most steps.
//
// Per 32-key step, with 16x16 MFMA tiles whose columns are the 16 queries:
//   S^T = K . (q + u)^T          two tiles (32 keys), contraction over head_dim
//   G^T = P_band . (q + v)^T     three tiles: the 47 table rows the step touches (tile 0 is the
//                                previous step's tile 2 inside a body range)
//   O^T += V^T . softmax(S + Bd)^T
// Key order inside a step is permuted so that the 8 scores a lane holds after the S^T tiles are the
// 8 consecutive keys it feeds to the PV product (tile 0 row 4a + e is key 8a + e, tile 1 row
// 4a + e is key 8a + 4 + e). V pages are stored transposed ([head_dim][block_size]), so the V^T
// operand is one 16-byte load of 8 consecutive frames per lane. The relative shift
// Bd[i][j] = G[i][j + 15 - i'] (i' = query inside the tile) moves data between lanes of one query
// column; it goes through a per-wave LDS tile.
//
// Table geometry: the row for (query i, key j) is R0 + j - i with R0 = centre - cache; only rows
// [R0 - (C - 1), R0 + T - 1] are read.
#include <math.h>
#include <stdlib.h>

#include "pkc_device.h"
#include "pkc_launch.h"
#include "pkc_step.h"

namespace pkc {

namespace {

// O^T merge tile: 16 query columns per dimension row, padded to 20 floats so that the two lane
// groups of a half-wave (4 dimension rows apart on write, 4 apart on read) sit 16 banks apart
constexpr int kOPitch = 20;
constexpr int kWaveLds = kD * kOPitch + 32;  // floats per wave: O^T tile + m + l (skew tile aliases it)
constexpr int kBtWindow = 128;          // block IDs each wave keeps in its LDS window

template <typename T>
struct ChunkArgs {
  const T* q;
  const T* k_pool;
  const T* v_pool;
  const int32_t* bt;
  const int32_t* cs;
  const int32_t* lens;   // real frames per stream, or null
  const int32_t* ws;     // window start per stream (bounded history), or null
  const T* pos;
  const T* u;
  const T* w;
  T* out;
  const T* k_new;   // fused only
  const T* v_new;
  T* k_pool_w;
  T* v_pool_w;
  int C, H, Hk, S, logS, N, M, max_cache, pos_len, per_row, per_key, qtiles;
  FastDiv div_qtiles, div_H, div_group;   // by qtiles, H and H / Hk
  int tail_cap, vt_pitch;            // LDS tail geometry (keys, elements per V^T row)
  // positional table geometry (elements): between consecutive rows, between the two 32-dim
  // halves of a row, and between heads. Row-major [.., P, H, D]: H D, 32, D. In 32-dim column
  // blocks [.., H, D / 32, P, 32]: 32, 32 P, D P - a 16-row fragment half is then one contiguous
  // kilobyte, whole 128-byte lines, where row-major rows give each load half-lines.
  int band_rs, band_hs, band_hd;
  int off_bt, off_kt, off_vt;        // byte offsets of the LDS regions
  int phys;                          // physical waves per workgroup (host-side choice)
  int B;                             // streams
  int rank;                          // run the streams longest cache first (host-side choice)
  FastDiv div_hq;                    // by H qtiles
  float scale_log2;
};

// The stream at place r (0-based) when the B streams are ordered longest cache first - by their
// body step count in 64 buckets, longest bucket first, index order inside a bucket. Each wave
// works it out on its own: every stream's bucket counted in a wave-private LDS histogram (hist,
// 64 ints), the counts' prefix over the buckets, the bucket holding place r, then that bucket's
// streams walked in index order. The order only decides which workgroup runs which stream; the
// arithmetic, and with it every result bit, is the same in any order.
__device__ __forceinline__ int stream_by_length(const int32_t* cs, int B, int max_cache, int r,
                                                int* hist) {
  const int lane = threadIdx.x & 63;
  const int kmax = (max_cache + 31) >> 5;
  auto bucket = [&](int c) {   // 0: the longest caches
    const int key = (clampi(c, 0, max_cache) + 31) >> 5;
    return 63 - (int)(((int64_t)key * 64) / (kmax + 1));
  };
  hist[lane] = 0;
  __builtin_amdgcn_wave_barrier();
  for (int s0 = 0; s0 < B; s0 += 64)
    if (s0 + lane < B) atomicAdd(&hist[bucket(cs[s0 + lane])], 1);
  __builtin_amdgcn_wave_barrier();
  const int cnt = hist[lane];
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  const int start = incl - cnt;
  const uint64_t hit = __ballot(start <= r && r < incl);
  const int J = hit ? (int)__builtin_ctzll(hit) : 0;
  int t = r - __shfl(start, J);
  for (int s0 = 0; s0 < B; s0 += 64) {
    const bool in = s0 + lane < B && bucket(cs[min(s0 + lane, B - 1)]) == J;
    const uint64_t m = __ballot(in);
    const int n = __popcll(m);
    if (t < n) {
      // the lane holding the t-th stream of the bucket in this group of 64
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      const uint64_t pick = __ballot(in && below == t);
      return __builtin_amdgcn_readfirstlane(s0 + (int)__builtin_ctzll(pick));
    }
    t -= n;
  }
  return min(r, B - 1);   // (not reached: place r < B lies in some bucket)
}

template <typename T>
struct StepRegs {
  typedef typename Frag<T>::type F;
  F k[2][2];   // [key tile][head_dim half]
  F v[4];      // [16-dim tile]
  F p[2][2];   // band tiles 1 and 2 [tile][head_dim half]
};

template <typename T> constexpr int kt_pitch() { return kD + 16 / (int)sizeof(T); }

// The keys of a (stream, head, query tile) unit are split over kWaves = 4 virtual waves, each
// with its own online softmax, merged in a fixed order: a stream's result bits depend on its own
// length only. kPhys physical waves run them, kWaves / kPhys each, one after another over a
// contiguous range of body steps (the loads run ahead across the virtual waves' boundaries):
// fewer physical waves per unit put more units on a CU at once, with identical results.
// kGen: per-stream chunk lengths or window starts may be given. Without them (the common case)
// both are compile-time constants, which keeps the prologue's instruction count down.
template <typename T, bool kFused, int kPhys, int kS, bool kRegTail, bool kPerKey, bool kGen,
          bool kRank = false>
__global__ void __launch_bounds__(kPhys * 64)
__attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1)))
chunk_attn_kernel(ChunkArgs<T> a) {
  typedef typename Frag<T>::type F;
  constexpr int kWaves = 4;                 // virtual waves of the arithmetic
  constexpr int kR = kWaves / kPhys;        // virtual waves per physical wave
  static_assert(kR * kPhys == kWaves, "physical waves divide the virtual ones");
  // (several virtual waves per physical wave only for chunks held in registers, at most 32
  // frames: the tail is then one step, the first virtual wave's)
  static_assert(kR == 1 || kRegTail, "virtual waves after the first have no tail step");
  constexpr int kThreads = kPhys * 64;
  constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte vector
  constexpr int NV = kD / VEC;          // vectors per row
  constexpr int KTP = kt_pitch<T>();
  const int S = kS ? kS : a.S;
  const int logS = kS == 16 ? 4 : (kS == 32 ? 5 : a.logS);

  extern __shared__ __align__(16) unsigned char smem[];
  float* s_wave = reinterpret_cast<float*>(smem);
  int* s_win = reinterpret_cast<int*>(smem + a.off_bt) + (threadIdx.x >> 6) * kBtWindow;
  T* s_kt = reinterpret_cast<T*>(smem + a.off_kt);
  T* s_vt = reinterpret_cast<T*>(smem + a.off_vt);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m16 = lane & 15;
  const int grp = lane >> 4;

  // Grid order (stream, h, query tile), tile fastest: consecutive workgroups go round-robin to the
  // XCDs, so for H a multiple of 8 each XCD serves one head and a shared table's band for that
  // head stays in that XCD's L2. The streams go in index order, or, when the grid runs in more
  // than one pass over the CUs (kRank), longest cache first: workgroups start roughly in grid
  // order, and a long stream reached last would set the launch's tail.
  const int id = blockIdx.x;
  int b, h, qt;
  if constexpr (kRank) {
    const int sr = fdiv(id, a.div_hq);             // the stream's place in that order
    const int rem = id - sr * (a.H * a.qtiles);
    h = fdiv(rem, a.div_qtiles);
    qt = rem - h * a.qtiles;
    b = stream_by_length(a.cs, a.B, a.max_cache, sr, s_win);
  } else {
    const int bh = fdiv(id, a.div_qtiles);
    qt = id - bh * a.qtiles;
    b = fdiv(bh, a.div_H);
    h = bh - b * a.H;
  }
  const int hk = fdiv(h, a.div_group);
  const int32_t* bt = a.bt + (size_t)b * a.M;
  // the cache length gates every page and table address below: its request goes first (the
  // scheduling barrier keeps the compiler from sinking it below the vector requests; scalar
  // loads return out of order, so it also goes after every kernel-argument load the code above
  // waits for)
  const int cs_raw = a.cs[b];
  __builtin_amdgcn_sched_barrier(0);

  // ---- 1. requests that need nothing: block IDs of pages [0, 128), queries, u, v, chunk -------
  // With bounded history the table row is a ring: the window's page pg sits at entry
  // (pb + pg) mod M, pb = window start / S (whole blocks), so the window follows the start.
  const int nwin = min(a.M, kBtWindow);
  const int pb = (kGen && a.ws) ? (max(a.ws[b], 0) >> logS) % a.M : 0;
  auto ring = [&](int pg) {
    if constexpr (!kGen) return pg;
    const int e = pg + pb;
    return e >= a.M ? e - a.M : e;
  };
  // (every load up to the body's first two steps is issued unconditionally, from a valid
  // address, so that each wait below counts exactly the loads issued after the one it needs)
  const int bt_lo_raw = bt[ring(min(lane, nwin - 1))];
  const int bt_hi_raw = bt[ring(min(lane + 64, nwin - 1))];
  const int bt_lo = lane < nwin ? bt_lo_raw : 0;
  const int bt_hi = lane + 64 < nwin ? bt_hi_raw : 0;
  F qq[2], uu[2], ww[2];
  {
    const int iq = min(qt * 16 + m16, a.C - 1);
    const T* qrow = a.q + (((size_t)b * a.C + iq) * a.H + h) * kD;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int d0 = 32 * half + 8 * grp;
      qq[half] = load8(qrow + d0);
      uu[half] = load8(a.u + h * kD + d0);
      ww[half] = load8(a.w + h * kD + d0);
    }
  }
  // the chunk's own frames (fused, short chunks: kR 16-byte vectors of K and of V per thread,
  // 32 frames in all)
  u32x4 nk[kR], nv[kR];
  if constexpr (kRegTail) {
#pragma unroll
    for (int it = 0; it < kR; ++it) {
      const int idx = tid + kThreads * it;
      const size_t row = ((size_t)(b * a.C + min(idx / NV, a.C - 1)) * a.Hk + hk) * kD + (idx % NV) * VEC;
      nk[it] = *reinterpret_cast<const u32x4*>(a.k_new + row);
      nv[it] = *reinterpret_cast<const u32x4*>(a.v_new + row);
    }
  }
  const int cache = clampi(cs_raw, 0, a.max_cache);
  // real frames of this stream's chunk: frames past them do not exist (not appended, not keys;
  // their output rows are zero); a stream with none is a padding lane and reads nothing
  const int n_real = (kGen && a.lens) ? clampi(a.lens[b], 0, a.C) : a.C;
  if (kGen && qt * 16 >= n_real) {
    for (int x = tid; x < 16 * NV; x += kThreads) {
      const int i = qt * 16 + x / NV;
      if (i < a.C)
        *reinterpret_cast<uint4*>(a.out + (((size_t)b * a.C + i) * a.H + h) * kD + (x % NV) * VEC) =
            uint4{0u, 0u, 0u, 0u};
    }
    return;   // uniform over the workgroup
  }
  const int T_len = cache + n_real;   // keys
  const int nbody = (cache + 31) >> 5;                 // body steps over the cached keys
  const int s_part = (cache & 31) ? nbody - 1 : -1;    // the partial one, if any
  const int ntail = (n_real + 31) >> 5;                // tail steps over the chunk's frames
  const size_t page = (size_t)S * kD;                  // elements of one (block, kv head) page
  const uint32_t blk_stride = (uint32_t)(a.Hk * S * kD);
  const T* kp = a.k_pool + (size_t)hk * page;
  const T* vp = a.v_pool + (size_t)hk * page;
  const int v0 = wave * kR;                                 // this wave's first virtual wave
  auto vbound = [&](int v) { return (v * nbody) / kWaves; };   // first body step of virtual wave v
  const int s_begin = vbound(v0);
  const int s_end = vbound(v0 + kR);
  const int nmine = s_end - s_begin;

  // a per-row table is built for the full chunk width: centred at cache + C - 1
  const int center = a.per_row ? (cache + a.C - 1) : (a.pos_len - 1) / 2;
  const int R0 = center - cache;
  const int rlo = R0 - (a.C - 1);
  const int rhi = R0 + T_len - 1;
  const int qlast = qt * 16 + 15;
  const T* ptab = a.pos + (a.per_row ? (size_t)b * a.pos_len * a.H * kD : 0) + (size_t)h * a.band_hd;
  const size_t prow = (size_t)a.band_rs;
  const int phalf = a.band_hs;
  auto band_row = [&](int r) { return ptab + (size_t)(uint32_t)clampi(r, rlo, rhi) * prow; };
  // per-key tables (WeNet's convention, no shift): row j is key j's own embedding; keys past the
  // last one read its row (they are masked)
  auto key_row = [&](int j) { return ptab + (size_t)(uint32_t)min(j, T_len - 1) * prow; };
  // P rows of a step's 32 keys in the key tiles' permuted order (tile tt row 4a + e is key
  // j0 + 8a + 4tt + e), into p[tt][half]
  auto load_key_rows = [&](F (&p)[2][2], int j0) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const T* row = key_row(j0 + 8 * (m16 >> 2) + 4 * tt + (m16 & 3)) + 8 * grp;
      p[tt][0] = load8(row);
      p[tt][1] = load8(row + phalf);
    }
  };

  // the window, and a page's block ID from it (pages past it: straight from the table). The
  // masked last body step can reach one page past the stream's pages: such pages read as block 0
  // in the window and as another entry of the row past it (their frames are masked).
  s_win[lane] = clampi(bt_lo, 0, a.N - 1);
  s_win[64 + lane] = clampi(bt_hi, 0, a.N - 1);
  auto block_of = [&](int pg) -> uint32_t {
    return (uint32_t)(pg < kBtWindow ? s_win[pg] : clampi(bt[ring(min(pg, a.M - 1))], 0, a.N - 1));
  };
  // ---- 2. loads of the first two body steps (band tile 0 of the first one too) ----------------
  auto load_step = [&](StepRegs<T>& r, int s) {
    const int j0 = 32 * s;
    // K pages are in 32-dim column blocks ([2][S][32] per page): half h of slot s's row is at
    // (h S + s) 32, so each load instruction covers whole 128-byte lines (4 consecutive slots'
    // halves, two lines, per key group)
    const int key = j0 + 8 * (m16 >> 2) + (m16 & 3);          // key of tile 0; tile 1 is key + 4
    const T* krow = kp + (uint64_t)block_of(key >> logS) * blk_stride +
                    (uint32_t)((key & (S - 1)) * 32 + 8 * grp);
    r.k[0][0] = load8_stream(krow);
    r.k[0][1] = load8_stream(krow + S * 32);
    r.k[1][0] = load8_stream(krow + 4 * 32);
    r.k[1][1] = load8_stream(krow + S * 32 + 4 * 32);
    const int kg = j0 + 8 * grp;
    const T* vb = vp + (uint64_t)block_of(kg >> logS) * blk_stride +
                  (uint32_t)(m16 * S + (kg & (S - 1)));
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) r.v[dt] = load8_stream(vb + 16 * dt * S);
    if constexpr (kPerKey) {
      load_key_rows(r.p, j0);
    } else {
      const int rb = R0 + j0 - qlast;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const T* row = band_row(rb + 16 * (t + 1) + m16) + 8 * grp;
        r.p[t][0] = load8(row);
        r.p[t][1] = load8(row + phalf);
      }
    }
  };
  // table rows of this wave's first tail step (band tiles 0, 1, 2, or the 32 keys' rows of a
  // per-key table in tb[0..1]): requested first, so that waiting for them waits for nothing
  // else; the tail step then runs while the body's data is still on its way. Only the waves
  // that have a tail step request them (the branch is uniform over each wave).
  F tb[3][2];
  if (v0 < ntail) {
    const int k0 = v0;
    if constexpr (kPerKey) {
      load_key_rows(*reinterpret_cast<F(*)[2][2]>(&tb[0]), cache + 32 * k0);
    } else {
      const int rb = R0 + cache + 32 * k0 - qlast;
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const T* row = band_row(rb + 16 * t + m16) + 8 * grp;
        tb[t][0] = load8(row);
        tb[t][1] = load8(row + phalf);
      }
    }
  }
  // the wave's first two body steps (a wave with fewer requests the last body step again, or
  // step 0 when there is none; those registers are never used)
  const int s_last = max(nbody - 1, 0);
  StepRegs<T> ra, rb2;
  F p0[2];
  {
    if (!kPerKey) {
      const T* row = band_row(R0 + 32 * min(s_begin, s_last) - qlast + m16) + 8 * grp;
      p0[0] = load8(row);
      p0[1] = load8(row + phalf);
    }
    load_step(ra, min(s_begin, s_last));
    load_step(rb2, min(s_begin + 1, s_last));
  }

  // the chunk's frames into the LDS tail (row t = frame t; V transposed, zero past the chunk),
  // after the body steps' loads are requested: waiting for the frames then leaves those loads in
  // flight, and the staging's LDS writes are not on their way
  if constexpr (kRegTail) {
#pragma unroll
    for (int it = 0; it < kR; ++it) {
      const int idx = tid + kThreads * it;
      if (idx < n_real * NV) {
        const int t = idx / NV;
        const int dv = (idx % NV) * VEC;
        *reinterpret_cast<u32x4*>(s_kt + t * KTP + dv) = nk[it];
        const uint32_t wd[4] = {nv[it][0], nv[it][1], nv[it][2], nv[it][3]};
#pragma unroll
        for (int c = 0; c < 8; ++c)
          reinterpret_cast<uint16_t*>(s_vt)[(dv + c) * a.vt_pitch + t] = (uint16_t)(wd[c >> 1] >> (16 * (c & 1)));
      }
    }
    for (int x = tid; x < (32 * ntail - n_real) * kD; x += kThreads)
      s_vt[(x % kD) * a.vt_pitch + n_real + x / kD] = from_f<T>(0.f);
  }


  // ---- 3. long chunks: the chunk's frames into the LDS tail with a loop ------------------------
  // (from k_new / v_new when fused, else from the pool, where an earlier append put them)
  if constexpr (!kRegTail) {
    for (int x = tid; x < 32 * ntail * NV; x += kThreads) {
      const int t = x / NV;
      const int dv = (x % NV) * VEC;
      if (t < n_real) {
        const int key = cache + t;
        const T* src = kFused ? a.k_new + ((size_t)(b * a.C + t) * a.Hk + hk) * kD + dv
                              : kp + (uint64_t)block_of(key >> logS) * blk_stride +
                                    (uint32_t)(((dv >> 5) * S + (key & (S - 1))) * 32 + (dv & 31));
        *reinterpret_cast<uint4*>(s_kt + t * KTP + dv) = *reinterpret_cast<const uint4*>(src);
      }
    }
    for (int x = tid; x < 32 * ntail * NV; x += kThreads) {
      const int t = x / NV;
      const int dv = (x % NV) * VEC;
      if (kFused && t < n_real) {
        const uint4 raw = *reinterpret_cast<const uint4*>(
            a.v_new + ((size_t)(b * a.C + t) * a.Hk + hk) * kD + dv);
        const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int k = 0; k < VEC; ++k) s_vt[(dv + k) * a.vt_pitch + t] = e[k];
      } else if (t >= n_real) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) s_vt[(dv + k) * a.vt_pitch + t] = from_f<T>(0.f);
      }
    }
    if (!kFused) {
      // frames from the transposed pages, element by element (thread column t = tid % 32 of
      // every 32-frame group, dimensions d = tid / 32 + 8 n)
      for (int c0 = 0; c0 < n_real; c0 += 32) {
        const int t = c0 + (tid & 31);
        if (t < n_real) {
          const int key = cache + t;
          const T* src = vp + (uint64_t)block_of(key >> logS) * blk_stride + (uint32_t)(key & (S - 1));
          for (int d = tid >> 5; d < kD; d += kThreads / 32) s_vt[d * a.vt_pitch + t] = src[d * S];
        }
      }
    }
  }

  // queries with the biases, pre-scaled into log2 units
  F qu[2], qv[2];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      set(qu[half], e, (get(qq[half], e) + get(uu[half], e)) * a.scale_log2);
      set(qv[half], e, (get(qq[half], e) + get(ww[half], e)) * a.scale_log2);
    }

  // Merge slot of virtual wave vv: its o^T tile (kD rows of the 16 query columns, pitch SP), then
  // m and l. With several physical waves each virtual wave has a slot at s_wave and its shift
  // tile aliases it. With one, the LDS is cut so that eight workgroups fit a CU: one shift tile at
  // s_wave for every virtual wave, the third wave's slot after it, the first two slots in the
  // chunk's staging area (free once the append below has read it), and the last wave's state
  // merged from its registers.
  constexpr bool kOne = kPhys == 1;
  constexpr int SP = kOne ? 16 : kOPitch;
  constexpr int SF = kD * SP + 32;
  auto slot = [&](int vv) -> float* {
    if constexpr (kOne) {
      return vv < 2 ? reinterpret_cast<float*>(smem + a.off_kt) + vv * SF : s_wave + kSkewFloats;
    }
    return s_wave + vv * kWaveLds;
  };
  auto shift_tile = [&](int vv) -> float* { return kOne ? s_wave : s_wave + vv * kWaveLds; };
  // the virtual wave being run (uniform over the wave), its shift tile and its online-softmax
  // state
  int v = v0;
  float* s_g = shift_tile(v0);
  Softmax st;
  // Transformer-XL steps keep the running maximum in the folded form (step_fold): the band
  // products start their accumulation at rr.nr, so the scores need no subtraction
  RunRef rr;
  auto reset = [&]() {
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    runref_init(rr);
  };
  reset();

  // tail steps of virtual wave vv over the chunk's frames, from LDS (its first one, when it is
  // this wave's first virtual wave, with the table rows requested at the start)
  auto tail_steps = [&](int vv) {
    for (int k = vv; k < ntail; k += kWaves) {
      const int j0 = cache + 32 * k;
      F kf[2][2], vf[4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const T* row = s_kt + (32 * k + 8 * (m16 >> 2) + 4 * tt + (m16 & 3)) * KTP + 8 * grp;
        kf[tt][0] = load8(row);
        kf[tt][1] = load8(row + 32);
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vf[dt] = load8(s_vt + (16 * dt + m16) * a.vt_pitch + 32 * k + 8 * grp);
      if constexpr (kPerKey) {
        F pk[2][2];
        if (k == v0) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int half = 0; half < 2; ++half) pk[tt][half] = tb[tt][half];   // prefetched
        } else {
          load_key_rows(pk, j0);
        }
        float x[2][4];
        per_key_scores<T>(kf, pk, qu, qv, x);
        softmax_pv<T, true>(st, x, vf, 0, T_len - j0);
      } else {
        F pb[3][2];
        if (k == v0) {
#pragma unroll
          for (int t = 0; t < 3; ++t)
#pragma unroll
            for (int half = 0; half < 2; ++half) pb[t][half] = tb[t][half];   // prefetched
        } else {
          const int rb = R0 + j0 - qlast;
#pragma unroll
          for (int t = 0; t < 3; ++t) {
            const T* row = band_row(rb + 16 * t + m16) + 8 * grp;
            pb[t][0] = load8(row);
            pb[t][1] = load8(row + phalf);
          }
        }
        floatx4 g[3];
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          g[t] = mma(pb[t][0], qv[0], rr.nr);
          g[t] = mma(pb[t][1], qv[1], g[t]);
        }
        step_fold<T, true>(st, rr, kf, vf, qu, g[0], g[1], g[2], s_g, T_len - j0);
      }
    }
  };
  // the state of virtual wave vv into its merge slot (with one physical wave, the last one's
  // stays in registers)
  auto flush = [&](int vv) {
    st.l = column_sum(st.l);
    if constexpr (!kPerKey) st.m = rr.m;   // (the folded steps keep the running maximum in rr)
    if (kOne && vv == kWaves - 1) return;
    float* s_o = slot(vv);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_o[(16 * dt + 4 * grp + e) * SP + m16] = st.o[dt][e];
    if (grp == 0) {
      s_o[kD * SP + m16] = st.m;
      s_o[kD * SP + 16 + m16] = st.l;
    }
  };

  // ---- 6. fused append: this tile's chunk frames from LDS into the pool ---------------------
  // (issued after the wave's last load, so no load wait queues behind these stores, and they
  // drain while the waves merge; with one physical wave, right after the tail step instead, so
  // that the staging area is free for the merge slots)
  auto append = [&]() {
    if (kFused && h == hk * (a.H / a.Hk)) {
      const int t_lo = qt * 16;
      const int t_hi = min(n_real, t_lo + 16);
      for (int x = tid; x < (t_hi - t_lo) * NV; x += kThreads) {
        const int t = t_lo + x / NV;
        const int dv = (x % NV) * VEC;
        const int key = cache + t;
        T* dst = a.k_pool_w + (size_t)hk * page + (uint64_t)block_of(key >> logS) * blk_stride +
                 (uint32_t)(((dv >> 5) * S + (key & (S - 1))) * 32 + (dv & 31));
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(s_kt + t * KTP + dv);
      }
      // V: 8-frame groups of one dimension, aligned to the page slots (never across a page: block
      // sizes are powers of two >= 8); one 16-byte store when all 8 frames belong to this tile
      const int f_lo = cache + t_lo, f_hi = cache + t_hi;
      const int g0 = (f_lo >> 3) << 3;
      const int ngroups = (f_hi - g0 + 7) >> 3;
      for (int x = tid; x < ngroups * kD; x += kThreads) {
        const int d = x & (kD - 1);
        const int kg = g0 + 8 * (x >> 6);
        T* dst = a.v_pool_w + (size_t)hk * page + (uint64_t)block_of(kg >> logS) * blk_stride +
                 (uint32_t)(d * S + (kg & (S - 1)));
        const T* row = s_vt + d * a.vt_pitch;
        if (kg >= f_lo && kg + 8 <= f_hi) {
          F v8;
#pragma unroll
          for (int c = 0; c < 8; ++c) set(v8, c, to_f(row[kg + c - cache]));
          store8(dst, v8);
        } else {
          for (int c = 0; c < 8; ++c)
            if (kg + c >= f_lo && kg + c < f_hi) dst[c] = row[kg + c - cache];
        }
      }
    }
  };

  // ---- 4. tail steps of the first virtual wave over the chunk's frames, from LDS, first (the
  // one workgroup barrier: the tail was staged by all threads; the body below uses only the
  // wave's own registers and LDS). The wave with a tail step runs it while its body data is
  // still arriving. -----------------------------------------------------------------------------
  __syncthreads();
  tail_steps(v0);
  if constexpr (kOne) append();

  // ---- 5. body steps, two register sets in turn ------------------------------------------------
  // With several virtual waves per physical wave, the step that opens a later virtual wave first
  // moves the finished one's state to its merge slot and starts the next, whose first band
  // product is computed from the band tile the step before loaded: the same rows and the same
  // products as a wave of its own would form.
  int vend = vbound(v0 + 1);
  if (nmine > 0) {
    floatx4 g_prev = {0.f, 0.f, 0.f, 0.f};
    F p_next[2];   // the band tile that opens the next virtual wave (its first step's tile 0)
    if (!kPerKey) {
      g_prev = mma(p0[0], qv[0], rr.nr);
      g_prev = mma(p0[1], qv[1], g_prev);
    }
    auto run = [&](StepRegs<T>& r, int s) {
      if constexpr (kR > 1) {
        if (s >= vend) {
          do {
            flush(v);
            ++v;
            vend = vbound(v + 1);
            s_g = shift_tile(v);
            reset();
          } while (s >= vend);
          if constexpr (!kPerKey) {
            // (when the virtual waves before it had no body step, the band tile requested with the
            // first steps is this step's first)
            const bool first = s == s_begin;
            g_prev = mma(first ? p0[0] : p_next[0], qv[0], rr.nr);
            g_prev = mma(first ? p0[1] : p_next[1], qv[1], g_prev);
          }
        }
      }
      // the last cached page may be partly filled: frames at or past cache are then excluded,
      // and their V is zeroed (the slots may hold anything)
      const bool part = s == s_part;
      if (part) zero_from(r.v, cache - (32 * s + 8 * grp));
      if constexpr (kPerKey) {
        float x[2][4];
        per_key_scores<T>(r.k, r.p, qu, qv, x);
        if (part) softmax_pv<T, true>(st, x, r.v, 0, cache - 32 * s);
        else softmax_pv<T, false>(st, x, r.v, 0, 32);
      } else {
        floatx4 g1 = mma(r.p[0][0], qv[0], rr.nr);
        g1 = mma(r.p[0][1], qv[1], g1);
        floatx4 g2 = mma(r.p[1][0], qv[0], rr.nr);
        g2 = mma(r.p[1][1], qv[1], g2);
        if constexpr (kR > 1) {
          // the next step opens another virtual wave: keep its first band tile
          if (s + 1 == vend && s + 1 < s_end) {
            p_next[0] = r.p[1][0];
            p_next[1] = r.p[1][1];
          }
        }
        if (part) step_fold<T, true>(st, rr, r.k, r.v, qu, g_prev, g1, g2, s_g, cache - 32 * s);
        else step_fold<T, false>(st, rr, r.k, r.v, qu, g_prev, g1, g2, s_g, 32);
        g_prev = g2;
      }
      if (s + 2 < s_end) load_step(r, s + 2);
    };
    if (nmine == 2) {
      // (straight-line: the first step's wait leaves the second step's loads outstanding; in
      // the loop, whose head is also reached without them, the compiler drained every load)
      run(ra, s_begin);
      run(rb2, s_begin + 1);
    } else {
      for (int s = s_begin; s < s_end; s += 2) {
        run(ra, s);
        if (s + 1 < s_end) run(rb2, s + 1);
      }
    }
  }
  // the virtual waves left: the current one, then any after it with no body step (and no tail
  // step: see above)
  flush(v);
  for (int vv = v + 1; vv < v0 + kR; ++vv) {
    reset();
    flush(vv);
  }
  if constexpr (!kOne) append();

  // ---- 7. merge the virtual waves' partial states in a fixed order ------------------------------
  if constexpr (kOne) {
    // one wave: each lane combines its own query column's dimensions 16 dt + 4 grp + e, the last
    // virtual wave's from its registers - the same operations, in the same order, as below
    const int i = qt * 16 + m16;
    float mw[kWaves], lw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = w < kWaves - 1 ? slot(w)[kD * SP + m16] : st.m;
      lw[w] = w < kWaves - 1 ? slot(w)[kD * SP + 16 + m16] : st.l;
    }
    float mmax = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mmax = fmaxf(mmax, mw[w]);
    float lsum = 0.f;
    float acc[4][4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[dt][e] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(mw[w] - mmax);
      lsum += f * lw[w];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[dt][e] += f * (w < kWaves - 1 ? slot(w)[(16 * dt + 4 * grp + e) * SP + m16] : st.o[dt][e]);
    }
    const float inv = 1.f / lsum;
    if (i < a.C) {
      T* dst = a.out + (((size_t)b * a.C + i) * a.H + h) * kD + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[16 * dt + e] = from_f<T>(acc[dt][e] * inv);
    }
    return;
  }
  __syncthreads();
  for (int x = tid; x < 16 * (kD / 4); x += kThreads) {
    const int il = x & 15;
    const int d0 = (x >> 4) * 4;
    const int i = qt * 16 + il;
    if (i >= a.C) continue;
    T* dst = a.out + (((size_t)b * a.C + i) * a.H + h) * kD + d0;
    if (kGen && i >= n_real) {
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[k] = from_f<T>(0.f);
      continue;
    }
    float mmax = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mmax = fmaxf(mmax, s_wave[w * kWaveLds + kD * kOPitch + il]);
    float lsum = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* so = s_wave + w * kWaveLds;
      const float f = fast_exp2(so[kD * kOPitch + il] - mmax);
      lsum += f * so[kD * kOPitch + 16 + il];
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] += f * so[(d0 + k) * kOPitch + il];
    }
    const float inv = 1.f / lsum;
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = from_f<T>(acc[k] * inv);
  }

}

// Virtual waves per unit: fixed (never chosen from the cohort size), so a stream's step-to-wave
// assignment and merge order, and with them its result bits, depend on its own length only. The
// physical waves per workgroup (launch_chunk_t) change the speed, not the bits.
template <typename T> constexpr int waves_of() { return 4; }

// LDS layout for kPhys physical waves: merge slots and shift tiles (with one physical wave one
// shift tile and one slot, the first two slots then reusing the chunk's staging area), block-ID
// windows, the chunk's K rows and V^T. Returns the bytes.
template <typename T>
size_t chunk_lds_layout(ChunkArgs<T>& a, int phys) {
  size_t off = phys == 1 ? (size_t)(kSkewFloats + kD * 16 + 32) * sizeof(float)
                         : (size_t)waves_of<T>() * kWaveLds * sizeof(float);
  a.off_bt = (int)off;
  off += (size_t)phys * kBtWindow * sizeof(int);
  a.off_kt = (int)off;
  off += (size_t)a.tail_cap * kt_pitch<T>() * sizeof(T);
  a.off_vt = (int)off;
  off += (size_t)kD * a.vt_pitch * sizeof(T);
  return off;
}

template <typename T, bool kFused, int kS, bool kRegTail, bool kPerKey = false, bool kGen = true,
          int kPhys = 4, bool kRank = false>
void launch_inst(const ChunkArgs<T>& a_in, dim3 grid, hipStream_t stream) {
  // (the layout follows the variant launched, whatever count the host asked for)
  ChunkArgs<T> a = a_in;
  a.phys = kPhys;
  const size_t smem = chunk_lds_layout(a, kPhys);
  if (smem > 64 * 1024) {
    // beyond the default dynamic LDS size (long chunks): opt in on every such call, so that no
    // state is kept between calls (a host-side attribute, no GPU work); MI355X allows 160 KB per
    // workgroup
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(
            &chunk_attn_kernel<T, kFused, kPhys, kS, kRegTail, kPerKey, kGen, kRank>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  }
  hipLaunchKernelGGL((chunk_attn_kernel<T, kFused, kPhys, kS, kRegTail, kPerKey, kGen, kRank>),
                     grid, dim3(kPhys * 64), smem, stream, a);
}

// the lean variant (no chunk lengths or window starts) at a.phys physical waves per workgroup
// (register-held chunks only: see the kernel; longest-first order at four physical waves)
template <typename T, bool kFused, int kS, bool kRegTail>
void launch_phys(const ChunkArgs<T>& a, dim3 grid, hipStream_t stream) {
  if constexpr (kRegTail) {
    if (a.phys == 1) return launch_inst<T, kFused, kS, true, false, false, 1>(a, grid, stream);
    if (a.phys == 2) return launch_inst<T, kFused, kS, true, false, false, 2>(a, grid, stream);
  }
  if (a.rank) return launch_inst<T, kFused, kS, kRegTail, false, false, 4, true>(a, grid, stream);
  launch_inst<T, kFused, kS, kRegTail, false, false, 4>(a, grid, stream);
}

// Instantiation for a call: the block sizes of the streaming workloads get constant page
// geometry and, without chunk lengths or window starts, the lean kGen = false variant (at 1, 2
// or 4 physical waves); fp32 (used for checking), per-key tables and the rest take the general
// ones, at 4.
template <typename T, bool kFused, bool kRegTail>
void launch_lean(const ChunkArgs<T>& a, dim3 grid, hipStream_t stream) {
  const bool gen = a.lens != nullptr || a.ws != nullptr;
  if (a.S == 16) {
    if (gen) return launch_inst<T, kFused, 16, kRegTail, false, true>(a, grid, stream);
    return launch_phys<T, kFused, 16, kRegTail>(a, grid, stream);
  }
  if (a.S == 32) {
    if (gen) return launch_inst<T, kFused, 32, kRegTail, false, true>(a, grid, stream);
    return launch_phys<T, kFused, 32, kRegTail>(a, grid, stream);
  }
  if (gen) return launch_inst<T, kFused, 0, kRegTail, false, true>(a, grid, stream);
  launch_inst<T, kFused, 0, kRegTail, false, false>(a, grid, stream);
}

template <typename T, bool kFused>
void launch_s(const ChunkArgs<T>& a, dim3 grid, hipStream_t stream) {
  // register-held chunk for fused bf16 chunks of at most 32 frames (one 16-byte vector of K and
  // one of V per thread, requested at kernel start)
  constexpr bool kRegOk = sizeof(T) == 2 && kFused;
  const bool reg_tail = kRegOk && a.C <= 32;
  if (a.per_key) {
    if constexpr (kRegOk) {
      if (reg_tail) return launch_inst<T, kFused, 0, true, true>(a, grid, stream);
    }
    return launch_inst<T, kFused, 0, false, true>(a, grid, stream);
  }
  if constexpr (sizeof(T) == 2) {
    if constexpr (kRegOk) {
      if (reg_tail) return launch_lean<T, kFused, true>(a, grid, stream);
    }
    return launch_lean<T, kFused, false>(a, grid, stream);
  }
  launch_inst<T, kFused, 0, false>(a, grid, stream);
}

// Physical waves per workgroup for a grid of `units` workgroups: one when the grid fills every
// wave slot of the GPU with one wave per unit (eight per CU at the kernel's two waves per SIMD),
// so that a large cohort runs eight units per CU at once instead of two; else four. (Two waves
// measured no faster than four on the ragged cohort.) PKC_CHUNK_WAVES = 1, 2 or 4 forces a count;
// the results are the same at any count. `cus`: the device's CU count, 0 if unknown.
int phys_waves(int64_t units, int cus) {
  if (const char* e = getenv("PKC_CHUNK_WAVES")) {
    const int w = atoi(e);
    if (w == 1 || w == 2 || w == 4) return w;
  }
  if (cus <= 0) return 4;
  return units >= (int64_t)cus * 8 ? 1 : 4;
}

// Longest cache first when the grid takes more than one pass over the CUs at `phys` physical
// waves per workgroup (two waves per SIMD: 8 / phys workgroups per CU), for at most 4096 streams
// (each workgroup walks every stream's length twice to find its own). PKC_CHUNK_ORDER = 0 or 1
// forces the choice; the results are the same either way.
int rank_streams(int64_t units, int batch, int phys, int cus) {
  if (const char* e = getenv("PKC_CHUNK_ORDER")) {
    const int o = atoi(e);
    if (o == 0 || o == 1) return batch <= 4096 ? o : 0;
  }
  if (cus <= 0 || batch > 4096) return 0;
  return units > (int64_t)cus * (8 / phys) ? 1 : 0;
}

template <typename T>
hipError_t launch_chunk_t(const AttnParams& p, hipStream_t stream) {
  ChunkArgs<T> a;
  a.q = (const T*)p.q;
  a.k_pool = (const T*)p.k_pool;
  a.v_pool = (const T*)p.v_pool;
  a.bt = p.block_tables;
  a.cs = p.cache_seqlens;
  a.lens = p.chunk_lens;
  a.ws = p.window_start;
  a.pos = (const T*)p.pos;
  a.u = (const T*)p.pos_bias_u;
  a.w = (const T*)p.pos_bias_v;
  a.out = (T*)p.out;
  a.k_new = (const T*)p.k_new;
  a.v_new = (const T*)p.v_new;
  a.k_pool_w = (T*)p.k_pool_w;
  a.v_pool_w = (T*)p.v_pool_w;
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
  a.per_row = p.pos_layout & PKC_POS_PER_ROW;
  a.per_key = (p.pos_layout & PKC_POS_PER_KEY) != 0;
  const bool blocked = (p.pos_layout & PKC_POS_COL_BLOCKED) != 0;
  a.band_rs = blocked ? 32 : p.n_head * kD;
  a.band_hs = blocked ? 32 * p.pos_len : 32;
  a.band_hd = blocked ? kD * p.pos_len : kD;
  a.qtiles = (p.chunk + 15) / 16;
  a.div_qtiles = make_fastdiv(a.qtiles);
  a.div_H = make_fastdiv(a.H);
  a.div_group = make_fastdiv(a.H / a.Hk);
  a.tail_cap = ((p.chunk + 31) / 32) * 32;
  a.vt_pitch = a.tail_cap + 16 / (int)sizeof(T);
  const LaunchGrid lg = chunk_attn_grid((int)sizeof(T), p.batch, p.n_head, p.chunk);
  // physical waves: fewer than 4 only for the register-held chunks of the lean bf16 variant
  const bool lean = sizeof(T) == 2 && p.k_new && p.chunk <= 32 && !p.chunk_lens &&
                    !p.window_start && !a.per_key && (p.block_size == 16 || p.block_size == 32);
  const int cus = device_cus();
  a.phys = lean ? phys_waves(lg.workgroups, cus) : 4;
  a.B = p.batch;
  a.div_hq = make_fastdiv(a.H * a.qtiles);
  // (ranked only in the bf16 variants without chunk lengths or window starts, at four physical
  // waves: the ones launch_phys dispatches)
  const bool rankable = sizeof(T) == 2 && !p.chunk_lens && !p.window_start && !a.per_key &&
                        (p.block_size == 16 || p.block_size == 32) && a.phys == 4;
  a.rank = rankable ? rank_streams(lg.workgroups, p.batch, a.phys, cus) : 0;
  const float scale = p.softmax_scale > 0.f ? p.softmax_scale : 1.f / sqrtf((float)p.head_dim);
  a.scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)lg.workgroups);
  // (launch_inst lays out the LDS of the variant it launches)
  if (p.k_new) launch_s<T, true>(a, grid, stream);
  else launch_s<T, false>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();   // (a failed query must not surface as the launch's error)
    return 0;
  }
  return cus;
}

size_t chunk_attn_lds_bytes(int dtype_bytes, int chunk, int, int, bool) {
  const int tail_cap = ((chunk + 31) / 32) * 32;
  const int vec = 16 / dtype_bytes;
  const int waves = dtype_bytes == 2 ? waves_of<bf16>() : waves_of<float>();
  return (size_t)waves * kWaveLds * 4 + (size_t)waves * kBtWindow * 4 +
         (size_t)tail_cap * (kD + vec) * dtype_bytes + (size_t)kD * (tail_cap + vec) * dtype_bytes;
}

LaunchGrid chunk_attn_grid(int dtype_bytes, int batch, int n_head, int chunk) {
  const int waves = dtype_bytes == 2 ? waves_of<bf16>() : waves_of<float>();
  return {mul_sat(mul_sat(batch, n_head), ((int64_t)chunk + 15) / 16), waves * 64};
}

hipError_t launch_chunk_attn(pkc_dtype dtype, const AttnParams& p, hipStream_t stream) {
  return dtype == PKC_BF16 ? launch_chunk_t<bf16>(p, stream) : launch_chunk_t<float>(p, stream);
}

}  // namespace pkc
