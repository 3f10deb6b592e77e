// Packed varlen relative-position attention for gfx950 (the offline forward).
//
// Sources: OASR docs, "Model Layer", "The engine-facing surface" (forward_offline_packed: gapless
// varlen rows, attention inside each utterance); "ASR Engine", section 4.1 (sequence packing);
// "Model Layer", fixed_attention_window declaration (Transformer-XL distances i - j). Each
// utterance of length L is the chunk case with no cache and C = L: query i and key j read table
// row L - 1 + j - i of the utterance's 2 L - 1 rows.
//
// Work decomposition. One workgroup of 4 waves per (utterance, query tile, head), the head
// varying fastest over the grid so that all tiles of one head share an XCD. For bf16 a wave owns
// 32 queries as two 16-query MFMA tiles (a workgroup 128); fp32, and the chunked_limited mask,
// keep one tile (64): every K, V and band fragment a wave reads from LDS then feeds both tiles,
// which halves the LDS reads per MFMA (the CU's LDS bandwidth, shared by its four SIMDs, bounded
// the step). Each tile keeps its own online softmax; no merge. The workgroup walks the
// utterance's keys in stages of two 32-key steps (one with one tile per wave): every stage's K
// rows and V rows are staged once in double-buffered LDS and read by all four waves, with one
// barrier per stage. The band rows (the table rows the queries touch) go through an LDS ring of
// 256 rows (128 with one tile per wave): the waves' windows overlap, so a stage brings in only
// the rows that enter the workgroup's window. Every global read is issued at least two steps
// before its rows are used: two-step stages request a stage's rows one stage ahead, one-step
// stages two. The step's arithmetic is step_tiles below, with the folded running-max reference
// of pkc_step.h. MFMA-bound in principle (6 L^2 D FLOP per utterance and head).
//
// Band tiles of a wave at a step: T_m = rows [xb + 16 m, xb + 16 m + 16), m = 0 .. kQT + 1, where
// query tile k (first query q0 + 16 k) reads T_{kQT-1-k}, T_{kQT-k} and T_{kQT+1-k}. The next step's
// T_0 and T_1 are this step's T_2 and T_3: the first band product of every tile, and (two tiles) the
// fragments of T_1, carry over in registers, so a step reads two new band tiles from LDS.
//
// V staging. For bf16, V rows stay in their natural [key][head_dim] order in LDS (one 16-byte
// write per thread) and the PV operand - 8 consecutive keys of one dimension per lane - comes
// from two transposing reads; the 4-dimension chunks of row r are XOR-swizzled by
// 4 ((r & 3) ^ ((r >> 4) & 1)), which puts the rows one half-wave reads (two key groups 16 rows
// apart) on distinct banks. fp32 stages V transposed to [head_dim][key].
//
// LDS layouts were chosen by measurement: a one-wave probe repeating each access pattern, read
// through SQ_LDS_BANK_CONFLICT, found every K, V, band and shift read of a step conflict-free
// with these layouts (the earlier padded pitches and natural key-group order cost 2 to 4 extra
// cycles per read).
//
// chunked_limited mask ("Model Layer", Nemotron encoder notes; kLimited): query i sees only the
// keys of its own chunk of `chunk` frames and of the `left` chunks before it. A workgroup then
// walks only the keys its 64 queries can see - its own frames plus the trained history, as one
// streaming step per query block - and each query column masks to its own range.
#include <type_traits>

#include "pkc_device.h"
#include "pkc_launch.h"
#include "pkc_step.h"

namespace pkc {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// 16-query tiles per wave: two for bf16 over the full context, one for fp32 and for the
// chunked_limited mask (a workgroup walks the union of its queries' visible keys, so smaller
// query tiles waste fewer masked steps)
template <typename T, bool kLim> constexpr int kQT = (sizeof(T) == 2 && !kLim) ? 2 : 1;
template <typename T, bool kLim> constexpr int kQTile = 16 * kQT<T, kLim> * kWaves;  // per workgroup

// 32-key steps per staging stage (one barrier, one K/V buffer): two with two query tiles per wave,
// so that a workgroup meets half as many barriers per key and its global reads run 128 keys
// ahead; one elsewhere
template <typename T, bool kLim> constexpr int kSubs = kQT<T, kLim> == 2 ? 2 : 1;
template <typename T> constexpr int kKP = kD + 16 / (int)sizeof(T);   // band / fp32 K row pitch
template <typename T> constexpr bool kSwK = sizeof(T) == 2;            // swizzled bf16 K rows
// Band ring rows. With two-step stages (bf16, two tiles): 128 bytes, unpadded, so that the two
// stages of K and V and the ring fit two workgroups per CU, the eight 16-byte chunks of slot x
// permuted by chunk ^ (x & 7). A band-tile read (16 consecutive slots, one chunk per lane group)
// and a staging write (8 lanes per slot) measured conflict-free on gfx950 at every starting slot;
// chunk ^ ((x >> 1) & 7) cost 3.2 extra cycles per read at most starting slots. Otherwise 160
// bytes for bf16 (a read of 16 consecutive rows measured conflict-free at any starting row; 144,
// 176 and 208 bytes cost 4 extra cycles per read).
template <typename T, bool kLim> constexpr bool kBandSwz = kSubs<T, kLim> == 2;
template <typename T, bool kLim> constexpr int kBP =
    kBandSwz<T, kLim> ? kD : (sizeof(T) == 2 ? kD + 16 : kKP<T>);
template <typename T> constexpr int kVP = 32 + 16 / (int)sizeof(T);   // V^T tile row pitch (fp32)
template <typename T> constexpr bool kTrV = sizeof(T) == 2;            // natural V rows + tr reads
// rows of the band ring: it spans the lowest row a stage reads to the highest it stages,
// 16 QT kWaves + 64 kSubs rows (256 with two tiles and two-step stages, 128 with one and one)
template <typename T, bool kLim> constexpr int kRing = 16 * kQT<T, kLim> * kWaves + 64 * kSubs<T, kLim>;
// waves per SIMD the register budget targets: bf16 two-tile waves 2, bf16 one-tile waves 3; fp32
// (one workgroup per CU by its LDS) 1
template <typename T, bool kLim> constexpr int kWavesPerSimd =
    sizeof(T) == 4 ? 1 : (kQT<T, kLim> == 2 ? 2 : 3);
constexpr int kSortMax = 64;   // utterances a wave ranks by length (one per lane)
// Lane group g holds the keys of key_group<true>(g) (groups 1 and 2 swapped): the shifted
// position values are then read conflict-free.
constexpr bool kPerm = true;
// swizzle of the 4-dimension chunks of natural V row r (bf16): with the swapped key groups the two
// lane groups of a half-wave read rows 16 apart, told apart by bit 4
__device__ __forceinline__ int v_swz(int r) { return 4 * ((r & 3) ^ ((r >> 4) & 1)); }
// bf16 K rows are 128 bytes, unpadded, with their eight 16-byte chunks permuted by chunk ^ k_swz(r).
// A key-tile read (16 lanes per row set 8 kg(a) + 4 tt + b, a, b < 4, one 16-byte chunk per lane
// group) measured conflict-free on gfx950 with either key-group order; a padded 144-byte pitch
// cost 4 extra cycles per read. Bit 2 of r is not used, so the tt = 1 rows share the tt = 0 rows'
// permutation.
__device__ __forceinline__ int k_swz(int r) {
  return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r ^ (r >> 4)) & 1) << 2);
}

// One 32-key step of a wave's QT query tiles, written in phases so that the tiles' independent
// work sits in one basic block and interleaves: the band products of every tile (accumulated onto
// -r); the relative shift of each tile through the wave's skew tile, tile after tile (LDS executes
// a wave's accesses in order, so tile k + 1's writes land after tile k's reads), each shifted
// column starting the accumulation of that tile's content product (S^T = K (q + u)^T), so the
// scores are x - r; a per-lane test of the scores against thr and one ballot for all tiles (a
// single uniform branch, rarely taken: the column maxima, the new running maxima, the rescale of
// the accumulators and the re-basing of the scores and the carried band product are done only
// there); then the probabilities exp2(x - r), the PV products and the row sums on the MFMA (an
// all-ones operand against the probabilities: the sums are those of the bf16-rounded
// probabilities the values are weighted with). Tile k's band tiles are pb[QT-1-k] and pb[QT-k]
// (g1, g2) after the carried product g_prev[k]. kMask: only keys lo[k] <= key < hi[k] of the step
// count for tile k (relative to the step's first key).
template <typename T, int QT, bool kMask>
__device__ __forceinline__ void step_tiles(Softmax (&st)[QT], RunRef (&rr)[QT],
                                           const typename Frag<T>::type (&kf)[2][2],
                                           const typename Frag<T>::type (&vf)[4],
                                           const typename Frag<T>::type (&qu)[QT][2],
                                           const typename Frag<T>::type (&qv)[QT][2],
                                           const typename Frag<T>::type (&pb)[QT + 1][2],
                                           floatx4 (&g_prev)[QT], float* s_g,
                                           const int (&lo)[QT], const int (&hi)[QT]) {
  typedef typename Frag<T>::type F;
  const int lane = threadIdx.x & 63;
  const int m16 = lane & 15;
  const int grp = lane >> 4;
  const int kg = key_group<kPerm>(grp);
  floatx4 g1[QT], g2[QT];
#pragma unroll
  for (int k = 0; k < QT; ++k) {
    g1[k] = mma(pb[QT - 1 - k][0], qv[k][0], rr[k].nr);
    g1[k] = mma(pb[QT - 1 - k][1], qv[k][1], g1[k]);
    g2[k] = mma(pb[QT - k][0], qv[k][0], rr[k].nr);
    g2[k] = mma(pb[QT - k][1], qv[k][1], g2[k]);
  }
  // shift: G^T[row][query] -> s_g[query * kSkewPitch + row]; the lane reads its 8 keys' values
  // from its own query column, shifted by 15 - query
  float* colw = s_g + m16 * kSkewPitch + 4 * grp;
  const float* colr = s_g + m16 * kSkewPitch + 15 - m16 + 8 * kg;
  floatx4 sc[QT][2];
#pragma unroll
  for (int k = 0; k < QT; ++k) {
    *reinterpret_cast<floatx4*>(colw) = g_prev[k];
    *reinterpret_cast<floatx4*>(colw + 16) = g1[k];
    *reinterpret_cast<floatx4*>(colw + 32) = g2[k];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      sc[k][tt] = floatx4{colr[4 * tt], colr[4 * tt + 1], colr[4 * tt + 2], colr[4 * tt + 3]};
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sc[k][tt] = mma(kf[tt][0], qu[k][0], sc[k][tt]);
      sc[k][tt] = mma(kf[tt][1], qu[k][1], sc[k][tt]);
    }
    g_prev[k] = g2[k];
  }
  float lm[QT];   // this lane's maximum over its 8 keys, relative to r
  bool over = false;
#pragma unroll
  for (int k = 0; k < QT; ++k) {
    float m = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (kMask) {
          const int key = 8 * kg + 4 * tt + e;
          sc[k][tt][e] = (key >= lo[k] && key < hi[k]) ? sc[k][tt][e] : -INFINITY;
        }
        m = fmaxf(m, sc[k][tt][e]);
      }
    lm[k] = m;
    over = over || m > rr[k].thr;
  }
  if (__ballot(over) != 0) {
#pragma unroll
    for (int k = 0; k < QT; ++k) {
      const float d = runref_move(rr[k], lm[k], st[k].o, st[k].ls);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) sc[k][tt] -= d;
      g_prev[k] -= d;
    }
  }
#pragma unroll
  for (int k = 0; k < QT; ++k) {
    F pf;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) set(pf, 4 * tt + e, fast_exp2(sc[k][tt][e]));
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st[k].o[dt] = mma(vf[dt], pf, st[k].o[dt]);
    st[k].ls = mma(ones8<T>(), pf, st[k].ls);
  }
}

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
  int H, Hk, qtiles, total, maxlen, num_seqs;
  FastDiv div_H, div_qtiles, div_group;   // by H, qtiles and H / Hk
  int chunk, left;            // chunked_limited mask (kLimited)
  float scale_log2;
};

// (register budget: kWavesPerSimd waves per SIMD)
template <typename T, bool kLimited>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kWavesPerSimd<T, kLimited>, kWavesPerSimd<T, kLimited>)))
varlen_attn_kernel(VarlenArgs<T> a) {
  typedef typename Frag<T>::type F;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NV = kD / VEC;
  constexpr int KP = kKP<T>;
  constexpr int VP = kVP<T>;
  constexpr int QT = kQT<T, kLimited>;                             // query tiles per wave
  constexpr int QTILE = kQTile<T, kLimited>;                       // queries per workgroup
  constexpr int SUBS = kSubs<T, kLimited>;                         // 32-key steps per stage
  constexpr int SK = 32 * SUBS;                                    // keys per stage
  constexpr int KT = kSwK<T> ? kD : KP;                            // K tile row pitch
  constexpr int TILE = SK * KT + (kTrV<T> ? SK * kD : kD * VP);   // elements of one K + V stage
  static_assert(kTrV<T> || SUBS == 1, "the transposed V tile holds one 32-key step");

  __shared__ __align__(16) T s_kv[2 * TILE];
  constexpr bool BSW = kBandSwz<T, kLimited>;
  constexpr int BP = kBP<T, kLimited>;
  constexpr int RING = kRing<T, kLimited>;
  static_assert((RING & (RING - 1)) == 0, "ring slots are row & (RING - 1)");
  static_assert(!BSW || sizeof(T) == 2, "the ring swizzle permutes 16-byte chunks of bf16 rows");
  __shared__ __align__(16) T s_band[RING * BP];   // row x of the table in slot x % RING
  // one shift tile per wave, used by its query tiles in turn (LDS executes a wave's accesses in
  // order, so a tile's writes never overtake the previous tile's reads)
  __shared__ __align__(16) float s_skew[kWaves * kSkewFloats];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m16 = lane & 15;
  const int grp = lane >> 4;

  // head fastest: workgroups go to the 8 XCDs round-robin, so with H a multiple of 8 every tile
  // of one head lands on the same XCD and that head's tables and K/V rows stay in its L2
  const int id = blockIdx.x;
  const int tix = fdiv(id, a.div_H);   // query tile of the launch
  const int h = id - tix * a.H;
  // Longest utterances first. Workgroups start roughly in index order and every tile of an
  // utterance walks its whole length, so a long utterance reached last sets the launch's tail.
  // With at most 64 utterances each wave ranks them by length (descending, ties by index), lays
  // their query tiles out in that order and takes tile tix of it; more keep the natural order.
  int s, qt;
  if (a.num_seqs <= kSortMax) {
    int Lu = -1, nq = 0;   // lane u: utterance u's length and query tiles
    if (lane < a.num_seqs) {
      const int lo_u = clampi(a.cu[lane], 0, a.total);
      Lu = min(clampi(a.cu[lane + 1], lo_u, a.total) - lo_u, a.maxlen);
      nq = (Lu + QTILE - 1) / QTILE;
    }
    int first = 0;         // tiles of the utterances ranked before lane u's
    for (int t = 0; t < a.num_seqs; ++t) {
      const int Lt = __builtin_amdgcn_readlane(Lu, t);
      const int nt = __builtin_amdgcn_readlane(nq, t);
      first += (Lt > Lu || (Lt == Lu && t < lane)) ? nt : 0;
    }
    const uint64_t own = __ballot(lane < a.num_seqs && tix >= first && tix < first + nq);
    if (own == 0) return;  // past the last tile (uniform over the workgroup)
    s = (int)__builtin_ctzll(own);
    qt = tix - __builtin_amdgcn_readlane(first, s);
  } else {
    s = fdiv(tix, a.div_qtiles);
    qt = tix - s * a.qtiles;
  }
  const int lo = clampi(a.cu[s], 0, a.total);
  // (an utterance longer than max_seqlen is cut to max_seqlen frames: the host bounds every byte
  // offset from an utterance's first row by 2 max_seqlen rows, so 32-bit offsets hold)
  const int L = min(clampi(a.cu[s + 1], lo, a.total) - lo, a.maxlen);
  if (qt * QTILE >= L) return;  // uniform over the workgroup
  const int hk = fdiv(h, a.div_group);
  const size_t krow = (size_t)a.Hk * kD;      // elements between consecutive frames of k / v
  const size_t prow = (size_t)a.H * kD;
  // uniform segment bases; per-lane 32-bit byte offsets from them (one offset serves K and V)
  const char* kseg = reinterpret_cast<const char*>(a.k + (size_t)lo * krow + (size_t)hk * kD);
  const char* vseg = reinterpret_cast<const char*>(a.v + (size_t)lo * krow + (size_t)hk * kD);
  const char* ptab = reinterpret_cast<const char*>(a.pos + (size_t)(2 * lo) * prow + (size_t)h * kD);
  const uint32_t krow_b = (uint32_t)(krow * sizeof(T));
  const uint32_t prow_b = (uint32_t)(prow * sizeof(T));
  const int q0 = qt * QTILE + 16 * QT * wave;   // this wave's first query
  const int R0 = L - 1;                         // table row of (i, j) is R0 + j - i
  const int rlo = 0, rhi = 2 * L - 2;
  // a wave whose queries all lie past the utterance stages rows and meets the barriers, but
  // computes nothing (uniform over the wave)
  const int ntile = min(QT, max(0, (L - q0 + 15) >> 4));

  // the queries and the biases, requested first; q + u and q + v (pre-scaled into log2 units) are
  // formed after the first steps' rows are requested, so that waiting for them does not hold up
  // those requests
  F qq[QT][2], uu[2], ww[2];
#pragma unroll
  for (int k = 0; k < QT; ++k) {
    const T* qrow = a.q + ((size_t)(lo + min(q0 + 16 * k + m16, L - 1)) * a.H + h) * kD;
#pragma unroll
    for (int half = 0; half < 2; ++half) qq[k][half] = load8(qrow + 32 * half + 8 * grp);
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int d0 = 32 * half + 8 * grp;
    uu[half] = load8(a.u + h * kD + d0);
    ww[half] = load8(a.w + h * kD + d0);
  }

  // Band window. With C0 = R0 - (qt QTILE + 16 QT - 1), wave w's band tile T_m at the step whose
  // first key is j0 starts at row C0 + j0 - 16 QT w + 16 m (tile k's rows R0 + j0 - i for its
  // queries i begin at T_{QT-1-k}). Step 0 reads T_0 .. T_{QT+1} of every wave, rows
  // [C0 + J - 48 QT, C0 + J + 16 QT + 32); a later step T_2 .. T_{QT+1} (QT = 2) or T_1, T_2 (QT = 1),
  // the 64 QT rows below the window top C0 + j0 + 16 QT + 32. A stage of SK keys at j0 reads up to
  // the top xw + j0 + SK; the SK rows above it enter for the next stage: they are fetched with that
  // stage's K/V rows, rows [xw + j0', xw + j0' + SK) for its first key j0', and staged during this
  // one. The ring spans the lowest row a stage reads to the highest it stages (at most
  // 16 QT kWaves + 2 SK rows), so the rows staged during a stage never take a slot that stage
  // reads, and a row is overwritten only after the barrier that ends its last use.
  const int C0 = R0 - (qt * QTILE + 16 * QT - 1);
  const int xw = C0 + 16 * QT;   // band rows fetched with the stage at key j0: [xw + j0, + SK)
  // (the row and column offsets are summed in 32 bits first: one offset from the uniform base)
  auto band_src = [&](int x, uint32_t col_b) {
    return ptab + ((uint32_t)clampi(x, rlo, rhi) * prow_b + col_b);
  };
  // Slot of a staged 16-byte chunk. Every row this thread stages is xw + (tid / NV) plus a multiple
  // of 16, and the swizzle (slot bits 0 .. 2) depends on no higher bit: one column per thread.
  const int st_col = BSW ? 8 * ((tid % NV) ^ ((xw + tid / NV) & 7)) : (tid % NV) * VEC;
  auto band_slot = [&](int x) { return s_band + (x & (RING - 1)) * BP; };

  Softmax st[QT];
  RunRef rr[QT];
#pragma unroll
  for (int k = 0; k < QT; ++k) {
    st[k].ls = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st[k].o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    runref_init(rr[k]);
  }
  float* s_g = s_skew + wave * kSkewFloats;

  // the keys this workgroup's queries can see: all of the utterance, or with the chunked_limited
  // mask the first visible key of its first query to the last of its last query; and per query
  // column (this lane's query of each tile, clamped into the utterance) its own range
  int j_first = 0, j_end = L, k_lo_q[QT], k_hi_q[QT];
#pragma unroll
  for (int k = 0; k < QT; ++k) {
    k_lo_q[k] = 0;
    k_hi_q[k] = L;
  }
  if constexpr (kLimited) {
    const int left = min(a.left, L);   // more chunks than frames sees everything anyway
    const int tq0 = qt * QTILE;
    const int tq1 = min(tq0 + QTILE, L) - 1;
    j_first = max(0, (tq0 / a.chunk - left) * a.chunk);
    j_end = min(L, (tq1 / a.chunk + 1) * a.chunk);
#pragma unroll
    for (int k = 0; k < QT; ++k) {
      const int iq = min(q0 + 16 * k + m16, L - 1);
      k_lo_q[k] = max(0, (iq / a.chunk - left) * a.chunk);
      k_hi_q[k] = min(L, (iq / a.chunk + 1) * a.chunk);
    }
  }
  const int s_first = j_first >> 5;
  const int nsteps = ((j_end + 31) >> 5) - s_first;   // 32-key steps
  const int J = 32 * s_first;
  // cooperative staging of one stage: SK K rows, the same SK V rows and the SK band rows entering
  // the window. Rows past the utterance read its last frame instead: every staged value is
  // finite, so a masked key (probability exactly 0) adds nothing, and every load is
  // unconditional - a wait never has to drain loads requested for a later stage.
  constexpr int NLD = SK * NV / kThreads;   // 16-byte vectors per thread per tensor
  static_assert(NLD * kThreads == SK * NV, "the staging threads cover the stage's rows exactly");
  static_assert(kThreads % NV == 0 && (kThreads / NV) % 16 == 0,
                "a thread's staged rows differ by multiples of 16");
  struct Rows { u32x4 k[NLD], v[NLD], b[NLD]; };
  // Two-step stages hold one stage's rows in registers: a stage stashes the next stage's rows as
  // it starts and reuses their registers for the stage after (ra; rb only in the prologue and the
  // first stage). One-step stages keep two register sets in flight and stash as they end, so
  // that a load has two steps to arrive either way.
  constexpr bool ONE = SUBS == 2;
  Rows ra, rb;
  auto fetch = [&](Rows& rr, int j0) {
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int idx = tid + kThreads * it;
      const uint32_t off = (uint32_t)min(j0 + idx / NV, L - 1) * krow_b + (idx % NV) * 16u;
      rr.k[it] = *reinterpret_cast<const u32x4*>(kseg + off);
      rr.v[it] = *reinterpret_cast<const u32x4*>(vseg + off);
      rr.b[it] = *reinterpret_cast<const u32x4*>(band_src(xw + j0 + idx / NV, (idx % NV) * 16u));
    }
  };
  auto stash = [&](const Rows& rr, T* stg, int j0) {
    const u32x4* kr = rr.k;
    const u32x4* vr = rr.v;
    T* sk = stg;
    T* sv = stg + SK * KT;
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int idx = tid + kThreads * it;
      const int r = idx / NV;
      const int dv = (idx % NV) * VEC;
      *reinterpret_cast<u32x4*>(band_slot(xw + j0 + r) + st_col) = rr.b[it];
      // (k_swz and v_swz read no bit of r above bit 4: row r of a stage and row r % 32 of its
      // step share a permutation)
      if constexpr (kSwK<T>)
        *reinterpret_cast<u32x4*>(sk + r * kD + 8 * ((dv >> 3) ^ k_swz(r))) = kr[it];
      else
        *reinterpret_cast<u32x4*>(sk + r * KP + dv) = kr[it];
      if constexpr (kTrV<T>) {
        *reinterpret_cast<u32x4*>(sv + r * kD + 4 * ((dv >> 2) ^ v_swz(r))) = vr[it];
      } else {
        const T* e = reinterpret_cast<const T*>(&vr[it]);
#pragma unroll
        for (int c = 0; c < VEC; ++c) sv[(dv + c) * VP + r] = e[c];
      }
    }
  };

  // band tile (16 rows from x, this lane's row x + m16) from the ring. Every row a lane reads is
  // xl plus a multiple of 16, so its two chunk columns are fixed.
  const int xl = C0 - 16 * QT * wave + m16;   // + j0 + 16 m: this lane's row of T_m
  const int bsw = BSW ? xl & 7 : 0;
  const int bcol_lo = 8 * (grp ^ bsw), bcol_hi = 8 * ((grp + 4) ^ bsw);
  auto band_tile = [&](int x, F& p_lo, F& p_hi) {
    const T* row = band_slot(x);
    p_lo = load8(row + bcol_lo);
    p_hi = load8(row + bcol_hi);
  };
  // requests in the order they are needed: stage 0's rows and the window's first rows (staged
  // directly, once), then stage 1's rows, which the prologue's waits then leave in flight. Stage
  // 0's window is 16 QT kWaves + SK rows: its top SK come with stage 0's fetch, the NPRE chunks of
  // SK below them here.
  constexpr int NPRE = QT * kWaves * 16 / SK;
  static_assert(SK * NPRE == 16 * QT * kWaves, "the window below its top chunk is whole chunks");
  fetch(ra, J);
  u32x4 pre[NPRE][NLD];
#pragma unroll
  for (int part = 0; part < NPRE; ++part)
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int idx = tid + kThreads * it;
      const int x = xw + J - SK * (NPRE - part) + idx / NV;
      pre[part][it] = *reinterpret_cast<const u32x4*>(band_src(x, (idx % NV) * 16u));
    }
  __builtin_amdgcn_sched_barrier(0);
  fetch(rb, J + SK);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int part = 0; part < NPRE; ++part)
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int idx = tid + kThreads * it;
      const int x = xw + J - SK * (NPRE - part) + idx / NV;
      *reinterpret_cast<u32x4*>(band_slot(x) + st_col) = pre[part][it];
    }
  F qu[QT][2], qv[QT][2];
#pragma unroll
  for (int k = 0; k < QT; ++k)
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        set(qu[k][half], e, (get(qq[k][half], e) + get(uu[half], e)) * a.scale_log2);
        set(qv[k][half], e, (get(qq[k][half], e) + get(ww[half], e)) * a.scale_log2);
      }
  stash(ra, s_kv, J);
  __syncthreads();
  // carried band state: the first band product of each tile (tile k: over T_{QT-1-k}), and with
  // two tiles the fragments of T_1
  floatx4 g_prev[QT];
  F c1[2];
  {
    F p_lo, p_hi;
#pragma unroll
    for (int k = 0; k < QT; ++k) {
      band_tile(xl + J + 16 * (QT - 1 - k), p_lo, p_hi);
      g_prev[k] = mma(p_lo, qv[k][0], floatx4{0.f, 0.f, 0.f, 0.f});
      g_prev[k] = mma(p_hi, qv[k][1], g_prev[k]);
    }
    if constexpr (QT == 2) band_tile(xl + J + 16, c1[0], c1[1]);
  }
  // One 32-key step at key j0 whose K and V rows start at `kv` (a stage buffer plus the step's
  // offset in it). kM: the step masks keys (every step with the chunked_limited mask, else only a
  // last step that runs past the utterance). A wave's tiles past the utterance compute on
  // clamped, finite rows and are never stored.
  auto step = [&](int j0, const T* kv, auto masked) {
    constexpr bool kM = decltype(masked)::value;
    F kf[2][2], vf[4];
    if constexpr (kSwK<T>) {
      const int r = 8 * key_group<kPerm>(m16 >> 2) + (m16 & 3);   // tile tt reads row r + 4 tt
      const int sw = k_swz(r);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const T* row = kv + (r + 4 * tt) * kD;
        kf[tt][0] = load8(row + 8 * (grp ^ sw));
        kf[tt][1] = load8(row + 8 * ((grp + 4) ^ sw));
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const T* row = kv + (8 * key_group<kPerm>(m16 >> 2) + 4 * tt + (m16 & 3)) * KP + 8 * grp;
        kf[tt][0] = load8(row);
        kf[tt][1] = load8(row + 32);
      }
    }
    if constexpr (kTrV<T>) {
      // lane m16 of the group addresses row 8 kg + m16 / 4 (+ 4), dimensions 16 dt + 4 (m16 % 4)
      const int r = 8 * key_group<kPerm>(grp) + (m16 >> 2);
      const T* vlo = kv + SK * KT + r * kD;
      const int sw = v_swz(r);   // the same for row r + 4
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int c = 4 * (((4 * dt) + (m16 & 3)) ^ sw);
        vf[dt] = load8_tr(vlo + c, vlo + 4 * kD + c);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        vf[dt] = load8(kv + SK * KT + (16 * dt + m16) * VP + 8 * key_group<kPerm>(grp));
    }
    // the new band tiles T_2 .. T_{QT+1} (with one tile per wave: T_1 and T_2)
    F pb[QT + 1][2];
    if constexpr (QT == 2) {
      pb[0][0] = c1[0];
      pb[0][1] = c1[1];
    }
#pragma unroll
    for (int m = (QT == 2 ? 1 : 0); m < QT + 1; ++m)
      band_tile(xl + j0 + 16 * (m + 1), pb[m][0], pb[m][1]);
    int lo_k[QT], hi_k[QT];
#pragma unroll
    for (int k = 0; k < QT; ++k) {
      lo_k[k] = kLimited ? k_lo_q[k] - j0 : 0;
      hi_k[k] = kLimited ? k_hi_q[k] - j0 : L - j0;
    }
    step_tiles<T, QT, kM>(st, rr, kf, vf, qu, qv, pb, g_prev, s_g, lo_k, hi_k);
    if constexpr (QT == 2) {
      c1[0] = pb[QT][0];
      c1[1] = pb[QT][1];
    }
  };
  // one stage (index `stage` from the first visible key): registers `nxt` already hold stage + 1,
  // `fre` receives stage + 2; a wave with no query inside the utterance skips the arithmetic
  // (uniform over the wave). A masked stage runs only its steps before the last visible key.
  // (With one register set, the barrier that ended the previous stage also ended every read of
  // the buffer and ring slots the stash at the start fills.)
  const bool active = ntile > 0;
  auto do_stage = [&](int stage, Rows& nxt, Rows& fre, auto masked) {
    constexpr bool kM = decltype(masked)::value;
    const int j0 = J + SK * stage;
    const T* cur = s_kv + (stage & 1) * TILE;
    if constexpr (ONE) stash(nxt, s_kv + ((stage + 1) & 1) * TILE, j0 + SK);
    fetch(fre, j0 + 2 * SK);   // (past the last stage: harmless re-reads of the last frame)
    if (active) {
#pragma unroll
      for (int u = 0; u < SUBS; ++u) {
        if (!kM || u == 0 || SUBS * stage + u < nsteps) step(j0 + 32 * u, cur + 32 * u * kD, masked);
      }
    }
    // (unconditional, also after the last stage: the rows are clamped re-reads going to a buffer
    // and ring slots no later read uses, and every path back to the loop head then has the same
    // loads in flight - a path with one more pending load made the compiler drain them all at
    // the head, which cut the look-ahead to one stage)
    if constexpr (!ONE) stash(nxt, s_kv + ((stage + 1) & 1) * TILE, j0 + SK);
    __syncthreads();
  };
  // stages in pairs (the two register sets swap roles), an odd last stage after the loop: the
  // loop has one exit, so no path reaches its head with the other set's loads still pending.
  // Without the mask the stages that lie wholly inside the utterance run unmasked, and a last
  // partial stage, masked, after them.
  const std::integral_constant<bool, true> mask_on;
  const std::integral_constant<bool, false> mask_off;
  // stages whose steps need no mask (whole 32-key steps inside the utterance, SUBS to a stage)
  const int nplain = kLimited ? 0 : ((j_end - J) >> 5) / SUBS;
  const int nstages = (nsteps + SUBS - 1) / SUBS;
  int stage = 0;
  if constexpr (ONE) {
    // the first stage stashes the prologue's second set; every later one reuses ra
    if (nplain > 0) do_stage(0, rb, ra, mask_off);
    else do_stage(0, rb, ra, mask_on);
    for (stage = 1; stage < nplain; ++stage) do_stage(stage, ra, ra, mask_off);
    if (stage < nstages) do_stage(stage, ra, ra, mask_on);
  } else {
  for (; stage + 1 < nplain; stage += 2) {
    do_stage(stage, rb, ra, mask_off);
    do_stage(stage + 1, ra, rb, mask_off);
  }
  if (stage < nplain) {
    do_stage(stage, rb, ra, mask_off);
    ++stage;
  }
  if constexpr (kLimited) {
    for (; stage + 1 < nstages; stage += 2) {
      do_stage(stage, rb, ra, mask_on);
      do_stage(stage + 1, ra, rb, mask_on);
    }
  }
  if (stage < nstages) {
    if (stage & 1) do_stage(stage, ra, rb, mask_on);
    else do_stage(stage, rb, ra, mask_on);
  }
  }

  // finish: every tile of every wave owns its 16 queries
#pragma unroll
  for (int k = 0; k < QT; ++k) {
    const float l = st[k].ls[0];
    const float inv = 1.f / l;
    const int i = q0 + 16 * k + m16;
    if (i < L) {
      T* dst = a.out + ((size_t)(lo + i) * a.H + h) * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[16 * dt + 4 * grp + e] = from_f<T>(st[k].o[dt][e] * inv);
    }
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
  const bool limited = p.mask_chunk > 0;
  const int qtile = limited ? kQTile<T, true> : kQTile<T, false>;
  a.qtiles = (p.max_seqlen + qtile - 1) / qtile;
  a.div_H = make_fastdiv(a.H);
  a.div_qtiles = make_fastdiv(a.qtiles);
  a.div_group = make_fastdiv(a.H / a.Hk);
  a.total = p.total;
  a.maxlen = p.max_seqlen;
  a.num_seqs = p.num_seqs;
  const float scale = p.softmax_scale > 0.f ? p.softmax_scale : 1.f / sqrtf((float)p.head_dim);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.chunk = p.mask_chunk;
  a.left = p.mask_left_chunks;
  const dim3 grid((unsigned)varlen_attn_grid((int)sizeof(T), p.num_seqs, p.n_head, p.max_seqlen,
                                             limited).workgroups);
  if (limited)
    hipLaunchKernelGGL((varlen_attn_kernel<T, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((varlen_attn_kernel<T, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

LaunchGrid varlen_attn_grid(int dtype_bytes, int num_seqs, int n_head, int max_seqlen,
                            bool limited) {
  const int qtile = dtype_bytes == 2 ? (limited ? kQTile<bf16, true> : kQTile<bf16, false>)
                                     : (limited ? kQTile<float, true> : kQTile<float, false>);
  return {mul_sat(mul_sat(num_seqs, n_head), ((int64_t)max_seqlen + qtile - 1) / qtile), kThreads};
}

hipError_t launch_varlen_attn(pkc_dtype dtype, const VarlenParams& p, hipStream_t stream) {
  return dtype == PKC_BF16 ? launch_varlen_t<bf16>(p, stream) : launch_varlen_t<float>(p, stream);
}

}  // namespace pkc
