// Paged K/V append: each stream's chunk K/V into the pages its block table names.
//
// Source: OASR docs, "ASR Engine", section 4.3 "Batched paged forward" -- one pool shared by the
// cohort, one block-table row per stream, the chunk written at logical frames
// [cache_seqlens[b], cache_seqlens[b] + C), cache_seqlens advanced only after the forward; step 6
// commits each stream's actual frames, so with per-stream chunk lengths n_b only the first n_b
// frames are written (a padding lane, n_b = 0, writes nothing; section 9). With bounded history
// (sections 6 and 9) a stream's frames are addressed by absolute position p = window_start + t
// through its table row used as a ring: block block_tables[b][(p / S) % M], slot p % S.
//
// One workgroup per (stream, kv head). K rows are copied 16 bytes per lane straight into their
// slots (K pages are stored in 32-dim column blocks, [head_dim / 32][block_size][32]). V pages are stored transposed ([head_dim][block_size])
// so that attention can read 8 consecutive frames of one dimension with one 16-byte load; the
// workgroup therefore stages the chunk's V rows in LDS and writes each dimension's run of frames,
// consecutive lanes writing consecutive slots.
#include "pkc_device.h"
#include "pkc_launch.h"

namespace pkc {

namespace {

constexpr int kThreads = 256;
constexpr int kTileFrames = 64;  // frames staged per LDS round

template <typename T>
__global__ void __launch_bounds__(kThreads)
paged_append_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new, T* __restrict__ k_pool,
                    T* __restrict__ v_pool, const int32_t* __restrict__ block_tables,
                    const int32_t* __restrict__ cache_seqlens, const int32_t* __restrict__ chunk_lens,
                    const int32_t* __restrict__ window_start, int chunk, int n_kv_head, int head_dim,
                    int block_size, int num_blocks, int max_blocks, int max_cache) {
  extern __shared__ unsigned char smem_raw[];
  T* sv = reinterpret_cast<T*>(smem_raw);  // [kTileFrames][head_dim + pad]
  constexpr int VEC = 16 / sizeof(T);
  const int pitch = head_dim + VEC;         // keeps 16-byte alignment, shifts banks per frame

  const int b = blockIdx.x / n_kv_head;
  const int g = blockIdx.x % n_kv_head;
  // absolute position of the chunk's first frame; the window start is a whole number of blocks
  const int start = window_start ? max(window_start[b], 0) / block_size * block_size : 0;
  const int cache = start + clampi(cache_seqlens[b], 0, max_cache);
  const int32_t* bt = block_tables + (size_t)b * max_blocks;
  const int nvec = head_dim / VEC;
  const int n_real = chunk_lens ? clampi(chunk_lens[b], 0, chunk) : chunk;

  for (int t0 = 0; t0 < n_real; t0 += kTileFrames) {
    const int nt = min(kTileFrames, n_real - t0);
    // K: direct copy; V: stage rows in LDS.
    for (int x = threadIdx.x; x < nt * nvec; x += kThreads) {
      const int t = t0 + x / nvec;
      const int dv = (x % nvec) * VEC;
      const int frame = cache + t;
      const int blk = clampi(bt[(frame / block_size) % max_blocks], 0, num_blocks - 1);
      const int slot = frame % block_size;
      const size_t src = (((size_t)b * chunk + t) * n_kv_head + g) * head_dim + dv;
      const uint4 kv = *reinterpret_cast<const uint4*>(k_new + src);
      // K pages in 32-dim column blocks: dim d of slot s at ((d / 32) S + s) 32 + d % 32
      *reinterpret_cast<uint4*>(k_pool + ((size_t)blk * n_kv_head + g) * block_size * head_dim +
                                ((dv >> 5) * block_size + slot) * 32 + (dv & 31)) = kv;
      *reinterpret_cast<uint4*>(sv + (x / nvec) * pitch + dv) = *reinterpret_cast<const uint4*>(v_new + src);
    }
    __syncthreads();
    // V: for each dimension, the run of frames goes to consecutive slots of the transposed page.
    for (int x = threadIdx.x; x < nt * head_dim; x += kThreads) {
      const int d = x / nt;
      const int tl = x % nt;
      const int frame = cache + t0 + tl;
      const int blk = clampi(bt[(frame / block_size) % max_blocks], 0, num_blocks - 1);
      const int slot = frame % block_size;
      v_pool[(((size_t)blk * n_kv_head + g) * head_dim + d) * block_size + slot] = sv[tl * pitch + d];
    }
    __syncthreads();
  }
}

// cache_seqlens[b] += real frames of stream b ("ASR Engine", section 4.3 step 6,
// commit_chunk_paged), on the device so that a captured step needs no host round trip. With a
// window start and a cap (bounded history, sections 6 and 9), whole oldest blocks are then
// dropped while the cache exceeds the cap.
__global__ void __launch_bounds__(kThreads)
commit_kernel(int32_t* __restrict__ cache_seqlens, const int32_t* __restrict__ chunk_lens,
              int32_t* __restrict__ window_start, int max_cached, int block_size, int batch,
              int chunk) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= batch) return;
  int cache = cache_seqlens[b] + (chunk_lens ? clampi(chunk_lens[b], 0, chunk) : chunk);
  if (window_start && cache > max_cached) {
    // only whole filled blocks leave: the next chunk is written right after the cached frames,
    // so a partly filled block stays (with a cap below one block, cache then stays above it)
    const int drop = min((cache - max_cached + block_size - 1) / block_size, max(cache, 0) / block_size);
    window_start[b] += drop * block_size;
    cache -= drop * block_size;
  }
  cache_seqlens[b] = max(cache, 0);
}

}  // namespace

LaunchGrid commit_grid(int batch) { return {((int64_t)batch + kThreads - 1) / kThreads, kThreads}; }

LaunchGrid paged_append_grid(int batch, int n_kv_head) {
  return {mul_sat(batch, n_kv_head), kThreads};
}

size_t paged_append_lds_bytes(int dtype_bytes, int head_dim) {
  return (size_t)kTileFrames * ((size_t)head_dim + 16 / dtype_bytes) * dtype_bytes;
}

hipError_t launch_commit(int32_t* cache_seqlens, const int32_t* chunk_lens, int32_t* window_start,
                         int max_cached, int block_size, int batch, int chunk, hipStream_t stream) {
  const LaunchGrid g = commit_grid(batch);
  hipLaunchKernelGGL(commit_kernel, dim3((unsigned)g.workgroups), dim3(g.threads), 0, stream,
                     cache_seqlens, chunk_lens, window_start, max_cached, block_size, batch, chunk);
  return hipGetLastError();
}

hipError_t launch_paged_append(pkc_dtype dtype, const AppendParams& p, hipStream_t stream) {
  const LaunchGrid g = paged_append_grid(p.batch, p.n_kv_head);
  const dim3 grid((unsigned)g.workgroups), block(g.threads);
  const size_t smem = paged_append_lds_bytes(dtype == PKC_BF16 ? 2 : 4, p.head_dim);
  if (dtype == PKC_BF16) {
    hipLaunchKernelGGL(paged_append_kernel<bf16>, grid, block, smem, stream,
                       (const bf16*)p.k_new, (const bf16*)p.v_new, (bf16*)p.k_pool, (bf16*)p.v_pool,
                       p.block_tables, p.cache_seqlens, p.chunk_lens, p.window_start, p.chunk,
                       p.n_kv_head, p.head_dim,
                       p.block_size, p.num_blocks, p.max_blocks, p.max_cache);
  } else {
    hipLaunchKernelGGL(paged_append_kernel<float>, grid, block, smem, stream,
                       (const float*)p.k_new, (const float*)p.v_new, (float*)p.k_pool,
                       (float*)p.v_pool, p.block_tables, p.cache_seqlens, p.chunk_lens,
                       p.window_start, p.chunk,
                       p.n_kv_head, p.head_dim, p.block_size, p.num_blocks, p.max_blocks, p.max_cache);
  }
  return hipGetLastError();
}

}  // namespace pkc
