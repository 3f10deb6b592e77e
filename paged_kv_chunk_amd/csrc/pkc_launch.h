// Host-side launch interface between the C ABI (api.hip) and the kernel files. Sizes have been
// validated by the caller; launchers only pick the instantiation and grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkc.h"

namespace pkc {

struct AppendParams {
  const void* k_new;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  const int32_t* block_tables;
  const int32_t* cache_seqlens;
  const int32_t* chunk_lens;   // real frames per stream, or null: all chunk frames
  const int32_t* window_start; // absolute position of each stream's first cached frame, or null
  int batch, chunk, n_kv_head, head_dim, block_size, num_blocks, max_blocks, max_cache;
};

struct AttnParams {
  const void* q;
  const void* k_pool;      // read
  const void* v_pool;      // read
  const int32_t* block_tables;
  const int32_t* cache_seqlens;
  const int32_t* chunk_lens;   // real frames per stream, or null: all chunk frames
  const int32_t* window_start; // absolute position of each stream's first cached frame, or null
  const void* pos;
  const void* pos_bias_u;
  const void* pos_bias_v;
  void* out;
  // fused append: when k_new is non-null the chunk's K/V come from k_new / v_new and are also
  // written into k_pool_w / v_pool_w (the same pools as k_pool / v_pool)
  const void* k_new;
  const void* v_new;
  void* k_pool_w;
  void* v_pool_w;
  int batch, chunk, n_head, n_kv_head, head_dim, block_size, num_blocks, max_blocks, max_cache;
  int pos_len, pos_layout;
  float softmax_scale;
};

struct VarlenParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_seqlens;
  const void* pos;
  const void* pos_bias_u;
  const void* pos_bias_v;
  void* out;
  int num_seqs, total, max_seqlen, n_head, n_kv_head, head_dim;
  int mask_chunk, mask_left_chunks;   // chunked_limited mask, or mask_chunk = 0: full context
  float softmax_scale;
};

// The GEMMs either side of the attention (gemm.hip): y[M, N] = x[M, K] w[N, K]^T (+ bias)
struct GemmParams {
  const void* x;
  const void* w;
  const void* bias;   // [N] or null
  void* y;
  int M, N, K;
};

// The chunk's fused Q/K/V projection, appending K/V into the pages as its epilogue
struct QkvParams {
  const void* x;      // [B, C, d_model]
  const void* w;      // [(H + 2 Hk) D, d_model]: rows of linear_q, linear_k, linear_v
  const void* bias;   // [(H + 2 Hk) D] or null
  void* q_out;        // [B, C, H, D]
  void* k_pool;
  void* v_pool;
  const int32_t* block_tables;
  const int32_t* cache_seqlens;
  const int32_t* chunk_lens;
  const int32_t* window_start;
  int batch, chunk, d_model, n_head, n_kv_head, head_dim, block_size, num_blocks, max_blocks,
      max_cache;
};

// linear_pos over sinusoidal tables generated in the kernel
struct PosProjParams {
  const void* w;              // [out_features, d_model]
  void* out;                  // [n_tables, rows, out_features]
  const int32_t* pos_start;   // [n_tables] or null: pos_first for every table
  int pos_first, pos_step, n_tables, rows, d_model, out_features;
};

// The memory-path ceiling of a fused launch (gather_read.hip): the same bytes, no arithmetic
struct GatherParams {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  const int32_t* block_tables;
  const int32_t* cache_seqlens;
  const void* pos;
  const void* pos_bias_u;
  const void* pos_bias_v;
  void* out;
  int batch, chunk, n_head, n_kv_head, block_size, num_blocks, max_blocks, max_cache;
  int pos_len, pos_layout, waves, split, reads;
};

hipError_t launch_paged_append(pkc_dtype dtype, const AppendParams& p, hipStream_t stream);
hipError_t launch_linear(pkc_dtype dtype, const GemmParams& p, hipStream_t stream);
hipError_t launch_qkv_append(pkc_dtype dtype, const QkvParams& p, hipStream_t stream);
hipError_t launch_pos_projection(pkc_dtype dtype, const PosProjParams& p, hipStream_t stream);
hipError_t launch_commit(int32_t* cache_seqlens, const int32_t* chunk_lens, int32_t* window_start,
                         int max_cached, int block_size, int batch, int chunk, hipStream_t stream);
hipError_t launch_chunk_attn(pkc_dtype dtype, const AttnParams& p, hipStream_t stream);
hipError_t launch_varlen_attn(pkc_dtype dtype, const VarlenParams& p, hipStream_t stream);
hipError_t launch_gather_read(const GatherParams& p, hipStream_t stream);


// Dynamic LDS of one chunk-attention workgroup, and the budget it must fit (the launcher opts in
// above the default 64 KiB).
size_t chunk_attn_lds_bytes(int dtype_bytes, int chunk, int max_cache, int block_size, bool fused);
constexpr size_t kMaxDynamicLds = 160 * 1024;
// Dynamic LDS of one append workgroup (staged frames x head_dim); at most the default 64 KiB.
size_t paged_append_lds_bytes(int dtype_bytes, int head_dim);
constexpr size_t kDefaultDynamicLds = 64 * 1024;

// Product of non-negative sizes, saturating at 2^62 (no int64 overflow for any int32 inputs).
inline int64_t mul_sat(int64_t a, int64_t b) {
  constexpr int64_t kCap = (int64_t)1 << 62;
  if (a <= 0 || b <= 0) return 0;
  return a > kCap / b ? kCap : a * b;
}

// Geometry of one launch: workgroups along x and threads per workgroup. HIP launches fewer than
// 2^32 work-items along a grid dimension (the dispatch packet's grid size is 32-bit), which also
// keeps the workgroup index below 2^31 for the kernels' multiply-shift divisions. The launchers
// take their grid from these functions, and the entry points refuse a launch that does not fit.
struct LaunchGrid {
  int64_t workgroups;
  int threads;
  bool fits() const { return workgroups <= ((((int64_t)1) << 32) - 1) / threads; }
};
LaunchGrid paged_append_grid(int batch, int n_kv_head);
LaunchGrid commit_grid(int batch);
LaunchGrid chunk_attn_grid(int dtype_bytes, int batch, int n_head, int chunk);
LaunchGrid varlen_attn_grid(int dtype_bytes, int num_seqs, int n_head, int max_seqlen,
                            bool limited);   // with the chunked_limited mask
LaunchGrid gather_read_grid(int batch, int n_head, int split, int waves);
// compute units of the current device, 0 if the query fails
int device_cus();
LaunchGrid gemm_grid(int64_t M, int64_t N);   // the tile shape the GEMM launchers pick for M x N

}  // namespace pkc
