// C ABI of libpkc.so: host-side validation, then one launch on the caller's stream.
// Validation never touches the GPU, so every error path returns before any HIP call.
#include <stdint.h>

#include "pkc.h"
#include "pkc_launch.h"

using namespace pkc;

namespace {

constexpr int kVersion = 400;  // 0.4.0: the projections either side of the attention

constexpr int32_t kMaxPosRows = (int32_t)1 << 25;   // rows of one positional table

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pkc_status check_dtype(pkc_dtype dtype) {
  return (dtype == PKC_F32 || dtype == PKC_BF16) ? PKC_OK : PKC_ERR_DTYPE;
}

// Checks shared by the append and the attention: pool geometry and capacity.
pkc_status check_pool(int32_t batch, int32_t chunk, int32_t n_kv_head, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_blocks,
                      int32_t max_cache) {
  if (batch <= 0 || chunk <= 0 || n_kv_head <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || max_blocks <= 0 || max_cache < 0)
    return PKC_ERR_SHAPE;
  if (head_dim % 8 != 0) return PKC_ERR_SHAPE;
  if (head_dim % 32 != 0) return PKC_ERR_UNSUPPORTED;   // K pages are in 32-dim column blocks
  if ((int64_t)max_cache + chunk > (int64_t)max_blocks * block_size) return PKC_ERR_CAPACITY;
  // every index below fits in int32 arithmetic inside the kernels except the flat offsets,
  // which the kernels form in size_t
  if ((int64_t)max_cache + chunk >= (int64_t)1 << 30) return PKC_ERR_SHAPE;
  return PKC_OK;
}

pkc_status check_attn(int32_t chunk, int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                      int32_t block_size, int32_t max_cache, int32_t pos_len, int32_t pos_layout) {
  if (n_head <= 0 || n_head % n_kv_head != 0) return PKC_ERR_SHAPE;
  if (pos_layout < 0 || pos_layout > (PKC_POS_PER_ROW | PKC_POS_PER_KEY | PKC_POS_COL_BLOCKED))
    return PKC_ERR_SHAPE;
  const int64_t longest = (int64_t)max_cache + chunk;
  if (pos_layout & PKC_POS_PER_KEY) {
    // one row per key, shared or per stream
    if (pos_len < longest) return PKC_ERR_SHAPE;
  } else if (pos_layout & PKC_POS_PER_ROW) {
    if (pos_len < 2 * longest - 1) return PKC_ERR_SHAPE;
  } else {
    if (pos_len <= 0 || pos_len % 2 != 1) return PKC_ERR_SHAPE;
    if ((pos_len - 1) / 2 < longest - 1) return PKC_ERR_SHAPE;
  }
  if (head_dim != 64) return PKC_ERR_UNSUPPORTED;
  if (block_size < 8 || (block_size & (block_size - 1)) != 0) return PKC_ERR_UNSUPPORTED;
  // the kernels step through one head's column-blocked table with 32-bit strides of 64 rows
  if (pos_len >= kMaxPosRows) return PKC_ERR_UNSUPPORTED;
  return PKC_OK;
}

pkc_status from_hip(hipError_t e) { return e == hipSuccess ? PKC_OK : PKC_ERR_HIP; }

// GEMM shapes the kernel is built for: whole 32-deep contraction stages, 16-feature output tiles,
// and a tile grid one launch holds
pkc_status check_gemm(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return PKC_ERR_SHAPE;
  if (M >= ((int64_t)1 << 30) || N >= ((int64_t)1 << 30) || K >= ((int64_t)1 << 30)) return PKC_ERR_SHAPE;
  if (K % 32 != 0 || N % 16 != 0) return PKC_ERR_UNSUPPORTED;
  if (!gemm_grid(M, N).fits()) return PKC_ERR_UNSUPPORTED;
  return PKC_OK;
}

}  // namespace

extern "C" {

int pkc_version(void) { return kVersion; }

const char* pkc_status_string(int status) {
  switch (status) {
    case PKC_OK: return "ok";
    case PKC_ERR_NULL: return "a required pointer is NULL";
    case PKC_ERR_SHAPE: return "a size is out of range or sizes disagree";
    case PKC_ERR_DTYPE: return "unknown element type";
    case PKC_ERR_UNSUPPORTED: return "configuration not supported by the built kernels";
    case PKC_ERR_CAPACITY: return "max_cache_seqlen + chunk_size exceeds max_blocks_per_seq * block_size";
    case PKC_ERR_HIP: return "HIP runtime error at launch";
    case PKC_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    default: return "unknown status";
  }
}

pkc_status paged_kv_append(pkc_dtype dtype, const void* k_new, const void* v_new, void* k_pool,
                           void* v_pool, const int32_t* block_tables, const int32_t* cache_seqlens,
                           const int32_t* chunk_lens, const int32_t* window_start, int32_t batch,
                           int32_t chunk_size, int32_t n_kv_head, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_cache_seqlen, hipStream_t stream) {
  pkc_status st = check_dtype(dtype);
  if (st != PKC_OK) return st;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !cache_seqlens) return PKC_ERR_NULL;
  st = check_pool(batch, chunk_size, n_kv_head, head_dim, block_size, num_blocks,
                  max_blocks_per_seq, max_cache_seqlen);
  if (st != PKC_OK) return st;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return PKC_ERR_ALIGN;
  if (!paged_append_grid(batch, n_kv_head).fits() ||
      paged_append_lds_bytes(dtype == PKC_BF16 ? 2 : 4, head_dim) > kDefaultDynamicLds)
    return PKC_ERR_UNSUPPORTED;
  AppendParams p{k_new, v_new, k_pool, v_pool, block_tables, cache_seqlens, chunk_lens,
                 window_start, batch, chunk_size,
                 n_kv_head, head_dim, block_size, num_blocks, max_blocks_per_seq, max_cache_seqlen};
  return from_hip(launch_paged_append(dtype, p, stream));
}

static pkc_status attn_common(pkc_dtype dtype, const void* q, const void* k_new, const void* v_new,
                              const void* k_pool, const void* v_pool, void* k_pool_w,
                              void* v_pool_w, const int32_t* block_tables,
                              const int32_t* cache_seqlens, const int32_t* chunk_lens,
                              const int32_t* window_start, const void* pos, int32_t pos_len,
                              int32_t pos_layout, const void* pos_bias_u, const void* pos_bias_v,
                              void* out, int32_t batch, int32_t chunk_size, int32_t n_head,
                              int32_t n_kv_head, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t max_cache_seqlen, float softmax_scale, hipStream_t stream,
                              bool launch = true) {
  pkc_status st = check_dtype(dtype);
  if (st != PKC_OK) return st;
  if (!q || !k_pool || !v_pool || !block_tables || !cache_seqlens || !pos || !pos_bias_u ||
      !pos_bias_v || !out)
    return PKC_ERR_NULL;
  st = check_pool(batch, chunk_size, n_kv_head, head_dim, block_size, num_blocks,
                  max_blocks_per_seq, max_cache_seqlen);
  if (st != PKC_OK) return st;
  st = check_attn(chunk_size, n_head, n_kv_head, head_dim, block_size, max_cache_seqlen, pos_len,
                  pos_layout);
  if (st != PKC_OK) return st;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(pos) ||
      !aligned16(pos_bias_u) || !aligned16(pos_bias_v) || !aligned16(out))
    return PKC_ERR_ALIGN;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return PKC_ERR_ALIGN;
  if (chunk_attn_lds_bytes(dtype == PKC_BF16 ? 2 : 4, chunk_size, max_cache_seqlen, block_size,
                           k_new != nullptr) > kMaxDynamicLds)
    return PKC_ERR_UNSUPPORTED;
  if (!chunk_attn_grid(dtype == PKC_BF16 ? 2 : 4, batch, n_head, chunk_size).fits())
    return PKC_ERR_UNSUPPORTED;
  AttnParams p{};
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.block_tables = block_tables;
  p.cache_seqlens = cache_seqlens;
  p.chunk_lens = chunk_lens;
  p.window_start = window_start;
  p.pos = pos;
  p.pos_bias_u = pos_bias_u;
  p.pos_bias_v = pos_bias_v;
  p.out = out;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_pool_w = k_pool_w;
  p.v_pool_w = v_pool_w;
  p.batch = batch;
  p.chunk = chunk_size;
  p.n_head = n_head;
  p.n_kv_head = n_kv_head;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.max_cache = max_cache_seqlen;
  p.pos_len = pos_len;
  p.pos_layout = pos_layout;
  p.softmax_scale = softmax_scale;
  if (!launch) return PKC_OK;
  return from_hip(launch_chunk_attn(dtype, p, stream));
}

pkc_status chunk_paged_relpos_attn(pkc_dtype dtype, const void* q, const void* k_pool,
                                   const void* v_pool, const int32_t* block_tables,
                                   const int32_t* cache_seqlens, const int32_t* chunk_lens,
                                   const int32_t* window_start, const void* pos, int32_t pos_len,
                                   int32_t pos_layout, const void* pos_bias_u,
                                   const void* pos_bias_v, void* out, int32_t batch,
                                   int32_t chunk_size, int32_t n_head, int32_t n_kv_head,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_cache_seqlen,
                                   float softmax_scale, hipStream_t stream) {
  return attn_common(dtype, q, nullptr, nullptr, k_pool, v_pool, nullptr, nullptr, block_tables,
                     cache_seqlens, chunk_lens, window_start, pos, pos_len, pos_layout, pos_bias_u,
                     pos_bias_v, out, batch,
                     chunk_size, n_head, n_kv_head, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_cache_seqlen, softmax_scale, stream);
}

pkc_status paged_kv_append_relpos_attn(pkc_dtype dtype, const void* q, const void* k_new,
                                       const void* v_new, void* k_pool, void* v_pool,
                                       const int32_t* block_tables, const int32_t* cache_seqlens,
                                       const int32_t* chunk_lens, const int32_t* window_start,
                                       const void* pos, int32_t pos_len, int32_t pos_layout,
                                       const void* pos_bias_u, const void* pos_bias_v, void* out,
                                       int32_t batch, int32_t chunk_size, int32_t n_head,
                                       int32_t n_kv_head, int32_t head_dim, int32_t block_size,
                                       int32_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t max_cache_seqlen, float softmax_scale,
                                       hipStream_t stream) {
  if (!k_new || !v_new) return PKC_ERR_NULL;
  return attn_common(dtype, q, k_new, v_new, k_pool, v_pool, k_pool, v_pool, block_tables,
                     cache_seqlens, chunk_lens, window_start, pos, pos_len, pos_layout, pos_bias_u,
                     pos_bias_v, out, batch,
                     chunk_size, n_head, n_kv_head, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_cache_seqlen, softmax_scale, stream);
}

pkc_status paged_kv_append_relpos_attn_layers(
    pkc_dtype dtype, int32_t n_layers, const void* const* q, const void* const* k_new,
    const void* const* v_new, void* const* k_pool, void* const* v_pool,
    const int32_t* block_tables, const int32_t* cache_seqlens, const int32_t* chunk_lens,
    const int32_t* window_start, const void* const* pos, int32_t pos_len, int32_t pos_layout,
    const void* const* pos_bias_u,
    const void* const* pos_bias_v, void* const* out, int32_t batch, int32_t chunk_size,
    int32_t n_head, int32_t n_kv_head, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_cache_seqlen, float softmax_scale, hipStream_t stream) {
  pkc_status st = check_dtype(dtype);
  if (st != PKC_OK) return st;
  if (n_layers <= 0) return PKC_ERR_SHAPE;
  if (!q || !k_new || !v_new || !k_pool || !v_pool || !pos || !pos_bias_u || !pos_bias_v || !out)
    return PKC_ERR_NULL;
  // every layer is validated before any is launched, so an error launches nothing
  for (int pass = 0; pass < 2; ++pass) {
    for (int l = 0; l < n_layers; ++l) {
      if (!k_new[l] || !v_new[l]) return PKC_ERR_NULL;
      st = attn_common(dtype, q[l], k_new[l], v_new[l], k_pool[l], v_pool[l], k_pool[l],
                       v_pool[l], block_tables, cache_seqlens, chunk_lens, window_start, pos[l],
                       pos_len,
                       pos_layout, pos_bias_u[l], pos_bias_v[l], out[l], batch, chunk_size,
                       n_head, n_kv_head, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_cache_seqlen, softmax_scale, stream, pass == 1);
      if (st != PKC_OK) return st;
    }
  }
  return PKC_OK;
}

pkc_status pkc_gather_read(pkc_dtype dtype, const void* q, const void* k_new, const void* v_new,
                           void* k_pool, void* v_pool, const int32_t* block_tables,
                           const int32_t* cache_seqlens, const void* pos, int32_t pos_len,
                           int32_t pos_layout, const void* pos_bias_u, const void* pos_bias_v,
                           void* out, int32_t batch, int32_t chunk_size, int32_t n_head,
                           int32_t n_kv_head, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_cache_seqlen, int32_t waves, int32_t split,
                           int32_t reads, hipStream_t stream) {
  if (!k_new || !v_new) return PKC_ERR_NULL;
  pkc_status st = attn_common(dtype, q, k_new, v_new, k_pool, v_pool, k_pool, v_pool,
                              block_tables, cache_seqlens, nullptr, nullptr, pos, pos_len,
                              pos_layout, pos_bias_u, pos_bias_v, out, batch, chunk_size, n_head,
                              n_kv_head, head_dim, block_size, num_blocks, max_blocks_per_seq,
                              max_cache_seqlen, 0.f, stream, false);
  if (st != PKC_OK) return st;
  if ((waves != 1 && waves != 4 && waves != 8) || (split != 1 && split != 2 && split != 4) ||
      (reads != 0 && reads != 1))
    return PKC_ERR_SHAPE;
  if (dtype != PKC_BF16 || chunk_size > 16 || (pos_layout & PKC_POS_PER_KEY))
    return PKC_ERR_UNSUPPORTED;
  if (!gather_read_grid(batch, n_head, split, waves).fits()) return PKC_ERR_UNSUPPORTED;
  GatherParams p{q, k_new, v_new, k_pool, v_pool, block_tables, cache_seqlens, pos, pos_bias_u,
                 pos_bias_v, out, batch, chunk_size, n_head, n_kv_head, block_size, num_blocks,
                 max_blocks_per_seq, max_cache_seqlen, pos_len, pos_layout, waves, split, reads};
  return from_hip(launch_gather_read(p, stream));
}

pkc_status paged_kv_commit(int32_t* cache_seqlens, const int32_t* chunk_lens,
                           int32_t* window_start, int32_t max_cached_frames, int32_t batch,
                           int32_t chunk_size, int32_t block_size, hipStream_t stream) {
  if (!cache_seqlens) return PKC_ERR_NULL;
  if (batch <= 0 || chunk_size <= 0) return PKC_ERR_SHAPE;
  if (window_start && (block_size <= 0 || max_cached_frames < 0)) return PKC_ERR_SHAPE;
  if (!commit_grid(batch).fits()) return PKC_ERR_UNSUPPORTED;
  return from_hip(launch_commit(cache_seqlens, chunk_lens, window_start, max_cached_frames,
                                block_size, batch, chunk_size, stream));
}

pkc_status varlen_packed_relpos_attn(pkc_dtype dtype, const void* q, const void* k, const void* v,
                                     const int32_t* cu_seqlens, int32_t num_seqs,
                                     int32_t total_frames, int32_t max_seqlen, const void* pos,
                                     const void* pos_bias_u, const void* pos_bias_v, void* out,
                                     int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                                     int32_t mask_chunk, int32_t mask_left_chunks,
                                     float softmax_scale, hipStream_t stream) {
  pkc_status st = check_dtype(dtype);
  if (st != PKC_OK) return st;
  if (!q || !k || !v || !cu_seqlens || !pos || !pos_bias_u || !pos_bias_v || !out)
    return PKC_ERR_NULL;
  if (num_seqs <= 0 || total_frames < 0 || max_seqlen < 0 || n_head <= 0 || n_kv_head <= 0 ||
      n_head % n_kv_head != 0 || head_dim <= 0 || head_dim % 8 != 0)
    return PKC_ERR_SHAPE;
  if ((int64_t)total_frames >= (int64_t)1 << 29 || (int64_t)max_seqlen > total_frames)
    return PKC_ERR_SHAPE;
  if (mask_chunk < 0 || mask_left_chunks < 0) return PKC_ERR_SHAPE;
  if (head_dim != 64) return PKC_ERR_UNSUPPORTED;
  // (the kernel addresses an utterance's rows by 32-bit byte offsets from its first row; its
  // table spans 2 max_seqlen rows)
  if (mul_sat(mul_sat((int64_t)2 * max_seqlen, n_head > n_kv_head ? n_head : n_kv_head),
              (int64_t)head_dim * (dtype == PKC_BF16 ? 2 : 4)) >= (int64_t)1 << 31)
    return PKC_ERR_UNSUPPORTED;
  if (!varlen_attn_grid(dtype == PKC_BF16 ? 2 : 4, num_seqs, n_head, max_seqlen, mask_chunk > 0)
           .fits())
    return PKC_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(pos) ||
      !aligned16(pos_bias_u) || !aligned16(pos_bias_v) || !aligned16(out))
    return PKC_ERR_ALIGN;
  if (total_frames == 0 || max_seqlen == 0) return PKC_OK;
  VarlenParams p{q, k, v, cu_seqlens, pos, pos_bias_u, pos_bias_v, out, num_seqs, total_frames,
                 max_seqlen, n_head, n_kv_head, head_dim, mask_chunk, mask_left_chunks,
                 softmax_scale};
  return from_hip(launch_varlen_attn(dtype, p, stream));
}


pkc_status pkc_linear(pkc_dtype dtype, const void* x, const void* w, const void* bias, void* y,
                      int32_t M, int32_t N, int32_t K, hipStream_t stream) {
  pkc_status st = check_dtype(dtype);
  if (st != PKC_OK) return st;
  if (!x || !w || !y) return PKC_ERR_NULL;
  st = check_gemm(M, N, K);
  if (st != PKC_OK) return st;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (bias && !aligned16(bias))) return PKC_ERR_ALIGN;
  GemmParams p{x, w, bias, y, M, N, K};
  return from_hip(launch_linear(dtype, p, stream));
}

pkc_status paged_kv_qkv_append(pkc_dtype dtype, const void* x, const void* w_qkv,
                               const void* b_qkv, void* q_out, void* k_pool, void* v_pool,
                               const int32_t* block_tables, const int32_t* cache_seqlens,
                               const int32_t* chunk_lens, const int32_t* window_start,
                               int32_t batch, int32_t chunk_size, int32_t d_model, int32_t n_head,
                               int32_t n_kv_head, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_cache_seqlen, hipStream_t stream) {
  pkc_status st = check_dtype(dtype);
  if (st != PKC_OK) return st;
  if (!x || !w_qkv || !q_out || !k_pool || !v_pool || !block_tables || !cache_seqlens)
    return PKC_ERR_NULL;
  st = check_pool(batch, chunk_size, n_kv_head, head_dim, block_size, num_blocks,
                  max_blocks_per_seq, max_cache_seqlen);
  if (st != PKC_OK) return st;
  if (n_head <= 0 || n_head % n_kv_head != 0) return PKC_ERR_SHAPE;
  st = check_gemm((int64_t)batch * chunk_size, ((int64_t)n_head + 2 * (int64_t)n_kv_head) * head_dim,
                  d_model);
  if (st != PKC_OK) return st;
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(q_out) || !aligned16(k_pool) ||
      !aligned16(v_pool) || (b_qkv && !aligned16(b_qkv)))
    return PKC_ERR_ALIGN;
  QkvParams p{x, w_qkv, b_qkv, q_out, k_pool, v_pool, block_tables, cache_seqlens, chunk_lens,
              window_start, batch, chunk_size, d_model, n_head, n_kv_head, head_dim, block_size,
              num_blocks, max_blocks_per_seq, max_cache_seqlen};
  return from_hip(launch_qkv_append(dtype, p, stream));
}

pkc_status rel_pos_projection(pkc_dtype dtype, const void* w_pos, const int32_t* pos_start,
                              int32_t pos_first, int32_t pos_step, int32_t n_tables, int32_t rows,
                              int32_t d_model, int32_t out_features, void* pos_out,
                              hipStream_t stream) {
  pkc_status st = check_dtype(dtype);
  if (st != PKC_OK) return st;
  if (!w_pos || !pos_out) return PKC_ERR_NULL;
  if (n_tables <= 0 || rows <= 0) return PKC_ERR_SHAPE;
  st = check_gemm((int64_t)n_tables * rows, out_features, d_model);
  if (st != PKC_OK) return st;
  // positions stay within +-2^24, the range the kernel's phase accuracy is stated for
  const int64_t last = (int64_t)pos_first + (int64_t)pos_step * (rows - 1);
  const int64_t span = (int64_t)1 << 24;
  if (!pos_start && (pos_first > span || pos_first < -span || last > span || last < -span))
    return PKC_ERR_SHAPE;
  if ((int64_t)pos_step * (rows - 1) > span || (int64_t)pos_step * (rows - 1) < -span) return PKC_ERR_SHAPE;
  if (!aligned16(w_pos) || !aligned16(pos_out)) return PKC_ERR_ALIGN;
  PosProjParams p{w_pos, pos_out, pos_start, pos_first, pos_step, n_tables, rows, d_model,
                  out_features};
  return from_hip(launch_pos_projection(dtype, p, stream));
}

}  // extern "C"
