/*
 * pkc.h - paged chunk attention with a Transformer-XL relative-position term, for AMD gfx950.
 *
 * C ABI of libpkc.so. Every entry point takes plain device pointers and sizes, validates them on
 * the host before launching anything, enqueues its kernels on the caller's HIP stream and returns
 * without synchronising. The library allocates no device memory and keeps no state between calls;
 * all buffers belong to the caller. Calls on different streams are independent.
 *
 * Sources (OASR documentation pages, cited by title and section):
 *   [ENG 4.3]  "ASR Engine", section 4.3 "Batched paged forward": a cohort of streams shares one
 *              block pool; each stream has a row of block_tables (B, blocks_per_seq) and an entry
 *              of cache_seqlens (B,); the chunk's K/V land in the stream's pages; cache_seqlens is
 *              advanced (commit_chunk_paged) only after the forward.
 *   [ENG 6]    "ASR Engine", section 6 "Paged KV cache" options: block_size_frames,
 *              max_blocks_per_seq; section 8: pool exhaustion is an error, not silent.
 *   [SCH 4.3]  "Scheduler", section 4.3 "Heterogeneous-offset batching": attention over the
 *              paged pool with per-stream lengths from cache_seqlens and the relative-position
 *              bias matrix_bd / sqrt(d_k) added to the scores.
 *   [MOD fix]  "Model Layer", "Three optional encoder declarations", fixed_attention_window: the
 *              Transformer-XL row used for chunk query i and key j is picked by their offset,
 *              cache + i - j frames; one table can serve the cohort when every stream has the
 *              same cache_seqlens, and each stream needs its own table when they differ.
 *   [MOD surf] "Model Layer", "The engine-facing surface": forward_chunk_paged (streaming chunk
 *              entry), forward_offline_packed (gapless varlen offline forward), n_kv_head and
 *              head_dim (paged-streaming geometry).
 *   [MOD nem]  "Model Layer", the Nemotron encoder notes: Transformer-XL relative position uses
 *              rel_shift while WeNet's convention needs no shift; the chunked_limited mask lets
 *              a query see its own chunk and a fixed number of earlier chunks, offline too.
 *   [ENG 9]    "ASR Engine", section 4.3 step 6 and sections 8-9: each stream commits its actual
 *              frames (a final window may be short); a cohort is padded to a wider graph shape
 *              through a padding lane whose rows compute only for themselves.
 *   [ENG 9p]   "ASR Engine", section 9: the positional projection of the relative-position table
 *              is sized by the cache rung (one projected row per table row).
 *   [MOD dec]  "Model Layer", the decoder notes (WeNet's linear_q / linear_k / linear_v /
 *              linear_out over the shared attention core; an activation folded into the GEMM
 *              epilogue) and "Heads" (projections at a GEMM-aligned width).
 *
 * Score of chunk query i (absolute position cache + i) against key j (0 <= j < cache + C):
 *     s[i][j] = ((q_i + u) . k_j + (q_i + v) . p[cache + i - j]) * softmax_scale
 * followed by a softmax over j and a weighted sum of v_j. No mask inside the window: every chunk
 * query sees every cached frame and every frame of its own chunk.
 *
 * Layouts (row-major, innermost last). B = batch, C = chunk_size, H = n_head, Hk = n_kv_head,
 * D = head_dim, S = block_size, N = num_blocks, M = max_blocks_per_seq:
 *   q, out          [B, C, H, D]
 *   k_new, v_new    [B, C, Hk, D]
 *   k_pool          [N, Hk, D / 32, S, 32]   one pool per layer; K pages in 32-dim column
 *                                            blocks: dim d of slot s is element (d / 32, s,
 *                                            d % 32), so each 32-dim half of every slot's row
 *                                            is contiguous (an MFMA fragment's half-row loads
 *                                            then cover whole 128-byte lines)
 *   v_pool          [N, Hk, D, S]            V is stored transposed inside each page
 *   block_tables    int32 [B, M]             logical frame t of stream b is in block
 *                                            block_tables[b][t / S], slot t % S
 *   cache_seqlens   int32 [B]                frames cached before this chunk
 *   window_start    int32 [B] or NULL        bounded history [ENG 6, 9]: absolute position of
 *                                            stream b's first cached frame, a multiple of S
 *                                            (rounded down otherwise). Absolute position p is in
 *                                            block block_tables[b][(p / S) % M], slot p % S:
 *                                            the row is a ring of M pages, and a recycled page
 *                                            is reused without rewriting the table. The cached
 *                                            frames are [w_b, w_b + cache_seqlens[b]), the chunk
 *                                            follows them; distances count inside the window
 *                                            (key index j below), so positions are unaffected.
 *                                            NULL: every window starts at 0 (no ring)
 *   chunk_lens      int32 [B] or NULL        real frames n_b <= C of each stream's chunk (NULL:
 *                                            every stream has C). Reading of [ENG 9]: frames
 *                                            t >= n_b do not exist - they are not appended, are
 *                                            not keys, and their output rows are zero. n_b = 0
 *                                            is a padding lane: nothing of it is read or written
 *                                            but its zero output rows
 *   pos_bias_u, _v  [H, D]
 *   pos (shared)    [pos_len, H, D]          row r holds distance (pos_len - 1) / 2 - r
 *   pos (per row)   [B, pos_len, H, D]       stream b's table: rows [0, 2 T_b - 1), centred at
 *                                            T_b - 1 (T_b = cache_seqlens[b] + C, the full
 *                                            chunk width whatever chunk_lens says); rows past
 *                                            that are never read
 *   pos, with PKC_POS_COL_BLOCKED            the same tables stored in 32-dim column blocks per
 *                   [H, D / 32, pos_len, 32] head: dim d of row r of head h is element
 *                or [B, H, D / 32, pos_len, 32]  (h, d / 32, r, d % 32). The rows a 16-row MFMA
 *                                            fragment reads are then contiguous (whole 128-byte
 *                                            lines, as in the K pages); row-major rows give every
 *                                            load instruction 16 half-lines instead
 * Query head h reads kv head h / (H / Hk). Element type: fp32 or bf16 for every floating-point
 * buffer of a call; accumulation is fp32 either way; bf16 outputs are rounded to nearest even.
 *
 * Device-side preconditions (not checkable on the host without a synchronisation):
 *   0 <= cache_seqlens[b] <= max_cache_seqlen; block_tables[b][t / S] in [0, N) for every
 *   t < cache_seqlens[b] + n_b; no two streams own the same page. Kernels clamp cache lengths,
 *   chunk lengths and block IDs into range, so a violation gives unspecified values but never an
 *   out-of-bounds access. The attention reads more of each table row than the stream's own
 *   pages: every workgroup reads the first min(M, 128) entries of its row into LDS, whatever the
 *   stream's length (the block IDs of later pages are read from the row as needed). When
 *   cache_seqlens[b] is not a multiple of 32, the last 32-key step of the cached frames also
 *   reads the frames past them: through the row's next entry, which may name another stream's
 *   page (or hold any value, clamped into [0, N)). Those frames are masked and their V zeroed
 *   before use, so such reads never change a result; they only touch valid pool memory.
 *   With window_start, w_b + max_cache_seqlen + C stays below 2^31 (positions are 32-bit).
 *
 * Launch limits, common to every entry point: HIP launches fewer than 2^32 work-items along a
 * grid dimension, so a call whose grid (workgroups x threads per workgroup, stated per entry point
 * below) would reach 2^32 is refused with PKC_ERR_UNSUPPORTED before anything is launched. Sizes
 * are combined in 64-bit (saturating) arithmetic on the host, so no int32 argument can wrap a check.
 */
#ifndef PKC_H
#define PKC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums below are 32-bit ints on both sides of the ABI. A C caller may pass any int where an
 * enum is expected (the entry points reject values they do not know), so in C++ they get int32_t
 * as a fixed underlying type, which makes every int32 value a valid value of the type. */
#ifdef __cplusplus
#define PKC_ENUM_BASE : int32_t
#else
#define PKC_ENUM_BASE
#endif

typedef enum pkc_status PKC_ENUM_BASE {
  PKC_OK = 0,
  PKC_ERR_NULL = 1,        /* a required pointer is NULL                                    */
  PKC_ERR_SHAPE = 2,       /* a size is out of range or sizes disagree                      */
  PKC_ERR_DTYPE = 3,       /* unknown element type                                          */
  PKC_ERR_UNSUPPORTED = 4, /* valid, but not built (e.g. head_dim != 64 for attention)      */
  PKC_ERR_CAPACITY = 5,    /* max_cache_seqlen + chunk_size > max_blocks_per_seq * block_size */
  PKC_ERR_HIP = 6,         /* the HIP runtime reported an error at launch                   */
  PKC_ERR_ALIGN = 7        /* a tensor pointer is not 16-byte aligned                       */
} pkc_status;

typedef enum pkc_dtype PKC_ENUM_BASE { PKC_F32 = 0, PKC_BF16 = 1 } pkc_dtype;

/* Layout of the positional tables (flags of the pos_layout argument). */
typedef enum pkc_pos_layout PKC_ENUM_BASE {
  PKC_POS_SHARED = 0,   /* one table by distance for the cohort                         */
  PKC_POS_PER_ROW = 1,  /* one table per stream                                          */
  PKC_POS_PER_KEY = 2,  /* rows are keys, not distances (WeNet's convention, no shift)   */
  PKC_POS_COL_BLOCKED = 4 /* storage in 32-dim column blocks per head (see Layouts)       */
} pkc_pos_layout;

/* Library version, major * 10000 + minor * 100 + patch. */
int pkc_version(void);

/* Static description of a status code. */
const char* pkc_status_string(int status);

/*
 * paged_kv_append - write each stream's new chunk K/V into its pages [ENG 4.3].
 *
 * For b < batch and t < n_b (chunk_lens[b], or chunk_size when chunk_lens is NULL), with
 * L = cache_seqlens[b] + t:
 *     k_pool[block_tables[b][L / S]][g][c][L % S][:] = k_new[b][t][g][32 c : 32 c + 32]
 *     v_pool[block_tables[b][L / S]][g][:][L % S] = v_new[b][t][g][:]
 * for every kv head g. No other pool element is touched; the copy is bit-exact. The caller then
 * runs the attention and afterwards advances cache_seqlens by n_b itself.
 * Grid: batch x n_kv_head workgroups of 256 threads; a workgroup stages 64 frames of V in LDS,
 * 64 (head_dim + 16 / element bytes) element bytes, which must fit the default 64 KiB
 * (head_dim <= 504 in bf16, <= 252 in fp32).
 * Errors: NULL pointers -> PKC_ERR_NULL; non-positive sizes or head_dim not a multiple of 8 ->
 * PKC_ERR_SHAPE; head_dim not a multiple of 32, the V staging beyond 64 KiB or the launch limits
 * -> PKC_ERR_UNSUPPORTED; max_cache_seqlen + chunk_size > max_blocks_per_seq * block_size ->
 * PKC_ERR_CAPACITY (the analogue of the pool/table ceiling errors of [ENG 6]).
 */
pkc_status paged_kv_append(pkc_dtype dtype, const void* k_new, const void* v_new, void* k_pool,
                           void* v_pool, const int32_t* block_tables, const int32_t* cache_seqlens,
                           const int32_t* chunk_lens, const int32_t* window_start, int32_t batch,
                           int32_t chunk_size, int32_t n_kv_head, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_cache_seqlen, hipStream_t stream);

/*
 * chunk_paged_relpos_attn - chunk attention over cached frames plus the chunk [SCH 4.3],
 * [MOD fix], as called once per layer inside forward_chunk_paged [MOD surf].
 *
 * The chunk's K/V must already be in the pools (paged_kv_append first). For every stream b,
 * head h and chunk query i < n_b, attends over the cache_seqlens[b] + n_b frames of stream b
 * read through block_tables, and writes out[b][i][h][:]; rows i >= n_b are written as zero
 * (n_b = chunk_lens[b], or chunk_size when chunk_lens is NULL).
 * pos_layout (pkc_pos_layout flags):
 *   0: pos is one shared table of pos_len rows (pos_len odd and
 *      (pos_len - 1) / 2 >= max_cache_seqlen + chunk_size - 1), indexed by distance around its
 *      centre (Transformer-XL, [MOD fix]).
 *   PKC_POS_PER_ROW: pos holds one such table per stream, pos_len rows apart
 *      (pos_len >= 2 * (max_cache_seqlen + chunk_size) - 1), centred at T_b - 1.
 *   PKC_POS_PER_KEY (WeNet's convention, [MOD nem]): no shift - row j of the table is the
 *      embedding of key j itself (the caller builds it from the keys' absolute positions, which
 *      start at offset - cache_seqlens), and the position term is (q_i + v) . p[j]. Shared, or
 *      with PKC_POS_PER_ROW one table per stream pos_len rows apart; pos_len >= max_cache_seqlen
 *      + chunk_size either way.
 *   PKC_POS_COL_BLOCKED combines with any of the above: the same tables, stored in 32-dim column
 *      blocks per head (Layouts above). The values and the results are those of the row-major
 *      tables; only the addresses differ.
 * softmax_scale <= 0 selects 1 / sqrt(head_dim).
 * Errors: as paged_kv_append; n_head % n_kv_head != 0 or a table too short -> PKC_ERR_SHAPE;
 * head_dim != 64, block_size not a power of two >= 8, a chunk too long for the kernel's LDS
 * staging, pos_len >= 2^25, or the launch limits (batch n_head ceil(chunk_size / 16) workgroups
 * of 256 threads: one per 16 queries of a stream and head) -> PKC_ERR_UNSUPPORTED. The kernel
 * stages the chunk's chunk_size frames in LDS (the cached frames stream from the pages), which
 * allows chunk_size <= 512 in bf16 and <= 256 in fp32.
 * Launch shape: each workgroup runs its keys as four fixed partitions merged in a fixed order, on
 * 4 wavefronts, or on 1 (64 threads) when the grid fills every wave slot of the GPU with one
 * wavefront per workgroup (bf16 fused entries, chunk_size <= 32, block_size 16 or 32, no
 * chunk_lens or window_start); the results are bitwise the same either way. The environment
 * variable PKC_CHUNK_WAVES = 1, 2 or 4, read at each launch, forces the count for those calls.
 * For those variants at 4 wavefronts, a grid larger than two workgroups per CU (at most 4096
 * streams) runs the streams longest cache first (each workgroup ranks the cache lengths itself);
 * PKC_CHUNK_ORDER = 0 or 1 forces it. The order changes which workgroup runs which stream, not
 * any result.
 */
pkc_status chunk_paged_relpos_attn(pkc_dtype dtype, const void* q, const void* k_pool,
                                   const void* v_pool, const int32_t* block_tables,
                                   const int32_t* cache_seqlens, const int32_t* chunk_lens,
                                   const int32_t* window_start, const void* pos, int32_t pos_len,
                                   int32_t pos_layout, const void* pos_bias_u,
                                   const void* pos_bias_v, void* out, int32_t batch,
                                   int32_t chunk_size, int32_t n_head, int32_t n_kv_head,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_cache_seqlen,
                                   float softmax_scale, hipStream_t stream);

/*
 * paged_kv_append_relpos_attn - one layer's step of the hot path in a single launch: the append
 * of paged_kv_append followed by the attention of chunk_paged_relpos_attn [ENG 4.3], [SCH 4.3].
 * The chunk's keys and values are taken from k_new / v_new for the attention and written into
 * the pools in the same kernel; the results equal the two calls in sequence. Arguments and errors
 * are those of the two calls (k_pool / v_pool are written).
 */
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
                                       hipStream_t stream);

/*
 * paged_kv_append_relpos_attn_layers - the fused append + attention of n_layers layers in one call
 * [ENG 4.3] (one PagedKVCache per layer sharing the block table and cache lengths; the streaming
 * step runs them in sequence), so that one host call enqueues a whole step and a caller can
 * capture it in a HIP graph.
 *
 * q, k_new, v_new, k_pool, v_pool, pos, pos_bias_u, pos_bias_v, out: HOST arrays of n_layers
 * device pointers, entry l being layer l's buffer of the layout above (entries may repeat, e.g.
 * one positional table for every layer). block_tables, cache_seqlens, chunk_lens, window_start
 * and every size argument are shared by the layers. Layer l's kernel is enqueued after layer
 * l - 1's on the stream; the results equal n_layers calls of paged_kv_append_relpos_attn. The
 * pointer arrays are read during the call only.
 * Errors: those of paged_kv_append_relpos_attn for any layer, n_layers <= 0 -> PKC_ERR_SHAPE.
 * Every layer is validated before any kernel is enqueued, so an error enqueues nothing.
 */
pkc_status paged_kv_append_relpos_attn_layers(
    pkc_dtype dtype, int32_t n_layers, const void* const* q, const void* const* k_new,
    const void* const* v_new, void* const* k_pool, void* const* v_pool,
    const int32_t* block_tables, const int32_t* cache_seqlens, const int32_t* chunk_lens,
    const int32_t* window_start, const void* const* pos, int32_t pos_len, int32_t pos_layout,
    const void* const* pos_bias_u,
    const void* const* pos_bias_v, void* const* out, int32_t batch, int32_t chunk_size,
    int32_t n_head, int32_t n_kv_head, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_cache_seqlen, float softmax_scale, hipStream_t stream);

/*
 * paged_kv_commit - after a step's layers: cache_seqlens[b] += n_b for every stream (n_b =
 * chunk_lens[b] clamped into [0, chunk_size], or chunk_size when chunk_lens is NULL) [ENG 4.3]
 * step 6 (commit_chunk_paged). It runs on the device, on the caller's stream, so a captured step
 * (layers + commit) can be replayed step after step with no host round trip: the attention reads
 * the cache lengths from device memory and sizes nothing by them, so one graph serves every
 * cache length up to the max_cache_seqlen it was captured with.
 * Bounded history [ENG 6, 9]: with window_start non-NULL, whole oldest blocks are then dropped
 * while cache_seqlens[b] > max_cached_frames: window_start[b] += block_size and cache_seqlens[b]
 * -= block_size (num_left_chunks = K is max_cached_frames = K * chunk_size with block_size
 * dividing chunk_size; recycle_streaming_history is the ring's own capacity, at most
 * max_blocks_per_seq * block_size - chunk_size). Without it, keeping cache_seqlens within
 * max_cache_seqlen is the caller's business (the next attention call clamps, it does not fail).
 * Only whole blocks that are already filled are dropped (at most cache_seqlens[b] / block_size
 * of them): the next chunk is written right after the cached frames, so the window start never
 * passes that position and cache_seqlens never goes negative; with a cap below one block a
 * partly filled last block therefore stays (e.g. 13 cached frames, block_size 8, cap 0: one block
 * goes, 5 frames stay). A negative stored length is written back as 0.
 * Errors: NULL cache_seqlens -> PKC_ERR_NULL; batch or chunk_size <= 0, or with window_start a
 * block_size <= 0 or a negative cap -> PKC_ERR_SHAPE.
 */
pkc_status paged_kv_commit(int32_t* cache_seqlens, const int32_t* chunk_lens,
                           int32_t* window_start, int32_t max_cached_frames, int32_t batch,
                           int32_t chunk_size, int32_t block_size, hipStream_t stream);

/*
 * varlen_packed_relpos_attn - full-context attention inside each utterance of a packed, gapless
 * row [MOD surf] (forward_offline_packed), with one relative-position table per utterance.
 *
 * q, out: [total_frames, H, D]; k, v: [total_frames, Hk, D]; cu_seqlens: int32 [num_seqs + 1],
 * cu_seqlens[0] = 0, nondecreasing, cu_seqlens[num_seqs] = total_frames; every segment length
 * <= max_seqlen. Utterance s (frames [cu_seqlens[s], cu_seqlens[s+1]), length L) has a table of
 * 2 L - 1 rows centred at L - 1 starting at row 2 cu_seqlens[s] of pos [2 total_frames, H, D]
 * (2 L rows are reserved per utterance, the last unused). Frames attend only within their own
 * utterance; empty utterances are allowed. The kernel clamps cu_seqlens into [0, total_frames],
 * so malformed offsets give unspecified values but no out-of-bounds access; an utterance longer
 * than max_seqlen is cut to its first max_seqlen frames (frames past them are not written; the
 * values of the rest are then unspecified).
 * mask_chunk > 0 applies the chunked_limited mask [MOD nem] inside every utterance: frame i (counted
 * from the utterance's first frame) sees only the frames of chunks i / mask_chunk -
 * mask_left_chunks ... i / mask_chunk, and each 64-frame query block computes only over the keys
 * its frames can see (its own frames plus the trained history). mask_chunk = 0: full context.
 * Errors: as above; a negative mask_chunk or mask_left_chunks -> PKC_ERR_SHAPE; head_dim != 64,
 * 2 max_seqlen max(H, Hk) head_dim element bytes at or past 2^31 (an utterance's rows are
 * addressed by 32-bit byte offsets), or the launch limits (num_seqs n_head ceil(max_seqlen / Q)
 * workgroups of 256 threads, one per Q queries of an utterance and head: Q = 128 in bf16, 64 in
 * fp32 and with the chunked_limited mask) -> PKC_ERR_UNSUPPORTED.
 */
pkc_status varlen_packed_relpos_attn(pkc_dtype dtype, const void* q, const void* k, const void* v,
                                     const int32_t* cu_seqlens, int32_t num_seqs,
                                     int32_t total_frames, int32_t max_seqlen, const void* pos,
                                     const void* pos_bias_u, const void* pos_bias_v, void* out,
                                     int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                                     int32_t mask_chunk, int32_t mask_left_chunks,
                                     float softmax_scale, hipStream_t stream);

/*
 * pkc_linear - y = x W^T + b, a linear layer [MOD dec] (linear_out, or any projection beside
 * the attention), on MFMA with fp32 accumulation.
 *
 * x [M, K], w [N, K] (out_features x in_features, the nn.Linear storage), bias [N] or NULL,
 * y [M, N]; all row-major, one dtype. y is written in full; nothing else is touched.
 * Grid: one workgroup per output tile (128 x 128, 128 x 64 or 64 x 64, picked by size; also
 * 128 x 192 and 32 x 64 for bf16 with K of 256, 512 or 1024, whose stages are loaded straight
 * into LDS), of 256 threads, or 512 for those direct stages with K of 512 or 1024 on tiles of 64
 * rows or more.
 * Errors: NULL x, w or y -> PKC_ERR_NULL; a non-positive size, or M, N or K at or past 2^30 ->
 * PKC_ERR_SHAPE; K not a multiple of 32, N not a multiple of 16 or the launch limits ->
 * PKC_ERR_UNSUPPORTED; a pointer not 16-byte aligned -> PKC_ERR_ALIGN.
 */
pkc_status pkc_linear(pkc_dtype dtype, const void* x, const void* w, const void* bias, void* y,
                      int32_t M, int32_t N, int32_t K, hipStream_t stream);

/*
 * paged_kv_qkv_append - the chunk's Q/K/V projection [MOD dec] with the append [ENG 4.3] as
 * its epilogue: the chunk's K/V rows go from the GEMM straight into the stream's pages.
 *
 * x [B, C, d_model]; w_qkv [(H + 2 Hk) D, d_model] stacks the rows of linear_q, linear_k and
 * linear_v in that order, b_qkv [(H + 2 Hk) D] or NULL likewise. With y = x w_qkv^T + b_qkv:
 *     q_out[b][t][h][:] = y[b][t][h D : (h + 1) D]                    (every t < C)
 * and, for t < n_b only, K = y[.., H D + g D : ...] and V = y[.., (H + Hk) D + g D : ...] are
 * written exactly where paged_kv_append would write k_new / v_new (same pools, layouts, block
 * tables, cache lengths, chunk lengths and window starts). K/V are rounded to the pool's dtype
 * once; no other pool element is touched. cache_seqlens is not advanced.
 * Errors: as paged_kv_append; n_head % n_kv_head != 0 -> PKC_ERR_SHAPE; d_model not a multiple
 * of 32 -> PKC_ERR_UNSUPPORTED; any of x, w_qkv, b_qkv, q_out not 16-byte aligned ->
 * PKC_ERR_ALIGN.
 */
pkc_status paged_kv_qkv_append(pkc_dtype dtype, const void* x, const void* w_qkv,
                               const void* b_qkv, void* q_out, void* k_pool, void* v_pool,
                               const int32_t* block_tables, const int32_t* cache_seqlens,
                               const int32_t* chunk_lens, const int32_t* window_start,
                               int32_t batch, int32_t chunk_size, int32_t d_model, int32_t n_head,
                               int32_t n_kv_head, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_cache_seqlen, hipStream_t stream);

/*
 * rel_pos_projection - linear_pos over sinusoidal tables [ENG 9p], [MOD fix]: the positional
 * tables the attention reads, without materialising the sinusoid.
 *
 * Row r of table t holds position p = pos_start[t] + pos_step r (pos_start int32 [n_tables] on
 * the device, or NULL for pos_first in every table). Its sinusoid e has, for i < d_model / 2,
 * e[2 i] = sin(p f_i) and e[2 i + 1] = cos(p f_i), f_i = 10000^(-2 i / d_model), and
 *     pos_out[t][r][:] = e W_pos^T      (w_pos [out_features, d_model], no bias)
 * pos_out [n_tables, rows, out_features]. A Transformer-XL table by distance centred at c
 * (row r holds distance c - r, the layout chunk_paged_relpos_attn reads) is pos_first = c,
 * pos_step = -1, rows = 2 c + 1; WeNet's per-key table of stream b [MOD nem] is
 * pos_start[b] = offset_b - cache_seqlens[b], pos_step = +1. The phase p f_i is formed and
 * reduced to a fraction of a turn in fp64, so its error (about 2^-25 turns) does not grow with
 * |p|; the sine and cosine are taken in fp32 and rounded to the dtype before the product. The
 * GEMM's grid and limits are those of pkc_linear with M = n_tables x rows.
 * Errors: NULL w_pos or pos_out -> PKC_ERR_NULL; non-positive n_tables or rows, or positions
 * beyond +-2^24 (the range the phase accuracy is stated for; checked for pos_first, the caller's
 * precondition for pos_start) -> PKC_ERR_SHAPE; d_model not a multiple of 32, out_features not a
 * multiple of 16 or the launch limits -> PKC_ERR_UNSUPPORTED; a pointer not 16-byte aligned ->
 * PKC_ERR_ALIGN.
 */
pkc_status rel_pos_projection(pkc_dtype dtype, const void* w_pos, const int32_t* pos_start,
                              int32_t pos_first, int32_t pos_step, int32_t n_tables, int32_t rows,
                              int32_t d_model, int32_t out_features, void* pos_out,
                              hipStream_t stream);

/*
 * pkc_gather_read - a measurement entry, not an attention: the memory-path ceiling of one
 * paged_kv_append_relpos_attn launch [ENG 4.3], [MOD fix]. It reads every byte that launch reads
 * (queries, u, v, k_new, v_new, the cached pages through block_tables, the positional band rows
 * of every 32-key step) with the attention kernel's own per-lane addresses, writes the chunk's
 * K/V into the pools exactly as paged_kv_append does, and writes unspecified values (an XOR of
 * what it read) into out. It does no arithmetic, so its launch time is what the access pattern
 * costs at a launch shape: waves (1, 4 or 8) wavefronts per workgroup and split (1, 2 or 4)
 * workgroups per (stream, head); split > 1 omits the merge a split attention would need.
 * reads = 0 runs the same grid but only writes out (reads nothing, appends nothing): the floor
 * that launching and retiring the grid costs.
 * Arguments are those of paged_kv_append_relpos_attn (no chunk lengths or window starts).
 * Errors: as paged_kv_append_relpos_attn; waves, split or reads outside those sets ->
 * PKC_ERR_SHAPE; fp32, chunk_size > 16 or PKC_POS_PER_KEY -> PKC_ERR_UNSUPPORTED.
 */
pkc_status pkc_gather_read(pkc_dtype dtype, const void* q, const void* k_new, const void* v_new,
                           void* k_pool, void* v_pool, const int32_t* block_tables,
                           const int32_t* cache_seqlens, const void* pos, int32_t pos_len,
                           int32_t pos_layout, const void* pos_bias_u, const void* pos_bias_v,
                           void* out, int32_t batch, int32_t chunk_size, int32_t n_head,
                           int32_t n_kv_head, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_cache_seqlen, int32_t waves, int32_t split,
                           int32_t reads, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKC_H */
