/*
 * pa.h — paged-KV decode attention for AMD MI355X (gfx950), C ABI.
 *
 * Three pieces, as the source pages describe a PagedAttention engine:
 *   1. pa_cache_write — append new K/V rows into the paged cache through a
 *      slot mapping, after any copy-on-write block copies;
 *   2. pa_decode      — single-query decode attention over the paged cache,
 *      addressed through per-sequence block tables;
 *   3. pa_bm_*        — a host-side block manager: free pool, per-sequence
 *      block tables, reference-counted sharing, fork and copy-on-write.
 *
 * Sources (page title, then the section on that page):
 *   [KVPA]  "KV Cache与PagedAttention深度解析：vLLM内存管理革命" (iopencloud.com)
 *   [KV2P]  "KV Cache从原理到实战：大模型推理内存管理演进与优化" (xnwp.cn)
 *   [NANO]  the zwxr.cn nano-vllm walkthrough (untitled in the extract)
 *   [INFRA] "大模型 (LLM) 推理加速核心技术解析：从 KV Cache 到 PagedAttention
 *           实战" (jsqmd.com)
 *
 * Conventions for every call:
 *   - Return value is a pa_status (0 = PA_OK).  No C++ exception crosses the
 *     ABI.  pa_strerror() names a status; pa_last_error() gives the detail of
 *     the last failure on the calling thread.
 *   - Device pointers are raw HIP device addresses owned by the caller; the
 *     library never allocates, frees or retains device memory, save the one
 *     fixed array per GPU that pa_decode_static (2a) uses in place of a
 *     workspace.  Host pointers are only read or written during the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued on it and the call returns without waiting; a
 *     device-side fault surfaces at the caller's next synchronisation.
 *   - Sizes and shapes are host integers.  Contents of device arrays (block
 *     ids, slots, lengths) are the caller's contract; the kernels clamp every
 *     index they read so a bad entry cannot address memory outside the
 *     buffers: a block-table id outside [0, num_blocks) is read as block 0;
 *     for other bad entries the result is unspecified.  With the environment
 *     variable PA_CHECK=1 the library copies those arrays to the host,
 *     validates them and returns PA_ERR_INVALID_ARG instead (slow; for
 *     debugging).  PA_CHECK is read on every call.
 *   - Other environment switches: PA_LOG=1 (read when a block manager is
 *     created) logs to stderr every block it takes from the free list and
 *     every reference it drops;
 *     PA_TUNE_VARIANT=0..2 (read once per process) overrides the decode
 *     kernels' pipeline variant, for tuning experiments only.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,  /* bad pointer, size, shape or alignment       */
  PA_ERR_UNSUPPORTED = -2,  /* shape/dtype combination with no kernel       */
  PA_ERR_WORKSPACE = -3,    /* workspace missing or too small; see *needed  */
  PA_ERR_OOM = -4,          /* block manager: not enough free blocks        */
  PA_ERR_NOT_FOUND = -5,    /* block manager: unknown sequence id           */
  PA_ERR_HIP = -6           /* a HIP runtime call failed                    */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0, /* IEEE binary32 */
  PA_F16 = 1, /* IEEE binary16 */
  /* INT8 KV cache ([KV2P] §5.2: INT8 halves the cache; one scale per group
   * of 128 elements).  kv_cache holds int8 codes, and a separate kv_scales
   * array [num_blocks, num_kv_heads, 2, block_size] float32 holds one scale
   * per (token, KV head) row of K and of V (the row of head_dim values is
   * the group).  Value = code * scale.  pa_cache_write takes binary16 key
   * and value rows and quantises them; pa_decode takes a binary16 query.
   * head_dim 64 or 128. */
  PA_I8 = 2
} pa_dtype;

/* Kernel family for pa_decode.  PA_KERNEL_AUTO picks per shape. */
typedef enum pa_kernel {
  PA_KERNEL_AUTO = 0,
  PA_KERNEL_VALU = 1, /* vector-ALU dot products, DPP lane reductions     */
  PA_KERNEL_MFMA = 2  /* matrix-core q.K^T and P.V tiles (f16, GQA only)  */
} pa_kernel;

/* Flag OR-ed into pa_decode's `kernel`: read K/V with plain (cached) loads.
 * By default K/V are streamed with non-temporal loads, since each byte is
 * read once per call; when many sequences share blocks (a common prefix),
 * keeping them cached lets the repeated reads hit on-chip caches. */
#define PA_KV_CACHED 0x100

/* -------------------------------------------------------------------------
 * 1. Cache write ([KVPA] §2.2 and §5.3; [KV2P] §2.1; [NANO] §2.3)
 *
 * Decoding computes K and V for the new token only and appends them to the
 * cache; with paging the row lands in block slot/block_size at row
 * slot%block_size.  Before the scatter, each (src, dst) pair in cow_pairs
 * copies the whole physical block src onto dst (K and V, every head, every
 * row): the copy-on-write a sequence needs before writing into a block it
 * shares ([NANO] §2.3, §5.5).  Both steps are enqueued on `stream`, copies
 * first.  For f32 / f16 pools the result is a byte copy (bit-exact).
 *
 * INT8 pools (PA_I8): each row x of head_dim values (one token, one KV head,
 * K or V) is stored as scale s = amax|x| / 127 and codes
 * clamp(rint(x / s), -127, 127), rint rounding ties to even, both divisions
 * IEEE binary32 on the binary16 inputs widened to binary32; a row of zeros
 * gets s = 0 and zero codes.  Copy-on-write copies move codes and scales.
 * Inputs must be finite.
 *
 *   key, value   device, [num_tokens, num_kv_heads, head_dim], dtype
 *                (binary16 for PA_I8), contiguous, 16-byte aligned
 *   kv_cache     device, [num_blocks, 2, num_kv_heads, block_size, head_dim],
 *                dtype, contiguous, 16-byte aligned; index 1 of dim 1 is V
 *   kv_scales    PA_I8: device, [num_blocks, num_kv_heads, 2, block_size]
 *                float32, 16-byte aligned (num_kv_heads * block_size even);
 *                otherwise NULL
 *   slot_mapping device, [num_tokens] int64; slot < 0 skips the row; slots
 *                must lie in [0, num_blocks*block_size) and be distinct
 *   cow_pairs    device, [num_cow, 2] int32 (src, dst) block ids, or NULL
 *                when num_cow == 0; destinations distinct and not sources
 *   num_tokens, num_cow >= 0 (0 = nothing to do)
 *   head_dim * element size must be a multiple of 16 bytes.
 * ------------------------------------------------------------------------- */
int pa_cache_write(const void* key, const void* value, void* kv_cache,
                   float* kv_scales, const int64_t* slot_mapping, int64_t num_tokens,
                   const int32_t* cow_pairs, int64_t num_cow,
                   int64_t num_blocks, int num_kv_heads, int head_dim,
                   int block_size, int dtype, void* stream);

/* -------------------------------------------------------------------------
 * 1b. Per-step upload of the host bookkeeping ([KVPA] §5.3: the block table
 *     lives on the host and is copied to the GPU for each attention call)
 *
 * Copies `bytes` from page-locked host memory (hipHostMalloc, e.g. a torch
 * pin_memory tensor; the GPU addresses it directly) to device memory with a
 * kernel on `stream` that reads the host buffer over the bus, instead of a
 * DMA transfer: for the few tens of kilobytes a decode step uploads (block
 * tables, lengths, slots, copy pairs) this saves the copy engine's round
 * trip and hand-off to the compute queue.  The host must not change `src`
 * until the stream has passed this call (record an event after it).
 *   dst    device, 16-byte aligned
 *   src    page-locked host (hipHostMalloc), 16-byte aligned; anything else
 *          (pageable or device memory) is PA_ERR_INVALID_ARG
 *   bytes  >= 0, a multiple of 4 (0 = nothing to do)
 * ------------------------------------------------------------------------- */
int pa_stage_from_host(void* dst, const void* src, int64_t bytes, void* stream);

/* The upload above and pa_cache_write in one launch (any copy-on-write pairs
 * in a launch before it): the step's tables reach stage_dst while the new
 * rows are scattered, saving a launch and its gap per decode step.  Same
 * arguments, rules and results as the two calls, with one more rule:
 * slot_mapping and cow_pairs are read by the launch that fills stage_dst, so
 * they must point to device memory or to page-locked host memory (e.g.
 * inside stage_src) — never into stage_dst; PA_ERR_INVALID_ARG otherwise. */
int pa_stage_and_write(void* stage_dst, const void* stage_src, int64_t stage_bytes,
                       const void* key, const void* value, void* kv_cache, float* kv_scales,
                       const int64_t* slot_mapping, int64_t num_tokens,
                       const int32_t* cow_pairs, int64_t num_cow, int64_t num_blocks,
                       int num_kv_heads, int head_dim, int block_size, int dtype,
                       void* stream);

/* -------------------------------------------------------------------------
 * 2. Decode attention ([KVPA] §2.1 formula, §4.3 block-table addressing,
 *    §7.2 online softmax; [NANO] §2.4 kernel structure; [KV2P] §5.3 GQA)
 *
 * For each sequence s and query head h, with G = num_q_heads/num_kv_heads,
 * g = h / G and n = context_lens[s]:
 *   out[s,h,:] = sum_t softmax_t(scale * q[s,h,:] . K_t) * V_t ,  t < n,
 * where token t is row t%block_size of physical block
 * block_tables[s, t/block_size]; K_t = kv_cache[b,0,g,row,:],
 * V_t = kv_cache[b,1,g,row,:].  Rows past n are never read; n == 0 gives 0.
 * With sliding_window = W > 0 only the last W tokens are keys:
 * max(0, n - W) <= t < n ([KV2P] §7.2, sliding-window attention); the
 * tiles before the window are not read.
 * Accumulation is float32; the output is float32.
 *
 *   out            device, [num_seqs, num_q_heads, head_dim] float32
 *   query          device, [num_seqs, num_q_heads, head_dim] dtype (binary16
 *                  for PA_I8), 16B aligned
 *   kv_cache       device, as for pa_cache_write
 *   kv_scales      PA_I8: the row scales written by pa_cache_write; K_t and
 *                  V_t above are then code * scale of their rows.  NULL
 *                  otherwise.
 *   block_tables   device, [num_seqs, max_blocks_per_seq] int32 (row stride =
 *                  max_blocks_per_seq); entries past ceil(n/block_size) unused
 *   context_lens   device, [num_seqs] int32, 0 <= n <= max_context_len and
 *                  n <= max_blocks_per_seq * block_size
 *   max_context_len host bound on context_lens (sizes the partition grid)
 *   scale          softmax scale, normally 1/sqrt(head_dim)
 *   sliding_window 0 = attend to the whole context; W > 0 = the last W
 *                  tokens; < 0 is PA_ERR_INVALID_ARG
 *   partition_size 0 = choose; -1 = single pass (one workgroup per (s, KV
 *                  head)); -2 = balanced: one grid of as many workgroups as
 *                  fit on the GPU at once, each taking an equal slice of all
 *                  (s, KV head, 16-token tile) work, for batches of at most
 *                  1024 sequences; > 0 = split each context into partitions
 *                  of this many tokens (a multiple of 16 and of block_size).
 *                  Split work is combined by a log-sum-exp merge kernel.
 *   kernel         a pa_kernel value, optionally | PA_KV_CACHED
 *   workspace      device scratch for split partials (caller-owned), may be
 *                  NULL when *workspace_needed is 0
 *   workspace_needed  out (may be NULL): bytes this call needs.  Calling with
 *                  out == NULL only computes it and returns PA_OK.
 * Supported: dtype f32, f16 or PA_I8; head_dim 64 or 128; block_size 8, 16
 * or 32; G in {1, 2, 4, 8}.  MFMA needs f16 or PA_I8 and G >= 2.  Anything
 * else returns PA_ERR_UNSUPPORTED.  A launch holds at most 2^24 - 1
 * workgroups: num_seqs * partitions * num_kv_heads (all but the balanced
 * schedule) and num_seqs * num_q_heads (any split schedule's merge) above
 * that return PA_ERR_INVALID_ARG, also for a size query.
 * ------------------------------------------------------------------------- */
int pa_decode(float* out, const void* query, const void* kv_cache,
              const float* kv_scales, const int32_t* block_tables,
              const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
              int block_size, int max_blocks_per_seq, int max_context_len,
              int64_t num_blocks, float scale, int sliding_window,
              int partition_size, int kernel, void* workspace,
              size_t workspace_bytes, size_t* workspace_needed, int dtype,
              void* stream);

/* -------------------------------------------------------------------------
 * 2a. Decode without a caller workspace — for callers that cannot allocate
 *     device memory: code under stream capture, tight serving loops,
 *     harnesses that forbid hipMalloc.
 *
 * pa_decode with the same arguments but the workspace ones, the same
 * kernels and the same results (bit for bit, for the same schedule).  The
 * split-context partials go to a device array of
 * pa_decode_static_capacity() bytes (64 MiB) that the library holds on each
 * GPU it runs on until the process ends; the call allocates and frees no
 * memory.  A call whose partials need more returns PA_ERR_WORKSPACE before
 * anything is enqueued; out == NULL only checks whether the call fits.  All
 * calls on one GPU share that array: calls that overlap on a GPU (on other
 * streams, or from other host threads without ordering) race; calls on one
 * stream are ordered.  The array needs no clearing between calls.
 * ------------------------------------------------------------------------- */
int pa_decode_static(float* out, const void* query, const void* kv_cache,
                     const float* kv_scales, const int32_t* block_tables,
                     const int32_t* context_lens, int num_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size,
                     int max_blocks_per_seq, int max_context_len, int64_t num_blocks,
                     float scale, int sliding_window, int partition_size, int kernel,
                     int dtype, void* stream);
size_t pa_decode_static_capacity(void);

/* -------------------------------------------------------------------------
 * 2b. Multi-token queries: causal attention of a prefill chunk ([KV2P] §5.4
 *     chunked prefill; [INFRA] §2 causal mask for T > 1; [KVPA] §4.3
 *     block-table addressing)
 *
 * Sequence s brings T_s = query_start[s+1] - query_start[s] new tokens whose
 * K/V are already in the cache (pa_cache_write first); n_s = context_lens[s]
 * counts them.  Query i of sequence s (row query_start[s] + i) sits at
 * position p = n_s - T_s + i and attends to keys t <= p:
 *   out[row, h, :] = sum_{t <= p} softmax_t(scale * q[row,h,:] . K_t) V_t,
 * with the paging and grouping of pa_decode.  T_s = 1 is the decode case;
 * T_s = n_s is an ordinary causal prefill.  With sliding_window = W > 0 a
 * query sees only the last W tokens up to its own position, p - W < t <= p
 * ([KV2P] §7.2, the decode's window at every query position); rows before
 * every query's window are not read.  Accumulation and output float32.
 *
 *   out            device, [total_queries, num_q_heads, head_dim] float32
 *   query          device, [total_queries, num_q_heads, head_dim] binary16
 *   kv_cache       device, binary16 or PA_I8 pool as for pa_cache_write
 *   kv_scales      PA_I8: the row scales written by pa_cache_write ([KV2P]
 *                  §5.2; K_t and V_t are then code * scale of their rows);
 *                  NULL otherwise
 *   block_tables   device, [num_seqs, max_blocks_per_seq] int32
 *   context_lens   device, [num_seqs] int32, T_s <= n_s <= max_blocks * bs
 *   query_start    device, [num_seqs + 1] int32, non-decreasing, from 0 to
 *                  total_queries
 *   max_query_len  host bound on every T_s (sizes the grid)
 *   scale          > 0 and finite (the kernel takes the running max on the
 *                  raw scores); PA_ERR_INVALID_ARG otherwise
 *   sliding_window 0 = every earlier key; W > 0 = the last W tokens up to
 *                  the query; < 0 is PA_ERR_INVALID_ARG
 *   kernel         PA_KERNEL_AUTO or PA_KERNEL_MFMA (PA_KV_CACHED is accepted
 *                  and has no effect: every K/V row is read by several
 *                  query blocks, so the prefill always uses cached loads)
 * Sequences with T_s > n_s, or whose rows leave [0, total_queries), produce
 * no output rows.  Supported: dtype
 * PA_F16 or PA_I8; head_dim 64 or 128; block_size 8, 16 or 32; G in
 * {1, 2, 4, 8}.
 * num_seqs * num_kv_heads * ceil(max_query_len * G / 128) workgroups above
 * 2^24 - 1 return PA_ERR_INVALID_ARG; a pool whose blocks exceed 32-bit
 * byte offsets (num_kv_heads * block_size * head_dim * 4 >= 2^32) returns
 * PA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
int pa_prefill(float* out, const void* query, const void* kv_cache,
               const float* kv_scales, const int32_t* block_tables,
               const int32_t* context_lens,
               const int32_t* query_start, int num_seqs, int total_queries,
               int num_q_heads, int num_kv_heads, int head_dim,
               int block_size, int max_blocks_per_seq, int max_query_len,
               int64_t num_blocks, float scale, int sliding_window, int kernel,
               int dtype, void* stream);

/* -------------------------------------------------------------------------
 * 3. Host block manager ([KVPA] §5.1-§5.3, §8.2; [KV2P] §6.2; [NANO] §2.3,
 *    §4.2)
 *
 * An opaque handle over host memory only; not thread-safe (one caller at a
 * time per handle).  Sequence ids are arbitrary int64 keys.  The free pool is
 * a stack that starts as [0, 1, ..., num_blocks-1] and hands out from the
 * top.  Every block carries a reference count = the number of tables that
 * hold it; it returns to the pool when the count reaches 0.  Every failing
 * call leaves the state unchanged.
 * ------------------------------------------------------------------------- */
typedef struct pa_bm pa_bm;

/* NULL on bad arguments (num_blocks <= 0, block_size <= 0) or no memory. */
pa_bm* pa_bm_create(int64_t num_blocks, int block_size);
void pa_bm_destroy(pa_bm* bm);

/* New sequence holding ceil(num_tokens/block_size) fresh blocks, count 1.
 * PA_ERR_INVALID_ARG if seq exists or num_tokens < 0; PA_ERR_OOM if too few
 * blocks are free. */
int pa_bm_allocate(pa_bm* bm, int64_t seq, int64_t num_tokens);

/* Append n blocks already held by other sequences to seq's table (creating
 * seq if needed) and add a reference to each: prefix reuse.  The blocks carry
 * num_tokens tokens (ceil(num_tokens/block_size) == n) and seq, if it exists,
 * must end on a block boundary. */
int pa_bm_share(pa_bm* bm, int64_t seq, const int32_t* blocks, int n,
                int64_t num_tokens);

/* child := copy of parent's table and token count, one more reference per
 * block.  PA_ERR_NOT_FOUND for an unknown parent; INVALID_ARG if child
 * exists. */
int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child);

/* Reserve the place of seq's next token.  *slot = block*block_size + row.
 * A fresh block is taken when the sequence ends on a block boundary; if the
 * last block is shared, a fresh block replaces it in seq's table and
 * *cow_src and *cow_dst name the copy to make (else both are -1). */
int pa_bm_append_slot(pa_bm* bm, int64_t seq, int64_t* slot, int32_t* cow_src,
                      int32_t* cow_dst);

/* Batched append_slot over n sequences, in order: slots[i] for seqs[i];
 * copy pairs packed into cow_pairs[2*k], cow_pairs[2*k+1] (room for n pairs)
 * with *num_cow = k.  All or nothing: on failure no sequence changes. */
int pa_bm_append_slots(pa_bm* bm, const int64_t* seqs, int n, int64_t* slots,
                       int32_t* cow_pairs, int* num_cow);

/* Drop one reference per table entry (table order) and forget seq. */
int pa_bm_free(pa_bm* bm, int64_t seq);

/* Copy seq's table into out[0..cap) (*n = its length, which may exceed cap:
 * then only cap entries are written) and its token count into *num_tokens.
 * Either out pointer may be NULL when cap == 0. */
int pa_bm_block_table(const pa_bm* bm, int64_t seq, int32_t* out, int cap,
                      int* n, int64_t* num_tokens);

/* Fill a padded [n, max_blocks] int32 table (-1 past each length) and the
 * int32 context lengths for seqs[0..n).  INVALID_ARG if a table is longer
 * than max_blocks. */
int pa_bm_block_tables(const pa_bm* bm, const int64_t* seqs, int n,
                       int32_t* tables, int max_blocks, int32_t* context_lens);

/* Pool counts: free blocks (plus evictable cached blocks when the prefix
 * cache is on), blocks with count >= 1, blocks with count >= 2. */
int pa_bm_stats(const pa_bm* bm, int64_t* num_free, int64_t* num_used,
                int64_t* num_shared);

/* Reference count of one block (>= 0), or PA_ERR_INVALID_ARG. */
int pa_bm_ref_count(const pa_bm* bm, int32_t block);

/* -------------------------------------------------------------------------
 * 3b. Prefix cache ([KVPA] §8.1-§8.2; [KV2P] §4.2-§4.3; [NANO] §3.2, §4.3)
 *
 * Requests that start with the same tokens share the blocks holding them.
 * Every full block is keyed by a chain hash of its token ids and position:
 * h_i = FNV-1a-64 over (h_{i-1} as 8 little-endian bytes, then the block's
 * token ids as 4 little-endian bytes each), h_{-1} = 0.  A lookup also
 * compares the stored parent hash and token ids, so a collision never hits.
 * Only full blocks are cached.  A cached block whose count reaches 0 stays
 * cached and becomes evictable; fresh blocks come from the free pool first,
 * then from evicting the least recently released evictable block, blocks
 * with at least protect_hits hits after all others (0 = plain LRU).  A
 * referenced block is never evicted.  With the cache on, pa_bm_stats'
 * num_free counts free plus evictable blocks.
 * ------------------------------------------------------------------------- */

/* Turn the prefix cache on; only on a manager that holds no sequence.
 * protect_hits >= 0: blocks with at least that many hits are evicted last
 * (0 = plain LRU).  admit_after >= 1: a full block enters the cache only at
 * the admit_after-th registration of its key (its tokens and position), so
 * prompts seen once do not push out reused ones ([KV2P] §4.3, cache
 * pollution); keys below the threshold are remembered for at most
 * num_blocks keys, the least recently seen forgotten first.  1 caches at the
 * first registration.  Errors: PA_ERR_INVALID_ARG. */
int pa_bm_enable_prefix_cache(pa_bm* bm, int protect_hits, int admit_after);

/* Admit a new sequence with prompt `tokens` [n] (host int32): its leading
 * full blocks that are cached are reused (one more reference each), the rest
 * of the prompt gets fresh blocks.  *cached_tokens (may be NULL) receives the
 * number of leading tokens whose K/V the reused blocks already hold; the
 * caller writes the others.  Errors: PA_ERR_INVALID_ARG (cache off, sequence
 * exists), PA_ERR_OOM (state unchanged). */
int pa_bm_allocate_prompt(pa_bm* bm, int64_t seq, const int32_t* tokens,
                          int64_t n, int64_t* cached_tokens);

/* Append the ids of the tokens appended since the known ids ended (decoded
 * tokens), so that their blocks can be registered; afterwards the known ids
 * must cover every token the sequence holds (else PA_ERR_INVALID_ARG). */
int pa_bm_record_tokens(pa_bm* bm, int64_t seq, const int32_t* tokens,
                        int64_t n);

/* Cache the sequence's full blocks whose token ids are known and whose K/V
 * the caller has written (call after the write).  A block whose key is
 * already cached under another block, or whose key has not yet reached the
 * admission threshold, stays private.  *newly_cached (may be NULL) receives
 * the number of blocks added. */
int pa_bm_register(pa_bm* bm, int64_t seq, int64_t* newly_cached);

/* out[7]: cached blocks, evictable blocks, lookups, reused (hit) blocks,
 * missed full blocks, evictions, registrations held back by the admission
 * threshold. */
int pa_bm_prefix_stats(const pa_bm* bm, int64_t* out);

/* ------------------------------------------------------------------------- */
const char* pa_strerror(int status);
const char* pa_last_error(void);
/* Library version string. */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PA_H_ */
