/*
 * pa.h -- C ABI of libpa.so: paged KV-cache attention for AMD MI355X (gfx950).
 *
 * The operations are those of a paged KV cache as the mini-vLLM pages describe
 * it:
 *   - K/V storage is split into fixed-size blocks of tokens, 16 per block
 *     (page "轻量级的vLLM", mini-vllm write-up, section 核心机制一：分页 KV Cache);
 *   - each sequence owns a block table mapping its logical blocks to physical
 *     ones, and attention finds the real K and V through it (page
 *     "从零实现一个 mini vLLM--开篇", section "5. 这个系列会怎么展开", stages four
 *     and five; page "vllm-v0 版本介绍", section 为什么需要推理框架？);
 *   - decode computes only the new token's K/V, appends them to the cache, and
 *     the new token attends to every cached token of its sequence (page
 *     "从零实现一个 mini vLLM--开篇", section "2. LLM 推理到底在慢什么");
 *   - chunked prefill is named as a later topic (same page, section 5, stage
 *     six); its reading here is stated at pa_prefill_chunk.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Memory     All array arguments are DEVICE pointers (hipMalloc'd or torch
 *             CUDA/HIP tensors), row-major and contiguous.  The caller owns
 *             every buffer, the workspace included; the library never allocates
 *             or frees device memory and keeps no state between calls.
 *  Layouts    q / key / value / out     [rows, heads, head_dim]
 *             k_cache / v_cache         [num_blocks, block_size, num_kv_heads, head_dim]
 *             block_tables              [num_seqs, max_blocks_per_seq] int32
 *             context_lens              [num_seqs] int32
 *             slot_mapping              [num_tokens] int32
 *  Heads      Query head h reads kv head h / (num_q_heads / num_kv_heads):
 *             consecutive query heads share one kv head (grouped-query heads).
 *  Types      dtype applies to q, key, value, caches and out alike, except
 *             for an fp8 cache (pa_reshape_and_cache_fp8, pa_decode_fp8).
 *             Attention accumulates in fp32; out is rounded to nearest even.
 *  Streams    stream is a hipStream_t (NULL = the legacy default stream).  Every
 *             call only enqueues work on it and returns; results are ready when
 *             the stream reaches that point.  Work on one stream runs in call
 *             order, so enqueue pa_reshape_and_cache before the attention call
 *             that must see the appended tokens.
 *  Errors     Every entry point returns a pa_status.  Argument checks run on the
 *             host before anything is enqueued; on an error nothing is launched
 *             and no buffer is touched.  The library never aborts or throws.
 *             Values inside device arrays are NOT checked (that would need a
 *             device-to-host copy): block ids must lie in [0, num_blocks),
 *             context_lens[s] <= max_blocks_per_seq * block_size, slots in one
 *             pa_reshape_and_cache call must be distinct, and every table entry
 *             below ceil(context_lens[s] / block_size) must be valid.  Table
 *             entries past that point are never read.
 *  Supported  block_size 16; head_dim 64 or 128; num_q_heads a multiple of
 *             num_kv_heads with at most 64 query heads per kv head; dtypes
 *             PA_F32 and PA_BF16 (pa_prefill_chunk: PA_BF16 only).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_F32 = 0,      /* IEEE binary32 */
    PA_BF16 = 1,     /* bfloat16 */
    PA_FP8_E4M3 = 2  /* OCP FP8 E4M3 ("E4M3FN": bias 7, max 448, no infinities);
                        storage of an fp8 cache only: accepted by the bit copies
                        pa_reshape_and_cache and pa_copy_blocks */
} pa_dtype;

typedef enum {
    PA_OK = 0,
    PA_EINVAL = -1,       /* an argument is out of its documented range */
    PA_EUNSUPPORTED = -2, /* valid, but a shape or dtype this build does not handle */
    PA_EWORKSPACE = -3,   /* workspace pointer NULL or smaller than required */
    PA_ELAUNCH = -4,      /* the HIP runtime refused a launch */
    PA_ENOMEM = -5        /* block manager: not enough free blocks, or no host memory
                             left (nothing changed) */
} pa_status;

/*
 * KV append.  For every new token i in [0, num_tokens) with
 * slot = slot_mapping[i] >= 0, copy key[i] ([num_kv_heads, head_dim]) into
 * k_cache[slot / block_size, slot % block_size] and value[i] into v_cache at
 * the same place, bit for bit.  Negative slots (padding tokens) are skipped.
 * key, value: [num_tokens, num_kv_heads, head_dim].  Slots must be distinct
 * and below num_blocks * block_size.  num_tokens == 0 is a no-op.
 */
int pa_reshape_and_cache(const void *key, const void *value,
                         void *k_cache, void *v_cache,
                         const int32_t *slot_mapping, int32_t num_tokens,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, pa_dtype dtype, void *stream);

/*
 * FP8 KV cache.  The pages name quantized inference as a later topic (page
 * "从零实现一个 mini vLLM--开篇", section "5. 这个系列会怎么展开", stage six,
 * and section "6. 我们不会一开始就做什么") without fixing a format; here a
 * cache may hold OCP FP8 E4M3 values with one scale per tensor: the value a
 * stored byte e stands for is k_scale * e4m3(e) in the K cache and
 * v_scale * e4m3(e) in the V cache.  Same layouts as above, one byte per
 * element.
 *
 * KV append into an fp8 cache: as pa_reshape_and_cache, but every element x
 * of key (value) is stored as the E4M3 value nearest to
 * min(max(x * (1/k_scale), -448), 448), ties to even, where 1/k_scale and the
 * product are IEEE single-precision operations (x read as fp32 from src_dtype
 * PA_F32 or PA_BF16).  NaN inputs store NaN (0x7F or 0xFF).  k_scale and
 * v_scale must be finite and > 0 with a finite reciprocal (PA_EINVAL).
 */
int pa_reshape_and_cache_fp8(const void *key, const void *value,
                             void *k_cache, void *v_cache,
                             const int32_t *slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int64_t num_blocks, pa_dtype src_dtype,
                             float k_scale, float v_scale, void *stream);

/*
 * Bytes of workspace pa_decode needs for these shapes (0 for invalid head
 * counts).  It does not depend on the context lengths, num_seqs or the block
 * table width, so one workspace serves every call with the same head counts
 * and head_dim (or fewer query heads per kv head).
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_blocks_per_seq, int32_t block_size);

/*
 * Paged-attention decode: one query row per sequence.  For sequence s and
 * query head h, with n = context_lens[s] (the cached tokens of s, the token
 * being decoded included) and kv = h / (num_q_heads / num_kv_heads):
 *   x_t = scale * <q[s,h,:], K_t>,  t = 0..n-1,
 *   out[s,h,:] = sum_t softmax(x)_t * V_t,
 * where token t of s lives in physical block block_tables[s, t / block_size]
 * at offset t % block_size.  n == 0 writes zeros.
 * q, out: [num_seqs, num_q_heads, head_dim].
 * workspace: device memory of at least pa_decode_workspace_size(...) bytes,
 * uninitialised is fine.  It carries partial results of contexts split across
 * waves from the first kernel of the call to the second, so calls that may
 * overlap in time must not share a workspace.
 * num_seqs is at most 8192.
 */
int pa_decode(void *out, const void *q,
              const void *k_cache, const void *v_cache,
              const int32_t *block_tables, int32_t max_blocks_per_seq,
              const int32_t *context_lens, int32_t num_seqs,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
              int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
              void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_decode with the main kernel timed: identical arguments, behaviour and
 * errors, plus two hipEvent_t handles, created by and owned by the caller
 * (either may be NULL).  The streaming kernel is launched with
 * hipExtLaunchKernel, which sets kernel_start to the kernel's start and
 * kernel_stop to its end, so hipEventElapsedTime(kernel_start, kernel_stop)
 * is that kernel's duration; the kernel that then merges split contexts is not
 * included.  For benchmarks and profilers; pa_decode is this call with both
 * events NULL.
 */
int pa_decode_timed(void *out, const void *q,
                    const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                    const int32_t *context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                    void *workspace, size_t workspace_bytes, void *stream,
                    void *kernel_start, void *kernel_stop);

/*
 * Decode step with the KV append fused in: for every sequence s with
 * n = context_lens[s] >= 1, key[s] and value[s] ([num_seqs, num_kv_heads,
 * head_dim]) are the new token's K and V at position n - 1.  They are written
 * to k_cache/v_cache at that position's slot (block_tables[s, (n-1)/16],
 * offset (n-1) % 16), and out is what pa_decode computes over positions
 * 0..n-1, position n-1 included.  The result is that of pa_reshape_and_cache
 * with slot_mapping[s] = that slot, followed by pa_decode, in the two kernel
 * launches of pa_decode: the attention takes the new rows from key/value, and
 * the split-context merge that follows also writes them to the cache.
 * Sequences with n = 0 append nothing and get zero rows.  Same arguments,
 * errors and workspace as pa_decode;
 * key/value must be non-NULL (PA_EINVAL otherwise) and must not overlap the
 * caches.  Position n-1's slot is overwritten whatever it held.
 */
int pa_decode_append(void *out, const void *q, const void *key, const void *value,
                     void *k_cache, void *v_cache,
                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t num_seqs,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_decode_append without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing.  The records of
 * contexts split across waves go to a fixed 16 MiB array that the library holds
 * on each device it runs on until the process ends.  A call needs
 * waves * 2 * h * (head_dim + 2) * 4 bytes of it plus 16 bytes per wave, where
 * h is the query heads per wave (the query heads per kv head rounded up to a
 * power of two, at most 8) and waves is 1024 on MI355X unless
 * pa_decode_set_launch chose another count: every supported shape fits at
 * 1024 waves; PA_EWORKSPACE for a call that does not fit (nothing is launched).
 * Every call on one device uses that device's array, so calls that may overlap
 * in time on one device race: enqueue them on one stream.  The array needs no
 * clearing (every record a call reads is written earlier in the same call).
 * Otherwise identical to pa_decode_append.
 */
int pa_decode_append_noalloc(void *out, const void *q, const void *key, const void *value,
                             void *k_cache, void *v_cache,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *context_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                             void *stream);

/*
 * pa_decode over fp8 caches (written by pa_reshape_and_cache_fp8): what
 * pa_decode computes with K_t and V_t the dequantized rows k_scale * e4m3(.)
 * and v_scale * e4m3(.).  q and out are bf16 (dtype must be PA_BF16, else
 * PA_EUNSUPPORTED).  The kernel forms bf16 products of q and the stored values
 * (every E4M3 value is exactly a bf16), applies scale * k_scale to the fp32
 * scores and v_scale to the fp32 output sums.  Same workspace, limits and
 * errors as pa_decode, plus the scale checks of pa_reshape_and_cache_fp8.
 */
int pa_decode_fp8(void *out, const void *q,
                  const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                  const int32_t *context_lens, int32_t num_seqs,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int64_t num_blocks, float scale,
                  float k_scale, float v_scale, pa_dtype dtype,
                  void *workspace, size_t workspace_bytes, void *stream);

/* pa_decode_fp8 with the streaming kernel timed, as pa_decode_timed. */
int pa_decode_fp8_timed(void *out, const void *q,
                        const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, int32_t max_blocks_per_seq,
                        const int32_t *context_lens, int32_t num_seqs,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int64_t num_blocks, float scale,
                        float k_scale, float v_scale, pa_dtype dtype,
                        void *workspace, size_t workspace_bytes, void *stream,
                        void *kernel_start, void *kernel_stop);

/* pa_decode_append with the streaming kernel timed, as pa_decode_timed. */
int pa_decode_append_timed(void *out, const void *q, const void *key, const void *value,
                           void *k_cache, void *v_cache,
                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *context_lens, int32_t num_seqs,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                           void *workspace, size_t workspace_bytes, void *stream,
                           void *kernel_start, void *kernel_stop);

/*
 * Launch shape of every later pa_decode* call in this process (all threads):
 * waves of the persistent streaming grid (0 = 4 per compute unit, for every
 * cache type; at most 4096, rounded down to a multiple of 4), blocks in flight
 * per wave (0 = the default 2; else 2, 3 or 4,
 * and for fp8 caches also 6 or 8) and the extra work-split cost of closing a
 * sequence in units of a quarter block (-1 = the default 4; else 0..64).  The
 * results of decode do not depend on these choices; they move only the split
 * points and the pipeline depth.  For tests and launch-shape sweeps; calls
 * already enqueued are unaffected.  PA_EINVAL for values out of range (nothing
 * changes then).
 */
int pa_decode_set_launch(int32_t waves, int32_t stages, int32_t switch_ticks);

/*
 * The decode step as a HIP graph, for callers that repeat it on fixed buffers
 * (the CUDA-graph-style launch the pages list among an engine's speed-ups:
 * page "vllm-v0 版本介绍", section 为什么需要推理框架？, item 3).
 * Records what pa_decode_append(<same arguments>) enqueues into a graph and
 * returns its executable instance in *graph_exec (caller owns it: release with
 * pa_graph_destroy).  The pointers and sizes are baked in; what the buffers
 * hold may change between launches (new q/key/value rows, tables, lengths, as
 * long as the shapes and num_seqs stay the same).  Nothing is run by this
 * call.  num_seqs must be > 0.  Errors as pa_decode_append; PA_ELAUNCH if the
 * runtime refuses the capture or the instantiation.
 */
int pa_decode_append_graph(void **graph_exec, void *out, const void *q, const void *key,
                           const void *value, void *k_cache, void *v_cache,
                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *context_lens, int32_t num_seqs,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                           void *workspace, size_t workspace_bytes);

/*
 * The decode step over fp8 caches: sequence s's new K/V row (row s of key and
 * value, bf16 [num_seqs, num_kv_heads, head_dim]) is quantized into the caches
 * at position n-1 = context_lens[s]-1 exactly as pa_reshape_and_cache_fp8 does
 * (e4m3 of x / scale, nearest even, saturated at +-448), then pa_decode_fp8
 * runs over all n tokens.  Three kernel launches: the quantized append first
 * (the fp8 streaming kernel reads every token from the cache; it cannot take
 * the new rows from the inputs as pa_decode_append does, because their bytes
 * exist only after quantization), then the two of pa_decode_fp8.  Sequences
 * with n = 0 append nothing and get zero rows.  Arguments, workspace and errors
 * as pa_decode_fp8; key/value must be non-NULL (PA_EINVAL otherwise) and must
 * not overlap the caches.
 */
int pa_decode_append_fp8(void *out, const void *q, const void *key, const void *value,
                         void *k_cache, void *v_cache,
                         const int32_t *block_tables, int32_t max_blocks_per_seq,
                         const int32_t *context_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, float scale,
                         float k_scale, float v_scale, pa_dtype dtype,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_decode_append_fp8 recorded as a HIP graph, as pa_decode_append_graph
 * records pa_decode_append (the scales are baked in with the pointers).
 */
int pa_decode_append_fp8_graph(void **graph_exec, void *out, const void *q, const void *key,
                               const void *value, void *k_cache, void *v_cache,
                               const int32_t *block_tables, int32_t max_blocks_per_seq,
                               const int32_t *context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int64_t num_blocks, float scale,
                               float k_scale, float v_scale, pa_dtype dtype,
                               void *workspace, size_t workspace_bytes);
/* Enqueue a graph from pa_decode_append_graph or pa_decode_append_fp8_graph on
 * stream (NULL = default). */
int pa_graph_launch(void *graph_exec, void *stream);
/* Release a graph instance (NULL is a no-op). */
int pa_graph_destroy(void *graph_exec);

/* Bytes of workspace pa_prefill_chunk needs (currently always 0). */
size_t pa_prefill_workspace_size(int32_t num_seqs, int32_t total_query_rows,
                                 int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int32_t block_size);

/*
 * Chunked prefill.  Sequence s owns query rows query_start_loc[s] ..
 * query_start_loc[s+1]-1: its c = query_start_loc[s+1] - query_start_loc[s]
 * newest tokens, whose K/V must already be in the cache (append them with
 * pa_reshape_and_cache first).  Row i of the chunk sits at absolute position
 * p = context_lens[s] - c + i and attends causally to tokens 0..p inclusive of
 * its own sequence, through the block table, with the same formula as
 * pa_decode.  0 <= c <= context_lens[s] is required.
 * q, out: [query_start_loc[num_seqs], num_q_heads, head_dim]; query_start_loc:
 * [num_seqs + 1] int32, non-decreasing, starting at 0.  total_query_rows is
 * query_start_loc[num_seqs] (the host's copy).
 */
int pa_prefill_chunk(void *out, const void *q,
                     const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *query_start_loc, int32_t total_query_rows,
                     const int32_t *context_lens, int32_t num_seqs,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_prefill_chunk over fp8 caches (written by pa_reshape_and_cache_fp8): the
 * same causal attention with K_t and V_t the dequantized rows
 * k_scale * e4m3(.) and v_scale * e4m3(.), so that a chunked-prefill step can
 * share the fp8 cache with pa_decode_fp8.  q and out are bf16 (dtype must be
 * PA_BF16).  As in pa_decode_fp8, the stored values are exact bf16 operands,
 * scale * k_scale applies to the fp32 scores and v_scale to the fp32 output
 * sums.  Same workspace and errors as pa_prefill_chunk, plus the scale checks
 * of pa_reshape_and_cache_fp8.
 */
int pa_prefill_chunk_fp8(void *out, const void *q,
                         const void *k_cache, const void *v_cache,
                         const int32_t *block_tables, int32_t max_blocks_per_seq,
                         const int32_t *query_start_loc, int32_t total_query_rows,
                         const int32_t *context_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, float scale,
                         float k_scale, float v_scale, pa_dtype dtype,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Copy on write.  For every pair p < num_pairs, block pairs[2p+1] of k_cache
 * and of v_cache becomes a bit copy of block pairs[2p] (all block_size slots,
 * all heads).  pairs is a DEVICE array [num_pairs, 2] of int32 block ids below
 * num_blocks; destinations must be distinct and must not be sources of the
 * same call (the copies run concurrently).  Used when a block shared by
 * several sequences (a common prompt prefix, page "vllm-v0 版本介绍", section
 * 为什么需要推理框架？, PagedAttention item) is about to be written by one of
 * them; pa_bm_append_batch reports such pairs.  num_pairs == 0 is a no-op.
 */
int pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int32_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int64_t num_blocks, pa_dtype dtype, void *stream);

/*
 * Streaming-read reference for benchmarks (not part of attention): reads every
 * byte of src once, 16 bytes per load with the non-temporal hint as the decode
 * kernel loads K and V, and XORs every 32-bit word of it into *xor_out (device
 * memory, which the caller sets before the call; zero gives the XOR of src).
 * The bytes read divided by the kernel's time is the plain read rate the gather
 * of the decode kernel is compared with.  bytes must be a multiple of 16 and src
 * 16-byte aligned (PA_EINVAL otherwise); bytes == 0 is a no-op.  Asynchronous on
 * stream; allocates nothing.
 */
int pa_stream_read_probe(const void *src, size_t bytes, uint32_t *xor_out, void *stream);

/*
 * Host block manager (CPU only, no device memory): hands out the pool's block
 * ids to sequences and builds the block tables, context lengths and slot
 * mappings the kernels above take.  A sequence gets a new block only when its
 * last one is full and returns all of them when it ends (page "轻量级的vLLM",
 * sections 核心机制一：分页 KV Cache and 核心机制二：连续批处理).  A forked
 * sequence shares every block of its parent (reference counted); the first
 * write into a shared, partly filled last block moves the writer to a fresh
 * copy (reported as a (src, dst) pair for pa_copy_blocks).
 * Policy: free blocks form a stack, block 0 on top at creation; allocation
 * pops, release pushes; a sequence releases its blocks last to first.  A call
 * that fails changes nothing.  Not thread safe: one manager per thread.
 */
typedef struct pa_block_manager pa_block_manager;

/* NULL if num_blocks is not in [1, INT32_MAX / 16] or block_size != 16. */
pa_block_manager *pa_bm_create(int64_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager *m);
/* Free blocks (-1 for NULL). */
int64_t pa_bm_num_free(const pa_block_manager *m);
/* Reference count of a block (0 = free), -1 when out of range. */
int32_t pa_bm_refcount(const pa_block_manager *m, int32_t block);
/* A new sequence holding num_tokens >= 0 tokens (their K/V are written by the
 * caller, e.g. pa_reshape_and_cache over the slots of pa_bm_batch_tables).
 * PA_EINVAL if seq_id exists, PA_ENOMEM if ceil(num_tokens/16) blocks are not
 * free. */
int pa_bm_add_sequence(pa_block_manager *m, int64_t seq_id, int64_t num_tokens);
/* child_id starts as a copy of parent_id sharing all its blocks. */
int pa_bm_fork(pa_block_manager *m, int64_t parent_id, int64_t child_id);
/* The sequence ends; blocks whose count drops to 0 are freed. */
int pa_bm_free(pa_block_manager *m, int64_t seq_id);
/* Tokens held by a sequence, -1 if unknown. */
int64_t pa_bm_num_tokens(const pa_block_manager *m, int64_t seq_id);
/*
 * One new token for each of the n distinct sequences seq_ids[i]: slot_mapping[i]
 * receives its slot (block * 16 + offset).  Copy-on-write pairs (src, dst) go
 * to copies[2*k], copies[2*k+1], k < *num_copies <= max_copies; apply them
 * (pa_copy_blocks) before writing the new tokens.  PA_EINVAL for unknown or
 * repeated ids or too little copy room, PA_ENOMEM if the blocks needed are not
 * free; in both cases nothing changes.
 */
int pa_bm_append_batch(pa_block_manager *m, const int64_t *seq_ids, int32_t n, int32_t *slot_mapping,
                       int32_t *copies, int32_t max_copies, int32_t *num_copies);
/* Rows of block_tables [n, max_blocks_per_seq] (padded with -1) and
 * context_lens [n] for seq_ids, host arrays; PA_EINVAL if a sequence is unknown
 * or holds more than max_blocks_per_seq blocks. */
int pa_bm_batch_tables(const pa_block_manager *m, const int64_t *seq_ids, int32_t n, int32_t *block_tables,
                       int32_t max_blocks_per_seq, int32_t *context_lens);

/* Static, human-readable text for a pa_status value. */
const char *pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
