/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-attention library.
 *
 * The operations: single-query decode attention (pa_decode) and causal
 * multi-token prefill attention (pa_prefill) over a paged KV cache.  K and
 * V live in fixed-size physical blocks shaped
 * [num_blocks, block_size, num_kv_heads, head_dim]; each sequence reaches its
 * tokens through a row of a block table that maps logical block i (tokens
 * [i*block_size, (i+1)*block_size)) to a physical block id.  Defined by the
 * pages:
 *   "paged-attention-and-vllm-inference" (astro-blog-cod.pages.dev), code
 *     block `paged_attention` (block-table indirection, partly filled last
 *     block, running max / running sum with rescale) and the kernel design
 *     points block (block table resident on the device, per-sequence lengths);
 *   "5.KV Cache 管理 & PagedAttention" (lowentro.cn), question 7 (GQA/MQA:
 *     a kv head serves Hq/Hkv consecutive query heads), question 8 (batch
 *     block table [B, max_blocks] int32 padded with -1, plus per-sequence
 *     lengths), question 9 (block allocator, reference counts), question 12
 *     (writing a new token at block = pos / bs, offset = pos % bs),
 *     question 13 (per-block loads inside the kernel), question 18
 *     (copy-on-write of a shared block), question 20 (shared prefix blocks),
 *     question 6 (causal prefill), question 19 (query tiles against the
 *     logical KV blocks with an online softmax);
 *   "KV Cache 优化与内存管理深度解析：PagedAttention 原理与实践"
 *     (aiattnstudio.link), `PagedAttentionKernel.kernel_design` (kernel
 *     arguments: query, caches, block_tables, seq_lens, output, block size).
 *
 * Conventions shared by every call
 *   - Tensors are passed as `pa_tensor` descriptors: a device address, a
 *     dtype, a rank, a shape and strides in elements.  The caller allocates
 *     and owns every device buffer; the library never allocates, frees or
 *     synchronises device memory.
 *   - Device work is enqueued asynchronously on `launch->stream` (a
 *     hipStream_t; NULL means the null stream).  A call returns once its
 *     kernels are enqueued.
 *   - Every argument is validated on the host before any HIP call, so a bad
 *     call fails with PA_ERR_INVALID_ARG / PA_ERR_UNSUPPORTED / PA_ERR_WORKSPACE
 *     and touches no device state.  Device-resident contents (block ids,
 *     lengths, slots) are trusted: block ids must lie in [0, num_blocks),
 *     seq_lens[b] <= max_blocks * block_size, slots must be unique and inside
 *     the cache.  A violation gives unspecified values in the outputs it
 *     touches, but every access stays inside the buffers of the call: a
 *     block id outside the pool reads block 0, a length is clamped to
 *     [0, max_blocks * block_size], a slot outside the cache is skipped and
 *     query_start_loc entries are clamped to [0, T].  A caller that wants
 *     to know when that happened passes launch->error_flags (below).
 *   - Every call returns PA_OK (0) or a negative status; pa_last_error()
 *     then holds a message (thread-local, valid until the next call on the
 *     same thread).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define PA_OK 0
#define PA_ERR_INVALID_ARG (-1)   /* bad shape, stride, dtype, null pointer   */
#define PA_ERR_WORKSPACE (-2)     /* split decode needs a larger workspace     */
#define PA_ERR_OUT_OF_BLOCKS (-3) /* allocator has no free block               */
#define PA_ERR_BAD_BLOCK (-4)     /* id out of range, not allocated, underflow */
#define PA_ERR_HIP (-5)           /* a HIP launch reported an error            */
#define PA_ERR_UNSUPPORTED (-6)   /* valid request outside the built variants  */
#define PA_ERR_NOT_FOUND (-7)     /* unknown sequence id                       */

/* element types */
#define PA_F32 0
#define PA_F16 1
#define PA_BF16 2
#define PA_FP8_E4M3 3 /* OCP E4M3FN, stored as one byte */
#define PA_I32 4
#define PA_I64 5

typedef struct pa_tensor {
  void* data;        /* device address, owned by the caller                    */
  int32_t dtype;     /* PA_F32 ... PA_I64                                      */
  int32_t ndim;      /* 1..4                                                   */
  int64_t shape[4];  /* extents, outermost first                               */
  int64_t stride[4]; /* strides in elements                                    */
  float scale;       /* fp8 tensors: stored value = decoded code * scale       */
} pa_tensor;

/* decode path selection (tests and tuning; 0 = automatic) */
#define PA_PATH_AUTO 0
#define PA_PATH_VALU 1 /* per-lane dot products, DPP reductions             */
#define PA_PATH_MFMA 2 /* query-group x K-tile and P x V on matrix cores    */

typedef struct pa_launch {
  void* stream;             /* hipStream_t; NULL = null stream                   */
  void* workspace;          /* device scratch for split decode, caller-owned     */
  size_t workspace_bytes;   /* its size                                          */
  int32_t partition_tokens; /* 0 = automatic (see pa_decode_plan); -1 = never
                               split; > 0: split each sequence into partitions
                               of this many tokens (a multiple of 16)            */
  int32_t path;             /* PA_PATH_*                                         */
  int32_t* error_flags;     /* NULL, or a device int32[PA_NUM_FLAGS] the caller
                               has zeroed: a kernel that meets device-resident
                               contents outside their contract and takes them
                               the documented way (see the conventions above)
                               stores 1 into the flag of that kind; flags are
                               never cleared by the library.  Calls that
                               overlap on one array may interleave their
                               stores (each only ever stores 1)              */
} pa_launch;

/* error_flags entries (indices) */
#define PA_FLAG_BLOCK_ID 0    /* a block id outside [0, num_blocks) was read   */
#define PA_FLAG_LENGTH 1      /* a length outside [0, max_blocks * block_size] */
#define PA_FLAG_SLOT 2        /* a cache-write slot >= num_blocks * block_size */
#define PA_FLAG_QUERY_START 3 /* query_start_loc outside [0, T] or decreasing */
#define PA_NUM_FLAGS 4

/*
 * pa_reshape_and_cache -- write new K/V tokens into their cache slots.
 *   key, value    [T, Hkv, D]   f32 | f16 | bf16; token stride free, the head
 *                               stride and the dim stride must be D and 1
 *   slot_mapping  [T]           i64; slot = block * block_size + offset;
 *                               a negative slot skips that token
 *   key_cache,
 *   value_cache   [N, bs, Hkv, D] contiguous; same dtype as key/value (bit
 *                               copy), or PA_FP8_E4M3: code = E4M3(x / scale)
 *                               with one fp32 division, round to nearest even,
 *                               saturating at +-448, NaN kept (the cache
 *                               tensor's `scale` is the per-tensor scale)
 *   launch        stream (workspace unused); NULL = null stream
 * Two tokens of one call must not share a slot (the written value is then
 * unspecified).  T = 0 is a no-op.
 */
int pa_reshape_and_cache(const pa_tensor* key, const pa_tensor* value,
                         const pa_tensor* slot_mapping, pa_tensor* key_cache,
                         pa_tensor* value_cache, const pa_launch* launch);

/*
 * pa_decode -- out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b, where K_b, V_b
 * are the first seq_lens[b] tokens of sequence b read through
 * block_tables[b] and kv head h / (Hq / Hkv).
 *   out           [B, Hq, D]    dtype of query; dim stride 1; rows 16-byte
 *                               aligned (like the query's)
 *   query         [B, Hq, D]    f32 | f16 | bf16; dim stride 1
 *   key_cache,
 *   value_cache   [N, bs, Hkv, D] contiguous; dtype of query, or PA_FP8_E4M3
 *                               with per-tensor `scale` (f16 / bf16 query)
 *   block_tables  [B, max_blocks] i32, column stride 1, entries past
 *                               ceil(seq_lens[b] / bs) are never read;
 *                               max_blocks * bs <= 2^30
 *                               (PA_ERR_INVALID_ARG otherwise)
 *   seq_lens      [B]           i32, 0 <= seq_lens[b] <= max_blocks * bs;
 *                               a zero length gives a zero output row
 *   scale         score scale (1/sqrt(D) for standard attention)
 *   block_size    bs, a multiple of 16 (16 and 32 are the usual sizes)
 *   num_kv_heads  Hkv; Hq % Hkv must be 0
 *   launch        stream, workspace (16-byte aligned) and partitioning;
 *                 NULL = null stream, automatic partitioning, no workspace
 * Supported head_dim: 64, 128.  When the chosen plan splits sequences into
 * pieces, per-piece (max, sum, partial output) triples go to the workspace
 * and a second kernel merges them; pa_decode_workspace_bytes gives the size
 * (pa_decode_plan describes the plan).  Results are deterministic (no
 * atomics) for a given plan.
 */
int pa_decode(pa_tensor* out, const pa_tensor* query,
              const pa_tensor* key_cache, const pa_tensor* value_cache,
              const pa_tensor* block_tables, const pa_tensor* seq_lens,
              float scale, int32_t block_size, int32_t num_kv_heads,
              const pa_launch* launch);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and launches
 * as pa_decode, but a split plan's (max, sum, partial output) triples and
 * merge plan go to a fixed device array the library holds (16 MiB per GPU
 * it runs on, kept until the process ends) instead of a caller workspace:
 *   launch   stream, partition_tokens, path and error_flags as for
 *            pa_decode; workspace must be NULL with workspace_bytes 0
 *            (PA_ERR_INVALID_ARG otherwise)
 * A plan whose triples do not fit returns PA_ERR_WORKSPACE before any
 * launch (the balanced plan needs (shares + B) * Hq * (D + 2) * 4 + 8 B
 * bytes, shares = 256, or 768 for an fp8 cache on the matrix cores: e.g.
 * 10.7 MB for B = 64, Hq = 64, D = 128).  Nothing in the array needs to
 * start cleared: the decode launch writes every entry the merge reads.
 * The first call on a device looks the array's address up (no allocation);
 * later calls reuse it.  Every call on one GPU shares that GPU's array, so
 * calls that overlap on one GPU (other streams, other host threads) race:
 * serialise them.
 */
int pa_decode_noalloc(pa_tensor* out, const pa_tensor* query,
                      const pa_tensor* key_cache, const pa_tensor* value_cache,
                      const pa_tensor* block_tables, const pa_tensor* seq_lens,
                      float scale, int32_t block_size, int32_t num_kv_heads,
                      const pa_launch* launch);

/*
 * pa_prefill -- causal attention of a batch of new tokens over the paged
 * cache ("5.KV Cache 管理 & PagedAttention", question 6, `MHAWithCache`
 * prefill branch, lower-triangular mask; question 19, query tiles against
 * the logical KV blocks of the block table with an online softmax;
 * question 3, section 3.3, prefill K/V kept in the cache).  Sequence b has
 * seq_lens[b] tokens in the cache, the new ones included (write them with
 * pa_reshape_and_cache first); its n_b = query_start_loc[b+1] -
 * query_start_loc[b] query rows are its last n_b tokens, so row i sits at
 * position p = seq_lens[b] - n_b + i and
 *   out[row, h] = softmax(scale * q[row, h] . K_b[0..p]^T) V_b[0..p]
 * with kv head h / (Hq / Hkv).  n_b == seq_lens[b] is a whole prompt;
 * n_b < seq_lens[b] continues a sequence whose earlier tokens are cached
 * (a chunked prompt, or a prefix shared through the prefix cache).  A row
 * whose position would be negative (n_b > seq_lens[b]) attends no token and
 * gets zeros.
 *   out             [T, Hq, D]    dtype of query; dim stride 1; rows 16-byte
 *                                 aligned (like the query's)
 *   query           [T, Hq, D]    f16 | bf16; dim stride 1; the rows of all
 *                                 sequences back to back
 *   key_cache,
 *   value_cache     [N, bs, Hkv, D] contiguous; dtype of query, or
 *                                 PA_FP8_E4M3 with per-tensor `scale`
 *   block_tables    [B, max_blocks] i32, column stride 1; entries past
 *                                 ceil(seq_lens[b] / bs) are never read;
 *                                 max_blocks * bs <= 2^30
 *                                 (PA_ERR_INVALID_ARG otherwise)
 *   seq_lens        [B] i32, 0 <= seq_lens[b] <= max_blocks * bs
 *   query_start_loc [B + 1] i32 (device), query_start_loc[0] = 0, rising to
 *                                 query_start_loc[B] = T
 *   max_query_len   an upper bound of every n_b (sizes the grid; a smaller
 *                   value is still correct, only slower); <= 0 uses T
 *   scale           score scale, positive and finite (1/sqrt(D) for standard
 *                   attention)
 *   block_size (a multiple of 16), num_kv_heads: as for pa_decode
 *   launch          stream; NULL = null stream.  Partitioning unused.  The
 *                   workspace is optional and only used for a bf16 query
 *                   with bf16 K/V: given pa_prefill_workspace_bytes(...)
 *                   bytes (4-byte aligned, caller-owned, any contents), the
 *                   P x V product runs in f16 (V converted exactly, which
 *                   holds for |v| < 2^16; smaller than 2^-14 rounds to f16's
 *                   subnormal spacing, an absolute error below 2^-25) and
 *                   a second launch recomputes, with the bf16 product, every
 *                   workgroup that met a wider V value; without it (or
 *                   smaller) the bf16 product runs throughout, P as a high
 *                   and a low bf16 part with a product each.  A bf16 query
 *                   with fp8 K/V always runs P x V in f16 (its values fit).
 * Supported head_dim: 64, 128.  Deterministic.  Asynchronous on
 * launch->stream; calls that share a workspace must not overlap.
 */
int pa_prefill(pa_tensor* out, const pa_tensor* query,
               const pa_tensor* key_cache, const pa_tensor* value_cache,
               const pa_tensor* block_tables, const pa_tensor* seq_lens,
               const pa_tensor* query_start_loc, int32_t max_query_len,
               float scale, int32_t block_size, int32_t num_kv_heads,
               const pa_launch* launch);

/*
 * Workspace bytes that let pa_prefill run a bf16 query's P x V product in
 * f16 (one int32 per workgroup of its grid): batch = B, num_rows = T and
 * max_query_len as passed to pa_prefill.  Negative status on negative sizes.
 */
int64_t pa_prefill_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_rows,
                                   int32_t max_query_len);

/*
 * pa_decode_shared_prefix -- pa_decode for a batch whose sequences all start
 * with the same cached prefix: the first prefix_tokens tokens of every
 * sequence are the tokens of the blocks listed in prefix_blocks, shared
 * through the block tables ("5.KV Cache 管理 & PagedAttention", question 20;
 * "KV Cache 优化与内存管理深度解析：PagedAttention 原理与实践",
 * `HashBasedCaching`).  The result is pa_decode's.  The prefix part of the
 * attention is taken for all (sequence, query head) rows of a kv head at
 * once, each row limited to its sequence's length, instead of once per
 * sequence: with rows = batch * (num_q_heads / num_kv_heads) below 1024,
 * inside the matrix-core decode launch in groups of 16 rows (the kernel's
 * query columns), from 1024 rows on as a separate launch of the prefill
 * kernel in 256-row tiles.  The rest of every sequence goes through the
 * decode kernel, and the merge kernel folds the partial results (the
 * pages' rescale identity across pieces).
 *   out, query, key_cache, value_cache, block_tables, seq_lens, scale,
 *   block_size, num_kv_heads: as for pa_decode, with an f16 or bf16 query
 *                 and a positive scale
 *   prefix_blocks [>= prefix_tokens / block_size] i32 (device), contiguous
 *   prefix_tokens a positive multiple of block_size; sequences shorter than
 *                 it attend only their own length of it
 *   launch        stream and workspace (16-byte aligned, at least
 *                 pa_decode_shared_prefix_workspace_bytes); partition_tokens
 *                 must be 0 (the plan is always the balanced schedule, so
 *                 the batch is at most 2048 sequences)
 * Below 1024 rows per kv head the decode runs on the matrix-core path (a
 * launch asking for the VALU path is refused).  Supported head_dim: 64,
 * 128.  Two launches (decode with the grouped prefix work, merge) or three
 * (prefix pass, decode of the rest, merge), deterministic.  Whether it is
 * faster than pa_decode depends on how much of the batch the prefix is;
 * the lengths stay on the device, so the caller chooses.
 */
int pa_decode_shared_prefix(pa_tensor* out, const pa_tensor* query,
                            const pa_tensor* key_cache, const pa_tensor* value_cache,
                            const pa_tensor* block_tables, const pa_tensor* seq_lens,
                            const pa_tensor* prefix_blocks, int32_t prefix_tokens,
                            float scale, int32_t block_size, int32_t num_kv_heads,
                            const pa_launch* launch);

/* Workspace bytes pa_decode_shared_prefix needs; a negative status on
 * invalid sizes. */
int64_t pa_decode_shared_prefix_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t block_size, int32_t max_blocks,
                                                int32_t prefix_tokens);

/*
 * pa_copy_blocks -- device copy of whole physical blocks, the data step of
 * copy-on-write ("5.KV Cache 管理 & PagedAttention", question 18,
 * copy_block): for each row (src, dst) of block_pairs,
 * key_cache[dst] = key_cache[src] and value_cache[dst] = value_cache[src].
 *   key_cache, value_cache  [N, bs, Hkv, D] contiguous, any one dtype
 *   block_pairs             [n, 2] i32 (device), rows independent; a dst
 *                           must not appear as another row's src or dst
 */
int pa_copy_blocks(pa_tensor* key_cache, pa_tensor* value_cache,
                   const pa_tensor* block_pairs, const pa_launch* launch);

/*
 * pa_swap_blocks -- copy whole blocks from one pair of pools to another,
 * for swapping blocks out to host memory and back in
 * ("KV Cache 优化与内存管理深度解析：PagedAttention 原理与实践", `CPUSwap`):
 * for each row (src, dst) of block_pairs,
 * dst_key_cache[dst] = src_key_cache[src], and the same for V.
 *   dst_key_cache, dst_value_cache  [N_dst, bs, Hkv, D] contiguous
 *   src_key_cache, src_value_cache  [N_src, bs, Hkv, D] contiguous, same
 *                           dtype and block shape as the destination
 *   block_pairs             [n, 2] i32, rows independent, no destination
 *                           block twice
 * Either pair of pools may live in pinned host memory (allocated with
 * hipHostMalloc, e.g. torch's pin_memory), which the kernel reads or writes
 * over the host link; block_pairs must be device-accessible.  Pairs with an
 * id outside its pool are skipped.  Asynchronous on launch->stream.
 */
int pa_swap_blocks(pa_tensor* dst_key_cache, pa_tensor* dst_value_cache,
                   const pa_tensor* src_key_cache, const pa_tensor* src_value_cache,
                   const pa_tensor* block_pairs, const pa_launch* launch);

/*
 * Workspace bytes pa_decode needs for these sizes and this partition request
 * (the same plan pa_decode makes; 0 when it does not split).  max_blocks is
 * the block-table width.  Returns a negative status on invalid sizes.
 */
int64_t pa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_blocks,
                                  int32_t partition_tokens);

/* how pa_decode spreads the work (pa_decode_plan) */
#define PA_SCHEDULE_SINGLE 0     /* one workgroup per sequence                 */
#define PA_SCHEDULE_PARTITIONS 1 /* fixed-size token partitions, then a merge  */
#define PA_SCHEDULE_BALANCED 2   /* equal shares of the batch's 16-token tiles
                                    per workgroup (256 in all; 768 smaller ones
                                    for an fp8 cache on the matrix cores), found
                                    on the device from seq_lens; sequences cut
                                    by a share boundary are merged afterwards */

typedef struct pa_decode_plan_info {
  int32_t schedule;         /* PA_SCHEDULE_*                                    */
  int32_t partition_tokens; /* PA_SCHEDULE_PARTITIONS: tokens per partition     */
  int64_t workspace_bytes;  /* what pa_decode_workspace_bytes returns           */
} pa_decode_plan_info;

/*
 * The plan pa_decode makes for these sizes and this partition request:
 * partition_tokens 0 (automatic) runs one pass per sequence (no split) when
 * the block table reaches at most 256 tokens (max_blocks * block_size), else
 * picks the balanced schedule when batch <= 2048, else 512-token
 * partitions; -1 never splits; > 0 asks for partitions of that many tokens.
 * Returns PA_OK or a negative status.
 */
int pa_decode_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t max_blocks,
                   int32_t partition_tokens, pa_decode_plan_info* info);

/* Thread-local message for the last failing call on this thread. */
const char* pa_last_error(void);

/* Short build description (target, variants). */
const char* pa_build_info(void);

/* ------------------------------------------------------------------------ *
 * Host-side block allocator ("5.KV Cache 管理 & PagedAttention", question 9).
 * A stack of free physical block ids guarded by a mutex.  Allocation pops the
 * top of the stack and sets the block's reference count to 1; incref shares
 * a block; decref releases one reference and pushes the block back when the
 * count reaches 0.  Plain CPU code: no device calls.
 * ------------------------------------------------------------------------ */
typedef struct pa_allocator pa_allocator;

/* free_order: the initial stack, bottom first (a permutation of 0..N-1), or
 * NULL for 0..N-1 (the first allocation then returns N-1).  Returns NULL on
 * invalid arguments (see pa_last_error). */
pa_allocator* pa_alloc_create(int32_t num_blocks, const int32_t* free_order);
/* The handle is dead after this call.  Block managers and prefix caches
 * built on the allocator may still be destroyed afterwards (in any order):
 * its memory is released when the last of them is. */
void pa_alloc_destroy(pa_allocator* a);
/* PA_ERR_OUT_OF_BLOCKS when the stack is empty. */
int pa_alloc_allocate(pa_allocator* a, int32_t* block_out);
/* PA_ERR_BAD_BLOCK when the id is out of range or not allocated. */
int pa_alloc_incref(pa_allocator* a, int32_t block);
int pa_alloc_decref(pa_allocator* a, int32_t block);
int32_t pa_alloc_num_free(const pa_allocator* a);
int32_t pa_alloc_num_blocks(const pa_allocator* a);
/* reference count, or PA_ERR_BAD_BLOCK for an id out of range */
int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block);

/* ------------------------------------------------------------------------ *
 * Sequence block manager on top of an allocator (same page, questions 10,
 * 12, 18, 20).  Each sequence owns a block table and a length.  Appending a
 * token allocates a block when the length fills the table and returns the
 * token's slot; appending into a block shared with another sequence first
 * moves the sequence to a private copy (copy-on-write) and reports the
 * (source, destination) pair the caller must copy on the device with
 * pa_copy_blocks before writing.  The manager does not own the allocator.
 * ------------------------------------------------------------------------ */
typedef struct pa_block_manager pa_block_manager;

pa_block_manager* pa_bm_create(pa_allocator* a, int32_t block_size);
void pa_bm_destroy(pa_block_manager* m);
/* New sequence whose first shared_tokens tokens live in the already allocated
 * blocks shared_blocks[0..n_shared) (each gets one more reference). */
int pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id,
                       const int32_t* shared_blocks, int32_t n_shared,
                       int64_t shared_tokens);
/* Reserve the slot of the sequence's next token; cow_src / cow_dst are -1 or
 * the block pair to copy first.  On PA_ERR_OUT_OF_BLOCKS nothing changes. */
int pa_bm_append_slot(pa_block_manager* m, int64_t seq_id, int64_t* slot_out,
                      int32_t* cow_src, int32_t* cow_dst);
/* child shares every block of parent (one more reference each). */
int pa_bm_fork(pa_block_manager* m, int64_t parent_id, int64_t child_id);
int pa_bm_free_sequence(pa_block_manager* m, int64_t seq_id);
int64_t pa_bm_seq_len(const pa_block_manager* m, int64_t seq_id);
int32_t pa_bm_num_blocks_of(const pa_block_manager* m, int64_t seq_id);
/* Fill host arrays block_tables[n, max_blocks] (padded with -1) and
 * seq_lens[n] for the listed sequences; PA_ERR_INVALID_ARG if a table does
 * not fit in max_blocks. */
int pa_bm_export(const pa_block_manager* m, const int64_t* seq_ids, int32_t n,
                 int32_t max_blocks, int32_t* block_tables, int32_t* seq_lens);

/* ------------------------------------------------------------------------ *
 * Prefix cache ("KV Cache 优化与内存管理深度解析：PagedAttention 原理与实践",
 * `HashBasedCaching`: block hashing and the prefix lookup walk-through, where
 * tokens [A,B,C,D,E,F] in 2-token blocks find blocks 7 and 3 for [A,B] and
 * [C,D] and need a new block for [E,F]; "5.KV Cache 管理 & PagedAttention",
 * question 20).  Maps the leading full blocks of token sequences to the
 * physical blocks that hold their K/V.  Block i's key is the whole token
 * prefix up to the end of block i (equal block contents after different
 * histories do not match); hits are verified token by token, so a hash
 * collision never yields a wrong block.  The cache holds one allocator
 * reference on every cached block.  Plain CPU code, thread-safe.
 * ------------------------------------------------------------------------ */
typedef struct pa_prefix_cache pa_prefix_cache;

/* NULL on invalid arguments.  The allocator must outlive the cache. */
pa_prefix_cache* pa_pc_create(pa_allocator* a, int32_t block_size);
/* Releases the cache's references. */
void pa_pc_destroy(pa_prefix_cache* c);
/* Longest cached run of leading full blocks of tokens[0..n_tokens):
 * writes their physical ids to blocks_out[0..k) (k <= max_blocks), takes
 * one reference on each for the caller (release with pa_alloc_decref, e.g.
 * after pa_bm_add_sequence has taken its own), and returns k, or a
 * negative status. */
int32_t pa_pc_match(pa_prefix_cache* c, const int32_t* tokens, int64_t n_tokens,
                    int32_t* blocks_out, int32_t max_blocks);
/* Caches the leading full blocks of a sequence: block i (i < n_blocks and
 * (i + 1) * block_size <= n_tokens) holds the K/V of tokens up to the end of
 * block i.  Prefixes already cached keep their block; every newly cached
 * block gets one cache reference.  Returns the number newly cached, or a
 * negative status (PA_ERR_BAD_BLOCK for a block that is not allocated). */
int32_t pa_pc_insert(pa_prefix_cache* c, const int32_t* tokens, int64_t n_tokens,
                     const int32_t* blocks, int32_t n_blocks);
/* Releases up to max_blocks cached blocks that nobody else references,
 * least recently matched or inserted first, leaves of the prefix tree
 * only.  Returns the number released. */
int32_t pa_pc_evict(pa_prefix_cache* c, int32_t max_blocks);
/* Number of cached blocks. */
int32_t pa_pc_size(const pa_prefix_cache* c);

/*
 * pa_bm_add_sequence_cached -- admit a new sequence through the prefix cache
 * ("5.KV Cache 管理 & PagedAttention", question 20, allocate_with_prefix:
 * the new table starts with the cached blocks of the longest matching
 * prefix, each with one more reference, blocks are allocated for the
 * remaining tokens, and the sequence's prefix is cached in turn;
 * "KV Cache 优化与内存管理深度解析：PagedAttention 原理与实践",
 * `HashBasedCaching` walk-through).  tokens[0 .. n_tokens) are the
 * sequence's token ids.  Steps: pa_pc_match; pa_bm_add_sequence with the
 * matched blocks (the match's own references are then released);
 * pa_bm_append_slot for every remaining token; pa_pc_insert of the
 * sequence's full blocks.  m and c must share one allocator and one block
 * size.
 *   slots_out  [n_tokens - matched] i64 (host): the cache slot of every
 *              token that was not found, in position order -- the K/V the
 *              caller writes with pa_reshape_and_cache before any call
 *              reads this sequence (or another that matches its blocks)
 * Returns the number of matched tokens (a multiple of the block size), or
 * a negative status; on PA_ERR_OUT_OF_BLOCKS (or any error after the
 * sequence was added) the sequence is removed again and every reference
 * it took is released.  Plain CPU code.
 */
int64_t pa_bm_add_sequence_cached(pa_block_manager* m, pa_prefix_cache* c, int64_t seq_id,
                                  const int32_t* tokens, int64_t n_tokens, int64_t* slots_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
